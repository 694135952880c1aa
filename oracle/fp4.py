"""fp64 oracle of the 4-bit QK^T path: block-scaled E2M1 (FP4) queries and keys with FourOverSix
scale selection, feeding the FP8 value path.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
library path.

LongLive DiT blog, section "1. NVFP4" ("What's a scale and what's a block?" and "FourOverSix"):
  * each element becomes a 4-bit E2M1 code, one of 0, +-0.5, +-1, +-1.5, +-2, +-3, +-4, +-6;
  * a block of elements shares one scale; dividing by it brings the block into [-6, 6];
  * FourOverSix: scaling the block maximum to 6 is not always best - when several elements sit
    near the maximum, scaling it to 4 avoids the wide 4-to-6 gap; the quantiser tries both and
    keeps the one with the smaller squared error;
  * the block-scaled matrix product applies the two scales inside the dot product.
Readings for MI355X (the blog's NVFP4 format - 16-element blocks with E4M3 scales - is not what the
gfx950 matrix cores take): the format is MXFP4 from the OCP microscaling specification, blocks of 32
consecutive elements along the head dimension with a power-of-two (E8M0) scale 2^e.  "Maximum to 6"
is the smallest e with 6 * 2^e >= amax; "maximum to 4" the smallest e with 4 * 2^e >= amax, which is
the same e or the next one up.  Each candidate rounds x / 2^e to the nearest E2M1 value (ties to the
even code; |x / 2^e| <= 6 by construction); under rule "4over6" the candidate with the smaller sum of
squared errors sum (2^e E2M1(code) - x)^2 over the block wins, the max-to-6 one on a tie.  With
power-of-two scales the max-to-4 candidate, when it differs, is 2^(e+1), whose grid below 6 * 2^e is
a subset of the grid of 2^e, so it never has the smaller error and the rule reduces to max-to-6 (the
OCP rule, rule "6"); the library implements max-to-6.  A block of zeros takes e = 0; E8M0 holds
2^-127 .. 2^127, so a block whose maximum is below 6 * 2^-127 takes e = -127.  Codes pack two per
byte, the even element in the low nibble; the scale byte is e + 127.
"""
from __future__ import annotations

import math

import numpy as np

from .fp8 import fp8_attention_ref

MX_BLOCK = 32
_E2M1 = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def e2m1_decode_table() -> np.ndarray:
    """value of each of the 16 codes: sign bit 8, magnitude index 0..7."""
    return np.array([(-1.0 if c & 8 else 1.0) * _E2M1[c & 7] for c in range(16)])


_POS4 = np.array(_E2M1)


def e2m1_encode(x) -> np.ndarray:
    """Nearest E2M1 value, ties to the even code, magnitudes saturated at 6."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), 6.0)
    hi = np.searchsorted(_POS4, a, side="left").clip(0, 7)
    lo = (hi - 1).clip(0, 7)
    dlo, dhi = a - _POS4[lo], _POS4[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a == 0.0, 0, code)
    return np.where(x < 0, code | 8, code).astype(np.uint8)


def smallest_exponent(amax: float, top: float) -> int:
    """Smallest e with top * 2^e >= amax (amax > 0)."""
    e = math.ceil(math.log2(amax / top)) - 1
    while top * 2.0 ** e < amax:
        e += 1
    return e


def mx4_quantize_ref(x, rule: str = "6") -> tuple:
    """x [..., D] -> (codes uint8 [..., D] (one code per element, unpacked), exps int [..., D/32]).
    rule "4over6": per block the better of the max-to-6 and max-to-4 scales by squared error;
    rule "6": always max-to-6."""
    x = np.asarray(x, dtype=np.float64)
    lead, D = x.shape[:-1], x.shape[-1]
    assert D % MX_BLOCK == 0
    xb = x.reshape(-1, D // MX_BLOCK, MX_BLOCK)
    dec = e2m1_decode_table()
    codes = np.zeros(xb.shape, dtype=np.uint8)
    exps = np.zeros(xb.shape[:2], dtype=np.int64)
    for r in range(xb.shape[0]):
        for b in range(xb.shape[1]):
            blk = xb[r, b]
            amax = float(np.abs(blk).max())
            if amax == 0.0:
                continue
            e6 = max(smallest_exponent(amax, 6.0), -127)
            best = None
            for e in ([e6, max(smallest_exponent(amax, 4.0), -127)] if rule == "4over6" else [e6]):
                c = e2m1_encode(blk / 2.0 ** e)
                err = math.fsum((dec[c] * 2.0 ** e - blk) ** 2)
                if best is None or err < best[0]:
                    best = (err, e, c)
            exps[r, b] = best[1]
            codes[r, b] = best[2]
    return codes.reshape(*lead, D), exps.reshape(*lead, D // MX_BLOCK)


def mx4_dequantize_ref(codes, exps) -> np.ndarray:
    """E2M1(code) * 2^e of the element's block, [..., D]."""
    codes = np.asarray(codes)
    D = codes.shape[-1]
    scale = np.repeat(np.ldexp(1.0, np.asarray(exps)), MX_BLOCK, axis=-1)
    return e2m1_decode_table()[codes] * scale[..., :D]


def fp4_attention_ref(q_codes, q_exps, k_codes, k_exps, v_codes, vscale, vmean, idx, counts, group: int,
                      scale: float, tie_rel: float = 0.0):
    """The FP8 value path with scores from the dequantised FP4 queries and keys: the block-scaled
    product of the blog is the exact dot product of the dequantised vectors.  tie_rel: as in
    fp8_attention_ref (then also the per-row slacks and loose rows)."""
    return fp8_attention_ref(mx4_dequantize_ref(q_codes, q_exps), mx4_dequantize_ref(k_codes, k_exps), v_codes,
                             vscale, vmean, idx, counts, group, scale, tie_rel=tie_rel)
