"""fp64 oracle of the FP8 value path: V-Smooth quantisation of V and ExpCast probabilities.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
library path.

V-Smart/ExpCast summary (itinai.com), its second and third paragraphs:
  * V-Smooth: the mean of each 128-token block of V is subtracted, only the residual is
    quantised to E4M3 with a scale per channel, and the mean comes back through the row
    sum the online softmax already keeps; the means cost 0.125 bit per element, i.e. one
    16-bit (bf16) value per channel and block of 128 tokens;
  * ExpCast-FP8: an E4M3 byte is close to 8 log2(v) + 56, so the probability byte is one
    multiply-add of the log-domain score plus a constant, with no exponential and no cast.

Readings where the summary is silent:
  * block mean: the exact mean of the block's tokens (the last block may be shorter),
    rounded to bf16 (nearest, ties to even); the residual r = v - mean in fp32;
  * channel scale: the power of two s = 2^e with the smallest e such that 448 s >= max |r|
    over all tokens of the head (s = 1 when the residual is 0), so r / s is exact and
    lands in [-448, 448]; codes = E4M3(r / s), nearest with ties to even;
  * probabilities: ExpCast inside the online softmax (LongLive DiT blog, "Online Softmax"),
    which runs over blocks of 64 listed keys in list order.  For the byte to be one
    multiply-add of the raw score plus an integer, the subtracted reference point m of a row
    must lie on the 1/8 grid of log2 units; for the sums gathered before a move to be rescaled
    exactly, a move must be by whole log2 units (then a byte before the move, scaled, is the
    byte after it).  The one free choice left is the grid phase, taken from the first block:
    m = ceil8(block max); a later block moves it only when one of its bytes would pass 126,
    the largest finite code (block max > m + 13/16), and then by the smallest whole number of
    log2 units that brings the block max to or below it.  While every byte is a normal code
    the result is therefore the one-pass ExpCast at that phase, whatever the block size and
    wherever the moves fall.  The byte is round-half-even(8 (x - m) + 120), set to 0 below 0:
    the bias 56 with the probability scaled by 2^8, so the row's largest weight sits near 256
    and only weights below 2^-14 of it fall into the subnormal codes;
  * the row sum adds the decoded probabilities; out = sum_j p_j (s v8_j + mean_b(j)) / l;
    lse = ln(l 2^(m - 8)).
Where a decision is integer (a code, a byte), the oracle takes it on the values the
definition above gives: fp32 for the residual, fp64 for the scores.

E4M3 ("fn" variant, OCP 8-bit floating point specification): 1 sign, 4 exponent bits
(bias 7), 3 mantissa bits; exponent 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN;
no infinities; largest normal 448.
"""
from __future__ import annotations

import math

import numpy as np

FP8_BLOCK = 64          # listed keys per online-softmax block
VS_BLOCK = 128          # tokens per V-Smooth mean block
EXPCAST_BIAS = 56.0 + 64.0      # E4M3 exponent bias 7 (x 8) plus the 2^8 scale
RESCALE_SLACK = 13.0 / 16.0     # a block max past m + 13/16 would give a byte above 126


def e4m3_decode_table() -> np.ndarray:
    """value of each of the 256 codes (NaN for S.1111.111)."""
    t = np.empty(256)
    for c in range(256):
        s, e, m = c >> 7, (c >> 3) & 15, c & 7
        if e == 15 and m == 7:
            t[c] = np.nan
            continue
        v = (m / 8.0) * 2.0 ** -6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
        t[c] = -v if s else v
    return t


_DEC = e4m3_decode_table()
_POS = np.array([_DEC[c] for c in range(127)])          # non-negative codes 0..126 (0 .. 448), ascending


def e4m3_encode(x) -> np.ndarray:
    """Round to the nearest E4M3 value, ties to the even code; saturate at +-448."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), 448.0)
    hi = np.searchsorted(_POS, a, side="left").clip(0, 126)      # first code with value >= a
    lo = (hi - 1).clip(0, 126)
    dlo, dhi = a - _POS[lo], _POS[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(a == 0.0, 0, code).astype(np.uint8)
    return np.where(x < 0, code | 0x80, code).astype(np.uint8)


def bf16_round(x: float) -> float:
    """Nearest bf16 value (8 significant bits), ties to even; x finite."""
    if x == 0.0:
        return 0.0
    f, e = math.frexp(x)                 # x = f 2^e, 0.5 <= |f| < 1
    y = f * 256.0                        # 8 significant bits above the point
    r = math.floor(y)
    frac = y - r
    if frac > 0.5 or (frac == 0.5 and r % 2 == 1):
        r += 1
    return math.ldexp(r, e - 8)


def channel_scale_exponent(amax: float) -> int:
    """Smallest e with 448 * 2^e >= amax (0 for amax == 0)."""
    if amax == 0.0:
        return 0
    e = math.ceil(math.log2(amax / 448.0)) - 1
    while 448.0 * 2.0 ** e < amax:
        e += 1
    return e


def vsmooth_quantize_ref(v) -> tuple:
    """v [B,H,N,D] (bf16 values) -> (codes uint8 [B,H,N,D], scale [B,H,D], mean [B,H,NB,D]),
    NB = ceil(N / 128): per block and channel the exact token mean rounded to bf16, the fp32
    residual, a power-of-two channel scale and the E4M3 codes of residual / scale."""
    v = np.asarray(v, dtype=np.float64)
    B, H, N, D = v.shape
    NB = -(-N // VS_BLOCK)
    mean = np.zeros((B, H, NB, D))
    for b in range(B):
        for h in range(H):
            for blk in range(NB):
                rows = v[b, h, blk * VS_BLOCK:min((blk + 1) * VS_BLOCK, N)]
                for d in range(D):
                    mean[b, h, blk, d] = bf16_round(math.fsum(rows[:, d]) / rows.shape[0])
    blk_of = np.arange(N) // VS_BLOCK
    r = v.astype(np.float32) - mean[:, :, blk_of, :].astype(np.float32)      # fp32 residual
    amax = np.abs(r).max(axis=2).astype(np.float64)
    e = np.vectorize(channel_scale_exponent)(amax)
    scale = np.ldexp(1.0, e)
    codes = e4m3_encode(r.astype(np.float64) / scale[:, :, None, :])
    return codes, scale, mean


def expcast_byte(x) -> np.ndarray:
    """ExpCast: E4M3 code of 2^(x + 8) as round-half-even(8 x + 120), 0 below, at most 126."""
    y = 8.0 * np.asarray(x, dtype=np.float64) + EXPCAST_BIAS
    b = np.rint(y)                      # numpy rint rounds half to even
    return np.clip(b, 0, 126).astype(np.uint8)


def dequantize_ref(codes, scale, mean) -> np.ndarray:
    """s * E4M3(code) + mean of the token's block, [B,H,N,D]."""
    codes = np.asarray(codes)
    N = codes.shape[2]
    return _DEC[codes] * scale[:, :, None, :] + mean[:, :, np.arange(N) // VS_BLOCK, :]


def fp8_attention_ref(q, k, codes, vscale, vmean, idx, counts, group: int, scale: float, block: int = FP8_BLOCK,
                      tie_rel: float = 0.0):
    """out, lse of the FP8 value path over per-group key lists.

    For each group and its listed keys J (list order), blocks of `block` keys: s2 = scale q.k log2 e
    (fp64); the row's reference point m8 = 8 m (an integer) is ceil(8 max) of the first block and moves
    by 8 ceil(max - m) only when a block's max exceeds m + 13/16; P-bytes = expcast(s2 - m); weights
    gathered earlier are scaled by 2^(m_old - m_new); O += decode(P) @ Vhat[J], l += sum decode(P), with
    Vhat = scale * E4M3(code) + block mean.  out = O / l; lse = ln(l) + (m - 8) ln 2.
    c = 0 gives out = 0, lse = -inf.

    Rounding ties.  The bytes and the first reference point are integer decisions on the scores.  A
    computation whose scores carry an error up to tie_rel * scale * log2 e * sum_d |q_d k_d| (for example
    fp32 dot products: tie_rel = (D + 2) 2^-24) may take a decision whose value lies that close to its
    boundary the other way; both results are ExpCast results of the same scores, one code apart in that
    byte (V-Smart/ExpCast summary, third paragraph).  With tie_rel > 0 the function also returns, per
    query row: out_slack, a bound on max_d |out' - out| over every such choice of the byte decisions
    (a byte rounded to the other neighbour changes its weight by dp_j, the difference of the two decoded
    codes, a byte of 127 standing for a move of the reference point: twice the code 8 below; then
    out' - out = sum_j e_j (Vhat_j - out) / (l + sum_j e_j) with |e_j| <= dp_j), as
    max_d sum_j dp_j |Vhat_jd - out_d| / (l - sum_j dp_j), all weights in the row's final frame;
    lse_slack = -ln(1 - sum_j dp_j / l); and loose, the rows whose first reference point ceil(8 max) is
    such a decision (the neighbouring phase moves every byte by one code, which no per-key bound covers).
    A move by one more whole log2 unit than needed rescales exactly and changes nothing but weights
    below the subnormal range, so it is not counted.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    B, H, Nq, D = q.shape
    G = -(-Nq // group)
    log2e = 1.0 / math.log(2.0)
    vhat = dequantize_ref(codes, vscale, vmean)
    Dv = vhat.shape[-1]
    out = np.zeros((B, H, Nq, Dv))
    lse = np.full((B, H, Nq), -np.inf)
    ties = tie_rel > 0.0
    out_slack = np.zeros((B, H, Nq))
    lse_slack = np.zeros((B, H, Nq))
    loose = np.zeros((B, H, Nq), dtype=bool)
    for b in range(B):
        for h in range(H):
            for g in range(G):
                r0, r1 = g * group, min((g + 1) * group, Nq)
                c = int(counts[b, h, g])
                if c == 0:
                    continue
                J = np.asarray(idx[b, h, g, :c], dtype=np.int64)
                s2 = np.matmul(q[b, h, r0:r1], k[b, h, J].T) * scale * log2e     # [rows, c], log2 units
                rows = r1 - r0
                m8 = np.zeros(rows)
                o = np.zeros((rows, Dv))
                l = np.zeros(rows)
                if ties:
                    # half-width of the uncertain window of each byte's pre-rounding value 8 (s2 - m) + 120
                    win = 8.0 * tie_rel * scale * log2e * np.matmul(np.abs(q[b, h, r0:r1]), np.abs(k[b, h, J]).T)
                    near_ties = []                                      # (row, list position, dp, m8 then)
                for j0 in range(0, c, block):
                    sb = s2[:, j0:j0 + block]
                    bm = sb.max(axis=1)
                    if j0 == 0:
                        m8 = np.ceil(8.0 * bm)
                        if ties:
                            wmax = win[np.arange(rows), sb.argmax(axis=1)]
                            x8 = 8.0 * bm
                            loose[b, h, r0:r1] = (np.ceil(x8) - x8 < wmax) | (x8 - np.floor(x8) < wmax)
                    else:
                        move = bm > m8 / 8.0 + RESCALE_SLACK
                        m8new = np.where(move, m8 + 8.0 * np.ceil(bm - m8 / 8.0), m8)
                        alpha = np.exp2((m8 - m8new) / 8.0)
                        o *= alpha[:, None]
                        l *= alpha
                        m8 = m8new
                    byte = expcast_byte(sb - m8[:, None] / 8.0)
                    p = _DEC[byte]
                    o += p @ vhat[b, h, J[j0:j0 + block]]
                    l += p.sum(axis=1)
                    if ties:
                        y = sb * 8.0 - m8[:, None] + EXPCAST_BIAS
                        near = np.abs(y - np.floor(y) - 0.5) < win[:, j0:j0 + block]
                        other = np.where(np.rint(y) == np.floor(y), np.floor(y) + 1.0, np.floor(y))
                        other = np.clip(other, 0.0, 127.0).astype(np.int64)
                        p_other = np.where(other == 127, 2.0 * _DEC[119], _DEC[np.minimum(other, 126)])
                        dp = np.where(near, np.abs(p_other - p), 0.0)
                        for rr, jj in zip(*np.nonzero(dp)):
                            near_ties.append((rr, j0 + jj, dp[rr, jj], m8[rr]))
                out[b, h, r0:r1] = o / l[:, None]
                lse[b, h, r0:r1] = (np.log2(l) + m8 / 8.0 - 8.0) / log2e
                if ties:
                    dsum = np.zeros(rows)
                    dvec = np.zeros((rows, Dv))
                    for rr, jj, d, m8_then in near_ties:
                        d *= np.exp2((m8_then - m8[rr]) / 8.0)          # into the row's final frame
                        dsum[rr] += d
                        dvec[rr] += d * np.abs(vhat[b, h, J[jj]] - out[b, h, r0 + rr])
                    frac = np.minimum(dsum / l, 0.999)
                    out_slack[b, h, r0:r1] = dvec.max(axis=1) / (l * (1.0 - frac))
                    lse_slack[b, h, r0:r1] = -np.log1p(-frac)
    if ties:
        return out, lse, out_slack, lse_slack, loose
    return out, lse
