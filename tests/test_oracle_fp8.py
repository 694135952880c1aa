"""The FP8 value-path oracle (E4M3, V-Smooth, ExpCast, FP8 attention) against its pins (CPU)."""
import oracle
import oracle_pins as pins


def test_e4m3():
    pins.check_e4m3(oracle.e4m3_decode_table, oracle.e4m3_encode)


def test_expcast():
    pins.check_expcast(oracle.expcast_byte, oracle.e4m3_decode_table)


def test_vsmooth():
    pins.check_vsmooth(oracle.vsmooth_quantize_ref, oracle.e4m3_decode_table)


def test_fp8_attention():
    pins.check_fp8_attention(oracle.vsmooth_quantize_ref, oracle.fp8_attention_ref, oracle.e4m3_decode_table,
                             oracle.dequantize_ref)


def test_fp8_reference_point():
    pins.check_fp8_reference_point(oracle.vsmooth_quantize_ref, oracle.fp8_attention_ref, oracle.e4m3_decode_table,
                                   oracle.dequantize_ref)


def test_fp8_tie_slack_bounds_other_roundings():
    """fp8_attention_ref's tie slacks bound the results of taking its near-tie decisions the other way.
    Scaling each key by (1 + d_j), |d_j| < tie_rel, moves every score by less than tie_rel * sum_d |q_d k_d|
    (the window the slacks are computed for); the ExpCast output depends on the scores only through its
    integer decisions (the bytes, the reference point), so outside the loose rows every perturbed result
    lies within the slacks of the unperturbed one.  The windows are wide enough here that many bytes
    change, so the check is not empty."""
    import numpy as np
    rng = np.random.default_rng(11)
    B, H, Nq, Nk, D, group, c = 1, 2, 96, 900, 64, 32, 640
    q = rng.standard_normal((B, H, Nq, D)) * 2.0
    k = rng.standard_normal((B, H, Nk, D))
    off = np.repeat(rng.uniform(-2, 2, size=(H, -(-Nk // 128), 1)), 128, axis=1)[:, :Nk][None]
    codes, vs, vm = oracle.vsmooth_quantize_ref(rng.standard_normal((B, H, Nk, D)) + off)
    G = -(-Nq // group)
    counts = np.full((B, H, G), c, dtype=np.int32)
    idx = np.stack([np.stack([np.sort(rng.choice(Nk, c, replace=False)) for _ in range(G)]) for _ in range(H)])[None]
    scale, tie_rel = 1.0 / np.sqrt(D), 1e-3
    out, lse, oslack, lslack, loose = oracle.fp8_attention_ref(q, k, codes, vs, vm, idx, counts, group, scale,
                                                               tie_rel=tie_rel)
    assert loose.sum() < loose.size // 4
    ok = ~loose
    changed = 0
    for _ in range(4):
        d = rng.uniform(-tie_rel, tie_rel, size=(B, H, Nk, 1)) * 0.999
        o2, l2 = oracle.fp8_attention_ref(q, k * (1.0 + d), codes, vs, vm, idx, counts, group, scale)
        diff = np.abs(o2 - out).max(axis=-1)
        assert np.all(diff[ok] <= oslack[ok] + 1e-9), f"output moved by {(diff - oslack)[ok].max():.3g} past its slack"
        assert np.all(np.abs(l2 - lse)[ok] <= lslack[ok] + 1e-12)
        changed += int((diff[ok] > 1e-9).sum())
    assert changed > 50, f"only {changed} rows changed"
