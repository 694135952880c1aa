"""Each copy of the oracle with one planted mistake must fail at least one pin.

The mutants are built on the CPU from the oracle's own source text with a
single textual change, executed in a fresh namespace.  This shows that the pins
in oracle_pins.py would catch a dropped term, a wrong sign or index, or a
transposed or swapped operand in the oracle.
"""
import importlib
import inspect
import types

import numpy as np
import pytest

import oracle_pins as pins


def _mutant(modname, old, new):
    mod = importlib.import_module(modname)
    src = inspect.getsource(mod)
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    src = src.replace(old, new, 1)
    m = types.ModuleType(modname + "_mutant")
    m.__dict__["__name__"] = modname + "_mutant"
    exec(compile(src, modname + "_mutant", "exec"), m.__dict__)
    return m


def _caught(checks):
    for check in checks:
        try:
            with np.errstate(all="ignore"):
                check()
        except Exception:     # an assertion or a crash both expose the mutant
            return True
    return False


FWD_MUTANTS = [
    ("scale dropped", "S = (q[b, h, r0:r1] @ k[b, h].T) * scale", "S = (q[b, h, r0:r1] @ k[b, h].T)"),
    ("masked full softmax (no renormalisation)",
     "S[:, ~keep] = -np.inf\n    P, lse = _softmax_rows(S)",
     "P, lse = _softmax_rows(S)\n    P[:, ~keep] = 0.0"),
    ("no max subtraction", "E = np.exp(S - m_safe)", "E = np.exp(S)"),
    ("lse without the max term", "m_safe[:, 0] + np.log(", "np.log("),
    ("softmax over the wrong axis", "m = S.max(axis=1, keepdims=True)", "m = S.max(axis=0, keepdims=True)"),
    ("keys reversed (wrong index)", "S = (q[b, h, r0:r1] @ k[b, h].T)", "S = (q[b, h, r0:r1] @ k[b, h][::-1].T)"),
    ("last kept key dropped", "J = np.asarray(idx[b, h, g, :c], dtype=np.int64)",
     "J = np.asarray(idx[b, h, g, :max(c - 1, 1)], dtype=np.int64)"),
    ("group rows shifted", "r0, r1 = g * group, min((g + 1) * group, Nq)\n    c =",
     "r0, r1 = max(g * group - 1, 0), min((g + 1) * group, Nq) - (1 if g else 0)\n    c ="),
    ("V rows reversed", "out[b, h, r0:r1] = P @ v[b, h]", "out[b, h, r0:r1] = P @ v[b, h][::-1]"),
    ("wrong sign in exponent", "E = np.exp(S - m_safe)", "E = np.exp(m_safe - S)"),
]

MASK_MUTANTS = [
    ("tail mean divides by M", "out[:, :, g] = q[:, :, r0:r1].sum(axis=2) / (r1 - r0)",
     "out[:, :, g] = q[:, :, r0:r1].sum(axis=2) / group"),
    ("score scale dropped", "return np.matmul(qm, np.swapaxes(k, -1, -2)) * scale",
     "return np.matmul(qm, np.swapaxes(k, -1, -2))"),
    ("keys transposed with groups", "return np.matmul(qm, np.swapaxes(k, -1, -2)) * scale",
     "return np.swapaxes(np.matmul(k, np.swapaxes(qm, -1, -2)), -1, -2)[..., ::-1] * scale"),
    ("top-k ties to the higher index", "np.lexsort((np.arange(n), -s_row))", "np.lexsort((-np.arange(n), -s_row))"),
    ("top-k keeps one too few", "kept = order[:topk]", "kept = order[:max(topk - 1, 1)]"),
    ("top-k keeps the lowest scores", "np.lexsort((np.arange(n), -s_row))", "np.lexsort((np.arange(n), s_row))"),
    ("threshold with the wrong sign of ln tau", "lse + math.log(tau)", "lse - math.log(tau)"),
    ("lse without the max term", "lse = m + math.log(", "lse = math.log("),
    ("fallback keeps the arg-min", "kept = np.array([int(np.argmax(s_row))])", "kept = np.array([int(np.argmin(s_row))])"),
    ("mean over the wrong axis", "q[:, :, r0:r1].sum(axis=2)", "q[:, :, r0:r1].sum(axis=3, keepdims=False)[..., None]"),
]


CACHED_MUTANTS = [
    ("min over the group's queries", "out[(b, h, g)] = (s - l_rows[:, None]).max(axis=0)",
     "out[(b, h, g)] = (s - l_rows[:, None]).min(axis=0)"),
    ("lse not subtracted", "out[(b, h, g)] = (s - l_rows[:, None]).max(axis=0)", "out[(b, h, g)] = s.max(axis=0)"),
    ("lse over the queries", "mx = s.max(axis=1, keepdims=True)\n            l_rows = (mx + np.log(np.exp(s - mx).sum(axis=1, keepdims=True)))[:, 0]",
     "mx = s.max(axis=0, keepdims=True)\n            l_rows = (mx + np.log(np.exp(s - mx).sum(axis=0, keepdims=True)))[0, :s.shape[0]]"),
    ("score scale dropped", "s = np.matmul(q[b, h, r0:r1], k[b, h].T) * scale", "s = np.matmul(q[b, h, r0:r1], k[b, h].T)"),
    ("group rows shifted", "r0, r1 = g * group, min((g + 1) * group, Nq)\n        s =",
     "r0, r1 = max(g * group - 1, 0), min((g + 1) * group, Nq) - (1 if g else 0)\n        s ="),
    ("wrong sign of ln tau", "log_tau = -math.inf if tau <= 0.0 else math.log(tau)", "log_tau = -math.inf if tau <= 0.0 else -math.log(tau)"),
    ("row lse without the max term", "return (m + np.log(", "return (np.log("),
]


DELTA_MUTANTS = [
    ("column max instead of sum", "out[(b, h, g)] = np.exp(s - lse[b, h, r0:r1, None]).sum(axis=0)",
     "out[(b, h, g)] = np.exp(s - lse[b, h, r0:r1, None]).max(axis=0)"),
    ("column sums without lse", "out[(b, h, g)] = np.exp(s - lse[b, h, r0:r1, None]).sum(axis=0)",
     "out[(b, h, g)] = np.exp(s).sum(axis=0)"),
    ("column sums over the wrong rows", "r0, r1 = g * group, min((g + 1) * group, Nq)\n        s = np.matmul(q[b, h, r0:r1], k[b, h].T) * scale\n        out[(b, h, g)] = np.exp(",
     "r0, r1 = g * group, min((g + 1) * group + 1, Nq)\n        s = np.matmul(q[b, h, r0:r1], k[b, h].T) * scale\n        out[(b, h, g)] = np.exp("),
    ("top-k ties to the higher index", "order = np.lexsort((np.arange(Nk), -row))", "order = np.lexsort((-np.arange(Nk), -row))"),
    ("top-k keeps the smallest sums", "order = np.lexsort((np.arange(Nk), -row))", "order = np.lexsort((np.arange(Nk), row))"),
    ("restricted softmax (renormalised)", "fresh[b, h, r0:r1] = np.matmul(np.exp(s - lse[b, h, r0:r1, None]), v[b, h, J])",
     "e = np.exp(s - lse[b, h, r0:r1, None]); fresh[b, h, r0:r1] = np.matmul(e / e.sum(axis=1, keepdims=True), v[b, h, J])"),
    ("stale part added", "out = np.asarray(out_prev, dtype=np.float64) - np.asarray(fresh_prev, dtype=np.float64) + fresh",
     "out = np.asarray(out_prev, dtype=np.float64) + np.asarray(fresh_prev, dtype=np.float64) - fresh"),
    ("delta without lse", "np.exp(s - lse[b, h, r0:r1, None]), v[b, h, J]", "np.exp(s), v[b, h, J]"),
    ("V rows not gathered", "v[b, h, J])", "v[b, h, :J.size])"),
    ("delta scale dropped", "s = np.matmul(q[b, h, r0:r1], k[b, h, J].T) * scale", "s = np.matmul(q[b, h, r0:r1], k[b, h, J].T)"),
]


FP8_MUTANTS = [
    ("ExpCast bias without the 2^8 scale", "EXPCAST_BIAS = 56.0 + 64.0", "EXPCAST_BIAS = 56.0 + 56.0"),
    ("ExpCast truncates", "b = np.rint(y)", "b = np.floor(y)"),
    ("reference point off the 1/8 grid", "m8 = np.ceil(8.0 * bm)\n", "m8 = 8.0 * bm\n"),
    ("reference point kept past saturation", "RESCALE_SLACK = 13.0 / 16.0", "RESCALE_SLACK = 2.0"),
    ("reference point moved by a fraction", "m8 + 8.0 * np.ceil(bm - m8 / 8.0)", "np.ceil(8.0 * bm)"),
    ("earlier blocks not rescaled", "o *= alpha[:, None]", "o *= 1.0"),
    ("block mean not restored", "return _DEC[codes] * scale[:, :, None, :] + mean[:, :, np.arange(N) // VS_BLOCK, :]",
     "return _DEC[codes] * scale[:, :, None, :]"),
    ("one mean per head", "VS_BLOCK = 128", "VS_BLOCK = 1 << 20"),
    ("mean not rounded to bf16", "mean[b, h, blk, d] = bf16_round(math.fsum(rows[:, d]) / rows.shape[0])",
     "mean[b, h, blk, d] = math.fsum(rows[:, d]) / rows.shape[0]"),
    ("channel scale not a power of two", "scale = np.ldexp(1.0, e)", "scale = np.where(amax > 0, amax / 448.0, 1.0)"),
    ("lse without the 2^-8", "(np.log2(l) + m8 / 8.0 - 8.0) / log2e", "(np.log2(l) + m8 / 8.0) / log2e"),
    ("E4M3 exponent bias 8", "else (1.0 + m / 8.0) * 2.0 ** (e - 7)", "else (1.0 + m / 8.0) * 2.0 ** (e - 8)"),
    ("ties away from even", "((dhi == dlo) & (hi % 2 == 0))", "(dhi == dlo)"),
    ("bf16 ties away from even", "if frac > 0.5 or (frac == 0.5 and r % 2 == 1):", "if frac >= 0.5:"),
]


@pytest.mark.parametrize("name,old,new", FP8_MUTANTS, ids=[m[0] for m in FP8_MUTANTS])
def test_fp8_mutant_is_caught(name, old, new):
    m = _mutant("oracle.fp8", old, new)
    checks = [lambda: pins.check_e4m3(m.e4m3_decode_table, m.e4m3_encode),
              lambda: pins.check_expcast(m.expcast_byte, m.e4m3_decode_table),
              lambda: pins.check_vsmooth(m.vsmooth_quantize_ref, m.e4m3_decode_table),
              lambda: pins.check_fp8_attention(m.vsmooth_quantize_ref, m.fp8_attention_ref, m.e4m3_decode_table,
                                               m.dequantize_ref),
              lambda: pins.check_fp8_reference_point(m.vsmooth_quantize_ref, m.fp8_attention_ref, m.e4m3_decode_table,
                                                     m.dequantize_ref)]
    assert _caught(checks), f"no pin catches the planted mistake: {name}"


REFERENCE_POINT_MUTANTS = ["reference point off the 1/8 grid", "reference point kept past saturation",
                           "reference point moved by a fraction", "earlier blocks not rescaled"]


@pytest.mark.parametrize("name", REFERENCE_POINT_MUTANTS)
def test_reference_point_mutant_fails_the_one_pass_pin(name):
    """The reference-point rule is pinned by a check that does not restate the blocked loop: each of these
    mutants fails the one-pass ExpCast equivalence on its own."""
    old, new = next((o, n) for (nm, o, n) in FP8_MUTANTS if nm == name)
    m = _mutant("oracle.fp8", old, new)
    assert _caught([lambda: pins.check_fp8_reference_point(m.vsmooth_quantize_ref, m.fp8_attention_ref,
                                                           m.e4m3_decode_table, m.dequantize_ref)]), name


FP4_MUTANTS = [
    ("E2M1 level 3 read as 2.5", "_E2M1 = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)",
     "_E2M1 = (0.0, 0.5, 1.0, 1.5, 2.0, 2.5, 4.0, 6.0)"),
    ("ties away from even", "((dhi == dlo) & (hi % 2 == 0))", "(dhi == dlo)"),
    ("maximum scaled to 4", "e6 = max(smallest_exponent(amax, 6.0), -127)", "e6 = max(smallest_exponent(amax, 4.0), -127)"),
    ("scale one binade too small", "    e = math.ceil(math.log2(amax / top)) - 1\n    while top * 2.0 ** e < amax:",
     "    e = math.ceil(math.log2(amax / top)) - 2\n    while top * 2.0 ** e < amax / 2:"),
    ("blocks of 16", "MX_BLOCK = 32", "MX_BLOCK = 16"),
    ("keys not dequantised", "mx4_dequantize_ref(k_codes, k_exps), v_codes", "k_codes.astype(float), v_codes"),
]


@pytest.mark.parametrize("name,old,new", FP4_MUTANTS, ids=[m[0] for m in FP4_MUTANTS])
def test_fp4_mutant_is_caught(name, old, new):
    m = _mutant("oracle.fp4", old, new)
    import oracle
    checks = [lambda: pins.check_e2m1(m.e2m1_decode_table, m.e2m1_encode),
              lambda: pins.check_mx4(m.mx4_quantize_ref, m.mx4_dequantize_ref, m.e2m1_decode_table),
              lambda: pins.check_fp4_attention(m.mx4_quantize_ref, m.fp4_attention_ref, oracle.fp8_attention_ref,
                                               oracle.vsmooth_quantize_ref, m.e2m1_decode_table)]
    assert _caught(checks), f"no pin catches the planted mistake: {name}"


@pytest.mark.parametrize("name,old,new", DELTA_MUTANTS, ids=[m[0] for m in DELTA_MUTANTS])
def test_delta_mutant_is_caught(name, old, new):
    m = _mutant("oracle.cached", old, new)
    checks = [lambda: pins.check_colsum(m.colsum_scores_ref, m.colsum_mask_ref, m.row_lse_ref),
              lambda: pins.check_delta(m.delta_fresh_ref, m.delta_forward_ref)]
    assert _caught(checks), f"no pin catches the planted mistake: {name}"


@pytest.mark.parametrize("name,old,new", CACHED_MUTANTS, ids=[m[0] for m in CACHED_MUTANTS])
def test_cached_mutant_is_caught(name, old, new):
    m = _mutant("oracle.cached", old, new)
    checks = [lambda: pins.check_cached_brute_force(m.cached_mask_ref),
              lambda: pins.check_cached_properties(m.cached_mask_ref, m.row_lse_ref)]
    assert _caught(checks), f"no pin catches the planted mistake: {name}"


@pytest.mark.parametrize("name,old,new", FWD_MUTANTS, ids=[m[0] for m in FWD_MUTANTS])
def test_forward_mutant_is_caught(name, old, new):
    m = _mutant("oracle.attention", old, new)
    checks = [lambda: pins.check_all_keys_equals_library(m.sparse_attention_ref),
              lambda: pins.check_brute_force_tiny(m.sparse_attention_ref),
              lambda: pins.check_closed_forms(m.sparse_attention_ref),
              lambda: pins.check_invariants(m.sparse_attention_ref, m.sparse_attention_probs_ref)]
    assert _caught(checks), f"no pin catches the planted mistake: {name}"


@pytest.mark.parametrize("name,old,new", MASK_MUTANTS, ids=[m[0] for m in MASK_MUTANTS])
def test_mask_mutant_is_caught(name, old, new):
    m = _mutant("oracle.mask", old, new)
    checks = [lambda: pins.check_group_mean(m.group_mean_ref),
              lambda: pins.check_group_scores(m.group_scores_ref),
              lambda: pins.check_topk(m.topk_select_ref),
              lambda: pins.check_thresh(m.thresh_select_ref)]
    assert _caught(checks), f"no pin catches the planted mistake: {name}"
