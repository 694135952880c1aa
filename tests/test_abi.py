"""The C ABI library: loads, exports every declared symbol, rejects bad arguments on the host.

CPU only: every call here fails validation before any HIP call is made.
"""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sattn.h")

OK, ERR_NULL, ERR_SHAPE, ERR_UNSUPPORTED, ERR_ARG, ERR_WORKSPACE, ERR_HIP, ERR_INDEX = range(8)


@pytest.fixture(scope="module")
def lib():
    import sparse_self_attention_amd as sattn
    if not os.path.exists(sattn.library_path()):
        from sparse_self_attention_amd import build
        build.build()
    return sattn._load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w]+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert {"sattn_mask", "sattn_forward", "attn_forward", "sattn_mask_workspace_bytes", "sattn_cached_mask",
            "sattn_colsum_mask", "sattn_delta_forward", "sattn_vsmooth_quantize", "sattn_fp8_forward",
            "sattn_vsmooth_workspace_bytes", "sattn_vsmooth_mean_stride", "sattn_mx4_quantize", "sattn_fp4_forward",
            "sattn_strerror", "sattn_last_error", "sattn_voxel_permutation", "sattn_permute_tokens",
            "sattn_forward_split", "sattn_forward_split_workspace_bytes"} <= set(names)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in sattn.h but not exported"


def test_strerror(lib):
    for s in range(8):
        assert lib.sattn_strerror(s)
    assert lib.sattn_strerror(99) == b"unknown status"


P = ctypes.c_void_p
FAKE = P(4096)   # non-NULL, aligned; never dereferenced because validation fails first


def fwd(lib, q=FAKE, k=FAKE, v=FAKE, idx=FAKE, counts=FAKE, cap=64, B=1, H=1, Nq=128, Nk=128, D=128, group=128,
        scale=0.1, out=FAKE, out_dtype=0, lse=P(0)):
    return lib.sattn_forward(q, k, v, idx, counts, cap, B, H, Nq, Nk, D, group, scale, out, out_dtype, lse, P(0))


def msk(lib, q=FAKE, k=FAKE, B=1, H=1, Nq=128, Nk=128, D=128, group=128, mode=0, topk=16, thresh=0.0, scale=0.1,
        idx=FAKE, counts=FAKE, cap=16, ws=FAKE, ws_bytes=1 << 40):
    return lib.sattn_mask(q, k, B, H, Nq, Nk, D, group, mode, topk, thresh, scale, idx, counts, cap, ws, ws_bytes,
                          P(0))


# Each case changes one argument of an otherwise well-formed call so that validation must fail
# before any launch; the D/group/mode cases make sure a later check cannot be reached.
FWD_CASES = [
    (dict(q=P(0)), ERR_NULL), (dict(idx=P(0)), ERR_NULL), (dict(out=P(0)), ERR_NULL), (dict(counts=P(0)), ERR_NULL),
    (dict(B=0), ERR_SHAPE), (dict(Nq=0), ERR_SHAPE), (dict(Nk=-1), ERR_SHAPE),
    (dict(D=96), ERR_UNSUPPORTED), (dict(D=256), ERR_UNSUPPORTED),
    (dict(group=8), ERR_UNSUPPORTED), (dict(group=100), ERR_UNSUPPORTED), (dict(group=272), ERR_UNSUPPORTED),
    (dict(scale=0.0), ERR_ARG), (dict(scale=float("nan")), ERR_ARG), (dict(scale=float("inf")), ERR_ARG),
    (dict(cap=0), ERR_ARG), (dict(out_dtype=2), ERR_ARG),
    (dict(q=P(4097)), ERR_ARG), (dict(lse=P(4098)), ERR_ARG),
    (dict(Nk=1 << 23), ERR_SHAPE),
]


@pytest.mark.parametrize("kw,code", FWD_CASES, ids=[str(c[0]) for c in FWD_CASES])
def test_forward_validation(lib, kw, code):
    assert fwd(lib, **kw) == code
    assert lib.sattn_last_error()


def fwd_split(lib, q=FAKE, k=FAKE, v=FAKE, idx=FAKE, counts=FAKE, cap=64, B=1, H=1, Nq=128, Nk=128, D=128, group=128,
              scale=0.1, splits=4, ws=FAKE, ws_bytes=1 << 40, out=FAKE, out_dtype=0, lse=P(0)):
    return lib.sattn_forward_split(q, k, v, idx, counts, cap, B, H, Nq, Nk, D, group, scale, splits, ws, ws_bytes, out,
                                   out_dtype, lse, P(0))


# sattn_forward's checks plus the split count and the workspace
SPLIT_CASES = FWD_CASES + [
    (dict(splits=0), ERR_ARG), (dict(splits=33), ERR_ARG), (dict(ws=P(4104)), ERR_ARG),
    (dict(ws=P(0)), ERR_WORKSPACE), (dict(ws_bytes=1024), ERR_WORKSPACE),
]


@pytest.mark.parametrize("kw,code", SPLIT_CASES, ids=[str(c[0]) for c in SPLIT_CASES])
def test_forward_split_validation(lib, kw, code):
    assert fwd_split(lib, **kw) == code
    assert lib.sattn_last_error()


def test_forward_split_workspace_query(lib):
    # per (row, part): D fp32 partials, then a (max, normaliser) pair; each section 256-byte aligned
    assert lib.sattn_forward_split_workspace_bytes(1, 12, 7040, 128, 4) == 12 * 7040 * 4 * (128 * 4 + 8)
    assert lib.sattn_forward_split_workspace_bytes(1, 1, 10, 64, 3) == 7680 + 256
    for bad in [(0, 1, 10, 64, 2), (1, 1, 10, 96, 2), (1, 1, 10, 64, 0), (1, 1, 10, 64, 33)]:
        assert lib.sattn_forward_split_workspace_bytes(*bad) == 0


MASK_CASES = [
    (dict(q=P(0)), ERR_NULL), (dict(counts=P(0)), ERR_NULL),
    (dict(H=0), ERR_SHAPE), (dict(D=32), ERR_UNSUPPORTED), (dict(group=24), ERR_UNSUPPORTED),
    (dict(Nk=200000), ERR_UNSUPPORTED), (dict(Nk=131073, topk=16), ERR_UNSUPPORTED),
    (dict(mode=2), ERR_ARG), (dict(topk=0), ERR_ARG), (dict(topk=129), ERR_ARG), (dict(cap=15), ERR_ARG),
    (dict(mode=1, thresh=-0.1, cap=128), ERR_ARG), (dict(mode=1, thresh=1.5, cap=128), ERR_ARG),
    (dict(mode=1, thresh=float("nan"), cap=128), ERR_ARG), (dict(mode=1, thresh=0.1, cap=127), ERR_ARG),
    (dict(scale=-1.0), ERR_ARG),
    (dict(ws=P(0)), ERR_WORKSPACE), (dict(ws_bytes=16), ERR_WORKSPACE), (dict(ws=P(4096 + 16)), ERR_WORKSPACE),
]


@pytest.mark.parametrize("kw,code", MASK_CASES, ids=[str(c[0]) for c in MASK_CASES])
def test_mask_validation(lib, kw, code):
    assert msk(lib, **kw) == code


def cmk(lib, q=FAKE, k=FAKE, lse=FAKE, B=1, H=1, Nq=128, Nk=128, D=128, group=128, tau=0.01, scale=0.1,
        idx=FAKE, counts=FAKE, cap=128):
    return lib.sattn_cached_mask(q, k, lse, B, H, Nq, Nk, D, group, tau, scale, idx, counts, cap, P(0))


CACHED_CASES = [
    (dict(q=P(0)), ERR_NULL), (dict(lse=P(0)), ERR_NULL), (dict(idx=P(0)), ERR_NULL), (dict(counts=P(0)), ERR_NULL),
    (dict(Nq=0), ERR_SHAPE), (dict(D=80), ERR_UNSUPPORTED), (dict(group=40), ERR_UNSUPPORTED),
    (dict(Nk=200000), ERR_UNSUPPORTED), (dict(tau=float("nan")), ERR_ARG), (dict(cap=0), ERR_ARG),
    (dict(scale=0.0), ERR_ARG), (dict(k=P(4104)), ERR_ARG), (dict(lse=P(4097)), ERR_ARG),
]


@pytest.mark.parametrize("kw,code", CACHED_CASES, ids=[str(c[0]) for c in CACHED_CASES])
def test_cached_mask_validation(lib, kw, code):
    assert cmk(lib, **kw) == code
    assert lib.sattn_last_error()


def csm(lib, q=FAKE, k=FAKE, lse=FAKE, B=1, H=1, Nq=128, Nk=128, D=128, group=128, topk=16, scale=0.1,
        idx=FAKE, counts=FAKE, cap=16, ws=FAKE, ws_bytes=1 << 40):
    return lib.sattn_colsum_mask(q, k, lse, B, H, Nq, Nk, D, group, topk, scale, idx, counts, cap, ws, ws_bytes, P(0))


COLSUM_CASES = [
    (dict(lse=P(0)), ERR_NULL), (dict(k=P(0)), ERR_NULL), (dict(B=0), ERR_SHAPE), (dict(D=48), ERR_UNSUPPORTED),
    (dict(group=72), ERR_UNSUPPORTED), (dict(Nk=140000), ERR_UNSUPPORTED), (dict(topk=0), ERR_ARG),
    (dict(topk=129), ERR_ARG), (dict(cap=15), ERR_ARG), (dict(scale=float("nan")), ERR_ARG),
    (dict(lse=P(4098)), ERR_ARG), (dict(ws=P(0)), ERR_WORKSPACE), (dict(ws_bytes=8), ERR_WORKSPACE),
]


@pytest.mark.parametrize("kw,code", COLSUM_CASES, ids=[str(c[0]) for c in COLSUM_CASES])
def test_colsum_mask_validation(lib, kw, code):
    assert csm(lib, **kw) == code


def dlt(lib, q=FAKE, k=FAKE, v=FAKE, idx=FAKE, counts=FAKE, cap=64, B=1, H=1, Nq=128, Nk=128, D=128, group=128,
        scale=0.1, lse=FAKE, out_prev=FAKE, fresh=FAKE, out=FAKE, out_dtype=1):
    return lib.sattn_delta_forward(q, k, v, idx, counts, cap, B, H, Nq, Nk, D, group, scale, lse, out_prev, fresh,
                                   out, out_dtype, P(0))


DELTA_CASES = [
    (dict(lse=P(0)), ERR_NULL), (dict(out_prev=P(0)), ERR_NULL), (dict(fresh=P(0)), ERR_NULL), (dict(v=P(0)), ERR_NULL),
    (dict(Nq=0), ERR_SHAPE), (dict(D=32), ERR_UNSUPPORTED), (dict(group=12), ERR_UNSUPPORTED),
    (dict(scale=-1.0), ERR_ARG), (dict(cap=0), ERR_ARG), (dict(out_dtype=5), ERR_ARG),
    (dict(fresh=P(4104)), ERR_ARG), (dict(out_prev=P(4100)), ERR_ARG), (dict(lse=P(4097)), ERR_ARG),
]


@pytest.mark.parametrize("kw,code", DELTA_CASES, ids=[str(c[0]) for c in DELTA_CASES])
def test_delta_forward_validation(lib, kw, code):
    assert dlt(lib, **kw) == code


def vsq(lib, v=FAKE, B=1, H=1, Nk=300, D=128, codes=FAKE, vscale=FAKE, vmean=FAKE, ws=FAKE, ws_bytes=1 << 40):
    return lib.sattn_vsmooth_quantize(v, B, H, Nk, D, codes, vscale, vmean, ws, ws_bytes, P(0))


VSMOOTH_CASES = [
    (dict(v=P(0)), ERR_NULL), (dict(codes=P(0)), ERR_NULL), (dict(vmean=P(0)), ERR_NULL), (dict(Nk=0), ERR_SHAPE),
    (dict(D=96), ERR_UNSUPPORTED), (dict(codes=P(4104)), ERR_ARG), (dict(vscale=P(4100)), ERR_ARG),
    (dict(vmean=P(4098)), ERR_ARG), (dict(ws=P(0)), ERR_WORKSPACE), (dict(ws_bytes=64), ERR_WORKSPACE),
    (dict(ws=P(4096 + 128)), ERR_WORKSPACE),
]


@pytest.mark.parametrize("kw,code", VSMOOTH_CASES, ids=[str(c[0]) for c in VSMOOTH_CASES])
def test_vsmooth_validation(lib, kw, code):
    assert vsq(lib, **kw) == code
    assert lib.sattn_last_error()


def f8f(lib, q=FAKE, k=FAKE, codes=FAKE, vscale=FAKE, vmean=FAKE, idx=FAKE, counts=FAKE, cap=64, B=1, H=1, Nq=128,
        Nk=128, D=128, group=128, scale=0.1, out=FAKE, out_dtype=1, lse=P(0)):
    return lib.sattn_fp8_forward(q, k, codes, vscale, vmean, idx, counts, cap, B, H, Nq, Nk, D, group, scale, out,
                                 out_dtype, lse, P(0))


FP8_CASES = [
    (dict(codes=P(0)), ERR_NULL), (dict(vscale=P(0)), ERR_NULL), (dict(vmean=P(0)), ERR_NULL), (dict(out=P(0)), ERR_NULL),
    (dict(B=0), ERR_SHAPE), (dict(D=32), ERR_UNSUPPORTED), (dict(group=24), ERR_UNSUPPORTED),
    (dict(scale=0.0), ERR_ARG), (dict(cap=0), ERR_ARG), (dict(out_dtype=3), ERR_ARG),
    (dict(codes=P(4104)), ERR_ARG), (dict(vscale=P(4100)), ERR_ARG), (dict(vmean=P(4104)), ERR_ARG),
    (dict(lse=P(4098)), ERR_ARG),
]


@pytest.mark.parametrize("kw,code", FP8_CASES, ids=[str(c[0]) for c in FP8_CASES])
def test_fp8_forward_validation(lib, kw, code):
    assert f8f(lib, **kw) == code
    assert lib.sattn_last_error()


def mxq(lib, x=FAKE, B=1, H=1, N=64, D=128, codes=FAKE, scales=FAKE):
    return lib.sattn_mx4_quantize(x, B, H, N, D, codes, scales, P(0))


MX4_CASES = [(dict(x=P(0)), ERR_NULL), (dict(scales=P(0)), ERR_NULL), (dict(N=0), ERR_SHAPE), (dict(D=96), ERR_UNSUPPORTED),
             (dict(codes=P(4104)), ERR_ARG), (dict(scales=P(4098)), ERR_ARG), (dict(x=P(4100)), ERR_ARG)]


@pytest.mark.parametrize("kw,code", MX4_CASES, ids=[str(c[0]) for c in MX4_CASES])
def test_mx4_quantize_validation(lib, kw, code):
    assert mxq(lib, **kw) == code
    assert lib.sattn_last_error()


def f4f(lib, q4=FAKE, qs=FAKE, k4=FAKE, ks=FAKE, codes=FAKE, vscale=FAKE, vmean=FAKE, idx=FAKE, counts=FAKE, cap=64,
        B=1, H=1, Nq=128, Nk=128, D=128, group=128, scale=0.1, out=FAKE, out_dtype=1, lse=P(0)):
    return lib.sattn_fp4_forward(q4, qs, k4, ks, codes, vscale, vmean, idx, counts, cap, B, H, Nq, Nk, D, group, scale,
                                 out, out_dtype, lse, P(0))


FP4_CASES = [(dict(q4=P(0)), ERR_NULL), (dict(ks=P(0)), ERR_NULL), (dict(vmean=P(0)), ERR_NULL), (dict(Nk=0), ERR_SHAPE),
             (dict(D=32), ERR_UNSUPPORTED), (dict(group=20), ERR_UNSUPPORTED), (dict(scale=float("inf")), ERR_ARG),
             (dict(cap=0), ERR_ARG), (dict(out_dtype=4), ERR_ARG), (dict(k4=P(4104)), ERR_ARG), (dict(qs=P(4098)), ERR_ARG)]


@pytest.mark.parametrize("kw,code", FP4_CASES, ids=[str(c[0]) for c in FP4_CASES])
def test_fp4_forward_validation(lib, kw, code):
    assert f4f(lib, **kw) == code
    assert lib.sattn_last_error()


def test_vsmooth_sizes(lib):
    assert lib.sattn_vsmooth_mean_stride(70200) == 552 and lib.sattn_vsmooth_mean_stride(128) == 4
    assert lib.sattn_vsmooth_mean_stride(129) == 4 and lib.sattn_vsmooth_mean_stride(513) == 8
    assert lib.sattn_vsmooth_mean_stride(0) == 0
    # bf16 means and fp32 block maxima of every (head, block, channel), each part 256-byte aligned
    assert lib.sattn_vsmooth_workspace_bytes(1, 24, 70200, 128) == 24 * 549 * 128 * 6
    assert lib.sattn_vsmooth_workspace_bytes(1, 1, 10, 96) == 0


def test_dense_validation(lib):
    f = lambda **kw: lib.attn_forward(kw.get("q", FAKE), FAKE, FAKE, kw.get("B", 1), 1, 64, 64, kw.get("D", 64),
                                      kw.get("scale", 0.1), kw.get("out", FAKE), kw.get("dt", 0), P(0), P(0))
    assert f(q=P(0)) == ERR_NULL and f(B=0) == ERR_SHAPE and f(D=80) == ERR_UNSUPPORTED
    assert f(scale=-2.0) == ERR_ARG and f(dt=7) == ERR_ARG and f(out=P(4100)) == ERR_ARG


def test_permute_validation(lib):
    f = lambda **kw: lib.sattn_permute_tokens(kw.get("src", FAKE), kw.get("dst", P(8192)), FAKE, 1, 1,
                                              kw.get("N", 8), kw.get("D", 64), kw.get("inv", 0), P(0))
    assert f(src=P(0)) == ERR_NULL and f(N=0) == ERR_SHAPE and f(D=48) == ERR_UNSUPPORTED
    assert f(inv=3) == ERR_ARG and f(dst=FAKE) == ERR_ARG


def test_workspace_query(lib):
    assert lib.sattn_mask_workspace_bytes(1, 2, 1024, 1024, 64, 64) > 2 * 16 * 1024 * 4
    assert lib.sattn_mask_workspace_bytes(1, 1, 10, 10, 96, 64) == 0
    assert lib.sattn_mask_workspace_bytes(1, 1, 10, 200000, 128, 64) == 0
    # long video: 549 groups x 70200 keys of fp32 scores per head; the staging is bounded
    ws = lib.sattn_mask_workspace_bytes(1, 24, 70200, 70200, 128, 128)
    assert 549 * 70200 * 4 <= ws <= 2100 * (1 << 20)


def test_voxel_permutation_matches_generator(lib):
    from synth import inputs
    import sparse_self_attention_amd as sattn
    for grid, vox in [((30, 45, 52), (4, 6, 8)), ((5, 6, 9), (2, 3, 4)), ((3, 3, 3), (1, 1, 1))]:
        perm = sattn.voxel_permutation(grid, vox).numpy()
        assert np.array_equal(perm, inputs.voxel_order(grid, vox))
    assert lib.sattn_voxel_permutation(0, 1, 1, 1, 1, 1, FAKE) == ERR_SHAPE
    assert lib.sattn_voxel_permutation(1, 1, 1, 1, 1, 1, P(0)) == ERR_NULL
