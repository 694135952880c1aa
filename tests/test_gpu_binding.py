"""The Python binding refuses a tensor that is not on the inputs' device (a host tensor's address would
reach a kernel) or whose dtype, shape or layout the C ABI does not take: every such call raises
ValueError before anything is launched, and the same call with device tensors runs."""
import os

import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
DEV = "cuda:0"
B, H, D, GROUP, NQ, NK, TOPK = 1, 2, 64, 64, 200, 500, 100
G = -(-NQ // GROUP)


@pytest.fixture(scope="module")
def sattn():
    import sparse_self_attention_amd as s
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    assert os.path.exists(s.library_path()), "libsattn.so is not built"
    return s


@pytest.fixture(scope="module")
def qkv():
    gen = torch.Generator(device=DEV)
    gen.manual_seed(5)
    mk = lambda n: torch.randn((B, H, n, D), device=DEV, generator=gen).to(torch.bfloat16)
    return mk(NQ), mk(NK), mk(NK)


def host(t):
    return t.detach().cpu()


def test_mask_and_forward_arguments(sattn, qkv):
    q, k, v = qkv
    idx, counts = sattn.mask(q, k, GROUP, topk=TOPK)
    ws = torch.empty(sattn.mask_workspace_bytes(B, H, NQ, NK, D, GROUP), dtype=torch.uint8, device=DEV)
    bad_mask = [dict(idx=host(idx)), dict(counts=host(counts)), dict(workspace=host(ws)),
                dict(idx=idx[..., :TOPK].view(B, H, G * TOPK))]
    for kw in bad_mask:
        with pytest.raises(ValueError):
            sattn.mask(q, k, GROUP, topk=TOPK, **kw)
    with pytest.raises(ValueError):
        sattn.mask(q, host(k), GROUP, topk=TOPK)
    out = torch.empty((B, H, NQ, D), dtype=torch.float32, device=DEV)
    lse = torch.empty((B, H, NQ), dtype=torch.float32, device=DEV)
    for args, kw in [((q, k, v, host(idx), counts), {}), ((q, k, v, idx, host(counts)), {}),
                     ((q, k, host(v), idx, counts), {}), ((q, k, v, idx, counts), dict(out=host(out))),
                     ((q, k, v, idx, counts), dict(lse=host(lse))),
                     ((q, k, v, idx, counts), dict(out=out[:, :, :NQ - 1])),
                     ((q, k, v, idx, counts), dict(lse=lse[:, :1]))]:
        with pytest.raises(ValueError):
            sattn.forward(*args, GROUP, **kw)
    sattn.forward(q, k, v, idx, counts, GROUP, out=out, lse=lse)
    for kw in [dict(out=host(out)), dict(lse=host(lse)), dict(out=out.to(torch.float16))]:
        with pytest.raises(ValueError):
            sattn.attn(q, k, v, **kw)
    sattn.attn(q, k, v, out=out, lse=lse)
    torch.cuda.synchronize()


def test_cached_colsum_and_delta_arguments(sattn, qkv):
    q, k, v = qkv
    _, lse = sattn.attn(q, k, v)
    idx = torch.empty((B, H, G, NK), dtype=torch.int32, device=DEV)
    counts = torch.empty((B, H, G), dtype=torch.int32, device=DEV)
    for kw in [dict(idx=host(idx)), dict(counts=host(counts))]:
        with pytest.raises(ValueError):
            sattn.cached_mask(q, k, lse, GROUP, **kw)
    with pytest.raises(ValueError):
        sattn.cached_mask(q, k, host(lse), GROUP)
    ws = torch.empty(sattn.mask_workspace_bytes(B, H, NQ, NK, D, GROUP), dtype=torch.uint8, device=DEV)
    with pytest.raises(ValueError):
        sattn.colsum_mask(q, k, lse, GROUP, TOPK, workspace=host(ws))
    si, sc = sattn.colsum_mask(q, k, lse, GROUP, TOPK, workspace=ws)
    fresh = torch.zeros((B, H, NQ, D), dtype=torch.float32, device=DEV)
    prev = torch.zeros_like(fresh)
    for kw in [dict(fresh=host(fresh), out_prev=prev), dict(fresh=fresh, out_prev=host(prev)),
               dict(fresh=fresh, out_prev=prev, out=host(fresh))]:
        with pytest.raises(ValueError):
            sattn.delta_forward(q, k, v, si, sc, GROUP, lse=lse, **kw)
    sattn.delta_forward(q, k, v, si, sc, GROUP, lse=lse, out_prev=prev, fresh=fresh)
    torch.cuda.synchronize()


def test_lowbit_and_permutation_arguments(sattn, qkv):
    q, k, v = qkv
    codes, vscale, vmean = sattn.vsmooth_quantize(v)
    for kw in [dict(codes=host(codes)), dict(vscale=host(vscale)), dict(vmean=host(vmean))]:
        with pytest.raises(ValueError):
            sattn.vsmooth_quantize(v, **kw)
    idx, counts = sattn.mask(q, k, GROUP, topk=TOPK)
    for vals in [(host(codes), vscale, vmean), (codes, host(vscale), vmean), (codes, vscale, host(vmean))]:
        with pytest.raises(ValueError):
            sattn.fp8_forward(q, k, *vals, idx, counts, GROUP)
    sattn.fp8_forward(q, k, codes, vscale, vmean, idx, counts, GROUP)
    q4, qs = sattn.mx4_quantize(q)
    k4, ks = sattn.mx4_quantize(k)
    with pytest.raises(ValueError):
        sattn.mx4_quantize(q, scales=host(qs))
    for args in [(q4, qs, k4, host(ks)), (q4, qs, host(k4), ks), (q4, host(qs), k4, ks)]:
        with pytest.raises(ValueError):
            sattn.fp4_forward(*args, codes, vscale, vmean, idx, counts, GROUP)
    with pytest.raises(ValueError):
        sattn.fp4_forward(q4, qs, k4, ks, codes, vscale, vmean, idx, host(counts), GROUP)
    sattn.fp4_forward(q4, qs, k4, ks, codes, vscale, vmean, idx, counts, GROUP)
    perm = torch.randperm(NK, generator=torch.Generator().manual_seed(3)).to(torch.int32)
    with pytest.raises(ValueError):
        sattn.permute_tokens(k, perm)                       # host permutation
    with pytest.raises(ValueError):
        sattn.permute_tokens(host(k), perm.to(DEV))
    with pytest.raises(ValueError):
        sattn.permute_tokens(k, perm.to(DEV), out=host(k))
    sattn.permute_tokens(k, perm.to(DEV))
    torch.cuda.synchronize()
