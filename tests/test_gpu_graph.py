"""The hot path (mask, then sparse forward) captured into a HIP graph through torch: every replay, with
eager work between the replays, reproduces the eager results bit for bit."""
import os

import numpy as np
import pytest

from gpu_util import to_device_bf16
from synth import inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
DEV = "cuda:0"


@pytest.fixture(scope="module")
def sattn():
    import sparse_self_attention_amd as s
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    assert os.path.exists(s.library_path()), "libsattn.so is not built"
    return s


def test_graph_replays_match_eager(sattn):
    rng = np.random.default_rng(17)
    B, H, D, group, Nq, Nk, topk = 1, 2, 128, 128, 1000, 6000, 1200
    bits = lambda shape, std: inputs.f32_to_bf16_bits((rng.standard_normal(shape) * std).astype(np.float32))
    q = to_device_bf16(bits((B, H, Nq, D), 2.0), DEV)
    k = to_device_bf16(bits((B, H, Nk, D), 1.0), DEV)
    v = to_device_bf16(bits((B, H, Nk, D), 1.0), DEV)
    G = -(-Nq // group)
    ws = torch.empty(sattn.mask_workspace_bytes(B, H, Nq, Nk, D, group), dtype=torch.uint8, device=DEV)

    def buffers():
        return (torch.empty((B, H, G, topk), dtype=torch.int32, device=DEV),
                torch.empty((B, H, G), dtype=torch.int32, device=DEV),
                torch.empty((B, H, Nq, D), dtype=torch.float32, device=DEV),
                torch.empty((B, H, Nq), dtype=torch.float32, device=DEV))

    def step(idx, cnt, out, lse):
        sattn.mask(q, k, group, topk=topk, idx=idx, counts=cnt, workspace=ws)
        sattn.forward(q, k, v, idx, cnt, group, out=out, lse=lse)

    ref = buffers()
    step(*ref)
    torch.cuda.synchronize()
    got = buffers()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(*got)                      # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(*got)
    for rep in range(3):
        got[0].fill_(-7)                # eager work between the replays
        got[2].zero_()
        got[3].fill_(1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b, name in zip(got, ref, ("idx", "counts", "out", "lse")):
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager run"


def test_threshold_mask_and_split_forward_graph_replays_match_eager(sattn):
    """A threshold mask (uneven lists) followed by the split-list forward in three parts, captured into one
    graph: every replay reproduces the eager lists, output and lse bit for bit."""
    rng = np.random.default_rng(23)
    B, H, D, group, Nq, Nk, splits = 1, 2, 128, 128, 900, 4000, 3
    bits = lambda shape, std: inputs.f32_to_bf16_bits((rng.standard_normal(shape) * std).astype(np.float32))
    q = to_device_bf16(bits((B, H, Nq, D), 2.0), DEV)
    k = to_device_bf16(bits((B, H, Nk, D), 1.0), DEV)
    v = to_device_bf16(bits((B, H, Nk, D), 1.0), DEV)
    G = -(-Nq // group)
    tau = 0.3 / Nk
    ws = torch.empty(sattn.mask_workspace_bytes(B, H, Nq, Nk, D, group), dtype=torch.uint8, device=DEV)
    sws = torch.empty(sattn.forward_split_workspace_bytes(B, H, Nq, D, splits), dtype=torch.uint8, device=DEV)

    def buffers():
        return (torch.empty((B, H, G, Nk), dtype=torch.int32, device=DEV),
                torch.empty((B, H, G), dtype=torch.int32, device=DEV),
                torch.empty((B, H, Nq, D), dtype=torch.bfloat16, device=DEV),
                torch.empty((B, H, Nq), dtype=torch.float32, device=DEV))

    def step(idx, cnt, out, lse):
        sattn.mask(q, k, group, thresh=tau, idx=idx, counts=cnt, workspace=ws)
        sattn.forward_split(q, k, v, idx, cnt, group, splits, workspace=sws, out=out, lse=lse)

    ref = buffers()
    step(*ref)
    torch.cuda.synchronize()
    c = ref[1].cpu().numpy()
    assert c.min() < c.max(), "the threshold lists should differ in length"
    got = buffers()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(*got)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(*got)
    for rep in range(3):
        got[0].fill_(-7)
        got[2].zero_()
        got[3].fill_(1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, a_, b_ in (("counts", got[1], ref[1]), ("out", got[2], ref[2]), ("lse", got[3], ref[3])):
            assert torch.equal(a_, b_), f"replay {rep}: {name} differs from the eager run"
        for h in range(H):
            for gi in range(G):
                n = int(ref[1][0, h, gi])
                assert torch.equal(got[0][0, h, gi, :n], ref[0][0, h, gi, :n]), f"replay {rep}: list ({h}, {gi})"


def test_lowbit_paths_graph_replays_match_eager(sattn):
    """V-Smooth quantisation + FP8 forward, and MXFP4 quantisation of Q and K + FP4-score forward, captured
    together into one graph: every replay reproduces the eager results bit for bit."""
    rng = np.random.default_rng(19)
    B, H, D, group, Nq, Nk, topk = 1, 2, 128, 128, 700, 5000, 900
    bits = lambda shape, std: inputs.f32_to_bf16_bits((rng.standard_normal(shape) * std).astype(np.float32))
    q = to_device_bf16(bits((B, H, Nq, D), 1.5), DEV)
    k = to_device_bf16(bits((B, H, Nk, D), 1.0), DEV)
    v = to_device_bf16(bits((B, H, Nk, D), 1.0), DEV)
    idx, cnt = sattn.mask(q, k, group, topk=topk)
    ws = torch.empty(sattn.vsmooth_workspace_bytes(B, H, Nk, D), dtype=torch.uint8, device=DEV)

    def buffers():
        codes, vscale, vmean = sattn.vsmooth_quantize(v, workspace=ws)
        q4, qs = sattn.mx4_quantize(q)
        k4, ks = sattn.mx4_quantize(k)
        o8, l8 = sattn.fp8_forward(q, k, codes, vscale, vmean, idx, cnt, group)
        o4, l4 = sattn.fp4_forward(q4, qs, k4, ks, codes, vscale, vmean, idx, cnt, group)
        return [codes, vscale, vmean, q4, qs, k4, ks, o8, l8, o4, l4]

    def step(b):
        codes, vscale, vmean, q4, qs, k4, ks, o8, l8, o4, l4 = b
        sattn.vsmooth_quantize(v, codes=codes, vscale=vscale, vmean=vmean, workspace=ws)
        sattn.mx4_quantize(q, codes=q4, scales=qs)
        sattn.mx4_quantize(k, codes=k4, scales=ks)
        sattn.fp8_forward(q, k, codes, vscale, vmean, idx, cnt, group, out=o8, lse=l8)
        sattn.fp4_forward(q4, qs, k4, ks, codes, vscale, vmean, idx, cnt, group, out=o4, lse=l4)

    ref = buffers()
    torch.cuda.synchronize()
    got = [t.clone() for t in ref]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(got)                       # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(got)
    for rep in range(3):
        for t in got:                   # eager work between the replays
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(got, ref)):
            assert torch.equal(a, b), f"replay {rep}: buffer {i} differs from the eager run"


def test_cached_and_delta_paths_graph_replays_match_eager(sattn):
    """Dense pass (lse), cached slice mask, Chipmunk column-sum lists and one delta step captured together:
    with the delta state reset before each replay, every replay reproduces the eager run bit for bit."""
    rng = np.random.default_rng(23)
    B, H, D, group, Nq, Nk, topk = 1, 2, 128, 128, 600, 3000, 500
    bits = lambda shape, std: inputs.f32_to_bf16_bits((rng.standard_normal(shape) * std).astype(np.float32))
    q = to_device_bf16(bits((B, H, Nq, D), 1.5), DEV)
    k = to_device_bf16(bits((B, H, Nk, D), 1.0), DEV)
    v = to_device_bf16(bits((B, H, Nk, D), 1.0), DEV)
    G = -(-Nq // group)
    ws = torch.empty(sattn.mask_workspace_bytes(B, H, Nq, Nk, D, group), dtype=torch.uint8, device=DEV)
    out_prev = torch.from_numpy(rng.standard_normal((B, H, Nq, D)).astype(np.float32)).to(DEV)

    def buffers():
        return [torch.empty((B, H, Nq, D), dtype=torch.float32, device=DEV),      # dense out
                torch.empty((B, H, Nq), dtype=torch.float32, device=DEV),         # lse
                torch.empty((B, H, G, Nk), dtype=torch.int32, device=DEV),        # cached lists
                torch.empty((B, H, G), dtype=torch.int32, device=DEV),
                torch.empty((B, H, G, topk), dtype=torch.int32, device=DEV),      # column-sum lists
                torch.empty((B, H, G), dtype=torch.int32, device=DEV),
                torch.zeros((B, H, Nq, D), dtype=torch.float32, device=DEV),      # delta state (fresh)
                torch.empty((B, H, Nq, D), dtype=torch.float32, device=DEV)]      # delta output

    def step(b):
        dout, lse, ci, cc, si, sc, fresh, out = b
        sattn.attn(q, k, v, out=dout, lse=lse)
        sattn.cached_mask(q, k, lse, group, idx=ci, counts=cc)
        sattn.colsum_mask(q, k, lse, group, topk, idx=si, counts=sc, workspace=ws)
        sattn.delta_forward(q, k, v, si, sc, group, lse=lse, out_prev=out_prev, fresh=fresh, out=out)

    ref = buffers()
    step(ref)
    torch.cuda.synchronize()
    got = buffers()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(got)                       # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(got)
    for rep in range(3):
        for t in got:                   # eager work between the replays; the delta state back to zero
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(got, ref)):
            assert torch.equal(a, b), f"replay {rep}: buffer {i} differs from the eager run"
