"""sattn_mask_noalloc (the mask with the library's fixed device scratch as its workspace) against sattn_mask
through the C ABI: identical key lists and counts, bit for bit, on two calls in a row, the second with a
smaller input (the scratch keeps the first call's contents), in top-k and threshold mode."""
import os

import numpy as np
import pytest

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


def _qk(rng, B, H, Nq, Nk, D):
    mk = lambda n: torch.from_numpy(
        inputs.f32_to_bf16_bits(rng.standard_normal((B, H, n, D)).astype(np.float32)).view(np.int16)).to(DEV)
    return mk(Nq).view(torch.bfloat16), mk(Nk).view(torch.bfloat16)


def _same_lists(sattn, q, k, group, **kw):
    idx_a, cnt_a = sattn.mask(q, k, group, **kw)
    B, H, G, cap = idx_a.shape
    idx_b = torch.full_like(idx_a, -7)
    cnt_b = torch.full_like(cnt_a, -7)
    sattn.mask_noalloc(q, k, group, idx=idx_b, counts=cnt_b, **kw)
    torch.cuda.synchronize()
    assert torch.equal(cnt_a, cnt_b), "counts differ"
    ia, ib, c = idx_a.cpu().numpy(), idx_b.cpu().numpy(), cnt_a.cpu().numpy()
    for b in range(B):
        for h in range(H):
            for g in range(G):
                n = int(c[b, h, g])
                assert np.array_equal(ia[b, h, g, :n], ib[b, h, g, :n]), (b, h, g)


@pytest.mark.parametrize("mode", ["topk", "thresh"])
def test_noalloc_mask_equals_mask(sattn, mode):
    rng = np.random.default_rng(101 if mode == "topk" else 102)
    # first call: the long-video shape on 3 heads (one head per pass of the scratch), 2 batches
    q, k = _qk(rng, 2, 3, 70200, 70200, 128)
    kw = {"topk": 14040} if mode == "topk" else {"thresh": 2e-5}
    _same_lists(sattn, q, k, 128, **kw)
    del q, k
    # second call, smaller: many heads per pass, D = 64, a ragged last group
    q, k = _qk(rng, 1, 5, 3000, 4000, 64)
    kw = {"topk": 500} if mode == "topk" else {"thresh": 1e-4}
    _same_lists(sattn, q, k, 64, **kw)


def test_noalloc_rejects_a_head_larger_than_the_scratch(sattn):
    q, k = _qk(np.random.default_rng(3), 1, 1, 131072, 131072, 64)
    idx = torch.empty((1, 1, 8192, 64), dtype=torch.int32, device=DEV)
    cnt = torch.empty((1, 1, 8192), dtype=torch.int32, device=DEV)
    with pytest.raises(sattn.SattnError) as e:
        sattn.mask_noalloc(q, k, 16, topk=64, idx=idx, counts=cnt)
    assert e.value.status == 3


def test_noalloc_mask_in_a_graph(sattn):
    """The caller the entry point is for: sattn_mask_noalloc captured into a HIP graph (no workspace to
    allocate), replayed three times with eager work between the replays; every replay's lists equal the
    eager sattn_mask's bit for bit."""
    rng = np.random.default_rng(104)
    group, topk = 128, 700
    q, k = _qk(rng, 1, 3, 1000, 5000, 128)
    ref_idx, ref_cnt = sattn.mask(q, k, group, topk=topk)
    idx = torch.empty_like(ref_idx)
    cnt = torch.empty_like(ref_cnt)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        sattn.mask_noalloc(q, k, group, topk=topk, idx=idx, counts=cnt)     # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sattn.mask_noalloc(q, k, group, topk=topk, idx=idx, counts=cnt)
    for rep in range(3):
        idx.fill_(-7)                  # eager work between the replays
        cnt.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(cnt, ref_cnt), f"replay {rep}: counts differ"
        assert torch.equal(idx, ref_idx), f"replay {rep}: lists differ"
