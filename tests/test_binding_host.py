"""Without a GPU: every binding entry point refuses host tensors with ValueError before it reaches the
library's compute calls (the library itself is only loaded)."""
import os

import pytest

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def sattn():
    import sparse_self_attention_amd as s
    if not os.path.exists(s.library_path()):
        pytest.skip("libsattn.so is not built")
    return s


def test_host_tensors_are_refused(sattn):
    B, H, N, D, group = 1, 1, 64, 64, 64
    q = torch.zeros((B, H, N, D), dtype=torch.bfloat16)
    idx = torch.zeros((B, H, 1, 8), dtype=torch.int32)
    counts = torch.zeros((B, H, 1), dtype=torch.int32)
    lse = torch.zeros((B, H, N), dtype=torch.float32)
    f32 = torch.zeros((B, H, N, D), dtype=torch.float32)
    u8 = torch.zeros((B, H, N, D), dtype=torch.uint8)
    calls = [
        lambda: sattn.mask(q, q, group, topk=8),
        lambda: sattn.forward(q, q, q, idx, counts, group),
        lambda: sattn.attn(q, q, q),
        lambda: sattn.cached_mask(q, q, lse, group),
        lambda: sattn.colsum_mask(q, q, lse, group, 8),
        lambda: sattn.delta_forward(q, q, q, idx, counts, group, lse=lse, out_prev=f32, fresh=f32),
        lambda: sattn.vsmooth_quantize(q),
        lambda: sattn.fp8_forward(q, q, u8, f32, q, idx, counts, group),
        lambda: sattn.mx4_quantize(q),
        lambda: sattn.fp4_forward(u8, u8, u8, u8, u8, f32, q, idx, counts, group),
        lambda: sattn.permute_tokens(q, torch.arange(N, dtype=torch.int32)),
    ]
    for i, call in enumerate(calls):
        with pytest.raises(ValueError):
            call()
