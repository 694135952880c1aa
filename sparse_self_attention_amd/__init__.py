"""Fine-grained (Mx1-slice / column-sparse) self-attention for AMD MI355X (gfx950).

A thin ctypes binding over the C ABI of libsattn.so (include/sattn.h).  Functions take torch
tensors, check dtype / device / layout, and pass raw device pointers and the current HIP stream;
all of the work runs in the library's HIP kernels.  There is no fallback: if libsattn.so is
missing or cannot be loaded, every call raises.

    idx, counts = mask(q, k, group=128, topk=k)            # or thresh=tau
    out, lse    = forward(q, k, v, idx, counts, group=128)
    out, lse    = attn(q, k, v)                            # dense control path
    idx, counts = cached_mask(q, k, lse, group=128)        # slices with a probability >= 0.5/N
    idx, counts = colsum_mask(q, k, lse, group=192, topk=k)  # Chipmunk column-sum selection
    out = delta_forward(q, k, v, idx, counts, 192, lse=lse, out_prev=out, fresh=fresh)  # sparse delta
    codes, vscale, vmean = vsmooth_quantize(v)             # V-Smooth E4M3 codes, scales, block means
    out, lse    = fp8_forward(q, k, codes, vscale, vmean, idx, counts, group=128)   # ExpCast + FP8 P.V
    q4, qs = mx4_quantize(q); k4, ks = mx4_quantize(k)   # MXFP4 queries and keys
    out, lse    = fp4_forward(q4, qs, k4, ks, codes, vscale, vmean, idx, counts, group=128)  # 4-bit QK^T
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

__all__ = ["mask", "mask_noalloc", "forward", "attn", "cached_mask", "colsum_mask", "delta_forward", "vsmooth_quantize",
           "fp8_forward", "mx4_quantize", "fp4_forward", "vsmooth_workspace_bytes", "mask_workspace_bytes", "voxel_permutation", "permute_tokens",
           "library_path", "SattnError", "TOPK", "THRESH"]

TOPK, THRESH = 0, 1
BF16, F32 = 0, 1
MASK_MAX_NK = 131072

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.environ.get("SATTN_LIBRARY", os.path.join(_PKG, "libsattn.so"))
_lib = None


class SattnError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str):
        super().__init__(f"{fn} failed with status {status}: {detail}")
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"libsattn.so not found at {_LIB_PATH}; build it with "
                           "`python -m sparse_self_attention_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    P, I, F, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.sattn_mask_workspace_bytes.argtypes = [I, I, I, I, I, I]
    lib.sattn_mask_workspace_bytes.restype = Z
    lib.sattn_mask.argtypes = [P, P, I, I, I, I, I, I, I, I, F, F, P, P, I, P, Z, P]
    lib.sattn_mask.restype = I
    lib.sattn_mask_noalloc.argtypes = [P, P, I, I, I, I, I, I, I, I, F, F, P, P, I, P]
    lib.sattn_mask_noalloc.restype = I
    lib.sattn_forward.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I, F, P, I, P, P]
    lib.sattn_forward.restype = I
    lib.sattn_forward_split_workspace_bytes.argtypes = [I, I, I, I, I]
    lib.sattn_forward_split_workspace_bytes.restype = Z
    lib.sattn_forward_split.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I, F, I, P, Z, P, I, P, P]
    lib.sattn_forward_split.restype = I
    lib.attn_forward.argtypes = [P, P, P, I, I, I, I, I, F, P, I, P, P]
    lib.attn_forward.restype = I
    lib.sattn_cached_mask.argtypes = [P, P, P, I, I, I, I, I, I, F, F, P, P, I, P]
    lib.sattn_cached_mask.restype = I
    lib.sattn_colsum_mask.argtypes = [P, P, P, I, I, I, I, I, I, I, F, P, P, I, P, Z, P]
    lib.sattn_colsum_mask.restype = I
    lib.sattn_delta_forward.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I, F, P, P, P, P, I, P]
    lib.sattn_delta_forward.restype = I
    lib.sattn_vsmooth_workspace_bytes.argtypes = [I, I, I, I]
    lib.sattn_vsmooth_workspace_bytes.restype = Z
    lib.sattn_vsmooth_mean_stride.argtypes = [I]
    lib.sattn_vsmooth_mean_stride.restype = I
    lib.sattn_vsmooth_quantize.argtypes = [P, I, I, I, I, P, P, P, P, Z, P]
    lib.sattn_vsmooth_quantize.restype = I
    lib.sattn_fp8_forward.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, F, P, I, P, P]
    lib.sattn_fp8_forward.restype = I
    lib.sattn_mx4_quantize.argtypes = [P, I, I, I, I, P, P, P]
    lib.sattn_mx4_quantize.restype = I
    lib.sattn_fp4_forward.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, F, P, I, P, P]
    lib.sattn_fp4_forward.restype = I
    lib.sattn_voxel_permutation.argtypes = [I, I, I, I, I, I, P]
    lib.sattn_voxel_permutation.restype = I
    lib.sattn_permute_tokens.argtypes = [P, P, P, I, I, I, I, I, P]
    lib.sattn_permute_tokens.restype = I
    lib.sattn_strerror.argtypes = [I]
    lib.sattn_strerror.restype = ctypes.c_char_p
    lib.sattn_last_error.argtypes = []
    lib.sattn_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(fn: str, status: int):
    if status != 0:
        lib = _load()
        raise SattnError(fn, status, lib.sattn_last_error().decode(errors="replace"))


def _stream_ptr(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t: Optional[torch.Tensor]):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _check_qkv(q, k, v=None):
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if t.dtype != torch.bfloat16:
            raise ValueError(f"{name} must be bfloat16")
        if t.dim() != 4 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous [B, H, N, D] tensor")
    _on(q.device, k=k, v=v)
    B, H, Nq, D = q.shape
    if k.shape[0] != B or k.shape[1] != H or k.shape[3] != D:
        raise ValueError("q and k disagree on B, H or D")
    if v is not None and v.shape != k.shape:
        raise ValueError("v must have the shape of k")
    return B, H, Nq, k.shape[2], D


def _check_lse(lse, B, H, Nq, dev=None):
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, Nq) or not lse.is_contiguous() or not lse.is_cuda:
        raise ValueError("lse must be a contiguous fp32 device tensor [B, H, Nq]")
    if dev is not None:
        _on(dev, lse=lse)


def _on(dev, **tensors):
    """Every tensor given (None skipped) must live on `dev`: a host pointer, or one of another device, would
    reach the kernels as an address they cannot use."""
    for name, t in tensors.items():
        if t is not None and (not t.is_cuda or t.device != dev):
            raise ValueError(f"{name} must be a tensor on {dev} (got {t.device})")


def _check_lists(idx, counts, B, H, G, dev):
    if idx.dtype != torch.int32 or counts.dtype != torch.int32 or not idx.is_contiguous() or not counts.is_contiguous():
        raise ValueError("idx and counts must be contiguous int32")
    if idx.dim() != 4 or tuple(idx.shape[:3]) != (B, H, G) or tuple(counts.shape) != (B, H, G):
        raise ValueError("idx must be [B, H, G, cap] and counts [B, H, G] with G = ceil(Nq / group)")
    _on(dev, idx=idx, counts=counts)


def _check_out(out, shape, dev):
    if out.dtype not in (torch.bfloat16, torch.float32) or tuple(out.shape) != tuple(shape) or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous bf16 or fp32 tensor of shape {tuple(shape)}")
    _on(dev, out=out)


def _check_workspace(ws, dev):
    if not ws.is_contiguous():
        raise ValueError("workspace must be contiguous")
    _on(dev, workspace=ws)
    return ws.numel() * ws.element_size()


def mask_workspace_bytes(B: int, H: int, Nq: int, Nk: int, D: int, group: int) -> int:
    return int(_load().sattn_mask_workspace_bytes(B, H, Nq, Nk, D, group))


def mask(q: torch.Tensor, k: torch.Tensor, group: int, *, topk: Optional[int] = None,
         thresh: Optional[float] = None, scale: Optional[float] = None, cap: Optional[int] = None,
         idx: Optional[torch.Tensor] = None, counts: Optional[torch.Tensor] = None,
         workspace: Optional[torch.Tensor] = None):
    """Per-group key lists from the group-mean query (sattn_mask).  Exactly one of topk / thresh."""
    lib = _load()
    B, H, Nq, Nk, D = _check_qkv(q, k)
    if (topk is None) == (thresh is None):
        raise ValueError("pass exactly one of topk= or thresh=")
    mode = TOPK if topk is not None else THRESH
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    G = -(-Nq // group)
    if cap is None:
        cap = int(topk) if mode == TOPK else Nk
    if idx is None:
        idx = torch.empty((B, H, G, cap), dtype=torch.int32, device=q.device)
    if counts is None:
        counts = torch.empty((B, H, G), dtype=torch.int32, device=q.device)
    _check_lists(idx, counts, B, H, G, q.device)
    need = lib.sattn_mask_workspace_bytes(B, H, Nq, Nk, D, group)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    ws_bytes = _check_workspace(workspace, q.device)
    st = lib.sattn_mask(_ptr(q), _ptr(k), B, H, Nq, Nk, D, group, mode, int(topk or 0),
                        float(thresh or 0.0), scale, _ptr(idx), _ptr(counts), idx.shape[-1],
                        _ptr(workspace), ws_bytes, _stream_ptr(q))
    _check("sattn_mask", st)
    return idx, counts


def mask_noalloc(q: torch.Tensor, k: torch.Tensor, group: int, *, topk: Optional[int] = None,
                 thresh: Optional[float] = None, scale: Optional[float] = None, idx: torch.Tensor,
                 counts: torch.Tensor):
    """sattn_mask with the library's fixed device scratch as workspace (sattn_mask_noalloc): the caller
    passes the outputs and nothing is allocated.  Calls that overlap on one GPU race on the scratch."""
    lib = _load()
    B, H, Nq, Nk, D = _check_qkv(q, k)
    if (topk is None) == (thresh is None):
        raise ValueError("pass exactly one of topk= or thresh=")
    mode = TOPK if topk is not None else THRESH
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    _check_lists(idx, counts, B, H, -(-Nq // group), q.device)
    st = lib.sattn_mask_noalloc(_ptr(q), _ptr(k), B, H, Nq, Nk, D, group, mode, int(topk or 0),
                                float(thresh or 0.0), scale, _ptr(idx), _ptr(counts), idx.shape[-1], _stream_ptr(q))
    _check("sattn_mask_noalloc", st)
    return idx, counts


def forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, idx: torch.Tensor, counts: torch.Tensor,
            group: int, *, scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
            lse: Optional[torch.Tensor] = None, out_dtype: torch.dtype = torch.bfloat16, want_lse: bool = True):
    """Sparse attention over per-group key lists (sattn_forward).  Returns (out, lse or None)."""
    lib = _load()
    B, H, Nq, Nk, D = _check_qkv(q, k, v)
    G = -(-Nq // group)
    _check_lists(idx, counts, B, H, G, q.device)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    if out is None:
        out = torch.empty((B, H, Nq, D), dtype=out_dtype, device=q.device)
    _check_out(out, q.shape, q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _check_lse(lse, B, H, Nq, q.device)
    st = lib.sattn_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(idx), _ptr(counts), idx.shape[-1], B, H, Nq, Nk, D,
                           group, scale, _ptr(out), F32 if out.dtype == torch.float32 else BF16, _ptr(lse),
                           _stream_ptr(q))
    _check("sattn_forward", st)
    return out, lse


def forward_split_workspace_bytes(B: int, H: int, Nq: int, D: int, splits: int) -> int:
    """Device workspace of sattn_forward_split for these sizes (0 if invalid)."""
    return int(_load().sattn_forward_split_workspace_bytes(B, H, Nq, D, splits))


def forward_split(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, idx: torch.Tensor, counts: torch.Tensor,
                  group: int, splits: int, *, scale: Optional[float] = None, workspace: Optional[torch.Tensor] = None,
                  out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                  out_dtype: torch.dtype = torch.bfloat16, want_lse: bool = True):
    """sattn_forward with each group's list in `splits` parts merged at the end (sattn_forward_split).
    Returns (out, lse or None)."""
    lib = _load()
    B, H, Nq, Nk, D = _check_qkv(q, k, v)
    G = -(-Nq // group)
    _check_lists(idx, counts, B, H, G, q.device)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    if out is None:
        out = torch.empty((B, H, Nq, D), dtype=out_dtype, device=q.device)
    _check_out(out, q.shape, q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _check_lse(lse, B, H, Nq, q.device)
    need = forward_split_workspace_bytes(B, H, Nq, D, splits)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    ws_bytes = _check_workspace(workspace, q.device)
    st = lib.sattn_forward_split(_ptr(q), _ptr(k), _ptr(v), _ptr(idx), _ptr(counts), idx.shape[-1], B, H, Nq, Nk,
                                 D, group, scale, int(splits), _ptr(workspace), ws_bytes, _ptr(out),
                                 F32 if out.dtype == torch.float32 else BF16, _ptr(lse), _stream_ptr(q))
    _check("sattn_forward_split", st)
    return out, lse


def attn(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, scale: Optional[float] = None,
         out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
         out_dtype: torch.dtype = torch.bfloat16, want_lse: bool = True):
    """Dense attention control path (attn_forward).  Returns (out, lse or None)."""
    lib = _load()
    B, H, Nq, Nk, D = _check_qkv(q, k, v)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    if out is None:
        out = torch.empty((B, H, Nq, D), dtype=out_dtype, device=q.device)
    _check_out(out, q.shape, q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _check_lse(lse, B, H, Nq, q.device)
    st = lib.attn_forward(_ptr(q), _ptr(k), _ptr(v), B, H, Nq, Nk, D, scale, _ptr(out),
                          F32 if out.dtype == torch.float32 else BF16, _ptr(lse), _stream_ptr(q))
    _check("attn_forward", st)
    return out, lse


def cached_mask(q: torch.Tensor, k: torch.Tensor, lse: torch.Tensor, group: int, *, tau: Optional[float] = None,
                scale: Optional[float] = None, cap: Optional[int] = None, idx: Optional[torch.Tensor] = None,
                counts: Optional[torch.Tensor] = None):
    """Full-attention slice mask from a dense pass's lse (sattn_cached_mask); tau defaults to 0.5 / Nk."""
    lib = _load()
    B, H, Nq, Nk, D = _check_qkv(q, k)
    _check_lse(lse, B, H, Nq, q.device)
    tau = 0.5 / Nk if tau is None else float(tau)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    G = -(-Nq // group)
    if cap is None:
        cap = Nk if idx is None else idx.shape[-1]
    if idx is None:
        idx = torch.empty((B, H, G, cap), dtype=torch.int32, device=q.device)
    if counts is None:
        counts = torch.empty((B, H, G), dtype=torch.int32, device=q.device)
    _check_lists(idx, counts, B, H, G, q.device)
    st = lib.sattn_cached_mask(_ptr(q), _ptr(k), _ptr(lse), B, H, Nq, Nk, D, group, tau, scale, _ptr(idx),
                               _ptr(counts), idx.shape[-1], _stream_ptr(q))
    _check("sattn_cached_mask", st)
    return idx, counts


def colsum_mask(q: torch.Tensor, k: torch.Tensor, lse: torch.Tensor, group: int, topk: int, *,
                scale: Optional[float] = None, cap: Optional[int] = None, idx: Optional[torch.Tensor] = None,
                counts: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """Top-k keys per group by column sums of attention probabilities with a given lse (sattn_colsum_mask)."""
    lib = _load()
    B, H, Nq, Nk, D = _check_qkv(q, k)
    _check_lse(lse, B, H, Nq, q.device)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    G = -(-Nq // group)
    if cap is None:
        cap = int(topk) if idx is None else idx.shape[-1]
    if idx is None:
        idx = torch.empty((B, H, G, cap), dtype=torch.int32, device=q.device)
    if counts is None:
        counts = torch.empty((B, H, G), dtype=torch.int32, device=q.device)
    _check_lists(idx, counts, B, H, G, q.device)
    need = lib.sattn_mask_workspace_bytes(B, H, Nq, Nk, D, group)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    ws_bytes = _check_workspace(workspace, q.device)
    st = lib.sattn_colsum_mask(_ptr(q), _ptr(k), _ptr(lse), B, H, Nq, Nk, D, group, int(topk), scale, _ptr(idx),
                               _ptr(counts), idx.shape[-1], _ptr(workspace), ws_bytes, _stream_ptr(q))
    _check("sattn_colsum_mask", st)
    return idx, counts


def delta_forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, idx: torch.Tensor, counts: torch.Tensor,
                  group: int, *, lse: torch.Tensor, out_prev: torch.Tensor, fresh: torch.Tensor,
                  scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                  out_dtype: torch.dtype = torch.float32):
    """Chipmunk sparse-delta step (sattn_delta_forward): returns out; updates fresh in place."""
    lib = _load()
    B, H, Nq, Nk, D = _check_qkv(q, k, v)
    G = -(-Nq // group)
    _check_lists(idx, counts, B, H, G, q.device)
    _check_lse(lse, B, H, Nq, q.device)
    for name, t in (("out_prev", out_prev), ("fresh", fresh)):
        if t.dtype != torch.float32 or t.shape != q.shape or not t.is_contiguous() or not t.is_cuda:
            raise ValueError(f"{name} must be a contiguous fp32 device tensor shaped like q")
        _on(q.device, **{name: t})
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    if out is None:
        out = torch.empty((B, H, Nq, D), dtype=out_dtype, device=q.device)
    _check_out(out, q.shape, q.device)
    st = lib.sattn_delta_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(idx), _ptr(counts), idx.shape[-1], B, H, Nq, Nk,
                                 D, group, scale, _ptr(lse), _ptr(out_prev), _ptr(fresh), _ptr(out),
                                 F32 if out.dtype == torch.float32 else BF16, _stream_ptr(q))
    _check("sattn_delta_forward", st)
    return out


def vsmooth_workspace_bytes(B: int, H: int, Nk: int, D: int) -> int:
    return int(_load().sattn_vsmooth_workspace_bytes(B, H, Nk, D))


def vsmooth_quantize(v: torch.Tensor, *, codes: Optional[torch.Tensor] = None, vscale: Optional[torch.Tensor] = None,
                     vmean: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """V-Smooth quantisation (sattn_vsmooth_quantize): returns (codes uint8 [B,H,Nk,D], vscale fp32 [B,H,D],
    vmean bf16 [B,H,D,S] = block mean / vscale, channel-major, S = sattn_vsmooth_mean_stride(Nk))."""
    lib = _load()
    if not v.is_cuda or v.dtype != torch.bfloat16 or v.dim() != 4 or not v.is_contiguous():
        raise ValueError("v must be a contiguous bf16 [B, H, N, D] device tensor")
    B, H, Nk, D = v.shape
    S = lib.sattn_vsmooth_mean_stride(Nk)
    if codes is None:
        codes = torch.empty((B, H, Nk, D), dtype=torch.uint8, device=v.device)
    if vscale is None:
        vscale = torch.empty((B, H, D), dtype=torch.float32, device=v.device)
    if vmean is None:
        vmean = torch.empty((B, H, D, S), dtype=torch.bfloat16, device=v.device)
    if (codes.dtype != torch.uint8 or tuple(codes.shape) != (B, H, Nk, D) or vscale.dtype != torch.float32
            or tuple(vscale.shape) != (B, H, D) or vmean.dtype != torch.bfloat16 or tuple(vmean.shape) != (B, H, D, S)
            or not (codes.is_contiguous() and vscale.is_contiguous() and vmean.is_contiguous())):
        raise ValueError("codes, vscale, vmean: contiguous uint8 [B,H,Nk,D], fp32 [B,H,D], bf16 [B,H,D,S]")
    _on(v.device, codes=codes, vscale=vscale, vmean=vmean)
    need = lib.sattn_vsmooth_workspace_bytes(B, H, Nk, D)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=v.device)
    ws_bytes = _check_workspace(workspace, v.device)
    st = lib.sattn_vsmooth_quantize(_ptr(v), B, H, Nk, D, _ptr(codes), _ptr(vscale), _ptr(vmean), _ptr(workspace),
                                    ws_bytes, _stream_ptr(v))
    _check("sattn_vsmooth_quantize", st)
    return codes, vscale, vmean


def fp8_forward(q: torch.Tensor, k: torch.Tensor, codes: torch.Tensor, vscale: torch.Tensor, vmean: torch.Tensor,
                idx: torch.Tensor, counts: torch.Tensor, group: int, *, scale: Optional[float] = None,
                out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                out_dtype: torch.dtype = torch.float32, want_lse: bool = True):
    """Sparse forward with ExpCast bytes and the E4M3 P.V product (sattn_fp8_forward).  Returns (out, lse)."""
    lib = _load()
    B, H, Nq, Nk, D = _check_qkv(q, k)
    G = -(-Nq // group)
    S = lib.sattn_vsmooth_mean_stride(Nk)
    _check_lists(idx, counts, B, H, G, q.device)
    if (codes.dtype != torch.uint8 or tuple(codes.shape) != (B, H, Nk, D) or vscale.dtype != torch.float32
            or tuple(vscale.shape) != (B, H, D) or vmean.dtype != torch.bfloat16 or tuple(vmean.shape) != (B, H, D, S)
            or not (codes.is_contiguous() and vscale.is_contiguous() and vmean.is_contiguous())):
        raise ValueError("codes, vscale, vmean must be what vsmooth_quantize returns for a V shaped like k")
    _on(q.device, codes=codes, vscale=vscale, vmean=vmean)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    if out is None:
        out = torch.empty((B, H, Nq, D), dtype=out_dtype, device=q.device)
    _check_out(out, q.shape, q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _check_lse(lse, B, H, Nq, q.device)
    st = lib.sattn_fp8_forward(_ptr(q), _ptr(k), _ptr(codes), _ptr(vscale), _ptr(vmean), _ptr(idx), _ptr(counts),
                               idx.shape[-1], B, H, Nq, Nk, D, group, scale, _ptr(out),
                               F32 if out.dtype == torch.float32 else BF16, _ptr(lse), _stream_ptr(q))
    _check("sattn_fp8_forward", st)
    return out, lse


def mx4_quantize(x: torch.Tensor, *, codes: Optional[torch.Tensor] = None, scales: Optional[torch.Tensor] = None):
    """MXFP4 quantisation of bf16 queries or keys (sattn_mx4_quantize): returns (codes uint8 [B,H,N,D/2],
    scales uint8 [B,H,N,4])."""
    lib = _load()
    if not x.is_cuda or x.dtype != torch.bfloat16 or x.dim() != 4 or not x.is_contiguous():
        raise ValueError("x must be a contiguous bf16 [B, H, N, D] device tensor")
    B, H, N, D = x.shape
    if codes is None:
        codes = torch.empty((B, H, N, D // 2), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((B, H, N, 4), dtype=torch.uint8, device=x.device)
    if (codes.dtype != torch.uint8 or tuple(codes.shape) != (B, H, N, D // 2) or scales.dtype != torch.uint8
            or tuple(scales.shape) != (B, H, N, 4) or not codes.is_contiguous() or not scales.is_contiguous()):
        raise ValueError("codes must be contiguous uint8 [B,H,N,D/2] and scales uint8 [B,H,N,4]")
    _on(x.device, codes=codes, scales=scales)
    _check("sattn_mx4_quantize", lib.sattn_mx4_quantize(_ptr(x), B, H, N, D, _ptr(codes), _ptr(scales), _stream_ptr(x)))
    return codes, scales


def fp4_forward(q4: torch.Tensor, q_scales: torch.Tensor, k4: torch.Tensor, k_scales: torch.Tensor,
                codes: torch.Tensor, vscale: torch.Tensor, vmean: torch.Tensor, idx: torch.Tensor,
                counts: torch.Tensor, group: int, *, scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                lse: Optional[torch.Tensor] = None, out_dtype: torch.dtype = torch.float32, want_lse: bool = True):
    """4-bit QK^T + FP8 value path (sattn_fp4_forward).  Returns (out, lse)."""
    lib = _load()
    for name, t in (("q4", q4), ("k4", k4), ("q_scales", q_scales), ("k_scales", k_scales)):
        if not t.is_cuda or t.dtype != torch.uint8 or t.dim() != 4 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous uint8 [B, H, N, *] device tensor")
    B, H, Nq, D2 = q4.shape
    D = 2 * D2
    Nk = k4.shape[2]
    if tuple(k4.shape) != (B, H, Nk, D2) or tuple(q_scales.shape) != (B, H, Nq, 4) or tuple(k_scales.shape) != (B, H, Nk, 4):
        raise ValueError("q4 / k4 must be [B,H,N,D/2] and their scales [B,H,N,4] (mx4_quantize)")
    G = -(-Nq // group)
    S = lib.sattn_vsmooth_mean_stride(Nk)
    _check_lists(idx, counts, B, H, G, q4.device)
    if (codes.dtype != torch.uint8 or tuple(codes.shape) != (B, H, Nk, D) or vscale.dtype != torch.float32
            or tuple(vscale.shape) != (B, H, D) or vmean.dtype != torch.bfloat16 or tuple(vmean.shape) != (B, H, D, S)
            or not (codes.is_contiguous() and vscale.is_contiguous() and vmean.is_contiguous())):
        raise ValueError("codes, vscale, vmean must be what vsmooth_quantize returns for V")
    _on(q4.device, k4=k4, q_scales=q_scales, k_scales=k_scales, codes=codes, vscale=vscale, vmean=vmean)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    if out is None:
        out = torch.empty((B, H, Nq, D), dtype=out_dtype, device=q4.device)
    _check_out(out, (B, H, Nq, D), q4.device)
    if lse is None and want_lse:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q4.device)
    if lse is not None:
        _check_lse(lse, B, H, Nq, q4.device)
    st = lib.sattn_fp4_forward(_ptr(q4), _ptr(q_scales), _ptr(k4), _ptr(k_scales), _ptr(codes), _ptr(vscale), _ptr(vmean),
                               _ptr(idx), _ptr(counts), idx.shape[-1], B, H, Nq, Nk, D, group, scale, _ptr(out),
                               F32 if out.dtype == torch.float32 else BF16, _ptr(lse), _stream_ptr(q4))
    _check("sattn_fp4_forward", st)
    return out, lse


def voxel_permutation(grid, voxel) -> torch.Tensor:
    """Host int32 permutation that makes every run of prod(voxel) tokens one voxel (sattn_voxel_permutation)."""
    lib = _load()
    T, Hg, Wg = grid
    perm = torch.empty(T * Hg * Wg, dtype=torch.int32)
    _check("sattn_voxel_permutation", lib.sattn_voxel_permutation(T, Hg, Wg, *voxel, _ptr(perm)))
    return perm


def permute_tokens(x: torch.Tensor, perm: torch.Tensor, inverse: bool = False,
                   out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Reorder the tokens of a bf16 [B,H,N,D] device tensor by a device int32 permutation."""
    lib = _load()
    if not x.is_cuda or x.dtype != torch.bfloat16 or x.dim() != 4 or not x.is_contiguous():
        raise ValueError("x must be a contiguous bf16 [B, H, N, D] device tensor")
    B, H, N, D = x.shape
    if out is None:
        out = torch.empty_like(x)
    if out.dtype != torch.bfloat16 or out.shape != x.shape or not out.is_contiguous():
        raise ValueError("out must be a contiguous bf16 tensor shaped like x")
    if perm.dtype != torch.int32 or perm.numel() != N or not perm.is_contiguous():
        raise ValueError("perm must be a contiguous device int32 tensor of N entries")
    _on(x.device, out=out, perm=perm)
    _check("sattn_permute_tokens", lib.sattn_permute_tokens(_ptr(x), _ptr(out), _ptr(perm), B, H, N, D,
                                                            1 if inverse else 0, _stream_ptr(x)))
    return out
