"""MI355X (gfx950) gathered sparse attention with per-head sinks.

Thin Python binding over the C ABI of include/sparse_attn.h: it checks tensor
devices, dtypes, shapes and contiguity, allocates outputs with torch and passes
torch's current HIP stream. Every step of the computation runs in the HIP
kernels of libsparse_attn.so; there is no other implementation to fall back on.

decode()       per-sequence caches: q [B,H,512], k/v [B,N,512], idx [B,kmax]
prefill()      one shared cache:    q [T,H,512], k/v [N,512],   idx [T,kmax]
topk()         exact per-row top-k of indexer scores (ascending, -1 padded)
pad_heads() / unpad_heads()   zero-padding of heads into a wider launch
"""
from __future__ import annotations

from typing import Optional, Tuple

import torch

from . import _lib
from ._lib import SA_BF16, SA_F32, SparseAttnError, load

HEAD_DIM = 512
__all__ = ["decode", "decode_noalloc", "prefill", "topk", "pad_heads", "unpad_heads", "workspace_bytes", "load",
           "SparseAttnError", "HEAD_DIM"]


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _need(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


def _on_device(ref: torch.Tensor, ref_name: str, **tensors) -> None:
    """Every given tensor (None allowed) lives on ref's device, and that device is a HIP
    device: a host tensor's pointer must never reach a kernel as a device pointer."""
    for name, t in tensors.items():
        if t is not None:
            _need(isinstance(t, torch.Tensor), f"{name} must be a torch.Tensor")
            _need(t.device == ref.device, f"{name} is on {t.device}, {ref_name} on {ref.device}")
    _need(ref.is_cuda, f"{ref_name} must be on a HIP device, not {ref.device}")


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return SA_BF16
    if t.dtype == torch.float32:
        return SA_F32
    raise ValueError(f"q/k/v must be bfloat16 or float32, got {t.dtype}")


def _attn(shared: bool, q, k_cache, v_cache, idx, sinks, scale, nsel, out, ws):
    _need(q.dim() == 3, "q must be [rows, H, D]")
    rows, H, D = q.shape
    _on_device(q, "q", k_cache=k_cache, v_cache=v_cache, idx=idx, sinks=sinks, nsel=nsel, out=out, ws=ws)
    lib = load()
    code = _dtype_code(q)
    _need(k_cache.dtype == q.dtype and v_cache.dtype == q.dtype, "q, k_cache and v_cache must share a dtype")
    if shared:
        _need(k_cache.dim() == 2 and k_cache.shape[1] == D, "prefill caches are [N, D]")
        n_ctx = k_cache.shape[0]
    else:
        _need(k_cache.dim() == 3 and k_cache.shape[0] == rows and k_cache.shape[2] == D,
              "decode caches are [B, N, D]")
        n_ctx = k_cache.shape[1]
    _need(v_cache.shape == k_cache.shape, "k_cache and v_cache shapes differ")
    _need(idx.dtype == torch.int32 and idx.dim() == 2 and idx.shape[0] == rows, "idx must be int32 [rows, kmax]")
    _need(sinks.dtype == torch.float32 and sinks.shape == (H,), "sinks must be float32 [H]")
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache), ("idx", idx), ("sinks", sinks)):
        _need(t.is_contiguous(), f"{name} must be contiguous")
    if nsel is not None:
        _need(nsel.dtype == torch.int32 and nsel.shape == (rows,) and nsel.is_contiguous(),
              "nsel must be contiguous int32 [rows]")
    if out is None:
        out = torch.empty((rows, H, D), dtype=torch.float32, device=q.device)
    _need(out.dtype == torch.float32 and out.shape == (rows, H, D) and out.is_contiguous(),
          "out must be contiguous float32 [rows, H, D]")
    kmax = idx.shape[1]
    need = 0
    if 1 <= kmax <= _lib.SA_MAX_KMAX:
        need = int(lib.sparse_attn_workspace_bytes(_lib.SA_OP_PREFILL if shared else _lib.SA_OP_DECODE,
                                                   rows, H, D, kmax, n_ctx))
    if ws is None and need > 0:
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    if ws is not None:
        _need(ws.dtype == torch.uint8 and ws.dim() == 1 and ws.is_contiguous(), "ws must be contiguous uint8 [bytes]")
    fn = lib.sparse_attn_prefill if shared else lib.sparse_attn_decode
    rc = fn(code, _ptr(q), _ptr(k_cache), _ptr(v_cache), n_ctx, _ptr(idx), _ptr(nsel), kmax,
            _ptr(sinks), float(scale), rows, H, D, _ptr(out), _ptr(ws), 0 if ws is None else ws.numel(), _stream(q))
    _lib.check(rc, fn.__name__, lib)
    return out


def decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, idx: torch.Tensor,
           sinks: torch.Tensor, scale: float, nsel: Optional[torch.Tensor] = None,
           out: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """sparse_attn_decode: B sequences, each with its own cache. Returns float32 [B, H, 512].

    ws: optional uint8 device workspace of at least workspace_bytes(SA_OP_DECODE, ...) bytes;
    allocated here when needed and not given."""
    return _attn(False, q, k_cache, v_cache, idx, sinks, scale, nsel, out, ws)


def prefill(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, idx: torch.Tensor,
            sinks: torch.Tensor, scale: float, nsel: Optional[torch.Tensor] = None,
            out: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """sparse_attn_prefill: T rows over one shared cache [N, 512]. Returns float32 [T, H, 512]."""
    return _attn(True, q, k_cache, v_cache, idx, sinks, scale, nsel, out, ws)


def decode_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, idx: torch.Tensor,
                   sinks: torch.Tensor, scale: float, nsel: Optional[torch.Tensor] = None,
                   out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """sparse_attn_decode_noalloc: decode with the library's static scratch as workspace (no device
    allocation by the library; pass `out` to allocate nothing at all). Calls that overlap on one GPU
    race on the scratch."""
    _need(q.dim() == 3, "q must be [rows, H, D]")
    rows, H, D = q.shape
    _on_device(q, "q", k_cache=k_cache, v_cache=v_cache, idx=idx, sinks=sinks, nsel=nsel, out=out)
    lib = load()
    code = _dtype_code(q)
    _need(k_cache.dtype == q.dtype and v_cache.dtype == q.dtype, "q, k_cache and v_cache must share a dtype")
    _need(k_cache.dim() == 3 and k_cache.shape[0] == rows and k_cache.shape[2] == D and v_cache.shape == k_cache.shape,
          "decode caches are [B, N, D]")
    _need(idx.dtype == torch.int32 and idx.dim() == 2 and idx.shape[0] == rows, "idx must be int32 [rows, kmax]")
    _need(sinks.dtype == torch.float32 and sinks.shape == (H,), "sinks must be float32 [H]")
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache), ("idx", idx), ("sinks", sinks)):
        _need(t.is_contiguous(), f"{name} must be contiguous")
    if nsel is not None:
        _need(nsel.dtype == torch.int32 and nsel.shape == (rows,) and nsel.is_contiguous(),
              "nsel must be contiguous int32 [rows]")
    if out is None:
        out = torch.empty((rows, H, D), dtype=torch.float32, device=q.device)
    _need(out.dtype == torch.float32 and out.shape == (rows, H, D) and out.is_contiguous(),
          "out must be contiguous float32 [rows, H, D]")
    rc = lib.sparse_attn_decode_noalloc(code, _ptr(q), _ptr(k_cache), _ptr(v_cache), k_cache.shape[1], _ptr(idx),
                                        _ptr(nsel), idx.shape[1], _ptr(sinks), float(scale), rows, H, D, _ptr(out),
                                        _stream(q))
    _lib.check(rc, "sparse_attn_decode_noalloc", lib)
    return out


def topk(scores: torch.Tensor, k: int, valid_len: Optional[torch.Tensor] = None,
         idx_out: Optional[torch.Tensor] = None,
         count_out: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """sparse_attn_topk: exact top-k per row. Returns (idx int32 [R, k], count int32 [R])."""
    _on_device(scores, "scores", valid_len=valid_len, idx_out=idx_out, count_out=count_out)
    lib = load()
    _need(scores.dtype == torch.float32 and scores.dim() == 2, "scores must be float32 [rows, n]")
    _need(scores.stride(1) == 1, "scores rows must be contiguous")
    rows, n = scores.shape
    ld = scores.stride(0) if rows > 1 else n
    if valid_len is not None:
        _need(valid_len.dtype == torch.int32 and valid_len.shape == (rows,) and valid_len.is_contiguous(),
              "valid_len must be contiguous int32 [rows]")
    if idx_out is None:
        idx_out = torch.empty((rows, k), dtype=torch.int32, device=scores.device)
    if count_out is None:
        count_out = torch.empty((rows,), dtype=torch.int32, device=scores.device)
    _need(idx_out.shape == (rows, k) and idx_out.dtype == torch.int32 and idx_out.is_contiguous(),
          "idx_out must be contiguous int32 [rows, k]")
    _need(count_out.shape == (rows,) and count_out.dtype == torch.int32 and count_out.is_contiguous(),
          "count_out must be contiguous int32 [rows]")
    rc = lib.sparse_attn_topk(_ptr(scores), rows, n, ld, _ptr(valid_len), int(k), _ptr(idx_out),
                              _ptr(count_out), None, 0, _stream(scores))
    _lib.check(rc, "sparse_attn_topk", lib)
    return idx_out, count_out


def pad_heads(q: torch.Tensor, sinks: torch.Tensor, h_pad: int, q_pad: Optional[torch.Tensor] = None,
              s_pad: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """sparse_attn_pad_heads: q [R, h, 512] -> [R, h_pad, 512] with zero heads; sinks -> zero-padded."""
    _need(q.dim() == 3, "q must be [rows, h, D]")
    rows, h, D = q.shape
    _on_device(q, "q", sinks=sinks, q_pad=q_pad, s_pad=s_pad)
    lib = load()
    _need(q.is_contiguous() and sinks.is_contiguous() and sinks.dtype == torch.float32 and sinks.shape == (h,),
          "q must be contiguous, sinks contiguous float32 [h]")
    if q_pad is None:
        q_pad = torch.empty((rows, h_pad, D), dtype=q.dtype, device=q.device)
    if s_pad is None:
        s_pad = torch.empty((h_pad,), dtype=torch.float32, device=q.device)
    _need(q_pad.shape == (rows, h_pad, D) and q_pad.dtype == q.dtype and q_pad.is_contiguous()
          and s_pad.shape == (h_pad,) and s_pad.dtype == torch.float32, "q_pad / s_pad")
    rc = lib.sparse_attn_pad_heads(_dtype_code(q), _ptr(q), rows, h, h_pad, D, _ptr(sinks), _ptr(q_pad),
                                   _ptr(s_pad), _stream(q))
    _lib.check(rc, "sparse_attn_pad_heads", lib)
    return q_pad, s_pad


def unpad_heads(out_pad: torch.Tensor, h_real: int, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """sparse_attn_unpad_heads: heads 0..h_real-1 of out_pad [R, h_pad, 512] (float32)."""
    _need(out_pad.dim() == 3, "out_pad must be [rows, h_pad, D]")
    rows, h_pad, D = out_pad.shape
    _on_device(out_pad, "out_pad", out=out)
    lib = load()
    _need(out_pad.is_contiguous() and out_pad.dtype == torch.float32, "out_pad must be contiguous float32")
    if out is None:
        out = torch.empty((rows, h_real, D), dtype=torch.float32, device=out_pad.device)
    _need(out.shape == (rows, h_real, D) and out.dtype == torch.float32 and out.is_contiguous(), "out")
    rc = lib.sparse_attn_unpad_heads(_ptr(out_pad), rows, h_pad, h_real, D, _ptr(out), _stream(out_pad))
    _lib.check(rc, "sparse_attn_unpad_heads", lib)
    return out


def gather_probe(k_cache: torch.Tensor, v_cache: torch.Tensor, idx: torch.Tensor, rows_in_flight: int = 16) -> None:
    """sparse_attn_gather_probe: the decode kernels' gathers alone (a bandwidth reference for benchmarks)."""
    _on_device(k_cache, "k_cache", v_cache=v_cache, idx=idx)
    lib = load()
    _need(k_cache.dtype == torch.bfloat16 and k_cache.dim() == 3 and k_cache.shape[2] == HEAD_DIM
          and v_cache.shape == k_cache.shape and v_cache.dtype == k_cache.dtype
          and k_cache.is_contiguous() and v_cache.is_contiguous(), "caches must be contiguous bf16 [B, N, 512]")
    _need(idx.dtype == torch.int32 and idx.dim() == 2 and idx.shape[0] == k_cache.shape[0] and idx.is_contiguous(),
          "idx must be contiguous int32 [B, kmax]")
    rc = lib.sparse_attn_gather_probe(_ptr(k_cache), _ptr(v_cache), k_cache.shape[1], _ptr(idx), idx.shape[0],
                                      idx.shape[1], int(rows_in_flight), _stream(k_cache))
    _lib.check(rc, "sparse_attn_gather_probe", lib)


def workspace_bytes(op: int, rows: int, heads: int, kmax: int, n_ctx: int) -> int:
    return int(load().sparse_attn_workspace_bytes(op, rows, heads, HEAD_DIM, kmax, n_ctx))
