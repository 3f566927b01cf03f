"""Torch-tensor front end of the C ABI: allocation and stream plumbing only."""
from __future__ import annotations

import math

import torch

from . import _abi


def _stream_handle(device: torch.device) -> int:
    return int(torch.cuda.current_stream(device).cuda_stream)


def _check_attn(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor):
    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise ValueError("q, k, v must be GPU tensors")
    if q.dim() != 4 or q.shape != k.shape or q.shape != v.shape:
        raise ValueError("q, k, v must share one [B, H, N, d] shape")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("q, k, v must all be bfloat16 or all float32")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous [B, H, N, d]")


def attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
              scale: float | None = None, out: torch.Tensor | None = None,
              lse: torch.Tensor | None = None):
    """O = softmax(scale q k^T) v per (batch, head), and the row logsumexp.

    q, k, v: contiguous [B, H, N, d] bf16 (fp32 accumulation) or fp32.
    Returns (O with q's dtype, lse fp32 [B, H, N]).  scale defaults to 1/sqrt(d).
    """
    _check_attn(q, k, v)
    B, H, N, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor like q")
    if lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B, H, N] tensor")
    fn = _abi.attn_fwd if q.dtype == torch.bfloat16 else _abi.attn_fwd_f32
    with torch.cuda.device(q.device):
        fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
           B, H, N, d, scale, causal, _stream_handle(q.device))
    return out, lse


def softmax(x: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """Stable softmax over the last dimension of a contiguous fp32 [B, N] GPU tensor.
    ``out`` may be ``x`` itself (in place)."""
    if not x.is_cuda or x.dtype != torch.float32 or x.dim() != 2 or not x.is_contiguous():
        raise ValueError("x must be a contiguous float32 [B, N] GPU tensor")
    if out is None:
        out = torch.empty_like(x)
    if out.shape != x.shape or out.dtype != x.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor like x")
    B, N = x.shape
    with torch.cuda.device(x.device):
        _abi.row_softmax(x.data_ptr(), out.data_ptr(), B, N, _stream_handle(x.device))
    return out
