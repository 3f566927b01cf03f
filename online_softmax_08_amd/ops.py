"""Torch-tensor front end of the C ABI: allocation and stream plumbing only."""
from __future__ import annotations

import math

import torch

from . import _abi


def _stream_handle(device: torch.device) -> int:
    return int(torch.cuda.current_stream(device).cuda_stream)


def _check_attn(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor):
    """q [B, H, N, d]; k, v [B, Hkv, N, d] with Hkv dividing H (grouped-query
    attention; Hkv = H is plain multi-head attention)."""
    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise ValueError("q, k, v must be GPU tensors")
    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape:
        raise ValueError("q must be [B, H, N, d] and k, v one [B, Hkv, N, d] shape")
    B, H, N, d = q.shape
    if k.shape[0] != B or k.shape[2] != N or k.shape[3] != d or k.shape[1] < 1 or H % k.shape[1]:
        raise ValueError("k, v must be [B, Hkv, N, d] with Hkv dividing q's H")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("q, k, v must all be bfloat16 or all float32")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous [B, H, N, d]")


def attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
              scale: float | None = None, out: torch.Tensor | None = None,
              lse: torch.Tensor | None = None):
    """O = softmax(scale q k^T) v per (batch, head), and the row logsumexp.

    q: contiguous [B, H, N, d], k, v: [B, Hkv, N, d] (Hkv dividing H; query
    head h reads key/value head h // (H // Hkv)), bf16 (fp32 accumulation) or
    fp32 (Hkv = H only).  Returns (O with q's dtype, lse fp32 [B, H, N]).
    scale defaults to 1/sqrt(d).
    """
    _check_attn(q, k, v)
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    if q.dtype == torch.float32 and Hkv != H:
        raise ValueError("the fp32 path takes as many key/value heads as query heads")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor like q")
    if lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B, H, N] tensor")
    with torch.cuda.device(q.device):
        args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr())
        if q.dtype == torch.float32:
            _abi.attn_fwd_f32(*args, B, H, N, d, scale, causal, _stream_handle(q.device))
        elif Hkv == H:
            _abi.attn_fwd(*args, B, H, N, d, scale, causal, _stream_handle(q.device))
        else:
            _abi.attn_fwd_gqa(*args, B, H, Hkv, N, d, scale, causal, _stream_handle(q.device))
    return out, lse


def attention_fp8(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, q_scale: float,
                  k_scale: float, v_scale: float, causal: bool = False,
                  scale: float | None = None):
    """attention() on fp8 inputs: q [B, H, N, d], k, v [B, Hkv, N, d] holding OCP
    FP8 E4M3 codes (torch.uint8 or torch.float8_e4m3fn, contiguous, on one GPU),
    each element standing for its decoded value times the tensor's scale.
    Returns (O bf16 [B, H, N, d], lse fp32 [B, H, N]); scale defaults to
    1/sqrt(d).
    """
    ts = (q, k, v)
    if not all(t.is_cuda for t in ts):
        raise ValueError("q, k, v must be GPU tensors")
    if not all(t.dtype in (torch.uint8, torch.float8_e4m3fn) for t in ts):
        raise ValueError("q, k, v must hold FP8 E4M3 codes (uint8 or float8_e4m3fn)")
    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape or not all(t.is_contiguous() for t in ts):
        raise ValueError("q must be [B, H, N, d] and k, v one [B, Hkv, N, d] shape, contiguous")
    B, H, N, d = q.shape
    if k.shape[0] != B or k.shape[2] != N or k.shape[3] != d or k.shape[1] < 1 or H % k.shape[1]:
        raise ValueError("k, v must be [B, Hkv, N, d] with Hkv dividing q's H")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    out = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=q.device)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    with torch.cuda.device(q.device):
        _abi.attn_fwd_fp8(q.data_ptr(), k.data_ptr(), v.data_ptr(), float(q_scale), float(k_scale),
                          float(v_scale), out.data_ptr(), lse.data_ptr(), B, H, k.shape[1], N, d,
                          scale, causal, _stream_handle(q.device))
    return out, lse


def quantize_fp8_rows(x: torch.Tensor, signs=None):
    """Block quantization of a bf16 tensor [..., d] (contiguous, on a GPU) along
    its last axis: one power-of-two scale per 32 elements, after the
    random-sign Hadamard rotation when signs (d values +-1, any sequence or
    CPU tensor) is given.  Returns (codes uint8 [..., d], scale bytes uint8
    [..., d / 32])."""
    if not x.is_cuda or x.dtype != torch.bfloat16 or not x.is_contiguous():
        raise ValueError("x must be a contiguous bf16 GPU tensor")
    d = x.shape[-1]
    rows = x.numel() // d if d else 0
    if signs is not None:
        signs = [int(s) for s in (signs.tolist() if isinstance(signs, torch.Tensor) else signs)]
        if len(signs) != d:
            raise ValueError("signs must hold d values")
    codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    scales = torch.empty(tuple(x.shape[:-1]) + (d // 32,), dtype=torch.uint8, device=x.device)
    with torch.cuda.device(x.device):
        _abi.fp8_quantize_rows(x.data_ptr(), signs, codes.data_ptr(), scales.data_ptr(), rows, d,
                               _stream_handle(x.device))
    return codes, scales


def quantize_fp8_cols(x: torch.Tensor):
    """Block quantization of a bf16 tensor [..., n, d] along the rows of each
    column of every [n, d] slice (the layout attention_fp8_mx takes for V).
    Returns (codes uint8 [..., n, d], scale bytes uint8 [..., ceil(n / 32), d])."""
    if not x.is_cuda or x.dtype != torch.bfloat16 or not x.is_contiguous() or x.dim() < 2:
        raise ValueError("x must be a contiguous bf16 GPU tensor [..., n, d]")
    n, d = x.shape[-2], x.shape[-1]
    slices = x.numel() // (n * d) if n * d else 0
    codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    scales = torch.empty(tuple(x.shape[:-2]) + ((n + 31) // 32, d), dtype=torch.uint8,
                         device=x.device)
    with torch.cuda.device(x.device):
        _abi.fp8_quantize_cols(x.data_ptr(), codes.data_ptr(), scales.data_ptr(), slices, n, d,
                               _stream_handle(x.device))
    return codes, scales


def attention_fp8_mx(q8: torch.Tensor, q_scales: torch.Tensor, k8: torch.Tensor,
                     k_scales: torch.Tensor, v8: torch.Tensor, v_scales: torch.Tensor,
                     causal: bool = False, scale: float | None = None):
    """attention() on block-quantized fp8 inputs: codes q8 [B, H, N, d], k8, v8
    [B, Hkv, N, d] (uint8 or float8_e4m3fn) with scale bytes q_scales
    [B, H, N, d/32], k_scales [B, Hkv, N, d/32], v_scales [B, Hkv, ceil(N/32), d]
    (what quantize_fp8_rows / quantize_fp8_cols return).  Returns (O bf16,
    lse fp32); scale defaults to 1/sqrt(d)."""
    ts = (q8, k8, v8, q_scales, k_scales, v_scales)
    if not all(t.is_cuda and t.is_contiguous() for t in ts):
        raise ValueError("every tensor must be a contiguous GPU tensor")
    if not all(t.dtype in (torch.uint8, torch.float8_e4m3fn) for t in (q8, k8, v8)):
        raise ValueError("q8, k8, v8 must hold FP8 E4M3 codes (uint8 or float8_e4m3fn)")
    if not all(t.dtype == torch.uint8 for t in (q_scales, k_scales, v_scales)):
        raise ValueError("scale bytes must be uint8")
    if q8.dim() != 4 or k8.shape != v8.shape:
        raise ValueError("q8 must be [B, H, N, d] and k8, v8 one [B, Hkv, N, d] shape")
    B, H, N, d = q8.shape
    Hkv = k8.shape[1]
    if k8.shape[0] != B or k8.shape[2] != N or k8.shape[3] != d or Hkv < 1 or H % Hkv:
        raise ValueError("k8, v8 must be [B, Hkv, N, d] with Hkv dividing q8's H")
    if (q_scales.shape != (B, H, N, d // 32) or k_scales.shape != (B, Hkv, N, d // 32)
            or v_scales.shape != (B, Hkv, (N + 31) // 32, d)):
        raise ValueError("scale bytes must be [B, H, N, d/32], [B, Hkv, N, d/32] and "
                         "[B, Hkv, ceil(N/32), d]")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    out = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=q8.device)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q8.device)
    with torch.cuda.device(q8.device):
        _abi.attn_fwd_fp8_mx(q8.data_ptr(), q_scales.data_ptr(), k8.data_ptr(), k_scales.data_ptr(),
                             v8.data_ptr(), v_scales.data_ptr(), out.data_ptr(), lse.data_ptr(),
                             B, H, Hkv, N, d, scale, causal, _stream_handle(q8.device))
    return out, lse


def attention_fp8_block(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, signs=None,
                        causal: bool = False, scale: float | None = None):
    """FP8 attention of bf16 q, k, v with the accuracy devices of the FP8
    method: q and k rotated by diag(signs) H / sqrt(d) (skipped when signs is
    None) and block-quantized along the head dimension, v block-quantized
    along the keys, then attention_fp8_mx.  Every step runs in the HIP
    library.  Returns (O bf16, lse fp32), the attention of the unrotated
    inputs up to the fp8 error."""
    q8, qs = quantize_fp8_rows(q, signs)
    k8, ks = quantize_fp8_rows(k, signs)
    v8, vs = quantize_fp8_cols(v)
    return attention_fp8_mx(q8, qs, k8, ks, v8, vs, causal=causal, scale=scale)


def attention_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                     cu_seqlens: torch.Tensor, max_seqlen: int, causal: bool = False,
                     scale: float | None = None):
    """Attention over packed variable-length sequences.

    q: contiguous bf16 [H, total, d] (every head's rows of all sequences end
    to end), k, v: [Hkv, total, d]; cu_seqlens: int32 GPU tensor [B + 1] of row offsets;
    max_seqlen: an upper bound of the lengths.  Returns (O bf16 [H, total, d],
    lse fp32 [H, total]).
    """
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda or t.dtype != torch.bfloat16 or t.dim() != 3 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous bfloat16 [heads, total, d] GPU tensor")
    if (k.shape != v.shape or k.shape[1:] != q.shape[1:] or k.shape[0] < 1
            or q.shape[0] % k.shape[0]):
        raise ValueError("q must be [H, total, d] and k, v [Hkv, total, d], Hkv dividing H")
    if (not cu_seqlens.is_cuda or cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1
            or not cu_seqlens.is_contiguous() or cu_seqlens.device != q.device):
        raise ValueError("cu_seqlens must be a contiguous int32 [B + 1] tensor on q's device")
    H, total, d = q.shape
    B = cu_seqlens.numel() - 1
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    out = torch.empty_like(q)
    lse = torch.empty((H, total), dtype=torch.float32, device=q.device)
    with torch.cuda.device(q.device):
        _abi.attn_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                             lse.data_ptr(), cu_seqlens.data_ptr(), max(B, 0), H, k.shape[0],
                             total, int(max_seqlen), d, scale, causal, _stream_handle(q.device))
    return out, lse


def attention_splitkv(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
                      scale: float | None = None, nsplit: int = 0,
                      workspace: torch.Tensor | None = None):
    """attention() for bf16 with the keys split into nsplit parallel ranges and
    the partial results merged (nsplit 0: the library's choice).

    ``workspace`` (optional) is a device uint8 tensor of at least the planned
    size; otherwise one is allocated.  Returns (O bf16, lse fp32 [B, H, N]).
    """
    _check_attn(q, k, v)
    if q.dtype != torch.bfloat16:
        raise ValueError("split-KV attention takes bfloat16 q, k, v")
    B, H, N, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    ns, ws_bytes = _abi.attn_fwd_splitkv_plan(B, H, N, d, causal, nsplit)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device)
    if not workspace.is_cuda or workspace.device != q.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on q's device")
    out = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    with torch.cuda.device(q.device):
        _abi.attn_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                              lse.data_ptr(), B, H, k.shape[1], N, d, scale, causal, ns,
                              workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                              _stream_handle(q.device))
    return out, lse


def attention_combine(o_part: torch.Tensor, lse_part: torch.Tensor):
    """Merge partial attention results over disjoint key sets.

    o_part: contiguous fp32 [S, B, H, N, d] (each normalised over its keys);
    lse_part: contiguous fp32 [S, B, H, N] (-inf: the partial saw no key).
    Returns (O bf16 [B, H, N, d], lse fp32 [B, H, N]).
    """
    if not (o_part.is_cuda and lse_part.is_cuda):
        raise ValueError("o_part and lse_part must be GPU tensors")
    if o_part.dtype != torch.float32 or lse_part.dtype != torch.float32:
        raise ValueError("o_part and lse_part must be float32")
    if o_part.dim() != 5 or tuple(lse_part.shape) != tuple(o_part.shape[:4]):
        raise ValueError("o_part must be [S, B, H, N, d] and lse_part [S, B, H, N]")
    if not (o_part.is_contiguous() and lse_part.is_contiguous()):
        raise ValueError("o_part and lse_part must be contiguous")
    S, B, H, N, d = o_part.shape
    out = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=o_part.device)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=o_part.device)
    with torch.cuda.device(o_part.device):
        _abi.attn_combine(o_part.data_ptr(), lse_part.data_ptr(), out.data_ptr(), lse.data_ptr(),
                          S, B, H, N, d, _stream_handle(o_part.device))
    return out, lse


def attention_backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor,
                       lse: torch.Tensor, grad_out: torch.Tensor, causal: bool = False,
                       scale: float | None = None, workspace: torch.Tensor | None = None):
    """Gradients (dq, dk, dv) of sum(grad_out * out) for out, lse = attention(q, k, v).

    q, out, grad_out: contiguous bf16 [B, H, N, d]; k, v: [B, Hkv, N, d]; lse:
    fp32 [B, H, N] from the same forward call.  dk, dv have k's shape.  ``workspace`` (optional) is a device
    uint8 tensor of at least attn_bwd_workspace_bytes(B, H, N) bytes.
    """
    _check_attn(q, k, v)
    if q.dtype != torch.bfloat16:
        raise ValueError("the backward pass takes bfloat16 q, k, v")
    for name, tsr in (("out", out), ("grad_out", grad_out)):
        if tsr.shape != q.shape or tsr.dtype != q.dtype or not tsr.is_contiguous() or tsr.device != q.device:
            raise ValueError(f"{name} must be a contiguous tensor like q")
    B, H, N, d = q.shape
    if lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B, H, N] tensor")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    ws_bytes = _abi.attn_bwd_workspace_bytes(B, H, N)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    with torch.cuda.device(q.device):
        _abi.attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                      grad_out.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                      dv.data_ptr(), B, H, k.shape[1], N, d, scale, causal, workspace.data_ptr(),
                      workspace.numel() * workspace.element_size(), _stream_handle(q.device))
    return dq, dk, dv


def attention_backward_split(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                             out: torch.Tensor, lse: torch.Tensor, grad_out: torch.Tensor,
                             causal: bool = False, scale: float | None = None, nsplit: int = 0,
                             workspace: torch.Tensor | None = None):
    """attention_backward() with the dK/dV query loop and the dQ key loop split
    into nsplit parallel ranges whose fp32 partials are summed (nsplit 0: the
    library's choice; it splits only small grids).

    ``workspace`` (optional) is a device uint8 tensor of at least the planned
    size (attn_bwd_split_plan); otherwise one is allocated.  Returns
    (dq, dk, dv).
    """
    _check_attn(q, k, v)
    if q.dtype != torch.bfloat16:
        raise ValueError("the backward pass takes bfloat16 q, k, v")
    for name, tsr in (("out", out), ("grad_out", grad_out)):
        if tsr.shape != q.shape or tsr.dtype != q.dtype or not tsr.is_contiguous() or tsr.device != q.device:
            raise ValueError(f"{name} must be a contiguous tensor like q")
    B, H, N, d = q.shape
    if lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B, H, N] tensor")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    ns, ws_bytes = _abi.attn_bwd_split_plan(B, H, k.shape[1], N, d, causal, nsplit)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device)
    if not workspace.is_cuda or workspace.device != q.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on q's device")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    with torch.cuda.device(q.device):
        _abi.attn_bwd_split(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                            grad_out.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                            dv.data_ptr(), B, H, k.shape[1], N, d, scale, causal, ns,
                            workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                            _stream_handle(q.device))
    return dq, dk, dv


def attention_varlen_backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                              out: torch.Tensor, lse: torch.Tensor, grad_out: torch.Tensor,
                              cu_seqlens: torch.Tensor, max_seqlen: int, causal: bool = False,
                              scale: float | None = None):
    """Gradients (dq, dk, dv) of sum(grad_out * out) for out, lse =
    attention_varlen(q, k, v, cu_seqlens, max_seqlen, causal, scale)."""
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out), ("grad_out", grad_out)):
        if not t.is_cuda or t.dtype != torch.bfloat16 or t.dim() != 3 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous bfloat16 [heads, total, d] GPU tensor")
    if out.shape != q.shape or grad_out.shape != q.shape or k.shape != v.shape or \
            k.shape[1:] != q.shape[1:] or q.shape[0] % k.shape[0]:
        raise ValueError("q, out, grad_out must be [H, total, d] and k, v [Hkv, total, d]")
    H, total, d = q.shape
    if lse.shape != (H, total) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [H, total] tensor")
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or cu_seqlens.device != q.device:
        raise ValueError("cu_seqlens must be an int32 [B + 1] tensor on q's device")
    B = cu_seqlens.numel() - 1
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    ws_bytes = _abi.attn_bwd_workspace_bytes(1, H, total)
    workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    with torch.cuda.device(q.device):
        _abi.attn_bwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                             grad_out.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                             dv.data_ptr(), cu_seqlens.data_ptr(), max(B, 0), H, k.shape[0],
                             total, int(max_seqlen), d, scale, causal, workspace.data_ptr(),
                             ws_bytes, _stream_handle(q.device))
    return dq, dk, dv


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
