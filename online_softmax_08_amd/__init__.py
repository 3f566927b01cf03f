"""MI355X (gfx950) fused online-softmax attention forward and stable row softmax.

The computation runs in hand-written HIP kernels inside ``libosm.so`` (built
by ``online_softmax_08_amd.build``); this package only marshals arguments.

* ``attn_fwd``, ``attn_fwd_f32``, ``attn_fwd_gqa``, ``attn_fwd_fp8``, ``attn_fwd_fp8_mx``,
  ``fp8_quantize_rows``, ``fp8_quantize_cols``, ``attn_fwd_varlen``,
  ``attn_fwd_splitkv_plan``,
  ``attn_fwd_splitkv``, ``attn_combine``, ``attn_bwd_workspace_bytes``,
  ``attn_bwd``, ``attn_bwd_noalloc``, ``attn_bwd_varlen``, ``attn_bwd_split_plan``,
  ``attn_bwd_split``, ``row_softmax``, ``osm_status_str`` are the C ABI of
  include/osm.h under the same names (device pointers as ints).
* ``attention``, ``attention_fp8``, ``quantize_fp8_rows``, ``quantize_fp8_cols``,
  ``attention_fp8_mx``, ``attention_fp8_block``, ``attention_varlen``, ``attention_splitkv``,
  ``attention_combine``,
  ``attention_backward``, ``attention_backward_split``, ``attention_varlen_backward``
  and ``softmax`` take
  torch tensors on the GPU,
  allocate the outputs with torch and launch on torch's current stream.
"""
from ._abi import (OsmError, attn_bwd, attn_bwd_noalloc, attn_bwd_split, attn_bwd_split_plan,
                   attn_bwd_varlen, attn_bwd_workspace_bytes, attn_combine,
                   attn_fwd,
                   attn_fwd_f32, attn_fwd_fp8, attn_fwd_fp8_mx, attn_fwd_gqa, attn_fwd_splitkv,
                   attn_fwd_splitkv_plan, fp8_quantize_cols, fp8_quantize_rows,
                   attn_fwd_varlen,
                   library_path, osm_status_str, row_softmax)
from .ops import (attention, attention_backward, attention_backward_split, attention_combine,
                  attention_fp8, attention_fp8_block, attention_fp8_mx,
                  attention_splitkv, quantize_fp8_cols, quantize_fp8_rows,
                  attention_varlen, attention_varlen_backward, softmax)

__all__ = ["OsmError", "attn_fwd", "attn_fwd_f32", "attn_fwd_gqa", "attn_fwd_fp8", "attn_fwd_fp8_mx",
           "fp8_quantize_rows", "fp8_quantize_cols", "attn_fwd_varlen",
           "attn_fwd_splitkv_plan",
           "attn_fwd_splitkv",
           "attn_combine", "attn_bwd_workspace_bytes", "attn_bwd", "attn_bwd_noalloc", "attn_bwd_varlen",
           "attn_bwd_split_plan", "attn_bwd_split", "row_softmax",
           "osm_status_str", "library_path", "attention", "attention_fp8", "attention_fp8_mx",
           "attention_fp8_block", "quantize_fp8_rows", "quantize_fp8_cols", "attention_varlen",
           "attention_splitkv",
           "attention_combine", "attention_backward", "attention_backward_split",
           "attention_varlen_backward", "softmax"]
