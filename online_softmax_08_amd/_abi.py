"""ctypes binding of libosm.so: the C ABI of include/osm.h under the same names.

Argument marshalling only: pointers are passed as Python ints (device
addresses), sizes as ints, the stream as its integer handle (0 = default
stream).  A nonzero status raises OsmError.  There is no fallback of any kind:
if the library is missing or fails to load, importing this module raises.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libosm.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build the HIP library first "
        "(python -c 'import __graft_entry__ as g; g.build()' or "
        "python online_softmax_08_amd/build.py)")

_lib = ctypes.CDLL(LIB_PATH)

_vp = ctypes.c_void_p
_i = ctypes.c_int
_f = ctypes.c_float

_lib.attn_fwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _vp]
_lib.attn_fwd.restype = _i
_lib.attn_fwd_f32.argtypes = [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _vp]
_lib.attn_fwd_f32.restype = _i
_lib.row_softmax.argtypes = [_vp, _vp, _i, _i, _vp]
_lib.row_softmax.restype = _i
_sz = ctypes.c_size_t
_lib.attn_fwd_varlen.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _i, _vp]
_lib.attn_fwd_varlen.restype = _i
_lib.attn_fwd_gqa.argtypes = [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _vp]
_lib.attn_fwd_gqa.restype = _i
_lib.attn_fwd_fp8.argtypes = [_vp, _vp, _vp, _f, _f, _f, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _vp]
_lib.attn_fwd_fp8.restype = _i
_lib.attn_fwd_fp8_mx.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f,
                                 _i, _vp]
_lib.attn_fwd_fp8_mx.restype = _i
_lib.fp8_quantize_rows.argtypes = [_vp, _vp, _vp, _vp, ctypes.c_longlong, _i, _vp]
_lib.fp8_quantize_rows.restype = _i
_lib.fp8_quantize_cols.argtypes = [_vp, _vp, _vp, ctypes.c_longlong, _i, _i, _vp]
_lib.fp8_quantize_cols.restype = _i
_lib.attn_fwd_splitkv_plan.argtypes = [_i, _i, _i, _i, _i, _i, ctypes.POINTER(_i),
                                       ctypes.POINTER(_sz)]
_lib.attn_fwd_splitkv_plan.restype = _i
_lib.attn_fwd_splitkv.argtypes = [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _i, _vp,
                                  _sz, _vp]
_lib.attn_fwd_splitkv.restype = _i
_lib.attn_combine.argtypes = [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _vp]
_lib.attn_combine.restype = _i
_lib.attn_bwd_workspace_bytes.argtypes = [_i, _i, _i]
_lib.attn_bwd_workspace_bytes.restype = _sz
_lib.attn_bwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f,
                          _i, _vp, _sz, _vp]
_lib.attn_bwd.restype = _i
_lib.attn_bwd_noalloc.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i,
                                  _f, _i, _vp]
_lib.attn_bwd_noalloc.restype = _i
_lib.attn_bwd_split_plan.argtypes = [_i, _i, _i, _i, _i, _i, _i, ctypes.POINTER(_i),
                                     ctypes.POINTER(_sz)]
_lib.attn_bwd_split_plan.restype = _i
_lib.attn_bwd_split.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i,
                                _f, _i, _i, _vp, _sz, _vp]
_lib.attn_bwd_split.restype = _i
_lib.attn_bwd_varlen.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i,
                                 _i, _i, _i, _f, _i, _vp, _sz, _vp]
_lib.attn_bwd_varlen.restype = _i
_lib.osm_status_str.argtypes = [_i]
_lib.osm_status_str.restype = ctypes.c_char_p

EXPORTS = ("attn_fwd", "attn_fwd_f32", "attn_fwd_gqa", "attn_fwd_fp8", "attn_fwd_fp8_mx",
           "fp8_quantize_rows", "fp8_quantize_cols", "attn_fwd_varlen", "attn_fwd_splitkv_plan",
           "attn_fwd_splitkv",
           "attn_combine", "attn_bwd_workspace_bytes", "attn_bwd", "attn_bwd_noalloc", "attn_bwd_varlen",
           "attn_bwd_split_plan", "attn_bwd_split", "row_softmax", "osm_status_str")

OSM_OK = 0
OSM_ERR_NULL = 1
OSM_ERR_SIZE = 2
OSM_ERR_HEAD_DIM = 3
OSM_ERR_SCALE = 4
OSM_ERR_ALIAS = 5
OSM_ERR_HIP = 6
OSM_ERR_ALIGN = 7
OSM_ERR_DEVICE = 8
OSM_ERR_SPLITS = 9
OSM_ERR_WORKSPACE = 10
OSM_ERR_HEADS = 11
OSM_ERR_SCRATCH = 12
OSM_ERR_SIGNS = 13
# attn_bwd_noalloc's limit on B * H * N (include/osm.h OSM_NOALLOC_BWD_MAX_ROWS)
NOALLOC_BWD_MAX_ROWS = 1 << 22


class OsmError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {osm_status_str(status)} (status {status})")


def library_path() -> str:
    return LIB_PATH


def osm_status_str(status: int) -> str:
    return _lib.osm_status_str(int(status)).decode()


def _call(fn: str, *args) -> None:
    st = getattr(_lib, fn)(*args)
    if st != OSM_OK:
        raise OsmError(fn, st)


def attn_fwd(Q: int, K: int, V: int, O: int, lse: int, B: int, H: int, N: int, d: int,
             scale: float, causal: bool, stream: int = 0) -> None:
    """bf16 attention forward; see include/osm.h."""
    _call("attn_fwd", Q, K, V, O, lse, B, H, N, d, scale, int(bool(causal)), stream)


def attn_fwd_f32(Q: int, K: int, V: int, O: int, lse: int, B: int, H: int, N: int, d: int,
                 scale: float, causal: bool, stream: int = 0) -> None:
    """fp32 attention forward; see include/osm.h."""
    _call("attn_fwd_f32", Q, K, V, O, lse, B, H, N, d, scale, int(bool(causal)), stream)


def row_softmax(x: int, y: int, B: int, N: int, stream: int = 0) -> None:
    """Stable row softmax of fp32 [B, N]; see include/osm.h."""
    _call("row_softmax", x, y, B, N, stream)


def attn_fwd_splitkv_plan(B: int, H: int, N: int, d: int, causal: bool,
                          nsplit: int = 0) -> tuple[int, int]:
    """(resolved split count, workspace bytes) for attn_fwd_splitkv; see include/osm.h."""
    n_out = _i(0)
    ws = _sz(0)
    _call("attn_fwd_splitkv_plan", B, H, N, d, int(bool(causal)), nsplit, ctypes.byref(n_out),
          ctypes.byref(ws))
    return n_out.value, ws.value


def attn_fwd_splitkv(Q: int, K: int, V: int, O: int, lse: int, B: int, H: int, Hkv: int,
                     N: int, d: int, scale: float, causal: bool, nsplit: int, workspace: int,
                     workspace_bytes: int, stream: int = 0) -> None:
    """bf16 attention forward over nsplit parallel key ranges; see include/osm.h."""
    _call("attn_fwd_splitkv", Q, K, V, O, lse, B, H, Hkv, N, d, scale, int(bool(causal)), nsplit,
          workspace, workspace_bytes, stream)


def attn_combine(O_part: int, lse_part: int, O: int, lse: int, S: int, B: int, H: int, N: int,
                 d: int, stream: int = 0) -> None:
    """Merge of S partial attention results; see include/osm.h."""
    _call("attn_combine", O_part, lse_part, O, lse, S, B, H, N, d, stream)


def attn_bwd_workspace_bytes(B: int, H: int, N: int) -> int:
    """Device bytes attn_bwd needs as workspace; see include/osm.h."""
    return int(_lib.attn_bwd_workspace_bytes(B, H, N))


def attn_bwd(Q: int, K: int, V: int, O: int, dO: int, lse: int, dQ: int, dK: int, dV: int,
             B: int, H: int, Hkv: int, N: int, d: int, scale: float, causal: bool, workspace: int,
             workspace_bytes: int, stream: int = 0) -> None:
    """Backward pass of attn_fwd / attn_fwd_gqa (dQ, dK, dV); see include/osm.h."""
    _call("attn_bwd", Q, K, V, O, dO, lse, dQ, dK, dV, B, H, Hkv, N, d, scale, int(bool(causal)),
          workspace, workspace_bytes, stream)


def attn_bwd_noalloc(Q: int, K: int, V: int, O: int, dO: int, lse: int, dQ: int, dK: int,
                     dV: int, B: int, H: int, Hkv: int, N: int, d: int, scale: float, causal: bool,
                     stream: int = 0) -> None:
    """attn_bwd with the row statistics in the library's static device scratch
    (no workspace, no allocation); see include/osm.h."""
    _call("attn_bwd_noalloc", Q, K, V, O, dO, lse, dQ, dK, dV, B, H, Hkv, N, d, scale,
          int(bool(causal)), stream)


def attn_bwd_split_plan(B: int, H: int, Hkv: int, N: int, d: int, causal: bool,
                        nsplit: int = 0) -> tuple[int, int]:
    """(resolved split count, workspace bytes) for attn_bwd_split; see include/osm.h."""
    n_out, ws = _i(0), _sz(0)
    _call("attn_bwd_split_plan", B, H, Hkv, N, d, int(bool(causal)), nsplit, ctypes.byref(n_out),
          ctypes.byref(ws))
    return n_out.value, ws.value


def attn_bwd_split(Q: int, K: int, V: int, O: int, dO: int, lse: int, dQ: int, dK: int, dV: int,
                   B: int, H: int, Hkv: int, N: int, d: int, scale: float, causal: bool,
                   nsplit: int, workspace: int, workspace_bytes: int, stream: int = 0) -> None:
    """attn_bwd with the query (dK, dV) and key (dQ) loops split into nsplit
    ranges and the fp32 partials summed; see include/osm.h."""
    _call("attn_bwd_split", Q, K, V, O, dO, lse, dQ, dK, dV, B, H, Hkv, N, d, scale,
          int(bool(causal)), nsplit, workspace, workspace_bytes, stream)


def attn_fwd_fp8(Q: int, K: int, V: int, q_scale: float, k_scale: float, v_scale: float, O: int,
                 lse: int, B: int, H: int, Hkv: int, N: int, d: int, scale: float, causal: bool,
                 stream: int = 0) -> None:
    """Attention forward on OCP FP8 E4M3 inputs with per-tensor scales; see include/osm.h."""
    _call("attn_fwd_fp8", Q, K, V, q_scale, k_scale, v_scale, O, lse, B, H, Hkv, N, d, scale,
          int(bool(causal)), stream)


def attn_fwd_fp8_mx(Q: int, q_scales: int, K: int, k_scales: int, V: int, v_scales: int, O: int,
                    lse: int, B: int, H: int, Hkv: int, N: int, d: int, scale: float,
                    causal: bool, stream: int = 0) -> None:
    """Attention forward on block-quantized FP8 inputs; see include/osm.h."""
    _call("attn_fwd_fp8_mx", Q, q_scales, K, k_scales, V, v_scales, O, lse, B, H, Hkv, N, d,
          scale, int(bool(causal)), stream)


def fp8_quantize_rows(X: int, signs, codes: int, scales: int, rows: int, d: int,
                      stream: int = 0) -> None:
    """Block quantization along rows, after the random-sign Hadamard rotation
    when signs (a host sequence of d values +-1) is given; see include/osm.h."""
    sp = None
    if signs is not None:
        vals = [int(x) for x in signs]
        sp = ctypes.cast((ctypes.c_byte * len(vals))(*vals), _vp)
    _call("fp8_quantize_rows", X, sp, codes, scales, rows, d, stream)


def fp8_quantize_cols(X: int, codes: int, scales: int, slices: int, n: int, d: int,
                      stream: int = 0) -> None:
    """Block quantization along the rows of each column; see include/osm.h."""
    _call("fp8_quantize_cols", X, codes, scales, slices, n, d, stream)


def attn_fwd_varlen(Q: int, K: int, V: int, O: int, lse: int, cu_seqlens: int, B: int, H: int,
                    Hkv: int, total: int, max_seqlen: int, d: int, scale: float, causal: bool,
                    stream: int = 0) -> None:
    """bf16 attention over packed variable-length sequences; see include/osm.h."""
    _call("attn_fwd_varlen", Q, K, V, O, lse, cu_seqlens, B, H, Hkv, total, max_seqlen, d, scale,
          int(bool(causal)), stream)


def attn_fwd_gqa(Q: int, K: int, V: int, O: int, lse: int, B: int, H: int, Hkv: int, N: int,
                 d: int, scale: float, causal: bool, stream: int = 0) -> None:
    """bf16 attention with Hkv key/value heads; see include/osm.h."""
    _call("attn_fwd_gqa", Q, K, V, O, lse, B, H, Hkv, N, d, scale, int(bool(causal)), stream)


def attn_bwd_varlen(Q: int, K: int, V: int, O: int, dO: int, lse: int, dQ: int, dK: int, dV: int,
                    cu_seqlens: int, B: int, H: int, Hkv: int, total: int, max_seqlen: int, d: int,
                    scale: float, causal: bool, workspace: int, workspace_bytes: int,
                    stream: int = 0) -> None:
    """Backward pass of attn_fwd_varlen; see include/osm.h."""
    _call("attn_bwd_varlen", Q, K, V, O, dO, lse, dQ, dK, dV, cu_seqlens, B, H, Hkv, total,
          max_seqlen, d, scale, int(bool(causal)), workspace, workspace_bytes, stream)
