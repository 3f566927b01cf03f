"""fp64 CPU oracle for exact attention forward and backward, the merge of
partial attention results, and the stable row softmax.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product path never does.  It
shares no code with the HIP library (``online_softmax_08_amd``) and imports
nothing from it.

The arithmetic lives in ``oracle.c`` (plain C, binary64), built by
``oracle.build.build()`` into ``liboracle.so`` next to it.  This module only
marshals numpy arrays to that library.  Each wrapper cites the passage its C
routine follows; the header of ``oracle.c`` names the pages.

Pinned by ``tests/test_oracle.py`` against the pages' worked examples, closed
forms, invariants, brute force and independent library routines; the pins'
power to catch plausible mistakes is itself checked by planting mistakes in
copies of ``oracle.c`` (``tests/test_oracle_mutants.py``).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")

_dp = ctypes.POINTER(ctypes.c_double)
_lp = ctypes.POINTER(ctypes.c_long)
_L = ctypes.c_long


def _f64(a) -> np.ndarray:
    """Exact upcast to a contiguous float64 array (bf16/fp32 -> fp64 is exact)."""
    try:
        import torch
        if isinstance(a, torch.Tensor):
            a = a.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover - torch is always present here
        pass
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(_dp)


def _u8(a) -> np.ndarray:
    """Contiguous uint8 view of codes or scale bytes (numpy or torch storage)."""
    try:
        import torch
        if isinstance(a, torch.Tensor):
            a = a.detach().to("cpu").contiguous().view(torch.uint8).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(a, dtype=np.uint8))


def _bptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_ubyte))


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise RuntimeError(f"oracle {what} failed with code {rc}")


class Oracle:
    """Marshalling front end of one build of ``oracle.c`` (by default the
    committed source; the mutant tests load deliberately broken copies)."""

    def __init__(self, lib_path: str = LIB_PATH):
        lib = ctypes.CDLL(lib_path)
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_row_softmax.argtypes = [_dp, _dp, _L, _L]
        lib.oracle_attn_fwd.argtypes = [_dp, _dp, _dp, _dp, _dp, _L, _L, _L, _L,
                                        ctypes.c_double, ctypes.c_int]
        lib.oracle_attn_rows.argtypes = [_dp, _dp, _dp, _L, _L, _L, _L,
                                         ctypes.c_double, ctypes.c_int,
                                         _lp, _lp, _L, _dp, _dp]
        lib.oracle_online_row_trace.argtypes = [_dp, _L, _L, _dp, _dp]
        lib.oracle_attn_online.argtypes = [_dp, _dp, _dp, _dp, _dp, _L, _L, _L, _L,
                                           ctypes.c_double, ctypes.c_int, _L, _L]
        lib.oracle_attn_merge.argtypes = [_dp, _dp, _dp, _dp, _L, _L, _L]
        lib.oracle_attn_bwd.argtypes = [_dp, _dp, _dp, _dp, _dp, _dp, _dp, _L, _L, _L, _L,
                                        ctypes.c_double, ctypes.c_int]
        lib.oracle_fp8_e4m3_decode.argtypes = [ctypes.POINTER(ctypes.c_ubyte), ctypes.c_double,
                                               _dp, _L]
        _bp = ctypes.POINTER(ctypes.c_ubyte)
        lib.oracle_fp8_e4m3_encode.argtypes = [_dp, ctypes.c_double, _bp, _L]
        lib.oracle_hadamard_rotate.argtypes = [_dp, _dp, _dp, _L, _L]
        lib.oracle_mx_quantize_rows.argtypes = [_dp, _bp, _bp, _L, _L]
        lib.oracle_mx_quantize_cols.argtypes = [_dp, _bp, _bp, _L, _L, _L]
        lib.oracle_mx_decode_rows.argtypes = [_bp, _bp, _dp, _L, _L]
        lib.oracle_mx_decode_cols.argtypes = [_bp, _bp, _dp, _L, _L, _L]
        for name in ("oracle_row_softmax", "oracle_attn_fwd", "oracle_attn_rows",
                     "oracle_online_row_trace", "oracle_attn_online", "oracle_attn_merge",
                     "oracle_attn_bwd", "oracle_fp8_e4m3_decode", "oracle_fp8_e4m3_encode",
                     "oracle_hadamard_rotate", "oracle_mx_quantize_rows",
                     "oracle_mx_quantize_cols", "oracle_mx_decode_rows",
                     "oracle_mx_decode_cols"):
            getattr(lib, name).restype = ctypes.c_int
        self._lib = lib

    def num_threads(self) -> int:
        """OpenMP threads the oracle's parallel loops use."""
        return int(self._lib.oracle_num_threads())

    def row_softmax(self, x) -> np.ndarray:
        """Three-pass stable softmax of every row of x [B, N]
        (Lesson 22, sections 2 and 3)."""
        x = _f64(x)
        if x.ndim != 2:
            raise ValueError("x must be [B, N]")
        y = np.empty_like(x)
        _check(self._lib.oracle_row_softmax(_ptr(x), _ptr(y), x.shape[0], x.shape[1]),
               "row_softmax")
        return y

    @staticmethod
    def _attn_shapes(Q, K, V):
        Q, K, V = _f64(Q), _f64(K), _f64(V)
        if Q.ndim != 4 or K.shape != Q.shape or V.shape != Q.shape:
            raise ValueError("Q, K, V must share one [B, H, N, d] shape")
        return Q, K, V

    def attn_fwd(self, Q, K, V, scale: float, causal: bool):
        """Exact attention, three passes per row with the score and probability
        rows materialised (Lesson 22, sections 12-14 and 34; four generations,
        2.4 for lse = m + ln l).  Returns (O [B,H,N,d], lse [B,H,N])."""
        Q, K, V = self._attn_shapes(Q, K, V)
        B, H, N, d = Q.shape
        O = np.empty_like(Q)
        lse = np.empty((B, H, N), dtype=np.float64)
        _check(self._lib.oracle_attn_fwd(_ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(lse),
                                         B, H, N, d, float(scale), int(bool(causal))),
               "attn_fwd")
        return O, lse

    def attn_rows(self, Q, K, V, scale: float, causal: bool, bh, qi):
        """The definition of ``attn_fwd`` evaluated for selected rows only:
        row r is query qi[r] of slice bh[r] (bh = b*H + h).  Returns
        (O_rows [nrows, d], lse_rows [nrows])."""
        Q, K, V = self._attn_shapes(Q, K, V)
        B, H, N, d = Q.shape
        bh = np.ascontiguousarray(np.asarray(bh, dtype=np.int64))
        qi = np.ascontiguousarray(np.asarray(qi, dtype=np.int64))
        if bh.shape != qi.shape or bh.ndim != 1:
            raise ValueError("bh and qi must be 1-D and of equal length")
        n = bh.shape[0]
        O = np.empty((n, d), dtype=np.float64)
        lse = np.empty((n,), dtype=np.float64)
        _check(self._lib.oracle_attn_rows(_ptr(Q), _ptr(K), _ptr(V), B, H, N, d,
                                          float(scale), int(bool(causal)),
                                          bh.ctypes.data_as(_lp), qi.ctypes.data_as(_lp),
                                          n, _ptr(O), _ptr(lse)),
               "attn_rows")
        return O, lse

    def online_row_trace(self, x, bc: int):
        """Online softmax state (m, l) after each block of bc scores of one row
        (Lesson 22, sections 18-20 and 33)."""
        x = _f64(x).ravel()
        nb = (x.shape[0] + bc - 1) // bc if bc >= 1 else 0
        m = np.empty((nb,), dtype=np.float64)
        l = np.empty((nb,), dtype=np.float64)
        _check(self._lib.oracle_online_row_trace(_ptr(x), x.shape[0], int(bc),
                                                 _ptr(m), _ptr(l)), "online_row_trace")
        return m, l

    def attn_online(self, Q, K, V, scale: float, causal: bool, br: int, bc: int):
        """Tiled online attention with query blocks of br rows and key blocks of
        bc (Lesson 22, sections 21-24 and 32).  Self-check of the recurrence."""
        Q, K, V = self._attn_shapes(Q, K, V)
        B, H, N, d = Q.shape
        O = np.empty_like(Q)
        lse = np.empty((B, H, N), dtype=np.float64)
        _check(self._lib.oracle_attn_online(_ptr(Q), _ptr(K), _ptr(V), _ptr(O),
                                            _ptr(lse), B, H, N, d, float(scale),
                                            int(bool(causal)), int(br), int(bc)),
               "attn_online")
        return O, lse

    def attn_merge(self, O_part, lse_part):
        """Merge of partial results over disjoint key sets, joined one by one
        with the rule of Lesson 22, section 22 (each normalised partial taken
        as the state m = lse_s, l = 1, a = O_s).  O_part [S, ..., d],
        lse_part [S, ...]; returns (O [..., d], lse [...])."""
        O_part, lse_part = _f64(O_part), _f64(lse_part)
        if O_part.ndim < 2 or lse_part.shape != O_part.shape[:-1]:
            raise ValueError("O_part must be [S, ..., d] and lse_part [S, ...]")
        S, d = O_part.shape[0], O_part.shape[-1]
        lead = O_part.shape[1:-1]
        rows = int(np.prod(lead)) if lead else 1
        O = np.empty(lead + (d,), dtype=np.float64)
        lse = np.empty(lead, dtype=np.float64)
        _check(self._lib.oracle_attn_merge(_ptr(O_part), _ptr(lse_part), _ptr(O), _ptr(lse),
                                           S, rows, d), "attn_merge")
        return O, lse

    def fp8_decode(self, codes, s: float = 1.0) -> np.ndarray:
        """float64 values of FP8 E4M3 codes (uint8 or torch float8_e4m3fn
        storage, any shape) times s (the FP8 variant of "Moving less",
        section 4.6; encoding in ``oracle.c``)."""
        try:
            import torch
            if isinstance(codes, torch.Tensor):
                codes = codes.detach().to("cpu").contiguous().view(torch.uint8).numpy()
        except ImportError:  # pragma: no cover
            pass
        x = np.ascontiguousarray(np.asarray(codes, dtype=np.uint8))
        y = np.empty(x.shape, dtype=np.float64)
        _check(self._lib.oracle_fp8_e4m3_decode(x.ctypes.data_as(ctypes.POINTER(ctypes.c_ubyte)),
                                                float(s), _ptr(y), _L(x.size)), "fp8_decode")
        return y

    def attn_fwd_fp8(self, Q8, K8, V8, q_scale: float, k_scale: float, v_scale: float,
                     scale: float, causal: bool):
        """attn_fwd on the decoded, scaled FP8 inputs (Q8, K8, V8: E4M3 codes of
        one shape [B, H, N, d]).  Returns (O, lse)."""
        return self.attn_fwd(self.fp8_decode(Q8, q_scale), self.fp8_decode(K8, k_scale),
                             self.fp8_decode(V8, v_scale), scale, causal)

    def fp8_encode(self, x, s: float = 1.0) -> np.ndarray:
        """E4M3 codes (uint8, shape of x) of x / s, rounded to the nearest
        code with ties to the even code (encoding in ``oracle.c``)."""
        x = _f64(x)
        out = np.empty(x.shape, dtype=np.uint8)
        _check(self._lib.oracle_fp8_e4m3_encode(_ptr(x), float(s), _bptr(out), _L(x.size)),
               "fp8_encode")
        return out

    def hadamard_rotate(self, X, signs) -> np.ndarray:
        """X [..., d] times diag(signs) H / sqrt(d), H the Sylvester Hadamard
        matrix (incoherent processing, "Moving less", section 4.6)."""
        X = _f64(X)
        signs = _f64(signs)
        d = X.shape[-1]
        if signs.shape != (d,):
            raise ValueError("signs must hold d values")
        Y = np.empty_like(X)
        _check(self._lib.oracle_hadamard_rotate(_ptr(X), _ptr(signs), _ptr(Y),
                                                _L(X.size // max(d, 1)), _L(d)), "hadamard_rotate")
        return Y

    def mx_quantize_rows(self, Y):
        """Block quantization along the last axis ("Moving less", section 4.6):
        blocks of 32 elements of a row, one power-of-two scale each.  Returns
        (codes uint8 [..., d], scale bytes uint8 [..., d / 32])."""
        Y = _f64(Y)
        d = Y.shape[-1]
        codes = np.empty(Y.shape, dtype=np.uint8)
        scales = np.empty(Y.shape[:-1] + (d // 32,), dtype=np.uint8)
        _check(self._lib.oracle_mx_quantize_rows(_ptr(Y), _bptr(codes), _bptr(scales),
                                                 _L(Y.size // max(d, 1)), _L(d)), "mx_quantize_rows")
        return codes, scales

    def mx_quantize_cols(self, Y):
        """Block quantization along the rows of each column of every [n, d]
        slice of Y [..., n, d]: blocks of 32 rows (the last one ragged).
        Returns (codes uint8 [..., n, d], scale bytes uint8 [..., ceil(n/32), d])."""
        Y = _f64(Y)
        n, d = Y.shape[-2], Y.shape[-1]
        slices = int(np.prod(Y.shape[:-2])) if Y.ndim > 2 else 1
        codes = np.empty(Y.shape, dtype=np.uint8)
        scales = np.empty(Y.shape[:-2] + ((n + 31) // 32, d), dtype=np.uint8)
        _check(self._lib.oracle_mx_quantize_cols(_ptr(Y), _bptr(codes), _bptr(scales),
                                                 _L(slices), _L(n), _L(d)), "mx_quantize_cols")
        return codes, scales

    def mx_decode_rows(self, codes, scales) -> np.ndarray:
        codes, scales = _u8(codes), _u8(scales)
        d = codes.shape[-1]
        if scales.shape != codes.shape[:-1] + (d // 32,):
            raise ValueError("scales must be [..., d / 32]")
        Y = np.empty(codes.shape, dtype=np.float64)
        _check(self._lib.oracle_mx_decode_rows(_bptr(codes), _bptr(scales), _ptr(Y),
                                               _L(codes.size // max(d, 1)), _L(d)), "mx_decode_rows")
        return Y

    def mx_decode_cols(self, codes, scales) -> np.ndarray:
        codes, scales = _u8(codes), _u8(scales)
        n, d = codes.shape[-2], codes.shape[-1]
        if scales.shape != codes.shape[:-2] + ((n + 31) // 32, d):
            raise ValueError("scales must be [..., ceil(n / 32), d]")
        slices = int(np.prod(codes.shape[:-2])) if codes.ndim > 2 else 1
        Y = np.empty(codes.shape, dtype=np.float64)
        _check(self._lib.oracle_mx_decode_cols(_bptr(codes), _bptr(scales), _ptr(Y),
                                               _L(slices), _L(n), _L(d)), "mx_decode_cols")
        return Y

    def attn_fwd_fp8_mx(self, Q8, q_sc, K8, k_sc, V8, v_sc, scale: float, causal: bool):
        """attn_fwd on block-quantized FP8 inputs: Q and K with one scale per
        32 head columns of a row, V with one per 32 keys of a column
        ([B, H, N, d] codes; scales [B, H, N, d/32] and [B, H, ceil(N/32), d])."""
        return self.attn_fwd(self.mx_decode_rows(Q8, q_sc), self.mx_decode_rows(K8, k_sc),
                             self.mx_decode_cols(V8, v_sc), scale, causal)

    def attn_bwd(self, Q, K, V, dO, scale: float, causal: bool):
        """Gradients of sum(dO * O) with respect to Q, K, V for the attention
        forward, by the chain rule with the probabilities recomputed from Q
        and K (Lesson 22, sections 30-31; four generations, 2.4).  Returns
        (dQ, dK, dV), each [B, H, N, d]."""
        Q, K, V = self._attn_shapes(Q, K, V)
        dO = _f64(dO)
        if dO.shape != Q.shape:
            raise ValueError("dO must have the shape of Q")
        B, H, N, d = Q.shape
        dQ, dK, dV = np.empty_like(Q), np.empty_like(Q), np.empty_like(Q)
        _check(self._lib.oracle_attn_bwd(_ptr(Q), _ptr(K), _ptr(V), _ptr(dO), _ptr(dQ),
                                         _ptr(dK), _ptr(dV), B, H, N, d, float(scale),
                                         int(bool(causal))), "attn_bwd")
        return dQ, dK, dV


_default: Oracle | None = None


def default() -> Oracle:
    """The oracle built from the committed ``oracle.c`` (built on first use)."""
    global _default
    if _default is None:
        if not os.path.exists(LIB_PATH):
            from . import build as _build
            _build.build()
        _default = Oracle(LIB_PATH)
    return _default


def num_threads() -> int:
    return default().num_threads()


def row_softmax(x):
    return default().row_softmax(x)


def attn_fwd(Q, K, V, scale, causal):
    return default().attn_fwd(Q, K, V, scale, causal)


def attn_rows(Q, K, V, scale, causal, bh, qi):
    return default().attn_rows(Q, K, V, scale, causal, bh, qi)


def online_row_trace(x, bc):
    return default().online_row_trace(x, bc)


def attn_online(Q, K, V, scale, causal, br, bc):
    return default().attn_online(Q, K, V, scale, causal, br, bc)


def attn_merge(O_part, lse_part):
    return default().attn_merge(O_part, lse_part)


def fp8_decode(codes, s=1.0):
    return default().fp8_decode(codes, s)


def attn_fwd_fp8(Q8, K8, V8, q_scale, k_scale, v_scale, scale, causal):
    return default().attn_fwd_fp8(Q8, K8, V8, q_scale, k_scale, v_scale, scale, causal)


def attn_bwd(Q, K, V, dO, scale, causal):
    return default().attn_bwd(Q, K, V, dO, scale, causal)


def fp8_encode(x, s=1.0):
    return default().fp8_encode(x, s)


def hadamard_rotate(X, signs):
    return default().hadamard_rotate(X, signs)


def mx_quantize_rows(Y):
    return default().mx_quantize_rows(Y)


def mx_quantize_cols(Y):
    return default().mx_quantize_cols(Y)


def mx_decode_rows(codes, scales):
    return default().mx_decode_rows(codes, scales)


def mx_decode_cols(codes, scales):
    return default().mx_decode_cols(codes, scales)


def attn_fwd_fp8_mx(Q8, q_sc, K8, k_sc, V8, v_sc, scale, causal):
    return default().attn_fwd_fp8_mx(Q8, q_sc, K8, k_sc, V8, v_sc, scale, causal)
