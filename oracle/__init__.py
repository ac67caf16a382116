"""Plain fp64 CPU oracle for C = A @ B, its fused epilogue and attention -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package. It shares no code with the HIP library and never imports
it. The arithmetic lives in `ref_gemm.c` (plain C, fp64, k-ascending sums);
`brute.py` is an exact rational cross-check for tiny shapes.

Dtype codes here are the oracle's own: "f32", "f16", "bf16".
Activation names: "none", "relu", "gelu".

Parity status: every function is pinned (tests/test_oracle.py) against the
pages' worked examples, closed forms, invariants and an exact brute force.
"""
import ctypes
import os

import numpy as np

from .build import LIB, build

_CODES = {"f32": 0, "f16": 1, "bf16": 2}
_BITS = {"f32": np.uint32, "f16": np.uint16, "bf16": np.uint16}
_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        lib = ctypes.CDLL(LIB)
        i64, p = ctypes.c_int64, ctypes.c_void_p
        lib.ref_threads.restype = ctypes.c_int
        lib.ref_decode.argtypes = [ctypes.c_int, p, i64, p]
        lib.ref_encode.argtypes = [ctypes.c_int, p, i64, p]
        lib.ref_gemm.argtypes = [i64, i64, i64, ctypes.c_int, p, i64, i64, p, i64, i64, p, i64]
        lib.ref_gemm.restype = ctypes.c_int
        lib.ref_gemm_entries.argtypes = [i64, ctypes.c_int, p, i64, i64, p, i64, i64, i64, p, p, p]
        lib.ref_gemm_rows.argtypes = [i64, i64, i64, i64, ctypes.c_int, p, i64, i64, p, i64, i64, p]
        d, c = ctypes.c_double, ctypes.c_int
        lib.ref_epilogue.argtypes = [i64, i64, p, i64, d, d, c, p, i64, i64, c, p, i64, c, c, p, i64]
        lib.ref_attention.argtypes = [i64, i64, i64, i64, i64, c, p, i64, i64, i64, p, i64, i64, i64,
                                      p, i64, i64, i64, d, c, p, p]
        lib.ref_attention.restype = c
        _lib = lib
    return _lib


def threads() -> int:
    """OpenMP threads the oracle uses."""
    return _load().ref_threads()


def _bits(x: np.ndarray, dtype: str) -> np.ndarray:
    want = _BITS[dtype]
    if x.dtype != want:
        raise TypeError(f"oracle expects raw {dtype} bits as {np.dtype(want).name}, got {x.dtype}")
    return x


def _operand(x: np.ndarray, dtype: str):
    """Base pointer and element strides of a (possibly strided) bit array view."""
    x = _bits(x, dtype)
    item = x.itemsize
    if any(s % item for s in x.strides) or any(s < 0 for s in x.strides):
        raise ValueError("oracle operands need non-negative, element-aligned strides")
    return x.ctypes.data, tuple(s // item for s in x.strides)


def decode(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact fp64 value of each element of a bit-pattern array."""
    b = np.ascontiguousarray(_bits(bits, dtype))
    out = np.empty(b.shape, dtype=np.float64)
    _load().ref_decode(_CODES[dtype], b.ctypes.data, b.size, out.ctypes.data)
    return out


def encode(values: np.ndarray, dtype: str) -> np.ndarray:
    """Round fp64 values to `dtype`, nearest with ties to even; returns bits."""
    v = np.ascontiguousarray(values, dtype=np.float64)
    out = np.empty(v.shape, dtype=_BITS[dtype])
    _load().ref_encode(_CODES[dtype], v.ctypes.data, v.size, out.ctypes.data)
    return out


def gemm(a_bits: np.ndarray, b_bits: np.ndarray, dtype: str) -> np.ndarray:
    """C = A @ B in fp64 (k-ascending sums over exactly decoded inputs).

    a_bits: [M, K] view of raw bits; b_bits: [K, N] view; any non-negative
    strides (a transposed view is read through its strides).
    """
    (M, K), (K2, N) = a_bits.shape, b_bits.shape
    if K != K2:
        raise ValueError(f"inner dimensions differ: {K} vs {K2}")
    pa, (sam, sak) = _operand(a_bits, dtype)
    pb, (sbk, sbn) = _operand(b_bits, dtype)
    c = np.zeros((M, N), dtype=np.float64)
    rc = _load().ref_gemm(M, N, K, _CODES[dtype], pa, sam, sak, pb, sbk, sbn, c.ctypes.data, N)
    if rc != 0:
        raise MemoryError("oracle could not allocate its fp64 operand copies")
    return c


def gemm_entries(a_bits: np.ndarray, b_bits: np.ndarray, dtype: str,
                 rows: np.ndarray, cols: np.ndarray) -> np.ndarray:
    """C[rows[t], cols[t]] for each t, each straight from the definition."""
    (M, K), (K2, N) = a_bits.shape, b_bits.shape
    if K != K2:
        raise ValueError(f"inner dimensions differ: {K} vs {K2}")
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    if rows.shape != cols.shape:
        raise ValueError("rows and cols must have the same shape")
    if rows.size and (rows.min() < 0 or rows.max() >= M or cols.min() < 0 or cols.max() >= N):
        raise IndexError("sampled index outside C")
    pa, (sam, sak) = _operand(a_bits, dtype)
    pb, (sbk, sbn) = _operand(b_bits, dtype)
    out = np.empty(rows.shape, dtype=np.float64)
    _load().ref_gemm_entries(K, _CODES[dtype], pa, sam, sak, pb, sbk, sbn,
                             rows.size, rows.ctypes.data, cols.ctypes.data, out.ctypes.data)
    return out


def gemm_rows(a_bits: np.ndarray, b_bits: np.ndarray, dtype: str,
              row0: int, nrows: int) -> np.ndarray:
    """Rows [row0, row0+nrows) of C, each entry straight from the definition."""
    (M, K), (K2, N) = a_bits.shape, b_bits.shape
    if K != K2:
        raise ValueError(f"inner dimensions differ: {K} vs {K2}")
    if row0 < 0 or nrows < 0 or row0 + nrows > M:
        raise IndexError("row range outside C")
    pa, (sam, sak) = _operand(a_bits, dtype)
    pb, (sbk, sbn) = _operand(b_bits, dtype)
    out = np.empty((nrows, N), dtype=np.float64)
    _load().ref_gemm_rows(row0, nrows, N, K, _CODES[dtype], pa, sam, sak, pb, sbk, sbn,
                          out.ctypes.data)
    return out


_ACTS = {"none": 0, "relu": 1, "gelu": 2}


def epilogue(p: np.ndarray, alpha=1.0, beta=0.0, r_bits=None, r_dtype=None,
             bias_bits=None, bias_dtype=None, per_row=False, act="none") -> np.ndarray:
    """act(alpha * P + beta * R + bias) in fp64 (ref_epilogue in ref_gemm.c).

    p: [M, N] fp64 product. alpha and beta are rounded to fp32 first (the
    values a caller of the GPU library can pass). r_bits: [M, N] view of raw
    bits (read only when beta != 0); bias_bits: 1-D view of raw bits, one per
    column (per_row False) or per row.
    """
    p = np.ascontiguousarray(p, dtype=np.float64)
    M, N = p.shape
    alpha, beta = float(np.float32(alpha)), float(np.float32(beta))
    rp, (srm, srn), rcode = None, (0, 0), 0
    if beta != 0.0:
        if r_bits is None or tuple(r_bits.shape) != (M, N):
            raise ValueError("beta != 0 needs an [M, N] residual")
        rp, (srm, srn) = _operand(r_bits, r_dtype)
        rcode = _CODES[r_dtype]
    bp, sb, bcode = None, 0, 0
    if bias_bits is not None:
        if bias_bits.ndim != 1 or bias_bits.shape[0] != (M if per_row else N):
            raise ValueError("bias length must be M (per_row) or N")
        bp, (sb,) = _operand(bias_bits, bias_dtype)
        bcode = _CODES[bias_dtype]
    out = np.empty((M, N), dtype=np.float64)
    _load().ref_epilogue(M, N, p.ctypes.data, N, alpha, beta, rcode, rp, srm, srn,
                         bcode, bp, sb, 1 if per_row else 0, _ACTS[act], out.ctypes.data, N)
    return out


def gemm_ex(a_bits: np.ndarray, b_bits: np.ndarray, dtype: str, **epi) -> np.ndarray:
    """The product followed by the fused epilogue (arguments of `epilogue`)."""
    return epilogue(gemm(a_bits, b_bits, dtype), **epi)


def attention(q_bits: np.ndarray, k_bits: np.ndarray, v_bits: np.ndarray, dtype: str,
              scale=None, causal=False):
    """softmax(scale * Q K^T [causal mask]) V in fp64 (ref_attention in ref_gemm.c).

    q_bits [batch, heads, seq_q, dim], k_bits / v_bits [batch, heads, seq_kv, dim]:
    views of raw bits with any non-negative strides and a unit stride along
    dim. scale defaults to 1/sqrt(dim) (taken as given otherwise, in fp64).
    Returns (O [batch, heads, seq_q, dim] fp64, lse [batch, heads, seq_q] fp64).
    """
    if q_bits.ndim != 4 or k_bits.ndim != 4 or v_bits.ndim != 4:
        raise ValueError("attention takes [batch, heads, seq, dim] arrays")
    B, H, Sq, D = q_bits.shape
    if k_bits.shape[:2] != (B, H) or v_bits.shape[:2] != (B, H) or k_bits.shape != v_bits.shape \
            or k_bits.shape[3] != D:
        raise ValueError("Q, K, V shapes disagree")
    Skv = k_bits.shape[2]
    ptrs, strides = [], []
    for x in (q_bits, k_bits, v_bits):
        ptr, st = _operand(x, dtype)
        if D > 1 and st[3] != 1:
            raise ValueError("oracle attention needs a unit stride along head_dim")
        ptrs.append(ptr)
        strides.append(st[:3])
    if scale is None:
        scale = 1.0 / np.sqrt(D) if D > 0 else 1.0
    o = np.zeros((B, H, Sq, D), dtype=np.float64)
    lse = np.zeros((B, H, Sq), dtype=np.float64)
    rc = _load().ref_attention(B, H, Sq, Skv, D, _CODES[dtype], ptrs[0], *strides[0], ptrs[1], *strides[1],
                               ptrs[2], *strides[2], float(scale), 1 if causal else 0, o.ctypes.data,
                               lse.ctypes.data)
    if rc != 0:
        raise MemoryError("oracle could not allocate its score row")
    return o, lse
