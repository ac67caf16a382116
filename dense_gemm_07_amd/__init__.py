"""Python binding of the MI355X dense GEMM library (C-ABI in include/dg.h).

Argument marshalling only: every step of the product runs in the HIP library
`lib/libdg.so`. PyTorch supplies device memory and the stream. There is no CPU
fallback: if the library is missing, every call raises.

    C = gemm(A, B)                      # C[M,N] = A[M,K] @ B[K,N], fp32 accumulate
    C = gemm(A, B, out_dtype=torch.float32)
    cfg, ms = autotune(A, B, out)       # benchmark candidates, cache the fastest
"""
import ctypes
import os

from .build import LIB

__all__ = [
    "Config", "DGError", "gemm", "gemm_config", "autotune", "select_config", "candidates",
    "validate", "tile_coords", "grid_shape", "cache_clear", "cache_save", "cache_load",
    "cache_size", "library", "DG_F32", "DG_F16", "DG_BF16", "VARIANT_SIMT", "VARIANT_MFMA",
]

DG_F32, DG_F16, DG_BF16 = 0, 1, 2
VARIANT_SIMT, VARIANT_MFMA = 0, 1
STATUS = {0: "DG_OK", 1: "DG_ERR_INVALID_VALUE", 2: "DG_ERR_UNSUPPORTED", 3: "DG_ERR_NO_CONFIG", 4: "DG_ERR_HIP"}


class DGError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


class Config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("block_m", "block_n", "block_k", "group_m", "waves", "stages", "variant", "xcd_remap")]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}

    def __repr__(self):
        return "Config(" + ", ".join(f"{k}={v}" for k, v in self.as_dict().items()) + ")"

    def __eq__(self, other):
        return isinstance(other, Config) and self.as_dict() == other.as_dict()


_lib = None
_i64, _i32, _p = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
_PROBLEM = [_i64, _i64, _i64, _p, _i64, _i64, _p, _i64, _i64, _p, _i64, _i64, ctypes.c_int, ctypes.c_int]


def library():
    """The loaded C-ABI library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            raise RuntimeError(f"HIP library {LIB} is not built; run `python -m dense_gemm_07_amd.build`")
        lib = ctypes.CDLL(LIB)
        lib.dg_gemm.argtypes = _PROBLEM + [_p]
        lib.dg_gemm_config.argtypes = _PROBLEM + [_p, ctypes.POINTER(Config)]
        lib.dg_autotune.argtypes = _PROBLEM + [_p, _i32, ctypes.POINTER(Config), ctypes.POINTER(ctypes.c_float)]
        lib.dg_select_config.argtypes = _PROBLEM + [ctypes.POINTER(Config), ctypes.POINTER(_i32)]
        lib.dg_validate.argtypes = _PROBLEM
        lib.dg_num_candidates.argtypes = [ctypes.c_int, ctypes.c_int]
        lib.dg_num_candidates.restype = _i32
        lib.dg_get_candidate.argtypes = [_i32, ctypes.c_int, ctypes.c_int, ctypes.POINTER(Config)]
        lib.dg_tile_coords.argtypes = [_i32] * 6 + [ctypes.POINTER(_i32), ctypes.POINTER(_i32)]
        lib.dg_grid_shape.argtypes = [_i64, _i64, _i64, ctypes.POINTER(Config)] + [ctypes.POINTER(_i64)] * 3
        lib.dg_cache_save.argtypes = [ctypes.c_char_p]
        lib.dg_cache_load.argtypes = [ctypes.c_char_p]
        lib.dg_cache_size.restype = _i32
        lib.dg_status_string.restype = ctypes.c_char_p
        lib.dg_last_error.restype = ctypes.c_char_p
        for name in ("dg_gemm", "dg_gemm_config", "dg_autotune", "dg_select_config", "dg_validate",
                     "dg_get_candidate", "dg_tile_coords", "dg_grid_shape", "dg_cache_clear",
                     "dg_cache_save", "dg_cache_load"):
            getattr(lib, name).restype = ctypes.c_int
        _lib = lib
    return _lib


def _check(status):
    if status != 0:
        raise DGError(status, library().dg_last_error().decode(errors="replace"))


def _dtype_code(dt):
    import torch
    codes = {torch.float32: DG_F32, torch.float16: DG_F16, torch.bfloat16: DG_BF16}
    if dt not in codes:
        raise TypeError(f"unsupported dtype {dt}; use float32, float16 or bfloat16")
    return codes[dt]


def _problem(a, b, out):
    """Marshal (A, B, C) tensors into the C-ABI problem arguments."""
    if a.dim() != 2 or b.dim() != 2 or out.dim() != 2:
        raise ValueError("gemm takes 2-D tensors")
    M, K = a.shape
    K2, N = b.shape
    if K != K2:
        raise ValueError(f"inner dimensions differ: A is {tuple(a.shape)}, B is {tuple(b.shape)}")
    if tuple(out.shape) != (M, N):
        raise ValueError(f"out must be {(M, N)}, got {tuple(out.shape)}")
    if a.dtype != b.dtype:
        raise TypeError(f"A and B must share a dtype ({a.dtype} vs {b.dtype})")
    for name, t in (("A", a), ("B", b), ("out", out)):
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be a GPU tensor (there is no CPU path)")
    return [M, N, K, a.data_ptr(), a.stride(0), a.stride(1), b.data_ptr(), b.stride(0), b.stride(1),
            out.data_ptr(), out.stride(0), out.stride(1), _dtype_code(a.dtype), _dtype_code(out.dtype)]


def _stream(t, stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream(t.device)
    return ctypes.c_void_p(s.cuda_stream)


def _out(a, b, out, out_dtype):
    import torch
    if out is None:
        out = torch.empty((a.shape[0], b.shape[1]), dtype=out_dtype or a.dtype, device=a.device)
    return out


def gemm(a, b, out=None, out_dtype=None, stream=None):
    """C = A @ B on the GPU (fp32 accumulation, RNE into C's dtype)."""
    out = _out(a, b, out, out_dtype)
    _check(library().dg_gemm(*_problem(a, b, out), _stream(a, stream)))
    return out


def gemm_config(a, b, config, out=None, out_dtype=None, stream=None):
    """C = A @ B with an explicit kernel configuration."""
    out = _out(a, b, out, out_dtype)
    _check(library().dg_gemm_config(*_problem(a, b, out), _stream(a, stream), ctypes.byref(config)))
    return out


def autotune(a, b, out=None, out_dtype=None, repeats=10, stream=None):
    """Benchmark every candidate on these buffers; cache and return the fastest."""
    out = _out(a, b, out, out_dtype)
    cfg, ms = Config(), ctypes.c_float()
    _check(library().dg_autotune(*_problem(a, b, out), _stream(a, stream), repeats,
                                 ctypes.byref(cfg), ctypes.byref(ms)))
    return cfg, ms.value


def select_config(a, b, out):
    """The config `gemm` would use (no GPU work) and whether it came from the cache."""
    cfg, hit = Config(), _i32()
    _check(library().dg_select_config(*_problem(a, b, out), ctypes.byref(cfg), ctypes.byref(hit)))
    return cfg, bool(hit.value)


def select_config_raw(M, N, K, strides_a, strides_b, strides_c, in_dtype, out_dtype,
                      ptr_a=0, ptr_b=0, ptr_c=0):
    """select_config from plain sizes/strides (pointers only set alignment)."""
    cfg, hit = Config(), _i32()
    _check(library().dg_select_config(M, N, K, ptr_a or None, *strides_a, ptr_b or None, *strides_b,
                                      ptr_c or None, *strides_c, in_dtype, out_dtype,
                                      ctypes.byref(cfg), ctypes.byref(hit)))
    return cfg, bool(hit.value)


def validate(M, N, K, ptr_a, strides_a, ptr_b, strides_b, ptr_c, strides_c, in_dtype, out_dtype):
    """Status code of the argument check dg_gemm performs (0 = DG_OK); no GPU work."""
    lib = library()
    return lib.dg_validate(M, N, K, ptr_a, *strides_a, ptr_b, *strides_b, ptr_c, *strides_c,
                           in_dtype, out_dtype)


def candidates(in_dtype, out_dtype):
    lib = library()
    out = []
    for i in range(lib.dg_num_candidates(in_dtype, out_dtype)):
        c = Config()
        _check(lib.dg_get_candidate(i, in_dtype, out_dtype, ctypes.byref(c)))
        out.append(c)
    return out


def tile_coords(grid_m, grid_n, group_m, xcd_remap, num_xcd, wg):
    pm, pn = _i32(), _i32()
    _check(library().dg_tile_coords(grid_m, grid_n, group_m, xcd_remap, num_xcd, wg,
                                    ctypes.byref(pm), ctypes.byref(pn)))
    return pm.value, pn.value


def grid_shape(M, N, K, config):
    gm, gn, ks = _i64(), _i64(), _i64()
    _check(library().dg_grid_shape(M, N, K, ctypes.byref(config), ctypes.byref(gm), ctypes.byref(gn),
                                   ctypes.byref(ks)))
    return gm.value, gn.value, ks.value


def cache_clear():
    _check(library().dg_cache_clear())


def cache_size():
    return library().dg_cache_size()


def cache_save(path):
    _check(library().dg_cache_save(os.fsencode(path)))


def cache_load(path):
    _check(library().dg_cache_load(os.fsencode(path)))
