"""Python binding of the MI355X dense GEMM library (C-ABI in include/dg.h).

Argument marshalling only: every step of the product runs in the HIP library
`lib/libdg.so`. PyTorch supplies device memory and the stream. There is no CPU
fallback: if the library is missing, every call raises.

    C = gemm(A, B)                      # C[M,N] = A[M,K] @ B[K,N], fp32 accumulate
    C = gemm(A, B, out_dtype=torch.float32)
    cfg, ms = autotune(A, B, out)       # benchmark candidates, cache the fastest
    C = gemm_ex(A, B, bias=b, activation="relu")       # fused epilogue
    C = gemm_ex(A3, B3)                 # strided batch: [batch, M, K] @ [batch, K, N]
    Y = linear(X, W, b)                 # autograd: Y = X @ W^T + b
    O, lse = attention(Q, K, V, causal=True)           # softmax(QK^T/sqrt(d)) V, blockwise
"""
import ctypes
import os

from .build import LIB

__all__ = [
    "Config", "DGError", "gemm", "gemm_config", "autotune", "select_config", "candidates",
    "Epilogue", "Batch", "gemm_ex", "gemm_ex_noalloc", "autotune_ex", "workspace_size", "select_config_ex", "matmul", "linear",
    "attention",
    "validate", "tile_coords", "grid_shape", "cache_clear", "cache_save", "cache_load",
    "cache_size", "library", "DG_F32", "DG_F16", "DG_BF16", "VARIANT_SIMT", "VARIANT_MFMA",
]

DG_F32, DG_F16, DG_BF16 = 0, 1, 2
VARIANT_SIMT, VARIANT_MFMA = 0, 1
ACTIVATIONS = {None: 0, "none": 0, "relu": 1, "gelu": 2}
STATUS = {0: "DG_OK", 1: "DG_ERR_INVALID_VALUE", 2: "DG_ERR_UNSUPPORTED", 3: "DG_ERR_NO_CONFIG", 4: "DG_ERR_HIP"}


class DGError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


class Config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("block_m", "block_n", "block_k", "group_m", "waves", "stages", "variant", "xcd_remap",
                 "k_splits")]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}

    def __repr__(self):
        return "Config(" + ", ".join(f"{k}={v}" for k, v in self.as_dict().items()) + ")"

    def __eq__(self, other):
        return isinstance(other, Config) and self.as_dict() == other.as_dict()


class Epilogue(ctypes.Structure):
    """dg_epilogue: C = act(alpha * A@B + beta * R + bias)."""
    _fields_ = [("alpha", ctypes.c_float), ("beta", ctypes.c_float), ("residual", ctypes.c_void_p),
                ("residual_dtype", ctypes.c_int32), ("stride_rm", ctypes.c_int64), ("stride_rn", ctypes.c_int64),
                ("bias", ctypes.c_void_p), ("bias_dtype", ctypes.c_int32), ("bias_per_row", ctypes.c_int32),
                ("bias_stride", ctypes.c_int64), ("activation", ctypes.c_int32)]


class Batch(ctypes.Structure):
    """dg_batch: strided batch of products."""
    _fields_ = [(n, ctypes.c_int64) for n in
                ("count", "stride_a", "stride_b", "stride_c", "stride_r", "stride_bias")]


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
        lib.dg_select_config_ex.argtypes = _PROBLEM + [ctypes.POINTER(Batch), _i64, ctypes.POINTER(Config),
                                                       ctypes.POINTER(_i32)]
        lib.dg_validate.argtypes = _PROBLEM
        lib.dg_gemm_ex.argtypes = _PROBLEM + [_p, ctypes.POINTER(Epilogue), ctypes.POINTER(Batch),
                                              ctypes.POINTER(Config), _p, _i64]
        lib.dg_gemm_ex_noalloc.argtypes = _PROBLEM + [_p, ctypes.POINTER(Epilogue), ctypes.POINTER(Batch),
                                                      ctypes.POINTER(Config)]
        lib.dg_autotune_ex.argtypes = _PROBLEM + [_p, ctypes.POINTER(Epilogue), ctypes.POINTER(Batch), _p, _i64,
                                                  _i32, ctypes.POINTER(Config), ctypes.POINTER(ctypes.c_float)]
        lib.dg_workspace_size.argtypes = [_i64, _i64, _i64, _i64, ctypes.POINTER(Config), ctypes.POINTER(_i64)]
        _st = ctypes.POINTER(_i64)
        lib.dg_attention_fwd.argtypes = [_i64] * 5 + [_p, _st, _p, _st, _p, _st, _p, _st, _p, ctypes.c_int,
                                                      ctypes.c_int, ctypes.c_float, _i32, _p]
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
        for name in ("dg_gemm", "dg_gemm_config", "dg_autotune", "dg_select_config", "dg_select_config_ex",
                     "dg_validate",
                     "dg_gemm_ex", "dg_gemm_ex_noalloc", "dg_autotune_ex", "dg_workspace_size", "dg_attention_fwd",
                     "dg_get_candidate", "dg_tile_coords", "dg_grid_shape", "dg_cache_clear",
                     "dg_cache_save", "dg_cache_load"):
            getattr(lib, name).restype = ctypes.c_int
        _lib = lib
    return _lib


def _check(status):
    if status != 0:
        raise DGError(status, library().dg_last_error().decode(errors="replace"))


_DTYPE_CODES = None


def _dtype_code(dt):
    global _DTYPE_CODES
    if _DTYPE_CODES is None:
        import torch
        _DTYPE_CODES = {torch.float32: DG_F32, torch.float16: DG_F16, torch.bfloat16: DG_BF16}
    code = _DTYPE_CODES.get(dt)
    if code is None:
        raise TypeError(f"unsupported dtype {dt}; use float32, float16 or bfloat16")
    return code


def _problem(a, b, out):
    """Marshal (A, B, C) tensors into the C-ABI problem arguments.

    This runs on every call, so it reads each tensor property once: for small
    products the host time of the call is the whole cost."""
    if a.dim() != 2 or b.dim() != 2 or out.dim() != 2:
        raise ValueError("gemm takes 2-D tensors")
    M, K = a.shape
    K2, N = b.shape
    if K != K2:
        raise ValueError(f"inner dimensions differ: A is {tuple(a.shape)}, B is {tuple(b.shape)}")
    if out.shape[0] != M or out.shape[1] != N:
        raise ValueError(f"out must be {(M, N)}, got {tuple(out.shape)}")
    in_dt = a.dtype
    if in_dt != b.dtype:
        raise TypeError(f"A and B must share a dtype ({in_dt} vs {b.dtype})")
    if not (a.is_cuda and b.is_cuda and out.is_cuda):
        raise ValueError("A, B and out must be GPU tensors (there is no CPU path)")
    sa, sb, so = a.stride(), b.stride(), out.stride()
    return [M, N, K, a.data_ptr(), sa[0], sa[1], b.data_ptr(), sb[0], sb[1],
            out.data_ptr(), so[0], so[1], _dtype_code(in_dt), _dtype_code(out.dtype)]


_raw_stream = None


def _stream(t, stream):
    """The HIP stream to launch on: `stream`, else torch's current stream on t's device."""
    global _raw_stream
    if stream is not None:
        return ctypes.c_void_p(stream.cuda_stream)
    if _raw_stream is None:
        import torch
        # torch's own accessor of the current stream's raw handle (what its
        # kernel launchers use); the public torch.cuda.current_stream() builds
        # a Python stream object per call (~2.5 us).
        _raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", False)
    if _raw_stream:
        return ctypes.c_void_p(_raw_stream(t.get_device()))
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _out(a, b, out, out_dtype):
    if out is None:
        import torch
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


def select_config_ex(M, N, K, strides_a, strides_b, strides_c, in_dtype, out_dtype, batch=1,
                     workspace_bytes=0, batch_strides=(0, 0, 0), ptr_a=0, ptr_b=0, ptr_c=0):
    """The config gemm_ex would choose (no GPU work) for `batch` products and a workspace size."""
    cfg, hit = Config(), _i32()
    bt = Batch(count=batch, stride_a=batch_strides[0], stride_b=batch_strides[1], stride_c=batch_strides[2])
    if batch > 1 and batch_strides == (0, 0, 0):
        bt.stride_c = M * N  # a dense stack of C matrices
    _check(library().dg_select_config_ex(M, N, K, ptr_a or None, *strides_a, ptr_b or None, *strides_b,
                                         ptr_c or None, *strides_c, in_dtype, out_dtype, ctypes.byref(bt),
                                         workspace_bytes, ctypes.byref(cfg), ctypes.byref(hit)))
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


# ---- dg_gemm_ex: fused epilogue, strided batch, split-K ------------------------

# Split-K workspace the binding keeps per (device, stream), grown on demand.
# One buffer per stream: two split-K calls on different streams would otherwise
# write their partial tiles into the same memory at the same time. Each buffer
# is allocated while its stream is current, so torch's caching allocator ties
# it to that stream: when a grown buffer replaces it, the old memory is handed
# out again only to later work on the same stream, which runs after every
# kernel already queued there that reads it.
DEFAULT_WORKSPACE_BYTES = 64 << 20
STREAM_K = -1  # DG_STREAM_K of include/dg.h: Config.k_splits for stream-K
NOALLOC_SCRATCH_BYTES = 32 << 20  # DG_NOALLOC_SCRATCH_BYTES of include/dg.h
_workspaces = {}


def _workspace(t, nbytes, stream):
    """The cached split-K workspace for t's GPU and `stream` (a raw HIP stream
    handle, ctypes.c_void_p), grown to nbytes if needed."""
    key = (t.get_device(), stream.value or 0)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        import torch
        dev = torch.device("cuda", key[0])
        s = torch.cuda.ExternalStream(key[1], device=dev) if key[1] else torch.cuda.default_stream(dev)
        with torch.cuda.stream(s):
            ws = torch.empty(max(nbytes, DEFAULT_WORKSPACE_BYTES), dtype=torch.uint8, device=dev)
        _workspaces[key] = ws
    return ws


def workspace_size(M, N, K, batch, config):
    """Bytes of workspace a config needs: split-K partials, or stream-K flags and
    partials (0 if it needs none)."""
    total = _i64()
    _check(library().dg_workspace_size(M, N, K, batch, ctypes.byref(config), ctypes.byref(total)))
    return total.value


def _batched(t, name, rank):
    """(shape, strides) of one product's view, batch stride and batch count (None if unbatched)."""
    if t.dim() == rank:
        return tuple(t.shape), tuple(t.stride()), 0, None
    if t.dim() == rank + 1:
        return tuple(t.shape[1:]), tuple(t.stride()[1:]), (t.stride(0) if t.shape[0] > 1 else 0), t.shape[0]
    raise ValueError(f"{name} must have {rank} or {rank + 1} dimensions, got {t.dim()}")


def _ex_args(a, b, out, alpha, beta, residual, bias, bias_per_row, activation):
    if a.dtype != b.dtype:
        raise TypeError(f"A and B must share a dtype ({a.dtype} vs {b.dtype})")
    (M, K), (sam, sak), sa, na = _batched(a, "A", 2)
    (K2, N), (sbk, sbn), sb, nb = _batched(b, "B", 2)
    cshape, (scm, scn), sc, nc = _batched(out, "out", 2)
    counts = {n for n in (na, nb, nc) if n is not None}
    if len(counts) > 1:
        raise ValueError(f"batch sizes differ: {sorted(counts)}")
    count = counts.pop() if counts else 1
    if nc is None and (na is not None or nb is not None):
        raise ValueError("a batched product needs a 3-D out")
    if K != K2:
        raise ValueError(f"inner dimensions differ: A is {tuple(a.shape)}, B is {tuple(b.shape)}")
    if cshape != (M, N):
        raise ValueError(f"out must be {(M, N)} per product, got {cshape}")
    for name, t in (("A", a), ("B", b), ("out", out), ("residual", residual), ("bias", bias)):
        if t is not None and not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor (there is no CPU path)")
    if activation not in ACTIVATIONS:
        raise ValueError(f"activation must be one of {sorted(k for k in ACTIVATIONS if k)}")
    epi = Epilogue(alpha=alpha, beta=beta, activation=ACTIVATIONS[activation])
    sr = 0
    if residual is not None:
        rshape, (srm, srn), sr, nr = _batched(residual, "residual", 2)
        if nr is not None and nr != count:
            raise ValueError("residual batch differs")
        if rshape != (M, N):
            raise ValueError(f"residual must be {(M, N)} per product")
        epi.residual = residual.data_ptr()
        epi.residual_dtype = _dtype_code(residual.dtype)
        epi.stride_rm, epi.stride_rn = srm, srn
    sbias = 0
    if bias is not None:
        (blen,), (bstride,), sbias, nbias = _batched(bias, "bias", 1)
        if nbias is not None and nbias != count:
            raise ValueError("bias batch differs")
        if blen != (M if bias_per_row else N):
            raise ValueError(f"bias must have {M if bias_per_row else N} entries")
        epi.bias = bias.data_ptr()
        epi.bias_dtype = _dtype_code(bias.dtype)
        epi.bias_per_row = 1 if bias_per_row else 0
        epi.bias_stride = bstride
    batch = Batch(count=count, stride_a=sa, stride_b=sb, stride_c=sc, stride_r=sr, stride_bias=sbias)
    prob = [M, N, K, a.data_ptr(), sam, sak, b.data_ptr(), sbk, sbn,
            out.data_ptr(), scm, scn, _dtype_code(a.dtype), _dtype_code(out.dtype)]
    return prob, epi, batch


def _ex_out(a, b, out, out_dtype):
    import torch
    if out is not None:
        return out
    dt = out_dtype or a.dtype
    if a.dim() == 2 and b.dim() == 2:
        return torch.empty((a.shape[0], b.shape[1]), dtype=dt, device=a.device)
    n = a.shape[0] if a.dim() == 3 else b.shape[0]
    return torch.empty((n, a.shape[-2], b.shape[-1]), dtype=dt, device=a.device)


def gemm_ex(a, b, out=None, out_dtype=None, *, alpha=1.0, beta=0.0, residual=None, bias=None,
            bias_per_row=False, activation=None, config=None, workspace=True, stream=None):
    """C = act(alpha * A @ B + beta * R + bias), for one product or a strided batch.

    a: [M, K] or [batch, M, K]; b: [K, N] or [batch, K, N] (a 2-D operand is
    shared by the batch); out: [M, N] or [batch, M, N]. residual: None (R is
    out's prior contents when beta != 0) or [M, N] / [batch, M, N]. bias: [N]
    (or [M] with bias_per_row) / [batch, N]. activation: None, "relu", "gelu".
    config: explicit Config (k_splits > 1 = split-K, STREAM_K = stream-K) or
    None for the library's choice. workspace: True = the binding's cached
    workspace (grown to what the config needs), a CUDA tensor of any dtype,
    or None/False for none.
    """
    out = _ex_out(a, b, out, out_dtype)
    prob, epi, batch = _ex_args(a, b, out, alpha, beta, residual, bias, bias_per_row, activation)
    ws_ptr, ws_bytes = None, 0
    raw = _stream(a, stream)
    if workspace is True:
        need = 0
        if config is not None and (config.k_splits > 1 or config.k_splits == STREAM_K):
            need = workspace_size(prob[0], prob[1], prob[2], batch.count, config)
        ws = _workspace(a, need, raw)
        ws_ptr, ws_bytes = ws.data_ptr(), ws.numel()
    elif workspace is not None and workspace is not False:
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    _check(library().dg_gemm_ex(*prob, raw, ctypes.byref(epi), ctypes.byref(batch),
                                ctypes.byref(config) if config is not None else None, ws_ptr, ws_bytes))
    return out


def gemm_ex_noalloc(a, b, out, *, alpha=1.0, beta=0.0, residual=None, bias=None, bias_per_row=False,
                    activation=None, config=None, stream=None):
    """dg_gemm_ex_noalloc: gemm_ex with split-K / stream-K partials in the library's fixed
    per-GPU scratch (NOALLOC_SCRATCH_BYTES), so neither the library nor this
    call allocates device memory; `out` must be given. Calls that overlap in
    time on one GPU share the scratch and race."""
    prob, epi, batch = _ex_args(a, b, out, alpha, beta, residual, bias, bias_per_row, activation)
    _check(library().dg_gemm_ex_noalloc(*prob, _stream(a, stream), ctypes.byref(epi), ctypes.byref(batch),
                                        ctypes.byref(config) if config is not None else None))
    return out


def autotune_ex(a, b, out=None, out_dtype=None, *, alpha=1.0, beta=0.0, residual=None, bias=None,
                bias_per_row=False, activation=None, workspace=True, repeats=10, stream=None):
    """dg_autotune_ex: tune (including split-K counts with a workspace) and cache the winner."""
    out = _ex_out(a, b, out, out_dtype)
    prob, epi, batch = _ex_args(a, b, out, alpha, beta, residual, bias, bias_per_row, activation)
    ws_ptr, ws_bytes = None, 0
    raw = _stream(a, stream)
    if workspace is True:
        ws = _workspace(a, 0, raw)
        ws_ptr, ws_bytes = ws.data_ptr(), ws.numel()
    elif workspace is not None and workspace is not False:
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    cfg, ms = Config(), ctypes.c_float()
    _check(library().dg_autotune_ex(*prob, raw, ctypes.byref(epi), ctypes.byref(batch), ws_ptr,
                                    ws_bytes, repeats, ctypes.byref(cfg), ctypes.byref(ms)))
    return cfg, ms.value


# ---- autograd --------------------------------------------------------------------
# The backward of C = A @ B is two more products of the same kernel family,
# taken through transposed views (strides only): dA = dC @ B^T, dB = A^T @ dC
# ("如何用Triton手写Kernel优化矩阵乘与Flash Attention？", 性能对比与工程落地建议:
# wrap the forward kernel in an autograd function).

def _autograd_fn():
    import torch

    class _MatMul(torch.autograd.Function):
        @staticmethod
        def forward(ctx, a, b):
            ctx.save_for_backward(a, b)
            return gemm_ex(a, b)

        @staticmethod
        def backward(ctx, dc):
            a, b = ctx.saved_tensors
            da = db = None
            if ctx.needs_input_grad[0]:
                da = gemm_ex(dc, b.transpose(-1, -2))
            if ctx.needs_input_grad[1]:
                if a.dim() == 3 and b.dim() == 2:
                    # shared B: dB sums over the batch, i.e. one product over the stacked rows
                    db = gemm_ex(a.reshape(-1, a.shape[-1]).transpose(0, 1), dc.reshape(-1, dc.shape[-1]))
                else:
                    db = gemm_ex(a.transpose(-1, -2), dc)
            return da, db

    class _Linear(torch.autograd.Function):
        @staticmethod
        def forward(ctx, x, w, bias):
            ctx.save_for_backward(x, w)
            ctx.has_bias = bias is not None
            return gemm_ex(x, w.t(), bias=bias)

        @staticmethod
        def backward(ctx, dy):
            x, w = ctx.saved_tensors
            dx = dw = db = None
            if ctx.needs_input_grad[0]:
                dx = gemm_ex(dy, w)
            if ctx.needs_input_grad[1]:
                dw = gemm_ex(dy.t(), x)
            if ctx.has_bias and ctx.needs_input_grad[2]:
                # column sums of dY as the product ones[1, rows] @ dY
                ones = dy.new_ones((1, dy.shape[0]))
                db = gemm_ex(ones, dy)[0]
            return dx, dw, db

    return _MatMul, _Linear


_fns = None


def matmul(a, b):
    """Differentiable C = A @ B (2-D, or batched 3-D) on the HIP kernels."""
    global _fns
    _fns = _fns or _autograd_fn()
    return _fns[0].apply(a, b)


def linear(x, weight, bias=None):
    """Differentiable Y = X @ W^T + bias (x: [rows, in], weight: [out, in], bias: [out])."""
    global _fns
    _fns = _fns or _autograd_fn()
    return _fns[1].apply(x, weight, bias)


# ---- attention forward ------------------------------------------------------------

def attention(q, k, v, out=None, out_dtype=None, scale=None, causal=False, return_lse=False, stream=None):
    """O = softmax(scale * Q K^T [causal]) V on the HIP kernel (dg_attention_fwd).

    q: [batch, heads, seq_q, head_dim]; k, v: [batch, heads, seq_kv, head_dim]
    (any strides with a unit head_dim stride). scale defaults to
    1/sqrt(head_dim). Returns O (and the fp32 log-sum-exp [batch, heads,
    seq_q] when return_lse).
    """
    import torch
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("attention takes [batch, heads, seq, head_dim] tensors")
    B, H, Sq, D = q.shape
    if k.shape[:2] != (B, H) or v.shape != k.shape or k.shape[3] != D:
        raise ValueError(f"shapes disagree: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share a dtype")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor (there is no CPU path)")
        if D > 1 and t.stride(3) != 1:
            raise ValueError(f"{name} needs a unit stride along head_dim")
    if out is None:
        out = torch.empty((B, H, Sq, D), dtype=out_dtype or q.dtype, device=q.device)
    if tuple(out.shape) != (B, H, Sq, D) or (D > 1 and out.stride(3) != 1):
        raise ValueError("out must be [batch, heads, seq_q, head_dim] with a unit head_dim stride")
    lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device) if return_lse else None

    def strides(t):
        return (_i64 * 3)(*t.stride()[:3])

    _check(library().dg_attention_fwd(B, H, Sq, k.shape[2], D, q.data_ptr(), strides(q), k.data_ptr(),
                                      strides(k), v.data_ptr(), strides(v), out.data_ptr(), strides(out),
                                      lse.data_ptr() if lse is not None else None, _dtype_code(q.dtype),
                                      _dtype_code(out.dtype), float(scale) if scale else 0.0,
                                      1 if causal else 0, _stream(q, stream)))
    return (out, lse) if return_lse else out
