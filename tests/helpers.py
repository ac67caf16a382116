"""Shared test helpers: tolerances, output decoding, sampling of large outputs."""
import math

import numpy as np
import torch

from dense_gemm_07_amd import inputs

# Significand bits and minimum normal exponent of each output format.
FORMATS = {"f32": (24, -126), "f16": (11, -14), "bf16": (8, -126)}


def ulp(dtype, x):
    """Unit in the last place of |x| in `dtype` (elementwise, numpy)."""
    p, emin = FORMATS[dtype]
    ax = np.abs(np.asarray(x, dtype=np.float64))
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    e = np.maximum(e, emin)
    return np.ldexp(1.0, (e - (p - 1)).astype(np.int64))


def tolerance(K, in_dtype, out_dtype, got, ref):
    """Allowed |C_gpu - C_ref| per element.

    1e-3 * sqrt(K) for fp16/bf16 inputs and 1e-5 * sqrt(K) for fp32 inputs
    (fp32 accumulation in an unspecified order), plus half an ulp of the
    output dtype at the larger of the two magnitudes: a correctly rounded
    fp16/bf16 output may differ from the fp64 reference by up to that much
    on its own.
    """
    base = (1e-5 if in_dtype == "f32" else 1e-3) * math.sqrt(max(K, 1))
    mag = np.maximum(np.abs(got), np.abs(ref))
    return base + 0.5 * ulp(out_dtype, mag)


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact fp64 values of a (GPU or CPU) tensor."""
    return t.detach().to("cpu").double().numpy()


def out_bits(t: torch.Tensor, out_dtype: str) -> np.ndarray:
    return inputs.bits(t.detach().to("cpu").contiguous(), out_dtype)


def assert_within(got, ref, K, in_dtype, out_dtype, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    tol = tolerance(K, in_dtype, out_dtype, got, ref)
    bad = err > tol
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; "
                             f"max err {err.max():.3e}; first bad {idx.tolist()} "
                             f"got {got[tuple(idx[0])]} ref {ref[tuple(idx[0])]}")
    return float(err.max()) if err.size else 0.0


def assert_bits_equal(got_bits, want_bits, what=""):
    """Bit-exact comparison, +0 and -0 counted equal."""
    g = np.asarray(got_bits).astype(np.uint32)
    w = np.asarray(want_bits).astype(np.uint32)
    sign = np.uint32(0x80000000 if np.asarray(got_bits).dtype == np.uint32 else 0x8000)
    zero_g = (g & ~sign) == 0
    zero_w = (w & ~sign) == 0
    same = (g == w) | (zero_g & zero_w)
    if not same.all():
        idx = np.argwhere(~same)[:5]
        raise AssertionError(f"{what}: {int((~same).sum())} of {same.size} differ; first {idx.tolist()} "
                             f"got {hex(int(g[tuple(idx[0])]))} want {hex(int(w[tuple(idx[0])]))}")


def sample_indices(M, N, n_random=2048, seed=0):
    """Rows/cols of C to check: tile edges (multiples of 32..256, +-1), corners, random."""
    rng = np.random.default_rng(seed)
    def edges(D):
        s = {0, D - 1}
        for t in (32, 64, 128, 256):
            for m in range(t, D, t * 7):
                s.update({m - 1, m})
        return np.array(sorted(x for x in s if 0 <= x < D), dtype=np.int64)
    er, ec = edges(M), edges(N)
    rr, cc = np.meshgrid(er[:40], ec[:40], indexing="ij")
    rows = np.concatenate([rr.ravel(), rng.integers(0, M, n_random)])
    cols = np.concatenate([cc.ravel(), rng.integers(0, N, n_random)])
    return rows, cols


def epilogue_tolerance(K, in_dtype, out_dtype, got, ref, alpha, terms, act):
    """Allowed |C_gpu - C_ref| for act(alpha * P + beta * R + bias).

    The product's own error (tolerance above, before rounding) scaled by
    |alpha|; the fp32 multiply, fused multiply-add and add of the epilogue
    each round once, bounded by 2^-22 * terms, where terms = |alpha*P| +
    |beta*R| + |bias| (fp64); ReLU is 1-Lipschitz; GELU's slope is below
    1.13 and its fp32 evaluation adds a few ulp of the result (2^-19 relative
    plus 2^-40 absolute); then half an ulp of the output dtype.
    """
    base = (1e-5 if in_dtype == "f32" else 1e-3) * math.sqrt(max(K, 1))
    pre = abs(float(alpha)) * base + 2.0 ** -22 * np.asarray(terms, dtype=np.float64)
    mag = np.maximum(np.abs(got), np.abs(ref))
    if act == "gelu":
        pre = 1.13 * pre + 2.0 ** -19 * mag + 2.0 ** -40
    return pre + 0.5 * ulp(out_dtype, mag)


def assert_within_tol(got, ref, tol, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    same_nan = np.isnan(got) & np.isnan(ref)
    assert np.all(np.isfinite(got) | same_nan), f"{what}: non-finite output"
    err = np.where(same_nan, 0.0, np.abs(got - ref))
    bad = err > tol
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; "
                             f"max err {err.max():.3e}; first bad {idx.tolist()} "
                             f"got {got[tuple(idx[0])]} ref {ref[tuple(idx[0])]}")
    return float(err.max()) if err.size else 0.0
