"""Seeded synthetic operands for C = A @ B.

This module draws random matrices and nothing else: it holds none of the
product's arithmetic, so both the HIP path and the CPU oracle may be fed from
it. It does not import the HIP library.

Recipe (one generator per call): a torch CPU generator seeded with `seed`
draws A first, then B, in fp32; each is then rounded to the input dtype by
torch's round-to-nearest-even cast. uniform[-1, 1) is `2*rand - 1`;
N(0, s) is `s * randn`. A column-major B is drawn as its row-major storage
[N, K] and handed out as the transposed view (strides (1, K)).
"""
import re
from dataclasses import dataclass

import numpy as np
import torch

TORCH_DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
BITS_TORCH = {"f32": torch.int32, "f16": torch.int16, "bf16": torch.int16}
BITS_NUMPY = {"f32": np.uint32, "f16": np.uint16, "bf16": np.uint16}


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    in_dtype: str
    out_dtype: str
    a_dist: tuple          # ("uniform",) or ("normal", std)
    b_dist: tuple
    b_colmajor: bool = False

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K

    def compulsory_bytes(self) -> int:
        isz = 4 if self.in_dtype == "f32" else 2
        osz = 4 if self.out_dtype == "f32" else 2
        return isz * (self.M * self.K + self.K * self.N) + osz * self.M * self.N


# The five workloads the pages' method is measured and checked on.
WORKLOADS = {
    w.name: w for w in [
        # the naive example's size (26 x 26), fp32 throughout
        Workload("tiny_26_f32", 26, 26, 26, "f32", "f32", ("uniform",), ("uniform",)),
        Workload("square_1024_f16", 1024, 1024, 1024, "f16", "f16", ("normal", 1.0), ("normal", 1.0)),
        Workload("ragged_1000x1500x777_bf16_colB", 1000, 1500, 777, "bf16", "f32",
                 ("uniform",), ("uniform",), b_colmajor=True),
        Workload("square_4096_bf16", 4096, 4096, 4096, "bf16", "bf16", ("normal", 0.02), ("normal", 0.02)),
        Workload("mlp_8192x14336x4096_bf16", 8192, 14336, 4096, "bf16", "bf16",
                 ("normal", 1.0), ("normal", 0.02)),
    ]
}


# Skinny products (few rows of A against the MLP weight shape): bandwidth-bound,
# measured in HBM GB/s. Not among the five workloads above.
SKINNY = {
    w.name: w for w in [
        Workload(f"skinny_m{m}_14336x4096_bf16", m, 14336, 4096, "bf16", "bf16", ("normal", 1.0), ("normal", 0.02))
        for m in (1, 16, 64, 128)
    ]
}


# Shapes for the split-K and batched measurements (few output tiles and a long
# K; a stack of attention-score-sized products). Not among the five workloads.
EXTRA = {
    w.name: w for w in [
        Workload("splitk_512x512x16384_bf16", 512, 512, 16384, "bf16", "bf16", ("normal", 0.02), ("normal", 0.02)),
        Workload("splitk_128x4096x8192_bf16", 128, 4096, 8192, "bf16", "bf16", ("normal", 0.02), ("normal", 0.02)),
        Workload("splitk_256x256x32768_bf16", 256, 256, 32768, "bf16", "f32", ("normal", 0.02), ("normal", 0.02)),
        Workload("splitk_2048x512x8192_bf16", 2048, 512, 8192, "bf16", "bf16", ("normal", 0.02), ("normal", 0.02)),
        Workload("splitk_512x512x4096_bf16", 512, 512, 4096, "bf16", "bf16", ("normal", 0.02), ("normal", 0.02)),
        Workload("splitk_128x128x8192_bf16", 128, 128, 8192, "bf16", "bf16", ("normal", 0.02), ("normal", 0.02)),
        Workload("splitk_64x64x65536_bf16", 64, 64, 65536, "bf16", "f32", ("normal", 0.02), ("normal", 0.02)),
        Workload("square_1024_bf16", 1024, 1024, 1024, "bf16", "bf16", ("normal", 0.02), ("normal", 0.02)),
        Workload("square_4096_f32", 4096, 4096, 4096, "f32", "f32", ("normal", 1.0), ("normal", 1.0)),
        Workload("bmm_1024x1024x128_bf16", 1024, 1024, 128, "bf16", "bf16", ("normal", 1.0), ("normal", 1.0)),
    ]
}


def find(name: str) -> Workload:
    """A workload by name from any of the tables, or a plain product named
    gemm_<M>x<N>x<K>_<dtype> (row-major operands from N(0, 0.02), output in
    the input dtype), for measurements across sizes."""
    for table in (WORKLOADS, SKINNY, EXTRA):
        if name in table:
            return table[name]
    m = re.fullmatch(r"gemm_(\d+)x(\d+)x(\d+)_(bf16|f16|f32)", name)
    if m:
        M, N, K = (int(x) for x in m.groups()[:3])
        dt = m.group(4)
        return Workload(name, M, N, K, dt, dt, ("normal", 0.02), ("normal", 0.02))
    raise KeyError(f"unknown workload {name!r}")


def make_batch(w: Workload, count: int, seed: int = 0):
    """(A, B) stacks [count, M, K] and [count, K, N] (same recipe, drawn in one go)."""
    gen = torch.Generator().manual_seed(seed)
    dt = TORCH_DTYPES[w.in_dtype]
    a = _draw((count, w.M, w.K), w.a_dist, gen).to(dt)
    b = _draw((count, w.K, w.N), w.b_dist, gen).to(dt)
    return a, b


def _draw(shape, dist, gen):
    if dist[0] == "uniform":
        return torch.rand(shape, generator=gen, dtype=torch.float32) * 2.0 - 1.0
    if dist[0] == "normal":
        return torch.randn(shape, generator=gen, dtype=torch.float32) * float(dist[1])
    raise ValueError(f"unknown distribution {dist}")


def make(w: Workload, seed: int = 0):
    """(A, B) as CPU tensors of w.in_dtype; A is [M, K], B a [K, N] view."""
    gen = torch.Generator().manual_seed(seed)
    dt = TORCH_DTYPES[w.in_dtype]
    a = _draw((w.M, w.K), w.a_dist, gen).to(dt)
    if w.b_colmajor:
        b = _draw((w.N, w.K), w.b_dist, gen).to(dt).t()
    else:
        b = _draw((w.K, w.N), w.b_dist, gen).to(dt)
    return a, b


def random_operands(M, N, K, in_dtype, seed=0, dist=("uniform",), b_colmajor=False,
                    a_colmajor=False):
    """Random operands of any shape and layout (same recipe as `make`)."""
    gen = torch.Generator().manual_seed(seed)
    dt = TORCH_DTYPES[in_dtype]
    a = _draw((K, M), dist, gen).to(dt).t() if a_colmajor else _draw((M, K), dist, gen).to(dt)
    b = _draw((N, K), dist, gen).to(dt).t() if b_colmajor else _draw((K, N), dist, gen).to(dt)
    return a, b


def integer_operands(M, N, K, in_dtype, seed=0, lo=-2, hi=2, b_colmajor=False,
                     a_colmajor=False):
    """Operands with small integer values in [lo, hi] (exact in every dtype)."""
    gen = torch.Generator().manual_seed(seed)
    dt = TORCH_DTYPES[in_dtype]

    def ints(shape):
        return torch.randint(lo, hi + 1, shape, generator=gen, dtype=torch.int32).to(dt)

    a = ints((K, M)).t() if a_colmajor else ints((M, K))
    b = ints((N, K)).t() if b_colmajor else ints((K, N))
    return a, b


def bits(t: torch.Tensor, in_dtype: str) -> np.ndarray:
    """Raw bit patterns of a CPU tensor as a numpy view with the same strides."""
    if t.device.type != "cpu":
        raise ValueError("bits() needs a CPU tensor")
    return t.view(BITS_TORCH[in_dtype]).numpy().view(BITS_NUMPY[in_dtype])


def to_device_like(t: torch.Tensor, device) -> torch.Tensor:
    """Copy to `device`, keeping a transposed view transposed (same strides)."""
    if t.is_contiguous():
        return t.to(device)
    if t.t().is_contiguous():
        return t.t().contiguous().to(device).t()
    return t.contiguous().to(device)
