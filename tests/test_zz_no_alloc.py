"""GPU parity of the allocation-free entry point dg_gemm_ex_noalloc.

It runs the same kernels as dg_gemm_ex, with split-K / stream-K partial tiles in the
library's fixed per-GPU scratch array instead of a caller workspace. Each case
calls it through the C-ABI and compares with dg_gemm_ex (given a workspace) on
the same inputs and config: bit-exact, since both run the same kernels with
the same K ranges; integer inputs also pin both to the oracle bit for bit.
Two calls in a row, the second smaller, show that what the scratch keeps from
the previous call never leaks into a result.
"""
import sys

import numpy as np
import pytest
import torch

import dense_gemm_07_amd as dg
import oracle
from dense_gemm_07_amd import inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    oracle.build()
    dg.library()
    yield
    torch.cuda.synchronize()


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def split_config(bm, bn, bk, stages, splits):
    for c in dg.candidates(dg.DG_BF16, dg.DG_BF16):
        if (c.block_m, c.block_n, c.block_k, c.stages) == (bm, bn, bk, stages):
            c.group_m, c.xcd_remap, c.k_splits = 8, 1, splits
            return c
    raise LookupError((bm, bn, bk, stages))


def bits(t, dtype):
    return inputs.bits(t.cpu(), dtype)


def run_pair(M, N, K, cfg, seed, epilogue):
    """dg_gemm_ex_noalloc and dg_gemm_ex (cached workspace) on the same integer
    inputs; returns both outputs' bits and the oracle's."""
    a, b = inputs.integer_operands(M, N, K, "bf16", seed=seed)
    ad, bd = a.to(DEV), b.to(DEV)
    bias = torch.randint(-3, 4, (N,), generator=torch.Generator().manual_seed(seed + 1)).float()
    kw = dict(bias=bias.to(DEV), activation="relu", alpha=2.0) if epilogue else {}
    c_free = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    c_ws = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    dg.gemm_ex_noalloc(ad, bd, c_free, config=cfg, **kw)
    dg.gemm_ex(ad, bd, out=c_ws, config=cfg, workspace=True, **kw)
    torch.cuda.synchronize()
    p = oracle.gemm(inputs.bits(a, "bf16"), inputs.bits(b, "bf16"), "bf16")
    if epilogue:
        p = oracle.epilogue(p, alpha=2.0, beta=0.0, bias_bits=inputs.bits(bias, "f32"), bias_dtype="f32",
                            act="relu")
    return bits(c_free, "f32"), bits(c_ws, "f32"), oracle.encode(p, "f32")


@pytest.mark.parametrize("epilogue", [False, True])
def test_noalloc_matches_workspace_entry_two_calls(epilogue):
    """Explicit split-K configs: a larger call, then a smaller one on another tile
    shape, each bit-exact against dg_gemm_ex and the oracle."""
    cases = [((300, 200, 4096), split_config(64, 64, 64, 4, 4), 11),
             ((100, 70, 2056), split_config(128, 128, 64, 2, 3), 12)]
    for (M, N, K), cfg, seed in cases:
        note(f"noalloc {M}x{N}x{K} splits={cfg.k_splits} tile={cfg.block_m}x{cfg.block_n} epilogue={epilogue}")
        free, ws, want = run_pair(M, N, K, cfg, seed, epilogue)
        assert np.array_equal(free, ws), f"{M}x{N}x{K}: noalloc differs from dg_gemm_ex"
        assert np.array_equal(free, want), f"{M}x{N}x{K}: noalloc differs from the oracle"


def test_noalloc_default_choice_two_calls():
    """cfg == NULL: the library's choice with the scratch as workspace (it splits
    these long-K, few-tile shapes); random inputs, bit-exact against dg_gemm_ex
    given a workspace of the same size, within tolerance of the oracle."""
    ws = torch.empty(dg.NOALLOC_SCRATCH_BYTES, dtype=torch.uint8, device=DEV)
    for (M, N, K), seed in (((136, 120, 8200), 21), ((40, 72, 4100), 22)):
        cfg, _ = dg.select_config_ex(M, N, K, (K, 1), (N, 1), (N, 1), dg.DG_BF16, dg.DG_BF16,
                                     workspace_bytes=dg.NOALLOC_SCRATCH_BYTES)
        note(f"noalloc default {M}x{N}x{K}: {cfg}")
        assert cfg.k_splits > 1, cfg
        a, b = inputs.random_operands(M, N, K, "bf16", seed=seed)
        ad, bd = a.to(DEV), b.to(DEV)
        c_free = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
        c_ws = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
        dg.gemm_ex_noalloc(ad, bd, c_free)
        dg.gemm_ex(ad, bd, out=c_ws, workspace=ws)
        torch.cuda.synchronize()
        assert np.array_equal(bits(c_free, "bf16"), bits(c_ws, "bf16")), f"{M}x{N}x{K}"
        ref = oracle.gemm(inputs.bits(a, "bf16"), inputs.bits(b, "bf16"), "bf16")
        got = c_free.float().cpu().double().numpy()
        half_ulp = 0.5 * np.ldexp(1.0, np.floor(np.log2(np.maximum(np.abs(ref), 2.0 ** -126))).astype(int) - 7)
        assert np.all(np.abs(got - ref) <= 1e-3 * np.sqrt(K) + half_ulp), f"{M}x{N}x{K}"


def test_noalloc_rejects_partials_beyond_scratch():
    """An explicit split whose partials exceed the scratch: DG_ERR_UNSUPPORTED,
    nothing enqueued (C keeps its contents)."""
    M = N = 2048
    K = 256
    cfg = split_config(64, 64, 64, 4, 4)  # 1024 tiles x 4 ranges x 16 KiB = 64 MiB of partials
    assert dg.workspace_size(M, N, K, 1, cfg) > dg.NOALLOC_SCRATCH_BYTES
    a = torch.zeros((M, K), dtype=torch.bfloat16, device=DEV)
    b = torch.zeros((K, N), dtype=torch.bfloat16, device=DEV)
    c = torch.full((M, N), 7.0, dtype=torch.float32, device=DEV)
    with pytest.raises(dg.DGError) as e:
        dg.gemm_ex_noalloc(a, b, c, config=cfg)
    assert e.value.status == 2 and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert bool((c == 7.0).all())


def test_noalloc_stream_k_two_calls():
    """Stream-K keeps its flags and partials in the scratch too: a 1000x1496x776
    product (384 tiles of 64x64, 1.5 rounds), then a smaller 128x128-tile call,
    bit-exact against dg_gemm_ex and the oracle."""
    cases = [((1000, 1496, 776), split_config(64, 64, 64, 4, dg.STREAM_K), 31),
             ((700, 296, 200), split_config(128, 128, 64, 2, dg.STREAM_K), 32)]
    for (M, N, K), cfg, seed in cases:
        note(f"noalloc stream-K {M}x{N}x{K} tile={cfg.block_m}x{cfg.block_n}")
        free, ws, want = run_pair(M, N, K, cfg, seed, epilogue=True)
        assert np.array_equal(free, ws), f"{M}x{N}x{K}: noalloc differs from dg_gemm_ex"
        assert np.array_equal(free, want), f"{M}x{N}x{K}: noalloc differs from the oracle"
