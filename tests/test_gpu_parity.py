"""GPU parity: the HIP library against the CPU oracle, element by element.

Every call goes through the C-ABI (Python ctypes binding). Bars:
- small-integer inputs: bit-exact (all partial sums are integers below 2^24,
  so fp32 accumulation is exact in any order; the output must be the
  round-to-nearest-even of the exact sum);
- random inputs: |C_gpu - C_ref| <= 1e-3*sqrt(K) (fp16/bf16 in) or
  1e-5*sqrt(K) (fp32 in), plus half an ulp of the output dtype (see
  helpers.tolerance).
"""
import itertools
import sys
import zlib

import numpy as np
import pytest
import torch

import dense_gemm_07_amd as dg
import oracle
from dense_gemm_07_amd import inputs
from helpers import assert_bits_equal, assert_within, out_bits, sample_indices, to_f64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TD = inputs.TORCH_DTYPES
CODE = {"f32": dg.DG_F32, "f16": dg.DG_F16, "bf16": dg.DG_BF16}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    oracle.build()
    dg.library()
    dg.cache_clear()
    yield
    torch.cuda.synchronize()


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run(a_cpu, b_cpu, out_dtype, config=None, out=None):
    a = inputs.to_device_like(a_cpu, DEV)
    b = inputs.to_device_like(b_cpu, DEV)
    if config is None:
        c = dg.gemm(a, b, out=out, out_dtype=TD[out_dtype])
    else:
        c = dg.gemm_config(a, b, config, out=out, out_dtype=TD[out_dtype])
    torch.cuda.synchronize()
    return c


def ref_full(a_cpu, b_cpu, in_dtype):
    return oracle.gemm(inputs.bits(a_cpu, in_dtype), inputs.bits(b_cpu, in_dtype), in_dtype)


def check_random(a_cpu, b_cpu, in_dtype, out_dtype, config=None, what=""):
    c = run(a_cpu, b_cpu, out_dtype, config)
    ref = ref_full(a_cpu, b_cpu, in_dtype)
    return assert_within(to_f64(c), ref, a_cpu.shape[1], in_dtype, out_dtype, what)


def check_exact(a_cpu, b_cpu, in_dtype, out_dtype, config=None, what=""):
    c = run(a_cpu, b_cpu, out_dtype, config)
    want = oracle.encode(ref_full(a_cpu, b_cpu, in_dtype), out_dtype)
    assert_bits_equal(out_bits(c, out_dtype), want, what)


# ---- the five workloads ---------------------------------------------------------

SMALL = ["tiny_26_f32", "square_1024_f16", "ragged_1000x1500x777_bf16_colB", "square_4096_bf16"]


@pytest.mark.parametrize("name", SMALL)
def test_workload_random_full(name):
    w = inputs.WORKLOADS[name]
    note(f"workload {name} (full oracle)")
    a, b = inputs.make(w)
    err = check_random(a, b, w.in_dtype, w.out_dtype, what=name)
    note(f"  max abs err {err:.3e}")


@pytest.mark.parametrize("name", list(inputs.WORKLOADS))
def test_workload_default_launch(name):
    """The launch configuration the benchmark times: gemm with the built-in
    config choice, at full size, sampled against the oracle."""
    w = inputs.WORKLOADS[name]
    note(f"workload {name} (default config, sampled oracle)")
    a_cpu, b_cpu = inputs.make(w)
    a = inputs.to_device_like(a_cpu, DEV)
    b = inputs.to_device_like(b_cpu, DEV)
    c = torch.full((w.M, w.N), float("nan"), dtype=TD[w.out_dtype], device=DEV)
    dg.cache_clear()
    cfg, hit = dg.select_config(a, b, c)
    assert not hit
    dg.gemm(a, b, out=c)
    torch.cuda.synchronize()
    note(f"  config {cfg}")
    rows, cols = sample_indices(w.M, w.N, 3000, seed=4)
    ref = oracle.gemm_entries(inputs.bits(a_cpu, w.in_dtype), inputs.bits(b_cpu, w.in_dtype), w.in_dtype,
                              rows, cols)
    got = to_f64(c)
    assert np.all(np.isfinite(got)), "C not fully written"
    assert_within(got[rows, cols], ref, w.K, w.in_dtype, w.out_dtype, name)


@pytest.mark.parametrize("name", list(inputs.WORKLOADS))
def test_workload_autotuned_launch(name):
    """bench.py --autotune: autotune, then gemm with the cached winner."""
    w = inputs.WORKLOADS[name]
    note(f"workload {name} (autotuned config, sampled oracle)")
    a_cpu, b_cpu = inputs.make(w)
    a = inputs.to_device_like(a_cpu, DEV)
    b = inputs.to_device_like(b_cpu, DEV)
    c = torch.empty((w.M, w.N), dtype=TD[w.out_dtype], device=DEV)
    cfg, ms = dg.autotune(a, b, out=c, repeats=3)
    c.fill_(float("nan"))
    dg.gemm(a, b, out=c)
    torch.cuda.synchronize()
    note(f"  chosen {cfg} ({ms:.4f} ms)")
    rows, cols = sample_indices(w.M, w.N, 3000, seed=1)
    ref = oracle.gemm_entries(inputs.bits(a_cpu, w.in_dtype), inputs.bits(b_cpu, w.in_dtype), w.in_dtype,
                              rows, cols)
    got = to_f64(c)
    assert np.all(np.isfinite(got)), "C not fully written"
    assert_within(got[rows, cols], ref, w.K, w.in_dtype, w.out_dtype, name)


@pytest.mark.parametrize("name", list(inputs.WORKLOADS))
def test_workload_integers_bit_exact(name):
    w = inputs.WORKLOADS[name]
    note(f"workload {name} integer inputs")
    a, b = inputs.integer_operands(w.M, w.N, w.K, w.in_dtype, seed=3, b_colmajor=w.b_colmajor)
    c = run(a, b, w.out_dtype)
    if w.M * w.N * w.K <= 1e11:
        want = oracle.encode(ref_full(a, b, w.in_dtype), w.out_dtype)
        assert_bits_equal(out_bits(c, w.out_dtype), want, name)
    else:
        rows, cols = sample_indices(w.M, w.N, 4000, seed=2)
        ref = oracle.gemm_entries(inputs.bits(a, w.in_dtype), inputs.bits(b, w.in_dtype), w.in_dtype, rows, cols)
        got = out_bits(c, w.out_dtype)[rows, cols]
        assert_bits_equal(got, oracle.encode(ref, w.out_dtype), name)


@pytest.mark.parametrize("name", list(inputs.WORKLOADS))
def test_workload_identity_bit_exact(name):
    """A @ E = A[:, :N] exactly (E[k, j] = [k == j]): pins layout and masks."""
    w = inputs.WORKLOADS[name]
    note(f"workload {name} identity")
    a, _ = inputs.make(w)
    e = torch.eye(w.K, w.N, dtype=TD[w.in_dtype])
    if w.b_colmajor:
        e = e.t().contiguous().t()
    c = run(a, e, w.out_dtype)
    want = torch.zeros(w.M, w.N, dtype=torch.float64)
    n = min(w.N, w.K)
    want[:, :n] = a[:, :n].double()
    want_bits = oracle.encode(want.numpy(), w.out_dtype)
    assert_bits_equal(out_bits(c, w.out_dtype), want_bits, name)


# ---- exhaustive tiny shapes --------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_tiny_shapes_exact(dtype):
    note(f"tiny shapes 1..8 {dtype}")
    for M, N, K in itertools.product(range(1, 9), repeat=3):
        a, b = inputs.integer_operands(M, N, K, dtype, seed=M * 64 + N * 8 + K)
        check_exact(a, b, dtype, "f32", what=f"{dtype} {M}x{N}x{K}")


# around tile multiples; the multiples of 8 keep the 16-byte vector paths, the rest
# take the element-load path
RAGGED = [1, 8, 15, 16, 17, 24, 31, 33, 40, 63, 64, 65, 72, 127, 129, 136, 200, 255, 257, 264, 300, 520]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("layout", ["nn", "nt", "tn", "tt"])
def test_ragged_sweep(dtype, layout):
    rng = np.random.default_rng(zlib.crc32(f"{dtype}{layout}".encode()))
    note(f"ragged sweep {dtype} {layout}")
    for t in range(40):
        M, N, K = (int(x) for x in rng.choice(RAGGED, 3))
        a, b = inputs.random_operands(M, N, K, dtype, seed=t, dist=("normal", 1.0),
                                      a_colmajor=layout[0] == "t", b_colmajor=layout[1] == "t")
        out = ["f32", "f16", "bf16"][t % 3]
        check_random(a, b, dtype, out, what=f"{dtype} {layout} {M}x{N}x{K}->{out}")


# ---- every candidate kernel ---------------------------------------------------------

@pytest.mark.parametrize("in_dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("layout", ["nn", "nt", "tn", "tt", "misaligned"])
def test_every_candidate_bit_exact(in_dtype, layout):
    # multiples of 8 that are not multiples of any tile: vector loads with
    # M/N edges and a K tail
    M, N, K = 296, 200, 152
    note(f"all candidates {in_dtype} {layout}")
    if layout == "misaligned":
        # leading dimensions that are not multiples of 8 elements and base
        # addresses off 16-byte alignment: views into larger device buffers
        big_a, big_b = inputs.integer_operands(M, N + 3, K + 5, in_dtype, seed=21)
        a, b = big_a[:, 1:K + 1], big_b[:K, 2:N + 2]
        a_dev, b_dev = big_a.to(DEV)[:, 1:K + 1], big_b.to(DEV)[:K, 2:N + 2]
    else:
        a, b = inputs.integer_operands(M, N, K, in_dtype, seed=22, a_colmajor=layout[0] == "t",
                                       b_colmajor=layout[1] == "t")
        a_dev, b_dev = inputs.to_device_like(a, DEV), inputs.to_device_like(b, DEV)
    for out in ("f32", "bf16"):
        want = oracle.encode(ref_full(a, b, in_dtype), out)
        for cfg in dg.candidates(CODE[in_dtype], CODE[out]):
            c = dg.gemm_config(a_dev, b_dev, cfg, out_dtype=TD[out])
            torch.cuda.synchronize()
            assert_bits_equal(out_bits(c, out), want, f"{cfg} {layout} -> {out}")


# ---- dtype pairs, strides, guard bands --------------------------------------------

@pytest.mark.parametrize("in_dtype,out_dtype", list(itertools.product(["f32", "f16", "bf16"], repeat=2)))
def test_dtype_pairs(in_dtype, out_dtype):
    a, b = inputs.random_operands(133, 77, 90, in_dtype, seed=31, dist=("normal", 1.0))
    check_random(a, b, in_dtype, out_dtype, what=f"{in_dtype}->{out_dtype}")


@pytest.mark.parametrize("in_dtype", ["f32", "bf16", "f16"])
def test_guard_bands_and_strided_c(in_dtype):
    """NaN outside the A/B views is never read; C padding is never written."""
    M, N, K = 130, 90, 70
    dt = TD[in_dtype]
    a_big = torch.full((M + 4, K + 9), float("nan"), dtype=dt)
    b_big = torch.full((K + 6, N + 11), float("nan"), dtype=dt)
    a_v, b_v = inputs.random_operands(M, N, K, in_dtype, seed=41, dist=("normal", 1.0))
    a_big[2:2 + M, 3:3 + K] = a_v
    b_big[1:1 + K, 5:5 + N] = b_v
    a_dev, b_dev = a_big.to(DEV), b_big.to(DEV)
    a = a_dev[2:2 + M, 3:3 + K]
    b = b_dev[1:1 + K, 5:5 + N]
    canary = -12345.0
    c_big = torch.full((M + 3, N + 7), canary, dtype=torch.float32, device=DEV)
    c = c_big[1:1 + M, 2:2 + N]
    dg.gemm(a, b, out=c)
    torch.cuda.synchronize()
    ref = ref_full(a_v, b_v, in_dtype)
    assert_within(to_f64(c), ref, K, in_dtype, "f32", "guard bands")
    full = c_big.cpu()
    mask = torch.ones_like(full, dtype=torch.bool)
    mask[1:1 + M, 2:2 + N] = False
    assert torch.all(full[mask] == canary), "wrote outside C's view"


@pytest.mark.parametrize("c_case", ["rows_aligned", "base_off", "stride_off"])
def test_c_row_vector_stores(c_case):
    """C as a view into a padded buffer: base and row stride 4-element aligned,
    base off by two elements, row stride off by two elements. Every candidate
    kernel and output dtype writes the view bit-exactly and nothing outside it
    (interior and edge tiles, every store width)."""
    M, N, K = 520, 584, 136  # several 256- and 64-wide interior tiles plus ragged edges
    width, col = {"rows_aligned": (N + 12, 4), "base_off": (N + 12, 2), "stride_off": (N + 10, 4)}[c_case]
    note(f"C row stores {c_case}: {M}x{N}x{K}, row stride {width}, column origin {col}")
    a, b = inputs.integer_operands(M, N, K, "bf16", seed=61)
    a_dev, b_dev = a.to(DEV), b.to(DEV)
    for out in ("bf16", "f16", "f32"):
        want = oracle.encode(ref_full(a, b, "bf16"), out)
        for cfg in dg.candidates(dg.DG_BF16, CODE[out]):
            c_big = torch.full((M + 2, width), float("nan"), dtype=TD[out], device=DEV)
            c = c_big[1:1 + M, col:col + N]
            dg.gemm_config(a_dev, b_dev, cfg, out=c, out_dtype=TD[out])
            torch.cuda.synchronize()
            assert_bits_equal(out_bits(c, out), want, f"{cfg} {c_case} -> {out}")
            outside = torch.ones(M + 2, width, dtype=torch.bool)
            outside[1:1 + M, col:col + N] = False
            assert torch.isnan(c_big.float().cpu()[outside]).all(), f"{cfg} {c_case} -> {out}: wrote outside C"


def test_transposed_c_and_transpose_identity():
    a, b = inputs.integer_operands(96, 160, 200, "bf16", seed=51)
    a_d, b_d = a.to(DEV), b.to(DEV)
    c = dg.gemm(a_d, b_d, out_dtype=torch.float32)
    # (A @ B)^T = B^T @ A^T, written into a column-major output view
    ct_store = torch.empty((96, 160), dtype=torch.float32, device=DEV)
    dg.gemm(b_d.t(), a_d.t(), out=ct_store.t())
    torch.cuda.synchronize()
    assert torch.equal(c.cpu(), ct_store.cpu())


def test_k_zero_writes_zeros_and_empty_is_noop():
    a = torch.empty((5, 0), dtype=torch.bfloat16, device=DEV)
    b = torch.empty((0, 7), dtype=torch.bfloat16, device=DEV)
    c = torch.full((5, 7), 3.0, dtype=torch.float32, device=DEV)
    dg.gemm(a, b, out=c)
    torch.cuda.synchronize()
    assert torch.all(c.cpu() == 0.0)
    a0 = torch.empty((0, 4), dtype=torch.bfloat16, device=DEV)
    b0 = torch.ones((4, 7), dtype=torch.bfloat16, device=DEV)
    c0 = torch.empty((0, 7), dtype=torch.float32, device=DEV)
    dg.gemm(a0, b0, out=c0)
    torch.cuda.synchronize()


def test_fp32_accumulation():
    """ones(1,4096) @ ones(4096,1) in fp16 is exactly 4096 (an fp16 sum stalls at 2048)."""
    a = torch.ones((1, 4096), dtype=torch.float16, device=DEV)
    b = torch.ones((4096, 1), dtype=torch.float16, device=DEV)
    c = dg.gemm(a, b, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert c.item() == 4096.0


def test_broadcast_stride_zero():
    row = torch.randn(1, 64).to(torch.bfloat16)
    a_cpu = row.expand(33, 64)          # stride (0, 1)
    b_cpu = torch.randn(64, 40).to(torch.bfloat16)
    a = row.to(DEV).expand(33, 64)
    c = dg.gemm(a, b_cpu.to(DEV), out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.gemm(inputs.bits(a_cpu, "bf16"), inputs.bits(b_cpu, "bf16"), "bf16")
    assert_within(to_f64(c), ref, 64, "bf16", "f32", "broadcast")


def test_invalid_arguments_launch_nothing():
    a = torch.ones((8, 8), dtype=torch.bfloat16, device=DEV)
    b = torch.ones((8, 8), dtype=torch.bfloat16, device=DEV)
    c = torch.full((8, 8), 7.0, dtype=torch.float32, device=DEV)
    bad = dg.Config(256, 256, 16, 8, 4, 2, dg.VARIANT_MFMA, 1)  # no such kernel
    with pytest.raises(dg.DGError) as e:
        dg.gemm_config(a, b, bad, out=c)
    assert e.value.status == 3
    torch.cuda.synchronize()
    assert torch.all(c.cpu() == 7.0)


@pytest.mark.parametrize("in_dtype", ["f16", "bf16"])
def test_no_unit_stride_operands(in_dtype):
    """Views with no unit stride on either axis take the element-load path."""
    M, N, K = 150, 90, 70
    big_a, big_b = inputs.integer_operands(2 * M, 2 * N, 2 * K, in_dtype, seed=61)
    a_cpu, b_cpu = big_a[::2, ::2], big_b[::2, ::2]          # strides (2*2K, 2), (2*2N, 2)
    a = big_a.to(DEV)[::2, ::2]
    b = big_b.to(DEV)[::2, ::2]
    for out in ("f32", "bf16"):
        want = oracle.encode(ref_full(a_cpu, b_cpu, in_dtype), out)
        c = dg.gemm(a, b, out_dtype=TD[out])
        torch.cuda.synchronize()
        assert_bits_equal(out_bits(c, out), want, f"strided {in_dtype} -> {out}")


def test_operands_beyond_31_bit_offsets():
    """Maximum sizes: a row-major B of 2 GiB (32768 x 32768 bf16), whose byte
    offsets no longer fit the direct loads' 31 bits, then the same matrix as a
    2 GiB row-major A with a small B. Sampled output columns / rows against
    the oracle, bit-exact on integer data (|C| <= 2 * 2 * K < 2^24)."""
    K = 32768
    g = torch.Generator().manual_seed(71)
    # B[k, j] = ((7k + 13j) mod 5) - 2, written on the device in row chunks.
    big = torch.empty((K, K), dtype=torch.bfloat16, device=DEV)
    cols = torch.arange(K, device=DEV, dtype=torch.int64)
    for k0 in range(0, K, 1024):
        ks = torch.arange(k0, k0 + 1024, device=DEV, dtype=torch.int64)[:, None]
        big[k0:k0 + 1024] = ((7 * ks + 13 * cols[None, :]) % 5 - 2).to(torch.bfloat16)
    small = torch.randint(-2, 3, (64, K), generator=g).to(torch.bfloat16)
    pick = [0, 1, 4095, 4096, 12345, 32766, 32767]

    note("A[64, 32768] @ B[32768, 32768] (B 2 GiB)")
    c = dg.gemm(small.to(DEV), big, out_dtype=torch.float32)
    torch.cuda.synchronize()
    b_cols = big[:, pick].cpu()
    want = oracle.encode(ref_full(small, b_cols, "bf16"), "f32")
    assert_bits_equal(out_bits(c[:, pick].contiguous(), "f32"), want, "2 GiB B, sampled columns")

    note("A[32768, 32768] @ B[32768, 64] (A 2 GiB)")
    c2 = dg.gemm(big, small.t().contiguous().to(DEV), out_dtype=torch.float32)
    torch.cuda.synchronize()
    a_rows = big[pick, :].cpu()
    want2 = oracle.encode(ref_full(a_rows, small.t().contiguous(), "bf16"), "f32")
    assert_bits_equal(out_bits(c2[pick, :].contiguous(), "f32"), want2, "2 GiB A, sampled rows")
    del big
