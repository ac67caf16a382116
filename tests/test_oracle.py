"""Pins for the CPU oracle: it is checked against things other than itself.

- the pages' worked examples (tests/golden, each file names its page/section);
- exact brute force over rationals on tiny shapes (independent decoding);
- closed forms (identity, permutation, all-ones) and invariants
  (transpose, zero padding of K, linearity, K-split);
- library codecs (numpy float16/float32, torch bfloat16) for the bit decoding
  and the round-to-nearest-even encoding.
A plausible slip in the oracle (a dropped term, a sign, a swapped index or
operand, a wrong stride) fails at least one of these.
"""
import itertools
import math
import random
from fractions import Fraction

import numpy as np
import pytest
import torch

from conftest import load_golden
from dense_gemm_07_amd import inputs
from oracle import brute

DTYPES = ["f32", "f16", "bf16"]


def as_bits(values, dtype):
    """Integer-valued nested list -> bit array of `dtype` (values are exact)."""
    t = torch.tensor(values, dtype=torch.float64).to(inputs.TORCH_DTYPES[dtype])
    return inputs.bits(t, dtype)


# ---- decoding ---------------------------------------------------------------

def test_decode_f16_every_pattern(oracle_mod):
    pats = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = oracle_mod.decode(pats, "f16")
    want = pats.view(np.float16).astype(np.float64)
    assert np.array_equal(got, want, equal_nan=True)
    assert np.array_equal(np.signbit(got), np.signbit(want))


def test_decode_bf16_every_pattern(oracle_mod):
    pats = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = oracle_mod.decode(pats, "bf16")
    want = torch.from_numpy(pats.view(np.int16)).view(torch.bfloat16).double().numpy()
    assert np.array_equal(got, want, equal_nan=True)
    assert np.array_equal(np.signbit(got), np.signbit(want))


def test_decode_f32_patterns(oracle_mod):
    rng = np.random.default_rng(1)
    pats = rng.integers(0, 1 << 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    special = np.array([0, 0x80000000, 1, 0x007FFFFF, 0x00800000, 0x7F7FFFFF,
                        0x7F800000, 0xFF800000, 0x7FC00000, 0x3F800000], dtype=np.uint32)
    pats = np.concatenate([pats, special])
    got = oracle_mod.decode(pats, "f32")
    want = pats.view(np.float32).astype(np.float64)
    assert np.array_equal(got, want, equal_nan=True)


# ---- encoding (round to nearest, ties to even) ------------------------------

def _probe_values(rng, n):
    mags = [rng.uniform(-1, 1, n) * 10.0 ** rng.uniform(-9, 6, n)]
    return np.concatenate(mags + [np.array([0.0, -0.0, 1.0, -2.5, 65504.0, 65519.9, 65520.0,
                                             1e-8, 6e-8, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26,
                                             np.inf, -np.inf])])


def test_encode_f16_matches_numpy(oracle_mod):
    rng = np.random.default_rng(2)
    v = _probe_values(rng, 100_000)
    got = oracle_mod.encode(v, "f16")
    want = v.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, want)


def test_encode_f16_every_midpoint(oracle_mod):
    # Midpoints between consecutive finite positive halves are the tie cases.
    pats = np.arange(0, 0x7BFF, dtype=np.uint16)
    lo = pats.view(np.float16).astype(np.float64)
    hi = (pats + 1).view(np.float16).astype(np.float64)
    mid = (lo + hi) / 2
    got = oracle_mod.encode(mid, "f16")
    even = np.where(pats % 2 == 0, pats, pats + 1).astype(np.uint16)
    assert np.array_equal(got, even)


def test_encode_f32_matches_numpy(oracle_mod):
    rng = np.random.default_rng(3)
    v = np.concatenate([_probe_values(rng, 100_000),
                        rng.uniform(-1, 1, 10_000) * 1e-40, np.array([3.5e38, 3.4028235677973366e38])])
    got = oracle_mod.encode(v, "f32")
    want = v.astype(np.float32).view(np.uint32)
    assert np.array_equal(got, want)


def test_encode_bf16_matches_torch_on_float32_values(oracle_mod):
    rng = np.random.default_rng(4)
    v = rng.standard_normal(100_000).astype(np.float32) * np.float32(10.0) ** rng.integers(-30, 30, 100_000).astype(np.float32)
    v = v[np.isfinite(v)]
    got = oracle_mod.encode(v.astype(np.float64), "bf16")
    want = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want)


def test_encode_bf16_hand_ties(oracle_mod):
    cases = {
        1.0 + 2.0 ** -8: 0x3F80,      # halfway 1.0 / 1+2^-7 -> even (1.0)
        1.0 + 3 * 2.0 ** -8: 0x3F82,  # halfway 1+2^-7 / 1+2^-6 -> even
        257.0: 0x4380,                # 256 | 258 -> 256
        259.0: 0x4382,                # 258 | 260 -> 260
        -259.0: 0xC382,
        (2 - 2.0 ** -8) * 2.0 ** 127: 0x7F80,  # halfway to overflow -> inf
        (2 - 2.0 ** -7) * 2.0 ** 127: 0x7F7F,  # largest finite
        2.0 ** -133: 0x0001,          # smallest subnormal
        2.0 ** -134: 0x0000,          # tie with zero -> even (zero)
        3 * 2.0 ** -134: 0x0002,      # tie 1|2 subnormal quanta -> 2
    }
    got = oracle_mod.encode(np.array(list(cases)), "bf16")
    assert [int(x) for x in got] == list(cases.values())


# ---- the pages' worked examples ---------------------------------------------

@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("fixture", ["p4_s3_1_product_2x2.txt", "p4_s3_2_product_4x4.txt", "hand_3x3.txt"])
def test_worked_products(oracle_mod, fixture, dtype):
    g = load_golden(fixture)
    c = oracle_mod.gemm(as_bits(g["A"], dtype), as_bits(g["B"], dtype), dtype)
    assert c.tolist() == [[float(x) for x in row] for row in g["C"]]
    # the exact brute force agrees too
    a = [[Fraction(x) for x in row] for row in g["A"]]
    b = [[Fraction(x) for x in row] for row in g["B"]]
    assert brute.matmul(a, b) == [[Fraction(x) for x in row] for row in g["C"]]


def test_tile_and_k_split(oracle_mod):
    g4 = load_golden("p4_s3_2_product_4x4.txt")
    ks = load_golden("p4_s3_3_k_split.txt")
    A = as_bits(g4["A"], "f32")
    B = as_bits(g4["B"], "f32")
    # tile (0, 0) read through strided sub-views of the full operands
    tile = oracle_mod.gemm(A[0:2, :], B[:, 0:2], "f32")
    assert tile.tolist() == [[float(x) for x in r] for r in g4["TILE00"]]
    r1 = oracle_mod.gemm(A[0:2, 0:2], B[0:2, 0:2], "f32")
    r2 = oracle_mod.gemm(A[0:2, 2:4], B[2:4, 0:2], "f32")
    assert r1.tolist() == [[float(x) for x in r] for r in ks["ROUND1"]]
    assert r2.tolist() == [[float(x) for x in r] for r in ks["ROUND2"]]
    assert (r1 + r2).tolist() == [[float(x) for x in r] for r in ks["ACC"]]


def test_addressing_examples(oracle_mod):
    g = load_golden("p4_s4_1_addressing.txt")
    flat = as_bits(g["AFLAT"], "f32").reshape(-1)
    A = flat.reshape(4, 4)  # row-major, element strides (4, 1)
    i, j, v = g["POINT"][0]
    assert A.strides[0] // A.itemsize == 4 and A.strides[1] // A.itemsize == 1
    assert i * 4 + j == g["OFFSET"][0][0]
    eye = as_bits(np.eye(4).tolist(), "f32")
    # A @ I read entry by entry picks A[1, 2] = 7
    assert oracle_mod.gemm_entries(A, eye, "f32", np.array([i]), np.array([j]))[0] == v
    # Program (1, 0), round 1: rows [2, 3], ks [0, 1]
    rows, ks_ = np.array([2, 3]), np.array([0, 1])
    offs = rows[:, None] * 4 + ks_[None, :]
    assert offs.tolist() == g["SUBOFFSETS"]
    sub = oracle_mod.gemm(A[2:4, 0:2], eye[0:2, 0:2], "f32")
    assert sub.tolist() == [[float(x) for x in r] for r in g["SUBVALUES"]]


# ---- exact brute force on tiny shapes ---------------------------------------

@pytest.mark.parametrize("dtype", DTYPES)
def test_brute_force_tiny_random(oracle_mod, dtype):
    rng = random.Random(5)
    for M, N, K in itertools.product(range(1, 6), repeat=3):
        a_t, b_t = inputs.random_operands(M, N, K, dtype, seed=rng.randrange(1 << 30),
                                          dist=("normal", 1.0), b_colmajor=bool(rng.getrandbits(1)))
        A, B = inputs.bits(a_t, dtype), inputs.bits(b_t, dtype)
        got = oracle_mod.gemm(A, B, dtype)
        fa = [[brute.value(int(A[i, k]), dtype) for k in range(K)] for i in range(M)]
        fb = [[brute.value(int(B[k, j]), dtype) for j in range(N)] for k in range(K)]
        exact = brute.matmul(fa, fb)
        for i in range(M):
            for j in range(N):
                bound = (K - 1) * 2.0 ** -53 * float(sum(abs(fa[i][k] * fb[k][j]) for k in range(K)))
                assert abs(Fraction(got[i, j]) - exact[i][j]) <= Fraction(bound), (M, N, K, i, j)


@pytest.mark.parametrize("dtype", DTYPES)
def test_brute_force_tiny_integers(oracle_mod, dtype):
    for M, N, K in itertools.product(range(1, 8), repeat=3):
        a_t, b_t = inputs.integer_operands(M, N, K, dtype, seed=M * 100 + N * 10 + K)
        A, B = inputs.bits(a_t, dtype), inputs.bits(b_t, dtype)
        got = oracle_mod.gemm(A, B, dtype)
        exact = brute.matmul([[int(x) for x in r] for r in a_t.double().tolist()],
                             [[int(x) for x in r] for r in b_t.double().tolist()])
        assert got.tolist() == [[float(x) for x in r] for r in exact]


# ---- closed forms -------------------------------------------------------------

@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("M,N,K", [(7, 5, 9), (33, 40, 17), (64, 3, 64)])
def test_identity_both_sides(oracle_mod, dtype, M, N, K):
    a_t, b_t = inputs.random_operands(M, N, K, dtype, seed=6, dist=("normal", 3.0))
    A, B = inputs.bits(a_t, dtype), inputs.bits(b_t, dtype)
    a_val = oracle_mod.decode(np.ascontiguousarray(A), dtype)
    b_val = oracle_mod.decode(np.ascontiguousarray(B), dtype)
    E_kn = as_bits(np.eye(K, N).tolist(), dtype)   # E[k, j] = [k == j]
    E_mk = as_bits(np.eye(M, K).tolist(), dtype)
    want_a = np.zeros((M, N))
    want_a[:, :min(N, K)] = a_val[:, :min(N, K)]
    assert np.array_equal(oracle_mod.gemm(A, E_kn, dtype), want_a)
    want_b = np.zeros((M, N))
    want_b[:min(M, K), :] = b_val[:min(M, K), :]
    assert np.array_equal(oracle_mod.gemm(E_mk, B, dtype), want_b)


@pytest.mark.parametrize("dtype", DTYPES)
def test_permutation_permutes_columns(oracle_mod, dtype):
    K = N = 23
    a_t, _ = inputs.random_operands(11, N, K, dtype, seed=7)
    A = inputs.bits(a_t, dtype)
    perm = np.random.default_rng(7).permutation(N)
    P = np.zeros((K, N))
    P[perm, np.arange(N)] = 1.0      # column j of A @ P is column perm[j] of A
    got = oracle_mod.gemm(A, as_bits(P.tolist(), dtype), dtype)
    a_val = oracle_mod.decode(np.ascontiguousarray(A), dtype)
    assert np.array_equal(got, a_val[:, perm])


def test_all_ones_and_fp32_accumulation(oracle_mod):
    ones_a = inputs.bits(torch.ones(1, 4096, dtype=torch.float16), "f16")
    ones_b = inputs.bits(torch.ones(4096, 1, dtype=torch.float16), "f16")
    assert oracle_mod.gemm(ones_a, ones_b, "f16")[0, 0] == 4096.0
    a = inputs.bits(torch.ones(5, 300, dtype=torch.bfloat16), "bf16")
    b = inputs.bits(torch.ones(300, 7, dtype=torch.bfloat16), "bf16")
    c = oracle_mod.gemm(a, b, "bf16")
    assert np.all(c == 300.0)
    # 300 is not a bf16 value: it rounds to 300 -> 0x4396 (exact: 300 = 1.171875 * 256)
    assert int(oracle_mod.encode(np.array([300.0]), "bf16")[0]) == 0x4396


def test_k_zero_is_empty_sum(oracle_mod):
    A = np.zeros((3, 0), dtype=np.uint16)
    B = np.zeros((0, 4), dtype=np.uint16)
    c = oracle_mod.gemm(A, B, "bf16")
    assert c.shape == (3, 4) and np.all(c == 0.0) and not np.any(np.signbit(c))


# ---- invariants ---------------------------------------------------------------

@pytest.mark.parametrize("dtype", DTYPES)
def test_transpose_identity_bit_exact(oracle_mod, dtype):
    a_t, b_t = inputs.random_operands(37, 29, 51, dtype, seed=8, dist=("normal", 1.0))
    A, B = inputs.bits(a_t, dtype), inputs.bits(b_t, dtype)
    c = oracle_mod.gemm(A, B, dtype)
    # (A @ B)^T = B^T @ A^T, operands passed as transposed (strided) views:
    # the same exact products in the same k order, so bit-identical.
    ct = oracle_mod.gemm(B.T, A.T, dtype)
    assert np.array_equal(c.T, ct)


@pytest.mark.parametrize("dtype", DTYPES)
def test_zero_padding_k_changes_nothing(oracle_mod, dtype):
    a_t, b_t = inputs.random_operands(19, 21, 13, dtype, seed=9, dist=("normal", 1.0))
    c = oracle_mod.gemm(inputs.bits(a_t, dtype), inputs.bits(b_t, dtype), dtype)
    a_pad = torch.cat([a_t, torch.zeros(19, 11, dtype=a_t.dtype)], dim=1)
    b_pad = torch.cat([b_t, torch.zeros(11, 21, dtype=b_t.dtype)], dim=0)
    c_pad = oracle_mod.gemm(inputs.bits(a_pad, dtype), inputs.bits(b_pad, dtype), dtype)
    assert np.array_equal(c, c_pad)


@pytest.mark.parametrize("dtype", DTYPES)
def test_linearity_on_integers(oracle_mod, dtype):
    a_t, b1 = inputs.integer_operands(17, 12, 40, dtype, seed=10)
    _, b2 = inputs.integer_operands(17, 12, 40, dtype, seed=11)
    A = inputs.bits(a_t, dtype)
    lhs = oracle_mod.gemm(A, inputs.bits((b1.double() + b2.double()).to(b1.dtype), dtype), dtype)
    rhs = oracle_mod.gemm(A, inputs.bits(b1, dtype), dtype) + oracle_mod.gemm(A, inputs.bits(b2, dtype), dtype)
    assert np.array_equal(lhs, rhs)


def test_blockwise_sum_equals_plain_sum_on_integers(oracle_mod):
    # "I Wrote a GPU Matmul Kernel From Scratch in Triton", Step 2: the
    # six-loop blockwise product (edges clipped) adds the same M*N*K products.
    a_t, b_t = inputs.integer_operands(10, 9, 11, "f32", seed=12)
    a = [[int(x) for x in r] for r in a_t.tolist()]
    b = [[int(x) for x in r] for r in b_t.tolist()]
    M, K, N, bs = 10, 11, 9, 4
    c = [[0] * N for _ in range(M)]
    for i in range(0, M, bs):
        for j in range(0, N, bs):
            for k in range(0, K, bs):
                for ii in range(i, min(i + bs, M)):
                    for jj in range(j, min(j + bs, N)):
                        c[ii][jj] += sum(a[ii][kk] * b[kk][jj] for kk in range(k, min(k + bs, K)))
    got = oracle_mod.gemm(inputs.bits(a_t, "f32"), inputs.bits(b_t, "f32"), "f32")
    assert got.tolist() == [[float(x) for x in r] for r in c]


def test_entries_and_rows_agree_with_full(oracle_mod):
    a_t, b_t = inputs.random_operands(40, 30, 70, "bf16", seed=13, b_colmajor=True)
    A, B = inputs.bits(a_t, "bf16"), inputs.bits(b_t, "bf16")
    full = oracle_mod.gemm(A, B, "bf16")
    rows = np.array([0, 39, 17, 5]); cols = np.array([0, 29, 3, 11])
    assert np.array_equal(oracle_mod.gemm_entries(A, B, "bf16", rows, cols), full[rows, cols])
    assert np.array_equal(oracle_mod.gemm_rows(A, B, "bf16", 7, 9), full[7:16])


def test_error_bound_of_fp64_sums(oracle_mod):
    # The oracle's own rounding stays inside K * 2^-53 * sum|products| of the
    # exact value, checked against exact rationals on a moderate problem.
    a_t, b_t = inputs.random_operands(3, 4, 500, "bf16", seed=14, dist=("normal", 1.0))
    A, B = inputs.bits(a_t, "bf16"), inputs.bits(b_t, "bf16")
    got = oracle_mod.gemm(A, B, "bf16")
    fa = [[brute.value(int(A[i, k]), "bf16") for k in range(500)] for i in range(3)]
    fb = [[brute.value(int(B[k, j]), "bf16") for j in range(4)] for k in range(500)]
    exact = brute.matmul(fa, fb)
    for i in range(3):
        for j in range(4):
            s = float(sum(abs(fa[i][k] * fb[k][j]) for k in range(500)))
            assert abs(Fraction(got[i, j]) - exact[i][j]) <= Fraction(500 * 2.0 ** -53 * s)
            assert math.isfinite(got[i, j])


# ---- fused epilogue -----------------------------------------------------------

@pytest.mark.parametrize("dtype", DTYPES)
def test_epilogue_hand_2x2(oracle_mod, dtype):
    g = load_golden("epilogue_2x2_hand.txt")
    a, b, r = as_bits(g["A"], dtype), as_bits(g["B"], dtype), as_bits(g["R"], dtype)
    bias = as_bits(g["BIAS"][0], dtype)
    alpha, beta = g["ALPHA"][0][0], g["BETA"][0][0]
    for per_row, tag in ((False, "COL"), (True, "ROW")):
        for act in ("none", "relu"):
            got = oracle_mod.gemm_ex(a, b, dtype, alpha=alpha, beta=beta, r_bits=r, r_dtype=dtype,
                                     bias_bits=bias, bias_dtype=dtype, per_row=per_row, act=act)
            assert got.tolist() == g[f"{tag}_{act.upper()}"], (tag, act)


# Standard normal CDF values from printed tables (Phi(x) to 16 digits).
PHI_TABLE = {
    -3.0: 0.0013498980316300946,
    -1.5: 0.0668072012688581,
    -1.0: 0.15865525393145707,
    0.5: 0.6914624612740131,
    1.0: 0.8413447460685429,
    2.0: 0.9772498680518208,
}


def test_gelu_matches_normal_cdf_table(oracle_mod):
    xs = np.array([list(PHI_TABLE)], dtype=np.float64)
    got = oracle_mod.epilogue(xs, act="gelu")[0]
    want = np.array([x * phi for x, phi in PHI_TABLE.items()])
    assert np.allclose(got, want, rtol=1e-14, atol=0)
    # GELU(0) = 0 and GELU(x) - GELU(-x) = x (since Phi(x) + Phi(-x) = 1)
    assert oracle_mod.epilogue(np.zeros((1, 1)), act="gelu")[0, 0] == 0.0
    x = np.linspace(-6, 6, 97).reshape(1, -1)
    g = oracle_mod.epilogue(x, act="gelu")
    gm = oracle_mod.epilogue(-x, act="gelu")
    assert np.allclose(g - gm, x, rtol=0, atol=1e-14)


def test_relu_special_values(oracle_mod):
    x = np.array([[-1.0, -0.0, 0.0, 2.5, np.nan, -np.inf, np.inf]])
    got = oracle_mod.epilogue(x, act="relu")[0]
    assert got[0] == 0.0 and not np.signbit(got[0])
    assert got[1] == 0.0 and np.signbit(got[1])  # -0 is not < 0: kept
    assert got[2] == 0.0 and got[3] == 2.5
    assert np.isnan(got[4]) and got[5] == 0.0 and got[6] == np.inf


def test_epilogue_beta_zero_never_reads_residual(oracle_mod):
    p = np.arange(6, dtype=np.float64).reshape(2, 3)
    r = np.full((2, 3), np.nan, dtype=np.float32).view(np.uint32)
    got = oracle_mod.epilogue(p, alpha=1.0, beta=0.0, r_bits=r, r_dtype="f32")
    assert np.array_equal(got, p)
    with_beta = oracle_mod.epilogue(p, alpha=1.0, beta=1.0, r_bits=r, r_dtype="f32")
    assert np.isnan(with_beta).all()


def test_epilogue_defaults_are_the_product(oracle_mod):
    a, b = inputs.random_operands(7, 9, 11, "bf16", seed=5)
    ab, bb = inputs.bits(a, "bf16"), inputs.bits(b, "bf16")
    p = oracle_mod.gemm(ab, bb, "bf16")
    assert np.array_equal(oracle_mod.gemm_ex(ab, bb, "bf16"), p)
    assert np.array_equal(oracle_mod.gemm_ex(ab, bb, "bf16", alpha=-4.0), -4.0 * p)


def test_epilogue_row_bias_is_column_bias_transposed(oracle_mod):
    rng = np.random.default_rng(3)
    p = rng.standard_normal((5, 4))
    bias = inputs.bits(torch.randn(5, generator=torch.Generator().manual_seed(2)).to(torch.float16), "f16")
    r = inputs.bits(torch.randn(5, 4, generator=torch.Generator().manual_seed(4)).to(torch.bfloat16), "bf16")
    rows = oracle_mod.epilogue(p, alpha=0.5, beta=3.0, r_bits=r, r_dtype="bf16", bias_bits=bias,
                               bias_dtype="f16", per_row=True, act="gelu")
    cols = oracle_mod.epilogue(p.T, alpha=0.5, beta=3.0, r_bits=r.T, r_dtype="bf16", bias_bits=bias,
                               bias_dtype="f16", per_row=False, act="gelu")
    assert np.array_equal(rows, cols.T)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_epilogue_brute_force(oracle_mod, dtype):
    """Exact rational arithmetic on tiny shapes: alpha*P + beta*R + bias (then ReLU)."""
    rnd = random.Random(11)
    dt = inputs.TORCH_DTYPES[dtype]
    for trial in range(40):
        M, N, K = rnd.randint(1, 4), rnd.randint(1, 4), rnd.randint(1, 4)
        gen = torch.Generator().manual_seed(100 + trial)
        a, b = torch.randn(M, K, generator=gen).to(dt), torch.randn(K, N, generator=gen).to(dt)
        r = torch.randn(M, N, generator=gen).to(dt)
        per_row = trial % 2 == 1
        bias = torch.randn(M if per_row else N, generator=gen).to(dt)
        alpha = rnd.choice([1.0, -0.5, 3.0, 0.1])
        beta = rnd.choice([0.0, 1.0, -2.0, 0.3])
        act = "relu" if trial % 3 == 0 else "none"
        ab, bb, rb, biasb = (inputs.bits(t, dtype) for t in (a, b, r, bias))
        got = oracle_mod.gemm_ex(ab, bb, dtype, alpha=alpha, beta=beta, r_bits=rb, r_dtype=dtype,
                                 bias_bits=biasb, bias_dtype=dtype, per_row=per_row, act=act)
        fa_ = [[brute.value(int(x), dtype) for x in row] for row in ab]
        fb_ = [[brute.value(int(x), dtype) for x in row] for row in bb]
        p = brute.matmul(fa_, fb_)
        fa, fb = Fraction(float(np.float32(alpha))), Fraction(float(np.float32(beta)))
        for i in range(M):
            for j in range(N):
                rv = brute.value(int(rb[i, j]), dtype)
                v = fa * p[i][j] + fb * rv + brute.value(int(biasb[i if per_row else j]), dtype)
                if act == "relu" and v < 0:
                    v = Fraction(0)
                scale = abs(fa * p[i][j]) + abs(fb * rv) + 1
                assert abs(Fraction(float(got[i, j])) - v) <= scale * Fraction(1, 2 ** 50), (trial, i, j)


# ---- attention ------------------------------------------------------------------

def attn_bits(shape, dtype, seed, scale=1.0):
    t = (torch.randn(shape, generator=torch.Generator().manual_seed(seed)) * scale).to(inputs.TORCH_DTYPES[dtype])
    return t, inputs.bits(t, dtype)


@pytest.mark.parametrize("causal", [False, True])
def test_attention_zero_queries_average_the_values(oracle_mod, causal):
    """Q = 0: every score is 0, so O is the plain mean of the allowed V rows and lse = log(count)."""
    B, H, Sq, Skv, D = 2, 3, 6, 6, 8
    q = np.zeros((B, H, Sq, D), dtype=np.uint16)  # +0 in bf16
    _, kb = attn_bits((B, H, Skv, D), "bf16", 1)
    vt, vb = attn_bits((B, H, Skv, D), "bf16", 2)
    o, lse = oracle_mod.attention(q, kb, vb, "bf16", causal=causal)
    v = vt.double().numpy()
    for i in range(Sq):
        n = i + 1 if causal else Skv
        assert np.allclose(o[:, :, i], v[:, :, :n].mean(axis=2), rtol=0, atol=1e-15)
        assert np.allclose(lse[:, :, i], math.log(n), rtol=0, atol=1e-15)


def test_attention_causal_first_row_and_single_key(oracle_mod):
    _, qb = attn_bits((1, 2, 5, 16), "f16", 3)
    _, kb = attn_bits((1, 2, 5, 16), "f16", 4)
    vt, vb = attn_bits((1, 2, 5, 16), "f16", 5)
    o, lse = oracle_mod.attention(qb, kb, vb, "f16", causal=True)
    assert np.array_equal(o[:, :, 0], vt[:, :, 0].double().numpy())  # one allowed key: weight exactly 1
    # lse of that row is the single score itself
    q0 = oracle_mod.decode(qb[:, :, 0], "f16")
    k0 = oracle_mod.decode(kb[:, :, 0], "f16")
    assert np.allclose(lse[:, :, 0], (q0 * k0).sum(-1) / 4.0, rtol=1e-15, atol=1e-15)
    # seq_kv = 1, no mask: every row is V[0]
    o1, _ = oracle_mod.attention(qb, kb[:, :, :1], vb[:, :, :1], "f16")
    assert np.array_equal(o1, np.broadcast_to(vt[:, :, :1].double().numpy(), o1.shape))


def test_attention_invariances(oracle_mod):
    B, H, Sq, Skv, D = 1, 2, 7, 9, 16
    _, qb = attn_bits((B, H, Sq, D), "bf16", 6)
    kt, _ = attn_bits((B, H, Skv, D), "bf16", 7)
    # column 3 of K holds small integers, so the shift below is exact in bf16
    kt[..., 3] = torch.randint(-4, 5, (B, H, Skv), generator=torch.Generator().manual_seed(12)).to(torch.bfloat16)
    kb = inputs.bits(kt, "bf16")
    vt, vb = attn_bits((B, H, Skv, D), "bf16", 8)
    o, lse = oracle_mod.attention(qb, kb, vb, "bf16")
    # permuting keys together with their values changes nothing (no mask)
    perm = np.random.default_rng(0).permutation(Skv)
    op, lp = oracle_mod.attention(qb, np.ascontiguousarray(kb[:, :, perm]), np.ascontiguousarray(vb[:, :, perm]), "bf16")
    assert np.allclose(op, o, rtol=0, atol=1e-13) and np.allclose(lp, lse, rtol=0, atol=1e-13)
    # adding the same vector u to every key shifts each row's scores by scale*q.u: O unchanged, lse shifted
    u = torch.zeros(D)
    u[3] = 2.0
    k2 = (kt.float() + u).to(torch.bfloat16)
    assert torch.equal(k2.float() - kt.float(), u.expand_as(kt))  # the shift is exact in bf16 here
    o2, l2 = oracle_mod.attention(qb, inputs.bits(k2, "bf16"), vb, "bf16")
    qd = oracle_mod.decode(qb, "bf16")
    assert np.allclose(o2, o, rtol=0, atol=1e-13)
    assert np.allclose(l2 - lse, qd[..., 3] * 2.0 / 4.0, rtol=0, atol=1e-13)
    # linear in V: small integers keep V1 + V2 exact in bf16
    g = torch.Generator().manual_seed(9)
    v1 = torch.randint(-4, 5, (B, H, Skv, D), generator=g).to(torch.bfloat16)
    v2 = torch.randint(-4, 5, (B, H, Skv, D), generator=g).to(torch.bfloat16)
    o1, _ = oracle_mod.attention(qb, kb, inputs.bits(v1, "bf16"), "bf16")
    o2_, _ = oracle_mod.attention(qb, kb, inputs.bits(v2, "bf16"), "bf16")
    o12, _ = oracle_mod.attention(qb, kb, inputs.bits(v1 + v2, "bf16"), "bf16")
    assert np.allclose(o12, o1 + o2_, rtol=0, atol=1e-13)


def test_attention_one_hot_limit_and_large_scores(oracle_mod):
    """A key aligned with the query and scores in the thousands: weight ~1 on it, no overflow."""
    D = 16
    q = torch.zeros(1, 1, 3, D)
    q[0, 0, :, 0] = 64.0
    k = torch.randn(1, 1, 5, D, generator=torch.Generator().manual_seed(10)) * 0.1
    k[0, 0, 2, 0] = 64.0   # score 64*64/4 = 1024 for key 2, the others near 0
    v = torch.randn(1, 1, 5, D, generator=torch.Generator().manual_seed(11))
    qb, kb, vb = (inputs.bits(t.to(torch.float16), "f16") for t in (q, k, v))
    o, lse = oracle_mod.attention(qb, kb, vb, "f16")
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    assert np.allclose(o[0, 0], np.broadcast_to(oracle_mod.decode(vb[0, 0, 2], "f16"), (3, D)), rtol=0, atol=1e-300)
    assert np.allclose(lse[0, 0], 1024.0, rtol=1e-15, atol=0)  # the other keys add exp(-1024) ~ 0


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_attention_hand_worked_softmax_weights(oracle_mod, dtype):
    """Scaled scores (0, 1, 2) against one-hot values: O holds the softmax weights themselves,
    which the fixture gives as hand-derived numbers (logistic at +-1, softmax of (0, 1, 2)).
    Fails for a softmax in another base, a missing or doubled 1/sqrt(head_dim) scale, a
    causal mask off by one, or lse without the row maximum."""
    g = load_golden("attention_softmax_hand.txt")

    def bits(rows):
        t = torch.tensor(rows, dtype=torch.float32).to(inputs.TORCH_DTYPES[dtype])
        return np.ascontiguousarray(inputs.bits(t, dtype).reshape(1, 1, len(rows), -1))

    q, k, v = bits(g["Q"]), bits(g["K"]), bits(g["V"])
    D = q.shape[-1]
    for causal, tag, nk in ((True, "CAUSAL", 3), (False, "FULL", 3), (False, "TWO", 2)):
        o, lse = oracle_mod.attention(q, np.ascontiguousarray(k[:, :, :nk]), np.ascontiguousarray(v[:, :, :nk]),
                                      dtype, causal=causal)
        want_o = np.zeros((3, D))
        want_o[:, :nk] = np.array(g[f"O_{tag}"], dtype=np.float64)
        assert np.allclose(o[0, 0], want_o, rtol=0, atol=2e-16), (tag, o[0, 0, :, :3])
        assert np.allclose(lse[0, 0], np.array(g[f"LSE_{tag}"], dtype=np.float64)[:, 0], rtol=0, atol=5e-16), tag
    # The same weights with the scale given explicitly: K doubled and scale 1/8.
    k2 = bits([[2 * x for x in row] for row in g["K"]])
    o, lse = oracle_mod.attention(q, k2, v, dtype, scale=0.125, causal=True)
    assert np.allclose(o[0, 0, :, :3], np.array(g["O_CAUSAL"], dtype=np.float64), rtol=0, atol=2e-16)
    assert np.allclose(lse[0, 0], np.array(g["LSE_CAUSAL"], dtype=np.float64)[:, 0], rtol=0, atol=5e-16)
