"""GPU parity of dg_gemm_ex: split-K, the fused epilogue, strided batches, autograd.

Every call goes through the C-ABI (ctypes binding) and is compared with the
CPU oracle element by element:
- small-integer inputs: bit-exact (every fp32 intermediate -- partial sums,
  the split-K partial tiles and their sum, alpha*acc, beta*R, bias -- is an
  integer or half-integer below 2^24, so the only rounding is the final one);
- random inputs: helpers.epilogue_tolerance (the product's tolerance, the
  epilogue's fp32 roundings, half an ulp of the output).
Operand layouts cover every load path: row/col-major 16-byte aligned (buffer
loads straight into LDS), misaligned by one element (16-byte register
loads), and a step-2 slice (element loads).
"""
import sys

import numpy as np
import pytest
import torch

import dense_gemm_07_amd as dg
import oracle
from dense_gemm_07_amd import inputs
from helpers import (assert_bits_equal, assert_within_tol, epilogue_tolerance, out_bits, sample_indices, to_f64,
                     ulp)

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


def place(t, layout):
    """Device copy of CPU tensor t (2-D) in a given memory layout."""
    if layout == "row":
        return t.contiguous().to(DEV)
    if layout == "col":
        return t.t().contiguous().to(DEV).t()
    if layout == "mis":  # row-major, base one element past 16-byte alignment
        buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=DEV)
        v = buf[1:].view(t.shape)
        v.copy_(t.to(DEV))
        return v
    if layout == "gap":  # every other column of a wider buffer: the column stride is 2
        buf = torch.zeros(t.shape[0], 2 * t.shape[1], dtype=t.dtype, device=DEV)
        v = buf[:, ::2]
        v.copy_(t.to(DEV))
        return v
    raise ValueError(layout)


def config(in_dtype, bm, bn, bk, stages=2, splits=1, group_m=8, xcd=1):
    for c in dg.candidates(CODE[in_dtype], CODE[in_dtype]):
        if (c.block_m, c.block_n, c.block_k, c.stages) == (bm, bn, bk, stages):
            c.group_m, c.xcd_remap, c.k_splits = group_m, xcd, splits
            return c
    raise LookupError((bm, bn, bk, stages))


def ref_product(a, b, in_dtype):
    return oracle.gemm(inputs.bits(a, in_dtype), inputs.bits(b, in_dtype), in_dtype)


def int_tensor(shape, dtype, seed, lo=-2, hi=2):
    g = torch.Generator().manual_seed(seed)
    return torch.randint(lo, hi + 1, shape, generator=g, dtype=torch.int32).to(TD[dtype])


# ---- split-K --------------------------------------------------------------------

SPLIT_SHAPES = [(200, 136, 1000), (64, 64, 4096), (130, 70, 777), (257, 300, 520), (33, 520, 2056)]
SPLIT_CFGS = [(64, 64, 64, 2), (64, 64, 32, 8), (128, 128, 64, 2), (256, 256, 64, 2), (128, 256, 64, 2)]
LAYOUTS = [("row", "row"), ("row", "col"), ("col", "row"), ("mis", "row"), ("gap", "col")]


@pytest.mark.parametrize("splits", [2, 3, 8])
@pytest.mark.parametrize("shape", SPLIT_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_split_k_integers_bit_exact(shape, splits):
    M, N, K = shape
    a, b = inputs.integer_operands(M, N, K, "bf16", seed=M + N + K + splits)
    want32 = ref_product(a, b, "bf16")
    for out_dtype in ("f32", "bf16"):
        want = oracle.encode(want32, out_dtype)
        for cfg_shape in SPLIT_CFGS:
            cfg = config("bf16", *cfg_shape, splits=splits)
            for la, lb in LAYOUTS:
                what = f"{shape} splits={splits} cfg={cfg_shape} {la}/{lb} -> {out_dtype}"
                note(what)
                if la == "gap" and cfg_shape[:3] == (256, 256, 64):
                    # element-load operands have no 256x256x64 kernel (it would spill)
                    with pytest.raises(dg.DGError) as e:
                        dg.gemm_ex(place(a, la), place(b, lb), out_dtype=TD[out_dtype], config=cfg)
                    assert e.value.status == 3, what
                    continue
                c = dg.gemm_ex(place(a, la), place(b, lb), out_dtype=TD[out_dtype], config=cfg)
                torch.cuda.synchronize()
                assert_bits_equal(out_bits(c, out_dtype), want, what)


def test_split_k_longest_k():
    """K = 2^20 with a 64 x 64 output: one tile, so the library's split (with a
    workspace) is the largest it makes (16 ranges of 65536), and the unsplit
    loop runs 16384 K steps. Sampled columns, bit-exact on integers
    (|C| <= 4K = 2^22 < 2^24)."""
    M, N, K = 64, 64, 1 << 20
    g = torch.Generator().manual_seed(91)
    a = torch.randint(-2, 3, (M, K), generator=g).to(torch.bfloat16)
    b = torch.randint(-2, 3, (K, N), generator=g).to(torch.bfloat16)
    cols = [0, 17, 63]
    want = oracle.encode(ref_product(a, b[:, cols].contiguous(), "bf16"), "f32")
    ad, bd = a.to(DEV), b.to(DEV)
    cfg, _ = dg.select_config_ex(M, N, K, ad.stride(), bd.stride(), (N, 1), CODE["bf16"], CODE["f32"],
                                 workspace_bytes=dg.DEFAULT_WORKSPACE_BYTES)
    assert cfg.k_splits == 16, cfg.k_splits
    for ws in (True, None):
        note(f"K = 2^20, workspace={ws}")
        c = dg.gemm_ex(ad, bd, out_dtype=torch.float32, workspace=ws)
        torch.cuda.synchronize()
        assert_bits_equal(out_bits(c[:, cols].contiguous(), "f32"), want, f"K=2^20 workspace={ws}")


@pytest.mark.parametrize("in_dtype,out_dtype", [("f16", "f16"), ("bf16", "f32"), ("bf16", "bf16")])
def test_split_k_random_within_tolerance(in_dtype, out_dtype):
    for (M, N, K), splits in [((300, 200, 3000), 4), ((96, 1000, 5000), 7), ((1, 700, 4100), 16)]:
        a, b = inputs.random_operands(M, N, K, in_dtype, seed=K)
        ref = ref_product(a, b, in_dtype)
        for cfg_shape in [(64, 64, 64, 4), (128, 128, 64, 2), (256, 256, 32, 3)]:
            for la, lb in [("row", "row"), ("mis", "col")]:
                what = f"{(M, N, K)} splits={splits} {cfg_shape} {la}/{lb} {in_dtype}->{out_dtype}"
                note(what)
                cfg = config(in_dtype, *cfg_shape, splits=splits)
                c = dg.gemm_ex(place(a, la), place(b, lb), out_dtype=TD[out_dtype], config=cfg)
                torch.cuda.synchronize()
                got = to_f64(c)
                tol = epilogue_tolerance(K, in_dtype, out_dtype, got, ref, 1.0, np.abs(ref), "none")
                assert_within_tol(got, ref, tol, what)


def test_split_k_deterministic_and_workspace_needs_no_init():
    M, N, K = 250, 190, 6000
    a, b = inputs.random_operands(M, N, K, "bf16", seed=9)
    ad, bd = place(a, "row"), place(b, "row")
    cfg = config("bf16", 64, 64, 64, stages=4, splits=6)
    total = dg.workspace_size(M, N, K, 1, cfg)
    assert total == 4 * 3 * 6 * 64 * 64 * 4  # 4 x 3 tiles, 6 ranges of 1024
    ws = torch.full((total // 4,), float("nan"), dtype=torch.float32, device=DEV)  # garbage contents
    runs = []
    for rep in range(3):
        note(f"determinism rep {rep}")
        c = dg.gemm_ex(ad, bd, config=cfg, workspace=ws)
        torch.cuda.synchronize()
        runs.append(out_bits(c, "bf16"))
        assert not torch.isnan(ws).any(), "a partial tile was not written"
    assert all(np.array_equal(runs[0], r) for r in runs[1:])
    ref = ref_product(a, b, "bf16")
    got = to_f64(c)
    assert_within_tol(got, ref, epilogue_tolerance(K, "bf16", "bf16", got, ref, 1.0, np.abs(ref), "none"), "split")


@pytest.mark.parametrize("K", [8, 9, 15, 40, 63, 65, 129, 448, 449, 512, 513, 777, 1029])
def test_k_contiguous_unaligned_small_tiles_bit_exact(K):
    """Both operands k-contiguous at leading dimensions that are not multiples
    of 8 and bases off 16-byte alignment: the small tiles' deep pipeline, whose
    every chunk is a 16-byte load clamped into the row (the chunk cut by K is
    read from K - 8 and shifted into place). K spans one slice, the group of
    eight steps, ragged tails, and split-K ranges down to 5 elements
    (K = 1029 cut for 16 ranges: 9 ranges of 128, the last of 5). Integers, bit-exact."""
    M, N = 130, 70
    a, b = inputs.integer_operands(M, N, K, "bf16", seed=K + 7)
    big_a = torch.zeros((M, K + 3), dtype=torch.bfloat16)
    big_a[:, 1:K + 1] = a
    big_b = torch.zeros((N, K + 1), dtype=torch.bfloat16)  # B's storage, one row per column of B
    big_b[:, :K] = b.t()
    a_dev = big_a.to(DEV)[:, 1:K + 1]                       # lda = K + 3, base 2 bytes past alignment
    b_dev = big_b.to(DEV)[:, :K].t()                        # B[k][n] at n * (K + 1) + k
    want32 = ref_product(a, b, "bf16")
    for cfg_shape, splits in [((64, 64, 64, 4), 1), ((64, 64, 32, 8), 1), ((64, 64, 64, 4), 16),
                              ((64, 64, 32, 2), 3)]:
        cfg = config("bf16", *cfg_shape, splits=splits)
        for out_dtype in ("f32", "bf16"):
            what = f"K={K} cfg={cfg_shape} splits={splits} -> {out_dtype}"
            note(what)
            c = dg.gemm_ex(a_dev, b_dev, out_dtype=TD[out_dtype], config=cfg)
            torch.cuda.synchronize()
            assert_bits_equal(out_bits(c, out_dtype), oracle.encode(want32, out_dtype), what)


def _offset_view(t, colmajor, pad):
    """Device view of CPU matrix t [rows, cols]: row-major (or column-major)
    storage whose leading dimension is `pad` elements wider than needed and
    whose base sits one element past a 16-byte boundary."""
    store = t.t() if colmajor else t
    r, c = store.shape
    big = torch.zeros((r, c + pad), dtype=t.dtype)
    big[:, 1:c + 1] = store
    v = big.to(DEV)[:, 1:c + 1]
    return v.t() if colmajor else v


@pytest.mark.parametrize("shape", [(257, 263, 777), (300, 9, 520), (9, 300, 100), (515, 130, 1000)],
                         ids=lambda s: "x".join(map(str, s)))
def test_staged_large_tiles_bit_exact(shape):
    """Contiguous operands off 16-byte alignment staged through registers into
    the direct kernel's LDS formats: large tiles, and 64x64 tiles when an
    operand is row-contiguous (the 64x64 configs run the padded-row register
    kernel when both are k-contiguous). Each operand k-contiguous or
    row-contiguous; edge tiles with fewer than 8 valid rows, K tails that are
    not multiples of 8, products of less than one tile. Integers, bit-exact."""
    M, N, K = shape
    a, b = inputs.integer_operands(M, N, K, "bf16", seed=M + 3 * N + 7 * K)
    want32 = ref_product(a, b, "bf16")
    for a_col in (False, True):
        for b_col in (False, True):
            ad = _offset_view(a, a_col, 3)
            bd = _offset_view(b, b_col, 5)
            for cfg_shape in [(256, 256, 64, 2), (256, 256, 32, 2), (128, 128, 64, 2), (256, 128, 64, 2),
                              (128, 256, 64, 2), (64, 64, 64, 2), (64, 64, 32, 2)]:
                cfg = config("bf16", *cfg_shape)
                for out_dtype in ("f32", "bf16"):
                    what = f"{shape} A {'col' if a_col else 'row'} B {'col' if b_col else 'row'} {cfg_shape} -> {out_dtype}"
                    note(what)
                    c = dg.gemm_ex(ad, bd, out_dtype=TD[out_dtype], config=cfg)
                    torch.cuda.synchronize()
                    assert_bits_equal(out_bits(c, out_dtype), oracle.encode(want32, out_dtype), what)


def test_split_k_workspace_per_stream():
    """The binding's cached workspace is one buffer per (device, stream): split-K
    calls queued on two streams at once write their partial tiles into
    different memory, and both results are exact (integers)."""
    M, N, K = 200, 136, 4096
    cfg = config("bf16", 64, 64, 64, stages=4, splits=8)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()  # default priority
    ops = [inputs.integer_operands(M, N, K, "bf16", seed=s) for s in (31, 32)]
    wants = [oracle.encode(ref_product(a, b, "bf16"), "f32") for a, b in ops]
    dev = [(a.to(DEV), b.to(DEV)) for a, b in ops]
    outs = [torch.empty(M, N, dtype=torch.float32, device=DEV) for _ in ops]
    torch.cuda.synchronize()
    for rep in range(3):
        note(f"two streams, rep {rep}")
        for (ad, bd), c, st in zip(dev, outs, (s1, s2)):
            dg.gemm_ex(ad, bd, out=c, config=cfg, stream=st)
        torch.cuda.synchronize()
        for c, want in zip(outs, wants):
            assert_bits_equal(out_bits(c, "f32"), want, f"stream rep {rep}")
    key = lambda st: (torch.device(DEV).index or 0, st.cuda_stream)
    w1, w2 = dg._workspaces[key(s1)], dg._workspaces[key(s2)]
    assert w1.data_ptr() != w2.data_ptr()


def test_split_k_counts_beyond_k_slices():
    """More splits than K slices: the ranges collapse to the non-empty ones."""
    M, N, K = 70, 90, 100  # two 64-slices
    a, b = inputs.integer_operands(M, N, K, "f16", seed=1)
    want = oracle.encode(ref_product(a, b, "f16"), "f16")
    for splits in (2, 5, 16):
        cfg = config("f16", 64, 64, 64, stages=4, splits=splits)
        assert dg.workspace_size(M, N, K, 1, cfg) == 4 * 2 * 64 * 64 * 4  # 2x2 tiles, 2 ranges
        note(f"K=100 splits={splits}")
        c = dg.gemm_ex(place(a, "row"), place(b, "row"), config=cfg)
        torch.cuda.synchronize()
        assert_bits_equal(out_bits(c, "f16"), want, f"splits={splits}")


def test_split_k_needs_workspace():
    a = torch.zeros(128, 4096, dtype=torch.bfloat16, device=DEV)
    b = torch.zeros(4096, 128, dtype=torch.bfloat16, device=DEV)
    cfg = config("bf16", 128, 128, 64, splits=4)
    with pytest.raises(dg.DGError) as e:
        dg.gemm_ex(a, b, config=cfg, workspace=None)
    assert e.value.status == 1
    small = torch.zeros(1024, dtype=torch.uint8, device=DEV)
    with pytest.raises(dg.DGError):
        dg.gemm_ex(a, b, config=cfg, workspace=small)
    with pytest.raises(dg.DGError):
        dg.gemm_config(a, b, cfg)


def test_default_choice_with_workspace_low_tile_count():
    """cfg == NULL with a workspace: the library may split K; the result must hold either way."""
    for (M, N, K) in [(128, 128, 8192), (16, 14336 // 4, 4096), (1000, 1500, 777)]:
        a, b = inputs.random_operands(M, N, K, "bf16", seed=M)
        ref = ref_product(a, b, "bf16")
        note(f"default choice {(M, N, K)}")
        c = dg.gemm_ex(place(a, "row"), place(b, "row"), out_dtype=torch.float32)
        torch.cuda.synchronize()
        got = to_f64(c)
        tol = epilogue_tolerance(K, "bf16", "f32", got, ref, 1.0, np.abs(ref), "none")
        assert_within_tol(got, ref, tol, f"default {(M, N, K)}")


# ---- fused epilogue ----------------------------------------------------------------

# (in, out, alpha, beta, residual, bias, act)
EPI_CASES = [
    ("bf16", "bf16", 1.0, 0.0, None, "f32col", "relu"),
    ("bf16", "f32", 2.0, 1.0, "inplace", None, "none"),
    ("f16", "f16", -0.5, -2.0, "f32", "f16row", "relu"),
    ("bf16", "f16", 1.0, 1.0, "bf16col", "bf16col", "none"),
    ("f16", "f32", 0.5, 3.0, "inplace", "f32row", "relu"),
    ("f32", "f32", 2.0, -1.0, "f16", "f32col", "relu"),
    ("f32", "bf16", 1.0, 0.0, None, "bf16row", "none"),
    ("bf16", "bf16", 1.0, 0.0, None, None, "relu"),
]


def make_epilogue_inputs(M, N, in_dtype, out_dtype, residual, bias, seed, integers):
    """(device residual or None, CPU residual, device bias, CPU bias, C prior (device or None))."""
    g = torch.Generator().manual_seed(seed)

    def draw(shape, dtype):
        if integers:
            return torch.randint(-8, 9, shape, generator=g, dtype=torch.int32).to(TD[dtype])
        return torch.randn(shape, generator=g).to(TD[dtype])

    r_dev = r_cpu = prior = None
    r_dtype = None
    if residual == "inplace":
        r_cpu, r_dtype = draw((M, N), out_dtype), out_dtype
        prior = r_cpu.to(DEV)
    elif residual is not None:
        col = residual.endswith("col")
        r_dtype = residual[:-3] if col else residual
        r_cpu = draw((M, N), r_dtype)
        r_dev = place(r_cpu, "col" if col else "row")
    b_dev = b_cpu = None
    b_dtype, per_row = None, False
    if bias is not None:
        b_dtype, per_row = bias[:-3], bias.endswith("row")
        b_cpu = draw((M if per_row else N,), b_dtype)
        b_dev = b_cpu.to(DEV)
    return r_dev, r_cpu, r_dtype, b_dev, b_cpu, b_dtype, per_row, prior


def check_epilogue(M, N, K, case, layouts, cfg=None, integers=True, seed=0):
    in_dtype, out_dtype, alpha, beta, residual, bias, act = case
    if integers:
        a, b = inputs.integer_operands(M, N, K, in_dtype, seed=seed)
    else:
        a, b = inputs.random_operands(M, N, K, in_dtype, seed=seed)
    r_dev, r_cpu, r_dtype, b_dev, b_cpu, b_dtype, per_row, prior = make_epilogue_inputs(
        M, N, in_dtype, out_dtype, residual, bias, seed + 1, integers)
    out = prior if prior is not None else torch.full((M, N), float("nan"), dtype=TD[out_dtype], device=DEV)
    what = f"{(M, N, K)} {case} {layouts} cfg={cfg and (cfg.block_m, cfg.block_n, cfg.k_splits)}"
    note(what)
    c = dg.gemm_ex(place(a, layouts[0]), place(b, layouts[1]), out=out, alpha=alpha, beta=beta,
                   residual=r_dev, bias=b_dev, bias_per_row=per_row, activation=act, config=cfg)
    torch.cuda.synchronize()
    p = ref_product(a, b, in_dtype)
    rb = inputs.bits(r_cpu, r_dtype) if r_cpu is not None else None
    bb = inputs.bits(b_cpu, b_dtype) if b_cpu is not None else None
    ref = oracle.epilogue(p, alpha=alpha, beta=beta, r_bits=rb, r_dtype=r_dtype, bias_bits=bb,
                          bias_dtype=b_dtype, per_row=per_row, act=act)
    if integers and act != "gelu":
        assert_bits_equal(out_bits(c, out_dtype), oracle.encode(ref, out_dtype), what)
    else:
        terms = np.abs(alpha * p)
        if rb is not None and beta != 0:
            terms = terms + np.abs(beta * oracle.decode(rb, r_dtype))
        if bb is not None:
            bv = oracle.decode(bb, b_dtype)
            terms = terms + np.abs(bv[:, None] if per_row else bv[None, :])
        got = to_f64(c)
        assert_within_tol(got, ref, epilogue_tolerance(K, in_dtype, out_dtype, got, ref, alpha, terms, act), what)


@pytest.mark.parametrize("case", EPI_CASES, ids=lambda c: "-".join(map(str, c)))
@pytest.mark.parametrize("layouts", [("row", "row"), ("mis", "col"), ("gap", "row")], ids="/".join)
def test_epilogue_integers_bit_exact(case, layouts):
    check_epilogue(150, 270, 200, case, layouts, seed=3)


@pytest.mark.parametrize("case", [c for c in EPI_CASES if c[0] != "f32"], ids=lambda c: "-".join(map(str, c)))
@pytest.mark.parametrize("cfg_shape", [(256, 256, 64, 2), (128, 128, 64, 2), (256, 256, 32, 3)],
                         ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("layouts", [("row", "row"), ("mis", "col")], ids="/".join)
def test_epilogue_large_tiles_bit_exact(case, cfg_shape, layouts):
    """The epilogue of the large tiles, interior and edge (800 = 3 x 256 + 32),
    through both kernels (direct-to-LDS, register-staged): their LDS holds
    more rows per pass than the 64x64 tiles of the default choice at small
    shapes."""
    check_epilogue(800, 800, 256, case, layouts, cfg=config(case[0], *cfg_shape), seed=7)


@pytest.mark.parametrize("out_dtype", ["bf16", "f32"])
@pytest.mark.parametrize("cfg_shape", [(256, 256, 64, 2), (128, 128, 64, 2)], ids=lambda s: "x".join(map(str, s)))
def test_epilogue_gelu_large_tiles(cfg_shape, out_dtype):
    """GELU with a column bias on the large tiles (interior tiles take the
    direct epilogue, edge tiles the staged one), random data, within the
    epilogue tolerance of the oracle."""
    case = ("bf16", out_dtype, 1.0, 0.0, None, "f32col", "gelu")
    check_epilogue(800, 800, 256, case, ("row", "row"), cfg=config("bf16", *cfg_shape), integers=False, seed=9)


def test_mlp_bias_gelu_full_size_sampled():
    """The fused epilogue that `bench.py --epilogue bias_gelu` times, at full
    size: the MLP-shaped product (8192 x 14336 x 4096 bf16, its default tile
    choice, every tile interior, so GELU runs in the register path) with an
    fp32 bias per column, sampled entries against the oracle's product and
    epilogue."""
    w = inputs.WORKLOADS["mlp_8192x14336x4096_bf16"]
    note("mlp bias + gelu, full size")
    a_cpu, b_cpu = inputs.make(w)
    bias = torch.randn(w.N, generator=torch.Generator().manual_seed(1))
    c = torch.full((w.M, w.N), float("nan"), dtype=TD[w.out_dtype], device=DEV)
    dg.gemm_ex(inputs.to_device_like(a_cpu, DEV), inputs.to_device_like(b_cpu, DEV), out=c, bias=bias.to(DEV),
               activation="gelu")
    torch.cuda.synchronize()
    rows, cols = sample_indices(w.M, w.N, 3000, seed=6)
    p = oracle.gemm_entries(inputs.bits(a_cpu, w.in_dtype), inputs.bits(b_cpu, w.in_dtype), w.in_dtype, rows, cols)
    bb = inputs.bits(bias, "f32")[cols]
    ref = oracle.epilogue(p.reshape(1, -1), bias_bits=bb, bias_dtype="f32", act="gelu")[0]
    got = to_f64(c[torch.from_numpy(rows).to(DEV), torch.from_numpy(cols).to(DEV)])
    assert np.all(np.isfinite(got)), "C not fully written"
    terms = np.abs(p) + np.abs(bias.double().numpy()[cols])
    assert_within_tol(got, ref, epilogue_tolerance(w.K, w.in_dtype, w.out_dtype, got, ref, 1.0, terms, "gelu"),
                      "mlp bias + gelu")


@pytest.mark.parametrize("case", [c for c in EPI_CASES if c[0] != "f32"], ids=lambda c: "-".join(map(str, c)))
def test_epilogue_with_split_k(case):
    for cfg_shape, splits in [((64, 64, 64, 4), 3), ((256, 256, 64, 2), 5)]:
        cfg = config(case[0], *cfg_shape, splits=splits)
        check_epilogue(300, 260, 1500, case, ("row", "row"), cfg=cfg, seed=5)


@pytest.mark.parametrize("act", ["gelu", "relu", "none"])
@pytest.mark.parametrize("in_dtype,out_dtype", [("bf16", "bf16"), ("f16", "f32"), ("f32", "f32")])
def test_epilogue_random(act, in_dtype, out_dtype):
    case = (in_dtype, out_dtype, 1.5, -0.75, "bf16col", "f32col", act)
    check_epilogue(257, 190, 333, case, ("row", "row"), integers=False, seed=7)
    check_epilogue(64, 64, 4096, case, ("mis", "col"), integers=False, seed=8)


@pytest.mark.parametrize("out_dtype", ["f32", "bf16", "f16"])
def test_gelu_alone_accuracy(out_dtype):
    """The epilogue's GELU by itself: C = GELU(x * 1) with K = 1, so the
    product is exact, over x in [-14, 14] (every bf16 value there that the
    grid hits). fp32 C uses the degree-9 tail: within 2^-19 relative of the
    oracle's erfc form (the device claims 7 ulp). 16-bit C uses the degree-6
    tail: within 1.5e-5 relative before the rounding, plus half an ulp."""
    xs = torch.linspace(-14.0, 14.0, 8001).to(torch.bfloat16).unique()
    M, N = xs.numel(), 64
    a = xs.reshape(M, 1)
    b = torch.ones(1, N, dtype=torch.bfloat16)
    note(f"gelu alone -> {out_dtype}")
    c = dg.gemm_ex(a.to(DEV), b.to(DEV), out_dtype=TD[out_dtype], activation="gelu")
    torch.cuda.synchronize()
    ref = oracle.epilogue(ref_product(a, b, "bf16"), act="gelu")
    got = to_f64(c)
    mag = np.maximum(np.abs(got), np.abs(ref))
    rel = 2.0 ** -19 if out_dtype == "f32" else 1.5e-5
    tol = rel * mag + 2.0 ** -40 + (0.5 * ulp(out_dtype, mag) if out_dtype != "f32" else 0.0)
    assert_within_tol(got, ref, tol, f"gelu alone -> {out_dtype}")


def test_epilogue_beta_zero_never_reads_c():
    a, b = inputs.integer_operands(100, 120, 64, "bf16", seed=2)
    out = torch.full((100, 120), float("nan"), dtype=torch.float32, device=DEV)
    note("beta=0 NaN C")
    dg.gemm_ex(place(a, "row"), place(b, "row"), out=out, alpha=2.0, beta=0.0)
    torch.cuda.synchronize()
    want = oracle.encode(2.0 * ref_product(a, b, "bf16"), "f32")
    assert_bits_equal(out_bits(out, "f32"), want, "beta=0")


def test_epilogue_k_zero():
    """K = 0: C = act(beta * R + bias), the product term is the empty sum."""
    M, N = 70, 40
    a = torch.zeros(M, 0, dtype=torch.bfloat16)
    b = torch.zeros(0, N, dtype=torch.bfloat16)
    r = int_tensor((M, N), "f32", 4, -5, 5)
    bias = int_tensor((N,), "bf16", 5, -5, 5)
    note("K=0 epilogue")
    c = dg.gemm_ex(a.to(DEV), b.to(DEV), out_dtype=torch.float32, beta=-1.0, residual=r.to(DEV),
                   bias=bias.to(DEV), activation="relu")
    torch.cuda.synchronize()
    ref = oracle.epilogue(np.zeros((M, N)), beta=-1.0, r_bits=inputs.bits(r, "f32"), r_dtype="f32",
                          bias_bits=inputs.bits(bias, "bf16"), bias_dtype="bf16", act="relu")
    assert_bits_equal(out_bits(c, "f32"), oracle.encode(ref, "f32"), "K=0")


# ---- strided batches -------------------------------------------------------------

def batch_ref(a, b, in_dtype, b_shared):
    return [ref_product(a[i], b if b_shared else b[i], in_dtype) for i in range(a.shape[0])]


@pytest.mark.parametrize("c_layout", ["contiguous", "interleaved"])
@pytest.mark.parametrize("b_kind", ["batched_row", "batched_col", "shared"])
def test_batch_integers_bit_exact(b_kind, c_layout):
    nb, M, N, K = 5, 90, 136, 200
    g = torch.Generator().manual_seed(11)
    a = torch.randint(-2, 3, (nb, M, K), generator=g).to(torch.bfloat16)
    if b_kind == "shared":
        b = torch.randint(-2, 3, (K, N), generator=g).to(torch.bfloat16)
        bd = b.to(DEV)
    else:
        b = torch.randint(-2, 3, (nb, K, N), generator=g).to(torch.bfloat16)
        bd = b.to(DEV) if b_kind == "batched_row" else b.transpose(1, 2).contiguous().to(DEV).transpose(1, 2)
    if c_layout == "contiguous":
        out = torch.empty(nb, M, N, dtype=torch.float32, device=DEV)
    else:  # [M, batch, N] storage: product i is out[:, i, :]
        out = torch.empty(M, nb, N, dtype=torch.float32, device=DEV).transpose(0, 1)
    bias = torch.randint(-3, 4, (nb, N), generator=g).to(torch.float32)
    for cfg in (None, config("bf16", 64, 64, 64, stages=4, splits=3)):
        note(f"batch {b_kind} {c_layout} cfg={cfg and cfg.k_splits}")
        dg.gemm_ex(a.to(DEV), bd, out=out, bias=bias.to(DEV), activation="relu", config=cfg)
        torch.cuda.synchronize()
        refs = batch_ref(a, b, "bf16", b_kind == "shared")
        for i in range(nb):
            ref = oracle.epilogue(refs[i], bias_bits=inputs.bits(bias[i], "f32"), bias_dtype="f32", act="relu")
            assert_bits_equal(out_bits(out[i], "f32"), oracle.encode(ref, "f32"), f"product {i}")


def test_batch_random_misaligned_with_residual():
    nb, M, N, K = 3, 130, 70, 333
    g = torch.Generator().manual_seed(12)
    a = torch.randn(nb, M, K, generator=g).to(torch.float16)
    b = torch.randn(nb, K, N, generator=g).to(torch.float16)
    r = torch.randn(nb, M, N, generator=g).to(torch.float16)
    abuf = torch.empty(a.numel() + 1, dtype=torch.float16, device=DEV)
    ad = abuf[1:].view(nb, M, K)
    ad.copy_(a.to(DEV))
    note("batch misaligned residual")
    c = dg.gemm_ex(ad, b.to(DEV), out_dtype=torch.float32, alpha=0.5, beta=2.0, residual=r.to(DEV))
    torch.cuda.synchronize()
    for i in range(nb):
        p = ref_product(a[i], b[i], "f16")
        rv = oracle.decode(inputs.bits(r[i], "f16"), "f16")
        ref = oracle.epilogue(p, alpha=0.5, beta=2.0, r_bits=inputs.bits(r[i], "f16"), r_dtype="f16")
        got = to_f64(c[i])
        tol = epilogue_tolerance(K, "f16", "f32", got, ref, 0.5, np.abs(0.5 * p) + np.abs(2 * rv), "none")
        assert_within_tol(got, ref, tol, f"product {i}")


def test_batch_empty_and_single():
    a = torch.zeros(0, 10, 20, dtype=torch.bfloat16, device=DEV)
    b = torch.zeros(0, 20, 30, dtype=torch.bfloat16, device=DEV)
    c = dg.gemm_ex(a, b)
    torch.cuda.synchronize()
    assert c.shape == (0, 10, 30)
    a1, b1 = inputs.integer_operands(40, 50, 60, "f16", seed=3)
    c1 = dg.gemm_ex(a1.to(DEV)[None], b1.to(DEV)[None])
    torch.cuda.synchronize()
    assert_bits_equal(out_bits(c1[0], "f16"), oracle.encode(ref_product(a1, b1, "f16"), "f16"), "batch of 1")


def test_batch_overlapping_c_rejected():
    a = torch.zeros(2, 8, 8, dtype=torch.bfloat16, device=DEV)
    buf = torch.zeros(100, dtype=torch.bfloat16, device=DEV)
    out = buf.as_strided((2, 8, 8), (4, 8, 1))  # products overlap
    with pytest.raises(dg.DGError) as e:
        dg.gemm_ex(a, a, out=out)
    assert e.value.status == 1


# ---- autograd (backward products through transposed views) -------------------------

def test_linear_autograd_integers_bit_exact():
    rows, fin, fout = 96, 136, 80
    g = torch.Generator().manual_seed(21)
    x = torch.randint(-2, 3, (rows, fin), generator=g).to(torch.bfloat16)
    w = torch.randint(-2, 3, (fout, fin), generator=g).to(torch.bfloat16)
    bias = torch.randint(-2, 3, (fout,), generator=g).to(torch.bfloat16)
    dy = torch.randint(-2, 3, (rows, fout), generator=g).to(torch.bfloat16)
    xd, wd, bd = (t.to(DEV).requires_grad_() for t in (x, w, bias))
    note("linear autograd")
    y = dg.linear(xd, wd, bd)
    y.backward(dy.to(DEV))
    torch.cuda.synchronize()
    xb, wb, dyb = (inputs.bits(t, "bf16") for t in (x, w, dy))
    want_y = oracle.epilogue(oracle.gemm(xb, wb.T, "bf16"), bias_bits=inputs.bits(bias, "bf16"), bias_dtype="bf16")
    assert_bits_equal(out_bits(y, "bf16"), oracle.encode(want_y, "bf16"), "y")
    assert_bits_equal(out_bits(xd.grad, "bf16"), oracle.encode(oracle.gemm(dyb, wb, "bf16"), "bf16"), "dx")
    assert_bits_equal(out_bits(wd.grad, "bf16"), oracle.encode(oracle.gemm(dyb.T, xb, "bf16"), "bf16"), "dw")
    db = oracle.decode(dyb, "bf16").sum(axis=0)
    assert_bits_equal(out_bits(bd.grad, "bf16"), oracle.encode(db, "bf16"), "dbias")


@pytest.mark.parametrize("shared_b", [False, True])
def test_matmul_autograd_batched(shared_b):
    nb, M, N, K = 3, 64, 72, 136
    g = torch.Generator().manual_seed(22)
    a = torch.randint(-2, 3, (nb, M, K), generator=g).to(torch.float16)
    b = torch.randint(-2, 3, (K, N) if shared_b else (nb, K, N), generator=g).to(torch.float16)
    dc = torch.randint(-2, 3, (nb, M, N), generator=g).to(torch.float16)
    ad, bd = a.to(DEV).requires_grad_(), b.to(DEV).requires_grad_()
    note(f"matmul autograd shared_b={shared_b}")
    c = dg.matmul(ad, bd)
    c.backward(dc.to(DEV))
    torch.cuda.synchronize()
    for i in range(nb):
        ai, dci = inputs.bits(a[i], "f16"), inputs.bits(dc[i], "f16")
        bi = inputs.bits(b if shared_b else b[i], "f16")
        assert_bits_equal(out_bits(ad.grad[i], "f16"), oracle.encode(oracle.gemm(dci, bi.T, "f16"), "f16"), "da")
    if shared_b:
        want = sum(oracle.gemm(inputs.bits(a[i], "f16").T, inputs.bits(dc[i], "f16"), "f16") for i in range(nb))
        assert_bits_equal(out_bits(bd.grad, "f16"), oracle.encode(want, "f16"), "db shared")
    else:
        for i in range(nb):
            want = oracle.gemm(inputs.bits(a[i], "f16").T, inputs.bits(dc[i], "f16"), "f16")
            assert_bits_equal(out_bits(bd.grad[i], "f16"), oracle.encode(want, "f16"), "db")


# ---- autotune over split counts ----------------------------------------------------

def test_autotune_ex_caches_and_matches():
    M, N, K = 128, 256, 8192
    a, b = inputs.random_operands(M, N, K, "bf16", seed=31)
    ad, bd = place(a, "row"), place(b, "row")
    bias = torch.randn(N, generator=torch.Generator().manual_seed(1)).to(torch.float32)
    dg.cache_clear()
    note("autotune_ex")
    cfg, ms = dg.autotune_ex(ad, bd, out_dtype=torch.float32, bias=bias.to(DEV), repeats=3)
    assert ms > 0
    c = dg.gemm_ex(ad, bd, out_dtype=torch.float32, bias=bias.to(DEV))
    torch.cuda.synchronize()
    p = ref_product(a, b, "bf16")
    ref = oracle.epilogue(p, bias_bits=inputs.bits(bias, "f32"), bias_dtype="f32")
    got = to_f64(c)
    tol = epilogue_tolerance(K, "bf16", "f32", got, ref, 1.0, np.abs(p) + np.abs(bias.double().numpy())[None], "none")
    assert_within_tol(got, ref, tol, f"autotuned {cfg}")
    with pytest.raises(dg.DGError):
        dg.autotune_ex(ad, bd, out=torch.zeros(M, N, device=DEV), beta=1.0)
    dg.cache_clear()


# ---- fp32 inputs on the matrix cores ------------------------------------------------

def f32_config(bm, splits=1):
    for c in dg.candidates(dg.DG_F32, dg.DG_F32):
        if c.variant == dg.VARIANT_MFMA and c.block_m == bm:
            c.group_m, c.xcd_remap, c.k_splits = 8, 1, splits
            return c
    raise LookupError(bm)


@pytest.mark.parametrize("layout", ["row/row", "row/col", "col/row", "col/col", "gap/col", "mis/row"])
def test_fp32_matrix_core_random(layout):
    """fp32 inputs on v_mfma_f32_32x32x2_f32: the library's choice (64x64 tiles
    here), the 128x128 tile, split-K and the fused epilogue, random normal
    inputs, within the fp32 tolerance of the oracle on every load mode
    (16-byte chunks along k or along the rows, element loads)."""
    M, N, K = 1032, 900, 1000  # multiples of 4, not of 8: 4-float chunks with M/N edges
    la, lb = layout.split("/")
    a, b = inputs.random_operands(M, N, K, "f32", seed=len(layout), dist=("normal", 1.0))
    ref = ref_product(a, b, "f32")
    ad, bd = place(a, la), place(b, lb)
    chosen, _ = dg.select_config(ad, bd, torch.empty(M, N, device=DEV))
    assert chosen.variant == dg.VARIANT_MFMA, chosen
    bias = torch.randn(N, generator=torch.Generator().manual_seed(5))
    for name, cfg in [("default", None), ("128", f32_config(128)), ("split4", f32_config(64, 4))]:
        for out_dtype in ("f32", "bf16"):
            what = f"fp32 {layout} {name} -> {out_dtype}"
            note(what)
            c = dg.gemm_ex(ad, bd, out_dtype=TD[out_dtype], config=cfg)
            torch.cuda.synchronize()
            got = to_f64(c)
            assert_within_tol(got, ref, epilogue_tolerance(K, "f32", out_dtype, got, ref, 1.0, np.abs(ref), "none"),
                              what)
    c = dg.gemm_ex(ad, bd, out_dtype=torch.float32, bias=bias.to(DEV), activation="relu", alpha=0.5)
    torch.cuda.synchronize()
    want = oracle.epilogue(ref, alpha=0.5, bias_bits=inputs.bits(bias, "f32"), bias_dtype="f32", act="relu")
    got = to_f64(c)
    assert_within_tol(got, want, epilogue_tolerance(K, "f32", "f32", got, want, 0.5,
                                                    np.abs(0.5 * ref) + np.abs(bias.double().numpy())[None], "relu"),
                      f"fp32 {layout} epilogue")
