"""GPU parity of stream-K (dg_config.k_splits = DG_STREAM_K) through dg_gemm_ex.

One workgroup per CU; each computes whole tiles while whole rounds remain and
shares out the K steps of the last, partial round. Checked against the CPU
oracle element by element:
- small-integer inputs: bit-exact (every partial tile and every sum of them is
  an integer below 2^24, so the order of the additions cannot matter);
- random inputs: within the product's tolerance, and identical from run to run
  (the owner of a tile adds the other workgroups' partials in K order).
Shapes cover more tiles than CUs with a partial last round (the case stream-K
is for), fewer tiles than CUs (every tile shared, many pieces per tile), and
exact multiples (no shared tiles); layouts cover every load path.
"""
import sys

import numpy as np
import pytest
import torch

import dense_gemm_07_amd as dg
import oracle
from dense_gemm_07_amd import inputs
from helpers import assert_bits_equal, assert_within_tol, epilogue_tolerance, out_bits, to_f64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TD = inputs.TORCH_DTYPES
CODE = {"f16": dg.DG_F16, "bf16": dg.DG_BF16}


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


def cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


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
    if layout == "miscol":  # column-major, base one element past 16-byte alignment
        buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=DEV)
        v = buf[1:].view(t.shape[1], t.shape[0])
        v.copy_(t.t().to(DEV))
        return v.t()
    if layout == "gap":  # every other column of a wider buffer: the column stride is 2
        buf = torch.zeros(t.shape[0], 2 * t.shape[1], dtype=t.dtype, device=DEV)
        v = buf[:, ::2]
        v.copy_(t.to(DEV))
        return v
    raise ValueError(layout)


def sk_config(in_dtype, bm, bn, bk=64, stages=None, group_m=8, xcd=1):
    """The stream-K config of a tile shape: 64x64 at 4 stages (the direct
    kernel's stream-K depth; register-staged operands ignore the count), the
    larger tiles at 2."""
    if stages is None:
        stages = 4 if bm == 64 else 2
    for c in dg.candidates(CODE[in_dtype], CODE[in_dtype]):
        if (c.block_m, c.block_n, c.block_k, c.stages) == (bm, bn, bk, stages):
            c.group_m, c.xcd_remap, c.k_splits = group_m, xcd, dg.STREAM_K
            return c
    raise LookupError((bm, bn, bk, stages))


def ref_product(a, b, in_dtype):
    return oracle.gemm(inputs.bits(a, in_dtype), inputs.bits(b, in_dtype), in_dtype)


def tiles(M, N, bm, bn, batch=1):
    return -(-M // bm) * -(-N // bn) * batch


# (tile shape, stages) with stream-K kernels: 64x64 direct at 4 stages, the
# others at 2 (the register-staged kernels take any stage count).
SK_CFGS = [((64, 64), 4), ((128, 128), 2)]
# Layouts whose kernels have stream-K instantiations: the direct kernel (row/row,
# row/col, col/row) and the padded-row register kernel (element loads, and on
# 64x64 tiles k-contiguous operands off alignment). Operands off alignment take
# the staged kernel otherwise (a row-contiguous one at any tile size, both
# k-contiguous from 128x128 up), which has none.
def layouts_for(bm):
    yes = [("row", "row"), ("row", "col"), ("col", "row"), ("gap", "col")]
    no = [("mis", "row"), ("col", "miscol")]
    (yes if bm == 64 else no).append(("mis", "col"))
    return yes, no


def shapes_for(bm, bn, n_cu):
    """A partial last round (1.5 rounds), an exact round count, fewer tiles
    than CUs, and a single tile with a long K. Every size is a multiple of 8,
    so the row- and column-major views stay 16-byte aligned (the "mis" and
    "gap" layouts take them off alignment)."""
    gm = 16
    gn = (3 * n_cu // 2) // gm  # 1.5 rounds of tiles
    return [(gm * bm - 24, gn * bn - 40, 296 if bm == 64 else 136),
            (gm * bm, (n_cu // gm) * bn, 136),
            (2 * bm + 8, bn - 8, 776),
            (bm, bn, 2056)]


@pytest.mark.parametrize("cfg_shape", SK_CFGS, ids=lambda s: f"{s[0][0]}x{s[0][1]}")
def test_stream_k_integers_bit_exact(cfg_shape):
    (bm, bn), stages = cfg_shape
    n_cu = cus()
    for (M, N, K) in shapes_for(bm, bn, n_cu):
        a, b = inputs.integer_operands(M, N, K, "bf16", seed=M + N + K)
        want32 = ref_product(a, b, "bf16")
        for out_dtype in ("f32", "bf16"):
            want = oracle.encode(want32, out_dtype)
            yes, no = layouts_for(bm)
            for la, lb in no:
                cfg = sk_config("bf16", bm, bn, stages=stages)
                with pytest.raises(dg.DGError) as e:
                    dg.gemm_ex(place(a, la), place(b, lb), out_dtype=TD[out_dtype], config=cfg)
                assert e.value.status == 3, (la, lb)
            for la, lb in yes:
                what = f"{(M, N, K)} tiles={tiles(M, N, bm, bn)} cus={n_cu} sk {bm}x{bn} {la}/{lb} -> {out_dtype}"
                note(what)
                cfg = sk_config("bf16", bm, bn, stages=stages)
                c = torch.full((M, N), float("nan"), dtype=TD[out_dtype], device=DEV)
                dg.gemm_ex(place(a, la), place(b, lb), out=c, config=cfg)
                torch.cuda.synchronize()
                assert_bits_equal(out_bits(c, out_dtype), want, what)


def test_stream_k_ragged_product_every_group_order():
    """The 1000x1500x777 product (column-major B, 384 tiles of 64x64) under
    stream-K for each launch order, f16 and bf16."""
    M, N, K = 1000, 1500, 777
    for in_dtype in ("bf16", "f16"):
        a, b = inputs.integer_operands(M, N, K, in_dtype, seed=7)
        want = oracle.encode(ref_product(a, b, in_dtype), "f32")
        ad, bd = place(a, "row"), place(b, "col")
        for group_m, xcd in [(8, 1), (1, 0), (4, 1), (16, 0)]:
            what = f"ragged {in_dtype} group_m={group_m} xcd={xcd}"
            note(what)
            cfg = sk_config(in_dtype, 64, 64, group_m=group_m, xcd=xcd)
            c = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
            dg.gemm_ex(ad, bd, out=c, config=cfg)
            torch.cuda.synchronize()
            assert_bits_equal(out_bits(c, "f32"), want, what)


def test_stream_k_epilogue_and_batch_bit_exact():
    """alpha * A@B + beta * R + bias with ReLU, a batch of three products (the
    tiles of all products are shared out together)."""
    M, N, K, nb = 520, 704, 400, 3
    g = torch.Generator().manual_seed(11)
    a = torch.randint(-2, 3, (nb, M, K), generator=g).to(torch.bfloat16)
    b = torch.randint(-2, 3, (nb, K, N), generator=g).to(torch.bfloat16)
    r = torch.randint(-4, 5, (nb, M, N), generator=g).float()
    bias = torch.randint(-4, 5, (nb, N), generator=g).float()
    assert tiles(M, N, 64, 64, nb) > cus()
    for bm, stages in [(64, 4), (128, 2)]:
        cfg = sk_config("bf16", bm, bm, stages=stages)
        what = f"epilogue batch sk {bm}"
        note(what)
        out = torch.full((nb, M, N), float("nan"), dtype=torch.float32, device=DEV)
        dg.gemm_ex(a.to(DEV), b.to(DEV), out=out, alpha=2.0, beta=-1.0, residual=r.to(DEV), bias=bias.to(DEV),
                   activation="relu", config=cfg)
        torch.cuda.synchronize()
        for i in range(nb):
            p = ref_product(a[i], b[i], "bf16")
            ref = oracle.epilogue(p, alpha=2.0, beta=-1.0, r_bits=inputs.bits(r[i], "f32"), r_dtype="f32",
                                  bias_bits=inputs.bits(bias[i], "f32"), bias_dtype="f32", act="relu")
            assert_bits_equal(out_bits(out[i], "f32"), oracle.encode(ref, "f32"), f"{what} product {i}")


def test_stream_k_random_deterministic_and_workspace_reuse():
    """Random inputs: within tolerance, bit-identical over repeated calls on one
    workspace whose contents start as garbage, with split-K calls on the same
    workspace in between (their partials overwrite the flag area)."""
    M, N, K = 1000, 1500, 777
    a, b = inputs.random_operands(M, N, K, "bf16", seed=3)
    ad, bd = place(a, "row"), place(b, "col")
    ref = ref_product(a, b, "bf16")
    cfg = sk_config("bf16", 64, 64)
    split = sk_config("bf16", 64, 64)
    split.k_splits = 4
    need = max(dg.workspace_size(M, N, K, 1, cfg), dg.workspace_size(M, N, K, 1, split))
    ws = torch.full((need // 4 + 64,), -1.0, dtype=torch.float32, device=DEV)
    ws.view(torch.int32)[: 2 * cus()] = -1  # every flag word all ones
    runs = []
    for rep in range(4):
        note(f"stream-K rep {rep}")
        c = dg.gemm_ex(ad, bd, out_dtype=torch.float32, config=cfg, workspace=ws)
        torch.cuda.synchronize()
        runs.append(out_bits(c, "f32"))
        if rep == 1:
            s = dg.gemm_ex(ad, bd, out_dtype=torch.float32, config=split, workspace=ws)
            torch.cuda.synchronize()
            got = to_f64(s)
            assert_within_tol(got, ref, epilogue_tolerance(K, "bf16", "f32", got, ref, 1.0, np.abs(ref), "none"),
                              "split-K between stream-K calls")
    assert all(np.array_equal(runs[0], r) for r in runs[1:]), "stream-K results differ between runs"
    got = to_f64(c)
    assert_within_tol(got, ref, epilogue_tolerance(K, "bf16", "f32", got, ref, 1.0, np.abs(ref), "none"), "stream-K")


def test_stream_k_k_edges():
    """K = 0 (C = epilogue of zero), K below one slice, K = one slice."""
    M, N = 700, 1300
    for K in (0, 5, 64, 65):
        for la, lb in [("row", "col"), ("gap", "col")]:
            if K % 8 and la == "row":
                la = "mis"
            a, b = inputs.integer_operands(M, N, K, "bf16", seed=K + 1)
            what = f"K={K} {la}/{lb}"
            note(what)
            cfg = sk_config("bf16", 64, 64)
            bias = torch.arange(N, dtype=torch.float32) % 5 - 2
            c = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
            dg.gemm_ex(place(a, la), place(b, lb), out=c, bias=bias.to(DEV), config=cfg)
            torch.cuda.synchronize()
            p = ref_product(a, b, "bf16") if K else np.zeros((M, N))
            ref = oracle.epilogue(p, bias_bits=inputs.bits(bias, "f32"), bias_dtype="f32")
            assert_bits_equal(out_bits(c, "f32"), oracle.encode(ref, "f32"), what)


def test_stream_k_argument_errors():
    a = torch.zeros(1000, 777, dtype=torch.bfloat16, device=DEV)
    b = torch.zeros(1500, 777, dtype=torch.bfloat16, device=DEV).t()
    cfg = sk_config("bf16", 64, 64)
    with pytest.raises(dg.DGError) as e:
        dg.gemm_ex(a, b, config=cfg, workspace=None)
    assert e.value.status == 1 and b"workspace" in dg.library().dg_last_error()
    small = torch.empty(1024, dtype=torch.uint8, device=DEV)
    with pytest.raises(dg.DGError) as e:
        dg.gemm_ex(a, b, config=cfg, workspace=small)
    assert e.value.status == 1
    for shape in [(64, 64, 32, 8), (256, 256, 64, 2)]:  # tile shapes without a stream-K kernel
        nosk = sk_config("bf16", *shape[:2], bk=shape[2], stages=shape[3])
        with pytest.raises(dg.DGError) as e:
            dg.gemm_ex(a, b, config=nosk)
        assert e.value.status == 3 and b"stream-K" in dg.library().dg_last_error()


def test_stream_k_matches_unsplit_and_is_not_the_default():
    """An explicit stream-K config gives the unsplit kernel's result bit for bit
    on integers; the library's own choice (given a workspace) stays unsplit,
    stream-K having measured slower on MI355X."""
    M, N, K = 1000, 1500, 777
    a, b = inputs.integer_operands(M, N, K, "bf16", seed=5)
    ad, bd = place(a, "row"), place(b, "col")
    cfg, _ = dg.select_config_ex(M, N, K, ad.stride(), bd.stride(), (N, 1), CODE["bf16"], dg.DG_F32,
                                 workspace_bytes=dg.DEFAULT_WORKSPACE_BYTES)
    assert cfg.k_splits == 1, cfg
    c_sk = dg.gemm_ex(ad, bd, out_dtype=torch.float32, config=sk_config("bf16", 64, 64))
    plain = sk_config("bf16", 64, 64)
    plain.k_splits = 1
    c_dp = dg.gemm_ex(ad, bd, out_dtype=torch.float32, config=plain, workspace=None)
    torch.cuda.synchronize()
    assert torch.equal(c_sk, c_dp)
    assert_bits_equal(out_bits(c_sk, "f32"), oracle.encode(ref_product(a, b, "bf16"), "f32"), "stream-K")
