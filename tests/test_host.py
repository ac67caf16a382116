"""CPU tests of the C-ABI library's host logic (no GPU work is started).

The library must load and export every entry point declared in include/dg.h;
argument validation, launch order, grid arithmetic, config selection and the
config cache are exercised through the C-ABI itself.
"""
import ctypes
import itertools
import os
import re

import pytest

import dense_gemm_07_amd as dg
from conftest import ROOT, load_golden, load_grid_counts

F32, F16, BF16 = dg.DG_F32, dg.DG_F16, dg.DG_BF16
OK, INVALID, NO_CONFIG = 0, 1, 3


def declared_symbols():
    text = open(os.path.join(ROOT, "include", "dg.h")).read()
    return sorted(set(re.findall(r"\b(dg_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = dg.library()
    names = declared_symbols()
    assert len(names) >= 15
    for n in names:
        assert hasattr(lib, n), f"{n} declared in dg.h but not exported"


def test_missing_library_fails_loudly(monkeypatch):
    monkeypatch.setattr(dg, "_lib", None)
    monkeypatch.setattr(dg, "LIB", "/nonexistent/libdg.so")
    with pytest.raises(RuntimeError, match="not built"):
        dg.library()


def test_status_strings():
    lib = dg.library()
    assert lib.dg_status_string(0) == b"DG_OK"
    assert lib.dg_status_string(3) == b"DG_ERR_NO_CONFIG"


# ---- launch order -------------------------------------------------------------

def test_group_major_layout_from_the_page():
    g = load_golden("p1_s4_group_major.txt")
    for label, group in (("ROWMAJOR", 1), ("GROUP2", 2)):
        grid = [[None] * 4 for _ in range(4)]
        for wg in range(16):
            m, n = dg.tile_coords(4, 4, group, 0, 8, wg)
            grid[m][n] = wg
        assert grid == g[label], label


@pytest.mark.parametrize("xcd", [0, 1])
def test_tile_map_is_a_bijection(xcd):
    for gm, gn in itertools.product([1, 2, 3, 5, 8, 13, 16, 17], repeat=2):
        for group in (1, 2, 3, 4, 8, 16):
            for nx in ((1, 8) if xcd else (8,)):
                seen = set()
                for wg in range(gm * gn):
                    m, n = dg.tile_coords(gm, gn, group, xcd, nx, wg)
                    assert 0 <= m < gm and 0 <= n < gn
                    seen.add((m, n))
                assert len(seen) == gm * gn, (gm, gn, group, xcd, nx)


def test_xcd_remap_gives_each_xcd_a_consecutive_run():
    # 16 x 16 tiles over 8 XCDs: with group 4, the 32 ids dispatched to one
    # XCD (wg % 8 == x) cover a compact 4-row x 8-column block of tiles.
    for x in range(8):
        tiles = {dg.tile_coords(16, 16, 4, 1, 8, wg) for wg in range(x, 256, 8)}
        rows = {m for m, _ in tiles}
        cols = {n for _, n in tiles}
        assert len(tiles) == 32 and len(rows) == 4 and len(cols) == 8, (x, sorted(tiles))


def test_tile_coords_rejects_bad_arguments():
    for args in [(0, 4, 1, 0, 8, 0), (4, 4, 0, 0, 8, 0), (4, 4, 1, 0, 8, 16), (4, 4, 1, 0, 8, -1)]:
        with pytest.raises(dg.DGError):
            dg.tile_coords(*args)


# ---- grid arithmetic (pages' counts) ------------------------------------------

def test_grid_counts_from_the_pages():
    for M, N, K, BM, BN, BK, gm, gn, ks, oob_r, oob_c, oob_k in load_grid_counts():
        cfg = dg.Config(BM, BN, BK, 1, 4, 1, dg.VARIANT_SIMT, 0)
        got_m, got_n, got_k = dg.grid_shape(M, N, max(K, 0), cfg)
        assert (got_m, got_n) == (gm, gn)
        if ks >= 0:
            assert got_k == ks
        if oob_r >= 0:
            assert got_m * BM - M == oob_r
        if oob_c >= 0:
            assert got_n * BN - N == oob_c
        if oob_k >= 0:
            assert got_k * BK - K == oob_k
    # "用 Triton 写 GPU Kernel" §3.4: 16 programs x 3 rounds = 48 small products
    gm, gn, ks = dg.grid_shape(8, 8, 6, dg.Config(2, 2, 2, 1, 4, 1, 0, 0))
    assert gm * gn * ks == 48


# ---- validation -----------------------------------------------------------------

P = 4096  # a stand-in device address (16-byte aligned); nothing is dereferenced


def v(M=4, N=4, K=4, a=P, sa=(4, 1), b=P, sb=(4, 1), c=P, sc=(4, 1), i=BF16, o=BF16):
    return dg.validate(M, N, K, a, sa, b, sb, c, sc, i, o)


def test_validate_accepts_good_arguments():
    assert v() == OK
    assert v(sa=(0, 0), sb=(0, 0)) == OK               # broadcast operands are allowed
    assert v(sb=(1, 4)) == OK                           # column-major B
    assert v(M=0, a=0, c=0) == OK                       # empty problem needs no pointers
    assert v(K=0, a=0, b=0) == OK                       # K = 0 writes zeros into C
    assert v(M=2, N=2, sc=(3, 2)) == OK                 # offsets 0,2,3,5: no overlap
    assert v(i=F32, o=F16, a=P + 4, b=P + 8) == OK


@pytest.mark.parametrize("kw", [
    dict(M=-1), dict(N=-1), dict(K=-1),
    dict(a=0), dict(b=0), dict(c=0),
    dict(sa=(-4, 1)), dict(sb=(4, -1)),
    dict(sc=(0, 1)), dict(sc=(4, 0)),
    dict(sc=(1, 1)), dict(sc=(2, 1)), dict(M=3, N=3, sc=(2, 1)),
    dict(a=P + 1), dict(c=P + 1), dict(i=F32, a=P + 2),
    dict(i=7), dict(o=-1),
])
def test_validate_rejects(kw):
    assert v(**kw) == INVALID


def test_validate_rejects_huge_dims():
    assert v(M=1 << 31) != OK


# ---- config selection ----------------------------------------------------------

def test_heuristic_choices():
    c, hit = dg.select_config_raw(4096, 4096, 4096, (4096, 1), (4096, 1), (4096, 1), BF16, BF16)
    assert not hit and c.variant == dg.VARIANT_MFMA and (c.block_m, c.block_n) == (256, 256)
    c, _ = dg.select_config_raw(26, 26, 26, (26, 1), (26, 1), (26, 1), F32, F32)
    assert c.variant == dg.VARIANT_SIMT
    # fp32 beyond tiny sizes: the fp32 matrix-core kernel, 128x128 once that fills the CUs;
    # the boundary is C within two 32x32 tiles
    c, _ = dg.select_config_raw(32, 64, 64, (64, 1), (64, 1), (64, 1), F32, F32)
    assert c.variant == dg.VARIANT_SIMT
    c, _ = dg.select_config_raw(64, 64, 64, (64, 1), (64, 1), (64, 1), F32, F32)
    assert c.variant == dg.VARIANT_MFMA and (c.block_m, c.block_k) == (64, 32)
    c, _ = dg.select_config_raw(1024, 1024, 1024, (1024, 1), (1024, 1), (1024, 1), F32, F32)
    assert c.variant == dg.VARIANT_MFMA and (c.block_m, c.block_k) == (64, 32)
    c, _ = dg.select_config_raw(4096, 4096, 4096, (4096, 1), (4096, 1), (4096, 1), F32, F16)
    assert c.variant == dg.VARIANT_MFMA and (c.block_m, c.block_k) == (128, 32)
    c, _ = dg.select_config_raw(1024, 1024, 1024, (1024, 1), (1024, 1), (1024, 1), F16, F16)
    assert c.variant == dg.VARIANT_MFMA and (1024 // c.block_m) * (1024 // c.block_n) >= 256


def test_heuristic_counts_rounds_of_tiles():
    # aligned bf16 squares: the tile shape with the least rounds x work per
    # workgroup / rate, not the biggest tile that fills the CUs
    want = {1536: (128, 128, 3), 2048: (128, 128, 3), 2560: (128, 128, 2), 3072: (256, 256, 2),
            3584: (256, 256, 2), 4096: (256, 256, 2), 6144: (256, 256, 2), 1024: (64, 64, 4)}
    for n, (bm, bn, st) in want.items():
        c, _ = dg.select_config_raw(n, n, n, (n, 1), (n, 1), (n, 1), BF16, BF16)
        assert (c.block_m, c.block_n, c.stages) == (bm, bn, st), (n, c)
    c, _ = dg.select_config_raw(8192, 14336, 4096, (4096, 1), (14336, 1), (14336, 1), BF16, BF16)
    assert (c.block_m, c.block_n) == (256, 256), c
    c, _ = dg.select_config_raw(16, 14336, 4096, (4096, 1), (14336, 1), (14336, 1), BF16, BF16)
    assert (c.block_m, c.block_n) == (64, 64), c


def test_heuristic_counts_rounds_for_staged_operands():
    # A off 16-byte alignment (base address 2 bytes past a boundary): the
    # register-staged kernels' rates in the same round-counting model
    want = {1536: (128, 128), 2560: (128, 256), 3072: (256, 256), 3584: (256, 256), 4096: (256, 256)}
    for n, tile in want.items():
        c, _ = dg.select_config_raw(n, n, n, (n, 1), (n, 1), (n, 1), BF16, BF16, ptr_a=0x1002, ptr_b=0x2000,
                                    ptr_c=0x3000)
        assert (c.block_m, c.block_n) == tile, (n, c)


def test_heuristic_bk32_for_short_unaligned_k():
    # both operands k-contiguous off 16-byte alignment (leading dimension 777
    # or 1555): BK 32 when BK 64 pads K by more than 5 %
    c, _ = dg.select_config_raw(1000, 1500, 777, (777, 1), (1, 777), (1500, 1), BF16, dg.DG_F32)
    assert (c.variant, c.block_m, c.block_n, c.block_k) == (dg.VARIANT_MFMA, 64, 64, 32), c
    c, _ = dg.select_config_raw(2000, 3000, 1555, (1555, 1), (1, 1555), (3000, 1), BF16, dg.DG_F32)
    assert c.block_k == 64, c
    # a row-contiguous B at the same K keeps BK 64
    c, _ = dg.select_config_raw(1000, 1500, 777, (777, 1), (1500, 1), (1500, 1), BF16, dg.DG_F32)
    assert c.block_k == 64, c
    # aligned operands (direct kernel) keep BK 64
    c, _ = dg.select_config_raw(1000, 1504, 776, (776, 1), (1, 776), (1504, 1), BF16, dg.DG_F32)
    assert c.block_k == 64, c


def test_candidates_are_distinct_and_complete():
    for i, o in itertools.product([F32, F16, BF16], repeat=2):
        cands = dg.candidates(i, o)
        assert cands, (i, o)
        keys = {tuple(c.as_dict().values()) for c in cands}
        assert len(keys) == len(cands)
        if i == F32:
            assert {c.variant for c in cands} == {dg.VARIANT_SIMT, dg.VARIANT_MFMA}
        else:
            assert all(c.variant == dg.VARIANT_MFMA for c in cands)
            assert {c.group_m for c in cands} >= {1, 8} and {c.xcd_remap for c in cands} == {0, 1}


def test_candidate_index_out_of_range():
    lib = dg.library()
    n = lib.dg_num_candidates(BF16, BF16)
    assert lib.dg_get_candidate(n, BF16, BF16, ctypes.byref(dg.Config())) == INVALID
    assert lib.dg_num_candidates(9, BF16) == 0


# ---- config cache ----------------------------------------------------------------

def test_cache_load_select_save_roundtrip(tmp_path):
    dg.cache_clear()
    # key: M N K batch in out la lb lc | block_m block_n block_k group_m waves stages variant xcd k_splits
    f = tmp_path / "cache.txt"
    f.write_text("dg-config-cache 2\n"
                 "4096 4096 4096 1 2 2 0 1 0  128 128 64 4 4 2 1 0 1\n"
                 "1024 1024 1024 1 2 2 0 1 0  128 128 64 8 4 2 1 1 4\n"
                 "1000 1500 777 1 2 2 3 3 0  64 64 64 8 4 4 1 1 -1\n"
                 "this line is garbage\n")
    dg.cache_load(str(f))
    assert dg.cache_size() == 3
    assert b"malformed" in dg.library().dg_last_error()
    c, hit = dg.select_config_raw(4096, 4096, 4096, (4096, 1), (4096, 1), (4096, 1), BF16, BF16)
    assert hit and (c.block_m, c.block_n, c.group_m, c.xcd_remap) == (128, 128, 4, 0)
    # a different layout class of B is a different key
    _, hit2 = dg.select_config_raw(4096, 4096, 4096, (4096, 1), (1, 4096), (4096, 1), BF16, BF16)
    assert not hit2
    # a cached split-K config runs unsplit where the call has no workspace
    c3, hit3 = dg.select_config_raw(1024, 1024, 1024, (1024, 1), (1024, 1), (1024, 1), BF16, BF16)
    assert hit3 and (c3.block_m, c3.k_splits) == (128, 1)
    # a cached stream-K config (k-contiguous unaligned operands, layout modes 3/3)
    ws = dict(batch=1, workspace_bytes=1 << 30)
    c4, hit4 = dg.select_config_ex(1000, 1500, 777, (777, 1), (1, 777), (1500, 1), BF16, BF16, **ws)
    assert hit4 and c4.k_splits == dg.STREAM_K, c4
    c5, _ = dg.select_config_ex(1000, 1500, 777, (777, 1), (1, 777), (1500, 1), BF16, BF16, batch=1,
                                workspace_bytes=1024)
    assert c5.k_splits == 1  # no room for its workspace: unsplit
    out = tmp_path / "saved.txt"
    dg.cache_save(str(out))
    lines = out.read_text().splitlines()
    assert lines[0] == "dg-config-cache 2" and len(lines) == 4
    assert any(ln.split()[-1] == "4" for ln in lines[1:])  # k_splits survives the round trip
    assert any(ln.split()[-1] == "-1" for ln in lines[1:])
    dg.cache_clear()
    assert dg.cache_size() == 0
    dg.cache_load(str(out))
    assert dg.cache_size() == 3
    dg.cache_clear()


def test_cache_load_rejects_older_format(tmp_path):
    f = tmp_path / "v1.txt"
    f.write_text("dg-config-cache 1\n4096 4096 4096 2 2 0 1 0  128 128 64 4 4 2 1 0\n")
    with pytest.raises(dg.DGError):
        dg.cache_load(str(f))


def test_cache_load_rejects_foreign_file(tmp_path):
    f = tmp_path / "x.txt"
    f.write_text("not a cache\n")
    with pytest.raises(dg.DGError):
        dg.cache_load(str(f))
    with pytest.raises(dg.DGError):
        dg.cache_load(str(tmp_path / "missing.txt"))


# ---- dg_gemm_ex: argument checks that fail before any GPU work ------------------

FAKE = 1 << 20  # a 256-byte aligned stand-in address; never dereferenced on these paths


def gemm_ex_status(M=64, N=64, K=64, a=(64, 1), b=(64, 1), c=(64, 1), epi=None, batch=None, cfg=None,
                   ws=None, ws_bytes=0, dt=BF16, out=BF16):
    lib = dg.library()
    return lib.dg_gemm_ex(M, N, K, FAKE, *a, FAKE, *b, FAKE, *c, dt, out, None,
                          ctypes.byref(epi) if epi else None, ctypes.byref(batch) if batch else None,
                          ctypes.byref(cfg) if cfg else None, ws, ws_bytes)


def mfma_cfg(bm=128, bn=128, bk=64, splits=1):
    for c in dg.candidates(BF16, BF16):
        if (c.block_m, c.block_n, c.block_k, c.stages) == (bm, bn, bk, 2):
            c.k_splits = splits
            return c
    raise LookupError


def test_gemm_ex_rejects_bad_epilogue():
    assert gemm_ex_status(epi=dg.Epilogue(alpha=1.0, activation=7)) == INVALID
    assert gemm_ex_status(epi=dg.Epilogue(alpha=1.0, bias=FAKE, bias_dtype=9)) == INVALID
    assert gemm_ex_status(epi=dg.Epilogue(alpha=1.0, bias=FAKE + 1, bias_dtype=F32)) == INVALID  # misaligned
    assert gemm_ex_status(epi=dg.Epilogue(alpha=1.0, bias=FAKE, bias_dtype=F32, bias_stride=-1)) == INVALID
    assert gemm_ex_status(epi=dg.Epilogue(alpha=1.0, beta=1.0, residual=FAKE, residual_dtype=F32,
                                          stride_rm=-1, stride_rn=1)) == INVALID
    assert gemm_ex_status(epi=dg.Epilogue(alpha=1.0, beta=1.0, residual=FAKE, residual_dtype=5)) == INVALID
    assert gemm_ex_status(epi=dg.Epilogue(alpha=1.0, beta=1.0, residual=FAKE + 2, residual_dtype=F32,
                                          stride_rm=64, stride_rn=1)) == INVALID
    assert b"residual" in dg.library().dg_last_error()


def test_gemm_ex_rejects_residual_overlapping_c():
    """A residual that shares memory with C must be C's own view; any other
    overlap lets one tile's workgroup read what another is writing."""
    def status(res, rdt, srm, srn, batch=None):
        return gemm_ex_status(epi=dg.Epilogue(alpha=1.0, beta=1.0, residual=res, residual_dtype=rdt,
                                              stride_rm=srm, stride_rn=srn), batch=batch)
    assert status(FAKE, BF16, 1, 64) == INVALID            # C transposed
    assert b"overlaps C" in dg.library().dg_last_error()
    assert status(FAKE + 128, BF16, 64, 1) == INVALID      # C one row down
    assert status(FAKE - 2, BF16, 64, 1) == INVALID        # C one element left
    assert status(FAKE, F32, 32, 1) == INVALID             # same bytes read as fp32
    # C's first product broadcast to the whole batch while C has two products
    assert status(FAKE, BF16, 64, 1, dg.Batch(count=2, stride_c=4096, stride_r=0)) == INVALID


def test_gemm_ex_rejects_bad_batch():
    assert gemm_ex_status(batch=dg.Batch(count=-1)) == INVALID
    assert gemm_ex_status(batch=dg.Batch(count=2, stride_a=-8)) == INVALID
    # C views of the two products overlap (stride_c smaller than one 64x64 view, not nested)
    assert gemm_ex_status(batch=dg.Batch(count=2, stride_c=32)) == INVALID
    assert b"overlap" in dg.library().dg_last_error()
    # an empty batch is a no-op, even with NULL pointers
    lib = dg.library()
    assert lib.dg_gemm_ex(64, 64, 64, None, 64, 1, None, 64, 1, None, 64, 1, BF16, BF16, None, None,
                          ctypes.byref(dg.Batch(count=0)), None, None, 0) == OK


def test_gemm_ex_split_k_argument_errors():
    cfg = mfma_cfg(splits=4)
    # no workspace / too small / misaligned
    assert gemm_ex_status(K=4096, cfg=cfg) == INVALID
    assert b"workspace" in dg.library().dg_last_error()
    assert gemm_ex_status(K=4096, cfg=cfg, ws=FAKE, ws_bytes=1024) == INVALID
    need = dg.workspace_size(64, 64, 4096, 1, cfg)
    assert gemm_ex_status(K=4096, cfg=cfg, ws=FAKE + 16, ws_bytes=need) == INVALID
    assert gemm_ex_status(K=4096, cfg=cfg, ws=FAKE, ws_bytes=-5) == INVALID
    # split-K is an MFMA feature
    simt = [c for c in dg.candidates(F32, F32) if c.variant == dg.VARIANT_SIMT][0]
    simt.k_splits = 2
    assert gemm_ex_status(K=4096, cfg=simt, dt=F32, out=F32, a=(4096, 1), b=(64, 1)) == NO_CONFIG


def test_workspace_size_arithmetic():
    cfg = mfma_cfg(128, 128, 64, splits=4)
    # 8 x 8 tiles, K ranges of 256: 4 ranges
    assert dg.workspace_size(1024, 1024, 1024, 1, cfg) == 64 * 4 * 128 * 128 * 4
    # batch multiplies tiles
    assert dg.workspace_size(1024, 1024, 1024, 3, cfg) == 3 * 64 * 4 * 128 * 128 * 4
    # K = 200, 3 requested: chunks of ceil(67/64)*64 = 128 -> 2 ranges
    cfg3 = mfma_cfg(128, 128, 64, splits=3)
    assert dg.workspace_size(128, 128, 200, 1, cfg3) == 2 * 128 * 128 * 4
    # one K slice or no split: nothing
    assert dg.workspace_size(1024, 1024, 64, 1, cfg) == 0
    assert dg.workspace_size(1024, 1024, 4096, 1, mfma_cfg(splits=1)) == 0
    assert dg.workspace_size(0, 1024, 4096, 1, cfg) == 0


def test_stream_k_argument_errors_and_workspace_size():
    """Stream-K (k_splits = DG_STREAM_K): a workspace of 8 bytes of flag per
    CU rounded up to 256, then one partial tile per CU (256 CUs on MI355X, and
    the library's assumption without a device); checked before any launch."""
    sk = mfma_cfg(128, 128, 64, splits=dg.STREAM_K)
    need = dg.workspace_size(1024, 1024, 1024, 1, sk)
    assert need == 256 * 8 + 256 * 128 * 128 * 4
    assert dg.workspace_size(0, 1024, 1024, 1, sk) == 0
    assert gemm_ex_status(K=4096, cfg=sk) == INVALID  # no workspace
    assert b"stream-K" in dg.library().dg_last_error()
    assert gemm_ex_status(K=4096, cfg=sk, ws=FAKE, ws_bytes=need - 1) == INVALID
    assert gemm_ex_status(K=4096, cfg=sk, ws=FAKE + 16, ws_bytes=need) == INVALID  # misaligned
    # tile shapes compiled without a stream-K kernel
    for bm, bk, stages in [(256, 64, 2), (128, 64, 3)]:
        c = next(x for x in dg.candidates(BF16, BF16) if (x.block_m, x.block_n, x.block_k, x.stages) == (bm, bm, bk, stages))
        c.k_splits = dg.STREAM_K
        assert gemm_ex_status(K=4096, cfg=c, ws=FAKE, ws_bytes=1 << 30) == NO_CONFIG
        assert b"no stream-K kernel" in dg.library().dg_last_error()
    simt = [c for c in dg.candidates(F32, F32) if c.variant == dg.VARIANT_SIMT][0]
    simt.k_splits = dg.STREAM_K
    assert gemm_ex_status(K=4096, cfg=simt, dt=F32, out=F32, a=(4096, 1), b=(64, 1), ws=FAKE,
                          ws_bytes=1 << 30) == NO_CONFIG
    # never the library's own choice
    for M, N, K in [(1000, 1500, 777), (4096, 4352, 4096), (5120, 5120, 1024)]:
        c, _ = dg.select_config_ex(M, N, K, (K, 1), (1, K), (N, 1), BF16, BF16, batch=1, workspace_bytes=1 << 30)
        assert c.k_splits != dg.STREAM_K, ((M, N, K), c)


def test_select_config_never_splits_without_workspace():
    for M, N, K in [(16, 4096, 8192), (128, 128, 65536), (1, 1, 1 << 20)]:
        c, _ = dg.select_config_raw(M, N, K, (K, 1), (N, 1), (N, 1), BF16, BF16)
        assert c.k_splits == 1


def test_autotune_ex_rejects_epilogue_reading_c():
    lib = dg.library()
    epi = dg.Epilogue(alpha=1.0, beta=0.5)
    st = lib.dg_autotune_ex(64, 64, 64, FAKE, 64, 1, FAKE, 64, 1, FAKE, 64, 1, BF16, BF16, None,
                            ctypes.byref(epi), None, None, 0, 1, None, None)
    assert st == INVALID and b"reads C" in lib.dg_last_error()


def test_gemm_ex_default_split_choice():
    """Split counts the library picks for dg_gemm_ex with a workspace (the measured rule)."""
    cases = {(1024, 1024, 1024): 1, (1, 14336, 4096): 1, (512, 512, 4096): 4, (256, 256, 32768): 16,
             (2048, 512, 8192): 1, (128, 4096, 8192): 2, (512, 512, 16384): 4, (128, 128, 8192): 8, (64, 64, 65536): 16}
    for (M, N, K), want in cases.items():
        c, _ = dg.select_config_ex(M, N, K, (K, 1), (N, 1), (N, 1), BF16, BF16, batch=1,
                                   workspace_bytes=1 << 30)
        assert (c.block_m, c.k_splits) == (64, want), ((M, N, K), c)
        assert dg.workspace_size(M, N, K, 1, c) <= 1 << 30
    # no (or too small a) workspace: never split
    c, _ = dg.select_config_ex(256, 256, 32768, (32768, 1), (256, 1), (256, 1), BF16, BF16, batch=1,
                               workspace_bytes=1024)
    assert c.k_splits == 1
    # a batch that fills the GPU needs no split
    c, _ = dg.select_config_ex(256, 256, 32768, (32768, 1), (256, 1), (256, 1), BF16, BF16, batch=64,
                               workspace_bytes=1 << 30)
    assert c.k_splits == 1


# ---- dg_attention_fwd: argument checks (no GPU work) -------------------------------

def attn_status(B=1, H=1, Sq=8, Skv=8, D=64, q=FAKE, k=FAKE, v=FAKE, o=FAKE, st=(512, 512, 64), dt=BF16, out=BF16):
    lib = dg.library()
    arr = lambda t: (ctypes.c_int64 * 3)(*t)
    return lib.dg_attention_fwd(B, H, Sq, Skv, D, q, arr(st), k, arr(st), v, arr(st), o, arr(st), None, dt, out,
                                ctypes.c_float(0.0), 0, None)


def test_attention_argument_checks():
    UNSUPPORTED = 2
    assert attn_status(B=-1) == INVALID
    assert attn_status(q=None) == INVALID
    assert attn_status(D=96) == UNSUPPORTED and b"head_dim" in dg.library().dg_last_error()
    assert attn_status(dt=F32) == UNSUPPORTED
    assert attn_status(q=FAKE + 2) == UNSUPPORTED           # Q not 16-byte aligned
    assert attn_status(st=(512, 512, 66)) == UNSUPPORTED    # seq stride not a multiple of 8
    assert attn_status(st=(512, 512, 32)) == INVALID        # O rows overlap (seq stride < head_dim)
    assert attn_status(Sq=0) == OK and attn_status(B=0) == OK  # nothing to do
    assert attn_status(Skv=1 << 30) == UNSUPPORTED
