"""Boundary checks that need no GPU: the C-ABI library loads, exports every
symbol include/gemvfp16.h declares, and its host-side argument validation
returns the documented status codes.  No call here reaches a kernel launch:
every call either fails validation or is a documented no-op (M or N == 0)."""
import ctypes
import os
import re

import pytest

import gemv_fp16_amd as gf

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gemvfp16.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(gf.LIB_PATH):
        from gemv_fp16_amd import build
        build.build()
    return gf.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_three_calls():
    names = declared_functions()
    for n in ("gemm_f16_nt", "gemm_f16_nt_splitk", "gemv_f16"):
        assert n in names


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert len(names) >= 14
    for n in names:
        assert hasattr(L, n), n
    assert sorted(names) == sorted(gf.EXPORTS)


def test_status_strings(L):
    for rc in (0, 1, 2, 3, 4):
        assert gf.status_string(rc).startswith(("GF_OK", "GF_ERR"))
    assert gf.status_string(99) == "unknown status"


FAKE = ctypes.c_void_p(0x10000)      # never dereferenced: every call below stops on the host
ODD = ctypes.c_void_p(0x10001)
NULL = ctypes.c_void_p(0)


def test_gemm_validation(L):
    s = NULL
    assert L.gemm_f16_nt(FAKE, FAKE, FAKE, -1, 4, 4, s) == gf.GF_ERR_INVALID_ARG
    assert L.gemm_f16_nt(FAKE, FAKE, FAKE, 4, -1, 4, s) == gf.GF_ERR_INVALID_ARG
    assert L.gemm_f16_nt(FAKE, FAKE, FAKE, 4, 4, -1, s) == gf.GF_ERR_INVALID_ARG
    assert L.gemm_f16_nt(NULL, FAKE, FAKE, 4, 4, 4, s) == gf.GF_ERR_INVALID_ARG
    assert L.gemm_f16_nt(FAKE, NULL, FAKE, 4, 4, 4, s) == gf.GF_ERR_INVALID_ARG
    assert L.gemm_f16_nt(FAKE, FAKE, NULL, 4, 4, 4, s) == gf.GF_ERR_INVALID_ARG
    assert L.gemm_f16_nt(ODD, FAKE, FAKE, 4, 4, 4, s) == gf.GF_ERR_INVALID_ARG
    assert L.gemm_f16_nt(FAKE, FAKE, ODD, 4, 4, 4, s) == gf.GF_ERR_INVALID_ARG
    # too large: M*K >= 2^31 elements
    assert L.gemm_f16_nt(FAKE, FAKE, FAKE, 65536, 4, 65536, s) == gf.GF_ERR_INVALID_ARG
    # empty outputs are no-ops, NULL allowed where the extent is empty
    assert L.gemm_f16_nt(NULL, FAKE, NULL, 0, 4, 4, s) == gf.GF_OK
    assert L.gemm_f16_nt(FAKE, NULL, NULL, 4, 0, 4, s) == gf.GF_OK
    assert L.gemm_f16_nt(NULL, NULL, NULL, 0, 0, 0, s) == gf.GF_OK


def test_gemm_cfg_validation(L):
    good = gf.GemmCfg(128, 128, 64, 2, 256, 1, 0)
    bad = gf.GemmCfg(128, 128, 48, 2, 256, 1, 0)
    illegal = gf.GemmCfg(256, 256, 64, 3, 256, 1, 0)  # 192 KiB of LDS
    badsched = gf.GemmCfg(128, 128, 64, 2, 256, 1, 1)  # ping-pong needs 512 threads
    assert L.gemm_f16_nt_cfg(FAKE, FAKE, FAKE, 4, 4, 4, None, NULL) == gf.GF_ERR_INVALID_ARG
    assert L.gemm_f16_nt_cfg(FAKE, FAKE, FAKE, 0, 4, 4, ctypes.byref(good), NULL) == gf.GF_OK
    assert L.gemm_f16_nt_cfg(FAKE, FAKE, FAKE, 0, 4, 4, ctypes.byref(bad), NULL) == gf.GF_ERR_UNSUPPORTED
    assert L.gemm_f16_nt_cfg(FAKE, FAKE, FAKE, 4, 4, 4, ctypes.byref(illegal), NULL) == gf.GF_ERR_UNSUPPORTED
    assert L.gemm_f16_nt_cfg(FAKE, FAKE, FAKE, 4, 4, 4, ctypes.byref(badsched), NULL) == gf.GF_ERR_UNSUPPORTED


def test_splitk_validation(L):
    s = NULL
    assert L.gemm_f16_nt_splitk(FAKE, FAKE, FAKE, 4, 4, 4, 0, s) == gf.GF_ERR_INVALID_ARG
    assert L.gemm_f16_nt_splitk(FAKE, FAKE, FAKE, 4, 4, 4, -3, s) == gf.GF_ERR_INVALID_ARG
    assert L.gemm_f16_nt_splitk(FAKE, FAKE, ctypes.c_void_p(0x10002), 4, 4, 4, 2, s) == gf.GF_ERR_INVALID_ARG
    assert L.gemm_f16_nt_splitk(FAKE, FAKE, FAKE, 0, 4, 4, 2, s) == gf.GF_OK
    ex = L.gemm_f16_nt_splitk_ex
    assert ex(FAKE, FAKE, FAKE, 4, 4, 4, 2, 7, NULL, 0, s) == gf.GF_ERR_INVALID_ARG      # bad mode
    assert ex(FAKE, FAKE, FAKE, 4, 4, 4, 2, gf.GF_SPLITK_TWOPASS, NULL, 0, s) == gf.GF_ERR_INVALID_ARG
    need = L.gemm_f16_nt_splitk_workspace_bytes(4, 4, 2)
    assert need == 2 * 4 * 4 * 4
    assert ex(FAKE, FAKE, FAKE, 4, 4, 4, 2, gf.GF_SPLITK_TWOPASS, FAKE, need - 1, s) == gf.GF_ERR_INVALID_ARG
    assert ex(FAKE, FAKE, FAKE, 4, 0, 4, 2, gf.GF_SPLITK_TWOPASS, NULL, 0, s) == gf.GF_OK
    assert L.gemm_f16_nt_splitk_workspace_bytes(-1, 4, 2) == 0
    assert L.gemm_f16_nt_splitk_workspace_bytes(4, 4, 0) == 0
    # the entry point that allocates nothing: its scratch limit, checked on the host
    na = L.gemm_f16_nt_splitk_noalloc
    assert L.gf_noalloc_scratch_bytes() == 64 << 20
    assert na(FAKE, FAKE, FAKE, 4096, 4096, 64, 2, s) == gf.GF_ERR_TOO_LARGE       # 128 MiB of partials
    assert na(FAKE, FAKE, FAKE, 1024, 1024, 64, 17, s) == gf.GF_ERR_TOO_LARGE
    assert na(FAKE, FAKE, FAKE, 4, 4, 4, 0, s) == gf.GF_ERR_INVALID_ARG
    assert na(FAKE, FAKE, FAKE, -1, 4, 4, 2, s) == gf.GF_ERR_INVALID_ARG
    assert na(FAKE, FAKE, ctypes.c_void_p(0x10002), 4, 4, 4, 2, s) == gf.GF_ERR_INVALID_ARG
    assert na(FAKE, FAKE, FAKE, 0, 4, 4, 2, s) == gf.GF_OK                          # empty C
    assert "64 MiB" in gf.status_string(gf.GF_ERR_TOO_LARGE)


def test_layout_validation(L):
    s = NULL
    assert L.gemm_f16(FAKE, FAKE, FAKE, 4, 4, 4, 2, 0, s) == gf.GF_ERR_INVALID_ARG     # bad flag
    assert L.gemm_f16(FAKE, FAKE, FAKE, 4, 4, 4, 0, -1, s) == gf.GF_ERR_INVALID_ARG
    assert L.gemm_f16_nn(FAKE, FAKE, FAKE, -1, 4, 4, s) == gf.GF_ERR_INVALID_ARG
    assert L.gemm_f16_tn(FAKE, NULL, FAKE, 4, 4, 4, s) == gf.GF_ERR_INVALID_ARG
    assert L.gemm_f16_nn(FAKE, FAKE, FAKE, 0, 4, 4, s) == gf.GF_OK                  # empty C
    cfg = gf.GemmCfg(128, 128, 64, 2, 256, 0, 0)          # schedule 0: no layout variants
    assert L.gemm_f16_cfg(FAKE, FAKE, FAKE, 4, 4, 4, 0, 1, ctypes.byref(cfg), s) == gf.GF_ERR_UNSUPPORTED
    assert L.gemm_f16_cfg(FAKE, FAKE, FAKE, 4, 4, 4, 0, 1, None, s) == gf.GF_ERR_INVALID_ARG


def test_skinny_validation(L):
    s = NULL
    sk = L.gemm_f16_nt_skinny
    assert sk(FAKE, FAKE, FAKE, 17, 64, 64, None, s) == gf.GF_ERR_UNSUPPORTED      # M > 16 needs K % 512 == 0
    assert sk(FAKE, FAKE, FAKE, 4, 64, 60, None, s) == gf.GF_ERR_UNSUPPORTED       # K % 8 != 0
    assert sk(ctypes.c_void_p(0x10002), FAKE, FAKE, 4, 64, 64, None, s) == gf.GF_ERR_UNSUPPORTED
    bad = gf.SkinnyCfg(3, 3, 8, 0)
    assert sk(FAKE, FAKE, FAKE, 4, 64, 64, ctypes.byref(bad), s) == gf.GF_ERR_UNSUPPORTED
    assert sk(FAKE, FAKE, FAKE, -1, 64, 64, None, s) == gf.GF_ERR_INVALID_ARG
    assert sk(FAKE, FAKE, NULL, 4, 0, 64, None, s) == gf.GF_OK                      # empty C
    assert len(gf.skinny_configs()) >= 4
    out = gf.SkinnyCfg()
    assert L.gf_skinny_config_get(-1, ctypes.byref(out)) == gf.GF_ERR_INVALID_ARG
    for m in (0, 65):
        assert L.gf_skinny_default_config(m, 64, 64, ctypes.byref(out)) == gf.GF_ERR_INVALID_ARG
    assert L.gf_skinny_default_config(40, 8192, 8192, ctypes.byref(out)) == gf.GF_OK
    assert (out.blocks, out.unroll, out.waves, out.stages) == (2, 0, 8, 2)      # 17..64 rows: LDS form
    assert gf.skinny_default_config(24, 4096, 8192) == {"blocks": 1, "unroll": 0, "waves": 8, "stages": 3}
    assert gf.skinny_default_config(64, 8192, 8192) == {"blocks": 1, "unroll": 0, "waves": 8, "stages": 2}
    assert sk(FAKE, FAKE, FAKE, 65, 64, 512, None, s) == gf.GF_ERR_UNSUPPORTED     # M > 64
    assert sk(FAKE, FAKE, FAKE, 40, 64, 1000, None, s) == gf.GF_ERR_UNSUPPORTED    # 17..64 rows need K % 512 == 0
    direct = gf.SkinnyCfg(1, 4, 8, 0)
    assert sk(FAKE, FAKE, FAKE, 40, 64, 512, ctypes.byref(direct), s) == gf.GF_ERR_UNSUPPORTED   # not the LDS form
    assert L.gf_skinny_default_config(4, 64, 64, None) == gf.GF_ERR_INVALID_ARG


def test_skinny_default_rule():
    """The skinny launch shape the library picks: every choice is compiled,
    and the shape-dependent choices hold."""
    compiled = gf.skinny_configs()
    for n in (64, 2048, 4096, 6144, 8192, 28672):
        for k in (64, 2048, 2560, 4096, 5120, 6144, 11008, 13824, 14336, 8192, 12288, 15360, 16384):
            for m in range(1, 17):
                assert gf.skinny_default_config(m, n, k) in compiled, (m, n, k)
    d = gf.skinny_default_config
    # 8192 x 8192: split form to M = 8, then three 16-row blocks through LDS
    assert d(1, 8192, 8192) == {"blocks": 512, "unroll": 4, "waves": 4, "stages": -1}
    assert d(8, 8192, 8192) == {"blocks": 512, "unroll": 4, "waves": 4, "stages": -1}
    assert d(16, 8192, 8192) == {"blocks": 3, "unroll": 0, "waves": 8, "stages": 2}
    # K = 16384: 4 waves with 8 chunks per lane to M = 4, 8 waves with 4 beyond
    assert d(4, 4096, 16384) == {"blocks": 512, "unroll": 8, "waves": 4, "stages": -1}
    assert d(5, 8192, 16384) == {"blocks": 256, "unroll": 4, "waves": 8, "stages": -1}
    # rows that do not split into whole 2048-chunk steps: the vector form with
    # a ragged last step for M <= 4 from K = 4096 (16 waves where N divides
    # the grid's 4096 waves evenly), the direct form for short rows
    assert d(1, 4096, 11008) == {"blocks": 1, "unroll": 4, "waves": 16, "stages": 1}
    assert d(2, 5120, 13824) == {"blocks": 1, "unroll": 4, "waves": 8, "stages": 1}
    assert d(4, 8192, 5120) == {"blocks": 1, "unroll": 4, "waves": 16, "stages": 1}
    assert d(4, 4096, 2560)["stages"] == 0
    assert d(8, 4096, 11008)["stages"] == 0
    # fewer than 4096 rows of B, or other K: the other forms
    assert d(2, 2048, 8192)["stages"] == 1
    assert d(8, 2048, 8192)["stages"] != -1
    assert d(8, 8192, 4096)["stages"] != -1
    # fewer rows of B: one block per workgroup through LDS from M = 5
    assert d(8, 4096, 14336) == {"blocks": 1, "unroll": 0, "waves": 16, "stages": 4}
    assert d(16, 6144, 6144) == {"blocks": 1, "unroll": 0, "waves": 8, "stages": 3}
    # and 16-wave vector workgroups for M <= 2 over a large B
    assert d(1, 4096, 14336) == {"blocks": 1, "unroll": 4, "waves": 16, "stages": 1}
    assert d(2, 2048, 8192)["waves"] == 8                   # 16 M elements: the 8-wave form
    assert d(4, 6144, 6144) == {"blocks": 1, "unroll": 4, "waves": 8, "stages": 1}
    # from 8192 rows of B with rows shorter than 8192: 16-wave vector workgroups for M <= 4
    # (also where K is not a multiple of 4096), one or two blocks per LDS workgroup beyond
    assert d(4, 28672, 4096) == {"blocks": 1, "unroll": 4, "waves": 16, "stages": 1}
    assert d(1, 12288, 6144) == {"blocks": 1, "unroll": 4, "waves": 16, "stages": 1}
    assert d(16, 16384, 4096) == {"blocks": 1, "unroll": 0, "waves": 8, "stages": 2}
    assert d(8, 8192, 2048) == {"blocks": 2, "unroll": 0, "waves": 8, "stages": 2}
    assert d(16, 8192, 2048) == {"blocks": 2, "unroll": 0, "waves": 8, "stages": 2}


def test_splitk_f16_validation(L):
    s = NULL
    f16 = L.gemm_f16_nt_splitk_f16
    need = L.gemm_f16_nt_splitk_workspace_bytes(4, 4, 2)
    assert f16(FAKE, FAKE, FAKE, 4, 4, 4, 0, FAKE, need, s) == gf.GF_ERR_INVALID_ARG     # split_k < 1
    assert f16(FAKE, FAKE, FAKE, -1, 4, 4, 2, FAKE, need, s) == gf.GF_ERR_INVALID_ARG
    assert f16(FAKE, FAKE, FAKE, 4, 4, 4, 2, NULL, need, s) == gf.GF_ERR_INVALID_ARG     # no workspace
    assert f16(FAKE, FAKE, FAKE, 4, 4, 4, 2, FAKE, need - 1, s) == gf.GF_ERR_INVALID_ARG
    assert f16(FAKE, FAKE, FAKE, 4, 4, 4, 2, ctypes.c_void_p(0x10002), need, s) == gf.GF_ERR_INVALID_ARG
    assert f16(FAKE, FAKE, ODD, 4, 4, 4, 2, FAKE, need, s) == gf.GF_ERR_INVALID_ARG      # C not 2-aligned
    assert f16(FAKE, FAKE, NULL, 0, 4, 4, 2, NULL, 0, s) == gf.GF_OK                    # empty output


def test_gemv_validation(L):
    s = NULL
    assert L.gemv_f16(FAKE, FAKE, FAKE, -1, 4, s) == gf.GF_ERR_INVALID_ARG
    assert L.gemv_f16(FAKE, FAKE, FAKE, 4, -1, s) == gf.GF_ERR_INVALID_ARG
    assert L.gemv_f16(NULL, FAKE, FAKE, 4, 4, s) == gf.GF_ERR_INVALID_ARG
    assert L.gemv_f16(FAKE, NULL, FAKE, 4, 4, s) == gf.GF_ERR_INVALID_ARG
    assert L.gemv_f16(FAKE, FAKE, NULL, 4, 4, s) == gf.GF_ERR_INVALID_ARG
    assert L.gemv_f16(FAKE, FAKE, ODD, 4, 4, s) == gf.GF_ERR_INVALID_ARG
    assert L.gemv_f16(NULL, NULL, NULL, 0, 4, s) == gf.GF_OK
    neg = gf.GemvCfg(1, 2, 4, -1)
    assert L.gemv_f16_cfg(FAKE, FAKE, FAKE, 4, 4, ctypes.byref(neg), s) == gf.GF_ERR_INVALID_ARG
    c = gf.GemvCfg(3, 3, 3, 0)
    assert L.gemv_f16_cfg(FAKE, FAKE, FAKE, 0, 4, ctypes.byref(c), s) == gf.GF_ERR_UNSUPPORTED
    assert L.gemv_f16_cfg(FAKE, FAKE, FAKE, 0, 4, None, s) == gf.GF_ERR_INVALID_ARG


def test_config_tables(L):
    cfgs = gf.gemm_configs()
    # 3x3x2x3x2 grid + deep BK=32 + ping-pong + one wave per SIMD
    assert len(cfgs) == 108 + 16 + 6 + 9
    assert sum(1 for c, ok in cfgs if ok and c["schedule"] == 1) >= 5
    assert sum(1 for c, ok in cfgs if ok and c["schedule"] in (2, 3)) == 9
    legal = [c for c, ok in cfgs if ok]
    assert len(legal) >= 90
    for c, ok in cfgs:
        lds = c["stages"] * (c["block_m"] + c["block_n"]) * c["block_k"] * 2
        if lds > 160 * 1024:
            assert not ok, c
        if c["stages"] > 4 and c["schedule"] != 2:
            assert not ok, c                      # only schedule 2 runs a 5-stage ring
    assert len(gf.gemv_configs()) >= 30
    d = gf.gemm_default_config(8192, 8192, 8192)
    assert (d["block_m"], d["block_n"]) == (256, 256)
    # short K: 512-thread tiles that leave room for more than one workgroup per CU
    assert gf.gemm_default_config(8192, 8192, 256) == dict(
        block_m=128, block_n=256, block_k=32, stages=3, threads=512, raster=0, schedule=0)
    assert gf.gemm_default_config(4096, 4096, 256) == dict(
        block_m=256, block_n=128, block_k=64, stages=1, threads=512, raster=0, schedule=0)
    assert gf.gemm_default_config(8192, 8192, 512)["block_n"] == 128
    assert gf.gemm_default_config(8192, 8192, 1024) == dict(
        block_m=256, block_n=256, block_k=64, stages=2, threads=512, raster=0, schedule=0)
    assert gf.gemm_default_config(8192, 8192, 2048)["threads"] == 256
    assert gf.gemm_default_config(2048, 2048, 256) == dict(
        block_m=64, block_n=128, block_k=64, stages=2, threads=256, raster=0, schedule=0)
    # mid-size shapes: the largest tile that still fills the 256 CUs
    d2 = gf.gemm_default_config(2048, 4096, 8192)
    assert (d2["block_m"], d2["block_n"], d2["stages"], d2["schedule"]) == (256, 128, 3, 2)
    d3 = gf.gemm_default_config(2048, 2048, 8192)
    assert (d3["block_m"], d3["block_n"], d3["stages"], d3["schedule"]) == (128, 128, 4, 2)
    d4 = gf.gemm_default_config(4096, 2048, 1024)        # short K: two 128 x 128 workgroups per CU
    assert (d4["block_m"], d4["block_n"], d4["stages"]) == (128, 128, 2)
    d5 = gf.gemm_default_config(1024, 1024, 4096)        # small: 64 x 64, three stages
    assert (d5["block_m"], d5["block_n"], d5["stages"]) == (64, 64, 3)
    assert any(c == {**d, "raster": 1} for c, ok in cfgs if ok)
    for c, ok in cfgs:
        if c["schedule"] == 1:
            assert c["threads"] == 512
        if c["schedule"] in (2, 3):
            assert c["threads"] == 256
    assert d["raster"] in (0, 1)
    # tile order of the one-wave-per-SIMD 256 x 256 kernel: grouped (panels of
    # 10 rows) to K = 4096, plain to K = 12288, panels of 4 rows from 16384
    assert [gf.gemm_default_config(8192, 8192, k)["raster"] for k in (2048, 4096, 8192, 12288, 16384, 32768)] == \
        [1, 1, 0, 0, 4, 4]
    dg = gf.gemv_default_config(8192, 8192)
    assert {**dg, "blocks": 0} in gf.gemv_configs() and dg["blocks"] >= 0
    assert dg["blocks"] > 0                                # tall W, K % 8192 == 0: the split form
    assert dg == {"rows_per_wave": 1, "unroll": 4, "waves": 4, "blocks": 512}
    dw = gf.gemv_default_config(4096, 16384)               # long rows: one row per split task
    assert dw == {"rows_per_wave": 1, "unroll": 2, "waves": 8, "blocks": 256}
    # K not a multiple of 8192: one row per wave, 8 chunks in flight when
    # rows split into whole 512-chunk steps, else 4
    assert gf.gemv_default_config(16384, 4096) == {"rows_per_wave": 1, "unroll": 8, "waves": 2, "blocks": 0}
    assert gf.gemv_default_config(4096, 14336) == {"rows_per_wave": 1, "unroll": 4, "waves": 4, "blocks": 0}
    for n, k in ((16384, 4096), (2048, 2048), (1024, 1024), (7, 13)):
        assert {**gf.gemv_default_config(n, k), "blocks": 0} in gf.gemv_configs()
    bad = gf.GemmCfg()
    assert L.gf_gemm_config_get(-1, ctypes.byref(bad)) == gf.GF_ERR_INVALID_ARG
    assert L.gf_gemm_config_get(len(cfgs), ctypes.byref(bad)) == gf.GF_ERR_INVALID_ARG


def test_sparse_validation(L):
    s = NULL
    c = L.sp24_compress_f16
    assert c(FAKE, FAKE, FAKE, 4, 24, s) == gf.GF_ERR_INVALID_ARG           # K % 16 != 0
    assert c(FAKE, FAKE, FAKE, -1, 32, s) == gf.GF_ERR_INVALID_ARG
    assert c(NULL, FAKE, FAKE, 4, 32, s) == gf.GF_ERR_INVALID_ARG
    assert c(FAKE, FAKE, ODD, 4, 32, s) == gf.GF_ERR_INVALID_ARG
    assert c(NULL, NULL, NULL, 0, 32, s) == gf.GF_OK                         # empty
    assert c(NULL, NULL, NULL, 4, 0, s) == gf.GF_OK
    g = L.gemm_sp_f16_nt
    assert g(FAKE, FAKE, FAKE, FAKE, 4, 4, 40, s) == gf.GF_ERR_INVALID_ARG   # K % 16 != 0
    assert g(FAKE, FAKE, FAKE, FAKE, -1, 4, 32, s) == gf.GF_ERR_INVALID_ARG
    assert g(FAKE, NULL, FAKE, FAKE, 4, 4, 32, s) == gf.GF_ERR_INVALID_ARG   # no metadata
    assert g(FAKE, FAKE, FAKE, ODD, 4, 4, 32, s) == gf.GF_ERR_INVALID_ARG
    assert g(FAKE, FAKE, FAKE, NULL, 0, 4, 32, s) == gf.GF_OK                # empty C
    assert g(FAKE, FAKE, FAKE, FAKE, 1 << 16, 4, 1 << 15, s) == gf.GF_ERR_INVALID_ARG   # 2^31 elements
    bad = gf.SpCfg(64, 64, 2, 0)
    assert L.gemm_sp_f16_nt_cfg(FAKE, FAKE, FAKE, FAKE, 4, 4, 32, ctypes.byref(bad), s) == gf.GF_ERR_UNSUPPORTED
    cfgs = gf.sp_configs()
    assert len(cfgs) == L.gf_sp_config_count() >= 4
    d = gf.sp_default_config(8192, 8192, 8192)
    assert {**d, "raster": 1} in cfgs
    # the paired form (stages = 0) is compiled for every tile shape; where
    # half-size tiles fill the chip but 256 x 256 ones do not, the default
    # is 128 x 256 with three stages
    assert {(c["block_m"], c["block_n"]) for c in cfgs if c["stages"] == 0} == \
        {(256, 256), (256, 128), (128, 256), (128, 128)}
    assert gf.sp_default_config(2048, 4096, 8192) == {"block_m": 128, "block_n": 256, "stages": 3, "raster": 1}
    assert gf.sp_default_config(4096, 4096, 8192)["stages"] == 3
    assert gf.sp_default_config(2048, 2048, 8192) == {"block_m": 128, "block_n": 128, "stages": 3, "raster": 1}
    out = gf.SpCfg()
    assert L.gf_sp_config_get(len(cfgs), ctypes.byref(out)) == gf.GF_ERR_INVALID_ARG


def test_every_default_tile_has_its_masked_and_fp32_variants():
    """Whatever tile the library picks for gemm_f16_nt must also run unaligned
    operands (its masked variant), so it must be one the config table marks
    for those variants: checked over a dense grid of shapes."""
    import itertools
    import re
    src = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                            "gemv_fp16_amd", "csrc", "gemm_configs.def")).read()
    core = {tuple(int(v) for v in m.groups()[:6])
            for m in re.finditer(r"^GF_GEMM\((\d+), (\d+), (\d+), (\d+), (\d+), (\d+), 1\)", src, re.M)}
    assert len(core) >= 10
    sizes = (17, 64, 256, 1000, 1024, 2048, 3072, 4096, 6144, 7168, 8192, 16384)
    ks = (8, 128, 256, 384, 512, 640, 1024, 1536, 2048, 4096, 8192, 16384)
    seen = set()
    for M, N, K in itertools.product(sizes, sizes, ks):
        d = gf.gemm_default_config(M, N, K)
        seen.add((d["block_m"], d["block_n"], d["block_k"], d["stages"], d["threads"], d["schedule"]))
    assert seen <= core, sorted(seen - core)
    assert len(seen) >= 7
