"""The build's M0 check on generated assembly (CPU only). The direct-to-LDS
loads of the fine kernels set M0 in inline assembly; the build rejects any
kernel in which the compiler itself uses M0. Planted violations in small
assembly texts must be found; the clean pattern must pass."""
import os

from block_sparse_video_cube_amd import build as B

GOOD = """
kern:
\ts_mov_b32 m0, s10
\ts_nop 0
\tglobal_load_lds_dwordx4 v1, s[6:7]
\tds_read_b128 v[2:5], v6
\ts_mov_b32 m0, vcc_lo   ; another load
\ts_nop 0
\tglobal_load_lds_dwordx4 v7, s[6:7]
\ts_endpgm
other:
\ts_mov_b32 m0, s1
\ts_sendmsg sendmsg(MSG_DEALLOC_VGPRS)
"""


def test_clean_pattern_passes():
    # `other` issues no direct-to-LDS load, so its own M0 use is not checked
    assert B.check_m0(GOOD) == []


def test_compiler_m0_use_is_found():
    bad = GOOD.replace("\tds_read_b128 v[2:5], v6\n", "\tv_movrels_b32 v2, v3\n\ts_mov_b32 m0, s4\n\tv_add_u32 v1, m0, v1\n")
    found = B.check_m0(bad)
    assert any("outside the direct-to-LDS loads" in f for f in found), found


def test_load_without_setup_is_found():
    bad = GOOD.replace("\ts_mov_b32 m0, s10\n\ts_nop 0\n", "")
    found = B.check_m0(bad)
    assert any("without its own M0 set-up" in f for f in found), found


def test_built_assembly_is_clean():
    """When the library has been built here, its kept assembly passes."""
    for src in B.M0_SOURCES:
        stem = os.path.splitext(src)[0]
        path = os.path.join(B.OBJ, f"{stem}-hip-amdgcn-amd-amdhsa-{B.ARCH}.s")
        if not os.path.exists(path):
            continue
        text = open(path).read()
        assert "global_load_lds_dwordx4" in text
        assert B.check_m0(text) == []
