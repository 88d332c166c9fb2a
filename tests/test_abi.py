"""C-ABI host tests (CPU only): the library loads, exports every symbol the
header declares, and rejects every host-checkable fault before any HIP call."""
import ctypes
import os
import re

import numpy as np
import pytest

import block_sparse_video_cube_amd as V
from block_sparse_video_cube_amd import _native as N

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vsa.h")
HEADERS = [os.path.join(ROOT, "include", h) for h in sorted(os.listdir(os.path.join(ROOT, "include")))
           if h.endswith(".h")]

OK, NULL, SHAPE, HEAD_DIM, DTYPE, TOPK, ALIGN, WORKSPACE, INDEX, UNSUP, HIP, SCALE = range(12)


def header_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(vsa_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_every_declared_symbol_is_exported_and_bound():
    lib = N.lib()
    names = header_functions()
    assert len(names) >= 17
    for name in names:
        assert hasattr(lib, name), name
        assert name in N.SIGNATURES, name
    assert set(N.SIGNATURES) == set(names)


def test_status_strings_and_version():
    lib = N.lib()
    for s in range(12):
        assert lib.vsa_status_string(s)
    assert lib.vsa_status_string(99) == b"unknown status"
    assert lib.vsa_version() == 100
    assert lib.vsa_max_cubes() >= 8192          # the 720p latent fits, and latents of 500k tokens


def _p(**kw):
    base = dict(B=1, heads=2, T=8, H=8, W=8, head_dim=64, dtype="bf16", topk=2)
    base.update(kw)
    return V.Problem(**base)


FAKE = ctypes.c_void_p(4096)          # aligned, never dereferenced (validation fails first)
MIS = ctypes.c_void_p(4096 + 4)


def _fwd(p, **ptrs):
    args = dict(q=FAKE, k=FAKE, v=FAKE, g_c=None, g_f=None, idx=FAKE, len=FAKE, o=FAKE, saved=None,
                ws=FAKE)
    args.update(ptrs)
    ws_bytes = ptrs.pop("ws_bytes", None)
    if ws_bytes is None:
        ws_bytes = V.workspace_bytes(p) if V.workspace_bytes(p) else 1 << 40
    # Every call below must fail validation: a success would launch on fake pointers.
    return N.lib().vsa_forward(ctypes.byref(p.c()), args["q"], args["k"], args["v"], args["g_c"], args["g_f"],
                               args["idx"], args["len"], args["o"], args["saved"], args["ws"], ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), SHAPE), (dict(heads=0), SHAPE), (dict(T=6), SHAPE), (dict(W=0), SHAPE), (dict(H=-4), SHAPE),
    (dict(head_dim=96), HEAD_DIM), (dict(head_dim=32), HEAD_DIM), (dict(dtype="f16"), DTYPE),
    (dict(topk=9), TOPK), (dict(topk=-1), TOPK), (dict(topk=0, list_stride=0), TOPK),
    (dict(topk=0, list_stride=9), TOPK), (dict(topk=4, list_stride=3), TOPK),
    (dict(scale=-1.0), SCALE), (dict(scale=float("nan")), SCALE), (dict(scale=float("inf")), SCALE),
    (dict(T=4, H=4 * 64, W=4 * 129), UNSUP),      # Nc = 8256 > vsa_max_cubes()
    (dict(pool="median"), UNSUP),                 # unknown pool_mode
    (dict(layout="zorder"), UNSUP),               # unknown layout
])
def test_problem_validation(kw, code):
    p = _p(**kw)
    assert _fwd(p) == code
    assert V.workspace_bytes(p) == 0 and V.saved_bytes(p) == 0


def test_tile_validation():
    lib = N.lib()
    c = ctypes.byref(_p().c())
    assert lib.vsa_tile(c, FAKE, None, None) == NULL
    assert lib.vsa_untile(c, MIS, FAKE, None) == ALIGN
    assert lib.vsa_tile(c, FAKE, FAKE, None) == UNSUP   # in place


def test_compatible_latent_host():
    lib = N.lib()
    o = [ctypes.c_int32() for _ in range(3)]
    refs = [ctypes.byref(v) for v in o]
    assert lib.vsa_compatible_latent(9, 13, 30, 0, 0, 0, *refs) == OK
    assert [v.value for v in o] == [12, 16, 32]
    assert lib.vsa_compatible_latent(24, 44, 80, 4, 4, 4, *refs) == OK
    assert [v.value for v in o] == [24, 44, 80]
    assert lib.vsa_compatible_latent(9, 13, 30, 2, 8, 8, *refs) == OK
    assert [v.value for v in o] == [10, 16, 32]
    assert lib.vsa_compatible_latent(0, 4, 4, 0, 0, 0, *refs) == SHAPE
    assert lib.vsa_compatible_latent(4, 4, 4, 3, 4, 4, *refs) == SHAPE      # not a power of two
    assert lib.vsa_compatible_latent(2**31 - 1, 4, 4, 0, 0, 0, *refs) == SHAPE
    assert lib.vsa_compatible_latent(4, 4, 4, 0, 0, 0, None, refs[1], refs[2]) == NULL


def test_crop_pad_validation():
    lib = N.lib()
    c = ctypes.byref(_p().c())                      # compatible grid 8 x 8 x 8
    other = ctypes.c_void_p(8192)
    assert lib.vsa_crop(c, FAKE, 9, 8, 8, other, None) == SHAPE
    assert lib.vsa_crop(c, FAKE, 5, 0, 8, other, None) == SHAPE
    assert lib.vsa_pad(c, None, 5, 5, 5, other, None) == NULL
    assert lib.vsa_pad(c, FAKE, 5, 5, 5, MIS, None) == ALIGN
    assert lib.vsa_crop(c, FAKE, 5, 5, 5, FAKE, None) == UNSUP   # in place
    assert lib.vsa_crop(ctypes.byref(_p(T=7).c()), FAKE, 5, 5, 5, other, None) == SHAPE


@pytest.mark.parametrize("cube,ok", [((4, 4, 4), True), ((2, 4, 4), True), ((4, 4, 8), True), ((1, 8, 8), True),
                                     ((8, 4, 4), True), ((2, 2, 8), True), ((4, 8, 2), False), ((3, 4, 4), False),
                                     ((2, 2, 4), False), ((4, 8, 8), True), ((1, 16, 16), True),
                                     ((8, 8, 8), False), ((2, 16, 16), False)])
def test_cube_shapes(cube, ok):
    """Cube sides: powers of two with Cw >= 4 and 32, 64, 128 or 256 tokens."""
    p = _p(T=8, H=16, W=16, cube=cube, topk=1)
    bt = cube[0] * cube[1] * cube[2]
    got = N.lib().vsa_workspace_bytes(ctypes.byref(p.c()), 0)
    assert (got > 0) == ok
    if ok:
        assert p.Nc == 8 * 16 * 16 // bt
    else:
        st = N.lib().vsa_forward(ctypes.byref(p.c()), *([FAKE] * 8), None, FAKE, 1 << 30, None)
        assert st in (SHAPE, UNSUP)


@pytest.mark.parametrize("kcube,ok", [((2, 4, 4), True), ((4, 4, 8), True), ((1, 8, 4), True), ((4, 4, 4), True),
                                      ((1, 4, 4), True), ((2, 2, 4), True), ((1, 1, 16), True),
                                      ((1, 2, 4), False), ((4, 2, 2), False), ((3, 4, 4), False),
                                      ((8, 4, 8), True), ((0, 4, 4), False), ((8, 8, 8), False)])
def test_key_block_shapes(kcube, ok):
    """Key blocks of their own shape (Bq x Bk tiles): powers of two, Cw >= 4,
    16 to 256 tokens, and all-zero sides mean the query cube."""
    p = _p(T=8, H=16, W=16, topk=1, kcube=kcube)
    got = N.lib().vsa_workspace_bytes(ctypes.byref(p.c()), 0)
    assert (got > 0) == ok
    if ok:
        assert p.Nk == 8 * 16 * 16 // (kcube[0] * kcube[1] * kcube[2])


def test_key_blocks_set_list_bounds_and_sizes():
    lib = N.lib()
    # 64-token query cubes, 32-token key blocks: Nq = 32, Nk = 64 at 8x16x16.
    p = _p(T=8, H=16, W=16, topk=64, kcube=(2, 4, 4))
    assert p.Nc == 32 and p.Nk == 64
    assert lib.vsa_workspace_bytes(ctypes.byref(p.c()), 0) > 0              # topk up to Nk
    assert lib.vsa_workspace_bytes(ctypes.byref(_p(T=8, H=16, W=16, topk=65, kcube=(2, 4, 4)).c()), 0) == 0
    # Same query cubes, 128-token key blocks: topk bound drops to Nk = 16.
    assert lib.vsa_workspace_bytes(ctypes.byref(_p(T=8, H=16, W=16, topk=17, kcube=(4, 4, 8)).c()), 0) == 0
    # Saved buffer holds K_c, V_c per key block: more key blocks, more bytes.
    base = _p(T=8, H=16, W=16, topk=4)
    assert V.saved_bytes(p) > V.saved_bytes(base)
    assert V.workspace_bytes(p, True) > V.workspace_bytes(base, True)
    # The all-zero key block is the query cube.
    assert V.saved_bytes(_p(T=8, H=16, W=16, topk=4, kcube=(4, 4, 4))) == V.saved_bytes(base)
    # One cube-major order: tiled layout needs key blocks = cubes.
    t = _p(T=8, H=16, W=16, topk=4, kcube=(2, 4, 4), layout="tiled")
    st = lib.vsa_forward(ctypes.byref(t.c()), *([FAKE] * 8), None, FAKE, 1 << 30, None)
    assert st == UNSUP


def test_check_lists_host_uses_key_block_range():
    p = V.Problem(1, 1, 8, 8, 8, 64, topk=0, list_stride=4, kcube=(2, 4, 4))   # Nq = 8, Nk = 16
    idx = np.array([[0, 9, 15, 0]] * 8, np.int32).reshape(1, 1, 8, 4)
    lens = np.full((1, 1, 8), 3, np.int32)
    V.check_lists_host(p, idx, lens)
    idx[0, 0, 3, 2] = 16
    with pytest.raises(V.VsaError) as e:
        V.check_lists_host(p, idx, lens)
    assert e.value.status == INDEX


def test_cube_must_divide_latent():
    p = _p(T=6, H=8, W=8, cube=(4, 4, 4))
    assert N.lib().vsa_workspace_bytes(ctypes.byref(p.c()), 0) == 0
    p = _p(T=6, H=8, W=8, cube=(2, 4, 8), topk=1)
    assert N.lib().vsa_workspace_bytes(ctypes.byref(p.c()), 0) > 0


def test_max_pool_problem_is_valid():
    p = _p(pool="max")
    assert V.workspace_bytes(p) > 0 and V.saved_bytes(p) > 0
    assert V.workspace_bytes(p, training=True) >= V.workspace_bytes(_p(), training=True)


@pytest.mark.parametrize("name", ["q", "k", "v", "idx", "len", "o", "ws"])
def test_null_pointers(name):
    assert _fwd(_p(), **{name: None}) == NULL


@pytest.mark.parametrize("name", ["q", "k", "v", "g_c", "g_f", "idx", "len", "o", "saved", "ws"])
def test_misaligned_pointers(name):
    assert _fwd(_p(), **{name: MIS}) == ALIGN


def test_workspace_too_small():
    p = _p()
    assert _fwd(p, ws_bytes=V.workspace_bytes(p) - 1) == WORKSPACE


def test_null_problem():
    lib = N.lib()
    assert lib.vsa_forward(None, *([FAKE] * 10), 0, None) == NULL
    assert lib.vsa_workspace_bytes(None, 0) == 0


def test_backward_checks_both_dtypes():
    lib = N.lib()
    for dt in ("bf16", "f32"):
        pb = _p(dtype=dt)
        args = [FAKE] * 7 + [None] + [FAKE] * 7 + [1 << 40, None]      # saved NULL
        assert lib.vsa_backward(ctypes.byref(pb.c()), *args) == NULL
        args = [FAKE] * 15 + [V.workspace_bytes(pb, True) - 1, None]
        assert lib.vsa_backward(ctypes.byref(pb.c()), *args) == WORKSPACE
        args = [FAKE] * 17 + [V.workspace_bytes(pb, True) - 1, None]
        assert lib.vsa_fine_backward(ctypes.byref(pb.c()), *args) == WORKSPACE


def test_stage_entry_points_validate():
    lib = N.lib()
    p = _p()
    c = ctypes.byref(p.c())
    assert lib.vsa_pool(c, FAKE, FAKE, None, FAKE, FAKE, FAKE, None) == NULL
    assert lib.vsa_pool(c, FAKE, FAKE, FAKE, FAKE, MIS, FAKE, None) == ALIGN
    assert lib.vsa_coarse(c, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, 1 << 40, None) == NULL  # top-K needs idx
    assert lib.vsa_coarse(c, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, None) == WORKSPACE
    assert lib.vsa_fine_forward(c, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, None) == WORKSPACE
    assert lib.vsa_fine_forward(c, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None) == NULL
    assert lib.vsa_combine(c, FAKE, MIS, None, None, FAKE, None) == ALIGN
    assert lib.vsa_combine_backward(c, FAKE, FAKE, FAKE, None, None, None, None, FAKE, FAKE, None, None) == NULL
    assert lib.vsa_combine_backward(c, FAKE, FAKE, FAKE, None, None, None, None, FAKE, FAKE, MIS, None) == ALIGN
    assert lib.vsa_index_transpose(c, FAKE, FAKE, None, FAKE, FAKE, 1 << 40, None) == NULL
    assert lib.vsa_index_transpose(c, FAKE, FAKE, FAKE, FAKE, FAKE, 1, None) == WORKSPACE
    assert lib.vsa_fine_backward(c, *([FAKE] * 17), 1, None) == WORKSPACE
    assert lib.vsa_coarse_backward(c, *([FAKE] * 10), 1, None) == WORKSPACE
    assert lib.vsa_validate_lists(c, FAKE, FAKE, None, None) == NULL
    bad = ctypes.byref(_p(head_dim=80).c())
    assert lib.vsa_pool(bad, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == HEAD_DIM


def test_workspace_and_saved_sizes_scale_with_problem():
    small = _p()
    big = _p(heads=4)
    assert V.workspace_bytes(big) > V.workspace_bytes(small) > 0
    assert V.saved_bytes(big) > V.saved_bytes(small) > 0
    assert V.workspace_bytes(small, True) >= V.workspace_bytes(small)
    p720 = V.Problem(1, 40, 24, 44, 80, 128, topk=32)
    # V T-tiles (bf16 N*d per head) dominate the inference workspace
    assert V.workspace_bytes(p720) >= 40 * 1320 * 1320 * 4   # the coarse logits


def test_check_lists_host():
    p = V.Problem(1, 1, 8, 8, 8, 64, topk=0, list_stride=4)
    idx = np.array([[0, 2, 5, -1]] * 8, np.int32).reshape(1, 1, 8, 4)
    lens = np.full((1, 1, 8), 3, np.int32)
    V.check_lists_host(p, idx, lens)
    lens0 = lens.copy(); lens0[0, 0, 3] = 0
    V.check_lists_host(p, idx, lens0)                     # empty row is valid
    for mutate in ("dup", "unsorted", "range", "neg", "len"):
        i2, l2 = idx.copy(), lens.copy()
        if mutate == "dup": i2[0, 0, 1, 1] = 0
        if mutate == "unsorted": i2[0, 0, 2, :3] = [5, 2, 0]
        if mutate == "range": i2[0, 0, 7, 2] = 8
        if mutate == "neg": i2[0, 0, 4, 0] = -1
        if mutate == "len": l2[0, 0, 6] = 5
        with pytest.raises(V.VsaError) as e:
            V.check_lists_host(p, i2, l2)
        assert e.value.status == INDEX


def test_noalloc_rejects_problems_beyond_its_scratch():
    """vsa_fine_combine_noalloc refuses B * heads * Nc above 1,048,576 (its
    static scratch) before any HIP call, and checks pointers like the others."""
    lib = N.lib()
    p = V.Problem(1, 1024, 32, 64, 64, 64, topk=0, list_stride=32)   # 1024 heads x 2048 cubes
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, None, None, None]
    assert lib.vsa_fine_combine_noalloc(ctypes.byref(p.c()), *args) == WORKSPACE
    small = _p(topk=0, list_stride=2)
    bad = list(args)
    bad[0] = None
    assert lib.vsa_fine_combine_noalloc(ctypes.byref(small.c()), *bad) == NULL
    bad = list(args)
    bad[1] = MIS
    assert lib.vsa_fine_combine_noalloc(ctypes.byref(small.c()), *bad) == ALIGN


def test_probe_arguments_rejected_on_the_host():
    """The measurement aids reject bad arguments before any HIP call."""
    lib = N.lib()
    buf = ctypes.c_void_p(16)   # never dereferenced: every call below fails its host checks
    assert lib.vsa_probe_mfma_valu(4, 0, 1, 10, None, None) == NULL
    assert lib.vsa_probe_mfma_valu(3, 0, 1, 10, buf, None) == UNSUP
    assert lib.vsa_probe_mfma_valu(4, 2, 1, 10, buf, None) == UNSUP
    assert lib.vsa_probe_mfma_valu(4, 0, 3, 10, buf, None) == UNSUP
    assert lib.vsa_probe_mfma_valu(4, 0, 2, 0, buf, None) == SHAPE
    assert lib.vsa_probe_stream_read(None, 1024, 4, 4, 0, buf, None) == NULL
    assert lib.vsa_probe_stream_read(ctypes.c_void_p(8), 1024, 4, 4, 0, buf, None) == ALIGN
    assert lib.vsa_probe_stream_read(buf, 1000, 4, 4, 0, buf, None) == ALIGN
    assert lib.vsa_probe_stream_read(buf, 0, 4, 4, 0, buf, None) == SHAPE
    assert lib.vsa_probe_stream_read(buf, 1024, 0, 4, 0, buf, None) == SHAPE
    assert lib.vsa_probe_stream_read(buf, 1024, 4, 3, 0, buf, None) == UNSUP
    assert lib.vsa_probe_stream_read(buf, 1024, 4, 4, 2, buf, None) == UNSUP
    assert lib.vsa_probe_l2_to_lds(0, None, 1 << 21, 4, 4, buf, None) == NULL
    assert lib.vsa_probe_l2_to_lds(0, buf, 1 << 21, 4, 4, None, None) == NULL
    assert lib.vsa_probe_l2_to_lds(0, ctypes.c_void_p(8), 1 << 21, 4, 4, buf, None) == ALIGN
    assert lib.vsa_probe_l2_to_lds(0, buf, 3 << 20, 4, 4, buf, None) == SHAPE
    assert lib.vsa_probe_l2_to_lds(0, buf, 8192, 4, 4, buf, None) == SHAPE
    assert lib.vsa_probe_l2_to_lds(0, buf, 1 << 21, 0, 4, buf, None) == SHAPE
    assert lib.vsa_probe_l2_to_lds(0, buf, 1 << 21, 4, 0, buf, None) == SHAPE
    assert lib.vsa_probe_l2_to_lds(2, buf, 1 << 21, 4, 4, buf, None) == UNSUP
