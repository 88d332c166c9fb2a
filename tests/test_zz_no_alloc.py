"""vsa_fine_combine_noalloc (the fine + combine entry point that allocates
nothing and keeps its scratch in a static device array) against
vsa_fine_combine on the same inputs, both called through the C ABI: two calls
in a row, the second on a smaller problem (the scratch keeps the first
call's contents). The two run the same kernels, so the results must agree
bit for bit."""
import ctypes

import numpy as np
import pytest
import torch

import block_sparse_video_cube_amd as V
import workloads as WL
from block_sparse_video_cube_amd import _native as N

DEV = "cuda:0"


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _case(B, heads, T, H, W, d, stride, seed):
    x = WL.make_inputs_custom(B, heads, d, T, H, W, dtype="bf16", seed=seed)
    nc = T * H * W // 64
    idx, lens = WL.random_lists(nc, B * heads * nc, 0, min(stride, nc), seed=seed, stride=stride)
    p = V.Problem(B, heads, T, H, W, d, topk=0, list_stride=stride)
    t = {k: torch.from_numpy(x[k]).to(DEV).to(torch.bfloat16).contiguous() for k in ("q", "k", "v", "g_c", "g_f")}
    t["idx"] = torch.from_numpy(idx.reshape(B, heads, nc, stride)).to(DEV)
    t["len"] = torch.from_numpy(lens.reshape(B, heads, nc)).to(DEV)
    gen = torch.Generator(device=DEV).manual_seed(seed)
    t["o_c"] = torch.randn((B, heads, nc, d), generator=gen, device=DEV, dtype=torch.float32)
    return p, t


def _run(p, t, noalloc):
    lib = N.lib()
    o = torch.empty_like(t["q"])
    of = torch.empty_like(t["q"])
    lse = torch.empty(t["q"].shape[:-1], dtype=torch.float32, device=DEV)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    args = [ctypes.byref(p.c()), *(_ptr(t[k]) for k in ("q", "k", "v", "idx", "len", "o_c", "g_c", "g_f")),
            _ptr(o), _ptr(of), _ptr(lse)]
    if noalloc:
        st = lib.vsa_fine_combine_noalloc(*args, stream)
    else:
        ws = torch.empty(V.workspace_bytes(p), dtype=torch.uint8, device=DEV)
        st = lib.vsa_fine_combine(*args, _ptr(ws), ws.numel(), stream)
    assert st == 0, N.STATUS_NAMES.get(st, st)
    torch.cuda.synchronize()
    return o, of, lse


@pytest.mark.gpu
def test_noalloc_matches_fine_combine_twice():
    cases = [(1, 4, 16, 32, 32, 128, 48, 5),   # 1024 query cubes
             (1, 2, 8, 16, 16, 64, 16, 6)]     # smaller: 64 query cubes
    for B, heads, T, H, W, d, stride, seed in cases:
        print(f"[noalloc] B={B} heads={heads} {T}x{H}x{W} d={d} stride={stride} seed={seed}", flush=True)
        p, t = _case(B, heads, T, H, W, d, stride, seed)
        ref = _run(p, t, noalloc=False)
        got = _run(p, t, noalloc=True)
        for a, b, name in zip(got, ref, ("o", "o_f", "lse_f")):
            assert torch.equal(a, b), name
