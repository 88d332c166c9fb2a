"""Seeded synthetic inputs for the VSA operator.

This module is shared by the CPU oracle and by the HIP path's tests and
benchmark. It draws random numbers and rounds them to bf16; it holds none
of the method's arithmetic (no pooling, no attention, no selection).

Every tensor is drawn from its own numpy ``default_rng([seed, stream, b, h])``
stream, so a single (b, h) slice of a large workload can be regenerated on its
own and is bit-identical to the same slice of the full tensor.

Stream ids: Q=0, K=1, V=2, G_c=3, G_f=4, spikes=5, low-rank=6, lists=7, dO=8.

Layout of every float tensor: [B, heads, T, H, W, d] (raster token order),
returned as float32 arrays. For bf16 workloads every value is exactly
representable in bf16 (rounded once, round-to-nearest-even), so the GPU path
(which casts to torch.bfloat16) and the oracle (which casts to float64) see
identical values.

The workloads stand in for the video-DiT settings the VSA pages describe
(pseudocode shape 16x32x32 with top-32, Wan-1.3B-like heads and head_dim,
a 720p long sequence); the pages' own data (generated videos, VBench) is not
available and is not reproduced.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import Dict, Optional, Sequence

import numpy as np

STREAM_Q, STREAM_K, STREAM_V, STREAM_GC, STREAM_GF = 0, 1, 2, 3, 4
STREAM_SPIKE, STREAM_LOWRANK, STREAM_LISTS, STREAM_DO = 5, 6, 7, 8

CUBE = 4  # cube edge along T, H and W
TILE = CUBE * CUBE * CUBE  # tokens per cube


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    heads: int
    head_dim: int
    T: int
    H: int
    W: int
    dtype: str  # "f32" or "bf16"
    topk: int  # > 0: top-K selection; 0: explicit lists
    values: str  # "scaled_normal", "spikes", "lowrank", "normal"
    backward: bool = False
    list_min: int = 0
    list_max: int = 0
    description: str = ""

    @property
    def N(self) -> int:
        return self.T * self.H * self.W

    @property
    def Nc(self) -> int:
        return self.N // TILE

    @property
    def list_stride(self) -> int:
        return self.topk if self.topk > 0 else self.list_max


WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("tiny_fp32_8x8x8", 1, 2, 64, 8, 8, 8, "f32", 2, "scaled_normal",
                 description="B=1 h=2 d=64, 8x8x8 latent (512 tokens, 8 cubes), top-2, fp32"),
        Workload("bf16_16x32x32_spikes", 1, 12, 64, 16, 32, 32, "bf16", 32, "spikes",
                 description="B=1 h=12 d=64, 16x32x32 latent (16384 tokens, 256 cubes), "
                             "top-32, 1% key spikes"),
        Workload("bf16_480p_20x28x52", 1, 12, 128, 20, 28, 52, "bf16", 32, "lowrank",
                 description="B=1 h=12 d=128, 20x28x52 latent (29120 tokens, 455 cubes), "
                             "top-32, rank-4 shared component"),
        Workload("bf16_720p_24x44x80", 1, 40, 128, 24, 44, 80, "bf16", 32, "lowrank",
                 description="B=1 h=40 d=128, 24x44x80 latent (84480 tokens, 1320 cubes), "
                             "top-32, rank-4 shared component"),
        Workload("train_bf16_16x32x32_varlen", 2, 12, 64, 16, 32, 32, "bf16", 0, "normal",
                 backward=True, list_min=8, list_max=64,
                 description="B=2 h=12 d=64, 16x32x32 latent, per-query-cube KV lists of "
                             "length U{8..64}, forward + backward"),
    ]
}

# Short aliases in the order the workloads are listed above.
ALIASES = {"C1": "tiny_fp32_8x8x8", "C2": "bf16_16x32x32_spikes", "C3": "bf16_480p_20x28x52",
           "C4": "bf16_720p_24x44x80", "C5": "train_bf16_16x32x32_varlen"}


def get(name: str) -> Workload:
    return WORKLOADS[ALIASES.get(name, name)]


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32."""
    u = np.array(x, dtype=np.float32, copy=True, order="C").view(np.uint32)
    lsb = u >> np.uint32(16)
    lsb &= np.uint32(1)
    lsb += np.uint32(0x7FFF)
    u += lsb
    u &= np.uint32(0xFFFF0000)
    return u.view(np.float32)


def _rng(seed: int, stream: int, b: int, h: int) -> np.random.Generator:
    return np.random.default_rng([seed, stream, b, h])


def _normal(seed: int, stream: int, b: int, h: int, shape) -> np.ndarray:
    return _rng(seed, stream, b, h).standard_normal(shape, dtype=np.float32)


def _uniform(seed: int, stream: int, b: int, h: int, shape) -> np.ndarray:
    return _rng(seed, stream, b, h).random(shape, dtype=np.float32)


def _head_qkv(w: Workload, seed: int, b: int, h: int):
    shape = (w.T, w.H, w.W, w.head_dim)
    q = _normal(seed, STREAM_Q, b, h, shape)
    k = _normal(seed, STREAM_K, b, h, shape)
    v = _normal(seed, STREAM_V, b, h, shape)
    if w.values == "scaled_normal":
        q /= 8.0
        k /= 8.0
        v /= 8.0
    elif w.values == "spikes":
        # 1% of key positions (rounded to nearest), uniform without replacement,
        # get +3.0 on every channel: "+3 sigma" spikes on unit-variance keys.
        n_spk = int(np.floor(0.01 * w.N + 0.5))
        pos = _rng(seed, STREAM_SPIKE, b, h).choice(w.N, size=n_spk, replace=False)
        k.reshape(w.N, w.head_dim)[pos] += np.float32(3.0)
    elif w.values == "lowrank":
        # Rank-4 component shared by Q, K and V of one head: one N(0,1) 4-vector per
        # cube, repeated over the cube's 64 tokens, times per-tensor loadings
        # W_X ~ N(0, 1/4) of shape [4, d] (adds unit variance per channel).
        g = _rng(seed, STREAM_LOWRANK, b, h)
        u_cube = g.standard_normal((w.Nc, 4), dtype=np.float32)
        loads = [g.standard_normal((4, w.head_dim), dtype=np.float32) * np.float32(0.5)
                 for _ in range(3)]
        u_grid = u_cube.reshape(w.T // CUBE, w.H // CUBE, w.W // CUBE, 4)
        for ax in range(3):  # spread each cube's vector over its 4x4x4 tokens
            u_grid = np.repeat(u_grid, CUBE, axis=ax)
        u_tok = u_grid.reshape(w.N, 4)
        for x, wx in zip((q, k, v), loads):
            x.reshape(w.N, w.head_dim)[...] += u_tok @ wx
    elif w.values != "normal":
        raise ValueError(w.values)
    if w.dtype == "bf16":
        q, k, v = round_bf16(q), round_bf16(k), round_bf16(v)
    return q, k, v


def _head_gates(w: Workload, seed: int, b: int, h: int):
    shape = (w.T, w.H, w.W, w.head_dim)
    gc = _uniform(seed, STREAM_GC, b, h, shape)
    gf = _uniform(seed, STREAM_GF, b, h, shape)
    if w.dtype == "bf16":
        gc, gf = round_bf16(gc), round_bf16(gf)
    return gc, gf


def _head_lists(w: Workload, seed: int, b: int, h: int):
    """Per query cube: length ~ U{list_min..list_max}, ascending distinct KV cubes."""
    g = _rng(seed, STREAM_LISTS, b, h)
    idx = np.full((w.Nc, w.list_max), -1, dtype=np.int32)
    lens = np.zeros(w.Nc, dtype=np.int32)
    for i in range(w.Nc):
        n = int(g.integers(w.list_min, w.list_max + 1))
        sel = np.sort(g.choice(w.Nc, size=n, replace=False))
        idx[i, :n] = sel
        lens[i] = n
    return idx, lens


def _head_dout(w: Workload, seed: int, b: int, h: int):
    d = _normal(seed, STREAM_DO, b, h, (w.T, w.H, w.W, w.head_dim))
    return round_bf16(d) if w.dtype == "bf16" else d


def make_inputs(name: str, seed: int = 0, heads: Optional[Sequence[int]] = None,
                batches: Optional[Sequence[int]] = None, gates: bool = True) -> dict:
    """Generate the inputs of a workload.

    heads / batches select a subset of (b, h) slices (default: all); the slices
    are identical to the same slices of the full tensors. Returns a dict with
    q, k, v (and g_c, g_f when ``gates``), idx/len for explicit-list workloads,
    d_o for backward workloads, and ``workload``.
    """
    w = get(name)
    hs = list(range(w.heads)) if heads is None else list(heads)
    bs = list(range(w.B)) if batches is None else list(batches)
    shp = (len(bs), len(hs), w.T, w.H, w.W, w.head_dim)
    out = {"workload": w, "heads": hs, "batches": bs}
    q = np.empty(shp, np.float32)
    k = np.empty(shp, np.float32)
    v = np.empty(shp, np.float32)
    if gates:
        gc = np.empty(shp, np.float32)
        gf = np.empty(shp, np.float32)
    if w.topk == 0:
        idx = np.empty((len(bs), len(hs), w.Nc, w.list_max), np.int32)
        lens = np.empty((len(bs), len(hs), w.Nc), np.int32)
    if w.backward:
        do = np.empty(shp, np.float32)
    def fill(bi_hi):
        bi, hi = bi_hi
        b, h = bs[bi], hs[hi]
        q[bi, hi], k[bi, hi], v[bi, hi] = _head_qkv(w, seed, b, h)
        if gates:
            gc[bi, hi], gf[bi, hi] = _head_gates(w, seed, b, h)
        if w.topk == 0:
            idx[bi, hi], lens[bi, hi] = _head_lists(w, seed, b, h)
        if w.backward:
            do[bi, hi] = _head_dout(w, seed, b, h)

    # Slices are independent streams, so filling them concurrently is
    # deterministic; numpy releases the GIL in the bulk draws and ufuncs.
    jobs = [(bi, hi) for bi in range(len(bs)) for hi in range(len(hs))]
    workers = max(1, min(len(jobs), 16, os.cpu_count() or 1))
    if workers == 1:
        for j in jobs:
            fill(j)
    else:
        with ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(fill, jobs))
    out.update(q=q, k=k, v=v)
    if gates:
        out.update(g_c=gc, g_f=gf)
    if w.topk == 0:
        out.update(idx=idx, len=lens)
    if w.backward:
        out.update(d_o=do)
    return out


def make_inputs_custom(B: int, heads: int, head_dim: int, T: int, H: int, W: int,
                       dtype: str = "bf16", seed: int = 0, values: str = "normal",
                       scale: float = 1.0) -> dict:
    """Plain N(0,1)*scale inputs and U(0,1) gates for shapes outside the named
    workloads (edge-case tests). Same stream convention."""
    w = Workload("custom", B, heads, head_dim, T, H, W, dtype, 1, values)
    shp = (B, heads, T, H, W, head_dim)
    out = {}
    for key, stream, uni in (("q", STREAM_Q, False), ("k", STREAM_K, False),
                             ("v", STREAM_V, False), ("g_c", STREAM_GC, True),
                             ("g_f", STREAM_GF, True), ("d_o", STREAM_DO, False)):
        arr = np.empty(shp, np.float32)
        for b in range(B):
            for h in range(heads):
                if uni:
                    arr[b, h] = _uniform(seed, stream, b, h, shp[2:])
                else:
                    arr[b, h] = _normal(seed, stream, b, h, shp[2:]) * np.float32(scale)
        out[key] = round_bf16(arr) if dtype == "bf16" else arr
    out["workload"] = w
    return out


def random_lists(Nc: int, n_rows: int, lmin: int, lmax: int, seed: int, stride: Optional[int] = None):
    """Ascending distinct KV-cube lists with lengths U{lmin..lmax} for n_rows rows."""
    stride = lmax if stride is None else stride
    g = np.random.default_rng([seed, STREAM_LISTS, 9999])
    idx = np.full((n_rows, max(stride, 1)), -1, np.int32)
    lens = np.zeros(n_rows, np.int32)
    for i in range(n_rows):
        n = int(g.integers(lmin, lmax + 1))
        idx[i, :n] = np.sort(g.choice(Nc, size=n, replace=False))
        lens[i] = n
    return idx, lens
