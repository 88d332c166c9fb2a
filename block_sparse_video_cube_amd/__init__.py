"""VSA (Video Sparse Attention) coarse-fine attention on AMD MI355X (gfx950).

Thin binding over the C ABI of libvsa.so (include/vsa.h): it allocates the
output tensors with torch on the current device, passes raw pointers and the
current HIP stream, and checks the returned status. Every step of the
operator runs in the library's HIP kernels.

Tensors: q, k, v, gates, outputs are [B, heads, T, H, W, head_dim]
contiguous on the GPU, bf16 or fp32. Index lists are int32
[B, heads, Nc, list_stride] with lengths int32 [B, heads, Nc].
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional

import torch

from ._native import VSA_BF16, VSA_F32, VsaError, VsaProblem, check, lib

__all__ = ["Problem", "VsaError", "forward", "backward", "pool", "coarse", "fine_forward", "fine_combine", "fine_combine_noalloc", "combine",
           "combine_backward", "index_transpose", "fine_backward", "coarse_backward",
           "check_lists_host", "validate_lists", "workspace_bytes", "saved_bytes", "max_cubes", "tile", "untile",
           "compatible_latent", "crop", "pad", "saved_views", "attention", "probe_mfma_valu", "probe_stream_read",
           "probe_l2_to_lds"]


@dataclass(frozen=True)
class Problem:
    B: int
    heads: int
    T: int
    H: int
    W: int
    head_dim: int
    dtype: str = "bf16"          # "bf16" or "f32"
    topk: int = 32               # > 0: top-K mode; 0: explicit lists
    list_stride: int = 0         # 0 => topk
    scale: float = 0.0           # 0 => 1/sqrt(head_dim)
    pool: str = "mean"           # cube pooling of the coarse stage: "mean" or "max"
    layout: str = "raster"       # token order: "raster" [B,h,T,H,W,d] or "tiled" [B,h,Nc,Bt,d]
    cube: tuple = (4, 4, 4)      # cube sides (Ct, Ch, Cw); Bt = Ct*Ch*Cw tokens per tile
    kcube: Optional[tuple] = None  # key-block sides; None => the cube (Bq x Bk tiles otherwise)

    @property
    def N(self) -> int:
        return self.T * self.H * self.W

    @property
    def Bt(self) -> int:
        return self.cube[0] * self.cube[1] * self.cube[2]

    @property
    def Nc(self) -> int:
        return self.N // self.Bt

    @property
    def key_cube(self) -> tuple:
        return tuple(self.kcube) if self.kcube is not None else tuple(self.cube)

    @property
    def Bk(self) -> int:
        k = self.key_cube
        return k[0] * k[1] * k[2]

    @property
    def Nk(self) -> int:
        return self.N // self.Bk

    @property
    def stride(self) -> int:
        return self.list_stride if self.list_stride else self.topk

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    def c(self) -> VsaProblem:
        code = {"bf16": VSA_BF16, "f32": VSA_F32}.get(self.dtype, 99)
        pool = {"mean": 0, "max": 1}.get(self.pool, 99)
        layout = {"raster": 0, "tiled": 1}.get(self.layout, 99)
        return VsaProblem(self.B, self.heads, self.T, self.H, self.W, self.head_dim, code,
                          float(self.scale), self.topk, self.list_stride, pool, layout, *self.cube,
                          *(self.kcube if self.kcube is not None else (0, 0, 0)))


def _numel(shape) -> int:
    n = 1
    for e in shape:
        n *= int(e)
    return n


class _Args:
    """Checks every tensor handed to one library call before anything is
    launched: the C ABI receives bare pointers and cannot tell a CPU tensor,
    a wrong dtype or a short buffer from a good one, and a kernel given one
    would read or write outside it. Each tensor must be a contiguous tensor on
    the same HIP device as the call's first tensor, of the expected dtype and
    with exactly the expected number of elements (any shape with that count
    is accepted, e.g. [B, h, N] for a [B, h, T, H, W] per-token array).
    Violations raise ValueError. Wrappers pass the library function through
    call(), which checks the devices last."""

    def __init__(self, where: str):
        self.where = where
        self.tensors = []

    def _common(self, name: str, t) -> None:
        if not t.is_contiguous():
            raise ValueError(f"{self.where}: {name} must be contiguous")
        self.tensors.append((name, t))

    def call(self, fn, *args):
        """Checks that every tensor seen is on one HIP device, then calls fn.
        (The device check comes last so that dtype and size errors of every
        argument are reported first.)"""
        dev = None
        for name, t in self.tensors:
            if t.device.type != "cuda":
                raise ValueError(f"{self.where}: {name} must be on a HIP (cuda) device, got {t.device}")
            if dev is None:
                dev = t.device
            elif t.device != dev:
                raise ValueError(f"{self.where}: {name} is on {t.device}, the call's tensors on {dev}")
        return fn(*args)

    def t(self, name: str, t, shape, dtype, required: bool = True):
        """Pointer of tensor t of `shape` (its element count) and `dtype`;
        None passes through when not required."""
        if t is None:
            if required:
                raise ValueError(f"{self.where}: {name} is required")
            return None
        if not isinstance(t, torch.Tensor):
            raise ValueError(f"{self.where}: {name} must be a torch.Tensor, got {type(t).__name__}")
        if t.dtype != dtype:
            raise ValueError(f"{self.where}: {name} must be {dtype}, got {t.dtype}")
        if t.numel() != _numel(shape):
            raise ValueError(f"{self.where}: {name} has {t.numel()} elements ({tuple(t.shape)}), "
                             f"expected {_numel(shape)} ({tuple(shape)})")
        self._common(name, t)
        return ctypes.c_void_p(t.data_ptr())

    def buf(self, name: str, t, min_bytes: int, required: bool = True):
        """Pointer and byte size of a raw buffer (workspace, saved) of at
        least min_bytes."""
        if t is None:
            if required:
                raise ValueError(f"{self.where}: {name} is required")
            return None, 0
        if not isinstance(t, torch.Tensor):
            raise ValueError(f"{self.where}: {name} must be a torch.Tensor, got {type(t).__name__}")
        nbytes = t.numel() * t.element_size()
        if nbytes < min_bytes:
            raise ValueError(f"{self.where}: {name} holds {nbytes} bytes, needs {min_bytes}")
        self._common(name, t)
        return ctypes.c_void_p(t.data_ptr()), nbytes


def _stream(device) -> ctypes.c_void_p:
    if device.type != "cuda":   # rejected by _Args.call before any library call
        return ctypes.c_void_p(0)
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _empty(shape, dtype, like: torch.Tensor) -> torch.Tensor:
    return torch.empty(shape, dtype=dtype, device=like.device)


def workspace_bytes(p: Problem, training: bool = False) -> int:
    return int(lib().vsa_workspace_bytes(ctypes.byref(p.c()), int(training)))


def saved_bytes(p: Problem) -> int:
    return int(lib().vsa_saved_bytes(ctypes.byref(p.c())))


def max_cubes() -> int:
    return int(lib().vsa_max_cubes())


def workspace(p: Problem, like: torch.Tensor, training: bool = False) -> torch.Tensor:
    n = workspace_bytes(p, training)
    if n == 0:
        raise VsaError(2, "workspace_bytes")
    return torch.empty(n, dtype=torch.uint8, device=like.device)


def _raster(p: Problem):
    """Shape of a token tensor in the problem's layout."""
    if p.layout == "tiled":
        return (p.B, p.heads, p.Nc, p.Bt, p.head_dim)
    return (p.B, p.heads, p.T, p.H, p.W, p.head_dim)


def _tokens(p: Problem):
    """Shape of a per-token fp32 array (LSE_f, delta) in the problem's layout."""
    return _raster(p)[:-1]


def _full(p: Problem):
    """Raster shape [B, h, T, H, W, d] whatever the problem's layout."""
    return (p.B, p.heads, p.T, p.H, p.W, p.head_dim)


def _cubes(p: Problem):
    """Cube-major shape [B, h, Nc, Bt, d]."""
    return (p.B, p.heads, p.Nc, p.Bt, p.head_dim)


def _lists(p: Problem):
    return (p.B, p.heads, p.Nc, p.stride), (p.B, p.heads, p.Nc)


def tile(p: Problem, x):
    """Cube-major copy [B, h, Nc, Bt, d] of a raster token tensor."""
    a = _Args("vsa_tile")
    px = a.t("x", x, _full(p), p.torch_dtype)
    xt = _empty(_cubes(p), x.dtype, x)
    check(a.call(lib().vsa_tile, ctypes.byref(p.c()), px, a.t("xt", xt, _cubes(p), p.torch_dtype), _stream(x.device)),
          "vsa_tile")
    return xt


def untile(p: Problem, xt):
    """Raster copy [B, h, T, H, W, d] of a cube-major token tensor."""
    a = _Args("vsa_untile")
    pxt = a.t("xt", xt, _cubes(p), p.torch_dtype)
    x = _empty(_full(p), xt.dtype, xt)
    check(a.call(lib().vsa_untile, ctypes.byref(p.c()), pxt, a.t("x", x, _full(p), p.torch_dtype), _stream(xt.device)),
          "vsa_untile")
    return x


def compatible_latent(T: int, H: int, W: int, cube: tuple = (4, 4, 4)) -> tuple:
    """Smallest latent with sides that are multiples of the cube's containing T x H x W."""
    o = [ctypes.c_int32() for _ in range(3)]
    check(lib().vsa_compatible_latent(T, H, W, *cube, *(ctypes.byref(v) for v in o)), "vsa_compatible_latent")
    return tuple(v.value for v in o)


def crop(p: Problem, x, T: int, H: int, W: int):
    """Raster [B, h, T, H, W, d] copy of the leading region of a token tensor of p (p's layout)."""
    a = _Args("vsa_crop")
    px = a.t("x", x, _raster(p), p.torch_dtype)
    shape = (p.B, p.heads, T, H, W, p.head_dim)
    if min(T, H, W) < 1:
        raise ValueError(f"vsa_crop: region {T}x{H}x{W} is empty")
    out = _empty(shape, x.dtype, x)
    check(a.call(lib().vsa_crop, ctypes.byref(p.c()), px, T, H, W, a.t("out", out, shape, p.torch_dtype), _stream(x.device)),
          "vsa_crop")
    return out


def pad(p: Problem, x):
    """Token tensor of p (p's layout) holding raster x [B, h, T, H, W, d] at the origin, zeros elsewhere."""
    if not isinstance(x, torch.Tensor) or x.dim() != 6:
        raise ValueError("vsa_pad: x must be a raster tensor [B, h, T, H, W, d]")
    T, H, W = x.shape[2:5]
    a = _Args("vsa_pad")
    px = a.t("x", x, (p.B, p.heads, T, H, W, p.head_dim), p.torch_dtype)
    out = _empty(_raster(p), x.dtype, x)
    check(a.call(lib().vsa_pad, ctypes.byref(p.c()), px, T, H, W, a.t("out", out, _raster(p), p.torch_dtype),
                        _stream(x.device)), "vsa_pad")
    return out


def _pooled(p: Problem, keys: bool = False):
    """Shape of a pooled tensor: per query cube, or per key block with keys."""
    return (p.B, p.heads, p.Nk if keys else p.Nc, p.head_dim)


def _qkv(a: _Args, p: Problem, q, k, v):
    td = p.torch_dtype
    return a.t("q", q, _raster(p), td), a.t("k", k, _raster(p), td), a.t("v", v, _raster(p), td)


def forward(p: Problem, q, k, v, g_c=None, g_f=None, idx=None, lens=None, training: bool = False,
            ws: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
            saved: Optional[torch.Tensor] = None):
    """Whole VSA forward. Returns (o, idx, lens, saved); saved is None unless
    training or a saved buffer (uint8, saved_bytes(p)) is passed in."""
    a = _Args("vsa_forward")
    td = p.torch_dtype
    pq, pk, pv = _qkv(a, p, q, k, v)
    pgc, pgf = a.t("g_c", g_c, _raster(p), td, False), a.t("g_f", g_f, _raster(p), td, False)
    if p.topk > 0:
        idx = _empty((p.B, p.heads, p.Nc, p.stride), torch.int32, q) if idx is None else idx
        lens = _empty((p.B, p.heads, p.Nc), torch.int32, q) if lens is None else lens
    elif idx is None or lens is None:
        raise ValueError("explicit-list mode (topk == 0) needs idx and lens")
    ishape, lshape = _lists(p)
    pidx, plen = a.t("idx", idx, ishape, torch.int32), a.t("lens", lens, lshape, torch.int32)
    o = _empty(_raster(p), td, q) if out is None else out
    po = a.t("out", o, _raster(p), td)
    if saved is None and training:
        saved = torch.empty(saved_bytes(p), dtype=torch.uint8, device=q.device)
    psaved, _ = a.buf("saved", saved, saved_bytes(p), required=False)
    ws = workspace(p, q) if ws is None else ws
    pws, nws = a.buf("ws", ws, workspace_bytes(p))
    check(a.call(lib().vsa_forward, ctypes.byref(p.c()), pq, pk, pv, pgc, pgf, pidx, plen, po, psaved, pws, nws,
                            _stream(q.device)), "vsa_forward")
    return o, idx, lens, saved


def saved_views(p: Problem, saved: torch.Tensor) -> dict:
    """Views of the tensors in a training forward's saved buffer, in the
    order the header documents (each region starts on a 256-byte boundary)."""
    off = 0

    def take(shape, dtype):
        nonlocal off
        n = _numel(shape)
        esz = torch.empty((), dtype=dtype).element_size()
        t = saved[off:off + n * esz].view(dtype).view(shape)
        off += (n * esz + 255) // 256 * 256
        return t

    out = {name: take(_pooled(p, name in ("k_c", "v_c")), torch.float32) for name in ("q_c", "k_c", "v_c", "o_c")}
    out["lse_c"] = take((p.B, p.heads, p.Nc), torch.float32)
    out["lse_f"] = take(_tokens(p), torch.float32)
    out["o_f"] = take(_raster(p), p.torch_dtype)
    return out


def backward(p: Problem, q, k, v, g_c, g_f, idx, lens, saved, d_o, ws: Optional[torch.Tensor] = None):
    """Whole VSA backward. Returns dict dq, dk, dv, dg_c, dg_f (gate grads None for NULL gates)."""
    a = _Args("vsa_backward")
    td = p.torch_dtype
    pq, pk, pv = _qkv(a, p, q, k, v)
    pgc, pgf = a.t("g_c", g_c, _raster(p), td, False), a.t("g_f", g_f, _raster(p), td, False)
    ishape, lshape = _lists(p)
    pidx, plen = a.t("idx", idx, ishape, torch.int32), a.t("lens", lens, lshape, torch.int32)
    psaved, _ = a.buf("saved", saved, saved_bytes(p))
    pdo = a.t("d_o", d_o, _raster(p), td)
    dq, dk, dv = (_empty(_raster(p), td, q) for _ in range(3))
    dgc = _empty(_raster(p), td, q) if g_c is not None else None
    dgf = _empty(_raster(p), td, q) if g_f is not None else None
    ws = workspace(p, q, training=True) if ws is None else ws
    pws, nws = a.buf("ws", ws, workspace_bytes(p, training=True))
    check(a.call(lib().vsa_backward, ctypes.byref(p.c()), pq, pk, pv, pgc, pgf, pidx, plen, psaved, pdo,
                             a.t("dq", dq, _raster(p), td), a.t("dk", dk, _raster(p), td),
                             a.t("dv", dv, _raster(p), td), a.t("dg_c", dgc, _raster(p), td, False),
                             a.t("dg_f", dgf, _raster(p), td, False), pws, nws, _stream(q.device)), "vsa_backward")
    return dict(dq=dq, dk=dk, dv=dv, dg_c=dgc, dg_f=dgf)


def pool(p: Problem, q, k, v, out=None):
    a = _Args("vsa_pool")
    pq, pk, pv = _qkv(a, p, q, k, v)
    qc, kc, vc = out if out is not None else (_empty(_pooled(p, keys), torch.float32, q) for keys in (0, 1, 1))
    f = torch.float32
    check(a.call(lib().vsa_pool, ctypes.byref(p.c()), pq, pk, pv, a.t("q_c", qc, _pooled(p), f),
                         a.t("k_c", kc, _pooled(p, True), f), a.t("v_c", vc, _pooled(p, True), f),
                         _stream(q.device)), "vsa_pool")
    return qc, kc, vc


def coarse(p: Problem, q_c, k_c, v_c, out=None, ws: Optional[torch.Tensor] = None):
    """Coarse stage; out = (o_c, lse_c, idx, lens) reuses caller buffers."""
    a = _Args("vsa_coarse")
    f = torch.float32
    pqc = a.t("q_c", q_c, _pooled(p), f)
    pkc, pvc = a.t("k_c", k_c, _pooled(p, True), f), a.t("v_c", v_c, _pooled(p, True), f)
    ws = workspace(p, q_c) if ws is None else ws
    pws, nws = a.buf("ws", ws, workspace_bytes(p))
    if out is not None:
        oc, lse, idx, lens = out
    else:
        oc = _empty(_pooled(p), torch.float32, q_c)
        lse = _empty((p.B, p.heads, p.Nc), torch.float32, q_c)
        idx = lens = None
        if p.topk > 0:
            idx = _empty((p.B, p.heads, p.Nc, p.stride), torch.int32, q_c)
            lens = _empty((p.B, p.heads, p.Nc), torch.int32, q_c)
    ishape, lshape = _lists(p)
    sel = p.topk > 0
    check(a.call(lib().vsa_coarse, ctypes.byref(p.c()), pqc, pkc, pvc, a.t("o_c", oc, _pooled(p), f),
                           a.t("lse_c", lse, (p.B, p.heads, p.Nc), f), a.t("idx", idx, ishape, torch.int32, sel),
                           a.t("lens", lens, lshape, torch.int32, sel), pws, nws, _stream(q_c.device)), "vsa_coarse")
    return oc, lse, idx, lens


def fine_forward(p: Problem, q, k, v, idx, lens, ws: Optional[torch.Tensor] = None):
    a = _Args("vsa_fine_forward")
    pq, pk, pv = _qkv(a, p, q, k, v)
    ishape, lshape = _lists(p)
    pidx, plen = a.t("idx", idx, ishape, torch.int32), a.t("lens", lens, lshape, torch.int32)
    ws = workspace(p, q) if ws is None else ws
    pws, nws = a.buf("ws", ws, workspace_bytes(p))
    of = _empty(_raster(p), p.torch_dtype, q)
    lse = _empty(_tokens(p), torch.float32, q)
    check(a.call(lib().vsa_fine_forward, ctypes.byref(p.c()), pq, pk, pv, pidx, plen, a.t("o_f", of, _raster(p), p.torch_dtype),
                                 a.t("lse_f", lse, _tokens(p), torch.float32), pws, nws, _stream(q.device)),
          "vsa_fine_forward")
    return of, lse


def fine_combine(p: Problem, q, k, v, idx, lens, o_c, g_c=None, g_f=None, ws: Optional[torch.Tensor] = None,
                 out: Optional[torch.Tensor] = None, with_fine: bool = False):
    """Fused fine stage + gated combine. Returns o, or (o, o_f, lse_f) with with_fine."""
    a = _Args("vsa_fine_combine")
    td = p.torch_dtype
    pq, pk, pv = _qkv(a, p, q, k, v)
    ishape, lshape = _lists(p)
    pidx, plen = a.t("idx", idx, ishape, torch.int32), a.t("lens", lens, lshape, torch.int32)
    poc = a.t("o_c", o_c, _pooled(p), torch.float32)
    pgc, pgf = a.t("g_c", g_c, _raster(p), td, False), a.t("g_f", g_f, _raster(p), td, False)
    ws = workspace(p, q) if ws is None else ws
    pws, nws = a.buf("ws", ws, workspace_bytes(p))
    o = _empty(_raster(p), td, q) if out is None else out
    of = _empty(_raster(p), td, q) if with_fine else None
    lse = _empty(_tokens(p), torch.float32, q) if with_fine else None
    check(a.call(lib().vsa_fine_combine, ctypes.byref(p.c()), pq, pk, pv, pidx, plen, poc, pgc, pgf,
                                 a.t("out", o, _raster(p), td), a.t("o_f", of, _raster(p), td, False),
                                 a.t("lse_f", lse, _tokens(p), torch.float32, False), pws, nws, _stream(q.device)),
          "vsa_fine_combine")
    return (o, of, lse) if with_fine else o


def fine_combine_noalloc(p: Problem, q, k, v, idx, lens, o_c, g_c=None, g_f=None,
                         out: Optional[torch.Tensor] = None, o_f: Optional[torch.Tensor] = None,
                         lse_f: Optional[torch.Tensor] = None):
    """fine_combine without a workspace: the library keeps its scratch in a
    static device array (B * heads * Nc <= 1,048,576; overlapping calls on
    one GPU race). Outputs are the caller's tensors when given (o_f / lse_f
    optional); nothing else is allocated when `out` is given. Returns o."""
    a = _Args("vsa_fine_combine_noalloc")
    td = p.torch_dtype
    pq, pk, pv = _qkv(a, p, q, k, v)
    ishape, lshape = _lists(p)
    pidx, plen = a.t("idx", idx, ishape, torch.int32), a.t("lens", lens, lshape, torch.int32)
    poc = a.t("o_c", o_c, _pooled(p), torch.float32)
    pgc, pgf = a.t("g_c", g_c, _raster(p), td, False), a.t("g_f", g_f, _raster(p), td, False)
    o = _empty(_raster(p), td, q) if out is None else out
    check(a.call(lib().vsa_fine_combine_noalloc, ctypes.byref(p.c()), pq, pk, pv, pidx, plen, poc, pgc, pgf,
                 a.t("out", o, _raster(p), td), a.t("o_f", o_f, _raster(p), td, False),
                 a.t("lse_f", lse_f, _tokens(p), torch.float32, False), _stream(q.device)),
          "vsa_fine_combine_noalloc")
    return o


def combine(p: Problem, o_c, o_f, g_c=None, g_f=None):
    a = _Args("vsa_combine")
    td = p.torch_dtype
    pof = a.t("o_f", o_f, _raster(p), td)
    poc = a.t("o_c", o_c, _pooled(p), torch.float32)
    pgc, pgf = a.t("g_c", g_c, _raster(p), td, False), a.t("g_f", g_f, _raster(p), td, False)
    o = _empty(_raster(p), td, o_f)
    check(a.call(lib().vsa_combine, ctypes.byref(p.c()), poc, pof, pgc, pgf, a.t("o", o, _raster(p), td),
                            _stream(o_f.device)), "vsa_combine")
    return o


def combine_backward(p: Problem, d_o, o_c, o_f, g_c=None, g_f=None):
    a = _Args("vsa_combine_backward")
    td, f = p.torch_dtype, torch.float32
    pdo = a.t("d_o", d_o, _raster(p), td)
    poc, pof = a.t("o_c", o_c, _pooled(p), f), a.t("o_f", o_f, _raster(p), td)
    pgc, pgf = a.t("g_c", g_c, _raster(p), td, False), a.t("g_f", g_f, _raster(p), td, False)
    dgc = _empty(_raster(p), td, d_o) if g_c is not None else None
    dgf = _empty(_raster(p), td, d_o) if g_f is not None else None
    dof = _empty(_raster(p), td, d_o)
    delta = _empty(_tokens(p), f, d_o)
    doc = _empty(_pooled(p), f, d_o)
    check(a.call(lib().vsa_combine_backward, ctypes.byref(p.c()), pdo, poc, pof, pgc, pgf,
                                     a.t("dg_c", dgc, _raster(p), td, False), a.t("dg_f", dgf, _raster(p), td, False),
                                     a.t("d_o_f", dof, _raster(p), td), a.t("delta", delta, _tokens(p), f),
                                     a.t("d_o_c", doc, _pooled(p), f), _stream(d_o.device)), "vsa_combine_backward")
    return dict(dg_c=dgc, dg_f=dgf, d_o_f=dof, delta=delta, d_o_c=doc)


def _k2q_shapes(p: Problem):
    return (p.B, p.heads, p.Nk + 1), (p.B, p.heads, p.Nc * p.stride)


def index_transpose(p: Problem, idx, lens, ws: Optional[torch.Tensor] = None):
    a = _Args("vsa_index_transpose")
    ishape, lshape = _lists(p)
    pidx, plen = a.t("idx", idx, ishape, torch.int32), a.t("lens", lens, lshape, torch.int32)
    ws = workspace(p, idx, training=True) if ws is None else ws
    pws, nws = a.buf("ws", ws, workspace_bytes(p, training=True))
    oshape, kshape = _k2q_shapes(p)
    off = _empty(oshape, torch.int32, idx)
    k2q = _empty(kshape, torch.int32, idx)
    check(a.call(lib().vsa_index_transpose, ctypes.byref(p.c()), pidx, plen, a.t("k2q_off", off, oshape, torch.int32),
                                    a.t("k2q", k2q, kshape, torch.int32), pws, nws, _stream(idx.device)),
          "vsa_index_transpose")
    return off, k2q


def fine_backward(p: Problem, q, k, v, idx, lens, k2q_off, k2q, lse_f, d_o_f, delta, dq_c, dk_c, dv_c,
                  ws: Optional[torch.Tensor] = None):
    a = _Args("vsa_fine_backward")
    td, f = p.torch_dtype, torch.float32
    pq, pk, pv = _qkv(a, p, q, k, v)
    ishape, lshape = _lists(p)
    oshape, kshape = _k2q_shapes(p)
    args = [pq, pk, pv, a.t("idx", idx, ishape, torch.int32), a.t("lens", lens, lshape, torch.int32),
            a.t("k2q_off", k2q_off, oshape, torch.int32), a.t("k2q", k2q, kshape, torch.int32),
            a.t("lse_f", lse_f, _tokens(p), f), a.t("d_o_f", d_o_f, _raster(p), td),
            a.t("delta", delta, _tokens(p), f), a.t("dq_c", dq_c, _pooled(p), f),
            a.t("dk_c", dk_c, _pooled(p, True), f), a.t("dv_c", dv_c, _pooled(p, True), f)]
    ws = workspace(p, q, training=True) if ws is None else ws
    pws, nws = a.buf("ws", ws, workspace_bytes(p, training=True))
    dq, dk, dv = (_empty(_raster(p), td, q) for _ in range(3))
    check(a.call(lib().vsa_fine_backward, ctypes.byref(p.c()), *args, a.t("dq", dq, _raster(p), td),
                                  a.t("dk", dk, _raster(p), td), a.t("dv", dv, _raster(p), td), pws, nws,
                                  _stream(q.device)), "vsa_fine_backward")
    return dq, dk, dv


def coarse_backward(p: Problem, q_c, k_c, v_c, o_c, lse_c, d_o_c, ws: Optional[torch.Tensor] = None):
    a = _Args("vsa_coarse_backward")
    f = torch.float32
    args = [a.t("q_c", q_c, _pooled(p), f), a.t("k_c", k_c, _pooled(p, True), f),
            a.t("v_c", v_c, _pooled(p, True), f), a.t("o_c", o_c, _pooled(p), f),
            a.t("lse_c", lse_c, (p.B, p.heads, p.Nc), f), a.t("d_o_c", d_o_c, _pooled(p), f)]
    ws = workspace(p, q_c, training=True) if ws is None else ws
    pws, nws = a.buf("ws", ws, workspace_bytes(p, training=True))
    dqc, dkc, dvc = (_empty(_pooled(p, keys), f, q_c) for keys in (0, 1, 1))
    check(a.call(lib().vsa_coarse_backward, ctypes.byref(p.c()), *args, a.t("dq_c", dqc, _pooled(p), f),
                                    a.t("dk_c", dkc, _pooled(p, True), f), a.t("dv_c", dvc, _pooled(p, True), f),
                                    pws, nws, _stream(q_c.device)), "vsa_coarse_backward")
    return dqc, dkc, dvc


def check_lists_host(p: Problem, idx, lens) -> None:
    """CPU check of explicit lists given as numpy int32 arrays (raises VsaError)."""
    import numpy as np
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    lens = np.ascontiguousarray(lens, dtype=np.int32)
    ishape, lshape = _lists(p)
    if idx.size != _numel(ishape) or lens.size != _numel(lshape):
        raise ValueError(f"vsa_check_lists_host: idx {idx.shape} / lens {lens.shape} do not hold "
                         f"{ishape} / {lshape} elements")
    check(lib().vsa_check_lists_host(ctypes.byref(p.c()), idx.ctypes.data_as(ctypes.c_void_p),
                                     lens.ctypes.data_as(ctypes.c_void_p)), "vsa_check_lists_host")


def validate_lists(p: Problem, idx, lens) -> None:
    """Device check of explicit lists (synchronises the current stream; raises VsaError)."""
    a = _Args("vsa_validate_lists")
    ishape, lshape = _lists(p)
    pidx, plen = a.t("idx", idx, ishape, torch.int32), a.t("lens", lens, lshape, torch.int32)
    flag = _empty((4,), torch.int32, idx)
    check(a.call(lib().vsa_validate_lists, ctypes.byref(p.c()), pidx, plen, a.t("flag", flag, (4,), torch.int32),
                                   _stream(idx.device)), "vsa_validate_lists")


# Measurement aids (include/vsa_probe.h); not steps of the operator.
def probe_mfma_valu(valu: int, op: int, waves_per_simd: int, iters: int, out) -> None:
    """Enqueues the MFMA / vector-ALU overlap probe on the current stream
    (out: float32, 65536 * waves_per_simd elements)."""
    a = _Args("vsa_probe_mfma_valu")
    po = a.t("out", out, (65536 * waves_per_simd,), torch.float32)
    check(a.call(lib().vsa_probe_mfma_valu, valu, op, waves_per_simd, iters, po, _stream(out.device)),
          "vsa_probe_mfma_valu")


def probe_stream_read(src, blocks: int, inflight: int, out, nontemporal: bool = False) -> None:
    """Enqueues a streaming read of all of src (any contiguous tensor whose
    byte size is a multiple of 16) on the current stream (out: float32,
    blocks * 256 elements), with non-temporal loads when asked."""
    a = _Args("vsa_probe_stream_read")
    if not isinstance(src, torch.Tensor):
        raise ValueError("vsa_probe_stream_read: src must be a torch.Tensor")
    a._common("src", src)
    po = a.t("out", out, (blocks * 256,), torch.float32)
    nbytes = src.numel() * src.element_size()
    check(a.call(lib().vsa_probe_stream_read, ctypes.c_void_p(src.data_ptr()), nbytes, blocks, inflight,
                 int(bool(nontemporal)), po, _stream(out.device)), "vsa_probe_stream_read")


def probe_l2_to_lds(mode: int, src, blocks: int, iters: int, out) -> None:
    """Enqueues the L2-to-LDS probe on the current stream: mode 0 direct-to-LDS
    loads, 1 loads into registers and LDS writes; src: a contiguous tensor
    whose byte size is a power of two (16 KB .. 1 GB); out: float32,
    blocks * 128 elements."""
    a = _Args("vsa_probe_l2_to_lds")
    if not isinstance(src, torch.Tensor):
        raise ValueError("vsa_probe_l2_to_lds: src must be a torch.Tensor")
    a._common("src", src)
    po = a.t("out", out, (blocks * 128,), torch.float32)
    nbytes = src.numel() * src.element_size()
    check(a.call(lib().vsa_probe_l2_to_lds, mode, ctypes.c_void_p(src.data_ptr()), nbytes, blocks, iters, po,
                 _stream(out.device)), "vsa_probe_l2_to_lds")


class _Attention(torch.autograd.Function):
    """forward / backward of the library as one differentiable operation (the
    selection is piecewise constant: idx and lens carry no gradient)."""

    @staticmethod
    def forward(ctx, p, q, k, v, g_c, g_f, idx, lens):
        o, idx, lens, saved = forward(p, q, k, v, g_c, g_f, idx=idx, lens=lens, training=True)
        ctx.p = p
        ctx.save_for_backward(q, k, v, g_c, g_f, idx, lens, saved)
        ctx.mark_non_differentiable(idx, lens)
        return o, idx, lens

    @staticmethod
    def backward(ctx, d_o, _d_idx, _d_lens):
        q, k, v, g_c, g_f, idx, lens, saved = ctx.saved_tensors
        g = backward(ctx.p, q, k, v, g_c, g_f, idx, lens, saved, d_o.contiguous())
        return None, g["dq"], g["dk"], g["dv"], g["dg_c"], g["dg_f"], None, None


def attention(p: Problem, q, k, v, g_c=None, g_f=None, idx=None, lens=None):
    """Differentiable VSA attention: returns (o, idx, lens); gradients flow to
    q, k, v and the gates given (NULL gates are the constant 1). In top-K mode
    idx / lens are outputs (fresh tensors unless given); in explicit-list mode
    (p.topk == 0) they are the caller's lists. Every tensor must be contiguous
    on the GPU in p's dtype and layout."""
    return _Attention.apply(p, q, k, v, g_c, g_f, idx, lens)
