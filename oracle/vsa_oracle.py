"""CPU oracle of the VSA coarse-fine attention operator, in float64.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module. The HIP
path never does, and this module imports nothing from it.

It is the plain definition of what the method computes, step by step, for
every (batch, head) independently. Sources (the VSA pages):

* "VSA: Faster Video Diffusion with Trainable Sparse Attention" summary page
  (paperlayer.ai, arXiv 2505.13389): section 2 "Methods" (cube partition,
  coarse stage, top-K, fine stage, gated combination), Appendix B
  "Pseudocode of VSA" (tile, mean-pool, dense block attention, repeat of the
  coarse output, top-k, masked fine attention, combination, untile).
* The NeurIPS 2025 reading notes on VSA (zhaoyang97.github.io Paper-Notes):
  "key designs" 1 (mean-pooled Q_c, K_c, V_c, cube-level A_c and O_c, row
  top-K giving mask M), 2 (fine token attention on the selected blocks),
  3 (O = O_c * G_c + O_f * G_f), 5 (adaptation starting from K = all cubes,
  G_c = 0, G_f removed, which equals full attention).
* The VSA2 summary pages (arXiv 2609.32882): each query may attend a variable
  number of key/value blocks; here, explicit per-query-cube block lists.

Readings where the pages are silent (each one is listed with its reason in
the design notes of the repository):
* softmax scale s = 1/sqrt(d) in both stages unless a scale is given;
* cubes in row-major order over (T/4, H/4, W/4), tokens inside a cube in
  row-major (t, y, x) order;
* top-K is taken on the logits (same set as on A_c: softmax is increasing
  within a row), ties going to the smaller cube index, no forced diagonal;
* masked logits are exactly -inf; an empty list gives O_f = 0, LSE_f = -inf;
* gates are elementwise, shaped like the output; a missing gate means 1;
* the top-K mask carries no gradient (it is piecewise constant);
* cube shapes other than (4, 4, 4) (the summary page's tile-size exploration,
  section 2 "Methods"): the same definitions with B = Ct*Ch*Cw tokens per cube,
  cubes row-major over the grid and tokens row-major inside a cube; with key
  blocks of their own shape (Bq x Bk tiles, as the page's 64 x 16 example),
  queries are pooled and attend per query cube, keys and values are pooled
  and selected per key block;
* the max-pool variant (ablation of the coarse pooling) takes the per-channel
  maximum over a cube; its gradient goes to the first maximum in cube order.

Parity status: every function here is pinned by the CPU tests in
``tests/test_oracle.py`` (library routines, closed forms, brute force,
finite differences). Agreement with the authors' own kernels is parity
unpinned: the pages print no tensors and no error bound.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np

CUBE = 4                      # cube edge (4, 4, 4): section 2 "Methods", App. B
TILE = CUBE * CUBE * CUBE     # 64 tokens per cube = one tile (block = 64)
DEFAULT_CUBE = (CUBE, CUBE, CUBE)
# Section 2 "Methods" of the summary page names the cube (Ct, Ch, Cw) with tile
# size B = Ct*Ch*Cw and its design exploration compares tile sizes; every
# function below takes the cube shape, (4, 4, 4) unless stated.


def _cube(cube) -> tuple:
    ct, ch, cw = (int(e) for e in cube)
    if min(ct, ch, cw) <= 0:
        raise ValueError("cube sides must be positive")
    return ct, ch, cw


# --------------------------------------------------------------------------
# Step 0: cube partition, tile and untile (section 2 "Methods"; App. B)
# --------------------------------------------------------------------------
def tiled_to_raster(T: int, H: int, W: int, cube=DEFAULT_CUBE) -> np.ndarray:
    """perm[p] = raster token index of tiled position p = B*c + l (B = Ct*Ch*Cw).

    Token (t, y, x) lies in cube c = ((t//Ct)*(H/Ch) + y//Ch)*(W/Cw) + x//Cw
    (row-major cube order) at local index l = ((t%Ct)*Ch + y%Ch)*Cw + x%Cw
    (row-major inside the cube).
    """
    ct, ch, cw = _cube(cube)
    if T % ct or H % ch or W % cw:
        raise ValueError(f"latent dims must be multiples of the cube {cube}")
    Hp, Wp = H // ch, W // cw
    t, y, x = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
    c = ((t // ct) * Hp + y // ch) * Wp + x // cw
    l = ((t % ct) * ch + y % ch) * cw + x % cw
    raster = (t * H + y) * W + x
    perm = np.empty(T * H * W, dtype=np.int64)
    perm[(c * (ct * ch * cw) + l).reshape(-1)] = raster.reshape(-1)
    return perm


def tile(x: np.ndarray, cube=DEFAULT_CUBE) -> np.ndarray:
    """[..., T, H, W, d] (raster) -> [..., Nc, B, d] (cube-major)."""
    T, H, W, d = x.shape[-4:]
    b = int(np.prod(_cube(cube)))
    flat = x.reshape(x.shape[:-4] + (T * H * W, d))
    return flat[..., tiled_to_raster(T, H, W, cube), :].reshape(
        x.shape[:-4] + (T * H * W // b, b, d))


def untile(xt: np.ndarray, T: int, H: int, W: int, cube=DEFAULT_CUBE) -> np.ndarray:
    """Inverse of ``tile``: [..., Nc, B, d] -> [..., T, H, W, d]."""
    d = xt.shape[-1]
    N = T * H * W
    out = np.empty(xt.shape[:-3] + (N, d), dtype=xt.dtype)
    out[..., tiled_to_raster(T, H, W, cube), :] = xt.reshape(xt.shape[:-3] + (N, d))
    return out.reshape(xt.shape[:-3] + (T, H, W, d))


def compatible_latent(T: int, H: int, W: int, cube=DEFAULT_CUBE) -> tuple:
    """Smallest latent whose sides are multiples of the cube's sides and which
    contains T x H x W. Section 5 "Limitation and Conclusion" of the summary
    page: (4, 4, 4) cubes need sides divisible by 4; a slightly larger latent
    is generated and the result cropped."""
    if min(T, H, W) <= 0:
        raise ValueError("latent sides must be positive")
    return tuple(-(-n // e) * e for n, e in zip((T, H, W), _cube(cube)))


def crop(x: np.ndarray, T: int, H: int, W: int) -> np.ndarray:
    """Leading T x H x W region of a raster tensor [..., Tc, Hc, Wc, d]."""
    return x[..., :T, :H, :W, :].copy()


def pad(x: np.ndarray, Tc: int, Hc: int, Wc: int) -> np.ndarray:
    """Raster [..., Tc, Hc, Wc, d] holding x [..., T, H, W, d] at the origin
    and zeros at every other token."""
    T, H, W, d = x.shape[-4:]
    out = np.zeros(x.shape[:-4] + (Tc, Hc, Wc, d), dtype=x.dtype)
    out[..., :T, :H, :W, :] = x
    return out


def untile_rows(rt: np.ndarray, T: int, H: int, W: int, cube=DEFAULT_CUBE) -> np.ndarray:
    """Inverse of tiling for per-token scalars: [..., Nc, B] -> [..., T, H, W]."""
    return untile(rt[..., None], T, H, W, cube)[..., 0]


# --------------------------------------------------------------------------
# Step 1: cube mean-pool (section 2 "Methods"; App. B; notes key design 1)
# --------------------------------------------------------------------------
POOL_MODES = ("mean", "max")


def pool(xt: np.ndarray, mode: str = "mean") -> np.ndarray:
    """X_c[c] = (1/B) * sum over the B tokens of cube c.  [..., Nc, B, d] -> [..., Nc, d].

    mode "max": the per-channel maximum over the cube's tokens instead, the
    pooling variant the VSA summary page's ablation study compares with
    average pooling (section 3 "Experiments", ablation studies)."""
    if mode == "max":
        return xt.max(axis=-2)
    if mode != "mean":
        raise ValueError(f"pool mode {mode!r}")
    return xt.sum(axis=-2) / xt.shape[-2]


# --------------------------------------------------------------------------
# Step 2: coarse dense attention over cubes (section 2; App. B; key design 1)
# --------------------------------------------------------------------------
def coarse_attention(qc: np.ndarray, kc: np.ndarray, vc: np.ndarray, scale: float):
    """For one (b, h): S_c = s*Q_c K_c^T, A_c = row softmax, O_c = A_c V_c.

    Returns (S_c, A_c, O_c, LSE_c) with LSE_c[i] = log sum_j exp(S_c[i, j]).
    """
    s = scale * (qc @ kc.T)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    z = e.sum(axis=1, keepdims=True)
    a = e / z
    return s, a, a @ vc, (m + np.log(z))[:, 0]


# --------------------------------------------------------------------------
# Step 3: row top-K and mask -> index lists (section 2; App. B; key design 1)
# --------------------------------------------------------------------------
def topk_rows(s: np.ndarray, k: int):
    """Row-wise top-K of the coarse logits of one (b, h).

    A stable descending sort keeps equal logits in ascending cube order, so ties
    go to the smaller index. Returns (idx [Nc, K] ascending, margin [Nc]) where
    margin = K-th largest minus (K+1)-th largest logit (+inf when K = Nc).
    """
    nc = s.shape[1]
    if not 1 <= k <= nc:
        raise ValueError("top-K must lie in [1, Nc]")
    order = np.argsort(-s, axis=1, kind="stable")
    idx = np.sort(order[:, :k], axis=1).astype(np.int64)
    srt = np.take_along_axis(s, order, axis=1)
    margin = np.full(s.shape[0], np.inf) if k == nc else srt[:, k - 1] - srt[:, k]
    return idx, margin


def lists_to_mask(idx: np.ndarray, lens: np.ndarray, nc: int) -> np.ndarray:
    """Block mask M [rows, Nc] with M[i, j] = 1 iff j is in list i."""
    m = np.zeros((idx.shape[0], nc), dtype=bool)
    for i in range(idx.shape[0]):
        m[i, idx[i, :lens[i]]] = True
    return m


def mask_to_lists(mask: np.ndarray, stride: Optional[int] = None):
    """Ascending index lists of a block mask; padding is -1."""
    lens = mask.sum(axis=1).astype(np.int64)
    stride = int(lens.max(initial=0)) if stride is None else stride
    idx = np.full((mask.shape[0], max(stride, 1)), -1, dtype=np.int64)
    for i in range(mask.shape[0]):
        sel = np.nonzero(mask[i])[0]
        idx[i, :sel.size] = sel
    return idx, lens


def transpose_lists(idx: np.ndarray, lens: np.ndarray, nc: int):
    """k2q[j] = ascending query cubes i whose list holds j (used by the backward)."""
    return mask_to_lists(lists_to_mask(idx, lens, nc).T.copy(), stride=idx.shape[0])


def _pool_error_bound(xt: np.ndarray, sig_bits: int) -> np.ndarray:
    """Bound on |fp32 mean-pool - exact mean| per (cube, channel), any order.

    The B inputs of a cube carry ``sig_bits`` significant bits (8 for bf16
    values, 24 for fp32). If every input is a multiple of 2^q and the sum of
    their magnitudes is below 2^(q+24), every partial sum is an fp32 number, so
    the fp32 sum is exact whatever the order; otherwise the classic recursive-
    summation bound gamma_(B-1) * sum|x| applies. Dividing by B (a power of
    two) is exact.
    """
    u = 2.0 ** -24
    mag = np.abs(xt)
    _, e = np.frexp(mag)                      # |x| = m * 2^e, 0.5 <= m < 1
    ulp_exp = np.where(mag > 0, e - sig_bits, np.iinfo(np.int32).max)
    q = ulp_exp.min(axis=-2)
    total = mag.sum(axis=-2)
    exact = total < np.ldexp(1.0, np.minimum(q + 24, 1000))
    b = xt.shape[-2]
    gamma = (b - 1) * u / (1 - (b - 1) * u)
    return np.where(exact, 0.0, gamma * total / b)


def logit_error_bound(qt: np.ndarray, kt: np.ndarray, scale: float, sig_bits: int = 8,
                      pool_mode: str = "mean") -> np.ndarray:
    """Per-row bound on |fp32 coarse logit - exact logit| for one (b, h).

    The fp32 path pools B inputs (error bounded by ``_pool_error_bound``),
    forms the d-term dot product x . y of the pooled rows and multiplies by
    the fp32 scale (a few unit roundings of |S|). The dot product is formed
    in one of two ways:
    * as an fp32 dot product: error at most gamma_d * sum |x||y|, any order
      (the standard forward error bound of recursive summation);
    * on bf16 matrix units, from the exact split of every pooled value into
      three bf16 pieces x = hi + mid + lo (|hi| <= (1+2^-8)|x|,
      |mid| <= 2^-8 (1+2^-8)|x|, |lo| <= 2^-16 |x|; bf16 keeps 8 significant
      bits): the products hi*hi summed in one fp32 accumulator, hi*mid,
      mid*hi, hi*lo, lo*hi and mid*mid (each exact in fp32) in a second, the
      two added. Its error is at most gamma_d (1+2^-8)^2 for the first sum,
      gamma_5d (2^-7 + 3*2^-16)(1+2^-8)^2 for the second, one rounding of the
      final addition and 2^-23 (1+2^-8) + 2^-32 for the dropped products
      (mid*lo, lo*mid, lo*lo), all times sum |x||y|: a larger factor than
      gamma_d, so it bounds both forms and is the one used.
    Returns tau[i] = max_j bound(i, j); two logits of a row compare the same
    way in fp32 and exactly whenever they differ by more than 2*tau[i].
    """
    u = 2.0 ** -24
    d = qt.shape[-1]
    gamma = lambda n: n * u / (1 - n * u)
    r = (1 + 2.0 ** -8) ** 2
    cross = (2.0 ** -7 + 3 * 2.0 ** -16) * r
    gd = (gamma(d) * r + gamma(5 * d) * cross + u * (1 + gamma(5 * d)) * (r + cross)
          + 2.0 ** -23 * (1 + 2.0 ** -8) + 2.0 ** -32)
    qc, kc = np.abs(pool(qt, pool_mode)), np.abs(pool(kt, pool_mode))
    if pool_mode == "max":   # a maximum of exact values is exact
        eq, ek = np.zeros_like(qc), np.zeros_like(kc)
    else:
        eq, ek = _pool_error_bound(qt, sig_bits), _pool_error_bound(kt, sig_bits)
    pooled = eq @ kc.T + qc @ ek.T + eq @ ek.T
    dot = gd * ((qc + eq) @ (kc + ek).T)
    b = scale * (pooled + dot) + 4 * u * scale * (qc @ kc.T + pooled)
    return b.max(axis=1)


# --------------------------------------------------------------------------
# Step 4: fine block-sparse attention (section 2; App. B; key design 2)
# --------------------------------------------------------------------------
def fine_gathered(qt, kt, vt, idx, lens, scale):
    """Token attention of each query cube over the tokens of its listed cubes.

    For one (b, h): qt, kt, vt [Nc, B, d]; idx [Nc, L] and lens [Nc].
    Returns O_f [Nc, B, d] and LSE_f [Nc, B]. An empty list gives O_f = 0
    and LSE_f = -inf.
    """
    nc, b, d = qt.shape
    of = np.zeros_like(qt)
    lse = np.full((nc, b), -np.inf)
    for i in range(nc):
        sel = idx[i, :lens[i]]
        if sel.size == 0:
            continue
        ks = kt[sel].reshape(-1, d)
        vs = vt[sel].reshape(-1, d)
        z = scale * (qt[i] @ ks.T)
        m = z.max(axis=1, keepdims=True)
        e = np.exp(z - m)
        l = e.sum(axis=1, keepdims=True)
        of[i] = (e @ vs) / l
        lse[i] = (m + np.log(l))[:, 0]
    return of, lse


def fine_literal(q, k, v, mask, scale, cube=DEFAULT_CUBE, kcube=None):
    """The App. B form: full token-level scores, unselected blocks set to -inf,
    row softmax, times V. For one (b, h) in raster layout, q/k/v [T, H, W, d],
    mask [Nq, Nk] (query cubes x key cubes; kcube = cube unless given).
    Quadratic in N: small shapes only. Returns (O_f, LSE_f) raster."""
    T, H, W, d = q.shape
    kcube = cube if kcube is None else kcube
    n = T * H * W
    qr, kr, vr = q.reshape(n, d), k.reshape(n, d), v.reshape(n, d)
    qcube_of = np.empty(n, dtype=np.int64)
    qcube_of[tiled_to_raster(T, H, W, cube)] = np.arange(n) // int(np.prod(_cube(cube)))
    kcube_of = np.empty(n, dtype=np.int64)
    kcube_of[tiled_to_raster(T, H, W, kcube)] = np.arange(n) // int(np.prod(_cube(kcube)))
    allowed = mask[qcube_of[:, None], kcube_of[None, :]]
    z = np.where(allowed, scale * (qr @ kr.T), -np.inf)
    o = np.zeros((n, d))
    lse = np.full(n, -np.inf)
    live = allowed.any(axis=1)
    m = z[live].max(axis=1, keepdims=True)
    e = np.exp(z[live] - m)
    l = e.sum(axis=1, keepdims=True)
    o[live] = (e @ vr) / l
    lse[live] = (m + np.log(l))[:, 0]
    return o.reshape(T, H, W, d), lse.reshape(T, H, W)


# --------------------------------------------------------------------------
# Step 5: gated combination and untile (section 2; App. B; key design 3)
# --------------------------------------------------------------------------
def repeat_coarse(oc: np.ndarray, T: int, H: int, W: int, cube=DEFAULT_CUBE) -> np.ndarray:
    """O_c of each cube repeated to its B tokens, raster layout [..., T, H, W, d]."""
    b = int(np.prod(_cube(cube)))
    return untile(np.repeat(oc[..., :, None, :], b, axis=-2), T, H, W, cube)


def combine(oc_rep, of, g_c=None, g_f=None):
    """O = O_c (repeated) * G_c + O_f * G_f, elementwise; a missing gate is 1."""
    gc = 1.0 if g_c is None else g_c
    gf = 1.0 if g_f is None else g_f
    return oc_rep * gc + of * gf


# --------------------------------------------------------------------------
# Whole forward
# --------------------------------------------------------------------------
def _bf16_exact(x) -> bool:
    """True when every value of x is a bf16 number (low 16 bits of fp32 zero)."""
    a = np.ascontiguousarray(x, dtype=np.float32)
    return bool(np.all((a.view(np.uint32) & np.uint32(0xFFFF)) == 0))


def _f64(x):
    return None if x is None else np.asarray(x, dtype=np.float64)


def forward(q, k, v, g_c=None, g_f=None, topk: int = 0, idx=None, lens=None,
            scale: Optional[float] = None, with_literal: bool = False, pool_mode: str = "mean",
            cube=DEFAULT_CUBE, kcube=None):
    """VSA forward for [B, h, T, H, W, d] inputs with query cubes of shape
    ``cube`` and key blocks of shape ``kcube`` (the same unless given: the
    Bq x Bk tiles of the summary page's tile-size exploration).

    topk > 0 selects the K best key blocks per query cube; topk == 0 uses the
    caller's lists idx [B, h, Nq, L] / lens [B, h, Nq]. Returns a dict of
    float64 results (raster layout unless the name says tiled / pooled).
    """
    sig_bits = 24 if np.asarray(q).dtype == np.float32 and not _bf16_exact(q) else 8
    q, k, v, g_c, g_f = map(_f64, (q, k, v, g_c, g_f))
    B, nh, T, H, W, d = q.shape
    cube = _cube(cube)
    kcube = cube if kcube is None else _cube(kcube)
    nq = T * H * W // int(np.prod(cube))
    nc = T * H * W // int(np.prod(kcube))     # key blocks: the coarse columns
    s = 1.0 / math.sqrt(d) if scale is None else float(scale)
    qt, kt, vt = tile(q, cube), tile(k, kcube), tile(v, kcube)
    qc, kc, vc = pool(qt, pool_mode), pool(kt, pool_mode), pool(vt, pool_mode)
    oc = np.empty_like(qc)
    lse_c = np.empty(qc.shape[:-1])
    s_c = np.empty((B, nh, nq, nc))
    if topk > 0:
        idx_o = np.empty((B, nh, nq, topk), dtype=np.int64)
        lens_o = np.full((B, nh, nq), topk, dtype=np.int64)
        margin = np.empty((B, nh, nq))
        tau = np.empty((B, nh, nq))
    else:
        idx_o = np.asarray(idx, dtype=np.int64)
        lens_o = np.asarray(lens, dtype=np.int64)
        margin = tau = None
    of_t = np.empty_like(qt)
    lse_t = np.empty(qt.shape[:-1])
    of_lit = np.empty_like(q) if with_literal else None
    for b in range(B):
        for h in range(nh):
            s_c[b, h], _, oc[b, h], lse_c[b, h] = coarse_attention(qc[b, h], kc[b, h], vc[b, h], s)
            if topk > 0:
                idx_o[b, h], margin[b, h] = topk_rows(s_c[b, h], topk)
                tau[b, h] = logit_error_bound(qt[b, h], kt[b, h], s, sig_bits, pool_mode)
            of_t[b, h], lse_t[b, h] = fine_gathered(qt[b, h], kt[b, h], vt[b, h],
                                                    idx_o[b, h], lens_o[b, h], s)
            if with_literal:
                m = lists_to_mask(idx_o[b, h], lens_o[b, h], nc)
                of_lit[b, h], _ = fine_literal(q[b, h], k[b, h], v[b, h], m, s, cube, kcube)
    of = untile(of_t, T, H, W, cube)
    oc_rep = repeat_coarse(oc, T, H, W, cube)
    out = dict(scale=s, pool_mode=pool_mode, cube=cube, kcube=kcube, q_c=qc, k_c=kc, v_c=vc, s_c=s_c, o_c=oc, lse_c=lse_c,
               idx=idx_o, len=lens_o, margin=margin, tau=tau,
               o_f=of, lse_f=untile_rows(lse_t, T, H, W, cube), o_c_rep=oc_rep,
               o=combine(oc_rep, of, g_c, g_f))
    if with_literal:
        out["o_f_literal"] = of_lit
    return out


# --------------------------------------------------------------------------
# Backward: calculus through steps 1, 2, 4, 5 with the mask held constant
# --------------------------------------------------------------------------
def combine_backward(d_o, oc_rep, of, g_c=None, g_f=None):
    """Gradients of O = O_c*G_c + O_f*G_f. Returns dG_c, dG_f, dO_f, dO_c_rep
    (dO_c_rep is the per-token gradient w.r.t. the repeated coarse output)."""
    gc = 1.0 if g_c is None else g_c
    gf = 1.0 if g_f is None else g_f
    return d_o * oc_rep, d_o * of, d_o * gf, d_o * gc


def fine_backward(qt, kt, vt, dof_t, of_t, lse_t, idx, lens, scale):
    """Gradient of the fine stage for one (b, h), tiled layout.

    With P = exp(s*q.k - LSE_f) on the listed blocks: dV = P^T dO_f,
    dP = dO_f V^T, D = rowsum(dO_f * O_f), dS = P * (dP - D),
    dQ = s*dS K, dK = s*dS^T Q. Returns dQ [Nq, Bq, d], dK, dV [Nk, Bk, d] and
    D [Nq, Bq].
    """
    nc, b, d = qt.shape
    bk = kt.shape[1]
    dq = np.zeros_like(qt)
    dk = np.zeros_like(kt)
    dv = np.zeros_like(vt)
    dd = (dof_t * of_t).sum(axis=-1)
    for i in range(nc):
        sel = idx[i, :lens[i]]
        if sel.size == 0:
            continue
        ks = kt[sel].reshape(-1, d)
        vs = vt[sel].reshape(-1, d)
        p = np.exp(scale * (qt[i] @ ks.T) - lse_t[i][:, None])
        dp = dof_t[i] @ vs.T
        ds = p * (dp - dd[i][:, None])
        dq[i] = scale * (ds @ ks)
        dk_sel = (scale * (ds.T @ qt[i])).reshape(-1, bk, d)
        dv_sel = (p.T @ dof_t[i]).reshape(-1, bk, d)
        np.add.at(dk, sel, dk_sel)
        np.add.at(dv, sel, dv_sel)
    return dq, dk, dv, dd


def coarse_backward(qc, kc, vc, doc, scale):
    """Dense attention backward over cubes for one (b, h): returns dQ_c, dK_c, dV_c."""
    _, a, oc, _ = coarse_attention(qc, kc, vc, scale)
    dv = a.T @ doc
    da = doc @ vc.T
    ds = a * (da - (da * a).sum(axis=1, keepdims=True))
    return scale * (ds @ kc), scale * (ds.T @ qc), dv


def pool_backward(dxc: np.ndarray, xt: Optional[np.ndarray] = None, mode: str = "mean",
                  tile_size: int = TILE) -> np.ndarray:
    """Gradient of the mean-pool: each of the B tokens of cube c gets dX_c[c]/B
    (B = xt.shape[-2] when xt is given, else tile_size).

    mode "max" (xt = the pooled input, tiled): per channel, the whole dX_c[c]
    goes to the token holding the maximum; among equal maxima, the first in
    cube order (reading: the subgradient a sequential scan picks)."""
    if mode == "max":
        arg = np.argmax(xt, axis=-2)                      # first maximum
        out = np.zeros(xt.shape, dtype=np.result_type(dxc, np.float64))
        np.put_along_axis(out, arg[..., None, :], dxc[..., None, :], axis=-2)
        return out
    b = xt.shape[-2] if xt is not None else tile_size
    return np.repeat(dxc[..., :, None, :], b, axis=-2) / b


def backward(q, k, v, g_c, g_f, d_o, fwd: dict):
    """Gradients dQ, dK, dV, dG_c, dG_f of sum(O * dO) for the forward ``fwd``
    (float64, raster layout), plus the intermediates the GPU also forms."""
    q, k, v, g_c, g_f, d_o = map(_f64, (q, k, v, g_c, g_f, d_o))
    B, nh, T, H, W, d = q.shape
    s = fwd["scale"]
    cube = fwd.get("cube", DEFAULT_CUBE)
    kcube = fwd.get("kcube") or cube
    dgc, dgf, dof, docr = combine_backward(d_o, fwd["o_c_rep"], fwd["o_f"], g_c, g_f)
    doc = tile(docr, cube).sum(axis=-2)   # the repeat's gradient sums over the cube
    qt, kt, vt = tile(q, cube), tile(k, kcube), tile(v, kcube)
    dof_t, of_t = tile(dof, cube), tile(fwd["o_f"], cube)
    lse_t = tile(fwd["lse_f"][..., None], cube)[..., 0]
    dqt, dkt, dvt = np.empty_like(qt), np.empty_like(kt), np.empty_like(vt)
    dd_t = np.empty(qt.shape[:-1])
    dqc, dkc, dvc = np.empty_like(fwd["q_c"]), np.empty_like(fwd["k_c"]), np.empty_like(fwd["v_c"])
    for b in range(B):
        for h in range(nh):
            dqt[b, h], dkt[b, h], dvt[b, h], dd_t[b, h] = fine_backward(
                qt[b, h], kt[b, h], vt[b, h], dof_t[b, h], of_t[b, h], lse_t[b, h],
                fwd["idx"][b, h], fwd["len"][b, h], s)
            dqc[b, h], dkc[b, h], dvc[b, h] = coarse_backward(
                fwd["q_c"][b, h], fwd["k_c"][b, h], fwd["v_c"][b, h], doc[b, h], s)
    pm = fwd.get("pool_mode", "mean")
    dq = untile(dqt + pool_backward(dqc, qt, pm), T, H, W, cube)
    dk = untile(dkt + pool_backward(dkc, kt, pm), T, H, W, kcube)
    dv = untile(dvt + pool_backward(dvc, vt, pm), T, H, W, kcube)
    return dict(dq=dq, dk=dk, dv=dv, dg_c=dgc, dg_f=dgf, d_o_f=dof, d_o_c=doc,
                delta=untile_rows(dd_t, T, H, W, cube), dq_c=dqc, dk_c=dkc, dv_c=dvc)


# --------------------------------------------------------------------------
# Work accounting (computed blocks only)
# --------------------------------------------------------------------------
def fine_flops_forward(lens: np.ndarray, d: int, tile_size: int = TILE) -> float:
    """4*B*B*d FLOPs per computed (query cube, key cube) block pair."""
    return 4.0 * tile_size * tile_size * d * float(np.sum(lens))


def coarse_flops(B: int, nh: int, nc: int, d: int) -> float:
    """4*Nc^2*d per (b, h): the pooled score matrix and A_c V_c."""
    return 4.0 * B * nh * nc * nc * d


def dense_flops(B: int, nh: int, n: int, d: int) -> float:
    """Full token attention at the same shape: 4*N^2*d per (b, h)."""
    return 4.0 * B * nh * n * n * d
