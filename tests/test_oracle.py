"""Pins of the CPU oracle against things other than itself (CPU only).

Each test ties one oracle step to a library routine, a closed form, brute
force, an independent re-derivation (torch pooling / repeat ops that never use
the oracle's index arithmetic), finite differences, or a number the pages
print. A plausible mistake (wrong cube order, dropped 1/64, transposed
operand, wrong sign in dS, missing coarse path in the gradient) fails at
least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import workloads as WL
from oracle import vsa_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_facts.json")


def _rand(shape, seed=0):
    return np.random.default_rng(seed).standard_normal(shape)


# ---------------------------------------------------------------- step 0: tile
@pytest.mark.parametrize("T,H,W", [(4, 4, 4), (8, 8, 8), (4, 8, 12), (12, 4, 8)])
def test_tile_matches_reshape_transpose(T, H, W):
    """Cube-major tiling equals the (T',4,H',4,W',4) reshape/transpose (an
    independent construction: row-major cubes, row-major (t,y,x) in a cube)."""
    d = 3
    x = _rand((2, T, H, W, d))
    ref = x.reshape(2, T // 4, 4, H // 4, 4, W // 4, 4, d).transpose(0, 1, 3, 5, 2, 4, 6, 7)
    ref = ref.reshape(2, T * H * W // 64, 64, d)
    np.testing.assert_array_equal(O.tile(x), ref)
    np.testing.assert_array_equal(O.untile(O.tile(x), T, H, W), x)


@pytest.mark.parametrize("cube", [(2, 4, 4), (4, 4, 8), (1, 8, 8), (4, 2, 8), (2, 2, 8)])
def test_tile_general_cube_matches_reshape_transpose(cube):
    """Other cube shapes (Ct, Ch, Cw): the same row-major construction."""
    ct, ch, cw = cube
    T, H, W, d = 2 * ct, 3 * ch, 2 * cw, 3
    x = _rand((2, T, H, W, d), 7)
    ref = x.reshape(2, T // ct, ct, H // ch, ch, W // cw, cw, d).transpose(0, 1, 3, 5, 2, 4, 6, 7)
    ref = ref.reshape(2, T * H * W // (ct * ch * cw), ct * ch * cw, d)
    np.testing.assert_array_equal(O.tile(x, cube), ref)
    np.testing.assert_array_equal(O.untile(O.tile(x, cube), T, H, W, cube), x)
    want = []
    for n, e in zip((T - 1, H, W + 1), cube):
        m = n
        while m % e:
            m += 1
        want.append(m)
    assert O.compatible_latent(T - 1, H, W + 1, cube) == tuple(want)


def test_tile_is_bijection():
    perm = O.tiled_to_raster(8, 12, 16)
    assert np.array_equal(np.sort(perm), np.arange(8 * 12 * 16))


def test_tile_rejects_non_multiple_of_4():
    with pytest.raises(ValueError):
        O.tiled_to_raster(8, 6, 8)


def test_compatible_latent_brute_force():
    """Smallest multiple of 4 not below each side, found by counting up."""
    for n in range(1, 41):
        m = n
        while m % 4:
            m += 1
        assert O.compatible_latent(n, 4, 4)[0] == m
        assert O.compatible_latent(4, n, 4)[1] == m
        assert O.compatible_latent(4, 4, n)[2] == m
    with pytest.raises(ValueError):
        O.compatible_latent(0, 4, 4)


def test_crop_pad_round_trip_and_zero_fill():
    x = _rand((2, 3, 5, 6, 7, 3), 2)
    Tc, Hc, Wc = O.compatible_latent(5, 6, 7)
    xp = O.pad(x, Tc, Hc, Wc)
    assert xp.shape == (2, 3, 8, 8, 8, 3)
    np.testing.assert_array_equal(O.crop(xp, 5, 6, 7), x)
    for t in range(Tc):
        for y in range(Hc):
            for w in range(Wc):
                inside = t < 5 and y < 6 and w < 7
                cell = xp[:, :, t, y, w, :]
                if inside:
                    np.testing.assert_array_equal(cell, x[:, :, t, y, w, :])
                else:
                    assert not cell.any()


# ---------------------------------------------------------------- step 1: pool
def test_pool_matches_avg_pool3d():
    """Mean-pool equals torch avg_pool3d(kernel=stride=4) in row-major cube order."""
    x = _rand((1, 2, 8, 12, 4, 5), 1)
    xt = torch.from_numpy(x).permute(0, 1, 5, 2, 3, 4).reshape(2, 5, 8, 12, 4)
    ref = F.avg_pool3d(xt, 4).reshape(2, 5, -1).transpose(1, 2).numpy()
    np.testing.assert_allclose(O.pool(O.tile(x))[0], ref, rtol=1e-13, atol=1e-15)


def test_pool_brute_force_and_invariants():
    T, H, W, d = 8, 4, 8, 2
    x = _rand((T, H, W, d), 2)
    got = O.pool(O.tile(x))
    Hp, Wp = H // 4, W // 4
    for tc in range(T // 4):
        for yc in range(Hp):
            for xc in range(Wp):
                c = (tc * Hp + yc) * Wp + xc
                acc = np.zeros(d)
                for t in range(4):
                    for y in range(4):
                        for xx in range(4):
                            acc += x[4 * tc + t, 4 * yc + y, 4 * xc + xx]
                np.testing.assert_allclose(got[c], acc / 64, rtol=1e-14)
    np.testing.assert_allclose(got.sum(0) * 64, x.reshape(-1, d).sum(0), rtol=1e-12)
    np.testing.assert_array_equal(O.pool(O.tile(np.full((4, 4, 8, 3), 2.5))), np.full((2, 3), 2.5))


# -------------------------------------------------------------- step 2: coarse
def test_coarse_matches_sdpa():
    qc, kc, vc = _rand((40, 16), 3), _rand((40, 16), 4), _rand((40, 16), 5)
    s = 0.3
    S, A, Oc, lse = O.coarse_attention(qc, kc, vc, s)
    ref = F.scaled_dot_product_attention(*(torch.from_numpy(t)[None] for t in (qc, kc, vc)),
                                         scale=s)[0].numpy()
    np.testing.assert_allclose(Oc, ref, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(A.sum(1), 1.0, rtol=1e-14)
    ref_lse = torch.logsumexp(torch.from_numpy(S), dim=1).numpy()
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-14)
    np.testing.assert_allclose(S, s * qc @ kc.T, rtol=1e-12, atol=1e-14)


def test_coarse_uniform_closed_form():
    """Equal keys give uniform weights: O_c is the mean of V_c in every row."""
    qc = _rand((6, 4), 6)
    kc = np.tile(_rand((1, 4), 7), (6, 1))
    vc = _rand((6, 4), 8)
    _, A, Oc, lse = O.coarse_attention(qc, kc, vc, 1.0)
    np.testing.assert_allclose(A, 1 / 6, rtol=1e-14)
    np.testing.assert_allclose(Oc, np.tile(vc.mean(0), (6, 1)), rtol=1e-13)
    np.testing.assert_allclose(lse, qc @ kc[0] + math.log(6), rtol=1e-13)


# --------------------------------------------------------------- step 3: top-K
def _topk_brute(row, k):
    """Sort (value desc, index asc) pairs by Python's sort and keep K."""
    pairs = sorted(((-v, j) for j, v in enumerate(row)))
    return sorted(j for _, j in pairs[:k])


def test_topk_brute_force_with_ties():
    rng = np.random.default_rng(9)
    s = rng.integers(0, 4, size=(30, 12)).astype(float)   # many ties
    for k in (1, 3, 7, 12):
        idx, margin = O.topk_rows(s, k)
        for i in range(s.shape[0]):
            assert list(idx[i]) == _topk_brute(s[i], k)
            sel = np.zeros(12, bool)
            sel[idx[i]] = True
            if k < 12:
                assert s[i][sel].min() >= s[i][~sel].max()
                srt = np.sort(s[i])[::-1]
                assert margin[i] == srt[k - 1] - srt[k]
            else:
                assert sel.all() and margin[i] == np.inf


def test_topk_rejects_bad_k():
    with pytest.raises(ValueError):
        O.topk_rows(np.zeros((2, 4)), 5)
    with pytest.raises(ValueError):
        O.topk_rows(np.zeros((2, 4)), 0)


def test_mask_list_round_trip_and_transpose():
    idx, lens = WL.random_lists(20, 20, 0, 9, seed=3)
    m = O.lists_to_mask(idx, lens, 20)
    assert np.array_equal(m.sum(1), lens)
    idx2, lens2 = O.mask_to_lists(m, stride=idx.shape[1])
    assert np.array_equal(lens2, lens)
    for i in range(20):
        assert np.array_equal(idx2[i, :lens[i]], idx[i, :lens[i]])
    k2q, kl = O.transpose_lists(idx, lens, 20)
    for j in range(20):
        for i in range(20):
            assert (i in k2q[j, :kl[j]]) == (j in idx[i, :lens[i]])
        assert np.all(np.diff(k2q[j, :kl[j]]) > 0)


def test_logit_error_bound_covers_fp32_pool_and_dot():
    """An fp32 recomputation of the coarse logits stays inside the bound."""
    w = WL.make_inputs("C2", heads=[0])
    qt, kt = O.tile(w["q"][0, 0].astype(np.float64)), O.tile(w["k"][0, 0].astype(np.float64))
    s = 1 / 8
    tau = O.logit_error_bound(qt, kt, s)
    qc32 = qt.astype(np.float32).sum(1, dtype=np.float32) / np.float32(64)
    kc32 = kt.astype(np.float32).sum(1, dtype=np.float32) / np.float32(64)
    s32 = (qc32 @ kc32.T).astype(np.float32) * np.float32(s)
    exact = s * (O.pool(qt) @ O.pool(kt).T)
    assert np.all(np.abs(s32 - exact).max(1) <= tau)
    assert np.all(tau < 1e-3)


def _bf16_round(x32):
    """Round fp32 values to the nearest bf16 (ties to even), kept as fp32."""
    b = x32.astype(np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000
    return b.astype(np.uint32).view(np.float32)


@pytest.mark.parametrize("name", ["C2", "C3"])
def test_logit_error_bound_covers_split_bf16_products(name):
    """The logits may be formed on bf16 matrix units from an exact split of
    each pooled fp32 value into three bf16 pieces, six piece products in two
    fp32 accumulators (hi*hi; hi*mid, mid*hi, hi*lo, lo*hi, mid*mid): the
    split is exact and an fp32 emulation of that arithmetic stays inside the
    bound; dropping the second accumulator would not."""
    w = WL.get(name)
    x = WL.make_inputs(name, heads=[0])
    qt, kt = O.tile(x["q"][0, 0].astype(np.float64)), O.tile(x["k"][0, 0].astype(np.float64))
    s = 1 / np.sqrt(w.head_dim)
    tau = O.logit_error_bound(qt, kt, s)
    exact = s * (O.pool(qt) @ O.pool(kt).T)

    def split(v):
        hi = _bf16_round(v)
        r1 = (v - hi).astype(np.float32)
        mid = _bf16_round(r1)
        lo = (r1 - mid).astype(np.float32)
        assert np.array_equal(_bf16_round(lo), lo)
        assert np.array_equal(hi.astype(np.float64) + mid + lo, v.astype(np.float64))
        return hi, mid, lo

    qc32 = qt.astype(np.float32).sum(1, dtype=np.float32) / np.float32(qt.shape[1])
    kc32 = kt.astype(np.float32).sum(1, dtype=np.float32) / np.float32(kt.shape[1])
    (qh, qm, ql), (kh, km, kl) = split(qc32), split(kc32)
    acc_hh = (qh @ kh.T).astype(np.float32)
    acc_x = np.zeros_like(acc_hh)
    for a_, b_ in ((qh, km), (qm, kh), (qh, kl), (ql, kh), (qm, km)):
        acc_x = (acc_x + (a_ @ b_.T).astype(np.float32)).astype(np.float32)
    s32 = ((acc_hh + acc_x).astype(np.float32) * np.float32(s)).astype(np.float32)
    assert np.all(np.abs(s32 - exact).max(1) <= tau)
    hh_only = (acc_hh * np.float32(s)).astype(np.float32)
    assert np.any(np.abs(hh_only - exact).max(1) > tau)


# --------------------------------------------------------------- step 4: fine
def test_fine_all_blocks_is_full_attention():
    """With every cube listed the fine stage is textbook attention (SDPA, float64)."""
    T, H, W, d = 8, 4, 8, 8
    q, k, v = _rand((T, H, W, d), 10), _rand((T, H, W, d), 11), _rand((T, H, W, d), 12)
    nc = T * H * W // 64
    idx = np.tile(np.arange(nc), (nc, 1))
    of, lse = O.fine_gathered(O.tile(q), O.tile(k), O.tile(v), idx, np.full(nc, nc), 0.4)
    ref = F.scaled_dot_product_attention(*(torch.from_numpy(t.reshape(1, -1, d)) for t in (q, k, v)),
                                         scale=0.4)[0].numpy()
    np.testing.assert_allclose(O.untile(of, T, H, W).reshape(-1, d), ref, rtol=1e-11, atol=1e-13)
    z = 0.4 * q.reshape(-1, d) @ k.reshape(-1, d).T
    np.testing.assert_allclose(O.untile_rows(lse, T, H, W).reshape(-1),
                               torch.logsumexp(torch.from_numpy(z), 1).numpy(), rtol=1e-13)


def test_fine_literal_equals_gathered_and_order_invariance():
    T, H, W, d = 8, 8, 4, 6
    q, k, v = _rand((T, H, W, d), 13), _rand((T, H, W, d), 14), _rand((T, H, W, d), 15)
    nc = T * H * W // 64
    idx, lens = WL.random_lists(nc, nc, 0, nc, seed=5)
    lens[0] = 0                                          # one empty list
    m = O.lists_to_mask(idx, lens, nc)
    of_l, lse_l = O.fine_literal(q, k, v, m, 0.5)
    of_g, lse_g = O.fine_gathered(O.tile(q), O.tile(k), O.tile(v), idx, lens, 0.5)
    np.testing.assert_allclose(O.untile(of_g, T, H, W), of_l, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(O.untile_rows(lse_g, T, H, W), lse_l, rtol=1e-13)
    assert np.all(of_g[0] == 0) and np.all(np.isneginf(lse_g[0]))
    # shuffled list order gives the same result
    rng = np.random.default_rng(1)
    idx_s = idx.copy()
    for i in range(nc):
        idx_s[i, :lens[i]] = rng.permutation(idx[i, :lens[i]])
    of_s, _ = O.fine_gathered(O.tile(q), O.tile(k), O.tile(v), idx_s, lens, 0.5)
    np.testing.assert_allclose(of_s, of_g, rtol=1e-12, atol=1e-14)


def test_fine_rows_of_p_sum_to_one():
    """V = constant c on every key gives O_f = c exactly where the row is live."""
    T, H, W, d = 4, 8, 8, 4
    q, k = _rand((T, H, W, d), 16), _rand((T, H, W, d), 17)
    v = np.full((T, H, W, d), 1.75)
    nc = 4
    idx, lens = WL.random_lists(nc, nc, 1, 3, seed=2)
    of, _ = O.fine_gathered(O.tile(q), O.tile(k), O.tile(v), idx, lens, 1.0)
    np.testing.assert_allclose(of, 1.75, rtol=1e-14)


# ------------------------------------------------------------ step 5: combine
def test_combine_gate_special_cases():
    oc, of = _rand((4, 4, 4, 3), 18), _rand((4, 4, 4, 3), 19)
    g = np.abs(_rand((4, 4, 4, 3), 20))
    np.testing.assert_array_equal(O.combine(oc, of, np.zeros_like(g), None), of)
    np.testing.assert_array_equal(O.combine(oc, of, None, np.zeros_like(g)), oc)
    np.testing.assert_allclose(O.combine(oc, of, 2 * g, g), 2 * oc * g + of * g, rtol=1e-15)


def test_repeat_coarse_matches_repeat_interleave():
    oc = _rand((1, 2, 8, 3), 21)          # 8 cubes of an 8x8x8 latent
    got = O.repeat_coarse(oc, 8, 8, 8)
    ref = torch.from_numpy(oc).reshape(1, 2, 2, 2, 2, 3)
    for ax in (2, 3, 4):
        ref = ref.repeat_interleave(4, dim=ax)
    np.testing.assert_array_equal(got, ref.numpy())


# ----------------------------------------------------------------- end to end
def _torch_vsa(q, k, v, g_c, g_f, mask, scale, pool_mode="mean", cube=(4, 4, 4), kcube=None):
    """Independent torch expression of the forward with a fixed block mask:
    avg_pool3d (or max_pool3d) pooling with the query cube (queries) or the
    key block (keys, values) as kernel, repeat_interleave broadcast,
    token-level masked softmax."""
    B, h, T, H, W, d = q.shape
    kcube = cube if kcube is None else kcube
    Tp, Hp, Wp = T // cube[0], H // cube[1], W // cube[2]
    pool3d = F.max_pool3d if pool_mode == "max" else F.avg_pool3d

    def pool(x, c):
        p = pool3d(x.permute(0, 1, 5, 2, 3, 4).reshape(B * h, d, T, H, W), tuple(c))
        return p.reshape(B, h, d, -1).transpose(-1, -2)

    qc, kc, vc = pool(q, cube), pool(k, kcube), pool(v, kcube)
    a = torch.softmax(scale * qc @ kc.transpose(-1, -2), dim=-1)
    oc = (a @ vc).reshape(B, h, Tp, Hp, Wp, d)
    for ax in (2, 3, 4):
        oc = oc.repeat_interleave(cube[ax - 2], dim=ax)
    def ids(c):
        cid = torch.arange((T // c[0]) * (H // c[1]) * (W // c[2])).reshape(T // c[0], H // c[1], W // c[2])
        for ax in (0, 1, 2):
            cid = cid.repeat_interleave(c[ax], dim=ax)
        return cid.reshape(-1)

    tok_mask = mask[:, :, ids(cube)][:, :, :, ids(kcube)]
    qr, kr, vr = (x.reshape(B, h, -1, d) for x in (q, k, v))
    z = (scale * qr @ kr.transpose(-1, -2)).masked_fill(~tok_mask, float("-inf"))
    of = (torch.softmax(z, dim=-1) @ vr).reshape(B, h, T, H, W, d)
    return oc * g_c + of * g_f


def test_forward_equals_independent_torch_expression():
    w = WL.make_inputs("C1")
    fwd = O.forward(w["q"], w["k"], w["v"], w["g_c"], w["g_f"], topk=2, with_literal=True)
    nc = 8
    mask = np.stack([[O.lists_to_mask(fwd["idx"][b, h], fwd["len"][b, h], nc)
                      for h in range(2)] for b in range(1)])
    ref = _torch_vsa(*(torch.from_numpy(w[x].astype(np.float64)) for x in ("q", "k", "v", "g_c", "g_f")),
                     torch.from_numpy(mask), 1 / 8)
    np.testing.assert_allclose(fwd["o"], ref.numpy(), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(fwd["o_f"], fwd["o_f_literal"], rtol=1e-12, atol=1e-14)
    assert np.all(np.diff(fwd["idx"], axis=-1) > 0)


def test_adaptation_start_equals_full_attention():
    """The pages: K = all cubes, G_c = 0 and G_f removed equals full attention
    (VSA summary page, section 2 'Pretrained adaptation'; reading notes key design 5)."""
    w = WL.make_inputs("C1")
    nc = 8
    fwd = O.forward(w["q"], w["k"], w["v"], np.zeros_like(w["g_c"]), None, topk=nc)
    for h in range(2):
        ref = F.scaled_dot_product_attention(
            *(torch.from_numpy(w[x][0, h].astype(np.float64).reshape(1, -1, 64)) for x in ("q", "k", "v")))
        np.testing.assert_allclose(fwd["o"][0, h].reshape(-1, 64), ref[0].numpy(), rtol=1e-11, atol=1e-13)


def test_topk_margin_consistent_with_selection():
    w = WL.make_inputs("C2", heads=[0])
    qt, kt = O.tile(w["q"][0, 0].astype(np.float64)), O.tile(w["k"][0, 0].astype(np.float64))
    S, _, _, _ = O.coarse_attention(O.pool(qt), O.pool(kt), O.pool(kt), 1 / 8)
    idx, margin = O.topk_rows(S, 32)
    assert np.all(margin >= 0)
    for i in range(0, 256, 37):
        sel = np.zeros(256, bool)
        sel[idx[i]] = True
        assert S[i][sel].min() - S[i][~sel].max() == pytest.approx(margin[i])


# ------------------------------------------------------------------- backward
def test_backward_matches_autograd_of_independent_expression():
    w = WL.make_inputs_custom(1, 2, 4, 8, 8, 8, dtype="f32", seed=3, scale=0.5)
    nc = 8
    idx, lens = WL.random_lists(nc, 2 * nc, 1, 5, seed=4)
    idx = idx.reshape(1, 2, nc, -1)
    lens = lens.reshape(1, 2, nc)
    fwd = O.forward(w["q"], w["k"], w["v"], w["g_c"], w["g_f"], topk=0, idx=idx, lens=lens)
    bwd = O.backward(w["q"], w["k"], w["v"], w["g_c"], w["g_f"], w["d_o"], fwd)
    mask = np.stack([[O.lists_to_mask(idx[0, h], lens[0, h], nc) for h in range(2)]])
    ts = {x: torch.from_numpy(w[x].astype(np.float64)).requires_grad_(True)
          for x in ("q", "k", "v", "g_c", "g_f")}
    out = _torch_vsa(ts["q"], ts["k"], ts["v"], ts["g_c"], ts["g_f"], torch.from_numpy(mask),
                     1 / math.sqrt(4))
    np.testing.assert_allclose(fwd["o"], out.detach().numpy(), rtol=1e-12, atol=1e-14)
    (out * torch.from_numpy(w["d_o"].astype(np.float64))).sum().backward()
    for name, key in (("dq", "q"), ("dk", "k"), ("dv", "v"), ("dg_c", "g_c"), ("dg_f", "g_f")):
        np.testing.assert_allclose(bwd[name], ts[key].grad.numpy(), rtol=1e-10, atol=1e-12,
                                   err_msg=name)


@pytest.mark.parametrize("cube", [(2, 4, 4), (4, 4, 8), (1, 8, 8)])
def test_general_cube_forward_backward_match_autograd(cube):
    """Other cube shapes (tile size B = 32, 128, 64): forward and backward of
    the oracle against the independent expression pooled with avg_pool3d over
    the cube, and the literal masked-dense form against the gathered one."""
    ct, ch, cw = cube
    T, H, W = 2 * ct, 2 * ch, 2 * cw
    w = WL.make_inputs_custom(1, 2, 4, T, H, W, dtype="f32", seed=8, scale=0.5)
    nc = 8
    idx, lens = WL.random_lists(nc, 2 * nc, 1, 5, seed=9)
    idx, lens = idx.reshape(1, 2, nc, -1), lens.reshape(1, 2, nc)
    fwd = O.forward(w["q"], w["k"], w["v"], w["g_c"], w["g_f"], topk=0, idx=idx, lens=lens,
                    with_literal=True, cube=cube)
    bwd = O.backward(w["q"], w["k"], w["v"], w["g_c"], w["g_f"], w["d_o"], fwd)
    mask = np.stack([[O.lists_to_mask(idx[0, h], lens[0, h], nc) for h in range(2)]])
    ts = {x: torch.from_numpy(w[x].astype(np.float64)).requires_grad_(True)
          for x in ("q", "k", "v", "g_c", "g_f")}
    out = _torch_vsa(ts["q"], ts["k"], ts["v"], ts["g_c"], ts["g_f"], torch.from_numpy(mask), 0.5, cube=cube)
    np.testing.assert_allclose(fwd["o"], out.detach().numpy(), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(fwd["o_f"], fwd["o_f_literal"], rtol=1e-12, atol=1e-14)
    (out * torch.from_numpy(w["d_o"].astype(np.float64))).sum().backward()
    for name, key in (("dq", "q"), ("dk", "k"), ("dv", "v"), ("dg_c", "g_c"), ("dg_f", "g_f")):
        np.testing.assert_allclose(bwd[name], ts[key].grad.numpy(), rtol=1e-10, atol=1e-12, err_msg=name)
    # adaptation start (K = all cubes, G_c = 0, G_f removed) is full attention for any cube
    full = O.forward(w["q"], w["k"], w["v"], np.zeros_like(w["g_c"]), None, topk=nc, cube=cube)
    for h in range(2):
        ref = F.scaled_dot_product_attention(
            *(torch.from_numpy(w[x][0, h].astype(np.float64).reshape(1, -1, 4)) for x in ("q", "k", "v")))
        np.testing.assert_allclose(full["o"][0, h].reshape(-1, 4), ref[0].numpy(), rtol=1e-11, atol=1e-13)


@pytest.mark.parametrize("cube,kcube", [((4, 4, 4), (2, 4, 4)), ((4, 4, 4), (4, 4, 8)), ((2, 4, 4), (4, 4, 4)),
                                       ((4, 4, 4), (1, 4, 4))])
def test_asymmetric_tiles_forward_backward_match_autograd(cube, kcube):
    """Query tiles and key blocks of different shapes (Bq x Bk tiles, the
    summary page's 64 x 16 example generalised): forward and backward against
    the independent expression, literal = gathered, and all key blocks kept
    with G_c = 0 and G_f removed equals full attention."""
    T, H, W = 8, 8, 16
    w = WL.make_inputs_custom(1, 2, 4, T, H, W, dtype="f32", seed=12, scale=0.5)
    nq = T * H * W // (cube[0] * cube[1] * cube[2])
    nk = T * H * W // (kcube[0] * kcube[1] * kcube[2])
    idx, lens = WL.random_lists(nk, 2 * nq, 1, min(nk, 5), seed=13)
    idx, lens = idx.reshape(1, 2, nq, -1), lens.reshape(1, 2, nq)
    fwd = O.forward(w["q"], w["k"], w["v"], w["g_c"], w["g_f"], topk=0, idx=idx, lens=lens,
                    with_literal=True, cube=cube, kcube=kcube)
    assert fwd["q_c"].shape[-2] == nq and fwd["k_c"].shape[-2] == nk and fwd["s_c"].shape[-2:] == (nq, nk)
    bwd = O.backward(w["q"], w["k"], w["v"], w["g_c"], w["g_f"], w["d_o"], fwd)
    mask = np.stack([[O.lists_to_mask(idx[0, h], lens[0, h], nk) for h in range(2)]])
    ts = {x: torch.from_numpy(w[x].astype(np.float64)).requires_grad_(True)
          for x in ("q", "k", "v", "g_c", "g_f")}
    out = _torch_vsa(ts["q"], ts["k"], ts["v"], ts["g_c"], ts["g_f"], torch.from_numpy(mask), 0.5,
                     cube=cube, kcube=kcube)
    np.testing.assert_allclose(fwd["o"], out.detach().numpy(), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(fwd["o_f"], fwd["o_f_literal"], rtol=1e-12, atol=1e-14)
    (out * torch.from_numpy(w["d_o"].astype(np.float64))).sum().backward()
    for name, key in (("dq", "q"), ("dk", "k"), ("dv", "v"), ("dg_c", "g_c"), ("dg_f", "g_f")):
        np.testing.assert_allclose(bwd[name], ts[key].grad.numpy(), rtol=1e-10, atol=1e-12, err_msg=name)
    full = O.forward(w["q"], w["k"], w["v"], np.zeros_like(w["g_c"]), None, topk=nk, cube=cube, kcube=kcube)
    for h in range(2):
        ref = F.scaled_dot_product_attention(
            *(torch.from_numpy(w[x][0, h].astype(np.float64).reshape(1, -1, 4)) for x in ("q", "k", "v")))
        np.testing.assert_allclose(full["o"][0, h].reshape(-1, 4), ref[0].numpy(), rtol=1e-11, atol=1e-13)


def test_max_pool_matches_max_pool3d_and_first_argmax():
    x = _rand((8, 8, 12, 5), 31)                       # T, H, W, d
    xt = O.tile(x[None, None])[0, 0]
    ref = F.max_pool3d(torch.from_numpy(x).permute(3, 0, 1, 2)[None], 4)[0]
    np.testing.assert_array_equal(O.pool(xt, "max"), ref.reshape(5, -1).T.numpy())
    # ties: the gradient of every (cube, channel) goes to its first maximum
    xt2 = np.round(xt * 2) / 2                         # many equal values
    g = _rand(O.pool(xt2, "max").shape, 32)
    got = O.pool_backward(g, xt2, "max")
    for c in range(xt2.shape[0]):
        for ch in range(5):
            col = xt2[c, :, ch]
            first = int(np.flatnonzero(col == col.max())[0])
            want = np.zeros(64)
            want[first] = g[c, ch]
            np.testing.assert_array_equal(got[c, :, ch], want)


def test_max_pool_forward_backward_match_autograd():
    """Max-pool variant end to end against the independent expression with
    max_pool3d (continuous inputs: no ties, so the subgradient is unique)."""
    w = WL.make_inputs_custom(1, 2, 4, 8, 8, 8, dtype="f32", seed=5, scale=0.5)
    nc = 8
    idx, lens = WL.random_lists(nc, 2 * nc, 1, 5, seed=6)
    idx, lens = idx.reshape(1, 2, nc, -1), lens.reshape(1, 2, nc)
    fwd = O.forward(w["q"], w["k"], w["v"], w["g_c"], w["g_f"], topk=0, idx=idx, lens=lens, pool_mode="max")
    bwd = O.backward(w["q"], w["k"], w["v"], w["g_c"], w["g_f"], w["d_o"], fwd)
    mask = np.stack([[O.lists_to_mask(idx[0, h], lens[0, h], nc) for h in range(2)]])
    ts = {x: torch.from_numpy(w[x].astype(np.float64)).requires_grad_(True)
          for x in ("q", "k", "v", "g_c", "g_f")}
    out = _torch_vsa(ts["q"], ts["k"], ts["v"], ts["g_c"], ts["g_f"], torch.from_numpy(mask), 0.5, "max")
    np.testing.assert_allclose(fwd["o"], out.detach().numpy(), rtol=1e-12, atol=1e-14)
    (out * torch.from_numpy(w["d_o"].astype(np.float64))).sum().backward()
    for name, key in (("dq", "q"), ("dk", "k"), ("dv", "v"), ("dg_c", "g_c"), ("dg_f", "g_f")):
        np.testing.assert_allclose(bwd[name], ts[key].grad.numpy(), rtol=1e-10, atol=1e-12, err_msg=name)
    # the variant differs from the mean-pool operator
    mean = O.forward(w["q"], w["k"], w["v"], w["g_c"], w["g_f"], topk=0, idx=idx, lens=lens)
    assert np.abs(mean["o"] - fwd["o"]).max() > 1e-3


def test_backward_finite_differences_topk_mode():
    """Central differences along random directions, top-K mode, where every
    row's selection margin is far above the perturbation (mask constant)."""
    w = WL.make_inputs_custom(1, 1, 4, 8, 8, 8, dtype="f32", seed=11, scale=1.0)
    args = {x: w[x].astype(np.float64) for x in ("q", "k", "v", "g_c", "g_f", "d_o")}
    fwd = O.forward(args["q"], args["k"], args["v"], args["g_c"], args["g_f"], topk=3)
    assert fwd["margin"].min() > 1e-4
    bwd = O.backward(args["q"], args["k"], args["v"], args["g_c"], args["g_f"], args["d_o"], fwd)
    rng = np.random.default_rng(0)
    eps = 1e-6

    def loss(a):
        f = O.forward(a["q"], a["k"], a["v"], a["g_c"], a["g_f"], topk=3)
        assert np.array_equal(f["idx"], fwd["idx"])
        return float((f["o"] * args["d_o"]).sum())

    for name, key in (("dq", "q"), ("dk", "k"), ("dv", "v"), ("dg_c", "g_c"), ("dg_f", "g_f")):
        dirn = rng.standard_normal(args[key].shape)
        ap = dict(args); ap[key] = args[key] + eps * dirn
        am = dict(args); am[key] = args[key] - eps * dirn
        fd = (loss(ap) - loss(am)) / (2 * eps)
        an = float((bwd[name] * dirn).sum())
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)


def test_backward_empty_lists_give_coarse_only_gradient():
    """With every list empty the fine stage contributes nothing; dV then comes
    from the coarse path alone and spreads evenly over each cube."""
    w = WL.make_inputs_custom(1, 1, 4, 4, 4, 8, dtype="f32", seed=5)
    idx = np.full((1, 1, 2, 1), -1)
    lens = np.zeros((1, 1, 2), np.int64)
    fwd = O.forward(w["q"], w["k"], w["v"], w["g_c"], w["g_f"], topk=0, idx=idx, lens=lens)
    assert np.all(fwd["o_f"] == 0)
    bwd = O.backward(w["q"], w["k"], w["v"], w["g_c"], w["g_f"], w["d_o"], fwd)
    dvt = O.tile(bwd["dv"])[0, 0]
    np.testing.assert_allclose(dvt, np.repeat(dvt[:, :1], 64, axis=1), rtol=1e-13)
    np.testing.assert_allclose(dvt[:, 0] * 64, bwd["dv_c"][0, 0], rtol=1e-13)


# ----------------------------------------------------------- page-stated facts
def test_page_facts_on_work_accounting():
    facts = {f["id"]: f for f in json.load(open(GOLDEN))["facts"]}
    cube = facts["cube_and_block"]["cube"]
    assert int(np.prod(cube)) == facts["cube_and_block"]["block"] == O.TILE
    T, H, W = facts["pseudocode_setting"]["video"]
    k = facts["pseudocode_setting"]["topk"]
    assert k == facts["default_topk"]["topk"]
    n = T * H * W
    nc = n // O.TILE
    assert abs(n - facts["sequence_16k"]["tokens_approx"]) / n < 0.05
    lens = np.full(nc, k)
    assert 1 - lens.sum() / nc ** 2 == facts["sparsity_at_tile_64"]["sparsity"]
    d = 64
    fine = O.fine_flops_forward(lens, d)
    dense = O.dense_flops(1, 1, n, d)
    assert dense / fine == pytest.approx(facts["attention_flop_reduction"]["factor_approx"], rel=0.05)
    coarse = O.coarse_flops(1, 1, nc, d)
    assert coarse / dense < facts["coarse_share_of_attention"]["max_fraction"]
    assert coarse / (coarse + fine) < facts["coarse_share_of_total"]["max_fraction"]


def test_pool_error_bound_exactness_claim():
    """Where the bound claims an fp32 mean-pool is exact, fp32 sums in several
    orders (forward, reverse, pairwise, shuffled) all equal the exact sum;
    elsewhere the error stays inside the bound."""
    w = WL.make_inputs("C3", heads=[2], gates=False)
    xt = O.tile(w["q"][0, 0].astype(np.float64))[:40]
    bound = O._pool_error_bound(xt, 8)
    exact = xt.sum(axis=1) / 64
    x32 = xt.astype(np.float32)
    rng = np.random.default_rng(0)
    orders = [np.arange(64), np.arange(64)[::-1], rng.permutation(64), rng.permutation(64)]
    for order in orders:
        acc = np.zeros(x32.shape[::2], np.float32)
        for l in order:
            acc = (acc + x32[:, l, :]).astype(np.float32)
        got = acc.astype(np.float64) / 64
        assert np.all(np.abs(got - exact) <= bound)
    pair = x32.copy()
    while pair.shape[1] > 1:
        pair = (pair[:, 0::2, :] + pair[:, 1::2, :]).astype(np.float32)
    assert np.all(np.abs(pair[:, 0, :].astype(np.float64) / 64 - exact) <= bound)
    assert (bound == 0).mean() > 0.9


# ------------------------------------------------- precision detection (tau)
def test_bf16_exact_detects_bf16_values():
    """_bf16_exact decides how many significant bits the inputs carry, hence
    tau and which top-K rows must match bit for bit. bf16-rounded values
    (torch's RNE conversion) are detected; generic fp32 values are not; a
    single fp32 value among bf16 ones is enough to fail."""
    import torch
    rng = np.random.default_rng(3)
    x = rng.standard_normal((2, 3, 8, 8, 8, 64)).astype(np.float32)
    xb = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert O._bf16_exact(xb)
    assert not O._bf16_exact(x)
    y = xb.copy()
    y.flat[12345] = np.float32(1.0) + np.float32(2.0 ** -20)
    assert not O._bf16_exact(y)
    assert O._bf16_exact(np.zeros(4, np.float32))
    # float64 inputs holding bf16 values are bf16-exact too (the check goes
    # through fp32, which represents them exactly)
    assert O._bf16_exact(xb.astype(np.float64))


def test_forward_picks_sig_bits_from_input_precision():
    """forward() bounds the pooling error with 8 significant bits for bf16
    inputs and 24 for generic fp32 inputs: its tau equals logit_error_bound
    called with those bits, and the fp32 bound is the larger one."""
    import torch
    rng = np.random.default_rng(4)
    shape = (1, 1, 8, 8, 16, 64)
    x32 = {n: rng.standard_normal(shape).astype(np.float32) for n in "qkv"}
    xbf = {n: torch.from_numpy(a).to(torch.bfloat16).to(torch.float32).numpy() for n, a in x32.items()}
    s = 1 / 8.0
    for xs, bits in ((xbf, 8), (x32, 24)):
        f = O.forward(xs["q"], xs["k"], xs["v"], topk=3)
        qt = O.tile(xs["q"].astype(np.float64))[0, 0]
        kt = O.tile(xs["k"].astype(np.float64))[0, 0]
        assert np.array_equal(f["tau"][0, 0], O.logit_error_bound(qt, kt, s, sig_bits=bits))
    f32 = O.forward(x32["q"], x32["k"], x32["v"], topk=3)["tau"]
    qt = O.tile(x32["q"].astype(np.float64))[0, 0]
    kt = O.tile(x32["k"].astype(np.float64))[0, 0]
    assert np.all(f32[0, 0] > O.logit_error_bound(qt, kt, s, sig_bits=8))
