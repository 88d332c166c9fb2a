"""Parity of the HIP path (through the C ABI) with the float64 CPU oracle.

Bars (from the operator's contract):
  * index lists: bit-exact on every row whose top-K margin exceeds twice the
    fp32 logit error bound; other (near-tie) rows must hold a valid top-K set;
  * fp32 problems: max |gpu - oracle| <= 1e-4;
  * bf16 problems: max |gpu - oracle| / max |oracle| <= 2e-2 per tensor;
  * fp32 intermediates of bf16 problems (pooled means, coarse output): 1e-4
    relative (the inputs are exact; fp32 rounding differs, and for the
    coarse output the head / tail bf16 split of its product, at most 3 * 2^-16
    relative per term).
Outputs are compared with the oracle re-run on the GPU's own lists, so a
legitimate near-tie choice cannot fail an output comparison.
"""
import dataclasses
import functools

import numpy as np
import pytest
import torch

import block_sparse_video_cube_amd as V
import workloads as WL
from oracle import vsa_oracle as O

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
BF16_REL = 2e-2
F32_ABS = 1e-4
# Sanity bound on the share of rows whose top-K margin is within the logit
# error bound (about 0.6% / 1.9% / 2.5% on the 16x32x32 / 480p / 720p inputs).
NEAR_FRAC = 0.05
# LSE_f bound: l is the fp32 sum of the probabilities whose bf16-rounded
# values multiply V, so however l is summed it is within the bf16 half-ulp
# relative error 2^-8 of the exact sum, i.e. |ln l - ln l_exact| <= 2^-8;
# plus fp32 slack.
LSE_ABS = 2.0 ** -8 + 1e-4


def dev(x, dtype):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV).to(dtype).contiguous()


def host(t):
    return t.detach().float().cpu().numpy() if t.dtype != torch.int32 else t.cpu().numpy()


def rel_err(got, ref):
    return float(np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-30))


def assert_close(got, ref, dtype, name, rel=BF16_REL, abs_=F32_ABS):
    if dtype == "f32":
        err = float(np.abs(got - ref).max())
        assert err <= abs_, f"{name}: max abs err {err:.3e} > {abs_}"
    else:
        err = rel_err(got, ref)
        assert err <= rel, f"{name}: rel err {err:.3e} > {rel}"


def problem_of(w, **kw):
    d = dict(B=w.B, heads=w.heads, T=w.T, H=w.H, W=w.W, head_dim=w.head_dim, dtype=w.dtype, topk=w.topk,
             list_stride=w.list_stride)
    d.update(kw)
    return V.Problem(**d)


def inputs_to_dev(x, dtype):
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    out = {k: dev(x[k], td) for k in ("q", "k", "v", "g_c", "g_f", "d_o") if k in x}
    for k in ("idx", "len"):
        if k in x:
            out[k] = dev(x[k], torch.int32)
    return out


def check_topk(gpu_idx, ref, k):
    """Index parity protocol. Returns the number of near-tie rows.

    Every id must lie in [0, Nk) and every row be strictly increasing. Rows
    whose K-th / (K+1)-th margin exceeds 2 tau must equal the oracle's list
    bit for bit. A near-tie row passes if its set is a valid top-K under the
    error bound: no chosen block is clearly below the K-th logit
    (S_j >= S_(K) - 2 tau) and every block clearly above it
    (S_j > S_(K) + 2 tau) is chosen."""
    s, tau, margin, ridx = ref["s_c"], ref["tau"], ref["margin"], ref["idx"]
    nk = s.shape[-1]
    assert gpu_idx.min() >= 0 and gpu_idx.max() < nk, (int(gpu_idx.min()), int(gpu_idx.max()), nk)
    assert np.all(np.diff(gpu_idx, axis=-1) > 0)
    strict = margin > 2 * tau
    same = (gpu_idx == ridx).all(axis=-1)
    bad = np.argwhere(strict & ~same)
    assert bad.size == 0, f"{len(bad)} rows with a clear top-K margin differ, e.g. {bad[:3].tolist()}"
    near = np.argwhere(~strict)
    for b, h, i in near:
        row = s[b, h, i]
        t = 2 * tau[b, h, i]
        kth = np.sort(row)[::-1][k - 1]
        chosen = np.zeros(nk, bool)
        chosen[gpu_idx[b, h, i]] = True
        assert np.all(row[chosen] >= kth - t), (b, h, i)
        assert np.all(chosen[row > kth + t]), (b, h, i)
    return len(near)


# ------------------------------------------------------------------ stages
@pytest.mark.parametrize("name", ["C1", "C2", "C3"])
def test_pool_parity(name):
    w = WL.get(name)
    x = WL.make_inputs(name, heads=[0, w.heads - 1], gates=False)
    p = problem_of(w, heads=2)
    d = inputs_to_dev(x, w.dtype)
    qc, kc, vc = V.pool(p, d["q"], d["k"], d["v"])
    torch.cuda.synchronize()
    for got, src in ((qc, "q"), (kc, "k"), (vc, "v")):
        ref = O.pool(O.tile(x[src].astype(np.float64)))
        err = rel_err(host(got), ref)
        assert err <= 1e-5, (src, err)


@pytest.mark.parametrize("name", ["C1", "C2", "C3"])
def test_coarse_parity_and_topk_protocol(name):
    w = WL.get(name)
    heads = list(range(w.heads)) if w.heads <= 12 else [0, 5, 11]
    heads = heads[:4]
    x = WL.make_inputs(name, heads=heads, gates=False)
    p = problem_of(w, heads=len(heads))
    d = inputs_to_dev(x, w.dtype)
    qc, kc, vc = V.pool(p, d["q"], d["k"], d["v"])
    oc, lse, idx, lens = V.coarse(p, qc, kc, vc)
    torch.cuda.synchronize()
    ref = O.forward(x["q"], x["k"], x["v"], topk=w.topk)
    near = check_topk(host(idx), ref, w.topk)
    assert near <= NEAR_FRAC * idx.shape[0] * idx.shape[1] * idx.shape[2] + 2
    assert np.all(host(lens) == w.topk)
    assert rel_err(host(oc), ref["o_c"]) <= 1e-4
    assert float(np.abs(host(lse) - ref["lse_c"]).max()) <= 1e-4 * max(1.0, np.abs(ref["lse_c"]).max())


@pytest.mark.parametrize("name,heads", [("C1", 2), ("C2", 2), ("C3", 2)])
def test_fine_forward_parity_ragged_lists(name, heads):
    """Explicit ragged lists: lengths 0..Nc, including empty and full rows."""
    w = WL.get(name)
    x = WL.make_inputs(name, heads=list(range(heads)), gates=False)
    nc = w.Nc
    stride = nc
    idx, lens = WL.random_lists(nc, heads * nc, 0, nc, seed=7, stride=stride)
    lens[0], lens[1] = 0, nc
    idx[1, :nc] = np.arange(nc)
    idx = idx.reshape(1, heads, nc, stride)
    lens = lens.reshape(1, heads, nc)
    p = problem_of(w, heads=heads, topk=0, list_stride=stride)
    d = inputs_to_dev(x, w.dtype)
    ws = V.workspace(p, d["q"])
    V.pool(p, d["q"], d["k"], d["v"])
    of, lse = V.fine_forward(p, d["q"], d["k"], d["v"], dev(idx, torch.int32), dev(lens, torch.int32), ws=ws)
    torch.cuda.synchronize()
    ref = O.forward(x["q"], x["k"], x["v"], topk=0, idx=idx, lens=lens)
    assert_close(host(of), ref["o_f"], w.dtype, "o_f")
    got_lse = host(lse)
    live = np.isfinite(ref["lse_f"])
    assert np.array_equal(np.isfinite(got_lse), live)
    assert float(np.abs(got_lse[live] - ref["lse_f"][live]).max()) <= LSE_ABS
    assert np.all(host(of)[~live] == 0)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("case", ["ramp", "jump"])
def test_fine_forward_rising_logits(case, d):
    """Logits that rise along the list far beyond the first chunk's maximum,
    so the online softmax must move its reference maximum mid-row: "ramp" adds
    about 3 nats per key cube (several moves per row), "jump" puts the last
    key cube 100 nats above the rest (2^144 overflows fp32 before the move).
    Every query cube lists every key cube in ascending order."""
    T, H, W, heads = 8, 8, 16, 2
    nc = T * H * W // 64
    rng = np.random.default_rng(11 + d)
    u = np.ones(d, np.float32)
    q = (u + 0.1 * rng.standard_normal((1, heads, T, H, W, d))).astype(np.float32)
    k = (0.1 * rng.standard_normal((1, heads, T, H, W, d))).astype(np.float32)
    v = rng.standard_normal((1, heads, T, H, W, d)).astype(np.float32)
    # key cube j of the (4, 4, 4) grid: tokens t in [4tc, 4tc+4), y in [4yc, ..), x in [4xc, ..)
    for j in range(nc):
        tc, r = divmod(j, (H // 4) * (W // 4))
        yc, xc = divmod(r, W // 4)
        b = 3.0 * j if case == "ramp" else (100.0 if j == nc - 1 else 0.0)
        k[:, :, 4 * tc:4 * tc + 4, 4 * yc:4 * yc + 4, 4 * xc:4 * xc + 4, :] += b * u / np.sqrt(d)
    q, k, v = (WL.round_bf16(a) for a in (q, k, v))
    idx = np.broadcast_to(np.arange(nc, dtype=np.int32), (1, heads, nc, nc)).copy()
    lens = np.full((1, heads, nc), nc, np.int32)
    p = V.Problem(1, heads, T, H, W, d, topk=0, list_stride=nc)
    tq, tk, tv = (dev(a, torch.bfloat16) for a in (q, k, v))
    of, lse = V.fine_forward(p, tq, tk, tv, dev(idx, torch.int32), dev(lens, torch.int32))
    torch.cuda.synchronize()
    ref = O.forward(q, k, v, topk=0, idx=idx, lens=lens)
    assert np.all(np.isfinite(host(of))) and np.all(np.isfinite(host(lse)))
    assert_close(host(of), ref["o_f"], "bf16", "o_f")
    assert float(np.abs(host(lse) - ref["lse_f"]).max()) <= LSE_ABS


@pytest.mark.parametrize("name", ["C1", "C2"])
def test_combine_parity(name):
    w = WL.get(name)
    x = WL.make_inputs(name, heads=[0, 1])
    p = problem_of(w, heads=2)
    rng = np.random.default_rng(3)
    oc = rng.standard_normal((1, 2, w.Nc, w.head_dim)).astype(np.float32)
    of = x["v"]                                  # any dtype-exact tensor
    d = inputs_to_dev(x, w.dtype)
    td = p.torch_dtype
    for gc, gf in ((d["g_c"], d["g_f"]), (None, d["g_f"]), (d["g_c"], None), (None, None)):
        o = V.combine(p, dev(oc, torch.float32), dev(of, td), gc, gf)
        torch.cuda.synchronize()
        ref = O.combine(O.repeat_coarse(oc.astype(np.float64), w.T, w.H, w.W), of.astype(np.float64),
                        None if gc is None else x["g_c"].astype(np.float64),
                        None if gf is None else x["g_f"].astype(np.float64))
        assert_close(host(o), ref, w.dtype, "o", rel=2 ** -7, abs_=1e-5)


# ------------------------------------------------------------------ end to end
def run_forward_and_compare(name, heads=None, training=False, gates=True):
    w = WL.get(name)
    hs = list(range(w.heads)) if heads is None else heads
    x = WL.make_inputs(name, heads=hs)
    p = problem_of(w, heads=len(hs))
    d = inputs_to_dev(x, w.dtype)
    gc, gf = (d["g_c"], d["g_f"]) if gates else (None, None)
    if w.topk > 0:
        o, idx, lens, saved = V.forward(p, d["q"], d["k"], d["v"], gc, gf, training=training)
    else:
        o, idx, lens, saved = V.forward(p, d["q"], d["k"], d["v"], gc, gf, idx=d["idx"], lens=d["len"],
                                        training=training)
    torch.cuda.synchronize()
    gi, gl = host(idx), host(lens)
    xg = (x["g_c"], x["g_f"]) if gates else (None, None)
    if w.topk > 0:
        ref_sel = O.forward(x["q"], x["k"], x["v"], topk=w.topk)
        near = check_topk(gi, ref_sel, w.topk)
    else:
        near = 0
    ref = O.forward(x["q"], x["k"], x["v"], *xg, topk=0, idx=gi, lens=gl)
    assert_close(host(o), ref["o"], w.dtype, f"{name} o")
    return near, (x, d, p, idx, lens, saved, ref)


@pytest.mark.parametrize("name", ["C1", "C2"])
@pytest.mark.parametrize("training", [False, True])
def test_forward_end_to_end(name, training):
    run_forward_and_compare(name, training=training)


def test_forward_480p_all_heads():
    """The 480p workload at full size (all 12 heads): selection and outputs
    of every query cube against the oracle."""
    w = WL.get("C3")
    near, _ = run_forward_and_compare("C3")
    assert near <= NEAR_FRAC * w.heads * w.Nc + 2


def test_forward_ungated():
    run_forward_and_compare("C2", heads=[3], gates=False)


def test_forward_saved_tensors():
    _, (x, d, p, idx, lens, saved, ref) = run_forward_and_compare("C2", heads=[1, 2], training=True)
    # the saved O_f / LSE_f equal the fine stage of the oracle on the same lists
    w = WL.get("C2")
    nbh, nc, D, N = 2, w.Nc, w.head_dim, w.N
    raw = saved
    off = 0

    def take(n, dtype, esize):
        nonlocal off
        t = raw[off:off + n * esize].view(dtype)
        off += (n * esize + 255) // 256 * 256
        return t

    for _ in range(4):
        take(nbh * nc * D, torch.float32, 4)
    take(nbh * nc, torch.float32, 4)
    lse_f = take(nbh * N, torch.float32, 4).reshape(1, 2, w.T, w.H, w.W)
    of = take(nbh * N * D, torch.bfloat16, 2).reshape(1, 2, w.T, w.H, w.W, D)
    assert_close(host(of), ref["o_f"], "bf16", "saved o_f")
    assert float(np.abs(host(lse_f) - ref["lse_f"]).max()) <= LSE_ABS


@functools.lru_cache(maxsize=1)
def _inputs_720p():
    """The 720p workload's inputs (all 40 heads), generated once per session."""
    return WL.make_inputs("C4")


# Heads of the 720p workload checked against the oracle: every query cube's
# selection and outputs (the oracle's fine stage costs about 1.6 s a head).
HEADS_720P = [0, 5, 10, 15, 21, 26, 33, 39]


@pytest.mark.timeout(900)
def test_forward_720p_heads():
    """The benchmark configuration at full size (all 40 heads on the GPU, the
    launch bench.py times); the oracle checks 8 heads completely: selection
    and the output of every query cube."""
    w = WL.get("C4")
    print("[720p] generating inputs", flush=True)
    x = _inputs_720p()
    print("[720p] running the HIP forward", flush=True)
    p = problem_of(w)
    d = inputs_to_dev(x, w.dtype)
    o, idx, lens, _ = V.forward(p, d["q"], d["k"], d["v"], d["g_c"], d["g_f"])
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all()
    heads = HEADS_720P
    gi = host(idx)[:, heads]
    assert (host(lens) == w.topk).all()
    got_o = host(o[:, heads])
    del o, d
    near = 0
    s = 1 / np.sqrt(w.head_dim)
    for hi, h in enumerate(heads):
        print(f"[720p] oracle head {h}", flush=True)
        qt, kt, vt, gct, gft = (O.tile(x[n][0, h].astype(np.float64)) for n in ("q", "k", "v", "g_c", "g_f"))
        qc, kc, vc = O.pool(qt), O.pool(kt), O.pool(vt)
        S, _, oc, _ = O.coarse_attention(qc, kc, vc, s)
        ridx, margin = O.topk_rows(S, w.topk)
        tau = O.logit_error_bound(qt, kt, s, sig_bits=8)
        ref = {"s_c": S[None, None], "tau": tau[None, None], "margin": margin[None, None], "idx": ridx[None, None]}
        near += check_topk(gi[:, hi:hi + 1], ref, w.topk)
        of_t, _ = O.fine_gathered(qt, kt, vt, gi[0, hi], np.full(w.Nc, w.topk), s)
        ref_o = oc[:, None, :] * gct + of_t * gft
        err = rel_err(O.tile(got_o[0, hi]), ref_o)
        assert err <= BF16_REL, (h, err)
    print(f"[720p] near-tie rows {near} of {len(heads) * w.Nc}", flush=True)
    assert near <= NEAR_FRAC * len(heads) * w.Nc + 2


@pytest.mark.timeout(900)
@pytest.mark.parametrize("T,H,W", [(32, 64, 64), (32, 128, 128)])
def test_forward_max_cubes_sampled(T, H, W):
    """The largest rows the coarse kernel holds in registers (32x64x64
    latent, 2048 cubes, 32 logits per lane) and the largest coarse problem
    the library accepts (32x128x128, Nc = vsa_max_cubes() = 8192 cubes, 524288
    tokens, rows streamed). Selection checked for every query cube, outputs
    for 32 sampled query cubes."""
    d, k = 64, 32
    nc = T * H * W // 64
    assert nc <= V.max_cubes()
    if T * H == 32 * 128:
        assert nc == V.max_cubes()
    print(f"[max cubes] {T}x{H}x{W}: {nc} cubes", flush=True)
    x = WL.make_inputs_custom(1, 1, d, T, H, W, dtype="bf16", seed=41)
    p = V.Problem(1, 1, T, H, W, d, topk=k)
    dd = inputs_to_dev(x, "bf16")
    o, idx, lens, _ = V.forward(p, dd["q"], dd["k"], dd["v"], dd["g_c"], dd["g_f"])
    torch.cuda.synchronize()
    gi = host(idx)
    assert (host(lens) == k).all()
    qt, kt, vt = (O.tile(x[n].astype(np.float64))[0, 0] for n in ("q", "k", "v"))
    s = 1 / np.sqrt(d)
    S, _, oc, _ = O.coarse_attention(O.pool(qt), O.pool(kt), O.pool(vt), s)
    ridx, margin = O.topk_rows(S, k)
    tau = O.logit_error_bound(qt, kt, s, sig_bits=8)
    ref = {"s_c": S[None, None], "tau": tau[None, None], "margin": margin[None, None], "idx": ridx[None, None]}
    near = check_topk(gi, ref, k)
    assert near <= NEAR_FRAC * nc + 2
    rows = np.sort(np.random.default_rng(1).choice(nc, 32, replace=False))
    of_rows, _ = O.fine_gathered(qt[rows], kt, vt, gi[0, 0][rows], np.full(32, k), s)
    gct = O.tile(x["g_c"].astype(np.float64))[0, 0][rows]
    gft = O.tile(x["g_f"].astype(np.float64))[0, 0][rows]
    ref_o = oc[rows][:, None, :] * gct + of_rows * gft
    got = O.tile(host(o))[0, 0][rows]
    assert rel_err(got, ref_o) <= BF16_REL


# ------------------------------------------------------------------ edge cases
def test_all_cubes_selected_is_full_attention():
    """K = Nc with G_c = 0 and no fine gate reproduces full attention."""
    x = WL.make_inputs_custom(1, 2, 64, 8, 8, 16, dtype="bf16", seed=4)
    p = V.Problem(1, 2, 8, 8, 16, 64, topk=16)
    d = inputs_to_dev(x, "bf16")
    zero = torch.zeros_like(d["q"])
    o, idx, lens, _ = V.forward(p, d["q"], d["k"], d["v"], zero, None)
    torch.cuda.synchronize()
    assert np.array_equal(host(idx), np.tile(np.arange(16), (1, 2, 16, 1)))
    for h in range(2):
        qf, kf, vf = (torch.from_numpy(x[k][0, h].astype(np.float64)).reshape(1, -1, 64) for k in ("q", "k", "v"))
        ref = torch.nn.functional.scaled_dot_product_attention(qf, kf, vf)[0].numpy()
        assert rel_err(host(o)[0, h].reshape(-1, 64), ref) <= BF16_REL


@pytest.mark.parametrize("dtype,d,k,stride", [("bf16", 64, 1, 3), ("bf16", 128, 5, 5), ("f32", 128, 3, 4),
                                              ("f32", 64, 8, 8)])
def test_shapes_and_k_range(dtype, d, k, stride):
    x = WL.make_inputs_custom(1, 3, d, 4, 8, 16, dtype=dtype, seed=9, scale=0.5)
    p = V.Problem(1, 3, 4, 8, 16, d, dtype=dtype, topk=k, list_stride=stride)
    dd = inputs_to_dev(x, dtype)
    o, idx, lens, _ = V.forward(p, dd["q"], dd["k"], dd["v"], dd["g_c"], dd["g_f"])
    torch.cuda.synchronize()
    gi = host(idx)
    if stride > k:
        assert np.all(gi[..., k:] == -1)
    gi = gi[..., :k]
    ref_sel = O.forward(x["q"], x["k"], x["v"], topk=k)
    check_topk(gi, ref_sel, k)
    ref = O.forward(x["q"], x["k"], x["v"], x["g_c"], x["g_f"], topk=0, idx=gi, lens=host(lens))
    assert_close(host(o), ref["o"], dtype, "o")


def test_scale_override():
    x = WL.make_inputs_custom(1, 1, 64, 8, 8, 8, dtype="bf16", seed=2)
    p = V.Problem(1, 1, 8, 8, 8, 64, topk=3, scale=0.37)
    d = inputs_to_dev(x, "bf16")
    o, idx, lens, _ = V.forward(p, d["q"], d["k"], d["v"], d["g_c"], d["g_f"])
    torch.cuda.synchronize()
    ref_sel = O.forward(x["q"], x["k"], x["v"], topk=3, scale=0.37)
    check_topk(host(idx), ref_sel, 3)
    ref = O.forward(x["q"], x["k"], x["v"], x["g_c"], x["g_f"], topk=0, idx=host(idx), lens=host(lens), scale=0.37)
    assert_close(host(o), ref["o"], "bf16", "o")


def test_repeat_calls_bitwise_identical():
    x = WL.make_inputs("C2", heads=[0, 1])
    p = problem_of(WL.get("C2"), heads=2)
    d = inputs_to_dev(x, "bf16")
    o1, i1, _, _ = V.forward(p, d["q"], d["k"], d["v"], d["g_c"], d["g_f"])
    o2, i2, _, _ = V.forward(p, d["q"], d["k"], d["v"], d["g_c"], d["g_f"])
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(i1, i2)


def test_validate_lists_device():
    p = V.Problem(1, 1, 8, 8, 8, 64, topk=0, list_stride=4)
    idx = np.array([[0, 2, 5, -1]] * 8, np.int32).reshape(1, 1, 8, 4)
    lens = np.full((1, 1, 8), 3, np.int32)
    V.validate_lists(p, dev(idx, torch.int32), dev(lens, torch.int32))
    bad = idx.copy()
    bad[0, 0, 5, 1] = 9
    with pytest.raises(V.VsaError) as e:
        V.validate_lists(p, dev(bad, torch.int32), dev(lens, torch.int32))
    assert e.value.status == 8
    badl = lens.copy()
    badl[0, 0, 2] = 7
    with pytest.raises(V.VsaError):
        V.validate_lists(p, dev(idx, torch.int32), dev(badl, torch.int32))


# ------------------------------------------------------------------ backward
def backward_compare(x, p, dtype, rel=BF16_REL, gates=True):
    d = inputs_to_dev(x, dtype)
    gc, gf = (d["g_c"], d["g_f"]) if gates else (None, None)
    o, idx, lens, saved = V.forward(p, d["q"], d["k"], d["v"], gc, gf, idx=d["idx"], lens=d["len"], training=True)
    g = V.backward(p, d["q"], d["k"], d["v"], gc, gf, idx, lens, saved, d["d_o"])
    torch.cuda.synchronize()
    xg = (x["g_c"], x["g_f"]) if gates else (None, None)
    fwd = O.forward(x["q"], x["k"], x["v"], *xg, topk=0, idx=x["idx"], lens=x["len"], pool_mode=p.pool,
                    cube=p.cube, kcube=p.kcube)
    assert_close(host(o), fwd["o"], dtype, "o")
    ref = O.backward(x["q"], x["k"], x["v"], *xg, x["d_o"], fwd)
    names = ("dq", "dk", "dv", "dg_c", "dg_f") if gates else ("dq", "dk", "dv")
    for nm in names:
        assert_close(host(g[nm]), ref[nm], dtype, nm, rel=rel)
    if not gates:
        assert g["dg_c"] is None and g["dg_f"] is None


def _small_train_inputs(d=64, seed=5, heads=2, T=8, H=16, W=16, cube=(4, 4, 4), kcube=None, dtype="bf16",
                        scale=1.0):
    """Ragged random lists (lengths U{0..Nk}), one empty row and one full row."""
    x = WL.make_inputs_custom(1, heads, d, T, H, W, dtype=dtype, seed=seed, scale=scale)
    nc = T * H * W // (cube[0] * cube[1] * cube[2])
    kc = cube if kcube is None else kcube
    nk = T * H * W // (kc[0] * kc[1] * kc[2])
    idx, lens = WL.random_lists(nk, heads * nc, 0, nk, seed=seed)
    lens[0], lens[1] = 0, nk
    idx[1, :nk] = np.arange(nk)
    x["idx"] = idx.reshape(1, heads, nc, nk)
    x["len"] = lens.reshape(1, heads, nc)
    p = V.Problem(1, heads, T, H, W, d, dtype=dtype, topk=0, list_stride=nk, cube=cube, kcube=kcube)
    return x, p


def test_backward_small_ragged_full_compare():
    x, p = _small_train_inputs()
    backward_compare(x, p, "bf16")


def test_backward_small_ungated():
    x, p = _small_train_inputs(seed=6)
    backward_compare(x, p, "bf16", gates=False)


@pytest.mark.parametrize("d", [64, 128])
def test_single_cube_latent(d):
    """The degenerate latent of one cube (4x4x4, Nc = 1): the coarse softmax
    is 1, top-1 keeps the only cube, and the fine stage is full attention
    over 64 tokens. Forward (top-K mode) and backward against the oracle."""
    x = WL.make_inputs_custom(1, 2, d, 4, 4, 4, dtype="bf16", seed=43)
    p = V.Problem(1, 2, 4, 4, 4, d, topk=1)
    dd = inputs_to_dev(x, "bf16")
    o, idx, lens, saved = V.forward(p, dd["q"], dd["k"], dd["v"], dd["g_c"], dd["g_f"], training=True)
    g = V.backward(p, dd["q"], dd["k"], dd["v"], dd["g_c"], dd["g_f"], idx, lens, saved, dd["d_o"])
    torch.cuda.synchronize()
    assert (host(idx) == 0).all() and (host(lens) == 1).all()
    fwd = O.forward(x["q"], x["k"], x["v"], x["g_c"], x["g_f"], topk=1)
    assert_close(host(o), fwd["o"], "bf16", "o")
    ref = O.backward(x["q"], x["k"], x["v"], x["g_c"], x["g_f"], x["d_o"], fwd)
    for nm in ("dq", "dk", "dv", "dg_c", "dg_f"):
        assert_close(host(g[nm]), ref[nm], "bf16", nm)


@pytest.mark.parametrize("d,pool,cube,kcube,gates", [
    (64, "mean", (4, 4, 4), None, True), (128, "max", (4, 4, 4), None, True), (64, "mean", (4, 4, 4), None, False),
    (128, "mean", (2, 4, 4), (4, 4, 8), True), (64, "max", (4, 4, 8), (1, 4, 4), True),
    (64, "mean", (4, 4, 4), (1, 4, 4), True), (64, "mean", (4, 8, 8), None, True),
    (128, "max", (1, 16, 16), (4, 8, 8), True)])
def test_backward_fp32(d, pool, cube, kcube, gates):
    """fp32 problems: the whole backward (fp32 kernels) on ragged lists with an
    empty and a full row, against the oracle to 1e-4 absolute."""
    x, p = _small_train_inputs(d=d, seed=61, T=8, H=16, W=16, cube=cube, kcube=kcube, dtype="f32", scale=0.25)
    backward_compare(x, dataclasses.replace(p, pool=pool), "f32", gates=gates)


def test_backward_head_dim_128():
    x, p = _small_train_inputs(d=128, seed=8, heads=1, T=8, H=8, W=16)
    backward_compare(x, p, "bf16")


def test_backward_training_config_sampled():
    """The training workload at full size on the GPU (B=2, 12 heads, lists of
    length U{8..64}); the oracle checks two (b, h) slices completely."""
    w = WL.get("C5")
    x = WL.make_inputs("C5")
    p = problem_of(w)
    d = inputs_to_dev(x, "bf16")
    o, idx, lens, saved = V.forward(p, d["q"], d["k"], d["v"], d["g_c"], d["g_f"], idx=d["idx"], lens=d["len"],
                                    training=True)
    g = V.backward(p, d["q"], d["k"], d["v"], d["g_c"], d["g_f"], idx, lens, saved, d["d_o"])
    torch.cuda.synchronize()
    for b, h in ((0, 0), (1, 7)):
        sl = {k: x[k][b:b + 1, h:h + 1] for k in ("q", "k", "v", "g_c", "g_f", "d_o", "idx", "len")}
        fwd = O.forward(sl["q"], sl["k"], sl["v"], sl["g_c"], sl["g_f"], topk=0, idx=sl["idx"], lens=sl["len"])
        assert_close(host(o[b:b + 1, h:h + 1]), fwd["o"], "bf16", "o")
        ref = O.backward(sl["q"], sl["k"], sl["v"], sl["g_c"], sl["g_f"], sl["d_o"], fwd)
        for nm in ("dq", "dk", "dv", "dg_c", "dg_f"):
            assert_close(host(g[nm][b:b + 1, h:h + 1]), ref[nm], "bf16", f"{nm}[{b},{h}]")


@pytest.mark.timeout(900)
def test_backward_720p_heads():
    """The 720p workload's training step at full size (all 40 heads, top-32
    lists from the forward, dO ~ N(0, 1) from a seeded generator): the
    gradients of three heads are checked completely against the oracle on the
    GPU's lists."""
    w = WL.get("C4")
    print("[720p bwd] generating inputs", flush=True)
    x = _inputs_720p()
    p = problem_of(w)
    d = inputs_to_dev(x, "bf16")
    gen = torch.Generator(device=DEV)
    gen.manual_seed(8)
    d_o = torch.randn(d["q"].shape, generator=gen, device=DEV, dtype=torch.float32).to(torch.bfloat16)
    print("[720p bwd] running the HIP forward + backward", flush=True)
    o, idx, lens, saved = V.forward(p, d["q"], d["k"], d["v"], d["g_c"], d["g_f"], training=True)
    g = V.backward(p, d["q"], d["k"], d["v"], d["g_c"], d["g_f"], idx, lens, saved, d_o)
    torch.cuda.synchronize()
    for h in (0, 21, 39):
        sl = {k: x[k][:, h:h + 1] for k in ("q", "k", "v", "g_c", "g_f")}
        gi, gl = host(idx)[:, h:h + 1], host(lens)[:, h:h + 1]
        print(f"[720p bwd] oracle forward + backward of head {h}", flush=True)
        fwd = O.forward(sl["q"], sl["k"], sl["v"], sl["g_c"], sl["g_f"], topk=0, idx=gi, lens=gl)
        assert_close(host(o[:, h:h + 1]), fwd["o"], "bf16", "o")
        ref = O.backward(sl["q"], sl["k"], sl["v"], sl["g_c"], sl["g_f"], host(d_o[:, h:h + 1]), fwd)
        for nm in ("dq", "dk", "dv", "dg_c", "dg_f"):
            assert_close(host(g[nm][:, h:h + 1]), ref[nm], "bf16", f"{nm}[head {h}]")


@pytest.mark.timeout(900)
def test_backward_long_clip():
    """A training step on a clip of 4096 cubes (32x64x128 latent, 262144
    tokens, one head, d = 64, top-32 lists from the forward). Past 2048
    cubes the coarse rows are streamed, the longest-first key order sorts
    4096 keys and the transposed lists' bitmask has 128 words per key block.
    Every output and gradient is checked against the oracle on the GPU's
    lists."""
    T, H, W, d, k = 32, 64, 128, 64, 32
    x = WL.make_inputs_custom(1, 1, d, T, H, W, dtype="bf16", seed=43)
    p = V.Problem(1, 1, T, H, W, d, topk=k)
    assert p.Nc == 4096
    print(f"[long clip bwd] {T}x{H}x{W}: {p.Nc} cubes", flush=True)
    dd = inputs_to_dev(x, "bf16")
    o, idx, lens, saved = V.forward(p, dd["q"], dd["k"], dd["v"], dd["g_c"], dd["g_f"], training=True)
    g = V.backward(p, dd["q"], dd["k"], dd["v"], dd["g_c"], dd["g_f"], idx, lens, saved, dd["d_o"])
    torch.cuda.synchronize()
    gi, gl = host(idx), host(lens)
    assert (gl == k).all()
    print("[long clip bwd] oracle forward + backward", flush=True)
    fwd = O.forward(x["q"], x["k"], x["v"], x["g_c"], x["g_f"], topk=0, idx=gi, lens=gl)
    assert_close(host(o), fwd["o"], "bf16", "o")
    ref = O.backward(x["q"], x["k"], x["v"], x["g_c"], x["g_f"], x["d_o"], fwd)
    for nm in ("dq", "dk", "dv", "dg_c", "dg_f"):
        assert_close(host(g[nm]), ref[nm], "bf16", nm)


def test_backward_stages():
    x, p = _small_train_inputs(seed=12)
    d = inputs_to_dev(x, "bf16")
    fwd = O.forward(x["q"], x["k"], x["v"], x["g_c"], x["g_f"], topk=0, idx=x["idx"], lens=x["len"])
    ref = O.backward(x["q"], x["k"], x["v"], x["g_c"], x["g_f"], x["d_o"], fwd)
    # index transpose: bit-exact against the oracle's transposed lists
    off, k2q = V.index_transpose(p, d["idx"], d["len"])
    torch.cuda.synchronize()
    off, k2q = host(off), host(k2q)
    for h in range(2):
        rk, rl = O.transpose_lists(x["idx"][0, h], x["len"][0, h], p.Nc)
        assert np.array_equal(np.diff(off[0, h]), rl)
        for j in range(p.Nc):
            assert np.array_equal(k2q[0, h, off[0, h, j]:off[0, h, j + 1]], rk[j, :rl[j]])
    # combine backward on the oracle's O_c / O_f (rounded to the GPU dtypes)
    ws = V.workspace(p, d["q"], training=True)
    oc32 = dev(fwd["o_c"].astype(np.float32), torch.float32)
    of16 = dev(fwd["o_f"].astype(np.float32), torch.bfloat16)
    cb = V.combine_backward(p, d["d_o"], oc32, of16, d["g_c"], d["g_f"])
    torch.cuda.synchronize()
    assert_close(host(cb["dg_c"]), ref["dg_c"], "bf16", "dg_c", rel=2 ** -7)
    assert_close(host(cb["d_o_f"]), ref["d_o_f"], "bf16", "d_o_f", rel=2 ** -7)
    assert rel_err(host(cb["d_o_c"]), ref["d_o_c"]) <= 1e-2
    assert rel_err(host(cb["delta"]), ref["delta"]) <= 1e-2
    # coarse backward on exact pooled inputs
    f32 = lambda a: dev(a.astype(np.float32), torch.float32)
    dqc, dkc, dvc = V.coarse_backward(p, f32(fwd["q_c"]), f32(fwd["k_c"]), f32(fwd["v_c"]), f32(fwd["o_c"]),
                                      f32(fwd["lse_c"]), f32(ref["d_o_c"]), ws)
    torch.cuda.synchronize()
    for got, nm in ((dqc, "dq_c"), (dkc, "dk_c"), (dvc, "dv_c")):
        assert rel_err(host(got), ref[nm]) <= 1e-4, nm


@pytest.mark.parametrize("dtype,pool,cube,kcube", [("bf16", "mean", (4, 4, 4), None),
                                                    ("bf16", "max", (4, 4, 4), (1, 4, 4)),
                                                    ("f32", "mean", (2, 4, 4), (4, 4, 8)),
                                                    ("f32", "max", (4, 4, 4), None),
                                                    ("bf16", "max", (4, 8, 8), (4, 4, 4)),
                                                    ("bf16", "mean", (4, 4, 4), (1, 16, 16)),
                                                    ("f32", "max", (1, 16, 16), None)])
def test_fine_backward_stage(dtype, pool, cube, kcube):
    """The fine-backward entry point on its own: the oracle's LSE_f, dO_f,
    delta and pooled gradients in (rounded to the GPU dtypes), the GPU's
    transposed lists; dQ, dK, dV (fine part plus pool backward) against the
    oracle's."""
    x, p = _small_train_inputs(seed=71, cube=cube, kcube=kcube, dtype=dtype, scale=1.0 if dtype == "bf16" else 0.25)
    p = dataclasses.replace(p, pool=pool)
    d = inputs_to_dev(x, dtype)
    fwd = O.forward(x["q"], x["k"], x["v"], x["g_c"], x["g_f"], topk=0, idx=x["idx"], lens=x["len"], pool_mode=pool,
                    cube=cube, kcube=kcube)
    ref = O.backward(x["q"], x["k"], x["v"], x["g_c"], x["g_f"], x["d_o"], fwd)
    f32 = lambda a: dev(np.asarray(a, dtype=np.float32), torch.float32)
    ws = V.workspace(p, d["q"], training=True)
    off, k2q = V.index_transpose(p, d["idx"], d["len"], ws=ws)
    dq, dk, dv = V.fine_backward(p, d["q"], d["k"], d["v"], d["idx"], d["len"], off, k2q, f32(fwd["lse_f"]),
                                 dev(np.asarray(ref["d_o_f"], dtype=np.float32), p.torch_dtype), f32(ref["delta"]),
                                 f32(ref["dq_c"]), f32(ref["dk_c"]), f32(ref["dv_c"]), ws)
    torch.cuda.synchronize()
    for got, nm in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        assert_close(host(got), ref[nm], dtype, nm)


@pytest.mark.parametrize("dtype,topk", [("bf16", 0), ("bf16", 5), ("f32", 0)])
def test_autograd_attention(dtype, topk):
    """The differentiable wrapper: torch autograd through the library's
    forward and backward, gradients against the oracle on the lists used."""
    x, p = _small_train_inputs(seed=81, dtype=dtype, scale=1.0 if dtype == "bf16" else 0.25)
    d = inputs_to_dev(x, dtype)
    leaves = [d[n].clone().requires_grad_(True) for n in ("q", "k", "v", "g_c", "g_f")]
    if topk:
        p = dataclasses.replace(p, topk=topk, list_stride=topk)
        o, idx, lens = V.attention(p, *leaves)
    else:
        o, idx, lens = V.attention(p, *leaves, idx=d["idx"], lens=d["len"])
    assert not idx.requires_grad and not lens.requires_grad
    o.backward(d["d_o"])
    torch.cuda.synchronize()
    gi, gl = host(idx), host(lens)
    fwd = O.forward(x["q"], x["k"], x["v"], x["g_c"], x["g_f"], topk=0, idx=gi, lens=gl)
    assert_close(host(o), fwd["o"], dtype, "o")
    ref = O.backward(x["q"], x["k"], x["v"], x["g_c"], x["g_f"], x["d_o"], fwd)
    for t, nm in zip(leaves, ("dq", "dk", "dv", "dg_c", "dg_f")):
        assert_close(host(t.grad), ref[nm], dtype, nm)


# ------------------------------------------------------- max-pool variant
@pytest.mark.parametrize("name", ["C1", "C2"])
def test_max_pool_forward_topk(name):
    """The max-pool variant: pooled maxima bit-exact (a maximum of exact
    inputs is exact in fp32), top-K protocol with the variant's error bound,
    end-to-end output on the GPU's lists."""
    w = WL.get(name)
    hs = [0, 1]
    x = WL.make_inputs(name, heads=hs)
    p = problem_of(w, heads=2, pool="max")
    d = inputs_to_dev(x, w.dtype)
    qc, kc, vc = V.pool(p, d["q"], d["k"], d["v"])
    o, idx, lens, _ = V.forward(p, d["q"], d["k"], d["v"], d["g_c"], d["g_f"])
    torch.cuda.synchronize()
    for got, src in ((qc, "q"), (kc, "k"), (vc, "v")):
        assert np.array_equal(host(got), O.pool(O.tile(x[src].astype(np.float64)), "max")), src
    ref_sel = O.forward(x["q"], x["k"], x["v"], topk=w.topk, pool_mode="max")
    gi = host(idx)
    near = check_topk(gi, ref_sel, w.topk)
    assert near <= NEAR_FRAC * gi.shape[0] * gi.shape[1] * gi.shape[2] + 2
    ref = O.forward(x["q"], x["k"], x["v"], x["g_c"], x["g_f"], topk=0, idx=gi, lens=host(lens), pool_mode="max")
    assert_close(host(o), ref["o"], w.dtype, "o")
    mean = O.forward(x["q"], x["k"], x["v"], x["g_c"], x["g_f"], topk=0, idx=gi, lens=host(lens))
    assert rel_err(mean["o"], ref["o"]) > 1e-2   # the variant is a different operator


@pytest.mark.parametrize("d", [64, 128])
def test_max_pool_backward(d):
    x, p = _small_train_inputs(d=d, seed=9, heads=2 if d == 64 else 1, T=8, H=8 if d == 128 else 16, W=16)
    backward_compare(x, dataclasses.replace(p, pool="max"), "bf16")


# ------------------------------------------------------------ tiled layout
def test_tile_untile_match_oracle():
    w = WL.get("C2")
    x = WL.make_inputs("C2", heads=[0, 1], gates=False)
    p = problem_of(w, heads=2)
    q = dev(x["q"], torch.bfloat16)
    qt = V.tile(p, q)
    back = V.untile(p, qt)
    torch.cuda.synchronize()
    assert np.array_equal(host(qt), O.tile(host(q)))
    assert torch.equal(back, q)


def _tiled(p, d, keys):
    return {k: (V.tile(p, d[k]) if d.get(k) is not None else None) for k in keys}


@pytest.mark.parametrize("name", ["C1", "C2"])
def test_tiled_layout_forward_equals_raster(name):
    """The cube-major layout runs the same arithmetic in the same order, so
    its outputs equal the raster run's bit for bit once untiled."""
    w = WL.get(name)
    x = WL.make_inputs(name, heads=[0, 1])
    p = problem_of(w, heads=2)
    pt = dataclasses.replace(p, layout="tiled")
    d = inputs_to_dev(x, w.dtype)
    o, idx, lens, saved = V.forward(p, d["q"], d["k"], d["v"], d["g_c"], d["g_f"], training=True)
    t = _tiled(p, d, ("q", "k", "v", "g_c", "g_f"))
    ot, idxt, lenst, savedt = V.forward(pt, t["q"], t["k"], t["v"], t["g_c"], t["g_f"], training=True)
    torch.cuda.synchronize()
    assert tuple(ot.shape) == (1, 2, w.Nc, 64, w.head_dim)
    assert torch.equal(idx, idxt) and torch.equal(lens, lenst)
    assert torch.equal(V.untile(p, ot), o)
    sv, svt = V.saved_views(p, saved), V.saved_views(pt, savedt)
    assert torch.equal(V.untile(p, svt["o_f"]), sv["o_f"])
    # per-token arrays follow the token order too
    lse_r = sv["lse_f"].reshape(1, 2, w.T // 4, 4, w.H // 4, 4, w.W // 4, 4)
    lse_t = lse_r.permute(0, 1, 2, 4, 6, 3, 5, 7).reshape(1, 2, w.Nc, 64)
    assert torch.equal(svt["lse_f"], lse_t)


def test_tiled_layout_backward_equals_raster():
    x, p = _small_train_inputs(seed=13)
    pt = dataclasses.replace(p, layout="tiled")
    d = inputs_to_dev(x, "bf16")
    o, idx, lens, saved = V.forward(p, d["q"], d["k"], d["v"], d["g_c"], d["g_f"], idx=d["idx"], lens=d["len"],
                                    training=True)
    g = V.backward(p, d["q"], d["k"], d["v"], d["g_c"], d["g_f"], idx, lens, saved, d["d_o"])
    t = _tiled(p, d, ("q", "k", "v", "g_c", "g_f", "d_o"))
    ot, _, _, savedt = V.forward(pt, t["q"], t["k"], t["v"], t["g_c"], t["g_f"], idx=d["idx"], lens=d["len"],
                                 training=True)
    gt = V.backward(pt, t["q"], t["k"], t["v"], t["g_c"], t["g_f"], idx, lens, savedt, t["d_o"])
    torch.cuda.synchronize()
    assert torch.equal(V.untile(p, ot), o)
    for nm in ("dq", "dk", "dv", "dg_c", "dg_f"):
        assert torch.equal(V.untile(p, gt[nm]), g[nm]), nm


# ------------------------------------------- latents not divisible by the cube
@pytest.mark.parametrize("layout", ["raster", "tiled"])
@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("f32", 128)])
def test_crop_pad_match_oracle(layout, dtype, d):
    T, H, W = 9, 13, 30
    Tc, Hc, Wc = V.compatible_latent(T, H, W)
    assert (Tc, Hc, Wc) == O.compatible_latent(T, H, W) == (12, 16, 32)
    p = V.Problem(1, 2, Tc, Hc, Wc, d, dtype=dtype, topk=2, layout=layout)
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    rng = np.random.default_rng(3)
    xs = dev(rng.standard_normal((1, 2, T, H, W, d)).astype(np.float32), td)
    ref = O.pad(host(xs), Tc, Hc, Wc)
    got = V.pad(p, xs)
    big = rng.standard_normal((1, 2, Tc, Hc, Wc, d)).astype(np.float32)
    bigd = dev(O.tile(big) if layout == "tiled" else big, td)
    cropped = V.crop(p, bigd, T, H, W)
    torch.cuda.synchronize()
    assert np.array_equal(host(got), O.tile(ref) if layout == "tiled" else ref)
    assert np.array_equal(host(cropped), O.crop(host(bigd) if layout == "raster" else
                                                O.untile(host(bigd), Tc, Hc, Wc), T, H, W))


def test_forward_on_compatible_latent_then_crop():
    """The remedy for latents whose sides are not multiples of 4: run the
    operator on the compatible (larger) latent and crop. In either token
    order the cropped output matches the oracle's pad -> forward -> crop."""
    T, H, W, heads, d = 7, 10, 13, 2, 64
    Tc, Hc, Wc = V.compatible_latent(T, H, W)
    x = WL.make_inputs_custom(1, heads, d, T, H, W, dtype="bf16", seed=21)
    nc = Tc * Hc * Wc // 64
    idx, lens = WL.random_lists(nc, heads * nc, 1, nc, seed=21, stride=nc)
    idx, lens = idx.reshape(1, heads, nc, nc), lens.reshape(1, heads, nc)
    ref = O.forward(*(O.pad(x[k], Tc, Hc, Wc) for k in ("q", "k", "v", "g_c", "g_f")), topk=0, idx=idx, lens=lens)
    ref_o = O.crop(ref["o"], T, H, W)
    d_in = inputs_to_dev(x, "bf16")
    idx_d, lens_d = dev(idx, torch.int32), dev(lens, torch.int32)
    outs = []
    for layout in ("raster", "tiled"):
        p = V.Problem(1, heads, Tc, Hc, Wc, d, topk=0, list_stride=nc, layout=layout)
        padded = [V.pad(p, d_in[k]) for k in ("q", "k", "v", "g_c", "g_f")]
        o, _, _, _ = V.forward(p, *padded, idx=idx_d, lens=lens_d)
        outs.append(V.crop(p, o, T, H, W))
    torch.cuda.synchronize()
    assert tuple(outs[0].shape) == (1, heads, T, H, W, d)
    assert torch.equal(outs[0], outs[1])
    assert_close(host(outs[0]), ref_o, "bf16", "o (cropped)")


# ------------------------------------------- other cube shapes (tile sizes)
CUBES = [(2, 4, 4), (4, 4, 8), (1, 8, 8),   # 32, 128 and another 64-token tile
         (4, 8, 8), (1, 16, 16)]            # 256-token tiles (split along t and along y)


@pytest.mark.parametrize("cube", CUBES)
@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("bf16", 128), ("f32", 64)])
def test_general_cube_forward_topk(cube, dtype, d):
    """Top-K selection bit-exact (near-tie protocol) and the output against the
    oracle on the GPU's lists, for tiles of 32, 64, 128 and 256 tokens."""
    T, H, W, heads = 8, 16, 32, 2
    bt = cube[0] * cube[1] * cube[2]
    nc = T * H * W // bt
    k = max(nc // 8, 1)
    x = WL.make_inputs_custom(1, heads, d, T, H, W, dtype=dtype, seed=17, scale=1.0 if dtype == "bf16" else 0.125)
    p = V.Problem(1, heads, T, H, W, d, dtype=dtype, topk=k, cube=cube)
    dd = inputs_to_dev(x, dtype)
    o, idx, lens, saved = V.forward(p, dd["q"], dd["k"], dd["v"], dd["g_c"], dd["g_f"], training=True)
    torch.cuda.synchronize()
    gi, gl = host(idx), host(lens)
    assert (gl == k).all()
    sel = O.forward(x["q"], x["k"], x["v"], topk=k, cube=cube)
    near = check_topk(gi, sel, k)
    assert near <= NEAR_FRAC * heads * nc
    ref = O.forward(x["q"], x["k"], x["v"], x["g_c"], x["g_f"], topk=0, idx=gi, lens=gl, cube=cube)
    assert_close(host(o), ref["o"], dtype, f"{cube} o")
    sv = V.saved_views(p, saved)
    assert_close(host(sv["o_f"]), ref["o_f"], dtype, f"{cube} o_f")
    lse = host(sv["lse_f"])
    assert np.abs(lse - ref["lse_f"]).max() <= (LSE_ABS if dtype == "bf16" else 1e-4)
    np.testing.assert_allclose(host(sv["q_c"]), ref["q_c"], rtol=1e-4, atol=1e-5)


@pytest.mark.parametrize("cube", CUBES)
@pytest.mark.parametrize("d", [64, 128])
def test_general_cube_backward(cube, d):
    x, p = _small_train_inputs(d=d, seed=19, T=8, H=16, W=16, cube=cube)
    backward_compare(x, p, "bf16")


@pytest.mark.parametrize("cube", [(4, 4, 8), (2, 4, 4), (4, 8, 8)])
def test_general_cube_tiled_equals_raster_and_max_pool(cube):
    x, p = _small_train_inputs(d=64, seed=23, T=8, H=16, W=16, cube=cube)
    pm = dataclasses.replace(p, pool="max")
    backward_compare(x, pm, "bf16")
    pt = dataclasses.replace(p, layout="tiled")
    d = inputs_to_dev(x, "bf16")
    o, idx, lens, saved = V.forward(p, d["q"], d["k"], d["v"], d["g_c"], d["g_f"], idx=d["idx"], lens=d["len"],
                                    training=True)
    g = V.backward(p, d["q"], d["k"], d["v"], d["g_c"], d["g_f"], idx, lens, saved, d["d_o"])
    t = _tiled(p, d, ("q", "k", "v", "g_c", "g_f", "d_o"))
    assert tuple(t["q"].shape) == (1, 2, p.Nc, p.Bt, 64)
    assert np.array_equal(host(t["q"]), O.tile(host(d["q"]), cube))
    ot, _, _, savedt = V.forward(pt, t["q"], t["k"], t["v"], t["g_c"], t["g_f"], idx=d["idx"], lens=d["len"],
                                 training=True)
    gt = V.backward(pt, t["q"], t["k"], t["v"], t["g_c"], t["g_f"], idx, lens, savedt, t["d_o"])
    torch.cuda.synchronize()
    assert torch.equal(V.untile(p, ot), o)
    for nm in ("dq", "dk", "dv", "dg_c", "dg_f"):
        if p.Bt == 256 and nm in ("dk", "dv"):
            # The fine kernels take a 256-token cube as two halves, numbered
            # row-major in the raster layout and 2c + h in the tiled one, so
            # dK / dV sum over the query halves in another order.
            assert_close(host(V.untile(p, gt[nm])), host(g[nm]), "bf16", nm)
        else:
            assert torch.equal(V.untile(p, gt[nm]), g[nm]), nm
    # crop / pad with this cube, from the tiled layout
    Tc, Hc, Wc = V.compatible_latent(7, 13, 9, cube)
    assert (Tc, Hc, Wc) == O.compatible_latent(7, 13, 9, cube)
    pc = V.Problem(1, 2, Tc, Hc, Wc, 64, topk=1, cube=cube, layout="tiled")
    xs = d["q"][:, :, :7, :13, :9].contiguous()
    xp = V.pad(pc, xs)
    back = V.crop(pc, xp, 7, 13, 9)
    torch.cuda.synchronize()
    assert np.array_equal(host(xp), O.tile(O.pad(host(xs), Tc, Hc, Wc), cube))
    assert torch.equal(back, xs)


# ------------------------------- key blocks of their own shape (Bq x Bk tiles)
# (query cube, key block): 64 x 32, 64 x 128, 32 x 128, 128 x 32 tokens, and
# 16-token key blocks (taken two per 32-key chunk): 64 x 16 (the summary
# page's tile), 32 x 16, 128 x 16.
TILE_PAIRS = [((4, 4, 4), (2, 4, 4)), ((4, 4, 4), (4, 4, 8)), ((2, 4, 4), (4, 4, 8)), ((4, 4, 8), (2, 4, 4)),
              ((4, 4, 4), (1, 4, 4)), ((2, 4, 4), (2, 2, 4)), ((4, 4, 8), (1, 4, 4)),
              # 256-token query cubes or key blocks (the fine kernels run on 128-token halves)
              ((4, 8, 8), (4, 4, 4)), ((4, 4, 4), (4, 8, 8)), ((4, 8, 8), (1, 16, 16)), ((4, 8, 8), (1, 4, 4))]


@pytest.mark.parametrize("cube,kcube", TILE_PAIRS)
@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("bf16", 128), ("f32", 64)])
def test_key_block_forward_topk(cube, kcube, dtype, d):
    """Nq x Nk coarse scores, top-K over key blocks bit-exact (near-tie
    protocol), pooled tensors per cube / per key block, and the output on the
    GPU's lists against the oracle."""
    T, H, W, heads = 8, 16, 32, 2
    nq = T * H * W // (cube[0] * cube[1] * cube[2])
    nk = T * H * W // (kcube[0] * kcube[1] * kcube[2])
    k = max(nk // 8, 1)
    x = WL.make_inputs_custom(1, heads, d, T, H, W, dtype=dtype, seed=29, scale=1.0 if dtype == "bf16" else 0.125)
    p = V.Problem(1, heads, T, H, W, d, dtype=dtype, topk=k, cube=cube, kcube=kcube)
    dd = inputs_to_dev(x, dtype)
    o, idx, lens, saved = V.forward(p, dd["q"], dd["k"], dd["v"], dd["g_c"], dd["g_f"], training=True)
    torch.cuda.synchronize()
    gi, gl = host(idx), host(lens)
    assert gi.shape == (1, heads, nq, k) and (gl == k).all()
    sel = O.forward(x["q"], x["k"], x["v"], topk=k, cube=cube, kcube=kcube)
    assert sel["s_c"].shape == (1, heads, nq, nk)
    near = check_topk(gi, sel, k)
    # Sanity bound on the near-tie share (every row is still checked): with
    # 16-token key blocks a row ranks 256 candidates for 32 places, and at 64
    # rows the 5% share is 3 rows, so up to 8 are allowed.
    assert near <= max(NEAR_FRAC * heads * nq, 8)
    ref = O.forward(x["q"], x["k"], x["v"], x["g_c"], x["g_f"], topk=0, idx=gi, lens=gl, cube=cube, kcube=kcube)
    assert_close(host(o), ref["o"], dtype, f"{cube}x{kcube} o")
    sv = V.saved_views(p, saved)
    assert_close(host(sv["o_f"]), ref["o_f"], dtype, f"{cube}x{kcube} o_f")
    lse = host(sv["lse_f"])
    assert np.abs(lse - ref["lse_f"]).max() <= (LSE_ABS if dtype == "bf16" else 1e-4)
    for nm in ("q_c", "k_c", "v_c"):
        np.testing.assert_allclose(host(sv[nm]), ref[nm], rtol=1e-4, atol=1e-5, err_msg=nm)
    np.testing.assert_allclose(host(sv["lse_c"]), ref["lse_c"], rtol=1e-4, atol=1e-4)


@pytest.mark.parametrize("cube,kcube", TILE_PAIRS)
@pytest.mark.parametrize("d", [64, 128])
def test_key_block_backward(cube, kcube, d):
    """Whole backward with ragged lists over key blocks (an empty list and a
    full one included): dQ walks key blocks, dK / dV walk query cubes."""
    x, p = _small_train_inputs(d=d, seed=31, T=8, H=16, W=16, cube=cube, kcube=kcube)
    backward_compare(x, p, "bf16")


@pytest.mark.parametrize("cube,kcube", [((4, 4, 4), (2, 4, 4)), ((2, 4, 4), (4, 4, 8)), ((4, 4, 4), (1, 4, 4))])
def test_key_block_max_pool_and_stages(cube, kcube):
    """Max pooling per key block, and the stage entry points chained by hand
    (pool, coarse, fine, combine, index transpose, backward stages) against
    the oracle's pieces."""
    x, p = _small_train_inputs(d=64, seed=37, T=8, H=16, W=16, cube=cube, kcube=kcube)
    backward_compare(x, dataclasses.replace(p, pool="max"), "bf16")
    d = inputs_to_dev(x, "bf16")
    qc, kc, vc = V.pool(p, d["q"], d["k"], d["v"])
    oc, lse_c, _, _ = V.coarse(p, qc, kc, vc)
    torch.cuda.synchronize()
    ref = O.forward(x["q"], x["k"], x["v"], x["g_c"], x["g_f"], topk=0, idx=x["idx"], lens=x["len"], cube=cube,
                    kcube=kcube)
    assert tuple(kc.shape) == (1, 2, p.Nk, 64) and tuple(qc.shape) == (1, 2, p.Nc, 64)
    for nm, t in (("q_c", qc), ("k_c", kc), ("v_c", vc), ("o_c", oc), ("lse_c", lse_c)):
        np.testing.assert_allclose(host(t), ref[nm], rtol=1e-4, atol=1e-5, err_msg=nm)
    off, k2q = V.index_transpose(p, d["idx"], d["len"])
    torch.cuda.synchronize()
    off, k2q = host(off), host(k2q)
    assert off.shape == (1, 2, p.Nk + 1)
    for h in range(2):
        rows = [[] for _ in range(p.Nk)]
        for i in range(p.Nc):
            for j in x["idx"][0, h, i, :x["len"][0, h, i]]:
                rows[j].append(i)
        got = [list(k2q[0, h, off[0, h, j]:off[0, h, j + 1]]) for j in range(p.Nk)]
        assert got == rows
    V.validate_lists(p, d["idx"], d["len"])


# ------------------------------------------------ seeded random configurations
def _random_case(seed):
    """A seeded random problem: cube and key-block shapes, latent, heads,
    head_dim, top-K or explicit ragged lists, list stride, pooling."""
    rng = np.random.default_rng([seed, 4242])
    cubes = [(4, 4, 4), (2, 4, 4), (4, 4, 8), (1, 8, 8), (2, 2, 8)]
    kblocks = [None, (2, 4, 4), (4, 4, 8), (1, 4, 4), (2, 2, 4), (4, 4, 4)]
    cube = cubes[rng.integers(len(cubes))]
    kcube = kblocks[rng.integers(len(kblocks))]
    kc = cube if kcube is None else kcube
    lcm = [max(a, b) for a, b in zip(cube, kc)]   # sides are powers of two
    T, H, W = (int(l * rng.integers(1, 4)) for l in lcm)
    while T * H * W < 2 * max(np.prod(cube), np.prod(kc)):
        W *= 2
    heads = int(rng.integers(1, 3))
    d = int(rng.choice([64, 128]))
    nq = T * H * W // int(np.prod(cube))
    nk = T * H * W // int(np.prod(kc))
    explicit = bool(rng.integers(2))
    pool = "max" if rng.integers(4) == 0 else "mean"
    if explicit:
        stride = int(rng.integers(1, nk + 1))
        topk = 0
    else:
        topk = int(rng.integers(1, nk + 1))
        stride = int(rng.integers(topk, nk + 1))
    return dict(cube=cube, kcube=kcube, T=T, H=H, W=W, heads=heads, d=d, nq=nq, nk=nk, explicit=explicit,
                topk=topk, stride=stride, pool=pool)


def _run_random(seed, dtype):
    c = _random_case(seed)
    print(f"[random {dtype} {seed}] {c}", flush=True)
    x = WL.make_inputs_custom(1, c["heads"], c["d"], c["T"], c["H"], c["W"], dtype=dtype, seed=100 + seed,
                              scale=1.0 if dtype == "bf16" else 0.25)
    p = V.Problem(1, c["heads"], c["T"], c["H"], c["W"], c["d"], dtype=dtype, topk=c["topk"],
                  list_stride=c["stride"], cube=c["cube"], kcube=c["kcube"], pool=c["pool"])
    dd = inputs_to_dev(x, dtype)
    if c["explicit"]:
        idx, lens = WL.random_lists(c["nk"], c["heads"] * c["nq"], 0, c["stride"], seed=seed, stride=c["stride"])
        x["idx"] = idx.reshape(1, c["heads"], c["nq"], c["stride"])
        x["len"] = lens.reshape(1, c["heads"], c["nq"])
        o, gi_t, gl_t, saved = V.forward(p, dd["q"], dd["k"], dd["v"], dd["g_c"], dd["g_f"],
                                         idx=dev(x["idx"], torch.int32), lens=dev(x["len"], torch.int32),
                                         training=True)
    else:
        o, gi_t, gl_t, saved = V.forward(p, dd["q"], dd["k"], dd["v"], dd["g_c"], dd["g_f"], training=True)
    g = V.backward(p, dd["q"], dd["k"], dd["v"], dd["g_c"], dd["g_f"], gi_t, gl_t, saved, dd["d_o"])
    torch.cuda.synchronize()
    gi, gl = host(gi_t), host(gl_t)
    if not c["explicit"]:
        assert (gl == c["topk"]).all()
        if c["stride"] > c["topk"]:
            assert np.all(gi[..., c["topk"]:] == -1)
        sel = O.forward(x["q"], x["k"], x["v"], topk=c["topk"], pool_mode=c["pool"], cube=c["cube"],
                        kcube=c["kcube"])
        check_topk(gi[..., :c["topk"]], sel, c["topk"])
    fwd = O.forward(x["q"], x["k"], x["v"], x["g_c"], x["g_f"], topk=0, idx=gi, lens=gl, pool_mode=c["pool"],
                    cube=c["cube"], kcube=c["kcube"])
    assert_close(host(o), fwd["o"], dtype, "o")
    ref = O.backward(x["q"], x["k"], x["v"], x["g_c"], x["g_f"], x["d_o"], fwd)
    for nm in ("dq", "dk", "dv", "dg_c", "dg_f"):
        assert_close(host(g[nm]), ref[nm], dtype, nm)


@pytest.mark.parametrize("seed", range(48))
def test_random_configurations(seed):
    """Forward and backward of seeded random problems against the oracle
    (bf16; top-K rows checked by the near-tie protocol, outputs on the GPU's
    lists)."""
    _run_random(seed, "bf16")


@pytest.mark.parametrize("seed", range(1000, 1020))
def test_random_configurations_fp32(seed):
    """The same for fp32 problems (fp32 kernels, 1e-4 absolute)."""
    _run_random(seed, "f32")


def _cube_constant(per_cube, T, H, W):
    """Token tensor [T, H, W, d] whose 64 tokens of cube c all equal per_cube[c]."""
    t, y, x = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
    c = ((t // 4) * (H // 4) + y // 4) * (W // 4) + x // 4
    return per_cube[c]


@pytest.mark.parametrize("case,k,latent", [("all_equal", 8, (16, 32, 32)), ("all_equal", 100, (16, 32, 32)),
                                           ("repeats", 32, (16, 32, 32)), ("repeats", 7, (16, 32, 32)),
                                           ("repeats", 64, (16, 32, 32)), ("distinct", 100, (16, 32, 32)),
                                           ("all_equal", 8, (32, 64, 128)), ("repeats", 32, (32, 64, 128)),
                                           ("distinct", 100, (32, 64, 128))])
def test_topk_exact_ties_match_oracle_bit_for_bit(case, k, latent):
    """Top-K with exact ties. Every cube's tokens are equal, so pooling is
    exact and the logits s * q_c . k_c are exact in fp32 (s = 1/8, multiples
    of 1/64): the GPU's lists must equal the oracle's (stable descending
    order, ties to the smaller cube id) on every row, whichever selection path
    the row takes (few candidates, or the radix select when more than 64
    values tie or K > 64), and for rows in registers (256 cubes) as well as
    streamed rows (4096 cubes)."""
    (T, H, W), d, heads = latent, 64, 2
    nc = T * H * W // 64
    rng = np.random.default_rng(17)
    qc = np.zeros((heads, nc, d), np.float32)
    kc = np.zeros((heads, nc, d), np.float32)
    for h in range(heads):
        qc[h, :, 0] = 1.0
        if case == "all_equal":
            kc[h, :, 0] = 0.5
        elif case == "repeats":   # 50 distinct values, each repeated
            kc[h, :, 0] = (np.arange(nc) * (7 + h) % 50) / 8.0
        else:                     # distinct where bf16 allows (values up to 255/8 are exact)
            kc[h, :, 0] = rng.permutation(nc) % 256 / 8.0
        qc[h, :, 1] = rng.integers(-4, 5, nc) / 4.0      # varies rows, leaves logits unchanged (k_c[:, 1] = 0)
    q = np.stack([_cube_constant(qc[h], T, H, W) for h in range(heads)])[None]
    kk = np.stack([_cube_constant(kc[h], T, H, W) for h in range(heads)])[None]
    v = rng.standard_normal((1, heads, T, H, W, d)).astype(np.float32)
    p = V.Problem(1, heads, T, H, W, d, topk=k)
    dq, dk, dv = (dev(a, torch.bfloat16) for a in (q, kk, v))
    qcg, kcg, vcg = V.pool(p, dq, dk, dv)
    _, _, idx, lens = V.coarse(p, qcg, kcg, vcg)
    torch.cuda.synchronize()
    gi = host(idx)
    assert (host(lens) == k).all()
    ridx = np.stack([O.topk_rows(O.coarse_attention(O.pool(O.tile(q[0, h].astype(np.float64))),
                                                    O.pool(O.tile(kk[0, h].astype(np.float64))),
                                                    O.pool(O.tile(v[0, h].astype(np.float64))), 1 / 8.0)[0], k)[0]
                     for h in range(heads)])[None]
    assert np.array_equal(gi, ridx), (case, k, np.argwhere((gi != ridx).any(-1))[:3].tolist())
