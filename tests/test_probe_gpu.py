"""The chip probes of include/vsa_probe.h on the GPU: the streaming read
reaches every element exactly once (its per-thread sums of a buffer of ones
add up to the element count, for ragged sizes, every in-flight depth and both
load kinds); the MFMA / vector-ALU probe and the L2-to-LDS probe run and
write their whole output (the latter the values of the chunks it moved)."""
import pytest
import torch

import block_sparse_video_cube_amd as V

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.mark.parametrize("nontemporal", [False, True])
@pytest.mark.parametrize("inflight", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("n_floats,blocks", [(4, 1), (1 << 20, 64), ((1 << 20) + 12, 64), (3 * 12345 * 4, 7)])
def test_stream_read_touches_every_element_once(n_floats, blocks, inflight, nontemporal):
    src = torch.ones(n_floats, dtype=torch.float32, device=DEV)
    out = torch.full((blocks * 256,), float("nan"), dtype=torch.float32, device=DEV)
    V.probe_stream_read(src, blocks, inflight, out, nontemporal)
    torch.cuda.synchronize()
    assert not torch.isnan(out).any()
    assert out.double().sum().item() == float(n_floats)


@pytest.mark.parametrize("waves", [1, 2])
@pytest.mark.parametrize("op,valu", [(0, 0), (0, 4), (0, 16), (1, 1), (1, 8)])
def test_mfma_valu_probe_runs(waves, op, valu):
    out = torch.full((65536 * waves,), float("nan"), dtype=torch.float32, device=DEV)
    V.probe_mfma_valu(valu, op, waves, 50, out)
    torch.cuda.synchronize()
    # exp2 chains may reach +inf; nothing may stay unwritten (NaN) or be NaN.
    assert not torch.isnan(out).any()
    if op == 0:
        assert torch.isfinite(out).all()


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("src_floats,blocks,iters", [(4096, 1, 2), (1 << 19, 37, 5), (1 << 16, 512, 3)])
def test_l2_to_lds_probe_moves_the_source(mode, src_floats, blocks, iters):
    src = torch.full((src_floats,), 3.0, dtype=torch.float32, device=DEV)
    out = torch.full((blocks * 128,), float("nan"), dtype=torch.float32, device=DEV)
    V.probe_l2_to_lds(mode, src, blocks, iters, out)
    torch.cuda.synchronize()
    # Every thread reads back one float of the two LDS stages, both filled
    # from the source once there are at least two iterations.
    assert (out == 3.0).all()
