"""The Python binding checks every tensor against the Problem before it
calls the C ABI (CPU only): wrong dtype, wrong element count, missing
required tensors, short workspaces and tensors off the GPU all raise
ValueError, so no kernel is ever handed a buffer it would overrun."""
import numpy as np
import pytest
import torch

import block_sparse_video_cube_amd as V


def _p(**kw):
    base = dict(B=1, heads=2, T=8, H=8, W=8, head_dim=64, dtype="bf16", topk=2)
    base.update(kw)
    return V.Problem(**base)


def _tok(p, dtype=None, device="cpu"):
    return torch.zeros((p.B, p.heads, p.T, p.H, p.W, p.head_dim), dtype=dtype or p.torch_dtype, device=device)


def test_cpu_tensors_are_rejected_before_any_launch():
    p = _p()
    q = _tok(p)
    with pytest.raises(ValueError, match="HIP"):
        V.forward(p, q, q, q)
    with pytest.raises(ValueError, match="HIP"):
        V.pool(p, q, q, q)
    with pytest.raises(ValueError, match="HIP"):
        V.tile(p, q)


def test_wrong_dtype_is_rejected():
    p = _p()
    q32 = _tok(p, torch.float32)
    with pytest.raises(ValueError, match="bfloat16"):
        V.forward(p, q32, q32, q32)
    pf = _p(dtype="f32")
    with pytest.raises(ValueError, match="float32"):
        V.pool(pf, _tok(pf, torch.bfloat16), _tok(pf), _tok(pf))


def test_wrong_size_is_rejected():
    p = _p()
    q = _tok(p)
    short = q[..., :32].contiguous()
    with pytest.raises(ValueError, match="k has"):
        V.forward(p, q, short, q)
    # a gate of another problem's size
    with pytest.raises(ValueError, match="g_c"):
        V.forward(p, q, q, q, g_c=torch.zeros(10, dtype=torch.bfloat16))


def test_lists_are_checked():
    p = _p(topk=0, list_stride=4)
    q = _tok(p)
    with pytest.raises(ValueError, match="needs idx and lens"):
        V.forward(p, q, q, q)
    idx64 = torch.zeros((1, 2, p.Nc, 4), dtype=torch.int64)
    lens = torch.zeros((1, 2, p.Nc), dtype=torch.int32)
    with pytest.raises(ValueError, match="idx must be torch.int32"):
        V.fine_forward(p, q, q, q, idx64, lens)
    idx_short = torch.zeros((1, 2, p.Nc, 3), dtype=torch.int32)
    with pytest.raises(ValueError, match="idx has"):
        V.fine_forward(p, q, q, q, idx_short, lens)
    with pytest.raises(ValueError, match="do not hold"):
        V.check_lists_host(p, np.zeros((1, 2, p.Nc, 3), np.int32), np.zeros((1, 2, p.Nc), np.int32))


def test_pooled_and_buffer_checks():
    p = _p()
    pc = torch.zeros((1, 2, p.Nc, 64), dtype=torch.float32)
    with pytest.raises(ValueError, match="q_c must be torch.float32"):
        V.coarse(p, pc.to(torch.bfloat16), pc, pc)
    with pytest.raises(ValueError, match="k_c has"):
        V.coarse(p, pc, pc[:, :, :1].contiguous(), pc)
    # a workspace shorter than the library needs
    with pytest.raises(ValueError, match="ws holds"):
        V.coarse(p, pc, pc, pc, ws=torch.zeros(16, dtype=torch.uint8))
    # a saved buffer shorter than saved_bytes
    q = _tok(p)
    idx = torch.zeros((1, 2, p.Nc, 2), dtype=torch.int32)
    lens = torch.zeros((1, 2, p.Nc), dtype=torch.int32)
    with pytest.raises(ValueError, match="saved holds"):
        V.backward(p, q, q, q, None, None, idx, lens, torch.zeros(8, dtype=torch.uint8), q)


def test_non_contiguous_is_rejected():
    p = _p()
    q = torch.zeros((p.B, p.heads, p.T, p.H, p.head_dim, p.W), dtype=torch.bfloat16).transpose(-1, -2)
    assert not q.is_contiguous()
    with pytest.raises(ValueError):
        V.pool(p, q, q, q)


def test_checks_pass_through_to_device_check():
    """Tensors of the right dtype and size reach the device check, the last
    one before the library call (a CPU tensor stops there)."""
    p = _p()
    q = _tok(p)
    a = V._Args("probe")
    assert a.t("q", q, (p.B, p.heads, p.N, p.head_dim), torch.bfloat16) is not None
    assert a.t("g", None, (1,), torch.bfloat16, required=False) is None
    called = []
    with pytest.raises(ValueError, match="HIP"):
        a.call(lambda: called.append(1))
    assert not called
