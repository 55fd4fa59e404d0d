"""The Python binding's own checks, decided before the library is called (CPU only).

Tensors on the host would reach the kernels as host addresses, so every entry point refuses them.
"""
import pytest

torch = pytest.importorskip("torch")

import causal_depthwise_conv1d_width_amd as cc  # noqa: E402


def test_entry_points_refuse_host_tensors():
    C, rows = 16, 8
    x = torch.zeros((rows, C), dtype=torch.bfloat16)
    w = torch.zeros((C, 4))
    cu = torch.tensor([0, rows], dtype=torch.int32)
    pool = torch.zeros((2, C, 4), dtype=torch.bfloat16)
    ci = torch.zeros((rows,), dtype=torch.int32)
    with pytest.raises(ValueError, match="GPU"):
        cc.conv1d_fwd(x, w, cu_seqlens=cu)
    with pytest.raises(ValueError, match="GPU"):
        cc.conv1d_bwd(x, x, w, cu_seqlens=cu)
    with pytest.raises(ValueError, match="GPU"):
        cc.conv1d_state_update(x, w, conv_state=pool, cache_indices=ci)
    with pytest.raises(ValueError, match="GPU"):
        cc.conv1d_state_update_spec(x.view(rows, 1, C), w, conv_state=pool, cache_indices=ci)
    xcf = torch.zeros((2, C, 32), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        cc.conv1d_fwd_cf(xcf, w)
    with pytest.raises(ValueError, match="GPU"):
        cc.conv1d_bwd_cf(xcf, xcf, w)


def test_shape_checks_come_first():
    C, rows = 16, 8
    x = torch.zeros((rows, C), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="weight"):
        cc.conv1d_fwd(x, torch.zeros((C, 9)), cu_seqlens=torch.tensor([0, rows], dtype=torch.int32))
    with pytest.raises(ValueError, match="weight"):
        cc.conv1d_fwd_cf(torch.zeros((2, C, 32), dtype=torch.bfloat16), torch.zeros((C, 9)))
    with pytest.raises(ValueError, match="bf16"):
        cc.conv1d_fwd(x.float(), torch.zeros((C, 4)), cu_seqlens=torch.tensor([0, rows], dtype=torch.int32))
