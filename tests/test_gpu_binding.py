"""The binding refuses output and index tensors too small for what the kernels write or read
(GPU tensors; every case fails validation before anything is launched)."""
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

import causal_depthwise_conv1d_width_amd as cc  # noqa: E402


def test_binding_refuses_undersized_tensors():
    print("[gpu] binding size checks", flush=True)
    dev = torch.device("cuda")
    C, rows, n = 64, 32, 4
    x = torch.zeros((rows, C), dtype=torch.bfloat16, device=dev)
    w = torch.zeros((C, 4), device=dev)
    cu = torch.tensor([0, 8, 16, 24, 32], dtype=torch.int32, device=dev)
    hist = torch.zeros((n, 3, C), dtype=torch.bfloat16, device=dev)
    bad = [
        dict(dweight=torch.zeros((C, 3), device=dev)),                       # wrong width
        dict(dweight=torch.zeros((C, 4), dtype=torch.float16, device=dev)),  # wrong dtype
        dict(dbias=torch.zeros((C - 1,), device=dev), want_dbias=True),
        dict(history=hist, dhistory=torch.zeros((n - 1, 3, C), dtype=torch.bfloat16, device=dev)),
        dict(history=hist[:2]),                                              # fewer row sets than sequences
        dict(history=hist, has_history=torch.ones((2,), dtype=torch.uint8, device=dev)),
        dict(dx=torch.zeros((rows - 1, C), dtype=torch.bfloat16, device=dev)),
    ]
    for kw in bad:
        with pytest.raises(ValueError):
            cc.conv1d_bwd(x, x, w, cu_seqlens=cu, **kw)
    with pytest.raises(ValueError):
        cc.conv1d_bwd(x, x[:rows - 1], w, cu_seqlens=cu)
    with pytest.raises(ValueError):
        cc.conv1d_fwd(x, w, seq_idx=torch.zeros((rows - 1,), dtype=torch.int32, device=dev), seqlen=rows)
    pool = torch.zeros((8, C, 6), dtype=torch.bfloat16, device=dev)
    ci = torch.arange(n, dtype=torch.int32, device=dev)
    with pytest.raises(ValueError):
        cc.conv1d_fwd(x, w, cu_seqlens=cu, conv_state=pool, cache_indices=ci[:2])
    with pytest.raises(ValueError):
        cc.conv1d_state_update(x[:n], w, conv_state=pool, cache_indices=ci[:2])
    with pytest.raises(ValueError):
        cc.conv1d_state_update(x[:n], w, conv_state=pool, cache_indices=ci,
                               out=torch.zeros((n - 1, C), dtype=torch.bfloat16, device=dev))
    xs = torch.zeros((n, 3, C), dtype=torch.bfloat16, device=dev)
    with pytest.raises(ValueError):
        cc.conv1d_state_update_spec(xs, w, conv_state=pool, cache_indices=ci,
                                    num_accepted=torch.ones((n - 1,), dtype=torch.int32, device=dev))
    with pytest.raises(ValueError):
        cc.conv1d_state_update_spec(xs, w, conv_state=pool, cache_indices=ci,
                                    out=torch.zeros((n, 2, C), dtype=torch.bfloat16, device=dev))
    xcf = torch.zeros((2, C, 32), dtype=torch.bfloat16, device=dev)
    with pytest.raises(ValueError):
        cc.conv1d_bwd_cf(xcf, xcf, w, dweight=torch.zeros((C,), device=dev))
    torch.cuda.synchronize()
