"""Channels-first [B, D, T] forward and backward (conv1d_fwd_cf / conv1d_bwd_cf) on the GPU against
the oracle: ragged T (the element-wise path), rows longer than one unrolled chunk, strided views,
empty T, bitwise-reproducible dweight, and the forward bit for bit equal to the channel-last one."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

import gpu_harness as gh  # noqa: E402
import causal_depthwise_conv1d_width_amd as cc  # noqa: E402
from causal_depthwise_conv1d_width_amd import workloads as wl  # noqa: E402

SHAPES = [  # B, D, T, act, bf16 taps, bias
    (4, 4096, 4096, "silu", False, True),  # the training shape of the per-token-ID workload, channels first
    (2, 13, 1000, "silu", True, True),
    (3, 5, 517, "none", False, False),  # T % 8 != 0: element-wise path
    (1, 3, 1, "silu", False, True),
    (2, 7, 5000, "silu", False, True),  # several unrolled chunks and a ragged last block
    (5, 64, 520, "silu", True, False),
]


def say(msg):
    print(f"[gpu] {msg}", flush=True)


def _case(rng, B, D, T, w_bf16, bias):
    x = wl.normal_bf16(rng, (B, D, T))
    dy = wl.normal_bf16(rng, (B, D, T))
    w = wl.to_bf16_bits(wl.uniform_f32(rng, (D, 4))) if w_bf16 else wl.uniform_f32(rng, (D, 4))
    b = (rng.standard_normal(D) * 0.1).astype(np.float32) if bias else None
    return x, dy, w, b


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"B{s[0]}_D{s[1]}_T{s[2]}_{s[3]}")
def test_cf_forward_backward_match_oracle(oracle, shape):
    B, D, T, act, w_bf16, bias = shape
    say(f"channels-first B={B} D={D} T={T} {act}")
    rng = np.random.default_rng(51 + B * 7 + T)
    x, dy, w, b = _case(rng, B, D, T, w_bf16, bias)
    xd, dyd = gh.dev_bits(x), gh.dev_bits(dy)
    y = cc.conv1d_fwd_cf(xd, gh.dev_taps(w), gh.dev_taps(b), activation=act)
    dx, dw, db = cc.conv1d_bwd_cf(xd, dyd, gh.dev_taps(w), gh.dev_taps(b), activation=act, want_dbias=True)
    torch.cuda.synchronize()
    yr = oracle.fwd_cf(x, w, b, act=act)
    dxr, dwr, dbr = oracle.bwd_cf(x, dy, w, b, act=act, want_db=True)
    gh.assert_bf16_close(gh.host_bits(y).reshape(B, D, T), yr, "cf y")
    gh.assert_bf16_close(gh.host_bits(dx).reshape(B, D, T), dxr, "cf dx")
    gh.assert_w_close(dw.cpu().numpy(), dwr, "cf dw")
    gh.assert_w_close(db.cpu().numpy(), dbr, "cf db")


def test_cf_dweight_bitwise_reproducible():
    say("channels-first determinism")
    rng = np.random.default_rng(57)
    x, dy, w, b = _case(rng, 4, 2048, 4096, False, True)
    xd, dyd, wd, bd = gh.dev_bits(x), gh.dev_bits(dy), gh.dev_taps(w), gh.dev_taps(b)
    ref = None
    for rep in range(4):
        ws = torch.full((cc.conv1d_bwd_cf_workspace_bytes(4, 2048) + 256,), rep * 37, dtype=torch.uint8,
                        device="cuda")
        _, dw, db = cc.conv1d_bwd_cf(xd, dyd, wd, bd, want_dbias=True, workspace=ws[256 * (rep % 2):])
        torch.cuda.synchronize()
        got = (dw.cpu().numpy().tobytes(), db.cpu().numpy().tobytes())
        if ref is None:
            ref = got
        assert got == ref, f"dweight/dbias bits changed on run {rep}"


def test_cf_strided_views(oracle):
    """x and y as views of wider buffers (extra time steps and channels), dy likewise."""
    say("channels-first strided views")
    rng = np.random.default_rng(58)
    B, D, T = 3, 24, 777
    x, dy, w, b = _case(rng, B, D, T, False, True)
    big = np.zeros((B, D + 5, T + 40), np.uint16)
    big[:, :D, :T] = x
    bigdy = np.zeros((B, D + 5, T + 40), np.uint16)
    bigdy[:, :D, :T] = dy
    xd = gh.dev_bits(big)[:, :D, :T]
    dyd = gh.dev_bits(bigdy)[:, :D, :T]
    yw = gh.dev_bits(np.full((B, D + 2, T + 9), wl.OUT_FILL, np.uint16))
    y = cc.conv1d_fwd_cf(xd, gh.dev_taps(w), gh.dev_taps(b), out=yw[:, 1:D + 1, 3:T + 3])
    dxw = gh.dev_bits(np.full((B, D + 2, T + 9), wl.OUT_FILL, np.uint16))
    dx, dw, db = cc.conv1d_bwd_cf(xd, dyd, gh.dev_taps(w), gh.dev_taps(b), dx=dxw[:, 1:D + 1, 3:T + 3], want_dbias=True)
    torch.cuda.synchronize()
    yr = oracle.fwd_cf(x, w, b)
    dxr, dwr, dbr = oracle.bwd_cf(x, dy, w, b, want_db=True)
    got_y = gh.host_bits(yw).reshape(B, D + 2, T + 9)
    got_dx = gh.host_bits(dxw).reshape(B, D + 2, T + 9)
    gh.assert_bf16_close(got_y[:, 1:D + 1, 3:T + 3], yr, "strided cf y")
    gh.assert_bf16_close(got_dx[:, 1:D + 1, 3:T + 3], dxr, "strided cf dx")
    for arr in (got_y, got_dx):
        mask = np.ones(arr.shape, bool)
        mask[:, 1:D + 1, 3:T + 3] = False
        assert (arr[mask] == wl.OUT_FILL).all(), "elements outside the view untouched"
    gh.assert_w_close(dw.cpu().numpy(), dwr, "strided cf dw")
    gh.assert_w_close(db.cpu().numpy(), dbr, "strided cf db")


def test_cf_empty_time_axis():
    say("channels-first T = 0")
    D = 40
    w = torch.rand((D, 4), device="cuda")
    x = torch.empty((2, D, 0), dtype=torch.bfloat16, device="cuda")
    y = cc.conv1d_fwd_cf(x, w)
    dx, dw, db = cc.conv1d_bwd_cf(x, x.clone(), w, torch.zeros(D, device="cuda"), want_dbias=True)
    torch.cuda.synchronize()
    assert y.shape == (2, D, 0) and dx.shape == (2, D, 0)
    assert (dw == 0).all() and (db == 0).all(), "no steps: zero dweight / dbias"


@pytest.mark.parametrize("W", [4, 8])
def test_cf_forward_equals_channel_last(W):
    """[4, 4096, 4096] channels first against the channel-last forward of the same values
    transposed to [B * T, D] with one sequence per T-row batch row: the same y bits (both kernels
    take bias, then taps 0..W-1 as FP32 FMAs, and the same SiLU)."""
    say(f"channels-first forward against channel-last, width {W}")
    rng = np.random.default_rng(42 + W)
    B, D, T = 4, 4096, 4096
    x = torch.empty(B, D, T, dtype=torch.bfloat16, device="cuda")
    x.normal_(generator=torch.Generator(device="cuda").manual_seed(15 + W))
    w = gh.dev_taps(wl.uniform_f32(rng, (D, W)))
    b = gh.dev_taps((rng.standard_normal(D) * 0.1).astype(np.float32))
    y_cf = cc.conv1d_fwd_cf(x, w, b)
    xl = x.transpose(1, 2).contiguous().view(B * T, D)
    y_cl = cc.conv1d_fwd(xl, w, b, seqlen=T)
    torch.cuda.synchronize()
    assert torch.equal(y_cf.transpose(1, 2).contiguous().view(B * T, D).view(torch.int16), y_cl.view(torch.int16))
