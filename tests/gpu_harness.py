"""Run a workload dict (see causal_depthwise_conv1d_width_amd.workloads) through the HIP library
and through the CPU oracle, and compare with the stated tolerances.

Tolerances (fixed by the target of the build, written here once):
  y, dx, dhist  |v - ref| <= 2^-7 |ref| + 1e-3           (bf16 outputs)
  dw, db        |v - ref| <= 1e-4 |ref| + 1e-4 rms(ref)  (FP32; the rms floor covers elements
                                                          that sum to almost zero)
  pool bytes, sentinel rows, untouched rows: bit-exact.
"""
import numpy as np
import torch

import causal_depthwise_conv1d_width_amd as cc
from causal_depthwise_conv1d_width_amd import workloads as wl

Y_RTOL, Y_ATOL = 2.0 ** -7, 1e-3
W_RTOL = 1e-4


def dev_bits(a, device="cuda"):
    """numpy uint16 bf16 bits -> torch bfloat16 on the device (same bits)."""
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)


def host_bits(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def dev_pool(pool, device="cuda"):
    """Same values and the same memory layout (strides) as the numpy pool."""
    st = tuple(s // 2 for s in pool.strides)
    t = torch.empty_strided(pool.shape, st, dtype=torch.bfloat16, device=device)
    t.copy_(dev_bits(np.ascontiguousarray(pool), device).view(pool.shape))
    return t


def host_pool(t):
    return host_bits(t.contiguous()).reshape(t.shape)


def dev_taps(a, device="cuda"):
    if a is None:
        return None
    if a.dtype == np.uint16:
        return dev_bits(a, device)
    return torch.from_numpy(a).to(device)


def dev_i32(a, device="cuda"):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)


def dev_u8(a, device="cuda"):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(device)


def gpu_fwd(case, out_fill=wl.OUT_FILL, x_dev=None, out=None):
    rows, C = case["x"].shape
    x = dev_bits(case["x"]) if x_dev is None else x_dev
    pool = dev_pool(case["pool"]) if case.get("pool") is not None else None
    if out is None:
        out = dev_bits(np.full((rows, C), out_fill, np.uint16))
    y = cc.conv1d_fwd(x, dev_taps(case["w"]), dev_taps(case.get("b")), cu_seqlens=dev_i32(case.get("cu_seqlens")),
                      seq_idx=dev_i32(case.get("seq_idx")), seqlen=case.get("seqlen"), conv_state=pool,
                      cache_indices=dev_i32(case.get("cache_indices")),
                      has_initial_state=dev_u8(case.get("has_initial_state")),
                      history=dev_bits(case["hist"]) if case.get("hist") is not None else None,
                      has_history=dev_u8(case.get("has_history")), activation=case.get("act", "silu"), out=out)
    torch.cuda.synchronize()
    return host_bits(y), (host_pool(pool) if pool is not None else None)


def gpu_bwd(case, workspace=None, dtail=None):
    x = dev_bits(case["x"])
    dy = dev_bits(case["dy"])
    rows, C = case["x"].shape
    hist = dev_bits(case["hist"]) if case.get("hist") is not None else None
    nseq = case["hist"].shape[0] if case.get("hist") is not None else 0
    dx = dev_bits(np.full((rows, C), wl.OUT_FILL, np.uint16))
    dh = dev_bits(np.full(case["hist"].shape, wl.OUT_FILL, np.uint16)) if hist is not None else None
    dx, dw, db, dh = cc.conv1d_bwd(x, dy, dev_taps(case["w"]), dev_taps(case.get("b")),
                                   cu_seqlens=dev_i32(case.get("cu_seqlens")), seq_idx=dev_i32(case.get("seq_idx")),
                                   seqlen=case.get("seqlen"), history=hist, has_history=dev_u8(case.get("has_history")),
                                   activation=case.get("act", "silu"), dx=dx, dhistory=dh,
                                   want_dbias=case.get("b") is not None, workspace=workspace,
                                   dtail=None if dtail is None else dev_bits(dtail))
    torch.cuda.synchronize()
    return (host_bits(dx), dw.cpu().numpy(), None if db is None else db.cpu().numpy(),
            None if dh is None else host_bits(dh).reshape(dh.shape))


def oracle_fwd(o, case):
    pool = np.array(case["pool"], copy=True, order="K") if case.get("pool") is not None else None
    y = o.fwd(case["x"], case["w"], case.get("b"), cu_seqlens=case.get("cu_seqlens"), seq_idx=case.get("seq_idx"),
              seqlen=case.get("seqlen"), pool=pool, cache_indices=case.get("cache_indices"),
              has_initial_state=case.get("has_initial_state"), hist=case.get("hist"),
              has_history=case.get("has_history"), act=case.get("act", "silu"))
    return y, pool


def oracle_bwd(o, case, dtail=None):
    return o.bwd(case["x"], case["dy"], case["w"], case.get("b"), cu_seqlens=case.get("cu_seqlens"),
                 seq_idx=case.get("seq_idx"), seqlen=case.get("seqlen"), hist=case.get("hist"),
                 has_history=case.get("has_history"), act=case.get("act", "silu"), dtail=dtail)


def f32(bits):
    return wl.bf16_bits_to_f32(bits).astype(np.float64)


def assert_bf16_close(got, ref, what, mask=None):
    """got/ref: bf16 bits. Untouched-marker cells must match bit for bit."""
    got = np.asarray(got)
    ref = np.asarray(ref)
    assert got.shape == ref.shape, f"{what}: shape {got.shape} vs {ref.shape}"
    fill = ref == wl.OUT_FILL
    assert np.array_equal(got[fill], ref[fill]), f"{what}: rows that must stay untouched were written"
    g, r = f32(got[~fill]), f32(ref[~fill])
    bad = ~(np.abs(g - r) <= Y_RTOL * np.abs(r) + Y_ATOL)
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {int(bad.sum())}/{bad.size} outside |d| <= 2^-7|ref| + 1e-3; "
                             f"e.g. got {g[bad][0]} ref {r[bad][0]}")


def assert_w_close(got, ref, what):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
    bad = ~(np.abs(got - ref) <= W_RTOL * np.abs(ref) + W_RTOL * rms)
    if bad.any():
        raise AssertionError(f"{what}: {int(bad.sum())}/{bad.size} outside 1e-4 relative "
                             f"(e.g. got {got[bad][0]} ref {ref[bad][0]}, rms {rms})")


def check_fwd(o, case, **kw):
    y, pool = gpu_fwd(case, **kw)
    yr, poolr = oracle_fwd(o, case)
    assert_bf16_close(y, yr, f"{case.get('name')}: y")
    if case.get("pool") is not None:
        assert np.array_equal(pool, poolr), f"{case.get('name')}: conv_state must match bit for bit"
    if case.get("cache_indices") is not None and case.get("cu_seqlens") is not None:
        cu = case["cu_seqlens"]
        for i, slot in enumerate(case["cache_indices"]):
            if slot == -1:
                assert (y[cu[i]:cu[i + 1]] == 0).all(), "sentinel rows must be +0"
    return y, pool


def check_bwd(o, case, dtail=None, **kw):
    dx, dw, db, dh = gpu_bwd(case, dtail=dtail, **kw)
    dxr, dwr, dbr, dhr = oracle_bwd(o, case, dtail=dtail)
    assert_bf16_close(dx, dxr, f"{case.get('name')}: dx")
    assert_w_close(dw, dwr, f"{case.get('name')}: dweight")
    if dbr is not None:
        assert_w_close(db, dbr, f"{case.get('name')}: dbias")
    if dhr is not None:
        assert_bf16_close(dh, dhr, f"{case.get('name')}: dhistory")
    return dx, dw, db, dh
