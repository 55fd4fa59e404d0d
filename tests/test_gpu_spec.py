"""Speculative multi-token state update (conv1d_state_update_spec) on the GPU against the oracle:
element-wise parity, the pool bit for bit, a prefill followed by a chain of speculative steps with
random accepted counts, K = 1 against the decode entry point, and strided token rows."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

import gpu_harness as gh  # noqa: E402
import causal_depthwise_conv1d_width_amd as cc  # noqa: E402
from causal_depthwise_conv1d_width_amd import workloads as wl  # noqa: E402


def say(msg):
    print(f"[gpu] {msg}", flush=True)


def _setup(rng, N, K, C, L, layout, w_bf16=False, sentinel=True):
    x = wl.normal_bf16(rng, (N, K, C))
    w = wl.to_bf16_bits(wl.uniform_f32(rng, (C, 4))) if w_bf16 else wl.uniform_f32(rng, (C, 4))
    b = (rng.standard_normal(C) * 0.1).astype(np.float32)
    vals = wl.normal_bf16(rng, (N + 4, C, L))
    ci = rng.permutation(N + 4)[:N].astype(np.int32)
    if sentinel and N > 1:
        ci[1] = -1
    acc = rng.integers(1, L - 1, size=N).astype(np.int32)
    return x, w, b, vals, ci, acc


@pytest.mark.parametrize("layout", ["hist", "chan"])
def test_spec_update_matches_oracle(oracle, layout):
    rng = np.random.default_rng(41)
    for C, N, K, L, act in ((5632, 64, 4, 6, "silu"), (13, 9, 2, 4, "none"), (1024, 7, 7, 9, "silu"),
                            (2048, 5, 1, 3, "silu"), (4096, 3, 3, 12, "silu")):
        say(f"spec update {layout} C={C} N={N} K={K} L={L}")
        x, w, b, vals, ci, acc = _setup(rng, N, K, C, L, layout, w_bf16=(C == 13))
        pool = gh.dev_pool(wl.pool_layout(vals.copy(), layout))
        out = gh.dev_bits(np.full((N, K, C), wl.OUT_FILL, np.uint16))
        y = cc.conv1d_state_update_spec(gh.dev_bits(x), gh.dev_taps(w), gh.dev_taps(b), conv_state=pool,
                                        cache_indices=gh.dev_i32(ci), num_accepted=gh.dev_i32(acc), activation=act,
                                        out=out)
        torch.cuda.synchronize()
        ref_pool = wl.pool_layout(vals.copy(), layout)
        yr = oracle.spec_update(x, w, b, pool=ref_pool, cache_indices=ci, accepted=acc, act=act)
        gh.assert_bf16_close(gh.host_bits(y).reshape(N, K, C), yr, f"spec y K={K}")
        assert np.array_equal(gh.host_pool(pool), ref_pool), f"spec state write-back K={K}"


def test_spec_chain_after_prefill(oracle):
    """Prefill, then speculative steps whose accepted counts come from the previous step: every
    step's outputs and the final pool match the oracle run of the same chain."""
    rng = np.random.default_rng(42)
    N, C, K, L = 16, 3072, 4, 7
    lengths = rng.integers(1, 300, size=N)
    cu = np.zeros(N + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    xp = wl.normal_bf16(rng, (int(cu[-1]), C))
    w = wl.uniform_f32(rng, (C, 4))
    b = (rng.standard_normal(C) * 0.1).astype(np.float32)
    vals = wl.normal_bf16(rng, (N + 3, C, L))
    ci = rng.permutation(N + 3)[:N].astype(np.int32)
    ci[5] = -1
    hi = (rng.random(N) < 0.5).astype(np.uint8)
    pool = gh.dev_pool(vals.copy())
    ref_pool = vals.copy()
    say("spec chain: prefill")
    y0 = cc.conv1d_fwd(gh.dev_bits(xp), gh.dev_taps(w), gh.dev_taps(b), cu_seqlens=gh.dev_i32(cu), conv_state=pool,
                       cache_indices=gh.dev_i32(ci), has_initial_state=gh.dev_u8(hi))
    yr0 = oracle.fwd(xp, w, b, cu_seqlens=cu, pool=ref_pool, cache_indices=ci, has_initial_state=hi)
    torch.cuda.synchronize()
    gh.assert_bf16_close(gh.host_bits(y0), yr0, "prefill y")
    acc = np.ones(N, dtype=np.int32)
    for step in range(5):
        say(f"spec chain: step {step}")
        xs = wl.normal_bf16(rng, (N, K, C))
        y = cc.conv1d_state_update_spec(gh.dev_bits(xs), gh.dev_taps(w), gh.dev_taps(b), conv_state=pool,
                                        cache_indices=gh.dev_i32(ci), num_accepted=gh.dev_i32(acc))
        yr = oracle.spec_update(xs, w, b, pool=ref_pool, cache_indices=ci, accepted=acc)
        torch.cuda.synchronize()
        gh.assert_bf16_close(gh.host_bits(y).reshape(N, K, C), yr, f"spec chain step {step}")
        assert np.array_equal(gh.host_pool(pool), ref_pool), f"spec chain pool after step {step}"
        acc = rng.integers(1, K + 1, size=N).astype(np.int32)


def test_spec_k1_equals_decode():
    rng = np.random.default_rng(43)
    for C, N, L in ((5632, 32, 4), (13, 5, 3)):
        say(f"spec K=1 vs decode C={C}")
        x, w, b, vals, ci, _ = _setup(rng, N, 1, C, L, "hist")
        p1, p2 = gh.dev_pool(vals.copy()), gh.dev_pool(vals.copy())
        y1 = cc.conv1d_state_update_spec(gh.dev_bits(x), gh.dev_taps(w), gh.dev_taps(b), conv_state=p1,
                                         cache_indices=gh.dev_i32(ci))
        y2 = cc.conv1d_state_update(gh.dev_bits(x[:, 0]), gh.dev_taps(w), gh.dev_taps(b), conv_state=p2,
                                    cache_indices=gh.dev_i32(ci))
        torch.cuda.synchronize()
        assert np.array_equal(gh.host_bits(y1)[:, 0], gh.host_bits(y2)), "K = 1 outputs == decode"
        assert np.array_equal(gh.host_pool(p1), gh.host_pool(p2)), "K = 1 state == decode"


def test_spec_strided_rows(oracle):
    """Token rows with a row stride larger than C (a view into a wider buffer), output likewise."""
    rng = np.random.default_rng(44)
    N, K, C, L, pad = 6, 3, 1536, 5, 512
    say("spec strided rows")
    x, w, b, vals, ci, acc = _setup(rng, N, K, C, L, "chan")
    wide = np.zeros((N, K, C + pad), np.uint16)
    wide[:, :, :C] = x
    xd = gh.dev_bits(wide)[:, :, :C]
    outw = gh.dev_bits(np.full((N, K, C + pad), wl.OUT_FILL, np.uint16))
    pool = gh.dev_pool(wl.pool_layout(vals.copy(), "chan"))
    cc.conv1d_state_update_spec(xd, gh.dev_taps(w), gh.dev_taps(b), conv_state=pool, cache_indices=gh.dev_i32(ci),
                                num_accepted=gh.dev_i32(acc), out=outw[:, :, :C])
    torch.cuda.synchronize()
    ref_pool = wl.pool_layout(vals.copy(), "chan")
    yr = oracle.spec_update(x, w, b, pool=ref_pool, cache_indices=ci, accepted=acc)
    got = gh.host_bits(outw).reshape(N, K, C + pad)
    gh.assert_bf16_close(got[:, :, :C], yr, "strided spec y")
    assert (got[:, :, C:] == wl.OUT_FILL).all(), "padding columns untouched"
    assert np.array_equal(gh.host_pool(pool), ref_pool)
