"""Randomized parity against the oracle: 3000 small problems from fixed seeds, each drawing its
sequence form (offsets, per-token IDs, batch rows), channel count (1..2050, partial strips and
odd counts), sequence count (0..140, both levels of the offsets lookup), lengths (1..1000), filter
width (2..8), slot pool (both layouts, -1 slots, 3..6 positions) or history rows, d(tail),
activation, tap and bias dtypes, and empty sequences.  Forward always, backward without a pool.
A failure names its seed; the case is rebuilt by make_case(seed).  Then 1500 decode steps,
speculative updates (1..8 tokens, 3..14 pool positions, random accepted counts) and channels-first
problems (widths 2..8, ragged T) the same way."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

import gpu_harness as gh  # noqa: E402
import causal_depthwise_conv1d_width_amd as cc  # noqa: E402
from causal_depthwise_conv1d_width_amd import workloads as wl  # noqa: E402

CHANNELS = [1, 2, 3, 7, 8, 13, 64, 127, 128, 130, 256, 510, 512, 514, 1000, 1024, 1032, 1536, 2048, 2050]
SEEDS = range(20000, 23000)


def make_case(seed):
    """(case, dtail, has_pool) for one seed; problems stay under ~3M elements."""
    rng = np.random.default_rng(seed)
    mode = str(rng.choice(["cu", "cu", "idx", "batch"]))
    C = int(rng.choice(CHANNELS))
    nseq = int(rng.choice([0, 1, 2, 5, 9, 30, 126, 127, 140]))
    max_len = int(rng.choice([1, 2, 3, 5, 10, 40, 300, 1000]))
    while nseq * max_len * C > 3_000_000 and max_len > 1:
        max_len //= 2
    pool = mode in ("cu", "batch") and rng.random() < 0.35
    hist = mode in ("cu", "batch") and not pool and rng.random() < 0.5
    W = 4 if pool else int(rng.choice([2, 3, 4, 4, 5, 6, 7, 8]))  # the pool form is width four
    case = wl.random_case(rng, C=C, nseq=nseq, max_len=max_len, mode=mode,
                          pool_layout_name=(str(rng.choice(["hist", "chan"])) if pool else None),
                          L=int(rng.choice([3, 4, 6])), with_hist=hist, w_f32=bool(rng.integers(0, 2)),
                          act=str(rng.choice(["silu", "silu", "none"])), force_empty=bool(rng.random() < 0.3),
                          sentinel=bool(rng.random() < 0.5))
    if W != 4:
        w = wl.uniform_f32(rng, (C, W))
        case["w"] = w if case["w"].dtype == np.float32 else wl.to_bf16_bits(w)
        if case.get("hist") is not None:
            case["hist"] = wl.normal_bf16(rng, (case["hist"].shape[0], W - 1, C))
    dtail = wl.normal_bf16(rng, (W - 1, C)) if mode == "cu" and not pool and rng.random() < 0.3 else None
    case["name"] = (f"seed{seed}-{mode}-C{C}-n{nseq}-L{max_len}-W{W}-"
                    f"{'pool' if pool else ('hist' if hist else 'plain')}{'-dtail' if dtail is not None else ''}")
    return case, dtail, pool


def test_random_problems(oracle):
    print(f"[gpu] random problems, seeds {SEEDS.start}..{SEEDS.stop - 1}", flush=True)
    failures = []
    for seed in SEEDS:
        case, dtail, pool = make_case(seed)
        try:
            gh.check_fwd(oracle, case)
            if not pool:
                gh.check_bwd(oracle, case, dtail=dtail)
        except AssertionError as e:
            failures.append(f"{case['name']}: {str(e)[:200]}")
    assert not failures, f"{len(failures)} of {len(SEEDS)} random problems differ:\n" + "\n".join(failures[:20])


SEEDS_SMALL = range(60000, 61500)


def _taps(rng, C, W):
    w = wl.uniform_f32(rng, (C, W))
    return w if rng.random() < 0.5 else wl.to_bf16_bits(w)


def _bias(rng, C):
    if rng.random() < 0.4:
        return None
    b = (rng.standard_normal(C) * 0.1).astype(np.float32)
    return b if rng.random() < 0.5 else wl.to_bf16_bits(b)


def check_small(oracle, seed):
    """One random decode step, speculative update or channels-first problem for `seed`."""
    rng = np.random.default_rng(seed)
    kind = str(rng.choice(["decode", "spec", "cf"]))
    act = str(rng.choice(["silu", "silu", "none"]))
    C = int(rng.choice(CHANNELS))
    if kind in ("decode", "spec"):
        N, layout = int(rng.integers(1, 70)), str(rng.choice(["hist", "chan"]))
        K = 1 if kind == "decode" else int(rng.integers(1, 9))
        L = int(rng.integers(max(3, K + 2), K + 7))
        w, b = _taps(rng, C, 4), _bias(rng, C)
        vals = wl.normal_bf16(rng, (N + 3, C, L))
        ci = rng.permutation(N + 3)[:N].astype(np.int32)
        if rng.random() < 0.5:
            ci[int(rng.integers(0, N))] = -1
        pool, ref_pool = gh.dev_pool(wl.pool_layout(vals.copy(), layout)), wl.pool_layout(vals.copy(), layout)
        name = f"seed{seed}-{kind}-C{C}-N{N}-K{K}-L{L}-{layout}-{act}"
        if kind == "decode":
            x = wl.normal_bf16(rng, (N, C))
            y = cc.conv1d_state_update(gh.dev_bits(x), gh.dev_taps(w), gh.dev_taps(b), conv_state=pool,
                                       cache_indices=gh.dev_i32(ci), activation=act)
            torch.cuda.synchronize()
            gh.assert_bf16_close(gh.host_bits(y), oracle.state_update(x, w, b, pool=ref_pool, cache_indices=ci, act=act),
                                 name + " y")
        else:
            x = wl.normal_bf16(rng, (N, K, C))
            acc = rng.integers(1, L - 1, size=N).astype(np.int32)
            y = cc.conv1d_state_update_spec(gh.dev_bits(x), gh.dev_taps(w), gh.dev_taps(b), conv_state=pool,
                                            cache_indices=gh.dev_i32(ci), num_accepted=gh.dev_i32(acc), activation=act,
                                            out=gh.dev_bits(np.full((N, K, C), wl.OUT_FILL, np.uint16)))
            torch.cuda.synchronize()
            yr = oracle.spec_update(x, w, b, pool=ref_pool, cache_indices=ci, accepted=acc, act=act)
            gh.assert_bf16_close(gh.host_bits(y).reshape(N, K, C), yr, name + " y")
        assert np.array_equal(gh.host_pool(pool), ref_pool), name + " pool"
        return
    B, T = int(rng.integers(1, 6)), int(rng.choice([1, 2, 5, 8, 100, 512, 513, 1000, 2048, 5000]))
    D = C if B * C * T <= 3_000_000 else max(1, 3_000_000 // (B * T))
    W = int(rng.choice([2, 3, 4, 4, 5, 6, 7, 8]))
    w, b = _taps(rng, D, W), _bias(rng, D)
    x, dy = wl.normal_bf16(rng, (B, D, T)), wl.normal_bf16(rng, (B, D, T))
    name = f"seed{seed}-cf-B{B}-D{D}-T{T}-W{W}-{act}"
    y = cc.conv1d_fwd_cf(gh.dev_bits(x), gh.dev_taps(w), gh.dev_taps(b), activation=act)
    dx, dw, db = cc.conv1d_bwd_cf(gh.dev_bits(x), gh.dev_bits(dy), gh.dev_taps(w), gh.dev_taps(b), activation=act,
                                  want_dbias=b is not None)
    torch.cuda.synchronize()
    gh.assert_bf16_close(gh.host_bits(y).reshape(B, D, T), oracle.fwd_cf(x, w, b, act=act), name + " y")
    dxr, dwr, dbr = oracle.bwd_cf(x, dy, w, b, act=act, want_db=b is not None)
    gh.assert_bf16_close(gh.host_bits(dx).reshape(B, D, T), dxr, name + " dx")
    gh.assert_w_close(dw.cpu().numpy(), dwr, name + " dw")
    if b is not None:
        gh.assert_w_close(db.cpu().numpy(), dbr, name + " db")


def test_random_decode_spec_channels_first(oracle):
    print(f"[gpu] random decode / speculative / channels-first problems, seeds {SEEDS_SMALL.start}.."
          f"{SEEDS_SMALL.stop - 1}", flush=True)
    failures = []
    for seed in SEEDS_SMALL:
        try:
            check_small(oracle, seed)
        except AssertionError as e:
            failures.append(str(e)[:200])
    assert not failures, f"{len(failures)} of {len(SEEDS_SMALL)} problems differ:\n" + "\n".join(failures[:20])
