"""Filter widths 2, 3 and 5..8 (taps [C, W], W-1 history rows) on the GPU against the oracle:
random packed sweeps in both sequence forms, sequences shorter than the history across range
boundaries, the context-parallel workload at full size (widths 3 and 8), and the channels-first
layout (widths 2, 3, 5 and 8)."""
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


def _narrow(case, W, rng):
    """The same problem with W taps and W-1 history rows; no pool (the pool form is width four)."""
    C = case["x"].shape[1]
    out = {k: v for k, v in case.items() if k not in ("pool", "cache_indices", "has_initial_state")}
    w = wl.uniform_f32(rng, (C, W))
    out["w"] = w if case["w"].dtype == np.float32 else wl.to_bf16_bits(w)
    if case.get("hist") is not None:
        out["hist"] = wl.normal_bf16(rng, (case["hist"].shape[0], W - 1, C))
    return out


@pytest.mark.parametrize("W", [2, 3, 5, 6, 7, 8])
@pytest.mark.parametrize("mode", ["cu", "idx"])
def test_width_sweep(oracle, W, mode):
    rng = np.random.default_rng(60 + W * 10 + (mode == "idx"))
    for q in range(24 if W < 4 else 12):
        C = int(rng.choice([1, 3, 13, 64, 520, 1024]))
        base = wl.random_case(rng, C=C, nseq=int(rng.integers(0, 9)), max_len=int(rng.choice([3, 40, 300])), mode=mode,
                              with_hist=(mode == "cu" and q % 2 == 0), w_f32=bool(q % 2),
                              act="silu" if q % 5 else "none", force_empty=(q % 4 == 1))
        case = _narrow(base, W, rng)
        case["name"] = f"width{W}-{mode}-{q}-C{C}"
        say(case["name"])
        gh.check_fwd(oracle, case)
        gh.check_bwd(oracle, case)


@pytest.mark.parametrize("W", [2, 3, 5, 8])
def test_width_short_sequences_across_ranges(oracle, W):
    """Many sequences of length 1..W (down to shorter than the history) with history rows, over
    enough rows that row-range boundaries fall inside and at the heads of them."""
    rng = np.random.default_rng(70 + W)
    C = 1024
    lengths = np.concatenate([rng.integers(1, max(5, W + 1), size=400), rng.integers(150, 260, size=6)])
    rng.shuffle(lengths)
    cu = np.zeros(len(lengths) + 1, np.int32)
    cu[1:] = np.cumsum(lengths)
    rows, n = int(cu[-1]), len(lengths)
    case = dict(name=f"width{W}-short", act="silu", cu_seqlens=cu, x=wl.normal_bf16(rng, (rows, C)),
                w=wl.uniform_f32(rng, (C, W)), b=(rng.standard_normal(C) * 0.1).astype(np.float32),
                dy=wl.normal_bf16(rng, (rows, C)), hist=wl.normal_bf16(rng, (n, W - 1, C)),
                has_history=(rng.random(n) < 0.6).astype(np.uint8))
    say(case["name"])
    gh.check_fwd(oracle, case)
    gh.check_bwd(oracle, case)


@pytest.mark.parametrize("W", [3, 8])
def test_width_context_parallel_full_size(oracle, W):
    rng = np.random.default_rng(75 + W)
    case = _narrow(wl.cp_share(), W, rng)
    case["name"] = f"width{W}-cp-share"
    say(case["name"])
    gh.check_fwd(oracle, case)
    gh.check_bwd(oracle, case)


@pytest.mark.parametrize("W", [2, 3, 5, 8])
def test_width_channels_first(oracle, W):
    rng = np.random.default_rng(80 + W)
    for B, D, T in ((2, 96, 1500), (3, 7, 517)):
        say(f"width{W} channels-first B={B} D={D} T={T}")
        x = wl.normal_bf16(rng, (B, D, T))
        dy = wl.normal_bf16(rng, (B, D, T))
        w = wl.uniform_f32(rng, (D, W))
        b = (rng.standard_normal(D) * 0.1).astype(np.float32)
        xd, dyd = gh.dev_bits(x), gh.dev_bits(dy)
        y = cc.conv1d_fwd_cf(xd, gh.dev_taps(w), gh.dev_taps(b))
        dx, dw, db = cc.conv1d_bwd_cf(xd, dyd, gh.dev_taps(w), gh.dev_taps(b), want_dbias=True)
        torch.cuda.synchronize()
        yr = oracle.fwd_cf(x, w, b)
        dxr, dwr, dbr = oracle.bwd_cf(x, dy, w, b, want_db=True)
        gh.assert_bf16_close(gh.host_bits(y).reshape(B, D, T), yr, "cf y")
        gh.assert_bf16_close(gh.host_bits(dx).reshape(B, D, T), dxr, "cf dx")
        assert dw.shape == (D, W)
        gh.assert_w_close(dw.cpu().numpy(), dwr, "cf dw")
        gh.assert_w_close(db.cpu().numpy(), dbr, "cf db")
