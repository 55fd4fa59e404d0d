"""Filter widths 2, 3 and 5..8 (taps [C, W], W-1 history rows) on the GPU against the oracle:
random packed sweeps in both sequence forms, sequences shorter than the history across range
boundaries, the context-parallel workload at full size (widths 3 and 8), the channels-first
layout (widths 2, 3, 5 and 8), and wide filters with leading zero taps equal to narrow ones bit
for bit."""
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


def _run_width(case, w, hist):
    """y, dx, dweight, dbias, d(history) of the full forward and backward for taps w [C, W]."""
    x, dy = gh.dev_bits(case["x"]), gh.dev_bits(case["dy"])
    b = gh.dev_taps(case.get("b"))
    kw = dict(cu_seqlens=gh.dev_i32(case.get("cu_seqlens")), seq_idx=gh.dev_i32(case.get("seq_idx")),
              seqlen=case.get("seqlen"))
    dh = None
    if hist is not None:
        kw.update(history=gh.dev_bits(hist), has_history=gh.dev_u8(case["has_history"]))
        dh = gh.dev_bits(np.full(hist.shape, wl.OUT_FILL, np.uint16))
    y = cc.conv1d_fwd(x, gh.dev_taps(w), b, **kw)
    dx, dw, db, dh = cc.conv1d_bwd(x, dy, gh.dev_taps(w), b, want_dbias=b is not None, dhistory=dh, **kw)
    torch.cuda.synchronize()
    return (gh.host_bits(y), gh.host_bits(dx), dw.view(torch.int32).cpu().numpy(),
            None if db is None else db.view(torch.int32).cpu().numpy(),
            None if dh is None else gh.host_bits(dh).reshape(hist.shape))


@pytest.mark.parametrize("wa,wb,work", [(3, 4, "cp"), (4, 5, "cp"), (4, 6, "cp"), (4, 7, "cp"), (4, 8, "cp"),
                                        (2, 8, "cp"), (3, 4, "ids"), (4, 8, "ids")])
def test_leading_zero_taps_equal_the_narrow_filter(wa, wb, work):
    """Width wb with wb - wa leading zero taps is width wa, bit for bit: y, dx, dbias, the last wa
    columns of dweight and the last wa - 1 rows of d(history) (the first wb - wa rows are zero; the
    extra history rows meet only zero taps).  Full-size context-parallel share (offsets, history
    rows) or per-token-ID workload (with bias): a different ring, tile and chunk path against the
    narrow one, since an FMA with a zero tap leaves the sum unchanged."""
    say(f"width {wb} with {wb - wa} zero leading taps against width {wa} ({work})")
    rng = np.random.default_rng(80 + 10 * wa + wb)
    case = wl.cp_share() if work == "cp" else wl.train_seq_ids()
    C, k = case["x"].shape[1], wb - wa
    wa_taps = wl.uniform_f32(rng, (C, wa))
    wb_taps = np.concatenate([np.zeros((C, k), np.float32), wa_taps], axis=1)
    ha = hb = None
    if case.get("hist") is not None:
        n = case["hist"].shape[0]
        ha = wl.normal_bf16(rng, (n, wa - 1, C))
        hb = np.ascontiguousarray(np.concatenate([wl.normal_bf16(rng, (n, k, C)), ha], axis=1))
    ya, dxa, dwa, dba, dha = _run_width(case, wa_taps, ha)
    yb, dxb, dwb, dbb, dhb = _run_width(case, wb_taps, hb)
    assert np.array_equal(ya, yb), "y"
    assert np.array_equal(dxa, dxb), "dx"
    assert np.array_equal(dwa, np.ascontiguousarray(dwb[:, k:])), "dweight of the shared taps"
    if dba is not None:
        assert np.array_equal(dba, dbb), "dbias"
    if dha is not None:
        live = case["has_history"].astype(bool)
        assert np.array_equal(dha, dhb[:, k:]), "d(history) of the shared history rows"
        assert (gh.f32(dhb[live][:, :k]) == 0).all(), "d(history) of rows that meet only zero taps"
