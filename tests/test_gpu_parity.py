"""GPU parity: the HIP library (through the C ABI) against the CPU oracle on the same seeded inputs.

Covers the five workloads at full size (forward; backward where the workload trains), sweeps of
small random problems that span several row tiles with ragged tails, the scalar (unaligned)
path, both pool layouts, and the degenerate cases (no rows, no sequences, empty sequences,
sequences of 1..3 rows on tile boundaries, all-sentinel batches).
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

import gpu_harness as gh  # noqa: E402
import causal_depthwise_conv1d_width_amd as cc  # noqa: E402
from causal_depthwise_conv1d_width_amd import workloads as wl  # noqa: E402


def _print_case(name, **kw):
    print(f"[gpu] {name} {kw}", flush=True)


# ------------------------------------------------------------------ the five workloads
def test_single_sequence_forward(oracle):
    case = wl.single_sequence()
    _print_case(case["name"])
    gh.check_fwd(oracle, case)


@pytest.mark.parametrize("layout", ["hist", "chan"])
def test_varlen_forward_pool(oracle, layout):
    case = wl.varlen_pool(layout)
    _print_case(case["name"])
    y, pool = gh.check_fwd(oracle, case)
    # the empty sequence keeps its slot untouched; the sentinel's slot too
    ci = case["cache_indices"]
    assert np.array_equal(pool[ci[case["empty"]]], case["pool"][ci[case["empty"]]])


def test_prefill_forward_pool_padding(oracle):
    case = wl.prefill_pool()
    _print_case(case["name"])
    y, _ = gh.check_fwd(oracle, case)
    assert (y[32512:] == wl.OUT_FILL).all(), "padding rows after the last offset must stay untouched"


def test_train_seq_ids_forward_backward(oracle):
    case = wl.train_seq_ids()
    _print_case(case["name"])
    gh.check_fwd(oracle, case)
    gh.check_bwd(oracle, case)


def test_cp_share_forward_backward(oracle):
    case = wl.cp_share()
    _print_case(case["name"])
    gh.check_fwd(oracle, case)
    gh.check_bwd(oracle, case)


# ------------------------------------------------------------------ sweeps
def _sweep_cases(seed, n, mode):
    rng = np.random.default_rng(seed)
    out = []
    for q in range(n):
        C = int(rng.choice([1, 3, 8, 13, 64, 520, 1032, 1024]))
        layout = [None, "hist", "chan"][q % 3] if mode == "cu" else None
        case = wl.random_case(rng, C=C, nseq=int(rng.integers(0, 9)), max_len=int(rng.choice([3, 40, 300])),
                              mode=mode, pool_layout_name=layout, with_hist=(mode == "cu" and layout is None and q % 2 == 0),
                              L=int(rng.choice([3, 4, 6])), w_f32=bool(q % 2), act="silu" if q % 5 else "none",
                              sentinel=(q % 3 == 1), force_empty=(q % 4 == 1))
        case["name"] = f"sweep-{mode}-{seed}-{q}-C{C}"
        out.append(case)
    return out


@pytest.mark.parametrize("mode", ["cu", "idx"])
def test_sweep_forward(oracle, mode):
    for case in _sweep_cases(100 if mode == "cu" else 200, 30, mode):
        _print_case(case["name"], rows=case["x"].shape[0])
        gh.check_fwd(oracle, case)


@pytest.mark.parametrize("mode", ["cu", "idx"])
def test_sweep_backward(oracle, mode):
    for case in _sweep_cases(300 if mode == "cu" else 400, 30, mode):
        case.pop("pool", None)
        case.pop("cache_indices", None)
        case.pop("has_initial_state", None)
        _print_case(case["name"], rows=case["x"].shape[0])
        gh.check_bwd(oracle, case)


def _boundary_case(rng, C, lengths, layout="hist", hist=False, act="silu", pad=5):
    """Sequences whose first rows land on wave (32/64-row) and block (128/256-row) boundaries."""
    lengths = np.asarray(lengths, np.int64)
    cu = np.zeros(len(lengths) + 1, np.int32)
    cu[1:] = np.cumsum(lengths)
    rows = int(cu[-1]) + pad
    n = len(lengths)
    case = dict(name=f"boundary-C{C}-{layout}-{'hist' if hist else 'pool'}", act=act, cu_seqlens=cu,
                x=wl.normal_bf16(rng, (rows, C)), w=wl.uniform_f32(rng, (C, 4)),
                b=(rng.standard_normal(C) * 0.1).astype(np.float32), dy=wl.normal_bf16(rng, (rows, C)))
    if hist:
        case["hist"] = wl.normal_bf16(rng, (n, 3, C))
        case["has_history"] = (rng.random(n) < 0.7).astype(np.uint8)
    elif layout is not None:
        case["pool"] = wl.pool_layout(wl.normal_bf16(rng, (n + 3, C, 4)), layout)
        ci = rng.permutation(n + 3)[:n].astype(np.int32)
        ci[::7] = -1
        case["cache_indices"] = ci
        case["has_initial_state"] = (rng.random(n) < 0.8).astype(np.uint8)
    return case


def _boundary_lengths():
    # prefix lengths chosen so sequence starts fall 1, 2, 3 rows before/after multiples of 32 and
    # 64, with sequences of length 1, 2, 3 and 4 straddling them
    return [31, 1, 1, 1, 28, 2, 2, 62, 3, 29, 4, 1, 93, 2, 1, 127, 3, 3, 1, 125, 1, 2, 254, 5, 0, 0, 2, 3, 60]


@pytest.mark.parametrize("layout", ["hist", "chan", None])
def test_tile_boundary_sequences_forward(oracle, layout):
    rng = np.random.default_rng(7)
    for C in (512, 24, 5):
        case = _boundary_case(rng, C, _boundary_lengths(), layout=layout, hist=(layout is None))
        _print_case(case["name"])
        gh.check_fwd(oracle, case)


def test_tile_boundary_sequences_backward(oracle):
    rng = np.random.default_rng(8)
    for C in (512, 24, 5):
        case = _boundary_case(rng, C, _boundary_lengths(), layout=None, hist=True)
        _print_case(case["name"])
        gh.check_bwd(oracle, case)
        case.pop("hist")
        case.pop("has_history")
        gh.check_bwd(oracle, case)


def _tile_edge_lengths(period, n_periods=6, seed=0):
    """Sequence lengths whose starts land on every offset from -3 to +4 around multiples of `period`
    (the forward's tile heights: 16 rows, 24 with a slot pool), with sequences of 1..4 rows, so
    tiles start on a sequence's rows 0..3 and hold one or several sequence starts."""
    rng = np.random.default_rng(seed)
    lengths, pos = [], 0
    for k in range(1, n_periods + 1):
        target = k * period + int(rng.integers(-3, 5))
        if target > pos:
            lengths.append(target - pos)
            pos = target
        for n in rng.permutation([1, 2, 3, 4])[: int(rng.integers(1, 4))]:
            lengths.append(int(n))
            pos += int(n)
    lengths.append(0)
    lengths.append(5)
    return lengths


@pytest.mark.parametrize("period", [16, 24])
@pytest.mark.parametrize("layout", ["hist", "chan", None])
def test_sequence_starts_around_tile_edges(oracle, period, layout):
    """Sequence starts on each row around the tile edges of the forward, with a pool (its tile
    boundaries move off a sequence's rows 1 and 2) or with history rows; forward and, without a
    pool, backward against the oracle."""
    rng = np.random.default_rng(40 + period)
    for seed in range(4):
        for C in (512, 1040):
            case = _boundary_case(rng, C, _tile_edge_lengths(period, seed=seed), layout=layout,
                                  hist=(layout is None), pad=3)
            case["name"] = f"tile-edges-p{period}-{layout}-s{seed}-C{C}"
            _print_case(case["name"], rows=case["x"].shape[0])
            gh.check_fwd(oracle, case)
            if layout is None:
                gh.check_bwd(oracle, case)


def test_degenerate_inputs(oracle):
    rng = np.random.default_rng(9)
    C = 16
    w = wl.uniform_f32(rng, (C, 4))
    # no rows at all
    for cu in (np.array([0], np.int32), np.array([0, 0, 0], np.int32)):
        case = dict(name="empty", x=np.zeros((0, C), np.uint16), w=w, b=None, cu_seqlens=cu,
                    dy=np.zeros((0, C), np.uint16), act="silu")
        gh.check_fwd(oracle, case)
        gh.check_bwd(oracle, case)
    # rows but no sequence / only empty sequences: nothing written, dweight = 0
    for cu in (np.array([0], np.int32), np.array([0, 0, 0], np.int32)):
        case = dict(name="padding-only", x=wl.normal_bf16(rng, (9, C)), w=w, b=None, cu_seqlens=cu,
                    dy=wl.normal_bf16(rng, (9, C)), act="silu")
        y, _ = gh.check_fwd(oracle, case)
        assert (y == wl.OUT_FILL).all()
        dx, dw, _, _ = gh.check_bwd(oracle, case)
        assert (dw == 0).all() and (dx == wl.OUT_FILL).all()
    # all sentinels: zero rows, pool untouched
    cu = np.array([0, 3, 9, 10], np.int32)
    pool = wl.normal_bf16(rng, (4, C, 4))
    case = dict(name="all-sentinel", x=wl.normal_bf16(rng, (12, C)), w=w, b=None, cu_seqlens=cu, pool=pool,
                cache_indices=np.array([-1, -1, -1], np.int32), has_initial_state=np.ones(3, np.uint8), act="silu")
    y, p = gh.check_fwd(oracle, case)
    assert (y[:10] == 0).all() and np.array_equal(p, pool)
    # empty fragment with history rows: d(history) = 0
    cu = np.array([0, 4, 4, 9], np.int32)
    case = dict(name="empty-fragment-hist", x=wl.normal_bf16(rng, (9, C)), w=w, b=None, cu_seqlens=cu,
                hist=wl.normal_bf16(rng, (3, 3, C)), has_history=np.ones(3, np.uint8),
                dy=wl.normal_bf16(rng, (9, C)), act="silu")
    dx, dw, _, dh = gh.check_bwd(oracle, case)
    assert (dh[1] == 0).all()


def test_batch_rows_form(oracle):
    """Neither offsets nor IDs: every batch row of `seqlen` rows is one sequence."""
    rng = np.random.default_rng(10)
    C, B, T = 64, 5, 77
    case = dict(name="batch-rows", x=wl.normal_bf16(rng, (B * T, C)), w=wl.uniform_f32(rng, (C, 4)),
                b=(rng.standard_normal(C) * 0.1).astype(np.float32), seqlen=T, dy=wl.normal_bf16(rng, (B * T, C)),
                act="silu")
    gh.check_fwd(oracle, case)
    gh.check_bwd(oracle, case)


def _batch_case(rng, B, T, C, kind, layout="hist", W=4):
    """B batch rows of T rows (one sequence each, no offsets or IDs) with a slot pool (kind "pool":
    a -1 sentinel when B > 1, mixed has_initial_state) or caller history rows (kind "hist")."""
    rows = B * T
    case = dict(name=f"batch-rows-{kind}-B{B}-T{T}-C{C}-{layout}-W{W}", x=wl.normal_bf16(rng, (rows, C)),
                w=wl.uniform_f32(rng, (C, W)), b=(rng.standard_normal(C) * 0.1).astype(np.float32), seqlen=T,
                dy=wl.normal_bf16(rng, (rows, C)), act="silu")
    if kind == "pool":
        slots = B + 3
        case["pool"] = wl.pool_layout(wl.normal_bf16(rng, (slots, C, 4)), layout)
        ci = rng.permutation(slots)[:B].astype(np.int32)
        if B > 1:
            ci[int(rng.integers(0, B))] = -1
        case["cache_indices"] = ci
        hi = (rng.random(B) < 0.5).astype(np.uint8)
        hi[0], hi[-1] = 1, 0 if B > 1 else 1
        case["has_initial_state"] = hi
    else:
        case["hist"] = wl.normal_bf16(rng, (B, W - 1, C))
        hh = (rng.random(B) < 0.6).astype(np.uint8)
        hh[0] = 1
        case["has_history"] = hh
    return case


@pytest.mark.parametrize("layout", ["hist", "chan"])
def test_batch_rows_with_pool(oracle, layout):
    """The batch-row form with a slot pool: the sequence of a batch row is its index, so its slot
    is cache_indices[row]; state read at the first row and written back after the last.  Batch
    rows that are not a multiple of the range length, shorter than the history, and one shape at
    full size (4 x 4096 rows of 5632 channels)."""
    rng = np.random.default_rng(41)
    shapes = [(5, 77, 64), (3, 1, 520), (4, 2, 13), (7, 3, 1024), (2, 333, 24), (6, 200, 5632), (4, 4096, 5632)]
    for B, T, C in shapes:
        case = _batch_case(rng, B, T, C, "pool", layout)
        _print_case(case["name"])
        y, pool = gh.check_fwd(oracle, case)
        for i, slot in enumerate(case["cache_indices"]):
            if slot == -1:
                assert (y[i * T:(i + 1) * T] == 0).all(), "sentinel batch row must be +0"


def test_batch_rows_with_history(oracle):
    """The batch-row form with caller history rows: forward, and backward with dx, dweight, dbias
    and d(history), at widths 4, 2 and 8, ragged batch rows, and 4 x 4096 x 5632."""
    rng = np.random.default_rng(42)
    shapes = [(5, 77, 64, 4), (3, 1, 520, 4), (4, 2, 13, 4), (7, 3, 1024, 4), (2, 333, 24, 4), (6, 200, 5632, 4),
              (3, 50, 128, 2), (4, 9, 264, 8), (4, 4096, 5632, 4)]
    for B, T, C, W in shapes:
        case = _batch_case(rng, B, T, C, "hist", W=W)
        _print_case(case["name"])
        gh.check_fwd(oracle, case)
        gh.check_bwd(oracle, case)


@pytest.mark.parametrize("form", ["idx", "batch", "cu"])
def test_forward_short_ranges_at_large_row_counts(oracle, form):
    """24584 x 5632 in all three sequence forms: many rounds of 16-row tiles, batch rows of 6146
    rows (not a multiple of 16), and sequences of every length, including 1..3 rows, straddling the
    tile boundaries."""
    rng = np.random.default_rng(31)
    C, B = 5632, 4
    rows = B * 6146  # batch rows of 6146 rows: not a multiple of 40
    x = wl.normal_bf16(rng, (rows, C))
    case = dict(name=f"short-ranges-{form}", x=x, w=wl.uniform_f32(rng, (C, 4)),
                b=(rng.standard_normal(C) * 0.1).astype(np.float32), act="silu")
    lengths, total = [], 0
    while total < rows:
        n = min(int(rng.choice([1, 2, 3, 4, 39, 40, 41, 97, 1000])), rows - total)
        lengths.append(n)
        total += n
    if form == "cu":
        case["cu_seqlens"] = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    elif form == "idx":
        case["seqlen"] = rows // B
        case["seq_idx"] = np.repeat(np.arange(len(lengths)), lengths).astype(np.int32)
    else:
        case["seqlen"] = rows // B
    _print_case(case["name"], rows=rows, C=C, seqs=len(lengths))
    gh.check_fwd(oracle, case)


@pytest.mark.parametrize("C", [2048, 3600, 4096, 8192])
@pytest.mark.parametrize("form", ["cu", "idx", "pool"])
def test_forward_block_orders(oracle, C, form):
    """The forward's block-to-tile order depends on the number of 512-channel strips: slices of the
    strip-major order per XCD for 4 strips (C = 2048), plain row-major order for 8 and 16 strips
    (C = 3600 with a partial last strip, 4096, 8192).  Sequences of 1..300 rows over ~1500 rows,
    history rows in the offsets form, a slot pool (with -1 slots) in the pool form, checked against
    the oracle."""
    rng = np.random.default_rng(41 + C)
    lengths, total = [], 0
    while total < 1500:
        n = int(rng.choice([1, 2, 3, 5, 17, 40, 300]))
        lengths.append(n)
        total += n
    rows = total
    case = dict(name=f"block-order-{form}-C{C}", x=wl.normal_bf16(rng, (rows, C)), w=wl.uniform_f32(rng, (C, 4)),
                b=(rng.standard_normal(C) * 0.1).astype(np.float32), act="silu")
    if form == "cu":
        case["cu_seqlens"] = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
        case["hist"] = wl.normal_bf16(rng, (len(lengths), 3, C))
        case["has_history"] = (rng.random(len(lengths)) < 0.6).astype(np.uint8)
    elif form == "pool":  # 24-row tiles, slots taken with the lookup
        n = len(lengths)
        case["cu_seqlens"] = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
        case["pool"] = wl.pool_layout(wl.normal_bf16(rng, (n + 2, C, 4)), "chan" if C % 3 else "hist")
        ci = rng.permutation(n + 2)[:n].astype(np.int32)
        ci[::5] = -1
        case["cache_indices"] = ci
        case["has_initial_state"] = (rng.random(n) < 0.7).astype(np.uint8)
    else:
        case["seqlen"] = rows
        case["seq_idx"] = np.repeat(np.arange(len(lengths)), lengths).astype(np.int32)
    _print_case(case["name"], rows=rows, C=C, seqs=len(lengths))
    gh.check_fwd(oracle, case)


@pytest.mark.parametrize("nseq", [126, 127, 300])
def test_sequence_lookup_levels(oracle, nseq):
    """The offsets lookup is one level of two offsets per lane up to 126 sequences (the forward with
    a pool also takes every slot from it) and a 64-ary search beyond: 126, 127 and 300 sequences of
    0..40 rows, with a pool (both layouts, -1 slots, mixed has_initial_state) in the forward and
    history rows in the backward, against the oracle."""
    rng = np.random.default_rng(61 + nseq)
    C = 1032  # three strips, the last one partial
    lengths = rng.integers(0, 41, size=nseq)
    lengths[rng.choice(nseq, 5, replace=False)] = rng.integers(1, 4, size=5)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    rows = int(cu[-1]) + 3
    x = wl.normal_bf16(rng, (rows, C))
    w = wl.uniform_f32(rng, (C, 4))
    b = (rng.standard_normal(C) * 0.1).astype(np.float32)
    for layout in ("hist", "chan"):
        slots = nseq + 5
        ci = rng.permutation(slots)[:nseq].astype(np.int32)
        ci[rng.choice(nseq, 7, replace=False)] = -1
        case = dict(name=f"lookup-{nseq}-pool-{layout}", x=x, w=w, b=b, act="silu", cu_seqlens=cu,
                    pool=wl.pool_layout(wl.normal_bf16(rng, (slots, C, 4)), layout), cache_indices=ci,
                    has_initial_state=(rng.random(nseq) < 0.6).astype(np.uint8))
        _print_case(case["name"], rows=rows, C=C)
        gh.check_fwd(oracle, case)
    case = dict(name=f"lookup-{nseq}-hist", x=x, w=w, b=b, act="silu", cu_seqlens=cu,
                hist=wl.normal_bf16(rng, (nseq, 3, C)), has_history=(rng.random(nseq) < 0.7).astype(np.uint8),
                dy=wl.normal_bf16(rng, (rows, C)))
    _print_case(case["name"], rows=rows, C=C)
    gh.check_fwd(oracle, case)
    gh.check_bwd(oracle, case)


@pytest.mark.parametrize("C", [5630, 1000, 5631, 5633])
def test_partly_active_waves_at_full_size(oracle, C):
    """Channel counts that leave the last wave of every strip row partly active (5630: 63 of 64
    lanes; 1000: 52 of 64), at the context-parallel share's shape (16384 rows, 12 fragments, 8 with
    history rows, d(tail)): the lanes past the last channel run as copies of the wave's last channel
    pair.  Forward and backward against the oracle on every element, dweight/dbias bit for bit
    across three runs."""
    rng = np.random.default_rng(77 + C)
    base = wl.cp_share()
    rows = base["x"].shape[0]
    n = len(base["cu_seqlens"]) - 1
    case = dict(name=f"partial-waves-C{C}", x=wl.normal_bf16(rng, (rows, C)), w=wl.uniform_f32(rng, (C, 4)),
                b=(rng.standard_normal(C) * 0.1).astype(np.float32), cu_seqlens=base["cu_seqlens"],
                hist=wl.normal_bf16(rng, (n, 3, C)), has_history=base["has_history"],
                dy=wl.normal_bf16(rng, (rows, C)), act="silu")
    dtail = wl.normal_bf16(rng, (3, C))
    _print_case(case["name"], rows=rows, C=C)
    gh.check_fwd(oracle, case)
    _, dw, db, _ = gh.check_bwd(oracle, case, dtail=dtail)
    for _ in range(2):
        _, dw2, db2, _ = gh.gpu_bwd(case, dtail=dtail)
        assert np.array_equal(dw.view(np.int32), dw2.view(np.int32)) and np.array_equal(db.view(np.int32), db2.view(np.int32))


@pytest.mark.parametrize("C", [2, 3, 127, 129, 641, 1537])
def test_odd_channel_counts(oracle, C):
    """Odd C: a lane's two channels are one dword access at a 2-byte aligned address, and the lane of
    the lone last channel takes the pair (C-2, C-1), which overlaps the pair before it.  At C = 129,
    641 and 1537 (one above a multiple of 128, and of 512) the two pairs sit in different waves, at
    1537 in different blocks.  Offsets with history rows and d(tail), per-token IDs, batch rows,
    and the slot pool (which keeps element-wise accesses at odd C, since it is updated in place);
    dweight/dbias bit for bit across two runs."""
    rng = np.random.default_rng(900 + C)
    forms = [("cu", None, True), ("cu", "hist", False), ("cu", "chan", False), ("idx", None, False),
             ("batch", None, True), ("batch", "chan", False)]
    for q, (mode, layout, hist) in enumerate(forms):
        case = wl.random_case(rng, C=C, nseq=int(rng.integers(1, 9)), max_len=int(rng.choice([3, 40, 300])),
                              mode=mode, pool_layout_name=layout, with_hist=hist, w_f32=bool(q % 2),
                              act="silu" if q % 3 else "none", sentinel=layout is not None)
        case["name"] = f"odd-C{C}-{mode}-{layout or ('hist' if hist else 'plain')}"
        _print_case(case["name"], rows=case["x"].shape[0])
        gh.check_fwd(oracle, case)
        if layout is None:
            dtail = wl.normal_bf16(rng, (3, C))
            _, dw, db, _ = gh.check_bwd(oracle, case, dtail=dtail)
            _, dw2, db2, _ = gh.gpu_bwd(case, dtail=dtail)
            assert np.array_equal(dw.view(np.int32), dw2.view(np.int32))
            assert db is None or np.array_equal(db.view(np.int32), db2.view(np.int32))


@pytest.mark.parametrize("C,ld,off", [(1000, 1001, 1), (5632, 5633, 1), (641, 643, 3)])
def test_misaligned_rows_backward(oracle, C, ld, off):
    """Rows that start on odd elements (an odd row stride, or a view one element into a buffer):
    x, dy and dx rows at 2-byte aligned addresses, against the oracle."""
    rng = np.random.default_rng(950 + off)
    rows = 1500
    cu = np.array([0, 1, 300, 301, 900, 1490], np.int32)
    n = len(cu) - 1
    xf, dyf = wl.normal_bf16(rng, (rows, ld + off)), wl.normal_bf16(rng, (rows, ld + off))
    w = wl.uniform_f32(rng, (C, 4))
    b = (rng.standard_normal(C) * 0.1).astype(np.float32)
    hist, hh = wl.normal_bf16(rng, (n, 3, C)), (rng.random(n) < 0.7).astype(np.uint8)
    dtail = wl.normal_bf16(rng, (3, C))
    _print_case(f"misaligned-bwd-C{C}-ld{ld}-off{off}", rows=rows)
    x, dy = gh.dev_bits(xf)[:, off:off + C], gh.dev_bits(dyf)[:, off:off + C]
    dx_full = torch.full((rows, ld + off), wl.OUT_FILL, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    dx = dx_full[:, off:off + C]
    dh = torch.empty(n, 3, C, dtype=torch.bfloat16, device="cuda")
    dx, dw, db, dh = cc.conv1d_bwd(x, dy, gh.dev_taps(w), gh.dev_taps(b), cu_seqlens=gh.dev_i32(cu),
                                   history=gh.dev_bits(hist), has_history=gh.dev_u8(hh), activation="silu",
                                   dx=dx, dhistory=dh, want_dbias=True, dtail=gh.dev_bits(dtail))
    torch.cuda.synchronize()
    dxr, dwr, dbr, dhr = oracle.bwd(np.ascontiguousarray(xf[:, off:off + C]), np.ascontiguousarray(dyf[:, off:off + C]),
                                    w, b, cu_seqlens=cu, hist=hist, has_history=hh, act="silu", dtail=dtail)
    gh.assert_bf16_close(gh.host_bits(dx)[: cu[-1]], dxr[: cu[-1]], "dx")
    gh.assert_w_close(dw.cpu().numpy(), dwr, "dw")
    gh.assert_w_close(db.cpu().numpy(), dbr, "db")
    dhg = gh.host_bits(dh).reshape(n, 3, C)
    for i in np.flatnonzero(hh):
        gh.assert_bf16_close(dhg[i], dhr[i], f"dhistory {i}")
    full = gh.host_bits(dx_full)
    assert (full[:, :off] == np.uint16(wl.OUT_FILL)).all() and (full[:, off + C:] == np.uint16(wl.OUT_FILL)).all()
