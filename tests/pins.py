"""Pins of the CPU oracle: checks against things other than the oracle itself.

Each ``pin_*`` takes an ``Oracle`` and raises AssertionError when the oracle disagrees with what
the pages and the mathematics fix.  They are collected by ``test_oracle_pins.py`` and are also
run against deliberately broken copies of the oracle by ``test_pins_have_teeth.py``.

Sources of truth used here (none of them calls the oracle's arithmetic):
  * closed-form values of round-to-nearest-even to bf16;
  * the dense Toeplitz formulation in ``bruteforce.py`` (fp64) and torch autograd through it;
  * torch's grouped ``conv1d`` for the one-segment, zero-history special case;
  * closed forms: identity taps, unit taps (pin tap order and history order), zero taps;
  * central finite differences of the fp64 loss;
  * the invariants the pages state: per-sequence reset, causality, state write-back of the last
    three raw inputs, empty and -1 sequences leaving the pool alone, has_initial_state false =
    zero history, chunked prefill = one call, fragments with history rows = the unsplit batch.
"""
import numpy as np
import torch

import bruteforce as bf
from causal_depthwise_conv1d_width_amd import workloads as wl

FILL = wl.OUT_FILL


def _fwd(o, case, y=None, pool=None):
    return o.fwd(case["x"], case["w"], case.get("b"), cu_seqlens=case.get("cu_seqlens"),
                 seq_idx=case.get("seq_idx"), seqlen=case.get("seqlen"),
                 pool=case.get("pool") if pool is None else pool,
                 cache_indices=case.get("cache_indices"),
                 has_initial_state=case.get("has_initial_state"), hist=case.get("hist"),
                 has_history=case.get("has_history"), act=case.get("act", "silu"), y=y)


def _bwd(o, case):
    return o.bwd(case["x"], case["dy"], case["w"], case.get("b"), cu_seqlens=case.get("cu_seqlens"),
                 seq_idx=case.get("seq_idx"), seqlen=case.get("seqlen"), hist=case.get("hist"),
                 has_history=case.get("has_history"), act=case.get("act", "silu"))


def _close(got, ref, rtol, atol, what):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    bad = np.abs(got - ref) > rtol * np.abs(ref) + atol
    assert not bad.any(), f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; " \
        f"first at {np.argwhere(bad)[0].tolist()}: got {got[bad][0]!r} ref {ref[bad][0]!r}"


def _cases(seed, n, **kw):
    rng = np.random.default_rng(seed)
    out = []
    for q in range(n):
        mode = "idx" if q % 4 == 3 else "cu"
        layout = [None, "hist", "chan"][q % 3] if mode == "cu" else None
        hist = mode == "cu" and layout is None and q % 2 == 0
        out.append(wl.random_case(rng, mode=mode, pool_layout_name=layout, with_hist=hist,
                                  L=int(rng.choice([3, 4, 6])), w_f32=bool(q % 2),
                                  act="silu" if q % 5 else "none", sentinel=(q % 3 == 1),
                                  force_empty=(q % 2 == 1), **kw))
    return out


# ------------------------------------------------------------------ rounding
def pin_rounding(o):
    one = 1.0
    # exact, ties-to-even, and just-above-tie cases around 1.0 (bf16 ulp at 1 is 2^-7)
    assert o.round_double(one) == 0x3F80
    assert o.round_double(one + 2.0 ** -8) == 0x3F80            # tie -> even (down)
    assert o.round_double(one + 3 * 2.0 ** -8) == 0x3F82        # tie -> even (up)
    assert o.round_double(one + 2.0 ** -8 + 2.0 ** -30) == 0x3F81  # above tie: float would tie
    assert o.round_double(-(one + 2.0 ** -8 + 2.0 ** -30)) == 0xBF81
    assert o.round_double(one + 2.0 ** -8 - 2.0 ** -30) == 0x3F80
    assert o.round_double(-2.5) == 0xC020
    assert o.round_double(0.0) == 0x0000
    assert o.round_float(one + 2.0 ** -8) == 0x3F80
    assert o.round_float(one + 3 * 2.0 ** -8) == 0x3F82
    assert o.round_float(one + 2.0 ** -8 + 2.0 ** -20) == 0x3F81
    assert o.round_float(3.0e38) == 0x7F62  # 3e38 -> 0x7F61C... rounds to nearest 0x7F62
    assert o.round_float(-0.0) == 0x8000


# ------------------------------------------------------------------ forward
def pin_forward_bruteforce(o, seed=11, n=24):
    for case in _cases(seed, n):
        pool0 = case["pool"].copy() if case.get("pool") is not None else None
        _, yref, covered, sent = bf.forward_f64(case)   # reference first: the oracle updates the pool
        yref = yref.numpy()
        y = _fwd(o, case)
        yo = bf.f64(y)
        live = covered & ~sent
        _close(yo[live], yref[live], 2.0 ** -8, 1e-5, "y vs dense Toeplitz")
        assert (y[sent] == 0).all(), "sentinel rows must be +0"
        assert (y[~covered] == FILL).all(), "rows past the last offset must stay untouched"
        if pool0 is not None:
            case_before = dict(case, pool=pool0)
            assert np.array_equal(case["pool"], bf.pool_after(case_before)), "pool write-back"


def pin_forward_conv1d_library(o, seed=12):
    import torch.nn.functional as F
    rng = np.random.default_rng(seed)
    for C, T in [(1, 1), (3, 2), (8, 9), (13, 40), (64, 17)]:
        for act in ("silu", "none"):
            x = wl.normal_bf16(rng, (T, C))
            w = wl.uniform_f32(rng, (C, 4))
            b = (rng.standard_normal(C) * 0.1).astype(np.float32)
            y = o.fwd(x, w, b, cu_seqlens=np.array([0, T], np.int32), act=act)
            xt = torch.tensor(bf.f64(x)).T[None]                     # [1, C, T]
            z = F.conv1d(F.pad(xt, (3, 0)), torch.tensor(w, dtype=torch.float64)[:, None, :],
                         torch.tensor(b, dtype=torch.float64), groups=C)[0].T
            ref = (F.silu(z) if act == "silu" else z).numpy()
            _close(bf.f64(y), ref, 2.0 ** -8, 1e-5, f"conv1d special case C={C} T={T} {act}")


def pin_forward_closed_forms(o, seed=13):
    rng = np.random.default_rng(seed)
    C, lengths = 5, [4, 1, 2, 0, 7]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    rows = int(cu[-1]) + 2
    x = wl.normal_bf16(rng, (rows, C))
    for layout in ("hist", "chan"):
        pool_vals = wl.normal_bf16(rng, (6, C, 4))
        ci = np.array([4, 0, 2, 5, 1], np.int32)
        hi = np.ones(5, np.uint8)
        for k in range(4):
            w = np.zeros((C, 4), np.float32)
            w[:, k] = 1.0
            pool = wl.pool_layout(pool_vals.copy(), layout)
            y = o.fwd(x, w, None, cu_seqlens=cu, pool=pool, cache_indices=ci, has_initial_state=hi, act="none")
            for i, (s, e) in enumerate(zip(cu[:-1], cu[1:])):
                ext = np.concatenate([pool_vals[ci[i], :, 0:3].T, x[s:e]], axis=0)  # u[-3..n-1]
                for t in range(e - s):
                    assert np.array_equal(y[s + t], ext[t + k]), \
                        f"unit tap {k}: y[t] must equal u[t-3+k] (tap order / history order)"
    # zero taps: y = silu(b) everywhere
    b = (rng.standard_normal(C) * 2).astype(np.float32)
    y = o.fwd(x, np.zeros((C, 4), np.float32), b, cu_seqlens=cu, act="silu")
    ref = b.astype(np.float64) / (1 + np.exp(-b.astype(np.float64)))
    _close(bf.f64(y[: cu[-1]]), np.broadcast_to(ref, (int(cu[-1]), C)), 2.0 ** -8, 0, "silu(bias)")


def pin_segment_invariants(o, seed=14):
    rng = np.random.default_rng(seed)
    for q in range(6):
        case = wl.random_case(rng, C=7, nseq=5, max_len=9, pool_layout_name=["hist", "chan", None][q % 3],
                              with_hist=(q % 3 == 2), sentinel=True, act=["silu", "none"][q % 2])
        pool0 = case["pool"].copy() if case.get("pool") is not None else None
        y = _fwd(o, case)
        cu = case["cu_seqlens"]
        # each sequence alone gives the same bits (state resets at every boundary)
        for i in range(len(cu) - 1):
            s, e = int(cu[i]), int(cu[i + 1])
            sub = dict(case, x=case["x"][s:e], cu_seqlens=np.array([0, e - s], np.int32))
            for key in ("cache_indices", "has_initial_state", "has_history"):
                if case.get(key) is not None:
                    sub[key] = case[key][i:i + 1]
            if case.get("hist") is not None:
                sub["hist"] = case["hist"][i:i + 1].copy()
            ys = _fwd(o, sub, pool=None if pool0 is None else pool0.copy())
            assert np.array_equal(ys, y[s:e]), "per-sequence reset"
        # causality: changing x[t] changes y only at rows t..t+3 of the same sequence
        rows = int(cu[-1])
        if rows:
            t = int(rng.integers(0, rows))
            x2 = case["x"].copy()
            x2[t] ^= 0x0040  # flip a mantissa bit
            y2 = _fwd(o, dict(case, x=x2), pool=None if pool0 is None else pool0.copy())
            i = int(np.searchsorted(cu, t, side="right") - 1)
            allowed = np.zeros(y.shape[0], bool)
            allowed[t:min(t + 4, int(cu[i + 1]))] = True
            changed = (y2 != y).any(axis=1)
            assert not (changed & ~allowed).any(), "causality / segment leak"


def pin_pool_invariants(o, seed=15):
    rng = np.random.default_rng(seed)
    C = 6
    for layout in ("hist", "chan"):
        for L in (3, 5):
            # chunked prefill: splitting a sequence and carrying the state gives identical bits
            x = wl.normal_bf16(rng, (23, C))
            w = wl.uniform_f32(rng, (C, 4))
            b = (rng.standard_normal(C) * 0.1).astype(np.float32)
            vals = wl.normal_bf16(rng, (3, C, L))
            ci = np.array([1], np.int32)
            for hi0 in (0, 1):
                p_full = wl.pool_layout(vals.copy(), layout)
                y_full = o.fwd(x, w, b, cu_seqlens=np.array([0, 23], np.int32), pool=p_full,
                               cache_indices=ci, has_initial_state=np.array([hi0], np.uint8))
                for cut in (0, 1, 2, 3, 11, 22, 23):
                    p = wl.pool_layout(vals.copy(), layout)
                    y1 = o.fwd(x[:cut], w, b, cu_seqlens=np.array([0, cut], np.int32), pool=p,
                               cache_indices=ci, has_initial_state=np.array([hi0], np.uint8))
                    y2 = o.fwd(x[cut:], w, b, cu_seqlens=np.array([0, 23 - cut], np.int32), pool=p,
                               cache_indices=ci, has_initial_state=np.array([1 if cut else hi0], np.uint8))
                    assert np.array_equal(np.concatenate([y1, y2]), y_full), f"chunked prefill cut={cut}"
                    assert np.array_equal(p, p_full), "carried state"
                # positions >= 3 and other slots are untouched
                ref = vals.copy()
                ref[1, :, 0:3] = x[-3:].T
                assert np.array_equal(p_full, ref), "write-back positions / other slots"
            # has_initial_state false == zero history
            p_zero = wl.pool_layout(np.zeros((3, C, L), np.uint16), layout)
            p_rand = wl.pool_layout(vals.copy(), layout)
            cu = np.array([0, 5], np.int32)
            ya = o.fwd(x[:5], w, b, cu_seqlens=cu, pool=p_zero, cache_indices=ci,
                       has_initial_state=np.array([1], np.uint8))
            yb = o.fwd(x[:5], w, b, cu_seqlens=cu, pool=p_rand, cache_indices=ci,
                       has_initial_state=np.array([0], np.uint8))
            yc = o.fwd(x[:5], w, b, cu_seqlens=cu, pool=wl.pool_layout(vals.copy(), layout),
                       cache_indices=ci, has_initial_state=None)
            assert np.array_equal(ya, yb) and np.array_equal(ya, yc), "has_initial_state false = zeros"
            # empty sequences and the -1 sentinel leave the pool alone; sentinel rows are +0
            p = wl.pool_layout(vals.copy(), layout)
            cu = np.array([0, 0, 4, 4], np.int32)
            y = o.fwd(x[:6], w, b, cu_seqlens=cu, pool=p, cache_indices=np.array([0, -1, 2], np.int32),
                      has_initial_state=np.array([1, 1, 1], np.uint8))
            assert np.array_equal(p, vals), "empty / sentinel sequences must not touch the pool"
            assert (y[0:4] == 0).all() and (y[4:6] == FILL).all(), "sentinel zeros / padding untouched"


def pin_decode_equals_unit_prefill(o, seed=16):
    rng = np.random.default_rng(seed)
    for layout in ("hist", "chan"):
        for L in (3, 4, 7):
            N, C = 6, 9
            x = wl.normal_bf16(rng, (N, C))
            w = wl.uniform_f32(rng, (C, 4)) if L != 4 else wl.to_bf16_bits(wl.uniform_f32(rng, (C, 4)))
            b = (rng.standard_normal(C) * 0.1).astype(np.float32)
            vals = wl.normal_bf16(rng, (8, C, L))
            ci = rng.permutation(8)[:N].astype(np.int32)
            ci[2] = -1
            p1 = wl.pool_layout(vals.copy(), layout)
            p2 = wl.pool_layout(vals.copy(), layout)
            for act in ("silu", "none"):
                yd = o.state_update(x, w, b, pool=p1, cache_indices=ci, act=act)
                yf = o.fwd(x, w, b, cu_seqlens=np.arange(N + 1, dtype=np.int32), pool=p2,
                           cache_indices=ci, has_initial_state=np.ones(N, np.uint8), act=act)
                assert np.array_equal(yd, yf), "decode step == unit-length prefill"
                assert np.array_equal(p1, p2), "decode state shift == prefill write-back"


def pin_cp_fragments_forward(o, seed=17):
    rng = np.random.default_rng(seed)
    for C in (8, 13):
        S = 50
        x = wl.normal_bf16(rng, (S, C))
        w = wl.uniform_f32(rng, (C, 4))
        doc_cu = np.array([0, 20, 50], np.int32)            # two documents
        y_full = o.fwd(x, w, None, cu_seqlens=doc_cu)
        # split into fragments; a fragment continuing a document reads the previous 3 rows
        for cuts in ([5, 20, 21, 22, 40], [1, 2, 3, 20, 47], [19, 20, 23]):
            frag = np.array([0, *cuts, S], np.int32)
            nf = len(frag) - 1
            hist = np.zeros((nf, 3, C), np.uint16)
            hh = np.zeros(nf, np.uint8)
            for f in range(nf):
                s = int(frag[f])
                if s not in doc_cu:                          # continues a document
                    hh[f] = 1
                    d0 = int(doc_cu[np.searchsorted(doc_cu, s, side="right") - 1])
                    for j in range(3):
                        r = s - 3 + j
                        hist[f, j] = x[r] if r >= d0 else 0
            y = o.fwd(x, w, None, cu_seqlens=frag, hist=hist, has_history=hh)
            assert np.array_equal(y, y_full), f"fragments with history rows == unsplit ({cuts})"


# ------------------------------------------------------------------ backward
def pin_backward_autograd(o, seed=18, n=16):
    rng = np.random.default_rng(seed)
    for q in range(n):
        mode = "idx" if q % 4 == 3 else "cu"
        case = wl.random_case(rng, mode=mode, with_hist=(mode == "cu" and q % 2 == 0),
                              w_f32=bool(q % 3), act="silu" if q % 5 else "none", force_empty=bool(q % 2))
        dx, dw, db, dh = _bwd(o, case)
        gx, gw, gb, gH, covered = bf.grads_f64(case)
        _close(bf.f64(dx[covered]), gx[covered], 2.0 ** -8, 1e-5, "dx vs autograd")
        assert (dx[~covered] == FILL).all(), "dx rows past the last offset untouched"
        scale = 1.0 + np.abs(gw).max()
        _close(dw, gw, 1e-5, 1e-5 * scale, "dw vs autograd")
        if case.get("b") is not None:
            _close(db, gb, 1e-5, 1e-5 * (1 + np.abs(gb).max()), "db vs autograd")
        if dh is not None:
            hh = case.get("has_history")
            for i in range(dh.shape[0]):
                if hh is None or hh[i]:
                    _close(bf.f64(dh[i]), gH[i], 2.0 ** -8, 1e-5, "dhist vs autograd")
                else:
                    assert (dh[i] == FILL).all(), "dhist rows without history untouched"


def pin_backward_finite_differences(o, seed=19):
    rng = np.random.default_rng(seed)
    for q in range(3):
        case = wl.random_case(rng, C=3, nseq=3, max_len=6, w_f32=True, bias=False, act="silu",
                              with_hist=(q == 1))
        _, dw, _, _ = _bwd(o, case)
        w0 = case["w"].astype(np.float64)
        h = 1e-5
        for c in range(3):
            for k in range(4):
                wp, wm = w0.copy(), w0.copy()
                wp[c, k] += h
                wm[c, k] -= h
                fd = (bf.loss_f64(case, wp) - bf.loss_f64(case, wm)) / (2 * h)
                assert abs(dw[c, k] - fd) <= 1e-5 * (1 + abs(fd)), f"dw[{c},{k}] vs central difference"


def pin_backward_linear_closed_form(o, seed=20):
    """act = none: dz = dy, so dw_k = sum_t dy[t] u[t-3+k], db = sum dy, dx = correlation of dy
    with the taps (numpy.correlate), per segment."""
    rng = np.random.default_rng(seed)
    C = 4
    lengths = [6, 0, 1, 9, 3]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    rows = int(cu[-1])
    x = wl.normal_bf16(rng, (rows, C))
    dy = wl.normal_bf16(rng, (rows, C))
    w = wl.uniform_f32(rng, (C, 4))
    b = np.zeros(C, np.float32)
    hist = wl.normal_bf16(rng, (len(lengths), 3, C))
    dx, dw, db, dh = o.bwd(x, dy, w, b, cu_seqlens=cu, hist=hist, act="none")
    xf, gf, hf = bf.f64(x), bf.f64(dy), bf.f64(hist)
    ref_dw = np.zeros((C, 4))
    ref_dx = np.zeros((rows, C))
    for i in range(len(lengths)):
        s, e = int(cu[i]), int(cu[i + 1])
        n = e - s
        for c in range(C):
            for j in range(3):
                ref = sum(w[c, j - tau] * gf[s + tau, c] for tau in range(min(j, n - 1) + 1))
                assert abs(bf.f64(dh[i, j, c]) - ref) <= 2.0 ** -8 * abs(ref) + 1e-6, "dhist closed form"
            if n == 0:
                continue
            u = np.concatenate([hf[i, :, c], xf[s:e, c]])
            for k in range(4):
                ref_dw[c, k] += np.dot(gf[s:e, c], u[k:k + n])
            # dx[t] = sum_k w_k dy[t+3-k]  ==  correlation of dy with reversed taps
            full = np.correlate(np.concatenate([gf[s:e, c], np.zeros(3)]), w[c, ::-1].astype(np.float64), mode="valid")
            ref_dx[s:e, c] = full[:n]
    _close(dw, ref_dw, 1e-6, 1e-6, "dw closed form")
    _close(db, gf.sum(axis=0), 1e-6, 1e-6, "db closed form")
    _close(bf.f64(dx), ref_dx, 2.0 ** -8, 1e-6, "dx closed form")


def pin_cp_fragments_backward(o, seed=21):
    """Splitting a document into fragments: dx of the unsplit call on the last three rows of the
    preceding fragment = local dx + the next fragment's d(history); dw adds over fragments."""
    rng = np.random.default_rng(seed)
    C, S, cut = 5, 30, 13
    x = wl.normal_bf16(rng, (S, C))
    dy = wl.normal_bf16(rng, (S, C))
    w = wl.uniform_f32(rng, (C, 4))
    dx_u, dw_u, _, _ = o.bwd(x, dy, w, None, cu_seqlens=np.array([0, S], np.int32))
    hist = np.zeros((2, 3, C), np.uint16)
    hist[1] = x[cut - 3:cut]
    hh = np.array([0, 1], np.uint8)
    dx_f, dw_f, _, dh = o.bwd(x, dy, w, None, cu_seqlens=np.array([0, cut, S], np.int32), hist=hist,
                              has_history=hh)
    _close(bf.f64(dx_f[cut:]), bf.f64(dx_u[cut:]), 0, 0, "dx after the cut")
    a, h, ref = bf.f64(dx_f[cut - 3:cut]), bf.f64(dh[1]), bf.f64(dx_u[cut - 3:cut])
    # each of the three values was rounded to bf16 once: allow one rounding of each part
    bad = np.abs(a + h - ref) > 2.0 ** -8 * (np.abs(a) + np.abs(h) + np.abs(ref)) + 1e-30
    assert not bad.any(), "dx + dhist on the halo rows"
    assert np.abs(a).max() > 0 and np.abs(h).max() > 0
    _close(dw_f, dw_u, 1e-5, 1e-5, "dw over fragments")


def _spec_setup(rng, N, K, C, L, layout, w_bf16):
    x = wl.normal_bf16(rng, (N, K, C))
    w = wl.to_bf16_bits(wl.uniform_f32(rng, (C, 4))) if w_bf16 else wl.uniform_f32(rng, (C, 4))
    b = (rng.standard_normal(C) * 0.1).astype(np.float32)
    slots = N + 3
    pool = wl.pool_layout(wl.normal_bf16(rng, (slots, C, L)), layout)
    ci = rng.permutation(slots)[:N].astype(np.int32)
    if N > 1:
        ci[1] = -1
    acc = rng.integers(1, L - 1, size=N).astype(np.int32)  # 1 .. L-2
    return x, w, b, pool, ci, acc


def pin_spec_update_bruteforce(o, seed=22):
    """Speculative K-token update (reading of the causal_conv1d_fn Notes): the K outputs of each
    sequence are the dense Toeplitz forward of its K tokens with history rows read at pool
    positions a-1, a, a+1; afterwards positions 0..K+1 hold the last K+2 raw values of
    [history, tokens]; later positions, and every -1 slot, stay untouched; -1 outputs are +0."""
    rng = np.random.default_rng(seed)
    for layout in ("hist", "chan"):
        for K, L, act in ((1, 3, "silu"), (2, 4, "none"), (3, 8, "silu"), (5, 7, "silu"), (4, 6, "none")):
            N, C = 5, 7
            x, w, b, pool, ci, acc = _spec_setup(rng, N, K, C, L, layout, w_bf16=(K % 2 == 0))
            pool0 = pool.copy()
            hist = np.zeros((N, 3, C), np.uint16)
            for i in range(N):
                if ci[i] >= 0:
                    hist[i] = pool0[ci[i], :, acc[i] - 1:acc[i] + 2].T
            case = dict(x=x.reshape(N * K, C), w=w, b=b, cu_seqlens=np.arange(0, N * K + 1, K, dtype=np.int32),
                        hist=hist, has_history=np.ones(N, np.uint8), act=act)
            _, yref, _, _ = bf.forward_f64(case)
            yref = yref.numpy().reshape(N, K, C)
            y = o.spec_update(x, w, b, pool=pool, cache_indices=ci, accepted=acc, act=act)
            expect = pool0.copy()
            for i in range(N):
                if ci[i] < 0:
                    assert (y[i] == 0).all(), "a -1 slot gives +0"
                    continue
                _close(bf.f64(y[i]), yref[i], 2.0 ** -8, 1e-5, f"spec update y (K={K}, L={L})")
                ext = np.concatenate([hist[i], x[i]], axis=0)  # [K + 3, C] raw bits
                expect[ci[i], :, 0:K + 2] = ext[1:].T
            assert np.array_equal(pool, expect), f"spec update state write-back (K={K}, L={L}, {layout})"


def pin_spec_protocol_equals_prefill(o, seed=23):
    """Speculative decoding end to end: prefill, then steps of K tokens where each step reports how
    many tokens of the previous step were accepted (1 for the first step after the prefill).  Every
    step's outputs must equal the dense forward over the accepted stream so far followed by that
    step's tokens; K = 1 steps with accepted count 1 must equal the decode step bit for bit."""
    rng = np.random.default_rng(seed)
    N, C, K, L = 3, 6, 4, 6
    w = wl.uniform_f32(rng, (C, 4))
    b = (rng.standard_normal(C) * 0.1).astype(np.float32)
    for layout in ("hist", "chan"):
        lengths = [int(v) for v in rng.integers(1, 6, size=N)]
        cu = np.zeros(N + 1, dtype=np.int32)
        cu[1:] = np.cumsum(lengths)
        xp = wl.normal_bf16(rng, (int(cu[-1]), C))
        pool = wl.pool_layout(wl.normal_bf16(rng, (N + 2, C, L)), layout)
        ci = np.array([2, 0, 3], dtype=np.int32)
        o.fwd(xp, w, b, cu_seqlens=cu, pool=pool, cache_indices=ci, has_initial_state=np.zeros(N, np.uint8))
        streams = [xp[cu[i]:cu[i + 1]] for i in range(N)]  # accepted raw tokens of each sequence so far
        acc = np.ones(N, dtype=np.int32)
        prev = None
        for step in range(4):
            xs = wl.normal_bf16(rng, (N, K, C))
            if prev is not None:
                for i in range(N):
                    streams[i] = np.concatenate([streams[i], prev[i, :acc[i]]], axis=0)
            y = o.spec_update(xs, w, b, pool=pool, cache_indices=ci, accepted=acc)
            for i in range(N):
                full = np.concatenate([streams[i], xs[i]], axis=0)
                n = full.shape[0]
                case = dict(x=full, w=w, b=b, cu_seqlens=np.array([0, n], np.int32), act="silu")
                _, yref, _, _ = bf.forward_f64(case)
                _close(bf.f64(y[i]), yref.numpy()[n - K:], 2.0 ** -8, 1e-5, f"spec protocol step {step}")
            prev = xs
            acc = rng.integers(1, K + 1, size=N).astype(np.int32)
    # K = 1, accepted 1: the decode step
    x1 = wl.normal_bf16(rng, (4, 1, C))
    vals = wl.normal_bf16(rng, (6, C, 3))
    ci = np.array([4, -1, 0, 2], dtype=np.int32)
    p1, p2 = vals.copy(), vals.copy()
    y1 = o.spec_update(x1, w, b, pool=p1, cache_indices=ci)
    y2 = o.state_update(x1[:, 0], w, b, pool=p2, cache_indices=ci)
    assert np.array_equal(y1[:, 0], y2) and np.array_equal(p1, p2), "K = 1 spec update == decode step"


def pin_channels_first_conv1d(o, seed=24):
    """Channels-first [B, D, T] (the layout the Megatron determinism note contrasts with channel-
    last): each (b, d) row is one sequence with zero history.  Forward = torch's grouped conv1d with
    three zeros of left padding in float64, then SiLU; backward = its autograd."""
    import torch.nn.functional as F
    rng = np.random.default_rng(seed)
    for B, D, T, act, w_bf16, bias, W in ((2, 5, 9, "silu", False, True, 4), (3, 4, 1, "silu", True, False, 4),
                                          (1, 7, 13, "none", False, True, 4), (2, 3, 2, "silu", False, False, 4),
                                          (2, 6, 40, "silu", True, True, 4), (2, 5, 11, "silu", False, True, 2),
                                          (3, 4, 17, "none", True, True, 3), (2, 5, 23, "silu", False, True, 8),
                                          (2, 3, 6, "silu", True, True, 6)):
        x = wl.normal_bf16(rng, (B, D, T))
        dy = wl.normal_bf16(rng, (B, D, T))
        w = wl.to_bf16_bits(wl.uniform_f32(rng, (D, W))) if w_bf16 else wl.uniform_f32(rng, (D, W))
        b = (rng.standard_normal(D) * 0.1).astype(np.float32) if bias else None
        xt = torch.tensor(bf.f64(x), requires_grad=True)
        wt = torch.tensor(bf.taps_f64(w), requires_grad=True)
        bt = torch.tensor(b.astype(np.float64) if bias else np.zeros(D), requires_grad=True)
        z = F.conv1d(F.pad(xt, (W - 1, 0)), wt[:, None, :], bias=bt, groups=D)
        yt = z * torch.sigmoid(z) if act == "silu" else z
        y = o.fwd_cf(x, w, b, act=act)
        _close(bf.f64(y), yt.detach().numpy(), 2.0 ** -8, 1e-5, "channels-first y vs grouped conv1d")
        (yt * torch.tensor(bf.f64(dy))).sum().backward()
        dx, dw, db = o.bwd_cf(x, dy, w, b, act=act, want_db=True)
        _close(bf.f64(dx), xt.grad.numpy(), 2.0 ** -8, 1e-5, "channels-first dx vs autograd")
        gw = wt.grad.numpy()
        _close(dw, gw, 1e-5, 1e-5 * (1.0 + np.abs(gw).max()), "channels-first dw vs autograd")
        gb = bt.grad.numpy()
        _close(db, gb, 1e-5, 1e-5 * (1.0 + np.abs(gb).max()), "channels-first db vs autograd")


def _narrow(case, W, rng):
    """The same packed problem with W taps and W-1 history rows (no pool: the pool form is width four)."""
    C = case["x"].shape[1]
    out = dict(case)
    for key in ("pool", "cache_indices", "has_initial_state"):
        out.pop(key, None)
    w = wl.uniform_f32(rng, (C, W))
    out["w"] = w if case["w"].dtype == np.float32 else wl.to_bf16_bits(w)
    if case.get("hist") is not None:
        out["hist"] = wl.normal_bf16(rng, (case["hist"].shape[0], W - 1, C))
    return out


def pin_width_bruteforce(o, seed=25):
    """Widths 2, 3 and 5..8 (Megatron-Core causal_conv1d_cp, Parameters weight [D, W]): forward
    against the dense Toeplitz form with W taps and W-1 history rows, backward against its
    autograd."""
    rng = np.random.default_rng(seed)
    for W in (2, 3, 5, 6, 7, 8):
        for q in range(8 if W < 4 else 5):
            mode = "idx" if q % 4 == 3 else "cu"
            base = wl.random_case(rng, mode=mode, with_hist=(mode == "cu" and q % 2 == 0), w_f32=bool(q % 3),
                                  act="silu" if q % 5 else "none", force_empty=bool(q % 2))
            case = _narrow(base, W, rng)
            _, yref, covered, _ = bf.forward_f64(case)
            y = _fwd(o, case)
            _close(bf.f64(y)[covered], yref.numpy()[covered], 2.0 ** -8, 1e-5, f"W={W} y vs dense Toeplitz")
            assert (y[~covered] == FILL).all(), "rows past the last offset untouched"
            dx, dw, db, dh = _bwd(o, case)
            gx, gw, gb, gH, covered = bf.grads_f64(case)
            assert dw.shape == (case["x"].shape[1], W)
            _close(bf.f64(dx[covered]), gx[covered], 2.0 ** -8, 1e-5, f"W={W} dx vs autograd")
            _close(dw, gw, 1e-5, 1e-5 * (1.0 + np.abs(gw).max()), f"W={W} dw vs autograd")
            if case.get("b") is not None:
                _close(db, gb, 1e-5, 1e-5 * (1 + np.abs(gb).max()), f"W={W} db vs autograd")
            if dh is not None:
                hh = case.get("has_history")
                for i in range(dh.shape[0]):
                    if hh is None or hh[i]:
                        _close(bf.f64(dh[i]), gH[i], 2.0 ** -8, 1e-5, f"W={W} dhist vs autograd")


def pin_width_closed_forms(o, seed=26):
    """Width 2 with taps (0, 1) passes the current value through (z = b + x); with taps (1, 0) it
    reads the previous value, which at a sequence start is the last history row."""
    rng = np.random.default_rng(seed)
    C, n = 5, 7
    x = wl.normal_bf16(rng, (n, C))
    hist = wl.normal_bf16(rng, (1, 1, C))
    cu = np.array([0, n], np.int32)
    ident = np.tile(np.array([0.0, 1.0], np.float32), (C, 1))
    y = o.fwd(x, ident, None, cu_seqlens=cu, hist=hist, act="none")
    assert np.array_equal(y, x), "width-2 identity tap"
    prev = np.tile(np.array([1.0, 0.0], np.float32), (C, 1))
    y = o.fwd(x, prev, None, cu_seqlens=cu, hist=hist, act="none")
    assert np.array_equal(y[0], hist[0, 0]) and np.array_equal(y[1:], x[:-1]), "width-2 previous-value tap"
    with_pool_rejected = False
    try:
        o.fwd(x, ident, None, cu_seqlens=cu, pool=np.zeros((2, C, 4), np.uint16),
              cache_indices=np.array([0], np.int32), act="none")
    except Exception:
        with_pool_rejected = True
    assert with_pool_rejected, "the pool form is width four only"


def pin_wide_closed_forms(o, seed=27):
    """Width 8: unit taps e_k read the extended sequence k - 7 rows back, bit for bit, so every tap
    and all seven history rows land where the order (oldest history row first, tap W-1 on the
    current row) says; with tap k = 1 only, a sequence of n rows reads history rows k .. 6 then
    its own first rows.  Per-token IDs reset to zero history at every boundary."""
    rng = np.random.default_rng(seed)
    C, n, W = 3, 11, 8
    x = wl.normal_bf16(rng, (n, C))
    hist = wl.normal_bf16(rng, (1, W - 1, C))
    cu = np.array([0, n], np.int32)
    u = np.concatenate([hist[0], x], axis=0)  # extended sequence, oldest first
    for k in range(W):
        e = np.zeros((C, W), np.float32)
        e[:, k] = 1.0
        y = o.fwd(x, e, None, cu_seqlens=cu, hist=hist, act="none")
        assert np.array_equal(y, u[k:k + n]), f"width-8 unit tap {k}"
    # per-token IDs: two documents, zero history at each start
    ids = np.array([0] * 5 + [1] * 6, np.int32)
    e = np.zeros((C, W), np.float32)
    e[:, 2] = 1.0  # reads five rows back
    y = o.fwd(x, e, None, seq_idx=ids, seqlen=n, act="none")
    want = np.zeros_like(x)
    want[5 + 5:] = x[5:6]
    assert np.array_equal(y, want), "width-8 tap reading five rows back, reset at a document start"
    rejected = False
    try:
        o.fwd(x, np.zeros((C, 9), np.float32), None, cu_seqlens=cu, act="none")
    except Exception:
        rejected = True
    assert rejected, "widths above 8 are rejected"


def pin_batch_rows_bruteforce(o, seed=28):
    """The batch-row form (no offsets, no IDs: every batch row of `seqlen` rows is one sequence)
    with a slot pool in both layouts (with -1 sentinels and mixed has_initial_state) and with
    caller history rows: forward against the dense Toeplitz form and the pool write-back rule,
    backward against its autograd (causal_conv1d_cp, Parameters x [B, T, D]; causal_conv1d_fn,
    Parameters conv_state and cache_indices)."""
    rng = np.random.default_rng(seed)
    for q in range(12):
        layout = ["hist", "chan", None][q % 3]
        case = wl.random_case(rng, mode="batch", nseq=int(rng.integers(1, 5)), max_len=int(rng.choice([1, 2, 3, 9])),
                              pool_layout_name=layout, with_hist=(layout is None), L=int(rng.choice([3, 4, 6])),
                              w_f32=bool(q % 2), act="silu" if q % 5 else "none", sentinel=(q % 2 == 0))
        pool0 = case["pool"].copy() if case.get("pool") is not None else None
        _, yref, covered, sent = bf.forward_f64(case)
        y = _fwd(o, case)
        live = covered & ~sent
        _close(bf.f64(y)[live], yref.numpy()[live], 2.0 ** -8, 1e-5, "batch rows: y vs dense Toeplitz")
        assert (y[sent] == 0).all(), "batch rows: sentinel rows must be +0"
        if pool0 is not None:
            assert np.array_equal(case["pool"], bf.pool_after(dict(case, pool=pool0))), "batch rows: pool write-back"
        else:
            dx, dw, db, dh = _bwd(o, case)
            gx, gw, gb, gH, covered = bf.grads_f64(case)
            _close(bf.f64(dx), gx, 2.0 ** -8, 1e-5, "batch rows: dx vs autograd")
            _close(dw, gw, 1e-5, 1e-5 * (1.0 + np.abs(gw).max()), "batch rows: dw vs autograd")
            hh = case.get("has_history")
            for i in range(dh.shape[0]):
                if hh[i]:
                    _close(bf.f64(dh[i]), gH[i], 2.0 ** -8, 1e-5, "batch rows: dhist vs autograd")
                else:
                    assert (dh[i] == FILL).all(), "batch rows: dhist of sequences without history untouched"


def pin_dtail_autograd(o, seed=29):
    """The next shard's gradient for the last W-1 values of the last sequence's extended sequence
    (cake_causal_conv1d_kcp, Returns; the history exchange of causal_conv1d_cp is differentiable):
    dx and d(history) against autograd of sum(dy * y) + <dtail, those values>, for last sequences
    longer and shorter than the history (the short ones pass part of dtail on to their own
    history rows), empty last sequences, batch rows and per-token IDs, widths 2, 4 and 8."""
    rng = np.random.default_rng(seed)
    for q in range(18):
        W = (4, 2, 8)[q % 3]
        mode = ("cu", "batch", "idx")[(q // 3) % 3]
        base = wl.random_case(rng, mode=mode, nseq=int(rng.integers(1, 5)), max_len=int(rng.choice([1, 2, 5, 12])),
                              with_hist=(mode != "idx"), w_f32=bool(q % 2), act="silu" if q % 4 else "none")
        if mode == "cu" and q % 2:  # a short or empty last fragment
            cu = base["cu_seqlens"].copy()
            cu[-1] = cu[-2] + min(int(rng.integers(0, 3)), int(cu[-1] - cu[-2]))
            base["cu_seqlens"] = cu
            base["x"] = base["x"][: cu[-1] + 1]
            base["dy"] = base["dy"][: cu[-1] + 1]
        case = _narrow(base, W, rng) if W != 4 else base
        C = case["x"].shape[1]
        dtail = wl.normal_bf16(rng, (W - 1, C))
        dx, _, _, dh = o.bwd(case["x"], case["dy"], case["w"], case.get("b"), cu_seqlens=case.get("cu_seqlens"),
                             seq_idx=case.get("seq_idx"), seqlen=case.get("seqlen"), hist=case.get("hist"),
                             has_history=case.get("has_history"), act=case.get("act", "silu"), dtail=dtail)
        gx, gH, covered = bf.grads_f64_with_tail(case, dtail)
        _close(bf.f64(dx[covered]), gx[covered], 2.0 ** -8, 1e-5, f"W={W} {mode}: dx with d(tail) vs autograd")
        assert (dx[~covered] == FILL).all(), "rows past the last offset untouched"
        if dh is not None:
            hh = case.get("has_history")
            for i in range(dh.shape[0]):
                if hh is None or hh[i]:
                    _close(bf.f64(dh[i]), gH[i], 2.0 ** -8, 1e-5, f"W={W} {mode}: dhist with d(tail) vs autograd")


def pin_dtail_shard_split(o, seed=30):
    """Two shards of one packed batch on one host: shard B's d(history) for its first fragment,
    passed back as shard A's d(tail), gives A's dx (and, when A's last fragment is shorter than the
    history, A's own d(history)) equal to the unsplit dx up to one bf16 rounding of each part; the
    dweight contributions of the shards add up to the unsplit one."""
    rng = np.random.default_rng(seed)
    C = 6
    for cut_in_frag, S in ((7, 40), (1, 30), (2, 31), (0, 25)):
        x, dy = wl.normal_bf16(rng, (S, C)), wl.normal_bf16(rng, (S, C))
        w = wl.uniform_f32(rng, (C, 4))
        doc_cu = np.array([0, 9, S], np.int32)      # two documents; the shard cut lies in the second
        cut = 9 + cut_in_frag if cut_in_frag else 12
        dx_u, dw_u, _, _ = o.bwd(x, dy, w, None, cu_seqlens=doc_cu)
        # shard A: rows [0, cut) = fragments [0, 9), [9, cut); shard B: rows [cut, S), continuing
        xa, dya = x[:cut], dy[:cut]
        ha = np.zeros((2, 3, C), np.uint16)
        dx_a0, _, _, _ = o.bwd(xa, dya, w, None, cu_seqlens=np.array([0, 9, cut], np.int32), hist=ha,
                               has_history=np.array([0, 0], np.uint8))
        hb = np.zeros((1, 3, C), np.uint16)
        for j in range(3):
            r = cut - 3 + j
            hb[0, j] = x[r] if r >= 9 else 0
        dx_b, dw_b, _, dh_b = o.bwd(x[cut:], dy[cut:], w, None, cu_seqlens=np.array([0, S - cut], np.int32), hist=hb,
                                    has_history=np.array([1], np.uint8))
        dx_a, dw_a, _, _ = o.bwd(xa, dya, w, None, cu_seqlens=np.array([0, 9, cut], np.int32), hist=ha,
                                 has_history=np.array([0, 0], np.uint8), dtail=dh_b[0])
        _close(bf.f64(dx_b), bf.f64(dx_u[cut:]), 0, 0, "shard B's dx equals the unsplit dx")
        ref, part, tail = bf.f64(dx_u[:cut]), bf.f64(dx_a0), np.zeros((cut, C))
        for j in range(3):
            if cut - 3 + j >= 9:
                tail[cut - 3 + j] = bf.f64(dh_b[0, j])
        assert np.array_equal(dx_a[:cut - 3], dx_a0[:cut - 3]), "d(tail) reaches only the last three rows"
        bad = np.abs(bf.f64(dx_a) - ref) > 2.0 ** -8 * (np.abs(part) + np.abs(tail) + np.abs(ref)) + 1e-30
        assert not bad.any(), f"shard A's dx with d(tail) = unsplit dx (cut {cut})"
        if tail.any():
            assert not np.array_equal(dx_a, dx_a0), "d(tail) must change dx"
        _close(o.combine(np.stack([dw_a, dw_b])), dw_u, 1e-5, 1e-5, "shard dweights add up")


def pin_combine_closed_forms(o):
    """Shard-ordered FP32 combine (assert_causal_conv1d_deterministic's fixed order): values whose
    FP32 sum depends on the order pin ascending shard order; one shard comes back bit for bit (also
    -0.0); zero shards give zeros; random sums lie within the FP32 bound of the exact sum."""
    big = np.float32(1e8)
    parts = np.array([[big, big, 1.0], [1.0, -big, big], [-big, 1.0, -big]], np.float32)[:, None, :]
    out = o.combine(parts)
    # (1e8 + 1) - 1e8 = 0 in FP32; (1e8 - 1e8) + 1 = 1; (1 + 1e8) - 1e8 = 0
    assert np.array_equal(out[0], np.array([0.0, 1.0, 0.0], np.float32)), out
    one = np.array([[[-0.0, 3.5e-40, -7.25]]], np.float32)
    assert np.array_equal(o.combine(one).view(np.uint32), one[0].view(np.uint32)), "one shard is the identity"
    assert np.array_equal(o.combine(np.zeros((0, 2, 3), np.float32)), np.zeros((2, 3), np.float32))
    rng = np.random.default_rng(31)
    p = rng.standard_normal((9, 5, 7)).astype(np.float32)
    exact = p.astype(np.float64).sum(axis=0)
    bound = 8 * 2.0 ** -24 * np.abs(p).astype(np.float64).sum(axis=0)
    assert (np.abs(o.combine(p) - exact) <= bound).all(), "within the FP32 bound of the exact sum"


ALL_PINS = [pin_rounding, pin_forward_bruteforce, pin_forward_conv1d_library, pin_forward_closed_forms,
            pin_segment_invariants, pin_pool_invariants, pin_decode_equals_unit_prefill,
            pin_cp_fragments_forward, pin_backward_autograd, pin_backward_finite_differences,
            pin_backward_linear_closed_form, pin_cp_fragments_backward, pin_spec_update_bruteforce,
            pin_spec_protocol_equals_prefill, pin_channels_first_conv1d,
            pin_width_bruteforce, pin_width_closed_forms, pin_wide_closed_forms, pin_batch_rows_bruteforce,
            pin_dtail_autograd, pin_dtail_shard_split, pin_combine_closed_forms]


def golden_dyadic():
    import json
    import os
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "exact_dyadic.json")) as f:
        return json.load(f)


def pin_golden_dyadic(o):
    """Hand-derived exact example (tests/golden/exact_dyadic.json): every value bit-exact."""
    g = golden_dyadic()
    bits = lambda v: wl.to_bf16_bits(np.asarray(v, np.float32))
    x = bits(g["x"])[:, None]
    w = np.asarray(g["w"], np.float32)[None, :]
    b = np.asarray([g["b"]], np.float32)
    hist = bits(g["history"]).reshape(1, 3, 1)
    cu = np.array([0, 5], np.int32)
    y = o.fwd(x, w, b, cu_seqlens=cu, hist=hist, act="none")
    assert np.array_equal(y[:, 0], bits(g["y"])), "golden y"
    dx, dw, db, dh = o.bwd(x, bits(g["dy"])[:, None], w, b, cu_seqlens=cu, hist=hist, act="none")
    assert np.array_equal(dx[:, 0], bits(g["dx"])), "golden dx"
    assert np.array_equal(dw[0], np.asarray(g["dw"], np.float32)), "golden dw"
    assert db[0] == np.float32(g["db"]), "golden db"
    assert np.array_equal(dh[0, :, 0], bits(g["dhist"])), "golden dhist"
    pc = g["pool_case"]
    for layout in ("hist", "chan"):
        pool = wl.pool_layout(bits(pc["history"] + [7.0]).reshape(1, 1, 4), layout)
        o.fwd(bits(pc["x"])[:, None], w, b, cu_seqlens=np.array([0, 2], np.int32), pool=pool,
              cache_indices=np.array([0], np.int32), has_initial_state=np.array([1], np.uint8), act="none")
        assert np.array_equal(pool[0, 0, :3], bits(pc["state_after"])) and pool[0, 0, 3] == bits([7.0])[0]


ALL_PINS.append(pin_golden_dyadic)
