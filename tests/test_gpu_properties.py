"""GPU properties beyond element-wise parity: determinism, decode = unit prefill, chunked prefill,
the context-parallel split, HIP-graph capture and replay with edited metadata, strided rows, arrays
beyond 2^31 elements (forward, backward, slot pool, channels-first), and identities between code
paths that must give the same bits: the three sequence forms, pool state against history rows,
bf16 against FP32 taps.  Everything goes through the C ABI (the torch binding only marshals)."""
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


def _width8(case, seed):
    """The same workload with taps [C, 8] and seven history rows per fragment."""
    rng = np.random.default_rng(seed)
    out = dict(case)
    C = case["x"].shape[1]
    out["w"] = wl.uniform_f32(rng, (C, 8))
    if case.get("hist") is not None:
        out["hist"] = wl.normal_bf16(rng, (case["hist"].shape[0], 7, C))
    return out


def test_dweight_bitwise_reproducible():
    """Ten backward runs, fresh and garbage-filled workspaces, another stream: identical dw/db bits
    (filter width 4, and width 8 with its nine-row partials)."""
    say("determinism: per-token-ID training and context-parallel share, widths 4 and 8")
    for case in (wl.train_seq_ids(), wl.cp_share(), _width8(wl.train_seq_ids(), 90), _width8(wl.cp_share(), 91)):
        x, dy = gh.dev_bits(case["x"]), gh.dev_bits(case["dy"])
        w, b = gh.dev_taps(case["w"]), gh.dev_taps(case.get("b"))
        kw = dict(cu_seqlens=gh.dev_i32(case.get("cu_seqlens")), seq_idx=gh.dev_i32(case.get("seq_idx")),
                  seqlen=case.get("seqlen"), history=gh.dev_bits(case["hist"]) if case.get("hist") is not None else None,
                  has_history=gh.dev_u8(case.get("has_history")), want_dbias=True)
        need = cc.conv1d_bwd_workspace_bytes(*case["x"].shape)
        ref = None
        side = torch.cuda.Stream()
        for run in range(10):
            ws = torch.empty(need + 4096, dtype=torch.uint8, device="cuda")
            ws.fill_(run * 37 % 256)
            ws = ws[256 * (run % 4):]  # different, still aligned, addresses
            stream = side if run % 2 else None
            with torch.cuda.stream(side if run % 2 else torch.cuda.current_stream()):
                _, dw, db, _ = cc.conv1d_bwd(x, dy, w, b, workspace=ws, stream=stream, **kw)
            torch.cuda.synchronize()
            bits = (dw.view(torch.int32).cpu().numpy(), db.view(torch.int32).cpu().numpy())
            if ref is None:
                ref = bits
            else:
                assert np.array_equal(bits[0], ref[0]) and np.array_equal(bits[1], ref[1]), f"run {run} differs"


def test_forward_recompute_bitwise_identical():
    say("forward recompute")
    case = wl.cp_share()
    y1, _ = gh.gpu_fwd(case)
    y2, _ = gh.gpu_fwd(case)
    assert np.array_equal(y1, y2)


@pytest.mark.parametrize("layout", ["hist", "chan"])
def test_decode_matches_oracle_and_unit_prefill(oracle, layout):
    say(f"decode {layout}")
    rng = np.random.default_rng(31)
    for C, N, L in ((5632, 64, 4), (13, 9, 3), (1024, 7, 6)):
        x = wl.normal_bf16(rng, (N, C))
        w = wl.uniform_f32(rng, (C, 4))
        b = (rng.standard_normal(C) * 0.1).astype(np.float32)
        vals = wl.normal_bf16(rng, (N + 5, C, L))
        ci = rng.permutation(N + 5)[:N].astype(np.int32)
        ci[1] = -1
        pool = gh.dev_pool(wl.pool_layout(vals.copy(), layout))
        y = cc.conv1d_state_update(gh.dev_bits(x), gh.dev_taps(w), gh.dev_taps(b), conv_state=pool,
                                   cache_indices=gh.dev_i32(ci))
        torch.cuda.synchronize()
        ref_pool = wl.pool_layout(vals.copy(), layout)
        yr = oracle.state_update(x, w, b, pool=ref_pool, cache_indices=ci)
        gh.assert_bf16_close(gh.host_bits(y), yr, "decode y")
        assert np.array_equal(gh.host_pool(pool), ref_pool), "decode state shift"
        # the same step as a prefill of unit-length sequences: identical bits
        case = dict(x=x, w=w, b=b, cu_seqlens=np.arange(N + 1, dtype=np.int32), pool=wl.pool_layout(vals.copy(), layout),
                    cache_indices=ci, has_initial_state=np.ones(N, np.uint8), act="silu")
        yf, pf = gh.gpu_fwd(case)
        assert np.array_equal(yf, gh.host_bits(y)) and np.array_equal(pf, ref_pool)


def test_chunked_prefill_equals_one_call():
    say("chunked prefill")
    rng = np.random.default_rng(32)
    C, n = 1536, 600
    x = wl.normal_bf16(rng, (n, C))
    w = wl.uniform_f32(rng, (C, 4))
    b = (rng.standard_normal(C) * 0.1).astype(np.float32)
    vals = wl.normal_bf16(rng, (2, C, 4))
    ci, hi = np.array([1], np.int32), np.array([1], np.uint8)
    full = dict(x=x, w=w, b=b, cu_seqlens=np.array([0, n], np.int32), pool=vals.copy(), cache_indices=ci,
                has_initial_state=hi, act="silu")
    y_full, p_full = gh.gpu_fwd(full)
    for cut in (1, 2, 3, 127, 128, 129, 300):
        pool = gh.dev_pool(vals.copy())
        ys = []
        for lo, hi_ in ((0, cut), (cut, n)):
            y = cc.conv1d_fwd(gh.dev_bits(x[lo:hi_]), gh.dev_taps(w), gh.dev_taps(b),
                              cu_seqlens=gh.dev_i32(np.array([0, hi_ - lo])), conv_state=pool,
                              cache_indices=gh.dev_i32(ci), has_initial_state=gh.dev_u8(hi))
            ys.append(gh.host_bits(y))
        torch.cuda.synchronize()
        assert np.array_equal(np.concatenate(ys), y_full), f"cut {cut}"
        assert np.array_equal(gh.host_pool(pool), p_full)


def test_context_parallel_split_on_gpu():
    """Fragments with the previous fragment's last three rows as history = the unsplit batch (y
    bit-exact); dx of the unsplit call on those rows = local dx + d(history); dw adds up."""
    say("cp split")
    rng = np.random.default_rng(33)
    C, S, cut = 2048, 1000, 437
    x, dy = wl.normal_bf16(rng, (S, C)), wl.normal_bf16(rng, (S, C))
    w = wl.uniform_f32(rng, (C, 4))
    whole = dict(x=x, w=w, b=None, cu_seqlens=np.array([0, S], np.int32), dy=dy, act="silu")
    y_u, _ = gh.gpu_fwd(whole)
    dx_u, dw_u, _, _ = gh.gpu_bwd(whole)
    hist = np.zeros((2, 3, C), np.uint16)
    hist[1] = x[cut - 3:cut]
    frag = dict(x=x, w=w, b=None, cu_seqlens=np.array([0, cut, S], np.int32), hist=hist,
                has_history=np.array([0, 1], np.uint8), dy=dy, act="silu")
    y_f, _ = gh.gpu_fwd(frag)
    assert np.array_equal(y_f, y_u)
    dx_f, dw_f, _, dh = gh.gpu_bwd(frag)
    assert np.array_equal(dx_f[cut:], dx_u[cut:])
    a, h, ref = gh.f32(dx_f[cut - 3:cut]), gh.f32(dh[1]), gh.f32(dx_u[cut - 3:cut])
    assert np.all(np.abs(a + h - ref) <= 2.0 ** -8 * (np.abs(a) + np.abs(h) + np.abs(ref)) + 1e-6)
    gh.assert_w_close(dw_f, dw_u, "dw over fragments")


def test_hip_graph_replay_with_edited_metadata(oracle):
    """Capture forward + backward once; between replays rewrite cu_seqlens / cache_indices /
    has_initial_state / has_history in place (same capacities) and check every replay."""
    say("graph capture")
    rng = np.random.default_rng(34)
    C, rows, N = 1024, 700, 5
    x, dy = wl.normal_bf16(rng, (rows, C)), wl.normal_bf16(rng, (rows, C))
    w = wl.uniform_f32(rng, (C, 4))
    b = (rng.standard_normal(C) * 0.1).astype(np.float32)
    vals = wl.normal_bf16(rng, (8, C, 4))
    hist = wl.normal_bf16(rng, (N, 3, C))
    dev = dict(x=gh.dev_bits(x), dy=gh.dev_bits(dy), w=gh.dev_taps(w), b=gh.dev_taps(b), hist=gh.dev_bits(hist),
               cu=torch.zeros(N + 1, dtype=torch.int32, device="cuda"), ci=torch.zeros(N, dtype=torch.int32, device="cuda"),
               hi=torch.zeros(N, dtype=torch.uint8, device="cuda"), hh=torch.zeros(N, dtype=torch.uint8, device="cuda"),
               pool=gh.dev_pool(vals.copy()), y=torch.empty(rows, C, dtype=torch.bfloat16, device="cuda"),
               y2=torch.empty(rows, C, dtype=torch.bfloat16, device="cuda"),
               dx=torch.empty(rows, C, dtype=torch.bfloat16, device="cuda"),
               dw=torch.empty(C, 4, dtype=torch.float32, device="cuda"),
               db=torch.empty(C, dtype=torch.float32, device="cuda"),
               dh=torch.empty(N, 3, C, dtype=torch.bfloat16, device="cuda"),
               ws=torch.empty(cc.conv1d_bwd_workspace_bytes(rows, C), dtype=torch.uint8, device="cuda"))

    def metadata():
        lengths = rng.integers(0, 200, size=N)
        lengths = np.minimum(lengths, rows // N)
        cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
        ci = rng.permutation(8)[:N].astype(np.int32)
        ci[int(rng.integers(0, N))] = -1
        return cu, ci, (rng.random(N) < 0.5).astype(np.uint8), (rng.random(N) < 0.5).astype(np.uint8)

    def run():
        cc.conv1d_fwd(dev["x"], dev["w"], dev["b"], cu_seqlens=dev["cu"], conv_state=dev["pool"],
                      cache_indices=dev["ci"], has_initial_state=dev["hi"], out=dev["y"])
        cc.conv1d_fwd(dev["x"], dev["w"], dev["b"], cu_seqlens=dev["cu"], history=dev["hist"],
                      has_history=dev["hh"], out=dev["y2"])
        cc.conv1d_bwd(dev["x"], dev["dy"], dev["w"], dev["b"], cu_seqlens=dev["cu"], history=dev["hist"],
                      has_history=dev["hh"], dx=dev["dx"], dweight=dev["dw"], dbias=dev["db"], dhistory=dev["dh"],
                      workspace=dev["ws"])

    meta = metadata()
    for t, m in zip((dev["cu"], dev["ci"], dev["hi"], dev["hh"]), meta):
        t.copy_(torch.from_numpy(m))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()  # warm up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    torch.cuda.synchronize()
    for replay in range(4):
        cu, ci, hi, hh = metadata()
        for t, m in zip((dev["cu"], dev["ci"], dev["hi"], dev["hh"]), (cu, ci, hi, hh)):
            t.copy_(torch.from_numpy(m))
        pool_before = gh.host_pool(dev["pool"])
        dev["y"].fill_(0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ref_pool = pool_before.copy()
        yr = oracle.fwd(x, w, b, cu_seqlens=cu, pool=ref_pool, cache_indices=ci, has_initial_state=hi, fill=0)
        yg = gh.host_bits(dev["y"])
        gh.assert_bf16_close(yg[: cu[-1]], yr[: cu[-1]], f"replay {replay}: y")
        assert np.array_equal(gh.host_pool(dev["pool"]), ref_pool), f"replay {replay}: pool"
        yr2 = oracle.fwd(x, w, b, cu_seqlens=cu, hist=hist, has_history=hh)
        gh.assert_bf16_close(gh.host_bits(dev["y2"])[: cu[-1]], yr2[: cu[-1]], f"replay {replay}: y (history)")
        dxr, dwr, dbr, dhr = oracle.bwd(x, dy, w, b, cu_seqlens=cu, hist=hist, has_history=hh)
        gh.assert_bf16_close(gh.host_bits(dev["dx"])[: cu[-1]], dxr[: cu[-1]], f"replay {replay}: dx")
        gh.assert_w_close(dev["dw"].cpu().numpy(), dwr, f"replay {replay}: dw")
        gh.assert_w_close(dev["db"].cpu().numpy(), dbr, f"replay {replay}: db")
        dhg = gh.host_bits(dev["dh"]).reshape(N, 3, C)
        for i in np.flatnonzero(hh):
            gh.assert_bf16_close(dhg[i], dhr[i], f"replay {replay}: dhist")


def test_strided_rows_and_scalar_path(oracle):
    """Row strides larger than C (a channel slice of a wider tensor) and misaligned rows."""
    say("strided rows")
    rng = np.random.default_rng(35)
    for C, ld, off in ((512, 640, 0), (512, 600, 8), (24, 27, 1), (1000, 1000, 3)):
        rows = 333
        full = wl.normal_bf16(rng, (rows, ld + off))
        xs = full[:, off:off + C]
        cu = np.array([0, 100, 101, 333], np.int32)
        w = wl.uniform_f32(rng, (C, 4))
        hist = wl.normal_bf16(rng, (3, 3, C))
        xdev = gh.dev_bits(full)[:, off:off + C]
        out_full = torch.empty(rows, ld + 5, dtype=torch.bfloat16, device="cuda")
        out = out_full[:, 5:5 + C]
        y = cc.conv1d_fwd(xdev, gh.dev_taps(w), None, cu_seqlens=gh.dev_i32(cu), history=gh.dev_bits(hist), out=out)
        torch.cuda.synchronize()
        yr = oracle.fwd(np.ascontiguousarray(xs), w, None, cu_seqlens=cu, hist=hist)
        gh.assert_bf16_close(gh.host_bits(y), yr, f"strided C={C} ld={ld} off={off}")


def test_64bit_row_offsets(oracle):
    """rows * C beyond 2^31 elements: row offsets must not wrap.  Checked on sampled channels."""
    say("64-bit offsets")
    rng = np.random.default_rng(36)
    rows, C = 4096 * 33, 16384  # 2.2e9 elements, 4.4 GB per tensor
    x = torch.empty(rows, C, dtype=torch.bfloat16, device="cuda")
    x.normal_(generator=torch.Generator(device="cuda").manual_seed(7))
    cu = np.array([0, 5, 70000, rows - 3, rows], np.int32)
    w = wl.uniform_f32(rng, (C, 4))
    y = cc.conv1d_fwd(x, gh.dev_taps(w), None, cu_seqlens=gh.dev_i32(cu))
    torch.cuda.synchronize()
    cols = np.array([0, 1, 777, 8191, 16383])
    tail = slice(rows - 70000, rows)
    xs = gh.host_bits(x[:, cols].contiguous())
    ys = gh.host_bits(y[:, cols].contiguous())
    yr = oracle.fwd(xs, np.ascontiguousarray(w[cols]), None, cu_seqlens=cu)
    gh.assert_bf16_close(ys[tail], yr[tail], "far rows")
    gh.assert_bf16_close(ys[:4096], yr[:4096], "near rows")
    del x, y
    torch.cuda.empty_cache()


def _big_normal(rows, C, seed):
    t = torch.empty(rows, C, dtype=torch.bfloat16, device="cuda")
    t.normal_(generator=torch.Generator(device="cuda").manual_seed(seed))
    return t


# Channels are independent in a depthwise filter, so a handful of channels of a huge array is an
# exact small problem for the oracle: every row of the sampled channels is checked.  At 16384
# channels row 131072 is element 2^31 and byte 2^32; sequences start on both sides of it.
_BIG_ROWS, _BIG_C = 4096 * 33, 16384
_BIG_COLS = np.array([0, 1, 777, 8191, 16383])


def test_64bit_row_offsets_backward_with_history(oracle):
    """The backward with history rows, dbias and d(tail) over rows * C beyond 2^31 elements
    (4.4 GB per tensor): dx on every row, dweight, dbias and d(history) of sampled channels
    against the oracle; and the forward with history rows over the same array."""
    say("64-bit offsets: forward and backward with history rows and d(tail)")
    rng = np.random.default_rng(37)
    rows, C, cols = _BIG_ROWS, _BIG_C, _BIG_COLS
    x, dy = _big_normal(rows, C, 8), _big_normal(rows, C, 9)
    cu = np.array([0, 5, 70000, 131070, 131073, rows - 3, rows], np.int32)
    nseq = len(cu) - 1
    hh = np.array([1, 0, 1, 1, 1, 0], np.uint8)
    hist = wl.normal_bf16(rng, (nseq, 3, C))
    w = wl.uniform_f32(rng, (C, 4))
    b = (rng.standard_normal(C) * 0.1).astype(np.float32)
    dtail = wl.normal_bf16(rng, (3, C))
    kw = dict(cu_seqlens=gh.dev_i32(cu), history=gh.dev_bits(hist), has_history=gh.dev_u8(hh))
    y = cc.conv1d_fwd(x, gh.dev_taps(w), gh.dev_taps(b), **kw)
    dh = gh.dev_bits(np.full((nseq, 3, C), wl.OUT_FILL, np.uint16))  # rows left untouched keep the marker
    dx, dw, db, dh = cc.conv1d_bwd(x, dy, gh.dev_taps(w), gh.dev_taps(b), want_dbias=True, dhistory=dh,
                                   dtail=gh.dev_bits(dtail), **kw)
    torch.cuda.synchronize()
    ci = torch.from_numpy(cols).cuda()
    xs, dys = gh.host_bits(x[:, ci].contiguous()), gh.host_bits(dy[:, ci].contiguous())
    ys, dxs = gh.host_bits(y[:, ci].contiguous()), gh.host_bits(dx[:, ci].contiguous())
    dws, dbs = dw[ci].cpu().numpy(), db[ci].cpu().numpy()
    dhs = gh.host_bits(dh[:, :, ci].contiguous()).reshape(nseq, 3, len(cols))
    del x, dy, y, dx
    torch.cuda.empty_cache()
    hs = np.ascontiguousarray(hist[:, :, cols])
    wc, bc = np.ascontiguousarray(w[cols]), np.ascontiguousarray(b[cols])
    yr = oracle.fwd(xs, wc, bc, cu_seqlens=cu, hist=hs, has_history=hh)
    gh.assert_bf16_close(ys, yr, "far-offset forward y")
    dxr, dwr, dbr, dhr = oracle.bwd(xs, dys, wc, bc, cu_seqlens=cu, hist=hs, has_history=hh,
                                    dtail=np.ascontiguousarray(dtail[:, cols]))
    gh.assert_bf16_close(dxs, dxr, "far-offset dx")
    gh.assert_w_close(dws, dwr, "far-offset dweight")
    gh.assert_w_close(dbs, dbr, "far-offset dbias")
    gh.assert_bf16_close(dhs, dhr, "far-offset d(history)")


def test_64bit_row_offsets_per_token_ids(oracle):
    """Per-token sequence IDs (4096-row batch rows) over rows * C beyond 2^31 elements: y and dx
    on every row, dweight and dbias of sampled channels against the oracle."""
    say("64-bit offsets: per-token IDs, forward and backward")
    rng = np.random.default_rng(38)
    rows, C, cols, T = _BIG_ROWS, _BIG_C, _BIG_COLS, 4096
    ids = np.empty(rows, np.int32)
    nxt = 0
    for b0 in range(0, rows, T):
        cuts = np.sort(rng.choice(np.arange(1, T), int(rng.integers(0, 6)), replace=False))
        bounds = np.concatenate([[0], cuts, [T]])
        for k in range(len(bounds) - 1):
            ids[b0 + bounds[k]:b0 + bounds[k + 1]] = nxt
            nxt += 1
    x, dy = _big_normal(rows, C, 10), _big_normal(rows, C, 11)
    w = wl.uniform_f32(rng, (C, 4))
    b = (rng.standard_normal(C) * 0.1).astype(np.float32)
    kw = dict(seq_idx=gh.dev_i32(ids), seqlen=T)
    y = cc.conv1d_fwd(x, gh.dev_taps(w), gh.dev_taps(b), **kw)
    dx, dw, db, _ = cc.conv1d_bwd(x, dy, gh.dev_taps(w), gh.dev_taps(b), want_dbias=True, **kw)
    torch.cuda.synchronize()
    ci = torch.from_numpy(cols).cuda()
    xs, dys = gh.host_bits(x[:, ci].contiguous()), gh.host_bits(dy[:, ci].contiguous())
    ys, dxs = gh.host_bits(y[:, ci].contiguous()), gh.host_bits(dx[:, ci].contiguous())
    dws, dbs = dw[ci].cpu().numpy(), db[ci].cpu().numpy()
    del x, dy, y, dx
    torch.cuda.empty_cache()
    wc, bc = np.ascontiguousarray(w[cols]), np.ascontiguousarray(b[cols])
    gh.assert_bf16_close(ys, oracle.fwd(xs, wc, bc, seq_idx=ids, seqlen=T), "far-offset per-token-ID y")
    dxr, dwr, dbr, _ = oracle.bwd(xs, dys, wc, bc, seq_idx=ids, seqlen=T)
    gh.assert_bf16_close(dxs, dxr, "far-offset per-token-ID dx")
    gh.assert_w_close(dws, dwr, "far-offset per-token-ID dweight")
    gh.assert_w_close(dbs, dbr, "far-offset per-token-ID dbias")


@pytest.mark.parametrize("layout", ["hist", "chan"])
def test_64bit_pool_offsets(oracle, layout):
    """A slot pool beyond 2^31 elements (33000 slots x 16384 channels x 4 positions, 4.3 GB; slot
    32768 starts at element 2^31): a prefill and then a decode step on slots near its end.  y, the
    decode outputs and the written states of sampled channels against the oracle, which gets only
    the used slots; a slot between them stays untouched."""
    say(f"64-bit offsets: slot pool, {layout} layout")
    rng = np.random.default_rng(39)
    C, slots, cols = _BIG_C, 33000, _BIG_COLS
    if layout == "hist":
        pool = torch.empty(slots, C, 4, dtype=torch.bfloat16, device="cuda")
    else:
        pool = torch.empty(slots, 4, C, dtype=torch.bfloat16, device="cuda").permute(0, 2, 1)
    pool.normal_(generator=torch.Generator(device="cuda").manual_seed(12))
    lengths = [5, 1, 300, 2, 77]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    ci = np.array([32999, 32768, 31000, -1, 32767], np.int32)
    hi = np.array([1, 0, 1, 1, 1], np.uint8)
    live = [int(s) for s in ci if s >= 0]
    small_ci = np.array([live.index(int(s)) if s >= 0 else -1 for s in ci], np.int32)
    used = torch.tensor(live, device="cuda")
    ccol = torch.from_numpy(cols).cuda()

    def used_state():  # [len(live), 5, 4] bits of the used slots at the sampled channels
        return gh.host_bits(pool[used][:, ccol, :].contiguous()).reshape(len(live), len(cols), 4)

    spare = gh.host_bits(pool[32998].contiguous())
    small_pool = used_state().copy()
    x = wl.normal_bf16(rng, (int(cu[-1]), C))
    w = wl.uniform_f32(rng, (C, 4))
    b = (rng.standard_normal(C) * 0.1).astype(np.float32)
    wc, bc = np.ascontiguousarray(w[cols]), np.ascontiguousarray(b[cols])
    y = cc.conv1d_fwd(gh.dev_bits(x), gh.dev_taps(w), gh.dev_taps(b), cu_seqlens=gh.dev_i32(cu), conv_state=pool,
                      cache_indices=gh.dev_i32(ci), has_initial_state=gh.dev_u8(hi))
    torch.cuda.synchronize()
    yr = oracle.fwd(np.ascontiguousarray(x[:, cols]), wc, bc, cu_seqlens=cu, pool=small_pool,
                    cache_indices=small_ci, has_initial_state=hi)
    gh.assert_bf16_close(gh.host_bits(y[:, ccol].contiguous()), yr, f"far-slot prefill y ({layout})")
    assert np.array_equal(used_state(), small_pool), f"far-slot prefill states ({layout})"
    # one decode token per sequence on the same slots
    xt = wl.normal_bf16(rng, (len(ci), C))
    yt = cc.conv1d_state_update(gh.dev_bits(xt), gh.dev_taps(w), gh.dev_taps(b), conv_state=pool,
                                cache_indices=gh.dev_i32(ci))
    torch.cuda.synchronize()
    ytr = oracle.state_update(np.ascontiguousarray(xt[:, cols]), wc, bc, pool=small_pool, cache_indices=small_ci)
    gh.assert_bf16_close(gh.host_bits(yt[:, ccol].contiguous()), ytr, f"far-slot decode y ({layout})")
    assert np.array_equal(used_state(), small_pool), f"far-slot decode states ({layout})"
    assert np.array_equal(gh.host_bits(pool[32998].contiguous()), spare), "an unused slot was written"
    del pool
    torch.cuda.empty_cache()


def test_64bit_offsets_channels_first(oracle):
    """Channels-first x [3, 16384, 65536] (3 * 2^30 elements, 6.4 GB per tensor; batch row 2 starts
    at element 2^31): forward and backward, y and dx of sampled channels on every step, dweight and
    dbias of those channels against the oracle."""
    say("64-bit offsets: channels-first")
    rng = np.random.default_rng(40)
    B, D, T = 3, 16384, 65536
    cols = _BIG_COLS
    x = torch.empty(B, D, T, dtype=torch.bfloat16, device="cuda")
    x.normal_(generator=torch.Generator(device="cuda").manual_seed(13))
    dy = torch.empty_like(x)
    dy.normal_(generator=torch.Generator(device="cuda").manual_seed(14))
    w = wl.uniform_f32(rng, (D, 4))
    b = (rng.standard_normal(D) * 0.1).astype(np.float32)
    y = cc.conv1d_fwd_cf(x, gh.dev_taps(w), gh.dev_taps(b))
    dx, dw, db = cc.conv1d_bwd_cf(x, dy, gh.dev_taps(w), gh.dev_taps(b), want_dbias=True)
    torch.cuda.synchronize()
    ccol = torch.from_numpy(cols).cuda()
    xs, dys = gh.host_bits(x[:, ccol, :].contiguous()), gh.host_bits(dy[:, ccol, :].contiguous())
    ys, dxs = gh.host_bits(y[:, ccol, :].contiguous()), gh.host_bits(dx[:, ccol, :].contiguous())
    dws, dbs = dw[ccol].cpu().numpy(), db[ccol].cpu().numpy()
    del x, dy, y, dx
    torch.cuda.empty_cache()
    shape = (B, len(cols), T)
    xs, dys, ys, dxs = xs.reshape(shape), dys.reshape(shape), ys.reshape(shape), dxs.reshape(shape)
    wc, bc = np.ascontiguousarray(w[cols]), np.ascontiguousarray(b[cols])
    gh.assert_bf16_close(ys, oracle.fwd_cf(xs, wc, bc), "far-offset channels-first y")
    dxr, dwr, dbr = oracle.bwd_cf(xs, dys, wc, bc, want_db=True)
    gh.assert_bf16_close(dxs, dxr, "far-offset channels-first dx")
    gh.assert_w_close(dws, dwr, "far-offset channels-first dweight")
    gh.assert_w_close(dbs, dbr, "far-offset channels-first dbias")


def test_sequence_forms_agree_bitwise():
    """The per-token-ID workload (16384 x 4096, 21 sequences over 4096-row batch rows) and the
    same sequences given as cu_seqlens offsets; then one sequence per batch row in all three
    forms: y, dx, dweight and dbias identical bit for bit (the forms only locate the same
    boundaries; every partial sum covers the same rows)."""
    say("sequence forms: per-token IDs against the same sequences as offsets")
    case = wl.train_seq_ids()
    ids, T = case["seq_idx"].astype(np.int64), case["seqlen"]
    rows = case["x"].shape[0]
    starts = [0] + [i for i in range(1, rows) if ids[i] != ids[i - 1] or i % T == 0]
    cu = np.array(starts + [rows], np.int32)
    assert len(cu) > 2
    x, dy = gh.dev_bits(case["x"]), gh.dev_bits(case["dy"])
    w, b = gh.dev_taps(case["w"]), gh.dev_taps(case.get("b"))
    out = {}
    for form, kw in (("idx", dict(seq_idx=gh.dev_i32(case["seq_idx"]), seqlen=T)), ("cu", dict(cu_seqlens=gh.dev_i32(cu)))):
        y = cc.conv1d_fwd(x, w, b, **kw)
        dx, dw, db, _ = cc.conv1d_bwd(x, dy, w, b, want_dbias=True, **kw)
        torch.cuda.synchronize()
        out[form] = (gh.host_bits(y), gh.host_bits(dx), dw.view(torch.int32).cpu().numpy(),
                     db.view(torch.int32).cpu().numpy())
    for name, a, c in zip(("y", "dx", "dweight", "dbias"), out["idx"], out["cu"]):
        assert np.array_equal(a, c), f"{name} differs between the per-token-ID and offsets forms"
    # one sequence per batch row: the batch-row form, IDs = batch row, offsets at every T rows
    forms = (("batch", dict(seqlen=T)),
             ("idx", dict(seq_idx=gh.dev_i32((np.arange(rows) // T).astype(np.int32)), seqlen=T)),
             ("cu", dict(cu_seqlens=gh.dev_i32(np.arange(0, rows + 1, T, dtype=np.int32)))))
    out = {}
    for form, kw in forms:
        y = cc.conv1d_fwd(x, w, b, **kw)
        dx, dw, db, _ = cc.conv1d_bwd(x, dy, w, b, want_dbias=True, **kw)
        torch.cuda.synchronize()
        out[form] = (gh.host_bits(y), gh.host_bits(dx), dw.view(torch.int32).cpu().numpy(),
                     db.view(torch.int32).cpu().numpy())
    for other in ("idx", "cu"):
        for name, a, c in zip(("y", "dx", "dweight", "dbias"), out["batch"], out[other]):
            assert np.array_equal(a, c), f"{name} differs between the batch-row and {other} forms"


@pytest.mark.parametrize("layout", ["hist", "chan"])
def test_pool_state_equals_history_rows(layout):
    """The prefill workload (32768 x 5632, 64 sequences, 256 padding rows) read its history from a
    slot pool (positions 0..2, 24-row tiles, slot lookup and write-back) and, with the same values
    as caller history rows (16-row tiles), gives the same y bits; sequences without initial state
    start from zeros in both; the padding rows stay untouched in both."""
    say(f"pool state against history rows ({layout} layout)")
    case = wl.prefill_pool()
    rng = np.random.default_rng(41)
    hi = (rng.random(len(case["cache_indices"])) < 0.7).astype(np.uint8)
    pool = wl.pool_layout(case["pool"], layout)
    hist = np.ascontiguousarray(case["pool"][case["cache_indices"]][:, :, 0:3].transpose(0, 2, 1))
    x = gh.dev_bits(case["x"])
    w, b = gh.dev_taps(case["w"]), gh.dev_taps(case["b"])
    cu = gh.dev_i32(case["cu_seqlens"])
    rows, C = case["x"].shape
    y_pool = gh.dev_bits(np.full((rows, C), wl.OUT_FILL, np.uint16))
    y_hist = gh.dev_bits(np.full((rows, C), wl.OUT_FILL, np.uint16))
    cc.conv1d_fwd(x, w, b, cu_seqlens=cu, conv_state=gh.dev_pool(pool), cache_indices=gh.dev_i32(case["cache_indices"]),
                  has_initial_state=gh.dev_u8(hi), out=y_pool)
    cc.conv1d_fwd(x, w, b, cu_seqlens=cu, history=gh.dev_bits(hist), has_history=gh.dev_u8(hi), out=y_hist)
    torch.cuda.synchronize()
    a, c = gh.host_bits(y_pool), gh.host_bits(y_hist)
    end = int(case["cu_seqlens"][-1])
    assert end < rows and (a[end:] == wl.OUT_FILL).all() and (c[end:] == wl.OUT_FILL).all()
    assert np.array_equal(a, c), "pool-state and history-row forwards differ"


@pytest.mark.parametrize("work", ["cp", "ids"])
def test_bf16_and_fp32_taps_agree_bitwise(work):
    """Taps and bias given as bf16, or as FP32 holding the same (bf16-representable) values: the
    same y, dx, dweight, dbias and d(history) bits at full size (both widen exactly to FP32)."""
    say(f"bf16 against FP32 taps ({work})")
    rng = np.random.default_rng(43)
    case = wl.cp_share() if work == "cp" else wl.train_seq_ids()
    C = case["x"].shape[1]
    wb = wl.to_bf16_bits(wl.uniform_f32(rng, (C, 4)))
    bb = wl.to_bf16_bits((rng.standard_normal(C) * 0.1).astype(np.float32))
    x, dy = gh.dev_bits(case["x"]), gh.dev_bits(case["dy"])
    kw = dict(cu_seqlens=gh.dev_i32(case.get("cu_seqlens")), seq_idx=gh.dev_i32(case.get("seq_idx")),
              seqlen=case.get("seqlen"))
    if case.get("hist") is not None:
        kw.update(history=gh.dev_bits(case["hist"]), has_history=gh.dev_u8(case["has_history"]))
    out = []
    for w, b in ((gh.dev_bits(wb), gh.dev_bits(bb)),
                 (torch.from_numpy(wl.bf16_bits_to_f32(wb)).cuda(), torch.from_numpy(wl.bf16_bits_to_f32(bb)).cuda())):
        dh = gh.dev_bits(np.full(case["hist"].shape, wl.OUT_FILL, np.uint16)) if case.get("hist") is not None else None
        y = cc.conv1d_fwd(x, w, b, **kw)
        dx, dw, db, dh = cc.conv1d_bwd(x, dy, w, b, want_dbias=True, dhistory=dh, **kw)
        torch.cuda.synchronize()
        out.append((gh.host_bits(y), gh.host_bits(dx), dw.view(torch.int32).cpu().numpy(),
                    db.view(torch.int32).cpu().numpy(), None if dh is None else gh.host_bits(dh)))
    for name, a, c in zip(("y", "dx", "dweight", "dbias", "d(history)"), *out):
        assert (a is None and c is None) or np.array_equal(a, c), f"{name} differs between bf16 and FP32 taps"


def test_graph_replay_equals_eager_at_full_size():
    """The context-parallel share (16384 x 5632) forward and backward captured once in a HIP graph:
    three replays, with eager calls on other buffers between them, give the eager call's y, dx,
    dweight and d(history) bits."""
    say("graph replay against eager, full size")
    case = wl.cp_share()
    x, dy = gh.dev_bits(case["x"]), gh.dev_bits(case["dy"])
    w = gh.dev_taps(case["w"])
    kw = dict(cu_seqlens=gh.dev_i32(case["cu_seqlens"]), history=gh.dev_bits(case["hist"]),
              has_history=gh.dev_u8(case["has_history"]))
    rows, C = case["x"].shape
    bufs = dict(y=torch.empty(rows, C, dtype=torch.bfloat16, device="cuda"),
                dx=torch.empty(rows, C, dtype=torch.bfloat16, device="cuda"),
                dw=torch.empty(C, 4, dtype=torch.float32, device="cuda"),
                dh=gh.dev_bits(np.full(case["hist"].shape, wl.OUT_FILL, np.uint16)),
                ws=torch.empty(cc.conv1d_bwd_workspace_bytes(rows, C), dtype=torch.uint8, device="cuda"))

    def run(o):
        cc.conv1d_fwd(x, w, None, out=o["y"], **kw)
        cc.conv1d_bwd(x, dy, w, None, dx=o["dx"], dweight=o["dw"], dhistory=o["dh"], workspace=o["ws"], **kw)

    def bits(o):
        return (gh.host_bits(o["y"]), gh.host_bits(o["dx"]), o["dw"].view(torch.int32).cpu().numpy(), gh.host_bits(o["dh"]))

    eager = {k: v.clone() for k, v in bufs.items()}
    run(eager)
    torch.cuda.synchronize()
    ref = bits(eager)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(bufs)  # warm up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(bufs)
    for replay in range(3):
        for k in ("y", "dx", "dw"):
            bufs[k].zero_()
        graph.replay()
        run(eager)  # eager work between replays, on other buffers
        torch.cuda.synchronize()
        for name, a, c in zip(("y", "dx", "dweight", "d(history)"), bits(bufs), ref):
            assert np.array_equal(a, c), f"replay {replay}: {name} differs from the eager call"
