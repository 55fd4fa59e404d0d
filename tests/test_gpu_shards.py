"""GPU: the one-GPU share of the context-parallel backward across shards.

- d(tail): the next shard's gradient of the last W-1 values of this shard's last sequence, added in
  FP32 before the single rounding (cake_causal_conv1d_kcp, Returns; the differentiable history
  exchange of core.ssm.causal_conv1d) - against the oracle with the same d(tail), in every sequence
  form, widths 2, 4 and 8, last sequences shorter than the history and empty.
- The context-parallel workload (x [16384, 5632], 12 fragments) split into two shards on one GPU:
  shard B's d(history) goes straight (device to device, no host arithmetic) into shard A's d(tail).
- The head of a multi-GPU backward: the call over a fragment's first W-1 rows alone returns that
  fragment's d(history) bit for bit, as the full call does.
- The shard-ordered dweight combine (assert_causal_conv1d_deterministic): bit-exact against the
  oracle's ordered sum, and bitwise stable from run to run.
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


def say(msg):
    print(f"[gpu] {msg}", flush=True)


def _widen(case, W, rng):
    out = dict(case)
    C = case["x"].shape[1]
    out["w"] = wl.uniform_f32(rng, (C, W))
    if case.get("hist") is not None:
        out["hist"] = wl.normal_bf16(rng, (case["hist"].shape[0], W - 1, C))
    return out


def test_dtail_matches_oracle(oracle):
    rng = np.random.default_rng(51)
    for q in range(24):
        W = (4, 2, 8)[q % 3]
        mode = ("cu", "batch", "idx")[(q // 3) % 3]
        C = int(rng.choice([8, 13, 64, 520, 1024]))
        base = wl.random_case(rng, C=C, mode=mode, nseq=int(rng.integers(1, 7)),
                              max_len=int(rng.choice([2, 5, 40, 300])), with_hist=(mode != "idx"),
                              w_f32=bool(q % 2), act="silu" if q % 4 else "none")
        if mode == "cu" and q % 2:  # last fragment of 0..2 rows
            cu = base["cu_seqlens"].copy()
            cu[-1] = cu[-2] + min(int(rng.integers(0, 3)), int(cu[-1] - cu[-2]))
            base["cu_seqlens"] = cu
        case = _widen(base, W, rng) if W != 4 else base
        case["name"] = f"dtail-{mode}-W{W}-C{C}-{q}"
        say(f"{case['name']} rows={case['x'].shape[0]}")
        gh.check_bwd(oracle, case, dtail=wl.normal_bf16(rng, (W - 1, C)))


def test_dtail_full_size(oracle):
    case = wl.cp_share()
    rng = np.random.default_rng(52)
    say("dtail on the context-parallel workload")
    gh.check_bwd(oracle, case, dtail=wl.normal_bf16(rng, (3, case["x"].shape[1])))


def _split(case, cut):
    """Shards A = rows [0, cut) and B = rows [cut, S) of a fragment list (cu_seqlens + history rows);
    the fragment holding row cut continues in B, whose first history rows are the three values of
    that fragment's extended sequence before row cut."""
    cu = case["cu_seqlens"].astype(np.int64)
    k = int(np.searchsorted(cu, cut, side="right")) - 1  # fragment holding row cut
    assert cu[k] < cut < cu[k + 1]
    s = int(cu[k])
    hh = case["has_history"]
    ext = np.concatenate([case["hist"][k] if hh[k] else np.zeros((3, case["x"].shape[1]), np.uint16),
                          case["x"][s:cut]], axis=0)  # fragment k's extended sequence up to row cut
    a = dict(case, name="shard-A", x=case["x"][:cut], dy=case["dy"][:cut],
             cu_seqlens=np.concatenate([cu[:k + 1], [cut]]).astype(np.int32),
             hist=np.ascontiguousarray(case["hist"][:k + 1]), has_history=hh[:k + 1].copy())
    b_hist = np.concatenate([ext[-3:][None], case["hist"][k + 1:]], axis=0)
    b = dict(case, name="shard-B", x=case["x"][cut:], dy=case["dy"][cut:],
             cu_seqlens=np.concatenate([[0], cu[k + 1:] - cut]).astype(np.int32),
             hist=np.ascontiguousarray(b_hist), has_history=np.concatenate([[1], hh[k + 1:]]).astype(np.uint8))
    return a, b


def _dev_case(case):
    d = dict(x=gh.dev_bits(case["x"]), dy=gh.dev_bits(case["dy"]), w=gh.dev_taps(case["w"]),
             cu=gh.dev_i32(case["cu_seqlens"]), hist=gh.dev_bits(case["hist"]), hh=gh.dev_u8(case["has_history"]))
    rows, C = case["x"].shape
    d["dx"] = torch.empty((rows, C), dtype=torch.bfloat16, device="cuda")
    d["dh"] = gh.dev_bits(np.full(case["hist"].shape, wl.OUT_FILL, np.uint16))  # rows left untouched keep this
    return d


def _bwd_dev(d, dtail=None, dweight=None):
    return cc.conv1d_bwd(d["x"], d["dy"], d["w"], None, cu_seqlens=d["cu"], history=d["hist"], has_history=d["hh"],
                         dx=d["dx"], dhistory=d["dh"], dweight=dweight, dtail=dtail)


@pytest.mark.parametrize("cut_in", [1, 2, 1000])
def test_two_shards_on_one_gpu(oracle, cut_in):
    """Split the context-parallel workload into two shards inside a fragment (1, 2 or 1000 rows into
    it: shard A's last fragment shorter than, or longer than, the history).  B runs first; its
    d(history) of the continuing fragment is passed as A's d(tail) on the device.
      - A's dx equals the oracle's dx for A given the oracle's own d(tail) from B (bf16 tolerance,
        widened only by the difference between the GPU's and the oracle's d(tail) bits, which
        enters dx one to one), and the unsplit oracle dx up to one bf16 rounding of the exchanged
        gradient (d(history) is bf16);
      - rows before A's last three are bit-identical with and without d(tail);
      - the shard-ordered combine of the two dweights is bitwise stable over 10 runs and within the
        dweight tolerance of the unsplit oracle."""
    whole = wl.cp_share()
    cu = whole["cu_seqlens"]
    k = int(np.argmax(np.diff(cu)))  # the longest fragment
    cut = int(cu[k]) + cut_in
    say(f"two shards, cut at row {cut} ({cut_in} rows into fragment {k})")
    A, B = _split(whole, cut)
    C = whole["x"].shape[1]
    dA, dB = _dev_case(A), _dev_case(B)
    dw_parts = torch.empty((2, C, 4), dtype=torch.float32, device="cuda")
    _bwd_dev(dB, dweight=dw_parts[1])
    _bwd_dev(dA, dtail=dB["dh"][0], dweight=dw_parts[0])
    torch.cuda.synchronize()
    dx_a = gh.host_bits(dA["dx"])
    dtail_gpu = gh.host_bits(dB["dh"][0])
    # the oracle chain: B, then A with the oracle's d(tail)
    dx_b_ref, dw_b_ref, _, dh_b_ref = gh.oracle_bwd(oracle, B)
    gh.assert_bf16_close(gh.host_bits(dB["dx"]), dx_b_ref, "shard B dx")
    gh.assert_bf16_close(dtail_gpu, dh_b_ref[0], "shard B d(history) of the continuing fragment")
    dx_a_ref, dw_a_ref, _, dh_a_ref = gh.oracle_bwd(oracle, A, dtail=np.ascontiguousarray(dh_b_ref[0]))
    n_last = cut - int(A["cu_seqlens"][-2])
    extra = np.zeros(dx_a.shape)
    for j in range(3):
        r = cut - 3 + j
        if r >= cut - n_last:
            extra[r] = np.abs(gh.f32(dtail_gpu[j]) - gh.f32(dh_b_ref[0][j]))
    g, r = gh.f32(dx_a), gh.f32(dx_a_ref)
    bad = ~(np.abs(g - r) <= gh.Y_RTOL * np.abs(r) + gh.Y_ATOL + extra)
    assert not bad.any(), f"shard A dx with d(tail): {int(bad.sum())} elements off"
    # d(history) of A's fragments; when the last one is shorter than the history, its rows n_last..2
    # take d(tail) values 0..2-n_last (same allowance for the d(tail) bits)
    dh_a = gh.host_bits(dA["dh"])
    gh.assert_bf16_close(dh_a[:-1], dh_a_ref[:-1], "shard A d(history)")
    if A["has_history"][-1]:
        extra_h = np.zeros((3, C))
        for j in range(n_last, 3):
            extra_h[j] = np.abs(gh.f32(dtail_gpu[j - n_last]) - gh.f32(dh_b_ref[0][j - n_last]))
        gh_, rh = gh.f32(dh_a[-1]), gh.f32(dh_a_ref[-1])
        assert (np.abs(gh_ - rh) <= gh.Y_RTOL * np.abs(rh) + gh.Y_ATOL + extra_h).all(), "d(history) of A's last fragment"
    # against the unsplit batch: one extra bf16 rounding of the exchanged gradient
    dx_u, dw_u, _, _ = gh.oracle_bwd(oracle, whole)
    tail_part = np.zeros(dx_a.shape)
    for j in range(3):
        r = cut - 3 + j
        if r >= cut - n_last:
            tail_part[r] = np.abs(gh.f32(dtail_gpu[j]))
    u = gh.f32(dx_u[:cut])
    bad = ~(np.abs(g - u) <= gh.Y_RTOL * np.abs(u) + gh.Y_ATOL + 2.0 ** -8 * tail_part)
    assert not bad.any(), f"shard A dx vs the unsplit batch: {int(bad.sum())} elements off"
    gh.assert_bf16_close(gh.host_bits(dB["dx"]), dx_u[cut:], "shard B dx vs the unsplit batch")
    # d(tail) touches only the last three rows
    dA2 = _dev_case(A)
    _bwd_dev(dA2)
    torch.cuda.synchronize()
    assert np.array_equal(gh.host_bits(dA2["dx"])[:cut - 3], dx_a[:cut - 3])
    # shard-ordered dweight
    outs = []
    for run in range(10):
        dw, _ = cc.conv1d_bwd_combine(dw_parts)
        torch.cuda.synchronize()
        outs.append(dw.view(torch.int32).cpu().numpy())
        assert np.array_equal(outs[0], outs[-1]), f"combine run {run} differs"
    gh.assert_w_close(dw.cpu().numpy(), dw_u, "shard-ordered dweight vs unsplit")


def test_head_call_gives_the_fragment_d_history(oracle):
    """The multi-GPU backward's head: conv1d_bwd over the first W-1 rows of a shard's first fragment
    alone (with its history rows) returns that fragment's d(history) bit for bit, as the full call
    does, since d(history) takes only the dz of those rows; and it matches the oracle."""
    whole = wl.cp_share()
    cu = whole["cu_seqlens"]
    k = int(np.argmax(np.diff(cu)))
    cut = int(cu[k]) + 1000
    _, B = _split(whole, cut)
    say(f"head call: shard from row {cut}")
    dB = _dev_case(B)
    _bwd_dev(dB)
    head = dict(B, name="head", x=B["x"][:3], dy=B["dy"][:3], cu_seqlens=np.array([0, 3], np.int32),
                hist=np.ascontiguousarray(B["hist"][:1]), has_history=np.ones(1, np.uint8))
    dH = _dev_case(head)
    _bwd_dev(dH)
    torch.cuda.synchronize()
    full, part = gh.host_bits(dB["dh"])[0], gh.host_bits(dH["dh"])[0]
    assert np.array_equal(full, part), "head call d(history) differs from the full call's"
    _, _, _, dh_ref = gh.oracle_bwd(oracle, head)
    gh.assert_bf16_close(part, dh_ref[0], "head call d(history) vs oracle")


def test_combine_bit_exact_against_oracle(oracle):
    """The ordered sum on seeded partials (values spread over many binades, so the order matters):
    bit-exact against the oracle's ordered sum; one shard is a bit copy; zero shards give zeros."""
    rng = np.random.default_rng(53)
    for S, C, W, with_b in ((2, 5632, 4, True), (7, 13, 8, False), (1, 64, 3, True), (33, 1000, 2, True), (0, 8, 4, True)):
        scale = np.exp2(rng.integers(-20, 20, size=(S, C, W))).astype(np.float32)
        p = (rng.standard_normal((S, C, W)).astype(np.float32) * scale).astype(np.float32)
        pb = (rng.standard_normal((S, C)).astype(np.float32) * np.float32(1e3)) if with_b else None
        say(f"combine S={S} C={C} W={W}")
        dw, db = cc.conv1d_bwd_combine(torch.from_numpy(p).cuda(), None if pb is None else torch.from_numpy(pb).cuda())
        torch.cuda.synchronize()
        ref = oracle.combine(p)
        assert np.array_equal(dw.cpu().numpy().view(np.uint32), ref.view(np.uint32)), "combine dweight bits"
        if pb is not None:
            assert np.array_equal(db.cpu().numpy().view(np.uint32), oracle.combine(pb).view(np.uint32)), "dbias bits"
