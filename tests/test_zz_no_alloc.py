"""GPU: the allocation-free backward (conv1d_bwd_noalloc) against conv1d_bwd, through the C ABI.

Same kernels and the same row-range split, so dx, dweight, dbias and d(history) must match bit
for bit.  Two calls in a row on the library's scratch, the second on a smaller problem (the
scratch keeps the first call's partials: every partial the second call reads must be its own),
then a third at a different width and sequence form.
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


def _outputs(case, W):
    rows, C = case["x"].shape
    nseq = case["hist"].shape[0] if case.get("hist") is not None else 0
    return dict(dx=gh.dev_bits(np.full((rows, C), wl.OUT_FILL, np.uint16)),
                dweight=torch.empty((C, W), dtype=torch.float32, device="cuda"),
                dbias=torch.empty((C,), dtype=torch.float32, device="cuda"),
                dhistory=gh.dev_bits(np.full((nseq, W - 1, C), wl.OUT_FILL, np.uint16)) if nseq else None)


def _run(fn, case, dtail, **extra):
    W = case["w"].shape[1]
    out = _outputs(case, W)
    kw = dict(cu_seqlens=gh.dev_i32(case.get("cu_seqlens")), seq_idx=gh.dev_i32(case.get("seq_idx")),
              seqlen=case.get("seqlen"), history=gh.dev_bits(case["hist"]) if case.get("hist") is not None else None,
              has_history=gh.dev_u8(case.get("has_history")), dtail=None if dtail is None else gh.dev_bits(dtail))
    x, dy = gh.dev_bits(case["x"]), gh.dev_bits(case["dy"])
    w, b = gh.dev_taps(case["w"]), gh.dev_taps(case.get("b"))
    if fn is cc.conv1d_bwd_noalloc:
        fn(x, dy, w, b, **out, **kw)
    else:
        fn(x, dy, w, b, dx=out["dx"], dweight=out["dweight"], dbias=out["dbias"], want_dbias=True,
           dhistory=out["dhistory"], **kw)
    torch.cuda.synchronize()
    return {k: (None if v is None else v.view(torch.int16 if v.dtype == torch.bfloat16 else torch.int32).cpu().numpy())
            for k, v in out.items()}


def test_noalloc_matches_conv1d_bwd(oracle):
    rng = np.random.default_rng(61)
    big = wl.cp_share()                                     # x [16384, 5632]: 11 strips x ~93 ranges of partials
    small = wl.random_case(rng, C=520, nseq=5, max_len=300, with_hist=True, act="silu")
    ids = wl.train_seq_ids()
    ids = dict(ids, x=ids["x"][:4096], dy=ids["dy"][:4096], seq_idx=ids["seq_idx"][:4096])  # one batch row
    ids["w"] = wl.uniform_f32(rng, (ids["x"].shape[1], 8))
    cases = [(big, wl.normal_bf16(rng, (3, big["x"].shape[1]))), (small, None), (ids, None)]
    for case, dtail in cases:
        print(f"[gpu] noalloc {case['name']} rows={case['x'].shape[0]} C={case['x'].shape[1]} W={case['w'].shape[1]}",
              flush=True)
        got = _run(cc.conv1d_bwd_noalloc, case, dtail)
        ref = _run(cc.conv1d_bwd, case, dtail)
        for k in got:
            if ref[k] is not None:
                assert np.array_equal(got[k], ref[k]), f"{case['name']}: {k} differs from conv1d_bwd"
        # and the parity bar itself, against the oracle
        dxr, dwr, dbr, _ = gh.oracle_bwd(oracle, case, dtail=dtail)
        gh.assert_bf16_close(got["dx"].view(np.uint16), dxr, f"{case['name']}: dx vs oracle")
        gh.assert_w_close(got["dweight"].view(np.float32), dwr, f"{case['name']}: dweight vs oracle")


def test_noalloc_refuses_oversized_problems():
    C = 600000
    x = torch.zeros((8, C), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((C, 8), dtype=torch.float32, device="cuda")
    with pytest.raises(RuntimeError, match="scratch"):
        cc.conv1d_bwd_noalloc(x, x.clone(), w, dx=torch.empty_like(x), dweight=torch.empty_like(w),
                              cu_seqlens=torch.tensor([0, 8], dtype=torch.int32, device="cuda"))
