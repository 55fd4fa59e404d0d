"""Host logic of bench.py, on the CPU: the algorithmic byte counts behind every GB/s figure, the
one-GPU refusal, and the guard that keeps stored counter figures from outliving the kernels they
were measured on."""
import json
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from causal_depthwise_conv1d_width_amd import workloads as wl  # noqa: E402


def _fwd_closed_form(C, r_read, r_out, n_state, w_bytes, b_bytes, meta):
    # each live input row read once, each output row written once, W-1 = 3 history values of C
    # bf16 per state read / state write / history set, the taps, the bias, the metadata
    return 2 * C * r_read + 2 * C * r_out + 6 * C * n_state + w_bytes + b_bytes + meta


def test_bytes_of_the_context_parallel_share():
    """x [16384, 5632] in 12 fragments, 8 reading history rows, fp32 taps, no bias."""
    case = wl.cp_share()
    C, R, nseq = 5632, 16384, 12
    n_hist = int(np.count_nonzero(case["has_history"]))
    assert n_hist == 8
    meta = (nseq + 1) * 4 + nseq  # cu_seqlens, has_history flags
    assert bench.fwd_bytes(case) == _fwd_closed_form(C, R, R, n_hist, 4 * C * 4, 0, meta) == 369_459_264
    # x and dy read, dx written; history rows read and their gradient written; taps; dweight
    bwd = 6 * C * R + 6 * C * n_hist + 6 * C * n_hist + 4 * C * 4 + 4 * C * 4 + meta
    assert bench.bwd_bytes(case) == bwd == 554_369_088


def test_bytes_of_the_prefill_with_a_pool():
    """32768 rows (32512 in 64 sequences), pool of 128 slots, every sequence live with state."""
    case = wl.prefill_pool()
    C, nseq = 5632, 64
    lengths = np.diff(case["cu_seqlens"].astype(np.int64))
    assert lengths.sum() == 32512 and (lengths > 0).all() and (case["cache_indices"] >= 0).all()
    assert case["has_initial_state"].all()
    n_state = 2 * nseq  # every sequence reads its state and writes it back
    meta = (nseq + 1) * 4 + nseq * 4 + nseq  # offsets, slots, has_initial_state
    expect = _fwd_closed_form(C, 32512, 32512, n_state, 4 * C * 4, 4 * C, meta)
    assert bench.fwd_bytes(case) == expect


def test_bytes_of_the_per_token_id_workload():
    case = wl.train_seq_ids()
    C, R = 4096, 16384
    meta = R * 4  # one ID per row
    assert bench.fwd_bytes(case) == _fwd_closed_form(C, R, R, 0, 4 * C * 4, 4 * C, meta)
    # + dweight [C, 4] and dbias [C] in FP32
    assert bench.bwd_bytes(case) == 6 * C * R + 4 * C * 4 + 4 * C + 4 * C * 4 + 4 * C + meta


def test_bytes_skip_sentinel_rows_and_count_state_of_live_sequences():
    """The small pool workload: a -1 slot's rows are neither read nor given state; an empty live
    sequence reads and writes no state."""
    case = wl.varlen_pool()
    cu = case["cu_seqlens"].astype(np.int64)
    ci, hi = case["cache_indices"], case["has_initial_state"]
    lengths = np.diff(cu)
    live = ci >= 0
    r_read = int(lengths[live].sum())
    n_state = int(sum(1 + int(hi[i]) for i in range(len(ci)) if live[i] and lengths[i] > 0))
    nseq = len(ci)
    meta = (nseq + 1) * 4 + nseq * 4 + nseq
    C = case["x"].shape[1]
    expect = _fwd_closed_form(C, r_read, int(cu[-1]), n_state, case["w"].size * 2, 0, meta)
    assert bench.fwd_bytes(case) == expect


def test_more_than_one_gpu_is_refused():
    """This build measures one GPU; --gpus 2 exits with status 2 and says so, before any GPU use."""
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert p.returncode == 2
    line = json.loads(p.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"]


def test_source_hash_ignores_comments_only():
    src = "int f() {  // a comment\n  return 1; /* more */\n}\n"
    same = "int f() {  // another comment\n\n  return 1;\n}   \n"
    other = "int f() {\n  return 2;\n}\n"
    assert bench._code_only(src) == bench._code_only(same)
    assert bench._code_only(src) != bench._code_only(other)


def test_stored_traffic_only_for_the_profiled_sources(tmp_path, monkeypatch):
    h = bench.kernel_source_hash()
    good = tmp_path / "good.md"
    good.write_text(f"    kernel_source_sha256_16: {h}\n    hbm_bytes_per_call: 5.5e+08\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(good))
    assert bench.stored_traffic() == 5.5e8
    stale = tmp_path / "stale.md"
    stale.write_text("    kernel_source_sha256_16: 0123456789abcdef\n    hbm_bytes_per_call: 5.5e+08\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(stale))
    assert bench.stored_traffic() is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.md"))
    assert bench.stored_traffic() is None
