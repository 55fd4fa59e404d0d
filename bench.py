"""Benchmark: effective HBM GB/s of the packed causal conv1d (+ SiLU), forward and backward.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step = one pass of the whole hot path over one batch of the context-parallel workload (the
largest single-GPU training workload): the forward (sequence lookup, history rows, stencil,
SiLU) and the backward (recompute, dx, per-block dweight partials + ordered reduce,
d(history)) over x [16384, 5632] bf16 in 12 fragments, 8 with 3 history rows.  Inputs are
resident in HBM before the timed region.  Steady state, as inside a training or serving loop:
the timed calls run back to back on one stream over a ring of independent buffer sets (4 for the
step workload, about 3 GB), so no call finds its operands in the 256 MB Infinity Cache and every
call's writes evict the previous calls' dirty lines, i.e. each written byte is paid for in HBM.
W untimed warm-up steps come first (default 200), then whole untimed passes until 40 ms of
load have gone by, before every timed ring: after an idle gap the clocks need some 20 ms of
sustained load to settle, and a warm-up shorter than that times the ramp.  HIP events on the
stream the library launches on bracket each batch of calls; `value` = algorithmic bytes of K
steps / the batch time.  Effective bytes count what the method must move,
each once (activations read and written, history rows, taps, gradients); halo re-reads and the
dweight partial workspace are overhead and not counted.

The same JSON line also carries every other workload (forward of the small and pool-prefill
workloads, forward and backward of the per-token-ID training workload, a decode step), copy
ceilings (torch's bf16 copy; hand-written copies of the step workload's bytes, contiguous and in
the forward's and backward's own access structure), the roofline object of the dominant call and
the CPU oracle timed on the host as a baseline.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E peak
WARM_MS = 40.0  # untimed load before every timed ring (clock ramp after idle gaps)
METRIC = "effective GB/s (fwd, bwd) of packed causal conv1d+SiLU; % of HBM peak"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_conv1d_bwd_kernel_cp_share.md")
KERNEL_SOURCES = ["conv1d_device.h", "conv1d_launch.h", "conv1d_fwd.hip", "conv1d_bwd.hip", "conv1d_cf.hip", "conv1d_api.cpp"]


# ------------------------------------------------------------------ algorithmic bytes
def _tap_bytes(a):
    return 0 if a is None else a.size * a.itemsize


def _segments(case):
    rows = case["x"].shape[0]
    if case.get("cu_seqlens") is not None:
        cu = case["cu_seqlens"].astype(np.int64)
        return [(int(cu[i]), int(cu[i + 1]), i) for i in range(len(cu) - 1)], int(cu[-1]), len(cu) - 1
    return None, rows, 0


def fwd_bytes(case):
    """2C per row read (live sequences) + 2C per row written + 2(W-1)C per history read / state
    write (W taps) + taps + bias + metadata."""
    rows, C = case["x"].shape
    H = case["w"].shape[1] - 1  # history rows
    segs, r_out, nseq = _segments(case)
    r_read, n_state = r_out, 0
    meta = 0
    if segs is not None:
        meta += (nseq + 1) * 4
        if case.get("pool") is not None:
            ci, hi = case["cache_indices"], case["has_initial_state"]
            meta += nseq * 4 + nseq
            r_read = sum(e - s for s, e, i in segs if ci[i] >= 0)
            n_state = sum((1 + int(hi[i])) for s, e, i in segs if ci[i] >= 0 and e > s)
        if case.get("hist") is not None:
            hh = case.get("has_history")
            meta += nseq
            n_state = sum(1 for s, e, i in segs if e > s and (hh is None or hh[i]))
    if case.get("seq_idx") is not None:
        meta += rows * 4
    return (2 * C * r_read + 2 * C * r_out + 2 * H * C * n_state + _tap_bytes(case["w"]) + _tap_bytes(case.get("b"))
            + meta)


def bwd_bytes(case):
    """6C per row (x, dy read; dx written) + 2(W-1)C per history row set read and as much for its
    gradient written + taps + bias + dweight (+ dbias) + metadata."""
    rows, C = case["x"].shape
    W = case["w"].shape[1]
    segs, r, nseq = _segments(case)
    n_hist, meta = 0, 0
    if segs is not None:
        meta += (nseq + 1) * 4
        if case.get("hist") is not None:
            hh = case.get("has_history")
            meta += nseq
            n_hist = sum(1 for s, e, i in segs if hh is None or hh[i])
    if case.get("seq_idx") is not None:
        meta += rows * 4
    has_b = case.get("b") is not None
    return (6 * C * r + 4 * (W - 1) * C * n_hist + _tap_bytes(case["w"]) + _tap_bytes(case.get("b")) + 4 * W * C
            + (4 * C if has_b else 0) + meta)


def _code_only(text):
    """The source without comments, blank lines and trailing blanks: edits to comments leave the
    hash (and so the stored counter figures) valid."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.rstrip() for line in text.splitlines() if line.strip())


def kernel_source_hash():
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "causal_depthwise_conv1d_width_amd", "csrc", name), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def stored_traffic():
    """HBM bytes per conv1d_bwd call from the committed rocprofv3 counter summary, if it was
    taken on the current kernel sources; else None."""
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    m_hash = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]{16})", text)
    m_bytes = re.search(r"hbm_bytes_per_call:\s*([0-9.eE+]+)", text)
    if not m_hash or not m_bytes or m_hash.group(1) != kernel_source_hash():
        return None
    return float(m_bytes.group(1))


# ------------------------------------------------------------------ GPU side
class Gpu:
    def __init__(self):
        import torch

        import causal_depthwise_conv1d_width_amd as cc
        from causal_depthwise_conv1d_width_amd import _lib
        _lib.load()  # fail loudly if the HIP library is missing
        self.torch, self.cc = torch, cc
        self.dev = torch.device("cuda", 0)
        self.stream = torch.cuda.current_stream()

    def bits(self, a):
        t = self.torch
        return t.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(t.bfloat16).to(self.dev)

    def taps(self, a):
        if a is None:
            return None
        return self.bits(a) if a.dtype == np.uint16 else self.torch.from_numpy(a).to(self.dev)

    def i32(self, a):
        return None if a is None else self.torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(self.dev)

    def u8(self, a):
        return None if a is None else self.torch.from_numpy(np.ascontiguousarray(a, np.uint8)).to(self.dev)

    def pool(self, a):
        t = self.torch
        st = tuple(s // 2 for s in a.strides)
        p = t.empty_strided(a.shape, st, dtype=t.bfloat16, device=self.dev)
        p.copy_(self.bits(np.ascontiguousarray(a)).view(a.shape))
        return p

    def prepare(self, case):
        """Device copies of a workload plus preallocated outputs: calls allocate nothing."""
        t = self.torch
        rows, C = case["x"].shape
        d = dict(x=self.bits(case["x"]), w=self.taps(case["w"]), b=self.taps(case.get("b")),
                 cu=self.i32(case.get("cu_seqlens")), seq_idx=self.i32(case.get("seq_idx")),
                 seqlen=case.get("seqlen"), act=case.get("act", "silu"))
        d["y"] = t.empty((rows, C), dtype=t.bfloat16, device=self.dev)
        if case.get("pool") is not None:
            d["pool"] = self.pool(case["pool"])
            d["ci"], d["hi"] = self.i32(case["cache_indices"]), self.u8(case["has_initial_state"])
        if case.get("hist") is not None:
            d["hist"], d["hh"] = self.bits(case["hist"]), self.u8(case.get("has_history"))
            d["dhist"] = t.empty_like(d["hist"])
        if case.get("dy") is not None:
            d["dy"] = self.bits(case["dy"])
            d["dx"] = t.empty((rows, C), dtype=t.bfloat16, device=self.dev)
            d["dw"] = t.empty((C, case["w"].shape[1]), dtype=t.float32, device=self.dev)
            d["db"] = t.empty((C,), dtype=t.float32, device=self.dev) if case.get("b") is not None else None
            need = self.cc.conv1d_bwd_workspace_bytes(rows, C)
            d["ws"] = t.empty((max(need, 1),), dtype=t.uint8, device=self.dev)
        return d

    def fwd(self, d):
        # repeated prefills keep updating the pool in place: same reads and writes every call
        return self.cc.conv1d_fwd(d["x"], d["w"], d["b"], cu_seqlens=d["cu"], seq_idx=d["seq_idx"],
                                  seqlen=d["seqlen"], conv_state=d.get("pool"), cache_indices=d.get("ci"),
                                  has_initial_state=d.get("hi"), history=d.get("hist"),
                                  has_history=d.get("hh"), activation=d["act"], out=d["y"])

    def bwd(self, d):
        return self.cc.conv1d_bwd(d["x"], d["dy"], d["w"], d["b"], cu_seqlens=d["cu"], seq_idx=d["seq_idx"],
                                  seqlen=d["seqlen"], history=d.get("hist"), has_history=d.get("hh"),
                                  activation=d["act"], dx=d["dx"], dweight=d["dw"], dbias=d["db"],
                                  want_dbias=d["db"] is not None, dhistory=d.get("dhist"),
                                  want_dhistory="dhist" in d, workspace=d["ws"])

    def ring(self, calls, k, warmup, warm_ms=0.0, wall=None):
        """Mean milliseconds per call over k back-to-back calls cycling through `calls` (zero-argument
        callables over independent buffer sets), bracketed by two HIP events on the library's stream.
        Untimed first: `warmup` calls, then whole passes until `warm_ms` of wall time have gone by
        (the clocks need some 20 ms of sustained load to settle after an idle gap).  If `wall` is a
        list, the host wall time of the timed calls (seconds) is appended to it."""
        t = self.torch
        for i in range(warmup):
            calls[i % len(calls)]()
        if warm_ms > 0:
            t0 = time.perf_counter()
            while True:
                for c in calls:
                    c()
                t.cuda.synchronize()
                if (time.perf_counter() - t0) * 1e3 >= warm_ms:
                    break
        ev0, ev1 = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        t.cuda.synchronize()
        w0 = time.perf_counter()
        ev0.record(self.stream)
        for i in range(k):
            calls[i % len(calls)]()
        ev1.record(self.stream)
        t.cuda.synchronize()
        if wall is not None:
            wall.append(time.perf_counter() - w0)
        return ev0.elapsed_time(ev1) / k

    def graph_ms(self, calls, per_graph=20, replays=10):
        """Milliseconds per call with the host out of the way: `per_graph` calls (cycling through
        `calls`) captured once into a HIP graph, replayed; for latency-bound calls, where an eager
        call costs more host time (argument checks, ctypes) than GPU time."""
        t = self.torch
        for c in calls:  # first calls outside the capture
            c()
        t.cuda.synchronize()
        side = t.cuda.Stream()
        side.wait_stream(t.cuda.current_stream())
        graph = t.cuda.CUDAGraph()
        with t.cuda.stream(side):
            with t.cuda.graph(graph, stream=side):
                for i in range(per_graph):
                    calls[i % len(calls)]()
        t.cuda.current_stream().wait_stream(side)
        for _ in range(3):
            graph.replay()
        t.cuda.synchronize()
        ev0, ev1 = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        ev0.record()
        for _ in range(replays):
            graph.replay()
        ev1.record()
        t.cuda.synchronize()
        return ev0.elapsed_time(ev1) / (replays * per_graph)

    def copy_ceiling(self, nbytes=1 << 30):
        """A plain bf16 device copy of nbytes (torch's copy kernel) under the same steady state:
        the practical HBM ceiling for a read-once / write-once stream."""
        t = self.torch
        bufs = [(t.empty(nbytes // 2, dtype=t.bfloat16, device=self.dev).normal_(),
                 t.empty(nbytes // 2, dtype=t.bfloat16, device=self.dev)) for _ in range(2)]
        ms = self.ring([lambda a=a, b=b: b.copy_(a) for a, b in bufs], 40, 0, warm_ms=WARM_MS)
        return 2 * nbytes / (ms * 1e-3) / 1e9


    def ceiling_lib(self):
        """The benchmark's copy kernels (csrc/ceiling.hip), or None when that library was not built."""
        import ctypes
        path = os.path.join(ROOT, "causal_depthwise_conv1d_width_amd", "libconv1d_ceiling.so")
        if not os.path.exists(path):
            return None
        lib = ctypes.CDLL(path)
        lib.ceiling_copy.restype = ctypes.c_int
        lib.ceiling_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                     ctypes.c_int64, ctypes.c_int, ctypes.c_int64, ctypes.c_void_p]
        st = self.stream.cuda_stream

        def call(a, b, d, shape, tr):
            rows, C = a.shape
            rc = lib.ceiling_copy(a.data_ptr(), None if b is None else b.data_ptr(), d.data_ptr(), rows, C, shape,
                                  tr, st)
            if rc != 0:
                raise RuntimeError(f"ceiling_copy returned {rc}")
        return call

    def shaped_ceilings(self, rows, C, nsets=4):
        """Hand-written copies (libconv1d_ceiling.so) moving the bytes of one forward and one
        backward call of a [rows, C] bf16 workload, timed like the convolution calls: a contiguous
        sweep (read once, write once; two reads for the backward's x and dy) and copies with the
        kernels' own access structure (the forward's short row tiles of 16 rows x 512 channels in
        row order; the backward's one round of ~1024 long row ranges with a 3-row halo, streamed
        in chunks of 4 rows as the kernel does, and of 8, and with its two reads fetched by
        direct-to-LDS 16-byte loads, a quarter of the load instructions).  None when the library
        was not built."""
        call = self.ceiling_lib()
        if call is None:
            return None
        t = self.torch
        sets = [tuple(t.empty((rows, C), dtype=t.bfloat16, device=self.dev).normal_() for _ in range(3))
                for _ in range(nsets)]

        nb1, nb2 = 2 * rows * C * 2, 3 * rows * C * 2
        res = {}
        for name, two, shape, tr in (("contiguous_1r1w", False, 0, 0), ("fwd_tiles16_1r1w", False, 1, 16),
                                     ("contiguous_2r1w", True, 0, 0), ("bwd_ranges_chunk4_2r1w", True, 2, 4),
                                     ("bwd_ranges_chunk8_2r1w", True, 2, 8), ("bwd_ranges_lds16B_2r1w", True, 3, 0)):
            ms = self.ring([lambda s=s: call(s[0], s[1] if two else None, s[2], shape, tr) for s in sets], 40, 0,
                           warm_ms=WARM_MS)
            res[name + "_GBps"] = round(gbps(nb2 if two else nb1, ms), 1)
        del sets
        return res


def gbps(nbytes, ms):
    return nbytes / (ms * 1e-3) / 1e9


# ------------------------------------------------------------------ CPU oracle baseline
def cpu_baseline(case, max_seconds=30.0):
    """The oracle as it stands (plain C loops, OpenMP over channel blocks) on the host cores: one
    warm pass, then timed passes of forward + backward until ~12 s of wall time have passed."""
    from oracle import Oracle
    o = Oracle()
    kw = dict(cu_seqlens=case.get("cu_seqlens"), seq_idx=case.get("seq_idx"), seqlen=case.get("seqlen"),
              hist=case.get("hist"), has_history=case.get("has_history"), act=case.get("act", "silu"))
    o.fwd(case["x"], case["w"], case.get("b"), **kw)
    times = []
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        o.fwd(case["x"], case["w"], case.get("b"), **kw)
        o.bwd(case["x"], case["dy"], case["w"], case.get("b"), **kw)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_start > 12.0 or len(times) >= 60 or sum(times) > max_seconds:
            break
    sec = sorted(times)[len(times) // 2]
    nbytes = fwd_bytes(case) + bwd_bytes(case)
    return {"value": round(nbytes / sec / 1e9, 3), "unit": "GB/s", "cores": o.threads(), "kind": "oracle",
            "sample": f"the full step workload (fwd + bwd over x [16384, 5632]), median of {len(times)} timed passes "
                      f"after one warm pass; {sec:.3f} s per pass, min {min(times):.3f} s",
            "cpu_model": _cpu_model(), "nproc": os.cpu_count(), "omp_num_threads": os.environ.get("OMP_NUM_THREADS")}


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


# ------------------------------------------------------------------ main
def layout_counters():
    """28 back-to-back calls of each kind over 4 buffer sets, one kind after another, so that a
    counter run can compare the channel-last kernels (the context-parallel share, x [16384, 5632])
    with the channels-first ones (x [4, 4096, 4096]), the runtime's copy of the same size and
    hand-written copies moving the channel-last calls' bytes in their access structure."""
    from causal_depthwise_conv1d_width_amd import workloads as wl
    g = Gpu()
    torch = g.torch
    c5 = wl.cp_share()
    cl = [g.prepare(c5) for _ in range(4)]
    rng = np.random.default_rng(5)
    B, D, T = 4, 4096, 4096
    w = g.taps(wl.uniform_f32(rng, (D, 4)))
    cf = []
    for _ in range(4):
        x = g.bits(wl.normal_bf16(rng, (B, D, T)))
        cf.append(dict(x=x, dy=g.bits(wl.normal_bf16(rng, (B, D, T))), y=torch.empty_like(x), dx=torch.empty_like(x),
                       dw=torch.empty((D, 4), dtype=torch.float32, device=g.dev),
                       ws=torch.empty((g.cc.conv1d_bwd_cf_workspace_bytes(B, D),), dtype=torch.uint8, device=g.dev)))
    cp = [(d["x"], torch.empty_like(d["x"])) for d in cl]
    calls = {
        "channel-last forward": [lambda d=d: g.fwd(d) for d in cl],
        "channels-first forward": [lambda d=d: g.cc.conv1d_fwd_cf(d["x"], w, out=d["y"]) for d in cf],
        "channel-last backward": [lambda d=d: g.bwd(d) for d in cl],
        "channels-first backward": [lambda d=d: g.cc.conv1d_bwd_cf(d["x"], d["dy"], w, dx=d["dx"], dweight=d["dw"],
                                                                    workspace=d["ws"]) for d in cf],
        "copy": [lambda a=a: a[1].copy_(a[0]) for a in cp],
    }
    call = g.ceiling_lib()
    if call is not None:  # hand-written copies of the channel-last calls' bytes in their access structure
        calls["forward-shaped copy (16-row tiles, 1 read)"] = [lambda d=d, a=a: call(d["x"], None, a[1], 1, 16)
                                                              for d, a in zip(cl, cp)]
        calls["backward-shaped copy (row ranges, 4-row chunks, 2 reads)"] = [
            lambda d=d, a=a: call(d["x"], d["dy"], a[1], 2, 4) for d, a in zip(cl, cp)]
        calls["backward-shaped copy through direct-to-LDS 16-byte loads (2 reads)"] = [
            lambda d=d, a=a: call(d["x"], d["dy"], a[1], 3, 0) for d, a in zip(cl, cp)]
        calls["contiguous copy (2 reads)"] = [lambda d=d, a=a: call(d["x"], d["dy"], a[1], 0, 0)
                                              for d, a in zip(cl, cp)]
    for name, cs in calls.items():
        for i in range(28):
            cs[i % 4]()
        torch.cuda.synchronize()
        print(json.dumps({"done": name, "calls": 28}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--no-extras", action="store_true", help="skip the other workloads and the copy ceiling")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-only-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB three times (counter calibration)")
    ap.add_argument("--layout-counters", action="store_true",
                    help="only run 28 calls each of the channel-last and channels-first forward and backward "
                         "and of a plain copy, one kind after another (for counter collection)")
    args = ap.parse_args()
    if args.layout_counters:
        layout_counters()
        return
    if args.copy_only_mib:
        import torch
        a = torch.empty(args.copy_only_mib << 19, dtype=torch.bfloat16, device="cuda").normal_()
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_each_way": a.numel() * 2, "copies": 3}), flush=True)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this build runs on one GPU: the multi-GPU context-parallel exchange is "
                                   "designed but not built; run with --gpus 1"}), flush=True)
        sys.exit(2)

    from causal_depthwise_conv1d_width_amd import workloads as wl
    g = Gpu()
    torch = g.torch

    case = wl.cp_share()
    sets = [g.prepare(case) for _ in range(4)]
    fb, bb = fwd_bytes(case), bwd_bytes(case)
    # step k: forward on set k % 4, backward on set (k + 2) % 4 -> consecutive calls never share data
    step_calls = []
    for k in range(4):
        step_calls.append(lambda k=k: g.fwd(sets[k]))
        step_calls.append(lambda k=k: g.bwd(sets[(k + 2) % 4]))
    walls = []
    # every ring first runs `--warmup` calls and then whole passes until WARM_MS of load have gone
    # by, all untimed: preparing the inputs leaves the GPU idle, and the clocks need some 20 ms of
    # sustained load to settle, whatever count of warm-up steps the caller asked for
    mean_step = 2 * g.ring(step_calls, 2 * args.steps, 2 * args.warmup, warm_ms=WARM_MS, wall=walls)
    wall = walls[0]
    mean_f = g.ring([lambda k=k: g.fwd(sets[k]) for k in range(4)], args.steps, 20, warm_ms=WARM_MS)
    mean_b = g.ring([lambda k=k: g.bwd(sets[k]) for k in range(4)], args.steps, 20, warm_ms=WARM_MS)
    value = gbps(fb + bb, mean_step)

    traffic = stored_traffic()
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(mean_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "storage_dtype": "bf16", "data": "synthetic",
        "config": {"workload": "context-parallel share: x [16384, 5632] bf16 in 12 fragments (8 read 3 history "
                               "rows), fp32 taps, no bias, SiLU; forward + backward (dx, dweight, d(history))",
                   "rows": 16384, "channels": 5632, "fragments": 12, "with_history": 8},
        "fwd": {"GBps": round(gbps(fb, mean_f), 1), "pct_of_peak": round(100 * gbps(fb, mean_f) / PEAK_HBM_GBPS, 2),
                "ms": round(mean_f, 4), "bytes": fb},
        "bwd": {"GBps": round(gbps(bb, mean_b), 1), "pct_of_peak": round(100 * gbps(bb, mean_b) / PEAK_HBM_GBPS, 2),
                "ms": round(mean_b, 4), "bytes": bb},
        "pct_of_peak": round(100 * value / PEAK_HBM_GBPS, 2),
        "wall_ms_per_step": round(1e3 * wall / args.steps, 4),
        "roofline": {"bound": "hbm", "kernel": "conv1d_bwd call (conv1d_bwd_kernel + conv1d_bwd_reduce_kernel)",
                     "achieved": round(gbps(bb, mean_b), 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(gbps(bb, mean_b) / PEAK_HBM_GBPS, 4),
                     "traffic": traffic, "algorithmic_bytes_per_launch": bb},
    }

    if not args.no_extras:
        extras = {"copy_ceiling_GBps": round(g.copy_ceiling(), 1)}
        ceil = g.shaped_ceilings(*case["x"].shape)
        if ceil is not None:
            extras["copy_ceilings_" + case["name"]] = ceil
            extras["copy_ceilings_rows16384_C4096"] = g.shaped_ceilings(16384, 4096)  # per-token-ID shape
        for make in (wl.single_sequence, wl.varlen_pool, wl.prefill_pool, wl.train_seq_ids):
            c = make()
            nb = fwd_bytes(c)
            nsets = int(min(8, max(2, -(-(1 << 30) // nb))))
            dd = [g.prepare(c) for _ in range(nsets)]
            if nb < (64 << 20):  # latency-bound: time replays of a captured graph (GPU time per call)
                ms = g.graph_ms([lambda d=d: g.fwd(d) for d in dd])
            else:
                ms = g.ring([lambda d=d: g.fwd(d) for d in dd], 40, 0, warm_ms=WARM_MS)
            r = {"fwd_GBps": round(gbps(nb, ms), 1), "fwd_us": round(1e3 * ms, 2), "fwd_bytes": nb}
            if c.get("dy") is not None:
                nbb = bwd_bytes(c)
                msb = g.ring([lambda d=d: g.bwd(d) for d in dd], 40, 0, warm_ms=WARM_MS)
                r.update({"bwd_GBps": round(gbps(nbb, msb), 1), "bwd_us": round(1e3 * msb, 2), "bwd_bytes": nbb})
            extras[c["name"]] = r
            del dd
            if make is wl.prefill_pool:  # decode step: one token for each of the 64 live slots of the prefill pool
                C = c["x"].shape[1]
                x1 = g.bits(c["x"][:64])
                pool = g.pool(c["pool"])
                ci = g.i32(c["cache_indices"])
                y1 = torch.empty_like(x1)
                w, b = g.taps(c["w"]), g.taps(c["b"])
                msd = g.graph_ms([lambda: g.cc.conv1d_state_update(x1, w, b, conv_state=pool, cache_indices=ci,
                                                                   out=y1)])
                nbd = 64 * C * 2 * 2 + 64 * C * 2 * 6 + 4 * C * 4 + C * 4 + 64 * 4
                extras["decode_N64_C5632"] = {"GBps": round(gbps(nbd, msd), 1), "us": round(1e3 * msd, 2),
                                              "bytes": nbd}
                # speculative step: 4 tokens for each of 64 sequences, history at the accepted offset
                K, L = 4, 6
                rng = np.random.default_rng(1006)
                xs = g.bits(wl.normal_bf16(rng, (64, K, C)))
                ys = torch.empty_like(xs)
                sp_pool = g.pool(wl.normal_bf16(rng, (128, C, L)))
                acc = g.i32(rng.integers(1, L - 1, size=64).astype(np.int32))
                mss = g.graph_ms([lambda: g.cc.conv1d_state_update_spec(xs, w, b, conv_state=sp_pool,
                                                                        cache_indices=ci, num_accepted=acc, out=ys)])
                # x and y rows, 3 history values read and K + 2 written per live channel, taps, bias, indices
                nbs = 2 * 64 * K * C * 2 + 64 * C * 2 * (3 + K + 2) + 4 * C * 4 + C * 4 + 2 * 64 * 4
                extras["spec_update_N64_K4_C5632"] = {"GBps": round(gbps(nbs, mss), 1), "us": round(1e3 * mss, 2),
                                                      "bytes": nbs}
        # filter widths 3 and 8 on the step workload: taps [C, W], W - 1 history rows per fragment
        for Wx, seed in ((3, 1008), (8, 1009)):
            rng = np.random.default_rng(seed)
            cw = dict(case)
            cw["w"] = wl.uniform_f32(rng, (case["x"].shape[1], Wx))
            cw["hist"] = wl.normal_bf16(rng, (case["hist"].shape[0], Wx - 1, case["x"].shape[1]))
            dw_sets = [g.prepare(cw) for _ in range(4)]
            nfw, nbw = fwd_bytes(cw), bwd_bytes(cw)
            msfw = g.ring([lambda d=d: g.fwd(d) for d in dw_sets], 40, 0, warm_ms=WARM_MS)
            msbw = g.ring([lambda d=d: g.bwd(d) for d in dw_sets], 40, 0, warm_ms=WARM_MS)
            extras[f"width{Wx}_" + case["name"]] = {"fwd_GBps": round(gbps(nfw, msfw), 1),
                                                   "fwd_us": round(1e3 * msfw, 2), "fwd_bytes": nfw,
                                                   "bwd_GBps": round(gbps(nbw, msbw), 1),
                                                   "bwd_us": round(1e3 * msbw, 2), "bwd_bytes": nbw}
            del dw_sets
        # channels-first [B, D, T]: the per-token-ID training shape (4 x 4096 x 4096), one sequence per row
        rng = np.random.default_rng(1007)
        B, D, T = 4, 4096, 4096
        wcf = g.taps(wl.uniform_f32(rng, (D, 4)))
        bcf = g.taps((rng.standard_normal(D) * 0.1).astype(np.float32))
        cfs = []
        for _ in range(4):
            xcf = g.bits(wl.normal_bf16(rng, (B, D, T)))
            cfs.append(dict(x=xcf, dy=g.bits(wl.normal_bf16(rng, (B, D, T))), y=torch.empty_like(xcf),
                            dx=torch.empty_like(xcf), dw=torch.empty((D, 4), dtype=torch.float32, device=g.dev),
                            db=torch.empty((D,), dtype=torch.float32, device=g.dev),
                            ws=torch.empty((g.cc.conv1d_bwd_cf_workspace_bytes(B, D),), dtype=torch.uint8,
                                           device=g.dev)))
        nbf = B * D * T * 2 * 2 + D * 16 + D * 4
        nbb = B * D * T * 2 * 3 + D * 16 + D * 4 + D * 16 + D * 4
        msf = g.ring([lambda d=d: g.cc.conv1d_fwd_cf(d["x"], wcf, bcf, out=d["y"]) for d in cfs], 40, 0, warm_ms=WARM_MS)
        msb = g.ring([lambda d=d: g.cc.conv1d_bwd_cf(d["x"], d["dy"], wcf, bcf, dx=d["dx"], dweight=d["dw"],
                                                     dbias=d["db"], want_dbias=True, workspace=d["ws"])
                      for d in cfs], 40, 0, warm_ms=WARM_MS)
        extras["channels_first_B4_D4096_T4096"] = {"fwd_GBps": round(gbps(nbf, msf), 1), "fwd_us": round(1e3 * msf, 2),
                                                   "fwd_bytes": nbf, "bwd_GBps": round(gbps(nbb, msb), 1),
                                                   "bwd_us": round(1e3 * msb, 2), "bwd_bytes": nbb}
        del cfs
        out["workloads"] = extras
        out["step_workload"] = case["name"]
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(case)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
