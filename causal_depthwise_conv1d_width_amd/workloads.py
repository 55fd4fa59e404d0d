"""Seeded synthetic inputs shaped like the pages' workloads.

This module only draws random numbers and lays out metadata; it holds none of the convolution's
arithmetic.  Both the GPU tests / benchmark and the CPU oracle consume exactly the bits it
produces.  bf16 tensors are numpy ``uint16`` arrays of bit patterns (round-to-nearest-even of a
float32 draw); FP32 taps and biases are ``float32``.

Every workload draws from its own ``numpy.random.default_rng`` seed (PCG64) in the order the code
reads.  The shapes follow the workload list of the packed causal conv1d pages:
  single_sequence   one sequence, T = 64, C = 64, FP32 taps + bias, zero history, SiLU (seed 1001);
  varlen_pool       eight packed sequences (lengths uniform in 0..512, one forced empty), C = 2048,
                    bf16 taps, no bias, slot pool [16, C, 4] with one -1 sentinel and random
                    has_initial_state (seed 1002);
  prefill_pool      32768 rows (last 256 padding), 64 lognormal-length sequences (median 256)
                    summing to 32512, C = 5632 (the GDP channel count 2048*2 + 4*128*2 + 4*128),
                    FP32 taps + bias, pool [128, C, 4], every sequence with initial state (seed 1003);
  train_seq_ids     training: 4 x 4096 rows, C = 4096, 1-8 documents per batch row marked by
                    per-token IDs, FP32 taps + bias, dy ~ N(0, 1) (seed 1004);
  cp_share          context-parallel share: 16384 rows, C = 5632, 12 fragments at random cut
                    points, 8 of which read 3 caller history rows, FP32 taps, no bias, dy ~ N(0, 1)
                    (seed 1005).
"""
import numpy as np

GDP_CHANNELS = 2048 * 2 + 4 * 128 * 2 + 4 * 128  # V(d_inner*M) + K(ngroups*d_state*M) + Q(ngroups*d_state)
OUT_FILL = 0x7FC1  # a NaN pattern the kernels never produce: marks rows that must stay untouched


def to_bf16_bits(a):
    """float32 -> bf16 bit patterns, round to nearest even (inputs are finite)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    lsb = (u >> 16) & np.uint32(1)
    r = u + np.uint32(0x7FFF)  # no uint32 overflow for finite values
    r += lsb
    return (r >> 16).astype(np.uint16)


def bf16_bits_to_f32(b):
    """bf16 bit patterns -> float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_bf16(rng, shape, sigma=1.0):
    return to_bf16_bits(rng.standard_normal(size=shape, dtype=np.float32) * np.float32(sigma))


def uniform_f32(rng, shape, lo=-0.5, hi=0.5):
    return rng.uniform(lo, hi, size=shape).astype(np.float32)


def pool_layout(values, layout):
    """Return a [slots, C, L] uint16 array holding `values` in the requested memory layout:
    'hist' = history axis contiguous (plain C order), 'chan' = channel axis contiguous."""
    if layout == "hist":
        return np.ascontiguousarray(values)
    if layout == "chan":
        return np.ascontiguousarray(values.transpose(0, 2, 1)).transpose(0, 2, 1)
    raise ValueError(layout)


def single_sequence():
    rng = np.random.default_rng(1001)
    T, C = 64, 64
    x = normal_bf16(rng, (T, C))
    w = uniform_f32(rng, (C, 4))
    b = (rng.standard_normal(C) * 0.1).astype(np.float32)
    return dict(name="single_seq_T64_C64", x=x, w=w, b=b,
                cu_seqlens=np.array([0, T], dtype=np.int32), act="silu")


def varlen_pool(layout="hist"):
    rng = np.random.default_rng(1002)
    N, C, slots, L = 8, 2048, 16, 4
    lengths = rng.integers(0, 513, size=N)
    empty = int(rng.integers(0, N))
    lengths[empty] = 0
    rows = int(lengths.sum())
    cu = np.zeros(N + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    x = normal_bf16(rng, (rows, C))
    w = to_bf16_bits(uniform_f32(rng, (C, 4)))
    pool = pool_layout(normal_bf16(rng, (slots, C, L)), layout)
    ci = rng.permutation(slots)[:N].astype(np.int32)
    nonempty = [i for i in range(N) if lengths[i] > 0]
    sentinel = int(nonempty[int(rng.integers(0, len(nonempty)))])
    ci[sentinel] = -1
    live_nonempty = [i for i in nonempty if i != sentinel]
    while True:  # both has_initial_state values must occur among live nonempty sequences
        hi = rng.random(N) < 0.5
        if len({bool(hi[i]) for i in live_nonempty}) == 2:
            break
    return dict(name=f"varlen_N8_C2048_pool16_{layout}", x=x, w=w, b=None, cu_seqlens=cu,
                pool=pool, cache_indices=ci, has_initial_state=hi.astype(np.uint8), act="silu",
                empty=empty, sentinel=sentinel)


def lognormal_lengths(rng, n, total, median=256.0, sigma=1.17):
    raw = rng.lognormal(np.log(median), sigma, size=n)
    lengths = np.maximum(1, np.floor(raw * total / raw.sum())).astype(np.int64)
    lengths[int(np.argmax(lengths))] += total - int(lengths.sum())
    assert lengths.min() >= 1 and int(lengths.sum()) == total
    return lengths


def prefill_pool():
    rng = np.random.default_rng(1003)
    N, rows, valid, C, slots, L = 64, 32768, 32512, GDP_CHANNELS, 128, 4
    lengths = lognormal_lengths(rng, N, valid)
    cu = np.zeros(N + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    x = normal_bf16(rng, (rows, C))
    w = uniform_f32(rng, (C, 4))
    b = (rng.standard_normal(C) * 0.1).astype(np.float32)
    pool = normal_bf16(rng, (slots, C, L))
    ci = rng.permutation(slots)[:N].astype(np.int32)
    hi = np.ones(N, dtype=np.uint8)
    return dict(name="prefill_rows32768_N64_C5632_pool128", x=x, w=w, b=b, cu_seqlens=cu,
                pool=pool, cache_indices=ci, has_initial_state=hi, act="silu")


def docs_seq_idx(rng, B, T, max_docs=8):
    """Per-token sequence IDs: a global counter that increases at every document start and at
    every batch-row start; 1..max_docs documents per row at distinct sorted cut points."""
    ids = np.empty(B * T, dtype=np.int32)
    nxt = 0
    for r in range(B):
        n_docs = int(rng.integers(1, max_docs + 1))
        cuts = np.sort(rng.choice(np.arange(1, T), size=n_docs - 1, replace=False))
        bounds = [0, *cuts.tolist(), T]
        for d in range(n_docs):
            ids[r * T + bounds[d]: r * T + bounds[d + 1]] = nxt
            nxt += 1
    return ids


def train_seq_ids():
    rng = np.random.default_rng(1004)
    B, T, C = 4, 4096, 4096
    seq_idx = docs_seq_idx(rng, B, T)
    x = normal_bf16(rng, (B * T, C))
    w = uniform_f32(rng, (C, 4))
    b = (rng.standard_normal(C) * 0.1).astype(np.float32)
    dy = normal_bf16(rng, (B * T, C))
    return dict(name="train_B4_T4096_C4096_seqidx", x=x, w=w, b=b, seq_idx=seq_idx,
                seqlen=T, dy=dy, act="silu")


def cp_share():
    rng = np.random.default_rng(1005)
    S, C, nfrag, nhist = 16384, GDP_CHANNELS, 12, 8
    cuts = np.sort(rng.choice(np.arange(1, S), size=nfrag - 1, replace=False))
    cu = np.array([0, *cuts.tolist(), S], dtype=np.int32)
    has_hist = np.zeros(nfrag, dtype=np.uint8)
    has_hist[rng.choice(nfrag, size=nhist, replace=False)] = 1
    hist = normal_bf16(rng, (nfrag, 3, C))
    x = normal_bf16(rng, (S, C))
    w = uniform_f32(rng, (C, 4))
    dy = normal_bf16(rng, (S, C))
    return dict(name="cp_share_S16384_C5632_12frag", x=x, w=w, b=None, cu_seqlens=cu,
                hist=hist, has_history=has_hist, dy=dy, act="silu")


# every workload, in the order of the list above
WORKLOADS = (single_sequence, varlen_pool, prefill_pool, train_seq_ids, cp_share)


def random_case(rng, *, C=None, nseq=None, max_len=10, mode="cu", pool_layout_name=None,
                slots=None, L=3, with_hist=False, w_f32=True, bias=None, act="silu",
                pad_rows=None, force_empty=False, sentinel=False):
    """A small random packed problem for sweeps: returns the same dict layout as the configs.

    mode: "cu" (offsets), "idx" (per-token IDs inside batch rows) or "batch" (nseq batch rows of one
    sequence each, no offsets or IDs); pools and history rows need "cu" or "batch"."""
    if C is None:
        C = int(rng.choice([1, 3, 8, 13, 64]))
    if nseq is None:
        nseq = int(rng.integers(0, 7))
    d = dict(name="random", act=act)
    if mode == "cu":
        lengths = rng.integers(0, max_len + 1, size=nseq)
        if force_empty and nseq > 0:
            lengths[int(rng.integers(0, nseq))] = 0
        cu = np.zeros(nseq + 1, dtype=np.int32)
        cu[1:] = np.cumsum(lengths)
        pad = int(rng.integers(0, 3)) if pad_rows is None else pad_rows
        rows = int(cu[-1]) + pad
        d["cu_seqlens"] = cu
    elif mode == "batch":  # neither offsets nor IDs: every batch row of T rows is one sequence
        nseq = max(nseq, 1)
        T = int(rng.integers(1, max_len + 1))
        d["seqlen"] = T
        rows = nseq * T
    else:  # "idx": per-token IDs inside batch rows
        B = int(rng.integers(1, 4))
        T = int(rng.integers(1, max_len + 1))
        d["seq_idx"] = docs_seq_idx(rng, B, T, max_docs=min(4, T)) if T > 1 else np.arange(B, dtype=np.int32)
        d["seqlen"] = T
        rows = B * T
    d["x"] = normal_bf16(rng, (rows, C))
    d["w"] = uniform_f32(rng, (C, 4)) if w_f32 else to_bf16_bits(uniform_f32(rng, (C, 4)))
    if bias is None:
        bias = bool(rng.integers(0, 2))
    if bias:
        bf = (rng.standard_normal(C) * 0.1).astype(np.float32)
        d["b"] = bf if rng.integers(0, 2) else to_bf16_bits(bf)
    else:
        d["b"] = None
    if mode in ("cu", "batch") and pool_layout_name is not None:
        slots = slots if slots is not None else nseq + 2
        d["pool"] = pool_layout(normal_bf16(rng, (slots, C, L)), pool_layout_name)
        ci = rng.permutation(slots)[:nseq].astype(np.int32)
        if sentinel and nseq > 0:
            ci[int(rng.integers(0, nseq))] = -1
        d["cache_indices"] = ci
        d["has_initial_state"] = (rng.random(nseq) < 0.5).astype(np.uint8)
    if mode in ("cu", "batch") and with_hist:
        d["hist"] = normal_bf16(rng, (nseq, 3, C))
        d["has_history"] = (rng.random(nseq) < 0.6).astype(np.uint8)
    d["dy"] = normal_bf16(rng, (rows, C))
    return d
