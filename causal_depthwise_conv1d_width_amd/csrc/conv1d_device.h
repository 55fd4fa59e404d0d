// conv1d_device.h -- device-side building blocks of the gfx950 kernels (library-internal).
//
// Data layout: activations are channel-last bf16 rows.  One lane owns CPL consecutive channels
// of a row (CPL = 2: one 4-byte load per row), a 64-lane wave covers 64*CPL channels of the same
// row, and the waves of a block sit side by side, so one row access of a block is one
// contiguous, fully coalesced segment of kBlockChannels*2 bytes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "conv1d_launch.h"

namespace cconv {

constexpr int kWave = 64;

// f(integral_constant<int, 0>), ..., f(integral_constant<int, N-1>): a loop whose index must stay
// a compile-time constant (it picks a register buffer) however large the body is.
template <int N, int I = 0, class F>
__device__ __forceinline__ void unroll_steps(F& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    unroll_steps<N, I + 1>(f);
  }
}

// ------------------------------------------------------------------ bf16 packing
template <int CPL>
struct Pk {
  uint32_t d[CPL / 2];  // CPL bf16 values, two per dword, channel order low half first
};

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2_a4 __attribute__((ext_vector_type(2), aligned(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// Two FP32 values -> two bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

template <int CPL>
__device__ __forceinline__ void unpack(const Pk<CPL>& p, float (&f)[CPL]) {
#pragma unroll
  for (int j = 0; j < CPL / 2; ++j) {
    f[2 * j] = bf16_lo(p.d[j]);
    f[2 * j + 1] = bf16_hi(p.d[j]);
  }
}

template <int CPL>
__device__ __forceinline__ Pk<CPL> pack(const float (&f)[CPL]) {
  Pk<CPL> p;
#pragma unroll
  for (int j = 0; j < CPL / 2; ++j) p.d[j] = pack_bf16x2(f[2 * j], f[2 * j + 1]);
  return p;
}

template <int CPL>
__device__ __forceinline__ Pk<CPL> zero_pk() {
  Pk<CPL> p;
#pragma unroll
  for (int j = 0; j < CPL / 2; ++j) p.d[j] = 0u;
  return p;
}

// ------------------------------------------------------------------ row loads / stores
#ifndef CCONV_NT_LOADS
#define CCONV_NT_LOADS 1
#endif
#ifndef CCONV_NT_STORES
#define CCONV_NT_STORES 1
#endif
// VEC: an active lane's CPL channels are one vector access.  At CPL = 8 / 4 that needs C % CPL == 0
// and 16- / 8-byte aligned row starts.  At CPL = 2 any row start will do: the pair is one dword
// access at a 2-byte aligned address, which the hardware serves in the unaligned access mode that
// the HSA runtime sets (the compiler emits the same single dword instruction for either alignment).
// Otherwise element-wise with bounds.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32_a2 __attribute__((aligned(2)));

// STREAM: the row is read exactly once here (non-temporal hint: do not keep it in the caches).
template <int CPL, bool VEC, bool STREAM = false>
__device__ __forceinline__ Pk<CPL> load_row(const uint16_t* __restrict__ row, int64_t c0, int64_t C) {
  Pk<CPL> p;
  if constexpr (VEC) {
    if constexpr (CPL == 8) {
      const u32x4* src = reinterpret_cast<const u32x4*>(row + c0);
      u32x4 v;
      if constexpr (STREAM && CCONV_NT_LOADS) v = __builtin_nontemporal_load(src);
      else v = *src;
      p.d[0] = v.x; p.d[1] = v.y; p.d[2] = v.z; p.d[3] = v.w;
    } else if constexpr (CPL == 4) {
      const u32x2* src = reinterpret_cast<const u32x2*>(row + c0);
      u32x2 v;
      if constexpr (STREAM && CCONV_NT_LOADS) v = __builtin_nontemporal_load(src);
      else v = *src;
      p.d[0] = v.x; p.d[1] = v.y;
    } else {
      const u32_a2* src = reinterpret_cast<const u32_a2*>(row + c0);
      if constexpr (STREAM && CCONV_NT_LOADS) p.d[0] = __builtin_nontemporal_load(src);
      else p.d[0] = *src;
    }
  } else {
#pragma unroll
    for (int j = 0; j < CPL / 2; ++j) {
      const uint32_t lo = (c0 + 2 * j < C) ? row[c0 + 2 * j] : 0u;
      const uint32_t hi = (c0 + 2 * j + 1 < C) ? row[c0 + 2 * j + 1] : 0u;
      p.d[j] = lo | (hi << 16);
    }
  }
  return p;
}

template <int CPL, bool VEC, bool STREAM = false>
__device__ __forceinline__ void store_row(uint16_t* __restrict__ row, int64_t c0, int64_t C, const Pk<CPL>& p) {
  if constexpr (VEC) {
    if constexpr (CPL == 8) {
      u32x4 v = {p.d[0], p.d[1], p.d[2], p.d[3]};
      u32x4* dst = reinterpret_cast<u32x4*>(row + c0);
      if constexpr (STREAM && CCONV_NT_STORES) __builtin_nontemporal_store(v, dst);
      else *dst = v;
    } else if constexpr (CPL == 4) {
      u32x2 v = {p.d[0], p.d[1]};
      u32x2* dst = reinterpret_cast<u32x2*>(row + c0);
      if constexpr (STREAM && CCONV_NT_STORES) __builtin_nontemporal_store(v, dst);
      else *dst = v;
    } else {
      u32_a2* dst = reinterpret_cast<u32_a2*>(row + c0);
      if constexpr (STREAM && CCONV_NT_STORES) __builtin_nontemporal_store(p.d[0], dst);
      else *dst = p.d[0];
    }
  } else {
#pragma unroll
    for (int j = 0; j < CPL / 2; ++j) {
      if (c0 + 2 * j < C) row[c0 + 2 * j] = (uint16_t)(p.d[j] & 0xffffu);
      if (c0 + 2 * j + 1 < C) row[c0 + 2 * j + 1] = (uint16_t)(p.d[j] >> 16);
    }
  }
}

// ------------------------------------------------------------------ taps
// Window geometry of filter width W: a ring of R register slots (R = 4 up to W = 4, R = 8 up to
// W = 8) and H = R - 1 history values.  The taps [C, W] sit in the last W of R slots,
// wk[R-W .. R-1] (slot R-1 on the current row); the leading R-W slots hold zeros and every loop
// over taps starts at R-W, so they are never multiplied.  Widths up to four keep the four-slot
// ring, so their code does not change with the wider form.
template <int W>
struct Win {
  static_assert(W >= 2 && W <= 8, "filter widths 2..8");
  static constexpr int R = W <= 4 ? 4 : 8;
  static constexpr int H = R - 1;
};

__device__ __forceinline__ float tap_f32(float v) { return v; }
__device__ __forceinline__ float tap_f32(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }
struct NoBias {};

// The taps and bias of one dtype pair, straight-line: TB = NoBias reads no bias.
template <typename TW, typename TB, int CPL, int W, int R>
__device__ __forceinline__ void load_taps_typed(const void* w, const void* b, const int64_t (&cc)[CPL],
                                                float (&wk)[R][CPL], float (&bias)[CPL]) {
#pragma unroll
  for (int ch = 0; ch < CPL; ++ch) {
    if constexpr (__is_same(TB, NoBias)) bias[ch] = 0.f;
    else bias[ch] = tap_f32(static_cast<const TB*>(b)[cc[ch]]);
#pragma unroll
    for (int k = 0; k < W; ++k) wk[R - W + k][ch] = tap_f32(static_cast<const TW*>(w)[cc[ch] * W + k]);
  }
}

// Every load reads an in-range channel (a lane's channels past the last one read channel C-1, and
// their values are then replaced by zeros), and the dtypes are tested once for the wave, so all the
// loads go out together and the set-up waits for them once.  A load per tap inside a per-lane test
// made every bf16 tap its own memory round trip.
template <int CPL, int W = 4, int R = Win<W>::R>
__device__ __forceinline__ void load_taps(const void* w, int w_f32, const void* b, int b_f32, int64_t c0,
                                          int64_t C, float (&wk)[R][CPL], float (&bias)[CPL]) {
  bool ok[CPL];
  int64_t cc[CPL];
#pragma unroll
  for (int ch = 0; ch < CPL; ++ch) {
    ok[ch] = c0 + ch < C;
    cc[ch] = ok[ch] ? c0 + ch : C - 1;
  }
#pragma unroll
  for (int k = 0; k < R - W; ++k)
#pragma unroll
    for (int ch = 0; ch < CPL; ++ch) wk[k][ch] = 0.f;
  if (w_f32) {
    if (!b) load_taps_typed<float, NoBias, CPL, W, R>(w, b, cc, wk, bias);
    else if (b_f32) load_taps_typed<float, float, CPL, W, R>(w, b, cc, wk, bias);
    else load_taps_typed<float, uint16_t, CPL, W, R>(w, b, cc, wk, bias);
  } else {
    if (!b) load_taps_typed<uint16_t, NoBias, CPL, W, R>(w, b, cc, wk, bias);
    else if (b_f32) load_taps_typed<uint16_t, float, CPL, W, R>(w, b, cc, wk, bias);
    else load_taps_typed<uint16_t, uint16_t, CPL, W, R>(w, b, cc, wk, bias);
  }
#pragma unroll
  for (int ch = 0; ch < CPL; ++ch) {
    if (!ok[ch]) {
#pragma unroll
      for (int k = R - W; k < R; ++k) wk[k][ch] = 0.f;
      bias[ch] = 0.f;
    }
  }
}

// H-row window w = [oldest, ..., newest]: drop the oldest, append row p.  Windows are built by
// shifting rows into the sequence history (never by a runtime register index).
template <int CPL, int H = 3>
__device__ __forceinline__ void shift_in(float (&w)[H][CPL], const Pk<CPL>& p) {
  float f[CPL];
  unpack(p, f);
#pragma unroll
  for (int ch = 0; ch < CPL; ++ch) {
#pragma unroll
    for (int j = 0; j + 1 < H; ++j) w[j][ch] = w[j + 1][ch];
    w[H - 1][ch] = f[ch];
  }
}

// Rows t-H .. t-1 (those >= 0), loaded before the sequence lookup says how many of them belong
// to t's sequence, so the lookup, these loads and the first chunk share one memory round trip;
// shift_window keeps only the last `dist` of them.
template <int CPL, bool VEC, int H = 3>
__device__ __forceinline__ void load_window(Pk<CPL> (&p)[H], const uint16_t* __restrict__ x, int64_t ld, int64_t t,
                                            int64_t c0, int64_t C, bool active) {
#pragma unroll
  for (int j = 0; j < H; ++j) {
    p[j] = zero_pk<CPL>();
    if (active && t - H + j >= 0) p[j] = load_row<CPL, VEC>(x + (t - H + j) * ld, c0, C);
  }
}

// h = the sequence's history positions 0..H-1; shift in the window rows load_window fetched.
template <int CPL, int H = 3>
__device__ __forceinline__ void shift_window(float (&h)[H][CPL], const Pk<CPL> (&p)[H], int64_t dist) {
#pragma unroll
  for (int j = 0; j < H; ++j)
    if (j >= H - dist) shift_in<CPL, H>(h, p[j]);
}

// ------------------------------------------------------------------ activation
// sigmoid via the hardware exp2 and reciprocal (about 1 ulp each): far below bf16 rounding.
__device__ __forceinline__ float sigmoid_f32(float z) {
  return __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

// ------------------------------------------------------------------ XCD-aware block order
// Workgroups are dealt round-robin to the 8 XCDs (each with its own L2).  Logical tiles are
// ordered row-range major (tile = row_range * n_strips + strip), so the channel strips of the
// same rows, which share DRAM pages, run side by side.  xcd_tile gives every XCD one contiguous
// range of logical tiles, so neighbouring row tiles of a strip (which share halo rows) run on the
// same XCD at about the same time; block_tile picks between that and the other orders of a
// launch (kOrder* in conv1d_launch.h).
__device__ __forceinline__ void tile_coords(uint32_t tile, uint32_t n_strips, uint32_t& strip, uint32_t& rb) {
  strip = tile % n_strips;
  rb = tile / n_strips;
}

__device__ __forceinline__ uint32_t xcd_tile(uint32_t b, uint32_t nb) {
  constexpr uint32_t X = 8;
  const uint32_t q = nb / X, r = nb % X, xcd = b % X, idx = b / X;
  return (xcd < r) ? xcd * (q + 1) + idx : r * (q + 1) + (xcd - r) * q + idx;
}

// This block's (strip, row block) in a launch of n_strips x n_rowblocks blocks, by tile order.
__device__ __forceinline__ void block_tile(uint32_t order, uint32_t n_strips, uint32_t n_rowblocks, uint32_t& strip,
                                           uint32_t& rb) {
  if (order == kOrderPlain) {
    tile_coords(blockIdx.x, n_strips, strip, rb);
    return;
  }
  const uint32_t t = xcd_tile(blockIdx.x, gridDim.x);
  if (order == kOrderXcdStrips) {
    strip = t / n_rowblocks;
    rb = t % n_rowblocks;
  } else {
    tile_coords(t, n_strips, strip, rb);
  }
}

// ------------------------------------------------------------------ integer helpers
// x / L and x mod L for x >= 0, L >= 1 (wave-uniform values): one 32-bit division when both fit
// (every row count here in practice), the 64-bit sequence otherwise.
__device__ __forceinline__ int64_t udiv64(int64_t x, int64_t L) {
  if ((((uint64_t)x | (uint64_t)L) >> 32) == 0) return (int64_t)((uint32_t)x / (uint32_t)L);
  return x / L;
}
__device__ __forceinline__ int64_t umod64(int64_t x, int64_t L) {
  if ((((uint64_t)x | (uint64_t)L) >> 32) == 0) return (int64_t)((uint32_t)x % (uint32_t)L);
  return x % L;
}
// position of row x in its batch row of L rows, for any x >= -L (rows before the first are taken
// modulo L as well)
__device__ __forceinline__ int64_t batch_pos(int64_t x, int64_t L) {
  if (x >= 0) return umod64(x, L);
  const int64_t m = umod64(-x, L);
  return m == 0 ? 0 : L - m;
}

// ------------------------------------------------------------------ sequence walking
// All row indices below are wave-uniform: every lane of a wave works on the same row.
struct SeqDesc {
  int64_t s, e;  // rows [s, e) of the sequence (IDX mode: e exact up to the scan limit)
  int64_t idx;   // sequence index (CU / BATCH modes), -1 in IDX mode
};

// Last row (exclusive) that belongs to some sequence, clamped to [0, rows].
template <int MODE>
__device__ __forceinline__ int64_t data_end(const SeqArgs& q, int64_t rows) {
  if constexpr (MODE == MODE_CU) {
    int64_t e = q.cu[q.nseq];
    return e < 0 ? 0 : (e > rows ? rows : e);
  } else {
    return rows;
  }
}

__device__ __forceinline__ int64_t cu_at(const SeqArgs& q, int64_t i, int64_t dend) {
  int64_t v = q.cu[i];
  return v < 0 ? 0 : (v > dend ? dend : v);
}

// IDX mode: first sequence start in (t, limit), or limit (t >= 0).  64 rows per step, one row per
// lane; the batch-row position of each step's first row is kept as a scalar, so a lane tests the
// batch-row start with an add and a compare.
__device__ __forceinline__ int64_t idx_next_start(const SeqArgs& q, int64_t t, int64_t limit) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t L = q.seqlen;
  int64_t m0 = umod64(t + 1, L);  // batch-row position of row t + 1
  for (int64_t base = t + 1; base < limit; base += kWave) {
    const int64_t r = base + lane;
    bool st = false;
    if (r < limit) {
      const int64_t pos = m0 + lane;
      const bool bstart = L >= kWave ? (pos == 0 || pos == L) : (umod64(pos, L) == 0);
      st = bstart || (q.seq_idx[r] != q.seq_idx[r - 1]);
    }
    const uint64_t m = __ballot(st);
    if (m) return base + (int64_t)__builtin_ctzll(m);
    m0 = umod64(m0 + kWave, L);
  }
  return limit;
}

// The sequence containing row t (t < dend), in two phases so that a kernel can issue the lookup's
// first loads before its row loads and use them after: seq_probe issues them (the first level of
// the offset search, or the IDs around row t), seq_resolve finishes the lookup with their values.
// `limit` bounds the IDX-mode forward scan.  seq_of_row does both at once.
// Up to kDualSeqs sequences the offset search is a single level of two offsets per lane.
constexpr int64_t kDualSeqs = 2 * kWave - 2;

struct SeqProbe {
  int32_t v, w;    // CU: raw offsets 2l and 2l+1 (up to kDualSeqs sequences), else the first
                   // search level's offset; IDX: IDs of rows r and r - 1
  int32_t s0, s1;  // with a slot array: the slots of sequences 2l and 2l+1 (CU form, up to
                   // kDualSeqs sequences), or of row t's batch row on every lane (BATCH form)
};

// `slots` (the pool's cache_indices, or nullptr): fetch the slot with the lookup, so that a tile
// knows its sequence's slot after one memory round trip (probe_slot).
template <int MODE, int HB = 3>
__device__ __forceinline__ SeqProbe seq_probe(const SeqArgs& q, int64_t t, int64_t limit,
                                              const int32_t* slots = nullptr) {
  SeqProbe p{0, 0, -1, -1};
  const int lane = threadIdx.x & (kWave - 1);
  if constexpr (MODE == MODE_CU) {
    const int64_t n = q.nseq;
    if (n <= kDualSeqs) {
      const int64_t o0 = 2 * (int64_t)lane, o1 = o0 + 1;
      if (o0 <= n) p.v = q.cu[o0];
      if (o1 <= n) p.w = q.cu[o1];
      if (slots) {
        if (o0 < n) p.s0 = slots[o0];
        if (o1 < n) p.s1 = slots[o1];
      }
    } else {
      const int64_t stride = (n + kWave - 2) / (kWave - 1);
      const int64_t off = (int64_t)lane * stride;
      if (off <= n) p.v = q.cu[off];
    }
  } else if constexpr (MODE == MODE_BATCH) {
    if (slots && q.seqlen > 0) {
      const int64_t i = udiv64(t, q.seqlen);
      if (i < q.nseq) p.s0 = slots[i];
    }
  } else if constexpr (MODE == MODE_IDX) {
    // lane l reads the IDs of row r = t - HB + l and of the row before it (pure loads: whether r
    // starts a batch row is worked out in seq_resolve)
    const int64_t r = t - HB + lane;
    if (r >= 0 && (lane <= HB || r < limit)) {
      p.v = q.seq_idx[r];
      p.w = r >= 1 ? q.seq_idx[r - 1] : ~p.v;
    }
  }
  return p;
}

template <int MODE, int HB = 3>
__device__ __forceinline__ SeqDesc seq_resolve(const SeqArgs& q, int64_t t, int64_t dend, int64_t limit,
                                               const SeqProbe& p) {
  SeqDesc d;
  const int lane = threadIdx.x & (kWave - 1);
  if constexpr (MODE == MODE_CU) {
    // largest i in [0, nseq) with cu[i] <= t.  Up to kDualSeqs sequences lane l holds cu[2l] and
    // cu[2l+1] from the probe: two ballots give the answer and its end offset at once.  Beyond,
    // a 64-ary search: lane l reads cu[lo + l*stride] (one load per lane per level; the first
    // level's values come from the probe), the highest lane whose offset is <= t narrows the
    // interval.  Lane 0 is taken as the floor without a test, as the offsets start at 0.  The
    // last level also hands over cu[i + 1] from the next lane.
    int64_t lo = 0, n = q.nseq;  // the answer lies in [lo, lo + n)
    bool first = true;
    if (n <= kDualSeqs) {
      const int64_t o0 = 2 * (int64_t)lane, o1 = o0 + 1;
      const int32_t hi = (int32_t)dend;
      const int32_t v0 = o0 <= n ? (p.v < 0 ? 0 : (p.v > hi ? hi : p.v)) : 0;
      const int32_t v1 = o1 <= n ? (p.w < 0 ? 0 : (p.w > hi ? hi : p.w)) : 0;
      const uint64_t m0 = __ballot(lane == 0 || (o0 < n && v0 <= t));
      const uint64_t m1 = __ballot(o1 < n && v1 <= t);
      const int k0 = 63 - __builtin_clzll(m0);
      const int k1 = m1 ? 63 - __builtin_clzll(m1) : -1;
      if (k1 >= k0) {  // sequence 2 k1 + 1 (< n, so lane k1 + 1 <= 63 holds its end)
        d.idx = 2 * (int64_t)k1 + 1;
        d.s = __builtin_amdgcn_readlane(v1, k1);
        d.e = __builtin_amdgcn_readlane(v0, k1 + 1 < kWave ? k1 + 1 : k1);
      } else {  // sequence 2 k0
        d.idx = 2 * (int64_t)k0;
        d.s = __builtin_amdgcn_readlane(v0, k0);
        d.e = __builtin_amdgcn_readlane(v1, k0);
      }
      if (d.e <= t) d.e = t + 1;  // only for metadata that breaks the contract: stay in bounds
      return d;
    }
    while (true) {
      const int64_t stride = n < kWave ? 1 : (n + kWave - 2) / (kWave - 1);
      const int64_t off = (int64_t)lane * stride;
      int32_t v = 0;
      if (off <= n) {  // lo + n <= nseq: in bounds; offsets are clamped into [0, dend]
        const int64_t raw = first ? (int64_t)p.v : (int64_t)q.cu[lo + off];
        v = (int32_t)(raw < 0 ? 0 : (raw > dend ? dend : raw));
      }
      first = false;
      const uint64_t m = __ballot(lane == 0 || (off < n && v <= t));
      const int k = 63 - __builtin_clzll(m);
      if (stride == 1) {
        d.idx = lo + k;
        d.s = __builtin_amdgcn_readlane(v, k);  // k is wave-uniform: scalar results
        d.e = __builtin_amdgcn_readlane(v, k + 1 < kWave ? k + 1 : k);
        break;
      }
      lo += (int64_t)k * stride;
      n = n - (int64_t)k * stride < stride ? n - (int64_t)k * stride : stride;
    }
    if (d.e <= t) d.e = t + 1;  // only for metadata that breaks the contract: stay in bounds
  } else if constexpr (MODE == MODE_BATCH) {
    d.idx = udiv64(t, q.seqlen);
    d.s = d.idx * q.seqlen;
    d.e = d.s + q.seqlen;
    if (d.e > dend) d.e = dend;
  } else {
    // only the distance to the sequence start up to HB (the history length) matters
    // (d.s = t - min(dist, HB)), and the next start below `limit`: lane l tests row t - HB + l,
    // one pass covers rows t-HB .. t+63-HB.  A row starts a sequence where it starts a batch row
    // (its position there, lane 0's plus the lane, is a multiple of seqlen) or its ID differs.
    const int64_t L = q.seqlen;
    const int64_t r = t - HB + lane;
    const int64_t pos = batch_pos(t - HB, L) + lane;
    const bool bstart = L >= kWave ? (pos == 0 || pos == L) : (umod64(pos, L) == 0);
    const bool valid = r >= 0 && (lane <= HB || r < limit);
    const uint64_t m = __ballot(valid && (bstart || p.v != p.w));
    const uint64_t back = m & (((1ull << HB) - 1) << 1);  // rows t-HB+1 .. t
    const int64_t dist = back ? HB - (63 - __builtin_clzll(back)) : HB;
    d.s = t - dist;
    d.idx = -1;
    const uint64_t ahead = m >> (HB + 1);  // rows t+1 ..
    if (ahead) d.e = t + 1 + (int64_t)__builtin_ctzll(ahead);
    else d.e = t + 64 - HB < limit ? idx_next_start(q, t + 63 - HB, limit) : limit;
  }
  return d;
}

template <int MODE, int HB = 3>
__device__ __forceinline__ SeqDesc seq_of_row(const SeqArgs& q, int64_t t, int64_t dend, int64_t limit) {
  return seq_resolve<MODE, HB>(q, t, dend, limit, seq_probe<MODE, HB>(q, t, limit));
}

// The slot of sequence idx (resolved from the same probe, which was given the slot array) when
// the probe fetched it: the offsets form up to kDualSeqs sequences, the batch-row form always.
template <int MODE>
__device__ __forceinline__ bool probe_slot(const SeqArgs& q, const SeqProbe& p, int64_t idx, int32_t& slot) {
  if constexpr (MODE == MODE_CU) {
    if (q.nseq > kDualSeqs || idx < 0 || idx >= q.nseq) return false;
    slot = __builtin_amdgcn_readlane((idx & 1) ? p.s1 : p.s0, (int)(idx >> 1));
    return true;
  } else if constexpr (MODE == MODE_BATCH) {
    if (idx < 0 || idx >= q.nseq) return false;
    slot = __builtin_amdgcn_readfirstlane(p.s0);
    return true;
  } else {
    return false;
  }
}

// The sequence that starts right where `cur` ended (cur.e < dend).  Empty sequences are skipped.
template <int MODE>
__device__ __forceinline__ SeqDesc next_seq(const SeqArgs& q, const SeqDesc& cur, int64_t dend, int64_t limit) {
  SeqDesc d;
  const int64_t t = cur.e;
  if constexpr (MODE == MODE_CU) {
    int64_t i = cur.idx + 1;
    while (i + 1 < q.nseq && cu_at(q, i + 1, dend) <= t) ++i;
    if (i >= q.nseq) i = q.nseq - 1;  // only for metadata that breaks the contract: stay in bounds
    d.idx = i;
    d.s = t;
    d.e = cu_at(q, i + 1, dend);
    if (d.e <= t) d.e = t + 1;
  } else if constexpr (MODE == MODE_BATCH) {
    d.idx = cur.idx + 1;
    d.s = t;
    d.e = t + q.seqlen;
    if (d.e > dend) d.e = dend;
  } else {
    d.idx = -1;
    d.s = t;
    d.e = idx_next_start(q, t, limit);
  }
  return d;
}

}  // namespace cconv
