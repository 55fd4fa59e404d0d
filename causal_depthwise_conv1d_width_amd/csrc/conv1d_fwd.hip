// conv1d_fwd.hip -- forward and decode kernels of the packed width-4 causal depthwise Conv1d.
//
// Operation: FlashInfer causal_conv1d_fn (Parameters x, weight, conv_state, cu_seqlens,
// cache_indices, has_initial_state, bias, out) with the optional activation and per-token
// sequence IDs of Megatron-Core causal_conv1d_cp, and the caller history rows of FlashInfer
// cake_causal_conv1d_kcp.
//
// Forward tiling (HBM-bound stencil, no MFMA):
//   block  = kWavesPerBlock waves side by side; lane = 8 consecutive channels; a block covers
//            kBlockChannels channels of a kFwdRows-row range, so each row it touches is one
//            contiguous segment.  Logical tiles run row-range major and each XCD gets one
//            contiguous slice of them, so the row ranges next to each other (which share the
//            three halo rows) and the channel strips of the same rows run together.
//   stream = every wave walks its rows top to bottom in unrolled 8-row chunks: 8 non-temporal
//            16-byte loads in flight per lane, then 8 stencil rows, 8 non-temporal stores.
//   halo   = the three rows before a wave's first row: raw inputs of the same sequence (cached
//            loads; the neighbouring range streamed them moments earlier on the same XCD), or
//            at a sequence start the sequence's history (pool positions 0..2, caller history
//            rows, or zeros).
//   taps   = FP32 in registers; z = b, then four FMAs in tap order 0..3 (tap 3 = current row).
//   window = a 4-slot register ring indexed by row mod 4 inside the unrolled chunk, so the
//            sliding window costs no register moves.
//   pool   = the wave that holds a sequence's first row is the only one that reads or writes
//            its slot (for its channels).  With a pool, row-range boundaries that fall on the
//            first three rows of a sequence move to that sequence's fourth row (or its end), so
//            no other wave ever needs the slot's old history, and the head writes the final
//            state (the last three raw values of the extended sequence) right after reading it.
#include "conv1d_device.h"

namespace cconv {

// ------------------------------------------------------------------ sequence history
// h[j][ch] = history position j (oldest first) of sequence idx, channel c0 + ch.
template <int CPL, bool VEC>
__device__ __forceinline__ void load_history(const PoolArgs& pool, const HistArgs& hist, int64_t idx,
                                             int32_t slot, bool live, int64_t c0, int64_t C, bool active,
                                             float (&h)[3][CPL]) {
#pragma unroll
  for (int j = 0; j < 3; ++j)
#pragma unroll
    for (int ch = 0; ch < CPL; ++ch) h[j][ch] = 0.f;
  if (idx < 0) return;  // history not needed
  if (pool.ptr) {
    const bool init = live && pool.has_init && pool.has_init[idx];
    if (init && active) {
      const uint16_t* base = pool.ptr + (int64_t)slot * pool.s_slot;
#pragma unroll
      for (int j = 0; j < 3; ++j)
#pragma unroll
        for (int ch = 0; ch < CPL; ++ch)
          if (c0 + ch < C)
            h[j][ch] = __uint_as_float((uint32_t)base[(c0 + ch) * pool.s_chan + j * pool.s_pos] << 16);
    }
  } else if (hist.ptr) {
    const bool has = !hist.has_hist || hist.has_hist[idx];
    if (has && active) {
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        Pk<CPL> p = load_row<CPL, VEC>(hist.ptr + (idx * 3 + j) * C, c0, C);
        unpack(p, h[j]);
      }
    }
  }
}

// Final state of a live nonempty sequence: pool positions 0..2 <- last three values of the
// extended sequence u = [h0, h1, h2, x[s], ..., x[e-1]] (raw bits; positions >= 3 untouched).
template <int CPL, bool VEC>
__device__ __forceinline__ void pool_writeback(const FwdArgs& a, int32_t slot, const SeqDesc& sd,
                                               const float (&h)[3][CPL], int64_t c0, bool active) {
  const int64_t n = sd.e - sd.s;
  // start from the history and shift in the sequence's last min(n, 3) rows
  float v[3][CPL];
#pragma unroll
  for (int j = 0; j < 3; ++j)
#pragma unroll
    for (int ch = 0; ch < CPL; ++ch) v[j][ch] = h[j][ch];
  for (int64_t k = (n > 3 ? n - 3 : 0); k < n; ++k) {
    Pk<CPL> p = zero_pk<CPL>();
    if (active) p = load_row<CPL, VEC>(a.x + (sd.s + k) * a.x_ld, c0, a.C);
    shift_in<CPL>(v, p);
  }
  if (!active) return;
  uint16_t* base = a.pool.ptr + (int64_t)slot * a.pool.s_slot;
#pragma unroll
  for (int j = 0; j < 3; ++j)
#pragma unroll
    for (int ch = 0; ch < CPL; ++ch)
      if (c0 + ch < a.C)
        base[(c0 + ch) * a.pool.s_chan + j * a.pool.s_pos] = (uint16_t)(__float_as_uint(v[j][ch]) >> 16);
}

// With a pool: move a row-range boundary r off the first three rows of its sequence.
template <int MODE>
__device__ __forceinline__ int64_t owner_boundary(const SeqArgs& q, int64_t r, int64_t dend) {
  if constexpr (MODE == MODE_IDX) {
    return r;  // the pool needs the cu_seqlens or batch-row form
  } else {
    if (r <= 0 || r >= dend) return r;
    const SeqDesc d = seq_of_row<MODE>(q, r, dend, dend);
    const int64_t k = r - d.s;
    if (k == 1 || k == 2) return d.s + 3 < d.e ? d.s + 3 : d.e;
    return r;
  }
}

// CH consecutive rows starting at q0 (rows past qlast re-read row qlast), every lane active,
// streamed (non-temporal).
template <int CPL, bool VEC, int CH>
__device__ __forceinline__ void load_chunk(Pk<CPL> (&buf)[CH], const uint16_t* __restrict__ x, int64_t ld, int64_t q0,
                                           int64_t qlast, int64_t c0, int64_t C) {
#pragma unroll
  for (int r = 0; r < CH; ++r) {
    const int64_t q = q0 + r < qlast ? q0 + r : qlast;
    buf[r] = load_row<CPL, VEC, true>(x + q * ld, c0, C);
  }
}

template <int CPL, bool SILU>
__device__ __forceinline__ Pk<CPL> stencil_row(const float (&wk)[4][CPL], const float (&bias)[CPL],
                                               const float (&u)[4][CPL], int r);

// CH rows starting at q0 from a loaded buffer: ring update, stencil, streamed store (all lanes).
template <int CPL, bool VEC, int CH, bool SILU>
__device__ __forceinline__ void stencil_chunk(const Pk<CPL> (&buf)[CH], uint16_t* __restrict__ y, int64_t ld,
                                              int64_t q0, int64_t c0, int64_t C, const float (&wk)[4][CPL],
                                              const float (&bias)[CPL], float (&u)[4][CPL]) {
#pragma unroll
  for (int r = 0; r < CH; ++r) {
    unpack(buf[r], u[r % 4]);
    store_row<CPL, VEC, true>(y + (q0 + r) * ld, c0, C, stencil_row<CPL, SILU>(wk, bias, u, r));
  }
}

// One output row from the ring: u[(r+1)%4], u[(r+2)%4], u[(r+3)%4] are rows t-3, t-2, t-1 and
// u[r%4] the current row.  z = b, then the four taps in order (FMA), FP32; y = act(z) in bf16.
template <int CPL, bool SILU>
__device__ __forceinline__ Pk<CPL> stencil_row(const float (&wk)[4][CPL], const float (&bias)[CPL],
                                               const float (&u)[4][CPL], int r) {
  float out[CPL];
#pragma unroll
  for (int ch = 0; ch < CPL; ++ch) {
    float z = bias[ch];
    z = __builtin_fmaf(wk[0][ch], u[(r + 1) % 4][ch], z);
    z = __builtin_fmaf(wk[1][ch], u[(r + 2) % 4][ch], z);
    z = __builtin_fmaf(wk[2][ch], u[(r + 3) % 4][ch], z);
    z = __builtin_fmaf(wk[3][ch], u[r % 4][ch], z);
    out[ch] = SILU ? z * sigmoid_f32(z) : z;
  }
  return pack(out);
}

// ------------------------------------------------------------------ forward kernel
#ifndef CCONV_FWD_CHUNK
#define CCONV_FWD_CHUNK 8
#endif
#ifndef CCONV_FWD_PIPELINE
#define CCONV_FWD_PIPELINE 1
#endif
#ifndef CCONV_FWD_WAVES_PER_EU
#define CCONV_FWD_WAVES_PER_EU 1
#endif

template <int CPL, bool VEC, int MODE, bool SILU>
__global__ void __launch_bounds__(kBlockThreads) __attribute__((amdgpu_waves_per_eu(CCONV_FWD_WAVES_PER_EU)))
conv1d_fwd_kernel(const FwdArgs a) {
  constexpr int CH = CCONV_FWD_CHUNK;  // rows per unrolled chunk; a multiple of the 4-slot ring

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint32_t strip, rb;
  tile_coords(xcd_tile(blockIdx.x, gridDim.x), a.n_strips, strip, rb);
  const int64_t C = a.C;
  const int64_t wc0 = (int64_t)strip * kBlockChannels + (int64_t)wave * kWaveChannels;
  if (wc0 >= C) return;  // the whole wave is past the last channel
  const int64_t c0 = wc0 + lane * CPL;
  const bool active = c0 < C;
  const bool full = VEC && wc0 + kWaveChannels <= C;  // every lane of the wave is active
  const int64_t dend = data_end<MODE>(a.seq, a.rows);
  const bool has_pool = a.pool.ptr != nullptr;

  int64_t ta = (int64_t)rb * kFwdRows;
  int64_t tb = ta + kFwdRows;
  if (has_pool) {
    ta = owner_boundary<MODE>(a.seq, ta, dend);
    tb = owner_boundary<MODE>(a.seq, tb, dend);
  }
  ta = ta < dend ? ta : dend;
  tb = tb < dend ? tb : dend;
  if (ta >= tb) return;

  float wk[4][CPL], bias[CPL];
  load_taps<CPL>(a.w, a.w_f32, a.b, a.b_f32, c0, C, wk, bias);

  float u[4][CPL];  // ring of the extended sequence: row q lives in slot (q - run start) mod 4
  SeqDesc sd = seq_of_row<MODE>(a.seq, ta, dend, tb);
  int64_t t = ta;
  bool first = true;
  while (true) {
    const int64_t dist = first ? (t - sd.s < 3 ? t - sd.s : 3) : 0;
    int32_t slot = -1;
    bool sentinel = false;
    if constexpr (MODE != MODE_IDX) {
      if (has_pool) {
        slot = a.pool.cache_indices[sd.idx];
        sentinel = !(slot >= 0 && slot < a.pool.slots);  // -1 (other values are out of contract)
      }
    }
    const int64_t run_end = sd.e < tb ? sd.e : tb;
    if (sentinel) {
      // -1 slot: +0 output, no state access, no input read
      const Pk<CPL> zero = zero_pk<CPL>();
      if (active)
        for (int64_t q = t; q < run_end; ++q) store_row<CPL, VEC, true>(a.y + q * a.y_ld, c0, C, zero);
    } else {
      float h[3][CPL];
      if constexpr (MODE != MODE_IDX) {
        load_history<CPL, VEC>(a.pool, a.hist, dist < 3 ? sd.idx : -1, slot, true, c0, C, active, h);
      } else {
#pragma unroll
        for (int j = 0; j < 3; ++j)
#pragma unroll
          for (int ch = 0; ch < CPL; ++ch) h[j][ch] = 0.f;
      }
      // window rows t-3, t-2, t-1 -> ring slots 1, 2, 3: the history, then the last `dist`
      // input rows of the same sequence shifted in (dist > 0 only on the first run; those rows
      // were just streamed by the neighbouring row range on this XCD, so they come from L2)
      for (int64_t k = 3 - dist; k < 3; ++k) {
        Pk<CPL> p = zero_pk<CPL>();
        if (active) p = load_row<CPL, VEC>(a.x + (t - 3 + k) * a.x_ld, c0, C);
        shift_in<CPL>(h, p);
      }
#pragma unroll
      for (int j = 0; j < 3; ++j)
#pragma unroll
        for (int ch = 0; ch < CPL; ++ch) u[j + 1][ch] = h[j][ch];
      if constexpr (MODE != MODE_IDX) {
        // at the sequence's first row dist == 0, so h still holds the untouched history
        if (has_pool && t == sd.s && sd.e > sd.s) pool_writeback<CPL, VEC>(a, slot, sd, h, c0, active);
      }

      // full chunks: software-pipelined, the next chunk's loads are in flight while this chunk
      // computes and stores; lanes past the last channel only occur in the last wave of a strip,
      // which takes the predicated tail path for everything
      const int64_t nrun = run_end - t;
      const int nfull = (full && CCONV_FWD_PIPELINE) ? (int)(nrun / CH) : 0;
      int64_t q0 = t;
      if (nfull > 0) {
        // Two register buffers, unrolled by two chunks: chunk j+1's loads are issued before
        // chunk j's stores, so waiting for a chunk's data never waits for the stores issued
        // before it (the vector memory counter is in order).  The next chunk's loads are issued
        // unconditionally; past the last full chunk they re-read the last row (a cache hit), so
        // every path back to the loop head carries the same outstanding loads and the compiler's
        // wait counts stay exact.
        const int64_t qlast = t + (int64_t)nfull * CH - 1;
        Pk<CPL> A[CH], B[CH];
        load_chunk<CPL, VEC, CH>(A, a.x, a.x_ld, q0, qlast, c0, C);
        for (int j = 0;; j += 2, q0 += 2 * CH) {
          load_chunk<CPL, VEC, CH>(B, a.x, a.x_ld, q0 + CH, qlast, c0, C);
          stencil_chunk<CPL, VEC, CH, SILU>(A, a.y, a.y_ld, q0, c0, C, wk, bias, u);
          if (j + 1 >= nfull) {
            q0 += CH;
            break;
          }
          load_chunk<CPL, VEC, CH>(A, a.x, a.x_ld, q0 + 2 * CH, qlast, c0, C);
          stencil_chunk<CPL, VEC, CH, SILU>(B, a.y, a.y_ld, q0 + CH, c0, C, wk, bias, u);
          if (j + 2 >= nfull) {
            q0 += 2 * CH;
            break;
          }
        }
      }
      // tail (and partially active waves): rows one chunk at a time with uniform row predicates
      for (; q0 < run_end; q0 += CH) {
        const int n = (int)(run_end - q0 < CH ? run_end - q0 : CH);
        Pk<CPL> xr[CH];
#pragma unroll
        for (int r = 0; r < CH; ++r) {
          xr[r] = zero_pk<CPL>();
          if (r < n && active) xr[r] = load_row<CPL, VEC, true>(a.x + (q0 + r) * a.x_ld, c0, C);
        }
#pragma unroll
        for (int r = 0; r < CH; ++r) {
          if (r < n) {
            unpack(xr[r], u[r % 4]);
            const Pk<CPL> out = stencil_row<CPL, SILU>(wk, bias, u, r);
            if (active) store_row<CPL, VEC, true>(a.y + (q0 + r) * a.y_ld, c0, C, out);
          }
        }
      }
    }
    t = run_end;
    if (t >= tb) break;
    sd = next_seq<MODE>(a.seq, sd, dend, tb);
    first = false;
  }
}

// ------------------------------------------------------------------ decode kernel
// One thread per (sequence, CPL-channel group).  y = act(b + w . [h0, h1, h2, x]), then the
// slot's positions 0..2 become [h1, h2, x]; slot -1 gives +0 and touches nothing.
template <int CPL, bool VEC, bool SILU>
__global__ void __launch_bounds__(kBlockThreads) conv1d_decode_kernel(const DecodeArgs a) {
  const int64_t gid = (int64_t)blockIdx.x * kBlockThreads + threadIdx.x;
  const int64_t groups = (a.C + CPL - 1) / CPL;
  if (gid >= a.nseq * groups) return;
  const int64_t i = gid / groups;
  const int64_t c0 = (gid - i * groups) * CPL;
  const int64_t C = a.C;
  const int32_t slot = a.pool.cache_indices[i];
  if (!(slot >= 0 && slot < a.pool.slots)) {
    store_row<CPL, VEC>(a.y + i * a.y_ld, c0, C, zero_pk<CPL>());
    return;
  }
  float wk[4][CPL], bias[CPL];
  load_taps<CPL>(a.w, a.w_f32, a.b, a.b_f32, c0, C, wk, bias);
  float xv[CPL];
  unpack(load_row<CPL, VEC>(a.x + i * a.x_ld, c0, C), xv);
  uint16_t* base = a.pool.ptr + (int64_t)slot * a.pool.s_slot;
  float out[CPL];
  uint16_t hb[3][CPL];
#pragma unroll
  for (int ch = 0; ch < CPL; ++ch) {
    const int64_t c = c0 + ch;
    float h[3] = {0.f, 0.f, 0.f};
    if (c < C) {
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        hb[j][ch] = base[c * a.pool.s_chan + j * a.pool.s_pos];
        h[j] = __uint_as_float((uint32_t)hb[j][ch] << 16);
      }
    }
    float z = bias[ch];
    z = __builtin_fmaf(wk[0][ch], h[0], z);
    z = __builtin_fmaf(wk[1][ch], h[1], z);
    z = __builtin_fmaf(wk[2][ch], h[2], z);
    z = __builtin_fmaf(wk[3][ch], xv[ch], z);
    out[ch] = SILU ? z * sigmoid_f32(z) : z;
  }
  store_row<CPL, VEC>(a.y + i * a.y_ld, c0, C, pack(out));
#pragma unroll
  for (int ch = 0; ch < CPL; ++ch) {
    const int64_t c = c0 + ch;
    if (c < C) {
      base[c * a.pool.s_chan + 0 * a.pool.s_pos] = hb[1][ch];
      base[c * a.pool.s_chan + 1 * a.pool.s_pos] = hb[2][ch];
      base[c * a.pool.s_chan + 2 * a.pool.s_pos] = (uint16_t)(__float_as_uint(xv[ch]) >> 16);
    }
  }
}

// ------------------------------------------------------------------ launchers
constexpr int kCpl = kChannelsPerLane;

template <int MODE, bool VEC, bool SILU>
static hipError_t fwd_go(const FwdArgs& a, hipStream_t s) {
  const uint32_t blocks = a.n_strips * a.n_rowblocks;
  void* args[] = {const_cast<FwdArgs*>(&a)};
  return hipLaunchKernel(reinterpret_cast<const void*>(&conv1d_fwd_kernel<kCpl, VEC, MODE, SILU>), dim3(blocks),
                         dim3(kBlockThreads), args, 0, s);
}

template <int MODE>
static hipError_t fwd_mode(const FwdArgs& a, bool vec, bool silu, hipStream_t s) {
  if (vec) return silu ? fwd_go<MODE, true, true>(a, s) : fwd_go<MODE, true, false>(a, s);
  return silu ? fwd_go<MODE, false, true>(a, s) : fwd_go<MODE, false, false>(a, s);
}

hipError_t launch_fwd(const FwdArgs& a, int mode, bool vec, bool silu, hipStream_t s) {
  if ((uint64_t)a.n_strips * a.n_rowblocks == 0) return hipSuccess;
  switch (mode) {
    case MODE_CU: return fwd_mode<MODE_CU>(a, vec, silu, s);
    case MODE_IDX: return fwd_mode<MODE_IDX>(a, vec, silu, s);
    default: return fwd_mode<MODE_BATCH>(a, vec, silu, s);
  }
}

template <bool VEC, bool SILU>
static hipError_t decode_go(const DecodeArgs& a, hipStream_t s) {
  const int64_t groups = (a.C + kCpl - 1) / kCpl;
  const int64_t blocks = (a.nseq * groups + kBlockThreads - 1) / kBlockThreads;
  void* args[] = {const_cast<DecodeArgs*>(&a)};
  return hipLaunchKernel(reinterpret_cast<const void*>(&conv1d_decode_kernel<kCpl, VEC, SILU>),
                         dim3((uint32_t)blocks), dim3(kBlockThreads), args, 0, s);
}

hipError_t launch_decode(const DecodeArgs& a, bool vec, bool silu, hipStream_t s) {
  if (a.nseq == 0) return hipSuccess;
  if (vec) return silu ? decode_go<true, true>(a, s) : decode_go<true, false>(a, s);
  return silu ? decode_go<false, true>(a, s) : decode_go<false, false>(a, s);
}

}  // namespace cconv
