// conv1d_bwd.hip -- training backward of the packed width-4 causal depthwise Conv1d.
//
// Operation: the gradients of the forward in conv1d_fwd.hip for the training path of FlashInfer
// cake_causal_conv1d_kcp (Returns: dx, a deterministic FP32 dweight, and the gradient of the
// history rows that the preceding fragment supplied) and Megatron-Core causal_conv1d_cp.  With
// z[t] = b + sum_k w_k u[t-3+k] and dz[t] = dy[t] * act'(z[t]):
//     dx[t]  = sum_k w_k dz[t+3-k]           (terms inside t's sequence only)
//     dw_k   = sum_t dz[t] u[t-3+k],  db = sum_t dz[t]
//     dh_j   = sum_{tau <= j} w_{j-tau} dz[s+tau]   (history row j of a continuing fragment)
//
// Tiling: as the forward (waves side by side in channels, lane = 8 channels), with kBwdRows-row
// ranges.  A wave needs x rows [ta-3, tb+3) and dy rows [ta, tb+3); its own rows are streamed
// once (non-temporal), the three look-behind and three look-ahead rows belong to the
// neighbouring row ranges, which stream them at the same time on the same XCD, so those few
// reads are served by L2.
//
// dweight/dbias are deterministic by construction: each lane accumulates its channels over its
// rows in row order (FP32) and owns those channels for the whole row range, so the range's
// [5, C] partial is written straight from registers to the workspace, and a second kernel adds
// the partials of all row ranges in ascending range order.  No atomics anywhere, so the bits
// depend only on the input values and the range length, never on scheduling or on the
// workspace address.
#include "conv1d_device.h"

namespace cconv {

template <int CPL, bool VEC>
__device__ __forceinline__ void load_hist_rows(const HistArgs& hist, int64_t idx, int64_t c0, int64_t C,
                                               bool active, float (&h)[3][CPL]) {
#pragma unroll
  for (int j = 0; j < 3; ++j)
#pragma unroll
    for (int ch = 0; ch < CPL; ++ch) h[j][ch] = 0.f;
  if (idx >= 0 && hist.ptr && active && (!hist.has_hist || hist.has_hist[idx])) {
#pragma unroll
    for (int j = 0; j < 3; ++j) unpack(load_row<CPL, VEC>(hist.ptr + (idx * 3 + j) * C, c0, C), h[j]);
  }
}

#ifndef CCONV_BWD_CHUNK
#define CCONV_BWD_CHUNK 4
#endif
#ifndef CCONV_BWD_PIPELINE
#define CCONV_BWD_PIPELINE 1
#endif
#ifndef CCONV_BWD_WAVES_PER_EU
#define CCONV_BWD_WAVES_PER_EU 1
#endif

// Per-lane state of the backward stream (CPL channels).
template <int CPL>
struct BwdState {
  float wk[4][CPL], bias[CPL];
  float u[4][CPL];    // extended-sequence ring, slot = (row - run start) mod 4
  float g[4][CPL];    // dz ring, same slots
  float acc[5][CPL];  // dw_0..3, db partial sums over the wave's rows
};

// One real row q (ring slot r): recompute z, dz = dy * act'(z); dweight/dbias sums when `own`.
template <int CPL, bool SILU>
__device__ __forceinline__ void bwd_row(BwdState<CPL>& st, const Pk<CPL>& xr, const Pk<CPL>& gr, int r, bool own) {
  unpack(xr, st.u[r % 4]);
  float dyv[CPL];
  unpack(gr, dyv);
#pragma unroll
  for (int ch = 0; ch < CPL; ++ch) {
    float z = st.bias[ch];
    z = __builtin_fmaf(st.wk[0][ch], st.u[(r + 1) % 4][ch], z);
    z = __builtin_fmaf(st.wk[1][ch], st.u[(r + 2) % 4][ch], z);
    z = __builtin_fmaf(st.wk[2][ch], st.u[(r + 3) % 4][ch], z);
    z = __builtin_fmaf(st.wk[3][ch], st.u[r % 4][ch], z);
    float dz = dyv[ch];
    if (SILU) {
      const float sg = sigmoid_f32(z);
      dz = dz * (sg * __builtin_fmaf(z, 1.0f - sg, 1.0f));
    }
    st.g[r % 4][ch] = dz;
  }
  if (own) {
#pragma unroll
    for (int ch = 0; ch < CPL; ++ch) {
      st.acc[0][ch] = __builtin_fmaf(st.g[r % 4][ch], st.u[(r + 1) % 4][ch], st.acc[0][ch]);
      st.acc[1][ch] = __builtin_fmaf(st.g[r % 4][ch], st.u[(r + 2) % 4][ch], st.acc[1][ch]);
      st.acc[2][ch] = __builtin_fmaf(st.g[r % 4][ch], st.u[(r + 3) % 4][ch], st.acc[2][ch]);
      st.acc[3][ch] = __builtin_fmaf(st.g[r % 4][ch], st.u[r % 4][ch], st.acc[3][ch]);
      st.acc[4][ch] += st.g[r % 4][ch];
    }
  }
}

// dx of the row three steps back: w3 dz[q-3] + w2 dz[q-2] + w1 dz[q-1] + w0 dz[q]
template <int CPL>
__device__ __forceinline__ Pk<CPL> bwd_dx(const BwdState<CPL>& st, int r) {
  float d[CPL];
#pragma unroll
  for (int ch = 0; ch < CPL; ++ch) {
    float v = st.wk[3][ch] * st.g[(r + 1) % 4][ch];
    v = __builtin_fmaf(st.wk[2][ch], st.g[(r + 2) % 4][ch], v);
    v = __builtin_fmaf(st.wk[1][ch], st.g[(r + 3) % 4][ch], v);
    v = __builtin_fmaf(st.wk[0][ch], st.g[r % 4][ch], v);
    d[ch] = v;
  }
  return pack(d);
}

// head of a continuing fragment: dh_j += w_{j-r} dz[s+r] for j >= r (r = 0, 1, 2)
template <int CPL>
__device__ __forceinline__ void bwd_dhist(const BwdState<CPL>& st, float (&dh)[3][CPL], int r) {
#pragma unroll
  for (int j = r; j < 3; ++j)
#pragma unroll
    for (int ch = 0; ch < CPL; ++ch) dh[j][ch] = __builtin_fmaf(st.wk[j - r][ch], st.g[r % 4][ch], dh[j][ch]);
}

// CH own rows starting at q0 (every lane active, all rows real and owned).  FIRST: q0 is the
// run's first row, so rows q0-3..q0-1 get no dx here, and a head fragment's d(history), which
// needs dz of the sequence's first three rows only, is finished and stored in this chunk.
template <int CPL, bool VEC, int CH, bool SILU, bool FIRST>
__device__ __forceinline__ void bwd_chunk(BwdState<CPL>& st, const Pk<CPL> (&X)[CH], const Pk<CPL> (&G)[CH],
                                          const BwdArgs& a, int64_t q0, int64_t c0, bool want_dh, int64_t hidx) {
  static_assert(CH >= 3, "the first chunk must hold a sequence's first three rows");
#pragma unroll
  for (int r = 0; r < CH; ++r) {
    bwd_row<CPL, SILU>(st, X[r], G[r], r, true);
    if (FIRST && r == 2 && want_dh) {
      float dh[3][CPL];
#pragma unroll
      for (int j = 0; j < 3; ++j)
#pragma unroll
        for (int ch = 0; ch < CPL; ++ch) dh[j][ch] = 0.f;
#pragma unroll
      for (int rr = 0; rr < 3; ++rr) bwd_dhist<CPL>(st, dh, rr);
#pragma unroll
      for (int j = 0; j < 3; ++j) store_row<CPL, VEC>(a.dhist + (hidx * 3 + j) * a.C, c0, a.C, pack(dh[j]));
    }
    if (!FIRST || r >= 3) store_row<CPL, VEC, true>(a.dx + (q0 + r - 3) * a.dx_ld, c0, a.C, bwd_dx<CPL>(st, r));
  }
}

template <int CPL, bool VEC, int CH>
__device__ __forceinline__ void bwd_load(Pk<CPL> (&X)[CH], Pk<CPL> (&G)[CH], const BwdArgs& a, int64_t q0, int64_t qlast,
                                         int64_t c0) {
#pragma unroll
  for (int r = 0; r < CH; ++r) {
    const int64_t q = q0 + r < qlast ? q0 + r : qlast;
    X[r] = load_row<CPL, VEC, true>(a.x + q * a.x_ld, c0, a.C);
    G[r] = load_row<CPL, VEC, true>(a.dy + q * a.dy_ld, c0, a.C);
  }
}

template <int CPL, bool VEC, int MODE, bool SILU>
__global__ void __launch_bounds__(kBlockThreads) __attribute__((amdgpu_waves_per_eu(CCONV_BWD_WAVES_PER_EU)))
conv1d_bwd_kernel(const BwdArgs a) {
  constexpr int CH = CCONV_BWD_CHUNK;  // rows per unrolled chunk (a multiple of the 4-slot rings)

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint32_t strip, rb;
  tile_coords(xcd_tile(blockIdx.x, gridDim.x), a.n_strips, strip, rb);
  const int64_t C = a.C;
  const int64_t wc0 = (int64_t)strip * kBlockChannels + (int64_t)wave * kWaveChannels;
  if (wc0 >= C) return;  // the whole wave is past the last channel: no partial to write
  const int64_t c0 = wc0 + lane * CPL;
  const bool active = c0 < C;
  const bool full = VEC && wc0 + kWaveChannels <= C;  // every lane of the wave is active
  const int64_t dend = data_end<MODE>(a.seq, a.rows);

  int64_t ta = (int64_t)rb * kBwdRows;
  int64_t tb = ta + kBwdRows;
  ta = ta < dend ? ta : dend;
  tb = tb < dend ? tb : dend;

  BwdState<CPL> st;
#pragma unroll
  for (int k = 0; k < 5; ++k)
#pragma unroll
    for (int ch = 0; ch < CPL; ++ch) st.acc[k][ch] = 0.f;

  if (ta < tb) {
    load_taps<CPL>(a.w, a.w_f32, a.b, a.b_f32, c0, C, st.wk, st.bias);
    const int64_t lim = (tb + 3 < dend) ? tb + 3 : dend;  // IDX scans need ends up to tb+3
    SeqDesc sd = seq_of_row<MODE>(a.seq, ta, dend, lim);
    int64_t t = ta;
    bool first = true;
    while (true) {
      const int64_t dist = first ? (t - sd.s < 3 ? t - sd.s : 3) : 0;
      float h[3][CPL];
      bool want_dh = false;
      if constexpr (MODE != MODE_IDX) {
        load_hist_rows<CPL, VEC>(a.hist, dist < 3 ? sd.idx : -1, c0, C, active, h);
        want_dh = a.dhist && t == sd.s && (!a.hist.has_hist || a.hist.has_hist[sd.idx]);
      } else {
#pragma unroll
        for (int j = 0; j < 3; ++j)
#pragma unroll
          for (int ch = 0; ch < CPL; ++ch) h[j][ch] = 0.f;
      }
      // window rows t-3..t-1: the history, then the last `dist` rows of the same sequence
      // (the previous row range streamed them moments earlier on this XCD: cached loads)
      for (int64_t k = 3 - dist; k < 3; ++k) {
        Pk<CPL> p = zero_pk<CPL>();
        if (active) p = load_row<CPL, VEC>(a.x + (t - 3 + k) * a.x_ld, c0, C);
        shift_in<CPL>(h, p);
      }
#pragma unroll
      for (int j = 0; j < 3; ++j)
#pragma unroll
        for (int ch = 0; ch < CPL; ++ch) st.u[j + 1][ch] = h[j][ch];

      const int64_t t_end = sd.e < tb ? sd.e : tb;  // rows of this run that the wave owns
      int64_t la_end = t_end;                        // plus same-sequence look-ahead rows
      if (t_end == tb) la_end = (sd.e < tb + 3) ? sd.e : tb + 3;
      if (la_end > dend) la_end = dend;
      const int64_t steps_end = t_end + 3;  // three trailing steps finish the last dx rows

      // full chunks of own rows, software-pipelined with two register buffers (see the forward)
      const int nfull = (full && CCONV_BWD_PIPELINE) ? (int)((t_end - t) / CH) : 0;
      int64_t q0 = t;
      bool dh_done = false;
      if (nfull > 0) {
        // two register buffers, unrolled by two chunks, next chunk's loads always issued (rows
        // past the last full chunk re-read its last row): see the forward kernel
        const int64_t qlast = t + (int64_t)nfull * CH - 1;
        Pk<CPL> XA[CH], GA[CH], XB[CH], GB[CH];
        bwd_load<CPL, VEC, CH>(XA, GA, a, q0, qlast, c0);
        bwd_load<CPL, VEC, CH>(XB, GB, a, q0 + CH, qlast, c0);
        bwd_chunk<CPL, VEC, CH, SILU, true>(st, XA, GA, a, q0, c0, want_dh, sd.idx);
        dh_done = true;
        for (int j = 1;; j += 2, q0 += 2 * CH) {
          if (j >= nfull) {
            q0 += CH;
            break;
          }
          bwd_load<CPL, VEC, CH>(XA, GA, a, q0 + 2 * CH, qlast, c0);
          bwd_chunk<CPL, VEC, CH, SILU, false>(st, XB, GB, a, q0 + CH, c0, want_dh, sd.idx);
          if (j + 1 >= nfull) {
            q0 += 2 * CH;
            break;
          }
          bwd_load<CPL, VEC, CH>(XB, GB, a, q0 + 3 * CH, qlast, c0);
          bwd_chunk<CPL, VEC, CH, SILU, false>(st, XA, GA, a, q0 + 2 * CH, c0, want_dh, sd.idx);
        }
      }
      // the rest: remaining own rows, look-ahead rows of the same sequence, and three trailing
      // steps (dz = 0 past the sequence's end) that finish the last dx rows
      float dh[3][CPL];
#pragma unroll
      for (int j = 0; j < 3; ++j)
#pragma unroll
        for (int ch = 0; ch < CPL; ++ch) dh[j][ch] = 0.f;
      for (; q0 < steps_end; q0 += CH) {
        Pk<CPL> xr[CH], gr[CH];
#pragma unroll
        for (int r = 0; r < CH; ++r) {
          const int64_t q = q0 + r;
          xr[r] = zero_pk<CPL>();
          gr[r] = zero_pk<CPL>();
          if (q < la_end && active) {
            if (q < t_end) {  // own rows: read once, streamed
              xr[r] = load_row<CPL, VEC, true>(a.x + q * a.x_ld, c0, C);
              gr[r] = load_row<CPL, VEC, true>(a.dy + q * a.dy_ld, c0, C);
            } else {  // look-ahead rows, owned by the next row range
              xr[r] = load_row<CPL, VEC>(a.x + q * a.x_ld, c0, C);
              gr[r] = load_row<CPL, VEC>(a.dy + q * a.dy_ld, c0, C);
            }
          }
        }
#pragma unroll
        for (int r = 0; r < CH; ++r) {
          const int64_t q = q0 + r;
          if (q < steps_end) {
            if (q < la_end) {
              bwd_row<CPL, SILU>(st, xr[r], gr[r], r, q < t_end);
            } else {
#pragma unroll
              for (int ch = 0; ch < CPL; ++ch) st.g[r % 4][ch] = 0.f;  // past the sequence's end
            }
            if (r < 3 && want_dh && q0 == t) bwd_dhist<CPL>(st, dh, r);
            if (q - 3 >= t) {
              const Pk<CPL> d = bwd_dx<CPL>(st, r);
              if (active) store_row<CPL, VEC, true>(a.dx + (q - 3) * a.dx_ld, c0, C, d);
            }
          }
        }
      }
      if constexpr (MODE != MODE_IDX) {
        if (want_dh && active && !dh_done) {
#pragma unroll
          for (int j = 0; j < 3; ++j) store_row<CPL, VEC>(a.dhist + (sd.idx * 3 + j) * C, c0, C, pack(dh[j]));
        }
      }
      t = t_end;
      if (t >= tb) break;
      sd = next_seq<MODE>(a.seq, sd, dend, lim);
      first = false;
    }
  }

  // ---- this lane's partial sums for its channels over this row range (every range writes one,
  // empty ranges write zeros, so the reduce can read all of them)
  if (active) {
#pragma unroll
    for (int k = 0; k < 5; ++k) {
      float* dst = a.part + ((int64_t)rb * 5 + k) * C + c0;
      if constexpr (VEC && CPL >= 4) {
#pragma unroll
        for (int q = 0; q < CPL; q += 4)
          *reinterpret_cast<f32x4*>(dst + q) = f32x4{st.acc[k][q], st.acc[k][q + 1], st.acc[k][q + 2], st.acc[k][q + 3]};
      } else if constexpr (VEC) {
        *reinterpret_cast<f32x2*>(dst) = f32x2{st.acc[k][0], st.acc[k][1]};
      } else {
#pragma unroll
        for (int ch = 0; ch < CPL; ++ch)
          if (c0 + ch < C) dst[ch] = st.acc[k][ch];
      }
    }
  }
}

// Ordered reduce of the per-range partials: out[o] = sum over row ranges p of part[p][o], for
// the flattened o = k*C + c (k = 0..3 dweight taps, 4 = dbias).  A wave owns 16 consecutive o;
// lane l sums the ranges p = l/16, l/16 + 4, l/16 + 8, ... in ascending order (each load of
// the wave reads four 64-byte runs), then a fixed two-level butterfly across lanes l, l^16,
// l^32, l^48 adds the four interleaved subsets:  (s0 + s1) + (s2 + s3).  The order is fixed, so
// dweight/dbias are bitwise reproducible; no atomics.  The remaining threads write zero
// d(history) rows of empty continuing fragments.
__global__ void __launch_bounds__(kBlockThreads) conv1d_bwd_reduce_kernel(const BwdArgs a, int64_t nhist_zero,
                                                                           int64_t n_red_waves) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t gwave = ((int64_t)blockIdx.x * kBlockThreads + threadIdx.x) / kWave;
  const int64_t C = a.C;
  const int64_t nout = 5 * C;
  if (gwave < n_red_waves) {
    const int64_t o = gwave * 16 + (lane & 15);
    const int sub = lane >> 4;
    const bool ok = o < nout;
    const int64_t n = a.n_rowblocks;
    float s = 0.f;
    if (ok) {
      const float* p = a.part + o;
      int64_t i = sub;
      for (; i + 12 < n; i += 16) {
        const float v0 = p[i * nout], v1 = p[(i + 4) * nout], v2 = p[(i + 8) * nout], v3 = p[(i + 12) * nout];
        s += v0;
        s += v1;
        s += v2;
        s += v3;
      }
      for (; i < n; i += 4) s += p[i * nout];
    }
    s += __shfl_xor(s, 16);  // s0+s1 (lanes 0-31), s2+s3 (lanes 32-63); fp add commutes exactly
    s += __shfl_xor(s, 32);  // (s0+s1) + (s2+s3) on every lane
    if (ok && lane < 16) {
      const int64_t k = o / C, c = o - k * C;
      if (k < 4) a.dw[c * 4 + k] = s;
      else if (a.db) a.db[c] = s;
    }
    return;
  }
  const int64_t hid = (int64_t)blockIdx.x * kBlockThreads + threadIdx.x - n_red_waves * kWave;
  if (hid < 0 || hid >= nhist_zero * C) return;
  const int64_t i = hid / C, c = hid - i * C;
  if (a.hist.has_hist && !a.hist.has_hist[i]) return;
  if (a.seq.cu[i + 1] != a.seq.cu[i]) return;  // nonempty: written by the tile kernel
#pragma unroll
  for (int j = 0; j < 3; ++j) a.dhist[(i * 3 + j) * C + c] = 0;
}

// ------------------------------------------------------------------ launchers
constexpr int kCpl = kChannelsPerLane;

template <int MODE, bool VEC, bool SILU>
static hipError_t bwd_go(const BwdArgs& a, hipStream_t s) {
  const uint32_t blocks = a.n_strips * a.n_rowblocks;
  if (blocks) {
    void* args[] = {const_cast<BwdArgs*>(&a)};
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&conv1d_bwd_kernel<kCpl, VEC, MODE, SILU>),
                                   dim3(blocks), dim3(kBlockThreads), args, 0, s);
    if (e != hipSuccess) return e;
  }
  // empty fragments that read history rows still get a (zero) d(history)
  const int64_t nz = (a.dhist && MODE == MODE_CU) ? a.seq.nseq : 0;
  int64_t n_red_waves = (5 * a.C + 15) / 16;
  const int64_t threads = n_red_waves * kWave + nz * a.C;
  const uint32_t rblocks = (uint32_t)((threads + kBlockThreads - 1) / kBlockThreads);
  int64_t nz_arg = nz;
  void* rargs[] = {const_cast<BwdArgs*>(&a), &nz_arg, &n_red_waves};
  return hipLaunchKernel(reinterpret_cast<const void*>(&conv1d_bwd_reduce_kernel), dim3(rblocks), dim3(kBlockThreads),
                         rargs, 0, s);
}

template <int MODE>
static hipError_t bwd_mode(const BwdArgs& a, bool vec, bool silu, hipStream_t s) {
  if (vec) return silu ? bwd_go<MODE, true, true>(a, s) : bwd_go<MODE, true, false>(a, s);
  return silu ? bwd_go<MODE, false, true>(a, s) : bwd_go<MODE, false, false>(a, s);
}

hipError_t launch_bwd(const BwdArgs& a, int mode, bool vec, bool silu, hipStream_t s) {
  switch (mode) {
    case MODE_CU: return bwd_mode<MODE_CU>(a, vec, silu, s);
    case MODE_IDX: return bwd_mode<MODE_IDX>(a, vec, silu, s);
    default: return bwd_mode<MODE_BATCH>(a, vec, silu, s);
  }
}

}  // namespace cconv
