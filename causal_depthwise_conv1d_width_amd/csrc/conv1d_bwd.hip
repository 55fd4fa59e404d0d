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
// Tiling: as the forward (4 waves x 64 lanes, lane = CPL channels), kBwdRowsPerWave rows per
// wave.  A wave needs x rows [ta-3, tb+3) and dy rows [ta, tb+3).  Before the block barrier
// each wave stages its first three and last three x/dy rows in LDS; the boundary buffers
// between waves then serve both neighbours (look-behind x for the next wave, look-ahead x/dy for
// the previous one) and the owner itself, so inside a block each row leaves HBM once.
//
// dweight/dbias are deterministic by construction: each lane accumulates its channels over its
// rows in row order (FP32), the four waves of a block are added in wave order through LDS, the
// block's [5, C] partial goes to the workspace, and a second kernel adds the partials of all
// row blocks in ascending block order.  No atomics anywhere, so the bits depend only on the
// input values and the row-block size, never on scheduling or on the workspace address.
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

template <int CPL, bool VEC, int MODE, bool SILU>
__global__ void __launch_bounds__(kThreads) conv1d_bwd_kernel(const BwdArgs a) {
  constexpr int KW = kBwdRowsPerWave;
  constexpr int CH = 4;  // rows per unrolled chunk (the 4-slot rings)
  // boundary buffers: bx[b][k] holds row (start of wave b) - 3 + k, k = 0..5
  __shared__ Pk<CPL> bx[kWaves + 1][6][kWave];
  __shared__ Pk<CPL> bdy[kWaves + 1][6][kWave];

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t tile = xcd_tile(blockIdx.x, gridDim.x);
  const uint32_t strip = tile / a.n_rowblocks, rb = tile % a.n_rowblocks;
  const int64_t C = a.C;
  const int64_t c0 = (int64_t)strip * (kWave * CPL) + lane * CPL;
  const bool active = c0 < C;
  const int64_t dend = data_end<MODE>(a.seq, a.rows);

  int64_t ta = (int64_t)rb * kBwdRowsPerBlock + (int64_t)wave * KW;
  int64_t tb = ta + KW;
  ta = ta < dend ? ta : dend;
  tb = tb < dend ? tb : dend;

  // ---- stage halos: own first / last three rows, plus the block's outer look-behind/ahead
  if (active) {
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const int64_t rf = ta + j;
      if (rf < tb) {
        bx[wave][3 + j][lane] = load_row<CPL, VEC>(a.x + rf * a.x_ld, c0, C);
        bdy[wave][3 + j][lane] = load_row<CPL, VEC>(a.dy + rf * a.dy_ld, c0, C);
      }
      const int64_t rl = tb - 3 + j;
      if (rl >= ta) {
        bx[wave + 1][j][lane] = load_row<CPL, VEC>(a.x + rl * a.x_ld, c0, C);
        bdy[wave + 1][j][lane] = load_row<CPL, VEC>(a.dy + rl * a.dy_ld, c0, C);
      }
      if (wave == 0) {
        const int64_t rb0 = ta - 3 + j;
        if (rb0 >= 0 && ta < tb) bx[0][j][lane] = load_row<CPL, VEC>(a.x + rb0 * a.x_ld, c0, C);
      }
      if (wave == kWaves - 1) {
        const int64_t ra = tb + j;
        if (ra < dend && ta < tb) {
          bx[kWaves][3 + j][lane] = load_row<CPL, VEC>(a.x + ra * a.x_ld, c0, C);
          bdy[kWaves][3 + j][lane] = load_row<CPL, VEC>(a.dy + ra * a.dy_ld, c0, C);
        }
      }
    }
  }
  __syncthreads();

  float acc[5][CPL];  // dw_0..3, db partial sums of this lane
#pragma unroll
  for (int k = 0; k < 5; ++k)
#pragma unroll
    for (int ch = 0; ch < CPL; ++ch) acc[k][ch] = 0.f;

  if (ta < tb) {
    float wk[4][CPL], bias[CPL];
    load_taps<CPL>(a.w, a.w_f32, a.b, a.b_f32, c0, C, wk, bias);

    // x / dy of a wave-uniform row q, from the boundary buffers when staged, else from HBM
    auto src = [&](int64_t q, const uint16_t* base, int64_t ld, Pk<CPL> (*buf)[6][kWave]) -> Pk<CPL> {
      if (q >= ta - 3 && q < ta + 3) return buf[wave][q - ta + 3][lane];
      if (q >= tb - 3 && q < tb + 3) return buf[wave + 1][q - tb + 3][lane];
      return load_row<CPL, VEC>(base + q * ld, c0, C);
    };

    float u[4][CPL];  // extended-sequence ring, slot = (row - run start) mod 4
    float g[4][CPL];  // dz ring, same slots
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
      {
        // window rows t-3..t-1: the history, then the last `dist` rows of the same sequence
        for (int64_t k = 3 - dist; k < 3; ++k) {
          Pk<CPL> p = zero_pk<CPL>();
          if (active) p = src(t - 3 + k, a.x, a.x_ld, bx);
          shift_in<CPL>(h, p);
        }
#pragma unroll
        for (int j = 0; j < 3; ++j)
#pragma unroll
          for (int ch = 0; ch < CPL; ++ch) u[j + 1][ch] = h[j][ch];
      }
      float dh[3][CPL];
#pragma unroll
      for (int j = 0; j < 3; ++j)
#pragma unroll
        for (int ch = 0; ch < CPL; ++ch) dh[j][ch] = 0.f;

      const int64_t t_end = sd.e < tb ? sd.e : tb;  // rows of this run that the wave owns
      int64_t la_end = t_end;                        // plus same-sequence look-ahead rows
      if (t_end == tb) la_end = (sd.e < tb + 3) ? sd.e : tb + 3;
      if (la_end > dend) la_end = dend;
      const int64_t steps_end = t_end + 3;  // three trailing steps finish the last dx rows

      for (int64_t q0 = t; q0 < steps_end; q0 += CH) {
        Pk<CPL> xr[CH], gr[CH];
#pragma unroll
        for (int r = 0; r < CH; ++r) {
          const int64_t q = q0 + r;
          xr[r] = zero_pk<CPL>();
          gr[r] = zero_pk<CPL>();
          if (q < la_end && active) {
            xr[r] = src(q, a.x, a.x_ld, bx);
            gr[r] = src(q, a.dy, a.dy_ld, bdy);
          }
        }
#pragma unroll
        for (int r = 0; r < CH; ++r) {
          const int64_t q = q0 + r;
          if (q < steps_end) {
            if (q < la_end) {
              unpack(xr[r], u[r % 4]);
              float dyv[CPL];
              unpack(gr[r], dyv);
#pragma unroll
              for (int ch = 0; ch < CPL; ++ch) {
                float z = bias[ch];
                z = __builtin_fmaf(wk[0][ch], u[(r + 1) % 4][ch], z);
                z = __builtin_fmaf(wk[1][ch], u[(r + 2) % 4][ch], z);
                z = __builtin_fmaf(wk[2][ch], u[(r + 3) % 4][ch], z);
                z = __builtin_fmaf(wk[3][ch], u[r % 4][ch], z);
                float dz = dyv[ch];
                if (SILU) {
                  const float sg = sigmoid_f32(z);
                  dz = dz * (sg * __builtin_fmaf(z, 1.0f - sg, 1.0f));
                }
                g[r % 4][ch] = dz;
              }
              if (q < t_end) {
#pragma unroll
                for (int ch = 0; ch < CPL; ++ch) {
                  acc[0][ch] = __builtin_fmaf(g[r % 4][ch], u[(r + 1) % 4][ch], acc[0][ch]);
                  acc[1][ch] = __builtin_fmaf(g[r % 4][ch], u[(r + 2) % 4][ch], acc[1][ch]);
                  acc[2][ch] = __builtin_fmaf(g[r % 4][ch], u[(r + 3) % 4][ch], acc[2][ch]);
                  acc[3][ch] = __builtin_fmaf(g[r % 4][ch], u[r % 4][ch], acc[3][ch]);
                  acc[4][ch] += g[r % 4][ch];
                }
              }
            } else {
#pragma unroll
              for (int ch = 0; ch < CPL; ++ch) g[r % 4][ch] = 0.f;  // past the sequence's end
            }
            if (r < 3 && want_dh && q0 == t) {
              // head of a continuing fragment: dh_j += w_{j-r} dz[s+r] for j >= r
#pragma unroll
              for (int j = r; j < 3; ++j)
#pragma unroll
                for (int ch = 0; ch < CPL; ++ch) dh[j][ch] = __builtin_fmaf(wk[j - r][ch], g[r % 4][ch], dh[j][ch]);
            }
            if (q - 3 >= t) {
              // dx[q-3] = w3 dz[q-3] + w2 dz[q-2] + w1 dz[q-1] + w0 dz[q]
              float d[CPL];
#pragma unroll
              for (int ch = 0; ch < CPL; ++ch) {
                float v = wk[3][ch] * g[(r + 1) % 4][ch];
                v = __builtin_fmaf(wk[2][ch], g[(r + 2) % 4][ch], v);
                v = __builtin_fmaf(wk[1][ch], g[(r + 3) % 4][ch], v);
                v = __builtin_fmaf(wk[0][ch], g[r % 4][ch], v);
                d[ch] = v;
              }
              if (active) store_row<CPL, VEC>(a.dx + (q - 3) * a.dx_ld, c0, C, pack(d));
            }
          }
        }
      }
      if constexpr (MODE != MODE_IDX) {
        if (want_dh && active) {
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

  // ---- block partial: waves 1..3 hand their sums to wave 0 through LDS, added in wave order
  __syncthreads();
  float* red = reinterpret_cast<float*>(&bx[0][0][0]);  // reuse: 3 x 5*CPL x 64 floats
  if (wave > 0) {
#pragma unroll
    for (int k = 0; k < 5; ++k)
#pragma unroll
      for (int ch = 0; ch < CPL; ++ch) red[((wave - 1) * 5 * CPL + k * CPL + ch) * kWave + lane] = acc[k][ch];
  }
  __syncthreads();
  if (wave == 0 && active) {
#pragma unroll
    for (int k = 0; k < 5; ++k) {
      float* dst = a.part + ((int64_t)rb * 5 + k) * C + c0;
#pragma unroll
      for (int ch = 0; ch < CPL; ++ch) {
        float s = acc[k][ch];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) s += red[((w - 1) * 5 * CPL + k * CPL + ch) * kWave + lane];
        if (c0 + ch < C) dst[ch] = s;
      }
    }
  }
}

// Ordered reduce: out[k][c] = sum over row blocks 0, 1, ..., n-1 of part[block][k][c].  One
// thread per (k, c); the extra threads write zero d(history) rows of empty continuing fragments.
__global__ void __launch_bounds__(kThreads) conv1d_bwd_reduce_kernel(const BwdArgs a, int64_t nhist_zero) {
  const int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t C = a.C;
  if (gid < 5 * C) {
    const int64_t k = gid / C, c = gid - k * C;
    if (k == 4 && !a.db) return;
    const float* p = a.part + k * C + c;
    const int64_t stride = 5 * C;
    float s = 0.f;
    const int64_t n = a.n_rowblocks;
    int64_t i = 0;
    for (; i + 8 <= n; i += 8) {
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = p[(i + j) * stride];
#pragma unroll
      for (int j = 0; j < 8; ++j) s += v[j];
    }
    for (; i < n; ++i) s += p[i * stride];
    if (k < 4) a.dw[c * 4 + k] = s;
    else a.db[c] = s;
    return;
  }
  const int64_t hid = gid - 5 * C;
  if (hid >= nhist_zero * C) return;
  const int64_t i = hid / C, c = hid - i * C;
  if (a.hist.has_hist && !a.hist.has_hist[i]) return;
  if (a.seq.cu[i + 1] != a.seq.cu[i]) return;  // nonempty: written by the tile kernel
#pragma unroll
  for (int j = 0; j < 3; ++j) a.dhist[(i * 3 + j) * C + c] = 0;
}

// ------------------------------------------------------------------ launchers
constexpr int kCpl = 8;

template <int MODE, bool VEC, bool SILU>
static hipError_t bwd_go(const BwdArgs& a, hipStream_t s) {
  const uint32_t blocks = a.n_strips * a.n_rowblocks;
  if (blocks) {
    void* args[] = {const_cast<BwdArgs*>(&a)};
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&conv1d_bwd_kernel<kCpl, VEC, MODE, SILU>),
                                   dim3(blocks), dim3(kThreads), args, 0, s);
    if (e != hipSuccess) return e;
  }
  // empty fragments that read history rows still get a (zero) d(history)
  const int64_t nz = (a.dhist && MODE == MODE_CU) ? a.seq.nseq : 0;
  const int64_t threads = 5 * a.C + nz * a.C;
  const uint32_t rblocks = (uint32_t)((threads + kThreads - 1) / kThreads);
  int64_t nz_arg = nz;
  void* rargs[] = {const_cast<BwdArgs*>(&a), &nz_arg};
  return hipLaunchKernel(reinterpret_cast<const void*>(&conv1d_bwd_reduce_kernel), dim3(rblocks), dim3(kThreads),
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
