// conv1d_cf.hip -- channels-first [B, D, T] forward and backward of the width-4 causal
// depthwise Conv1d.
//
// Layout: the one Megatron-Core core.ssm.causal_conv1d contrasts with channel-last in
// assert_causal_conv1d_deterministic.  There, each dweight element takes one contribution per
// batch row rather than batch * ceil(seqlen / 128).  T is contiguous and every (b, d) row is one
// sequence with zero history.  Same operation as the channel-last kernels: z = b, then taps 0..3
// as FP32 FMAs (tap 3 on the current step), y = act(z) in bf16.
//
// Tiling (HBM-bound, no MFMA): one wave per (b, d) row, the four waves of a block on four
// consecutive rows, so a block's accesses stay inside one compact stretch of memory.  In each
// 512-step block of a row, lane l owns steps 8l .. 8l+7: one 16-byte load and store per lane,
// fully coalesced.  The three steps before a lane's first come from lane l-1 by a wave shuffle,
// or for lane 0 from lane 63 of the previous block (kept in scalar registers).  A row's blocks
// are loaded kCfUnroll (forward) or kCfUnrollBwd (backward) at a time.
//
// Backward: dz is recomputed per block.  dx of a block needs dz of the three steps after each
// lane: lanes 0..62 take them from lane l+1 by a shuffle, lane 63 from lane 0 of the next block.
// So a block's dx is written one block later, from its dz kept in registers; after the row's
// last block, the steps past T have dz = 0.  Each lane accumulates its dweight/dbias sums in step
// order.  At the end of the row a fixed shuffle tree adds the 64 lanes and lane 0 writes the
// row's [5] partial to part[b][k][d].  The ordered reduce then adds the B partials of each
// channel in a fixed order: bitwise reproducible, no atomics.
#include "conv1d_device.h"

namespace cconv {

constexpr int kCfSteps = 8;                // time steps per lane per 512-step block
constexpr int kCfBlock = kWave * kCfSteps;  // 512
#ifndef CCONV_CF_UNROLL
#define CCONV_CF_UNROLL 4
#endif
#ifndef CCONV_CF_UNROLL_BWD
#define CCONV_CF_UNROLL_BWD 2
#endif
constexpr int kCfUnroll = CCONV_CF_UNROLL;         // forward: blocks loaded together
constexpr int kCfUnrollBwd = CCONV_CF_UNROLL_BWD;  // backward (two streams): 2 blocks, ~1% faster than 4
constexpr int kCfRowsPerBlock = kBlockThreads / kWave;

// Steps t .. t+7 of a row into four packed dwords (zeros past T).  VEC: T % 8 == 0 and the row
// start is 16-byte aligned, so a lane's eight steps are either all inside or all past T.
template <bool VEC>
__device__ __forceinline__ void cf_load(uint32_t (&v)[4], const uint16_t* __restrict__ row, int64_t t, int64_t T) {
  if constexpr (VEC) {
    if (t < T) {
      const u32x4 q = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(row + t));
      v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
    } else {
      v[0] = v[1] = v[2] = v[3] = 0u;
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t lo = t + 2 * j < T ? row[t + 2 * j] : 0u;
      const uint32_t hi = t + 2 * j + 1 < T ? row[t + 2 * j + 1] : 0u;
      v[j] = lo | (hi << 16);
    }
  }
}

template <bool VEC>
__device__ __forceinline__ void cf_store(uint16_t* __restrict__ row, int64_t t, int64_t T, const float (&f)[8]) {
  uint32_t v[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) v[j] = pack_bf16x2(f[2 * j], f[2 * j + 1]);
  if constexpr (VEC) {
    if (t < T) __builtin_nontemporal_store(u32x4{v[0], v[1], v[2], v[3]}, reinterpret_cast<u32x4*>(row + t));
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (t + 2 * j < T) row[t + 2 * j] = (uint16_t)(v[j] & 0xffffu);
      if (t + 2 * j + 1 < T) row[t + 2 * j + 1] = (uint16_t)(v[j] >> 16);
    }
  }
}

// e[0..H-1] = the H steps before the lane's first, e[H..H+7] = its eight steps (H = 3 up to
// width four, 7 up to width eight: at most one lane's eight steps back).  They come from lane
// l-1; lane 0 takes the previous block's lane 63 (c[0..3], its four dwords).
template <int H>
__device__ __forceinline__ void cf_window(float (&e)[H + 8], const uint32_t (&v)[4], const uint32_t (&c)[4], int lane) {
  static_assert(H >= 1 && H <= 7, "history of one lane at most");
  constexpr int D0 = (8 - H) / 2;  // first dword of lane l-1 that holds a needed step
  uint32_t p[4];
#pragma unroll
  for (int q = D0; q < 4; ++q) {
    p[q] = __shfl_up(v[q], 1);
    if (lane == 0) p[q] = c[q];
  }
#pragma unroll
  for (int i = 0; i < H; ++i) {  // step 8-H+i of lane l-1
    const int st = 8 - H + i;
    e[i] = (st & 1) ? bf16_hi(p[st >> 1]) : bf16_lo(p[st >> 1]);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    e[H + 2 * j] = bf16_lo(v[j]);
    e[H + 1 + 2 * j] = bf16_hi(v[j]);
  }
}

// Taps [D, W] in the last W of R slots (slot R-1 on the current step; R = 4 up to width four, 8
// up to width eight); leading slots are zero and never used (every tap loop starts at R - W).
template <int W, int R = Win<W>::R>
__device__ __forceinline__ void cf_taps(const CfArgs& a, int64_t d, float (&wk)[R], float& bias) {
#pragma unroll
  for (int k = 0; k < R; ++k) {
    const int64_t i = d * W + (k - (R - W));
    wk[k] = k < R - W ? 0.f
                      : (a.w_f32 ? static_cast<const float*>(a.w)[i]
                                 : __uint_as_float((uint32_t)static_cast<const uint16_t*>(a.w)[i] << 16));
  }
  bias = 0.f;
  if (a.b) bias = a.b_f32 ? static_cast<const float*>(a.b)[d]
                          : __uint_as_float((uint32_t)static_cast<const uint16_t*>(a.b)[d] << 16);
}

// ------------------------------------------------------------------ forward
template <bool VEC, bool SILU, int W>
__global__ void __launch_bounds__(kBlockThreads) conv1d_fwd_cf_kernel(const CfArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t row = (int64_t)blockIdx.x * kCfRowsPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (row >= a.B * a.D) return;
  const int64_t bi = row / a.D, d = row - bi * a.D, T = a.T;
  const uint16_t* x = a.x + bi * a.x_sb + d * a.x_sd;
  uint16_t* y = a.out + bi * a.o_sb + d * a.o_sd;
  constexpr int R = Win<W>::R, H = Win<W>::H;
  float wk[R], bias;
  cf_taps<W>(a, d, wk, bias);
  uint32_t c[4] = {0u, 0u, 0u, 0u};  // steps before the row: zero history
  for (int64_t t0 = 0; t0 < T; t0 += (int64_t)kCfUnroll * kCfBlock) {
    uint32_t v[kCfUnroll][4];
#pragma unroll
    for (int u = 0; u < kCfUnroll; ++u) cf_load<VEC>(v[u], x, t0 + u * kCfBlock + lane * kCfSteps, T);
#pragma unroll
    for (int u = 0; u < kCfUnroll; ++u) {
      const int64_t tb = t0 + u * kCfBlock;
      if (tb >= T) break;
      float e[H + 8], out[8];
      cf_window<H>(e, v[u], c, lane);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float z = bias;
#pragma unroll
        for (int k = R - W; k < R; ++k) z = __builtin_fmaf(wk[k], e[j + k], z);
        out[j] = SILU ? z * sigmoid_f32(z) : z;
      }
      cf_store<VEC>(y, tb + lane * kCfSteps, T, out);
#pragma unroll
      for (int q = 0; q < 4; ++q) c[q] = __builtin_amdgcn_readlane(v[u][q], kWave - 1);
    }
  }
}

// ------------------------------------------------------------------ backward
// dx of the eight steps of a lane from their dz and the dz of the next H steps (n[0..H-1]);
// tap slot k multiplies the dz R-1-k steps later, slots below R - W are left out.
template <int W, int R = Win<W>::R>
__device__ __forceinline__ void cf_dx(float (&dx)[8], const float (&dz)[8], const float (&n)[R - 1],
                                      const float (&wk)[R]) {
  float g[R + 7];
#pragma unroll
  for (int j = 0; j < 8; ++j) g[j] = dz[j];
#pragma unroll
  for (int i = 0; i < R - 1; ++i) g[8 + i] = n[i];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float s = wk[R - 1] * g[j];
#pragma unroll
    for (int k = R - 2; k >= R - W; --k) s = __builtin_fmaf(wk[k], g[j + R - 1 - k], s);
    dx[j] = s;
  }
}

template <bool VEC, bool SILU, int W>
__global__ void __launch_bounds__(kBlockThreads) conv1d_bwd_cf_kernel(const CfArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t row = (int64_t)blockIdx.x * kCfRowsPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (row >= a.B * a.D) return;
  const int64_t bi = row / a.D, d = row - bi * a.D, T = a.T;
  const uint16_t* x = a.x + bi * a.x_sb + d * a.x_sd;
  const uint16_t* dy = a.dy + bi * a.dy_sb + d * a.dy_sd;
  uint16_t* dx = a.out + bi * a.o_sb + d * a.o_sd;
  constexpr int R = Win<W>::R, H = Win<W>::H;
  float wk[R], bias;
  cf_taps<W>(a, d, wk, bias);
  float acc[R + 1];  // tap slots, then db
#pragma unroll
  for (int k = 0; k <= R; ++k) acc[k] = 0.f;
  float pdz[8];              // dz of the previous block (its dx is still to be written)
  int64_t ptb = -1;          // start of that block, -1 = none
  uint32_t c[4] = {0u, 0u, 0u, 0u};
  for (int64_t t0 = 0; t0 < T; t0 += (int64_t)kCfUnrollBwd * kCfBlock) {
    uint32_t v[kCfUnrollBwd][4], gv[kCfUnrollBwd][4];
#pragma unroll
    for (int u = 0; u < kCfUnrollBwd; ++u) {
      const int64_t t = t0 + u * kCfBlock + lane * kCfSteps;
      cf_load<VEC>(v[u], x, t, T);
      cf_load<VEC>(gv[u], dy, t, T);
    }
#pragma unroll
    for (int u = 0; u < kCfUnrollBwd; ++u) {
      const int64_t tb = t0 + u * kCfBlock;
      if (tb >= T) break;
      const int64_t t = tb + lane * kCfSteps;
      float e[H + 8], dz[8];
      cf_window<H>(e, v[u], c, lane);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float z = bias;
#pragma unroll
        for (int k = R - W; k < R; ++k) z = __builtin_fmaf(wk[k], e[j + k], z);
        float g = (j & 1) ? bf16_hi(gv[u][j >> 1]) : bf16_lo(gv[u][j >> 1]);
        if (SILU) {
          const float sg = sigmoid_f32(z);
          g = g * (sg * __builtin_fmaf(z, 1.0f - sg, 1.0f));
        }
        dz[j] = g;
      }
      if (tb + kCfBlock > T) {  // a row's last block may be partial (wave-uniform test): no gradient past T
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (t + j >= T) dz[j] = 0.f;
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
#pragma unroll
        for (int k = R - W; k < R; ++k) acc[k] = __builtin_fmaf(dz[j], e[j + k], acc[k]);
        acc[R] += dz[j];
      }
      if (ptb >= 0) {  // the previous block's dx: lane 63 takes this block's first H dz
        float n[H];
#pragma unroll
        for (int i = 0; i < H; ++i) {
          n[i] = __shfl_down(pdz[i], 1);
          const float h = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(dz[i]), 0));
          if (lane == kWave - 1) n[i] = h;
        }
        float o[8];
        cf_dx<W>(o, pdz, n, wk);
        cf_store<VEC>(dx, ptb + lane * kCfSteps, T, o);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) pdz[j] = dz[j];
      ptb = tb;
#pragma unroll
      for (int q = 0; q < 4; ++q) c[q] = __builtin_amdgcn_readlane(v[u][q], kWave - 1);
    }
  }
  if (ptb >= 0) {  // the last block: no steps after it
    float n[H];
#pragma unroll
    for (int i = 0; i < H; ++i) {
      n[i] = __shfl_down(pdz[i], 1);
      if (lane == kWave - 1) n[i] = 0.f;
    }
    float o[8];
    cf_dx<W>(o, pdz, n, wk);
    cf_store<VEC>(dx, ptb + lane * kCfSteps, T, o);
  }
  // the row's partial: a fixed butterfly over the 64 lanes, lane 0 writes
#pragma unroll
  for (int k = 0; k <= R; ++k) {
    float s = acc[k];
    s += __shfl_xor(s, 32);
    s += __shfl_xor(s, 16);
    s += __shfl_xor(s, 8);
    s += __shfl_xor(s, 4);
    s += __shfl_xor(s, 2);
    s += __shfl_xor(s, 1);
    if (lane == 0) a.part[(bi * (R + 1) + k) * a.D + d] = s;
  }
}

// ------------------------------------------------------------------ launchers
template <bool VEC, bool SILU, int W>
static hipError_t cf_go(const CfArgs& a, bool bwd, hipStream_t s) {
  const int64_t rows = a.B * a.D;
  const uint32_t blocks = (uint32_t)((rows + kCfRowsPerBlock - 1) / kCfRowsPerBlock);
  void* args[] = {const_cast<CfArgs*>(&a)};
  const void* fn = bwd ? reinterpret_cast<const void*>(&conv1d_bwd_cf_kernel<VEC, SILU, W>)
                       : reinterpret_cast<const void*>(&conv1d_fwd_cf_kernel<VEC, SILU, W>);
  return hipLaunchKernel(fn, dim3(blocks), dim3(kBlockThreads), args, 0, s);
}

template <int W>
static hipError_t cf_width(const CfArgs& a, bool vec, bool silu, bool bwd, hipStream_t s) {
  if (vec) return silu ? cf_go<true, true, W>(a, bwd, s) : cf_go<true, false, W>(a, bwd, s);
  return silu ? cf_go<false, true, W>(a, bwd, s) : cf_go<false, false, W>(a, bwd, s);
}

static hipError_t cf_dispatch(const CfArgs& a, bool vec, bool silu, bool bwd, hipStream_t s) {
  if (a.B * a.D == 0) return hipSuccess;
  switch (a.width) {
    case 2: return cf_width<2>(a, vec, silu, bwd, s);
    case 3: return cf_width<3>(a, vec, silu, bwd, s);
    case 5: return cf_width<5>(a, vec, silu, bwd, s);
    case 6: return cf_width<6>(a, vec, silu, bwd, s);
    case 7: return cf_width<7>(a, vec, silu, bwd, s);
    case 8: return cf_width<8>(a, vec, silu, bwd, s);
    default: return cf_width<4>(a, vec, silu, bwd, s);
  }
}

hipError_t launch_fwd_cf(const CfArgs& a, bool vec, bool silu, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  return cf_dispatch(a, vec, silu, false, s);
}

hipError_t launch_bwd_cf(const CfArgs& a, bool vec, bool silu, hipStream_t s) {
  return cf_dispatch(a, vec, silu, true, s);
}

}  // namespace cconv
