// conv1d_bwd.hip -- training backward of the packed depthwise causal Conv1d (filter width 4;
// widths 2..8 as well).
//
// Operation: the gradients of the forward in conv1d_fwd.hip for the training path of FlashInfer
// cake_causal_conv1d_kcp (Returns: dx, a deterministic FP32 dweight, and the gradient of the
// history rows that the preceding fragment supplied) and Megatron-Core causal_conv1d_cp.  With
// W taps, z[t] = b + sum_k w_k u[t-(W-1)+k] and dz[t] = dy[t] * act'(z[t]):
//     dx[t]  = sum_k w_k dz[t+(W-1)-k]       (terms inside t's sequence only)
//     dw_k   = sum_t dz[t] u[t-(W-1)+k],  db = sum_t dz[t]
//     dh_j   = sum_{tau <= j} w_{j-tau} dz[s+tau]   (history row j of a continuing fragment)
//
// Tiling: waves side by side in channels as in the forward (lane = CPL channels), but where the
// forward launches many rounds of short tiles, the backward launches one round of about kBwdBlocks
// long row ranges, one dweight/dbias partial each.  The window is a ring of R register slots (R = 4
// up to width four, 8 up to width eight) with H = R - 1 history rows.  A wave streams x and dy over
// its own rows [ta, tb) and up to H look-ahead rows of the sequence that holds row tb - 1; the H
// look-behind and the look-ahead rows belong to the neighbouring ranges (cached loads).  The step
// at row q produces the value of row q - H (at width four: w3 dz[q-3] + w2 dz[q-2] + w1 dz[q-1] +
// w0 dz[q]): dx when q - H is a row of q's sequence, d(history) row j when it is the sequence's
// history row j (the dz ring holds zeros before a sequence's start).  Where a sequence ends, the
// values of its last H rows are flushed with the dz of later rows left out (plus the caller's
// d(tail) rows, the gradient arriving from the next fragment, when the sequence is the array's
// last), and the stream goes straight on.
//
// dweight/dbias are deterministic by construction: each lane accumulates its channels over its
// rows in row order (FP32) and owns those channels for the whole row range, so the range's
// [R + 1, C] partial is written straight from registers to the workspace, and a second kernel
// adds the partials of all row ranges in ascending range order.  No atomics anywhere, so the bits
// depend only on the input values and the range length, never on scheduling or on the
// workspace address.
#include <mutex>
#include <type_traits>

#include "conv1d_device.h"

namespace cconv {

// Width W: W-1 history rows fill the last W-1 of the H window slots (j >= R-W), the rest stay zero.
template <int CPL, bool VEC, int W, int H = Win<W>::H>
__device__ __forceinline__ void load_hist_rows(const HistArgs& hist, int64_t idx, int64_t c0, int64_t C,
                                               bool active, float (&h)[H][CPL]) {
  constexpr int R = Win<W>::R;
#pragma unroll
  for (int j = 0; j < H; ++j)
#pragma unroll
    for (int ch = 0; ch < CPL; ++ch) h[j][ch] = 0.f;
  if (idx >= 0 && hist.ptr && active && (!hist.has_hist || hist.has_hist[idx])) {
#pragma unroll
    for (int j = R - W; j < H; ++j)
      unpack(load_row<CPL, VEC>(hist.ptr + (idx * (W - 1) + j - (R - W)) * C, c0, C), h[j]);
  }
}

#ifndef CCONV_BWD_CHUNK
#define CCONV_BWD_CHUNK 4
#endif
#ifndef CCONV_BWD_PIPELINE
#define CCONV_BWD_PIPELINE 1
#endif
#ifndef CCONV_BWD_DEPTH
#define CCONV_BWD_DEPTH 2
#endif


constexpr float kNegLog2e = -1.44269504088896341f;  // -1 / ln(2)

// Per-lane state of the backward stream (CPL channels) with a ring of R slots.
template <int CPL, int R>
struct BwdState {
  float wk[R][CPL], bias[CPL];  // with SiLU: taps and bias times -log2(e) (see bwd_row)
  float u[R][CPL];        // extended-sequence ring, slot = (row - run start) mod R
  float g[R][CPL];        // dz ring, same slots
  float acc[R + 1][CPL];  // dw per tap slot, then db: partial sums over the wave's rows
};

// One real row q (ring slot r): recompute z, dz = dy * act'(z); dweight/dbias sums when `own`.
// Tap slot k (k = R-W .. R-1) reads ring slot (r+1+k) % R: rows q-(R-1) .. q.
// With SiLU the whole stream runs scaled, to save the multiply in front of the exp2: taps and
// bias hold -log2(e) times their values, so the recompute yields zs = -log2(e) z, the exponent
// of sigma(z) = 1 / (1 + 2^zs); and the dz ring holds dzs = -ln(2) dz, so a tap times a dz ring
// value is w dz again (dx, d(history)), while the dweight/dbias sums come out as -ln(2) times
// theirs and are scaled back once, when the partial is written.
//   -ln2 (1 + z (1 - sigma)) = zs * ln2^2 (1 - sigma) - ln2,  since z = -ln2 zs.
template <int CPL, bool SILU, int W, int R = Win<W>::R>
__device__ __forceinline__ void bwd_row(BwdState<CPL, R>& st, const Pk<CPL>& xr, const Pk<CPL>& gr, int r, bool own) {
  constexpr float kLn2 = 0.693147180559945309f;
  constexpr float kLn2Sq = 0.480453013918201424f;
  unpack(xr, st.u[r % R]);
  float dyv[CPL];
  unpack(gr, dyv);
#pragma unroll
  for (int ch = 0; ch < CPL; ++ch) {
    float z = st.bias[ch];
#pragma unroll
    for (int k = R - W; k < R; ++k) z = __builtin_fmaf(st.wk[k][ch], st.u[(r + 1 + k) % R][ch], z);
    float dz = dyv[ch];
    if constexpr (SILU) {
      const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(z));  // z is zs here
      const float t = __builtin_fmaf(sg, -kLn2Sq, kLn2Sq);                         // ln2^2 (1 - sigma)
      dz = dz * (sg * __builtin_fmaf(z, t, -kLn2));                                // dzs
    }
    st.g[r % R][ch] = dz;
  }
  if (own) {
#pragma unroll
    for (int ch = 0; ch < CPL; ++ch) {
#pragma unroll
      for (int k = R - W; k < R; ++k)
        st.acc[k][ch] = __builtin_fmaf(st.g[r % R][ch], st.u[(r + 1 + k) % R][ch], st.acc[k][ch]);
      st.acc[R][ch] += st.g[r % R][ch];
    }
  }
}

// The value of row p = q - (R-1) at step q (ring slot r of row q): sum over tap slots k of
// w_k dz[p + R-1-k], i.e. the last tap on dz[p] and the first tap on dz[p + W-1]; tap slots below
// R-W left out (slot k reads ring slot (r+R-k) % R).  Ring slots of rows before a sequence's
// start hold dz = 0, so for the rows before a sequence this is the gradient of its history rows.
template <int CPL, int W, int R = Win<W>::R>
__device__ __forceinline__ void bwd_back(const BwdState<CPL, R>& st, int r, float (&d)[CPL]) {
#pragma unroll
  for (int ch = 0; ch < CPL; ++ch) {
    float v = st.wk[R - 1][ch] * st.g[(r + 1) % R][ch];
#pragma unroll
    for (int k = R - 2; k >= R - W; --k) v = __builtin_fmaf(st.wk[k][ch], st.g[(r + R - k) % R][ch], v);
    d[ch] = v;
  }
}

// The sequence a wave is streaming, and whether this wave writes its d(history) rows (it holds
// the sequence's first row and the sequence reads caller history rows).
struct BwdSeq {
  SeqDesc sd;
  bool dh;
};

// Where the value of row p goes: dx when p is a row of the current sequence inside the wave's own
// range [ta, tb); d(history) row p - s + W - 1 when p is one of the W-1 history rows of a
// sequence whose head this wave streams; nowhere otherwise (rows of the neighbouring ranges, and
// for W < 4 the rows before the history).
template <int CPL, bool VEC, int W>
__device__ __forceinline__ void bwd_route(const BwdArgs& a, const BwdSeq& cs, int64_t p, int64_t ta, int64_t tb,
                                          const float (&v)[CPL], int64_t c0, bool active) {
  if (p >= cs.sd.s) {
    if (p >= ta && p < tb && active) store_row<CPL, VEC, true>(a.dx + p * a.dx_ld, c0, a.C, pack(v));
  } else if (cs.dh && active && p - cs.sd.s + W - 1 >= 0) {
    store_row<CPL, VEC>(a.dhist + (cs.sd.idx * (W - 1) + (p - cs.sd.s + W - 1)) * a.C, c0, a.C, pack(v));
  }
}

// Is sd the last sequence of the call (the one whose tail continues into the next shard)?
template <int MODE>
__device__ __forceinline__ bool bwd_is_last(const BwdArgs& a, const SeqDesc& sd) {
  if constexpr (MODE == MODE_IDX) {
    return sd.e >= a.rows;  // no empty sequences in this form: the last one ends at the last row
  } else {
    return sd.idx == a.seq.nseq - 1;
  }
}

// The current sequence ends right before row e (ring slot r): the values of its last H rows
// e-H .. e-1 only take dz of rows before e (tap slots below R-W left out), summed in the order of
// bwd_back.  For the last sequence of the call, the next shard's gradient of the last W-1 values
// of its extended sequence (d(tail) row j: the value W-1-j rows before e) is added in FP32
// before the single rounding; values before the sequence's first row go to its d(history) rows
// like every other value there (cake_causal_conv1d_kcp, Returns).
template <int CPL, bool VEC, int MODE, int W, int R = Win<W>::R>
__device__ __forceinline__ void bwd_flush(const BwdArgs& a, const BwdState<CPL, R>& st, const BwdSeq& cs, int r,
                                          int64_t e, int64_t ta, int64_t tb, int64_t c0, bool active) {
  constexpr int H = R - 1;
  float v[H][CPL];  // v[j-1]: row e - j
#pragma unroll
  for (int j = H; j >= 1; --j) {
#pragma unroll
    for (int ch = 0; ch < CPL; ++ch) {
      // tap slot k of row e-j reads dz of row e-j+R-1-k, ring slot (r + 2R-1-j-k) % R
      float t = st.wk[R - 1][ch] * st.g[(r + R - j) % R][ch];
#pragma unroll
      for (int k = R - 2; k >= (R - W > R - j ? R - W : R - j); --k)
        t = __builtin_fmaf(st.wk[k][ch], st.g[(r + 2 * R - 1 - j - k) % R][ch], t);
      v[j - 1][ch] = t;
    }
  }
  if (a.dtail && active && bwd_is_last<MODE>(a, cs.sd)) {
#pragma unroll
    for (int j = 1; j <= W - 1; ++j) {
      float f[CPL];
      unpack(load_row<CPL, VEC>(a.dtail + (int64_t)(W - 1 - j) * a.C, c0, a.C), f);
#pragma unroll
      for (int ch = 0; ch < CPL; ++ch) v[j - 1][ch] += f[ch];
    }
  }
#pragma unroll
  for (int j = H; j >= 1; --j) bwd_route<CPL, VEC, W>(a, cs, e - j, ta, tb, v[j - 1], c0, active);
}

template <int MODE>
__device__ __forceinline__ bool bwd_wants_dh(const BwdArgs& a, const SeqDesc& sd) {
  if constexpr (MODE == MODE_IDX) {
    return false;  // caller history rows need the cu_seqlens or batch-row form
  } else {
    return a.dhist && (!a.hist.has_hist || a.hist.has_hist[sd.idx]);
  }
}

// Row q = cs.sd.s (ring slot r), the first row of a sequence, is next: the H window slots take
// its history and dz = 0.
template <int CPL, bool VEC, int MODE, int W, int R = Win<W>::R>
__device__ __forceinline__ void bwd_enter(const BwdArgs& a, BwdState<CPL, R>& st, BwdSeq& cs, int r, int64_t c0,
                                          bool active) {
  constexpr int H = R - 1;
  float h[H][CPL];
  if constexpr (MODE != MODE_IDX) {
    load_hist_rows<CPL, VEC, W>(a.hist, cs.sd.idx, c0, a.C, active, h);
  } else {
#pragma unroll
    for (int j = 0; j < H; ++j)
#pragma unroll
      for (int ch = 0; ch < CPL; ++ch) h[j][ch] = 0.f;
  }
  cs.dh = bwd_wants_dh<MODE>(a, cs.sd);
#pragma unroll
  for (int j = 0; j < H; ++j)
#pragma unroll
    for (int ch = 0; ch < CPL; ++ch) {
      st.u[(r + 1 + j) % R][ch] = h[j][ch];
      st.g[(r + 1 + j) % R][ch] = 0.f;
    }
}

// CH rows starting at q0 (ring slot of row q0 + r is r mod R).  The stream covers the own rows
// [ta, tb) and then up to H look-ahead rows of the sequence that holds row tb - 1, which finish
// the last dx rows; it ends (done) at that sequence's end or at tb + H.  A chunk of own rows of
// one sequence, at least H rows past both its start and the range start, is a straight
// recompute-and-dx; any other chunk takes the row-by-row path.
template <int CPL, bool VEC, int MODE, int CH, bool SILU, bool FULL, int W, int R = Win<W>::R>
__device__ __forceinline__ void bwd_chunk(const BwdArgs& a, BwdState<CPL, R>& st, BwdSeq& cs, const Pk<CPL> (&X)[CH],
                                          const Pk<CPL> (&G)[CH], int64_t q0, int64_t ta, int64_t tb, int64_t dend,
                                          int64_t lim, int64_t c0, bool active, bool& done) {
  constexpr int H = R - 1;
  if (q0 + CH <= tb && cs.sd.e >= q0 + CH && q0 >= cs.sd.s + H && q0 >= ta + H) {
#pragma unroll
    for (int r = 0; r < CH; ++r) {
      bwd_row<CPL, SILU, W>(st, X[r], G[r], r, true);
      float d[CPL];
      bwd_back<CPL, W>(st, r, d);
      if (FULL || active) store_row<CPL, VEC, true>(a.dx + (q0 + r - H) * a.dx_ld, c0, a.C, pack(d));
    }
    return;
  }
#pragma unroll
  for (int r = 0; r < CH; ++r) {
    const int64_t q = q0 + r;
    if (!done && q == cs.sd.e) {
      bwd_flush<CPL, VEC, MODE, W>(a, st, cs, r, q, ta, tb, c0, active);
      if (q >= tb) {
        done = true;
      } else {
        cs.sd = next_seq<MODE>(a.seq, cs.sd, dend, lim);
        bwd_enter<CPL, VEC, MODE, W>(a, st, cs, r, c0, active);
      }
    }
    if (!done && q >= tb + H) done = true;
    if (!done) {
      bwd_row<CPL, SILU, W>(st, X[r], G[r], r, q < tb);
      float d[CPL];
      bwd_back<CPL, W>(st, r, d);
      bwd_route<CPL, VEC, W>(a, cs, q - H, ta, tb, d, c0, active);
    }
  }
}

// CH rows of x and dy from q0; past the last full chunk (last row qlast) it re-reads that chunk
template <int CPL, bool VEC, int CH>
__device__ __forceinline__ void bwd_load(Pk<CPL> (&X)[CH], Pk<CPL> (&G)[CH], const BwdArgs& a, int64_t q0, int64_t qlast,
                                         int64_t c0) {
  const int64_t qs = q0 + CH - 1 <= qlast ? q0 : qlast - (CH - 1);
  const uint16_t* xr = a.x + qs * a.x_ld;
  const uint16_t* gr = a.dy + qs * a.dy_ld;
#pragma unroll
  for (int r = 0; r < CH; ++r) {
    X[r] = load_row<CPL, VEC, true>(xr + r * a.x_ld, c0, a.C);
    G[r] = load_row<CPL, VEC, true>(gr + r * a.dy_ld, c0, a.C);
  }
}

// Occupancy floor: a launch is sized for 4 waves per SIMD (one round of ~1024 blocks), so every
// width-four variant is held to 128 VGPRs (an earlier form of the per-token-ID variant took 131
// and fell to 3 waves).  They fit without spilling: the kernel-resource test checks that no
// kernel uses scratch or LDS.
#ifndef CCONV_BWD_WAVES_PER_EU
#define CCONV_BWD_WAVES_PER_EU 4
#endif
// The floor holds for widths up to four.  The eight-slot ring of wider filters needs more than
// 128 VGPRs: width five fits 168 (3 waves per SIMD) without spilling except in the per-token-ID
// form; widths six to eight spill under that floor (and ran 9-20% slower), so the rest run at
// the occupancy their registers allow.
#if CCONV_BWD_WAVES_PER_EU > 0
#define CCONV_BWD_OCCUPANCY                                                                 \
  __attribute__((amdgpu_waves_per_eu(W <= 4                           ? CCONV_BWD_WAVES_PER_EU \
                                     : (W == 5 && MODE != MODE_IDX) ? 3                        \
                                                                    : 1)))
#else
#define CCONV_BWD_OCCUPANCY
#endif

template <int CPL, bool VEC, int MODE, bool SILU, int W>
__global__ void __launch_bounds__(kBlockThreads) CCONV_BWD_OCCUPANCY conv1d_bwd_kernel(const BwdArgs a) {
  constexpr int R = Win<W>::R, H = Win<W>::H;  // ring slots, history values
  constexpr int CH = CCONV_BWD_CHUNK % R == 0 ? CCONV_BWD_CHUNK : R;  // rows per unrolled chunk
  static_assert(CH % R == 0, "chunks must keep the ring slot of a row fixed");

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint32_t strip, rb;
  block_tile(a.tile_order, a.n_strips, a.n_rowblocks, strip, rb);
  const int64_t C = a.C;
  const int64_t wc0 = (int64_t)strip * kBlockChannels + (int64_t)wave * kWaveChannels;
  if (wc0 >= C) return;  // the whole wave is past the last channel: no partial to write
  // With vectors, the lanes of a partly active wave that lie past the last channel work as copies
  // of the wave's last channel pair: the same loads and arithmetic, and stores of the same bits
  // (dx, d(history), the range's partial sums) to the same addresses in the same instructions
  // (lanes never exchange data).  Every wave then streams through the pipeline unpredicated.
  // With an odd C the lane of the lone last channel takes the pair (C-2, C-1); channel C-2 is then
  // computed twice, perhaps in two waves, over the same rows in the same order, so both store the
  // same bits.  No output overlaps an input, so the order of those stores does not matter.
  const int64_t c0 = VEC && wc0 + lane * CPL + (CPL - 1) >= C ? C - CPL : wc0 + lane * CPL;
  const bool active = VEC || c0 < C;
  const int64_t dend = data_end<MODE>(a.seq, a.rows);

  int64_t ta = (int64_t)rb * a.range_rows;
  int64_t tb = ta + a.range_rows;
  ta = ta < dend ? ta : dend;
  tb = tb < dend ? tb : dend;

  BwdState<CPL, R> st;
#pragma unroll
  for (int k = 0; k < R + 1; ++k)
#pragma unroll
    for (int ch = 0; ch < CPL; ++ch) st.acc[k][ch] = 0.f;

  if (ta < tb) {
    load_taps<CPL, W>(a.w, a.w_f32, a.b, a.b_f32, c0, C, st.wk, st.bias);
    if constexpr (SILU) {  // the scaled stream of bwd_row
#pragma unroll
      for (int ch = 0; ch < CPL; ++ch) {
#pragma unroll
        for (int k = R - W; k < R; ++k) st.wk[k][ch] *= kNegLog2e;
        st.bias[ch] *= kNegLog2e;
      }
    }
    const int64_t lim = (tb + H < dend) ? tb + H : dend;  // sequence ends matter up to tb + H

    // full chunks of own rows, software-pipelined with NB register buffers (see the forward)
    const int nfull = (VEC && CCONV_BWD_PIPELINE) ? (int)((tb - ta) / CH) : 0;
    const int64_t qlast = ta + (int64_t)nfull * CH - 1;
    int64_t q0 = ta;
    constexpr int NB = CCONV_BWD_DEPTH;
    static_assert(NB >= 2, "at least two buffers");
    Pk<CPL> X[NB][CH], G[NB][CH];
    if (nfull > 0) {  // in flight during the set-up
#pragma unroll
      for (int b = 0; b + 1 < NB; ++b) bwd_load<CPL, VEC, CH>(X[b], G[b], a, q0 + b * CH, qlast, c0);
    }

    // the window rows ta-H .. ta-1 and the sequence holding row ta
    Pk<CPL> wrow[H];
    load_window<CPL, VEC, H>(wrow, a.x, a.x_ld, ta, c0, C, active);
    // the look-ahead rows tb .. lim-1 (at most three at widths up to four: the next range's first
    // rows), loaded with the set-up: the end of the range then never waits on a memory round
    // trip.  Named values, not an array: the row select below would otherwise become a runtime
    // index, and the compiler then moved the array to LDS (the backward ran 10% slower).  Wider
    // filters load their look-ahead rows at the end of the range.
    Pk<CPL> lx0 = zero_pk<CPL>(), lx1 = zero_pk<CPL>(), lx2 = zero_pk<CPL>();
    Pk<CPL> lg0 = zero_pk<CPL>(), lg1 = zero_pk<CPL>(), lg2 = zero_pk<CPL>();
    if (H == 3 && active && tb < lim) {
      lx0 = load_row<CPL, VEC>(a.x + tb * a.x_ld, c0, C);
      lg0 = load_row<CPL, VEC>(a.dy + tb * a.dy_ld, c0, C);
    }
    if (H == 3 && active && tb + 1 < lim) {
      lx1 = load_row<CPL, VEC>(a.x + (tb + 1) * a.x_ld, c0, C);
      lg1 = load_row<CPL, VEC>(a.dy + (tb + 1) * a.dy_ld, c0, C);
    }
    if (H == 3 && active && tb + 2 < lim) {
      lx2 = load_row<CPL, VEC>(a.x + (tb + 2) * a.x_ld, c0, C);
      lg2 = load_row<CPL, VEC>(a.dy + (tb + 2) * a.dy_ld, c0, C);
    }
    BwdSeq cs;
    cs.sd = seq_of_row<MODE, H>(a.seq, ta, dend, lim);
    const int64_t dist = ta - cs.sd.s < H ? ta - cs.sd.s : H;
    float h[H][CPL];
    cs.dh = false;
    if constexpr (MODE != MODE_IDX) {
      load_hist_rows<CPL, VEC, W>(a.hist, dist < H ? cs.sd.idx : -1, c0, C, active, h);
      if (dist == 0) cs.dh = bwd_wants_dh<MODE>(a, cs.sd);
    } else {
#pragma unroll
      for (int j = 0; j < H; ++j)
#pragma unroll
        for (int ch = 0; ch < CPL; ++ch) h[j][ch] = 0.f;
    }
    // window rows ta-H..ta-1: the history, then the last `dist` rows of the same sequence (the
    // previous row range streamed them moments earlier on this XCD: cached loads); dz = 0 there
    shift_window<CPL, H>(h, wrow, dist);
#pragma unroll
    for (int j = 0; j < H; ++j)
#pragma unroll
      for (int ch = 0; ch < CPL; ++ch) st.u[j + 1][ch] = h[j][ch];
#pragma unroll
    for (int j = 0; j < R; ++j)
#pragma unroll
      for (int ch = 0; ch < CPL; ++ch) st.g[j][ch] = 0.f;

    bool done = false;
    if (nfull > 0) {
      // NB register buffers, unrolled by NB chunks, look-ahead loads always issued (rows past the
      // last full chunk re-read its last row): see the forward kernel
      // the buffer index is a template constant (step<b>), not a loop variable: at width eight
      // the loop body is too large for the compiler to unroll, and a runtime buffer index moved
      // the buffers to LDS
      bool more = true;
      int j = 0;
      auto step = [&](auto bc) {
        constexpr int b = decltype(bc)::value;
        if (more) {
          bwd_load<CPL, VEC, CH>(X[(b + NB - 1) % NB], G[(b + NB - 1) % NB], a, q0 + (NB - 1) * CH, qlast, c0);
          bwd_chunk<CPL, VEC, MODE, CH, SILU, true, W>(a, st, cs, X[b], G[b], q0, ta, tb, dend, lim, c0, active,
                                                       done);
          q0 += CH;
          more = j + b + 1 < nfull;
        }
      };
      for (; more; j += NB) unroll_steps<NB>(step);
    }
    // the rest: remaining own rows (and partially active waves), then the look-ahead rows
    // (fetched with the set-up at widths up to four: q - tb is 0, 1 or 2 there)
    for (; !done; q0 += CH) {
#pragma unroll
      for (int r = 0; r < CH; ++r) {
        const int64_t q = q0 + r;
        X[0][r] = zero_pk<CPL>();
        G[0][r] = zero_pk<CPL>();
        if (active && q < lim) {
          if (q < tb) {
            X[0][r] = load_row<CPL, VEC, true>(a.x + q * a.x_ld, c0, C);
            G[0][r] = load_row<CPL, VEC, true>(a.dy + q * a.dy_ld, c0, C);
          } else if constexpr (H == 3) {
            X[0][r] = q == tb ? lx0 : (q == tb + 1 ? lx1 : lx2);
            G[0][r] = q == tb ? lg0 : (q == tb + 1 ? lg1 : lg2);
          } else {
            X[0][r] = load_row<CPL, VEC>(a.x + q * a.x_ld, c0, C);
            G[0][r] = load_row<CPL, VEC>(a.dy + q * a.dy_ld, c0, C);
          }
        }
      }
      bwd_chunk<CPL, VEC, MODE, CH, SILU, false, W>(a, st, cs, X[0], G[0], q0, ta, tb, dend, lim, c0, active, done);
    }
  }

  // ---- this lane's partial sums for its channels over this row range (every range writes one,
  // empty ranges write zeros, so the reduce can read all of them)
  if (active) {
    const int rows_out = a.db ? R + 1 : R;  // the dbias row only when it is wanted
    if constexpr (SILU) {  // the sums ran on dzs = -ln(2) dz (bwd_row)
#pragma unroll
      for (int k = 0; k < R + 1; ++k)
#pragma unroll
        for (int ch = 0; ch < CPL; ++ch) st.acc[k][ch] *= kNegLog2e;
    }
#pragma unroll
    for (int k = 0; k < R + 1; ++k) {
      if (k == R && rows_out == R) continue;  // (a compile-time k: a runtime loop bound here moved
                                              // the sums to scratch at the eight-slot widths)
      float* dst = a.part + ((int64_t)rb * (R + 1) + k) * C + c0;
      if constexpr (VEC && CPL >= 4) {
#pragma unroll
        for (int q = 0; q < CPL; q += 4)
          *reinterpret_cast<f32x4*>(dst + q) = f32x4{st.acc[k][q], st.acc[k][q + 1], st.acc[k][q + 2], st.acc[k][q + 3]};
      } else if constexpr (VEC) {
        *reinterpret_cast<f32x2_a4*>(dst) = f32x2{st.acc[k][0], st.acc[k][1]};  // c0 may be odd
      } else {
#pragma unroll
        for (int ch = 0; ch < CPL; ++ch)
          if (c0 + ch < C) dst[ch] = st.acc[k][ch];
      }
    }
  }
}

// Ordered reduce of the per-range partials: out[o] = sum over row ranges p of part[p][o], for
// the flattened o = k*C + c (k = 0..R-1 dweight tap slots, R = dbias; R = 4 up to width four,
// 8 up to width eight).  A wave owns 16 consecutive o;
// lane l sums the ranges p = l/16, l/16 + 4, l/16 + 8, ... in ascending order (each load of
// the wave reads four 64-byte runs; 32 loads are in flight per step, so up to 128 ranges take
// one memory round trip), then a fixed two-level butterfly across lanes l, l^16,
// l^32, l^48 adds the four interleaved subsets:  (s0 + s1) + (s2 + s3).  The order is fixed, so
// dweight/dbias are bitwise reproducible; no atomics.  The remaining threads write zero
// d(history) rows of empty continuing fragments (zeros, or the d(tail) rows when the empty
// fragment is the last sequence: its extended sequence is its history alone).
__global__ void __launch_bounds__(kBlockThreads) conv1d_bwd_reduce_kernel(const BwdArgs a, int64_t nhist_zero,
                                                                           int64_t n_red_waves) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t gwave = ((int64_t)blockIdx.x * kBlockThreads + threadIdx.x) / kWave;
  const int64_t C = a.C;
  const int R = partial_rows(a.width) - 1;
  const int64_t nout = (R + 1) * C;  // the partial's stride; its dbias row is read only when wanted
  if (gwave < n_red_waves) {
    const int64_t o = gwave * 16 + (lane & 15);
    const int sub = lane >> 4;
    const bool ok = o < (a.db ? nout : R * C);
    const int64_t n = a.n_rowblocks;
    float s = 0.f;
    if (ok) {
      // 32 partials of the subset per step, all loads issued before the first add: a call waits
      // for ceil(n / 128) memory round trips, not one per four partials
      const float* p = a.part + o;
      for (int64_t i0 = sub; i0 < n; i0 += 128) {
        float v[32];
#pragma unroll
        for (int k = 0; k < 32; ++k) v[k] = i0 + 4 * k < n ? p[(i0 + 4 * k) * nout] : 0.f;
#pragma unroll
        for (int k = 0; k < 32; ++k)
          if (i0 + 4 * k < n) s += v[k];
      }
    }
    s += __shfl_xor(s, 16);  // s0+s1 (lanes 0-31), s2+s3 (lanes 32-63); fp add commutes exactly
    s += __shfl_xor(s, 32);  // (s0+s1) + (s2+s3) on every lane
    if (ok && lane < 16) {
      const int64_t k = o / C, c = o - k * C;
      if (k < R) {  // tap slot k holds filter tap k - (R - width); lower slots are padding
        if (k >= R - a.width) a.dw[c * a.width + k - (R - a.width)] = s;
      }
      else if (a.db) a.db[c] = s;
    }
    return;
  }
  const int64_t hid = (int64_t)blockIdx.x * kBlockThreads + threadIdx.x - n_red_waves * kWave;
  if (hid < 0 || hid >= nhist_zero * C) return;
  const int64_t i = hid / C, c = hid - i * C;
  if (a.hist.has_hist && !a.hist.has_hist[i]) return;
  if (a.seq.cu[i + 1] != a.seq.cu[i]) return;  // nonempty: written by the tile kernel
  const bool tail = a.dtail && i == a.seq.nseq - 1;
  for (int j = 0; j < a.width - 1; ++j) a.dhist[(i * (a.width - 1) + j) * C + c] = tail ? a.dtail[j * C + c] : 0;
}

// Shard-ordered combine of per-shard dweight / dbias contributions: one thread per output element,
// acc = p[0] then acc = acc + p[s] for s = 1 .. n-1 in ascending shard order (FP32, no
// reassociation: the library is built without contraction or fast-math), so the result depends
// only on the values and their order (core.ssm.causal_conv1d, assert_causal_conv1d_deterministic).
// Eight shards' loads are issued ahead of their adds.
__global__ void __launch_bounds__(kBlockThreads) conv1d_combine_kernel(const CombineArgs a) {
  const int64_t e = (int64_t)blockIdx.x * kBlockThreads + threadIdx.x;
  const int64_t ndw = a.C * a.width;
  const float* p;
  float* out;
  int64_t n, idx;
  if (e < ndw) {
    p = a.dw_parts, out = a.dw, n = ndw, idx = e;
  } else if (a.db && e < ndw + a.C) {
    p = a.db_parts, out = a.db, n = a.C, idx = e - ndw;
  } else {
    return;
  }
  float acc = a.nshards > 0 ? p[idx] : 0.f;
  for (int64_t s0 = 1; s0 < a.nshards; s0 += 8) {
    float v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = s0 + k < a.nshards ? p[(s0 + k) * n + idx] : 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (s0 + k < a.nshards) acc = acc + v[k];
  }
  out[idx] = acc;
}

// ------------------------------------------------------------------ library-held scratch
// conv1d_bwd_noalloc's partial workspace: a file-scope device array, one copy per GPU, held until
// the process ends.  Host code never passes the array's name to a kernel (on the host it is only a
// stand-in for the symbol): the device address comes from hipGetSymbolAddress, taken once per
// device with that device current, and kept per device.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device (nullptr: not looked up)
}  // namespace

hipError_t bwd_scratch(hipStream_t stream, void** ptr) {
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  int dev = cur;
  if (stream) {
    hipDevice_t d = 0;
    e = hipStreamGetDevice(stream, &d);
    if (e != hipSuccess) return e;
    dev = (int)d;
  }
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

// ------------------------------------------------------------------ launchers
constexpr int kCpl = kChannelsPerLane;

// Waves of the ordered reduce: 16 outputs each over the partial rows it reads (the dbias row only
// when dbias is wanted).
static int64_t reduce_waves(const BwdArgs& a) {
  const int64_t rows = partial_rows(a.width) - (a.db ? 0 : 1);
  return (rows * a.C + 15) / 16;
}

template <int MODE, bool VEC, bool SILU, int W>
static hipError_t bwd_go(const BwdArgs& a, hipStream_t s) {
  const uint32_t blocks = a.n_strips * a.n_rowblocks;
  if (blocks) {
    void* args[] = {const_cast<BwdArgs*>(&a)};
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&conv1d_bwd_kernel<kCpl, VEC, MODE, SILU, W>),
                                   dim3(blocks), dim3(kBlockThreads), args, 0, s);
    if (e != hipSuccess) return e;
  }
  // empty fragments that read history rows still get a (zero) d(history)
  const int64_t nz = (a.dhist && MODE == MODE_CU) ? a.seq.nseq : 0;
  int64_t n_red_waves = reduce_waves(a);
  const int64_t threads = n_red_waves * kWave + nz * a.C;
  const uint32_t rblocks = (uint32_t)((threads + kBlockThreads - 1) / kBlockThreads);
  int64_t nz_arg = nz;
  void* rargs[] = {const_cast<BwdArgs*>(&a), &nz_arg, &n_red_waves};
  return hipLaunchKernel(reinterpret_cast<const void*>(&conv1d_bwd_reduce_kernel), dim3(rblocks), dim3(kBlockThreads),
                         rargs, 0, s);
}

template <int MODE, int W>
static hipError_t bwd_mode(const BwdArgs& a, bool vec, bool silu, hipStream_t s) {
  if (vec) return silu ? bwd_go<MODE, true, true, W>(a, s) : bwd_go<MODE, true, false, W>(a, s);
  return silu ? bwd_go<MODE, false, true, W>(a, s) : bwd_go<MODE, false, false, W>(a, s);
}

template <int W>
static hipError_t bwd_width(const BwdArgs& a, int mode, bool vec, bool silu, hipStream_t s) {
  switch (mode) {
    case MODE_CU: return bwd_mode<MODE_CU, W>(a, vec, silu, s);
    case MODE_IDX: return bwd_mode<MODE_IDX, W>(a, vec, silu, s);
    default: return bwd_mode<MODE_BATCH, W>(a, vec, silu, s);
  }
}

hipError_t launch_reduce(const BwdArgs& a, hipStream_t s) {
  int64_t n_red_waves = reduce_waves(a);
  const int64_t threads = n_red_waves * kWave;
  const uint32_t rblocks = (uint32_t)((threads + kBlockThreads - 1) / kBlockThreads);
  int64_t nz_arg = 0;
  void* rargs[] = {const_cast<BwdArgs*>(&a), &nz_arg, &n_red_waves};
  return hipLaunchKernel(reinterpret_cast<const void*>(&conv1d_bwd_reduce_kernel), dim3(rblocks), dim3(kBlockThreads),
                         rargs, 0, s);
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
  const int64_t n = a.C * a.width + (a.db ? a.C : 0);
  const uint32_t blocks = (uint32_t)((n + kBlockThreads - 1) / kBlockThreads);
  if (blocks == 0) return hipSuccess;
  void* args[] = {const_cast<CombineArgs*>(&a)};
  return hipLaunchKernel(reinterpret_cast<const void*>(&conv1d_combine_kernel), dim3(blocks), dim3(kBlockThreads),
                         args, 0, s);
}

hipError_t launch_bwd(const BwdArgs& a, int mode, bool vec, bool silu, hipStream_t s) {
  switch (a.width) {
    case 2: return bwd_width<2>(a, mode, vec, silu, s);
    case 3: return bwd_width<3>(a, mode, vec, silu, s);
    case 5: return bwd_width<5>(a, mode, vec, silu, s);
    case 6: return bwd_width<6>(a, mode, vec, silu, s);
    case 7: return bwd_width<7>(a, mode, vec, silu, s);
    case 8: return bwd_width<8>(a, mode, vec, silu, s);
    default: return bwd_width<4>(a, mode, vec, silu, s);
  }
}

}  // namespace cconv
