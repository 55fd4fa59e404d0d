// conv1d_fwd.hip -- forward and decode kernels of the packed depthwise causal Conv1d (filter width 4;
// widths 2..8 for the forward without a pool).
//
// Operation: FlashInfer causal_conv1d_fn (Parameters x, weight, conv_state, cu_seqlens,
// cache_indices, has_initial_state, bias, out) with the optional activation and per-token
// sequence IDs of Megatron-Core causal_conv1d_cp, and the caller history rows of FlashInfer
// cake_causal_conv1d_kcp.
//
// Forward tiling (HBM-bound stencil, no MFMA):
//   block  = kWavesPerBlock waves side by side; lane = CPL consecutive channels; a block covers
//            kBlockChannels channels (a strip) of fwd_tile_rows() rows, so each row it touches is
//            one contiguous segment.  A launch is many rounds of these short tiles in an order
//            chosen by the strip count (block_tile): row-major slices per XCD, plain row-major
//            order, or strip-major slices per XCD.  The resident blocks sweep bands of rows, as a
//            copy does, and the dispatcher balances the load to the end of the launch.
//   loads  = one memory round trip per block: every row of the tile (non-temporal), the H window
//            rows above it (the tile above read them moments ago, mostly on this XCD), the taps,
//            the sequence offsets and, with a pool, the slots, all issued before any of them is
//            used; row addresses never wait for the metadata.
//   window = a ring of R register slots indexed by row mod R inside the unrolled tile, so the
//            sliding window costs no register moves.  Where a sequence starts inside the tile,
//            its window slots are re-seeded from that sequence's history (pool positions 0..2,
//            caller history rows, or zeros) right before its first row.
//   taps   = FP32 in registers; z = b, then W FMAs in tap order 0..W-1 (tap W-1 = current row).
//   width  = W taps and W-1 history values in a ring of R = 4 register slots (W <= 4) or 8 (W <= 8).
//   pool   = the block that holds a sequence's first row is the only one that reads or writes
//            its slot (for its channels).  With a pool, tile boundaries that fall on the first
//            three rows of a sequence move to that sequence's fourth row (or its end), so no
//            other block ever needs the slot's old history, and the head writes the final state
//            (the last three raw values of the extended sequence) right after reading it.
#include "conv1d_device.h"

namespace cconv {

// ------------------------------------------------------------------ sequence history
// h[j][ch] = history position j (oldest first) of sequence idx, channel c0 + ch.  Width W has
// W-1 history values; they fill the last W-1 of the H window slots (j >= R-W), the rest stay zero.
template <int CPL, bool VEC, int W, int H = Win<W>::H>
__device__ __forceinline__ void load_history(const PoolArgs& pool, const HistArgs& hist, int64_t idx,
                                             int32_t slot, bool live, int64_t c0, int64_t C, bool active,
                                             float (&h)[H][CPL]) {
  constexpr int R = Win<W>::R;
#pragma unroll
  for (int j = 0; j < H; ++j)
#pragma unroll
    for (int ch = 0; ch < CPL; ++ch) h[j][ch] = 0.f;
  if (idx < 0) return;  // history not needed
  if (W == 4 && pool.ptr) {  // the pool form is width four
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
      for (int j = R - W; j < H; ++j) {
        Pk<CPL> p = load_row<CPL, VEC>(hist.ptr + (idx * (W - 1) + j - (R - W)) * C, c0, C);
        unpack(p, h[j]);
      }
    }
  }
}

// Final state of a live nonempty sequence: pool positions 0..2 <- last three values of the
// extended sequence u = [h0, h1, h2, x[s], ..., x[e-1]] (raw bits; positions >= 3 untouched).
// Only kernels launched without a pool contain this (never taken) form, a row at a time, which
// leaves their register allocation as it is; pool kernels enter sequences through fwd_enter_pool.
template <int CPL, bool VEC>
__device__ __forceinline__ void pool_writeback(const FwdArgs& a, int32_t slot, const SeqDesc& sd,
                                               const float (&h)[3][CPL], int64_t c0, bool active) {
  const int64_t n = sd.e - sd.s;
  // start from the history and shift in the sequence's last min(n, 3) rows, in row order
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

// With a pool: move a tile boundary r off the first three rows of its sequence.
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

// One output row from the ring of R slots: u[(r+1+k)%R] is row t-(R-1)+k and u[r%R] the current
// row.  z = b, then the W taps in order (FMA), FP32; y = act(z) in bf16.
template <int CPL, bool SILU, int W, int R = Win<W>::R>
__device__ __forceinline__ Pk<CPL> stencil_row(const float (&wk)[R][CPL], const float (&bias)[CPL],
                                               const float (&u)[R][CPL], int r) {
  float out[CPL];
#pragma unroll
  for (int ch = 0; ch < CPL; ++ch) {
    float z = bias[ch];
#pragma unroll
    for (int k = R - W; k < R; ++k) z = __builtin_fmaf(wk[k][ch], u[(r + 1 + k) % R][ch], z);
    out[ch] = SILU ? z * sigmoid_f32(z) : z;
  }
  return pack(out);
}

// ------------------------------------------------------------------ forward kernel
// The sequence a wave is streaming: its rows, its pool slot, and whether its output is forced to
// zero (a -1 slot).
struct FwdSeq {
  SeqDesc sd;
  int32_t slot;
  bool zero;
  int64_t pre_idx = -1;  // the sequence whose slot the lookup already fetched (pre_slot), or -1
  int32_t pre_slot = -1;
};

template <int MODE>
__device__ __forceinline__ void fwd_slot(const FwdArgs& a, FwdSeq& cs) {
  cs.slot = -1;
  cs.zero = false;
  if constexpr (MODE != MODE_IDX) {
    if (a.pool.ptr) {
      cs.slot = cs.sd.idx == cs.pre_idx ? cs.pre_slot : a.pool.cache_indices[cs.sd.idx];
      cs.zero = !(cs.slot >= 0 && cs.slot < a.pool.slots);  // -1 (other values are out of contract)
    }
  }
}

// Entering a sequence in a kernel launched with a slot pool (width four, offsets or batch rows).
// The slot, its has-initial-state flag and the sequence's last three input rows do not depend on
// one another, so they are read together, from in-range addresses and without tests between them;
// the old state, which needs the slot, follows in a second round trip, and the final state is
// written right after it.  With vectors C is even, so both channels of a lane exist.
template <int CPL, bool VEC, int MODE>
__device__ __forceinline__ void fwd_enter_pool(const FwdArgs& a, FwdSeq& cs, int64_t c0, bool active, float (&h)[3][CPL]) {
  const int64_t idx = cs.sd.idx, s = cs.sd.s, n = cs.sd.e - cs.sd.s;
  const int32_t slot = idx == cs.pre_idx ? cs.pre_slot : a.pool.cache_indices[idx];
  const uint8_t* hi = a.pool.has_init ? a.pool.has_init : reinterpret_cast<const uint8_t*>(a.pool.cache_indices);
  const uint8_t init_raw = hi[idx];
  Pk<CPL> last[3];
#pragma unroll
  for (int j = 0; j < 3; ++j) {  // rows s+n-3+j, clamped into the array (used only when >= s)
    int64_t row = s + n - 3 + j;
    row = row < s ? s : row;
    row = row < a.rows ? row : a.rows - 1;
    last[j] = zero_pk<CPL>();
    if (VEC || active) last[j] = load_row<CPL, VEC>(a.x + row * a.x_ld, c0, a.C);
  }
  cs.slot = slot;
  cs.zero = !(slot >= 0 && slot < a.pool.slots);  // -1 (other values are out of contract)
#pragma unroll
  for (int j = 0; j < 3; ++j)
#pragma unroll
    for (int ch = 0; ch < CPL; ++ch) h[j][ch] = 0.f;
  if (cs.zero) return;
  uint16_t* base = a.pool.ptr + (int64_t)slot * a.pool.s_slot;
  if (a.pool.has_init && init_raw && (VEC || active)) {
#pragma unroll
    for (int j = 0; j < 3; ++j)
#pragma unroll
      for (int ch = 0; ch < CPL; ++ch)
        if (VEC || c0 + ch < a.C)
          h[j][ch] = __uint_as_float((uint32_t)base[(c0 + ch) * a.pool.s_chan + j * a.pool.s_pos] << 16);
  }
  if (n <= 0 || !(VEC || active)) return;
  // final state: the history shifted by the sequence's last min(n, 3) rows, in row order
  float v[3][CPL];
#pragma unroll
  for (int j = 0; j < 3; ++j)
#pragma unroll
    for (int ch = 0; ch < CPL; ++ch) v[j][ch] = h[j][ch];
#pragma unroll
  for (int j = 0; j < 3; ++j)
    if (n - 3 + j >= 0) shift_in<CPL>(v, last[j]);
#pragma unroll
  for (int j = 0; j < 3; ++j)
#pragma unroll
    for (int ch = 0; ch < CPL; ++ch)
      if (VEC || c0 + ch < a.C)
        base[(c0 + ch) * a.pool.s_chan + j * a.pool.s_pos] = (uint16_t)(__float_as_uint(v[j][ch]) >> 16);
}

// Row q = cs.sd.s, the first row of a sequence, is next: h <- its history, and with a pool the
// head writes the sequence's final state (the head wave is the only one that touches the slot).
// POOL: the kernel is the one launched with a slot pool.
template <int CPL, bool VEC, int MODE, int W, bool POOL, int H = Win<W>::H>
__device__ __forceinline__ void fwd_enter(const FwdArgs& a, FwdSeq& cs, int64_t c0, bool active, float (&h)[H][CPL]) {
  if constexpr (POOL && MODE != MODE_IDX && W == 4) {
    fwd_enter_pool<CPL, VEC, MODE>(a, cs, c0, active, h);
    return;
  }
  fwd_slot<MODE>(a, cs);
#pragma unroll
  for (int j = 0; j < H; ++j)
#pragma unroll
    for (int ch = 0; ch < CPL; ++ch) h[j][ch] = 0.f;
  if constexpr (MODE != MODE_IDX) {
    if (!cs.zero) {
      load_history<CPL, VEC, W>(a.pool, a.hist, cs.sd.idx, cs.slot, true, c0, a.C, active, h);
      if constexpr (W == 4) {
        if (a.pool.ptr && cs.sd.e > cs.sd.s) pool_writeback<CPL, VEC>(a, cs.slot, cs.sd, h, c0, active);
      }
    }
  }
}

// n (<= CH) rows starting at q0 from a loaded buffer.  Ring slot of row q is (q - tile start)
// mod R = r mod R, as q0 - tile start is a multiple of CH.  A chunk inside one sequence is a
// straight stencil; a chunk where sequences start re-seeds the three window slots from the new
// sequence's history right before its first row.
template <int CPL, bool VEC, int MODE, int CH, bool SILU, bool FULL, int W, bool POOL, int R = Win<W>::R>
__device__ __forceinline__ void fwd_chunk(const FwdArgs& a, const Pk<CPL> (&buf)[CH], int n, int64_t q0, int64_t tb,
                                          int64_t dend, FwdSeq& cs, int64_t c0, bool active,
                                          const float (&wk)[R][CPL], const float (&bias)[CPL], float (&u)[R][CPL]) {
  constexpr int H = R - 1;
  if (n == CH && cs.sd.e >= q0 + CH) {
    if (cs.zero) {
      if (FULL || active) {
#pragma unroll
        for (int r = 0; r < CH; ++r) store_row<CPL, VEC, true>(a.y + (q0 + r) * a.y_ld, c0, a.C, zero_pk<CPL>());
      }
    } else {
#pragma unroll
      for (int r = 0; r < CH; ++r) {
        unpack(buf[r], u[r % R]);
        const Pk<CPL> out = stencil_row<CPL, SILU, W>(wk, bias, u, r);
        if (FULL || active) store_row<CPL, VEC, true>(a.y + (q0 + r) * a.y_ld, c0, a.C, out);
      }
    }
    return;
  }
#pragma unroll
  for (int r = 0; r < CH; ++r) {
    if (r < n) {
      const int64_t q = q0 + r;
      if (q == cs.sd.e) {  // a new sequence starts at row q (empty ones are skipped)
        cs.sd = next_seq<MODE>(a.seq, cs.sd, dend, tb);
        float h[H][CPL];
        fwd_enter<CPL, VEC, MODE, W, POOL>(a, cs, c0, active, h);
#pragma unroll
        for (int j = 0; j < H; ++j)
#pragma unroll
          for (int ch = 0; ch < CPL; ++ch) u[(r + 1 + j) % R][ch] = h[j][ch];
      }
      unpack(buf[r], u[r % R]);
      Pk<CPL> out = zero_pk<CPL>();
      if (!cs.zero) out = stencil_row<CPL, SILU, W>(wk, bias, u, r);
      if (FULL || active) store_row<CPL, VEC, true>(a.y + q * a.y_ld, c0, a.C, out);
    }
  }
}

// The window of the row before a tile that starts at row ta of sequence cs (ring slots
// 1..H get rows ta-H .. ta-1): the sequence's history, then the last `dist` input rows of the
// sequence (wrow holds rows ta-H .. ta-1, loaded before the lookup).  At the sequence's first row
// this enters the sequence (history, pool write-back); elsewhere only its -1 status matters, and
// with a pool a tile never starts on a sequence's rows 1 and 2, so the slot is not touched.
template <int CPL, bool VEC, int MODE, int W, bool POOL, int R = Win<W>::R, int H = Win<W>::H>
__device__ __forceinline__ void fwd_start(const FwdArgs& a, FwdSeq& cs, int64_t ta, const Pk<CPL> (&wrow)[H],
                                          int64_t c0, bool active, float (&u)[R][CPL]) {
  const int64_t dist = ta - cs.sd.s < H ? ta - cs.sd.s : H;
  float h[H][CPL];
  if (dist == 0) {
    fwd_enter<CPL, VEC, MODE, W, POOL>(a, cs, c0, active, h);
  } else {
    fwd_slot<MODE>(a, cs);
#pragma unroll
    for (int j = 0; j < H; ++j)
#pragma unroll
      for (int ch = 0; ch < CPL; ++ch) h[j][ch] = 0.f;
    if constexpr (MODE != MODE_IDX) {
      if (!cs.zero && dist < H) load_history<CPL, VEC, W>(a.pool, a.hist, cs.sd.idx, cs.slot, true, c0, a.C, active, h);
    }
  }
  shift_window<CPL, H>(h, wrow, dist);
#pragma unroll
  for (int j = 0; j < H; ++j)
#pragma unroll
    for (int ch = 0; ch < CPL; ++ch) u[j + 1][ch] = h[j][ch];
}

// Taps and bias of a wave whose lanes are all active: straight-line loads, the dtype branches
// taken once for the wave.
template <int CPL, int W, int R = Win<W>::R>
__device__ __forceinline__ void load_taps_full(const FwdArgs& a, int64_t c0, float (&wk)[R][CPL], float (&bias)[CPL]) {
#pragma unroll
  for (int k = 0; k < R - W; ++k)
#pragma unroll
    for (int ch = 0; ch < CPL; ++ch) wk[k][ch] = 0.f;
  if (a.w_f32) {
    const float* p = static_cast<const float*>(a.w) + c0 * W;
#pragma unroll
    for (int ch = 0; ch < CPL; ++ch)
#pragma unroll
      for (int k = 0; k < W; ++k) wk[R - W + k][ch] = p[ch * W + k];
  } else {
    const uint16_t* p = static_cast<const uint16_t*>(a.w) + c0 * W;
#pragma unroll
    for (int ch = 0; ch < CPL; ++ch)
#pragma unroll
      for (int k = 0; k < W; ++k) wk[R - W + k][ch] = __uint_as_float((uint32_t)p[ch * W + k] << 16);
  }
#pragma unroll
  for (int ch = 0; ch < CPL; ++ch) bias[ch] = 0.f;
  if (a.b) {
    if (a.b_f32) {
#pragma unroll
      for (int ch = 0; ch < CPL; ++ch) bias[ch] = static_cast<const float*>(a.b)[c0 + ch];
    } else {
#pragma unroll
      for (int ch = 0; ch < CPL; ++ch) bias[ch] = __uint_as_float((uint32_t)static_cast<const uint16_t*>(a.b)[c0 + ch] << 16);
    }
  }
}

// Rows q0 .. q0+R-1 of x that lie below te (zeros past te, not loaded).
template <int CPL, bool VEC, int R>
__device__ __forceinline__ void fwd_rows(const FwdArgs& a, int64_t q0, int64_t te, int64_t c0, bool active,
                                         Pk<CPL> (&dst)[R]) {
#pragma unroll
  for (int r = 0; r < R; ++r) {
    dst[r] = zero_pk<CPL>();
    if (q0 + r < te && active) dst[r] = load_row<CPL, VEC>(a.x + (q0 + r) * a.x_ld, c0, a.C);
  }
}

// Rows [ta, te) R at a time in a rolled loop (ring slot of row q is (q - ta) mod R), each chunk's
// loads issued one chunk ahead of its use (`rows` arrives holding the chunk at ta): the path for
// tiles where a sequence starts or the data ends, tiles a pool moved, partly active waves.  The
// sequence-start code then exists once per kernel.
template <int CPL, bool VEC, int MODE, bool SILU, int W, bool POOL, int R = Win<W>::R>
__device__ __forceinline__ void fwd_rolled(const FwdArgs& a, FwdSeq& cs, int64_t ta, int64_t te, int64_t dend,
                                           int64_t c0, bool active, const float (&wk)[R][CPL],
                                           const float (&bias)[CPL], float (&u)[R][CPL], Pk<CPL> (&rows)[R]) {
  for (int64_t q0 = ta; q0 < te; q0 += R) {
    const int n = (int)(te - q0 < R ? te - q0 : R);
    Pk<CPL> next[R];
    fwd_rows<CPL, VEC, R>(a, q0 + R, te, c0, active, next);
    fwd_chunk<CPL, VEC, MODE, R, SILU, false, W, POOL>(a, rows, n, q0, te, dend, cs, c0, active, wk, bias, u);
#pragma unroll
    for (int r = 0; r < R; ++r) rows[r] = next[r];
  }
}

// The rows [ta, tb) of one strip by the general path (predicated loads and lanes).  One memory
// round trip for the set-up, as in the tile path: the lookup's loads (with a pool, the slots too),
// the taps, the window rows above and the first chunk of rows are all issued before any is used.
template <int CPL, bool VEC, int MODE, bool SILU, int W, bool POOL>
__device__ __forceinline__ void fwd_general(const FwdArgs& a, int64_t ta, int64_t tb, int64_t c0, bool active) {
  constexpr int R = Win<W>::R, H = Win<W>::H;
  const int64_t dend = data_end<MODE>(a.seq, a.rows);
  const int64_t te = tb < dend ? tb : dend;
  if (ta >= te) return;
  const SeqProbe pr = seq_probe<MODE, H>(a.seq, ta, te, POOL ? a.pool.cache_indices : nullptr);
  float wk[R][CPL], bias[CPL];
  load_taps<CPL, W>(a.w, a.w_f32, a.b, a.b_f32, c0, a.C, wk, bias);
  Pk<CPL> wrow[H];
  load_window<CPL, VEC, H>(wrow, a.x, a.x_ld, ta, c0, a.C, active);
  Pk<CPL> rows[R];
  fwd_rows<CPL, VEC, R>(a, ta, te, c0, active, rows);
  FwdSeq cs;
  cs.sd = seq_resolve<MODE, H>(a.seq, ta, dend, te, pr);
  if constexpr (POOL) {
    int32_t sl;
    if (probe_slot<MODE>(a.seq, pr, cs.sd.idx, sl)) {
      cs.pre_idx = cs.sd.idx;
      cs.pre_slot = sl;
    }
  }
  float u[R][CPL];
  fwd_start<CPL, VEC, MODE, W, POOL>(a, cs, ta, wrow, c0, active, u);
  fwd_rolled<CPL, VEC, MODE, SILU, W, POOL>(a, cs, ta, te, dend, c0, active, wk, bias, u, rows);
}

template <int CPL, bool VEC, int MODE, bool SILU, int W, bool POOL>
__global__ void __launch_bounds__(kBlockThreads) conv1d_fwd_kernel(const FwdArgs a) {
  constexpr int R = Win<W>::R, H = Win<W>::H;  // ring slots, history values
  constexpr int RT = fwd_tile_rows(MODE, POOL, W);  // rows per tile
  static_assert(RT % R == 0 && RT % 4 == 0, "tiles hold whole ring periods");
  constexpr int NT = RT / R;                    // register chunks of a tile

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint32_t strip, rb;
  block_tile(a.tile_order, a.n_strips, a.n_rowblocks, strip, rb);
  const int64_t C = a.C;
  const int64_t wc0 = (int64_t)strip * kBlockChannels + (int64_t)wave * kWaveChannels;
  if (wc0 >= C) return;  // the whole wave is past the last channel
  // With vectors, the lanes of a partly active wave that lie past the last channel work as copies
  // of the wave's last channel pair: the same loads, history and arithmetic, and stores of the same
  // bits to the same addresses in the same instructions (lanes never exchange data).  Every wave
  // then takes the tile path with no per-lane predicate.  With an odd C (never with a pool: the
  // slot is updated in place) the lane of the lone last channel takes the pair (C-2, C-1); channel
  // C-2 is then computed twice, perhaps in two waves, from the same inputs, and both store the same
  // bits.  No output overlaps an input, so the order of those stores does not matter.
  const int64_t c0 = VEC && wc0 + lane * CPL + (CPL - 1) >= C ? C - CPL : wc0 + lane * CPL;
  const bool active = VEC || c0 < C;
  constexpr bool has_pool = POOL;  // a slot pool (width four, offsets or batch rows)
  static_assert(!POOL || (W == 4 && MODE != MODE_IDX), "the pool form is width four with host-known sequences");
  const int64_t ta = (int64_t)rb * RT;
  const int64_t tb = ta + RT < a.rows ? ta + RT : a.rows;

  if constexpr (!VEC) {  // rows that do not allow vectors: the general path, predicated per lane
    int64_t ta2 = ta, tb2 = tb;
    if constexpr (has_pool) {
      const int64_t de = data_end<MODE>(a.seq, a.rows);
      ta2 = owner_boundary<MODE>(a.seq, ta < de ? ta : de, de);
      tb2 = owner_boundary<MODE>(a.seq, tb < de ? tb : de, de);
    }
    if (ta2 < tb2) fwd_general<CPL, VEC, MODE, SILU, W, POOL>(a, ta2, tb2, c0, active);
    return;
  }

  // ---- one memory round trip: the sequence lookup's first loads (for both tile ends with a
  // pool), the taps, the H window rows above the tile (the tile above read them moments ago on
  // this XCD), every row of the tile (non-temporal; rows past the tile re-read its last row).
  // Row addresses never wait for the metadata, and the lookup's loads go first, so resolving it
  // waits for them alone.  The chunk index of every buffer access is a template constant: a
  // runtime index would move the buffers out of registers.
  const SeqProbe pa = seq_probe<MODE, H>(a.seq, ta, tb, has_pool ? a.pool.cache_indices : nullptr);
  SeqProbe pb{0, 0};
  if (has_pool && tb < a.rows) pb = seq_probe<MODE, H>(a.seq, tb, tb);
  const int64_t dend = data_end<MODE>(a.seq, a.rows);
  float wk[R][CPL], bias[CPL];
  load_taps_full<CPL, W>(a, c0, wk, bias);
  Pk<CPL> wrow[H];
#pragma unroll
  for (int j = 0; j < H; ++j) {
    wrow[j] = zero_pk<CPL>();
    if (ta - H + j >= 0) wrow[j] = load_row<CPL, VEC>(a.x + (ta - H + j) * a.x_ld, c0, C);
  }
  Pk<CPL> buf[NT][R];
  const int64_t qlast = tb - 1;
  auto load = [&](auto cc) {
    constexpr int c = decltype(cc)::value;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int64_t q = ta + c * R + r;
      buf[c][r] = load_row<CPL, VEC, true>(a.x + (q <= qlast ? q : qlast) * a.x_ld, c0, C);
    }
  };
  unroll_steps<NT>(load);

  const int64_t te = tb < dend ? tb : dend;  // rows of the tile that belong to some sequence
  if (ta >= te) return;
  FwdSeq cs;
  cs.sd = seq_resolve<MODE, H>(a.seq, ta, dend, te, pa);
  if constexpr (has_pool) {  // the slot came with the lookup: no dependent load before the stores
    int32_t sl;
    if (probe_slot<MODE>(a.seq, pa, cs.sd.idx, sl)) {
      cs.pre_idx = cs.sd.idx;
      cs.pre_slot = sl;
    }
  }
  if constexpr (has_pool) {
    // tile boundaries on a sequence's rows 1 and 2 move to its row 3: the head tile alone owns
    // the slot.  A moved tile takes the general path.
    int64_t ta2 = ta, tb2 = tb;
    if (ta > 0 && (ta - cs.sd.s == 1 || ta - cs.sd.s == 2)) ta2 = cs.sd.s + 3 < cs.sd.e ? cs.sd.s + 3 : cs.sd.e;
    if (tb > 0 && tb < dend) {
      const SeqDesc d = seq_resolve<MODE, H>(a.seq, tb, dend, dend, pb);
      if (tb - d.s == 1 || tb - d.s == 2) tb2 = d.s + 3 < d.e ? d.s + 3 : d.e;
    }
    if (ta2 != ta || tb2 != tb) {
      if (ta2 < tb2) fwd_general<CPL, VEC, MODE, SILU, W, POOL>(a, ta2, tb2, c0, active);
      return;
    }
  }
  float u[R][CPL];
  fwd_start<CPL, VEC, MODE, W, POOL>(a, cs, ta, wrow, c0, active, u);

  if (te - ta == RT && cs.sd.e >= te) {
    // ---- the whole tile inside one sequence: one straight stencil (ring slot of row ta+c*R+r is r)
    auto step = [&](auto cc) {
      constexpr int c = decltype(cc)::value;
      const int64_t q0 = ta + (int64_t)c * R;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        unpack(buf[c][r], u[r]);
        const Pk<CPL> out = cs.zero ? zero_pk<CPL>() : stencil_row<CPL, SILU, W>(wk, bias, u, r);
        store_row<CPL, VEC, true>(a.y + (q0 + r) * a.y_ld, c0, C, out);
      }
    };
    unroll_steps<NT>(step);
    return;
  }
  // ---- a tile where a sequence starts or the data ends: the rows already in registers, R at a
  // time in a rolled loop that shifts the buffer down one chunk per step (static register indices,
  // one copy of the sequence-start code)
#pragma unroll 1
  for (int64_t q0 = ta; q0 < te; q0 += R) {
    const int n = (int)(te - q0 < R ? te - q0 : R);
    fwd_chunk<CPL, VEC, MODE, R, SILU, true, W, POOL>(a, buf[0], n, q0, te, dend, cs, c0, active, wk, bias, u);
#pragma unroll
    for (int c = 0; c + 1 < NT; ++c)
#pragma unroll
      for (int r = 0; r < R; ++r) buf[c][r] = buf[c + 1][r];
  }
}

// ------------------------------------------------------------------ decode / speculative update
// One thread per (sequence, CPL-channel group), K tokens per sequence (K = 1: the decode step).
// The history is pool positions a-1 .. a+1 for the sequence's accepted count a (1 without one);
// y_t = act(b + w . window) over the extended sequence [h0, h1, h2, x_1 .. x_K]; afterwards
// positions 0 .. K+1 hold its last K + 2 raw values.  All three history values are in registers
// before the first write, and each thread owns its channels of the slot, so the in-place shift
// needs no ordering between threads.
template <int CPL, bool VEC, bool SILU>
__global__ void __launch_bounds__(kBlockThreads) conv1d_decode_kernel(const DecodeArgs a) {
  const int64_t gid = (int64_t)blockIdx.x * kBlockThreads + threadIdx.x;
  const int64_t groups = (a.C + CPL - 1) / CPL;
  if (gid >= a.nseq * groups) return;
  const int64_t i = gid / groups;
  const int64_t c0 = (gid - i * groups) * CPL;
  const int64_t C = a.C, K = a.K;
  // One memory round trip before the slot is known: the slot, the accepted count, the first four
  // token rows and the taps, none of which depends on the slot.  Only the pool reads wait for it.
  // The accepted count is read unconditionally (from the slot's own entry when there is none), the
  // taps last (their dtype test joins with a wait), and a -1 slot selects zeros rather than
  // branching away, so no load waits behind another.
  const int32_t slot = a.pool.cache_indices[i];
  const int32_t acc_raw = (a.accepted ? a.accepted : a.pool.cache_indices)[i];
  Pk<CPL> xr[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) xr[j] = j < K ? load_row<CPL, VEC>(a.x + (i * K + j) * a.x_ld, c0, C) : zero_pk<CPL>();
  float wk[4][CPL], bias[CPL];
  load_taps<CPL>(a.w, a.w_f32, a.b, a.b_f32, c0, C, wk, bias);
  const int32_t acc = a.accepted ? acc_raw : 1;
  const bool live = slot >= 0 && slot < a.pool.slots;
  int64_t o = (int64_t)acc - 1;                // first history position
  const int64_t omax = a.pool.len - 3;         // out-of-contract counts are clamped
  o = o < 0 ? 0 : (o > omax ? omax : o);
  uint16_t* base = a.pool.ptr + (int64_t)(live ? slot : 0) * a.pool.s_slot;
  uint16_t hb[3][CPL];
  float u[3][CPL];
  // With vectors C is even, so both channels of a lane exist: the three history reads of both go
  // out together under the one test of the slot.
#pragma unroll
  for (int ch = 0; ch < CPL; ++ch)
#pragma unroll
    for (int j = 0; j < 3; ++j) hb[j][ch] = 0;
  if (live) {
#pragma unroll
    for (int ch = 0; ch < CPL; ++ch) {
      const int64_t c = c0 + ch;
#pragma unroll
      for (int j = 0; j < 3; ++j)
        if (VEC || c < C) hb[j][ch] = base[c * a.pool.s_chan + (o + j) * a.pool.s_pos];
    }
#pragma unroll
    for (int ch = 0; ch < CPL; ++ch) {
      const int64_t c = c0 + ch;
      if (VEC || c < C) {
        base[c * a.pool.s_chan] = hb[1][ch];
        base[c * a.pool.s_chan + a.pool.s_pos] = hb[2][ch];
      }
    }
  }
#pragma unroll
  for (int ch = 0; ch < CPL; ++ch)
#pragma unroll
    for (int j = 0; j < 3; ++j) u[j][ch] = __uint_as_float((uint32_t)hb[j][ch] << 16);
  // tokens in groups of four: the four row loads of a later group are issued together
  for (int64_t t0 = 0; t0 < K; t0 += 4) {
    if (t0 > 0) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        xr[j] = t0 + j < K ? load_row<CPL, VEC>(a.x + (i * K + t0 + j) * a.x_ld, c0, C) : zero_pk<CPL>();
    }
    float xv[4][CPL];
#pragma unroll
    for (int j = 0; j < 4; ++j) unpack(xr[j], xv[j]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (t0 + j < K) {
        const int64_t t = t0 + j;
        float out[CPL];
#pragma unroll
        for (int ch = 0; ch < CPL; ++ch) {
          float z = bias[ch];
          z = __builtin_fmaf(wk[0][ch], u[0][ch], z);
          z = __builtin_fmaf(wk[1][ch], u[1][ch], z);
          z = __builtin_fmaf(wk[2][ch], u[2][ch], z);
          z = __builtin_fmaf(wk[3][ch], xv[j][ch], z);
          out[ch] = live ? (SILU ? z * sigmoid_f32(z) : z) : 0.f;
        }
        store_row<CPL, VEC>(a.y + (i * K + t) * a.y_ld, c0, C, pack(out));
#pragma unroll
        for (int ch = 0; ch < CPL; ++ch) {
          const int64_t c = c0 + ch;
          if (live && (VEC || c < C)) base[c * a.pool.s_chan + (t + 2) * a.pool.s_pos] = (uint16_t)(__float_as_uint(xv[j][ch]) >> 16);
          u[0][ch] = u[1][ch];
          u[1][ch] = u[2][ch];
          u[2][ch] = xv[j][ch];
        }
      }
    }
  }
}

// ------------------------------------------------------------------ launchers
constexpr int kCpl = kChannelsPerLane;

template <int MODE, bool VEC, bool SILU, int W, bool POOL>
static hipError_t fwd_go(const FwdArgs& a, hipStream_t s) {
  const uint32_t blocks = a.n_strips * a.n_rowblocks;
  void* args[] = {const_cast<FwdArgs*>(&a)};
  return hipLaunchKernel(reinterpret_cast<const void*>(&conv1d_fwd_kernel<kCpl, VEC, MODE, SILU, W, POOL>),
                         dim3(blocks), dim3(kBlockThreads), args, 0, s);
}

template <int MODE, int W, bool POOL>
static hipError_t fwd_mode(const FwdArgs& a, bool vec, bool silu, hipStream_t s) {
  if (vec) return silu ? fwd_go<MODE, true, true, W, POOL>(a, s) : fwd_go<MODE, true, false, W, POOL>(a, s);
  return silu ? fwd_go<MODE, false, true, W, POOL>(a, s) : fwd_go<MODE, false, false, W, POOL>(a, s);
}

template <int W>
static hipError_t fwd_width(const FwdArgs& a, int mode, bool vec, bool silu, hipStream_t s) {
  if constexpr (W == 4) {
    if (a.pool.ptr) {  // the pool form: offsets or batch rows
      if (mode == MODE_CU) return fwd_mode<MODE_CU, 4, true>(a, vec, silu, s);
      return fwd_mode<MODE_BATCH, 4, true>(a, vec, silu, s);
    }
  }
  switch (mode) {
    case MODE_CU: return fwd_mode<MODE_CU, W, false>(a, vec, silu, s);
    case MODE_IDX: return fwd_mode<MODE_IDX, W, false>(a, vec, silu, s);
    default: return fwd_mode<MODE_BATCH, W, false>(a, vec, silu, s);
  }
}

hipError_t launch_fwd(const FwdArgs& a, int mode, bool vec, bool silu, hipStream_t s) {
  if ((uint64_t)a.n_strips * a.n_rowblocks == 0) return hipSuccess;
  switch (a.width) {
    case 2: return fwd_width<2>(a, mode, vec, silu, s);
    case 3: return fwd_width<3>(a, mode, vec, silu, s);
    case 5: return fwd_width<5>(a, mode, vec, silu, s);
    case 6: return fwd_width<6>(a, mode, vec, silu, s);
    case 7: return fwd_width<7>(a, mode, vec, silu, s);
    case 8: return fwd_width<8>(a, mode, vec, silu, s);
    default: return fwd_width<4>(a, mode, vec, silu, s);
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
