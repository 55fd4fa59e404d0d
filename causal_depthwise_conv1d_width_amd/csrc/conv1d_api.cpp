// conv1d_api.cpp -- the C ABI of include/conv1d.h: host-side validation and kernel launches.
//
// Every entry point checks what the host can check (pointers, dtypes, sizes, strides, layouts,
// byte-range overlaps, workspace size) and returns CONV1D_EINVAL / CONV1D_EWORKSPACE before
// anything is enqueued.  It never reads device memory and never synchronizes, so the calls are
// stream-ordered and can be captured in a HIP graph (FlashInfer causal_conv1d_fn, Notes).
#include "conv1d.h"

#include <stdint.h>

#include "conv1d_launch.h"

using namespace cconv;

namespace {

struct Span {
  uintptr_t lo = 0, hi = 0;  // [lo, hi); empty when lo == hi
};

Span span_rows(const void* p, int64_t rows, int64_t C, int64_t ld, int64_t esz) {
  Span s;
  if (!p || rows <= 0 || C <= 0) return s;
  s.lo = reinterpret_cast<uintptr_t>(p);
  s.hi = s.lo + (uintptr_t)(((rows - 1) * ld + C) * esz);
  return s;
}

Span span_bytes(const void* p, int64_t bytes) {
  Span s;
  if (!p || bytes <= 0) return s;
  s.lo = reinterpret_cast<uintptr_t>(p);
  s.hi = s.lo + (uintptr_t)bytes;
  return s;
}

bool overlap(const Span& a, const Span& b) {
  return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi;
}

// Byte ranges of the sequence metadata (offsets / IDs) and of per-sequence arrays.
Span span_seq(const conv1d_seq* s, int64_t rows) {
  if (s->cu_seqlens) return span_bytes(s->cu_seqlens, (s->nseq + 1) * 4);
  if (s->seq_idx) return span_bytes(s->seq_idx, rows * 4);
  return Span{};
}

bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

// The channel-last kernels move a lane's kChannelsPerLane channels of a row as one vector when
// the channel count, every row stride and every row base allow it; otherwise they take the
// element-wise path (same results).  A pair of channels is one dword access at any 2-byte aligned
// address, so with pairs any C >= 2 and any row stride will do; with an odd C the last pair
// overlaps the one before it.  Kernels that update state in place (the slot pool) need C to be a
// multiple of kChannelsPerLane on top, so that no two lanes own the same channel (vec_inplace).
constexpr int64_t kVecElems = kChannelsPerLane;
constexpr uintptr_t kVecBytes = 2 * kChannelsPerLane;
bool vec_rows(int64_t C, int64_t ld, const void* p) {
  if (kChannelsPerLane == 2) return C >= 2 && aligned(p, 2);
  return C % kVecElems == 0 && ld % kVecElems == 0 && aligned(p, kVecBytes);
}
bool vec_inplace(int64_t C) { return C % kVecElems == 0; }

// Byte extents and element counts are computed in int64.  Sizes and strides whose products could
// overflow it are rejected up front (no allocation comes near 2^56 elements).
constexpr int64_t kMaxElems = (int64_t)1 << 56;
bool mul_ok(int64_t a, int64_t b) {
  return a >= 0 && b >= 0 && a <= kMaxElems && b <= kMaxElems && (b == 0 || a <= kMaxElems / b);
}

int mode_of(const conv1d_seq* s) {
  if (s->cu_seqlens) return MODE_CU;
  return s->seq_idx ? MODE_IDX : MODE_BATCH;
}

// Sequence description: checks the form and returns the host-known sequence count (-1 = IDX).
int check_seq(const conv1d_seq* s, int64_t rows, int64_t* nseq_out) {
  if (!s) return CONV1D_EINVAL;
  if (s->cu_seqlens) {
    if (s->seq_idx || s->nseq < 0) return CONV1D_EINVAL;
    *nseq_out = s->nseq;
    return CONV1D_OK;
  }
  if (s->seqlen < 1 || rows % s->seqlen != 0) return CONV1D_EINVAL;
  *nseq_out = s->seq_idx ? -1 : rows / s->seqlen;
  return CONV1D_OK;
}

bool dtype_ok(int d) { return d == CONV1D_BF16 || d == CONV1D_F32; }
int64_t dsize(int d) { return d == CONV1D_F32 ? 4 : 2; }

// Pool layout: [slots, C, len] with the channel or history axis contiguous, no self-overlap
// inside a slot and no overlap between slots (causal_conv1d_fn, Parameters conv_state).
int check_pool(const conv1d_pool* p, int64_t C, int64_t nseq, Span* out) {
  if (p->len < 3 || p->slots < 1 || p->s_slot < 1 || p->s_chan < 1 || p->s_pos < 1) return CONV1D_EINVAL;
  if (!mul_ok(p->slots, p->s_slot) || !mul_ok(C, p->s_chan) || !mul_ok(p->len, p->s_pos)) return CONV1D_EINVAL;
  if (p->s_chan != 1 && p->s_pos != 1) return CONV1D_EINVAL;
  if (p->s_pos == 1 && C > 1 && p->s_chan < p->len) return CONV1D_EINVAL;  // (c, j) must not alias
  if (p->s_chan == 1 && p->s_pos != 1 && p->s_pos < C) return CONV1D_EINVAL;
  if (p->s_chan == 1 && p->s_pos == 1 && C > 1) return CONV1D_EINVAL;
  const int64_t extent = (C - 1) * p->s_chan + (p->len - 1) * p->s_pos + 1;
  if (p->slots > 1 && p->s_slot < extent) return CONV1D_EINVAL;  // slots must not overlap
  if (nseq > 0 && !p->cache_indices) return CONV1D_EINVAL;
  *out = span_bytes(p->ptr, ((p->slots - 1) * p->s_slot + extent) * 2);
  return CONV1D_OK;
}

// Channels-first array [B, D, T]: rows (b, d) at b * sb + d * sd, T contiguous, no two rows overlapping.
bool cf_layout_ok(int64_t B, int64_t D, int64_t T, int64_t sb, int64_t sd) {
  if (!mul_ok(B, sb) || !mul_ok(D, sd) || !mul_ok(T, 2) || B > 0x7fffffff) return false;
  if (D > 1 && sd < T) return false;
  if (B > 1 && sb < (D - 1) * sd + T) return false;
  return sb >= 0 && sd >= 0;
}

Span span_cf(const void* p, int64_t B, int64_t D, int64_t T, int64_t sb, int64_t sd) {
  if (!p || B <= 0 || D <= 0 || T <= 0) return Span{};
  return span_bytes(p, ((B - 1) * sb + (D - 1) * sd + T) * 2);
}

// ws was sized by the launcher; the partial slabs need FP32 alignment
constexpr size_t kWsAlign = 256;

uint32_t ceil_div(int64_t a, int64_t b) { return (uint32_t)((a + b - 1) / b); }

}  // namespace

extern "C" {

size_t conv1d_fwd_workspace_bytes(int64_t rows, int64_t C, int64_t nseq) {
  (void)rows;
  (void)C;
  (void)nseq;
  return 0;  // uniform row tiles with an in-kernel sequence lookup: no chunk map
}

size_t conv1d_bwd_workspace_bytes(int64_t rows, int64_t C) {
  if (rows <= 0 || C <= 0 || !mul_ok(rows, C)) return 0;  // out-of-range sizes fail in the call itself
  const int64_t rr = range_rows_for(rows, ceil_div(C, kBlockChannels), kBwdBlocks, kBwdFixedRows);
  const size_t nrb = (size_t)((rows + rr - 1) / rr);
  // room for any filter width (partial_rows(width) <= partial_rows(kMaxWidth))
  const size_t bytes = nrb * (size_t)partial_rows(kMaxWidth) * (size_t)C * sizeof(float);
  return (bytes + kWsAlign - 1) / kWsAlign * kWsAlign;
}

size_t conv1d_bwd_cf_workspace_bytes(int64_t B, int64_t D) {
  if (B <= 0 || D <= 0 || !mul_ok(B, D)) return 0;  // out-of-range sizes fail in the call itself
  const size_t bytes = (size_t)B * (size_t)partial_rows(kMaxWidth) * (size_t)D * sizeof(float);  // any width
  return (bytes + kWsAlign - 1) / kWsAlign * kWsAlign;
}

const char* conv1d_status_str(int status) {
  switch (status) {
    case CONV1D_OK: return "ok";
    case CONV1D_EINVAL: return "invalid argument (host-checkable precondition failed; nothing launched)";
    case CONV1D_EWORKSPACE: return "workspace missing or too small";
    case CONV1D_EUNSUPPORTED: return "unsupported configuration";
    case CONV1D_EHIP: return "HIP launch error";
    case CONV1D_ETOOLARGE: return "problem too large for the library's scratch (CONV1D_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

int conv1d_fwd(const void* x, int64_t rows, int64_t C, int64_t x_ld, const void* w, int w_dtype, int width,
               const void* b, int b_dtype, const conv1d_seq* seq, const conv1d_pool* pool,
               const conv1d_hist* hist, int act, void* y, int64_t y_ld, void* ws, size_t ws_bytes,
               hipStream_t stream) {
  (void)ws;
  (void)ws_bytes;
  if (rows < 0 || C < 1 || x_ld < C || y_ld < C || !w || !dtype_ok(w_dtype)) return CONV1D_EINVAL;
  if (width < 2 || width > kMaxWidth) return CONV1D_EINVAL;
  if (b && !dtype_ok(b_dtype)) return CONV1D_EINVAL;
  if (act != CONV1D_ACT_NONE && act != CONV1D_ACT_SILU) return CONV1D_EINVAL;
  if (rows > 0 && (!x || !y)) return CONV1D_EINVAL;
  if (!mul_ok(rows, x_ld) || !mul_ok(rows, y_ld) || !mul_ok(C, 16)) return CONV1D_EINVAL;
  int64_t nseq = 0;
  if (check_seq(seq, rows, &nseq) != CONV1D_OK) return CONV1D_EINVAL;
  if (!mul_ok(nseq > 0 ? nseq : 0, 8 * C)) return CONV1D_EINVAL;
  const int mode = mode_of(seq);
  const bool use_pool = pool && pool->ptr;
  const bool use_hist = hist && hist->ptr;
  if (use_pool && use_hist) return CONV1D_EINVAL;
  if ((use_pool || use_hist) && mode == MODE_IDX) return CONV1D_EINVAL;
  if (use_pool && width != 4) return CONV1D_EINVAL;  // the pool form is width four

  const Span sx = span_rows(x, rows, C, x_ld, 2), sy = span_rows(y, rows, C, y_ld, 2);
  const Span sw = span_bytes(w, width * C * dsize(w_dtype)), sb = span_bytes(b, C * dsize(b_dtype));
  Span sp, sh;
  if (use_pool && check_pool(pool, C, nseq, &sp) != CONV1D_OK) return CONV1D_EINVAL;
  if (use_hist) sh = span_bytes(hist->ptr, nseq * (width - 1) * C * 2);
  // out must not share storage with any operand; the pool must not alias the other operands
  const Span sm = span_seq(seq, rows);
  const Span sci = use_pool ? span_bytes(pool->cache_indices, nseq * 4) : Span{};
  const Span shi = use_pool ? span_bytes(pool->has_initial_state, nseq) : Span{};
  const Span shh = use_hist ? span_bytes(hist->has_history, nseq) : Span{};
  const Span ins[8] = {sx, sw, sb, sh, sm, sci, shi, shh};
  for (const Span& in : ins)
    if (overlap(sy, in) || overlap(sp, in)) return CONV1D_EINVAL;
  if (overlap(sy, sp)) return CONV1D_EINVAL;
  if (rows == 0) return CONV1D_OK;

  const bool vec = vec_rows(C, x_ld, x) && vec_rows(C, y_ld, y) && (!use_hist || vec_rows(C, C, hist->ptr)) &&
                   (!use_pool || vec_inplace(C));
  const int64_t rr = fwd_tile_rows(mode, use_pool, width);
  const uint64_t nblk = (uint64_t)ceil_div(C, kBlockChannels) * ceil_div(rows, rr);
  if (nblk > 0x7fffffffull) return CONV1D_EINVAL;

  FwdArgs a{};
  a.x = static_cast<const uint16_t*>(x);
  a.y = static_cast<uint16_t*>(y);
  a.x_ld = x_ld;
  a.y_ld = y_ld;
  a.rows = rows;
  a.C = C;
  a.w = w;
  a.b = b;
  a.w_f32 = w_dtype == CONV1D_F32;
  a.b_f32 = b_dtype == CONV1D_F32;
  a.width = width;
  a.seq = SeqArgs{seq->cu_seqlens, mode == MODE_BATCH ? nseq : seq->nseq, seq->seq_idx, seq->seqlen};
  if (use_pool)
    a.pool = PoolArgs{static_cast<uint16_t*>(pool->ptr), pool->slots, pool->len, pool->s_slot, pool->s_chan, pool->s_pos,
                      pool->cache_indices, pool->has_initial_state};
  if (use_hist) a.hist = HistArgs{static_cast<const uint16_t*>(hist->ptr), hist->has_history};
  a.range_rows = rr;
  a.n_strips = ceil_div(C, kBlockChannels);
  a.n_rowblocks = ceil_div(rows, rr);
  a.tile_order = fwd_tile_order(a.n_strips);
  return launch_fwd(a, mode, vec, act == CONV1D_ACT_SILU, stream) == hipSuccess ? CONV1D_OK : CONV1D_EHIP;
}

// Decode and speculative update share one host path and one kernel (K = 1, all accepted = 1 is
// the decode step).
static int state_update_common(const void* x, int64_t nseq, int64_t K, int64_t C, int64_t x_ld, const void* w,
                               int w_dtype, const void* b, int b_dtype, const conv1d_pool* pool,
                               const int32_t* accepted, int act, void* y, int64_t y_ld, hipStream_t stream) {
  if (nseq < 0 || K < 1 || C < 1 || x_ld < C || y_ld < C || !w || !dtype_ok(w_dtype)) return CONV1D_EINVAL;
  if (b && !dtype_ok(b_dtype)) return CONV1D_EINVAL;
  if (act != CONV1D_ACT_NONE && act != CONV1D_ACT_SILU) return CONV1D_EINVAL;
  if (!pool || !pool->ptr) return CONV1D_EINVAL;
  if (nseq > 0 && (!x || !y)) return CONV1D_EINVAL;
  if (!mul_ok(nseq, K) || !mul_ok(nseq * K, x_ld) || !mul_ok(nseq * K, y_ld) || !mul_ok(C, 16)) return CONV1D_EINVAL;
  Span sp;
  if (check_pool(pool, C, nseq, &sp) != CONV1D_OK) return CONV1D_EINVAL;
  if (pool->len < K + 2) return CONV1D_EINVAL;
  const int64_t rows = nseq * K;
  const Span sx = span_rows(x, rows, C, x_ld, 2), sy = span_rows(y, rows, C, y_ld, 2);
  const Span sw = span_bytes(w, 4 * C * dsize(w_dtype)), sb = span_bytes(b, C * dsize(b_dtype));
  const Span sci = span_bytes(pool->cache_indices, nseq * 4);
  const Span sacc = span_bytes(accepted, nseq * 4);
  const Span ins[5] = {sx, sw, sb, sci, sacc};
  for (const Span& in : ins)
    if (overlap(sy, in) || overlap(sp, in)) return CONV1D_EINVAL;
  if (overlap(sy, sp)) return CONV1D_EINVAL;
  if (nseq == 0) return CONV1D_OK;
  if ((uint64_t)nseq * ceil_div(C, kChannelsPerLane) / kBlockThreads > 0x7fffffffull) return CONV1D_EINVAL;
  const bool vec = vec_rows(C, x_ld, x) && vec_rows(C, y_ld, y) && vec_inplace(C);
  DecodeArgs a{};
  a.x = static_cast<const uint16_t*>(x);
  a.y = static_cast<uint16_t*>(y);
  a.x_ld = x_ld;
  a.y_ld = y_ld;
  a.nseq = nseq;
  a.K = K;
  a.C = C;
  a.w = w;
  a.b = b;
  a.w_f32 = w_dtype == CONV1D_F32;
  a.b_f32 = b_dtype == CONV1D_F32;
  a.pool = PoolArgs{static_cast<uint16_t*>(pool->ptr), pool->slots, pool->len, pool->s_slot, pool->s_chan, pool->s_pos,
                    pool->cache_indices, nullptr};
  a.accepted = accepted;
  return launch_decode(a, vec, act == CONV1D_ACT_SILU, stream) == hipSuccess ? CONV1D_OK : CONV1D_EHIP;
}

int conv1d_state_update(const void* x, int64_t nseq, int64_t C, int64_t x_ld, const void* w, int w_dtype,
                        const void* b, int b_dtype, const conv1d_pool* pool, int act, void* y, int64_t y_ld,
                        hipStream_t stream) {
  return state_update_common(x, nseq, 1, C, x_ld, w, w_dtype, b, b_dtype, pool, nullptr, act, y, y_ld, stream);
}

int conv1d_state_update_spec(const void* x, int64_t nseq, int64_t K, int64_t C, int64_t x_ld, const void* w,
                             int w_dtype, const void* b, int b_dtype, const conv1d_pool* pool,
                             const int32_t* num_accepted, int act, void* y, int64_t y_ld, hipStream_t stream) {
  return state_update_common(x, nseq, K, C, x_ld, w, w_dtype, b, b_dtype, pool, num_accepted, act, y, y_ld, stream);
}

// The backward behind conv1d_bwd and conv1d_bwd_noalloc: with use_scratch, the partials go to the
// library's own scratch (the problem must fit it) and ws / ws_bytes are ignored; otherwise ws is
// the caller's workspace, checked against the size query.
static int bwd_common(const void* x, const void* dy, int64_t rows, int64_t C, int64_t x_ld, int64_t dy_ld,
                      const void* w, int w_dtype, int width, const void* b, int b_dtype, const conv1d_seq* seq,
                      const conv1d_hist* hist, int act, void* dx, int64_t dx_ld, float* dw, float* db,
                      void* dhist, const void* dtail, void* ws, size_t ws_bytes, bool use_scratch,
                      hipStream_t stream) {
  if (rows < 0 || C < 1 || x_ld < C || dy_ld < C || dx_ld < C || !w || !dtype_ok(w_dtype) || !dw)
    return CONV1D_EINVAL;
  if (width < 2 || width > kMaxWidth) return CONV1D_EINVAL;
  if (b && !dtype_ok(b_dtype)) return CONV1D_EINVAL;
  if (act != CONV1D_ACT_NONE && act != CONV1D_ACT_SILU) return CONV1D_EINVAL;
  if (rows > 0 && (!x || !dy || !dx)) return CONV1D_EINVAL;
  if (!mul_ok(rows, x_ld) || !mul_ok(rows, dy_ld) || !mul_ok(rows, dx_ld) || !mul_ok(C, 16)) return CONV1D_EINVAL;
  int64_t nseq = 0;
  if (check_seq(seq, rows, &nseq) != CONV1D_OK) return CONV1D_EINVAL;
  if (!mul_ok(nseq > 0 ? nseq : 0, 8 * C)) return CONV1D_EINVAL;
  const int mode = mode_of(seq);
  const bool use_hist = hist && hist->ptr;
  if (use_hist && mode == MODE_IDX) return CONV1D_EINVAL;
  if (dhist && !use_hist) return CONV1D_EINVAL;
  if (use_scratch) {
    ws = nullptr;
    ws_bytes = 0;
  }
  const size_t need = use_scratch ? 0 : conv1d_bwd_workspace_bytes(rows, C);
  if (ws_bytes < need || (need > 0 && !ws)) return CONV1D_EWORKSPACE;
  if (ws && !aligned(ws, 16)) return CONV1D_EINVAL;

  const Span sx = span_rows(x, rows, C, x_ld, 2), sdy = span_rows(dy, rows, C, dy_ld, 2);
  const Span sdx = span_rows(dx, rows, C, dx_ld, 2);
  const Span sw = span_bytes(w, width * C * dsize(w_dtype)), sb = span_bytes(b, C * dsize(b_dtype));
  const Span sdw = span_bytes(dw, width * C * 4), sdb = span_bytes(db, C * 4);
  const Span sh = use_hist ? span_bytes(hist->ptr, nseq * (width - 1) * C * 2) : Span{};
  const Span sdh = dhist ? span_bytes(dhist, nseq * (width - 1) * C * 2) : Span{};
  const Span sdt = span_bytes(dtail, (width - 1) * C * 2);
  const Span sws = span_bytes(ws, (int64_t)need);
  const Span sm = span_seq(seq, rows);
  const Span shh = use_hist ? span_bytes(hist->has_history, nseq) : Span{};
  const Span outs[5] = {sdx, sdw, sdb, sdh, sws};
  const Span ins[8] = {sx, sdy, sw, sb, sh, sm, shh, sdt};
  for (int i = 0; i < 5; ++i) {
    for (int j = 0; j < 8; ++j)
      if (overlap(outs[i], ins[j])) return CONV1D_EINVAL;
    for (int j = i + 1; j < 5; ++j)
      if (overlap(outs[i], outs[j])) return CONV1D_EINVAL;
  }

  const bool vec = vec_rows(C, x_ld, x) && vec_rows(C, dy_ld, dy) && vec_rows(C, dx_ld, dx) &&
                   (!use_hist || vec_rows(C, C, hist->ptr)) && (!dhist || vec_rows(C, C, dhist)) &&
                   (!dtail || vec_rows(C, C, dtail));
  const int64_t rr = range_rows_for(rows, ceil_div(C, kBlockChannels), kBwdBlocks, kBwdFixedRows);
  const uint64_t nblk = (uint64_t)ceil_div(C, kBlockChannels) * ceil_div(rows, rr);
  if (nblk > 0x7fffffffull || (uint64_t)((36 + (nseq > 0 ? nseq : 0)) * C) / 256 > 0x7fffffffull)
    return CONV1D_EINVAL;
  if (use_scratch && rows > 0) {
    // this width's partials: (ranges) x partial_rows(width) x C FP32
    const uint64_t bytes = (uint64_t)ceil_div(rows, rr) * (uint64_t)partial_rows(width) * (uint64_t)C * 4;
    if (bytes > kScratchBytes) return CONV1D_ETOOLARGE;
    if (bwd_scratch(stream, &ws) != hipSuccess) return CONV1D_EHIP;
  }

  BwdArgs a{};
  a.x = static_cast<const uint16_t*>(x);
  a.dy = static_cast<const uint16_t*>(dy);
  a.dx = static_cast<uint16_t*>(dx);
  a.x_ld = x_ld;
  a.dy_ld = dy_ld;
  a.dx_ld = dx_ld;
  a.rows = rows;
  a.C = C;
  a.w = w;
  a.b = b;
  a.w_f32 = w_dtype == CONV1D_F32;
  a.b_f32 = b_dtype == CONV1D_F32;
  a.width = width;
  a.seq = SeqArgs{seq->cu_seqlens, mode == MODE_BATCH ? nseq : seq->nseq, seq->seq_idx, seq->seqlen};
  if (use_hist) a.hist = HistArgs{static_cast<const uint16_t*>(hist->ptr), hist->has_history};
  a.dhist = static_cast<uint16_t*>(dhist);
  a.dtail = static_cast<const uint16_t*>(dtail);
  a.part = static_cast<float*>(ws);
  a.dw = dw;
  a.db = db;
  a.range_rows = rr;
  a.n_strips = ceil_div(C, kBlockChannels);
  a.n_rowblocks = ceil_div(rows, rr);
  a.tile_order = bwd_tile_order(a.n_strips);
  return launch_bwd(a, mode, vec, act == CONV1D_ACT_SILU, stream) == hipSuccess ? CONV1D_OK : CONV1D_EHIP;
}

int conv1d_bwd(const void* x, const void* dy, int64_t rows, int64_t C, int64_t x_ld, int64_t dy_ld,
               const void* w, int w_dtype, int width, const void* b, int b_dtype, const conv1d_seq* seq,
               const conv1d_hist* hist, int act, void* dx, int64_t dx_ld, float* dw, float* db,
               void* dhist, const void* dtail, void* ws, size_t ws_bytes, hipStream_t stream) {
  return bwd_common(x, dy, rows, C, x_ld, dy_ld, w, w_dtype, width, b, b_dtype, seq, hist, act, dx, dx_ld, dw, db,
                    dhist, dtail, ws, ws_bytes, false, stream);
}

int conv1d_bwd_noalloc(const void* x, const void* dy, int64_t rows, int64_t C, int64_t x_ld, int64_t dy_ld,
                       const void* w, int w_dtype, int width, const void* b, int b_dtype, const conv1d_seq* seq,
                       const conv1d_hist* hist, int act, void* dx, int64_t dx_ld, float* dw, float* db,
                       void* dhist, const void* dtail, hipStream_t stream) {
  return bwd_common(x, dy, rows, C, x_ld, dy_ld, w, w_dtype, width, b, b_dtype, seq, hist, act, dx, dx_ld, dw, db,
                    dhist, dtail, nullptr, 0, true, stream);
}

int conv1d_bwd_combine(const float* dw_parts, const float* db_parts, int64_t nshards, int64_t C, int width,
                       float* dw, float* db, hipStream_t stream) {
  if (nshards < 0 || C < 1 || width < 2 || width > kMaxWidth || !dw) return CONV1D_EINVAL;
  if ((nshards > 0 && !dw_parts) || (db && nshards > 0 && !db_parts)) return CONV1D_EINVAL;
  if (!mul_ok(nshards, C * kMaxWidth) || !mul_ok(C, 4 * kMaxWidth)) return CONV1D_EINVAL;
  if ((uint64_t)((width + 1) * C) / kBlockThreads > 0x7fffffffull) return CONV1D_EINVAL;
  const Span sp = span_bytes(dw_parts, nshards * C * width * 4);
  const Span spb = db ? span_bytes(db_parts, nshards * C * 4) : Span{};
  const Span sdw = span_bytes(dw, C * width * 4), sdb = span_bytes(db, C * 4);
  if (overlap(sdw, sp) || overlap(sdw, spb) || overlap(sdb, sp) || overlap(sdb, spb) || overlap(sdw, sdb))
    return CONV1D_EINVAL;
  CombineArgs a{};
  a.dw_parts = dw_parts;
  a.db_parts = db ? db_parts : nullptr;
  a.dw = dw;
  a.db = db;
  a.nshards = nshards;
  a.C = C;
  a.width = width;
  return launch_combine(a, stream) == hipSuccess ? CONV1D_OK : CONV1D_EHIP;
}

int conv1d_fwd_cf(const void* x, int64_t B, int64_t D, int64_t T, int64_t x_sb, int64_t x_sd, const void* w,
                  int w_dtype, int width, const void* b, int b_dtype, int act, void* y, int64_t y_sb, int64_t y_sd,
                  hipStream_t stream) {
  if (B < 0 || D < 1 || T < 0 || !w || !dtype_ok(w_dtype) || width < 2 || width > kMaxWidth) return CONV1D_EINVAL;
  if (b && !dtype_ok(b_dtype)) return CONV1D_EINVAL;
  if (act != CONV1D_ACT_NONE && act != CONV1D_ACT_SILU) return CONV1D_EINVAL;
  if (!cf_layout_ok(B, D, T, x_sb, x_sd) || !cf_layout_ok(B, D, T, y_sb, y_sd)) return CONV1D_EINVAL;
  if (B * T > 0 && (!x || !y)) return CONV1D_EINVAL;
  const Span sx = span_cf(x, B, D, T, x_sb, x_sd), sy = span_cf(y, B, D, T, y_sb, y_sd);
  const Span sw = span_bytes(w, width * D * dsize(w_dtype)), sb = span_bytes(b, D * dsize(b_dtype));
  if (overlap(sy, sx) || overlap(sy, sw) || overlap(sy, sb)) return CONV1D_EINVAL;
  if (B * T == 0) return CONV1D_OK;
  if ((uint64_t)(B * D + 3) / 4 > 0x7fffffffull) return CONV1D_EINVAL;
  const bool vec = T % 8 == 0 && x_sb % 8 == 0 && x_sd % 8 == 0 && y_sb % 8 == 0 && y_sd % 8 == 0 &&
                   aligned(x, 16) && aligned(y, 16);
  CfArgs a{};
  a.x = static_cast<const uint16_t*>(x);
  a.out = static_cast<uint16_t*>(y);
  a.B = B;
  a.D = D;
  a.T = T;
  a.x_sb = x_sb;
  a.x_sd = x_sd;
  a.o_sb = y_sb;
  a.o_sd = y_sd;
  a.w = w;
  a.b = b;
  a.w_f32 = w_dtype == CONV1D_F32;
  a.b_f32 = b_dtype == CONV1D_F32;
  a.width = width;
  return launch_fwd_cf(a, vec, act == CONV1D_ACT_SILU, stream) == hipSuccess ? CONV1D_OK : CONV1D_EHIP;
}

int conv1d_bwd_cf(const void* x, const void* dy, int64_t B, int64_t D, int64_t T, int64_t x_sb, int64_t x_sd,
                  int64_t dy_sb, int64_t dy_sd, const void* w, int w_dtype, int width, const void* b, int b_dtype,
                  int act, void* dx, int64_t dx_sb, int64_t dx_sd, float* dw, float* db, void* ws, size_t ws_bytes,
                  hipStream_t stream) {
  if (B < 0 || D < 1 || T < 0 || !w || !dtype_ok(w_dtype) || !dw || width < 2 || width > kMaxWidth) return CONV1D_EINVAL;
  if (b && !dtype_ok(b_dtype)) return CONV1D_EINVAL;
  if (act != CONV1D_ACT_NONE && act != CONV1D_ACT_SILU) return CONV1D_EINVAL;
  if (!cf_layout_ok(B, D, T, x_sb, x_sd) || !cf_layout_ok(B, D, T, dy_sb, dy_sd) ||
      !cf_layout_ok(B, D, T, dx_sb, dx_sd))
    return CONV1D_EINVAL;
  if (B * T > 0 && (!x || !dy || !dx)) return CONV1D_EINVAL;
  const size_t need = conv1d_bwd_cf_workspace_bytes(B, D);
  if (ws_bytes < need || (need > 0 && !ws)) return CONV1D_EWORKSPACE;
  if (ws && !aligned(ws, 16)) return CONV1D_EINVAL;
  const Span sx = span_cf(x, B, D, T, x_sb, x_sd), sdy = span_cf(dy, B, D, T, dy_sb, dy_sd);
  const Span sdx = span_cf(dx, B, D, T, dx_sb, dx_sd);
  const Span sw = span_bytes(w, width * D * dsize(w_dtype)), sb = span_bytes(b, D * dsize(b_dtype));
  const Span sdw = span_bytes(dw, width * D * 4), sdb = span_bytes(db, D * 4), sws = span_bytes(ws, (int64_t)need);
  const Span outs[4] = {sdx, sdw, sdb, sws};
  const Span ins[4] = {sx, sdy, sw, sb};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 4; ++j)
      if (overlap(outs[i], ins[j])) return CONV1D_EINVAL;
    for (int j = i + 1; j < 4; ++j)
      if (overlap(outs[i], outs[j])) return CONV1D_EINVAL;
  }
  if ((uint64_t)(B * D + 3) / 4 > 0x7fffffffull || (uint64_t)(36 * D) / 256 > 0x7fffffffull) return CONV1D_EINVAL;
  const bool vec = T % 8 == 0 && x_sb % 8 == 0 && x_sd % 8 == 0 && dy_sb % 8 == 0 && dy_sd % 8 == 0 &&
                   dx_sb % 8 == 0 && dx_sd % 8 == 0 && aligned(x, 16) && aligned(dy, 16) && aligned(dx, 16);
  CfArgs a{};
  a.x = static_cast<const uint16_t*>(x);
  a.dy = static_cast<const uint16_t*>(dy);
  a.out = static_cast<uint16_t*>(dx);
  a.B = B;
  a.D = D;
  a.T = T;
  a.x_sb = x_sb;
  a.x_sd = x_sd;
  a.dy_sb = dy_sb;
  a.dy_sd = dy_sd;
  a.o_sb = dx_sb;
  a.o_sd = dx_sd;
  a.w = w;
  a.b = b;
  a.w_f32 = w_dtype == CONV1D_F32;
  a.b_f32 = b_dtype == CONV1D_F32;
  a.width = width;
  a.part = static_cast<float*>(ws);
  if (launch_bwd_cf(a, vec, act == CONV1D_ACT_SILU, stream) != hipSuccess) return CONV1D_EHIP;
  BwdArgs r{};
  r.C = D;
  r.width = width;
  r.part = a.part;
  r.dw = dw;
  r.db = db;
  r.n_rowblocks = (uint32_t)B;
  return launch_reduce(r, stream) == hipSuccess ? CONV1D_OK : CONV1D_EHIP;
}

}  // extern "C"
