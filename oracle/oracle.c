/*
 * oracle.c -- plain CPU reference for the packed width-4 depthwise causal Conv1d (+ SiLU).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or calls this file;
 * only the tests, the smoke check and the benchmark's CPU-baseline leg do.  It shares no
 * code, header, table or helper with the HIP library.
 *
 * What it computes, and where the pages say so:
 *   - flashinfer.mamba.causal_conv1d_fn (FlashInfer docs), Parameters x / weight / conv_state /
 *     cu_seqlens / cache_indices / has_initial_state / bias / out, and Notes:
 *       width-four taps [C,4], tap 3 on the current token, bias added before the four FMAs,
 *       FP32 accumulation and SiLU, raw inputs kept as history, -1 slot gives zero output and
 *       no state access, positions 0:3 of a live slot receive the last three raw values of a
 *       nonempty sequence, empty sequences and rows past the last offset are left alone.
 *   - core.ssm.causal_conv1d.causal_conv1d_cp (Megatron-Core docs), Parameters weight /
 *     bias / activation / global_seq_idx: optional bias and activation, per-token sequence IDs
 *     with a state reset at every sequence boundary.
 *   - flashinfer.cake_causal_conv1d_train.cake_causal_conv1d_kcp (FlashInfer docs), summary and
 *     Returns: a fragment that continues a document reads history rows instead of zeros, and the
 *     backward produces dx, a deterministic FP32 dweight and the gradient of the history rows;
 *     the successor's history-row gradient comes back into the shard's last rows (d(tail)).
 *   - core.ssm.causal_conv1d.assert_causal_conv1d_deterministic (Megatron-Core docs): dweight
 *     contributions added in a fixed order, here per-shard partials in ascending shard order.
 *
 * Readings where the pages leave a step open (all listed in the design notes):
 *   - history position j (j = 0,1,2) holds the raw input 3-j rows before the segment's first
 *     row, oldest first; the same order is used for the caller's history rows;
 *   - the FP32 accumulation is z = fma(w3,u[t], fma(w2,u[t-1], fma(w1,u[t-2], fma(w0,u[t-3], b))));
 *   - SiLU is z*sigmoid(z), evaluated in double from that FP32 z, rounded once to bf16 (RNE);
 *   - the backward is computed in double from the same FP32 z; dweight/dbias are rounded to
 *     float once at the end; dx and d(history) are rounded to bf16 (RNE) once;
 *   - the speculative update (causal_conv1d_fn, Notes: accepted count 1 after a prefill) reads
 *     its history at positions a-1 .. a+1 and leaves the last K + 2 raw values at 0 .. K+1.
 *
 * The loops below follow the definition directly: per segment, per channel, build the extended
 * sequence u = [h0, h1, h2, x[s], ..., x[e-1]] and apply the stencil.  OpenMP only splits the
 * channels; every per-channel sum keeps its serial order, so results do not depend on the
 * thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OR_OK 0
#define OR_INVALID 1
#define OR_NOMEM 2

/* ---------------------------------------------------------------- bf16 bit handling */

static float bf16_bits_to_float(uint16_t h) {
  uint32_t u = (uint32_t)h << 16; /* bf16 is the top half of an IEEE binary32 */
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

/* round-to-nearest-even of a binary32 value to bf16 (8 significant bits) */
static uint16_t float_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0; /* NaN: never produced by valid input */
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7fffu + lsb;
  return (uint16_t)(u >> 16);
}

/* round-to-nearest-even of a double to bf16, without the double rounding that going through
   float could introduce: when the float lands exactly on a bf16 halfway point, the exact
   residual d - (double)f decides the direction. */
static uint16_t double_to_bf16_rne(double d) {
  float f = (float)d;
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  if ((u & 0x7fffffffu) >= 0x7f800000u) return float_to_bf16_rne(f);
  if ((u & 0xffffu) == 0x8000u) {
    double r = d - (double)f; /* exact: f is d rounded to 24 bits (Sterbenz) */
    if (r != 0.0) {
      uint32_t mag_up = ((r > 0.0) == (f > 0.0));
      return (uint16_t)((u >> 16) + mag_up);
    }
  }
  return float_to_bf16_rne(f);
}

static double sigmoid_d(double z) { return 1.0 / (1.0 + exp(-z)); }

/* ---------------------------------------------------------------- segments */

typedef struct {
  int64_t s, e; /* rows [s, e) */
  int64_t i;    /* sequence index: into cache_indices / has_initial_state / history */
} seg_t;

/* Segments of the packed rows.
   cu_seqlens given: sequence i covers rows [cu[i], cu[i+1]) (flashinfer causal_conv1d_fn,
     Parameters cu_seqlens).
   seq_idx given: maximal runs of equal ID inside one batch row of `seqlen` rows; the state resets
     at every boundary (causal_conv1d_cp, Parameters global_seq_idx).
   neither: each batch row of `seqlen` rows is one sequence.
   Returns the count, or -1 on invalid metadata. */
static int64_t build_segments(int64_t rows, const int32_t* cu, int64_t nseq, const int32_t* seq_idx,
                              int64_t seqlen, seg_t** out) {
  seg_t* v = NULL;
  int64_t n = 0;
  if (cu) {
    if (nseq < 0 || cu[0] != 0 || cu[nseq] > rows) return -1;
    v = (seg_t*)malloc(sizeof(seg_t) * (size_t)(nseq > 0 ? nseq : 1));
    if (!v) return -1;
    for (int64_t i = 0; i < nseq; ++i) {
      if (cu[i + 1] < cu[i]) { free(v); return -1; }
      v[n].s = cu[i];
      v[n].e = cu[i + 1];
      v[n].i = i;
      ++n;
    }
  } else {
    if (seqlen <= 0 || rows % seqlen != 0) return -1;
    v = (seg_t*)malloc(sizeof(seg_t) * (size_t)(rows > 0 ? rows : 1));
    if (!v) return -1;
    for (int64_t b0 = 0; b0 < rows; b0 += seqlen) {
      int64_t s = b0;
      for (int64_t t = b0 + 1; t <= b0 + seqlen; ++t) {
        int boundary = (t == b0 + seqlen);
        if (!boundary && seq_idx) {
          if (seq_idx[t] < 0) { free(v); return -1; }
          boundary = (seq_idx[t] != seq_idx[t - 1]);
        }
        if (boundary) {
          v[n].s = s;
          v[n].e = t;
          v[n].i = n;
          ++n;
          s = t;
        }
      }
      if (seq_idx && seq_idx[b0] < 0) { free(v); return -1; }
    }
  }
  *out = v;
  return n;
}

static float load_tap(const void* w, int is_f32, int64_t idx) {
  return is_f32 ? ((const float*)w)[idx] : bf16_bits_to_float(((const uint16_t*)w)[idx]);
}

typedef struct {
  /* slot pool: element (slot, c, j) at pool[slot*s_slot + c*s_chan + j*s_pos] */
  uint16_t* pool;
  int64_t slots, len, s_slot, s_chan, s_pos;
  const int32_t* cache_indices;
  const uint8_t* has_init;
  /* caller history rows: element (i, j, c) at hist[(i*H + j)*C + c], H = width - 1 */
  const uint16_t* hist;
  const uint8_t* has_hist;
  int64_t H;
} ctx_t;

/* raw bits of history position j of sequence i, channel c (0 when the sequence starts from zero) */
static uint16_t history_bits(const ctx_t* k, int64_t i, int64_t c, int64_t C, int j) {
  if (k->pool) {
    int32_t slot = k->cache_indices[i];
    if (slot >= 0 && k->has_init && k->has_init[i])
      return k->pool[slot * k->s_slot + c * k->s_chan + j * k->s_pos];
    return 0;
  }
  if (k->hist && (!k->has_hist || k->has_hist[i])) return k->hist[(i * k->H + j) * C + c];
  return 0;
}

static int validate_pool(const ctx_t* k, int64_t nseq, int64_t C) {
  if (!k->pool) return OR_OK;
  if (!k->cache_indices || k->len < 3 || k->slots < 0) return OR_INVALID;
  if (k->s_slot <= 0 || k->s_chan <= 0 || k->s_pos <= 0) return OR_INVALID;
  for (int64_t i = 0; i < nseq; ++i) {
    int32_t a = k->cache_indices[i];
    if (a == -1) continue;
    if (a < 0 || a >= k->slots) return OR_INVALID; /* only -1 is the sentinel */
    for (int64_t j = 0; j < i; ++j)
      if (k->cache_indices[j] == a) return OR_INVALID; /* live slots are unique */
  }
  (void)C;
  return OR_OK;
}

static int set_threads(int nthreads) {
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
  return omp_get_max_threads();
#else
  (void)nthreads;
  return 1;
#endif
}

/* one output value of the stencil, exactly in the stated FP32 order */
static float stencil_f32(float b, float w0, float w1, float w2, float w3, float um3, float um2,
                         float um1, float u0) {
  float z = b;
  z = fmaf(w0, um3, z);
  z = fmaf(w1, um2, z);
  z = fmaf(w2, um1, z);
  z = fmaf(w3, u0, z);
  return z;
}

/* the same for W taps: z = b, then tap k on u[k] (tap W-1 on the current value), k = 0..W-1 */
static float stencil_w(float b, const float* wt, const float* u, int W) {
  float z = b;
  for (int kk = 0; kk < W; ++kk) z = fmaf(wt[kk], u[kk], z);
  return z;
}

/* ================================================================ forward
   y[t][c] for every row of every segment; pool positions 0:3 of live nonempty sequences.
   width W (2..8): taps [C, W], W - 1 history values (caller history rows [nseq, W-1, C]); the
   pool form is width four only.  act: 0 = identity, 1 = SiLU.  Returns OR_OK / OR_INVALID /
   OR_NOMEM. */
int oracle_fwd(const uint16_t* x, int64_t rows, int64_t C, int64_t x_ld, const void* w, int w_f32,
               int width, const void* b, int b_f32, const int32_t* cu_seqlens, int64_t nseq,
               const int32_t* seq_idx, int64_t seqlen, uint16_t* pool, int64_t slots, int64_t len,
               int64_t s_slot, int64_t s_chan, int64_t s_pos, const int32_t* cache_indices,
               const uint8_t* has_init, const uint16_t* hist, const uint8_t* has_hist, int act,
               uint16_t* y, int64_t y_ld, int nthreads) {
  if (!x && rows > 0) return OR_INVALID;
  if (!w || !y || C < 1 || x_ld < C || y_ld < C || rows < 0 || (act != 0 && act != 1))
    return OR_INVALID;
  if (width < 2 || width > 8 || (pool && width != 4)) return OR_INVALID;
  if (pool && hist) return OR_INVALID;
  if ((pool || hist) && !cu_seqlens && seq_idx) return OR_INVALID;
  const int W = width, H = width - 1;
  seg_t* segs = NULL;
  int64_t ns = build_segments(rows, cu_seqlens, nseq, seq_idx, seqlen, &segs);
  if (ns < 0) return OR_INVALID;
  ctx_t k = {pool, slots, len, s_slot, s_chan, s_pos, cache_indices, has_init, hist, has_hist, H};
  if (validate_pool(&k, ns, C) != OR_OK) { free(segs); return OR_INVALID; }
  int64_t maxlen = 0;
  for (int64_t q = 0; q < ns; ++q)
    if (segs[q].e - segs[q].s > maxlen) maxlen = segs[q].e - segs[q].s;
  set_threads(nthreads);
  int err = 0;
#pragma omp parallel
  {
    uint16_t* ubits = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(maxlen + H));
    float* u = (float*)malloc(sizeof(float) * (size_t)(maxlen + H));
    if (!ubits || !u) {
#pragma omp atomic write
      err = 1;
    } else {
#pragma omp for schedule(static)
      for (int64_t cb = 0; cb < (C + 63) / 64; ++cb) {
        for (int64_t c = cb * 64; c < C && c < cb * 64 + 64; ++c) {
          float wt[8];
          for (int kk = 0; kk < W; ++kk) wt[kk] = load_tap(w, w_f32, c * W + kk);
          float bias = b ? load_tap(b, b_f32, c) : 0.0f;
          for (int64_t q = 0; q < ns; ++q) {
            int64_t s = segs[q].s, n = segs[q].e - segs[q].s, i = segs[q].i;
            if (pool && cache_indices[i] == -1) { /* sentinel: +0 output, no state access */
              for (int64_t t = 0; t < n; ++t) y[(s + t) * y_ld + c] = 0;
              continue;
            }
            /* extended sequence: u[0..H-1] = history, u[H+t] = x[s+t] */
            for (int j = 0; j < H; ++j) ubits[j] = history_bits(&k, i, c, C, j);
            for (int64_t t = 0; t < n; ++t) ubits[H + t] = x[(s + t) * x_ld + c];
            for (int64_t t = 0; t < n + H; ++t) u[t] = bf16_bits_to_float(ubits[t]);
            for (int64_t t = 0; t < n; ++t) {
              float z = stencil_w(bias, wt, u + t, W);
              uint16_t out;
              if (act == 1) {
                double zd = (double)z;
                out = double_to_bf16_rne(zd * sigmoid_d(zd));
              } else {
                out = float_to_bf16_rne(z);
              }
              y[(s + t) * y_ld + c] = out;
            }
            /* state write-back: the last three raw values of the extended sequence */
            if (pool && n > 0) {
              int32_t slot = cache_indices[i];
              for (int j = 0; j < 3; ++j)
                pool[slot * s_slot + c * s_chan + j * s_pos] = ubits[n + j];
            }
          }
        }
      }
    }
    free(ubits);
    free(u);
  }
  free(segs);
  return err ? OR_NOMEM : OR_OK;
}

/* ================================================================ decode step
   One new token per sequence against its slot's history (has_initial_state taken as true for
   every sequence), followed by the state shift h <- [h1, h2, x].  The -1 sentinel gives +0 and
   leaves the pool alone.  Written independently of oracle_fwd; the tests pin the two equal. */
int oracle_state_update(const uint16_t* x, int64_t nseq, int64_t C, int64_t x_ld, const void* w,
                        int w_f32, const void* b, int b_f32, uint16_t* pool, int64_t slots,
                        int64_t len, int64_t s_slot, int64_t s_chan, int64_t s_pos,
                        const int32_t* cache_indices, int act, uint16_t* y, int64_t y_ld) {
  if (!w || !pool || !cache_indices || C < 1 || x_ld < C || y_ld < C || nseq < 0) return OR_INVALID;
  if (nseq > 0 && (!x || !y)) return OR_INVALID;
  ctx_t k = {pool, slots, len, s_slot, s_chan, s_pos, cache_indices, NULL, NULL, NULL, 3};
  if (validate_pool(&k, nseq, C) != OR_OK) return OR_INVALID;
  for (int64_t i = 0; i < nseq; ++i) {
    int32_t slot = cache_indices[i];
    for (int64_t c = 0; c < C; ++c) {
      if (slot == -1) { y[i * y_ld + c] = 0; continue; }
      uint16_t* h = pool + slot * s_slot + c * s_chan;
      uint16_t h0 = h[0], h1 = h[s_pos], h2 = h[2 * s_pos], xv = x[i * x_ld + c];
      float z = stencil_f32(b ? load_tap(b, b_f32, c) : 0.0f, load_tap(w, w_f32, c * 4 + 0),
                            load_tap(w, w_f32, c * 4 + 1), load_tap(w, w_f32, c * 4 + 2),
                            load_tap(w, w_f32, c * 4 + 3), bf16_bits_to_float(h0),
                            bf16_bits_to_float(h1), bf16_bits_to_float(h2), bf16_bits_to_float(xv));
      if (act == 1) {
        double zd = (double)z;
        y[i * y_ld + c] = double_to_bf16_rne(zd * sigmoid_d(zd));
      } else {
        y[i * y_ld + c] = float_to_bf16_rne(z);
      }
      h[0] = h1;
      h[s_pos] = h2;
      h[2 * s_pos] = xv;
    }
  }
  return OR_OK;
}

/* ================================================================ speculative multi-token update
   Reading of flashinfer.mamba.causal_conv1d_fn, Notes (the first speculative update after a
   prefill uses accepted count 1), stated in the design notes:
     - a slot's positions hold raw inputs, oldest first;
     - a step feeds K tokens x_1..x_K per sequence, and `accepted` says how many tokens of the
       previous step were kept, so the three raw values before x_1 sit at positions a-1, a, a+1
       (after a prefill a = 1: positions 0..2, where the prefill leaves them);
     - y_k is the stencil over the extended sequence u = [h0, h1, h2, x_1, ..., x_K];
     - afterwards positions 0..K+1 hold u[1..K+2], the last K + 2 raw values.  Whatever prefix a'
       of these K tokens the next step accepts, the three values before its first token are then
       at positions a'-1 .. a'+1.
   Positions >= K + 2 are left alone, a -1 slot gives +0 and no state access, K = 1 with a = 1 is
   the ordinary decode step.  Needs L >= K + 2 and 1 <= a <= L - 2 for every live sequence. */
int oracle_spec_update(const uint16_t* x, int64_t nseq, int64_t K, int64_t C, int64_t x_ld,
                       const void* w, int w_f32, const void* b, int b_f32, uint16_t* pool,
                       int64_t slots, int64_t len, int64_t s_slot, int64_t s_chan, int64_t s_pos,
                       const int32_t* cache_indices, const int32_t* accepted, int act, uint16_t* y,
                       int64_t y_ld) {
  if (!w || !pool || !cache_indices || C < 1 || K < 1 || x_ld < C || y_ld < C || nseq < 0 ||
      (act != 0 && act != 1))
    return OR_INVALID;
  if (nseq > 0 && (!x || !y)) return OR_INVALID;
  if (len < K + 2) return OR_INVALID;
  ctx_t k = {pool, slots, len, s_slot, s_chan, s_pos, cache_indices, NULL, NULL, NULL, 3};
  if (validate_pool(&k, nseq, C) != OR_OK) return OR_INVALID;
  for (int64_t i = 0; i < nseq; ++i) {
    int32_t a = accepted ? accepted[i] : 1;
    if (cache_indices[i] != -1 && (a < 1 || a > len - 2)) return OR_INVALID;
  }
  uint16_t* u = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(K + 3));
  if (!u) return OR_NOMEM;
  for (int64_t i = 0; i < nseq; ++i) {
    int32_t slot = cache_indices[i];
    int64_t a = accepted ? accepted[i] : 1;
    for (int64_t c = 0; c < C; ++c) {
      if (slot == -1) {
        for (int64_t t = 0; t < K; ++t) y[(i * K + t) * y_ld + c] = 0;
        continue;
      }
      uint16_t* h = pool + slot * s_slot + c * s_chan;
      for (int j = 0; j < 3; ++j) u[j] = h[(a - 1 + j) * s_pos];
      for (int64_t t = 0; t < K; ++t) u[3 + t] = x[(i * K + t) * x_ld + c];
      for (int64_t t = 0; t < K; ++t) {
        float z = stencil_f32(b ? load_tap(b, b_f32, c) : 0.0f, load_tap(w, w_f32, c * 4 + 0),
                              load_tap(w, w_f32, c * 4 + 1), load_tap(w, w_f32, c * 4 + 2),
                              load_tap(w, w_f32, c * 4 + 3), bf16_bits_to_float(u[t]),
                              bf16_bits_to_float(u[t + 1]), bf16_bits_to_float(u[t + 2]),
                              bf16_bits_to_float(u[t + 3]));
        if (act == 1) {
          double zd = (double)z;
          y[(i * K + t) * y_ld + c] = double_to_bf16_rne(zd * sigmoid_d(zd));
        } else {
          y[(i * K + t) * y_ld + c] = float_to_bf16_rne(z);
        }
      }
      for (int64_t j = 0; j < K + 2; ++j) h[j * s_pos] = u[j + 1];
    }
  }
  free(u);
  return OR_OK;
}

/* ================================================================ backward
   Given dy = dL/dy, produce dx = dL/dx (bf16), dw[c][k] = dL/dw (float), db[c] = dL/db (float,
   when db != NULL) and, for sequences that read caller history rows, dhist[i][j][c] = dL/dh_j
   (bf16).  The FP32 z of the forward is recomputed exactly; everything after it is double.  With
   W taps and H = W - 1 history values:
     dz[t]  = dy[t] * act'(z[t])           silu'(z) = s(z) * (1 + z * (1 - s(z)))
     dx[t]  = sum_{k : t+H-k inside the segment} w_k * dz[t+H-k]
     dw_k   = sum over segments and t of dz[t] * u[t+k]      (u[H+t] = x[s+t])
     db     = sum of dz
     dh_j   = sum_{tau = 0 .. min(j, n-1)} w_{j-tau} * dz[tau]
   Rows outside every segment are not written.
   dtail (bf16 [H, C], or NULL): the gradient that arrives from the next shard for the last H values
   of the last segment's extended sequence u (cake_causal_conv1d_kcp, Returns: the successor's
   history-row gradient flows back into this shard; core.ssm.causal_conv1d, _exchange_initial_states
   is differentiable).  Tail value j is u[n+j] of the last segment: it adds to dx[s+n+j-H] when
   n+j >= H, else to that segment's dh_{n+j}; the sum stays in double and is rounded once. */
int oracle_bwd(const uint16_t* x, const uint16_t* dy, int64_t rows, int64_t C, int64_t x_ld,
               int64_t dy_ld, const void* w, int w_f32, int width, const void* b, int b_f32,
               const int32_t* cu_seqlens, int64_t nseq, const int32_t* seq_idx, int64_t seqlen,
               const uint16_t* hist, const uint8_t* has_hist, int act, uint16_t* dx, int64_t dx_ld,
               float* dw, float* db, uint16_t* dhist, const uint16_t* dtail, int nthreads) {
  if ((!x || !dy || !dx) && rows > 0) return OR_INVALID;
  if (!w || !dw || C < 1 || x_ld < C || dy_ld < C || dx_ld < C || rows < 0 ||
      (act != 0 && act != 1))
    return OR_INVALID;
  if (width < 2 || width > 8) return OR_INVALID;
  if (hist && !cu_seqlens && seq_idx) return OR_INVALID;
  if (dhist && !hist) return OR_INVALID;
  const int W = width, H = width - 1;
  seg_t* segs = NULL;
  int64_t ns = build_segments(rows, cu_seqlens, nseq, seq_idx, seqlen, &segs);
  if (ns < 0) return OR_INVALID;
  ctx_t k = {NULL, 0, 0, 0, 0, 0, NULL, NULL, hist, has_hist, H};
  int64_t maxlen = 0;
  for (int64_t q = 0; q < ns; ++q)
    if (segs[q].e - segs[q].s > maxlen) maxlen = segs[q].e - segs[q].s;
  set_threads(nthreads);
  int err = 0;
#pragma omp parallel
  {
    double* u = (double*)malloc(sizeof(double) * (size_t)(maxlen + H));
    float* uf = (float*)malloc(sizeof(float) * (size_t)(maxlen + H));
    double* dz = (double*)malloc(sizeof(double) * (size_t)(maxlen + 1));
    if (!u || !uf || !dz) {
#pragma omp atomic write
      err = 1;
    } else {
#pragma omp for schedule(static)
      for (int64_t cb = 0; cb < (C + 63) / 64; ++cb) {
        for (int64_t c = cb * 64; c < C && c < cb * 64 + 64; ++c) {
          float wf[8];
          for (int q = 0; q < W; ++q) wf[q] = load_tap(w, w_f32, c * W + q);
          float bias = b ? load_tap(b, b_f32, c) : 0.0f;
          double dw_acc[8] = {0, 0, 0, 0, 0, 0, 0, 0}, db_acc = 0;
          for (int64_t q = 0; q < ns; ++q) {
            int64_t s = segs[q].s, n = segs[q].e - segs[q].s, i = segs[q].i;
            for (int j = 0; j < H; ++j) u[j] = bf16_bits_to_float(history_bits(&k, i, c, C, j));
            for (int64_t t = 0; t < n; ++t) u[H + t] = bf16_bits_to_float(x[(s + t) * x_ld + c]);
            for (int64_t t = 0; t < n + H; ++t) uf[t] = (float)u[t];
            for (int64_t t = 0; t < n; ++t) {
              float z = stencil_w(bias, wf, uf + t, W);
              double g = bf16_bits_to_float(dy[(s + t) * dy_ld + c]);
              if (act == 1) {
                double zd = (double)z, sg = sigmoid_d(zd);
                g *= sg * (1.0 + zd * (1.0 - sg));
              }
              dz[t] = g;
            }
            const int tail = dtail && q == ns - 1; /* the last segment takes the next shard's gradient */
            for (int64_t t = 0; t < n; ++t) {
              double acc = 0;
              for (int kk = 0; kk < W; ++kk) {
                int64_t tau = t + H - kk;
                if (tau < n) acc += (double)wf[kk] * dz[tau];
              }
              if (tail && t + H - n >= 0) acc += bf16_bits_to_float(dtail[(t + H - n) * C + c]);
              dx[(s + t) * dx_ld + c] = double_to_bf16_rne(acc);
            }
            for (int64_t t = 0; t < n; ++t) {
              for (int kk = 0; kk < W; ++kk) dw_acc[kk] += dz[t] * u[t + kk];
              db_acc += dz[t];
            }
            if (dhist && (!has_hist || has_hist[i])) {
              for (int j = 0; j < H; ++j) {
                double acc = 0;
                for (int64_t tau = 0; tau <= j && tau < n; ++tau) acc += (double)wf[j - tau] * dz[tau];
                if (tail && j - n >= 0) acc += bf16_bits_to_float(dtail[(j - n) * C + c]);
                dhist[(i * H + j) * C + c] = double_to_bf16_rne(acc);
              }
            }
          }
          for (int kk = 0; kk < W; ++kk) dw[c * W + kk] = (float)dw_acc[kk];
          if (db) db[c] = (float)db_acc;
        }
      }
    }
    free(u);
    free(uf);
    free(dz);
  }
  free(segs);
  return err ? OR_NOMEM : OR_OK;
}

/* ================================================================ shard-ordered combine
   The deterministic mode of core.ssm.causal_conv1d (assert_causal_conv1d_deterministic): per-shard
   FP32 dweight / dbias contributions are added in a fixed order instead of by atomics.  Reading:
   out[e] = (((p_0[e] + p_1[e]) + p_2[e]) + ...) + p_{S-1}[e], one FP32 addition per shard in
   ascending shard order, starting from shard 0's value (so one shard is returned bit for bit).
   parts: [nshards, n] float, contiguous.  nshards = 0 gives zeros. */
int oracle_combine(const float* parts, int64_t nshards, int64_t n, float* out) {
  if (nshards < 0 || n < 0 || (n > 0 && (!out || (nshards > 0 && !parts)))) return OR_INVALID;
  for (int64_t e = 0; e < n; ++e) {
    float acc = nshards > 0 ? parts[e] : 0.0f;
    for (int64_t sh = 1; sh < nshards; ++sh) acc = acc + parts[sh * n + e];
    out[e] = acc;
  }
  return OR_OK;
}

uint16_t oracle_round_double_to_bf16(double d) { return double_to_bf16_rne(d); }
uint16_t oracle_round_float_to_bf16(float f) { return float_to_bf16_rne(f); }
int oracle_max_threads(void) { return set_threads(0); }
