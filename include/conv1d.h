/*
 * conv1d.h -- C ABI of the MI355X (gfx950) packed depthwise causal Conv1d (+ SiLU), filter
 * width 4 (widths 2..8 for every form without a slot pool).
 *
 * The operation (FlashInfer docs, flashinfer.mamba.causal_conv1d_fn, Parameters and Notes):
 * for every packed sequence with rows [s, e) and channel c, with the extended sequence
 *     u[-3], u[-2], u[-1] = the sequence's history (zeros unless stated otherwise),
 *     u[t] = x[s + t]                                              (raw bf16 inputs),
 *     z[t] = b[c] + w[c][0]*u[t-3] + w[c][1]*u[t-2] + w[c][2]*u[t-1] + w[c][3]*u[t]
 * accumulated in FP32 (bias first, then taps 0..3 as fused multiply-adds; tap 3 multiplies the
 * current token), and y[s + t][c] = act(z[t]) rounded to bf16 (round to nearest even), where
 * act is SiLU (z * sigmoid(z), FP32) or the identity (the Megatron-Core page
 * core.ssm.causal_conv1d.causal_conv1d_cp makes bias and activation optional).
 *
 * Conventions shared by every entry point:
 *   - All data pointers are DEVICE pointers; the caller owns every buffer.  The library never
 *     allocates, never reads device memory on the host, never synchronizes, and keeps no
 *     mutable global state: every call only enqueues kernels on `stream` (a hipStream_t, NULL =
 *     the null stream), so calls can be captured in a HIP graph and replayed with device
 *     metadata (offsets, slots, flags) changed in place within the same capacities
 *     (causal_conv1d_fn, Notes).
 *   - bf16 tensors are 16-bit bf16 bit patterns.  x, y, dy, dx are row-major [rows, C] with a
 *     row stride (`*_ld`, in elements, >= C) and contiguous channels.
 *   - Taps w are a contiguous [C, W] array of FP32 or bf16 (`w_dtype`) with filter width
 *     W = `width` in 2..8 (causal_conv1d_fn has W = 4; causal_conv1d_cp, Parameters weight,
 *     takes [D, W]).  Read the formula above with W taps in the same order: z = b + sum over
 *     k of w[c][k]*u[t-(W-1)+k], tap W - 1 on the current token, and the history is W - 1
 *     values (u[-(W-1)] .. u[-1], oldest first).  The slot-pool forms (conv1d_fwd with a pool,
 *     conv1d_state_update*) are width four only.
 *     The optional bias is a contiguous [C] array of FP32 or bf16 (`b_dtype`), NULL for none
 *     (causal_conv1d_fn, Parameters weight and bias).
 *   - Host-checkable preconditions are validated before anything is enqueued; a violation
 *     returns CONV1D_EINVAL (or CONV1D_EWORKSPACE) and launches nothing.  Device-side values
 *     (offsets, sequence IDs, slot numbers) are the caller's constraint and are not checked:
 *     offsets must start at 0, be nondecreasing and end at most at `rows`; live slots must be
 *     unique and in [0, slots); sequence IDs must be non-negative (causal_conv1d_fn, Notes;
 *     causal_conv1d_cp, Parameters global_seq_idx).  Violating them gives unspecified results,
 *     but no access outside the buffers the host-side sizes describe: offsets are clamped to
 *     [0, rows], a slot outside [0, slots) acts as -1, accepted counts are clamped to the pool.
 *   - Sizes and strides whose products could exceed 2^56 elements (so that byte extents would
 *     overflow 64-bit arithmetic) are rejected with CONV1D_EINVAL.
 *   - Any C >= 1 and any row stride are accepted.  In the channel-last calls a lane's two
 *     channels move as one dword access whenever C >= 2 and the row bases are 2-byte aligned, at
 *     any row stride (an odd C or odd stride gives unaligned dwords, which the GPU serves), except
 *     that calls updating the slot pool in place also need an even C.  The channels-first calls
 *     move vectors when T and the strides are multiples of 8 and the bases 16-byte aligned.
 *     Otherwise an element-wise path runs.  Results are identical.
 *   - Two calls that run concurrently must not share live slots or workspaces.
 */
#ifndef CONV1D_H
#define CONV1D_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CONV1D_OK = 0,
  CONV1D_EINVAL = 1,      /* a host-checkable precondition failed; nothing was launched     */
  CONV1D_EWORKSPACE = 2,  /* workspace missing or smaller than the *_workspace_bytes query  */
  CONV1D_EUNSUPPORTED = 3,/* reserved; not returned by this version                         */
  CONV1D_EHIP = 4,        /* the HIP runtime reported a launch error                        */
  CONV1D_ETOOLARGE = 5    /* conv1d_bwd_noalloc: the problem needs more than the library's
                             scratch (CONV1D_NOALLOC_SCRATCH_BYTES); nothing was launched     */
} conv1d_status;

/* Size of the device scratch conv1d_bwd_noalloc keeps on every GPU it runs on. */
#define CONV1D_NOALLOC_SCRATCH_BYTES ((size_t)20 << 20)

typedef enum { CONV1D_BF16 = 0, CONV1D_F32 = 1 } conv1d_dtype;
typedef enum { CONV1D_ACT_NONE = 0, CONV1D_ACT_SILU = 1 } conv1d_act;

/* How the packed rows split into independent sequences; the convolution state resets at every
   sequence start.  Exactly one form is used:
   - cu_seqlens != NULL: int32 [nseq + 1] offsets, sequence i = rows [cu[i], cu[i+1]); rows at
     or after cu[nseq] belong to no sequence and are never written; empty sequences are allowed
     (causal_conv1d_fn, Parameters cu_seqlens).  seq_idx must be NULL.
   - seq_idx != NULL: int32 [rows] per-token sequence IDs (>= 0) inside batch rows of `seqlen`
     rows (rows % seqlen == 0); a sequence starts at every batch-row start and wherever the ID
     differs from the previous row's (causal_conv1d_cp, Parameters x and global_seq_idx).
   - both NULL: every batch row of `seqlen` rows is one sequence (rows % seqlen == 0). */
typedef struct {
  const int32_t* cu_seqlens;
  int64_t nseq;
  const int32_t* seq_idx;
  int64_t seqlen;
} conv1d_seq;

/* In-place bf16 state pool [slots, C, len] (causal_conv1d_fn, Parameters conv_state,
   cache_indices, has_initial_state).  Element (slot, c, j) is at
   ptr + slot*s_slot + c*s_chan + j*s_pos (strides in elements); either s_chan == 1 or
   s_pos == 1, and slots must not overlap.  History position j (j = 0, 1, 2) holds the raw
   input 3 - j rows before the sequence's first row (oldest first).
   cache_indices: int32 [nseq] slot of each sequence; -1 gives +0 output rows and no state
   access.  has_initial_state: uint8 [nseq] (NULL = all false); true reads positions 0..2 as
   the history, false starts from zeros.  After the call, positions 0..2 of the slot of every
   live nonempty sequence hold the last three values of its extended sequence u; positions
   >= 3, other slots and slots of empty sequences are unchanged.  Needs the cu_seqlens or the
   batch-row form (the host must know nseq). */
typedef struct {
  void* ptr;
  int64_t slots, len, s_slot, s_chan, s_pos;
  const int32_t* cache_indices;
  const uint8_t* has_initial_state;
} conv1d_pool;

/* Caller-supplied history rows for the context-parallel share of one GPU
   (flashinfer.cake_causal_conv1d_train.cake_causal_conv1d_kcp, summary: a fragment that
   continues a document reads the preceding fragment's rows instead of zeros).  ptr: contiguous
   bf16 [nseq, W - 1, C]; row j of entry i is the raw input W - 1 - j rows before sequence i's
   first row.  has_history: uint8 [nseq], NULL = every sequence reads its rows; sequences with 0 start
   from zeros.  Needs the cu_seqlens or the batch-row form. */
typedef struct {
  const void* ptr;
  const uint8_t* has_history;
} conv1d_hist;

/* Forward over packed rows (causal_conv1d_fn; causal_conv1d_cp; cake_causal_conv1d_kcp).
   x, y: bf16 [rows, C] with strides x_ld, y_ld.  seq: required.  pool, hist: optional
   (NULL), not both.  act: conv1d_act.  y must not overlap x, w, b, the pool or hist; rows of y
   outside every sequence are not written.  ws/ws_bytes: unused (0 bytes needed; may be NULL).
   Returns a conv1d_status. */
int conv1d_fwd(const void* x, int64_t rows, int64_t C, int64_t x_ld, const void* w, int w_dtype, int width,
               const void* b, int b_dtype, const conv1d_seq* seq, const conv1d_pool* pool,
               const conv1d_hist* hist, int act, void* y, int64_t y_ld, void* ws, size_t ws_bytes,
               hipStream_t stream);

/* One decode step per sequence (causal_conv1d_fn, Notes: the step after prefill).  x, y: bf16
   [nseq, C] (one new token per sequence).  For a live slot: y = act(b + w . [h0, h1, h2, x])
   with the slot's positions 0..2 as h, then positions 0..2 become [h1, h2, x]; slot -1 gives
   +0 and no state access.  Equal, bit for bit, to conv1d_fwd on unit-length sequences with
   has_initial_state all true.  pool is required (its has_initial_state field is ignored). */
int conv1d_state_update(const void* x, int64_t nseq, int64_t C, int64_t x_ld, const void* w,
                        int w_dtype, const void* b, int b_dtype, const conv1d_pool* pool, int act,
                        void* y, int64_t y_ld, hipStream_t stream);

/* Speculative multi-token update (causal_conv1d_fn, Notes: the first speculative update after
   a prefill uses accepted count 1).  Reading: each of nseq sequences feeds K tokens, and
   num_accepted[i] = a tells how many tokens of the previous update were kept, so the three raw
   history values sit at pool positions a-1, a, a+1 (a = 1 right after a prefill: positions
   0..2, where conv1d_fwd leaves them).  Token t of sequence i is row i*K + t of x and y (bf16,
   strides x_ld, y_ld): y = act(b + w . window) over the extended sequence [h0, h1, h2, x_1..x_K].
   Afterwards positions 0..K+1 of the slot hold its last K + 2 raw values, so whichever prefix a'
   of these K tokens the next update accepts finds its history at positions a'-1 .. a'+1;
   positions >= K + 2 are untouched.  Slot -1 gives +0 and no state access.  K = 1 with every
   a = 1 is conv1d_state_update.
   pool: required, len >= K + 2 (its has_initial_state field is ignored: the history is always
   read).  num_accepted: device int32 [nseq], or NULL for all 1; values must lie in [1, len - 2]
   (device data is never read on the host: values outside are clamped into that range).
   y must not overlap x, w, b, num_accepted or the pool.  Returns a conv1d_status. */
int conv1d_state_update_spec(const void* x, int64_t nseq, int64_t K, int64_t C, int64_t x_ld,
                             const void* w, int w_dtype, const void* b, int b_dtype,
                             const conv1d_pool* pool, const int32_t* num_accepted, int act, void* y,
                             int64_t y_ld, hipStream_t stream);

/* Training backward (cake_causal_conv1d_kcp, Returns: dx and a deterministic FP32 dweight;
   causal_conv1d_cp).  Given dy = dL/dy (bf16 [rows, C], stride dy_ld), recomputes the forward
   z and writes
     dx   bf16 [rows, C] (stride dx_ld): dL/dx, rows outside every sequence untouched;
     dw   FP32 [C, W]: dL/dw, contiguous (required);
     db   FP32 [C]: dL/db (NULL to skip; computed whether or not b is given);
     dhist bf16 [nseq, W - 1, C]: dL/d(history rows) for sequences that read history rows
          (requires hist; NULL to skip; rows of other sequences untouched).
   dtail: bf16 [W - 1, C] contiguous, or NULL.  The gradient the next shard sends back for the
   last W - 1 values of the LAST sequence's extended sequence [history rows, x rows] (the
   sequence that continues into the next shard: its d(history) output there; cake_causal_conv1d_kcp,
   Returns, and the differentiable history exchange of core.ssm.causal_conv1d,
   _exchange_initial_states).  Row j belongs to the value W - 1 - j positions before the end of
   that extended sequence: it is added in FP32, before the single bf16 rounding, to dx of that
   row, or to the sequence's d(history) row when the sequence is shorter than W - 1 rows (an
   empty last sequence passes dtail to its d(history) whole).  The last sequence is sequence
   nseq - 1 (cu_seqlens and batch-row forms) or the one holding row rows - 1 (per-token IDs).
   dw and db are sums of per-range FP32 partials combined in a fixed order by a second kernel
   (no atomics), so they are bitwise identical from run to run and independent of the
   workspace address.  ws: device scratch of at least conv1d_bwd_workspace_bytes(rows, C)
   bytes, 16-byte aligned, not overlapping any operand.  The query does not take the filter
   width: it reserves for width eight (one FP32 partial of 9 x C values per row range), which
   is 1.8 times what widths up to four use (5 x C).  No pool. */
int conv1d_bwd(const void* x, const void* dy, int64_t rows, int64_t C, int64_t x_ld, int64_t dy_ld,
               const void* w, int w_dtype, int width, const void* b, int b_dtype, const conv1d_seq* seq,
               const conv1d_hist* hist, int act, void* dx, int64_t dx_ld, float* dw, float* db,
               void* dhist, const void* dtail, void* ws, size_t ws_bytes, hipStream_t stream);

/* conv1d_bwd without a workspace argument, for callers that cannot allocate device memory (code
   under HIP graph capture, tight serving loops, harnesses that forbid allocation).  Same
   arguments, checks, kernels and results (bit for bit) as conv1d_bwd; the per-range FP32
   partials go to a scratch array the library holds on each GPU instead: a file-scope device
   array of CONV1D_NOALLOC_SCRATCH_BYTES (20 MiB), kept until the process ends; its address is
   looked up once per device, on the first call there.  The call itself allocates nothing.
   Limit: (number of row ranges) * (5 for widths up to four, 9 above) * C * 4 bytes must fit in
   the scratch; that holds for every C up to 524288 channels (and wider ones while the rows are
   few); larger problems return CONV1D_ETOOLARGE with nothing launched.  Every call on one GPU
   shares that GPU's scratch: calls that overlap in time on the same GPU (different streams,
   threads or graphs) race on it and must be serialized by the caller.  The scratch keeps the
   last call's partials; every call overwrites all the partials it reads, so nothing needs
   clearing. */
int conv1d_bwd_noalloc(const void* x, const void* dy, int64_t rows, int64_t C, int64_t x_ld, int64_t dy_ld,
                       const void* w, int w_dtype, int width, const void* b, int b_dtype, const conv1d_seq* seq,
                       const conv1d_hist* hist, int act, void* dx, int64_t dx_ld, float* dw, float* db,
                       void* dhist, const void* dtail, hipStream_t stream);

/* Shard-ordered combine of dweight / dbias contributions (core.ssm.causal_conv1d,
   assert_causal_conv1d_deterministic: deterministic reductions instead of atomics; the one-GPU
   share of gathering per-rank partials and adding them in rank order).  dw_parts: FP32
   [nshards, C, W] contiguous (each shard's dw from conv1d_bwd, stacked in shard order);
   db_parts: FP32 [nshards, C] or NULL.  Writes dw [C, W] and, when db is not NULL, db [C]:
   element e is ((p[0][e] + p[1][e]) + p[2][e]) + ... + p[nshards-1][e], one FP32 addition per
   shard in ascending shard order, so the bits depend only on the values and their order
   (one shard is copied bit for bit; nshards = 0 gives zeros).  Outputs must not overlap the
   inputs.  Returns a conv1d_status. */
int conv1d_bwd_combine(const float* dw_parts, const float* db_parts, int64_t nshards, int64_t C, int width,
                       float* dw, float* db, hipStream_t stream);

/* Channels-first layout [B, D, T], T contiguous (core.ssm.causal_conv1d,
   assert_causal_conv1d_deterministic names it: there a dweight element takes one contribution
   per batch row instead of batch * ceil(seqlen / 128)).  Every (b, d) row is one sequence with
   zero history; the operation is the same stencil (z = b, taps 0..W-1, tap W-1 on the current
   step, FP32, then act; taps [D, W], dw [D, W]).  Strides are in elements: row (b, d) starts at b * sb + d * sd; rows
   must not overlap (sd >= T, sb >= (D - 1) * sd + T).  x, y, dy, dx: bf16.  y / dx must not
   overlap any input.  Returns a conv1d_status. */
int conv1d_fwd_cf(const void* x, int64_t B, int64_t D, int64_t T, int64_t x_sb, int64_t x_sd, const void* w,
                  int w_dtype, int width, const void* b, int b_dtype, int act, void* y, int64_t y_sb, int64_t y_sd,
                  hipStream_t stream);

/* Channels-first backward: dx [B, D, T] bf16, dw FP32 [D, W] (required), db FP32 [D] (NULL to
   skip).  One FP32 partial per (batch row, channel) goes to ws, and a second kernel adds the B
   partials of each channel in a fixed order, so dw and db are bitwise reproducible.  ws: at least
   conv1d_bwd_cf_workspace_bytes(B, D) bytes, 16-byte aligned, not overlapping any operand. */
int conv1d_bwd_cf(const void* x, const void* dy, int64_t B, int64_t D, int64_t T, int64_t x_sb, int64_t x_sd,
                  int64_t dy_sb, int64_t dy_sd, const void* w, int w_dtype, int width, const void* b, int b_dtype,
                  int act, void* dx, int64_t dx_sb, int64_t dx_sd, float* dw, float* db, void* ws, size_t ws_bytes,
                  hipStream_t stream);

/* Workspace sizes in bytes (host-only, pure functions of the capacities). */
size_t conv1d_fwd_workspace_bytes(int64_t rows, int64_t C, int64_t nseq);
size_t conv1d_bwd_workspace_bytes(int64_t rows, int64_t C);
size_t conv1d_bwd_cf_workspace_bytes(int64_t B, int64_t D);

/* Static description of a status code. */
const char* conv1d_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* CONV1D_H */
