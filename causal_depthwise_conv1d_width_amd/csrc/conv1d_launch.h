// conv1d_launch.h -- library-internal launch parameters shared by the host entry points
// (conv1d_api.cpp) and the kernels.  Everything here is plain data: pointers are device
// pointers that the host has validated but never dereferences.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "conv1d.h"

namespace cconv {

// Tiling.  A block is kWavesPerBlock waves side by side in channels: lane = CPL channels, wave =
// 64*CPL channels, block = kBlockChannels channels (a strip) of some rows.  The forward gives a
// block one short tile of fwd_tile_rows() rows and launches many rounds of tiles.  The backward gives
// a block one row range streamed top to bottom, straight across sequence boundaries; the range
// length is chosen per launch (range_rows) so that one launch is about kBwdBlocks blocks: with 256
// CUs that is a single wave of resident blocks of equal work, and one [R + 1, C] FP32
// dweight/dbias partial per range in the workspace.
#ifndef CCONV_WAVES_PER_BLOCK
#define CCONV_WAVES_PER_BLOCK 4
#endif
#ifndef CCONV_BWD_BLOCKS
#define CCONV_BWD_BLOCKS 1024
#endif
#ifndef CCONV_CPL
#define CCONV_CPL 2
#endif
constexpr int kChannelsPerLane = CCONV_CPL;
constexpr int kWavesPerBlock = CCONV_WAVES_PER_BLOCK;
constexpr int kBlockThreads = 64 * kWavesPerBlock;
constexpr int kWaveChannels = 64 * kChannelsPerLane;
constexpr int kBlockChannels = kWavesPerBlock * kWaveChannels;
#ifndef CCONV_BWD_FIXED_ROWS
#define CCONV_BWD_FIXED_ROWS 0
#endif
constexpr int64_t kBwdBlocks = CCONV_BWD_BLOCKS;
constexpr int64_t kBwdFixedRows = CCONV_BWD_FIXED_ROWS;
#ifndef CCONV_RANGE_ALIGN
#define CCONV_RANGE_ALIGN 8
#endif
constexpr int64_t kRangeAlign = CCONV_RANGE_ALIGN;  // range lengths are multiples of this
constexpr int64_t kMinRangeRows = 8;                 // and at least this many rows

// Rows per range for `rows` rows of `n_strips` channel strips and a target block count.  A
// positive `fixed` length overrides the target (a build-time tuning knob).
//
// The dispatcher deals a one-round launch to the CUs in turn (blocks b, b + 256, b + 512, ...
// share a CU), and blocks on a CU that holds fewer of them stream faster.  Yet neither an
// exactly even split (16384 rows x 11 strips: 93 ranges of 177 rows) nor any fixed length from
// 48 to 232 rows beat floor(target / n_strips) ranges per strip rounded up to 8 rows (90 ranges
// of 184 rows there): the memory system as a whole, not the most loaded CU, sets the rate.
inline int64_t range_rows_for(int64_t rows, int64_t n_strips, int64_t target_blocks, int64_t fixed = 0) {
  if (fixed > 0) return fixed;
  int64_t per_strip = target_blocks / (n_strips > 0 ? n_strips : 1);
  if (per_strip < 1) per_strip = 1;
  int64_t r = (rows + per_strip - 1) / per_strip;
  r = (r + kRangeAlign - 1) / kRangeAlign * kRangeAlign;
  return r > kMinRangeRows ? r : kMinRangeRows;
}

// The forward's tile: fwd_tile_rows() rows of one strip per block, a launch of many rounds of them
// (measured on x [16384, 5632]: 16-row tiles 64.5 us, 32-row 65.4 us, 8-row 72 us, one round of
// long ranges 72.4 us).  A pool's tiles carry the slot lookup and state write-back: 24 rows
// (prefill 136 us against 148 us for 16).  Wider filters read W-1 rows above every tile: 24 rows
// (width 5 / 8: 65.3 / 67.4 us against 67.5 / 72.0 us for 16, the same as 32).
#ifndef CCONV_FWD_TILE_ROWS
#define CCONV_FWD_TILE_ROWS 16
#endif
#ifndef CCONV_FWD_TILE_ROWS_IDX
#define CCONV_FWD_TILE_ROWS_IDX 16
#endif
#ifndef CCONV_FWD_TILE_ROWS_POOL
#define CCONV_FWD_TILE_ROWS_POOL 24
#endif
#ifndef CCONV_FWD_TILE_ROWS_WIDE
#define CCONV_FWD_TILE_ROWS_WIDE 24
#endif
// rows per forward tile by sequence form (MODE_CU, MODE_IDX, MODE_BATCH), whether a pool is
// given, and the filter width
__host__ __device__ constexpr int fwd_tile_rows(int mode, bool pool, int width) {
  return pool ? CCONV_FWD_TILE_ROWS_POOL
              : (width > 4 ? CCONV_FWD_TILE_ROWS_WIDE : (mode == 1 ? CCONV_FWD_TILE_ROWS_IDX : CCONV_FWD_TILE_ROWS));
}

// Block -> tile order of a launch.  The dispatcher deals blocks to the 8 XCDs in turn (block b to
// XCD b mod 8), and each XCD has its own L2.
//   kOrderXcdRows:   each XCD takes one contiguous slice of the row-major tile space, a band of
//                    rows over every strip, so a tile and the one above it share an L2; the 8 XCDs
//                    stream 8 bands at once;
//   kOrderPlain:     tile = block in row-major order: the whole GPU streams one band of rows, and
//                    with a multiple of 8 strips every strip stays on one XCD;
//   kOrderXcdStrips: each XCD takes one contiguous slice of the strip-major tile space (a part of
//                    one strip, top to bottom): for 1, 2 or 4 strips.
// Copies of the forward's tile shape (16 rows, 1 read 1 write, TB/s) by strip count:
//   strips  rows-order  plain  strips-order
//      4       5.02     5.31      5.54
//      8       5.63     6.18      6.22
//     11       6.00     5.95      5.44
//     12       6.09     5.99      5.92
//     16       6.33     6.58      6.65
// With 8 bands of rows at a power-of-two row pitch, the bands sit a power of two apart and the XCDs
// meet in the same memory channels.
enum : uint32_t { kOrderXcdRows = 0, kOrderPlain = 1, kOrderXcdStrips = 2 };
#ifndef CCONV_FWD_ORDER
#define CCONV_FWD_ORDER -1
#endif
#ifndef CCONV_BWD_ORDER
#define CCONV_BWD_ORDER -1
#endif
inline uint32_t fwd_tile_order(int64_t n_strips) {
  if (CCONV_FWD_ORDER >= 0) return (uint32_t)CCONV_FWD_ORDER;
  if (n_strips % 8 == 0) return kOrderPlain;
  if (8 % n_strips == 0) return kOrderXcdStrips;
  return kOrderXcdRows;
}
// The backward's one round of long row ranges has every range in flight at once, so the order only
// decides which L2 a range and its neighbours share.  Copies of that shape (2 reads, 1 write, TB/s,
// rows order / plain) by strip count: 4: 5.28 / 4.82, 6: 5.13 / 5.09, 7: 5.17 / 5.03,
// 8: 5.77 / 5.39, 9: 5.15 / 5.35, 10: 5.29 / 5.26, 11: 5.32 / 5.50, 12: 5.11 / 4.87,
// 13: 5.29 / 5.17, 15: 5.12 / 5.06, 16: 5.54 / 4.82.  No rule beats rows order across them.
inline uint32_t bwd_tile_order(int64_t n_strips) {
  if (CCONV_BWD_ORDER >= 0) return (uint32_t)CCONV_BWD_ORDER;
  (void)n_strips;
  return kOrderXcdRows;
}

// Rows of one range's dweight/dbias partial: a tap slot per register-ring slot (4 up to filter
// width four, 8 up to width eight; the first R - W are padding), then dbias.
constexpr int kMaxWidth = 8;
__host__ __device__ inline int partial_rows(int width) { return width <= 4 ? 5 : 9; }

// How rows split into sequences: cu_seqlens offsets, per-token sequence IDs, or batch rows.
enum { MODE_CU = 0, MODE_IDX = 1, MODE_BATCH = 2 };

struct SeqArgs {
  const int32_t* cu;       // [nseq + 1] or nullptr
  int64_t nseq;            // number of sequences (cu form or batch-row form)
  const int32_t* seq_idx;  // [rows] or nullptr
  int64_t seqlen;          // batch-row length (IDX / BATCH forms)
};

struct PoolArgs {
  uint16_t* ptr;  // nullptr: no pool
  int64_t slots, len, s_slot, s_chan, s_pos;
  const int32_t* cache_indices;
  const uint8_t* has_init;
};

struct HistArgs {
  const uint16_t* ptr;  // nullptr: no history rows; else contiguous [nseq, W-1, C]
  const uint8_t* has_hist;
};

struct FwdArgs {
  const uint16_t* x;
  uint16_t* y;
  int64_t x_ld, y_ld, rows, C;
  const void* w;  // [C, width]
  const void* b;
  int w_f32, b_f32, width;
  SeqArgs seq;
  PoolArgs pool;  // width 4 only
  HistArgs hist;
  int64_t range_rows;  // rows per row range
  uint32_t n_strips, n_rowblocks;
  uint32_t tile_order;  // kOrder*
};

struct DecodeArgs {
  const uint16_t* x;  // token t of sequence i is row i*K + t
  uint16_t* y;
  int64_t x_ld, y_ld, nseq, K, C;
  const void* w;
  const void* b;
  int w_f32, b_f32;
  PoolArgs pool;            // pool.len >= K + 2
  const int32_t* accepted;  // [nseq] or nullptr (all 1): history at positions a-1 .. a+1
};

struct BwdArgs {
  const uint16_t* x;
  const uint16_t* dy;
  uint16_t* dx;
  int64_t x_ld, dy_ld, dx_ld, rows, C;
  const void* w;  // [C, width]
  const void* b;
  int w_f32, b_f32, width;
  SeqArgs seq;
  HistArgs hist;
  uint16_t* dhist;  // nullptr: not requested
  const uint16_t* dtail;  // nullptr, or bf16 [width-1, C]: the next shard's gradient of the last
                          // width-1 values of the last sequence's extended sequence
  float* part;      // workspace: [n_rowblocks, partial_rows(width), C] FP32 per-block partials
  float* dw;        // [C, width]
  float* db;        // [C] or nullptr
  int64_t range_rows;  // rows per row range
  uint32_t n_strips, n_rowblocks;
  uint32_t tile_order;  // kOrder*
};

// Channels-first [B, D, T] (T contiguous): every (b, d) row is one sequence with zero history.
// Forward: y = act(conv(x)).  Backward: dx, and one FP32 [5, D] dweight/dbias partial per batch
// row in `part` ([B, 5, D]), combined by the ordered reduce.
struct CfArgs {
  const uint16_t* x;
  const uint16_t* dy;  // backward only
  uint16_t* out;       // forward: y; backward: dx
  int64_t B, D, T;
  int64_t x_sb, x_sd, dy_sb, dy_sd, o_sb, o_sd;
  const void* w;  // [D, width]
  const void* b;
  int w_f32, b_f32, width;
  float* part;  // backward only
};

// Shard-ordered combine: out[e] = ((p[0][e] + p[1][e]) + ...) + p[n-1][e] in FP32, for the
// dweight [C, width] and dbias [C] contributions of n shards stacked shard-major.
struct CombineArgs {
  const float* dw_parts;  // [nshards, C * width]
  const float* db_parts;  // [nshards, C] or nullptr
  float* dw;              // [C * width]
  float* db;              // [C] or nullptr
  int64_t nshards, C;
  int width;
};

// Launchers (return hipError_t of the launch).  mode: 0 = cu_seqlens, 1 = seq_idx, 2 = batch rows.
hipError_t launch_fwd(const FwdArgs& a, int mode, bool vec, bool silu, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, bool vec, bool silu, hipStream_t stream);
hipError_t launch_bwd(const BwdArgs& a, int mode, bool vec, bool silu, hipStream_t stream);
// the ordered reduce alone: dw / db from a.part over a.n_rowblocks partials of a.C channels
hipError_t launch_reduce(const BwdArgs& a, hipStream_t stream);
hipError_t launch_fwd_cf(const CfArgs& a, bool vec, bool silu, hipStream_t stream);
hipError_t launch_bwd_cf(const CfArgs& a, bool vec, bool silu, hipStream_t stream);
hipError_t launch_combine(const CombineArgs& a, hipStream_t stream);

// The library-held backward scratch of conv1d_bwd_noalloc (kScratchBytes on every GPU it runs
// on): its device address on the GPU of `stream`, looked up once per device.
constexpr size_t kScratchBytes = CONV1D_NOALLOC_SCRATCH_BYTES;
hipError_t bwd_scratch(hipStream_t stream, void** ptr);

}  // namespace cconv
