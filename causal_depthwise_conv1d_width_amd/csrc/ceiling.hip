// ceiling.hip -- copy kernels that bound what the convolution kernels can stream (a measurement
// aid for the benchmark; not part of the convolution's C ABI in include/conv1d.h).
//
// Each copy moves the bytes a convolution call moves, in one of two access structures:
//   contiguous: a grid-stride sweep of 16-byte vectors over the flat array (1024 blocks);
//   tiles:      the forward's structure: short tiles of `tile_rows` rows x 512 channels, one per
//               block, in the forward's tile order, every lane 4 bytes of a row, the 3 rows above
//               a tile read as well;
//   ranges:     the backward's structure: about 1024 blocks in one round, each streaming one row
//               range of 512 channels in chunks of 4 or 8 rows (the next chunk's loads issued
//               before this chunk's stores), the 3 rows above and below a range read as well.
// With two sources, dst = a ^ b (a backward reads x and dy and writes dx).  Rows are [rows, C]
// bf16 with C a multiple of 8, row stride C.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t xcd_slice(uint32_t b, uint32_t nb) {
  constexpr uint32_t X = 8;  // XCDs: blocks are dealt to them round-robin
  const uint32_t q = nb / X, r = nb % X, xcd = b % X, idx = b / X;
  return (xcd < r) ? xcd * (q + 1) + idx : r * (q + 1) + (xcd - r) * q + idx;
}

struct CopyArgs {
  const uint16_t* a;
  const uint16_t* b;  // second source or nullptr
  uint16_t* dst;
  int64_t rows, C, tile_rows;
  uint32_t n_strips;
};

// The source count is a template constant: a runtime test around the second load puts it in a
// branch of its own, and the wait for it then lands right behind it (no loads left in flight).
template <bool TWO>
__global__ void __launch_bounds__(256) copy_contiguous(const CopyArgs p) {
  const int64_t n = p.rows * p.C / 8;
  const u32x4* a = reinterpret_cast<const u32x4*>(p.a);
  const u32x4* b = reinterpret_cast<const u32x4*>(p.b);
  u32x4* d = reinterpret_cast<u32x4*>(p.dst);
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    u32x4 v = __builtin_nontemporal_load(a + i);
    if constexpr (TWO) v ^= __builtin_nontemporal_load(b + i);
    __builtin_nontemporal_store(v, d + i);
  }
}

// Tile order as the forward's: plain row-major order for a multiple of 8 strips, XCD slices of
// the strip-major order for 1, 2 or 4 strips, XCD slices of the row-major order otherwise.
template <int R>
__global__ void __launch_bounds__(256) copy_tiles(const CopyArgs p) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t nrb = gridDim.x / p.n_strips;
  uint32_t strip, rb;
  if (p.n_strips % 8 == 0) {
    strip = blockIdx.x % p.n_strips;
    rb = blockIdx.x / p.n_strips;
  } else if (8 % p.n_strips == 0) {
    const uint32_t t = xcd_slice(blockIdx.x, gridDim.x);
    strip = t / nrb;
    rb = t % nrb;
  } else {
    const uint32_t t = xcd_slice(blockIdx.x, gridDim.x);
    strip = t % p.n_strips;
    rb = t / p.n_strips;
  }
  const int64_t c0 = (int64_t)strip * 512 + wave * 128 + lane * 2;
  if (c0 >= p.C) return;
  const int64_t ta = (int64_t)rb * R;
  uint32_t halo = 0;
  for (int j = 1; j <= 3; ++j)
    if (ta - j >= 0) halo ^= *reinterpret_cast<const uint32_t*>(p.a + (ta - j) * p.C + c0);
  uint32_t v[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t q = ta + r < p.rows ? ta + r : p.rows - 1;
    v[r] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p.a + q * p.C + c0));
  }
#pragma unroll
  for (int r = 0; r < R; ++r)
    if (ta + r < p.rows)  // the halo feeds every value (never actually changing it)
      __builtin_nontemporal_store(v[r] ^ (uint32_t)(halo == 0x9e3779b9u), reinterpret_cast<uint32_t*>(p.dst + (ta + r) * p.C + c0));
}

template <bool TWO>
__device__ __forceinline__ uint32_t ld2(const CopyArgs& p, int64_t q, int64_t c0) {
  uint32_t v = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p.a + q * p.C + c0));
  if constexpr (TWO) v ^= __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p.b + q * p.C + c0));
  return v;
}

template <bool TWO, int CH>
__global__ void __launch_bounds__(256) copy_ranges(const CopyArgs p) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t t = xcd_slice(blockIdx.x, gridDim.x);
  const uint32_t strip = t % p.n_strips, rb = t / p.n_strips;
  const int64_t c0 = (int64_t)strip * 512 + wave * 128 + lane * 2;
  if (c0 >= p.C) return;
  int64_t ta = (int64_t)rb * p.tile_rows, tb = ta + p.tile_rows;
  ta = ta < p.rows ? ta : p.rows;
  tb = tb < p.rows ? tb : p.rows;
  uint32_t halo = 0;
  for (int j = 1; j <= 3; ++j) {
    if (ta - j >= 0) halo ^= *reinterpret_cast<const uint32_t*>(p.a + (ta - j) * p.C + c0);
    if (tb + j - 1 < p.rows) halo ^= ld2<TWO>(p, tb + j - 1, c0);
  }
  const int64_t nfull = (tb - ta) / CH;
  uint32_t A[CH], B[CH];
  int64_t q = ta;
  if (nfull > 0) {
#pragma unroll
    for (int r = 0; r < CH; ++r) A[r] = ld2<TWO>(p, q + r, c0);
  }
  const uint32_t h = (uint32_t)(halo == 0x9e3779b9u);
  for (int64_t k = 0; k < nfull; k += 2) {
    const int64_t qn = k + 1 < nfull ? q + CH : q;
#pragma unroll
    for (int r = 0; r < CH; ++r) B[r] = ld2<TWO>(p, qn + r, c0);
#pragma unroll
    for (int r = 0; r < CH; ++r) __builtin_nontemporal_store(A[r] ^ h, reinterpret_cast<uint32_t*>(p.dst + (q + r) * p.C + c0));
    q += CH;
    if (k + 1 >= nfull) break;
    const int64_t qn2 = k + 2 < nfull ? q + CH : q;
#pragma unroll
    for (int r = 0; r < CH; ++r) A[r] = ld2<TWO>(p, qn2 + r, c0);
#pragma unroll
    for (int r = 0; r < CH; ++r) __builtin_nontemporal_store(B[r] ^ h, reinterpret_cast<uint32_t*>(p.dst + (q + r) * p.C + c0));
    q += CH;
  }
  for (; q < tb; ++q) *reinterpret_cast<uint32_t*>(p.dst + q * p.C + c0) = ld2<TWO>(p, q, c0) ^ h;
}

// The ranges copy with its two read streams fetched by gfx950's direct-to-LDS 16-byte loads: one
// instruction moves 4 rows x 256 B of a wave's 128 channels (lane l: row l / 16, bytes 16 (l % 16)
// of it) into the wave's own LDS, so a 4-row chunk takes 2 load instructions instead of 8 and a
// chunk in flight holds no registers; D chunk slots per wave.  Each lane then reads its 2 channels
// of every row from LDS and stores them with one 4-byte store per row.  Only the wave itself reads
// its LDS slots, so no barrier is needed; the wait for a slot is an explicit vmcnt (the compiler
// does not order LDS reads after these loads): the D - 1 load pairs and (D - 1) x 4 stores issued
// after a chunk's loads may still be in flight when it is read.  Whole waves only (C % 128 == 0).
#define CEILING_WAIT_VM(n) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(n) : "memory")
typedef __attribute__((address_space(3))) void lds_void;

template <int D>
__global__ void __launch_bounds__(256) copy_ranges_lds(const CopyArgs p) {
  __shared__ __attribute__((aligned(16))) uint32_t slots[4][D][2][256];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t t = xcd_slice(blockIdx.x, gridDim.x);
  const uint32_t strip = t % p.n_strips, rb = t / p.n_strips;
  const int64_t wch = (int64_t)strip * 512 + wave * 128;
  if (wch >= p.C) return;
  const int64_t c0 = wch + lane * 2;
  int64_t ta = (int64_t)rb * p.tile_rows, tb = ta + p.tile_rows;
  ta = ta < p.rows ? ta : p.rows;
  tb = tb < p.rows ? tb : p.rows;
  uint32_t halo = 0;
  for (int j = 1; j <= 3; ++j) {
    if (ta - j >= 0) halo ^= *reinterpret_cast<const uint32_t*>(p.a + (ta - j) * p.C + c0);
    if (tb + j - 1 < p.rows) halo ^= ld2<true>(p, tb + j - 1, c0);
  }
  const uint32_t h = (uint32_t)(halo == 0x9e3779b9u);
  const int nfull = (int)((tb - ta) / 4);
  const uint16_t* xa = p.a + wch + (lane & 15) * 8;
  const uint16_t* ga = p.b + wch + (lane & 15) * 8;
  auto issue = [&](int c, int slot) {  // chunk c (rows ta + 4c ..) into a slot
    const int64_t q = ta + 4 * (int64_t)c + (lane >> 4);
    __builtin_amdgcn_global_load_lds(static_cast<const void*>(xa + q * p.C), (lds_void*)&slots[wave][slot][0][0], 16, 0, 0);
    __builtin_amdgcn_global_load_lds(static_cast<const void*>(ga + q * p.C), (lds_void*)&slots[wave][slot][1][0], 16, 0, 0);
  };
  if (nfull > 0) {
#pragma unroll
    for (int s = 0; s < D - 1; ++s) issue(s < nfull ? s : nfull - 1, s);
    for (int k = 0; k < nfull; ++k) {
      const int c = k + D - 1;  // past the last chunk: re-read it into the slot just consumed
      issue(c < nfull ? c : nfull - 1, c % D);
      if (k < D - 1)
        CEILING_WAIT_VM(2 * (D - 1));  // no stores yet behind this chunk's loads
      else
        CEILING_WAIT_VM((D - 1) * (2 + 4));
      const int slot = k % D;
      const int64_t q = ta + 4 * (int64_t)k;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        __builtin_nontemporal_store(slots[wave][slot][0][r * 64 + lane] ^ slots[wave][slot][1][r * 64 + lane] ^ h,
                                    reinterpret_cast<uint32_t*>(p.dst + (q + r) * p.C + c0));
    }
    CEILING_WAIT_VM(0);  // no load may still write this block's LDS when the wave ends
  }
  for (int64_t q = ta + 4 * (int64_t)nfull; q < tb; ++q)
    *reinterpret_cast<uint32_t*>(p.dst + q * p.C + c0) = ld2<true>(p, q, c0) ^ h;
}

}  // namespace

extern "C" {

// shape: 0 contiguous, 1 tiles of `tile_rows` (16 or 24) rows, 2 one round of row ranges streamed
// in chunks of `tile_rows` (4 or 8) rows, 3 the same ranges through direct-to-LDS loads (two
// sources, C % 128 == 0; tile_rows ignored).
// b: second source (nullptr for one).  Returns a hipError_t; -1 for sizes it does not take.
int ceiling_copy(const void* a, const void* b, void* dst, int64_t rows, int64_t C, int shape, int64_t tile_rows,
                 hipStream_t stream) {
  if (rows < 1 || C < 8 || C % 8 != 0 || !a || !dst) return -1;
  CopyArgs p{static_cast<const uint16_t*>(a), static_cast<const uint16_t*>(b), static_cast<uint16_t*>(dst), rows, C,
             tile_rows, (uint32_t)((C + 511) / 512)};
  void* args[] = {&p};
  const bool two = b != nullptr;
  if (shape == 0)
    return hipLaunchKernel(two ? reinterpret_cast<const void*>(&copy_contiguous<true>)
                               : reinterpret_cast<const void*>(&copy_contiguous<false>),
                           dim3(1024), dim3(256), args, 0, stream);
  if (shape == 1) {
    if (tile_rows != 16 && tile_rows != 24) return -1;
    const uint32_t blocks = p.n_strips * (uint32_t)((rows + tile_rows - 1) / tile_rows);
    const void* k = tile_rows == 16 ? reinterpret_cast<const void*>(&copy_tiles<16>)
                                    : reinterpret_cast<const void*>(&copy_tiles<24>);
    return hipLaunchKernel(k, dim3(blocks), dim3(256), args, 0, stream);
  }
  // ranges: floor(1024 / strips) ranges per strip, lengths rounded up to 8 rows (as the backward)
  if (shape == 3 ? (!two || C % 128 != 0) : (shape != 2 || (tile_rows != 4 && tile_rows != 8))) return -1;
  const int ch = (int)tile_rows;
  int64_t per = 1024 / p.n_strips;
  per = per < 1 ? 1 : per;
  int64_t rr = (rows + per - 1) / per;
  rr = (rr + 7) / 8 * 8;
  p.tile_rows = rr;
  const uint32_t blocks = p.n_strips * (uint32_t)((rows + rr - 1) / rr);
  const void* k = shape == 3 ? reinterpret_cast<const void*>(&copy_ranges_lds<4>)
                  : two ? (ch == 4 ? reinterpret_cast<const void*>(&copy_ranges<true, 4>)
                                 : reinterpret_cast<const void*>(&copy_ranges<true, 8>))
                      : (ch == 4 ? reinterpret_cast<const void*>(&copy_ranges<false, 4>)
                                 : reinterpret_cast<const void*>(&copy_ranges<false, 8>));
  return hipLaunchKernel(k, dim3(blocks), dim3(256), args, 0, stream);
}

}  // extern "C"
