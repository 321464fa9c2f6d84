// The bf16 MFMA tile core shared by the fused projection and the embedding front end's two
// convolutions (each a matrix product once its inputs are laid out as rows).
//
// One workgroup (8 waves) forms a tile of Y^T = W X^T: 256 rows of W ("features", K
// contiguous) against 32 TW * 4 rows of X ("tokens"), TW = 2 for a full 256-token tile and
// 1 for a 128-token half tile.  v_mfma_f32_32x32x16_bf16 with A = 32 W rows and B = 32 X
// rows; wave w owns features 128 (w / 4) .. +127 and tokens 32 TW (w % 4) .. +32 TW - 1 as
// TW x 4 accumulators of 32 x 32.  In that layout accumulator [ti][fi], element r holds
// feature 32 fi + row_of(r) and token 32 ti + col, with row_of(r) = 8 (r / 4) + 4 hl + r % 4
// (col = lane % 32, hl = lane / 32): a lane holds one token and half of every 32-feature
// block, in runs of four consecutive features.
//
// K streams through LDS in stages of 64 (128-byte rows), two stages of 32 KB W + 32 KB X.
// Tiles go from HBM/L2 straight into LDS (buffer loads with the LDS destination); the lane
// that fills (row r, 16-byte slot p) fetches chunk p ^ pswz(r) of that row, so the fragment
// reads (16 consecutive rows at one chunk) cover all 64 banks.  One barrier per stage; the
// next stage's loads are in flight during the current stage's products.
//
// X rows need not be contiguous: the caller gives each tile row's byte offset in its buffer
// (or an offset past the buffer's end for rows that must read as zero) and the per-stage
// offset added to all rows, which lets a convolution gather its input windows directly.
#pragma once

#include "neo_internal.h"

#include <type_traits>

namespace neo {
namespace gemm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = kGemmThreads;  // 8 waves, two per SIMD
constexpr int kFT = 256;               // features per tile
constexpr int kTT = 256;               // tokens per full tile
constexpr int kGroup = 4;              // token tiles per group of the tile order
constexpr int kKS = 64;                // K per stage
constexpr int kRowB = kKS * 2;         // one LDS tile row: 128 bytes = 8 chunks
constexpr int kWTileB = kFT * kRowB;   // 32 KB
constexpr int kXTileB = kTT * kRowB;   // 32 KB
constexpr int kBufFlags = 0x00020000;  // raw buffer, 32-bit data format (gfx9 family)
constexpr uint32_t kAbsentRow = 0x80000000u;  // row offset past any buffer: reads zeros

// Chunk c of LDS row r sits in slot c ^ pswz(r): 16 consecutive rows read at one chunk then
// cover all 64 banks (rows 128 bytes apart pair up per 256 bytes; the XOR spreads each
// pair's eight rows over the eight slots).
__device__ __forceinline__ int pswz(int r) { return (r >> 1) & 7; }

// The descriptor's fields are workgroup-uniform; passing them through readfirstlane keeps
// them in scalar registers (the compiler otherwise may keep them in vector registers and
// wrap every load in a loop over distinct descriptor values).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t nbytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
  void* up = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(up, (short)0, (int)__builtin_amdgcn_readfirstlane(nbytes),
                                           kBufFlags);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

// accumulator element r's feature row inside its 32-feature block
__device__ __forceinline__ int row_of(int r, int hl) { return (r >> 2) * 8 + 4 * hl + (r & 3); }

// ---- tile order ------------------------------------------------------------------------
// n_ftiles x n_ttiles tiles.  Whole rounds over the CUs run as full tiles; the surplus
// tiles run as two 128-token halves each, so the last round is as long as the others.
// Tile ids run over groups of kGroup token tiles (token tile fastest) and each XCD takes
// consecutive ids, so the 32 tiles an XCD holds at once form a 4 x 8 block sharing its
// x and W rows in L2.
struct Plan {
  int n_ftiles, n_ttiles, n_full, n_half;
};

struct Tile {
  int f0, t0;
  bool full;
};

__device__ __forceinline__ Tile tile_of(uint32_t b, const Plan& p) {
  auto decode = [&](uint32_t id, int& ft, int& tt) __attribute__((always_inline)) {
    const uint32_t per = (uint32_t)(kGroup * p.n_ftiles), g = id / per, r = id % per;
    const int first = (int)g * kGroup;
    const int gs = p.n_ttiles - first < kGroup ? p.n_ttiles - first : kGroup;
    ft = (int)(r / (uint32_t)gs);
    tt = first + (int)(r % (uint32_t)gs);
  };
  int ft, tt;
  if (b < (uint32_t)p.n_full) {
    decode(xcd_remap(b, (uint32_t)p.n_full), ft, tt);
    return Tile{ft * kFT, tt * kTT, true};
  }
  const uint32_t h = xcd_remap(b - (uint32_t)p.n_full, (uint32_t)p.n_half);
  decode((uint32_t)p.n_full + h / 2, ft, tt);
  return Tile{ft * kFT, tt * kTT + 128 * (int)(h & 1), false};
}

// Host side: the plan and the grid (n_full + n_half workgroups of kThreads) for F features
// by T tokens.  The CU count comes from the current device (256 if it cannot be read).
inline Plan make_plan(int64_t F, int64_t T) {
  const int64_t n_ftiles = (F + kFT - 1) / kFT;
  const int64_t n_ttiles = (T + kTT - 1) / kTT;
  const int64_t n_tiles = n_ftiles * n_ttiles;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    cus = 256;
  const int64_t surplus = n_tiles >= cus ? n_tiles % cus : 0;
  return Plan{(int)n_ftiles, (int)n_ttiles, (int)(n_tiles - surplus), (int)(2 * surplus)};
}

static_assert(kFT == 256 && kTT == 256, "gemm_max_blocks assumes 256 x 256 tiles");

// ---- the main loop ---------------------------------------------------------------------
// acc (zeroed here) receives this wave's TW x 4 accumulators of the tile.
//   rw          W rows of this tile (row r at r * w_row_bytes), resource bounded by the rows
//               that exist, so missing feature rows read as zeros;
//   rx, xrow    X resource and xrow(r): byte offset of tile row r (r < 128 TW), or
//               kAbsentRow for rows that must read as zeros;
//   xk          xk(s): byte offset added to every X row for stage s (K [64 s, 64 s + 64));
//   S           number of stages (K / 64); kEvenS promises that S is even, which lets the
//               loop drop its mid-trip exit (the merge convolution's S = 4 C1 / 64 needs
//               this to stay within the register file).
// The LDS buffers are four separate objects of the caller (two stages of W and of X), so
// the compiler sees that a stage load cannot alias the fragment reads of the other stage.
template <int TW, bool kEvenS = false, class XRow, class XK>
__device__ __forceinline__ void mainloop(f32x16 (&acc)[TW][4], __amdgpu_buffer_rsrc_t rw,
                                         uint32_t w_row_bytes, __amdgpu_buffer_rsrc_t rx,
                                         XRow xrow, XK xk, int S, uint8_t* lw0, uint8_t* lw1,
                                         uint8_t* lx0, uint8_t* lx1) {
  auto wbuf = [&](int b) __attribute__((always_inline)) -> uint8_t* { return b == 0 ? lw0 : lw1; };
  auto xbuf = [&](int b) __attribute__((always_inline)) -> uint8_t* { return b == 0 ? lx0 : lx1; };
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, hl = lane >> 5, col = lane & 31;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int hh = wave >> 2, tg = wave & 3;

  // staging: a tile is a run of 1 KB blocks of 8 rows; lane L of a block lands in row
  // 8*blk + L/8, slot L%8, and so fetches chunk (L%8) ^ pswz(row) of that row.  Wave w loads
  // W blocks 4w .. 4w+3 and X blocks 2 TW w .. 2 TW w + 2 TW - 1.
  int wofs[4];
  uint32_t xofs[2 * TW];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 8 * (4 * wave + i) + (lane >> 3);
    wofs[i] = row * (int)w_row_bytes + (((lane & 7) ^ pswz(row)) << 4);
  }
#pragma unroll
  for (int i = 0; i < 2 * TW; ++i) {
    const int row = 8 * (2 * TW * wave + i) + (lane >> 3);
    xofs[i] = xrow(row) + (uint32_t)(((lane & 7) ^ pswz(row)) << 4);
  }
  auto load_stage = [&](int s, int b) __attribute__((always_inline)) {
    const int koff = s * kRowB;
    const uint32_t xoff = xk(s);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rw, (__attribute__((address_space(3))) void*)(wbuf(b) + (4 * wave_u + i) * 1024), 16,
          wofs[i] + koff, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 2 * TW; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rx, (__attribute__((address_space(3))) void*)(xbuf(b) + (2 * TW * wave_u + i) * 1024), 16,
          (int)(xofs[i] + xoff), 0, 0, 0);
  };

  // fragment reads: W row 128 hh + 32 fi + col and X row 32 TW tg + 32 ti + col, chunk
  // 2 kk + hl.  The swizzle depends on the row's bits 1..3 only, which those multiples of
  // 32 leave alone.
  int ofs[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) ofs[kk] = col * kRowB + (((2 * kk + hl) ^ pswz(col)) << 4);
  const int wrow0 = hh * 128 * kRowB, xrow0 = tg * 32 * TW * kRowB;

#pragma unroll
  for (int ti = 0; ti < TW; ++ti)
#pragma unroll
    for (int fi = 0; fi < 4; ++fi)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[ti][fi][r] = 0.0f;

  load_stage(0, 0);
  __syncthreads();

  // stage s lives in buffer s % 2 (a compile-time constant at every call site) while
  // stage s + 1 loads into the other; fragments are read one k-step ahead of their MFMAs
  auto stage = [&](int s, auto s2) __attribute__((always_inline)) {
    constexpr int B = decltype(s2)::value;
    if (s + 1 < S) load_stage(s + 1, B ^ 1);
    const uint8_t* wb = wbuf(B) + wrow0;
    const uint8_t* xb = xbuf(B) + xrow0;
    bf16x8 af[2][4], bf[2][TW];
    auto fetch = [&](int kk, int slot) __attribute__((always_inline)) {
#pragma unroll
      for (int ti = 0; ti < TW; ++ti)
        bf[slot][ti] = as_bf16x8(*reinterpret_cast<const uint4*>(xb + ti * 32 * kRowB + ofs[kk]));
#pragma unroll
      for (int fi = 0; fi < 4; ++fi)
        af[slot][fi] = as_bf16x8(*reinterpret_cast<const uint4*>(wb + fi * 32 * kRowB + ofs[kk]));
    };
    fetch(0, 0);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      if (kk + 1 < 4) fetch(kk + 1, (kk + 1) & 1);
#pragma unroll
      for (int ti = 0; ti < TW; ++ti)
#pragma unroll
        for (int fi = 0; fi < 4; ++fi)
          acc[ti][fi] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[kk & 1][fi], bf[kk & 1][ti],
                                                                acc[ti][fi], 0, 0, 0);
    }
    __syncthreads();
  };
  using C0 = std::integral_constant<int, 0>;
  using C1 = std::integral_constant<int, 1>;
  for (int s = 0; s < S; s += 2) {
    stage(s, C0{});
    if (!kEvenS && s + 1 >= S) break;
    stage(s + 1, C1{});
  }
}

// ---- the main loop with X built in registers ---------------------------------------------
// For an X that is not stored as bf16 rows (the patch convolution reads fp32 pixels): the
// caller's xload(s, xr) issues this thread's global loads of stage s into xr (kXR 16-byte
// registers), and xstore(xbuf, xr) converts them and writes them into an X tile buffer in
// the layout the fragment reads expect (row r, 16-byte chunk c in slot c ^ pswz(r)).  W rows
// arrive by LDS-direct loads as in mainloop.  Stage s + 1's X is loaded into registers
// during stage s - 1 and written to LDS during stage s, after the first k-step's products,
// into the buffer every wave finished reading at the barrier before; the products are
// those of mainloop, in the same order, so the sums are bit-identical to mainloop's on the
// same bf16 rows.
template <int TW, int kXR, class XLoad, class XStore>
__device__ __forceinline__ void mainloop_xreg(f32x16 (&acc)[TW][4], __amdgpu_buffer_rsrc_t rw,
                                              uint32_t w_row_bytes, XLoad xload, XStore xstore,
                                              int S, uint8_t* lw0, uint8_t* lw1, uint8_t* lx0,
                                              uint8_t* lx1) {
  auto wbuf = [&](int b) __attribute__((always_inline)) -> uint8_t* { return b == 0 ? lw0 : lw1; };
  auto xbuf = [&](int b) __attribute__((always_inline)) -> uint8_t* { return b == 0 ? lx0 : lx1; };
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, hl = lane >> 5, col = lane & 31;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int hh = wave >> 2, tg = wave & 3;

  // W staging as in mainloop: wave w loads W blocks 4w .. 4w+3
  int wofs[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 8 * (4 * wave + i) + (lane >> 3);
    wofs[i] = row * (int)w_row_bytes + (((lane & 7) ^ pswz(row)) << 4);
  }
  auto load_w = [&](int s, int b) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rw, (__attribute__((address_space(3))) void*)(wbuf(b) + (4 * wave_u + i) * 1024), 16,
          wofs[i] + s * kRowB, 0, 0, 0);
  };

  int ofs[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) ofs[kk] = col * kRowB + (((2 * kk + hl) ^ pswz(col)) << 4);
  const int wrow0 = hh * 128 * kRowB, xrow0 = tg * 32 * TW * kRowB;

#pragma unroll
  for (int ti = 0; ti < TW; ++ti)
#pragma unroll
    for (int fi = 0; fi < 4; ++fi)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[ti][fi][r] = 0.0f;

  uint4 xr[kXR];
  load_w(0, 0);
  xload(0, xr);
  xstore(xbuf(0), xr);
  if (1 < S) xload(1, xr);
  __syncthreads();

  auto stage = [&](int s, auto s2) __attribute__((always_inline)) {
    constexpr int B = decltype(s2)::value;
    if (s + 1 < S) load_w(s + 1, B ^ 1);
    const uint8_t* wb = wbuf(B) + wrow0;
    const uint8_t* xb = xbuf(B) + xrow0;
    bf16x8 af[2][4], bf[2][TW];
    auto fetch = [&](int kk, int slot) __attribute__((always_inline)) {
#pragma unroll
      for (int ti = 0; ti < TW; ++ti)
        bf[slot][ti] = as_bf16x8(*reinterpret_cast<const uint4*>(xb + ti * 32 * kRowB + ofs[kk]));
#pragma unroll
      for (int fi = 0; fi < 4; ++fi)
        af[slot][fi] = as_bf16x8(*reinterpret_cast<const uint4*>(wb + fi * 32 * kRowB + ofs[kk]));
    };
    fetch(0, 0);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      if (kk + 1 < 4) fetch(kk + 1, (kk + 1) & 1);
      if (kk == 1 && s + 1 < S) {
        xstore(xbuf(B ^ 1), xr);
        if (s + 2 < S) xload(s + 2, xr);
      }
#pragma unroll
      for (int ti = 0; ti < TW; ++ti)
#pragma unroll
        for (int fi = 0; fi < 4; ++fi)
          acc[ti][fi] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[kk & 1][fi], bf[kk & 1][ti],
                                                                acc[ti][fi], 0, 0, 0);
    }
    __syncthreads();
  };
  using C0 = std::integral_constant<int, 0>;
  using C1 = std::integral_constant<int, 1>;
  for (int s = 0; s < S; s += 2) {
    stage(s, C0{});
    if (s + 1 >= S) break;
    stage(s + 1, C1{});
  }
}

}  // namespace gemm
}  // namespace neo
