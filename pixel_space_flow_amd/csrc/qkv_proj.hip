// Generation-branch q/k/v projection fused with the q/k prologue.
//
// "SenseNova-U1.5 (NEO-unify) architecture", §Mixture of Transformers: every layer holds
// a second weight set for the generation branch (q/k/v projections, split-half q/k
// norms); §Three rotary axes: q and k are normalised as two 64-dim halves and rotated on
// three axes.  This kernel computes [q | k | v] = x W^T for the noisy image tokens and
// applies norm + rotary to the q and k heads before anything leaves the chip, so the
// projection never round-trips through HBM.
//
// Layout: x [N, hidden] bf16, W [(Hq + 2 Hkv) * 128, hidden] bf16 with rows ordered q heads,
// k heads, v heads; outputs q [N, Hq, 128], k [N, Hkv, 128], v [N, Hkv, 128] bf16.
//
// Work mapping:
//   * the product is formed transposed, Y^T = W x^T, with v_mfma_f32_32x32x16_bf16: A = 32
//     rows of W (features), B = x^T (32 tokens), both read as 16-byte fragments of
//     row-major LDS tiles (hidden contiguous);
//   * a workgroup (8 waves) covers 256 features (two heads) x 256 tokens; wave w owns head
//     w / 4 of the pair and tokens 64 (w % 4) .. +63, as 4 x 2 accumulators of 32 x 32;
//   * tiles beyond a whole number of rounds over the CUs run as two 128-token halves (one
//     32-token accumulator column per wave), so the last round is as long as the others
//     and every CU ends at about the same time;
//   * in the accumulator layout each lane holds one token and 64 of its head's 128
//     features (the other 64 are in lane ^ 32).  The two RMS statistics are then in-lane
//     sums plus one swap with lane ^ 32, and every rotary pair (i, i + w/2) of a slice
//     sits in the same lane: temporal pairs across accumulators 0 and 1, height and width
//     pairs 16 rows apart inside accumulators 2 and 3;
//   * the hidden dimension streams through LDS in stages of 64, two stages deep (64 KB
//     each); tiles go from HBM/L2 straight into LDS (buffer loads with the LDS
//     destination) with the rows' 16-byte chunks XOR-swizzled on the fetch side, one
//     barrier per stage;
//   * fp32 accumulation; norm and rotary in fp32 (angles formed in fp64 revolutions and
//     reduced modulo one turn, as in the stand-alone prologue); one rounding to bf16.
#include "neo_internal.h"

#include <math.h>

#include <type_traits>

namespace neo {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = kProjThreads;  // 8 waves, two per SIMD
constexpr int kFT = 256;                // features per workgroup (two heads)
constexpr int kTT = 256;                // tokens per workgroup
constexpr int kGroup = 4;               // token tiles per group of the tile order
constexpr int kKS = 64;                 // hidden dims per stage
constexpr int kRowB = kKS * 2;          // one LDS tile row: 128 bytes = 8 chunks
constexpr int kWTileB = kFT * kRowB;    // 32 KB
constexpr int kXTileB = kTT * kRowB;    // 32 KB
constexpr int kBufFlags = 0x00020000;   // raw buffer, 32-bit data format (gfx9 family)

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

// One tile of 256 features x (32 TW * 4) tokens: TW = 2 for a full tile, 1 for a half.
template <int TW>
__device__ __forceinline__ void proj_tile(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, int N, int hidden, int Hq,
    int Hkv, int f0, int t0, const float* __restrict__ wq_t, const float* __restrict__ wq_hw,
    const float* __restrict__ wk_t, const float* __restrict__ wk_hw,
    const int32_t* __restrict__ pos, double r_t, double r_hw, float eps,
    uint16_t* __restrict__ q_out, uint16_t* __restrict__ k_out, uint16_t* __restrict__ v_out,
    uint8_t* lw0, uint8_t* lw1, uint8_t* lx0, uint8_t* lx1) {
  constexpr int kTTile = 128 * TW;  // tokens of this tile
  auto wbuf = [&](int b) __attribute__((always_inline)) -> uint8_t* { return b == 0 ? lw0 : lw1; };
  auto xbuf = [&](int b) __attribute__((always_inline)) -> uint8_t* { return b == 0 ? lx0 : lx1; };
  const int heads = Hq + 2 * Hkv;
  const int F = heads * 128;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, hl = lane >> 5, col = lane & 31;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int hh = wave >> 2, tg = wave & 3;  // head of the pair; token group of 32 TW

  // tile resources end at the matrix rows, so rows past F or N arrive as zeros
  const int wrows = F - f0 < kFT ? F - f0 : kFT;
  // (a half tile cut from the last token tile may start at or past N: no rows at all)
  const int xleft = N - t0 < 0 ? 0 : N - t0;
  const int xrows = xleft < kTTile ? xleft : kTTile;
  const uint32_t row_bytes = (uint32_t)hidden * 2;
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(w + (int64_t)f0 * hidden, (uint32_t)wrows * row_bytes);
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(x + (int64_t)t0 * hidden, (uint32_t)xrows * row_bytes);

  // staging: a tile is a run of 1 KB blocks of 8 rows; lane L of a block lands in row
  // 8*blk + L/8, slot L%8, and so fetches chunk (L%8) ^ pswz(row) of that row.  Wave w loads
  // W blocks 4w .. 4w+3 and x blocks 2 TW w .. 2 TW w + 2 TW - 1.
  int wofs[4], xofs[2 * TW];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 8 * (4 * wave + i) + (lane >> 3);
    wofs[i] = row * (int)row_bytes + (((lane & 7) ^ pswz(row)) << 4);
  }
#pragma unroll
  for (int i = 0; i < 2 * TW; ++i) {
    const int row = 8 * (2 * TW * wave + i) + (lane >> 3);
    xofs[i] = row * (int)row_bytes + (((lane & 7) ^ pswz(row)) << 4);
  }
  auto load_stage = [&](int s, int b) __attribute__((always_inline)) {
    const int koff = s * kRowB;  // hidden dims [64 s, 64 s + 64)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rw, (__attribute__((address_space(3))) void*)(wbuf(b) + (4 * wave_u + i) * 1024), 16,
          wofs[i] + koff, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 2 * TW; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rx, (__attribute__((address_space(3))) void*)(xbuf(b) + (2 * TW * wave_u + i) * 1024), 16,
          xofs[i] + koff, 0, 0, 0);
  };

  // fragment reads: W row 128 hh + 32 fi + col and x row 32 tb + col, chunk 2 kk + hl.  The
  // swizzle depends on the row's bits 1..3 only, which 128 hh + 32 fi and 32 tb leave alone.
  int ofs[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) ofs[kk] = col * kRowB + (((2 * kk + hl) ^ pswz(col)) << 4);
  const int wrow0 = hh * 128 * kRowB, xrow0 = tg * 32 * TW * kRowB;

  f32x16 acc[TW][4];
#pragma unroll
  for (int ti = 0; ti < TW; ++ti)
#pragma unroll
    for (int fi = 0; fi < 4; ++fi)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[ti][fi][r] = 0.0f;

  const int S = hidden / kKS;
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
    if (s + 1 >= S) break;
    stage(s + 1, C1{});
  }

  // ---- epilogue: this wave's head (global head gh), token t = t0 + 32 tb + col --------
  const int gh = f0 / 128 + hh;
  if (gh >= heads) return;
#pragma unroll
  for (int ti = 0; ti < TW; ++ti) {
    f32x16(&acc_t)[4] = acc[ti];
  const int t = t0 + tg * 32 * TW + ti * 32 + col;
  const bool tvalid = t < N;
  // accumulator fi, element r holds feature 32 fi + row(r) of the head
  auto row_of = [&](int r) __attribute__((always_inline)) { return (r >> 2) * 8 + 4 * hl + (r & 3); };

  const int kind = gh < Hq ? 0 : (gh < Hq + Hkv ? 1 : 2);  // q, k, v
  if (kind < 2) {
    const float* nw_t = kind == 0 ? wq_t : wk_t;
    const float* nw_hw = kind == 0 ? wq_hw : wk_hw;
    float ss0 = 0.0f, ss1 = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      ss0 = fmaf(acc_t[0][r], acc_t[0][r], ss0);
      ss0 = fmaf(acc_t[1][r], acc_t[1][r], ss0);
      ss1 = fmaf(acc_t[2][r], acc_t[2][r], ss1);
      ss1 = fmaf(acc_t[3][r], acc_t[3][r], ss1);
    }
    ss0 += __shfl_xor(ss0, 32);
    ss1 += __shfl_xor(ss1, 32);
    const float rinv0 = rsqrtf(ss0 * (1.0f / 64.0f) + eps);
    const float rinv1 = rsqrtf(ss1 * (1.0f / 64.0f) + eps);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int d = row_of(r);
      acc_t[0][r] *= rinv0 * nw_t[d];
      acc_t[1][r] *= rinv0 * nw_t[32 + d];
      acc_t[2][r] *= rinv1 * nw_hw[d];
      acc_t[3][r] *= rinv1 * nw_hw[32 + d];
    }
    // rotary.  Frequencies r^i (i the pair index) from r^(8a) r^(4 hl) r^b, i = 8a + 4hl + b
    const double p_t = tvalid ? (double)pos[t] : 0.0;
    const double p_h = tvalid ? (double)pos[N + t] : 0.0;
    const double p_w = tvalid ? (double)pos[2 * (int64_t)N + t] : 0.0;
    constexpr double kInv2Pi = 0.15915494309189533576888376337251436;
    auto angle = [&](double p, double freq, float& sn, float& cs) __attribute__((always_inline)) {
      double rev = p * freq * kInv2Pi;
      rev -= rint(rev);  // exact: the angle modulo one turn, in [-1/2, 1/2]
      sincospif((float)(2.0 * rev), &sn, &cs);
    };
    {
      // temporal slice: dims [0, 64), pairs (i, i + 32); i = row(r) in accumulator 0
      const double r2 = r_t * r_t, r4 = r2 * r2, r8 = r4 * r4;
      const double rb[4] = {1.0, r_t, r2, r2 * r_t};
      const double rhl = hl ? r4 : 1.0;
      double ra = rhl;
#pragma unroll
      for (int a = 0; a < 4; ++a) {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int r = a * 4 + b;
          float sn, cs;
          angle(p_t, ra * rb[b], sn, cs);
          const float y0 = acc_t[0][r], y1 = acc_t[1][r];
          acc_t[0][r] = y0 * cs - y1 * sn;
          acc_t[1][r] = y1 * cs + y0 * sn;
        }
        ra *= r8;
      }
    }
    {
      // height / width slices: dims [64, 96) and [96, 128), pairs (i, i + 16) with
      // i = row(r) < 16, i.e. elements r and r + 8 of accumulators 2 and 3
      const double r2 = r_hw * r_hw, r4 = r2 * r2, r8 = r4 * r4;
      const double rb[4] = {1.0, r_hw, r2, r2 * r_hw};
      const double rhl = hl ? r4 : 1.0;
      double ra = rhl;
#pragma unroll
      for (int a = 0; a < 2; ++a) {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int r = a * 4 + b;
          const double freq = ra * rb[b];
          float sn, cs;
          angle(p_h, freq, sn, cs);
          float y0 = acc_t[2][r], y1 = acc_t[2][r + 8];
          acc_t[2][r] = y0 * cs - y1 * sn;
          acc_t[2][r + 8] = y1 * cs + y0 * sn;
          angle(p_w, freq, sn, cs);
          y0 = acc_t[3][r];
          y1 = acc_t[3][r + 8];
          acc_t[3][r] = y0 * cs - y1 * sn;
          acc_t[3][r + 8] = y1 * cs + y0 * sn;
        }
        ra *= r8;
      }
    }
  }
  if (!tvalid) continue;
  uint16_t* orow = kind == 0 ? q_out + ((int64_t)t * Hq + gh) * 128
                 : kind == 1 ? k_out + ((int64_t)t * Hkv + (gh - Hq)) * 128
                             : v_out + ((int64_t)t * Hkv + (gh - Hq - Hkv)) * 128;
#pragma unroll
  for (int fi = 0; fi < 4; ++fi)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const uint32_t lo = pack_bf16x2(acc_t[fi][rg * 4 + 0], acc_t[fi][rg * 4 + 1]);
      const uint32_t hi = pack_bf16x2(acc_t[fi][rg * 4 + 2], acc_t[fi][rg * 4 + 3]);
      *reinterpret_cast<uint2*>(orow + fi * 32 + rg * 8 + 4 * hl) = make_uint2(lo, hi);
    }
  }
}

// Work split: tiles of 256 features x 256 tokens; when their count is not a multiple of
// the CU count, the surplus tiles are cut into halves of 128 tokens and launched after the
// full ones, so every CU ends up with about the same work (one full tile and one half
// where the surplus is half the CU count, as at 4096 tokens and 48 heads).
__global__ __launch_bounds__(kThreads, 1) void qkv_proj_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, int N, int hidden, int Hq,
    int Hkv, int n_ftiles, int n_ttiles, int n_full, int n_half, const float* __restrict__ wq_t,
    const float* __restrict__ wq_hw, const float* __restrict__ wk_t,
    const float* __restrict__ wk_hw, const int32_t* __restrict__ pos, double r_t, double r_hw,
    float eps, uint16_t* __restrict__ q_out, uint16_t* __restrict__ k_out,
    uint16_t* __restrict__ v_out) {
  // four separate LDS objects (two stages of W and x tiles), so the compiler sees that a
  // stage load cannot alias the fragment reads of the other stage
  __shared__ __attribute__((aligned(1024))) uint8_t lw0[kWTileB], lw1[kWTileB], lx0[kXTileB],
      lx1[kXTileB];
  // within each kind the order is remapped so that an XCD's workgroups take consecutive
  // tile ids, and ids run over groups of kGroup token tiles (token tile fastest), so the
  // 32 tiles an XCD holds at once form a 4 x 8 block that shares its x and W rows in L2
  const uint32_t b = blockIdx.x;
  auto tile_of = [&](uint32_t id, int& ft, int& tt) __attribute__((always_inline)) {
    const uint32_t per = (uint32_t)(kGroup * n_ftiles), g = id / per, r = id % per;
    const int first = (int)g * kGroup;
    const int gs = n_ttiles - first < kGroup ? n_ttiles - first : kGroup;
    ft = (int)(r / (uint32_t)gs);
    tt = first + (int)(r % (uint32_t)gs);
  };
  if (b < (uint32_t)n_full) {
    int ft, tt;
    tile_of(xcd_remap(b, (uint32_t)n_full), ft, tt);
    proj_tile<2>(x, w, N, hidden, Hq, Hkv, ft * kFT, tt * kTT, wq_t, wq_hw, wk_t, wk_hw, pos, r_t,
                 r_hw, eps, q_out, k_out, v_out, lw0, lw1, lx0, lx1);
  } else {
    const uint32_t h = xcd_remap(b - (uint32_t)n_full, (uint32_t)n_half);
    int ft, tt;
    tile_of((uint32_t)n_full + h / 2, ft, tt);
    proj_tile<1>(x, w, N, hidden, Hq, Hkv, ft * kFT, tt * kTT + 128 * (int)(h & 1), wq_t, wq_hw,
                 wk_t, wk_hw, pos, r_t, r_hw, eps, q_out, k_out, v_out, lw0, lw1, lx0, lx1);
  }
}

}  // namespace

hipError_t launch_qkv_proj_bf16(const void* x, const void* w, int64_t N, int hidden, int Hq,
                                int Hkv, const float* wq_t, const float* wq_hw, const float* wk_t,
                                const float* wk_hw, const int32_t* pos, double theta,
                                double theta_hw, float eps, void* q_out, void* k_out,
                                void* v_out, hipStream_t stream) {
  if (N == 0) return hipSuccess;
  const int heads = Hq + 2 * Hkv;
  const int64_t n_ftiles = (heads * 128 + kFT - 1) / kFT;
  const int64_t n_ttiles = (N + kTT - 1) / kTT;
  const int64_t n_tiles = n_ftiles * n_ttiles;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    cus = 256;
  // surplus tiles beyond a whole number of rounds are split in two (see the kernel)
  const int64_t surplus = n_tiles >= cus ? n_tiles % cus : 0;
  const int64_t n_full = n_tiles - surplus, n_half = 2 * surplus;
  const double r_t = pow(theta, -2.0 / 64.0);
  const double r_hw = pow(theta_hw, -2.0 / 32.0);
  hipLaunchKernelGGL(qkv_proj_bf16_kernel, dim3((unsigned)(n_full + n_half)), dim3(kThreads), 0,
                     stream, static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w), (int)N,
                     hidden, Hq, Hkv, (int)n_ftiles, (int)n_ttiles, (int)n_full, (int)n_half, wq_t, wq_hw, wk_t,
                     wk_hw, pos, r_t, r_hw, eps,
                     static_cast<uint16_t*>(q_out), static_cast<uint16_t*>(k_out),
                     static_cast<uint16_t*>(v_out));
  return hipGetLastError();
}

}  // namespace neo
