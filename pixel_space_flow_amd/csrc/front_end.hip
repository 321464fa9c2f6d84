// The generation branch's embedding front end: noisy pixels -> image-token embeddings.
//
// "SenseNova-U1.5 (NEO-unify) architecture", §Vision tower -- no transformer blocks: a
// 16x16 stride-16 patch convolution, GELU, an interleaved two-axis rotary (base 1e4; the
// first half of the channels turns with the column position, the second half with the row
// position), and a 2x2 stride-2 convolution into the backbone width -- one token per 32x32
// pixels.  §Timestep and noise-scale conditioning: two embedders over a 256-wide [cos, sin]
// sinusoid basis (the noise scale normalised by its maximum) whose outputs are summed and
// added to every image token.  "SenseNova-U1 ... NEO-unify Architecture" §2.1 prints the
// two convolutions of NEOVisionEmbeddings.
//
// Kernels:
//   patchify_bf16_kernel   pixels fp32 [B, 3, H, W] -> patch rows bf16 [B P, 768], ordered
//                          (channel, ky, kx) like a flattened convolution weight (streaming);
//   patch_gemm_kernel      rows x w1^T on the shared MFMA tile core, epilogue bias + GELU +
//                          rotary, bf16 features [B P, C1];
//   cond_hidden_kernel     first embedder layer: silu(wa e + ba) for both embedders (one
//                          wave per output row; reads wa once);
//   cond_out_kernel        second layer: wb_t h_t + bb_t + wb_s h_s + bb_s (one wave per
//                          row; streams wb once);
//   merge_gemm_kernel      the 2x2 convolution as a matrix product whose input rows are
//                          gathered from the patch features (each 64-wide K stage lies in
//                          one window cell, so a row's offset is its top-left patch plus a
//                          per-stage cell offset), epilogue + b2 + cond, fp32 tokens.
#include "gemm_tile.h"

#include <math.h>

namespace neo {
namespace {

using gemm::f32x16;
using gemm::kThreads;

constexpr int kPatch = 16;
constexpr int kPatchK = 3 * kPatch * kPatch;  // 768
constexpr int kStreamThreads = 256;
constexpr int kSinDim = 256;

// ---- patchify --------------------------------------------------------------------------
// One strip = up to 16 consecutive patches of one patch row (image b, patch row py, patches
// px0 .. px0 + 15).  Its pixels are 3 channels x 16 pixel rows of 16 * 16 contiguous floats:
// 48 runs of up to 1 KB, read with consecutive lanes on consecutive 16-byte pieces.  They are
// rounded to bf16 into a patch-major LDS image (row stride 776 elements, so that the
// patches' rows fall on different banks) and leave as whole 1536-byte patch rows, again with
// consecutive lanes on consecutive 16-byte pieces.
constexpr int kStrip = 16;               // patches per strip
constexpr int kStagedRow = kPatchK + 8;  // bf16 per staged patch row
__global__ __launch_bounds__(kStreamThreads) void patchify_bf16_kernel(
    const float* __restrict__ z, int64_t strips, int H, int W, int gw, int spr, int64_t P,
    uint16_t* __restrict__ patches) {
  __shared__ __attribute__((aligned(16))) uint16_t st[kStrip * kStagedRow];
  const int gh = H / kPatch;
  for (int64_t s = blockIdx.x; s < strips; s += gridDim.x) {
    const int sx = (int)(s % spr);
    const int64_t rest = s / spr;
    const int py = (int)(rest % gh);
    const int64_t b = rest / gh;
    const int px0 = sx * kStrip;
    const int np = gw - px0 < kStrip ? gw - px0 : kStrip;  // patches in this strip
    const int ncols = np * kPatch;                         // pixels per run
    for (int u = threadIdx.x; u < 3 * kPatch * 64; u += kStreamThreads) {
      const int run = u >> 6, x = 4 * (u & 63);  // run = channel * 16 + ky
      if (x < ncols) {
        const int c = run >> 4, ky = run & 15;
        const float4 a = *reinterpret_cast<const float4*>(
            z + ((b * 3 + c) * H + (int64_t)(py * kPatch + ky)) * W + px0 * kPatch + x);
        uint2 w;
        w.x = pack_bf16x2(a.x, a.y);
        w.y = pack_bf16x2(a.z, a.w);
        *reinterpret_cast<uint2*>(st + (x >> 4) * kStagedRow + c * 256 + ky * 16 + (x & 15)) = w;
      }
    }
    __syncthreads();
    for (int u = threadIdx.x; u < np * (kPatchK / 8); u += kStreamThreads) {
      const int p = u / (kPatchK / 8), e = (u - p * (kPatchK / 8)) * 8;
      *reinterpret_cast<uint4*>(patches + (b * P + (int64_t)py * gw + px0 + p) * kPatchK + e) =
          *reinterpret_cast<const uint4*>(st + p * kStagedRow + e);
    }
    __syncthreads();  // the next strip reuses the staging area
  }
}

// ---- patch convolution + GELU + rotary --------------------------------------------------
// GELU(x) = x Phi(x) = x (1 + erf(x / sqrt 2)) / 2, with erf from Abramowitz & Stegun,
// Handbook of Mathematical Functions, formula 7.1.26 (Hastings): for u >= 0,
// erf(u) = 1 - t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) exp(-u^2), t = 1 / (1 + p u), with
// absolute error below 1.5e-7 -- far under the bf16 rounding of the result -- at the cost
// of one reciprocal and one exponential; erf is odd.
__device__ __forceinline__ float gelu(float x) {
  constexpr float p = 0.3275911f, a1 = 0.254829592f, a2 = -0.284496736f, a3 = 1.421413741f,
                  a4 = -1.453152027f, a5 = 1.061405429f;
  const float u = fabsf(x) * 0.70710678118654752f;
  const float t = __builtin_amdgcn_rcpf(fmaf(p, u, 1.0f));
  const float poly = t * fmaf(t, fmaf(t, fmaf(t, fmaf(t, a5, a4), a3), a2), a1);
  // exp(-u^2) = 2^(-u^2 log2 e); underflows to zero for large |x|, where erf is +-1
  const float e = __builtin_amdgcn_exp2f(-u * u * 1.4426950408889634f);
  const float erf_abs = fmaf(-poly, e, 1.0f);
  return 0.5f * x * (1.0f + copysignf(erf_abs, x));
}

// The epilogue of a patch-convolution tile: bias, GELU, rotary, bf16 stores.
template <int TW>
__device__ __forceinline__ void patch_epilogue(f32x16 (&acc)[TW][4], const float* __restrict__ b1,
                                               int64_t M, int C1, int gw, int P, float l2f,
                                               int f0, int t0, uint16_t* __restrict__ hout) {
  const int lane = threadIdx.x & 63, hl = lane >> 5, col = lane & 31;
  const int wave = threadIdx.x >> 6, hh = wave >> 2, tg = wave & 3;
  // per-lane constants shared by both token columns: the bias of each feature and the
  // rotary rate (revolutions per grid step) of each feature pair
  const int half_c = C1 >> 1;
  float4 bias[4][4];
  float rate[4][4][2];
#pragma unroll
  for (int fi = 0; fi < 4; ++fi)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const int f = f0 + 128 * hh + 32 * fi + rg * 8 + 4 * hl;  // features f .. f + 3
      bias[fi][rg] = f < C1 ? *reinterpret_cast<const float4*>(b1 + f) : make_float4(0, 0, 0, 0);
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int fe = f + 2 * e;
        const int i = ((fe >= half_c ? fe - half_c : fe) >> 1);
        rate[fi][rg][e] = exp2f(-(float)i * l2f) * 0.15915494309189535f;
      }
    }
#pragma unroll
  for (int ti = 0; ti < TW; ++ti) {
    const int64_t m = (int64_t)t0 + tg * 32 * TW + ti * 32 + col;  // patch row
    if (m >= M) continue;
    const int mi = (int)(m % P);
    const float px = (float)(mi % gw), py = (float)(mi / gw);
#pragma unroll
    for (int fi = 0; fi < 4; ++fi) {
      const int fb = f0 + 128 * hh + 32 * fi;  // first feature of this accumulator
      if (fb >= C1) continue;
      uint16_t* orow = hout + m * C1 + fb;
      // the first C1/2 features turn with the column, the rest with the row (C1/2 is a
      // multiple of 32, so a 32-feature block lies in one half)
      const float pos = fb >= half_c ? py : px;
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const float bb[4] = {bias[fi][rg].x, bias[fi][rg].y, bias[fi][rg].z, bias[fi][rg].w};
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x = acc[ti][fi][rg * 4 + e] + bb[e];
          v[e] = gelu(x);
        }
        // pairs (f, f + 1), f even: elements e = 0, 1 and 2, 3.  The angle is taken in
        // revolutions and reduced to one turn inside sincos_turns, which needs no wide
        // argument reduction (positions are below 2^11, so the fp32 revolutions carry an
        // absolute error under 1e-4 turn at the largest image and ~1e-6 at 2048 px).
#pragma unroll
        for (int e = 0; e < 4; e += 2) {
          float sn, cs;
          sincos_turns(pos * rate[fi][rg][e >> 1], &sn, &cs);
          const float a = v[e], b = v[e + 1];
          v[e] = a * cs - b * sn;
          v[e + 1] = a * sn + b * cs;
        }
        *reinterpret_cast<uint2*>(orow + rg * 8 + 4 * hl) =
            make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
      }
    }
  }
}

// A tile whose X rows are the bf16 patch rows of patchify_bf16_kernel.
template <int TW>
__device__ __forceinline__ void patch_tile(const uint16_t* __restrict__ patches,
                                           const uint16_t* __restrict__ w1,
                                           const float* __restrict__ b1, int64_t M, int C1,
                                           int gw, int P, float l2f, int f0, int t0,
                                           uint16_t* __restrict__ hout, uint8_t* lw0,
                                           uint8_t* lw1, uint8_t* lx0, uint8_t* lx1) {
  constexpr int kTTile = 128 * TW;
  constexpr uint32_t kRowBytes = kPatchK * 2;
  const int wrows = C1 - f0 < gemm::kFT ? C1 - f0 : gemm::kFT;
  const int64_t xleft = M - t0 < 0 ? 0 : M - t0;
  const int xrows = xleft < kTTile ? (int)xleft : kTTile;
  const __amdgpu_buffer_rsrc_t rw = gemm::make_rsrc(w1 + (int64_t)f0 * kPatchK, (uint32_t)wrows * kRowBytes);
  const __amdgpu_buffer_rsrc_t rx =
      gemm::make_rsrc(patches + (int64_t)t0 * kPatchK, (uint32_t)xrows * kRowBytes);
  f32x16 acc[TW][4];
  gemm::mainloop<TW>(
      acc, rw, kRowBytes, rx,
      [&](int r) __attribute__((always_inline)) { return (uint32_t)r * kRowBytes; },
      [&](int s) __attribute__((always_inline)) { return (uint32_t)(s * gemm::kRowB); },
      kPatchK / gemm::kKS, lw0, lw1, lx0, lx1);
  patch_epilogue<TW>(acc, b1, M, C1, gw, P, l2f, f0, t0, hout);
}

__global__ __launch_bounds__(kThreads, 1) void patch_gemm_kernel(
    const uint16_t* __restrict__ patches, const uint16_t* __restrict__ w1,
    const float* __restrict__ b1, int64_t M, int C1, int gw, int P, float l2f, gemm::Plan plan,
    uint16_t* __restrict__ hout) {
  __shared__ __attribute__((aligned(1024))) uint8_t lw0[gemm::kWTileB], lw1[gemm::kWTileB],
      lx0[gemm::kXTileB], lx1[gemm::kXTileB];
  const gemm::Tile tl = gemm::tile_of(blockIdx.x, plan);
  if (tl.full)
    patch_tile<2>(patches, w1, b1, M, C1, gw, P, l2f, tl.f0, tl.t0, hout, lw0, lw1, lx0, lx1);
  else
    patch_tile<1>(patches, w1, b1, M, C1, gw, P, l2f, tl.f0, tl.t0, hout, lw0, lw1, lx0, lx1);
}

// A tile whose X rows are gathered from the fp32 pixels and rounded to bf16 on their way
// into LDS -- the rows patchify_bf16_kernel would write, so the result is bit-identical to
// patchify followed by patch_tile.  K stage s covers channel s / 4 and pixel rows
// 4 (s % 4) .. +3 of each patch; its 16-byte LDS chunk q holds pixel row q / 2, columns
// 8 (q % 2) .. +7.  Thread t fills, for tile row r = t / (8 / (2 TW)) and column half
// t % 2, the chunks of 2 TW consecutive pixel rows: two 16-byte loads of 8 fp32 each.  Along
// a patch row the tile's rows are consecutive 64-byte runs of the same pixel row, so
// consecutive lanes read consecutive 32-byte pieces.
template <int TW>
__device__ __forceinline__ void patch_px_tile(const float* __restrict__ z, uint32_t z_bytes,
                                              int H, int W, const uint16_t* __restrict__ w1,
                                              const float* __restrict__ b1, int64_t M, int C1,
                                              int gw, int P, float l2f, int f0, int t0,
                                              uint16_t* __restrict__ hout, uint8_t* lw0,
                                              uint8_t* lw1, uint8_t* lx0, uint8_t* lx1) {
  constexpr uint32_t kRowBytes = kPatchK * 2;
  constexpr int kJ = 2 * TW;  // pixel rows per thread and stage
  const int wrows = C1 - f0 < gemm::kFT ? C1 - f0 : gemm::kFT;
  const __amdgpu_buffer_rsrc_t rw = gemm::make_rsrc(w1 + (int64_t)f0 * kPatchK, (uint32_t)wrows * kRowBytes);
  const __amdgpu_buffer_rsrc_t rz = gemm::make_rsrc(z, z_bytes);
  const int tid = threadIdx.x;
  const int r = tid / (8 / kJ), half = tid & 1, jb = ((tid >> 1) % (4 / kJ)) * kJ;
  // byte offset of this thread's first piece (channel 0, pixel row 0 of its patch), or past
  // the pixels for rows beyond the last patch; every offset is below 2^31 + z_bytes < 2^32
  uint32_t base = gemm::kAbsentRow;
  const int64_t m = (int64_t)t0 + r;
  if (m < M) {
    const uint32_t b = (uint32_t)(m / P), mi = (uint32_t)(m - (int64_t)b * P);
    const uint32_t py = mi / (uint32_t)gw, px = mi - py * (uint32_t)gw;
    base = (((b * 3u * (uint32_t)H + 16u * py) * (uint32_t)W) + 16u * px + 8u * (uint32_t)half) * 4u;
  }
  const uint32_t row_b = (uint32_t)W * 4u;  // one pixel row
  const int slot0 = r * gemm::kRowB;
  f32x16 acc[TW][4];
  gemm::mainloop_xreg<TW, 2 * kJ>(
      acc, rw, kRowBytes,
      [&](int s, uint4 (&xr)[2 * kJ]) __attribute__((always_inline)) {
        const uint32_t so = ((uint32_t)(s >> 2) * (uint32_t)H + 4u * (uint32_t)(s & 3)) * row_b;
#pragma unroll
        for (int jj = 0; jj < kJ; ++jj) {
          const uint32_t off = base + so + (uint32_t)(jb + jj) * row_b;
          xr[2 * jj] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rz, (int)off, 0, 0));
          xr[2 * jj + 1] =
              __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rz, (int)(off + 16u), 0, 0));
        }
      },
      [&](uint8_t* xb, const uint4 (&xr)[2 * kJ]) __attribute__((always_inline)) {
#pragma unroll
        for (int jj = 0; jj < kJ; ++jj) {
          const float4 a = __builtin_bit_cast(float4, xr[2 * jj]);
          const float4 c = __builtin_bit_cast(float4, xr[2 * jj + 1]);
          const int q = 2 * (jb + jj) + half;
          *reinterpret_cast<uint4*>(xb + slot0 + ((q ^ gemm::pswz(r)) << 4)) =
              make_uint4(pack_bf16x2(a.x, a.y), pack_bf16x2(a.z, a.w), pack_bf16x2(c.x, c.y),
                         pack_bf16x2(c.z, c.w));
        }
      },
      kPatchK / gemm::kKS, lw0, lw1, lx0, lx1);
  patch_epilogue<TW>(acc, b1, M, C1, gw, P, l2f, f0, t0, hout);
}

__global__ __launch_bounds__(kThreads, 1) void patch_px_gemm_kernel(
    const float* __restrict__ z, uint32_t z_bytes, int H, int W,
    const uint16_t* __restrict__ w1, const float* __restrict__ b1, int64_t M, int C1, int gw,
    int P, float l2f, gemm::Plan plan, uint16_t* __restrict__ hout) {
  __shared__ __attribute__((aligned(1024))) uint8_t lw0[gemm::kWTileB], lw1[gemm::kWTileB],
      lx0[gemm::kXTileB], lx1[gemm::kXTileB];
  const gemm::Tile tl = gemm::tile_of(blockIdx.x, plan);
  if (tl.full)
    patch_px_tile<2>(z, z_bytes, H, W, w1, b1, M, C1, gw, P, l2f, tl.f0, tl.t0, hout, lw0, lw1,
                     lx0, lx1);
  else
    patch_px_tile<1>(z, z_bytes, H, W, w1, b1, M, C1, gw, P, l2f, tl.f0, tl.t0, hout, lw0, lw1,
                     lx0, lx1);
}

// ---- time and noise-scale embedders ----------------------------------------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Row j of embedder e (0: time, 1: noise scale): hidden[e][j] = silu(wa_e[j] . basis_e + ba_e[j])
// with basis_e the [cos, sin] sinusoid of arg[e]; lane l takes basis entries 4l .. 4l+3.
__global__ __launch_bounds__(kStreamThreads) void cond_hidden_kernel(
    float arg_t, float arg_s, int D, const uint16_t* __restrict__ wa_t,
    const float* __restrict__ ba_t, const uint16_t* __restrict__ wa_s,
    const float* __restrict__ ba_s, float* __restrict__ hidden) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * (kStreamThreads / 64) + (threadIdx.x >> 6);
  if (row >= 2 * (int64_t)D) return;
  const int e = row >= D ? 1 : 0;
  const int j = (int)(row - (int64_t)e * D);
  const float arg = e ? arg_s : arg_t;
  const uint16_t* wa = (e ? wa_s : wa_t) + (int64_t)j * kSinDim;
  const uint2 wv = *reinterpret_cast<const uint2*>(wa + 4 * lane);
  const float w4[4] = {bf16_lo(wv.x), bf16_hi(wv.x), bf16_lo(wv.y), bf16_hi(wv.y)};
  // frequencies exp(-ln(10000) k / 128) = 2^(-k log2(10000) / 128)
  constexpr float kL2 = 13.287712379549449f / 128.0f;
  float acc = 0.0f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int i = 4 * lane + q;
    const int k = i & 127;
    float sn, cs;
    sincosf(arg * exp2f(-(float)k * kL2), &sn, &cs);
    acc = fmaf(w4[q], i < 128 ? cs : sn, acc);
  }
  acc = wave_sum(acc);
  if (lane == 0) {
    const float x = acc + (e ? ba_s : ba_t)[j];
    hidden[row] = x / (1.0f + expf(-x));
  }
}

// cond[j] = wb_t[j] . hidden[0] + bb_t[j] + wb_s[j] . hidden[1] + bb_s[j]: one wave per row,
// lane l reading 16-byte chunks l, l + 64, ... of both weight rows.
__global__ __launch_bounds__(kStreamThreads) void cond_out_kernel(
    int D, const float* __restrict__ hidden, const uint16_t* __restrict__ wb_t,
    const float* __restrict__ bb_t, const uint16_t* __restrict__ wb_s,
    const float* __restrict__ bb_s, float* __restrict__ cond) {
  const int lane = threadIdx.x & 63;
  const int j = blockIdx.x * (kStreamThreads / 64) + (threadIdx.x >> 6);
  if (j >= D) return;
  const int chunks = D >> 3;
  float acc = 0.0f;
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const uint4* wr = reinterpret_cast<const uint4*>((e ? wb_s : wb_t) + (int64_t)j * D);
    const float4* hv = reinterpret_cast<const float4*>(hidden + (int64_t)e * D);
    for (int c = lane; c < chunks; c += 64) {
      const uint4 w8 = wr[c];
      const float4 h0 = hv[2 * c], h1 = hv[2 * c + 1];
      acc = fmaf(bf16_lo(w8.x), h0.x, acc);
      acc = fmaf(bf16_hi(w8.x), h0.y, acc);
      acc = fmaf(bf16_lo(w8.y), h0.z, acc);
      acc = fmaf(bf16_hi(w8.y), h0.w, acc);
      acc = fmaf(bf16_lo(w8.z), h1.x, acc);
      acc = fmaf(bf16_hi(w8.z), h1.y, acc);
      acc = fmaf(bf16_lo(w8.w), h1.z, acc);
      acc = fmaf(bf16_hi(w8.w), h1.w, acc);
    }
  }
  acc = wave_sum(acc);
  if (lane == 0) cond[j] = acc + bb_t[j] + bb_s[j];
}

// ---- 2x2 merge convolution + bias + conditioning ----------------------------------------
template <int TW>
__device__ __forceinline__ void merge_tile(const uint16_t* __restrict__ h,
                                           const uint16_t* __restrict__ w2,
                                           const float* __restrict__ b2,
                                           const float* __restrict__ cond, int64_t Ntot,
                                           int Nimg, int tw, int gw, int64_t P, int C1, int D,
                                           uint32_t h_bytes, int S, int f0, int t0,
                                           float* __restrict__ tokens, uint8_t* lw0,
                                           uint8_t* lw1, uint8_t* lx0, uint8_t* lx1) {
  const int lane = threadIdx.x & 63, hl = lane >> 5, col = lane & 31;
  const int wave = threadIdx.x >> 6, hh = wave >> 2, tg = wave & 3;
  const uint32_t w_row_bytes = (uint32_t)C1 * 8;   // K = 4 C1 bf16
  const uint32_t h_row_bytes = (uint32_t)C1 * 2;
  const int wrows = D - f0 < gemm::kFT ? D - f0 : gemm::kFT;
  const __amdgpu_buffer_rsrc_t rw = gemm::make_rsrc(w2 + (int64_t)f0 * 4 * C1, (uint32_t)wrows * w_row_bytes);
  const __amdgpu_buffer_rsrc_t rx = gemm::make_rsrc(h, h_bytes);
  const int cpr = C1 / gemm::kKS;  // K stages per window cell
  f32x16 acc[TW][4];
  gemm::mainloop<TW, true>(
      acc, rw, w_row_bytes, rx,
      [&](int r) __attribute__((always_inline)) {
        // the token's top-left patch row (cell dy = dx = 0); every count here is below
        // 2^31 (the features are under 2 GiB), so 32-bit arithmetic is exact
        const uint32_t n = (uint32_t)t0 + (uint32_t)r;
        if (n >= (uint32_t)Ntot) return gemm::kAbsentRow;
        const uint32_t b = n / (uint32_t)Nimg, m = n - b * (uint32_t)Nimg;
        const uint32_t ty = m / (uint32_t)tw, tx = m - ty * (uint32_t)tw;
        return (b * (uint32_t)P + 2 * ty * (uint32_t)gw + 2 * tx) * h_row_bytes;
      },
      [&](int s) __attribute__((always_inline)) {
        // window cell q = s / cpr (s < 4 cpr), (dy, dx) = (q / 2, q % 2)
        const int q = (s >= cpr) + (s >= 2 * cpr) + (s >= 3 * cpr), cs = s - q * cpr;
        return (uint32_t)(((q >> 1) * gw + (q & 1)) * (int)h_row_bytes + cs * gemm::kRowB);
      },
      S, lw0, lw1, lx0, lx1);

  // Each 32-token x 128-feature block goes out through LDS, so that every lane stores a
  // whole 16-byte chunk and each half-wave a complete 512-byte row segment.  The tile
  // buffers are free (the main loop ends with a barrier after its last fragment read).
  // Wave w stages in its own 16 KB: row = token, 16-byte chunk c of a row in slot
  // c ^ (row mod 32).
  uint8_t* ob = ((wave >> 1) == 0 ? lw0 : (wave >> 1) == 1 ? lw1 : (wave >> 1) == 2 ? lx0 : lx1) +
                (wave & 1) * 16384;
  const int fw = f0 + 128 * hh;  // the wave's first feature
#pragma unroll
  for (int ti = 0; ti < TW; ++ti) {
#pragma unroll
    for (int fi = 0; fi < 4; ++fi) {
      const int fb = fw + 32 * fi;
      if (fb >= D) continue;
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int f = fb + rg * 8 + 4 * hl;
        const float4 bb = *reinterpret_cast<const float4*>(b2 + f);
        const float4 cc = *reinterpret_cast<const float4*>(cond + f);
        float4 o;
        o.x = acc[ti][fi][rg * 4 + 0] + bb.x + cc.x;
        o.y = acc[ti][fi][rg * 4 + 1] + bb.y + cc.y;
        o.z = acc[ti][fi][rg * 4 + 2] + bb.z + cc.z;
        o.w = acc[ti][fi][rg * 4 + 3] + bb.w + cc.w;
        const int slot = (8 * fi + 2 * rg + hl) ^ col;
        *reinterpret_cast<float4*>(ob + col * 512 + slot * 16) = o;
      }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the block is in LDS
    asm volatile("" ::: "memory");
    const int64_t nb = (int64_t)t0 + tg * 32 * TW + ti * 32;  // first token of the block
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = 2 * i + (lane >> 5), c = lane & 31;
      const float4 v = *reinterpret_cast<const float4*>(ob + r * 512 + ((c ^ r) * 16));
      if (nb + r < Ntot && fw + 4 * c < D)
        *reinterpret_cast<float4*>(tokens + (nb + r) * D + fw + 4 * c) = v;
    }
    asm volatile("" ::: "memory");  // the next block reuses the staging area after these reads
  }
}

__global__ __launch_bounds__(kThreads, 1) void merge_gemm_kernel(
    const uint16_t* __restrict__ h, const uint16_t* __restrict__ w2, const float* __restrict__ b2,
    const float* __restrict__ cond, int64_t Ntot, int Nimg, int tw, int gw, int64_t P, int C1,
    int D, uint32_t h_bytes, int S, gemm::Plan plan, float* __restrict__ tokens) {
  __shared__ __attribute__((aligned(1024))) uint8_t lw0[gemm::kWTileB], lw1[gemm::kWTileB],
      lx0[gemm::kXTileB], lx1[gemm::kXTileB];
  const gemm::Tile tl = gemm::tile_of(blockIdx.x, plan);
  if (tl.full)
    merge_tile<2>(h, w2, b2, cond, Ntot, Nimg, tw, gw, P, C1, D, h_bytes, S, tl.f0, tl.t0, tokens,
                  lw0, lw1, lx0, lx1);
  else
    merge_tile<1>(h, w2, b2, cond, Ntot, Nimg, tw, gw, P, C1, D, h_bytes, S, tl.f0, tl.t0, tokens,
                  lw0, lw1, lx0, lx1);
}

}  // namespace

hipError_t launch_gen_patchify(const float* z, int B, int H, int W, void* patches,
                               hipStream_t stream) {
  const int gw = W / kPatch;
  const int spr = (gw + kStrip - 1) / kStrip;  // strips per patch row
  const int64_t strips = (int64_t)B * (H / kPatch) * spr;
  if (strips == 0) return hipSuccess;
  const int64_t P = (int64_t)(H / kPatch) * gw;
  const int64_t cap = 256 * 8;
  hipLaunchKernelGGL(patchify_bf16_kernel, dim3((unsigned)(strips < cap ? strips : cap)),
                     dim3(kStreamThreads), 0, stream, z, strips, H, W, gw, spr, P,
                     static_cast<uint16_t*>(patches));
  return hipGetLastError();
}

hipError_t launch_gen_patch_embed(const void* patches, int B, int H, int W, const void* w1,
                                  const float* b1, int C1, double theta, void* h,
                                  hipStream_t stream) {
  const int gw = W / kPatch;
  const int P = (H / kPatch) * gw;
  const int64_t M = (int64_t)B * P;
  if (M == 0) return hipSuccess;
  const gemm::Plan plan = gemm::make_plan(C1, M);
  // pair i of a half of width C1/2 turns at theta^(-2i/(C1/2)) = 2^(-i l2f)
  const float l2f = (float)(2.0 * log2(theta) / (C1 / 2));
  hipLaunchKernelGGL(patch_gemm_kernel, dim3((unsigned)(plan.n_full + plan.n_half)),
                     dim3(kThreads), 0, stream, static_cast<const uint16_t*>(patches),
                     static_cast<const uint16_t*>(w1), b1, M, C1, gw, P, l2f, plan,
                     static_cast<uint16_t*>(h));
  return hipGetLastError();
}

hipError_t launch_gen_patch_embed_px(const float* z, int B, int H, int W, const void* w1,
                                     const float* b1, int C1, double theta, void* h,
                                     hipStream_t stream) {
  const int gw = W / kPatch;
  const int P = (H / kPatch) * gw;
  const int64_t M = (int64_t)B * P;
  if (M == 0) return hipSuccess;
  const gemm::Plan plan = gemm::make_plan(C1, M);
  const float l2f = (float)(2.0 * log2(theta) / (C1 / 2));
  const uint32_t z_bytes = (uint32_t)((int64_t)B * 3 * H * W * 4);
  hipLaunchKernelGGL(patch_px_gemm_kernel, dim3((unsigned)(plan.n_full + plan.n_half)),
                     dim3(kThreads), 0, stream, z, z_bytes, H, W, static_cast<const uint16_t*>(w1),
                     b1, M, C1, gw, P, l2f, plan, static_cast<uint16_t*>(h));
  return hipGetLastError();
}

hipError_t launch_gen_cond_hidden(float arg_t, float arg_s, int D, const void* wa_t,
                                  const float* ba_t, const void* wa_s, const float* ba_s,
                                  float* hidden, hipStream_t stream) {
  const int64_t rows = 2 * (int64_t)D;
  const int per = kStreamThreads / 64;
  hipLaunchKernelGGL(cond_hidden_kernel, dim3((unsigned)((rows + per - 1) / per)),
                     dim3(kStreamThreads), 0, stream, arg_t, arg_s, D,
                     static_cast<const uint16_t*>(wa_t), ba_t, static_cast<const uint16_t*>(wa_s),
                     ba_s, hidden);
  return hipGetLastError();
}

hipError_t launch_gen_cond_out(int D, const float* hidden, const void* wb_t, const float* bb_t,
                               const void* wb_s, const float* bb_s, float* cond,
                               hipStream_t stream) {
  const int per = kStreamThreads / 64;
  hipLaunchKernelGGL(cond_out_kernel, dim3((unsigned)((D + per - 1) / per)), dim3(kStreamThreads),
                     0, stream, D, hidden, static_cast<const uint16_t*>(wb_t), bb_t,
                     static_cast<const uint16_t*>(wb_s), bb_s, cond);
  return hipGetLastError();
}

hipError_t launch_gen_merge_embed(const void* h, int B, int H, int W, int C1, const void* w2,
                                  const float* b2, const float* cond, int D, float* tokens,
                                  hipStream_t stream) {
  const int gw = W / kPatch, tw = W / (2 * kPatch);
  const int Nimg = (H / (2 * kPatch)) * tw;
  const int64_t Ntot = (int64_t)B * Nimg;
  if (Ntot == 0) return hipSuccess;
  const int64_t P = (int64_t)(H / kPatch) * gw;
  const uint32_t h_bytes = (uint32_t)((int64_t)B * P * C1 * 2);
  const gemm::Plan plan = gemm::make_plan(D, Ntot);
  hipLaunchKernelGGL(merge_gemm_kernel, dim3((unsigned)(plan.n_full + plan.n_half)),
                     dim3(kThreads), 0, stream, static_cast<const uint16_t*>(h),
                     static_cast<const uint16_t*>(w2), b2, cond, Ntot, Nimg, tw, gw, P, C1, D,
                     h_bytes, 4 * C1 / gemm::kKS, plan, tokens);
  return hipGetLastError();
}

}  // namespace neo
