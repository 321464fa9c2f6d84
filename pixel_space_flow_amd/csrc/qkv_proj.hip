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
// The matrix product is the shared tile core (gemm_tile.h): 256 features (two heads) x 256
// tokens per workgroup, wave w owning head w / 4 of the pair and 64 tokens.  The epilogue
// here relies on its accumulator layout: each lane holds one token and 64 of its head's 128
// features (the other 64 are in lane ^ 32).  The two RMS statistics are then in-lane sums
// plus one swap with lane ^ 32, and every rotary pair (i, i + w/2) of a slice sits in the
// same lane: temporal pairs across accumulators 0 and 1, height and width pairs 16 rows
// apart inside accumulators 2 and 3.  fp32 accumulation; norm and rotary in fp32 (angles
// formed in fp64 revolutions and reduced modulo one turn, as in the stand-alone prologue);
// one rounding to bf16.
#include "gemm_tile.h"

#include <math.h>

namespace neo {
namespace {

using gemm::f32x16;
using gemm::kThreads;

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
  const int heads = Hq + 2 * Hkv;
  const int F = heads * 128;

  const int lane = threadIdx.x & 63, hl = lane >> 5, col = lane & 31;
  const int wave = threadIdx.x >> 6, hh = wave >> 2, tg = wave & 3;

  // tile resources end at the matrix rows, so rows past F or N arrive as zeros
  const int wrows = F - f0 < gemm::kFT ? F - f0 : gemm::kFT;
  // (a half tile cut from the last token tile may start at or past N: no rows at all)
  const int xleft = N - t0 < 0 ? 0 : N - t0;
  const int xrows = xleft < kTTile ? xleft : kTTile;
  const uint32_t row_bytes = (uint32_t)hidden * 2;
  const __amdgpu_buffer_rsrc_t rw =
      gemm::make_rsrc(w + (int64_t)f0 * hidden, (uint32_t)wrows * row_bytes);
  const __amdgpu_buffer_rsrc_t rx =
      gemm::make_rsrc(x + (int64_t)t0 * hidden, (uint32_t)xrows * row_bytes);
  f32x16 acc[TW][4];
  gemm::mainloop<TW>(
      acc, rw, row_bytes, rx,
      [&](int r) __attribute__((always_inline)) { return (uint32_t)r * row_bytes; },
      [&](int s) __attribute__((always_inline)) { return (uint32_t)(s * gemm::kRowB); },
      hidden / gemm::kKS, lw0, lw1, lx0, lx1);

  // ---- epilogue: this wave's head (global head gh), token t = t0 + 32 tb + col --------
  const int gh = f0 / 128 + hh;
  if (gh >= heads) return;
#pragma unroll
  for (int ti = 0; ti < TW; ++ti) {
    f32x16(&acc_t)[4] = acc[ti];
  const int t = t0 + tg * 32 * TW + ti * 32 + col;
  const bool tvalid = t < N;
  // accumulator fi, element r holds feature 32 fi + row(r) of the head
  auto row_of = [&](int r) __attribute__((always_inline)) { return gemm::row_of(r, hl); };

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
      sincos_turns((float)rev, &sn, &cs);
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
  // The 32 x 128 block goes out through LDS, so that each lane stores whole 16-byte
  // chunks and four lanes-of-16 cover four complete 256-byte rows.  The tile buffers are
  // free: the main loop ends with a barrier after its last fragment read.  Wave w stages in
  // 8 KB of its own 16 KB (row = token, chunk c of a row in slot c ^ (row mod 16)).
  uint8_t* ob = ((wave >> 1) == 0 ? lw0 : (wave >> 1) == 1 ? lw1 : (wave >> 1) == 2 ? lx0 : lx1) +
                (wave & 1) * 16384 + ti * 8192;
#pragma unroll
  for (int fi = 0; fi < 4; ++fi)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const uint32_t lo = pack_bf16x2(acc_t[fi][rg * 4 + 0], acc_t[fi][rg * 4 + 1]);
      const uint32_t hi = pack_bf16x2(acc_t[fi][rg * 4 + 2], acc_t[fi][rg * 4 + 3]);
      const int slot = (fi * 4 + rg) ^ (col & 15);
      *reinterpret_cast<uint2*>(ob + col * 256 + slot * 16 + hl * 8) = make_uint2(lo, hi);
    }
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the block is in LDS
  asm volatile("" ::: "memory");
  const int tb = t0 + tg * 32 * TW + ti * 32;  // first token of the block
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = 4 * i + (lane >> 4), c = lane & 15;
    const uint4 vrow = *reinterpret_cast<const uint4*>(ob + r * 256 + ((c ^ (r & 15)) * 16));
    const int tr = tb + r;
    if (tr < N) {
      uint16_t* orow = kind == 0 ? q_out + ((int64_t)tr * Hq + gh) * 128
                     : kind == 1 ? k_out + ((int64_t)tr * Hkv + (gh - Hq)) * 128
                                 : v_out + ((int64_t)tr * Hkv + (gh - Hq - Hkv)) * 128;
      *reinterpret_cast<uint4*>(orow + c * 8) = vrow;
    }
  }
  }
}

// Work split: tiles of 256 features x 256 tokens; when their count is not a multiple of
// the CU count, the surplus tiles are cut into halves of 128 tokens and launched after the
// full ones, so every CU ends up with about the same work (one full tile and one half
// where the surplus is half the CU count, as at 4096 tokens and 48 heads).
__global__ __launch_bounds__(kThreads, 1) void qkv_proj_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, int N, int hidden, int Hq,
    int Hkv, gemm::Plan plan, const float* __restrict__ wq_t,
    const float* __restrict__ wq_hw, const float* __restrict__ wk_t,
    const float* __restrict__ wk_hw, const int32_t* __restrict__ pos, double r_t, double r_hw,
    float eps, uint16_t* __restrict__ q_out, uint16_t* __restrict__ k_out,
    uint16_t* __restrict__ v_out) {
  __shared__ __attribute__((aligned(1024))) uint8_t lw0[gemm::kWTileB], lw1[gemm::kWTileB],
      lx0[gemm::kXTileB], lx1[gemm::kXTileB];
  const gemm::Tile tl = gemm::tile_of(blockIdx.x, plan);
  if (tl.full)
    proj_tile<2>(x, w, N, hidden, Hq, Hkv, tl.f0, tl.t0, wq_t, wq_hw, wk_t, wk_hw, pos, r_t,
                 r_hw, eps, q_out, k_out, v_out, lw0, lw1, lx0, lx1);
  else
    proj_tile<1>(x, w, N, hidden, Hq, Hkv, tl.f0, tl.t0, wq_t, wq_hw, wk_t, wk_hw, pos, r_t,
                 r_hw, eps, q_out, k_out, v_out, lw0, lw1, lx0, lx1);
}

}  // namespace

hipError_t launch_qkv_proj_bf16(const void* x, const void* w, int64_t N, int hidden, int Hq,
                                int Hkv, const float* wq_t, const float* wq_hw, const float* wk_t,
                                const float* wk_hw, const int32_t* pos, double theta,
                                double theta_hw, float eps, void* q_out, void* k_out,
                                void* v_out, hipStream_t stream) {
  if (N == 0) return hipSuccess;
  const gemm::Plan plan = gemm::make_plan((int64_t)(Hq + 2 * Hkv) * 128, N);
  const double r_t = pow(theta, -2.0 / 64.0);
  const double r_hw = pow(theta_hw, -2.0 / 32.0);
  hipLaunchKernelGGL(qkv_proj_bf16_kernel, dim3((unsigned)(plan.n_full + plan.n_half)),
                     dim3(kThreads), 0, stream, static_cast<const uint16_t*>(x),
                     static_cast<const uint16_t*>(w), (int)N, hidden, Hq, Hkv, plan, wq_t, wq_hw,
                     wk_t, wk_hw, pos, r_t, r_hw, eps, static_cast<uint16_t*>(q_out),
                     static_cast<uint16_t*>(k_out), static_cast<uint16_t*>(v_out));
  return hipGetLastError();
}

}  // namespace neo
