// Fused split-half QK-RMSNorm + three-axis rotary for the generation block.
//
// "SenseNova-U1.5 (NEO-unify) architecture", §Three rotary axes: each 128-dim head
// row is normalised as two independent 64-dim halves (q_norm / q_norm_hw, k_norm /
// k_norm_hw, weights of shape [64]); then dims [0:64) rotate with the temporal index
// (base rope_theta), [64:96) with the height index and [96:128) with the width index
// (base rope_theta_hw).  Pairs are half-split inside each slice (§Vision tower: the
// backbone uses the half-split convention).
//
// Work mapping (HBM-bound, 512 B moved per bf16 row):
//   * one wavefront per token; the token's Hq query rows and Hkv key rows are
//     contiguous in memory and are walked four rows at a time (16 lanes per row);
//   * lane `sub` (0..15) of a row owns dims [8*sub, 8*sub+8): one 16-byte load and one
//     16-byte store per lane, so every access is fully coalesced;
//   * the two RMS statistics are 8-lane butterflies (lanes 0..7 hold dims [0:64),
//     lanes 8..15 hold [64:128));
//   * every rotary partner sits in a fixed other lane of the same row (sub^4 in the
//     temporal slice, sub^2 in the height/width slices) and is fetched by a lane swap;
//   * the 8 angles a lane needs depend only on the token, so they are computed once per
//     token and reused for all Hq + Hkv rows.  The angle is formed in fp64 revolutions
//     and reduced to [-1/2, 1/2] before the fp32 sincospi, so it stays accurate for
//     large temporal positions;
//   * fp32 arithmetic, one rounding to the output dtype after the rotary.
#include "neo_internal.h"

#include <math.h>

namespace neo {
namespace {

template <bool kBf16>
struct RowIO;

template <>
struct RowIO<true> {
  static __device__ __forceinline__ void load(const void* base, int64_t row, int sub, float v[8]) {
    const uint4 w = *(reinterpret_cast<const uint4*>(
        static_cast<const uint16_t*>(base) + row * kHeadDim + sub * 8));
    v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x);
    v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
    v[4] = bf16_lo(w.z); v[5] = bf16_hi(w.z);
    v[6] = bf16_lo(w.w); v[7] = bf16_hi(w.w);
  }
  static __device__ __forceinline__ void store(void* base, int64_t row, int sub, const float v[8]) {
    uint4 w;
    w.x = pack_bf16x2(v[0], v[1]);
    w.y = pack_bf16x2(v[2], v[3]);
    w.z = pack_bf16x2(v[4], v[5]);
    w.w = pack_bf16x2(v[6], v[7]);
    *(reinterpret_cast<uint4*>(static_cast<uint16_t*>(base) + row * kHeadDim + sub * 8)) = w;
  }
};

template <>
struct RowIO<false> {
  static __device__ __forceinline__ void load(const void* base, int64_t row, int sub, float v[8]) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) +
                                                      row * kHeadDim + sub * 8);
    const float4 a = p[0], b = p[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  static __device__ __forceinline__ void store(void* base, int64_t row, int sub, const float v[8]) {
    float4* p = reinterpret_cast<float4*>(static_cast<float*>(base) + row * kHeadDim + sub * 8);
    p[0] = make_float4(v[0], v[1], v[2], v[3]);
    p[1] = make_float4(v[4], v[5], v[6], v[7]);
  }
};

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

// r_t = rope_theta^(-2/64), r_hw = rope_theta_hw^(-2/32): the frequency of pair i in a
// slice is r^i.  Both are formed on the host in fp64.
template <bool kBf16>
__global__ __launch_bounds__(kThreads) void qknorm_rope3_kernel(
    const void* q_in, const void* k_in, void* q_out, void* k_out, int64_t ntok, int Hq,
    int Hkv, const float* __restrict__ wq_t, const float* __restrict__ wq_hw,
    const float* __restrict__ wk_t, const float* __restrict__ wk_hw,
    const int32_t* __restrict__ pos, double r_t, double r_hw, float eps) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int sub = lane & 15;  // which 8 dims of the row
  const int grp = lane >> 4;  // which of the 4 rows in flight
  const int half = sub >> 3;  // 0: dims [0:64) temporal half, 1: dims [64:128)
  const int axis = sub < 8 ? 0 : (sub < 12 ? 1 : 2);
  // first element of a rotary pair gets  a*cos - b*sin, the second  b*cos + a*sin
  const bool first = sub < 8 ? (sub & 4) == 0 : (sub & 2) == 0;
  const float sgn = first ? -1.0f : 1.0f;
  const int partner_xor = sub < 8 ? 4 : 2;

  // norm weights for this lane's 8 dims
  float wq[8], wk[8];
  {
    const int off = (sub & 7) * 8;
    const float* pq = half ? wq_hw : wq_t;
    const float* pk = half ? wk_hw : wk_t;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      wq[e] = pq[off + e];
      wk[e] = pk[off + e];
    }
  }
  // frequencies in revolutions per unit position: r^i / (2 pi), i = pair index
  double inv_rev[8];
  {
    const int i0 = sub < 8 ? (sub * 8) & 31 : ((sub - 8) * 8) & 15;
    const double r = axis == 0 ? r_t : r_hw;
    double pw = 1.0, base = r;
    for (int k = i0; k > 0; k >>= 1) {  // r^i0 by binary powering
      if (k & 1) pw *= base;
      base *= base;
    }
    constexpr double kInv2Pi = 0.15915494309189533576888376337251436;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      inv_rev[e] = pw * kInv2Pi;
      pw *= r;
    }
  }

  const int rows = Hq + Hkv;
  for (int64_t t = (int64_t)blockIdx.x * kWaves + wave; t < ntok;
       t += (int64_t)gridDim.x * kWaves) {
    float cs[8], sn[8];
    {
      const double p = (double)pos[(int64_t)axis * ntok + t];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        double rev = p * inv_rev[e];
        rev -= rint(rev);  // exact: the angle modulo one turn, in [-1/2, 1/2]
        sincospif((float)(2.0 * rev), &sn[e], &cs[e]);
      }
    }
    // rows in batches of 16 (four per 16-lane group): the batch's loads are all issued
    // before its first store, so four loads per lane are in flight (each row is still
    // loaded before it is stored, which keeps the in-place call correct)
    for (int r0 = 0; r0 < rows; r0 += 16) {
      float x[4][8];
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        const int r = r0 + 4 * gi + grp;
        if (r < rows) {
          if (r < Hq)
            RowIO<kBf16>::load(q_in, t * Hq + r, sub, x[gi]);
          else
            RowIO<kBf16>::load(k_in, t * Hkv + (r - Hq), sub, x[gi]);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) x[gi][e] = 0.0f;
        }
      }
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        const int r = r0 + 4 * gi + grp;
        const bool valid = r < rows;
        const bool is_q = r < Hq;
        float ss = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) ss = fmaf(x[gi][e], x[gi][e], ss);
        ss += __shfl_xor(ss, 1);
        ss += __shfl_xor(ss, 2);
        ss += __shfl_xor(ss, 4);
        const float rinv = rsqrtf(ss * (1.0f / kHalfDim) + eps);
        float y[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = x[gi][e] * rinv * (is_q ? wq[e] : wk[e]);
        float out[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float yp = __shfl_xor(y[e], partner_xor);
          out[e] = fmaf(y[e], cs[e], sgn * yp * sn[e]);
        }
        if (valid) {
          if (is_q)
            RowIO<kBf16>::store(q_out, t * Hq + r, sub, out);
          else
            RowIO<kBf16>::store(k_out, t * Hkv + (r - Hq), sub, out);
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_qknorm_rope3(bool bf16, const void* q_in, const void* k_in, void* q_out,
                               void* k_out, int64_t T, int Hq, int Hkv, const float* wq_t,
                               const float* wq_hw, const float* wk_t, const float* wk_hw,
                               const int32_t* pos, double theta, double theta_hw, float eps,
                               hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const double r_t = pow(theta, -2.0 / 64.0);
  const double r_hw = pow(theta_hw, -2.0 / 32.0);
  // one wave per token, at most 8 workgroups of 4 waves per CU on 256 CUs
  int64_t blocks = (T + kWaves - 1) / kWaves;
  if (blocks > 256 * 8) blocks = 256 * 8;
  dim3 grid((unsigned)blocks), block(kThreads);
  if (bf16)
    hipLaunchKernelGGL(qknorm_rope3_kernel<true>, grid, block, 0, stream, q_in, k_in, q_out,
                       k_out, T, Hq, Hkv, wq_t, wq_hw, wk_t, wk_hw, pos, r_t, r_hw, eps);
  else
    hipLaunchKernelGGL(qknorm_rope3_kernel<false>, grid, block, 0, stream, q_in, k_in, q_out,
                       k_out, T, Hq, Hkv, wq_t, wq_hw, wk_t, wk_hw, pos, r_t, r_hw, eps);
  return hipGetLastError();
}

}  // namespace neo
