// Internal declarations shared by the HIP translation units of libneo.
// Nothing here is part of the public ABI (that is include/neo.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace neo {

constexpr int kHeadDim = 128;
constexpr int kHalfDim = 64;

// threads per workgroup of the attention (bf16 / fp32) and matrix-product (projection,
// front-end convolution) launches; a launch's work-items (workgroups x threads) must fit
// the dispatch's 32-bit grid size
constexpr int kAttnBf16Threads = 512;
constexpr int kAttnF32Threads = 256;
constexpr int kGemmThreads = 512;

// ---- launchers (host side); each returns the hipError_t of its launch --------------

hipError_t launch_qknorm_rope3(bool bf16, const void* q_in, const void* k_in, void* q_out,
                               void* k_out, int64_t T, int Hq, int Hkv, const float* wq_t,
                               const float* wq_hw, const float* wk_t, const float* wk_hw,
                               const int32_t* pos, double theta, double theta_hw, float eps,
                               hipStream_t stream);

hipError_t launch_gen_attn_bf16(const void* q, const void* k_img, const void* v_img,
                                const void* k_pre, const void* v_pre, const int32_t* cu_q,
                                const int32_t* cu_p, int B, int Hq, int Hkv, int max_q,
                                int max_p, float scale, void* out, float* lse, int64_t Tq,
                                int64_t Tp, hipStream_t stream);

hipError_t launch_prefill_attn_bf16(const void* q, const void* k, const void* v,
                                    const int32_t* tidx, const int32_t* cu, int B, int Hq,
                                    int Hkv, int max_len, float scale, void* out, float* lse,
                                    int64_t T, hipStream_t stream);

hipError_t launch_gen_attn_f32(const float* q, const float* k_img, const float* v_img,
                               const float* k_pre, const float* v_pre, const int32_t* cu_q,
                               const int32_t* cu_p, int B, int Hq, int Hkv, int max_q, int max_p,
                               float scale, float* out, float* lse, int64_t Tq, int64_t Tp,
                               hipStream_t stream);

hipError_t launch_qkv_proj_bf16(const void* x, const void* w, int64_t N, int hidden, int Hq,
                                int Hkv, const float* wq_t, const float* wq_hw, const float* wk_t,
                                const float* wk_hw, const int32_t* pos, double theta,
                                double theta_hw, float eps, void* q_out, void* k_out,
                                void* v_out, hipStream_t stream);

// upper bound of the workgroups a matrix-product launch uses for F features by T tokens
inline int64_t gemm_max_blocks(int64_t F, int64_t T) { return 2 * ((F + 255) / 256) * ((T + 255) / 256); }

// generation-branch embedding front end
hipError_t launch_gen_patchify(const float* z, int B, int H, int W, void* patches,
                               hipStream_t stream);
hipError_t launch_gen_patch_embed(const void* patches, int B, int H, int W, const void* w1,
                                  const float* b1, int C1, double theta, void* h,
                                  hipStream_t stream);
hipError_t launch_gen_patch_embed_px(const float* z, int B, int H, int W, const void* w1,
                                     const float* b1, int C1, double theta, void* h,
                                     hipStream_t stream);
hipError_t launch_gen_cond_hidden(float arg_t, float arg_s, int D, const void* wa_t,
                                  const float* ba_t, const void* wa_s, const float* ba_s,
                                  float* hidden, hipStream_t stream);
hipError_t launch_gen_cond_out(int D, const float* hidden, const void* wb_t, const float* bb_t,
                               const void* wb_s, const float* bb_s, float* cond,
                               hipStream_t stream);
hipError_t launch_gen_merge_embed(const void* h, int B, int H, int W, int C1, const void* w2,
                                  const float* b2, const float* cond, int D, float* tokens,
                                  hipStream_t stream);

hipError_t launch_euler_step(float* z, const float* x0, int64_t n, float coef,
                             hipStream_t stream);

// z <- z + coef * (sum_b w[b] * x[b] - z) over nb = 1..3 branch inputs
hipError_t launch_euler_step_cfg(float* z, const float* const x[3], const float w[3], int nb,
                                 int64_t n, float coef, hipStream_t stream);

// ---- device helpers -----------------------------------------------------------------

// bf16 <-> fp32 on raw 16-bit patterns.  The conversion to bf16 rounds to nearest
// even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// sin and cos of 2 pi rev for an angle given in turns, |rev| <= 2^20.  The angle is reduced
// to r = rev - round(rev) in [-1/2, 1/2] (exact: rev and round(rev) lie within a factor of
// two of each other, or the rounding is 0), then taken by the hardware sine and cosine,
// whose input is in turns: on [-1/2, 1/2] they are within 1.3e-7 of the true values
// (measured against fp64 on 2^22 evenly spaced points).
__device__ __forceinline__ void sincos_turns(float rev, float* s, float* c) {
  const float r = rev - rintf(rev);
  *s = __builtin_amdgcn_sinf(r);
  *c = __builtin_amdgcn_cosf(r);
}

// XCD-aware remap of the linear workgroup id.  Workgroups are handed to the 8 XCDs
// round-robin, so consecutive logical ids would land on different L2s.  This maps the
// hardware order onto contiguous logical ranges per XCD, so workgroups that read the
// same K/V run behind the same L2.  A bijection for any total count.
__device__ __forceinline__ uint32_t xcd_remap(uint32_t lin, uint32_t total) {
  constexpr uint32_t kXcd = 8;
  uint32_t q = total / kXcd, r = total % kXcd;
  uint32_t xcd = lin % kXcd, idx = lin / kXcd;
  return xcd < r ? xcd * (q + 1) + idx : r * (q + 1) + (xcd - r) * q + idx;
}

}  // namespace neo
