// x0-prediction to velocity plus one Euler step of the pixel-space rectified flow.
//
// "SenseNova-U1.5 (NEO-unify) architecture", §Flow matching without a VAE: the pixel
// head predicts the clean image x0; the sampler forms v = (x0 - z) / max(1 - t, t_eps)
// and steps z <- z + (t_next - t) * v.  patchify is a permutation, so the update is
// elementwise on the flat pixel array.
//
// HBM-bound (12 B per element: read z and x0, write z).  The scalar
// c = (t_next - t) / max(1 - t, t_eps) is formed once on the host in fp64 and each
// element does z + c * (x0 - z) in fp32 with a fused multiply-add.  16-byte vector
// accesses when both pointers allow it, a scalar path otherwise.
#include "neo_internal.h"

namespace neo {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void euler_vec4_kernel(float4* z, const float4* x0,
                                                              int64_t n4, float c) {
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (; i < n4; i += stride) {
    float4 a = z[i];
    const float4 b = x0[i];
    a.x = fmaf(c, b.x - a.x, a.x);
    a.y = fmaf(c, b.y - a.y, a.y);
    a.z = fmaf(c, b.z - a.z, a.z);
    a.w = fmaf(c, b.w - a.w, a.w);
    z[i] = a;
  }
}

__global__ __launch_bounds__(kThreads) void euler_scalar_kernel(float* z, const float* x0,
                                                                int64_t n, float c) {
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (; i < n; i += stride) z[i] = fmaf(c, x0[i] - z[i], z[i]);
}

int64_t grid_for(int64_t items) {
  int64_t blocks = (items + kThreads - 1) / kThreads;
  // enough workgroups to fill 256 CUs many times over; the loop covers the rest
  const int64_t cap = 256 * 16;
  return blocks < 1 ? 1 : (blocks > cap ? cap : blocks);
}

}  // namespace

hipError_t launch_euler_step(float* z, const float* x0, int64_t n, float coef,
                             hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const bool aligned = ((reinterpret_cast<uintptr_t>(z) | reinterpret_cast<uintptr_t>(x0)) & 15) == 0;
  const int64_t n4 = aligned ? n / 4 : 0;
  if (n4 > 0) {
    hipLaunchKernelGGL(euler_vec4_kernel, dim3((unsigned)grid_for(n4)), dim3(kThreads), 0, stream,
                       reinterpret_cast<float4*>(z), reinterpret_cast<const float4*>(x0), n4,
                       coef);
  }
  const int64_t done = n4 * 4;
  if (done < n) {
    hipLaunchKernelGGL(euler_scalar_kernel, dim3((unsigned)grid_for(n - done)), dim3(kThreads), 0,
                       stream, z + done, x0 + done, n - done, coef);
  }
  return hipGetLastError();
}

}  // namespace neo
