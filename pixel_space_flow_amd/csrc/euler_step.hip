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

// Guided step over NB = 1..3 branch predictions of x0 (classifier-free guidance fused
// with the Euler update; "SenseNova-U1 ... NEO-unify Architecture" paper notes, §2.7).
// The guidance weights w sum to one, so the guided x0 is sum_b w_b x_b and the step is
// the plain Euler update on it: z + c * (sum_b w_b x_b - z).  HBM-bound: 4 (NB + 2) bytes
// per element.
template <int NB>
__global__ __launch_bounds__(kThreads) void euler_cfg_vec4_kernel(
    float4* z, const float4* x0, const float4* x1,
    const float4* x2, int64_t n4, float w0, float w1, float w2, float c) {
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (; i < n4; i += stride) {
    float4 a = z[i];
    const float4 p = x0[i];
    float4 g = make_float4(w0 * p.x, w0 * p.y, w0 * p.z, w0 * p.w);
    if (NB > 1) {
      const float4 q = x1[i];
      g.x = fmaf(w1, q.x, g.x);
      g.y = fmaf(w1, q.y, g.y);
      g.z = fmaf(w1, q.z, g.z);
      g.w = fmaf(w1, q.w, g.w);
    }
    if (NB > 2) {
      const float4 r = x2[i];
      g.x = fmaf(w2, r.x, g.x);
      g.y = fmaf(w2, r.y, g.y);
      g.z = fmaf(w2, r.z, g.z);
      g.w = fmaf(w2, r.w, g.w);
    }
    a.x = fmaf(c, g.x - a.x, a.x);
    a.y = fmaf(c, g.y - a.y, a.y);
    a.z = fmaf(c, g.z - a.z, a.z);
    a.w = fmaf(c, g.w - a.w, a.w);
    z[i] = a;
  }
}

template <int NB>
__global__ __launch_bounds__(kThreads) void euler_cfg_scalar_kernel(
    float* z, const float* x0, const float* x1,
    const float* x2, int64_t n, float w0, float w1, float w2, float c) {
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (; i < n; i += stride) {
    float g = w0 * x0[i];
    if (NB > 1) g = fmaf(w1, x1[i], g);
    if (NB > 2) g = fmaf(w2, x2[i], g);
    z[i] = fmaf(c, g - z[i], z[i]);
  }
}

int64_t grid_for(int64_t items) {
  int64_t blocks = (items + kThreads - 1) / kThreads;
  // enough workgroups to fill 256 CUs many times over (32 per CU measured best for
  // streaming float4 passes at 50 MB per array); the loop covers the rest
  const int64_t cap = 256 * 32;
  return blocks < 1 ? 1 : (blocks > cap ? cap : blocks);
}

template <int NB>
hipError_t launch_cfg(float* z, const float* const x[3], const float w[3], int64_t n, float c,
                      hipStream_t stream) {
  uintptr_t bits = reinterpret_cast<uintptr_t>(z);
  for (int b = 0; b < NB; ++b) bits |= reinterpret_cast<uintptr_t>(x[b]);
  const int64_t n4 = (bits & 15) == 0 ? n / 4 : 0;
  // pointers of branches this instantiation does not read are never dereferenced
  const float* x1 = NB > 1 ? x[1] : x[0];
  const float* x2 = NB > 2 ? x[2] : x[0];
  if (n4 > 0) {
    hipLaunchKernelGGL(euler_cfg_vec4_kernel<NB>, dim3((unsigned)grid_for(n4)), dim3(kThreads), 0,
                       stream, reinterpret_cast<float4*>(z), reinterpret_cast<const float4*>(x[0]),
                       reinterpret_cast<const float4*>(x1), reinterpret_cast<const float4*>(x2),
                       n4, w[0], w[1], w[2], c);
  }
  const int64_t done = n4 * 4;
  if (done < n) {
    hipLaunchKernelGGL(euler_cfg_scalar_kernel<NB>, dim3((unsigned)grid_for(n - done)),
                       dim3(kThreads), 0, stream, z + done, x[0] + done, x1 + done, x2 + done,
                       n - done, w[0], w[1], w[2], c);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_euler_step_cfg(float* z, const float* const x[3], const float w[3], int nb,
                                 int64_t n, float coef, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  switch (nb) {
    case 1: return launch_cfg<1>(z, x, w, n, coef, stream);
    case 2: return launch_cfg<2>(z, x, w, n, coef, stream);
    default: return launch_cfg<3>(z, x, w, n, coef, stream);
  }
}

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
