// Generation-pass attention: image queries over [frozen prefix ; image block], no mask,
// no cache write, grouped-query heads.
//
// "SenseNova-U1.5 (NEO-unify) architecture": §Mixture of Transformers (the generation
// pass reads the keys/values the understanding pass wrote and does not update the
// cache) and §GQA fusion does not apply (the generation pass is unmasked).  For query
// head h the KV head is h / (Hq / Hkv).  The frozen cache is token-major [S, H, D]
// ("SenseNova-U1 ... NEO-unify Architecture" paper notes, §4.4 KV cache reuse); the
// prefix and the image block are two separate segments read in place, no concatenation.
//
// bf16 kernel (the production path), one workgroup of 4 waves per
// (sample, KV head, group of 4 chunks); a chunk is 32 query tokens of one query head:
//   * the 4 chunks of a workgroup share one KV head, so every K/V tile staged in LDS
//     feeds 4 waves (with Hq/Hkv = 4 these are the 4 query heads of one KV group over
//     the same 32 tokens);
//   * scores are formed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: A = a
//     32-key slice of the K tile (rows = keys), B = the wave's Q^T held in registers.
//     In the 32x32 accumulator layout each lane then holds one query (lane % 32) and
//     16 keys, so the softmax row statistics are in-lane plus one swap with lane ^ 32;
//   * the same layout is exactly the B operand of O^T = V^T P^T, so P goes from the
//     score accumulator to the second MFMA without any data movement.  V is staged in
//     LDS transposed ([dim][key]) so each lane reads its keys with two 8-byte loads;
//   * online softmax in fp32 on exp2 with the 1/sqrt(d) * log2(e) scale folded into one
//     FMA; the row sum adds the bf16-rounded weights that the PV product uses.  The
//     running maximum is raised only when a tile's maximum exceeds it by more than 2^8,
//     so the O rescale (64 multiplies per lane) runs on the first tile and almost never
//     afterwards, while every exponent stays <= 2^8; the final O / l is
//     the same quotient whichever reference maximum was used;
//   * K/V tiles of 64 keys are double-buffered in LDS (2 x 34 KB); the next tile's
//     global loads are issued before the current tile's MFMAs and written to the other
//     buffer afterwards, one barrier per tile;
//   * key rows past the sample's end are zero-filled and their scores set to -inf;
//   * the workgroup order is remapped so each XCD works on contiguous (sample, KV head)
//     ranges and its L2 holds that head's K/V.
//
// fp32 kernel: a plain online-softmax kernel on the vector ALUs (two lanes per query
// row, 64 dims each), for fp32 inputs where bf16 MFMA would not meet fp32 accuracy.
#include "neo_internal.h"

#include <math.h>

namespace neo {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kBN = 64;                      // keys per tile
constexpr int kKS = kHeadDim + 8;            // K tile row stride (bf16), 272 B
constexpr int kVS = kBN + 4;                 // V^T tile row stride (bf16), 136 B
constexpr int kKTile = kBN * kKS;            // bf16 elements
constexpr int kVTile = kHeadDim * kVS;       // bf16 elements
constexpr int kStage = kKTile + kVTile;      // one K + V^T stage
constexpr float kTau = 8.0f;                 // lazy-rescale threshold (log2 units)
constexpr bf16x2 kOnes2 = {(__bf16)1.0f, (__bf16)1.0f};

struct TileRegs {
  uint4 k[4];
  uint4 v[4];
};

struct SampleView {
  const uint16_t* k_pre;
  const uint16_t* v_pre;
  const uint16_t* k_img;
  const uint16_t* v_img;
  int64_t p0, i0;  // first prefix row, first image row of the sample
  int P, Lk;       // prefix length, total keys
  int Hkv, g;
};

__device__ __forceinline__ uint4 load_key_row(const SampleView& s, const uint16_t* pre,
                                              const uint16_t* img, int j, int dg) {
  const uint16_t* row = nullptr;
  if (j < s.P)
    row = pre + ((s.p0 + j) * s.Hkv + s.g) * kHeadDim;
  else if (j < s.Lk)
    row = img + ((s.i0 + (j - s.P)) * s.Hkv + s.g) * kHeadDim;
  if (row == nullptr) return make_uint4(0, 0, 0, 0);
  return *reinterpret_cast<const uint4*>(row + dg * 8);
}

// K rows: thread (dg = tid % 16, r = tid / 16) loads rows r, r+16, r+32, r+48.
// V rows: the same thread loads the 4 consecutive rows 4r..4r+3 (for the transpose).
__device__ __forceinline__ void load_tile(TileRegs& R, const SampleView& s, int tile, int tid) {
  const int dg = tid & 15, r = tid >> 4;
  const int base = tile * kBN;
#pragma unroll
  for (int i = 0; i < 4; ++i) R.k[i] = load_key_row(s, s.k_pre, s.k_img, base + r + 16 * i, dg);
#pragma unroll
  for (int i = 0; i < 4; ++i) R.v[i] = load_key_row(s, s.v_pre, s.v_img, base + 4 * r + i, dg);
}

__device__ __forceinline__ uint32_t word(const uint4& u, int w) {
  return w == 0 ? u.x : (w == 1 ? u.y : (w == 2 ? u.z : u.w));
}

__device__ __forceinline__ void store_tile(uint16_t* stage, const TileRegs& R, int tid) {
  const int dg = tid & 15, r = tid >> 4;
  uint16_t* Ks = stage;
  uint16_t* VT = stage + kKTile;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    *reinterpret_cast<uint4*>(Ks + (r + 16 * i) * kKS + dg * 8) = R.k[i];
  // transpose: dim 8*dg + e of keys 4r..4r+3 becomes 4 consecutive bf16 of row (8*dg + e)
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int w = e >> 1;
    const uint32_t a0 = word(R.v[0], w), a1 = word(R.v[1], w);
    const uint32_t a2 = word(R.v[2], w), a3 = word(R.v[3], w);
    uint32_t lo, hi;
    if (e & 1) {
      lo = (a0 >> 16) | (a1 & 0xffff0000u);
      hi = (a2 >> 16) | (a3 & 0xffff0000u);
    } else {
      lo = (a0 & 0xffffu) | (a1 << 16);
      hi = (a2 & 0xffffu) | (a3 << 16);
    }
    *reinterpret_cast<uint2*>(VT + (dg * 8 + e) * kVS + 4 * r) = make_uint2(lo, hi);
  }
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

__global__ __launch_bounds__(kThreads, 2) void gen_attn_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_img,
    const uint16_t* __restrict__ v_img, const uint16_t* __restrict__ k_pre,
    const uint16_t* __restrict__ v_pre, const int32_t* __restrict__ cu_q,
    const int32_t* __restrict__ cu_p, int Hq, int Hkv, int n_cg, int max_q, int max_p,
    int64_t Tq, int64_t Tp, float scale_log2, uint16_t* __restrict__ out,
    float* __restrict__ lse) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * kStage];

  const uint32_t id = xcd_remap(blockIdx.x, gridDim.x);
  const int cg = (int)(id % (uint32_t)n_cg);
  const int rest = (int)(id / (uint32_t)n_cg);
  const int g = rest % Hkv;
  const int b = rest / Hkv;

  // sample extents, clamped to the buffers whatever cu_seqlens hold
  int64_t qa = cu_q[b], qb = cu_q[b + 1];
  qa = qa < 0 ? 0 : (qa > Tq ? Tq : qa);
  qb = qb < qa ? qa : (qb > Tq ? Tq : qb);
  int64_t pa = cu_p[b], pb_ = cu_p[b + 1];
  pa = pa < 0 ? 0 : (pa > Tp ? Tp : pa);
  pb_ = pb_ < pa ? pa : (pb_ > Tp ? Tp : pb_);
  const int N = (int)((qb - qa) < max_q ? (qb - qa) : max_q);
  const int P = (int)((pb_ - pa) < max_p ? (pb_ - pa) : max_p);

  const int G = Hq / Hkv;
  const int nchunks = G * ((N + 31) / 32);
  if (cg * kWaves >= nchunks) return;  // whole workgroup idle

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, hl = lane >> 5, col = lane & 31;
  const int c = cg * kWaves + wave;
  const bool active = c < nchunks;
  const int h = g * G + (active ? c % G : 0);
  const int qi = (active ? c / G : 0) * 32 + col;  // query index inside the sample
  const bool qvalid = active && qi < N;

  SampleView sv;
  sv.k_pre = k_pre; sv.v_pre = v_pre; sv.k_img = k_img; sv.v_img = v_img;
  sv.p0 = pa; sv.i0 = qa; sv.P = P; sv.Lk = P + N; sv.Hkv = Hkv; sv.g = g;

  // this lane's slice of Q^T: query qi, dims 16*s + 8*hl .. +7 for k-step s
  bf16x8 qf[8];
  if (qvalid) {
    const uint16_t* qr = q + ((qa + qi) * Hq + h) * kHeadDim + 8 * hl;
#pragma unroll
    for (int s = 0; s < 8; ++s) qf[s] = as_bf16x8(*reinterpret_cast<const uint4*>(qr + 16 * s));
  } else {
#pragma unroll
    for (int s = 0; s < 8; ++s) qf[s] = as_bf16x8(make_uint4(0, 0, 0, 0));
  }

  f32x16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.0f;
  float m = -INFINITY, lsum = 0.0f;

  const int Lk = sv.Lk;
  const int ntiles = (Lk + kBN - 1) / kBN;
  TileRegs R;
  load_tile(R, sv, 0, tid);
  store_tile(smem, R, tid);
  __syncthreads();

  for (int it = 0; it < ntiles; ++it) {
    const uint16_t* Ks = smem + (it & 1) * kStage;
    const uint16_t* VT = Ks + kKTile;
    const bool more = it + 1 < ntiles;
    if (more) load_tile(R, sv, it + 1, tid);

    if (active) {
      f32x16 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] = 0.0f;
        const uint16_t* krow = Ks + (kb * 32 + col) * kKS + 8 * hl;
#pragma unroll
        for (int st = 0; st < 8; ++st) {
          const bf16x8 a = as_bf16x8(*reinterpret_cast<const uint4*>(krow + 16 * st));
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[st], s[kb], 0, 0, 0);
        }
      }
      // keys past the end of the sample (last tile only)
      if ((it + 1) * kBN > Lk) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = it * kBN + kb * 32 + (r >> 2) * 8 + hl * 4 + (r & 3);
            if (key >= Lk) s[kb][r] = -INFINITY;
          }
      }
      float mx = s[0][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mx2 = mx * scale_log2;
      const bool need = mx2 > m + kTau;
      if (__ballot(need) != 0) {
        const float mnew = need ? mx2 : m;
        const float alpha = __builtin_amdgcn_exp2f(m - mnew);
        lsum *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
        m = mnew;
      }
      // P in bf16; the row sum adds the same rounded weights (v_dot2 against (1, 1)),
      // so the normalised weights sum to one exactly and a near one-hot softmax
      // returns the dominant value without the weight's rounding error
      bf16x8 pb[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        uint32_t pk[4];
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(s[u >> 1][(u & 1) * 8 + e], scale_log2, -m));
          const float p1 =
              __builtin_amdgcn_exp2f(fmaf(s[u >> 1][(u & 1) * 8 + e + 1], scale_log2, -m));
          pk[e >> 1] = pack_bf16x2(p0, p1);
          lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[e >> 1]), kOnes2,
                                                 lsum, false);
        }
        pb[u] = as_bf16x8(make_uint4(pk[0], pk[1], pk[2], pk[3]));
      }
      // O^T += V^T P^T: k-slot (hl, e) of step u is key 32*(u/2) + 16*(u%2) + 4*hl + 8*(e/4) + e%4
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const uint16_t* vrow = VT + (db * 32 + col) * kVS + 4 * hl;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int kbase = 32 * (u >> 1) + 16 * (u & 1);
          const uint2 lo = *reinterpret_cast<const uint2*>(vrow + kbase);
          const uint2 hi = *reinterpret_cast<const uint2*>(vrow + kbase + 8);
          const bf16x8 a = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[u], o[db], 0, 0, 0);
        }
      }
    }
    if (more) store_tile(smem + ((it + 1) & 1) * kStage, R, tid);
    __syncthreads();
  }

  const float ltot = lsum + __shfl_xor(lsum, 32);
  if (qvalid) {
    const float inv = 1.0f / ltot;
    uint16_t* orow = out + ((qa + qi) * Hq + h) * kHeadDim + 4 * hl;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const uint32_t w0 = pack_bf16x2(o[db][rg * 4 + 0] * inv, o[db][rg * 4 + 1] * inv);
        const uint32_t w1 = pack_bf16x2(o[db][rg * 4 + 2] * inv, o[db][rg * 4 + 3] * inv);
        *reinterpret_cast<uint2*>(orow + db * 32 + rg * 8) = make_uint2(w0, w1);
      }
    if (lse != nullptr && hl == 0)
      lse[(int64_t)h * Tq + qa + qi] = (m + __log2f(ltot)) * 0.69314718055994530942f;
  }
}

// ---------------------------------------------------------------------------------------
// fp32 path
// ---------------------------------------------------------------------------------------
constexpr int kF32Keys = 32;

__global__ __launch_bounds__(kThreads) void gen_attn_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k_img, const float* __restrict__ v_img,
    const float* __restrict__ k_pre, const float* __restrict__ v_pre,
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_p, int Hq, int Hkv,
    int n_rb, int max_q, int max_p, int64_t Tq, int64_t Tp, float scale,
    float* __restrict__ out, float* __restrict__ lse) {
  __shared__ float Ks[kF32Keys][kHeadDim];
  __shared__ float Vs[kF32Keys][kHeadDim];
  const uint32_t id = xcd_remap(blockIdx.x, gridDim.x);
  const int rb = (int)(id % (uint32_t)n_rb);
  const int rest = (int)(id / (uint32_t)n_rb);
  const int g = rest % Hkv;
  const int b = rest / Hkv;

  int64_t qa = cu_q[b], qb = cu_q[b + 1];
  qa = qa < 0 ? 0 : (qa > Tq ? Tq : qa);
  qb = qb < qa ? qa : (qb > Tq ? Tq : qb);
  int64_t pa = cu_p[b], pb_ = cu_p[b + 1];
  pa = pa < 0 ? 0 : (pa > Tp ? Tp : pa);
  pb_ = pb_ < pa ? pa : (pb_ > Tp ? Tp : pb_);
  const int N = (int)((qb - qa) < max_q ? (qb - qa) : max_q);
  const int P = (int)((pb_ - pa) < max_p ? (pb_ - pa) : max_p);
  const int G = Hq / Hkv;
  const int rows = N * G;
  const int rows_per_block = kThreads / 2;
  if (rb * rows_per_block >= rows) return;

  const int tid = threadIdx.x;
  const int half = tid & 1;
  const int row = rb * rows_per_block + (tid >> 1);
  const bool valid = row < rows;
  const int tok = valid ? row / G : 0;
  const int h = g * G + (valid ? row % G : 0);

  float qv[64], ov[64];
  const float* qr = q + ((qa + tok) * Hq + h) * kHeadDim + half * 64;
#pragma unroll
  for (int d = 0; d < 64; ++d) {
    qv[d] = valid ? qr[d] : 0.0f;
    ov[d] = 0.0f;
  }
  float m = -INFINITY, l = 0.0f;
  const int Lk = P + N;
  for (int k0 = 0; k0 < Lk; k0 += kF32Keys) {
    for (int e = tid; e < kF32Keys * kHeadDim; e += kThreads) {
      const int j = k0 + e / kHeadDim, d = e % kHeadDim;
      float kv = 0.0f, vv = 0.0f;
      if (j < P) {
        kv = k_pre[((pa + j) * Hkv + g) * kHeadDim + d];
        vv = v_pre[((pa + j) * Hkv + g) * kHeadDim + d];
      } else if (j < Lk) {
        kv = k_img[((qa + j - P) * Hkv + g) * kHeadDim + d];
        vv = v_img[((qa + j - P) * Hkv + g) * kHeadDim + d];
      }
      Ks[e / kHeadDim][d] = kv;
      Vs[e / kHeadDim][d] = vv;
    }
    __syncthreads();
    float s[kF32Keys];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < kF32Keys; ++j) {
      float dot = 0.0f;
#pragma unroll
      for (int d = 0; d < 64; ++d) dot = fmaf(qv[d], Ks[j][half * 64 + d], dot);
      dot += __shfl_xor(dot, 1);
      s[j] = (k0 + j < Lk) ? dot * scale : -INFINITY;
      mx = fmaxf(mx, s[j]);
    }
    const float mnew = fmaxf(m, mx);
    const float alpha = expf(m - mnew);
    l *= alpha;
#pragma unroll
    for (int d = 0; d < 64; ++d) ov[d] *= alpha;
#pragma unroll
    for (int j = 0; j < kF32Keys; ++j) {
      const float p = expf(s[j] - mnew);
      l += p;
#pragma unroll
      for (int d = 0; d < 64; ++d) ov[d] = fmaf(p, Vs[j][half * 64 + d], ov[d]);
    }
    m = mnew;
    __syncthreads();
  }
  if (valid) {
    float* orow = out + ((qa + tok) * Hq + h) * kHeadDim + half * 64;
    const float inv = 1.0f / l;
#pragma unroll
    for (int d = 0; d < 64; ++d) orow[d] = ov[d] * inv;
    if (lse != nullptr && half == 0) lse[(int64_t)h * Tq + qa + tok] = m + logf(l);
  }
}

}  // namespace

hipError_t launch_gen_attn_bf16(const void* q, const void* k_img, const void* v_img,
                                const void* k_pre, const void* v_pre, const int32_t* cu_q,
                                const int32_t* cu_p, int B, int Hq, int Hkv, int max_q,
                                int max_p, float scale, void* out, float* lse, int64_t Tq,
                                int64_t Tp, hipStream_t stream) {
  if (max_q == 0 || Tq == 0) return hipSuccess;
  const int G = Hq / Hkv;
  const int64_t chunks = (int64_t)G * ((max_q + 31) / 32);
  const int64_t n_cg = (chunks + kWaves - 1) / kWaves;
  const int64_t blocks = n_cg * Hkv * B;
  const float scale_log2 = (float)((double)scale * 1.4426950408889634073599246810019);
  hipLaunchKernelGGL(gen_attn_bf16_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k_img),
                     static_cast<const uint16_t*>(v_img), static_cast<const uint16_t*>(k_pre),
                     static_cast<const uint16_t*>(v_pre), cu_q, cu_p, Hq, Hkv, (int)n_cg,
                     max_q, max_p, Tq, Tp, scale_log2, static_cast<uint16_t*>(out), lse);
  return hipGetLastError();
}

hipError_t launch_gen_attn_f32(const float* q, const float* k_img, const float* v_img,
                               const float* k_pre, const float* v_pre, const int32_t* cu_q,
                               const int32_t* cu_p, int B, int Hq, int Hkv, int max_q, int max_p,
                               float scale, float* out, float* lse, int64_t Tq, int64_t Tp,
                               hipStream_t stream) {
  if (max_q == 0 || Tq == 0) return hipSuccess;
  const int G = Hq / Hkv;
  const int64_t rows = (int64_t)max_q * G;
  const int64_t n_rb = (rows + kThreads / 2 - 1) / (kThreads / 2);
  const int64_t blocks = n_rb * Hkv * B;
  hipLaunchKernelGGL(gen_attn_f32_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, q,
                     k_img, v_img, k_pre, v_pre, cu_q, cu_p, Hq, Hkv, (int)n_rb, max_q, max_p, Tq,
                     Tp, scale, out, lse);
  return hipGetLastError();
}

}  // namespace neo
