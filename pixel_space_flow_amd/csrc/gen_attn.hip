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
// bf16 kernel (the production path): one workgroup of 8 waves per (sample, KV head,
// group of 8 chunks); a chunk is 32 query tokens of one query head.
//   * the 8 chunks of a workgroup share one KV head, so every K/V tile staged in LDS
//     feeds 8 waves (with Hq/Hkv = 4: the 4 query heads of one KV group over 64 tokens);
//   * scores are formed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: A = a
//     32-key slice of the K tile (rows = keys), B = the wave's Q^T held in registers.
//     In the 32x32 accumulator layout each lane then holds one query (lane % 32) and
//     16 keys, so the softmax row statistics are in-lane plus one swap with lane ^ 32;
//   * the same layout is exactly the B operand of O^T = V^T P^T, so P goes from the
//     score accumulator to the second MFMA without any data movement.  V stays
//     row-major in LDS and is read with ds_read_b64_tr_b16, whose 16-lane transpose
//     hands each lane 4 consecutive keys of one dim;
//   * LDS rows are XOR-swizzled at 16-byte granularity (no padding), which keeps the
//     staging writes, the K reads and the transposed V reads free of bank conflicts;
//   * waves w and w+4 share a SIMD; the upper four run half a tile behind (the PV
//     product of the previous tile first), so one wave's softmax overlaps the other's
//     matrix products instead of both waves contending for the same unit at once;
//   * online softmax in fp32 on exp2 with the 1/sqrt(d) * log2(e) scale folded into one
//     FMA; the row sum adds the bf16-rounded weights that the PV product uses.  The
//     running maximum is raised only when a tile's maximum exceeds it by more than 2^8,
//     so the O rescale (64 multiplies per lane) runs on the first tile and almost never
//     afterwards, while every exponent stays <= 2^8; the final O / l is the same
//     quotient whichever reference maximum was used;
//   * K/V tiles of 64 keys from raw buffer loads: the resource of each tile ends at its
//     segment's end, so rows past it read as zeros (their scores are then set to -inf)
//     with no per-row address arithmetic.  Three LDS stages; the next tile's loads are
//     in flight during the current tile's math, one barrier per tile;
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

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kThreads = 512;                // 8 waves, two per SIMD
constexpr int kWaves = kThreads / 64;
constexpr int kBN = 64;                      // keys per tile
constexpr int kRowBytes = kHeadDim * 2;      // one K or V row in LDS (no padding)
constexpr int kTileBytes = kBN * kRowBytes;  // 16 KB
constexpr float kTwoTau = 256.0f;            // bound on any softmax weight (2^8)
constexpr bf16x2 kOnes2 = {(__bf16)1.0f, (__bf16)1.0f};
constexpr int kBufFlags = 0x00020000;        // raw buffer, 32-bit data format (gfx9 family)

// LDS tiles hold 64 rows of 16 chunks (16 bytes = 8 dims each).  Chunk c of row r is
// stored at slot c ^ swz(r), which makes all three access patterns conflict-free:
// the row-wise 16-byte writes, the K-fragment reads (16 consecutive rows, one chunk)
// and the transposed V reads (4 consecutive rows, 4 consecutive chunks per half-wave).
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)nbytes,
                                           kBufFlags);
}

__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, int voff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0));
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

// Key segments of one (sample, KV head): the frozen prefix, then the image block.
struct Segments {
  const uint8_t* kbase[2];
  const uint8_t* vbase[2];
  int len[2];
  int ntiles[2];
  int64_t row_bytes;    // Hkv * 128 * 2
  uint32_t row_bytes32;
  uint32_t tile_bytes;  // 64 rows
};

// One tile = 64 consecutive rows of one key segment.  The buffer resource starts at the
// tile's first row and ends at the segment's end, so the hardware range check returns
// zeros for rows past the segment: no branches and no per-row address arithmetic.
__device__ __forceinline__ void tile_rsrc(const Segments& S, int it, __amdgpu_buffer_rsrc_t& rk,
                                          __amdgpu_buffer_rsrc_t& rv) {
  const bool pre = it < S.ntiles[0];
  const int tl = pre ? it : it - S.ntiles[0];
  const int rows = (pre ? S.len[0] : S.len[1]) - tl * kBN;
  // one sample's segment spans < 2^31 bytes (checked by the caller), so 32-bit offsets
  const uint32_t off = (uint32_t)tl * S.tile_bytes;
  const uint32_t nbytes = (uint32_t)(rows < kBN ? rows : kBN) * S.row_bytes32;
  rk = make_rsrc((pre ? S.kbase[0] : S.kbase[1]) + off, nbytes);
  rv = make_rsrc((pre ? S.vbase[0] : S.vbase[1]) + off, nbytes);
}

__device__ __forceinline__ int tile_valid(const Segments& S, int it) {
  const int seg = it < S.ntiles[0] ? 0 : 1;
  const int tl = seg == 0 ? it : it - S.ntiles[0];
  return S.len[seg] - tl * kBN;
}

// Staging: thread t moves 16-byte chunks q = t and t + 512 of one K tile and one V tile
// (row q / 16, chunk q % 16) from HBM to registers, then to their swizzled LDS slots.
struct Stage {
  uint4 k[2], v[2];
};

// LDS: two K tiles and two V tiles.  Iteration t computes tile t's scores (K buffer
// t % 2) and tile t-1's PV product (V buffer (t-1) % 2) while tile t+1's K and tile t's
// V are staged into the other buffers.
constexpr int kLdsBytes = 4 * kTileBytes;  // 64 KB

__global__ __launch_bounds__(kThreads, 1) void gen_attn_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_img,
    const uint16_t* __restrict__ v_img, const uint16_t* __restrict__ k_pre,
    const uint16_t* __restrict__ v_pre, const int32_t* __restrict__ cu_q,
    const int32_t* __restrict__ cu_p, int Hq, int Hkv, int n_cg, int max_q, int max_p,
    int64_t Tq, int64_t Tp, float scale_log2, uint16_t* __restrict__ out,
    float* __restrict__ lse) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kLdsBytes];

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

  Segments S;
  S.row_bytes = (int64_t)Hkv * kHeadDim * 2;
  S.row_bytes32 = (uint32_t)S.row_bytes;
  S.tile_bytes = (uint32_t)S.row_bytes * kBN;
  S.kbase[0] = reinterpret_cast<const uint8_t*>(k_pre + (pa * Hkv + g) * kHeadDim);
  S.vbase[0] = reinterpret_cast<const uint8_t*>(v_pre + (pa * Hkv + g) * kHeadDim);
  S.kbase[1] = reinterpret_cast<const uint8_t*>(k_img + (qa * Hkv + g) * kHeadDim);
  S.vbase[1] = reinterpret_cast<const uint8_t*>(v_img + (qa * Hkv + g) * kHeadDim);
  S.len[0] = P;
  S.len[1] = N;
  S.ntiles[0] = (P + kBN - 1) / kBN;
  S.ntiles[1] = (N + kBN - 1) / kBN;
  const int ntiles = S.ntiles[0] + S.ntiles[1];

  // staging offsets: global (inside a tile) and LDS (inside a tile)
  int goff[2], soff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int qc = tid + kThreads * i;
    const int row = qc >> 4, chunk = qc & 15;
    goff[i] = row * (int)S.row_bytes + chunk * 16;
    soff[i] = row * kRowBytes + ((chunk ^ swz(row)) << 4);
  }

  // K-fragment reads (A operand of S^T = K Q^T): row kb*32 + col, chunk 2*st + hl.  The
  // swizzle depends on row % 16 only, so kb adds the constant 32 rows (immediate offset).
  const int j16 = lane & 15, grp = (lane >> 4) & 1;
  int kofs[8];
#pragma unroll
  for (int st = 0; st < 8; ++st) kofs[st] = col * kRowBytes + (((2 * st + hl) ^ swz(col)) << 4);
  // V-fragment reads (A operand of O^T = V^T P^T, transposed): within each 16-lane group,
  // lane j addresses row key0 + j/4 at dims dim0 + 4*(j%4) and receives dim dim0 + j of
  // rows key0 .. key0+3.  For step u, read r and dim block db: key0 = 32*(u/2) + 16*(u%2)
  // + 8*r + 4*hl, dim0 = 32*db + 16*grp.  The u part is a multiple of 16 rows (immediate).
  int vofs[2][4];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int row = 8 * r + 4 * hl + (j16 >> 2);
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int chunk = 4 * db + 2 * grp + ((j16 & 3) >> 1);
      vofs[r][db] = row * kRowBytes + ((chunk ^ swz(row)) << 4) + ((j16 & 1) << 3);
    }
  }

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
  // m: reference maximum (log2 units); every weight exp2(s*c - m) is kept <= 2^8
  float m = -INFINITY, lsum = 0.0f;

  Stage R;
  auto load_k = [&](int t) {
    __amdgpu_buffer_rsrc_t rk, rv;
    tile_rsrc(S, t, rk, rv);
#pragma unroll
    for (int i = 0; i < 2; ++i) R.k[i] = buf_load16(rk, goff[i]);
  };
  auto load_v = [&](int t) {
    __amdgpu_buffer_rsrc_t rk, rv;
    tile_rsrc(S, t, rk, rv);
#pragma unroll
    for (int i = 0; i < 2; ++i) R.v[i] = buf_load16(rv, goff[i]);
  };
  auto store_k = [&](uint8_t* base) {
#pragma unroll
    for (int i = 0; i < 2; ++i) *reinterpret_cast<uint4*>(base + soff[i]) = R.k[i];
  };
  auto store_v = [&](uint8_t* base) {
#pragma unroll
    for (int i = 0; i < 2; ++i) *reinterpret_cast<uint4*>(base + soff[i]) = R.v[i];
  };

  // scores of one tile from the K tile at Ks (16 MFMAs, two interleaved chains)
  auto qk = [&](const uint8_t* Ks, f32x16 (&sacc)[2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.0f;
#pragma unroll
    for (int st = 0; st < 8; ++st)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 a = as_bf16x8(
            *reinterpret_cast<const uint4*>(Ks + kofs[st] + kb * 32 * kRowBytes));
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[st], sacc[kb], 0, 0, 0);
      }
  };

  // keys past the end of the segment (its last tile only) score -inf
  auto mask = [&](int t, f32x16 (&sacc)[2]) {
    const int nvalid = tile_valid(S, t);
    if (nvalid < kBN) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kb * 32 + (r >> 2) * 8 + hl * 4 + (r & 3);
          if (key >= nvalid) sacc[kb][r] = -INFINITY;
        }
    }
  };

  // P = exp2(s*c - m) in bf16 and the row sum of the same rounded weights (v_dot2 against
  // (1, 1)), so the normalised weights sum to one exactly.  Returns this tile's sum.
  auto exp_tile = [&](const f32x16 (&sacc)[2], bf16x8 (&pw)[4]) -> float {
    float tsum = 0.0f;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      uint32_t pk[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[u >> 1][(u & 1) * 8 + e], scale_log2, -m));
        const float p1 =
            __builtin_amdgcn_exp2f(fmaf(sacc[u >> 1][(u & 1) * 8 + e + 1], scale_log2, -m));
        pk[e >> 1] = pack_bf16x2(p0, p1);
        tsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[e >> 1]), kOnes2,
                                               tsum, false);
      }
      pw[u] = as_bf16x8(make_uint4(pk[0], pk[1], pk[2], pk[3]));
    }
    return tsum;
  };

  // O^T += V^T P^T from the V tile at Vs (16 MFMAs, four chains).  k-slot (hl, e) of
  // step u is key 32*(u/2) + 16*(u%2) + 4*hl + 8*(e/4) + e%4.
  auto pv = [&](const uint8_t* Vs, const bf16x8 (&pw)[4]) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint8_t* vu = Vs + (32 * (u >> 1) + 16 * (u & 1)) * kRowBytes;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vu + vofs[0][db]));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vu + vofs[1][db]));
        const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
        const bf16x8 av = as_bf16x8(make_uint4(l2.x, l2.y, h2.x, h2.y));
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pw[u], o[db], 0, 0, 0);
      }
    }
  };

  // Softmax weights of the current tile, with the previous tile's PV product issued
  // first so the exponentials run in its shadow.  The common path uses the running
  // reference m as is: if this tile's sum of rounded weights stays <= 2^8 on every
  // lane, no weight exceeds 2^8 and nothing else is needed.  Otherwise (the first tile,
  // or a new larger score), the true maximum is taken, O and l are rescaled -- after
  // the previous PV product, which used the old m -- and the weights are recomputed.
  auto softmax_pv = [&](const f32x16 (&sacc)[2], bf16x8 (&pw)[4], const uint8_t* Vprev,
                        const bf16x8 (&pprev)[4], bool have_prev) {
    if (have_prev) pv(Vprev, pprev);
    float tsum = exp_tile(sacc, pw);
    if (__ballot(!(tsum <= kTwoTau)) != 0) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mnew = fmaxf(m, mx * scale_log2);
      const float alpha = __builtin_amdgcn_exp2f(m - mnew);
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
      m = mnew;
      tsum = exp_tile(sacc, pw);
    }
    lsum += tsum;
  };

  uint8_t* const kb0 = smem;
  uint8_t* const kb1 = smem + kTileBytes;
  uint8_t* const vb0 = smem + 2 * kTileBytes;
  uint8_t* const vb1 = smem + 3 * kTileBytes;

  // prologue: K(0) in LDS
  load_k(0);
  store_k(kb0);
  __syncthreads();

  f32x16 sacc[2];
  bf16x8 pa_[4], pb2[4];  // P of even / odd tiles

  // iteration t: stage K(t+1), V(t); scores of tile t; PV of tile t-1 with tile t's
  // softmax.  Kcur/Knext and Vprev/Vcur alternate with the parity of t.
  auto iteration = [&](int t, const uint8_t* Kcur, uint8_t* Knext, const uint8_t* Vprev,
                       uint8_t* Vcur, bf16x8 (&pcur)[4], const bf16x8 (&pprev)[4]) {
    const bool kmore = t + 1 < ntiles;
    if (kmore) load_k(t + 1);
    load_v(t);
    if (active) {
      qk(Kcur, sacc);
      mask(t, sacc);
      softmax_pv(sacc, pcur, Vprev, pprev, t > 0);
    }
    if (kmore) store_k(Knext);
    store_v(Vcur);
    __syncthreads();
  };

  int t = 0;
  for (; t + 1 < ntiles; t += 2) {
    iteration(t, kb0, kb1, vb1, vb0, pa_, pb2);
    iteration(t + 1, kb1, kb0, vb0, vb1, pb2, pa_);
  }
  if (t < ntiles) {
    iteration(t, kb0, kb1, vb1, vb0, pa_, pb2);
    if (active) pv(vb0, pa_);
  } else if (active) {
    pv(vb1, pb2);
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
constexpr int kF32Threads = 256;

__global__ __launch_bounds__(kF32Threads) void gen_attn_f32_kernel(
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
  const int rows_per_block = kF32Threads / 2;
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
    for (int e = tid; e < kF32Keys * kHeadDim; e += kF32Threads) {
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
  const int64_t n_rb = (rows + kF32Threads / 2 - 1) / (kF32Threads / 2);
  const int64_t blocks = n_rb * Hkv * B;
  hipLaunchKernelGGL(gen_attn_f32_kernel, dim3((unsigned)blocks), dim3(kF32Threads), 0, stream, q,
                     k_img, v_img, k_pre, v_pre, cu_q, cu_p, Hq, Hkv, (int)n_rb, max_q, max_p, Tq,
                     Tp, scale, out, lse);
  return hipGetLastError();
}

}  // namespace neo
