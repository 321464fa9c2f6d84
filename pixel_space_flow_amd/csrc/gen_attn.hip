// Generation-pass attention: image queries over [frozen prefix ; image block], no mask,
// no cache write, grouped-query heads.
//
// "SenseNova-U1.5 (NEO-unify) architecture": §Mixture of Transformers (the generation
// branch reads the cache filled by the understanding branch and leaves it unchanged)
// and §GQA fusion does not apply (the generation graph has no attention mask input).  For query
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
//   * software pipeline over 32-key sub-tiles: each of the 8 slots of a step issues one
//     score MFMA of sub-tile s+1, one PV MFMA of sub-tile s-1 and one pair of weights of
//     sub-tile s, so the exponentials of one sub-tile run under the matrix products of
//     its neighbours inside every wave; the LDS operands are read three slots ahead;
//   * online softmax in fp32 on exp2 with the 1/sqrt(d) * log2(e) scale folded into one
//     FMA; the row sum adds the bf16-rounded weights that the PV product uses.  The
//     running maximum is raised only when a sub-tile's sum of weights exceeds 2^8, so
//     the O rescale (64 multiplies per lane) runs on the first sub-tile and almost never
//     afterwards, while every weight stays <= 2^8; the final O / l is the same quotient
//     whichever reference maximum was used;
//   * K/V tiles of 64 keys go from HBM/L2 straight into LDS (buffer loads with the LDS
//     destination, no register round trip).  The resource of each tile ends at its
//     segment's end, so rows past it arrive as zeros (their scores are then set to
//     -inf) with no per-row address arithmetic.  Three K and three V buffers: the loads
//     of K tile T+2 and V tile T+1 are in flight during the math of tile T; one barrier
//     per tile.  LDS rows are XOR-swizzled at 16-byte granularity, which keeps the
//     K-fragment reads and the transposed V reads free of bank conflicts;
//   * the workgroup order is remapped so each XCD works on contiguous (sample, KV head)
//     ranges and its L2 holds that head's K/V.
//
// fp32 kernel: a plain online-softmax kernel on the vector ALUs (two lanes per query
// row, 64 dims each), for fp32 inputs where bf16 MFMA would not meet fp32 accuracy.
#include "neo_internal.h"

#include <math.h>

#include <type_traits>

namespace neo {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kBN = 64;                      // keys per LDS tile (one barrier per tile)
constexpr int kRow = kHeadDim * 2;          // one K or V row in LDS (no padding)
constexpr int kTileBytes = kBN * kRow;       // 16 KB
constexpr float kTwoTau = 256.0f;            // bound on any softmax weight (2^8)
constexpr bf16x2 kOnes2 = {(__bf16)1.0f, (__bf16)1.0f};
constexpr int kBufFlags = 0x00020000;        // raw buffer, 32-bit data format (gfx9 family)
constexpr int kPrefetch = 3;                 // slots of LDS operands read ahead (<= 3)
constexpr int kLoadSlotK = 1, kLoadSlotV = 3;  // slots that issue the next tiles' loads

// LDS tiles hold 64 rows of 16 chunks (16 bytes = 8 dims each).  Chunk c of row r is
// stored at slot c ^ swz(r), which keeps the K-fragment reads (16 consecutive rows, one
// chunk) and the transposed V reads (4 consecutive rows, 4 consecutive chunks per
// half-wave) free of bank conflicts.  Tiles are written by buffer loads that deliver
// straight into LDS: one such load fills 1 KB (lane L writes bytes 16L .. 16L+15), so
// the swizzle is applied on the fetch side (lane L fetches the chunk that belongs in its
// slot).  Three K and three V tiles: in iteration T the waves read K tiles T, T+1 and V
// tiles T-1, T while K tile T+2 and V tile T+1 are in flight.
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)nbytes,
                                           kBufFlags);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

// Key segments of one (sample, KV head): the frozen prefix, then the image block.
struct Segments {
  const uint8_t* kbase[2];
  const uint8_t* vbase[2];
  int len[2];
  int ntiles[2];
  uint32_t row_bytes;   // Hkv * 128 * 2
  uint32_t tile_bytes;  // 64 rows
};

// One LDS tile = 64 consecutive rows of one key segment.  The buffer resource starts at
// the tile's first row and ends at the segment's end, so the hardware range check
// returns zeros for rows past the segment: no branches, no per-row address arithmetic.
// One sample's segment spans < 2^31 bytes (checked by the caller): 32-bit offsets.
__device__ __forceinline__ void tile_rsrc(const Segments& S, int it, __amdgpu_buffer_rsrc_t& rk,
                                          __amdgpu_buffer_rsrc_t& rv) {
  const bool pre = it < S.ntiles[0];
  const int tl = pre ? it : it - S.ntiles[0];
  const int rows = (pre ? S.len[0] : S.len[1]) - tl * kBN;
  const uint32_t off = (uint32_t)tl * S.tile_bytes;
  const uint32_t nbytes = (uint32_t)(rows < kBN ? rows : kBN) * S.row_bytes;
  rk = make_rsrc((pre ? S.kbase[0] : S.kbase[1]) + off, nbytes);
  rv = make_rsrc((pre ? S.vbase[0] : S.vbase[1]) + off, nbytes);
}

// valid keys of 32-key sub-tile s (may be <= 0 on a segment's last LDS tile)
__device__ __forceinline__ int sub_valid(const Segments& S, int s) {
  const int it = s >> 1;
  const bool pre = it < S.ntiles[0];
  const int tl = pre ? it : it - S.ntiles[0];
  return (pre ? S.len[0] : S.len[1]) - tl * kBN - (s & 1) * 32;
}

// Last position of the run of equal temporal indices that contains position `start`
// (within a sample the indices are non-decreasing and equal ones are contiguous).  All
// lanes of the wave call it with the same arguments.  A probe covers 1024 positions:
// lane L reads positions base + 64 j + L for j < 16 (16 coalesced loads, all issued before
// any is examined), so a run of up to 1024 positions -- a whole image block -- costs one
// memory round trip rather than one per 64 positions.
__device__ __forceinline__ int run_end(const int32_t* ix, int start, int n, int lane) {
  const int v0 = ix[start];
  for (int base = start + 1; base < n; base += 1024) {
    int v[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int p = base + 64 * j + lane;
      v[j] = p < n ? ix[p] : 0;  // no read at or past n
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int p = base + 64 * j + lane;
      const uint64_t bal = __ballot(p >= n || v[j] != v0);
      if (bal != 0) return base + 64 * j + (int)__builtin_ctzll(bal) - 1;
    }
  }
  return n - 1;
}

// The bf16 attention body.  kPrefill = false: the generation pass (image queries over
// [prefix ; image block], unmasked).  kPrefill = true: the understanding pass over one
// sequence with the block-causal mask ("SenseNova-U1.5 (NEO-unify) architecture",
// §Block-causal attention: key j is open to query i when their temporal indices are
// equal or j <= i).  With a sample's indices non-decreasing and equal indices contiguous,
// query i sees exactly the keys 0 .. end(i), end(i) = max(i, last position of its index
// run); the prefill variant runs the same pipeline with no prefix segment, the key range
// of a workgroup cut at end() of its last query, and each lane masking keys past its own
// end().  ("SenseNova-U1 ... NEO-unify Architecture" paper notes, §2.5, Fig. 6: image
// query blocks extend the key range, text blocks stay causal.)
//
// kWaves is 8 (two waves per SIMD, 64 query tokens of one KV group per workgroup) or 4 (one
// wave per SIMD, 32 tokens; the prefill's form for grids that would otherwise leave CUs
// idle; the generation pass uses the split-key form below for those).
template <bool kPrefill, int kWaves>
__device__ __forceinline__ void attn_bf16_body(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_img,
    const uint16_t* __restrict__ v_img, const uint16_t* __restrict__ k_pre,
    const uint16_t* __restrict__ v_pre, const int32_t* __restrict__ cu_q,
    const int32_t* __restrict__ cu_p, const int32_t* __restrict__ tidx, int Hq, int Hkv,
    int n_cg, int max_q, int max_p, int64_t Tq, int64_t Tp, float scale_log2,
    uint16_t* __restrict__ out, float* __restrict__ lse) {
  // six separate LDS objects, so the compiler sees that a tile load into one buffer
  // cannot alias fragment reads from another and does not wait for it
  __shared__ __attribute__((aligned(1024))) uint8_t lk0[kTileBytes], lk1[kTileBytes],
      lk2[kTileBytes], lv0[kTileBytes], lv1[kTileBytes], lv2[kTileBytes];
  auto kbuf = [&](int b) __attribute__((always_inline)) -> uint8_t* {
    return b == 0 ? lk0 : (b == 1 ? lk1 : lk2);
  };
  auto vbuf = [&](int b) __attribute__((always_inline)) -> uint8_t* {
    return b == 0 ? lv0 : (b == 1 ? lv1 : lv2);
  };

  const uint32_t id = xcd_remap(blockIdx.x, gridDim.x);
  // prefill: the heaviest workgroups (latest queries, longest key ranges) start first
  const int cg0 = (int)(id % (uint32_t)n_cg);
  const int cg = kPrefill ? n_cg - 1 - cg0 : cg0;
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
  const int P = kPrefill ? 0 : (int)((pb_ - pa) < max_p ? (pb_ - pa) : max_p);

  const int G = Hq / Hkv;
  const int nchunks = G * ((N + 31) / 32);
  if (cg * kWaves >= nchunks) return;  // whole workgroup idle

  constexpr int kThreads = kWaves * 64;
  constexpr int kBlk = 16 / kWaves;  // 1 KB staging blocks per wave and tile
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, hl = lane >> 5, col = lane & 31;
  const int c = cg * kWaves + wave;
  const bool active = c < nchunks;
  const int h = g * G + (active ? c % G : 0);
  const int qi = (active ? c / G : 0) * 32 + col;  // query index inside the sample
  const bool qvalid = active && qi < N;

  // prefill: the keys the workgroup's queries may see are 0 .. kmax-1; lane_lim is the
  // number of keys this lane's query may see, lim_min the smallest over the wave.  They are
  // found after the first tile loads are issued (prefill_limits below), so the probes of
  // the temporal indices overlap those loads.
  // wave_tiles: the tiles any lane of this wave may see; past them the wave only stages
  // tiles for the others (its scores would all be masked)
  int kmax = N, lane_lim = 1 << 30, lim_min = 1 << 30, wave_tiles = 1 << 30;
  auto prefill_limits = [&]() __attribute__((always_inline)) {
    const int32_t* ix = tidx + qa;
    const int last_c = (cg * kWaves + kWaves < nchunks ? cg * kWaves + kWaves : nchunks) - 1;
    const int wg_last = ((last_c / G) * 32 + 32 < N ? (last_c / G) * 32 + 32 : N) - 1;
    // wave-uniform by construction; readfirstlane tells the compiler, so the key range and
    // every per-tile condition derived from it stay scalar
    kmax = __builtin_amdgcn_readfirstlane(run_end(ix, wg_last, N, lane) + 1);
    if (active) {
      const int t0 = (c / G) * 32;
      const int nq = N - t0 < 32 ? N - t0 : 32;
      const int my = qvalid ? ix[qi] : 0;
      // e: the last query of the wave in this lane's run.  Runs are contiguous, so it is the
      // first run boundary (query m with an index different from query m + 1's) at or after
      // this lane's query, or the wave's last query if the run reaches it
      const int next = __shfl(my, (lane & 32) | ((col + 1) & 31));
      const uint32_t bounds =
          (uint32_t)__ballot(col < nq - 1 && my != next);  // lanes 0..31 (one half suffices)
      const uint32_t from_me = bounds >> col;
      const int e = from_me != 0 ? col + __builtin_ctz(from_me) : nq - 1;
      // the wave's last query ends the same run as the workgroup's last one when their
      // indices are equal (indices are non-decreasing), which spares the second probe
      const int wave_last = t0 + nq - 1;
      const int wave_end = ix[wave_last] == ix[wg_last] ? kmax - 1 : run_end(ix, wave_last, N, lane);
      lane_lim = (e == nq - 1 ? wave_end : t0 + e) + 1;
      if (!qvalid) lane_lim = kmax;
      lim_min = __builtin_amdgcn_readfirstlane(lane_lim);  // lane 0's limit, the smallest
      // limits are non-decreasing along the wave: its last query sees the most keys
      const int lim_max = __builtin_amdgcn_readlane(lane_lim, nq - 1);
      wave_tiles = (lim_max + kBN - 1) / kBN;
    }
  };

  Segments S;
  S.row_bytes = (uint32_t)Hkv * kHeadDim * 2;
  S.tile_bytes = S.row_bytes * kBN;
  S.kbase[0] = reinterpret_cast<const uint8_t*>(k_pre + (pa * Hkv + g) * kHeadDim);
  S.vbase[0] = reinterpret_cast<const uint8_t*>(v_pre + (pa * Hkv + g) * kHeadDim);
  S.kbase[1] = reinterpret_cast<const uint8_t*>(k_img + (qa * Hkv + g) * kHeadDim);
  S.vbase[1] = reinterpret_cast<const uint8_t*>(v_img + (qa * Hkv + g) * kHeadDim);
  // the image segment's rows bound the tile loads (the prefill cuts its key range at kmax
  // through the tile count and masks keys past each lane's limit)
  S.len[0] = P;
  S.len[1] = N;
  S.ntiles[0] = (P + kBN - 1) / kBN;
  S.ntiles[1] = (N + kBN - 1) / kBN;
  int ntiles = S.ntiles[0] + S.ntiles[1];  // the prefill recomputes it from kmax below

  // staging: wave w fills 1 KB blocks kBlk*w .. kBlk*w + kBlk-1 of each tile (block blk
  // holds rows 4*blk .. +3); lane L of block blk lands in row 4*blk + L/16, slot L%16 and
  // so fetches chunk (L%16) ^ swz(row) of that row
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  int goff[kBlk];
#pragma unroll
  for (int i = 0; i < kBlk; ++i) {
    const int row = 4 * (kBlk * wave + i) + (lane >> 4);
    goff[i] = row * (int)S.row_bytes + (((lane & 15) ^ swz(row)) << 4);
  }

  // K-fragment reads (A operand of S^T = K Q^T): row 32*half + col, chunk 2*st + hl.  The
  // swizzle depends on row % 16 only, so the half adds a constant 32 rows.
  int kofs[8];
#pragma unroll
  for (int st = 0; st < 8; ++st) kofs[st] = col * kRow + (((2 * st + hl) ^ swz(col)) << 4);
  // V-fragment reads (A operand of O^T = V^T P^T, transposed): within each 16-lane group,
  // lane j addresses row key0 + j/4 at dims dim0 + 4*(j%4) and receives dim dim0 + j of
  // rows key0 .. key0+3.  For sub-tile half h, step u, read r and dim block db:
  // key0 = 32*h + 16*u + 8*r + 4*hl, dim0 = 32*db + 16*grp; h and u add multiples of 16
  // rows (constant offsets).
  const int j16 = lane & 15, grp = (lane >> 4) & 1;
  int vofs[2][4];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int row = 8 * r + 4 * hl + (j16 >> 2);
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int chunk = 4 * db + 2 * grp + ((j16 & 3) >> 1);
      vofs[r][db] = row * kRow + ((chunk ^ swz(row)) << 4) + ((j16 & 1) << 3);
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

  // K (V) tile t into K (V) buffer buf, straight from HBM/L2 into LDS
  auto load_k = [&](int t, int buf) {
    __amdgpu_buffer_rsrc_t rk, rv;
    tile_rsrc(S, t, rk, rv);
#pragma unroll
    for (int i = 0; i < kBlk; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rk, (__attribute__((address_space(3))) void*)(kbuf(buf) + (kBlk * wave_u + i) * 1024),
          16, goff[i], 0, 0, 0);
  };
  auto load_v = [&](int t, int buf) {
    __amdgpu_buffer_rsrc_t rk, rv;
    tile_rsrc(S, t, rk, rv);
#pragma unroll
    for (int i = 0; i < kBlk; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rv, (__attribute__((address_space(3))) void*)(vbuf(buf) + (kBlk * wave_u + i) * 1024),
          16, goff[i], 0, 0, 0);
  };
  // fragment reads from K buffer kb / V buffer vb, sub-tile half h
  auto kread = [&](int kb, int h, int st) -> bf16x8 {
    return as_bf16x8(*reinterpret_cast<const uint4*>(kbuf(kb) + h * 32 * kRow + kofs[st]));
  };
  // V^T fragment for step u (16 keys) and dim block db: two transposed 8-byte reads
  auto vread = [&](const uint8_t* vb, int u, int db) -> bf16x8 {
    const uint8_t* p = vb + 16 * u * kRow;
    const uint2 lo = __builtin_bit_cast(
        uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + vofs[0][db])));
    const uint2 hi = __builtin_bit_cast(
        uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + vofs[1][db])));
    return as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
  };

  // keys of sub-tile s past its segment's end score -inf
  // (prefill: also keys past this lane's own end; sub-tile s starts at key 32*s there)
  auto mask = [&](int s, f32x16& sacc) {
    const int nvalid = sub_valid(S, s);
    const bool edge = kPrefill ? (nvalid < 32 || 32 * s + 32 > lim_min) : nvalid < 32;
    if (edge) {
      // key = (r/4)*8 + hl*4 + r%4; compare its constant part with one limit
      int lim = nvalid;
      if (kPrefill) lim = lane_lim - 32 * s < lim ? lane_lim - 32 * s : lim;
      lim -= hl * 4;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if ((r >> 2) * 8 + (r & 3) >= lim) sacc[r] = -INFINITY;
    }
  };

  // two weights p = exp2(s*c - m) as one packed bf16 word, and the row sum of the same
  // rounded weights (v_dot2 against (1, 1)) so the normalised weights sum to one.
  // Pair i of 8: PV step u = i/4, word i%4.
  auto exp_pair = [&](const f32x16& sacc, int i, uint32_t (&pk)[2][4], float& tsum) {
    const int u = i >> 2, e = (i & 3) * 2;
    const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[u * 8 + e], scale_log2, -m));
    const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[u * 8 + e + 1], scale_log2, -m));
    pk[u][i & 3] = pack_bf16x2(p0, p1);
    tsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[u][i & 3]), kOnes2, tsum,
                                           false);
  };
  auto pack_p = [&](const uint32_t (&pk)[2][4], bf16x8 (&pw)[2]) {
#pragma unroll
    for (int u = 0; u < 2; ++u) pw[u] = as_bf16x8(make_uint4(pk[u][0], pk[u][1], pk[u][2], pk[u][3]));
  };

  // Pipeline over 32-key sub-tiles.  Slot i (0..7) of the step at sub-tile s issues one
  // MFMA of the scores of sub-tile s+1 (one chain), one MFMA of the PV product of
  // sub-tile s-1 (four chains; k-slot (hl, e) of step u is key 16*u + 4*hl + 8*(e/4) +
  // e%4) and one pair of weights of sub-tile s.  On the first step the "previous" P is
  // all zeros (against V tile 0, already staged and finite); on the last step the scores
  // of the non-existent next sub-tile come from a resident K buffer and are discarded.
  // The LDS operands of each slot are read kPrefetch slots ahead into a ring of four;
  // every such read targets a tile that is already resident (see the staging order).
  // The common path uses the running reference m as is: if the sub-tile's sum of rounded
  // weights stays <= 2^8 on every lane, no weight exceeds 2^8.  Otherwise (the first
  // sub-tile, or a new larger score) the true maximum is taken, O and l are rescaled --
  // after the PV product of s-1, which used the old m -- and the weights are recomputed.
  bf16x8 kf[4], vf[4];
  // LDS buffers are compile-time constants at every call site below, so each address is
  // this lane's base plus an immediate offset
  auto fetch = [&](int kb, int khalf, int vb, int vhalf, int i, int r)
                   __attribute__((always_inline)) {
    kf[r] = kread(kb, khalf, i);
    vf[r] = vread(vbuf(vb) + vhalf * 32 * kRow, i >> 2, i & 3);
  };
  auto finish_step = [&](int s, f32x16& scur, f32x16& snext, bf16x8 (&pcur)[2],
                         uint32_t (&pk)[2][4], float tsum) {
    pack_p(pk, pcur);
    if (__ballot(!(tsum <= kTwoTau)) != 0) {
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, scur[r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mnew = fmaxf(m, mx * scale_log2);
      const float alpha = __builtin_amdgcn_exp2f(m - mnew);
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
      m = mnew;
      tsum = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) exp_pair(scur, i, pk, tsum);
      pack_p(pk, pcur);
    }
    lsum += tsum;
    mask(s + 1, snext);
  };

  // prologue: K tiles 0 and 1, V tile 0; V buffer 2 cleared (the first step's PV
  // product reads it against an all-zero P); scores of sub-tile 0
  load_k(0, 0);
  load_v(0, 0);
  if (ntiles > 1) load_k(1, 1);
  if constexpr (kPrefill) {
    prefill_limits();
    ntiles = (kmax + kBN - 1) / kBN;
  }
  for (int i = tid; i < kTileBytes / 16; i += kThreads)
    reinterpret_cast<uint4*>(lv2)[i] = make_uint4(0, 0, 0, 0);
  __syncthreads();
  const f32x16 zero16 = {};
  f32x16 sa, sb;
  bf16x8 pa_[2], pb2[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) pb2[u] = as_bf16x8(make_uint4(0, 0, 0, 0));
  // PV product of the last sub-tile a wave computed: the second half of the tile in V buffer
  // vb, with its weights in pb2
  auto pv_last = [&](int vb) {
    const uint8_t* va = vbuf(vb) + 32 * kRow;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      o[i & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vread(va, i >> 2, i & 3), pb2[i >> 2],
                                                         o[i & 3], 0, 0, 0);
  };

  if (active) {
    sa = zero16;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      sa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kread(0, 0, i), qf[i], sa, 0, 0, 0);
    mask(0, sa);
    // operands of the first slots of iteration 0: K tile 0 (second half), V "tile -1"
#pragma unroll
    for (int k = 0; k < kPrefetch; ++k) fetch(0, 1, 2, 1, k, k & 3);
  }

  // iteration T: steps at sub-tiles 2T (scores in sa) and 2T+1; stage K tile T+2 and V
  // tile T+1.  Tile t lives in buffer t % 3 (T3 = T % 3 is a compile-time constant).
  // Reads in iteration T touch K tiles T, T+1 and V tiles T-1, T; the reads prefetched
  // for the first slots of iteration T+1 touch K tile T+1 and V tile T; the stores go to
  // the buffers of K tile T-1 and V tile T-2, which nothing reads any more.
  auto iteration = [&](int T, auto t3) __attribute__((always_inline)) {
    constexpr int T3 = decltype(t3)::value;
    constexpr int b0 = T3, b1 = (T3 + 1) % 3, bm1 = (T3 + 2) % 3;
    const bool kmore = T + 2 < ntiles, vmore = T + 1 < ntiles;
    if (!active || T >= wave_tiles) {
      if (kmore) load_k(T + 2, bm1);
      if (vmore) load_v(T + 1, b1);
      // a prefill wave whose keys end before the workgroup's: the PV product of its last
      // sub-tile (second half of tile T - 1, still resident), which the next step would do
      if (kPrefill && active && T == wave_tiles) pv_last(bm1);
    } else {
      uint32_t pk[2][4];
      float tsum = 0.0f;
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const int h = k >> 3, i = k & 7;
        f32x16& scur = h == 0 ? sa : sb;
        f32x16& snext = h == 0 ? sb : sa;
        bf16x8 (&pcur)[2] = h == 0 ? pa_ : pb2;
        bf16x8 (&pprev)[2] = h == 0 ? pb2 : pa_;
        if (i == 0) tsum = 0.0f;
        {
          const int kk = k + kPrefetch;
          if (kk < 8)  // step at sub-tile 2T: K of 2T+1, V of 2T-1
            fetch(b0, 1, bm1, 1, kk, kk & 3);
          else if (kk < 16)  // step at sub-tile 2T+1: K of 2T+2, V of 2T
            fetch(b1, 0, b0, 0, kk - 8, kk & 3);
          else  // first step of iteration T+1: K of 2T+3, V of 2T+1
            fetch(b1, 1, b0, 1, kk - 16, kk & 3);
        }
        snext = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[k & 3], qf[i], i == 0 ? zero16 : snext,
                                                        0, 0, 0);
        o[i & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[k & 3], pprev[i >> 2], o[i & 3], 0, 0, 0);
        // the next tiles' loads (scalar descriptor set-up, then LDS-direct loads) go under
        // the matrix products of early slots rather than right after the barrier
        if (k == kLoadSlotK && kmore) load_k(T + 2, bm1);
        if (k == kLoadSlotV && vmore) load_v(T + 1, b1);
        // the weights of the slot are bracketed by a raised-priority window.  The weights are
        // pure values that the compiler mostly schedules outside the window, so it seldom
        // holds the exponentials, but the markers shift the slot's schedule: measured ~2%
        // faster than without them in same-box A/B.  A window around the products instead
        // gained nothing, and pinning the weights inside the window was ~4% slower.
        __builtin_amdgcn_s_setprio(1);
        exp_pair(scur, i, pk, tsum);
        __builtin_amdgcn_s_setprio(0);
        __builtin_amdgcn_sched_barrier(0);
        if (i == 7) finish_step(2 * T + h, scur, snext, pcur, pk, tsum);
      }
    }
    __syncthreads();
  };
  using C0 = std::integral_constant<int, 0>;
  using C1 = std::integral_constant<int, 1>;
  using C2 = std::integral_constant<int, 2>;
  for (int T = 0; T < ntiles; T += 3) {
    iteration(T, C0{});
    if (T + 1 >= ntiles) break;
    iteration(T + 1, C1{});
    if (T + 2 >= ntiles) break;
    iteration(T + 2, C2{});
  }
  // last sub-tile's PV product (its P is in pb2), for waves that ran to the last tile
  if (active && wave_tiles >= ntiles) pv_last((ntiles - 1) % 3);

  const float ltot = lsum + __shfl_xor(lsum, 32);
  // The output goes through LDS (free once every wave is past its last tile) so that each
  // lane stores whole 16-byte chunks of 256-byte rows: wave w stages its 32 x 128 block in
  // 8 KB of one former K/V buffer, row = query, chunk c of a row in slot c ^ (row % 16).
  __syncthreads();
  uint8_t* ob = ((wave >> 1) == 0 ? lk0 : (wave >> 1) == 1 ? lk1 : (wave >> 1) == 2 ? lk2 : lv0) +
                (wave & 1) * 8192;
  if (active) {
    const float inv = qvalid ? 1.0f / ltot : 0.0f;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const uint32_t w0 = pack_bf16x2(o[db][rg * 4 + 0] * inv, o[db][rg * 4 + 1] * inv);
        const uint32_t w1 = pack_bf16x2(o[db][rg * 4 + 2] * inv, o[db][rg * 4 + 3] * inv);
        const int slot = (db * 4 + rg) ^ (col & 15);
        *reinterpret_cast<uint2*>(ob + col * 256 + slot * 16 + hl * 8) = make_uint2(w0, w1);
      }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's rows are in LDS
    asm volatile("" ::: "memory");
    const int q0 = qi - col;  // the wave's first query
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = 4 * i + (lane >> 4), cch = lane & 15;
      const uint4 vrow = *reinterpret_cast<const uint4*>(ob + r * 256 + ((cch ^ (r & 15)) * 16));
      if (q0 + r < N)
        *reinterpret_cast<uint4*>(out + ((qa + q0 + r) * Hq + h) * kHeadDim + cch * 8) = vrow;
    }
    if (qvalid && lse != nullptr && hl == 0)
      lse[(int64_t)h * Tq + qa + qi] = (m + __log2f(ltot)) * 0.69314718055994530942f;
  }
}

// Split-key form, for launches that would leave CUs idle (one or few short images).  A
// workgroup of 8 waves covers 32 query tokens of one KV group (4 chunks of 32 query rows,
// one per query head) and splits the keys between two groups of waves: waves 0-3 take
// the first half, waves 4-7 the second, so every SIMD still runs two waves.  Keys are
// counted in 32-key sub-tiles, each inside one segment (prefix first, then image): ns of
// them; half 0 takes sub-tiles [0, ns0), half 1 [ns0, ns), ns0 = ceil(ns / 2).  LDS tile T
// (64 rows, swizzled as above) holds half 0's sub-tile T in rows 0-31 and half 1's
// sub-tile ns0 + T in rows 32-63, so each wave reads only its half of every tile and the
// pipeline advances one 32-key step per tile: the step at sub-tile T issues the scores of
// T + 1, the PV product of T - 1 and the weights of T.  Tile t lives in buffer t % 3; in
// iteration T the waves read K tiles T + 1, T + 2 and V tiles T - 1, T, while K tile T + 3
// and V tile T + 1 are loaded into the buffers of K tile T and V tile T - 2.  At the end the
// second group hands its (m, l, O) to the first through LDS and the first group merges,
// normalises and stores.  A half with no keys (ns = 1) contributes l = 0.
__device__ __forceinline__ void gen_attn_split_body(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_img,
    const uint16_t* __restrict__ v_img, const uint16_t* __restrict__ k_pre,
    const uint16_t* __restrict__ v_pre, const int32_t* __restrict__ cu_q,
    const int32_t* __restrict__ cu_p, int Hq, int Hkv, int n_cg, int max_q, int max_p,
    int64_t Tq, int64_t Tp, float scale_log2, uint16_t* __restrict__ out,
    float* __restrict__ lse) {
  __shared__ __attribute__((aligned(1024))) uint8_t lk0[kTileBytes], lk1[kTileBytes],
      lk2[kTileBytes], lv0[kTileBytes], lv1[kTileBytes], lv2[kTileBytes];
  auto kbuf = [&](int b) __attribute__((always_inline)) -> uint8_t* {
    return b == 0 ? lk0 : (b == 1 ? lk1 : lk2);
  };
  auto vbuf = [&](int b) __attribute__((always_inline)) -> uint8_t* {
    return b == 0 ? lv0 : (b == 1 ? lv1 : lv2);
  };
  constexpr int kQW = 4;  // query waves per workgroup (one per key half pair)

  const uint32_t id = xcd_remap(blockIdx.x, gridDim.x);
  const int cg = (int)(id % (uint32_t)n_cg);
  const int rest = (int)(id / (uint32_t)n_cg);
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
  const int nchunks = G * ((N + 31) / 32);
  if (cg * kQW >= nchunks) return;  // whole workgroup idle

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, hl = lane >> 5, col = lane & 31;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int qw = wave & 3, hw = wave >> 2;  // query wave, key half
  const int c = cg * kQW + qw;
  const bool active = c < nchunks;
  const int h = g * G + (active ? c % G : 0);
  const int qi = (active ? c / G : 0) * 32 + col;
  const bool qvalid = active && qi < N;

  // 32-key sub-tiles: np0 in the prefix, then the image's
  const int np0 = (P + 31) / 32, ns = np0 + (N + 31) / 32, ns0 = (ns + 1) / 2;
  const int first = __builtin_amdgcn_readfirstlane(hw ? ns0 : 0);
  const int count = __builtin_amdgcn_readfirstlane(hw ? ns - ns0 : ns0);
  const bool work = active && count > 0;

  const uint32_t row_bytes = (uint32_t)Hkv * kHeadDim * 2;
  const uint8_t* kb0 = reinterpret_cast<const uint8_t*>(k_pre + (pa * Hkv + g) * kHeadDim);
  const uint8_t* vb0 = reinterpret_cast<const uint8_t*>(v_pre + (pa * Hkv + g) * kHeadDim);
  const uint8_t* kb1 = reinterpret_cast<const uint8_t*>(k_img + (qa * Hkv + g) * kHeadDim);
  const uint8_t* vb1 = reinterpret_cast<const uint8_t*>(v_img + (qa * Hkv + g) * kHeadDim);
  // keys of this half's sub-tile t that exist (0 past the half's end)
  auto sub_rows = [&](int t) -> int {
    const int gs = first + t;
    const bool pre = gs < np0;
    const int rows = (pre ? P : N) - 32 * (pre ? gs : gs - np0);
    return t < count ? (rows < 32 ? rows : 32) : 0;
  };
  // buffer resources of this half's sub-tile t: from its first row to the end of its rows
  auto sub_rsrc = [&](int t, bool isv) -> __amdgpu_buffer_rsrc_t {
    const int gs = first + t;
    const bool pre = gs < np0;
    const int rows = sub_rows(t);
    const uint32_t off = (uint32_t)(pre ? gs : gs - np0) * 32u * row_bytes;
    const uint8_t* base = isv ? (pre ? vb0 : vb1) : (pre ? kb0 : kb1);
    const uint32_t nbytes = rows <= 0 ? 0u : (uint32_t)rows * row_bytes;
    return make_rsrc(base + (t < count ? off : 0u), nbytes);
  };

  // staging: wave w fills LDS rows 8w .. 8w+7 of each tile (blocks 2w, 2w+1), i.e. rows
  // 8*qw .. 8*qw+7 of its own half's sub-tile
  int goff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int rin = 8 * qw + 4 * i + (lane >> 4);  // row inside the sub-tile (= LDS row % 32)
    goff[i] = rin * (int)row_bytes + (((lane & 15) ^ swz(rin)) << 4);
  }
  // fragment offsets include the half's 32-row offset
  int kofs[8];
#pragma unroll
  for (int st = 0; st < 8; ++st)
    kofs[st] = (32 * hw + col) * kRow + (((2 * st + hl) ^ swz(col)) << 4);
  const int j16 = lane & 15, grp = (lane >> 4) & 1;
  int vofs[2][4];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int row = 8 * r + 4 * hl + (j16 >> 2);
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int chunk = 4 * db + 2 * grp + ((j16 & 3) >> 1);
      vofs[r][db] = (32 * hw + row) * kRow + ((chunk ^ swz(row)) << 4) + ((j16 & 1) << 3);
    }
  }

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

  auto load_k = [&](int t, int buf) {
    const __amdgpu_buffer_rsrc_t rk = sub_rsrc(t, false);
#pragma unroll
    for (int i = 0; i < 2; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rk, (__attribute__((address_space(3))) void*)(kbuf(buf) + (2 * wave_u + i) * 1024), 16,
          goff[i], 0, 0, 0);
  };
  auto load_v = [&](int t, int buf) {
    const __amdgpu_buffer_rsrc_t rv = sub_rsrc(t, true);
#pragma unroll
    for (int i = 0; i < 2; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rv, (__attribute__((address_space(3))) void*)(vbuf(buf) + (2 * wave_u + i) * 1024), 16,
          goff[i], 0, 0, 0);
  };
  auto kread = [&](int kb, int st) -> bf16x8 {
    return as_bf16x8(*reinterpret_cast<const uint4*>(kbuf(kb) + kofs[st]));
  };
  auto vread = [&](const uint8_t* vb, int u, int db) -> bf16x8 {
    const uint8_t* p = vb + 16 * u * kRow;
    const uint2 lo = __builtin_bit_cast(
        uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + vofs[0][db])));
    const uint2 hi = __builtin_bit_cast(
        uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + vofs[1][db])));
    return as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
  };
  // keys of sub-tile t past its rows score -inf
  auto mask = [&](int t, f32x16& sacc) {
    const int nvalid = sub_rows(t);
    if (nvalid < 32) {
      const int lim = nvalid - hl * 4;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if ((r >> 2) * 8 + (r & 3) >= lim) sacc[r] = -INFINITY;
    }
  };
  auto exp_pair = [&](const f32x16& sacc, int i, uint32_t (&pk)[2][4], float& tsum) {
    const int u = i >> 2, e = (i & 3) * 2;
    const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[u * 8 + e], scale_log2, -m));
    const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[u * 8 + e + 1], scale_log2, -m));
    pk[u][i & 3] = pack_bf16x2(p0, p1);
    tsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[u][i & 3]), kOnes2, tsum,
                                           false);
  };
  auto pack_p = [&](const uint32_t (&pk)[2][4], bf16x8 (&pw)[2]) {
#pragma unroll
    for (int u = 0; u < 2; ++u) pw[u] = as_bf16x8(make_uint4(pk[u][0], pk[u][1], pk[u][2], pk[u][3]));
  };
  bf16x8 kf[4], vf[4];
  auto fetch = [&](int kb, int vb, int i, int r) __attribute__((always_inline)) {
    kf[r] = kread(kb, i);
    vf[r] = vread(vbuf(vb), i >> 2, i & 3);
  };
  // the same lazy-maximum step end as the unsplit body
  auto finish_step = [&](int t, f32x16& scur, f32x16& snext, bf16x8 (&pcur)[2],
                         uint32_t (&pk)[2][4], float tsum) {
    pack_p(pk, pcur);
    if (__ballot(!(tsum <= kTwoTau)) != 0) {
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, scur[r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mnew = fmaxf(m, mx * scale_log2);
      const float alpha = __builtin_amdgcn_exp2f(m - mnew);
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
      m = mnew;
      tsum = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) exp_pair(scur, i, pk, tsum);
      pack_p(pk, pcur);
    }
    lsum += tsum;
    mask(t + 1, snext);
  };

  // prologue: K tiles 0, 1, 2 and V tile 0; V buffer 2 cleared (the PV product of the
  // first step reads it against an all-zero P); scores of sub-tile 0
  load_k(0, 0);
  load_v(0, 0);
  if (ns0 > 1) load_k(1, 1);
  if (ns0 > 2) load_k(2, 2);
  for (int i = tid; i < kTileBytes / 16; i += 512)
    reinterpret_cast<uint4*>(lv2)[i] = make_uint4(0, 0, 0, 0);
  __syncthreads();
  const f32x16 zero16 = {};
  f32x16 sa, sb;
  bf16x8 pa_[2], pb2[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) pb2[u] = as_bf16x8(make_uint4(0, 0, 0, 0));
  if (work) {
    sa = zero16;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      sa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kread(0, i), qf[i], sa, 0, 0, 0);
    mask(0, sa);
#pragma unroll
    for (int k = 0; k < kPrefetch; ++k) fetch(1, 2, k, k);
  }

  // iteration T (T6 = T % 6 compile-time): buffers T % 3, register roles by T % 2
  auto iteration = [&](int T, auto t6) __attribute__((always_inline)) {
    constexpr int T6 = decltype(t6)::value;
    constexpr int b0 = T6 % 3, b1 = (T6 + 1) % 3, b2 = (T6 + 2) % 3;  // tiles T, T+1, T+2 (T-1)
    f32x16& scur = (T6 & 1) == 0 ? sa : sb;
    f32x16& snext = (T6 & 1) == 0 ? sb : sa;
    bf16x8 (&pcur)[2] = (T6 & 1) == 0 ? pa_ : pb2;
    bf16x8 (&pprev)[2] = (T6 & 1) == 0 ? pb2 : pa_;
    const bool kmore = T + 3 < ns0, vmore = T + 1 < ns0;
    if (!work) {
      if (kmore) load_k(T + 3, b0);
      if (vmore) load_v(T + 1, b1);
    } else {
      uint32_t pk[2][4];
      float tsum = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        {
          const int ii = i + kPrefetch;
          if (ii < 8)  // this step: K of sub-tile T+1, V of T-1 (buffer of tile T+2 mod 3)
            fetch(b1, b2, ii, ii & 3);
          else  // the first slots of the next step: K of T+2, V of T
            fetch(b2, b0, ii - 8, ii & 3);
        }
        snext = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i & 3], qf[i], i == 0 ? zero16 : snext,
                                                        0, 0, 0);
        o[i & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[i & 3], pprev[i >> 2], o[i & 3], 0, 0, 0);
        if (i == kLoadSlotK && kmore) load_k(T + 3, b0);
        if (i == kLoadSlotV && vmore) load_v(T + 1, b1);
        __builtin_amdgcn_s_setprio(1);
        exp_pair(scur, i, pk, tsum);
        __builtin_amdgcn_s_setprio(0);
        __builtin_amdgcn_sched_barrier(0);
        if (i == 7) finish_step(T, scur, snext, pcur, pk, tsum);
      }
    }
    __syncthreads();
  };
  using C0 = std::integral_constant<int, 0>;
  using C1 = std::integral_constant<int, 1>;
  using C2 = std::integral_constant<int, 2>;
  using C3 = std::integral_constant<int, 3>;
  using C4 = std::integral_constant<int, 4>;
  using C5 = std::integral_constant<int, 5>;
  for (int T = 0; T < ns0; T += 6) {
    iteration(T, C0{});
    if (T + 1 >= ns0) break;
    iteration(T + 1, C1{});
    if (T + 2 >= ns0) break;
    iteration(T + 2, C2{});
    if (T + 3 >= ns0) break;
    iteration(T + 3, C3{});
    if (T + 4 >= ns0) break;
    iteration(T + 4, C4{});
    if (T + 5 >= ns0) break;
    iteration(T + 5, C5{});
  }
  // PV product of the last sub-tile, ns0 - 1: V tile ns0 - 1 (buffer (ns0 - 1) % 3), its
  // weights in pa_ (ns0 odd) or pb2 (ns0 even)
  if (work) {
    const uint8_t* va = vbuf((ns0 - 1) % 3);
    bf16x8 pl[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) pl[u] = (ns0 & 1) ? pa_[u] : pb2[u];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      o[i & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vread(va, i >> 2, i & 3), pl[i >> 2],
                                                         o[i & 3], 0, 0, 0);
  }
  float ltot = lsum + __shfl_xor(lsum, 32);
  if (!work) ltot = 0.0f;

  // merge: the second group's (m, l, O) through LDS (the K buffers and V buffer 0 hold the
  // four waves' O, 16 KB each, V buffer 1 their m and l), combined by the first group
  __syncthreads();
  uint8_t* mo = qw == 0 ? lk0 : (qw == 1 ? lk1 : (qw == 2 ? lk2 : lv0));
  float2* ml = reinterpret_cast<float2*>(lv1) + qw * 64 + lane;
  if (hw == 1 && active) {
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg)
        reinterpret_cast<float4*>(mo)[(db * 4 + rg) * 64 + lane] =
            make_float4(o[db][rg * 4], o[db][rg * 4 + 1], o[db][rg * 4 + 2], o[db][rg * 4 + 3]);
    *ml = make_float2(work ? m : -INFINITY, ltot);
  }
  __syncthreads();
  if (hw == 0 && active) {
    const float2 mlb = *ml;
    const float mnew = fmaxf(m, mlb.x);
    const float sa_ = __builtin_amdgcn_exp2f(m - mnew);
    const float sb_ = mlb.y > 0.0f ? __builtin_amdgcn_exp2f(mlb.x - mnew) : 0.0f;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const float4 ob = reinterpret_cast<const float4*>(mo)[(db * 4 + rg) * 64 + lane];
        o[db][rg * 4] = o[db][rg * 4] * sa_ + ob.x * sb_;
        o[db][rg * 4 + 1] = o[db][rg * 4 + 1] * sa_ + ob.y * sb_;
        o[db][rg * 4 + 2] = o[db][rg * 4 + 2] * sa_ + ob.z * sb_;
        o[db][rg * 4 + 3] = o[db][rg * 4 + 3] * sa_ + ob.w * sb_;
      }
    ltot = ltot * sa_ + mlb.y * sb_;
    m = mnew;
  }
  __syncthreads();

  // the first group normalises and stores, through LDS as in the unsplit body
  uint8_t* ob = ((qw >> 1) == 0 ? lk0 : lk1) + (qw & 1) * 8192;
  if (hw == 0 && active) {
    const float inv = qvalid ? 1.0f / ltot : 0.0f;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const uint32_t w0 = pack_bf16x2(o[db][rg * 4 + 0] * inv, o[db][rg * 4 + 1] * inv);
        const uint32_t w1 = pack_bf16x2(o[db][rg * 4 + 2] * inv, o[db][rg * 4 + 3] * inv);
        const int slot = (db * 4 + rg) ^ (col & 15);
        *reinterpret_cast<uint2*>(ob + col * 256 + slot * 16 + hl * 8) = make_uint2(w0, w1);
      }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's rows are in LDS
    asm volatile("" ::: "memory");
    const int q0 = qi - col;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = 4 * i + (lane >> 4), cch = lane & 15;
      const uint4 vrow = *reinterpret_cast<const uint4*>(ob + r * 256 + ((cch ^ (r & 15)) * 16));
      if (q0 + r < N)
        *reinterpret_cast<uint4*>(out + ((qa + q0 + r) * Hq + h) * kHeadDim + cch * 8) = vrow;
    }
    if (qvalid && lse != nullptr && hl == 0)
      lse[(int64_t)h * Tq + qa + qi] = (m + __log2f(ltot)) * 0.69314718055994530942f;
  }
}

// The eight- and four-wave launches are separate kernels (distinct names in kernel traces).
#define NEO_GEN_ATTN_KERNEL(name, waves)                                                       \
  __global__ __launch_bounds__(waves * 64, 1) void name(                                       \
      const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_img,                      \
      const uint16_t* __restrict__ v_img, const uint16_t* __restrict__ k_pre,                  \
      const uint16_t* __restrict__ v_pre, const int32_t* __restrict__ cu_q,                    \
      const int32_t* __restrict__ cu_p, int Hq, int Hkv, int n_cg, int max_q, int max_p,       \
      int64_t Tq, int64_t Tp, float scale_log2, uint16_t* __restrict__ out,                    \
      float* __restrict__ lse) {                                                               \
    attn_bf16_body<false, waves>(q, k_img, v_img, k_pre, v_pre, cu_q, cu_p, nullptr, Hq, Hkv,  \
                                 n_cg, max_q, max_p, Tq, Tp, scale_log2, out, lse);            \
  }
NEO_GEN_ATTN_KERNEL(gen_attn_bf16_kernel, 8)

__global__ __launch_bounds__(512, 1) void gen_attn_bf16_split_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_img,
    const uint16_t* __restrict__ v_img, const uint16_t* __restrict__ k_pre,
    const uint16_t* __restrict__ v_pre, const int32_t* __restrict__ cu_q,
    const int32_t* __restrict__ cu_p, int Hq, int Hkv, int n_cg, int max_q, int max_p,
    int64_t Tq, int64_t Tp, float scale_log2, uint16_t* __restrict__ out,
    float* __restrict__ lse) {
  gen_attn_split_body(q, k_img, v_img, k_pre, v_pre, cu_q, cu_p, Hq, Hkv, n_cg, max_q, max_p, Tq,
                      Tp, scale_log2, out, lse);
}

#define NEO_PREFILL_ATTN_KERNEL(name, waves)                                                   \
  __global__ __launch_bounds__(waves * 64, 1) void name(                                       \
      const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,                          \
      const uint16_t* __restrict__ v, const int32_t* __restrict__ cu,                          \
      const int32_t* __restrict__ tidx, int Hq, int Hkv, int n_cg, int max_len, int64_t T,     \
      float scale_log2, uint16_t* __restrict__ out, float* __restrict__ lse) {                 \
    attn_bf16_body<true, waves>(q, k, v, k, v, cu, cu, tidx, Hq, Hkv, n_cg, max_len, 0, T, T,  \
                                scale_log2, out, lse);                                         \
  }
NEO_PREFILL_ATTN_KERNEL(prefill_attn_bf16_kernel, 8)
NEO_PREFILL_ATTN_KERNEL(prefill_attn_bf16_w4_kernel, 4)

// ---------------------------------------------------------------------------------------
// fp32 path
// ---------------------------------------------------------------------------------------
constexpr int kF32Keys = 32;
constexpr int kF32Threads = kAttnF32Threads;

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

// Workgroups of 64 query tokens (8 waves) while the launch has more than kSmallGrid of them;
// at or below it (at most half of the 256 CUs busy) workgroups of 32 query tokens, twice as
// many: the generation pass splits their keys between two groups of 4 waves (the split-key
// kernel), the prefill runs them as 4 waves.
#ifndef NEO_ATTN_SMALL_GRID
#define NEO_ATTN_SMALL_GRID 128
#endif
constexpr int64_t kSmallGrid = NEO_ATTN_SMALL_GRID;

// waves per workgroup for `chunks` 32-row query chunks per (sample, KV head)
int attn_waves(int64_t chunks, int64_t per_chunk_groups) {
  return ((chunks + 7) / 8) * per_chunk_groups <= kSmallGrid ? 4 : 8;
}

hipError_t launch_gen_attn_bf16(const void* q, const void* k_img, const void* v_img,
                                const void* k_pre, const void* v_pre, const int32_t* cu_q,
                                const int32_t* cu_p, int B, int Hq, int Hkv, int max_q,
                                int max_p, float scale, void* out, float* lse, int64_t Tq,
                                int64_t Tp, hipStream_t stream) {
  if (max_q == 0 || Tq == 0) return hipSuccess;
  const int G = Hq / Hkv;
  const int64_t chunks = (int64_t)G * ((max_q + 31) / 32);
  // small launches: 4 query chunks per workgroup, their keys split between two wave groups
  const bool split = attn_waves(chunks, (int64_t)Hkv * B) == 4;
  const int per_cg = split ? 4 : 8;
  const int64_t n_cg = (chunks + per_cg - 1) / per_cg;
  const int64_t blocks = n_cg * Hkv * B;
  const float scale_log2 = (float)((double)scale * 1.4426950408889634073599246810019);
  auto kern = split ? gen_attn_bf16_split_kernel : gen_attn_bf16_kernel;
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(512), 0, stream,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k_img),
                     static_cast<const uint16_t*>(v_img), static_cast<const uint16_t*>(k_pre),
                     static_cast<const uint16_t*>(v_pre), cu_q, cu_p, Hq, Hkv, (int)n_cg,
                     max_q, max_p, Tq, Tp, scale_log2, static_cast<uint16_t*>(out), lse);
  return hipGetLastError();
}

hipError_t launch_prefill_attn_bf16(const void* q, const void* k, const void* v,
                                    const int32_t* tidx, const int32_t* cu, int B, int Hq,
                                    int Hkv, int max_len, float scale, void* out, float* lse,
                                    int64_t T, hipStream_t stream) {
  if (max_len == 0 || T == 0) return hipSuccess;
  const int G = Hq / Hkv;
  const int64_t chunks = (int64_t)G * ((max_len + 31) / 32);
  const int waves = attn_waves(chunks, (int64_t)Hkv * B);
  const int64_t n_cg = (chunks + waves - 1) / waves;
  const int64_t blocks = n_cg * Hkv * B;
  const float scale_log2 = (float)((double)scale * 1.4426950408889634073599246810019);
  auto kern = waves == 8 ? prefill_attn_bf16_kernel : prefill_attn_bf16_w4_kernel;
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(waves * 64), 0, stream,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), cu, tidx, Hq, Hkv, (int)n_cg, max_len, T,
                     scale_log2, static_cast<uint16_t*>(out), lse);
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
