// a1 - block scoring: FP32 dot product of each verify query's 128-dim index
// query with the compressed key of every full 4-token block of its request.
//
// The arex-research.com article (section on the four optimisations, item 2)
// describes the MTP-verify reuse this kernel is built around: up to 4 queries
// of one request share a single load of each compressed-key tile, so each key
// byte crosses HBM once per request.
//
// The contraction of a 16-row key tile with the request's queries is one
// bf16 MFMA 16x16x32 chain (4 steps over the 128 dimensions): the key rows
// are the M side, the queries the N side (4 of 16 columns used - the matrix
// core still does it in a fraction of the issue time of packed dot products
// plus a cross-lane reduction).  Products of two BF16 values are exact and
// accumulate in FP32.
//
// Step kk of the chain contracts dimensions 32kk .. 32kk+31: lane l = 16g + n
// of a wave loads bytes 64kk + 16g .. 64kk + 16g + 15 of key row n of a
// 16-row group, so one load instruction reads 64 contiguous bytes of each of
// 16 rows and the two instructions of a 128-byte line follow each other.  The
// result leaves lane (g, n) with query n's scores of rows 4g .. 4g+3, stored
// as one 16-byte vector.
//
// Each wave takes tiles of 16U rows.  Up to 16,384 workgroups a wave has one
// tile (measured fastest on MI355X from 50K-token batches to 1M-token rows);
// on larger batches waves loop over several tiles, with the next tile's loads
// issued before the current one is contracted.
#include "qsa_common.hpp"
#include "qsa_launch.hpp"

namespace qsa {

constexpr int kScoreWaves = 4;             // waves per workgroup
constexpr int kKeyPolicy = 0;              // buffer-load cache policy of the key stream
constexpr int kRowBytes = QSA_INDEX_DIM * 2;

template <int U>
struct KeyTile {
  u32x4 w[U][4];    // group u, step kk: dimensions 32kk + 8g .. 32kk + 8g + 7 of row 16u + n
};

template <int U>
__device__ __forceinline__ void load_tile(KeyTile<U>& t, __amdgpu_buffer_rsrc_t rs, int row0, int n, int g) {
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int off = (row0 + 16 * u + n) * kRowBytes + 16 * g;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      t.w[u][kk] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off + 64 * kk, 0,
                                                                                    kKeyPolicy));
  }
}

// Contract one tile and store the scores of rows below nblk (one 16-byte
// store per lane when the score rows are 16-byte aligned).
template <int U>
__device__ __forceinline__ void score_tile(const KeyTile<U>& t, const bf16x8 (&qb)[4], float* qrow, bool qvalid,
                                           bool vec, int row0, int nblk, int g) {
#pragma unroll
  for (int u = 0; u < U; ++u) {
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, t.w[u][kk]), qb[kk], acc, 0, 0, 0);
    const int row = row0 + 16 * u + 4 * g;
    if (qvalid) {
      if (vec && row + 3 < nblk) {
        *reinterpret_cast<f32x4*>(qrow + row) = acc;
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (row + i < nblk) qrow[row + i] = acc[i];
      }
    }
  }
}

// Grid (x, request).  Wave w of workgroup x takes tiles x*4 + w, then every
// gridDim.x * 4 tiles after it, of its request's rows.
template <int U>
__global__ __launch_bounds__(256) void score_kernel(Meta m, const uint16_t* __restrict__ idx_q,
                                                    const uint16_t* __restrict__ ckeys,
                                                    float* __restrict__ scores, int64_t ld, int vec) {
  constexpr int R = 16 * U;
  const int r = blockIdx.y;
  int nblk = m.seq_len[r] >> 2;
  if (nblk > m.max_blocks) nblk = m.max_blocks;
  const int ntiles = (nblk + R - 1) / R;
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int stride = gridDim.x * kScoreWaves;
  int tile = blockIdx.x * kScoreWaves + wave;
  if (tile >= ntiles) return;                 // no barriers below: waves leave on their own
  const int n = lane & 15, g = lane >> 4;

  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(ckeys) + (int64_t)m.blk_start[r] * QSA_INDEX_DIM, 0, nblk * kRowBytes, 0x00020000);
  KeyTile<U> a, b;
  load_tile<U>(a, rs, tile * R, n, g);

  const int qs = m.q_start[r];
  const int nq = m.q_start[r + 1] - qs;
  const bool qvalid = n < nq;
  bf16x8 qb[4];
  {
    const uint16_t* qp = idx_q + (int64_t)(qs + (qvalid ? n : 0)) * QSA_INDEX_DIM + 8 * g;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      qb[kk] = __builtin_bit_cast(bf16x8, qvalid ? *reinterpret_cast<const u32x4*>(qp + 32 * kk)
                                                 : u32x4{0u, 0u, 0u, 0u});
  }
  float* qrow = scores + (int64_t)(qs + (qvalid ? n : 0)) * ld;

  // Ping-pong over two register tiles: the loads of the next tile are in
  // flight while the current one is contracted.
  for (;;) {
    int next = tile + stride;
    if (next < ntiles) load_tile<U>(b, rs, next * R, n, g);
    __builtin_amdgcn_sched_barrier(0);
    score_tile<U>(a, qb, qrow, qvalid, vec != 0, tile * R, nblk, g);
    if (next >= ntiles) break;
    tile = next;
    next = tile + stride;
    if (next < ntiles) load_tile<U>(a, rs, next * R, n, g);
    __builtin_amdgcn_sched_barrier(0);
    score_tile<U>(b, qb, qrow, qvalid, vec != 0, tile * R, nblk, g);
    if (next >= ntiles) break;
    tile = next;
  }
}

hipError_t launch_score(const Meta& m, const void* idx_q, const void* ckeys, float* scores, int64_t ld,
                        hipStream_t stream) {
  const int64_t mb = m.max_blocks;
  if (mb == 0) return hipSuccess;
  constexpr int U = 1;
  constexpr int kTargetWgs = 16384;           // beyond this, waves loop over several tiles
  const int64_t tiles = (mb + 16 * U - 1) / (16 * U);
  int64_t gx = (tiles + kScoreWaves - 1) / kScoreWaves;
  const int64_t cap = (kTargetWgs + m.num_req - 1) / m.num_req;
  if (gx > cap) gx = cap;
  const dim3 grid((unsigned)gx, (unsigned)m.num_req);
  const int vec = (ld % 4 == 0) && (reinterpret_cast<uintptr_t>(scores) % 16 == 0);
  score_kernel<U><<<grid, 256, 0, stream>>>(m, static_cast<const uint16_t*>(idx_q),
                                            static_cast<const uint16_t*>(ckeys), scores, ld, vec);
  return hipGetLastError();
}

}  // namespace qsa
