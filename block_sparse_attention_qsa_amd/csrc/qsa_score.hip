// a1 - block scoring: FP32 dot product of each verify query's 128-dim index
// query with the compressed key of every full 4-token block of its request.
//
// The arex-research.com article (section on the four optimisations, item 2)
// describes the MTP-verify reuse this kernel is built around: up to 4 queries
// of one request share a single load of each compressed-key tile, so each key
// byte crosses HBM once per request.
//
// The contraction of a 16-row key tile with the request's queries is one
// bf16 MFMA chain (qsa_score_tile.hpp).  Each wave takes 16-row tiles; up to
// 16,384 workgroups a wave has one tile (measured fastest on MI355X from
// 50K-token batches to 1M-token rows); on larger batches waves loop over
// several tiles.
#include "qsa_launch.hpp"
#include "qsa_score_tile.hpp"

namespace qsa {

constexpr int kScoreWaves = 4;             // waves per workgroup

// Store the scores of rows row .. row+3 below nblk (one 16-byte store when
// the score rows are 16-byte aligned) at byte qoff + 4 * row of the buffer
// rs.  With kWt the stores are device-scope (they write through the L2),
// so the end of the kernel does not have a few MB of dirty L2 lines to
// write back before the selection can start: −0.5 µs per step for a
// 32-request batch, +0.7 µs for one 1M-token request, whose four long rows
// stream better through the L2.
template <bool kWt>
__device__ __forceinline__ void store_scores(__amdgpu_buffer_rsrc_t rs, uint32_t qoff, f32x4 acc, bool vec, int row,
                                             int nblk) {
  constexpr int kCpol = kWt ? kCpolDevice : 0;
  if (vec && row + 3 < nblk) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc), rs, qoff + 4 * row, 0, kCpol);
  } else {
    // (__float_as_uint of the element: a bit cast of a vector-element
    // subscript reads element 0 with this compiler)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (row + i < nblk)
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[i]), rs, qoff + 4 * (row + i), 0, kCpol);
  }
}

// Grid (x, request).  Wave w of workgroup x takes tiles x*4 + w, then every
// gridDim.x * 4 tiles after it, of its request's rows.  A wave's tile goes
// to its own 4 KiB of LDS (direct-to-LDS loads, whole lines, non-temporal),
// is read back into MFMA operands, and the next tile's loads are issued
// into the same LDS before the current tile is contracted.
template <bool kWt>
__global__ __launch_bounds__(256) void score_kernel(Meta m, const uint16_t* __restrict__ idx_q,
                                                    const uint16_t* __restrict__ ckeys,
                                                    float* __restrict__ scores, int64_t ld, int vec) {
  __shared__ __attribute__((aligned(16))) uint8_t tile_s[kScoreWaves][kTileBytes];
  const int r = blockIdx.y;
  // All of the request's metadata is read at once (one scalar round trip
  // after the kernel arguments), before anything depends on it.
  const int seq = m.seq_len[r], row0 = m.blk_start[r], qs = m.q_start[r], qe = m.q_start[r + 1];
  asm volatile("" ::"s"(seq), "s"(row0), "s"(qs), "s"(qe));   // keeps the four loads together, up here
  int nblk = seq >> 2;
  if (threadIdx.x == 0 && blockIdx.x == 0) {
    QSA_DCHECK(m.err, qe - qs >= 1 && qe - qs <= QSA_MAX_Q_PER_REQ && seq >= qe - qs, QSA_ERROR_BAD_QUERIES);
    QSA_DCHECK(m.err, nblk <= m.max_blocks, QSA_ERROR_BAD_BLOCKS);
  }
  if (nblk > m.max_blocks) nblk = m.max_blocks;
  const int ntiles = (nblk + 15) / 16;
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int stride = gridDim.x * kScoreWaves;
  int tile = blockIdx.x * kScoreWaves + wave;
  if (tile >= ntiles) return;                 // no barriers below: waves leave on their own
  const int n = lane & 15, g = lane >> 4;
  uint8_t* my_tile = tile_s[wave];

  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(ckeys) + (int64_t)row0 * QSA_INDEX_DIM, 0, nblk * kKeyRowBytes, 0x00020000);
  load_key_tile_lds(my_tile, rs, tile * 16, lane);
  __builtin_amdgcn_sched_barrier(0);          // key loads before the query loads

  const int nq = qe - qs;
  const bool qvalid = n < nq;
  bf16x8 qb[4];
  load_index_queries(qb, idx_q, qs, nq, n, g);
  // the request's first score row as the (wave-uniform) buffer base, each
  // lane's query row as an offset
  const __amdgpu_buffer_rsrc_t srs =
      __builtin_amdgcn_make_buffer_rsrc(scores + (int64_t)qs * ld, 0, 0x7fffffff, 0x00020000);
  const uint32_t qoff = (uint32_t)((qvalid ? n : 0) * ld * 4);

  for (;;) {
    __builtin_amdgcn_s_waitcnt(0);            // this wave's tile (and the queries) have landed
    KeyTile t;
    read_key_tile_lds(t, my_tile, n, g);
    const int next = tile + stride;
    if (next < ntiles) {
      __builtin_amdgcn_s_waitcnt(0);          // LDS reads done before the buffer is refilled
      load_key_tile_lds(my_tile, rs, next * 16, lane);
    }
    __builtin_amdgcn_sched_barrier(0);
    const f32x4 sc = contract_key_tile(t, qb);
    if (qvalid) store_scores<kWt>(srs, qoff, sc, vec != 0, tile * 16 + 4 * g, nblk);
    if (next >= ntiles) break;
    tile = next;
  }
}

hipError_t launch_score(const Meta& m, const void* idx_q, const void* ckeys, float* scores, int64_t ld,
                        hipStream_t stream) {
  const int64_t mb = m.max_blocks;
  if (mb == 0) return hipSuccess;
  constexpr int kTargetWgs = 16384;           // beyond this, waves loop over several tiles
  const int64_t tiles = (mb + 15) / 16;
  int64_t gx = (tiles + kScoreWaves - 1) / kScoreWaves;
  const int64_t cap = (kTargetWgs + m.num_req - 1) / m.num_req;
  if (gx > cap) gx = cap;
  const dim3 grid((unsigned)gx, (unsigned)m.num_req);
  const int vec = (ld % 4 == 0) && (reinterpret_cast<uintptr_t>(scores) % 16 == 0);
  const uint16_t* iq = static_cast<const uint16_t*>(idx_q);
  const uint16_t* ck = static_cast<const uint16_t*>(ckeys);
  if (m.num_req > 1) score_kernel<true><<<grid, 256, 0, stream>>>(m, iq, ck, scores, ld, vec);
  else score_kernel<false><<<grid, 256, 0, stream>>>(m, iq, ck, scores, ld, vec);
  return hipGetLastError();
}

}  // namespace qsa
