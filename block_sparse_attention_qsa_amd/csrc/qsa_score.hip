// a1 - block scoring: FP32 dot product of each verify query's 128-dim index
// query with the compressed key of every full 4-token block of its request.
//
// The arex-research.com article (section on the four optimisations, item 2)
// describes the MTP-verify reuse this kernel is built around: up to 4 queries
// of one request share a single load of each compressed-key tile.  Here a
// wave reads 4 key rows (1 KiB, 16 lanes x 16 B per row, fully coalesced) per
// load instruction and scores every row against all of the request's queries
// from registers, so each key byte crosses HBM once per request.  The
// contraction is 4 queries x 128: far too thin for MFMA, so it runs on the
// packed BF16 dot-product VALU op with FP32 accumulation and a DPP reduction
// across the 16 lanes of a row.
#include "qsa_common.hpp"
#include "qsa_launch.hpp"

namespace qsa {

// ROWS_PER_WAVE rows per wave, 4 waves per workgroup.
template <int ITERS>
__global__ __launch_bounds__(256) void score_kernel(Meta m, const uint16_t* __restrict__ idx_q,
                                                    const uint16_t* __restrict__ ckeys,
                                                    float* __restrict__ scores, int64_t ld) {
  constexpr int kRowsPerWg = 16 * ITERS;
  const int r = blockIdx.y;
  int nblk = m.seq_len[r] >> 2;
  if (nblk > m.max_blocks) nblk = m.max_blocks;
  const int row0 = blockIdx.x * kRowsPerWg;
  if (row0 >= nblk) return;
  const int qs = m.q_start[r];
  const int nq = m.q_start[r + 1] - qs;
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int sub = lane & 15;      // 8 dims per lane: sub*8 .. sub*8+7
  const int rsub = lane >> 4;     // row within a group of 4

  u32x4 iq[QSA_MAX_Q_PER_REQ];
#pragma unroll
  for (int qi = 0; qi < QSA_MAX_Q_PER_REQ; ++qi) {
    if (qi < nq)
      iq[qi] = *reinterpret_cast<const u32x4*>(idx_q + (int64_t)(qs + qi) * QSA_INDEX_DIM + sub * 8);
    else
      iq[qi] = u32x4{0u, 0u, 0u, 0u};
  }

  const uint16_t* kbase = ckeys + (int64_t)m.blk_start[r] * QSA_INDEX_DIM + sub * 8;
  u32x4 kr[ITERS];
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    const int row = row0 + it * 16 + wave * 4 + rsub;
    if (row < nblk)
      kr[it] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kbase + (int64_t)row * QSA_INDEX_DIM));
    else
      kr[it] = u32x4{0u, 0u, 0u, 0u};
  }

  // Lane sub = 4Q + x of a 16-lane row ends with query Q's score for that
  // row: a butterfly over the row sums the four queries' partial dot
  // products at once (exchange with lane ^ 8, then with the mirrored lane of
  // the 8-lane half, then inside the quad), 5 DPP adds instead of 4 x 4.
  const bool hi8 = (sub & 8) != 0, hi4 = (sub & 4) != 0;
  const int qsel = sub >> 2;
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    const int row = row0 + it * 16 + wave * 4 + rsub;
    float a[QSA_MAX_Q_PER_REQ];
#pragma unroll
    for (int qi = 0; qi < QSA_MAX_Q_PER_REQ; ++qi) {
      float acc = 0.f;
      acc = fdot2_bf16(kr[it].x, iq[qi].x, acc);
      acc = fdot2_bf16(kr[it].y, iq[qi].y, acc);
      acc = fdot2_bf16(kr[it].z, iq[qi].z, acc);
      acc = fdot2_bf16(kr[it].w, iq[qi].w, acc);
      a[qi] = acc;
    }
    const float k0 = hi8 ? a[2] : a[0], k1 = hi8 ? a[3] : a[1];
    const float s0 = hi8 ? a[0] : a[2], s1 = hi8 ? a[1] : a[3];
    const float b0 = k0 + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(s0), 0x128, 0xF, 0xF, false));
    const float b1 = k1 + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(s1), 0x128, 0xF, 0xF, false));
    const float kk = hi4 ? b1 : b0, ss = hi4 ? b0 : b1;
    float c = kk + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(ss), 0x141, 0xF, 0xF, false));
    c += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(c), 0x4E, 0xF, 0xF, false));
    c += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(c), 0xB1, 0xF, 0xF, false));
    if ((sub & 3) == 0 && qsel < nq && row < nblk) scores[(int64_t)(qs + qsel) * ld + row] = c;
  }
}

hipError_t launch_score(const Meta& m, const void* idx_q, const void* ckeys, float* scores, int64_t ld,
                        hipStream_t stream) {
  const int64_t mb = m.max_blocks;
  if (mb == 0) return hipSuccess;
  auto wgs = [&](int rows) { return ((mb + rows - 1) / rows) * (int64_t)m.num_req; };
  const uint16_t* iq = static_cast<const uint16_t*>(idx_q);
  const uint16_t* ck = static_cast<const uint16_t*>(ckeys);
  if (wgs(64) >= 1024) {
    dim3 grid((unsigned)((mb + 63) / 64), (unsigned)m.num_req);
    score_kernel<4><<<grid, 256, 0, stream>>>(m, iq, ck, scores, ld);
  } else if (wgs(32) >= 1024) {
    dim3 grid((unsigned)((mb + 31) / 32), (unsigned)m.num_req);
    score_kernel<2><<<grid, 256, 0, stream>>>(m, iq, ck, scores, ld);
  } else {
    dim3 grid((unsigned)((mb + 15) / 16), (unsigned)m.num_req);
    score_kernel<1><<<grid, 256, 0, stream>>>(m, iq, ck, scores, ld);
  }
  return hipGetLastError();
}

}  // namespace qsa
