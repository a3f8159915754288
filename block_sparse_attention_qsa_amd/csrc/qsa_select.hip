// a2 - top-k block selection by radix select, and a3 - the position buffer.
//
// The arex-research.com article (section on the four optimisations, item 1)
// keeps at most 512 full blocks per query from an FP32 score buffer with a
// persistent radix selector, and keeps the current partial block without
// selection, which fixes the position buffer at 2,051 entries.  The 10100.com
// article (first optimisation) adds the last step: locate the kept pieces in
// the KV cache.
//
// One 1024-thread workgroup handles one query:
//   1. FP32 scores -> order-preserving uint32 keys (-0.0 folded onto +0.0),
//      staged in LDS when they fit (else re-read from the L2-resident buffer).
//   2. Three MSB-first radix passes (11, 11, 10 bits) with LDS histograms find
//      the key T of the k-th best block and how many blocks equal to T to keep.
//   3. An ordered compaction (two block scans over contiguous per-thread
//      segments) keeps every key > T and the lowest-index keys == T, so ties go
//      to the lower block index and the output comes out in ascending order.
#include "qsa_common.hpp"
#include "qsa_launch.hpp"

namespace qsa {

constexpr int kKeyCap = 16384;   // keys staged in LDS (64 KiB)

template <bool kWritePos>
__global__ __launch_bounds__(kSelectThreads) void select_kernel(Meta m, const float* __restrict__ scores,
                                                                int64_t ld, int k, int32_t* __restrict__ sel,
                                                                int32_t* __restrict__ n_sel,
                                                                int32_t* __restrict__ pos,
                                                                int32_t* __restrict__ n_pos, int width) {
  constexpr int NT = kSelectThreads;
  __shared__ uint32_t keys_lds[kKeyCap];
  __shared__ uint32_t hist[kRadixBins];
  __shared__ uint32_t scan_scratch[NT / kWave + 1];
  __shared__ uint32_t s_prefix, s_krem;

  const int q = blockIdx.x;
  const int tid = threadIdx.x;
  const int r = request_of(m.q_start, m.num_req, q);
  const int qs = m.q_start[r];
  const int nq = m.q_start[r + 1] - qs;
  const int L = m.seq_len[r] - nq + 1 + (q - qs);
  int nf = L >> 2;
  if (nf > m.max_blocks) nf = m.max_blocks;
  const int pl = L & 3;
  const int kv0 = m.kv_start[r];
  const float* srow = scores + (int64_t)q * ld;
  int32_t* sel_row = sel + (int64_t)q * k;
  int32_t* pos_row = kWritePos ? pos + (int64_t)q * width : nullptr;

  if (nf <= k) {
    // every full block is kept: positions are simply the causal prefix
    for (int i = tid; i < k; i += NT) sel_row[i] = i < nf ? i : -1;
    if (kWritePos) {
      const int np = 4 * nf + pl;
      for (int i = tid; i < width; i += NT) pos_row[i] = i < np ? kv0 + i : -1;
    }
    if (tid == 0) {
      n_sel[q] = nf;
      if (kWritePos) n_pos[q] = 4 * nf + pl;
    }
    return;
  }

  const bool in_lds = nf <= kKeyCap;
  if (in_lds)
    for (int i = tid; i < nf; i += NT) keys_lds[i] = score_key(srow[i]);
  auto key_at = [&](int i) -> uint32_t { return in_lds ? keys_lds[i] : score_key(srow[i]); };

  uint32_t prefix = 0u, pmask = 0u, krem = (uint32_t)k;
#pragma unroll 1
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const uint32_t dmask = pass == 2 ? 0x3FFu : 0x7FFu;
    for (int i = tid; i < kRadixBins; i += NT) hist[i] = 0u;
    __syncthreads();
    for (int i = tid; i < nf; i += NT) {
      const uint32_t key = key_at(i);
      if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & dmask], 1u);
    }
    __syncthreads();
    // thread t owns bins 2047-2t (upper) and 2046-2t (lower); scan from the top
    const int bu = kRadixBins - 1 - 2 * tid;
    const uint32_t hu = hist[bu], hl = hist[bu - 1];
    uint32_t tot;
    const uint32_t above = block_exclusive_scan<NT>(hu + hl, scan_scratch, &tot);
    if (above < krem && krem <= above + hu) {
      s_prefix = prefix | ((uint32_t)bu << shift);
      s_krem = krem - above;
    } else if (above + hu < krem && krem <= above + hu + hl) {
      s_prefix = prefix | ((uint32_t)(bu - 1) << shift);
      s_krem = krem - above - hu;
    }
    __syncthreads();
    prefix = s_prefix;
    krem = s_krem;
    pmask |= dmask << shift;
  }
  const uint32_t T = prefix;        // key of the k-th best block
  const uint32_t need_eq = krem;    // blocks equal to T that are kept (lowest indices first)

  const int E = (nf + NT - 1) / NT;
  const int beg = min(tid * E, nf), end = min(beg + E, nf);
  uint32_t eq = 0;
  for (int i = beg; i < end; ++i) eq += key_at(i) == T;
  uint32_t tot;
  const uint32_t eq_before = block_exclusive_scan<NT>(eq, scan_scratch, &tot);
  uint32_t cnt = 0, seen = eq_before;
  for (int i = beg; i < end; ++i) {
    const uint32_t key = key_at(i);
    if (key > T) ++cnt;
    else if (key == T) { cnt += seen < need_eq; ++seen; }
  }
  uint32_t o = block_exclusive_scan<NT>(cnt, scan_scratch, &tot);
  seen = eq_before;
  for (int i = beg; i < end; ++i) {
    const uint32_t key = key_at(i);
    bool take = key > T;
    if (key == T) { take = seen < need_eq; ++seen; }
    if (take) {
      sel_row[o] = i;
      if (kWritePos) {
        const int p0 = kv0 + 4 * i;
        pos_row[4 * o + 0] = p0;
        pos_row[4 * o + 1] = p0 + 1;
        pos_row[4 * o + 2] = p0 + 2;
        pos_row[4 * o + 3] = p0 + 3;
      }
      ++o;
    }
  }
  if (kWritePos) {
    for (int i = 4 * k + tid; i < width; i += NT) {
      const int t = i - 4 * k;
      pos_row[i] = t < pl ? kv0 + 4 * nf + t : -1;
    }
  }
  if (tid == 0) {
    n_sel[q] = k;
    if (kWritePos) n_pos[q] = 4 * k + pl;
  }
}

__global__ __launch_bounds__(256) void build_index_kernel(Meta m, const int32_t* __restrict__ sel,
                                                          const int32_t* __restrict__ n_sel, int k,
                                                          int32_t* __restrict__ pos, int32_t* __restrict__ n_pos,
                                                          int width) {
  const int q = blockIdx.x;
  const int r = request_of(m.q_start, m.num_req, q);
  const int qs = m.q_start[r];
  const int nq = m.q_start[r + 1] - qs;
  const int L = m.seq_len[r] - nq + 1 + (q - qs);
  int nf = L >> 2;
  if (nf > m.max_blocks) nf = m.max_blocks;
  const int pl = L & 3;
  const int kv0 = m.kv_start[r];
  int ns = n_sel[q];
  ns = ns < 0 ? 0 : (ns > k ? k : ns);
  const int np = 4 * ns + pl;
  const int32_t* srow = sel + (int64_t)q * k;
  int32_t* prow = pos + (int64_t)q * width;
  for (int i = threadIdx.x; i < width; i += blockDim.x) {
    int v;
    if (i < 4 * ns) v = kv0 + 4 * srow[i >> 2] + (i & 3);
    else if (i < np) v = kv0 + 4 * nf + (i - 4 * ns);
    else v = -1;
    prow[i] = v;
  }
  if (threadIdx.x == 0) n_pos[q] = np;
}

hipError_t launch_select(const Meta& m, const float* scores, int64_t ld, int k, int32_t* sel, int32_t* n_sel,
                         int32_t* pos, int32_t* n_pos, int width, hipStream_t stream) {
  if (pos)
    select_kernel<true><<<m.num_q, kSelectThreads, 0, stream>>>(m, scores, ld, k, sel, n_sel, pos, n_pos, width);
  else
    select_kernel<false><<<m.num_q, kSelectThreads, 0, stream>>>(m, scores, ld, k, sel, n_sel, nullptr, nullptr,
                                                                 width);
  return hipGetLastError();
}

hipError_t launch_build_index(const Meta& m, const int32_t* sel, const int32_t* n_sel, int k, int32_t* pos,
                              int32_t* n_pos, int width, hipStream_t stream) {
  build_index_kernel<<<m.num_q, 256, 0, stream>>>(m, sel, n_sel, k, pos, n_pos, width);
  return hipGetLastError();
}

}  // namespace qsa
