// a2 - top-k block selection by radix select, and a3 - the position buffer.
//
// The arex-research.com article (section on the four optimisations, item 1)
// keeps at most 512 full blocks per query from an FP32 score buffer with a
// persistent radix selector, and keeps the current partial block without
// selection, which fixes the position buffer at 2,051 entries.  The 10100.com
// article (first optimisation) adds the last step: locate the kept pieces in
// the KV cache.
//
// One 1024-thread workgroup handles one query.  Rows of up to 65,536 blocks
// are held in registers (contiguous segment per thread); longer rows use a
// streaming variant that stages only the threshold bin's keys in LDS.
//   1. FP32 scores -> order-preserving uint32 keys (-0.0 folded onto +0.0),
//      staged in LDS when they fit.
//   2. Three MSB-first radix passes (11, 11, 10 bits) with LDS histograms find
//      the key T of the k-th best block and how many blocks equal to T to keep.
//   3. An ordered compaction (one packed block scan over contiguous
//      per-thread segments) keeps every key > T and the lowest-index keys == T,
//      so ties go to the lower block index and the output is ascending.
// Scans are DPP shift-scans inside each 16-lane row; the bucket search after a
// histogram pass is done by a single wave.  When the keys do not fit in LDS,
// the first pass streams the score buffer and only the keys falling in the
// chosen top-level bin are staged for the remaining passes.
#include "qsa_common.hpp"
#include "qsa_launch.hpp"

namespace qsa {

constexpr int kKeyCap = 32768;   // keys staged in LDS (128 KiB of the 160 KiB a workgroup may use)
constexpr int kBatch = 8;        // loads a thread keeps in flight while streaming scores

// Histogram increment for a wave: when every active lane carries the same
// bin (long runs of tied scores) one lane adds the whole count.
__device__ __forceinline__ void hist_add(uint32_t* hist, uint32_t bin, bool active) {
  const uint64_t act = __ballot(active);
  if (act == 0) return;
  const int first = __builtin_ctzll(act);
  const uint32_t b0 = (uint32_t)__builtin_amdgcn_readlane((int)bin, first);
  if (__ballot(active && bin != b0) == 0) {
    if (lane_id() == first) atomicAdd(&hist[b0], (uint32_t)__popcll(act));
  } else if (active) {
    atomicAdd(&hist[bin], 1u);
  }
}

// One wave finds, scanning hist[2047 .. 0] from the top, the bin where the
// running count first reaches krem, and publishes the refined prefix, the
// count still to take inside that bin and the bin's population.  Level one:
// lane l sums bins 2016-32l .. 2047-32l and a wave scan picks the lane; level
// two: lanes 0..31 take that lane's 32 bins (highest first) and a second scan
// picks the bin.  No loops, no per-bin branches.
__device__ __forceinline__ void find_bucket(const uint32_t* hist, uint32_t krem, uint32_t prefix, int shift,
                                            uint32_t* s_prefix, uint32_t* s_krem, uint32_t* s_count) {
  const int lane = lane_id();
  const int lo = kRadixBins - 32 - 32 * lane;
  const u32x4* h4 = reinterpret_cast<const u32x4*>(hist + lo);
  uint32_t sum = 0;
#pragma unroll
  for (int v = 0; v < 8; ++v) {
    const u32x4 x = h4[v];
    sum += x.x + x.y + x.z + x.w;
  }
  const uint32_t inc = wave_inclusive_scan(sum);
  const uint32_t exc = inc - sum;
  const uint64_t hit = __ballot(exc < krem && krem <= inc);
  if (hit == 0) return;                                // unreachable while krem <= population
  const int lh = __builtin_ctzll(hit);
  const uint32_t above = (uint32_t)__builtin_amdgcn_readlane((int)exc, lh);
  const int lo_h = kRadixBins - 32 - 32 * lh;
  const uint32_t cb = lane < 32 ? hist[lo_h + 31 - lane] : 0u;
  const uint32_t run = above + wave_inclusive_scan(cb) - cb;
  const uint64_t hit2 = __ballot(lane < 32 && run < krem && krem <= run + cb);
  if (hit2 == 0) return;
  if (lane == __builtin_ctzll(hit2)) {
    *s_prefix = prefix | ((uint32_t)(lo_h + 31 - lane) << shift);
    *s_krem = krem - run;
    *s_count = cb;
  }
}

// Register-resident selector for rows of at most E * 1024 keys: thread t
// holds the contiguous keys [t*E, t*E + E) in registers through the histogram
// passes and the ordered compaction.
template <int E, bool kWritePos>
__global__ __launch_bounds__(kSelectThreads) void select_reg_kernel(Meta m, const float* __restrict__ scores,
                                                                    int64_t ld, int k, int32_t* __restrict__ sel,
                                                                    int32_t* __restrict__ n_sel,
                                                                    int32_t* __restrict__ pos,
                                                                    int32_t* __restrict__ n_pos, int width) {
  constexpr int NT = kSelectThreads;
  __shared__ uint32_t hist[2][kRadixBins];
  __shared__ uint32_t scan_scratch[NT / kWave];
  __shared__ uint32_t s_prefix, s_krem, s_count;

  const int q = blockIdx.x;
  const int tid = threadIdx.x, wave = tid / kWave;
  const float* srow = scores + (int64_t)q * ld;

  // Score loads are issued first, speculatively: thread t owns the fixed segment
  // [t*E, t*E + E) clipped to the row stride, so the loads do not wait for the
  // request metadata; keys past the query's block count are zeroed afterwards.
  const int beg = tid * E;
  const bool vec = (reinterpret_cast<uintptr_t>(srow) & 15) == 0;
  float sv[E];
#pragma unroll
  for (int v = 0; v < E / 4; ++v) {
    const int i = beg + 4 * v;
    if (vec && i + 4 <= ld) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(srow + i);
      sv[4 * v] = x.x;
      sv[4 * v + 1] = x.y;
      sv[4 * v + 2] = x.z;
      sv[4 * v + 3] = x.w;
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u) sv[4 * v + u] = i + u < ld ? srow[i + u] : 0.f;
    }
  }

  const int r = request_of(m.q_start, m.num_req, q);
  const int qs = m.q_start[r];
  const int nq = m.q_start[r + 1] - qs;
  const int L = m.seq_len[r] - nq + 1 + (q - qs);
  int nf = L >> 2;
  if (nf > m.max_blocks) nf = m.max_blocks;
  if (nf > E * NT) nf = E * NT;                      // launcher picks E >= max_blocks / 1024
  const int pl = L & 3;
  const int kv0 = m.kv_start[r];
  int32_t* sel_row = sel + (int64_t)q * k;
  int32_t* pos_row = kWritePos ? pos + (int64_t)q * width : nullptr;

  if (nf <= k) {
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

  // ---- keys of this thread's segment.  Slots past the row hold key 0: every
  // finite score maps to a key >= 0x00800000 (top-11-bit digit >= 4), so with
  // nf > k the zeros sit alone in the lowest bin and never reach the threshold.
  const int cnt = max(0, min(E, nf - beg));
  uint32_t kk[E];
#pragma unroll
  for (int e = 0; e < E; ++e) kk[e] = e < cnt ? score_key(sv[e]) : 0u;
  for (int i = tid; i < 2 * kRadixBins; i += NT) (&hist[0][0])[i] = 0u;
  __syncthreads();

  // ---- MSB-first radix passes (11, 11, 10 bits); stop early once the
  // threshold bin is taken whole.
  uint32_t prefix = 0u, pmask = 0u, krem = (uint32_t)k;
#pragma unroll 1
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const uint32_t dmask = pass == 2 ? 0x3FFu : 0x7FFu;
    uint32_t* cur = hist[pass & 1];
    uint32_t* nxt = hist[(pass + 1) & 1];
#pragma unroll
    for (int e = 0; e < E; ++e) hist_add(cur, (kk[e] >> shift) & dmask, (kk[e] & pmask) == prefix);
    for (int i = tid; i < kRadixBins; i += NT) nxt[i] = 0u;   // last read before the previous barrier
    __syncthreads();
    if (wave == 0) find_bucket(cur, krem, prefix, shift, &s_prefix, &s_krem, &s_count);
    __syncthreads();
    prefix = s_prefix;
    krem = s_krem;
    const uint32_t bin_count = s_count;
    pmask |= dmask << shift;
    if (krem == bin_count) break;
  }
  const uint32_t T = prefix, M = pmask, need = krem;

  // ---- ordered compaction: keep (key & M) > T, and the first `need` keys with
  // (key & M) == T in index order.  One packed scan: > T count in the high 12
  // bits, == T count in the low 20.
  uint32_t gt = 0, eq = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const uint32_t km = kk[e] & M;
    gt += km > T;
    eq += km == T;
  }
  uint32_t tot;
  const uint32_t before = block_exclusive_scan<NT>((gt << 20) | eq, scan_scratch, &tot);
  const uint32_t eq_before = before & 0xFFFFFu;
  uint32_t o = (before >> 20) + min(eq_before, need);
  uint32_t seen = eq_before;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const uint32_t km = kk[e] & M;
    bool take = km > T;
    if (km == T) {
      take = seen < need;
      ++seen;
    }
    if (take) {
      const int i = beg + e;
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

template <bool kWritePos>
__global__ __launch_bounds__(kSelectThreads) void select_stream_kernel(Meta m, const float* __restrict__ scores,
                                                                int64_t ld, int k, int32_t* __restrict__ sel,
                                                                int32_t* __restrict__ n_sel,
                                                                int32_t* __restrict__ pos,
                                                                int32_t* __restrict__ n_pos, int width) {
  constexpr int NT = kSelectThreads;
  __shared__ uint32_t keys_lds[kKeyCap];
  __shared__ uint32_t hist[kRadixBins];
  __shared__ uint32_t scan_scratch[NT / kWave];
  __shared__ uint32_t s_prefix, s_krem, s_count, s_ncand;

  const int q = blockIdx.x;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
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

  // ---- 1. keys.  All nf keys go to LDS when they fit; otherwise the first
  // radix pass streams the score buffer and only the keys of the chosen
  // top-level bin are staged for the later passes.
  const bool staged = nf <= kKeyCap;
  if (staged) {
#pragma unroll
    for (int b = 0; b < kKeyCap / NT; b += kBatch) {
      float v[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int i = (b + u) * NT + tid;
        v[u] = i < nf ? srow[i] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int i = (b + u) * NT + tid;
        if (i < nf) keys_lds[i] = score_key(v[u]);
      }
    }
  }

  // ---- 2. MSB-first radix passes over 11, 11 and 10 bits.
  int nkeys = staged ? nf : 0;
  bool from_lds = staged;
  uint32_t prefix = 0u, pmask = 0u, krem = (uint32_t)k;
#pragma unroll 1
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const uint32_t dmask = pass == 2 ? 0x3FFu : 0x7FFu;
    for (int i = tid; i < kRadixBins; i += NT) hist[i] = 0u;
    __syncthreads();
    if (from_lds) {
      for (int i0 = 0; i0 < nkeys; i0 += NT) {
        const int i = i0 + tid;
        const uint32_t key = i < nkeys ? keys_lds[i] : 0u;
        hist_add(hist, (key >> shift) & dmask, i < nkeys && (key & pmask) == prefix);
      }
    } else {
      for (int base = 0; base < nf; base += NT * kBatch) {
        float v[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const int i = base + u * NT + tid;
          v[u] = i < nf ? srow[i] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const int i = base + u * NT + tid;
          const uint32_t key = score_key(v[u]);
          hist_add(hist, (key >> shift) & dmask, i < nf && (key & pmask) == prefix);
        }
      }
    }
    __syncthreads();
    if (wave == 0) find_bucket(hist, krem, prefix, shift, &s_prefix, &s_krem, &s_count);
    if (tid == 0) s_ncand = 0u;
    __syncthreads();
    // every thread reads the shared results of this pass before any thread can
    // reach the next pass (which clears hist and rewrites them after a barrier)
    prefix = s_prefix;
    krem = s_krem;
    const uint32_t bin_count = s_count;
    pmask |= dmask << shift;
    if (!from_lds && bin_count <= (uint32_t)kKeyCap) {
      // stage the keys of the chosen top-level bin (wave-aggregated append)
      for (int base = 0; base < nf; base += NT * kBatch) {
        float v[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const int i = base + u * NT + tid;
          v[u] = i < nf ? srow[i] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const int i = base + u * NT + tid;
          const uint32_t key = score_key(v[u]);
          const bool mine = i < nf && (key & pmask) == prefix;
          const uint64_t bal = __ballot(mine);
          if (bal) {
            uint32_t wbase = 0;
            if (lane == 0) wbase = atomicAdd(&s_ncand, (uint32_t)__popcll(bal));
            wbase = (uint32_t)__builtin_amdgcn_readfirstlane((int)wbase);
            const uint32_t rank =
                __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
            if (mine) keys_lds[wbase + rank] = key;
          }
        }
      }
      __syncthreads();
      nkeys = (int)s_ncand;
      from_lds = true;
    }
  }
  const uint32_t T = prefix;        // key of the k-th best block
  const uint32_t need_eq = krem;    // blocks equal to T that are kept (lowest indices first)

  // ---- 3. ordered compaction over contiguous per-thread segments [beg, end):
  // one packed scan gives, before this thread, the count of keys > T (high
  // 12 bits) and of keys == T (low 20 bits); the kept keys before it are
  // gt_before + min(eq_before, need_eq).
  const int E = (nf + NT - 1) / NT;
  const int beg = min(tid * E, nf), end = min(beg + E, nf);
  uint32_t gt = 0, eq = 0;
  for (int i0 = beg; i0 < end; i0 += kBatch) {
    uint32_t kk[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int i = i0 + u;
      kk[u] = i < end ? (staged ? keys_lds[i] : score_key(srow[i])) : 0u;
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      gt += (i0 + u < end) && kk[u] > T;
      eq += (i0 + u < end) && kk[u] == T;
    }
  }
  uint32_t tot;
  const uint32_t before = block_exclusive_scan<NT>((gt << 20) | eq, scan_scratch, &tot);
  const uint32_t eq_before = before & 0xFFFFFu;
  uint32_t o = (before >> 20) + min(eq_before, need_eq);
  uint32_t seen = eq_before;
  for (int i0 = beg; i0 < end; i0 += kBatch) {
    uint32_t kk[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int i = i0 + u;
      kk[u] = i < end ? (staged ? keys_lds[i] : score_key(srow[i])) : 0u;
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int i = i0 + u;
      bool take = false;
      if (i < end) {
        take = kk[u] > T;
        if (kk[u] == T) {
          take = seen < need_eq;
          ++seen;
        }
      }
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

template <bool kWritePos>
static void launch_select_t(const Meta& m, const float* scores, int64_t ld, int k, int32_t* sel, int32_t* n_sel,
                            int32_t* pos, int32_t* n_pos, int width, hipStream_t stream) {
  const dim3 grid(m.num_q), block(kSelectThreads);
  if (m.max_blocks <= 16 * kSelectThreads)
    select_reg_kernel<16, kWritePos><<<grid, block, 0, stream>>>(m, scores, ld, k, sel, n_sel, pos, n_pos, width);
  else if (m.max_blocks <= 32 * kSelectThreads)
    select_reg_kernel<32, kWritePos><<<grid, block, 0, stream>>>(m, scores, ld, k, sel, n_sel, pos, n_pos, width);
  else if (m.max_blocks <= 64 * kSelectThreads)
    select_reg_kernel<64, kWritePos><<<grid, block, 0, stream>>>(m, scores, ld, k, sel, n_sel, pos, n_pos, width);
  else
    select_stream_kernel<kWritePos><<<grid, block, 0, stream>>>(m, scores, ld, k, sel, n_sel, pos, n_pos, width);
}

hipError_t launch_select(const Meta& m, const float* scores, int64_t ld, int k, int32_t* sel, int32_t* n_sel,
                         int32_t* pos, int32_t* n_pos, int width, hipStream_t stream) {
  if (pos)
    launch_select_t<true>(m, scores, ld, k, sel, n_sel, pos, n_pos, width, stream);
  else
    launch_select_t<false>(m, scores, ld, k, sel, n_sel, nullptr, nullptr, width, stream);
  return hipGetLastError();
}

hipError_t launch_build_index(const Meta& m, const int32_t* sel, const int32_t* n_sel, int k, int32_t* pos,
                              int32_t* n_pos, int width, hipStream_t stream) {
  build_index_kernel<<<m.num_q, 256, 0, stream>>>(m, sel, n_sel, k, pos, n_pos, width);
  return hipGetLastError();
}

}  // namespace qsa
