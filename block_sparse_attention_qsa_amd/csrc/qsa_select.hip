// a2 - top-k block selection by radix select, and a3 - the position buffer.
//
// The arex-research.com article (section on the four optimisations, item 1)
// keeps at most 512 full blocks per query from an FP32 score buffer with a
// persistent radix selector, and keeps the current partial block without
// selection, which fixes the position buffer at 2,051 entries.  The 10100.com
// article (first optimisation) adds the last step: locate the kept pieces in
// the KV cache.
//
// One selector body (select_row), chosen launches by the longest row of the
// batch:
//   * rows of up to 32,768 blocks: select_reg_kernel, one workgroup per query
//     with the whole row in registers (a linear value grid finds the bin of
//     the k-th best score, its few candidates are ranked exactly; any row the
//     grid cannot split - no finite range, NaN scores, a crowded threshold
//     bin - falls back to exact MSB-first radix passes over order-preserving
//     keys);
//   * longer rows (up to 4M-token contexts): select_slice_kernel keeps the
//     top k of every 8,192- or 16,384-block slice with the same body, then
//     select_cand_kernel keeps the top k of those candidates per query.
// Both keep every block above the threshold and the lowest-index blocks that
// tie with it, and write sel (and, fused, pos) in ascending order.

#include "qsa_common.hpp"
#include "qsa_launch.hpp"

namespace qsa {

constexpr int kCandCap = 256;    // threshold-bin population ranked directly
constexpr int kHotLanes = 8;     // first scores of a wave in the top bin that make it count that bin

// Inside the fully unrolled per-element loops: a scheduling fence every 4
// elements, so the compiler does not compute all E derived values before
// consuming them (with 32 keys per thread in registers that would spill).
__device__ __forceinline__ void sched_fence(int e) {
  if ((e & 3) == 3) __builtin_amdgcn_sched_barrier(0);
}

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
// count still to take inside that bin and the bin's population (and, when
// s_total is given, the histogram's total).  Level one: lane l sums bins
// 2016-32l .. 2047-32l and a wave scan picks the lane; level two: lanes 0..31
// take that lane's 32 bins (highest first) and a second scan picks the bin.
// No loops, no per-bin branches.
__device__ __forceinline__ void find_bucket(const uint32_t* hist, uint32_t krem, uint32_t prefix, int shift,
                                            uint32_t* s_prefix, uint32_t* s_krem, uint32_t* s_count,
                                            uint32_t* s_total = nullptr) {
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
  if (s_total && lane == kWave - 1) *s_total = inc;
  const uint32_t exc = inc - sum;
  const uint64_t hit = __ballot(exc < krem && krem <= inc);
  if (hit == 0) return;                                // krem exceeds the population
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

// Per-thread bit set over the E elements of a segment (bit e = element e).
template <int E>
struct ElemBits {
  static constexpr int W = (E + 31) / 32;
  uint32_t w[W];
  __device__ __forceinline__ void clear() {
#pragma unroll
    for (int i = 0; i < W; ++i) w[i] = 0u;
  }
  // elements pushed from E-1 down to 0 land at their own bit
  __device__ __forceinline__ void push(int e, bool b) { w[e >> 5] = w[e >> 5] + w[e >> 5] + (uint32_t)b; }
  __device__ __forceinline__ void set(int e, bool b) { w[e >> 5] |= (uint32_t)b << (e & 31); }
  __device__ __forceinline__ bool test(int e) const { return (w[e >> 5] >> (e & 31)) & 1u; }
  __device__ __forceinline__ uint32_t count() const {
    uint32_t c = 0;
#pragma unroll
    for (int i = 0; i < W; ++i) c += __popc(w[i]);
    return c;
  }
};

// Grid bin of a score, plus one: trunc(clamp(x * inv + c, 0, 2048)) with
// c = 1.5 - lo * inv, one fused multiply-add.  The fused product, the clamp
// and the truncation are monotone, so a larger score never lands in a lower
// bin; NaN (empty slots) gets 0.  For x >= lo the unclamped value is 1.5 up
// to the rounding of c, so every score of the row lands in [1, 2048] unless
// |c| is near 2^23 (a row whose range is tiny next to its magnitude): a score
// that then gets 0 is missed by the histogram like a NaN, and the row takes
// the exact radix passes instead of the grid.
__device__ __forceinline__ int grid_bin1(float x, float c, float inv) {
  float t = __builtin_fmaf(x, inv, c);
  t = fminf(fmaxf(t, 0.f), 2048.f);
  return (int)t;
}

__device__ __forceinline__ float wave_max_f32(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false)));
  const float a = fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0)),
                        __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16)));
  const float b = fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32)),
                        __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48)));
  return fmaxf(a, b);
}

__device__ __forceinline__ float wave_min_f32(float v) {
  v = fminf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false)));
  v = fminf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false)));
  v = fminf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false)));
  v = fminf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false)));
  const float a = fminf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0)),
                        __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16)));
  const float b = fminf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32)),
                        __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48)));
  return fminf(a, b);
}

// Register-resident selector for rows of at most E * NT blocks, NT threads
// per query.  Thread t owns the contiguous segment [t*E, t*E + E): its
// scores stay in registers from the load to the end.
//   1. One block reduction gives the row's smallest and largest score.  When
//      both are finite and differ, one histogram pass bins the scores on a
//      linear grid of 2,048 bins spanning [min, max] (grid_bin1 is monotone,
//      so the bins partition the row in score order).  On dot-product scores
//      the grid spreads the row evenly, the histogram atomics barely collide
//      and the bin B0 holding the k-th best score is small.
//   2. Each thread classifies its elements once into two bit sets: above B0
//      (kept) and inside B0 (candidates).  Without a finite range (or with a
//      NaN score, found by the histogram missing blocks) every element is a
//      candidate.
//   3. The candidates decide the rest: kept whole when B0 fits; otherwise,
//      when there are at most kCandCap of them (staged in LDS during step 2),
//      each one's exact rank (score descending, index ascending) is counted
//      and the kept ones are marked in an LDS bitmap; if they all tie, the
//      lowest indices are kept; failing both, MSB-first radix passes over 11,
//      11 and 10 key bits find the threshold key.
//   4. One packed block scan of (kept, tie) counts places each thread's kept
//      blocks in index order; tie blocks go to the lowest indices first.  The
//      kept indices are staged in LDS and leave as coalesced rows of sel and
//      pos.
// The per-element work of the common path is a bin, two compares and a
// ballot; only the few candidates take branches.
// What the selector body reads and writes:
//   kRowQuery  query q's score row; writes sel / n_sel (and pos / n_pos);
//   kRowSlice  slice lr.slice (E * NT blocks) of query q's score row; writes
//              the kept blocks' indices and scores, min(k, slice length) of
//              them, to the candidate rows at lr.slice * k;
//   kRowCand   query q's candidate row (every slice's kept blocks, slice by
//              slice, each in ascending index order); writes sel / n_sel (and
//              pos / n_pos) for the kept candidates' block indices.
// A block of the row's top k is in its slice's top k (the order is total),
// and every slice but the last keeps exactly k, so the candidate row is dense
// and in ascending block order: the lower-index-wins rule carries over.
constexpr int kRowQuery = 0, kRowSlice = 1, kRowCand = 2;
struct LongRows {
  float* cscore;     // [num_q][cstride] candidate scores
  int32_t* cidx;     // [num_q][cstride] their block indices
  int cstride;       // candidate row stride: slices * k
  int slice_blocks;  // blocks per slice
  int slice;         // kRowSlice: the slice this workgroup selects from
};

// Slices of 8,192 blocks (8 scores per thread: twice the workgroups, half
// the work each) while the candidate rows stay within 16,384 entries, of
// 16,384 blocks up to the longest rows (at most 64 slices, 32,768 candidates).
inline int long_slice_blocks(int max_blocks) { return max_blocks <= 32 * 8192 ? 8192 : 16384; }

// What a selector writes beside sel / n_sel: nothing, the position rows
// (width 4k + 3, -1 padded) and n_pos, or, for qsa_decode's own attention,
// one slot per 4-slot run (the run's first position: kept blocks, then the
// partial block; rows of k + 1 entries, those past the runs unwritten) and
// n_pos.
constexpr int kPosNone = 0, kPosFull = 1, kPosHeads = 2;

// sel / pos rows for the ns kept block indices in sel_s[] (ascending),
// nf full blocks and a partial block of pl tokens.
template <int NT, int kPosOut>
__device__ __forceinline__ void write_selection(const int32_t* sel_s, int ns, int k, int nf, int pl, const Meta& m,
                                                int r, int kv0, bool paged, int32_t* __restrict__ sel_row,
                                                int32_t* __restrict__ pos_row, int width,
                                                int32_t* __restrict__ n_sel, int32_t* __restrict__ n_pos, int q) {
  const int tid = threadIdx.x;
  // the clamp only guards the position buffer against a broken invariant: a
  // kept index always lies in [0, nf)
  for (int i = tid; i < k; i += NT) sel_row[i] = i < ns ? min(max(sel_s[i], 0), nf - 1) : -1;
  if (kPosOut == kPosFull) {
    const int np = 4 * ns + pl;
    for (int i = tid; i < width; i += NT) {
      int v = -1;
      if (i < 4 * ns) {
        const int b = min(max(sel_s[i >> 2], 0), nf - 1);
        v = (paged ? token_slot(m, r, 4 * b) : kv0 + 4 * b) + (i & 3);
      } else if (i < np) {
        v = (paged ? token_slot(m, r, 4 * nf) : kv0 + 4 * nf) + (i - 4 * ns);
      }
      pos_row[i] = v;
    }
  } else if (kPosOut == kPosHeads) {
    const int nr = ns + (pl > 0 ? 1 : 0);
    for (int i = tid; i < nr; i += NT) {
      const int b = i < ns ? min(max(sel_s[i], 0), nf - 1) : nf;
      pos_row[i] = paged ? token_slot(m, r, 4 * b) : kv0 + 4 * b;
    }
  }
  if (tid == 0) {
    n_sel[q] = ns;
    if (kPosOut != kPosNone) n_pos[q] = 4 * ns + pl;
  }
}

// sel / pos rows when every one of the nf <= k full blocks is kept.
template <int NT, int kPosOut>
__device__ __forceinline__ void write_all_blocks(int nf, int k, int pl, const Meta& m, int r, int kv0, bool paged,
                                                 int32_t* __restrict__ sel_row, int32_t* __restrict__ pos_row,
                                                 int width, int32_t* __restrict__ n_sel, int32_t* __restrict__ n_pos,
                                                 int q) {
  const int tid = threadIdx.x;
  for (int i = tid; i < k; i += NT) sel_row[i] = i < nf ? i : -1;
  if (kPosOut == kPosFull) {
    const int np = 4 * nf + pl;
    for (int i = tid; i < width; i += NT) pos_row[i] = i < np ? (paged ? token_slot(m, r, i) : kv0 + i) : -1;
  } else if (kPosOut == kPosHeads) {
    const int nr = nf + (pl > 0 ? 1 : 0);
    for (int i = tid; i < nr; i += NT) pos_row[i] = paged ? token_slot(m, r, 4 * i) : kv0 + 4 * i;
  }
  if (tid == 0) {
    n_sel[q] = nf;
    if (kPosOut != kPosNone) n_pos[q] = 4 * nf + pl;
  }
}

// Issues the loads of thread t's segment [t*E, t*E + E) of a score row at
// srow.  They go through a buffer descriptor bounded by row_ld floats, so
// reads past it return 0 without a branch and every load of a thread is in
// flight at once (slots past the row's length are discarded by the caller's
// selection).  A wide load never straddles the bound: 16-byte groups are
// taken when the segment width and the row stride are multiples of 4, 8-byte
// pairs (E is even) when the stride is even, single scores otherwise.
template <int E>
__device__ __forceinline__ void load_segment(float (&sv)[E], const float* srow, int64_t row_ld, int64_t rstride) {
  const int beg = threadIdx.x * E;
  const uint32_t row_bytes = (uint32_t)min(max(row_ld, (int64_t)0), (int64_t)(1 << 28)) * 4u;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(srow), 0, (int)row_bytes, 0x00020000);
  if (E % 4 == 0 && (rstride & 3) == 0) {
#pragma unroll
    for (int v = 0; v < E / 4; ++v) {
      const f32x4 x =
          __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (beg + 4 * v) * 4, 0, 0));
      sv[4 * v] = x.x;
      sv[4 * v + 1] = x.y;
      sv[4 * v + 2] = x.z;
      sv[4 * v + 3] = x.w;
    }
  } else if (E % 4 != 0 && (rstride & 1) == 0) {
#pragma unroll
    for (int v = 0; v < E / 2; ++v) {
      const f32x2 x =
          __builtin_bit_cast(f32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, (beg + 2 * v) * 4, 0, 0));
      sv[2 * v] = x.x;
      sv[2 * v + 1] = x.y;
    }
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e)
      sv[e] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, (beg + e) * 4, 0, 0));
  }
}

// The selector core, run by a whole NT-thread workgroup on one row of n
// entries whose segment [t*E, t*E + E) thread t holds in sv (load_segment).
// Keeps the min(k, n) entries ranked first by (score descending, slot
// ascending) and stages their slots, ascending, in sel_s[0 .. ns) (with
// kScores their scores in score_s); returns ns.  Ends with a barrier after
// the staging, so sel_s can be read by any thread.
template <int E, int NT, bool kScores>
__device__ __forceinline__ int select_core(const float (&sv)[E], const int nf, const int k, int32_t* sel_s,
                                           float* score_s) {
  constexpr int NW = NT / kWave;
  constexpr int kMapWords = E * NT / 32;
  static_assert(E % 2 == 0 && E >= 8 && E <= 32, "segment widths");
  // two histograms behind one guard word: the grid pass adds at hist_g[bin + 1]
  // and a NaN score (bin + 1 = 0) in a full wave lands in the guard, unread
  // (the grid total then misses it and the row takes the radix passes)
  __shared__ uint32_t hist_g[1 + 2 * kRadixBins];
  uint32_t* const hist0 = hist_g + 1;
  __shared__ uint32_t keepmap[kMapWords];   // kept candidates, bit per slot
  __shared__ float red_s[2 * NW];           // per-wave score range of the row
  __shared__ uint32_t red2_s[2 * NW];       // per-wave key range of the candidates
  __shared__ uint32_t scan_s[NW];
  __shared__ u32x2 cand_s[kCandCap];
  __shared__ uint32_t s_prefix, s_krem, s_count, s_total, s_ncand;

  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  const int beg = tid * E;

  // LDS set-up overlaps the loads still in flight
  for (int i = tid; i < kRadixBins; i += NT) hist0[i] = 0u;
  for (int i = tid; i < kMapWords; i += NT) keepmap[i] = 0u;
  if (tid == 0) s_ncand = 0u;

  const int cnt = max(0, min(E, nf - beg));
  if (nf <= k) {
    // every entry is kept
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (e < cnt) {
        sel_s[beg + e] = beg + e;
        if (kScores) score_s[beg + e] = sv[e];
      }
    __syncthreads();
    return max(nf, 0);
  }
  const bool wave_full = __ballot(cnt != E) == 0;    // every lane holds E entries
  const bool wave_empty = __ballot(cnt != 0) == 0;   // no lane holds an entry

  // Slots past the row become NaN: the range reduction skips them and their
  // grid bin is -1.
  float xr[E];
#pragma unroll
  for (int e = 0; e < E; ++e) xr[e] = e < cnt ? sv[e] : __builtin_nanf("");
// score e of this thread's segment (e is a compile-time constant in the unrolled loops)
#define QSA_X(e) xr[e]

  // ---- 1. score range of the row (NaN skipped)
  float vmax = -__builtin_inff(), vmin = __builtin_inff();
  if (!wave_empty) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      vmax = fmaxf(vmax, QSA_X(e));
      vmin = fminf(vmin, QSA_X(e));
    }
  }
  vmax = wave_max_f32(vmax);
  vmin = wave_min_f32(vmin);
  if (lane == 0) {
    red_s[wave] = vmax;
    red_s[NW + wave] = vmin;
  }
  __syncthreads();
  const float hi = wave_max_f32(lane < NW ? red_s[lane] : -__builtin_inff());
  const float lo = wave_min_f32(lane < NW ? red_s[NW + lane] : __builtin_inff());
  const float span = hi - lo;
  const float inv = (float)kRadixBins / span;
  const float cgrid = 1.5f - lo * inv;
  bool grid = __builtin_isfinite(lo) && __builtin_isfinite(hi) && span > 0.f && __builtin_isfinite(inv) && inv > 0.f &&
              __builtin_isfinite(cgrid);

  // ---- 2. grid histogram, then classification
  int B0 = 0, h = 0;
  uint32_t krem = (uint32_t)k, c0 = (uint32_t)nf;
  // Each element's grid bin from the histogram pass is kept (bin + 1, 0 for
  // none; two per word), so classifying needs no second bin computation.
  uint32_t bins[E / 2];
  if (grid) {
    const float c0f = fresh_uniform(cgrid), inv0 = fresh_uniform(inv);
    // A wave whose first scores land in the grid's top bin several times
    // (the row's maximum and those within a bin width of it: a row with many
    // blocks tied at the top) counts that bin per thread and adds it once,
    // instead of one LDS atomic per score serialised on one word.  Other
    // waves pay one ballot for the test.
    uint32_t ntop = 0u;
    const bool hot = !wave_empty && __popcll(__ballot(grid_bin1(QSA_X(0), c0f, inv0) == kRadixBins)) >= kHotLanes;
// the histogram pass of one wave: HOT counts the top bin, FULL skips the test
// for empty slots (bin 0)
#define QSA_HIST_PASS(HOT, FULL)                                 \
  _Pragma("unroll") for (int e = 0; e < E; ++e) {               \
    const int b1 = grid_bin1(QSA_X(e), c0f, inv0);              \
    const bool top = (HOT) && b1 == kRadixBins;                 \
    if (HOT) ntop += top ? 1u : 0u;                             \
    if (((FULL) || b1 > 0) && !top) atomicAdd(&hist_g[b1], 1u); \
    if (e & 1) bins[e >> 1] |= (uint32_t)b1 << 16;              \
    else bins[e >> 1] = (uint32_t)b1;                           \
    sched_fence(e);                                             \
  }
    if (wave_full) {
      if (hot) {
        QSA_HIST_PASS(true, true)
      } else {
        QSA_HIST_PASS(false, true)
      }
    } else if (!wave_empty) {
      if (hot) {
        QSA_HIST_PASS(true, false)
      } else {
        QSA_HIST_PASS(false, false)
      }
    }
#undef QSA_HIST_PASS
    if (hot) {
      const uint32_t wtop = (uint32_t)__builtin_amdgcn_readlane((int)wave_inclusive_scan(ntop), kWave - 1);
      if (lane == 0) atomicAdd(&hist_g[kRadixBins], wtop);
    }
    for (int i = tid; i < kRadixBins; i += NT) hist0[kRadixBins + i] = 0u;
    __syncthreads();
    if (wave == 0) find_bucket(hist0, krem, 0u, 0, &s_prefix, &s_krem, &s_count, &s_total);
    __syncthreads();
    h = 1;
    if (fresh_uniform(s_total) == (uint32_t)nf) {
      B0 = fresh_uniform((int)s_prefix);
      krem = fresh_uniform(s_krem);
      c0 = fresh_uniform(s_count);
    } else {
      grid = false;   // a NaN score missed the histogram: no grid
    }
  }
  const bool ranked = grid && krem != c0 && c0 <= (uint32_t)kCandCap;
  ElemBits<E> above, inb;
  above.clear();
  inb.clear();
  if (grid) {
    if (!wave_empty) {
      const uint32_t b1 = (uint32_t)B0 + 1u;
#pragma unroll
      for (int e = E - 1; e >= 0; --e) {
        const uint32_t b = (bins[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
        above.push(e, b > b1);
        inb.push(e, b == b1);
      }
      if (ranked) {
        // Stage this thread's candidates (few in a row, so most waves skip
        // this): one LDS append per thread that has any.
        const uint32_t mine = inb.count();
        if (__ballot(mine != 0u)) {
          uint32_t slot = mine != 0u ? atomicAdd(&s_ncand, mine) : 0u;
#pragma unroll
          for (int e = 0; e < E; ++e) {
            if (inb.test(e)) {
              if (slot < (uint32_t)kCandCap) cand_s[slot] = u32x2{score_key(QSA_X(e)), (uint32_t)(beg + e)};
              ++slot;
            }
          }
        }
      }
    }
  } else {
#pragma unroll
    for (int e = E - 1; e >= 0; --e) inb.push(e, e < cnt);   // every entry is a candidate
  }

  // ---- 3. resolve the candidates
  ElemBits<E> keep = above, ties;
  ties.clear();
  uint32_t need = 0u;
  if (grid && krem == c0) {
#pragma unroll
    for (int i = 0; i < ElemBits<E>::W; ++i) keep.w[i] |= inb.w[i];   // B0 kept whole
  } else if (ranked) {
    __syncthreads();
    if (tid < (int)c0) {
      const u32x2 me = cand_s[tid];
      uint32_t ahead = 0u;
      for (int j = 0; j < (int)c0; ++j) {
        const u32x2 o = cand_s[j];
        ahead += (o.x > me.x) | ((o.x == me.x) & (o.y < me.y));
      }
      if (ahead < krem) atomicOr(&keepmap[me.y >> 5], 1u << (me.y & 31));
    }
    __syncthreads();
    {
      // this thread's E bits start at bit tid*E and may run into the next word
      const int bit0 = tid * E, sh = bit0 & 31;
      uint32_t word = keepmap[bit0 >> 5] >> sh;
      if (sh + E > 32) word |= keepmap[(bit0 >> 5) + 1] << (32 - sh);
      keep.w[0] |= E == 32 ? word : (word & ((1u << (E & 31)) - 1u));
    }
  } else {
    // many candidates (or no grid): done at once if they all tie
    uint32_t bmax = 0u, bmin = 0xFFFFFFFFu;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if (inb.test(e)) {
        const uint32_t key = score_key(QSA_X(e));
        bmax = max(bmax, key);
        bmin = min(bmin, key);
      }
    }
    bmax = wave_max_u32(bmax);
    bmin = wave_min_u32(bmin);
    if (lane == 0) {
      red2_s[wave] = bmax;
      red2_s[NW + wave] = bmin;
    }
    __syncthreads();
    bmax = lds_slots_max(red2_s, NW);
    bmin = lds_slots_min(red2_s + NW, NW);
    if (bmax == bmin) {
      ties = inb;         // all tie: the lowest slots are kept
      need = krem;
    } else {
      // MSB-first radix passes (11, 11, 10 key bits) over the candidates;
      // stop once the threshold bin is taken whole
      uint32_t prefix = 0u, pmask = 0u;
#pragma unroll 1
      for (int pass = 0; pass < 3; ++pass) {
        const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
        const uint32_t dmask = pass == 2 ? 0x3FFu : 0x7FFu;
        uint32_t* cur = hist0 + h * kRadixBins;
        uint32_t* nxt = hist0 + (h ^ 1) * kRadixBins;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const uint32_t key = score_key(QSA_X(e));
          hist_add(cur, (key >> shift) & dmask, inb.test(e) && (key & pmask) == prefix);
          sched_fence(e);
        }
        for (int i = tid; i < kRadixBins; i += NT) nxt[i] = 0u;   // last read before the previous barrier
        __syncthreads();
        if (wave == 0) find_bucket(cur, krem, prefix, shift, &s_prefix, &s_krem, &s_count);
        __syncthreads();
        prefix = s_prefix;
        krem = s_krem;
        const uint32_t bin_count = s_count;
        pmask |= dmask << shift;
        h ^= 1;
        if (krem == bin_count) break;
      }
      // split the candidates around the threshold (key & pmask) == prefix
      const uint32_t T = fresh_uniform(prefix), M = fresh_uniform(pmask);
      need = krem;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        if (inb.test(e)) {
          const uint32_t km = score_key(QSA_X(e)) & M;
          keep.set(e, km > T);
          ties.set(e, km == T);
        }
      }
    }
  }

  // ---- 4. ordered compaction: one packed scan, kept count in the high 12
  // bits and tie count in the low 20
  need = fresh_uniform(need);
  const uint32_t nkeep = keep.count(), ntie = ties.count();
  uint32_t tot;
  const uint32_t before = block_exclusive_scan<NT>((nkeep << 20) | ntie, scan_s, &tot);
  const uint32_t tie_before = before & 0xFFFFFu;
  // ties kept by earlier threads, and by this one (need - kept never wraps)
  const uint32_t kept = min(tie_before, need);
  uint32_t take = min(need - kept, ntie);
#pragma unroll
  for (int i = 0; i < ElemBits<E>::W; ++i) {
    uint32_t t = ties.w[i];
    while (take != 0u && t != 0u) {
      const uint32_t low = t & (0u - t);
      keep.w[i] |= low;
      t ^= low;
      --take;
    }
  }
  uint32_t o = (before >> 20) + kept;
#pragma unroll
  for (int i = 0; i < ElemBits<E>::W; ++i) {
    uint32_t t = keep.w[i];
    while (t != 0u) {
      const int e = 32 * i + __builtin_ctz(t);
      t &= t - 1u;
      if (o < (uint32_t)k) {
        sel_s[o] = beg + e;
        if (kScores) score_s[o] = QSA_X(e);
      }
      ++o;
    }
  }
  const int ns = (int)min((tot >> 20) + min(tot & 0xFFFFFu, need), (uint32_t)k);
  __syncthreads();
  return ns;
}
#undef QSA_X

// The selector body for query q, run by a whole NT-thread workgroup: loads
// its row (see below), handles the rows that need no selection and runs
// select_core on the rest.
template <int E, int NT, int kPosOut, int kRow = kRowQuery>
__device__ __forceinline__ void select_row(const Meta& m, const float* __restrict__ scores, int64_t ld, int k,
                                           int32_t* __restrict__ sel, int32_t* __restrict__ n_sel,
                                           int32_t* __restrict__ pos, int32_t* __restrict__ n_pos, int width,
                                           const int q, const LongRows& lr) {
  __shared__ int32_t sel_s[QSA_TOPK];
  __shared__ float score_s[kRow == kRowSlice ? QSA_TOPK : 1];   // a slice's kept scores
  const int tid = threadIdx.x;
  constexpr int S = E * NT;
  const float* srow = kRow == kRowCand ? lr.cscore + (int64_t)q * lr.cstride
                                       : scores + (int64_t)q * ld + (kRow == kRowSlice ? (int64_t)lr.slice * S : 0);
  const int64_t row_ld = kRow == kRowCand ? (int64_t)lr.cstride
                                          : (kRow == kRowSlice ? ld - (int64_t)lr.slice * S : ld);
  const int64_t rstride = kRow == kRowCand ? (int64_t)lr.cstride : ld;

  // Score loads are issued first, speculatively: thread t owns the fixed
  // segment [t*E, t*E + E), so the loads do not wait for the request metadata.
  float sv[E];
  load_segment<E>(sv, srow, row_ld, rstride);

  const int r = request_of(m.q_start, m.num_req, q);
  const int qs = m.q_start[r];
  const int nq = m.q_start[r + 1] - qs;
  const int L = m.seq_len[r] - nq + 1 + (q - qs);
  int nfq = L >> 2;                                  // the query's full blocks
  if (tid == 0 && kRow != kRowSlice) {
    QSA_DCHECK(m.err, nq >= 1 && nq <= QSA_MAX_Q_PER_REQ && m.seq_len[r] >= nq, QSA_ERROR_BAD_QUERIES);
    QSA_DCHECK(m.err, nfq <= m.max_blocks, QSA_ERROR_BAD_BLOCKS);
  }
  if (nfq > m.max_blocks) nfq = m.max_blocks;
  int nf;                                            // entries of the row selected from here
  if (kRow == kRowQuery) {
    nf = min(nfq, S);                                // launcher picks E * NT >= max_blocks
    nfq = nf;
  } else if (kRow == kRowSlice) {
    nf = max(0, min(S, nfq - lr.slice * S));
  } else {
    const int SB = lr.slice_blocks;
    const int P = (nfq + SB - 1) / SB;
    nf = P <= 1 ? min(k, nfq) : (P - 1) * k + min(k, nfq - (P - 1) * SB);
    nf = min(nf, S);
  }
  const int pl = L & 3;
  const bool paged = m.page_table != nullptr;
  const int kv0 = paged ? 0 : m.kv_start[r];
  int32_t* sel_row = kRow == kRowSlice ? nullptr : sel + (int64_t)q * k;
  int32_t* pos_row = kPosOut != kPosNone ? pos + (int64_t)q * width : nullptr;
  const int32_t* cidx_row = kRow == kRowCand ? lr.cidx + (int64_t)q * lr.cstride : nullptr;
  float* cs_out = kRow == kRowSlice ? lr.cscore + (int64_t)q * lr.cstride + (int64_t)lr.slice * k : nullptr;
  int32_t* ci_out = kRow == kRowSlice ? lr.cidx + (int64_t)q * lr.cstride + (int64_t)lr.slice * k : nullptr;
  const int beg = tid * E;

  if (kRow == kRowSlice && nf <= k) {                // the whole slice is kept
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (beg + e < nf) {
        cs_out[beg + e] = sv[e];
        ci_out[beg + e] = lr.slice * S + beg + e;
      }
    return;
  }
  if (kRow == kRowCand && nf <= k) {                 // every candidate is kept
    for (int i = tid; i < nf; i += NT) sel_s[i] = cidx_row[i];
    __syncthreads();
    write_selection<NT, kPosOut>(sel_s, nf, k, nfq, pl, m, r, kv0, paged, sel_row, pos_row, width, n_sel, n_pos,
                                   q);
    return;
  }
  if (nf <= k) {
    write_all_blocks<NT, kPosOut>(nf, k, pl, m, r, kv0, paged, sel_row, pos_row, width, n_sel, n_pos, q);
    return;
  }

  const int ns = select_core<E, NT, kRow == kRowSlice>(sv, nf, k, sel_s, score_s);
  if (kRow == kRowSlice) {
    for (int i = tid; i < ns; i += NT) {
      cs_out[i] = score_s[i];
      ci_out[i] = lr.slice * S + sel_s[i];
    }
    return;
  }
  if (kRow == kRowCand) {
    for (int i = tid; i < ns; i += NT) sel_s[i] = cidx_row[sel_s[i]];   // candidate -> block index
    __syncthreads();
  }
  write_selection<NT, kPosOut>(sel_s, ns, k, nfq, pl, m, r, kv0, paged, sel_row, pos_row, width, n_sel, n_pos, q);
}

// The attention's work list for a ragged batch (AttnPlan), built by one
// NT-thread workgroup (NT > num_q): an extra workgroup of the selection
// launch inside qsa_decode, or a launch of its own before the stage
// attention.  Query q has n positions - 4 min(nf, k) + L mod 4 from the
// metadata (what the selection in the same launch writes as n_pos), or the
// given counts - and nch = ceil(n / 32) chunks; the chunks per split cps spread the
// batch's chunks over kAttnTargetWgs workgroups in whole 4-chunk steps.  Each
// (query, KV head) unit gets nch / cps full splits and, when the division
// leaves a rest, one shorter split; full splits come first in the list, the
// shorter ones after them by decreasing size (a counting sort; ties in any
// order - each item's arithmetic, and the order of its unit's merge, do not
// depend on where it sits in the list).
template <int NT>
__device__ __forceinline__ void build_attn_plan(const Meta& m, const AttnPlan& pl) {
  __shared__ uint32_t scan_s[NT / kWave];
  __shared__ uint32_t hist_s[kMaxSplitChunks + 1], base_s[kMaxSplitChunks + 1];
  const int tid = threadIdx.x;
  const int H = pl.num_kv_heads;
  for (int i = tid; i <= kMaxSplitChunks; i += NT) hist_s[i] = 0u;
  int nch = 0;
  if (tid < m.num_q) {
    int n;
    if (pl.n_pos != nullptr) {
      n = min(max(pl.n_pos[tid], 0), pl.pos_cap);
    } else {
      const int r = request_of(m.q_start, m.num_req, tid);
      const int qs = m.q_start[r];
      const int nq = m.q_start[r + 1] - qs;
      const int L = max(m.seq_len[r] - nq + 1 + (tid - qs), 0);
      const int nf = min(L >> 2, m.max_blocks);
      n = 4 * min(nf, pl.k) + (L & 3);
    }
    nch = (n + kChunk - 1) / kChunk;
  }
  uint32_t tot;
  block_exclusive_scan<NT>((uint32_t)nch, scan_s, &tot);
  __syncthreads();                        // scan_s is read by every wave before it is reused
  int cps = (int)(((uint64_t)tot * (uint32_t)H + kAttnTargetWgs - 1) / kAttnTargetWgs);
  cps = (cps + kAttnWaves - 1) / kAttnWaves * kAttnWaves;
  cps = min(max(cps, pl.cps_min), kMaxSplitChunks);
  const int f = tid < m.num_q ? nch / cps : 0;
  const int rest = tid < m.num_q ? nch - f * cps : 0;
  const bool part = tid < m.num_q && (rest > 0 || nch == 0);   // a unit without positions still gets one item
  const int S = f + (part ? 1 : 0);
  uint32_t nfull;
  const uint32_t fbefore = block_exclusive_scan<NT>((uint32_t)f, scan_s, &nfull);
  if (part) atomicAdd(&hist_s[rest], 1u);
  __syncthreads();
  if (tid < kWave) {
    // running totals of the rests, longest first: lane l takes the sizes
    // kMaxSplitChunks - 2l and - 2l - 1
    static_assert(2 * kWave > kMaxSplitChunks, "two sizes per lane");
    const int i0 = 2 * tid, i1 = 2 * tid + 1;
    const uint32_t h0 = i0 <= kMaxSplitChunks ? hist_s[kMaxSplitChunks - i0] : 0u;
    const uint32_t h1 = i1 <= kMaxSplitChunks ? hist_s[kMaxSplitChunks - i1] : 0u;
    const uint32_t inc = wave_inclusive_scan(h0 + h1);
    const uint32_t before = inc - h0 - h1;
    if (i0 <= kMaxSplitChunks) base_s[kMaxSplitChunks - i0] = before;
    if (i1 <= kMaxSplitChunks) base_s[kMaxSplitChunks - i1] = before + h0;
    if (tid == kWave - 1) {
      pl.words[0] = (int32_t)((nfull + inc) * (uint32_t)H);
      pl.words[1] = cps;
    }
  }
  __syncthreads();
  uint32_t* items = reinterpret_cast<uint32_t*>(pl.words + kPlanHeader);
  if (tid < m.num_q) {
    for (int s = 0; s < f; ++s)
      for (int g = 0; g < H; ++g) items[(fbefore + s) * H + g] = plan_item(tid, g, s, S);
    if (part) {
      const uint32_t slot = nfull + atomicAdd(&base_s[rest], 1u);   // base_s now serves as the cursor
      for (int g = 0; g < H; ++g) items[slot * H + g] = plan_item(tid, g, f, S);
    }
  }
}

// The work list alone (the stage attention on a ragged batch).
__global__ __launch_bounds__(512) void attn_plan_kernel(Meta m, AttnPlan plan) { build_attn_plan<512>(m, plan); }

template <int E, int NT, int kPosOut, bool kPlan = false>
__global__ __launch_bounds__(NT) void select_reg_kernel(Meta m, const float* __restrict__ scores, int64_t ld,
                                                        int k, int32_t* __restrict__ sel,
                                                        int32_t* __restrict__ n_sel, int32_t* __restrict__ pos,
                                                        int32_t* __restrict__ n_pos, int width, AttnPlan plan) {
  if (kPlan && (int)blockIdx.x == m.num_q) {   // the extra workgroup: the attention's work list
    build_attn_plan<NT>(m, plan);
    return;
  }
  select_row<E, NT, kPosOut>(m, scores, ld, k, sel, n_sel, pos, n_pos, width, (int)blockIdx.x, LongRows{});
}

// Long rows, launch 1: grid (query, slice); each workgroup keeps the top k
// of one E * 1,024-block slice of its query's row.
template <int E>
__global__ __launch_bounds__(kSelectThreads) void select_slice_kernel(Meta m, const float* __restrict__ scores,
                                                                      int64_t ld, int k, LongRows lr) {
  lr.slice = (int)blockIdx.y;
  select_row<E, kSelectThreads, kPosNone, kRowSlice>(m, scores, ld, k, nullptr, nullptr, nullptr, nullptr, 0,
                                                  (int)blockIdx.x, lr);
}

// Long rows, launch 2: one NT-thread workgroup per query keeps the top k of
// the query's candidate row and writes sel (and pos).
template <int E, int NT, int kPosOut, bool kPlan = false>
__global__ __launch_bounds__(NT) void select_cand_kernel(Meta m, int k, int32_t* __restrict__ sel,
                                                         int32_t* __restrict__ n_sel, int32_t* __restrict__ pos,
                                                         int32_t* __restrict__ n_pos, int width, LongRows lr,
                                                         AttnPlan plan) {
  if (kPlan && (int)blockIdx.x == m.num_q) {   // the extra workgroup: the attention's work list
    build_attn_plan<NT>(m, plan);
    return;
  }
  select_row<E, NT, kPosOut, kRowCand>(m, nullptr, 0, k, sel, n_sel, pos, n_pos, width, (int)blockIdx.x, lr);
}

// Position buffer from a selection: of the first min(n_sel, k) entries of
// the (ascending) selection row, those below nf are used; later ones are not
// full blocks of this query and are dropped, so that a selection made for a
// longer query can be reused.
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
  const bool paged = m.page_table != nullptr;
  const int kv0 = paged ? 0 : m.kv_start[r];
  int given = n_sel[q];
  QSA_DCHECK(m.err, given >= 0 && given <= k, QSA_ERROR_BAD_SELECTION);
  given = given < 0 ? 0 : (given > k ? k : given);
  const int32_t* srow = sel + (int64_t)q * k;
#ifdef QSA_DEBUG_CHECKS
  for (int i = threadIdx.x; i + 1 < given; i += blockDim.x)
    QSA_DCHECK(m.err, srow[i] < srow[i + 1], QSA_ERROR_BAD_SELECTION);
  if (threadIdx.x == 0)
    QSA_DCHECK(m.err, nq >= 1 && nq <= QSA_MAX_Q_PER_REQ && m.seq_len[r] >= nq, QSA_ERROR_BAD_QUERIES);
#endif
  // 256 threads, k <= 512: entries tid and tid + 256 per thread
  const int i0 = threadIdx.x, i1 = threadIdx.x + 256;
  const bool ok0 = i0 < given && srow[i0] >= 0 && srow[i0] < nf;
  const bool ok1 = i1 < given && srow[i1] >= 0 && srow[i1] < nf;
  const int ns = __syncthreads_count(ok0) + __syncthreads_count(ok1);
  const int np = 4 * ns + pl;
  int32_t* prow = pos + (int64_t)q * width;
  for (int i = threadIdx.x; i < width; i += blockDim.x) {
    int v = -1;
    if (i < 4 * ns) {
      const int b = srow[i >> 2];
      v = (paged ? token_slot(m, r, 4 * b) : kv0 + 4 * b) + (i & 3);
    } else if (i < np) {
      v = (paged ? token_slot(m, r, 4 * nf) : kv0 + 4 * nf) + (i - 4 * ns);
    }
    prow[i] = v;
  }
  if (threadIdx.x == 0) n_pos[q] = np;
}

template <int kPosOut>
static void launch_select_t(const Meta& m, const float* scores, int64_t ld, int k, int32_t* sel, int32_t* n_sel,
                            int32_t* pos, int32_t* n_pos, int width, uint32_t* ms_ws, const AttnPlan& plan,
                            hipStream_t stream) {
  // one more workgroup than queries builds the attention's work list
  const unsigned nwg = (unsigned)m.num_q + (plan.words != nullptr ? 1u : 0u);
  // Rows up to 16,384 blocks: the narrowest even segment that covers the
  // longest row (at least 8 scores per thread), so that the busiest SIMD of
  // the workgroup runs as few score slots as the row needs.
  if (m.max_blocks <= 16384) {
    const int e = max(8, ((m.max_blocks + kSelectThreads - 1) / kSelectThreads + 1) & ~1);
    const dim3 g(nwg);
#define QSA_SELECT_REG(EW)                                                                                    \
  do {                                                                                                         \
    if (plan.words)                                                                                            \
      select_reg_kernel<EW, kSelectThreads, kPosOut, true>                                                    \
          <<<g, kSelectThreads, 0, stream>>>(m, scores, ld, k, sel, n_sel, pos, n_pos, width, plan);          \
    else                                                                                                       \
      select_reg_kernel<EW, kSelectThreads, kPosOut>                                                          \
          <<<g, kSelectThreads, 0, stream>>>(m, scores, ld, k, sel, n_sel, pos, n_pos, width, plan);          \
  } while (0)
    if (e <= 8) QSA_SELECT_REG(8);
    else if (e <= 10) QSA_SELECT_REG(10);
    else if (e <= 12) QSA_SELECT_REG(12);
    else if (e <= 14) QSA_SELECT_REG(14);
    else QSA_SELECT_REG(16);
#undef QSA_SELECT_REG
    return;
  }
  if (m.max_blocks <= kLongRowBlocks) {
    if (plan.words)
      select_reg_kernel<kLongRowBlocks / kSelectThreads, kSelectThreads, kPosOut, true>
          <<<nwg, kSelectThreads, 0, stream>>>(m, scores, ld, k, sel, n_sel, pos, n_pos, width, plan);
    else
      select_reg_kernel<kLongRowBlocks / kSelectThreads, kSelectThreads, kPosOut>
          <<<nwg, kSelectThreads, 0, stream>>>(m, scores, ld, k, sel, n_sel, pos, n_pos, width, plan);
    return;
  }
  // Longer rows: every slice keeps its top k, then one workgroup per query
  // selects among the slices' candidates.
  const int SB = long_slice_blocks(m.max_blocks);
  const int P = (m.max_blocks + SB - 1) / SB;
  LongRows lr;
  lr.cstride = P * k;
  lr.cscore = reinterpret_cast<float*>(ms_ws);
  lr.cidx = reinterpret_cast<int32_t*>(ms_ws) + (int64_t)m.num_q * lr.cstride;
  lr.slice_blocks = SB;
  lr.slice = 0;
  const dim3 sgrid((unsigned)m.num_q, (unsigned)P);
  if (SB == 8192) select_slice_kernel<8><<<sgrid, kSelectThreads, 0, stream>>>(m, scores, ld, k, lr);
  else select_slice_kernel<16><<<sgrid, kSelectThreads, 0, stream>>>(m, scores, ld, k, lr);
  // the candidate step: 8 candidates per thread while they fit, on 512
  // threads for the few candidates of up to 8 slices
#define QSA_SELECT_CAND(EW, NTW)                                                                        \
  do {                                                                                                 \
    if (plan.words)                                                                                    \
      select_cand_kernel<EW, NTW, kPosOut, true><<<nwg, NTW, 0, stream>>>(m, k, sel, n_sel, pos, n_pos, width, \
                                                                          lr, plan);                   \
    else                                                                                               \
      select_cand_kernel<EW, NTW, kPosOut><<<nwg, NTW, 0, stream>>>(m, k, sel, n_sel, pos, n_pos, width, lr, \
                                                                    plan);                             \
  } while (0)
  if (lr.cstride <= 8 * 512) QSA_SELECT_CAND(8, 512);
  else if (lr.cstride <= 8 * kSelectThreads) QSA_SELECT_CAND(8, kSelectThreads);
  else if (lr.cstride <= 16 * kSelectThreads) QSA_SELECT_CAND(16, kSelectThreads);
  else QSA_SELECT_CAND(32, kSelectThreads);
#undef QSA_SELECT_CAND
}

size_t select_workspace_bytes(int num_q, int max_blocks) {
  if (max_blocks <= kLongRowBlocks) return 0;
  // candidate scores and block indices: slices * k of each per query (k <= 512)
  const int64_t slices = (max_blocks + long_slice_blocks(max_blocks) - 1) / long_slice_blocks(max_blocks);
  return (size_t)num_q * (size_t)(slices * QSA_TOPK) * 2 * sizeof(uint32_t);
}

hipError_t launch_select(const Meta& m, const float* scores, int64_t ld, int k, int32_t* sel, int32_t* n_sel,
                         int32_t* pos, int32_t* n_pos, int width, bool run_heads, void* ws, const AttnPlan& plan,
                         hipStream_t stream) {
  uint32_t* ms_ws = static_cast<uint32_t*>(ws);
  if (pos && run_heads)
    launch_select_t<kPosHeads>(m, scores, ld, k, sel, n_sel, pos, n_pos, width, ms_ws, plan, stream);
  else if (pos)
    launch_select_t<kPosFull>(m, scores, ld, k, sel, n_sel, pos, n_pos, width, ms_ws, plan, stream);
  else
    launch_select_t<kPosNone>(m, scores, ld, k, sel, n_sel, nullptr, nullptr, width, ms_ws, plan, stream);
  return hipGetLastError();
}

hipError_t launch_attn_plan(const Meta& m, const AttnPlan& plan, hipStream_t stream) {
  attn_plan_kernel<<<1, 512, 0, stream>>>(m, plan);
  return hipGetLastError();
}

hipError_t launch_build_index(const Meta& m, const int32_t* sel, const int32_t* n_sel, int k, int32_t* pos,
                              int32_t* n_pos, int width, hipStream_t stream) {
  build_index_kernel<<<m.num_q, 256, 0, stream>>>(m, sel, n_sel, k, pos, n_pos, width);
  return hipGetLastError();
}

}  // namespace qsa
