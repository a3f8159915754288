// Device-side helpers shared by the QSA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qsa.h"

namespace qsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kChunk = 32;             // positions per attention step of one wave
constexpr int kAttnWaves = 4;          // waves per attention workgroup
constexpr int kSelectThreads = 1024;   // threads of one top-k workgroup
constexpr int kRadixBins = 2048;       // 11-bit digits: passes over bits 31..21, 20..10, 9..0
constexpr int kMaxSplits = (QSA_WIDTH + kChunk * kAttnWaves - 1) / (kChunk * kAttnWaves);  // 17
constexpr int kCounterStride = 32;     // uint32 words per arrival counter (one 128-byte line)
// Attention splits a (query, KV head) unit over several workgroups only while
// the units number fewer than this many workgroups, so at most
// kAttnTargetWgs - 1 split-arrival counters are ever in use and their
// indices (query * Hkv + KV head) stay below kAttnTargetWgs.
constexpr int kAttnTargetWgs = 512;
// Every workspace starts with a control region of fixed size that holds all
// counters any call can use: the attention's split-arrival counters (one
// 128-byte line per unit index) and as many lines again for the selector's
// per-query hand-offs.  Its placement and size do not depend on the batch, so
// one zero-filled workspace serves calls of any geometry: other calls' score
// rows, partials or candidates never overlap a counter.
constexpr size_t kCtlAttnBytes = (size_t)kAttnTargetWgs * kCounterStride * 4;   // 64 KiB
constexpr size_t kCtlBytes = 2 * kCtlAttnBytes;
// Cache-policy bit SC1 of a buffer load/store: device scope.  Such accesses
// bypass the per-XCD caches, so workgroups on different XCDs see each
// other's data without any cache flush or invalidation.
constexpr int kCpolDevice = 16;

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// Index of the request that owns query q: the largest r with q_start[r] <= q.
__device__ __forceinline__ int request_of(const int32_t* __restrict__ q_start, int num_req, int q) {
  int lo = 0, hi = num_req - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (q_start[mid] <= q) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Order-preserving map FP32 -> uint32 (larger float -> larger key).  Adding
// +0.0 turns -0.0 into +0.0 so that the two compare equal; NaN keeps its sign
// and sorts beyond the infinities.
__device__ __forceinline__ uint32_t score_key(float s) {
  const uint32_t u = __float_as_uint(s + 0.0f);
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

// Inverse of score_key (-0.0 comes back as +0.0; key 0 comes back as NaN).
__device__ __forceinline__ float key_value(uint32_t key) {
  const uint32_t flip = (uint32_t)((int32_t)~key >> 31) | 0x80000000u;
  return __uint_as_float(key ^ flip);
}

// DPP sum over the 16 lanes of a row; every lane of the row gets the total.
__device__ __forceinline__ float row16_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));
  return v;
}

// A copy of a wave-uniform value that the compiler cannot prove equal to the
// original: values derived from it are recomputed instead of being kept live
// across phases (which would cost a register per element).
template <class T>
__device__ __forceinline__ T fresh_uniform(T x) {
  static_assert(sizeof(T) == 4, "32-bit values only");
  int v = __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x));
  asm volatile("" : "+s"(v));
  return __builtin_bit_cast(T, v);
}


// Wave-wide maximum / minimum (all 64 lanes active); the result is uniform.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));
  const uint32_t a = max((uint32_t)__builtin_amdgcn_readlane((int)v, 0), (uint32_t)__builtin_amdgcn_readlane((int)v, 16));
  const uint32_t b = max((uint32_t)__builtin_amdgcn_readlane((int)v, 32), (uint32_t)__builtin_amdgcn_readlane((int)v, 48));
  return max(a, b);
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));
  const uint32_t a = min((uint32_t)__builtin_amdgcn_readlane((int)v, 0), (uint32_t)__builtin_amdgcn_readlane((int)v, 16));
  const uint32_t b = min((uint32_t)__builtin_amdgcn_readlane((int)v, 32), (uint32_t)__builtin_amdgcn_readlane((int)v, 48));
  return min(a, b);
}

// Wave-wide inclusive prefix sum of unsigned values: a DPP shift-scan inside
// each 16-lane row (lanes shifted in from outside the row read 0), then the
// row totals are added through lane reads.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, true);   // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, true);   // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, true);   // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, true);   // row_shr:8
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 15);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 31);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 47);
  const int row = lane_id() >> 4;
  return v + (row > 0 ? r0 : 0u) + (row > 1 ? r1 : 0u) + (row > 2 ? r2 : 0u);
}

// Block-wide exclusive prefix sum for blockDim.x == NT (multiple of 64,
// at most 4096).  `scratch` needs NT/64 words of LDS.  Returns this thread's
// exclusive prefix and the block total.  One barrier inside; the caller must
// separate two calls that share `scratch` by a barrier.  The wave totals are
// combined by a second wave scan over lanes 0..NT/64-1 (no per-thread loop
// over them, which would hold NT/64 registers).
template <int NT>
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* scratch, uint32_t* total) {
  constexpr int NW = NT / kWave;
  static_assert(NW <= kWave, "one wave combines the wave totals");
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
  const uint32_t inc = wave_inclusive_scan(v);
  if (lane == kWave - 1) scratch[wave] = inc;
  __syncthreads();
  const uint32_t t = lane < NW ? scratch[lane] : 0u;
  const uint32_t tinc = wave_inclusive_scan(t);
  *total = (uint32_t)__builtin_amdgcn_readlane((int)tinc, NW - 1);
  const uint32_t before = wave > 0 ? (uint32_t)__builtin_amdgcn_readlane((int)tinc, wave - 1) : 0u;
  return before + inc - v;
}

// Combine per-wave values that waves 0..nw-1 published in slots[0..nw-1]
// (nw <= 64): lane l reads slot l and a wave reduction finishes; uniform.
__device__ __forceinline__ uint32_t lds_slots_max(const uint32_t* slots, int nw) {
  return wave_max_u32(lane_id() < nw ? slots[lane_id()] : 0u);
}
__device__ __forceinline__ uint32_t lds_slots_min(const uint32_t* slots, int nw) {
  return wave_min_u32(lane_id() < nw ? slots[lane_id()] : 0xFFFFFFFFu);
}

// Rows longer than this many blocks are selected in two launches (slices,
// then their candidates); shorter ones by one workgroup per query.
constexpr int kLongRowBlocks = 32768;

// Attention split geometry shared by the launcher and the workspace sizing.
struct AttnSplit {
  int splits;            // workgroups per (query, KV head): the grid's third dimension
  int chunks_per_split;  // 32-position chunks per workgroup (multiple of kAttnWaves); with
                         // ragged, the least the work list takes
};

// ragged = false: every unit is split alike, into enough workgroups that
// about kAttnTargetWgs are resident (two 4-wave workgroups per CU).
// ragged = true (batches of several requests, whose units' position counts
// differ): room for up to twice as many splits per unit; the work list
// (AttnPlan) sizes the splits from the batch's total positions, so that a
// long unit gets several workgroups and a short one a single one, and the
// grid's workgroups past the list leave at once.  Only while the units
// number fewer than kAttnTargetWgs (their arrival counters must fit the
// control region).
__host__ __device__ inline AttnSplit attn_split(int num_q, int num_kv_heads, int width, bool ragged = false) {
  const int chunks = (width + kChunk - 1) / kChunk;
  const int units = num_q * num_kv_heads;
  const int target = ragged ? 2 * kAttnTargetWgs : kAttnTargetWgs;
  int splits = units >= kAttnTargetWgs ? 1 : (target + units - 1) / units;
  int max_splits = (chunks + kAttnWaves - 1) / kAttnWaves;   // <= kMaxSplits for width <= QSA_WIDTH
  if (splits > max_splits) splits = max_splits;
  if (splits < 1) splits = 1;
  int cps = (chunks + splits - 1) / splits;
  cps = (cps + kAttnWaves - 1) / kAttnWaves * kAttnWaves;
  splits = (chunks + cps - 1) / cps;
  AttnSplit a;
  a.splits = splits;
  a.chunks_per_split = cps;
  return a;
}

// The most chunks one attention split takes: a whole 2,051-position row,
// its 65 chunks rounded up to whole 4-chunk steps.
constexpr int kMaxSplitChunks = ((QSA_WIDTH + kChunk - 1) / kChunk + kAttnWaves - 1) / kAttnWaves * kAttnWaves;

// Work list of the attention for a ragged batch, written by one extra
// workgroup of the selection launch inside qsa_decode (or by a launch of its
// own before qsa_sparse_attn): kPlanHeader header words
// ([0] items, [1] chunks per split), then one word per item (query, KV
// head, split, the unit's splits): every split of the full chunk count
// first, then each unit's last, shorter split, longest first (a longest-
// first list: the long work starts first, short work fills in at the end).
// Attention workgroup w takes item w.
constexpr int kPlanHeader = 16;
// An item packs (query, KV head, split, splits) into 9 + 8 + 5 + 5 bits: a
// list exists only while query x KV head units number under 512 on a batch
// of two or more queries, so q < 256 and g < 256 whenever both are in use
// (q < 512 alone), and a unit has at most kMaxSplits (17) splits.
constexpr int kPlanQBits = 9, kPlanGBits = 8, kPlanSBits = 5;
static_assert(kMaxSplits < (1 << kPlanSBits), "split index and count fit their fields");
static_assert(kAttnTargetWgs <= (1 << kPlanQBits) && kAttnTargetWgs / 2 <= (1 << kPlanGBits),
              "query and KV head indices of a listed batch fit their fields");
__host__ __device__ inline uint32_t plan_item(int q, int g, int s, int S) {
  return (uint32_t)q | ((uint32_t)g << kPlanQBits) | ((uint32_t)s << (kPlanQBits + kPlanGBits)) |
         ((uint32_t)S << (kPlanQBits + kPlanGBits + kPlanSBits));
}
__host__ __device__ inline void plan_unpack(uint32_t e, int& q, int& g, int& s, int& S) {
  q = (int)(e & ((1u << kPlanQBits) - 1u));
  g = (int)((e >> kPlanQBits) & ((1u << kPlanGBits) - 1u));
  s = (int)((e >> (kPlanQBits + kPlanGBits)) & ((1u << kPlanSBits) - 1u));
  S = (int)((e >> (kPlanQBits + kPlanGBits + kPlanSBits)) & ((1u << kPlanSBits) - 1u));
}
struct AttnPlan {
  int32_t* words;         // header + items (workspace); nullptr: no plan
  int num_kv_heads;
  int k;                  // selection size (positions of a query: 4 min(L/4, k) + L mod 4)
  int cps_min;            // least chunks per split (so no unit needs more splits than the grid has)
  const int32_t* n_pos;   // the position counts to plan for (clamped to pos_cap), or nullptr: from the metadata
  int pos_cap;
};

// Whether a batch takes the ragged split geometry (see attn_split).
__host__ __device__ inline bool attn_ragged(int num_req, int num_q, int num_kv_heads) {
  return num_req > 1 && num_q * num_kv_heads < kAttnTargetWgs;
}

}  // namespace qsa
