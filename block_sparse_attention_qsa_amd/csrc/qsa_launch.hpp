// Host-side launchers of the QSA kernels (internal to libqsa.so).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qsa.h"
#include "qsa_common.hpp"

namespace qsa {

struct Meta {
  int num_req, num_q, max_blocks;
  const int32_t* q_start;
  const int32_t* seq_len;
  const int32_t* kv_start;
  const int32_t* blk_start;
  const int32_t* page_table;   // nullptr: contiguous requests from kv_start
  int page_size, pages_per_req;
  uint32_t* err;               // the device's error word (QSA_ERROR_* bits)
};

// Debug builds (QSA_DEBUG_CHECKS) check device-side preconditions and set a
// bit of the error word when one fails; release builds compile the checks
// away.  Either way the kernels go on with clamped values.
#ifdef QSA_DEBUG_CHECKS
#define QSA_DCHECK(err, cond, bit) \
  do {                             \
    if (!(cond)) atomicOr((err), (uint32_t)(bit)); \
  } while (0)
#else
#define QSA_DCHECK(err, cond, bit) \
  do {                             \
  } while (0)
#endif

// KV slot of token t of request r: kv_start[r] + t, or through the page table
// (page_size a multiple of 4, so a block's 4 tokens are 4 consecutive slots).
// The logical page is clamped to the table row.
__device__ __forceinline__ int32_t token_slot(const Meta& m, int r, int t) {
  if (m.page_table == nullptr) return m.kv_start[r] + t;
  int p = t / m.page_size;
  QSA_DCHECK(m.err, p < m.pages_per_req, QSA_ERROR_BAD_PAGE);
  p = p < m.pages_per_req ? p : m.pages_per_req - 1;
  const int32_t page = m.page_table[(int64_t)r * m.pages_per_req + p];
  QSA_DCHECK(m.err, page >= 0, QSA_ERROR_BAD_PAGE);
  return page * m.page_size + t % m.page_size;
}

struct AttnArgs {
  const void* q;            // BF16 [num_q][Hq][128]
  const void* k_cache;      // [slots][Hkv][128] BF16 or FP8
  const void* v_cache;
  const float* k_scale;     // [Hkv] (FP8 only)
  const float* v_scale;
  int kv_fp8;
  int num_q_heads, num_kv_heads;
  const int32_t* pos;       // [num_q][width] positions, or with run_heads one slot per 4-slot run
  const int32_t* n_pos;     // [num_q]
  int width;
  int run_heads;
  float sm_scale;
  void* out;                // [num_q][Hq][128]
  int out_bf16;
  float* partials;          // split partial results (workspace)
  uint32_t* counters;       // [num_q][Hkv] split arrival counters (workspace, zero)
  const int32_t* plan;      // the work list the selection wrote for a ragged batch, or nullptr
  uint32_t* err;            // error word (QSA_ERROR_* bits) or nullptr
};

hipError_t launch_score(const Meta& m, const void* idx_q, const void* ckeys, float* scores, int64_t ld,
                        hipStream_t stream);
// Writes sel/n_sel, and, when pos != nullptr, n_pos and either the position
// rows (width entries per query) or, with run_heads, one slot per 4-slot run
// (the first position of each kept block, then of the partial block; rows of
// width >= k + 1 entries).  Rows longer than 32,768 blocks keep their slices'
// candidates in select_workspace_bytes() of workspace at ws (256-byte aligned;
// no initial contents needed).
// With plan.words, one extra workgroup writes the attention's work list for
// a ragged batch there (AttnPlan; attn_plan_bytes()).
hipError_t launch_select(const Meta& m, const float* scores, int64_t ld, int k, int32_t* sel,
                         int32_t* n_sel, int32_t* pos, int32_t* n_pos, int width, bool run_heads, void* ws,
                         const AttnPlan& plan, hipStream_t stream);
size_t select_workspace_bytes(int num_q, int max_blocks);
// The attention's work list for a ragged batch of at most 511 queries, from
// plan.n_pos, in a launch of its own.
hipError_t launch_attn_plan(const Meta& m, const AttnPlan& plan, hipStream_t stream);
hipError_t launch_build_index(const Meta& m, const int32_t* sel, const int32_t* n_sel, int k, int32_t* pos,
                              int32_t* n_pos, int width, hipStream_t stream);
hipError_t launch_attn(const Meta& m, const AttnArgs& a, hipStream_t stream);
hipError_t launch_compress_keys(const Meta& m, const int32_t* prev_len, const void* tok_keys, void* ckeys,
                                hipStream_t stream);

// Zero-fills bytes (a multiple of 16) at p with a kernel on stream.
hipError_t launch_zero_fill(void* p, size_t bytes, hipStream_t stream);

// Bytes of the attention's work list for a ragged batch of this geometry
// (0 when the batch could not take one).
size_t attn_plan_bytes(int num_q, int num_kv_heads, int width);
// Bytes of split partials the attention needs for this geometry.
size_t attn_partial_bytes(int num_q, int num_kv_heads, int group, int width);

}  // namespace qsa
