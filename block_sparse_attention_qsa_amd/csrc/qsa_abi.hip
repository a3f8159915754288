// C ABI of libqsa.so: host-side validation, workspace layout and dispatch of
// the QSA kernels.  Every entry point only enqueues work on the caller's
// stream; see include/qsa.h for the contract of each call.
#include <math.h>

#include <mutex>

#include "qsa.h"
#include "qsa_common.hpp"
#include "qsa_launch.hpp"

namespace qsa {

// Zero-fill of n bytes (a multiple of 16) at p, as a kernel (so that it can
// sit in a captured graph).
__global__ __launch_bounds__(256) void zero_fill_kernel(u32x4* p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256)
    p[i] = u32x4{0u, 0u, 0u, 0u};
}

hipError_t launch_zero_fill(void* p, size_t bytes, hipStream_t stream) {
  const size_t n16 = bytes / 16;
  const unsigned grid = (unsigned)((n16 + 255) / 256 < 1024 ? (n16 + 255) / 256 : 1024);
  zero_fill_kernel<<<grid, 256, 0, stream>>>(static_cast<u32x4*>(p), n16);
  return hipGetLastError();
}

}  // namespace qsa

namespace {

using qsa::Meta;

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Largest score row stride qsa_score takes: the four rows of a request are
// addressed by 32-bit byte offsets from its first one.
constexpr int64_t kMaxScoreLd = int64_t(1) << 26;

struct WsLayout {
  size_t counters, plan, partials, attn_end, scores, sel, n_sel, pos, n_pos, msel, total;
};

// Row stride of the workspace score buffer: a multiple of 4 floats so that
// score rows are 16-byte aligned.
inline int64_t score_ld(int max_blocks) { return ((int64_t)(max_blocks > 0 ? max_blocks : 1) + 3) & ~(int64_t)3; }

WsLayout ws_layout(int num_q, int max_blocks, int hq, int hkv, int k) {
  WsLayout w;
  const int width = QSA_BLOCK * k + QSA_BLOCK - 1;
  size_t off = 0;
  // fixed control region first (see kCtlBytes), whatever the geometry
  w.counters = off; off += align_up(qsa::kCtlBytes);
  w.plan = off; off += align_up(qsa::attn_plan_bytes(num_q, hkv, width));
  w.partials = off; off += align_up(qsa::attn_partial_bytes(num_q, hkv, hq / hkv, width));
  w.attn_end = off;
  w.scores = off; off += align_up((size_t)num_q * (size_t)score_ld(max_blocks) * sizeof(float));
  w.sel = off; off += align_up((size_t)num_q * k * sizeof(int32_t));
  w.n_sel = off; off += align_up((size_t)num_q * sizeof(int32_t));
  w.pos = off; off += align_up((size_t)num_q * width * sizeof(int32_t));
  w.n_pos = off; off += align_up((size_t)num_q * sizeof(int32_t));
  // the long-row selector's slice candidates (qsa_select_topk places them
  // right after the control region instead)
  w.msel = off; off += align_up(qsa::select_workspace_bytes(num_q, max_blocks));
  w.total = off;
  return w;
}

qsa_status check_batch(const qsa_batch* b) {
  if (!b) return QSA_ERR_NULL;
  if (!b->q_start || !b->seq_len || !b->blk_start) return QSA_ERR_NULL;
  if (!b->page_table && !b->kv_start) return QSA_ERR_NULL;
  if (b->num_req < 1 || b->num_req > QSA_MAX_REQUESTS) return QSA_ERR_SHAPE;
  if (b->num_q < b->num_req || b->num_q > QSA_MAX_Q_PER_REQ * b->num_req) return QSA_ERR_SHAPE;
  if (b->max_blocks < 0 || b->max_blocks > QSA_MAX_BLOCKS) return QSA_ERR_SHAPE;
  if (b->page_table) {
    if (b->page_size < QSA_BLOCK || b->page_size % QSA_BLOCK != 0 || b->pages_per_req < 1) return QSA_ERR_SHAPE;
    if ((int64_t)b->page_size * b->pages_per_req > INT32_MAX) return QSA_ERR_SHAPE;
  }
  return QSA_OK;
}

qsa_status check_heads(int32_t hq, int32_t hkv) {
  if (hq < 1 || hkv < 1 || hq % hkv != 0) return QSA_ERR_SHAPE;
  if (hq / hkv > QSA_MAX_GQA_GROUP) return QSA_ERR_UNSUPPORTED;
  if ((int64_t)hq * hkv > (1 << 16)) return QSA_ERR_SHAPE;
  return QSA_OK;
}

qsa_status check_k(int32_t k) { return (k < 1 || k > QSA_TOPK) ? QSA_ERR_SHAPE : QSA_OK; }

qsa_status check_ws(const void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return QSA_OK;
  if (!ws || ws_bytes < need || ((uintptr_t)ws % kAlign) != 0) return QSA_ERR_WORKSPACE;
  return QSA_OK;
}

qsa_status check_attn_args(const void* q, const void* kc, const void* vc, int32_t kv_dtype, const float* ks,
                           const float* vs, float sm_scale, void* out, int32_t out_dtype) {
  if (!q || !kc || !vc || !out) return QSA_ERR_NULL;
  if (kv_dtype != QSA_KV_BF16 && kv_dtype != QSA_KV_FP8_E4M3) return QSA_ERR_UNSUPPORTED;
  if (kv_dtype == QSA_KV_FP8_E4M3 && (!ks || !vs)) return QSA_ERR_NULL;
  if (out_dtype != QSA_OUT_F32 && out_dtype != QSA_OUT_BF16) return QSA_ERR_UNSUPPORTED;
  if (reinterpret_cast<uintptr_t>(out) % (out_dtype == QSA_OUT_F32 ? 16 : 8) != 0) return QSA_ERR_SHAPE;
  if (!(sm_scale > 0.f) || !isfinite(sm_scale)) return QSA_ERR_SHAPE;
  return QSA_OK;
}

// The per-device error word (QSA_ERROR_* bits, see qsa_error_read): one copy
// per device, zero when the library's code is loaded there.  Kernels get its
// device address, looked up once per device.
__device__ uint32_t error_word;

constexpr int kMaxDevices = 64;
std::once_flag g_err_once[kMaxDevices];
uint32_t* g_err_ptr[kMaxDevices];

uint32_t* device_error_word() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::call_once(g_err_once[dev], [dev]() {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(error_word)) != hipSuccess) p = nullptr;
    g_err_ptr[dev] = static_cast<uint32_t*>(p);
  });
  return g_err_ptr[dev];
}

Meta meta_of(const qsa_batch* b) {
  Meta m;
  m.err = device_error_word();
  m.num_req = b->num_req;
  m.num_q = b->num_q;
  m.max_blocks = b->max_blocks;
  m.q_start = b->q_start;
  m.seq_len = b->seq_len;
  m.kv_start = b->kv_start;
  m.blk_start = b->blk_start;
  m.page_table = b->page_table;
  m.page_size = b->page_table ? b->page_size : 0;
  m.pages_per_req = b->page_table ? b->pages_per_req : 0;
  return m;
}

inline qsa_status launched(hipError_t e) { return e == hipSuccess ? QSA_OK : QSA_ERR_LAUNCH; }

#define QSA_TRY(x)                  \
  do {                              \
    qsa_status st_ = (x);           \
    if (st_ != QSA_OK) return st_;  \
  } while (0)


qsa_status check_decode_args(const qsa_batch* batch, const void* idx_q, const void* ckeys, const void* q,
                             const void* k_cache, const void* v_cache, int32_t kv_dtype, const float* k_scale,
                             const float* v_scale, int32_t num_q_heads, int32_t num_kv_heads, int32_t k,
                             float sm_scale, void* out, int32_t out_dtype) {
  QSA_TRY(check_batch(batch));
  QSA_TRY(check_heads(num_q_heads, num_kv_heads));
  QSA_TRY(check_k(k));
  QSA_TRY(check_attn_args(q, k_cache, v_cache, kv_dtype, k_scale, v_scale, sm_scale, out, out_dtype));
  if (!idx_q || !ckeys) return QSA_ERR_NULL;
  return QSA_OK;
}

// a1 -> a4 on the workspace at base (layout w, already checked).
qsa_status decode_body(const qsa_batch* batch, const void* idx_q, const void* ckeys, const void* q,
                       const void* k_cache, const void* v_cache, int32_t kv_dtype, const float* k_scale,
                       const float* v_scale, int32_t num_q_heads, int32_t num_kv_heads, int32_t k, float sm_scale,
                       void* out, int32_t out_dtype, int32_t* sel_opt, int32_t* n_sel_opt, int32_t* pos_opt,
                       int32_t* n_pos_opt, char* base, const WsLayout& w, hipStream_t stream) {
  const int width = QSA_BLOCK * k + QSA_BLOCK - 1;
  float* scores = reinterpret_cast<float*>(base + w.scores);
  int32_t* sel = sel_opt ? sel_opt : reinterpret_cast<int32_t*>(base + w.sel);
  int32_t* n_sel = n_sel_opt ? n_sel_opt : reinterpret_cast<int32_t*>(base + w.n_sel);
  int32_t* pos = pos_opt ? pos_opt : reinterpret_cast<int32_t*>(base + w.pos);
  int32_t* n_pos = n_pos_opt ? n_pos_opt : reinterpret_cast<int32_t*>(base + w.n_pos);
  const Meta m = meta_of(batch);
  const int64_t ld = score_ld(batch->max_blocks);

  // Without a position buffer to return, the selector hands the attention one
  // slot per 4-slot run (a quarter of the position rows) instead.
  const bool run_heads = pos_opt == nullptr;
  QSA_TRY(launched(qsa::launch_score(m, idx_q, ckeys, scores, ld, stream)));
  // a ragged batch: the selection launch also writes the attention's work list
  qsa::AttnPlan plan{nullptr, num_kv_heads, k, 0, nullptr, 0};
  if (qsa::attn_ragged(m.num_req, m.num_q, num_kv_heads)) {
    plan.words = reinterpret_cast<int32_t*>(base + w.plan);
    plan.cps_min = qsa::attn_split(m.num_q, num_kv_heads, width, true).chunks_per_split;
  }
  QSA_TRY(launched(qsa::launch_select(m, scores, ld, k, sel, n_sel, pos, n_pos, run_heads ? k + 1 : width, run_heads,
                                      base + w.msel, plan, stream)));
  qsa::AttnArgs a;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.kv_fp8 = kv_dtype == QSA_KV_FP8_E4M3;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.pos = pos;
  a.n_pos = n_pos;
  a.width = run_heads ? k + 1 : width;
  a.run_heads = run_heads;
  a.sm_scale = sm_scale;
  a.out = out;
  a.out_bf16 = out_dtype == QSA_OUT_BF16;
  a.partials = reinterpret_cast<float*>(base + w.partials);
  a.counters = reinterpret_cast<uint32_t*>(base + w.counters);
  a.plan = plan.words;
  a.err = m.err;
  return launched(qsa::launch_attn(m, a, stream));
}

// Scratch memory of qsa_decode_static: one copy of this array per device the
// library runs on, held until the process ends.  Host code never passes the
// array's name to a kernel (on the host it only names the symbol): it uses the
// device address hipGetSymbolAddress returns for the current device, looked
// up once per device.
__device__ __align__(256) uint8_t scratch[QSA_STATIC_SCRATCH_BYTES];

std::once_flag g_scratch_once[kMaxDevices];
char* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// The device address of the current device's scratch.  The first call on a
// device looks it up and enqueues on `stream` a kernel that zero-fills its
// control region (counters must start at zero; every later call leaves them
// zero again).  No allocation: the array exists from the moment the library's
// code is loaded on the device.
qsa_status static_scratch(char** base, hipStream_t stream) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return QSA_ERR_LAUNCH;
  bool first = false;
  std::call_once(g_scratch_once[dev], [&]() {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = static_cast<char*>(p);
    first = true;
  });
  if (g_scratch_err[dev] != hipSuccess || g_scratch_ptr[dev] == nullptr) return QSA_ERR_LAUNCH;
  if (first) QSA_TRY(launched(qsa::launch_zero_fill(g_scratch_ptr[dev], qsa::kCtlBytes, stream)));
  *base = g_scratch_ptr[dev];
  return QSA_OK;
}
}  // namespace

extern "C" {

int qsa_abi_version(void) { return QSA_ABI_VERSION; }

const char* qsa_status_string(int status) {
  switch (status) {
    case QSA_OK: return "ok";
    case QSA_ERR_NULL: return "a required pointer is NULL";
    case QSA_ERR_SHAPE: return "a size argument is out of range or inconsistent";
    case QSA_ERR_UNSUPPORTED: return "unsupported dtype or head geometry";
    case QSA_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case QSA_ERR_LAUNCH: return "kernel launch failed";
    case QSA_ERR_SCRATCH: return "the batch needs more scratch than qsa_decode_static holds (QSA_STATIC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

int qsa_debug_build(void) {
#ifdef QSA_DEBUG_CHECKS
  return 1;
#else
  return 0;
#endif
}

qsa_status qsa_error_read(uint32_t* bits, int clear) {
  if (!bits) return QSA_ERR_NULL;
  if (hipDeviceSynchronize() != hipSuccess) return QSA_ERR_LAUNCH;
  if (hipMemcpyFromSymbol(bits, HIP_SYMBOL(error_word), sizeof(uint32_t)) != hipSuccess) return QSA_ERR_LAUNCH;
  if (clear) {
    const uint32_t zero = 0u;
    if (hipMemcpyToSymbol(HIP_SYMBOL(error_word), &zero, sizeof(uint32_t)) != hipSuccess) return QSA_ERR_LAUNCH;
    if (hipDeviceSynchronize() != hipSuccess) return QSA_ERR_LAUNCH;
  }
  return QSA_OK;
}

size_t qsa_workspace_bytes(const qsa_batch* batch, int32_t num_q_heads, int32_t num_kv_heads, int32_t k) {
  if (check_batch(batch) != QSA_OK || check_heads(num_q_heads, num_kv_heads) != QSA_OK || check_k(k) != QSA_OK)
    return 0;
  return ws_layout(batch->num_q, batch->max_blocks, num_q_heads, num_kv_heads, k).total;
}

qsa_status qsa_score(const qsa_batch* batch, const void* idx_q, const void* ckeys, float* scores, int64_t ld,
                     hipStream_t stream) {
  QSA_TRY(check_batch(batch));
  if (!idx_q || !ckeys || !scores) return QSA_ERR_NULL;
  if (ld < batch->max_blocks || ld > kMaxScoreLd) return QSA_ERR_SHAPE;
  return launched(qsa::launch_score(meta_of(batch), idx_q, ckeys, scores, ld, stream));
}

qsa_status qsa_select_topk(const qsa_batch* batch, const float* scores, int64_t ld, int32_t k, int32_t* sel,
                           int32_t* n_sel, void* ws, size_t ws_bytes, hipStream_t stream) {
  QSA_TRY(check_batch(batch));
  QSA_TRY(check_k(k));
  if (!scores || !sel || !n_sel) return QSA_ERR_NULL;
  if (ld < batch->max_blocks) return QSA_ERR_SHAPE;
  // long rows keep their slices' candidates in the workspace, after its
  // control region (never over a counter another call may rely on)
  const size_t cand = qsa::select_workspace_bytes(batch->num_q, batch->max_blocks);
  QSA_TRY(check_ws(ws, ws_bytes, cand ? qsa::kCtlBytes + cand : 0));
  return launched(qsa::launch_select(meta_of(batch), scores, ld, k, sel, n_sel, nullptr, nullptr,
                                     QSA_BLOCK * k + QSA_BLOCK - 1, false,
                                     cand ? static_cast<char*>(ws) + qsa::kCtlBytes : nullptr, qsa::AttnPlan{nullptr, 0, 0, 0, nullptr, 0},
                                     stream));
}

qsa_status qsa_select_positions(const qsa_batch* batch, const float* scores, int64_t ld, int32_t k, int32_t* sel,
                                int32_t* n_sel, int32_t* pos, int32_t* n_pos, void* ws, size_t ws_bytes,
                                hipStream_t stream) {
  QSA_TRY(check_batch(batch));
  QSA_TRY(check_k(k));
  if (!scores || !sel || !n_sel || !pos || !n_pos) return QSA_ERR_NULL;
  if (ld < batch->max_blocks) return QSA_ERR_SHAPE;
  const size_t cand = qsa::select_workspace_bytes(batch->num_q, batch->max_blocks);
  QSA_TRY(check_ws(ws, ws_bytes, cand ? qsa::kCtlBytes + cand : 0));
  return launched(qsa::launch_select(meta_of(batch), scores, ld, k, sel, n_sel, pos, n_pos,
                                     QSA_BLOCK * k + QSA_BLOCK - 1, false,
                                     cand ? static_cast<char*>(ws) + qsa::kCtlBytes : nullptr, qsa::AttnPlan{nullptr, 0, 0, 0, nullptr, 0},
                                     stream));
}

qsa_status qsa_build_index(const qsa_batch* batch, const int32_t* sel, const int32_t* n_sel, int32_t k,
                           int32_t* pos, int32_t* n_pos, hipStream_t stream) {
  QSA_TRY(check_batch(batch));
  QSA_TRY(check_k(k));
  if (!sel || !n_sel || !pos || !n_pos) return QSA_ERR_NULL;
  return launched(qsa::launch_build_index(meta_of(batch), sel, n_sel, k, pos, n_pos,
                                          QSA_BLOCK * k + QSA_BLOCK - 1, stream));
}

qsa_status qsa_sparse_attn(const qsa_batch* batch, const void* q, const void* k_cache, const void* v_cache,
                           int32_t kv_dtype, const float* k_scale, const float* v_scale, int32_t num_q_heads,
                           int32_t num_kv_heads, const int32_t* pos, const int32_t* n_pos, int32_t width,
                           float sm_scale, void* out, int32_t out_dtype, void* ws, size_t ws_bytes,
                           hipStream_t stream) {
  QSA_TRY(check_batch(batch));
  QSA_TRY(check_heads(num_q_heads, num_kv_heads));
  QSA_TRY(check_attn_args(q, k_cache, v_cache, kv_dtype, k_scale, v_scale, sm_scale, out, out_dtype));
  if (!pos || !n_pos) return QSA_ERR_NULL;
  if (width < QSA_BLOCK + QSA_BLOCK - 1 || width > QSA_WIDTH || (width - (QSA_BLOCK - 1)) % QSA_BLOCK != 0)
    return QSA_ERR_SHAPE;
  const int k = (width - (QSA_BLOCK - 1)) / QSA_BLOCK;
  const WsLayout w = ws_layout(batch->num_q, batch->max_blocks, num_q_heads, num_kv_heads, k);
  // A ragged batch writes its work list there even when no unit is split;
  // otherwise only split units (partials and arrival counters) use it.
  const bool ragged = qsa::attn_ragged(batch->num_req, batch->num_q, num_kv_heads);
  QSA_TRY(check_ws(ws, ws_bytes, ragged || w.attn_end > w.partials ? w.attn_end : 0));
  char* base = static_cast<char*>(ws);
  qsa::AttnArgs a;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.kv_fp8 = kv_dtype == QSA_KV_FP8_E4M3;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.pos = pos;
  a.n_pos = n_pos;
  a.width = width;
  a.run_heads = 0;
  a.sm_scale = sm_scale;
  a.out = out;
  a.out_bf16 = out_dtype == QSA_OUT_BF16;
  a.partials = reinterpret_cast<float*>(base + w.partials);
  a.counters = reinterpret_cast<uint32_t*>(base + w.counters);
  a.plan = nullptr;
  a.err = device_error_word();
  const qsa::Meta m = meta_of(batch);
  if (ragged) {
    // a ragged batch: a work list from the given position counts first
    qsa::AttnPlan plan{reinterpret_cast<int32_t*>(base + w.plan), num_kv_heads, k,
                       qsa::attn_split(m.num_q, num_kv_heads, width, true).chunks_per_split, n_pos, width};
    QSA_TRY(launched(qsa::launch_attn_plan(m, plan, stream)));
    a.plan = plan.words;
  }
  return launched(qsa::launch_attn(m, a, stream));
}

qsa_status qsa_compress_keys(const qsa_batch* batch, const int32_t* prev_len, const void* tok_keys, void* ckeys,
                             hipStream_t stream) {
  QSA_TRY(check_batch(batch));
  if (!prev_len || !tok_keys || !ckeys) return QSA_ERR_NULL;
  return launched(qsa::launch_compress_keys(meta_of(batch), prev_len, tok_keys, ckeys, stream));
}

qsa_status qsa_decode(const qsa_batch* batch, const void* idx_q, const void* ckeys, const void* q,
                      const void* k_cache, const void* v_cache, int32_t kv_dtype, const float* k_scale,
                      const float* v_scale, int32_t num_q_heads, int32_t num_kv_heads, int32_t k, float sm_scale,
                      void* out, int32_t out_dtype, int32_t* sel_opt, int32_t* n_sel_opt, int32_t* pos_opt,
                      int32_t* n_pos_opt, void* ws, size_t ws_bytes, hipStream_t stream) {
  QSA_TRY(check_decode_args(batch, idx_q, ckeys, q, k_cache, v_cache, kv_dtype, k_scale, v_scale, num_q_heads,
                            num_kv_heads, k, sm_scale, out, out_dtype));
  const WsLayout w = ws_layout(batch->num_q, batch->max_blocks, num_q_heads, num_kv_heads, k);
  QSA_TRY(check_ws(ws, ws_bytes, w.total));
  return decode_body(batch, idx_q, ckeys, q, k_cache, v_cache, kv_dtype, k_scale, v_scale, num_q_heads,
                     num_kv_heads, k, sm_scale, out, out_dtype, sel_opt, n_sel_opt, pos_opt, n_pos_opt,
                     static_cast<char*>(ws), w, stream);
}

qsa_status qsa_decode_static(const qsa_batch* batch, const void* idx_q, const void* ckeys, const void* q,
                             const void* k_cache, const void* v_cache, int32_t kv_dtype, const float* k_scale,
                             const float* v_scale, int32_t num_q_heads, int32_t num_kv_heads, int32_t k,
                             float sm_scale, void* out, int32_t out_dtype, int32_t* sel_opt, int32_t* n_sel_opt,
                             int32_t* pos_opt, int32_t* n_pos_opt, hipStream_t stream) {
  QSA_TRY(check_decode_args(batch, idx_q, ckeys, q, k_cache, v_cache, kv_dtype, k_scale, v_scale, num_q_heads,
                            num_kv_heads, k, sm_scale, out, out_dtype));
  const WsLayout w = ws_layout(batch->num_q, batch->max_blocks, num_q_heads, num_kv_heads, k);
  if (w.total > QSA_STATIC_SCRATCH_BYTES) return QSA_ERR_SCRATCH;
  char* base = nullptr;
  QSA_TRY(static_scratch(&base, stream));
  return decode_body(batch, idx_q, ckeys, q, k_cache, v_cache, kv_dtype, k_scale, v_scale, num_q_heads,
                     num_kv_heads, k, sm_scale, out, out_dtype, sel_opt, n_sel_opt, pos_opt, n_pos_opt, base, w,
                     stream);
}

}  // extern "C"
