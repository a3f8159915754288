/*
 * qsa.h - C ABI of the QSA block-sparse decode attention library (libqsa.so).
 *
 * The operation follows the QSA selection pipeline described in the
 * arex-research.com article on TokenSpeed serving Qwen3.8-Flash-Next, section
 * on the four optimisations (sparse selection, CuTe DSL kernels, MTP reuse),
 * items 1-3, and the 10100.com article's section on the first optimisation:
 *
 *   tokens are grouped into 4-token micro-blocks, each full block has a
 *   compressed index key; every query scores all of its full blocks into an
 *   FP32 buffer (a1), keeps at most 512 of them by top-k (a2), keeps its current
 *   partial block without selection, which fixes the position buffer at 2,051
 *   entries (a3), and attends only over those positions with BF16 queries and
 *   BF16 or FP8 E4M3 KV (a4).  Up to 4 MTP-verify queries of one request share
 *   every compressed-key load.
 *
 * Conventions for every entry point
 *   - Pointers marked [dev] are device memory owned by the caller; [host] are
 *     host memory read during the call only.  The library allocates, frees and
 *     synchronises nothing and never reads device memory back to the host: a
 *     call validates its host arguments and enqueues kernels on `stream`.
 *   - Errors are returned as qsa_status; nothing is enqueued when a host-side
 *     check fails.  QSA_ERR_LAUNCH reports a failed kernel launch.
 *   - Device-side metadata (the qsa_batch arrays) is trusted: 1 <= nq_r <= 4,
 *     nq_r <= seq_len[r], request regions inside the caches, scores finite.
 *     Kernels clamp block counts to max_blocks so that reads of the score
 *     buffer stay inside [0, ld), and logical pages to the page-table row.
 *     The debug build checks these and reports breaches in the error word.
 *   - Calls on different streams with disjoint outputs and workspaces are
 *     independent; the library keeps no state between calls besides the
 *     per-device error word (qsa_error_read) and qsa_decode_static's scratch.
 *
 * Query geometry.  Request r owns queries q_start[r] .. q_start[r+1]-1 (its
 * nq_r MTP verify queries, or one decode query).  seq_len[r] counts the
 * request's cached tokens including this step's verify tokens, so verify query
 * j (0-based) has causal length L = seq_len[r] - nq_r + 1 + j, nf = L / 4 full
 * blocks and a partial block of L % 4 tokens (nothing when L % 4 == 0).
 * Token t of request r lives in KV slot slot_r(t) = kv_start[r] + t, or, when
 * the batch carries a page table (paged KV cache), in slot
 *   slot_r(t) = page_table[r * pages_per_req + t / page_size] * page_size + t % page_size
 * with page_size a multiple of 4, so the 4 tokens of a block always sit in 4
 * consecutive slots.  The compressed key of full block b is row
 * blk_start[r] + b of the key array (keys are not paged).
 */
#ifndef QSA_H
#define QSA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QSA_ABI_VERSION 2
#define QSA_BLOCK 4                                  /* tokens per micro-block            */
#define QSA_TOPK 512                                 /* max full blocks kept per query    */
#define QSA_WIDTH (QSA_BLOCK * QSA_TOPK + QSA_BLOCK - 1) /* 2,051 position-buffer entries */
#define QSA_INDEX_DIM 128                            /* compressed key / index query dim  */
#define QSA_HEAD_DIM 128                             /* attention head dim                */
#define QSA_MAX_Q_PER_REQ 4                          /* verify queries sharing a key load */
#define QSA_MAX_GQA_GROUP 16                         /* query heads per KV head           */
#define QSA_MAX_REQUESTS 16384                       /* num_q <= 4 * 16384 = 65536     */
#define QSA_MAX_BLOCKS (1 << 20)                     /* full blocks per request (4M tokens) */
#define QSA_STATIC_SCRATCH_BYTES ((size_t)64 << 20)  /* scratch of qsa_decode_static: 64 MiB */

typedef enum {
  QSA_OK = 0,
  QSA_ERR_NULL = 1,        /* a required pointer is NULL                          */
  QSA_ERR_SHAPE = 2,       /* a size argument is out of range or inconsistent     */
  QSA_ERR_UNSUPPORTED = 3, /* dtype / head geometry this build does not provide   */
  QSA_ERR_WORKSPACE = 4,   /* workspace missing, misaligned or too small          */
  QSA_ERR_LAUNCH = 5,      /* the HIP runtime rejected a kernel launch            */
  QSA_ERR_SCRATCH = 6      /* qsa_decode_static: the batch needs more scratch than
                              QSA_STATIC_SCRATCH_BYTES                             */
} qsa_status;

/* Bits of the per-device error word (qsa_error_read), set by the debug build
 * (libqsa_debug.so, compiled with QSA_DEBUG_CHECKS) when a device-side
 * metadata precondition that release builds trust does not hold.  Kernels set
 * a bit and go on with the same clamped values release builds use; release
 * builds never set any. */
#define QSA_ERROR_BAD_QUERIES 0x1u    /* a request with nq_r outside 1..4, or seq_len[r] < nq_r,
                                         or a prev_len outside 0..seq_len[r]               */
#define QSA_ERROR_BAD_PAGE 0x2u       /* a token past the request's page-table row, or a
                                         negative physical page                           */
#define QSA_ERROR_BAD_POSITIONS 0x4u  /* a position buffer breaking the 4-slot run rule of
                                         qsa_sparse_attn, or n_pos outside 1..width        */
#define QSA_ERROR_BAD_BLOCKS 0x8u     /* seq_len[r] / 4 > max_blocks                       */
#define QSA_ERROR_BAD_SELECTION 0x10u /* qsa_build_index given n_sel outside 0..k, or a
                                         selection row that is not ascending              */

typedef enum { QSA_KV_BF16 = 0, QSA_KV_FP8_E4M3 = 1 } qsa_kv_dtype; /* FP8 = OCP E4M3FN */
typedef enum { QSA_OUT_F32 = 0, QSA_OUT_BF16 = 1 } qsa_out_dtype;

/* Batch description: host scalars plus device metadata arrays. */
typedef struct {
  int32_t num_req;           /* [host] B >= 1                                          */
  int32_t num_q;             /* [host] total queries = q_start[B]                      */
  int32_t max_blocks;        /* [host] >= max over r of seq_len[r] / 4, <= QSA_MAX_BLOCKS */
  const int32_t* q_start;    /* [dev]  int32[B+1], q_start[0] = 0, 1..4 queries each  */
  const int32_t* seq_len;    /* [dev]  int32[B], cached tokens incl. verify tokens     */
  const int32_t* kv_start;   /* [dev]  int32[B], first KV slot of request r            */
  const int32_t* blk_start;  /* [dev]  int32[B], first compressed-key row of request r */
  const int32_t* page_table; /* [dev]  int32[B][pages_per_req] physical page of each
                                       logical page, or NULL for contiguous requests
                                       (then kv_start is used and the two fields below
                                       are ignored)                                  */
  int32_t page_size;         /* [host] tokens per page, a positive multiple of 4       */
  int32_t pages_per_req;     /* [host] row stride of page_table, >= 1                  */
} qsa_batch;

/* Version of this ABI (QSA_ABI_VERSION). */
int qsa_abi_version(void);

/* Static, human-readable text for a status code. */
const char* qsa_status_string(int status);

/* 1 in the debug build (device-side precondition checks), 0 otherwise. */
int qsa_debug_build(void);

/* Diagnostics: the OR of the QSA_ERROR_* bits kernels have set on the current
 * device since the word was last cleared, into *bits [host]; clear != 0 resets
 * it.  The word (one per device, zero when the library is loaded) is, with
 * qsa_decode_static's scratch, all the state the library keeps.  Unlike every
 * other call this one synchronises: it waits for the device to finish its work
 * and copies 4 bytes back. */
qsa_status qsa_error_read(uint32_t* bits, int clear);

/* Bytes of device workspace qsa_select_topk / qsa_sparse_attn / qsa_decode need
 * for this batch and head geometry (0 when none).  The workspace must be
 * 256-byte aligned and ZERO-FILLED before its first use.  It starts with a
 * control region of fixed size (128 KiB) that holds every counter any call
 * uses, at offsets that do not depend on the batch; the rest (scores,
 * selections, the attention's work list for batches of several requests,
 * split partials, candidates) needs no initial contents.  Every
 * call leaves the counters it used at zero again, so one zero fill serves any
 * number of calls, of any batch geometry, on the same stream, provided each
 * call is given at least the bytes this function returns for its own batch
 * (one workspace sized for the largest batch serves them all).  Calls that
 * overlap in time must not share a workspace. */
size_t qsa_workspace_bytes(const qsa_batch* batch, int32_t num_q_heads, int32_t num_kv_heads,
                           int32_t k);

/* a1 - block scores.  For every query q of request r and every full block
 * b < seq_len[r] / 4:   scores[q * ld + b] = fp32( sum_d idx_q[q][d] * ckeys[blk_start[r] + b][d] ).
 * idx_q  [dev] BF16 [num_q][128] row-major; ckeys [dev] BF16 [rows][128] row-major;
 * scores [dev] FP32 [num_q][ld], max_blocks <= ld <= 2^26.  Products are exact and the sum is
 * accumulated in FP32 (exact whenever all partial sums are integers below 2^24).
 * Each key row is read from memory once per request and used for all of its
 * queries.  Entries b >= seq_len[r] / 4 are not written. */
qsa_status qsa_score(const qsa_batch* batch, const void* idx_q, const void* ckeys, float* scores,
                     int64_t ld, hipStream_t stream);

/* a2 - top-k block selection.  For query q with nf full blocks: if nf <= k all
 * blocks 0..nf-1 are kept; otherwise the k blocks ranked first by (score
 * descending, block index ascending) are kept - the lower index wins ties and
 * -0.0 equals +0.0.  sel [dev] int32 [num_q][k] receives the kept block indices in
 * ascending order, -1 after the last; n_sel [dev] int32 [num_q] their count.
 * scores as written by qsa_score; 1 <= k <= 512.  ws: qsa_workspace_bytes() for
 * this batch (any head counts); rows longer than 32,768 blocks are selected in
 * two steps (the top k of every 8,192-block slice, 16,384 past 262,144 blocks,
 * then the top k of those candidates) that keep the candidates in the
 * workspace after its control region, so no counter is disturbed; batches of
 * shorter rows use no workspace (ws may then be NULL). */
qsa_status qsa_select_topk(const qsa_batch* batch, const float* scores, int64_t ld, int32_t k,
                           int32_t* sel, int32_t* n_sel, void* ws, size_t ws_bytes,
                           hipStream_t stream);

/* a2 + a3 in one launch, as qsa_decode runs them: the selection of
 * qsa_select_topk and, from it, the position buffer of qsa_build_index (with
 * the query's own full blocks, so every kept block is used), both written by
 * the selecting kernel.  The arex-research.com article (four optimisations,
 * item 1) keeps the selected blocks and the current partial block in one
 * 2,051-wide buffer; the 10100.com article (first optimisation) has the
 * selected pieces' cache positions found right after selection.  Arguments as
 * for qsa_select_topk, plus pos [dev] int32 [num_q][4k+3] and n_pos [dev]
 * int32 [num_q] as for qsa_build_index. */
qsa_status qsa_select_positions(const qsa_batch* batch, const float* scores, int64_t ld, int32_t k,
                                int32_t* sel, int32_t* n_sel, int32_t* pos, int32_t* n_pos, void* ws,
                                size_t ws_bytes, hipStream_t stream);

/* a3 - position buffer.  For query q of request r, of the first min(n_sel[q], k)
 * entries of sel[q] (ascending, as qsa_select_topk writes them) the n entries
 * below nf - the blocks that are full for this query - are used:
 *   pos[q][4i + t] = slot_r(4 * sel[q][i] + t)            (i < n, t < 4)
 *   pos[q][4n + t] = slot_r(4 * nf + t)                   (t < L % 4, the partial block)
 *   pos[q][i]      = -1                                   (i >= n_pos[q], up to 4k+3)
 * n_pos[q] = 4n + L % 4.  pos [dev] int32 [num_q][4k+3]; n_pos [dev] int32 [num_q].
 * Entries at or past nf are dropped rather than trusted, so a selection made
 * at an earlier step can be reused when later MTP draft steps (or a step
 * after rejected drafts) attend with other lengths, as the arex-research.com
 * article (four optimisations, MTP reuse) describes for draft steps. */
qsa_status qsa_build_index(const qsa_batch* batch, const int32_t* sel, const int32_t* n_sel,
                           int32_t k, int32_t* pos, int32_t* n_pos, hipStream_t stream);

/* a4 - gather attention over the position buffer.  For query q and head h with
 * KV head g = h / (num_q_heads / num_kv_heads):
 *   out[q][h] = sum_i softmax_i( sm_scale * q[q][h] . K(pos_i, g) ) * V(pos_i, g),  i < n_pos[q]
 * where K(s, g) is k_cache[s][g][:] (BF16) or its FP8 E4M3FN byte decoded times
 * k_scale[g] (likewise V with v_scale).  q [dev] BF16 [num_q][Hq][128];
 * k_cache, v_cache [dev] [slots][Hkv][128] of BF16 or FP8; k_scale, v_scale [dev]
 * FP32 [Hkv], required for FP8 and ignored for BF16; out [dev] [num_q][Hq][128] FP32
 * (16-byte aligned) or BF16 (8-byte aligned); a misaligned out is QSA_ERR_SHAPE.
 * pos [dev] int32 [num_q][width], width = 4k+3, and n_pos [dev] int32 [num_q],
 * 1 <= n_pos[q] <= width.  Position buffers are made of 4-slot runs, as
 * qsa_build_index writes them (one run per kept block, then the partial
 * block): for every i < n_pos[q],  pos[q][i] = pos[q][i - i % 4] + i % 4.
 * The runs may come in any order; entries past n_pos[q] are not read.  A
 * buffer that breaks the run rule gives undefined output in release builds
 * and sets QSA_ERROR_BAD_POSITIONS in a debug build (qsa_error_read above).
 * Hq % Hkv == 0 and Hq / Hkv <= 16.  ws: qsa_workspace_bytes() for this k.
 * A batch of several requests with fewer than 512 (query, KV head) units
 * takes two launches: one workgroup lays out a longest-first work list from
 * n_pos in the workspace, then the attention splits the units by it. */
qsa_status qsa_sparse_attn(const qsa_batch* batch, const void* q, const void* k_cache,
                           const void* v_cache, int32_t kv_dtype, const float* k_scale,
                           const float* v_scale, int32_t num_q_heads, int32_t num_kv_heads,
                           const int32_t* pos, const int32_t* n_pos, int32_t width,
                           float sm_scale, void* out, int32_t out_dtype, void* ws,
                           size_t ws_bytes, hipStream_t stream);

/* The step before a1: compressed keys of the blocks completed by newly
 * appended tokens.  For request r, every block b with
 * prev_len[r] <= 4b + 3 < seq_len[r] gets
 *   ckeys[blk_start[r] + b][d] = bf16_rne( (k(4b) + k(4b+1) + k(4b+2) + k(4b+3)) / 4 )
 * where k(t) = tok_keys[slot_r(t)][d] is the BF16 per-token index key, the sum
 * is taken in FP64 in that order and rounded once to BF16 (nearest, ties to
 * even).  The pages compute a compressed index key for every 4-token block
 * (arex-research.com article, four optimisations, item 1) without stating the
 * compression; the mean of the block's token keys is this library's stand-in.
 * prev_len [dev] int32 [B] (0 <= prev_len[r] <= seq_len[r]); tok_keys [dev] BF16
 * [slots][128]; ckeys [dev] BF16 [rows][128].  Other rows are not written. */
qsa_status qsa_compress_keys(const qsa_batch* batch, const int32_t* prev_len, const void* tok_keys,
                             void* ckeys, hipStream_t stream);

/* a1..a4 in one call, the whole decode / MTP-verify step of one QSA layer for
 * the batch.  This is the stand-in for the chain the arex-research.com article
 * (four optimisations, item 4) overlaps with programmatic dependent launch on
 * its hardware (selection and attention, 1.249 us saved at batch 1): here the
 * stages are consecutive kernels on one stream with no host involvement
 * between them.  Scores, selection and positions live in the
 * workspace, and
 * sel_opt [num_q][k] / n_sel_opt / pos_opt [num_q][4k+3] / n_pos_opt, when not
 * NULL, receive copies of the selection and position buffers for inspection.
 * Arguments as for the stage calls above. */
qsa_status qsa_decode(const qsa_batch* batch, const void* idx_q, const void* ckeys, const void* q,
                      const void* k_cache, const void* v_cache, int32_t kv_dtype,
                      const float* k_scale, const float* v_scale, int32_t num_q_heads,
                      int32_t num_kv_heads, int32_t k, float sm_scale, void* out,
                      int32_t out_dtype, int32_t* sel_opt, int32_t* n_sel_opt, int32_t* pos_opt,
                      int32_t* n_pos_opt, void* ws, size_t ws_bytes, hipStream_t stream);

/* qsa_decode without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation.  The call itself allocates nothing: its scratch
 * (scores, selections, split partials, counters - what qsa_decode keeps in
 * the caller's workspace) is a file-scope device array of the library,
 * QSA_STATIC_SCRATCH_BYTES (64 MiB) per device, which every device the
 * library runs on holds from the moment the library's code is loaded there
 * until the process ends.  A batch whose qsa_workspace_bytes() exceeds that
 * size is rejected with QSA_ERR_SCRATCH before anything is enqueued.  The
 * first call on a device also enqueues, on `stream`, a kernel that zero-fills
 * the scratch's counter region; every call leaves those counters zero again.
 * All calls on one device share that device's scratch: calls that overlap in
 * time on one device (other streams, other host threads) race and must be
 * serialised by the caller.  Otherwise arguments, outputs and results are
 * those of qsa_decode, with the same kernels. */
qsa_status qsa_decode_static(const qsa_batch* batch, const void* idx_q, const void* ckeys, const void* q,
                             const void* k_cache, const void* v_cache, int32_t kv_dtype,
                             const float* k_scale, const float* v_scale, int32_t num_q_heads,
                             int32_t num_kv_heads, int32_t k, float sm_scale, void* out,
                             int32_t out_dtype, int32_t* sel_opt, int32_t* n_sel_opt,
                             int32_t* pos_opt, int32_t* n_pos_opt, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* QSA_H */
