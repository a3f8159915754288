/* A plain C99 program against include/qsa.h and libqsa.so: the boundary is
 * usable from C without any C++ or PyTorch.  It calls only entry points that
 * need no GPU (version, status strings, workspace sizing, argument checks
 * that return before anything is enqueued) and exits non-zero on the first
 * mismatch. */
#include <stdio.h>
#include <string.h>

#include "qsa.h"

#define EXPECT(cond)                                                    \
  do {                                                                  \
    if (!(cond)) {                                                      \
      fprintf(stderr, "abi_check: failed at line %d: %s\n", __LINE__, #cond); \
      return 1;                                                         \
    }                                                                   \
  } while (0)

int main(void) {
  int32_t meta[8] = {0, 4, 12500, 0, 0, 0, 0, 0};
  qsa_batch b;
  memset(&b, 0, sizeof b);
  b.num_req = 1;
  b.num_q = 4;
  b.max_blocks = 12500;
  b.q_start = meta;          /* host addresses stand in for device ones: no call below reads them */
  b.seq_len = meta + 2;
  b.kv_start = meta + 4;
  b.blk_start = meta + 5;

  EXPECT(qsa_abi_version() == QSA_ABI_VERSION);
  EXPECT(strlen(qsa_status_string(QSA_OK)) > 0);
  EXPECT(qsa_debug_build() == 0);

  /* the 50,000-token batch-1 geometry needs workspace, a k of 0 none */
  EXPECT(qsa_workspace_bytes(&b, 32, 4, QSA_TOPK) > 0);
  EXPECT(qsa_workspace_bytes(&b, 32, 4, 0) == 0);
  EXPECT(qsa_workspace_bytes(NULL, 32, 4, QSA_TOPK) == 0);

  /* argument checks return before anything is enqueued */
  EXPECT(qsa_score(NULL, meta, meta, NULL, 12500, NULL) == QSA_ERR_NULL);
  EXPECT(qsa_score(&b, meta, meta, (float*)meta, 100, NULL) == QSA_ERR_SHAPE);
  EXPECT(qsa_select_topk(&b, (const float*)meta, 12500, 0, meta, meta, NULL, 0, NULL) != QSA_OK);
  EXPECT(qsa_build_index(&b, meta, meta, QSA_TOPK, NULL, meta, NULL) == QSA_ERR_NULL);
  EXPECT(qsa_decode(&b, meta, meta, meta, meta, meta, QSA_KV_BF16, NULL, NULL, 32, 4, QSA_TOPK, 0.0f, meta,
                    QSA_OUT_F32, NULL, NULL, NULL, NULL, NULL, 0, NULL) != QSA_OK);
  b.num_q = 5;               /* five queries in one request */
  EXPECT(qsa_score(&b, meta, meta, (float*)meta, 12500, NULL) == QSA_ERR_SHAPE);

  printf("abi_check: ok (ABI %d)\n", qsa_abi_version());
  return 0;
}
