/* A plain C11 program against include/tiled_attn.h and libtiled_attn.so: it prints,
 * as one JSON object, the layout of every struct the header declares, the header's
 * constants, and the results of calls that return before any launch (argument
 * errors, size helpers, the auto-dispatch plan).  tests/test_abi.py compiles it with
 * gcc and compares each value with what the Python binding uses, so the header, the
 * library and the binding cannot drift apart unnoticed.  No GPU is touched. */
#include <stddef.h>
#include <stdio.h>

#include "tiled_attn.h"

#define FIELD(T, f) printf("\"%s.%s\": [%zu, %zu], ", #T, #f, offsetof(T, f), sizeof(((T*)0)->f))
#define SIZE(T) printf("\"sizeof %s\": %zu, ", #T, sizeof(T))
#define CONST(c) printf("\"%s\": %lld, ", #c, (long long)(c))

int main(void) {
  printf("{");
  SIZE(attn_mask_desc);
  FIELD(attn_mask_desc, flags); FIELD(attn_mask_desc, window_left);
  FIELD(attn_mask_desc, window_right); FIELD(attn_mask_desc, block_size);
  FIELD(attn_mask_desc, doc_offsets); FIELD(attn_mask_desc, num_docs);
  FIELD(attn_mask_desc, doc_stride);
  SIZE(attn_score_mod);
  FIELD(attn_score_mod, flags); FIELD(attn_score_mod, slopes); FIELD(attn_score_mod, rel_bias);
  FIELD(attn_score_mod, rel_radius); FIELD(attn_score_mod, softcap);
  SIZE(attn_blockmask);
  FIELD(attn_blockmask, Bm); FIELD(attn_blockmask, Hm); FIELD(attn_blockmask, nQt);
  FIELD(attn_blockmask, nKt); FIELD(attn_blockmask, part_num); FIELD(attn_blockmask, part_idx);
  FIELD(attn_blockmask, full_num); FIELD(attn_blockmask, full_idx);
  SIZE(attn_auto_plan);
  FIELD(attn_auto_plan, path); FIELD(attn_auto_plan, num_splits);
  FIELD(attn_auto_plan, workspace_bytes);

  CONST(ATTN_DTYPE_BF16); CONST(ATTN_DTYPE_F16);
  CONST(ATTN_MASK_CAUSAL); CONST(ATTN_MASK_WINDOW); CONST(ATTN_MASK_DOCUMENT);
  CONST(ATTN_MASK_BLOCK_CAUSAL);
  CONST(ATTN_SCHED_NO_PAIRING); CONST(ATTN_SCHED_NO_XCD_REMAP); CONST(ATTN_SCHED_REVERSE);
  CONST(ATTN_SCORE_ALIBI); CONST(ATTN_SCORE_ALIBI_SYM); CONST(ATTN_SCORE_REL_BIAS);
  CONST(ATTN_SCORE_SOFTCAP);
  CONST(ATTN_BLOCKMASK_TILE); CONST(ATTN_PATH_PREFILL); CONST(ATTN_PATH_SPLITKV);
  CONST(ATTN_ERR_NULL); CONST(ATTN_ERR_HEAD_DIM);

  /* calls that return before any launch */
  const int64_t st[3] = {0, 0, 0};
  printf("\"fwd_null\": %d, ",
         attn_fwd(NULL, st, NULL, st, NULL, st, NULL, st, NULL, 1, 1, 1, 1, 1, 64, ATTN_DTYPE_BF16,
                  0.125f, NULL, NULL, NULL));
  attn_auto_plan plan;
  const int rc = attn_fwd_auto_plan(16, 32, 8, 16, 32768, 128, NULL, &plan);
  printf("\"plan\": [%d, %d, %d, %llu], ", rc, (int)plan.path, (int)plan.num_splits,
         (unsigned long long)plan.workspace_bytes);
  printf("\"bwd_ws\": %zu, ", attn_bwd_workspace_bytes(2, 16, 4096));
  printf("\"bm_bytes\": %zu, ", attn_blockmask_bytes(1, 1, 256, 256));
  printf("\"noalloc_max\": %zu, ", attn_decode_noalloc_max_bytes());
  printf("\"status_head_dim\": \"%s\"", attn_status_str(ATTN_ERR_HEAD_DIM));
  printf("}\n");
  return 0;
}
