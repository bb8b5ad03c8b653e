/* A plain C99 program against include/mla_verify.h: the header must parse as
 * C and the library must link and answer from C. It prints the status of
 * mla_plan for one verify shape (batch 1, q_len 9, 8 heads, 65,545 positions),
 * the ABI version and the plan. No device is needed. */
#include "mla_verify.h"
#include <stdio.h>

int main(void) {
  mla_plan_t p;
  mla_q_t q = {0};
  mla_kv_t kv = {0};
  mla_mask_t m = {0};
  q.batch = 1;
  q.q_len = 9;
  q.heads = 8;
  q.sm_scale = 0.0721687836f;
  kv.dtype = MLA_KV_BF16;
  kv.pool_rows = 131090;
  kv.slot_stride = 65545;
  m.kind = MLA_MASK_CAUSAL;
  const int st = mla_plan(&q, &kv, &m, 0, &p);
  printf("%d %d %d %d %d %d %zu\n", st, mla_abi_version(), p.nsplit, p.row_blocks, p.row_groups, p.waves_per_group,
         p.workspace_bytes);
  printf("%s\n", mla_status_string(MLA_ERR_ALIGN));
  return st == MLA_OK ? 0 : 1;
}
