/* A plain C11 client of include/forkkv.h: the fork bookkeeping and the decode plan through
 * the C ABI alone (no device memory, no GPU).  It replays a fixed script and prints what the
 * library reports; tests/test_abi_client.py compiles it, runs it and checks the output
 * against the pool model and the Python binding.
 *
 * Script: a base-only root of 45 rows; a0 forks all 45 (unaligned: the tail is packed) and
 * appends 10; a1 forks the first 32 (aligned) and appends 20; a2 forks a1's first 40 rows
 * (unaligned, inside a1's private page) and appends 3.
 *
 * Output lines: "seq NAME LEN b0 .. b7 r0 .. r7" (tables, 8 pages), "cow SRC DST N" (every
 * copy-on-write row copy reported, in order), "plan ITEMS SLOTS BLOB_INTS", "blob i0 i1 ..",
 * "err CASE CODE" (calls that must fail before any device work, with the code returned),
 * then "ok".  Any failing call prints "fail NAME CODE" and exits with 1. */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "forkkv.h"

#define CHECK(call)                                                   \
  do {                                                                \
    int rc_ = (call);                                                 \
    if (rc_ != FORKKV_OK) {                                           \
      printf("fail %s %d (%s)\n", #call, rc_, forkkv_strerror(rc_)); \
      return 1;                                                       \
    }                                                                 \
  } while (0)

static void print_cow(const forkkv_cow_op* c) {
  if (c->n_rows > 0) printf("cow %d %d %d\n", c->src_bpage, c->dst_bpage, c->n_rows);
}

int main(void) {
  enum { MAXP = 8 };
  forkkv_pool_desc d = {64, 64, 16, 2, 64, 8, FORKKV_DTYPE_F32, NULL, NULL};
  forkkv_pool* pool = NULL;
  CHECK(forkkv_pool_create(&d, NULL, NULL, &pool));

  forkkv_seq root, a[3];
  forkkv_cow_op cow;
  CHECK(forkkv_seq_create(pool, 0, &root));
  CHECK(forkkv_seq_append(pool, root, 45, NULL, NULL, &cow));
  print_cow(&cow);
  CHECK(forkkv_fork(pool, root, 45, &a[0], &cow));
  print_cow(&cow);
  CHECK(forkkv_seq_append(pool, a[0], 10, NULL, NULL, &cow));
  print_cow(&cow);
  CHECK(forkkv_fork(pool, root, 32, &a[1], &cow));
  print_cow(&cow);
  CHECK(forkkv_seq_append(pool, a[1], 20, NULL, NULL, &cow));
  print_cow(&cow);
  CHECK(forkkv_fork(pool, a[1], 40, &a[2], &cow));
  print_cow(&cow);
  CHECK(forkkv_seq_append(pool, a[2], 3, NULL, NULL, &cow));
  print_cow(&cow);

  int32_t btab[3 * MAXP], rtab[3 * MAXP], lens[3];
  CHECK(forkkv_export_tables(pool, a, 3, MAXP, btab, rtab, lens));
  for (int i = 0; i < 3; ++i) {
    printf("seq a%d %d", i, lens[i]);
    for (int j = 0; j < MAXP; ++j) printf(" %d", btab[i * MAXP + j]);
    for (int j = 0; j < MAXP; ++j) printf(" %d", rtab[i * MAXP + j]);
    printf("\n");
  }

  forkkv_plan* plan = NULL;
  forkkv_plan_info info;
  CHECK(forkkv_plan_decode(pool, a, 3, 4, NULL, &plan));
  CHECK(forkkv_plan_get_info(plan, &info));
  const size_t n_ints = info.plan_bytes / sizeof(int32_t);
  printf("plan %d %d %zu\n", info.n_items, info.n_slots, n_ints);
  int32_t* blob = (int32_t*)malloc(info.plan_bytes);
  if (!blob) return 1;
  CHECK(forkkv_plan_export(plan, blob));
  printf("blob");
  for (size_t i = 0; i < n_ints; ++i) printf(" %d", blob[i]);
  printf("\n");
  free(blob);
  /* error paths that are decided before any device work */
  {
    forkkv_decode_args da;
    memset(&da, 0, sizeof da);
    printf("err decode_null %d\n", forkkv_residual_attn_decode(NULL, NULL));
    da.pool = pool;
    da.plan = plan;
    printf("err decode_no_storage %d\n", forkkv_residual_attn_decode(&da, NULL));
    forkkv_prefill_args pa;
    memset(&pa, 0, sizeof pa);
    printf("err prefill_null %d\n", forkkv_residual_attn_prefill(NULL, NULL));
    pa.pool = pool;
    pa.n_agents = 1;
    pa.chunk_len = 1;
    pa.num_q_heads = 4;
    printf("err prefill_no_storage %d\n", forkkv_residual_attn_prefill(&pa, NULL));
    printf("err upload_null %d\n", forkkv_plan_upload(plan, NULL, NULL));
    forkkv_plan* bad = NULL;
    printf("err plan_heads %d\n", forkkv_plan_decode(pool, a, 3, 3, NULL, &bad));
    forkkv_seq c2;
    printf("err fork_past_end %d\n", forkkv_fork(pool, a[2], 1000, &c2, &cow));
    forkkv_pool_desc d8 = d;
    forkkv_pool* p8 = NULL;
    d8.page_size = 8;
    printf("err page_size %d\n", forkkv_pool_create(&d8, NULL, NULL, &p8));
  }
  CHECK(forkkv_plan_destroy(plan));
  for (int i = 0; i < 3; ++i) CHECK(forkkv_seq_free(pool, a[i]));
  printf("err append_freed %d\n", forkkv_seq_append(pool, a[0], 1, NULL, NULL, &cow));
  CHECK(forkkv_seq_free(pool, root));
  forkkv_stats st;
  CHECK(forkkv_pool_stats(pool, &st));
  if (st.live_bpages != 0 || st.live_rpages != 0) {
    printf("fail leak %d %d\n", st.live_bpages, st.live_rpages);
    return 1;
  }
  CHECK(forkkv_pool_destroy(pool));
  printf("ok\n");
  return 0;
}
