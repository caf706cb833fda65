/* Randomized exercise of the host half of the C ABI (pool bookkeeping, forks, eviction and
 * refill, batched appends, decode plans and their rebuilds, table exports, error paths),
 * built with AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_sanitizers.py.
 * No device work: the pools have no device storage.  After every operation the pool's
 * counters must agree with its reference counts and free lists.  Prints "ok" at the end;
 * any sanitizer report or violated check ends the run with a nonzero status. */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "forkkv.h"

static unsigned long long g_state = 88172645463325252ull;
static unsigned rnd(unsigned n) { /* xorshift64, then reduce */
  g_state ^= g_state << 13;
  g_state ^= g_state >> 7;
  g_state ^= g_state << 17;
  return n ? (unsigned)(g_state % n) : 0u;
}

#define CHECK(cond)                                                    \
  do {                                                                 \
    if (!(cond)) {                                                     \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      exit(1);                                                         \
    }                                                                  \
  } while (0)

enum { NB = 96, NR = 160, MAXSEQ = 64, MAXPAGES = 64 };

static forkkv_seq g_seqs[MAXSEQ];
/* successful operations of each kind, printed at the end */
static long g_plans, g_rebuilds, g_forks, g_evictions, g_refills, g_batches;
static int g_has_res[MAXSEQ];
static int g_nseq = 0;

static void check_invariants(const forkkv_pool* pool) {
  forkkv_stats st;
  CHECK(forkkv_pool_stats(pool, &st) == FORKKV_OK);
  CHECK(st.live_bpages + st.free_bpages == NB);
  CHECK(st.live_rpages + st.free_rpages == NR);
  int32_t refb[NB], refr[NR], fl[NR], n = 0;
  CHECK(forkkv_refcounts(pool, 0, refb) == FORKKV_OK);
  CHECK(forkkv_refcounts(pool, 1, refr) == FORKKV_OK);
  long long sb = 0, sr = 0;
  int live_b = 0, live_r = 0;
  for (int i = 0; i < NB; ++i) {
    CHECK(refb[i] >= 0);
    sb += refb[i];
    live_b += refb[i] > 0;
  }
  for (int i = 0; i < NR; ++i) {
    CHECK(refr[i] >= 0);
    sr += refr[i];
    live_r += refr[i] > 0;
  }
  CHECK(sb == st.bpage_refs && sr == st.rpage_refs);
  CHECK(live_b == st.live_bpages && live_r == st.live_rpages);
  CHECK(forkkv_free_list(pool, 0, fl, NR, &n) == FORKKV_OK && n == st.free_bpages);
  for (int i = 0; i < n; ++i) CHECK(fl[i] >= 0 && fl[i] < NB && refb[fl[i]] == 0);
  CHECK(forkkv_free_list(pool, 1, fl, NR, &n) == FORKKV_OK && n == st.free_rpages);
  for (int i = 0; i < n; ++i) CHECK(fl[i] >= 0 && fl[i] < NR && refr[fl[i]] == 0);
}

static int pick_live(void) { return g_nseq ? (int)rnd((unsigned)g_nseq) : -1; }

static void remove_seq(int i) {
  g_seqs[i] = g_seqs[g_nseq - 1];
  g_has_res[i] = g_has_res[g_nseq - 1];
  --g_nseq;
}

static void exercise_plans(forkkv_pool* pool) {
  forkkv_seq batch[MAXSEQ];
  int nb = 0;
  for (int i = 0; i < g_nseq; ++i)
    if (g_has_res[i] && rnd(3)) batch[nb++] = g_seqs[i];
  forkkv_plan_opts o;
  memset(&o, 0, sizeof o);
  o.kernel = (int32_t)rnd(3);
  o.max_agents_per_item = (int32_t)rnd(4);
  o.pages_per_item = (int32_t)rnd(5);
  o.spare_items = (int32_t)rnd(3);
  forkkv_plan* plan = NULL;
  const int32_t heads = rnd(2) ? 8 : 4;
  const int rc = forkkv_plan_decode(pool, batch, nb, heads, &o, &plan);
  CHECK(rc == FORKKV_OK || rc == FORKKV_ESTATE || rc == FORKKV_EUNSUPPORTED);
  if (rc != FORKKV_OK) return;
  ++g_plans;
  forkkv_plan_info info;
  CHECK(forkkv_plan_get_info(plan, &info) == FORKKV_OK);
  CHECK(info.n_items <= info.item_capacity && info.n_slots <= info.slot_capacity);
  int32_t* blob = (int32_t*)malloc(info.plan_bytes);
  CHECK(blob != NULL);
  CHECK(forkkv_plan_export(plan, blob) == FORKKV_OK);
  CHECK(blob[1] == nb && blob[2] == info.n_items);
  free(blob);
  /* decode steps: reserve a token for the batch, rebuild when pages moved */
  for (int step = 0; step < 3 && nb > 0; ++step) {
    int32_t pages = 0;
    forkkv_cow_op cows[MAXSEQ];
    int32_t bs[MAXSEQ], rs[MAXSEQ];
    const int arc = forkkv_seq_append_batch(pool, batch, nb, 1, bs, rs, cows, &pages);
    CHECK(arc == FORKKV_OK || arc == FORKKV_ENOMEM || arc == FORKKV_ESTATE);
    if (arc != FORKKV_OK) break;
    int32_t same = -1;
    const int rrc = forkkv_plan_rebuild(plan, pool, batch, nb, &same);
    CHECK(rrc == FORKKV_OK || rrc == FORKKV_ESTATE);
    CHECK(rrc != FORKKV_OK || same == 0 || same == 1);
    g_rebuilds += rrc == FORKKV_OK;
    check_invariants(pool);
  }
  /* errors decided on the host */
  CHECK(forkkv_plan_rebuild(NULL, pool, batch, nb, NULL) == FORKKV_EINVAL);
  CHECK(forkkv_plan_upload(plan, NULL, NULL) == FORKKV_EINVAL);
  CHECK(forkkv_plan_set_timing(plan, 7) == FORKKV_EINVAL);
  forkkv_decode_args da;
  memset(&da, 0, sizeof da);
  da.pool = pool;
  da.plan = plan;
  {
    const int drc = forkkv_residual_attn_decode(&da, NULL);
    CHECK(drc == FORKKV_ESTATE || drc == FORKKV_EINVAL || drc == FORKKV_OK);
  }
  CHECK(forkkv_plan_destroy(plan) == FORKKV_OK);
}

int main(int argc, char** argv) {
  const int scripts = argc > 1 ? atoi(argv[1]) : 200;
  for (int sc = 0; sc < scripts; ++sc) {
    int32_t border[NB], rorder[NR];
    for (int i = 0; i < NB; ++i) border[i] = i;
    for (int i = 0; i < NR; ++i) rorder[i] = i;
    for (int i = NB - 1; i > 0; --i) {
      const int j = (int)rnd((unsigned)i + 1);
      const int32_t t = border[i];
      border[i] = border[j];
      border[j] = t;
    }
    forkkv_pool_desc d;
    memset(&d, 0, sizeof d);
    d.num_bpages = NB;
    d.num_rpages = NR;
    d.page_size = 16;
    d.num_kv_heads = 2;
    d.head_dim = 128;
    d.rank = 16;
    d.dtype = FORKKV_DTYPE_BF16;
    d.bpage_order = border;
    d.rpage_order = rorder;
    forkkv_pool* pool = NULL;
    CHECK(forkkv_pool_create(&d, NULL, NULL, &pool) == FORKKV_OK);
    g_nseq = 0;
    for (int op = 0; op < 120; ++op) {
      const unsigned what = rnd(11);
      const int i = pick_live();
      forkkv_cow_op cow;
      if (what == 0 || g_nseq == 0) { /* create */
        if (g_nseq == MAXSEQ) continue;
        forkkv_seq s;
        const int res = (int)rnd(2);
        CHECK(forkkv_seq_create(pool, res, &s) == FORKKV_OK);
        g_seqs[g_nseq] = s;
        g_has_res[g_nseq++] = res;
      } else if (what <= 2) { /* append */
        const int rc = forkkv_seq_append(pool, g_seqs[i], (int32_t)rnd(40), NULL, NULL, &cow);
        CHECK(rc == FORKKV_OK || rc == FORKKV_ENOMEM || rc == FORKKV_ESTATE);
      } else if (what <= 4) { /* fork */
        if (g_nseq == MAXSEQ) continue;
        int32_t len = 0;
        CHECK(forkkv_seq_len(pool, g_seqs[i], &len) == FORKKV_OK);
        forkkv_seq c;
        const int32_t at = rnd(2) ? len : (int32_t)rnd((unsigned)len + 1);
        const int rc = forkkv_fork_ex(pool, g_seqs[i], at, (int32_t)rnd(3), (int32_t)rnd(20), &c,
                                      &cow);
        CHECK(rc == FORKKV_OK || rc == FORKKV_ENOMEM || rc == FORKKV_ESTATE ||
              rc == FORKKV_EINVAL);
        if (rc == FORKKV_OK) {
          ++g_forks;
          g_seqs[g_nseq] = c;
          g_has_res[g_nseq++] = 1;
        }
      } else if (what == 5) { /* free */
        CHECK(forkkv_seq_free(pool, g_seqs[i]) == FORKKV_OK);
        CHECK(forkkv_seq_free(pool, g_seqs[i]) == FORKKV_EINVAL);
        remove_seq(i);
      } else if (what == 6) { /* evict one base page of a sequence */
        int32_t bt[MAXPAGES], rt[MAXPAGES], n = 0;
        if (forkkv_seq_pages(pool, g_seqs[i], &n) != FORKKV_OK || n == 0 || n > MAXPAGES) continue;
        CHECK(forkkv_export_tables(pool, &g_seqs[i], 1, MAXPAGES, bt, rt, NULL) == FORKKV_OK);
        const int32_t lp = (int32_t)rnd((unsigned)n);
        if (bt[lp] >= 0) {
          CHECK(forkkv_evict_bpages(pool, &bt[lp], 1) == FORKKV_OK);
          ++g_evictions;
        }
      } else if (what == 7) { /* refill the first gap of a sequence, for it alone */
        int32_t bt[MAXPAGES], rt[MAXPAGES], n = 0, got[1];
        if (forkkv_seq_pages(pool, g_seqs[i], &n) != FORKKV_OK || n == 0 || n > MAXPAGES) continue;
        CHECK(forkkv_export_tables(pool, &g_seqs[i], 1, MAXPAGES, bt, rt, NULL) == FORKKV_OK);
        for (int32_t lp = 0; lp < n; ++lp)
          if (bt[lp] < 0) {
            const int rc = forkkv_refill_bpages(pool, &g_seqs[i], 1, lp, lp + 1, got);
            CHECK(rc == FORKKV_OK || rc == FORKKV_ENOMEM || rc == FORKKV_EINVAL);
            g_refills += rc == FORKKV_OK;
            break;
          }
      } else if (what == 8) { /* batched append over a few distinct sequences */
        forkkv_seq batch[4];
        int nb = 0;
        for (int k = 0; k < g_nseq && nb < 4; ++k)
          if (rnd(2)) batch[nb++] = g_seqs[k];
        forkkv_cow_op cows[4];
        int32_t bs[4 * 20], rs[4 * 20], pages = 0;
        const int32_t rows = (int32_t)rnd(20);
        const int rc = forkkv_seq_append_batch(pool, batch, nb, rows, bs, rs, cows, &pages);
        CHECK(rc == FORKKV_OK || rc == FORKKV_ENOMEM || rc == FORKKV_ESTATE);
        g_batches += rc == FORKKV_OK;
      } else if (what == 9) { /* exports */
        int32_t bt[4 * MAXPAGES], rt[4 * MAXPAGES], lens[4], st[4 * MAXPAGES], al = 0;
        int nb = 0;
        forkkv_seq batch[4];
        for (int k = 0; k < g_nseq && nb < 4; ++k) batch[nb++] = g_seqs[k];
        int rc = forkkv_export_tables(pool, batch, nb, MAXPAGES, bt, rt, lens);
        CHECK(rc == FORKKV_OK || rc == FORKKV_EINVAL);
        rc = forkkv_export_starts(pool, batch, nb, MAXPAGES, st, &al);
        CHECK(rc == FORKKV_OK || rc == FORKKV_EINVAL);
        rc = forkkv_export_tables(pool, batch, nb, 0, bt, rt, lens);
        CHECK(rc == FORKKV_OK || rc == FORKKV_EINVAL);
      } else { /* decode plans, steps, rebuilds */
        exercise_plans(pool);
      }
      check_invariants(pool);
    }
    /* error paths on handles that do not exist */
    CHECK(forkkv_seq_append(pool, 12345, 1, NULL, NULL, NULL) == FORKKV_EINVAL);
    CHECK(forkkv_seq_append(pool, -1, 1, NULL, NULL, NULL) == FORKKV_EINVAL);
    CHECK(forkkv_fork(pool, 12345, 0, NULL, NULL) == FORKKV_EINVAL);
    CHECK(forkkv_evict_bpages(pool, NULL, 1) == FORKKV_EINVAL);
    while (g_nseq) {
      CHECK(forkkv_seq_free(pool, g_seqs[0]) == FORKKV_OK);
      remove_seq(0);
    }
    forkkv_stats st;
    CHECK(forkkv_pool_stats(pool, &st) == FORKKV_OK);
    CHECK(st.live_bpages == 0 && st.live_rpages == 0);
    CHECK(forkkv_pool_destroy(pool) == FORKKV_OK);
  }
  printf("plans=%ld rebuilds=%ld forks=%ld evictions=%ld refills=%ld batches=%ld\n", g_plans,
         g_rebuilds, g_forks, g_evictions, g_refills, g_batches);
  printf("ok\n");
  return 0;
}
