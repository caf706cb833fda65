/*
 * forkkv.h -- C ABI of the ResidualAttention library for AMD MI355X (gfx950).
 *
 * What the library computes
 * -------------------------
 * Many LoRA agents that share a long prefix share ONE base KV cache ("bCache":
 * the base projections xW_k after RoPE and xW_v), aliased page by page through
 * copy-on-write forks, and each agent keeps a private rank-r residual cache
 * ("rCache": xA_k and xA_v, no RoPE).  For agent a with up-projections B_k,a and
 * B_v,a (ForkKV study note, "2. Q1 / Q2 / Q3" Q2; "4. 作者证明", the
 * "Reconstruction" and "Attention fusion" equations):
 *
 *   K_a[t] = bK[t] + RoPE_t( s * rK_a[t] * B_k,a )          (deferred RoPE)
 *   V_a[t] = bV[t] + s * rV_a[t] * B_v,a
 *   o      = softmax(sm_scale * q K_a^T) V_a
 *          = [ sum_t p_t bV[t] + s * (sum_t p_t rV_a[t]) B_v,a ] / sum_t p_t
 *
 * The second form (associativity, the note's Eq.(4)) is what the kernels use:
 * B_v is applied once, after the online softmax.  RoPE is the rotate-half form
 * (dimension j paired with j + d/2, angle t * theta^(-2j/d)); query head g
 * reads KV head g / (Hq/Hkv).
 *
 * Storage (caller-owned device memory; the pages leave the layout open)
 * -----------------------------------------------------------------------
 *   bcache: [num_bpages][2][Hkv][P*d] elements: plane 0 = post-RoPE keys,
 *           plane 1 = values, one P x d tile per (page, plane, KV head).
 *   rcache: [num_rpages][2][P*r] elements: plane 0 = key residual, plane 1 =
 *           value residual, one P x r tile per (page, plane).
 *   Inside a tile the elements are in the order the gfx950 matrix cores consume
 *   them, so that every lane's MFMA operand is one contiguous 16- or 8-byte piece
 *   (row t = position within the page, x = dimension, k = rank):
 *     key            (t, x): (x / 8) * 128 + t * 8 + x % 8
 *     value          (t, x): ((x / 16) * 4 + t / 4) * 64 + (x % 16) * 4 + t % 4
 *     key residual   (t, k): (k / 4) * 64 + t * 4 + k % 4
 *     value residual (t, k): (t / 4) * (4 * r) + k * 4 + t % 4
 *   Element type: FORKKV_DTYPE_BF16 (bfloat16) or FORKKV_DTYPE_F32.  P = 16,
 *   d a multiple of 16 (<= 256), r a multiple of 4 (<= 64).
 *   A slot is page * P + row.  Position t of a sequence lives in page
 *   table[t / P], row t % P -- unless a frozen tail (see forkkv_fork_ex) sits in
 *   its history: then logical page j holds the rows from its start position
 *   pstart[j] (forkkv_export_starts) up to the next page's start, and the kernels
 *   take the start table as an extra argument.
 *
 * Fork bookkeeping (host side, bit-exact deterministic)
 * -----------------------------------------------------
 * ForkKV note "3. 架构 / 方法图" (Figure 6): a forked agent maps the parent's
 * read-only base pages (Step 1) and gets its own residual pages (Step 2).
 * ForkServe README "Design vs APC" / "Methods": fork aliases the parent's frames
 * in O(pages); a write allocates private pages only; an unaligned trunk tail is
 * packed into a private page by copying its n_valid rows; "Status": a freed
 * parent does not drop the trunk (every base page is reference counted).
 * Free lists are FIFO queues seeded with the pool's page order; allocation takes
 * from the head, release appends to the tail (base pages, then residual pages,
 * each in table order).  Sequence handles are 0, 1, 2, ... and never reused.
 * Every call is all-or-nothing: on an error nothing changes.
 *
 * Conventions
 * -----------
 * All functions return FORKKV_OK (0) or a negative error code; no exception
 * crosses the ABI.  "host" pointers are CPU memory, "device" pointers are HIP
 * device memory.  Arguments are validated before any launch; launches are
 * asynchronous on the given stream and the caller keeps every buffer alive until
 * the stream has finished.  A pool or plan handle must not be used from two
 * threads at once.  Device buffers of elements (pools, q, B_k, B_v, new rows,
 * outputs, workspaces) start on a 16-byte boundary (hipMalloc and PyTorch
 * allocations do); calls given another address return FORKKV_EINVAL.  Integer
 * tables (block tables, start tables, positions) need only their natural alignment.
 */
#ifndef FORKKV_H
#define FORKKV_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  FORKKV_OK = 0,
  FORKKV_EINVAL = -1,      /* bad argument or handle */
  FORKKV_ENOMEM = -2,      /* page pool exhausted (state unchanged) */
  FORKKV_EHIP = -3,        /* a HIP call or kernel launch failed */
  FORKKV_ESTATE = -4,      /* call not valid in the current state (e.g. plan not uploaded) */
  FORKKV_EUNSUPPORTED = -5, /* shape or dtype outside what the kernels implement */
  FORKKV_ETOOBIG = -6       /* plan's workspace exceeds the static scratch (no-alloc decode) */
};

enum { FORKKV_DTYPE_F32 = 0, FORKKV_DTYPE_BF16 = 1 };

/* Treatment of an unaligned tail at a fork (forkkv_fork_ex). */
enum { FORKKV_FORK_PACK = 0, FORKKV_FORK_FREEZE = 1, FORKKV_FORK_AUTO = 2 };

/* Decode kernel selection (forkkv_plan_opts.kernel). */
enum { FORKKV_KERNEL_AUTO = 0, FORKKV_KERNEL_GENERIC = 1, FORKKV_KERNEL_MFMA = 2 };

typedef struct forkkv_pool forkkv_pool;
typedef struct forkkv_plan forkkv_plan;
typedef int32_t forkkv_seq;

typedef struct {
  int32_t num_bpages;   /* pages in the base pool */
  int32_t num_rpages;   /* pages in the residual pool */
  int32_t page_size;    /* P; must be 16 */
  int32_t num_kv_heads; /* Hkv */
  int32_t head_dim;     /* d; multiple of 16, 16..256 */
  int32_t rank;         /* r; multiple of 4, 4..64 */
  int32_t dtype;        /* FORKKV_DTYPE_* */
  const int32_t* bpage_order; /* host, nullable: initial base free-list order, a permutation */
  const int32_t* rpage_order; /* host, nullable: initial residual free-list order */
} forkkv_pool_desc;

/* A copy of the first n_rows rows of base page src into base page dst (all KV heads, K and V). */
typedef struct {
  int32_t src_bpage;
  int32_t dst_bpage;
  int32_t n_rows; /* 0 = no copy needed */
} forkkv_cow_op;

typedef struct {
  int32_t live_bpages, live_rpages;
  int32_t free_bpages, free_rpages;
  int32_t shared_bpages;           /* base pages with reference count > 1 */
  int64_t bpage_refs, rpage_refs;  /* sums of reference counts */
  int64_t live_bytes_b, live_bytes_r;
} forkkv_stats;

/* Human-readable text of an error code (static storage). */
const char* forkkv_strerror(int code);

/* Bytes the caller must allocate for the two device pools of a descriptor. */
int forkkv_pool_bytes(const forkkv_pool_desc* desc, size_t* bcache_bytes, size_t* rcache_bytes);

/* Create the host bookkeeping of a pool.  bcache / rcache (device, nullable) are the
 * caller's pool buffers; with NULL the pool does bookkeeping only and device calls on
 * it return FORKKV_ESTATE.  The handle owns host metadata only. */
int forkkv_pool_create(const forkkv_pool_desc* desc, void* bcache, void* rcache,
                       forkkv_pool** out);
int forkkv_pool_destroy(forkkv_pool* pool);

/* New empty sequence; with_residual = 0 makes a base-only snapshot (no rCache pages). */
int forkkv_seq_create(forkkv_pool* pool, int32_t with_residual, forkkv_seq* out);

/* Reserve n rows at the end of seq.  bslots / rslots (host, nullable, n entries) receive
 * the slot of each new row (rslots = -1 for a base-only sequence).  cow (host, nullable)
 * receives the copy-on-write row copy the append needed (n_rows = 0 if none); the caller
 * runs it with forkkv_cow_copy before writing the new rows. */
int forkkv_seq_append(forkkv_pool* pool, forkkv_seq seq, int32_t n, int32_t* bslots,
                      int32_t* rslots, forkkv_cow_op* cow);

/* Fork a new agent sharing the parent's first alias_len rows (0 <= alias_len <= len).
 * Full base pages are aliased (reference count + 1); a partial tail is packed into a
 * private page (cow receives the row copy).  The child gets fresh residual pages for
 * [0, alias_len), which the caller fills. */
int forkkv_fork(forkkv_pool* pool, forkkv_seq parent, int32_t alias_len, forkkv_seq* child,
                forkkv_cow_op* cow);

/* Fork with a choice for the unaligned tail (ForkServe README, "Design vs APC": the
 * adaptive tail, pages_pack = k * ceil((r + l) / P) versus pages_freeze = 1 + k * ceil(l / P)).
 *   FORKKV_FORK_PACK   as forkkv_fork: the child copies the tail's rows into a private page.
 *   FORKKV_FORK_FREEZE the parent's partial last page becomes read-only for the parent and the
 *                      child (no copy); later rows of either go to fresh pages, so their pages
 *                      no longer start at multiples of P (the slot map, forkkv_export_starts).
 *                      Only at the parent's end (alias_len == len), else FORKKV_EINVAL.
 *   FORKKV_FORK_AUTO   pack when tail rows + suffix_hint <= P (the child's expected suffix
 *                      fits the tail page) or the cut is not at the parent's end, else freeze.
 * Whole pages below alias_len -- full pages and frozen tails -- are aliased as by forkkv_fork.
 * Errors: FORKKV_EINVAL (bad handle, alias_len, mode or suffix_hint < 0), FORKKV_ESTATE (an
 * aliased page was evicted), FORKKV_ENOMEM. */
int forkkv_fork_ex(forkkv_pool* pool, forkkv_seq parent, int32_t alias_len, int32_t mode,
                   int32_t suffix_hint, forkkv_seq* child, forkkv_cow_op* cow);

/* Reserve `rows` rows at the end of each of the n distinct sequences seqs (one decode step
 * of a batch: rows = 1), as forkkv_seq_append does for each in order, all or nothing (on
 * FORKKV_ENOMEM nothing changes).  bslots / rslots (host, nullable, n * rows) receive the
 * slots, agent-major; cows (host, nullable, n entries) the copy-on-write row copy of each
 * sequence (n_rows = 0 if none); *new_pages (nullable) the number of base pages the call
 * took from the free list -- nonzero means some agent entered a new page, after which a
 * decode plan over the batch needs forkkv_plan_rebuild. */
int forkkv_seq_append_batch(forkkv_pool* pool, const forkkv_seq* seqs, int32_t n, int32_t rows,
                            int32_t* bslots, int32_t* rslots, forkkv_cow_op* cows,
                            int32_t* new_pages);

/* Release a sequence: each page's reference count drops; pages reaching 0 return to the
 * tail of their free list. */
int forkkv_seq_free(forkkv_pool* pool, forkkv_seq seq);
int forkkv_seq_len(const forkkv_pool* pool, forkkv_seq seq, int32_t* len);
/* Number of logical pages of seq (ceil(len / P), plus one per frozen tail it holds). */
int forkkv_seq_pages(const forkkv_pool* pool, forkkv_seq seq, int32_t* n_pages);

/* Block tables of n sequences (host outputs): btab, rtab [n][max_pages] page ids padded
 * with -1 (rtab all -1 for base-only sequences); seq_lens [n] (nullable). */
int forkkv_export_tables(const forkkv_pool* pool, const forkkv_seq* seqs, int32_t n,
                         int32_t max_pages, int32_t* btab, int32_t* rtab, int32_t* seq_lens);

/* Start position of each logical page of n sequences (host output pstart [n][max_pages],
 * -1 padded): page j holds rows pstart[j] .. pstart[j+1]-1 (the last page up to len-1).
 * *aligned (host, nullable) = 1 when every page starts at j * P (no frozen tail), in which
 * case the kernels need no start table. */
int forkkv_export_starts(const forkkv_pool* pool, const forkkv_seq* seqs, int32_t n,
                         int32_t max_pages, int32_t* pstart, int32_t* aligned);

/* Decoupled eviction (ForkKV study note, "Error / eviction recovery"; implementation detail
 * 1): evict base pages (host pages[n], distinct, live) from every sequence that maps them.
 * Their table entries become -1 and they return to the tail of the base free list in the
 * order given; residual pages are untouched (the rCache survives).  A sequence with a
 * missing base page is a partial hit: appends, forks over the gap and decode plans return
 * FORKKV_ESTATE until it is refilled.  Errors: FORKKV_EINVAL. */
int forkkv_evict_bpages(forkkv_pool* pool, const int32_t* pages, int32_t n);

/* Partial-hit refill: map fresh base pages into logical pages [lp0, lp1) of the n listed
 * sequences (host seqs[n], distinct), each of which must miss exactly those pages and agree
 * on their start positions and row counts.  One page per logical page is shared by all of
 * them (reference count n); new_pages (host, nullable, lp1 - lp0 entries) receives them.
 * The caller then stores the recomputed base rows (post-RoPE xW_k and xW_v) there, e.g. with
 * forkkv_write_rows without residual rows.  Errors: FORKKV_EINVAL, FORKKV_ENOMEM. */
int forkkv_refill_bpages(forkkv_pool* pool, const forkkv_seq* seqs, int32_t n, int32_t lp0,
                         int32_t lp1, int32_t* new_pages);

int forkkv_pool_stats(const forkkv_pool* pool, forkkv_stats* out);

/* Free-list contents in queue order (which = 0 base, 1 residual); host out[cap]; *n = size. */
int forkkv_free_list(const forkkv_pool* pool, int32_t which, int32_t* out, int32_t cap,
                     int32_t* n);

/* Reference counts of every page (which = 0 base, 1 residual); host out[num pages]. */
int forkkv_refcounts(const forkkv_pool* pool, int32_t which, int32_t* out);

/* Run copy-on-write row copies on the device pool (ForkServe README "Status": n_valid
 * rows, not P).  Needs the pool's device buffers. */
int forkkv_cow_copy(forkkv_pool* pool, const forkkv_cow_op* ops, int32_t n_ops,
                    hipStream_t stream);

/* ---------------------------------------------------------------------------------
 * Decode plan.  Groups (logical page, physical base page) entries that several agents
 * alias into work items, so that each shared base page is read once for all its
 * agents, and cuts long runs into split-K items whose partial softmax states are
 * merged afterwards.  Integer only, deterministic; built on the host from the pool's
 * tables and lengths, which it captures.
 * --------------------------------------------------------------------------------- */
typedef struct {
  int32_t kernel;             /* FORKKV_KERNEL_*; 0 = auto */
  int32_t max_agents_per_item;/* 0 = the kernel's maximum */
  int32_t pages_per_item;     /* split-K length: pages per item (generic kernel) or pages per
                                 wave (MFMA kernel, <= 64); 0 = auto (MFMA: items sized so the
                                 grid fits one round of resident waves, balanced per wave) */
  int32_t spare_items;        /* room for items beyond the first build's, so rebuilds after
                                 page crossings keep the launch; 0 = one per agent */
} forkkv_plan_opts;

typedef struct {
  int32_t n_agents, n_items, n_slots, kernel, item_ints, num_q_heads;
  size_t plan_bytes;      /* device bytes forkkv_plan_upload needs */
  size_t workspace_bytes; /* device workspace forkkv_residual_attn_decode needs */
  int32_t item_capacity;  /* items the decode launch covers (>= n_items; only grows) */
  int32_t slot_capacity;  /* split-K partial slots the workspace holds (>= n_slots) */
} forkkv_plan_info;

/* Build the decode plan of the n sequences seqs (agent a = seqs[a]) for num_q_heads
 * query heads.  opts is nullable.  Kernel coverage: the MFMA kernel takes bf16, d = 128,
 * r = 16 and up to 16 query heads per KV head; the generic kernel every pool shape whose
 * group G = num_q_heads / Hkv has G * d <= 8192 and G * r <= 2048 (its LDS plan may use up
 * to 160 KiB); other shapes return FORKKV_EUNSUPPORTED, as does prefill for them.
 * The plan captures each agent's length and last page; the lengths also live in its
 * device copy, where decode with append advances them (see below). */
int forkkv_plan_decode(const forkkv_pool* pool, const forkkv_seq* seqs, int32_t n,
                       int32_t num_q_heads, const forkkv_plan_opts* opts, forkkv_plan** out);
/* Rebuild a plan in place from the pool's current state (same options), e.g. after a
 * decode step with append took an agent into a new page or a copy-on-write.  Capacities
 * only grow: *same_launch (nullable) is 1 when the batch size, item capacity, slot
 * capacity and kernel are unchanged, so that -- after forkkv_plan_upload to the same device
 * buffer, which must hold plan_bytes -- a decode launch captured before (a HIP graph) stays
 * valid; 0 when the caller must check plan_bytes / workspace_bytes and launch anew.  On an
 * error the plan is unchanged.  The device copy is stale until the next upload. */
int forkkv_plan_rebuild(forkkv_plan* plan, const forkkv_pool* pool, const forkkv_seq* seqs,
                        int32_t n, int32_t* same_launch);
int forkkv_plan_get_info(const forkkv_plan* plan, forkkv_plan_info* out);
/* Copy the plan's integer blob (plan_bytes / 4 int32) to host memory, for inspection. */
int forkkv_plan_export(const forkkv_plan* plan, int32_t* host_blob);
/* Copy the plan blob to a caller-owned device buffer of plan_bytes, asynchronously on
 * stream (from one of two pinned staging buffers the plan owns; the call waits only for the
 * copy made two uploads earlier from the same buffer).  The plan remembers the buffer.
 * Order the upload before the decode calls that use it (same stream, or an event).  Not
 * for use inside a stream capture. */
int forkkv_plan_upload(forkkv_plan* plan, void* dev_buf, hipStream_t stream);
int forkkv_plan_destroy(forkkv_plan* plan);

/* Per-kernel timing.
 *   FORKKV_TIMING_OFF (0): no timing.
 *   FORKKV_TIMING_EVENTS (1): HIP events recorded on the launch stream around each launch of
 *     the plan's split kernel and combine kernel; forkkv_plan_timing waits for them and
 *     returns the summed milliseconds and the number of timed launches, then clears the sums.
 *   FORKKV_TIMING_SPLIT_ONLY (2): measurement only -- decode calls with this plan launch the
 *     split-K kernel alone (no combine, the output is not written, no events), so that a
 *     caller can time the split kernel from replays of a captured graph of such calls, the
 *     same way it times whole decode calls.
 * Other values return FORKKV_EINVAL. */
enum { FORKKV_TIMING_OFF = 0, FORKKV_TIMING_EVENTS = 1, FORKKV_TIMING_SPLIT_ONLY = 2 };
int forkkv_plan_set_timing(forkkv_plan* plan, int32_t enable);
int forkkv_plan_timing(forkkv_plan* plan, double* split_ms, double* combine_ms,
                       int32_t* launches);

/* ---------------------------------------------------------------------------------
 * Decode: one query per agent over its cached keys 0 .. len-1 (len captured by the
 * plan).  ForkKV note "7. 实现 cross-reference" (kernel; core barriers (1) deferred
 * RoPE and (2) B_v lifted out of the loop with a rescaled residual accumulator).
 * --------------------------------------------------------------------------------- */
typedef struct {
  const forkkv_pool* pool;  /* geometry, dtype and device pools */
  const forkkv_plan* plan;  /* built for this batch and uploaded */
  const void* q;            /* device [N][Hq][d], post-RoPE, pool dtype */
  const void* Bk;           /* device [N][r][Hkv*d], pool dtype */
  const void* Bv;           /* device [N][r][Hkv*d], pool dtype */
  const int32_t* btab;      /* device [N][max_pages], as exported from the pool */
  const int32_t* rtab;      /* device [N][max_pages] */
  int32_t max_pages;        /* row stride of btab / rtab */
  float lora_scale;         /* s */
  float sm_scale;           /* softmax scale > 0, e.g. 1/sqrt(d) */
  float rope_theta;         /* theta */
  void* out;                /* device [N][Hq][d], pool dtype; an agent with len 0 gets 0 */
  void* workspace;          /* device, workspace_bytes of the plan */
  size_t workspace_bytes;
  const int32_t* pstart;    /* device [N][max_pages] page start positions (forkkv_export_starts);
                               nullable when every page starts at a multiple of P.  Required
                               when a batch sequence holds a frozen tail (ForkServe README,
                               "Design vs APC": the fork-aware slot map) */
} forkkv_decode_args;

/* Page ids are read from btab / rtab at launch; the plan fixes only which agents share
 * which logical pages.  The plan refuses missing base pages, but an entry changed after
 * the build to -1 or to an id outside its pool is taken as a missing page (the rule under
 * "Missing pages" below); for a base page that several batch sequences share, the change
 * must be made in every holder's row.
 *
 * Errors: FORKKV_EINVAL (null pointers, a plan of another geometry, max_pages below the
 * plan's, a small workspace, non-finite scales, sm_scale <= 0, theta <= 0, no pstart
 * for a plan over a frozen tail);
 * FORKKV_ESTATE (pool without device storage, plan not uploaded); FORKKV_EHIP. */
int forkkv_residual_attn_decode(const forkkv_decode_args* args, hipStream_t stream);

/* ---------------------------------------------------------------------------------
 * Decode without allocation, for callers that cannot call hipMalloc or bring a device
 * workspace (code under HIP stream capture, tight serving loops, harnesses that forbid
 * allocation).  Same computation, kernels and output as forkkv_residual_attn_decode; the
 * split-K workspace is instead a static device array of the library, one per GPU, of
 * FORKKV_NOALLOC_SCRATCH_BYTES (32 MiB: the MFMA plans of the Llama3-8B and Qwen2.5-14B
 * decode workloads need 3.2, 7.8 and 20.7 MiB), held until the process ends.
 *   args->workspace and args->workspace_bytes are ignored (pass NULL / 0).
 *   No plan timing is recorded (forkkv_plan_set_timing is ignored by this call).
 *   The first call on a device resolves that device's array address (hipGetSymbolAddress,
 *   with the device current); no call allocates device or host memory.
 *   Nothing in the array needs clearing between calls: the split kernel writes every
 *   partial slot the combine reads.  All calls on one GPU share its array, so calls that
 *   overlap on one GPU (two streams, two threads) race and must be serialised by the
 *   caller; calls on one stream are ordered and safe.
 * Errors: as forkkv_residual_attn_decode, plus FORKKV_ETOOBIG when the plan's
 * workspace_bytes exceed FORKKV_NOALLOC_SCRATCH_BYTES (decided on the host, before any
 * device work).
 * --------------------------------------------------------------------------------- */
#define FORKKV_NOALLOC_SCRATCH_BYTES (32u << 20)
int forkkv_residual_attn_decode_noalloc(const forkkv_decode_args* args, hipStream_t stream);

/* ---------------------------------------------------------------------------------
 * Decode step with append: each agent's newest token is stored into the pools first, then
 * the agent's query attends to its keys 0 .. len-1, the new token included, where len is
 * the length in the plan's device copy.  Within one call the rows are written before any
 * attention reads them (Penelope review, 部件二: each layer writes the batch's K/V, then
 * attends).  After the call every device length has advanced by one, so the next call
 * appends at the following position with the same plan: a serving loop replays one call
 * (or one captured graph) step after step with no host work on the plan.
 *
 * Serving loop.  Before the first step the caller reserves the token with forkkv_seq_append
 * (or forkkv_seq_append_batch) and builds and uploads the plan, whose lengths then count it.
 * Each later step it reserves the next token on the host the same way.  When a reservation
 * took an agent into a new page or needed a copy-on-write (ForkServe README, "Design vs
 * APC": a tail page shared after a fork is first packed into a private page, an
 * n_valid-row copy, not a whole page), the caller runs the copy (forkkv_cow_copy), brings
 * the device tables up to date, and calls forkkv_plan_rebuild and forkkv_plan_upload
 * before the step; otherwise nothing.  A token whose row would fall outside its agent's
 * last page (a crossing without a rebuild) is neither stored nor attended to.
 * --------------------------------------------------------------------------------- */
typedef struct {
  forkkv_decode_args decode; /* as for decode; every plan length counts the new token (>= 1)
                                and q is post-RoPE at position len - 1 */
  const void* k_new;         /* device [N][Hkv][d], post-RoPE base key of the new token */
  const void* v_new;         /* device [N][Hkv][d] */
  const void* rk_new;        /* device [N][r], key residual of the new token (no RoPE) */
  const void* rv_new;        /* device [N][r] */
} forkkv_decode_append_args;

/* Same errors as forkkv_residual_attn_decode; FORKKV_EINVAL also for a null row pointer or
 * a plan length below 1.  The new rows land at position len - 1 of each agent: row
 * (len - 1) - (start of its last page), in the pages the tables name for the plan's last
 * page of the agent.  A sequence appears at most once in the batch.  On the MFMA kernel the
 * split kernel stores the rows itself, ahead of the pages that hold them; the generic
 * kernel runs a row-write kernel first.  The combine kernel advances the lengths. */
int forkkv_residual_attn_decode_append(const forkkv_decode_append_args* args,
                                       hipStream_t stream);

/* ---------------------------------------------------------------------------------
 * Chunked prefill: agent a appends C rows at positions start_pos[a] .. start_pos[a]+C-1
 * (the caller has already reserved them with forkkv_seq_append and uploaded the tables).
 * The kernel first stores the chunk rows into the pools, then every chunk query
 * attends causally to keys 0 .. its own position (Penelope review, 部件二: each layer
 * writes the batch's K/V first, then attends).
 *
 * With a position list (positions != NULL) row i of agent a sits at positions[a][i]
 * instead: e.g. the rows of a hole inside the history, recomputed by a prefill-only
 * request, followed by the real request's new tail -- both keep their original positions
 * and run in one launch (Penelope review, 部件二, the phantom request).  All rows are
 * stored first; query i then attends to keys 0 .. positions[a][i], reading the rows just
 * stored.  Positions must strictly increase per agent and lie inside the tables; every
 * position must have been reserved (history rows of the hole, appended rows of the tail).
 * start_pos / start_pos_host are then ignored and may be NULL.
 * --------------------------------------------------------------------------------- */
typedef struct {
  const forkkv_pool* pool;
  int32_t n_agents;         /* N */
  int32_t chunk_len;        /* C >= 1 */
  int32_t num_q_heads;      /* Hq, a multiple of Hkv */
  const void* q;            /* device [N][C][Hq][d], post-RoPE */
  const void* k_new;        /* device [N][C][Hkv][d], post-RoPE base keys of the chunk */
  const void* v_new;        /* device [N][C][Hkv][d] */
  const void* rk_new;       /* device [N][C][r] */
  const void* rv_new;       /* device [N][C][r] */
  const void* Bk;           /* device [N][r][Hkv*d] */
  const void* Bv;           /* device [N][r][Hkv*d] */
  const int32_t* btab;      /* device [N][max_pages], covering start_pos + C */
  const int32_t* rtab;      /* device [N][max_pages] */
  int32_t max_pages;
  const int32_t* start_pos;      /* device [N] */
  const int32_t* start_pos_host; /* host [N], same values (validation and launch shape) */
  float lora_scale, sm_scale, rope_theta;  /* finite; sm_scale > 0, rope_theta > 0 */
  void* out;                /* device [N][C][Hq][d] */
  const int32_t* positions;      /* nullable: device [N][C], row positions (see above) */
  const int32_t* positions_host; /* host [N][C], same values; required with positions */
  const int32_t* pstart;         /* nullable: device [N][max_pages] page start positions, for
                                    sequences holding a frozen tail (the slot map) */
  int32_t kernel;                /* FORKKV_KERNEL_*: 0 = auto (the MFMA kernel where it covers
                                    the shape: bf16, d = 128, r = 16, G <= 16); GENERIC runs
                                    the generic kernel; MFMA returns FORKKV_EUNSUPPORTED for a
                                    shape it does not cover */
} forkkv_prefill_args;

/* Missing pages.  A base table entry of -1 (a page evicted with forkkv_evict_bpages and not
 * yet refilled) holds no keys: no query attends to its positions, and chunk rows that fall
 * on it are not stored.  A residual table entry of -1 (a sequence without residual pages,
 * such as a base-only snapshot) reads as zero residual rows (the key and value are the base
 * rows alone), and chunk residual rows that fall on it are not stored.  Both kernels follow
 * this rule, here and in decode.
 *
 * Errors: FORKKV_EINVAL for null pointers, C < 1, a head count that is not a multiple of
 * Hkv, rows outside the tables, positions that do not strictly increase, scales out of
 * range, or an unknown kernel;
 * FORKKV_EUNSUPPORTED for a shape no kernel covers (or the MFMA kernel asked for a shape
 * it does not cover); FORKKV_ESTATE when the pool has no device storage; FORKKV_EHIP when a
 * launch fails. */

int forkkv_residual_attn_prefill(const forkkv_prefill_args* args, hipStream_t stream);

/* ---------------------------------------------------------------------------------
 * Row write without attention: store rows into the pools at given positions, bit exact.
 * Used after a partial-hit refill (forkkv_refill_bpages; ForkKV study note, "Error /
 * eviction recovery": only the base projection xW is recomputed and re-inserted, the
 * surviving residual xA_i is reused) with rk_new = rv_new = NULL, which leaves the
 * residual pool untouched; with residual rows it is the row-store half of a prefill.
 * Row i of sequence a goes to position positions[a][i], in the page the tables (and the
 * slot map, if given) name for it.
 * --------------------------------------------------------------------------------- */
typedef struct {
  const forkkv_pool* pool;
  int32_t n_seqs;                /* N */
  int32_t n_rows;                /* R >= 1 rows per sequence */
  const int32_t* btab;           /* device [N][max_pages] */
  const int32_t* rtab;           /* device [N][max_pages]; may be NULL when rk_new is */
  const int32_t* pstart;         /* nullable: device [N][max_pages] page start positions */
  int32_t max_pages;
  const int32_t* positions;      /* device [N][R], strictly increasing per sequence */
  const int32_t* positions_host; /* host [N][R], same values (validation, launch shape) */
  const void* k_new;             /* device [N][R][Hkv][d], post-RoPE base keys */
  const void* v_new;             /* device [N][R][Hkv][d] */
  const void* rk_new;            /* nullable: device [N][R][r] (NULL together with rv_new) */
  const void* rv_new;
} forkkv_write_args;

/* Errors: FORKKV_EINVAL (null pointers, R < 1, positions not strictly increasing or outside
 * the tables, only one of rk_new / rv_new given); FORKKV_ESTATE (no device storage);
 * FORKKV_EHIP.  A row whose table entry is -1 (an evicted page) is not stored. */
int forkkv_write_rows(const forkkv_write_args* args, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* FORKKV_H */
