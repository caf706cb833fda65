// Internal declarations shared by the host library and the HIP kernels.
#pragma once

#include <cstddef>
#include <algorithm>
#include <cstdint>
#include <deque>
#include <vector>

#include <hip/hip_runtime_api.h>

#include "forkkv.h"

namespace forkkv {

constexpr int kPage = 16;

// One decode work item: a run of logical pages that every listed agent maps to the same
// physical base pages, processed by one workgroup per KV head.
//   [0] first logical page   [1] number of pages   [2] number of agents
//   [3] 1 if the item holds the last logical page of one of its agents (decode with append
//       stores that agent's new row there), else 0
//   [4 .. 4+kItemAgents) agent indices
//   [4+kItemAgents .. 4+2*kItemAgents) partial slot of each agent; the slots of one agent
//   are consecutive (slot_ptr[a] .. slot_ptr[a+1]), so the combine needs no slot list
constexpr int kItemAgents = 8;
constexpr int kItemInts = 4 + 2 * kItemAgents;

// Plan blob header (int32 words), followed by the sections at the given offsets.
enum : int {
  kHdrMagic = 0, kHdrAgents, kHdrItems, kHdrSlots, kHdrItemInts, kHdrQHeads,
  kHdrOffItems, kHdrOffLens, kHdrOffSlotPtr, kHdrOffSlotList, kHdrKernel, kHdrGroup,
  kHdrOffLastPage,   // per agent: its last logical page (-1 without rows)
  kHdrItemCapacity,  // items the launch grid covers (the items section has room for them)
  kHdrSlotCapacity,  // split-K slots the workspace holds
  kHdrWords = 16
};
constexpr int32_t kPlanMagic = 0x464b5631;  // "FKV1"

struct Seq {
  bool alive = true;
  bool has_res = false;
  bool closed = false;            // the last page takes no more rows (a frozen tail)
  int32_t len = 0;
  int32_t missing = 0;            // base table entries that are -1 (evicted, not refilled)
  std::vector<int32_t> bpages, rpages;
  std::vector<int32_t> starts;    // position of row 0 of each logical page (the slot map)

  // rows of logical page j that belong to this sequence
  int32_t rows(size_t j) const {
    const int32_t end = j + 1 < starts.size() ? starts[j + 1] : len;
    return end - starts[j];
  }
  // rows that still fit in the last page
  int32_t room() const {
    if (bpages.empty() || closed) return 0;
    return kPage - rows(bpages.size() - 1);
  }
  bool aligned() const {  // every page starts at a multiple of the page size
    for (size_t j = 0; j < starts.size(); ++j)
      if (starts[j] != static_cast<int32_t>(j) * kPage) return false;
    return true;
  }
  bool missing_base() const { return missing > 0; }
};

}  // namespace forkkv

struct forkkv_pool {
  forkkv_pool_desc desc{};
  void* bcache = nullptr;
  void* rcache = nullptr;
  std::deque<int32_t> free_b, free_r;
  std::vector<int32_t> ref_b, ref_r;
  std::vector<forkkv::Seq> seqs;
};

namespace forkkv {
// A maximal run of logical pages over which one set of agents maps the same physical page.
struct Run {
  std::vector<int32_t> agents;
  int32_t lp0, lp1;  // [lp0, lp1)
};
}  // namespace forkkv

struct forkkv_plan {
  forkkv_pool_desc geo{};   // geometry copy (orders cleared)
  void* bcache = nullptr;
  void* rcache = nullptr;
  forkkv_plan_opts opts{};  // the options it was built with (kept by rebuilds)
  int32_t n_agents = 0, n_items = 0, n_slots = 0, num_q_heads = 0, kernel = 0;
  int32_t item_capacity = 0, slot_capacity = 0;  // launch grid / workspace sizes (only grow)
  int32_t group = 0;        // agents per item the kernel was planned for
  bool aligned = true;      // every page of every agent starts at a multiple of P
  std::vector<int32_t> blob;
  void* dev = nullptr;      // caller's device copy
  size_t workspace_bytes = 0;
  size_t ws_off_acc = 0, ws_off_accr = 0;
  int32_t max_pages_needed = 0;
  int32_t max_agent_slots = 0;  // the largest number of partials of one agent
  // timing: (kind, begin, end) per timed launch, kind 0 = split, 1 = combine
  bool timing = false;       // FORKKV_TIMING_EVENTS
  bool split_only = false;   // FORKKV_TIMING_SPLIT_ONLY
  struct Timed { int kind; hipEvent_t b, e; };
  std::vector<Timed> pending;
  std::vector<hipEvent_t> spare;
  // what a rebuild can reuse: the batch, its base page tables and the runs found in them
  std::vector<int32_t> seq_ids;
  std::vector<std::vector<int32_t>> bpages_seen;
  std::vector<forkkv::Run> runs;
  // asynchronous upload: two pinned staging buffers, each with the event of its last copy
  void* staging[2] = {nullptr, nullptr};
  size_t staging_bytes[2] = {0, 0};
  hipEvent_t staged[2] = {nullptr, nullptr};
  int next_staging = 0;
};

namespace forkkv {

// Element offsets inside the pool tiles (P = 16): the order in which the gfx950 matrix
// cores consume them, so that each lane's MFMA operand is one contiguous 8- or 16-byte
// piece at lane * size (see include/forkkv.h, "Storage").
struct TileOrder {
  __host__ __device__ static constexpr int key(int t, int x) { return (x / 8) * 128 + t * 8 + x % 8; }
  __host__ __device__ static constexpr int value(int t, int x) {
    return ((x / 16) * 4 + t / 4) * 64 + (x % 16) * 4 + t % 4;
  }
  __host__ __device__ static constexpr int res_key(int t, int k) { return (k / 4) * 64 + t * 4 + k % 4; }
  __host__ __device__ static constexpr int res_value(int t, int k, int r) {
    return (t / 4) * (4 * r) + k * 4 + t % 4;
  }
};

// Launch parameters of the decode kernels (passed by value).
struct DecodeParams {
  const void* q;
  const void* Bk;
  const void* Bv;
  const void* bcache;
  const void* rcache;
  const int32_t* btab;
  const int32_t* rtab;
  const int32_t* plan;      // device blob
  const int32_t* pstart;    // nullable: [N][max_pages] start position of each page
  float* ws_ml;             // [slots][Hq][2]  (running max in log2 units, sum)
  float* ws_acc;            // [slots][Hq][d]
  float* ws_accr;           // [slots][Hq][r]
  void* out;
  // decode with append (MFMA kernel): each agent's new rows, stored by the workgroups of the
  // item holding its last row before any page is read; null for a plain decode
  const void* k_new;   // [N][Hkv][d]
  const void* v_new;   // [N][Hkv][d]
  const void* rk_new;  // [N][r]
  const void* rv_new;  // [N][r]
  // decode with append: the plan's device lengths, each advanced by one by the combine
  // kernel once the call has read them (the next call appends at the following position)
  int32_t* advance;
  // n_items is the launch's item capacity; the kernels read the live count from the plan
  int32_t n_agents, n_items, num_q_heads, num_kv_heads, head_dim, rank, group;
  int32_t max_pages, num_bpages, num_rpages;
  int32_t off_items, off_lens, off_slot_ptr, off_slot_list, off_lastpage;
  int32_t max_agent_slots;  // the largest number of split-K partials of one agent
  float lora_scale, sm_scale_log2, rope_theta;
};

struct PrefillParams {
  const void* q;
  const void* k_new;
  const void* v_new;
  const void* rk_new;
  const void* rv_new;
  const void* Bk;
  const void* Bv;
  void* bcache;
  void* rcache;
  const int32_t* btab;
  const int32_t* rtab;
  const int32_t* start_pos;
  const int32_t* positions;  // nullable: [N][C] position of every row (strictly increasing
                             // per agent); null: row i of agent a at start_pos[a] + i
  const int32_t* pstart;     // nullable: [N][max_pages] start position of each page
  bool write_res;            // the row write stores the residual rows too
  void* out;
  int32_t n_agents, chunk_len, num_q_heads, num_kv_heads, head_dim, rank, group;
  int32_t max_pages, num_bpages, num_rpages;
  int32_t pos_bias;         // row i of agent a is stored at position start_pos[a] + pos_bias + i
  float lora_scale, sm_scale_log2, rope_theta;
};

// Position of row i of agent a (both kernels and the row write agree on it).
__host__ __device__ inline int row_position(const PrefillParams& p, int a, int i) {
  return p.positions ? p.positions[size_t(a) * p.chunk_len + i] : p.start_pos[a] + p.pos_bias + i;
}

// The slot map.  Logical page lp of agent a holds the positions from its start up to the
// next page's start (P rows for a full page, fewer for a frozen tail); without a start
// table (null) page lp starts at lp * P.
__host__ __device__ inline int page_start(const int32_t* pstart, int max_pages, int a, int lp) {
  return pstart ? pstart[size_t(a) * max_pages + lp] : lp * kPage;
}
// Rows of page lp held by agent a of length len (<= P; <= 0 past the end).
__host__ __device__ inline int page_rows(const int32_t* pstart, int max_pages, int a, int lp,
                                         int len) {
  int end = len, st = lp * kPage;
  if (pstart) {
    const int32_t* row = pstart + size_t(a) * max_pages;
    st = row[lp];
    if (lp + 1 < max_pages && row[lp + 1] >= 0 && row[lp + 1] < end) end = row[lp + 1];
  }
  return end - st < kPage ? end - st : kPage;
}
// Logical page of position t >= 0: the last page whose start is <= t (binary search; the
// starts increase and are -1 past the last page).
__host__ __device__ inline int page_of(const int32_t* pstart, int max_pages, int a, int t) {
  if (!pstart) return t / kPage;
  const int32_t* row = pstart + size_t(a) * max_pages;
  int lo = 0, hi = max_pages - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (row[mid] >= 0 && row[mid] <= t) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// Kernel launchers (defined in the .hip translation units).  They return hipError_t
// from the launch.
hipError_t launch_decode_generic(const DecodeParams& p, int dtype, int max_agents,
                                 hipStream_t s);
hipError_t launch_decode_mfma(const DecodeParams& p, hipStream_t s);
hipError_t launch_combine(const DecodeParams& p, int dtype, hipStream_t s);
hipError_t launch_prefill_write(const PrefillParams& p, int dtype, hipStream_t s);
hipError_t launch_prefill_generic(const PrefillParams& p, int dtype, hipStream_t s);
hipError_t launch_prefill_mfma(const PrefillParams& p, const int32_t* start_host,
                               hipStream_t s);
hipError_t launch_cow_copy(void* bcache, int dtype, int num_kv_heads, int head_dim,
                           int32_t src_page, int32_t dst_page, int32_t n_rows, hipStream_t s);

// Device address of the current device's static split-K scratch (scratch.hip).
void* noalloc_scratch(hipError_t* err);

// Limits of the generic kernel.
constexpr int kGenericThreads = 256;
constexpr int kGenericAccPerThread = 32;   // rows * d <= 256 * 32
constexpr int kGenericAccrPerThread = 8;   // rows * r <= 256 * 8
constexpr int kGenericMaxRows = 64;
// A gfx950 workgroup may use the CU's whole 160 KiB of LDS; launches above the default
// 64 KiB of dynamic LDS raise the kernel's limit first.
constexpr int kMaxLds = 160 * 1024;
constexpr int kDefaultDynLds = 64 * 1024;

// LDS plan of the generic kernel (byte offsets), shared by the kernel and the host code that
// sizes its launches and items.
struct GenLds {
  int inv, cs, bk, bv, kq, rk, rv, s, alpha, m, l, accr, total;
};
__host__ __device__ inline GenLds gen_lds(int na, int rows, int d, int r) {
  GenLds L{};
  int o = 0;
  auto take = [&](int bytes) { int at = o; o += (bytes + 15) & ~15; return at; };
  L.inv = take(8 * (d / 2));
  L.cs = take(4 * kPage * d);  // [P][d/2][2]
  L.bk = take(4 * kPage * d);
  L.bv = take(4 * kPage * d);
  L.kq = take(4 * kPage * d);
  L.rk = take(4 * na * kPage * r);
  L.rv = take(4 * na * kPage * r);
  L.s = take(4 * rows * kPage);
  L.alpha = take(4 * rows);
  L.m = take(4 * rows);
  L.l = take(4 * rows);
  L.accr = take(4 * rows * r);
  L.total = o;
  return L;
}

// The MFMA decode kernel: waves per workgroup, and agents per wave for a GQA group of
// `group` query heads (the wave's 16 query columns hold whole groups, at most 4 agents).
constexpr int kMfmaWaves = 4;
constexpr int kMfmaHeadDim = 128, kMfmaRank = 16;  // the one shape the MFMA kernels take
inline int mfma_agents_per_group(int group) {
  return group >= 1 && group <= 16 ? (16 / group < 4 ? 16 / group : 4) : 0;
}
int generic_max_agents(int group, int head_dim, int rank);
int generic_lds_bytes(int na, int rows, int d, int r);
bool prefill_mfma_enabled();
bool mfma_supported(int dtype, int head_dim, int rank, int group);
int mfma_group_agents(int group);
int mfma_agents_per_wave(int group);

}  // namespace forkkv
