// Decode work plan: page-keyed work items with split-K cuts.
//
// Every (logical page, physical base page) that several agents alias becomes part of
// one work item listing all those agents, so the shared base page is streamed from HBM
// once and scored against every aliasing agent (ForkKV study note, "2. Q1 / Q2 / Q3" Q2:
// the base cache is shared globally; "3. 架构 / 方法图", Figure 6: forked agents map the
// parent's pages).  Long runs are cut into items of a bounded number of pages whose
// partial softmax states are merged by the combine kernel.
//
// A plan is step-stable: the per-step state of decode with append (each agent's length)
// lives in the plan's device copy and the append call advances it, so successive steps
// reuse one plan and one launch until an agent enters a new page (ForkServe README,
// "Methods": a write allocates residual pages only).  Then forkkv_plan_rebuild redoes the
// items in place; offsets and the launch grid come from capacities that only grow, so a
// rebuild within them leaves a captured launch valid.
#include <algorithm>
#include <cstring>
#include <new>

#include "forkkv_internal.h"

using forkkv::kItemAgents;
using forkkv::kItemInts;
using forkkv::kPage;

namespace {

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

using forkkv::Run;

// Build the plan of seqs into *pl (host side only: blob, sizes, capacities).  min_items and
// min_slots are capacities the plan must keep (those of the plan being rebuilt, or 0).
// prev (nullable): the plan being rebuilt; its runs up to the first logical page whose base
// pages changed are kept, and the scan resumes there (a decode step only changes the
// agents' last pages).
int build(const forkkv_pool* p, const forkkv_seq* seqs, int32_t n, int32_t num_q_heads,
          const forkkv_plan_opts& o, int32_t min_items, int32_t min_slots,
          const forkkv_plan* prev, forkkv_plan* pl) {
  const forkkv_pool_desc& g = p->desc;
  if (num_q_heads < g.num_kv_heads || num_q_heads % g.num_kv_heads) return FORKKV_EINVAL;
  const int group_q = num_q_heads / g.num_kv_heads;
  std::vector<const forkkv::Seq*> S(n);
  std::vector<int32_t> np(n);
  int32_t max_np = 0;
  {
    for (int32_t a = 0; a < n; ++a) {
      if (seqs[a] < 0 || static_cast<size_t>(seqs[a]) >= p->seqs.size()) return FORKKV_EINVAL;
      S[a] = &p->seqs[seqs[a]];
      if (!S[a]->alive || !S[a]->has_res) return FORKKV_EINVAL;
      np[a] = static_cast<int32_t>(S[a]->bpages.size());
      max_np = std::max(max_np, np[a]);
    }
  }
  // a partial hit (an evicted base page) must be refilled before it can be attended to
  for (int32_t a = 0; a < n; ++a)
    if (S[a]->missing_base()) return FORKKV_ESTATE;
  bool aligned = true;
  for (int32_t a = 0; a < n; ++a) aligned = aligned && S[a]->aligned();
  int kernel = o.kernel;
  const bool mfma_ok = forkkv::mfma_supported(g.dtype, g.head_dim, g.rank, group_q);
  if (kernel == FORKKV_KERNEL_AUTO) kernel = mfma_ok ? FORKKV_KERNEL_MFMA : FORKKV_KERNEL_GENERIC;
  int cap;
  if (kernel == FORKKV_KERNEL_MFMA) {
    if (!mfma_ok) return FORKKV_EUNSUPPORTED;
    cap = forkkv::mfma_group_agents(group_q);
    // A full item's agent groups share the workgroup's four waves: keep their count a
    // divisor of four (three agents per wave: items of six, not eight), so no wave idles.
    const int per_wave = forkkv::mfma_agents_per_wave(group_q);
    int groups = (cap + per_wave - 1) / per_wave;
    while (4 % groups) --groups;
    cap = std::min(cap, groups * per_wave);
  } else if (kernel == FORKKV_KERNEL_GENERIC) {
    cap = forkkv::generic_max_agents(group_q, g.head_dim, g.rank);
    if (cap < 1) return FORKKV_EUNSUPPORTED;
  } else {
    return FORKKV_EINVAL;
  }
  if (o.max_agents_per_item < 0 || o.pages_per_item < 0 || o.spare_items < 0) return FORKKV_EINVAL;
  if (o.max_agents_per_item > 0) cap = std::min(cap, o.max_agents_per_item);
  const int ppi = o.pages_per_item > 0 ? o.pages_per_item : 16;

  // 1. Maximal runs of logical pages over which one set of agents maps the same physical
  //    page.  A run open at lp - 1 continues at lp when all its agents map one physical page
  //    there and no other agent of the batch maps that page; the agents left over start new
  //    runs, one per physical page, ordered by their first agent.  Per logical page: one
  //    agreement check per agent of an open run, one holder count per run (and per agent
  //    outside the agreeing runs), flat arrays, no allocation in the common case.
  std::vector<const int32_t*> bp(n);
  for (int32_t a = 0; a < n; ++a) bp[a] = S[a]->bpages.data();
  std::vector<Run> runs;
  std::vector<int32_t> open, next_open, pending, agree;
  std::vector<int32_t> holders(g.num_bpages, 0);  // groups mapping a page at lp (reset after)
  std::vector<char> taken(n, 0);
  int32_t lp_start = 0;
  const bool reuse = prev && aligned && prev->seq_ids.size() == static_cast<size_t>(n) &&
                     std::equal(seqs, seqs + n, prev->seq_ids.begin()) &&
                     prev->bpages_seen.size() == static_cast<size_t>(n);
  if (reuse) {
    // the first logical page at which any agent's base pages differ from the last build
    lp_start = max_np;
    for (int32_t a = 0; a < n; ++a) {
      const std::vector<int32_t>& old = prev->bpages_seen[a];
      const int32_t common = std::min<int32_t>(np[a], static_cast<int32_t>(old.size()));
      int32_t k = static_cast<int32_t>(
          std::mismatch(bp[a], bp[a] + common, old.begin()).first - bp[a]);
      if (k == common && np[a] == static_cast<int32_t>(old.size())) k = max_np;
      lp_start = std::min(lp_start, k);
    }
    // runs that began before lp_start are kept (cut at lp_start); those open at lp_start - 1
    // are the open set the scan resumes with
    for (const Run& r : prev->runs) {
      if (r.lp0 >= lp_start) break;  // runs are in order of their first page
      runs.push_back(r);
      if (r.lp1 >= lp_start) {
        runs.back().lp1 = lp_start;
        open.push_back(static_cast<int32_t>(runs.size()) - 1);
      }
    }
  }
  for (int32_t lp = lp_start; lp < max_np; ++lp) {
    // Under a slot map the kernels take a shared page's start and row count from one of its
    // holders: every holder must see the page at the same start with the same last row (the
    // pool only ever shares full pages and frozen tails, so this always holds).
    if (!aligned) {
      for (int32_t a = 0; a < n; ++a) {
        if (lp >= np[a]) continue;
        for (int32_t b = a + 1; b < n; ++b) {
          if (lp >= np[b] || bp[b][lp] != bp[a][lp]) continue;
          if (S[b]->starts[lp] != S[a]->starts[lp] || S[b]->rows(lp) != S[a]->rows(lp))
            return FORKKV_ESTATE;
        }
      }
    }
    // (a) open runs whose agents still agree on one page
    agree.clear();
    for (int32_t ri : open) {
      const Run& r = runs[ri];
      const int32_t a0 = r.agents[0];
      if (lp >= np[a0]) continue;
      const int32_t pg = bp[a0][lp];
      bool same = true;
      for (size_t k = 1; same && k < r.agents.size(); ++k) {
        const int32_t a = r.agents[k];
        same = lp < np[a] && bp[a][lp] == pg;
      }
      if (!same) continue;
      agree.push_back(ri);
      ++holders[pg];
      for (int32_t a : r.agents) taken[a] = 1;
    }
    // (b) the other agents' pages; (c) a run continues if nobody else maps its page
    pending.clear();
    for (int32_t a = 0; a < n; ++a)
      if (lp < np[a] && !taken[a]) {
        pending.push_back(a);
        ++holders[bp[a][lp]];
      }
    next_open.clear();
    for (int32_t ri : agree) {
      const Run& r = runs[ri];
      if (holders[bp[r.agents[0]][lp]] == 1) {
        runs[ri].lp1 = lp + 1;
        next_open.push_back(ri);
      } else {
        pending.insert(pending.end(), r.agents.begin(), r.agents.end());
      }
      for (int32_t a : r.agents) taken[a] = 0;
    }
    // (d) new runs: the pending agents grouped by physical page (agents ascending within a
    //     group), groups in the order of their first agent
    const size_t first_new = runs.size();
    if (!pending.empty()) {
      std::sort(pending.begin(), pending.end(), [&](int32_t x, int32_t y) {
        const int32_t px = bp[x][lp], py = bp[y][lp];
        return px != py ? px < py : x < y;
      });
      for (size_t i = 0; i < pending.size();) {
        size_t j = i;
        Run r{{}, lp, lp + 1};
        while (j < pending.size() && bp[pending[j]][lp] == bp[pending[i]][lp])
          r.agents.push_back(pending[j++]);
        runs.push_back(std::move(r));
        i = j;
      }
      std::sort(runs.begin() + first_new, runs.end(),
                [](const Run& x, const Run& y) { return x.agents[0] < y.agents[0]; });
    }
    for (size_t k = first_new; k < runs.size(); ++k) next_open.push_back(static_cast<int32_t>(k));
    open.swap(next_open);
    // (e) reset the holder counts touched at this page
    for (int32_t ri : agree) holders[bp[runs[ri].agents[0]][lp]] = 0;
    for (int32_t a : pending) holders[bp[a][lp]] = 0;
  }

  // 2. Cut runs into items: agent chunks of <= cap, page chunks of <= item_pages(chunk).
  //
  // The MFMA kernel runs four waves per item: the chunk's agents form n_groups groups of
  // up to A agents and the item's pages are split into 4 / n_groups sub-ranges, one per
  // wave.  Its items are sized so that the whole grid fits one round of resident waves when
  // possible (256 compute units x 8 waves on MI355X) and every wave does about the same
  // work: a page costs a wave about kPageShared + kPageAgent x (agents of its group) (the
  // shared base score, softmax and value product, then the per-agent key rebuild, rotation
  // and score), so waves of small groups take proportionally more pages.  At most 64 pages
  // per wave: a wave keeps its page ids in one register.
  constexpr int32_t kPageShared = 11, kPageAgent = 4;  // measured VALU-issue ratio
  const int A = kernel == FORKKV_KERNEL_MFMA ? forkkv::mfma_agents_per_wave(group_q) : 0;
  auto n_sub_of = [&](int32_t na) { return 4 / ((na + A - 1) / A); };
  auto page_cost = [&](int32_t na) { return kPageShared + kPageAgent * std::min(na, A); };
  int32_t target = 0;   // MFMA: cost budget per wave
  int32_t fixed_pw = 0; // MFMA: explicit pages per wave (tuning)
  auto pages_per_wave = [&](int32_t na) {
    if (fixed_pw > 0) return fixed_pw;
    return std::max<int32_t>(1, std::min<int32_t>(64, target / page_cost(na)));
  };
  if (kernel == FORKKV_KERNEL_MFMA) {
    const int64_t slots = 2048;
    auto waves_now = [&]() {
      int64_t wv = 0;
      for (const Run& r : runs)
        for (size_t a0 = 0; a0 < r.agents.size(); a0 += cap) {
          const int32_t na = static_cast<int32_t>(std::min<size_t>(cap, r.agents.size() - a0));
          const int32_t item_pages = pages_per_wave(na) * n_sub_of(na);
          wv += 4 * int64_t((r.lp1 - r.lp0 + item_pages - 1) / item_pages);
        }
      return wv * g.num_kv_heads;
    };
    if (o.pages_per_item > 0) {
      fixed_pw = std::max(1, std::min(64, o.pages_per_item));
    } else {
      // smallest per-wave budget whose grid fits one round (waves only fall as it grows)
      const int32_t top = 64 * page_cost(A);
      int32_t lo = page_cost(1), hi = top;
      target = hi;
      if (waves_now() <= slots) {
        while (lo < hi) {
          target = lo + (hi - lo) / 2;
          if (waves_now() <= slots) hi = target;
          else lo = target + 1;
        }
        target = lo;
      }
    }
  }
  std::vector<int32_t> items;
  std::vector<int32_t> per_agent(n, 0);  // partials per agent (slot numbering below)
  int32_t n_slots = 0;
  for (const Run& r : runs) {
    for (size_t a0 = 0; a0 < r.agents.size(); a0 += cap) {
      const int32_t na = static_cast<int32_t>(std::min<size_t>(cap, r.agents.size() - a0));
      const int32_t item_pages =
          kernel == FORKKV_KERNEL_MFMA ? pages_per_wave(na) * n_sub_of(na) : ppi;
      for (int32_t lp = r.lp0; lp < r.lp1; lp += item_pages) {
        const int32_t npg = std::min(item_pages, r.lp1 - lp);
        int32_t it[kItemInts];
        std::fill(it, it + kItemInts, -1);
        it[0] = lp;
        it[1] = npg;
        it[2] = na;
        it[3] = 0;  // set below when the item holds an agent's last page
        for (int32_t j = 0; j < na; ++j) {
          const int32_t a = r.agents[a0 + j];
          it[4 + j] = a;
          it[4 + kItemAgents + j] = per_agent[a]++;  // index within the agent, for now
          if (np[a] - 1 >= lp && np[a] - 1 < lp + npg) it[3] = 1;
        }
        n_slots += na;
        items.insert(items.end(), it, it + kItemInts);
      }
    }
  }
  const int32_t n_items = static_cast<int32_t>(items.size() / kItemInts);
  // slots of agent a: slot_ptr[a] + (its index), consecutive per agent
  std::vector<int32_t> slot_ptr(n + 1, 0);
  int32_t max_agent_slots = 0;
  for (int32_t a = 0; a < n; ++a) {
    slot_ptr[a + 1] = slot_ptr[a] + per_agent[a];
    max_agent_slots = std::max(max_agent_slots, per_agent[a]);
  }
  for (int32_t i = 0; i < n_items; ++i) {
    int32_t* it = items.data() + size_t(i) * kItemInts;
    for (int32_t j = 0; j < it[2]; ++j) it[4 + kItemAgents + j] += slot_ptr[it[4 + j]];
  }
  // capacities: the launch grid covers item_capacity items and the workspace slot_capacity
  // slots, so a rebuild that stays within both keeps the launch (and a captured graph) valid
  const int32_t spare = o.spare_items > 0 ? o.spare_items : n;
  int32_t item_cap = std::max(min_items, n_items);
  if (n_items > min_items) item_cap = n_items + spare;
  int32_t slot_cap = std::max(min_slots, n_slots);
  if (n_slots > min_slots) slot_cap = n_slots + spare * cap;

  pl->seq_ids.assign(seqs, seqs + n);
  pl->bpages_seen.resize(n);
  for (int32_t a = 0; a < n; ++a) pl->bpages_seen[a].assign(bp[a], bp[a] + np[a]);
  pl->runs = std::move(runs);
  pl->geo = g;
  pl->geo.bpage_order = pl->geo.rpage_order = nullptr;
  pl->bcache = p->bcache;
  pl->rcache = p->rcache;
  pl->opts = o;
  pl->n_agents = n;
  pl->n_items = n_items;
  pl->n_slots = n_slots;
  pl->item_capacity = item_cap;
  pl->slot_capacity = slot_cap;
  pl->num_q_heads = num_q_heads;
  pl->kernel = kernel;
  pl->group = cap;
  pl->aligned = aligned;
  pl->max_agent_slots = max_agent_slots;
  pl->max_pages_needed = max_np;

  std::vector<int32_t>& b = pl->blob;
  b.assign(forkkv::kHdrWords, 0);
  b[forkkv::kHdrMagic] = forkkv::kPlanMagic;
  b[forkkv::kHdrAgents] = n;
  b[forkkv::kHdrItems] = n_items;
  b[forkkv::kHdrSlots] = n_slots;
  b[forkkv::kHdrItemInts] = kItemInts;
  b[forkkv::kHdrQHeads] = num_q_heads;
  b[forkkv::kHdrKernel] = kernel;
  b[forkkv::kHdrGroup] = cap;
  b[forkkv::kHdrItemCapacity] = item_cap;
  b[forkkv::kHdrSlotCapacity] = slot_cap;
  b[forkkv::kHdrOffItems] = static_cast<int32_t>(b.size());
  b.insert(b.end(), items.begin(), items.end());
  b.resize(b.size() + size_t(item_cap - n_items) * kItemInts, 0);  // room for later items
  b[forkkv::kHdrOffLens] = static_cast<int32_t>(b.size());
  for (int32_t a = 0; a < n; ++a) b.push_back(S[a]->len);
  b[forkkv::kHdrOffSlotPtr] = static_cast<int32_t>(b.size());
  b.insert(b.end(), slot_ptr.begin(), slot_ptr.end());
  b[forkkv::kHdrOffSlotList] = static_cast<int32_t>(b.size());  // empty: slots are ranges
  // last logical page of each agent: decode with append stores the new token there, at row
  // (length - 1) - (page start), with the length read on the device
  b[forkkv::kHdrOffLastPage] = static_cast<int32_t>(b.size());
  for (int32_t a = 0; a < n; ++a) b.push_back(S[a]->len > 0 ? np[a] - 1 : -1);

  const size_t rows = size_t(slot_cap) * num_q_heads;
  pl->ws_off_acc = align256(rows * 2 * sizeof(float));
  pl->ws_off_accr = pl->ws_off_acc + align256(rows * g.head_dim * sizeof(float));
  pl->workspace_bytes = pl->ws_off_accr + align256(rows * g.rank * sizeof(float));
  return FORKKV_OK;
}

void release_staging(forkkv_plan* pl) {
  for (int k = 0; k < 2; ++k) {
    if (pl->staged[k]) {
      (void)hipEventSynchronize(pl->staged[k]);
      (void)hipEventDestroy(pl->staged[k]);
      pl->staged[k] = nullptr;
    }
    if (pl->staging[k]) (void)hipHostFree(pl->staging[k]);
    pl->staging[k] = nullptr;
    pl->staging_bytes[k] = 0;
  }
}

}  // namespace


extern "C" {

int forkkv_plan_decode(const forkkv_pool* p, const forkkv_seq* seqs, int32_t n,
                       int32_t num_q_heads, const forkkv_plan_opts* opts, forkkv_plan** out) {
  if (!p || !out || n < 0 || (n > 0 && !seqs)) return FORKKV_EINVAL;
  forkkv_plan_opts o{};
  if (opts) o = *opts;
  forkkv_plan* pl = new (std::nothrow) forkkv_plan();
  if (!pl) return FORKKV_ENOMEM;
  const int rc = build(p, seqs, n, num_q_heads, o, 0, 0, nullptr, pl);
  if (rc != FORKKV_OK) {
    delete pl;
    return rc;
  }
  *out = pl;
  return FORKKV_OK;
}

int forkkv_plan_rebuild(forkkv_plan* pl, const forkkv_pool* p, const forkkv_seq* seqs,
                        int32_t n, int32_t* same_launch) {
  if (!pl || !p || n < 0 || (n > 0 && !seqs)) return FORKKV_EINVAL;
  forkkv_plan fresh;
  const int rc = build(p, seqs, n, pl->num_q_heads, pl->opts, pl->item_capacity,
                       pl->slot_capacity, pl, &fresh);
  if (rc != FORKKV_OK) return rc;  // the plan is unchanged
  const bool same = fresh.n_agents == pl->n_agents && fresh.item_capacity == pl->item_capacity &&
                    fresh.slot_capacity == pl->slot_capacity && fresh.kernel == pl->kernel &&
                    fresh.aligned == pl->aligned && fresh.group == pl->group;
  pl->geo = fresh.geo;
  pl->bcache = fresh.bcache;
  pl->rcache = fresh.rcache;
  pl->n_agents = fresh.n_agents;
  pl->n_items = fresh.n_items;
  pl->n_slots = fresh.n_slots;
  pl->item_capacity = fresh.item_capacity;
  pl->slot_capacity = fresh.slot_capacity;
  pl->kernel = fresh.kernel;
  pl->group = fresh.group;
  pl->aligned = fresh.aligned;
  pl->blob.swap(fresh.blob);
  pl->seq_ids.swap(fresh.seq_ids);
  pl->bpages_seen.swap(fresh.bpages_seen);
  pl->runs.swap(fresh.runs);
  pl->workspace_bytes = fresh.workspace_bytes;
  pl->ws_off_acc = fresh.ws_off_acc;
  pl->ws_off_accr = fresh.ws_off_accr;
  pl->max_pages_needed = fresh.max_pages_needed;
  pl->max_agent_slots = fresh.max_agent_slots;
  pl->dev = nullptr;  // the device copy is stale until the next upload
  if (same_launch) *same_launch = same ? 1 : 0;
  return FORKKV_OK;
}

int forkkv_plan_get_info(const forkkv_plan* pl, forkkv_plan_info* info) {
  if (!pl || !info) return FORKKV_EINVAL;
  info->n_agents = pl->n_agents;
  info->n_items = pl->n_items;
  info->n_slots = pl->n_slots;
  info->kernel = pl->kernel;
  info->item_ints = kItemInts;
  info->num_q_heads = pl->num_q_heads;
  info->plan_bytes = pl->blob.size() * sizeof(int32_t);
  info->workspace_bytes = pl->workspace_bytes;
  info->item_capacity = pl->item_capacity;
  info->slot_capacity = pl->slot_capacity;
  return FORKKV_OK;
}

int forkkv_plan_export(const forkkv_plan* pl, int32_t* host_blob) {
  if (!pl || !host_blob) return FORKKV_EINVAL;
  std::copy(pl->blob.begin(), pl->blob.end(), host_blob);
  return FORKKV_OK;
}

int forkkv_plan_upload(forkkv_plan* pl, void* dev, hipStream_t stream) {
  if (!pl || !dev) return FORKKV_EINVAL;
  // Two pinned staging buffers alternate; the copy out of one must have run before it is
  // refilled, two uploads later (in a serving loop, long done).  No stream-wide wait.
  const int k = pl->next_staging;
  const size_t bytes = pl->blob.size() * sizeof(int32_t);
  if (pl->staged[k] && hipEventSynchronize(pl->staged[k]) != hipSuccess) return FORKKV_EHIP;
  if (pl->staging_bytes[k] < bytes) {
    if (pl->staging[k]) (void)hipHostFree(pl->staging[k]);
    pl->staging[k] = nullptr;
    pl->staging_bytes[k] = 0;
    void* h = nullptr;
    if (hipHostMalloc(&h, bytes, hipHostMallocDefault) != hipSuccess) return FORKKV_EHIP;
    pl->staging[k] = h;
    pl->staging_bytes[k] = bytes;
  }
  if (!pl->staged[k] &&
      hipEventCreateWithFlags(&pl->staged[k], hipEventDisableTiming) != hipSuccess) {
    pl->staged[k] = nullptr;
    return FORKKV_EHIP;
  }
  std::memcpy(pl->staging[k], pl->blob.data(), bytes);
  if (hipMemcpyAsync(dev, pl->staging[k], bytes, hipMemcpyHostToDevice, stream) != hipSuccess)
    return FORKKV_EHIP;
  if (hipEventRecord(pl->staged[k], stream) != hipSuccess) return FORKKV_EHIP;
  pl->next_staging = 1 - k;
  pl->dev = dev;
  return FORKKV_OK;
}

int forkkv_plan_destroy(forkkv_plan* pl) {
  if (!pl) return FORKKV_EINVAL;
  for (auto& t : pl->pending) {
    (void)hipEventDestroy(t.b);
    (void)hipEventDestroy(t.e);
  }
  for (hipEvent_t e : pl->spare) (void)hipEventDestroy(e);
  release_staging(pl);
  delete pl;
  return FORKKV_OK;
}

}  // extern "C"
