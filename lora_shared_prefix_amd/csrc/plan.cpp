// Decode work plan: page-keyed work items with split-K cuts.
//
// Every (logical page, physical base page) that several agents alias becomes part of
// one work item listing all those agents, so the shared base page is streamed from HBM
// once and scored against every aliasing agent (ForkKV study note, "2. Q1 / Q2 / Q3" Q2:
// the base cache is shared globally; "3. 架构 / 方法图", Figure 6: forked agents map the
// parent's pages).  Long runs are cut into items of a bounded number of pages whose
// partial softmax states are merged by the combine kernel.
#include <algorithm>
#include <map>
#include <new>

#include "forkkv_internal.h"

using forkkv::kItemAgents;
using forkkv::kItemInts;
using forkkv::kPage;

namespace {

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct Run {
  std::vector<int32_t> agents;
  int32_t lp0, lp1;  // [lp0, lp1)
};

}  // namespace


extern "C" {

int forkkv_plan_decode(const forkkv_pool* p, const forkkv_seq* seqs, int32_t n,
                       int32_t num_q_heads, const forkkv_plan_opts* opts, forkkv_plan** out) {
  if (!p || !out || n < 0 || (n > 0 && !seqs)) return FORKKV_EINVAL;
  const forkkv_pool_desc& g = p->desc;
  if (num_q_heads < g.num_kv_heads || num_q_heads % g.num_kv_heads) return FORKKV_EINVAL;
  const int group_q = num_q_heads / g.num_kv_heads;
  std::vector<const forkkv::Seq*> S(n);
  int32_t max_np = 0;
  for (int32_t a = 0; a < n; ++a) {
    if (seqs[a] < 0 || static_cast<size_t>(seqs[a]) >= p->seqs.size()) return FORKKV_EINVAL;
    S[a] = &p->seqs[seqs[a]];
    if (!S[a]->alive || !S[a]->has_res) return FORKKV_EINVAL;
    max_np = std::max<int32_t>(max_np, static_cast<int32_t>(S[a]->bpages.size()));
  }
  // a partial hit (an evicted base page) must be refilled before it can be attended to
  for (int32_t a = 0; a < n; ++a)
    if (S[a]->missing_base()) return FORKKV_ESTATE;
  bool aligned = true;
  for (int32_t a = 0; a < n; ++a) aligned = aligned && S[a]->aligned();
  forkkv_plan_opts o{};
  if (opts) o = *opts;
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
  if (o.max_agents_per_item < 0 || o.pages_per_item < 0) return FORKKV_EINVAL;
  if (o.max_agents_per_item > 0) cap = std::min(cap, o.max_agents_per_item);
  int ppi = o.pages_per_item > 0 ? o.pages_per_item : 16;

  // 1. Maximal runs of logical pages with an identical set of agents sharing the page.
  std::vector<Run> runs;
  std::map<std::vector<int32_t>, size_t> open;  // agent set -> run index still open
  for (int32_t lp = 0; lp < max_np; ++lp) {
    std::map<int32_t, std::vector<int32_t>> by_page;  // physical page -> agents (ascending)
    for (int32_t a = 0; a < n; ++a)
      if (lp < static_cast<int32_t>(S[a]->bpages.size())) by_page[S[a]->bpages[lp]].push_back(a);
    std::map<std::vector<int32_t>, size_t> next_open;
    // order groups by their first agent for determinism
    std::vector<std::vector<int32_t>> groups;
    for (auto& kv : by_page) groups.push_back(kv.second);
    // Under a slot map the kernels take a shared page's start and row count from one of its
    // holders: every holder must see the page at the same start with the same last row (the
    // pool only ever shares full pages and frozen tails, so this always holds).
    if (!aligned)
      for (const auto& ag : groups) {
        const forkkv::Seq& s0 = *S[ag[0]];
        for (int32_t a : ag) {
          const forkkv::Seq& s = *S[a];
          if (s.starts[lp] != s0.starts[lp] || s.rows(lp) != s0.rows(lp)) return FORKKV_ESTATE;
        }
      }
    std::sort(groups.begin(), groups.end(),
              [](const std::vector<int32_t>& x, const std::vector<int32_t>& y) { return x[0] < y[0]; });
    for (auto& ag : groups) {
      auto it = open.find(ag);
      if (it != open.end()) {
        runs[it->second].lp1 = lp + 1;
        next_open[ag] = it->second;
      } else {
        runs.push_back(Run{ag, lp, lp + 1});
        next_open[ag] = runs.size() - 1;
      }
    }
    open.swap(next_open);
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
        const int32_t np = std::min(item_pages, r.lp1 - lp);
        int32_t it[kItemInts];
        std::fill(it, it + kItemInts, -1);
        it[0] = lp;
        it[1] = np;
        it[2] = na;
        it[3] = 0;
        for (int32_t j = 0; j < na; ++j) {
          const int32_t a = r.agents[a0 + j];
          it[4 + j] = a;
          it[4 + kItemAgents + j] = per_agent[a]++;  // index within the agent, for now
          const int32_t last = static_cast<int32_t>(S[a]->bpages.size()) - 1;
          if (S[a]->len > 0 && last >= lp && last < lp + np) it[3] |= 1 << j;
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

  forkkv_plan* pl = new (std::nothrow) forkkv_plan();
  if (!pl) return FORKKV_ENOMEM;
  pl->geo = g;
  pl->bcache = p->bcache;
  pl->rcache = p->rcache;
  pl->n_agents = n;
  pl->n_items = n_items;
  pl->n_slots = n_slots;
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
  b[forkkv::kHdrOffItems] = static_cast<int32_t>(b.size());
  b.insert(b.end(), items.begin(), items.end());
  b[forkkv::kHdrOffLens] = static_cast<int32_t>(b.size());
  for (int32_t a = 0; a < n; ++a) b.push_back(S[a]->len);
  b[forkkv::kHdrOffSlotPtr] = static_cast<int32_t>(b.size());
  b.insert(b.end(), slot_ptr.begin(), slot_ptr.end());
  b[forkkv::kHdrOffSlotList] = static_cast<int32_t>(b.size());  // empty: slots are ranges
  // slots of each agent's last row: where decode with append stores the new token
  b[forkkv::kHdrOffAppend] = static_cast<int32_t>(b.size());
  for (int32_t a = 0; a < n; ++a) {
    const forkkv::Seq& sq = *S[a];
    int32_t bs = -1, rs = -1;
    if (sq.len > 0) {
      const size_t last = sq.bpages.size() - 1;
      const int32_t row = sq.len - 1 - sq.starts[last];
      bs = sq.bpages[last] * forkkv::kPage + row;
      rs = sq.rpages[last] * forkkv::kPage + row;
    }
    b.push_back(bs);
    b.push_back(rs);
  }

  const size_t rows = size_t(n_slots) * num_q_heads;
  pl->ws_off_acc = align256(rows * 2 * sizeof(float));
  pl->ws_off_accr = pl->ws_off_acc + align256(rows * g.head_dim * sizeof(float));
  pl->workspace_bytes = pl->ws_off_accr + align256(rows * g.rank * sizeof(float));
  *out = pl;
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
  return FORKKV_OK;
}

int forkkv_plan_export(const forkkv_plan* pl, int32_t* host_blob) {
  if (!pl || !host_blob) return FORKKV_EINVAL;
  std::copy(pl->blob.begin(), pl->blob.end(), host_blob);
  return FORKKV_OK;
}

int forkkv_plan_upload(forkkv_plan* pl, void* dev, hipStream_t stream) {
  if (!pl || !dev) return FORKKV_EINVAL;
  if (hipMemcpyAsync(dev, pl->blob.data(), pl->blob.size() * sizeof(int32_t),
                     hipMemcpyHostToDevice, stream) != hipSuccess)
    return FORKKV_EHIP;
  // the host blob must stay valid until the copy has run: wait for it
  if (hipStreamSynchronize(stream) != hipSuccess) return FORKKV_EHIP;
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
  delete pl;
  return FORKKV_OK;
}

}  // extern "C"
