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
  forkkv_plan_opts o{};
  if (opts) o = *opts;
  int kernel = o.kernel;
  const bool mfma_ok = forkkv::mfma_supported(g.dtype, g.head_dim, g.rank, group_q);
  if (kernel == FORKKV_KERNEL_AUTO) kernel = mfma_ok ? FORKKV_KERNEL_MFMA : FORKKV_KERNEL_GENERIC;
  int cap;
  if (kernel == FORKKV_KERNEL_MFMA) {
    if (!mfma_ok) return FORKKV_EUNSUPPORTED;
    cap = forkkv::mfma_group_agents(group_q);
  } else if (kernel == FORKKV_KERNEL_GENERIC) {
    cap = forkkv::generic_max_agents(group_q, g.head_dim, g.rank);
    if (cap < 1) return FORKKV_EUNSUPPORTED;
  } else {
    return FORKKV_EINVAL;
  }
  if (o.max_agents_per_item < 0 || o.pages_per_item < 0) return FORKKV_EINVAL;
  if (o.max_agents_per_item > 0) cap = std::min(cap, o.max_agents_per_item);
  int ppi = o.pages_per_item > 0 ? o.pages_per_item : (kernel == FORKKV_KERNEL_MFMA ? 32 : 16);
  // the MFMA kernel keeps a wave's page ids in one register: at most 64 pages per item
  if (kernel == FORKKV_KERNEL_MFMA) ppi = std::min(ppi, 64);

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

  // 2. Cut runs into items: agent chunks of <= cap, page chunks of <= ppi.
  std::vector<int32_t> items;
  std::vector<std::vector<int32_t>> agent_slots(n);
  int32_t n_slots = 0;
  for (const Run& r : runs) {
    for (size_t a0 = 0; a0 < r.agents.size(); a0 += cap) {
      const int32_t na = static_cast<int32_t>(std::min<size_t>(cap, r.agents.size() - a0));
      for (int32_t lp = r.lp0; lp < r.lp1; lp += ppi) {
        const int32_t np = std::min(ppi, r.lp1 - lp);
        int32_t it[kItemInts];
        std::fill(it, it + kItemInts, -1);
        it[0] = lp;
        it[1] = np;
        it[2] = na;
        it[3] = n_slots;
        for (int32_t j = 0; j < na; ++j) {
          it[4 + j] = r.agents[a0 + j];
          agent_slots[r.agents[a0 + j]].push_back(n_slots + j);
        }
        n_slots += na;
        items.insert(items.end(), it, it + kItemInts);
      }
    }
  }
  const int32_t n_items = static_cast<int32_t>(items.size() / kItemInts);

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
  int32_t acc = 0;
  b.push_back(0);
  for (int32_t a = 0; a < n; ++a) {
    acc += static_cast<int32_t>(agent_slots[a].size());
    b.push_back(acc);
  }
  b[forkkv::kHdrOffSlotList] = static_cast<int32_t>(b.size());
  for (int32_t a = 0; a < n; ++a) b.insert(b.end(), agent_slots[a].begin(), agent_slots[a].end());

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
