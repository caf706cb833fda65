// C-ABI entry points of the attention calls: argument validation, launch, timing.
#include <cmath>

#include "forkkv_internal.h"

using forkkv::kPage;

namespace {

constexpr float kLog2e = 1.4426950408889634f;

bool same_geometry(const forkkv_pool_desc& a, const forkkv_pool_desc& b) {
  return a.num_bpages == b.num_bpages && a.num_rpages == b.num_rpages &&
         a.num_kv_heads == b.num_kv_heads && a.head_dim == b.head_dim && a.rank == b.rank &&
         a.dtype == b.dtype && a.page_size == b.page_size;
}

hipEvent_t get_event(forkkv_plan* pl) {
  if (!pl->spare.empty()) {
    hipEvent_t e = pl->spare.back();
    pl->spare.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Scales are finite; the softmax scale is also > 0 (the MFMA prefill kernel takes each
// row's maximum of the raw scores and scales it afterwards, and scales masked scores of
// -inf), theta > 0.
bool finite(float x) { return std::isfinite(x); }

// Device buffers are read and written with 8- and 16-byte vector accesses.
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
template <typename... P>
bool all_aligned16(const P*... ps) { return (aligned16(ps) && ...); }

}  // namespace

extern "C" {

int forkkv_plan_set_timing(forkkv_plan* pl, int32_t enable) {
  if (!pl || enable < FORKKV_TIMING_OFF || enable > FORKKV_TIMING_SPLIT_ONLY) return FORKKV_EINVAL;
  pl->timing = enable == FORKKV_TIMING_EVENTS;
  pl->split_only = enable == FORKKV_TIMING_SPLIT_ONLY;
  return FORKKV_OK;
}

int forkkv_plan_timing(forkkv_plan* pl, double* split_ms, double* combine_ms, int32_t* launches) {
  if (!pl) return FORKKV_EINVAL;
  double sms = 0.0, cms = 0.0;
  int32_t count = 0;
  int rc = FORKKV_OK;
  for (auto& t : pl->pending) {
    float ms = 0.f;
    if (hipEventSynchronize(t.e) != hipSuccess || hipEventElapsedTime(&ms, t.b, t.e) != hipSuccess)
      rc = FORKKV_EHIP;
    if (t.kind == 0) {
      sms += ms;
      ++count;
    } else {
      cms += ms;
    }
    pl->spare.push_back(t.b);
    pl->spare.push_back(t.e);
  }
  pl->pending.clear();
  if (split_ms) *split_ms = sms;
  if (combine_ms) *combine_ms = cms;
  if (launches) *launches = count;
  return rc;
}

}  // extern "C"

namespace {

// Validate decode arguments and fill the kernel parameters (no launch).
int prepare_decode(const forkkv_decode_args* a, forkkv::DecodeParams* out) {
  if (!a || !a->pool || !a->plan) return FORKKV_EINVAL;
  const forkkv_pool* pool = a->pool;
  const forkkv_plan* pl = a->plan;
  if (!same_geometry(pool->desc, pl->geo)) return FORKKV_EINVAL;
  if (!pool->bcache) return FORKKV_ESTATE;
  if (pl->n_agents == 0) return FORKKV_OK;
  if (!pl->dev) return FORKKV_ESTATE;
  if (!a->q || !a->Bk || !a->Bv || !a->btab || !a->rtab || !a->out) return FORKKV_EINVAL;
  if (!all_aligned16(a->q, a->Bk, a->Bv, a->out, a->workspace)) return FORKKV_EINVAL;
  if (a->max_pages < pl->max_pages_needed) return FORKKV_EINVAL;
  if (!pl->aligned && !a->pstart) return FORKKV_EINVAL;  // a frozen tail needs the slot map
  if (pl->n_slots > 0 && (!a->workspace || a->workspace_bytes < pl->workspace_bytes))
    return FORKKV_EINVAL;
  if (!finite(a->lora_scale) || !finite(a->sm_scale) || !(a->sm_scale > 0.f) ||
      !(a->rope_theta > 0.f) || !finite(a->rope_theta))
    return FORKKV_EINVAL;

  const forkkv_pool_desc& g = pool->desc;
  forkkv::DecodeParams& p = *out;
  p = forkkv::DecodeParams{};
  p.q = a->q;
  p.Bk = a->Bk;
  p.Bv = a->Bv;
  p.bcache = pool->bcache;
  p.rcache = pool->rcache;
  p.btab = a->btab;
  p.rtab = a->rtab;
  p.pstart = a->pstart;
  p.plan = static_cast<const int32_t*>(pl->dev);
  char* ws = static_cast<char*>(a->workspace);
  p.ws_ml = reinterpret_cast<float*>(ws);
  p.ws_acc = reinterpret_cast<float*>(ws + pl->ws_off_acc);
  p.ws_accr = reinterpret_cast<float*>(ws + pl->ws_off_accr);
  p.out = a->out;
  p.n_agents = pl->n_agents;
  p.n_items = pl->item_capacity;  // the launch grid; the kernels read the live count
  p.num_q_heads = pl->num_q_heads;
  p.num_kv_heads = g.num_kv_heads;
  p.head_dim = g.head_dim;
  p.rank = g.rank;
  p.group = pl->num_q_heads / g.num_kv_heads;
  p.max_pages = a->max_pages;
  p.num_bpages = g.num_bpages;
  p.num_rpages = g.num_rpages;
  p.off_items = pl->blob[forkkv::kHdrOffItems];
  p.off_lens = pl->blob[forkkv::kHdrOffLens];
  p.off_slot_ptr = pl->blob[forkkv::kHdrOffSlotPtr];
  p.off_slot_list = pl->blob[forkkv::kHdrOffSlotList];
  p.off_lastpage = pl->blob[forkkv::kHdrOffLastPage];
  p.max_agent_slots = pl->max_agent_slots;
  p.lora_scale = a->lora_scale;
  p.sm_scale_log2 = a->sm_scale * kLog2e;
  p.rope_theta = a->rope_theta;
  return FORKKV_OK;
}

// Split kernel + combine on the stream, with the plan's optional event timing.
int launch_decode(forkkv_plan* pl, const forkkv::DecodeParams& p, int dtype, hipStream_t stream,
                  bool allow_timing = true) {
  hipEvent_t ev[4] = {nullptr, nullptr, nullptr, nullptr};
  if (pl->timing && allow_timing) {
    for (auto& e : ev) {
      e = get_event(pl);
      if (!e) return FORKKV_EHIP;
    }
  }
  if (pl->item_capacity > 0) {
    if (ev[0] && hipEventRecord(ev[0], stream) != hipSuccess) return FORKKV_EHIP;
    hipError_t err = pl->kernel == FORKKV_KERNEL_MFMA
                         ? forkkv::launch_decode_mfma(p, stream)
                         : forkkv::launch_decode_generic(p, dtype, pl->group, stream);
    if (err != hipSuccess) return FORKKV_EHIP;
    if (ev[1] && hipEventRecord(ev[1], stream) != hipSuccess) return FORKKV_EHIP;
  }
  if (pl->split_only) return hipGetLastError() == hipSuccess ? FORKKV_OK : FORKKV_EHIP;
  if (ev[2] && hipEventRecord(ev[2], stream) != hipSuccess) return FORKKV_EHIP;
  if (forkkv::launch_combine(p, dtype, stream) != hipSuccess) return FORKKV_EHIP;
  if (ev[3] && hipEventRecord(ev[3], stream) != hipSuccess) return FORKKV_EHIP;
  if (pl->timing && allow_timing) {
    if (pl->item_capacity > 0) {
      pl->pending.push_back({0, ev[0], ev[1]});
    } else {
      pl->spare.push_back(ev[0]);
      pl->spare.push_back(ev[1]);
    }
    pl->pending.push_back({1, ev[2], ev[3]});
  }
  if (hipGetLastError() != hipSuccess) return FORKKV_EHIP;
  return FORKKV_OK;
}

}  // namespace

extern "C" {

int forkkv_residual_attn_decode(const forkkv_decode_args* a, hipStream_t stream) {
  forkkv::DecodeParams p;
  const int rc = prepare_decode(a, &p);
  if (rc != FORKKV_OK || a->plan->n_agents == 0) return rc;
  (void)hipGetLastError();  // clear a stale error so the checks below see only ours
  return launch_decode(const_cast<forkkv_plan*>(a->plan), p, a->pool->desc.dtype, stream);
}

int forkkv_residual_attn_decode_noalloc(const forkkv_decode_args* a, hipStream_t stream) {
  if (!a || !a->plan) return FORKKV_EINVAL;
  if (a->plan->workspace_bytes > FORKKV_NOALLOC_SCRATCH_BYTES) return FORKKV_ETOOBIG;
  forkkv_decode_args args = *a;
  args.workspace = nullptr;
  args.workspace_bytes = 0;
  if (a->plan->n_slots > 0) {
    hipError_t err = hipSuccess;
    args.workspace = forkkv::noalloc_scratch(&err);
    if (!args.workspace) return FORKKV_EHIP;
    args.workspace_bytes = FORKKV_NOALLOC_SCRATCH_BYTES;
  }
  forkkv::DecodeParams p;
  const int rc = prepare_decode(&args, &p);
  if (rc != FORKKV_OK || a->plan->n_agents == 0) return rc;
  (void)hipGetLastError();
  return launch_decode(const_cast<forkkv_plan*>(a->plan), p, a->pool->desc.dtype, stream,
                       /*allow_timing=*/false);
}

int forkkv_residual_attn_decode_append(const forkkv_decode_append_args* a, hipStream_t stream) {
  if (!a) return FORKKV_EINVAL;
  forkkv::DecodeParams p;
  const int rc = prepare_decode(&a->decode, &p);
  const forkkv_plan* pl = a->decode.plan;
  if (rc != FORKKV_OK || pl->n_agents == 0) return rc;
  if (!a->k_new || !a->v_new || !a->rk_new || !a->rv_new) return FORKKV_EINVAL;
  if (!all_aligned16(a->k_new, a->v_new, a->rk_new, a->rv_new)) return FORKKV_EINVAL;
  // every agent's captured length counts its new token
  const int32_t off_lens = pl->blob[forkkv::kHdrOffLens];
  for (int32_t i = 0; i < pl->n_agents; ++i)
    if (pl->blob[off_lens + i] < 1) return FORKKV_EINVAL;
  const forkkv_pool_desc& g = a->decode.pool->desc;
  forkkv::PrefillParams w{};
  w.k_new = a->k_new;
  w.v_new = a->v_new;
  w.rk_new = a->rk_new;
  w.rv_new = a->rv_new;
  w.bcache = a->decode.pool->bcache;
  w.rcache = a->decode.pool->rcache;
  w.btab = a->decode.btab;
  w.rtab = a->decode.rtab;
  w.pstart = a->decode.pstart;
  w.write_res = true;
  w.start_pos = p.plan + off_lens;  // the plan's lengths, on the device
  w.pos_bias = -1;                  // the new token sits at position length - 1
  w.n_agents = pl->n_agents;
  w.chunk_len = 1;
  w.num_q_heads = pl->num_q_heads;
  w.num_kv_heads = g.num_kv_heads;
  w.head_dim = g.head_dim;
  w.rank = g.rank;
  w.group = p.group;
  w.max_pages = a->decode.max_pages;
  w.num_bpages = g.num_bpages;
  w.num_rpages = g.num_rpages;
  (void)hipGetLastError();
  // the combine kernel advances the device lengths once the call has read them
  p.advance = static_cast<int32_t*>(pl->dev) + off_lens;
  if (pl->kernel == FORKKV_KERNEL_MFMA) {
    // the split kernel stores the new rows itself, ahead of the pages that hold them
    p.k_new = a->k_new;
    p.v_new = a->v_new;
    p.rk_new = a->rk_new;
    p.rv_new = a->rv_new;
  } else if (forkkv::launch_prefill_write(w, g.dtype, stream) != hipSuccess) {
    return FORKKV_EHIP;
  }
  return launch_decode(const_cast<forkkv_plan*>(pl), p, g.dtype, stream);
}

int forkkv_residual_attn_prefill(const forkkv_prefill_args* a, hipStream_t stream) {
  if (!a || !a->pool) return FORKKV_EINVAL;
  const forkkv_pool* pool = a->pool;
  const forkkv_pool_desc& g = pool->desc;
  if (!pool->bcache) return FORKKV_ESTATE;
  if (a->n_agents < 0 || a->chunk_len < 1) return FORKKV_EINVAL;
  if (a->num_q_heads < g.num_kv_heads || a->num_q_heads % g.num_kv_heads) return FORKKV_EINVAL;
  if (a->n_agents == 0) return FORKKV_OK;
  const bool listed = a->positions != nullptr;
  if (!a->q || !a->k_new || !a->v_new || !a->rk_new || !a->rv_new || !a->Bk || !a->Bv ||
      !a->btab || !a->rtab || !a->out)
    return FORKKV_EINVAL;
  if (!all_aligned16(a->q, a->k_new, a->v_new, a->rk_new, a->rv_new, a->Bk, a->Bv, a->out))
    return FORKKV_EINVAL;
  if (listed ? !a->positions_host : (!a->start_pos || !a->start_pos_host)) return FORKKV_EINVAL;
  if (a->max_pages < 1) return FORKKV_EINVAL;
  if (!finite(a->lora_scale) || !finite(a->sm_scale) || !(a->sm_scale > 0.f) ||
      !(a->rope_theta > 0.f) || !finite(a->rope_theta))
    return FORKKV_EINVAL;
  if (a->kernel != FORKKV_KERNEL_AUTO && a->kernel != FORKKV_KERNEL_GENERIC &&
      a->kernel != FORKKV_KERNEL_MFMA)
    return FORKKV_EINVAL;
  const int64_t cap = int64_t(a->max_pages) * kPage;
  for (int32_t i = 0; i < a->n_agents; ++i) {
    if (listed) {
      const int32_t* pos = a->positions_host + size_t(i) * a->chunk_len;
      if (pos[0] < 0) return FORKKV_EINVAL;
      for (int32_t c = 1; c < a->chunk_len; ++c)
        if (pos[c] <= pos[c - 1]) return FORKKV_EINVAL;
      if (pos[a->chunk_len - 1] >= cap) return FORKKV_EINVAL;
    } else {
      const int64_t s = a->start_pos_host[i];
      if (s < 0 || s + a->chunk_len > cap) return FORKKV_EINVAL;
    }
  }
  forkkv::PrefillParams p{};
  p.q = a->q;
  p.k_new = a->k_new;
  p.v_new = a->v_new;
  p.rk_new = a->rk_new;
  p.rv_new = a->rv_new;
  p.Bk = a->Bk;
  p.Bv = a->Bv;
  p.bcache = pool->bcache;
  p.rcache = pool->rcache;
  p.btab = a->btab;
  p.rtab = a->rtab;
  p.start_pos = a->start_pos;
  p.positions = a->positions;
  p.pstart = a->pstart;
  p.write_res = true;
  p.out = a->out;
  p.n_agents = a->n_agents;
  p.chunk_len = a->chunk_len;
  p.num_q_heads = a->num_q_heads;
  p.num_kv_heads = g.num_kv_heads;
  p.head_dim = g.head_dim;
  p.rank = g.rank;
  p.group = a->num_q_heads / g.num_kv_heads;
  p.max_pages = a->max_pages;
  p.num_bpages = g.num_bpages;
  p.num_rpages = g.num_rpages;
  p.lora_scale = a->lora_scale;
  p.sm_scale_log2 = a->sm_scale * kLog2e;
  p.rope_theta = a->rope_theta;
  if (p.group > forkkv::kGenericMaxRows || forkkv::generic_max_agents(p.group, p.head_dim, p.rank) < 1)
    return FORKKV_EUNSUPPORTED;

  // (the MFMA prefill kernel has an instantiation for the slot map, like the decode kernel)
  const bool mfma_ok = forkkv::mfma_supported(g.dtype, g.head_dim, g.rank, p.group) &&
                       forkkv::prefill_mfma_enabled();
  if (a->kernel == FORKKV_KERNEL_MFMA && !mfma_ok) return FORKKV_EUNSUPPORTED;
  const bool mfma = mfma_ok && a->kernel != FORKKV_KERNEL_GENERIC;
  (void)hipGetLastError();
  if (forkkv::launch_prefill_write(p, g.dtype, stream) != hipSuccess) return FORKKV_EHIP;
  hipError_t err = mfma ? forkkv::launch_prefill_mfma(p, a->start_pos_host, stream)
                        : forkkv::launch_prefill_generic(p, g.dtype, stream);
  if (err != hipSuccess) return FORKKV_EHIP;
  if (hipGetLastError() != hipSuccess) return FORKKV_EHIP;
  return FORKKV_OK;
}

int forkkv_write_rows(const forkkv_write_args* a, hipStream_t stream) {
  if (!a || !a->pool) return FORKKV_EINVAL;
  const forkkv_pool* pool = a->pool;
  const forkkv_pool_desc& g = pool->desc;
  if (!pool->bcache) return FORKKV_ESTATE;
  if (a->n_seqs < 0 || a->n_rows < 1 || a->max_pages < 1) return FORKKV_EINVAL;
  if (a->n_seqs == 0) return FORKKV_OK;
  const bool res = a->rk_new != nullptr;
  if ((a->rv_new != nullptr) != res) return FORKKV_EINVAL;
  if (!a->btab || (res && !a->rtab) || !a->positions || !a->positions_host || !a->k_new ||
      !a->v_new)
    return FORKKV_EINVAL;
  if (!all_aligned16(a->k_new, a->v_new, a->rk_new, a->rv_new)) return FORKKV_EINVAL;
  const int64_t cap = int64_t(a->max_pages) * kPage;
  for (int32_t i = 0; i < a->n_seqs; ++i) {
    const int32_t* pos = a->positions_host + size_t(i) * a->n_rows;
    if (pos[0] < 0 || pos[a->n_rows - 1] >= cap) return FORKKV_EINVAL;
    for (int32_t c = 1; c < a->n_rows; ++c)
      if (pos[c] <= pos[c - 1]) return FORKKV_EINVAL;
  }
  forkkv::PrefillParams w{};
  w.k_new = a->k_new;
  w.v_new = a->v_new;
  w.rk_new = a->rk_new;
  w.rv_new = a->rv_new;
  w.bcache = pool->bcache;
  w.rcache = pool->rcache;
  w.btab = a->btab;
  w.rtab = a->rtab;
  w.pstart = a->pstart;
  w.write_res = res;
  w.positions = a->positions;
  w.n_agents = a->n_seqs;
  w.chunk_len = a->n_rows;
  w.num_kv_heads = g.num_kv_heads;
  w.head_dim = g.head_dim;
  w.rank = g.rank;
  w.max_pages = a->max_pages;
  w.num_bpages = g.num_bpages;
  w.num_rpages = g.num_rpages;
  (void)hipGetLastError();
  if (forkkv::launch_prefill_write(w, g.dtype, stream) != hipSuccess) return FORKKV_EHIP;
  return FORKKV_OK;
}

}  // extern "C"
