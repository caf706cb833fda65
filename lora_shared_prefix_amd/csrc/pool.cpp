// Host bookkeeping of the forked, disaggregated page pools.
//
// ForkKV study note, "3. 架构 / 方法图" (Figure 6): a new agent maps the parent's
// read-only base pages and allocates only its own residual pages.  ForkServe README,
// "Design vs APC", "Methods" (CoW tree) and "Status": fork aliases the parent's frames,
// writes allocate private pages, an unaligned tail is packed by copying its n_valid rows
// or frozen into one read-only page shared by the trunk and its children (the adaptive
// tail), and reference counts keep a trunk alive after its parent is freed.  ForkKV study
// note, "Error / eviction recovery": base pages can be evicted while the residual pages
// survive, and refilled later (partial hit).
#include <algorithm>
#include <cstring>
#include <new>

#include "forkkv_internal.h"

using forkkv::Seq;
using forkkv::kPage;

namespace {

int32_t ceil_div(int64_t a, int64_t b) { return static_cast<int32_t>((a + b - 1) / b); }

size_t elem_bytes(int dtype) { return dtype == FORKKV_DTYPE_F32 ? 4 : 2; }

bool valid_desc(const forkkv_pool_desc* d) {
  if (!d) return false;
  if (d->page_size != kPage) return false;
  if (d->num_bpages < 1 || d->num_rpages < 1) return false;
  if (d->num_kv_heads < 1 || d->num_kv_heads > 64) return false;
  // tiles are stored in matrix-core operand order: 16-dim and 4-rank blocks
  if (d->head_dim < 16 || d->head_dim > 256 || (d->head_dim % 16)) return false;
  if (d->rank < 4 || d->rank > 64 || (d->rank % 4)) return false;
  if (d->dtype != FORKKV_DTYPE_F32 && d->dtype != FORKKV_DTYPE_BF16) return false;
  return true;
}

bool valid_order(const int32_t* order, int32_t n) {
  if (!order) return true;
  std::vector<char> seen(n, 0);
  for (int32_t i = 0; i < n; ++i) {
    if (order[i] < 0 || order[i] >= n || seen[order[i]]) return false;
    seen[order[i]] = 1;
  }
  return true;
}

Seq* get_seq(forkkv_pool* p, forkkv_seq h) {
  if (!p || h < 0 || static_cast<size_t>(h) >= p->seqs.size() || !p->seqs[h].alive) return nullptr;
  return &p->seqs[h];
}

const Seq* get_seq(const forkkv_pool* p, forkkv_seq h) {
  if (!p || h < 0 || static_cast<size_t>(h) >= p->seqs.size() || !p->seqs[h].alive) return nullptr;
  return &p->seqs[h];
}

int32_t take(std::deque<int32_t>& fl, std::vector<int32_t>& ref) {
  int32_t pg = fl.front();
  fl.pop_front();
  ref[pg] = 1;
  return pg;
}

void clear_cow(forkkv_cow_op* cow) {
  if (cow) *cow = forkkv_cow_op{-1, -1, 0};
}

}  // namespace

extern "C" {

const char* forkkv_strerror(int code) {
  switch (code) {
    case FORKKV_OK: return "ok";
    case FORKKV_EINVAL: return "invalid argument";
    case FORKKV_ENOMEM: return "page pool exhausted";
    case FORKKV_EHIP: return "HIP error";
    case FORKKV_ESTATE: return "invalid state";
    case FORKKV_EUNSUPPORTED: return "unsupported shape or dtype";
    case FORKKV_ETOOBIG: return "plan needs more split-K workspace than the static scratch holds";
    default: return "unknown error";
  }
}

int forkkv_pool_bytes(const forkkv_pool_desc* d, size_t* bbytes, size_t* rbytes) {
  if (!valid_desc(d)) return FORKKV_EINVAL;
  const size_t e = elem_bytes(d->dtype);
  if (bbytes) *bbytes = size_t(d->num_bpages) * 2 * d->num_kv_heads * kPage * d->head_dim * e;
  if (rbytes) *rbytes = size_t(d->num_rpages) * 2 * kPage * d->rank * e;
  return FORKKV_OK;
}

int forkkv_pool_create(const forkkv_pool_desc* d, void* bcache, void* rcache,
                       forkkv_pool** out) {
  if (!out || !valid_desc(d)) return FORKKV_EINVAL;
  if (!valid_order(d->bpage_order, d->num_bpages) || !valid_order(d->rpage_order, d->num_rpages))
    return FORKKV_EINVAL;
  if ((bcache == nullptr) != (rcache == nullptr)) return FORKKV_EINVAL;
  // (the kernels read pool tiles with 16-byte vector loads)
  if ((reinterpret_cast<uintptr_t>(bcache) | reinterpret_cast<uintptr_t>(rcache)) & 15u)
    return FORKKV_EINVAL;
  forkkv_pool* p = new (std::nothrow) forkkv_pool();
  if (!p) return FORKKV_ENOMEM;
  p->desc = *d;
  p->desc.bpage_order = nullptr;
  p->desc.rpage_order = nullptr;
  p->bcache = bcache;
  p->rcache = rcache;
  p->ref_b.assign(d->num_bpages, 0);
  p->ref_r.assign(d->num_rpages, 0);
  for (int32_t i = 0; i < d->num_bpages; ++i)
    p->free_b.push_back(d->bpage_order ? d->bpage_order[i] : i);
  for (int32_t i = 0; i < d->num_rpages; ++i)
    p->free_r.push_back(d->rpage_order ? d->rpage_order[i] : i);
  *out = p;
  return FORKKV_OK;
}

int forkkv_pool_destroy(forkkv_pool* p) {
  if (!p) return FORKKV_EINVAL;
  delete p;
  return FORKKV_OK;
}

int forkkv_seq_create(forkkv_pool* p, int32_t with_residual, forkkv_seq* out) {
  if (!p || !out) return FORKKV_EINVAL;
  Seq s;
  s.has_res = with_residual != 0;
  p->seqs.push_back(std::move(s));
  *out = static_cast<forkkv_seq>(p->seqs.size() - 1);
  return FORKKV_OK;
}

int forkkv_seq_append(forkkv_pool* p, forkkv_seq h, int32_t n, int32_t* bslots,
                      int32_t* rslots, forkkv_cow_op* cow) {
  Seq* s = get_seq(p, h);
  if (!s || n < 0) return FORKKV_EINVAL;
  if (s->missing_base()) return FORKKV_ESTATE;
  const int64_t new_len = int64_t(s->len) + n;
  if (new_len > INT32_MAX / 2) return FORKKV_EINVAL;
  // rows fill the last page while it has room (a frozen tail has none), then fresh pages
  const int32_t room = s->room();
  const int32_t grow = ceil_div(std::max<int64_t>(0, int64_t(n) - room), kPage);
  const size_t last = s->bpages.empty() ? 0 : s->bpages.size() - 1;
  // A write into a shared partial last page needs a private copy first.
  const bool need_cow = n > 0 && room > 0 && s->rows(last) > 0 && p->ref_b[s->bpages[last]] > 1;
  const int32_t need_b = grow + (need_cow ? 1 : 0);
  const int32_t need_r = s->has_res ? grow : 0;
  if (need_b > static_cast<int32_t>(p->free_b.size()) ||
      need_r > static_cast<int32_t>(p->free_r.size()))
    return FORKKV_ENOMEM;
  clear_cow(cow);
  if (need_cow) {
    const int32_t old = s->bpages[last];
    const int32_t fresh = take(p->free_b, p->ref_b);
    p->ref_b[old] -= 1;
    s->bpages[last] = fresh;
    if (cow) *cow = forkkv_cow_op{old, fresh, s->rows(last)};
  }
  const size_t first_new = s->bpages.size();
  const int32_t nxt = s->len + room;  // start of the first fresh page
  for (int32_t i = 0; i < grow; ++i) {
    s->bpages.push_back(take(p->free_b, p->ref_b));
    s->starts.push_back(nxt + i * kPage);
    if (s->has_res) s->rpages.push_back(take(p->free_r, p->ref_r));
  }
  for (int32_t i = 0; i < n; ++i) {
    const int32_t t = s->len + i;
    size_t j;
    int32_t row;
    if (t < nxt) {
      j = last;
      row = t - s->starts[last];
    } else {
      j = first_new + (t - nxt) / kPage;
      row = (t - nxt) % kPage;
    }
    if (bslots) bslots[i] = s->bpages[j] * kPage + row;
    if (rslots) rslots[i] = s->has_res ? s->rpages[j] * kPage + row : -1;
  }
  s->len = static_cast<int32_t>(new_len);
  if (grow) s->closed = false;
  return FORKKV_OK;
}

int forkkv_seq_append_batch(forkkv_pool* p, const forkkv_seq* seqs, int32_t n, int32_t rows,
                            int32_t* bslots, int32_t* rslots, forkkv_cow_op* cows,
                            int32_t* new_pages) {
  if (!p || n < 0 || rows < 0 || (n > 0 && !seqs)) return FORKKV_EINVAL;
  // validate everything and count the pages the whole batch needs before changing anything
  int64_t need_b = 0, need_r = 0;
  std::vector<char> seen(p->seqs.size(), 0);
  for (int32_t i = 0; i < n; ++i) {
    const Seq* s = get_seq(const_cast<const forkkv_pool*>(p), seqs[i]);
    if (!s || seen[seqs[i]]) return FORKKV_EINVAL;
    seen[seqs[i]] = 1;
    if (s->missing_base()) return FORKKV_ESTATE;
    if (int64_t(s->len) + rows > INT32_MAX / 2) return FORKKV_EINVAL;
    const int32_t room = s->room();
    const int32_t grow = ceil_div(std::max<int64_t>(0, int64_t(rows) - room), kPage);
    const size_t last = s->bpages.empty() ? 0 : s->bpages.size() - 1;
    const bool need_cow =
        rows > 0 && room > 0 && s->rows(last) > 0 && p->ref_b[s->bpages[last]] > 1;
    need_b += grow + (need_cow ? 1 : 0);
    need_r += s->has_res ? grow : 0;
  }
  if (need_b > static_cast<int64_t>(p->free_b.size()) ||
      need_r > static_cast<int64_t>(p->free_r.size()))
    return FORKKV_ENOMEM;
  for (int32_t i = 0; i < n; ++i) {
    const int rc = forkkv_seq_append(p, seqs[i], rows, bslots ? bslots + size_t(i) * rows : nullptr,
                                     rslots ? rslots + size_t(i) * rows : nullptr,
                                     cows ? cows + i : nullptr);
    if (rc != FORKKV_OK) return rc;  // (cannot happen after the checks above)
  }
  if (new_pages) *new_pages = static_cast<int32_t>(need_b);
  return FORKKV_OK;
}

int forkkv_fork(forkkv_pool* p, forkkv_seq parent, int32_t alias_len, forkkv_seq* child,
                forkkv_cow_op* cow) {
  return forkkv_fork_ex(p, parent, alias_len, FORKKV_FORK_PACK, 0, child, cow);
}

int forkkv_fork_ex(forkkv_pool* p, forkkv_seq parent, int32_t alias_len, int32_t mode,
                   int32_t suffix_hint, forkkv_seq* child, forkkv_cow_op* cow) {
  Seq* ps = get_seq(p, parent);
  if (!ps || !child || alias_len < 0 || alias_len > ps->len || suffix_hint < 0 ||
      (mode != FORKKV_FORK_PACK && mode != FORKKV_FORK_FREEZE && mode != FORKKV_FORK_AUTO))
    return FORKKV_EINVAL;
  // whole pages (full, or frozen tails) below alias_len are aliased; the page cut by
  // alias_len, or the parent's open partial last page, is the unaligned tail
  const size_t n_pg = ps->bpages.size();
  size_t whole = 0, tail_j = 0;
  int32_t tail = 0;
  for (size_t j = 0; j < n_pg; ++j) {
    const int32_t st = ps->starts[j], nr = ps->rows(j);
    if (st >= alias_len) break;
    const bool open = j + 1 == n_pg && !ps->closed && nr < kPage;
    if (st + nr <= alias_len && !open) {
      ++whole;
    } else {
      tail_j = j;
      tail = alias_len - st;
      break;
    }
  }
  for (size_t j = 0; j < whole + (tail ? 1 : 0); ++j)
    if (ps->bpages[j] < 0) return FORKKV_ESTATE;
  if (mode == FORKKV_FORK_AUTO)
    mode = (tail + suffix_hint <= kPage || alias_len != ps->len) ? FORKKV_FORK_PACK
                                                                  : FORKKV_FORK_FREEZE;
  if (tail && mode == FORKKV_FORK_FREEZE && alias_len != ps->len) return FORKKV_EINVAL;
  const bool freeze = tail && mode == FORKKV_FORK_FREEZE;
  const int32_t need_b = (tail && !freeze) ? 1 : 0;
  const int32_t need_r = static_cast<int32_t>(whole) + (tail ? 1 : 0);
  if (need_b > static_cast<int32_t>(p->free_b.size()) ||
      need_r > static_cast<int32_t>(p->free_r.size()))
    return FORKKV_ENOMEM;
  clear_cow(cow);
  Seq c;
  c.has_res = true;
  c.bpages.assign(ps->bpages.begin(), ps->bpages.begin() + whole);
  c.starts.assign(ps->starts.begin(), ps->starts.begin() + whole);
  for (int32_t pg : c.bpages) p->ref_b[pg] += 1;
  if (tail) {
    c.starts.push_back(ps->starts[tail_j]);
    if (freeze) {
      const int32_t pg = ps->bpages[tail_j];
      p->ref_b[pg] += 1;
      c.bpages.push_back(pg);
      ps->closed = true;
      c.closed = true;
    } else {
      const int32_t src = ps->bpages[tail_j];
      const int32_t fresh = take(p->free_b, p->ref_b);
      c.bpages.push_back(fresh);
      if (cow) *cow = forkkv_cow_op{src, fresh, tail};
    }
  } else if (whole && ps->rows(whole - 1) < kPage &&
             ps->starts[whole - 1] + ps->rows(whole - 1) == alias_len) {
    c.closed = true;  // ends on a frozen tail
  }
  for (int32_t i = 0; i < need_r; ++i) c.rpages.push_back(take(p->free_r, p->ref_r));
  c.len = alias_len;
  p->seqs.push_back(std::move(c));  // may reallocate: ps is not used after this
  *child = static_cast<forkkv_seq>(p->seqs.size() - 1);
  return FORKKV_OK;
}

int forkkv_seq_free(forkkv_pool* p, forkkv_seq h) {
  Seq* s = get_seq(p, h);
  if (!s) return FORKKV_EINVAL;
  for (int32_t pg : s->bpages)
    if (pg >= 0 && --p->ref_b[pg] == 0) p->free_b.push_back(pg);  // (-1: evicted)
  for (int32_t pg : s->rpages)
    if (--p->ref_r[pg] == 0) p->free_r.push_back(pg);
  s->alive = false;
  s->closed = false;
  s->len = 0;
  s->bpages.clear();
  s->rpages.clear();
  s->starts.clear();
  return FORKKV_OK;
}

int forkkv_evict_bpages(forkkv_pool* p, const int32_t* pages, int32_t n) {
  if (!p || n < 0 || (n > 0 && !pages)) return FORKKV_EINVAL;
  std::vector<char> gone(p->desc.num_bpages, 0);
  for (int32_t i = 0; i < n; ++i) {
    const int32_t pg = pages[i];
    if (pg < 0 || pg >= p->desc.num_bpages || p->ref_b[pg] == 0 || gone[pg]) return FORKKV_EINVAL;
    gone[pg] = 1;
  }
  for (Seq& s : p->seqs) {
    if (!s.alive) continue;
    for (int32_t& pg : s.bpages)
      if (pg >= 0 && gone[pg]) {
        pg = -1;
        ++s.missing;
      }
  }
  for (int32_t i = 0; i < n; ++i) {
    p->ref_b[pages[i]] = 0;
    p->free_b.push_back(pages[i]);
  }
  return FORKKV_OK;
}

int forkkv_refill_bpages(forkkv_pool* p, const forkkv_seq* seqs, int32_t n, int32_t lp0,
                         int32_t lp1, int32_t* new_pages) {
  if (!p || n < 1 || !seqs || lp0 < 0 || lp1 <= lp0) return FORKKV_EINVAL;
  std::vector<Seq*> ss;
  for (int32_t i = 0; i < n; ++i) {
    Seq* s = get_seq(p, seqs[i]);
    if (!s) return FORKKV_EINVAL;
    for (int32_t k = 0; k < i; ++k)
      if (seqs[k] == seqs[i]) return FORKKV_EINVAL;
    ss.push_back(s);
  }
  for (Seq* s : ss) {
    if (static_cast<size_t>(lp1) > s->bpages.size()) return FORKKV_EINVAL;
    for (int32_t j = lp0; j < lp1; ++j)
      if (s->bpages[j] != -1) return FORKKV_EINVAL;
  }
  for (Seq* s : ss)
    for (int32_t j = lp0; j < lp1; ++j)
      if (s->starts[j] != ss[0]->starts[j] || s->rows(j) != ss[0]->rows(j)) return FORKKV_EINVAL;
  if (lp1 - lp0 > static_cast<int32_t>(p->free_b.size())) return FORKKV_ENOMEM;
  for (int32_t j = lp0; j < lp1; ++j) {
    const int32_t pg = take(p->free_b, p->ref_b);
    p->ref_b[pg] = n;
    for (Seq* s : ss) {
      s->bpages[j] = pg;
      --s->missing;
    }
    if (new_pages) new_pages[j - lp0] = pg;
  }
  return FORKKV_OK;
}

int forkkv_seq_len(const forkkv_pool* p, forkkv_seq h, int32_t* len) {
  const Seq* s = get_seq(p, h);
  if (!s || !len) return FORKKV_EINVAL;
  *len = s->len;
  return FORKKV_OK;
}

int forkkv_seq_pages(const forkkv_pool* p, forkkv_seq h, int32_t* n_pages) {
  const Seq* s = get_seq(p, h);
  if (!s || !n_pages) return FORKKV_EINVAL;
  *n_pages = static_cast<int32_t>(s->bpages.size());
  return FORKKV_OK;
}

int forkkv_export_tables(const forkkv_pool* p, const forkkv_seq* seqs, int32_t n,
                         int32_t max_pages, int32_t* btab, int32_t* rtab, int32_t* seq_lens) {
  if (!p || n < 0 || (n > 0 && !seqs) || max_pages < 0) return FORKKV_EINVAL;
  if (n > 0 && (!btab || !rtab)) return FORKKV_EINVAL;
  for (int32_t i = 0; i < n; ++i) {
    const Seq* s = get_seq(p, seqs[i]);
    if (!s || static_cast<int32_t>(s->bpages.size()) > max_pages) return FORKKV_EINVAL;
  }
  for (int32_t i = 0; i < n; ++i) {
    const Seq* s = get_seq(p, seqs[i]);
    int32_t* bt = btab + size_t(i) * max_pages;
    int32_t* rt = rtab + size_t(i) * max_pages;
    std::fill(bt, bt + max_pages, -1);
    std::fill(rt, rt + max_pages, -1);
    std::copy(s->bpages.begin(), s->bpages.end(), bt);
    std::copy(s->rpages.begin(), s->rpages.end(), rt);
    if (seq_lens) seq_lens[i] = s->len;
  }
  return FORKKV_OK;
}

int forkkv_export_starts(const forkkv_pool* p, const forkkv_seq* seqs, int32_t n,
                         int32_t max_pages, int32_t* pstart, int32_t* aligned) {
  if (!p || n < 0 || (n > 0 && (!seqs || !pstart)) || max_pages < 0) return FORKKV_EINVAL;
  for (int32_t i = 0; i < n; ++i) {
    const Seq* s = get_seq(p, seqs[i]);
    if (!s || static_cast<int32_t>(s->starts.size()) > max_pages) return FORKKV_EINVAL;
  }
  int32_t all = 1;
  for (int32_t i = 0; i < n; ++i) {
    const Seq* s = get_seq(p, seqs[i]);
    int32_t* row = pstart + size_t(i) * max_pages;
    std::fill(row, row + max_pages, -1);
    std::copy(s->starts.begin(), s->starts.end(), row);
    if (!s->aligned()) all = 0;
  }
  if (aligned) *aligned = all;
  return FORKKV_OK;
}

int forkkv_pool_stats(const forkkv_pool* p, forkkv_stats* st) {
  if (!p || !st) return FORKKV_EINVAL;
  forkkv_stats z{};
  z.free_bpages = static_cast<int32_t>(p->free_b.size());
  z.free_rpages = static_cast<int32_t>(p->free_r.size());
  z.live_bpages = p->desc.num_bpages - z.free_bpages;
  z.live_rpages = p->desc.num_rpages - z.free_rpages;
  for (int32_t c : p->ref_b) {
    z.bpage_refs += c;
    if (c > 1) ++z.shared_bpages;
  }
  for (int32_t c : p->ref_r) z.rpage_refs += c;
  const size_t e = elem_bytes(p->desc.dtype);
  z.live_bytes_b = int64_t(z.live_bpages) * 2 * p->desc.num_kv_heads * kPage * p->desc.head_dim * e;
  z.live_bytes_r = int64_t(z.live_rpages) * 2 * kPage * p->desc.rank * e;
  *st = z;
  return FORKKV_OK;
}

int forkkv_free_list(const forkkv_pool* p, int32_t which, int32_t* out, int32_t cap, int32_t* n) {
  if (!p || !n || (which != 0 && which != 1) || cap < 0) return FORKKV_EINVAL;
  const std::deque<int32_t>& fl = which == 0 ? p->free_b : p->free_r;
  *n = static_cast<int32_t>(fl.size());
  if (out) {
    int32_t i = 0;
    for (auto it = fl.begin(); it != fl.end() && i < cap; ++it) out[i++] = *it;
  }
  return FORKKV_OK;
}

int forkkv_refcounts(const forkkv_pool* p, int32_t which, int32_t* out) {
  if (!p || !out || (which != 0 && which != 1)) return FORKKV_EINVAL;
  const std::vector<int32_t>& r = which == 0 ? p->ref_b : p->ref_r;
  std::copy(r.begin(), r.end(), out);
  return FORKKV_OK;
}

int forkkv_cow_copy(forkkv_pool* p, const forkkv_cow_op* ops, int32_t n_ops, hipStream_t stream) {
  if (!p || n_ops < 0 || (n_ops > 0 && !ops)) return FORKKV_EINVAL;
  if (!p->bcache) return FORKKV_ESTATE;
  for (int32_t i = 0; i < n_ops; ++i) {
    const forkkv_cow_op& o = ops[i];
    if (o.n_rows == 0) continue;
    if (o.n_rows < 0 || o.n_rows > kPage || o.src_bpage < 0 || o.dst_bpage < 0 ||
        o.src_bpage >= p->desc.num_bpages || o.dst_bpage >= p->desc.num_bpages ||
        o.src_bpage == o.dst_bpage)
      return FORKKV_EINVAL;
  }
  for (int32_t i = 0; i < n_ops; ++i) {
    const forkkv_cow_op& o = ops[i];
    if (o.n_rows == 0) continue;
    if (forkkv::launch_cow_copy(p->bcache, p->desc.dtype, p->desc.num_kv_heads,
                                p->desc.head_dim, o.src_bpage, o.dst_bpage, o.n_rows,
                                stream) != hipSuccess)
      return FORKKV_EHIP;
  }
  return FORKKV_OK;
}

}  // extern "C"
