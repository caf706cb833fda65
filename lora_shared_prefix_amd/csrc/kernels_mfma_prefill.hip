// MFMA (matrix-core) chunked-prefill ResidualAttention kernel for gfx950, bf16 storage,
// d = 128, r = 16, page size 16 (after the chunk rows have been stored).
//
#include "kernels_mfma_common.h"

namespace forkkv {
namespace {

// Chunked prefill (after the chunk rows have been stored): one workgroup per (agent, KV
// head, block of 256 query rows), rows = (query, head within the GQA group) flattened; 8
// waves of 32 rows.  Each iteration covers two pages (32 keys).  The eight waves rebuild
// the agent's full keys K = bK + RoPE(s * rK B_k) of both pages together (wave w: page
// w / 4, reconstruction tiles w % 4 and w % 4 + 4 -- a RoPE partner pair) into LDS in
// score-MFMA operand order and stage both value tiles; then every wave scores its rows,
// updates its online softmax and accumulates acc += P bV and acc_r += P rV with K = 32
// keys per MFMA; B_v is applied once in the epilogue (ForkKV study note,
// "7. 实现 cross-reference"; Penelope review, 部件二, for the write-then-attend order and
// the causal mask that includes the query itself).
constexpr int kPfWaves = 8;
constexpr int kPfThreads = 64 * kPfWaves;
constexpr int kPfRowsPerWave = 32;
constexpr int kPfRows = kPfRowsPerWave * kPfWaves;  // rows per workgroup

// cos and sin (fp64) of a moderate angle (here reduced to at most 2 pi before the call):
// a reduction by a small number q of quarter turns leaves t = x - q pi/2 in
// [-pi/4, pi/4] (pi/2 in two parts, a fused step each, so t is exact to rounding), where the
// Taylor series of sin t through t^15 and of cos t through t^16 are exact to below 1e-16.
// Far lighter in registers than the general library routine, which must also reduce huge
// arguments.
__device__ __forceinline__ void sincos_turn(double x, double& s, double& c) {
  constexpr double kHalfPiHi = 1.5707963267948966192;
  constexpr double kHalfPiLo = 6.123233995736766036e-17;
  const double q = rint(x * 0.63661977236758134308);  // x / (pi/2), rounded
  const double t = fma(-q, kHalfPiLo, fma(-q, kHalfPiHi, x));
  const double u = t * t;
  double ps = -1.0 / 1307674368000.0;  // -1/15!
  ps = fma(ps, u, 1.0 / 6227020800.0);
  ps = fma(ps, u, -1.0 / 39916800.0);
  ps = fma(ps, u, 1.0 / 362880.0);
  ps = fma(ps, u, -1.0 / 5040.0);
  ps = fma(ps, u, 1.0 / 120.0);
  ps = fma(ps, u, -1.0 / 6.0);
  const double st = fma(ps * u, t, t);
  double pc = 1.0 / 20922789888000.0;  // 1/16!
  pc = fma(pc, u, -1.0 / 87178291200.0);
  pc = fma(pc, u, 1.0 / 479001600.0);
  pc = fma(pc, u, -1.0 / 3628800.0);
  pc = fma(pc, u, 1.0 / 40320.0);
  pc = fma(pc, u, -1.0 / 720.0);
  pc = fma(pc, u, 1.0 / 24.0);
  pc = fma(pc, u, -0.5);
  const double ct = fma(pc, u, 1.0);
  const int k = static_cast<int>(q) & 3;  // sin and cos of t + k pi/2
  s = k == 0 ? st : k == 1 ? ct : k == 2 ? -st : -ct;
  c = k == 0 ? ct : k == 1 ? -st : k == 2 ? -ct : st;
}

// kMap: the agents hold frozen tails, so pages start where the page start table says (the
// slot map) and a page may hold fewer than 16 rows; without it page lp starts at lp * P and
// none of that bookkeeping is compiled in.
template <bool kMap>
__global__ void __launch_bounds__(kPfThreads) __attribute__((amdgpu_waves_per_eu(2)))
prefill_mfma_kernel(PrefillParams p, int n_rblocks) {
  __shared__ __align__(16) uint4 s_k[2][2][4 * 64];   // [buf][page][chunk * 64 + lane]
  // value operands in PV-MFMA order: [buf][tile t * 64 + reader lane], the 16 bytes a lane
  // feeds one K = 32 MFMA (8 bytes of page 0, then 8 of page 1)
  __shared__ __align__(16) uint4 s_v[2][8 * 64];
  __shared__ __align__(16) uint4 s_rv[2][64];         // [buf][lane], same page halves
  __shared__ int s_miss[2][2];                          // [buf][page]: base page missing
  __shared__ int s_pos[2][2], s_vrows[2][2];            // [buf][page]: start, valid rows
  __shared__ double s_om[kD / 2];                        // RoPE frequencies w_j (fp64)
  // the ones operand of the denominator product, read from here at each use: held in
  // registers it would be rebuilt by copies wherever its registers serve as temporaries
  __shared__ __align__(16) uint4 s_ones;
  // cos and sin of k * 32 w_j (k < 32: the iterations since the last exact anchor)
  __shared__ __align__(16) float s_ct[32][kD / 2], s_st[32][kD / 2];
  const int Hkv = p.num_kv_heads, G = p.group, Hq = p.num_q_heads, C = p.chunk_len;
  // the workgroups of one KV head share an XCD (block ids are dealt round robin over the
  // 8 XCDs), so the shared prefix of that head streams through one L2
  const int b = blockIdx.x;
  const int h = b % Hkv;
  const int sblk = b / Hkv;
  const int rb = sblk % n_rblocks, a = sblk / n_rblocks;
  if (a >= p.n_agents) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pg = w >> 2, tp = w & 3;  // staging role: page of the pair, tile pair / quarter
  const int col = lane & 15, g4 = lane >> 4;
  const int total_rows = C * G;
  const int row0 = rb * kPfRows;
  const int last_row = min(total_rows, row0 + kPfRows) - 1;
  // positions increase along the chunk: the block's queries span first_pos .. last_pos
  const int first_pos = row_position(p, a, row0 / G);
  const int last_pos = row_position(p, a, last_row / G);
  const int end_pos = row_position(p, a, C - 1) + 1;  // rows at or past end_pos: unwritten
  // pages any row of the block sees
  const int lp_end = page_of(kMap ? p.pstart : nullptr, p.max_pages, a, last_pos) + 1;
  const int n_it = (lp_end + 1) / 2;
  const int n = Hkv * kD;
  const uint16_t* bcache = static_cast<const uint16_t*>(p.bcache);
  const uint16_t* rcache = static_cast<const uint16_t*>(p.rcache);
  const uint16_t* q = static_cast<const uint16_t*>(p.q);
  const uint16_t* Bk = static_cast<const uint16_t*>(p.Bk);
  const size_t tile = size_t(kPage) * kD;

  // this wave's two row tiles: row = row0 + 32 w + 16 rt + col (as a score column)
  bf8 qv[2][4];
  int qpos[2];
  bool rok[2];
  for (int rt = 0; rt < 2; ++rt) {
    const int row = row0 + kPfRowsPerWave * w + 16 * rt + col;
    rok[rt] = row < total_rows;
    const int qi = rok[rt] ? row / G : 0, g = rok[rt] ? row % G : 0;
    qpos[rt] = row_position(p, a, qi);
    const uint16_t* qrow = q + ((size_t(a) * C + qi) * Hq + h * G + g) * kD;
    for (int c = 0; c < 4; ++c) {
      U4 t;
      t.u = rok[rt] ? *reinterpret_cast<const uint4*>(qrow + 32 * c + 8 * g4) : make_uint4(0, 0, 0, 0);
      qv[rt][c] = t.b;
    }
  }
  // B_k A operands of this wave's reconstruction tiles T = tp and tp + 4
  s4 bkop[2];
  for (int u = 0; u < 2; ++u) {
    const int T = tp + 4 * u;
    const int dim = h * kD + perm_dim(T, col);
    const uint16_t* src = Bk + size_t(a) * kR * n + dim;
    U2 v;
    v.u.x = uint32_t(src[size_t(4 * g4) * n]) | (uint32_t(src[size_t(4 * g4 + 1) * n]) << 16);
    v.u.y = uint32_t(src[size_t(4 * g4 + 2) * n]) | (uint32_t(src[size_t(4 * g4 + 3) * n]) << 16);
    bkop[u] = v.s;
  }
  // RoPE of this lane's 4 frequencies j_i = perm_dim(tp, 4 g4 + i) = f0 + i at position
  // t = 16 (2 it + pg) + col: exact (fp64-reduced) at an anchor every 32 iterations, and in
  // between the anchor's angle plus k steps of 32 w_j (one angle addition with the table
  // entry k, so no error accumulates between anchors).
  if (tid < kD / 2)
    s_om[tid] = exp2(-2.0 * tid / kD * log2(static_cast<double>(p.rope_theta)));
  if (tid == 0) s_ones = make_uint4(0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u);
  __syncthreads();
  for (int x = tid; x < 32 * (kD / 2); x += kPfThreads) {
    const int k = x / (kD / 2), j = x % (kD / 2);
    double ang = static_cast<double>(2 * kPage * k) * s_om[j];
    ang = fma(-kTwoPi, floor(ang * kInvTwoPi), ang);
    double sv, cv;
    sincos_turn(ang, sv, cv);
    s_ct[k][j] = static_cast<float>(cv);
    s_st[k][j] = static_cast<float>(sv);
  }
  __syncthreads();
  const int f0 = perm_dim(tp, 4 * g4);
  float rc[4], rs[4];  // the anchor's cos and sin, times the adapter scale s
  int kk = 0;          // iterations since the anchor (wave-uniform, < 32)
  int next_base = pg * kPage;  // the page start the angles stand at
  // exact cos/sin (fp64-reduced angle) of this lane's key position base + col
  auto anchor_at = [&](int base) {
    for (int i = 0; i < 4; ++i) {
      double ang = static_cast<double>(base + col) * s_om[f0 + i];
      ang = fma(-kTwoPi, floor(ang * kInvTwoPi), ang);
      double sv, cv;
      sincos_turn(ang, sv, cv);
      rc[i] = static_cast<float>(cv) * p.lora_scale;
      rs[i] = static_cast<float>(sv) * p.lora_scale;
    }
    kk = 0;
  };

  // global pieces of this wave's staging role, held in registers one iteration ahead
  struct PfBuf {
    uint2 bk[2];  // base keys under this lane's two reconstruction tiles (4 dims each)
    uint2 rk;     // key-residual B operand of page pg
    uint4 v;      // quarter tp of page pg's value tile (operand pieces of lanes 2l, 2l+1)
    uint2 rv;     // value-residual operand of page pg (staged by the tp == 0 waves)
    bool miss;    // page pg's base page is missing (evicted): its keys take no part
    int pos, nx;  // with the slot map: the page's start and the next page's (-1: none)
  };
  // Page ids: lane i holds the ids of this wave's page at iteration 64 k + i (block k),
  // checked against the pools once here (a missing or out-of-pool page is -1); a page's ids
  // then come from a readlane.  A missing base page is read from page 0 (any in-pool page)
  // and then masked; a missing residual page reads the zero page.
  int ids_b = -1, ids_r = -1;
  int ids_st = 0, ids_nx = 0;  // with the slot map: start of the page and of the next one
  auto fetch_ids = [&](int blk) {
    const int lp = min(2 * (64 * blk + lane) + pg, lp_end - 1);
    const int bp = p.btab[size_t(a) * p.max_pages + lp];
    const int rp = p.rtab[size_t(a) * p.max_pages + lp];
    ids_b = (bp >= 0 && bp < p.num_bpages) ? bp : -1;
    ids_r = (rp >= 0 && rp < p.num_rpages) ? rp : -1;
    if constexpr (kMap) {
      const int32_t* row = p.pstart + size_t(a) * p.max_pages;
      ids_st = row[lp];
      ids_nx = lp + 1 < p.max_pages ? row[lp + 1] : -1;
    }
  };
  auto load = [&](int it, PfBuf& B) {
    if ((it & 63) == 0) fetch_ids(it >> 6);  // wave-uniform
    const int ib = __builtin_amdgcn_readlane(ids_b, it & 63);
    const int ir = __builtin_amdgcn_readlane(ids_r, it & 63);
    B.miss = ib < 0;
    if constexpr (kMap) {
      B.pos = __builtin_amdgcn_readlane(ids_st, it & 63);
      B.nx = __builtin_amdgcn_readlane(ids_nx, it & 63);
    }
    const size_t pb = max(ib, 0);
    const uint16_t* kt = bcache + (pb * 2 * Hkv + h) * tile;
    const uint16_t* vt = bcache + (pb * 2 * Hkv + Hkv + h) * tile;
    const uint16_t* rb_ = ir >= 0 ? rcache + size_t(ir) * 2 * kPage * kR : g_zero_res;
    for (int u = 0; u < 2; ++u) {
      // dims perm_dim(T, 4 g4 + i), i = 0..3: 4 consecutive dims of one 8-dim block
      const int x0 = perm_dim(tp + 4 * u, 4 * g4);
      B.bk[u] = *reinterpret_cast<const uint2*>(kt + (x0 / 8) * 128 + col * 8 + x0 % 8);
    }
    B.rk = *reinterpret_cast<const uint2*>(rb_ + 4 * lane);
    B.v = *reinterpret_cast<const uint4*>(vt + 512 * tp + 8 * lane);
    B.rv = *reinterpret_cast<const uint2*>(rb_ + kPage * kR + 4 * lane);
  };

  f4 acc[2][8];
  f4 accr[2];
  float m_run[2] = {-INFINITY, -INFINITY};
  // softmax denominators: a matrix product of the bf16 probabilities with a ones operand,
  // so every lane of a row holds that row's sum (the same rounded weights as acc)
  f4 l_acc[2] = {f4{0.f, 0.f, 0.f, 0.f}, f4{0.f, 0.f, 0.f, 0.f}};
  // m_run + 8 (the rescale threshold) and the reference the exponents are taken against
  // (-1e30 while a row has no key yet: no -inf - -inf), both updated only on a rescale;
  // m_raw is the threshold in raw-score units (m_thr / qscale, qscale > 0), so that a
  // page's test costs no multiplication
  float m_thr[2] = {-INFINITY, -INFINITY}, m_ref[2] = {-1e30f, -1e30f};
  float m_raw[2] = {-INFINITY, -INFINITY};
  for (int rt = 0; rt < 2; ++rt) {
    for (int t = 0; t < 8; ++t) acc[rt][t] = f4{0.f, 0.f, 0.f, 0.f};
    accr[rt] = f4{0.f, 0.f, 0.f, 0.f};
  }
  const float qscale = p.sm_scale_log2, inv_qscale = 1.f / qscale;
  auto m2 = [](int tv, uint32_t& lo, uint32_t& hi) {
    if (tv < 4) {
      if (tv <= 0) lo = 0;
      else if (tv == 1) lo &= 0xffffu;
      if (tv <= 2) hi = 0;
      else if (tv == 3) hi &= 0xffffu;
    }
  };

  auto stage = [&](int it, const PfBuf& B) {
    const int buf = it & 1;
    const int lp = 2 * it + pg;
    // the page's first position; the recurrence below stands at next_base, and is re-anchored
    // (fp64) every 32 iterations (by the loop below) and wherever a page does not start where
    // it stands (a frozen tail in between)
    const int base = kMap ? B.pos : lp * kPage;
    if (kMap && base != next_base) anchor_at(base);
    next_base = base + 2 * kPage;
    // this iteration's cos and sin: the anchor's angle plus kk steps
    const float4 ct = *reinterpret_cast<const float4*>(&s_ct[kk][f0]);
    const float4 st = *reinterpret_cast<const float4*>(&s_st[kk][f0]);
    ++kk;
    const float tc[4] = {ct.x, ct.y, ct.z, ct.w}, ts[4] = {st.x, st.y, st.z, st.w};
    float cc[4], ss[4];
    for (int i = 0; i < 4; ++i) {
      cc[i] = __builtin_fmaf(rc[i], tc[i], -rs[i] * ts[i]);
      ss[i] = __builtin_fmaf(rs[i], tc[i], rc[i] * ts[i]);
    }
    // rebuild this wave's two key tiles of page pg: K = bK + RoPE(s * rK B_k)
    U2 rk;
    rk.u = B.rk;
    f4 d0 = mfma16(bkop[0], rk.s, f4{0.f, 0.f, 0.f, 0.f});
    f4 d1 = mfma16(bkop[1], rk.s, f4{0.f, 0.f, 0.f, 0.f});
    float k0[4], k1[4];
    const uint32_t bw0[2] = {B.bk[0].x, B.bk[0].y}, bw1[2] = {B.bk[1].x, B.bk[1].y};
    for (int i = 0; i < 4; ++i) {
      const float x = d0[i], y = d1[i];
      const float b0 = __uint_as_float((i & 1) ? (bw0[i >> 1] & 0xffff0000u) : (bw0[i >> 1] << 16));
      const float b1 = __uint_as_float((i & 1) ? (bw1[i >> 1] & 0xffff0000u) : (bw1[i >> 1] << 16));
      // two fused steps each: bK + x c - y s and bK + y c + x s
      k0[i] = __builtin_fmaf(x, cc[i], __builtin_fmaf(-y, ss[i], b0));
      k1[i] = __builtin_fmaf(y, cc[i], __builtin_fmaf(x, ss[i], b1));
    }
    // tile T = tp lands in chunk tp/2, half (tp & 1); tile tp + 4 in chunk tp/2 + 2
    uint2* sk = reinterpret_cast<uint2*>(&s_k[buf][pg][0]);
    sk[((tp >> 1) * 64 + lane) * 2 + (tp & 1)] =
        make_uint2(pack_bf16x2(k0[0], k0[1]), pack_bf16x2(k0[2], k0[3]));
    sk[(((tp >> 1) + 2) * 64 + lane) * 2 + (tp & 1)] =
        make_uint2(pack_bf16x2(k1[0], k1[1]), pack_bf16x2(k1[2], k1[3]));
    // Value rows past the last stored position (or past the pages this block needs) hold
    // arbitrary bytes (even NaN); a zero probability times NaN is NaN, so they are zeroed.
    // The 16 bytes this lane stages are the operand pieces of reader lanes 2l and 2l+1
    // (tokens 4 g .. 4 g + 3, g = ((2l) mod 64) / 16); its value-residual piece is its own.
    // rows of the page that hold keys: up to the next page's start (a frozen tail holds fewer
    // than 16) and up to the last stored position
    int last = (lp < lp_end && !B.miss) ? end_pos - base : 0;
    if (kMap && B.nx >= 0) last = min(last, B.nx - base);
    uint4 v = B.v;
    uint2 rv = B.rv;
    if (last < kPage) {  // wave-uniform: the pages at the end of the sequence, missing pages
      const int tvv = last - 4 * (((2 * lane) & 63) >> 4);
      m2(tvv, v.x, v.y);
      m2(tvv, v.z, v.w);
      m2(last - 4 * g4, rv.x, rv.y);
    }
    // v holds reader lanes 2l and 2l + 1 of tile t = 2 tp + l / 32 (l = lane mod 32): each
    // 8-byte piece goes to this page's half of that reader's slot
    {
      uint2* sv = reinterpret_cast<uint2*>(&s_v[buf][0]);
      const int slot = (2 * tp + (lane >> 5)) * 64 + ((2 * lane) & 63);
      sv[2 * slot + pg] = make_uint2(v.x, v.y);
      sv[2 * (slot + 1) + pg] = make_uint2(v.z, v.w);
    }
    if (tp == 0) {
      reinterpret_cast<uint2*>(&s_rv[buf][0])[2 * lane + pg] = rv;
      if (lane == 0) {
        s_miss[buf][pg] = B.miss;
        s_pos[buf][pg] = base;
        s_vrows[buf][pg] = min(max(last, 0), kPage);
      }
    }
  };

  auto compute = [&](int it) {
    const int buf = it & 1;
    // Row tile 0's scores first, then row tile 1's; then per row tile its softmax and its
    // PV products, so that the vector work of one row tile is issued while the matrix
    // cores run the other's products.
    f4 sc4[2][2];  // [row tile][page]
    {
      U4 kop[2][4];
      for (int pgi = 0; pgi < 2; ++pgi)
        for (int c = 0; c < 4; ++c) kop[pgi][c].u = s_k[buf][pgi][c * 64 + lane];
      for (int rt = 0; rt < 2; ++rt)
        for (int pgi = 0; pgi < 2; ++pgi) {
          f4 sv = f4{0.f, 0.f, 0.f, 0.f};
          for (int c = 0; c < 4; ++c) sv = mfma32(kop[pgi][c].b, qv[rt][c], sv);
          sc4[rt][pgi] = sv;
        }
    }
    // Both pages exist and lie entirely before the block's first query position (every key
    // precedes every query):
    // no mask at all.  Rows past the chunk have zero q and are never written, so they need
    // none either.  (Wave-uniform.)
    const bool miss[2] = {s_miss[buf][0] != 0, s_miss[buf][1] != 0};  // wave-uniform
    bool unmasked = 2 * it + 1 < lp_end && (2 * it + 1) * kPage + kPage - 1 < first_pos &&
                    !miss[0] && !miss[1];
    int pbase[2] = {2 * it * kPage, (2 * it + 1) * kPage}, pvr[2] = {kPage, kPage};
    if constexpr (kMap) {  // starts and valid rows of the pair, as staged
      for (int pgi = 0; pgi < 2; ++pgi) {
        pbase[pgi] = s_pos[buf][pgi];
        pvr[pgi] = s_vrows[buf][pgi];
      }
      unmasked = 2 * it + 1 < lp_end && pvr[0] == kPage && pvr[1] == kPage &&
                 pbase[1] + kPage - 1 < first_pos && !miss[0] && !miss[1];
    }
    for (int rt = 0; rt < 2; ++rt) {
      // raw scores (q.k); the softmax scale (> 0, log2 units) is applied inside the exp
      float sc[8];
      if (unmasked) {
        for (int pgi = 0; pgi < 2; ++pgi)
          for (int i = 0; i < 4; ++i) sc[4 * pgi + i] = sc4[rt][pgi][i];
      } else {
        for (int pgi = 0; pgi < 2; ++pgi) {
          const int lp = 2 * it + pgi;
          // keys i <= lim of this lane's four: causal (key position <= query position), and
          // with the slot map only the page's valid rows
          int lim = (lp < lp_end && !miss[pgi]) ? qpos[rt] - pbase[pgi] - 4 * g4 : -1;
          if constexpr (kMap) lim = min(lim, pvr[pgi] - 1 - 4 * g4);
          for (int i = 0; i < 4; ++i) sc[4 * pgi + i] = i <= lim ? sc4[rt][pgi][i] : -INFINITY;
        }
      }
      // Lazy rescale: the running maximum moves only when a row's maximum passes it by more
      // than 8 (a factor 256 of headroom in the fp32 sums).  A row's maximum passes the
      // threshold exactly when one of its four lanes' own maxima does, so the cross-lane
      // reduction is needed only then.
      float lmax = -INFINITY;
      for (int e = 0; e < 8; ++e) lmax = fmaxf(lmax, sc[e]);
      // (an m_raw rounded low only adds a rescale that changes nothing; rounded high it lets
      // an exponent reach 8 plus a rounding error, inside the headroom)
      if (__builtin_amdgcn_ballot_w64(lmax > m_raw[rt]) != 0) {
        const float pmax = max_over_rows(lmax) * qscale;
        const bool grow = pmax > m_thr[rt];
        const float m_new = grow ? pmax : m_run[rt];
        const float alpha = __builtin_amdgcn_exp2f(m_run[rt] - m_new);
        l_acc[rt] *= alpha;
        for (int t = 0; t < 8; ++t) acc[rt][t] *= alpha;
        accr[rt] *= alpha;
        m_run[rt] = m_new;
        m_thr[rt] = m_new + 8.f;
        m_raw[rt] = m_thr[rt] * inv_qscale;
        m_ref[rt] = max2(m_new, -1e30f);
      }
      float pr[8];
      for (int e = 0; e < 8; ++e) pr[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[e], qscale, -m_ref[rt]));
      U4 pb;  // P^T operand, K = 32 keys: elements 0..3 page 0, 4..7 page 1
      pb.u = make_uint4(pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3]),
                        pack_bf16x2(pr[4], pr[5]), pack_bf16x2(pr[6], pr[7]));
      for (int t = 0; t < 8; ++t) {
        U4 vop;
        vop.u = s_v[buf][t * 64 + lane];
        acc[rt][t] = mfma32(vop.b, pb.b, acc[rt][t]);
      }
      U4 rvop;
      rvop.u = s_rv[buf][lane];
      accr[rt] = mfma32(rvop.b, pb.b, accr[rt]);
      U4 ones;
      ones.u = s_ones;
      l_acc[rt] = mfma32(ones.b, pb.b, l_acc[rt]);
    }
  };

  // The register buffer is refilled for iteration it + 1 as soon as iteration it has been
  // staged, so those loads fly during the whole compute phase.  Two LDS
  // buffers alternate, so one barrier per iteration suffices: iteration it + 1 stages into
  // the other buffer, and iteration it + 2 waits behind the next barrier.
  // The iterations run in blocks of 32, each starting from an exact (fp64) anchor, so the
  // page loop itself carries only the recurrence.
  PfBuf pb_;
  load(0, pb_);
  for (int it0 = 0; it0 < n_it; it0 += 32) {
    next_base = kMap ? pb_.pos : (2 * it0 + pg) * kPage;
    anchor_at(next_base);
    const int it1 = min(it0 + 32, n_it);
    for (int it = it0; it < it1; ++it) {
      stage(it, pb_);
      load(min(it + 1, n_it - 1), pb_);
      __syncthreads();
      compute(it);
    }
  }

  // ---- epilogue: o = (acc + s * acc_r B_v) / l, B_v applied once ------------------------
  __syncthreads();  // the staging buffers are reused below
  float* s_accr = reinterpret_cast<float*>(&s_v[0][0]);          // [wave][16 ranks][32 rows]
  float* s_bv = reinterpret_cast<float*>(&s_k[0][0][0]);         // [16 ranks][128 dims]
  const uint16_t* Bv = static_cast<const uint16_t*>(p.Bv);
  for (int x = tid; x < kR * kD; x += kPfThreads) {
    const int k = x / kD, dim = x % kD;
    s_bv[x] = __uint_as_float(uint32_t(Bv[size_t(a) * kR * n + size_t(k) * n + h * kD + dim]) << 16);
  }
  for (int rt = 0; rt < 2; ++rt)
    for (int i = 0; i < 4; ++i) s_accr[(w * kR + 4 * g4 + i) * 32 + 16 * rt + col] = accr[rt][i];
  __syncthreads();
  uint16_t* out = static_cast<uint16_t*>(p.out);
  for (int rt = 0; rt < 2; ++rt) {
    const float l = l_acc[rt][0];
    if (!rok[rt]) continue;
    const int row = row0 + kPfRowsPerWave * w + 16 * rt + col;
    const int qi = row / G, g = row % G;
    float ar[kR];
    for (int k = 0; k < kR; ++k) ar[k] = s_accr[(w * kR + k) * 32 + 16 * rt + col];
    const float inv = l > 0.f ? 1.f / l : 0.f;
    uint16_t* orow = out + ((size_t(a) * C + qi) * Hq + h * G + g) * kD;
    for (int t = 0; t < 8; ++t) {
      float o[4];
      for (int i = 0; i < 4; ++i) {
        const int dim = 16 * t + 4 * g4 + i;
        float res = 0.f;
        for (int k = 0; k < kR; ++k) res += ar[k] * s_bv[k * kD + dim];
        o[i] = (acc[rt][t][i] + p.lora_scale * res) * inv;
      }
      *reinterpret_cast<uint2*>(orow + 16 * t + 4 * g4) =
          make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
    }
  }
}

}  // namespace

hipError_t launch_prefill_mfma(const PrefillParams& p, const int32_t*, hipStream_t s) {
  const int n_rblocks = (p.chunk_len * p.group + kPfRows - 1) / kPfRows;
  const int blocks = p.num_kv_heads * n_rblocks * p.n_agents;
  if (p.pstart)
    hipLaunchKernelGGL(prefill_mfma_kernel<true>, dim3(blocks), dim3(kPfThreads), 0, s, p,
                       n_rblocks);
  else
    hipLaunchKernelGGL(prefill_mfma_kernel<false>, dim3(blocks), dim3(kPfThreads), 0, s, p,
                       n_rblocks);
  return hipGetLastError();
}


}  // namespace forkkv
