// MFMA (matrix-core) split-K decode kernel of ResidualAttention for gfx950, bf16 storage,
// d = 128, r = 16, page size 16: up to 16 query columns (agents x GQA group) per wave; with
// decode-with-append it also stores the new rows first.
//
// ForkKV study note, "7. 实现 cross-reference" (kernel; core barriers (1) and (2)) and
// "4. 作者证明" (Eq.(4), reproduction checks 3, 4 and 6): for each page the key of every
// aliasing agent is rebuilt on chip as bK + RoPE(s * rK B_k) -- RoPE after the
// up-projection -- and the value path keeps a rank-r accumulator acc_r, rescaled with the
// base accumulator, so that B_v is applied once, after the loop (combine kernel).
//
// Work layout (one workgroup = one KV head x one plan item = a run of logical pages that
// all the item's agents map to the same physical base pages):
//   * the base key/value tile of a page is loaded once per agent group and scored for all
//     the group's agents and GQA heads: S_base = bK Q^T is one MFMA tile for all of them;
//   * the residual key rK B_k is an MFMA (K = rank = 16) per agent and page; its result
//     lands with the RoPE partners (dims j and j + 64) in the same lane, so the deferred
//     rotation is applied in registers; S_a = S_base + RoPE(K_res,a) Q^T (MFMA again);
//   * online softmax per query column with wave shuffles for the max and sum;
//   * acc^T += bV^T P^T (shared by the group) and acc_r^T += rV_a^T P_a^T (per agent);
//   * waves split the item's agents into groups and its pages into sub-ranges; partial
//     states of one group are merged in LDS with the log-sum-exp rule, then written as
//     one split-K partial per (item, agent, q head).
//
// (MFMA lane layouts and the shared helpers: kernels_mfma_common.h.)
#include "kernels_mfma_common.h"

namespace forkkv {
namespace {

constexpr int kWaves = 4;     // waves per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kTrigPad = 72;  // padded row of the static in-page trig table (fp16)

// LDS layout (bytes)
constexpr int kBkBytes = kItemAgents * 8 * 64 * 8;      // [agent][tile][lane][4 bf16]
constexpr int kTrigBytes = 2 * kPage * kTrigPad * 2;    // cos, sin: [c][j] (scaled by s)
constexpr int kPageTrigBytes = kWaves * 2 * 64 * 2;     // per wave: cos[64], sin[64]
constexpr int kQhBytes = kWaves * 4 * 64 * 16;          // per wave: bf16 q, [chunk][lane]
constexpr int kMergeVecs = 1 + 8 + 1;                   // (m, l, -, -) | acc[8] | accr (float4)
constexpr int kMergeBytes = kMergeVecs * kWaves * 64 * 16;
constexpr int kLdsMain = kBkBytes + kTrigBytes + kPageTrigBytes + kQhBytes;
constexpr int kLdsBytes = kLdsMain > kMergeBytes ? kLdsMain : kMergeBytes;

// A: agents per group (columns = agents x G <= 16).  kMap: the batch holds a frozen tail and
// page starts come from the start table (the slot map); without it page lp starts at lp * P
// and none of that bookkeeping is compiled in.
template <int A, bool kMap>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
decode_mfma_kernel(DecodeParams p, int n_items) {
  __shared__ __align__(16) unsigned char lds[kLdsBytes];
  const int Hkv = p.num_kv_heads;
  // XCD-aware block order: consecutive blocks run on different XCDs (round robin), so the
  // KV heads of one item are given block ids that share an XCD (and its L2), where the
  // residual pages -- common to all heads -- are then fetched once.
  const int b = blockIdx.x;
  const int xcd = b & 7, s = b >> 3;
  const int h = s % Hkv;
  const int item = xcd + 8 * (s / Hkv);
  // The grid covers the plan's item capacity and the items section has room for that many
  // records, zero past the live count (the whole section is uploaded): a record with no
  // agents is an empty item, so the live count itself is never read.  The agent and slot
  // entries are read with constant indices (a few wide scalar loads instead of a chain of
  // dependent ones) and picked later by wave-uniform selects.
  if (item >= n_items) return;
  const int32_t* it = p.plan + p.off_items + item * kItemInts;
  int ia[kItemAgents], is[kItemAgents];
#pragma unroll
  for (int k = 0; k < kItemAgents; ++k) {
    ia[k] = it[4 + k];
    is[k] = it[4 + kItemAgents + k];
  }
  const int lp0 = it[0], np = it[1], na = it[2], holds_last = it[3];
  // (the empty statements take the record's values as operands, so that all of its loads are
  // issued before the test below -- one memory round trip -- rather than sunk past it)
  asm volatile("" : : "s"(lp0), "s"(np), "s"(na), "s"(holds_last));
#pragma unroll
  for (int k = 0; k < kItemAgents; ++k) asm volatile("" : : "s"(ia[k]), "s"(is[k]));
  if (na <= 0) return;  // past the live count

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform per wave
  const int col = lane & 15, g4 = lane >> 4;
  const int G = p.group, Hq = p.num_q_heads;
  const int n_groups = (na + A - 1) / A;
  const int n_sub = kWaves / n_groups;  // >= 1 (the plan keeps na <= 4A)
  const int gi = w % n_groups, si = w / n_groups;
  const bool active = si < n_sub;
  const int j0 = gi * A;
  const int na_g = min(A, na - j0);

  const uint16_t* bcache = static_cast<const uint16_t*>(p.bcache);
  const uint16_t* rcache = static_cast<const uint16_t*>(p.rcache);
  const uint16_t* Bk = static_cast<const uint16_t*>(p.Bk);
  const uint16_t* q = static_cast<const uint16_t*>(p.q);
  const int n = Hkv * kD;

  uint2* bkl = reinterpret_cast<uint2*>(lds);                          // [j][T][lane]
  _Float16* trig_c = reinterpret_cast<_Float16*>(lds + kBkBytes);      // [c][kTrigPad]
  _Float16* trig_s = trig_c + kPage * kTrigPad;
  _Float16* ptrig = reinterpret_cast<_Float16*>(lds + kBkBytes + kTrigBytes) + w * 128;
  uint4* qb_lds =
      reinterpret_cast<uint4*>(lds + kBkBytes + kTrigBytes + kPageTrigBytes) + w * 4 * 64;

  // ---- prologue ---------------------------------------------------------------------------
  // Every load that depends on nothing else is issued first (this wave's query columns, the
  // group's agents and lengths, the page ids of the sub-range, the B_k rows), so that their
  // latencies overlap; the first page's key tiles follow as soon as its ids are in, and the
  // on-chip set-up (B_k packed into operand order, trig tables) runs while they are in flight.
  const int pps = (np + n_sub - 1) / n_sub;
  const int lpa = active ? lp0 + si * pps : 0;
  const int lpb = active ? min(lp0 + np, lpa + pps) : 0;
  const size_t tile = size_t(kPage) * kD;  // elements per (page, plane, head) tile

  // ---- this wave's agents and query columns ------------------------------------------------
  int agent[A], slot[A];  // wave-uniform
#pragma unroll
  for (int j = 0; j < A; ++j) {
    int av = ia[0], sv = is[0];
#pragma unroll
    for (int k = 1; k < kItemAgents; ++k)
      if (j0 + j == k) {
        av = ia[k];
        sv = is[k];
      }
    const bool ok = active && j < na_g;
    agent[j] = ok ? av : 0;
    slot[j] = ok ? sv : 0;

  }
  const int jc = col / G;                   // agent (within group) of this lane's column
  const bool col_ok = active && col < na_g * G;
  int a_col = agent[0];
#pragma unroll
  for (int j = 1; j < A; ++j)
    if (jc == j) a_col = agent[j];
  if (!col_ok) a_col = 0;
  const int32_t* const pstart = kMap ? p.pstart : nullptr;  // the slot map (see above)
  U4 qraw[4];
  {
    const uint16_t* qrow = q + (size_t(a_col) * Hq + h * G + col % G) * kD;
    for (int c = 0; c < 4; ++c)  // (a_col is a valid agent; unused columns are zeroed later)
      qraw[c].u = *reinterpret_cast<const uint4*>(qrow + 32 * c + 8 * g4);
  }
  // Page ids of this wave's sub-range (at most 64 pages: the plan sizes items so that no
  // wave gets more): lane i holds the ids of page lpa + i, so a page's ids come from a
  // readlane instead of a memory round trip.  Ids are checked here, once: out-of-pool ids
  // become -1 (page skipped / zero residual).
  const int id_base = lpa;
  int vb = -1;
  int vr[A];
  {
    const int lpi = id_base + lane;
    const bool in = lpa < lpb && lpi < lpb;
    vb = in ? p.btab[size_t(agent[0]) * p.max_pages + lpi] : -1;
    if (vb >= p.num_bpages) vb = -1;
    for (int j = 0; j < A; ++j) {
      vr[j] = (in && j < na_g) ? p.rtab[size_t(agent[j]) * p.max_pages + lpi] : -1;
      if (vr[j] >= p.num_rpages) vr[j] = -1;
    }
  }
  // B_k,a[:, h*d:(h+1)*d] goes to LDS in MFMA A-operand order without a staging pass: a
  // work unit (agent jj, rank group g, dims 8pc .. 8pc+7) loads the four rank rows 4g .. 4g+3
  // of its eight dims (16 contiguous bytes each, coalesced over pc) and later packs, per
  // dim, the four ranks into the operand piece of the lane that consumes them.  Unit
  // u = tid + kThreads * i, so jj = wave + kWaves * i is wave-uniform; all loads are issued
  // here (units past the item's agents re-read its first agent and are not stored).
  constexpr int kBkUnits = kItemAgents * 4 * (kD / 8) / kThreads;
  static_assert(4 * (kD / 8) == 64, "a wave's units are one agent's");
  uint4 bkr[kBkUnits][4];
#pragma unroll
  for (int i = 0; i < kBkUnits; ++i) {
    const int jj = w + kWaves * i, g = (lane >> 4) & 3, pc = lane & 15;
    int a = ia[0];
#pragma unroll
    for (int k = 1; k < kItemAgents; ++k)
      if (jj == k && k < na) a = ia[k];
#pragma unroll
    for (int r = 0; r < 4; ++r)
      bkr[i][r] = *reinterpret_cast<const uint4*>(Bk + (size_t(a) * kR + 4 * g + r) * n + h * kD +
                                                  8 * pc);
  }
  // The agents' lengths (an agent's last page's valid rows): lane j holds group agent j's
  // (0 for unused slots), loaded after every vector load above and read (readlane) only where
  // needed -- the last page of the sub-range -- so no earlier step waits for it.
  int vlen = 0;
  {
    int aj = agent[0];
#pragma unroll
    for (int j = 1; j < A; ++j)
      if (lane == j) aj = agent[j];
    const int l = p.plan[p.off_lens + aj];
    vlen = l & -int(active && lane < na_g);  // (a mask, not a branch around the load)
  }
  auto rlen_of = [&](int j) { return __builtin_amdgcn_readlane(vlen, j); };
  // With the slot map, lane i also holds page lpa + i's start and the position its rows end
  // at, from the first agent's start table: a base page that several agents map holds the
  // same rows for each of them (a shared page is full or a frozen tail), so only an agent's
  // own length can cut it shorter.
  int vst = 0, vend = 0;
  if constexpr (kMap) {
    const int lpi = id_base + lane;
    const bool in = lpa < lpb && lpi < lpb;
    const int32_t* row = p.pstart + size_t(agent[0]) * p.max_pages;
    vst = in ? row[lpi] : 0;
    const int nx = (in && lpi + 1 < p.max_pages) ? row[lpi + 1] : -1;
    vend = nx >= 0 ? nx : rlen_of(0);
  }
  const float qscale = p.sm_scale_log2;

  f4 acc[8];
  for (int t = 0; t < 8; ++t) acc[t] = f4{0.f, 0.f, 0.f, 0.f};
  f4 accr = f4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  // Page buffers.  One key-side buffer (base key tile, residual keys) holds page lp while
  // its scores are formed and is refilled with page lp + 1 in place, each half as soon as
  // it has been read; the value-side operands of page lp are loaded when its scores start
  // and used last.
  struct KBuf {
    U4 kt[4];
    U2 rk[A];
    int bp;
    const uint16_t* rb[A];  // residual pages of the group's agents (wave-uniform)
  };
  struct VBuf {
    U2 vt[8];
    U2 rv[A];
  };
  const uint16_t* const zero_res = g_zero_res;
  // RoPE state of the page loop, set up below: cos/sin of the current page's angle (lane j =
  // frequency j), the per-page step, the position the recurrence stands at, and w_j
  float pc = 1.f, ps = 0.f, step_c = 1.f, step_s = 0.f, omega_f = 0.f;
  int next_pos = 0;
  // The rotated residual keys are formed in fp16 (packed arithmetic) and scored against an
  // fp16 copy of q, kept in registers (it is read by every agent's score of every page);
  // the shared base tile is scored in bf16 against the bf16 q, kept in LDS (this wave's
  // slot, lane-linear) and read once per page.  Both are filled in the set-up below.
  H8 qhr[4];

  // residual page of agent j at page lp (the zero page where the sequence has none)
  auto res_page = [&](int lp, int j) -> const uint16_t* {
    const int rp = __builtin_amdgcn_readlane(vr[j], lp - id_base);
    return rp >= 0 ? rcache + size_t(rp) * 2 * kPage * kR : zero_res;
  };
  // The page routines take the group's agent count NA as a compile-time constant, so the
  // per-agent work is straight-line code.
  // key tiles and residual key rows of page lp, in two halves: the page loop refills one
  // buffer in place, each half as soon as the previous page's copy has been consumed
  auto load_kt = [&](int lp, KBuf& B) {
    B.bp = __builtin_amdgcn_readlane(vb, lp - id_base);
    const uint16_t* kt_base = bcache + (size_t(max(B.bp, 0)) * 2 * Hkv + h) * tile;
    // tiles are stored in operand order: lane l's piece is the l-th 16 B (K) / 8 B (V)
    for (int c = 0; c < 4; ++c)
      B.kt[c].u = *reinterpret_cast<const uint4*>(kt_base + 512 * c + 8 * lane);
  };
  auto load_rk = [&](int lp, KBuf& B, auto na_c) {
    constexpr int NA = decltype(na_c)::value;
#pragma unroll
    for (int j = 0; j < NA; ++j) {
      B.rb[j] = res_page(lp, j);
      B.rk[j].u = *reinterpret_cast<const uint2*>(B.rb[j] + 4 * lane);
    }
  };
  auto load_k = [&](int lp, KBuf& B, auto na_c) {
    load_kt(lp, B);
    load_rk(lp, B, na_c);
  };
  auto load_vt = [&](const KBuf& B, U2 (&vt)[8]) {
    const uint16_t* vt_base = bcache + (size_t(max(B.bp, 0)) * 2 * Hkv + Hkv + h) * tile;
    for (int t = 0; t < 8; ++t)
      vt[t].u = *reinterpret_cast<const uint2*>(vt_base + 256 * t + 4 * lane);
  };
  auto load_rv = [&](const KBuf& B, VBuf& V, auto na_c) {
    constexpr int NA = decltype(na_c)::value;
#pragma unroll
    for (int j = 0; j < NA; ++j)
      V.rv[j].u = *reinterpret_cast<const uint2*>(B.rb[j] + kPage * kR + 4 * lane);
  };
  auto load_v = [&](const KBuf& B, VBuf& V, auto na_c) {
    load_vt(B, V.vt);
    load_rv(B, V, na_c);
  };

  // A page's work is split into trig_for (RoPE angles), scores (key tiles and rotated
  // residual keys against the queries) and softmax_acc (online softmax, P V).  The angles of
  // page lp + 1 are formed right after the scores of page lp, where their LDS round trip
  // overlaps the softmax's cross-lane maximum instead of opening the next page.

  // s * cos / s * sin of (t0 + c) * w_j for the page scores() forms next, for
  // j = 32*half + 8*g4 + e (c = this lane's key row), as fp16 pairs (e, e + 1)
  h2 ct[2][4], st[2][4];
  // Angles of page lp (every page of the sub-range passes through here once, in order,
  // skipped pages included): lane j holds cos/sin(t0 * w_j) of the recurrence, which then
  // advances by one page; with the slot map a page whose start differs from the
  // recurrence's position re-anchors it first.  Past the sub-range's end (lp >= lpb) the
  // values are computed and never used.
  auto trig_for = [&](int lp) {
    if constexpr (kMap) {
      const int pos0 = __builtin_amdgcn_readlane(vst, min(lp, lpb - 1) - id_base);
      if (pos0 != next_pos) {  // wave-uniform
        float sv, cv;
        sincosf(static_cast<float>(pos0 - next_pos) * omega_f, &sv, &cv);
        const float c = mul_sub(pc, cv, ps, sv);
        ps = mul_add(ps, cv, pc, sv);
        pc = c;
      }
      next_pos = pos0 + kPage;
    }
    ptrig[lane] = static_cast<_Float16>(pc);
    ptrig[64 + lane] = static_cast<_Float16>(ps);
    {  // advance to the next page: rotate by 16 * w_j
      const float c = mul_sub(pc, step_c, ps, step_s);
      ps = mul_add(ps, step_c, pc, step_s);
      pc = c;
    }
    // (LDS operations of one wave execute in order: the reads below see the writes above)
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int jb = 32 * half + 8 * g4;
      H8 c0, s0, cc, ss;
      c0.u = *reinterpret_cast<const uint4*>(ptrig + jb);
      s0.u = *reinterpret_cast<const uint4*>(ptrig + 64 + jb);
      cc.u = *reinterpret_cast<const uint4*>(trig_c + col * kTrigPad + jb);
      ss.u = *reinterpret_cast<const uint4*>(trig_s + col * kTrigPad + jb);
      for (int e = 0; e < 4; ++e) {
        ct[half][e] = mul_sub2(c0.p[e], cc.p[e], s0.p[e], ss.p[e]);
        st[half][e] = mul_add2(s0.p[e], cc.p[e], c0.p[e], ss.p[e]);
      }
    }
  };

  // Scores of the page whose key-side operands B holds (angles from trig_for of that page):
  // the shared base tile, plus for each agent its rotated residual key; this lane's column's
  // agent is selected.  The page's value-side operands are loaded into V first, except what
  // the caller has already loaded a page ahead: pre_c is 0 (nothing), 1 (the base value
  // tiles) or 2 (all of them).  B is refilled with page lp_next's key-side operands as its
  // own are consumed.  Rows past a page's valid rows give
  // arbitrary scores (their bytes may even be NaN); softmax_acc masks them out before any
  // arithmetic.
  auto scores = [&](KBuf& B, VBuf& V, int lp_next, auto na_c, auto pre_c) -> f4 {
    constexpr int NA = decltype(na_c)::value;
    if constexpr (decltype(pre_c)::value == 0) load_v(B, V, na_c);
    else if constexpr (decltype(pre_c)::value == 1) load_rv(B, V, na_c);
    f4 sb = f4{0.f, 0.f, 0.f, 0.f};
    for (int c = 0; c < 4; ++c) {
      U4 qb;
      qb.u = qb_lds[c * 64 + lane];
      sb = mfma32(B.kt[c].b, qb.b, sb);
    }
    load_kt(lp_next, B);  // the key tiles have been read: refill them with page lp_next's
    // Work units u = (agent, half), agent-major: half h covers score chunks h and h + 2, i.e.
    // the reconstruction tiles T = 2h, 2h+1 and their RoPE partners T + 4.  The units are
    // software-pipelined: the reconstruction MFMAs of unit u + 1 are issued before the
    // rotation arithmetic of unit u, so the matrix core and the vector ALU work together.
    // An agent's residual score is complete after its second unit and is then selected
    // for the columns it owns.
    constexpr int NU = 2 * NA;
    f4 ssel = f4{0.f, 0.f, 0.f, 0.f}, sj = f4{0.f, 0.f, 0.f, 0.f};
    // B_k operands of a unit (four 8-byte LDS reads), fetched one unit before their use
    auto bk_ops = [&](int u, U2 (&a)[4]) {
      const int j = u / 2, half = u % 2;
      const uint2* bkj = bkl + (j0 + j) * 8 * 64 + lane;
      const int Ts[4] = {2 * half, 2 * half + 1, 2 * half + 4, 2 * half + 5};
      for (int k = 0; k < 4; ++k) a[k].u = bkj[Ts[k] * 64];
    };
    auto recon = [&](int u, const U2 (&a)[4], f4 (&d)[4]) {
      const int j = u / 2;
      for (int k = 0; k < 4; ++k) d[k] = mfma16(a[k].s, B.rk[j].s, f4{0.f, 0.f, 0.f, 0.f});
    };
    auto rotate_score = [&](int u, const f4 (&d)[4]) {
      const int j = u / 2, half = u % 2;
      // rotate the partner pairs (tile k, tile k + 2) on packed fp16 values
      H8 k0, k2;
      for (int k = 0; k < 2; ++k) {
        for (int q2 = 0; q2 < 2; ++q2) {
          const h2 x = pack_f16x2(d[k][2 * q2], d[k][2 * q2 + 1]);
          const h2 y = pack_f16x2(d[k + 2][2 * q2], d[k + 2][2 * q2 + 1]);
          const h2 c = ct[half][2 * k + q2], sn = st[half][2 * k + q2];
          k0.p[2 * k + q2] = mul_sub2(x, c, y, sn);
          k2.p[2 * k + q2] = mul_add2(y, c, x, sn);
        }
      }
      if (half == 0) sj = sb;  // each agent's residual score accumulates onto the base score
      sj = mfma32h(k0.v, qhr[half].v, sj);
      sj = mfma32h(k2.v, qhr[half + 2].v, sj);
      if (half == 1) ssel = (j == 0 || jc == j) ? sj : ssel;
    };
    f4 dA[4], dB[4];
    U2 oA[4], oB[4];
    bk_ops(0, oA);
    if (NU > 1) bk_ops(1, oB);
    recon(0, oA, dA);
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      if (u % 2 == 0) {
        if (u + 2 < NU) bk_ops(u + 2, oA);
        if (u + 1 < NU) recon(u + 1, oB, dB);
        rotate_score(u, dA);
      } else {
        if (u + 2 < NU) bk_ops(u + 2, oB);
        if (u + 1 < NU) recon(u + 1, oA, dA);
        rotate_score(u, dB);
      }
    }
    load_rk(lp_next, B, na_c);  // likewise the residual key rows, after the last reconstruction
    return ssel;
  };

  // Rows of page lp held by the group's agents (the page's start is common to them all):
  // the most and the fewest, and those of this lane's column's agent.
  struct Rows {
    int vrows, minrows, rows_col;
  };
  auto page_rows_of = [&](int lp, auto na_c) -> Rows {
    constexpr int NA = decltype(na_c)::value;
    int pos0 = 0, pend = 0;
    if constexpr (kMap) {
      pos0 = __builtin_amdgcn_readlane(vst, lp - id_base);
      pend = __builtin_amdgcn_readlane(vend, lp - id_base);
    }
    Rows R{0, kPage, 0};
    int prow[NA];
#pragma unroll
    for (int j = 0; j < NA; ++j) {
      prow[j] = kMap ? min(min(rlen_of(j), pend) - pos0, kPage)
                     : page_rows(nullptr, p.max_pages, agent[j], lp, rlen_of(j));
      R.vrows = max(R.vrows, prow[j]);
      R.minrows = min(R.minrows, prow[j]);
    }
    R.rows_col = prow[0];
#pragma unroll
    for (int j = 1; j < NA; ++j)
      if (jc == j) R.rows_col = prow[j];
    return R;
  };

  // Online softmax over a page's 16 keys, per column (log2 domain), then acc += P bV and
  // acc_r += P_a rV_a.  kFull: every agent of the group holds all 16 rows of the page, so
  // nothing is masked (R is not read).
  auto softmax_acc = [&](f4 ssel, VBuf& V, auto na_c, auto full_c, const Rows& R) {
    constexpr int NA = decltype(na_c)::value;
    constexpr bool kFull = decltype(full_c)::value;
    float sc[4];
    float pmax = -INFINITY;
    if (kFull || R.minrows >= kPage) {
      // every agent of the group has all 16 keys of the page; columns without an agent
      // (zero q) only ever touch their own, unwritten, state
      for (int i = 0; i < 4; ++i) {
        sc[i] = ssel[i] * qscale;
        pmax = fmaxf(pmax, sc[i]);
      }
    } else {
      for (int i = 0; i < 4; ++i) {
        sc[i] = (col_ok && 4 * g4 + i < R.rows_col) ? ssel[i] * qscale : -INFINITY;
        pmax = fmaxf(pmax, sc[i]);
      }
    }
    pmax = max_over_rows(pmax);
    // The reference maximum m_run only moves when a column's page maximum exceeds it by
    // more than 8 (log2 units): probabilities then stay below 2^8 and the rescale of the
    // accumulators (acc AND acc_r, by the same factor) is skipped on almost every page.
    const bool grow = pmax > m_run + 8.f;
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {  // wave-uniform branch
      const float m_new = grow ? pmax : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 when m_run = -inf
      l_run *= alpha;
      for (int t = 0; t < 8; ++t) acc[t] *= alpha;
      accr *= alpha;
      m_run = m_new;
    }
    // arguments are <= 8; v_exp_f32 flushes results below 2^-126 to zero, which only drops
    // probabilities negligible next to the reference's 1.0
    const float m_ref = max2(m_run, -1e30f);  // no -inf - -inf for columns without keys
    float pr[4];
    for (int i = 0; i < 4; ++i) pr[i] = __builtin_amdgcn_exp2f(sc[i] - m_ref);
    l_run += (pr[0] + pr[1] + pr[2] + pr[3]);

    U2 pb;
    pb.u = make_uint2(pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3]));
    if constexpr (!kFull) {
      // value rows past the page's valid rows are zeroed: P is 0 there, but their bytes
      // are arbitrary (even NaN)
      const int tv = R.vrows - 4 * g4;  // valid tokens among this lane's 4 (V operands)
      if (tv < 4) {
        auto mask4 = [&](uint2 v) {
          if (tv <= 0) v.x = 0;
          else if (tv == 1) v.x &= 0xffffu;
          if (tv <= 2) v.y = 0;
          else if (tv == 3) v.y &= 0xffffu;
          return v;
        };
        for (int t = 0; t < 8; ++t) V.vt[t].u = mask4(V.vt[t].u);
        for (int j = 0; j < NA; ++j) V.rv[j].u = mask4(V.rv[j].u);
      }
    }
    for (int t = 0; t < 8; ++t) acc[t] = mfma16(V.vt[t].s, pb.s, acc[t]);
#pragma unroll
    for (int j = 0; j < NA; ++j) {
      U2 pj;
      pj.u = (jc == j) ? pb.u : make_uint2(0, 0);
      accr = mfma16(V.rv[j].s, pj.s, accr);
    }
  };

  // the group's agent count as a compile-time constant for the page routines
  auto with_na = [&](auto f) __attribute__((always_inline)) {  // na_g is wave-uniform
    if (na_g >= A) f(std::integral_constant<int, A>{});
    if constexpr (A > 3) if (na_g == 3) f(std::integral_constant<int, 3>{});
    if constexpr (A > 2) if (na_g == 2) f(std::integral_constant<int, 2>{});
    if constexpr (A > 1) if (na_g == 1) f(std::integral_constant<int, 1>{});
  };
  // Decode with append: the new token of every item agent whose last page lies in this item's
  // pages is stored first -- this KV head's key and value rows, and the residual rows (the
  // same bytes from every head's workgroup) -- and the workgroup waits for the stores before
  // any page is read.  Only this item's workgroups read those pages: a row just appended sits
  // in a page private to its agent.  The token sits at position length - 1 (the length on
  // the device, which the previous call advanced), in the agent's last page.
  static_assert(kThreads == 2 * kD, "one thread per key and per value element of a row");
  if (p.k_new != nullptr && holds_last != 0) {  // uniform over the workgroup
    uint16_t* const bw = const_cast<uint16_t*>(bcache);
    uint16_t* const rw = const_cast<uint16_t*>(rcache);
    // every item agent's last page and length in one round trip: lane j loads item agent
    // j's (lanes past the item's agents its first agent's, not used)
    int aj = ia[0];
#pragma unroll
    for (int k = 1; k < kItemAgents; ++k)
      if (lane == k && k < na) aj = ia[k];
    const int vlast = p.plan[p.off_lastpage + aj];
    const int vlen_n = p.plan[p.off_lens + aj];
#pragma unroll
    for (int j = 0; j < kItemAgents; ++j) {
      if (j >= na) continue;  // uniform
      const int a = ia[j];
      const int lp_last = __builtin_amdgcn_readlane(vlast, j);
      if (lp_last < lp0 || lp_last >= lp0 + np) continue;  // uniform
      const int row = __builtin_amdgcn_readlane(vlen_n, j) - 1 -
                      page_start(p.pstart, p.max_pages, a, lp_last);
      // (a row past the page: the caller did not rebuild the plan after a page crossing)
      if (row < 0 || row >= kPage) continue;
      const int bpg = p.btab[size_t(a) * p.max_pages + lp_last];
      const int rpg = p.rtab[size_t(a) * p.max_pages + lp_last];
      if (bpg < 0 || rpg < 0 || bpg >= p.num_bpages || rpg >= p.num_rpages) continue;
      const int brow = row, rrow = row;
      if (tid < kD) {
        const uint16_t* kn = static_cast<const uint16_t*>(p.k_new) + (size_t(a) * Hkv + h) * kD;
        bw[(size_t(bpg) * 2 * Hkv + h) * tile + TileOrder::key(brow, tid)] = kn[tid];
      } else {
        const int x = tid - kD;
        const uint16_t* vn = static_cast<const uint16_t*>(p.v_new) + (size_t(a) * Hkv + h) * kD;
        bw[(size_t(bpg) * 2 * Hkv + Hkv + h) * tile + TileOrder::value(brow, x)] = vn[x];
      }
      if (tid < kR) {
        const uint16_t* rkn = static_cast<const uint16_t*>(p.rk_new) + size_t(a) * kR;
        rw[size_t(rpg) * 2 * kPage * kR + TileOrder::res_key(rrow, tid)] = rkn[tid];
      } else if (tid < 2 * kR) {
        const int k = tid - kR;
        const uint16_t* rvn = static_cast<const uint16_t*>(p.rv_new) + size_t(a) * kR;
        rw[size_t(rpg) * 2 * kPage * kR + kPage * kR + TileOrder::res_value(rrow, k, kR)] = rvn[k];
      }
    }
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this thread's stores have completed
    __syncthreads();
  }
  // the first page's key-side operands (all A agents' residual rows: a missing one reads
  // the zero page), before the set-up below
  KBuf first;
  if (lpa < lpb) load_k(lpa, first, std::integral_constant<int, A>{});

  // ---- on-chip set-up, while the loads above are in flight ----------------------------
  // w_j = theta^(-2j/d) = 2^(-(2j/d) log2 theta); lane j keeps w_j in fp64 (j = lane).  Every
  // thread's trig-table entries are for its own lane's frequency: (c, j) = (w + 4i, lane).
  const double log2_theta = log2(static_cast<double>(p.rope_theta));
  const double omega = exp2(-2.0 * lane / kD * log2_theta);
  omega_f = static_cast<float>(omega);
  constexpr int kTrigPer = kPage * 64 / kThreads;
  float tcv[kTrigPer], tsv[kTrigPer];
  const float rev_f = static_cast<float>(omega * kInvTwoPi);  // w_j in revolutions
#pragma unroll
  for (int i = 0; i < kTrigPer; ++i) {
    // in-page offsets c < 16: the angle c * w_j is at most 15 rad (2.4 revolutions), well
    // inside the hardware sine/cosine's domain; their error is far below the fp16 the table
    // is stored in
    const float x = static_cast<float>(w + kWaves * i) * rev_f;
    tsv[i] = __builtin_amdgcn_sinf(x);
    tcv[i] = __builtin_amdgcn_cosf(x);
  }
  // pack the B_k units into operand order: dim x sits in tile T, row m with
  // x = perm_dim(T, m), and the lane 16 g + m of that tile holds ranks 4g .. 4g+3
#pragma unroll
  for (int i = 0; i < kBkUnits; ++i) {
    const int jj = w + kWaves * i, g = (lane >> 4) & 3, pc = lane & 15;
    if (jj < na) {  // wave-uniform
      const uint32_t r0[4] = {bkr[i][0].x, bkr[i][0].y, bkr[i][0].z, bkr[i][0].w};
      const uint32_t r1[4] = {bkr[i][1].x, bkr[i][1].y, bkr[i][1].z, bkr[i][1].w};
      const uint32_t r2[4] = {bkr[i][2].x, bkr[i][2].y, bkr[i][2].z, bkr[i][2].w};
      const uint32_t r3[4] = {bkr[i][3].x, bkr[i][3].y, bkr[i][3].z, bkr[i][3].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int x = 8 * pc + e;
        const int T = 2 * (x >> 5) + ((x & 7) >> 2), m = 4 * ((x & 31) >> 3) + (x & 3);
        // ranks (4g, 4g+1) and (4g+2, 4g+3) of dim x: the low or high halves of word e/2
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        uint2 v;
        v.x = __builtin_amdgcn_perm(r1[e >> 1], r0[e >> 1], sel);
        v.y = __builtin_amdgcn_perm(r3[e >> 1], r2[e >> 1], sel);
        bkl[(jj * 8 + T) * 64 + 16 * g + m] = v;
      }
    }
  }
#pragma unroll
  for (int i = 0; i < kTrigPer; ++i) {
    const int c = w + kWaves * i;
    trig_c[c * kTrigPad + lane] = static_cast<_Float16>(tcv[i] * p.lora_scale);
    trig_s[c * kTrigPad + lane] = static_cast<_Float16>(tsv[i] * p.lora_scale);
  }
  for (int c = 0; c < 4; ++c) {
    if (!col_ok) qraw[c].u = make_uint4(0, 0, 0, 0);  // columns without an agent score zero
    qb_lds[c * 64 + lane] = qraw[c].u;
    const uint32_t wds[4] = {qraw[c].u.x, qraw[c].u.y, qraw[c].u.z, qraw[c].u.w};
    for (int e = 0; e < 4; ++e)
      qhr[c].p[e] = pack_f16x2(__uint_as_float(wds[e] << 16), __uint_as_float(wds[e] & 0xffff0000u));
  }
  __syncthreads();

  // cos/sin(t0 * w_j) for lane j = frequency j, at this wave's first page, with the angle
  // t0 * w_j formed and reduced to [-pi, pi] in fp64; later pages follow by the rotation
  // (cos, sin)(16 w_j).  Over the at most 64 pages of a wave the recurrence drifts by a few
  // 1e-6 rad at most.  Pages start at lp * P unless a frozen tail precedes them (the slot
  // map): a page whose start differs from the recurrence's position re-anchors it by the
  // (at most P - 1 positions) gap.
  next_pos = (active && lpa < lpb) ? page_start(pstart, p.max_pages, agent[0], lpa) : 0;
  {
    double ang = static_cast<double>(next_pos) * omega;
    ang = fma(-kTwoPi, rint(ang * kInvTwoPi), ang);
    sincosf(static_cast<float>(ang), &ps, &pc);
    sincosf(static_cast<float>(kPage * omega), &step_s, &step_c);
  }

  using Full = std::true_type;
  using Masked = std::false_type;
  // Key-side prefetches are issued unconditionally (past the end they re-read the last page,
  // an L2 hit).  One key-side buffer B serves both loops (refilled in place by scores).
  //
  // General loop (the slot map, or a sub-range holding a page id outside the pool): every
  // page is masked by its agents' rows, and a page without a base id is skipped.
  auto run_general = [&](auto na_c) __attribute__((always_inline)) {
    KBuf B = first;
    VBuf v;
    trig_for(lpa);
    for (int lp = lpa; lp < lpb; ++lp) {
      const bool have = B.bp >= 0;
      const f4 s = scores(B, v, min(lp + 1, lpb - 1), na_c, std::integral_constant<int, 0>{});
      trig_for(lp + 1);
      if (have) softmax_acc(s, v, na_c, Masked{}, page_rows_of(lp, na_c));
    }
  };
  // Loops over full pages (pages start at lp * P and every id is in the pool).  Every page
  // of the sub-range but its last is full for every agent of the group: a page with fewer
  // rows is an agent's last and no other agent maps it (a fork copies a partial tail), so it
  // ends its item.  Only the last page is masked.  Value operands loaded a page before their
  // use: the four-agent kernel (whose registers do not hold a second full value buffer
  // without spilling) takes run_fast_ahead_vt on every sub-range -- the base value tiles of
  // page lp + 1 are loaded into the one buffer right after page lp's value products have
  // read it; the other kernels take run_fast_ahead on sub-ranges of 8 pages or more (all
  // value operands, two buffers, the loop taken two pages at a time) and run_fast, which
  // loads them when the page's scores start, on shorter ones, where that set-up does not pay.
  auto run_fast_ahead = [&](auto na_c) __attribute__((always_inline)) {
    KBuf B = first;
    VBuf va, vb;
    load_v(B, va, na_c);
    trig_for(lpa);
    // page lp's scores refill B with page lp + 1's key side; that page's values are loaded
    // right after, a page ahead of their use, into the other buffer
    auto page = [&](int lp, VBuf& cur, VBuf& nxt) __attribute__((always_inline)) {
      const f4 s = scores(B, cur, lp + 1, na_c, std::integral_constant<int, 2>{});
      load_v(B, nxt, na_c);
      trig_for(lp + 1);
      softmax_acc(s, cur, na_c, Full{}, Rows{});
    };
    int lp = lpa;
    for (; lp + 2 < lpb; lp += 2) {
      page(lp, va, vb);
      page(lp + 1, vb, va);
    }
    if (lp + 1 < lpb) {
      page(lp, va, vb);
      const f4 s = scores(B, vb, lpb - 1, na_c, std::integral_constant<int, 2>{});
      softmax_acc(s, vb, na_c, Masked{}, page_rows_of(lpb - 1, na_c));
    } else {
      const f4 s = scores(B, va, lpb - 1, na_c, std::integral_constant<int, 2>{});
      softmax_acc(s, va, na_c, Masked{}, page_rows_of(lpb - 1, na_c));
    }
  };
  auto run_fast_ahead_vt = [&](auto na_c) __attribute__((always_inline)) {
    KBuf B = first;
    VBuf v;
    load_vt(B, v.vt);
    trig_for(lpa);
    // page lp + 1's base value tiles are loaded as soon as page lp's value products have
    // read the buffer, a whole page before their own use; no memory read may be scheduled
    // above those products (a read hoisted there would need a second buffer and a register
    // copy at the loop's end, which waits for every load issued in the page)
    // Wave priority falls by one level per quarter of the sub-range done: of the two waves
    // that share a SIMD (one from each workgroup on the compute unit), the one further behind
    // is issued first, instead of the older workgroup's running ahead and leaving the other's
    // to finish alone.
    __builtin_amdgcn_s_setprio(3);
    for (int lp = lpa; lp + 1 < lpb; ++lp) {
      const f4 s = scores(B, v, lp + 1, na_c, std::integral_constant<int, 1>{});
      trig_for(lp + 1);
      softmax_acc(s, v, na_c, Full{}, Rows{});
      __builtin_amdgcn_sched_barrier(0x078F);
      load_vt(B, v.vt);
      const int done4 = 4 * (lp + 1 - lpa), tot = lpb - lpa;
      if (done4 >= 3 * tot) __builtin_amdgcn_s_setprio(0);
      else if (done4 >= 2 * tot) __builtin_amdgcn_s_setprio(1);
      else if (done4 >= tot) __builtin_amdgcn_s_setprio(2);
    }
    const f4 s = scores(B, v, lpb - 1, na_c, std::integral_constant<int, 1>{});
    softmax_acc(s, v, na_c, Masked{}, page_rows_of(lpb - 1, na_c));
    __builtin_amdgcn_s_setprio(0);
  };
  auto run_fast = [&](auto na_c) __attribute__((always_inline)) {
    KBuf B = first;
    VBuf v;
    trig_for(lpa);
    for (int lp = lpa; lp + 1 < lpb; ++lp) {
      const f4 s = scores(B, v, lp + 1, na_c, std::integral_constant<int, 0>{});
      trig_for(lp + 1);
      softmax_acc(s, v, na_c, Full{}, Rows{});
    }
    const f4 s = scores(B, v, lpb - 1, na_c, std::integral_constant<int, 0>{});
    softmax_acc(s, v, na_c, Masked{}, page_rows_of(lpb - 1, na_c));
  };
  if (lpa < lpb) {
    const bool bad = lane < lpb - lpa && vb < 0;  // a page id outside the pool
    bool general = __builtin_amdgcn_ballot_w64(bad) != 0;
    if constexpr (kMap) {
      // With the slot map a page before the sub-range's last one can hold fewer than 16 rows
      // (a frozen tail): such a sub-range takes the general loop.  Otherwise every page but
      // the last is full for every agent of the group and starts where the previous one
      // ends, exactly as without the slot map, and the loops below apply (the angles
      // re-anchor at the first page if its start is not a multiple of 16).
      const bool short_mid = lane < lpb - lpa - 1 && vend - vst != kPage;
      general = general || __builtin_amdgcn_ballot_w64(short_mid) != 0;
      // (the two-agent instantiation keeps the general loop only: with the fast loops beside
      // it, its registers spill)
      if constexpr (A == 2) general = true;
    }
    if (!general) {
      if constexpr (A >= 4) with_na(run_fast_ahead_vt);
      else if (lpb - lpa >= 8) with_na(run_fast_ahead);
      else with_na(run_fast);
    } else {
      with_na(run_general);
    }
  }

  // ---- merge the sub-range partials of each group (LSE rule), write split-K partials ----
  // Every wave of a group takes part: the n_sub partials' (m, l) give one set of weights, and
  // wave si merges and stores the accumulator tiles [si * 8 / n_sub, (si + 1) * 8 / n_sub)
  // (wave 0 also acc_r and (m, l)).  With one sub-range there is nothing to merge.
  l_run += shfl_xor(l_run, 16);
  l_run += shfl_xor(l_run, 32);
  const int per = 8 / n_sub, t0 = si * per;  // this wave's accumulator tiles
  if (n_sub > 1) {  // uniform over the workgroup
    __syncthreads();  // LDS is reused for the merge
    // [vector][wave][lane] of float4: (m, l, -, -), acc[0..7], acc_r -- each wave's row of a
    // vector is 1 KiB of consecutive lanes (no bank conflicts)
    float4* mb = reinterpret_cast<float4*>(lds);
    auto mslot = [&](int v, int wv) { return (v * kWaves + wv) * 64 + lane; };
    mb[mslot(0, w)] = make_float4(m_run, l_run, 0.f, 0.f);
    for (int t = 0; t < 8; ++t) mb[mslot(1 + t, w)] = make_float4(acc[t][0], acc[t][1], acc[t][2], acc[t][3]);
    mb[mslot(9, w)] = make_float4(accr[0], accr[1], accr[2], accr[3]);
    __syncthreads();
    if (!active) return;
    int ow[kWaves];
    float om[kWaves], ol[kWaves];
    float M = -INFINITY;
#pragma unroll
    for (int o = 0; o < kWaves; ++o) {
      ow[o] = gi + (o < n_sub ? o : 0) * n_groups;  // (partners past n_sub are never read)
      const float4 ml = mb[mslot(0, ow[o])];
      om[o] = ml.x;
      ol[o] = ml.y;
      if (o < n_sub) M = fmaxf(M, om[o]);
    }
    float wo[kWaves], L = 0.f;
#pragma unroll
    for (int o = 0; o < kWaves; ++o) {
      wo[o] = (o < n_sub && M != -INFINITY) ? exp2f(om[o] - M) : 0.f;
      if (o < n_sub) L += wo[o] * ol[o];
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      if (t < t0 || t >= t0 + per) continue;
      f4 v = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int o = 0; o < kWaves; ++o)
        if (o < n_sub) {
          const float4 x = mb[mslot(1 + t, ow[o])];
          v[0] += wo[o] * x.x;
          v[1] += wo[o] * x.y;
          v[2] += wo[o] * x.z;
          v[3] += wo[o] * x.w;
        }
      acc[t] = v;
    }
    if (si == 0) {
      f4 v = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int o = 0; o < kWaves; ++o)
        if (o < n_sub) {
          const float4 x = mb[mslot(9, ow[o])];
          v[0] += wo[o] * x.x;
          v[1] += wo[o] * x.y;
          v[2] += wo[o] * x.z;
          v[3] += wo[o] * x.w;
        }
      accr = v;
    }
    m_run = M;
    l_run = L;
  } else if (!active) {
    return;
  }
  if (!col_ok) return;
  int s_col = slot[0];
#pragma unroll
  for (int j = 1; j < A; ++j)
    if (jc == j) s_col = slot[j];
  const size_t row = size_t(s_col) * Hq + h * G + col % G;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    if (t < t0 || t >= t0 + per) continue;
    *reinterpret_cast<float4*>(p.ws_acc + row * kD + 16 * t + 4 * g4) =
        make_float4(acc[t][0], acc[t][1], acc[t][2], acc[t][3]);
  }
  if (si != 0) return;
  *reinterpret_cast<float4*>(p.ws_accr + row * kR + 4 * g4) =
      make_float4(accr[0], accr[1], accr[2], accr[3]);
  if (g4 == 0) {
    p.ws_ml[row * 2] = m_run;
    p.ws_ml[row * 2 + 1] = l_run;
  }
}

}  // namespace

static_assert(kWaves == kMfmaWaves, "the planner sizes items for this many waves");
static_assert(kD == kMfmaHeadDim && kR == kMfmaRank, "the shape the planner routes here");


hipError_t launch_decode_mfma(const DecodeParams& p, hipStream_t s) {
  const int A = mfma_agents_per_group(p.group);
  const int n_items = p.n_items;
  const int blocks = 8 * p.num_kv_heads * ((n_items + 7) / 8);
#define FORKKV_DECODE_LAUNCH(NA, MAP) \
  hipLaunchKernelGGL((decode_mfma_kernel<NA, MAP>), dim3(blocks), dim3(kThreads), 0, s, p, n_items)
  const bool map = p.pstart != nullptr;
  switch (A * 2 + (map ? 1 : 0)) {
    case 8: FORKKV_DECODE_LAUNCH(4, false); break;
    case 9: FORKKV_DECODE_LAUNCH(4, true); break;
    case 6: FORKKV_DECODE_LAUNCH(3, false); break;
    case 7: FORKKV_DECODE_LAUNCH(3, true); break;
    case 4: FORKKV_DECODE_LAUNCH(2, false); break;
    case 5: FORKKV_DECODE_LAUNCH(2, true); break;
    case 2: FORKKV_DECODE_LAUNCH(1, false); break;
    case 3: FORKKV_DECODE_LAUNCH(1, true); break;
    default: return hipErrorInvalidValue;
  }
#undef FORKKV_DECODE_LAUNCH
  return hipGetLastError();
}

}  // namespace forkkv
