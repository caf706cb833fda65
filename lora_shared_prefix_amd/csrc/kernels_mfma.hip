// MFMA (matrix-core) ResidualAttention kernels for gfx950, bf16 storage, d = 128, r = 16,
// page size 16: the split-K decode kernel (up to 16 query columns -- agents x GQA group --
// per wave; with decode-with-append it also stores the new rows first) and, further down,
// the chunked-prefill kernel.
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
// MFMA lane layouts used (checked on gfx950): for a 16x16xK instruction lane l supplies
// A[l % 16][kpl * (l / 16) + e] and B[kpl * (l / 16) + e][l % 16] (kpl = K / 4) and
// receives D[4 * (l / 16) + i][l % 16].
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdlib>
#include <type_traits>

#include "forkkv_internal.h"

namespace forkkv {
namespace {

typedef short s4 __attribute__((__vector_size__(4 * sizeof(short))));
typedef __bf16 bf8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f4 __attribute__((__vector_size__(4 * sizeof(float))));

constexpr int kD = 128;       // head dim
constexpr int kR = 16;        // rank
constexpr int kWaves = 4;     // waves per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kTrigPad = 72;  // padded row of the static in-page trig table (fp16)
constexpr double kTwoPi = 6.283185307179586476925286766559;
constexpr double kInvTwoPi = 0.15915494309189533576888376337251;

// LDS layout (bytes)
constexpr int kBkBytes = kItemAgents * 8 * 64 * 8;      // [agent][tile][lane][4 bf16]
constexpr int kTrigBytes = 2 * kPage * kTrigPad * 2;    // cos, sin: [c][j] (scaled by s)
constexpr int kPageTrigBytes = kWaves * 2 * 64 * 2;     // per wave: cos[64], sin[64]
constexpr int kQhBytes = kWaves * 4 * 64 * 16;          // per wave: bf16 q, [chunk][lane]
constexpr int kMergeFloats = 4 + 32 + 4;                // m, l, pad, pad | acc[32] | accr[4]
constexpr int kMergeBytes = kWaves * 64 * kMergeFloats * 4;
constexpr int kLdsMain = kBkBytes + kTrigBytes + kPageTrigBytes + kQhBytes;
constexpr int kLdsBytes = kLdsMain > kMergeBytes ? kLdsMain : kMergeBytes;

__device__ __forceinline__ f4 mfma16(s4 a, s4 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f4 mfma32(bf8 a, bf8 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
typedef _Float16 h8 __attribute__((__vector_size__(8 * sizeof(_Float16))));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ f4 mfma32h(h8 a, h8 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
union H8 {
  h2 p[4];
  h8 v;
  uint4 u;
};
// Two floats -> fp16 pair, round to nearest even (v_cvt_pk_f16_f32).
__device__ __forceinline__ h2 pack_f16x2(float lo, float hi) {
  const float2 f = {lo, hi};
  typedef float fv2 __attribute__((ext_vector_type(2)));
  return __builtin_convertvector(fv2{f.x, f.y}, h2);
}
// a * b - c * d and a * b + c * d with one fixed rounding sequence (c * d rounded, then one
// fused multiply-add), so every instantiation of the kernels rounds the same way.
__device__ __forceinline__ h2 mul_sub2(h2 a, h2 b, h2 c, h2 d) {
#pragma clang fp contract(off)
  const h2 t = c * d;
  return __builtin_elementwise_fma(a, b, -t);
}
__device__ __forceinline__ h2 mul_add2(h2 a, h2 b, h2 c, h2 d) {
#pragma clang fp contract(off)
  const h2 t = c * d;
  return __builtin_elementwise_fma(a, b, t);
}
__device__ __forceinline__ float mul_sub(float a, float b, float c, float d) {
#pragma clang fp contract(off)
  const float t = c * d;
  return __builtin_fmaf(a, b, -t);
}
__device__ __forceinline__ float mul_add(float a, float b, float c, float d) {
#pragma clang fp contract(off)
  const float t = c * d;
  return __builtin_fmaf(a, b, t);
}
// Zero residual page, read in place of a page a sequence does not have.
__device__ __align__(16) uint16_t g_zero_res[2 * kPage * kR];

typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
typedef float fl2 __attribute__((ext_vector_type(2)));

// Two floats -> packed bf16 pair, round to nearest even (one v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const fl2 f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf2));
}

__device__ __forceinline__ float shfl_xor(float v, int mask) {
  return __shfl_xor(v, mask, 64);
}
// max(a, b) for values that are finite or -inf: one median-of-three against the largest
// finite float (fmaxf would first quiet possible signalling NaNs, one extra instruction per
// operand, and a bound of +inf is folded back into fmaxf by the compiler)
__device__ __forceinline__ float max2(float a, float b) {
  return __builtin_amdgcn_fmed3f(a, b, 3.402823466e38f);
}
// max over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (one query column's rows): two
// butterfly steps with the cross-row lane swaps (no LDS round trip)
__device__ __forceinline__ float max_over_rows(float v) {
  const uint32_t x = __float_as_uint(v);
  const auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  v = max2(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const uint32_t y = __float_as_uint(v);
  const auto b = __builtin_amdgcn_permlane32_swap(y, y, false, false);
  return max2(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

union U4 {
  uint4 u;
  bf8 b;
};
union U2 {
  uint2 u;
  s4 s;
};

// Dimension held by reconstruction tile T, row m (a permutation of 0..127 chosen so that
// (a) tiles T and T + 4 hold the RoPE partners j and j + 64 at the same row, and (b) the
// lane that receives rows 4g..4g+3 of tiles 2c, 2c+1 holds dims 32c + 8g .. 32c + 8g + 7,
// i.e. exactly the natural-order K slice it must supply to the 16x16x32 score MFMA.
__device__ __forceinline__ int perm_dim(int T, int m) {
  return 32 * (T >> 1) + 8 * (m >> 2) + 4 * (T & 1) + (m & 3);
}

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
  const int lp0 = it[0], np = it[1], na = it[2];
  // (the empty statements take the record's values as operands, so that all of its loads are
  // issued before the test below -- one memory round trip -- rather than sunk past it)
  asm volatile("" : : "s"(lp0), "s"(np), "s"(na));
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
  int agent[A], slot[A], rlen[A];  // wave-uniform
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
    rlen[j] = ok ? p.plan[p.off_lens + agent[j]] : 0;
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
    vend = nx >= 0 ? nx : rlen[0];
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
  const float qscale = p.sm_scale_log2;

  f4 acc[8];
  for (int t = 0; t < 8; ++t) acc[t] = f4{0.f, 0.f, 0.f, 0.f};
  f4 accr = f4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  // Page buffers.  The key-side operands of page lp + 1 (base key tile, residual keys) are
  // loaded while page lp is computed (two register buffers, used alternately); the
  // value-side operands of page lp are loaded when its computation starts and used last.
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
  auto load_v = [&](const KBuf& B, VBuf& V, auto na_c) {
    constexpr int NA = decltype(na_c)::value;
    const uint16_t* vt_base = bcache + (size_t(max(B.bp, 0)) * 2 * Hkv + Hkv + h) * tile;
    for (int t = 0; t < 8; ++t)
      V.vt[t].u = *reinterpret_cast<const uint2*>(vt_base + 256 * t + 4 * lane);
#pragma unroll
    for (int j = 0; j < NA; ++j)
      V.rv[j].u = *reinterpret_cast<const uint2*>(B.rb[j] + kPage * kR + 4 * lane);
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
  // agent is selected.  The page's value-side operands are loaded into V first, and B is
  // refilled with page lp_next's key-side operands as its own are consumed.  Rows past a page's valid rows give arbitrary scores
  // (their bytes may even be NaN); softmax_acc masks them out before any arithmetic.
  auto scores = [&](KBuf& B, VBuf& V, int lp_next, auto na_c) -> f4 {
    constexpr int NA = decltype(na_c)::value;
    load_v(B, V, na_c);
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
      if (half == 0) sj = f4{0.f, 0.f, 0.f, 0.f};
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
    return ssel + sb;
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
      prow[j] = kMap ? min(min(rlen[j], pend) - pos0, kPage)
                     : page_rows(nullptr, p.max_pages, agent[j], lp, rlen[j]);
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
  if (p.k_new != nullptr) {  // uniform over the grid
    uint16_t* const bw = const_cast<uint16_t*>(bcache);
    uint16_t* const rw = const_cast<uint16_t*>(rcache);
#pragma unroll
    for (int j = 0; j < kItemAgents; ++j) {
      if (j >= na) continue;  // uniform
      const int a = ia[j];
      const int lp_last = p.plan[p.off_lastpage + a];
      if (lp_last < lp0 || lp_last >= lp0 + np) continue;  // uniform
      const int row = p.plan[p.off_lens + a] - 1 - page_start(p.pstart, p.max_pages, a, lp_last);
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
      const f4 s = scores(B, v, min(lp + 1, lpb - 1), na_c);
      trig_for(lp + 1);
      if (have) softmax_acc(s, v, na_c, Masked{}, page_rows_of(lp, na_c));
    }
  };
  // Loop over full pages (pages start at lp * P and every id is in the pool).  Every page of
  // the sub-range but its last is full for every agent of the group: a page with fewer rows
  // is an agent's last and no other agent maps it (a fork copies a partial tail), so it ends
  // its item.  Only the last page is masked.
  auto run_fast = [&](auto na_c) __attribute__((always_inline)) {
    KBuf B = first;
    VBuf v;
    trig_for(lpa);
    for (int lp = lpa; lp + 1 < lpb; ++lp) {
      const f4 s = scores(B, v, lp + 1, na_c);
      trig_for(lp + 1);
      softmax_acc(s, v, na_c, Full{}, Rows{});
    }
    const f4 s = scores(B, v, lpb - 1, na_c);
    softmax_acc(s, v, na_c, Masked{}, page_rows_of(lpb - 1, na_c));
  };
  if (lpa < lpb) {
    if constexpr (kMap) {
      with_na(run_general);
    } else {
      const bool bad = lane < lpb - lpa && vb < 0;  // a page id outside the pool
      if (__builtin_amdgcn_ballot_w64(bad) == 0) with_na(run_fast);
      else with_na(run_general);
    }
  }

  // ---- merge the sub-range partials of each group (LSE rule), write split-K partials ----
  l_run += shfl_xor(l_run, 16);
  l_run += shfl_xor(l_run, 32);
  __syncthreads();  // LDS is reused for the merge
  float* mb = reinterpret_cast<float*>(lds) + (w * 64 + lane) * kMergeFloats;
  mb[0] = m_run;
  mb[1] = l_run;
  for (int t = 0; t < 8; ++t)
    for (int i = 0; i < 4; ++i) mb[4 + 4 * t + i] = acc[t][i];
  for (int i = 0; i < 4; ++i) mb[36 + i] = accr[i];
  __syncthreads();
  if (!active || si != 0) return;
  for (int o = 1; o < n_sub; ++o) {
    const float* ob = reinterpret_cast<float*>(lds) + ((gi + o * n_groups) * 64 + lane) * kMergeFloats;
    const float m2 = ob[0];
    const float M = fmaxf(m_run, m2);
    if (M == -INFINITY) continue;
    const float w1 = exp2f(m_run - M), w2 = exp2f(m2 - M);
    l_run = l_run * w1 + ob[1] * w2;
    for (int t = 0; t < 8; ++t)
      for (int i = 0; i < 4; ++i) acc[t][i] = acc[t][i] * w1 + ob[4 + 4 * t + i] * w2;
    for (int i = 0; i < 4; ++i) accr[i] = accr[i] * w1 + ob[36 + i] * w2;
    m_run = M;
  }
  if (!col_ok) return;
  int s_col = slot[0];
#pragma unroll
  for (int j = 1; j < A; ++j)
    if (jc == j) s_col = slot[j];
  const size_t row = size_t(s_col) * Hq + h * G + col % G;
  for (int t = 0; t < 8; ++t)
    *reinterpret_cast<float4*>(p.ws_acc + row * kD + 16 * t + 4 * g4) =
        make_float4(acc[t][0], acc[t][1], acc[t][2], acc[t][3]);
  *reinterpret_cast<float4*>(p.ws_accr + row * kR + 4 * g4) =
      make_float4(accr[0], accr[1], accr[2], accr[3]);
  if (g4 == 0) {
    p.ws_ml[row * 2] = m_run;
    p.ws_ml[row * 2 + 1] = l_run;
  }
}

// ---------------------------------------------------------------------------------------
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
  // RoPE of this lane's 4 frequencies j_i = perm_dim(tp, 4 g4 + i) at position
  // t = 16 (2 it + pg) + col: exact (fp64-reduced) every 32 iterations, a rotation by
  // 32 w_j per iteration in between.
  const double log2_theta = log2(static_cast<double>(p.rope_theta));
  float stc[4], sts[4];
  for (int i = 0; i < 4; ++i) {
    const double om = exp2(-2.0 * perm_dim(tp, 4 * g4 + i) / kD * log2_theta);
    double sv, cv;
    sincos(2 * kPage * om, &sv, &cv);
    stc[i] = static_cast<float>(cv);
    sts[i] = static_cast<float>(sv);
  }
  float rc[4], rs[4];
  int next_base = pg * kPage;  // the page start the recurrence stands at
  // exact cos/sin (fp64-reduced angle) of this lane's key position base + col
  auto anchor_at = [&](int base) {
    for (int i = 0; i < 4; ++i) {
      const double om = exp2(-2.0 * perm_dim(tp, 4 * g4 + i) / kD * log2_theta);
      double ang = static_cast<double>(base + col) * om;
      ang = fma(-kTwoPi, floor(ang * kInvTwoPi), ang);
      double sv, cv;
      sincos(ang, &sv, &cv);
      rc[i] = static_cast<float>(cv) * p.lora_scale;
      rs[i] = static_cast<float>(sv) * p.lora_scale;
    }
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
  float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};
  for (int rt = 0; rt < 2; ++rt) {
    for (int t = 0; t < 8; ++t) acc[rt][t] = f4{0.f, 0.f, 0.f, 0.f};
    accr[rt] = f4{0.f, 0.f, 0.f, 0.f};
  }
  const float qscale = p.sm_scale_log2;
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
    // (fp64) every 32 iterations and wherever a page does not start where it stands (a frozen
    // tail in between)
    const int base = kMap ? B.pos : lp * kPage;
    if (((it & 31) == 0 && it) || (kMap && base != next_base)) anchor_at(base);
    next_base = base + 2 * kPage;
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
      k0[i] = b0 + (x * rc[i] - y * rs[i]);
      k1[i] = b1 + (y * rc[i] + x * rs[i]);
    }
    for (int i = 0; i < 4; ++i) {  // advance to the next iteration (two pages on)
      const float c = rc[i] * stc[i] - rs[i] * sts[i];
      rs[i] = rs[i] * stc[i] + rc[i] * sts[i];
      rc[i] = c;
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
      float sc[8], pmax = -INFINITY;
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
      for (int e = 0; e < 8; ++e) pmax = fmaxf(pmax, sc[e]);
      pmax = max_over_rows(pmax) * qscale;
      const bool grow = pmax > m_run[rt] + 8.f;
      if (__builtin_amdgcn_ballot_w64(grow) != 0) {
        const float m_new = grow ? pmax : m_run[rt];
        const float alpha = __builtin_amdgcn_exp2f(m_run[rt] - m_new);
        l_run[rt] *= alpha;
        for (int t = 0; t < 8; ++t) acc[rt][t] *= alpha;
        accr[rt] *= alpha;
        m_run[rt] = m_new;
      }
      const float m_ref = max2(m_run[rt], -1e30f);
      float pr[8];
      for (int e = 0; e < 8; ++e) pr[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[e], qscale, -m_ref));
      l_run[rt] += ((pr[0] + pr[1]) + (pr[2] + pr[3])) + ((pr[4] + pr[5]) + (pr[6] + pr[7]));
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
    }
  };

  // The register buffer is refilled for iteration it + 1 as soon as iteration it has been
  // staged, so those loads fly during the whole compute phase.  Two LDS
  // buffers alternate, so one barrier per iteration suffices: iteration it + 1 stages into
  // the other buffer, and iteration it + 2 waits behind the next barrier.
  PfBuf pb_;
  load(0, pb_);
  anchor_at(pg * kPage);  // (re-anchored at the first page's start where the slot map says)
  for (int it = 0; it < n_it; ++it) {
    stage(it, pb_);
    load(min(it + 1, n_it - 1), pb_);
    __syncthreads();
    compute(it);
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
    float l = l_run[rt];
    l += shfl_xor(l, 16);
    l += shfl_xor(l, 32);
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
