// Generic (VALU, fp32 arithmetic) ResidualAttention kernels for gfx950, any supported
// shape and element type, plus the split-K combine, the prefill row write and the
// copy-on-write row copy.
//
// The attention kernel follows the fused form of the ForkKV study note
// ("7. 实现 cross-reference", core barriers (1) and (2); "4. 作者证明", Eq.(4)):
// per page, the full key of each agent is rebuilt in on-chip memory as
// bK + RoPE(s * rK B_k) (RoPE after the up-projection), scores go through an online
// softmax whose rescale factor multiplies both the base accumulator and the rank-r
// residual accumulator, and B_v is applied once after the loop (here in the combine
// kernel, or in the epilogue of the prefill kernel).
#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>

#include "forkkv_internal.h"

namespace forkkv {
namespace {

// ---- element access ---------------------------------------------------------------------
template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float ld(const float* p, size_t i) { return p[i]; }
  static __device__ __forceinline__ void st(float* p, size_t i, float v) { p[i] = v; }
};
template <> struct Elem<uint16_t> {  // bfloat16 bit patterns
  static __device__ __forceinline__ float ld(const uint16_t* p, size_t i) {
    return __uint_as_float(uint32_t(p[i]) << 16);
  }
  static __device__ __forceinline__ void st(uint16_t* p, size_t i, float v) {
    uint32_t u = __float_as_uint(v);
    if ((u & 0x7fffffffu) > 0x7f800000u) {
      p[i] = 0x7fc0;  // quiet NaN
      return;
    }
    u += 0x7fffu + ((u >> 16) & 1u);  // round to nearest, ties to even
    p[i] = static_cast<uint16_t>(u >> 16);
  }
};

constexpr double kTwoPi = 6.283185307179586476925286766559;

// Dynamic LDS layout of the generic attention kernel.

// Rows of the workgroup: decode = (agent j of the item, q head within the group);
// prefill = (query of the block, q head within the group), one agent.
template <typename T, bool kPrefill>
__global__ void __launch_bounds__(kGenericThreads)
residual_attn_generic(DecodeParams dp, PrefillParams pp) {
  extern __shared__ __align__(16) unsigned char lds[];
  using E = Elem<T>;
  const int tid = threadIdx.x;
  const int h = blockIdx.y;
  const int d = kPrefill ? pp.head_dim : dp.head_dim;
  const int r = kPrefill ? pp.rank : dp.rank;
  const int G = kPrefill ? pp.group : dp.group;
  const int Hq = kPrefill ? pp.num_q_heads : dp.num_q_heads;
  const int Hkv = kPrefill ? pp.num_kv_heads : dp.num_kv_heads;
  const int max_pages = kPrefill ? pp.max_pages : dp.max_pages;
  const int nbp = kPrefill ? pp.num_bpages : dp.num_bpages;
  const int nrp = kPrefill ? pp.num_rpages : dp.num_rpages;
  const float ls = kPrefill ? pp.lora_scale : dp.lora_scale;
  const float qscale = kPrefill ? pp.sm_scale_log2 : dp.sm_scale_log2;
  const float theta = kPrefill ? pp.rope_theta : dp.rope_theta;
  const T* bcache = static_cast<const T*>(kPrefill ? pp.bcache : dp.bcache);
  const T* rcache = static_cast<const T*>(kPrefill ? pp.rcache : dp.rcache);
  const int32_t* btab = kPrefill ? pp.btab : dp.btab;
  const int32_t* rtab = kPrefill ? pp.rtab : dp.rtab;
  const int32_t* pstart = kPrefill ? pp.pstart : dp.pstart;  // slot map (nullable)
  const T* q = static_cast<const T*>(kPrefill ? pp.q : dp.q);
  const T* Bk = static_cast<const T*>(kPrefill ? pp.Bk : dp.Bk);
  const int half = d / 2;
  const int n = Hkv * d;

  // ---- work description -----------------------------------------------------------------
  int na, lp_begin, lp_end, rows;
  int agents[kItemAgents];
  int slot_of[kItemAgents];
  int limit[kItemAgents];  // decode: keys t < limit[j]
  int a_pf = 0, q0 = 0, last_pos = 0, C = 0, QB = 0;
  if constexpr (kPrefill) {
    a_pf = blockIdx.z;
    C = pp.chunk_len;
    QB = kGenericMaxRows / G;
    if (QB * G * d > kGenericThreads * kGenericAccPerThread) QB = kGenericThreads * kGenericAccPerThread / (G * d);
    if (QB * G * r > kGenericThreads * kGenericAccrPerThread) QB = kGenericThreads * kGenericAccrPerThread / (G * r);
    q0 = blockIdx.x * QB;
    const int nq = min(QB, C - q0);
    last_pos = row_position(pp, a_pf, q0 + nq - 1);  // positions increase along the chunk
    rows = nq * G;
    na = 1;
    agents[0] = a_pf;
    lp_begin = 0;
    lp_end = page_of(pstart, max_pages, a_pf, last_pos) + 1;
  } else {
    // the grid covers the plan's item capacity; items past the live count are empty
    if (static_cast<int>(blockIdx.x) >= dp.plan[kHdrItems]) return;  // uniform per block
    const int32_t* it = dp.plan + dp.off_items + blockIdx.x * kItemInts;
    lp_begin = it[0];
    lp_end = it[0] + it[1];
    na = it[2];
    for (int j = 0; j < kItemAgents; ++j) {
      agents[j] = j < na ? it[4 + j] : 0;
      slot_of[j] = j < na ? it[4 + kItemAgents + j] : 0;
      limit[j] = j < na ? dp.plan[dp.off_lens + agents[j]] : 0;
    }
    rows = na * G;
  }
  const GenLds L = gen_lds(na, rows, d, r);
  double* inv = reinterpret_cast<double*>(lds + L.inv);
  float* cs = reinterpret_cast<float*>(lds + L.cs);
  float* sbk = reinterpret_cast<float*>(lds + L.bk);
  float* sbv = reinterpret_cast<float*>(lds + L.bv);
  float* skq = reinterpret_cast<float*>(lds + L.kq);
  float* srk = reinterpret_cast<float*>(lds + L.rk);
  float* srv = reinterpret_cast<float*>(lds + L.rv);
  float* sS = reinterpret_cast<float*>(lds + L.s);
  float* salpha = reinterpret_cast<float*>(lds + L.alpha);
  float* sm = reinterpret_cast<float*>(lds + L.m);
  float* sl = reinterpret_cast<float*>(lds + L.l);
  float* saccr = reinterpret_cast<float*>(lds + L.accr);

  for (int j = tid; j < half; j += kGenericThreads)
    inv[j] = pow(static_cast<double>(theta), -2.0 * j / d);
  for (int i = tid; i < rows; i += kGenericThreads) {
    sm[i] = -INFINITY;
    sl[i] = 0.f;
  }
  float acc[kGenericAccPerThread];
  float accr[kGenericAccrPerThread];
#pragma unroll
  for (int i = 0; i < kGenericAccPerThread; ++i) acc[i] = 0.f;
#pragma unroll
  for (int i = 0; i < kGenericAccrPerThread; ++i) accr[i] = 0.f;
  __syncthreads();

  // row -> (agent slot j, query index, head within group)
  auto row_agent = [&](int row) { return kPrefill ? 0 : row / G; };

  for (int lp = lp_begin; lp < lp_end; ++lp) {
    const int bpg = btab[size_t(agents[0]) * max_pages + lp];
    if (bpg < 0 || bpg >= nbp) continue;  // never read outside the pool
    const size_t kbase = (size_t(bpg) * 2 * Hkv + h) * kPage * d;
    const size_t vbase = (size_t(bpg) * 2 * Hkv + Hkv + h) * kPage * d;
    // Rows no query of this workgroup may read are never loaded: their contents are
    // arbitrary (even NaN) and a zero probability times NaN would still be NaN.  The page's
    // first position (shared by the item's agents, which map the same page) and the rows
    // each agent holds come from the slot map.
    const int pos0 = page_start(pstart, max_pages, agents[0], lp);
    int vrows;
    int prow[kItemAgents];  // rows of this page held by agent j
    if constexpr (kPrefill) {
      prow[0] = max(0, min(page_rows(pstart, max_pages, a_pf, lp, INT_MAX), last_pos + 1 - pos0));
      vrows = prow[0];
    } else {
      vrows = 0;
      for (int j = 0; j < na; ++j) {
        prow[j] = max(0, page_rows(pstart, max_pages, agents[j], lp, limit[j]));
        vrows = max(vrows, prow[j]);
      }
    }
    for (int i = tid; i < kPage * d; i += kGenericThreads) {
      // stored tiles are in matrix-core operand order; see TileOrder
      const int kt = (i % (kPage * 8)) / 8, kx = (i / (kPage * 8)) * 8 + i % 8;
      sbk[kt * d + kx] = kt < vrows ? E::ld(bcache, kbase + i) : 0.f;
      const int vt = ((i / 64) % 4) * 4 + i % 4, vx = (i / 256) * 16 + (i % 64) / 4;
      sbv[vt * d + vx] = vt < vrows ? E::ld(bcache, vbase + i) : 0.f;
    }
    bool rok[kItemAgents];
    for (int j = 0; j < na; ++j) {
      const int rpg = rtab[size_t(agents[j]) * max_pages + lp];
      rok[j] = rpg >= 0 && rpg < nrp;
      const size_t rb = size_t(rok[j] ? rpg : 0) * 2 * kPage * r;
      for (int i = tid; i < kPage * r; i += kGenericThreads) {
        const int kt = (i % 64) / 4, kk = (i / 64) * 4 + i % 4;
        srk[(j * kPage + kt) * r + kk] = (rok[j] && kt < vrows) ? E::ld(rcache, rb + i) : 0.f;
        const int vt = (i / (4 * r)) * 4 + i % 4, vk = (i % (4 * r)) / 4;
        srv[(j * kPage + vt) * r + vk] =
            (rok[j] && vt < vrows) ? E::ld(rcache, rb + kPage * r + i) : 0.f;
      }
    }
    for (int i = tid; i < kPage * half; i += kGenericThreads) {
      const int row = i / half, jj = i % half;
      double ang = static_cast<double>(pos0 + row) * inv[jj];
      ang -= kTwoPi * floor(ang / kTwoPi);
      double sv, cv;
      sincos(ang, &sv, &cv);
      cs[2 * i] = static_cast<float>(cv);
      cs[2 * i + 1] = static_cast<float>(sv);
    }
    __syncthreads();

    for (int j = 0; j < na; ++j) {
      const T* bk_a = Bk + size_t(agents[j]) * r * n + size_t(h) * d;
      for (int i = tid; i < kPage * half; i += kGenericThreads) {
        const int row = i / half, jj = i % half;
        float x = 0.f, y = 0.f;
        for (int k = 0; k < r; ++k) {
          const float rk = srk[(j * kPage + row) * r + k];
          x += rk * E::ld(bk_a, size_t(k) * n + jj);
          y += rk * E::ld(bk_a, size_t(k) * n + jj + half);
        }
        const float c = cs[2 * i], s = cs[2 * i + 1];
        skq[row * d + jj] = sbk[row * d + jj] + ls * (x * c - y * s);
        skq[row * d + jj + half] = sbk[row * d + jj + half] + ls * (y * c + x * s);
      }
      __syncthreads();
      const int row0 = kPrefill ? 0 : j * G;
      const int nrows = kPrefill ? rows : G;
      for (int i = tid; i < nrows * kPage; i += kGenericThreads) {
        const int row = row0 + i / kPage, t = i % kPage;
        const int pos = pos0 + t;
        size_t qoff;
        bool valid;
        if constexpr (kPrefill) {
          const int qi = q0 + row / G, g = row % G;
          qoff = ((size_t(a_pf) * C + qi) * Hq + h * G + g) * d;
          valid = t < prow[0] && pos <= row_position(pp, a_pf, qi);
        } else {
          const int g = row % G;
          qoff = (size_t(agents[j]) * Hq + h * G + g) * d;
          valid = t < prow[j];
        }
        float sc = -INFINITY;
        if (valid) {
          float dot = 0.f;
          for (int dd = 0; dd < d; ++dd) dot += E::ld(q, qoff + dd) * skq[t * d + dd];
          sc = dot * qscale;
        }
        sS[row * kPage + t] = sc;
      }
      __syncthreads();
    }

    // online softmax (log2 domain): rescale factor alpha applies to acc AND acc_r
    for (int row = tid; row < rows; row += kGenericThreads) {
      const float m_old = sm[row];
      float mx = -INFINITY;
      for (int t = 0; t < kPage; ++t) mx = fmaxf(mx, sS[row * kPage + t]);
      const float m_new = fmaxf(m_old, mx);
      float alpha = 1.f, sum = 0.f;
      if (m_new != -INFINITY) {
        alpha = exp2f(m_old - m_new);
        for (int t = 0; t < kPage; ++t) {
          const float p = exp2f(sS[row * kPage + t] - m_new);
          sS[row * kPage + t] = p;
          sum += p;
        }
      } else {
        for (int t = 0; t < kPage; ++t) sS[row * kPage + t] = 0.f;
      }
      salpha[row] = alpha;
      sl[row] = alpha * sl[row] + sum;
      sm[row] = m_new;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kGenericAccPerThread; ++i) {
      const int e = tid + i * kGenericThreads;
      if (e < rows * d) {
        const int row = e / d, dd = e % d;
        float v = 0.f;
        for (int t = 0; t < kPage; ++t) v += sS[row * kPage + t] * sbv[t * d + dd];
        acc[i] = salpha[row] * acc[i] + v;
      }
    }
#pragma unroll
    for (int i = 0; i < kGenericAccrPerThread; ++i) {
      const int e = tid + i * kGenericThreads;
      if (e < rows * r) {
        const int row = e / r, k = e % r, j = row_agent(row);
        float v = 0.f;
        for (int t = 0; t < kPage; ++t) v += sS[row * kPage + t] * srv[(j * kPage + t) * r + k];
        accr[i] = salpha[row] * accr[i] + v;
      }
    }
    __syncthreads();
  }

  if constexpr (kPrefill) {
    // epilogue: o = (acc + s * acc_r B_v) / l   (B_v applied once)
#pragma unroll
    for (int i = 0; i < kGenericAccrPerThread; ++i) {
      const int e = tid + i * kGenericThreads;
      if (e < rows * r) saccr[e] = accr[i];
    }
    __syncthreads();
    const T* Bv = static_cast<const T*>(pp.Bv);
    const T* bv_a = Bv + size_t(a_pf) * r * n + size_t(h) * d;
    T* out = static_cast<T*>(pp.out);
#pragma unroll
    for (int i = 0; i < kGenericAccPerThread; ++i) {
      const int e = tid + i * kGenericThreads;
      if (e < rows * d) {
        const int row = e / d, dd = e % d;
        float v = acc[i];
        float res = 0.f;
        for (int k = 0; k < r; ++k) res += saccr[row * r + k] * E::ld(bv_a, size_t(k) * n + dd);
        v += ls * res;
        const float l = sl[row];
        const int qi = q0 + row / G, g = row % G;
        E::st(out, ((size_t(a_pf) * C + qi) * Hq + h * G + g) * d + dd, l > 0.f ? v / l : 0.f);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < kGenericAccPerThread; ++i) {
      const int e = tid + i * kGenericThreads;
      if (e < rows * d) {
        const int row = e / d, dd = e % d, j = row / G, g = row % G;
        dp.ws_acc[(size_t(slot_of[j]) * Hq + h * G + g) * d + dd] = acc[i];
      }
    }
#pragma unroll
    for (int i = 0; i < kGenericAccrPerThread; ++i) {
      const int e = tid + i * kGenericThreads;
      if (e < rows * r) {
        const int row = e / r, k = e % r, j = row / G, g = row % G;
        dp.ws_accr[(size_t(slot_of[j]) * Hq + h * G + g) * r + k] = accr[i];
      }
    }
    for (int row = tid; row < rows; row += kGenericThreads) {
      const int j = row / G, g = row % G;
      const size_t o = (size_t(slot_of[j]) * Hq + h * G + g) * 2;
      dp.ws_ml[o] = sm[row];
      dp.ws_ml[o + 1] = sl[row];
    }
  }
}

// Split-K merge with a log-sum-exp rule, then the one-time B_v up-projection:
// o = (sum_i w_i acc_i + s * (sum_i w_i acc_r,i) B_v) / sum_i w_i l_i, w_i = 2^(m_i - M).
// One block per output row (agent, q head).  Thread (group sg of 8, lane l of 32) takes
// partials sg, sg + 8, ... and dims 4l..4l+3 (+128): all of its loads of a chunk are issued
// before any is used, so a row costs about one memory round trip; each thread merges its
// partials online and the eight groups are merged through LDS with the same rule.
constexpr int kCombineGroups = 8;
// partials per thread per chunk: a template parameter, the smallest of 2, 4, 8, 12 that
// covers the plan's largest per-agent partial count in one chunk (fewer wasted loads)

template <typename T, int kDG, int kCombinePer>
__global__ void __launch_bounds__(256) combine_kernel(DecodeParams p) {
  // kDG = float4 dim groups per thread: the 32 lanes of a group cover 128 dims each
  using E = Elem<T>;
  constexpr int kBvRegs = 16;  // B_v rows fetched before the merge; the rest after it
  __shared__ float s_m[kCombineGroups];
  __shared__ float s_l[kCombineGroups];
  __shared__ float4 s_acc[kCombineGroups][32 * kDG];
  __shared__ float4 s_ar[kCombineGroups][16];
  __shared__ float s_arf[64];
  const int row_out = blockIdx.x, tid = threadIdx.x;
  const int sg = tid >> 5, l32 = tid & 31;
  const int d = p.head_dim, r = p.rank, Hq = p.num_q_heads;
  const int a = row_out / Hq, g = row_out % Hq, h = g / p.group;
  const int n = p.num_kv_heads * d;
  // the partials of agent a are slots s0 .. s1-1 (consecutive)
  const int s0 = p.plan[p.off_slot_ptr + a], s1 = p.plan[p.off_slot_ptr + a + 1];
  const int ar_q = min(4 * l32, r - 4);     // rank quad this lane reads (clamped)
  const int od = min(tid, d - 1);           // output dim of this thread
  const T* bv = static_cast<const T*>(p.Bv) + size_t(a) * r * n + size_t(h) * d + od;
  float bvv[kBvRegs];
#pragma unroll
  for (int k = 0; k < kBvRegs; ++k) bvv[k] = E::ld(bv, size_t(min(k, r - 1)) * n);

  float m_t = -INFINITY, l_t = 0.f;
  float4 A4[kDG], Ar4 = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int e = 0; e < kDG; ++e) A4[e] = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int c0 = s0; c0 < s1; c0 += kCombineGroups * kCombinePer) {
    float mv[kCombinePer], lv[kCombinePer];
    float4 av[kCombinePer][kDG], arv[kCombinePer];
    // every load of the chunk is issued before any is used (indices clamped in range)
#pragma unroll
    for (int u = 0; u < kCombinePer; ++u) {
      const int i = c0 + sg + kCombineGroups * u;
      const size_t row = size_t(min(i, s1 - 1)) * Hq + g;
      const float2 ml = *reinterpret_cast<const float2*>(p.ws_ml + row * 2);
      mv[u] = i < s1 ? ml.x : -INFINITY;
      lv[u] = ml.y;
#pragma unroll
      for (int e = 0; e < kDG; ++e)
        av[u][e] = *reinterpret_cast<const float4*>(p.ws_acc + row * d +
                                                    min(4 * l32 + 128 * e, d - 4));
      arv[u] = *reinterpret_cast<const float4*>(p.ws_accr + row * r + ar_q);
    }
    float mc = m_t;
#pragma unroll
    for (int u = 0; u < kCombinePer; ++u) mc = fmaxf(mc, mv[u]);
    if (mc != -INFINITY) {
      const float sc = exp2f(m_t - mc);  // 0 while nothing merged yet
      l_t *= sc;
#pragma unroll
      for (int e = 0; e < kDG; ++e) {
        A4[e].x *= sc; A4[e].y *= sc; A4[e].z *= sc; A4[e].w *= sc;
      }
      Ar4.x *= sc; Ar4.y *= sc; Ar4.z *= sc; Ar4.w *= sc;
      m_t = mc;
#pragma unroll
      for (int u = 0; u < kCombinePer; ++u) {
        const float wgt = mv[u] == -INFINITY ? 0.f : exp2f(mv[u] - mc);
        l_t += wgt * lv[u];
#pragma unroll
        for (int e = 0; e < kDG; ++e) {
          A4[e].x += wgt * av[u][e].x; A4[e].y += wgt * av[u][e].y;
          A4[e].z += wgt * av[u][e].z; A4[e].w += wgt * av[u][e].w;
        }
        Ar4.x += wgt * arv[u].x; Ar4.y += wgt * arv[u].y;
        Ar4.z += wgt * arv[u].z; Ar4.w += wgt * arv[u].w;
      }
    }
  }
  // merge the eight groups (threads of one group hold the same m_t and l_t)
  if (l32 == 0) {
    s_m[sg] = m_t;
    s_l[sg] = l_t;
  }
  __syncthreads();
  float M = -INFINITY;
  for (int k = 0; k < kCombineGroups; ++k) M = fmaxf(M, s_m[k]);
  const float sc = (m_t == -INFINITY) ? 0.f : exp2f(m_t - M);
#pragma unroll
  for (int e = 0; e < kDG; ++e) {
    float4 v = A4[e];
    v.x *= sc; v.y *= sc; v.z *= sc; v.w *= sc;
    if (4 * l32 + 128 * e < d) s_acc[sg][l32 + 32 * e] = v;
  }
  if (4 * l32 < r) s_ar[sg][l32] = make_float4(Ar4.x * sc, Ar4.y * sc, Ar4.z * sc, Ar4.w * sc);
  __syncthreads();
  if (tid < r) {
    float ar = 0.f;
    for (int k = 0; k < kCombineGroups; ++k) {
      const float4 v = s_ar[k][tid >> 2];
      ar += (tid & 3) == 0 ? v.x : (tid & 3) == 1 ? v.y : (tid & 3) == 2 ? v.z : v.w;
    }
    s_arf[tid] = ar;
  }
  __syncthreads();
  float Lsum = 0.f;
  for (int k = 0; k < kCombineGroups; ++k)
    Lsum += (s_m[k] == -INFINITY) ? 0.f : exp2f(s_m[k] - M) * s_l[k];
  // output: thread tid writes dim tid (d <= 256); B_v is applied once, to the merged sum
  if (tid < d) {
    float acc = 0.f;
    const int q4 = tid >> 2, c4 = tid & 3;
    for (int k = 0; k < kCombineGroups; ++k) {
      const float4 v = s_acc[k][q4];
      acc += c4 == 0 ? v.x : c4 == 1 ? v.y : c4 == 2 ? v.z : v.w;
    }
    float res = 0.f;
#pragma unroll
    for (int k = 0; k < kBvRegs; ++k)
      if (k < r) res += s_arf[k] * bvv[k];
    for (int k = kBvRegs; k < r; ++k) res += s_arf[k] * E::ld(bv, size_t(k) * n);
    const float o = Lsum > 0.f ? (acc + p.lora_scale * res) / Lsum : 0.f;
    E::st(static_cast<T*>(p.out), (size_t(a) * Hq + g) * d + tid, o);
  }
  // decode with append: the call has read every length; the next call appends one further
  if (p.advance && g == 0 && tid == 0) p.advance[a] += 1;
}

// The same merge for d = 128, r = 16, one wave per output row and no LDS: quarter qd of the
// wave (16 lanes) takes partials qd, qd + 4, ...; lane l of a quarter holds dims 8l .. 8l+7
// of acc and entry l of acc_r.  The quarters are merged with cross-lane swaps (same rule),
// after which every lane holds the whole merged state; quarter qd then applies B_v rows
// 4qd .. 4qd+3 to its dims and the four products are summed across quarters.  B_v is read
// before the partials, so one memory round trip covers a row.
template <typename T> struct Row8;
template <> struct Row8<uint16_t> {  // 8 bf16 values (16 bytes)
  uint4 u;
  __device__ __forceinline__ void load(const uint16_t* p) { u = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ float get(int e) const {
    const uint32_t w = e < 2 ? u.x : e < 4 ? u.y : e < 6 ? u.z : u.w;
    return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
  }
};
template <> struct Row8<float> {
  float4 lo, hi;
  __device__ __forceinline__ void load(const float* p) {
    lo = *reinterpret_cast<const float4*>(p);
    hi = *reinterpret_cast<const float4*>(p + 4);
  }
  __device__ __forceinline__ float get(int e) const {
    const float4 v = e < 4 ? lo : hi;
    const int k = e & 3;
    return k == 0 ? v.x : k == 1 ? v.y : k == 2 ? v.z : v.w;
  }
};

template <typename T, int kPer>
__global__ void __launch_bounds__(64) combine_row_kernel(DecodeParams p) {
  constexpr int kDim = 128, kRank = 16;
  using E = Elem<T>;
  const int row_out = blockIdx.x, lane = threadIdx.x;
  const int qd = lane >> 4, l16 = lane & 15;
  const int Hq = p.num_q_heads;
  const int a = row_out / Hq, g = row_out % Hq, h = g / p.group;
  const size_t n = size_t(p.num_kv_heads) * kDim;
  const int s0 = p.plan[p.off_slot_ptr + a], s1 = p.plan[p.off_slot_ptr + a + 1];
  const T* bv = static_cast<const T*>(p.Bv) + size_t(a) * kRank * n + size_t(h) * kDim + 8 * l16;
  Row8<T> bvr[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) bvr[k].load(bv + size_t(4 * qd + k) * n);

  float m_t = -INFINITY, l_t = 0.f, ar = 0.f;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  for (int c0 = s0; c0 < s1; c0 += 4 * kPer) {
    float mv[kPer], lv[kPer], arv[kPer];
    float4 a0[kPer], a1[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {  // every load of the chunk before any use
      const int i = c0 + qd + 4 * u;
      const size_t row = size_t(min(i, s1 - 1)) * Hq + g;
      const float2 ml = *reinterpret_cast<const float2*>(p.ws_ml + row * 2);
      mv[u] = i < s1 ? ml.x : -INFINITY;
      lv[u] = ml.y;
      a0[u] = *reinterpret_cast<const float4*>(p.ws_acc + row * kDim + 8 * l16);
      a1[u] = *reinterpret_cast<const float4*>(p.ws_acc + row * kDim + 8 * l16 + 4);
      arv[u] = p.ws_accr[row * kRank + l16];
    }
    float mc = m_t;
#pragma unroll
    for (int u = 0; u < kPer; ++u) mc = fmaxf(mc, mv[u]);
    if (mc == -INFINITY) continue;  // nothing merged yet (uniform per quarter)
    const float sc = exp2f(m_t - mc);  // 0 while nothing merged yet
    l_t *= sc;
    ar *= sc;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= sc;
    m_t = mc;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const float wgt = mv[u] == -INFINITY ? 0.f : exp2f(mv[u] - mc);
      l_t += wgt * lv[u];
      ar += wgt * arv[u];
      acc[0] += wgt * a0[u].x; acc[1] += wgt * a0[u].y;
      acc[2] += wgt * a0[u].z; acc[3] += wgt * a0[u].w;
      acc[4] += wgt * a1[u].x; acc[5] += wgt * a1[u].y;
      acc[6] += wgt * a1[u].z; acc[7] += wgt * a1[u].w;
    }
  }
  // merge the quarters: partner quarter qd ^ 1, then qd ^ 2
#pragma unroll
  for (int mask = 16; mask <= 32; mask *= 2) {
    const float mo = __shfl_xor(m_t, mask, 64);
    const float lo = __shfl_xor(l_t, mask, 64);
    const float aro = __shfl_xor(ar, mask, 64);
    float acco[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acco[e] = __shfl_xor(acc[e], mask, 64);
    const float M = fmaxf(m_t, mo);
    const float w1 = m_t == -INFINITY ? 0.f : exp2f(m_t - M);
    const float w2 = mo == -INFINITY ? 0.f : exp2f(mo - M);
    l_t = l_t * w1 + lo * w2;
    ar = ar * w1 + aro * w2;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = acc[e] * w1 + acco[e] * w2;
    m_t = M;
  }
  // B_v, once: quarter qd sums ranks 4qd .. 4qd+3 (acc_r entry k sits in lane k)
  float res[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) res[e] = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float rk = __shfl(ar, 4 * qd + k, 64);
#pragma unroll
    for (int e = 0; e < 8; ++e) res[e] += rk * bvr[k].get(e);
  }
#pragma unroll
  for (int mask = 16; mask <= 32; mask *= 2)
#pragma unroll
    for (int e = 0; e < 8; ++e) res[e] += __shfl_xor(res[e], mask, 64);
  if (qd == 0) {
    T* o = static_cast<T*>(p.out) + (size_t(a) * Hq + g) * kDim + 8 * l16;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      E::st(o, e, l_t > 0.f ? (acc[e] + p.lora_scale * res[e]) / l_t : 0.f);
  }
  // decode with append: the call has read every length; the next call appends one further
  if (p.advance && g == 0 && lane == 0) p.advance[a] += 1;
}

// Store the chunk rows at their slots (bit-exact copies in the pool layout).  The slot of
// position t is its page under the slot map and its offset from the page's start; a row
// whose slot falls outside a page (a malformed start table) is not stored.
template <typename T>
__global__ void __launch_bounds__(256) prefill_write_kernel(PrefillParams p) {
  const int i = blockIdx.x, a = blockIdx.y, tid = threadIdx.x;
  const int d = p.head_dim, r = p.rank, Hkv = p.num_kv_heads, C = p.chunk_len;
  const int t = row_position(p, a, i);
  const int lp = page_of(p.pstart, p.max_pages, a, t);
  const int row = t - page_start(p.pstart, p.max_pages, a, lp);
  if (lp < 0 || lp >= p.max_pages || row < 0 || row >= kPage) return;
  const int bpg = p.btab[size_t(a) * p.max_pages + lp];
  const int rpg = p.write_res ? p.rtab[size_t(a) * p.max_pages + lp] : -1;
  T* bc = static_cast<T*>(p.bcache);
  T* rc = static_cast<T*>(p.rcache);
  const T* kn = static_cast<const T*>(p.k_new) + (size_t(a) * C + i) * Hkv * d;
  const T* vn = static_cast<const T*>(p.v_new) + (size_t(a) * C + i) * Hkv * d;
  if (bpg >= 0 && bpg < p.num_bpages) {
    for (int idx = tid; idx < Hkv * d; idx += blockDim.x) {
      const int h = idx / d, dd = idx % d;
      bc[(size_t(bpg) * 2 * Hkv + h) * kPage * d + TileOrder::key(row, dd)] = kn[idx];
      bc[(size_t(bpg) * 2 * Hkv + Hkv + h) * kPage * d + TileOrder::value(row, dd)] = vn[idx];
    }
  }
  if (rpg >= 0 && rpg < p.num_rpages) {
    const T* rkn = static_cast<const T*>(p.rk_new) + (size_t(a) * C + i) * r;
    const T* rvn = static_cast<const T*>(p.rv_new) + (size_t(a) * C + i) * r;
    for (int k = tid; k < r; k += blockDim.x) {
      rc[size_t(rpg) * 2 * kPage * r + TileOrder::res_key(row, k)] = rkn[k];
      rc[size_t(rpg) * 2 * kPage * r + kPage * r + TileOrder::res_value(row, k, r)] = rvn[k];
    }
  }
}

// Copy the first n rows of base page src into page dst, every KV head, K and V planes.
template <typename T>
__global__ void __launch_bounds__(256) cow_copy_kernel(T* bc, int Hkv, int d, int src, int dst,
                                                       int nrows) {
  const int total = 2 * Hkv * kPage * d;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < total; i += gridDim.x * blockDim.x) {
    const int plane = i / (Hkv * kPage * d);
    const int rem = i % (kPage * d);
    const int row = plane == 0 ? (rem % (kPage * 8)) / 8 : ((rem / 64) % 4) * 4 + rem % 4;
    if (row < nrows) bc[size_t(dst) * total + i] = bc[size_t(src) * total + i];
  }
}

int prefill_rows(int G, int d, int r) {
  int QB = kGenericMaxRows / G;
  if (QB * G * d > kGenericThreads * kGenericAccPerThread) QB = kGenericThreads * kGenericAccPerThread / (G * d);
  if (QB * G * r > kGenericThreads * kGenericAccrPerThread) QB = kGenericThreads * kGenericAccrPerThread / (G * r);
  return QB;
}

}  // namespace

// Launch one instantiation of the generic kernel with lds bytes of dynamic LDS.
template <typename T, bool kPrefill>
hipError_t launch_generic(dim3 grid, int lds, hipStream_t s, const DecodeParams& dp,
                          const PrefillParams& pp) {
  if (lds > kMaxLds) return hipErrorInvalidValue;
  if (lds > kDefaultDynLds) {
    const hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&residual_attn_generic<T, kPrefill>),
        hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((residual_attn_generic<T, kPrefill>), grid, dim3(kGenericThreads), lds, s,
                     dp, pp);
  return hipGetLastError();
}

hipError_t launch_decode_generic(const DecodeParams& p, int dtype, int max_agents, hipStream_t s) {
  const int rows = max_agents * p.group;
  const int lds = gen_lds(max_agents, rows, p.head_dim, p.rank).total;
  dim3 grid(p.n_items, p.num_kv_heads);
  PrefillParams none{};
  return dtype == FORKKV_DTYPE_F32 ? launch_generic<float, false>(grid, lds, s, p, none)
                                   : launch_generic<uint16_t, false>(grid, lds, s, p, none);
}

template <typename T, int kDG>
void launch_combine_per(const DecodeParams& p, dim3 grid, hipStream_t s) {
  const int need = (p.max_agent_slots + kCombineGroups - 1) / kCombineGroups;
  if (need <= 2)
    hipLaunchKernelGGL((combine_kernel<T, kDG, 2>), grid, dim3(256), 0, s, p);
  else if (need <= 4)
    hipLaunchKernelGGL((combine_kernel<T, kDG, 4>), grid, dim3(256), 0, s, p);
  else if (need <= 8)
    hipLaunchKernelGGL((combine_kernel<T, kDG, 8>), grid, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((combine_kernel<T, kDG, 12>), grid, dim3(256), 0, s, p);
}

template <typename T>
void launch_combine_rows(const DecodeParams& p, dim3 grid, hipStream_t s) {
  // partials per lane per chunk: the smallest of 2, 4, 8, 16 covering the largest agent's
  const int need = (p.max_agent_slots + 3) / 4;
  if (need <= 2)
    hipLaunchKernelGGL((combine_row_kernel<T, 2>), grid, dim3(64), 0, s, p);
  else if (need <= 4)
    hipLaunchKernelGGL((combine_row_kernel<T, 4>), grid, dim3(64), 0, s, p);
  else if (need <= 8)
    hipLaunchKernelGGL((combine_row_kernel<T, 8>), grid, dim3(64), 0, s, p);
  else
    hipLaunchKernelGGL((combine_row_kernel<T, 16>), grid, dim3(64), 0, s, p);
}

hipError_t launch_combine(const DecodeParams& p, int dtype, hipStream_t s) {
  if (p.head_dim > 256 || p.rank > 64) return hipErrorInvalidValue;
  dim3 grid(p.n_agents * p.num_q_heads);
  if (p.head_dim == 128 && p.rank == 16) {
    if (dtype == FORKKV_DTYPE_F32) launch_combine_rows<float>(p, grid, s);
    else launch_combine_rows<uint16_t>(p, grid, s);
    return hipGetLastError();
  }
  const bool wide = p.head_dim > 128;
  if (dtype == FORKKV_DTYPE_F32) {
    if (wide) launch_combine_per<float, 2>(p, grid, s);
    else launch_combine_per<float, 1>(p, grid, s);
  } else {
    if (wide) launch_combine_per<uint16_t, 2>(p, grid, s);
    else launch_combine_per<uint16_t, 1>(p, grid, s);
  }
  return hipGetLastError();
}

hipError_t launch_prefill_write(const PrefillParams& p, int dtype, hipStream_t s) {
  dim3 grid(p.chunk_len, p.n_agents);
  if (dtype == FORKKV_DTYPE_F32)
    hipLaunchKernelGGL(prefill_write_kernel<float>, grid, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(prefill_write_kernel<uint16_t>, grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_prefill_generic(const PrefillParams& p, int dtype, hipStream_t s) {
  const int QB = prefill_rows(p.group, p.head_dim, p.rank);
  if (QB < 1) return hipErrorInvalidValue;
  const int lds = gen_lds(1, QB * p.group, p.head_dim, p.rank).total;
  dim3 grid((p.chunk_len + QB - 1) / QB, p.num_kv_heads, p.n_agents);
  DecodeParams none{};
  return dtype == FORKKV_DTYPE_F32 ? launch_generic<float, true>(grid, lds, s, none, p)
                                   : launch_generic<uint16_t, true>(grid, lds, s, none, p);
}

hipError_t launch_cow_copy(void* bcache, int dtype, int Hkv, int d, int32_t src, int32_t dst,
                           int32_t n_rows, hipStream_t s) {
  const int total = 2 * Hkv * kPage * d;
  const int blocks = (total + 255) / 256;
  if (dtype == FORKKV_DTYPE_F32)
    hipLaunchKernelGGL(cow_copy_kernel<float>, dim3(blocks), dim3(256), 0, s,
                       static_cast<float*>(bcache), Hkv, d, src, dst, n_rows);
  else
    hipLaunchKernelGGL(cow_copy_kernel<uint16_t>, dim3(blocks), dim3(256), 0, s,
                       static_cast<uint16_t*>(bcache), Hkv, d, src, dst, n_rows);
  return hipGetLastError();
}

}  // namespace forkkv
