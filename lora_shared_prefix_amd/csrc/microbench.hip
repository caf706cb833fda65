// Device ceilings measured on the box the bench runs on (not part of the ResidualAttention
// library; built into libforkkv_microbench.so and called by bench.py):
//   * a read-only streaming reduction: every 16-byte vector of a buffer larger than the
//     256 MB Infinity Cache is read once per pass and summed (uint64 per workgroup), so the
//     caller can check the sum -- the practical HBM read ceiling for a kernel that, like the
//     decode split kernel, only reads;
//   * a bf16 matrix-core loop: every wave runs chains of independent 16x16x32 bf16 MFMAs on
//     operands read from memory (A = 1, B = 1/32, so each instruction adds exactly 1.0 to
//     every accumulator element) and writes its accumulators' sum, which the caller checks --
//     the practical dense bf16 MFMA ceiling;
//   * a pipe probe: how the matrix cores of a SIMD share it with another wave's vector,
//     transcendental or LDS work.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

constexpr int kThreads = 256;

// kUnroll independent 16-byte loads in flight per thread; kNt: non-temporal loads (the
// data streams through the caches without displacing other lines)
template <int kUnroll, bool kNt>
__global__ void __launch_bounds__(kThreads)
stream_read_kernel(const uint4* __restrict__ buf, size_t n_vec, unsigned long long* partials) {
  const size_t stride = size_t(gridDim.x) * kThreads;
  size_t i = size_t(blockIdx.x) * kThreads + threadIdx.x;
  unsigned long long sum = 0;
  typedef unsigned int u4v __attribute__((ext_vector_type(4)));
  auto ld = [&](size_t k) -> uint4 {
    if constexpr (kNt) {
      const u4v v = __builtin_nontemporal_load(reinterpret_cast<const u4v*>(buf) + k);
      return make_uint4(v.x, v.y, v.z, v.w);
    }
    return buf[k];
  };
  for (; i + (kUnroll - 1) * stride < n_vec; i += kUnroll * stride) {
    uint4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = ld(i + u * stride);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      sum += (unsigned long long)v[u].x + v[u].y + v[u].z + v[u].w;
  }
  for (; i < n_vec; i += stride) {
    const uint4 v = ld(i);
    sum += (unsigned long long)v.x + v.y + v.z + v.w;
  }
  // wave reduction, then across the block's waves through LDS
  for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off, 64);
  __shared__ unsigned long long ws[kThreads / 64];
  if ((threadIdx.x & 63) == 0) ws[threadIdx.x >> 6] = sum;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned long long s = 0;
    for (int w = 0; w < kThreads / 64; ++w) s += ws[w];
    partials[blockIdx.x] = s;
  }
}

typedef __bf16 bf8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f4 __attribute__((__vector_size__(4 * sizeof(float))));
constexpr int kChains = 8;  // independent accumulators per wave (covers the MFMA latency)

__global__ void __launch_bounds__(kThreads)
mfma_bf16_kernel(const uint4* __restrict__ ops, int iters, float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  union { uint4 u; bf8 b; } a, b;
  a.u = ops[0];  // eight bf16 1.0
  b.u = ops[1];  // eight bf16 1/32
  f4 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = f4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c)
      acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.b, b.b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  // every element of every accumulator holds iters: s = 4 * kChains * iters in each lane
  if (lane == 0) out[(size_t(blockIdx.x) * kThreads + threadIdx.x) / 64] = s;
}

// How the instruction pipes of one SIMD are shared: 512-thread workgroups, one per compute
// unit, so waves w and w + 4 share a SIMD.  Waves 0-3 (when kM) run 16 bf16 16x16x32 MFMAs
// per trip in kChainsP independent accumulator chains; waves 4-7 run one kind of work per
// trip: kMode 0 nothing, 1 = 64 independent fp32 FMAs, 2 = 64 exp2, 3 = 16 ds_read_b128.
// With kBoth, waves 0-3 run that same work instead of MFMAs.  Each wave writes one value
// derived from its results (so nothing is optimized away).
constexpr int kProbeThreads = 512;
constexpr int kProbeLds = 8 * kProbeThreads;  // uint4 elements

template <int kMode, bool kM, int kChainsP, bool kBoth = false>
__global__ void __launch_bounds__(kProbeThreads) __attribute__((amdgpu_waves_per_eu(2)))
pipe_probe_kernel(const uint4* __restrict__ ops, int iters, float* __restrict__ out) {
  __shared__ uint4 lds[kProbeLds];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int i = threadIdx.x; i < kProbeLds; i += kProbeThreads) lds[i] = make_uint4(i, 1, 2, 3);
  __syncthreads();
  float result = 0.f;
  if (w < 4 && !kBoth) {
    if constexpr (kM) {
      union { uint4 u; bf8 b; } a, b;
      a.u = ops[0];
      b.u = ops[1];
      f4 acc[kChainsP];
#pragma unroll
      for (int c = 0; c < kChainsP; ++c) acc[c] = f4{0.f, 0.f, 0.f, 0.f};
      for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int r = 0; r < 16 / kChainsP; ++r)
#pragma unroll
          for (int c = 0; c < kChainsP; ++c)
            acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.b, b.b, acc[c], 0, 0, 0);
      }
#pragma unroll
      for (int c = 0; c < kChainsP; ++c) result += acc[c][0];
    }
  } else {
    float x[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] = -1.0f - 0.001f * (lane + k);
    unsigned int acc = 0;
    for (int i = 0; i < iters; ++i) {
      if constexpr (kMode == 1) {
#pragma unroll
        for (int r = 0; r < 8; ++r)
#pragma unroll
          for (int k = 0; k < 8; ++k) x[k] = __builtin_fmaf(x[k], 0.9999f, -0.0001f);
      } else if constexpr (kMode == 2) {
#pragma unroll
        for (int r = 0; r < 8; ++r)
#pragma unroll
          for (int k = 0; k < 8; ++k) x[k] = __builtin_amdgcn_exp2f(x[k]) - 1.5f;
      } else if constexpr (kMode == 3) {
#pragma unroll
        for (int k = 0; k < 16; ++k) {  // index < 8 * 512: always inside lds
          const uint4 v = lds[((i + k) & 7) * kProbeThreads + (w & 3) * 64 + lane];
          acc += v.x ^ v.y ^ v.z ^ v.w;
        }
      }
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) result += x[k];
    result += static_cast<float>(acc & 1u);
  }
  if (lane == 0) out[blockIdx.x * (kProbeThreads / 64) + w] = result;
}

}  // namespace

extern "C" {

// Sum of all 32-bit words of buf (n_bytes, a multiple of 16, 16-byte aligned) into
// n_blocks uint64 partials (device).  Returns the hipError_t of the launch.
// variant: 0 = 4 loads in flight per thread, 1 = 8, 2 = 8 non-temporal.
int mb_stream_read(const void* buf, size_t n_bytes, unsigned long long* partials, int n_blocks,
                   int variant, hipStream_t stream) {
  const uint4* b = static_cast<const uint4*>(buf);
  const size_t n = n_bytes / 16;
  if (variant == 0)
    hipLaunchKernelGGL((stream_read_kernel<4, false>), dim3(n_blocks), dim3(kThreads), 0, stream,
                       b, n, partials);
  else if (variant == 1)
    hipLaunchKernelGGL((stream_read_kernel<8, false>), dim3(n_blocks), dim3(kThreads), 0, stream,
                       b, n, partials);
  else if (variant == 2)
    hipLaunchKernelGGL((stream_read_kernel<8, true>), dim3(n_blocks), dim3(kThreads), 0, stream,
                       b, n, partials);
  else
    return static_cast<int>(hipErrorInvalidValue);
  return static_cast<int>(hipGetLastError());
}

// n_blocks x 4 waves, each running kChains chains of iters bf16 16x16x32 MFMAs; out gets one
// float per wave (4 * kChains * iters when correct).  ops: 32 bytes of device memory holding
// eight bf16 1.0 followed by eight bf16 1/32.  Flops per call: n_blocks * 4 * kChains * iters
// * 2 * 16 * 16 * 32.
int mb_mfma_bf16(const void* ops, int iters, float* out, int n_blocks, hipStream_t stream) {
  hipLaunchKernelGGL(mfma_bf16_kernel, dim3(n_blocks), dim3(kThreads), 0, stream,
                     static_cast<const uint4*>(ops), iters, out);
  return static_cast<int>(hipGetLastError());
}

int mb_mfma_chains() { return kChains; }

// The pipe probe above: n_blocks workgroups of 512 threads (one per compute unit on
// MI355X: n_blocks = 256), iters trips.  mode 0..3 selects the work of waves 4-7, mfma (0/1)
// whether waves 0-3 run their MFMAs (2: waves 0-3 run the same work as waves 4-7), chains
// (1, 2, 4 or 16) the MFMAs' independent accumulator chains.  ops as for mb_mfma_bf16; out: n_blocks * 8 floats.  Returns the hipError_t of the
// launch (hipErrorInvalidValue for an unknown combination).
int mb_pipe_probe(int mode, int mfma, int chains, const void* ops, int iters, float* out,
                  int n_blocks, hipStream_t stream) {
  const uint4* o = static_cast<const uint4*>(ops);
  if (mfma == 2) {  // both waves of a SIMD run the same work
    if (chains != 4 || mode < 1 || mode > 3) return static_cast<int>(hipErrorInvalidValue);
    if (mode == 1)
      hipLaunchKernelGGL((pipe_probe_kernel<1, false, 4, true>), dim3(n_blocks),
                         dim3(kProbeThreads), 0, stream, o, iters, out);
    else if (mode == 2)
      hipLaunchKernelGGL((pipe_probe_kernel<2, false, 4, true>), dim3(n_blocks),
                         dim3(kProbeThreads), 0, stream, o, iters, out);
    else
      hipLaunchKernelGGL((pipe_probe_kernel<3, false, 4, true>), dim3(n_blocks),
                         dim3(kProbeThreads), 0, stream, o, iters, out);
    return static_cast<int>(hipGetLastError());
  }
#define MB_PROBE(M, F, C)                                                                  \
  if (mode == M && (mfma != 0) == F && chains == C) {                                      \
    hipLaunchKernelGGL((pipe_probe_kernel<M, F, C>), dim3(n_blocks), dim3(kProbeThreads), 0, \
                       stream, o, iters, out);                                             \
    return static_cast<int>(hipGetLastError());                                            \
  }
  MB_PROBE(0, true, 1) MB_PROBE(0, true, 2) MB_PROBE(0, true, 4) MB_PROBE(0, true, 16)
  MB_PROBE(1, true, 4) MB_PROBE(1, false, 4)
  MB_PROBE(2, true, 4) MB_PROBE(2, false, 4)
  MB_PROBE(3, true, 4) MB_PROBE(3, false, 4)
#undef MB_PROBE
  return static_cast<int>(hipErrorInvalidValue);
}

}  // extern "C"
