// What each kernel covers (host side): the shapes the MFMA kernels take, how many agents a
// decode work item holds for each kernel, and the generic kernel's limits.  The planner
// and the C-ABI entry points decide with these; the kernels are built to them.
#include "forkkv_internal.h"

namespace forkkv {

// bf16, d = 128, r = 16 and a GQA group of at most 16 query heads (one wave's columns).
bool mfma_supported(int dtype, int head_dim, int rank, int group) {
  return dtype == FORKKV_DTYPE_BF16 && head_dim == kMfmaHeadDim && rank == kMfmaRank &&
         mfma_agents_per_group(group) >= 1;
}

int mfma_agents_per_wave(int group) { return mfma_agents_per_group(group); }

// Agents per plan item: up to four groups (one per wave) of mfma_agents_per_group(G) each,
// at most kItemAgents.
int mfma_group_agents(int group) {
  const int A = mfma_agents_per_group(group);
  return A > 0 ? std::min(kItemAgents, kMfmaWaves * A) : 0;
}

bool prefill_mfma_enabled() { return true; }

int generic_lds_bytes(int na, int rows, int d, int r) { return gen_lds(na, rows, d, r).total; }

// The most agents an item of the generic kernel holds: its rows (agents x G) must fit the
// thread-owned accumulators and its LDS plan the workgroup's LDS.
int generic_max_agents(int group, int head_dim, int rank) {
  int best = 0;
  for (int na = 1; na <= kItemAgents; ++na) {
    const int rows = na * group;
    if (rows > kGenericMaxRows) break;
    if (rows * head_dim > kGenericThreads * kGenericAccPerThread) break;
    if (rows * rank > kGenericThreads * kGenericAccrPerThread) break;
    if (gen_lds(na, rows, head_dim, rank).total > kMaxLds) break;
    best = na;
  }
  return best;
}

}  // namespace forkkv
