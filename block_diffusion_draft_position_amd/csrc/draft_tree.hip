// The draft side of a round in one launch after the top-K chunk pass: per-position
// top-K merge (DDTree page "策展 · X (Twitter)", section 運作流程 step 1), tree
// selection under the node budget (核心創新; 運作流程 step 2; 理論基礎) and the
// ancestor-only mask with position ids (核心創新; 運作流程 step 3).
//
// One workgroup per sequence.  Wave 0 merges draft position 0's chunk lists
// (topk::merge_row) straight into the tree builder's LDS table, the other waves the
// remaining positions, each row flagged in LDS once written.  Wave 0 then selects and
// numbers the tree (tree::build, synchronising with wave barriers), waiting on a
// row's flag only when a round first needs it, so the build overlaps the merges of
// the deeper positions; finally every wave forms mask rows from the canonical parent
// array the builder left in LDS (mask::rows).  The results are identical to
// ddt_topk -> ddt_build_tree -> ddt_tree_mask; this path saves two launches and the
// global round trips between them.
#include "build_tree_device.h"
#include "topk_device.h"
#include "tree_mask_device.h"

namespace ddt {
namespace {

// waves per workgroup: as many merge waves as registers allow next to the builder
__host__ __device__ constexpr int waves_for(int J, int ME) {
  return (J >= 16 || ME >= 64) ? 4 : (J >= 4 || ME == 32) ? 8 : 16;
}

template <int J, int SK, int ME>
__global__ void __launch_bounds__(waves_for(J, ME) * kWave)
draft_tree_kernel(const unsigned long long* __restrict__ cand, const float2* __restrict__ stats,
                  int nchunks, const int32_t* __restrict__ bonus,
                  Prefix pre, int L, int K, int B,
                  int32_t* __restrict__ topk_tok, float* __restrict__ topk_logq,
                  int32_t* __restrict__ tree_tok, int32_t* __restrict__ tree_parent,
                  int32_t* __restrict__ tree_depth, float* __restrict__ node_logq,
                  int32_t* __restrict__ num_nodes, uint32_t* __restrict__ mask,
                  int32_t* __restrict__ pos_ids) {
  constexpr int NW = waves_for(J, ME);
  extern __shared__ __align__(16) unsigned char smem_raw[];
  __shared__ int nn_s;
  __shared__ int ready[DDT_MAX_L];  // row i of the LDS table is written
  const int s = blockIdx.x;
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int N = B + 1;
  const int LK = L * K;
  const int W = (N + 31) / 32;
  topk::WaveLds* wl = reinterpret_cast<topk::WaveLds*>(smem_raw);
  tree::TreeSmem sm = tree::carve(smem_raw + NW * sizeof(topk::WaveLds), N, LK);
  // the builder's scalars, requested now so they arrive during the merge
  const int bonus_tok = bonus[s];
  const int P = (pos_ids && pre.cu) ? (int)pre.length(s) : 0;

  for (int i = threadIdx.x; i < DDT_MAX_L; i += NW * kWave) ready[i] = 0;
  __syncthreads();
  // wave 0 takes position 0 only, so that it reaches the build early; waves 1 .. NW-1
  // take the others in turn
  for (int i = wave; i < L; i = wave == 0 ? L : (i < NW ? NW + wave - 1 : i + NW - 1)) {
    const int64_t row = (int64_t)s * L + i;
    float rv;
    int ri;
    double lse;
    topk::merge_row<ME>(row, nchunks, K, cand, stats, wl[wave], rv, ri, lse);
    if (lane < K) {
      const float lqv = (float)((double)rv - lse);
      sm.lq[i * K + lane] = lqv;
      sm.ltok[i * K + lane] = ri;
      if (topk_tok) topk_tok[row * K + lane] = ri;
      if (topk_logq) topk_logq[row * K + lane] = lqv;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");  // the row, then its flag
    if (lane == 0) __hip_atomic_store(&ready[i], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
  if (wave == 0) {
    const int64_t o = (int64_t)s * N;
    const int n = tree::build<J, SK>(sm, L, K, B, bonus_tok, tree_tok + o, tree_parent + o,
                                     tree_depth + o, node_logq ? node_logq + o : nullptr,
                                     (pos_ids && pre.cu) ? pos_ids + o : nullptr, P,
                                     [] { topk::wave_lds_sync(); },
                                     [&](int m) {
                                       for (;;) {
                                         bool ok = true;
                                         for (int i = lane; i < m; i += kWave)
                                           ok &= __hip_atomic_load(&ready[i], __ATOMIC_RELAXED,
                                                                   __HIP_MEMORY_SCOPE_WORKGROUP) != 0;
                                         if (!ballot(!ok)) break;
                                         __builtin_amdgcn_s_sleep(1);
                                       }
                                       __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
                                     });
    if (lane == 0) {
      num_nodes[s] = n;
      nn_s = n;
    }
  }
  __syncthreads();
  mask::rows(sm.cpar, nn_s, N, W, mask + (int64_t)s * N * W, threadIdx.x, NW * kWave, 0, N * W);
}

template <int J, int SK, int ME>
hipError_t launch_jkm(const unsigned long long* cand, const float2* stats, int nchunks,
                      const int32_t* bonus, Prefix pre, int S, int L, int K, int B,
                      int32_t* topk_tok, float* topk_logq, int32_t* tree_tok, int32_t* parent,
                      int32_t* depth, float* node_logq, int32_t* num_nodes, uint32_t* mask,
                      int32_t* pos_ids, hipStream_t st) {
  constexpr int NW = waves_for(J, ME);
  const size_t smem = NW * sizeof(topk::WaveLds) + tree::smem_bytes(B + 1, L * K);
  if (smem > 48 * 1024) {
    const hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&draft_tree_kernel<J, SK, ME>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((draft_tree_kernel<J, SK, ME>), dim3(S), dim3(NW * kWave), smem, st, cand,
                     stats, nchunks, bonus, pre, L, K, B, topk_tok, topk_logq, tree_tok,
                     parent, depth, node_logq, num_nodes, mask, pos_ids);
  return hipGetLastError();
}

template <int J, int ME>
hipError_t launch_jm(int K, const unsigned long long* cand, const float2* stats, int nchunks,
                     const int32_t* bonus, Prefix pre, int S, int L, int B,
                     int32_t* topk_tok, float* topk_logq, int32_t* tree_tok, int32_t* parent,
                     int32_t* depth, float* node_logq, int32_t* num_nodes, uint32_t* mask,
                     int32_t* pos_ids, hipStream_t st) {
#define DDT_ARGS_SK                                                                         \
  cand, stats, nchunks, bonus, pre, S, L, K, B, topk_tok, topk_logq, tree_tok, parent, \
      depth, node_logq, num_nodes, mask, pos_ids, st
  if constexpr (J <= 2) {
    if (K <= 8) return launch_jkm<J, 8, ME>(DDT_ARGS_SK);
    if (K <= 16) return launch_jkm<J, 16, ME>(DDT_ARGS_SK);
  }
  return launch_jkm<J, 0, ME>(DDT_ARGS_SK);
#undef DDT_ARGS_SK
}

int slots_for(int B) { return (int)ceil_div(B + 1, kWave); }

int j_for(int B) {
  const int slots = slots_for(B);
  return slots <= 1 ? 1 : slots <= 2 ? 2 : slots <= 4 ? 4 : slots <= 8 ? 8 : 16;
}

}  // namespace

bool draft_tree_uses_fused(int L, int K, int B, const TopkPlan& plan) {
  (void)K;
  return waves_for(j_for(B), plan.merge_e) >= std::min(L, 16);
}

hipError_t launch_draft_tree(const void* ws, const TopkPlan& plan, const int32_t* bonus,
                             Prefix pre, int S, int L, int K, int B,
                             int32_t* topk_tok, float* topk_logq, int32_t* tree_tok,
                             int32_t* parent, int32_t* depth, float* node_logq,
                             int32_t* num_nodes, uint32_t* mask, int32_t* pos_ids,
                             hipStream_t st) {
  if (!draft_tree_uses_fused(L, K, B, plan)) {
    // too few merge waves fit next to this builder: merge, build and mask separately
    hipError_t e = launch_topk_merge((int64_t)S * L, K, topk_tok, topk_logq,
                                     const_cast<void*>(ws), plan, st);
    if (e != hipSuccess) return e;
    e = launch_build_tree(topk_tok, topk_logq, bonus, S, L, K, B, tree_tok, parent, depth,
                          node_logq, num_nodes, st);
    if (e != hipSuccess) return e;
    return launch_tree_mask(parent, depth, num_nodes, pre, S, B, mask, pos_ids, st);
  }
  unsigned long long* cand;
  float2* stats;
  topk_ws_parts(const_cast<void*>(ws), (int64_t)S * L, K, plan, &cand, &stats);
  const int slots = slots_for(B);
#define DDT_ARGS                                                                               \
  K, cand, stats, plan.nchunks, bonus, pre, S, L, B, topk_tok, topk_logq, tree_tok, parent, \
      depth, node_logq, num_nodes, mask, pos_ids, st
#define DDT_J(JJ)                                                              \
  return plan.merge_e == 8 ? launch_jm<JJ, 8>(DDT_ARGS)    \
       : plan.merge_e == 32 ? launch_jm<JJ, 32>(DDT_ARGS) \
                            : launch_jm<JJ, 64>(DDT_ARGS)
  if (slots <= 1) DDT_J(1);
  if (slots <= 2) DDT_J(2);
  if (slots <= 4) DDT_J(4);
  if (slots <= 8) DDT_J(8);
  DDT_J(16);
#undef DDT_J
#undef DDT_ARGS
}

}  // namespace ddt
