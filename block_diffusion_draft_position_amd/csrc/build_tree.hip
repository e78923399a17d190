// Draft-tree construction under a node budget: the B most probable draft prefixes
// (DDTree page "策展 · X (Twitter)": section 核心創新 for the best-first selection
// under a budget, 運作流程 step 2 for the construction, 理論基礎 for the factorised
// prefix probability and the prefix-closure of the optimum).
//
// One wavefront per sequence.  The candidates form a K-ary tree whose depth-i
// children are position i's top-K tokens, sorted by probability.  Every selected
// node u (the root included) owns a stream: its not-yet-selected children in rank
// order, scoring score(u) + logq[depth(u)][r] for r = cursor(u) .. K-1, a
// non-increasing sequence.  A candidate outside the streams descends from a stream
// candidate y and scores at most score(y) + logq[depth(y)][0].  So with
//     tau = max over streams u of  head(u) + logq[depth(u) + 1][0]
// (head(u) = u's best remaining child), every stream candidate scoring above tau
// ranks ahead of every candidate not yet in a stream, and one round selects all of
// them at once: they are the next pops of a best-first heap, as a set.  If that is
// more than the remaining budget R, the round keeps the R best of them (a radix
// select over the fp64 scores); if it is none (probability-1 positions), it takes
// the single best stream head.  Flat drafts finish in two or three rounds; a
// confident chain takes about one round per depth.
//
// Selection is by the fp64 score (sum of the fp32 log-probabilities along the
// path); equal scores at the budget boundary are taken in node order.
// The selected nodes are then renumbered canonically: by depth, then the parent's
// canonical index, then sibling rank (a stream is consumed from its head, so a
// node's selected children are exactly ranks 0 .. cursor-1).
#include "build_tree_device.h"

namespace ddt {
namespace {

template <int J, int SK>
__global__ void __launch_bounds__(kWave)
build_tree_kernel(const int32_t* __restrict__ topk_tok, const float* __restrict__ topk_logq,
                  const int32_t* __restrict__ bonus, int L, int K, int B,
                  int32_t* __restrict__ tree_tok, int32_t* __restrict__ tree_parent,
                  int32_t* __restrict__ tree_depth, float* __restrict__ node_logq,
                  int32_t* __restrict__ num_nodes) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  const int s = blockIdx.x;
  const int lane = threadIdx.x;
  const int N = B + 1;
  const int LK = L * K;
  tree::TreeSmem sm = tree::carve(smem_raw, N, LK);
  const float* lq_g = topk_logq + (int64_t)s * LK;
  const int32_t* tok_g = topk_tok + (int64_t)s * LK;
  const int bonus_tok = bonus[s];  // requested with the table, used at the end
  for (int i = lane; i < LK; i += kWave) {
    sm.lq[i] = lq_g[i];
    sm.ltok[i] = tok_g[i];
  }
  __syncthreads();
  const int64_t o = (int64_t)s * N;
  const int n = tree::build<J, SK>(sm, L, K, B, bonus_tok, tree_tok + o, tree_parent + o,
                                   tree_depth + o, node_logq ? node_logq + o : nullptr, nullptr,
                                   0, [] { __syncthreads(); }, [](int) {});  // the table is loaded
  if (lane == 0) num_nodes[s] = n;
}

template <int J, int SK>
hipError_t launch_jk(const int32_t* tok, const float* logq, const int32_t* bonus, int S, int L,
                     int K, int B, int32_t* tree_tok, int32_t* parent, int32_t* depth,
                     float* node_logq, int32_t* num_nodes, hipStream_t st) {
  const size_t smem = tree::smem_bytes(B + 1, L * K);
  if (smem > 48 * 1024) {
    const hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&build_tree_kernel<J, SK>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((build_tree_kernel<J, SK>), dim3(S), dim3(kWave), smem, st, tok, logq, bonus,
                     L, K, B, tree_tok, parent, depth, node_logq, num_nodes);
  return hipGetLastError();
}

template <int J>
hipError_t launch_j(const int32_t* tok, const float* logq, const int32_t* bonus, int S, int L,
                    int K, int B, int32_t* tree_tok, int32_t* parent, int32_t* depth,
                    float* node_logq, int32_t* num_nodes, hipStream_t st) {
  if constexpr (J <= 2) {
    if (K <= 8)
      return launch_jk<J, 8>(tok, logq, bonus, S, L, K, B, tree_tok, parent, depth, node_logq,
                             num_nodes, st);
    if (K <= 16)
      return launch_jk<J, 16>(tok, logq, bonus, S, L, K, B, tree_tok, parent, depth, node_logq,
                              num_nodes, st);
  }
  return launch_jk<J, 0>(tok, logq, bonus, S, L, K, B, tree_tok, parent, depth, node_logq,
                         num_nodes, st);
}

}  // namespace

hipError_t launch_build_tree(const int32_t* tok, const float* logq, const int32_t* bonus, int S,
                             int L, int K, int B, int32_t* tree_tok, int32_t* parent,
                             int32_t* depth, float* node_logq, int32_t* num_nodes,
                             hipStream_t st) {
  // one stream per node: B + 1 of them, 64 per register slot
  const int slots = (int)ceil_div(B + 1, kWave);
#define DDT_J(JJ) \
  return launch_j<JJ>(tok, logq, bonus, S, L, K, B, tree_tok, parent, depth, node_logq, num_nodes, st)
  if (slots <= 1) DDT_J(1);
  if (slots <= 2) DDT_J(2);
  if (slots <= 4) DDT_J(4);
  if (slots <= 8) DDT_J(8);
  DDT_J(16);
#undef DDT_J
}

}  // namespace ddt
