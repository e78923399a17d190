// Draft-tree construction under a node budget: best-first selection of the B most
// probable draft prefixes (DDTree page "策展 · X (Twitter)": section 核心創新 for the
// best-first heap and budget, 運作流程 step 2 for the construction, 理論基礎 for
// the factorised prefix probability and the prefix-closure of the optimum).
//
// One wavefront per sequence.  The candidate prefixes form a K-ary tree whose
// depth-i children are position i's top-K tokens, sorted by probability, so a
// node's children are visited in rank order: each tree node u keeps one frontier
// entry, "u's next unselected child", whose key is score(u) + logq[depth(u)][cursor(u)].
// Popping the best entry selects that child c; then u's entry moves to its next
// child and c gets an entry for its first child.  Every pop therefore touches two
// entries, and the frontier never holds more than one entry per selected node.
//
// Entries live in registers: node u at lane u % 64, slot u / 64.  Each lane caches
// its best slot; a pop is one DPP max-reduction plus two exec-masked updates.  The
// top-K log-probabilities sit in registers too (depth row = register, rank = lane),
// so a pop reads them with v_readlane instead of an LDS round trip.
// Scores are summed in fp64; the comparison key is the fp32 rounding of that sum
// (rounding is monotone, so a child's key never exceeds its parent's and the popped
// set stays prefix-closed).
//
// After B pops the selected nodes are renumbered canonically: by depth, then parent's
// canonical index, then sibling rank (children of a node are selected in rank order,
// so its selected children are exactly ranks 0..cursor-1).
#include <limits.h>

#include "ddt_internal.h"

namespace ddt {
namespace {

struct TreeSmem {
  float* lq;      // [L*K]
  int* ltok;      // [L*K]
  int* parent;    // [N] node (pop order) -> parent node
  int* rank;      // [N]
  int* depth;     // [N]
  int* nkids;     // [N] selected children
  double* score;  // [N]
  int* canon;     // [N] node -> canonical index
  int* order;     // [N] canonical index -> node
  int* first;     // [N] node -> canonical index of its first child
};

__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = lane_id();
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  return v;
}

template <int J, int LM>
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

  TreeSmem sm;
  {
    unsigned char* p = smem_raw;
    sm.score = reinterpret_cast<double*>(p);
    p += sizeof(double) * N;
    sm.lq = reinterpret_cast<float*>(p);
    p += sizeof(float) * LK;
    sm.ltok = reinterpret_cast<int*>(p);
    p += sizeof(int) * LK;
    int* ip = reinterpret_cast<int*>(p);
    sm.parent = ip;
    sm.rank = ip + N;
    sm.depth = ip + 2 * N;
    sm.nkids = ip + 3 * N;
    sm.canon = ip + 4 * N;
    sm.order = ip + 5 * N;
    sm.first = ip + 6 * N;
  }
  const float* lq_g = topk_logq + (int64_t)s * LK;
  const int32_t* tok_g = topk_tok + (int64_t)s * LK;
  // logq table in registers: ltab[d] holds depth-row d, rank = lane (K <= 64)
  float ltab[LM];
#pragma unroll
  for (int d = 0; d < LM; ++d) ltab[d] = (d < L && lane < K) ? lq_g[d * K + lane] : -INFINITY;
  for (int i = lane; i < LK; i += kWave) sm.ltok[i] = tok_g[i];
  for (int i = lane; i < N; i += kWave) sm.nkids[i] = 0;

  // frontier entries, node u at (lane u % 64, slot u / 64)
  float key[J];
  double ex[J];     // exact key: score(u) + logq[depth(u)][cursor(u)]
  double sc[J];     // score(u)
  int meta[J];      // depth(u) | cursor(u) << 8; cursor = rank of u's next child
#pragma unroll
  for (int j = 0; j < J; ++j) {
    key[j] = -INFINITY;
    ex[j] = 0.0;
    sc[j] = 0.0;
    meta[j] = 0;
  }
  {
    const float r0 = readlane(ltab[0], 0);
    if (lane == 0) {  // the root's first child
      ex[0] = (double)r0;
      key[0] = r0;
    }
  }
  float bkey = key[0];
  int bslot = 0;

  int n = 1;  // nodes so far (root included)
  for (int t = 0; t < B; ++t) {
    const float M = wave_max(bkey);
    if (M == -INFINITY) break;  // candidate tree exhausted
    const int w = __ffsll((long long)ballot(bkey == M)) - 1;
    const int j = J == 1 ? 0 : __builtin_amdgcn_readfirstlane(readlane(bslot, w));
    const double ex_u = readlane_f64(ex[j], w);
    const double sc_u = readlane_f64(sc[j], w);
    const int meta_u = __builtin_amdgcn_readfirstlane(readlane(meta[j], w));
    const int dep_u = meta_u & 0xff;
    const int nc = (meta_u >> 8) + 1;  // u's next child rank
    const int c = n++;                 // the selected child
    const int dep_c = dep_u + 1;
    const float l_sib = nc < K ? readlane(ltab[dep_u], nc) : -INFINITY;
    const float l_kid = dep_c < L ? readlane(ltab[dep_c < LM ? dep_c : 0], 0) : -INFINITY;
    if (lane == 0) {
      sm.parent[c] = j * kWave + w;
      sm.rank[c] = nc - 1;
      sm.depth[c] = dep_c;
      sm.score[c] = ex_u;
    }
    // u moves on to its next child
    if (lane == w) {
      const double e = sc_u + (double)l_sib;
      meta[j] = dep_u | (nc << 8);
      ex[j] = e;
      key[j] = l_sib == -INFINITY ? -INFINITY : (float)e;
      bkey = key[0];
      bslot = 0;
#pragma unroll
      for (int i = 1; i < J; ++i)
        if (key[i] > bkey) {
          bkey = key[i];
          bslot = i;
        }
    }
    // c starts at its first child
    const int jc = c / kWave;
    if (lane == c % kWave && jc < J) {
      const double e = ex_u + (double)l_kid;
      const float kk = l_kid == -INFINITY ? -INFINITY : (float)e;
      ex[jc] = e;
      sc[jc] = ex_u;
      meta[jc] = dep_c;
      key[jc] = kk;
      if (kk > bkey) {
        bkey = kk;
        bslot = jc;
      }
    }
  }
  // children counts of every node
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int u = j * kWave + lane;
    if (u < n) sm.nkids[u] = meta[j] >> 8;
  }
  if (lane == 0) {
    sm.parent[0] = -1;
    sm.rank[0] = -1;
    sm.depth[0] = 0;
    sm.score[0] = 0.0;
    sm.canon[0] = 0;
    sm.order[0] = 0;
  }
  __syncthreads();

  // canonical renumbering, one depth at a time
  int lvl_lo = 0, lvl_hi = 1;  // canonical range of the previous depth
  for (int d = 1; lvl_hi < n && d <= L; ++d) {
    // exclusive scan of children counts over the previous depth, in canonical order
    int base = lvl_hi;
    for (int p0 = lvl_lo; p0 < lvl_hi; p0 += kWave) {
      const int p = p0 + lane;
      const int v = p < lvl_hi ? sm.order[p] : 0;
      const int cnt = p < lvl_hi ? sm.nkids[v] : 0;
      const int incl = wave_incl_scan(cnt);
      if (p < lvl_hi) sm.first[v] = base + incl - cnt;
      base += readlane(incl, kWave - 1);
    }
    __syncthreads();
    for (int x0 = 1; x0 < n; x0 += kWave) {
      const int x = x0 + lane;
      if (x < n && sm.depth[x] == d) {
        const int ci = sm.first[sm.parent[x]] + sm.rank[x];
        sm.canon[x] = ci;
        sm.order[ci] = x;
      }
    }
    __syncthreads();
    lvl_lo = lvl_hi;
    lvl_hi = base;
  }

  // write out in canonical order
  const int64_t o = (int64_t)s * N;
  for (int ci = lane; ci < N; ci += kWave) {
    if (ci < n) {
      const int x = sm.order[ci];
      const int d = sm.depth[x];
      tree_tok[o + ci] = d == 0 ? bonus[s] : sm.ltok[(d - 1) * K + sm.rank[x]];
      tree_parent[o + ci] = d == 0 ? -1 : sm.canon[sm.parent[x]];
      tree_depth[o + ci] = d;
      if (node_logq) node_logq[o + ci] = (float)sm.score[x];
    } else {
      tree_tok[o + ci] = -1;
      tree_parent[o + ci] = -1;
      tree_depth[o + ci] = -1;
      if (node_logq) node_logq[o + ci] = -INFINITY;
    }
  }
  if (lane == 0) num_nodes[s] = n;
}

template <int J, int LM>
hipError_t launch_j(const int32_t* tok, const float* logq, const int32_t* bonus, int S, int L,
                    int K, int B, int32_t* tree_tok, int32_t* parent, int32_t* depth,
                    float* node_logq, int32_t* num_nodes, hipStream_t st) {
  const int N = B + 1;
  const size_t smem = sizeof(double) * N + (sizeof(float) + sizeof(int)) * (size_t)L * K +
                      sizeof(int) * 7 * (size_t)N;
  if (smem > 48 * 1024) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&build_tree_kernel<J, LM>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((build_tree_kernel<J, LM>), dim3(S), dim3(kWave), smem, st, tok, logq, bonus,
                     L, K, B, tree_tok, parent, depth, node_logq, num_nodes);
  return hipGetLastError();
}

template <int J>
hipError_t launch_l(const int32_t* tok, const float* logq, const int32_t* bonus, int S, int L,
                    int K, int B, int32_t* tree_tok, int32_t* parent, int32_t* depth,
                    float* node_logq, int32_t* num_nodes, hipStream_t st) {
  if (L <= 16)
    return launch_j<J, 16>(tok, logq, bonus, S, L, K, B, tree_tok, parent, depth, node_logq, num_nodes, st);
  return launch_j<J, 64>(tok, logq, bonus, S, L, K, B, tree_tok, parent, depth, node_logq, num_nodes, st);
}

}  // namespace

hipError_t launch_build_tree(const int32_t* tok, const float* logq, const int32_t* bonus, int S,
                             int L, int K, int B, int32_t* tree_tok, int32_t* parent,
                             int32_t* depth, float* node_logq, int32_t* num_nodes,
                             hipStream_t st) {
  // frontier entries: one per node that can still get children, at most B of them
  // are ever created (the last selected node's entry is never popped).
  const int slots = (int)ceil_div(B + 1, kWave);
#define DDT_J(JJ) \
  return launch_l<JJ>(tok, logq, bonus, S, L, K, B, tree_tok, parent, depth, node_logq, num_nodes, st)
  if (slots <= 1) DDT_J(1);
  if (slots <= 2) DDT_J(2);
  if (slots <= 4) DDT_J(4);
  if (slots <= 8) DDT_J(8);
  DDT_J(16);
#undef DDT_J
}

}  // namespace ddt
