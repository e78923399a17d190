// Adaptive node budget (DDTree page "策展 · X (Twitter)": section 實驗結果與權衡, the
// speedup peaks at an intermediate budget as verification cost grows; section 理論基礎,
// Proposition 1: the expected acceptance of a tree is the sum of its prefix
// probabilities, Proposition 2: the top-b prefixes form a tree).
//
// For a tree built at budget B, the tree at any budget b <= B is its b most probable
// prefixes, and its expected acceptance E(b) is the sum of their probabilities.  With
// the caller's verify cost per budget, each sequence takes B* = argmax_b (E(b) + 1) /
// cost[b] and its tree is cut to those B* prefixes, in place.
//
// One workgroup per sequence (at most 1024 nodes):
//   * every non-root node's rank in pop order (log-probability descending, equal values
//     by smaller index: shallower first, then canonical order within a depth) by
//     counting the nodes ahead of it over the scores staged in LDS;
//   * wave 0 forms E(b) = sum of exp of the first b scores in fp64 (a contiguous run of
//     ranks per lane, then the lanes' running offsets) and the ratio for every b, and
//     keeps the largest (equal ratios to the smaller b);
//   * the survivors (root and ranks < B*) keep their canonical order: a node's new index
//     is the number of survivors before it, found by ballots over the index order; each
//     survivor is written to its new slot with its parent's new index, and the tail is
//     padding.  Everything is read into LDS before the first write.
#include "ddt_internal.h"

namespace ddt {
namespace {

constexpr int kThreads = 256;

__global__ void __launch_bounds__(kThreads)
adapt_budget_kernel(const float* __restrict__ cost, int N, int32_t* __restrict__ tree_tok,
                    int32_t* __restrict__ parent, int32_t* __restrict__ depth,
                    float* __restrict__ node_logq, int32_t* __restrict__ num_nodes,
                    int32_t* __restrict__ budget_out, float* __restrict__ expected_out) {
  extern __shared__ __align__(16) unsigned char smem[];
  float* lq = reinterpret_cast<float*>(smem);     // [N] node log-probabilities
  int* tok = reinterpret_cast<int*>(lq + N);      // [N]
  int* par = tok + N;                             // [N]
  int* dep = par + N;                             // [N]
  int* ord = dep + N;                             // [N] rank -> node
  int* rk = ord + N;                              // [N] node -> rank (root: -1)
  int* nidx = rk + N;                             // [N] node -> new index (-1: cut)
  __shared__ int bstar_s;
  __shared__ double estar_s;
  const int s = blockIdx.x;
  const int64_t o = (int64_t)s * N;
  const int nn = num_nodes[s];
  for (int i = threadIdx.x; i < N; i += kThreads) {
    lq[i] = node_logq[o + i];
    tok[i] = tree_tok[o + i];
    par[i] = parent[o + i];
    dep[i] = depth[o + i];
  }
  __syncthreads();
  // ranks of the non-root nodes 1 .. nn-1
  for (int i = 1 + threadIdx.x; i < nn; i += kThreads) {
    const float v = lq[i];
    int r = 0;
    for (int j = 1; j < nn; ++j) {
      const float w = lq[j];
      r += (w > v) || (w == v && j < i);
    }
    rk[i] = r;
    ord[r] = i;
  }
  if (threadIdx.x == 0) rk[0] = -1;
  __syncthreads();
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    const int m = nn - 1;                         // candidates b = 0 .. m
    const int per = (m + kWave - 1) / kWave;      // ranks per lane, a contiguous run
    const int r0 = lane * per;
    double part = 0.0;
    for (int r = r0; r < min(m, r0 + per); ++r) part += exp((double)lq[ord[r]]);
    // exclusive running offset of this lane's run
    double incl = part;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      const double up = __shfl_up(incl, d);
      if (lane >= d) incl += up;
    }
    double e = incl - part;
    // ratio for b = r + 1 after adding rank r; b = 0 belongs to lane 0
    double bj = -1.0, be = 0.0;
    int bb = INT32_MAX;
    if (lane == 0) {
      bj = 1.0 / (double)cost[0];
      bb = 0;
    }
    for (int r = r0; r < min(m, r0 + per); ++r) {
      e += exp((double)lq[ord[r]]);
      const double j = (e + 1.0) / (double)cost[r + 1];
      if (j > bj) {
        bj = j;
        bb = r + 1;
        be = e;
      }
    }
    // largest ratio over the wave, equal ratios to the smaller budget
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      const double oj = __shfl_xor(bj, d);
      const int ob = __shfl_xor(bb, d);
      const double oe = __shfl_xor(be, d);
      if (oj > bj || (oj == bj && ob < bb)) {
        bj = oj;
        bb = ob;
        be = oe;
      }
    }
    if (lane == 0) {
      bstar_s = bb;
      estar_s = be;
    }
    // new indices of the survivors, in index order
    int run = 0;
    for (int base = 0; base < nn; base += kWave) {
      const int i = base + lane;
      const bool keep = i < nn && (i == 0 || rk[i] < bb);
      const unsigned long long msk = ballot(keep);
      if (i < nn) nidx[i] = keep ? run + __popcll(msk & ((1ull << lane) - 1ull)) : -1;
      run += __popcll(msk);
    }
  }
  __syncthreads();
  const int bstar = bstar_s;
  for (int i = threadIdx.x; i < nn; i += kThreads) {
    const int ni = nidx[i];
    if (ni >= 0) {
      tree_tok[o + ni] = tok[i];
      parent[o + ni] = par[i] < 0 ? -1 : nidx[par[i]];
      depth[o + ni] = dep[i];
      node_logq[o + ni] = lq[i];
    }
  }
  for (int i = bstar + 1 + threadIdx.x; i < N; i += kThreads) {
    tree_tok[o + i] = -1;
    parent[o + i] = -1;
    depth[o + i] = -1;
    node_logq[o + i] = -INFINITY;
  }
  if (threadIdx.x == 0) {
    num_nodes[s] = bstar + 1;
    budget_out[s] = bstar;
    if (expected_out) expected_out[s] = (float)estar_s;
  }
}

}  // namespace

hipError_t launch_adapt_budget(const float* cost, int S, int B, int32_t* tree_tok, int32_t* parent,
                               int32_t* depth, float* node_logq, int32_t* num_nodes,
                               int32_t* budget_out, float* expected_out, hipStream_t st) {
  const int N = B + 1;
  const size_t smem = (size_t)N * (sizeof(float) + 6 * sizeof(int));
  hipLaunchKernelGGL(adapt_budget_kernel, dim3(S), dim3(kThreads), smem, st, cost, N, tree_tok,
                     parent, depth, node_logq, num_nodes, budget_out, expected_out);
  return hipGetLastError();
}

}  // namespace ddt
