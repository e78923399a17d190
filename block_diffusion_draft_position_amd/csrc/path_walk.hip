// Tree walk along the path (DDTree page "策展 · X (Twitter)", section 運作流程 step 4:
// from the root, the target's token at the current node either matches a child, which
// is accepted and becomes the current node, or ends the round as the bonus token).
//
// The walk's outputs depend only on the target's rows at the nodes it visits, at most
// L + 1 of the N rows.  This kernel follows the walk node by node, one workgroup per
// sequence, and reads just those rows: per step the workgroup finds the current node's
// arg-max (larger value, then smaller id; the sampling score fl(fl(x * inv_t) + g)
// with a noise row) and then the smallest-index child carrying that token.
//
// A step reads one row of V logits on one CU, so it is bound by that CU's issue rate
// rather than by HBM.  The scan therefore spends as few VALU operations per logit as
// it can: a thread keeps the maximum of each float4 it loads (two max operations per
// four logits) and one running best float4 (value, index) with a strict comparison, so
// that of equal maxima the earlier float4 stays; at the end of the row it reloads its
// best float4 and takes the first element equal to the maximum.  Each thread visits
// its float4s in increasing order, so its candidate is the smallest id holding its
// maximum, and the workgroup's reduction breaks equal values by the smaller id.  A
// thread that saw only -inf keeps its first float4.  Scores are finite or -inf (the
// interface excludes NaN), so the no-NaN build of this file changes no result.
//
// With a step budget (the hybrid walk), a sequence whose walk is still going after
// max_steps accepted tokens hands over to the subtree scan: the kernel records the
// current node, the tokens accepted so far and the size of the current node's subtree
// (state[s] = {node, accepted, count}), and lists the subtree's nodes in
// list[s, 0 .. count) in no particular order (a node's subtree is itself and every node
// whose parent chain reaches it).  The scan then reads only those rows and continues
// the walk from that node.
#include <limits.h>

#include "ddt_internal.h"

namespace ddt {
namespace {

constexpr int kThreads = 1024;
// float4 loads per thread in flight: 16 of the row, or 8 of the row and 8 of the noise
template <bool SAMPLE>
constexpr int kUnroll = SAMPLE ? 8 : 16;

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <bool SAMPLE>
__device__ __forceinline__ f32x4 scores(f32x4 x, f32x4 g, float inv_t) {
  if constexpr (SAMPLE) {
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = sample_score(x[e], inv_t, g[e]);
  }
  return x;
}

// The arg-max of one row under `better` (scores: the logits, or with SAMPLE the
// sampling scores against the noise row g).  Every thread returns the workgroup's
// winner; -1 if the row holds no candidate (cannot happen for a row of finite or -inf
// values, kept so that the scan and this walk agree on any input).
template <bool SAMPLE>
__device__ int row_argmax(const float* __restrict__ row, const float* __restrict__ g, float inv_t,
                          int V, bool vec_ok, float* rv, int* ri, int* win) {
  const int tid = threadIdx.x, lane = tid % kWave, w = tid / kWave;
  float bv = -INFINITY;
  int bi = INT_MAX;
  if (vec_ok) {
    const int nv4 = V / 4;
    const f32x4* r4 = reinterpret_cast<const f32x4*>(row);
    const f32x4* g4 = reinterpret_cast<const f32x4*>(g);
    float gv = -INFINITY;  // the maximum of the best float4 so far
    int gi = -1;           // its index
    constexpr int U = kUnroll<SAMPLE>;
    for (int b0 = tid; b0 < nv4; b0 += kThreads * U) {
      f32x4 x[U], n[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = b0 + u * kThreads;
        x[u] = i < nv4 ? r4[i] : f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
        if constexpr (SAMPLE) n[u] = i < nv4 ? g4[i] : f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const f32x4 y = scores<SAMPLE>(x[u], n[u], inv_t);
        const float m = fmaxf(fmaxf(y[0], y[1]), fmaxf(y[2], y[3]));
        if (m > gv) {  // padding (-inf) never passes; the earlier float4 keeps a tie
          gv = m;
          gi = b0 + u * kThreads;
        }
      }
    }
    if (gi < 0 && tid < nv4) gi = tid;  // every score -inf: the first float4 holds the minimum id
    if (gi >= 0) {
      const f32x4 y = scores<SAMPLE>(r4[gi], SAMPLE ? g4[gi] : f32x4{}, inv_t);
      int e = 3;
#pragma unroll
      for (int q = 2; q >= 0; --q)
        if (y[q] == gv) e = q;
      bv = gv;
      bi = 4 * gi + e;
    }
  } else {
    for (int v = tid; v < V; v += kThreads) {
      const float y = SAMPLE ? sample_score(row[v], inv_t, g[v]) : row[v];
      if (better(y, v, bv, bi)) {
        bv = y;
        bi = v;
      }
    }
  }
  wave_argmax(bv, bi);
  if (lane == 0) {
    rv[w] = bv;
    ri[w] = bi;
  }
  __syncthreads();
  if (w == 0) {
    float v2 = lane < kThreads / kWave ? rv[lane] : -INFINITY;
    int i2 = lane < kThreads / kWave ? ri[lane] : INT_MAX;
    wave_argmax(v2, i2);
    if (lane == 0) *win = i2 == INT_MAX ? -1 : i2;
  }
  __syncthreads();
  return *win;
}

template <bool SAMPLE>
__global__ void __launch_bounds__(kThreads)
path_walk_kernel(const int32_t* __restrict__ tree_tok, const int32_t* __restrict__ parent,
                 const int32_t* __restrict__ num_nodes, const float* __restrict__ target,
                 const int32_t* __restrict__ depth, const float* __restrict__ gumbel, float inv_t,
                 int N, int L, int V, bool vec_ok, int max_steps, unsigned* __restrict__ state,
                 int32_t* __restrict__ list, int32_t* __restrict__ accept_len,
                 int32_t* __restrict__ acc_nodes, int32_t* __restrict__ acc_tok,
                 int32_t* __restrict__ bonus_out) {
  extern __shared__ int psm[];  // tok[N], parent[N], depth[N]
  __shared__ float rv[kThreads / kWave];
  __shared__ int ri[kThreads / kWave];
  __shared__ int want_s, child_s, count_s;
  const int s = blockIdx.x;
  const int tid = threadIdx.x;
  const int nn = min(max(num_nodes[s], 1), N);
  int* tk = psm;
  int* pr = psm + N;
  int* dp = psm + 2 * N;
  for (int i = tid; i < N; i += kThreads) {
    tk[i] = tree_tok[(int64_t)s * N + i];
    pr[i] = parent[(int64_t)s * N + i];
    if (SAMPLE) dp[i] = depth[(int64_t)s * N + i];
  }
  if (tid == 0) {
    child_s = INT_MAX;
    count_s = 0;
  }
  __syncthreads();
  int cur = 0, a = 0;
  for (;;) {
    if (a == max_steps) {
      // hand over to the scan: list cur's subtree.  Parents precede their children, so
      // a member's chain falls from it to cur in at most L links; a chain that leaves
      // that order or runs longer belongs to no valid tree and lists nothing
      for (int n = cur + tid; n < nn; n += kThreads) {
        int x = n;
        for (int k = 0; k <= L && x > cur; ++k) {
          const int p = pr[x];
          x = (p >= 0 && p < x) ? p : -1;
        }
        if (x == cur) list[(int64_t)s * N + atomicAdd(&count_s, 1)] = n;
      }
      __syncthreads();
      if (tid == 0) {
        state[4 * s] = (unsigned)cur;
        state[4 * s + 1] = (unsigned)a;
        state[4 * s + 2] = (unsigned)count_s;
      }
      return;  // the scan writes this sequence's remaining outputs
    }
    const float* row = target + ((int64_t)s * N + cur) * V;
    const float* g = SAMPLE ? gumbel + ((int64_t)s * (L + 1) + dp[cur]) * V : nullptr;
    const int want = row_argmax<SAMPLE>(row, g, inv_t, V, vec_ok, rv, ri, &want_s);
    // the smallest-index child of cur carrying want (a child follows its parent)
    for (int c = tid + 1; c < nn; c += kThreads)
      if (pr[c] == cur && tk[c] == want) atomicMin(&child_s, c);
    __syncthreads();
    const int c = child_s;
    if (c == INT_MAX || a >= L) {
      if (tid == 0) {
        accept_len[s] = a;
        bonus_out[s] = want;
      }
      break;
    }
    if (tid == 0) {
      acc_nodes[(int64_t)s * L + a] = c;
      acc_tok[(int64_t)s * L + a] = want;
    }
    ++a;
    cur = c;
    __syncthreads();  // every thread has read child_s
    if (tid == 0) child_s = INT_MAX;  // read again only after the next step's barriers
  }
  for (int j = a + tid; j < L; j += kThreads) {
    acc_nodes[(int64_t)s * L + j] = -1;
    acc_tok[(int64_t)s * L + j] = -1;
  }
}

}  // namespace

hipError_t launch_path_walk(const int32_t* tree_tok, const int32_t* parent,
                            const int32_t* num_nodes, const float* target, int S, int B, int L,
                            int64_t vocab, int32_t* accept_len, int32_t* acc_nodes,
                            int32_t* acc_tok, int32_t* bonus_out, hipStream_t st,
                            const int32_t* depth, const float* gumbel, float inv_t,
                            int max_steps, unsigned* state, int32_t* list) {
  const int N = B + 1;
  const bool vec_ok = (reinterpret_cast<uintptr_t>(target) % 16 == 0) && (vocab % 4 == 0) &&
                      (reinterpret_cast<uintptr_t>(gumbel) % 16 == 0);
  const size_t smem = 3 * sizeof(int) * N;
  if (gumbel)
    hipLaunchKernelGGL((path_walk_kernel<true>), dim3(S), dim3(kThreads), smem, st, tree_tok, parent,
                       num_nodes, target, depth, gumbel, inv_t, N, L, (int)vocab, vec_ok, max_steps,
                       state, list, accept_len, acc_nodes, acc_tok, bonus_out);
  else
    hipLaunchKernelGGL((path_walk_kernel<false>), dim3(S), dim3(kThreads), smem, st, tree_tok, parent,
                       num_nodes, target, depth, gumbel, inv_t, N, L, (int)vocab, vec_ok, max_steps,
                       state, list, accept_len, acc_nodes, acc_tok, bonus_out);
  return hipGetLastError();
}

}  // namespace ddt
