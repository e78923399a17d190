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
#include <limits.h>

#include "ddt_internal.h"

namespace ddt {
namespace {

struct TreeSmem {
  double* score;  // [N] node -> prefix log-probability
  float* lq;      // [L*K]
  int* ltok;      // [L*K]
  int* hist;      // [256] radix-select histogram
  int* parent;    // [N] node (selection order) -> parent node
  int* rank;      // [N]
  int* depth;     // [N]
  int* nkids;     // [N] selected children
  int* canon;     // [N] node -> canonical index
  int* order;     // [N] canonical index -> node
  int* first;     // [N] node -> canonical index of its first child
};

__host__ __device__ constexpr size_t tree_smem_bytes(int N, int LK) {
  return sizeof(double) * (size_t)N + (sizeof(float) + sizeof(int)) * (size_t)LK +
         sizeof(int) * 256 + sizeof(int) * 7 * (size_t)N;
}

__device__ __forceinline__ int wave_sum_i(int v) {
  v += xchg<1>(v);
  v += xchg<2>(v);
  v += xchg<4>(v);
  v += xchg<8>(v);
  v += xchg<16>(v);
  v += xchg<32>(v);
  return v;
}

__device__ __forceinline__ int wave_min_i(int v) {
  v = min(v, xchg<1>(v));
  v = min(v, xchg<2>(v));
  v = min(v, xchg<4>(v));
  v = min(v, xchg<8>(v));
  v = min(v, xchg<16>(v));
  v = min(v, xchg<32>(v));
  return v;
}

__device__ __forceinline__ double wave_max_d(double v) {
  v = fmax(v, xchg<1>(v));
  v = fmax(v, xchg<2>(v));
  v = fmax(v, xchg<4>(v));
  v = fmax(v, xchg<8>(v));
  v = fmax(v, xchg<16>(v));
  v = fmax(v, xchg<32>(v));
  return v;
}

// inclusive prefix sum over lanes
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = lane_id();
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  return v;
}

// order-preserving map of an fp64 score to uint64 (larger score -> larger key)
__device__ __forceinline__ unsigned long long key_of(double x) {
  const unsigned long long b = __builtin_bit_cast(unsigned long long, x);
  return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}

template <int J>
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
    sm.hist = reinterpret_cast<int*>(p);
    p += sizeof(int) * 256;
    int* ip = reinterpret_cast<int*>(p);
    sm.parent = ip;
    sm.rank = ip + N;
    sm.depth = ip + 2 * N;
    sm.nkids = ip + 3 * N;
    sm.canon = ip + 4 * N;
    sm.order = ip + 5 * N;
    sm.first = ip + 6 * N;
  }
  {
    const float* lq_g = topk_logq + (int64_t)s * LK;
    const int32_t* tok_g = topk_tok + (int64_t)s * LK;
    for (int i = lane; i < LK; i += kWave) {
      sm.lq[i] = lq_g[i];
      sm.ltok[i] = tok_g[i];
    }
  }
  __syncthreads();
  auto lq = [&](int d, int r) -> double { return (double)sm.lq[d * K + r]; };
  // bound on the children of a depth-(d) candidate: logq[d][0], none past depth L
  auto best_child = [&](int d) -> double { return d < L ? lq(d, 0) : -INFINITY; };

  // stream of node u at (lane u % 64, slot u / 64)
  double sc[J];    // score(u)
  double head[J];  // score of u's next child, -inf once the stream is closed
  double nxt[J];   // best_child(depth(u) + 1)
  int dep[J];      // depth(u)
  int cur[J];      // rank of u's next child; K when closed
#pragma unroll
  for (int j = 0; j < J; ++j) {
    sc[j] = 0.0;
    head[j] = -INFINITY;
    nxt[j] = -INFINITY;
    dep[j] = 0;
    cur[j] = K;
  }
  if (lane == 0) {  // the root
    cur[0] = 0;
    head[0] = lq(0, 0);
    nxt[0] = best_child(1);
  }

  // candidates of stream j scoring above th: a prefix of the stream, found by bisection
  auto above = [&](int j, double th) -> int {
    if (cur[j] >= K) return 0;
    int lo = cur[j], hi = K;  // first rank at or below th lies in [lo, hi]
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (sc[j] + lq(dep[j], mid) > th)
        lo = mid + 1;
      else
        hi = mid;
    }
    return lo - cur[j];
  };

  int n = 1;  // nodes selected so far, root included
  while (n - 1 < B) {
    const int R = B - (n - 1);
    bool live = false;
    double tl = -INFINITY;
#pragma unroll
    for (int j = 0; j < J; ++j)
      if (cur[j] < K) {
        live = true;
        tl = fmax(tl, head[j] + nxt[j]);
      }
    if (!ballot(live)) break;  // the candidate tree is exhausted
    const double tau = wave_max_d(tl);
    int cnt[J];
    int mine = 0;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      cnt[j] = above(j, tau);
      mine += cnt[j];
    }
    int total = wave_sum_i(mine);

    if (total == 0) {
      // nothing clears tau: take the single best head, the lowest node on ties
      double hb = -INFINITY;
#pragma unroll
      for (int j = 0; j < J; ++j)
        if (cur[j] < K) hb = fmax(hb, head[j]);
      const double hm = wave_max_d(hb);
      int pick = INT_MAX;
#pragma unroll
      for (int j = J - 1; j >= 0; --j)
        if (cur[j] < K && head[j] == hm) pick = j * kWave + lane;
      pick = wave_min_i(pick);
#pragma unroll
      for (int j = 0; j < J; ++j) cnt[j] = (j * kWave + lane == pick) ? 1 : 0;
      total = 1;
    } else if (total > R) {
      // keep the R best.  Radix select over the 64-bit keys finds T, the R-th
      // largest key, and how many keys equal to T belong in (k).
      unsigned long long prefix = 0ull, pmask = 0ull;
      int k = R;
      for (int shift = 56; shift >= 0; shift -= 8) {
        for (int b = lane; b < 256; b += kWave) sm.hist[b] = 0;
        __syncthreads();
#pragma unroll
        for (int j = 0; j < J; ++j)
          for (int i = 0; i < cnt[j]; ++i) {
            const unsigned long long key = key_of(sc[j] + lq(dep[j], cur[j] + i));
            if ((key & pmask) == prefix) atomicAdd(&sm.hist[(key >> shift) & 255u], 1);
          }
        __syncthreads();
        // lane l holds bins 255-4l .. 252-4l: the scan runs from the top bin down
        int h[4], loc = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          h[q] = sm.hist[255 - 4 * lane - q];
          loc += h[q];
        }
        const int incl = wave_incl_scan(loc);
        const int excl = incl - loc;
        const int src = max(__ffsll((long long)ballot(excl < k && incl >= k)) - 1, 0);
        int bin = 0, higher = 0;
        if (lane == src) {
          int acc = excl;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            if (acc + h[q] >= k) {
              bin = 255 - 4 * lane - q;
              higher = acc;
              break;
            }
            acc += h[q];
          }
        }
        bin = readlane(bin, src);
        higher = readlane(higher, src);
        k -= higher;
        prefix |= (unsigned long long)bin << shift;
        pmask |= 255ull << shift;
        __syncthreads();
      }
      // per stream: the keys above T, then the first k keys equal to T in node order
      int gt[J], eq[J];
#pragma unroll
      for (int j = 0; j < J; ++j) {
        gt[j] = 0;
        eq[j] = 0;
        for (int i = 0; i < cnt[j]; ++i) {
          const unsigned long long key = key_of(sc[j] + lq(dep[j], cur[j] + i));
          gt[j] += key > prefix;
          eq[j] += key == prefix;
        }
      }
      int before = 0;
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int incl = wave_incl_scan(eq[j]);
        const int take = min(max(k - (before + incl - eq[j]), 0), eq[j]);
        cnt[j] = gt[j] + take;
        before += readlane(incl, kWave - 1);
      }
      total = R;
    }

    // the round's nodes get ids n .. n + total - 1 in (slot, lane) order
    int base = n;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int incl = wave_incl_scan(cnt[j]);
      const int firstid = base + incl - cnt[j];
      const int u = j * kWave + lane;
      for (int i = 0; i < cnt[j]; ++i) {
        const int x = firstid + i;
        sm.parent[x] = u;
        sm.rank[x] = cur[j] + i;
        sm.depth[x] = dep[j] + 1;
        sm.score[x] = sc[j] + lq(dep[j], cur[j] + i);
      }
      if (cnt[j] > 0) {
        cur[j] += cnt[j];
        head[j] = cur[j] < K ? sc[j] + lq(dep[j], cur[j]) : -INFINITY;
      }
      base += readlane(incl, kWave - 1);
    }
    __syncthreads();
    // each new node opens its stream
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int x = j * kWave + lane;
      if (x >= n && x < n + total) {
        dep[j] = sm.depth[x];
        sc[j] = sm.score[x];
        const bool open = dep[j] < L;
        cur[j] = open ? 0 : K;
        head[j] = open ? sc[j] + lq(dep[j], 0) : -INFINITY;
        nxt[j] = best_child(dep[j] + 1);
      }
    }
    n += total;
  }
  // selected children of every node: ranks 0 .. cursor-1 of an open stream
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int u = j * kWave + lane;
    if (u < n) sm.nkids[u] = dep[j] < L ? cur[j] : 0;
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
      const int c = p < lvl_hi ? sm.nkids[v] : 0;
      const int incl = wave_incl_scan(c);
      if (p < lvl_hi) sm.first[v] = base + incl - c;
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

template <int J>
hipError_t launch_j(const int32_t* tok, const float* logq, const int32_t* bonus, int S, int L,
                    int K, int B, int32_t* tree_tok, int32_t* parent, int32_t* depth,
                    float* node_logq, int32_t* num_nodes, hipStream_t st) {
  const size_t smem = tree_smem_bytes(B + 1, L * K);
  if (smem > 48 * 1024) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&build_tree_kernel<J>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((build_tree_kernel<J>), dim3(S), dim3(kWave), smem, st, tok, logq, bonus, L,
                     K, B, tree_tok, parent, depth, node_logq, num_nodes);
  return hipGetLastError();
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
