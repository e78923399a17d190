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

#include <type_traits>

#include "ddt_internal.h"

namespace ddt {
namespace {

constexpr int kRankCap = 256;  // final rounds with at most this many candidates rank them exactly

struct TreeSmem {
  unsigned long long* key;  // [kRankCap] final-round candidate keys
  int* sel;                 // [kRankCap] candidate taken?
  double* score;  // [N] node -> prefix log-probability
  double* head;   // [N] node -> score of its first child (-inf: no children possible)
  double* nxt;    // [N] node -> bound on its grandchildren's step, logq[depth + 1][0]
  float* lq;      // [L*K]
  int* ltok;      // [L*K]
  int* hist;      // [256] radix-select histogram
  int* parent;    // [N] node (selection order) -> parent node
  int* rank;      // [N] node -> sibling rank
  int* depth;     // [N] node -> depth
  int* canon;     // [N] node -> canonical index
  int* order;     // [N] canonical index -> node
  int* nkc;       // [N] canonical index -> number of selected children
  int* first;     // [N] node -> canonical index of its first child
};

__host__ __device__ constexpr size_t tree_smem_bytes(int N, int LK) {
  return (sizeof(unsigned long long) + sizeof(int)) * kRankCap + 3 * sizeof(double) * (size_t)N +
         (sizeof(float) + sizeof(int)) * (size_t)LK + sizeof(int) * 256 + sizeof(int) * 7 * (size_t)N;
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

template <bool MAX>
__device__ __forceinline__ unsigned long long wave_ext_u64(unsigned long long v) {
  auto step = [&](unsigned long long o) { v = MAX ? (o > v ? o : v) : (o < v ? o : v); };
  auto x = [&](auto tag) {
    constexpr int S = decltype(tag)::value;
    const int lo = xchg<S>((int)(unsigned)(v & 0xffffffffull));
    const int hi = xchg<S>((int)(unsigned)(v >> 32));
    return ((unsigned long long)(unsigned)hi << 32) | (unsigned)lo;
  };
  step(x(std::integral_constant<int, 1>{}));
  step(x(std::integral_constant<int, 2>{}));
  step(x(std::integral_constant<int, 4>{}));
  step(x(std::integral_constant<int, 8>{}));
  step(x(std::integral_constant<int, 16>{}));
  step(x(std::integral_constant<int, 32>{}));
  return v;
}
__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) { return wave_ext_u64<true>(v); }
__device__ __forceinline__ unsigned long long wave_min_u64(unsigned long long v) { return wave_ext_u64<false>(v); }

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
    sm.key = reinterpret_cast<unsigned long long*>(p);
    p += sizeof(unsigned long long) * kRankCap;
    sm.score = reinterpret_cast<double*>(p);
    p += sizeof(double) * N;
    sm.head = reinterpret_cast<double*>(p);
    p += sizeof(double) * N;
    sm.nxt = reinterpret_cast<double*>(p);
    p += sizeof(double) * N;
    sm.sel = reinterpret_cast<int*>(p);
    p += sizeof(int) * kRankCap;
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
    sm.canon = ip + 3 * N;
    sm.order = ip + 4 * N;
    sm.nkc = ip + 5 * N;
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
  // bound on the children of a depth-d candidate: logq[d][0], none past depth L
  auto best_child = [&](int d) -> double { return d < L ? lq(d, 0) : -INFINITY; };

  // node u lives at (lane u % 64, slot u / 64): its stream and its place in the tree
  double sc[J];    // score(u)
  double head[J];  // score of u's next child, -inf once the stream is closed
  double nxt[J];   // best_child(depth(u) + 1)
  int dep[J];      // depth(u)
  int cur[J];      // rank of u's next child; K when closed
  int par[J];      // parent(u)
  int rnk[J];      // sibling rank of u
#pragma unroll
  for (int j = 0; j < J; ++j) {
    sc[j] = 0.0;
    head[j] = -INFINITY;
    nxt[j] = -INFINITY;
    dep[j] = 0;
    cur[j] = K;
    par[j] = -1;
    rnk[j] = -1;
  }
  if (lane == 0) {  // the root
    cur[0] = 0;
    head[0] = lq(0, 0);
    nxt[0] = best_child(1);
  }

  // candidates of stream j scoring above th: a prefix of the stream.  Small K reads
  // the whole row at once; larger K bisects.
  auto above = [&](int j, double th) -> int {
    if (cur[j] >= K) return 0;
    if (K <= 16) {
      int c = 0;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (r < K && r >= cur[j]) c += sc[j] + lq(dep[j], r) > th;
      return c;
    }
    int lo = cur[j], hi = K;  // the first rank at or below th lies in [lo, hi]
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
      // keep the R best.  Candidates are numbered in node order: slot, lane, rank.
      int off[J];
      {
        int base = 0;
#pragma unroll
        for (int j = 0; j < J; ++j) {
          const int incl = wave_scan(cnt[j]);
          off[j] = base + incl - cnt[j];
          base += readlane(incl, kWave - 1);
        }
      }
      if (total <= kRankCap) {
        // exact ranks: larger key first, equal keys in node order
#pragma unroll
        for (int j = 0; j < J; ++j)
          for (int i = 0; i < cnt[j]; ++i)
            sm.key[off[j] + i] = key_of(sc[j] + lq(dep[j], cur[j] + i));
        const int Tp = (total + 7) & ~7;
        if (lane < Tp - total) sm.key[total + lane] = 0ull;  // below every real key
        __syncthreads();
        for (int i0 = 0; i0 < total; i0 += kWave) {
          const int i = i0 + lane;
          const unsigned long long mk = i < total ? sm.key[i] : ~0ull;
          int r = 0;
          for (int j0 = 0; j0 < Tp; j0 += 8) {
            unsigned long long kj[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) kj[u] = sm.key[j0 + u];
#pragma unroll
            for (int u = 0; u < 8; ++u) r += kj[u] > mk || (kj[u] == mk && j0 + u < i);
          }
          if (i < total) sm.sel[i] = r < R;
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < J; ++j) {
          int c = 0;
          for (int i = 0; i < cnt[j]; ++i) c += sm.sel[off[j] + i];
          cnt[j] = c;
        }
      } else {
        // radix select over the 64-bit keys, 8 bits per pass from the first bit where
        // the candidates differ; k counts how many keys of the current bin belong in,
        // and the passes stop once that bin is taken whole
        unsigned long long kmax = 0ull, kmin = ~0ull;
#pragma unroll
        for (int j = 0; j < J; ++j)
          if (cnt[j] > 0) {
            kmax = max(kmax, key_of(sc[j] + lq(dep[j], cur[j])));
            kmin = min(kmin, key_of(sc[j] + lq(dep[j], cur[j] + cnt[j] - 1)));
          }
        kmax = wave_max_u64(kmax);
        kmin = wave_min_u64(kmin);
        const unsigned long long diff = kmax ^ kmin;
        const int top = diff ? 63 - __clzll((long long)diff) : -1;
        unsigned long long pmask = top >= 63 ? 0ull : (~0ull << (top + 1));
        unsigned long long prefix = kmax & pmask;
        int k = R;
        for (int hi = top; hi >= 0; hi -= 8) {
          const int lo = max(hi - 7, 0);
          const int nbins = 1 << (hi - lo + 1);
          const unsigned long long dmask = (unsigned long long)(nbins - 1);
          for (int b = lane; b < 256; b += kWave) sm.hist[b] = 0;
          __syncthreads();
#pragma unroll
          for (int j = 0; j < J; ++j)
            for (int i = 0; i < cnt[j]; ++i) {
              const unsigned long long key = key_of(sc[j] + lq(dep[j], cur[j] + i));
              if ((key & pmask) == prefix) atomicAdd(&sm.hist[(key >> lo) & dmask], 1);
            }
          __syncthreads();
          // lane l holds bins nbins-1-4l .. nbins-4-4l: the scan runs from the top bin down
          int h[4], loc = 0;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int bi = nbins - 1 - 4 * lane - q;
            h[q] = bi >= 0 ? sm.hist[bi] : 0;
            loc += h[q];
          }
          const int incl = wave_scan(loc);
          const int excl = incl - loc;
          const int src = max(__ffsll((long long)ballot(excl < k && incl >= k)) - 1, 0);
          int bin = 0, higher = 0, inbin = 0;
          if (lane == src) {
            int acc = excl;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              if (acc + h[q] >= k) {
                bin = nbins - 1 - 4 * lane - q;
                higher = acc;
                inbin = h[q];
                break;
              }
              acc += h[q];
            }
          }
          bin = readlane(bin, src);
          higher = readlane(higher, src);
          inbin = readlane(inbin, src);
          k -= higher;
          prefix |= (unsigned long long)bin << lo;
          pmask |= dmask << lo;
          __syncthreads();
          if (inbin == k) break;
        }
        // per stream: the keys above the bin, then the first k keys in the bin in node order
        int gt[J], eq[J];
#pragma unroll
        for (int j = 0; j < J; ++j) {
          gt[j] = 0;
          eq[j] = 0;
          for (int i = 0; i < cnt[j]; ++i) {
            const unsigned long long key = key_of(sc[j] + lq(dep[j], cur[j] + i)) & pmask;
            gt[j] += key > prefix;
            eq[j] += key == prefix;
          }
        }
        int before = 0;
#pragma unroll
        for (int j = 0; j < J; ++j) {
          const int incl = wave_scan(eq[j]);
          const int take = min(max(k - (before + incl - eq[j]), 0), eq[j]);
          cnt[j] = gt[j] + take;
          before += readlane(incl, kWave - 1);
        }
      }
      total = R;
    }

    // the round's nodes get ids n .. n + total - 1 in (slot, lane) order; the parent
    // writes each child's whole stream state so the child opens it in one LDS read
    int base = n;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int incl = wave_scan(cnt[j]);
      const int firstid = base + incl - cnt[j];
      const int u = j * kWave + lane;
      if (cnt[j] > 0) {
        const bool kids_open = dep[j] + 1 < L;  // may the children have children?
        const double nn2 = best_child(dep[j] + 2);
#pragma unroll 4
        for (int i = 0; i < cnt[j]; ++i) {
          const int x = firstid + i;
          const double sx = sc[j] + lq(dep[j], cur[j] + i);
          if (x < N) {
            sm.parent[x] = u;
            sm.rank[x] = cur[j] + i;
            sm.depth[x] = dep[j] + 1;
            sm.score[x] = sx;
            sm.head[x] = kids_open ? sx + nxt[j] : -INFINITY;
            sm.nxt[x] = nn2;
          }
        }
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
        par[j] = sm.parent[x];
        rnk[j] = sm.rank[x];
        head[j] = sm.head[x];
        nxt[j] = sm.nxt[x];
        cur[j] = dep[j] < L ? 0 : K;
      }
    }
    n += total;
  }
  // a stream is consumed from its head, so u's selected children are ranks 0 .. nk-1
  int nk[J];
#pragma unroll
  for (int j = 0; j < J; ++j) nk[j] = (j * kWave + lane < n && dep[j] < L) ? cur[j] : 0;

  // canonical renumbering, one depth at a time.  Depth d's canonical order is known;
  // a scan of its child counts gives each node the canonical index of its first child.
  if (lane == 0) {
    sm.order[0] = 0;
    sm.nkc[0] = nk[0];
    sm.canon[0] = 0;
  }
  int cn[J];  // canonical index of the lane's nodes
#pragma unroll
  for (int j = 0; j < J; ++j) cn[j] = (j == 0 && lane == 0) ? 0 : -1;
  __syncthreads();
  int lvl_lo = 0, lvl_hi = 1;  // canonical range of the previous depth
  for (int d = 1; lvl_hi < n && d <= L; ++d) {
    int base = lvl_hi;
    for (int p0 = lvl_lo; p0 < lvl_hi; p0 += kWave) {
      const int p = p0 + lane;
      const bool in = p < lvl_hi;
      const int v = in ? sm.order[p] : 0;
      const int c = in ? sm.nkc[p] : 0;
      const int incl = wave_scan(c);
      if (in) sm.first[v] = base + incl - c;
      base += readlane(incl, kWave - 1);
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int x = j * kWave + lane;
      if (x < n && x > 0 && dep[j] == d) {
        const int ci = sm.first[par[j]] + rnk[j];
        cn[j] = ci;
        if (ci >= 0 && ci < N) {
          sm.order[ci] = x;
          sm.nkc[ci] = nk[j];
        }
        sm.canon[x] = ci;
      }
    }
    __syncthreads();
    lvl_lo = lvl_hi;
    lvl_hi = base;
  }

  // each node writes its own entry; lanes past n write the padding
  const int64_t o = (int64_t)s * N;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int x = j * kWave + lane;
    if (x < n) {
      const int ci = cn[j];
      if (ci >= 0 && ci < N) {
        const int d = dep[j];
        tree_tok[o + ci] = d == 0 ? bonus[s] : sm.ltok[(d - 1) * K + rnk[j]];
        tree_parent[o + ci] = d == 0 ? -1 : sm.canon[par[j]];
        tree_depth[o + ci] = d;
        if (node_logq) node_logq[o + ci] = (float)sc[j];
      }
    } else if (x < N) {
      tree_tok[o + x] = -1;
      tree_parent[o + x] = -1;
      tree_depth[o + x] = -1;
      if (node_logq) node_logq[o + x] = -INFINITY;
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
