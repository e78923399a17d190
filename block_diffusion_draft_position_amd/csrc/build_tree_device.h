// Device side of the draft-tree construction, shared by the tree kernel and the fused
// draft-tree kernel.  See build_tree.hip for the method.
#pragma once

#include <limits.h>

#include <type_traits>

#include "ddt_internal.h"

namespace ddt {
namespace tree {

constexpr int kRankCap = 256;  // final rounds with at most this many candidates rank them exactly
constexpr int kGatherCap = 2048;  // radix selects over at most this many keys read them from LDS

struct TreeSmem {
  unsigned long long* key;  // [kGatherCap] final-round candidate keys
  int* sel;                 // [kRankCap] candidate taken?
  double* score;  // [N] node -> prefix log-probability
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
  int* cpar;      // [N] canonical index -> canonical parent (-1: root or padding)
};

__host__ __device__ constexpr size_t smem_bytes(int N, int LK) {
  return sizeof(unsigned long long) * kGatherCap + sizeof(int) * kRankCap + sizeof(double) * (size_t)N +
         (sizeof(float) + sizeof(int)) * (size_t)LK + sizeof(int) * 256 + sizeof(int) * 8 * (size_t)N;
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


// Lays the tree's LDS arrays out from p.
__device__ inline TreeSmem carve(unsigned char* p, int N, int LK) {
  TreeSmem sm;
  sm.key = reinterpret_cast<unsigned long long*>(p);
  p += sizeof(unsigned long long) * kGatherCap;
  sm.score = reinterpret_cast<double*>(p);
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
  sm.cpar = ip + 7 * N;
  return sm;
}

// Builds one sequence's tree with one wave.  sm.lq / sm.ltok hold the sequence's
// [L, K] top-K log-probabilities and tokens.  Writes the N-entry output rows (node_logq
// and pos_ids may be null; pos_ids gets P + depth) and sm.cpar, and returns num_nodes.  sync() orders the wave's LDS
// traffic: a workgroup barrier when the wave is alone, a wave barrier otherwise.
// J register slots of streams per lane.  SK > 0 (K <= SK, SK = 8 or 16, J <= 2) caches
// each stream's logq row in SK registers for the round, so its reads are issued
// together and the per-rank loops run SK steps.  rows(m) returns once rows 0 .. m-1
// of sm.lq / sm.ltok are in place (the fused kernel merges them while this runs): the
// root needs rows 0 and 1, and round r at most rows 0 .. r + 2, since every round
// deepens the tree by at most one.
template <int J, int SK, typename Sync, typename Rows>
__device__ __forceinline__ int build(TreeSmem& sm, int L, int K, int B, int bonus_tok,
                     int32_t* __restrict__ tree_tok, int32_t* __restrict__ tree_parent,
                     int32_t* __restrict__ tree_depth, float* __restrict__ node_logq,
                     int32_t* __restrict__ pos_ids, int P, Sync sync, Rows rows) {
  const int lane = lane_id();
  const int N = B + 1;
  auto lq = [&](int d, int r) -> double { return (double)sm.lq[d * K + r]; };
  // bound on the children of a depth-d candidate: logq[d][0], none past depth L
  auto best_child = [&](int d) -> double { return d < L ? lq(d, 0) : -INFINITY; };

  // node u lives at (lane u % 64, slot u / 64): its stream and its place in the tree
  double sc[J];    // score(u)
  double head[J];  // score of u's next child, -inf once the stream is closed
  float nxt[J];    // best_child(depth(u) + 1), a logq entry
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
  rows(min(L, 2));
  if (lane == 0) {  // the root
    cur[0] = 0;
    head[0] = lq(0, 0);
    nxt[0] = best_child(1);
    sm.depth[0] = 0;
    sm.score[0] = 0.0;
  }

  // candidates of stream j scoring above th: a prefix of the stream.  Small K reads
  // the whole row at once; larger K bisects.
  constexpr int KW = SK > 0 ? SK : 1;
  float rowv[SK ? J : 1][KW];  // SK: this round's logq row of each stream
  auto above = [&](int j, double th) -> int {
    if (cur[j] >= K) return 0;
    if constexpr (SK > 0) {
      int c = 0;
#pragma unroll
      for (int r = 0; r < KW; ++r)
        if (r < K && r >= cur[j]) c += sc[j] + (double)rowv[j][r] > th;
      return c;
    }
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
  for (int round = 0; n - 1 < B; ++round) {
    rows(min(L, round + 3));
    const int R = B - (n - 1);
    // slots that hold nodes (and so streams): per-slot work and wave scans stop there
    const int jn = (n + kWave - 1) / kWave;
    if constexpr (SK > 0) {
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const bool open = cur[j] < K;
        const int rb = (open ? dep[j] : 0) * K;
#pragma unroll
        for (int r = 0; r < KW; ++r) rowv[j][r] = (open && r < K) ? sm.lq[rb + r] : -INFINITY;
      }
    }
    bool live = false;
    double tl = -INFINITY;
#pragma unroll
    for (int j = 0; j < J; ++j)
      if (j < jn && cur[j] < K) {
        live = true;
        tl = fmax(tl, head[j] + (double)nxt[j]);
      }
    if (!ballot(live)) break;  // the candidate tree is exhausted
    // in the first round the root (lane 0, slot 0) holds the only stream, so the
    // round's maximum and count are lane 0's own
    const bool root_only = n == 1;
    const double tau = root_only ? readlane_f64(tl, 0) : wave_max_d(tl);
    int cnt[J];
    int mine = 0;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      cnt[j] = j < jn ? above(j, tau) : 0;
      mine += cnt[j];
    }
    // uniform across the wave: the compiler then keeps the counts, the budget and the
    // search prefixes below in scalar registers and branches on them without masks
    int total = __builtin_amdgcn_readfirstlane(root_only ? mine : wave_sum_i(mine));

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
          off[j] = base;
          if (j < jn) {
            const int incl = wave_scan(cnt[j]);
            off[j] = base + incl - cnt[j];
            base += readlane(incl, kWave - 1);
          }
        }
      }
      // Candidate keys: the fp64 score's order-preserving 64 bits.  Candidate i of
      // stream j (rank cur + i) has node-order number off[j] + i (parent's selection
      // order, then rank); equal scores are taken in that order, in every cut below.
      if (total <= kRankCap) {
#pragma unroll
        for (int j = 0; j < J; ++j) {
          if constexpr (SK > 0) {
#pragma unroll
            for (int r = 0; r < KW; ++r)
              if (r >= cur[j] && r < cur[j] + cnt[j])
                sm.key[off[j] + r - cur[j]] = key_of(sc[j] + (double)rowv[j][r]);
          } else {
            for (int i = 0; i < cnt[j]; ++i)
              sm.key[off[j] + i] = key_of(sc[j] + lq(dep[j], cur[j] + i));
          }
        }
        if (total <= kWave) {
          // one candidate per lane (lane = node-order number): the R-th largest key t by
          // a ballot search two bits at a time (three independent ballots per step),
          // stopping once exactly R keys reach the prefix.  If more than R keys are >= t,
          // the keys equal to t tie at the boundary and the lowest lanes among them fill
          // the budget.  Each stream then keeps its candidates in the taken set.
          sync();
          const bool has = lane < total;
          const unsigned long long mk = has ? sm.key[lane] : 0ull;
          unsigned long long t = 0ull;
          int nge = total;  // keys >= t
          for (int b = 62; b >= 0; b -= 2) {
            const unsigned long long c1 = t | (1ull << b), c2 = t | (2ull << b), c3 = t | (3ull << b);
            // mk = 0 where no candidate, below every threshold
            const int n1 = __popcll(ballot(mk >= c1));
            const int n2 = __popcll(ballot(mk >= c2));
            const int n3 = __popcll(ballot(mk >= c3));
            if (n3 >= R) {
              t = c3;
              nge = n3;
            } else if (n2 >= R) {
              t = c2;
              nge = n2;
            } else if (n1 >= R) {
              t = c1;
              nge = n1;
            }
            if (nge == R) break;
          }
          // lanes holding t that are taken: all of them, or the lowest R - (keys > t)
          unsigned long long eqt = ballot(has && mk == t);
          if (nge > R) {
            int need = R - __popcll(ballot(mk > t));
            unsigned long long keep = 0ull;
            for (; need > 0; --need) {
              const unsigned long long low = eqt & (~eqt + 1ull);
              keep |= low;
              eqt ^= low;
            }
            eqt = keep;
          }
          auto taken = [&](unsigned long long key, int idx) {
            return key > t || (key == t && ((eqt >> idx) & 1ull));
          };
#pragma unroll
          for (int j = 0; j < J; ++j) {
            int c = 0;
            if constexpr (SK > 0) {
#pragma unroll
              for (int r = 0; r < KW; ++r)
                c += r >= cur[j] && r < cur[j] + cnt[j] &&
                     taken(key_of(sc[j] + (double)rowv[j][r]), off[j] + r - cur[j]);
            } else {
              for (int i = 0; i < cnt[j]; ++i)
                c += taken(key_of(sc[j] + lq(dep[j], cur[j] + i)), off[j] + i);
            }
            cnt[j] = c;
          }
          sync();  // sm.key is read again by the next cut
        } else {
          // exact ranks: each candidate counts the keys above its own and the equal keys
          // of lower node order
          const int Tp = (total + 7) & ~7;
          if (lane < Tp - total) sm.key[total + lane] = 0ull;  // below every real key
          sync();
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
          sync();
#pragma unroll
          for (int j = 0; j < J; ++j) {
            int c = 0;
            if constexpr (SK > 0) {
              int sv[KW];
#pragma unroll
              for (int i = 0; i < KW; ++i) sv[i] = i < cnt[j] ? sm.sel[off[j] + i] : 0;
#pragma unroll
              for (int i = 0; i < KW; ++i) c += sv[i];
            } else {
              for (int i = 0; i < cnt[j]; ++i) c += sm.sel[off[j] + i];
            }
            cnt[j] = c;
          }
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
        // Up to kGatherCap candidates: their keys are formed once, in node order, and
        // every pass reads them from LDS with all lanes; beyond, each pass recomputes
        // them stream by stream.
        const bool gathered = total <= kGatherCap;
        if (gathered) {
#pragma unroll
          for (int j = 0; j < J; ++j)
            if (j < jn) {
#pragma unroll 4
              for (int i = 0; i < cnt[j]; ++i) sm.key[off[j] + i] = key_of(sc[j] + lq(dep[j], cur[j] + i));
            }
        }
        for (int hi = top; hi >= 0; hi -= 8) {
          const int lo = max(hi - 7, 0);
          const int nbins = 1 << (hi - lo + 1);
          const unsigned long long dmask = (unsigned long long)(nbins - 1);
          for (int b = lane; b < 256; b += kWave) sm.hist[b] = 0;
          sync();
          if (gathered) {
#pragma unroll 4
            for (int f = lane; f < total; f += kWave) {
              const unsigned long long key = sm.key[f];
              if ((key & pmask) == prefix) atomicAdd(&sm.hist[(key >> lo) & dmask], 1);
            }
          } else {
#pragma unroll
            for (int j = 0; j < J; ++j)
              for (int i = 0; i < cnt[j]; ++i) {
                const unsigned long long key = key_of(sc[j] + lq(dep[j], cur[j] + i));
                if ((key & pmask) == prefix) atomicAdd(&sm.hist[(key >> lo) & dmask], 1);
              }
          }
          sync();
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
          sync();
          if (inbin == k) break;
        }
        // per stream: the keys above the bin, then the first k keys in the bin in node order
        int gt[J], eq[J];
#pragma unroll
        for (int j = 0; j < J; ++j) {
          gt[j] = 0;
          eq[j] = 0;
          if (j >= jn) continue;
          if (gathered) {
            // a stream's keys are sorted (largest first), so both counts are searches:
            // the first key at or below the prefix, and the first key below it
            auto first = [&](bool strict) {
              int lo = 0, len = cnt[j];
              while (len > 0) {
                const int half = len >> 1;
                const unsigned long long key = sm.key[off[j] + lo + half] & pmask;
                if (strict ? key > prefix : key >= prefix) {
                  lo += half + 1;
                  len -= half + 1;
                } else {
                  len = half;
                }
              }
              return lo;
            };
            gt[j] = first(true);
            eq[j] = first(false) - gt[j];
          } else {
            for (int i = 0; i < cnt[j]; ++i) {
              const unsigned long long key = key_of(sc[j] + lq(dep[j], cur[j] + i)) & pmask;
              gt[j] += key > prefix;
              eq[j] += key == prefix;
            }
          }
        }
        int before = 0;
#pragma unroll
        for (int j = 0; j < J; ++j) {
          cnt[j] = 0;
          if (j < jn) {
            const int incl = wave_scan(eq[j]);
            const int take = min(max(k - (before + incl - eq[j]), 0), eq[j]);
            cnt[j] = gt[j] + take;
            before += readlane(incl, kWave - 1);
          }
        }
      }
      total = R;
    }

    if (root_only) {
      // the root's children ranks 0 .. total-1 become nodes 1 .. total, one per lane
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int x = j * kWave + lane;
        if (j * kWave <= total && x >= 1 && x <= total) {
          sm.parent[x] = 0;
          sm.rank[x] = x - 1;
        }
      }
      if (lane == 0) {
        if constexpr (SK > 0) {
          float hv = -INFINITY;
#pragma unroll
          for (int r = 0; r < KW; ++r)
            if (r == total) hv = rowv[0][r];
          head[0] = total < K ? (double)hv : -INFINITY;
        } else {
          head[0] = total < K ? lq(0, total) : -INFINITY;
        }
        cur[0] = total;
      }
    } else {
      // the round's nodes get ids n .. n + total - 1 in (slot, lane) order.  A parent
      // records only (parent, rank) for each new child; the child's own lane then reads
      // its parent's depth and score and its logq row.
      int base = n;
#pragma unroll
      for (int j = 0; j < J; ++j) {
        if (j < jn) {  // no streams past jn, so no candidates
          const int incl = wave_scan(cnt[j]);
          const int firstid = base + incl - cnt[j];
          const int u = j * kWave + lane;
          if (cnt[j] > 0) {
            for (int i = 0; i < cnt[j]; ++i) {
              const int x = firstid + i;
              if (x < N) {
                sm.parent[x] = u;
                sm.rank[x] = cur[j] + i;
              }
            }
            const int cn = cur[j] + cnt[j];
            if constexpr (SK > 0) {
              float hv = -INFINITY;
#pragma unroll
              for (int r = 0; r < KW; ++r)
                if (r == cn) hv = rowv[j][r];
              head[j] = cn < K ? sc[j] + (double)hv : -INFINITY;
            } else {
              head[j] = cn < K ? sc[j] + lq(dep[j], cn) : -INFINITY;
            }
            cur[j] = cn;
          }
          base += readlane(incl, kWave - 1);
        }
      }
    }
    sync();
    // each new node opens its stream
#pragma unroll
    for (int j = 0; j < J; ++j) {
      if (j * kWave < n + total) {
        const int x = j * kWave + lane;
        if (x >= n && x < n + total) {
          const int u = sm.parent[x];
          const int r = sm.rank[x];
          const int pd = sm.depth[u];
          const double ps = sm.score[u];
          dep[j] = pd + 1;
          sc[j] = ps + lq(pd, r);
          const bool open = dep[j] < L;
          cur[j] = open ? 0 : K;
          head[j] = open ? sc[j] + lq(dep[j], 0) : -INFINITY;
          nxt[j] = dep[j] + 1 < L ? sm.lq[(dep[j] + 1) * K] : -INFINITY;
          sm.depth[x] = dep[j];
          sm.score[x] = sc[j];
        }
      }
    }
    n += total;
  }
  // parent and rank of the lane's nodes (the root's are -1), read back once
  int par[J], rnk[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int x = j * kWave + lane;
    par[j] = (x > 0 && x < n) ? sm.parent[x] : -1;
    rnk[j] = (x > 0 && x < n) ? sm.rank[x] : -1;
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
  sync();
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
    sync();
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int x = j * kWave + lane;
      if (j * kWave < n && x < n && x > 0 && dep[j] == d) {
        const int ci = sm.first[par[j]] + rnk[j];
        cn[j] = ci;
        if (ci >= 0 && ci < N) {
          sm.order[ci] = x;
          sm.nkc[ci] = nk[j];
        }
        sm.canon[x] = ci;
      }
    }
    sync();
    lvl_lo = lvl_hi;
    lvl_hi = base;
  }

  // each node writes its own entry; lanes past n write the padding
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int x = j * kWave + lane;
    if (x < n) {
      const int ci = cn[j];
      if (ci >= 0 && ci < N) {
        const int d = dep[j];
        const int pc = d == 0 ? -1 : sm.canon[par[j]];
        tree_tok[ci] = d == 0 ? bonus_tok : sm.ltok[(d - 1) * K + rnk[j]];
        tree_parent[ci] = pc;
        tree_depth[ci] = d;
        if (node_logq) node_logq[ci] = (float)sc[j];
        if (pos_ids) pos_ids[ci] = P + d;
        sm.cpar[ci] = pc;
      }
    } else if (x < N) {
      tree_tok[x] = -1;
      tree_parent[x] = -1;
      tree_depth[x] = -1;
      if (node_logq) node_logq[x] = -INFINITY;
      if (pos_ids) pos_ids[x] = -1;
      sm.cpar[x] = -1;
    }
  }
  return n;
}

}  // namespace tree
}  // namespace ddt
