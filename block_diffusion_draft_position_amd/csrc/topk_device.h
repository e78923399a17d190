// Device pieces of the top-K step shared by the top-K kernels and the fused
// draft-tree kernel: 64-bit (value, id) keys, the wave-level top-K selection and the
// merge of one row's chunk lists and softmax statistics.  See topk.hip for the method.
#pragma once

#include <float.h>
#include <limits.h>

#include "ddt_internal.h"

namespace ddt {
namespace topk {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kCap = 256;  // candidates ranked by counting

typedef float f32x4 __attribute__((ext_vector_type(4)));

struct WaveLds {
  unsigned long long ck[kCap + kWave];  // candidates, then one spare slot per lane
  unsigned long long ok[kWave];  // the top K in rank order
};

// Orders LDS traffic among the lanes of one wave (all the top-K code needs): the
// wave's LDS instructions execute in order, so a compiler barrier with wavefront-scope
// fences suffices, and waves of a larger workgroup do not have to meet.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// order-preserving map of a float to uint32
__device__ __forceinline__ unsigned fkey(float v) {
  const unsigned b = __builtin_bit_cast(unsigned, v + 0.f);  // -0 -> +0
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// (value, id) <-> one 64-bit word: the value's key above the complement of the id;
// 0 means "none"
__device__ __forceinline__ unsigned long long pack(float v, int id) {
  if (id == INT_MAX) return 0ull;
  return ((unsigned long long)fkey(v) << 32) | (unsigned)(0xffffffffu - (unsigned)id);
}

__device__ __forceinline__ void unpack(unsigned long long key, float& v, int& id) {
  const unsigned k = (unsigned)(key >> 32);
  v = key ? __builtin_bit_cast(float, (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k) : -INFINITY;
  id = key ? (int)(0xffffffffu - (unsigned)(key & 0xffffffffull)) : INT_MAX;
}

// the value whose fkey is k, for k from a non-NaN value (-0 never occurs: fkey maps it
// to +0's key, whose inverse is +0)
__device__ __forceinline__ float unfkey(unsigned k) {
  return __builtin_bit_cast(float, (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

__device__ __forceinline__ unsigned long long readlane_u64(unsigned long long v, int lane) {
  const unsigned lo = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)v, lane);
  const unsigned hi = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)(v >> 32), lane);
  return ((unsigned long long)hi << 32) | lo;
}

__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
#define DDT_MAXSTEP(S)                                                                        \
  {                                                                                           \
    const unsigned lo = (unsigned)xchg<S>((int)(unsigned)v);                                  \
    const unsigned hi = (unsigned)xchg<S>((int)(unsigned)(v >> 32));                          \
    const unsigned long long o = ((unsigned long long)hi << 32) | lo;                         \
    v = o > v ? o : v;                                                                        \
  }
  DDT_MAXSTEP(1) DDT_MAXSTEP(2) DDT_MAXSTEP(4) DDT_MAXSTEP(8) DDT_MAXSTEP(16) DDT_MAXSTEP(32)
#undef DDT_MAXSTEP
  return v;
}

// The wave-level top-K below works in two stages.  A single wave pays a full pipeline
// latency for each dependent step (about 40 cycles for a VALU op, 70 for a ballot and
// popcount) and about 8 cycles per independent VALU op, so each stage is kept to a
// few dependent steps and little work per element:
//   1. kth_upper: th bounds the K-th largest lane maximum from below, found on the
//      upper 32 key bits (the value bits) two bits at a time, three independent ballots
//      per step, stopping once exactly K lanes reach it.  At least K keys reach th, so
//      the top K all do; usually few others do (about K ln(64 / (64 - K)) for random
//      data).
//   2. rank_select: those candidates are gathered in LDS as 64-bit keys and each counts
//      the keys above its own, which is its rank (keys are unique: they embed the id).
//      More than kCap candidates (adversarial layouts) falls back to K rounds of a
//      wave-wide maximum.

// the largest th (on 32-bit upper key halves) that at least K lanes' mh reach; 0 when
// fewer than K lanes hold keys
__device__ __forceinline__ unsigned kth_upper(unsigned mh, int K) {
  unsigned th = 0;
  for (int b = 30; b >= 0; b -= 2) {
    const unsigned c1 = th | (1u << b), c2 = th | (2u << b), c3 = th | (3u << b);
    const int n1 = __popcll(ballot(mh >= c1));
    const int n2 = __popcll(ballot(mh >= c2));
    const int n3 = __popcll(ballot(mh >= c3));
    int n = K + 1;
    if (n3 >= K) {
      th = c3;
      n = n3;
    } else if (n2 >= K) {
      th = c2;
      n = n2;
    } else if (n1 >= K) {
      th = c1;
      n = n1;
    }
    if (n == K) break;
  }
  return th;
}

// The C <= kCap candidate keys in sm.ck[0, C) (stored by this wave, not yet synced)
// each count the keys above their own, which is their rank; on return lane i < K
// holds the i-th largest in rk, other lanes 0.
__device__ __forceinline__ void rank_count(int C, int K, unsigned long long& rk, WaveLds& sm) {
  const int lane = lane_id();
  const int Cp = (C + 1) & ~1;  // the counting loop reads two keys at a time
  if (lane < Cp - C) sm.ck[C + lane] = 0ull;
  wave_lds_sync();
  for (int i0 = 0; i0 < C; i0 += kWave) {
    const int i = i0 + lane;
    const unsigned long long me = i < C ? sm.ck[i] : 0ull;
    int r = 0;
#pragma unroll 4
    for (int j = 0; j < Cp; j += 2) {
      const ulonglong2 x = *reinterpret_cast<const ulonglong2*>(&sm.ck[j]);
      r += (x.x > me) + (x.y > me);
    }
    if (i < C && r < K) sm.ok[r] = me;
  }
  wave_lds_sync();
  rk = lane < min(C, K) ? sm.ok[lane] : 0ull;
  wave_lds_sync();  // sm is free again
}

// Top K of the candidates: element e of the lane when cand(e) (its key keyof(e), with
// valid(e) marking the elements that exist at all), plus the carried key rk when
// carry.  On return lane i < K holds the i-th largest key in rk; other lanes hold 0.
template <int E, typename Valid, typename Cand, typename KeyOf>
__device__ void rank_select(Valid valid, Cand cand, KeyOf keyof, bool carry,
                            unsigned long long& rk, int K, WaveLds& sm) {
  const int lane = lane_id();
  int cnt = carry;
#pragma unroll
  for (int e = 0; e < E; ++e) cnt += cand(e);
  const int incl = wave_scan(cnt);
  const int C = readlane(incl, kWave - 1);
  if (C <= kCap) {
    // every element is stored, a non-candidate into this lane's spare slot, so the
    // gather has no branches
    int o = incl - cnt;
    sm.ck[carry ? o : kCap + lane] = rk;
    o += carry;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const bool c = cand(e);
      sm.ck[c ? o : kCap + lane] = keyof(e);
      o += c;
    }
    rank_count(C, K, rk, sm);
  } else {
    unsigned long long taken = 0ull;  // bit e: element e taken
    bool carry_taken = false;         // the carried key taken
    unsigned long long out = 0ull;
    for (int r = 0; r < K; ++r) {
      unsigned long long b = carry_taken ? 0ull : rk;
#pragma unroll
      for (int e = 0; e < E; ++e)
        if (valid(e) && !((taken >> e) & 1ull) && keyof(e) > b) b = keyof(e);
      const unsigned long long w = wave_max_u64(b);
      if (w == 0ull) break;  // nothing left anywhere
      if (b == w) {
        if (rk == w) carry_taken = true;
#pragma unroll
        for (int e = 0; e < E; ++e)
          if (valid(e) && keyof(e) == w) taken |= 1ull << e;
      }
      if (lane == r) out = w;
    }
    rk = out;
  }
}

// Top K of the wave's keys: E per lane (0 = none) plus one carried key rk per lane.
template <int E>
__device__ void wave_topk(const unsigned long long (&key)[E], unsigned long long& rk, int K,
                          WaveLds& sm) {
  unsigned mh = (unsigned)(rk >> 32);
#pragma unroll
  for (int e = 0; e < E; ++e) mh = max(mh, (unsigned)(key[e] >> 32));
  const unsigned th = kth_upper(mh, K);
  const unsigned long long t = th ? (unsigned long long)th << 32 : 1ull;
  rank_select<E>([&](int e) { return key[e] != 0ull; }, [&](int e) { return key[e] >= t; },
                 [&](int e) { return key[e]; }, rk >= t, rk, K, sm);
}

// Top K of one chunk of the logits row x, E per lane in v (element e of the lane has
// id lo + ((e / 4) * 64 + lane) * 4 + e % 4; ids at or past vocab do not exist), with
// m the lane's maximum (-inf over absent elements).  The result is wave_topk's on the
// elements' keys, but the keys are formed for the candidates only: the bound th on
// the upper key bits becomes a bound tau on the values (fkey is monotone; no NaNs),
// each element slot is skipped by a uniform branch when no lane holds a candidate
// there, and a lane's candidates are stored at offsets from a ballot's bit count.
template <int E>
__device__ void chunk_topk(const float (&v)[E], const float* __restrict__ x, int lo, int vocab,
                           float m, int K, unsigned long long& rk, WaveLds& sm) {
  const int lane = lane_id();
  auto idof = [&](int e) { return lo + ((e / 4) * kWave + lane) * 4 + e % 4; };
  const bool full = lo + kWave * E <= vocab;  // every element exists
  // the lane maximum's upper key bits: 0 for a lane without elements (its first id is
  // its smallest)
  const unsigned mh = idof(0) < vocab ? fkey(m) : 0u;
  const unsigned th = kth_upper(mh, K);
  // keys >= th << 32 (>= 1 when th = 0) are the existing elements of value >= tau;
  // at or below -inf's key (0x007fffff) every existing element qualifies
  const float tau = th <= 0x007fffffu ? -INFINITY : unfkey(th);
  auto cand = [&](int e) { return (full || idof(e) < vocab) && v[e] >= tau; };
  int C = 0;  // candidates so far (uniform)
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const bool c = cand(e);
    const unsigned long long msk = ballot(c);
    if (msk) {
      if (c) {
        // candidates in the lanes below this one
        const unsigned below = __builtin_amdgcn_mbcnt_lo((unsigned)msk, 0u);
        const int o = C + (int)__builtin_amdgcn_mbcnt_hi((unsigned)(msk >> 32), below);
        if (o < kCap) sm.ck[o] = pack(v[e], idof(e));
      }
      C += (int)__popcll(msk);
    }
  }
  rk = 0ull;
  if (C <= kCap) {
    rank_count(C, K, rk, sm);
  } else {
    // more than kCap candidates (many equal values): K rounds of a wave-wide maximum
    // over the keys not taken yet.  The values are read again from the row, four at a
    // time, in every round: keeping them or their keys live into this rare path took
    // the kernel from 30 to over 100 registers (a third of its occupancy).
    static_assert(E <= 32, "one bit per element");
    unsigned taken = 0u;  // bit e: element e taken
    unsigned long long out = 0ull;
    for (int r = 0; r < K; ++r) {
      unsigned long long b = 0ull;
      int be = 0;
#pragma unroll 1
      for (int g = 0; g < E / 4; ++g) {  // four contiguous elements at a time
        const int id0 = idof(4 * g);
        float w[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) w[q] = id0 + q < vocab ? x[id0 + q] : 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int e = 4 * g + q;
          const bool ok = id0 + q < vocab && !((taken >> e) & 1u);
          const unsigned long long ke = ok ? pack(w[q], id0 + q) : 0ull;
          if (ke > b) {
            b = ke;
            be = e;
          }
        }
      }
      const unsigned long long w = wave_max_u64(b);
      if (w == 0ull) break;  // nothing left anywhere
      if (b == w) taken |= 1u << be;  // keys are unique: one lane, one element
      if (lane == r) out = w;
    }
    rk = out;
  }
}

// One wave merges row `row`'s chunk lists (nchunks lists of k keys, each sorted best
// first) and statistics: on return lane i < k holds the row's i-th best (rv, ri), and
// lse its log-sum-exp.  Lane c holds chunk c's list (E >= k keys; 64 chunks per batch),
// so a lane's maximum is its chunk's best key and the threshold of wave_topk is the
// k-th best chunk head: only a handful of keys beyond the top k reach it.  The
// statistics (up to kStat per lane) and the first batch of keys are loaded together.
template <int E>
__device__ void merge_row(int64_t row, int nchunks, int k, const unsigned long long* __restrict__ cand,
                          const float2* __restrict__ stats, WaveLds& sm, float& rv, int& ri,
                          double& lse) {
  constexpr int kStat = 4;
  const int lane = lane_id();
  const float2* st = stats + row * nchunks;
  const unsigned long long* cr = cand + row * (int64_t)nchunks * k;
  float2 sv[kStat];
#pragma unroll
  for (int q = 0; q < kStat; ++q) {
    const int i = q * kWave + lane;
    sv[q] = i < nchunks ? st[i] : make_float2(-INFINITY, 0.f);
  }
  unsigned long long kv[E];
  auto load = [&](int c) {
#pragma unroll
    for (int e = 0; e < E; ++e) kv[e] = (c < nchunks && e < k) ? cr[(int64_t)c * k + e] : 0ull;
  };
  load(lane);
  float mm = -INFINITY;
#pragma unroll
  for (int q = 0; q < kStat; ++q) mm = fmaxf(mm, sv[q].x);
  for (int i = kStat * kWave + lane; i < nchunks; i += kWave) mm = fmaxf(mm, st[i].x);
  const float MM = wave_max(mm);
  double ss = 0.0;
#pragma unroll
  for (int q = 0; q < kStat; ++q)
    if (q * kWave + lane < nchunks)
      ss += (double)sv[q].y * (double)__builtin_amdgcn_exp2f((sv[q].x - MM) * kLog2e);
  for (int i = kStat * kWave + lane; i < nchunks; i += kWave) {
    const float2 t = st[i];
    ss += (double)t.y * (double)__builtin_amdgcn_exp2f((t.x - MM) * kLog2e);
  }
  // the sum stays fp64; its logarithm is taken in fp32 (one instruction instead of a
  // long software routine; absolute error about 2e-6 for sums up to 2^31)
  lse = (double)MM + (double)(__builtin_amdgcn_logf((float)wave_sum(ss)) * 0.6931471805599453f);

  unsigned long long rk = 0ull;
  for (int c0 = 0; c0 < nchunks; c0 += kWave) {
    if (c0 > 0) load(c0 + lane);
    wave_topk<E>(kv, rk, k, sm);
  }
  unpack(rk, rv, ri);
}

}  // namespace topk
}  // namespace ddt
