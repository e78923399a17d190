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
  unsigned long long ck[kCap];   // candidates
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

// Top-K of the wave's keys: E per lane (0 = none) plus one carried key rk per lane.
// Keys are unique (they embed the id), so every rank below is exact.  On return
// lane i < K holds the i-th largest key in rk; other lanes hold 0.
//
// A single wave pays a full pipeline latency for each dependent step (about 40 cycles
// for a VALU op, 70 for a ballot and popcount) and about 8 cycles per independent
// VALU op, so each stage below is kept to a few dependent steps:
//   1. t bounds the K-th largest lane maximum from below (a ballot search on the value
//      bits).  At least K keys reach t, so the top K all do; usually few others do
//      (about K ln(64 / (64 - K)) for random data).
//   2. the keys >= t are gathered in LDS and each counts the candidates above it;
//      its count is its rank.
//   More than kCap candidates (adversarial layouts) falls back to K rounds of a
//   wave-wide maximum.
template <int E>
__device__ void wave_topk(const unsigned long long (&key)[E], unsigned long long& rk, int K,
                          WaveLds& sm) {
  const int lane = lane_id();
  unsigned long long mk = rk;
#pragma unroll
  for (int e = 0; e < E; ++e) mk = key[e] > mk ? key[e] : mk;
  // t: the largest 64-bit key whose upper half at least K lane maxima reach, found two
  // bits at a time on the upper halves (the value bits; three independent ballots per
  // step).  Once exactly K lanes reach it no larger threshold keeps K, so the search
  // stops there.
  const unsigned mh = (unsigned)(mk >> 32);
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
  // keys are non-zero exactly when present; with fewer than K present lanes th stays 0
  const unsigned long long t = th ? (unsigned long long)th << 32 : 1ull;

  int cnt = rk >= t;
#pragma unroll
  for (int e = 0; e < E; ++e) cnt += key[e] >= t;
  const int incl = wave_scan(cnt);
  const int C = readlane(incl, kWave - 1);
  if (C <= kCap) {
    int o = incl - cnt;
    if (rk >= t) sm.ck[o++] = rk;
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (key[e] >= t) sm.ck[o++] = key[e];
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
  } else {
    unsigned long long taken = 0ull;  // bit e: key[e] taken; bit E: the carried key
    unsigned long long out = 0ull;
    for (int r = 0; r < K; ++r) {
      unsigned long long b = ((taken >> E) & 1ull) ? 0ull : rk;
#pragma unroll
      for (int e = 0; e < E; ++e)
        if (!((taken >> e) & 1ull) && key[e] > b) b = key[e];
      const unsigned long long w = wave_max_u64(b);
      if (w == 0ull) break;  // nothing left anywhere
      if (b == w) {
        if (rk == w && !((taken >> E) & 1ull)) taken |= 1ull << E;
#pragma unroll
        for (int e = 0; e < E; ++e)
          if (key[e] == w) taken |= 1ull << e;
      }
      if (lane == r) out = w;
    }
    rk = out;
  }
}

// One wave merges row `row`'s chunk lists (nchunks * k keys) and statistics: on
// return lane i < k holds the row's i-th best (rv, ri), and lse its log-sum-exp.
// The statistics (up to kStat per lane) and the first batch of keys are loaded
// together, so a row costs one memory latency per batch of 64 * E keys.
template <int E>
__device__ void merge_row(int64_t row, int nchunks, int k, const unsigned long long* __restrict__ cand,
                          const float2* __restrict__ stats, WaveLds& sm, float& rv, int& ri,
                          double& lse) {
  constexpr int kStat = 4;
  const int lane = lane_id();
  const float2* st = stats + row * nchunks;
  const int n = nchunks * k;
  const unsigned long long* cr = cand + row * (int64_t)n;
  float2 sv[kStat];
#pragma unroll
  for (int q = 0; q < kStat; ++q) {
    const int i = q * kWave + lane;
    sv[q] = i < nchunks ? st[i] : make_float2(-INFINITY, 0.f);
  }
  unsigned long long kv[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int i = e * kWave + lane;
    kv[e] = i < n ? cr[i] : 0ull;
  }
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
  for (int b0 = 0; b0 < n; b0 += kWave * E) {
    if (b0 > 0) {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int i = b0 + e * kWave + lane;
        kv[e] = i < n ? cr[i] : 0ull;
      }
    }
    wave_topk<E>(kv, rk, k, sm);
  }
  unpack(rk, rv, ri);
}

}  // namespace topk
}  // namespace ddt
