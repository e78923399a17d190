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
  float cv[kCap];
  int ci[kCap];
  float ov[kWave];
  int oi[kWave];
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
  const unsigned b = __builtin_bit_cast(unsigned, v);
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

// Top-K of the wave's values: E per lane, v[e] with id idof(e) (INT_MAX = none),
// plus one carried entry (rv, ri) per lane.  On return lane i < K holds the i-th
// best in (rv, ri); other lanes hold (-inf, INT_MAX).  Ids must be distinct.
template <int E, typename IdOf>
__device__ void wave_topk(const float (&v)[E], IdOf idof, float& rv, int& ri, int K, WaveLds& sm) {
  const int lane = lane_id();
  const unsigned rk = ri != INT_MAX ? fkey(rv) : 0u;
  unsigned mk = rk;
#pragma unroll
  for (int e = 0; e < E; ++e)
    if (idof(e) != INT_MAX) mk = max(mk, fkey(v[e]));
  // t = the largest key with at least K lanes whose maximum reaches it
  unsigned t = 0;
  for (int b = 31; b >= 0; --b) {
    const unsigned c = t | (1u << b);
    if (__popcll(ballot(mk >= c)) >= K) t = c;
  }
  t = max(t, 1u);
  int cnt = rk >= t;
#pragma unroll
  for (int e = 0; e < E; ++e) cnt += idof(e) != INT_MAX && fkey(v[e]) >= t;
  const int incl = wave_scan(cnt);
  const int C = readlane(incl, kWave - 1);
  if (C <= kCap) {
    int o = incl - cnt;
    if (rk >= t) {
      sm.cv[o] = rv;
      sm.ci[o] = ri;
      ++o;
    }
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (idof(e) != INT_MAX && fkey(v[e]) >= t) {
        sm.cv[o] = v[e];
        sm.ci[o] = idof(e);
        ++o;
      }
    // pad to a multiple of 8 so the counting loop below can read 8 at a time
    const int Cp = (C + 7) & ~7;
    if (lane < Cp - C) {
      sm.cv[C + lane] = -INFINITY;
      sm.ci[C + lane] = INT_MAX;
    }
    wave_lds_sync();
    for (int i0 = 0; i0 < C; i0 += kWave) {
      const int i = i0 + lane;
      const float mv = i < C ? sm.cv[i] : -INFINITY;
      const int mi = i < C ? sm.ci[i] : INT_MAX;
      int r = 0;
      for (int j0 = 0; j0 < Cp; j0 += 8) {
        float jv[8];
        int ji[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          jv[u] = sm.cv[j0 + u];
          ji[u] = sm.ci[j0 + u];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) r += better(jv[u], ji[u], mv, mi);
      }
      if (i < C && r < K) {
        sm.ov[r] = mv;
        sm.oi[r] = mi;
      }
    }
    wave_lds_sync();
    const int nout = min(C, K);
    rv = lane < nout ? sm.ov[lane] : -INFINITY;
    ri = lane < nout ? sm.oi[lane] : INT_MAX;
    wave_lds_sync();
  } else {
    // many values tie at the threshold: take the K best one at a time
    unsigned long long taken = 0ull;  // bit e: v[e] taken; bit E: the carried entry
    float outv = -INFINITY;
    int outi = INT_MAX;
    for (int r = 0; r < K; ++r) {
      float bv = -INFINITY;
      int bi = INT_MAX, be = -1;
      if (ri != INT_MAX && !((taken >> E) & 1ull)) {
        bv = rv;
        bi = ri;
        be = E;
      }
#pragma unroll
      for (int e = 0; e < E; ++e)
        if (!((taken >> e) & 1ull) && idof(e) != INT_MAX && better(v[e], idof(e), bv, bi)) {
          bv = v[e];
          bi = idof(e);
          be = e;
        }
      float wv = bv;
      int wi = bi;
      wave_argmax(wv, wi);
      if (wi == INT_MAX) break;  // nothing left anywhere
      if (be >= 0 && bi == wi) taken |= 1ull << be;
      if (lane == r) {
        outv = wv;
        outi = wi;
      }
    }
    rv = outv;
    ri = outi;
  }
}

// One wave merges row `row`'s chunk lists (nchunks * k keys) and statistics: on
// return lane i < k holds the row's i-th best (rv, ri), and lse its log-sum-exp.
template <int E>
__device__ void merge_row(int64_t row, int nchunks, int k, const unsigned long long* __restrict__ cand,
                          const float2* __restrict__ stats, WaveLds& sm, float& rv, int& ri,
                          double& lse) {
  const int lane = lane_id();
  const float2* st = stats + row * nchunks;
  float mm = -INFINITY;
  for (int i = lane; i < nchunks; i += kWave) mm = fmaxf(mm, st[i].x);
  const float MM = wave_max(mm);
  double ss = 0.0;
  for (int i = lane; i < nchunks; i += kWave) {
    const float2 t = st[i];
    ss += (double)t.y * (double)__builtin_amdgcn_exp2f((t.x - MM) * kLog2e);
  }
  lse = (double)MM + log(wave_sum(ss));

  const int n = nchunks * k;
  const unsigned long long* cr = cand + row * (int64_t)n;
  rv = -INFINITY;
  ri = INT_MAX;
  for (int b0 = 0; b0 < n; b0 += kWave * E) {
    float v[E];
    int id[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int i = b0 + e * kWave + lane;
      unpack(i < n ? cr[i] : 0ull, v[e], id[e]);
    }
    wave_topk<E>(v, [&](int e) { return id[e]; }, rv, ri, k, sm);
  }
}

}  // namespace topk
}  // namespace ddt
