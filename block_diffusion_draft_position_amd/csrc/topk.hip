// Per-position softmax statistics and top-K over the vocabulary.
//
// The drafter's marginal q_i of each draft position (DDTree page "策展 · X
// (Twitter)", section 運作流程 step 1) arrives as a row of fp32 logits.  We need
// the K largest logits (larger first, equal logits by smaller id) and
// log q = logit - logsumexp(row).
//
// Two kernels, one wave per workgroup, no atomics:
//   topk_partial  a wave owns a chunk of 64*E logits of one row and loads all of it
//                 into registers with 16-byte loads issued together (one memory
//                 latency per chunk).  It forms the chunk's max and sum of
//                 exp(x - max) (fp32 per lane, fp64 across the wave) and the chunk's
//                 top-K list (wave_topk below), and writes both to the workspace:
//                 the list as 64-bit keys, the statistics as a (max, sum) pair.
//   topk_merge    one wave per row reads every chunk's keys, spread over all 64
//                 lanes, merges them with the same wave_topk, folds the statistics
//                 into the log-sum-exp (fp64) and writes tokens and log-probabilities.
//
// wave_topk: a bit-by-bit ballot search finds t, the K-th largest of the 64 per-lane
// maxima.  At least K lanes hold a value >= t, so every member of the top-K is >= t,
// and usually only a few more values are (about K ln(64/(64-K)) for random data).
// Those candidates are gathered in LDS and each one's rank is counted exactly; if
// there are too many (heavy ties), K rounds of wave arg-max take the K best instead.
#include <float.h>
#include <limits.h>

#include "ddt_internal.h"

namespace ddt {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kCap = 256;  // candidates ranked by counting

typedef float f32x4 __attribute__((ext_vector_type(4)));

struct WaveLds {
  float cv[kCap];
  int ci[kCap];
  float ov[kWave];
  int oi[kWave];
};

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
    __syncthreads();
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
    __syncthreads();
    const int nout = min(C, K);
    rv = lane < nout ? sm.ov[lane] : -INFINITY;
    ri = lane < nout ? sm.oi[lane] : INT_MAX;
    __syncthreads();
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

template <int E>
__global__ void __launch_bounds__(kWave)
topk_partial(const float* __restrict__ logits, int64_t stride, int vocab, int k, int nchunks,
             bool vec_ok, unsigned long long* __restrict__ cand, float2* __restrict__ stats) {
  __shared__ WaveLds sm;
  const int c = (int)(blockIdx.x % (unsigned)nchunks);
  const int64_t row = blockIdx.x / (unsigned)nchunks;
  const int lane = threadIdx.x;
  const float* x = logits + row * stride;
  const int lo = c * kWave * E;

  float v[E];
#pragma unroll
  for (int b = 0; b < E / 4; ++b) {
    const int base = lo + (b * kWave + lane) * 4;
    if (vec_ok && base + 3 < vocab) {
      const f32x4 t = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(x + base));
#pragma unroll
      for (int q = 0; q < 4; ++q) v[4 * b + q] = t[q];
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) v[4 * b + q] = base + q < vocab ? x[base + q] : -INFINITY;
    }
  }
  auto idof = [&](int e) -> int {
    const int i = lo + ((e / 4) * kWave + lane) * 4 + e % 4;
    return i < vocab ? i : INT_MAX;
  };
  float m = -INFINITY;
#pragma unroll
  for (int e = 0; e < E; ++e)
    if (idof(e) != INT_MAX) m = fmaxf(m, v[e]);
  const float M = wave_max(m);
  float se = 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e)
    if (idof(e) != INT_MAX) se += __builtin_amdgcn_exp2f((v[e] - M) * kLog2e);
  const double S = wave_sum((double)se);

  float rv = -INFINITY;
  int ri = INT_MAX;
  wave_topk<E>(v, idof, rv, ri, k, sm);
  const int64_t slot = row * nchunks + c;
  if (lane < k) cand[slot * k + lane] = pack(rv, ri);
  if (lane == 0) stats[slot] = make_float2(M, (float)S);
}

template <int E>
__global__ void __launch_bounds__(kWave)
topk_merge(int nchunks, int k, const unsigned long long* __restrict__ cand,
           const float2* __restrict__ stats, int32_t* __restrict__ out_tok,
           float* __restrict__ out_logq) {
  __shared__ WaveLds sm;
  const int64_t row = blockIdx.x;
  const int lane = threadIdx.x;
  const float2* st = stats + row * nchunks;
  float mm = -INFINITY;
  for (int i = lane; i < nchunks; i += kWave) mm = fmaxf(mm, st[i].x);
  const float MM = wave_max(mm);
  double ss = 0.0;
  for (int i = lane; i < nchunks; i += kWave) {
    const float2 t = st[i];
    ss += (double)t.y * (double)__builtin_amdgcn_exp2f((t.x - MM) * kLog2e);
  }
  const double lse = (double)MM + log(wave_sum(ss));

  const int n = nchunks * k;
  const unsigned long long* cr = cand + row * (int64_t)n;
  float rv = -INFINITY;
  int ri = INT_MAX;
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
  if (lane < k) {
    out_tok[row * k + lane] = ri;
    out_logq[row * k + lane] = (float)((double)rv - lse);
  }
}

}  // namespace

TopkPlan topk_plan(int64_t rows, int64_t vocab, int k) {
  TopkPlan p;
  // chunk length: short chunks (more waves) for small problems, long ones once the
  // grid is full anyway
  const int64_t full = 4 * (int64_t)cu_count();
  p.e = 32;
  for (int e : {8, 16}) {
    if (rows * ceil_div(vocab, (int64_t)kWave * e * 2) < full) {
      p.e = e;
      break;
    }
  }
  p.nchunks = (int)ceil_div(vocab, (int64_t)kWave * p.e);
  p.merge_e = (int64_t)p.nchunks * k <= kWave * 8 ? 8 : 32;
  const size_t nslot = (size_t)rows * p.nchunks;
  p.ws_bytes = align_up(nslot * k * sizeof(unsigned long long), 256) +
               align_up(nslot * sizeof(float2), 256);
  return p;
}

hipError_t launch_topk(const float* logits, int64_t rows, int64_t vocab, int64_t stride, int k,
                       int32_t* tok, float* logq, void* ws, const TopkPlan& plan, hipStream_t st) {
  const size_t nslot = (size_t)rows * plan.nchunks;
  unsigned long long* cand = static_cast<unsigned long long*>(ws);
  float2* stt = reinterpret_cast<float2*>(static_cast<char*>(ws) +
                                          align_up(nslot * k * sizeof(unsigned long long), 256));
  const bool vec_ok = (reinterpret_cast<uintptr_t>(logits) % 16 == 0) && (stride % 4 == 0);
  const dim3 grid((unsigned)(rows * plan.nchunks));
#define DDT_PART(EE)                                                                            \
  hipLaunchKernelGGL(topk_partial<EE>, grid, dim3(kWave), 0, st, logits, stride, (int)vocab, k, \
                     plan.nchunks, vec_ok, cand, stt)
  if (plan.e == 8)
    DDT_PART(8);
  else if (plan.e == 16)
    DDT_PART(16);
  else
    DDT_PART(32);
#undef DDT_PART
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (plan.merge_e == 8)
    hipLaunchKernelGGL(topk_merge<8>, dim3((unsigned)rows), dim3(kWave), 0, st, plan.nchunks, k,
                       cand, stt, tok, logq);
  else
    hipLaunchKernelGGL(topk_merge<32>, dim3((unsigned)rows), dim3(kWave), 0, st, plan.nchunks, k,
                       cand, stt, tok, logq);
  return hipGetLastError();
}

}  // namespace ddt
