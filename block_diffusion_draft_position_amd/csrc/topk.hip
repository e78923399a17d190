// Per-position softmax statistics and top-K over the vocabulary.
//
// The drafter's marginal q_i of each draft position (DDTree page "策展 · X
// (Twitter)", section 運作流程 step 1) arrives as a row of fp32 logits.  We need
// the K largest logits (larger first, equal logits by smaller id) and
// log q = logit - logsumexp(row).
//
// Two kernels, no atomics; every wave works on its own (four chunk waves share a
// workgroup: C1 +1% rounds/s over one-wave workgroups):
//   topk_partial  a wave owns a chunk of 64*E logits of one row and loads all of it
//                 into registers with 16-byte loads issued together (one memory
//                 latency per chunk).  It forms the chunk's max and sum of
//                 exp(x - max) (fp32 per lane, fp64 across the wave) and the chunk's
//                 top-K list (chunk_topk: wave_topk's selection with keys formed for
//                 the candidates only), and writes both to the workspace:
//                 the list as 64-bit keys, the statistics as a (max, sum) pair.
//   topk_merge    one wave per row reads every chunk's list, one list per lane,
//                 merges them with the same wave_topk, folds the statistics into the
//                 log-sum-exp (fp64 sum) and writes tokens and log-probabilities.
//
// wave_topk works on 64-bit keys (the value's order-preserving bits above the
// complemented id, so one unsigned compare orders by value, then smaller id): the
// K-th largest lane maximum bounds the top K from below, the keys above that bound
// are gathered in LDS, and each one's rank is counted exactly (topk_device.h).
#include "topk_device.h"

namespace ddt {
namespace {

using namespace topk;

constexpr int kPartWaves = 4;  // chunk waves per workgroup, each on its own

template <int E>
__global__ void __launch_bounds__(kPartWaves * kWave)
topk_partial(const float* __restrict__ logits, int64_t stride, int vocab, int k, int nchunks,
             int64_t nslots, bool vec_ok, unsigned long long* __restrict__ cand,
             float2* __restrict__ stats) {
  __shared__ WaveLds sms[kPartWaves];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int64_t slot0 = (int64_t)blockIdx.x * kPartWaves + wave;  // (row, chunk) of this wave
  if (slot0 >= nslots) return;
  WaveLds& sm = sms[wave];
  const int c = (int)(slot0 % nchunks);
  const int64_t row = slot0 / nchunks;
  const int lane = threadIdx.x % kWave;
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
  // elements past the row's end hold -inf: they add nothing to the maximum or the sum
  float m = -INFINITY;
#pragma unroll
  for (int e = 0; e < E; ++e) m = fmaxf(m, v[e]);
  const float M = wave_max(m);
  // a chunk of masked (-inf) logits only sums to 0, not to exp(-inf - -inf) = NaN
  const float Ms = M == -INFINITY ? 0.f : M;
  float se = 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) se += __builtin_amdgcn_exp2f((v[e] - Ms) * kLog2e);
  const double S = wave_sum((double)se);

  unsigned long long rk;
  chunk_topk<E>(v, x, lo, vocab, m, k, rk, sm);
  const int64_t slot = row * nchunks + c;
  if (lane < k) cand[slot * k + lane] = rk;
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
  float rv;
  int ri;
  double lse;
  merge_row<E>(row, nchunks, k, cand, stats, sm, rv, ri, lse);
  if (lane < k) {
    out_tok[row * k + lane] = ri;
    out_logq[row * k + lane] = (float)((double)rv - lse);
  }
}

}  // namespace

TopkPlan topk_plan(int64_t rows, int64_t vocab, int k) {
  TopkPlan p;
  // chunk length: short chunks (more waves) for small problems, 32 logits per lane
  // once that still gives two waves per CU (fewer, shorter chunk lists to merge: one
  // merge batch for V = 128256; over 16 per lane +1.3% rounds/s at C2, +0.9% and +1.5%
  // at C3 with B = 512 and 64; C1 keeps 8, 2% ahead of 32), else 16.  The chunk pass
  // takes 46 registers at 32 per lane (eight waves per SIMD) because it forms keys for
  // its candidates only.
  const int64_t full = 4 * (int64_t)cu_count();
  p.e = rows * ceil_div(vocab, (int64_t)kWave * 8 * 2) < full ? 8
        : rows * ceil_div(vocab, (int64_t)kWave * 32) < full / 2 ? 16
                                                              : 32;
  p.nchunks = (int)ceil_div(vocab, (int64_t)kWave * p.e);
  p.merge_e = k <= 8 ? 8 : k <= 32 ? 32 : 64;  // keys per lane: one chunk list each
  const size_t nslot = (size_t)rows * p.nchunks;
  p.ws_bytes = align_up(nslot * k * sizeof(unsigned long long), 256) +
               align_up(nslot * sizeof(float2), 256);
  return p;
}

void topk_ws_parts(void* ws, int64_t rows, int k, const TopkPlan& plan, unsigned long long** cand,
                   float2** stats) {
  const size_t nslot = (size_t)rows * plan.nchunks;
  *cand = static_cast<unsigned long long*>(ws);
  *stats = reinterpret_cast<float2*>(static_cast<char*>(ws) +
                                     align_up(nslot * k * sizeof(unsigned long long), 256));
}

hipError_t launch_topk_partial(const float* logits, int64_t rows, int64_t vocab, int64_t stride,
                               int k, void* ws, const TopkPlan& plan, hipStream_t st) {
  unsigned long long* cand;
  float2* stt;
  topk_ws_parts(ws, rows, k, plan, &cand, &stt);
  const bool vec_ok = (reinterpret_cast<uintptr_t>(logits) % 16 == 0) && (stride % 4 == 0);
  const int64_t nslots = rows * plan.nchunks;
  const dim3 grid((unsigned)ceil_div(nslots, kPartWaves));
#define DDT_PART(EE)                                                                            \
  hipLaunchKernelGGL(topk_partial<EE>, grid, dim3(kPartWaves * kWave), 0, st, logits, stride,   \
                     (int)vocab, k, plan.nchunks, nslots, vec_ok, cand, stt)
  if (plan.e == 8)
    DDT_PART(8);
  else if (plan.e == 16)
    DDT_PART(16);
  else
    DDT_PART(32);
#undef DDT_PART
  return hipGetLastError();
}

hipError_t launch_topk_merge(int64_t rows, int k, int32_t* tok, float* logq, void* ws,
                             const TopkPlan& plan, hipStream_t st) {
  unsigned long long* cand;
  float2* stt;
  topk_ws_parts(ws, rows, k, plan, &cand, &stt);
  if (plan.merge_e == 8)
    hipLaunchKernelGGL(topk_merge<8>, dim3((unsigned)rows), dim3(kWave), 0, st, plan.nchunks, k,
                       cand, stt, tok, logq);
  else if (plan.merge_e == 32)
    hipLaunchKernelGGL(topk_merge<32>, dim3((unsigned)rows), dim3(kWave), 0, st, plan.nchunks, k,
                       cand, stt, tok, logq);
  else
    hipLaunchKernelGGL(topk_merge<64>, dim3((unsigned)rows), dim3(kWave), 0, st, plan.nchunks, k,
                       cand, stt, tok, logq);
  return hipGetLastError();
}

hipError_t launch_topk(const float* logits, int64_t rows, int64_t vocab, int64_t stride, int k,
                       int32_t* tok, float* logq, void* ws, const TopkPlan& plan, hipStream_t st) {
  hipError_t e = launch_topk_partial(logits, rows, vocab, stride, k, ws, plan, st);
  if (e != hipSuccess) return e;
  return launch_topk_merge(rows, k, tok, logq, ws, plan, st);
}

}  // namespace ddt
