// Per-position softmax statistics and top-K over the vocabulary.
//
// The drafter's marginal q_i of each draft position (DDTree page "策展 · X
// (Twitter)", section 運作流程 step 1) arrives as a row of fp32 logits.  We need
// the K largest logits (largest first, equal logits by smaller id) and
// log q = logit - logsumexp(row).
//
// Two kernels, both HBM-streaming:
//   topk_partial  one 256-thread workgroup per (row, chunk).  Each wave streams an
//                 interleaved part of the chunk with 16-byte loads, keeping
//                 (a) a running max and an fp64 sum of exp(x - max) per lane, and
//                 (b) a sorted top-K list spread over the wave, lane i holding the
//                 i-th best.  The list starts as a bitonic sort of the first 64
//                 values; after that a value enters only if it beats the K-th
//                 entry, which is rare, and enters by a one-lane DPP shift.  The
//                 four waves' lists and sums are merged in LDS, one result per
//                 workgroup.
//   topk_merge    one wave per row merges the chunks' lists and sums and writes
//                 tokens and log-probabilities.
#include <float.h>
#include <limits.h>

#include "ddt_internal.h"

namespace ddt {
namespace {

constexpr int kThreads = 256;
constexpr int kWavesPerBlock = kThreads / kWave;
constexpr float kLog2e = 1.4426950408889634f;

struct Stat {
  float m;
  float pad;
  double s;  // sum of exp(x - m)
};

// Wave-wide sorted list: lane i < k holds the i-th best (val, id).
struct TopList {
  float val;
  int id;
  float thr_val;  // k-th best so far (uniform)
  int thr_id;

  // Start from one value per lane (invalid lanes contribute nothing).
  __device__ void seed(float v, int i, bool valid, int k) {
    val = valid ? v : -INFINITY;
    id = valid ? i : INT_MAX;
    wave_sort(val, id);
    thr_val = readlane(val, k - 1);
    thr_id = readlane(id, k - 1);
  }

  // Insert the uniform candidate (v, i) if it beats the k-th entry.
  __device__ void insert(float v, int i, int k) {
    if (!better(v, i, thr_val, thr_id)) return;
    const int lane = lane_id();
    const bool ahead = lane < k && better(val, id, v, i);
    const int pos = __popcll(ballot(ahead));
    const float up_v = shift_up1(val, -INFINITY);
    const int up_i = shift_up1(id, INT_MAX);
    if (lane > pos) {
      val = up_v;
      id = up_i;
    }
    if (lane == pos) {
      val = v;
      id = i;
    }
    thr_val = readlane(val, k - 1);
    thr_id = readlane(id, k - 1);
  }

  // Offer one value per lane; the (few) qualifying ones are inserted one by one.
  __device__ void offer(float v, int i, bool valid, int k) {
    unsigned long long m = ballot(valid && better(v, i, thr_val, thr_id));
    while (m) {
      const int src = __ffsll((long long)m) - 1;
      m &= m - 1;
      insert(readlane(v, src), readlane(i, src), k);
    }
  }
};

__device__ __forceinline__ void stat_add4(float& m, double& s, const float (&x)[4]) {
  const float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
  if (mx > m) {
    s = (m == -INFINITY) ? 0.0 : s * exp2((double)(m - mx) * (double)kLog2e);
    m = mx;
  }
  if (m == -INFINITY) return;  // nothing valid seen yet
  const float e = __builtin_amdgcn_exp2f((x[0] - m) * kLog2e) + __builtin_amdgcn_exp2f((x[1] - m) * kLog2e) +
                  __builtin_amdgcn_exp2f((x[2] - m) * kLog2e) + __builtin_amdgcn_exp2f((x[3] - m) * kLog2e);
  s += (double)e;
}

// Merge (m, s) pairs: returns the pair for the union.
__device__ __forceinline__ void stat_merge(float& m, double& s, float m2, double s2) {
  if (m2 == -INFINITY) return;
  if (m == -INFINITY) {
    m = m2;
    s = s2;
    return;
  }
  const float mx = fmaxf(m, m2);
  s = s * exp2((double)(m - mx) * (double)kLog2e) + s2 * exp2((double)(m2 - mx) * (double)kLog2e);
  m = mx;
}

__global__ void __launch_bounds__(kThreads)
topk_partial(const float* __restrict__ logits, int nchunks, int64_t stride, int vocab, int k,
             int64_t chunk_len, bool vec_ok, float* __restrict__ cand_val,
             int* __restrict__ cand_id, Stat* __restrict__ stats) {
  __shared__ float lv[kWavesPerBlock][kWave];
  __shared__ int li[kWavesPerBlock][kWave];
  __shared__ float lm[kWavesPerBlock];
  __shared__ double ls[kWavesPerBlock];
  const int c = (int)(blockIdx.x % nchunks);
  const int64_t row = blockIdx.x / nchunks;
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid % kWave;
  const float* x = logits + row * stride;
  const int lo = (int)(c * chunk_len);
  const int hi = (int)min<int64_t>((int64_t)lo + chunk_len, vocab);
  const int niter = (hi - lo + kThreads * 4 - 1) / (kThreads * 4);  // uniform over the block

  TopList list;
  float m = -INFINITY;
  double s = 0.0;
  for (int it = 0; it < niter; ++it) {
    const int base = lo + (it * kThreads + tid) * 4;
    float v[4];
    if (vec_ok && base + 3 < hi) {
      const float4 t = *reinterpret_cast<const float4*>(x + base);
      v[0] = t.x;
      v[1] = t.y;
      v[2] = t.z;
      v[3] = t.w;
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = (base + j < hi) ? x[base + j] : -INFINITY;
    }
    stat_add4(m, s, v);
    if (it == 0) {
      list.seed(v[0], base, base < hi, k);
#pragma unroll
      for (int j = 1; j < 4; ++j) list.offer(v[j], base + j, base + j < hi, k);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) list.offer(v[j], base + j, base + j < hi, k);
    }
  }
  // per-wave results to LDS
  const float wm = wave_max(m);
  const double ws = wave_sum(m == -INFINITY ? 0.0 : s * exp2((double)(m - wm) * (double)kLog2e));
  lv[wave][lane] = lane < k ? list.val : -INFINITY;
  li[wave][lane] = lane < k ? list.id : INT_MAX;
  if (lane == 0) {
    lm[wave] = wm;
    ls[wave] = ws;
  }
  __syncthreads();
  if (wave != 0) return;
  // wave 0 folds in the other waves' lists and sums
  float fm = lm[0];
  double fs = ls[0];
#pragma unroll
  for (int w = 1; w < kWavesPerBlock; ++w) stat_merge(fm, fs, lm[w], ls[w]);
  for (int w = 1; w < kWavesPerBlock; ++w) {
    const float v = lv[w][lane];
    const int i = li[w][lane];
    list.offer(v, i, lane < k && i != INT_MAX, k);
  }
  const int64_t slot = row * nchunks + c;
  if (lane < k) {
    cand_val[slot * k + lane] = list.val;
    cand_id[slot * k + lane] = list.id;
  }
  if (lane == 0) {
    Stat st;
    st.m = fm;
    st.pad = 0.f;
    st.s = fs;
    stats[slot] = st;
  }
}

__global__ void __launch_bounds__(kWave)
topk_merge(int nlists, int k, const float* __restrict__ cand_val, const int* __restrict__ cand_id,
           const Stat* __restrict__ stats, int32_t* __restrict__ out_tok,
           float* __restrict__ out_logq) {
  const int64_t row = blockIdx.x;
  const int lane = threadIdx.x;
  const Stat* st = stats + row * nlists;

  // log-sum-exp over the chunks, fp64
  float m = -INFINITY;
  double s = 0.0;
  for (int i = lane; i < nlists; i += kWave) {
    const Stat t = st[i];
    stat_merge(m, s, t.m, t.s);
  }
  const float M = wave_max(m);
  s = wave_sum(m == -INFINITY ? 0.0 : s * exp2((double)(m - M) * (double)kLog2e));
  const double lse = (double)M + log(s);

  const int n = nlists * k;
  const float* cv = cand_val + row * (int64_t)n;
  const int* ci = cand_id + row * (int64_t)n;
  TopList list;
  {
    const bool valid = lane < n;
    list.seed(valid ? cv[lane] : -INFINITY, valid ? ci[lane] : INT_MAX, valid && ci[lane] != INT_MAX, k);
  }
  constexpr int kBatch = 4;  // batches loaded together, so their loads overlap
  for (int b0 = kWave; b0 < n; b0 += kBatch * kWave) {
    float v[kBatch];
    int id[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int i = b0 + j * kWave + lane;
      v[j] = i < n ? cv[i] : -INFINITY;
      id[j] = i < n ? ci[i] : INT_MAX;
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) list.offer(v[j], id[j], id[j] != INT_MAX, k);
  }
  if (lane < k) {
    out_tok[row * k + lane] = list.id;
    out_logq[row * k + lane] = (float)((double)list.val - lse);
  }
}

}  // namespace

TopkPlan topk_plan(int64_t rows, int64_t vocab, int k) {
  TopkPlan p;
  const int64_t target_blocks = 1024;
  const int64_t max_chunks = std::max<int64_t>(1, vocab / 2048);
  int64_t nch = std::min<int64_t>(std::max<int64_t>(1, ceil_div(target_blocks, rows)), max_chunks);
  int64_t len = (int64_t)align_up((size_t)ceil_div(vocab, nch), 4);
  nch = ceil_div(vocab, len);
  p.nchunks = (int)nch;
  p.chunk_len = len;
  const size_t nslot = (size_t)rows * nch;
  p.ws_bytes = align_up(nslot * k * sizeof(float), 256) + align_up(nslot * k * sizeof(int), 256) +
               align_up(nslot * sizeof(Stat), 256);
  return p;
}

hipError_t launch_topk(const float* logits, int64_t rows, int64_t vocab, int64_t stride, int k,
                       int32_t* tok, float* logq, void* ws, const TopkPlan& plan, hipStream_t st) {
  const size_t nslot = (size_t)rows * plan.nchunks;
  char* w = static_cast<char*>(ws);
  float* cv = reinterpret_cast<float*>(w);
  w += align_up(nslot * k * sizeof(float), 256);
  int* ci = reinterpret_cast<int*>(w);
  w += align_up(nslot * k * sizeof(int), 256);
  Stat* stt = reinterpret_cast<Stat*>(w);
  const bool vec_ok = (reinterpret_cast<uintptr_t>(logits) % 16 == 0) && (stride % 4 == 0);
  hipLaunchKernelGGL(topk_partial, dim3((unsigned)(plan.nchunks * rows)), dim3(kThreads), 0, st,
                     logits, plan.nchunks, stride, (int)vocab, k, plan.chunk_len, vec_ok, cv, ci,
                     stt);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(topk_merge, dim3((unsigned)rows), dim3(kWave), 0, st, plan.nchunks, k, cv, ci,
                     stt, tok, logq);
  return hipGetLastError();
}

}  // namespace ddt
