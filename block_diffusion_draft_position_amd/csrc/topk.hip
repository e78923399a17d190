// Per-position softmax statistics and top-K over the vocabulary.
//
// The drafter's marginal q_i of each draft position (DDTree page "策展 · X
// (Twitter)", section 運作流程 step 1) arrives as a row of fp32 logits.  We need
// the K largest logits (largest first, equal logits by smaller id) and
// log q = logit - logsumexp(row).
//
// Two kernels, both HBM-streaming:
//   topk_partial  grid (chunks, rows), 256 threads.  Each wave streams an
//                 interleaved part of one chunk with 16-byte loads, keeping
//                 (a) a running max and an fp64 sum of exp(x - max) per lane, and
//                 (b) a sorted top-K list spread over the wave, lane i holding
//                 the i-th best.  A value enters the list only if it beats the
//                 current K-th entry, which after the first few hundred elements
//                 is rare, so the stream runs at load rate.
//   topk_merge    one wave per row merges the lists and statistics of all
//                 chunks and writes tokens and log-probabilities.
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

  __device__ void init() {
    val = -INFINITY;
    id = INT_MAX;
    thr_val = -INFINITY;
    thr_id = INT_MAX;
  }

  // Insert the uniform candidate (v, i) if it beats the k-th entry.
  __device__ void insert(float v, int i, int k) {
    if (!better(v, i, thr_val, thr_id)) return;
    const int lane = lane_id();
    const bool ahead = lane < k && better(val, id, v, i);
    const int pos = __popcll(ballot(ahead));
    const float up_v = __shfl_up(val, 1);
    const int up_i = __shfl_up(id, 1);
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

  // Offer one value per lane; candidates are inserted one at a time.
  __device__ void offer(float v, int i, bool valid, int k) {
    unsigned long long m = ballot(valid && better(v, i, thr_val, thr_id));
    while (m) {
      const int src = __ffsll((long long)m) - 1;
      m &= m - 1;
      insert(readlane(v, src), readlane(i, src), k);
    }
  }
};

__device__ __forceinline__ void stat_add4(float& m, double& s, float x0, float x1, float x2,
                                          float x3) {
  const float mx = fmaxf(fmaxf(x0, x1), fmaxf(x2, x3));
  if (mx > m) {
    s = (m == -INFINITY) ? 0.0 : s * exp2((double)(m - mx) * (double)kLog2e);
    m = mx;
  }
  if (m == -INFINITY) return;  // nothing valid seen yet (ragged tail)
  const float e = __builtin_amdgcn_exp2f((x0 - m) * kLog2e) + __builtin_amdgcn_exp2f((x1 - m) * kLog2e) +
                  __builtin_amdgcn_exp2f((x2 - m) * kLog2e) + __builtin_amdgcn_exp2f((x3 - m) * kLog2e);
  s += (double)e;
}

__global__ void __launch_bounds__(kThreads)
topk_partial(const float* __restrict__ logits, int64_t rows, int64_t stride, int vocab, int k,
             int64_t chunk_len, bool vec_ok, float* __restrict__ cand_val,
             int* __restrict__ cand_id, Stat* __restrict__ stats) {
  const int nchunks = (int)(gridDim.x / rows);
  const int c = (int)(blockIdx.x % nchunks);
  const int64_t row = blockIdx.x / nchunks;
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid % kWave;
  const float* x = logits + row * stride;
  const int lo = (int)(c * chunk_len);
  const int hi = (int)min<int64_t>((int64_t)lo + chunk_len, vocab);

  TopList list;
  list.init();
  float m = -INFINITY;
  double s = 0.0;

  int base = lo + tid * 4;
  if (vec_ok) {
    for (; base + 3 < hi; base += kThreads * 4) {
      const float4 v = *reinterpret_cast<const float4*>(x + base);
      stat_add4(m, s, v.x, v.y, v.z, v.w);
      list.offer(v.x, base + 0, true, k);
      list.offer(v.y, base + 1, true, k);
      list.offer(v.z, base + 2, true, k);
      list.offer(v.w, base + 3, true, k);
    }
  }
  // scalar path (unaligned rows) and the ragged tail
  for (; base < hi; base += kThreads * 4) {
    float v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = (base + j < hi) ? x[base + j] : -INFINITY;
    stat_add4(m, s, v[0], v[1], v[2], v[3]);
#pragma unroll
    for (int j = 0; j < 4; ++j) list.offer(v[j], base + j, base + j < hi, k);
  }
  // lanes that never saw a value keep m = -inf, s = 0
  const float wm = wave_max(m);
  const double ws = wave_sum(m == -INFINITY ? 0.0 : s * exp2((double)(m - wm) * (double)kLog2e));
  const int64_t slot = (row * nchunks + c) * kWavesPerBlock + wave;
  if (lane < k) {
    cand_val[slot * k + lane] = list.val;
    cand_id[slot * k + lane] = list.id;
  }
  if (lane == 0) {
    Stat st;
    st.m = wm;
    st.pad = 0.f;
    st.s = ws;
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

  // log-sum-exp over lists, fp64
  float m = -INFINITY;
  for (int i = lane; i < nlists; i += kWave) m = fmaxf(m, st[i].m);
  const float M = wave_max(m);
  double s = 0.0;
  for (int i = lane; i < nlists; i += kWave) {
    const Stat t = st[i];
    if (t.m != -INFINITY) s += t.s * exp2((double)(t.m - M) * (double)kLog2e);
  }
  s = wave_sum(s);
  const double lse = (double)M + log(s);

  TopList list;
  list.init();
  const int64_t n = (int64_t)nlists * k;
  const float* cv = cand_val + row * n;
  const int* ci = cand_id + row * n;
  for (int64_t b = 0; b < n; b += kWave) {
    const int64_t i = b + lane;
    const bool valid = i < n;
    const float v = valid ? cv[i] : -INFINITY;
    const int id = valid ? ci[i] : INT_MAX;
    list.offer(v, id, valid && id != INT_MAX, k);
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
  const size_t nslot = (size_t)rows * nch * kWavesPerBlock;
  p.ws_bytes = align_up(nslot * k * sizeof(float), 256) + align_up(nslot * k * sizeof(int), 256) +
               align_up(nslot * sizeof(Stat), 256);
  return p;
}

hipError_t launch_topk(const float* logits, int64_t rows, int64_t vocab, int64_t stride, int k,
                       int32_t* tok, float* logq, void* ws, const TopkPlan& plan, hipStream_t st) {
  const size_t nslot = (size_t)rows * plan.nchunks * kWavesPerBlock;
  char* w = static_cast<char*>(ws);
  float* cv = reinterpret_cast<float*>(w);
  w += align_up(nslot * k * sizeof(float), 256);
  int* ci = reinterpret_cast<int*>(w);
  w += align_up(nslot * k * sizeof(int), 256);
  Stat* stt = reinterpret_cast<Stat*>(w);
  const bool vec_ok = (reinterpret_cast<uintptr_t>(logits) % 16 == 0) && (stride % 4 == 0);
  hipLaunchKernelGGL(topk_partial, dim3((unsigned)(plan.nchunks * rows)), dim3(kThreads), 0, st,
                     logits, rows, stride, (int)vocab, k, plan.chunk_len, vec_ok, cv, ci, stt);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(topk_merge, dim3((unsigned)rows), dim3(kWave), 0, st,
                     plan.nchunks * kWavesPerBlock, k, cv, ci, stt, tok, logq);
  return hipGetLastError();
}

}  // namespace ddt
