// Greedy tree walk (DDTree page "策展 · X (Twitter)", section 運作流程 step 4: follow
// the target's decoding rule from the root, accept while its token matches a child,
// carry the first mismatch as the next bonus token).
//
//   argmax_partial  grid (rows x chunks), 256 threads: argmax of one chunk of one
//                   node's target logits (larger value first, equal values by
//                   smaller id), 16-byte streaming loads.  Rows of padding nodes
//                   are skipped.
//   walk_kernel     one wave per sequence: merges the chunk results into the
//                   target's token at every node, then walks the tree.
#include <limits.h>

#include "ddt_internal.h"

namespace ddt {
namespace {

constexpr int kThreads = 256;

struct ArgMax {
  float v;
  int i;
};

__device__ __forceinline__ void take(ArgMax& a, float v, int i) {
  if (better(v, i, a.v, a.i)) {
    a.v = v;
    a.i = i;
  }
}

__global__ void __launch_bounds__(kThreads)
argmax_partial(const float* __restrict__ target, const int32_t* __restrict__ num_nodes, int N,
               int vocab, int nchunks, int64_t chunk_len, bool vec_ok,
               ArgMax* __restrict__ part) {
  __shared__ ArgMax red[kThreads / kWave];
  const int64_t rowc = blockIdx.x;
  const int c = (int)(rowc % nchunks);
  const int64_t row = rowc / nchunks;  // s * N + n
  const int s = (int)(row / N);
  const int n = (int)(row % N);
  if (n >= num_nodes[s]) return;
  const float* x = target + row * (int64_t)vocab;
  const int lo = (int)(c * chunk_len);
  const int hi = (int)min<int64_t>((int64_t)lo + chunk_len, vocab);
  const int tid = threadIdx.x;
  ArgMax a{-INFINITY, INT_MAX};
  for (int base = lo + tid * 4; base < hi; base += kThreads * 4) {
    if (vec_ok && base + 3 < hi) {
      const float4 v = *reinterpret_cast<const float4*>(x + base);
      take(a, v.x, base);
      take(a, v.y, base + 1);
      take(a, v.z, base + 2);
      take(a, v.w, base + 3);
    } else {
      for (int j = 0; j < 4 && base + j < hi; ++j) take(a, x[base + j], base + j);
    }
  }
  wave_argmax(a.v, a.i);
  if (tid % kWave == 0) red[tid / kWave] = a;
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < kThreads / kWave; ++w) take(a, red[w].v, red[w].i);
    part[rowc] = a;
  }
}

__global__ void __launch_bounds__(kWave)
walk_kernel(const int32_t* __restrict__ tree_tok, const int32_t* __restrict__ parent,
            const int32_t* __restrict__ num_nodes, const ArgMax* __restrict__ part, int N, int L,
            int nchunks, int32_t* __restrict__ accept_len, int32_t* __restrict__ acc_nodes,
            int32_t* __restrict__ acc_tok, int32_t* __restrict__ bonus_out) {
  extern __shared__ int smem[];
  int* want = smem;          // [N] target's greedy token at each node
  int* tok = smem + N;       // [N]
  int* par = smem + 2 * N;   // [N]
  const int s = blockIdx.x;
  const int lane = threadIdx.x;
  const int nn = num_nodes[s];
  for (int n = lane; n < nn; n += kWave) {
    tok[n] = tree_tok[(int64_t)s * N + n];
    par[n] = parent[(int64_t)s * N + n];
    const ArgMax* p = part + ((int64_t)s * N + n) * nchunks;
    ArgMax a = p[0];
    for (int c = 1; c < nchunks; ++c) take(a, p[c].v, p[c].i);
    want[n] = a.i;
  }
  __syncthreads();
  int cur = 0;
  int a = 0;
  while (a < L) {
    const int wt = want[cur];
    int found = -1;
    for (int x0 = 0; x0 < nn && found < 0; x0 += kWave) {
      const int x = x0 + lane;
      const bool hit = x < nn && par[x] == cur && tok[x] == wt;
      const unsigned long long m = ballot(hit);
      if (m) found = x0 + __ffsll((long long)m) - 1;
    }
    if (found < 0) break;
    if (lane == 0) {
      acc_nodes[(int64_t)s * L + a] = found;
      acc_tok[(int64_t)s * L + a] = tok[found];
    }
    cur = found;
    ++a;
  }
  for (int i = a + lane; i < L; i += kWave) {
    acc_nodes[(int64_t)s * L + i] = -1;
    acc_tok[(int64_t)s * L + i] = -1;
  }
  if (lane == 0) {
    accept_len[s] = a;
    bonus_out[s] = want[cur];
  }
}

}  // namespace

WalkPlan walk_plan(int S, int B, int64_t vocab) {
  WalkPlan p;
  const int64_t rows = (int64_t)S * (B + 1);
  const int64_t target_blocks = 2048;
  const int64_t max_chunks = std::max<int64_t>(1, vocab / 4096);
  int64_t nch = std::min<int64_t>(std::max<int64_t>(1, ceil_div(target_blocks, rows)), max_chunks);
  const int64_t len = (int64_t)align_up((size_t)ceil_div(vocab, nch), 4);
  nch = ceil_div(vocab, len);
  p.nchunks = (int)nch;
  p.chunk_len = len;
  p.ws_bytes = align_up((size_t)rows * nch * sizeof(ArgMax), 256);
  return p;
}

hipError_t launch_tree_walk(const int32_t* tree_tok, const int32_t* parent,
                            const int32_t* num_nodes, const float* target, int S, int B, int L,
                            int64_t vocab, int32_t* accept_len, int32_t* acc_nodes,
                            int32_t* acc_tok, int32_t* bonus_out, void* ws, const WalkPlan& plan,
                            hipStream_t st) {
  const int N = B + 1;
  ArgMax* part = static_cast<ArgMax*>(ws);
  const bool vec_ok = (reinterpret_cast<uintptr_t>(target) % 16 == 0) && (vocab % 4 == 0);
  const int64_t blocks = (int64_t)S * N * plan.nchunks;
  hipLaunchKernelGGL(argmax_partial, dim3((unsigned)blocks), dim3(kThreads), 0, st, target,
                     num_nodes, N, (int)vocab, plan.nchunks, plan.chunk_len, vec_ok, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(walk_kernel, dim3(S), dim3(kWave), 3 * sizeof(int) * N, st, tree_tok, parent,
                     num_nodes, part, N, L, plan.nchunks, accept_len, acc_nodes, acc_tok,
                     bonus_out);
  return hipGetLastError();
}

}  // namespace ddt
