// KV commit between verification rounds (DDTree page "策展 · X (Twitter)", section
// 運作流程: a round starts from a bonus token not yet run through the target, scores
// the tree in one target forward, and carries the walk's first mismatch into the next
// round as its bonus).  After the walk, the root and the accepted nodes have been run
// forward, each attending to exactly the prefix and its ancestors, which is their
// causal context in the continued sequence; their tree K/V rows, root first, are
// appended to the sequence's cache region and its length advances by a + 1.
//
// One workgroup per sequence: it reads the sequence's length, accept length and
// accepted node indices, copies the a + 1 rows of K and of V in 16-byte pieces (a row
// is Hkv * D elements, a multiple of 16 bytes for every supported D and dtype), then
// one thread writes the new length.  No other workgroup touches the sequence, so the
// length is read before any write without a race.
#include "ddt_internal.h"

namespace ddt {
namespace {

constexpr int kThreads = 256;

__global__ void __launch_bounds__(kThreads)
commit_kv_kernel(uint4* __restrict__ k_cache, uint4* __restrict__ v_cache,
                 const int64_t* __restrict__ cu_prefix, int64_t* __restrict__ prefix_len,
                 const uint4* __restrict__ k_tree, const uint4* __restrict__ v_tree,
                 const int32_t* __restrict__ acc_nodes, const int32_t* __restrict__ accept_len,
                 int N, int L, int row16, int32_t* __restrict__ appended) {
  __shared__ int rows[DDT_MAX_L + 1];  // tree rows to append: the root, then the path
  __shared__ int ok_s;
  const int s = blockIdx.x;
  const int64_t start = cu_prefix[s];
  const int64_t cap = cu_prefix[s + 1] - start;
  const int64_t P = prefix_len[s];
  const int a = accept_len[s];
  if (threadIdx.x == 0) ok_s = 1;
  __syncthreads();
  const bool a_ok = a >= 0 && a <= L;
  if (a_ok) {
    for (int j = threadIdx.x; j <= a; j += kThreads) {
      const int node = j == 0 ? 0 : acc_nodes[(int64_t)s * L + j - 1];
      rows[j] = node;
      if (node < 0 || node >= N) ok_s = 0;
    }
  }
  __syncthreads();
  const bool ok = a_ok && ok_s && P >= 0 && P + a + 1 <= cap;
  if (ok) {
    const int total = (a + 1) * row16;
    for (int i = threadIdx.x; i < total; i += kThreads) {
      const int j = i / row16, c = i % row16;
      const int64_t src = ((int64_t)s * N + rows[j]) * row16 + c;
      const int64_t dst = (start + P + j) * row16 + c;
      k_cache[dst] = k_tree[src];
      v_cache[dst] = v_tree[src];
    }
  }
  __syncthreads();  // every thread has read prefix_len[s] above
  if (threadIdx.x == 0) {
    if (ok) prefix_len[s] = P + a + 1;
    if (appended) appended[s] = ok ? a + 1 : -1;
  }
}

}  // namespace

hipError_t launch_commit_kv(void* k_cache, void* v_cache, const int64_t* cu_prefix,
                            int64_t* prefix_len, const void* k_tree, const void* v_tree,
                            const int32_t* acc_nodes, const int32_t* accept_len, int S, int N,
                            int L, int64_t row_bytes, int32_t* appended, hipStream_t st) {
  hipLaunchKernelGGL(commit_kv_kernel, dim3(S), dim3(kThreads), 0, st, static_cast<uint4*>(k_cache),
                     static_cast<uint4*>(v_cache), cu_prefix, prefix_len,
                     static_cast<const uint4*>(k_tree), static_cast<const uint4*>(v_tree), acc_nodes,
                     accept_len, N, L, (int)(row_bytes / 16), appended);
  return hipGetLastError();
}

}  // namespace ddt
