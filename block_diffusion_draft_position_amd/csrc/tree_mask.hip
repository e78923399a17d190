// Compile a draft tree into its ancestor-only attention mask and position ids
// (DDTree page "策展 · X (Twitter)": section 核心創新 for the ancestor-only mask,
// 運作流程 step 3 for compiling the tree into the target's inputs).
//
// A sequence's N * W (node, word) items are cut into slices of kThreads * kPerThread,
// one workgroup each; every workgroup stages the sequence's parent array in LDS and
// forms its slice of the rows with mask::rows (tree_mask_device.h).  A deep tree's
// items each walk up to L parent links, so the slices spread that over CUs (C3,
// B = 512: 8721 items of a single sequence).
#include "tree_mask_device.h"

namespace ddt {
namespace {

constexpr int kThreads = 256;
constexpr int kPerThread = 1;  // items per thread in a slice (4: -0.75% rounds/s at C3, B = 512)

__global__ void __launch_bounds__(kThreads)
tree_mask_kernel(const int32_t* __restrict__ parent, const int32_t* __restrict__ depth,
                 const int32_t* __restrict__ num_nodes, Prefix pre,
                 int N, int W, int slices, uint32_t* __restrict__ mask,
                 int32_t* __restrict__ pos_ids) {
  extern __shared__ int par[];
  const int s = blockIdx.x / slices;
  const int slice = blockIdx.x % slices;
  const int nn = num_nodes[s];
  const int32_t* pg = parent + (int64_t)s * N;
  for (int i = threadIdx.x; i < N; i += kThreads) par[i] = pg[i];
  __syncthreads();
  const int per = kThreads * kPerThread;
  mask::rows(par, nn, N, W, mask + (int64_t)s * N * W, threadIdx.x, kThreads, slice * per,
             min(N * W, (slice + 1) * per));
  if (pos_ids && slice == 0) {
    const int32_t P = (int32_t)pre.length(s);
    for (int n = threadIdx.x; n < N; n += kThreads)
      pos_ids[(int64_t)s * N + n] = (n < nn) ? P + depth[(int64_t)s * N + n] : -1;
  }
}

}  // namespace

hipError_t launch_tree_mask(const int32_t* parent, const int32_t* depth, const int32_t* num_nodes,
                            Prefix pre, int S, int B, uint32_t* mask,
                            int32_t* pos_ids, hipStream_t st) {
  const int N = B + 1;
  const int W = (N + 31) / 32;
  const int slices = (int)ceil_div(N * W, kThreads * kPerThread);
  hipLaunchKernelGGL(tree_mask_kernel, dim3(S * slices), dim3(kThreads), sizeof(int) * N, st, parent,
                     depth, num_nodes, pre, N, W, slices, mask, pre.cu ? pos_ids : nullptr);
  return hipGetLastError();
}

}  // namespace ddt
