// Compile a draft tree into its ancestor-only attention mask and position ids
// (DDTree page "策展 · X (Twitter)": section 核心創新 for the ancestor-only mask,
// 運作流程 step 3 for compiling the tree into the target's inputs).
//
// One thread per (sequence, node).  The thread zeroes its mask row, then walks
// parent links to the root, OR-ing each ancestor's bit into the current word and
// storing a word whenever the walk crosses into a lower word (parents have smaller
// indices than their children, so the walk visits words in descending order).
#include "ddt_internal.h"

namespace ddt {
namespace {

__global__ void __launch_bounds__(256)
tree_mask_kernel(const int32_t* __restrict__ parent, const int32_t* __restrict__ depth,
                 const int32_t* __restrict__ num_nodes, const int64_t* __restrict__ cu_prefix,
                 int S, int N, int W, uint32_t* __restrict__ mask, int32_t* __restrict__ pos_ids) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)S * N) return;
  const int s = (int)(idx / N);
  const int n = (int)(idx % N);
  const int nn = num_nodes[s];
  const int32_t* par = parent + (int64_t)s * N;
  uint32_t* row = mask + idx * W;
  for (int w = 0; w < W; ++w) row[w] = 0u;
  if (n < nn) {
    int x = n;
    int cw = x >> 5;
    uint32_t acc = 0u;
    int guard = N;  // a malformed parent array cannot loop forever
    while (x >= 0 && guard-- > 0) {
      const int xw = x >> 5;
      if (xw != cw) {
        row[cw] = acc;
        acc = 0u;
        cw = xw;
      }
      acc |= 1u << (x & 31);
      const int p = par[x];
      x = (p < x) ? p : -1;
    }
    row[cw] = acc;
  }
  if (pos_ids) {
    const int32_t d = depth[idx];
    pos_ids[idx] = (n < nn) ? (int32_t)(cu_prefix[s + 1] - cu_prefix[s]) + d : -1;
  }
}

}  // namespace

hipError_t launch_tree_mask(const int32_t* parent, const int32_t* depth, const int32_t* num_nodes,
                            const int64_t* cu_prefix, int S, int B, uint32_t* mask,
                            int32_t* pos_ids, hipStream_t st) {
  const int N = B + 1;
  const int W = (N + 31) / 32;
  const int64_t total = (int64_t)S * N;
  hipLaunchKernelGGL(tree_mask_kernel, dim3((unsigned)ceil_div(total, 256)), dim3(256), 0, st,
                     parent, depth, num_nodes, cu_prefix, S, N, W, mask,
                     cu_prefix ? pos_ids : nullptr);
  return hipGetLastError();
}

}  // namespace ddt
