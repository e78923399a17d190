// Device side of the ancestor-mask compilation, shared by the mask kernel and the
// fused draft-tree kernel.  See tree_mask.hip for the method.
#pragma once

#include "ddt_internal.h"

namespace ddt {
namespace mask {

// Mask rows [N, W] of one sequence from its parent array in LDS (canonical order,
// parents before children): items it0 .. it1-1 of the N * W (node, word) items, by
// threads tid = 0 .. nthreads-1 of the caller.  A thread owns one item at a time and
// walks parent links from the node: parents have smaller indices, so the walk passes
// the word's 32 node ids in one stretch and stops below it.  Items are numbered
// row-major, so the stores of a wave are contiguous.
__device__ inline void rows(const int* __restrict__ par, int nn, int N, int W,
                            uint32_t* __restrict__ mrow, int tid, int nthreads, int it0,
                            int it1) {
  for (int it = it0 + tid; it < it1; it += nthreads) {
    const int n = it / W;
    const int w = it % W;
    uint32_t acc = 0u;
    if (n < nn && (n >> 5) >= w) {
      int x = n;
      int guard = N;  // a malformed parent array cannot loop forever
      while (x >= (w << 5) && guard-- > 0) {
        if ((x >> 5) == w) acc |= 1u << (x & 31);
        const int p = par[x];
        x = (p < x) ? p : -1;
      }
    }
    mrow[it] = acc;
  }
}

}  // namespace mask
}  // namespace ddt
