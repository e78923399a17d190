// Greedy tree walk (DDTree page "策展 · X (Twitter)", section 運作流程 step 4: follow
// the target's decoding rule from the root, accept while its token matches a child,
// carry the first mismatch as the next bonus token).
//
// One kernel.  A workgroup takes one batch of one node's row of target logits (waves x
// 64 lanes x 32 logits: 16 waves for a row that fits one batch, 8 otherwise, down to
// 2 when the grid would leave CUs idle), loaded with 16-byte loads issued together,
// and finds its arg-max: larger value first, equal values by smaller id.  Longer rows
// are split over several workgroups, so a grid of a few hundred rows has no row left
// over for a lone second round.  The winner enters the node's 64-bit key in the
// workspace (the order-preserving image of the value above the complement of the id)
// by a returning atomic maximum; a per-row counter finds the row's last batch, which
// bumps the sequence's counter; the workgroup that completes the sequence reads the
// node keys, clears keys and counters for the next call, and walks the tree.  Only
// wave 0 of a workgroup goes past its LDS reduction: the others leave at once instead
// of holding their slots through the atomics.  Padding nodes (past num_nodes) are
// skipped.  Keys and counters pass between workgroups through device-scope atomics
// only: each atomic's result is awaited before the next is issued, so no cache-wide
// fence is needed.
#include <limits.h>

#include "ddt_internal.h"

namespace ddt {
namespace {

constexpr int kMaxWaves = 16;  // waves per workgroup
constexpr int kE = 32;         // logits per lane per batch
constexpr int kGather = 6;     // node keys per lane loaded together by the walking wave

typedef float f32x4 __attribute__((ext_vector_type(4)));

// order-preserving map of a float to uint32
__device__ __forceinline__ unsigned fkey(float v) {
  const unsigned b = __builtin_bit_cast(unsigned, v + 0.f);  // -0 -> +0: they compare equal
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// (value, id) -> key: larger value wins, then smaller id.  0 means "none".
__device__ __forceinline__ unsigned long long pack(float v, int id) {
  return ((unsigned long long)fkey(v) << 32) | (unsigned)(0xffffffffu - (unsigned)id);
}

__device__ __forceinline__ int unpack_id(unsigned long long key) {
  return (int)(0xffffffffu - (unsigned)(key & 0xffffffffull));
}

// ONE: the whole grid runs at once, so the scan is on the latency path and takes the
// batch maximum first (a short dependent chain); when workgroups stream in rounds, the
// compare-as-you-go scan keeps up with the loads better (measured).  Two workgroups
// per CU (8 waves per SIMD, at most 64 VGPRs): the row loads of one hide the other's scan.
template <bool ONE>
__global__ void __launch_bounds__(kMaxWaves * kWave) __attribute__((amdgpu_waves_per_eu(8, 8)))
tree_walk_kernel(const int32_t* __restrict__ tree_tok, const int32_t* __restrict__ parent,
                 const int32_t* __restrict__ num_nodes, const float* __restrict__ target, int N,
                 int L, int vocab, int nseg, bool vec_ok, unsigned long long* __restrict__ best,
                 unsigned* __restrict__ counters, unsigned* __restrict__ rowcnt,
                 int32_t* __restrict__ accept_len,
                 int32_t* __restrict__ acc_nodes, int32_t* __restrict__ acc_tok,
                 int32_t* __restrict__ bonus_out) {
  __shared__ unsigned long long red[kMaxWaves];
  extern __shared__ int smem[];
  const int64_t row = blockIdx.x / (unsigned)nseg;  // s * N + n
  const int seg = (int)(blockIdx.x % (unsigned)nseg);  // the row's batch this workgroup scans
  const int s = (int)(row / N);
  const int n = (int)(row % N);
  const int nn = num_nodes[s];
  if (n >= nn) return;
  const int nw = blockDim.x / kWave;
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid % kWave;
  const float* x = target + row * (int64_t)vocab;

  float bv = -INFINITY;
  int bi = INT_MAX;
  {
    const int lo = (seg * nw + wave) * kWave * kE;
    float v[kE];
#pragma unroll
    for (int b = 0; b < kE / 4; ++b) {
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
    if constexpr (ONE) {
      // the batch's maximum first, then the first element that holds it: elements are
      // visited in increasing id order, so ties go to the smaller id
      float mb = -INFINITY;
#pragma unroll
      for (int e = 0; e < kE; ++e) mb = fmaxf(mb, v[e]);
      int ib = INT_MAX;
#pragma unroll
      for (int e = kE - 1; e >= 0; --e) {
        const int i = lo + ((e / 4) * kWave + lane) * 4 + e % 4;
        if (v[e] == mb && i < vocab) ib = i;
      }
      if (ib != INT_MAX && better(mb, ib, bv, bi)) {
        bv = mb;
        bi = ib;
      }
    } else {
#pragma unroll
      for (int e = 0; e < kE; ++e) {
        const int i = lo + ((e / 4) * kWave + lane) * 4 + e % 4;
        if (i < vocab && better(v[e], i, bv, bi)) {
          bv = v[e];
          bi = i;
        }
      }
    }
  }
  wave_argmax(bv, bi);
  if (lane == 0) red[wave] = bi == INT_MAX ? 0ull : pack(bv, bi);
  __syncthreads();
  // wave 0 finishes the workgroup alone; the other waves free their slots now rather
  // than waiting out the atomics' round trips
  if (wave != 0) return;
  bool last = false;
  if (lane == 0) {
    unsigned long long k = red[0];
    for (int w = 1; w < nw; ++w) k = red[w] > k ? red[w] : k;
    // the row's key is the maximum over its segments; the counters count finished
    // segments per row and finished rows per sequence.  Each atomic's result is
    // awaited before the next one is issued, which orders them without a fence.
    const unsigned long long old = atomicMax(&best[row], k);
    asm volatile("" ::"v"((unsigned)old) : "memory");  // the maximum has been performed
    bool row_done = true;
    if (nseg > 1) {
      const unsigned pr = atomicAdd(&rowcnt[row], 1u);
      asm volatile("" ::"v"(pr) : "memory");
      row_done = pr == (unsigned)nseg - 1u;
      if (row_done) __hip_atomic_store(&rowcnt[row], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (row_done) {
      const unsigned prev = atomicAdd(&counters[s], 1u);
      last = prev == (unsigned)nn - 1u;
    }
  }
  if (!__builtin_amdgcn_readfirstlane(last)) return;

  // the sequence's last workgroup (its wave 0): collect the target's token at every
  // node, walk
  int* want = smem;         // [N] target's greedy token at each node
  int* tok = smem + N;      // [N]
  int* par = smem + 2 * N;  // [N]
  // kGather nodes per lane have their loads in flight together: a load at a time made
  // this gather a chain of round trips (C3, B = 512: 6 us for 513 nodes)
  for (int i0 = 0; i0 < nn; i0 += kGather * kWave) {
    unsigned long long k[kGather];
    int t[kGather], p[kGather];
#pragma unroll
    for (int j = 0; j < kGather; ++j) {
      const int i = i0 + j * kWave + lane;
      if (i < nn) {
        k[j] = __hip_atomic_load(best + (int64_t)s * N + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        t[j] = tree_tok[(int64_t)s * N + i];
        p[j] = parent[(int64_t)s * N + i];
      }
    }
#pragma unroll
    for (int j = 0; j < kGather; ++j) {
      const int i = i0 + j * kWave + lane;
      if (i < nn) {
        // cleared for the next call, whose maxima start from 0
        __hip_atomic_store(best + (int64_t)s * N + i, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        want[i] = unpack_id(k[j]);
        tok[i] = t[j];
        par[i] = p[j];
      }
    }
  }
  if (lane == 0) __hip_atomic_store(&counters[s], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  // the wave's LDS writes above before its reads below
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  int cur = 0;
  int a = 0;
  while (a < L) {
    const int wt = want[cur];
    int found = -1;
    for (int x0 = 0; x0 < nn && found < 0; x0 += kWave) {
      const int xi = x0 + lane;
      const bool hit = xi < nn && par[xi] == cur && tok[xi] == wt;
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
  // A row that fits one batch of 16 waves is one workgroup; longer rows are split into
  // batches of 8 waves (8 * 64 * kE logits), one workgroup each, so no row makes a lone
  // extra round of the grid (8-wave batches measured 5-6% faster than 16 on C2 and C3).
  // A grid of fewer workgroups than CUs splits its rows further, down to 2-wave
  // batches, so that more CUs stream the logits (C1: 33 rows become 264 workgroups;
  // 1% more rounds/s than 4-wave batches and 2.5% more than 16, paired runs).
  const int64_t per_wave = (int64_t)kWave * kE;
  int w = vocab <= kMaxWaves * per_wave ? kMaxWaves : kMaxWaves / 2;
  while (w > 2 && rows * ceil_div(vocab, (int64_t)w * per_wave) < cu_count()) w /= 2;
  p.waves = (int)std::min<int64_t>(w, ceil_div(vocab, per_wave));
  p.nbatch = (int)ceil_div(vocab, (int64_t)p.waves * per_wave);
  // the whole grid at once on the CUs: the scan is on the latency path
  p.short_scan = rows * p.nbatch <= cu_count();
  p.counter_bytes = align_up((size_t)S * sizeof(unsigned), 256);
  p.rowcnt_bytes = align_up((size_t)rows * sizeof(unsigned), 256);
  p.ws_bytes = p.counter_bytes + p.rowcnt_bytes + align_up((size_t)rows * sizeof(unsigned long long), 256);
  return p;
}

hipError_t launch_tree_walk(const int32_t* tree_tok, const int32_t* parent,
                            const int32_t* num_nodes, const float* target, int S, int B, int L,
                            int64_t vocab, int32_t* accept_len, int32_t* acc_nodes,
                            int32_t* acc_tok, int32_t* bonus_out, void* ws, const WalkPlan& plan,
                            hipStream_t st) {
  const int N = B + 1;
  unsigned* counters = static_cast<unsigned*>(ws);
  unsigned* rowcnt = reinterpret_cast<unsigned*>(static_cast<char*>(ws) + plan.counter_bytes);
  unsigned long long* best = reinterpret_cast<unsigned long long*>(
      static_cast<char*>(ws) + plan.counter_bytes + plan.rowcnt_bytes);
  const bool vec_ok = (reinterpret_cast<uintptr_t>(target) % 16 == 0) && (vocab % 4 == 0);
  const dim3 grid((unsigned)((int64_t)S * N * plan.nbatch)), block(plan.waves * kWave);
  const size_t smem = 3 * sizeof(int) * N;
  if (plan.short_scan)
    hipLaunchKernelGGL(tree_walk_kernel<true>, grid, block, smem, st, tree_tok, parent, num_nodes,
                       target, N, L, (int)vocab, plan.nbatch, vec_ok, best, counters, rowcnt,
                       accept_len, acc_nodes, acc_tok, bonus_out);
  else
    hipLaunchKernelGGL(tree_walk_kernel<false>, grid, block, smem, st, tree_tok, parent, num_nodes,
                       target, N, L, (int)vocab, plan.nbatch, vec_ok, best, counters, rowcnt,
                       accept_len, acc_nodes, acc_tok, bonus_out);
  return hipGetLastError();
}

}  // namespace ddt
