// Greedy tree walk (DDTree page "策展 · X (Twitter)", section 運作流程 step 4: follow
// the target's decoding rule from the root, accept while its token matches a child,
// carry the first mismatch as the next bonus token).
//
// Three strategies with identical outputs.  The row scan below finds every node's
// arg-max and then walks; the path walk (path_walk.hip) follows the walk and reads only
// the rows of the nodes it visits; the hybrid runs the path walk for a few steps and
// hands a walk that goes on to the subtree scan (below), which reads only the rows of
// the reached node's subtree.  walk_mode (below) picks one per call.
//
// The row scan.  A workgroup takes one batch of one node's row of target logits (waves x
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
// skipped.  Keys and counters pass between workgroups through agent-scope atomics
// only, which gfx950 performs at the device's point of coherence, and each atomic's
// result is awaited before the next is issued: a workgroup's maximum is performed
// before its counter update is issued.  Under the HIP memory model these relaxed
// atomics on different addresses do not by themselves order the maximum before the
// last workgroup's reads; making the counter updates release/acquire operations does,
// but compiles to an L2 writeback and invalidate per workgroup and measured C2 at
// 2080 rounds/s against 5950 (C1 -8%), so the ordering rests on the hardware's.
#include <limits.h>

#include <atomic>
#include <mutex>

#include "ddt_internal.h"

namespace ddt {
namespace {

// Workspace of the allocation-free walk entry point: one copy per GPU, zero at module
// load, and every walk leaves what it used zero again.
constexpr size_t kWalkScratchBytes = size_t(1) << 20;
static __device__ __align__(256) unsigned char scratch[kWalkScratchBytes];

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

// The sequence's last workgroup (its wave 0): collect the target's token at every node
// from the keys, clear keys and counter for the next call, and walk from node cur with
// a tokens already accepted (the root and 0, or where the path walk handed over: nodes
// outside that subtree have no key, and the walk never reaches them).
__device__ __forceinline__ void finish_walk(int s, int N, int L, int nn, int cur, int a,
                                            const int32_t* __restrict__ tree_tok,
                                            const int32_t* __restrict__ parent,
                                            unsigned long long* __restrict__ best,
                                            unsigned* __restrict__ counters, int* smem,
                                            int32_t* __restrict__ accept_len,
                                            int32_t* __restrict__ acc_nodes,
                                            int32_t* __restrict__ acc_tok,
                                            int32_t* __restrict__ bonus_out) {
  const int lane = threadIdx.x % kWave;
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

// ONE: the whole grid runs at once, so the scan is on the latency path and takes the
// batch maximum first (a short dependent chain); when workgroups stream in rounds, the
// compare-as-you-go scan keeps up with the loads better (measured).  Two workgroups
// per CU (8 waves per SIMD, at most 64 VGPRs): the row loads of one hide the other's scan.
// SAMPLE: temperature sampling by the Gumbel-max rule.  The score of token v at node n
// is fl(fl(x_v * inv_t) + g[s, depth(n), v]), an fp32 multiply and an fp32 add each
// rounded on its own (sample_score), so the arg-max is decided in the same arithmetic
// as the definition; the noise row is shared by a depth's nodes and read through the
// caches.  It holds two rows' loads at once, so it runs four waves per SIMD.
template <bool ONE, bool SAMPLE>
__global__ void __launch_bounds__(kMaxWaves * kWave) __attribute__((amdgpu_waves_per_eu(SAMPLE ? 4 : 8, 8)))
tree_walk_kernel(const int32_t* __restrict__ tree_tok, const int32_t* __restrict__ parent,
                 const int32_t* __restrict__ num_nodes, const float* __restrict__ target,
                 const int32_t* __restrict__ depth, const float* __restrict__ gumbel, float inv_t,
                 int N, int L, int vocab, int nseg, bool vec_ok, unsigned long long* __restrict__ best,
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
  const float* gn = nullptr;
  if constexpr (SAMPLE) gn = gumbel + ((int64_t)s * (L + 1) + depth[row]) * vocab;

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
        if constexpr (SAMPLE) {
          const f32x4 g = *reinterpret_cast<const f32x4*>(gn + base);
#pragma unroll
          for (int q = 0; q < 4; ++q) v[4 * b + q] = sample_score(t[q], inv_t, g[q]);
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) v[4 * b + q] = t[q];
        }
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float e = -INFINITY;
          if (base + q < vocab) {
            e = x[base + q];
            if constexpr (SAMPLE) e = sample_score(e, inv_t, gn[base + q]);
          }
          v[4 * b + q] = e;
        }
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
    // segments per row and finished rows per sequence.  Each increment is a release at
    // agent scope, publishing this workgroup's maximum; the workgroup that finishes a
    // row takes an acquire fence before passing the row on, and the sequence's last
    // one another before it reads best[], so it sees every maximum.  (Acquire-release
    // increments in every workgroup made C1's round 8.6% longer than relaxed ones, this
    // form 6%: each acquire invalidates the XCD's L2 under the other workgroups' logit
    // reads, and each release writes it back.)
    atomicMax(&best[row], k);
    bool row_done = true;
    if (nseg > 1) {
      const unsigned pr = __hip_atomic_fetch_add(&rowcnt[row], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
      row_done = pr == (unsigned)nseg - 1u;
      if (row_done) {
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        __hip_atomic_store(&rowcnt[row], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    if (row_done) {
      const unsigned prev = __hip_atomic_fetch_add(&counters[s], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
      last = prev == (unsigned)nn - 1u;
    }
  }
  if (!__builtin_amdgcn_readfirstlane(last)) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");  // every row's maximum, before best[] is read

  // the sequence's last workgroup (its wave 0): collect the target's token at every
  // node, walk.  (finish_walk above is the same code, for the subtree scan; written out
  // here because through that function the compiler kept a pointer live across the
  // scan and spilled it in the maximum-first variant.)
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

// The hybrid's scan: the rows of the subtree the path walk handed over (state[s] =
// {node, accepted, count}, the rows in list[s, 0 .. count)), a fixed grid of gs
// workgroups per sequence looping over the (row, batch) items, so that a sequence the
// path walk finished (count 0) costs its workgroups one load each.  An item is scanned
// as in tree_walk_kernel (compare-as-you-go) and counted the same way; the two
// reduction buffers alternate between items, so one barrier per item keeps a wave from
// overwriting what wave 0 still reads.  The workgroup that completes the sequence has
// no items left (its last item completed the count), clears the list and the state,
// and walks on from the hand-off node.
template <bool SAMPLE>
__global__ void __launch_bounds__(kMaxWaves * kWave) __attribute__((amdgpu_waves_per_eu(SAMPLE ? 4 : 8, 8)))
subtree_scan_kernel(const int32_t* __restrict__ tree_tok, const int32_t* __restrict__ parent,
                    const int32_t* __restrict__ num_nodes, const float* __restrict__ target,
                    const int32_t* __restrict__ depth, const float* __restrict__ gumbel,
                    float inv_t, int N, int L, int vocab, int nseg, int gs, bool vec_ok,
                    unsigned long long* __restrict__ best, unsigned* __restrict__ counters,
                    unsigned* __restrict__ rowcnt, unsigned* __restrict__ state,
                    int32_t* __restrict__ list, int32_t* __restrict__ accept_len,
                    int32_t* __restrict__ acc_nodes, int32_t* __restrict__ acc_tok,
                    int32_t* __restrict__ bonus_out) {
  __shared__ unsigned long long red[2][kMaxWaves];
  extern __shared__ int smem[];
  const int s = (int)(blockIdx.x / (unsigned)gs);
  const int g = (int)(blockIdx.x % (unsigned)gs);
  // the first item's list entry is read together with the state, not after it (g < gs
  // <= N * nseg keeps it inside the sequence's list); each later one a step ahead
  int next = list[(int64_t)s * N + g / nseg];
  const int nn = min(max(num_nodes[s], 1), N);
  // (clamped: a workspace that was not zero on entry gives wrong outputs, not stray reads)
  const int count = __builtin_amdgcn_readfirstlane(min((int)state[4 * s + 2], nn));
  const int items = count * nseg;
  if (g >= items) return;  // also every workgroup of a sequence the path walk finished
  const int nw = blockDim.x / kWave;
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid % kWave;
  int buf = 0;
  for (int j = g; j < items; j += gs) {
    const int seg = j % nseg;
    const int n = __builtin_amdgcn_readfirstlane(min(max(next, 0), nn - 1));
    if (j + gs < items) next = list[(int64_t)s * N + (j + gs) / nseg];
    const int64_t row = (int64_t)s * N + n;
    const float* x = target + row * (int64_t)vocab;
    const float* gn = nullptr;
    if constexpr (SAMPLE) gn = gumbel + ((int64_t)s * (L + 1) + depth[row]) * vocab;
    // the batch's loads all issued before any compare: one memory latency per item
    float bv = -INFINITY;
    int bi = INT_MAX;
    const int lo = (seg * nw + wave) * kWave * kE;
    float v[kE];
#pragma unroll
    for (int b = 0; b < kE / 4; ++b) {
      const int base = lo + (b * kWave + lane) * 4;
      if (vec_ok && base + 3 < vocab) {
        const f32x4 t = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(x + base));
        if constexpr (SAMPLE) {
          const f32x4 gv = *reinterpret_cast<const f32x4*>(gn + base);
#pragma unroll
          for (int q = 0; q < 4; ++q) v[4 * b + q] = sample_score(t[q], inv_t, gv[q]);
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) v[4 * b + q] = t[q];
        }
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float e = -INFINITY;
          if (base + q < vocab) {
            e = x[base + q];
            if constexpr (SAMPLE) e = sample_score(e, inv_t, gn[base + q]);
          }
          v[4 * b + q] = e;
        }
      }
    }
#pragma unroll
    for (int e = 0; e < kE; ++e) {
      const int i = lo + ((e / 4) * kWave + lane) * 4 + e % 4;
      if (i < vocab && better(v[e], i, bv, bi)) {
        bv = v[e];
        bi = i;
      }
    }
    wave_argmax(bv, bi);
    if (lane == 0) red[buf][wave] = bi == INT_MAX ? 0ull : pack(bv, bi);
    __syncthreads();
    if (wave == 0) {
      bool last = false;
      if (lane == 0) {
        unsigned long long key = red[buf][0];
        for (int w = 1; w < nw; ++w) key = red[buf][w] > key ? red[buf][w] : key;
        // as in tree_walk_kernel: release increments, acquire fences where read
        atomicMax(&best[row], key);
        bool row_done = true;
        if (nseg > 1) {
          const unsigned pr = __hip_atomic_fetch_add(&rowcnt[row], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
          row_done = pr == (unsigned)nseg - 1u;
          if (row_done) {
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            __hip_atomic_store(&rowcnt[row], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
        }
        if (row_done) {
          const unsigned prev = __hip_atomic_fetch_add(&counters[s], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
          last = prev == (unsigned)count - 1u;
        }
      }
      if (__builtin_amdgcn_readfirstlane(last)) {
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");  // every row's maximum
        // readfirstlane waits for the loads, so they complete before the stores below
        const int cur = __builtin_amdgcn_readfirstlane(min(max((int)state[4 * s], 0), nn - 1));
        const int a = __builtin_amdgcn_readfirstlane(min(max((int)state[4 * s + 1], 0), L));
        for (int i = lane; i < count; i += kWave) list[(int64_t)s * N + i] = 0;
        if (lane < 3) state[4 * s + lane] = 0u;
        finish_walk(s, N, L, nn, cur, a, tree_tok, parent, best, counters, smem, accept_len,
                    acc_nodes, acc_tok, bonus_out);
        return;
      }
    }
    buf ^= 1;
  }
}

__global__ void __launch_bounds__(256) zero_fill(uint4* __restrict__ p, size_t n16) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0, 0, 0, 0);
}

}  // namespace

size_t walk_scratch_bytes() { return kWalkScratchBytes; }

hipError_t walk_scratch(void** ptr, hipStream_t st) {
  static std::mutex mu;
  static void* addr[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(mu);
  if (!addr[dev]) {
    // the array's device address on this device; the host-side name is not one
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    // cleared once on this device, on the caller's stream, before its first walk (a
    // fill kernel, not a memset, so that a call under stream capture records it too)
    hipLaunchKernelGGL(zero_fill, dim3(256), dim3(256), 0, st, static_cast<uint4*>(p),
                       kWalkScratchBytes / sizeof(uint4));
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

// the caller's choice (ddt_tree_walk_strategy); 0 lets the planner decide
static std::atomic<int> g_walk_strategy{0};

int set_walk_strategy(int mode) {
  if (mode < 0 || mode > 3) return -1;
  return g_walk_strategy.exchange(mode);
}

// Which walk.  The row scan reads all S * N rows at once: about 6 us plus the logits at
// 6 TB/s.  The path walk reads one row per accepted token plus one, in sequence, each on
// one CU: about 2 us plus, per step, 1 us and a row at 90 GB/s (figures measured on
// MI355X).  Its time grows with the accepted length, which is not known in advance.
//   * Path walk when it wins even with half the block accepted (L / 2 tokens, a middle
//     value for the mean acceptance lengths the DDTree page reports, 實驗結果與權衡:
//     about 11 of 16 at best): 32 sequences of 65 nodes over 128256 logits, where the
//     scan reads 1 GB; also the tiny rows of 64 logits.
//   * Row scan when the scan is short anyway (under 15 us: one sequence of up to about
//     100 nodes over 128256 logits, or a 32000-entry vocabulary).
//   * Otherwise the hybrid: the path walk for up to kHybridSteps accepted tokens, then
//     the scan over the subtree of the node it reached.  A walk that ends early (the
//     common case) costs a few path steps plus a scan launch whose workgroups find
//     nothing to do; a long one costs those steps plus a scan of the remaining
//     subtree, which is smaller than the tree.
constexpr int kHybridSteps = 3;

WalkMode walk_mode(int S, int B, int L, int64_t vocab, int* steps) {
  *steps = kHybridSteps;
  switch (g_walk_strategy.load()) {
    case 1: return WalkMode::kScan;
    case 2: return WalkMode::kPath;
    case 3: return WalkMode::kHybrid;
    default: break;
  }
  const double t_step = 1e-6 + (double)vocab * 4.0 / 9e10;
  const double t_path = 2e-6 + (L / 2 + 1) * t_step;
  const double t_scan = 6e-6 + (double)S * (B + 1) * (double)vocab * 4.0 / 6e12;
  if (t_path < t_scan) return WalkMode::kPath;
  if (t_scan < 15e-6) return WalkMode::kScan;
  return WalkMode::kHybrid;
}

WalkPlan walk_plan(int S, int B, int64_t vocab) {
  WalkPlan p;
  const int64_t rows = (int64_t)S * (B + 1);
  // A row that fits one batch of 16 waves is one workgroup; longer rows are split into
  // batches of 8 waves (8 * 64 * kE logits), one workgroup each, so no row makes a lone
  // extra round of the grid (8-wave batches measured 5-6% faster than 16 on C2 and C3).
  // A grid of fewer workgroups than CUs splits a 16-wave row into 8-wave batches, and
  // no further: every batch publishes its maximum with an agent-scope release (an L2
  // writeback), so a few wide batches beat many narrow ones that reach more CUs
  // (paired runs against splitting down to 2-wave batches: C1, 33 rows in 66 instead
  // of 264 workgroups, 46.8 -> 45.5 us per round; C3 B = 16 63.5 -> 61.4 us).
  const int64_t per_wave = (int64_t)kWave * kE;
  int w = vocab <= kMaxWaves * per_wave ? kMaxWaves : kMaxWaves / 2;
  while (w > 8 && rows * ceil_div(vocab, (int64_t)w * per_wave) < cu_count()) w /= 2;
  p.waves = (int)std::min<int64_t>(w, ceil_div(vocab, per_wave));
  p.nbatch = (int)ceil_div(vocab, (int64_t)p.waves * per_wave);
  // the whole grid at once on the CUs: the scan is on the latency path
  p.short_scan = rows * p.nbatch <= cu_count();
  p.counter_bytes = align_up((size_t)S * sizeof(unsigned), 256);
  p.rowcnt_bytes = align_up((size_t)rows * sizeof(unsigned), 256);
  p.key_bytes = align_up((size_t)rows * sizeof(unsigned long long), 256);
  p.state_bytes = align_up((size_t)S * 4 * sizeof(unsigned), 256);
  p.ws_bytes = p.counter_bytes + p.rowcnt_bytes + p.key_bytes + p.state_bytes +
               align_up((size_t)rows * sizeof(int32_t), 256);
  return p;
}

hipError_t launch_tree_walk(const int32_t* tree_tok, const int32_t* parent,
                            const int32_t* num_nodes, const float* target, int S, int B, int L,
                            int64_t vocab, int32_t* accept_len, int32_t* acc_nodes,
                            int32_t* acc_tok, int32_t* bonus_out, void* ws, const WalkPlan& plan,
                            hipStream_t st, const int32_t* depth, const float* gumbel,
                            float inv_t) {
  const int N = B + 1;
  char* w = static_cast<char*>(ws);
  unsigned* counters = reinterpret_cast<unsigned*>(w);
  unsigned* rowcnt = reinterpret_cast<unsigned*>(w + plan.counter_bytes);
  unsigned long long* best = reinterpret_cast<unsigned long long*>(w + plan.counter_bytes + plan.rowcnt_bytes);
  unsigned* state = reinterpret_cast<unsigned*>(w + plan.counter_bytes + plan.rowcnt_bytes + plan.key_bytes);
  int32_t* list = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(state) + plan.state_bytes);
  const bool vec_ok = (reinterpret_cast<uintptr_t>(target) % 16 == 0) && (vocab % 4 == 0) &&
                      (reinterpret_cast<uintptr_t>(gumbel) % 16 == 0);
  int steps = 0;
  const WalkMode mode = walk_mode(S, B, L, vocab, &steps);
  if (mode == WalkMode::kPath)
    return launch_path_walk(tree_tok, parent, num_nodes, target, S, B, L, vocab, accept_len,
                            acc_nodes, acc_tok, bonus_out, st, depth, gumbel, inv_t, -1, nullptr,
                            nullptr);
  const size_t smem = 3 * sizeof(int) * N;
  if (mode == WalkMode::kHybrid) {
    const hipError_t e = launch_path_walk(tree_tok, parent, num_nodes, target, S, B, L, vocab,
                                          accept_len, acc_nodes, acc_tok, bonus_out, st, depth,
                                          gumbel, inv_t, steps, state, list);
    if (e != hipSuccess) return e;
    // about two workgroups per CU over all sequences, at most one per item
    const int gs = (int)std::max<int64_t>(
        1, std::min<int64_t>((int64_t)N * plan.nbatch, ceil_div(2 * (int64_t)cu_count(), S)));
    const dim3 sgrid((unsigned)((int64_t)S * gs)), sblock(plan.waves * kWave);
    if (gumbel)
      hipLaunchKernelGGL((subtree_scan_kernel<true>), sgrid, sblock, smem, st, tree_tok, parent,
                         num_nodes, target, depth, gumbel, inv_t, N, L, (int)vocab, plan.nbatch, gs,
                         vec_ok, best, counters, rowcnt, state, list, accept_len, acc_nodes, acc_tok,
                         bonus_out);
    else
      hipLaunchKernelGGL((subtree_scan_kernel<false>), sgrid, sblock, smem, st, tree_tok, parent,
                         num_nodes, target, depth, gumbel, inv_t, N, L, (int)vocab, plan.nbatch, gs,
                         vec_ok, best, counters, rowcnt, state, list, accept_len, acc_nodes, acc_tok,
                         bonus_out);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)((int64_t)S * N * plan.nbatch)), block(plan.waves * kWave);
#define DDT_WALK(ONE, SAMPLE)                                                                  \
  hipLaunchKernelGGL((tree_walk_kernel<ONE, SAMPLE>), grid, block, smem, st, tree_tok, parent, \
                     num_nodes, target, depth, gumbel, inv_t, N, L, (int)vocab, plan.nbatch,     \
                     vec_ok, best, counters, rowcnt, accept_len, acc_nodes, acc_tok, bonus_out)
  if (gumbel) {
    if (plan.short_scan)
      DDT_WALK(true, true);
    else
      DDT_WALK(false, true);
  } else if (plan.short_scan) {
    DDT_WALK(true, false);
  } else {
    DDT_WALK(false, false);
  }
#undef DDT_WALK
  return hipGetLastError();
}

}  // namespace ddt
