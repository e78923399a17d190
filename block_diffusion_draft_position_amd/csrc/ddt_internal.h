// Internal declarations shared by the HIP sources of libddt (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ddt.h"

namespace ddt {

constexpr int kWave = 64;

// ---------------------------------------------------------------- device helpers
// Total order used for top-K and argmax: larger value first, equal values by
// smaller id.  Inputs are finite.
__device__ __forceinline__ bool better(float av, int ai, float bv, int bi) {
  return av > bv || (av == bv && ai < bi);
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ unsigned long long ballot(bool p) { return __ballot(p); }

template <typename T>
__device__ __forceinline__ T readlane(T v, int lane) {
  static_assert(sizeof(T) == 4, "32-bit only");
  return __builtin_bit_cast(T, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

__device__ __forceinline__ double readlane_f64(double v, int lane) {
  const long long b = __builtin_bit_cast(long long, v);
  const int lo = __builtin_amdgcn_readlane((int)(b & 0xffffffff), lane);
  const int hi = __builtin_amdgcn_readlane((int)(b >> 32), lane);
  return __builtin_bit_cast(double, ((long long)hi << 32) | (unsigned int)lo);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// ---------------------------------------------------------------- device properties
int cu_count();  // compute units of the current device (cached per device)

// ---------------------------------------------------------------- launchers
// Each returns hipSuccess or the launch error.  Arguments are validated by the
// C entry points before these are called.

// top-K
struct TopkPlan {
  int nchunks;
  int64_t chunk_len;
  size_t ws_bytes;
};
TopkPlan topk_plan(int64_t rows, int64_t vocab, int k);
hipError_t launch_topk(const float* logits, int64_t rows, int64_t vocab, int64_t stride, int k,
                       int32_t* tok, float* logq, void* ws, const TopkPlan& plan,
                       hipStream_t st);

// tree build
hipError_t launch_build_tree(const int32_t* tok, const float* logq, const int32_t* bonus, int S,
                             int L, int K, int B, int32_t* tree_tok, int32_t* parent,
                             int32_t* depth, float* node_logq, int32_t* num_nodes, hipStream_t st);

// mask
hipError_t launch_tree_mask(const int32_t* parent, const int32_t* depth, const int32_t* num_nodes,
                            const int64_t* cu_prefix, int S, int B, uint32_t* mask,
                            int32_t* pos_ids, hipStream_t st);

// attention
struct AttnPlan {
  int dtype, D, G, R;        // R = G * N query rows per (sequence, KV head)
  int waves;                 // waves per workgroup, 32 rows each
  int row_groups;            // workgroups along the rows
  int rows_pad;              // row_groups * waves * 32
  int nsplit;                // prefix splits (+1 tree split follows)
  int64_t chunk;             // prefix keys per split (multiple of 64)
  size_t ws_bytes;
};
AttnPlan attn_plan(int S, int B, int Hq, int Hkv, int D, int dtype, int64_t max_prefix);
hipError_t launch_tree_attention(const void* q, const void* kc, const void* vc,
                                 const int64_t* cu_prefix, const void* kt, const void* vt,
                                 const uint32_t* mask, const int32_t* num_nodes, int S, int B,
                                 int Hq, int Hkv, int D, float scale, void* out, float* lse,
                                 void* ws, const AttnPlan& plan, hipStream_t st);

// walk
struct WalkPlan {
  int nchunks;
  int64_t chunk_len;
  size_t ws_bytes;
};
WalkPlan walk_plan(int S, int B, int64_t vocab);
hipError_t launch_tree_walk(const int32_t* tree_tok, const int32_t* parent,
                            const int32_t* num_nodes, const float* target, int S, int B, int L,
                            int64_t vocab, int32_t* accept_len, int32_t* acc_nodes,
                            int32_t* acc_tok, int32_t* bonus_out, void* ws, const WalkPlan& plan,
                            hipStream_t st);

// Benchmark timing of the attention's main kernel (see ddt_attention_profiling).
// prof_begin returns the stop event to record after the kernel, or nullptr when
// profiling is off; it records the start event itself.
hipEvent_t prof_begin(hipStream_t st);
hipError_t prof_record(hipEvent_t ev, hipStream_t st);

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace ddt
