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

// The sampling score fl(fl(x * t) + g) of the walk at temperature > 0: contraction into
// a fused multiply-add would round once instead of twice and could change the arg-max,
// so it is switched off here.
__device__ __forceinline__ float sample_score(float x, float t, float g) {
#pragma clang fp contract(off)
  return x * t + g;
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ unsigned long long ballot(bool p) { return __builtin_amdgcn_ballot_w64(p); }

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

// ---- cross-lane exchange without LDS: DPP row permutes and the gfx950 permlane swaps.
// xchg<S>(v) returns the value of a partner lane in the other half of v's aligned
// group of 2S lanes (S = 1, 2, 4, 8, 16, 32).  For S = 4 and 8 the partner is the
// mirrored lane, not lane ^ S; any pairing of the two halves serves a butterfly
// reduction.
template <int CTRL>
__device__ __forceinline__ int dpp(int v, int old) {
  return __builtin_amdgcn_update_dpp(old, v, CTRL, 0xf, 0xf, false);
}

template <int S>
__device__ __forceinline__ int xchg(int v) {
  if constexpr (S == 1) return dpp<0xB1>(v, v);   // quad_perm [1,0,3,2]
  if constexpr (S == 2) return dpp<0x4E>(v, v);   // quad_perm [2,3,0,1]
  if constexpr (S == 4) return dpp<0x141>(v, v);  // row_half_mirror
  if constexpr (S == 8) return dpp<0x140>(v, v);  // row_mirror
  // The swaps exchange 16-lane rows (S = 16) or 32-lane halves (S = 32) between
  // two registers; with v in both, one result is v and the other is the partner.
  if constexpr (S == 16) {
    const auto p = __builtin_amdgcn_permlane16_swap((unsigned)v, (unsigned)v, false, false);
    return (int)(p[0] == (unsigned)v ? p[1] : p[0]);
  }
  if constexpr (S == 32) {
    const auto p = __builtin_amdgcn_permlane32_swap((unsigned)v, (unsigned)v, false, false);
    return (int)(p[0] == (unsigned)v ? p[1] : p[0]);
  }
}

template <int S>
__device__ __forceinline__ float xchg(float v) {
  return __builtin_bit_cast(float, xchg<S>(__builtin_bit_cast(int, v)));
}

template <int S>
__device__ __forceinline__ double xchg(double v) {
  const long long b = __builtin_bit_cast(long long, v);
  const int lo = xchg<S>((int)(b & 0xffffffff));
  const int hi = xchg<S>((int)(b >> 32));
  return __builtin_bit_cast(double, ((long long)hi << 32) | (unsigned int)lo);
}

// Reductions over the wave; every lane receives the result.
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, xchg<1>(v));
  v = fmaxf(v, xchg<2>(v));
  v = fmaxf(v, xchg<4>(v));
  v = fmaxf(v, xchg<8>(v));
  v = fmaxf(v, xchg<16>(v));
  v = fmaxf(v, xchg<32>(v));
  return v;
}

__device__ __forceinline__ double wave_sum(double v) {
  v += xchg<1>(v);
  v += xchg<2>(v);
  v += xchg<4>(v);
  v += xchg<8>(v);
  v += xchg<16>(v);
  v += xchg<32>(v);
  return v;
}

// Inclusive prefix sum over the wave, lane 0 first: shifts within each 16-lane row,
// then the row broadcasts carry row totals forward (lane 15 into rows 1 and 3, lane
// 31 into rows 2 and 3).  Lanes a DPP source does not reach add the 0 they start from.
__device__ __forceinline__ int wave_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return v;
}

// (value, id) pairs under `better`
template <int S>
__device__ __forceinline__ void argmax_step(float& v, int& i) {
  const float ov = xchg<S>(v);
  const int oi = xchg<S>(i);
  if (better(ov, oi, v, i)) {
    v = ov;
    i = oi;
  }
}

__device__ __forceinline__ void wave_argmax(float& v, int& i) {
  argmax_step<1>(v, i);
  argmax_step<2>(v, i);
  argmax_step<4>(v, i);
  argmax_step<8>(v, i);
  argmax_step<16>(v, i);
  argmax_step<32>(v, i);
}

// ---------------------------------------------------------------- prefix layout
// Sequence s's prefix keys are cache rows cu[s] .. cu[s] + length(s); the length is
// len[s] when given (rows up to cu[s + 1] are then capacity for appends), else
// cu[s + 1] - cu[s].  A null cu means no prefix at all.
struct Prefix {
  const int64_t* cu;
  const int64_t* len;
  __device__ __forceinline__ int64_t start(int s) const { return cu ? cu[s] : 0; }
  __device__ __forceinline__ int64_t length(int s) const {
    return !cu ? 0 : len ? len[s] : cu[s + 1] - cu[s];
  }
};

// ---------------------------------------------------------------- device properties
int cu_count();  // compute units of the current device (cached per device)

// ---------------------------------------------------------------- launchers
// Each returns hipSuccess or the launch error.  Arguments are validated by the
// C entry points before these are called.

// top-K
struct TopkPlan {
  int e;        // logits per lane: a wave's chunk is 64 * e
  int nchunks;  // chunks per row
  int merge_e;  // keys per lane per merge batch
  size_t ws_bytes;
};
TopkPlan topk_plan(int64_t rows, int64_t vocab, int k);
hipError_t launch_topk(const float* logits, int64_t rows, int64_t vocab, int64_t stride, int k,
                       int32_t* tok, float* logq, void* ws, const TopkPlan& plan,
                       hipStream_t st);
// the per-chunk half of top-K: chunk lists and statistics into ws (topk_ws_parts)
hipError_t launch_topk_partial(const float* logits, int64_t rows, int64_t vocab, int64_t stride,
                               int k, void* ws, const TopkPlan& plan, hipStream_t st);
void topk_ws_parts(void* ws, int64_t rows, int k, const TopkPlan& plan, unsigned long long** cand,
                   float2** stats);
// the per-row half of top-K, from the chunk lists in ws
hipError_t launch_topk_merge(int64_t rows, int k, int32_t* tok, float* logq, void* ws,
                             const TopkPlan& plan, hipStream_t st);

// tree build
hipError_t launch_build_tree(const int32_t* tok, const float* logq, const int32_t* bonus, int S,
                             int L, int K, int B, int32_t* tree_tok, int32_t* parent,
                             int32_t* depth, float* node_logq, int32_t* num_nodes, hipStream_t st);

// top-K merge + tree + mask of every sequence from the chunk lists that
// launch_topk_partial left in ws: one launch when a workgroup can give every draft
// position its own merge wave (draft_tree_uses_fused), else the three kernels.
hipError_t launch_draft_tree(const void* ws, const TopkPlan& plan, const int32_t* bonus,
                             Prefix pre, int S, int L, int K, int B,
                             int32_t* topk_tok, float* topk_logq, int32_t* tree_tok,
                             int32_t* parent, int32_t* depth, float* node_logq,
                             int32_t* num_nodes, uint32_t* mask, int32_t* pos_ids,
                             hipStream_t st);
bool draft_tree_uses_fused(int L, int K, int B, const TopkPlan& plan);

// mask
hipError_t launch_tree_mask(const int32_t* parent, const int32_t* depth, const int32_t* num_nodes,
                            Prefix pre, int S, int B, uint32_t* mask,
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
                                 Prefix pre, const void* kt, const void* vt,
                                 const uint32_t* mask, const int32_t* num_nodes, int S, int B,
                                 int Hq, int Hkv, int D, float scale, void* out, float* lse,
                                 void* ws, const AttnPlan& plan, hipStream_t st);

// walk (greedy, or with gumbel [S, L+1, vocab] and depth: sampling at 1 / inv_t)
struct WalkPlan {
  int waves;             // waves per workgroup
  int nbatch;            // batches of waves * 64 * 32 logits per row: one workgroup each
  bool short_scan;       // the grid fits the CUs at once: latency-path scan
  size_t counter_bytes;  // per-sequence completion counters at the front of the workspace
  size_t rowcnt_bytes;   // then per-row counters of finished batches
  size_t key_bytes;      // then one 64-bit arg-max key per node
  size_t state_bytes;    // then the hybrid walk's hand-off {node, accepted, count} per sequence
  size_t ws_bytes;       // all of the above + the hand-off subtree's rows, one int per node
};
WalkPlan walk_plan(int S, int B, int64_t vocab);
// The walk's strategy: the row scan alone, the path walk alone, or the hybrid (the path
// walk for *steps accepted tokens, then the scan over the reached node's subtree).
enum class WalkMode { kScan, kPath, kHybrid };
WalkMode walk_mode(int S, int B, int L, int64_t vocab, int* steps);
// the walk along the path: one workgroup per sequence, the visited rows only.
// depth/gumbel/inv_t as launch_tree_walk (gumbel null: greedy).  max_steps < 0: walk to
// the end; else hand over after max_steps accepted tokens through state [S][4] and the
// subtree's rows list [S, N] (both zero on entry).
hipError_t launch_path_walk(const int32_t* tree_tok, const int32_t* parent,
                            const int32_t* num_nodes, const float* target, int S, int B, int L,
                            int64_t vocab, int32_t* accept_len, int32_t* acc_nodes,
                            int32_t* acc_tok, int32_t* bonus_out, hipStream_t st,
                            const int32_t* depth, const float* gumbel, float inv_t,
                            int max_steps, unsigned* state, int32_t* list);
// 0: the planner decides; 1: always the row scan; 2: always the path walk; 3: always
// the hybrid.  Returns the previous mode, or -1 for an invalid one.
int set_walk_strategy(int mode);
// The walk's static scratch (a file-scope device array of walk_scratch_bytes()): its
// device address on the current device, looked up with hipGetSymbolAddress once per
// device, whose first lookup also enqueues a zero fill on st.
size_t walk_scratch_bytes();
hipError_t walk_scratch(void** ptr, hipStream_t st);
hipError_t launch_tree_walk(const int32_t* tree_tok, const int32_t* parent,
                            const int32_t* num_nodes, const float* target, int S, int B, int L,
                            int64_t vocab, int32_t* accept_len, int32_t* acc_nodes,
                            int32_t* acc_tok, int32_t* bonus_out, void* ws, const WalkPlan& plan,
                            hipStream_t st, const int32_t* depth = nullptr,
                            const float* gumbel = nullptr, float inv_t = 1.f);

// adaptive budget: per sequence, B* from the tree's scores and the cost table, and the
// tree cut to its top-B* prefixes in place (one workgroup per sequence)
hipError_t launch_adapt_budget(const float* cost, int S, int B, int32_t* tree_tok, int32_t* parent,
                               int32_t* depth, float* node_logq, int32_t* num_nodes,
                               int32_t* budget_out, float* expected_out, hipStream_t st);

// KV commit: appends each sequence's root and accepted nodes' tree K/V rows to its
// cache region and advances prefix_len (one workgroup per sequence).
hipError_t launch_commit_kv(void* k_cache, void* v_cache, const int64_t* cu_prefix,
                            int64_t* prefix_len, const void* k_tree, const void* v_tree,
                            const int32_t* acc_nodes, const int32_t* accept_len, int S, int N,
                            int L, int64_t row_bytes, int32_t* appended, hipStream_t st);

// verifier epilogue: LM head + arg-max per hidden row (partials per vocabulary tile in
// ws, then a per-row reduce), and the tree walk driven by the resulting tokens
struct LmPlan {
  int vt, mt;       // tile: vocabulary rows x hidden rows
  int nvt;          // vocabulary tiles
  size_t ws_bytes;  // partials [S * N, nvt] (value, id)
};
LmPlan lm_head_plan(int S, int B, int64_t vocab, int d);
hipError_t launch_lm_head(const void* hidden, const void* weight, const int32_t* num_nodes, int S,
                          int B, int d, int64_t vocab, int32_t* node_tok, float* node_max,
                          void* ws, const LmPlan& p, hipStream_t st);
hipError_t launch_tree_walk_tokens(const int32_t* tree_tok, const int32_t* parent,
                                   const int32_t* num_nodes, const int32_t* node_tok, int S, int B,
                                   int L, int32_t* accept_len, int32_t* acc_nodes, int32_t* acc_tok,
                                   int32_t* bonus_out, hipStream_t st);
// Benchmark timing of the epilogue's tile kernel: as prof_events, one start/stop pair
// per launch while epilogue profiling is on.
bool lm_prof_events(hipEvent_t* start, hipEvent_t* stop);

// Benchmark timing of the attention's main kernel and of the whole attention step
// (see ddt_attention_profiling).  While profiling is on, prof_events hands out a
// start/stop event pair that the launch attaches to the main kernel's dispatch
// (hipExtLaunchKernelGGL), so the pair brackets the kernel's execution, not its
// enqueueing; a launch that runs a second kernel (the split merge) asks for
// step_stop too and attaches it as that kernel's stop event.  Without profiling it
// returns false.
bool prof_events(hipEvent_t* start, hipEvent_t* stop, hipEvent_t* step_stop);

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace ddt
