// C entry points of libddt: argument validation, workspace sizing and launch.
// The operations are defined in include/ddt.h, next to their citations.
#include <math.h>

#include <mutex>
#include <utility>
#include <vector>

#include "ddt_internal.h"

namespace ddt {

int cu_count() {
  static std::mutex mu;
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64) {
    std::lock_guard<std::mutex> lk(mu);
    if (cache[dev] > 0) return cache[dev];
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  if (dev < 64) {
    std::lock_guard<std::mutex> lk(mu);
    cache[dev] = n;
  }
  return n;
}

namespace {
struct ProfEvents {
  hipEvent_t start, stop, step_stop;
  bool step_used;
};
struct Prof {
  std::mutex mu;
  bool on = false;
  std::vector<ProfEvents> pool;
  size_t used = 0;
};
// one pool per timed kernel: the attention's main kernel, the epilogue's tile kernel
Prof& prof(int which = 0) {
  static Prof p[2];
  return p[which];
}

bool take_events(Prof& p, hipEvent_t* start, hipEvent_t* stop, hipEvent_t* step_stop) {
  std::lock_guard<std::mutex> lk(p.mu);
  if (!p.on) return false;
  if (p.used == p.pool.size()) {
    hipEvent_t ev[3] = {nullptr, nullptr, nullptr};
    for (int i = 0; i < 3; ++i) {
      if (hipEventCreate(&ev[i]) != hipSuccess) {
        for (int j = 0; j < i; ++j) (void)hipEventDestroy(ev[j]);
        return false;
      }
    }
    p.pool.push_back({ev[0], ev[1], ev[2], false});
  }
  auto& e = p.pool[p.used++];
  e.step_used = step_stop != nullptr;
  *start = e.start;
  *stop = e.stop;
  if (step_stop) *step_stop = e.step_stop;
  return true;
}

int set_profiling(Prof& p, int enable) {
  std::lock_guard<std::mutex> lk(p.mu);
  p.on = enable != 0;
  if (!p.on) {
    int rc = DDT_OK;
    for (auto& ev : p.pool)
      for (hipEvent_t e : {ev.start, ev.stop, ev.step_stop})
        if (hipEventDestroy(e) != hipSuccess) rc = DDT_ERR_HIP;
    p.pool.clear();
    p.used = 0;
    return rc;
  }
  return DDT_OK;
}

// sums of the recorded (start, stop) and (start, step stop) intervals since the last
// read, and their count
int read_timing(Prof& p, double* main_ms, double* step_ms, int* count) {
  std::lock_guard<std::mutex> lk(p.mu);
  double tm = 0.0, ts = 0.0;
  int n = 0;
  for (size_t i = 0; i < p.used; ++i) {
    const ProfEvents& e = p.pool[i];
    const hipEvent_t last = e.step_used ? e.step_stop : e.stop;
    if (hipEventSynchronize(last) != hipSuccess) return DDT_ERR_HIP;
    float a = 0.f, b = 0.f;
    if (hipEventElapsedTime(&a, e.start, e.stop) != hipSuccess) return DDT_ERR_HIP;
    if (hipEventElapsedTime(&b, e.start, last) != hipSuccess) return DDT_ERR_HIP;
    tm += a;
    ts += b;
    ++n;
  }
  p.used = 0;
  *main_ms = tm;
  if (step_ms) *step_ms = ts;
  *count = n;
  return DDT_OK;
}
}  // namespace

bool prof_events(hipEvent_t* start, hipEvent_t* stop, hipEvent_t* step_stop) {
  return take_events(prof(0), start, stop, step_stop);
}

bool lm_prof_events(hipEvent_t* start, hipEvent_t* stop) {
  return take_events(prof(1), start, stop, nullptr);
}

}  // namespace ddt

using namespace ddt;

namespace {

inline int hip_status(hipError_t e) { return e == hipSuccess ? DDT_OK : DDT_ERR_HIP; }
inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

}  // namespace

extern "C" {

const char* ddt_status_string(int status) {
  switch (status) {
    case DDT_OK: return "ok";
    case DDT_ERR_INVALID_ARG: return "invalid argument";
    case DDT_ERR_UNSUPPORTED: return "unsupported configuration";
    case DDT_ERR_WORKSPACE: return "workspace too small";
    case DDT_ERR_HIP: return "HIP launch failure";
    case DDT_ERR_TOO_LARGE: return "problem larger than the library's static scratch";
    default: return "unknown status";
  }
}

// ------------------------------------------------------------------ top-K
size_t ddt_topk_workspace_size(int64_t rows, int64_t vocab, int k) {
  if (rows < 1 || vocab < 1 || k < 1 || k > DDT_MAX_K) return 0;
  return topk_plan(rows, vocab, k).ws_bytes;
}

int ddt_topk(const float* logits, int64_t rows, int64_t vocab, int64_t row_stride, int k,
             int32_t* out_tok, float* out_logq, void* ws, size_t ws_bytes, void* stream) {
  if (!logits || !out_tok || !out_logq) return DDT_ERR_INVALID_ARG;
  if (rows < 1 || rows > INT32_MAX || vocab < 1 || vocab > INT32_MAX || row_stride < vocab)
    return DDT_ERR_INVALID_ARG;
  if (k < 1 || k > DDT_MAX_K || k > vocab) return DDT_ERR_INVALID_ARG;
  const TopkPlan plan = topk_plan(rows, vocab, k);
  if (rows * plan.nchunks > INT32_MAX) return DDT_ERR_UNSUPPORTED;
  if (!ws || ws_bytes < plan.ws_bytes) return DDT_ERR_WORKSPACE;
  return hip_status(launch_topk(logits, rows, vocab, row_stride, k, out_tok, out_logq, ws, plan,
                                as_stream(stream)));
}

// ------------------------------------------------------------------ tree build
int ddt_build_tree(const int32_t* topk_tok, const float* topk_logq, const int32_t* bonus, int S,
                   int L, int K, int B, int32_t* tree_tok, int32_t* parent, int32_t* depth,
                   float* node_logq, int32_t* num_nodes, void* stream) {
  if (!topk_tok || !topk_logq || !bonus || !tree_tok || !parent || !depth || !num_nodes)
    return DDT_ERR_INVALID_ARG;
  if (S < 1 || L < 1 || L > DDT_MAX_L || K < 1 || K > DDT_MAX_K || B < 0 || B > DDT_MAX_B)
    return DDT_ERR_INVALID_ARG;
  return hip_status(launch_build_tree(topk_tok, topk_logq, bonus, S, L, K, B, tree_tok, parent,
                                      depth, node_logq, num_nodes, as_stream(stream)));
}

// ------------------------------------------------------------------ mask
int ddt_tree_mask(const int32_t* parent, const int32_t* depth, const int32_t* num_nodes,
                  const int64_t* cu_prefix, const int64_t* prefix_len, int S, int B,
                  uint32_t* mask, int32_t* pos_ids, void* stream) {
  if (!parent || !depth || !num_nodes || !mask) return DDT_ERR_INVALID_ARG;
  if (S < 1 || B < 0 || B > DDT_MAX_B) return DDT_ERR_INVALID_ARG;
  return hip_status(launch_tree_mask(parent, depth, num_nodes, Prefix{cu_prefix, prefix_len}, S, B,
                                     mask, pos_ids, as_stream(stream)));
}

// ------------------------------------------------------------------ steps 1-3 fused
size_t ddt_draft_tree_workspace_size(int S, int L, int64_t vocab, int K) {
  if (S < 1 || L < 1 || vocab < 1 || K < 1 || K > DDT_MAX_K) return 0;
  return topk_plan((int64_t)S * L, vocab, K).ws_bytes;
}

int ddt_draft_tree(const float* logits, int64_t row_stride, const int32_t* bonus,
                   const int64_t* cu_prefix, const int64_t* prefix_len, int S, int L,
                   int64_t vocab, int K, int B,
                   int32_t* topk_tok, float* topk_logq, int32_t* tree_tok, int32_t* parent,
                   int32_t* depth, float* node_logq, int32_t* num_nodes, uint32_t* mask,
                   int32_t* pos_ids, void* ws, size_t ws_bytes, void* stream) {
  if (!logits || !bonus || !topk_tok || !topk_logq || !tree_tok || !parent || !depth ||
      !num_nodes || !mask)
    return DDT_ERR_INVALID_ARG;
  if (S < 1 || L < 1 || L > DDT_MAX_L || B < 0 || B > DDT_MAX_B || vocab < 1 ||
      vocab > INT32_MAX || row_stride < vocab || K < 1 || K > DDT_MAX_K || K > vocab)
    return DDT_ERR_INVALID_ARG;
  const int64_t rows = (int64_t)S * L;
  const TopkPlan plan = topk_plan(rows, vocab, K);
  if (rows * plan.nchunks > INT32_MAX) return DDT_ERR_UNSUPPORTED;
  if (!ws || ws_bytes < plan.ws_bytes) return DDT_ERR_WORKSPACE;
  const hipStream_t st = as_stream(stream);
  hipError_t e = launch_topk_partial(logits, rows, vocab, row_stride, K, ws, plan, st);
  if (e != hipSuccess) return DDT_ERR_HIP;
  return hip_status(launch_draft_tree(ws, plan, bonus, Prefix{cu_prefix, prefix_len}, S, L, K, B,
                                      topk_tok, topk_logq, tree_tok, parent, depth, node_logq,
                                      num_nodes, mask, cu_prefix ? pos_ids : nullptr, st));
}

// ------------------------------------------------------------------ attention
static int attn_check(int S, int B, int Hq, int Hkv, int D, int dtype) {
  if (S < 1 || B < 0 || B > DDT_MAX_B || Hq < 1 || Hkv < 1 || Hq % Hkv != 0)
    return DDT_ERR_INVALID_ARG;
  if (D != 32 && D != 64 && D != 128) return DDT_ERR_UNSUPPORTED;
  if (dtype != DDT_F32 && dtype != DDT_BF16) return DDT_ERR_UNSUPPORTED;
  if ((int64_t)S * (B + 1) * Hq > INT32_MAX) return DDT_ERR_UNSUPPORTED;
  return DDT_OK;
}

size_t ddt_tree_attention_workspace_size(int S, int B, int Hq, int Hkv, int D, int dtype,
                                         int64_t max_prefix) {
  if (attn_check(S, B, Hq, Hkv, D, dtype) != DDT_OK || max_prefix < 0) return 0;
  return attn_plan(S, B, Hq, Hkv, D, dtype, max_prefix).ws_bytes;
}

int ddt_tree_attention(const void* q, const void* k_cache, const void* v_cache,
                       const int64_t* cu_prefix, const int64_t* prefix_len,
                       const void* k_tree, const void* v_tree,
                       const uint32_t* mask, const int32_t* num_nodes, int S, int B, int Hq,
                       int Hkv, int D, int dtype, float scale, int64_t max_prefix, void* out,
                       float* lse, void* ws, size_t ws_bytes, void* stream) {
  if (!q || !cu_prefix || !k_tree || !v_tree || !mask || !num_nodes || !out)
    return DDT_ERR_INVALID_ARG;
  // an empty cache may be passed as NULL; the kernels then treat every P_s as 0
  if ((!k_cache || !v_cache) && max_prefix != 0) return DDT_ERR_INVALID_ARG;
  const int c = attn_check(S, B, Hq, Hkv, D, dtype);
  if (c != DDT_OK) return c;
  if (!(scale > 0.f) || !isfinite(scale) || max_prefix < 0) return DDT_ERR_INVALID_ARG;
  // the bf16 kernels address a tile's 64 key rows with 32-bit byte offsets
  if (dtype == DDT_BF16 && (int64_t)Hkv * D * 2 * 64 > INT32_MAX) return DDT_ERR_UNSUPPORTED;
  const AttnPlan plan = attn_plan(S, B, Hq, Hkv, D, dtype, max_prefix);
  if (plan.ws_bytes > 0 && (!ws || ws_bytes < plan.ws_bytes)) return DDT_ERR_WORKSPACE;
  if ((int64_t)S * Hkv * (plan.nsplit + 1) * plan.row_groups + 8 * (int64_t)plan.row_groups > INT32_MAX)
    return DDT_ERR_UNSUPPORTED;
  return hip_status(launch_tree_attention(q, k_cache, v_cache, Prefix{cu_prefix, prefix_len},
                                          k_tree, v_tree, mask,
                                          num_nodes, S, B, Hq, Hkv, D, scale, out, lse, ws, plan,
                                          as_stream(stream)));
}

// ------------------------------------------------------------------ adaptive budget
int ddt_adapt_budget(const float* cost, int S, int B, int32_t* tree_tok, int32_t* parent,
                     int32_t* depth, float* node_logq, int32_t* num_nodes, int32_t* budget_out,
                     float* expected_out, void* stream) {
  if (!cost || !tree_tok || !parent || !depth || !node_logq || !num_nodes || !budget_out)
    return DDT_ERR_INVALID_ARG;
  if (S < 1 || B < 0 || B > DDT_MAX_B) return DDT_ERR_INVALID_ARG;
  return hip_status(launch_adapt_budget(cost, S, B, tree_tok, parent, depth, node_logq, num_nodes,
                                        budget_out, expected_out, as_stream(stream)));
}

// ------------------------------------------------------------------ KV commit
int ddt_commit_kv(void* k_cache, void* v_cache, const int64_t* cu_prefix, int64_t* prefix_len,
                  const void* k_tree, const void* v_tree, const int32_t* acc_nodes,
                  const int32_t* accept_len, int S, int B, int L, int Hkv, int D, int dtype,
                  int32_t* appended, void* stream) {
  if (!k_cache || !v_cache || !cu_prefix || !prefix_len || !k_tree || !v_tree || !acc_nodes ||
      !accept_len)
    return DDT_ERR_INVALID_ARG;
  if (S < 1 || B < 0 || B > DDT_MAX_B || L < 1 || L > DDT_MAX_L || Hkv < 1) return DDT_ERR_INVALID_ARG;
  if (D != 32 && D != 64 && D != 128) return DDT_ERR_UNSUPPORTED;
  if (dtype != DDT_F32 && dtype != DDT_BF16) return DDT_ERR_UNSUPPORTED;
  for (const void* p : {(const void*)k_cache, (const void*)v_cache, k_tree, v_tree})
    if (reinterpret_cast<uintptr_t>(p) % 16 != 0) return DDT_ERR_INVALID_ARG;
  const int64_t row_bytes = (int64_t)Hkv * D * (dtype == DDT_BF16 ? 2 : 4);
  if (row_bytes / 16 > INT32_MAX / (DDT_MAX_L + 1)) return DDT_ERR_UNSUPPORTED;
  return hip_status(launch_commit_kv(k_cache, v_cache, cu_prefix, prefix_len, k_tree, v_tree,
                                     acc_nodes, accept_len, S, B + 1, L, row_bytes, appended,
                                     as_stream(stream)));
}

// ------------------------------------------------------------------ walk
size_t ddt_tree_walk_workspace_size(int S, int B, int64_t vocab) {
  if (S < 1 || B < 0 || B > DDT_MAX_B || vocab < 1) return 0;
  return walk_plan(S, B, vocab).ws_bytes;
}

int ddt_tree_walk(const int32_t* tree_tok, const int32_t* parent, const int32_t* num_nodes,
                  const float* target_logits, int S, int B, int L, int64_t vocab,
                  int32_t* accept_len, int32_t* acc_nodes, int32_t* acc_tok, int32_t* bonus_out,
                  void* ws, size_t ws_bytes, void* stream) {
  if (!tree_tok || !parent || !num_nodes || !target_logits || !accept_len || !acc_nodes ||
      !acc_tok || !bonus_out)
    return DDT_ERR_INVALID_ARG;
  if (S < 1 || L < 1 || L > DDT_MAX_L || B < 0 || B > DDT_MAX_B || vocab < 1 || vocab > INT32_MAX)
    return DDT_ERR_INVALID_ARG;
  const WalkPlan plan = walk_plan(S, B, vocab);
  if (!ws || ws_bytes < plan.ws_bytes) return DDT_ERR_WORKSPACE;
  return hip_status(launch_tree_walk(tree_tok, parent, num_nodes, target_logits, S, B, L, vocab,
                                     accept_len, acc_nodes, acc_tok, bonus_out, ws, plan,
                                     as_stream(stream)));
}

int ddt_tree_walk_strategy(int mode) {
  const int prev = set_walk_strategy(mode);
  return prev < 0 ? DDT_ERR_INVALID_ARG : prev;
}

int ddt_tree_walk_mode(int S, int B, int L, int64_t vocab) {
  if (S < 1 || L < 1 || L > DDT_MAX_L || B < 0 || B > DDT_MAX_B || vocab < 1 || vocab > INT32_MAX)
    return DDT_ERR_INVALID_ARG;
  int steps = 0;
  switch (walk_mode(S, B, L, vocab, &steps)) {
    case WalkMode::kScan: return DDT_WALK_SCAN;
    case WalkMode::kPath: return DDT_WALK_PATH;
    default: return DDT_WALK_HYBRID;
  }
}

size_t ddt_lm_head_argmax_workspace_size(int S, int B, int64_t vocab, int d) {
  if (S < 1 || B < 0 || B > DDT_MAX_B || vocab < 1 || vocab > INT32_MAX - 512 || d < 64 ||
      d > 65536 || d % 64 != 0)
    return 0;
  return lm_head_plan(S, B, vocab, d).ws_bytes;
}

int ddt_lm_head_argmax(const void* hidden, const void* weight, const int32_t* num_nodes, int S,
                       int B, int d, int64_t vocab, int32_t* node_tok, float* node_max, void* ws,
                       size_t ws_bytes, void* stream) {
  if (!hidden || !weight || !node_tok) return DDT_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(hidden) % 16 != 0 || reinterpret_cast<uintptr_t>(weight) % 16 != 0)
    return DDT_ERR_INVALID_ARG;
  if (S < 1 || B < 0 || B > DDT_MAX_B || vocab < 1 || vocab > INT32_MAX - 512 || d < 64 || d > 65536)
    return DDT_ERR_INVALID_ARG;
  if (d % 64 != 0) return DDT_ERR_UNSUPPORTED;
  if ((int64_t)S * (B + 1) * ((vocab + 255) / 256) > INT32_MAX) return DDT_ERR_UNSUPPORTED;
  const LmPlan plan = lm_head_plan(S, B, vocab, d);
  if (!ws || ws_bytes < plan.ws_bytes) return DDT_ERR_WORKSPACE;
  return hip_status(launch_lm_head(hidden, weight, num_nodes, S, B, d, vocab, node_tok, node_max,
                                   ws, plan, as_stream(stream)));
}

int ddt_tree_walk_tokens(const int32_t* tree_tok, const int32_t* parent, const int32_t* num_nodes,
                         const int32_t* node_tok, int S, int B, int L, int32_t* accept_len,
                         int32_t* acc_nodes, int32_t* acc_tok, int32_t* bonus_out, void* stream) {
  if (!tree_tok || !parent || !num_nodes || !node_tok || !accept_len || !acc_nodes || !acc_tok ||
      !bonus_out)
    return DDT_ERR_INVALID_ARG;
  if (S < 1 || L < 1 || L > DDT_MAX_L || B < 0 || B > DDT_MAX_B) return DDT_ERR_INVALID_ARG;
  return hip_status(launch_tree_walk_tokens(tree_tok, parent, num_nodes, node_tok, S, B, L,
                                            accept_len, acc_nodes, acc_tok, bonus_out,
                                            as_stream(stream)));
}

int ddt_tree_walk_sample(const int32_t* tree_tok, const int32_t* parent, const int32_t* depth,
                         const int32_t* num_nodes, const float* target_logits, const float* gumbel,
                         float inv_temperature, int S, int B, int L, int64_t vocab,
                         int32_t* accept_len, int32_t* acc_nodes, int32_t* acc_tok,
                         int32_t* bonus_out, void* ws, size_t ws_bytes, void* stream) {
  if (!tree_tok || !parent || !depth || !num_nodes || !target_logits || !gumbel || !accept_len ||
      !acc_nodes || !acc_tok || !bonus_out)
    return DDT_ERR_INVALID_ARG;
  if (S < 1 || L < 1 || L > DDT_MAX_L || B < 0 || B > DDT_MAX_B || vocab < 1 || vocab > INT32_MAX)
    return DDT_ERR_INVALID_ARG;
  if (!(inv_temperature >= 0.f) || !isfinite(inv_temperature)) return DDT_ERR_INVALID_ARG;
  const WalkPlan plan = walk_plan(S, B, vocab);
  if (!ws || ws_bytes < plan.ws_bytes) return DDT_ERR_WORKSPACE;
  return hip_status(launch_tree_walk(tree_tok, parent, num_nodes, target_logits, S, B, L, vocab,
                                     accept_len, acc_nodes, acc_tok, bonus_out, ws, plan,
                                     as_stream(stream), depth, gumbel, inv_temperature));
}

int ddt_tree_walk_noalloc(const int32_t* tree_tok, const int32_t* parent, const int32_t* num_nodes,
                          const float* target_logits, int S, int B, int L, int64_t vocab,
                          int32_t* accept_len, int32_t* acc_nodes, int32_t* acc_tok,
                          int32_t* bonus_out, void* stream) {
  if (!tree_tok || !parent || !num_nodes || !target_logits || !accept_len || !acc_nodes ||
      !acc_tok || !bonus_out)
    return DDT_ERR_INVALID_ARG;
  if (S < 1 || L < 1 || L > DDT_MAX_L || B < 0 || B > DDT_MAX_B || vocab < 1 || vocab > INT32_MAX)
    return DDT_ERR_INVALID_ARG;
  const WalkPlan plan = walk_plan(S, B, vocab);
  if (plan.ws_bytes > walk_scratch_bytes()) return DDT_ERR_TOO_LARGE;
  const hipStream_t st = as_stream(stream);
  void* ws = nullptr;
  if (walk_scratch(&ws, st) != hipSuccess) return DDT_ERR_HIP;
  return hip_status(launch_tree_walk(tree_tok, parent, num_nodes, target_logits, S, B, L, vocab,
                                     accept_len, acc_nodes, acc_tok, bonus_out, ws, plan, st));
}

size_t ddt_tree_walk_noalloc_max_bytes(void) { return walk_scratch_bytes(); }

// ------------------------------------------------------------------ benchmark aid
int ddt_attention_profiling(int enable) { return set_profiling(prof(0), enable); }

int ddt_attention_timing(double* main_ms, double* step_ms, int* count) {
  if (!main_ms || !step_ms || !count) return DDT_ERR_INVALID_ARG;
  return read_timing(prof(0), main_ms, step_ms, count);
}

int ddt_lm_head_profiling(int enable) { return set_profiling(prof(1), enable); }

int ddt_lm_head_timing(double* tiles_ms, int* count) {
  if (!tiles_ms || !count) return DDT_ERR_INVALID_ARG;
  return read_timing(prof(1), tiles_ms, nullptr, count);
}

}  // extern "C"
