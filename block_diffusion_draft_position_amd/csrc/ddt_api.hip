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
struct Prof {
  std::mutex mu;
  bool on = false;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> pool;
  size_t used = 0;
};
Prof& prof() {
  static Prof p;
  return p;
}
}  // namespace

bool prof_events(hipEvent_t* start, hipEvent_t* stop) {
  Prof& p = prof();
  std::lock_guard<std::mutex> lk(p.mu);
  if (!p.on) return false;
  if (p.used == p.pool.size()) {
    hipEvent_t a = nullptr, b = nullptr;
    if (hipEventCreate(&a) != hipSuccess) return false;
    if (hipEventCreate(&b) != hipSuccess) {
      (void)hipEventDestroy(a);
      return false;
    }
    p.pool.emplace_back(a, b);
  }
  auto& ev = p.pool[p.used++];
  *start = ev.first;
  *stop = ev.second;
  return true;
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
                  const int64_t* cu_prefix, int S, int B, uint32_t* mask, int32_t* pos_ids,
                  void* stream) {
  if (!parent || !depth || !num_nodes || !mask) return DDT_ERR_INVALID_ARG;
  if (S < 1 || B < 0 || B > DDT_MAX_B) return DDT_ERR_INVALID_ARG;
  return hip_status(launch_tree_mask(parent, depth, num_nodes, cu_prefix, S, B, mask, pos_ids,
                                     as_stream(stream)));
}

// ------------------------------------------------------------------ steps 1-3 fused
size_t ddt_draft_tree_workspace_size(int S, int L, int64_t vocab, int K) {
  if (S < 1 || L < 1 || vocab < 1 || K < 1 || K > DDT_MAX_K) return 0;
  return topk_plan((int64_t)S * L, vocab, K).ws_bytes;
}

int ddt_draft_tree(const float* logits, int64_t row_stride, const int32_t* bonus,
                   const int64_t* cu_prefix, int S, int L, int64_t vocab, int K, int B,
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
  return hip_status(launch_draft_tree(ws, plan, bonus, cu_prefix, S, L, K, B, topk_tok, topk_logq,
                                      tree_tok, parent, depth, node_logq, num_nodes, mask,
                                      cu_prefix ? pos_ids : nullptr, st));
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
                       const int64_t* cu_prefix, const void* k_tree, const void* v_tree,
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
  const AttnPlan plan = attn_plan(S, B, Hq, Hkv, D, dtype, max_prefix);
  if (plan.ws_bytes > 0 && (!ws || ws_bytes < plan.ws_bytes)) return DDT_ERR_WORKSPACE;
  if ((int64_t)S * Hkv * (plan.nsplit + 1) * plan.row_groups + 8 * (int64_t)plan.row_groups > INT32_MAX)
    return DDT_ERR_UNSUPPORTED;
  return hip_status(launch_tree_attention(q, k_cache, v_cache, cu_prefix, k_tree, v_tree, mask,
                                          num_nodes, S, B, Hq, Hkv, D, scale, out, lse, ws, plan,
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

// ------------------------------------------------------------------ benchmark aid
int ddt_attention_profiling(int enable) {
  Prof& p = prof();
  std::lock_guard<std::mutex> lk(p.mu);
  p.on = enable != 0;
  if (!p.on) {
    int rc = DDT_OK;
    for (auto& ev : p.pool) {
      if (hipEventDestroy(ev.first) != hipSuccess) rc = DDT_ERR_HIP;
      if (hipEventDestroy(ev.second) != hipSuccess) rc = DDT_ERR_HIP;
    }
    p.pool.clear();
    p.used = 0;
    return rc;
  }
  return DDT_OK;
}

int ddt_attention_timing(double* total_ms, int* count) {
  if (!total_ms || !count) return DDT_ERR_INVALID_ARG;
  Prof& p = prof();
  std::lock_guard<std::mutex> lk(p.mu);
  double t = 0.0;
  int n = 0;
  for (size_t i = 0; i < p.used; ++i) {
    if (hipEventSynchronize(p.pool[i].second) != hipSuccess) return DDT_ERR_HIP;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, p.pool[i].first, p.pool[i].second) != hipSuccess) return DDT_ERR_HIP;
    t += ms;
    ++n;
  }
  p.used = 0;
  *total_ms = t;
  *count = n;
  return DDT_OK;
}

}  // extern "C"
