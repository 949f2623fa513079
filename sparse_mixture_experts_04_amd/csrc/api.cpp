// C ABI of the MoE layer (declared in include/moe.h): argument checks,
// workspace carving and the launch sequence.  Every check runs on the host
// before anything is enqueued.
#include <algorithm>
#include <cmath>
#include "../../include/moe.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <limits>

#include "kernels.hpp"

namespace moe {

int device_cu_count() {
  static std::atomic<int> cache[256];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 256) return 256;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

}  // namespace moe

namespace {

size_t align256(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }

size_t esize(const moe_config* c) { return c->dtype == MOE_BF16 ? 2 : 4; }

moe_status check_cfg(const moe_config* c) {
  if (c == nullptr) return MOE_ERR_INVALID_ARG;
  if (c->dtype != MOE_F32 && c->dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (c->num_tokens < 0 || c->hidden_size <= 0 || c->intermediate_size <= 0) return MOE_ERR_INVALID_ARG;
  if (c->num_experts < 1 || c->num_experts_per_tok < 1 || c->num_experts_per_tok > c->num_experts)
    return MOE_ERR_INVALID_ARG;
  if (c->num_experts > moe::kMaxExpertsAbi) return MOE_ERR_UNSUPPORTED;
  if (c->hidden_size % 64 != 0 || c->intermediate_size % 64 != 0) return MOE_ERR_UNSUPPORTED;
  const int64_t pairs = static_cast<int64_t>(c->num_tokens) * c->num_experts_per_tok;
  if (pairs > std::numeric_limits<int32_t>::max()) return MOE_ERR_UNSUPPORTED;
  const int64_t widest = c->hidden_size > c->intermediate_size ? c->hidden_size : c->intermediate_size;
  if (pairs > 0 && widest > (int64_t{1} << 62) / pairs) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

bool capacity_mode(const moe_config* c) { return c->expert_capacity >= 0; }

size_t pairs_of(const moe_config* c) {
  return static_cast<size_t>(c->num_tokens) * static_cast<size_t>(c->num_experts_per_tok);
}

size_t route_bytes(const moe_config* c) {
  return moe::router_scratch_bytes(c->num_tokens, c->hidden_size, c->num_experts, c->dtype);
}
size_t dispatch_bytes(const moe_config* c) {
  return moe::dispatch_scratch_bytes(c->num_tokens, c->num_experts, c->num_experts_per_tok, capacity_mode(c));
}
size_t dispatch_reroute_bytes(const moe_config* c) {
  return moe::dispatch_scratch_bytes(c->num_tokens, c->num_experts, c->num_experts_per_tok, capacity_mode(c),
                                     /*reroute=*/true);
}
size_t h_bytes(const moe_config* c) { return align256(pairs_of(c) * c->intermediate_size * esize(c)); }
size_t xp_bytes(const moe_config* c) { return align256(pairs_of(c) * c->hidden_size * esize(c)); }

// Bound on the rows one expert holds, used only to pick the expert-GEMM
// variant: routing picks k distinct experts per token, so at most T rows per
// expert (and at most C under a capacity).  The expert kernels compute any
// row count correctly -- an expert beyond the bound costs extra passes -- so
// offsets from repeated ids (a caller's own ids, or non-finite logits) stay
// in bounds and are computed in full.
int rows_per_expert_bound(const moe_config* c) {
  int b = c->num_tokens;
  if (c->expert_capacity >= 0 && c->expert_capacity < b) b = c->expert_capacity;
  return b;
}

// Whether the up-projection reads X through perm (the 256x256 kernel or the
// decode kernel runs, and X fits 32-bit buffer offsets).
bool gathers(const moe_config* c) {
  return moe::grouped_gemm_gathers(c->dtype, c->hidden_size, c->intermediate_size, rows_per_expert_bound(c),
                                   c->num_tokens, static_cast<int>(pairs_of(c)), c->num_experts);
}

moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

}  // namespace

extern "C" {

const char* moe_status_string(moe_status status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG: invalid argument";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: shape outside the supported limits";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "MOE_ERR_WORKSPACE_TOO_SMALL: workspace smaller than moe_workspace_size";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: a HIP runtime call or kernel launch failed";
  }
  return "unknown moe_status";
}

const char* moe_version(void) { return "moe-gfx950 1 (router, dispatch, grouped MFMA GEMM, combine)"; }

moe_status moe_capacity_from_factor(int32_t batch, int32_t seq_len, int32_t num_experts, int32_t num_experts_per_tok,
                                    double capacity_factor, int32_t* capacity) {
  if (capacity == nullptr || batch < 0 || seq_len < 0 || num_experts < 1 || num_experts_per_tok < 1 ||
      num_experts_per_tok > num_experts || !(capacity_factor > 0.0) || !std::isfinite(capacity_factor))
    return MOE_ERR_INVALID_ARG;
  if (seq_len == 1) {
    *capacity = std::min(512, 2 * batch);  // 2 * batch <= 2^31 - 2
    return MOE_OK;
  }
  const double tokens = static_cast<double>(batch) * seq_len;
  const double per_expert = tokens / num_experts;
  double c = std::floor(per_expert * num_experts_per_tok * capacity_factor / num_experts);
  if (c > tokens) c = tokens;
  if (c > 2147483647.0) return MOE_ERR_INVALID_ARG;
  *capacity = static_cast<int32_t>(c);
  return MOE_OK;
}

moe_status moe_workspace_size(const moe_config* cfg, int32_t op, size_t* bytes) {
  if (bytes == nullptr) return MOE_ERR_INVALID_ARG;
  if (moe_status s = check_cfg(cfg); s != MOE_OK) return s;
  switch (op) {
    case MOE_OP_ROUTE: *bytes = route_bytes(cfg); return MOE_OK;
    case MOE_OP_ROUTE_STATS:
      *bytes = align256(route_bytes(cfg)) + moe::router_stats_scratch_bytes(cfg->num_tokens, cfg->num_experts);
      return MOE_OK;
    case MOE_OP_DISPATCH: *bytes = dispatch_bytes(cfg); return MOE_OK;
    case MOE_OP_EXPERT_FFN: *bytes = h_bytes(cfg); return MOE_OK;
    case MOE_OP_FORWARD:
      *bytes = align256(route_bytes(cfg)) + align256(dispatch_bytes(cfg)) + 2 * xp_bytes(cfg) + h_bytes(cfg);
      return MOE_OK;
    case MOE_OP_DISPATCH_REROUTE: *bytes = dispatch_reroute_bytes(cfg); return MOE_OK;
    case MOE_OP_FORWARD_REROUTE:
      *bytes = align256(route_bytes(cfg)) + align256(dispatch_reroute_bytes(cfg)) + 2 * xp_bytes(cfg) + h_bytes(cfg);
      return MOE_OK;
    default: return MOE_ERR_INVALID_ARG;
  }
}

moe_status moe_route(const moe_config* cfg, const void* X, const void* Wg, const float* gate_bias,
                     int32_t* topk_ids, float* topk_w, void* ws, size_t ws_bytes, void* stream) {
  if (moe_status s = check_cfg(cfg); s != MOE_OK) return s;
  if (cfg->num_tokens == 0) return MOE_OK;
  if (!X || !Wg || !topk_ids || !topk_w) return MOE_ERR_INVALID_ARG;
  const size_t need = route_bytes(cfg);
  if (ws_bytes < need) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if (ws == nullptr) return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_router(cfg->dtype, X, Wg, gate_bias, cfg->num_tokens, cfg->hidden_size,
                                       cfg->num_experts, cfg->num_experts_per_tok, topk_ids, topk_w, ws,
                                       as_stream(stream)));
}

moe_status moe_route_ranked(const moe_config* cfg, const void* X, const void* Wg, const float* gate_bias,
                            int32_t* topk_ids, float* topk_w, uint8_t* expert_order, void* ws, size_t ws_bytes,
                            void* stream) {
  if (moe_status s = check_cfg(cfg); s != MOE_OK) return s;
  if (cfg->num_tokens == 0) return MOE_OK;
  if (!X || !Wg || !topk_ids || !topk_w || !expert_order) return MOE_ERR_INVALID_ARG;
  const size_t need = route_bytes(cfg);
  if (ws_bytes < need) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if (ws == nullptr) return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_router(cfg->dtype, X, Wg, gate_bias, cfg->num_tokens, cfg->hidden_size,
                                       cfg->num_experts, cfg->num_experts_per_tok, topk_ids, topk_w, ws,
                                       as_stream(stream), /*select=*/true, 1.f, nullptr, expert_order));
}

moe_status moe_route_stats(const moe_config* cfg, const void* X, const void* Wg, const float* gate_bias,
                           float temperature, int32_t* topk_ids, float* topk_w, float* prob_mean, float* sel_freq,
                           float* aux, void* ws, size_t ws_bytes, void* stream) {
  if (moe_status s = check_cfg(cfg); s != MOE_OK) return s;
  if (!(temperature > 0.f) || !std::isfinite(temperature)) return MOE_ERR_INVALID_ARG;
  if (cfg->num_tokens == 0) return MOE_OK;
  if (!X || !Wg || !topk_ids || !topk_w || !prob_mean || !sel_freq || !aux) return MOE_ERR_INVALID_ARG;
  size_t need = 0;
  moe_workspace_size(cfg, MOE_OP_ROUTE_STATS, &need);
  if (ws_bytes < need) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if (ws == nullptr) return MOE_ERR_INVALID_ARG;
  float* prob_sum = reinterpret_cast<float*>(static_cast<unsigned char*>(ws) + align256(route_bytes(cfg)));
  if (hipError_t e = moe::launch_router(cfg->dtype, X, Wg, gate_bias, cfg->num_tokens, cfg->hidden_size,
                                        cfg->num_experts, cfg->num_experts_per_tok, topk_ids, topk_w, ws,
                                        as_stream(stream), /*select=*/true, 1.f / temperature, prob_sum);
      e != hipSuccess)
    return MOE_ERR_HIP;
  return hip_status(moe::launch_router_stats(prob_sum, topk_ids, cfg->num_tokens, cfg->num_experts,
                                             cfg->num_experts_per_tok, prob_mean, sel_freq, aux,
                                             as_stream(stream)));
}

moe_status moe_dispatch(const moe_config* cfg, const int32_t* topk_ids, const void* X, int32_t* expert_counts,
                        int32_t* expert_offsets, int32_t* perm, int32_t* inv_perm, void* Xp, void* ws,
                        size_t ws_bytes, void* stream) {
  if (moe_status s = check_cfg(cfg); s != MOE_OK) return s;
  if (!expert_counts || !expert_offsets) return MOE_ERR_INVALID_ARG;
  if (cfg->num_tokens > 0 && (!topk_ids || !X || !perm || !inv_perm)) return MOE_ERR_INVALID_ARG;
  const size_t need = dispatch_bytes(cfg);
  if (ws_bytes < need) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if (need > 0 && ws == nullptr) return MOE_ERR_INVALID_ARG;
  const moe::DispatchScratch sc = moe::carve_dispatch_scratch(ws, cfg->num_tokens, cfg->num_experts,
                                                              cfg->num_experts_per_tok, capacity_mode(cfg));
  return hip_status(moe::launch_dispatch(cfg->dtype, topk_ids, X, cfg->num_tokens, cfg->hidden_size, cfg->num_experts,
                                         cfg->num_experts_per_tok, cfg->expert_capacity, expert_counts,
                                         expert_offsets, perm, inv_perm, Xp, sc, as_stream(stream)));
}

moe_status moe_dispatch_reroute(const moe_config* cfg, const int32_t* topk_ids, const uint8_t* expert_order,
                                const void* X, int32_t* expert_counts, int32_t* expert_offsets, int32_t* perm,
                                int32_t* inv_perm, void* Xp, void* ws, size_t ws_bytes, void* stream) {
  if (moe_status s = check_cfg(cfg); s != MOE_OK) return s;
  if (!expert_counts || !expert_offsets) return MOE_ERR_INVALID_ARG;
  if (cfg->num_tokens > 0 && (!topk_ids || !X || !perm || !inv_perm)) return MOE_ERR_INVALID_ARG;
  if (cfg->num_tokens > 0 && capacity_mode(cfg) && !expert_order) return MOE_ERR_INVALID_ARG;
  const size_t need = dispatch_reroute_bytes(cfg);
  if (ws_bytes < need) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if (need > 0 && ws == nullptr) return MOE_ERR_INVALID_ARG;
  const moe::DispatchScratch sc = moe::carve_dispatch_scratch(ws, cfg->num_tokens, cfg->num_experts,
                                                              cfg->num_experts_per_tok, capacity_mode(cfg),
                                                              /*reroute=*/true);
  return hip_status(moe::launch_dispatch_reroute(cfg->dtype, topk_ids, expert_order, X, cfg->num_tokens,
                                                 cfg->hidden_size, cfg->num_experts, cfg->num_experts_per_tok,
                                                 cfg->expert_capacity, expert_counts, expert_offsets, perm, inv_perm,
                                                 Xp, sc, as_stream(stream)));
}

moe_status moe_expert_up(const moe_config* cfg, const void* Xp, const int32_t* expert_offsets, const void* W1,
                         void* H, void* stream) {
  if (moe_status s = check_cfg(cfg); s != MOE_OK) return s;
  if (cfg->num_tokens == 0) return MOE_OK;
  if (!Xp || !expert_offsets || !W1 || !H) return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_grouped_gemm(cfg->dtype, true, Xp, W1, H, expert_offsets, cfg->num_experts,
                                             cfg->intermediate_size, cfg->hidden_size,
                                             static_cast<int>(pairs_of(cfg)), rows_per_expert_bound(cfg),
                                             as_stream(stream)));
}

moe_status moe_expert_up_gather_supported(const moe_config* cfg, int32_t* supported) {
  if (supported == nullptr) return MOE_ERR_INVALID_ARG;
  *supported = 0;
  if (moe_status s = check_cfg(cfg); s != MOE_OK) return s;
  *supported = gathers(cfg) ? 1 : 0;
  return MOE_OK;
}

moe_status moe_expert_up_gather(const moe_config* cfg, const void* X, const int32_t* perm,
                                const int32_t* expert_offsets, const void* W1, void* H, void* stream) {
  if (moe_status s = check_cfg(cfg); s != MOE_OK) return s;
  if (cfg->num_tokens == 0) return MOE_OK;
  if (!gathers(cfg)) return MOE_ERR_UNSUPPORTED;
  if (!X || !perm || !expert_offsets || !W1 || !H) return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_grouped_gemm_gather(true, X, cfg->num_tokens, perm, cfg->num_experts_per_tok, W1,
                                                    H, expert_offsets, cfg->num_experts, cfg->intermediate_size,
                                                    cfg->hidden_size, static_cast<int>(pairs_of(cfg)),
                                                    rows_per_expert_bound(cfg), as_stream(stream)));
}

moe_status moe_expert_down(const moe_config* cfg, const void* H, const int32_t* expert_offsets, const void* W2,
                           void* Yp, void* stream) {
  if (moe_status s = check_cfg(cfg); s != MOE_OK) return s;
  if (cfg->num_tokens == 0) return MOE_OK;
  if (!H || !expert_offsets || !W2 || !Yp) return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_grouped_gemm(cfg->dtype, false, H, W2, Yp, expert_offsets, cfg->num_experts,
                                             cfg->hidden_size, cfg->intermediate_size,
                                             static_cast<int>(pairs_of(cfg)), rows_per_expert_bound(cfg),
                                             as_stream(stream)));
}

moe_status moe_expert_ffn(const moe_config* cfg, const void* Xp, const int32_t* expert_offsets, const void* W1,
                          const void* W2, void* Yp, void* ws, size_t ws_bytes, void* stream) {
  if (moe_status s = check_cfg(cfg); s != MOE_OK) return s;
  if (cfg->num_tokens == 0) return MOE_OK;
  if (!Xp || !expert_offsets || !W1 || !W2 || !Yp) return MOE_ERR_INVALID_ARG;
  if (ws_bytes < h_bytes(cfg)) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if (ws == nullptr) return MOE_ERR_INVALID_ARG;
  if (moe_status s = moe_expert_up(cfg, Xp, expert_offsets, W1, ws, stream); s != MOE_OK) return s;
  return moe_expert_down(cfg, ws, expert_offsets, W2, Yp, stream);
}

moe_status moe_combine(const moe_config* cfg, const void* Yp, const int32_t* inv_perm, const float* topk_w,
                       void* out, void* stream) {
  if (moe_status s = check_cfg(cfg); s != MOE_OK) return s;
  if (cfg->num_tokens == 0) return MOE_OK;
  if (!Yp || !inv_perm || !topk_w || !out) return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_combine(cfg->dtype, Yp, inv_perm, topk_w, out, cfg->num_tokens, cfg->hidden_size,
                                        cfg->num_experts_per_tok, as_stream(stream)));
}

moe_status moe_forward(const moe_config* cfg, const void* X, const void* Wg, const float* gate_bias, const void* W1,
                       const void* W2, void* out, int32_t* topk_ids, float* topk_w, int32_t* expert_counts,
                       int32_t* expert_offsets, int32_t* perm, int32_t* inv_perm, void* ws, size_t ws_bytes,
                       void* stream) {
  if (moe_status s = check_cfg(cfg); s != MOE_OK) return s;
  if (!expert_counts || !expert_offsets) return MOE_ERR_INVALID_ARG;
  if (cfg->num_tokens > 0 &&
      (!X || !Wg || !W1 || !W2 || !out || !topk_ids || !topk_w || !perm || !inv_perm))
    return MOE_ERR_INVALID_ARG;
  size_t need = 0;
  moe_workspace_size(cfg, MOE_OP_FORWARD, &need);
  if (ws_bytes < need) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if (ws == nullptr) return MOE_ERR_INVALID_ARG;
  unsigned char* p = static_cast<unsigned char*>(ws);
  void* rws = p;
  p += align256(route_bytes(cfg));
  void* dws = p;
  p += align256(dispatch_bytes(cfg));
  void* Xp = p;
  p += xp_bytes(cfg);
  void* H = p;
  p += h_bytes(cfg);
  void* Yp = p;
  const moe::RouterSplit split =
      moe::router_split(cfg->num_tokens, cfg->hidden_size, cfg->num_experts, cfg->dtype, rws);
  // Where the up-projection can read each pair's token row from X through
  // perm, the dispatch writes indices only.
  const bool gather = gathers(cfg);
  void* const Xp_out = gather ? nullptr : Xp;
  if (split.partial != nullptr && moe::dispatch_is_single_block(cfg->num_tokens, cfg->num_experts_per_tok)) {
    // Small batch with a K-split router: the router writes its partial
    // logits only, and one block selects and dispatches (one launch fewer,
    // same results as moe_route followed by moe_dispatch).
    if (hipError_t e = moe::launch_router(cfg->dtype, X, Wg, gate_bias, cfg->num_tokens, cfg->hidden_size,
                                          cfg->num_experts, cfg->num_experts_per_tok, topk_ids, topk_w, rws,
                                          as_stream(stream), /*select=*/false);
        e != hipSuccess)
      return MOE_ERR_HIP;
    if (hipError_t e = moe::launch_topk_dispatch_small(
            cfg->dtype, split.partial, split.nsplit, gate_bias, topk_ids, topk_w, X, cfg->num_tokens,
            cfg->hidden_size, cfg->num_experts, cfg->num_experts_per_tok, cfg->expert_capacity, expert_counts,
            expert_offsets, perm, inv_perm, Xp_out, as_stream(stream));
        e != hipSuccess)
      return MOE_ERR_HIP;
  } else {
    if (moe_status s = moe_route(cfg, X, Wg, gate_bias, topk_ids, topk_w, rws, route_bytes(cfg), stream);
        s != MOE_OK)
      return s;
    if (moe_status s = moe_dispatch(cfg, topk_ids, X, expert_counts, expert_offsets, perm, inv_perm, Xp_out, dws,
                                    dispatch_bytes(cfg), stream);
        s != MOE_OK)
      return s;
  }
  if (cfg->num_tokens == 0) return MOE_OK;
  if (moe_status s = gather ? moe_expert_up_gather(cfg, X, perm, expert_offsets, W1, H, stream)
                            : moe_expert_up(cfg, Xp, expert_offsets, W1, H, stream);
      s != MOE_OK)
    return s;
  if (moe_status s = moe_expert_down(cfg, H, expert_offsets, W2, Yp, stream); s != MOE_OK) return s;
  return moe_combine(cfg, Yp, inv_perm, topk_w, out, stream);
}

moe_status moe_forward_reroute(const moe_config* cfg, const void* X, const void* Wg, const float* gate_bias,
                               const void* W1, const void* W2, void* out, int32_t* topk_ids, float* topk_w,
                               uint8_t* expert_order, int32_t* expert_counts, int32_t* expert_offsets, int32_t* perm,
                               int32_t* inv_perm, void* ws, size_t ws_bytes, void* stream) {
  if (moe_status s = check_cfg(cfg); s != MOE_OK) return s;
  if (!expert_counts || !expert_offsets) return MOE_ERR_INVALID_ARG;
  if (cfg->num_tokens > 0 &&
      (!X || !Wg || !W1 || !W2 || !out || !topk_ids || !topk_w || !expert_order || !perm || !inv_perm))
    return MOE_ERR_INVALID_ARG;
  size_t need = 0;
  moe_workspace_size(cfg, MOE_OP_FORWARD_REROUTE, &need);
  if (ws_bytes < need) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if (ws == nullptr) return MOE_ERR_INVALID_ARG;
  unsigned char* p = static_cast<unsigned char*>(ws);
  void* rws = p;
  p += align256(route_bytes(cfg));
  void* dws = p;
  p += align256(dispatch_reroute_bytes(cfg));
  void* Xp = p;
  p += xp_bytes(cfg);
  void* H = p;
  p += h_bytes(cfg);
  void* Yp = p;
  const bool gather = gathers(cfg);
  if (moe_status s =
          moe_route_ranked(cfg, X, Wg, gate_bias, topk_ids, topk_w, expert_order, rws, route_bytes(cfg), stream);
      s != MOE_OK)
    return s;
  if (moe_status s = moe_dispatch_reroute(cfg, topk_ids, expert_order, X, expert_counts, expert_offsets, perm,
                                          inv_perm, gather ? nullptr : Xp, dws, dispatch_reroute_bytes(cfg), stream);
      s != MOE_OK)
    return s;
  if (cfg->num_tokens == 0) return MOE_OK;
  if (moe_status s = gather ? moe_expert_up_gather(cfg, X, perm, expert_offsets, W1, H, stream)
                            : moe_expert_up(cfg, Xp, expert_offsets, W1, H, stream);
      s != MOE_OK)
    return s;
  if (moe_status s = moe_expert_down(cfg, H, expert_offsets, W2, Yp, stream); s != MOE_OK) return s;
  return moe_combine(cfg, Yp, inv_perm, topk_w, out, stream);
}

}  // extern "C"
