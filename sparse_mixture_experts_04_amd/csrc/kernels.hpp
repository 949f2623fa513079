// Host-side launchers of the gfx950 kernels (internal to libmoe).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

constexpr int kDtypeF32 = 0;
constexpr int kDtypeBF16 = 1;

// Tokens per dispatch chunk: one wave, one token per lane.
constexpr int kDispatchChunk = 64;
constexpr int kMaxExpertsAbi = 64;  // expert ids fit one wave (64 lanes)

// Scratch of the dispatcher, carved from the caller's workspace.
struct DispatchScratch {
  int32_t* chunk_base;   // [nchunks][cols] (dropless: cols rounded up to 4): per-chunk histogram, then (three-launch path) its chunk-exclusive prefix
  int32_t* chunk_kept;   // [nchunks][E]:  kept pairs per chunk, then prefix (capacity only)
  int32_t* slot_base;    // [k][E]: pairs of expert e in slots < s (capacity only)
  int8_t* keep;          // [T*k]: keep flag per pair (capacity only)
  // Rerouting only:
  int32_t* ids2;         // [T*k]: expert of each pair after rerouting
  int32_t* drop_hist;    // [nchunks][k]: dropped pairs per chunk and slot, then prefix
  int32_t* drop_seg;     // [k+1]: start of each slot's segment of the dropped-pair list
  int32_t* drop_list;    // [T*k]: dropped pair ids in (slot, token) order
  int32_t* drop_next;    // [T*k]: list index of the same token's next dropped slot, -1 if none
  uint64_t* drop_used;   // [T*k]: experts the token's earlier dropped slots moved to
  uint8_t* drop_rows;    // [T*k][32 or 64]: the token's preference order, per list entry
};

size_t dispatch_scratch_bytes(int T, int E, int k, bool capacity, bool reroute = false);
DispatchScratch carve_dispatch_scratch(void* ws, int T, int E, int k, bool capacity, bool reroute = false);

// Router scratch: the transposed gate and, when T is small, the partial
// logits of the K splits.
size_t router_scratch_bytes(int T, int d, int E, int dtype);
// select = false with a K-split router (small T) writes only the partial
// logits: the caller selects (launch_topk_dispatch_small).
// inv_tau: 1 / router temperature (weights exp((l_s - l_0) * inv_tau) / sum);
// prob_sum (may be null): [ceil(T/16)][2E] per-16-token-tile sums of the full
// router probabilities and selection counts, for launch_router_stats.
// order (may be null): [T][E] bytes, every token's experts in preference order.
hipError_t launch_router(int dtype, const void* X, const void* Wg, const float* bias, int T, int d, int E, int k,
                         int32_t* ids, float* w, void* scratch, hipStream_t stream, bool select = true,
                         float inv_tau = 1.f, float* prob_sum = nullptr, uint8_t* order = nullptr);

// The load-balancing statistics from launch_router's prob_sum (at the start
// of a router_stats_scratch_bytes(T, E) scratch, whose rest holds the block
// partials): prob_mean[E], sel_freq[E] and aux[1] (E * their dot product).
size_t router_stats_scratch_bytes(int T, int E);
hipError_t launch_router_stats(float* prob_sum, const int32_t* ids, int T, int E, int k, float* prob_mean,
                               float* sel_freq, float* aux, hipStream_t stream);
// Where the K-split partial logits live in the router scratch ([nsplit][T][E]
// float); partial == nullptr when the router runs in one pass.
struct RouterSplit {
  const float* partial;
  int nsplit;
};
RouterSplit router_split(int T, int d, int E, int dtype, void* scratch);

// Xp == nullptr computes counts, offsets, perm and inv_perm only (for an
// expert GEMM that gathers the token rows itself).
hipError_t launch_dispatch(int dtype, const int32_t* ids, const void* X, int T, int d, int E, int k, int capacity,
                           int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv_perm, void* Xp,
                           const DispatchScratch& scratch, hipStream_t stream);

// The capacity dispatch with the pairs over capacity rerouted to their
// token's next-best expert with room (order: [T][E] preference order from
// launch_router); scratch carved with reroute = true.  capacity < 0: the
// plain dispatch.
hipError_t launch_dispatch_reroute(int dtype, const int32_t* ids, const uint8_t* order, const void* X, int T, int d,
                                   int E, int k, int capacity, int32_t* counts, int32_t* offsets, int32_t* perm,
                                   int32_t* inv_perm, void* Xp, const DispatchScratch& scratch, hipStream_t stream);

// Small batches (the single-block dispatch: T <= 256, k <= 8) with a K-split
// router: one block sums the partial logits, selects the top-k (writing ids
// and weights) and runs the whole dispatch.  Same results as the router's
// own selection followed by launch_dispatch.
bool dispatch_is_single_block(int T, int k);
hipError_t launch_topk_dispatch_small(int dtype, const float* partial, int nsplit, const float* bias, int32_t* ids,
                                      float* w, const void* X, int T, int d, int E, int k, int capacity,
                                      int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv_perm, void* Xp,
                                      hipStream_t stream);

// C[r, :] = act(A[r, :] . B[e]^T) for the rows r of each expert segment.
// A: [rows, K]; B: [E, N, K]; C: [rows, N]; rows bounded by max_rows.
// max_tokens_per_expert is a hint that picks the kernel (the few-rows
// kernels for decode shapes); any row count is computed correctly.
hipError_t launch_grouped_gemm(int dtype, bool gelu, const void* A, const void* B, void* C,
                               const int32_t* offsets, int E, int N, int K, int max_rows,
                               int max_tokens_per_expert, hipStream_t stream);

// The same product with the rows of A gathered: row r of the expert-ordered
// operand is X[gidx[r] / gdiv], X: [src_rows, K] (gidx = the dispatch
// permutation and gdiv = k read each pair's token row).  Only where
// grouped_gemm_gathers() holds, i.e. where launch_grouped_gemm runs its
// 256x256 kernel or its decode (few-rows, whole-line) kernel and X fits
// 32-bit buffer offsets; max_tokens_per_expert, rows (the pairs the operand
// can hold, max_rows of the launch) and E pick the kernel as there.
bool grouped_gemm_gathers(int dtype, int K, int N, int max_tokens_per_expert, int src_rows, int rows, int E);
hipError_t launch_grouped_gemm_gather(bool gelu, const void* X, int src_rows, const int32_t* gidx, int gdiv,
                                      const void* B, void* C, const int32_t* offsets, int E, int N, int K,
                                      int max_rows, int max_tokens_per_expert, hipStream_t stream);

hipError_t launch_combine(int dtype, const void* Yp, const int32_t* inv_perm, const float* topk_w, void* out, int T,
                          int d, int k, hipStream_t stream);

int device_cu_count();

}  // namespace moe
