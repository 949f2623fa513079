/*
 * moe.h -- C ABI of the sparse Mixture-of-Experts FFN layer forward pass on
 * one MI355X (gfx950) holding all experts.
 *
 * The layer, as the source pages state it:
 *   router   : logits = X W_g (+ b); softmax over the E experts; top-k; the k
 *              weights renormalised to sum to 1
 *              ["Qwen2-MoE代码解析：MoE架构原理、工程实现与部署避坑指南"
 *               (jsqmd.com/news/1061813) §3.1; Qwen2-MoE walk-through
 *               (mlqm.cn/news/48291) §3.2, steps 1-2]
 *   dispatch : (token, slot) pairs grouped by expert; with an expert
 *              capacity C, pairs beyond C per expert are dropped
 *              [jsqmd §3.1 detail 3, §3.4; mlqm §2.2 (C = ceil(T/E)*k);
 *               "GPT-4 activates 2%" article (wmrh.cn/news/106769) §2.2]
 *   experts  : per expert Linear -> GELU -> Linear [mlqm §2.2; wmrh §2.2]
 *   combine  : weighted sum of each token's k expert outputs
 *              [jsqmd §3.1 detail 2]
 *
 * Conventions shared by every entry point
 *   - Pointers are DEVICE pointers unless stated.  The caller owns every
 *     buffer; the library never allocates or frees device memory.
 *   - Row-major layouts.  X, out: [T, d].  W_g: [d, E].  Expert weights use
 *     the nn.Linear [out, in] layout: W1: [E, F, d], W2: [E, d, F].
 *     Intermediates Xp, Yp: [T*k, d] (rows past N unused), H: [T*k, F].
 *   - Element type of X, W_g, W1, W2, Xp, H, Yp and out is cfg->dtype
 *     (MOE_F32 = float, MOE_BF16 = bfloat16 bit patterns).  gate_bias and
 *     topk_w are float; ids, counts, offsets, perm and inv_perm are int32.
 *   - Accumulation is fp32; GELU is the tanh form
 *     0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))).
 *   - Every call only enqueues work on `stream` (a hipStream_t; NULL = the
 *     null stream) and never synchronises or reads results back.  Buffers must
 *     stay valid until the stream has run the work.
 *   - Arguments are checked on the host before anything is enqueued; a bad
 *     argument returns an error and enqueues nothing.  A HIP launch failure
 *     returns MOE_ERR_HIP (work enqueued before it may have run).
 *   - Calls that share a workspace or outputs on different streams race.
 *
 * Limits: 1 <= E <= 64; 1 <= k <= E; d and F positive multiples of 64;
 * T >= 0 (T = 0 is a no-op); T*k*max(d, F) < 2^62 elements.
 * expert_capacity < 0 selects dropless routing; C >= 0 keeps at most C pairs
 * per expert (C = 0 drops every pair and out is all zeros).
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,        /* null pointer, T < 0, k outside [1, E], bad dtype ... */
  MOE_ERR_UNSUPPORTED = 2,        /* E > 64, d or F not a multiple of 64 */
  MOE_ERR_WORKSPACE_TOO_SMALL = 3,
  MOE_ERR_HIP = 4                 /* a HIP runtime call or kernel launch failed */
} moe_status;

typedef enum moe_dtype { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* The layer's shape.  num_experts / num_experts_per_tok / expert_capacity are
 * the configuration fields named in jsqmd §2.2 and mlqm §2.2.  Host pointer. */
typedef struct moe_config {
  int32_t num_tokens;          /* T = batch * seq, tokens flattened           */
  int32_t hidden_size;         /* d                                           */
  int32_t intermediate_size;   /* F, expert FFN inner size                    */
  int32_t num_experts;         /* E                                           */
  int32_t num_experts_per_tok; /* k                                           */
  int32_t expert_capacity;     /* C; < 0: dropless                            */
  int32_t dtype;               /* moe_dtype of X, weights, out, intermediates */
} moe_config;

/* Which entry point a workspace is sized for. */
typedef enum moe_op {
  MOE_OP_DISPATCH = 0,   /* moe_dispatch                                  */
  MOE_OP_EXPERT_FFN = 1, /* moe_expert_ffn (holds H)                      */
  MOE_OP_FORWARD = 2,    /* moe_forward (all scratch + Xp + H + Yp)       */
  MOE_OP_ROUTE = 3,      /* moe_route (partial logits when K is split)    */
  MOE_OP_ROUTE_STATS = 4, /* moe_route_stats (as moe_route + per-tile sums) */
  MOE_OP_DISPATCH_REROUTE = 5, /* moe_dispatch_reroute (as moe_dispatch + ids) */
  MOE_OP_FORWARD_REROUTE = 6   /* moe_forward_reroute                         */
} moe_op;

/* Human-readable name of a status.  Static string; never NULL. */
const char* moe_status_string(moe_status status);

/* Library build description (static string). */
const char* moe_version(void);

/* Host only: the expert capacity from a capacity factor [jsqmd §3.4]:
 * with T = batch * seq_len and tokens_per_expert = T / E (the mean tokens per
 * expert), C = floor(tokens_per_expert * k * capacity_factor / E), at most T;
 * in autoregressive decoding (seq_len == 1) C = min(512, 2 * batch) instead
 * [jsqmd §5.2].  The result goes into moe_config.expert_capacity.
 * Errors: INVALID_ARG for batch < 0, seq_len < 0, E < 1, k outside [1, E],
 * a factor that is not finite and > 0, a null capacity, or C beyond int32. */
moe_status moe_capacity_from_factor(int32_t batch, int32_t seq_len, int32_t num_experts,
                                    int32_t num_experts_per_tok, double capacity_factor,
                                    int32_t* capacity);

/* Bytes of device workspace `op` needs for `cfg` (host only, no HIP call).
 * *bytes receives the size; 0 is possible.  Errors: INVALID_ARG, UNSUPPORTED. */
moe_status moe_workspace_size(const moe_config* cfg, int32_t op, size_t* bytes);

/* Router: gate projection, softmax over E, top-k, renormalisation
 * [jsqmd §3.1; mlqm §3.2 steps 1-2].
 *   X [T, d], Wg [d, E] (dtype), gate_bias [E] float or NULL (a per-expert
 *   logit bias, the domain bias of mlqm §6).
 *   topk_ids [T, k] int32 out: slot 0 holds the most probable expert; slots in
 *   descending probability; equal logits go to the lower expert id.  A NaN
 *   or -inf logit ranks as the lowest finite value, so the k ids are always
 *   distinct experts.
 *   topk_w [T, k] float out: p_s / sum_j p_j over the k selected experts.
 *   ws / ws_bytes: workspace of moe_workspace_size(cfg, MOE_OP_ROUTE) bytes:
 *   the gate transposed to [16*ceil(E/16), d] and, when T is small (the gate
 *   projection is then split over K across blocks), the partial logits. */
moe_status moe_route(const moe_config* cfg, const void* X, const void* Wg,
                     const float* gate_bias, int32_t* topk_ids, float* topk_w,
                     void* ws, size_t ws_bytes, void* stream);

/* Router with a temperature, and the load-balancing statistics of the batch
 * [jsqmd §3.3, its load_balancing_loss listing; the temperature of the
 * router softmax: wmrh §5.2].  Same outputs as moe_route, the weights now
 * exp((l_s - l_0)/tau) / sum_j exp((l_j - l_0)/tau) over the selected logits
 * (tau = 1 gives moe_route's bits; the selection does not depend on tau), and
 *   prob_mean [E] float out: mean over the T tokens of softmax(logits / tau)
 *   sel_freq  [E] float out: fraction of the tokens whose top-k holds expert e
 *   aux       [1] float out: E * sum_e prob_mean[e] * sel_freq[e]
 *                            (k for balanced routing, E for a collapse at k = 1)
 * All three are device pointers; the sums run in a fixed order (deterministic).
 * temperature: finite and > 0, else INVALID_ARG.  T = 0 writes nothing.
 * ws / ws_bytes: moe_workspace_size(cfg, MOE_OP_ROUTE_STATS). */
moe_status moe_route_stats(const moe_config* cfg, const void* X, const void* Wg,
                           const float* gate_bias, float temperature, int32_t* topk_ids,
                           float* topk_w, float* prob_mean, float* sel_freq, float* aux,
                           void* ws, size_t ws_bytes, void* stream);

/* Dispatcher: group the (token, slot) pairs by expert
 * [jsqmd §3.1 detail 3; wmrh §2.2; capacity: jsqmd §3.4, mlqm §2.2].
 *   topk_ids [T, k] int32 in; X [T, d] in.
 *   expert_counts [E] out: pairs routed to each expert (before any drop).
 *   expert_offsets [E+1] out: exclusive scan of the kept counts; expert e's
 *     rows are [offsets[e], offsets[e+1]); offsets[E] = N, the kept pairs.
 *   perm [T*k] out: row r < N holds the pair id t*k+s; rows >= N hold -1.
 *     Rows are ordered by (expert, token, slot) -- stable by token.
 *   inv_perm [T*k] out: the row of pair t*k+s, or -1 if the pair was dropped.
 *   Xp [T*k, d] out: row r = X[perm[r] / k] for r < N; rows >= N untouched.
 *     Xp may be NULL: then only counts, offsets, perm and inv_perm are
 *     written (for moe_expert_up_gather, which reads X through perm).
 *   Capacity (C >= 0): each expert keeps its pairs in (slot, token) order up
 *   to C; the rest are dropped.  Ids outside [0, E) are treated as dropped
 *   and not counted.
 *   ws / ws_bytes: workspace of moe_workspace_size(cfg, MOE_OP_DISPATCH). */
moe_status moe_dispatch(const moe_config* cfg, const int32_t* topk_ids, const void* X,
                        int32_t* expert_counts, int32_t* expert_offsets, int32_t* perm,
                        int32_t* inv_perm, void* Xp, void* ws, size_t ws_bytes, void* stream);

/* Expert up-projection: H[r] = gelu(W1[e] Xp[r]) for every row r of expert
 * e's segment [offsets[e], offsets[e+1]) (the first Linear and the GELU of
 * mlqm §2.2).  Xp [T*k, d], W1 [E, F, d] in; H [T*k, F] out (rows >= N
 * untouched). expert_offsets [E+1] is read on the device. */
moe_status moe_expert_up(const moe_config* cfg, const void* Xp, const int32_t* expert_offsets,
                         const void* W1, void* H, void* stream);

/* The up-projection with the dispatch's row copy folded in: H[r] =
 * gelu(W1[e] X[perm[r] / k]) for every row r of expert e's segment -- the
 * same values, bit for bit, as moe_dispatch's Xp followed by moe_expert_up.
 * X [T, d], perm [T*k] (from moe_dispatch), expert_offsets [E+1], W1 [E, F, d]
 * in; H [T*k, F] out (rows >= N untouched).  Entries of perm in an expert's
 * segment that name no token of X contribute zero rows.
 * Errors: UNSUPPORTED unless moe_expert_up_gather_supported says 1. */
moe_status moe_expert_up_gather(const moe_config* cfg, const void* X, const int32_t* perm,
                                const int32_t* expert_offsets, const void* W1, void* H,
                                void* stream);

/* Host only: *supported = 1 if moe_expert_up_gather runs for cfg, else 0:
 * bf16, T*d*2 < 2^31 bytes, and either more than 64 pairs per expert possible
 * (min(T, C) > 64) or at most 64 with d a multiple of 128 and F a multiple
 * of 8.  moe_forward then gathers too and leaves the Xp
 * part of its workspace unwritten. */
moe_status moe_expert_up_gather_supported(const moe_config* cfg, int32_t* supported);

/* Expert down-projection: Yp[r] = W2[e] H[r] for every row r of expert e's
 * segment [offsets[e], offsets[e+1]): the second Linear of each expert's
 * Linear -> GELU -> Linear FFN [mlqm §2.2: every expert is a standard FFN;
 * wmrh §2.2: Linear-GELU-Linear], run only on the rows dispatched to it
 * [mlqm §3.2 step 4].  H [T*k, F], W2 [E, d, F] in; Yp [T*k, d] out (rows
 * >= N untouched).  expert_offsets [E+1] is read on the device. */
moe_status moe_expert_down(const moe_config* cfg, const void* H, const int32_t* expert_offsets,
                           const void* W2, void* Yp, void* stream);

/* Both expert projections: Yp[r] = W2[e] gelu(W1[e] Xp[r]), the whole
 * expert FFN of every dispatched row [mlqm §2.2; wmrh §2.2: Linear-GELU-
 * Linear; mlqm §3.2 step 4: each expert runs on its own tokens].  H lives in
 * ws (moe_workspace_size(cfg, MOE_OP_EXPERT_FFN)). */
moe_status moe_expert_ffn(const moe_config* cfg, const void* Xp, const int32_t* expert_offsets,
                          const void* W1, const void* W2, void* Yp, void* ws, size_t ws_bytes,
                          void* stream);

/* Combine: out[t] = sum over kept slots s of topk_w[t, s] * Yp[inv_perm[t*k+s]]
 * [jsqmd §3.1 detail 2], accumulated in fp32, stored in dtype; a token with
 * no kept slot gets zeros.  Yp [T*k, d], inv_perm [T*k], topk_w [T, k] in;
 * out [T, d] out. */
moe_status moe_combine(const moe_config* cfg, const void* Yp, const int32_t* inv_perm,
                       const float* topk_w, void* out, void* stream);

/* The whole layer [mlqm §3.2 steps 1-5]: route, dispatch, expert FFN,
 * combine.  The routing and dispatch results are written to the caller's
 * buffers (same meaning as above) so that every stage can be checked; Xp, H
 * and Yp live in ws (moe_workspace_size(cfg, MOE_OP_FORWARD)).  Where
 * moe_expert_up_gather_supported holds, the up-projection reads X through
 * perm and Xp is not written. */
moe_status moe_forward(const moe_config* cfg, const void* X, const void* Wg,
                       const float* gate_bias, const void* W1, const void* W2, void* out,
                       int32_t* topk_ids, float* topk_w, int32_t* expert_counts,
                       int32_t* expert_offsets, int32_t* perm, int32_t* inv_perm,
                       void* ws, size_t ws_bytes, void* stream);

/* Router that also returns every token's full preference order, the list
 * the over-capacity rerouting below walks [jsqmd §3.1 (softmax, top-k);
 * §3.4 (drop_tokens = False)].  Same topk_ids and topk_w, bit for bit, as
 * moe_route, and
 *   expert_order [T, E] uint8 out: row t holds all E expert ids of token t
 *   in descending probability, equal logits to the lower id; its first k
 *   entries equal topk_ids[t].
 * ws / ws_bytes: as moe_route (moe_workspace_size(cfg, MOE_OP_ROUTE)). */
moe_status moe_route_ranked(const moe_config* cfg, const void* X, const void* Wg,
                            const float* gate_bias, int32_t* topk_ids, float* topk_w,
                            uint8_t* expert_order, void* ws, size_t ws_bytes, void* stream);

/* Dispatch with over-capacity pairs rerouted instead of dropped [jsqmd §3.4:
 * with drop_tokens = False a token over an expert's capacity goes to a
 * next-best expert].  The capacity cut of moe_dispatch stands (the pairs it
 * keeps do not move).  The pairs it drops are then taken in the same
 * (slot, token) priority; each moves to the first expert of its token's
 * expert_order past position k-1 that holds fewer than C pairs and that the
 * token does not already use (an earlier slot may have moved there); a pair
 * that finds none stays dropped.  Weights are unchanged: a moved pair still
 * carries topk_w[t, s].
 *   topk_ids [T, k], expert_order [T, E] (from moe_route_ranked) in.  Each
 *   row of expert_order must be a permutation of [0, E) whose first k
 *   entries are the token's ids; a byte >= E is never taken as a
 *   destination.
 *   Outputs as moe_dispatch, under the final assignment: expert_counts holds
 *   the routed counts of topk_ids (before the cut); offsets, perm, inv_perm
 *   and Xp group the computed pairs by the expert they end at, rows ordered
 *   by (expert, token).  The expert of a computed pair is the e with
 *   offsets[e] <= inv_perm[t*k+s] < offsets[e+1].
 *   expert_capacity < 0: nothing overflows, the result is moe_dispatch's.
 *   ws / ws_bytes: moe_workspace_size(cfg, MOE_OP_DISPATCH_REROUTE) bytes.
 * The placement runs in one workgroup and takes time in proportion to the
 * dropped pairs. */
moe_status moe_dispatch_reroute(const moe_config* cfg, const int32_t* topk_ids,
                                const uint8_t* expert_order, const void* X,
                                int32_t* expert_counts, int32_t* expert_offsets, int32_t* perm,
                                int32_t* inv_perm, void* Xp, void* ws, size_t ws_bytes,
                                void* stream);

/* The whole layer with over-capacity rerouting: moe_route_ranked,
 * moe_dispatch_reroute, the expert FFN and the combine, with the
 * intermediates in ws (moe_workspace_size(cfg, MOE_OP_FORWARD_REROUTE)).
 * Arguments as moe_forward plus expert_order [T, E] uint8 out. */
moe_status moe_forward_reroute(const moe_config* cfg, const void* X, const void* Wg,
                               const float* gate_bias, const void* W1, const void* W2, void* out,
                               int32_t* topk_ids, float* topk_w, uint8_t* expert_order,
                               int32_t* expert_counts, int32_t* expert_offsets, int32_t* perm,
                               int32_t* inv_perm, void* ws, size_t ws_bytes, void* stream);

/* Bytes of the device array moe_forward_noalloc uses as its workspace (per GPU). */
#define MOE_NOALLOC_MAX_WORKSPACE_BYTES ((size_t)64 << 20)

/* moe_forward without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation.  Same arguments, results and bits as moe_forward
 * minus ws / ws_bytes: the workspace is a device array inside the library,
 * MOE_NOALLOC_MAX_WORKSPACE_BYTES (64 MiB) on every GPU the library runs on,
 * held until the process ends.  The call allocates nothing (no hipMalloc,
 * no allocating library routine); its first call on a device looks up that
 * device's copy of the array.
 * Limit: moe_workspace_size(cfg, MOE_OP_FORWARD) must be at most
 * MOE_NOALLOC_MAX_WORKSPACE_BYTES (decode-sized batches and small prefills),
 * else MOE_ERR_WORKSPACE_TOO_SMALL and nothing is enqueued.
 * Every call on one GPU shares that GPU's array and leaves its contents to
 * the next call: calls that overlap on one GPU (different streams or host
 * threads without ordering between them) race. */
moe_status moe_forward_noalloc(const moe_config* cfg, const void* X, const void* Wg,
                               const float* gate_bias, const void* W1, const void* W2, void* out,
                               int32_t* topk_ids, float* topk_w, int32_t* expert_counts,
                               int32_t* expert_offsets, int32_t* perm, int32_t* inv_perm,
                               void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
