// Top-k selection and renormalisation of router logits, shared by the
// router kernels and the single-block small-batch dispatch.
//
// Method ("Qwen2-MoE代码解析" (jsqmd.com/news/1061813) §3.1; Qwen2-MoE
// walk-through (mlqm.cn/news/48291) §3.2 step 2): the k largest softmax
// probabilities are those of the k largest logits (softmax is monotone), and
// after renormalisation p_s / sum_j p_j = exp(l_s - l_0) / sum_j exp(l_j - l_0)
// over the selected logits (l_0 the largest), so the softmax denominator is
// never formed.  Equal logits go to the lower expert id.
#pragma once

#include "common.hpp"

namespace moe {

__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

// A (logit, expert) pair as a 64-bit key whose unsigned order is better()'s:
// the high word is the logit's bit pattern mapped so that unsigned order is
// float order (negative zero taken as positive zero, which better() treats
// as equal), the low word is 63 - expert, so the lower id wins a tie.  Valid
// for every non-NaN logit, infinities included, and expert ids below 64.
__device__ __forceinline__ uint32_t ordered_bits(float v) {
  uint32_t u = __builtin_bit_cast(uint32_t, v);
  u = u == 0x80000000u ? 0u : u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ uint64_t pair_key(uint32_t ordered, int e) {
  return (static_cast<uint64_t>(ordered) << 32) | static_cast<uint32_t>(63 - e);
}
__device__ __forceinline__ float key_value(uint64_t key) {
  const uint32_t o = static_cast<uint32_t>(key >> 32);
  return __builtin_bit_cast(float, (o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}
__device__ __forceinline__ int key_expert(uint64_t key) { return 63 - static_cast<int>(static_cast<uint32_t>(key)); }

// One step of a 16-lane arg-max over four keys at once: take the keys of the
// lane that DPP control kCtrl names in this lane's row of 16, keep the larger.
// DPP moves are plain VALU operations (no LDS round trip, unlike a lane
// shuffle), and the four independent chains hide each other's latency.
template <int kCtrl>
__device__ __forceinline__ void argmax_dpp_step(uint64_t (&b)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = __builtin_amdgcn_update_dpp(0, static_cast<uint32_t>(b[i]), kCtrl, 0xF, 0xF, false);
    const uint32_t hi = __builtin_amdgcn_update_dpp(0, static_cast<uint32_t>(b[i] >> 32), kCtrl, 0xF, 0xF, false);
    const uint64_t o = (static_cast<uint64_t>(hi) << 32) | lo;
    b[i] = o > b[i] ? o : b[i];
  }
}

// Sum and max over each row of 16 lanes, left in every lane of the row (the
// same pairing as argmax16: every step pairs each lane with one holding the
// complementary part of the row).
template <int kCtrl>
__device__ __forceinline__ float dpp_move(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl, 0xF, 0xF, false));
}
__device__ __forceinline__ float sum16(float v) {
  v += dpp_move<0xB1>(v);
  v += dpp_move<0x4E>(v);
  v += dpp_move<0x141>(v);
  v += dpp_move<0x140>(v);
  return v;
}
__device__ __forceinline__ float max16(float v) {
  v = fmaxf(v, dpp_move<0xB1>(v));
  v = fmaxf(v, dpp_move<0x4E>(v));
  v = fmaxf(v, dpp_move<0x141>(v));
  v = fmaxf(v, dpp_move<0x140>(v));
  return v;
}

// Arg-max over each row of 16 lanes, left in every lane of the row: pairs
// (quad_perm 1,0,3,2), quads (quad_perm 2,3,0,1), then the two quads of each
// half-row (row_half_mirror: lane i with 7-i) and the two halves
// (row_mirror: lane i with 15-i).  The key order is total, so the result
// does not depend on the pairing.
__device__ __forceinline__ void argmax16(uint64_t (&b)[4]) {
  argmax_dpp_step<0xB1>(b);
  argmax_dpp_step<0x4E>(b);
  argmax_dpp_step<0x141>(b);
  argmax_dpp_step<0x140>(b);
}

// Step R of the places in a 16-lane row: compare this lane's NT values with
// those of the lane that row rotation R brings here (its lane index comes
// along the same rotation, so the direction of the rotation does not matter).
template <int NT, int R>
__device__ __forceinline__ void place_steps(const f32x4_t (&acc)[NT], int i, int n, int (&place)[NT]) {
  if constexpr (R < 16) {
    const int n2 = R == 0 ? n : __builtin_amdgcn_update_dpp(0, n, 0x120 + R, 0xF, 0xF, false);
#pragma unroll
    for (int t2 = 0; t2 < NT; ++t2) {
      const float v2 = R == 0 ? acc[t2][i] : dpp_move<0x120 + R>(acc[t2][i]);
#pragma unroll
      for (int t = 0; t < NT; ++t) place[t] += better(v2, t2 * 16 + n2, acc[t][i], t * 16 + n) ? 1 : 0;
    }
    place_steps<NT, R + 1>(acc, i, n, place);
  }
}

// Top-k + renormalisation for one 16-token row tile held in MFMA C layout:
// acc[t][i] is the logit of token row (lane>>4)*4+i and expert t*16+(lane&15).
// sel_val / sel_id: LDS scratch [16][k] of the calling wave.
// inv_tau: 1 / router temperature.  The selection is on the logits (the
// softmax at any temperature > 0 is monotone); the weights are
// exp((l_s - l_0) * inv_tau) / sum_j exp((l_j - l_0) * inv_tau) over the
// selected logits ("Qwen2-MoE代码解析" §3.1; the temperature: "GPT-4
// activates 2%" article §5.2).  inv_tau = 1 gives the same bits as no
// temperature.
// prob_sum (may be null): row tok0/16 of a [ceil(T/16)][2E] array receives,
// per expert, the sum over the tile's tokens of the full router
// probability softmax(logits * inv_tau), then the number of the tile's
// tokens that select the expert -- the per-tile parts of the load-balancing
// statistics ("Qwen2-MoE代码解析" §3.3).
// order (may be null): [T][E] bytes; row t receives all E experts of token t
// in preference order (the order of better(), so its first k entries are
// the selected ids), the list the over-capacity rerouting walks
// ("Qwen2-MoE代码解析" §3.4).
template <int NT>
__device__ __forceinline__ void topk_tile(f32x4_t (&acc)[NT], const float* __restrict__ bias, int E, int k,
                                          int tok0, int T_tokens, float* sel_val, int* sel_id,
                                          int32_t* __restrict__ topk_ids, float* __restrict__ topk_w,
                                          float inv_tau = 1.f, float* __restrict__ prob_sum = nullptr,
                                          uint8_t* __restrict__ order = nullptr) {
  const int lane = threadIdx.x % kWave;
  const int n = lane & 15;
  const int grp = lane >> 4;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int e = t * 16 + n;
    const float b = (e < E && bias != nullptr) ? bias[e] : 0.f;
    // Live experts hold values in [-FLT_MAX, +inf]: a NaN or -inf logit
    // becomes -FLT_MAX.  -inf then marks only the padding lanes (e >= E)
    // and the experts the selection below has taken, so better() is a total
    // order on every input and each round takes a new expert: the k ids are
    // distinct and the preference order is a permutation of the E experts
    // even for non-finite hidden states.  Finite logits are unchanged.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float v = acc[t][i] + b;
      acc[t][i] = (e < E) ? (__builtin_isnan(v) ? -3.402823466e38f : fmaxf(v, -3.402823466e38f)) : -INFINITY;
    }
  }
  // Load-balancing statistics of the tile (prob_sum != null): col[t] sums the
  // full softmax probability of expert t*16+n over the tile's live tokens,
  // cnt[t] counts the tokens that select it.
  const bool stats = prob_sum != nullptr && tok0 < T_tokens;  // a tile wholly past T has no row
  float col[NT], cnt[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) col[t] = cnt[t] = 0.f;
  if (stats) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float m = acc[0][i];
#pragma unroll
      for (int t = 1; t < NT; ++t) m = fmaxf(m, acc[t][i]);
      m = max16(m);
      float z[NT], den = 0.f;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        z[t] = t * 16 + n < E ? expf((acc[t][i] - m) * inv_tau) : 0.f;
        den += z[t];
      }
      den = sum16(den);
      const bool live = tok0 + grp * 4 + i < T_tokens;
#pragma unroll
      for (int t = 0; t < NT; ++t) col[t] += live ? z[t] / den : 0.f;
    }
  }
  if (order != nullptr) {
    // Each expert's place in its token's order: the number of experts of
    // the row that beat it (better() is a total order, so the places are a
    // permutation).  The 16 lanes of a row see each other's values through
    // the 15 row rotations (DPP row_ror), 16 steps instead of E arg-max rounds.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int place[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) place[t] = 0;
      place_steps<NT, 0>(acc, i, n, place);
      const int tok = tok0 + grp * 4 + i;
      if (tok < T_tokens) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
          if (t * 16 + n < E) order[static_cast<int64_t>(tok) * E + place[t]] = static_cast<uint8_t>(t * 16 + n);
      }
    }
  }
  // k rounds on the pair keys: each round takes every row's best remaining
  // expert and gives it the key of a -inf logit (what the padding lanes
  // hold), so the next round finds the next one.  k <= E live experts, so a
  // round never takes a padding lane.  Only the high words are kept: the low
  // word of lane n's entry t is 63 - (16t + n) in every row.
  uint32_t hw[NT][4];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) hw[t][i] = ordered_bits(acc[t][i]);
  const uint32_t taken_hw = ordered_bits(-INFINITY);
#pragma unroll 1
  for (int s = 0; s < k; ++s) {
    uint64_t best[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // The lane's own best: the largest high word, the lowest t on a tie.
      uint32_t bh = hw[0][i];
      int be = n;
#pragma unroll
      for (int t = 1; t < NT; ++t) {
        const bool gt = hw[t][i] > bh;
        bh = gt ? hw[t][i] : bh;
        be = gt ? t * 16 + n : be;
      }
      best[i] = pair_key(bh, be);
    }
    argmax16(best);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int bi = key_expert(best[i]);
      const bool live = tok0 + grp * 4 + i < T_tokens;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const bool taken = t * 16 + n == bi;
        hw[t][i] = taken ? taken_hw : hw[t][i];
        cnt[t] += live && taken ? 1.f : 0.f;
      }
      if (n == 0) {
        sel_val[(grp * 4 + i) * kMaxExperts + s] = key_value(best[i]);
        sel_id[(grp * 4 + i) * kMaxExperts + s] = bi;
      }
    }
  }
  if (stats) {
    // Row tok0/16 of prob_sum ([ceil(T/16)][2E]): probability sums, then counts.
    float* row = prob_sum + static_cast<int64_t>(tok0 / 16) * 2 * E;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      float c = col[t], q = cnt[t];
      c += __shfl_xor(c, 16);
      c += __shfl_xor(c, 32);
      q += __shfl_xor(q, 16);
      q += __shfl_xor(q, 32);
      const int e = t * 16 + n;
      if (grp == 0 && e < E) {
        row[e] = c;
        row[E + e] = q;
      }
    }
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  for (int idx = lane; idx < 16 * k; idx += kWave) {
    const int row = idx / k;
    const int s = idx % k;
    const int tok = tok0 + row;
    if (tok >= T_tokens) continue;
    const float* v = sel_val + row * kMaxExperts;
    const float l0 = v[0];
    float den = 0.f;
    for (int j = 0; j < k; ++j) den += expf((v[j] - l0) * inv_tau);
    const int64_t o = static_cast<int64_t>(tok) * k + s;
    topk_ids[o] = sel_id[row * kMaxExperts + s];
    topk_w[o] = expf((v[s] - l0) * inv_tau) / den;
  }
}

// Sum the K-split partial logits of tokens tok0 .. tok0+15 in split order into
// logit[16][kMaxExperts] (LDS), then select with wave 0.  Called by a whole
// block of kThreads threads (a multiple of 64: each thread sums the entries
// (token, expert) of its expert for every kThreads/64-th token, 8 loads in
// flight); the caller synchronises the block before and after.
template <int NT, int kThreads = 1024>
__device__ __forceinline__ void topk_from_partials(const float* __restrict__ partial, int nsplit,
                                                   const float* __restrict__ bias, int T_tokens, int E, int k,
                                                   int tok0, float (*logit)[kMaxExperts], float* sel_val,
                                                   int* sel_id, int32_t* __restrict__ topk_ids,
                                                   float* __restrict__ topk_w, float inv_tau = 1.f,
                                                   float* __restrict__ prob_sum = nullptr,
                                                   uint8_t* __restrict__ order = nullptr) {
  static_assert(kThreads % kMaxExperts == 0 && kThreads <= 16 * kMaxExperts, "whole rows of (token, expert) entries");
  const int e = threadIdx.x % kMaxExperts;
  for (int r = threadIdx.x / kMaxExperts; r < 16; r += kThreads / kMaxExperts) {
    const int tok = tok0 + r;
    float v = 0.f;
    if (tok < T_tokens && e < E) {
      const float* src = partial + static_cast<int64_t>(tok) * E + e;
      const int64_t stride = static_cast<int64_t>(T_tokens) * E;
      for (int s0 = 0; s0 < nsplit; s0 += 8) {
        float a[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) a[j] = (s0 + j < nsplit) ? src[(s0 + j) * stride] : 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) v += a[j];  // split order
      }
    }
    logit[r][e] = v;
  }
  __syncthreads();
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    const int n = lane & 15;
    const int grp = lane >> 4;
    f32x4_t acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int e = t * 16 + n;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[t][i] = (e < E) ? logit[grp * 4 + i][e] : 0.f;
    }
    topk_tile<NT>(acc, bias, E, k, tok0, T_tokens, sel_val, sel_id, topk_ids, topk_w, inv_tau, prob_sum, order);
  }
}

}  // namespace moe
