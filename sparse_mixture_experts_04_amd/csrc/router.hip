// Router kernels: gate projection on MFMA, softmax-free top-k selection on the
// logits with 16-lane shuffle reductions, and renormalised weights.
//
// Method ("Qwen2-MoE代码解析" (jsqmd.com/news/1061813) §3.1; Qwen2-MoE
// walk-through (mlqm.cn/news/48291) §3.2 steps 1-2): logits = X W_g (+ b),
// p = softmax(logits), the k largest p are selected and divided by their sum.
// Softmax is monotone, so the k largest logits are the k largest p, and
//   p_s / sum_j p_j = exp(l_s - l_0) / sum_j exp(l_j - l_0)
// over the selected logits l_j (l_0 the largest): the full softmax
// denominator cancels and never has to be formed.
//
// Work layout.  W_g ([d, E], experts contiguous) is first transposed into the
// workspace as WgT [16*ceil(E/16)][d] (rows past E zero), so that MFMA
// B fragments are 16-byte loads of 8 consecutive k.  A block then owns 32
// tokens (two 16-row MFMA tiles) and every expert (up to four 16-column
// tiles) over a range of K; each of its 4 waves streams a quarter of that
// range straight from global memory (X from HBM, WgT from L2), with no LDS
// staging and no block-wide sync inside the K loop, and the 4 partial logit
// tiles are summed in LDS.
// When there are too few token blocks to fill the GPU (decode), K is split
// across blocks: each writes partial logits to the workspace and a second
// kernel sums the splits in a fixed order and selects.  The reduction over K
// runs in a fixed order, so results are deterministic.
#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "topk.hpp"

namespace moe {
namespace {

constexpr int kRouterThreads = 256;               // 4 waves

// Temperature and load-balancing statistics of a routing call (see topk_tile).
struct RouteExtra {
  float inv_tau;
  float* prob_sum;
  uint8_t* order;  // [T][E] preference order of every token, or null
};
constexpr int kRouterTok = 32;                    // tokens per block: 2 row tiles of 16
constexpr int kRowTiles = kRouterTok / 16;
constexpr int kChunkBytes = 64;                   // K bytes per MFMA k-step per row (4 lane groups x 16 B)

// One 16-byte chunk of A (token row) and B (gate column) into a 16x16 tile.
template <typename T> struct RouterMma;
template <> struct RouterMma<uint16_t> {
  static __device__ __forceinline__ f32x4_t run(u32x4_t a, u32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
};
template <> struct RouterMma<float> {
  static __device__ __forceinline__ f32x4_t run(u32x4_t a, u32x4_t b, f32x4_t c) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[q]), __uint_as_float(b[q]), c, 0, 0, 0);
    return c;
  }
};

// WgT[e][k] = W_g[k][e] for e < E, 0 for E <= e < 16*NT.  One block per 32
// rows of k: the rows are read with 16-byte loads (a run of 32 rows of W_g is
// contiguous) and written back as 16-byte runs of 8 (bf16) or 4 (fp32) k.
template <typename T, int NT>
__global__ __launch_bounds__(256) void gate_transpose_kernel(const T* __restrict__ Wg, int d, int E,
                                                             T* __restrict__ WgT) {
  constexpr int kCols = NT * 16;
  constexpr int kRows = 32;
  constexpr int kPer16 = 16 / sizeof(T);
  __shared__ T tile[kRows][kCols + 2];
  const int k0 = blockIdx.x * kRows;
  const T* src = Wg + static_cast<int64_t>(k0) * E;  // kRows * E contiguous elements (d % 64 == 0)
  if (E % kPer16 == 0) {
    for (int v = threadIdx.x; v < kRows * E / kPer16; v += 256) {
      const u32x4_t x = ld16(src + v * kPer16);
      const T* xe = reinterpret_cast<const T*>(&x);
      const int flat = v * kPer16;
#pragma unroll
      for (int q = 0; q < kPer16; ++q) tile[(flat + q) / E][(flat + q) % E] = xe[q];
    }
  } else {
    for (int i = threadIdx.x; i < kRows * E; i += 256) tile[i / E][i % E] = src[i];
  }
  for (int i = threadIdx.x; i < kRows * (kCols - E); i += 256) tile[i / (kCols - E)][E + i % (kCols - E)] = T(0);
  __syncthreads();
  for (int i = threadIdx.x; i < kCols * (kRows / kPer16); i += 256) {
    const int e = i / (kRows / kPer16);
    const int c = i % (kRows / kPer16);
    u32x4_t v;
    T* ve = reinterpret_cast<T*>(&v);
#pragma unroll
    for (int q = 0; q < kPer16; ++q) ve[q] = tile[c * kPer16 + q][e];
    st16(WgT + static_cast<int64_t>(e) * d + k0 + c * kPer16, v);
  }
}

// B fragment of k-step `kstep` read straight from W_g [d, E]: lane (n, grp)
// gathers the kPer16 consecutive k of column col (used when only a few
// blocks run, so the transpose launch would cost more than the gathers).
template <typename T>
__device__ __forceinline__ u32x4_t gather_b(const T* __restrict__ Wg, int E, int col, int k0) {
  constexpr int kPer16 = 16 / sizeof(T);
  u32x4_t r;
  T* re = reinterpret_cast<T*>(&r);
#pragma unroll
  for (int q = 0; q < kPer16; ++q) re[q] = col < E ? Wg[static_cast<int64_t>(k0 + q) * E + col] : T(0);
  return r;
}

// Partial (or complete) logits of 32 tokens x all experts over K range
// [kbeg, kend) of split blockIdx.y.  partial == nullptr: finish with top-k.
// kDirect: B fragments gathered from W_g itself (WgT unused).
template <typename T, int NT, bool kDirect>
__global__ __launch_bounds__(kRouterThreads) void router_kernel(
    const T* __restrict__ X, const T* __restrict__ WgT, const T* __restrict__ Wg, const float* __restrict__ bias,
    int T_tokens, int d, int E, int k, int split_len, float* __restrict__ partial, int32_t* __restrict__ topk_ids,
    float* __restrict__ topk_w, float inv_tau, float* __restrict__ prob_sum, uint8_t* __restrict__ order) {
  constexpr int kStepElems = kChunkBytes / sizeof(T);  // K per k-step (32 bf16 / 16 fp32)
  __shared__ f32x4_t red[4][kRowTiles][NT][kWave];
  __shared__ float sel_val[2][16 * kMaxExperts];
  __shared__ int sel_id[2][16 * kMaxExperts];

  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int n = lane & 15;
  const int grp = lane >> 4;
  const int tok0 = blockIdx.x * kRouterTok;
  const int kbeg = blockIdx.y * split_len;
  const int kend = min(d, kbeg + split_len);

  // Row pointers of the two row tiles (rows past T repeat the last token; never stored).
  const unsigned char* xrow[kRowTiles];
#pragma unroll
  for (int r = 0; r < kRowTiles; ++r)
    xrow[r] = reinterpret_cast<const unsigned char*>(X + static_cast<int64_t>(min(tok0 + r * 16 + n, T_tokens - 1)) * d) +
              grp * 16;
  const unsigned char* wrow[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
    wrow[t] = kDirect ? nullptr
                      : reinterpret_cast<const unsigned char*>(WgT + static_cast<int64_t>(t * 16 + n) * d) + grp * 16;

  f32x4_t acc[kRowTiles][NT];
#pragma unroll
  for (int r = 0; r < kRowTiles; ++r)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[r][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // This wave's quarter of [kbeg, kend), in k-steps of kStepElems.
  const int nsteps = (kend - kbeg) / kStepElems;
  const int s_lo = wave * nsteps / 4;
  const int s_hi = (wave + 1) * nsteps / 4;
  constexpr int kUnroll = NT <= 2 ? 8 : 4;  // 16-byte loads in flight per lane: kUnroll * (2 + NT)
  int st = s_lo;
  for (; st + kUnroll <= s_hi; st += kUnroll) {
    u32x4_t a[kUnroll][kRowTiles], b[kUnroll][NT];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t off = static_cast<int64_t>(kbeg + (st + u) * kStepElems) * sizeof(T);
#pragma unroll
      for (int r = 0; r < kRowTiles; ++r) a[u][r] = ld16(xrow[r] + off);
#pragma unroll
      for (int t = 0; t < NT; ++t)
        b[u][t] = kDirect ? gather_b(Wg, E, t * 16 + n, kbeg + (st + u) * kStepElems + grp * (16 / sizeof(T)))
                          : ld16(wrow[t] + off);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int r = 0; r < kRowTiles; ++r) acc[r][t] = RouterMma<T>::run(a[u][r], b[u][t], acc[r][t]);
  }
  for (; st < s_hi; ++st) {
    const int64_t off = static_cast<int64_t>(kbeg + st * kStepElems) * sizeof(T);
    u32x4_t a[kRowTiles];
#pragma unroll
    for (int r = 0; r < kRowTiles; ++r) a[r] = ld16(xrow[r] + off);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const u32x4_t b = kDirect ? gather_b(Wg, E, t * 16 + n, kbeg + st * kStepElems + grp * (16 / sizeof(T)))
                                : ld16(wrow[t] + off);
#pragma unroll
      for (int r = 0; r < kRowTiles; ++r) acc[r][t] = RouterMma<T>::run(a[r], b, acc[r][t]);
    }
  }

  // Sum the 4 waves' partial tiles (fixed order: wave 0 + 1 + 2 + 3).
#pragma unroll
  for (int r = 0; r < kRowTiles; ++r)
#pragma unroll
    for (int t = 0; t < NT; ++t) red[wave][r][t][lane] = acc[r][t];
  __syncthreads();
  if (wave >= kRowTiles) return;
  const int r = wave;  // wave r finishes row tile r
  f32x4_t sum[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    sum[t] = red[0][r][t][lane];
#pragma unroll
    for (int w = 1; w < 4; ++w) sum[t] += red[w][r][t][lane];
  }
  const int rtok0 = tok0 + r * 16;
  if (partial != nullptr) {
    // partial[split][token][e]
    float* out = partial + static_cast<int64_t>(blockIdx.y) * T_tokens * E;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int e = t * 16 + n;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = rtok0 + grp * 4 + i;
        if (e < E && tok < T_tokens) out[static_cast<int64_t>(tok) * E + e] = sum[t][i];
      }
    }
    return;
  }
  topk_tile<NT>(sum, bias, E, k, rtok0, T_tokens, sel_val[r], sel_id[r], topk_ids, topk_w, inv_tau, prob_sum,
                order);
}

// bf16 router for many tokens when the whole transposed gate fits in LDS
// (16*ceil(E/16) * d <= 64K elements): one persistent block per CU
// transposes W_g into LDS itself (no transpose launch, and the gate is read
// from L2 once per CU rather than once per 32 tokens), then streams its own
// contiguous range of 16*RT tokens.
//
// * W_g^T in LDS: row e (16*NT rows, rows >= E zero) holds the d gate values
//   of expert e; its 16-byte chunk c sits at chunk c ^ (e & 15), so the 16
//   rows of one fragment read hit 16 distinct bank groups.
// * K runs in 64-wide double steps.  Lane (m, g) loads 32 bytes of token row
//   m, k = 64s + 16g .. 16g + 15 (four lanes cover a row's whole 128-byte
//   line), and feeds its two halves to two 16x16x32 MFMAs; the B fragments
//   of the same k come from LDS, so both operands use one K order.
// * The 4 waves split the row tiles (RT >= 4) or, for RT < 4, the double
//   steps; split partials are summed in LDS in wave order (deterministic).
// * The owner wave of each 16-token row tile selects the top k.
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (N > 0) {
    static_for<N - 1>(f);
    f(std::integral_constant<int, N - 1>{});
  }
}

constexpr int kLdsRouterScratch = 4 * 2 * 16 * kMaxExperts * 4;  // per-wave top-k scratch, 32 KB
constexpr int kLdsRouterMaxGate = 64 * 1024;                      // gate elements that fit beside it

// With kSplit the gate does not fit in LDS whole: K is cut into gridDim.y
// slices of dlen, block (x, y) keeps slice y of the gate in LDS, streams
// that slice of its tokens' rows and writes the slice's partial logits to
// partial[y][token][e]; router_topk_kernel then sums the slices in order and
// selects.  Without kSplit, dlen = d and the block selects itself.
// With kSplit the gate comes from WgT ([16*NT][d], written by
// gate_transpose_kernel): the block copies its slice into LDS with direct
// buffer->LDS loads, the chunk swizzle applied to the global offsets.
template <int NT, int RT, bool kSplit>
__global__ __launch_bounds__(kRouterThreads, 1) void router_lds_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ Wg, const float* __restrict__ bias, int T_tokens,
    int d, int dlen, int E, int k, int32_t* __restrict__ topk_ids, float* __restrict__ topk_w, float inv_tau,
    float* __restrict__ prob_sum, uint8_t* __restrict__ order, float* __restrict__ partial,
    const uint16_t* __restrict__ WgT) {
  constexpr int WT = RT >= 4 ? 4 : RT;  // token groups of waves
  constexpr int WK = 4 / WT;            // K splits per token group
  constexpr int RW = RT / WT;           // row tiles per wave
  constexpr int kU = RW == 1 ? 8 : 4;   // double steps in flight per batch (16 loads per lane)
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  unsigned char* const gate = smem;
  const int row_bytes = dlen * 2;
  unsigned char* const scratch = smem + static_cast<size_t>(16 * NT) * row_bytes;
  const int kbeg = kSplit ? static_cast<int>(blockIdx.y) * dlen : 0;  // this block's K slice [kbeg, kbeg + dlen)
  const uint16_t* const Wg_s = Wg + static_cast<int64_t>(kbeg) * E;

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int n = lane & 15;
  const int grp = lane >> 4;

  const int wt = wave / WK;
  const int wk = wave % WK;
  const int nds = dlen / 64;
  float* const sel_val = reinterpret_cast<float*>(scratch + wave * (2 * 16 * kMaxExperts * 4));
  int* const sel_id = reinterpret_cast<int*>(scratch + wave * (2 * 16 * kMaxExperts * 4) + 16 * kMaxExperts * 4);
  f32x4_t* const red = reinterpret_cast<f32x4_t*>(scratch);  // [4 waves][RW][NT][64 lanes], aliases the top-k scratch

  // Token rows of this wave in the current pass, and its double steps
  // s = wk, wk + WK, ... in batches of kU, two batches in flight.
  const unsigned char* xrow[RW];
  auto set_rows = [&](int tok_base) {
#pragma unroll
    for (int r = 0; r < RW; ++r) {
      const int tok = min(tok_base + (wt * RW + r) * 16 + n, T_tokens - 1);  // rows past T repeat the last token
      xrow[r] = reinterpret_cast<const unsigned char*>(X + static_cast<int64_t>(tok) * d + kbeg) + grp * 32;
    }
  };
  const int nsteps = (nds - wk + WK - 1) / WK;
  const int nbatch = (nsteps + kU - 1) / kU;
  typedef u32x4_t Batch[kU][RW][2];
  auto load_batch = [&](int b, Batch& a) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int st = wk + (b * kU + u) * WK;
      if (st < nds) {
#pragma unroll
        for (int r = 0; r < RW; ++r) {
          const int64_t off = static_cast<int64_t>(st) * 128;
          a[u][r][0] = ld16(xrow[r] + off);
          a[u][r][1] = ld16(xrow[r] + off + 16);
        }
      }
    }
  };
  Batch bufA, bufB;
  int tok_base = blockIdx.x * 16 * RT;  // < T_tokens: the grid has no block without tokens
  set_rows(tok_base);

  if constexpr (kSplit) {
    // Slice rows e = 0 .. 16*NT-1 of WgT, 2*dlen bytes each: instruction j
    // of this wave fills LDS bytes [1024 (4j + wave), +1024), lane l its
    // chunk p = 64 (4j + wave) % (row chunks) + l of row e, which holds the
    // slice's chunk p ^ (e & 15) (XOR within runs of 16 chunks, so one
    // instruction reads one contiguous 1 KB run of WgT).
    const __amdgpu_buffer_rsrc_t grsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(WgT), 0, 16 * NT * d * 2, 0x00020000);
    const int row_chunks = dlen / 8;
    const int n_instr = 16 * NT * row_chunks / kWave;
    for (int j = wave; j < n_instr; j += kRouterThreads / kWave) {
      const int p_lin = j * kWave + lane;
      const int e = p_lin / row_chunks;
      const int p = p_lin % row_chunks;
      const int goff = (e * d + kbeg + ((p ^ (e & 15)) << 3)) * 2;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(grsrc, (__attribute__((address_space(3))) void*)(gate + j * 1024), 16,
                                               goff, 0, 0, 0);
    }
    load_batch(0, bufA);
    if (nbatch > 1) load_batch(1, bufB);
    __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));  // vmcnt(0): the slice (and the first batches) landed
  } else {
  // ---- W_g^T into LDS: unit (kb, eg) = 8 consecutive k x 8 experts, read as
  // 8 rows of 16 bytes (W_g is [d, E], experts contiguous) and written as 8
  // rows-of-W_g^T chunks of 16 bytes.
    constexpr int kBatch = 4;  // units per thread with their loads in flight together
    const int egs = 2 * NT;    // 8-expert groups, padding included
    const int units = (dlen / 8) * egs;
    // Vector loads go through a buffer resource over the slice of W_g
    // (dlen*E*2 < 2^31 bytes, as dlen*16*NT <= 64K): padding experts and
    // units past the end take an offset beyond the range and read zeros, so
    // no load sits behind a branch.  E not a multiple of 8 (rows not 16-byte
    // aligned): 2-byte loads.
    const __amdgpu_buffer_rsrc_t wrsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(Wg_s), 0, dlen * E * 2, 0x00020000);
    // One batch of units; the first also issues the first two batches of
    // token loads right after its gate loads, so all are in flight together.
    auto do_batch = [&](int u0, auto vec_c, auto first_c) {
      constexpr bool kVec = decltype(vec_c)::value;
      {
        uint32_t in[kBatch][8][4];
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
          const int u = u0 + b * kRouterThreads;
          const int kb = u / egs;
          const int eg = u % egs;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            if constexpr (kVec) {
              const int off =
                  u < units && eg * 8 < E ? ((kb * 8 + j) * E + eg * 8) * 2 : static_cast<int>(0x80000000u);
              const u32x4_t v = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(wrsrc, off, 0, 0));
#pragma unroll
              for (int q = 0; q < 4; ++q) in[b][j][q] = v[q];
            } else {
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const int e0 = eg * 8 + 2 * q;
                const int o = (kb * 8 + j) * E + e0;
                const uint32_t lo = u < units && e0 < E ? Wg_s[o] : 0u;
                const uint32_t hi = u < units && e0 + 1 < E ? Wg_s[o + 1] : 0u;
                in[b][j][q] = lo | (hi << 16);
              }
            }
          }
        }
        if constexpr (decltype(first_c)::value) {
          load_batch(0, bufA);
          if (nbatch > 1) load_batch(1, bufB);
        }
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
          const int u = u0 + b * kRouterThreads;
          if (u >= units) break;
          const int kb = u / egs;
          const int eg = u % egs;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            // expert eg*8+i: its 8 values of k = 8kb .. 8kb+7, two per word
            u32x4_t o;
#pragma unroll
            for (int p = 0; p < 4; ++p) {
              const uint32_t lo = in[b][2 * p][i >> 1], hi = in[b][2 * p + 1][i >> 1];
              o[p] = (i & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
            }
            const int e = eg * 8 + i;
            *reinterpret_cast<u32x4_t*>(gate + e * row_bytes + ((kb ^ (e & 15)) << 4)) = o;
          }
        }
      }
    };
    auto transpose = [&](auto vec_c) {
      do_batch(tid, vec_c, std::true_type{});
      for (int u0 = tid + kBatch * kRouterThreads; u0 < units; u0 += kBatch * kRouterThreads)
        do_batch(u0, vec_c, std::false_type{});
    };
    if (E % 8 == 0) transpose(std::true_type{});
    else transpose(std::false_type{});
  }
  __syncthreads();

  for (;;) {
    f32x4_t acc[RW][NT];
#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[r][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    auto mma_step = [&](int st, const u32x4_t (&a)[RW][2]) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int c = st * 8 + grp * 2 + h;  // 16-byte chunk of k = 64s + 16g + 8h
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const int e = t * 16 + n;
          const u32x4_t b = *reinterpret_cast<const u32x4_t*>(gate + e * row_bytes + ((c ^ n) << 4));
#pragma unroll
          for (int r = 0; r < RW; ++r) acc[r][t] = RouterMma<uint16_t>::run(a[r][h], b, acc[r][t]);
        }
      }
    };
    auto mma_batch = [&](int b, const Batch& a) {
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int st = wk + (b * kU + u) * WK;
        if (st < nds) mma_step(st, a[u]);
      }
    };
    // Batches b and b + 1 are in flight at the top of each iteration.
    for (int b = 0; b < nbatch; b += 2) {
      mma_batch(b, bufA);
      if (b + 2 < nbatch) load_batch(b + 2, bufA);
      if (b + 1 < nbatch) {
        mma_batch(b + 1, bufB);
        if (b + 3 < nbatch) load_batch(b + 3, bufB);
      }
    }
    // The next pass's first token loads go out before this pass's selection,
    // which they overlap.
    const int cur_base = tok_base;
    tok_base += gridDim.x * 16 * RT;
    const bool more = tok_base < T_tokens;
    if (more) {
      set_rows(tok_base);
      load_batch(0, bufA);
      if (nbatch > 1) load_batch(1, bufB);
    }

    if constexpr (WK > 1) {
      // Sum the K splits of each token group in wave order.
#pragma unroll
      for (int r = 0; r < RW; ++r)
#pragma unroll
        for (int t = 0; t < NT; ++t) red[((wave * RW + r) * NT + t) * kWave + lane] = acc[r][t];
      __syncthreads();
      if (wk == 0) {
#pragma unroll
        for (int r = 0; r < RW; ++r)
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            f32x4_t v = red[((wave * RW + r) * NT + t) * kWave + lane];
#pragma unroll
            for (int w = 1; w < WK; ++w) v += red[(((wave + w) * RW + r) * NT + t) * kWave + lane];
            acc[r][t] = v;
          }
      }
      __syncthreads();  // the sums are read before the top-k scratch (same LDS) is written
    }
    if (wk == 0) {
      // One call per row tile with a constant index: a loop over r would
      // index acc dynamically, and the compiler would move acc to memory.
      static_for<RW>([&](auto r_c) {
        constexpr int r = decltype(r_c)::value;
        const int rtok0 = cur_base + (wt * RW + r) * 16;
        if constexpr (kSplit) {
          // Partial logits in fragment order, [slice][tile][t][lane] of
          // f32x4 (lane (n, grp), element i: token 16*tile + 4grp + i,
          // expert 16t + n), so each store and each load of
          // router_topk_frag_kernel moves whole 1 KB rows.
          f32x4_t* out = reinterpret_cast<f32x4_t*>(partial) +
                         (static_cast<int64_t>(blockIdx.y) * ((T_tokens + 15) / 16) + rtok0 / 16) * NT * kWave;
          if (rtok0 < T_tokens) {
#pragma unroll
            for (int t = 0; t < NT; ++t) out[t * kWave + lane] = acc[r][t];
          }
        } else {
          topk_tile<NT>(acc[r], bias, E, k, rtok0, T_tokens, sel_val, sel_id, topk_ids, topk_w, inv_tau, prob_sum,
                        order);
        }
      });
    }
    if (!more) break;
    __syncthreads();  // the scratch is reused by the next pass
  }
}

// Sum the K-split partial logits in split order, then top-k.  A block of 512
// threads owns 16 tokens: each thread sums the splits of two (token, expert)
// entries with 8 loads in flight, the sums meet in LDS, and wave 0 selects
// (512 threads leave the selection the registers it needs).
constexpr int kTopkThreads = 512;
template <int NT>
__global__ __launch_bounds__(kTopkThreads) void router_topk_kernel(const float* __restrict__ partial, int nsplit,
                                                           const float* __restrict__ bias, int T_tokens, int E, int k,
                                                           int32_t* __restrict__ topk_ids,
                                                           float* __restrict__ topk_w, float inv_tau,
                                                           float* __restrict__ prob_sum,
                                                           uint8_t* __restrict__ order) {
  __shared__ float logit[16][kMaxExperts];
  __shared__ float sel_val[16 * kMaxExperts];
  __shared__ int sel_id[16 * kMaxExperts];
  topk_from_partials<NT, kTopkThreads>(partial, nsplit, bias, T_tokens, E, k, blockIdx.x * 16, logit, sel_val,
                                       sel_id, topk_ids, topk_w, inv_tau, prob_sum, order);
}

// Sum the K-slice partial logits of router_lds_kernel<..., true> (fragment
// order, see there) in slice order, then top-k: each wave owns one 16-token
// tile and loads its nslices x NT fragments (1 KB each) with all loads in
// flight.  The sums run in the same order as router_topk_kernel's, so the
// logits are the same bits.
template <int NT>
__global__ __launch_bounds__(kRouterThreads) void router_topk_frag_kernel(
    const f32x4_t* __restrict__ partial, int nslices, const float* __restrict__ bias, int T_tokens, int E, int k,
    int32_t* __restrict__ topk_ids, float* __restrict__ topk_w, float inv_tau, float* __restrict__ prob_sum,
    uint8_t* __restrict__ order) {
  constexpr int kMaxSlices = 8;
  __shared__ float sel_val[kRouterThreads / kWave][16 * kMaxExperts];
  __shared__ int sel_id[kRouterThreads / kWave][16 * kMaxExperts];
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int ntiles = (T_tokens + 15) / 16;
  const int tile = blockIdx.x * (kRouterThreads / kWave) + wave;
  if (tile >= ntiles) return;
  f32x4_t v[kMaxSlices][NT];
#pragma unroll
  for (int sl = 0; sl < kMaxSlices; ++sl)
#pragma unroll
    for (int t = 0; t < NT; ++t)
      if (sl < nslices) v[sl][t] = partial[(static_cast<int64_t>(sl) * ntiles + tile) * NT * kWave + t * kWave + lane];
  f32x4_t acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int sl = 0; sl < kMaxSlices; ++sl)
      if (sl < nslices) acc[t] += v[sl][t];  // slice order
  }
  topk_tile<NT>(acc, bias, E, k, tile * 16, T_tokens, sel_val[wave], sel_id[wave], topk_ids, topk_w, inv_tau,
                prob_sum, order);
}

// The load-balancing statistics from the per-tile sums of topk_tile
// ("Qwen2-MoE代码解析" §3.3): prob_sum is [ntiles][2E] (probability sums,
// then selection counts, per 16-token tile).  Stage 1: block b sums tiles
// 64b .. 64b+63 (thread (c, j) sums 8 of them with independent loads, the 8
// partials meet in a fixed order) into part[b][2E].  Stage 2 (one block)
// sums the blocks in order and writes prob_mean = sum / T, sel_freq =
// count / T and aux = E * sum_e prob_mean[e] * sel_freq[e] (expert order).
// Every sum runs in a fixed order, so the result is deterministic.
constexpr int kStatsTilesPerBlock = 64;
constexpr int kStatsThreads = 1024;  // 128 columns x 8 row groups

__global__ __launch_bounds__(kStatsThreads) void router_stats_partial_kernel(const float* __restrict__ prob_sum,
                                                                             int ntiles, int E,
                                                                             float* __restrict__ part) {
  __shared__ float s_part[8][2 * kMaxExperts];
  const int c = threadIdx.x % (2 * kMaxExperts);
  const int j = threadIdx.x / (2 * kMaxExperts);
  const int cols = 2 * E;
  const int r0 = blockIdx.x * kStatsTilesPerBlock + j * 8;
  float v = 0.f;
  if (c < cols) {
    float x[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int r = min(r0 + q, ntiles - 1);  // in range; a row past the end is read and masked
      x[q] = prob_sum[static_cast<int64_t>(r) * cols + c];
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) v += r0 + q < ntiles ? x[q] : 0.f;
  }
  s_part[j][c] = v;
  __syncthreads();
  if (threadIdx.x < cols) {
    float t = 0.f;
#pragma unroll
    for (int q = 0; q < 8; ++q) t += s_part[q][threadIdx.x];
    part[static_cast<int64_t>(blockIdx.x) * cols + threadIdx.x] = t;
  }
}

__global__ __launch_bounds__(2 * kMaxExperts) void router_stats_final_kernel(const float* __restrict__ part,
                                                                             int nblocks, int T_tokens, int E,
                                                                             float* __restrict__ prob_mean,
                                                                             float* __restrict__ sel_freq,
                                                                             float* __restrict__ aux) {
  __shared__ float s_v[2 * kMaxExperts];
  const int c = threadIdx.x;
  const int cols = 2 * E;
  float v = 0.f;
  if (c < cols)
    for (int b = 0; b < nblocks; ++b) v += part[static_cast<int64_t>(b) * cols + c];
  const float inv_t = 1.f / static_cast<float>(T_tokens);
  s_v[c] = v * inv_t;
  __syncthreads();
  if (c < E) {
    prob_mean[c] = s_v[c];
    sel_freq[c] = s_v[E + c];
  }
  if (c == 0) {
    float a = 0.f;
    for (int e = 0; e < E; ++e) a += s_v[e] * s_v[E + e];
    aux[0] = static_cast<float>(E) * a;
  }
}

// K per split: the whole d when there are enough token blocks, else d split
// into pieces of at least 256 so roughly 256 blocks run.
int split_len_of(int T_tokens, int d) {
  const int tok_blocks = (T_tokens + kRouterTok - 1) / kRouterTok;
  if (tok_blocks >= 128 || d <= 256) return d;
  int want = (256 + tok_blocks - 1) / tok_blocks;
  const int max_splits = d / 256;
  if (want > max_splits) want = max_splits;
  if (want <= 1) return d;
  int len = (d + want - 1) / want;
  len = (len + 127) / 128 * 128;  // whole k-steps for every wave
  return len;
}

size_t align256(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }

size_t gate_t_bytes(int d, int E, size_t esize) { return align256(static_cast<size_t>((E + 15) / 16) * 16 * d * esize); }

// Whether router_lds_kernel runs: bf16, no K split, W_g^T fits in LDS, and
// d a multiple of 128 (the chunk swizzle permutes chunks within runs of 16).
bool lds_router(int dtype, int T_tokens, int d, int E) {
  return dtype == kDtypeBF16 && split_len_of(T_tokens, d) == d && d % 128 == 0 &&
         (E + 15) / 16 * 16 * d <= kLdsRouterMaxGate;
}

// K slices of the split LDS router, or 0 where it does not run: bf16, many
// tokens (no small-batch K split), a gate too large for LDS whole, and d
// cut into 2..8 equal slices that are multiples of 128 and fit in LDS
// (d = 4096 with 64 experts: 4 slices of 1024).
int lds_router_slices(int dtype, int T_tokens, int d, int E) {
  if (dtype != kDtypeBF16 || split_len_of(T_tokens, d) != d || d % 128 != 0) return 0;
  const int rows = (E + 15) / 16 * 16;
  if (rows * d <= kLdsRouterMaxGate) return 0;
  for (int n = 2; n <= 8; ++n)
    if (d % (n * 128) == 0 && rows * (d / n) <= kLdsRouterMaxGate) return n;
  return 0;
}

template <int NT, int RT, bool kSplit>
hipError_t launch_lds_rt(const uint16_t* X, const uint16_t* Wg, const float* bias, int T_tokens, int d, int dlen,
                         int E, int k, int32_t* ids, float* w, dim3 grid, const RouteExtra& x, float* partial,
                         const uint16_t* WgT, hipStream_t stream) {
  const size_t lds = static_cast<size_t>(16 * NT) * dlen * 2 + kLdsRouterScratch;
  static const hipError_t attr =
      hipFuncSetAttribute(reinterpret_cast<const void*>(&router_lds_kernel<NT, RT, kSplit>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, kLdsRouterMaxGate * 2 + kLdsRouterScratch);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((router_lds_kernel<NT, RT, kSplit>), grid, dim3(kRouterThreads), lds, stream, X, Wg, bias,
                     T_tokens, d, dlen, E, k, ids, w, x.inv_tau, x.prob_sum, x.order, partial, WgT);
  return hipGetLastError();
}

// nslices = 1: the whole gate in LDS, every block selects.  nslices > 1:
// the K slices, partial logits into `partial`, then router_topk_kernel.
template <int NT>
hipError_t launch_lds(const uint16_t* X, const uint16_t* Wg, const float* bias, int T_tokens, int d, int E, int k,
                      int32_t* ids, float* w, const RouteExtra& x, int nslices, float* partial, uint16_t* WgT,
                      hipStream_t stream) {
  // One block per CU (fewer if there are fewer 16-token tiles), each with a
  // contiguous range of 16*RT tokens per pass; with slices, the CUs are
  // shared out among the slices.  The grid then shrinks to the blocks that
  // have tokens in their first pass.
  const int tiles = (T_tokens + 15) / 16;
  const int cus = std::max(1, std::min(device_cu_count() / nslices, tiles));
  const int per = (tiles + cus - 1) / cus;
  const int rt = per <= 1 ? 1 : per <= 2 ? 2 : per <= 4 ? 4 : 8;
  const dim3 grid(std::min(cus, (tiles + rt - 1) / rt), nslices);
  const int dlen = d / nslices;
  hipError_t e;
  if (nslices == 1) {
    if (rt == 1)
      return launch_lds_rt<NT, 1, false>(X, Wg, bias, T_tokens, d, d, E, k, ids, w, grid, x, nullptr, nullptr, stream);
    if (rt == 2)
      return launch_lds_rt<NT, 2, false>(X, Wg, bias, T_tokens, d, d, E, k, ids, w, grid, x, nullptr, nullptr, stream);
    if (rt == 4)
      return launch_lds_rt<NT, 4, false>(X, Wg, bias, T_tokens, d, d, E, k, ids, w, grid, x, nullptr, nullptr, stream);
    return launch_lds_rt<NT, 8, false>(X, Wg, bias, T_tokens, d, d, E, k, ids, w, grid, x, nullptr, nullptr, stream);
  }
  // The gate transposed once into the workspace, then copied slice by slice.
  hipLaunchKernelGGL((gate_transpose_kernel<uint16_t, NT>), dim3(d / 32), dim3(256), 0, stream, Wg, d, E, WgT);
  if (rt == 1)
    e = launch_lds_rt<NT, 1, true>(X, Wg, bias, T_tokens, d, dlen, E, k, ids, w, grid, x, partial, WgT, stream);
  else if (rt == 2)
    e = launch_lds_rt<NT, 2, true>(X, Wg, bias, T_tokens, d, dlen, E, k, ids, w, grid, x, partial, WgT, stream);
  else if (rt == 4)
    e = launch_lds_rt<NT, 4, true>(X, Wg, bias, T_tokens, d, dlen, E, k, ids, w, grid, x, partial, WgT, stream);
  else
    e = launch_lds_rt<NT, 8, true>(X, Wg, bias, T_tokens, d, dlen, E, k, ids, w, grid, x, partial, WgT, stream);
  if (e != hipSuccess) return e;
  const int waves = kRouterThreads / kWave;
  hipLaunchKernelGGL((router_topk_frag_kernel<NT>), dim3((tiles + waves - 1) / waves), dim3(kRouterThreads), 0, stream,
                     reinterpret_cast<const f32x4_t*>(partial), nslices, bias, T_tokens, E, k, ids, w, x.inv_tau,
                     x.prob_sum, x.order);
  return hipGetLastError();
}

template <typename T, int NT>
hipError_t launch_nt(const T* X, const T* Wg, const float* bias, int T_tokens, int d, int E, int k, int32_t* ids,
                     float* w, unsigned char* scratch, bool select, const RouteExtra& x, hipStream_t stream) {
  if constexpr (std::is_same<T, uint16_t>::value) {
    if (lds_router(kDtypeBF16, T_tokens, d, E))
      return launch_lds<NT>(X, Wg, bias, T_tokens, d, E, k, ids, w, x, 1, nullptr, nullptr, stream);
    if (const int ns = lds_router_slices(kDtypeBF16, T_tokens, d, E); ns > 1)
      return launch_lds<NT>(X, Wg, bias, T_tokens, d, E, k, ids, w, x, ns,
                            reinterpret_cast<float*>(scratch + gate_t_bytes(d, E, sizeof(T))),
                            reinterpret_cast<uint16_t*>(scratch), stream);
  }
  T* WgT = reinterpret_cast<T*>(scratch);
  float* partial = reinterpret_cast<float*>(scratch + gate_t_bytes(d, E, sizeof(T)));
  const int split_len = split_len_of(T_tokens, d);
  const int nsplit = (d + split_len - 1) / split_len;
  const dim3 grid((T_tokens + kRouterTok - 1) / kRouterTok, nsplit);
  if (nsplit > 1) {
    // few token blocks: gather from W_g directly, no transpose launch
    hipLaunchKernelGGL((router_kernel<T, NT, true>), grid, dim3(kRouterThreads), 0, stream, X, WgT, Wg, bias, T_tokens,
                       d, E, k, split_len, partial, ids, w, x.inv_tau, x.prob_sum, x.order);
  } else {
    hipLaunchKernelGGL((gate_transpose_kernel<T, NT>), dim3(d / 32), dim3(256), 0, stream, Wg, d, E, WgT);
    hipLaunchKernelGGL((router_kernel<T, NT, false>), grid, dim3(kRouterThreads), 0, stream, X, WgT, Wg, bias,
                       T_tokens, d, E, k, split_len, nullptr, ids, w, x.inv_tau, x.prob_sum, x.order);
  }
  if (nsplit > 1 && select)
    hipLaunchKernelGGL((router_topk_kernel<NT>), dim3((T_tokens + 15) / 16), dim3(kTopkThreads), 0, stream, partial,
                       nsplit, bias, T_tokens, E, k, ids, w, x.inv_tau, x.prob_sum, x.order);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const T* X, const T* Wg, const float* bias, int T_tokens, int d, int E, int k, int32_t* ids,
                    float* w, unsigned char* scratch, bool select, const RouteExtra& x, hipStream_t stream) {
  switch ((E + 15) / 16) {
    case 1: return launch_nt<T, 1>(X, Wg, bias, T_tokens, d, E, k, ids, w, scratch, select, x, stream);
    case 2: return launch_nt<T, 2>(X, Wg, bias, T_tokens, d, E, k, ids, w, scratch, select, x, stream);
    case 3: return launch_nt<T, 3>(X, Wg, bias, T_tokens, d, E, k, ids, w, scratch, select, x, stream);
    default: return launch_nt<T, 4>(X, Wg, bias, T_tokens, d, E, k, ids, w, scratch, select, x, stream);
  }
}

}  // namespace

size_t router_scratch_bytes(int T_tokens, int d, int E, int dtype) {
  if (T_tokens <= 0) return 0;
  const size_t esize = dtype == kDtypeBF16 ? 2 : 4;
  const int split_len = split_len_of(T_tokens, d);
  const int nsplit = (d + split_len - 1) / split_len;
  size_t b = gate_t_bytes(d, E, esize);
  if (nsplit > 1) b += static_cast<size_t>(nsplit) * T_tokens * E * sizeof(float);
  // the split LDS router's partial logits in fragment order (16 x 16*NT per
  // tile and slice; it never splits for few tokens)
  if (const int ns = lds_router_slices(dtype, T_tokens, d, E); ns > 1)
    b += static_cast<size_t>(ns) * ((T_tokens + 15) / 16) * 16 * ((E + 15) / 16 * 16) * sizeof(float);
  return b;
}

RouterSplit router_split(int T_tokens, int d, int E, int dtype, void* scratch) {
  RouterSplit r{nullptr, 1};
  if (T_tokens <= 0) return r;
  const int split_len = split_len_of(T_tokens, d);
  r.nsplit = (d + split_len - 1) / split_len;
  if (r.nsplit > 1)
    r.partial = reinterpret_cast<const float*>(static_cast<unsigned char*>(scratch) +
                                               gate_t_bytes(d, E, dtype == kDtypeBF16 ? 2 : 4));
  return r;
}

hipError_t launch_router(int dtype, const void* X, const void* Wg, const float* bias, int T_tokens, int d, int E,
                         int k, int32_t* ids, float* w, void* scratch, hipStream_t stream, bool select,
                         float inv_tau, float* prob_sum, uint8_t* order) {
  if (T_tokens <= 0) return hipSuccess;
  unsigned char* sc = static_cast<unsigned char*>(scratch);
  const RouteExtra x{inv_tau, prob_sum, order};
  if (dtype == kDtypeBF16)
    return launch_t(static_cast<const uint16_t*>(X), static_cast<const uint16_t*>(Wg), bias, T_tokens, d, E, k, ids,
                    w, sc, select, x, stream);
  return launch_t(static_cast<const float*>(X), static_cast<const float*>(Wg), bias, T_tokens, d, E, k, ids, w, sc,
                  select, x, stream);
}

size_t router_stats_scratch_bytes(int T_tokens, int E) {
  if (T_tokens <= 0) return 0;
  const size_t ntiles = static_cast<size_t>((T_tokens + 15) / 16);
  const size_t nblocks = (ntiles + kStatsTilesPerBlock - 1) / kStatsTilesPerBlock;
  return align256(ntiles * 2 * E * sizeof(float)) + nblocks * 2 * E * sizeof(float);
}

hipError_t launch_router_stats(float* prob_sum, const int32_t* ids, int T_tokens, int E, int k, float* prob_mean,
                               float* sel_freq, float* aux, hipStream_t stream) {
  (void)ids;
  (void)k;
  if (T_tokens <= 0) return hipSuccess;
  const int ntiles = (T_tokens + 15) / 16;
  const int nblocks = (ntiles + kStatsTilesPerBlock - 1) / kStatsTilesPerBlock;
  float* part = reinterpret_cast<float*>(reinterpret_cast<unsigned char*>(prob_sum) +
                                         align256(static_cast<size_t>(ntiles) * 2 * E * sizeof(float)));
  hipLaunchKernelGGL(router_stats_partial_kernel, dim3(nblocks), dim3(kStatsThreads), 0, stream, prob_sum, ntiles, E,
                     part);
  hipLaunchKernelGGL(router_stats_final_kernel, dim3(1), dim3(2 * kMaxExperts), 0, stream, part, nblocks, T_tokens,
                     E, prob_mean, sel_freq, aux);
  return hipGetLastError();
}

}  // namespace moe
