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
#include "common.hpp"
#include "kernels.hpp"
#include "topk.hpp"

namespace moe {
namespace {

constexpr int kRouterThreads = 256;               // 4 waves
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
    float* __restrict__ topk_w) {
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
  topk_tile<NT>(sum, bias, E, k, rtok0, T_tokens, sel_val[r], sel_id[r], topk_ids, topk_w);
}

// Sum the K-split partial logits in split order, then top-k.  A block of 1024
// threads owns 16 tokens: one thread per (token, expert) entry sums the splits
// with 8 loads in flight, the sums meet in LDS, and wave 0 selects.
template <int NT>
__global__ __launch_bounds__(1024) void router_topk_kernel(const float* __restrict__ partial, int nsplit,
                                                           const float* __restrict__ bias, int T_tokens, int E, int k,
                                                           int32_t* __restrict__ topk_ids,
                                                           float* __restrict__ topk_w) {
  __shared__ float logit[16][kMaxExperts];
  __shared__ float sel_val[16 * kMaxExperts];
  __shared__ int sel_id[16 * kMaxExperts];
  topk_from_partials<NT>(partial, nsplit, bias, T_tokens, E, k, blockIdx.x * 16, logit, sel_val, sel_id, topk_ids,
                         topk_w);
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

template <typename T, int NT>
hipError_t launch_nt(const T* X, const T* Wg, const float* bias, int T_tokens, int d, int E, int k, int32_t* ids,
                     float* w, unsigned char* scratch, bool select, hipStream_t stream) {
  T* WgT = reinterpret_cast<T*>(scratch);
  float* partial = reinterpret_cast<float*>(scratch + gate_t_bytes(d, E, sizeof(T)));
  const int split_len = split_len_of(T_tokens, d);
  const int nsplit = (d + split_len - 1) / split_len;
  const dim3 grid((T_tokens + kRouterTok - 1) / kRouterTok, nsplit);
  if (nsplit > 1) {
    // few token blocks: gather from W_g directly, no transpose launch
    hipLaunchKernelGGL((router_kernel<T, NT, true>), grid, dim3(kRouterThreads), 0, stream, X, WgT, Wg, bias, T_tokens,
                       d, E, k, split_len, partial, ids, w);
  } else {
    hipLaunchKernelGGL((gate_transpose_kernel<T, NT>), dim3(d / 32), dim3(256), 0, stream, Wg, d, E, WgT);
    hipLaunchKernelGGL((router_kernel<T, NT, false>), grid, dim3(kRouterThreads), 0, stream, X, WgT, Wg, bias,
                       T_tokens, d, E, k, split_len, nullptr, ids, w);
  }
  if (nsplit > 1 && select)
    hipLaunchKernelGGL((router_topk_kernel<NT>), dim3((T_tokens + 15) / 16), dim3(1024), 0, stream, partial, nsplit,
                       bias, T_tokens, E, k, ids, w);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const T* X, const T* Wg, const float* bias, int T_tokens, int d, int E, int k, int32_t* ids,
                    float* w, unsigned char* scratch, bool select, hipStream_t stream) {
  switch ((E + 15) / 16) {
    case 1: return launch_nt<T, 1>(X, Wg, bias, T_tokens, d, E, k, ids, w, scratch, select, stream);
    case 2: return launch_nt<T, 2>(X, Wg, bias, T_tokens, d, E, k, ids, w, scratch, select, stream);
    case 3: return launch_nt<T, 3>(X, Wg, bias, T_tokens, d, E, k, ids, w, scratch, select, stream);
    default: return launch_nt<T, 4>(X, Wg, bias, T_tokens, d, E, k, ids, w, scratch, select, stream);
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
                         int k, int32_t* ids, float* w, void* scratch, hipStream_t stream, bool select) {
  if (T_tokens <= 0) return hipSuccess;
  unsigned char* sc = static_cast<unsigned char*>(scratch);
  if (dtype == kDtypeBF16)
    return launch_t(static_cast<const uint16_t*>(X), static_cast<const uint16_t*>(Wg), bias, T_tokens, d, E, k, ids,
                    w, sc, select, stream);
  return launch_t(static_cast<const float*>(X), static_cast<const float*>(Wg), bias, T_tokens, d, E, k, ids, w, sc,
                  select, stream);
}

}  // namespace moe
