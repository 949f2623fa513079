// Router kernel: gate projection on MFMA, softmax-free top-k selection on the
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
// Layout of the work: a wave owns 16 tokens and every expert (E <= 64, i.e.
// up to four 16-column MFMA tiles).  Per stage each lane streams 64 contiguous
// bytes of its token's row (4 x 16 B), so a row is read front to back by 4
// lanes.  The stage's slice of W_g ([d, E], experts contiguous) is staged
// through LDS transposed to [expert][k] so MFMA B fragments are 16-byte reads.
// The MFMA reduction order over k is a permutation of the plain order, the
// same one on A and B, so the products are unchanged.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int kRouterWaves = 2;               // waves per block
constexpr int kRouterThreads = kRouterWaves * kWave;
constexpr int kTokPerWave = 16;
constexpr int kStageBytes = 256;              // bytes of one row per stage (16 chunks)
constexpr int kSwRowBytes = kStageBytes + 16; // padded LDS row of the transposed gate slice

// One 16-byte chunk of A (token row) and B (gate column) into the 16x16 tile.
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

__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

template <typename T, int NT>
__global__ __launch_bounds__(kRouterThreads) void router_kernel(
    const T* __restrict__ X, const T* __restrict__ Wg, const float* __restrict__ bias,
    int T_tokens, int d, int E, int k, int32_t* __restrict__ topk_ids, float* __restrict__ topk_w) {
  constexpr int kPer16 = 16 / sizeof(T);             // elements per 16-byte chunk
  constexpr int kStageElems = kStageBytes / sizeof(T);
  __shared__ __attribute__((aligned(16))) unsigned char sW[NT * 16 * kSwRowBytes];
  __shared__ float sel_val[kRouterWaves][kTokPerWave][kMaxExperts];
  __shared__ int sel_id[kRouterWaves][kTokPerWave][kMaxExperts];

  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int n = lane & 15;      // MFMA column / A row within the 16-row tile
  const int grp = lane >> 4;    // 0..3
  const int tok0 = (blockIdx.x * kRouterWaves + wave) * kTokPerWave;

  // Columns >= E of the staged slice stay zero for the whole kernel.
  for (int i = threadIdx.x; i < NT * 16 * kSwRowBytes / 4; i += kRouterThreads)
    reinterpret_cast<uint32_t*>(sW)[i] = 0u;

  const int arow = min(tok0 + n, T_tokens - 1);     // clamp: rows past T are computed and ignored
  const unsigned char* xrow = reinterpret_cast<const unsigned char*>(X + static_cast<int64_t>(arow) * d);
  const int row_bytes = d * static_cast<int>(sizeof(T));
  const int nstages = (row_bytes + kStageBytes - 1) / kStageBytes;

  auto load_x = [&](int st, u32x4_t (&r)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int off = st * kStageBytes + (grp * 4 + j) * 16;
      r[j] = off < row_bytes ? ld16(xrow + off) : u32x4_t{0u, 0u, 0u, 0u};
    }
  };

  // Gate slice of one stage: kStageElems rows of W_g, each E elements.
  const bool vec_ok = (E % kPer16) == 0;
  const int nvec = vec_ok ? kStageElems * (E / kPer16) : kStageElems * E;
  constexpr int kMaxW = (kStageElems * NT * 16 / kPer16 + kRouterThreads - 1) / kRouterThreads;
  u32x4_t wreg[kMaxW];
  auto load_w = [&](int st) {
    const int k0 = st * kStageElems;
#pragma unroll
    for (int i = 0; i < kMaxW; ++i) {
      const int v = threadIdx.x + i * kRouterThreads;
      u32x4_t r = {0u, 0u, 0u, 0u};
      if (vec_ok && v < nvec) {
        const int vpr = E / kPer16;
        const int kk = v / vpr;
        if (k0 + kk < d) r = ld16(Wg + static_cast<int64_t>(k0 + kk) * E + (v % vpr) * kPer16);
      }
      wreg[i] = r;
    }
  };
  auto store_w = [&](int st) {
    const int k0 = st * kStageElems;
    if (vec_ok) {
      const int vpr = E / kPer16;
#pragma unroll
      for (int i = 0; i < kMaxW; ++i) {
        const int v = threadIdx.x + i * kRouterThreads;
        if (v < nvec) {
          const int kk = v / vpr;
          const int e0 = (v % vpr) * kPer16;
          const T* src = reinterpret_cast<const T*>(&wreg[i]);
#pragma unroll
          for (int q = 0; q < kPer16; ++q)
            reinterpret_cast<T*>(sW + (e0 + q) * kSwRowBytes)[kk] = src[q];
        }
      }
    } else {
      for (int v = threadIdx.x; v < nvec; v += kRouterThreads) {
        const int kk = v / E;
        const int e = v % E;
        T val = (k0 + kk < d) ? Wg[static_cast<int64_t>(k0 + kk) * E + e] : T(0);
        reinterpret_cast<T*>(sW + e * kSwRowBytes)[kk] = val;
      }
    }
  };

  f32x4_t acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  u32x4_t xa[4], xb[4];
  load_x(0, xa);
  load_w(0);
  for (int st = 0; st < nstages; ++st) {
    __syncthreads();
    store_w(st);
    __syncthreads();
    if (st + 1 < nstages) {
      load_x(st + 1, xb);
      load_w(st + 1);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const u32x4_t b = *reinterpret_cast<const u32x4_t*>(sW + (t * 16 + n) * kSwRowBytes + (grp * 4 + j) * 16);
        acc[t] = RouterMma<T>::run(xa[j], b, acc[t]);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) xa[j] = xb[j];
  }

  // acc[t][i] is the logit of token row grp*4+i and expert t*16+n.
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int e = t * 16 + n;
    const float b = (e < E && bias != nullptr) ? bias[e] : 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[t][i] = (e < E) ? acc[t][i] + b : -INFINITY;
  }

  for (int s = 0; s < k; ++s) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float bv = acc[0][i];
      int bi = n;
#pragma unroll
      for (int t = 1; t < NT; ++t)
        if (better(acc[t][i], t * 16 + n, bv, bi)) { bv = acc[t][i]; bi = t * 16 + n; }
#pragma unroll
      for (int m = 1; m < 16; m <<= 1) {
        const float ov = __shfl_xor(bv, m, 16);
        const int oi = __shfl_xor(bi, m, 16);
        if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
      }
      if ((bi & 15) == n) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
          if (t == (bi >> 4)) acc[t][i] = -INFINITY;
      }
      if (n == 0) {
        sel_val[wave][grp * 4 + i][s] = bv;
        sel_id[wave][grp * 4 + i][s] = bi;
      }
    }
  }
  __builtin_amdgcn_wave_barrier();
  __syncthreads();

  for (int idx = lane; idx < kTokPerWave * k; idx += kWave) {
    const int row = idx / k;
    const int s = idx % k;
    const int tok = tok0 + row;
    if (tok >= T_tokens) continue;
    const float l0 = sel_val[wave][row][0];
    float den = 0.f;
    for (int j = 0; j < k; ++j) den += expf(sel_val[wave][row][j] - l0);
    const int64_t o = static_cast<int64_t>(tok) * k + s;
    topk_ids[o] = sel_id[wave][row][s];
    topk_w[o] = expf(sel_val[wave][row][s] - l0) / den;
  }
}

template <typename T>
hipError_t launch_router_t(const T* X, const T* Wg, const float* bias, int T_tokens, int d, int E, int k,
                           int32_t* ids, float* w, hipStream_t stream) {
  const int tok_per_block = kRouterWaves * kTokPerWave;
  const dim3 grid((T_tokens + tok_per_block - 1) / tok_per_block);
  const int nt = (E + 15) / 16;
  switch (nt) {
    case 1: hipLaunchKernelGGL((router_kernel<T, 1>), grid, dim3(kRouterThreads), 0, stream, X, Wg, bias, T_tokens, d, E, k, ids, w); break;
    case 2: hipLaunchKernelGGL((router_kernel<T, 2>), grid, dim3(kRouterThreads), 0, stream, X, Wg, bias, T_tokens, d, E, k, ids, w); break;
    case 3: hipLaunchKernelGGL((router_kernel<T, 3>), grid, dim3(kRouterThreads), 0, stream, X, Wg, bias, T_tokens, d, E, k, ids, w); break;
    default: hipLaunchKernelGGL((router_kernel<T, 4>), grid, dim3(kRouterThreads), 0, stream, X, Wg, bias, T_tokens, d, E, k, ids, w); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_router(int dtype, const void* X, const void* Wg, const float* bias, int T_tokens, int d,
                         int E, int k, int32_t* ids, float* w, hipStream_t stream) {
  if (T_tokens <= 0) return hipSuccess;
  if (dtype == kDtypeBF16)
    return launch_router_t(static_cast<const uint16_t*>(X), static_cast<const uint16_t*>(Wg), bias, T_tokens, d, E,
                           k, ids, w, stream);
  return launch_router_t(static_cast<const float*>(X), static_cast<const float*>(Wg), bias, T_tokens, d, E, k, ids,
                         w, stream);
}

}  // namespace moe
