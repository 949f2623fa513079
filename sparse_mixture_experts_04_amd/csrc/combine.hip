// Combine kernel: out[t] = sum over kept slots s of w[t, s] * Yp[inv_perm[t*k+s]],
// accumulated in fp32 ("Qwen2-MoE代码解析" (jsqmd.com/news/1061813) §3.1
// detail 2: the renormalised routing weights weight the experts' outputs).
// A dropped slot (inv_perm = -1) adds nothing; a token with no kept slot is 0.
// Each thread owns one 16-byte chunk of one output row, so every row of Yp is
// read with full 16-byte vector loads and each output row is written once;
// no atomics, so the sum order (slot 0 first) is fixed.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int kCombineThreads = 256;

// One token per blockIdx.x; each thread owns one 16-byte chunk of the output
// row (blockIdx.y covers rows longer than 256 chunks) and issues the loads of
// KS slots together, so a round of KS slots costs one memory round trip.  No
// load sits behind a branch: the slot indices are clamped to k-1 and a
// dropped slot reads row 0 and is then masked out (a branch per load would
// make each wait for the previous one).
template <typename T, int KS>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(const T* __restrict__ Yp,
                                                                  const int32_t* __restrict__ inv_perm,
                                                                  const float* __restrict__ topk_w,
                                                                  T* __restrict__ out, int T_tok, int d, int k) {
  constexpr int kPer = Elem<T>::kPer16B;
  const int t = blockIdx.x;
  const int v = blockIdx.y * kCombineThreads + threadIdx.x;
  const int nvec = d / kPer;
  if (v >= nvec) return;
  const int64_t p0 = static_cast<int64_t>(t) * k;
  const int Tk = T_tok * k;
  float acc[kPer];
#pragma unroll
  for (int q = 0; q < kPer; ++q) acc[q] = 0.f;
  for (int s0 = 0; s0 < k; s0 += KS) {
    int row[KS];
    float w[KS];
#pragma unroll
    for (int j = 0; j < KS; ++j) {
      const int sc = min(s0 + j, k - 1);
      row[j] = inv_perm[p0 + sc];
      w[j] = topk_w[p0 + sc];
    }
    bool ok[KS];
    u32x4_t y[KS];
#pragma unroll
    for (int j = 0; j < KS; ++j) {
      ok[j] = s0 + j < k && row[j] >= 0 && row[j] < Tk;  // dropped (or an invalid row index) adds nothing
      y[j] = ld16_nt(Yp + static_cast<int64_t>(ok[j] ? row[j] : 0) * d + v * kPer);
    }
#pragma unroll
    for (int j = 0; j < KS; ++j) {
      const T* ye = reinterpret_cast<const T*>(&y[j]);
#pragma unroll
      for (int q = 0; q < kPer; ++q) acc[q] += ok[j] ? w[j] * Elem<T>::to_f32(ye[q]) : 0.f;
    }
  }
  u32x4_t o;
  T* oe = reinterpret_cast<T*>(&o);
#pragma unroll
  for (int q = 0; q < kPer; ++q) oe[q] = Elem<T>::from_f32(acc[q]);
  st16_nt(out + static_cast<int64_t>(t) * d + v * kPer, o);
}

template <typename T>
hipError_t launch_t(const T* Yp, const int32_t* inv_perm, const float* w, T* out, int T_tok, int d, int k,
                    hipStream_t stream) {
  const int nvec = d / Elem<T>::kPer16B;
  const dim3 grid(T_tok, (nvec + kCombineThreads - 1) / kCombineThreads);
  if (k <= 2)
    hipLaunchKernelGGL((combine_kernel<T, 2>), grid, dim3(kCombineThreads), 0, stream, Yp, inv_perm, w, out, T_tok, d,
                       k);
  else if (k <= 4)
    hipLaunchKernelGGL((combine_kernel<T, 4>), grid, dim3(kCombineThreads), 0, stream, Yp, inv_perm, w, out, T_tok, d,
                       k);
  else
    hipLaunchKernelGGL((combine_kernel<T, 8>), grid, dim3(kCombineThreads), 0, stream, Yp, inv_perm, w, out, T_tok, d,
                       k);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_combine(int dtype, const void* Yp, const int32_t* inv_perm, const float* topk_w, void* out,
                          int T_tok, int d, int k, hipStream_t stream) {
  if (T_tok <= 0) return hipSuccess;
  if (dtype == kDtypeBF16)
    return launch_t(static_cast<const uint16_t*>(Yp), inv_perm, topk_w, static_cast<uint16_t*>(out), T_tok, d, k,
                    stream);
  return launch_t(static_cast<const float*>(Yp), inv_perm, topk_w, static_cast<float*>(out), T_tok, d, k, stream);
}

}  // namespace moe
