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
// row (blockIdx.y covers rows longer than 256 chunks) and issues the k slot
// loads together, so a step costs one memory round trip.
template <typename T>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(const T* __restrict__ Yp,
                                                                  const int32_t* __restrict__ inv_perm,
                                                                  const float* __restrict__ topk_w,
                                                                  T* __restrict__ out, int T_tok, int d, int k) {
  constexpr int kPer = Elem<T>::kPer16B;
  constexpr int kMaxSlots = 8;  // slots whose loads are issued together; more are handled in rounds
  const int t = blockIdx.x;
  const int v = blockIdx.y * kCombineThreads + threadIdx.x;
  const int nvec = d / kPer;
  if (v >= nvec) return;
  const int64_t p0 = static_cast<int64_t>(t) * k;
  const int Tk = T_tok * k;
  float acc[kPer];
#pragma unroll
  for (int q = 0; q < kPer; ++q) acc[q] = 0.f;
  for (int s0 = 0; s0 < k; s0 += kMaxSlots) {
    u32x4_t y[kMaxSlots];
    float w[kMaxSlots];
#pragma unroll
    for (int j = 0; j < kMaxSlots; ++j) {
      const int s = s0 + j;
      w[j] = 0.f;
      y[j] = u32x4_t{0u, 0u, 0u, 0u};
      if (s < k) {
        const int row = inv_perm[p0 + s];
        if (row >= 0 && row < Tk) {  // dropped (or an invalid row index) adds nothing
          w[j] = topk_w[p0 + s];
          y[j] = ld16_nt(Yp + static_cast<int64_t>(row) * d + v * kPer);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < kMaxSlots; ++j) {
      const T* ye = reinterpret_cast<const T*>(&y[j]);
#pragma unroll
      for (int q = 0; q < kPer; ++q) acc[q] += w[j] * Elem<T>::to_f32(ye[q]);
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
  hipLaunchKernelGGL(combine_kernel<T>, grid, dim3(kCombineThreads), 0, stream, Yp, inv_perm, w, out, T_tok, d, k);
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
