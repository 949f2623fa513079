// Combine kernel: out[t] = sum over kept slots s of w[t, s] * Yp[inv_perm[t*k+s]],
// accumulated in fp32 ("Qwen2-MoE代码解析" (jsqmd.com/news/1061813) §3.1
// detail 2: the renormalised routing weights weight the experts' outputs).
// A dropped slot (inv_perm = -1) adds nothing; a token with no kept slot is 0.
// Each thread owns one 16-byte chunk of the output row, so every row of Yp is
// read with full 16-byte vector loads and each output row is written once;
// no atomics, so the sum order (slot 0 first) is fixed.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int kCombineThreads = 256;
constexpr int kCombineTok = 8;

template <typename T>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(const T* __restrict__ Yp,
                                                                  const int32_t* __restrict__ inv_perm,
                                                                  const float* __restrict__ topk_w,
                                                                  T* __restrict__ out, int T_tok, int d, int k) {
  constexpr int kPer = Elem<T>::kPer16B;
  extern __shared__ int s_dyn[];
  int* s_row = s_dyn;                                              // [kCombineTok][k]
  float* s_w = reinterpret_cast<float*>(s_dyn + kCombineTok * k);  // [kCombineTok][k]
  const int tok0 = blockIdx.x * kCombineTok;
  const int ntok = min(kCombineTok, T_tok - tok0);
  for (int i = threadIdx.x; i < ntok * k; i += kCombineThreads) {
    const int64_t p = static_cast<int64_t>(tok0) * k + i;
    s_row[i] = inv_perm[p];
    s_w[i] = topk_w[p];
  }
  __syncthreads();
  const int nvec = d / kPer;
  for (int idx = threadIdx.x; idx < ntok * nvec; idx += kCombineThreads) {
    const int tt = idx / nvec;
    const int v = idx % nvec;
    float acc[kPer];
#pragma unroll
    for (int q = 0; q < kPer; ++q) acc[q] = 0.f;
    for (int s = 0; s < k; ++s) {
      const int row = s_row[tt * k + s];
      if (row < 0 || row >= T_tok * k) continue;  // dropped (or an invalid row index)
      const float w = s_w[tt * k + s];
      const u32x4_t y = ld16(Yp + static_cast<int64_t>(row) * d + v * kPer);
      const T* ye = reinterpret_cast<const T*>(&y);
#pragma unroll
      for (int q = 0; q < kPer; ++q) acc[q] += w * Elem<T>::to_f32(ye[q]);
    }
    u32x4_t o;
    T* oe = reinterpret_cast<T*>(&o);
#pragma unroll
    for (int q = 0; q < kPer; ++q) oe[q] = Elem<T>::from_f32(acc[q]);
    st16(out + static_cast<int64_t>(tok0 + tt) * d + v * kPer, o);
  }
}

template <typename T>
hipError_t launch_t(const T* Yp, const int32_t* inv_perm, const float* w, T* out, int T_tok, int d, int k,
                    hipStream_t stream) {
  const int nblocks = (T_tok + kCombineTok - 1) / kCombineTok;
  const size_t shm = static_cast<size_t>(kCombineTok) * k * (sizeof(int) + sizeof(float));
  hipLaunchKernelGGL(combine_kernel<T>, dim3(nblocks), dim3(kCombineThreads), shm, stream, Yp, inv_perm, w, out,
                     T_tok, d, k);
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
