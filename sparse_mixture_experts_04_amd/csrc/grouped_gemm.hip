// Grouped GEMM over the experts' row segments on MFMA, with the GELU of the
// first expert Linear fused into its epilogue.
//
// Method: every expert is Linear -> GELU -> Linear without biases (Qwen2-MoE
// walk-through (mlqm.cn/news/48291) §2.2; "GPT-4 activates 2%" article
// (wmrh.cn/news/106769) §2.2), run only on the rows dispatched to it.  The
// walk-through's §3.2 loops over the experts one after another; here one
// launch covers all experts: a persistent grid walks a tile list built on the
// device from expert_offsets, so nothing is read back to the host.
//
//   C[r, n] = act( sum_k A[r, k] * B[e][n, k] ),  r in [offsets[e], offsets[e+1])
//
// Both operands are K-contiguous (B uses nn.Linear's [out, in] layout), so
// the 16-byte chunks that MFMA fragments consume are contiguous in memory and
// in LDS.  Tiles: BM x BN per block, 128 bytes of K per stage (64 bf16 or 32
// fp32), double-buffered LDS with an XOR swizzle of the 16-byte chunks so the
// fragment reads of 8 consecutive rows hit distinct banks.  Each wave owns a
// (BM/WM) x (BN/WN) sub-tile of 32x32 MFMA tiles.  The reduction order over K
// is a fixed permutation of the plain order, the same on A and B.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int kRowBytes = 128;                 // bytes of K per stage and row
constexpr int kChunks = kRowBytes / 16;        // 16-byte chunks per row and stage

template <typename T> struct GemmMma;
template <> struct GemmMma<uint16_t> {  // one 32x32x16 bf16 MFMA per 16-byte chunk pair
  static __device__ __forceinline__ f32x16_t run(u32x4_t a, u32x4_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                   0, 0, 0);
  }
};
template <> struct GemmMma<float> {     // four 32x32x2 fp32 MFMAs per 16-byte chunk pair
  static __device__ __forceinline__ f32x16_t run(u32x4_t a, u32x4_t b, f32x16_t c) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[q]), __uint_as_float(b[q]), c, 0, 0, 0);
    return c;
  }
};

__device__ __forceinline__ int swz(int row, int chunk) { return row * kRowBytes + ((chunk ^ (row & 7)) << 4); }

template <typename T, int BM, int BN, int WM, int WN, bool kGelu>
__global__ __launch_bounds__(WM * WN * kWave) void grouped_gemm_kernel(const T* __restrict__ A,
                                                                       const T* __restrict__ B, T* __restrict__ C,
                                                                       const int32_t* __restrict__ offsets, int E,
                                                                       int N, int K, int max_rows) {
  constexpr int kThreads = WM * WN * kWave;
  constexpr int kWTM = BM / WM;  // wave tile rows
  constexpr int kWTN = BN / WN;  // wave tile cols
  constexpr int kTM = kWTM / 32;
  constexpr int kTN = kWTN / 32;
  constexpr int kALd = BM * kChunks / kThreads;  // 16-byte loads per thread per stage
  constexpr int kBLd = BN * kChunks / kThreads;
  static_assert(kALd * kThreads == BM * kChunks && kBLd * kThreads == BN * kChunks, "tile/threads mismatch");
  static_assert(kTM >= 1 && kTN >= 1, "wave tile must hold 32x32 MFMA tiles");

  __shared__ __attribute__((aligned(16))) unsigned char sA[2][BM * kRowBytes];
  __shared__ __attribute__((aligned(16))) unsigned char sB[2][BN * kRowBytes];
  __shared__ int s_tile_base[kMaxExperts + 1];  // first m-tile of each expert
  __shared__ int s_seg0[kMaxExperts];            // expert row segments, clamped to [0, max_rows]
  __shared__ int s_seg1[kMaxExperts];

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = tid / kWave;
  const int wm = wave / WN;
  const int wn = wave % WN;

  if (tid < kWave) {
    const int e = tid;
    int mt = 0, seg0 = 0, seg1 = 0;
    if (e < E) {
      // Offsets come from device memory; clamping keeps every access inside
      // the [max_rows, K] and [max_rows, N] buffers even if they are corrupt.
      seg0 = min(max(offsets[e], 0), max_rows);
      seg1 = min(max(offsets[e + 1], seg0), max_rows);
      mt = (seg1 - seg0 + BM - 1) / BM;
    }
    int incl = mt;
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) {
      const int o = __shfl_up(incl, m);
      if (lane >= m) incl += o;
    }
    if (e < E) {
      s_tile_base[e + 1] = incl;
      s_seg0[e] = seg0;
      s_seg1[e] = seg1;
    }
    if (e == 0) s_tile_base[0] = 0;
  }
  __syncthreads();

  const int n_tiles_n = (N + BN - 1) / BN;
  const int total = s_tile_base[E] * n_tiles_n;
  const int G = gridDim.x;
  // Blocks are dealt round-robin to the 8 XCDs; give each XCD a contiguous run
  // of tiles so tiles that share a weight tile share that XCD's L2.
  int first = blockIdx.x;
  if ((G & 7) == 0) first = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);

  const int kstages = K * static_cast<int>(sizeof(T)) / kRowBytes;
  const int64_t row_stride = static_cast<int64_t>(K) * sizeof(T);  // bytes

  for (int tile = first; tile < total; tile += G) {
    // tile -> (expert, n-tile, m-tile): expert-major, m-tile fastest.
    int e = 0;
    while (e + 1 < E && s_tile_base[e + 1] * n_tiles_n <= tile) ++e;
    const int mt_e = s_tile_base[e + 1] - s_tile_base[e];
    const int local = tile - s_tile_base[e] * n_tiles_n;
    const int nt = local / mt_e;
    const int mt = local % mt_e;
    const int seg0 = s_seg0[e];
    const int seg1 = s_seg1[e];
    const int m0 = seg0 + mt * BM;
    const int n0 = nt * BN;

    const unsigned char* Ab = reinterpret_cast<const unsigned char*>(A);
    const unsigned char* Bb = reinterpret_cast<const unsigned char*>(B + static_cast<int64_t>(e) * N * K);

    // Per-thread load slots: chunk q = tid + i*kThreads -> row q/8, chunk q%8.
    const unsigned char* a_src[kALd];
    int a_dst[kALd];
#pragma unroll
    for (int i = 0; i < kALd; ++i) {
      const int q = tid + i * kThreads;
      const int r = q / kChunks;
      const int c = q % kChunks;
      const int grow = min(m0 + r, seg1 - 1);  // rows past the segment repeat its last row; never stored
      a_src[i] = Ab + grow * row_stride + c * 16;
      a_dst[i] = swz(r, c);
    }
    const unsigned char* b_src[kBLd];
    int b_dst[kBLd];
#pragma unroll
    for (int i = 0; i < kBLd; ++i) {
      const int q = tid + i * kThreads;
      const int r = q / kChunks;
      const int c = q % kChunks;
      const int gn = min(n0 + r, N - 1);
      b_src[i] = Bb + gn * row_stride + c * 16;
      b_dst[i] = swz(r, c);
    }

    f32x16_t acc[kTM][kTN];
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
      for (int j = 0; j < kTN; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

    u32x4_t ra[kALd], rb[kBLd];
#pragma unroll
    for (int i = 0; i < kALd; ++i) ra[i] = ld16(a_src[i]);
#pragma unroll
    for (int i = 0; i < kBLd; ++i) rb[i] = ld16(b_src[i]);
    __syncthreads();  // previous tile's readers of buffer 0 are done
#pragma unroll
    for (int i = 0; i < kALd; ++i) *reinterpret_cast<u32x4_t*>(sA[0] + a_dst[i]) = ra[i];
#pragma unroll
    for (int i = 0; i < kBLd; ++i) *reinterpret_cast<u32x4_t*>(sB[0] + b_dst[i]) = rb[i];
    __syncthreads();

    const int frow = lane % 32;
    const int fhalf = lane / 32;
    for (int ks = 0; ks < kstages; ++ks) {
      const int cur = ks & 1;
      if (ks + 1 < kstages) {
        const int64_t off = static_cast<int64_t>(ks + 1) * kRowBytes;
#pragma unroll
        for (int i = 0; i < kALd; ++i) ra[i] = ld16(a_src[i] + off);
#pragma unroll
        for (int i = 0; i < kBLd; ++i) rb[i] = ld16(b_src[i] + off);
      }
#pragma unroll
      for (int kk = 0; kk < kChunks / 2; ++kk) {
        const int ch = kk * 2 + fhalf;
        u32x4_t fa[kTM], fb[kTN];
#pragma unroll
        for (int i = 0; i < kTM; ++i)
          fa[i] = *reinterpret_cast<const u32x4_t*>(sA[cur] + swz(wm * kWTM + i * 32 + frow, ch));
#pragma unroll
        for (int j = 0; j < kTN; ++j)
          fb[j] = *reinterpret_cast<const u32x4_t*>(sB[cur] + swz(wn * kWTN + j * 32 + frow, ch));
#pragma unroll
        for (int i = 0; i < kTM; ++i)
#pragma unroll
          for (int j = 0; j < kTN; ++j) acc[i][j] = GemmMma<T>::run(fa[i], fb[j], acc[i][j]);
      }
      if (ks + 1 < kstages) {
#pragma unroll
        for (int i = 0; i < kALd; ++i) *reinterpret_cast<u32x4_t*>(sA[cur ^ 1] + a_dst[i]) = ra[i];
#pragma unroll
        for (int i = 0; i < kBLd; ++i) *reinterpret_cast<u32x4_t*>(sB[cur ^ 1] + b_dst[i]) = rb[i];
      }
      __syncthreads();
    }

    // Epilogue.  acc[i][j][q]: row (q/4)*8 + fhalf*4 + q%4, column frow of the 32x32 tile.
#pragma unroll
    for (int i = 0; i < kTM; ++i) {
#pragma unroll
      for (int j = 0; j < kTN; ++j) {
        const int col = n0 + wn * kWTN + j * 32 + frow;
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int row = m0 + wm * kWTM + i * 32 + (q / 4) * 8 + fhalf * 4 + (q % 4);
          if (row < seg1 && col < N) {
            float v = acc[i][j][q];
            if (kGelu) v = gelu_tanh(v);
            C[static_cast<int64_t>(row) * N + col] = Elem<T>::from_f32(v);
          }
        }
      }
    }
  }
}

struct GemmShape {
  int BM, BN;
};

template <typename T, int BM, int BN, int WM, int WN>
hipError_t launch_cfg(bool gelu, const T* A, const T* B, T* C, const int32_t* offsets, int E, int N, int K,
                      int max_rows, hipStream_t stream) {
  const int n_tiles_n = (N + BN - 1) / BN;
  const int64_t upper = (static_cast<int64_t>((max_rows + BM - 1) / BM) + E) * n_tiles_n;
  const int blocks_per_cu = 2;
  int64_t grid = static_cast<int64_t>(device_cu_count()) * blocks_per_cu;
  if (upper < grid) grid = upper;
  if (grid < 1) grid = 1;
  if (gelu)
    hipLaunchKernelGGL((grouped_gemm_kernel<T, BM, BN, WM, WN, true>), dim3(static_cast<unsigned>(grid)),
                       dim3(WM * WN * kWave), 0, stream, A, B, C, offsets, E, N, K, max_rows);
  else
    hipLaunchKernelGGL((grouped_gemm_kernel<T, BM, BN, WM, WN, false>), dim3(static_cast<unsigned>(grid)),
                       dim3(WM * WN * kWave), 0, stream, A, B, C, offsets, E, N, K, max_rows);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_grouped_gemm(int dtype, bool gelu, const void* A, const void* B, void* C, const int32_t* offsets,
                               int E, int N, int K, int max_rows, hipStream_t stream) {
  if (max_rows <= 0) return hipSuccess;
  if (dtype == kDtypeBF16)
    return launch_cfg<uint16_t, 128, 128, 2, 2>(gelu, static_cast<const uint16_t*>(A), static_cast<const uint16_t*>(B),
                                                static_cast<uint16_t*>(C), offsets, E, N, K, max_rows, stream);
  return launch_cfg<float, 64, 64, 2, 2>(gelu, static_cast<const float*>(A), static_cast<const float*>(B),
                                         static_cast<float*>(C), offsets, E, N, K, max_rows, stream);
}

}  // namespace moe
