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
#include <type_traits>

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

// ---------------------------------------------------------------------------
// bf16 main kernel: 256x256 tiles, 8 waves of 128 token rows x 64 weight
// rows (or 4 waves of 128x128), 32x32x16 MFMAs, fed by direct buffer->LDS
// loads through a ring of LDS units.
//
// * A unit is 64 K-elements (128 bytes: one full cache line per row) of the
//   256 rows of one operand, 32 KB.  A stage is one weight unit and one token
//   unit.  Five units (160 KB of LDS) form a ring: while stage s is consumed,
//   stage s+1 has landed or is landing and the weight unit of stage s+2 is in
//   flight, so the weight rows (the operand that misses L2 most) are requested
//   two stages ahead and the token rows one stage ahead.  The two unit streams
//   run continuously across the persistent block's tiles.
// * Loads go through buffer resources whose range covers only the tile's
//   valid rows: rows past an expert's segment or past N read as zero without
//   any clamping, and per-lane offsets are 32-bit and fixed for the kernel.
// * LDS layout: row r of a unit at r*128; its 16-byte chunk c at chunk
//   c ^ key(r), with keys chosen so the fragment reads of every 16 lanes hit 16
//   distinct 16-byte bank groups (64 banks).
// * The weight rows are the MFMA A operand and the token rows the B operand,
//   so a lane of the 32x32 result holds one token row.  The weight rows of
//   each 32-row fragment are read in the order pi(x) = 16*((x>>2)&1) +
//   4*(x>>3) + (x&3), which makes a lane's 16 results 16 consecutive output
//   columns: two 16-byte stores.
// * One barrier per stage (four 16-element k-steps).
constexpr int kBig = 256;                                 // BM = BN
// Waves per block of the 256x256 kernel: 8, two per SIMD, each computing 128
// token rows x 64 weight rows (128 accumulator registers), so one wave's
// waits on loads, LDS reads or the barrier are covered by the other wave's
// MFMAs.  The kernel also builds with 4 waves (one per SIMD, 128 x 128 each,
// 256 accumulator registers); the results are bitwise the same (same
// fragments, same K order per output), and on MI355X 8 waves measured
// 1.5-5% faster on every expert GEMM of the prefill, capacity and skewed
// layers.
constexpr int kBigWaves = 8;
constexpr int kUnitRow = 128;                             // K bytes per row per unit
constexpr int kUnitBytes = kBig * kUnitRow;               // 32 KB
constexpr int kSlots = 5;
constexpr size_t kBigLds = static_cast<size_t>(kSlots) * kUnitBytes;  // 160 KB
// Word 3 of a raw (unstructured) buffer resource on the gfx9 family: 32-bit
// data format, no swizzle; bounds are checked against num_records in bytes.
constexpr int kRsrcWord3 = 0x00020000;

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ int key_x(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int key_w(int r) { return ((r >> 1) & 3) | (((r >> 4) & 1) << 2); }

// x * sigmoid(2u) = 0.5 x (1 + tanh(u)), u = sqrt(2/pi) (x + 0.044715 x^3),
// with the hardware exp2 and reciprocal (about 1 ulp each).  -2 log2(e) u is
// formed as x * (c + 0.044715 c x^2), c = -2 log2(e) sqrt(2/pi): five VALU
// operations and two transcendentals per value.  Large |x| saturates
// correctly: exp2 -> inf gives -0, exp2 -> 0 gives x.
__device__ __forceinline__ float gelu_tanh_fast(float x) {
  constexpr float kC = -2.0f * 1.4426950408889634f * 0.7978845608028654f;
  const float p = fmaf(kC * 0.044715f, x * x, kC);
  return x * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(x * p));
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  // gfx9 s_waitcnt: vmcnt[3:0] and [15:14], expcnt[6:4] (7 = no wait), lgkmcnt[11:8] (15 = no wait)
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
template <int N>
__device__ __forceinline__ void wait_vmcnt_lgkm0() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

struct TileCoord {
  int e, m0, n0, rows;  // rows: the tile's token rows [m0, m0 + rows)
};

// kGather: the token rows are not stored in expert order.  Row r of the
// expert-ordered operand is row gidx[r] / gdiv of A, which then has src_rows
// rows: the dispatch permutation (entries token*k + slot) read with gdiv = k
// gathers each token's hidden state straight from the layer input.
template <bool kGelu, bool kGather, int kWaves>
__global__ __launch_bounds__(kWaves * kWave) void grouped_gemm_bf16_256(const uint16_t* __restrict__ A,
                                                                        const uint16_t* __restrict__ B,
                                                                        uint16_t* __restrict__ C,
                                                                        const int32_t* __restrict__ offsets, int E,
                                                                        int N, int K, int max_rows,
                                                                        const int32_t* __restrict__ gidx, int gdiv,
                                                                        int src_rows) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  static_assert(kWaves == 4 || kWaves == 8, "4 waves (one per SIMD) or 8 (two per SIMD)");
  // Waves split the tile into 2 token halves x kWN weight parts; a wave
  // holds kWF 32-row weight fragments and fills kRowsW rows of each unit.
  constexpr int kWN = kWaves / 2;
  constexpr int kWF = 8 / kWN;
  constexpr int kRowsW = kBig / kWaves;
  constexpr int kLd = kRowsW / 8;  // 16-byte loads per lane per unit

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // uniform: LDS bases stay scalar
  const int wm = wave / kWN;  // token half of the tile
  const int wn = wave % kWN;  // weight part of the tile

  // Expert table, held by every wave in registers: lane e has expert e's row
  // segment [seg0, seg1) (clamped to [0, max_rows]: offsets come from device
  // memory) and the running count of m-tiles before and through it.
  // An expert of R rows gets ceil(R/H) m-tiles of equal height (rounded up
  // to 32 rows, the last one shorter): with H = 256 a 530-row expert runs
  // tiles of 192, 192 and 146 rows rather than 256, 256 and 18, and each
  // tile runs only as many 32-row token fragments as it has rows.  Equal
  // fragment counts keep the m-tiles that share a weight tile in lockstep
  // (a 463-row expert under H = 192: 160, 160, 143 rather than 192, 192, 79).
  int t_seg0 = 0, t_seg1 = 0;
  if (lane < E) {
    t_seg0 = min(max(offsets[lane], 0), max_rows);
    t_seg1 = min(max(offsets[lane + 1], t_seg0), max_rows);
  }
  const int t_rows = t_seg1 - t_seg0;
  const int n_tiles_n = (N + kBig - 1) / kBig;
  const int G = gridDim.x;
  // The height cap H (128, 192 or 256 rows) is chosen per launch from an
  // estimate of the run: the G blocks take the tiles in rounds, so the run
  // is about ceil(tiles / G) rounds of one tile each, and a tile of h rows
  // costs about kTileCost[h/64 - 1] (relative per-stage times of 64-, 128-,
  // 192- and 256-row tiles measured on MI355X with a weight tile per tile).
  // The estimate overstates what smaller tiles gain (they share each weight
  // tile among more m-tiles, and the GPU is partly bandwidth-bound), so a
  // smaller cap must be estimated at least 8% faster.  Experts of 460-570
  // rows on 8 n-tiles (N = 2048) run 3 full rounds of 192-row tiles about
  // 2.5% faster than 2.5 rounds of 256-row ones.  Every block computes the
  // same choice.
  int H = kBig;
  {
    constexpr int kTileCost[4] = {70, 76, 88, 100};
    int best = 0;
#pragma unroll
    for (int c = 4; c >= 2; --c) {
      int m = (t_rows + 64 * c - 1) / (64 * c);
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) m += __shfl_xor(m, o);
      const int rounds = (m * n_tiles_n + G - 1) / G;
      const int est = rounds * kTileCost[c - 1];
      if (c == 4) {
        best = est;
      } else if (est * 100 < best * 92) {
        best = est;
        H = 64 * c;
      }
    }
    H = __builtin_amdgcn_readfirstlane(H);
  }
  int t_mt = 0, t_h = H;
  if (lane < E) {
    t_mt = (t_rows + H - 1) / H;
    if (t_mt > 0) t_h = min(H, ((t_rows + t_mt - 1) / t_mt + 31) & ~31);
  }
  int t_incl = t_mt;
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) {
    const int o = __shfl_up(t_incl, m);
    if (lane >= m) t_incl += o;
  }
  const int total = __builtin_amdgcn_readlane(t_incl, E - 1) * n_tiles_n;
  int first = blockIdx.x;
  if ((G & 7) == 0) first = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
  if (first >= total) return;
  const int kstages = K * 2 / kUnitRow;
  const int row_stride = K * 2;  // bytes; 256 rows of it fit in 31 bits (checked by the host)

  // tile -> (expert, m-tile, n-tile).  Within an expert, tiles run in groups
  // of up to kGroupM m-tiles: all n-tiles of the group, m-tile fastest, so a
  // block's run of consecutive tiles (one XCD's share) covers a few m-tiles x
  // a few n-tiles and reuses both operands from that XCD's L2.
  auto coord = [&](int tile) {
    constexpr int kGroupM = 8;
    const unsigned long long done = __ballot(lane < E && t_incl * n_tiles_n <= tile);
    const int e = __builtin_amdgcn_readfirstlane(static_cast<int>(__popcll(done)));
    const int incl = __builtin_amdgcn_readlane(t_incl, e);
    const int mt_e = __builtin_amdgcn_readlane(t_mt, e);
    const int local = tile - (incl - mt_e) * n_tiles_n;
    const int group = local / (kGroupM * n_tiles_n);
    const int first_m = group * kGroupM;
    const int gsize = min(kGroupM, mt_e - first_m);
    const int in = local - group * kGroupM * n_tiles_n;
    TileCoord t;
    t.e = e;
    t.n0 = (in / gsize) * kBig;
    t.m0 = __builtin_amdgcn_readlane(t_seg0, e) + (first_m + in % gsize) * __builtin_amdgcn_readlane(t_h, e);
    t.rows = min(__builtin_amdgcn_readlane(t_h, e), __builtin_amdgcn_readlane(t_seg1, e) - t.m0);
    return t;
  };

  // ---- producers: one stream of weight units and one of token units.
  // Instruction i of this wave fills rows wave*kRowsW + i*8 .. +7 of a unit
  // (1 KB of LDS); lane p fills row wave*kRowsW + i*8 + p/8, physical chunk p%8.
  int vw[kLd], vx[kLd];
#pragma unroll
  for (int i = 0; i < kLd; ++i) {
    const int r = wave * kRowsW + i * 8 + (lane >> 3);
    vw[i] = r * row_stride + (((lane & 7) ^ key_w(r)) << 4);
    vx[i] = r * row_stride + (((lane & 7) ^ key_x(r)) << 4);
  }
  const unsigned char* const Ab = reinterpret_cast<const unsigned char*>(A);
  const unsigned char* const Bb = reinterpret_cast<const unsigned char*>(B);
  struct Stream {
    const unsigned char* base;  // first row of the tile's operand
    int rows;                   // valid rows (0 past the last tile)
    int tile, ks, slot;
  };
  Stream ws{nullptr, 0, first, 0, 0};  // weight unit of stage s -> slot 2s mod 5
  Stream xs{nullptr, 0, first, 0, 1};  // token unit of stage s -> slot 2s+1 mod 5
  auto setup_w = [&](Stream& s) {
    if (s.tile < total) {
      const TileCoord t = coord(s.tile);
      s.base = Bb + (static_cast<int64_t>(t.e) * N + t.n0) * row_stride;
      s.rows = min(N - t.n0, kBig);
    } else {
      s.rows = 0;
    }
  };
  // Gathered token rows: the token stream's per-lane offsets change with the
  // tile.  g[i] receives the gather index of row wave*kRowsW + i*8 + lane/8 of
  // a tile; the stage loop loads them at the start of the stage whose token
  // unit is the stream's last of its tile, before that stage's weight unit,
  // so the stage wait (which leaves only that weight unit in flight) covers
  // them and the offsets are formed at the stream's tile switch without a
  // wait of their own.
  auto load_gidx = [&](int* g, int tile) {
    if (tile < total) {
      const TileCoord t = coord(tile);
      const __amdgpu_buffer_rsrc_t grsrc = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<int32_t*>(gidx) + t.m0, 0, t.rows * 4, kRsrcWord3);
#pragma unroll
      for (int i = 0; i < kLd; ++i)
        g[i] = __builtin_amdgcn_raw_buffer_load_b32(grsrc, (wave * kRowsW + i * 8 + (lane >> 3)) * 4, 0, 0);
    }
  };
  auto setup_x = [&](Stream& s, const int* g) {
    if (s.tile < total) {
      const TileCoord t = coord(s.tile);
      if constexpr (kGather) {
        // Rows past the tile (or a source row out of range) get an offset
        // beyond the resource: they load zeros.
        s.base = Ab;
        s.rows = src_rows;
#pragma unroll
        for (int i = 0; i < kLd; ++i) {
          const int r = wave * kRowsW + i * 8 + (lane >> 3);
          const unsigned src = static_cast<unsigned>(g[i]) / static_cast<unsigned>(gdiv);
          vx[i] = r < t.rows && src < static_cast<unsigned>(src_rows)
                      ? static_cast<int>(src) * row_stride + (((lane & 7) ^ key_x(r)) << 4)
                      : static_cast<int>(0x80000000u);
        }
      } else {
        s.base = Ab + static_cast<int64_t>(t.m0) * row_stride;
        s.rows = t.rows;
      }
    } else {
      s.rows = 0;
    }
  };
  // Issue one unit (kLd loads of 1 KB per wave).  Past the last tile the
  // range is empty: the loads return zeros into a free slot without touching
  // memory.
  auto issue = [&](const Stream& s, const int* voff) {
    const int koff = s.ks * kUnitRow;
    const int nrec = max(s.rows * row_stride - koff, 0);
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned char*>(s.base) + koff, 0, nrec, kRsrcWord3);
    unsigned char* dst = smem + s.slot * kUnitBytes + wave * kRowsW * kUnitRow;
#pragma unroll
    for (int i = 0; i < kLd; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_ptr_t)(dst + i * 8 * kUnitRow), 16, voff[i], 0, 0, 0);
  };
  auto advance_w = [&](Stream& s) {
    s.slot = s.slot + 2 >= kSlots ? s.slot + 2 - kSlots : s.slot + 2;
    if (++s.ks == kstages) {
      s.ks = 0;
      s.tile += G;
      setup_w(s);
    }
  };
  // g: the gather indices of tile s.tile + G (used only when the stream
  // moves there).
  auto advance_x = [&](Stream& s, const int* g) {
    s.slot = s.slot + 2 >= kSlots ? s.slot + 2 - kSlots : s.slot + 2;
    if (++s.ks == kstages) {
      s.ks = 0;
      s.tile += G;
      setup_x(s, g);
    }
  };

  setup_w(ws);
  int gp[kLd];
  if constexpr (kGather) load_gidx(gp, first);
  setup_x(xs, gp);
  // Prologue: stages 0 and 1 (units 0..3).
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    issue(ws, vw);
    advance_w(ws);
    issue(xs, vx);
    if constexpr (kGather)
      if (xs.ks == kstages - 1) load_gidx(gp, xs.tile + G);
    advance_x(xs, gp);
  }

  const int frow = lane & 31;
  const int fhalf = lane >> 5;
  const int wrow = ((frow >> 2) & 1) * 16 + (frow >> 3) * 4 + (frow & 3);  // pi(frow)
  const int kx = key_x(frow);  // = key_x of every token row this lane reads
  const int kw = key_w(wrow);  // = key_w of every weight row this lane reads
  int c_wslot = 0, c_xslot = 1;

  // Fragments of one 16-element k-step: kWF weight and up to 4 token
  // fragments.  Token fragment j of this wave covers tile rows
  // (2j + wm)*32 .. +31: the two token-half waves interleave, so a tile of R
  // rows has ceil(R/32) fragments with rows and each wave runs
  // nj = ceil(ceil(R/32)/2) of them (both waves the same count, so the
  // per-stage barrier costs no idle MFMA time).
  u32x4_t wf0[kWF], xf0[4], wf1[kWF], xf1[4];
  auto frag_addr_w = [&](int kk, int i) {
    return smem + c_wslot * kUnitBytes + (wn * (kWF * 32) + i * 32 + wrow) * kUnitRow +
           (((kk * 2 + fhalf) ^ kw) << 4);
  };
  auto frag_addr_x = [&](int kk, int j) {
    return smem + c_xslot * kUnitBytes + ((2 * j + wm) * 32 + frow) * kUnitRow + (((kk * 2 + fhalf) ^ kx) << 4);
  };
  auto read_frags = [&](auto nj_c, int kk, u32x4_t (&wf)[kWF], u32x4_t (&xf)[4]) {
    constexpr int NJ = decltype(nj_c)::value;
#pragma unroll
    for (int i = 0; i < kWF; ++i) wf[i] = *reinterpret_cast<const u32x4_t*>(frag_addr_w(kk, i));
#pragma unroll
    for (int j = 0; j < NJ; ++j) xf[j] = *reinterpret_cast<const u32x4_t*>(frag_addr_x(kk, j));
  };
  // One k-step block, in a fixed issue order: its kWF*NJ MFMAs, with the
  // kWF+NJ fragment reads of k-step `kk_next` (into wn/xn) spread over the
  // first half of them and, if `s` is given, a unit's kLd buffer->LDS loads
  // spread over the first kLd, so neither the LDS nor the load queue holds up
  // the MFMA stream.
  auto block = [&](auto nj_c, f32x16_t (&acc)[kWF][4], const u32x4_t (&wa)[kWF], const u32x4_t (&xa)[4],
                   int kk_next, u32x4_t (&wn_)[kWF], u32x4_t (&xn_)[4], const Stream* s, const int* voff) {
    constexpr int NJ = decltype(nj_c)::value;
    constexpr int kM = kWF * NJ;
    constexpr int kR = kWF + NJ;
    constexpr int kRq = (kM + 1) / 2;
    constexpr int kLq = kM < kLd ? kM : kLd;
    __amdgpu_buffer_rsrc_t rsrc;
    unsigned char* dst = smem;
    if (s != nullptr) {
      const int koff = s->ks * kUnitRow;
      const int nrec = max(s->rows * row_stride - koff, 0);
      rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned char*>(s->base) + koff, 0, nrec, kRsrcWord3);
      dst = smem + s->slot * kUnitBytes + wave * kRowsW * kUnitRow;
    }
#pragma unroll
    for (int q = 0; q < kM; ++q) {
      const int i = q / NJ, j = q % NJ;
      acc[i][j] = GemmMma<uint16_t>::run(wa[i], xa[j], acc[i][j]);
      if (kk_next >= 0 && q < kRq) {
#pragma unroll
        for (int r = q * kR / kRq; r < (q + 1) * kR / kRq; ++r) {
          if (r < kWF) wn_[r] = *reinterpret_cast<const u32x4_t*>(frag_addr_w(kk_next, r));
          else xn_[r - kWF] = *reinterpret_cast<const u32x4_t*>(frag_addr_x(kk_next, r - kWF));
        }
      }
      if (s != nullptr && q < kLq) {
#pragma unroll
        for (int l = q * kLd / kLq; l < (q + 1) * kLd / kLq; ++l)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_ptr_t)(dst + l * 8 * kUnitRow), 16, voff[l], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto barrier = [&]() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  // Stage 0 must be resident before its first fragments are read (stage 1,
  // 2*kLd loads, may still be in flight).
  wait_vmcnt<2 * kLd>();
  barrier();
  // Stores of the last epilogue: issued after the next stage's data, so the
  // stage-end wait may leave them in flight (vector memory operations
  // retire in issue order: loads and stores count down vmcnt in one order).
  int pending_st = 0;

  // One tile: all K stages with nj token fragments per wave, then its
  // epilogue.  k-step 0 of the tile's first stage is read here (the previous
  // tile's last block read it with that tile's nj).
  auto run_tile = [&](auto nj_c, const TileCoord& tc) {
    constexpr int NJ = decltype(nj_c)::value;
    f32x16_t acc[kWF][4];
#pragma unroll
    for (int i = 0; i < kWF; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;
    read_frags(nj_c, 0, wf0, xf0);

    for (int ks = 0; ks < kstages; ++ks) {
      int gn[kLd];
      if constexpr (kGather) {
        if (xs.ks == kstages - 1) load_gidx(gn, xs.tile + G);
        __builtin_amdgcn_sched_barrier(0);
      }
      // k-step 0 of this stage is in wf0/xf0.  Its block also issues the
      // weight unit two stages ahead.
      block(nj_c, acc, wf0, xf0, 1, wf1, xf1, &ws, vw);
      advance_w(ws);
      block(nj_c, acc, wf1, xf1, 2, wf0, xf0, nullptr, nullptr);
      block(nj_c, acc, wf0, xf0, 3, wf1, xf1, nullptr, nullptr);
      // The next stage must have landed; the weight unit issued above may stay
      // in flight, and right after an epilogue so may its stores (2 per
      // accumulator group, issued between the next stage's token unit and
      // that weight unit).  lgkmcnt(0): this wave's reads of this stage are
      // complete, so after the barrier its two units are free.
      switch (pending_st) {
        case 0: wait_vmcnt_lgkm0<kLd>(); break;
        case 4: wait_vmcnt_lgkm0<kLd + 4>(); break;
        case 8: wait_vmcnt_lgkm0<kLd + 8>(); break;
        case 12: wait_vmcnt_lgkm0<kLd + 12>(); break;
        default: wait_vmcnt_lgkm0<kLd + 16>(); break;  // 16 (more with 4 waves: a lower count only waits longer)
      }
      pending_st = 0;
      barrier();
      __builtin_amdgcn_sched_barrier(0);
      c_wslot = c_wslot + 2 >= kSlots ? c_wslot + 2 - kSlots : c_wslot + 2;
      c_xslot = c_xslot + 2 >= kSlots ? c_xslot + 2 - kSlots : c_xslot + 2;
      // Refill a freed slot with the token unit of the stage after next, and
      // read k-step 0 of the next stage (past the last stage: a free slot
      // whose values go unused).
      block(nj_c, acc, wf1, xf1, 0, wf0, xf0, &xs, vx);
      advance_x(xs, gn);
    }
    pending_st = 2 * kWF * NJ;

    // acc[i][j][q]: token row m0 + (2j + wm)*32 + frow, column n0 + wn*kWF*32 + i*32 + 16*fhalf + q.
    // Stores go through a buffer resource over the tile's rows of C; a
    // column past N gets an offset beyond the range.  The hardware drops
    // out-of-range stores, so the epilogue has no branches and each group of
    // 16 accumulators is read, converted and stored before the next.
    const __amdgpu_buffer_rsrc_t crsrc = __builtin_amdgcn_make_buffer_rsrc(
        C + static_cast<int64_t>(tc.m0) * N, 0, tc.rows * N * 2, kRsrcWord3);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int roff = ((2 * j + wm) * 32 + frow) * N * 2;
#pragma unroll
      for (int i = 0; i < kWF; ++i) {
        const int col = tc.n0 + wn * (kWF * 32) + i * 32 + 16 * fhalf;
        const int off = col < N ? roff + col * 2 : static_cast<int>(0x80000000u);
        // Redefine the group's accumulators here (an empty asm on their
        // registers), after the previous group's stores: otherwise the
        // compiler copies all of them out of the accumulator registers at the
        // loop exit and runs out of registers for the GELU.
        asm volatile("" : "+a"(acc[i][j])::"memory");
        float v[16];
#pragma unroll
        for (int q = 0; q < 16; ++q) v[q] = kGelu ? gelu_tanh_fast(acc[i][j][q]) : acc[i][j][q];
        u32x4_t lo, hi;
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          lo[h] = pack_bf16x2(v[2 * h], v[2 * h + 1]);
          hi[h] = pack_bf16x2(v[8 + 2 * h], v[8 + 2 * h + 1]);
        }
        __builtin_amdgcn_raw_buffer_store_b128(lo, crsrc, off, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(hi, crsrc, off + 16, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  for (int tile = first; tile < total; tile += G) {
    const TileCoord tc = coord(tile);
    const int nj = (((tc.rows + 31) >> 5) + 1) >> 1;  // 1..4
    if (nj >= 4) run_tile(std::integral_constant<int, 4>{}, tc);
    else if (nj == 3) run_tile(std::integral_constant<int, 3>{}, tc);
    else if (nj == 2) run_tile(std::integral_constant<int, 2>{}, tc);
    else run_tile(std::integral_constant<int, 1>{}, tc);
  }
  wait_vmcnt<0>();
}

template <bool kGelu, bool kGather>
hipError_t launch_big(const uint16_t* A, const uint16_t* B, uint16_t* C, const int32_t* offsets, int E, int N, int K,
                      int max_rows, const int32_t* gidx, int gdiv, int src_rows, hipStream_t stream) {
  static const hipError_t attr =
      hipFuncSetAttribute(reinterpret_cast<const void*>(&grouped_gemm_bf16_256<kGelu, kGather, kBigWaves>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(kBigLds));
  if (attr != hipSuccess) return attr;
  // 32-bit buffer offsets: 256 rows of K (operands) or N (results) bf16, and
  // for a gather all src_rows rows of A, must stay below 2^31 bytes.
  if (static_cast<int64_t>(K) * 2 * kBig >= (int64_t{1} << 31) ||
      static_cast<int64_t>(N) * 2 * kBig >= (int64_t{1} << 31))
    return hipErrorInvalidValue;
  if (kGather && (gidx == nullptr || gdiv < 1 || src_rows < 0 ||
                  static_cast<int64_t>(src_rows) * K * 2 >= (int64_t{1} << 31)))
    return hipErrorInvalidValue;
  const int n_tiles_n = (N + kBig - 1) / kBig;
  // At most this many tiles (m-tiles of at least 128 rows but the last of each expert).
  const int64_t upper = (static_cast<int64_t>((max_rows + 127) / 128) + E) * n_tiles_n;
  int64_t grid = device_cu_count();
  if (upper < grid) grid = upper;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL((grouped_gemm_bf16_256<kGelu, kGather, kBigWaves>), dim3(static_cast<unsigned>(grid)),
                     dim3(kBigWaves * kWave), kBigLds, stream, A, B, C, offsets, E, N, K, max_rows, gidx, gdiv,
                     src_rows);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Skinny variant for few rows per expert where the decode variant below does
// not run (K not a multiple of 128 or N not of 8, or up to 64 rows per expert
// on a batch averaging more than 16): the layer is bound by streaming each
// active expert's weights once.  A one-wave block owns 16 weight rows (one
// 16-row MFMA A tile) over the whole K and up to 64 of the expert's token
// rows (up to four 16-column B tiles),
// so every weight byte is loaded exactly once, with 8 k-steps of loads in
// flight per lane.  Small blocks keep the per-CU work even when the number of
// (expert, row tile) pairs is not a multiple of the CU count.  The result tile
// is transposed (weights on rows): a lane holds 4 consecutive output columns
// of one token row.  Blocks map to (active expert, 16-row tile) on the
// device; blocks past the end exit.
constexpr int kSkinnyRows = 16;          // weight rows per wave
constexpr int kSkinnyMaxTok = 64;        // token rows per expert this kernel handles
constexpr int kSkinnyUnroll = 8;

template <bool kGelu, int kGroups>
__global__ __launch_bounds__(kWave) void grouped_gemm_bf16_skinny(const uint16_t* __restrict__ A,
                                                                  const uint16_t* __restrict__ B,
                                                                  uint16_t* __restrict__ C,
                                                                  const int32_t* __restrict__ offsets, int E, int N,
                                                                  int K, int max_rows) {
  __shared__ int s_tile_base[kMaxExperts + 1];
  __shared__ int s_seg0[kMaxExperts];
  __shared__ int s_seg1[kMaxExperts];
  const int lane = threadIdx.x;
  const int n_tiles = (N + kSkinnyRows - 1) / kSkinnyRows;
  {
    const int e = lane;
    int nt = 0, seg0 = 0, seg1 = 0;
    if (e < E) {
      seg0 = min(max(offsets[e], 0), max_rows);
      seg1 = min(max(offsets[e + 1], seg0), max_rows);
      nt = seg1 > seg0 ? n_tiles : 0;
    }
    int incl = nt;
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
  const int tile = blockIdx.x;
  if (tile >= s_tile_base[E]) return;
  int e = 0;
  while (e + 1 < E && s_tile_base[e + 1] <= tile) ++e;
  const int n0 = (tile - s_tile_base[e]) * kSkinnyRows;
  const int seg0 = s_seg0[e];
  const int all_rows = s_seg1[e] - seg0;

  const int r16 = lane & 15;
  const int g = lane >> 4;  // 16-byte chunk of a 64-byte k-step
  const int64_t stride = static_cast<int64_t>(K) * 2;
  const unsigned char* wp = reinterpret_cast<const unsigned char*>(B) +
                            (static_cast<int64_t>(e) * N + min(n0 + r16, N - 1)) * stride + g * 16;
  // A pass covers kGroups*16 token rows; an expert with more rows than that
  // (more than the bound the kernel was picked for) gets further passes.
  for (int tok0 = 0; tok0 < all_rows; tok0 += kGroups * 16) {
  const int rows = min(all_rows - tok0, kGroups * 16);
  const int groups = (rows + 15) / 16;
  const unsigned char* xp[kGroups];
#pragma unroll
  for (int j = 0; j < kGroups; ++j)
    xp[j] = reinterpret_cast<const unsigned char*>(A) +
            static_cast<int64_t>(seg0 + tok0 + min(j * 16 + r16, rows - 1)) * stride + g * 16;
  f32x4_t acc[kGroups];
#pragma unroll
  for (int j = 0; j < kGroups; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Register double buffering: the loads of the next kSkinnyUnroll steps are
  // in flight while the MFMAs of the current ones run.  Token loads are
  // unconditional (rows past the expert's last one repeat it; those results
  // are never stored), so the loop has no branches.
  constexpr int kU = kGroups == 1 ? kSkinnyUnroll : kSkinnyUnroll / 2;
  const int steps = K / 32;  // 64 bytes of K per step
  const int nblk = steps / kU;
  u32x4_t wa[2][kU], xb[2][kU][kGroups];
  auto load = [&](int buf, int blk) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t off = static_cast<int64_t>(blk * kU + u) * 64;
      wa[buf][u] = ld16(wp + off);
#pragma unroll
      for (int j = 0; j < kGroups; ++j) xb[buf][u][j] = ld16(xp[j] + off);
    }
  };
  auto mma = [&](int buf) {
#pragma unroll
    for (int u = 0; u < kU; ++u)
#pragma unroll
      for (int j = 0; j < kGroups; ++j)
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, wa[buf][u]),
                                                         __builtin_bit_cast(bf16x8_t, xb[buf][u][j]), acc[j], 0, 0, 0);
  };
  if (nblk > 0) load(0, 0);
  int blk = 0;
  for (; blk + 2 <= nblk; blk += 2) {
    load(1, blk + 1);
    mma(0);
    if (blk + 2 < nblk) load(0, blk + 2);
    mma(1);
  }
  if (blk < nblk) mma(0);  // odd block count: the last block sits in buffer 0
  for (int st = nblk * kU; st < steps; ++st) {
    const int64_t off = static_cast<int64_t>(st) * 64;
    const u32x4_t w = ld16(wp + off);
#pragma unroll
    for (int j = 0; j < kGroups; ++j) {
      const u32x4_t x = ld16(xp[j] + off);
      acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, w), __builtin_bit_cast(bf16x8_t, x),
                                                       acc[j], 0, 0, 0);
    }
  }
  // acc[j][q]: weight row n0 + g*4 + q, token row j*16 + r16.
#pragma unroll
  for (int j = 0; j < kGroups; ++j) {
    const int tok = j * 16 + r16;
    if (j >= groups || tok >= rows) continue;
    const int col = n0 + g * 4;
    if (col >= N) continue;
    float v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = kGelu ? gelu_tanh_fast(acc[j][q]) : acc[j][q];
    *reinterpret_cast<uint2*>(C + static_cast<int64_t>(seg0 + tok0 + tok) * N + col) =
        make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
  }
  }
}

// ---------------------------------------------------------------------------
// Decode variant (at most 64 token rows per expert possible): weight streaming with
// whole-line loads.  One 16x16x32 MFMA takes as its A operand 4 weight rows x
// 4 K-slices of 32 (each lane's 16 bytes; the 16 lanes of a row cover 256
// contiguous bytes of it) and as its B operand 4 token rows x the same 4
// K-slices.  Of the 16x16 products only the 4x4 diagonal blocks (matching
// K-slices) are wanted: lane l holds slice l%4 of the pair (weight row l/16,
// token (l%16)/4) in accumulator l%4, and two lane shuffles finish each dot
// product.  The 4x redundant MFMA work is cheap here, and in exchange every
// load instruction reads 4 rows x 256 contiguous bytes, which with the
// non-temporal policy streams the weights at close to full HBM bandwidth.
// A wave owns 8 weight rows (2 groups of 4) over the whole K, and a block is
// that one wave: many small blocks keep the weight stream evenly spread over
// the CUs to the end (1.7-2.5% faster than blocks of 4 waves and 32 rows on
// the decode layer's projections).  A pass covers kTG groups of 4
// token rows; token groups past the expert's row count are skipped (uniform
// per wave), and an expert with more rows than one pass holds gets further
// passes, so any row count is computed.  kGather: token row r of the
// expert-ordered operand is row gidx[r] / gdiv of A (src_rows rows), as in the
// 256x256 kernel; an index naming no row of A gives a zero row.
constexpr int kGvGroups = 2;        // 4-row weight groups per wave
constexpr int kGvWaves = 1;
constexpr int kGvRows = kGvWaves * kGvGroups * 4;  // weight rows per block
// Largest bound on the rows per expert (from the batch and capacity; the real
// counts are on the device) for which this kernel runs; see gemv_runs.
constexpr int kGvMaxTok = 64;

template <bool kGelu, int kTG, bool kGather>
__global__ __launch_bounds__(kGvWaves * kWave) void grouped_gemm_bf16_gemv(const uint16_t* __restrict__ A,
                                                                          const uint16_t* __restrict__ B,
                                                                          uint16_t* __restrict__ C,
                                                                          const int32_t* __restrict__ offsets,
                                                                          int E, int N, int K, int max_rows,
                                                                          const int32_t* __restrict__ gidx, int gdiv,
                                                                          int src_rows) {
  __shared__ int s_tile_base[kMaxExperts + 1];
  __shared__ int s_seg0[kMaxExperts];
  __shared__ int s_seg1[kMaxExperts];
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = tid / kWave;
  const int n_tiles = (N + kGvRows - 1) / kGvRows;
  if (tid < kWave) {
    const int e = lane;
    int nt = 0, seg0 = 0, seg1 = 0;
    if (e < E) {
      seg0 = min(max(offsets[e], 0), max_rows);
      seg1 = min(max(offsets[e + 1], seg0), max_rows);
      nt = seg1 > seg0 ? n_tiles : 0;
    }
    int incl = nt;
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
  const int tile = blockIdx.x;
  if (tile >= s_tile_base[E]) return;
  int e = 0;
  while (e + 1 < E && s_tile_base[e + 1] <= tile) ++e;
  const int n0 = (tile - s_tile_base[e]) * kGvRows + wave * kGvGroups * 4;
  if (n0 >= N) return;  // N is a multiple of 8: a wave's rows are all valid or all past the end
  const int seg0 = s_seg0[e];
  const int rows = s_seg1[e] - seg0;

  const int i16 = lane & 15;
  const int g = lane >> 4;
  const int row_bytes = K * 2;
  const int lane_off = 64 * (i16 & 3) + 16 * g;  // byte offset within a 256-byte K-chunk
  const unsigned char* wp[kGvGroups];
#pragma unroll
  for (int rg = 0; rg < kGvGroups; ++rg)
    wp[rg] = reinterpret_cast<const unsigned char*>(B) +
             (static_cast<int64_t>(e) * N + n0 + rg * 4 + (i16 >> 2)) * row_bytes + lane_off;
  constexpr int kU = 2;        // 256-byte K-chunks per step, register double-buffered across steps
  const int nchunk = K / 128;  // K is a multiple of 128 (checked by the host)
  const int nstep = nchunk / kU;

  for (int tok0 = 0; tok0 < rows; tok0 += kTG * 4) {
    const int ntok = min(rows - tok0, kTG * 4);
    const int ntg = (ntok + 3) / 4;
    const unsigned char* xp[kTG];
    bool xok[kTG];  // the row names a row of A (always, without a gather)
#pragma unroll
    for (int tg = 0; tg < kTG; ++tg) {
      const int r = seg0 + tok0 + min(tg * 4 + (i16 >> 2), ntok - 1);
      int64_t src = r;
      xok[tg] = true;
      if constexpr (kGather) {
        const unsigned u = static_cast<unsigned>(gidx[r]) / static_cast<unsigned>(gdiv);
        xok[tg] = u < static_cast<unsigned>(src_rows);
        src = xok[tg] ? u : 0;
      }
      xp[tg] = reinterpret_cast<const unsigned char*>(A) + src * row_bytes + lane_off;
    }
    auto ldx = [&](int tg, int64_t off) {
      const u32x4_t x = ld16(xp[tg] + off);
      return xok[tg] ? x : u32x4_t{0u, 0u, 0u, 0u};
    };

    f32x4_t acc[kGvGroups][kTG];
#pragma unroll
    for (int rg = 0; rg < kGvGroups; ++rg)
#pragma unroll
      for (int tg = 0; tg < kTG; ++tg) acc[rg][tg] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    u32x4_t wa[2][kU][kGvGroups], xa[2][kU][kTG];
    auto load = [&](int buf, int step) {
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int64_t off = static_cast<int64_t>(step * kU + u) * 256;
#pragma unroll
        for (int rg = 0; rg < kGvGroups; ++rg) wa[buf][u][rg] = ld16_nt(wp[rg] + off);
#pragma unroll
        for (int tg = 0; tg < kTG; ++tg)
          if (tg < ntg) xa[buf][u][tg] = ldx(tg, off);
      }
    };
    auto mma = [&](int buf) {
#pragma unroll
      for (int u = 0; u < kU; ++u)
#pragma unroll
        for (int tg = 0; tg < kTG; ++tg)
          if (tg < ntg) {
#pragma unroll
            for (int rg = 0; rg < kGvGroups; ++rg)
              acc[rg][tg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, wa[buf][u][rg]),
                                                                    __builtin_bit_cast(bf16x8_t, xa[buf][u][tg]),
                                                                    acc[rg][tg], 0, 0, 0);
          }
    };
    if (nstep > 0) load(0, 0);
    int st = 0;
    for (; st + 2 <= nstep; st += 2) {
      load(1, st + 1);
      mma(0);
      if (st + 2 < nstep) load(0, st + 2);
      mma(1);
    }
    if (st < nstep) mma(0);
    for (int c = nstep * kU; c < nchunk; ++c) {  // odd chunk count: one chunk left
      const int64_t off = static_cast<int64_t>(c) * 256;
      u32x4_t w[kGvGroups];
#pragma unroll
      for (int rg = 0; rg < kGvGroups; ++rg) w[rg] = ld16_nt(wp[rg] + off);
#pragma unroll
      for (int tg = 0; tg < kTG; ++tg)
        if (tg < ntg) {
          const u32x4_t x = ldx(tg, off);
#pragma unroll
          for (int rg = 0; rg < kGvGroups; ++rg)
            acc[rg][tg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, w[rg]),
                                                                  __builtin_bit_cast(bf16x8_t, x), acc[rg][tg], 0, 0, 0);
        }
    }

    // Lane l keeps accumulator l%4 (matching K-slices) and sums it with lanes
    // l^1, l^2: lane 16r + 4t then holds weight row 4rg + r, token 4tg + t.
    const int q = lane & 3;
#pragma unroll
    for (int tg = 0; tg < kTG; ++tg) {
      if (tg >= ntg) break;
#pragma unroll
      for (int rg = 0; rg < kGvGroups; ++rg) {
        float v = q == 0 ? acc[rg][tg][0] : q == 1 ? acc[rg][tg][1] : q == 2 ? acc[rg][tg][2] : acc[rg][tg][3];
        v += __shfl_xor(v, 1);
        v += __shfl_xor(v, 2);
        const int tok = tg * 4 + (i16 >> 2);
        if (q == 0 && tok < ntok) {
          if (kGelu) v = gelu_tanh_fast(v);
          C[static_cast<int64_t>(seg0 + tok0 + tok) * N + n0 + rg * 4 + g] = f32_to_bf16(v);
        }
      }
    }
  }
}

template <bool kGelu, int kTG, bool kGather = false>
hipError_t launch_gemv(const uint16_t* A, const uint16_t* B, uint16_t* C, const int32_t* offsets, int E, int N, int K,
                       int max_rows, hipStream_t stream, const int32_t* gidx = nullptr, int gdiv = 1,
                       int src_rows = 0) {
  if (kGather && (gidx == nullptr || gdiv < 1 || src_rows < 0)) return hipErrorInvalidValue;
  const int active = max_rows < E ? max_rows : E;
  const int64_t blocks = static_cast<int64_t>(active) * ((N + kGvRows - 1) / kGvRows);
  hipLaunchKernelGGL((grouped_gemm_bf16_gemv<kGelu, kTG, kGather>), dim3(static_cast<unsigned>(blocks)),
                     dim3(kGvWaves * kWave), 0, stream, A, B, C, offsets, E, N, K, max_rows, gidx, gdiv, src_rows);
  return hipGetLastError();
}

template <bool kGelu, int kGroups>
hipError_t launch_skinny(const uint16_t* A, const uint16_t* B, uint16_t* C, const int32_t* offsets, int E, int N,
                         int K, int max_rows, hipStream_t stream) {
  // at most min(E, max_rows) experts have rows
  const int active = max_rows < E ? max_rows : E;
  const int64_t blocks = static_cast<int64_t>(active) * ((N + kSkinnyRows - 1) / kSkinnyRows);
  hipLaunchKernelGGL((grouped_gemm_bf16_skinny<kGelu, kGroups>), dim3(static_cast<unsigned>(blocks)), dim3(kWave), 0,
                     stream, A, B, C, offsets, E, N, K, max_rows);
  return hipGetLastError();
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

// The decode kernel runs for this shape: whole 128-element K chunks, 8-row
// weight groups, and few rows per expert.  A pass of it holds 16 rows, so a
// bound above 16 costs an expert that gets more than 16 rows extra passes
// over its weights; up to a bound of 64 it still runs when the batch averages
// at most 16 rows per expert (rows <= 16 E), where most experts need one pass
// and it streams at about 6 TB/s against 3.8 TB/s for the skinny kernel at 64
// tokens and 5.1 at 32 (d = 3584, F = 2560, E = 64, k = 2).  A batch that can
// fill its experts to 64 rows runs the skinny kernel, which reads each weight
// once.
bool gemv_runs(int K, int N, int max_tokens_per_expert, int rows, int E) {
  if (K % 128 != 0 || N % (kGvGroups * 4) != 0) return false;
  return max_tokens_per_expert <= 16 ||
         (max_tokens_per_expert <= kGvMaxTok && static_cast<int64_t>(rows) <= int64_t{16} * E);
}

}  // namespace

hipError_t launch_grouped_gemm(int dtype, bool gelu, const void* A, const void* B, void* C, const int32_t* offsets,
                               int E, int N, int K, int max_rows, int max_tokens_per_expert, hipStream_t stream) {
  if (max_rows <= 0) return hipSuccess;
  if (dtype == kDtypeBF16) {
    const uint16_t* a = static_cast<const uint16_t*>(A);
    const uint16_t* b = static_cast<const uint16_t*>(B);
    uint16_t* c = static_cast<uint16_t*>(C);
    if (gemv_runs(K, N, max_tokens_per_expert, max_rows, E)) {
      if (max_tokens_per_expert <= 4)
        return gelu ? launch_gemv<true, 1>(a, b, c, offsets, E, N, K, max_rows, stream)
                    : launch_gemv<false, 1>(a, b, c, offsets, E, N, K, max_rows, stream);
      if (max_tokens_per_expert <= 8)
        return gelu ? launch_gemv<true, 2>(a, b, c, offsets, E, N, K, max_rows, stream)
                    : launch_gemv<false, 2>(a, b, c, offsets, E, N, K, max_rows, stream);
      return gelu ? launch_gemv<true, 4>(a, b, c, offsets, E, N, K, max_rows, stream)
                  : launch_gemv<false, 4>(a, b, c, offsets, E, N, K, max_rows, stream);
    }
    if (max_tokens_per_expert <= 16)
      return gelu ? launch_skinny<true, 1>(a, b, c, offsets, E, N, K, max_rows, stream)
                  : launch_skinny<false, 1>(a, b, c, offsets, E, N, K, max_rows, stream);
    if (max_tokens_per_expert <= 32)
      return gelu ? launch_skinny<true, 2>(a, b, c, offsets, E, N, K, max_rows, stream)
                  : launch_skinny<false, 2>(a, b, c, offsets, E, N, K, max_rows, stream);
    if (max_tokens_per_expert <= kSkinnyMaxTok)
      return gelu ? launch_skinny<true, 4>(a, b, c, offsets, E, N, K, max_rows, stream)
                  : launch_skinny<false, 4>(a, b, c, offsets, E, N, K, max_rows, stream);
    return gelu ? launch_big<true, false>(a, b, c, offsets, E, N, K, max_rows, nullptr, 1, 0, stream)
                : launch_big<false, false>(a, b, c, offsets, E, N, K, max_rows, nullptr, 1, 0, stream);
  }
  return launch_cfg<float, 64, 64, 2, 2>(gelu, static_cast<const float*>(A), static_cast<const float*>(B),
                                         static_cast<float*>(C), offsets, E, N, K, max_rows, stream);
}

bool grouped_gemm_gathers(int dtype, int K, int N, int max_tokens_per_expert, int src_rows, int rows, int E) {
  return dtype == kDtypeBF16 &&
         (max_tokens_per_expert > kSkinnyMaxTok || gemv_runs(K, N, max_tokens_per_expert, rows, E)) &&
         static_cast<int64_t>(src_rows) * K * 2 < (int64_t{1} << 31);
}

hipError_t launch_grouped_gemm_gather(bool gelu, const void* X, int src_rows, const int32_t* gidx, int gdiv,
                                      const void* B, void* C, const int32_t* offsets, int E, int N, int K,
                                      int max_rows, int max_tokens_per_expert, hipStream_t stream) {
  if (max_rows <= 0) return hipSuccess;
  const uint16_t* a = static_cast<const uint16_t*>(X);
  const uint16_t* b = static_cast<const uint16_t*>(B);
  uint16_t* c = static_cast<uint16_t*>(C);
  if (gemv_runs(K, N, max_tokens_per_expert, max_rows, E)) {
    if (max_tokens_per_expert <= 4)
      return gelu ? launch_gemv<true, 1, true>(a, b, c, offsets, E, N, K, max_rows, stream, gidx, gdiv, src_rows)
                  : launch_gemv<false, 1, true>(a, b, c, offsets, E, N, K, max_rows, stream, gidx, gdiv, src_rows);
    if (max_tokens_per_expert <= 8)
      return gelu ? launch_gemv<true, 2, true>(a, b, c, offsets, E, N, K, max_rows, stream, gidx, gdiv, src_rows)
                  : launch_gemv<false, 2, true>(a, b, c, offsets, E, N, K, max_rows, stream, gidx, gdiv, src_rows);
    return gelu ? launch_gemv<true, 4, true>(a, b, c, offsets, E, N, K, max_rows, stream, gidx, gdiv, src_rows)
                : launch_gemv<false, 4, true>(a, b, c, offsets, E, N, K, max_rows, stream, gidx, gdiv, src_rows);
  }
  if (max_tokens_per_expert <= kSkinnyMaxTok) return hipErrorInvalidValue;  // no gathering kernel for this shape
  return gelu ? launch_big<true, true>(a, b, c, offsets, E, N, K, max_rows, gidx, gdiv, src_rows, stream)
              : launch_big<false, true>(a, b, c, offsets, E, N, K, max_rows, gidx, gdiv, src_rows, stream);
}

}  // namespace moe
