// Dispatcher kernels: per-chunk expert histogram, exclusive scan, stable
// scatter of the (token, slot) pairs into expert-contiguous rows, and the
// capacity cut.
//
// Method: the pairs are regrouped by expert id ("Qwen2-MoE代码解析"
// (jsqmd.com/news/1061813) §3.1 detail 3 sorts them; the "GPT-4 activates 2%"
// article (wmrh.cn/news/106769) §2.2 gathers each expert's token slices).
// With an expert capacity C ("Qwen2-MoE代码解析" §3.4; C = ceil(T/E)*k in
// the Qwen2-MoE walk-through (mlqm.cn/news/48291) §2.2), an expert keeps at
// most C pairs, taken in (slot rank, token index) order; the others are
// dropped.
//
// The order of the rows is (expert, token, slot), so it is a counting sort:
//   row(t, s) = offsets[e] + #kept pairs of e in earlier chunks
//             + #kept pairs of e earlier in the same chunk.
// A chunk is 64 tokens, one per lane; "earlier in the chunk" is a popcount of
// a wave ballot that matches expert ids bit by bit (7 ballots per slot).
// No global atomics, so the result is deterministic.
//
// Kernels (dropless): count -> scatter with the scan folded in (each block
// sums the chunk histograms it needs), or count -> scan -> scatter when the
// histograms are too large for every block to sum.
// Kernels (capacity): count per (slot, expert) -> scan (priority bases and
// offsets) -> keep -> scan of kept counts -> scatter.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "topk.hpp"

namespace moe {
namespace {

constexpr int kNone = kMaxExperts;   // id of an invalid, dropped or absent pair (bit 6 set)
constexpr int kScanThreads = 1024;
constexpr int kScatterTok = 16;      // tokens per scatter block
constexpr int kScatterThreads = 256;

struct Ballots {
  uint64_t b[7];
};

__device__ __forceinline__ Ballots ballots_of(int e) {
  Ballots r;
#pragma unroll
  for (int i = 0; i < 7; ++i) r.b[i] = __ballot((e >> i) & 1);
  return r;
}

// Lanes whose ballot value equals e.
__device__ __forceinline__ uint64_t match(const Ballots& B, int e) {
  uint64_t m = ~0ull;
#pragma unroll
  for (int i = 0; i < 7; ++i) m &= ((e >> i) & 1) ? B.b[i] : ~B.b[i];
  return m;
}

// Copy hidden-state rows tok0 .. tok0+ntok-1 of X to their dispatched rows
// (row_of[t * row_stride + s], -1 = none).  Each thread issues 8 16-byte loads
// before their stores, so the copy is not one memory round trip per chunk;
// a load past the end re-reads the last chunk (its value unused) instead of
// sitting behind a branch, which would make each load wait for the previous.
template <int kThreads, typename T>
__device__ __forceinline__ void copy_rows(const T* __restrict__ X, T* __restrict__ Xp, int d, int k, int tok0,
                                          int ntok, const int* row_of, int row_stride) {
  constexpr int kBatch = 8;
  const int nvec = d * static_cast<int>(sizeof(T)) / 16;
  const int total = ntok * nvec;
  for (int base = threadIdx.x; base < total; base += kThreads * kBatch) {
    u32x4_t val[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int idx = min(base + j * kThreads, total - 1);
      const int tt = idx / nvec;
      const int v = idx % nvec;
      val[j] = ld16_nt(reinterpret_cast<const unsigned char*>(X + static_cast<int64_t>(tok0 + tt) * d) + v * 16);
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int idx = base + j * kThreads;
      if (idx < total) {
        const int tt = idx / nvec;
        const int v = idx % nvec;
        for (int s = 0; s < k; ++s) {
          const int row = row_of[tt * row_stride + s];
          if (row >= 0) st16(reinterpret_cast<unsigned char*>(Xp + static_cast<int64_t>(row) * d) + v * 16, val[j]);
        }
      }
    }
  }
}

__device__ __forceinline__ int load_id(const int32_t* ids, int t, int T, int k, int s, int E) {
  if (t >= T) return kNone;
  const int e = ids[static_cast<int64_t>(t) * k + s];
  return (e >= 0 && e < E) ? e : kNone;
}

// The expert ids of token t's slots s0 .. s0+N-1 (kNone for s >= k, t >= T,
// or an id outside [0, E)), all N loads issued together: through a buffer
// resource over ids an invalid slot takes an offset past the range and reads
// zero, so no load sits behind a branch (a branch per load makes the
// compiler wait for each load before the next).  ids beyond 2^31 bytes use
// plain loads.
template <int N>
__device__ __forceinline__ void load_ids(const int32_t* __restrict__ ids, int t, int T, int k, int E, int s0,
                                         int (&e)[N]) {
  if (static_cast<int64_t>(T) * k * 4 < (int64_t{1} << 31)) {
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<int32_t*>(ids), 0, T * k * 4, 0x00020000);
    int v[N];
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const bool ok = s0 + j < k && t < T;
      v[j] = static_cast<int>(
          __builtin_amdgcn_raw_buffer_load_b32(r, ok ? (t * k + s0 + j) * 4 : static_cast<int>(0x80000000u), 0, 0));
    }
#pragma unroll
    for (int j = 0; j < N; ++j) e[j] = (s0 + j < k && t < T && v[j] >= 0 && v[j] < E) ? v[j] : kNone;
  } else {
#pragma unroll
    for (int j = 0; j < N; ++j) e[j] = s0 + j < k ? load_id(ids, t, T, k, s0 + j, E) : kNone;
  }
}

// The keep flags of token t's slots 0 .. N-1 (0 for s >= k or t >= T), the
// same way.
template <int N>
__device__ __forceinline__ void load_keep(const int8_t* __restrict__ keep, int t, int T, int k, int (&kp)[N]) {
  if (static_cast<int64_t>(T) * k < (int64_t{1} << 31)) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(keep), 0, T * k, 0x00020000);
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const bool ok = j < k && t < T;
      kp[j] = __builtin_amdgcn_raw_buffer_load_b8(r, ok ? t * k + j : static_cast<int>(0x80000000u), 0, 0);
    }
  } else {
#pragma unroll
    for (int j = 0; j < N; ++j) kp[j] = (j < k && t < T) ? keep[static_cast<int64_t>(t) * k + j] : 0;
  }
}

// Histogram of one chunk: cols = E (dropless, col = e) or k*E (capacity,
// col = s*E + e), stored as row blockIdx.x of hist with row stride `stride`.
// Dropless rows may be padded (cols <= stride <= 64; the padding gets
// zeros); capacity rows are not (stride = cols).  One wave, a token per lane;
// for each slot lane e counts the lanes holding expert e from the
// expert-id-bit ballots, so no cell takes atomics (a skewed routing would
// serialise them on its few hot experts).
__global__ __launch_bounds__(kWave) void dispatch_count_kernel(const int32_t* __restrict__ ids, int T, int E, int k,
                                                               bool per_slot, int stride,
                                                               int32_t* __restrict__ hist) {
  const int lane = threadIdx.x;
  const int t = blockIdx.x * kDispatchChunk + lane;
  int32_t* out = hist + static_cast<int64_t>(blockIdx.x) * stride;
  int cnt = 0;
  for (int s0 = 0; s0 < k; s0 += 8) {
    int e[8];
    load_ids(ids, t, T, k, E, s0, e);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (s0 + j < k) {
        const int c = __popcll(match(ballots_of(e[j]), lane));
        if (!per_slot) cnt += c;
        else if (lane < E) out[(s0 + j) * E + lane] = c;
      }
    }
  }
  if (!per_slot && lane < stride) out[lane] = cnt;
}

enum ScanMode { kScanDropless = 0, kScanCapacity1 = 1, kScanCapacity2 = 2, kScanOffsets = 3 };

// One block.  Replaces M[c][col] by its exclusive prefix over chunks c, then
//   dropless:  counts[e] = total, offsets = exclusive scan of totals;
//   capacity1: counts[e] = sum over slots, slot_base[s][e] = pairs of e in
//              slots < s, offsets from min(counts, C);
//   capacity2: nothing more (offsets were written by capacity1);
//   offsets:   offsets = exclusive scan of the column totals (counts kept).
// Then perm rows >= N get -1.
__global__ __launch_bounds__(kScanThreads) void dispatch_scan_kernel(int32_t* __restrict__ M, int nrows, int ncols,
                                                                     int mode, int E, int k, int capacity,
                                                                     int32_t* __restrict__ counts,
                                                                     int32_t* __restrict__ offsets,
                                                                     int32_t* __restrict__ slot_base,
                                                                     int32_t* __restrict__ perm, int total_pairs) {
  __shared__ int s_part[kScanThreads];
  __shared__ int s_tot[kMaxExperts * kMaxExperts];
  __shared__ int s_N;
  const int tid = threadIdx.x;
  for (int col0 = 0; col0 < ncols; col0 += kScanThreads) {
    const int gcols = min(kScanThreads, ncols - col0);
    const int P = kScanThreads / gcols;
    const int ci = tid % gcols;
    const int p = tid / gcols;
    const int L = (nrows + P - 1) / P;
    const int r0 = p * L;
    const int r1 = min(nrows, r0 + L);
    // Up to kScanRegRows rows per thread are loaded once, all together;
    // beyond that rows go in batches of kScanBatch independent loads, so a
    // thread's L rows cost ceil(L / kScanBatch) memory round trips per pass.  The
    // loads go through a buffer resource over M: a row past the thread's
    // range takes an offset beyond the resource and reads zero, so no load
    // sits behind a branch (which would serialise them).  M beyond 2^31
    // bytes (past 8 M tokens at k*E = 4096 columns) uses plain loads.
    constexpr int kScanBatch = 16;
    constexpr int kScanRegRows = 64;  // rows per thread held in registers when they all fit
    const __amdgpu_buffer_rsrc_t mrsrc =
        __builtin_amdgcn_make_buffer_rsrc(M, 0, nrows * ncols * 4, 0x00020000);
    auto scan_col = [&](auto buffered_c) {
      constexpr bool kBuf = decltype(buffered_c)::value;
      auto load_row = [&](int r) {
        if constexpr (!kBuf) {
          return r < r1 ? M[static_cast<int64_t>(r) * ncols + col0 + ci] : 0;
        } else {
          const int off = r < r1 ? (r * ncols + col0 + ci) * 4 : static_cast<int>(0x80000000u);
          return static_cast<int>(__builtin_amdgcn_raw_buffer_load_b32(mrsrc, off, 0, 0));
        }
      };
      // All of the thread's rows in registers (16, 32 or 64 loads, the fewest
      // that cover them; past 32 only the thread's L, which keeps the
      // registers within the kernel's budget): one round of loads serves
      // both passes.
      auto reg_rows = [&](auto n_c) {
        constexpr int kN = decltype(n_c)::value;
        int v[kN];
#pragma unroll
        for (int j = 0; j < kN; ++j) v[j] = kN <= 32 || j < L ? load_row(r0 + j) : 0;  // rows past r1 read zero
        int sum = 0;
#pragma unroll
        for (int j = 0; j < kN; ++j) sum += v[j];
        s_part[tid] = sum;
        __syncthreads();
        if (p < P) {
          int base = 0;
          for (int q = 0; q < p; ++q) base += s_part[q * gcols + ci];
          if (p == P - 1) s_tot[col0 + ci] = base + sum;
#pragma unroll
          for (int j = 0; j < kN; ++j) {
            if (r0 + j < r1) M[static_cast<int64_t>(r0 + j) * ncols + col0 + ci] = base;
            base += v[j];
          }
        }
      };
      if (kBuf && L <= 16) return reg_rows(std::integral_constant<int, 16>{});
      if (kBuf && L <= 32) return reg_rows(std::integral_constant<int, 32>{});
      if (kBuf && L <= kScanRegRows) return reg_rows(std::integral_constant<int, kScanRegRows>{});
      int sum = 0;
      if (p < P)
        for (int rb = r0; rb < r1; rb += kScanBatch) {
          int v[kScanBatch];
#pragma unroll
          for (int j = 0; j < kScanBatch; ++j) v[j] = load_row(rb + j);
#pragma unroll
          for (int j = 0; j < kScanBatch; ++j) sum += v[j];
        }
      s_part[tid] = sum;
      __syncthreads();
      if (p < P) {
        int base = 0;
        for (int q = 0; q < p; ++q) base += s_part[q * gcols + ci];
        if (p == P - 1) s_tot[col0 + ci] = base + sum;
        for (int rb = r0; rb < r1; rb += kScanBatch) {
          int v[kScanBatch];
#pragma unroll
          for (int j = 0; j < kScanBatch; ++j) v[j] = load_row(rb + j);
#pragma unroll
          for (int j = 0; j < kScanBatch; ++j) {
            if (rb + j < r1) M[static_cast<int64_t>(rb + j) * ncols + col0 + ci] = base;
            base += v[j];
          }
        }
      }
    };
    if (static_cast<int64_t>(nrows) * ncols * 4 < (int64_t{1} << 31)) scan_col(std::true_type{});
    else scan_col(std::false_type{});
    __syncthreads();
  }
  if (tid < kWave) {
    // Lane e: expert e's total (and, capacity1, its slot bases), then the
    // offsets as an exclusive scan over the lanes.
    const int e = tid;
    int add = 0;  // what expert e adds to the offsets
    if (e < E) {
      if (mode == kScanDropless) {
        counts[e] = s_tot[e];
        add = s_tot[e];
      } else if (mode == kScanCapacity1) {
        int n = 0;
        for (int s = 0; s < k; ++s) {
          slot_base[s * E + e] = n;
          n += s_tot[s * E + e];
        }
        counts[e] = n;
        add = min(n, capacity);
      } else if (mode == kScanOffsets) {
        add = s_tot[e];
      }
    }
    if (mode != kScanCapacity2) {
      int incl = add;
#pragma unroll
      for (int m = 1; m < kWave; m <<= 1) {
        const int o = __shfl_up(incl, m);
        if (e >= m) incl += o;
      }
      if (e < E) offsets[e] = incl - add;
      const int total = __shfl(incl, kWave - 1);
      if (e == 0) {
        offsets[E] = total;
        s_N = total;
      }
    } else if (e == 0) {
      s_N = offsets[E];
    }
  }
  __syncthreads();
  if (mode != kScanCapacity1)
    for (int r = s_N + tid; r < total_pairs; r += kScanThreads) perm[r] = -1;
}

// Capacity: decide which pairs are kept and count them per chunk and expert.
// Priority of pair (t, s) with expert e = pairs of e in slots < s (all tokens)
// + pairs of e in slot s of earlier chunks + earlier tokens of this chunk in
// slot s with expert e.  Kept iff priority < C.
__global__ __launch_bounds__(kWave) void dispatch_keep_kernel(const int32_t* __restrict__ ids, int T, int E, int k,
                                                              int capacity, const int32_t* __restrict__ chunk_base,
                                                              const int32_t* __restrict__ slot_base,
                                                              int8_t* __restrict__ keep,
                                                              int32_t* __restrict__ chunk_kept) {
  __shared__ int s_kept[kMaxExperts];
  const int lane = threadIdx.x;
  if (lane < E) s_kept[lane] = 0;
  __syncthreads();
  const int t = blockIdx.x * kDispatchChunk + lane;
  const uint64_t below = (1ull << lane) - 1ull;
  const int32_t* cb = chunk_base + static_cast<int64_t>(blockIdx.x) * k * E;
  for (int s0 = 0; s0 < k; s0 += 8) {
    int ev[8];
    load_ids(ids, t, T, k, E, s0, ev);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int s = s0 + j;
      if (s >= k) break;
      const int e = ev[j];
      const Ballots B = ballots_of(e);
      bool kept = false;
      if (e != kNone) {
        const int prio = slot_base[s * E + e] + cb[s * E + e] + __popcll(match(B, e) & below);
        kept = prio < capacity;
        if (kept) atomicAdd(&s_kept[e], 1);
      }
      if (t < T) keep[static_cast<int64_t>(t) * k + s] = kept ? 1 : 0;
    }
  }
  __syncthreads();
  if (lane < E) chunk_kept[static_cast<int64_t>(blockIdx.x) * E + lane] = s_kept[lane];
}

// Rerouting of the pairs the capacity cut drops ("Qwen2-MoE代码解析" §3.4:
// with drop_tokens = False a token over an expert's capacity goes to a
// next-best expert instead of being discarded).  The cut made by
// dispatch_keep_kernel stands.  The pairs it drops are taken in the same
// (slot rank, token index) priority; each takes the first expert past its
// token's top-k, in the token's preference order, that still has room and
// that the token does not already use (an earlier slot may have moved
// there); a pair that finds none stays dropped.  Its weight is unchanged.
//
// Three steps.  (1) Per 64-token chunk, the dropped pairs of each slot are
// counted; (2) a scan over the chunks gives each its place in one list in
// priority order (slot-major segments); (3) per chunk, each dropped pair is
// written to the list with a copy of its token's preference order and the
// list index of the token's next dropped slot.  Then (4) one workgroup of
// 1024 threads places the list, 1024 pairs at a time within one slot's
// segment: every thread picks its pair's first candidate that is neither
// full (as the room stood at the start of the round) nor used by its token.
// That pick is the sequential rule's iff fewer earlier pairs of the round
// picked the same expert than it had room: the candidates before it were
// full at the start and room only shrinks.  The pairs before the first one
// that fails commit, and the round restarts there.  The first pair of a round
// never fails, and the failing pair's expert is full after the commit, so
// the rounds number at most ceil(segment / 1024) per slot plus E in all.  A
// pair passes the experts it used on to its token's next dropped slot.
constexpr int kRerouteThreads = 1024;

// (1) Dropped pairs per (chunk, slot); the assignment starts as a copy of ids.
__global__ __launch_bounds__(kWave) void dispatch_drop_count_kernel(const int32_t* __restrict__ ids,
                                                                    const int8_t* __restrict__ keep, int T, int E,
                                                                    int k, int32_t* __restrict__ drop_hist,
                                                                    int32_t* __restrict__ ids2) {
  const int lane = threadIdx.x;
  const int t = blockIdx.x * kDispatchChunk + lane;
  for (int s = 0; s < k; ++s) {
    bool dropped = false;
    if (t < T) {
      const int64_t pr = static_cast<int64_t>(t) * k + s;
      const int e = ids[pr];
      ids2[pr] = e;
      dropped = keep[pr] == 0 && e >= 0 && e < E;
    }
    const uint64_t b = __ballot(dropped);
    if (lane == 0) drop_hist[static_cast<int64_t>(blockIdx.x) * k + s] = __popcll(b);
  }
}

// (3) The list: entry i holds the pair id, the token's preference order
// (rstride = 32 or 64 bytes, padded with a copy of position 0), the list index of the token's next dropped slot (-1: none) and
// the experts the token uses: its top-k here, plus, while placing, where
// its earlier slots moved.
__global__ __launch_bounds__(kWave) void dispatch_drop_list_kernel(
    const int32_t* __restrict__ ids, const int8_t* __restrict__ keep, const uint8_t* __restrict__ order, int T,
    int E, int k, int rstride, const int32_t* __restrict__ drop_hist, const int32_t* __restrict__ drop_seg,
    int32_t* __restrict__ list, uint8_t* __restrict__ rows, int32_t* __restrict__ next,
    uint64_t* __restrict__ used) {
  const int lane = threadIdx.x;
  const int t = blockIdx.x * kDispatchChunk + lane;
  const uint64_t below = (1ull << lane) - 1ull;
  int prev = -1;  // list index of this token's previous dropped slot
  for (int s = 0; s < k; ++s) {
    bool dropped = false;
    if (t < T) {
      const int64_t pr = static_cast<int64_t>(t) * k + s;
      const int e = ids[pr];
      dropped = keep[pr] == 0 && e >= 0 && e < E;
    }
    const uint64_t b = __ballot(dropped);
    if (dropped) {
      const int pos = drop_seg[s] + drop_hist[static_cast<int64_t>(blockIdx.x) * k + s] + __popcll(b & below);
      list[pos] = t * k + s;
      const uint8_t* src = order + static_cast<int64_t>(t) * E;
      uint8_t* dst = rows + static_cast<int64_t>(pos) * rstride;
      for (int q = 0; q < rstride; ++q) dst[q] = src[q < E ? q : 0];
      // The token's top-k experts count as used, so a scan of the whole row
      // skips positions below k (and the padding, a copy of position 0).
      uint64_t topk = 0ull;
      for (int j = 0; j < k; ++j) {
        const int e = ids[static_cast<int64_t>(t) * k + j];
        if (e >= 0 && e < E) topk |= 1ull << e;
      }
      for (int q = 0; q < k; ++q) topk |= 1ull << (src[q] & 63);
      next[pos] = -1;
      used[pos] = topk;
      if (prev >= 0) next[prev] = pos;
      prev = pos;
    }
  }
}

// (4) Placement, one workgroup.  NQ = 32 or 64: the row length (E <= NQ).
template <int NQ>
__global__ __launch_bounds__(kRerouteThreads) void dispatch_reroute_kernel(
    const int32_t* __restrict__ counts, const int32_t* __restrict__ drop_seg, const int32_t* __restrict__ list,
    const uint8_t* __restrict__ rows, const int32_t* __restrict__ next, uint64_t* __restrict__ used, int E, int k,
    int capacity, int8_t* __restrict__ keep, int32_t* __restrict__ ids2) {
  __shared__ int s_room[kMaxExperts];
  __shared__ int s_cnt[kRerouteThreads / kWave][kMaxExperts];
  __shared__ int s_first;
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = tid / kWave;
  const uint64_t below = (1ull << lane) - 1ull;
  if (tid < kMaxExperts) s_room[tid] = tid < E ? capacity - min(max(counts[tid], 0), capacity) : 0;
  int s = 0;
  int seg_end = drop_seg[1];
  const int m = drop_seg[k];
  int c0 = 0;
  while (c0 < m && c0 >= seg_end) seg_end = drop_seg[++s + 1];  // rounds stay inside one slot's segment
  // The round's entries: pair id, the list index of its token's next
  // dropped slot, the experts its token uses (its top-k and where its
  // earlier slots moved, written in an earlier segment: read past the L1),
  // and the preference order as words.  The entries of the round after are
  // fetched while this one runs (into the second set) when that round stays
  // in the segment; they are used if this round commits all its entries.
  struct Entry {
    int pair, nx;
    uint64_t mine;
    u32x4_t wv[NQ / 16];
  };
  Entry cur{}, pre{};
  auto load = [&](Entry& en, int base) {
    const int i = base + tid;
    if (i < seg_end) {
      en.pair = list[i];
      en.nx = next[i];
      en.mine = __hip_atomic_load(&used[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const u32x4_t* row = reinterpret_cast<const u32x4_t*>(rows + static_cast<int64_t>(i) * NQ);
#pragma unroll
      for (int w = 0; w < NQ / 16; ++w) en.wv[w] = row[w];
    }
  };
  if (c0 < m) load(cur, c0);
  __syncthreads();
  while (c0 < m) {
    const int i = c0 + tid;
    const bool valid = i < seg_end;
    const bool ahead = c0 + kRerouteThreads < seg_end;  // the next round, if this one commits all, is in the segment
    if (ahead) load(pre, c0 + kRerouteThreads);
    // Full experts (and ids past E) as they stand at the start of the round.
    const uint64_t full = __ballot(lane >= E || s_room[lane] <= 0);
    int pick = kNone;
    if (valid) {
      // Last to first, so the earliest available position wins; the top-k
      // (and the padding, a copy of position 0) are in `mine`.  A byte of
      // the order that names no expert (>= E: a caller's malformed order) is
      // never available, so every pick indexes the per-expert tables in range.
      const uint64_t avail = ~(full | cur.mine);
      const uint32_t lo = static_cast<uint32_t>(avail), hi = static_cast<uint32_t>(avail >> 32);
#pragma unroll
      for (int q = NQ - 1; q >= 0; --q) {
        const uint32_t e = __builtin_amdgcn_ubfe(cur.wv[q >> 4][(q >> 2) & 3], (q & 3) * 8, 8);
        const uint32_t bit = NQ == 32 ? __builtin_amdgcn_ubfe(lo, e & 31, 1)
                                      : __builtin_amdgcn_ubfe(e < 32 ? lo : hi, e & 31, 1);
        const bool ok = bit != 0 && e < static_cast<uint32_t>(E);
        pick = ok ? static_cast<int>(e) : pick;
      }
    }
    // Rank of each pick among the round's earlier picks of the same expert.
    const Ballots B = ballots_of(pick);
    const int rank_w = pick != kNone ? __popcll(match(B, pick) & below) : 0;
    if (lane < E) s_cnt[wave][lane] = __popcll(match(B, lane));
    if (tid == 0) s_first = min(seg_end, c0 + kRerouteThreads);  // the round's end if nothing fails
    __syncthreads();
    if (pick != kNone) {
      int rank = rank_w;
#pragma unroll
      for (int w = 0; w < kRerouteThreads / kWave; ++w) {
        const int c = s_cnt[w][pick];
        rank += w < wave ? c : 0;
      }
      if (rank >= s_room[pick]) atomicMin(&s_first, i);
    }
    __syncthreads();
    const int f = s_first;  // > c0: the round's first pair never fails
    const bool commit = valid && i < f;
    if (commit) {
      if (pick != kNone) {
        ids2[cur.pair] = pick;
        keep[cur.pair] = 1;
      }
      if (cur.nx >= 0) used[cur.nx] = cur.mine | (pick != kNone ? 1ull << pick : 0ull);
    }
    const uint64_t live = __ballot(commit);
    if (lane < E) {
      const int dec = __popcll(match(B, lane) & live);
      if (dec > 0) atomicSub(&s_room[lane], dec);
    }
    const bool all = f == c0 + kRerouteThreads;
    c0 = f;
    const bool new_seg = c0 >= seg_end;
    if (!new_seg) {
      if (all && ahead) cur = pre;  // fetched during this round
      else load(cur, c0);           // a conflict moved the start: fetch across the barrier
    } else {
      __threadfence();  // a new segment reads used[] written in this one
    }
    __syncthreads();
    if (new_seg && c0 < m) {
      while (c0 >= seg_end) seg_end = drop_seg[++s + 1];
      load(cur, c0);
    }
  }
}

// Kept pairs per 64-token chunk and expert, under the rerouted assignment.
__global__ __launch_bounds__(kWave) void dispatch_count_kept_kernel(const int32_t* __restrict__ ids,
                                                                    const int8_t* __restrict__ keep, int T, int E,
                                                                    int k, int32_t* __restrict__ chunk_kept) {
  __shared__ int s_hist[kMaxExperts];
  const int lane = threadIdx.x;
  s_hist[lane] = 0;
  __syncthreads();
  const int t = blockIdx.x * kDispatchChunk + lane;
  if (t < T)
    for (int s = 0; s < k; ++s) {
      const int64_t pr = static_cast<int64_t>(t) * k + s;
      const int e = ids[pr];
      if (keep[pr] != 0 && e >= 0 && e < E) atomicAdd(&s_hist[e], 1);
    }
  __syncthreads();
  if (lane < E) chunk_kept[static_cast<int64_t>(blockIdx.x) * E + lane] = s_hist[lane];
}

// Rows of the pairs of 16 tokens, then the copy of their hidden states.
// Wave 0 ranks all 64 tokens of the enclosing chunk and keeps its 16.
template <typename T, int KMAX, bool kCap>
__global__ __launch_bounds__(kScatterThreads) void dispatch_scatter_kernel(
    const int32_t* __restrict__ ids, const T* __restrict__ X, int T_tok, int d, int E, int k,
    const int32_t* __restrict__ chunk_base, const int32_t* __restrict__ offsets, const int8_t* __restrict__ keep,
    int32_t* __restrict__ perm, int32_t* __restrict__ inv_perm, T* __restrict__ Xp) {
  __shared__ int s_row[kScatterTok][KMAX];
  const int tok0 = blockIdx.x * kScatterTok;
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    const int chunk = tok0 / kDispatchChunk;
    const int t = chunk * kDispatchChunk + lane;
    const uint64_t below = (1ull << lane) - 1ull;
    int e[KMAX];
    int cnt[KMAX];
    load_ids(ids, t, T_tok, k, E, 0, e);
    if constexpr (kCap) {
      int kp[KMAX];
      load_keep(keep, t, T_tok, k, kp);
#pragma unroll
      for (int s = 0; s < KMAX; ++s)
        if (!kp[s]) e[s] = kNone;
    }
#pragma unroll
    for (int s = 0; s < KMAX; ++s) cnt[s] = 0;
#pragma unroll
    for (int s2 = 0; s2 < KMAX; ++s2) {
      if (s2 < k) {
        const Ballots B = ballots_of(e[s2]);
#pragma unroll
        for (int s = 0; s < KMAX; ++s)
          if (s < k) cnt[s] += __popcll(match(B, e[s]) & below);
      }
    }
    const bool mine = t >= tok0 && t < tok0 + kScatterTok;
#pragma unroll
    for (int s = 0; s < KMAX; ++s) {
      if (s < k && mine) {
        int row = -1;
        if (e[s] != kNone) {
          int same = 0;  // same expert in an earlier slot of this token (only for repeated ids)
#pragma unroll
          for (int s2 = 0; s2 < KMAX; ++s2)
            if (s2 < s && e[s2] == e[s]) ++same;
          row = offsets[e[s]] + chunk_base[static_cast<int64_t>(chunk) * E + e[s]] + cnt[s] + same;
          if (row < 0 || row >= T_tok * k) row = -1;  // unreachable for consistent scratch; keeps stores in bounds
          if (t < T_tok && row >= 0) perm[row] = t * k + s;
        }
        if (t < T_tok) inv_perm[static_cast<int64_t>(t) * k + s] = row;
        s_row[t - tok0][s] = (t < T_tok) ? row : -1;
      }
    }
  }
  if (Xp == nullptr) return;  // indices only: the expert GEMM gathers the rows itself
  __syncthreads();
  copy_rows<kScatterThreads>(X, Xp, d, k, tok0, min(kScatterTok, T_tok - tok0), &s_row[0][0], KMAX);
}

// Dropless rows with the scan folded into the scatter, so the dispatch is
// two launches (count, then this).  Every block sums the count kernel's
// per-chunk histograms H[c][e] (row stride Ep = E rounded up to 4, padded
// with zeros) for itself: tot[e] over all chunks and pre[e] over the chunks
// before its own; offsets = exclusive scan of tot, and its pairs' rows
// follow as in dispatch_scatter_kernel with offsets[e] + pre[e] as the
// chunk's base.  The sums are integer, so every block holds the bits one
// scan would give.  A block covers ntb = 64 tokens (one chunk) when it only
// writes indices, or 16 (a quarter chunk, four blocks summing the same
// histograms) when it also copies rows, for more blocks on the copy.  The
// reads cost nblocks * nchunks * Ep * 4 bytes of L2, so the launcher takes
// this path only while nchunks * Ep <= kScanScatterMaxCells.  Block 0 writes
// counts and offsets; all blocks share the -1 tail of perm.
constexpr int kScanScatterMaxCells = 16384;  // 64 KB of histograms per block
constexpr int kScanScatterBatch = 16;        // 16-byte loads in flight per thread

template <typename T, int KMAX>
__global__ __launch_bounds__(kScatterThreads) void dispatch_scan_scatter_kernel(
    const int32_t* __restrict__ ids, const T* __restrict__ X, int T_tok, int d, int E, int k, int ntb,
    const int32_t* __restrict__ H, int Ep, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ perm, int32_t* __restrict__ inv_perm, T* __restrict__ Xp) {
  __shared__ u32x4_t s_tot[kScatterThreads];
  __shared__ u32x4_t s_pre[kScatterThreads];
  __shared__ int s_base[kMaxExperts];
  __shared__ int s_N;
  __shared__ int s_row[kDispatchChunk][KMAX];
  const int tid = threadIdx.x;
  const int tok0 = blockIdx.x * ntb;
  const int chunk = tok0 / kDispatchChunk;
  const int nchunks = (T_tok + kDispatchChunk - 1) / kDispatchChunk;
  const int total_pairs = T_tok * k;
  // Thread (cg, g) sums columns 4cg .. 4cg+3 over rows g, g + G, ...
  const int ncg = Ep / 4;
  const int G = kScatterThreads / ncg;
  const int cg = tid % ncg;
  const int g = tid / ncg;
  // Wave 0's id loads go out first, to overlap the histogram reads.
  const int lane = tid % kWave;
  const int t = chunk * kDispatchChunk + lane;
  int e[KMAX];
  if (tid < kWave) load_ids(ids, t, T_tok, k, E, 0, e);
  u32x4_t tot = {0u, 0u, 0u, 0u};
  u32x4_t pre = {0u, 0u, 0u, 0u};
  if (g < G) {
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<int32_t*>(H), 0, nchunks * Ep * 4, 0x00020000);
    for (int r0 = g; r0 < nchunks; r0 += G * kScanScatterBatch) {
      u32x4_t v[kScanScatterBatch];
#pragma unroll
      for (int q = 0; q < kScanScatterBatch; ++q) {
        const int row = r0 + q * G;
        const int off = row < nchunks ? (row * Ep + cg * 4) * 4 : static_cast<int>(0x80000000u);
        v[q] = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
      }
#pragma unroll
      for (int q = 0; q < kScanScatterBatch; ++q) {
        tot += v[q];
        if (r0 + q * G < chunk) pre += v[q];
      }
    }
  }
  s_tot[tid] = tot;
  s_pre[tid] = pre;
  __syncthreads();
  if (tid < kWave) {
    // Lane e: expert e's total and prefix, then the exclusive scan over e.
    int te = 0;
    int pe = 0;
    if (lane < E) {
      const int* st = reinterpret_cast<const int*>(s_tot);
      const int* sp = reinterpret_cast<const int*>(s_pre);
      for (int q = 0; q < G; ++q) {
        te += st[q * Ep + lane];
        pe += sp[q * Ep + lane];
      }
    }
    int incl = te;
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) {
      const int o = __shfl_up(incl, m);
      if (lane >= m) incl += o;
    }
    const int excl = incl - te;
    const int N = __shfl(incl, kWave - 1);
    if (lane < E) s_base[lane] = excl + pe;
    if (lane == 0) s_N = N;
    if (blockIdx.x == 0) {
      if (lane < E) {
        counts[lane] = te;
        offsets[lane] = excl;
      }
      if (lane == 0) offsets[E] = N;
    }
  }
  __syncthreads();
  if (tid < kWave) {
    // Ranks within the chunk, as in dispatch_scatter_kernel.
    const uint64_t below = (1ull << lane) - 1ull;
    int cnt[KMAX];
#pragma unroll
    for (int s = 0; s < KMAX; ++s) cnt[s] = 0;
#pragma unroll
    for (int s2 = 0; s2 < KMAX; ++s2) {
      if (s2 < k) {
        const Ballots B = ballots_of(e[s2]);
#pragma unroll
        for (int s = 0; s < KMAX; ++s)
          if (s < k) cnt[s] += __popcll(match(B, e[s]) & below);
      }
    }
    const bool mine = t >= tok0 && t < tok0 + ntb;
#pragma unroll
    for (int s = 0; s < KMAX; ++s) {
      if (s < k && mine) {
        int row = -1;
        if (e[s] != kNone) {
          int same = 0;
#pragma unroll
          for (int s2 = 0; s2 < KMAX; ++s2)
            if (s2 < s && e[s2] == e[s]) ++same;
          row = s_base[e[s]] + cnt[s] + same;
          if (row < 0 || row >= total_pairs) row = -1;  // unreachable for consistent histograms; keeps stores in bounds
          if (t < T_tok && row >= 0) perm[row] = t * k + s;
        }
        if (t < T_tok) inv_perm[static_cast<int64_t>(t) * k + s] = row;
        s_row[t - tok0][s] = (t < T_tok) ? row : -1;
      }
    }
  }
  for (int q = s_N + blockIdx.x * kScatterThreads + tid; q < total_pairs; q += gridDim.x * kScatterThreads)
    perm[q] = -1;
  if (Xp == nullptr) return;
  __syncthreads();
  copy_rows<kScatterThreads>(X, Xp, d, k, tok0, min(ntb, T_tok - tok0), &s_row[0][0], KMAX);
}

// Small T (<= 256 tokens, k <= 8): the whole dispatch in one block of 4
// waves, one 64-token chunk per wave -- histogram, scans, capacity cut,
// ranks, perm/inv_perm and the row copy -- so decode pays one launch.
constexpr int kSmallMaxT = 4 * kDispatchChunk;
constexpr int kSmallMaxK = 8;

// Run by a whole block of kThreads (>= 256) threads: the index work uses the
// first 4 waves (one 64-token chunk each; the other waves hold no tokens), the
// row copy uses every thread.  Xp == nullptr skips the copy.
template <int kThreads, typename T, bool kCap>
__device__ __forceinline__ void dispatch_small_block(const int32_t* __restrict__ ids, const T* __restrict__ X,
                                                     int T_tok, int d, int E, int k, int capacity,
                                                     int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                     int32_t* __restrict__ perm, int32_t* __restrict__ inv_perm,
                                                     T* __restrict__ Xp) {
  // per chunk, per (slot, expert): pairs, then exclusive prefix over chunks
  __shared__ int s_cnt[4][kSmallMaxK * kMaxExperts];
  __shared__ int s_slot_base[kSmallMaxK * kMaxExperts];  // capacity: pairs of e in slots < s
  __shared__ int s_kept[4][kMaxExperts];                 // kept pairs per chunk/expert, then prefix
  __shared__ int s_off[kMaxExperts + 1];
  __shared__ int s_row[kSmallMaxT][kSmallMaxK];
  const int lane = threadIdx.x % kWave;
  const int chunk = threadIdx.x / kWave;   // waves 4.. hold no tokens (t >= 256 >= T_tok)
  const int t = chunk * kDispatchChunk + lane;
  const uint64_t below = (1ull << lane) - 1ull;
  const int cols = k * E;

  for (int i = threadIdx.x; i < 4 * kSmallMaxK * kMaxExperts; i += kThreads) (&s_cnt[0][0])[i] = 0;
  for (int i = threadIdx.x; i < 4 * kMaxExperts; i += kThreads) (&s_kept[0][0])[i] = 0;
  __syncthreads();
  int e[kSmallMaxK];
  load_ids(ids, t, T_tok, k, E, 0, e);
#pragma unroll
  for (int s = 0; s < kSmallMaxK; ++s)
    if (e[s] != kNone) atomicAdd(&s_cnt[chunk][s * E + e[s]], 1);
  __syncthreads();
  // exclusive prefix over the 4 chunks per column; column totals
  for (int c = threadIdx.x; c < cols; c += kThreads) {
    int acc = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int v = s_cnt[q][c];
      s_cnt[q][c] = acc;
      acc += v;
    }
    s_slot_base[c] = acc;  // column total for now
  }
  __syncthreads();
  if (threadIdx.x < kWave) {
    // per expert: routed count, slot bases (capacity), kept count, offsets (one wave scan)
    const int ex = lane;
    int n = 0, kept = 0;
    if (ex < E) {
      for (int s = 0; s < k; ++s) {
        const int tot = s_slot_base[s * E + ex];
        s_slot_base[s * E + ex] = n;
        n += tot;
      }
      counts[ex] = n;
      kept = kCap ? min(n, capacity) : n;
    }
    int incl = kept;
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) {
      const int o = __shfl_up(incl, m);
      if (lane >= m) incl += o;
    }
    if (ex < E) s_off[ex] = incl - kept;
    if (ex == E - 1) s_off[E] = incl;
  }
  __syncthreads();
  if (kCap) {
    // keep flags by (slot, token) priority; dropped pairs become kNone
#pragma unroll
    for (int s = 0; s < kSmallMaxK; ++s) {
      if (s < k) {
        const Ballots B = ballots_of(e[s]);
        if (e[s] != kNone) {
          const int prio = s_slot_base[s * E + e[s]] + s_cnt[chunk][s * E + e[s]] + __popcll(match(B, e[s]) & below);
          if (prio < capacity) atomicAdd(&s_kept[chunk][e[s]], 1);
          else e[s] = kNone;
        }
      }
    }
    __syncthreads();
    if (threadIdx.x < E) {
      int acc = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int v = s_kept[q][threadIdx.x];
        s_kept[q][threadIdx.x] = acc;
        acc += v;
      }
    }
  } else {
    // dropless: the chunk base of expert e is the prefix of all slots' counts
    __syncthreads();
    if (threadIdx.x < E) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        int acc = 0;
        for (int s = 0; s < k; ++s) acc += s_cnt[q][s * E + threadIdx.x];
        s_kept[q][threadIdx.x] = acc;
      }
    }
  }
  __syncthreads();
  // ranks within the chunk, in (token, slot) order per expert
  int cnt[kSmallMaxK];
#pragma unroll
  for (int s = 0; s < kSmallMaxK; ++s) cnt[s] = 0;
#pragma unroll
  for (int s2 = 0; s2 < kSmallMaxK; ++s2) {
    if (s2 < k) {
      const Ballots B = ballots_of(e[s2]);
#pragma unroll
      for (int s = 0; s < kSmallMaxK; ++s)
        if (s < k) cnt[s] += __popcll(match(B, e[s]) & below);
    }
  }
  const int Tk = T_tok * k;
#pragma unroll
  for (int s = 0; s < kSmallMaxK; ++s) {
    if (s < k && t < T_tok) {
      int row = -1;
      if (e[s] != kNone) {
        int same = 0;
#pragma unroll
        for (int s2 = 0; s2 < kSmallMaxK; ++s2)
          if (s2 < s && e[s2] == e[s]) ++same;
        row = s_off[e[s]] + s_kept[chunk][e[s]] + cnt[s] + same;
        if (row < 0 || row >= Tk) row = -1;  // unreachable for consistent counts; keeps stores in bounds
        if (row >= 0) perm[row] = t * k + s;
      }
      inv_perm[t * k + s] = row;
      s_row[t][s] = row;
    }
  }
  if (threadIdx.x <= E) offsets[threadIdx.x] = s_off[threadIdx.x];
  for (int r = s_off[E] + threadIdx.x; r < Tk; r += kThreads) perm[r] = -1;
  __syncthreads();
  if (Xp != nullptr) copy_rows<kThreads>(X, Xp, d, k, 0, T_tok, &s_row[0][0], kSmallMaxK);
}

// At most 64 tokens: the whole dispatch in one wave with no block barrier,
// token t on lane t (its ids in e[], kNone for slots >= k, tokens >= T and
// ids outside [0, E)).  Lane ex also stands for expert ex: per-expert counts
// come from expert-id-bit ballots, the offsets from one wave scan, and a
// pair's expert-indexed values (slot base, offset) from a lane shuffle.  The
// results are those of dispatch_small_block: capacity by (slot, token)
// priority, rows stable by (expert, token, slot).  row_of (LDS, [64][k_stride])
// receives each pair's row for the row copy.  Called by one whole wave.
template <bool kCap>
__device__ __forceinline__ void dispatch_one_wave(int (&e)[kSmallMaxK], int T_tok, int E, int k, int capacity,
                                                  int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                  int32_t* __restrict__ perm, int32_t* __restrict__ inv_perm,
                                                  int* row_of, int k_stride) {
  const int lane = threadIdx.x % kWave;
  const uint64_t below = (1ull << lane) - 1ull;
  // routed pairs of expert `lane`, and (capacity) its pairs in slots < s
  int routed = 0;
  int slot_base[kSmallMaxK];
#pragma unroll
  for (int s = 0; s < kSmallMaxK; ++s) {
    slot_base[s] = routed;
    if (s < k) routed += __popcll(match(ballots_of(e[s]), lane));
  }
  int kept = routed;
  if (kCap) {
    // a pair is kept if fewer than C pairs of its expert come before it in
    // (slot, token) order; dropped pairs become kNone
#pragma unroll
    for (int s = 0; s < kSmallMaxK; ++s) {
      if (s < k) {
        const Ballots B = ballots_of(e[s]);
        const int base = __shfl(slot_base[s], e[s] & (kWave - 1));
        if (e[s] != kNone && base + __popcll(match(B, e[s]) & below) >= capacity) e[s] = kNone;
      }
    }
    kept = 0;
#pragma unroll
    for (int s = 0; s < kSmallMaxK; ++s)
      if (s < k) kept += __popcll(match(ballots_of(e[s]), lane));
  }
  if (lane >= E) routed = kept = 0;  // no id names expert >= E
  int incl = kept;
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) {
    const int o = __shfl_up(incl, m);
    if (lane >= m) incl += o;
  }
  const int off = incl - kept;
  const int total = __shfl(incl, kWave - 1);
  if (lane < E) {
    counts[lane] = routed;
    offsets[lane] = off;
  }
  if (lane == 0) offsets[E] = total;
  // rank of each pair among its expert's kept pairs of earlier tokens (any
  // slot) and earlier slots of its own token
  int cnt[kSmallMaxK];
#pragma unroll
  for (int s = 0; s < kSmallMaxK; ++s) cnt[s] = 0;
#pragma unroll
  for (int s2 = 0; s2 < kSmallMaxK; ++s2) {
    if (s2 < k) {
      const Ballots B = ballots_of(e[s2]);
#pragma unroll
      for (int s = 0; s < kSmallMaxK; ++s)
        if (s < k) cnt[s] += __popcll(match(B, e[s]) & below);
    }
  }
  const int Tk = T_tok * k;
#pragma unroll
  for (int s = 0; s < kSmallMaxK; ++s) {
    if (s < k) {
      const int base = __shfl(off, e[s] & (kWave - 1));
      if (lane < T_tok) {
        int row = -1;
        if (e[s] != kNone) {
          int same = 0;
#pragma unroll
          for (int s2 = 0; s2 < kSmallMaxK; ++s2)
            if (s2 < s && e[s2] == e[s]) ++same;
          row = base + cnt[s] + same;
          if (row < 0 || row >= Tk) row = -1;  // unreachable for consistent counts; keeps stores in bounds
          if (row >= 0) perm[row] = lane * k + s;
        }
        inv_perm[lane * k + s] = row;
        if (row_of != nullptr) row_of[lane * k_stride + s] = row;
      }
    }
  }
  for (int r = total + lane; r < Tk; r += kWave) perm[r] = -1;
}

template <typename T, bool kCap>
__global__ __launch_bounds__(256) void dispatch_small_kernel(const int32_t* __restrict__ ids, const T* __restrict__ X,
                                                             int T_tok, int d, int E, int k, int capacity,
                                                             int32_t* __restrict__ counts,
                                                             int32_t* __restrict__ offsets,
                                                             int32_t* __restrict__ perm,
                                                             int32_t* __restrict__ inv_perm, T* __restrict__ Xp) {
  if (T_tok <= kWave) {
    __shared__ int s_row1[kWave][kSmallMaxK];
    if (threadIdx.x < kWave) {
      int e[kSmallMaxK];
      load_ids(ids, threadIdx.x, T_tok, k, E, 0, e);
      dispatch_one_wave<kCap>(e, T_tok, E, k, capacity, counts, offsets, perm, inv_perm, &s_row1[0][0], kSmallMaxK);
    }
    if (Xp == nullptr) return;
    __syncthreads();
    copy_rows<256>(X, Xp, d, k, 0, T_tok, &s_row1[0][0], kSmallMaxK);
    return;
  }
  dispatch_small_block<256, T, kCap>(ids, X, T_tok, d, E, k, capacity, counts, offsets, perm, inv_perm, Xp);
}

// Top-k of a K-split router plus the whole dispatch, in one block of 1024
// threads: 16 tokens at a time, every thread sums one (token, expert) entry
// of the partial logits in split order and wave 0 selects; then the
// dispatch of all T tokens (the ids just written are visible to the block
// after the barrier).
template <typename T, bool kCap, int NT>
__global__ __launch_bounds__(1024) void topk_dispatch_small_kernel(const float* __restrict__ partial, int nsplit,
                                                                   const float* __restrict__ bias,
                                                                   int32_t* __restrict__ ids, float* __restrict__ w,
                                                                   const T* __restrict__ X, int T_tok, int d, int E,
                                                                   int k, int capacity, int32_t* __restrict__ counts,
                                                                   int32_t* __restrict__ offsets,
                                                                   int32_t* __restrict__ perm,
                                                                   int32_t* __restrict__ inv_perm,
                                                                   T* __restrict__ Xp) {
  __shared__ float logit[16][kMaxExperts];
  __shared__ float sel_val[16 * kMaxExperts];
  __shared__ int sel_id[16 * kMaxExperts];
  __shared__ int s_ids[kWave][kSmallMaxK];  // T <= 64: each pass's selected ids, kept for the one-wave dispatch
  __shared__ int s_row1[kWave][kSmallMaxK];
  const bool one_wave = T_tok <= kWave;
  for (int tok0 = 0; tok0 < T_tok; tok0 += 16) {
    topk_from_partials<NT>(partial, nsplit, bias, T_tok, E, k, tok0, logit, sel_val, sel_id, ids, w);
    __syncthreads();
    if (one_wave && threadIdx.x < 16 * kSmallMaxK) {
      const int r = threadIdx.x / kSmallMaxK, s = threadIdx.x % kSmallMaxK;
      if (tok0 + r < T_tok) s_ids[tok0 + r][s] = sel_id[r * kMaxExperts + s];  // slots >= k are not read
    }
  }
  if (!one_wave) {
    dispatch_small_block<1024, T, kCap>(ids, X, T_tok, d, E, k, capacity, counts, offsets, perm, inv_perm, Xp);
    return;
  }
  __syncthreads();
  if (threadIdx.x < kWave) {
    const int t = threadIdx.x;
    int e[kSmallMaxK];
#pragma unroll
    for (int s = 0; s < kSmallMaxK; ++s) {
      const int v = (s < k && t < T_tok) ? s_ids[t][s] : -1;
      e[s] = (v >= 0 && v < E) ? v : kNone;
    }
    dispatch_one_wave<kCap>(e, T_tok, E, k, capacity, counts, offsets, perm, inv_perm, &s_row1[0][0], kSmallMaxK);
  }
  if (Xp == nullptr) return;
  __syncthreads();
  copy_rows<1024>(X, Xp, d, k, 0, T_tok, &s_row1[0][0], kSmallMaxK);
}

template <typename T, int KMAX>
hipError_t launch_scatter_k(bool cap, int nblocks, const int32_t* ids, const T* X, int T_tok, int d, int E, int k,
                            const int32_t* cb, const int32_t* offsets, const int8_t* keep, int32_t* perm,
                            int32_t* inv_perm, T* Xp, hipStream_t stream) {
  if (cap)
    hipLaunchKernelGGL((dispatch_scatter_kernel<T, KMAX, true>), dim3(nblocks), dim3(kScatterThreads), 0, stream, ids,
                       X, T_tok, d, E, k, cb, offsets, keep, perm, inv_perm, Xp);
  else
    hipLaunchKernelGGL((dispatch_scatter_kernel<T, KMAX, false>), dim3(nblocks), dim3(kScatterThreads), 0, stream,
                       ids, X, T_tok, d, E, k, cb, offsets, keep, perm, inv_perm, Xp);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_scatter(bool cap, int nblocks, const int32_t* ids, const T* X, int T_tok, int d, int E, int k,
                          const int32_t* cb, const int32_t* offsets, const int8_t* keep, int32_t* perm,
                          int32_t* inv_perm, T* Xp, hipStream_t stream) {
  if (k <= 2) return launch_scatter_k<T, 2>(cap, nblocks, ids, X, T_tok, d, E, k, cb, offsets, keep, perm, inv_perm, Xp, stream);
  if (k <= 4) return launch_scatter_k<T, 4>(cap, nblocks, ids, X, T_tok, d, E, k, cb, offsets, keep, perm, inv_perm, Xp, stream);
  if (k <= 8) return launch_scatter_k<T, 8>(cap, nblocks, ids, X, T_tok, d, E, k, cb, offsets, keep, perm, inv_perm, Xp, stream);
  return launch_scatter_k<T, kMaxExperts>(cap, nblocks, ids, X, T_tok, d, E, k, cb, offsets, keep, perm, inv_perm, Xp, stream);
}

template <typename T, int KMAX>
hipError_t launch_scan_scatter_k(int nblocks, int ntb, const int32_t* ids, const T* X, int T_tok, int d, int E, int k,
                                 const int32_t* H, int Ep, int32_t* counts, int32_t* offsets, int32_t* perm,
                                 int32_t* inv_perm, T* Xp, hipStream_t stream) {
  hipLaunchKernelGGL((dispatch_scan_scatter_kernel<T, KMAX>), dim3(nblocks), dim3(kScatterThreads), 0, stream, ids, X,
                     T_tok, d, E, k, ntb, H, Ep, counts, offsets, perm, inv_perm, Xp);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_scan_scatter(int nblocks, int ntb, const int32_t* ids, const T* X, int T_tok, int d, int E, int k,
                               const int32_t* H, int Ep, int32_t* counts, int32_t* offsets, int32_t* perm,
                               int32_t* inv_perm, T* Xp, hipStream_t stream) {
  if (k <= 2)
    return launch_scan_scatter_k<T, 2>(nblocks, ntb, ids, X, T_tok, d, E, k, H, Ep, counts, offsets, perm, inv_perm,
                                       Xp, stream);
  if (k <= 4)
    return launch_scan_scatter_k<T, 4>(nblocks, ntb, ids, X, T_tok, d, E, k, H, Ep, counts, offsets, perm, inv_perm,
                                       Xp, stream);
  if (k <= 8)
    return launch_scan_scatter_k<T, 8>(nblocks, ntb, ids, X, T_tok, d, E, k, H, Ep, counts, offsets, perm, inv_perm,
                                       Xp, stream);
  return launch_scan_scatter_k<T, kMaxExperts>(nblocks, ntb, ids, X, T_tok, d, E, k, H, Ep, counts, offsets, perm,
                                               inv_perm, Xp, stream);
}

size_t align256(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }

}  // namespace

size_t dispatch_scratch_bytes(int T, int E, int k, bool capacity, bool reroute) {
  const size_t nchunks = (static_cast<size_t>(T) + kDispatchChunk - 1) / kDispatchChunk;
  size_t b = align256(nchunks * (capacity ? k * E : (E + 3) & ~3) * sizeof(int32_t));
  if (capacity) {
    b += align256(nchunks * E * sizeof(int32_t));
    b += align256(static_cast<size_t>(k) * E * sizeof(int32_t));
    b += align256(static_cast<size_t>(T) * k);
    if (reroute) {
      const size_t pairs = static_cast<size_t>(T) * k;
      b += align256(pairs * sizeof(int32_t));             // ids2
      b += align256(nchunks * k * sizeof(int32_t));       // drop_hist
      b += align256((static_cast<size_t>(k) + 1) * sizeof(int32_t));  // drop_seg
      b += align256(pairs * sizeof(int32_t));             // drop_list
      b += align256(pairs * sizeof(int32_t));             // drop_next
      b += align256(pairs * sizeof(uint64_t));            // drop_used
      b += align256(pairs * (E <= 32 ? 32 : 64));         // drop_rows (rows of 32 or 64 bytes)
    }
  }
  return b;
}

DispatchScratch carve_dispatch_scratch(void* ws, int T, int E, int k, bool capacity, bool reroute) {
  const size_t nchunks = (static_cast<size_t>(T) + kDispatchChunk - 1) / kDispatchChunk;
  unsigned char* p = static_cast<unsigned char*>(ws);
  DispatchScratch s{};
  s.chunk_base = reinterpret_cast<int32_t*>(p);
  p += align256(nchunks * (capacity ? k * E : (E + 3) & ~3) * sizeof(int32_t));
  if (capacity) {
    s.chunk_kept = reinterpret_cast<int32_t*>(p);
    p += align256(nchunks * E * sizeof(int32_t));
    s.slot_base = reinterpret_cast<int32_t*>(p);
    p += align256(static_cast<size_t>(k) * E * sizeof(int32_t));
    s.keep = reinterpret_cast<int8_t*>(p);
    p += align256(static_cast<size_t>(T) * k);
    if (reroute) {
      const size_t pairs = static_cast<size_t>(T) * k;
      s.ids2 = reinterpret_cast<int32_t*>(p);
      p += align256(pairs * sizeof(int32_t));
      s.drop_hist = reinterpret_cast<int32_t*>(p);
      p += align256(nchunks * k * sizeof(int32_t));
      s.drop_seg = reinterpret_cast<int32_t*>(p);
      p += align256((static_cast<size_t>(k) + 1) * sizeof(int32_t));
      s.drop_list = reinterpret_cast<int32_t*>(p);
      p += align256(pairs * sizeof(int32_t));
      s.drop_next = reinterpret_cast<int32_t*>(p);
      p += align256(pairs * sizeof(int32_t));
      s.drop_used = reinterpret_cast<uint64_t*>(p);
      p += align256(pairs * sizeof(uint64_t));
      s.drop_rows = reinterpret_cast<uint8_t*>(p);
    }
  }
  return s;
}

bool dispatch_is_single_block(int T, int k) { return T > 0 && T <= kSmallMaxT && k <= kSmallMaxK; }

namespace {
template <typename T, bool kCap>
hipError_t launch_topk_dispatch_t(const float* partial, int nsplit, const float* bias, int32_t* ids, float* w,
                                  const T* X, int T_tok, int d, int E, int k, int capacity, int32_t* counts,
                                  int32_t* offsets, int32_t* perm, int32_t* inv_perm, T* Xp, hipStream_t stream) {
#define MOE_TOPK_DISPATCH(NT)                                                                                      \
  hipLaunchKernelGGL((topk_dispatch_small_kernel<T, kCap, NT>), dim3(1), dim3(1024), 0, stream, partial, nsplit, \
                     bias, ids, w, X, T_tok, d, E, k, capacity, counts, offsets, perm, inv_perm, Xp)
  switch ((E + 15) / 16) {
    case 1: MOE_TOPK_DISPATCH(1); break;
    case 2: MOE_TOPK_DISPATCH(2); break;
    case 3: MOE_TOPK_DISPATCH(3); break;
    default: MOE_TOPK_DISPATCH(4); break;
  }
#undef MOE_TOPK_DISPATCH
  return hipGetLastError();
}
}  // namespace

hipError_t launch_topk_dispatch_small(int dtype, const float* partial, int nsplit, const float* bias, int32_t* ids,
                                      float* w, const void* X, int T, int d, int E, int k, int capacity,
                                      int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv_perm, void* Xp,
                                      hipStream_t stream) {
  if (!dispatch_is_single_block(T, k) || partial == nullptr) return hipErrorInvalidValue;
  const bool cap = capacity >= 0;
  if (dtype == kDtypeBF16) {
    const uint16_t* x = static_cast<const uint16_t*>(X);
    uint16_t* xp = static_cast<uint16_t*>(Xp);
    return cap ? launch_topk_dispatch_t<uint16_t, true>(partial, nsplit, bias, ids, w, x, T, d, E, k, capacity, counts,
                                                        offsets, perm, inv_perm, xp, stream)
               : launch_topk_dispatch_t<uint16_t, false>(partial, nsplit, bias, ids, w, x, T, d, E, k, capacity,
                                                         counts, offsets, perm, inv_perm, xp, stream);
  }
  const float* x = static_cast<const float*>(X);
  float* xp = static_cast<float*>(Xp);
  return cap ? launch_topk_dispatch_t<float, true>(partial, nsplit, bias, ids, w, x, T, d, E, k, capacity, counts,
                                                   offsets, perm, inv_perm, xp, stream)
             : launch_topk_dispatch_t<float, false>(partial, nsplit, bias, ids, w, x, T, d, E, k, capacity, counts,
                                                    offsets, perm, inv_perm, xp, stream);
}

hipError_t launch_dispatch(int dtype, const int32_t* ids, const void* X, int T, int d, int E, int k, int capacity,
                           int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv_perm, void* Xp,
                           const DispatchScratch& sc, hipStream_t stream) {
  const bool cap = capacity >= 0;
  const int nchunks = (T + kDispatchChunk - 1) / kDispatchChunk;
  const int total_pairs = T * k;
  if (dispatch_is_single_block(T, k)) {
    if (dtype == kDtypeBF16) {
      if (cap)
        hipLaunchKernelGGL((dispatch_small_kernel<uint16_t, true>), dim3(1), dim3(256), 0, stream, ids,
                           static_cast<const uint16_t*>(X), T, d, E, k, capacity, counts, offsets, perm, inv_perm,
                           static_cast<uint16_t*>(Xp));
      else
        hipLaunchKernelGGL((dispatch_small_kernel<uint16_t, false>), dim3(1), dim3(256), 0, stream, ids,
                           static_cast<const uint16_t*>(X), T, d, E, k, capacity, counts, offsets, perm, inv_perm,
                           static_cast<uint16_t*>(Xp));
    } else {
      if (cap)
        hipLaunchKernelGGL((dispatch_small_kernel<float, true>), dim3(1), dim3(256), 0, stream, ids,
                           static_cast<const float*>(X), T, d, E, k, capacity, counts, offsets, perm, inv_perm,
                           static_cast<float*>(Xp));
      else
        hipLaunchKernelGGL((dispatch_small_kernel<float, false>), dim3(1), dim3(256), 0, stream, ids,
                           static_cast<const float*>(X), T, d, E, k, capacity, counts, offsets, perm, inv_perm,
                           static_cast<float*>(Xp));
    }
    return hipGetLastError();
  }
  if (T <= 0) {
    // No tokens: every expert is empty.
    hipLaunchKernelGGL(dispatch_scan_kernel, dim3(1), dim3(kScanThreads), 0, stream, sc.chunk_base, 0, E,
                       static_cast<int>(kScanDropless), E, k, capacity, counts, offsets, sc.slot_base, perm, 0);
    return hipGetLastError();
  }
  const int cols = cap ? k * E : E;
  const int Ep = (E + 3) & ~3;
  if (!cap && static_cast<int64_t>(nchunks) * Ep <= kScanScatterMaxCells) {
    // Dropless, histograms small enough for every block to sum: two launches.
    hipLaunchKernelGGL(dispatch_count_kernel, dim3(nchunks), dim3(kWave), 0, stream, ids, T, E, k,
                       false, Ep, sc.chunk_base);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    const int ntb = Xp != nullptr ? kScatterTok : kDispatchChunk;
    const int nblocks = (T + ntb - 1) / ntb;
    if (dtype == kDtypeBF16)
      return launch_scan_scatter<uint16_t>(nblocks, ntb, ids, static_cast<const uint16_t*>(X), T, d, E, k,
                                           sc.chunk_base, Ep, counts, offsets, perm, inv_perm,
                                           static_cast<uint16_t*>(Xp), stream);
    return launch_scan_scatter<float>(nblocks, ntb, ids, static_cast<const float*>(X), T, d, E, k, sc.chunk_base, Ep,
                                      counts, offsets, perm, inv_perm, static_cast<float*>(Xp), stream);
  }
  hipLaunchKernelGGL(dispatch_count_kernel, dim3(nchunks), dim3(kWave), 0, stream, ids, T, E, k, cap,
                     cols, sc.chunk_base);
  hipLaunchKernelGGL(dispatch_scan_kernel, dim3(1), dim3(kScanThreads), 0, stream, sc.chunk_base, nchunks, cols,
                     static_cast<int>(cap ? kScanCapacity1 : kScanDropless), E, k, capacity, counts, offsets,
                     sc.slot_base, perm, total_pairs);
  const int32_t* row_base = sc.chunk_base;
  if (cap) {
    hipLaunchKernelGGL(dispatch_keep_kernel, dim3(nchunks), dim3(kWave), 0, stream, ids, T, E, k, capacity,
                       sc.chunk_base, sc.slot_base, sc.keep, sc.chunk_kept);
    hipLaunchKernelGGL(dispatch_scan_kernel, dim3(1), dim3(kScanThreads), 0, stream, sc.chunk_kept, nchunks, E,
                       static_cast<int>(kScanCapacity2), E, k, capacity, counts, offsets, sc.slot_base, perm,
                       total_pairs);
    row_base = sc.chunk_kept;
  }
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  const int nblocks = (T + kScatterTok - 1) / kScatterTok;
  if (dtype == kDtypeBF16)
    return launch_scatter<uint16_t>(cap, nblocks, ids, static_cast<const uint16_t*>(X), T, d, E, k, row_base, offsets,
                                    sc.keep, perm, inv_perm, static_cast<uint16_t*>(Xp), stream);
  return launch_scatter<float>(cap, nblocks, ids, static_cast<const float*>(X), T, d, E, k, row_base, offsets, sc.keep,
                               perm, inv_perm, static_cast<float*>(Xp), stream);
}

hipError_t launch_dispatch_reroute(int dtype, const int32_t* ids, const uint8_t* order, const void* X, int T, int d,
                                   int E, int k, int capacity, int32_t* counts, int32_t* offsets, int32_t* perm,
                                   int32_t* inv_perm, void* Xp, const DispatchScratch& sc, hipStream_t stream) {
  // Without a capacity nothing overflows: the plain dispatch.  No tokens:
  // every expert is empty (the plain dispatch's path).
  if (capacity < 0 || T <= 0)
    return launch_dispatch(dtype, ids, X, T, d, E, k, capacity, counts, offsets, perm, inv_perm, Xp, sc, stream);
  if (order == nullptr || sc.ids2 == nullptr) return hipErrorInvalidValue;
  const int nchunks = (T + kDispatchChunk - 1) / kDispatchChunk;
  const int total_pairs = T * k;
  const int cols = k * E;
  hipLaunchKernelGGL(dispatch_count_kernel, dim3(nchunks), dim3(kWave), 0, stream, ids, T, E, k, true,
                     cols, sc.chunk_base);
  hipLaunchKernelGGL(dispatch_scan_kernel, dim3(1), dim3(kScanThreads), 0, stream, sc.chunk_base, nchunks, cols,
                     static_cast<int>(kScanCapacity1), E, k, capacity, counts, offsets, sc.slot_base, perm,
                     total_pairs);
  hipLaunchKernelGGL(dispatch_keep_kernel, dim3(nchunks), dim3(kWave), 0, stream, ids, T, E, k, capacity,
                     sc.chunk_base, sc.slot_base, sc.keep, sc.chunk_kept);
  hipLaunchKernelGGL(dispatch_drop_count_kernel, dim3(nchunks), dim3(kWave), 0, stream, ids, sc.keep, T, E, k,
                     sc.drop_hist, sc.ids2);
  hipLaunchKernelGGL(dispatch_scan_kernel, dim3(1), dim3(kScanThreads), 0, stream, sc.drop_hist, nchunks, k,
                     static_cast<int>(kScanOffsets), k, k, capacity, nullptr, sc.drop_seg, nullptr, nullptr, 0);
  const int rstride = E <= 32 ? 32 : 64;
  hipLaunchKernelGGL(dispatch_drop_list_kernel, dim3(nchunks), dim3(kWave), 0, stream, ids, sc.keep, order, T, E, k,
                     rstride, sc.drop_hist, sc.drop_seg, sc.drop_list, sc.drop_rows, sc.drop_next, sc.drop_used);
  if (E <= 32)
    hipLaunchKernelGGL(dispatch_reroute_kernel<32>, dim3(1), dim3(kRerouteThreads), 0, stream, counts, sc.drop_seg,
                       sc.drop_list, sc.drop_rows, sc.drop_next, sc.drop_used, E, k, capacity, sc.keep, sc.ids2);
  else
    hipLaunchKernelGGL(dispatch_reroute_kernel<64>, dim3(1), dim3(kRerouteThreads), 0, stream, counts, sc.drop_seg,
                       sc.drop_list, sc.drop_rows, sc.drop_next, sc.drop_used, E, k, capacity, sc.keep, sc.ids2);
  hipLaunchKernelGGL(dispatch_count_kept_kernel, dim3(nchunks), dim3(kWave), 0, stream, sc.ids2, sc.keep, T, E, k,
                     sc.chunk_kept);
  hipLaunchKernelGGL(dispatch_scan_kernel, dim3(1), dim3(kScanThreads), 0, stream, sc.chunk_kept, nchunks, E,
                     static_cast<int>(kScanOffsets), E, k, capacity, counts, offsets, sc.slot_base, perm,
                     total_pairs);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  const int nblocks = (T + kScatterTok - 1) / kScatterTok;
  if (dtype == kDtypeBF16)
    return launch_scatter<uint16_t>(true, nblocks, sc.ids2, static_cast<const uint16_t*>(X), T, d, E, k,
                                    sc.chunk_kept, offsets, sc.keep, perm, inv_perm, static_cast<uint16_t*>(Xp),
                                    stream);
  return launch_scatter<float>(true, nblocks, sc.ids2, static_cast<const float*>(X), T, d, E, k, sc.chunk_kept,
                               offsets, sc.keep, perm, inv_perm, static_cast<float*>(Xp), stream);
}

}  // namespace moe
