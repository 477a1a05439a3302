// SwiGLU experts as one grouped GEMM launch per projection, scheduled on the
// device from the per-expert offsets (no host synchronisation).
//
// Groups: the E routed experts (rows = that expert's segment of the
// expert-contiguous order) and, optionally, the shared expert as group E
// (rows = all T tokens, identity gather).  Each group's tiles are
// (m-tile, n-tile) pairs; a tiny schedule kernel turns offsets into the first
// tile id of every group, and each workgroup finds its group by binary search.
//
//   up   : h[r, n]   = silu(x_r . W1[n]) * (x_r . W3[n])     (fp32 accumulate)
//   down : out[r, n] = h_r . W2[n]
// x rows are gathered through sorted_token inside the operand loads.
//
// Skinny tiles (16 tokens) stream weights straight from HBM into the MFMA
// A operand: each weight element is used once per tile, so staging it in LDS
// would add latency without reuse.  The token operand is the B side (16
// columns) and is read through the caches.
#include "common.h"
#include "kernels.h"

#include <algorithm>
#include <numeric>
#include <type_traits>
#include <utility>

namespace moe {

// Three schedules of E + 2 ints each: the up launch, the down launch, and the
// down launch of the shared expert fused with the combine.  Entry g is the
// first tile of group g, entry E + 1 the launch's tile count.
__global__ __launch_bounds__(1024) void ffn_schedule_kernel(const int32_t* __restrict__ offsets,
                                                            int E, int ntok, int routed,
                                                            int shared_up, int shared_down,
                                                            int bm, int bm_dn, int nt_up, int nt_up_s,
                                                            int nt_dn, int bm_s, int nt_dn_s, int e_begin,
                                                            int e_end,
                                                            int32_t* __restrict__ sched) {
  __shared__ int sc[3][1024];
  const int g = threadIdx.x;
  int c[3] = {0, 0, 0};
  if (routed && g < E && g >= e_begin && g < e_end) {   // experts outside the range get no tiles
    const int M = offsets[g + 1] - offsets[g];
    c[0] = (M + bm - 1) / bm * nt_up;
    c[1] = (M + bm_dn - 1) / bm_dn * nt_dn;
  } else if (g == E) {
    c[0] = shared_up ? (ntok + bm - 1) / bm * nt_up_s : 0;
    c[1] = shared_down == 1 ? (ntok + bm_dn - 1) / bm_dn * nt_dn : 0;
    c[2] = shared_down == 2 ? (ntok + bm_s - 1) / bm_s * nt_dn_s : 0;
  }
#pragma unroll
  for (int s = 0; s < 3; ++s) sc[s][g] = c[s];
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    int v[3];
#pragma unroll
    for (int s = 0; s < 3; ++s) v[s] = g >= o ? sc[s][g - o] : 0;
    __syncthreads();
#pragma unroll
    for (int s = 0; s < 3; ++s) sc[s][g] += v[s];
    __syncthreads();
  }
#pragma unroll
  for (int s = 0; s < 3; ++s) {
    if (g <= E) sched[s * (E + 2) + g] = sc[s][g] - c[s];
    if (g == E) sched[s * (E + 2) + E + 1] = sc[s][g];
  }
}

typedef __attribute__((ext_vector_type(8))) int i32x8_t_;

struct TileInfo {
  int g;        // group (E = shared)
  int row0;     // first row of the group in the expert-contiguous order
  int M;        // rows of the group
  int mt, nt;   // tile coordinates
  int m0;       // first row of the m-tile within the group
  int mrows;    // rows of the m-tile (> 0)
};

// Maps this workgroup to a tile; returns false when it has none.  The grid is
// an upper bound on the tile count (the real count is only known on the
// device), so the XCD-aware remap runs over the real count rounded up to 8:
// every XCD then gets an equal, contiguous range of tiles (all n-tiles and
// m-tiles of an expert next to each other, sharing its rows in that XCD's
// L2), and the surplus workgroups exit.  A group of M rows is cut into
// ceil(M / bm) m-tiles of equal size (rounded up to the 32-row sub-tile, or to
// bm when bm < 32), the last one taking the remainder: m-tiles of one expert
// then take about the same time and stream its weight slices together, so the
// second reads them from L2.
// With split_shared the routed tiles and the shared expert's tiles are split
// over the 8 XCDs separately, each XCD taking an equal contiguous share of
// both.  One range over the whole order puts all the shared expert's tiles -
// full-height m-tiles, where routed m-tiles average fewer rows - on the last
// XCD, which then has 7-16 % more sub-tiles to multiply than the others on
// the prefill workloads.  That pays where a tile's time follows its rows (the
// fp8 up launch: 3.21 -> 2.97 ms on the 8192-token layer; the 256-token bf16
// up tiles: about 1 %), not where it follows its weight bytes (the
// 128 x 512 bf16 up tiles: 3.22 -> 3.29 ms).  The grid needs up to two more
// workgroups per XCD.
__device__ __forceinline__ bool find_tile(const int32_t* __restrict__ sched,
                                          const int32_t* __restrict__ offsets, int E, int ntok,
                                          int bm, TileInfo& ti, bool split_shared = false) {
  const int total = sched[E + 1];
  int tile;
  if (split_shared) {
    const int Sr = sched[E], Ss = total - Sr;
    const int x = blockIdx.x & 7, j = blockIdx.x >> 3;
    const int r0 = (int)((long)Sr * x / 8), r1 = (int)((long)Sr * (x + 1) / 8);
    const int s0 = (int)((long)Ss * x / 8), s1 = (int)((long)Ss * (x + 1) / 8);
    if (j < r1 - r0) tile = r0 + j;
    else if (j - (r1 - r0) < s1 - s0) tile = Sr + s0 + j - (r1 - r0);
    else return false;
  } else {
    const int n8 = (total + 7) & ~7;
    if ((int)blockIdx.x >= n8) return false;
    tile = xcd_remap(blockIdx.x, n8);
    if (tile >= total) return false;
  }
  int lo = 0, hi = E + 1;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (sched[mid] <= tile) lo = mid; else hi = mid;
  }
  ti.g = lo;
  if (lo == E) { ti.row0 = 0; ti.M = ntok; }
  else { ti.row0 = offsets[lo]; ti.M = offsets[lo + 1] - ti.row0; }
  const int mtiles = (ti.M + bm - 1) / bm;
  const int local = tile - sched[lo];
  ti.mt = local % mtiles;
  ti.nt = local / mtiles;
  const int gran = bm < 32 ? bm : 32;
  const int per = min(bm, ((ti.M + mtiles - 1) / mtiles + gran - 1) / gran * gran);
  ti.m0 = ti.mt * per;                 // (mtiles - 1) * per < M: every m-tile has rows
  ti.mrows = min(per, ti.M - ti.m0);
  return true;
}

// Expert weights are stored in 16-row x 64-byte tiles (the layout
// moe_pack_weights writes): tile (row/16, byte/64) of a matrix with row_bytes
// bytes per row is 1 KB, made of the 16-byte pieces (row%16, (byte%64)/16) in
// the order (row%16) + 16*((byte%64)/16) - the order in which the 64 lanes of
// a wave hold a 16x16x32 bf16 MFMA A operand.  A wave's fragment loads are
// then whole 128-byte lines, contiguous per tile.  Consecutive 64-byte chunks
// of a row are 1 KB apart.
__device__ __forceinline__ size_t wtile_off(int row, int byte, int row_bytes) {
  return ((size_t)(row >> 4) * (row_bytes >> 6) + (byte >> 6)) * 1024 +
         16 * ((row & 15) + 16 * ((byte >> 4) & 3)) + (byte & 15);
}
constexpr int kChunkStride = 1024;   // bytes between consecutive 64-byte K chunks of a tiled row

// Double-buffered K loop over 64-byte chunks: U chunks per stage, NA A-operand
// rows (16-row tiles, tiled weights) against one B operand (a plain row).
// nchunk must be a multiple of U.
template <typename T, int NA, int U>
__device__ __forceinline__ void kloop(const char* const (&ap)[NA], const char* bp, int nchunk,
                                      f32x4_t (&acc)[NA]) {
  uint4 a0[U][NA], b0[U], a1[U][NA], b1[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    b0[u] = ldg16(bp + 64 * u);
#pragma unroll
    for (int j = 0; j < NA; ++j) a0[u][j] = ldg16_stream(ap[j] + kChunkStride * u);
  }
  for (int c = 0; c < nchunk; c += 2 * U) {
    if (c + U < nchunk) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        b1[u] = ldg16(bp + 64 * (c + U + u));
#pragma unroll
        for (int j = 0; j < NA; ++j) a1[u][j] = ldg16_stream(ap[j] + kChunkStride * (c + U + u));
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int j = 0; j < NA; ++j) acc[j] = Chunk<T>::mma(acc[j], a0[u][j], b0[u]);
    if (c + 2 * U < nchunk) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        b0[u] = ldg16(bp + 64 * (c + 2 * U + u));
#pragma unroll
        for (int j = 0; j < NA; ++j) a0[u][j] = ldg16_stream(ap[j] + kChunkStride * (c + 2 * U + u));
      }
    }
    if (c + U < nchunk) {
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int j = 0; j < NA; ++j) acc[j] = Chunk<T>::mma(acc[j], a1[u][j], b1[u]);
    }
  }
}

template <typename T> __device__ __forceinline__ void store4(T* p, const float (&v)[4]);
template <> __device__ __forceinline__ void store4<uint16_t>(uint16_t* p, const float (&v)[4]) {
  uint2 o;
  o.x = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
  o.y = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
  *reinterpret_cast<uint2*>(p) = o;
}
template <> __device__ __forceinline__ void store4<float>(float* p, const float (&v)[4]) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}

constexpr int kSkinnyWaves = 4;
constexpr int kUpNT = 2;     // 16-row tiles of W1 (and of W3) per wave
constexpr int kDnNT = 2;     // 16-row tiles of W2 per wave (bf16, fp32)
constexpr int kDnNT8 = 4;    // 16-row tiles of W2 per wave (fp8)
constexpr int kUpBN = kSkinnyWaves * 16 * kUpNT;   // h columns per workgroup
constexpr int kDnBN = kSkinnyWaves * 16 * kDnNT;   // output columns per workgroup
constexpr int kDnBN8 = kSkinnyWaves * 16 * kDnNT8;
static_assert(kUpBN == 128, "the fp8 decode up kernel covers 128 h columns per workgroup");

template <typename T>
__global__ __launch_bounds__(256) void up_skinny_kernel(FfnProblem p) {
  TileInfo ti;
  if (!find_tile(p.sched, p.offsets, p.E, p.ntok, 16, ti)) return;
  const bool shared = ti.g == p.E;
  const int N = shared ? p.inter_s : p.inter;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, grp = lane >> 4;
  const int nbase = ti.nt * kUpBN + wave * 16 * kUpNT;
  if (nbase >= N) return;
  const int mi = ti.m0 + min(r, ti.mrows - 1);
  const int xrow = shared ? mi : p.sorted_token[ti.row0 + mi];
  const char* bp = reinterpret_cast<const char*>(static_cast<const T*>(p.x) + (size_t)xrow * p.dim) + 16 * grp;
  const T* W1 = shared ? static_cast<const T*>(p.ws1) : static_cast<const T*>(p.w1) + (size_t)(ti.g - p.e_begin) * N * p.dim;
  const T* W3 = shared ? static_cast<const T*>(p.ws3) : static_cast<const T*>(p.w3) + (size_t)(ti.g - p.e_begin) * N * p.dim;
  const int rb = p.dim * (int)sizeof(T);
  const char* ap[2 * kUpNT];
#pragma unroll
  for (int j = 0; j < kUpNT; ++j) {
    const int n = nbase + 16 * j + r;
    ap[j] = reinterpret_cast<const char*>(W1) + wtile_off(n, 16 * grp, rb);
    ap[kUpNT + j] = reinterpret_cast<const char*>(W3) + wtile_off(n, 16 * grp, rb);
  }
  f32x4_t acc[2 * kUpNT];
#pragma unroll
  for (int j = 0; j < 2 * kUpNT; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  kloop<T, 2 * kUpNT, 2>(ap, bp, p.dim * (int)sizeof(T) / 64, acc);

  const int m = ti.m0 + r;
  if (r < ti.mrows) {
    T* hrow = shared ? static_cast<T*>(p.hs) + (size_t)m * N
                     : static_cast<T*>(p.h) + (size_t)(ti.row0 + m) * N;
#pragma unroll
    for (int j = 0; j < kUpNT; ++j) {
      const int n = nbase + 16 * j + 4 * grp;
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = silu(acc[j][i]) * acc[kUpNT + j][i];
      store4<T>(hrow + n, v);
    }
  }
}

// The fused combine of a shared-expert down tile: the tile's outputs go to
// LDS rounded to the layer dtype (the shared module's output), then the whole
// workgroup forms y for the tile's tokens and columns (combine.h).
template <typename T, int NP>
__device__ __forceinline__ void combine_from_lds(const FfnProblem& p, const Slot* slots, const T* s_tile,
                                                 int ld, const TileInfo& ti, int n0, int bn) {
  const int ncols = min(bn, p.dim - n0);
  if (p.comb.layer_acc)
    combine_tile<T, true, NP>(p.comb, slots, s_tile, ld, ti.m0, ti.mrows, n0, ncols, p.dim);
  else
    combine_tile<T, false, NP>(p.comb, slots, s_tile, ld, ti.m0, ti.mrows, n0, ncols, p.dim);
}

// kComb: the launch holds only the shared expert's tiles, and each ends with
// the combine instead of storing the shared output.
template <typename T, bool kComb>
__global__ __launch_bounds__(256) void down_skinny_kernel(FfnProblem p) {
  constexpr int LD = kDnBN + 8;                     // LDS row of the combine tile (elements)
  __shared__ __attribute__((aligned(16))) T s_tile[kComb ? 16 * LD : 1];
  __shared__ __attribute__((aligned(16))) Slot slots[kComb ? 16 * kRegSlots : 1];
  TileInfo ti;
  const int32_t* sched = p.sched + (kComb ? 2 : 1) * (p.E + 2);
  if (!find_tile(sched, p.offsets, p.E, p.ntok, 16, ti)) return;
  SlotLoad sl;                                      // the tokens' routing, loaded under the K loop
  if constexpr (kComb) slots_issue(p.comb, ti.m0, ti.mrows, sl);
  const bool shared = ti.g == p.E;
  const int K = shared ? p.inter_s : p.inter;
  const int N = p.dim;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, grp = lane >> 4;
  const int nbase = ti.nt * kDnBN + wave * 16 * kDnNT;
  if (!kComb && nbase >= N) return;
  const bool active = nbase < N;                    // waves past the last column still meet the barrier
  const int mi = ti.m0 + min(r, ti.mrows - 1);
  const T* hrow = shared ? static_cast<const T*>(p.hs) + (size_t)mi * K
                         : static_cast<const T*>(p.h) + (size_t)(ti.row0 + mi) * K;
  const char* bp = reinterpret_cast<const char*>(hrow) + 16 * grp;
  const T* W2 = shared ? static_cast<const T*>(p.ws2) : static_cast<const T*>(p.w2) + (size_t)(ti.g - p.e_begin) * N * K;
  const char* ap[kDnNT];
#pragma unroll
  for (int j = 0; j < kDnNT; ++j)
    ap[j] = reinterpret_cast<const char*>(W2) + wtile_off(min(nbase + 16 * j + r, N - 1), 16 * grp, K * (int)sizeof(T));
  f32x4_t acc[kDnNT];
#pragma unroll
  for (int j = 0; j < kDnNT; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  if (active) kloop<T, kDnNT, 2>(ap, bp, K * (int)sizeof(T) / 64, acc);

  const int m = ti.m0 + r;
  if constexpr (kComb) {
    if (active && r < ti.mrows) {
#pragma unroll
      for (int j = 0; j < kDnNT; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float v = to_layer<T>(acc[j][i]);
          T* d = s_tile + r * LD + wave * 16 * kDnNT + 16 * j + 4 * grp + i;
          if constexpr (sizeof(T) == 2) *d = (T)(__float_as_uint(v) >> 16);
          else *d = v;
        }
    }
    slots_store(p.comb, ti.mrows, sl, slots);
    __syncthreads();
    combine_from_lds<T, 1>(p, slots, s_tile, LD, ti, ti.nt * kDnBN, kDnBN);
    return;
  }
  if (r < ti.mrows) {
    T* orow = shared ? static_cast<T*>(p.shared_out) + (size_t)m * N
                     : static_cast<T*>(p.out) + (size_t)(ti.row0 + m) * N;
#pragma unroll
    for (int j = 0; j < kDnNT; ++j) {
      float v[4] = {acc[j][0], acc[j][1], acc[j][2], acc[j][3]};
      store4<T>(orow + nbase + 16 * j + 4 * grp, v);
    }
  }
}

// ---------------------------------------------------------------------------
// Stream tiles (prefill): 64 to 256 token rows x 256 or 512 weight rows per
// workgroup of 8 waves (two per SIMD), on v_mfma_f32_32x32x16_bf16 (the
// 32x32 shape runs at full rate on gfx950; 16x16x32 issues at half rate).
// A tile covers a whole expert whenever it has no more rows than the tile,
// so each weight slice is fetched from HBM once per expert.
//   A operand = one or two 32-row weight tiles per wave, loaded straight from
//     global memory through a ring of register stages (two or three K slices
//     of 32 or 64 elements in flight); for the up projection rows 0-15 of a
//     tile are W1 rows and rows 16-31 the same rows of W3, so a lane's result
//     elements i and i+8 are the two branches of one h column and SwiGLU
//     needs no data exchange.
//   B operand = token rows, staged in LDS (four or eight buffers, one
//     workgroup barrier per half of them) and read by all 8 waves (each token
//     fragment feeds the wave's one or two A tiles): the slice of every
//     n-tile of an expert is the same, so it is mostly L2-resident.
// Loaded HBM latency is several microseconds, so weights run several K
// slices ahead and token slices are loaded into registers a few steps before
// their LDS store.
// Memory counters retire in issue order; each step issues its token slice
// before its weight slice, so waiting for a token slice to store never forces
// a newer weight slice to land early.  The K loop is instantiated for the
// number of 32-row token sub-tiles it computes.  LDS rows are padded by 16
// bytes so the fragment reads of a wave spread over the banks.
// ---------------------------------------------------------------------------
// Tile shape of the stream kernel: BM token rows, WAVES waves of NA 32-row
// weight tiles each, BK-element K slices.
template <int BM_, int WAVES_, int RING_, int XD_ = 2, int NB_ = 4, int WPE_ = 2, bool NTW_ = false,
          int NA_ = 1, int BK_ = 64>
struct SCfg {
  static constexpr int BM = BM_;
  static constexpr int WAVES = WAVES_;
  static constexpr int THREADS = WAVES * 64;
  static constexpr int MT = BM / 32;               // 32-row token sub-tiles
  static constexpr int NA = NA_;                   // 32-row weight tiles per wave
  static constexpr int BN = WAVES * 32 * NA;       // weight rows per tile
  static constexpr int UPBN = BN / 2;              // h columns per up tile
  static constexpr int BK = BK_;                   // K elements per step (32 or 64)
  static constexpr int KS = BK / 16;               // MFMA k-steps per step
  static constexpr int STRIDE = 2 * BK + 16;       // LDS bytes per token row
  static constexpr int LDS = BM * STRIDE;
  static constexpr int TPR = 2 * BK / 16;          // threads per token row (16 B each)
  static constexpr int ROWS_PER_PASS = THREADS / TPR;
  static constexpr int XLOADS = (BM + ROWS_PER_PASS - 1) / ROWS_PER_PASS;
  static constexpr int RING = RING_;               // weight register stages (RING-1 slices ahead)
  static constexpr int XD = XD_;                   // token register stages
  static constexpr int NB = NB_;                   // token LDS buffers
  static constexpr int D = NB / 2;                 // steps per barrier; slice kt+D is stored after step kt
  static constexpr int UNROLL = std::lcm(std::lcm(RING, XD), D);   // steps with compile-time stage indices
  static constexpr int WPE = WPE_;                 // waves per SIMD (workgroups per CU * WAVES / 4)
  static constexpr bool NTW = NTW_;                // weights through non-temporal loads
  static_assert(NB == 2 || NB == 4 || NB == 8, "two, four or eight token buffers");
};
// whole experts of ~128-192 tokens (down projection), one workgroup per CU
using SBig = SCfg<192, 8, 4, 3>;
// The up projection of the same batches: 128 tokens x 512 weight rows, two
// 32-row A tiles per wave sharing each token fragment, 32-element K steps so
// a 4-stage weight ring fits beside the doubled accumulators, 8 token
// buffers (a barrier every 4 steps).  Half the n-tiles of 256-row tiles, so
// half the token re-reads through L2 and half the LDS fragment reads per
// MFMA (up launch of the DeepSeek-V3 layer at 4096 tokens 3.37 -> 3.20 ms;
// on the down projection the same tiles were slower, and 192-token or
// 64-element-step versions with deeper rings need scratch)
using SBigUp = SCfg<128, 8, 4, 2, 8, 2, false, 2, 32>;
using SHuge = SCfg<256, 8, 2, 1>; // experts of many hundred tokens: larger tiles, shallower rings
// 64-token tiles of 256 weight rows (8 waves); used while experts average
// fewer than 32 rows, so their weights are always read non-temporally
using SMid = SCfg<64, 8, 4, 2, 4, 2, true>;
// 128-token tiles with non-temporal weight loads, for batches averaging
// 32-64 rows per expert: an expert fills one m-tile, so each weight slice is
// read about once
using SBigNT = SCfg<128, 8, 4, 3, 4, 2, true>;
// The shared expert's down tiles fused with the combine (one launch of T
// rows): every m-tile reads the same weight slices, so ordinary loads.
#ifndef MOE_COMB_BM
#define MOE_COMB_BM 128
#endif
using SComb = SCfg<MOE_COMB_BM, 8, 4, (MOE_COMB_BM >= 128 ? 3 : 2), 4, 2, false>;

template <class C>
struct StreamSrc {
  const char* x[C::XLOADS];  // token rows (tid / TPR) + ROWS_PER_PASS*i, at byte 16*(tid % TPR)
  const char* w[C::NA];      // this lane's row of each weight tile, at byte 16*(lane/32)
  int lds_st;                // LDS byte offset of this thread's token chunk
  bool xact[C::XLOADS];      // row inside the tile (for BM not a multiple of the pass)
};

__device__ __forceinline__ f32x16_t mma32(f32x16_t c, uint4 a, uint4 b) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

template <class C, int MT, bool kNTW = C::NTW>
__device__ __forceinline__ void stream_kloop(char (&sx)[C::NB][C::LDS], const StreamSrc<C>& S, int nk,
                                             f32x16_t (&acc)[C::NA][C::MT]) {
  const int lane = threadIdx.x & 63, fr = lane & 31, fg = lane >> 5;
  uint4 wr[C::RING][C::NA][C::KS];   // weight slices in flight: [slice % RING][tile][k-step]
  // token load passes that reach the MT*32 rows this instantiation reads
  constexpr int XL = std::min(C::XLOADS, (32 * MT + C::ROWS_PER_PASS - 1) / C::ROWS_PER_PASS);
  uint4 xr[C::XD][C::XLOADS]; // token slices in flight between load and LDS store: [slice % XD]
  auto wload = [&](uint4 (&dst)[C::NA][C::KS], int kt) {
    kt = kt < nk ? kt : nk - 1;
#pragma unroll
    for (int j = 0; j < C::NA; ++j)
#pragma unroll
      for (int s = 0; s < C::KS; ++s) {   // k-step s: bytes 32s + 16*(lane/32) of the 2*BK-byte slice
        const char* a = S.w[j] + ((kt * 2 * C::BK + 32 * s) >> 6) * kChunkStride + (s & 1) * 512;
        dst[j][s] = kNTW ? ldg16_stream(a) : ldg16(a);
      }
  };
  auto xload = [&](uint4 (&dst)[C::XLOADS], int kt) {
    kt = kt < nk ? kt : nk - 1;
#pragma unroll
    for (int i = 0; i < XL; ++i) dst[i] = ldg16(S.x[i] + kt * (2 * C::BK));
  };
  auto xstore = [&](const uint4 (&src)[C::XLOADS], int buf) {
#pragma unroll
    for (int i = 0; i < XL; ++i)
      if (S.xact[i]) *reinterpret_cast<uint4*>(&sx[buf][S.lds_st + C::ROWS_PER_PASS * i * C::STRIDE]) = src[i];
  };
  // token slice j lives in LDS buffer j % NB.  Slices 0 .. D-1 go to LDS
  // first; slices D .. D+XD-2 wait in registers.
#pragma unroll
  for (int j = 0; j < C::D; ++j) {
    xload(xr[j % C::XD], j);
    xstore(xr[j % C::XD], j);
  }
#pragma unroll
  for (int j = C::D; j < C::D + C::XD - 1; ++j) xload(xr[j % C::XD], j);
#pragma unroll
  for (int j = 0; j < C::RING - 1; ++j) wload(wr[j], j);
  __syncthreads();
  // step kt (R = kt % UNROLL, compile-time): issue token slice kt+D-1+XD,
  // then weight slice kt+RING-1; compute slice kt; store token slice kt+D
  // (issued XD-1 steps earlier) into the buffer slice kt+D-NB left, so the
  // newer slices stay in flight across the barrier.  One barrier every D
  // steps: it orders the stores of the D slices before it against their
  // reads D steps later, and the reads of the D slices before it against
  // the stores that reuse their buffers.
  auto step = [&](int kt, auto R) {
    constexpr int r = decltype(R)::value;
    constexpr int ws = r % C::RING;
    xload(xr[(r + C::D - 1 + C::XD) % C::XD], kt + C::D - 1 + C::XD);
    wload(wr[(ws + C::RING - 1) % C::RING], kt + C::RING - 1);
    __builtin_amdgcn_sched_barrier(0);
    const char* sb = sx[kt % C::NB] + fr * C::STRIDE + 16 * fg;
    // fragments of k-step s+1 are read from LDS while k-step s is multiplied
    uint4 fx[2][MT];
#pragma unroll
    for (int a = 0; a < MT; ++a) fx[0][a] = *reinterpret_cast<const uint4*>(sb + 32 * a * C::STRIDE);
    __builtin_amdgcn_sched_group_barrier(0x100, MT, 0);     // DS read
#pragma unroll
    for (int s = 0; s < C::KS; ++s) {
#pragma unroll
      for (int a = 0; a < MT; ++a) {
        if (s + 1 < C::KS)
          fx[(s + 1) & 1][a] = *reinterpret_cast<const uint4*>(sb + 32 * a * C::STRIDE + 32 * (s + 1));
#pragma unroll
        for (int j = 0; j < C::NA; ++j) acc[j][a] = mma32(acc[j][a], wr[ws][j][s], fx[s & 1][a]);
        if (s + 1 < C::KS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, C::NA, 0);   // MFMA
      }
    }
    xstore(xr[(r + C::D) % C::XD], (kt + C::D) % C::NB);
    if (r % C::D == C::D - 1) __syncthreads();
  };
  auto body = [&](int kt0, auto... R) { (step(kt0 + decltype(R)::value, R), ...); };
  auto tail = [&](int kt0, auto... R) {
    ((kt0 + decltype(R)::value < nk ? step(kt0 + decltype(R)::value, R) : void()), ...);
  };
  const int nmain = nk - nk % C::UNROLL;
  int kt = 0;
  [&]<int... I>(std::integer_sequence<int, I...>) {
    for (; kt < nmain; kt += C::UNROLL) body(kt, std::integral_constant<int, I>{}...);
    tail(kt, std::integral_constant<int, I>{}...);
  }(std::make_integer_sequence<int, C::UNROLL>{});
}

// The combine tile of a shared-expert down tile reuses the token LDS buffers:
// BM rows of BN bf16 outputs, rows padded by 16 bytes.
template <int BM, int BN>
constexpr int comb_ld() { return BN + 8; }

template <class C, bool kUp, bool kComb = false>
__device__ __forceinline__ void stream_tile(FfnProblem& p, char (&sx)[C::NB][C::LDS], Slot* slots) {
  static_assert(!kComb || C::BM * comb_ld<C::BM, C::BN>() * 2 <= C::NB * C::LDS,
                "the combine tile fits in the token buffers");
  TileInfo ti;
  const int32_t* sched = p.sched + (kUp ? 0 : kComb ? 2 : 1) * (p.E + 2);
  if (!find_tile(sched, p.offsets, p.E, p.ntok, C::BM, ti, kUp && C::BM == SHuge::BM)) return;
  static_assert(!kComb || C::BM <= C::THREADS, "one thread stages each token's slots");
  SlotLoad sl;                                      // the tokens' routing, loaded under the K loop
  if constexpr (kComb) slots_issue(p.comb, ti.m0, ti.mrows, sl);
  const bool shared = ti.g == p.E;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = kUp ? p.dim : (shared ? p.inter_s : p.inter);
  const int N = kUp ? (shared ? p.inter_s : p.inter) : p.dim;   // h columns / output columns
  const int m0 = ti.m0;
  const int rows_left = ti.mrows;

  StreamSrc<C> S;
  const int lc = tid % C::TPR, lr = tid / C::TPR;
#pragma unroll
  for (int i = 0; i < C::XLOADS; ++i) {
    const int tr = lr + C::ROWS_PER_PASS * i;
    S.xact[i] = tr < C::BM;
    const int m = m0 + min(tr, rows_left - 1);
    const uint16_t* row;
    if (kUp) {
      const int tok = shared ? m : p.sorted_token[ti.row0 + m];
      row = static_cast<const uint16_t*>(p.x) + (size_t)tok * K;
    } else {
      row = shared ? static_cast<const uint16_t*>(p.hs) + (size_t)m * K
                   : static_cast<const uint16_t*>(p.h) + (size_t)(ti.row0 + m) * K;
    }
    S.x[i] = reinterpret_cast<const char*>(row) + 16 * lc;
  }
  S.lds_st = lr * C::STRIDE + 16 * lc;

  const int fr = lane & 31, fg = lane >> 5;
  // weight tile j of the wave: up - h columns ncol[j] + [0,16), A rows 0-15
  // from W1 and 16-31 the same rows of W3; down - output columns ncol[j] + [0,32)
  int ncol[C::NA];
  bool tile_active[C::NA];
  bool wave_active = false;
#pragma unroll
  for (int j = 0; j < C::NA; ++j) {
    if (kUp) {
      ncol[j] = ti.nt * C::UPBN + (wave * C::NA + j) * 16;
      const int n = min(ncol[j] + (fr & 15), N - 1);
      const uint16_t* W = fr < 16 ? (shared ? static_cast<const uint16_t*>(p.ws1)
                                            : static_cast<const uint16_t*>(p.w1) + (size_t)(ti.g - p.e_begin) * N * K)
                                  : (shared ? static_cast<const uint16_t*>(p.ws3)
                                            : static_cast<const uint16_t*>(p.w3) + (size_t)(ti.g - p.e_begin) * N * K);
      S.w[j] = reinterpret_cast<const char*>(W) + wtile_off(n, 16 * fg, 2 * K);
    } else {
      ncol[j] = ti.nt * C::BN + (wave * C::NA + j) * 32;
      const uint16_t* W2 = shared ? static_cast<const uint16_t*>(p.ws2)
                                  : static_cast<const uint16_t*>(p.w2) + (size_t)(ti.g - p.e_begin) * N * K;
      S.w[j] = reinterpret_cast<const char*>(W2) + wtile_off(min(ncol[j] + fr, N - 1), 16 * fg, 2 * K);
    }
    tile_active[j] = ncol[j] < N;
    wave_active = wave_active || tile_active[j];
  }
  // every wave runs the same instantiation: the token slices are loaded by
  // all threads of the workgroup (a weight tile past the last column computes
  // on a clamped weight row and stores nothing)
  int m_active = (rows_left + 31) >> 5;
  m_active = m_active > C::MT ? C::MT : m_active;

  f32x16_t acc[C::NA][C::MT];
#pragma unroll
  for (int j = 0; j < C::NA; ++j)
#pragma unroll
    for (int a = 0; a < C::MT; ++a)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[j][a][i] = 0.f;

  const int nk = K / C::BK;
  // the K loop is instantiated for every sub-tile count, so no MFMA or token
  // load is spent on 32-row sub-tiles past the tile's last row
  // In the 128 x 512 up tiles a routed expert of one m-tile reads each
  // weight slice exactly once, so its weights go through non-temporal loads;
  // experts of several m-tiles share the slices through L2 and keep ordinary
  // loads (per tile: c2 up 3.18 -> 3.15 ms; for every tile it was slower)
  constexpr bool kNtSingle = kUp && std::is_same_v<C, SBigUp>;
  if (kNtSingle && ti.g < p.E && ti.M <= C::BM) {
    [&]<int... I>(std::integer_sequence<int, I...>) {
      ((m_active == I + 1 ? stream_kloop<C, I + 1, true>(sx, S, nk, acc) : void()), ...);
    }(std::make_integer_sequence<int, C::MT>{});
  } else {
    [&]<int... I>(std::integer_sequence<int, I...>) {
      ((m_active == I + 1 ? stream_kloop<C, I + 1>(sx, S, nk, acc) : void()), ...);
    }(std::make_integer_sequence<int, C::MT>{});
  }
  if constexpr (kComb) {
    constexpr int LD = comb_ld<C::BM, C::BN>();
    uint16_t* st = reinterpret_cast<uint16_t*>(&sx[0][0]);
    slots_store(p.comb, rows_left, sl, slots);
    __syncthreads();                  // every wave is done with the token buffers
    const int ml = lane & 31, rg = 4 * (lane >> 5);
#pragma unroll
    for (int j = 0; j < C::NA; ++j) {
      if (!tile_active[j]) continue;
#pragma unroll
      for (int a = 0; a < C::MT; ++a) {
        const int r = 32 * a + ml;
        if (a >= m_active || r >= rows_left) continue;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          uint2 o;
          o.x = (uint32_t)f32_to_bf16(acc[j][a][4 * q]) | ((uint32_t)f32_to_bf16(acc[j][a][4 * q + 1]) << 16);
          o.y = (uint32_t)f32_to_bf16(acc[j][a][4 * q + 2]) | ((uint32_t)f32_to_bf16(acc[j][a][4 * q + 3]) << 16);
          *reinterpret_cast<uint2*>(st + r * LD + (wave * C::NA + j) * 32 + 8 * q + rg) = o;
        }
      }
    }
    __syncthreads();
    combine_from_lds<uint16_t, 4>(p, slots, st, LD, ti, ti.nt * C::BN, C::BN);
    return;
  }
  if (!wave_active) return;

  // epilogue: lane holds D[row = 8*(i/4) + 4*(lane/32) + i%4][col = lane % 32]
  // (row = weight row of the tile, col = token of the sub-tile)
  const int ml = lane & 31, rg = 4 * (lane >> 5);
#pragma unroll
  for (int j = 0; j < C::NA; ++j) {
    if (!tile_active[j]) continue;
#pragma unroll
    for (int a = 0; a < C::MT; ++a) {
      const int m = m0 + 32 * a + ml;
      if (a >= m_active || m >= m0 + rows_left) continue;
      if (kUp) {
        uint16_t* hrow = shared ? static_cast<uint16_t*>(p.hs) + (size_t)m * N
                                : static_cast<uint16_t*>(p.h) + (size_t)(ti.row0 + m) * N;
#pragma unroll
        for (int q = 0; q < 2; ++q) {       // rows 8q + rg + [0,4) of W1, 16 + same of W3
          float v[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = silu(acc[j][a][4 * q + i]) * acc[j][a][8 + 4 * q + i];
          store4<uint16_t>(hrow + ncol[j] + 8 * q + rg, v);
        }
      } else {
        uint16_t* orow = shared ? static_cast<uint16_t*>(p.shared_out) + (size_t)m * N
                                : static_cast<uint16_t*>(p.out) + (size_t)(ti.row0 + m) * N;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float v[4] = {acc[j][a][4 * q], acc[j][a][4 * q + 1], acc[j][a][4 * q + 2], acc[j][a][4 * q + 3]};
          store4<uint16_t>(orow + ncol[j] + 8 * q + rg, v);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// fp8 stream tiles (prefill), 192 tokens: the bf16 stream-tile layout (8 waves x 32
// weight rows, W1 rows 0-15 and the same W3 rows 16-31 in one A tile, 32-row
// token sub-tiles from LDS) on v_mfma_scale_f32_32x32x64_f8f6f4 - A lane l:
// row l%32, bytes 32*(l/32)..+31 of a 64-byte K half; B likewise for the token
// row; D as the bf16 32x32 tile, so D elements i < 8 are W1 rows (or the
// first 16 W2 rows) and i >= 8 the W3 rows.  Two MFMAs per 128-wide K block.
// Block scales ("promotion"): each block's two MFMAs go into a fresh partial
// product P, then acc += s * P with s = w_scale * a_scale (one s per half of
// the elements): sum_kb s_kb * (W_kb X_kb) in fp32, with no reciprocal, so a
// zero or tiny scale stays exact and nothing overflows.  P is double-buffered
// across sub-tiles: the promotion of sub-tile a-1 is issued after the MFMAs
// of sub-tile a, so it never waits for them.  Token slices carry their
// per-row activation scale into LDS.  The 32-row fragment pattern reads LDS without
// bank conflicts (a 16x16x128 pattern conflicts on half its cycles), and 192
// tokens cover most experts of an 8192-token batch in two m-tiles.  The up
// epilogue quantises h per 1x128 block: the 8 waves' 16-column slices of a
// token row form exactly one block, so the amax is reduced across waves in LDS.
// ---------------------------------------------------------------------------
using F8 = SCfg<192, 8, 3, 1>;   // 192 tokens, 8 waves x 32 weight rows, a weight ring of 3
constexpr int kF8MT = F8::BM / 32;

struct StreamSrcF8 {
  const char* x[F8::XLOADS];    // token rows (tid / 8) + 64*i, byte 16*(tid % 8) of the 128-byte block
  const float* xs[F8::XLOADS];  // their activation scales, [row][K/128]
  const char* w;                 // this lane's weight row (tiled layout) at bytes 32*(lane/32) of a K half
  const float* ws[2];            // block scales of the rows of D elements i < 8 and i >= 8, [K/128]
  int lds_st;
  bool xact[F8::XLOADS];
};

template <int MT, bool kNT>
__device__ __forceinline__ void stream_fp8_kloop(char (&sx)[F8::NB][F8::LDS], float (&sxs)[F8::NB][F8::BM],
                                                  const StreamSrcF8& S, int nk,
                                                  f32x16_t (&acc)[kF8MT]) {
  constexpr int XL = std::min(F8::XLOADS, (32 * MT + F8::ROWS_PER_PASS - 1) / F8::ROWS_PER_PASS);
  constexpr int RING = F8::RING;
  constexpr int XD = F8::XD, NB = F8::NB, D = F8::D;
  constexpr int UNROLL = F8::UNROLL;
  const int lane = threadIdx.x & 63, fr = lane & 31, fg = lane >> 5;
  i32x8_t_ wr[RING][2];          // [slice % RING][K half]
  float wsc[RING][2];            // [slice % RING][D half]
  uint4 xr[XD][F8::XLOADS];      // token slices between load and LDS store: [slice % XD]
  float xsr[XD][F8::XLOADS];
  auto wload = [&](i32x8_t_ (&dst)[2], float (&sc)[2], int kt) {
    kt = kt < nk ? kt : nk - 1;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const char* a = S.w + kt * (2 * kChunkStride) + j * kChunkStride;
      const uint4 lo = kNT ? ldg16_stream(a) : ldg16(a);
      const uint4 hi = kNT ? ldg16_stream(a + 256) : ldg16(a + 256);
      dst[j] = i32x8_t_{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      sc[j] = S.ws[j][kt];
    }
  };
  auto xload = [&](uint4 (&dst)[F8::XLOADS], float (&sc)[F8::XLOADS], int kt) {
    kt = kt < nk ? kt : nk - 1;
#pragma unroll
    for (int i = 0; i < XL; ++i) {
      dst[i] = ldg16(S.x[i] + kt * 128);
      sc[i] = S.xs[i][kt];       // the 8 lanes of a row load the same scale
    }
  };
  auto xstore = [&](const uint4 (&src)[F8::XLOADS], const float (&sc)[F8::XLOADS], int buf) {
#pragma unroll
    for (int i = 0; i < XL; ++i) {
      static_assert(F8::BM % F8::ROWS_PER_PASS == 0, "every token load pass lands inside the tile");
      *reinterpret_cast<uint4*>(&sx[buf][S.lds_st + F8::ROWS_PER_PASS * i * F8::STRIDE]) = src[i];
      sxs[buf][(threadIdx.x >> 3) + F8::ROWS_PER_PASS * i] = sc[i];   // equal values from the row's 8 lanes
    }
  };
  // Token slice j lives in LDS buffer j % NB; slice kt+D is stored after step
  // kt, one barrier every D steps (the staging of the bf16 stream loop).
  // Order of issue: a step issues its weight slice first, computes, stores
  // the token slice issued at the end of the step before and issues the next
  // one last, ahead of the barrier.  A token slice is thus in flight for a
  // whole step plus the barrier wait (issued after the barrier, it had only
  // the step), weight slices for RING-1 = 2 steps; memory counters retire in
  // issue order, so the store's wait covers only loads issued before it.
#pragma unroll
  for (int j = 0; j < D; ++j) {
    xload(xr[j % XD], xsr[j % XD], j);
    xstore(xr[j % XD], xsr[j % XD], j);
  }
#pragma unroll
  for (int j = 0; j < RING - 1; ++j) wload(wr[j], wsc[j], j);
#pragma unroll
  for (int j = D; j < D + XD; ++j) xload(xr[j % XD], xsr[j % XD], j);
  __syncthreads();
  auto step = [&](int kt, auto R) {
    constexpr int r = decltype(R)::value;
    constexpr int ws = r % RING;
    wload(wr[(ws + RING - 1) % RING], wsc[(ws + RING - 1) % RING], kt + RING - 1);
    __builtin_amdgcn_sched_barrier(0);
    const char* sb = sx[kt % NB] + fr * F8::STRIDE + 32 * fg;
    const float* sbs = sxs[kt % NB] + fr;
    // the fragments and scale of sub-tile a are read from LDS just before its
    // MFMAs (one buffer: the registers went to the weight ring; the other wave
    // of the SIMD covers the read latency); the promotion of sub-tile a-1
    // follows the MFMAs of sub-tile a, so it never waits for them
    i32x8_t_ bx[2];
    f32x16_t part[2];              // partial products of the block, sub-tiles a-1 and a
    // acc += s * partial with s = w_scale * a_scale, one s per half of D
    auto promote = [&](int a, float as) {
      const float s0 = wsc[ws][0] * as, s1 = wsc[ws][1] * as;
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][i] = fmaf(part[a & 1][i], i < 8 ? s0 : s1, acc[a][i]);
    };
    float as_prev = 0.f;
#pragma unroll
    for (int a = 0; a < MT; ++a) {
#pragma unroll
      for (int j = 0; j < 2; ++j) bx[j] = *reinterpret_cast<const i32x8_t_*>(sb + 32 * a * F8::STRIDE + 64 * j);
      const float as = sbs[32 * a];
      __builtin_amdgcn_sched_barrier(0);
      const f32x16_t zero = {};
      f32x16_t c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wr[ws][0], bx[0], zero, 0, 0, 0, 127, 0, 127);
      part[a & 1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wr[ws][1], bx[1], c, 0, 0, 0, 127, 0, 127);
      if (a > 0) promote(a - 1, as_prev);
      as_prev = as;
      __builtin_amdgcn_sched_barrier(0);
    }
    promote(MT - 1, as_prev);
    xstore(xr[(r + D) % XD], xsr[(r + D) % XD], (kt + D) % NB);
    xload(xr[(r + D) % XD], xsr[(r + D) % XD], kt + D + XD);
    if (r % D == D - 1) __syncthreads();
  };
  auto body = [&](int kt0, auto... R) { (step(kt0 + decltype(R)::value, R), ...); };
  auto tail = [&](int kt0, auto... R) {
    ((kt0 + decltype(R)::value < nk ? step(kt0 + decltype(R)::value, R) : void()), ...);
  };
  const int nmain = nk - nk % UNROLL;
  int kt = 0;
  [&]<int... I>(std::integer_sequence<int, I...>) {
    for (; kt < nmain; kt += UNROLL) body(kt, std::integral_constant<int, I>{}...);
    tail(kt, std::integral_constant<int, I>{}...);
  }(std::make_integer_sequence<int, UNROLL>{});
}

template <bool kUp, bool kNT, bool kComb = false>
__global__ __launch_bounds__(512, 1) __attribute__((amdgpu_waves_per_eu(2, 2)))
void stream_fp8_kernel(FfnProblem p) {
  __shared__ __attribute__((aligned(16))) char sx[F8::NB][F8::LDS];
  __shared__ float sxs[F8::NB][F8::BM];
  __shared__ float wamax[kUp ? F8::WAVES : 1][F8::BM];
  __shared__ __attribute__((aligned(16))) Slot slots[kComb ? F8::BM * kRegSlots : 1];
  static_assert(!kComb || F8::BM * comb_ld<F8::BM, F8::BN>() * 2 <= F8::NB * F8::LDS,
                "the combine tile fits in the token buffers");
  static_assert(!kComb || F8::BM <= F8::THREADS, "one thread stages each token's slots");
  TileInfo ti;
  const int32_t* sched = p.sched + (kUp ? 0 : kComb ? 2 : 1) * (p.E + 2);
  if (!find_tile(sched, p.offsets, p.E, p.ntok, F8::BM, ti, kUp)) return;
  const bool shared = ti.g == p.E;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = kUp ? p.dim : (shared ? p.inter_s : p.inter), KB = K / 128;
  const int N = kUp ? (shared ? p.inter_s : p.inter) : p.dim;
  const int m0 = ti.m0;
  const int rows_left = ti.mrows;

  StreamSrcF8 S;
  const int lc = tid & 7, lr = tid >> 3;
#pragma unroll
  for (int i = 0; i < F8::XLOADS; ++i) {
    const int tr = lr + F8::ROWS_PER_PASS * i;
    S.xact[i] = tr < F8::BM;
    const int m = m0 + min(tr, rows_left - 1);
    size_t row;
    const uint8_t* base;
    const float* sbase;
    if (kUp) {
      row = shared ? (size_t)m : (size_t)p.sorted_token[ti.row0 + m];
      base = p.xq;
      sbase = p.xs;
    } else {
      row = shared ? (size_t)m : (size_t)(ti.row0 + m);
      base = static_cast<const uint8_t*>(shared ? p.hs : p.h);
      sbase = shared ? p.hsscale : p.hscale;
    }
    S.x[i] = reinterpret_cast<const char*>(base + row * K) + 16 * lc;
    S.xs[i] = sbase + row * KB;
  }
  S.lds_st = lr * F8::STRIDE + 16 * lc;

  const int fr = lane & 31, fg = lane >> 5;
  int ncol0;                      // up: first h column of the wave; down: first output column
  if (kUp) {
    // A rows 0-15: W1 rows ncol0 + [0,16); rows 16-31: the same rows of W3
    ncol0 = ti.nt * F8::UPBN + wave * 16;          // N % 128 == 0: always inside
    const size_t eoff = shared ? 0 : (size_t)(ti.g - p.e_begin) * N * K;
    const size_t soff = shared ? 0 : (size_t)(ti.g - p.e_begin) * (N / 128) * KB;
    const uint8_t* W = static_cast<const uint8_t*>(fr < 16 ? (shared ? p.ws1 : p.w1) : (shared ? p.ws3 : p.w3)) + eoff;
    S.w = reinterpret_cast<const char*>(W) + wtile_off(ncol0 + (fr & 15), 32 * fg, K);
    S.ws[0] = (shared ? p.ws1s : p.w1s) + soff + (size_t)(ncol0 / 128) * KB;
    S.ws[1] = (shared ? p.ws3s : p.w3s) + soff + (size_t)(ncol0 / 128) * KB;
  } else {
    ncol0 = ti.nt * F8::BN + wave * 32;
    const int nrow = min(ncol0, N - 32);            // N % 128 == 0: a wave is all in or all out
    const uint8_t* W2 = static_cast<const uint8_t*>(shared ? p.ws2 : p.w2) + (shared ? 0 : (size_t)(ti.g - p.e_begin) * N * K);
    const float* W2s = (shared ? p.ws2s : p.w2s + (size_t)(ti.g - p.e_begin) * (N / 128) * KB) + (size_t)(nrow / 128) * KB;
    S.w = reinterpret_cast<const char*>(W2) + wtile_off(nrow + fr, 32 * fg, K);
    S.ws[0] = S.ws[1] = W2s;                        // 32 rows inside one 128-row block
  }
  const bool wave_active = ncol0 < N;
  int m_active = (rows_left + 31) >> 5;
  m_active = m_active > kF8MT ? kF8MT : m_active;   // the same for every wave

  f32x16_t acc[kF8MT];
#pragma unroll
  for (int a = 0; a < kF8MT; ++a)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[a][i] = 0.f;
  [&]<int... I>(std::integer_sequence<int, I...>) {
    ((m_active == I + 1 ? stream_fp8_kloop<I + 1, kNT>(sx, sxs, S, KB, acc) : void()), ...);
  }(std::make_integer_sequence<int, kF8MT>{});

  // D[row = 8*(i/4) + 4*(lane/32) + i%4][col = lane % 32]
  const int ml = lane & 31, rg = 4 * (lane >> 5);
  if (kUp) {
    // h = silu(a1) * a3 for h columns ncol0 + 8q + rg + i; the 8 waves' 16 columns
    // of a token row form one 1x128 block, so its amax is reduced across waves
#pragma unroll
    for (int a = 0; a < kF8MT; ++a) {
      float am = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {   // h replaces the W1 half of the accumulator
        acc[a][i] = silu(acc[a][i]) * acc[a][8 + i];
        am = fmaxf(am, fabsf(acc[a][i]));
      }
      am = fmaxf(am, __shfl_xor(am, 32, kWave));
      if (fg == 0) wamax[wave][32 * a + ml] = am;
    }
    __syncthreads();
#pragma unroll
    for (int a = 0; a < kF8MT; ++a) {
      const int m = m0 + 32 * a + ml;
      if (a >= m_active || m >= m0 + rows_left) continue;
      float am = 0.f;
#pragma unroll
      for (int w = 0; w < F8::WAVES; ++w) am = fmaxf(am, wamax[w][32 * a + ml]);
      const float scale = am > 0.f ? __fdiv_rn(am, 448.0f) : 1.0f;
      const size_t row = shared ? (size_t)m : (size_t)(ti.row0 + m);
      uint8_t* hq = static_cast<uint8_t*>(shared ? p.hs : p.h) + row * N;
#pragma unroll
      for (int q = 0; q < 2; ++q) {   // rows 8q + rg + [0,4) of W1, 16 + the same of W3
        uint32_t pk = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          pk |= (uint32_t)f32_to_e4m3(__fdiv_rn(acc[a][4 * q + i], scale)) << (8 * i);
        *reinterpret_cast<uint32_t*>(hq + ncol0 + 8 * q + rg) = pk;
      }
      if (wave == 0 && fg == 0) (shared ? p.hsscale : p.hscale)[row * (N / 128) + ti.nt] = scale;
    }
  } else if constexpr (kComb) {
    constexpr int LD = comb_ld<F8::BM, F8::BN>();
    uint16_t* st = reinterpret_cast<uint16_t*>(&sx[0][0]);
    {
      // the tokens' routing (loaded here: the K loop has no registers to spare)
      SlotLoad sl;
      slots_issue(p.comb, ti.m0, ti.mrows, sl);
      slots_store(p.comb, ti.mrows, sl, slots);
    }
    __syncthreads();                  // every wave is done with the token buffers
    if (wave_active) {
#pragma unroll
      for (int a = 0; a < kF8MT; ++a) {
        const int r = 32 * a + ml;
        if (a >= m_active || r >= rows_left) continue;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          uint2 o;
          o.x = (uint32_t)f32_to_bf16(acc[a][4 * q]) | ((uint32_t)f32_to_bf16(acc[a][4 * q + 1]) << 16);
          o.y = (uint32_t)f32_to_bf16(acc[a][4 * q + 2]) | ((uint32_t)f32_to_bf16(acc[a][4 * q + 3]) << 16);
          *reinterpret_cast<uint2*>(st + r * LD + wave * 32 + 8 * q + rg) = o;
        }
      }
    }
    __syncthreads();
    combine_from_lds<uint16_t, 4>(p, slots, st, LD, ti, ti.nt * F8::BN, F8::BN);
  } else {
    if (!wave_active) return;
#pragma unroll
    for (int a = 0; a < kF8MT; ++a) {
      const int m = m0 + 32 * a + ml;
      if (a >= m_active || m >= m0 + rows_left) continue;
      uint16_t* orow = static_cast<uint16_t*>(shared ? p.shared_out : p.out) +
                       (shared ? (size_t)m : (size_t)(ti.row0 + m)) * N;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float v[4] = {acc[a][4 * q], acc[a][4 * q + 1], acc[a][4 * q + 2], acc[a][4 * q + 3]};
        store4<uint16_t>(orow + ncol0 + 8 * q + rg, v);
      }
    }
  }
}

template <class C, bool kUp, bool kComb = false>
__global__ __launch_bounds__(C::THREADS) __attribute__((amdgpu_waves_per_eu(C::WPE, C::WPE)))
void stream_bf16_kernel(FfnProblem p) {
  __shared__ __attribute__((aligned(16))) char sx[C::NB][C::LDS];
  __shared__ __attribute__((aligned(16))) Slot slots[kComb ? C::BM * kRegSlots : 1];
  stream_tile<C, kUp, kComb>(p, sx, slots);
}

// ---------------------------------------------------------------------------
// fp8 experts (OCP e4m3fn weights with one fp32 scale per 128x128 block;
// activations quantised per 1x128 block).  One v_mfma 16x16x128 f8f6f4 covers
// exactly one 128-wide K block, so each block's partial product is formed in
// a fresh accumulator and added to the fp32 result times
// w_scale[n/128][kb] * a_scale[m][kb] ("promotion"): the scales never enter
// the MFMA.  A operand: lane l holds row l%16, bytes 32*(l/16) .. +31 of the
// K block; B operand likewise for the token row; result D[4*(l/16)+i][l%16].
// ---------------------------------------------------------------------------

__device__ __forceinline__ f32x4_t mma_fp8(uint4 a0, uint4 a1, uint4 b0, uint4 b1) {
  i32x8_t_ a = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
  i32x8_t_ b = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
  const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
  // formats 0/0 = e4m3 for both operands; scale exponents 127 = 2^0 (no MX scaling)
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, z, 0, 0, 0, 127, 0, 127);
}

// Activation quantiser: rows of `cols` bf16 -> e4m3 codes + one fp32 scale
// per 1x128 block.  scale = amax / 448 (1 when amax = 0); code =
// e4m3(v / scale), IEEE division, round to nearest even, saturating.
// 16 threads per block, 8 elements each.
__global__ __launch_bounds__(256) void quant_fp8_kernel(const uint16_t* __restrict__ x, long rows,
                                                        int cols, uint8_t* __restrict__ q,
                                                        float* __restrict__ sc) {
  const long nblk = rows * (cols / 128);
  const long blk = ((long)blockIdx.x * blockDim.x + threadIdx.x) >> 4;
  const int sub = threadIdx.x & 15;
  const bool ok = blk < nblk;
  const long b = ok ? blk : nblk - 1;
  const long r = b / (cols / 128), cb = b % (cols / 128);
  const uint16_t* src = x + r * cols + cb * 128 + sub * 8;
  const uint4 u = *reinterpret_cast<const uint4*>(src);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
  float v[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) { v[2 * i] = __uint_as_float(w[i] << 16); v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u); }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o, kWave));
  const float scale = amax > 0.f ? __fdiv_rn(amax, 448.0f) : 1.0f;
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) lo |= (uint32_t)f32_to_e4m3(__fdiv_rn(v[i], scale)) << (8 * i);
#pragma unroll
  for (int i = 0; i < 4; ++i) hi |= (uint32_t)f32_to_e4m3(__fdiv_rn(v[4 + i], scale)) << (8 * i);
  if (ok) {
    *reinterpret_cast<uint2*>(q + r * cols + cb * 128 + sub * 8) = make_uint2(lo, hi);
    if (sub == 0) sc[r * (cols / 128) + cb] = scale;
  }
}

// Up projection, fp8, skinny tiles (16 tokens x 128 h columns per workgroup,
// i.e. one 1x128 h quantisation block per token row).  Wave w owns h columns
// [32w, 32w+32) of the tile: W1 sub-tiles j=0,1 and W3 sub-tiles j=2,3.
__global__ __launch_bounds__(256) void up_skinny_fp8_kernel(FfnProblem p) {
  __shared__ float wamax[kSkinnyWaves][16];
  TileInfo ti;
  if (!find_tile(p.sched, p.offsets, p.E, p.ntok, 16, ti)) return;
  const bool shared = ti.g == p.E;
  const int N = shared ? p.inter_s : p.inter;
  const int K = p.dim, KB = K / 128;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, grp = lane >> 4;
  const int nbase = ti.nt * 128 + wave * 32;          // N % 128 == 0: always inside
  const int mi = ti.m0 + min(r, ti.mrows - 1);
  const int tok = shared ? mi : p.sorted_token[ti.row0 + mi];
  const char* bp = reinterpret_cast<const char*>(p.xq + (size_t)tok * K) + 32 * grp;
  const float* bsc = p.xs + (size_t)tok * KB;
  const uint8_t* W1 = static_cast<const uint8_t*>(shared ? p.ws1 : p.w1) + (shared ? 0 : (size_t)(ti.g - p.e_begin) * N * K);
  const uint8_t* W3 = static_cast<const uint8_t*>(shared ? p.ws3 : p.w3) + (shared ? 0 : (size_t)(ti.g - p.e_begin) * N * K);
  const float* S1 = (shared ? p.ws1s : p.w1s + (size_t)(ti.g - p.e_begin) * (N / 128) * KB) + (size_t)(nbase / 128) * KB;
  const float* S3 = (shared ? p.ws3s : p.w3s + (size_t)(ti.g - p.e_begin) * (N / 128) * KB) + (size_t)(nbase / 128) * KB;
  const char* ap[4];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    ap[j] = reinterpret_cast<const char*>(W1) + wtile_off(nbase + 16 * j + r, 32 * grp, K);
    ap[j + 2] = reinterpret_cast<const char*>(W3) + wtile_off(nbase + 16 * j + r, 32 * grp, K);
  }
  f32x4_t acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  uint4 a[2][4][2], b[2][2];
  auto load = [&](int s, int kb) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      a[s][j][0] = ldg16_stream(ap[j] + 2 * kChunkStride * kb);
      a[s][j][1] = ldg16_stream(ap[j] + 2 * kChunkStride * kb + 256);
    }
    b[s][0] = ldg16(bp + 128 * kb);
    b[s][1] = ldg16(bp + 128 * kb + 16);
  };
  auto comp = [&](int s, int kb) {
    const float xsc = bsc[kb];
    const float s1 = S1[kb] * xsc, s3 = S3[kb] * xsc;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4_t part = mma_fp8(a[s][j][0], a[s][j][1], b[s][0], b[s][1]);
      const float sc = j < 2 ? s1 : s3;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[j][i] = fmaf(part[i], sc, acc[j][i]);
    }
  };
  load(0, 0);
  for (int kb = 0; kb < KB; kb += 2) {
    if (kb + 1 < KB) load(1, kb + 1);
    comp(0, kb);
    if (kb + 2 < KB) load(0, kb + 2);
    if (kb + 1 < KB) comp(1, kb + 1);
  }
  // note: bsc is indexed per lane (token of column r); the promotion factor
  // is per (token, K block) x per (128-row weight block, K block)
  // h = silu(a1) * a3 for h columns nbase + 16j + 4*grp + i, token column r
  float h[2][4];
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) { h[j][i] = silu(acc[j][i]) * acc[j + 2][i]; amax = fmaxf(amax, fabsf(h[j][i])); }
  amax = fmaxf(amax, __shfl_xor(amax, 16, kWave));
  amax = fmaxf(amax, __shfl_xor(amax, 32, kWave));
  if (grp == 0) wamax[wave][r] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(wamax[0][r], wamax[1][r]), fmaxf(wamax[2][r], wamax[3][r]));
  const float scale = amax > 0.f ? __fdiv_rn(amax, 448.0f) : 1.0f;
  const int m = ti.m0 + r;
  if (r < ti.mrows) {
    const size_t row = shared ? (size_t)m : (size_t)(ti.row0 + m);
    uint8_t* hq = static_cast<uint8_t*>(shared ? p.hs : p.h) + row * N;
    float* hsc = (shared ? p.hsscale : p.hscale) + row * (N / 128);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      uint32_t pk = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) pk |= (uint32_t)f32_to_e4m3(__fdiv_rn(h[j][i], scale)) << (8 * i);
      *reinterpret_cast<uint32_t*>(hq + nbase + 16 * j + 4 * grp) = pk;
    }
    if (wave == 0 && grp == 0) hsc[ti.nt] = scale;
  }
}

// Down projection, fp8, skinny tiles: 16 tokens x 256 output columns
// (kComb: the shared expert's tiles, ending with the fused combine).
template <bool kComb>
__global__ __launch_bounds__(256) void down_skinny_fp8_kernel(FfnProblem p) {
  constexpr int LD = kDnBN8 + 8;                    // LDS row of the combine tile (elements)
  __shared__ __attribute__((aligned(16))) uint16_t s_tile[kComb ? 16 * LD : 1];
  __shared__ __attribute__((aligned(16))) Slot slots[kComb ? 16 * kRegSlots : 1];
  TileInfo ti;
  const int32_t* sched = p.sched + (kComb ? 2 : 1) * (p.E + 2);
  if (!find_tile(sched, p.offsets, p.E, p.ntok, 16, ti)) return;
  SlotLoad sl;                                      // the tokens' routing, loaded under the K loop
  if constexpr (kComb) slots_issue(p.comb, ti.m0, ti.mrows, sl);
  const bool shared = ti.g == p.E;
  const int K = shared ? p.inter_s : p.inter, KB = K / 128;
  const int N = p.dim;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, grp = lane >> 4;
  const int nbase = ti.nt * kDnBN8 + wave * 16 * kDnNT8;
  if (!kComb && nbase >= N) return;
  const bool active = nbase < N;                    // waves past the last column still meet the barrier
  const int mi = ti.m0 + min(r, ti.mrows - 1);
  const size_t hrow = shared ? (size_t)mi : (size_t)(ti.row0 + mi);
  const char* bp = reinterpret_cast<const char*>(static_cast<const uint8_t*>(shared ? p.hs : p.h) + hrow * K) + 32 * grp;
  const float* bsc = (shared ? p.hsscale : p.hscale) + hrow * KB;
  const uint8_t* W2 = static_cast<const uint8_t*>(shared ? p.ws2 : p.w2) + (shared ? 0 : (size_t)(ti.g - p.e_begin) * N * K);
  const float* S2 = (shared ? p.ws2s : p.w2s + (size_t)(ti.g - p.e_begin) * (N / 128) * KB);
  const char* ap[kDnNT8];
  const float* sp[kDnNT8];
#pragma unroll
  for (int j = 0; j < kDnNT8; ++j) {
    const int n = min(nbase + 16 * j, N - 16);
    ap[j] = reinterpret_cast<const char*>(W2) + wtile_off(n + r, 32 * grp, K);
    sp[j] = S2 + (size_t)(n / 128) * KB;
  }
  f32x4_t acc[kDnNT8];
#pragma unroll
  for (int j = 0; j < kDnNT8; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  uint4 a[2][kDnNT8][2], b[2][2];
  auto load = [&](int s, int kb) {
#pragma unroll
    for (int j = 0; j < kDnNT8; ++j) {
      a[s][j][0] = ldg16_stream(ap[j] + 2 * kChunkStride * kb);
      a[s][j][1] = ldg16_stream(ap[j] + 2 * kChunkStride * kb + 256);
    }
    b[s][0] = ldg16(bp + 128 * kb);
    b[s][1] = ldg16(bp + 128 * kb + 16);
  };
  auto comp = [&](int s, int kb) {
    const float hsc = bsc[kb];
#pragma unroll
    for (int j = 0; j < kDnNT8; ++j) {
      const f32x4_t part = mma_fp8(a[s][j][0], a[s][j][1], b[s][0], b[s][1]);
      const float sc = sp[j][kb] * hsc;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[j][i] = fmaf(part[i], sc, acc[j][i]);
    }
  };
  if (active) {
    load(0, 0);
    for (int kb = 0; kb < KB; kb += 2) {
      if (kb + 1 < KB) load(1, kb + 1);
      comp(0, kb);
      if (kb + 2 < KB) load(0, kb + 2);
      if (kb + 1 < KB) comp(1, kb + 1);
    }
  }
  const int m = ti.m0 + r;
  if constexpr (kComb) {
    if (active && r < ti.mrows) {
#pragma unroll
      for (int j = 0; j < kDnNT8; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          s_tile[r * LD + wave * 16 * kDnNT8 + 16 * j + 4 * grp + i] = f32_to_bf16(acc[j][i]);
    }
    slots_store(p.comb, ti.mrows, sl, slots);
    __syncthreads();
    combine_from_lds<uint16_t, 2>(p, slots, s_tile, LD, ti, ti.nt * kDnBN8, kDnBN8);
    return;
  }
  if (r < ti.mrows) {
    uint16_t* orow = static_cast<uint16_t*>(shared ? p.shared_out : p.out) + (shared ? (size_t)m : (size_t)(ti.row0 + m)) * N;
#pragma unroll
    for (int j = 0; j < kDnNT8; ++j) {
      float v[4] = {acc[j][0], acc[j][1], acc[j][2], acc[j][3]};
      store4<uint16_t>(orow + nbase + 16 * j + 4 * grp, v);
    }
  }
}

static inline int ceil_div(long a, long b) { return (int)((a + b - 1) / b); }

// Upper bound on the tiles of one projection: sum_g ceil(M_g / bm) <= R/bm + nonempty groups.
static long max_tiles(long R, int E, int ntok, bool shared, int bm, int nt_routed, int nt_shared) {
  long routed_m = R / bm + std::min<long>(E, R) + 1;
  long t = routed_m * nt_routed;
  if (shared) t += (long)ceil_div(ntok, bm) * nt_shared;
  return t;
}

size_t ffn_h_bytes(int ntok, int topk, int inter, int inter_s, WKind wk, bool act_f32) {
  const size_t esz = wk == WKind::FP8 ? 1 : (act_f32 ? 4 : 2);
  return ((size_t)ntok * topk * inter + (size_t)ntok * inter_s) * esz;
}

enum class Tiles { Skinny, Mid, Big, Huge };

// Tile shape for a batch, on the average rows per expert R / E (thresholds
// from batch-size sweeps on the DeepSeek-V3 shape): 16-token skinny tiles
// below 8 rows (decode: weight streaming, each expert's weights read once);
// from there every 16-token m-tile would re-read its expert's weights, so
// stream tiles take over - 64-token tiles below 32 rows, 128-token tiles
// below 64, whole-expert tiles up to 384 rows (128 x 512 up tiles, 192 x 256
// down tiles), 256-token tiles above
// (hot experts of many hundred rows).  fp8 weights switch to their 192-token
// stream tiles from 12 rows.  Stream tiles need widths that are multiples of 64.
static Tiles pick_tiles(const FfnProblem& p, bool has_shared) {
  const long R = (long)p.ntok * p.topk;
  if (p.wkind == WKind::FP8) return R >= 12L * p.E ? Tiles::Big : Tiles::Skinny;
  if (p.wkind != WKind::BF16) return Tiles::Skinny;
  if (p.dim % 64 || p.inter % 64 || (has_shared && p.inter_s % 64)) return Tiles::Skinny;
  if (R >= 384L * p.E) return Tiles::Huge;
  if (R >= 32L * p.E) return Tiles::Big;
  if (R >= 8L * p.E) return Tiles::Mid;
  return Tiles::Skinny;
}

// Tile kind, tile sizes and grid sizes of the projection launches.
struct FfnPlan {
  Tiles t;
  bool nt;              // stream tiles read their weights non-temporally
  int bm, threads;            // tile rows and threads of the up launch
  int nt_up, nt_up_s;         // its n-tiles per routed expert and for the shared expert
  int bm_dn, threads_dn, nt_dn;   // the down launch
  int bm_s, threads_s, nt_dn_s;   // the shared down + combine launch
  long g_up, g_dn, g_dn_s;    // workgroups (multiples of 8): up, down, shared down + combine
};

static long round8(long n) { return (n + 7) / 8 * 8; }

static FfnPlan plan_ffn(const FfnProblem& p) {
  FfnPlan L{};
  const long R = (long)p.ntok * p.topk;
  const bool has_shared = p.inter_s > 0 && (p.shared_up || p.shared_down != SharedDown::None);
  L.t = pick_tiles(p, has_shared);
  const bool f8 = p.wkind == WKind::FP8;
  // stream tiles read their weights non-temporally while experts average
  // fewer than 64 rows (one or two m-tiles each): measured faster there,
  // slower once the m-tiles of an expert share weight slices in L2
  L.nt = R < 64L * p.E;
  int bn_up = kUpBN, bn_dn = p.wkind == WKind::FP8 ? kDnBN8 : kDnBN;   // skinny tiles
  L.bm = 16, L.threads = 256;
  if (L.t == Tiles::Big && f8) L.bm = F8::BM, bn_up = F8::UPBN, bn_dn = F8::BN, L.threads = F8::THREADS;
  else if (L.t == Tiles::Huge) L.bm = SHuge::BM, bn_up = SHuge::UPBN, bn_dn = SHuge::BN, L.threads = SHuge::THREADS;
  else if (L.t == Tiles::Big && L.nt) L.bm = SBigNT::BM, bn_up = SBigNT::UPBN, bn_dn = SBigNT::BN, L.threads = SBigNT::THREADS;
  else if (L.t == Tiles::Big) L.bm = SBigUp::BM, bn_up = SBigUp::UPBN, bn_dn = SBig::BN, L.threads = SBigUp::THREADS;
  else if (L.t == Tiles::Mid) L.bm = SMid::BM, bn_up = SMid::UPBN, bn_dn = SMid::BN, L.threads = SMid::THREADS;
  L.bm_dn = L.bm, L.threads_dn = L.threads;
  if (L.t == Tiles::Big && !f8 && !L.nt) L.bm_dn = SBig::BM, L.threads_dn = SBig::THREADS;
  L.nt_up = ceil_div(p.inter, bn_up);
  L.nt_up_s = has_shared ? ceil_div(p.inter_s, bn_up) : 0;
  L.nt_dn = ceil_div(p.dim, bn_dn);
  // the bf16 stream kinds fuse the combine on SComb tiles; the others on the
  // down launch's own tiles
  const bool comb_cfg = !f8 && L.t != Tiles::Skinny;
  L.bm_s = comb_cfg ? SComb::BM : L.bm_dn;
  L.threads_s = comb_cfg ? SComb::THREADS : L.threads_dn;
  L.nt_dn_s = comb_cfg ? ceil_div(p.dim, SComb::BN) : L.nt_dn;
  const long Rr = p.routed ? R : 0;
  L.g_up = Rr || p.shared_up ? round8(max_tiles(Rr, p.E, p.ntok, p.shared_up, L.bm, L.nt_up, L.nt_up_s)) : 0;
  if (L.g_up) L.g_up += 16;   // the split of routed and shared tiles over the XCDs (find_tile)
  const bool dn_store = p.shared_down == SharedDown::Store;
  L.g_dn = Rr || dn_store ? round8(max_tiles(Rr, p.E, p.ntok, dn_store, L.bm_dn, L.nt_dn, L.nt_dn)) : 0;
  L.g_dn_s = p.shared_down == SharedDown::Combine ? round8((long)ceil_div(p.ntok, L.bm_s) * L.nt_dn_s) : 0;
  return L;
}

static long quant_blocks(int ntok, int dim) { return ((long)ntok * (dim / 128) * 16 + 255) / 256; }

static long plan_items(const FfnProblem& p, const FfnPlan& L) {
  long items = std::max(std::max(L.g_up * L.threads, L.g_dn * L.threads_dn), L.g_dn_s * L.threads_s);
  if (p.wkind == WKind::FP8) items = std::max(items, quant_blocks(p.ntok, p.dim) * 256);
  return items;
}

long ffn_max_items(int ntok, int topk, int E, int dim, int inter, int inter_s, WKind wk,
                   bool has_shared) {
  FfnProblem p{};
  p.ntok = ntok; p.topk = topk; p.E = E; p.dim = dim; p.inter = inter; p.inter_s = inter_s;
  p.wkind = wk;
  p.routed = true;
  p.shared_up = has_shared && inter_s > 0;
  // storing the shared output takes the largest down grid of the three ways
  p.shared_down = p.shared_up ? SharedDown::Store : SharedDown::None;
  return plan_items(p, plan_ffn(p));
}

// The down projection launch: routed (and stored shared) tiles, or with kComb
// the shared expert's tiles fused with the combine.
template <bool kComb>
static void launch_down(const FfnProblem& q, const FfnPlan& L, int grid, hipStream_t st) {
  const Tiles t = L.t;
  const bool f8 = q.wkind == WKind::FP8, nt = L.nt;
  if (t == Tiles::Big && f8 && nt) stream_fp8_kernel<false, true, kComb><<<grid, F8::THREADS, 0, st>>>(q);
  else if (t == Tiles::Big && f8) stream_fp8_kernel<false, false, kComb><<<grid, F8::THREADS, 0, st>>>(q);
  else if (f8) down_skinny_fp8_kernel<kComb><<<grid, 256, 0, st>>>(q);
  else if (t == Tiles::Skinny && q.wkind == WKind::BF16) down_skinny_kernel<uint16_t, kComb><<<grid, 256, 0, st>>>(q);
  else if (t == Tiles::Skinny) down_skinny_kernel<float, kComb><<<grid, 256, 0, st>>>(q);
  else if constexpr (kComb) stream_bf16_kernel<SComb, false, true><<<grid, SComb::THREADS, 0, st>>>(q);
  else if (t == Tiles::Huge) stream_bf16_kernel<SHuge, false, false><<<grid, SHuge::THREADS, 0, st>>>(q);
  else if (t == Tiles::Big && nt) stream_bf16_kernel<SBigNT, false, false><<<grid, SBigNT::THREADS, 0, st>>>(q);
  else if (t == Tiles::Big) stream_bf16_kernel<SBig, false, false><<<grid, SBig::THREADS, 0, st>>>(q);
  else stream_bf16_kernel<SMid, false, false><<<grid, SMid::THREADS, 0, st>>>(q);
}

hipError_t launch_ffn(const FfnProblem& p, hipStream_t st) {
  const FfnPlan L = plan_ffn(p);
  // a launch counts its work-items in 32 bits; refuse before enqueuing anything
  if (plan_items(p, L) > kMaxLaunchItems) return hipErrorInvalidConfiguration;
  const Tiles t = L.t;
  const bool f8 = p.wkind == WKind::FP8, nt = L.nt;
  ffn_schedule_kernel<<<1, 1024, 0, st>>>(p.routed ? p.offsets : nullptr, p.E, p.ntok,
                                          p.routed ? 1 : 0, p.shared_up ? 1 : 0,
                                          (int)p.shared_down, L.bm, L.bm_dn, L.nt_up, L.nt_up_s, L.nt_dn,
                                          L.bm_s, L.nt_dn_s, p.e_begin, p.e_end, p.sched);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const FfnProblem& q = p;
  const int g_up = (int)L.g_up, g_dn = (int)L.g_dn, g_dn_s = (int)L.g_dn_s;
  auto mark = [&](int i) { if (p.ev[i]) (void)hipEventRecord(p.ev[i], st); };
  if (f8 && g_up) {   // quantise x once (the 1x128 blocks do not depend on the expert)
    quant_fp8_kernel<<<(int)quant_blocks(p.ntok, p.dim), 256, 0, st>>>(
        static_cast<const uint16_t*>(p.x), p.ntok, p.dim, const_cast<uint8_t*>(p.xq),
        const_cast<float*>(p.xs));
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  mark(0);
  if (g_up == 0) {}
  else if (t == Tiles::Big && f8 && nt) stream_fp8_kernel<true, true><<<g_up, F8::THREADS, 0, st>>>(q);
  else if (t == Tiles::Big && f8) stream_fp8_kernel<true, false><<<g_up, F8::THREADS, 0, st>>>(q);
  else if (t == Tiles::Huge) stream_bf16_kernel<SHuge, true><<<g_up, SHuge::THREADS, 0, st>>>(q);
  else if (t == Tiles::Big && nt) stream_bf16_kernel<SBigNT, true><<<g_up, SBigNT::THREADS, 0, st>>>(q);
  else if (t == Tiles::Big) stream_bf16_kernel<SBigUp, true><<<g_up, SBigUp::THREADS, 0, st>>>(q);
  else if (t == Tiles::Mid) stream_bf16_kernel<SMid, true><<<g_up, SMid::THREADS, 0, st>>>(q);
  else if (p.wkind == WKind::FP8) up_skinny_fp8_kernel<<<g_up, 256, 0, st>>>(q);
  else if (p.wkind == WKind::BF16) up_skinny_kernel<uint16_t><<<g_up, 256, 0, st>>>(q);
  else up_skinny_kernel<float><<<g_up, 256, 0, st>>>(q);
  mark(1);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  mark(2);
  if (g_dn) launch_down<false>(q, L, g_dn, st);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (g_dn_s) launch_down<true>(q, L, g_dn_s, st);
  mark(3);
  return hipGetLastError();
}

hipError_t launch_quant_x(const uint16_t* x, int rows, int cols, uint8_t* xq, float* xs,
                          hipStream_t st) {
  if (quant_blocks(rows, cols) * 256 > kMaxLaunchItems) return hipErrorInvalidConfiguration;
  quant_fp8_kernel<<<(int)quant_blocks(rows, cols), 256, 0, st>>>(
      x, rows, cols, xq, xs);
  return hipGetLastError();
}

}  // namespace moe
