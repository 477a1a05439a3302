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
#include <type_traits>

namespace moe {

__global__ __launch_bounds__(1024) void ffn_schedule_kernel(const int32_t* __restrict__ offsets,
                                                            int E, int ntok, int has_shared,
                                                            int bm_up, int nt_up, int nt_up_s,
                                                            int bm_dn, int nt_dn,
                                                            int32_t* __restrict__ sched) {
  __shared__ int su[1024], sd[1024];
  const int g = threadIdx.x;
  int cu = 0, cd = 0;
  if (g < E) {
    const int M = offsets[g + 1] - offsets[g];
    cu = (M + bm_up - 1) / bm_up * nt_up;
    cd = (M + bm_dn - 1) / bm_dn * nt_dn;
  } else if (g == E && has_shared) {
    cu = (ntok + bm_up - 1) / bm_up * nt_up_s;
    cd = (ntok + bm_dn - 1) / bm_dn * nt_dn;
  }
  su[g] = cu;
  sd[g] = cd;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int vu = g >= o ? su[g - o] : 0;
    const int vd = g >= o ? sd[g - o] : 0;
    __syncthreads();
    su[g] += vu;
    sd[g] += vd;
    __syncthreads();
  }
  if (g <= E) {
    sched[g] = su[g] - cu;
    sched[E + 2 + g] = sd[g] - cd;
  }
  if (g == E) {
    sched[E + 1] = su[g];
    sched[E + 2 + E + 1] = sd[g];
  }
}

struct TileInfo {
  int g;        // group (E = shared)
  int row0;     // first row of the group in the expert-contiguous order
  int M;        // rows of the group
  int mt, nt;   // tile coordinates
};

// Maps this workgroup to a tile; returns false when it has none.  The grid is
// an upper bound on the tile count (the real count is only known on the
// device), so the XCD-aware remap runs over the real count rounded up to 8:
// every XCD then gets an equal, contiguous range of tiles (all n-tiles and
// m-tiles of an expert next to each other, sharing its rows in that XCD's
// L2), and the surplus workgroups exit.
__device__ __forceinline__ bool find_tile(const int32_t* __restrict__ sched,
                                          const int32_t* __restrict__ offsets, int E, int ntok,
                                          int bm, TileInfo& ti) {
  const int total = sched[E + 1];
  const int n8 = (total + 7) & ~7;
  if ((int)blockIdx.x >= n8) return false;
  const int tile = xcd_remap(blockIdx.x, n8);
  if (tile >= total) return false;
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
  return true;
}

// Double-buffered K loop over 64-byte chunks: U chunks per stage, NA A-operand
// rows (16-row tiles) against one B operand.  nchunk must be a multiple of U.
template <typename T, int NA, int U>
__device__ __forceinline__ void kloop(const char* const (&ap)[NA], const char* bp, int nchunk,
                                      f32x4_t (&acc)[NA]) {
  uint4 a0[U][NA], b0[U], a1[U][NA], b1[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    b0[u] = ldg16(bp + 64 * u);
#pragma unroll
    for (int j = 0; j < NA; ++j) a0[u][j] = ldg16(ap[j] + 64 * u);
  }
  for (int c = 0; c < nchunk; c += 2 * U) {
    if (c + U < nchunk) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        b1[u] = ldg16(bp + 64 * (c + U + u));
#pragma unroll
        for (int j = 0; j < NA; ++j) a1[u][j] = ldg16(ap[j] + 64 * (c + U + u));
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
        for (int j = 0; j < NA; ++j) a0[u][j] = ldg16(ap[j] + 64 * (c + 2 * U + u));
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
constexpr int kDnNT = 4;     // 16-row tiles of W2 per wave
constexpr int kUpBN = kSkinnyWaves * 16 * kUpNT;   // h columns per workgroup
constexpr int kDnBN = kSkinnyWaves * 16 * kDnNT;   // output columns per workgroup

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
  const int mi = min(ti.mt * 16 + r, ti.M - 1);
  const int xrow = shared ? mi : p.sorted_token[ti.row0 + mi];
  const char* bp = reinterpret_cast<const char*>(static_cast<const T*>(p.x) + (size_t)xrow * p.dim) + 16 * grp;
  const T* W1 = shared ? static_cast<const T*>(p.ws1) : static_cast<const T*>(p.w1) + (size_t)ti.g * N * p.dim;
  const T* W3 = shared ? static_cast<const T*>(p.ws3) : static_cast<const T*>(p.w3) + (size_t)ti.g * N * p.dim;
  const char* ap[2 * kUpNT];
#pragma unroll
  for (int j = 0; j < kUpNT; ++j) {
    const int n = nbase + 16 * j + r;
    ap[j] = reinterpret_cast<const char*>(W1 + (size_t)n * p.dim) + 16 * grp;
    ap[kUpNT + j] = reinterpret_cast<const char*>(W3 + (size_t)n * p.dim) + 16 * grp;
  }
  f32x4_t acc[2 * kUpNT];
#pragma unroll
  for (int j = 0; j < 2 * kUpNT; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  kloop<T, 2 * kUpNT, 2>(ap, bp, p.dim * (int)sizeof(T) / 64, acc);

  const int m = ti.mt * 16 + r;
  if (m < ti.M) {
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

template <typename T>
__global__ __launch_bounds__(256) void down_skinny_kernel(FfnProblem p) {
  TileInfo ti;
  const int32_t* sched = p.sched + p.E + 2;
  if (!find_tile(sched, p.offsets, p.E, p.ntok, 16, ti)) return;
  const bool shared = ti.g == p.E;
  const int K = shared ? p.inter_s : p.inter;
  const int N = p.dim;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, grp = lane >> 4;
  const int nbase = ti.nt * kDnBN + wave * 16 * kDnNT;
  if (nbase >= N) return;
  const int mi = min(ti.mt * 16 + r, ti.M - 1);
  const T* hrow = shared ? static_cast<const T*>(p.hs) + (size_t)mi * K
                         : static_cast<const T*>(p.h) + (size_t)(ti.row0 + mi) * K;
  const char* bp = reinterpret_cast<const char*>(hrow) + 16 * grp;
  const T* W2 = shared ? static_cast<const T*>(p.ws2) : static_cast<const T*>(p.w2) + (size_t)ti.g * N * K;
  const char* ap[kDnNT];
#pragma unroll
  for (int j = 0; j < kDnNT; ++j)
    ap[j] = reinterpret_cast<const char*>(W2 + (size_t)(nbase + 16 * j + r) * K) + 16 * grp;
  f32x4_t acc[kDnNT];
#pragma unroll
  for (int j = 0; j < kDnNT; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  kloop<T, kDnNT, 2>(ap, bp, K * (int)sizeof(T) / 64, acc);

  const int m = ti.mt * 16 + r;
  if (m < ti.M) {
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
// Stream tiles (prefill): up to 192 token rows x 256 weight rows per
// workgroup of 8 waves (two per SIMD), on v_mfma_f32_32x32x16_bf16 (the
// 32x32 shape runs at full rate on gfx950; 16x16x32 issues at half rate).
// A tile covers a whole expert whenever it has <= 192 tokens, so each weight
// slice is fetched from HBM once per expert.
//   A operand = 32 weight rows per wave, loaded straight from global memory
//     through a ring of 4 register stages (three 64-element K slices in
//     flight); for the up projection rows 0-15 are W1 rows and rows 16-31 the
//     same rows of W3, so a lane's result elements i and i+8 are the two
//     branches of one h column and SwiGLU needs no data exchange.
//   B operand = token rows, staged in LDS (double-buffered) and read by all 8
//     waves: the slice of every n-tile of an expert is the same, so it is
//     L2-resident.
// Loaded HBM latency is several microseconds, so both operands run three
// 64-element slices ahead (token slices in registers until their LDS store).
// Memory counters retire in issue order; with equal lookahead, waiting for
// the token slice to store never forces a newer weight slice to land early.  The K loop is instantiated for the
// number of 32-row token sub-tiles it computes.  LDS rows are padded by 16
// bytes so the fragment reads of a wave spread over the banks.
// ---------------------------------------------------------------------------
constexpr int kSBM = 192;             // token rows per tile
constexpr int kSMT = kSBM / 32;       // 32-row token sub-tiles per tile
constexpr int kSWaves = 8;
constexpr int kSBN = kSWaves * 32;    // weight rows per tile
constexpr int kSUpBN = kSBN / 2;      // h columns per up tile
constexpr int kSBK = 64;              // K elements per step (bf16)
constexpr int kSKs = kSBK / 16;       // MFMA k-steps per step
constexpr int kSStride = 2 * kSBK + 16;   // LDS bytes per token row
constexpr int kSLds = kSBM * kSStride;
constexpr int kSTPR = 2 * kSBK / 16;                       // threads per token row
constexpr int kSRowsPerPass = kSWaves * 64 / kSTPR;       // token rows per load pass
constexpr int kSXLoads = kSBM / kSRowsPerPass;             // 16-byte token loads per thread
constexpr int kSRing = 4;

struct StreamSrc {
  const char* x[kSXLoads];   // token rows (tid / kSTPR) + kSRowsPerPass*i, at byte 16*(tid % kSTPR)
  const char* w;             // this lane's weight row, at byte 16*(lane/32)
  int lds_st;                // LDS byte offset of this thread's token chunk
};


__device__ __forceinline__ f32x16_t mma32(f32x16_t c, uint4 a, uint4 b) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

template <int MT>
__device__ __forceinline__ void stream_kloop(char (&sx)[2][kSLds], const StreamSrc& S, int nk,
                                             f32x16_t (&acc)[kSMT]) {
  const int lane = threadIdx.x & 63, fr = lane & 31, fg = lane >> 5;
  uint4 wr[kSRing][kSKs];        // weight slices kt .. kt+3: [slice % 4][k-step]
  uint4 xr[kSRing][kSXLoads];    // token slices kt+1 .. kt+3 in flight: [slice % 4]
  auto wload = [&](uint4 (&dst)[kSKs], int kt) {
    kt = kt < nk ? kt : nk - 1;
#pragma unroll
    for (int s = 0; s < kSKs; ++s) dst[s] = ldg16(S.w + kt * (2 * kSBK) + 32 * s);
  };
  auto xload = [&](uint4 (&dst)[kSXLoads], int kt) {
    kt = kt < nk ? kt : nk - 1;
#pragma unroll
    for (int i = 0; i < kSXLoads; ++i) dst[i] = ldg16(S.x[i] + kt * (2 * kSBK));
  };
  auto xstore = [&](const uint4 (&src)[kSXLoads], int buf) {
#pragma unroll
    for (int i = 0; i < kSXLoads; ++i)
      *reinterpret_cast<uint4*>(&sx[buf][S.lds_st + kSRowsPerPass * i * kSStride]) = src[i];
  };
  // slices 0..2 of both operands in flight, token slice 0 into LDS
#pragma unroll
  for (int j = 0; j < kSRing - 1; ++j) {
    xload(xr[j], j);
    wload(wr[j], j);
  }
  xstore(xr[0], 0);
  __syncthreads();
  // step kt (R = kt % 4, compile-time): issue token and weight slice kt+3 (in
  // that order), compute slice kt, store token slice kt+1.  The store waits
  // for token slice kt+1 and whatever was issued before it - slices <= kt -
  // so slices kt+2 and kt+3 stay in flight across the barrier.
  auto step = [&](int kt, auto R) {
    constexpr int r = decltype(R)::value;
    xload(xr[(r + 3) % 4], kt + 3);
    wload(wr[(r + 3) % 4], kt + 3);
    __builtin_amdgcn_sched_barrier(0);
    const char* sb = sx[r & 1] + fr * kSStride + 16 * fg;
#pragma unroll
    for (int s = 0; s < kSKs; ++s) {
      uint4 fx[MT];
#pragma unroll
      for (int a = 0; a < MT; ++a)
        fx[a] = *reinterpret_cast<const uint4*>(sb + 32 * a * kSStride + 32 * s);
#pragma unroll
      for (int a = 0; a < MT; ++a) acc[a] = mma32(acc[a], wr[r][s], fx[a]);
    }
    xstore(xr[(r + 1) % 4], (r + 1) & 1);
    __syncthreads();
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  const int nmain = nk & ~3;
  int kt = 0;
  for (; kt < nmain; kt += 4) {
    step(kt, I0{});
    step(kt + 1, I1{});
    step(kt + 2, I2{});
    step(kt + 3, I3{});
  }
  if (kt < nk) step(kt, I0{});
  if (kt + 1 < nk) step(kt + 1, I1{});
  if (kt + 2 < nk) step(kt + 2, I2{});
}

template <bool kUp>
__global__ __launch_bounds__(512, 1) __attribute__((amdgpu_waves_per_eu(2, 2)))
void stream_bf16_kernel(FfnProblem p) {
  __shared__ __attribute__((aligned(16))) char sx[2][kSLds];
  TileInfo ti;
  const int32_t* sched = kUp ? p.sched : p.sched + p.E + 2;
  if (!find_tile(sched, p.offsets, p.E, p.ntok, kSBM, ti)) return;
  const bool shared = ti.g == p.E;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = kUp ? p.dim : (shared ? p.inter_s : p.inter);
  const int N = kUp ? (shared ? p.inter_s : p.inter) : p.dim;   // h columns / output columns
  const int m0 = ti.mt * kSBM;
  const int rows_left = ti.M - m0;

  StreamSrc S;
  const int lc = tid % kSTPR, lr = tid / kSTPR;
#pragma unroll
  for (int i = 0; i < kSXLoads; ++i) {
    const int m = m0 + min(lr + kSRowsPerPass * i, rows_left - 1);
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
  S.lds_st = lr * kSStride + 16 * lc;

  const int fr = lane & 31, fg = lane >> 5;
  int ncol0;                        // first output column of the wave
  bool wave_active;
  if (kUp) {
    // A rows 0-15: W1 rows ncol0 + [0,16); rows 16-31: the same rows of W3
    ncol0 = ti.nt * kSUpBN + wave * 16;
    wave_active = ncol0 < N;
    const int n = min(ncol0 + (fr & 15), N - 1);
    const uint16_t* W = fr < 16 ? (shared ? static_cast<const uint16_t*>(p.ws1)
                                          : static_cast<const uint16_t*>(p.w1) + (size_t)ti.g * N * K)
                                : (shared ? static_cast<const uint16_t*>(p.ws3)
                                          : static_cast<const uint16_t*>(p.w3) + (size_t)ti.g * N * K);
    S.w = reinterpret_cast<const char*>(W + (size_t)n * K) + 16 * fg;
  } else {
    ncol0 = ti.nt * kSBN + wave * 32;
    wave_active = ncol0 < N;
    const uint16_t* W2 = shared ? static_cast<const uint16_t*>(p.ws2)
                                : static_cast<const uint16_t*>(p.w2) + (size_t)ti.g * N * K;
    S.w = reinterpret_cast<const char*>(W2 + (size_t)min(ncol0 + fr, N - 1) * K) + 16 * fg;
  }
  int m_active = (rows_left + 31) >> 5;
  m_active = m_active > kSMT ? kSMT : m_active;
  if (!wave_active) m_active = 1;

  f32x16_t acc[kSMT];
#pragma unroll
  for (int a = 0; a < kSMT; ++a)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[a][i] = 0.f;

  const int nk = K / kSBK;
  if (m_active > 4) stream_kloop<kSMT>(sx, S, nk, acc);
  else if (m_active > 2) stream_kloop<4>(sx, S, nk, acc);
  else if (m_active > 1) stream_kloop<2>(sx, S, nk, acc);
  else stream_kloop<1>(sx, S, nk, acc);
  if (!wave_active) return;

  // epilogue: lane holds D[row = 8*(i/4) + 4*(lane/32) + i%4][col = lane % 32]
  // (row = weight row of the wave, col = token of the sub-tile)
  const int ml = lane & 31, rg = 4 * (lane >> 5);
#pragma unroll
  for (int a = 0; a < kSMT; ++a) {
    const int m = m0 + 32 * a + ml;
    if (a >= m_active || m >= ti.M) continue;
    if (kUp) {
      uint16_t* hrow = shared ? static_cast<uint16_t*>(p.hs) + (size_t)m * N
                              : static_cast<uint16_t*>(p.h) + (size_t)(ti.row0 + m) * N;
#pragma unroll
      for (int q = 0; q < 2; ++q) {       // rows 8q + rg + [0,4) of W1, 16 + same of W3
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = silu(acc[a][4 * q + i]) * acc[a][8 + 4 * q + i];
        store4<uint16_t>(hrow + ncol0 + 8 * q + rg, v);
      }
    } else {
      uint16_t* orow = shared ? static_cast<uint16_t*>(p.shared_out) + (size_t)m * N
                              : static_cast<uint16_t*>(p.out) + (size_t)(ti.row0 + m) * N;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float v[4] = {acc[a][4 * q], acc[a][4 * q + 1], acc[a][4 * q + 2], acc[a][4 * q + 3]};
        store4<uint16_t>(orow + ncol0 + 8 * q + rg, v);
      }
    }
  }
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
typedef __attribute__((ext_vector_type(8))) int i32x8_t_;

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
  const int mi = min(ti.mt * 16 + r, ti.M - 1);
  const int tok = shared ? mi : p.sorted_token[ti.row0 + mi];
  const char* bp = reinterpret_cast<const char*>(p.xq + (size_t)tok * K) + 32 * grp;
  const float* bsc = p.xs + (size_t)tok * KB;
  const uint8_t* W1 = static_cast<const uint8_t*>(shared ? p.ws1 : p.w1) + (shared ? 0 : (size_t)ti.g * N * K);
  const uint8_t* W3 = static_cast<const uint8_t*>(shared ? p.ws3 : p.w3) + (shared ? 0 : (size_t)ti.g * N * K);
  const float* S1 = (shared ? p.ws1s : p.w1s + (size_t)ti.g * (N / 128) * KB) + (size_t)(nbase / 128) * KB;
  const float* S3 = (shared ? p.ws3s : p.w3s + (size_t)ti.g * (N / 128) * KB) + (size_t)(nbase / 128) * KB;
  const char* ap[4];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    ap[j] = reinterpret_cast<const char*>(W1 + (size_t)(nbase + 16 * j + r) * K) + 32 * grp;
    ap[j + 2] = reinterpret_cast<const char*>(W3 + (size_t)(nbase + 16 * j + r) * K) + 32 * grp;
  }
  f32x4_t acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  uint4 a[2][4][2], b[2][2];
  auto load = [&](int s, int kb) {
#pragma unroll
    for (int j = 0; j < 4; ++j) { a[s][j][0] = ldg16(ap[j] + 128 * kb); a[s][j][1] = ldg16(ap[j] + 128 * kb + 16); }
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
  const int m = ti.mt * 16 + r;
  if (m < ti.M) {
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

// Down projection, fp8, skinny tiles: 16 tokens x 256 output columns.
__global__ __launch_bounds__(256) void down_skinny_fp8_kernel(FfnProblem p) {
  TileInfo ti;
  const int32_t* sched = p.sched + p.E + 2;
  if (!find_tile(sched, p.offsets, p.E, p.ntok, 16, ti)) return;
  const bool shared = ti.g == p.E;
  const int K = shared ? p.inter_s : p.inter, KB = K / 128;
  const int N = p.dim;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, grp = lane >> 4;
  const int nbase = ti.nt * kDnBN + wave * 16 * kDnNT;
  if (nbase >= N) return;
  const int mi = min(ti.mt * 16 + r, ti.M - 1);
  const size_t hrow = shared ? (size_t)mi : (size_t)(ti.row0 + mi);
  const char* bp = reinterpret_cast<const char*>(static_cast<const uint8_t*>(shared ? p.hs : p.h) + hrow * K) + 32 * grp;
  const float* bsc = (shared ? p.hsscale : p.hscale) + hrow * KB;
  const uint8_t* W2 = static_cast<const uint8_t*>(shared ? p.ws2 : p.w2) + (shared ? 0 : (size_t)ti.g * N * K);
  const float* S2 = (shared ? p.ws2s : p.w2s + (size_t)ti.g * (N / 128) * KB);
  const char* ap[kDnNT];
  const float* sp[kDnNT];
#pragma unroll
  for (int j = 0; j < kDnNT; ++j) {
    const int n = nbase + 16 * j;
    ap[j] = reinterpret_cast<const char*>(W2 + (size_t)(n + r) * K) + 32 * grp;
    sp[j] = S2 + (size_t)(n / 128) * KB;
  }
  f32x4_t acc[kDnNT];
#pragma unroll
  for (int j = 0; j < kDnNT; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  uint4 a[2][kDnNT][2], b[2][2];
  auto load = [&](int s, int kb) {
#pragma unroll
    for (int j = 0; j < kDnNT; ++j) { a[s][j][0] = ldg16(ap[j] + 128 * kb); a[s][j][1] = ldg16(ap[j] + 128 * kb + 16); }
    b[s][0] = ldg16(bp + 128 * kb);
    b[s][1] = ldg16(bp + 128 * kb + 16);
  };
  auto comp = [&](int s, int kb) {
    const float hsc = bsc[kb];
#pragma unroll
    for (int j = 0; j < kDnNT; ++j) {
      const f32x4_t part = mma_fp8(a[s][j][0], a[s][j][1], b[s][0], b[s][1]);
      const float sc = sp[j][kb] * hsc;
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
  const int m = ti.mt * 16 + r;
  if (m < ti.M) {
    uint16_t* orow = static_cast<uint16_t*>(shared ? p.shared_out : p.out) + (shared ? (size_t)m : (size_t)(ti.row0 + m)) * N;
#pragma unroll
    for (int j = 0; j < kDnNT; ++j) {
      float v[4] = {acc[j][0], acc[j][1], acc[j][2], acc[j][3]};
      store4<uint16_t>(orow + nbase + 16 * j + 4 * grp, v);
    }
  }
}

static inline int ceil_div(long a, long b) { return (int)((a + b - 1) / b); }
static inline int round8(long n) { return (int)((n + 7) / 8 * 8); }

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

hipError_t launch_ffn(const FfnProblem& p, hipStream_t st) {
  const bool has_shared = p.ws1 != nullptr && p.shared_out != nullptr && p.inter_s > 0;
  const long R = (long)p.ntok * p.topk;
  // stream tiles once experts see enough tokens to reuse a weight slice
  const bool wide = p.wkind == WKind::BF16 && R >= 48L * p.E && p.dim % kSBK == 0 &&
                    p.inter % kSBK == 0 && (!has_shared || p.inter_s % kSBK == 0);
  const int bm = wide ? kSBM : 16;
  const int bn_up = wide ? kSUpBN : kUpBN, bn_dn = wide ? kSBN : kDnBN;
  const int nt_up = ceil_div(p.inter, bn_up), nt_up_s = has_shared ? ceil_div(p.inter_s, bn_up) : 0;
  const int nt_dn = ceil_div(p.dim, bn_dn);
  ffn_schedule_kernel<<<1, 1024, 0, st>>>(p.offsets, p.E, p.ntok, has_shared ? 1 : 0, bm, nt_up,
                                          nt_up_s, bm, nt_dn, p.sched);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  FfnProblem q = p;
  if (!has_shared) { q.ws1 = q.ws3 = q.ws2 = nullptr; q.shared_out = nullptr; }
  const int g_up = round8(max_tiles(R, p.E, p.ntok, has_shared, bm, nt_up, nt_up_s));
  const int g_dn = round8(max_tiles(R, p.E, p.ntok, has_shared, bm, nt_dn, nt_dn));
  auto mark = [&](int i) { if (p.ev[i]) (void)hipEventRecord(p.ev[i], st); };
  if (wide) {
    mark(0);
    stream_bf16_kernel<true><<<g_up, 512, 0, st>>>(q);
    mark(1);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    mark(2);
    stream_bf16_kernel<false><<<g_dn, 512, 0, st>>>(q);
    mark(3);
  } else if (p.wkind == WKind::F32) {
    mark(0);
    up_skinny_kernel<float><<<g_up, 256, 0, st>>>(q);
    mark(1);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    mark(2);
    down_skinny_kernel<float><<<g_dn, 256, 0, st>>>(q);
    mark(3);
  } else if (p.wkind == WKind::BF16) {
    mark(0);
    up_skinny_kernel<uint16_t><<<g_up, 256, 0, st>>>(q);
    mark(1);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    mark(2);
    down_skinny_kernel<uint16_t><<<g_dn, 256, 0, st>>>(q);
    mark(3);
  } else {   // fp8: quantise x once (the 1x128 blocks do not depend on the expert)
    quant_fp8_kernel<<<(int)(((long)p.ntok * (p.dim / 128) * 16 + 255) / 256), 256, 0, st>>>(
        static_cast<const uint16_t*>(p.x), p.ntok, p.dim, const_cast<uint8_t*>(p.xq),
        const_cast<float*>(p.xs));
    if ((err = hipGetLastError()) != hipSuccess) return err;
    mark(0);
    up_skinny_fp8_kernel<<<g_up, 256, 0, st>>>(q);
    mark(1);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    mark(2);
    down_skinny_fp8_kernel<<<g_dn, 256, 0, st>>>(q);
    mark(3);
  }
  return hipGetLastError();
}

hipError_t launch_quant_x(const uint16_t* x, int rows, int cols, uint8_t* xq, float* xs,
                          hipStream_t st) {
  quant_fp8_kernel<<<(int)(((long)rows * (cols / 128) * 16 + 255) / 256), 256, 0, st>>>(
      x, rows, cols, xq, xs);
  return hipGetLastError();
}

}  // namespace moe
