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

// Returns false when this workgroup has no tile.
__device__ __forceinline__ bool find_tile(const int32_t* __restrict__ sched,
                                          const int32_t* __restrict__ offsets, int E, int ntok,
                                          int bm, int tile, TileInfo& ti) {
  if (tile >= sched[E + 1]) return false;
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
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  if (!find_tile(p.sched, p.offsets, p.E, p.ntok, 16, tile, ti)) return;
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
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int32_t* sched = p.sched + p.E + 2;
  if (!find_tile(sched, p.offsets, p.E, p.ntok, 16, tile, ti)) return;
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
  const int bm = 16;
  const int nt_up = ceil_div(p.inter, kUpBN), nt_up_s = has_shared ? ceil_div(p.inter_s, kUpBN) : 0;
  const int nt_dn = ceil_div(p.dim, kDnBN);
  ffn_schedule_kernel<<<1, 1024, 0, st>>>(p.offsets, p.E, p.ntok, has_shared ? 1 : 0, bm, nt_up,
                                          nt_up_s, bm, nt_dn, p.sched);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  FfnProblem q = p;
  if (!has_shared) { q.ws1 = q.ws3 = q.ws2 = nullptr; q.shared_out = nullptr; }
  const int g_up = round8(max_tiles(R, p.E, p.ntok, has_shared, bm, nt_up, nt_up_s));
  const int g_dn = round8(max_tiles(R, p.E, p.ntok, has_shared, bm, nt_dn, nt_dn));
  auto mark = [&](int i) { if (p.ev[i]) (void)hipEventRecord(p.ev[i], st); };
  if (p.wkind == WKind::F32) {
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
  } else {
    return hipErrorNotSupported;
  }
  return hipGetLastError();
}

hipError_t launch_quant_x(const uint16_t*, int, int, uint8_t*, float*, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace moe
