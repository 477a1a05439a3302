// Gate kernels: router logits on MFMA, then per-token group-limited top-k.
//
// Source: "DeepSeek-V3.2-Exp · Expert scores" (formula z = x_ffn W_r; the
// router weight is held in bf16 and applied in fp32; Gate.forward excerpt).
#include "common.h"
#include "kernels.h"

namespace moe {

// ---------------------------------------------------------------------------
// logits[T, E] (fp32) = x[T, dim] . W_r[E, dim]^T
//
// One workgroup = 4 waves computes a 16 (experts) x 16 (tokens) tile; the
// waves split K into interleaved 64-byte chunks and the partial tiles are
// summed in LDS in a fixed order.  A operand = router rows, B operand = token
// rows, so each lane ends with 4 consecutive experts of one token.
// bf16 x bf16 products are exact in fp32 and accumulate in fp32.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void router_logits_kernel(const T* __restrict__ x,
                                                            const T* __restrict__ wr,
                                                            float* __restrict__ logits,
                                                            int ntok, int dim, int E) {
  __shared__ f32x4_t part[4][kWave];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * 16, e0 = blockIdx.y * 16;
  const int r = lane & 15, g = lane >> 4;
  const int tok = min(t0 + r, ntok - 1);
  const int ex = min(e0 + r, E - 1);
  const char* xa = reinterpret_cast<const char*>(x + (size_t)tok * dim) + 16 * g;
  const char* wa = reinterpret_cast<const char*>(wr + (size_t)ex * dim) + 16 * g;
  const int nchunk = dim * (int)sizeof(T) / 64;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  int c = wave;
  for (; c + 12 < nchunk; c += 16) {   // 4 chunks in flight per wave
    uint4 a0 = ldg16(wa + 64 * c), b0 = ldg16(xa + 64 * c);
    uint4 a1 = ldg16(wa + 64 * (c + 4)), b1 = ldg16(xa + 64 * (c + 4));
    uint4 a2 = ldg16(wa + 64 * (c + 8)), b2 = ldg16(xa + 64 * (c + 8));
    uint4 a3 = ldg16(wa + 64 * (c + 12)), b3 = ldg16(xa + 64 * (c + 12));
    acc = Chunk<T>::mma(acc, a0, b0);
    acc = Chunk<T>::mma(acc, a1, b1);
    acc = Chunk<T>::mma(acc, a2, b2);
    acc = Chunk<T>::mma(acc, a3, b3);
  }
  for (; c < nchunk; c += 4) acc = Chunk<T>::mma(acc, ldg16(wa + 64 * c), ldg16(xa + 64 * c));
  part[wave][lane] = acc;
  __syncthreads();
  if (wave == 0) {
    f32x4_t s = part[0][lane];
    s += part[1][lane];
    s += part[2][lane];
    s += part[3][lane];
    const int t = t0 + r;                 // column of D = token
    const int e = e0 + 4 * g;             // rows of D = 4 consecutive experts
    if (t < ntok) {
      float* out = logits + (size_t)t * E;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (e + i < E) out[e + i] = s[i];
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 router on v_mfma_f32_32x32x16_bf16: a workgroup of 4 waves computes a
// 128-token x 128-expert tile; wave w owns the 64 x 64 quarter (tokens
// 64*(w&1), experts 64*(w>>1)) as 2 x 2 MFMA tiles (A operand = token rows,
// B operand = router rows, so a lane ends with one expert of 16 tokens per
// tile and each result row is a coalesced 128-byte store).  Both operand
// tiles go through LDS in 64-element K slices, double-buffered, each slice
// loaded into registers two steps ahead.  When the tiles alone cannot fill
// the GPU, K is split over blockIdx.z; the split partials go to a workspace
// and the selection kernel sums them in split order as it reads them, so the
// result does not depend on timing.
// ---------------------------------------------------------------------------
constexpr int kRtTile = 128;              // tokens and experts per workgroup
constexpr int kRtStride = 144;            // LDS bytes per 128-byte row slice (padded)
constexpr int kRtPass = 4;                // 16-byte loads per operand per thread per slice
constexpr int kRtMaxSplits = 16;

int router_splits(int ntok, int E, int dim, int* steps_per_split) {
  const int tiles = ((ntok + kRtTile - 1) / kRtTile) * ((E + kRtTile - 1) / kRtTile);
  const int nk = dim / 64;
  if (tiles <= 0 || nk <= 0) {
    if (steps_per_split) *steps_per_split = nk;
    return 1;
  }
  int S = (512 + tiles - 1) / tiles;
  S = S < 1 ? 1 : S;
  S = S > kRtMaxSplits ? kRtMaxSplits : S;
  S = S > nk ? nk : S;
  const int per = (nk + S - 1) / S;
  if (steps_per_split) *steps_per_split = per;
  return (nk + per - 1) / per;
}

__global__ __launch_bounds__(256, 2) void router_mfma_kernel(const uint16_t* __restrict__ x,
                                                             const uint16_t* __restrict__ wr,
                                                             float* __restrict__ out, int ntok,
                                                             int dim, int E, int steps_per_split,
                                                             size_t split_stride) {
  __shared__ __attribute__((aligned(16))) char sx[2][kRtTile * kRtStride];
  __shared__ __attribute__((aligned(16))) char sw[2][kRtTile * kRtStride];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tb = blockIdx.x * kRtTile, eb = blockIdx.y * kRtTile;
  const int nk = dim / 64;
  const int k0 = blockIdx.z * steps_per_split;
  const int k1 = min(nk, k0 + steps_per_split);
  // staging: thread tid moves bytes 16*(tid%8) of rows tid/8 + 32*i (i < 4) of both tiles
  const int lc = tid & 7, lr = tid >> 3;
  const char* xg[kRtPass];
  const char* wg[kRtPass];
#pragma unroll
  for (int i = 0; i < kRtPass; ++i) {
    xg[i] = reinterpret_cast<const char*>(x + (size_t)min(tb + lr + 32 * i, ntok - 1) * dim) + 16 * lc;
    wg[i] = reinterpret_cast<const char*>(wr + (size_t)min(eb + lr + 32 * i, E - 1) * dim) + 16 * lc;
  }
  const int st_off = lr * kRtStride + 16 * lc;
  uint4 rx[2][kRtPass], rw[2][kRtPass];
  auto gload = [&](uint4 (&dx)[kRtPass], uint4 (&dw)[kRtPass], int kt) {
    kt = kt < k1 ? kt : k1 - 1;
#pragma unroll
    for (int i = 0; i < kRtPass; ++i) {
      dx[i] = ldg16(xg[i] + kt * 128);
      dw[i] = ldg16(wg[i] + kt * 128);
    }
  };
  auto sstore = [&](const uint4 (&dx)[kRtPass], const uint4 (&dw)[kRtPass], int buf) {
#pragma unroll
    for (int i = 0; i < kRtPass; ++i) {
      *reinterpret_cast<uint4*>(&sx[buf][st_off + 32 * i * kRtStride]) = dx[i];
      *reinterpret_cast<uint4*>(&sw[buf][st_off + 32 * i * kRtStride]) = dw[i];
    }
  };
  // fragments: lane reads row (32j + lane%32) of its quarter, bytes 16*(lane/32) + 32s
  const int fr = lane & 31, fg = lane >> 5;
  const int xq = (64 * (wave & 1) + fr) * kRtStride + 16 * fg;
  const int wq = (64 * (wave >> 1) + fr) * kRtStride + 16 * fg;
  f32x16_t acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.f;
  auto comp = [&](int buf) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      uint4 fa[2], fb[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        fa[j] = *reinterpret_cast<const uint4*>(&sx[buf][xq + 32 * j * kRtStride + 32 * s]);
        fb[j] = *reinterpret_cast<const uint4*>(&sw[buf][wq + 32 * j * kRtStride + 32 * s]);
      }
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, fa[a]),
                                                              __builtin_bit_cast(bf16x8_t, fb[b]),
                                                              acc[a][b], 0, 0, 0);
    }
  };
  gload(rx[0], rw[0], k0);
  gload(rx[1], rw[1], k0 + 1);
  sstore(rx[0], rw[0], 0);
  __syncthreads();
  // step kt: issue slice kt+2 into the registers slice kt held, multiply slice
  // kt, store slice kt+1 into the other LDS buffer
  int kt = k0;
  for (; kt + 2 <= k1; kt += 2) {
    gload(rx[0], rw[0], kt + 2);
    comp(0);
    sstore(rx[1], rw[1], 1);
    __syncthreads();
    gload(rx[1], rw[1], kt + 3);
    comp(1);
    sstore(rx[0], rw[0], 0);
    __syncthreads();
  }
  if (kt < k1) comp(0);

  // D[row = 8*(i/4) + 4*(lane/32) + i%4][col = lane%32]: token row, expert column
  float* o = out + (size_t)blockIdx.z * split_stride;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int e = eb + 64 * (wave >> 1) + 32 * b + fr;
    if (e >= E) continue;
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int t = tb + 64 * (wave & 1) + 32 * a + 8 * (i / 4) + 4 * fg + (i % 4);
        if (t < ntok) o[(size_t)t * E + e] = acc[a][b][i];
      }
  }
}

// ---------------------------------------------------------------------------
// Selection: one wave per token.
//   s = sigmoid(z) or softmax(z); s' = s + bias (selection only)
//   n_groups > 1: group score = top-2 sum of s' (bias given) or max s' (no
//   bias); keep the topk_groups best groups (ties -> lower group id)
//   topk rounds of a wave arg-max over the candidates, ordered by
//   (s' descending, expert id ascending); the winner's unbiased s is its weight
//   sigmoid: w /= sum(w); then w *= route_scale
// Lane l holds experts l, l+64, ... (PL = ceil(E/64) per lane, E <= 512).
// ---------------------------------------------------------------------------
constexpr int kSelWaves = 4;

// `logits` holds `splits` partial logit arrays of ntok*E values each (one when
// the router did not split K); they are summed in split order, in fp32.  The
// loads of up to 16 splits are in flight at once (all of them: the router
// One step of the wave arg-max: take the (value, id, score) of the lane that
// DPP control kCtrl names when it ranks higher - a larger value, or an equal
// value and a lower id.
template <int kCtrl>
__device__ __forceinline__ void argmax_dpp_step(float& v, int& i, float& s) {
  const float ov = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF, false));
  const int oi = __builtin_amdgcn_update_dpp(0, i, kCtrl, 0xF, 0xF, false);
  const float os = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(s), kCtrl, 0xF, 0xF, false));
  if (ov > v || (ov == v && oi < i)) { v = ov; i = oi; s = os; }
}

// Arg-max over the wave under that order, result in every lane.  Swaps of
// lane pairs within quads (quad_perm 1,0,3,2 and 2,3,0,1), then within
// 8-lane halves (row_half_mirror: k <-> 7-k) and 16-lane rows (row_mirror:
// k <-> 15-k) leave every lane with its row's best; the four rows' bests are
// compared in uniform registers.  DPP moves take a few cycles where a
// shuffle through the LDS crossbar takes a round trip, and the k selection
// rounds run this back to back.
__device__ __forceinline__ void wave_argmax(float& v, int& i, float& s) {
  argmax_dpp_step<0xB1>(v, i, s);
  argmax_dpp_step<0x4E>(v, i, s);
  argmax_dpp_step<0x141>(v, i, s);
  argmax_dpp_step<0x140>(v, i, s);
  float bv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  int bi = __builtin_amdgcn_readlane(i, 0);
  float bs = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s), 0));
#pragma unroll
  for (int r = 16; r < kWave; r += 16) {
    const float ov = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), r));
    const int oi = __builtin_amdgcn_readlane(i, r);
    const float os = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s), r));
    if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; bs = os; }
  }
  v = bv; i = bi; s = bs;
}

// splits K at most 16 ways), then summed in split order.
template <int PL>
__global__ __launch_bounds__(256) void gate_select_kernel(
    const float* __restrict__ logits, int splits, const float* __restrict__ bias, int ntok, int E,
    int n_groups, int topk_groups, int topk, int score_softmax, float route_scale,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w) {
  __shared__ float sel[kSelWaves][512];
  __shared__ float gscore[kSelWaves][64];
  __shared__ int gkeep[kSelWaves][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x * kSelWaves + wave;
  const bool active = t < ntok;
  const int tt = active ? t : ntok - 1;

  constexpr int kMaxPerLane = PL;
  constexpr int QR = 64 / PL < 16 ? 64 / PL : 16;   // splits whose loads are in flight together
  float s[kMaxPerLane], sp[kMaxPerLane];
  const float* zrow = logits + (size_t)tt * E;
  const size_t stride = (size_t)ntok * E;
#pragma unroll
  for (int j = 0; j < kMaxPerLane; ++j) s[j] = lane + 64 * j < E ? zrow[lane + 64 * j] : 0.f;
  for (int q0 = 1; q0 < splits; q0 += QR) {  // summed in split order
    float v[QR][kMaxPerLane];
#pragma unroll
    for (int qq = 0; qq < QR; ++qq)
#pragma unroll
      for (int j = 0; j < kMaxPerLane; ++j) {
        const int e = lane + 64 * j;
        v[qq][j] = (q0 + qq < splits && e < E) ? zrow[(size_t)(q0 + qq) * stride + e] : 0.f;
      }
#pragma unroll
    for (int qq = 0; qq < QR; ++qq)
#pragma unroll
      for (int j = 0; j < kMaxPerLane; ++j) s[j] += v[qq][j];
  }
  if (score_softmax) {
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < kMaxPerLane; ++j)
      if (lane + 64 * j < E) m = fmaxf(m, s[j]);
    m = wave_max(m);
    float sum = 0.f;
#pragma unroll
    for (int j = 0; j < kMaxPerLane; ++j) {
      s[j] = lane + 64 * j < E ? expf(s[j] - m) : 0.f;
      sum += s[j];
    }
    sum = wave_sum(sum);
#pragma unroll
    for (int j = 0; j < kMaxPerLane; ++j) s[j] = s[j] / sum;
  } else {
#pragma unroll
    for (int j = 0; j < kMaxPerLane; ++j) s[j] = 1.0f / (1.0f + expf(-s[j]));
  }
#pragma unroll
  for (int j = 0; j < kMaxPerLane; ++j) {
    const int e = lane + 64 * j;
    sp[j] = (bias != nullptr && e < E) ? s[j] + bias[e] : s[j];
  }

  // candidate mask from the group stage
  bool cand[kMaxPerLane];
#pragma unroll
  for (int j = 0; j < kMaxPerLane; ++j) cand[j] = lane + 64 * j < E;
  if (n_groups > 1) {
#pragma unroll
    for (int j = 0; j < kMaxPerLane; ++j)
      if (lane + 64 * j < E) sel[wave][lane + 64 * j] = sp[j];
    __syncthreads();
    const int gsz = E / n_groups;
    if (lane < n_groups) {
      const float* gp = &sel[wave][lane * gsz];
      float gs;
      if (bias != nullptr) {          // sum of the two largest
        float a = -INFINITY, b = -INFINITY;
        for (int i = 0; i < gsz; ++i) {
          const float v = gp[i];
          if (v > a) { b = a; a = v; } else if (v > b) { b = v; }
        }
        gs = a + b;
      } else {
        gs = -INFINITY;
        for (int i = 0; i < gsz; ++i) gs = fmaxf(gs, gp[i]);
      }
      gscore[wave][lane] = gs;
    }
    __syncthreads();
    if (lane < n_groups) {
      const float mine = gscore[wave][lane];
      int rank = 0;
      for (int q = 0; q < n_groups; ++q) {
        const float o = gscore[wave][q];
        rank += (o > mine) || (o == mine && q < lane);
      }
      gkeep[wave][lane] = rank < topk_groups;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kMaxPerLane; ++j) {
      const int e = lane + 64 * j;
      if (e < E) cand[j] = gkeep[wave][e / gsz] != 0;
    }
  }

  // topk rounds of wave arg-max on (s' desc, id asc)
  float wsum = 0.f;
  float my_w = 0.f;
  int my_idx = 0;
  for (int k = 0; k < topk; ++k) {
    float bv = -INFINITY, bs = 0.f;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int j = 0; j < kMaxPerLane; ++j) {
      const int e = lane + 64 * j;
      if (cand[j] && (sp[j] > bv || (sp[j] == bv && e < bi))) { bv = sp[j]; bi = e; bs = s[j]; }
    }
    wave_argmax(bv, bi, bs);
#pragma unroll
    for (int j = 0; j < kMaxPerLane; ++j)
      if (lane + 64 * j == bi) cand[j] = false;
    wsum += bs;
    if (lane == k) { my_w = bs; my_idx = bi; }
  }
  if (active && lane < topk) {
    float w = score_softmax ? my_w : my_w / wsum;
    topk_idx[(size_t)t * topk + lane] = my_idx;
    topk_w[(size_t)t * topk + lane] = w * route_scale;
  }
}

// gate_select_kernel<PL> with PL = ceil(E / 64) rounded up to a power of two
static void launch_select(const float* logits, int splits, const float* bias, int ntok, int E,
                          int n_groups, int topk_groups, int topk, int softmax, float route_scale,
                          int32_t* topk_idx, float* topk_w, hipStream_t st) {
  const int g = (ntok + kSelWaves - 1) / kSelWaves;
  if (E <= 64)
    gate_select_kernel<1><<<g, 256, 0, st>>>(logits, splits, bias, ntok, E, n_groups, topk_groups, topk, softmax, route_scale, topk_idx, topk_w);
  else if (E <= 128)
    gate_select_kernel<2><<<g, 256, 0, st>>>(logits, splits, bias, ntok, E, n_groups, topk_groups, topk, softmax, route_scale, topk_idx, topk_w);
  else if (E <= 256)
    gate_select_kernel<4><<<g, 256, 0, st>>>(logits, splits, bias, ntok, E, n_groups, topk_groups, topk, softmax, route_scale, topk_idx, topk_w);
  else
    gate_select_kernel<8><<<g, 256, 0, st>>>(logits, splits, bias, ntok, E, n_groups, topk_groups, topk, softmax, route_scale, topk_idx, topk_w);
}

hipError_t launch_gate(const void* x, const void* wr, bool f32, const float* bias, int ntok,
                       int dim, int E, int n_groups, int topk_groups, int topk, bool softmax,
                       float route_scale, float* logits, float* rpart, int32_t* topk_idx,
                       float* topk_w, hipStream_t st) {
  if (f32) {
    dim3 g1((ntok + 15) / 16, (E + 15) / 16);
    router_logits_kernel<float><<<g1, 256, 0, st>>>((const float*)x, (const float*)wr, logits,
                                                   ntok, dim, E);
  } else {
    int per = 0;
    const int S = router_splits(ntok, E, dim, &per);
    const size_t n = (size_t)ntok * E;
    dim3 g((ntok + kRtTile - 1) / kRtTile, (E + kRtTile - 1) / kRtTile, S);
    router_mfma_kernel<<<g, 256, 0, st>>>((const uint16_t*)x, (const uint16_t*)wr,
                                          S > 1 ? rpart : logits, ntok, dim, E, per, n);
    if (S > 1) {   // the selection sums the split partials as it reads them
      hipError_t err = hipGetLastError();
      if (err != hipSuccess) return err;
      launch_select(rpart, S, bias, ntok, E, n_groups, topk_groups, topk, softmax ? 1 : 0,
                    route_scale, topk_idx, topk_w, st);
      return hipGetLastError();
    }
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  launch_select(logits, 1, bias, ntok, E, n_groups, topk_groups, topk, softmax ? 1 : 0,
                route_scale, topk_idx, topk_w, st);
  return hipGetLastError();
}

}  // namespace moe
