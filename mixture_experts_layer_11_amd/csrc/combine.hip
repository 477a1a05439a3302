// Weighted combine of the expert outputs plus the shared expert.
//
// Source: "DeepSeek-V3.2-Exp · Weighted expert sum" (y_routed = sum_i G_i E_i;
// MoE.forward excerpt: an fp32 accumulator, y[idx] += expert(x[idx]) * weight,
// then the shared expert is added; cast back to the input dtype at the end).
// Gather form: each token reads its topk rows of the expert outputs (found
// through row_of), so there are no atomics and the sum order is fixed: the
// token's experts in ascending id (the page's loop order), then the shared
// output.  Product then add, each rounded to fp32, as the page's two-step
// update does.
// Layer-dtype form (the original DeepSeek-V3 MoE.forward, hackaday.io log
// "Time to jump right in and swim with the big fish": y = zeros_like(x), a loop
// over experts in ascending id doing y[idx] += expert(x[idx]) * weights, then
// y + z): the slots are visited in ascending row - rows are expert-contiguous,
// so that is ascending expert id - and the running sum is cast to the layer
// dtype after every addition.
#include "common.h"
#include "kernels.h"

// The page's update rounds the product and then the sum: no fused multiply-add
// anywhere in this file (the compiler would otherwise contract them).
#pragma clang fp contract(off)

namespace moe {

template <typename T> struct Vec8;
template <> struct Vec8<uint16_t> {
  __device__ __forceinline__ static void load(const uint16_t* p, float (&v)[8]) {
    const uint4 u = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
  __device__ __forceinline__ static void store(uint16_t* p, const float (&v)[8]) {
    uint4 u;
    u.x = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
    u.y = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
    u.z = (uint32_t)f32_to_bf16(v[4]) | ((uint32_t)f32_to_bf16(v[5]) << 16);
    u.w = (uint32_t)f32_to_bf16(v[6]) | ((uint32_t)f32_to_bf16(v[7]) << 16);
    *reinterpret_cast<uint4*>(p) = u;
  }
};
template <> struct Vec8<float> {
  __device__ __forceinline__ static void load(const float* p, float (&v)[8]) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  __device__ __forceinline__ static void store(float* p, const float (&v)[8]) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
  }
};

// A token's slots in ascending row order (rows are expert-contiguous, so this
// is ascending expert id): the rows and weights of at most KMAX slots are
// loaded into registers and sorted by a fully unrolled exchange network
// (compile-time indices, so nothing leaves the registers).  Unused slots get
// row INT_MAX and sort last.
template <int KMAX>
__device__ __forceinline__ void sorted_slots(const int32_t* __restrict__ rt, const float* __restrict__ wt,
                                             int topk, int (&r)[KMAX], float (&w)[KMAX]) {
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    r[k] = k < topk ? rt[k] : 0x7fffffff;
    w[k] = k < topk ? wt[k] : 0.f;
  }
#pragma unroll
  for (int i = 0; i < KMAX; ++i)
#pragma unroll
    for (int j = i + 1; j < KMAX; ++j)
      if (r[j] < r[i]) {
        const int tr = r[i]; r[i] = r[j]; r[j] = tr;
        const float tw = w[i]; w[i] = w[j]; w[j] = tw;
      }
}

template <typename T> __device__ __forceinline__ float to_layer(float v);
template <> __device__ __forceinline__ float to_layer<uint16_t>(float v) {
  return __uint_as_float((uint32_t)f32_to_bf16(v) << 16);
}
template <> __device__ __forceinline__ float to_layer<float>(float v) { return v; }

// kLayer = false: fp32 running sum, one cast at the end; true: the running
// sum is cast to the layer dtype after every addition.
template <typename T, int KMAX, bool kLayer>
__global__ __launch_bounds__(256) void combine_kernel(const T* __restrict__ out,
                                                      const int32_t* __restrict__ row_of,
                                                      const float* __restrict__ w,
                                                      const T* __restrict__ shared_out,
                                                      T* __restrict__ y, int dim, int topk,
                                                      const int32_t* __restrict__ offsets,
                                                      int e_begin, int e_end) {
  const int t = blockIdx.x;
  const int col = (blockIdx.y * blockDim.x + threadIdx.x) * 8;
  if (col >= dim) return;
  // rows of the expert range (all rows without offsets)
  const int lo = offsets != nullptr ? offsets[e_begin] : 0;
  const int hi = offsets != nullptr ? offsets[e_end] : 0x7fffffff;
  int rs[KMAX];
  float ws[KMAX];
  sorted_slots<KMAX>(row_of + (size_t)t * topk, w + (size_t)t * topk, topk, rs, ws);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    if (j < topk && rs[j] >= lo && rs[j] < hi) {
      float v[8];
      Vec8<T>::load(out + (size_t)rs[j] * dim + col, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float a = acc[i] + v[i] * ws[j];   // two roundings (contract off)
        acc[i] = kLayer ? to_layer<T>(a) : a;
      }
    }
  }
  if (shared_out != nullptr) {
    float v[8];
    Vec8<T>::load(shared_out + (size_t)t * dim + col, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = acc[i] + v[i];
  }
  Vec8<T>::store(y + (size_t)t * dim + col, acc);
}

template <typename T, bool kLayer>
static void launch_combine_t(dim3 grid, hipStream_t st, const void* out, const int32_t* row_of,
                             const float* w, const void* shared_out, void* y, int dim, int topk,
                             const int32_t* offsets, int eb, int ee) {
  if (topk <= 8)
    combine_kernel<T, 8, kLayer><<<grid, 256, 0, st>>>((const T*)out, row_of, w, (const T*)shared_out,
                                                       (T*)y, dim, topk, offsets, eb, ee);
  else
    combine_kernel<T, kMaxTopk, kLayer><<<grid, 256, 0, st>>>((const T*)out, row_of, w,
                                                              (const T*)shared_out, (T*)y, dim, topk,
                                                              offsets, eb, ee);
}

hipError_t launch_combine(const void* expert_out, const int32_t* row_of, const float* topk_w,
                          const void* shared_out, void* y, int ntok, int dim, int topk,
                          bool act_f32, bool layer_acc, const int32_t* offsets, int eb, int ee,
                          hipStream_t st) {
  dim3 grid(ntok, (dim / 8 + 255) / 256);
  const void* o = expert_out;
  if (act_f32 && layer_acc) launch_combine_t<float, true>(grid, st, o, row_of, topk_w, shared_out, y, dim, topk, offsets, eb, ee);
  else if (act_f32) launch_combine_t<float, false>(grid, st, o, row_of, topk_w, shared_out, y, dim, topk, offsets, eb, ee);
  else if (layer_acc) launch_combine_t<uint16_t, true>(grid, st, o, row_of, topk_w, shared_out, y, dim, topk, offsets, eb, ee);
  else launch_combine_t<uint16_t, false>(grid, st, o, row_of, topk_w, shared_out, y, dim, topk, offsets, eb, ee);
  return hipGetLastError();
}

}  // namespace moe
