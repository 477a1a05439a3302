// Weighted combine of the routed expert outputs and the shared expert output,
// shared by the stand-alone combine kernel (combine.hip) and the epilogue of
// the shared expert's down-projection tiles (ffn.hip).
//
// Source: "DeepSeek-V3.2-Exp · Weighted expert sum" (y_routed = sum_i G_i E_i;
// the MoE.forward excerpt keeps the sum in fp32, visits the experts in
// ascending id, adds the shared expert after the routed ones and converts to
// the input dtype once at the end).  Each token reads its topk rows of the
// expert outputs (found through row_of): no atomics, and a fixed order - the
// token's experts in ascending id (ascending row, since rows are
// expert-contiguous), then the shared output - with the product and the sum
// each rounded to fp32 (no fused multiply-add), the page's two-step update.
// The original DeepSeek-V3 class (hackaday.io log "Time to jump right in and
// swim with the big fish", its MoE.forward) keeps the running sum in the layer
// dtype instead: kLayer casts it after every addition.
#pragma once

#include "common.h"

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

// Round to the layer dtype and back (the value a layer-dtype tensor would hold).
template <typename T> __device__ __forceinline__ float to_layer(float v);
template <> __device__ __forceinline__ float to_layer<uint16_t>(float v) {
  return __uint_as_float((uint32_t)f32_to_bf16(v) << 16);
}
template <> __device__ __forceinline__ float to_layer<float>(float v) { return v; }

// Largest topk whose slots are sorted in registers; larger topk sort in LDS.
constexpr int kRegSlots = 8;

// A token's slots (at most kRegSlots) in ascending row order: rows and weights
// in registers, sorted by a fully unrolled exchange network (compile-time
// indices).  Unused slots get row INT_MAX and sort last.
__device__ __forceinline__ void sorted_slots8(const int32_t* __restrict__ rt, const float* __restrict__ wt,
                                              int topk, int (&r)[kRegSlots], float (&w)[kRegSlots]) {
#pragma unroll
  for (int k = 0; k < kRegSlots; ++k) {
    r[k] = k < topk ? rt[k] : 0x7fffffff;
    w[k] = k < topk ? wt[k] : 0.f;
  }
#pragma unroll
  for (int i = 0; i < kRegSlots; ++i)
#pragma unroll
    for (int j = i + 1; j < kRegSlots; ++j)
      if (r[j] < r[i]) {
        const int tr = r[i]; r[i] = r[j]; r[j] = tr;
        const float tw = w[i]; w[i] = w[j]; w[j] = tw;
      }
}

// What the combine reads besides the shared expert's output.
struct CombineArgs {
  const void* out;            // routed expert outputs [T*topk, dim], expert-contiguous rows
  const int32_t* row_of;      // [T, topk] row of assignment (t, k)
  const float* w;             // [T, topk] routing weights
  void* y;                    // [T, dim] layer dtype; NULL = no fused combine
  const int32_t* offsets;     // [E+1], or NULL: only rows [offsets[e_begin], offsets[e_end]) count
  int e_begin, e_end;
  int topk;
  bool layer_acc;             // running sum in the layer dtype (cast after each addition)
};

// y[t, col .. col+7] for one token and 8 columns: the routed sum in ascending
// row order plus the shared values s (already in the layer dtype).  The rows
// and weights come sorted (at most kRegSlots slots).
template <typename T, bool kLayer>
__device__ __forceinline__ void combine8(const CombineArgs& c, int dim, int t, int col,
                                         const int (&rs)[kRegSlots], const float (&ws)[kRegSlots],
                                         const float (&s)[8]) {
#pragma clang fp contract(off)
  const int lo = c.offsets != nullptr ? c.offsets[c.e_begin] : 0;
  const int hi = c.offsets != nullptr ? c.offsets[c.e_end] : 0x7fffffff;
  const T* out = static_cast<const T*>(c.out);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < kRegSlots; ++j) {
    if (j < c.topk && rs[j] >= lo && rs[j] < hi) {
      float v[8];
      Vec8<T>::load(out + (size_t)rs[j] * dim + col, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float a = acc[i] + v[i] * ws[j];   // two roundings (contract off)
        acc[i] = kLayer ? to_layer<T>(a) : a;
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = acc[i] + s[i];
  Vec8<T>::store(static_cast<T*>(c.y) + (size_t)t * dim + col, acc);
}

// The routed sum for one (token, 8 columns) piece, without the store: the
// token's rows are loaded first (all at once), then summed in ascending row.
template <typename T, bool kLayer>
__device__ __forceinline__ void routed8(const CombineArgs& c, int dim, int lo, int hi, int col,
                                        const int (&rs)[kRegSlots], const float (&ws)[kRegSlots],
                                        float (&acc)[8]) {
#pragma clang fp contract(off)
  const T* out = static_cast<const T*>(c.out);
  float v[kRegSlots][8];
#pragma unroll
  for (int j = 0; j < kRegSlots; ++j) {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[j][i] = 0.f;
    if (j < c.topk && rs[j] >= lo && rs[j] < hi) Vec8<T>::load(out + (size_t)rs[j] * dim + col, v[j]);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
#pragma unroll
  for (int j = 0; j < kRegSlots; ++j) {
    if (j < c.topk && rs[j] >= lo && rs[j] < hi) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float a = acc[i] + v[j][i] * ws[j];   // two roundings (contract off)
        acc[i] = kLayer ? to_layer<T>(a) : a;
      }
    }
  }
}

template <typename T>
__device__ __forceinline__ void lds_vals8(const T* sp, float (&s)[8]) {
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    if constexpr (sizeof(T) == 2) s[k] = __uint_as_float((uint32_t)sp[k] << 16);
    else s[k] = sp[k];
  }
}

// The fused epilogue of a shared-expert down tile: the tile's shared outputs
// sit in LDS as layer-dtype values, s_tile[r * ld + j] for token t0 + r and
// column n0 + j; every thread of the workgroup takes (token, 8-column) pieces,
// so the routed rows are read as coalesced 16-byte pieces, two pieces at a
// time so that 2 x kRegSlots row reads are in flight per thread.
template <typename T, bool kLayer>
__device__ __forceinline__ void combine_tile(const CombineArgs& c, const T* s_tile, int ld, int t0,
                                             int rows, int n0, int ncols, int dim) {
#pragma clang fp contract(off)
  const int chunks = ncols >> 3;
  const int items = rows * chunks;
  const int lo = c.offsets != nullptr ? c.offsets[c.e_begin] : 0;
  const int hi = c.offsets != nullptr ? c.offsets[c.e_end] : 0x7fffffff;
  const int step = blockDim.x;
  for (int i = threadIdx.x; i < items; i += 2 * step) {
    const int i2 = i + step;
    const bool two = i2 < items;
    const int ra = i / chunks, ca = i - ra * chunks;
    const int ib = two ? i2 : i;
    const int rb = ib / chunks, cb = ib - rb * chunks;
    int rsa[kRegSlots], rsb[kRegSlots];
    float wsa[kRegSlots], wsb[kRegSlots];
    sorted_slots8(c.row_of + (size_t)(t0 + ra) * c.topk, c.w + (size_t)(t0 + ra) * c.topk, c.topk, rsa, wsa);
    sorted_slots8(c.row_of + (size_t)(t0 + rb) * c.topk, c.w + (size_t)(t0 + rb) * c.topk, c.topk, rsb, wsb);
    float acc_a[8], acc_b[8];
    routed8<T, kLayer>(c, dim, lo, hi, n0 + 8 * ca, rsa, wsa, acc_a);
    routed8<T, kLayer>(c, dim, lo, hi, n0 + 8 * cb, rsb, wsb, acc_b);
    float sa[8], sb[8];
    lds_vals8<T>(s_tile + ra * ld + 8 * ca, sa);
    lds_vals8<T>(s_tile + rb * ld + 8 * cb, sb);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      acc_a[k] = acc_a[k] + sa[k];
      acc_b[k] = acc_b[k] + sb[k];
    }
    Vec8<T>::store(static_cast<T*>(c.y) + (size_t)(t0 + ra) * dim + n0 + 8 * ca, acc_a);
    if (two) Vec8<T>::store(static_cast<T*>(c.y) + (size_t)(t0 + rb) * dim + n0 + 8 * cb, acc_b);
  }
}

}  // namespace moe
