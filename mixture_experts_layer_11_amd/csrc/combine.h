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
  using Raw = uint4;   // 8 values as loaded
  __device__ __forceinline__ static Raw load_raw(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ static Raw zero() { return make_uint4(0u, 0u, 0u, 0u); }
  __device__ __forceinline__ static void unpack(const Raw& u, float (&v)[8]) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
  __device__ __forceinline__ static void load(const uint16_t* p, float (&v)[8]) { unpack(load_raw(p), v); }
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
  struct Raw { float4 a, b; };
  __device__ __forceinline__ static Raw load_raw(const float* p) {
    return Raw{*reinterpret_cast<const float4*>(p), *reinterpret_cast<const float4*>(p + 4)};
  }
  __device__ __forceinline__ static Raw zero() {
    return Raw{make_float4(0.f, 0.f, 0.f, 0.f), make_float4(0.f, 0.f, 0.f, 0.f)};
  }
  __device__ __forceinline__ static void unpack(const Raw& u, float (&v)[8]) {
    v[0] = u.a.x; v[1] = u.a.y; v[2] = u.a.z; v[3] = u.a.w; v[4] = u.b.x; v[5] = u.b.y; v[6] = u.b.z; v[7] = u.b.w;
  }
  __device__ __forceinline__ static void load(const float* p, float (&v)[8]) { unpack(load_raw(p), v); }
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

// The routing of a combine tile's tokens, staged in LDS: kRegSlots slots per
// token in ascending row, rows that do not count (past topk, or outside the
// expert range) marked kNoRow so they sort last and are skipped.
constexpr int32_t kNoRow = 0x7fffffff;
struct __attribute__((aligned(8))) Slot {
  int32_t row;
  float w;
};

// A token's raw routing (row_of and weights) in registers, loaded by thread r
// of the workgroup for token t0 + r; stored to LDS sorted by slots_store.
struct SlotLoad {
  int32_t r[kRegSlots];
  float w[kRegSlots];
};

__device__ __forceinline__ void slots_issue(const CombineArgs& c, int t0, int rows, SlotLoad& L) {
  const int r = threadIdx.x;
#pragma unroll
  for (int k = 0; k < kRegSlots; ++k) {
    const bool ld = r < rows && k < c.topk;
    L.r[k] = ld ? c.row_of[(size_t)(t0 + r) * c.topk + k] : kNoRow;
    L.w[k] = ld ? c.w[(size_t)(t0 + r) * c.topk + k] : 0.f;
  }
}

// Sort thread r's slots by row (a fully unrolled exchange network) and store
// them as token r's LDS slots; the caller's next workgroup barrier publishes
// them.  Requires rows <= blockDim.x.
__device__ __forceinline__ void slots_store(const CombineArgs& c, int rows, SlotLoad L, Slot* slots) {
  const int r = threadIdx.x;
  if (r >= rows) return;
  const int lo = c.offsets != nullptr ? c.offsets[c.e_begin] : 0;
  const int hi = c.offsets != nullptr ? c.offsets[c.e_end] : kNoRow;
#pragma unroll
  for (int k = 0; k < kRegSlots; ++k)
    if (L.r[k] < lo || L.r[k] >= hi) L.r[k] = kNoRow;
#pragma unroll
  for (int i = 0; i < kRegSlots; ++i)
#pragma unroll
    for (int j = i + 1; j < kRegSlots; ++j)
      if (L.r[j] < L.r[i]) {
        const int tr = L.r[i]; L.r[i] = L.r[j]; L.r[j] = tr;
        const float tw = L.w[i]; L.w[i] = L.w[j]; L.w[j] = tw;
      }
  int4* d = reinterpret_cast<int4*>(slots + r * kRegSlots);
#pragma unroll
  for (int k = 0; k < kRegSlots; k += 2)
    d[k / 2] = make_int4(L.r[k], __float_as_int(L.w[k]), L.r[k + 1], __float_as_int(L.w[k + 1]));
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
// column n0 + j, and the tokens' sorted slots in LDS (slots_store).  Every
// thread of the workgroup takes (token, 8-column) pieces, NP at a time: the
// routed rows of all NP pieces are loaded first (NP x kRegSlots coalesced
// 16-byte reads in flight per thread), then each piece is summed in ascending
// row, its shared value added last, and stored.
template <typename T, bool kLayer, int NP>
__device__ __forceinline__ void combine_tile(const CombineArgs& c, const Slot* slots, const T* s_tile, int ld,
                                             int t0, int rows, int n0, int ncols, int dim) {
#pragma clang fp contract(off)
  const int chunks = ncols >> 3;
  const int items = rows * chunks;
  const int step = blockDim.x;
  const T* out = static_cast<const T*>(c.out);
  for (int i0 = threadIdx.x; i0 < items; i0 += NP * step) {
    int pr[NP], pc[NP];
    uint32_t used[NP];            // bit k: slot k holds a routed row of the sum
    float ws[NP][kRegSlots];
    typename Vec8<T>::Raw v[NP][kRegSlots];
#pragma unroll
    for (int q = 0; q < NP; ++q) {
      const int i = i0 + q * step;
      const bool live = i < items;
      const int ii = live ? i : i0;
      pr[q] = ii / chunks;
      pc[q] = ii - pr[q] * chunks;
      used[q] = 0u;
      const int4* sl = reinterpret_cast<const int4*>(slots + pr[q] * kRegSlots);
#pragma unroll
      for (int k = 0; k < kRegSlots; k += 2) {
        const int4 e = sl[k / 2];
        const int rr[2] = {e.x, e.z};
        ws[q][k] = __int_as_float(e.y);
        ws[q][k + 1] = __int_as_float(e.w);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          if (live && rr[h] != kNoRow) {
            v[q][k + h] = Vec8<T>::load_raw(out + (size_t)rr[h] * dim + n0 + 8 * pc[q]);
            used[q] |= 1u << (k + h);
          } else {
            v[q][k + h] = Vec8<T>::zero();
          }
        }
      }
    }
#pragma unroll
    for (int q = 0; q < NP; ++q) {
      if (i0 + q * step >= items) continue;
      float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < kRegSlots; ++k) {
        if (!(used[q] & (1u << k))) continue;
        float x[8];
        Vec8<T>::unpack(v[q][k], x);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float a = acc[e] + x[e] * ws[q][k];   // two roundings (contract off)
          acc[e] = kLayer ? to_layer<T>(a) : a;
        }
      }
      float sv[8];
      lds_vals8<T>(s_tile + pr[q] * ld + 8 * pc[q], sv);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = acc[e] + sv[e];
      Vec8<T>::store(static_cast<T*>(c.y) + (size_t)(t0 + pr[q]) * dim + n0 + 8 * pc[q], acc);
    }
  }
}

}  // namespace moe
