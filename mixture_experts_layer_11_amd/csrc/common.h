// Shared device helpers for the MoE kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(8))) int i32x8_t;

constexpr int kWave = 64;

// ---- number formats -------------------------------------------------------

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// fp32 -> OCP e4m3fn code, round to nearest even, saturating to +-448.
// Normal range: round the fp32 mantissa to 3 bits and rebias the exponent
// (127 -> 7); below 2^-6 the spacing is 2^-9, so round |v| * 2^9 to an
// integer (exact scaling, then RNE).
__device__ __forceinline__ uint8_t f32_to_e4m3(float v) {
  uint32_t u = __float_as_uint(v);
  uint32_t sign = (u >> 24) & 0x80u;
  uint32_t mag = u & 0x7FFFFFFFu;
  int code;
  if (mag < 0x3C800000u) {                       // |v| < 2^-6
    code = static_cast<int>(__builtin_rintf(__uint_as_float(mag) * 512.0f));
  } else {
    uint32_t r = (mag + 0x7FFFFu + ((mag >> 20) & 1u)) >> 20;
    code = static_cast<int>(r) - (120 << 3);
  }
  code = code > 0x7E ? 0x7E : code;
  return static_cast<uint8_t>(code == 0 ? 0 : (code | sign));
}

// silu(a) = a * sigmoid(a), with the hardware reciprocal (about 1 ulp) in place
// of an IEEE division: the result is rounded to bf16 or e4m3 next.  exp(-a)
// overflowing to inf gives a * 0, the limit.
__device__ __forceinline__ float silu(float a) { return a * __builtin_amdgcn_rcpf(1.0f + __expf(-a)); }

// ---- wave reductions ------------------------------------------------------

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// ---- MFMA on 64-byte k-chunks ----------------------------------------------
// A "chunk" is 64 contiguous bytes of a K-contiguous row: lane group
// g = lane/16 holds bytes [16g, 16g+16).  Rows of the A operand are lane%16,
// columns of the B operand are lane%16.  Both operands use the same k
// assignment, so the dot product covers the whole chunk.
//   bf16: 32 elements -> one v_mfma_f32_16x16x32_bf16
//   f32 : 16 elements -> four v_mfma_f32_16x16x4_f32 (element j of each group)
// Result lane layout (16x16): D[row = 4*(lane/16) + i][col = lane%16], i<4.

template <typename T> struct Chunk;

template <> struct Chunk<uint16_t> {
  static constexpr int kElems = 32;
  __device__ __forceinline__ static f32x4_t mma(f32x4_t c, uint4 a, uint4 b) {
    bf16x8_t av = __builtin_bit_cast(bf16x8_t, a);
    bf16x8_t bv = __builtin_bit_cast(bf16x8_t, b);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, c, 0, 0, 0);
  }
};

template <> struct Chunk<float> {
  static constexpr int kElems = 16;
  __device__ __forceinline__ static f32x4_t mma(f32x4_t c, uint4 a, uint4 b) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
    return c;
  }
};

__device__ __forceinline__ uint4 ldg16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// Non-temporal 16-byte load, for data read once (expert weights in the decode
// kernels): streaming reads this way run at 7.0-7.3 TB/s on MI355X against
// 6.2-6.5 TB/s for ordinary loads.
typedef unsigned int u32x4_nt_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ldg16_stream(const void* p) {
  const u32x4_nt_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Physical workgroup id -> logical tile id so that consecutive logical tiles
// run on the same XCD (the dispatcher places workgroup i on XCD i % 8).
// `n` must be a multiple of 8.
__device__ __forceinline__ int xcd_remap(int pid, int n) {
  return (pid & 7) * (n >> 3) + (pid >> 3);
}

}  // namespace moe
