// Stand-alone weighted combine: y = cast(sum_k w O[row_of] + S) for layers
// whose combine is not fused into the shared expert's down projection (no
// shared expert, more than kRegSlots experts per token, or a shared output
// computed elsewhere).  The arithmetic and its order are those of combine.h.
#include "combine.h"
#include "kernels.h"

namespace moe {

// One workgroup per (token, 2048 columns): 256 threads of 8 columns each.
// Up to kRegSlots slots are sorted in registers by every thread; more slots
// (topk up to kMaxTopk) are ranked once per workgroup in LDS - slot k's rank
// is the number of the token's rows below its own (rows are distinct) - and
// read back in rank order.
template <typename T, bool kLds>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs c, const T* __restrict__ shared_out,
                                                      int dim) {
  const int t = blockIdx.x;
  const int col = (blockIdx.y * blockDim.x + threadIdx.x) * 8;
  float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if constexpr (!kLds) {
    if (col >= dim) return;
    int rs[kRegSlots];
    float ws[kRegSlots];
    sorted_slots8(c.row_of + (size_t)t * c.topk, c.w + (size_t)t * c.topk, c.topk, rs, ws);
    if (shared_out != nullptr) Vec8<T>::load(shared_out + (size_t)t * dim + col, s);
    if (c.layer_acc) combine8<T, true>(c, dim, t, col, rs, ws, s);
    else combine8<T, false>(c, dim, t, col, rs, ws, s);
  } else {
#pragma clang fp contract(off)
    __shared__ int srow[kMaxTopk];
    __shared__ float sw[kMaxTopk];
    const int k = threadIdx.x;
    if (k < c.topk) {
      const int* rt = c.row_of + (size_t)t * c.topk;
      const int mine = rt[k];
      int rank = 0;
      for (int j = 0; j < c.topk; ++j) rank += rt[j] < mine ? 1 : 0;
      srow[rank] = mine;
      sw[rank] = c.w[(size_t)t * c.topk + k];
    }
    __syncthreads();
    if (col >= dim) return;
    const int lo = c.offsets != nullptr ? c.offsets[c.e_begin] : 0;
    const int hi = c.offsets != nullptr ? c.offsets[c.e_end] : 0x7fffffff;
    const T* out = static_cast<const T*>(c.out);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < c.topk; ++j) {
      const int r = srow[j];
      if (r < lo || r >= hi) continue;
      const float w = sw[j];
      float v[8];
      Vec8<T>::load(out + (size_t)r * dim + col, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float a = acc[i] + v[i] * w;       // two roundings (contract off)
        acc[i] = c.layer_acc ? to_layer<T>(a) : a;
      }
    }
    if (shared_out != nullptr) Vec8<T>::load(shared_out + (size_t)t * dim + col, s);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = acc[i] + s[i];
    Vec8<T>::store(static_cast<T*>(c.y) + (size_t)t * dim + col, acc);
  }
}

hipError_t launch_combine(const CombineArgs& c, const void* shared_out, int ntok, int dim,
                          bool act_f32, hipStream_t st) {
  dim3 grid(ntok, (dim / 8 + 255) / 256);
  const bool lds = c.topk > kRegSlots;
  if (act_f32 && lds) combine_kernel<float, true><<<grid, 256, 0, st>>>(c, (const float*)shared_out, dim);
  else if (act_f32) combine_kernel<float, false><<<grid, 256, 0, st>>>(c, (const float*)shared_out, dim);
  else if (lds) combine_kernel<uint16_t, true><<<grid, 256, 0, st>>>(c, (const uint16_t*)shared_out, dim);
  else combine_kernel<uint16_t, false><<<grid, 256, 0, st>>>(c, (const uint16_t*)shared_out, dim);
  return hipGetLastError();
}

}  // namespace moe
