// Dispatch: expert-contiguous order of the (token, slot) assignments.
//
// Source: "DeepSeek-V3.2-Exp · Weighted expert sum", MoE.forward excerpt: a
// bincount of the chosen indices, then per expert the (token, slot) pairs in
// the row-major order torch.where yields.  Here: a blocked counting sort.
//   count  : per block of kPermBlock tokens, per-expert counts (LDS atomics;
//            the totals do not depend on their order)
//   scan   : per expert, exclusive prefix over blocks; then exclusive prefix
//            over experts -> counts, offsets, and each block's base row
//   scatter: per block, one thread per expert walks the block's tokens in
//            ascending order and hands out consecutive rows
// No step depends on the order of atomics, so the result is bit-exact.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kPermBlock = 64;   // tokens per block

__global__ __launch_bounds__(256) void permute_count_kernel(const int32_t* __restrict__ idx,
                                                            int ntok, int topk, int E,
                                                            int32_t* __restrict__ blk_count) {
  __shared__ int hist[kMaxExperts];
  for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
  __syncthreads();
  const int t0 = blockIdx.x * kPermBlock;
  const int n = min(kPermBlock, ntok - t0) * topk;
  const int32_t* p = idx + (size_t)t0 * topk;
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const int e = p[i];
    if (e >= 0 && e < E) atomicAdd(&hist[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) blk_count[(size_t)blockIdx.x * E + e] = hist[e];
}

// single workgroup of 1024 threads (E <= kMaxExperts <= 1024)
__global__ __launch_bounds__(1024) void permute_scan_kernel(int32_t* __restrict__ blk_count,
                                                            int nblk, int E,
                                                            int32_t* __restrict__ counts,
                                                            int32_t* __restrict__ offsets) {
  __shared__ int buf[1024];
  const int e = threadIdx.x;
  int total = 0;
  if (e < E) {
    for (int b = 0; b < nblk; ++b) {
      const int c = blk_count[(size_t)b * E + e];
      blk_count[(size_t)b * E + e] = total;     // exclusive prefix over blocks
      total += c;
    }
  }
  buf[e] = e < E ? total : 0;
  __syncthreads();
  // inclusive Hillis-Steele scan over experts
  for (int o = 1; o < 1024; o <<= 1) {
    const int v = e >= o ? buf[e - o] : 0;
    __syncthreads();
    buf[e] += v;
    __syncthreads();
  }
  if (e < E) {
    const int excl = buf[e] - total;
    counts[e] = total;
    offsets[e] = excl;
    for (int b = 0; b < nblk; ++b) blk_count[(size_t)b * E + e] += excl;   // block base rows
    if (e == E - 1) offsets[E] = buf[e];
  }
}

__global__ __launch_bounds__(256) void permute_scatter_kernel(
    const int32_t* __restrict__ idx, int ntok, int topk, int E,
    const int32_t* __restrict__ blk_base, int32_t* __restrict__ sorted_token,
    int32_t* __restrict__ row_of) {
  __shared__ int32_t sidx[kPermBlock * kMaxTopk];
  const int t0 = blockIdx.x * kPermBlock;
  const int nt = min(kPermBlock, ntok - t0);
  const int32_t* p = idx + (size_t)t0 * topk;
  for (int i = threadIdx.x; i < nt * topk; i += blockDim.x) sidx[i] = p[i];
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int pos = blk_base[(size_t)blockIdx.x * E + e];
    for (int t = 0; t < nt; ++t) {
      for (int k = 0; k < topk; ++k) {
        if (sidx[t * topk + k] == e) {
          sorted_token[pos] = t0 + t;
          row_of[(size_t)(t0 + t) * topk + k] = pos;
          ++pos;
        }
      }
    }
  }
}

size_t permute_scratch_bytes(int ntok, int E) {
  const size_t nblk = (size_t)(ntok + kPermBlock - 1) / kPermBlock;
  return nblk * (size_t)E * sizeof(int32_t);
}

hipError_t launch_permute(const int32_t* idx, int ntok, int topk, int E, int32_t* counts,
                          int32_t* offsets, int32_t* sorted_token, int32_t* row_of,
                          int32_t* scratch, hipStream_t st) {
  const int nblk = (ntok + kPermBlock - 1) / kPermBlock;
  permute_count_kernel<<<nblk, 256, 0, st>>>(idx, ntok, topk, E, scratch);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  permute_scan_kernel<<<1, 1024, 0, st>>>(scratch, nblk, E, counts, offsets);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  permute_scatter_kernel<<<nblk, 256, 0, st>>>(idx, ntok, topk, E, scratch, sorted_token, row_of);
  return hipGetLastError();
}

}  // namespace moe
