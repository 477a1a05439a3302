// Dispatch: expert-contiguous order of the (token, slot) assignments.
//
// Source: "DeepSeek-V3.2-Exp · Weighted expert sum", MoE.forward excerpt: a
// bincount of the chosen indices, then per expert the (token, slot) pairs in
// the row-major order torch.where yields.  Here: a blocked counting sort.
//   count  : per block of kPermBlock tokens, per-expert bit masks of the
//            block's tokens (LDS atomic OR), counted by popcount
//   scan   : per expert, exclusive prefix over blocks; then exclusive prefix
//            over experts -> counts, offsets, and each block's base row
//   scatter: per block, a bit mask per expert of the block's tokens that
//            chose it (LDS atomic OR); the row of assignment (t, k) to expert
//            e is the block base of e plus the number of earlier tokens of the
//            block in e's mask (a token picks an expert at most once, so this
//            is its rank in row-major order)
// No step depends on the order of atomics, so the result is bit-exact.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kPermBlock = 256;   // tokens per block
constexpr int kPermWords = kPermBlock / 64;   // 64-bit mask words per expert

__global__ __launch_bounds__(256) void permute_count_kernel(const int32_t* __restrict__ idx,
                                                            int ntok, int topk, int E,
                                                            int32_t* __restrict__ blk_count) {
  // per-expert bit masks of the block's tokens (the scatter builds the same
  // masks), counted by popcount: a repeated id in a row counts once
  __shared__ unsigned long long mask[kMaxExperts][kPermWords];
  for (int i = threadIdx.x; i < E * kPermWords; i += blockDim.x) (&mask[0][0])[i] = 0ull;
  __syncthreads();
  const int t0 = blockIdx.x * kPermBlock;
  const int n = min(kPermBlock, ntok - t0) * topk;
  const int32_t* p = idx + (size_t)t0 * topk;
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const int e = p[i], t = i / topk;
    if (e >= 0 && e < E) atomicOr(&mask[e][t >> 6], 1ull << (t & 63));
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int c = 0;
#pragma unroll
    for (int w = 0; w < kPermWords; ++w) c += __popcll(mask[e][w]);
    blk_count[(size_t)blockIdx.x * E + e] = c;
  }
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
    for (int b0 = 0; b0 < nblk; b0 += 8) {      // 8 independent loads in flight
      int c[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) c[j] = b0 + j < nblk ? blk_count[(size_t)(b0 + j) * E + e] : 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (b0 + j < nblk) blk_count[(size_t)(b0 + j) * E + e] = total;   // exclusive prefix over blocks
        total += c[j];
      }
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
  __shared__ unsigned long long mask[kMaxExperts][kPermWords];
  for (int i = threadIdx.x; i < E * kPermWords; i += blockDim.x) (&mask[0][0])[i] = 0ull;
  __syncthreads();
  const int t0 = blockIdx.x * kPermBlock;
  const int n = min(kPermBlock, ntok - t0) * topk;
  const int32_t* p = idx + (size_t)t0 * topk;
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const int e = p[i], t = i / topk;
    if (e >= 0 && e < E) atomicOr(&mask[e][t >> 6], 1ull << (t & 63));
  }
  __syncthreads();
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const int e = p[i], t = i / topk, k = i - t * topk;
    if (e < 0 || e >= E) continue;
    int rank = __popcll(mask[e][t >> 6] & ((1ull << (t & 63)) - 1ull));
    for (int w = 0; w < (t >> 6); ++w) rank += __popcll(mask[e][w]);
    const int pos = blk_base[(size_t)blockIdx.x * E + e] + rank;
    sorted_token[pos] = t0 + t;
    row_of[(size_t)(t0 + t) * topk + k] = pos;
  }
}

// All three steps in one workgroup when the tokens fit one block (decode):
// the same counting sort without the block-count round trip through global
// memory and without two launches.
__global__ __launch_bounds__(1024) void permute_one_block_kernel(const int32_t* __restrict__ idx,
                                                                 int ntok, int topk, int E,
                                                                 int32_t* __restrict__ counts,
                                                                 int32_t* __restrict__ offsets,
                                                                 int32_t* __restrict__ sorted_token,
                                                                 int32_t* __restrict__ row_of) {
  __shared__ int buf[1024];
  __shared__ int base[kMaxExperts];
  __shared__ unsigned long long mask[kMaxExperts][kPermWords];
  const int tid = threadIdx.x;
  for (int i = tid; i < E * kPermWords; i += blockDim.x) (&mask[0][0])[i] = 0ull;
  __syncthreads();
  const int n = ntok * topk;
  for (int i = tid; i < n; i += blockDim.x) {
    const int e = idx[i], t = i / topk;
    if (e >= 0 && e < E) atomicOr(&mask[e][t >> 6], 1ull << (t & 63));
  }
  __syncthreads();
  // per-expert count = popcount of its mask; exclusive scan over experts
  int total = 0;
  if (tid < E)
    for (int w = 0; w < kPermWords; ++w) total += __popcll(mask[tid][w]);
  buf[tid] = tid < E ? total : 0;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int v = tid >= o ? buf[tid - o] : 0;
    __syncthreads();
    buf[tid] += v;
    __syncthreads();
  }
  if (tid < E) {
    base[tid] = buf[tid] - total;
    counts[tid] = total;
    offsets[tid] = buf[tid] - total;
    if (tid == E - 1) offsets[E] = buf[tid];
  }
  __syncthreads();
  for (int i = tid; i < n; i += blockDim.x) {
    const int e = idx[i], t = i / topk, k = i - t * topk;
    if (e < 0 || e >= E) continue;
    int rank = __popcll(mask[e][t >> 6] & ((1ull << (t & 63)) - 1ull));
    for (int w = 0; w < (t >> 6); ++w) rank += __popcll(mask[e][w]);
    const int pos = base[e] + rank;
    sorted_token[pos] = t;
    row_of[(size_t)t * topk + k] = pos;
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
  if (nblk == 1) {
    permute_one_block_kernel<<<1, 1024, 0, st>>>(idx, ntok, topk, E, counts, offsets, sorted_token,
                                                 row_of);
    return hipGetLastError();
  }
  permute_count_kernel<<<nblk, 256, 0, st>>>(idx, ntok, topk, E, scratch);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  permute_scan_kernel<<<1, 1024, 0, st>>>(scratch, nblk, E, counts, offsets);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  permute_scatter_kernel<<<nblk, 256, 0, st>>>(idx, ntok, topk, E, scratch, sorted_token, row_of);
  return hipGetLastError();
}

}  // namespace moe
