// Expert weights into the tiled layout the FFN kernels read: 16-row x
// 64-byte tiles of 1 KB, each the 64 16-byte pieces in wave-lane order
// (piece (row%16) + 16 * (column chunk%4)).  One thread moves one 16-byte
// piece; destination writes are contiguous.
#include "common.h"
#include "kernels.h"

namespace moe {

__global__ __launch_bounds__(256) void pack_weights_kernel(const uint8_t* __restrict__ src,
                                                            int64_t rows, int64_t row_bytes,
                                                            uint8_t* __restrict__ dst) {
  const int64_t pieces = rows * (row_bytes / 16);
  const int64_t chunks = row_bytes / 64;   // 64-byte chunks per row = tiles per row tile
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < pieces;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t tile = t >> 6;
    const int piece = (int)(t & 63);
    const int64_t row = (tile / chunks) * 16 + (piece & 15);
    const int64_t byte = (tile % chunks) * 64 + 16 * (piece >> 4);
    *reinterpret_cast<uint4*>(dst + 16 * t) =
        *reinterpret_cast<const uint4*>(src + row * row_bytes + byte);
  }
}

hipError_t launch_pack_weights(const uint8_t* src, int64_t rows, int64_t row_bytes, uint8_t* dst,
                               hipStream_t st) {
  const int64_t pieces = rows * (row_bytes / 16);
  const int64_t blocks = (pieces + 255) / 256;
  pack_weights_kernel<<<(int)(blocks < 65536 ? blocks : 65536), 256, 0, st>>>(src, rows, row_bytes, dst);
  return hipGetLastError();
}

}  // namespace moe
