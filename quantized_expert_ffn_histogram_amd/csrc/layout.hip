// Conversion of packed 4-bit codes from row-major [rows][K/2] to the tiled
// layout the kernels also read (packed_offset): the bytes of one 128-wide K
// stage of a 32-row weight block become one contiguous 2 KB run, so the
// grouped GEMM's per-stage weight loads use whole 128-byte lines instead of
// the half lines of a row-major stage (64 bytes of each row), whose other
// half is evicted before the next stage asks for it.
//
// A pure permutation of bytes, done once when the weights are loaded.
#include "moe_internal.h"

namespace strata {
namespace {

// Thread i writes destination bytes [16i, 16i + 16): row r of its tile, 16
// bytes c of the row's 64.  Grid-stride over the 16-byte units.
__global__ __launch_bounds__(256) void tile_weights_kernel(const uint4 *__restrict__ src, uint4 *__restrict__ dst,
                                                           size_t units, uint32_t rb) {
  const uint32_t tiles_per_block = rb >> 6;
  for (size_t u = (size_t)blockIdx.x * 256 + threadIdx.x; u < units; u += (size_t)gridDim.x * 256) {
    const size_t tile = u >> 7;                        // 2048-byte tiles
    const uint32_t r = (uint32_t)(u >> 2) & 31u, c = (uint32_t)u & 3u;
    const size_t blk = tile / tiles_per_block, j = tile % tiles_per_block;
    const size_t off = (blk * 32 + r) * rb + j * 64 + c * 16;  // row-major source offset
    dst[u] = src[off >> 4];
  }
}

}  // namespace

hipError_t launch_tile_weights(const uint8_t *src, uint8_t *dst, long long rows, int K, hipStream_t s) {
  const size_t units = (size_t)rows * (size_t)(K / 2) / 16;
  if (units == 0) return hipSuccess;
  const size_t want = (units + 255) / 256;
  const int grid = (int)(want < 16384 ? want : 16384);
  tile_weights_kernel<<<grid, 256, 0, s>>>(reinterpret_cast<const uint4 *>(src), reinterpret_cast<uint4 *>(dst),
                                           units, (uint32_t)(K / 2));
  return hipGetLastError();
}

}  // namespace strata
