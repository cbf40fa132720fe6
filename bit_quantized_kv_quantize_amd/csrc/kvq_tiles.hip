// kvq_tiles.hip - whole-block copies between pools: the device side of saving and restoring quantised
// blocks ("Agent Memory Below the Prompt", technical summary 2.1: blocks persisted and reloaded as they
// are stored; QKVShare methodology: the CacheCard handed to another agent). A tile is position independent
// (it holds only its own rows' codes, parameters and width bitmap), so moving it is a plain byte copy.
#include "kvq_internal.hpp"

namespace kvq {
namespace {

// Grid (n_blocks, H): workgroup (i, h) copies tile (src_ids[i], h) of src to tile (dst_ids[i], h) of dst,
// 16 bytes per thread per step (tile sizes are multiples of 256 bytes).
__global__ __launch_bounds__(256) void copy_blocks_k(uint32_t tile_bytes, int H, const uint8_t* __restrict__ src,
                                                    const int32_t* __restrict__ src_ids, uint8_t* __restrict__ dst,
                                                    const int32_t* __restrict__ dst_ids) {
  const int i = blockIdx.x, h = blockIdx.y;
  const uint4* s = reinterpret_cast<const uint4*>(src + ((size_t)src_ids[i] * H + h) * tile_bytes);
  uint4* d = reinterpret_cast<uint4*>(dst + ((size_t)dst_ids[i] * H + h) * tile_bytes);
  for (uint32_t k = threadIdx.x; k < tile_bytes / 16; k += 256) d[k] = s[k];
}

}  // namespace

hipError_t launch_copy_blocks(const TileGeom& g, const uint8_t* src, const int32_t* src_ids, uint8_t* dst,
                              const int32_t* dst_ids, int n_blocks, hipStream_t stream) {
  hipLaunchKernelGGL(copy_blocks_k, dim3(n_blocks, g.H), dim3(256), 0, stream, g.tile_bytes, g.H, src, src_ids, dst,
                     dst_ids);
  return hipGetLastError();
}

}  // namespace kvq
