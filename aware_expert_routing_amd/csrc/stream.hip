// Read-only HBM stream (moe_read_stream): the achievable read rate of this
// GPU for a plain contiguous scan, against which the expert FFN's streaming
// rate is judged. Each workgroup reads a contiguous block with 16-byte loads,
// 8 per thread in flight, folds the words with XOR (so no load can be
// removed) and writes one word.
#include "moe_internal.h"

namespace moe {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void read_stream_kernel(const u32x4_t *__restrict__ src, size_t n16,
                                                          uint32_t *__restrict__ out) {
  const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const size_t lo = size_t(blockIdx.x) * per;
  const size_t hi = lo + per < n16 ? lo + per : n16;
  u32x4_t acc = {0u, 0u, 0u, 0u};
  size_t i = lo + threadIdx.x;
  for (; i + 7 * 256 < hi; i += 8 * 256) {
    u32x4_t v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = __builtin_nontemporal_load(src + i + q * 256);
#pragma unroll
    for (int q = 0; q < 8; ++q) acc ^= v[q];
  }
  for (; i < hi; i += 256) acc ^= src[i];
  const uint32_t w = acc.x ^ acc.y ^ acc.z ^ acc.w;
  __shared__ uint32_t red[256];
  red[threadIdx.x] = w;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int t = 0; t < 256; ++t) r ^= red[t];
    out[blockIdx.x] = r;
  }
}

}  // namespace

hipError_t launch_read_stream(const void *src, size_t bytes, uint32_t *out, hipStream_t s) {
  read_stream_kernel<<<kReadStreamBlocks, 256, 0, s>>>(static_cast<const u32x4_t *>(src), bytes / 16, out);
  return hipGetLastError();
}

}  // namespace moe
