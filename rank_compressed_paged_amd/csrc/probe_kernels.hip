// HBM stream-read ceiling probe: the plain sequential read rate one MI355X
// sustains; the latent scan is compared with it as well as with the 8 TB/s peak.
// Every lane reads 16-byte words in a grid-stride loop with U loads in
// flight; the values are folded so the loads cannot be removed.

#include "common.h"
#include "starkv.h"

namespace starkv {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int U>
__global__ void __launch_bounds__(1024)
stream_read_kernel(const u32x4* __restrict__ src, size_t n, uint32_t* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (U - 1) * stride < n; i += U * stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n; i += stride) {
    const u32x4 v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;   // data-dependent: keeps every load
}

}  // namespace starkv

extern "C" starkv_status starkv_stream_read_probe(const void* src, size_t bytes, uint32_t* sink, int32_t grid,
                                                  int32_t block, void* stream) {
  if (!src || !sink || bytes == 0 || bytes % 16 != 0 || grid < 1 || block < 64 || block > 1024 ||
      block % 64 != 0 || (reinterpret_cast<uintptr_t>(src) & 15) != 0)
    return STARKV_ERR_INVALID_ARG;
  hipLaunchKernelGGL(starkv::stream_read_kernel<8>, dim3(grid), dim3(block), 0, static_cast<hipStream_t>(stream),
                     static_cast<const starkv::u32x4*>(src), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? STARKV_OK : STARKV_ERR_HIP;
}
