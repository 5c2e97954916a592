// Streaming-read probe: the HBM read rate a plain kernel reaches on this GPU,
// the ceiling beside the partition kernels' achieved bandwidth.  It reads
// with the partition kernels' own 16-byte non-temporal loads, coalesced
// (consecutive lanes, consecutive 16-byte words), and folds every word into
// a 32-bit XOR so that no load is dead and the result can be checked
// exactly.  Two patterns, as neither is best at every size (measured on
// MI355X): SLAB = false, the workgroups interleave over the buffer (grid
// stride, 8 loads in flight per lane); SLAB = true, each workgroup reads one
// contiguous slab (16 in flight per lane).
#pragma once

#include "pa_common.h"

namespace pa {

// n16 16-byte words; workgroup w stores the XOR of the 32-bit words it read
// in sink[w].  256 threads.
template <bool SLAB>
__global__ __launch_bounds__(256) void stream_read(const u32x4* __restrict__ src, uint64_t n16,
                                                   uint32_t* __restrict__ sink) {
  constexpr int U = SLAB ? 16 : 8;
  u32x4 x = {0u, 0u, 0u, 0u};
  uint64_t i, end, stride;
  if constexpr (SLAB) {
    const uint64_t per = (n16 + gridDim.x - 1) / gridDim.x;
    const uint64_t b0 = (uint64_t)blockIdx.x * per;
    i = b0 + threadIdx.x;
    end = b0 + per < n16 ? b0 + per : n16;  // below b0 when the slab is empty
    stride = 256;
  } else {
    i = (uint64_t)blockIdx.x * 256 + threadIdx.x;
    end = n16;
    stride = (uint64_t)gridDim.x * 256;
  }
  for (; i + (U - 1) * stride < end; i += U * stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < U; ++u) x ^= v[u];
  }
  for (; i < end; i += stride) x ^= __builtin_nontemporal_load(src + i);
  uint32_t r = x[0] ^ x[1] ^ x[2] ^ x[3];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) r ^= __shfl_xor(r, off);
  __shared__ uint32_t s_wave[4];
  if ((threadIdx.x & 63) == 0) s_wave[threadIdx.x >> 6] = r;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = s_wave[0] ^ s_wave[1] ^ s_wave[2] ^ s_wave[3];
}

}  // namespace pa
