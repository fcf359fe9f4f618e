// Streaming-read probe (a measurement helper, not part of the W12 method): the HBM read
// ceiling the GEMM kernels are compared with, and the known-size kernel that calibrates
// the HBM traffic counters for the loads the GEMM issues.  Every workgroup reads 16-byte
// units of [buf, buf + bytes) in a grid-stride loop with the same nontemporal buffer loads
// the GEMM uses for W12 tiles, four per thread in flight, and each wave stores the XOR of
// what it read (so no load is dead).  Units past the end read as zero (buffer loads past
// the resource's size), so no lane needs a bounds test.
#include "w12_internal.h"

namespace w12 {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kStreamT = 256;
constexpr int kStreamU = 4;
constexpr int kCpolStream = 2;   // nontemporal, as the GEMM's W12 tile loads

__global__ __launch_bounds__(kStreamT) void k_stream_read(const uint8_t* buf, uint32_t bytes,
                                                          uint32_t* sink) {
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(buf), (short)0, (int)bytes, 0x00020000);
  const uint32_t stride = gridDim.x * (uint32_t)kStreamT;
  const uint32_t n16 = bytes / 16u;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (uint32_t i = blockIdx.x * (uint32_t)kStreamT + threadIdx.x; i < n16; i += kStreamU * stride) {
    u32x4 v[kStreamU];
#pragma unroll
    for (int u = 0; u < kStreamU; ++u) {
      const uint32_t j = i + (uint32_t)u * stride;
      // offsets of units past the end (j >= n16, bytes < 2^32) read as zero
      v[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, j < n16 ? j * 16u : bytes, 0, kCpolStream);
    }
#pragma unroll
    for (int u = 0; u < kStreamU; ++u) acc ^= v[u];
  }
  uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x ^= __shfl_xor(x, off);
  if ((threadIdx.x & 63u) == 0u) sink[blockIdx.x * (kStreamT / 64) + threadIdx.x / 64u] = x;
}

hipError_t launch_stream_read(const void* buf, uint32_t bytes, uint32_t workgroups, uint32_t* sink,
                              hipStream_t s) {
  hipLaunchKernelGGL(k_stream_read, dim3(workgroups), dim3(kStreamT), 0, s, (const uint8_t*)buf,
                     bytes, sink);
  return hipGetLastError();
}

}  // namespace w12
