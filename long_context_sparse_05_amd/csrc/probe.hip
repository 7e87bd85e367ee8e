// probe.hip -- a plain streaming read of device memory, the measured
// bandwidth ceiling the decode roofline is reported against.
//
// Every workgroup reads a contiguous slice of the buffer with the same loads
// the token-scoring kernel streams keys with (16-byte non-temporal loads,
// each wave instruction covering 1 KiB), eight per thread in flight, and
// folds the words with XOR so the loads are not dead; one word per
// workgroup is written to the sink.
#include <hip/hip_ext.h>

#include "../../include/misa_indexer.h"
#include "common.hpp"

namespace misa {

__global__ __launch_bounds__(256) void stream_read_kernel(const uint4 *buf, size_t n16, size_t per_wg,
                                                          uint32_t *sink) {
  constexpr int U = 8;
  const size_t lo = (size_t)blockIdx.x * per_wg, hi = min(lo + per_wg, n16);
  uint32_t acc = 0;
  for (size_t i0 = lo + threadIdx.x; i0 < hi; i0 += (size_t)256 * U) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = load_nt16(buf + min(i0 + (size_t)256 * u, hi - 1));
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  acc = wave_sum(acc);
  if ((threadIdx.x & 63) == 0) atomicXor(&sink[blockIdx.x], acc);
}

}  // namespace misa

extern "C" int misa_stream_read(const void *buf, size_t bytes, int32_t wgs, uint32_t *sink,
                                void *stream, void *ev_start, void *ev_stop) {
  if (!buf || !sink) return MISA_ERR_NULL;
  if (((uintptr_t)buf & 15) || (bytes & 15)) return MISA_ERR_UNSUPPORTED;
  if (bytes == 0 || wgs < 1 || wgs > 65535) return MISA_ERR_SHAPE;
  const size_t n16 = bytes / 16;
  const size_t per_wg = (n16 + wgs - 1) / wgs;
  const int grid = (int)((n16 + per_wg - 1) / per_wg);
  if (ev_start || ev_stop)
    hipExtLaunchKernelGGL(misa::stream_read_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream,
                          (hipEvent_t)ev_start, (hipEvent_t)ev_stop, 0, (const uint4 *)buf, n16, per_wg, sink);
  else
    hipLaunchKernelGGL(misa::stream_read_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream,
                       (const uint4 *)buf, n16, per_wg, sink);
  return hipGetLastError() == hipSuccess ? MISA_OK : MISA_ERR_HIP;
}
