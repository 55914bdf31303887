// Plain 16-byte-vector device copy: the reference stream for bandwidth and
// for scaling hardware traffic counters (bytes read == bytes written == size).
#include <hip/hip_ext.h>

#include "sikv_internal.h"

namespace sikv {

namespace {

__global__ __launch_bounds__(256) void copy_kernel(uint4* __restrict__ dst,
                                                   const uint4* __restrict__ src, int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
    dst[i] = src[i];
}

}  // namespace

hipError_t launch_copy(void* dst, const void* src, size_t bytes, const Launch& s) {
  const int64_t n16 = (int64_t)(bytes / 16);
  int64_t blocks = (n16 + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) blocks = 1;
  return launch_k(KID_COPY, copy_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                  static_cast<uint4*>(dst), static_cast<const uint4*>(src), n16);
}

}  // namespace sikv
