// Measurement utility of libclusterattn: a plain device-to-device copy,
// used to measure the HBM bandwidth this device achieves, against which the
// attention kernels' effective bandwidth is reported next to the vendor
// peak.  16-byte loads and stores, grid-stride, no LDS.
#include "../../include/cluster_attn.h"
#include "common.h"

namespace ca {
namespace {

__global__ void __launch_bounds__(256) copy16_kernel(const uint4* __restrict__ src,
                                                     uint4* __restrict__ dst, size_t n16) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  // four independent 16-byte loads in flight per thread
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    dst[i] = a;
    dst[i + stride] = b;
    dst[i + 2 * stride] = c;
    dst[i + 3 * stride] = d;
  }
  for (; i < n16; i += stride) dst[i] = src[i];
}

__global__ void copy1_kernel(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                             size_t n) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = src[i];
}

}  // namespace
}  // namespace ca

extern "C" ca_status cluster_attn_device_copy(void* dst, const void* src, size_t bytes,
                                              void* hip_stream) {
  if (bytes == 0) return CA_OK;
  if (!dst || !src) return CA_ERR_NULL;
  if (((uintptr_t)dst | (uintptr_t)src) & 15) return CA_ERR_UNSUPPORTED;
  const uintptr_t d0 = (uintptr_t)dst, s0 = (uintptr_t)src;
  if (d0 < s0 + bytes && s0 < d0 + bytes) return CA_ERR_ALIAS;
  hipStream_t st = (hipStream_t)hip_stream;
  const size_t n16 = bytes / 16;
  if (n16) {
    // 8 workgroups of 256 threads per CU over the 256 CUs
    const size_t want = (n16 + 255) / 256;
    const unsigned grid = (unsigned)(want < 2048 ? want : 2048);
    hipLaunchKernelGGL(ca::copy16_kernel, dim3(grid), dim3(256), 0, st, (const uint4*)src,
                       (uint4*)dst, n16);
  }
  const size_t tail = bytes - n16 * 16;
  if (tail)
    hipLaunchKernelGGL(ca::copy1_kernel, dim3(1), dim3(64), 0, st,
                       (const uint8_t*)src + n16 * 16, (uint8_t*)dst + n16 * 16, tail);
  return hipGetLastError() == hipSuccess ? CA_OK : CA_ERR_HIP;
}
