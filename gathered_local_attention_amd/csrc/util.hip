// Measurement utility of libclusterattn: a plain device-to-device copy,
// used to measure the HBM bandwidth this device achieves, against which the
// attention kernels' effective bandwidth is reported next to the vendor
// peak.  Each workgroup copies one contiguous chunk, eight 16-byte loads in
// flight per thread, with non-temporal loads and stores (streamed data is
// not kept in the caches); no LDS.
#include "../../include/cluster_attn.h"
#include "common.h"

namespace ca {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int kCopyUnroll = 8;

__global__ void __launch_bounds__(256) copy16_kernel(const u32x4* __restrict__ src,
                                                     u32x4* __restrict__ dst, size_t n16) {
  const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const size_t lo = (size_t)blockIdx.x * per;
  const size_t hi = lo + per < n16 ? lo + per : n16;
  size_t i = lo + threadIdx.x;
  for (; i + (kCopyUnroll - 1) * 256 < hi; i += kCopyUnroll * 256) {
    u32x4 r[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) r[u] = __builtin_nontemporal_load(src + i + u * 256);
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) __builtin_nontemporal_store(r[u], dst + i + u * 256);
  }
  for (; i < hi; i += 256) dst[i] = src[i];
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
    // up to 16 workgroups of 256 threads per CU over the 256 CUs, each on a
    // contiguous chunk of at least 4 KiB
    const size_t want = (n16 + 255) / 256;
    const unsigned grid = (unsigned)(want < 4096 ? want : 4096);
    hipLaunchKernelGGL(ca::copy16_kernel, dim3(grid), dim3(256), 0, st, (const ca::u32x4*)src,
                       (ca::u32x4*)dst, n16);
  }
  const size_t tail = bytes - n16 * 16;
  if (tail)
    hipLaunchKernelGGL(ca::copy1_kernel, dim3(1), dim3(64), 0, st,
                       (const uint8_t*)src + n16 * 16, (uint8_t*)dst + n16 * 16, tail);
  return hipGetLastError() == hipSuccess ? CA_OK : CA_ERR_HIP;
}
