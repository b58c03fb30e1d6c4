// Integer helpers shared by the sampler's and the merge plan's large-image
// paths: a zero fill, and per-segment exclusive scans of int32 counts.
#include "common.h"

namespace ca {

namespace {

constexpr int kZeroThreads = 256;
constexpr int kScanThreads = 1024;
constexpr int kScanChunk = 8192;

__global__ void __launch_bounds__(kZeroThreads) zero_i32_kernel(int64_t n, int32_t* __restrict__ x) {
  const int64_t i = (int64_t)blockIdx.x * kZeroThreads + threadIdx.x;
  if (i < n) x[i] = 0;
}

// one workgroup per segment: off[s, 0..n] = exclusive prefix sums of
// cnt[s, 0..n-1], off[s, n] = the total; counts staged through LDS in
// chunks of kScanChunk, one workgroup scan per chunk
__global__ void __launch_bounds__(kScanThreads)
segment_scan_kernel(int n, const int32_t* __restrict__ cnt_all, int32_t* __restrict__ off_all) {
  __shared__ int32_t v[kScanChunk];
  __shared__ int tmp[17];
  const int64_t s = blockIdx.x;
  const int32_t* cnt = cnt_all + s * n;
  int32_t* off = off_all + s * (n + 1);
  constexpr int kPer = kScanChunk / kScanThreads;
  int carry = 0;
  for (int c0 = 0; c0 < n; c0 += kScanChunk) {
    const int m = min(kScanChunk, n - c0);
    for (int x = threadIdx.x; x < m; x += kScanThreads) v[x] = cnt[c0 + x];
    __syncthreads();
    const int r0 = threadIdx.x * kPer;
    int run = 0;
#pragma unroll
    for (int r = 0; r < kPer; ++r) run += r0 + r < m ? v[r0 + r] : 0;
    int tot;
    int acc = carry + block_exclusive_scan(run, tmp, kScanThreads, &tot);
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
      if (r0 + r < m) {
        const int c = v[r0 + r];
        v[r0 + r] = acc;
        acc += c;
      }
    }
    __syncthreads();
    for (int x = threadIdx.x; x < m; x += kScanThreads) off[c0 + x] = v[x];
    carry += tot;
    __syncthreads();
  }
  if (threadIdx.x == 0) off[n] = carry;
}

}  // namespace

void launch_zero_i32(int64_t n, int32_t* x, hipStream_t st) {
  if (n <= 0) return;
  hipLaunchKernelGGL(zero_i32_kernel, dim3((unsigned)((n + kZeroThreads - 1) / kZeroThreads)),
                     dim3(kZeroThreads), 0, st, n, x);
}

void launch_segment_scan(int segments, int n, const int32_t* cnt, int32_t* off, hipStream_t st) {
  if (segments <= 0) return;
  hipLaunchKernelGGL(segment_scan_kernel, dim3((unsigned)segments), dim3(kScanThreads), 0, st, n,
                     cnt, off);
}

}  // namespace ca
