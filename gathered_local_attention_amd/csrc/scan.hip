// Integer helpers shared by the sampler's and the merge plan's large-image
// paths: a zero fill, per-segment exclusive scans of int32 counts, and a
// stable sort of the long segments of a segmented list.
#include "common.h"

#include <algorithm>

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

constexpr int kSortThreads = 1024;
constexpr int kSortWaves = kSortThreads / 64;
constexpr int kSortGrid = 512;

// Stable LSD radix sort (8-bit digits, `passes` of them from the lowest) of
// every segment longer than min_len.  Segment s of image b is
// vals[b * stride + off[b * (S + 1) + s] .. off[b * (S + 1) + s + 1]);
// tmp has the same layout (scratch).  Each workgroup first lists the long
// segments among a block of kSortThreads (one check per thread), then sorts
// them one after another: per pass a digit histogram, its scan, and a
// scatter tile by tile in element order (ranks inside a wave from ballots of
// the digit bits, then prefixes over the waves), so equal digits keep their
// order.  The last pass writes the sorted values to out (same positions), or
// with kPairs each value v as (v / K, bits of wgt[b * stride + v]) to out2.
template <bool kPairs>
__global__ void __launch_bounds__(kSortThreads)
long_segment_sort_kernel(int B, int S, int64_t stride, int min_len, int passes,
                         const int32_t* __restrict__ off_all, int32_t* __restrict__ vals,
                         int32_t* __restrict__ tmp, int32_t* __restrict__ out,
                         int2* __restrict__ out2, int K, const float* __restrict__ wgt) {
  __shared__ int hist[256];
  __shared__ int base[256];
  __shared__ int wcnt[kSortWaves][256];
  __shared__ int tmp17[17];
  __shared__ int nlong;
  __shared__ int64_t longs[kSortThreads];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t nseg = (int64_t)B * S;
  for (int64_t g0 = (int64_t)blockIdx.x * kSortThreads; g0 < nseg;
       g0 += (int64_t)gridDim.x * kSortThreads) {
    if (tid == 0) nlong = 0;
    __syncthreads();
    {
      const int64_t g = g0 + tid;
      if (g < nseg) {
        const int64_t b = g / S;
        const int64_t o = b * (S + 1) + (g - b * S);
        if (off_all[o + 1] - off_all[o] > min_len) longs[atomicAdd(&nlong, 1)] = g;
      }
    }
    __syncthreads();
    const int nl = nlong;
    for (int li = 0; li < nl; ++li) {
      const int64_t g = longs[li];
      const int64_t b = g / S;
      const int64_t o = b * (S + 1) + (g - b * S);
      const int lo = off_all[o], L = off_all[o + 1] - lo;
      int32_t* v0 = vals + b * stride + lo;
      int32_t* v1 = tmp + b * stride + lo;
      for (int x = tid; x < kSortWaves * 256; x += kSortThreads) (&wcnt[0][0])[x] = 0;
      for (int pass = 0; pass < passes; ++pass) {
        const int sh = 8 * pass;
        const int32_t* src = (pass & 1) ? v1 : v0;
        int32_t* dst = (pass & 1) ? v0 : v1;
        const bool last = pass == passes - 1;
        if (tid < 256) hist[tid] = 0;
        __syncthreads();
        for (int i = tid; i < L; i += kSortThreads) atomicAdd(&hist[(src[i] >> sh) & 255], 1);
        __syncthreads();
        int tot;
        const int ex = block_exclusive_scan(tid < 256 ? hist[tid] : 0, tmp17, kSortThreads, &tot);
        if (tid < 256) base[tid] = ex;
        __syncthreads();
        for (int t0 = 0; t0 < L; t0 += kSortThreads) {
          const int i = t0 + tid;
          const bool ok = i < L;
          const int v = ok ? src[i] : 0;
          const int dg = (v >> sh) & 255;
          // lanes of this wave holding the same digit
          uint64_t peers = __ballot(ok);
#pragma unroll
          for (int bit = 0; bit < 8; ++bit) {
            const uint64_t bb = __ballot(ok && ((dg >> bit) & 1));
            peers &= ((dg >> bit) & 1) ? bb : ~bb;
          }
          const int rank = __popcll(peers & ((1ull << lane) - 1ull));
          if (ok && rank == 0) wcnt[wv][dg] = __popcll(peers);
          __syncthreads();
          if (tid < 256) {   // prefixes over the waves, and the tile's count
            int acc = 0;
            for (int w = 0; w < kSortWaves; ++w) {
              const int c = wcnt[w][tid];
              wcnt[w][tid] = acc;
              acc += c;
            }
            hist[tid] = acc;
          }
          __syncthreads();
          if (ok) {
            const int pos = base[dg] + wcnt[wv][dg] + rank;
            if (!last) dst[pos] = v;
            else if (kPairs) out2[b * stride + lo + pos] = make_int2(v / K, __float_as_int(wgt[b * stride + v]));
            else out[b * stride + lo + pos] = v;
          }
          __syncthreads();
          if (tid < 256) base[tid] += hist[tid];
          for (int x = tid; x < kSortWaves * 256; x += kSortThreads) (&wcnt[0][0])[x] = 0;
          __syncthreads();
        }
      }
    }
    __syncthreads();   // the list is reused by the next block of segments
  }
}

int value_passes(int64_t max_value) {
  int bits = 0;
  while (bits < 31 && (int64_t(1) << bits) <= max_value) ++bits;
  return std::max(1, (bits + 7) / 8);
}

}  // namespace

void launch_long_segment_sort(int B, int S, int64_t stride, int64_t max_value, const int32_t* off,
                              int32_t* vals, int32_t* tmp, int32_t* out, int2* out2, int K,
                              const float* wgt, hipStream_t st) {
  if ((int64_t)B * S <= 0) return;
  const int64_t blocks = ((int64_t)B * S + kSortThreads - 1) / kSortThreads;
  const unsigned grid = (unsigned)std::min<int64_t>(blocks, kSortGrid);
  const int passes = value_passes(max_value);
  if (out2)
    hipLaunchKernelGGL(long_segment_sort_kernel<true>, dim3(grid), dim3(kSortThreads), 0, st, B, S,
                       stride, kLongSegment, passes, off, vals, tmp, out, out2, K, wgt);
  else
    hipLaunchKernelGGL(long_segment_sort_kernel<false>, dim3(grid), dim3(kSortThreads), 0, st, B, S,
                       stride, kLongSegment, passes, off, vals, tmp, out, out2, K, wgt);
}

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
