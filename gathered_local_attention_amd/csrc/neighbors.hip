// Neighbour-list build for local cluster attention on gfx950.
//
// Source: English notes page "AFFMAE: Scalable Vision Pre-Training for
// High-Resolution Microscopy Segmentation on Desktop Hardware", "Overall
// Architecture" (explicit 2D coordinate per token, local balanced
// clustering) and "Limitations & Future Work" (space-filling curves as the
// lookup structure; off-grid gather cost).  The pages give no algorithm; the
// library's reading is: 16-bit fixed-point quantisation, Morton order with x
// in the even bits, clusters = consecutive runs of 8 in that order (ties by
// token index), and each cluster's list = itself plus the k-1 clusters with
// the nearest integer centroid sums (ties by cluster index).
//
// Kernels (all integer after one exact fp64 quantisation):
//   rank_kernel    per segment (an image, or a 2048-token chunk of a large
//                  image): every token's rank among the segment's
//                  (code, token) keys, counted against the whole segment
//                  held in LDS.  Writes perm / packed coordinates directly
//                  when the segment is the whole image, else the chunk's
//                  keys in sorted order.
//   merge_kernel   large images only: a token's image-wide rank is its rank
//                  in its own chunk plus, for every other chunk, the number of
//                  keys below it (binary search over that chunk staged in LDS).
//   select_kernel  per cluster: brute-force scan of all clusters of the image
//                  (candidate centroids staged in LDS tiles), keeping the k-1
//                  smallest (d2 << 24 | index) keys; then the key lists.
#include "common.h"

namespace ca {

namespace {

constexpr int kRankThreads = 256;
constexpr int kSelectThreads = 256;
constexpr int kSelectTile = 1024;

__device__ __forceinline__ uint32_t spread16(uint32_t v) {
  v &= 0xFFFFu;
  v = (v | (v << 8)) & 0x00FF00FFu;
  v = (v | (v << 4)) & 0x0F0F0F0Fu;
  v = (v | (v << 2)) & 0x33333333u;
  v = (v | (v << 1)) & 0x55555555u;
  return v;
}

__device__ __forceinline__ uint32_t quantize_axis(float c, double step) {
  // (c + 0.5) and the power-of-two step are exact in fp64, so this equals
  // floor((c + 0.5) * step) of the real numbers.
  double q = floor(((double)c + 0.5) * step);
  q = q < 0.0 ? 0.0 : (q > 65535.0 ? 65535.0 : q);
  return (uint32_t)q;
}

// Rank the tokens of one segment.  grid = (ceil(L / 256), segments), where a
// segment is [seg_start, seg_start + L) of image `b`.
__global__ void __launch_bounds__(kRankThreads)
rank_kernel(const float* __restrict__ coords, int N, int seg_len, int segs_per_image, double step,
            int32_t* __restrict__ perm, uint32_t* __restrict__ qsorted,
            uint64_t* __restrict__ chunk_keys) {
  __shared__ uint64_t keys[kSortChunk];
  const int seg = blockIdx.y;
  const int b = seg / segs_per_image;
  const int start = (seg % segs_per_image) * seg_len;
  const int L = min(seg_len, N - start);
  const float2* xy = reinterpret_cast<const float2*>(coords) + (int64_t)b * N + start;

  for (int e = threadIdx.x; e < L; e += kRankThreads) {
    float2 c = xy[e];
    uint32_t code = spread16(quantize_axis(c.x, step)) | (spread16(quantize_axis(c.y, step)) << 1);
    keys[e] = ((uint64_t)code << 32) | (uint32_t)(start + e);
  }
  __syncthreads();

  const int e = blockIdx.x * kRankThreads + threadIdx.x;
  if (e >= L) return;
  const uint64_t mine = keys[e];
  int rank = 0;
  int u = 0;
  for (; u + 4 <= L; u += 4) {
    rank += (keys[u] < mine) + (keys[u + 1] < mine) + (keys[u + 2] < mine) + (keys[u + 3] < mine);
  }
  for (; u < L; ++u) rank += (keys[u] < mine);

  if (segs_per_image == 1) {
    const int64_t at = (int64_t)b * N + rank;
    perm[at] = (int32_t)(uint32_t)mine;
    float2 c = xy[e];
    qsorted[at] = quantize_axis(c.x, step) | (quantize_axis(c.y, step) << 16);
  } else {
    chunk_keys[(int64_t)b * N + start + rank] = mine;
  }
}

// Image-wide ranks for images split into chunks.  grid = (chunks, B); each
// block owns one chunk (up to 2048 tokens, 8 per thread).
__global__ void __launch_bounds__(kRankThreads)
merge_kernel(const float* __restrict__ coords, int N, double step,
             const uint64_t* __restrict__ chunk_keys, int32_t* __restrict__ perm,
             uint32_t* __restrict__ qsorted) {
  __shared__ uint64_t other[kSortChunk];
  constexpr int kPer = kSortChunk / kRankThreads;
  const int a = blockIdx.x;
  const int b = blockIdx.y;
  const int nchunks = (N + kSortChunk - 1) / kSortChunk;
  const uint64_t* img = chunk_keys + (int64_t)b * N;
  const int a0 = a * kSortChunk;
  const int La = min(kSortChunk, N - a0);

  uint64_t mine[kPer];
  int rank[kPer];
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    const int e = threadIdx.x + r * kRankThreads;
    mine[r] = e < La ? img[a0 + e] : ~0ull;
    rank[r] = e;   // position inside its own (sorted) chunk
  }

  for (int c = 0; c < nchunks; ++c) {
    if (c == a) continue;
    const int c0 = c * kSortChunk;
    const int Lc = min(kSortChunk, N - c0);
    __syncthreads();
    for (int e = threadIdx.x; e < Lc; e += kRankThreads) other[e] = img[c0 + e];
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
      int lo = 0, hi = Lc;   // number of keys < mine[r]
      while (lo < hi) {
        int mid = (lo + hi) >> 1;
        if (other[mid] < mine[r]) lo = mid + 1; else hi = mid;
      }
      rank[r] += lo;
    }
  }

  const float2* xy = reinterpret_cast<const float2*>(coords) + (int64_t)b * N;
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    const int e = threadIdx.x + r * kRankThreads;
    if (e >= La) continue;
    const int tok = (int)(uint32_t)mine[r];
    const int64_t at = (int64_t)b * N + rank[r];
    perm[at] = tok;
    float2 c = xy[tok];
    qsorted[at] = quantize_axis(c.x, step) | (quantize_axis(c.y, step) << 16);
  }
}

__device__ __forceinline__ int2 centroid_sum(const uint32_t* __restrict__ q8) {
  int sx = 0, sy = 0;
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    uint32_t p = q8[m];
    sx += (int)(p & 0xFFFFu);
    sy += (int)(p >> 16);
  }
  return make_int2(sx, sy);
}

// Nearest clusters and key lists.  grid = (ceil(C / 256), B).
template <int KM1>
__global__ void __launch_bounds__(kSelectThreads)
select_kernel(int N, const uint32_t* __restrict__ qsorted, const int32_t* __restrict__ perm,
              int32_t* __restrict__ nbr, int32_t* __restrict__ key_idx) {
  __shared__ int2 cand[kSelectTile];
  const int C = N / 8;
  const int b = blockIdx.y;
  const int c = blockIdx.x * kSelectThreads + threadIdx.x;
  const uint32_t* qimg = qsorted + (int64_t)b * N;
  const int2 me = c < C ? centroid_sum(qimg + 8 * c) : make_int2(0, 0);

  uint64_t best[KM1 > 0 ? KM1 : 1];
#pragma unroll
  for (int r = 0; r < (KM1 > 0 ? KM1 : 1); ++r) best[r] = ~0ull;

  for (int t0 = 0; t0 < C; t0 += kSelectTile) {
    const int T = min(kSelectTile, C - t0);
    __syncthreads();
    for (int e = threadIdx.x; e < T; e += kSelectThreads) cand[e] = centroid_sum(qimg + 8 * (t0 + e));
    __syncthreads();
    if constexpr (KM1 > 0) {
    if (c >= C) continue;
    for (int e = 0; e < T; ++e) {
      const int2 s = cand[e];
      const int64_t dx = s.x - me.x, dy = s.y - me.y;
      const uint64_t key = ((uint64_t)(dx * dx + dy * dy) << 24) | (uint32_t)(t0 + e);
      if (t0 + e == c || key >= best[KM1 - 1]) continue;
      // insertion into the sorted top list
      uint64_t x = key;
#pragma unroll
      for (int r = 0; r < KM1; ++r) {
        const uint64_t lo = x < best[r] ? x : best[r];
        const uint64_t hi = x < best[r] ? best[r] : x;
        best[r] = lo;
        x = hi;
      }
    }
    }
  }
  if (c >= C) return;

  constexpr int K = KM1 + 1;
  int32_t ids[K];
  ids[0] = c;
#pragma unroll
  for (int r = 0; r < KM1; ++r) ids[r + 1] = best[r] == ~0ull ? -1 : (int32_t)(best[r] & 0xFFFFFFu);
  int32_t* nrow = nbr + ((int64_t)b * C + c) * K;
  int32_t* krow = key_idx + ((int64_t)b * C + c) * K * 8;
  const int32_t* pimg = perm + (int64_t)b * N;
#pragma unroll
  for (int s = 0; s < K; ++s) {
    nrow[s] = ids[s];
#pragma unroll
    for (int m = 0; m < 8; ++m) krow[s * 8 + m] = ids[s] >= 0 ? pimg[ids[s] * 8 + m] : -1;
  }
}

}  // namespace

hipError_t launch_build_neighbors(const float* coords, int B, int N, int grid_side, int k,
                                  int32_t* perm, int32_t* nbr, int32_t* key_idx, void* ws,
                                  hipStream_t st) {
  int bits = 0;   // ceil(log2(grid_side)); grid_side is validated to [1, 65536]
  while ((1 << bits) < grid_side) ++bits;
  const double step = (double)(1u << (16 - bits));
  BuildWorkspace w = build_layout(ws, B, N);
  const int C = N / 8;
  if (N <= kSortChunk) {
    dim3 grid((N + kRankThreads - 1) / kRankThreads, B);
    hipLaunchKernelGGL(rank_kernel, grid, dim3(kRankThreads), 0, st, coords, N, N, 1, step, perm,
                       w.qsorted, (uint64_t*)nullptr);
  } else {
    const int chunks = (N + kSortChunk - 1) / kSortChunk;
    dim3 grid(kSortChunk / kRankThreads, B * chunks);
    hipLaunchKernelGGL(rank_kernel, grid, dim3(kRankThreads), 0, st, coords, N, kSortChunk, chunks,
                       step, perm, w.qsorted, w.keys);
    hipLaunchKernelGGL(merge_kernel, dim3(chunks, B), dim3(kRankThreads), 0, st, coords, N, step,
                       (const uint64_t*)w.keys, perm, w.qsorted);
  }
  dim3 sgrid((C + kSelectThreads - 1) / kSelectThreads, B);
  switch (k) {
#define CA_SEL(KK)                                                                              \
  case KK:                                                                                      \
    hipLaunchKernelGGL(select_kernel<KK - 1>, sgrid, dim3(kSelectThreads), 0, st, N,            \
                       (const uint32_t*)w.qsorted, (const int32_t*)perm, nbr, key_idx);         \
    break;
    CA_SEL(1) CA_SEL(2) CA_SEL(3) CA_SEL(4) CA_SEL(5) CA_SEL(6) CA_SEL(7) CA_SEL(8)
#undef CA_SEL
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace ca
