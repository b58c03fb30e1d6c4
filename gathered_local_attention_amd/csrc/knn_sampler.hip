// KNN-cache point sampler of the point-wise decoder, on gfx950.
//
// Source: English notes page "AFFMAE: Scalable Vision Pre-Training for
// High-Resolution Microscopy Segmentation on Desktop Hardware", "Key Designs"
// item 2 (point-wise deformable cross-attention decoder: a query samples at
// q = r + offset and aggregates its nearest visible tokens with
// w = softmax(-p d)) and item 3 (KNN cache lookup: an H x W x K table of the K
// nearest visible tokens of every grid cell; a query is quantised to its
// nearest cell, so the search becomes a lookup plus a distance calculation;
// distance and softmax weighting fused in one kernel, forward and backward).
// The pages give no formula beyond w; the library's readings:
//   table     cell (row i, column j) has its centre at (j, i); its K nearest
//             tokens by squared distance of the 16-bit fixed-point
//             coordinates (the neighbour build's quantisation), ties to the
//             lower token index, -1 padding;
//   query     cell column clamp(floor(x + 1/2), 0, G-1), row likewise (fp64);
//   weights   d_k = |q - x_k| of the f32 coordinates, w = stable softmax of
//             -p d over the valid slots, out = sum_k w_k F[token_k];
//   backward  gradients of F, of the query coordinates and of p (token
//             coordinates constant; dd/dq taken as 0 at d = 0).
//
// Kernels:
//   knn_table_kernel      workgroups of (image, part of its cells): the
//                         image's tokens counting-sorted into square buckets
//                         of the fixed-point grid (about two tokens each) in
//                         LDS; one wave per 8 x 8-cell tile (lane = cell)
//                         grows a window of buckets around the tile ring by
//                         ring, every lane testing every token of the window,
//                         and stops once each lane's K-th best is strictly
//                         closer than any token outside the window can be.
//   knn_bucket_count/place, knn_table_search_kernel  the same for images
//                         above 4096 tokens, with the buckets in global
//                         memory (bucketed once per image).
//   knn_fwd_kernel        a wave serves a run of queries: one lane per
//                         query works out the cell, slots, distances and
//                         weights into LDS, then lane groups sum the K
//                         gathered rows, each lane the 16-byte chunks it
//                         owns (group width: the one leaving the fewest
//                         lanes idle, up to 3 chunks per lane for bf16/f16).
//   knn_bwd_query_kernel  the same waves: weights again, <dO, F_k> by
//                         bf16/fp16 dot-2 instructions reduced over the
//                         group, dq and the wave's share of dp; slots and
//                         weights kept for the feature gradient (and, for
//                         images above 4096 tokens, references counted per
//                         token).
//   knn_pcount/pprefix/scan/pplace  token-major entry lists (entry =
//                         query * K + slot, stored as its (query, weight)
//                         pair) by a stable counting sort over partitions of
//                         2048 entries (ranks inside a partition: per-wave
//                         counts, then ballot matching of equal tokens in
//                         each 64-entry batch): each token's segment is in
//                         entry order, so the feature gradient is summed in
//                         a fixed order; the count launch also builds the
//                         tokens' spatial walk order.  Images above 4096
//                         tokens: knn_lplace/lrank (cursor placement, then
//                         each entry's rank in its segment: the same lists).
//   knn_dfeat_kernel      a lane group per token: dF = sum over its entries
//                         of w * dO (gathered rows), written once (0 for
//                         tokens no query reaches).
//   dp                    fixed-order reduction of the per-wave dp shares,
//                         by the feature-gradient kernel's first workgroup.
// Nothing in the backward uses floating-point atomics: the results are
// bitwise reproducible.
#include "common.h"

#include <type_traits>

namespace ca {

namespace {

constexpr int kTabThreads = 256;
constexpr int kTabMaxBuckets = 64 * 64;   // LDS buckets of the small-image build (at most 2048 used)
constexpr int kTabMaxTokens = kKnnSmallTokens;
constexpr int kKnnThreads = 256;          // 4 waves
constexpr int kPart = kKnnPart;           // entries per partition of the stable counting sort
// search keys (d2 << kTokBits | token): d2 < 2^33, tokens < 2^24
constexpr int kTokBits = 24;
constexpr uint64_t kTokMask = (uint64_t(1) << kTokBits) - 1;

// ---------------------------------------------------------------------------
// Table build.  Buckets are squares of 2^bs fixed-point units (about two
// tokens each, at least a cell: knn_buckets).  Small images (up to
// kTabMaxTokens tokens) are bucketed in LDS by every workgroup of the image
// (cheap); larger ones once, in global memory, by the bucket kernels below.
// Either way one wave per 8 x 8-cell tile (lane = cell) grows a window of
// buckets around its tile ring by ring, every lane testing every token of
// the window (uniform loops: no divergence but the insertions), and stops
// once every lane's K-th best is strictly closer than any token outside the
// window can be: a token beyond the window's top edge at fixed-point row
// R0 * 2^bs has Y <= R0 * 2^bs - 1, so |Y - cy| >= cy - R0 * 2^bs + 1;
// likewise on the other three sides.  The keys are whole (distance, token)
// pairs, so the order in which the bucketing left a bucket's tokens does not
// matter: the table is unique.
// ---------------------------------------------------------------------------
constexpr int kTabTiles = kTabThreads / 64;

// start[x] = first token of bucket x in tok (row-major buckets), the end of
// the last bucket is `total`.  kWide: start and tok are in global memory;
// a row's tokens are loaded 64 at a time, one per lane, and handed round the
// wave by readlane.  Otherwise they are in LDS and read by every lane.
template <int KM, bool kWide>
__device__ __forceinline__ void table_tile(const int* start, const uint2* tok, int total,
                                           const KnnBuckets& bg, int G, int K, int tile,
                                           int32_t* __restrict__ table_img) {
  const int lane = threadIdx.x & 63;
  const int tiles_side = (G + 7) >> 3;
  const int Pb = bg.Pb, nb = bg.nb, bs = bg.bs, shift = bg.shift;
  const int i0 = (tile / tiles_side) * 8, j0 = (tile % tiles_side) * 8;
  const int i = i0 + (lane >> 3), j = j0 + (lane & 7);
  const bool valid = i < G && j < G;
  const int64_t cx = (int64_t)(2 * j + 1) << (shift - 1);   // (j + 1/2) s
  const int64_t cy = (int64_t)(2 * i + 1) << (shift - 1);
  // the tile's own buckets (cells up to min(G, i0 + 8) - 1)
  const int ilast = min(G, i0 + 8) - 1, jlast = min(G, j0 + 8) - 1;
  const int tr0 = (i0 << shift) >> bs, tr1 = (((ilast + 1) << shift) - 1) >> bs;
  const int tc0 = (j0 << shift) >> bs, tc1 = (((jlast + 1) << shift) - 1) >> bs;
  // the K smallest keys seen, unordered (slots past K stay 0, so they are
  // never the largest), the largest of them and its slot; sorted at the end
  uint64_t best[KM];
#pragma unroll
  for (int r = 0; r < KM; ++r) best[r] = r < K ? ~0ull : 0ull;
  uint64_t worst = ~0ull;
  int wslot = 0;
  auto insert = [&](uint2 e) {
    const int64_t dx = (int64_t)(e.x & 0xFFFFu) - cx, dy = (int64_t)(e.x >> 16) - cy;
    const uint64_t x = ((uint64_t)(dx * dx + dy * dy) << kTokBits) | e.y;
    if (x >= worst) return;
#pragma unroll
    for (int r = 0; r < KM; ++r) best[r] = r == wslot ? x : best[r];
    worst = best[0];
    wslot = 0;
#pragma unroll
    for (int r = 1; r < KM; ++r) {
      const bool w = best[r] > worst;
      worst = w ? best[r] : worst;
      wslot = w ? r : wslot;
    }
  };
  // tokens of the buckets (by, bx0 .. bx1): one contiguous range
  auto scan_row = [&](int by, int bx0, int bx1) {
    const int bb0 = by * Pb + bx0, bb1 = by * Pb + bx1;
    if constexpr (kWide) {
      const int t0 = __builtin_amdgcn_readfirstlane(start[bb0]);
      const int t1 = __builtin_amdgcn_readfirstlane(start[bb1 + 1]);
      for (int c = t0; c < t1; c += 64) {
        const uint2 mine = c + lane < t1 ? tok[c + lane] : make_uint2(0u, 0u);
        const int n = min(64, t1 - c);
        for (int u = 0; u < n; ++u) {
          uint2 e;
          e.x = (uint32_t)__builtin_amdgcn_readlane((int)mine.x, u);
          e.y = (uint32_t)__builtin_amdgcn_readlane((int)mine.y, u);
          insert(e);
        }
      }
    } else {
      // wave-uniform bounds; four tokens read per step, so that one LDS
      // wait covers them
      const int t0 = __builtin_amdgcn_readfirstlane(start[bb0]);
      const int t1 = __builtin_amdgcn_readfirstlane(bb1 + 1 < nb ? start[bb1 + 1] : total);
      for (int t = t0; t < t1; t += 4) {
        uint2 e[4];
#pragma unroll
        for (int h = 0; h < 4; ++h) e[h] = tok[min(t + h, t1 - 1)];
#pragma unroll
        for (int h = 0; h < 4; ++h)
          if (t + h < t1) insert(e[h]);
      }
    }
  };
  for (int m = 0;; ++m) {
    const int r0 = tr0 - m, r1 = tr1 + m, c0 = tc0 - m, c1 = tc1 + m;   // window (buckets)
    if (m == 0) {
      for (int by = r0; by <= r1; ++by) scan_row(by, c0, c1);
    } else {
      const int cl = max(c0, 0), ch = min(c1, Pb - 1);
      if (r0 >= 0) scan_row(r0, cl, ch);
      if (r1 <= Pb - 1) scan_row(r1, cl, ch);
      for (int by = max(r0 + 1, 0); by <= min(r1 - 1, Pb - 1); ++by) {
        if (c0 >= 0) scan_row(by, c0, c0);
        if (c1 <= Pb - 1) scan_row(by, c1, c1);
      }
    }
    if (r0 <= 0 && c0 <= 0 && r1 >= Pb - 1 && c1 >= Pb - 1) break;   // every bucket seen
    int64_t lb = INT64_MAX;
    if (r0 > 0) lb = min(lb, cy - ((int64_t)r0 << bs) + 1);
    if (r1 < Pb - 1) lb = min(lb, ((int64_t)(r1 + 1) << bs) - cy);
    if (c0 > 0) lb = min(lb, cx - ((int64_t)c0 << bs) + 1);
    if (c1 < Pb - 1) lb = min(lb, ((int64_t)(c1 + 1) << bs) - cx);
    const bool done = !valid || (worst != ~0ull && (int64_t)(worst >> kTokBits) < lb * lb);
    if (__all(done)) break;
  }
  if (!valid) return;
  // ascending order (odd-even transposition over the K slots; the zero
  // slots past K are left out)
#pragma unroll
  for (int p = 0; p < KM; ++p)
#pragma unroll
    for (int r = p & 1; r + 1 < KM; r += 2)
      if (r + 1 < K) {
        const uint64_t lo = best[r] < best[r + 1] ? best[r] : best[r + 1];
        const uint64_t hi = best[r] < best[r + 1] ? best[r + 1] : best[r];
        best[r] = lo;
        best[r + 1] = hi;
      }
  int32_t* row = table_img + ((int64_t)i * G + j) * K;
#pragma unroll
  for (int r = 0; r < KM; ++r)
    if (r < K) row[r] = best[r] == ~0ull ? -1 : (int32_t)(best[r] & kTokMask);
}

// Small images.  grid = (B, parts): part y of an image takes kTabTiles tiles
// (one wave each) and repeats the image's bucketing in LDS.
template <int KM>
__global__ void __launch_bounds__(kTabThreads)
knn_table_kernel(const float* __restrict__ coords, int N, int G, int K, int32_t* __restrict__ table) {
  __shared__ int start[kTabMaxBuckets];
  __shared__ uint2 tok[kTabMaxTokens];     // (qx | qy << 16, token)
  __shared__ int tmp[17];
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const KnnBuckets bg = knn_buckets(N, G);
  const double step = (double)(1 << bg.shift);
  const int nb = bg.nb, bs = bg.bs, Pb = bg.Pb;
  const float2* xy = reinterpret_cast<const float2*>(coords) + (int64_t)b * N;

  for (int x = tid; x < nb; x += kTabThreads) start[x] = 0;
  __syncthreads();
  constexpr int kPer = kTabMaxTokens / kTabThreads;   // tokens per thread
  uint32_t pk[kPer];
  int bk[kPer], rk[kPer];
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    const int e = tid + r * kTabThreads;
    bk[r] = -1;
    if (e < N) {
      const float2 c = xy[e];
      const uint32_t qx = quantize_axis(c.x, step), qy = quantize_axis(c.y, step);
      pk[r] = qx | (qy << 16);
      bk[r] = (int)((qy >> bs) * (uint32_t)Pb + (qx >> bs));
      rk[r] = atomicAdd(&start[bk[r]], 1);
    }
  }
  __syncthreads();
  // exclusive scan of the counts
  constexpr int kBPer = kTabMaxBuckets / kTabThreads;
  int cnt[kBPer];
  int run = 0;
#pragma unroll
  for (int r = 0; r < kBPer; ++r) {
    const int x = tid * kBPer + r;
    cnt[r] = x < nb ? start[x] : 0;
    run += cnt[r];
  }
  int total;
  int acc = block_exclusive_scan(run, tmp, kTabThreads, &total);
#pragma unroll
  for (int r = 0; r < kBPer; ++r) {
    const int x = tid * kBPer + r;
    if (x < nb) start[x] = acc;
    acc += cnt[r];
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < kPer; ++r)
    if (bk[r] >= 0) tok[start[bk[r]] + rk[r]] = make_uint2(pk[r], (uint32_t)(tid + r * kTabThreads));
  __syncthreads();
  const int tiles_side = (G + 7) >> 3;
  const int tile = blockIdx.y * kTabTiles + (tid >> 6);
  if (tile >= tiles_side * tiles_side) return;
  table_tile<KM, false>(start, tok, total, bg, G, K, tile, table + (int64_t)b * G * G * K);
}

// Large images: the tokens counting-sorted into the buckets in global
// memory (count with integer atomics, scan, place), then searched.
__global__ void __launch_bounds__(kKnnThreads)
knn_bucket_count_kernel(const float* __restrict__ coords, int64_t n_tok, int N, int G,
                        int32_t* __restrict__ bcnt, int32_t* __restrict__ brank) {
  const int64_t x = (int64_t)blockIdx.x * kKnnThreads + threadIdx.x;
  if (x >= n_tok) return;
  const int64_t b = x / N;
  const KnnBuckets bg = knn_buckets(N, G);
  const double step = (double)(1 << bg.shift);
  const float2 c = reinterpret_cast<const float2*>(coords)[x];
  const uint32_t qx = quantize_axis(c.x, step), qy = quantize_axis(c.y, step);
  const int bk = (int)((qy >> bg.bs) * (uint32_t)bg.Pb + (qx >> bg.bs));
  brank[x] = atomicAdd(&bcnt[b * bg.nb + bk], 1);
}

// tok (when given): (qx | qy << 16, token) at its bucket place; order (when
// given): the token number there (the spatial walk order)
__global__ void __launch_bounds__(kKnnThreads)
knn_bucket_place_kernel(const float* __restrict__ coords, int64_t n_tok, int N, int G,
                        const int32_t* __restrict__ bstart, const int32_t* __restrict__ brank,
                        uint2* __restrict__ tok, int32_t* __restrict__ order) {
  const int64_t x = (int64_t)blockIdx.x * kKnnThreads + threadIdx.x;
  if (x >= n_tok) return;
  const int64_t b = x / N;
  const int e = (int)(x - b * N);
  const KnnBuckets bg = knn_buckets(N, G);
  const double step = (double)(1 << bg.shift);
  const float2 c = reinterpret_cast<const float2*>(coords)[x];
  const uint32_t qx = quantize_axis(c.x, step), qy = quantize_axis(c.y, step);
  const int bk = (int)((qy >> bg.bs) * (uint32_t)bg.Pb + (qx >> bg.bs));
  const int64_t pos = b * N + bstart[b * (bg.nb + 1) + bk] + brank[x];
  if (tok) tok[pos] = make_uint2(qx | (qy << 16), (uint32_t)e);
  if (order) order[pos] = e;
}

// grid = (B, parts), as the small-image kernel, reading the bucket arrays
template <int KM>
__global__ void __launch_bounds__(kTabThreads)
knn_table_search_kernel(int N, int G, int K, const int32_t* __restrict__ bstart,
                        const uint2* __restrict__ btok, int32_t* __restrict__ table) {
  const int b = blockIdx.x;
  const KnnBuckets bg = knn_buckets(N, G);
  const int tiles_side = (G + 7) >> 3;
  const int tile = blockIdx.y * kTabTiles + (threadIdx.x >> 6);
  if (tile >= tiles_side * tiles_side) return;
  table_tile<KM, true>(bstart + (int64_t)b * (bg.nb + 1), btok + (int64_t)b * N, N, bg, G, K, tile,
                       table + (int64_t)b * G * G * K);
}

// ---------------------------------------------------------------------------
// Per-query weights, shared by the forward and the query-major backward.
// ---------------------------------------------------------------------------
// KM = compile-time bound on K (4, 8 or 16): register arrays sized to it
template <int KM>
struct QueryWeights {
  int slot[KM];
  float w[KM];    // 0 on empty slots
  float d[KM];    // 0 on empty slots
  float2 diff[KM];
};

template <int KM>
__device__ __forceinline__ void query_weights(const float2 q, int b, int G, int K, int N, float p,
                                              const float2* __restrict__ xy,
                                              const int32_t* __restrict__ table,
                                              QueryWeights<KM>& qw) {
  // nearest cell: floor(x + 1/2) in fp64 (exact for f32 inputs), clamped
  int j = (int)fmin(fmax(floor((double)q.x + 0.5), 0.0), (double)(G - 1));
  int i = (int)fmin(fmax(floor((double)q.y + 0.5), 0.0), (double)(G - 1));
  const int32_t* row = table + (((int64_t)b * G + i) * G + j) * K;
  // the row, then every slot's coordinates, loaded unconditionally (clamped
  // indices, masked below) so that the loads are issued together
  int sl[KM];
#pragma unroll
  for (int k = 0; k < KM; ++k) sl[k] = row[min(k, K - 1)];
  float2 x[KM];
#pragma unroll
  for (int k = 0; k < KM; ++k) x[k] = N > 0 ? xy[min(max(sl[k], 0), N - 1)] : make_float2(0.f, 0.f);
  float mx = -INFINITY;
#pragma unroll
  for (int k = 0; k < KM; ++k) {
    const bool ok = k < K && sl[k] >= 0 && sl[k] < N;
    const float dx = q.x - x[k].x, dy = q.y - x[k].y;
    qw.slot[k] = ok ? sl[k] : -1;
    qw.diff[k] = ok ? make_float2(dx, dy) : make_float2(0.f, 0.f);
    qw.d[k] = ok ? sqrtf(fmaf(dx, dx, dy * dy)) : 0.f;
    if (ok) mx = fmaxf(mx, -p * qw.d[k]);
  }
  float sum = 0.f;
#pragma unroll
  for (int k = 0; k < KM; ++k) {
    qw.w[k] = 0.f;
    if (qw.slot[k] >= 0) {
      qw.w[k] = __builtin_amdgcn_exp2f((-p * qw.d[k] - mx) * 1.4426950408889634f);
      sum += qw.w[k];
    }
  }
  const float inv = sum > 0.f ? 1.f / sum : 0.f;
#pragma unroll
  for (int k = 0; k < KM; ++k) qw.w[k] *= inv;
}

// 16 bytes of a feature row as floats
template <typename T>
struct Chunk;
template <>
struct Chunk<float> {
  static constexpr int E = 4;
  static constexpr int NR = 4;   // chunks per lane at most
  __device__ static uint4 raw(const float* p) { return *reinterpret_cast<const uint4*>(p); }
  __device__ static void cvt(uint4 a, float* v) {
    v[0] = __uint_as_float(a.x); v[1] = __uint_as_float(a.y);
    v[2] = __uint_as_float(a.z); v[3] = __uint_as_float(a.w);
  }
  __device__ static void load(const float* p, float* v) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  }
  __device__ static void store(float* p, const float* v) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  }
  // acc + <a, b> over the chunk, in order
  __device__ static float dot(uint4 a, uint4 b, float acc) {
    acc = fmaf(__uint_as_float(a.x), __uint_as_float(b.x), acc);
    acc = fmaf(__uint_as_float(a.y), __uint_as_float(b.y), acc);
    acc = fmaf(__uint_as_float(a.z), __uint_as_float(b.z), acc);
    return fmaf(__uint_as_float(a.w), __uint_as_float(b.w), acc);
  }
};
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
// acc + a0 b0 + a1 b1 of two packed pairs, one instruction (v_dot2c_f32_*):
// the half-precision products are exact in fp32
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc, bf16*) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b),
                                         acc, false);
}
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc, f16*) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), acc,
                                false);
}
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
// eight bf16 / fp16 values: widening is exact, narrowing rounds to nearest even
template <typename H, typename V>
struct HalfChunk {
  static constexpr int E = 8;
  static constexpr int NR = 3;   // chunks per lane at most
  __device__ static uint4 raw(const H* p) { return *reinterpret_cast<const uint4*>(p); }
  __device__ static void cvt(uint4 a, float* v) {
    const f32x8 f = __builtin_convertvector(__builtin_bit_cast(V, a), f32x8);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = f[e];
  }
  __device__ static void load(const H* p, float* v) {
    const f32x8 f = __builtin_convertvector(__builtin_bit_cast(V, *reinterpret_cast<const uint4*>(p)), f32x8);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = f[e];
  }
  __device__ static void store(H* p, const float* v) {
    const f32x8 f = {v[0], v[1], v[2], v[3], v[4], v[5], v[6], v[7]};
    *reinterpret_cast<uint4*>(p) = __builtin_bit_cast(uint4, __builtin_convertvector(f, V));
  }
  // acc + <a, b> over the chunk: four pair products, each pair summed first
  __device__ static float dot(uint4 a, uint4 b, float acc) {
    acc = dot2(a.x, b.x, acc, (H*)nullptr);
    acc = dot2(a.y, b.y, acc, (H*)nullptr);
    acc = dot2(a.z, b.z, acc, (H*)nullptr);
    return dot2(a.w, b.w, acc, (H*)nullptr);
  }
};
template <>
struct Chunk<bf16> : HalfChunk<bf16, bf16x8> {};
template <>
struct Chunk<f16> : HalfChunk<f16, f16x8> {};


// Lane-group geometry: a group of L = 2^lg lanes serves one query (or one
// token); lane `sub` of the group covers chunks sub, sub + L.
struct Group {
  int64_t id;   // global query / token number
  int sub;
  bool valid;
};
__device__ __forceinline__ Group group_of(int lg, int64_t total) {
  const int lane = threadIdx.x & 63;
  Group g;
  const int64_t wave = (int64_t)blockIdx.x * (kKnnThreads / 64) + (threadIdx.x >> 6);
  g.id = wave * (64 >> lg) + (lane >> lg);
  g.sub = lane & ((1 << lg) - 1);
  g.valid = g.id < total;
  return g;
}

// ---------------------------------------------------------------------------
// Forward.  out[b, m] = sum_k w_k F[b, slot_k].  A wave serves qwv
// consecutive queries (eight passes of its lane groups): first one lane per
// query works out the slots and weights (the dependent chain query -> table
// row -> token coordinates is paid once per wave) and leaves them in LDS;
// then lane groups of L lanes (16 bytes of the row each) gather and sum the
// rows, 64 / L queries at a time.
// ---------------------------------------------------------------------------
template <int KM>
struct WaveSlots {
  int slot[64][KM];
  float w[64][KM];
};

template <int KM>
__device__ __forceinline__ void wave_slots(int64_t base, int64_t total, int qwv, int N, int M, int G, int K,
                                           float p, const float* __restrict__ coords,
                                           const float* __restrict__ queries,
                                           const int32_t* __restrict__ table, WaveSlots<KM>& ws,
                                           QueryWeights<KM>& qw) {
  const int lane = threadIdx.x & 63;
  const int64_t id = base + lane;
#pragma unroll
  for (int k = 0; k < KM; ++k) {
    qw.slot[k] = -1;
    qw.w[k] = 0.f;
    qw.d[k] = 0.f;
    qw.diff[k] = make_float2(0.f, 0.f);
  }
  if (lane < qwv && id < total) {
    const int64_t b = id / M;
    const float2 q = reinterpret_cast<const float2*>(queries)[id];
    query_weights(q, (int)b, G, K, N, p, reinterpret_cast<const float2*>(coords) + b * N, table, qw);
  }
#pragma unroll
  for (int k = 0; k < KM; ++k) {
    ws.slot[lane][k] = qw.slot[k];
    ws.w[lane][k] = qw.w[k];
  }
  __builtin_amdgcn_wave_barrier();   // one wave: its LDS writes precede its reads
}

template <typename T, int KM, int NRM>
__global__ void __launch_bounds__(kKnnThreads)
knn_fwd_kernel(int N, int M, int Cf, int G, int K, int lg, float p, int64_t total, int qwv,
               const float* __restrict__ coords, const T* __restrict__ feats,
               const float* __restrict__ queries, const int32_t* __restrict__ table,
               T* __restrict__ out) {
  using Ck = Chunk<T>;
  __shared__ WaveSlots<KM> sw[kKnnThreads / 64];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t base = ((int64_t)xcd_remap(blockIdx.x, gridDim.x) * (kKnnThreads / 64) + wv) * qwv;
  if (base >= total) return;
  QueryWeights<KM> qw;
  wave_slots<KM>(base, total, qwv, N, M, G, K, p, coords, queries, table, sw[wv], qw);
  const int L = 1 << lg;
  const int grp = lane >> lg, sub = lane & (L - 1);
  const int nch = Cf / Ck::E;
  const int nr = (nch - sub + L - 1) / L;   // chunks of this lane
  const int cs = min(sub, nch - 1);   // idle lanes (sub >= nch, nr = 0) load inside the row
#pragma unroll 2
  for (int u0 = 0; u0 < qwv; u0 += 64 >> lg) {
    const int u = u0 + grp;
    const int64_t id = base + u;
    if (id >= total) break;
    const int64_t b = id / M;
    const T* fimg = feats + b * N * Cf;
    int sl[KM];
    float wt[KM];
#pragma unroll
    for (int k = 0; k < KM; ++k) {
      sl[k] = sw[wv].slot[u][k];
      wt[k] = sw[wv].w[u][k];
    }
    // every chunk's rows in flight before the sums: an empty slot reads a
    // valid row (masked afterwards); a lane with fewer chunks than NRM skips
    // the last round's loads
    uint4 raw[NRM][KM];
    if (N > 0) {
#pragma unroll
      for (int r = 0; r < NRM; ++r)
        if (r < nr) {
#pragma unroll
          for (int k = 0; k < KM; ++k)
            raw[r][k] = Ck::raw(fimg + (int64_t)max(sl[k], 0) * Cf + (cs + r * L) * Ck::E);
        }
    }
#pragma unroll
    for (int r = 0; r < NRM; ++r) {
      if (r >= nr) break;
      float acc[Ck::E];
#pragma unroll
      for (int e = 0; e < Ck::E; ++e) acc[e] = 0.f;
#pragma unroll
      for (int k = 0; k < KM; ++k) {
        if (sl[k] < 0) raw[r][k] = make_uint4(0u, 0u, 0u, 0u);
        float v[Ck::E];
        Ck::cvt(raw[r][k], v);
#pragma unroll
        for (int e = 0; e < Ck::E; ++e) acc[e] = fmaf(wt[k], v[e], acc[e]);
      }
      Ck::store(out + id * Cf + (cs + r * L) * Ck::E, acc);
    }
  }
}

// ---------------------------------------------------------------------------
// Backward, query-major part.  Same wave layout as the forward: (1) lane =
// query: slots and weights (kept in registers, in LDS for the groups, and
// in the workspace for the feature gradient); (2) lane groups: <dO, F_k>
// reduced over the group, into LDS; (3) lane = query again: dq and the
// query's share of dp.
// ---------------------------------------------------------------------------
template <typename T, int KM, int NRM>
__global__ void __launch_bounds__(kKnnThreads) __attribute__((amdgpu_waves_per_eu(sizeof(T) == 2 && KM <= 8 ? (NRM == 1 ? 4 : NRM == 2 ? 3 : 2) : 1)))
knn_bwd_query_kernel(int N, int M, int Cf, int G, int K, int lg, float p, int64_t total, int qwv,
                     const float* __restrict__ coords, const T* __restrict__ feats,
                     const float* __restrict__ queries, const int32_t* __restrict__ table,
                     const T* __restrict__ dout, float* __restrict__ dq, float* __restrict__ dpart,
                     int32_t* __restrict__ ent_slot, float* __restrict__ ent_w,
                     int32_t* __restrict__ cnt) {
  using Ck = Chunk<T>;
  __shared__ WaveSlots<KM> sw[kKnnThreads / 64];
  __shared__ float sg[kKnnThreads / 64][64][KM];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t base = ((int64_t)xcd_remap(blockIdx.x, gridDim.x) * (kKnnThreads / 64) + wv) * qwv;
  if (base >= total) return;
  QueryWeights<KM> qw;
  wave_slots<KM>(base, total, qwv, N, M, G, K, p, coords, queries, table, sw[wv], qw);
  {
    const int64_t id = base + lane;
    if (lane < qwv && id < total) {
#pragma unroll
      for (int k = 0; k < KM; ++k) {
        if (k >= K) break;
        ent_slot[id * K + k] = qw.slot[k];
        ent_w[id * K + k] = qw.w[k];
      }
    }
  }
  const int L = 1 << lg;
  const int grp = lane >> lg, sub = lane & (L - 1);
  const int nch = Cf / Ck::E;
  const int nr = (nch - sub + L - 1) / L;   // chunks of this lane
  const int cs = min(sub, nch - 1);   // idle lanes (sub >= nch, nr = 0) load inside the row
  for (int u0 = 0; u0 < qwv; u0 += 64 >> lg) {   // uniform trip count: shuffles below
    const int u = u0 + grp;
    const int64_t id = base + u;
    const bool live = id < total;
    const int64_t b = (live ? id : base) / M;
    const T* fimg = feats + b * N * Cf;
    int sl[KM];
#pragma unroll
    for (int k = 0; k < KM; ++k) sl[k] = live ? sw[wv].slot[u][k] : -1;
    float gk[KM];
#pragma unroll
    for (int k = 0; k < KM; ++k) gk[k] = 0.f;
    // all loads issued before the sums (see the forward), masked afterwards
    uint4 raw[NRM][KM], oraw[NRM];
    const int64_t oid = live ? id : base;
#pragma unroll
    for (int r = 0; r < NRM; ++r)
      if (r < nr) {
        const int c = cs + r * L;
        oraw[r] = Ck::raw(dout + oid * Cf + c * Ck::E);
        if (N > 0) {
#pragma unroll
          for (int k = 0; k < KM; ++k) raw[r][k] = Ck::raw(fimg + (int64_t)max(sl[k], 0) * Cf + c * Ck::E);
        }
      }
#pragma unroll
    for (int r = 0; r < NRM; ++r) {
      if (r >= nr || !live) break;
#pragma unroll
      for (int k = 0; k < KM; ++k) {
        if (sl[k] < 0) raw[r][k] = make_uint4(0u, 0u, 0u, 0u);
        gk[k] = Ck::dot(oraw[r], raw[r][k], gk[k]);
      }
    }
    if (L >= KM) {
      // Sum over the group with the values split as they go: at offsets
      // 1, 2, 4, ... a lane keeps half of its values (the half picked by the
      // offset's bit of its lane number) and adds the partner's copy of that
      // half; after log2(KM) such rounds lane l holds one value, index
      // rev(l mod KM), summed over KM lanes, and the remaining offsets add
      // the group's other lanes.  A fixed pattern: deterministic.
      float vv[KM];
#pragma unroll
      for (int k = 0; k < KM; ++k) vv[k] = gk[k];
#pragma unroll
      for (int o = 1, V = KM; o < KM; o <<= 1, V >>= 1) {
        const bool hi = (lane & o) != 0;
#pragma unroll
        for (int i = 0; i < V / 2; ++i) {
          const float send = hi ? vv[i] : vv[i + V / 2];
          const float keep = hi ? vv[i + V / 2] : vv[i];
          vv[i] = keep + __shfl_xor(send, o, 64);
        }
      }
      for (int o = KM; o < L; o <<= 1) vv[0] += __shfl_xor(vv[0], o, 64);
      if ((sub & ~(KM - 1)) == 0) {
        int idx = 0;   // value index held by this lane: bit j of the lane -> KM / 2^(j+1)
#pragma unroll
        for (int o = 1, h = KM / 2; o < KM; o <<= 1, h >>= 1) idx += (lane & o) ? h : 0;
        sg[wv][u][idx] = vv[0];
      }
    } else {
      for (int off = 1; off < L; off <<= 1)
#pragma unroll
        for (int k = 0; k < KM; ++k) gk[k] += __shfl_xor(gk[k], off, 64);
      if (sub == 0)
#pragma unroll
        for (int k = 0; k < KM; ++k) sg[wv][u][k] = gk[k];
    }
  }
  __builtin_amdgcn_wave_barrier();
  const int64_t id0 = base + lane;
  const bool mine = lane < qwv && id0 < total;
  const int64_t id = mine ? id0 : base;   // idle lanes mirror the first query (shuffle below)
  float g[KM];
#pragma unroll
  for (int k = 0; k < KM; ++k) g[k] = sg[wv][lane][k];
  float delta = 0.f;
#pragma unroll
  for (int k = 0; k < KM; ++k) delta = fmaf(qw.w[k], g[k], delta);
  float dqx = 0.f, dqy = 0.f, dps = 0.f;
#pragma unroll
  for (int k = 0; k < KM; ++k) {
    if (qw.slot[k] < 0) continue;
    const float ds = qw.w[k] * (g[k] - delta);   // dL / d(-p d_k)
    dps = fmaf(-ds, qw.d[k], dps);
    if (qw.d[k] > 0.f) {
      const float f = -p * ds / qw.d[k];
      dqx = fmaf(f, qw.diff[k].x, dqx);
      dqy = fmaf(f, qw.diff[k].y, dqy);
    }
  }
  if (mine) reinterpret_cast<float2*>(dq)[id] = make_float2(dqx, dqy);
  // the wave's dp shares summed in a fixed order (lanes past the end add 0)
  float sdp = mine ? dps : 0.f;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) sdp += __shfl_xor(sdp, o, 64);
  if (lane == 0) dpart[base / qwv] = sdp;
  // the entries' counts per token (integer atomics, order independent),
  // last: nothing in this wave waits on them.  Large images only (pcnt =
  // the per-token counts); small ones count per partition in
  // knn_pcount_kernel instead.
  if (mine && cnt) {
    const int64_t b = id / M;
#pragma unroll
    for (int k = 0; k < KM; ++k)
      if (k < K && qw.slot[k] >= 0) atomicAdd(&cnt[b * N + qw.slot[k]], 1);
  }
}

// Spatial walk order of the tokens for the feature gradient: the tokens of
// an image bucketed on a coarse grid (about two per bucket) in LDS, so that
// the waves resident at one time work on neighbouring tokens, which share
// most of their queries (and so the dO rows they gather stay in L2).  Any
// order gives the same result: each token's sum has its own fixed order.
// One workgroup of NT threads per image of at most kTabMaxTokens tokens;
// start holds kTabMaxBuckets ints of LDS, tmp 17.
template <int NT>
__device__ __forceinline__ void order_image(const float* __restrict__ coords, int N, int G, int64_t b,
                                            int* start, int* tmp, int32_t* __restrict__ order) {
  const int tid = threadIdx.x;
  const KnnBuckets bg = knn_buckets(N, G);
  const double step = (double)(1 << bg.shift);
  const int bs = bg.bs, Pb = bg.Pb, nb = bg.nb;
  const float2* xy = reinterpret_cast<const float2*>(coords) + b * N;
  for (int x = tid; x < nb; x += NT) start[x] = 0;
  __syncthreads();
  constexpr int kPer = kTabMaxTokens / NT;
  int bk[kPer], rk[kPer];
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    const int e = tid + r * NT;
    bk[r] = -1;
    if (e < N) {
      const float2 c = xy[e];
      const uint32_t qx = quantize_axis(c.x, step), qy = quantize_axis(c.y, step);
      // buckets in row-major order of the coarse grid
      bk[r] = (int)((qy >> bs) * (uint32_t)Pb + (qx >> bs));
      rk[r] = atomicAdd(&start[bk[r]], 1);
    }
  }
  __syncthreads();
  constexpr int kBPer = kTabMaxBuckets / NT;
  int cnt[kBPer];
  int run = 0;
#pragma unroll
  for (int r = 0; r < kBPer; ++r) {
    const int x = tid * kBPer + r;
    cnt[r] = x < nb ? start[x] : 0;
    run += cnt[r];
  }
  int total;
  int acc = block_exclusive_scan(run, tmp, NT, &total);
#pragma unroll
  for (int r = 0; r < kBPer; ++r) {
    const int x = tid * kBPer + r;
    if (x < nb) start[x] = acc;
    acc += cnt[r];
  }
  __syncthreads();
  int32_t* ord = order + b * N;
#pragma unroll
  for (int r = 0; r < kPer; ++r)
    if (bk[r] >= 0) ord[start[bk[r]] + rk[r]] = tid + r * NT;
}

// Per partition of kPart entries, the count of its entries per token,
// accumulated in LDS (images of at most kTabMaxTokens tokens; integer
// atomics, order independent) and written out whole (zeros included): one
// workgroup of kChunkThreads per partition, each thread kChunkPer entries.
// The launch also carries the walk order: workgroups nparts .. nparts + B - 1
// build it for one image each (order_image).
constexpr int kChunkWaves = 8;
constexpr int kChunkThreads = 64 * kChunkWaves;
constexpr int kChunkPer = kPart / kChunkThreads;   // entries per thread
__global__ void __launch_bounds__(kChunkThreads)
knn_pcount_kernel(int N, int G, int64_t MK, int P, int64_t nparts, const int32_t* __restrict__ ent_slot,
                  const float* __restrict__ coords, int32_t* __restrict__ pcnt,
                  int32_t* __restrict__ order) {
  static_assert(kPart % kChunkThreads == 0, "whole entries per thread");
  static_assert(kTabMaxBuckets == kTabMaxTokens, "one LDS array serves both");
  __shared__ int32_t c[kTabMaxTokens];
  __shared__ int tmp[17];
  const int64_t part = blockIdx.x;
  if (part >= nparts) {
    order_image<kChunkThreads>(coords, N, G, part - nparts, c, tmp, order);
    return;
  }
  const int64_t b = part / P;
  const int s = (int)(part - b * P);
  const int64_t e0 = (int64_t)s * kPart;
  int tv[kChunkPer];
#pragma unroll
  for (int r = 0; r < kChunkPer; ++r) {
    const int64_t x = e0 + r * kChunkThreads + threadIdx.x;
    tv[r] = x < MK ? ent_slot[b * MK + x] : -1;
  }
  for (int t = threadIdx.x; t < N; t += kChunkThreads) c[t] = 0;
  __syncthreads();
#pragma unroll
  for (int r = 0; r < kChunkPer; ++r)
    if (tv[r] >= 0) atomicAdd(&c[tv[r]], 1);
  __syncthreads();
  int32_t* row = pcnt + (b * P + s) * N;
  for (int t = threadIdx.x; t < N; t += kChunkThreads) row[t] = c[t];
}

// Token-major entry lists, in entry order (entry = query * K + slot), each
// entry stored as its (query, weight) pair, by a stable counting sort.  The
// entries of an image are cut into partitions of kPart consecutive entries:
// (1) per partition and token, the count of its entries, in LDS
// (knn_pcount_kernel); (2) per token, the counts turned into exclusive
// prefixes over the partitions, and the token's total; (3) the totals
// scanned into segment starts (launch_segment_scan); (4) per partition, every
// entry placed at segment start + the partition's prefix + the number of
// earlier entries of the same token in the partition.

// Per token, the partition counts turned into exclusive prefixes over the
// partitions, and the token's total.  Workgroup = 64 consecutive tokens of
// one image (lane = token: coalesced rows of the counts); its kPrefWaves
// waves split the partitions into contiguous ranges, sum them, exchange the
// range sums through LDS, and rewrite their ranges as running prefixes.
constexpr int kPrefWaves = 16;
__global__ void __launch_bounds__(64 * kPrefWaves)
knn_pprefix_kernel(int N, int P, int tgroups, int32_t* __restrict__ pcnt,
                   int32_t* __restrict__ cnt) {
  __shared__ int part[kPrefWaves][64];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t b = blockIdx.x / tgroups;
  const int t = (int)(blockIdx.x - b * tgroups) * 64 + lane;
  const bool live = t < N;
  const int per = (P + kPrefWaves - 1) / kPrefWaves;
  const int s0 = wv * per, s1 = min(P, s0 + per);
  int32_t* col = pcnt + b * P * N + (live ? t : 0);
  int sum = 0;
  for (int s = s0; s < s1; s += 8) {   // eight loads in flight
    int v[8];
#pragma unroll
    for (int h = 0; h < 8; ++h) v[h] = (live && s + h < s1) ? col[(int64_t)(s + h) * N] : 0;
#pragma unroll
    for (int h = 0; h < 8; ++h) sum += v[h];
  }
  part[wv][lane] = sum;
  __syncthreads();
  int acc = 0;
  for (int w = 0; w < wv; ++w) acc += part[w][lane];
  if (wv == kPrefWaves - 1 && live) cnt[b * N + t] = acc + sum;
  for (int s = s0; s < s1; s += 8) {
    int v[8];
#pragma unroll
    for (int h = 0; h < 8; ++h) v[h] = (live && s + h < s1) ? col[(int64_t)(s + h) * N] : 0;
#pragma unroll
    for (int h = 0; h < 8; ++h) {
      if (live && s + h < s1) col[(int64_t)(s + h) * N] = acc;
      acc += v[h];
    }
  }
}

// One workgroup of kChunkWaves waves per partition.  Wave w takes the
// partition's entries [w kChunkRun, (w + 1) kChunkRun) (wave order is entry
// order) in batches of 64: (1) each wave counts its entries per token in
// its own LDS row (integer atomics); (2) per token, the rows become the
// waves' first places: segment start + the partition's prefix + the counts
// of the earlier waves; (3) each wave walks its batches in order: lanes
// holding the same token find each other by matching the token's bits with
// ballots, an entry goes to its wave's place + the number of equal tokens
// in lower lanes, and the last such lane advances the place.  Dynamic LDS:
// kChunkWaves x N ints.
constexpr int kChunkRun = kPart / kChunkWaves;    // entries per wave
constexpr int kChunkBatches = kChunkRun / 64;
__global__ void __launch_bounds__(kChunkThreads)
knn_pplace_kernel(int N, int K, int64_t MK, int P, const int32_t* __restrict__ ent_slot,
                  const float* __restrict__ ent_w, const int32_t* __restrict__ off_all,
                  const int32_t* __restrict__ pcnt, int2* __restrict__ ent_all) {
  static_assert(kChunkRun % 64 == 0, "whole batches per wave");
  extern __shared__ int32_t cw[];   // [kChunkWaves][N]
  const int64_t part = blockIdx.x;
  const int64_t b = part / P;
  const int s = (int)(part - b * P);
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t ew0 = (int64_t)s * kPart + wv * kChunkRun;
  int tk[kChunkBatches];
  float wk[kChunkBatches];
#pragma unroll
  for (int h = 0; h < kChunkBatches; ++h) {
    const int64_t x = ew0 + h * 64 + lane;
    tk[h] = x < MK ? ent_slot[b * MK + x] : -1;
    wk[h] = x < MK ? ent_w[b * MK + x] : 0.f;
  }
  for (int t = threadIdx.x; t < N; t += kChunkThreads)
#pragma unroll
    for (int w = 0; w < kChunkWaves; ++w) cw[w * N + t] = 0;
  __syncthreads();
  int32_t* mine = cw + wv * N;
#pragma unroll
  for (int h = 0; h < kChunkBatches; ++h)
    if (tk[h] >= 0) atomicAdd(&mine[tk[h]], 1);
  __syncthreads();
  const int32_t* off = off_all + b * (N + 1);
  const int32_t* pre = pcnt + (b * P + s) * N;
  for (int t = threadIdx.x; t < N; t += kChunkThreads) {
    int base = off[t] + pre[t];
#pragma unroll
    for (int w = 0; w < kChunkWaves; ++w) {
      const int c = cw[w * N + t];
      cw[w * N + t] = base;
      base += c;
    }
  }
  __syncthreads();
  const int nbits = N > 1 ? 32 - __clz(N - 1) : 0;   // token bits
  const uint64_t below = (uint64_t(1) << lane) - 1;
  const uint64_t upto = lane == 63 ? ~uint64_t(0) : (uint64_t(2) << lane) - 1;
  int2* ent = ent_all + b * MK;
#pragma unroll
  for (int h = 0; h < kChunkBatches; ++h) {
    const int t = tk[h];
    // lanes holding the same valid token (0 for an empty slot)
    const bool ok = t >= 0;
    uint64_t same = __ballot(ok);
    for (int i = 0; i < nbits; ++i) {
      const bool bit = (t >> i) & 1;
      const uint64_t on = __ballot(ok && bit);
      same &= bit ? on : ~on;
    }
    if (ok) {
      const int pos = mine[t] + __popcll(same & below);
      ent[pos] = make_int2((int)((ew0 + h * 64 + lane) / K), __float_as_int(wk[h]));
      if ((same & ~upto) == 0) mine[t] = pos + 1;
    }
  }
}

// Large images: token-major entry lists by per-token cursors.  (1) The
// query-major kernel counts the entries per token; (2) launch_segment_scan
// turns the counts into segment starts; (3) every entry takes a place in
// its token's segment of lst from an integer atomic on the token's cursor
// (in no fixed order); (4) every entry is moved to segment start + its rank
// among the segment's entries by entry number (segments longer than
// kLongSegment are sorted by launch_long_segment_sort instead, bounding the
// cost).  The lists come out in entry order, as from the stable counting
// sort of small images.
// The lanes of a wave holding the same token (consecutive entries: a few
// neighbouring queries, which share most of their tokens) find each other
// by ballots over the bits in which the wave's token ids differ: the mask
// of the lanes whose key equals this lane's (0 where !ok).  Wave-uniform.
__device__ __forceinline__ uint64_t wave_same_key(uint32_t key, bool ok) {
  const uint32_t key0 = (uint32_t)__builtin_amdgcn_readfirstlane((int)key);
  uint32_t diff = ok ? key ^ key0 : 0u;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) diff |= (uint32_t)__shfl_xor((int)diff, o, 64);
  uint64_t same = __ballot(ok);
  for (uint32_t d = diff; d != 0u; d &= d - 1u) {
    const int i = __builtin_ctz(d);
    const bool bit = (key >> i) & 1u;
    const uint64_t on = __ballot(ok && bit);
    same &= bit ? on : ~on;
  }
  return ok ? same : uint64_t(0);
}

// Such a group takes its places with one atomic: the lowest lane adds the
// group's count, and each lane takes the returned base + its rank in the
// group (its entries stay in entry order, side by side).
__global__ void __launch_bounds__(kKnnThreads)
knn_lplace_kernel(int N, int64_t MK, int64_t n_ent, const int32_t* __restrict__ ent_slot,
                  const int32_t* __restrict__ off_all, int32_t* __restrict__ cur,
                  int32_t* __restrict__ lst) {
  const int64_t x = (int64_t)blockIdx.x * kKnnThreads + threadIdx.x;
  const int lane = threadIdx.x & 63;
  const int t = x < n_ent ? ent_slot[x] : -1;
  const bool ok = t >= 0;
  const int64_t b = ok ? x / MK : 0;
  const uint32_t key = ok ? (uint32_t)(b * N + t) : 0u;   // B N < 2^31
  const uint64_t same = wave_same_key(key, ok);
  const int rank = __popcll(same & ((uint64_t(1) << lane) - 1));
  const int leader = same ? __builtin_ctzll(same) : lane;
  int base = 0;
  if (ok && rank == 0) base = atomicAdd(&cur[key], __popcll(same));
  base = __shfl(base, leader, 64);
  if (ok) lst[b * MK + off_all[b * (N + 1) + t] + base + rank] = (int32_t)(x - b * MK);
}

__global__ void __launch_bounds__(kKnnThreads)
knn_lrank_kernel(int N, int K, int64_t MK, int64_t n_ent, const int32_t* __restrict__ ent_slot,
                 const float* __restrict__ ent_w, const int32_t* __restrict__ off_all,
                 const int32_t* __restrict__ lst, int2* __restrict__ ent_all) {
  // the lanes of a wave with the same token hold consecutive entries of
  // its segment: the lowest counts the segment's entries below its own, the
  // others add their rank in the group
  const int64_t x = (int64_t)blockIdx.x * kKnnThreads + threadIdx.x;
  const int lane = threadIdx.x & 63;
  const int t = x < n_ent ? ent_slot[x] : -1;
  const bool ok = t >= 0;
  const int64_t b = ok ? x / MK : 0;
  const uint64_t same = wave_same_key(ok ? (uint32_t)(b * N + t) : 0u, ok);
  const int rank = __popcll(same & ((uint64_t(1) << lane) - 1));
  const int leader = same ? __builtin_ctzll(same) : lane;
  const int e = (int)(x - b * MK);
  const int a = ok ? off_all[b * (N + 1) + t] : 0, z = ok ? off_all[b * (N + 1) + t + 1] : 0;
  const bool mine = ok && z - a <= kLongSegment;   // longer: launch_long_segment_sort
  int below = 0;
  if (mine && rank == 0) {
    const int32_t* seg = lst + b * MK;
    int y = a;
    for (; y + 8 <= z; y += 8) {   // eight loads in flight
      int v[8];
#pragma unroll
      for (int h = 0; h < 8; ++h) v[h] = seg[y + h];
#pragma unroll
      for (int h = 0; h < 8; ++h) below += v[h] < e;
    }
    for (; y < z; ++y) below += seg[y] < e;
  }
  below = __shfl(below, leader, 64);
  if (mine) ent_all[b * MK + a + below + rank] = make_int2(e / K, __float_as_int(ent_w[x]));
}


// dp = sum of the per-wave shares, in a fixed order, by one workgroup of
// NT threads
template <int NT>
__device__ __forceinline__ void dp_reduce(int64_t n, const float* __restrict__ dpart,
                                          float* __restrict__ dp, float* red) {
  float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};   // eight loads in flight
  int64_t i = threadIdx.x;
  for (; i + 7 * NT < n; i += 8 * NT)
#pragma unroll
    for (int u = 0; u < 8; ++u) a[u] += dpart[i + u * NT];
  for (; i < n; i += NT) a[0] += dpart[i];
  red[threadIdx.x] = ((a[0] + a[1]) + (a[2] + a[3])) + ((a[4] + a[5]) + (a[6] + a[7]));
  __syncthreads();
  for (int o = NT / 2; o >= 1; o >>= 1) {
    if ((int)threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) dp[0] = red[0];
}

// images without tokens: dp alone (one workgroup)
__global__ void __launch_bounds__(1024)
knn_dp_kernel(int64_t n, const float* __restrict__ dpart, float* __restrict__ dp) {
  __shared__ float red[1024];
  dp_reduce<1024>(n, dpart, dp, red);
}

// ---------------------------------------------------------------------------
// Backward, token-major part: dF[b, t] = sum over its entries of w dO[b, m].
// ---------------------------------------------------------------------------
// A group of L lanes per token (16 bytes of the row per lane); `split` waves
// share a token group and take its batches of kB entries in turn (wave w:
// batches w, w + split, ...); their partial sums are added in wave order
// through LDS, so every token's sum has one fixed order.  The (query,
// weight) pairs of the next batch load while the current batch's dO rows
// are in flight.  Workgroups are dealt XCD-aware over S image streams:
// workgroup i belongs to stream x = i mod S (dispatched to XCD i mod 8) and
// takes its token group of the images x, x + S, ... in turn; with S a
// multiple of 8 (or S = B) an image stays on one XCD, and S is picked so
// that the dO rows of the images in flight on an XCD fit its L2.  The first
// workgroup also sums the dp shares (complete: the query-major kernel has
// finished).
template <typename T, int NRM>
__global__ void __launch_bounds__(kKnnThreads) __attribute__((amdgpu_waves_per_eu(NRM == 1 ? 8 : 1)))
knn_dfeat_kernel(int B, int N, int M, int Cf, int64_t MK, int lg, int split, int S,
                 const T* __restrict__ dout, const int32_t* __restrict__ off_all,
                 const int2* __restrict__ ent_all, const int32_t* __restrict__ order,
                 T* __restrict__ dfeat, int64_t n_dp, const float* __restrict__ dpart,
                 float* __restrict__ dp) {
  using Ck = Chunk<T>;
  // entries (rows) per batch: four for one-chunk rows, which keeps the
  // kernel within 64 registers (eight waves per SIMD hide the dependent
  // order -> offsets -> pairs -> rows chain of the short token lists)
  constexpr int kB = NRM == 1 ? 4 : 8;
  constexpr int kW = kKnnThreads / 64;           // waves per workgroup
  __shared__ float part[kW][NRM * Ck::E][64];
  if (blockIdx.x == 0) {
    __shared__ float red[kKnnThreads];
    dp_reduce<kKnnThreads>(n_dp, dpart, dp, red);
  }
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int x = (int)(blockIdx.x % S), gi = (int)(blockIdx.x / S);
  const int L = 1 << lg, sub = lane & (L - 1);
  // `split` waves share a token group; the workgroup covers kW / split groups
  const int grp = gi * (kW / split) + wv / split, sw = wv % split;
  const int pos = grp * (64 >> lg) + (lane >> lg);   // token position in the walk order
  const int nch = Cf / Ck::E;
  const int nr = (nch - sub + L - 1) / L;            // chunks of this lane
  const int cs = min(sub, nch - 1);   // idle lanes (sub >= nch, nr = 0) load inside the row
  for (int img = x; img < B; img += S) {
    const int64_t b = img;
    const bool live = pos < N;
    const int t = live ? order[b * N + pos] : 0;
    const int a = live ? off_all[b * (N + 1) + t] : 0;
    const int z = live ? off_all[b * (N + 1) + t + 1] : 0;
    const int2* ent = ent_all + b * MK;
    const T* oimg = dout + b * M * Cf;
    float acc[NRM][Ck::E];
#pragma unroll
    for (int r = 0; r < NRM; ++r)
#pragma unroll
      for (int e = 0; e < Ck::E; ++e) acc[r][e] = 0.f;
    int u = a + sw * kB;
    int2 pr[kB];
    if (u < z) {
#pragma unroll
      for (int h = 0; h < kB; ++h) pr[h] = ent[min(u + h, z - 1)];
    }
    while (u < z) {
      // this batch's rows (clamped entries, masked afterwards; a lane with
      // fewer chunks than NRM skips the last round), then the next batch's
      // pairs (clamped inside the segment)
      uint4 raw[NRM][kB];
#pragma unroll
      for (int r = 0; r < NRM; ++r)
        if (r < nr) {
#pragma unroll
          for (int h = 0; h < kB; ++h)
            raw[r][h] = Ck::raw(oimg + (int64_t)pr[h].x * Cf + (cs + r * L) * Ck::E);
        }
      const int un = u + split * kB;
      int2 nx[kB];
#pragma unroll
      for (int h = 0; h < kB; ++h) nx[h] = ent[min(un + h, z - 1)];
#pragma unroll
      for (int r = 0; r < NRM; ++r) {
        if (r >= nr) break;
#pragma unroll
        for (int h = 0; h < kB; ++h) {
          if (u + h >= z) raw[r][h] = make_uint4(0u, 0u, 0u, 0u);
          float v[Ck::E];
          Ck::cvt(raw[r][h], v);
          const float wt = __int_as_float(pr[h].y);
#pragma unroll
          for (int q = 0; q < Ck::E; ++q) acc[r][q] = fmaf(wt, v[q], acc[r][q]);
        }
      }
#pragma unroll
      for (int h = 0; h < kB; ++h) pr[h] = nx[h];
      u = un;
    }
    // partial sums of the group's other waves to its first, added in wave order
    if (split > 1) {
      if (sw > 0) {
#pragma unroll
        for (int r = 0; r < NRM; ++r)
#pragma unroll
          for (int q = 0; q < Ck::E; ++q) part[wv][r * Ck::E + q][lane] = acc[r][q];
      }
      __syncthreads();
      if (sw == 0) {
        for (int v2 = 1; v2 < split; ++v2)
#pragma unroll
          for (int r = 0; r < NRM; ++r)
#pragma unroll
            for (int q = 0; q < Ck::E; ++q) acc[r][q] += part[wv + v2][r * Ck::E + q][lane];
      }
      __syncthreads();   // part is reused by the next image
    }
    if (sw == 0 && live) {
#pragma unroll
      for (int r = 0; r < NRM; ++r) {
        if (r >= nr) break;
        Ck::store(dfeat + (b * N + t) * Cf + (cs + r * L) * Ck::E, acc[r]);
      }
    }
  }
}

// Lane-group width 2^lg for rows of Cf / E chunks: the width whose
// rounds (chunks per lane, at most maxr) leave the fewest lanes idle, the
// wider one on ties (e.g. 96 chunks: 32 lanes x 3, not 64 lanes x 2 with
// half the lanes idle in the second round).
int group_log2(int Cf, int E, int maxr) {
  const int nch = Cf / E;
  int best = 6;
  int64_t bn = 0, bd = 1;   // best utilisation nch / (L r), as a fraction
  for (int lg = 6; lg >= 0; --lg) {
    const int L = 1 << lg, r = (nch + L - 1) / L;
    if (r > maxr) break;
    if ((int64_t)nch * bd > bn * (int64_t)(L * r)) {
      bn = nch;
      bd = (int64_t)L * r;
      best = lg;
    }
  }
  return best;
}

// Chunks of 16 bytes per lane at most (lane groups of 2^lg lanes)
int chunks_per_lane(int Cf, int E, int lg) { return (Cf / E + (1 << lg) - 1) >> lg; }

// Lane-group width of a row type: at most Chunk<T>::NR chunks per lane
template <typename T>
int row_group_log2(int Cf) { return group_log2(Cf, Chunk<T>::E, Chunk<T>::NR); }

// Kernel instance by the chunks a lane holds at most (1 .. Chunk<T>::NR)
template <typename T, typename F>
void with_chunks(int nrm, F&& f) {
  if (nrm <= 1) f(std::integral_constant<int, 1>{});
  else if (nrm <= 2) f(std::integral_constant<int, 2>{});
  else if constexpr (Chunk<T>::NR == 3) f(std::integral_constant<int, 3>{});
  else if (nrm <= 3) f(std::integral_constant<int, 3>{});
  else f(std::integral_constant<int, 4>{});
}

// Queries per wave of the forward and the query-major backward: eight
// passes of 64 / L queries (L lanes per query), at most 64.
int queries_per_wave(int lg) { return std::min(64, 512 >> lg); }

unsigned blocks_for(int64_t total, int qwv) {
  const int64_t waves = (total + qwv - 1) / qwv;
  return (unsigned)((waves + kKnnThreads / 64 - 1) / (kKnnThreads / 64));
}

unsigned waves_grid(int64_t groups, int lg) {
  const int64_t per_wave = 64 >> lg;
  const int64_t waves = (groups + per_wave - 1) / per_wave;
  return (unsigned)((waves + kKnnThreads / 64 - 1) / (kKnnThreads / 64));
}

template <typename T>
hipError_t fwd_t(int B, int N, int M, int Cf, int G, int K, float p, const float* coords,
                 const void* feats, const float* queries, const int32_t* table, void* out,
                 hipStream_t st) {
  const int lg = row_group_log2<T>(Cf);
  const int64_t total = (int64_t)B * M;
  const int qwv = queries_per_wave(lg);
  const dim3 grid = dim3(blocks_for(total, qwv));
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, dim3(kKnnThreads), 0, st, N, M, Cf, G, K, lg, p, total, qwv,
                       coords, (const T*)feats, queries, table, (T*)out);
  };
  with_chunks<T>(chunks_per_lane(Cf, Chunk<T>::E, lg), [&](auto nrm) {
    constexpr int R = decltype(nrm)::value;
    if (K <= 4) go(knn_fwd_kernel<T, 4, R>);
    else if (K <= 8) go(knn_fwd_kernel<T, 8, R>);
    else go(knn_fwd_kernel<T, 16, R>);
  });
  return hipGetLastError();
}

template <typename T>
hipError_t bwd_t(int B, int N, int M, int Cf, int G, int K, float p, const float* coords,
                 const void* feats, const float* queries, const int32_t* table, const void* dout,
                 void* dfeat, float* dq, float* dp, const KnnWorkspace& w, hipStream_t st) {
  const int lg = row_group_log2<T>(Cf);
  const int64_t nq = (int64_t)B * M, ntok = (int64_t)B * N, nent = nq * K;
  auto grid1 = [](int64_t n) { return dim3((unsigned)((n + kKnnThreads - 1) / kKnnThreads)); };
  const int64_t MK = (int64_t)M * K;
  const int P = (int)((MK + kPart - 1) / kPart);
  const int64_t nparts = (int64_t)B * P;
  const int qwv = queries_per_wave(lg);
  // small images: counts per partition of kPart entries in LDS, stable
  // counting sort; large ones: per-token counts by integer atomics in the
  // query-major kernel, cursor placement and ranking
  const bool large = knn_large_lists(N, M, K);
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(blocks_for(nq, qwv)), dim3(kKnnThreads), 0, st, N, M, Cf, G, K,
                       lg, p, nq, qwv, coords, (const T*)feats, queries, table, (const T*)dout, dq,
                       w.dpart, w.slot, w.wgt, large ? w.cnt : nullptr);
  };
  // empty sizes launch nothing but what writes outputs (dF, dp)
  if (large && ntok > 0)
    launch_zero_i32(ntok, w.cnt, st);
  const int nrm = chunks_per_lane(Cf, Chunk<T>::E, lg);
  if (nq > 0) {
    with_chunks<T>(nrm, [&](auto nr) {
      constexpr int R = decltype(nr)::value;
      if (K <= 4) go(knn_bwd_query_kernel<T, 4, R>);
      else if (K <= 8) go(knn_bwd_query_kernel<T, 8, R>);
      else go(knn_bwd_query_kernel<T, 16, R>);
    });
  }
  const int64_t n_dp = nq > 0 ? (nq + qwv - 1) / qwv : 0;   // one dp share per wave of the query kernel
  if (ntok > 0) {
    if (!large) {
      // partition counts, and the walk order in B more workgroups
      hipLaunchKernelGGL(knn_pcount_kernel, dim3((unsigned)(nparts + B)), dim3(kChunkThreads), 0, st,
                         N, G, MK, P, nparts, (const int32_t*)w.slot, coords, w.pcnt, w.order);
      const int tgroups = (N + 63) / 64;
      hipLaunchKernelGGL(knn_pprefix_kernel, dim3((unsigned)(B * tgroups)), dim3(64 * kPrefWaves), 0,
                         st, N, P, tgroups, w.pcnt, w.cnt);
      launch_segment_scan(B, N, w.cnt, w.off, st);
      if (nparts > 0)
        hipLaunchKernelGGL(knn_pplace_kernel, dim3((unsigned)nparts), dim3(kChunkThreads),
                           (unsigned)(kChunkWaves * N * sizeof(int32_t)), st, N, K, MK, P,
                           (const int32_t*)w.slot, (const float*)w.wgt, (const int32_t*)w.off,
                           (const int32_t*)w.pcnt, w.ent);
    } else {
      launch_segment_scan(B, N, w.cnt, w.off, st);
      launch_zero_i32(ntok, w.cnt, st);
      if (nent > 0) {
        hipLaunchKernelGGL(knn_lplace_kernel, grid1(nent), dim3(kKnnThreads), 0, st, N, MK, nent,
                           (const int32_t*)w.slot, (const int32_t*)w.off, w.cnt, w.lst);
        // tokens of more than kLongSegment entries: a stable sort; the rest ranked
        launch_long_segment_sort(B, N, MK, MK - 1, (const int32_t*)w.off, w.lst, w.srt, nullptr,
                                 w.ent, K, (const float*)w.wgt, st);
        hipLaunchKernelGGL(knn_lrank_kernel, grid1(nent), dim3(kKnnThreads), 0, st, N, K, MK, nent,
                           (const int32_t*)w.slot, (const float*)w.wgt, (const int32_t*)w.off,
                           (const int32_t*)w.lst, w.ent);
      }
      // walk order: the tokens in bucket order
      const KnnBuckets bg = knn_buckets(N, G);
      const int64_t nbk = (int64_t)B * bg.nb;
      launch_zero_i32(nbk, w.bk.bcnt, st);
      hipLaunchKernelGGL(knn_bucket_count_kernel, grid1(ntok), dim3(kKnnThreads), 0, st, coords,
                         ntok, N, G, w.bk.bcnt, w.bk.brank);
      launch_segment_scan(B, bg.nb, w.bk.bcnt, w.bk.bstart, st);
      hipLaunchKernelGGL(knn_bucket_place_kernel, grid1(ntok), dim3(kKnnThreads), 0, st, coords,
                         ntok, N, G, (const int32_t*)w.bk.bstart, (const int32_t*)w.bk.brank,
                         (uint2*)nullptr, w.order);
    }
    // waves per token group: one when tokens have few entries, more when many
    const int64_t ept = N > 0 ? MK / N : 0;   // entries per token, on average
    const int split = ept < 16 ? 1 : (ept < 48 ? 2 : 4);
    const int groups = (N + (64 >> lg) - 1) / (64 >> lg);   // token groups per image
    const int wgs = (groups * split + kKnnThreads / 64 - 1) / (kKnnThreads / 64);
    // image streams: as many images in flight per XCD as keep their dO rows
    // within about 3 MiB of its L2
    const int64_t dimg = std::max<int64_t>(1, (int64_t)M * Cf * (int64_t)sizeof(T));
    const int per_xcd = (int)std::max<int64_t>(1, std::min<int64_t>((3 << 20) / dimg, (B + 7) / 8));
    const int S = std::min(B, 8 * per_xcd);
    with_chunks<T>(nrm, [&](auto nr) {
      hipLaunchKernelGGL((knn_dfeat_kernel<T, decltype(nr)::value>), dim3((unsigned)(S * wgs)),
                         dim3(kKnnThreads), 0, st, B, N, M, Cf, MK, lg, split, S, (const T*)dout,
                         (const int32_t*)w.off, (const int2*)w.ent, (const int32_t*)w.order,
                         (T*)dfeat, n_dp, (const float*)w.dpart, dp);
    });
  } else {
    hipLaunchKernelGGL(knn_dp_kernel, dim3(1), dim3(1024), 0, st, n_dp, (const float*)w.dpart, dp);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_knn_table(const float* coords, int B, int N, int G, int K, int32_t* table,
                            void* ws, hipStream_t st) {
  const int tiles_side = (G + 7) / 8;
  const int parts = (tiles_side * tiles_side + kTabTiles - 1) / kTabTiles;
  if (N <= kTabMaxTokens) {
    auto go = [&](auto kern) {
      hipLaunchKernelGGL(kern, dim3(B, parts), dim3(kTabThreads), 0, st, coords, N, G, K, table);
    };
    if (K <= 4) go(knn_table_kernel<4>);
    else if (K <= 8) go(knn_table_kernel<8>);
    else go(knn_table_kernel<16>);
    return hipGetLastError();
  }
  const KnnTableWorkspace w = knn_table_layout(ws, B, N);
  const KnnBuckets bg = knn_buckets(N, G);
  const int64_t ntok = (int64_t)B * N, nbk = (int64_t)B * bg.nb;
  auto grid1 = [](int64_t n) { return dim3((unsigned)((n + kKnnThreads - 1) / kKnnThreads)); };
  launch_zero_i32(nbk, w.bcnt, st);
  hipLaunchKernelGGL(knn_bucket_count_kernel, grid1(ntok), dim3(kKnnThreads), 0, st, coords, ntok,
                     N, G, w.bcnt, w.brank);
  launch_segment_scan(B, bg.nb, w.bcnt, w.bstart, st);
  hipLaunchKernelGGL(knn_bucket_place_kernel, grid1(ntok), dim3(kKnnThreads), 0, st, coords, ntok,
                     N, G, (const int32_t*)w.bstart, (const int32_t*)w.brank, w.tok,
                     (int32_t*)nullptr);
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(B, parts), dim3(kTabThreads), 0, st, N, G, K,
                       (const int32_t*)w.bstart, (const uint2*)w.tok, table);
  };
  if (K <= 4) go(knn_table_search_kernel<4>);
  else if (K <= 8) go(knn_table_search_kernel<8>);
  else go(knn_table_search_kernel<16>);
  return hipGetLastError();
}

hipError_t launch_knn_fwd(int dt, int B, int N, int M, int Cf, int G, int K, float p,
                          const float* coords, const void* feats, const float* queries,
                          const int32_t* table, void* out, hipStream_t st) {
  switch (dt) {
    case 0: return fwd_t<float>(B, N, M, Cf, G, K, p, coords, feats, queries, table, out, st);
    case 1: return fwd_t<bf16>(B, N, M, Cf, G, K, p, coords, feats, queries, table, out, st);
    default: return fwd_t<f16>(B, N, M, Cf, G, K, p, coords, feats, queries, table, out, st);
  }
}

hipError_t launch_knn_bwd(int dt, int B, int N, int M, int Cf, int G, int K, float p,
                          const float* coords, const void* feats, const float* queries,
                          const int32_t* table, const void* dout, void* dfeat, float* dq,
                          float* dp, void* ws, hipStream_t st) {
  const KnnWorkspace w = knn_layout(ws, B, N, M, K);
  switch (dt) {
    case 0:
      return bwd_t<float>(B, N, M, Cf, G, K, p, coords, feats, queries, table, dout, dfeat, dq,
                          dp, w, st);
    case 1:
      return bwd_t<bf16>(B, N, M, Cf, G, K, p, coords, feats, queries, table, dout,
                                   dfeat, dq, dp, w, st);
    default:
      return bwd_t<f16>(B, N, M, Cf, G, K, p, coords, feats, queries, table, dout, dfeat, dq,
                           dp, w, st);
  }
}

}  // namespace ca
