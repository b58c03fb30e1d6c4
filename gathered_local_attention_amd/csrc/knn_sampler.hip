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
//   knn_fwd_kernel        a group of lanes per query, 16 bytes of the
//                         feature row per lane: cell, slots, distances and
//                         weights (computed redundantly by the group's lanes),
//                         then the weighted sum of the K gathered rows.
//   knn_bwd_query_kernel  the same groups: weights again, <dO, F_k> reduced
//                         over the group, dq and the query's share of dp;
//                         slots and weights kept for the feature gradient
//                         and references counted per token.
//   knn_pprefix/scan/pplace  token-major entry lists (entry =
//                         query * K + slot) by a stable counting sort over
//                         partitions of the entries: each token's segment is
//                         in entry order, so the feature gradient is summed
//                         in a fixed order.
//   knn_dfeat_kernel      a lane group per token: dF = sum over its entries
//                         of w * dO (gathered rows), written once (0 for
//                         tokens no query reaches).
//   knn_dp_kernel         fixed-order reduction of the per-wave dp shares.
// Nothing in the backward uses floating-point atomics: the results are
// bitwise reproducible.
#include "common.h"

namespace ca {

namespace {

constexpr int kKnnMaxK = 16;
constexpr int kTabThreads = 256;
constexpr int kTabMaxBuckets = 64 * 64;   // grid sides up to 64
constexpr int kTabMaxTokens = 4096;
constexpr int kKnnThreads = 256;          // 4 waves
constexpr int kPart = kKnnPart;           // entries per partition of the stable counting sort

__device__ __forceinline__ int ceil_log2(int v) {
  int b = 0;
  while ((1 << b) < v) ++b;
  return b;
}

// ---------------------------------------------------------------------------
// Table build.  grid = (B, parts): part y of an image takes kTabTiles tiles
// of 8 x 8 cells (one wave each) and repeats the image's bucketing (cheap:
// at most 4096 tokens).  Buckets are squares of 2^bs fixed-point units,
// bs chosen so that an image holds about two tokens per bucket (at least a
// cell, at most the whole range).
// ---------------------------------------------------------------------------
constexpr int kTabTiles = kTabThreads / 64;

template <int KM>
__global__ void __launch_bounds__(kTabThreads)
knn_table_kernel(const float* __restrict__ coords, int N, int G, int K, int32_t* __restrict__ table) {
  __shared__ int start[kTabMaxBuckets];
  __shared__ uint2 tok[kTabMaxTokens];     // (qx | qy << 16, token)
  __shared__ int tmp[17];
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int shift = 16 - ceil_log2(G);     // fixed-point units per cell: s = 2^shift
  const double step = (double)(1 << shift);
  int pb = 0;                              // bucket grid side 2^pb: about N / 2 buckets
  while (pb < 16 - shift && (1 << (2 * pb + 2)) <= max(N, 1) / 2) ++pb;
  const int bs = 16 - pb;                  // bucket side 2^bs units (>= one cell)
  const int Pb = 1 << pb;
  const int nb = Pb * Pb;
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

  // One wave per tile (lane = cell).  The wave scans a window of buckets
  // around its tile that grows one ring at a time, every lane testing every
  // token of the window (uniform loops: no divergence but the insertions).
  // It stops once every lane's K-th best is strictly closer than any token
  // outside the window can be: a token beyond the window's top edge at
  // fixed-point row R0 * 2^bs has Y <= R0 * 2^bs - 1, so |Y - cy| >=
  // cy - R0 * 2^bs + 1; likewise on the other three sides.
  const int lane = tid & 63;
  const int tiles_side = (G + 7) >> 3;
  const int tile = blockIdx.y * kTabTiles + (tid >> 6);
  if (tile >= tiles_side * tiles_side) return;
  const int i0 = (tile / tiles_side) * 8, j0 = (tile % tiles_side) * 8;
  const int i = i0 + (lane >> 3), j = j0 + (lane & 7);
  const bool valid = i < G && j < G;
  const int64_t cx = (int64_t)(2 * j + 1) << (shift - 1);   // (j + 1/2) s
  const int64_t cy = (int64_t)(2 * i + 1) << (shift - 1);
  // the tile's own buckets (cells up to min(G, i0 + 8) - 1)
  const int ilast = min(G, i0 + 8) - 1, jlast = min(G, j0 + 8) - 1;
  const int tr0 = (i0 << shift) >> bs, tr1 = (((ilast + 1) << shift) - 1) >> bs;
  const int tc0 = (j0 << shift) >> bs, tc1 = (((jlast + 1) << shift) - 1) >> bs;
  // keys (d2 << 12 | token): d2 < 2^33, tokens < 2^12
  uint64_t best[KM];
#pragma unroll
  for (int r = 0; r < KM; ++r) best[r] = ~0ull;
  uint64_t worst = ~0ull;   // best[K - 1]
  // tokens of the buckets (by, bx0 .. bx1): one contiguous range (row-major
  // bucket order)
  auto scan_row = [&](int by, int bx0, int bx1) {
    const int bb0 = by * Pb + bx0, bb1 = by * Pb + bx1;
    const int t0 = start[bb0], t1 = bb1 + 1 < nb ? start[bb1 + 1] : total;
    for (int t = t0; t < t1; ++t) {
      const uint2 e = tok[t];
      const int64_t dx = (int64_t)(e.x & 0xFFFFu) - cx, dy = (int64_t)(e.x >> 16) - cy;
      uint64_t x = ((uint64_t)(dx * dx + dy * dy) << 12) | e.y;
      if (x >= worst) continue;
#pragma unroll
      for (int r = 0; r < KM; ++r) {
        if (r < K) {
          const uint64_t lo = x < best[r] ? x : best[r];
          const uint64_t hi = x < best[r] ? best[r] : x;
          best[r] = lo;
          x = hi;
        }
        if (r == K - 1) worst = best[r];
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
    const bool done = !valid || (worst != ~0ull && (int64_t)(worst >> 12) < lb * lb);
    if (__all(done)) break;
  }
  if (!valid) return;
  int32_t* row = table + (((int64_t)b * G + i) * G + j) * K;
#pragma unroll
  for (int r = 0; r < KM; ++r)
    if (r < K) row[r] = best[r] == ~0ull ? -1 : (int32_t)(best[r] & 0xFFFu);
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
  static constexpr int NR = 4;   // chunks per lane at most (1024 channels)
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
};
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
// eight bf16 / fp16 values: widening is exact, narrowing rounds to nearest even
template <typename H, typename V>
struct HalfChunk {
  static constexpr int E = 8;
  static constexpr int NR = 2;   // chunks per lane at most (1024 channels)
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
};
template <>
struct Chunk<bf16> : HalfChunk<bf16, bf16x8> {};
template <>
struct Chunk<f16> : HalfChunk<f16, f16x8> {};

constexpr int kMaxChunksPerLane = 4;   // rows up to 256 chunks of 16 bytes (1024 f32 channels)

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

template <typename T, int KM>
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
    // every chunk's rows in flight before the sums: the loads are
    // unconditional (an empty slot or a chunk past the row reads a valid
    // place, the data is then masked), so that no branch splits them
    uint4 raw[Ck::NR][KM];
    if (N > 0) {
#pragma unroll
      for (int r = 0; r < Ck::NR; ++r)
#pragma unroll
        for (int k = 0; k < KM; ++k)
          raw[r][k] = Ck::raw(fimg + (int64_t)max(sl[k], 0) * Cf + (cs + (r < nr ? r * L : 0)) * Ck::E);
    }
#pragma unroll
    for (int r = 0; r < Ck::NR; ++r) {
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
template <typename T, int KM>
__global__ void __launch_bounds__(kKnnThreads) __attribute__((amdgpu_waves_per_eu(sizeof(T) == 2 && KM <= 8 ? 4 : 1)))
knn_bwd_query_kernel(int N, int M, int Cf, int G, int K, int lg, float p, int64_t total, int qwv,
                     const float* __restrict__ coords, const T* __restrict__ feats,
                     const float* __restrict__ queries, const int32_t* __restrict__ table,
                     const T* __restrict__ dout, float* __restrict__ dq, float* __restrict__ dpart,
                     int32_t* __restrict__ ent_slot, float* __restrict__ ent_w, int P,
                     int32_t* __restrict__ pcnt) {
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
    // unconditional loads (see the forward), masked afterwards
    uint4 raw[Ck::NR][KM], oraw[Ck::NR];
    const int64_t oid = live ? id : base;
#pragma unroll
    for (int r = 0; r < Ck::NR; ++r) {
      const int c = cs + (r < nr ? r * L : 0);
      oraw[r] = Ck::raw(dout + oid * Cf + c * Ck::E);
      if (N > 0) {
#pragma unroll
        for (int k = 0; k < KM; ++k) raw[r][k] = Ck::raw(fimg + (int64_t)max(sl[k], 0) * Cf + c * Ck::E);
      }
    }
#pragma unroll
    for (int r = 0; r < Ck::NR; ++r) {
      if (r >= nr || !live) break;
      float o[Ck::E];
      Ck::cvt(oraw[r], o);
#pragma unroll
      for (int k = 0; k < KM; ++k) {
        if (sl[k] < 0) raw[r][k] = make_uint4(0u, 0u, 0u, 0u);
        float v[Ck::E];
        Ck::cvt(raw[r][k], v);
#pragma unroll
        for (int e = 0; e < Ck::E; ++e) gk[k] = fmaf(o[e], v[e], gk[k]);
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
  // the entries' counts per partition of kPart entries and token (integer
  // atomics, order independent), last: nothing in this wave waits on them;
  // without pcnt they are counted by knn_pcount_kernel instead
  if (mine && pcnt) {
    const int64_t b = id / M;
    const int64_t e0 = (id - b * M) * K;   // first entry of this query in its image
#pragma unroll
    for (int k = 0; k < KM; ++k)
      if (k < K && qw.slot[k] >= 0) atomicAdd(&pcnt[(b * P + (e0 + k) / kPart) * N + qw.slot[k]], 1);
  }
}

// Per partition of kPart entries, the count of its entries per token,
// accumulated in LDS (images of at most kTabMaxTokens tokens) and written
// out whole (zeros included): one workgroup per partition.
__global__ void __launch_bounds__(kKnnThreads)
knn_pcount_kernel(int N, int64_t MK, int P, const int32_t* __restrict__ ent_slot,
                  int32_t* __restrict__ pcnt) {
  static_assert(kPart == kKnnThreads, "one entry per thread");
  __shared__ int32_t c[kTabMaxTokens];
  const int64_t part = blockIdx.x;
  const int64_t b = part / P;
  const int s = (int)(part - b * P);
  const int64_t e0 = (int64_t)s * kPart;
  const int n = (int)min((int64_t)kPart, MK - e0);
  for (int t = threadIdx.x; t < N; t += kKnnThreads) c[t] = 0;
  __syncthreads();
  if ((int)threadIdx.x < n) {
    const int t = ent_slot[b * MK + e0 + threadIdx.x];
    if (t >= 0) atomicAdd(&c[t], 1);
  }
  __syncthreads();
  int32_t* row = pcnt + (b * P + s) * N;
  for (int t = threadIdx.x; t < N; t += kKnnThreads) row[t] = c[t];
}

__global__ void __launch_bounds__(kKnnThreads)
knn_zero_kernel(int64_t n, int32_t* __restrict__ x) {
  const int64_t i = (int64_t)blockIdx.x * kKnnThreads + threadIdx.x;
  if (i < n) x[i] = 0;
}

// per image: segment offsets of the token-major lists (counts staged through
// LDS in chunks, one workgroup scan per chunk)
constexpr int kScanThreads = 1024;
constexpr int kScanChunk = 8192;
__global__ void __launch_bounds__(kScanThreads)
knn_scan_kernel(int N, const int32_t* __restrict__ cnt_all, int32_t* __restrict__ off_all) {
  __shared__ int32_t v[kScanChunk];
  __shared__ int tmp[17];
  const int64_t b = blockIdx.x;
  const int32_t* cnt = cnt_all + b * N;
  int32_t* off = off_all + b * (N + 1);
  constexpr int kPer = kScanChunk / kScanThreads;
  int carry = 0;
  for (int c0 = 0; c0 < N; c0 += kScanChunk) {
    const int n = min(kScanChunk, N - c0);
    for (int x = threadIdx.x; x < n; x += kScanThreads) v[x] = cnt[c0 + x];
    __syncthreads();
    const int r0 = threadIdx.x * kPer;
    int run = 0;
#pragma unroll
    for (int r = 0; r < kPer; ++r) run += r0 + r < n ? v[r0 + r] : 0;
    int tot;
    int acc = carry + block_exclusive_scan(run, tmp, kScanThreads, &tot);
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
      if (r0 + r < n) {
        const int c = v[r0 + r];
        v[r0 + r] = acc;
        acc += c;
      }
    }
    __syncthreads();
    for (int x = threadIdx.x; x < n; x += kScanThreads) off[c0 + x] = v[x];
    carry += tot;
    __syncthreads();
  }
  if (threadIdx.x == 0) off[N] = carry;
}

// Token-major entry lists, in entry order (entry = query * K + slot), by a
// stable counting sort.  The entries of an image are cut into partitions of
// kPart consecutive entries: (1) per partition and token, the count of its
// entries (integer atomics in the query-major kernel: the counts do not
// depend on their order), or per partition in LDS (knn_pcount_kernel) when
// the image fits; (2) per token, the counts turned into exclusive
// prefixes over the partitions, and the token's total; (3) the totals
// scanned into segment starts (knn_scan_kernel); (4) per partition, every
// entry placed at segment start + the partition's prefix + the number of
// earlier entries of the same token in the partition.

__global__ void __launch_bounds__(kKnnThreads)
knn_pprefix_kernel(int N, int P, int64_t n_tok, int32_t* __restrict__ pcnt, int32_t* __restrict__ cnt) {
  const int64_t x = (int64_t)blockIdx.x * kKnnThreads + threadIdx.x;
  if (x >= n_tok) return;
  const int64_t b = x / N;
  const int t = (int)(x - b * N);
  int acc = 0;
  for (int s0 = 0; s0 < P; s0 += 16) {   // sixteen loads in flight
    int v[16];
#pragma unroll
    for (int h = 0; h < 16; ++h) v[h] = s0 + h < P ? pcnt[(b * P + s0 + h) * N + t] : 0;
#pragma unroll
    for (int h = 0; h < 16; ++h) {
      if (s0 + h < P) pcnt[(b * P + s0 + h) * N + t] = acc;
      acc += v[h];
    }
  }
  cnt[x] = acc;
}

// one workgroup per partition; wave w ranks the partition's entries
// w*64 .. w*64+63 (one per lane) against the earlier entries of the partition
__global__ void __launch_bounds__(kKnnThreads)
knn_pplace_kernel(int N, int64_t MK, int P, const int32_t* __restrict__ ent_slot,
                  const int32_t* __restrict__ off_all, const int32_t* __restrict__ pcnt,
                  int32_t* __restrict__ ent_all) {
  static_assert(kPart == kKnnThreads, "one entry per thread");
  __shared__ __align__(16) int32_t tok[kPart];
  const int64_t part = blockIdx.x;
  const int64_t b = part / P;
  const int s = (int)(part - b * P);
  const int64_t e0 = (int64_t)s * kPart;
  const int n = (int)min((int64_t)kPart, MK - e0);
  const int u = threadIdx.x;
  const int t = u < n ? ent_slot[b * MK + e0 + u] : -1;
  tok[u] = t;
  __syncthreads();
  const int ymax = (threadIdx.x & ~63) + 64;   // the wave's entries are below this
  int rank = 0;
  const int4* t4 = reinterpret_cast<const int4*>(tok);
  for (int y4 = 0; y4 < ymax / 4; ++y4) {
    const int4 v = t4[y4];
    const int y = 4 * y4;
    rank += (v.x == t && y < u) + (v.y == t && y + 1 < u) + (v.z == t && y + 2 < u) +
            (v.w == t && y + 3 < u);
  }
  if (t >= 0)
    ent_all[b * MK + off_all[b * (N + 1) + t] + pcnt[(b * P + s) * N + t] + rank] = (int32_t)(e0 + u);
}

// Spatial walk order of the tokens for the feature gradient: the tokens of
// an image bucketed on a coarse grid (about two per bucket) in LDS, so that
// the waves resident at one time work on neighbouring tokens, which share
// most of their queries (and so the dO rows they gather stay in L2).  Any
// order gives the same result: each token's sum has its own fixed order.
// grid = B, for images of at most kTabMaxTokens tokens.
__global__ void __launch_bounds__(kTabThreads)
knn_order_kernel(const float* __restrict__ coords, int N, int G, int32_t* __restrict__ order) {
  __shared__ int start[kTabMaxBuckets];
  const int b = blockIdx.x, tid = threadIdx.x;
  const int shift = 16 - ceil_log2(G);
  const double step = (double)(1 << shift);
  int pb = 0;
  while (pb < 16 - shift && (1 << (2 * pb + 2)) <= max(N, 1) / 2) ++pb;
  const int bs = 16 - pb, Pb = 1 << pb, nb = Pb * Pb;
  const float2* xy = reinterpret_cast<const float2*>(coords) + (int64_t)b * N;
  for (int x = tid; x < nb; x += kTabThreads) start[x] = 0;
  __syncthreads();
  constexpr int kPer = kTabMaxTokens / kTabThreads;
  int bk[kPer], rk[kPer];
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    const int e = tid + r * kTabThreads;
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
  __shared__ int tmp[17];
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
  int32_t* ord = order + (int64_t)b * N;
#pragma unroll
  for (int r = 0; r < kPer; ++r)
    if (bk[r] >= 0) ord[start[bk[r]] + rk[r]] = tid + r * kTabThreads;
}

// ---------------------------------------------------------------------------
// Backward, token-major part: dF[b, t] = sum over its entries of w dO[b, m].
// ---------------------------------------------------------------------------
// Workgroup = one group of 64 / L tokens (L lanes per token, 16 bytes of the
// row per lane) and its four waves split each token's entries: wave w takes
// the batches w, w + 4, ... of kB entries, and the four partial sums are
// added in wave order through LDS, so every token's sum has one fixed order.
// Workgroups are dealt XCD-aware: workgroup 8 i + x (dispatched to XCD x)
// takes token group i of the images x, x + 8, x + 16, ... one after the
// other, so that the workgroups of one XCD work on one image at a time and
// its dO rows stay in that XCD's L2 (with fewer than 8 images, X = B
// streams).
template <typename T>
__global__ void __launch_bounds__(kKnnThreads)
knn_dfeat_kernel(int B, int N, int M, int Cf, int K, int lg, int split, const T* __restrict__ dout,
                 const int32_t* __restrict__ off_all, const int32_t* __restrict__ ent_all,
                 const float* __restrict__ ent_w, const int32_t* __restrict__ order,
                 T* __restrict__ dfeat) {
  using Ck = Chunk<T>;
  constexpr int kB = 8;                          // entries (rows) per batch
  constexpr int kW = kKnnThreads / 64;           // waves per workgroup
  __shared__ float part[kW][Ck::NR * Ck::E][64];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int X = min(B, 8);                      // image streams (one per XCD when B >= 8)
  const int x = (int)(blockIdx.x % X), gi = (int)(blockIdx.x / X);
  const int L = 1 << lg, sub = lane & (L - 1);
  // `split` waves share a token group; the workgroup covers kW / split groups
  const int grp = gi * (kW / split) + wv / split, sw = wv % split;
  const int pos = grp * (64 >> lg) + (lane >> lg);   // token position in the walk order
  const int nch = Cf / Ck::E;
  const int nr = (nch - sub + L - 1) / L;            // chunks of this lane
  const int cs = min(sub, nch - 1);   // idle lanes (sub >= nch, nr = 0) load inside the row
  const int64_t per = (int64_t)M * K;
  for (int img = x; img < B; img += X) {
    const int64_t b = img;
    const bool live = pos < N;
    const int t = live ? (order ? order[b * N + pos] : pos) : 0;
    const int a = live ? off_all[b * (N + 1) + t] : 0;
    const int z = live ? off_all[b * (N + 1) + t + 1] : 0;
    const int32_t* ent = ent_all + b * per;
    const float* wimg = ent_w + b * per;
    const T* oimg = dout + b * M * Cf;
    float acc[Ck::NR][Ck::E];
#pragma unroll
    for (int r = 0; r < Ck::NR; ++r)
#pragma unroll
      for (int e = 0; e < Ck::E; ++e) acc[r][e] = 0.f;
    for (int u = a + sw * kB; u < z; u += split * kB) {
      int e[kB];
      float wt[kB];
      // unconditional loads (a batch past the segment end re-reads entry u),
      // masked afterwards
#pragma unroll
      for (int h = 0; h < kB; ++h) e[h] = ent[u + h < z ? u + h : u];
#pragma unroll
      for (int h = 0; h < kB; ++h) wt[h] = wimg[e[h]];
      uint4 raw[Ck::NR][kB];
#pragma unroll
      for (int r = 0; r < Ck::NR; ++r)
#pragma unroll
        for (int h = 0; h < kB; ++h)
          raw[r][h] = Ck::raw(oimg + (int64_t)(e[h] / K) * Cf + (cs + (r < nr ? r * L : 0)) * Ck::E);
#pragma unroll
      for (int r = 0; r < Ck::NR; ++r) {
        if (r >= nr) break;
#pragma unroll
        for (int h = 0; h < kB; ++h) {
          if (u + h >= z) raw[r][h] = make_uint4(0u, 0u, 0u, 0u);
          float v[Ck::E];
          Ck::cvt(raw[r][h], v);
#pragma unroll
          for (int q = 0; q < Ck::E; ++q) acc[r][q] = fmaf(wt[h], v[q], acc[r][q]);
        }
      }
    }
    // partial sums of the group's other waves to its first, added in wave order
    if (split > 1) {
      if (sw > 0) {
#pragma unroll
        for (int r = 0; r < Ck::NR; ++r)
#pragma unroll
          for (int q = 0; q < Ck::E; ++q) part[wv][r * Ck::E + q][lane] = acc[r][q];
      }
      __syncthreads();
      if (sw == 0) {
        for (int v2 = 1; v2 < split; ++v2)
#pragma unroll
          for (int r = 0; r < Ck::NR; ++r)
#pragma unroll
            for (int q = 0; q < Ck::E; ++q) acc[r][q] += part[wv + v2][r * Ck::E + q][lane];
      }
      __syncthreads();   // part is reused by the next image
    }
    if (sw == 0 && live) {
#pragma unroll
      for (int r = 0; r < Ck::NR; ++r) {
        if (r >= nr) break;
        Ck::store(dfeat + (b * N + t) * Cf + (cs + r * L) * Ck::E, acc[r]);
      }
    }
  }
}

// dp = sum of the per-query shares, in a fixed order (one workgroup)
__global__ void __launch_bounds__(1024)
knn_dp_kernel(int64_t n, const float* __restrict__ dpart, float* __restrict__ dp) {
  __shared__ float red[1024];
  float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};   // eight loads in flight
  int64_t i = threadIdx.x;
  for (; i + 7 * 1024 < n; i += 8 * 1024)
#pragma unroll
    for (int u = 0; u < 8; ++u) a[u] += dpart[i + u * 1024];
  for (; i < n; i += 1024) a[0] += dpart[i];
  red[threadIdx.x] = ((a[0] + a[1]) + (a[2] + a[3])) + ((a[4] + a[5]) + (a[6] + a[7]));
  __syncthreads();
  for (int o = 512; o >= 1; o >>= 1) {
    if ((int)threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) dp[0] = red[0];
}

int group_log2(int Cf, int E) {
  const int nch = Cf / E;
  int lg = 0;
  while ((1 << lg) < nch && lg < 6) ++lg;
  return lg;
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
  const int lg = group_log2(Cf, Chunk<T>::E);
  const int64_t total = (int64_t)B * M;
  const int qwv = queries_per_wave(lg);
  const dim3 grid = dim3(blocks_for(total, qwv));
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, dim3(kKnnThreads), 0, st, N, M, Cf, G, K, lg, p, total, qwv,
                       coords, (const T*)feats, queries, table, (T*)out);
  };
  if (K <= 4) go(knn_fwd_kernel<T, 4>);
  else if (K <= 8) go(knn_fwd_kernel<T, 8>);
  else go(knn_fwd_kernel<T, 16>);
  return hipGetLastError();
}

template <typename T>
hipError_t bwd_t(int B, int N, int M, int Cf, int G, int K, float p, const float* coords,
                 const void* feats, const float* queries, const int32_t* table, const void* dout,
                 void* dfeat, float* dq, float* dp, const KnnWorkspace& w, hipStream_t st) {
  const int lg = group_log2(Cf, Chunk<T>::E);
  const int64_t nq = (int64_t)B * M, ntok = (int64_t)B * N, nent = nq * K;
  auto grid1 = [](int64_t n) { return dim3((unsigned)((n + kKnnThreads - 1) / kKnnThreads)); };
  const int64_t MK = (int64_t)M * K;
  const int P = (int)((MK + kPart - 1) / kPart);
  const int64_t npc = (int64_t)B * P * N, nparts = (int64_t)B * P;
  const int qwv = queries_per_wave(lg);
  // partition counts: in LDS per partition for images that fit, else by
  // integer atomics in the query-major kernel into zeroed counters
  const bool lds_count = N <= kTabMaxTokens;
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(blocks_for(nq, qwv)), dim3(kKnnThreads), 0, st, N, M, Cf, G, K,
                       lg, p, nq, qwv, coords, (const T*)feats, queries, table, (const T*)dout, dq,
                       w.dpart, w.slot, w.wgt, P, lds_count ? nullptr : w.pcnt);
  };
  // empty sizes launch nothing but what writes outputs (dF, dp)
  if (npc > 0 && !lds_count)
    hipLaunchKernelGGL(knn_zero_kernel, grid1(npc), dim3(kKnnThreads), 0, st, npc, w.pcnt);
  if (nq > 0) {
    if (K <= 4) go(knn_bwd_query_kernel<T, 4>);
    else if (K <= 8) go(knn_bwd_query_kernel<T, 8>);
    else go(knn_bwd_query_kernel<T, 16>);
  }
  if (npc > 0 && lds_count)
    hipLaunchKernelGGL(knn_pcount_kernel, dim3((unsigned)nparts), dim3(kKnnThreads), 0, st, N, MK,
                       P, (const int32_t*)w.slot, w.pcnt);
  if (ntok > 0) {
    hipLaunchKernelGGL(knn_pprefix_kernel, grid1(ntok), dim3(kKnnThreads), 0, st, N, P, ntok,
                       w.pcnt, w.cnt);
    hipLaunchKernelGGL(knn_scan_kernel, dim3(B), dim3(kScanThreads), 0, st, N,
                       (const int32_t*)w.cnt, w.off);
    if (nparts > 0)
      hipLaunchKernelGGL(knn_pplace_kernel, dim3((unsigned)nparts), dim3(kKnnThreads), 0, st, N, MK,
                         P, (const int32_t*)w.slot, (const int32_t*)w.off, (const int32_t*)w.pcnt,
                         w.ent);
    const bool ordered = N <= kTabMaxTokens && G <= 65536;
    if (ordered)
      hipLaunchKernelGGL(knn_order_kernel, dim3(B), dim3(kTabThreads), 0, st, coords, N, G, w.order);
    // waves per token group: one when tokens have few entries, more when many
    const int64_t ept = N > 0 ? MK / N : 0;   // entries per token, on average
    const int split = ept < 16 ? 1 : (ept < 48 ? 2 : 4);
    const int groups = (N + (64 >> lg) - 1) / (64 >> lg);   // token groups per image
    const int wgs = (groups * split + kKnnThreads / 64 - 1) / (kKnnThreads / 64);
    hipLaunchKernelGGL(knn_dfeat_kernel<T>, dim3((unsigned)(std::min(B, 8) * wgs)), dim3(kKnnThreads), 0, st,
                       B, N, M, Cf, K, lg, split, (const T*)dout, (const int32_t*)w.off,
                       (const int32_t*)w.ent, (const float*)w.wgt,
                       ordered ? (const int32_t*)w.order : nullptr, (T*)dfeat);
  }
  const int64_t nwaves = (nq + qwv - 1) / qwv;   // one dp share per wave of the query kernel
  hipLaunchKernelGGL(knn_dp_kernel, dim3(1), dim3(1024), 0, st, nq > 0 ? nwaves : 0,
                     (const float*)w.dpart, dp);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_knn_table(const float* coords, int B, int N, int G, int K, int32_t* table,
                            hipStream_t st) {
  const int tiles_side = (G + 7) / 8;
  const int parts = (tiles_side * tiles_side + kTabTiles - 1) / kTabTiles;
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(B, parts), dim3(kTabThreads), 0, st, coords, N, G, K, table);
  };
  if (K <= 4) go(knn_table_kernel<4>);
  else if (K <= 8) go(knn_table_kernel<8>);
  else go(knn_table_kernel<16>);
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
