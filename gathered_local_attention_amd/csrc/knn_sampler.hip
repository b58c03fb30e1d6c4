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
//                         image's tokens counting-sorted into the buckets of
//                         the fixed-point grid (bucket side = one cell) in
//                         LDS; one thread per cell searches rings of buckets
//                         around its own and stops once its K-th best is
//                         closer than any bucket of the next ring can be.
//   knn_fwd_kernel        a group of lanes per query, 16 bytes of the
//                         feature row per lane: cell, slots, distances and
//                         weights (computed redundantly by the group's lanes),
//                         then the weighted sum of the K gathered rows.
//   knn_bwd_query_kernel  the same groups: weights again, <dO, F_k> reduced
//                         over the group, dq and the query's share of dp;
//                         slots and weights kept for the feature gradient
//                         and references counted per token.
//   knn_scan/place/sort   token-major entry lists (entry = query * K + slot),
//                         each token's segment ordered by entry, so that the
//                         feature gradient is summed in a fixed order.
//   knn_dfeat_kernel      a lane group per token: dF = sum over its entries
//                         of w * dO (gathered rows), written once (0 for
//                         tokens no query reaches).
//   knn_dp_kernel         fixed-order reduction of the per-query dp shares.
// Nothing in the backward uses floating-point atomics: the results are
// bitwise reproducible.
#include "common.h"

namespace ca {

namespace {

constexpr int kKnnMaxK = 16;
constexpr int kTabThreads = 1024;
constexpr int kTabMaxBuckets = 64 * 64;   // grid sides up to 64
constexpr int kTabMaxTokens = 4096;
constexpr int kKnnThreads = 256;          // 4 waves

__device__ __forceinline__ int ceil_log2(int v) {
  int b = 0;
  while ((1 << b) < v) ++b;
  return b;
}

// ---------------------------------------------------------------------------
// Table build.  grid = (B, parts); the parts of an image split its cells and
// each repeats the bucketing (cheap: at most 4096 tokens).
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kTabThreads)
knn_table_kernel(const float* __restrict__ coords, int N, int G, int K, int32_t* __restrict__ table) {
  __shared__ int start[kTabMaxBuckets];
  __shared__ uint2 tok[kTabMaxTokens];     // (qx | qy << 16, token)
  __shared__ int tmp[17];
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int bits = ceil_log2(G);
  const int shift = 16 - bits;             // fixed-point units per cell: s = 2^shift
  const int P = 1 << bits;                 // bucket grid side (>= G)
  const int nb = P * P;
  const double step = (double)(1 << shift);
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
      bk[r] = (int)((qy >> shift) * (uint32_t)P + (qx >> shift));
      rk[r] = atomicAdd(&start[bk[r]], 1);
    }
  }
  __syncthreads();
  // exclusive scan of the counts (up to 4 buckets per thread)
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

  const int cells = G * G;
  const int per = (cells + gridDim.y - 1) / gridDim.y;
  const int cbeg = blockIdx.y * per, cend = min(cells, cbeg + per);
  for (int cell = cbeg + tid; cell < cend; cell += kTabThreads) {
    const int i = cell / G, j = cell - (cell / G) * G;
    const int64_t cx = (int64_t)(2 * j + 1) << (shift - 1);   // (j + 1/2) s
    const int64_t cy = (int64_t)(2 * i + 1) << (shift - 1);
    // keys (d2 << 12 | token): d2 < 2^33, tokens < 2^12
    uint64_t best[kKnnMaxK];
#pragma unroll
    for (int r = 0; r < kKnnMaxK; ++r) best[r] = ~0ull;
    uint64_t worst = ~0ull;   // best[K - 1], kept apart (K is a runtime value)
    for (int R = 0; R < P; ++R) {
      const int y0 = i - R, y1 = i + R;
      for (int by = max(y0, 0); by <= min(y1, P - 1); ++by) {
        const bool edge = by == y0 || by == y1;
        const int dxs = (edge || R == 0) ? 1 : 2 * R;   // inner rows: the two end buckets
        for (int bx = j - R; bx <= j + R; bx += dxs) {
          if (bx < 0 || bx >= P) continue;
          const int bb = by * P + bx;
          const int t0 = start[bb], t1 = bb + 1 < nb ? start[bb + 1] : total;
          for (int t = t0; t < t1; ++t) {
            const uint2 e = tok[t];
            const int64_t dx = (int64_t)(e.x & 0xFFFFu) - cx, dy = (int64_t)(e.x >> 16) - cy;
            uint64_t x = ((uint64_t)(dx * dx + dy * dy) << 12) | e.y;
            if (x >= worst) continue;
#pragma unroll
            for (int r = 0; r < kKnnMaxK; ++r) {
              if (r < K) {
                const uint64_t lo = x < best[r] ? x : best[r];
                const uint64_t hi = x < best[r] ? best[r] : x;
                best[r] = lo;
                x = hi;
              }
              if (r == K - 1) worst = best[r];
            }
          }
        }
      }
      // every bucket of ring R + 1 lies at least (R + 1/2) s from the centre
      // along one axis: stop once the K-th best is strictly closer
      const int64_t lb = (int64_t)(2 * R + 1) << (shift - 1);
      if (worst != ~0ull && (int64_t)(worst >> 12) < lb * lb) break;
    }
    int32_t* row = table + ((int64_t)b * cells + cell) * K;
#pragma unroll
    for (int r = 0; r < kKnnMaxK; ++r)
      if (r < K) row[r] = best[r] == ~0ull ? -1 : (int32_t)(best[r] & 0xFFFu);
  }
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
  float mx = -INFINITY;
#pragma unroll
  for (int k = 0; k < KM; ++k) {
    qw.slot[k] = -1;
    qw.d[k] = 0.f;
    qw.diff[k] = make_float2(0.f, 0.f);
    if (k < K) {
      const int s = row[k];
      if (s >= 0 && s < N) {
        const float2 x = xy[s];
        const float dx = q.x - x.x, dy = q.y - x.y;
        qw.slot[k] = s;
        qw.diff[k] = make_float2(dx, dy);
        qw.d[k] = sqrtf(fmaf(dx, dx, dy * dy));
        mx = fmaxf(mx, -p * qw.d[k]);
      }
    }
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
// Forward.  out[b, m] = sum_k w_k F[b, slot_k].
// ---------------------------------------------------------------------------
template <typename T, int KM>
__global__ void __launch_bounds__(kKnnThreads)
knn_fwd_kernel(int N, int M, int Cf, int G, int K, int lg, float p, int64_t total,
               const float* __restrict__ coords, const T* __restrict__ feats,
               const float* __restrict__ queries, const int32_t* __restrict__ table,
               T* __restrict__ out) {
  using Ck = Chunk<T>;
  const Group g = group_of(lg, total);
  if (!g.valid) return;
  const int L = 1 << lg;
  const int64_t b = g.id / M;
  const float2 q = reinterpret_cast<const float2*>(queries)[g.id];
  const float2* xy = reinterpret_cast<const float2*>(coords) + b * N;
  QueryWeights<KM> qw;
  query_weights(q, (int)b, G, K, N, p, xy, table, qw);
  const int nch = Cf / Ck::E;
  const T* fimg = feats + b * N * Cf;
#pragma unroll
  for (int r = 0; r < kMaxChunksPerLane; ++r) {
    const int c = g.sub + r * L;
    if (c >= nch) break;
    float acc[Ck::E];
#pragma unroll
    for (int e = 0; e < Ck::E; ++e) acc[e] = 0.f;
    // all K rows in flight before the sums
    float v[KM][Ck::E];
#pragma unroll
    for (int k = 0; k < KM; ++k)
      if (qw.slot[k] >= 0) Ck::load(fimg + (int64_t)qw.slot[k] * Cf + c * Ck::E, v[k]);
#pragma unroll
    for (int k = 0; k < KM; ++k)
      if (qw.slot[k] >= 0)
#pragma unroll
        for (int e = 0; e < Ck::E; ++e) acc[e] = fmaf(qw.w[k], v[k][e], acc[e]);
    Ck::store(out + g.id * Cf + c * Ck::E, acc);
  }
}

// ---------------------------------------------------------------------------
// Backward, query-major part.
// ---------------------------------------------------------------------------
template <typename T, int KM>
__global__ void __launch_bounds__(kKnnThreads)
knn_bwd_query_kernel(int N, int M, int Cf, int G, int K, int lg, float p, int64_t total,
                     const float* __restrict__ coords, const T* __restrict__ feats,
                     const float* __restrict__ queries, const int32_t* __restrict__ table,
                     const T* __restrict__ dout, float* __restrict__ dq, float* __restrict__ dpart,
                     int32_t* __restrict__ ent_slot, float* __restrict__ ent_w,
                     int32_t* __restrict__ cnt) {
  using Ck = Chunk<T>;
  const Group g = group_of(lg, total);
  const int L = 1 << lg;
  const int64_t id = g.valid ? g.id : 0;   // idle lanes mirror query 0 (shuffles need them)
  const int64_t b = id / M;
  const float2 q = reinterpret_cast<const float2*>(queries)[id];
  const float2* xy = reinterpret_cast<const float2*>(coords) + b * N;
  QueryWeights<KM> qw;
  query_weights(q, (int)b, G, K, N, p, xy, table, qw);
  const int nch = Cf / Ck::E;
  const T* fimg = feats + b * N * Cf;
  float gk[KM];
#pragma unroll
  for (int k = 0; k < KM; ++k) gk[k] = 0.f;
#pragma unroll
  for (int r = 0; r < kMaxChunksPerLane; ++r) {
    const int c = g.sub + r * L;
    if (c >= nch) break;
    float o[Ck::E];
    Ck::load(dout + id * Cf + c * Ck::E, o);
    float v[KM][Ck::E];
#pragma unroll
    for (int k = 0; k < KM; ++k)
      if (qw.slot[k] >= 0) Ck::load(fimg + (int64_t)qw.slot[k] * Cf + c * Ck::E, v[k]);
#pragma unroll
    for (int k = 0; k < KM; ++k)
      if (qw.slot[k] >= 0)
#pragma unroll
        for (int e = 0; e < Ck::E; ++e) gk[k] = fmaf(o[e], v[k][e], gk[k]);
  }
  // <dO, F_k> over the group's lanes (aligned groups of L lanes)
  for (int off = 1; off < L; off <<= 1)
#pragma unroll
    for (int k = 0; k < KM; ++k) gk[k] += __shfl_xor(gk[k], off, 64);
  if (!g.valid || g.sub != 0) return;
  float delta = 0.f;
#pragma unroll
  for (int k = 0; k < KM; ++k) delta = fmaf(qw.w[k], gk[k], delta);
  float dqx = 0.f, dqy = 0.f, dps = 0.f;
#pragma unroll
  for (int k = 0; k < KM; ++k) {
    if (qw.slot[k] < 0) continue;
    const float ds = qw.w[k] * (gk[k] - delta);   // dL / d(-p d_k)
    dps = fmaf(-ds, qw.d[k], dps);
    if (qw.d[k] > 0.f) {
      const float f = -p * ds / qw.d[k];
      dqx = fmaf(f, qw.diff[k].x, dqx);
      dqy = fmaf(f, qw.diff[k].y, dqy);
    }
  }
  reinterpret_cast<float2*>(dq)[id] = make_float2(dqx, dqy);
  dpart[id] = dps;
  int32_t* cimg = cnt + b * N;
#pragma unroll
  for (int k = 0; k < KM; ++k) {
    if (k >= K) break;
    ent_slot[id * K + k] = qw.slot[k];
    ent_w[id * K + k] = qw.w[k];
    if (qw.slot[k] >= 0) atomicAdd(&cimg[qw.slot[k]], 1);
  }
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
knn_scan_kernel(int N, const int32_t* __restrict__ cnt_all, int32_t* __restrict__ off_all,
                int32_t* __restrict__ cur_all) {
  __shared__ int32_t v[kScanChunk];
  __shared__ int tmp[17];
  const int64_t b = blockIdx.x;
  const int32_t* cnt = cnt_all + b * N;
  int32_t* off = off_all + b * (N + 1);
  int32_t* cur = cur_all + b * N;
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
    for (int x = threadIdx.x; x < n; x += kScanThreads) {
      off[c0 + x] = v[x];
      cur[c0 + x] = v[x];
    }
    carry += tot;
    __syncthreads();
  }
  if (threadIdx.x == 0) off[N] = carry;
}

// one thread per (query, slot): the entry into its token's segment
__global__ void __launch_bounds__(kKnnThreads)
knn_place_kernel(int N, int M, int K, int64_t n_ent, const int32_t* __restrict__ ent_slot,
                 int32_t* __restrict__ cur_all, int32_t* __restrict__ ent_all) {
  const int64_t x = (int64_t)blockIdx.x * kKnnThreads + threadIdx.x;
  if (x >= n_ent) return;
  const int s = ent_slot[x];
  if (s < 0) return;
  const int64_t per = (int64_t)M * K;
  const int64_t b = x / per;
  const int pos = atomicAdd(&cur_all[b * N + s], 1);
  ent_all[b * per + pos] = (int32_t)(x - b * per);
}

// One thread per token sorts its segment by entry.  Short segments are
// sorted by their thread in LDS; longer ones afterwards by the whole wave,
// each lane ranking its entries by counting.
constexpr int kSortShort = 32;
__global__ void __launch_bounds__(kKnnThreads)
knn_sort_kernel(int N, int M, int K, int64_t n_tok, const int32_t* __restrict__ off_all,
                int32_t* __restrict__ ent_all) {
  __shared__ int32_t buf[kKnnThreads / 64][64 * kSortShort];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t x = (int64_t)blockIdx.x * kKnnThreads + threadIdx.x;
  const bool valid = x < n_tok;
  const int64_t b = valid ? x / N : 0;
  const int t = valid ? (int)(x - b * N) : 0;
  const int64_t per = (int64_t)M * K;
  int32_t* ent = ent_all + b * per;
  const int a = valid ? off_all[b * (N + 1) + t] : 0;
  const int z = valid ? off_all[b * (N + 1) + t + 1] : 0;
  const int n = z - a;
  int32_t* mine = &buf[w][lane * kSortShort];
  if (n <= kSortShort) {
    for (int u = 0; u < n; ++u) {
      const int32_t key = ent[a + u];
      int y = u - 1;
      while (y >= 0 && mine[y] > key) {
        mine[y + 1] = mine[y];
        --y;
      }
      mine[y + 1] = key;
    }
    for (int u = 0; u < n; ++u) ent[a + u] = mine[u];
  }
  // long segments: the wave ranks them one after the other
  uint64_t longs = __ballot(n > kSortShort);
  int32_t* wbuf = &buf[w][0];
  while (longs) {
    const int src = __builtin_ctzll(longs);
    longs &= longs - 1;
    const int la = __shfl(a, src, 64), ln = __shfl(n, src, 64);
    const int64_t lb = __shfl((int)b, src, 64);
    int32_t* le = ent_all + lb * per + la;
    if (ln <= 64 * kSortShort) {
      __builtin_amdgcn_s_waitcnt(0);   // earlier LDS traffic of the wave is done
      for (int u = lane; u < ln; u += 64) wbuf[u] = le[u];
      __builtin_amdgcn_s_waitcnt(0);
      __builtin_amdgcn_wave_barrier();
      for (int u = lane; u < ln; u += 64) {   // ranks from the LDS copy, distinct entries
        const int32_t key = wbuf[u];
        int r = 0;
        for (int y = 0; y < ln; ++y) r += wbuf[y] < key;
        le[r] = key;
      }
      __builtin_amdgcn_s_waitcnt(0);
      __builtin_amdgcn_wave_barrier();
    } else if (lane == 0) {   // very long: one lane, in place
      for (int u = 1; u < ln; ++u) {
        const int32_t key = le[u];
        int y = u - 1;
        while (y >= 0 && le[y] > key) {
          le[y + 1] = le[y];
          --y;
        }
        le[y + 1] = key;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Backward, token-major part: dF[b, t] = sum over its entries of w dO[b, m].
// ---------------------------------------------------------------------------
template <typename T>
__global__ void __launch_bounds__(kKnnThreads)
knn_dfeat_kernel(int N, int M, int Cf, int K, int lg, int64_t total, const T* __restrict__ dout,
                 const int32_t* __restrict__ off_all, const int32_t* __restrict__ ent_all,
                 const float* __restrict__ ent_w, T* __restrict__ dfeat) {
  using Ck = Chunk<T>;
  const Group g = group_of(lg, total);
  if (!g.valid) return;
  const int L = 1 << lg;
  const int64_t b = g.id / N;
  const int t = (int)(g.id - b * N);
  const int64_t per = (int64_t)M * K;
  const int a = off_all[b * (N + 1) + t], z = off_all[b * (N + 1) + t + 1];
  const int32_t* ent = ent_all + b * per;
  const float* wimg = ent_w + b * per;
  const T* oimg = dout + b * M * Cf;
  const int nch = Cf / Ck::E;
#pragma unroll
  for (int r = 0; r < kMaxChunksPerLane; ++r) {
    const int c = g.sub + r * L;
    if (c >= nch) break;
    float acc[Ck::E];
#pragma unroll
    for (int e = 0; e < Ck::E; ++e) acc[e] = 0.f;
    int u = a;
    for (; u + 4 <= z; u += 4) {   // four rows in flight
      float v[4][Ck::E], wt[4];
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const int e = ent[u + h];
        wt[h] = wimg[e];
        Ck::load(oimg + (int64_t)(e / K) * Cf + c * Ck::E, v[h]);
      }
#pragma unroll
      for (int h = 0; h < 4; ++h)
#pragma unroll
        for (int e = 0; e < Ck::E; ++e) acc[e] = fmaf(wt[h], v[h][e], acc[e]);
    }
    for (; u < z; ++u) {
      const int e = ent[u];
      float v[Ck::E];
      Ck::load(oimg + (int64_t)(e / K) * Cf + c * Ck::E, v);
      const float wt = wimg[e];
#pragma unroll
      for (int h = 0; h < Ck::E; ++h) acc[h] = fmaf(wt, v[h], acc[h]);
    }
    Ck::store(dfeat + g.id * Cf + c * Ck::E, acc);
  }
}

// dp = sum of the per-query shares, in a fixed order (one workgroup)
__global__ void __launch_bounds__(1024)
knn_dp_kernel(int64_t n, const float* __restrict__ dpart, float* __restrict__ dp) {
  __shared__ float red[1024];
  float s = 0.f;
  for (int64_t i = threadIdx.x; i < n; i += 1024) s += dpart[i];
  red[threadIdx.x] = s;
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
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(waves_grid(total, lg)), dim3(kKnnThreads), 0, st, N, M, Cf, G, K,
                       lg, p, total, coords, (const T*)feats, queries, table, (T*)out);
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
  // empty sizes launch nothing but the dp reduction (which then writes 0)
  if (ntok > 0) hipLaunchKernelGGL(knn_zero_kernel, grid1(ntok), dim3(kKnnThreads), 0, st, ntok, w.cnt);
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(waves_grid(nq, lg)), dim3(kKnnThreads), 0, st, N, M, Cf, G, K,
                       lg, p, nq, coords, (const T*)feats, queries, table, (const T*)dout, dq,
                       w.dpart, w.slot, w.wgt, w.cnt);
  };
  if (nq > 0) {
    if (K <= 4) go(knn_bwd_query_kernel<T, 4>);
    else if (K <= 8) go(knn_bwd_query_kernel<T, 8>);
    else go(knn_bwd_query_kernel<T, 16>);
  }
  if (ntok > 0) {
    hipLaunchKernelGGL(knn_scan_kernel, dim3(B), dim3(kScanThreads), 0, st, N,
                       (const int32_t*)w.cnt, w.off, w.cur);
    if (nq > 0)
      hipLaunchKernelGGL(knn_place_kernel, grid1(nent), dim3(kKnnThreads), 0, st, N, M, K, nent,
                         (const int32_t*)w.slot, w.cur, w.ent);
    hipLaunchKernelGGL(knn_sort_kernel, grid1(ntok), dim3(kKnnThreads), 0, st, N, M, K, ntok,
                       (const int32_t*)w.off, w.ent);
    hipLaunchKernelGGL(knn_dfeat_kernel<T>, dim3(waves_grid(ntok, lg)), dim3(kKnnThreads), 0, st,
                       N, M, Cf, K, lg, ntok, (const T*)dout, (const int32_t*)w.off,
                       (const int32_t*)w.ent, (const float*)w.wgt, (T*)dfeat);
  }
  hipLaunchKernelGGL(knn_dp_kernel, dim3(1), dim3(1024), 0, st, nq, (const float*)w.dpart, dp);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_knn_table(const float* coords, int B, int N, int G, int K, int32_t* table,
                            hipStream_t st) {
  const int parts = std::max(1, std::min(8, (G * G + kTabThreads - 1) / kTabThreads));
  hipLaunchKernelGGL(knn_table_kernel, dim3(B, parts), dim3(kTabThreads), 0, st, coords, N, G, K,
                     table);
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
