// Neighbour-list build for local cluster attention on gfx950, for 2D
// tokens and (templated on the dimension) 3D tokens.
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
// Kernels (all integer after one exact fp64 quantisation; candidate
// distances are screened in fp32 with a bound that never drops a tie):
//   build_small_kernel  images of at most 2048 tokens: the whole build in one
//                       1024-thread workgroup per image (counting sort of the
//                       (code, token) keys on the top code bits plus in-bucket
//                       insertion sort, bitonic fallback; centroid sums
//                       decoded from the sorted codes; 4-lane split scan).
//   segsort_kernel      larger images: every 1024-token segment sorted in
//                       LDS (a merge sort).
//   merge_round_kernel  pairwise merge of sorted runs (1024, 2048, ... tokens):
//                       a key's place is its place in its own run plus the
//                       count of partner-run keys below it (binary search).
//                       The last round writes the token order.
//   centroid_box_kernel integer centroid sums, and the bounding box of every
//                       64 consecutive clusters (one tile).
//   select_box_kernel   per cluster: candidate scan of its own tile, then of
//                       every other tile whose box lies within the current
//                       (k-1)-th best distance of some cluster of the wave;
//                       keeps the k-1 smallest (d2 << kIdxBits | index) keys,
//                       then writes the key lists.
//
// Ragged images: an image of n tokens has ceil(n / 8) clusters, the last
// one holding n mod 8 members when 8 does not divide n; its q_idx row and
// the key slots of its absent members are -1.  Centroids are compared
// through their means (sums scaled by mean_scale).  A packed batch of
// images of different sizes (Geom with offsets) is built image by image:
// images of at most Geom::small_max (2048 or 4096) tokens by the in-LDS
// kernel, larger ones by the segment / merge path; both skip the other's
// images.
//
// 3D tokens (notes page, "Limitations & Future Work": 3D voxels named as
// the open extension): the same steps with three axes, each quantised to 14
// bits, a 42-bit Morton code with x, y, z in bits 3b, 3b+1, 3b+2, and a
// 64-bit sort key (code << 22 | token).
#include "common.h"

#include <algorithm>

namespace ca {

namespace {

constexpr int kRankThreads = 256;

__host__ __device__ __forceinline__ uint32_t spread16(uint32_t v) {
  v &= 0xFFFFu;
  v = (v | (v << 8)) & 0x00FF00FFu;
  v = (v | (v << 4)) & 0x0F0F0F0Fu;
  v = (v | (v << 2)) & 0x33333333u;
  v = (v | (v << 1)) & 0x55555555u;
  return v;
}

__host__ __device__ __forceinline__ uint32_t compact16(uint32_t v) {
  v &= 0x55555555u;
  v = (v | (v >> 1)) & 0x33333333u;
  v = (v | (v >> 2)) & 0x0F0F0F0Fu;
  v = (v | (v >> 4)) & 0x00FF00FFu;
  v = (v | (v >> 8)) & 0x0000FFFFu;
  return v;
}

// bit b of v (b < 21) -> bit 3b, by shifting groups into place
__host__ __device__ __forceinline__ uint64_t spread3(uint32_t v) {
  uint64_t x = v & 0x1FFFFFu;
  x = (x | (x << 32)) & 0x001F00000000FFFFull;
  x = (x | (x << 16)) & 0x001F0000FF0000FFull;
  x = (x | (x << 8)) & 0x100F00F00F00F00Full;
  x = (x | (x << 4)) & 0x10C30C30C30C30C3ull;
  x = (x | (x << 2)) & 0x1249249249249249ull;
  return x;
}

// bits 3b of x -> bit b (the inverse of spread3)
__host__ __device__ __forceinline__ uint32_t compact3(uint64_t x) {
  x &= 0x1249249249249249ull;
  x = (x | (x >> 2)) & 0x10C30C30C30C30C3ull;
  x = (x | (x >> 4)) & 0x100F00F00F00F00Full;
  x = (x | (x >> 8)) & 0x001F0000FF0000FFull;
  x = (x | (x >> 16)) & 0x001F00000000FFFFull;
  x = (x | (x >> 32)) & 0x00000000001FFFFFull;
  return (uint32_t)x;
}

// What differs between 2D and 3D tokens: the fixed-point width, the Morton
// interleave, the split of the 64-bit sort key into code and token, and the
// centroid vector types.  Sort keys are (code << kTokBits | token) in both,
// so the top 11 key bits are the top 11 code bits.
template <int DIM> struct Space;

template <> struct Space<2> {
  static constexpr int kTokBits = 32;
  static constexpr uint32_t kQMax = 0xFFFFu;
  typedef uint32_t Packed;   // quantised coordinates of a sorted token: qx | qy << 16
  typedef int2 ICent;        // scaled centroid sums (integers)
  typedef float2 FCent;      // the same as exact floats (below 2^22)
  static __device__ __forceinline__ uint64_t code(const float* __restrict__ c, int64_t e,
                                                  double step) {
    const float2 p = reinterpret_cast<const float2*>(c)[e];
    return spread16(quantize_axis(p.x, step)) | (spread16(quantize_axis(p.y, step)) << 1);
  }
  static __device__ __forceinline__ void axes(uint64_t code, int (&q)[2]) {
    q[0] = (int)compact16((uint32_t)code);
    q[1] = (int)compact16((uint32_t)code >> 1);
  }
  static __device__ __forceinline__ Packed pack(uint64_t code) {
    return compact16((uint32_t)code) | (compact16((uint32_t)code >> 1) << 16);
  }
  static __device__ __forceinline__ void unpack(Packed w, int (&q)[2]) {
    q[0] = (int)(w & 0xFFFFu);
    q[1] = (int)(w >> 16);
  }
  static __device__ __forceinline__ ICent icent(const int (&s)[2]) { return make_int2(s[0], s[1]); }
  static __device__ __forceinline__ FCent fcent(const int (&s)[2]) {
    return make_float2((float)s[0], (float)s[1]);
  }
};

template <> struct Space<3> {
  static constexpr int kTokBits = 22;
  static constexpr uint32_t kQMax = 0x3FFFu;
  typedef uint64_t Packed;   // the Morton code itself
  typedef int4 ICent;
  typedef float4 FCent;
  static __device__ __forceinline__ uint32_t q14(float c, double step) {
    double q = floor(((double)c + 0.5) * step);   // exact, as in quantize_axis
    q = q < 0.0 ? 0.0 : (q > (double)kQMax ? (double)kQMax : q);
    return (uint32_t)q;
  }
  static __device__ __forceinline__ uint64_t code(const float* __restrict__ c, int64_t e,
                                                  double step) {
    const float* p = c + 3 * e;
    return spread3(q14(p[0], step)) | (spread3(q14(p[1], step)) << 1) |
           (spread3(q14(p[2], step)) << 2);
  }
  static __device__ __forceinline__ void axes(uint64_t code, int (&q)[3]) {
    q[0] = (int)compact3(code);
    q[1] = (int)compact3(code >> 1);
    q[2] = (int)compact3(code >> 2);
  }
  static __device__ __forceinline__ Packed pack(uint64_t code) { return code; }
  static __device__ __forceinline__ void unpack(Packed w, int (&q)[3]) { axes(w, q); }
  static __device__ __forceinline__ ICent icent(const int (&s)[3]) {
    return make_int4(s[0], s[1], s[2], 0);
  }
  static __device__ __forceinline__ FCent fcent(const int (&s)[3]) {
    return make_float4((float)s[0], (float)s[1], (float)s[2], 0.f);
  }
};

__device__ __forceinline__ void get(int2 v, int (&a)[2]) { a[0] = v.x; a[1] = v.y; }
__device__ __forceinline__ void get(int4 v, int (&a)[3]) { a[0] = v.x; a[1] = v.y; a[2] = v.z; }
__device__ __forceinline__ void get(float2 v, float (&a)[2]) { a[0] = v.x; a[1] = v.y; }
__device__ __forceinline__ void get(float4 v, float (&a)[3]) { a[0] = v.x; a[1] = v.y; a[2] = v.z; }

template <int DIM> __device__ __forceinline__ uint64_t tok_mask() {
  return (uint64_t(1) << Space<DIM>::kTokBits) - 1;
}

// One round of the image-wide merge sort.  Sorted runs of `run` keys (a
// power of two) are merged pairwise; grid = (ceil(Nmax / 256), B), one
// thread per key.  Keys are unique (they hold the token index), so a key's
// place in the merged run is its place in its own run plus the number of
// keys of the partner run below it (an image already in one run is
// copied).  The last round (out == nullptr) writes the q_idx rows (token
// ids) and the quantised coordinates of the sorted tokens, decoded from the
// code, at the image's cluster slots.
template <int DIM>
__global__ void __launch_bounds__(kRankThreads)
merge_round_kernel(Geom g, int run, const uint64_t* __restrict__ in, uint64_t* __restrict__ out,
                   int32_t* __restrict__ q_idx, typename Space<DIM>::Packed* __restrict__ qsorted) {
  const int x = blockIdx.x * kRankThreads + threadIdx.x;
  int t0, n, c0, nc;
  g.image(blockIdx.y, t0, n, c0, nc);
  if (n <= g.small_max || x >= n) return;
  const uint64_t* img = in + t0;
  const uint64_t key = img[x];
  const int p0 = x & ~(2 * run - 1);
  const bool first = x - p0 < run;
  const int own0 = first ? p0 : p0 + run;
  int lo = first ? p0 + run : p0;
  int hi = first ? min(p0 + 2 * run, n) : p0 + run;
  hi = max(hi, lo);   // a last run without partner
  const int base = lo;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (img[mid] < key) lo = mid + 1; else hi = mid;
  }
  const int pos = p0 + (x - own0) + (lo - base);
  if (out) {
    out[(int64_t)t0 + pos] = key;
  } else {
    const int64_t at = (int64_t)c0 * 8 + pos;
    q_idx[at] = g.tok_base(t0) + (int32_t)(key & tok_mask<DIM>());
    qsorted[at] = Space<DIM>::pack(key >> Space<DIM>::kTokBits);
  }
}

// Scaled centroid sums of every cluster and the bounding box (per axis
// minimum and maximum, stored as two centroid vectors) of every tile of
// kBoxTile consecutive clusters of an image.  grid = (ceil(Cmax / kBoxTile),
// B), one wavefront per tile.  The absent members of a partial last cluster
// get -1 in q_idx here.
template <int DIM>
__global__ void __launch_bounds__(kBoxTile)
centroid_box_kernel(Geom g, const typename Space<DIM>::Packed* __restrict__ qsorted,
                    typename Space<DIM>::FCent* __restrict__ cent_all,
                    typename Space<DIM>::FCent* __restrict__ box_all, int32_t* __restrict__ q_idx) {
  typedef Space<DIM> S;
  const int t = blockIdx.x;
  const int b = blockIdx.y;
  int t0, n, c0, nc;
  g.image(b, t0, n, c0, nc);
  if (n <= g.small_max) return;
  const int c = t * kBoxTile + threadIdx.x;
  float lo[DIM], hi[DIM];
#pragma unroll
  for (int a = 0; a < DIM; ++a) {
    lo[a] = INFINITY;
    hi[a] = -INFINITY;
  }
  if (c < nc) {
    const int members = min(8, n - 8 * c);
    const typename S::Packed* q8 = qsorted + ((int64_t)c0 + c) * 8;
    int sum[DIM] = {};
    for (int m = 0; m < members; ++m) {
      int q[DIM];
      S::unpack(q8[m], q);
#pragma unroll
      for (int a = 0; a < DIM; ++a) sum[a] += q[a];
    }
    const int f = mean_scale(members, n);
#pragma unroll
    for (int a = 0; a < DIM; ++a) {
      sum[a] *= f;   // below 2^22: exact as floats
      lo[a] = hi[a] = (float)sum[a];
    }
    cent_all[(int64_t)c0 + c] = S::fcent(sum);
    for (int m = members; m < 8; ++m) q_idx[((int64_t)c0 + c) * 8 + m] = -1;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
#pragma unroll
    for (int a = 0; a < DIM; ++a) {
      lo[a] = fminf(lo[a], __shfl_xor(lo[a], o, 64));
      hi[a] = fmaxf(hi[a], __shfl_xor(hi[a], o, 64));
    }
  }
  if (threadIdx.x == 0) {
    int il[DIM], ih[DIM];   // the floats hold integers: the conversion is exact
#pragma unroll
    for (int a = 0; a < DIM; ++a) {
      il[a] = (int)lo[a];
      ih[a] = (int)hi[a];
    }
    const int64_t at = ((int64_t)b * gridDim.x + t) * 2;
    if (nc > t * kBoxTile) {
      box_all[at] = S::fcent(il);
      box_all[at + 1] = S::fcent(ih);
    }
  }
}

template <int KM1>
__device__ __forceinline__ void top_insert(uint64_t (&best)[KM1 > 0 ? KM1 : 1], uint64_t x) {
  if constexpr (KM1 > 0) {
    if (x >= best[KM1 - 1]) return;
#pragma unroll
    for (int r = 0; r < KM1; ++r) {
      const uint64_t lo = x < best[r] ? x : best[r];
      const uint64_t hi = x < best[r] ? best[r] : x;
      best[r] = lo;
      x = hi;
    }
  }
}

// Scan one tile of candidate centroids (staged in this wave's LDS row) for
// the lanes with `need`, keeping the KM1 smallest (d2 << kIdxBits | index)
// keys.  A scaled centroid sum is at most lcm(8, n mod 8) <= 56 times the
// largest fixed-point coordinate, so in 2D d2 <= 2 (56 * 65535)^2 < 2^45 and
// in 3D d2 <= 3 (56 * 16383)^2 < 2^42: with kIdxBits = 19 index bits a key
// fills at most all 64 bits (the static_asserts below tie the three
// constants together).  Candidates are screened with an fp32 distance whose error bound
// (relative 2^-22) cannot drop a candidate at or below the current KM1-th
// best; the survivors are compared exactly in 64 bits, so the kept set does
// not depend on the order of the scan.
static_assert(2.0 * (56.0 * 65535.0) * (56.0 * 65535.0) < 18446744073709551616.0 / (1u << kIdxBits),
              "2D (distance, index) sort keys overflow 64 bits");
static_assert(3.0 * (56.0 * 16383.0) * (56.0 * 16383.0) < 18446744073709551616.0 / (1u << kIdxBits),
              "3D (distance, index) sort keys overflow 64 bits");

template <int KM1, int DIM>
__device__ __forceinline__ void scan_tile(const typename Space<DIM>::FCent* __restrict__ cent,
                                          typename Space<DIM>::FCent* __restrict__ row, int t0,
                                          int T, int c, const float (&me)[DIM], bool need,
                                          uint64_t (&best)[KM1 > 0 ? KM1 : 1], float& thr) {
  typedef typename Space<DIM>::FCent FC;
  const int lane = threadIdx.x & 63;
  FC mine;
  if (lane < T) mine = cent[t0 + lane];
  else mine = FC{};
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // earlier reads of the row are done
  row[lane] = mine;
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // the row is written (one wave)
  if (!need) return;
  for (int i0 = 0; i0 < T; i0 += 8) {
    float cc[8][DIM];
    if constexpr (DIM == 2) {
      const float4* row4 = reinterpret_cast<const float4*>(row);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float4 q = row4[(i0 >> 1) + u];
        cc[2 * u][0] = q.x;
        cc[2 * u][1] = q.y;
        cc[2 * u + 1][0] = q.z;
        cc[2 * u + 1][1] = q.w;
      }
    } else {
#pragma unroll
      for (int u = 0; u < 8; ++u) get(row[i0 + u], cc[u]);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int e = i0 + u;
      float d[DIM];
#pragma unroll
      for (int a = 0; a < DIM; ++a) d[a] = cc[u][a] - me[a];   // exact
      float d2f = d[0] * d[0];
#pragma unroll
      for (int a = 1; a < DIM; ++a) d2f = fmaf(d[a], d[a], d2f);
      if (e >= T || d2f > thr || t0 + e == c) continue;
      int64_t d2 = 0;
#pragma unroll
      for (int a = 0; a < DIM; ++a) d2 += (int64_t)(int)d[a] * (int)d[a];
      const uint64_t key = ((uint64_t)d2 << kIdxBits) | (uint32_t)(t0 + e);
      if (key >= best[KM1 - 1]) continue;
      uint64_t x = key;
#pragma unroll
      for (int r = 0; r < KM1; ++r) {
        const uint64_t lo = x < best[r] ? x : best[r];
        const uint64_t hi = x < best[r] ? best[r] : x;
        best[r] = lo;
        x = hi;
      }
      if (best[KM1 - 1] != ~0ull) thr = (float)(best[KM1 - 1] >> kIdxBits) * (1.0f + 0x1p-20f);
    }
  }
}

__device__ __forceinline__ float wave_minf(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fminf(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ __forceinline__ float wave_maxf(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}

// squared distance from point p to the box [lo, hi] (exact for integer floats)
template <int DIM>
__device__ __forceinline__ float box_d2(const float (&lo)[DIM], const float (&hi)[DIM],
                                        const float (&plo)[DIM], const float (&phi)[DIM]) {
  float s = 0.f;
#pragma unroll
  for (int a = 0; a < DIM; ++a) {
    const float d = fmaxf(fmaxf(lo[a] - phi[a], plo[a] - hi[a]), 0.f);
    s = fmaf(d, d, s);
  }
  return s;
}

// Nearest clusters and key lists.  grid = (ceil(C / kBoxTile), B); the
// kSelWaves wavefronts of a workgroup serve the same tile of clusters, one
// lane per cluster.  Every wave scans the own tile (which sets each lane's
// threshold, its current KM1-th best distance), then the tiles whose
// bounding box lies within the largest threshold of the wave from the
// bounding box of the wave's clusters are dealt round-robin to the waves;
// each scans a dealt tile for the lanes whose own threshold still reaches
// the tile's box.  The waves' lists are merged at the end.
constexpr int kSelWaves = 4;

template <int KM1, int DIM>
__global__ void __launch_bounds__(kBoxTile * kSelWaves)
select_box_kernel(Geom g, const typename Space<DIM>::FCent* __restrict__ cent_all,
                  const typename Space<DIM>::FCent* __restrict__ box_all,
                  const int32_t* __restrict__ q_idx, int32_t* __restrict__ nbr,
                  int32_t* __restrict__ key_idx) {
  typedef typename Space<DIM>::FCent FC;
  constexpr int KB = KM1 > 0 ? KM1 : 1;
  __shared__ __align__(16) FC cand[kSelWaves][kBoxTile];
  __shared__ uint64_t part[kSelWaves - 1][KB][kBoxTile];
  const int b = blockIdx.y;
  int t0, n, c0, C;
  g.image(b, t0, n, c0, C);
  const int ntiles = (C + kBoxTile - 1) / kBoxTile;
  const int own = blockIdx.x;
  if (n <= g.small_max || own >= ntiles) return;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c = own * kBoxTile + lane;
  const bool valid = c < C;
  const FC* cent = cent_all + c0;
  const FC* box = box_all + (int64_t)b * gridDim.x * 2;
  float me[DIM];
  {
    FC mc;
    if (valid) mc = cent[c];
    else mc = FC{};
    get(mc, me);
  }

  uint64_t best[KB];
#pragma unroll
  for (int r = 0; r < KB; ++r) best[r] = ~0ull;
  float thr = INFINITY;

  if constexpr (KM1 > 0) {
    scan_tile<KM1, DIM>(cent, cand[w], own * kBoxTile, min(kBoxTile, C - own * kBoxTile), c, me,
                        valid, best, thr);
    // bounding box of the wave's clusters and its largest threshold
    float mlo[DIM], mhi[DIM];
#pragma unroll
    for (int a = 0; a < DIM; ++a) {
      mlo[a] = wave_minf(valid ? me[a] : INFINITY);
      mhi[a] = wave_maxf(valid ? me[a] : -INFINITY);
    }
    const float mthr = wave_maxf(valid ? thr : -INFINITY);
    int dealt = 0;   // candidate tiles seen so far (all waves agree)
    for (int g0 = 0; g0 < ntiles; g0 += 64) {
      const int tl = g0 + lane;
      bool cand_tile = false;
      if (tl < ntiles && tl != own) {
        float lo[DIM], hi[DIM];
        get(box[2 * tl], lo);
        get(box[2 * tl + 1], hi);
        cand_tile = box_d2<DIM>(lo, hi, mlo, mhi) <= mthr;
      }
      uint64_t mask = __ballot(cand_tile);
      while (mask) {
        const int bit = __builtin_ctzll(mask);
        mask &= mask - 1;
        if (dealt++ % kSelWaves != w) continue;
        const int tt = g0 + bit;
        float lo[DIM], hi[DIM];
        get(box[2 * tt], lo);
        get(box[2 * tt + 1], hi);
        const bool need = valid && box_d2<DIM>(lo, hi, me, me) <= thr;
        if (!__any(need)) continue;
        scan_tile<KM1, DIM>(cent, cand[w], tt * kBoxTile, min(kBoxTile, C - tt * kBoxTile), c, me,
                            need, best, thr);
      }
    }
    // merge the waves' lists into wave 0; every wave holds the own tile's
    // survivors, so keys already present are skipped (keys are unique per
    // candidate)
    if (w > 0) {
#pragma unroll
      for (int r = 0; r < KM1; ++r) part[w - 1][r][lane] = best[r];
    }
    __syncthreads();
    if (w > 0) return;
#pragma unroll
    for (int v = 0; v < kSelWaves - 1; ++v) {
#pragma unroll
      for (int r = 0; r < KM1; ++r) {
        const uint64_t x = part[v][r][lane];
        bool dup = false;
#pragma unroll
        for (int q = 0; q < KM1; ++q) dup = dup || best[q] == x;
        if (!dup) top_insert<KM1>(best, x);
      }
    }
  } else {
    if (w > 0) return;
  }
  if (!valid) return;

  constexpr int K = KM1 + 1;
  constexpr uint64_t kIdxMask = (uint64_t(1) << kIdxBits) - 1;
  int32_t ids[K];
  ids[0] = c;
#pragma unroll
  for (int r = 0; r < KM1; ++r) ids[r + 1] = best[r] == ~0ull ? -1 : (int32_t)(best[r] & kIdxMask);
  const int cb = g.clu_base(c0);
  int32_t* nrow = nbr + ((int64_t)c0 + c) * K;
  int4* krow = reinterpret_cast<int4*>(key_idx + ((int64_t)c0 + c) * K * 8);
  // q_idx rows of the image: token ids as written out, -1 for absent members
  const int4* pimg = reinterpret_cast<const int4*>(q_idx + (int64_t)c0 * 8);
  const int4 none = make_int4(-1, -1, -1, -1);
#pragma unroll
  for (int s = 0; s < K; ++s) {
    nrow[s] = ids[s] >= 0 ? cb + ids[s] : -1;
    krow[2 * s] = ids[s] >= 0 ? pimg[2 * ids[s]] : none;
    krow[2 * s + 1] = ids[s] >= 0 ? pimg[2 * ids[s] + 1] : none;
  }
}

// ---------------------------------------------------------------------------
// Whole build for an image of at most KPT * 1024 tokens (2048 or 4096) in
// one 1024-thread workgroup, everything staged in LDS: (code, token) keys
// are sorted (counting sort with in-bucket insertion, bitonic fallback),
// the cluster centroid sums are decoded from the sorted codes, and each
// cluster's candidate scan is split over up to 16 lanes whose top lists are
// merged with lane shuffles.  grid = (B, parts).
// ---------------------------------------------------------------------------
constexpr int kSmallThreads = 1024;

// 64-bit lane move with a DPP pattern (both halves moved the same way)
template <int CTRL>
__device__ __forceinline__ uint64_t dpp64(uint64_t v) {
  const int lo = __builtin_amdgcn_mov_dpp((int)(uint32_t)v, CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_mov_dpp((int)(uint32_t)(v >> 32), CTRL, 0xF, 0xF, false);
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}

// Minimum over each aligned group of `lanes` lanes (a power of two <= 16,
// wave-uniform), every lane active: quad swaps, then the half-row and row
// mirrors, which pair each quad (eight) with the other one of its eight
// (sixteen).  Register moves instead of LDS-crossbar shuffles.
__device__ __forceinline__ uint64_t group_min64(uint64_t m, int lanes) {
  uint64_t x;
  if (lanes > 1) { x = dpp64<0xB1>(m); m = x < m ? x : m; }    // quad_perm [1,0,3,2]
  if (lanes > 2) { x = dpp64<0x4E>(m); m = x < m ? x : m; }    // quad_perm [2,3,0,1]
  if (lanes > 4) { x = dpp64<0x141>(m); m = x < m ? x : m; }   // row_half_mirror
  if (lanes > 8) { x = dpp64<0x140>(m); m = x < m ? x : m; }   // row_mirror
  return m;
}

constexpr int kBuckets = 2 * kSmallThreads;       // counting-sort buckets (11 key bits)
constexpr int kMaxBucket = 32;                    // larger buckets -> bitonic fallback

__device__ __forceinline__ int64_t sq_dist(int2 a, int2 b) {
  const int dx = a.x - b.x, dy = a.y - b.y;
  return (int64_t)dx * dx + (int64_t)dy * dy;
}
__device__ __forceinline__ int64_t sq_dist(int4 a, int4 b) {
  const int dx = a.x - b.x, dy = a.y - b.y, dz = a.z - b.z;
  return (int64_t)dx * dx + (int64_t)dy * dy + (int64_t)dz * dz;
}

// Sort up to KPT * 1024 (code << token bits | token) keys of a whole image
// in LDS, KPT per thread (kk, ~0 past the end), into keys[0 .. n).
// Counting sort on the top 11 key bits (2048 buckets), then an insertion
// sort inside each bucket restores the exact order whatever the arrival
// order of the atomics.  Buckets hold about one key for the grid-like
// layouts of the workloads; if any bucket exceeds kMaxBucket keys the
// workgroup falls back to a bitonic sort.  Ends with a barrier.
constexpr int kBucketShift = 53;

template <int KPT>
__device__ __forceinline__ void lds_sort_keys(const uint64_t (&kk)[KPT], int n, uint64_t* keys,
                                              int* bcnt, int* bstart, int* scan_tmp,
                                              int* overflow) {
  const int tid = threadIdx.x;
  int bk[KPT], arr[KPT];
#pragma unroll
  for (int r = 0; r < KPT; ++r)
    bk[r] = tid + r * kSmallThreads < n ? (int)(kk[r] >> kBucketShift) : -1;
  bcnt[tid] = 0;
  bcnt[tid + kSmallThreads] = 0;
  if (tid == 0) *overflow = 0;
  __syncthreads();
#pragma unroll
  for (int r = 0; r < KPT; ++r) arr[r] = bk[r] >= 0 ? atomicAdd(&bcnt[bk[r]], 1) : 0;
  __syncthreads();
  const int c0 = bcnt[2 * tid], c1 = bcnt[2 * tid + 1];
  if (c0 > kMaxBucket || c1 > kMaxBucket) *overflow = 1;
  int total;
  const int ex = block_exclusive_scan(c0 + c1, scan_tmp, kSmallThreads, &total);
  bstart[2 * tid] = ex;
  bstart[2 * tid + 1] = ex + c0;
  __syncthreads();
  if (!*overflow) {
#pragma unroll
    for (int r = 0; r < KPT; ++r)
      if (bk[r] >= 0) keys[bstart[bk[r]] + arr[r]] = kk[r];
    __syncthreads();
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int s0 = h ? ex + c0 : ex, m = h ? c1 : c0;
      for (int x = 1; x < m; ++x) {
        const uint64_t key = keys[s0 + x];
        int y = x - 1;
        while (y >= 0 && keys[s0 + y] > key) {
          keys[s0 + y + 1] = keys[s0 + y];
          --y;
        }
        keys[s0 + y + 1] = key;
      }
    }
  } else {
    int P = 2;
    while (P < n) P <<= 1;
#pragma unroll
    for (int r = 0; r < KPT; ++r) {
      const int e = tid + r * kSmallThreads;
      if (e < P) keys[e] = kk[r];
    }
    __syncthreads();
    for (int k = 2; k <= P; k <<= 1) {
      for (int j = k >> 1; j > 0; j >>= 1) {
        for (int i = tid; i < P / 2; i += kSmallThreads) {
          const int a = ((i & ~(j - 1)) << 1) | (i & (j - 1));
          const uint64_t x = keys[a], y = keys[a + j];
          if ((x > y) == ((a & k) == 0)) {
            keys[a] = y;
            keys[a + j] = x;
          }
        }
        __syncthreads();
      }
    }
  }
  __syncthreads();
}

// Larger images: every run of kSegSort consecutive tokens sorted in LDS.
// A segment of a large image covers a narrow strip of its space, so a
// counting sort on fixed key bits would crowd few buckets; this is a merge
// sort instead: each thread sorts its four keys, then eight rounds merge
// sorted runs pairwise (a key's place = its place in its run + the number
// of partner-run keys below it, by binary search in LDS; keys are unique;
// positions past the segment's L keys are never read).
// grid = (B * segs), one 256-thread workgroup per 1024-key segment; the
// sorted runs go to run_keys at the segment's place.
constexpr int kSegThreads = 256;
constexpr int kSegSort = 4 * kSegThreads;   // keys per segment

template <int DIM>
__global__ void __launch_bounds__(kSegThreads)
segsort_kernel(const float* __restrict__ coords, Geom g, int segs_per_image, double step,
               uint64_t* __restrict__ run_keys) {
  __shared__ uint64_t buf[2][kSegSort];
  const int b = blockIdx.x / segs_per_image;
  const int start = (blockIdx.x % segs_per_image) * kSegSort;
  int t0, n, c0, nc;
  g.image(b, t0, n, c0, nc);
  if (n <= g.small_max) return;                       // built by the in-LDS kernel
  const int L = min(kSegSort, n - start);
  if (L <= 0) return;
  const float* img = coords + ((int64_t)t0 + start) * DIM;
  const int tid = threadIdx.x;
  // this thread's four consecutive keys (padding ~0 sorts last), sorted
  uint64_t k[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int e = 4 * tid + r;
    k[r] = e < L ? (Space<DIM>::code(img, e, step) << Space<DIM>::kTokBits) | (uint32_t)(start + e)
                 : ~0ull;
  }
  auto cswap = [](uint64_t& a, uint64_t& c) {
    const uint64_t lo = a < c ? a : c, hi = a < c ? c : a;
    a = lo;
    c = hi;
  };
  cswap(k[0], k[1]);
  cswap(k[2], k[3]);
  cswap(k[0], k[2]);
  cswap(k[1], k[3]);
  cswap(k[1], k[2]);
#pragma unroll
  for (int r = 0; r < 4; ++r) buf[0][4 * tid + r] = k[r];
  __syncthreads();
  int cur = 0;
  for (int run = 4; run < kSegSort; run *= 2) {
    const uint64_t* in = buf[cur];
    uint64_t* out = buf[cur ^ 1];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int x = 4 * tid + r;
      if (x >= L) continue;   // positions past the segment's keys take no part
      const uint64_t key = in[x];
      const int p0 = x & ~(2 * run - 1);
      const bool first = x - p0 < run;
      int lo = first ? p0 + run : p0;
      int hi = first ? min(p0 + 2 * run, L) : p0 + run;
      hi = max(hi, lo);   // a last run without partner
      const int base = lo;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (in[mid] < key) lo = mid + 1; else hi = mid;
      }
      out[p0 + (x - (first ? p0 : p0 + run)) + (lo - base)] = key;
    }
    cur ^= 1;
    __syncthreads();
  }
  uint64_t* dst = run_keys + (int64_t)t0 + start;
  for (int e = tid; e < L; e += kSegThreads) dst[e] = buf[cur][e];
}

template <int KM1, int KPT, int DIM>
__global__ void __launch_bounds__(kSmallThreads)
build_small_kernel(const float* __restrict__ coords, Geom g, double step, int parts, int lanes,
                   int32_t* __restrict__ q_idx, int32_t* __restrict__ nbr,
                   int32_t* __restrict__ key_idx) {
  typedef Space<DIM> S;
  typedef typename S::ICent IC;
  constexpr int kMaxN = KPT * kSmallThreads;
  __shared__ uint64_t keys[kMaxN];
  __shared__ int bcnt[kBuckets];
  __shared__ int bstart[kBuckets];
  __shared__ IC cent[kMaxN / 8];
  __shared__ int scan_tmp[17];
  __shared__ int overflow;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  int t0, N, cl0, C;
  g.image(b, t0, N, cl0, C);
  if (N > kMaxN || N == 0) return;   // larger images: segment / merge path
  const int tb = g.tok_base(t0), cb = g.clu_base(cl0);
  const float* img = coords + (int64_t)t0 * DIM;

  // sort the (code << kTokBits | token) keys in LDS
  uint64_t kk[KPT];
#pragma unroll
  for (int r = 0; r < KPT; ++r) {
    const int e = tid + r * kSmallThreads;
    kk[r] = e < N ? (S::code(img, e, step) << S::kTokBits) | (uint32_t)e : ~0ull;
  }
  lds_sort_keys<KPT>(kk, N, keys, bcnt, bstart, scan_tmp, &overflow);

  // centroid sums decoded from the sorted codes, scaled to compare means
  for (int c = tid; c < C; c += kSmallThreads) {
    const int members = min(8, N - 8 * c);
    int sum[DIM] = {};
    for (int m = 0; m < members; ++m) {
      int q[DIM];
      S::axes(keys[8 * c + m] >> S::kTokBits, q);
#pragma unroll
      for (int a = 0; a < DIM; ++a) sum[a] += q[a];
    }
    const int f = mean_scale(members, N);
#pragma unroll
    for (int a = 0; a < DIM; ++a) sum[a] *= f;
    cent[c] = S::icent(sum);
  }
  const uint64_t tmask = tok_mask<DIM>();
  if (blockIdx.y == 0) {   // q_idx rows: token ids, -1 past the end of the order
    int32_t* qimg = q_idx + (int64_t)cl0 * 8;
    for (int e = tid; e < 8 * C; e += kSmallThreads)
      qimg[e] = e < N ? tb + (int32_t)(keys[e] & tmask) : -1;
  }
  __syncthreads();

  // Candidate scan.  Workgroup y of the image takes clusters
  // [y*CP, (y+1)*CP) (CP = ceil(C / parts)); `lanes` lanes (a power of two
  // <= 16) share a cluster: lane q scans the candidates at Morton offsets
  // +1, -1, +2, -2, ... (mod C) numbered q, q + lanes, ..., so the nearest
  // in Morton order come first.  Keys are exact (d2 << kIdxBits | index)
  // in 64 bits from integer scaled centroid sums (below 2^22), and a
  // candidate is inserted only when it beats the lane's current k-1-th
  // best, which after the first few near candidates is rare (the wavefront
  // stays off the divergent insertion path).  The kept set does not depend
  // on the order.
  constexpr int KB = KM1 > 0 ? KM1 : 1;
  const int CP = (C + parts - 1) / parts;
  const int q = tid & (lanes - 1);
  const int cl = tid / lanes;
  const int c = blockIdx.y * CP + cl;
  const bool mine = cl < CP && c < C;
  uint64_t best[KB];
#pragma unroll
  for (int r = 0; r < KB; ++r) best[r] = ~0ull;
  if constexpr (KM1 > 0) {
    if (mine) {
      const IC me = cent[c];
      constexpr int U = 4;   // candidates read per iteration (independent LDS loads)
      for (int s0 = q; s0 < C; s0 += U * lanes) {
        uint64_t key[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int sn = s0 + u * lanes;                  // candidate number
          const int o = (sn + 1) >> 1;                    // Morton offset magnitude
          int e = (sn & 1) ? c + o : c - o;
          e = e >= C ? e - C : (e < 0 ? e + C : e);
          const IC cc = cent[(sn > 0 && sn < C) ? e : c];
          const int64_t d2 = sq_dist(cc, me);
          // sn == 0 is the cluster itself; sn >= C is past the end
          key[u] = (sn > 0 && sn < C) ? ((uint64_t)d2 << kIdxBits) | (uint32_t)e : ~0ull;
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
          if (key[u] < best[KM1 - 1]) top_insert<KM1>(best, key[u]);
      }
    }
    // Merge the sorted partial lists of the lanes of a cluster (aligned lane
    // groups) by a tournament: KM1 times, the smallest head over the group
    // is taken and its lane (keys are unique) drops its head.
    uint64_t merged[KB];
#pragma unroll
    for (int r = 0; r < KM1; ++r) {
      const uint64_t m = group_min64(best[0], lanes);
      merged[r] = m;
      if (best[0] == m && m != ~0ull) {
#pragma unroll
        for (int u = 0; u + 1 < KM1; ++u) best[u] = best[u + 1];
        best[KM1 - 1] = ~0ull;
      }
    }
#pragma unroll
    for (int r = 0; r < KM1; ++r) best[r] = merged[r];
  }
  if (!mine) return;

  constexpr int K = KM1 + 1;
  constexpr uint64_t kIdxMask = (uint64_t(1) << kIdxBits) - 1;
  int32_t ids[K];
  ids[0] = c;
#pragma unroll
  for (int r = 0; r < KM1; ++r) ids[r + 1] = best[r] == ~0ull ? -1 : (int32_t)(best[r] & kIdxMask);
  if (q == 0) {
#pragma unroll
    for (int s = 0; s < K; ++s) nbr[((int64_t)cl0 + c) * K + s] = ids[s] >= 0 ? cb + ids[s] : -1;
  }
  // the lanes of the cluster write its slot groups round-robin
  int4* krow = reinterpret_cast<int4*>(key_idx + ((int64_t)cl0 + c) * K * 8);
  auto tok = [&](int e) { return e < N ? tb + (int)(keys[e] & tmask) : -1; };
#pragma unroll
  for (int s = 0; s < K; ++s) {
    if ((s & (lanes - 1)) != q) continue;
    int4 lo = make_int4(-1, -1, -1, -1), hi = lo;
    if (ids[s] >= 0) {
      const int base = 8 * ids[s];
      lo = make_int4(tok(base), tok(base + 1), tok(base + 2), tok(base + 3));
      hi = make_int4(tok(base + 4), tok(base + 5), tok(base + 6), tok(base + 7));
    }
    krow[2 * s] = lo;
    krow[2 * s + 1] = hi;
  }
}

template <int DIM>
hipError_t build_t(const float* coords, const Geom& geom, int B, int64_t T, int64_t Ct,
                   int grid_side, int k, int32_t* q_idx, int32_t* nbr, int32_t* key_idx,
                   void* ws, hipStream_t st) {
  typedef Space<DIM> S;
  int bits = 0;   // ceil(log2(grid_side)); grid_side is validated
  while ((1 << bits) < grid_side) ++bits;
  const int qbits = DIM == 2 ? 16 : 14;
  const double step = (double)(1u << (qbits - bits));
  Geom g = geom;
  const int N = g.N, C = g.C;   // sizes of the (largest) image
  // 2048 keys per workgroup suffice up to 2048 tokens; 4096 up to kSmallBuild
  g.small_max = N <= 2 * kSmallThreads ? 2 * kSmallThreads : kSmallBuild;
  BuildWorkspace w = build_layout(ws, B, T, Ct, N);
  // images of at most g.small_max tokens: up to 8 workgroups per image
  // share its clusters (each repeats the in-LDS sort), with up to 16 lanes
  // per cluster in the candidate scan
  const bool packed = g.tok_off != nullptr;
  if (N <= g.small_max || packed) {
    const int cs = std::min(C, g.small_max / 8);
    const int parts = std::max(1, std::min(8, (cs + 31) / 32));
    const int cp = (cs + parts - 1) / parts;
    int lanes = 16;
    while (lanes > 1 && lanes * cp > kSmallThreads) lanes >>= 1;
    const bool wide = g.small_max > 2 * kSmallThreads;
    switch (k) {
#define CA_SMALL(KK)                                                                               \
  case KK:                                                                                         \
    if (wide)                                                                                      \
      hipLaunchKernelGGL((build_small_kernel<KK - 1, 4, DIM>), dim3(B, parts), dim3(kSmallThreads), \
                         0, st, coords, g, step, parts, lanes, q_idx, nbr, key_idx);               \
    else                                                                                           \
      hipLaunchKernelGGL((build_small_kernel<KK - 1, 2, DIM>), dim3(B, parts), dim3(kSmallThreads), \
                         0, st, coords, g, step, parts, lanes, q_idx, nbr, key_idx);               \
    break;
      CA_SMALL(1) CA_SMALL(2) CA_SMALL(3) CA_SMALL(4) CA_SMALL(5) CA_SMALL(6) CA_SMALL(7) CA_SMALL(8)
#undef CA_SMALL
      default:
        return hipErrorInvalidValue;
    }
    if (N <= g.small_max) return hipGetLastError();
  }
  // larger images: segment ranks, merge rounds, centroids and boxes, selection
  typedef typename S::Packed P;
  typedef typename S::FCent FC;
  const int segs = (N + kSegSort - 1) / kSegSort;
  hipLaunchKernelGGL(segsort_kernel<DIM>, dim3(B * segs), dim3(kSegThreads), 0, st, coords, g,
                     segs, step, w.keys[0]);
  int cur = 0;
  const dim3 mgrid((N + kRankThreads - 1) / kRankThreads, B);
  for (int run = kSegSort; run < N; run *= 2) {
    const bool last = 2 * run >= N;
    hipLaunchKernelGGL(merge_round_kernel<DIM>, mgrid, dim3(kRankThreads), 0, st, g, run,
                       (const uint64_t*)w.keys[cur], last ? nullptr : w.keys[cur ^ 1], q_idx,
                       (P*)w.qsorted);
    cur ^= 1;
  }
  const dim3 tgrid((C + kBoxTile - 1) / kBoxTile, B);
  hipLaunchKernelGGL(centroid_box_kernel<DIM>, tgrid, dim3(kBoxTile), 0, st, g,
                     (const P*)w.qsorted, (FC*)w.cent, (FC*)w.box, q_idx);
  switch (k) {
#define CA_SEL(KK)                                                                                 \
  case KK:                                                                                         \
    hipLaunchKernelGGL((select_box_kernel<KK - 1, DIM>), tgrid, dim3(kBoxTile * kSelWaves), 0, st, \
                       g, (const FC*)w.cent, (const FC*)w.box, (const int32_t*)q_idx, nbr,         \
                       key_idx);                                                                   \
    break;
    CA_SEL(1) CA_SEL(2) CA_SEL(3) CA_SEL(4) CA_SEL(5) CA_SEL(6) CA_SEL(7) CA_SEL(8)
#undef CA_SEL
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_build_neighbors(const float* coords, const Geom& g, int dims, int B, int64_t T,
                                  int64_t Ct, int grid_side, int k, int32_t* q_idx, int32_t* nbr,
                                  int32_t* key_idx, void* ws, hipStream_t st) {
  if (dims == 2)
    return build_t<2>(coords, g, B, T, Ct, grid_side, k, q_idx, nbr, key_idx, ws, st);
  if (dims == 3)
    return build_t<3>(coords, g, B, T, Ct, grid_side, k, q_idx, nbr, key_idx, ws, st);
  return hipErrorInvalidValue;
}

}  // namespace ca
