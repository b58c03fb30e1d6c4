// Internal helpers shared by the HIP translation units of libclusterattn.
// Not part of the public ABI (see include/cluster_attn.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ca {

// ---- element types -------------------------------------------------------
// bf16 and fp16 travel as the compiler's native __bf16 / _Float16 types;
// conversions to and from float are exact (widening) or round-to-nearest-even
// (narrowing), which is what the outputs promise.
typedef __bf16 bf16;
typedef _Float16 f16;

template <typename T> __device__ __forceinline__ float to_f32(T x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f32(float x) { return (T)x; }

// ---- reverse (key-major) slot list entry ---------------------------------
// One entry per (query cluster i, key cluster j) pair with at least one slot
// of i's list pointing into j: `mult` holds, byte n, how many slots of i hold
// the n-th member of j (0..255; a list has at most 64 slots).
struct RevEntry {
  int32_t i;
  int32_t pad;
  uint64_t mult;
};

// ---- workspace layout of the backward pass --------------------------------
// Two parts: the per-call part (LSE/Delta pairs of pass A, read by pass B)
// and the plan (the transposed slot lists, a function of q_idx and key_idx
// alone, so it can be built once and reused by every backward call on the
// same lists).
struct BwdWorkspace {
  // per call
  float2* ld;        // [B, N, H]   (LSE * log2(e), Delta) per query and head
  float4* ld_none;   // (+inf, 0, +inf, 0): the pair read for an absent query
  // plan
  int32_t* inv;      // [B, N]      token -> position in q_idx (c*cs + m)
  int32_t* cnt;      // [B, C]      entries per key cluster
  int2* seg;         // [B, C]      (start, end) of every key cluster's entries, absolute
  int32_t* cursor;   // [B, C]
  int32_t* nent;     // [B, C]      entries staged per query cluster
  RevEntry* stage;   // [B, C, nk]  entry of the first slot of i pointing into j
  RevEntry* rev;     // [B, C*nk]   per key cluster, sorted by i (image b from b*C*nk)
  int32_t* rtok;     // [B, C*nk, cs] query tokens of entry e (q_idx row of its i)
  size_t bytes;
};

static inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct Carver {
  char* b;
  size_t p = 0;
  void* take(size_t n) {
    size_t at = p;
    p = align_up(p + n, 256);
    return b ? (void*)(b + at) : (void*)nullptr;
  }
};

// the per-call part at `base` (other fields left null)
static inline BwdWorkspace call_layout(void* base, int64_t B, int64_t N, int64_t H) {
  BwdWorkspace w{};
  Carver c{(char*)base};
  w.ld = (float2*)c.take((size_t)(B * N * H) * sizeof(float2));
  w.ld_none = (float4*)c.take(sizeof(float4));
  w.bytes = c.p;
  return w;
}

// the plan at `base` (per-call fields left null)
static inline BwdWorkspace plan_layout(void* base, int64_t B, int64_t N, int64_t C, int64_t nk) {
  BwdWorkspace w{};
  Carver c{(char*)base};
  w.inv = (int32_t*)c.take((size_t)(B * N) * sizeof(int32_t));
  w.cnt = (int32_t*)c.take((size_t)(B * C) * sizeof(int32_t));
  w.seg = (int2*)c.take((size_t)(B * C) * sizeof(int2));
  w.cursor = (int32_t*)c.take((size_t)(B * C) * sizeof(int32_t));
  w.nent = (int32_t*)c.take((size_t)(B * C) * sizeof(int32_t));
  w.stage = (RevEntry*)c.take((size_t)(B * C * nk) * sizeof(RevEntry));
  w.rev = (RevEntry*)c.take((size_t)(B * C * nk) * sizeof(RevEntry));
  w.rtok = (int32_t*)c.take((size_t)(B * C * nk) * 8 * sizeof(int32_t));
  w.bytes = c.p;
  return w;
}

// both parts in one buffer: the per-call part, then the plan
static inline BwdWorkspace bwd_layout(void* base, int64_t B, int64_t N, int64_t H, int64_t C,
                                      int64_t nk) {
  const BwdWorkspace a = call_layout(base, B, N, H);
  BwdWorkspace w = plan_layout(base ? (char*)base + a.bytes : nullptr, B, N, C, nk);
  w.ld = a.ld;
  w.ld_none = a.ld_none;
  w.bytes += a.bytes;
  return w;
}

// ---- workspace layout of the neighbour build ------------------------------
constexpr int kSortChunk = 2048;   // images up to this many tokens: backward plan in LDS
constexpr int kSmallBuild = 4096;  // images up to this many tokens are built in LDS
constexpr int kBoxTile = 64;       // consecutive clusters per bounding box
constexpr int kIdxBits = 19;       // cluster index bits of a (distance, index) key
constexpr int64_t kMaxTokensPerImage = int64_t(8) << kIdxBits;

// Where the images of a batch lie.  Equal-size images (tok_off == nullptr):
// image b holds tokens [b*N, (b+1)*N) and clusters [b*C, (b+1)*C), and the
// lists carry image-local ids.  Packed images of different sizes: the
// device arrays tok_off / clu_off [B+1] give both ranges, and the lists
// carry batch-global ids.  N and C are then the largest image's sizes.
struct Geom {
  const int32_t* tok_off;
  const int32_t* clu_off;
  int N, C;
  int small_max;   // images up to this size are built in LDS, larger ones by segments
  __device__ __forceinline__ void image(int b, int& t0, int& n, int& c0, int& nc) const {
    if (tok_off) {
      t0 = tok_off[b];
      n = tok_off[b + 1] - t0;
      c0 = clu_off[b];
      nc = clu_off[b + 1] - c0;
    } else {
      t0 = b * N;
      n = N;
      c0 = b * C;
      nc = C;
    }
  }
  // base added to the image-local token / cluster ids written out
  __device__ __forceinline__ int tok_base(int t0) const { return tok_off ? t0 : 0; }
  __device__ __forceinline__ int clu_base(int c0) const { return tok_off ? c0 : 0; }
};

// A cluster's centroid is compared through its mean; the integer sums of
// its members' fixed-point coordinates are scaled by L / members, with L the
// least common multiple of the two cluster sizes of the image (8, and
// n mod 8 for the partial last cluster), which makes every centroid L times
// the mean, exactly.  Images whose size is a multiple of 8 keep the plain
// sums (factor 1).  Factors are at most 8 (scaled sums below 2^22).
__host__ __device__ __forceinline__ int mean_scale(int members, int n) {
  const int r = n & 7;
  if (r == 0) return 1;
  const int L = 8 * r / (r & -r);   // lcm(8, r): gcd(8, r) is r's lowest set bit
  return L / members;
}

struct BuildWorkspace {
  void* qsorted;       // [Ct * 8] quantised coordinates in cluster order (<= 8 bytes each)
  uint64_t* keys[2];   // [T]      (code << token bits | token) in sorted runs, two buffers
  void* cent;          // [Ct]     scaled centroid sums (float2 in 2D, float4 in 3D)
  void* box;           // [B, ceil(Cmax / kBoxTile), 2]  per-tile (min, max) centroid vectors
  size_t bytes;
};

// Everything is only needed when some image has more than kSmallBuild
// tokens: T tokens and Ct clusters in the batch, the largest image maxN.
static inline BuildWorkspace build_layout(void* base, int64_t B, int64_t T, int64_t Ct,
                                          int64_t maxN) {
  BuildWorkspace w;
  size_t p = 0;
  char* b = (char*)base;
  auto take = [&](size_t n) {
    size_t at = p;
    p = align_up(p + n, 256);
    return b ? (void*)(b + at) : (void*)nullptr;
  };
  const bool big = maxN > kSmallBuild;
  const int64_t tiles = ((maxN + 7) / 8 + kBoxTile - 1) / kBoxTile;
  // sized for 3D (the larger vectors); 2D uses the front of each part
  w.qsorted = take(big ? (size_t)(Ct * 8) * sizeof(uint64_t) : 0);
  w.keys[0] = (uint64_t*)take(big ? (size_t)T * sizeof(uint64_t) : 0);
  w.keys[1] = (uint64_t*)take(big ? (size_t)T * sizeof(uint64_t) : 0);
  w.cent = take(big ? (size_t)Ct * sizeof(float4) : 0);
  w.box = take(big ? (size_t)(B * tiles * 2) * sizeof(float4) : 0);
  w.bytes = p;
  return w;
}

// ---- spatial buckets of the KNN sampler -----------------------------------
constexpr int kKnnPart = 2048;         // entries per partition of the stable counting sort
constexpr int kKnnSmallTokens = 4096;  // images up to this many tokens are bucketed in LDS

__host__ __device__ inline int knn_ceil_log2(int v) {
  int b = 0;
  while ((1 << b) < v) ++b;
  return b;
}

// Square buckets of 2^bs fixed-point units, Pb = 2^pb to a side: about two
// tokens per bucket, a bucket at least one cell (2^shift units) wide.
struct KnnBuckets {
  int shift, pb, bs, Pb, nb;
};
__host__ __device__ inline KnnBuckets knn_buckets(int N, int G) {
  KnnBuckets g;
  g.shift = 16 - knn_ceil_log2(G);
  g.pb = 0;
  const int half = (N > 1 ? N : 1) / 2;
  while (g.pb < 16 - g.shift && (int64_t(1) << (2 * g.pb + 2)) <= half) ++g.pb;
  g.bs = 16 - g.pb;
  g.Pb = 1 << g.pb;
  g.nb = g.Pb * g.Pb;
  return g;
}
// the largest bucket count of an image of N tokens over every grid side
static inline int64_t knn_max_buckets(int64_t N) {
  int pb = 0;
  const int64_t half = (N > 1 ? N : 1) / 2;
  while (pb < 16 && (int64_t(1) << (2 * pb + 2)) <= half) ++pb;
  return int64_t(1) << (2 * pb);
}

// ---- workspace layout of the KNN table build (images above kKnnSmallTokens)
struct KnnTableWorkspace {
  int32_t* bcnt;    // [B, nb]       tokens per bucket, then placement cursors
  int32_t* bstart;  // [B, nb + 1]   bucket starts
  int32_t* brank;   // [B, N]        rank of each token in its bucket
  uint2* tok;       // [B, N]        (qx | qy << 16, token) in bucket order
  size_t bytes;
};

static inline KnnTableWorkspace knn_table_layout(void* base, int64_t B, int64_t N) {
  KnnTableWorkspace w;
  size_t p = 0;
  char* b = (char*)base;
  auto take = [&](size_t n) {
    size_t at = p;
    p = align_up(p + n, 256);
    return b ? (void*)(b + at) : (void*)nullptr;
  };
  const bool large = N > kKnnSmallTokens;
  const int64_t nb = large ? knn_max_buckets(N) : 0;
  w.bcnt = (int32_t*)take((size_t)(B * nb) * 4);
  w.bstart = (int32_t*)take(large ? (size_t)(B * (nb + 1)) * 4 : 0);
  w.brank = (int32_t*)take(large ? (size_t)(B * N) * 4 : 0);
  w.tok = (uint2*)take(large ? (size_t)(B * N) * 8 : 0);
  w.bytes = p;
  return w;
}

// ---- workspace layout of the KNN sampler backward ---------------------------
// Images up to kKnnSmallTokens tokens sort the entries by token with
// partition counts (pcnt); larger ones place them by per-token cursors into
// lst, rank them inside each token's segment, and bucket the tokens for the
// walk order (the table build's bucket arrays).
// Images above kKnnSmallTokens tokens build the token lists by cursors and
// ranks; smaller ones by the partitioned counting sort (its counts [B, P, N],
// P = M K / kKnnPart, hold at most N / kKnnPart <= 2 ints per entry).
__host__ __device__ inline bool knn_large_lists(int64_t N, int64_t M, int64_t K) {
  (void)M;
  (void)K;
  return N > kKnnSmallTokens;
}

struct KnnWorkspace {
  int32_t* cnt;     // [B, N]        entries per token (then cursors, large images)
  int32_t* off;     // [B, N + 1]    segment starts (per image, relative)
  int32_t* pcnt;    // [B, P, N]     per partition of kKnnPart entries: counts, then prefixes
  int32_t* lst;     // [B, M * K]    (large images, same place as pcnt) entries, unranked
  int32_t* srt;     // [B, M * K]    (large images) sort scratch of the longest segments
  int32_t* slot;    // [B, M, K]     token of every (query, slot), -1 empty
  float* wgt;       // [B, M, K]     its weight
  int2* ent;        // [B, M * K]    (query, weight bits) of the entries, by token
  float* dpart;     // [B, M]        per-query share of dL/dp
  int32_t* order;   // [B, N]        walk order of the tokens (feature gradient)
  KnnTableWorkspace bk;   // large images: bucket arrays of the walk order
  size_t bytes;
};

static inline KnnWorkspace knn_layout(void* base, int64_t B, int64_t N, int64_t M, int64_t K) {
  KnnWorkspace w;
  size_t p = 0;
  char* b = (char*)base;
  auto take = [&](size_t n) {
    size_t at = p;
    p = align_up(p + n, 256);
    return b ? (void*)(b + at) : (void*)nullptr;
  };
  const bool large = knn_large_lists(N, M, K);
  w.cnt = (int32_t*)take((size_t)(B * N) * 4);
  w.off = (int32_t*)take((size_t)(B * (N + 1)) * 4);
  const int64_t P = (M * K + kKnnPart - 1) / kKnnPart;
  w.pcnt = (int32_t*)take(large ? (size_t)(B * M * K) * 4 : (size_t)(B * P * N) * 4);
  w.lst = w.pcnt;
  w.srt = (int32_t*)take(large ? (size_t)(B * M * K) * 4 : 0);
  w.slot = (int32_t*)take((size_t)(B * M * K) * 4);
  w.wgt = (float*)take((size_t)(B * M * K) * 4);
  w.ent = (int2*)take((size_t)(B * M * K) * 8);
  w.dpart = (float*)take((size_t)(B * M) * 4);
  w.order = (int32_t*)take((size_t)(B * N) * 4);
  // large lists: bucket arrays for the walk order (sized as the table
  // build's for an image above kKnnSmallTokens tokens)
  const int64_t nbk = large ? knn_max_buckets(N) : 0;
  w.bk.bcnt = (int32_t*)take((size_t)(B * nbk) * 4);
  w.bk.bstart = (int32_t*)take(large ? (size_t)(B * (nbk + 1)) * 4 : 0);
  w.bk.brank = (int32_t*)take(large ? (size_t)(B * N) * 4 : 0);
  w.bk.tok = nullptr;
  w.bk.bytes = 0;
  w.bytes = p;
  return w;
}

// ---- workspace layout of the merge plan (images above kMergeSmallTokens) ---
constexpr int kMergeSmallTokens = 4096;   // images up to this many tokens are planned in LDS

// anchor buckets of the large-image plan: squares of 2^bsh fixed-point
// units, Pb = 2^pb to a side, about two anchors per bucket
struct MergeBuckets {
  int pb, bsh, Pb, nb;
};
__host__ __device__ inline MergeBuckets merge_buckets(int k) {
  MergeBuckets g;
  g.pb = 0;
  const int half = (k > 1 ? k : 1) / 2;
  while (g.pb < 15 && (int64_t(1) << (2 * g.pb + 2)) <= half) ++g.pb;
  g.bsh = 16 - g.pb;
  g.Pb = 1 << g.pb;
  g.nb = g.Pb * g.Pb;
  return g;
}

constexpr int kMergeSelChunk = 4096;      // tokens per chunk of the anchor placement

struct MergeWorkspace {
  uint32_t* sk;     // [B, N]        order-preserving keys of the scores
  uint2* sel;       // [B]           (k-th largest key, how many keys equal to it are taken)
  int2* chunk;      // [B, nch]      keys above / equal to the k-th before each chunk
  int32_t* apos;    // [B, N]        anchor position of every token, -1 if none
  int32_t* abcnt;   // [B, nb]       anchors per bucket
  int32_t* abstart; // [B, nb + 1]   bucket starts
  int32_t* abrank;  // [B, k]        rank of each anchor in its bucket
  uint2* abk;       // [B, k]        (qx | qy << 16, position) in bucket order
  int32_t* gcnt;    // [B, k]        group sizes
  int32_t* gcur;    // [B, k]        placement cursors
  int32_t* glst;    // [B, N]        members in placement order
  int32_t* gtmp;    // [B, N]        sort scratch of the largest groups
  size_t bytes;
};

static inline MergeWorkspace merge_layout(void* base, int64_t B, int64_t N, int64_t k) {
  MergeWorkspace w;
  size_t p = 0;
  char* b = (char*)base;
  auto take = [&](size_t n) {
    size_t at = p;
    p = align_up(p + n, 256);
    return b ? (void*)(b + at) : (void*)nullptr;
  };
  const bool large = N > kMergeSmallTokens;
  const int64_t nb = large ? merge_buckets((int)k).nb : 0;
  const int64_t n = large ? N : 0, kk = large ? k : 0;
  const int64_t nch = large ? (N + kMergeSelChunk - 1) / kMergeSelChunk : 0;
  w.sk = (uint32_t*)take((size_t)(B * n) * 4);
  w.sel = (uint2*)take(large ? (size_t)B * 8 : 0);
  w.chunk = (int2*)take((size_t)(B * nch) * 8);
  w.apos = (int32_t*)take((size_t)(B * n) * 4);
  w.abcnt = (int32_t*)take((size_t)(B * nb) * 4);
  w.abstart = (int32_t*)take(large ? (size_t)(B * (nb + 1)) * 4 : 0);
  w.abrank = (int32_t*)take((size_t)(B * kk) * 4);
  w.abk = (uint2*)take((size_t)(B * kk) * 8);
  w.gcnt = (int32_t*)take((size_t)(B * kk) * 4);
  w.gcur = (int32_t*)take((size_t)(B * kk) * 4);
  w.glst = (int32_t*)take((size_t)(B * n) * 4);
  w.gtmp = (int32_t*)take((size_t)(B * n) * 4);
  w.bytes = p;
  return w;
}

// ---- wave helpers (64-lane wavefronts) ------------------------------------
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// Inclusive prefix sum across the 64 lanes of a wavefront.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(v, o, 64);
    if (lane >= o) v += y;
  }
  return v;
}

// Exclusive prefix sum of one value per thread over a workgroup of
// `nthreads` (a multiple of 64, at most 1024) with two barriers; `tmp` is
// 16 ints of LDS.  Returns the exclusive prefix and writes the total.
__device__ __forceinline__ int block_exclusive_scan(int v, int* tmp, int nthreads, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int inc = wave_inclusive_scan(v);
  if (lane == 63) tmp[w] = inc;
  __syncthreads();
  if (w == 0) {
    const int nw = nthreads >> 6;
    const int t = lane < nw ? tmp[lane] : 0;
    const int ti = wave_inclusive_scan(t);
    if (lane < nw) tmp[lane] = ti - t;
    if (lane == nw - 1) tmp[16 + 0] = ti;
  }
  __syncthreads();
  *total = tmp[16];
  return tmp[w] + inc - v;
}

// Workgroup w of n is dispatched to XCD w % 8; this numbering gives XCD x a
// contiguous range of n/8 workgroups (their data then shares that XCD's L2).
__device__ __forceinline__ int xcd_remap(int w, int n) {
  // dispatch sends workgroup w to XCD w % 8; give XCD x a contiguous range
  const int x = w & 7, i = w >> 3;
  const int q = n >> 3, r = n & 7;
  return x * q + min(x, r) + i;
}

// 16-bit fixed-point coordinate of one axis: clamp(floor((c + 0.5) * step),
// 0, 65535), step = 2^(16 - ceil(log2 G)) (shared by the neighbour build and
// the KNN table).
__device__ __forceinline__ uint32_t quantize_axis(float c, double step) {
  // (c + 0.5) and the power-of-two step are exact in fp64, so this equals
  // floor((c + 0.5) * step) of the real numbers.
  double q = floor(((double)c + 0.5) * step);
  q = q < 0.0 ? 0.0 : (q > 65535.0 ? 65535.0 : q);
  return (uint32_t)q;
}

// ---- launchers (defined in the .hip files) ---------------------------------
// Attention launchers take B images of N tokens and C clusters each (q_idx
// [B, C, 8], C = ceil(N / 8)); a packed batch runs as one image (B = 1) of
// all T tokens and Ct clusters with batch-global ids.
// dims = 2: coords [.., 2] (16-bit fixed point per axis); dims = 3: coords
// [.., 3] (14-bit fixed point per axis).
hipError_t launch_build_neighbors(const float* coords, const Geom& g, int dims, int B, int64_t T,
                                  int64_t Ct, int grid_side, int k, int32_t* q_idx, int32_t* nbr,
                                  int32_t* key_idx, void* ws, hipStream_t st);

hipError_t launch_fwd_valu(int dt, int B, int N, int C, int H, int nk, float scale, const void* q,
                           const void* k, const void* v, const int32_t* q_idx,
                           const int32_t* key_idx, void* o, float* lse, hipStream_t st);

// `packed` (optional): the images of a packed batch (B images, N = T tokens,
// C = Ct clusters in total; packed->N the largest image), planned one
// workgroup per image when every image fits in LDS.
hipError_t launch_bwd_plan(int B, int N, int C, int nk, const int32_t* q_idx,
                           const int32_t* key_idx, const BwdWorkspace& w, hipStream_t st,
                           const Geom* packed = nullptr);

// Backward launchers: pass bit 1 = pass A (Delta, dQ; needs nothing from the
// plan), bit 2 = pass B (dK, dV; needs pass A and the plan).
hipError_t launch_bwd_valu(int pass, int dt, int B, int N, int C, int H, int nk, float scale,
                           const void* q, const void* k, const void* v, const void* o,
                           const void* dout, const float* lse, const int32_t* q_idx,
                           const int32_t* key_idx, void* dq, void* dk, void* dv,
                           const BwdWorkspace& w, hipStream_t st);

bool mfma_supported(int dt, int B, int N, int C, int H, int nk);

hipError_t launch_fwd_mfma(int dt, int B, int N, int C, int H, float scale, const void* q,
                           const void* k, const void* v, const int32_t* q_idx,
                           const int32_t* key_idx, void* o, float* lse, hipStream_t st);

hipError_t launch_bwd_mfma(int pass, int dt, int B, int N, int C, int H, int nk, float scale,
                           const void* q, const void* k, const void* v, const void* o,
                           const void* dout, const float* lse, const int32_t* q_idx,
                           const int32_t* key_idx, void* dq, void* dk, void* dv,
                           const BwdWorkspace& w, hipStream_t st);

// Integer helpers (scan.hip): x[0..n) = 0; per segment s of n counts,
// off[s, 0..n] = exclusive prefix sums and the total (off has n + 1 entries
// per segment)
void launch_zero_i32(int64_t n, int32_t* x, hipStream_t st);
void launch_segment_scan(int segments, int n, const int32_t* cnt, int32_t* off, hipStream_t st);
// Segments longer than kLongSegment of a segmented list (B images of S
// segments; segment s of image b is vals[b * stride + off[b * (S + 1) + s] ..
// off[... + 1]), values in [0, max_value]) sorted stably by value into out
// (or, with out2, as (value / K, bits of wgt[b * stride + value]) pairs);
// tmp: scratch of vals' layout.  Shorter segments are left alone (their
// rank kernels handle them).
constexpr int kLongSegment = 256;
void launch_long_segment_sort(int B, int S, int64_t stride, int64_t max_value, const int32_t* off,
                              int32_t* vals, int32_t* tmp, int32_t* out, int2* out2, int K,
                              const float* wgt, hipStream_t st);

// KNN-cache point sampler (knn_sampler.hip)
hipError_t launch_knn_table(const float* coords, int B, int N, int G, int K, int32_t* table, void* ws,
                            hipStream_t st);
hipError_t launch_knn_fwd(int dt, int B, int N, int M, int Cf, int G, int K, float p,
                          const float* coords, const void* feats, const float* queries,
                          const int32_t* table, void* out, hipStream_t st);
hipError_t launch_knn_bwd(int dt, int B, int N, int M, int Cf, int G, int K, float p,
                          const float* coords, const void* feats, const float* queries,
                          const int32_t* table, const void* dout, void* dfeat, float* dq,
                          float* dp, void* ws, hipStream_t st);

// Adaptive token merging (token_merge.hip)
hipError_t launch_merge_plan(const float* coords, const float* scores, int B, int N, int k, int G,
                             int32_t* anchors, int32_t* assign, int32_t* members,
                             int32_t* offsets, void* ws, hipStream_t st);
hipError_t launch_merge_fwd(int dt, int B, int N, int k, int Cf, const void* feats,
                            const float* coords, const float* scores, const int32_t* members,
                            const int32_t* offsets, void* out_f, float* out_x, hipStream_t st);
hipError_t launch_merge_bwd(int dt, int B, int N, int k, int Cf, const void* feats,
                            const float* coords, const float* scores, const int32_t* members,
                            const int32_t* offsets, const void* dout_f, const float* dout_x,
                            void* dfeats, float* dcoords, float* dscores, hipStream_t st);

}  // namespace ca
