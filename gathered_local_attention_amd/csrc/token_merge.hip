// Adaptive off-grid token merging on gfx950.
//
// Source: English notes page "AFFMAE: Scalable Vision Pre-Training for
// High-Resolution Microscopy Segmentation on Desktop Hardware", "Key Designs"
// item 1 (adaptive off-grid token merging: every token keeps its 2D
// coordinate; a lightweight MLP scores the tokens, the top-k by the
// retention rate become anchors, and the other tokens are merged,
// differentiably, into their nearest anchors, features and spatial support
// alike).  The library's readings of what the page leaves open:
//   scores    an input (the scoring MLP is outside); k given by the caller;
//   anchors   the k largest scores, ties to the lower token index, listed in
//             ascending token index;
//   assign    an anchor to itself, any other token to the anchor nearest by
//             squared distance of the 16-bit fixed-point coordinates (the
//             neighbour build's quantisation), ties to the earlier anchor;
//   merge     within a group the softmax of the members' scores weighs
//             features and coordinates: F'_a = sum w_i F_i, X'_a = sum w_i X_i;
//   backward  gradients of F, X and the scores (anchors, assignment fixed).
//
// Kernels:
//   merge_assign_kernel  up to 8 workgroups per image (up to 4096 tokens,
//                      all in LDS; each workgroup repeats the selection):
//                      top-k by a radix select of the score keys, anchors
//                      by a workgroup scan in token order, and for its slice
//                      of the tokens the nearest anchor by a ring search over
//                      a bucket grid of the anchors (exact int64 keys).
//   merge_members_kernel one workgroup per image: the groups' member lists
//                      by a counting sort on the anchor, each group then
//                      sorted by token index.
//   merge_select/abucket/assign_wide/g* kernels  the same plan for images
//                      above 4096 tokens, in global memory (a workspace).
//   merge_fwd_kernel   a lane group per anchor (16 bytes of the row per
//                      lane): the group's softmax, then the weighted sums.
//   merge_bwd_kernel   the same groups: g_i = <dF'_a, F_i> + <dX'_a, X_i>
//                      (group reductions), dF_i = w_i dF'_a, dX_i = w_i dX'_a,
//                      ds_i = w_i (g_i - sum_j w_j g_j); every token written
//                      once (it belongs to one group): no atomics.
#include "common.h"

#include <algorithm>

namespace ca {

namespace {

constexpr int kPlanT = 1024;
constexpr int kMaxTok = kMergeSmallTokens;
constexpr int kMergeThreads = 256;
constexpr int kRingLanes = 4;   // lanes per token in the nearest-anchor search

typedef float mf32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 mbf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 mf16x8 __attribute__((ext_vector_type(8)));

// 16 bytes of a row as floats (exact widening; RNE narrowing on store)
template <typename T> struct Row16;
template <> struct Row16<float> {
  static constexpr int E = 4;
  static constexpr int NR = 4;   // chunks per lane at most (1024 channels, 64 lanes)
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
template <typename H, typename V> struct Row16Half {
  static constexpr int E = 8;
  static constexpr int NR = 2;   // chunks per lane at most (1024 channels, 64 lanes)
  __device__ static uint4 raw(const H* p) { return *reinterpret_cast<const uint4*>(p); }
  __device__ static void cvt(uint4 a, float* v) {
    const mf32x8 f = __builtin_convertvector(__builtin_bit_cast(V, a), mf32x8);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = f[e];
  }
  __device__ static void load(const H* p, float* v) {
    const mf32x8 f = __builtin_convertvector(__builtin_bit_cast(V, *reinterpret_cast<const uint4*>(p)), mf32x8);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = f[e];
  }
  __device__ static void store(H* p, const float* v) {
    const mf32x8 f = {v[0], v[1], v[2], v[3], v[4], v[5], v[6], v[7]};
    *reinterpret_cast<uint4*>(p) = __builtin_bit_cast(uint4, __builtin_convertvector(f, V));
  }
};
template <> struct Row16<bf16> : Row16Half<bf16, mbf16x8> {};
template <> struct Row16<f16> : Row16Half<f16, mf16x8> {};


// ---------------------------------------------------------------------------
// Plan: anchors, assignment, member lists.  Assignment grid = B x S
// workgroups of 1024 threads, the image in LDS:
//  1. top-k by a radix select on order-preserving 32-bit keys of the scores
//     (8-bit digits from the top): the k-th largest key, then the tokens
//     above it and the first ones (in token order) equal to it;
//  2. anchor positions by a workgroup scan in token order;
//  3. the anchors bucketed on a coarse grid (about two per bucket); every
//     other token of the workgroup's slice searches rings of buckets around
//     its own until its best is strictly closer than anything outside the
//     searched window can be;
//  4. (members kernel) member lists by a counting sort on the anchor (LDS
//     atomics), each group's members then sorted by token index.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t score_key(float x) {
  // larger float -> larger key; -0 and +0 share one key (they compare equal)
  const uint32_t u = __float_as_uint(x == 0.f ? 0.f : x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Radix select of the k-th largest of the keys sk[0..N) by 8-bit digits
// from the top, called by every thread of a kPlanT workgroup (sk in LDS or
// in global memory, written before the call and visible to the workgroup).
// On return sel[0] is the k-th largest key and sel[1] the number of keys
// equal to it that belong to the k largest (the first ones in token order).
__device__ __forceinline__ void radix_select(const uint32_t* sk, int N, int k, int* hist,
                                             uint32_t* sel) {
  const int tid = threadIdx.x;
  if (tid == 0) {
    sel[0] = 0u;
    sel[1] = (uint32_t)k;
  }
  for (int dg = 3; dg >= 0; --dg) {
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    const uint32_t pre = sel[0];
    const uint32_t hmask = dg == 3 ? 0u : (0xFFFFFFFFu << (8 * (dg + 1)));
    for (int i0 = tid; i0 < N; i0 += kPlanT * 8) {   // eight keys in flight
      uint32_t kv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) kv[u] = i0 + u * kPlanT < N ? sk[i0 + u * kPlanT] : 0u;
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (i0 + u * kPlanT < N && (kv[u] & hmask) == pre) atomicAdd(&hist[(kv[u] >> (8 * dg)) & 255u], 1);
    }
    __syncthreads();
    if (tid < 64) {
      // the digit where the count from the top reaches `want`: lane l holds
      // bins 255 - 4l .. 252 - 4l, a wave scan gives the counts above them
      const uint32_t want = sel[1];
      int h[4];
      int sum = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        h[j] = hist[255 - 4 * tid - j];
        sum += h[j];
      }
      const int incl = wave_inclusive_scan(sum);
      int cum = incl - sum;
      if ((uint32_t)cum < want && (uint32_t)incl >= want) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if ((uint32_t)(cum + h[j]) >= want) {
            sel[0] = pre | ((uint32_t)(255 - 4 * tid - j) << (8 * dg));
            sel[1] = want - (uint32_t)cum;
            break;
          }
          cum += h[j];
        }
      }
    }
    __syncthreads();
  }
}

__global__ void __launch_bounds__(kPlanT)
merge_assign_kernel(const float* __restrict__ coords, const float* __restrict__ scores, int N,
                    int k, int G, int S, int32_t* __restrict__ anchors,
                    int32_t* __restrict__ assign) {
  __shared__ uint32_t sk[kMaxTok];                    // score keys
  __shared__ uint32_t qc[kMaxTok];                    // token fixed-point (qx | qy << 16)
  __shared__ int32_t apos[kMaxTok];                   // token -> anchor position, or -1
  __shared__ uint2 abk[kMaxTok];                      // anchors in bucket order: (qc, position)
  __shared__ int32_t bstart[kMaxTok];                 // bucket starts (<= 4096 buckets)
  __shared__ int hist[256];
  __shared__ uint32_t sel[2];                         // selected prefix, still wanted
  __shared__ int tmp[17];
  const int b = blockIdx.x / S, slice = blockIdx.x % S, tid = threadIdx.x;
  const int bits = [&] { int v = 0; while ((1 << v) < G) ++v; return v; }();
  const double step = (double)(1u << (16 - bits));
  const float* s = scores + (int64_t)b * N;
  const float2* xy = reinterpret_cast<const float2*>(coords) + (int64_t)b * N;
  for (int i = tid; i < N; i += kPlanT) {
    sk[i] = score_key(s[i]);
    const float2 c = xy[i];
    qc[i] = quantize_axis(c.x, step) | (quantize_axis(c.y, step) << 16);
  }
  // 1. radix select of the k-th largest key
  radix_select(sk, N, k, hist, sel);
  const uint32_t kth = sel[0], n_eq = sel[1];   // take n_eq of the keys equal to kth
  // 2. flags in token order (thread t owns tokens 4t .. 4t+3), then positions
  //    (one scan of the packed counts of keys above and equal to the k-th:
  //    the anchors before a thread's tokens are the larger keys before them
  //    and the first n_eq equal keys in token order)
  constexpr int R = kMaxTok / kPlanT;
  int gt_local = 0, eq_local = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int i = tid * R + r;
    gt_local += (i < N && sk[i] > kth) ? 1 : 0;
    eq_local += (i < N && sk[i] == kth) ? 1 : 0;
  }
  int tot;
  const int ex = block_exclusive_scan((gt_local << 16) | eq_local, tmp, kPlanT, &tot);
  int eq_before = ex & 0xFFFF;
  int pos = (ex >> 16) + min(eq_before, (int)n_eq);
  bool an[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int i = tid * R + r;
    an[r] = false;
    if (i < N) {
      if (sk[i] > kth) an[r] = true;
      else if (sk[i] == kth) an[r] = (uint32_t)(eq_before++) < n_eq;
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int i = tid * R + r;
    if (i < N) {
      apos[i] = an[r] ? pos : -1;
      if (an[r] && slice == 0) anchors[(int64_t)b * k + pos] = i;
      pos += an[r] ? 1 : 0;
    }
  }
  // 3. anchors bucketed: side 2^bsh fixed-point units, about two per bucket
  int pb = 0;
  while (pb < 6 && (1 << (2 * pb + 2)) <= max(k, 1) / 2) ++pb;
  const int bsh = 16 - pb, Pb = 1 << pb, nb = Pb * Pb;
  for (int x = tid; x < nb; x += kPlanT) bstart[x] = 0;
  __syncthreads();
  int abkt[R], arank[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int i = tid * R + r;
    abkt[r] = -1;
    if (i < N && an[r]) {
      const uint32_t q = qc[i];
      abkt[r] = (int)(((q >> 16) >> bsh) * (uint32_t)Pb + ((q & 0xFFFFu) >> bsh));
      arank[r] = atomicAdd(&bstart[abkt[r]], 1);
    }
  }
  __syncthreads();
  int cnt[R];
  int run = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int x = tid * R + r;
    cnt[r] = x < nb ? bstart[x] : 0;
    run += cnt[r];
  }
  __syncthreads();
  int acc = block_exclusive_scan(run, tmp, kPlanT, &tot);
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int x = tid * R + r;
    if (x < nb) bstart[x] = acc;
    acc += cnt[r];
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int i = tid * R + r;
    if (abkt[r] >= 0) abk[bstart[abkt[r]] + arank[r]] = make_uint2(qc[i], (uint32_t)apos[i]);
  }
  __syncthreads();
  // nearest anchor of the slice's tokens: rings of buckets around its own,
  // kRingLanes lanes per token sharing each ring's buckets (group minimum
  // after every ring, so the stop test is the same on all of them); keys
  // (d2 << 12 | position) exact in 64 bits
  const int per = (N + S - 1) / S, i0 = slice * per, i1 = min(N, i0 + per);
  const int u = tid % kRingLanes;
  for (int i = i0 + tid / kRingLanes; i < i1; i += kPlanT / kRingLanes) {
    int a = apos[i];
    if (a < 0) {
      const uint32_t q = qc[i];
      const int64_t x = q & 0xFFFFu, y = q >> 16;
      const int bx0 = (int)(x >> bsh), by0 = (int)(y >> bsh);
      uint64_t best = ~0ull;
      for (int Rg = 0; Rg < Pb; ++Rg) {
        const int y0 = by0 - Rg, y1 = by0 + Rg, x0 = bx0 - Rg, x1 = bx0 + Rg;
        // ring Rg holds 8 Rg buckets (one for Rg = 0): the top row, the
        // bottom row, then the two side columns alternately
        const int nring = Rg == 0 ? 1 : 8 * Rg, w = 2 * Rg + 1;
        for (int j = u; j < nring; j += kRingLanes) {
          int by, bx;
          if (j < w) {
            by = y0;
            bx = x0 + j;
          } else if (j < 2 * w) {
            by = y1;
            bx = x0 + j - w;
          } else {
            const int m = j - 2 * w;
            by = y0 + 1 + (m >> 1);
            bx = (m & 1) ? x1 : x0;
          }
          if (bx < 0 || bx >= Pb || by < 0 || by >= Pb) continue;
          const int bb = by * Pb + bx;
          const int t0 = bstart[bb], t1 = bb + 1 < nb ? bstart[bb + 1] : k;
          for (int t = t0; t < t1; ++t) {
            const uint2 e = abk[t];
            const int64_t ix = (int64_t)(e.x & 0xFFFFu) - x, iy = (int64_t)(e.x >> 16) - y;
            const uint64_t kk = ((uint64_t)(ix * ix + iy * iy) << 12) | e.y;
            best = kk < best ? kk : best;
          }
        }
#pragma unroll
        for (int m = 1; m < kRingLanes; m <<= 1) {
          const uint64_t o = ((uint64_t)(uint32_t)__shfl_xor((int)(best >> 32), m) << 32) |
                             (uint32_t)__shfl_xor((int)(uint32_t)best, m);
          best = o < best ? o : best;
        }
        // a token outside the searched window lies beyond one of its edges
        int64_t lb = INT64_MAX;
        if (y0 > 0) lb = min(lb, y - ((int64_t)y0 << bsh) + 1);
        if (y1 < Pb - 1) lb = min(lb, ((int64_t)(y1 + 1) << bsh) - y);
        if (x0 > 0) lb = min(lb, x - ((int64_t)x0 << bsh) + 1);
        if (x1 < Pb - 1) lb = min(lb, ((int64_t)(x1 + 1) << bsh) - x);
        if (best != ~0ull && (lb == INT64_MAX || (int64_t)(best >> 12) < lb * lb)) break;
      }
      a = (int)(best & 0xFFFu);
    }
    if (u == 0) assign[(int64_t)b * N + i] = a;
  }
}

// Member lists of every image from the assignment.  grid = B, 1024 threads:
// group sizes by LDS counters, group starts by a scan, members placed in
// arrival order, then every group's members sorted by token index (a thread
// per group when no group exceeds 32 tokens, else a bitonic sort of all the
// (group, token) keys).
__global__ void __launch_bounds__(kPlanT)
merge_members_kernel(int N, int k, const int32_t* __restrict__ assign,
                     int32_t* __restrict__ members, int32_t* __restrict__ offsets) {
  __shared__ uint32_t key[kMaxTok];                   // group counts, then sort keys
  __shared__ int32_t gstart[kMaxTok];
  __shared__ uint32_t tok[kMaxTok];
  __shared__ int tmp[17];
  constexpr int R = kMaxTok / kPlanT;
  const int b = blockIdx.x, tid = threadIdx.x;
  for (int x = tid; x < k; x += kPlanT) key[x] = 0u;
  __syncthreads();
  int ga[R], gslot[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int i = tid + r * kPlanT;
    ga[r] = -1;
    if (i < N) {
      ga[r] = assign[(int64_t)b * N + i];
      gslot[r] = (int)atomicAdd(&key[ga[r]], 1u);   // arrival order; fixed by the sort below
    }
  }
  __syncthreads();
  int gc[R];
  int grun = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int x = tid * R + r;
    gc[r] = x < k ? (int)key[x] : 0;
    grun += gc[r];
  }
  __syncthreads();
  int tot;
  int gacc = block_exclusive_scan(grun, tmp, kPlanT, &tot);
  int32_t* off = offsets + (int64_t)b * (k + 1);
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int x = tid * R + r;
    if (x < k) {
      gstart[x] = gacc;
      off[x] = gacc;
    }
    gacc += gc[r];
  }
  if (tid == 0) off[k] = N;
  __syncthreads();
#pragma unroll
  for (int r = 0; r < R; ++r)
    if (ga[r] >= 0) tok[gstart[ga[r]] + gslot[r]] = (uint32_t)(tid + r * kPlanT);
  __syncthreads();
  int32_t* mem = members + (int64_t)b * N;
  int gmax = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) gmax = max(gmax, gc[r]);
  if (__syncthreads_or(gmax > 32)) {
    // some group is large: bitonic sort of all (group << 12 | token) keys
    int P2 = 1;
    while (P2 < N) P2 <<= 1;
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (ga[r] >= 0) key[tid + r * kPlanT] = ((uint32_t)ga[r] << 12) | (uint32_t)(tid + r * kPlanT);
    for (int i = N + tid; i < P2; i += kPlanT) key[i] = 0xFFFFFFFFu;
    __syncthreads();
    for (int kk = 2; kk <= P2; kk <<= 1) {
      for (int j = kk >> 1; j > 0; j >>= 1) {
        for (int i = tid; i < P2 / 2; i += kPlanT) {
          const int lo = ((i & ~(j - 1)) << 1) | (i & (j - 1));
          const uint32_t xk = key[lo], yk = key[lo + j];
          if ((xk > yk) == ((lo & kk) == 0)) {
            key[lo] = yk;
            key[lo + j] = xk;
          }
        }
        __syncthreads();
      }
    }
    for (int i = tid; i < N; i += kPlanT) mem[i] = (int32_t)(key[i] & 0xFFFu);
    return;
  }
  for (int g = tid; g < k; g += kPlanT) {
    const int g0 = gstart[g], g1 = g + 1 < k ? gstart[g + 1] : N;
    for (int u = g0 + 1; u < g1; ++u) {   // insertion sort of at most 32 tokens
      const uint32_t v = tok[u];
      int y = u - 1;
      while (y >= g0 && tok[y] > v) {
        tok[y + 1] = tok[y];
        --y;
      }
      tok[y + 1] = v;
    }
    for (int u = g0; u < g1; ++u) mem[u] = (int32_t)tok[u];
  }
}

// ---------------------------------------------------------------------------
// Plan of images above kMaxTok tokens, in global memory (workspace):
//  1. merge_select_kernel, one workgroup per image: the score keys, their
//     radix select and the counts of keys above / equal to the selected one
//     before every chunk of tokens; merge_flag_kernel, a workgroup per
//     chunk: anchor flags and positions in token order;
//  2. the anchors counting-sorted into square buckets (merge_buckets);
//  3. merge_assign_wide_kernel: kRingLanes lanes per token, the ring search
//     of the small-image kernel over the global bucket arrays;
//  4. member lists: group sizes (integer atomics, in the assignment kernel),
//     offsets by a scan, every
//     token placed by its group's cursor (in no fixed order), then moved to
//     group start + its rank by token index inside the group (groups of
//     more than kLongSegment members sorted by launch_long_segment_sort).
// Keys (d2 << 24 | anchor position) are exact for k < 2^24.
// ---------------------------------------------------------------------------
constexpr int kWideKeyBits = 24;

// 1a. one workgroup per image: the score keys and their radix select, then
// per chunk of kMergeSelChunk tokens the counts of keys above and equal to
// the k-th one (a wave per chunk), turned into exclusive prefixes over the
// chunks; the image's bucket and group counters are zeroed here too
__global__ void __launch_bounds__(kPlanT)
merge_select_kernel(const float* __restrict__ scores, int N, int k, int nb, int nch,
                    uint32_t* __restrict__ sk_all, uint2* __restrict__ sel_all,
                    int2* __restrict__ chunk_all, int32_t* __restrict__ abcnt,
                    int32_t* __restrict__ gcnt, int32_t* __restrict__ gcur) {
  __shared__ int hist[256];
  __shared__ uint32_t sel[2];
  __shared__ int tmp[17];
  __shared__ int2 ccnt[1024];
  const int64_t b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const float* s = scores + b * N;
  uint32_t* sk = sk_all + b * N;
  for (int i = tid; i < N; i += kPlanT) sk[i] = score_key(s[i]);
  for (int i = tid; i < nb; i += kPlanT) abcnt[b * nb + i] = 0;
  for (int i = tid; i < k; i += kPlanT) {
    gcnt[b * k + i] = 0;
    gcur[b * k + i] = 0;
  }
  radix_select(sk, N, k, hist, sel);
  const uint32_t kth = sel[0], n_eq = sel[1];
  if (tid == 0) sel_all[b] = make_uint2(kth, n_eq);
  int carry_gt = 0, carry_eq = 0;
  for (int c0 = 0; c0 < nch; c0 += 1024) {   // up to 1024 chunks per round
    for (int c = c0 + wv; c < min(nch, c0 + 1024); c += kPlanT / 64) {
      int gt = 0, eq = 0;
      const int t0 = c * kMergeSelChunk, t1 = min(N, t0 + kMergeSelChunk);
      for (int i0 = t0 + lane; i0 < t1; i0 += 64 * 8) {
        uint32_t kv[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) kv[u] = i0 + u * 64 < t1 ? sk[i0 + u * 64] : 0u;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const bool in = i0 + u * 64 < t1;
          gt += (in && kv[u] > kth) ? 1 : 0;
          eq += (in && kv[u] == kth) ? 1 : 0;
        }
      }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        gt += __shfl_xor(gt, o, 64);
        eq += __shfl_xor(eq, o, 64);
      }
      if (lane == 0) ccnt[c - c0] = make_int2(gt, eq);
    }
    __syncthreads();
    const bool have = c0 + tid < nch;
    const int2 mine = have ? ccnt[tid] : make_int2(0, 0);
    int tg, te;
    const int pg = block_exclusive_scan(mine.x, tmp, kPlanT, &tg);
    __syncthreads();
    const int pe = block_exclusive_scan(mine.y, tmp, kPlanT, &te);
    if (have) chunk_all[b * nch + c0 + tid] = make_int2(carry_gt + pg, carry_eq + pe);
    carry_gt += tg;
    carry_eq += te;
    __syncthreads();
  }
}

// 1b. grid B x nch: the anchors of one chunk, by a workgroup scan of its
// keys in token order from the chunk's prefixes (thread t owns 4 tokens)
__global__ void __launch_bounds__(kPlanT)
merge_flag_kernel(int N, int k, int nch, const uint32_t* __restrict__ sk_all,
                  const uint2* __restrict__ sel_all, const int2* __restrict__ chunk_all,
                  int32_t* __restrict__ apos_all, int32_t* __restrict__ anchors) {
  static_assert(kMergeSelChunk == kPlanT * 4, "four tokens per thread");
  __shared__ int tmp[17];
  const int64_t b = blockIdx.x / nch;
  const int c = (int)(blockIdx.x - b * nch), tid = threadIdx.x;
  const uint2 sl = sel_all[b];
  const uint32_t kth = sl.x, n_eq = sl.y;
  const int2 pre = chunk_all[b * nch + c];
  const uint32_t* sk = sk_all + b * N;
  int32_t* apos = apos_all + b * N;
  constexpr int R = 4;
  const int base = c * kMergeSelChunk + tid * R;
  uint32_t kv[R];
  int gt_local = 0, eq_local = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int i = base + r;
    kv[r] = i < N ? sk[i] : 0u;
    gt_local += (i < N && kv[r] > kth) ? 1 : 0;
    eq_local += (i < N && kv[r] == kth) ? 1 : 0;
  }
  int tot;
  const int ex = block_exclusive_scan((gt_local << 16) | eq_local, tmp, kPlanT, &tot);
  int eq_before = pre.y + (ex & 0xFFFF);
  int pos = pre.x + (ex >> 16) + min(eq_before, (int)n_eq);
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int i = base + r;
    if (i < N) {
      bool an = false;
      if (kv[r] > kth) an = true;
      else if (kv[r] == kth) an = (uint32_t)(eq_before++) < n_eq;
      apos[i] = an ? pos : -1;
      if (an) anchors[b * k + pos] = i;
      pos += an ? 1 : 0;
    }
  }
}

__device__ __forceinline__ uint32_t fixed_point(const float2 c, double step) {
  return quantize_axis(c.x, step) | (quantize_axis(c.y, step) << 16);
}

__global__ void __launch_bounds__(kMergeThreads)
merge_abucket_count_kernel(const float* __restrict__ coords, int N, int k, int G, int64_t n_anc,
                           const int32_t* __restrict__ anchors, int32_t* __restrict__ abcnt,
                           int32_t* __restrict__ abrank) {
  const int64_t x = (int64_t)blockIdx.x * kMergeThreads + threadIdx.x;
  if (x >= n_anc) return;
  const int64_t b = x / k;
  const MergeBuckets mb = merge_buckets(k);
  const double step = (double)(1u << (16 - knn_ceil_log2(G)));
  const uint32_t q = fixed_point(reinterpret_cast<const float2*>(coords)[b * N + anchors[x]], step);
  const int bk = (int)(((q >> 16) >> mb.bsh) * (uint32_t)mb.Pb + ((q & 0xFFFFu) >> mb.bsh));
  abrank[x] = atomicAdd(&abcnt[b * mb.nb + bk], 1);
}

__global__ void __launch_bounds__(kMergeThreads)
merge_abucket_place_kernel(const float* __restrict__ coords, int N, int k, int G, int64_t n_anc,
                           const int32_t* __restrict__ anchors, const int32_t* __restrict__ abstart,
                           const int32_t* __restrict__ abrank, uint2* __restrict__ abk) {
  const int64_t x = (int64_t)blockIdx.x * kMergeThreads + threadIdx.x;
  if (x >= n_anc) return;
  const int64_t b = x / k;
  const int pos = (int)(x - b * k);
  const MergeBuckets mb = merge_buckets(k);
  const double step = (double)(1u << (16 - knn_ceil_log2(G)));
  const uint32_t q = fixed_point(reinterpret_cast<const float2*>(coords)[b * N + anchors[x]], step);
  const int bk = (int)(((q >> 16) >> mb.bsh) * (uint32_t)mb.Pb + ((q & 0xFFFFu) >> mb.bsh));
  abk[b * k + abstart[b * (mb.nb + 1) + bk] + abrank[x]] = make_uint2(q, (uint32_t)pos);
}

// kRingLanes lanes per token (an aligned group: its lanes enter and leave
// every loop together, so the group's shuffles see active lanes only)
__global__ void __launch_bounds__(kMergeThreads)
merge_assign_wide_kernel(const float* __restrict__ coords, int N, int k, int G, int64_t n_tok,
                         const int32_t* __restrict__ apos_all, const int32_t* __restrict__ abstart_all,
                         const uint2* __restrict__ abk_all, int32_t* __restrict__ assign,
                         int32_t* __restrict__ gcnt) {
  const int64_t t = ((int64_t)blockIdx.x * kMergeThreads + threadIdx.x) / kRingLanes;
  const int u = threadIdx.x % kRingLanes;
  if (t >= n_tok) return;
  const int64_t b = t / N;
  int a = apos_all[t];
  if (a < 0) {
    const MergeBuckets mb = merge_buckets(k);
    const int bsh = mb.bsh, Pb = mb.Pb;
    const int32_t* abstart = abstart_all + b * (mb.nb + 1);
    const uint2* abk = abk_all + b * k;
    const double step = (double)(1u << (16 - knn_ceil_log2(G)));
    const uint32_t q = fixed_point(reinterpret_cast<const float2*>(coords)[t], step);
    const int64_t x = q & 0xFFFFu, y = q >> 16;
    const int bx0 = (int)(x >> bsh), by0 = (int)(y >> bsh);
    uint64_t best = ~0ull;
    for (int Rg = 0; Rg < Pb; ++Rg) {
      const int y0 = by0 - Rg, y1 = by0 + Rg, x0 = bx0 - Rg, x1 = bx0 + Rg;
      const int nring = Rg == 0 ? 1 : 8 * Rg, w = 2 * Rg + 1;
      for (int j = u; j < nring; j += kRingLanes) {
        int by, bx;
        if (j < w) {
          by = y0;
          bx = x0 + j;
        } else if (j < 2 * w) {
          by = y1;
          bx = x0 + j - w;
        } else {
          const int m = j - 2 * w;
          by = y0 + 1 + (m >> 1);
          bx = (m & 1) ? x1 : x0;
        }
        if (bx < 0 || bx >= Pb || by < 0 || by >= Pb) continue;
        const int bb = by * Pb + bx;
        const int t0 = abstart[bb], t1 = abstart[bb + 1];
        for (int e = t0; e < t1; ++e) {
          const uint2 v = abk[e];
          const int64_t ix = (int64_t)(v.x & 0xFFFFu) - x, iy = (int64_t)(v.x >> 16) - y;
          const uint64_t kk = ((uint64_t)(ix * ix + iy * iy) << kWideKeyBits) | v.y;
          best = kk < best ? kk : best;
        }
      }
#pragma unroll
      for (int m = 1; m < kRingLanes; m <<= 1) {
        const uint64_t o = ((uint64_t)(uint32_t)__shfl_xor((int)(best >> 32), m) << 32) |
                           (uint32_t)__shfl_xor((int)(uint32_t)best, m);
        best = o < best ? o : best;
      }
      int64_t lb = INT64_MAX;
      if (y0 > 0) lb = min(lb, y - ((int64_t)y0 << bsh) + 1);
      if (y1 < Pb - 1) lb = min(lb, ((int64_t)(y1 + 1) << bsh) - y);
      if (x0 > 0) lb = min(lb, x - ((int64_t)x0 << bsh) + 1);
      if (x1 < Pb - 1) lb = min(lb, ((int64_t)(x1 + 1) << bsh) - x);
      if (best != ~0ull && (lb == INT64_MAX || (int64_t)(best >> kWideKeyBits) < lb * lb)) break;
    }
    a = (int)(best & ((1ull << kWideKeyBits) - 1));
  }
  if (u == 0) {
    assign[t] = a;
    atomicAdd(&gcnt[b * k + a], 1);   // group sizes (integer atomics: any order)
  }
}

__global__ void __launch_bounds__(kMergeThreads)
merge_gplace_kernel(int N, int k, int64_t n_tok, const int32_t* __restrict__ assign,
                    const int32_t* __restrict__ offsets, int32_t* __restrict__ cur,
                    int32_t* __restrict__ glst) {
  const int64_t t = (int64_t)blockIdx.x * kMergeThreads + threadIdx.x;
  if (t >= n_tok) return;
  const int64_t b = t / N;
  const int a = assign[t];
  const int r = atomicAdd(&cur[b * k + a], 1);
  glst[b * N + offsets[b * (k + 1) + a] + r] = (int32_t)(t - b * N);
}

__global__ void __launch_bounds__(kMergeThreads)
merge_grank_kernel(int N, int k, int64_t n_tok, const int32_t* __restrict__ assign,
                   const int32_t* __restrict__ offsets, const int32_t* __restrict__ glst,
                   int32_t* __restrict__ members) {
  const int64_t t = (int64_t)blockIdx.x * kMergeThreads + threadIdx.x;
  if (t >= n_tok) return;
  const int64_t b = t / N;
  const int i = (int)(t - b * N);
  const int a = assign[t];
  const int lo = offsets[b * (k + 1) + a], hi = offsets[b * (k + 1) + a + 1];
  if (hi - lo > kLongSegment) return;   // sorted by launch_long_segment_sort
  const int32_t* seg = glst + b * N;
  int rank = 0, y = lo;
  for (; y + 4 <= hi; y += 4) {   // four loads in flight
    const int v0 = seg[y], v1 = seg[y + 1], v2 = seg[y + 2], v3 = seg[y + 3];
    rank += (v0 < i) + (v1 < i) + (v2 < i) + (v3 < i);
  }
  for (; y < hi; ++y) rank += seg[y] < i;
  members[b * N + lo + rank] = i;
}

// Lane groups: L = 2^lg lanes per anchor, 64 / L anchors per wave.
struct MGroup {
  int64_t id;
  int sub;
  bool valid;
};
__device__ __forceinline__ MGroup mgroup(int lg, int64_t total) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * (kMergeThreads / 64) + (threadIdx.x >> 6);
  MGroup g;
  g.id = wave * (64 >> lg) + (lane >> lg);
  g.sub = lane & ((1 << lg) - 1);
  g.valid = g.id < total;
  return g;
}

// softmax statistics of a group's scores: max and 1 / sum of exp.  Members
// are read four at a time with clamped indices (every load of a batch
// issues together), the extra ones masked.
constexpr int kMB = 4;
// one batch of scores (members u .. u + kMB - 1 of a group ending at z)
// into the running max and sum
__device__ __forceinline__ void softmax_batch(const float* v, int u, int z, float& mx, float& sum) {
  float m2 = mx;
#pragma unroll
  for (int h = 0; h < kMB; ++h) m2 = u + h < z ? fmaxf(m2, v[h]) : m2;
  sum *= __builtin_amdgcn_exp2f((mx - m2) * 1.4426950408889634f);   // rescale to the new max
  mx = m2;
#pragma unroll
  for (int h = 0; h < kMB; ++h)
    sum += u + h < z ? __builtin_amdgcn_exp2f((v[h] - mx) * 1.4426950408889634f) : 0.f;
}
// the statistics of a group whose first batch of scores v0 is at hand:
// max and 1 / sum of exp
__device__ __forceinline__ void group_softmax(const int32_t* __restrict__ mem, int a, int z,
                                              const float* __restrict__ s, const float* v0,
                                              float& mx, float& inv) {
  mx = -INFINITY;
  float sum = 0.f;
  softmax_batch(v0, a, z, mx, sum);
  for (int u = a + kMB; u < z; u += kMB) {
    float v[kMB];
#pragma unroll
    for (int h = 0; h < kMB; ++h) v[h] = s[mem[min(u + h, z - 1)]];
    softmax_batch(v, u, z, mx, sum);
  }
  inv = sum > 0.f ? 1.f / sum : 0.f;
}

// A group's first batch of members, with their scores, coordinates and the
// lane's chunks of their rows, all loads issued together (clamped indices:
// an empty group reads member 0 of the image, masked by the callers)
template <typename T>
struct FirstBatch {
  int mi[kMB];
  float sv[kMB];
  float2 x[kMB];
  uint4 row[Row16<T>::NR][kMB];
  __device__ void load(const int32_t* __restrict__ mem, int a, int z, const float* __restrict__ s,
                       const float2* __restrict__ xy, const T* __restrict__ fimg, int Cf, int sub,
                       int L, int nr) {
#pragma unroll
    for (int h = 0; h < kMB; ++h) mi[h] = mem[z > a ? min(a + h, z - 1) : 0];
#pragma unroll
    for (int h = 0; h < kMB; ++h) {
      sv[h] = s[mi[h]];
      x[h] = xy[mi[h]];
    }
#pragma unroll
    for (int r = 0; r < Row16<T>::NR; ++r)
      if (r < nr) {
#pragma unroll
        for (int h = 0; h < kMB; ++h)
          row[r][h] = Row16<T>::raw(fimg + (int64_t)mi[h] * Cf + (sub + r * L) * Row16<T>::E);
      }
  }
};

template <typename T>
__global__ void __launch_bounds__(kMergeThreads)
merge_fwd_kernel(int N, int k, int Cf, int lg, int64_t total, const T* __restrict__ feats,
                 const float* __restrict__ coords, const float* __restrict__ scores,
                 const int32_t* __restrict__ members, const int32_t* __restrict__ offsets,
                 T* __restrict__ out_f, float* __restrict__ out_x) {
  using Rw = Row16<T>;
  const MGroup g = mgroup(lg, total);
  if (!g.valid) return;
  const int L = 1 << lg;
  const int64_t b = g.id / k;
  const int an = (int)(g.id - b * k);
  const int32_t* mem = members + b * N;
  const int a = offsets[b * (k + 1) + an], z = offsets[b * (k + 1) + an + 1];
  const float* s = scores + b * N;
  const int nch = Cf / Rw::E;
  const T* fimg = feats + b * N * Cf;
  const float2* xy = reinterpret_cast<const float2*>(coords) + b * N;
  const int nr = (nch - g.sub + L - 1) / L;   // chunks of this lane
  FirstBatch<T> fb;
  fb.load(mem, a, z, s, xy, fimg, Cf, g.sub, L, nr);
  float mx, inv;
  group_softmax(mem, a, z, s, fb.sv, mx, inv);
  float acc[Rw::NR][Rw::E];
#pragma unroll
  for (int r = 0; r < Rw::NR; ++r)
#pragma unroll
    for (int e = 0; e < Rw::E; ++e) acc[r][e] = 0.f;
  float ax = 0.f, ay = 0.f;
  // one batch of kMB members: weights, rows (loaded), coordinates
  auto batch = [&](int u, const float* sv, const float2* x, const uint4 (*row)[kMB]) {
    float w[kMB];
#pragma unroll
    for (int h = 0; h < kMB; ++h)
      w[h] = u + h < z ? __builtin_amdgcn_exp2f((sv[h] - mx) * 1.4426950408889634f) * inv : 0.f;
#pragma unroll
    for (int r = 0; r < Rw::NR; ++r) {
      if (r >= nr) break;
#pragma unroll
      for (int h = 0; h < kMB; ++h) {
        float v[Rw::E];
        Rw::cvt(row[r][h], v);
#pragma unroll
        for (int e = 0; e < Rw::E; ++e) acc[r][e] = fmaf(w[h], v[e], acc[r][e]);
      }
    }
#pragma unroll
    for (int h = 0; h < kMB; ++h) {
      ax = fmaf(w[h], x[h].x, ax);
      ay = fmaf(w[h], x[h].y, ay);
    }
  };
  batch(a, fb.sv, fb.x, fb.row);
  for (int u = a + kMB; u < z; u += kMB) {   // larger groups: four members at a time, loads first
    FirstBatch<T> nb;
    nb.load(mem, u, z, s, xy, fimg, Cf, g.sub, L, nr);
    batch(u, nb.sv, nb.x, nb.row);
  }
#pragma unroll
  for (int r = 0; r < Rw::NR; ++r) {
    const int c = g.sub + r * L;
    if (c >= nch) break;
    Rw::store(out_f + g.id * Cf + c * Rw::E, acc[r]);
  }
  if (g.sub == 0) reinterpret_cast<float2*>(out_x)[g.id] = make_float2(ax, ay);
}

template <typename T>
__global__ void __launch_bounds__(kMergeThreads)
merge_bwd_kernel(int N, int k, int Cf, int lg, int64_t total, const T* __restrict__ feats,
                 const float* __restrict__ coords, const float* __restrict__ scores,
                 const int32_t* __restrict__ members, const int32_t* __restrict__ offsets,
                 const T* __restrict__ dout_f, const float* __restrict__ dout_x,
                 T* __restrict__ dfeats, float* __restrict__ dcoords, float* __restrict__ dscores) {
  using Rw = Row16<T>;
  const MGroup g = mgroup(lg, total);
  const int L = 1 << lg;
  const int64_t id = g.valid ? g.id : 0;   // idle lanes mirror anchor 0 (group shuffles)
  const int64_t b = id / k;
  const int an = (int)(id - b * k);
  const int nch = Cf / Rw::E;
  // the anchor's output gradient first (independent of the member lists)
  float dof[Rw::NR][Rw::E];
#pragma unroll
  for (int r = 0; r < Rw::NR; ++r) {
    const int c = g.sub + r * L;
#pragma unroll
    for (int e = 0; e < Rw::E; ++e) dof[r][e] = 0.f;
    if (c < nch) Rw::load(dout_f + id * Cf + c * Rw::E, dof[r]);
  }
  const float2 dox = reinterpret_cast<const float2*>(dout_x)[id];
  const int32_t* mem = members + b * N;
  const int a = offsets[b * (k + 1) + an], z = offsets[b * (k + 1) + an + 1];
  const float* s = scores + b * N;
  const T* fimg = feats + b * N * Cf;
  const float2* xy = reinterpret_cast<const float2*>(coords) + b * N;
  const int nr = (nch - g.sub + L - 1) / L;   // chunks of this lane
  FirstBatch<T> fb;
  fb.load(mem, a, z, s, xy, fimg, Cf, g.sub, L, nr);
  float mx, inv;
  group_softmax(mem, a, z, s, fb.sv, mx, inv);
  float gbar = 0.f;
  // one batch of kMB members (same trip count for the whole group: the
  // group shuffles): dF rows, <dO, F_i> + <dO_x, x_i> = g_i into gi, the
  // weights into w, the coordinate gradients
  auto batch = [&](int u, const int* mi, const float* sv, const float2* x, const uint4 (*row)[kMB],
                   float* w, float* gi) {
    float dot[kMB];
#pragma unroll
    for (int h = 0; h < kMB; ++h) {
      w[h] = u + h < z ? __builtin_amdgcn_exp2f((sv[h] - mx) * 1.4426950408889634f) * inv : 0.f;
      dot[h] = 0.f;
    }
#pragma unroll
    for (int r = 0; r < Rw::NR; ++r) {
      if (r >= nr) break;
      const int c = g.sub + r * L;
#pragma unroll
      for (int h = 0; h < kMB; ++h) {
        float v[Rw::E], d[Rw::E];
        Rw::cvt(row[r][h], v);
#pragma unroll
        for (int e = 0; e < Rw::E; ++e) {
          dot[h] = fmaf(dof[r][e], v[e], dot[h]);
          d[e] = w[h] * dof[r][e];
        }
        if (g.valid && u + h < z) Rw::store(dfeats + (b * N + mi[h]) * Cf + c * Rw::E, d);
      }
    }
    for (int o = 1; o < L; o <<= 1)
#pragma unroll
      for (int h = 0; h < kMB; ++h) dot[h] += __shfl_xor(dot[h], o, 64);
#pragma unroll
    for (int h = 0; h < kMB; ++h) {
      gi[h] = dot[h] + dox.x * x[h].x + dox.y * x[h].y;
      gbar = fmaf(w[h], gi[h], gbar);
      if (g.valid && g.sub == 0 && u + h < z)
        reinterpret_cast<float2*>(dcoords)[b * N + mi[h]] = make_float2(w[h] * dox.x, w[h] * dox.y);
    }
  };
  float w0[kMB], g0[kMB];
  batch(a, fb.mi, fb.sv, fb.x, fb.row, w0, g0);
  for (int u = a + kMB; u < z; u += kMB) {   // larger groups: later batches, loads first
    FirstBatch<T> nb;
    nb.load(mem, u, z, s, xy, fimg, Cf, g.sub, L, nr);
    float w[kMB], gi[kMB];
    batch(u, nb.mi, nb.sv, nb.x, nb.row, w, gi);
    if (g.valid && g.sub == 0)
#pragma unroll
      for (int h = 0; h < kMB; ++h)
        if (u + h < z) dscores[b * N + nb.mi[h]] = gi[h];   // g_i for now; finished below
  }
  if (!g.valid || g.sub != 0) return;
  // dL/ds_i = w_i (g_i - sum_j w_j g_j): the first batch from registers
#pragma unroll
  for (int h = 0; h < kMB; ++h)
    if (a + h < z) dscores[b * N + fb.mi[h]] = w0[h] * (g0[h] - gbar);
  for (int u = a + kMB; u < z; ++u) {
    const int i = mem[u];
    const float w = __builtin_amdgcn_exp2f((s[i] - mx) * 1.4426950408889634f) * inv;
    dscores[b * N + i] = w * (dscores[b * N + i] - gbar);
  }
}

int mgroup_log2(int Cf, int E) {
  const int nch = Cf / E;
  int lg = 0;
  while ((1 << lg) < nch && lg < 6) ++lg;
  return lg;
}

unsigned mgrid(int64_t groups, int lg) {
  const int64_t per_wave = 64 >> lg;
  const int64_t waves = (groups + per_wave - 1) / per_wave;
  return (unsigned)((waves + kMergeThreads / 64 - 1) / (kMergeThreads / 64));
}

template <typename T>
hipError_t fwd_t(int B, int N, int k, int Cf, const void* feats, const float* coords,
                 const float* scores, const int32_t* members, const int32_t* offsets, void* out_f,
                 float* out_x, hipStream_t st) {
  const int lg = mgroup_log2(Cf, Row16<T>::E);
  const int64_t total = (int64_t)B * k;
  hipLaunchKernelGGL(merge_fwd_kernel<T>, dim3(mgrid(total, lg)), dim3(kMergeThreads), 0, st, N, k,
                     Cf, lg, total, (const T*)feats, coords, scores, members, offsets, (T*)out_f,
                     out_x);
  return hipGetLastError();
}

template <typename T>
hipError_t bwd_t(int B, int N, int k, int Cf, const void* feats, const float* coords,
                 const float* scores, const int32_t* members, const int32_t* offsets,
                 const void* dout_f, const float* dout_x, void* dfeats, float* dcoords,
                 float* dscores, hipStream_t st) {
  const int lg = mgroup_log2(Cf, Row16<T>::E);
  const int64_t total = (int64_t)B * k;
  hipLaunchKernelGGL(merge_bwd_kernel<T>, dim3(mgrid(total, lg)), dim3(kMergeThreads), 0, st, N, k,
                     Cf, lg, total, (const T*)feats, coords, scores, members, offsets,
                     (const T*)dout_f, dout_x, (T*)dfeats, dcoords, dscores);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_merge_plan(const float* coords, const float* scores, int B, int N, int k, int G,
                             int32_t* anchors, int32_t* assign, int32_t* members,
                             int32_t* offsets, void* ws, hipStream_t st) {
  if (N <= kMaxTok) {
    // the ring search of an image is spread over S workgroups (each repeats
    // the selection and the bucketing) so that a batch fills the chip
    const int S = std::max(1, std::min({8, (N + 255) / 256, std::max(1, 256 / std::max(B, 1))}));
    hipLaunchKernelGGL(merge_assign_kernel, dim3(B * S), dim3(kPlanT), 0, st, coords, scores, N, k,
                       G, S, anchors, assign);
    hipLaunchKernelGGL(merge_members_kernel, dim3(B), dim3(kPlanT), 0, st, N, k, assign, members,
                       offsets);
    return hipGetLastError();
  }
  const MergeWorkspace w = merge_layout(ws, B, N, k);
  const MergeBuckets mb = merge_buckets(k);
  const int nch = (N + kMergeSelChunk - 1) / kMergeSelChunk;
  const int64_t n_tok = (int64_t)B * N, n_anc = (int64_t)B * k;
  auto grid = [](int64_t n) { return dim3((unsigned)((n + kMergeThreads - 1) / kMergeThreads)); };
  hipLaunchKernelGGL(merge_select_kernel, dim3(B), dim3(kPlanT), 0, st, scores, N, k, mb.nb, nch,
                     w.sk, w.sel, w.chunk, w.abcnt, w.gcnt, w.gcur);
  hipLaunchKernelGGL(merge_flag_kernel, dim3((unsigned)(B * nch)), dim3(kPlanT), 0, st, N, k, nch,
                     (const uint32_t*)w.sk, (const uint2*)w.sel, (const int2*)w.chunk, w.apos,
                     anchors);
  hipLaunchKernelGGL(merge_abucket_count_kernel, grid(n_anc), dim3(kMergeThreads), 0, st, coords, N,
                     k, G, n_anc, (const int32_t*)anchors, w.abcnt, w.abrank);
  launch_segment_scan(B, mb.nb, w.abcnt, w.abstart, st);
  hipLaunchKernelGGL(merge_abucket_place_kernel, grid(n_anc), dim3(kMergeThreads), 0, st, coords, N,
                     k, G, n_anc, (const int32_t*)anchors, (const int32_t*)w.abstart,
                     (const int32_t*)w.abrank, w.abk);
  hipLaunchKernelGGL(merge_assign_wide_kernel, grid(n_tok * kRingLanes), dim3(kMergeThreads), 0, st,
                     coords, N, k, G, n_tok, (const int32_t*)w.apos, (const int32_t*)w.abstart,
                     (const uint2*)w.abk, assign, w.gcnt);
  launch_segment_scan(B, k, w.gcnt, offsets, st);
  hipLaunchKernelGGL(merge_gplace_kernel, grid(n_tok), dim3(kMergeThreads), 0, st, N, k, n_tok,
                     (const int32_t*)assign, (const int32_t*)offsets, w.gcur, w.glst);
  // groups of more than kLongSegment members: a stable sort; the rest ranked
  launch_long_segment_sort(B, k, N, N - 1, offsets, w.glst, w.gtmp, members, nullptr, 0, nullptr,
                           st);
  hipLaunchKernelGGL(merge_grank_kernel, grid(n_tok), dim3(kMergeThreads), 0, st, N, k, n_tok,
                     (const int32_t*)assign, (const int32_t*)offsets, (const int32_t*)w.glst,
                     members);
  return hipGetLastError();
}

hipError_t launch_merge_fwd(int dt, int B, int N, int k, int Cf, const void* feats,
                            const float* coords, const float* scores, const int32_t* members,
                            const int32_t* offsets, void* out_f, float* out_x, hipStream_t st) {
  switch (dt) {
    case 0: return fwd_t<float>(B, N, k, Cf, feats, coords, scores, members, offsets, out_f, out_x, st);
    case 1: return fwd_t<bf16>(B, N, k, Cf, feats, coords, scores, members, offsets, out_f, out_x, st);
    default: return fwd_t<f16>(B, N, k, Cf, feats, coords, scores, members, offsets, out_f, out_x, st);
  }
}

hipError_t launch_merge_bwd(int dt, int B, int N, int k, int Cf, const void* feats,
                            const float* coords, const float* scores, const int32_t* members,
                            const int32_t* offsets, const void* dout_f, const float* dout_x,
                            void* dfeats, float* dcoords, float* dscores, hipStream_t st) {
  switch (dt) {
    case 0:
      return bwd_t<float>(B, N, k, Cf, feats, coords, scores, members, offsets, dout_f, dout_x,
                          dfeats, dcoords, dscores, st);
    case 1:
      return bwd_t<bf16>(B, N, k, Cf, feats, coords, scores, members, offsets, dout_f, dout_x,
                         dfeats, dcoords, dscores, st);
    default:
      return bwd_t<f16>(B, N, k, Cf, feats, coords, scores, members, offsets, dout_f, dout_x,
                        dfeats, dcoords, dscores, st);
  }
}

}  // namespace ca
