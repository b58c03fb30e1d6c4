// Matrix-core (MFMA) cluster attention kernels for gfx950, bf16 / fp16,
// clusters of 8 and 48 key slots.
//
// What is computed: exact softmax attention of every query cluster over the
// 48 gathered key slots of its neighbour clusters, forward (O, LSE) and
// backward (dQ, dK, dV) - the local cluster attention of the English notes
// page "AFFMAE: Scalable Vision Pre-Training for High-Resolution Microscopy
// Segmentation on Desktop Hardware" ("Overall Architecture"), run as the
// numerically stable mixed-precision Flash-style kernels its arXiv abstract
// describes: bf16/fp16 operands, fp32 statistics and accumulation, logits in
// log2 units so every exponential is one v_exp_f32.
//
// Tiling (one 64-lane wavefront per (cluster, pair of heads), no LDS):
//  * v_mfma_f32_16x16x32 operand layout (checked on the hardware): lane
//    l = c + 16 g holds row/column c and reduction indices [8g, 8g+8); the
//    16x16 fp32 result puts rows 4g..4g+3 of column c in lane l.
//  * A cluster has 8 queries, half a 16-wide tile, so the two heads of a
//    pair share one tile: columns 0-7 are head h0, 8-15 head h1.  Products
//    whose other operand differs per head run as two MFMAs with the unused
//    half of one operand zeroed (block-diagonal), which costs no more than
//    a half-empty tile and keeps every lane of the softmax busy.
//  * Products that contract over keys (P.V, dS.K) or queries (dS^T.Q,
//    P^T.dO) need the gathered rows transposed.  A wave does that in
//    registers by multiplying the rows, as loaded, with a 0/1 selection
//    matrix on the MFMA unit (exact: one nonzero product per output).
//  * Probabilities and dS enter the bf16 products as a hi + lo pair
//    (x = hi + lo exactly to ~16 bits) so their rounding stays far below
//    the output rounding.
//  * Workgroups of 4 wavefronts are remapped so that each XCD (eight,
//    dispatched round-robin) walks one contiguous Morton range of clusters:
//    neighbouring clusters share their gathered K/V rows in that XCD's L2.
#include "common.h"

namespace ca {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int D = 32;
constexpr int CS = 8;
constexpr int NK = 48;
constexpr int kWaves = 4;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <typename T> struct Mfma;

template <> struct Mfma<bf16> {
  typedef __bf16 v8 __attribute__((ext_vector_type(8)));
  static constexpr uint32_t kOne = 0x3F80u;
  static __device__ __forceinline__ f32x4 mma32(uint4 a, uint4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8, a),
                                                   __builtin_bit_cast(v8, b), c, 0, 0, 0);
  }
};

template <> struct Mfma<f16> {
  typedef _Float16 v8 __attribute__((ext_vector_type(8)));
  static constexpr uint32_t kOne = 0x3C00u;
  static __device__ __forceinline__ f32x4 mma32(uint4 a, uint4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8, a),
                                                  __builtin_bit_cast(v8, b), c, 0, 0, 0);
  }
};

// A 16x16x16 product (4 reduction elements per lane) run on the 16x16x32
// instruction with the upper half of every lane's reduction slice zeroed.
// Only the 16x16x32 form is used so that every MFMA in a chain has the same
// shape (and the same lane layout, which was checked on the hardware).
template <typename T>
__device__ __forceinline__ f32x4 mma16(uint2 a, uint2 b, f32x4 c) {
  return Mfma<T>::mma32(make_uint4(a.x, a.y, 0u, 0u), make_uint4(b.x, b.y, 0u, 0u), c);
}

template <typename T>
__device__ __forceinline__ uint32_t bits16(T x) {
  return (uint32_t)__builtin_bit_cast(unsigned short, x);
}

// pack two floats (RNE) into one dword of T
template <typename T>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  return bits16<T>((T)a) | (bits16<T>((T)b) << 16);
}

template <typename T>
__device__ __forceinline__ uint2 pack4(f32x4 x) {
  return make_uint2(pack2<T>(x[0], x[1]), pack2<T>(x[2], x[3]));
}

// hi/lo split of 4 floats: x ~= hi + lo with hi = T(x), lo = T(x - hi)
template <typename T>
__device__ __forceinline__ void split4(const float* x, uint2& hi, uint2& lo) {
  T h[4];
  float r[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[i] = (T)x[i];
    r[i] = x[i] - (float)h[i];
  }
  hi = make_uint2(bits16<T>(h[0]) | (bits16<T>(h[1]) << 16), bits16<T>(h[2]) | (bits16<T>(h[3]) << 16));
  lo = make_uint2(pack2<T>(r[0], r[1]), pack2<T>(r[2], r[3]));
}

__device__ __forceinline__ uint4 cat(uint2 a, uint2 b) { return make_uint4(a.x, a.y, b.x, b.y); }
__device__ __forceinline__ uint4 sel(bool c, uint4 a) {
  return c ? a : make_uint4(0u, 0u, 0u, 0u);
}
__device__ __forceinline__ uint2 sel(bool c, uint2 a) { return c ? a : make_uint2(0u, 0u); }

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// 0/1 selection matrix as a B operand: B[k][c] = (k == c + 16 * half), the
// reduction index k = 8g + e of element e in lane group g.
template <typename T>
__device__ __forceinline__ uint4 selector(int g, int c16, int half) {
  uint32_t w[4];
#pragma unroll
  for (int e2 = 0; e2 < 4; ++e2) {
    uint32_t lo = (8 * g + 2 * e2 == c16 + 16 * half) ? Mfma<T>::kOne : 0u;
    uint32_t hi = (8 * g + 2 * e2 + 1 == c16 + 16 * half) ? Mfma<T>::kOne : 0u;
    w[e2] = lo | (hi << 16);
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// Transpose one 16-row x 32-dim A-operand tile (lane c16+16g holds row c16,
// dims [8g, 8g+8)) into the two 16x16 halves as A operands over rows:
// out[half] holds rows 4g..4g+3 of dim c16 + 16*half (packed to T).
template <typename T>
__device__ __forceinline__ void transpose_rows(uint4 rows, const uint4 (&id)[2], uint2 (&out)[2]) {
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) out[hf] = pack4<T>(Mfma<T>::mma32(rows, id[hf], z));
}

__device__ __forceinline__ int xcd_remap(int w, int n) {
  // dispatch sends workgroup w to XCD w % 8; give XCD x a contiguous range
  const int x = w & 7, i = w >> 3;
  const int q = n >> 3, r = n & 7;
  return x * q + min(x, r) + i;
}

__device__ __forceinline__ float shfl_max16_32(float v) {
  v = fmaxf(v, __shfl_xor(v, 16, 64));
  return fmaxf(v, __shfl_xor(v, 32, 64));
}
__device__ __forceinline__ float shfl_sum16_32(float v) {
  v += __shfl_xor(v, 16, 64);
  return v + __shfl_xor(v, 32, 64);
}

// ---------------------------------------------------------------------------
// forward
// ---------------------------------------------------------------------------
template <typename T, bool kSplit>
__global__ void __launch_bounds__(64 * kWaves)
fwd_mfma_kernel(int N, int H, int HP, int64_t n_items, float scale_log2, const T* __restrict__ q,
                const T* __restrict__ k, const T* __restrict__ v,
                const int32_t* __restrict__ q_idx, const int32_t* __restrict__ key_idx,
                T* __restrict__ o, float* __restrict__ lse) {
  const int lane = threadIdx.x & 63;
  const int64_t item = (int64_t)xcd_remap(blockIdx.x, gridDim.x) * kWaves + (threadIdx.x >> 6);
  if (item >= n_items) return;
  const int64_t bc = item / HP;
  const int h0 = 2 * (int)(item - bc * HP), h1 = h0 + 1;
  const int64_t img = bc / (N / CS) * (int64_t)N;
  const int c16 = lane & 15, g = lane >> 4;
  const bool left = c16 < 8;
  const int hq = left ? h0 : h1;
  const bool h1ok = h1 < H;

  // indices
  int kt[3];
  uint32_t valid[3];
#pragma unroll
  for (int b = 0; b < 3; ++b) {
    kt[b] = key_idx[bc * NK + 16 * b + c16];
    valid[b] = (uint32_t)__ballot(kt[b] >= 0) & 0xFFFFu;
    kt[b] = max(kt[b], 0);
  }
  const int qtok = q_idx[bc * CS + (c16 & 7)];

  // operands: Q^T as B (own head), K and V rows as A for both heads
  const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
  const uint4 qv = (hq < H) ? ld16(q + ((img + qtok) * H + hq) * D + 8 * g) : zero;
  uint4 ka[3][2], va[3][2];
#pragma unroll
  for (int b = 0; b < 3; ++b) {
    const int64_t r = (img + kt[b]) * H;
    ka[b][0] = ld16(k + (r + h0) * D + 8 * g);
    va[b][0] = ld16(v + (r + h0) * D + 8 * g);
    ka[b][1] = h1ok ? ld16(k + (r + h1) * D + 8 * g) : zero;
    va[b][1] = h1ok ? ld16(v + (r + h1) * D + 8 * g) : zero;
  }

  // S^T = K Q^T, lane holds keys 16b+4g+i of column c16
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  float x[3][4];
  float mx = -INFINITY;
#pragma unroll
  for (int b = 0; b < 3; ++b) {
    f32x4 s = Mfma<T>::mma32(ka[b][0], sel(left, qv), z);
    s = Mfma<T>::mma32(ka[b][1], sel(!left, qv), s);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[b][i] = ((valid[b] >> (4 * g + i)) & 1u) ? s[i] * scale_log2 : -INFINITY;
      mx = fmaxf(mx, x[b][i]);
    }
  }
  mx = shfl_max16_32(mx);
  const float mref = mx == -INFINITY ? 0.f : mx;
  float l = 0.f;
#pragma unroll
  for (int b = 0; b < 3; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[b][i] = __builtin_amdgcn_exp2f(x[b][i] - mref);
      l += x[b][i];
    }
  l = shfl_sum16_32(l);

  // P as B operands (reduction over keys): step 0 = blocks 0,1, step 1 = block 2
  uint2 ph[3], pl[3];
#pragma unroll
  for (int b = 0; b < 3; ++b) {
    if (kSplit) {
      split4<T>(x[b], ph[b], pl[b]);
    } else {
      ph[b] = make_uint2(pack2<T>(x[b][0], x[b][1]), pack2<T>(x[b][2], x[b][3]));
      pl[b] = make_uint2(0u, 0u);
    }
  }

  // V^T tiles via the selection matrix, then O^T = V^T P^T
  uint4 id[2];
  id[0] = selector<T>(g, c16, 0);
  id[1] = selector<T>(g, c16, 1);
  f32x4 oacc[2] = {z, z};
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    if (hh == 1 && !h1ok) break;
    const bool mine = (hh == 0) == left;   // this head's columns
    uint2 vt[3][2];
#pragma unroll
    for (int b = 0; b < 3; ++b) transpose_rows<T>(va[b][hh], id, vt[b]);
    const uint4 b0h = sel(mine, cat(ph[0], ph[1]));
    const uint2 b1h = sel(mine, ph[2]);
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      oacc[hf] = Mfma<T>::mma32(cat(vt[0][hf], vt[1][hf]), b0h, oacc[hf]);
      oacc[hf] = mma16<T>(vt[2][hf], b1h, oacc[hf]);
      if (kSplit) {
        oacc[hf] = Mfma<T>::mma32(cat(vt[0][hf], vt[1][hf]), sel(mine, cat(pl[0], pl[1])), oacc[hf]);
        oacc[hf] = mma16<T>(vt[2][hf], sel(mine, pl[2]), oacc[hf]);
      }
    }
  }

  if (hq >= H) return;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  T* dst = o + ((img + qtok) * H + hq) * D + 4 * g;
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
    *reinterpret_cast<uint2*>(dst + 16 * hf) = pack4<T>(oacc[hf] * inv);
  if (g == 0) lse[(img + qtok) * H + hq] = l > 0.f ? (mx + __log2f(l)) * kLn2 : -INFINITY;
}

// ---------------------------------------------------------------------------
// backward pass A (query-major): Delta and dQ
// ---------------------------------------------------------------------------
template <typename T, bool kSplit>
__global__ void __launch_bounds__(64 * kWaves)
bwd_q_mfma_kernel(int N, int H, int HP, int64_t n_items, float scale, const T* __restrict__ q,
                  const T* __restrict__ k, const T* __restrict__ v, const T* __restrict__ o,
                  const T* __restrict__ dout, const float* __restrict__ lse,
                  const int32_t* __restrict__ q_idx, const int32_t* __restrict__ key_idx,
                  T* __restrict__ dq, float* __restrict__ delta) {
  const int lane = threadIdx.x & 63;
  const int64_t item = (int64_t)xcd_remap(blockIdx.x, gridDim.x) * kWaves + (threadIdx.x >> 6);
  if (item >= n_items) return;
  const int64_t bc = item / HP;
  const int h0 = 2 * (int)(item - bc * HP), h1 = h0 + 1;
  const int64_t img = bc / (N / CS) * (int64_t)N;
  const int c16 = lane & 15, g = lane >> 4;
  const bool left = c16 < 8;
  const int hq = left ? h0 : h1;
  const bool h1ok = h1 < H, qok = hq < H;
  const float scale_log2 = scale * kLog2e;

  int kt[3];
  uint32_t valid[3];
#pragma unroll
  for (int b = 0; b < 3; ++b) {
    kt[b] = key_idx[bc * NK + 16 * b + c16];
    valid[b] = (uint32_t)__ballot(kt[b] >= 0) & 0xFFFFu;
    kt[b] = max(kt[b], 0);
  }
  const int qtok = q_idx[bc * CS + (c16 & 7)];
  const int64_t qrow = ((img + qtok) * H + hq) * D + 8 * g;
  const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
  const uint4 qv = qok ? ld16(q + qrow) : zero;
  const uint4 dov = qok ? ld16(dout + qrow) : zero;
  const uint4 ov = qok ? ld16(o + qrow) : zero;
  const float lse2 = qok ? lse[(img + qtok) * H + hq] * kLog2e : 0.f;
  uint4 ka[3][2], va[3][2];
#pragma unroll
  for (int b = 0; b < 3; ++b) {
    const int64_t r = (img + kt[b]) * H;
    ka[b][0] = ld16(k + (r + h0) * D + 8 * g);
    va[b][0] = ld16(v + (r + h0) * D + 8 * g);
    ka[b][1] = h1ok ? ld16(k + (r + h1) * D + 8 * g) : zero;
    va[b][1] = h1ok ? ld16(v + (r + h1) * D + 8 * g) : zero;
  }

  // Delta = <dO, O> per (query, head) column
  float dl = 0.f;
  {
    const T* a = reinterpret_cast<const T*>(&dov);
    const T* bb = reinterpret_cast<const T*>(&ov);
#pragma unroll
    for (int e = 0; e < 8; ++e) dl = fmaf((float)a[e], (float)bb[e], dl);
  }
  dl = shfl_sum16_32(dl);
  if (qok && g == 0) delta[(img + qtok) * H + hq] = dl;

  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  float ds[3][4];
#pragma unroll
  for (int b = 0; b < 3; ++b) {
    f32x4 s = Mfma<T>::mma32(ka[b][0], sel(left, qv), z);
    s = Mfma<T>::mma32(ka[b][1], sel(!left, qv), s);
    f32x4 dp = Mfma<T>::mma32(va[b][0], sel(left, dov), z);
    dp = Mfma<T>::mma32(va[b][1], sel(!left, dov), dp);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool ok = (valid[b] >> (4 * g + i)) & 1u;
      const float p = ok ? __builtin_amdgcn_exp2f(fmaf(s[i], scale_log2, -lse2)) : 0.f;
      ds[b][i] = p * (dp[i] - dl);
    }
  }
  uint2 dh[3], dlo[3];
#pragma unroll
  for (int b = 0; b < 3; ++b) {
    if (kSplit) {
      split4<T>(ds[b], dh[b], dlo[b]);
    } else {
      dh[b] = make_uint2(pack2<T>(ds[b][0], ds[b][1]), pack2<T>(ds[b][2], ds[b][3]));
    }
  }

  uint4 id[2];
  id[0] = selector<T>(g, c16, 0);
  id[1] = selector<T>(g, c16, 1);
  f32x4 acc[2] = {z, z};
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    if (hh == 1 && !h1ok) break;
    const bool mine = (hh == 0) == left;
    uint2 ktt[3][2];
#pragma unroll
    for (int b = 0; b < 3; ++b) transpose_rows<T>(ka[b][hh], id, ktt[b]);
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      acc[hf] = Mfma<T>::mma32(cat(ktt[0][hf], ktt[1][hf]), sel(mine, cat(dh[0], dh[1])), acc[hf]);
      acc[hf] = mma16<T>(ktt[2][hf], sel(mine, dh[2]), acc[hf]);
      if (kSplit) {
        acc[hf] = Mfma<T>::mma32(cat(ktt[0][hf], ktt[1][hf]), sel(mine, cat(dlo[0], dlo[1])), acc[hf]);
        acc[hf] = mma16<T>(ktt[2][hf], sel(mine, dlo[2]), acc[hf]);
      }
    }
  }
  if (!qok) return;
  T* dst = dq + ((img + qtok) * H + hq) * D + 4 * g;
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
    *reinterpret_cast<uint2*>(dst + 16 * hf) = pack4<T>(acc[hf] * scale);
}

// ---------------------------------------------------------------------------
// backward pass B (key-major): dK and dV over the transposed lists
// ---------------------------------------------------------------------------
template <typename T, bool kSplit>
__global__ void __launch_bounds__(64 * kWaves)
bwd_kv_mfma_kernel(int N, int H, int HP, int64_t n_items, float scale, const T* __restrict__ q,
                   const T* __restrict__ k, const T* __restrict__ v, const T* __restrict__ dout,
                   const float* __restrict__ lse, const int32_t* __restrict__ q_idx,
                   const float* __restrict__ delta, const int32_t* __restrict__ off_all,
                   const RevEntry* __restrict__ rev_all, int nk, T* __restrict__ dk,
                   T* __restrict__ dv) {
  const int lane = threadIdx.x & 63;
  const int64_t item = (int64_t)xcd_remap(blockIdx.x, gridDim.x) * kWaves + (threadIdx.x >> 6);
  if (item >= n_items) return;
  const int C = N / CS;
  const int64_t bj = item / HP;
  const int h0 = 2 * (int)(item - bj * HP), h1 = h0 + 1;
  const int64_t b = bj / C;
  const int j = (int)(bj - b * C);
  const int64_t img = b * N;
  const int c16 = lane & 15, g = lane >> 4;
  const bool left = c16 < 8;
  const int hk = left ? h0 : h1;
  const bool h1ok = h1 < H, kok = hk < H;
  const float scale_log2 = scale * kLog2e;

  // own key rows as B operands (column c16 = key c16&7 of head hk)
  const int ktok = q_idx[bj * CS + (c16 & 7)];
  const int64_t krow = ((img + ktok) * H + hk) * D + 8 * g;
  const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
  const uint4 kB = kok ? ld16(k + krow) : zero;
  const uint4 vB = kok ? ld16(v + krow) : zero;

  const int32_t* off = off_all + b * (C + 1);
  const RevEntry* rev = rev_all + b * (int64_t)C * nk;
  const int e0 = off[j], e1 = off[j + 1];

  uint4 id[2];
  id[0] = selector<T>(g, c16, 0);
  id[1] = selector<T>(g, c16, 1);
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  f32x4 dka[2] = {z, z}, dva[2] = {z, z};

  for (int e = e0; e < e1; e += 2) {
    // A-operand rows: row c16 = query c16&7 of entry e + (c16 >> 3)
    const int ea = e + (c16 >> 3);
    const bool eok = ea < e1;
    const RevEntry ent = rev[eok ? ea : e];
    const int qtok = eok ? q_idx[(b * C + ent.i) * CS + (c16 & 7)] : 0;
    const int64_t r = (img + qtok) * H;
    const uint4 qa0 = ld16(q + (r + h0) * D + 8 * g);
    const uint4 da0 = ld16(dout + (r + h0) * D + 8 * g);
    const uint4 qa1 = h1ok ? ld16(q + (r + h1) * D + 8 * g) : zero;
    const uint4 da1 = h1ok ? ld16(dout + (r + h1) * D + 8 * g) : zero;

    // this lane's output rows 4g..4g+3 belong to entry e + (g >> 1)
    const int eo = e + (g >> 1);
    const bool ook = eo < e1;
    const RevEntry ento = rev[ook ? eo : e];
    const float mult = ook && kok ? (float)((ento.mult >> (8 * (c16 & 7))) & 0xFFu) : 0.f;
    float l2[4], dl[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // query of row 4g+i is held (as qtok) by lane 4g+i
      const int t = __shfl(qtok, 4 * g + i, 64);
      const int64_t at = (img + t) * H + (kok ? hk : 0);
      l2[i] = mult != 0.f ? lse[at] * kLog2e : 0.f;
      dl[i] = mult != 0.f ? delta[at] : 0.f;
    }

    f32x4 s = Mfma<T>::mma32(qa0, sel(left, kB), z);
    s = Mfma<T>::mma32(qa1, sel(!left, kB), s);
    f32x4 dp = Mfma<T>::mma32(da0, sel(left, vB), z);
    dp = Mfma<T>::mma32(da1, sel(!left, vB), dp);
    float p[4], ds[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[i] = mult != 0.f ? mult * __builtin_amdgcn_exp2f(fmaf(s[i], scale_log2, -l2[i])) : 0.f;
      ds[i] = p[i] * (dp[i] - dl[i]);
    }
    uint2 ph, pl, dh, dlo;
    if (kSplit) {
      split4<T>(p, ph, pl);
      split4<T>(ds, dh, dlo);
    } else {
      ph = make_uint2(pack2<T>(p[0], p[1]), pack2<T>(p[2], p[3]));
      dh = make_uint2(pack2<T>(ds[0], ds[1]), pack2<T>(ds[2], ds[3]));
    }

#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      if (hh == 1 && !h1ok) break;
      const bool mine = (hh == 0) == left;
      uint2 dot[2], qt[2];
      transpose_rows<T>(hh == 0 ? da0 : da1, id, dot);
      transpose_rows<T>(hh == 0 ? qa0 : qa1, id, qt);
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        dva[hf] = mma16<T>(dot[hf], sel(mine, ph), dva[hf]);
        dka[hf] = mma16<T>(qt[hf], sel(mine, dh), dka[hf]);
        if (kSplit) {
          dva[hf] = mma16<T>(dot[hf], sel(mine, pl), dva[hf]);
          dka[hf] = mma16<T>(qt[hf], sel(mine, dlo), dka[hf]);
        }
      }
    }
  }

  if (!kok) return;
  T* dkd = dk + ((img + ktok) * H + hk) * D + 4 * g;
  T* dvd = dv + ((img + ktok) * H + hk) * D + 4 * g;
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    *reinterpret_cast<uint2*>(dkd + 16 * hf) = pack4<T>(dka[hf] * scale);
    *reinterpret_cast<uint2*>(dvd + 16 * hf) = pack4<T>(dva[hf]);
  }
}

template <typename T, bool S>
hipError_t fwd_t(int B, int N, int H, float scale, const void* q, const void* k, const void* v,
                 const int32_t* q_idx, const int32_t* key_idx, void* o, float* lse,
                 hipStream_t st) {
  const int HP = (H + 1) / 2;
  const int64_t items = (int64_t)B * (N / CS) * HP;
  const int64_t wgs = (items + kWaves - 1) / kWaves;
  hipLaunchKernelGGL((fwd_mfma_kernel<T, S>), dim3((unsigned)wgs), dim3(64 * kWaves), 0, st, N, H,
                     HP, items, scale * kLog2e, (const T*)q, (const T*)k, (const T*)v, q_idx,
                     key_idx, (T*)o, lse);
  return hipGetLastError();
}

template <typename T, bool S>
hipError_t bwd_t(int B, int N, int H, int nk, float scale, const void* q, const void* k,
                 const void* v, const void* o, const void* dout, const float* lse,
                 const int32_t* q_idx, const int32_t* key_idx, void* dq, void* dk, void* dv,
                 const BwdWorkspace& w, hipStream_t st) {
  const int HP = (H + 1) / 2;
  const int64_t items = (int64_t)B * (N / CS) * HP;
  const int64_t wgs = (items + kWaves - 1) / kWaves;
  hipLaunchKernelGGL((bwd_q_mfma_kernel<T, S>), dim3((unsigned)wgs), dim3(64 * kWaves), 0, st, N,
                     H, HP, items, scale, (const T*)q, (const T*)k, (const T*)v, (const T*)o,
                     (const T*)dout, lse, q_idx, key_idx, (T*)dq, w.delta);
  hipLaunchKernelGGL((bwd_kv_mfma_kernel<T, S>), dim3((unsigned)wgs), dim3(64 * kWaves), 0, st, N,
                     H, HP, items, scale, (const T*)q, (const T*)k, (const T*)v, (const T*)dout,
                     lse, q_idx, (const float*)w.delta, (const int32_t*)w.off,
                     (const RevEntry*)w.rev, nk, (T*)dk, (T*)dv);
  return hipGetLastError();
}

}  // namespace

bool mfma_supported(int dt, int nk) { return (dt == 1 || dt == 2) && nk == NK; }

hipError_t launch_fwd_mfma(int dt, int B, int N, int H, float scale, const void* q, const void* k,
                           const void* v, const int32_t* q_idx, const int32_t* key_idx, void* o,
                           float* lse, hipStream_t st) {
  if (dt == 1) return fwd_t<bf16, true>(B, N, H, scale, q, k, v, q_idx, key_idx, o, lse, st);
  if (dt == 2) return fwd_t<f16, true>(B, N, H, scale, q, k, v, q_idx, key_idx, o, lse, st);
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_mfma(int dt, int B, int N, int H, int nk, float scale, const void* q,
                           const void* k, const void* v, const void* o, const void* dout,
                           const float* lse, const int32_t* q_idx, const int32_t* key_idx,
                           void* dq, void* dk, void* dv, const BwdWorkspace& w, hipStream_t st) {
  if (dt == 1)
    return bwd_t<bf16, true>(B, N, H, nk, scale, q, k, v, o, dout, lse, q_idx, key_idx, dq, dk, dv,
                             w, st);
  if (dt == 2)
    return bwd_t<f16, true>(B, N, H, nk, scale, q, k, v, o, dout, lse, q_idx, key_idx, dq, dk, dv,
                            w, st);
  return hipErrorInvalidValue;
}

}  // namespace ca
