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
//    16x16 fp32 result puts rows 4g..4g+3 of column c in lane l.  Only this
//    one MFMA shape is used: chaining it with 16x16x16 accumulations gave
//    wrong results on this target, so 16-deep products are run on it with
//    the upper half of every lane's reduction slice zeroed.
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
//    (x = hi + lo to ~16 bits) so their rounding stays far below the
//    output rounding.
//  * Gathers are 16-byte loads addressed by 32-bit byte offsets from the
//    tensor base; per-item indices are wave-uniform and live in scalar
//    registers.  Workgroups of 4 wavefronts are remapped so that each XCD
//    (eight, dispatched round-robin) walks one contiguous Morton range of
//    clusters: neighbouring clusters share their gathered rows in its L2.
#include "common.h"

#include <algorithm>

namespace ca {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int D = 32;
constexpr int CS = 8;
constexpr int NK = 48;
constexpr int kWaves = 4;
constexpr uint32_t kRow = D * 2;   // bytes of one head row (bf16 / fp16)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <typename T> struct Mfma;

template <> struct Mfma<bf16> {
  typedef __bf16 v8 __attribute__((ext_vector_type(8)));
  typedef __bf16 v2 __attribute__((ext_vector_type(2)));
  static constexpr uint32_t kOne = 0x3F80u;
  static __device__ __forceinline__ f32x4 mma(uint4 a, uint4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8, a),
                                                   __builtin_bit_cast(v8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x2 unpack(uint32_t w) {
    return f32x2{__uint_as_float(w << 16), __uint_as_float(w & 0xFFFF0000u)};
  }
};

template <> struct Mfma<f16> {
  typedef _Float16 v8 __attribute__((ext_vector_type(8)));
  typedef _Float16 v2 __attribute__((ext_vector_type(2)));
  static constexpr uint32_t kOne = 0x3C00u;
  static __device__ __forceinline__ f32x4 mma(uint4 a, uint4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8, a),
                                                  __builtin_bit_cast(v8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x2 unpack(uint32_t w) {
    return __builtin_convertvector(__builtin_bit_cast(v2, w), f32x2);
  }
};

// two floats -> one dword of T (round to nearest even, one instruction)
template <typename T>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{a, b}), typename Mfma<T>::v2));
}

template <typename T>
__device__ __forceinline__ uint2 pack4(f32x4 x) {
  return make_uint2(pack2<T>(x[0], x[1]), pack2<T>(x[2], x[3]));
}

// x ~= hi + lo with hi = T(x) and lo = T(x - hi), for 4 floats
template <typename T>
__device__ __forceinline__ void split4(const float (&x)[4], uint2& hi, uint2& lo) {
  hi = make_uint2(pack2<T>(x[0], x[1]), pack2<T>(x[2], x[3]));
  const f32x2 a = Mfma<T>::unpack(hi.x), b = Mfma<T>::unpack(hi.y);
  lo = make_uint2(pack2<T>(x[0] - a[0], x[1] - a[1]), pack2<T>(x[2] - b[0], x[3] - b[1]));
}

__device__ __forceinline__ uint4 cat(uint2 a, uint2 b) { return make_uint4(a.x, a.y, b.x, b.y); }
__device__ __forceinline__ uint4 pad(uint2 a) { return make_uint4(a.x, a.y, 0u, 0u); }
__device__ __forceinline__ uint4 sel(bool c, uint4 a) {
  return c ? a : make_uint4(0u, 0u, 0u, 0u);
}

// 16-byte load at a 32-bit byte offset from a (wave-uniform) base pointer
__device__ __forceinline__ uint4 ld16(const void* base, uint32_t off) {
  return *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(base) + off);
}
template <typename V>
__device__ __forceinline__ void stv(void* base, uint32_t off, V v) {
  *reinterpret_cast<V*>(reinterpret_cast<char*>(base) + off) = v;
}

// 0/1 selection matrix as a B operand: B[k][c] = (k == c + 16 * half), the
// reduction index k = 8g + e of element e in lane group g.
template <typename T>
__device__ __forceinline__ uint4 selector(int g, int c16, int half) {
  uint32_t w[4];
#pragma unroll
  for (int e2 = 0; e2 < 4; ++e2) {
    const uint32_t lo = (8 * g + 2 * e2 == c16 + 16 * half) ? Mfma<T>::kOne : 0u;
    const uint32_t hi = (8 * g + 2 * e2 + 1 == c16 + 16 * half) ? Mfma<T>::kOne : 0u;
    w[e2] = lo | (hi << 16);
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// Transpose a 16-row x 32-dim A-operand tile (lane c16+16g holds row c16,
// dims [8g, 8g+8)) into two halves usable as A operands over rows: out[h]
// holds rows 4g..4g+3 of dim c16 + 16h (packed to T).
template <typename T>
__device__ __forceinline__ void transpose_rows(uint4 rows, const uint4 (&id)[2], uint2 (&out)[2]) {
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) out[hf] = pack4<T>(Mfma<T>::mma(rows, id[hf], z));
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

// wave-uniform item index of this wavefront (scalar register)
__device__ __forceinline__ int wave_item() {
  const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  return xcd_remap(blockIdx.x, gridDim.x) * kWaves + w;
}

// ---------------------------------------------------------------------------
// forward
// ---------------------------------------------------------------------------
// A wavefront walks `ipw` consecutive items (cluster, head pair) as a
// software pipeline: the indices of item t+2 and the gathered rows of item
// t+1 are in flight while item t is computed, so the two dependent memory
// round trips (list, then rows) overlap the math of earlier items.
struct FwdIdx {
  int bc, h0;        // wave-uniform
  int kt[3];         // key token of A-row c16 in each 16-slot block
  int qtok;          // query token of column c16
};

template <typename T>
struct FwdData {
  uint4 qv;
  uint4 ka[3][2], va[3][2];
  uint32_t valid[3];
};

__device__ __forceinline__ void fwd_load_idx(int item, int HP, const int32_t* __restrict__ q_idx,
                                             const int32_t* __restrict__ key_idx, int c16,
                                             FwdIdx& x) {
  x.bc = item / HP;
  x.h0 = 2 * (item - x.bc * HP);
#pragma unroll
  for (int b = 0; b < 3; ++b) x.kt[b] = key_idx[x.bc * NK + 16 * b + c16];
  x.qtok = q_idx[x.bc * CS + (c16 & 7)];
}

template <typename T>
__device__ __forceinline__ void fwd_load_rows(const FwdIdx& x, int N, int H, const T* __restrict__ q,
                                              const T* __restrict__ k, const T* __restrict__ v,
                                              int c16, int g, FwdData<T>& d) {
  const int img = x.bc / (N / CS) * N;
  const bool left = c16 < 8;
  const int hq = left ? x.h0 : x.h0 + 1;
  const bool h1ok = x.h0 + 1 < H;
  const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
  const uint32_t lo16 = 16u * g;
  d.qv = (hq < H) ? ld16(q, (uint32_t)((img + x.qtok) * H + hq) * kRow + lo16) : zero;
#pragma unroll
  for (int b = 0; b < 3; ++b) {
    d.valid[b] = (uint32_t)__ballot(x.kt[b] >= 0) & 0xFFFFu;
    const uint32_t r = (uint32_t)((img + max(x.kt[b], 0)) * H + x.h0) * kRow + lo16;
    d.ka[b][0] = ld16(k, r);
    d.va[b][0] = ld16(v, r);
    d.ka[b][1] = h1ok ? ld16(k, r + kRow) : zero;
    d.va[b][1] = h1ok ? ld16(v, r + kRow) : zero;
  }
}

template <typename T>
__device__ __forceinline__ void fwd_compute(const FwdIdx& x, const FwdData<T>& d, int N, int H,
                                            float scale_log2, const uint4 (&id)[2], int c16, int g,
                                            T* __restrict__ o, float* __restrict__ lse) {
  const int img = x.bc / (N / CS) * N;
  const bool left = c16 < 8;
  const int h0 = x.h0, hq = left ? h0 : h0 + 1;
  const bool h1ok = h0 + 1 < H;

  // S^T = K Q^T, lane holds keys 16b+4g+i of column c16
  const uint4 qL = sel(left, d.qv), qR = sel(!left, d.qv);
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  float xs[3][4];
  float mx = -INFINITY;
#pragma unroll
  for (int b = 0; b < 3; ++b) {
    f32x4 s = Mfma<T>::mma(d.ka[b][0], qL, z);
    if (h1ok) s = Mfma<T>::mma(d.ka[b][1], qR, s);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      xs[b][i] = ((d.valid[b] >> (4 * g + i)) & 1u) ? s[i] * scale_log2 : -INFINITY;
      mx = fmaxf(mx, xs[b][i]);
    }
  }
  mx = shfl_max16_32(mx);
  const float mref = mx == -INFINITY ? 0.f : mx;
  float l = 0.f;
#pragma unroll
  for (int b = 0; b < 3; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      xs[b][i] = __builtin_amdgcn_exp2f(xs[b][i] - mref);
      l += xs[b][i];
    }
  l = shfl_sum16_32(l);

  // P as B operands over keys: step 0 = blocks 0,1 (32 keys), step 1 = block 2
  uint2 ph[3], pl[3];
#pragma unroll
  for (int b = 0; b < 3; ++b) split4<T>(xs[b], ph[b], pl[b]);

  // V^T tiles via the selection matrix, then O^T = V^T P^T
  f32x4 oacc[2] = {z, z};
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    if (hh == 1 && !h1ok) break;
    const bool mine = (hh == 0) == left;   // this head's columns
    uint2 vt[3][2];
#pragma unroll
    for (int b = 0; b < 3; ++b) transpose_rows<T>(d.va[b][hh], id, vt[b]);
    const uint4 b0h = sel(mine, cat(ph[0], ph[1])), b0l = sel(mine, cat(pl[0], pl[1]));
    const uint4 b1h = sel(mine, pad(ph[2])), b1l = sel(mine, pad(pl[2]));
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const uint4 a01 = cat(vt[0][hf], vt[1][hf]), a2 = pad(vt[2][hf]);
      oacc[hf] = Mfma<T>::mma(a01, b0h, oacc[hf]);
      oacc[hf] = Mfma<T>::mma(a2, b1h, oacc[hf]);
      oacc[hf] = Mfma<T>::mma(a01, b0l, oacc[hf]);
      oacc[hf] = Mfma<T>::mma(a2, b1l, oacc[hf]);
    }
  }

  if (hq >= H) return;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const uint32_t orow = (uint32_t)((img + x.qtok) * H + hq) * kRow + 8u * g;
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) stv<uint2>(o, orow + 32u * hf, pack4<T>(oacc[hf] * inv));
  if (g == 0) lse[(img + x.qtok) * H + hq] = l > 0.f ? (mx + __log2f(l)) * kLn2 : -INFINITY;
}

template <typename T>
__global__ void __launch_bounds__(64 * kWaves)
fwd_mfma_kernel(int N, int H, int HP, int n_items, int ipw, float scale_log2,
                const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
                const int32_t* __restrict__ q_idx, const int32_t* __restrict__ key_idx,
                T* __restrict__ o, float* __restrict__ lse) {
  const int first = wave_item() * ipw;
  if (first >= n_items) return;
  const int last = min(first + ipw, n_items);
  const int lane = threadIdx.x & 63;
  const int c16 = lane & 15, g = lane >> 4;
  uint4 id[2];
  id[0] = selector<T>(g, c16, 0);
  id[1] = selector<T>(g, c16, 1);

  FwdIdx xi, xn, xnn;
  FwdData<T> di, dn;
  fwd_load_idx(first, HP, q_idx, key_idx, c16, xi);
  fwd_load_rows<T>(xi, N, H, q, k, v, c16, g, di);
  if (first + 1 < last) fwd_load_idx(first + 1, HP, q_idx, key_idx, c16, xn);
  for (int it = first; it < last; ++it) {
    if (it + 1 < last) {
      fwd_load_rows<T>(xn, N, H, q, k, v, c16, g, dn);
      if (it + 2 < last) fwd_load_idx(it + 2, HP, q_idx, key_idx, c16, xnn);
    }
    fwd_compute<T>(xi, di, N, H, scale_log2, id, c16, g, o, lse);
    xi = xn;
    di = dn;
    xn = xnn;
  }
}

// ---------------------------------------------------------------------------
// backward pass A (query-major): Delta and dQ
// ---------------------------------------------------------------------------
template <typename T>
__global__ void __launch_bounds__(64 * kWaves)
bwd_q_mfma_kernel(int N, int H, int HP, int n_items, float scale, const T* __restrict__ q,
                  const T* __restrict__ k, const T* __restrict__ v, const T* __restrict__ o,
                  const T* __restrict__ dout, const float* __restrict__ lse,
                  const int32_t* __restrict__ q_idx, const int32_t* __restrict__ key_idx,
                  T* __restrict__ dq, float2* __restrict__ ld) {
  const int item = wave_item();
  if (item >= n_items) return;
  const int lane = threadIdx.x & 63;
  const int bc = item / HP;
  const int h0 = 2 * (item - bc * HP), h1 = h0 + 1;
  const int img = bc / (N / CS) * N;
  const int c16 = lane & 15, g = lane >> 4;
  const bool left = c16 < 8;
  const int hq = left ? h0 : h1;
  const bool h1ok = h1 < H, qok = hq < H;
  const float scale_log2 = scale * kLog2e;
  const uint4 zero = make_uint4(0u, 0u, 0u, 0u);

  int kt[3];
  uint32_t valid[3];
#pragma unroll
  for (int b = 0; b < 3; ++b) {
    kt[b] = key_idx[bc * NK + 16 * b + c16];
    valid[b] = (uint32_t)__ballot(kt[b] >= 0) & 0xFFFFu;
    kt[b] = max(kt[b], 0);
  }
  const int qtok = q_idx[bc * CS + (c16 & 7)];
  const uint32_t lo16 = 16u * g;
  const int qh = (img + qtok) * H + hq;
  const uint32_t qrow = (uint32_t)qh * kRow + lo16;
  const uint4 qv = qok ? ld16(q, qrow) : zero;
  const uint4 dov = qok ? ld16(dout, qrow) : zero;
  const uint4 ov = qok ? ld16(o, qrow) : zero;
  const float lse2 = qok ? lse[qh] * kLog2e : 0.f;
  uint4 ka[3][2], va[3][2];
#pragma unroll
  for (int b = 0; b < 3; ++b) {
    const uint32_t r = (uint32_t)((img + kt[b]) * H + h0) * kRow + lo16;
    ka[b][0] = ld16(k, r);
    va[b][0] = ld16(v, r);
    ka[b][1] = h1ok ? ld16(k, r + kRow) : zero;
    va[b][1] = h1ok ? ld16(v, r + kRow) : zero;
  }

  // Delta = <dO, O> per (query, head) column; stored with LSE for pass B
  float dl = 0.f;
  {
    const uint32_t a[4] = {dov.x, dov.y, dov.z, dov.w};
    const uint32_t c[4] = {ov.x, ov.y, ov.z, ov.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const f32x2 x = Mfma<T>::unpack(a[e]), y = Mfma<T>::unpack(c[e]);
      dl = fmaf(x[0], y[0], fmaf(x[1], y[1], dl));
    }
  }
  dl = shfl_sum16_32(dl);
  if (qok && g == 0) ld[qh] = make_float2(lse2, dl);

  const uint4 qL = sel(left, qv), qR = sel(!left, qv);
  const uint4 dL = sel(left, dov), dR = sel(!left, dov);
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  float ds[3][4];
#pragma unroll
  for (int b = 0; b < 3; ++b) {
    f32x4 s = Mfma<T>::mma(ka[b][0], qL, z);
    f32x4 dp = Mfma<T>::mma(va[b][0], dL, z);
    if (h1ok) {
      s = Mfma<T>::mma(ka[b][1], qR, s);
      dp = Mfma<T>::mma(va[b][1], dR, dp);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool ok = (valid[b] >> (4 * g + i)) & 1u;
      const float p = ok ? __builtin_amdgcn_exp2f(fmaf(s[i], scale_log2, -lse2)) : 0.f;
      ds[b][i] = p * (dp[i] - dl);
    }
  }
  uint2 dh[3], dlo[3];
#pragma unroll
  for (int b = 0; b < 3; ++b) split4<T>(ds[b], dh[b], dlo[b]);

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
    const uint4 b0h = sel(mine, cat(dh[0], dh[1])), b0l = sel(mine, cat(dlo[0], dlo[1]));
    const uint4 b1h = sel(mine, pad(dh[2])), b1l = sel(mine, pad(dlo[2]));
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const uint4 a01 = cat(ktt[0][hf], ktt[1][hf]), a2 = pad(ktt[2][hf]);
      acc[hf] = Mfma<T>::mma(a01, b0h, acc[hf]);
      acc[hf] = Mfma<T>::mma(a2, b1h, acc[hf]);
      acc[hf] = Mfma<T>::mma(a01, b0l, acc[hf]);
      acc[hf] = Mfma<T>::mma(a2, b1l, acc[hf]);
    }
  }
  if (!qok) return;
  const uint32_t drow = (uint32_t)qh * kRow + 8u * g;
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) stv<uint2>(dq, drow + 32u * hf, pack4<T>(acc[hf] * scale));
}

// ---------------------------------------------------------------------------
// backward pass B (key-major): dK and dV over the transposed lists
// ---------------------------------------------------------------------------
// Each iteration takes 4 referencing clusters (32 query rows in two 16-row
// blocks): S = Q K_j^T and dP = dO V_j^T per block, then dV^T += dO^T P and
// dK^T += Q^T dS with the 32 rows as one reduction.
template <typename T>
__global__ void __launch_bounds__(64 * kWaves)
bwd_kv_mfma_kernel(int N, int H, int HP, int n_items, float scale, const T* __restrict__ q,
                   const T* __restrict__ k, const T* __restrict__ v, const T* __restrict__ dout,
                   const int32_t* __restrict__ q_idx, const float2* __restrict__ ld,
                   const int32_t* __restrict__ off_all, const RevEntry* __restrict__ rev_all,
                   int nk, T* __restrict__ dk, T* __restrict__ dv) {
  const int item = wave_item();
  if (item >= n_items) return;
  const int lane = threadIdx.x & 63;
  const int C = N / CS;
  const int bj = item / HP;
  const int h0 = 2 * (item - bj * HP), h1 = h0 + 1;
  const int b = bj / C;
  const int j = bj - b * C;
  const int img = b * N;
  const int c16 = lane & 15, g = lane >> 4;
  const bool left = c16 < 8;
  const int hk = left ? h0 : h1;
  const bool h1ok = h1 < H, kok = hk < H;
  const float scale_log2 = scale * kLog2e;
  const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
  const uint32_t lo16 = 16u * g;

  // own key rows as B operands (column c16 = key c16&7 of head hk)
  const int ktok = q_idx[bj * CS + (c16 & 7)];
  const int kh = (img + ktok) * H + hk;
  const uint32_t krow = (uint32_t)kh * kRow + lo16;
  const uint4 kB = kok ? ld16(k, krow) : zero;
  const uint4 vB = kok ? ld16(v, krow) : zero;
  const uint4 kL = sel(left, kB), kR = sel(!left, kB);
  const uint4 vL = sel(left, vB), vR = sel(!left, vB);

  const int32_t* off = off_all + b * (C + 1);
  const RevEntry* rev = rev_all + (int64_t)b * C * nk;
  const int e0 = off[j], e1 = off[j + 1];

  uint4 id[2];
  id[0] = selector<T>(g, c16, 0);
  id[1] = selector<T>(g, c16, 1);
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  f32x4 dka[2] = {z, z}, dva[2] = {z, z};
  const int kcol = c16 & 7;

  for (int e = e0; e < e1; e += 4) {
    // the (up to) 4 entries of this step, wave-uniform
    int ei[4];
    uint64_t em[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const RevEntry r = rev[min(e + u, e1 - 1)];
      ei[u] = r.i;
      em[u] = e + u < e1 ? r.mult : 0ull;
    }
    uint4 qa[2][2], da[2][2];
    float p[2][4], ds[2][4];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      // A-operand row c16 = query c16&7 of entry 2qb + (c16>>3)
      const int ea = (c16 >> 3) ? ei[2 * qb + 1] : ei[2 * qb];
      const int qtok = q_idx[(b * C + ea) * CS + (c16 & 7)];
      const uint32_t r = (uint32_t)((img + qtok) * H + h0) * kRow + lo16;
      qa[qb][0] = ld16(q, r);
      da[qb][0] = ld16(dout, r);
      qa[qb][1] = h1ok ? ld16(q, r + kRow) : zero;
      da[qb][1] = h1ok ? ld16(dout, r + kRow) : zero;
      // this lane's output rows 4g..4g+3 belong to entry 2qb + (g>>1)
      const uint64_t m64 = (g >> 1) ? em[2 * qb + 1] : em[2 * qb];
      const float mult = kok ? (float)((m64 >> (8 * kcol)) & 0xFFu) : 0.f;
      float2 lds[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = __shfl(qtok, 4 * g + i, 64);   // query of row 4g+i
        lds[i] = mult != 0.f ? ld[(img + t) * H + hk] : make_float2(0.f, 0.f);
      }
      f32x4 s = Mfma<T>::mma(qa[qb][0], kL, z);
      f32x4 dp = Mfma<T>::mma(da[qb][0], vL, z);
      if (h1ok) {
        s = Mfma<T>::mma(qa[qb][1], kR, s);
        dp = Mfma<T>::mma(da[qb][1], vR, dp);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[qb][i] = mult != 0.f ? mult * __builtin_amdgcn_exp2f(fmaf(s[i], scale_log2, -lds[i].x)) : 0.f;
        ds[qb][i] = p[qb][i] * (dp[i] - lds[i].y);
      }
    }
    uint2 ph[2], pl[2], dh[2], dlo[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      split4<T>(p[qb], ph[qb], pl[qb]);
      split4<T>(ds[qb], dh[qb], dlo[qb]);
    }
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      if (hh == 1 && !h1ok) break;
      const bool mine = (hh == 0) == left;
      uint2 dot[2][2], qt[2][2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        transpose_rows<T>(da[qb][hh], id, dot[qb]);
        transpose_rows<T>(qa[qb][hh], id, qt[qb]);
      }
      const uint4 bph = sel(mine, cat(ph[0], ph[1])), bpl = sel(mine, cat(pl[0], pl[1]));
      const uint4 bdh = sel(mine, cat(dh[0], dh[1])), bdl = sel(mine, cat(dlo[0], dlo[1]));
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const uint4 ad = cat(dot[0][hf], dot[1][hf]), aq = cat(qt[0][hf], qt[1][hf]);
        dva[hf] = Mfma<T>::mma(ad, bph, dva[hf]);
        dva[hf] = Mfma<T>::mma(ad, bpl, dva[hf]);
        dka[hf] = Mfma<T>::mma(aq, bdh, dka[hf]);
        dka[hf] = Mfma<T>::mma(aq, bdl, dka[hf]);
      }
    }
  }

  if (!kok) return;
  const uint32_t orow = (uint32_t)kh * kRow + 8u * g;
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    stv<uint2>(dk, orow + 32u * hf, pack4<T>(dka[hf] * scale));
    stv<uint2>(dv, orow + 32u * hf, pack4<T>(dva[hf]));
  }
}

// Items per wavefront: enough wavefronts to give every SIMD of the 256 CUs
// about four, each pipelining its run of consecutive items.
int items_per_wave(int items) {
  constexpr int kTargetWaves = 256 * 4 * 4;
  return std::max(1, std::min(8, (items + kTargetWaves - 1) / kTargetWaves));
}

template <typename T>
hipError_t fwd_t(int B, int N, int H, float scale, const void* q, const void* k, const void* v,
                 const int32_t* q_idx, const int32_t* key_idx, void* o, float* lse,
                 hipStream_t st) {
  const int HP = (H + 1) / 2;
  const int items = B * (N / CS) * HP;
  const int ipw = items_per_wave(items);
  const int waves = (items + ipw - 1) / ipw;
  const int wgs = (waves + kWaves - 1) / kWaves;
  hipLaunchKernelGGL((fwd_mfma_kernel<T>), dim3(wgs), dim3(64 * kWaves), 0, st, N, H, HP, items,
                     ipw, scale * kLog2e, (const T*)q, (const T*)k, (const T*)v, q_idx, key_idx,
                     (T*)o, lse);
  return hipGetLastError();
}

template <typename T>
hipError_t bwd_t(int B, int N, int H, int nk, float scale, const void* q, const void* k,
                 const void* v, const void* o, const void* dout, const float* lse,
                 const int32_t* q_idx, const int32_t* key_idx, void* dq, void* dk, void* dv,
                 const BwdWorkspace& w, hipStream_t st) {
  const int HP = (H + 1) / 2;
  const int items = B * (N / CS) * HP;
  const int wgs = (items + kWaves - 1) / kWaves;
  hipLaunchKernelGGL((bwd_q_mfma_kernel<T>), dim3(wgs), dim3(64 * kWaves), 0, st, N, H, HP, items,
                     scale, (const T*)q, (const T*)k, (const T*)v, (const T*)o, (const T*)dout, lse,
                     q_idx, key_idx, (T*)dq, w.ld);
  hipLaunchKernelGGL((bwd_kv_mfma_kernel<T>), dim3(wgs), dim3(64 * kWaves), 0, st, N, H, HP, items,
                     scale, (const T*)q, (const T*)k, (const T*)v, (const T*)dout, q_idx,
                     (const float2*)w.ld, (const int32_t*)w.off, (const RevEntry*)w.rev, nk, (T*)dk,
                     (T*)dv);
  return hipGetLastError();
}

}  // namespace

bool mfma_supported(int dt, int B, int N, int H, int nk) {
  // 32-bit byte offsets and item counts
  const int64_t bytes = (int64_t)B * N * H * D * 2;
  const int64_t items = (int64_t)B * (N / CS) * ((H + 1) / 2);
  return (dt == 1 || dt == 2) && nk == NK && bytes < (int64_t(1) << 31) &&
         items < (int64_t(1) << 30);
}

hipError_t launch_fwd_mfma(int dt, int B, int N, int H, float scale, const void* q, const void* k,
                           const void* v, const int32_t* q_idx, const int32_t* key_idx, void* o,
                           float* lse, hipStream_t st) {
  if (dt == 1) return fwd_t<bf16>(B, N, H, scale, q, k, v, q_idx, key_idx, o, lse, st);
  if (dt == 2) return fwd_t<f16>(B, N, H, scale, q, k, v, q_idx, key_idx, o, lse, st);
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_mfma(int dt, int B, int N, int H, int nk, float scale, const void* q,
                           const void* k, const void* v, const void* o, const void* dout,
                           const float* lse, const int32_t* q_idx, const int32_t* key_idx,
                           void* dq, void* dk, void* dv, const BwdWorkspace& w, hipStream_t st) {
  if (dt == 1)
    return bwd_t<bf16>(B, N, H, nk, scale, q, k, v, o, dout, lse, q_idx, key_idx, dq, dk, dv, w,
                       st);
  if (dt == 2)
    return bwd_t<f16>(B, N, H, nk, scale, q, k, v, o, dout, lse, q_idx, key_idx, dq, dk, dv, w,
                      st);
  return hipErrorInvalidValue;
}

}  // namespace ca
