// Window-tiled matrix-core cluster attention for gfx950 (bf16 / fp16).
//
// What is computed: the local cluster attention of the English notes page
// "AFFMAE: Scalable Vision Pre-Training for High-Resolution Microscopy
// Segmentation on Desktop Hardware" ("Overall Architecture"): every query
// cluster attends, with a plain scaled-dot-product softmax, to the key slots
// of its list; forward (O, LSE) and backward (dQ, dK, dV).  The arXiv abstract
// of the same paper asks for numerically stable, mixed-precision,
// Flash-style kernels: bf16/fp16 operands, fp32 statistics and accumulation,
// an online (running-max) softmax, logits in log2 units.
//
// Structure (one workgroup of two wavefronts per tile = (window, head)):
//  * A window is 8 consecutive clusters (64 query rows); the plan of
//    tile_plan.hip lists the distinct key tokens of their lists (u of them,
//    about 144 at the stage-1 shape against 384 slots) and how many slots of
//    each cluster hold each key.  The workgroup stages the window's 64 query
//    rows and the u key rows of one head in LDS with direct-to-LDS loads
//    (four lanes per 64-byte row, whole rows per instruction), then computes
//    the 64 x u logit block densely: S^T = K Q^T on 16x16x32 MFMA tiles with
//    every lane live, the probabilities weighted by the multiplicity (0 masks
//    a key outside a cluster's list; 2 counts a repeated slot twice), and
//    O^T = V^T P^T with V read through the transposing LDS read.  Each
//    wavefront owns 32 query rows and walks the keys 64 at a time with a
//    running maximum and sum (Flash-style), so its registers do not grow with
//    u; unions longer than the staging buffer take several passes.
//  * Query-major backward pass: the same staging plus the rows of dO and O
//    and the LSE; dS = P (dP - Delta), dQ^T = K^T dS^T; writes dQ and
//    (LSE log2 e, Delta) per query row for the key-major pass.
//  * Key-major backward pass: the window's 64 key rows stay in registers;
//    the query clusters reading them (from the plan, ordered by cluster,
//    with a 64-byte multiplicity row each) stream through LDS 24 at a time;
//    S = Q K^T, dP = dO V^T, dV^T += dO^T P, dK^T += Q^T dS.  Each dK/dV row
//    is written once by one workgroup: no atomics, bitwise reproducible.
//  * Row r of a staged block keeps 16-byte chunk c at position c ^ sw(r), a
//    swizzle under which both the MFMA row reads (16 rows, one chunk) and the
//    transposing reads (4 rows, two chunks) spread over all LDS banks.
//  * Workgroups are numbered so that each XCD takes a contiguous range of
//    windows (all heads): the key rows shared by neighbouring windows and
//    the heads of one token row stay in that XCD's L2.
#include "common.h"
#include "mfma_util.h"

namespace ca {

namespace {

constexpr int kTThreads = 128;   // two wavefronts per tile
constexpr uint32_t kRowB = 64;   // bytes of one head row
constexpr float kLog2eT = 1.4426950408889634f;
constexpr float kLn2T = 0.6931471805599453f;

__device__ __forceinline__ uint32_t sw(int r) {
  return (uint32_t)(((((r >> 1) ^ (r >> 2)) & 1) << 1) | (((r >> 1) ^ (r >> 3)) & 1));
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)p;
}

// byte offset of chunk position `pos` of row `r` of a staged block
__device__ __forceinline__ uint32_t row_chunk(int r, uint32_t chunk) {
  return (uint32_t)r * kRowB + 16u * (chunk ^ sw(r));
}

constexpr int kRecBytes = 4 * kQRecHead + 12 * 512;   // a query record, nk <= 64

// Direct-to-LDS copy of `bytes` (a multiple of 16) contiguous bytes, split
// over the workgroup's two wavefronts (instruction i by wavefront i & 1).
__device__ __forceinline__ void copy_lds(const void* src, uint32_t src_off, int bytes, uint32_t dst,
                                         int lane, int wv) {
  const int n16 = bytes >> 4;
  for (int i = wv; 64 * i < n16; i += 2) {
    const int p = 64 * i + lane;
    if (p < n16) dma16(src, src_off + 16u * (uint32_t)p, dst + 1024u * (uint32_t)i);
  }
}

// Gather the head-h rows of up to 64 tokens (`nrows` a multiple of 16) into a
// staged block: instruction i fills rows 16 i .. 16 i + 15 (wavefront wv
// issues i = wv and wv + 2); lane l fetches chunk (l & 3) ^ sw(row) of row
// 16 i + l / 4, so that position l & 3 of the row holds it.  `toks` (LDS):
// the row tokens, -1 taking `fallback`.
__device__ __forceinline__ void gather64(const void* src, const int32_t* toks, int fallback,
                                         int nrows, uint32_t dst, int base, int H, int h,
                                         int lane, int wv) {
  const int r0 = 16 * wv + (lane >> 2), r1 = r0 + 32;
  int t0 = r0 < nrows ? toks[r0] : fallback;
  int t1 = r1 < nrows ? toks[r1] : fallback;
  t0 = t0 < 0 ? fallback : t0;
  t1 = t1 < 0 ? fallback : t1;
  const uint32_t c0 = (uint32_t)(lane & 3) ^ sw(r0), c1 = (uint32_t)(lane & 3) ^ sw(r1);
  if (16 * wv < nrows)
    dma16(src, ((uint32_t)(base + t0) * (uint32_t)H + (uint32_t)h) * kRowB + 16u * c0,
          dst + 1024u * (uint32_t)wv);
  if (16 * wv + 32 < nrows)
    dma16(src, ((uint32_t)(base + t1) * (uint32_t)H + (uint32_t)h) * kRowB + 16u * c1,
          dst + 1024u * (uint32_t)(wv + 2));
}

// four multiplicity bytes -> floats
__device__ __forceinline__ float mbyte(uint32_t w, int i) {
  return (float)((w >> (8 * i)) & 0xffu);
}

// A operands of a 16-row block read transposed: lane 4e + qq of row group g
// receives dim 16 hf + (lane & 15) of rows r0 + 4 g + e and r0 + 16 + 4 g + e
__device__ __forceinline__ uint4 tr_pair(const char* blk, int r0, int hf, int g, int e, int qq) {
  const uint32_t c = (uint32_t)(2 * hf + (qq >> 1));
  const int ra = r0 + 4 * g + e, rb = ra + 16;
  return cat(lds_tr8(blk, row_chunk(ra, c) + 8u * (qq & 1)),
             lds_tr8(blk, row_chunk(rb, c) + 8u * (qq & 1)));
}

// ---------------------------------------------------------------------------
// forward
// ---------------------------------------------------------------------------
// Per tile: the query record (flat copy), the 64 query rows, then the key
// rows of the window's union streamed 64 at a time through two buffers: the
// next chunk's gathers are issued before the current chunk is computed.
struct FwdLds {
  static constexpr int kRec = 0, kQ = kRecBytes, kKv = kQ + 4096,
                       kBytes = kKv + 2 * 8192;   // per buffer: K 4 KiB then V 4 KiB
};

template <typename T, int NB>
__device__ __forceinline__ void fwd_step(const char* kbuf, const char* vbuf, const uint8_t* mt,
                                         int kmax, int col0, const uint4 (&qv)[2],
                                         const int (&cl)[2], float scale_log2, float (&mrun)[2],
                                         float (&lrun)[2], f32x4 (&oacc)[2][2], int c16, int g,
                                         int e, int qq) {
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  uint4 ka[NB];
#pragma unroll
  for (int kb = 0; kb < NB; ++kb) ka[kb] = lds16(kbuf, row_chunk(16 * kb + c16, (uint32_t)g));
  uint4 vt[NB / 2][2];
#pragma unroll
  for (int kg = 0; kg < NB / 2; ++kg)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) vt[kg][hf] = tr_pair(vbuf, 32 * kg, hf, g, e, qq);
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    f32x4 s[NB];
    uint32_t mw[NB];
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) {
      s[kb] = Mfma<T>::mma(ka[kb], qv[cb], z);
      mw[kb] = *reinterpret_cast<const uint32_t*>(mt + cl[cb] * kmax + col0 + 16 * kb + 4 * g);
    }
    float lmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NB; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float t = mbyte(mw[kb], i) != 0.f ? s[kb][i] * scale_log2 : -INFINITY;
        s[kb][i] = t;
        lmax = fmaxf(lmax, t);
      }
    const float mnew = fmaxf(mrun[cb], shfl_max16_32(lmax));
    const float mref = mnew == -INFINITY ? 0.f : mnew;
    const float alpha = __builtin_amdgcn_exp2f(mrun[cb] - mref);
    mrun[cb] = mnew;
    float lsum = 0.f;
#pragma unroll
    for (int kb = 0; kb < NB; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // a masked key has t = -inf, so its term is 0 * 0
        const float p = mbyte(mw[kb], i) * __builtin_amdgcn_exp2f(s[kb][i] - mref);
        s[kb][i] = p;
        lsum += p;
      }
    lrun[cb] = lrun[cb] * alpha + lsum;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) oacc[cb][hf] *= alpha;
#pragma unroll
    for (int kg = 0; kg < NB / 2; ++kg) {
      const uint4 bp = cat(pack4<T>(s[2 * kg]), pack4<T>(s[2 * kg + 1]));
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) oacc[cb][hf] = Mfma<T>::mma(vt[kg][hf], bp, oacc[cb][hf]);
    }
  }
}

template <typename T>
__global__ void __launch_bounds__(kTThreads)
fwd_tile_kernel(int H, int ntiles, int kmax, int qstride, float scale_log2,
                const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
                const int32_t* __restrict__ qrec, T* __restrict__ o, float* __restrict__ lse) {
  typedef FwdLds L;
  __shared__ __attribute__((aligned(1024))) char lds[L::kBytes];
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  if (tile >= ntiles) return;
  const int w = tile / H, h = tile - w * H;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int c16 = lane & 15, g = lane >> 4;
  const int e = c16 >> 2, qq = c16 & 3;
  const int32_t* rec = reinterpret_cast<const int32_t*>(lds + L::kRec);
  const int32_t* ktok = rec + kQRecHead;
  const uint8_t* mt = reinterpret_cast<const uint8_t*>(rec + kQRecHead + kmax);
  const char* sq = lds + L::kQ;

  copy_lds(qrec, (uint32_t)((int64_t)w * qstride * 4), 4 * kQRecHead + 12 * kmax,
           lds_addr(lds + L::kRec), lane, wv);
  wait_vm<0>();
  __syncthreads();
  const int nc = __builtin_amdgcn_readfirstlane(rec[1]);
  const int u = __builtin_amdgcn_readfirstlane(rec[2]);
  const int base = __builtin_amdgcn_readfirstlane(rec[3]);
  const int q0 = __builtin_amdgcn_readfirstlane(rec[4]);
  const int32_t* qtok = rec + 4;
  const int upad = (u + 31) & ~31;
  const int nch = (upad + 63) >> 6;
  if (nch > 0) {
    gather64(q, qtok, q0, 64, lds_addr(sq), base, H, h, lane, wv);
    const int r = min(64, upad);
    gather64(k, ktok, q0, r, lds_addr(lds + L::kKv), base, H, h, lane, wv);
    gather64(v, ktok, q0, r, lds_addr(lds + L::kKv + 4096), base, H, h, lane, wv);
  }
  const bool active = 4 * wv < nc;
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  uint4 qv[2] = {make_uint4(0u, 0u, 0u, 0u), make_uint4(0u, 0u, 0u, 0u)};
  int cl[2];
  float mrun[2] = {-INFINITY, -INFINITY}, lrun[2] = {0.f, 0.f};
  f32x4 oacc[2][2] = {{z, z}, {z, z}};
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) cl[cb] = 4 * wv + 2 * cb + (c16 >> 3);

  for (int c = 0; c < nch; ++c) {
    wait_vm<0>();
    __syncthreads();
    if (c == 0 && active) {
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) qv[cb] = lds16(sq, row_chunk(32 * wv + 16 * cb + c16, (uint32_t)g));
    }
    if (c + 1 < nch) {   // the next chunk's rows land while this one is computed
      const int r = min(64, upad - 64 * (c + 1));
      const uint32_t nb = lds_addr(lds + L::kKv + 8192 * ((c + 1) & 1));
      gather64(k, ktok + 64 * (c + 1), q0, r, nb, base, H, h, lane, wv);
      gather64(v, ktok + 64 * (c + 1), q0, r, nb + 4096u, base, H, h, lane, wv);
    }
    if (!active) continue;
    const char* kb = lds + L::kKv + 8192 * (c & 1);
    if (upad - 64 * c >= 64)
      fwd_step<T, 4>(kb, kb + 4096, mt, kmax, 64 * c, qv, cl, scale_log2, mrun, lrun, oacc, c16, g,
                     e, qq);
    else
      fwd_step<T, 2>(kb, kb + 4096, mt, kmax, 64 * c, qv, cl, scale_log2, mrun, lrun, oacc, c16, g,
                     e, qq);
  }
  if (!active) return;
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const float l = shfl_sum16_32(lrun[cb]);
    const float inv = l > 0.f ? __builtin_amdgcn_rcpf(l) : 0.f;
    const int tq = qtok[32 * wv + 16 * cb + c16];
    if (tq < 0) continue;
    const uint32_t qrow = (uint32_t)(base + tq) * (uint32_t)H + (uint32_t)h;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
      stv<uint2>(o, qrow * kRowB + 32u * hf + 8u * g, pack4<T>(oacc[cb][hf] * inv));
    if (g == 0) lse[qrow] = l > 0.f ? (mrun[cb] + __log2f(l)) * kLn2T : -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// backward, query-major pass: Delta, dQ, and (LSE log2 e, Delta) per row
// ---------------------------------------------------------------------------
struct BqLds {
  static constexpr int kRec = 0, kQ = kRecBytes, kDo = kQ + 4096, kLse = kDo + 4096,
                       kKv = kLse + 256, kBytes = kKv + 2 * 8192;
};

template <typename T, int NB>
__device__ __forceinline__ void bwdq_step(const char* kbuf, const char* vbuf, const uint8_t* mt,
                                          int kmax, int col0, const uint4 (&qv)[2],
                                          const uint4 (&dov)[2], const int (&cl)[2],
                                          const float (&lse2)[2], const float (&dl)[2],
                                          float scale_log2, f32x4 (&acc)[2][2], int c16, int g,
                                          int e, int qq) {
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  uint4 ka[NB], va[NB];
#pragma unroll
  for (int kb = 0; kb < NB; ++kb) {
    ka[kb] = lds16(kbuf, row_chunk(16 * kb + c16, (uint32_t)g));
    va[kb] = lds16(vbuf, row_chunk(16 * kb + c16, (uint32_t)g));
  }
  uint4 kt[NB / 2][2];
#pragma unroll
  for (int kg = 0; kg < NB / 2; ++kg)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) kt[kg][hf] = tr_pair(kbuf, 32 * kg, hf, g, e, qq);
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    f32x4 s[NB];
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) {
      s[kb] = Mfma<T>::mma(ka[kb], qv[cb], z);
      const f32x4 dp = Mfma<T>::mma(va[kb], dov[cb], z);
      const uint32_t mw =
          *reinterpret_cast<const uint32_t*>(mt + cl[cb] * kmax + col0 + 16 * kb + 4 * g);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float m = mbyte(mw, i);
        const float p = m * __builtin_amdgcn_exp2f(fmaf(s[kb][i], scale_log2, -lse2[cb]));
        s[kb][i] = m != 0.f ? p * (dp[i] - dl[cb]) : 0.f;   // dS
      }
    }
#pragma unroll
    for (int kg = 0; kg < NB / 2; ++kg) {
      const uint4 bd = cat(pack4<T>(s[2 * kg]), pack4<T>(s[2 * kg + 1]));
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) acc[cb][hf] = Mfma<T>::mma(kt[kg][hf], bd, acc[cb][hf]);
    }
  }
}

template <typename T>
__global__ void __launch_bounds__(kTThreads)
bwdq_tile_kernel(int H, int ntiles, int kmax, int qstride, float scale,
                 const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
                 const T* __restrict__ o, const T* __restrict__ dout,
                 const float* __restrict__ lse, const int32_t* __restrict__ qrec,
                 T* __restrict__ dq, float2* __restrict__ ld, float4* __restrict__ ld_none) {
  typedef BqLds L;
  __shared__ __attribute__((aligned(1024))) char lds[L::kBytes];
  // the (LSE log2 e, Delta) pair the key-major pass reads for an absent
  // query: P = exp2(s - inf) = 0 there
  if (blockIdx.x == 0 && threadIdx.x == 0) *ld_none = make_float4(INFINITY, 0.f, INFINITY, 0.f);
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  if (tile >= ntiles) return;
  const int w = tile / H, h = tile - w * H;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int c16 = lane & 15, g = lane >> 4;
  const int e = c16 >> 2, qq = c16 & 3;
  const int32_t* rec = reinterpret_cast<const int32_t*>(lds + L::kRec);
  const int32_t* ktok = rec + kQRecHead;
  const uint8_t* mt = reinterpret_cast<const uint8_t*>(rec + kQRecHead + kmax);
  const float* sl = reinterpret_cast<const float*>(lds + L::kLse);
  const char* sq = lds + L::kQ;
  const char* sdo = lds + L::kDo;
  const float scale_log2 = scale * kLog2eT;

  copy_lds(qrec, (uint32_t)((int64_t)w * qstride * 4), 4 * kQRecHead + 12 * kmax,
           lds_addr(lds + L::kRec), lane, wv);
  wait_vm<0>();
  __syncthreads();
  const int nc = __builtin_amdgcn_readfirstlane(rec[1]);
  const int u = __builtin_amdgcn_readfirstlane(rec[2]);
  const int base = __builtin_amdgcn_readfirstlane(rec[3]);
  const int q0 = __builtin_amdgcn_readfirstlane(rec[4]);
  const int32_t* qtok = rec + 4;
  const int upad = (u + 31) & ~31;
  const int nch = (upad + 63) >> 6;
  const bool active = 4 * wv < nc;
  // this lane's O pieces (for Delta) straight into registers: row = query
  // column, 16 bytes of dims 8 g .. 8 g + 7
  uint4 ov[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int tq = qtok[32 * wv + 16 * cb + c16];
    const uint32_t qrow = (uint32_t)(base + (tq < 0 ? q0 : tq)) * (uint32_t)H + (uint32_t)h;
    ov[cb] = ld16(o, qrow * kRowB + 16u * (uint32_t)g);
  }
  gather64(q, qtok, q0, 64, lds_addr(sq), base, H, h, lane, wv);
  gather64(dout, qtok, q0, 64, lds_addr(sdo), base, H, h, lane, wv);
  if (wv == 0) {
    const int t = qtok[lane] < 0 ? q0 : qtok[lane];
    dma4(lse, ((uint32_t)(base + t) * (uint32_t)H + (uint32_t)h) * 4u, lds_addr(sl));
  }
  if (nch > 0) {
    const int r = min(64, upad);
    gather64(k, ktok, q0, r, lds_addr(lds + L::kKv), base, H, h, lane, wv);
    gather64(v, ktok, q0, r, lds_addr(lds + L::kKv + 4096), base, H, h, lane, wv);
  }
  wait_vm<0>();
  __syncthreads();

  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  uint4 qv[2], dov[2];
  int cl[2];
  float lse2[2], dl[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int row = 32 * wv + 16 * cb + c16;
    qv[cb] = lds16(sq, row_chunk(row, (uint32_t)g));
    dov[cb] = lds16(sdo, row_chunk(row, (uint32_t)g));
    cl[cb] = 4 * wv + 2 * cb + (c16 >> 3);
    lse2[cb] = sl[row] * kLog2eT;
    // Delta of query row `row`: eight dims per lane, summed over the 4 lanes
    const uint32_t a[4] = {dov[cb].x, dov[cb].y, dov[cb].z, dov[cb].w};
    const uint32_t b[4] = {ov[cb].x, ov[cb].y, ov[cb].z, ov[cb].w};
    float d = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x2 xa = Mfma<T>::unpack(a[i]), ya = Mfma<T>::unpack(b[i]);
      d = fmaf(xa[0], ya[0], fmaf(xa[1], ya[1], d));
    }
    dl[cb] = shfl_sum16_32(d);
  }
  f32x4 acc[2][2] = {{z, z}, {z, z}};   // dQ^T [cb][dim half]

  for (int c = 0; c < nch; ++c) {
    if (c > 0) {
      wait_vm<0>();
      __syncthreads();
    }
    if (c + 1 < nch) {
      const int r = min(64, upad - 64 * (c + 1));
      const uint32_t nb = lds_addr(lds + L::kKv + 8192 * ((c + 1) & 1));
      gather64(k, ktok + 64 * (c + 1), q0, r, nb, base, H, h, lane, wv);
      gather64(v, ktok + 64 * (c + 1), q0, r, nb + 4096u, base, H, h, lane, wv);
    }
    if (!active) continue;
    const char* kb = lds + L::kKv + 8192 * (c & 1);
    if (upad - 64 * c >= 64)
      bwdq_step<T, 4>(kb, kb + 4096, mt, kmax, 64 * c, qv, dov, cl, lse2, dl, scale_log2, acc, c16,
                      g, e, qq);
    else
      bwdq_step<T, 2>(kb, kb + 4096, mt, kmax, 64 * c, qv, dov, cl, lse2, dl, scale_log2, acc, c16,
                      g, e, qq);
  }
  if (!active) return;
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int tq = qtok[32 * wv + 16 * cb + c16];
    if (tq < 0) continue;
    const uint32_t qrow = (uint32_t)(base + tq) * (uint32_t)H + (uint32_t)h;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
      stv<uint2>(dq, qrow * kRowB + 32u * hf + 8u * g, pack4<T>(acc[cb][hf] * scale));
    if (g == 0) ld[qrow] = make_float2(lse2[cb], dl[cb]);
  }
}

// ---------------------------------------------------------------------------
// backward, key-major pass: dK, dV of the window's 64 keys
// ---------------------------------------------------------------------------
// Entries (query clusters reading the window) are held 32 at a time; their
// query rows stream 8 entries (64 rows) per chunk through two buffers.  The
// window's own K/V rows are staged once (in the second buffer, which the
// first chunk does not use) and kept in registers.
constexpr int kEntHeld = 32;
constexpr int kChunkEnt = 8;

struct BkvLds {
  // per buffer: Q 4 KiB, dO 4 KiB, LSE log2 e 256 B, Delta 256 B
  static constexpr int kBuf = 8192 + 512;
  static constexpr int kRec = 0, kEn = 512, kBuf0 = kEn + kEntHeld * kEnt * 4,
                       kBuf1 = kBuf0 + kBuf, kBytes = kBuf1 + kBuf;
};

// query rows of entries [e0, e0 + n) of the held block (n <= 8): rows
// 8 x + m = member m of entry x; rows up to a multiple of 32 (padding rows
// take `fallback` and read the (+inf, 0) pair)
__device__ __forceinline__ void kv_chunk_rows(const void* q, const void* dout, const float2* ld,
                                              uint32_t ld_none, const int32_t* en, int e0, int n,
                                              int fallback, uint32_t buf, int base, int H, int h,
                                              int lane, int wv) {
  const int nrows = 32 * ((8 * n + 31) >> 5);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int i = wv + 2 * j;
    if (16 * i < nrows) {
      const int row = 16 * i + (lane >> 2);
      int t = (row >> 3) < n ? en[(e0 + (row >> 3)) * kEnt + (row & 7)] : -1;
      t = t < 0 ? fallback : t;
      const uint32_t chunk = (uint32_t)(lane & 3) ^ sw(row);
      const uint32_t off = ((uint32_t)(base + t) * (uint32_t)H + (uint32_t)h) * kRowB + 16u * chunk;
      dma16(q, off, buf + 1024u * (uint32_t)i);
      dma16(dout, off, buf + 4096u + 1024u * (uint32_t)i);
    }
  }
  if (wv == 0) {   // (LSE log2 e, Delta) of the 64 rows as two 4-byte gathers
    const int t = (lane >> 3) < n ? en[(e0 + (lane >> 3)) * kEnt + (lane & 7)] : -1;
    const uint32_t off =
        t >= 0 ? ((uint32_t)(base + t) * (uint32_t)H + (uint32_t)h) * 8u : ld_none;
    dma4(ld, off, buf + 8192u);
    dma4(ld, off + 4u, buf + 8192u + 256u);
  }
}

template <typename T, int NQ>
__device__ __forceinline__ void bwdkv_step(const char* buf, const uint8_t* enb, int e0,
                                           int n, const uint4 (&kreg)[2], const uint4 (&vreg)[2],
                                           float scale_log2, f32x4 (&dka)[2][2],
                                           f32x4 (&dva)[2][2], int wv, int c16, int g, int e,
                                           int qq) {
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  const char* sq = buf;
  const char* sdo = buf + 4096;
  const float* sl2 = reinterpret_cast<const float*>(buf + 8192);
  const float* sdl = reinterpret_cast<const float*>(buf + 8192 + 256);
#pragma unroll
  for (int qg = 0; qg < NQ / 2; ++qg) {
    f32x4 pp[2][2], dd[2][2];   // [query block of the pair][key block]
#pragma unroll
    for (int qh = 0; qh < 2; ++qh) {
      const int qb = 2 * qg + qh;
      const int row = 16 * qb + c16;
      const uint4 qa = lds16(sq, row_chunk(row, (uint32_t)g));
      const uint4 da = lds16(sdo, row_chunk(row, (uint32_t)g));
      const int rr = 16 * qb + 4 * g;   // rows rr .. rr + 3 of this lane
      const int er = rr >> 3;           // their entry (in the chunk)
      const float4 l2 = *reinterpret_cast<const float4*>(sl2 + rr);
      const float4 dl4 = *reinterpret_cast<const float4*>(sdl + rr);
      const float l2a[4] = {l2.x, l2.y, l2.z, l2.w};
      const float dla[4] = {dl4.x, dl4.y, dl4.z, dl4.w};
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const f32x4 sv = Mfma<T>::mma(qa, kreg[kb], z);
        const f32x4 pv = Mfma<T>::mma(da, vreg[kb], z);
        const int key = 32 * wv + 16 * kb + c16;
        const float m = er < n ? (float)enb[(e0 + er) * (kEnt * 4) + 32 + key] : 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = m * __builtin_amdgcn_exp2f(fmaf(sv[i], scale_log2, -l2a[i]));
          pp[qh][kb][i] = m != 0.f ? p : 0.f;
          dd[qh][kb][i] = m != 0.f ? p * (pv[i] - dla[i]) : 0.f;
        }
      }
    }
    // dV^T += dO^T P, dK^T += Q^T dS over these 32 rows
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const uint4 dt = tr_pair(sdo, 32 * qg, hf, g, e, qq);
      const uint4 qt = tr_pair(sq, 32 * qg, hf, g, e, qq);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        dva[hf][kb] = Mfma<T>::mma(dt, cat(pack4<T>(pp[0][kb]), pack4<T>(pp[1][kb])), dva[hf][kb]);
        dka[hf][kb] = Mfma<T>::mma(qt, cat(pack4<T>(dd[0][kb]), pack4<T>(dd[1][kb])), dka[hf][kb]);
      }
    }
  }
}

template <typename T>
__global__ void __launch_bounds__(kTThreads)
bwdkv_tile_kernel(int H, int ntiles, float scale, const T* __restrict__ q,
                  const T* __restrict__ k, const T* __restrict__ v, const T* __restrict__ dout,
                  const float2* __restrict__ ld, uint32_t ld_none,
                  const int32_t* __restrict__ krec, const int32_t* __restrict__ kent,
                  T* __restrict__ dk, T* __restrict__ dv) {
  typedef BkvLds L;
  __shared__ __attribute__((aligned(1024))) char lds[L::kBytes];
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  if (tile >= ntiles) return;
  const int w = tile / H, h = tile - w * H;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int c16 = lane & 15, g = lane >> 4;
  const int e = c16 >> 2, qq = c16 & 3;
  const int32_t* rk = reinterpret_cast<const int32_t*>(lds + L::kRec);
  const int32_t* en = reinterpret_cast<const int32_t*>(lds + L::kEn);
  const uint8_t* enb = reinterpret_cast<const uint8_t*>(lds + L::kEn);
  const float scale_log2 = scale * kLog2eT;
  const uint32_t buf0 = lds_addr(lds + L::kBuf0), buf1 = lds_addr(lds + L::kBuf1);

  copy_lds(krec, (uint32_t)(w * kKRec * 4), 288, lds_addr(rk), lane, wv);
  wait_vm<0>();
  __syncthreads();
  const int start = __builtin_amdgcn_readfirstlane(rk[0]);
  const int E = __builtin_amdgcn_readfirstlane(rk[1]);
  const int base = __builtin_amdgcn_readfirstlane(rk[3]);
  const int nc = __builtin_amdgcn_readfirstlane(rk[4]);
  const int32_t* ktok = rk + 8;
  const int k0tok = __builtin_amdgcn_readfirstlane(ktok[0]);
  // own K and V rows into the second buffer, the first held entries
  gather64(k, ktok, k0tok, 64, buf1, base, H, h, lane, wv);
  gather64(v, ktok, k0tok, 64, buf1 + 4096u, base, H, h, lane, wv);
  int held = min(E, kEntHeld);
  copy_lds(kent, (uint32_t)start * (uint32_t)(kEnt * 4), held * kEnt * 4, lds_addr(en), lane, wv);
  wait_vm<0>();
  __syncthreads();
  const bool active = 32 * wv < 8 * nc;
  uint4 kreg[2], vreg[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int row = 32 * wv + 16 * kb + c16;
    kreg[kb] = lds16(lds + L::kBuf1, row_chunk(row, (uint32_t)g));
    vreg[kb] = lds16(lds + L::kBuf1 + 4096, row_chunk(row, (uint32_t)g));
  }
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  f32x4 dka[2][2] = {{z, z}, {z, z}}, dva[2][2] = {{z, z}, {z, z}};   // [dim half][key block]

  for (int h0 = 0; h0 < E; h0 += kEntHeld) {
    if (h0 > 0) {   // more than kEntHeld entries: the next block of them
      __syncthreads();
      held = min(E - h0, kEntHeld);
      copy_lds(kent, (uint32_t)(start + h0) * (uint32_t)(kEnt * 4), held * kEnt * 4,
               lds_addr(en), lane, wv);
      wait_vm<0>();
      __syncthreads();
    } else {
      __syncthreads();   // every wavefront has read the own K/V rows from buffer 1
    }
    const int nchk = (held + kChunkEnt - 1) / kChunkEnt;
    kv_chunk_rows(q, dout, ld, ld_none, en, 0, min(kChunkEnt, held), k0tok, buf0, base, H, h,
                  lane, wv);
    for (int c = 0; c < nchk; ++c) {
      wait_vm<0>();
      __syncthreads();
      if (c + 1 < nchk)
        kv_chunk_rows(q, dout, ld, ld_none, en, kChunkEnt * (c + 1),
                      min(kChunkEnt, held - kChunkEnt * (c + 1)), k0tok, (c + 1) & 1 ? buf1 : buf0,
                      base, H, h, lane, wv);
      if (!active) continue;
      const int n = min(kChunkEnt, held - kChunkEnt * c);
      const char* buf = lds + ((c & 1) ? L::kBuf1 : L::kBuf0);
      if (n > 4)
        bwdkv_step<T, 4>(buf, enb, kChunkEnt * c, n, kreg, vreg, scale_log2, dka, dva, wv, c16, g,
                         e, qq);
      else
        bwdkv_step<T, 2>(buf, enb, kChunkEnt * c, n, kreg, vreg, scale_log2, dka, dva, wv, c16, g,
                         e, qq);
    }
  }
  if (!active) return;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int tk = ktok[32 * wv + 16 * kb + c16];
    if (tk < 0) continue;
    const uint32_t krow = (uint32_t)(base + tk) * (uint32_t)H + (uint32_t)h;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      stv<uint2>(dk, krow * kRowB + 32u * hf + 8u * g, pack4<T>(dka[hf][kb] * scale));
      stv<uint2>(dv, krow * kRowB + 32u * hf + 8u * g, pack4<T>(dva[hf][kb]));
    }
  }
}

template <typename T>
hipError_t fwd_tile_t(int B, int C, int H, int nk, float scale, const void* q, const void* k,
                      const void* v, const BwdWorkspace& w, void* o, float* lse,
                      hipStream_t st) {
  const int64_t ntiles = windows_of(B, C) * H;
  if (ntiles == 0) return hipSuccess;
  hipLaunchKernelGGL((fwd_tile_kernel<T>), dim3((unsigned)ntiles), dim3(kTThreads), 0, st, H,
                     (int)ntiles, 8 * nk, qrec_stride(nk), scale * kLog2eT, (const T*)q,
                     (const T*)k, (const T*)v, (const int32_t*)w.qrec, (T*)o, lse);
  return hipGetLastError();
}

template <typename T>
hipError_t bwd_tile_t(int pass, int B, int C, int H, int nk, float scale, const void* q,
                      const void* k, const void* v, const void* o, const void* dout,
                      const float* lse, void* dq, void* dk, void* dv, const BwdWorkspace& w,
                      hipStream_t st) {
  const int64_t ntiles = windows_of(B, C) * H;
  if (ntiles == 0) return hipSuccess;
  if (pass & 1)
    hipLaunchKernelGGL((bwdq_tile_kernel<T>), dim3((unsigned)ntiles), dim3(kTThreads), 0, st, H,
                       (int)ntiles, 8 * nk, qrec_stride(nk), scale, (const T*)q, (const T*)k,
                       (const T*)v, (const T*)o, (const T*)dout, lse, (const int32_t*)w.qrec,
                       (T*)dq, w.ld, w.ld_none);
  if (pass & 2) {
    const uint32_t ld_none = (uint32_t)((const char*)w.ld_none - (const char*)w.ld);
    hipLaunchKernelGGL((bwdkv_tile_kernel<T>), dim3((unsigned)ntiles), dim3(kTThreads), 0, st, H,
                       (int)ntiles, scale, (const T*)q, (const T*)k, (const T*)v, (const T*)dout,
                       (const float2*)w.ld, ld_none, (const int32_t*)w.krec,
                       (const int32_t*)w.kent, (T*)dk, (T*)dv);
  }
  return hipGetLastError();
}

}  // namespace

bool tile_supported(int dt, int B, int N, int C, int H, int nk) {
  // 32-bit byte offsets (the workspace's LSE/Delta pairs included), tile counts
  const int64_t bytes = (int64_t)B * N * H * 32 * 2;
  return (dt == 1 || dt == 2) && nk % 8 == 0 && nk >= 8 && nk <= 64 &&
         bytes < (int64_t(1) << 31) && windows_of(B, C) * H < (int64_t(1) << 31);
}

hipError_t launch_fwd_tile(int dt, int B, int N, int C, int H, int nk, float scale, const void* q,
                           const void* k, const void* v, const BwdWorkspace& w, void* o,
                           float* lse, hipStream_t st) {
  (void)N;
  if (dt == 1) return fwd_tile_t<bf16>(B, C, H, nk, scale, q, k, v, w, o, lse, st);
  if (dt == 2) return fwd_tile_t<f16>(B, C, H, nk, scale, q, k, v, w, o, lse, st);
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_tile(int pass, int dt, int B, int N, int C, int H, int nk, float scale,
                           const void* q, const void* k, const void* v, const void* o,
                           const void* dout, const float* lse, void* dq, void* dk, void* dv,
                           const BwdWorkspace& w, hipStream_t st) {
  (void)N;
  if (dt == 1)
    return bwd_tile_t<bf16>(pass, B, C, H, nk, scale, q, k, v, o, dout, lse, dq, dk, dv, w, st);
  if (dt == 2)
    return bwd_tile_t<f16>(pass, B, C, H, nk, scale, q, k, v, o, dout, lse, dq, dk, dv, w, st);
  return hipErrorInvalidValue;
}

}  // namespace ca
