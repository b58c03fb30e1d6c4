// Window-tiled matrix-core cluster attention for gfx950 (bf16 / fp16).
//
// What is computed: the local cluster attention of the English notes page
// "AFFMAE: Scalable Vision Pre-Training for High-Resolution Microscopy
// Segmentation on Desktop Hardware" ("Overall Architecture"): every query
// cluster attends, with a plain scaled-dot-product softmax, to the key slots
// of its list; forward (O, LSE) and backward (dQ, dK, dV).  The arXiv abstract
// of the same paper asks for numerically stable, mixed-precision,
// Flash-style kernels: bf16/fp16 operands, fp32 statistics and accumulation,
// logits in log2 units with the row maximum subtracted.
//
// Structure: one workgroup of four wavefronts per tile = (window of 8
// consecutive clusters, pair of heads); the window plan (tile_plan.hip)
// describes the window.
//  * A token's rows of two consecutive heads are one 128-byte line, so every
//    gather moves whole cache lines (a single head's 64-byte row would cost
//    the L2 and the texture path nearly as much as the full line).
//  * Forward and query-major backward pass: the workgroup stages the distinct
//    key and value rows of the window's lists once in LDS (direct-to-LDS
//    loads); at the stage-1 shape a window's 384 slots hold about 144
//    distinct keys, so each key row is gathered 2.7 times less often than per
//    cluster.  Each wavefront computes one pair of clusters for both heads,
//    each cluster on its own 48 slots only: the two clusters share a
//    16-column MFMA tile (columns 0-7 and 8-15), block-diagonal over two
//    16x16x32 MFMAs whose A operands are the two clusters' slot rows, read
//    from LDS through the plan's slot table.  Query-side rows (Q, and for the
//    backward dO, O and the LSE) go straight to the registers of the
//    wavefront that uses them.  The softmax (fp32, row maximum, exp2) runs
//    on 12 logits per lane; O^T = V^T P^T reads V transposed
//    (ds_read_b64_tr_b16).
//  * Query-major backward: dS = P (dP - Delta), dQ^T = K^T dS^T; writes dQ
//    and (LSE log2 e, Delta) per query row for the key-major pass.
//  * Key-major backward: the window's own K and V rows in registers, the Q
//    and dO rows of the query clusters reading them (merged, so each query
//    row is gathered once per window) staged in LDS kKRecEnt clusters at a
//    time; each wavefront takes a pair of key clusters and walks their
//    (query cluster, multiplicities) items four at a time: S = Q K^T,
//    dP = dO V^T, dV^T += dO^T P, dK^T += Q^T dS.  Each dK/dV row is written
//    once by one workgroup: no atomics, bitwise reproducible.
//  * Workgroups are numbered so that each XCD takes a contiguous range of
//    windows (all heads): the rows shared by neighbouring windows and the
//    heads of one token row stay in that XCD's L2.
#include "common.h"
#include "mfma_util.h"

namespace ca {

namespace {

constexpr int kTThreads = 256;   // four wavefronts per tile
constexpr uint32_t kRowB = 64;   // bytes of one head row in global memory
constexpr float kLog2eT = 1.4426950408889634f;
constexpr float kLn2T = 0.6931471805599453f;

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)p;
}

// byte offset of logical chunk `chunk` (0..7) of staged row `r`
__device__ __forceinline__ uint32_t lrow(int r, uint32_t chunk) {
  return (uint32_t)r * kLdsRow + 16u * (chunk ^ row_swz(r));
}

// Direct-to-LDS copy of `bytes` (a multiple of 16) contiguous bytes, split
// over the workgroup's four wavefronts (instruction i by wavefront i & 3).
__device__ __forceinline__ void copy_lds(const void* src, uint32_t src_off, int bytes, uint32_t dst,
                                         int lane, int wv) {
  const int n16 = bytes >> 4;
  for (int i = wv; 64 * i < n16; i += 4) {
    const int p = 64 * i + lane;
    if (p < n16) dma16(src, src_off + 16u * (uint32_t)p, dst + 1024u * (uint32_t)i);
  }
}

// Logical chunk that lane `lane` fetches when an instruction fills staged rows
// 8 i .. 8 i + 7 (lane l: row 8 i + l / 8, position l & 7): the chunk that
// belongs at that position.  With one head per row only chunks 0..3 exist;
// the lanes of positions 4..7 then fetch a duplicate that is never read.
template <int HP>
__device__ __forceinline__ uint32_t dma_chunk(int lane, int i) {
  const uint32_t c = (uint32_t)((lane ^ (lane >> 3) ^ i) & 7);
  return HP == 2 ? c : (c & 3u);
}

// The four slot-table offsets (16-slot blocks 0..3) of table row x of cluster c
__device__ __forceinline__ void slot_offsets(const uint16_t* tab, int c, int x, uint32_t (&o)[4]) {
  const uint2 v = *reinterpret_cast<const uint2*>(tab + (c * 16 + x) * 4);
  o[0] = v.x & 0xffffu;
  o[1] = v.x >> 16;
  o[2] = v.y & 0xffffu;
  o[3] = v.y >> 16;
}

// ---------------------------------------------------------------------------
// query-major staging: the query record of a (sub-)window and the key and
// value rows (heads h0 .. h0 + HP - 1) of its distinct keys
// ---------------------------------------------------------------------------
struct QLds {
  static constexpr int kRec = 0, kK = 2304, kV = kK + kLdsRow * kUnionCap,
                       kBytes = kV + kLdsRow * kUnionCap;
};
static_assert(kQRec * 4 <= QLds::kK, "query record fits its LDS region");
static_assert(kUnionCap % 32 == 0, "staged key rows come in groups of 32");
constexpr int kKvIns = kUnionCap / 32;   // K (or V) instructions per wavefront, at most

// Stage one (sub-)window record at `rec_off` (ints) and its K/V rows (not
// waited for).  Returns the record's cluster count, 0 for the record of a
// split window (nothing gathered).
template <int HP>
__device__ __forceinline__ int stage_kv(const int32_t* qrec, int64_t rec_off, char* lds,
                                        const void* k, const void* v, int H, int h0, int lane,
                                        int wv) {
  const int32_t* rec = reinterpret_cast<const int32_t*>(lds + QLds::kRec);
  copy_lds(qrec, (uint32_t)(rec_off * 4), kQRec * 4, lds_addr(rec), lane, wv);
  wait_vm<0>();
  __syncthreads();
  if (__builtin_amdgcn_readfirstlane(rec[4]) & kQSplit) return 0;
  const int u = __builtin_amdgcn_readfirstlane(rec[2]);
  const int base = __builtin_amdgcn_readfirstlane(rec[3]);
  const int q0 = __builtin_amdgcn_readfirstlane(rec[8]);
  const int upad = (u + 31) & ~31;
  // instruction i = wv + 4 j fills rows 8 i .. 8 i + 7 of K and of V; the
  // tokens first (the key tokens are padded to upad with a valid token)
  const int lr = lane >> 3;
  int tk[kKvIns];
#pragma unroll
  for (int j = 0; j < kKvIns; ++j) {
    const int i = wv + 4 * j;
    tk[j] = 8 * i < upad ? rec[kQRecHead + 8 * i + lr] : q0;
  }
  const uint32_t hrow = (uint32_t)H * kRowB;
  const uint32_t dk = lds_addr(lds + QLds::kK), dv = lds_addr(lds + QLds::kV);
#pragma unroll
  for (int j = 0; j < kKvIns; ++j) {
    const int i = wv + 4 * j;
    if (8 * i < upad) {
      const uint32_t off =
          (uint32_t)(base + tk[j]) * hrow + (uint32_t)h0 * kRowB + 16u * dma_chunk<HP>(lane, i);
      dma16(k, off, dk + 1024u * (uint32_t)i);
      dma16(v, off, dv + 1024u * (uint32_t)i);
    }
  }
  return __builtin_amdgcn_readfirstlane(rec[1]);
}

// Which pair of which record a wavefront computes: with the window split
// into nsub sub-windows, sub-window s is computed by the 4 / nsub
// wavefronts [s * 4 / nsub, (s + 1) * 4 / nsub), pair wv - s * 4 / nsub.
__device__ __forceinline__ int my_pair(int wv, int s, int nsub) {
  const int per = 4 / nsub;
  const int p = wv - s * per;
  return (p >= 0 && p < per) ? p : -1;
}

// Byte offset of chunk g of the head-h0 row of query 16 p + c16 of the
// staged record (an absent query reads the record's first query).
__device__ __forceinline__ uint32_t query_row(const int32_t* rec, int p, int c16, int g, int H,
                                              int h0) {
  const int t = rec[8 + 16 * p + c16];
  const int q0 = rec[8];
  return ((uint32_t)(rec[3] + (t < 0 ? q0 : t)) * (uint32_t)H + (uint32_t)h0) * kRowB +
         16u * (uint32_t)g;
}

// ---------------------------------------------------------------------------
// forward: one pair of clusters (2p, 2p + 1) of the staged record, HP heads
// ---------------------------------------------------------------------------
template <typename T, int NB, int HP, bool HOLES>
__device__ void fwd_pair(const char* lds, int p, int nc, int H, int h0, float csl, bool neg,
                         const uint4 (&qin)[HP], T* __restrict__ o, float* __restrict__ lse,
                         int lane) {
  const int32_t* rec = reinterpret_cast<const int32_t*>(lds + QLds::kRec);
  const uint16_t* tab = reinterpret_cast<const uint16_t*>(rec + kQSlotOff);
  const unsigned long long* masks = reinterpret_cast<const unsigned long long*>(rec + kQMaskOff);
  const char* sk = lds + QLds::kK;
  const char* sv = lds + QLds::kV;
  const int c16 = lane & 15, g = lane >> 4, e = c16 >> 2, qq = c16 & 3;
  const bool left = c16 < 8;
  const int a = 2 * p, b = min(2 * p + 1, nc - 1);   // an absent b reads a valid cluster
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  uint32_t ka[4], kb[4], va[4], vb[4];
  slot_offsets(tab, a, c16, ka);
  slot_offsets(tab, b, c16, kb);
  slot_offsets(tab, a, 4 * g + e, va);
  slot_offsets(tab, b, 4 * g + e, vb);
  uint32_t vm[NB];
  if (HOLES) {
    const bool bok = 2 * p + 1 < nc;
    const unsigned long long m = left ? masks[a] : (bok ? masks[b] : 0ull);
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) vm[blk] = (uint32_t)(m >> (16 * blk + 4 * g)) & 0xfu;
  }
  const int tq = rec[8 + 16 * p + c16];
  const uint32_t qrow = (uint32_t)(rec[3] + tq) * (uint32_t)H + (uint32_t)h0;
#pragma unroll
  for (int hh = 0; hh < HP; ++hh) {
    uint4 qv = qin[hh];
    if (neg) {   // a negative scale: -|scale| with Q negated (exact)
      qv.x ^= 0x80008000u;
      qv.y ^= 0x80008000u;
      qv.z ^= 0x80008000u;
      qv.w ^= 0x80008000u;
    }
    const uint4 qL = sel(left, qv), qR = sel(!left, qv);
    const uint32_t gx = 16u * (uint32_t)(4 * hh + g);
    f32x4 s[NB];
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
      s[blk] = Mfma<T>::mma(lds16(sk, ka[blk] ^ gx), qL, z);
      s[blk] = Mfma<T>::mma(lds16(sk, kb[blk] ^ gx), qR, s[blk]);
    }
    float mx = -INFINITY;
#pragma unroll
    for (int blk = 0; blk < NB; ++blk)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        mx = fmaxf(mx, HOLES && !((vm[blk] >> i) & 1u) ? -INFINITY : s[blk][i]);
    mx = shfl_max16_32(mx);
    const float mref = mx == -INFINITY ? 0.f : mx * csl;
    float l = 0.f;
    uint2 ph[NB];
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
      f32x4 pr;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float pv = __builtin_amdgcn_exp2f(fmaf(s[blk][i], csl, -mref));
        if (HOLES) pv = ((vm[blk] >> i) & 1u) ? pv : 0.f;
        pr[i] = pv;
        l += pv;
      }
      ph[blk] = pack4<T>(pr);
    }
    l = shfl_sum16_32(l);
    f32x4 oacc[2] = {z, z};
#pragma unroll
    for (int kg = 0; kg < (NB + 1) / 2; ++kg) {
      const int b0 = 2 * kg, b1 = 2 * kg + 1;
      const uint4 bp = cat(ph[b0], b1 < NB ? ph[b1 < NB ? b1 : b0] : make_uint2(0u, 0u));
      const uint4 bpa = sel(left, bp), bpb = sel(!left, bp);
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const uint32_t x =
            16u * (uint32_t)(4 * hh + 2 * hf + (qq >> 1)) + 8u * (uint32_t)(qq & 1);
        const uint4 aa = cat(lds_tr8(sv, va[b0] ^ x), lds_tr8(sv, va[b1] ^ x));
        const uint4 ab = cat(lds_tr8(sv, vb[b0] ^ x), lds_tr8(sv, vb[b1] ^ x));
        oacc[hf] = Mfma<T>::mma(aa, bpa, oacc[hf]);
        oacc[hf] = Mfma<T>::mma(ab, bpb, oacc[hf]);
      }
    }
    if (tq >= 0) {
      const float inv = l > 0.f ? __builtin_amdgcn_rcpf(l) : 0.f;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
        stv<uint2>(o, (qrow + hh) * kRowB + 32u * hf + 8u * g, pack4<T>(oacc[hf] * inv));
      if (g == 0) lse[qrow + hh] = l > 0.f ? (mref + __log2f(l)) * kLn2T : -INFINITY;
    }
  }
}

template <typename T, int NB, int HP>
__device__ __forceinline__ void fwd_pair_any(const char* lds, int p, int nc, int H, int h0,
                                             float csl, bool neg, const uint4 (&qv)[HP], T* o,
                                             float* lse, int lane) {
  const int32_t* rec = reinterpret_cast<const int32_t*>(lds + QLds::kRec);
  if (rec[2] == 0) {   // no slot of the window holds a token: O = 0, LSE = -inf
    const int c16 = lane & 15, g = lane >> 4;
    const int tq = rec[8 + 16 * p + c16];
    if (tq < 0) return;
    const uint32_t qrow = (uint32_t)(rec[3] + tq) * (uint32_t)H + (uint32_t)h0;
#pragma unroll
    for (int hh = 0; hh < HP; ++hh) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
        stv<uint2>(o, (qrow + hh) * kRowB + 32u * hf + 8u * g, make_uint2(0u, 0u));
      if (g == 0) lse[qrow + hh] = -INFINITY;
    }
    return;
  }
  const bool holes = (rec[4] & kQHoles) || 2 * p + 1 >= nc;
  if (holes) fwd_pair<T, NB, HP, true>(lds, p, nc, H, h0, csl, neg, qv, o, lse, lane);
  else fwd_pair<T, NB, HP, false>(lds, p, nc, H, h0, csl, neg, qv, o, lse, lane);
}

template <typename T, int NB, int HP>
__global__ void __launch_bounds__(kTThreads)
fwd_tile_kernel(int H, int ntiles, int nrec, float scale_log2, const T* __restrict__ q,
                const T* __restrict__ k, const T* __restrict__ v, const int32_t* __restrict__ qrec,
                T* __restrict__ o, float* __restrict__ lse) {
  __shared__ __attribute__((aligned(1024))) char lds[QLds::kBytes];
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  if (tile >= ntiles) return;
  const int hg = H / HP;   // head groups per window
  const int w = tile / hg, h0 = (tile - w * hg) * HP;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int c16 = lane & 15, g = lane >> 4;
  const bool neg = scale_log2 < 0.f;
  const float csl = fabsf(scale_log2);
  const int32_t* rec = reinterpret_cast<const int32_t*>(lds + QLds::kRec);
  const int64_t r0 = (int64_t)w * nrec * kQRecStride;
  int nc = stage_kv<HP>(qrec, r0, lds, k, v, H, h0, lane, wv);
  uint4 qv[HP];
  if (!(rec[4] & kQSplit)) {
    const bool mine = 2 * wv < nc;
    if (mine) {
      const uint32_t off = query_row(rec, wv, c16, g, H, h0);
#pragma unroll
      for (int hh = 0; hh < HP; ++hh) qv[hh] = ld16(q, off + kRowB * hh);
    }
    wait_vm<0>();
    __syncthreads();
    if (mine) fwd_pair_any<T, NB, HP>(lds, wv, nc, H, h0, csl, neg, qv, o, lse, lane);
    return;
  }
  // more distinct keys than one staging holds: the sub-windows one by one
  const int nsub = __builtin_amdgcn_readfirstlane(rec[5]);
  for (int s = 0; s < nsub; ++s) {
    __syncthreads();
    nc = stage_kv<HP>(qrec, r0 + (int64_t)(1 + s) * kQRecStride, lds, k, v, H, h0, lane, wv);
    const int p = my_pair(wv, s, nsub);
    const bool mine = p >= 0 && 2 * p < nc;
    if (mine) {
      const uint32_t off = query_row(rec, p, c16, g, H, h0);
#pragma unroll
      for (int hh = 0; hh < HP; ++hh) qv[hh] = ld16(q, off + kRowB * hh);
    }
    wait_vm<0>();
    __syncthreads();
    if (mine) fwd_pair_any<T, NB, HP>(lds, p, nc, H, h0, csl, neg, qv, o, lse, lane);
  }
}

// ---------------------------------------------------------------------------
// backward, query-major pass: one pair of clusters (2p, 2p + 1), HP heads
// ---------------------------------------------------------------------------
// The query-side inputs of a wavefront's pair, straight from global memory:
// lane (c16, g) holds chunk g of the Q, dO and O rows of query 16 p + c16 and
// that query's LSE, per head.
template <int HP>
struct QRows {
  uint4 q[HP], d[HP], o[HP];
  float lse[HP];
};

template <int HP>
__device__ __forceinline__ void load_qrows(QRows<HP>& r, const int32_t* rec, int p, int H, int h0,
                                           const void* q, const void* dout, const void* o,
                                           const float* lse, int lane) {
  const int c16 = lane & 15, g = lane >> 4;
  const uint32_t off = query_row(rec, p, c16, g, H, h0);
  const uint32_t li = (off >> 6);   // (token * H + h0): the row index of the head-h0 row
#pragma unroll
  for (int hh = 0; hh < HP; ++hh) {
    r.q[hh] = ld16(q, off + kRowB * hh);
    r.d[hh] = ld16(dout, off + kRowB * hh);
    r.o[hh] = ld16(o, off + kRowB * hh);
    r.lse[hh] = lse[li + hh];
  }
}

template <typename T, int NB, int HP, bool HOLES>
__device__ void bwdq_pair(const char* lds, int p, int nc, int H, int h0, float scale,
                          const QRows<HP>& in, T* __restrict__ dq, float2* __restrict__ ld,
                          int lane) {
  const int32_t* rec = reinterpret_cast<const int32_t*>(lds + QLds::kRec);
  const uint16_t* tab = reinterpret_cast<const uint16_t*>(rec + kQSlotOff);
  const unsigned long long* masks = reinterpret_cast<const unsigned long long*>(rec + kQMaskOff);
  const char* sk = lds + QLds::kK;
  const char* sv = lds + QLds::kV;
  const int c16 = lane & 15, g = lane >> 4, e = c16 >> 2, qq = c16 & 3;
  const bool left = c16 < 8;
  const int a = 2 * p, b = min(2 * p + 1, nc - 1);
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  const float scale_log2 = scale * kLog2eT;
  uint32_t ka[4], kb[4], va[4], vb[4];
  slot_offsets(tab, a, c16, ka);
  slot_offsets(tab, b, c16, kb);
  slot_offsets(tab, a, 4 * g + e, va);
  slot_offsets(tab, b, 4 * g + e, vb);
  uint32_t vm[NB];
  if (HOLES) {
    const bool bok = 2 * p + 1 < nc;
    const unsigned long long m = left ? masks[a] : (bok ? masks[b] : 0ull);
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) vm[blk] = (uint32_t)(m >> (16 * blk + 4 * g)) & 0xfu;
  }
  const int tq = rec[8 + 16 * p + c16];
  const uint32_t qrow = (uint32_t)(rec[3] + tq) * (uint32_t)H + (uint32_t)h0;
#pragma unroll
  for (int hh = 0; hh < HP; ++hh) {
    const float lse2 = in.lse[hh] * kLog2eT;
    // Delta of the column's query: eight dims per lane, summed over the 4 lanes
    float dl = 0.f;
    {
      const uint32_t x[4] = {in.d[hh].x, in.d[hh].y, in.d[hh].z, in.d[hh].w};
      const uint32_t y[4] = {in.o[hh].x, in.o[hh].y, in.o[hh].z, in.o[hh].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x2 xa = Mfma<T>::unpack(x[i]), ya = Mfma<T>::unpack(y[i]);
        dl = fmaf(xa[0], ya[0], fmaf(xa[1], ya[1], dl));
      }
    }
    dl = shfl_sum16_32(dl);
    const uint4 qL = sel(left, in.q[hh]), qR = sel(!left, in.q[hh]);
    const uint4 dL = sel(left, in.d[hh]), dR = sel(!left, in.d[hh]);
    const uint32_t gx = 16u * (uint32_t)(4 * hh + g);
    uint2 dh[NB];
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
      f32x4 sv4 = Mfma<T>::mma(lds16(sk, ka[blk] ^ gx), qL, z);
      sv4 = Mfma<T>::mma(lds16(sk, kb[blk] ^ gx), qR, sv4);
      f32x4 dp = Mfma<T>::mma(lds16(sv, ka[blk] ^ gx), dL, z);
      dp = Mfma<T>::mma(lds16(sv, kb[blk] ^ gx), dR, dp);
      f32x4 ds;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float pv = __builtin_amdgcn_exp2f(fmaf(sv4[i], scale_log2, -lse2));
        if (HOLES) pv = ((vm[blk] >> i) & 1u) ? pv : 0.f;
        ds[i] = pv * (dp[i] - dl);
      }
      dh[blk] = pack4<T>(ds);
    }
    f32x4 acc[2] = {z, z};
#pragma unroll
    for (int kg = 0; kg < (NB + 1) / 2; ++kg) {
      const int b0 = 2 * kg, b1 = 2 * kg + 1;
      const uint4 bd = cat(dh[b0], b1 < NB ? dh[b1 < NB ? b1 : b0] : make_uint2(0u, 0u));
      const uint4 bda = sel(left, bd), bdb = sel(!left, bd);
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const uint32_t x =
            16u * (uint32_t)(4 * hh + 2 * hf + (qq >> 1)) + 8u * (uint32_t)(qq & 1);
        const uint4 aa = cat(lds_tr8(sk, va[b0] ^ x), lds_tr8(sk, va[b1] ^ x));
        const uint4 ab = cat(lds_tr8(sk, vb[b0] ^ x), lds_tr8(sk, vb[b1] ^ x));
        acc[hf] = Mfma<T>::mma(aa, bda, acc[hf]);
        acc[hf] = Mfma<T>::mma(ab, bdb, acc[hf]);
      }
    }
    if (tq >= 0) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
        stv<uint2>(dq, (qrow + hh) * kRowB + 32u * hf + 8u * g, pack4<T>(acc[hf] * scale));
      if (g == 0) ld[qrow + hh] = make_float2(lse2, dl);
    }
  }
}

template <typename T, int NB, int HP>
__device__ __forceinline__ void bwdq_pair_any(const char* lds, int p, int nc, int H, int h0,
                                              float scale, const QRows<HP>& in, T* dq,
                                              float2* ld, int lane) {
  const int32_t* rec = reinterpret_cast<const int32_t*>(lds + QLds::kRec);
  if (rec[2] == 0) {   // no slot of the window holds a token: dQ = 0
    const int c16 = lane & 15, g = lane >> 4;
    const int tq = rec[8 + 16 * p + c16];
    if (tq < 0) return;
    const uint32_t qrow = (uint32_t)(rec[3] + tq) * (uint32_t)H + (uint32_t)h0;
#pragma unroll
    for (int hh = 0; hh < HP; ++hh) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
        stv<uint2>(dq, (qrow + hh) * kRowB + 32u * hf + 8u * g, make_uint2(0u, 0u));
      if (g == 0) ld[qrow + hh] = make_float2(-INFINITY, 0.f);
    }
    return;
  }
  const bool holes = (rec[4] & kQHoles) || 2 * p + 1 >= nc;
  if (holes) bwdq_pair<T, NB, HP, true>(lds, p, nc, H, h0, scale, in, dq, ld, lane);
  else bwdq_pair<T, NB, HP, false>(lds, p, nc, H, h0, scale, in, dq, ld, lane);
}

template <typename T, int NB, int HP>
__global__ void __launch_bounds__(kTThreads)
bwdq_tile_kernel(int H, int ntiles, int nrec, float scale, const T* __restrict__ q,
                 const T* __restrict__ k, const T* __restrict__ v, const T* __restrict__ o,
                 const T* __restrict__ dout, const float* __restrict__ lse,
                 const int32_t* __restrict__ qrec, T* __restrict__ dq, float2* __restrict__ ld,
                 float4* __restrict__ ld_none) {
  __shared__ __attribute__((aligned(1024))) char lds[QLds::kBytes];
  // the (LSE log2 e, Delta) pair the key-major pass reads for an absent
  // query: P = exp2(s - inf) = 0 there
  if (blockIdx.x == 0 && threadIdx.x == 0) *ld_none = make_float4(INFINITY, 0.f, INFINITY, 0.f);
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  if (tile >= ntiles) return;
  const int hg = H / HP;
  const int w = tile / hg, h0 = (tile - w * hg) * HP;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int32_t* rec = reinterpret_cast<const int32_t*>(lds + QLds::kRec);
  const int64_t r0 = (int64_t)w * nrec * kQRecStride;
  int nc = stage_kv<HP>(qrec, r0, lds, k, v, H, h0, lane, wv);
  QRows<HP> in;
  if (!(rec[4] & kQSplit)) {
    const bool mine = 2 * wv < nc;
    if (mine) load_qrows<HP>(in, rec, wv, H, h0, q, dout, o, lse, lane);
    wait_vm<0>();
    __syncthreads();
    if (mine) bwdq_pair_any<T, NB, HP>(lds, wv, nc, H, h0, scale, in, dq, ld, lane);
    return;
  }
  const int nsub = __builtin_amdgcn_readfirstlane(rec[5]);
  for (int s = 0; s < nsub; ++s) {
    __syncthreads();
    nc = stage_kv<HP>(qrec, r0 + (int64_t)(1 + s) * kQRecStride, lds, k, v, H, h0, lane, wv);
    const int p = my_pair(wv, s, nsub);
    const bool mine = p >= 0 && 2 * p < nc;
    if (mine) load_qrows<HP>(in, rec, p, H, h0, q, dout, o, lse, lane);
    wait_vm<0>();
    __syncthreads();
    if (mine) bwdq_pair_any<T, NB, HP>(lds, p, nc, H, h0, scale, in, dq, ld, lane);
  }
}

// ---------------------------------------------------------------------------
// backward, key-major pass
// ---------------------------------------------------------------------------
// LDS of one key window: its record (with the first merged entries' query
// tokens), the items of its key clusters (when there are at most kItemCap),
// the query tokens of later chunks of merged entries, the Q and dO rows of up
// to kKRecEnt merged entries and their (LSE log2 e, Delta) pairs per head.
constexpr int kItemCap = 128;
constexpr int kLArr = 4 * ((8 * kKRecEnt + 63) / 64) * 64;   // bytes of one LSE/Delta array
struct KLds {
  static constexpr int kRec = 0, kItems = 1024, kTok = kItems + 16 * kItemCap,
                       kQ = kTok + 32 * kKRecEnt, kDo = kQ + kLdsRow * 8 * kKRecEnt,
                       kL = kDo + kLdsRow * 8 * kKRecEnt, kBytes = kL + 4 * kLArr;
};
static_assert(kKRec * 4 <= KLds::kItems, "key record fits its LDS region");
static_assert(KLds::kL % 16 == 0 && kLArr % 16 == 0, "LSE/Delta arrays are read as float4");

// rows of merged entries [e0, e0 + n) (n <= kKRecEnt; their tokens at `tok`):
// row 8 x + m = member m of entry e0 + x; the Q and dO rows (heads h0, h0 + 1
// of a 128-byte staged row), and per head the (LSE log2 e, Delta) pairs as
// two 4-byte gathers into arrays 2 hh and 2 hh + 1 (an absent member reads
// the (+inf, 0) pair at byte offset ld_none)
template <int HP>
__device__ __forceinline__ void kv_rows(const void* q, const void* dout, const float2* ld,
                                        uint32_t ld_none, const int32_t* tok, int n, int fallback,
                                        char* lds, int base, int H, int h0, int lane, int wv) {
  const int lr = lane >> 3;
  const uint32_t hrow = (uint32_t)H * kRowB;
  for (int i = wv; i < n; i += 4) {   // instruction i: rows 8 i .. 8 i + 7 = entry e0 + i
    int t = tok[8 * i + lr];
    t = t < 0 ? fallback : t;
    const uint32_t off =
        (uint32_t)(base + t) * hrow + (uint32_t)h0 * kRowB + 16u * dma_chunk<HP>(lane, i);
    dma16(q, off, lds_addr(lds + KLds::kQ) + 1024u * (uint32_t)i);
    dma16(dout, off, lds_addr(lds + KLds::kDo) + 1024u * (uint32_t)i);
  }
  const int nrows = 8 * n;
  for (int i = wv; 64 * i < nrows; i += 4) {
    const int row = 64 * i + lane;
    const int t = row < nrows ? tok[row] : -1;
#pragma unroll
    for (int hh = 0; hh < HP; ++hh) {
      const uint32_t off =
          t >= 0 ? ((uint32_t)(base + t) * (uint32_t)H + (uint32_t)(h0 + hh)) * 8u : ld_none;
      dma4(ld, off, lds_addr(lds + KLds::kL + (2 * hh) * kLArr) + 256u * (uint32_t)i);
      dma4(ld, off + 4u, lds_addr(lds + KLds::kL + (2 * hh + 1) * kLArr) + 256u * (uint32_t)i);
    }
  }
}

// One pair of key clusters (2 p, 2 p + 1), HP heads, over the staged merged
// entries [e0, e0 + n): their items with a merged index in that range, four
// at a time in lockstep.  `items` (LDS or global) holds the window's items;
// [ia, ia_end) and [ib, ib_end) are the two clusters' remaining ranges (the
// cursors advance past the processed items).
template <typename T, int HP>
__device__ void kv_pair(const char* lds, const RevEntry* items, int& ia, int ia_end, int& ib,
                        int ib_end, int e0, int n, const uint4 (&kreg)[HP],
                        const uint4 (&vreg)[HP], float scale_log2, f32x4 (&dka)[HP][2],
                        f32x4 (&dva)[HP][2], int lane) {
  const char* sq = lds + KLds::kQ;
  const char* sdo = lds + KLds::kDo;
  const int c16 = lane & 15, g = lane >> 4, e = c16 >> 2, qq = c16 & 3;
  const bool left = c16 < 8;
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  // items of each cluster that fall in this chunk
  auto count = [&](int c, int c_end) {
    int m = 0;
    while (c + m < c_end) {
      const int i = __builtin_amdgcn_readfirstlane(items[c + m].i);
      if (i >= e0 + n) break;
      ++m;
    }
    return m;
  };
  const int na = count(ia, ia_end), nb = count(ib, ib_end);
  const int ngr = (max(na, nb) + 3) >> 2;
  for (int gi = 0; gi < ngr; ++gi) {
    // item x (0..3) of this group for cluster a / b: its staged row base
    // (8 * (merged index - e0)) and multiplicities; past the end: entry e0
    // (valid rows) with multiplicity 0
    int ra[4], rb[4];
    uint64_t ma[4], mb[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int t = 4 * gi + x;
      ra[x] = 0;
      rb[x] = 0;
      ma[x] = 0ull;
      mb[x] = 0ull;
      if (t < na) {
        const RevEntry ea = items[ia + t];
        ra[x] = 8 * (ea.i - e0);
        ma[x] = ea.mult;
      }
      if (t < nb) {
        const RevEntry eb = items[ib + t];
        rb[x] = 8 * (eb.i - e0);
        mb[x] = eb.mult;
      }
    }
    // S and dP rows: columns 0-7 are a's keys over a's item rows, 8-15 b's
    // over b's; block qb holds items 2 qb, 2 qb + 1
    int rowa[2], rowb[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int xa = 2 * qb + (c16 >> 3);
      rowa[qb] = (xa == 0 ? ra[0] : xa == 1 ? ra[1] : xa == 2 ? ra[2] : ra[3]) + (c16 & 7);
      rowb[qb] = (xa == 0 ? rb[0] : xa == 1 ? rb[1] : xa == 2 ? rb[2] : rb[3]) + (c16 & 7);
    }
    // P and dS: lane (key column c16, row group g) holds rows 4 g .. 4 g + 3
    // of each block, i.e. members 4 (g & 1) .. + 3 of item 2 qb + (g >> 1)
    // of its own cluster
    int rbase[2];
    float mlt[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int x = 2 * qb + (g >> 1);
      rbase[qb] = (left ? (x == 0 ? ra[0] : x == 1 ? ra[1] : x == 2 ? ra[2] : ra[3])
                        : (x == 0 ? rb[0] : x == 1 ? rb[1] : x == 2 ? rb[2] : rb[3])) +
                  4 * (g & 1);
      const uint64_t mm = left ? (x == 0 ? ma[0] : x == 1 ? ma[1] : x == 2 ? ma[2] : ma[3])
                               : (x == 0 ? mb[0] : x == 1 ? mb[1] : x == 2 ? mb[2] : mb[3]);
      mlt[qb] = (float)((uint32_t)(mm >> (8 * (c16 & 7))) & 0xffu);
    }
    // dV^T += dO^T P and dK^T += Q^T dS: lane 4 e + qq of row group g reads
    // rows 16 blk + 4 g + e = member 4 (g & 1) + e of item 2 blk + (g >> 1)
    const int xa0 = (g >> 1), xa1 = 2 + (g >> 1);
    const int mrow = 4 * (g & 1) + e;
    const int ta0 = (xa0 == 0 ? ra[0] : ra[1]) + mrow, ta1 = (xa1 == 2 ? ra[2] : ra[3]) + mrow;
    const int tb0 = (xa0 == 0 ? rb[0] : rb[1]) + mrow, tb1 = (xa1 == 2 ? rb[2] : rb[3]) + mrow;
#pragma unroll
    for (int hh = 0; hh < HP; ++hh) {
      const float* sl2 = reinterpret_cast<const float*>(lds + KLds::kL + (2 * hh) * kLArr);
      const float* sdl = reinterpret_cast<const float*>(lds + KLds::kL + (2 * hh + 1) * kLArr);
      const uint4 kL = sel(left, kreg[hh]), kR = sel(!left, kreg[hh]);
      const uint4 vL = sel(left, vreg[hh]), vR = sel(!left, vreg[hh]);
      const uint32_t gq = (uint32_t)(4 * hh + g);
      f32x4 s[2], dp[2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        s[qb] = Mfma<T>::mma(lds16(sq, lrow(rowa[qb], gq)), kL, z);
        s[qb] = Mfma<T>::mma(lds16(sq, lrow(rowb[qb], gq)), kR, s[qb]);
        dp[qb] = Mfma<T>::mma(lds16(sdo, lrow(rowa[qb], gq)), vL, z);
        dp[qb] = Mfma<T>::mma(lds16(sdo, lrow(rowb[qb], gq)), vR, dp[qb]);
      }
      uint2 ph[2], dh[2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const float m = mlt[qb];
        const float4 l2 = *reinterpret_cast<const float4*>(sl2 + rbase[qb]);
        const float4 dl4 = *reinterpret_cast<const float4*>(sdl + rbase[qb]);
        const float l2a[4] = {l2.x, l2.y, l2.z, l2.w};
        const float dla[4] = {dl4.x, dl4.y, dl4.z, dl4.w};
        f32x4 pp, dd;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float pv = m * __builtin_amdgcn_exp2f(fmaf(s[qb][i], scale_log2, -l2a[i]));
          pp[i] = m != 0.f ? pv : 0.f;
          dd[i] = m != 0.f ? pv * (dp[qb][i] - dla[i]) : 0.f;
        }
        ph[qb] = pack4<T>(pp);
        dh[qb] = pack4<T>(dd);
      }
      const uint4 bp = cat(ph[0], ph[1]), bd = cat(dh[0], dh[1]);
      const uint4 bpa = sel(left, bp), bpb = sel(!left, bp);
      const uint4 bda = sel(left, bd), bdb = sel(!left, bd);
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const uint32_t c = (uint32_t)(4 * hh + 2 * hf + (qq >> 1));
        const uint32_t hb = 8u * (uint32_t)(qq & 1);
        const uint4 da =
            cat(lds_tr8(sdo, lrow(ta0, c) + hb), lds_tr8(sdo, lrow(ta1, c) + hb));
        const uint4 db =
            cat(lds_tr8(sdo, lrow(tb0, c) + hb), lds_tr8(sdo, lrow(tb1, c) + hb));
        const uint4 qa = cat(lds_tr8(sq, lrow(ta0, c) + hb), lds_tr8(sq, lrow(ta1, c) + hb));
        const uint4 qb2 = cat(lds_tr8(sq, lrow(tb0, c) + hb), lds_tr8(sq, lrow(tb1, c) + hb));
        dva[hh][hf] = Mfma<T>::mma(da, bpa, dva[hh][hf]);
        dva[hh][hf] = Mfma<T>::mma(db, bpb, dva[hh][hf]);
        dka[hh][hf] = Mfma<T>::mma(qa, bda, dka[hh][hf]);
        dka[hh][hf] = Mfma<T>::mma(qb2, bdb, dka[hh][hf]);
      }
    }
  }
  ia += na;
  ib += nb;
}

template <typename T, int HP>
__global__ void __launch_bounds__(kTThreads)
bwdkv_tile_kernel(int H, int ntiles, float scale, const T* __restrict__ q,
                  const T* __restrict__ k, const T* __restrict__ v, const T* __restrict__ dout,
                  const float2* __restrict__ ld, uint32_t ld_none,
                  const int32_t* __restrict__ krec, const int32_t* __restrict__ kent,
                  const RevEntry* __restrict__ kitem, T* __restrict__ dk, T* __restrict__ dv) {
  __shared__ __attribute__((aligned(1024))) char lds[KLds::kBytes];
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  if (tile >= ntiles) return;
  const int hg = H / HP;
  const int w = tile / hg, h0 = (tile - w * hg) * HP;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int c16 = lane & 15, g = lane >> 4;
  const bool left = c16 < 8;
  const int32_t* rk = reinterpret_cast<const int32_t*>(lds + KLds::kRec);
  const float scale_log2 = scale * kLog2eT;

  copy_lds(krec, (uint32_t)(w * kKRec * 4), kKRec * 4, lds_addr(rk), lane, wv);
  wait_vm<0>();
  __syncthreads();
  const int start = __builtin_amdgcn_readfirstlane(rk[0]);
  const int E = __builtin_amdgcn_readfirstlane(rk[1]);
  const int base = __builtin_amdgcn_readfirstlane(rk[3]);
  const int nc = __builtin_amdgcn_readfirstlane(rk[4]);
  const int32_t* ktok = rk + 8;
  const int k0tok = __builtin_amdgcn_readfirstlane(ktok[0]);
  const int x0 = __builtin_amdgcn_readfirstlane(rk[72]);
  const int xend = __builtin_amdgcn_readfirstlane(rk[72 + 2 * (nc - 1)] + rk[73 + 2 * (nc - 1)]);
  const bool items_lds = xend - x0 <= kItemCap;
  if (items_lds)
    copy_lds(kitem, (uint32_t)x0 * 16u, (xend - x0) * 16, lds_addr(lds + KLds::kItems), lane, wv);
  const int n0 = min(E, kKRecEnt);
  const int32_t* tok0 = rk + kKRecHead;
  if (n0 > 0) kv_rows<HP>(q, dout, ld, ld_none, tok0, n0, k0tok, lds, base, H, h0, lane, wv);
  // own K and V rows of this wavefront's key clusters 2 wv, 2 wv + 1 (key
  // column c16 is row 16 wv + c16), straight to registers
  const bool active = 2 * wv < nc;
  const int tk = ktok[16 * wv + c16];
  uint4 kreg[HP], vreg[HP];
  {
    const uint32_t off =
        ((uint32_t)(base + (tk < 0 ? k0tok : tk)) * (uint32_t)H + (uint32_t)h0) * kRowB +
        16u * (uint32_t)g;
#pragma unroll
    for (int hh = 0; hh < HP; ++hh) {
      kreg[hh] = ld16(k, off + kRowB * hh);
      vreg[hh] = ld16(v, off + kRowB * hh);
    }
  }
  wait_vm<0>();
  __syncthreads();

  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  f32x4 dka[HP][2], dva[HP][2];
#pragma unroll
  for (int hh = 0; hh < HP; ++hh) {
    dka[hh][0] = dka[hh][1] = z;
    dva[hh][0] = dva[hh][1] = z;
  }
  // item cursors of the two key clusters (LDS or global item indices)
  const int ca = 2 * wv, cb = min(2 * wv + 1, nc - 1);
  const int bok = 2 * wv + 1 < nc;
  const int off = items_lds ? x0 : 0;
  int ia = __builtin_amdgcn_readfirstlane(rk[72 + 2 * ca]) - off;
  const int ia_end = ia + __builtin_amdgcn_readfirstlane(rk[73 + 2 * ca]);
  int ib = __builtin_amdgcn_readfirstlane(rk[72 + 2 * cb]) - off;
  const int ib_end = bok ? ib + __builtin_amdgcn_readfirstlane(rk[73 + 2 * cb]) : ib;
  const RevEntry* items_l = reinterpret_cast<const RevEntry*>(lds + KLds::kItems);
  int32_t* tokbuf = reinterpret_cast<int32_t*>(lds + KLds::kTok);

  for (int e0 = 0; e0 < E; e0 += kKRecEnt) {
    const int n = min(kKRecEnt, E - e0);
    if (e0 > 0) {   // a further chunk of merged entries: their tokens, then their rows
      __syncthreads();
      copy_lds(kent, (uint32_t)(start + e0) * (uint32_t)(kEnt * 4), n * kEnt * 4,
               lds_addr(tokbuf), lane, wv);
      wait_vm<0>();
      __syncthreads();
      kv_rows<HP>(q, dout, ld, ld_none, tokbuf, n, k0tok, lds, base, H, h0, lane, wv);
      wait_vm<0>();
      __syncthreads();
    }
    if (!active) continue;
    if (items_lds)
      kv_pair<T, HP>(lds, items_l, ia, ia_end, ib, ib_end, e0, n, kreg, vreg, scale_log2, dka,
                     dva, lane);
    else
      kv_pair<T, HP>(lds, kitem, ia, ia_end, ib, ib_end, e0, n, kreg, vreg, scale_log2, dka,
                     dva, lane);
  }
  if (!active) return;
  if (tk < 0 || (!left && !bok)) return;
  const uint32_t row = (uint32_t)(base + tk) * (uint32_t)H + (uint32_t)h0;
#pragma unroll
  for (int hh = 0; hh < HP; ++hh) {
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      stv<uint2>(dk, (row + hh) * kRowB + 32u * hf + 8u * g, pack4<T>(dka[hh][hf] * scale));
      stv<uint2>(dv, (row + hh) * kRowB + 32u * hf + 8u * g, pack4<T>(dva[hh][hf]));
    }
  }
}

// tiles = windows x head groups (two heads per tile when H is even)
template <typename T, int NB, int HP>
hipError_t fwd_tile_t(int B, int C, int H, int nk, float scale, const void* q, const void* k,
                      const void* v, const BwdWorkspace& w, void* o, float* lse,
                      hipStream_t st) {
  const int64_t ntiles = windows_of(B, C) * (H / HP);
  if (ntiles == 0) return hipSuccess;
  hipLaunchKernelGGL((fwd_tile_kernel<T, NB, HP>), dim3((unsigned)ntiles), dim3(kTThreads), 0, st,
                     H, (int)ntiles, qrec_slots(nk), scale * kLog2eT, (const T*)q, (const T*)k,
                     (const T*)v, (const int32_t*)w.qrec, (T*)o, lse);
  return hipGetLastError();
}

template <typename T, int NB, int HP>
hipError_t bwd_tile_t(int pass, int B, int C, int H, int nk, float scale, const void* q,
                      const void* k, const void* v, const void* o, const void* dout,
                      const float* lse, void* dq, void* dk, void* dv, const BwdWorkspace& w,
                      hipStream_t st) {
  const int64_t ntiles = windows_of(B, C) * (H / HP);
  if (ntiles == 0) return hipSuccess;
  if (pass & 1)
    hipLaunchKernelGGL((bwdq_tile_kernel<T, NB, HP>), dim3((unsigned)ntiles), dim3(kTThreads), 0,
                       st, H, (int)ntiles, qrec_slots(nk), scale, (const T*)q, (const T*)k,
                       (const T*)v, (const T*)o, (const T*)dout, lse, (const int32_t*)w.qrec,
                       (T*)dq, w.ld, w.ld_none);
  if (pass & 2) {
    const uint32_t ld_none = (uint32_t)((const char*)w.ld_none - (const char*)w.ld);
    hipLaunchKernelGGL((bwdkv_tile_kernel<T, HP>), dim3((unsigned)ntiles), dim3(kTThreads), 0, st,
                       H, (int)ntiles, scale, (const T*)q, (const T*)k, (const T*)v,
                       (const T*)dout, (const float2*)w.ld, ld_none, (const int32_t*)w.krec,
                       (const int32_t*)w.kent, (const RevEntry*)w.kitem, (T*)dk, (T*)dv);
  }
  return hipGetLastError();
}

template <typename T, int HP>
hipError_t fwd_tile_nb(int B, int C, int H, int nk, float scale, const void* q, const void* k,
                       const void* v, const BwdWorkspace& w, void* o, float* lse,
                       hipStream_t st) {
  switch ((nk + 15) >> 4) {
    case 1: return fwd_tile_t<T, 1, HP>(B, C, H, nk, scale, q, k, v, w, o, lse, st);
    case 2: return fwd_tile_t<T, 2, HP>(B, C, H, nk, scale, q, k, v, w, o, lse, st);
    case 3: return fwd_tile_t<T, 3, HP>(B, C, H, nk, scale, q, k, v, w, o, lse, st);
    default: return fwd_tile_t<T, 4, HP>(B, C, H, nk, scale, q, k, v, w, o, lse, st);
  }
}

template <typename T, int HP>
hipError_t bwd_tile_nb(int pass, int B, int C, int H, int nk, float scale, const void* q,
                       const void* k, const void* v, const void* o, const void* dout,
                       const float* lse, void* dq, void* dk, void* dv, const BwdWorkspace& w,
                       hipStream_t st) {
  switch ((nk + 15) >> 4) {
    case 1: return bwd_tile_t<T, 1, HP>(pass, B, C, H, nk, scale, q, k, v, o, dout, lse, dq, dk, dv, w, st);
    case 2: return bwd_tile_t<T, 2, HP>(pass, B, C, H, nk, scale, q, k, v, o, dout, lse, dq, dk, dv, w, st);
    case 3: return bwd_tile_t<T, 3, HP>(pass, B, C, H, nk, scale, q, k, v, o, dout, lse, dq, dk, dv, w, st);
    default: return bwd_tile_t<T, 4, HP>(pass, B, C, H, nk, scale, q, k, v, o, dout, lse, dq, dk, dv, w, st);
  }
}

template <typename T>
hipError_t fwd_tile_hp(int B, int C, int H, int nk, float scale, const void* q, const void* k,
                       const void* v, const BwdWorkspace& w, void* o, float* lse,
                       hipStream_t st) {
  if (H % 2 == 0) return fwd_tile_nb<T, 2>(B, C, H, nk, scale, q, k, v, w, o, lse, st);
  return fwd_tile_nb<T, 1>(B, C, H, nk, scale, q, k, v, w, o, lse, st);
}

template <typename T>
hipError_t bwd_tile_hp(int pass, int B, int C, int H, int nk, float scale, const void* q,
                       const void* k, const void* v, const void* o, const void* dout,
                       const float* lse, void* dq, void* dk, void* dv, const BwdWorkspace& w,
                       hipStream_t st) {
  if (H % 2 == 0)
    return bwd_tile_nb<T, 2>(pass, B, C, H, nk, scale, q, k, v, o, dout, lse, dq, dk, dv, w, st);
  return bwd_tile_nb<T, 1>(pass, B, C, H, nk, scale, q, k, v, o, dout, lse, dq, dk, dv, w, st);
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
  if (dt == 1) return fwd_tile_hp<bf16>(B, C, H, nk, scale, q, k, v, w, o, lse, st);
  if (dt == 2) return fwd_tile_hp<f16>(B, C, H, nk, scale, q, k, v, w, o, lse, st);
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_tile(int pass, int dt, int B, int N, int C, int H, int nk, float scale,
                           const void* q, const void* k, const void* v, const void* o,
                           const void* dout, const float* lse, void* dq, void* dk, void* dv,
                           const BwdWorkspace& w, hipStream_t st) {
  (void)N;
  if (dt == 1)
    return bwd_tile_hp<bf16>(pass, B, C, H, nk, scale, q, k, v, o, dout, lse, dq, dk, dv, w, st);
  if (dt == 2)
    return bwd_tile_hp<f16>(pass, B, C, H, nk, scale, q, k, v, o, dout, lse, dq, dk, dv, w, st);
  return hipErrorInvalidValue;
}

}  // namespace ca
