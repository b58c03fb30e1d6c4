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
// consecutive clusters, head); the window plan (tile_plan.hip) describes it.
//  * Forward and query-major backward pass: the workgroup stages the
//    window's 64 query rows and the distinct key (and value) rows of its
//    lists once in LDS with direct-to-LDS loads, four lanes per 64-byte row;
//    at the stage-1 shape a window's 384 slots hold about 144 distinct keys,
//    so each key row is gathered 2.7 times less often than per cluster.
//    Each wavefront then computes one pair of clusters, each on its own 48
//    slots only: the two clusters share a 16-column MFMA tile (columns 0-7
//    and 8-15), block-diagonal over two 16x16x32 MFMAs whose A operands are
//    the two clusters' slot rows, read from LDS through the plan's slot
//    table.  The softmax (fp32, row maximum, exp2) runs on 12 logits per
//    lane; O^T = V^T P^T reads V transposed (ds_read_b64_tr_b16).
//  * Query-major backward: dS = P (dP - Delta), dQ^T = K^T dS^T; writes dQ
//    and (LSE log2 e, Delta) per query row for the key-major pass.
//  * Key-major backward: the window's 64 key rows (own K, V in registers),
//    the rows of the query clusters reading them (merged, so each query row
//    is gathered once per window) staged in LDS 24 clusters at a time; each
//    wavefront takes a pair of key clusters and walks their (query cluster,
//    multiplicities) items four at a time: S = Q K^T, dP = dO V^T,
//    dV^T += dO^T P, dK^T += Q^T dS.  Each dK/dV row is written once by one
//    workgroup: no atomics, bitwise reproducible.
//  * Row r of a staged block keeps 16-byte chunk c at position
//    c ^ row_swz(r), a swizzle under which both the MFMA row reads (16 rows,
//    one chunk) and the transposing reads (4 rows, two chunks) spread over
//    the LDS banks.
//  * Workgroups are numbered so that each XCD takes a contiguous range of
//    windows (all heads): the rows shared by neighbouring windows and the
//    heads of one token row stay in that XCD's L2.
#include "common.h"
#include "mfma_util.h"

namespace ca {

namespace {

constexpr int kTThreads = 256;   // four wavefronts per tile
constexpr uint32_t kRowB = 64;   // bytes of one head row
constexpr float kLog2eT = 1.4426950408889634f;
constexpr float kLn2T = 0.6931471805599453f;

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)p;
}

// byte offset of chunk `chunk` of row `r` of a staged block
__device__ __forceinline__ uint32_t row_chunk(int r, uint32_t chunk) {
  return (uint32_t)r * kRowB + 16u * (chunk ^ row_swz(r));
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

// Gather the head-h rows of `nrows` tokens (a multiple of 16) into a staged
// block: instruction i fills rows 16 i .. 16 i + 15 (wavefront wv issues
// i = wv, wv + 4, ...); lane l fetches chunk (l & 3) ^ row_swz(row) of row
// 16 i + l / 4, so that position l & 3 of the row holds it.  `toks` (LDS):
// the tokens of rows below `nvalid`; -1, and every row from nvalid on, take
// `fallback`.
__device__ __forceinline__ void gather_rows(const void* src, const int32_t* toks, int fallback,
                                            int nrows, int nvalid, uint32_t dst, int base, int H,
                                            int h, int lane, int wv) {
  for (int i = wv; 16 * i < nrows; i += 4) {
    const int row = 16 * i + (lane >> 2);
    int t = row < nvalid ? toks[row] : -1;
    t = t < 0 ? fallback : t;
    const uint32_t chunk = (uint32_t)(lane & 3) ^ row_swz(row);
    dma16(src, ((uint32_t)(base + t) * (uint32_t)H + (uint32_t)h) * kRowB + 16u * chunk,
          dst + 1024u * (uint32_t)i);
  }
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
// query-major staging: the query record of a (sub-)window, its 64 query
// rows, the key and value rows of its distinct keys (and, for the
// backward, the dO and O rows and the LSE of the queries)
// ---------------------------------------------------------------------------
struct QLds {
  static constexpr int kRec = 0, kQ = 2304, kK = kQ + 4096, kV = kK + 64 * kUnionCap,
                       kFwdBytes = kV + 64 * kUnionCap, kDo = kFwdBytes, kO = kDo + 4096,
                       kLse = kO + 4096, kBwdBytes = kLse + 256;
};
static_assert(kQRec * 4 <= QLds::kQ, "query record fits its LDS region");
static_assert(kUnionCap % 32 == 0, "staged key rows come in groups of 32");

// Stage one (sub-)window record at `rec_off` (ints) and its rows.  Returns
// the record's cluster count.  `bwd`: also dO, O and the LSE.
template <bool BWD>
__device__ __forceinline__ int stage_window(const int32_t* qrec, int64_t rec_off, char* lds,
                                            const void* q, const void* k, const void* v,
                                            const void* o, const void* dout, const float* lse,
                                            int H, int h, int lane, int wv) {
  const int32_t* rec = reinterpret_cast<const int32_t*>(lds + QLds::kRec);
  copy_lds(qrec, (uint32_t)(rec_off * 4), kQRec * 4, lds_addr(rec), lane, wv);
  wait_vm<0>();
  __syncthreads();
  // a split window's own record only says how to find its sub-windows
  if (__builtin_amdgcn_readfirstlane(rec[4]) & kQSplit) return 0;
  const int u = __builtin_amdgcn_readfirstlane(rec[2]);
  const int base = __builtin_amdgcn_readfirstlane(rec[3]);
  const int q0 = __builtin_amdgcn_readfirstlane(rec[8]);
  const int32_t* qtok = rec + 8;
  const int upad = (u + 31) & ~31;
  gather_rows(q, qtok, q0, 64, 64, lds_addr(lds + QLds::kQ), base, H, h, lane, wv);
  gather_rows(k, rec + kQRecHead, q0, upad, upad, lds_addr(lds + QLds::kK), base, H, h, lane, wv);
  gather_rows(v, rec + kQRecHead, q0, upad, upad, lds_addr(lds + QLds::kV), base, H, h, lane, wv);
  if (BWD) {
    gather_rows(dout, qtok, q0, 64, 64, lds_addr(lds + QLds::kDo), base, H, h, lane, wv);
    gather_rows(o, qtok, q0, 64, 64, lds_addr(lds + QLds::kO), base, H, h, lane, wv);
    if (wv == 0) {
      const int t = qtok[lane] < 0 ? q0 : qtok[lane];
      dma4(lse, ((uint32_t)(base + t) * (uint32_t)H + (uint32_t)h) * 4u,
           lds_addr(lds + QLds::kLse));
    }
  }
  wait_vm<0>();
  __syncthreads();
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

// ---------------------------------------------------------------------------
// forward: one pair of clusters (2p, 2p + 1) of the staged record
// ---------------------------------------------------------------------------
template <typename T, int NB, bool HOLES>
__device__ void fwd_pair(const char* lds, int p, int nc, int H, int h, float csl, bool neg,
                         T* __restrict__ o, float* __restrict__ lse, int lane) {
  const int32_t* rec = reinterpret_cast<const int32_t*>(lds + QLds::kRec);
  const uint16_t* tab = reinterpret_cast<const uint16_t*>(rec + kQSlotOff);
  const unsigned long long* masks = reinterpret_cast<const unsigned long long*>(rec + kQMaskOff);
  const char* sq = lds + QLds::kQ;
  const char* sk = lds + QLds::kK;
  const char* sv = lds + QLds::kV;
  const int base = rec[3];
  const int c16 = lane & 15, g = lane >> 4, e = c16 >> 2, qq = c16 & 3;
  const bool left = c16 < 8;
  const int a = 2 * p, b = min(2 * p + 1, nc - 1);   // an absent b reads a valid cluster
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};

  uint4 qv = lds16(sq, row_chunk(16 * p + c16, (uint32_t)g));
  if (neg) {   // a negative scale: -|scale| with Q negated (exact)
    qv.x ^= 0x80008000u;
    qv.y ^= 0x80008000u;
    qv.z ^= 0x80008000u;
    qv.w ^= 0x80008000u;
  }
  const uint4 qL = sel(left, qv), qR = sel(!left, qv);
  uint32_t ka[4], kb[4], va[4], vb[4];
  slot_offsets(tab, a, c16, ka);
  slot_offsets(tab, b, c16, kb);
  slot_offsets(tab, a, 4 * g + e, va);
  slot_offsets(tab, b, 4 * g + e, vb);
  const uint32_t gx = 16u * (uint32_t)g;
  f32x4 s[NB];
#pragma unroll
  for (int blk = 0; blk < NB; ++blk) {
    s[blk] = Mfma<T>::mma(lds16(sk, ka[blk] ^ gx), qL, z);
    s[blk] = Mfma<T>::mma(lds16(sk, kb[blk] ^ gx), qR, s[blk]);
  }
  uint32_t vm[NB];
  if (HOLES) {
    const bool bok = 2 * p + 1 < nc;
    const unsigned long long m = left ? masks[a] : (bok ? masks[b] : 0ull);
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) vm[blk] = (uint32_t)(m >> (16 * blk + 4 * g)) & 0xfu;
  }
  float mx = -INFINITY;
#pragma unroll
  for (int blk = 0; blk < NB; ++blk)
#pragma unroll
    for (int i = 0; i < 4; ++i) mx = fmaxf(mx, HOLES && !((vm[blk] >> i) & 1u) ? -INFINITY : s[blk][i]);
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
      const uint32_t x = 16u * (uint32_t)(2 * hf + (qq >> 1)) + 8u * (uint32_t)(qq & 1);
      const uint4 aa = cat(lds_tr8(sv, va[b0] ^ x), lds_tr8(sv, va[b1] ^ x));
      const uint4 ab = cat(lds_tr8(sv, vb[b0] ^ x), lds_tr8(sv, vb[b1] ^ x));
      oacc[hf] = Mfma<T>::mma(aa, bpa, oacc[hf]);
      oacc[hf] = Mfma<T>::mma(ab, bpb, oacc[hf]);
    }
  }
  const int tq = rec[8 + 16 * p + c16];
  if (tq < 0) return;
  const float inv = l > 0.f ? __builtin_amdgcn_rcpf(l) : 0.f;
  const uint32_t qrow = (uint32_t)(base + tq) * (uint32_t)H + (uint32_t)h;
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
    stv<uint2>(o, qrow * kRowB + 32u * hf + 8u * g, pack4<T>(oacc[hf] * inv));
  if (g == 0) lse[qrow] = l > 0.f ? (mref + __log2f(l)) * kLn2T : -INFINITY;
}

template <typename T, int NB>
__device__ __forceinline__ void fwd_pair_any(const char* lds, int p, int nc, int H, int h,
                                             float csl, bool neg, T* o, float* lse, int lane) {
  const int32_t* rec = reinterpret_cast<const int32_t*>(lds + QLds::kRec);
  if (rec[2] == 0) {   // no slot of the window holds a token: O = 0, LSE = -inf
    const int c16 = lane & 15, g = lane >> 4;
    const int tq = rec[8 + 16 * p + c16];
    if (tq < 0) return;
    const uint32_t qrow = (uint32_t)(rec[3] + tq) * (uint32_t)H + (uint32_t)h;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) stv<uint2>(o, qrow * kRowB + 32u * hf + 8u * g, make_uint2(0u, 0u));
    if (g == 0) lse[qrow] = -INFINITY;
    return;
  }
  const bool holes = (rec[4] & kQHoles) || 2 * p + 1 >= nc;
  if (holes) fwd_pair<T, NB, true>(lds, p, nc, H, h, csl, neg, o, lse, lane);
  else fwd_pair<T, NB, false>(lds, p, nc, H, h, csl, neg, o, lse, lane);
}

template <typename T, int NB>
__global__ void __launch_bounds__(kTThreads)
fwd_tile_kernel(int H, int ntiles, int nrec, float scale_log2, const T* __restrict__ q,
                const T* __restrict__ k, const T* __restrict__ v, const int32_t* __restrict__ qrec,
                T* __restrict__ o, float* __restrict__ lse) {
  __shared__ __attribute__((aligned(1024))) char lds[QLds::kFwdBytes];
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  if (tile >= ntiles) return;
  const int w = tile / H, h = tile - w * H;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const bool neg = scale_log2 < 0.f;
  const float csl = fabsf(scale_log2);
  const int64_t r0 = (int64_t)w * nrec * kQRecStride;
  int nc = stage_window<false>(qrec, r0, lds, q, k, v, nullptr, nullptr, nullptr, H, h, lane, wv);
  const int32_t* rec = reinterpret_cast<const int32_t*>(lds + QLds::kRec);
  if (!(rec[4] & kQSplit)) {
    if (2 * wv < nc) fwd_pair_any<T, NB>(lds, wv, nc, H, h, csl, neg, o, lse, lane);
    return;
  }
  // more distinct keys than one staging holds: the sub-windows one by one
  const int nsub = __builtin_amdgcn_readfirstlane(rec[5]);
  for (int s = 0; s < nsub; ++s) {
    __syncthreads();
    nc = stage_window<false>(qrec, r0 + (int64_t)(1 + s) * kQRecStride, lds, q, k, v, nullptr,
                             nullptr, nullptr, H, h, lane, wv);
    const int p = my_pair(wv, s, nsub);
    if (p >= 0 && 2 * p < nc) fwd_pair_any<T, NB>(lds, p, nc, H, h, csl, neg, o, lse, lane);
  }
}

// ---------------------------------------------------------------------------
// backward, query-major pass: one pair of clusters (2p, 2p + 1)
// ---------------------------------------------------------------------------
template <typename T, int NB, bool HOLES>
__device__ void bwdq_pair(const char* lds, int p, int nc, int H, int h, float scale,
                          T* __restrict__ dq, float2* __restrict__ ld, int lane) {
  const int32_t* rec = reinterpret_cast<const int32_t*>(lds + QLds::kRec);
  const uint16_t* tab = reinterpret_cast<const uint16_t*>(rec + kQSlotOff);
  const unsigned long long* masks = reinterpret_cast<const unsigned long long*>(rec + kQMaskOff);
  const char* sq = lds + QLds::kQ;
  const char* sk = lds + QLds::kK;
  const char* sv = lds + QLds::kV;
  const char* sdo = lds + QLds::kDo;
  const char* so = lds + QLds::kO;
  const float* sl = reinterpret_cast<const float*>(lds + QLds::kLse);
  const int base = rec[3];
  const int c16 = lane & 15, g = lane >> 4, e = c16 >> 2, qq = c16 & 3;
  const bool left = c16 < 8;
  const int a = 2 * p, b = min(2 * p + 1, nc - 1);
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  const float scale_log2 = scale * kLog2eT;

  const int row = 16 * p + c16;
  const uint4 qv = lds16(sq, row_chunk(row, (uint32_t)g));
  const uint4 dov = lds16(sdo, row_chunk(row, (uint32_t)g));
  const uint4 ov = lds16(so, row_chunk(row, (uint32_t)g));
  const float lse2 = sl[row] * kLog2eT;
  // Delta of the column's query: eight dims per lane, summed over the 4 lanes
  float dl = 0.f;
  {
    const uint32_t x[4] = {dov.x, dov.y, dov.z, dov.w};
    const uint32_t y[4] = {ov.x, ov.y, ov.z, ov.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x2 xa = Mfma<T>::unpack(x[i]), ya = Mfma<T>::unpack(y[i]);
      dl = fmaf(xa[0], ya[0], fmaf(xa[1], ya[1], dl));
    }
  }
  dl = shfl_sum16_32(dl);
  const uint4 qL = sel(left, qv), qR = sel(!left, qv);
  const uint4 dL = sel(left, dov), dR = sel(!left, dov);
  uint32_t ka[4], kb[4], va[4], vb[4];
  slot_offsets(tab, a, c16, ka);
  slot_offsets(tab, b, c16, kb);
  slot_offsets(tab, a, 4 * g + e, va);
  slot_offsets(tab, b, 4 * g + e, vb);
  const uint32_t gx = 16u * (uint32_t)g;
  uint32_t vm[NB];
  if (HOLES) {
    const bool bok = 2 * p + 1 < nc;
    const unsigned long long m = left ? masks[a] : (bok ? masks[b] : 0ull);
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) vm[blk] = (uint32_t)(m >> (16 * blk + 4 * g)) & 0xfu;
  }
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
      const uint32_t x = 16u * (uint32_t)(2 * hf + (qq >> 1)) + 8u * (uint32_t)(qq & 1);
      const uint4 aa = cat(lds_tr8(sk, va[b0] ^ x), lds_tr8(sk, va[b1] ^ x));
      const uint4 ab = cat(lds_tr8(sk, vb[b0] ^ x), lds_tr8(sk, vb[b1] ^ x));
      acc[hf] = Mfma<T>::mma(aa, bda, acc[hf]);
      acc[hf] = Mfma<T>::mma(ab, bdb, acc[hf]);
    }
  }
  const int tq = rec[8 + row];
  if (tq < 0) return;
  const uint32_t qrow = (uint32_t)(base + tq) * (uint32_t)H + (uint32_t)h;
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
    stv<uint2>(dq, qrow * kRowB + 32u * hf + 8u * g, pack4<T>(acc[hf] * scale));
  if (g == 0) ld[qrow] = make_float2(lse2, dl);
}

template <typename T, int NB>
__device__ __forceinline__ void bwdq_pair_any(const char* lds, int p, int nc, int H, int h,
                                              float scale, T* dq, float2* ld, int lane) {
  const int32_t* rec = reinterpret_cast<const int32_t*>(lds + QLds::kRec);
  if (rec[2] == 0) {   // no slot of the window holds a token: dQ = 0
    const int c16 = lane & 15, g = lane >> 4;
    const int tq = rec[8 + 16 * p + c16];
    if (tq < 0) return;
    const uint32_t qrow = (uint32_t)(rec[3] + tq) * (uint32_t)H + (uint32_t)h;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) stv<uint2>(dq, qrow * kRowB + 32u * hf + 8u * g, make_uint2(0u, 0u));
    if (g == 0) ld[qrow] = make_float2(-INFINITY, 0.f);
    return;
  }
  const bool holes = (rec[4] & kQHoles) || 2 * p + 1 >= nc;
  if (holes) bwdq_pair<T, NB, true>(lds, p, nc, H, h, scale, dq, ld, lane);
  else bwdq_pair<T, NB, false>(lds, p, nc, H, h, scale, dq, ld, lane);
}

template <typename T, int NB>
__global__ void __launch_bounds__(kTThreads)
bwdq_tile_kernel(int H, int ntiles, int nrec, float scale, const T* __restrict__ q,
                 const T* __restrict__ k, const T* __restrict__ v, const T* __restrict__ o,
                 const T* __restrict__ dout, const float* __restrict__ lse,
                 const int32_t* __restrict__ qrec, T* __restrict__ dq, float2* __restrict__ ld,
                 float4* __restrict__ ld_none) {
  __shared__ __attribute__((aligned(1024))) char lds[QLds::kBwdBytes];
  // the (LSE log2 e, Delta) pair the key-major pass reads for an absent
  // query: P = exp2(s - inf) = 0 there
  if (blockIdx.x == 0 && threadIdx.x == 0) *ld_none = make_float4(INFINITY, 0.f, INFINITY, 0.f);
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  if (tile >= ntiles) return;
  const int w = tile / H, h = tile - w * H;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int64_t r0 = (int64_t)w * nrec * kQRecStride;
  int nc = stage_window<true>(qrec, r0, lds, q, k, v, o, dout, lse, H, h, lane, wv);
  const int32_t* rec = reinterpret_cast<const int32_t*>(lds + QLds::kRec);
  if (!(rec[4] & kQSplit)) {
    if (2 * wv < nc) bwdq_pair_any<T, NB>(lds, wv, nc, H, h, scale, dq, ld, lane);
    return;
  }
  const int nsub = __builtin_amdgcn_readfirstlane(rec[5]);
  for (int s = 0; s < nsub; ++s) {
    __syncthreads();
    nc = stage_window<true>(qrec, r0 + (int64_t)(1 + s) * kQRecStride, lds, q, k, v, o, dout,
                            lse, H, h, lane, wv);
    const int p = my_pair(wv, s, nsub);
    if (p >= 0 && 2 * p < nc) bwdq_pair_any<T, NB>(lds, p, nc, H, h, scale, dq, ld, lane);
  }
}

// ---------------------------------------------------------------------------
// backward, key-major pass
// ---------------------------------------------------------------------------
// LDS of one key window: its record (with the first merged entries' query
// tokens), the items of its key clusters (when there are at most kItemCap),
// the query tokens of later chunks of merged entries, the Q and dO rows and
// the (LSE log2 e, Delta) pairs of up to kKRecEnt merged entries, and the
// window's own K and V rows.
constexpr int kItemCap = 128;
struct KLds {
  static constexpr int kRec = 0, kItems = 1152, kTok = kItems + 16 * kItemCap,
                       kQ = kTok + 32 * kKRecEnt, kDo = kQ + 64 * 8 * kKRecEnt,
                       kL2 = kDo + 64 * 8 * kKRecEnt, kDl = kL2 + 32 * kKRecEnt,
                       kKo = kDl + 32 * kKRecEnt, kVo = kKo + 4096, kBytes = kVo + 4096;
};
static_assert(kKRec * 4 <= KLds::kItems, "key record fits its LDS region");

// rows of merged entries [e0, e0 + n) (n <= kKRecEnt; their tokens at `tok`):
// row 8 x + m = member m of entry e0 + x; Q and dO rows, and the (LSE log2 e,
// Delta) pairs as two 4-byte gathers (an absent member reads the (+inf, 0)
// pair at byte offset ld_none)
__device__ __forceinline__ void kv_rows(const void* q, const void* dout, const float2* ld,
                                        uint32_t ld_none, const int32_t* tok, int n, int fallback,
                                        char* lds, int base, int H, int h, int lane, int wv) {
  const int nrows = 8 * n;
  gather_rows(q, tok, fallback, (nrows + 15) & ~15, nrows, lds_addr(lds + KLds::kQ), base, H, h,
              lane, wv);
  gather_rows(dout, tok, fallback, (nrows + 15) & ~15, nrows, lds_addr(lds + KLds::kDo), base, H,
              h, lane, wv);
  for (int i = wv; 64 * i < nrows; i += 4) {
    const int row = 64 * i + lane;
    const int t = row < nrows ? tok[row] : -1;
    const uint32_t off =
        t >= 0 ? ((uint32_t)(base + t) * (uint32_t)H + (uint32_t)h) * 8u : ld_none;
    dma4(ld, off, lds_addr(lds + KLds::kL2) + 256u * (uint32_t)i);
    dma4(ld, off + 4u, lds_addr(lds + KLds::kDl) + 256u * (uint32_t)i);
  }
}

// One pair of key clusters (2 p, 2 p + 1) over the staged merged entries
// [e0, e0 + n): their items with a merged index in that range, four at a
// time in lockstep.  `items` (LDS or global) holds the window's items;
// [ia, ia_end) and [ib, ib_end) are the two clusters' remaining ranges (the
// cursors advance past the processed items).
template <typename T, bool GLOBAL_ITEMS>
__device__ void kv_pair(const char* lds, const RevEntry* items, int& ia, int ia_end, int& ib,
                        int ib_end, int e0, int n, const uint4 (&kreg)[2], const uint4 (&vreg)[2],
                        float scale_log2, f32x4 (&dka)[2], f32x4 (&dva)[2], int lane) {
  const char* sq = lds + KLds::kQ;
  const char* sdo = lds + KLds::kDo;
  const float* sl2 = reinterpret_cast<const float*>(lds + KLds::kL2);
  const float* sdl = reinterpret_cast<const float*>(lds + KLds::kDl);
  const int c16 = lane & 15, g = lane >> 4, e = c16 >> 2, qq = c16 & 3;
  const bool left = c16 < 8;
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  const uint4 kL = sel(left, kreg[0]), kR = sel(!left, kreg[0]);
  const uint4 vL = sel(left, vreg[0]), vR = sel(!left, vreg[0]);
  (void)kreg[1];
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
      const bool oka = t < na, okb = t < nb;
      ra[x] = 0;
      rb[x] = 0;
      ma[x] = 0ull;
      mb[x] = 0ull;
      if (oka) {
        const RevEntry ea = items[ia + t];
        ra[x] = 8 * (ea.i - e0);
        ma[x] = ea.mult;
      }
      if (okb) {
        const RevEntry eb = items[ib + t];
        rb[x] = 8 * (eb.i - e0);
        mb[x] = eb.mult;
      }
    }
    // S = Q K^T and dP = dO V^T per 16-row block (items 2 qb, 2 qb + 1):
    // columns 0-7 are a's keys over a's item rows, 8-15 b's over b's
    f32x4 s[2], dp[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int xa = 2 * qb + (c16 >> 3);
      const int rowa = (xa == 0 ? ra[0] : xa == 1 ? ra[1] : xa == 2 ? ra[2] : ra[3]) + (c16 & 7);
      const int rowb = (xa == 0 ? rb[0] : xa == 1 ? rb[1] : xa == 2 ? rb[2] : rb[3]) + (c16 & 7);
      s[qb] = Mfma<T>::mma(lds16(sq, row_chunk(rowa, (uint32_t)g)), kL, z);
      s[qb] = Mfma<T>::mma(lds16(sq, row_chunk(rowb, (uint32_t)g)), kR, s[qb]);
      dp[qb] = Mfma<T>::mma(lds16(sdo, row_chunk(rowa, (uint32_t)g)), vL, z);
      dp[qb] = Mfma<T>::mma(lds16(sdo, row_chunk(rowb, (uint32_t)g)), vR, dp[qb]);
    }
    // P and dS: lane (key column c16, row group g) holds rows 4 g .. 4 g + 3
    // of each block, i.e. members 4 (g & 1) .. + 3 of item 2 qb + (g >> 1)
    // of its own cluster
    uint2 ph[2], dh[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int x = 2 * qb + (g >> 1);
      const int rbase = left ? (x == 0 ? ra[0] : x == 1 ? ra[1] : x == 2 ? ra[2] : ra[3])
                             : (x == 0 ? rb[0] : x == 1 ? rb[1] : x == 2 ? rb[2] : rb[3]);
      const uint64_t mm = left ? (x == 0 ? ma[0] : x == 1 ? ma[1] : x == 2 ? ma[2] : ma[3])
                               : (x == 0 ? mb[0] : x == 1 ? mb[1] : x == 2 ? mb[2] : mb[3]);
      const float m = (float)((uint32_t)(mm >> (8 * (c16 & 7))) & 0xffu);
      const int r = rbase + 4 * (g & 1);
      const float4 l2 = *reinterpret_cast<const float4*>(sl2 + r);
      const float4 dl4 = *reinterpret_cast<const float4*>(sdl + r);
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
    // dV^T += dO^T P and dK^T += Q^T dS: lane 4 e + qq of row group g reads
    // rows 16 blk + 4 g + e = member 4 (g & 1) + e of item 2 blk + (g >> 1)
    const int xa0 = (g >> 1), xa1 = 2 + (g >> 1);
    const int mrow = 4 * (g & 1) + e;
    const int ta0 = (xa0 == 0 ? ra[0] : ra[1]) + mrow, ta1 = (xa1 == 2 ? ra[2] : ra[3]) + mrow;
    const int tb0 = (xa0 == 0 ? rb[0] : rb[1]) + mrow, tb1 = (xa1 == 2 ? rb[2] : rb[3]) + mrow;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const uint32_t c = (uint32_t)(2 * hf + (qq >> 1));
      const uint32_t hb = 8u * (uint32_t)(qq & 1);
      const uint4 da = cat(lds_tr8(sdo, row_chunk(ta0, c) + hb), lds_tr8(sdo, row_chunk(ta1, c) + hb));
      const uint4 db = cat(lds_tr8(sdo, row_chunk(tb0, c) + hb), lds_tr8(sdo, row_chunk(tb1, c) + hb));
      const uint4 qa = cat(lds_tr8(sq, row_chunk(ta0, c) + hb), lds_tr8(sq, row_chunk(ta1, c) + hb));
      const uint4 qb2 = cat(lds_tr8(sq, row_chunk(tb0, c) + hb), lds_tr8(sq, row_chunk(tb1, c) + hb));
      dva[hf] = Mfma<T>::mma(da, bpa, dva[hf]);
      dva[hf] = Mfma<T>::mma(db, bpb, dva[hf]);
      dka[hf] = Mfma<T>::mma(qa, bda, dka[hf]);
      dka[hf] = Mfma<T>::mma(qb2, bdb, dka[hf]);
    }
  }
  ia += na;
  ib += nb;
}

template <typename T>
__global__ void __launch_bounds__(kTThreads)
bwdkv_tile_kernel(int H, int ntiles, float scale, const T* __restrict__ q,
                  const T* __restrict__ k, const T* __restrict__ v, const T* __restrict__ dout,
                  const float2* __restrict__ ld, uint32_t ld_none,
                  const int32_t* __restrict__ krec, const int32_t* __restrict__ kent,
                  const RevEntry* __restrict__ kitem, T* __restrict__ dk, T* __restrict__ dv) {
  __shared__ __attribute__((aligned(1024))) char lds[KLds::kBytes];
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  if (tile >= ntiles) return;
  const int w = tile / H, h = tile - w * H;
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
  gather_rows(k, ktok, k0tok, 64, 64, lds_addr(lds + KLds::kKo), base, H, h, lane, wv);
  gather_rows(v, ktok, k0tok, 64, 64, lds_addr(lds + KLds::kVo), base, H, h, lane, wv);
  if (items_lds)
    copy_lds(kitem, (uint32_t)x0 * 16u, (xend - x0) * 16, lds_addr(lds + KLds::kItems), lane, wv);
  const int n0 = min(E, kKRecEnt);
  const int32_t* tok0 = rk + kKRecHead;
  if (n0 > 0) kv_rows(q, dout, ld, ld_none, tok0, n0, k0tok, lds, base, H, h, lane, wv);
  wait_vm<0>();
  __syncthreads();

  // own K and V rows of this wavefront's key clusters 2 wv, 2 wv + 1: key
  // column c16 is row 16 wv + c16
  const bool active = 2 * wv < nc;
  uint4 kreg[2], vreg[2];
  const int krow = 16 * wv + c16;
  kreg[0] = lds16(lds + KLds::kKo, row_chunk(krow, (uint32_t)g));
  vreg[0] = lds16(lds + KLds::kVo, row_chunk(krow, (uint32_t)g));
  kreg[1] = kreg[0];
  vreg[1] = vreg[0];
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  f32x4 dka[2] = {z, z}, dva[2] = {z, z};
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
      kv_rows(q, dout, ld, ld_none, tokbuf, n, k0tok, lds, base, H, h, lane, wv);
      wait_vm<0>();
      __syncthreads();
    }
    if (!active) continue;
    if (items_lds)
      kv_pair<T, false>(lds, items_l, ia, ia_end, ib, ib_end, e0, n, kreg, vreg, scale_log2, dka,
                        dva, lane);
    else
      kv_pair<T, true>(lds, kitem, ia, ia_end, ib, ib_end, e0, n, kreg, vreg, scale_log2, dka,
                       dva, lane);
  }
  if (!active) return;
  const int tk = ktok[16 * wv + c16];
  if (tk < 0 || (!left && !bok)) return;
  const uint32_t row = (uint32_t)(base + tk) * (uint32_t)H + (uint32_t)h;
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    stv<uint2>(dk, row * kRowB + 32u * hf + 8u * g, pack4<T>(dka[hf] * scale));
    stv<uint2>(dv, row * kRowB + 32u * hf + 8u * g, pack4<T>(dva[hf]));
  }
}

template <typename T, int NB>
hipError_t fwd_tile_t(int B, int C, int H, int nk, float scale, const void* q, const void* k,
                      const void* v, const BwdWorkspace& w, void* o, float* lse,
                      hipStream_t st) {
  const int64_t ntiles = windows_of(B, C) * H;
  if (ntiles == 0) return hipSuccess;
  hipLaunchKernelGGL((fwd_tile_kernel<T, NB>), dim3((unsigned)ntiles), dim3(kTThreads), 0, st, H,
                     (int)ntiles, qrec_slots(nk), scale * kLog2eT, (const T*)q, (const T*)k,
                     (const T*)v, (const int32_t*)w.qrec, (T*)o, lse);
  return hipGetLastError();
}

template <typename T, int NB>
hipError_t bwd_tile_t(int pass, int B, int C, int H, int nk, float scale, const void* q,
                      const void* k, const void* v, const void* o, const void* dout,
                      const float* lse, void* dq, void* dk, void* dv, const BwdWorkspace& w,
                      hipStream_t st) {
  const int64_t ntiles = windows_of(B, C) * H;
  if (ntiles == 0) return hipSuccess;
  if (pass & 1)
    hipLaunchKernelGGL((bwdq_tile_kernel<T, NB>), dim3((unsigned)ntiles), dim3(kTThreads), 0, st,
                       H, (int)ntiles, qrec_slots(nk), scale, (const T*)q, (const T*)k,
                       (const T*)v, (const T*)o, (const T*)dout, lse, (const int32_t*)w.qrec,
                       (T*)dq, w.ld, w.ld_none);
  if (pass & 2) {
    const uint32_t ld_none = (uint32_t)((const char*)w.ld_none - (const char*)w.ld);
    hipLaunchKernelGGL((bwdkv_tile_kernel<T>), dim3((unsigned)ntiles), dim3(kTThreads), 0, st, H,
                       (int)ntiles, scale, (const T*)q, (const T*)k, (const T*)v, (const T*)dout,
                       (const float2*)w.ld, ld_none, (const int32_t*)w.krec,
                       (const int32_t*)w.kent, (const RevEntry*)w.kitem, (T*)dk, (T*)dv);
  }
  return hipGetLastError();
}

template <typename T>
hipError_t fwd_tile_nb(int B, int C, int H, int nk, float scale, const void* q, const void* k,
                       const void* v, const BwdWorkspace& w, void* o, float* lse,
                       hipStream_t st) {
  switch ((nk + 15) >> 4) {
    case 1: return fwd_tile_t<T, 1>(B, C, H, nk, scale, q, k, v, w, o, lse, st);
    case 2: return fwd_tile_t<T, 2>(B, C, H, nk, scale, q, k, v, w, o, lse, st);
    case 3: return fwd_tile_t<T, 3>(B, C, H, nk, scale, q, k, v, w, o, lse, st);
    default: return fwd_tile_t<T, 4>(B, C, H, nk, scale, q, k, v, w, o, lse, st);
  }
}

template <typename T>
hipError_t bwd_tile_nb(int pass, int B, int C, int H, int nk, float scale, const void* q,
                       const void* k, const void* v, const void* o, const void* dout,
                       const float* lse, void* dq, void* dk, void* dv, const BwdWorkspace& w,
                       hipStream_t st) {
  switch ((nk + 15) >> 4) {
    case 1: return bwd_tile_t<T, 1>(pass, B, C, H, nk, scale, q, k, v, o, dout, lse, dq, dk, dv, w, st);
    case 2: return bwd_tile_t<T, 2>(pass, B, C, H, nk, scale, q, k, v, o, dout, lse, dq, dk, dv, w, st);
    case 3: return bwd_tile_t<T, 3>(pass, B, C, H, nk, scale, q, k, v, o, dout, lse, dq, dk, dv, w, st);
    default: return bwd_tile_t<T, 4>(pass, B, C, H, nk, scale, q, k, v, o, dout, lse, dq, dk, dv, w, st);
  }
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
  if (dt == 1) return fwd_tile_nb<bf16>(B, C, H, nk, scale, q, k, v, w, o, lse, st);
  if (dt == 2) return fwd_tile_nb<f16>(B, C, H, nk, scale, q, k, v, w, o, lse, st);
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_tile(int pass, int dt, int B, int N, int C, int H, int nk, float scale,
                           const void* q, const void* k, const void* v, const void* o,
                           const void* dout, const float* lse, void* dq, void* dk, void* dv,
                           const BwdWorkspace& w, hipStream_t st) {
  (void)N;
  if (dt == 1)
    return bwd_tile_nb<bf16>(pass, B, C, H, nk, scale, q, k, v, o, dout, lse, dq, dk, dv, w, st);
  if (dt == 2)
    return bwd_tile_nb<f16>(pass, B, C, H, nk, scale, q, k, v, o, dout, lse, dq, dk, dv, w, st);
  return hipErrorInvalidValue;
}

}  // namespace ca
