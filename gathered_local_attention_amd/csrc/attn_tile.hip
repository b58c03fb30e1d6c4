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

// Gather `nrows` (a multiple of 16, at most 16 * MAXI * 2) head rows into a
// staged block: instruction i (of this wavefront: i = wv, wv + 2, ...)
// fills rows 16 i .. 16 i + 15; lane l fetches chunk (l & 3) ^ sw(row) of
// row 16 i + l / 4, so that LDS position l & 3 of that row holds it.
// `toks` (LDS) gives the token of each row; -1 takes `fallback`.
template <int MAXI>
__device__ __forceinline__ void gather_rows(const void* src, const int32_t* toks, int fallback,
                                            int nrows, uint32_t dst, int base, int H, int h,
                                            int lane, int wv) {
  const int ni = nrows >> 4;
  int tk[MAXI];
#pragma unroll
  for (int j = 0; j < MAXI; ++j) {
    const int i = wv + 2 * j;
    const int t = i < ni ? toks[16 * i + (lane >> 2)] : 0;
    tk[j] = t < 0 ? fallback : t;
  }
#pragma unroll
  for (int j = 0; j < MAXI; ++j) {
    const int i = wv + 2 * j;
    if (i < ni) {
      const int row = 16 * i + (lane >> 2);
      const uint32_t chunk = (uint32_t)(lane & 3) ^ sw(row);
      dma16(src, ((uint32_t)(base + tk[j]) * (uint32_t)H + (uint32_t)h) * kRowB + 16u * chunk,
            dst + 1024u * (uint32_t)i);
    }
  }
}

// four multiplicity bytes -> floats
__device__ __forceinline__ float mbyte(uint32_t w, int i) {
  return (float)((w >> (8 * i)) & 0xffu);
}

// query record of window w: head + key tokens and multiplicities of the
// chunk [k0, k0 + KCH) into LDS (head and tokens by wavefront 0, the eight
// multiplicity rows split over both)
template <int KCH>
__device__ __forceinline__ void load_qrec(const int32_t* qrec, int64_t rec_off, int kmax, int k0,
                                          bool head, uint32_t l_head, uint32_t l_kt, uint32_t l_mt,
                                          int lane, int wv) {
  const uint32_t ro = (uint32_t)(rec_off * 4);
  if (wv == 0) {
    if (head && lane < kQRecHead / 4) dma16(qrec, ro + 16u * lane, l_head);
    if (lane < KCH / 4) dma16(qrec, ro + 4u * (kQRecHead + k0) + 16u * lane, l_kt);
  }
  constexpr int kPer = KCH / 16;   // 16-byte pieces per multiplicity row
#pragma unroll
  for (int i = wv; i * 64 < 8 * kPer; i += 2) {
    const int p = 64 * i + lane;
    if (p < 8 * kPer) {
      const int c = p / kPer, col = p - c * kPer;
      dma16(qrec, ro + 4u * (kQRecHead + kmax) + (uint32_t)(c * kmax + k0 + 16 * col),
            l_mt + 1024u * (uint32_t)i);
    }
  }
}

// ---------------------------------------------------------------------------
// forward
// ---------------------------------------------------------------------------
template <int KCH>
struct FwdLds {
  static constexpr int kHead = 0, kKt = 512, kMt = kKt + 4 * KCH, kQ = kMt + 8 * KCH,
                       kK = kQ + 64 * 64, kV = kK + 64 * KCH, kBytes = kV + 64 * KCH;
};

template <typename T, int KCH>
__global__ void __launch_bounds__(kTThreads)
fwd_tile_kernel(int H, int ntiles, int kmax, int qstride, float scale_log2,
                const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
                const int32_t* __restrict__ qrec, T* __restrict__ o, float* __restrict__ lse) {
  typedef FwdLds<KCH> L;
  __shared__ __attribute__((aligned(1024))) char lds[L::kBytes];
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  if (tile >= ntiles) return;
  const int w = tile / H, h = tile - w * H;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int c16 = lane & 15, g = lane >> 4;
  const int e = c16 >> 2, qq = c16 & 3;
  const int32_t* rh = reinterpret_cast<const int32_t*>(lds + L::kHead);
  const int32_t* kt = reinterpret_cast<const int32_t*>(lds + L::kKt);
  const uint8_t* mt = reinterpret_cast<const uint8_t*>(lds + L::kMt);
  const char* sq = lds + L::kQ;
  const char* sk = lds + L::kK;
  const char* sv = lds + L::kV;
  const int64_t rec_off = (int64_t)w * qstride;

  load_qrec<KCH>(qrec, rec_off, kmax, 0, true, lds_addr(lds + L::kHead), lds_addr(kt),
                 lds_addr(mt), lane, wv);
  wait_vm<0>();
  __syncthreads();
  const int nc = rh[1], u = rh[2], base = rh[3];
  const int q0 = rh[4];
  const int32_t* qtok = rh + 4;
  gather_rows<2>(q, qtok, q0, 64, lds_addr(sq), base, H, h, lane, wv);
  int nrows = min(u, KCH);
  nrows = (nrows + 31) & ~31;
  gather_rows<KCH / 32>(k, kt, q0, nrows, lds_addr(sk), base, H, h, lane, wv);
  gather_rows<KCH / 32>(v, kt, q0, nrows, lds_addr(sv), base, H, h, lane, wv);
  wait_vm<0>();
  __syncthreads();

  const bool active = 4 * wv < nc;   // this wavefront's clusters exist
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  uint4 qv[2];
  int cl[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int row = 32 * wv + 16 * cb + c16;
    qv[cb] = lds16(sq, row_chunk(row, (uint32_t)g));
    cl[cb] = 4 * wv + 2 * cb + (c16 >> 3);
  }
  float mrun[2] = {-INFINITY, -INFINITY}, lrun[2] = {0.f, 0.f};
  f32x4 oacc[2][2] = {{z, z}, {z, z}};

  for (int k0 = 0; k0 < u; k0 += KCH) {
    if (k0 > 0) {   // a further chunk of the window's keys (long lists only)
      __syncthreads();
      load_qrec<KCH>(qrec, rec_off, kmax, k0, false, 0u, lds_addr(kt), lds_addr(mt), lane, wv);
      wait_vm<0>();
      __syncthreads();
      nrows = (min(u - k0, KCH) + 31) & ~31;
      gather_rows<KCH / 32>(k, kt, q0, nrows, lds_addr(sk), base, H, h, lane, wv);
      gather_rows<KCH / 32>(v, kt, q0, nrows, lds_addr(sv), base, H, h, lane, wv);
      wait_vm<0>();
      __syncthreads();
    }
    if (!active) continue;
    for (int s = 0; s < nrows; s += 64) {
      const int nb = min(4, (nrows - s) >> 4);   // 4 or 2 key blocks of 16
      f32x4 sacc[4][2];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        if (kb < nb) {
          const int kr = s + 16 * kb + c16;
          const uint4 ka = lds16(sk, row_chunk(kr, (uint32_t)g));
#pragma unroll
          for (int cb = 0; cb < 2; ++cb) sacc[kb][cb] = Mfma<T>::mma(ka, qv[cb], z);
        }
      }
      uint4 bp[2][2];
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        uint32_t mw[4];
        float t[4][4];
        float lmax = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          if (kb < nb) {
            mw[kb] = *reinterpret_cast<const uint32_t*>(mt + cl[cb] * KCH + s + 16 * kb + 4 * g);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              t[kb][i] = sacc[kb][cb][i] * scale_log2;
              if ((mw[kb] >> (8 * i)) & 0xffu) lmax = fmaxf(lmax, t[kb][i]);
            }
          }
        }
        const float mnew = fmaxf(mrun[cb], shfl_max16_32(lmax));
        const float mref = mnew == -INFINITY ? 0.f : mnew;
        const float alpha = __builtin_amdgcn_exp2f(mrun[cb] - mref);
        float lsum = 0.f;
        float p[4][4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          if (kb < nb) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float m = mbyte(mw[kb], i);
              p[kb][i] = m != 0.f ? m * __builtin_amdgcn_exp2f(t[kb][i] - mref) : 0.f;
              lsum += p[kb][i];
            }
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) p[kb][i] = 0.f;
          }
        }
        lrun[cb] = lrun[cb] * alpha + lsum;
        mrun[cb] = mnew;
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) oacc[cb][hf] *= alpha;
#pragma unroll
        for (int kg = 0; kg < 2; ++kg) {
          const f32x4 pa = {p[2 * kg][0], p[2 * kg][1], p[2 * kg][2], p[2 * kg][3]};
          const f32x4 pb = {p[2 * kg + 1][0], p[2 * kg + 1][1], p[2 * kg + 1][2], p[2 * kg + 1][3]};
          bp[cb][kg] = cat(pack4<T>(pa), pack4<T>(pb));
        }
      }
      // O^T += V^T P^T: lane 4e + qq of row group g reads dims
      // 16 hf + 4 qq .. of key row s + 32 kg + 16 blk + 4 g + e
#pragma unroll
      for (int kg = 0; kg < 2; ++kg) {
        if (2 * kg < nb) {
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
            uint2 vt[2];
#pragma unroll
            for (int blk = 0; blk < 2; ++blk) {
              const int kr = s + 32 * kg + 16 * blk + 4 * g + e;
              vt[blk] = lds_tr8(sv, row_chunk(kr, (uint32_t)(2 * hf + (qq >> 1))) + 8u * (qq & 1));
            }
            const uint4 va = cat(vt[0], vt[1]);
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) oacc[cb][hf] = Mfma<T>::mma(va, bp[cb][kg], oacc[cb][hf]);
          }
        }
      }
    }
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
template <int KCH>
struct BqLds {
  static constexpr int kHead = 0, kKt = 512, kMt = kKt + 4 * KCH, kLse = kMt + 8 * KCH,
                       kQ = kLse + 256, kDo = kQ + 4096, kO = kDo + 4096, kK = kO + 4096,
                       kV = kK + 64 * KCH, kBytes = kV + 64 * KCH;
};

template <typename T, int KCH>
__global__ void __launch_bounds__(kTThreads)
bwdq_tile_kernel(int H, int ntiles, int kmax, int qstride, float scale,
                 const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
                 const T* __restrict__ o, const T* __restrict__ dout,
                 const float* __restrict__ lse, const int32_t* __restrict__ qrec,
                 T* __restrict__ dq, float2* __restrict__ ld, float4* __restrict__ ld_none) {
  typedef BqLds<KCH> L;
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
  const int32_t* rh = reinterpret_cast<const int32_t*>(lds + L::kHead);
  const int32_t* kt = reinterpret_cast<const int32_t*>(lds + L::kKt);
  const uint8_t* mt = reinterpret_cast<const uint8_t*>(lds + L::kMt);
  const float* sl = reinterpret_cast<const float*>(lds + L::kLse);
  const char* sq = lds + L::kQ;
  const char* sdo = lds + L::kDo;
  const char* so = lds + L::kO;
  const char* sk = lds + L::kK;
  const char* sv = lds + L::kV;
  const int64_t rec_off = (int64_t)w * qstride;
  const float scale_log2 = scale * kLog2eT;

  load_qrec<KCH>(qrec, rec_off, kmax, 0, true, lds_addr(lds + L::kHead), lds_addr(kt),
                 lds_addr(mt), lane, wv);
  wait_vm<0>();
  __syncthreads();
  const int nc = rh[1], u = rh[2], base = rh[3];
  const int q0 = rh[4];
  const int32_t* qtok = rh + 4;
  gather_rows<2>(q, qtok, q0, 64, lds_addr(sq), base, H, h, lane, wv);
  gather_rows<2>(dout, qtok, q0, 64, lds_addr(sdo), base, H, h, lane, wv);
  gather_rows<2>(o, qtok, q0, 64, lds_addr(so), base, H, h, lane, wv);
  if (wv == 0) {
    const int t = qtok[lane] < 0 ? q0 : qtok[lane];
    dma4(lse, ((uint32_t)(base + t) * (uint32_t)H + (uint32_t)h) * 4u, lds_addr(sl));
  }
  int nrows = (min(u, KCH) + 31) & ~31;
  gather_rows<KCH / 32>(k, kt, q0, nrows, lds_addr(sk), base, H, h, lane, wv);
  gather_rows<KCH / 32>(v, kt, q0, nrows, lds_addr(sv), base, H, h, lane, wv);
  wait_vm<0>();
  __syncthreads();

  const bool active = 4 * wv < nc;
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  uint4 qv[2], dov[2];
  int cl[2];
  float lse2[2], dl[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int row = 32 * wv + 16 * cb + c16;
    qv[cb] = lds16(sq, row_chunk(row, (uint32_t)g));
    dov[cb] = lds16(sdo, row_chunk(row, (uint32_t)g));
    const uint4 ov = lds16(so, row_chunk(row, (uint32_t)g));
    cl[cb] = 4 * wv + 2 * cb + (c16 >> 3);
    lse2[cb] = sl[row] * kLog2eT;
    // Delta of query row `row`: eight dims per lane, summed over the 4 lanes
    const uint32_t a[4] = {dov[cb].x, dov[cb].y, dov[cb].z, dov[cb].w};
    const uint32_t b[4] = {ov.x, ov.y, ov.z, ov.w};
    float d = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x2 xa = Mfma<T>::unpack(a[i]), ya = Mfma<T>::unpack(b[i]);
      d = fmaf(xa[0], ya[0], fmaf(xa[1], ya[1], d));
    }
    dl[cb] = shfl_sum16_32(d);
  }
  f32x4 acc[2][2] = {{z, z}, {z, z}};   // dQ^T [cb][dim half]

  for (int k0 = 0; k0 < u; k0 += KCH) {
    if (k0 > 0) {
      __syncthreads();
      load_qrec<KCH>(qrec, rec_off, kmax, k0, false, 0u, lds_addr(kt), lds_addr(mt), lane, wv);
      wait_vm<0>();
      __syncthreads();
      nrows = (min(u - k0, KCH) + 31) & ~31;
      gather_rows<KCH / 32>(k, kt, q0, nrows, lds_addr(sk), base, H, h, lane, wv);
      gather_rows<KCH / 32>(v, kt, q0, nrows, lds_addr(sv), base, H, h, lane, wv);
      wait_vm<0>();
      __syncthreads();
    }
    if (!active) continue;
    for (int s = 0; s < nrows; s += 64) {
      const int nb = min(4, (nrows - s) >> 4);
      f32x4 sacc[4][2], pacc[4][2];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        if (kb < nb) {
          const int kr = s + 16 * kb + c16;
          const uint4 ka = lds16(sk, row_chunk(kr, (uint32_t)g));
          const uint4 va = lds16(sv, row_chunk(kr, (uint32_t)g));
#pragma unroll
          for (int cb = 0; cb < 2; ++cb) {
            sacc[kb][cb] = Mfma<T>::mma(ka, qv[cb], z);
            pacc[kb][cb] = Mfma<T>::mma(va, dov[cb], z);
          }
        }
      }
      uint4 bds[2][2];
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        float ds[4][4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          if (kb < nb) {
            const uint32_t mw =
                *reinterpret_cast<const uint32_t*>(mt + cl[cb] * KCH + s + 16 * kb + 4 * g);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float m = mbyte(mw, i);
              const float p =
                  m * __builtin_amdgcn_exp2f(fmaf(sacc[kb][cb][i], scale_log2, -lse2[cb]));
              ds[kb][i] = m != 0.f ? p * (pacc[kb][cb][i] - dl[cb]) : 0.f;
            }
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) ds[kb][i] = 0.f;
          }
        }
#pragma unroll
        for (int kg = 0; kg < 2; ++kg) {
          const f32x4 da = {ds[2 * kg][0], ds[2 * kg][1], ds[2 * kg][2], ds[2 * kg][3]};
          const f32x4 db = {ds[2 * kg + 1][0], ds[2 * kg + 1][1], ds[2 * kg + 1][2],
                            ds[2 * kg + 1][3]};
          bds[cb][kg] = cat(pack4<T>(da), pack4<T>(db));
        }
      }
      // dQ^T += K^T dS^T (K read transposed)
#pragma unroll
      for (int kg = 0; kg < 2; ++kg) {
        if (2 * kg < nb) {
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
            uint2 ktr[2];
#pragma unroll
            for (int blk = 0; blk < 2; ++blk) {
              const int kr = s + 32 * kg + 16 * blk + 4 * g + e;
              ktr[blk] = lds_tr8(sk, row_chunk(kr, (uint32_t)(2 * hf + (qq >> 1))) + 8u * (qq & 1));
            }
            const uint4 ka = cat(ktr[0], ktr[1]);
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) acc[cb][hf] = Mfma<T>::mma(ka, bds[cb][kg], acc[cb][hf]);
          }
        }
      }
    }
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
constexpr int kEch = 24;   // entries (query clusters) staged per step

struct BkvLds {
  static constexpr int kRec = 0, kKk = 512, kKv = kKk + 4096, kEn = kKv + 4096,
                       kQ = kEn + kEch * kEnt * 4, kDo = kQ + kEch * 8 * 64,
                       kL2 = kDo + kEch * 8 * 64, kDl = kL2 + kEch * 8 * 4,
                       kBytes = kDl + kEch * 8 * 4;
};

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
  const float* sl2 = reinterpret_cast<const float*>(lds + L::kL2);
  const float* sdl = reinterpret_cast<const float*>(lds + L::kDl);
  const char* skk = lds + L::kKk;
  const char* skv = lds + L::kKv;
  const char* sq = lds + L::kQ;
  const char* sdo = lds + L::kDo;
  const float scale_log2 = scale * kLog2eT;

  if (wv == 0 && lane < 18) dma16(krec, (uint32_t)(w * kKRec * 4) + 16u * lane, lds_addr(rk));
  wait_vm<0>();
  __syncthreads();
  const int start = rk[0], E = rk[1], base = rk[3], nc = rk[4];
  const int32_t* ktok = rk + 8;
  const int k0tok = ktok[0];
  gather_rows<2>(k, ktok, k0tok, 64, lds_addr(skk), base, H, h, lane, wv);
  gather_rows<2>(v, ktok, k0tok, 64, lds_addr(skv), base, H, h, lane, wv);

  // entries [e0, e0 + n) into LDS: 6 sixteen-byte pieces per entry
  auto load_entries = [&](int e0, int n) {
    for (int i = wv; 64 * i < 6 * n; i += 2) {
      const int p = 64 * i + lane;
      if (p < 6 * n) dma16(kent, (uint32_t)(start + e0) * (uint32_t)(kEnt * 4) + 16u * p,
                           lds_addr(en) + 1024u * (uint32_t)i);
    }
  };
  load_entries(0, min(E, kEch));
  wait_vm<0>();
  __syncthreads();

  const bool active = 32 * wv < 8 * nc;
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  uint4 kreg[2], vreg[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int row = 32 * wv + 16 * kb + c16;
    kreg[kb] = lds16(skk, row_chunk(row, (uint32_t)g));
    vreg[kb] = lds16(skv, row_chunk(row, (uint32_t)g));
  }
  f32x4 dka[2][2] = {{z, z}, {z, z}}, dva[2][2] = {{z, z}, {z, z}};   // [dim half][key block]

  for (int e0 = 0; e0 < E; e0 += kEch) {
    const int n = min(kEch, E - e0);
    if (e0 > 0) {
      __syncthreads();
      load_entries(e0, n);
      wait_vm<0>();
      __syncthreads();
    }
    const int ngr = (n + 3) >> 2;   // groups of 4 entries = 32 query rows
    const int nrows = 32 * ngr;
    // query rows: token of row r = member r & 7 of entry r >> 3 (past the
    // n-th entry, or an absent member: the window's first key token)
    {
      const int ni = nrows >> 4;
#pragma unroll
      for (int j = 0; j < (kEch * 8 / 16 + 1) / 2; ++j) {
        const int i = wv + 2 * j;
        if (i < ni) {
          const int row = 16 * i + (lane >> 2);
          int t = (row >> 3) < n ? en[(row >> 3) * kEnt + (row & 7)] : -1;
          t = t < 0 ? k0tok : t;
          const uint32_t chunk = (uint32_t)(lane & 3) ^ sw(row);
          const uint32_t off = ((uint32_t)(base + t) * (uint32_t)H + (uint32_t)h) * kRowB + 16u * chunk;
          dma16(q, off, lds_addr(sq) + 1024u * (uint32_t)i);
          dma16(dout, off, lds_addr(sdo) + 1024u * (uint32_t)i);
        }
      }
      // (LSE log2 e, Delta) of every row, as two 4-byte gathers; an absent
      // or padding row reads the (+inf, 0) pair
#pragma unroll
      for (int j = 0; j < (kEch * 8 / 64 + 1) / 2; ++j) {
        const int i = wv + 2 * j;
        if (64 * i < nrows) {
          const int row = 64 * i + lane;
          const int t = (row >> 3) < n ? en[(row >> 3) * kEnt + (row & 7)] : -1;
          const uint32_t off =
              t >= 0 ? ((uint32_t)(base + t) * (uint32_t)H + (uint32_t)h) * 8u : ld_none;
          dma4(ld, off, lds_addr(sl2) + 256u * (uint32_t)i);
          dma4(ld, off + 4u, lds_addr(sdl) + 256u * (uint32_t)i);
        }
      }
    }
    wait_vm<0>();
    __syncthreads();
    if (!active) continue;

    for (int gi = 0; gi < ngr; ++gi) {
      const int r0 = 32 * gi;
      f32x4 sv[2][2], pv[2][2];   // [query block][key block]
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const int row = r0 + 16 * qb + c16;
        const uint4 qa = lds16(sq, row_chunk(row, (uint32_t)g));
        const uint4 da = lds16(sdo, row_chunk(row, (uint32_t)g));
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          sv[qb][kb] = Mfma<T>::mma(qa, kreg[kb], z);
          pv[qb][kb] = Mfma<T>::mma(da, vreg[kb], z);
        }
      }
      float pp[2][2][4], dd[2][2][4];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const int rr = r0 + 16 * qb + 4 * g;   // rows rr .. rr + 3 of this lane
        const int er = rr >> 3;                // their entry
        const float4 l2 = *reinterpret_cast<const float4*>(sl2 + rr);
        const float4 dl4 = *reinterpret_cast<const float4*>(sdl + rr);
        const float l2a[4] = {l2.x, l2.y, l2.z, l2.w};
        const float dla[4] = {dl4.x, dl4.y, dl4.z, dl4.w};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const int key = 32 * wv + 16 * kb + c16;
          const float m = er < n ? (float)enb[er * (kEnt * 4) + 32 + key] : 0.f;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float p = m * __builtin_amdgcn_exp2f(fmaf(sv[qb][kb][i], scale_log2, -l2a[i]));
            pp[qb][kb][i] = m != 0.f ? p : 0.f;
            dd[qb][kb][i] = m != 0.f ? p * (pv[qb][kb][i] - dla[i]) : 0.f;
          }
        }
      }
      uint4 bp[2], bd[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const f32x4 p0 = {pp[0][kb][0], pp[0][kb][1], pp[0][kb][2], pp[0][kb][3]};
        const f32x4 p1 = {pp[1][kb][0], pp[1][kb][1], pp[1][kb][2], pp[1][kb][3]};
        const f32x4 d0 = {dd[0][kb][0], dd[0][kb][1], dd[0][kb][2], dd[0][kb][3]};
        const f32x4 d1 = {dd[1][kb][0], dd[1][kb][1], dd[1][kb][2], dd[1][kb][3]};
        bp[kb] = cat(pack4<T>(p0), pack4<T>(p1));
        bd[kb] = cat(pack4<T>(d0), pack4<T>(d1));
      }
      // dV^T += dO^T P, dK^T += Q^T dS: rows r0 + 16 blk + 4 g + e transposed
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        uint2 dt[2], qt[2];
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
          const int row = r0 + 16 * blk + 4 * g + e;
          const uint32_t off = row_chunk(row, (uint32_t)(2 * hf + (qq >> 1))) + 8u * (qq & 1);
          dt[blk] = lds_tr8(sdo, off);
          qt[blk] = lds_tr8(sq, off);
        }
        const uint4 da = cat(dt[0], dt[1]), qa = cat(qt[0], qt[1]);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          dva[hf][kb] = Mfma<T>::mma(da, bp[kb], dva[hf][kb]);
          dka[hf][kb] = Mfma<T>::mma(qa, bd[kb], dka[hf][kb]);
        }
      }
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

constexpr int kFwdKch = 256;   // key rows staged per pass (forward)
constexpr int kBqKch = 192;    // key rows staged per pass (query-major backward)

template <typename T>
hipError_t fwd_tile_t(int B, int C, int H, int nk, float scale, const void* q, const void* k,
                      const void* v, const BwdWorkspace& w, void* o, float* lse,
                      hipStream_t st) {
  const int64_t ntiles = windows_of(B, C) * H;
  if (ntiles == 0) return hipSuccess;
  hipLaunchKernelGGL((fwd_tile_kernel<T, kFwdKch>), dim3((unsigned)ntiles), dim3(kTThreads), 0,
                     st, H, (int)ntiles, 8 * nk, qrec_stride(nk), scale * kLog2eT, (const T*)q,
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
    hipLaunchKernelGGL((bwdq_tile_kernel<T, kBqKch>), dim3((unsigned)ntiles), dim3(kTThreads), 0,
                       st, H, (int)ntiles, 8 * nk, qrec_stride(nk), scale, (const T*)q,
                       (const T*)k, (const T*)v, (const T*)o, (const T*)dout, lse,
                       (const int32_t*)w.qrec, (T*)dq, w.ld, w.ld_none);
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
