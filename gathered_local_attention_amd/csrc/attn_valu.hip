// Vector-ALU cluster attention kernels (any dtype, any nk <= 64).
//
// These serve the fp32 interface (where exact fp32 products are wanted) and
// every list length the matrix-core kernels do not take.  They compute the
// same quantities as the MFMA kernels: exact softmax attention restricted to
// each cluster's gathered key slots (English notes page "AFFMAE: Scalable
// Vision Pre-Training for High-Resolution Microscopy Segmentation on Desktop
// Hardware", "Overall Architecture": local cluster attention; arXiv abstract
// of the same paper: numerically stable Flash-style kernels), with fp32
// statistics and accumulation.
//
// Mapping: one 64-lane wavefront per (image, cluster, head).  In the slot
// phase lane s owns key slot s (its gathered K/V row lives in LDS); in the
// row phase lane (m, g) owns query m and dims [4g, 4g+4).  A -1 member of a
// partial cluster is no query: its rows are read from a clamped (valid)
// token and nothing is written for it; as a key it only appears as -1
// slots.
#include "common.h"

namespace ca {

namespace {

constexpr int D = 32;
constexpr int CS = 8;
constexpr int kPad = D + 1;   // LDS row stride (floats) to spread banks

template <typename T>
__device__ __forceinline__ void load_row(const T* __restrict__ src, float* dst) {
#pragma unroll
  for (int d = 0; d < D; ++d) dst[d] = to_f32(src[d]);
}

// ---------------------------------------------------------------------------
// forward: O and LSE
// ---------------------------------------------------------------------------
template <typename T>
__global__ void __launch_bounds__(64)
fwd_valu_kernel(int N, int C, int H, int nk, float scale, const T* __restrict__ q,
                const T* __restrict__ k, const T* __restrict__ v, const int32_t* __restrict__ q_idx,
                const int32_t* __restrict__ key_idx, T* __restrict__ o, float* __restrict__ lse) {
  __shared__ float qs[CS][kPad];
  __shared__ float ks[64][kPad];
  __shared__ float ps[CS][64];
  __shared__ int32_t ts[64];
  __shared__ int32_t qt[CS];

  const int h = blockIdx.x % H;
  const int bc = blockIdx.x / H;          // b * C + c
  const int b = bc / C;
  const int lane = threadIdx.x;
  const int64_t img = (int64_t)b * N;

  if (lane < CS) qt[lane] = q_idx[(int64_t)bc * CS + lane];
  const int t = lane < nk ? key_idx[(int64_t)bc * nk + lane] : -1;
  ts[lane] = t;
  __syncthreads();
  {
    const int m = lane >> 3, g = lane & 7;
    const T* src = q + ((img + max(qt[m], 0)) * H + h) * D + 4 * g;
#pragma unroll
    for (int e = 0; e < 4; ++e) qs[m][4 * g + e] = to_f32(src[e]);
  }
  if (t >= 0) load_row(k + ((img + t) * H + h) * D, ks[lane]);
  __syncthreads();

  float mx[CS], l[CS];
#pragma unroll
  for (int m = 0; m < CS; ++m) {
    float s = -INFINITY;
    if (t >= 0) {
      float acc = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) acc = fmaf(qs[m][d], ks[lane][d], acc);
      s = acc * scale;
    }
    mx[m] = wave_max(s);
    const float p = (t >= 0) ? __expf(s - mx[m]) : 0.f;
    l[m] = wave_sum(p);
    ps[m][lane] = p;
  }
  __syncthreads();

  const int m = lane >> 3, g = lane & 7;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < nk; ++s) {
    const int ts_ = ts[s];
    if (ts_ < 0) continue;
    const float p = ps[m][s];
    const T* vr = v + ((img + ts_) * H + h) * D + 4 * g;
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] = fmaf(p, to_f32(vr[e]), acc[e]);
  }
  float lm = 0.f, mm = 0.f;
#pragma unroll
  for (int r = 0; r < CS; ++r) if (r == m) { lm = l[r]; mm = mx[r]; }
  const float inv = lm > 0.f ? 1.f / lm : 0.f;
  if (qt[m] < 0) return;   // absent member
  T* dst = o + ((img + qt[m]) * H + h) * D + 4 * g;
#pragma unroll
  for (int e = 0; e < 4; ++e) dst[e] = from_f32<T>(acc[e] * inv);
  if (g == 0) lse[(img + qt[m]) * H + h] = lm > 0.f ? mm + __logf(lm) : -INFINITY;
}

// ---------------------------------------------------------------------------
// backward pass A (query-major): Delta and dQ
// ---------------------------------------------------------------------------
template <typename T>
__global__ void __launch_bounds__(64)
bwd_q_valu_kernel(int N, int C, int H, int nk, float scale, const T* __restrict__ q,
                  const T* __restrict__ k, const T* __restrict__ v, const T* __restrict__ o,
                  const T* __restrict__ dout, const float* __restrict__ lse,
                  const int32_t* __restrict__ q_idx, const int32_t* __restrict__ key_idx,
                  T* __restrict__ dq, float2* __restrict__ ld) {
  __shared__ float qs[CS][kPad];
  __shared__ float dos[CS][kPad];
  __shared__ float ks[64][kPad];
  __shared__ float vs[64][kPad];
  __shared__ float dss[CS][64];
  __shared__ float lses[CS], dels[CS];
  __shared__ int32_t ts[64];
  __shared__ int32_t qt[CS];

  const int h = blockIdx.x % H;
  const int bc = blockIdx.x / H;
  const int b = bc / C;
  const int lane = threadIdx.x;
  const int64_t img = (int64_t)b * N;

  if (lane < CS) qt[lane] = q_idx[(int64_t)bc * CS + lane];
  const int t = lane < nk ? key_idx[(int64_t)bc * nk + lane] : -1;
  ts[lane] = t;
  __syncthreads();
  const int m = lane >> 3, g = lane & 7;
  const int qm = max(qt[m], 0);   // absent member: any valid row, never written
  {
    const int64_t row = ((img + qm) * H + h) * D + 4 * g;
    float part = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      qs[m][4 * g + e] = to_f32(q[row + e]);
      const float dov = to_f32(dout[row + e]);
      dos[m][4 * g + e] = dov;
      part = fmaf(dov, to_f32(o[row + e]), part);
    }
    part += __shfl_xor(part, 1, 64);
    part += __shfl_xor(part, 2, 64);
    part += __shfl_xor(part, 4, 64);
    if (g == 0) {
      dels[m] = part;
      lses[m] = lse[(img + qm) * H + h];
      if (qt[m] >= 0) ld[(img + qm) * H + h] = make_float2(lses[m] * 1.4426950408889634f, part);
    }
  }
  if (t >= 0) {
    load_row(k + ((img + t) * H + h) * D, ks[lane]);
    load_row(v + ((img + t) * H + h) * D, vs[lane]);
  }
  __syncthreads();

#pragma unroll
  for (int mm = 0; mm < CS; ++mm) {
    float ds = 0.f;
    if (t >= 0) {
      float sacc = 0.f, pacc = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) {
        sacc = fmaf(qs[mm][d], ks[lane][d], sacc);
        pacc = fmaf(dos[mm][d], vs[lane][d], pacc);
      }
      const float p = __expf(sacc * scale - lses[mm]);
      ds = p * (pacc - dels[mm]);
    }
    dss[mm][lane] = ds;
  }
  __syncthreads();

  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < nk; ++s) {
    if (ts[s] < 0) continue;
    const float ds = dss[m][s];
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] = fmaf(ds, ks[s][4 * g + e], acc[e]);
  }
  if (qt[m] < 0) return;
  T* dst = dq + ((img + qt[m]) * H + h) * D + 4 * g;
#pragma unroll
  for (int e = 0; e < 4; ++e) dst[e] = from_f32<T>(acc[e] * scale);
}

// ---------------------------------------------------------------------------
// backward pass B (key-major): dK and dV over the transposed lists
// ---------------------------------------------------------------------------
template <typename T>
__global__ void __launch_bounds__(64)
bwd_kv_valu_kernel(int N, int C, int H, int nk, float scale, const T* __restrict__ q,
                   const T* __restrict__ k, const T* __restrict__ v, const T* __restrict__ dout,
                   const float* __restrict__ lse, const int32_t* __restrict__ q_idx,
                   const float2* __restrict__ ld, const int2* __restrict__ seg_all,
                   const RevEntry* __restrict__ rev_all, T* __restrict__ dk, T* __restrict__ dv) {
  __shared__ float kj[CS][kPad];
  __shared__ float vj[CS][kPad];
  __shared__ float qs[CS][kPad];
  __shared__ float dos[CS][kPad];
  __shared__ float pp[CS][CS], dd[CS][CS];
  __shared__ float lses[CS], dels[CS];
  __shared__ int32_t kt[CS];

  const int h = blockIdx.x % H;
  const int bj = blockIdx.x / H;
  const int b = bj / C;
  const int j = bj - b * C;
  const int lane = threadIdx.x;
  const int64_t img = (int64_t)b * N;
  const int hi = lane >> 3, lo = lane & 7;

  if (lane < CS) kt[lane] = q_idx[(int64_t)bj * CS + lane];
  __syncthreads();
  {
    const int64_t row = ((img + max(kt[hi], 0)) * H + h) * D + 4 * lo;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      kj[hi][4 * lo + e] = to_f32(k[row + e]);
      vj[hi][4 * lo + e] = to_f32(v[row + e]);
    }
  }
  const RevEntry* rev = rev_all;   // absolute entry ranges
  const int2 sg = seg_all[bj];
  const int e0 = sg.x, e1 = sg.y;

  float dka[4] = {0.f, 0.f, 0.f, 0.f}, dva[4] = {0.f, 0.f, 0.f, 0.f};
  for (int e = e0; e < e1; ++e) {
    const RevEntry ent = rev[e];
    __syncthreads();
    const int qraw = q_idx[((int64_t)b * C + ent.i) * CS + hi];   // -1: absent query
    {
      const int qtok = max(qraw, 0);
      const int64_t row = ((img + qtok) * H + h) * D + 4 * lo;
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        qs[hi][4 * lo + x] = to_f32(q[row + x]);
        dos[hi][4 * lo + x] = to_f32(dout[row + x]);
      }
      if (lo == 0) {
        lses[hi] = lse[(img + qtok) * H + h];
        dels[hi] = ld[(img + qtok) * H + h].y;
      }
    }
    __syncthreads();
    {
      // lane (m = hi, n = lo): query m of cluster ent.i against key n of j
      const int mult = qraw >= 0 ? (int)((ent.mult >> (8 * lo)) & 0xFFu) : 0;
      float p = 0.f, ds = 0.f;
      if (mult) {
        float sacc = 0.f, pacc = 0.f;
#pragma unroll
        for (int d = 0; d < D; ++d) {
          sacc = fmaf(qs[hi][d], kj[lo][d], sacc);
          pacc = fmaf(dos[hi][d], vj[lo][d], pacc);
        }
        p = (float)mult * __expf(sacc * scale - lses[hi]);
        ds = p * (pacc - dels[hi]);
      }
      pp[hi][lo] = p;
      dd[hi][lo] = ds;
    }
    __syncthreads();
    // lane (n = hi, dims 4*lo..): accumulate over the 8 queries
#pragma unroll
    for (int mm = 0; mm < CS; ++mm) {
      const float p = pp[mm][hi], ds = dd[mm][hi];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        dka[x] = fmaf(ds, qs[mm][4 * lo + x], dka[x]);
        dva[x] = fmaf(p, dos[mm][4 * lo + x], dva[x]);
      }
    }
  }
  if (kt[hi] < 0) return;   // absent member of a partial key cluster
  const int64_t row = ((img + kt[hi]) * H + h) * D + 4 * lo;
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    dk[row + x] = from_f32<T>(dka[x] * scale);
    dv[row + x] = from_f32<T>(dva[x]);
  }
}

template <typename T>
hipError_t fwd_t(int B, int N, int C, int H, int nk, float scale, const void* q, const void* k,
                 const void* v, const int32_t* q_idx, const int32_t* key_idx, void* o, float* lse,
                 hipStream_t st) {
  const int64_t blocks = (int64_t)B * C * H;
  hipLaunchKernelGGL(fwd_valu_kernel<T>, dim3((unsigned)blocks), dim3(64), 0, st, N, C, H, nk,
                     scale, (const T*)q, (const T*)k, (const T*)v, q_idx, key_idx, (T*)o, lse);
  return hipGetLastError();
}

template <typename T>
hipError_t bwd_t(int pass, int B, int N, int C, int H, int nk, float scale, const void* q,
                 const void* k, const void* v, const void* o, const void* dout, const float* lse,
                 const int32_t* q_idx, const int32_t* key_idx, void* dq, void* dk, void* dv,
                 const BwdWorkspace& w, hipStream_t st) {
  const int64_t blocks = (int64_t)B * C * H;
  if (pass & 1)
    hipLaunchKernelGGL(bwd_q_valu_kernel<T>, dim3((unsigned)blocks), dim3(64), 0, st, N, C, H, nk,
                       scale, (const T*)q, (const T*)k, (const T*)v, (const T*)o, (const T*)dout,
                       lse, q_idx, key_idx, (T*)dq, w.ld);
  if (pass & 2)
    hipLaunchKernelGGL(bwd_kv_valu_kernel<T>, dim3((unsigned)blocks), dim3(64), 0, st, N, C, H, nk,
                       scale, (const T*)q, (const T*)k, (const T*)v, (const T*)dout, lse, q_idx,
                       (const float2*)w.ld, (const int2*)w.seg, (const RevEntry*)w.rev,
                       (T*)dk, (T*)dv);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_valu(int dt, int B, int N, int C, int H, int nk, float scale, const void* q,
                           const void* k, const void* v, const int32_t* q_idx,
                           const int32_t* key_idx, void* o, float* lse, hipStream_t st) {
  switch (dt) {
    case 0: return fwd_t<float>(B, N, C, H, nk, scale, q, k, v, q_idx, key_idx, o, lse, st);
    case 1: return fwd_t<bf16>(B, N, C, H, nk, scale, q, k, v, q_idx, key_idx, o, lse, st);
    case 2: return fwd_t<f16>(B, N, C, H, nk, scale, q, k, v, q_idx, key_idx, o, lse, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_valu(int pass, int dt, int B, int N, int C, int H, int nk, float scale,
                           const void* q, const void* k, const void* v, const void* o,
                           const void* dout, const float* lse, const int32_t* q_idx,
                           const int32_t* key_idx, void* dq, void* dk, void* dv,
                           const BwdWorkspace& w, hipStream_t st) {
  switch (dt) {
    case 0: return bwd_t<float>(pass, B, N, C, H, nk, scale, q, k, v, o, dout, lse, q_idx, key_idx, dq, dk, dv, w, st);
    case 1: return bwd_t<bf16>(pass, B, N, C, H, nk, scale, q, k, v, o, dout, lse, q_idx, key_idx, dq, dk, dv, w, st);
    case 2: return bwd_t<f16>(pass, B, N, C, H, nk, scale, q, k, v, o, dout, lse, q_idx, key_idx, dq, dk, dv, w, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace ca
