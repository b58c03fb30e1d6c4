// Window plan of the window-tiled attention kernels.
//
// The notes page "AFFMAE: Scalable Vision Pre-Training for High-Resolution
// Microscopy Segmentation on Desktop Hardware" ("Limitations & Future Work")
// names the off-grid gather/scatter traffic as the cost of the method: every
// key row is read by each of the clusters whose list holds it.  Consecutive
// clusters in Morton order are spatial neighbours, so their lists overlap
// heavily; a window of kWin of them reads each distinct key token once.  This
// file builds, per window, what the kernels need to do that:
//
//  qwin_plan_kernel (one wavefront per window): the window's query tokens,
//    the distinct key tokens of its lists in ascending order (a bitonic sort
//    of the (token, slot) pairs of all its slots in registers) and how many
//    slots of each of its clusters hold each of them.  Exact integers: the
//    record is a function of the lists alone.
//  kwin_plan_kernel (one wavefront per window, after the transposed lists of
//    bwd_plan.hip): the query clusters that read any key of the window,
//    merged from the window's key clusters' entry lists (each ordered by
//    query cluster) into one list ordered by query cluster, with a 64-byte
//    multiplicity row per entry.
#include "common.h"

#include <algorithm>

namespace ca {

namespace {

__device__ __forceinline__ uint64_t umin64(uint64_t a, uint64_t b) { return a < b ? a : b; }
__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a < b ? b : a; }

// Ascending bitonic sort of 512 keys held 8 per lane: element e = 8 lane + r.
__device__ __forceinline__ void bitonic512(uint64_t (&k)[8], int lane) {
#pragma unroll
  for (int size = 2; size <= 512; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      if (stride >= 8) {
        const int lx = stride >> 3;
        const bool lower = (lane & lx) == 0;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const uint64_t o = __shfl_xor(k[r], lx, 64);
          const bool up = ((8 * lane + r) & size) == 0;
          k[r] = (lower == up) ? umin64(k[r], o) : umax64(k[r], o);
        }
      } else {
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          if (r & stride) continue;
          const int r2 = r | stride;
          const bool up = ((8 * lane + r) & size) == 0;
          const uint64_t lo = umin64(k[r], k[r2]), hi = umax64(k[r], k[r2]);
          k[r] = up ? lo : hi;
          k[r2] = up ? hi : lo;
        }
      }
    }
  }
}

// One wavefront per window w of image b = w / nwi (packed batch: nwi = all
// windows, b = 0).  Slots of the window: its clusters' key lists, back to
// back (s = c * nk + slot < 8 nk <= 512).
__global__ void __launch_bounds__(64)
qwin_plan_kernel(int N, int C, int nk, int nwi, int packed, const int32_t* __restrict__ q_idx,
                 const int32_t* __restrict__ key_idx, int32_t* __restrict__ qrec) {
  __shared__ uint32_t mt[2 * 512];   // multiplicity bytes [8][8 nk]
  const int w = blockIdx.x;
  const int lane = threadIdx.x;
  const int b = w / nwi, wi = w - b * nwi;
  const int c0 = wi * kWin;
  const int nc = min(kWin, C - c0);
  const int64_t gc0 = (int64_t)b * C + c0;
  const int kmax = 8 * nk;
  int32_t* rec = qrec + (int64_t)w * qrec_stride(nk);

  const int qt = (lane >> 3) < nc ? q_idx[gc0 * 8 + lane] : -1;
  for (int x = lane; x < 2 * kmax; x += 64) mt[x] = 0u;
  const int ns = nc * nk;
  uint64_t key[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const int s = 8 * lane + r;
    const int t = s < ns ? key_idx[gc0 * nk + s] : -1;
    key[r] = t >= 0 ? ((uint64_t)(uint32_t)t << 9) | (uint32_t)s : ~0ull;
  }
  bitonic512(key, lane);

  // distinct tokens: the first element of every run of equal tokens
  const uint64_t last_prev = __shfl_up(key[7], 1, 64);
  int flag[8], cnt = 0;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const uint64_t prev = r ? key[r - 1] : (lane ? last_prev : ~0ull);
    flag[r] = key[r] != ~0ull && (r == 0 && lane == 0 ? true : (prev >> 9) != (key[r] >> 9));
    cnt += flag[r];
  }
  const int incl = wave_inclusive_scan(cnt);
  const int u = __shfl(incl, 63, 64);
  int rank = incl - cnt - 1;   // rank of the current run's token
  __syncthreads();             // mt cleared
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    if (key[r] == ~0ull) continue;
    rank += flag[r];
    const uint32_t tok = (uint32_t)(key[r] >> 9);
    const int s = (int)(key[r] & 511u);
    if (flag[r]) rec[kQRecHead + rank] = (int32_t)tok;
    // at most nk slots of one cluster hold one token: a byte never carries
    const int at = (s / nk) * kmax + rank;
    atomicAdd(&mt[at >> 2], 1u << (8 * (at & 3)));
  }
  __syncthreads();
  // pad the key tokens to a multiple of 32 with a valid token
  const int pad_tok = u > 0 ? (int)(__shfl(key[0], 0, 64) >> 9) : __shfl(qt, 0, 64);
  const int upad = (u + 31) & ~31;
  for (int x = u + lane; x < upad; x += 64) rec[kQRecHead + x] = pad_tok;
  for (int x = lane; x < 2 * kmax; x += 64) rec[kQRecHead + kmax + x] = (int32_t)mt[x];
  rec[4 + lane] = qt;
  if (lane == 0) {
    rec[0] = (int32_t)gc0;
    rec[1] = nc;
    rec[2] = u;
    rec[3] = packed ? 0 : b * N;
  }
}

// One wavefront per key window.  Lanes 0..7 walk the entry lists of the
// window's key clusters (each ordered by query cluster i); every step takes
// the smallest i among the list heads and writes one merged entry: the
// query tokens of i and, in bytes 8 j .. 8 j + 7, the multiplicities of key
// cluster j's members (0 where i does not read j).  The window's raw entries
// are staged in LDS when they fit, so that the merge steps do not wait on
// global memory.
constexpr int kKwinLds = 256;   // raw entries staged per window

__global__ void __launch_bounds__(64)
kwin_plan_kernel(int N, int C, int nwi, int packed, const int32_t* __restrict__ q_idx,
                 const int2* __restrict__ seg, const RevEntry* __restrict__ rev,
                 const int32_t* __restrict__ rtok, int32_t* __restrict__ krec,
                 int32_t* __restrict__ kent) {
  __shared__ int32_t ri[kKwinLds];
  __shared__ uint64_t rm[kKwinLds];
  const int w = blockIdx.x;
  const int lane = threadIdx.x;
  const int b = w / nwi, wi = w - b * nwi;
  const int c0 = wi * kWin;
  const int nc = min(kWin, C - c0);
  const int64_t gc0 = (int64_t)b * C + c0;
  int32_t* rec = krec + (int64_t)w * kKRec;

  rec[8 + lane] = (lane >> 3) < nc ? q_idx[gc0 * 8 + lane] : -1;
  const int2 sg = lane < nc ? seg[gc0 + lane] : make_int2(0, 0);
  const int start = __shfl(sg.x, 0, 64);
  const int stop_all = __shfl(sg.y, nc - 1, 64);
  const bool staged = stop_all - start <= kKwinLds;
  if (staged) {
    for (int x = start + lane; x < stop_all; x += 64) {
      ri[x - start] = rev[x].i;
      rm[x - start] = rev[x].mult;
    }
  }
  __syncthreads();
  int cur = sg.x;
  const int stop = sg.y;
  int out = start;
  for (;;) {
    const bool live = lane < nc && cur < stop;
    int my = 0x7fffffff;
    if (live) my = staged ? ri[cur - start] : rev[cur].i;
    int m = my;
    m = min(m, __shfl_xor(m, 1, 64));
    m = min(m, __shfl_xor(m, 2, 64));
    m = min(m, __shfl_xor(m, 4, 64));
    m = __shfl(m, 0, 64);
    if (m == 0x7fffffff) break;
    const bool take = live && my == m;
    const uint64_t takers = __ballot(take);
    const int f = __ffsll((unsigned long long)takers) - 1;
    const int fcur = __shfl(cur, f, 64);
    int32_t* e = kent + (int64_t)out * kEnt;
    if (lane < 8) {
      const uint64_t mb = take ? (staged ? rm[cur - start] : rev[cur].mult) : 0ull;
      e[8 + 2 * lane] = (int32_t)(uint32_t)mb;
      e[9 + 2 * lane] = (int32_t)(uint32_t)(mb >> 32);
    } else if (lane < 16) {
      e[lane - 8] = rtok[(int64_t)fcur * 8 + (lane - 8)];
    }
    if (take) ++cur;
    ++out;
  }
  if (lane == 0) {
    rec[0] = start;
    rec[1] = out - start;
    rec[2] = (int32_t)gc0;
    rec[3] = packed ? 0 : b * N;
    rec[4] = nc;
    rec[5] = rec[6] = rec[7] = 0;
  }
}

}  // namespace

hipError_t launch_tile_plan(int B, int N, int C, int nk, bool packed, const int32_t* q_idx,
                            const int32_t* key_idx, const BwdWorkspace& w, hipStream_t st) {
  const int nwi = (C + kWin - 1) / kWin;
  const int64_t nw = (int64_t)B * nwi;
  if (nw == 0) return hipSuccess;
  hipLaunchKernelGGL(qwin_plan_kernel, dim3((unsigned)nw), dim3(64), 0, st, N, C, nk, nwi,
                     packed ? 1 : 0, q_idx, key_idx, w.qrec);
  hipLaunchKernelGGL(kwin_plan_kernel, dim3((unsigned)nw), dim3(64), 0, st, N, C, nwi,
                     packed ? 1 : 0, q_idx, (const int2*)w.seg, (const RevEntry*)w.rev,
                     (const int32_t*)w.rtok, w.krec, w.kent);
  return hipGetLastError();
}

}  // namespace ca
