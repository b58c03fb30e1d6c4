// Window plan of the window-tiled attention kernels.
//
// The notes page "AFFMAE: Scalable Vision Pre-Training for High-Resolution
// Microscopy Segmentation on Desktop Hardware" ("Limitations & Future Work")
// names the off-grid gather/scatter traffic as the cost of the method: every
// key row is read by each of the clusters whose list holds it.  Consecutive
// clusters in Morton order are spatial neighbours, so their lists overlap
// heavily; a window of kWin of them reads each distinct key token once.  This
// file builds, per window, what the kernels need to do that (the layout is
// described in common.h):
//
//  qwin_plan_kernel (one wavefront per window): the window's query tokens,
//    its distinct key tokens in ascending order (a bitonic sort of the
//    (token, slot) pairs of all its slots in registers), and for every slot
//    the LDS offset of its token's staged row.  A window with more distinct
//    keys than the kernels stage is also described as sub-windows.  Exact
//    integers: the records are a function of the lists alone.
//  kwin_plan_kernel (one wavefront per window, after the transposed lists of
//    bwd_plan.hip): the query clusters that read any key of the window,
//    merged from the window's key clusters' entry lists (each ordered by
//    query cluster) into one list ordered by query cluster; every (query
//    cluster, key cluster) pair gets its merged index.
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

// LDS scratch of one query record while it is built
struct QrecLds {
  uint16_t slot[8 * 16 * 4];
  unsigned long long mask[8];
};

// Write the record of the clusters [c_lo, c_lo + ncl) of a window from the
// sorted (token << 9 | slot) keys: elements outside the range are ignored.
// Returns the number of distinct tokens (or writes nothing but the count if
// it exceeds kUnionCap and `only_count`).
__device__ int write_qrec(const uint64_t (&key)[8], int lane, int nk, int c_lo, int ncl,
                          int32_t* rec, QrecLds& s, bool only_count) {
  // element in range: a valid key whose slot's cluster is in [c_lo, c_lo + ncl)
  bool in[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const int c = (int)(key[r] & 511u) / nk;
    in[r] = key[r] != ~0ull && c >= c_lo && c < c_lo + ncl;
  }
  // distinct tokens among the elements in range: an element starts a new
  // token unless an earlier element in range has the same token; equal
  // tokens are adjacent, so it is enough to know the token of the last
  // element in range before it
  uint64_t lastin = ~0ull;   // token of the last in-range element of this lane
#pragma unroll
  for (int r = 0; r < 8; ++r)
    if (in[r]) lastin = key[r] >> 9;
  // the last in-range token of the lanes below: a max-scan works because
  // tokens ascend along the sorted order
  uint64_t carry = lastin == ~0ull ? 0ull : lastin + 1;   // 0 = none
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint64_t y = __shfl_up(carry, o, 64);
    if (lane >= o) carry = umax64(carry, y);
  }
  uint64_t prev = __shfl_up(carry, 1, 64);
  if (lane == 0) prev = 0;
  int flag[8], cnt = 0;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    flag[r] = 0;
    if (!in[r]) continue;
    const uint64_t t1 = (key[r] >> 9) + 1;
    flag[r] = t1 != prev;
    prev = t1;
    cnt += flag[r];
  }
  const int incl = wave_inclusive_scan(cnt);
  const int u = __shfl(incl, 63, 64);
  if (only_count && u > kUnionCap) return u;
  // clear the slot table (every slot at row 0) and the masks
  for (int x = lane; x < 8 * 16 * 4; x += 64) s.slot[x] = 0;
  if (lane < 8) s.mask[lane] = 0ull;
  __syncthreads();
  int rank = incl - cnt - 1;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    if (!in[r]) continue;
    rank += flag[r];
    const int sl = (int)(key[r] & 511u);
    const int c = sl / nk - c_lo, j = sl - (sl / nk) * nk;
    if (flag[r]) rec[kQRecHead + rank] = (int32_t)(key[r] >> 9);
    s.slot[(c * 16 + (j & 15)) * 4 + (j >> 4)] =
        (uint16_t)(rank * kLdsRow + 16 * (int)row_swz(rank));
    atomicOr(&s.mask[c], 1ull << j);
  }
  __syncthreads();
  return u;
}

// One wavefront per window w of image b = w / nwi (packed batch: nwi = all
// windows, b = 0).  Slots of the window: its clusters' key lists, back to
// back (s = c * nk + slot < 8 nk <= 512).
__global__ void __launch_bounds__(64)
qwin_plan_kernel(int N, int C, int nk, int nwi, int packed, const int32_t* __restrict__ q_idx,
                 const int32_t* __restrict__ key_idx, int32_t* __restrict__ qrec) {
  __shared__ QrecLds s;
  const int w = blockIdx.x;
  const int lane = threadIdx.x;
  const int b = w / nwi, wi = w - b * nwi;
  const int c0 = wi * kWin;
  const int nc = min(kWin, C - c0);
  const int64_t gc0 = (int64_t)b * C + c0;
  const int nb = (nk + 15) >> 4;   // 16-slot blocks per list
  const int nrec = qrec_slots(nk);
  int32_t* rec = qrec + (int64_t)w * nrec * kQRecStride;

  const int qt = (lane >> 3) < nc ? q_idx[gc0 * 8 + lane] : -1;
  const int ns = nc * nk;
  uint64_t key[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const int sl = 8 * lane + r;
    const int t = sl < ns ? key_idx[gc0 * nk + sl] : -1;
    key[r] = t >= 0 ? ((uint64_t)(uint32_t)t << 9) | (uint32_t)sl : ~0ull;
  }
  bitonic512(key, lane);

  // one record: clusters [c_lo, c_lo + ncl) at `out`
  auto emit = [&](int32_t* out, int c_lo, int ncl, bool only_count) {
    const int u = write_qrec(key, lane, nk, c_lo, ncl, out, s, only_count);
    if (only_count && u > kUnionCap) return u;
    // (every lane takes part in the shuffle: its source lanes must be active)
    const int qs = __shfl(qt, (lane + 8 * c_lo) & 63, 64);
    const int q = (lane >> 3) < ncl ? qs : -1;
    const int q0 = __shfl(qt, 8 * c_lo, 64);
    // pad the key tokens to a multiple of 32 with a valid token
    const int pad_tok = q0;
    const int upad = (u + 31) & ~31;
    for (int x = u + lane; x < upad; x += 64) out[kQRecHead + x] = pad_tok;
    const uint32_t* st = reinterpret_cast<const uint32_t*>(s.slot);
    for (int x = lane; x < 8 * 16 * 4 / 2; x += 64) out[kQSlotOff + x] = (int32_t)st[x];
    bool holes = false;
    if (lane < 8) {
      const unsigned long long full = nb * 16 >= 64 ? ~0ull : (1ull << (nb * 16)) - 1ull;
      const unsigned long long m = s.mask[lane];
      out[kQMaskOff + 2 * lane] = (int32_t)(uint32_t)m;
      out[kQMaskOff + 2 * lane + 1] = (int32_t)(uint32_t)(m >> 32);
      holes = lane < ncl && m != full;
    }
    holes = __ballot(holes) != 0ull;
    out[8 + lane] = q;
    if (lane == 0) {
      out[0] = (int32_t)(gc0 + c_lo);
      out[1] = ncl;
      out[2] = u;
      out[3] = packed ? 0 : b * N;
      out[4] = holes ? kQHoles : 0;
      out[5] = 0;
      out[6] = out[7] = 0;
    }
    __syncthreads();
    return u;
  };
  const int u = emit(rec, 0, nc, true);
  if (u > kUnionCap) {   // too many distinct keys: sub-windows
    const int sw = sub_window(nk);
    const int nsub = (nc + sw - 1) / sw;
    for (int j = 0; j < nsub; ++j)
      emit(rec + (1 + j) * kQRecStride, j * sw, min(sw, nc - j * sw), false);
    rec[8 + lane] = qt;
    if (lane == 0) {
      rec[0] = (int32_t)gc0;
      rec[1] = nc;
      rec[2] = u;
      rec[3] = packed ? 0 : b * N;
      rec[4] = kQSplit;
      rec[5] = nsub;
    }
  }
}

// One wavefront per key window.  Lanes 0..7 walk the entry lists of the
// window's key clusters (each ordered by query cluster i); every step takes
// the smallest i among the list heads, writes one merged entry (the query
// tokens of i) and gives each key cluster whose head it was the merged
// index.  The window's raw entries are staged in LDS when they fit, so that
// the merge steps do not wait on global memory.
constexpr int kKwinLds = 256;   // raw entries staged per window

__global__ void __launch_bounds__(64)
kwin_plan_kernel(int N, int C, int nwi, int packed, const int32_t* __restrict__ q_idx,
                 const int2* __restrict__ seg, const RevEntry* __restrict__ rev,
                 const int32_t* __restrict__ rtok, int32_t* __restrict__ krec,
                 int32_t* __restrict__ kent, RevEntry* __restrict__ kitem) {
  __shared__ int32_t ri[kKwinLds];
  __shared__ unsigned long long rm[kKwinLds];
  __shared__ int32_t rt[kKwinLds * 8];
  const int w = blockIdx.x;
  const int lane = threadIdx.x;
  const int b = w / nwi, wi = w - b * nwi;
  const int c0 = wi * kWin;
  const int nc = min(kWin, C - c0);
  const int64_t gc0 = (int64_t)b * C + c0;
  int32_t* rec = krec + (int64_t)w * kKRec;

  rec[8 + lane] = (lane >> 3) < nc ? q_idx[gc0 * 8 + lane] : -1;
  const int2 sg = lane < nc ? seg[gc0 + lane] : make_int2(0, 0);
  if (lane < 8) {
    rec[72 + 2 * lane] = sg.x;
    rec[73 + 2 * lane] = sg.y - sg.x;
  }
  const int start = __shfl(sg.x, 0, 64);
  const int stop_all = __shfl(sg.y, nc - 1, 64);
  const bool staged = stop_all - start <= kKwinLds;
  if (staged) {
    for (int x = start + lane; x < stop_all; x += 64) {
      ri[x - start] = rev[x].i;
      rm[x - start] = rev[x].mult;
    }
    for (int x = 8 * start + lane; x < 8 * stop_all; x += 64) rt[x - 8 * start] = rtok[x];
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
    if (take) {
      RevEntry it;
      it.i = out - start;
      it.pad = 0;
      it.mult = staged ? rm[cur - start] : rev[cur].mult;
      kitem[cur] = it;
      ++cur;
    }
    if (lane >= 8 && lane < 16) {
      const int t =
          staged ? rt[(fcur - start) * 8 + (lane - 8)] : rtok[(int64_t)fcur * 8 + (lane - 8)];
      kent[(int64_t)out * kEnt + (lane - 8)] = t;
      if (out - start < kKRecEnt) rec[kKRecHead + (out - start) * 8 + (lane - 8)] = t;
    }
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
                     (const int32_t*)w.rtok, w.krec, w.kent, w.kitem);
  return hipGetLastError();
}

}  // namespace ca
