// Prefix sums over a wavefront and a workgroup with DPP lane moves: six
// dependent VALU steps per wavefront instead of six LDS-crossbar shuffles.
#pragma once
#include "common.h"

namespace ca {
namespace {

// Inclusive prefix sum across the 64 lanes (every lane active): shifts by
// 1, 2, 4 and 8 within each 16-lane row (lanes without a source add 0),
// then the last lane of rows 0 and 2 into rows 1 and 3, and lane 31 into
// rows 2 and 3.
__device__ __forceinline__ int wave_inclusive_scan_dpp(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);    // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);    // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);    // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);    // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);   // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);   // row_bcast:31
  return v;
}

// block_exclusive_scan with the DPP wavefront scan: exclusive prefix sum of
// one value per thread over `nthreads` (a multiple of 64, at most 1024),
// two barriers, `tmp` 17 ints of LDS; returns the prefix, writes the total.
__device__ __forceinline__ int block_exclusive_scan_dpp(int v, int* tmp, int nthreads, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int inc = wave_inclusive_scan_dpp(v);
  if (lane == 63) tmp[w] = inc;
  __syncthreads();
  if (w == 0) {
    const int nw = nthreads >> 6;
    const int t = lane < nw ? tmp[lane] : 0;
    const int ti = wave_inclusive_scan_dpp(t);
    if (lane < nw) tmp[lane] = ti - t;
    if (lane == nw - 1) tmp[16] = ti;
  }
  __syncthreads();
  *total = tmp[16];
  return tmp[w] + inc - v;
}

}  // namespace
}  // namespace ca
