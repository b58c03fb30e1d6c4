// Transposed (key-major) slot lists for the backward pass.
//
// The query-major lists say which keys each query cluster reads; dK and dV
// need the converse: for every key cluster j, which query clusters i read
// any of j's tokens, and how many of i's slots point at each member of j.
// Building that converse lets the key-major backward pass own its outputs
// (no atomics on the gradients, bitwise reproducible sums).  It is derived
// from the per-image lists of the forward, whose construction the English
// notes page "AFFMAE: Scalable Vision Pre-Training for High-Resolution
// Microscopy Segmentation on Desktop Hardware" ("Overall Architecture":
// local balanced clustering) leaves to the implementation.
//
// One workgroup per image, five phases separated by workgroup barriers:
//   1. inv[token] = position of the token in q_idx; zero the counters.
//   2. per query cluster i: group its slots by key cluster j (first
//      occurrence order), stage one entry (i, per-member multiplicities) per
//      distinct j and count entries per j.
//   3. exclusive scan of the counts -> segment offsets.
//   4. scatter the staged entries into their segments.
//   5. sort every segment by i (the scatter order is not deterministic).
#include "common.h"

namespace ca {

namespace {

constexpr int kPlanThreads = 256;
constexpr int kMaxNk = 64;

__global__ void __launch_bounds__(kPlanThreads)
plan_kernel(int N, int nk, const int32_t* __restrict__ q_idx, const int32_t* __restrict__ key_idx,
            int32_t* __restrict__ inv_all, int32_t* __restrict__ cnt_all,
            int32_t* __restrict__ off_all, int32_t* __restrict__ cur_all,
            int32_t* __restrict__ nent_all, RevEntry* __restrict__ stage_all,
            RevEntry* __restrict__ rev_all) {
  __shared__ int32_t slots[kPlanThreads][kMaxNk + 1];
  __shared__ int32_t scan[kPlanThreads];
  const int b = blockIdx.x;
  const int C = N / 8;
  const int tid = threadIdx.x;
  const int32_t* qi = q_idx + (int64_t)b * N;
  const int32_t* ki = key_idx + (int64_t)b * C * nk;
  int32_t* inv = inv_all + (int64_t)b * N;
  int32_t* cnt = cnt_all + (int64_t)b * C;
  int32_t* off = off_all + (int64_t)b * (C + 1);
  int32_t* cur = cur_all + (int64_t)b * C;
  int32_t* nent = nent_all + (int64_t)b * C;
  RevEntry* stage = stage_all + (int64_t)b * C * nk;
  RevEntry* rev = rev_all + (int64_t)b * C * nk;

  // 1 (inv starts at -1 so that a q_idx that is not a permutation leaves
  //    unreached tokens marked invalid instead of holding stale values)
  for (int t = tid; t < N; t += kPlanThreads) inv[t] = -1;
  for (int j = tid; j < C; j += kPlanThreads) cnt[j] = 0;
  __syncthreads();
  for (int p = tid; p < N; p += kPlanThreads) inv[qi[p]] = p;
  __threadfence_block();
  __syncthreads();

  // 2
  for (int i0 = 0; i0 < C; i0 += kPlanThreads) {
    const int i = i0 + tid;
    if (i < C) {
      int32_t* my = slots[tid];
      for (int s = 0; s < nk; ++s) {
        const int t = ki[(int64_t)i * nk + s];
        my[s] = t >= 0 ? inv[t] : -1;     // (j << 3) | n
      }
      int ne = 0;
      for (int s = 0; s < nk; ++s) {
        const int js = my[s];
        if (js < 0) continue;
        bool first = true;
        for (int u = s - 1; u >= 0; --u) {
          if (my[u] >= 0 && (my[u] >> 3) == (js >> 3)) { first = false; break; }
        }
        if (!first) continue;
        uint64_t mult = 0;
        for (int u = s; u < nk; ++u) {
          if (my[u] >= 0 && (my[u] >> 3) == (js >> 3)) mult += 1ull << (8 * (my[u] & 7));
        }
        RevEntry e;
        e.i = js >> 3;      // key cluster while staged
        e.pad = 0;
        e.mult = mult;
        stage[(int64_t)i * nk + ne] = e;
        ++ne;
        atomicAdd(&cnt[js >> 3], 1);
      }
      nent[i] = ne;
    }
  }
  __threadfence_block();
  __syncthreads();

  // 3
  int carry = 0;
  for (int j0 = 0; j0 < C; j0 += kPlanThreads) {
    const int j = j0 + tid;
    const int v = j < C ? cnt[j] : 0;
    scan[tid] = v;
    __syncthreads();
    for (int o = 1; o < kPlanThreads; o <<= 1) {
      const int add = tid >= o ? scan[tid - o] : 0;
      __syncthreads();
      scan[tid] += add;
      __syncthreads();
    }
    if (j < C) {
      const int start = carry + scan[tid] - v;
      off[j] = start;
      cur[j] = start;
    }
    carry += scan[kPlanThreads - 1];
    __syncthreads();
  }
  if (tid == 0) off[C] = carry;
  __threadfence_block();
  __syncthreads();

  // 4
  for (int i = tid; i < C; i += kPlanThreads) {
    const int ne = nent[i];
    for (int e = 0; e < ne; ++e) {
      RevEntry s = stage[(int64_t)i * nk + e];
      const int j = s.i;
      const int pos = atomicAdd(&cur[j], 1);
      RevEntry r;
      r.i = i;
      r.pad = 0;
      r.mult = s.mult;
      rev[pos] = r;
    }
  }
  __threadfence_block();
  __syncthreads();

  // 5
  for (int j = tid; j < C; j += kPlanThreads) {
    const int a = off[j], z = off[j + 1];
    for (int x = a + 1; x < z; ++x) {
      RevEntry key = rev[x];
      int y = x - 1;
      while (y >= a && rev[y].i > key.i) {
        rev[y + 1] = rev[y];
        --y;
      }
      rev[y + 1] = key;
    }
  }
}

}  // namespace

hipError_t launch_bwd_plan(int B, int N, int nk, const int32_t* q_idx, const int32_t* key_idx,
                           const BwdWorkspace& w, hipStream_t st) {
  if (nk > kMaxNk) return hipErrorInvalidValue;
  hipLaunchKernelGGL(plan_kernel, dim3(B), dim3(kPlanThreads), 0, st, N, nk, q_idx, key_idx,
                     w.inv, w.cnt, w.off, w.cursor, w.nent, w.stage, w.rev);
  return hipGetLastError();
}

}  // namespace ca
