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
// plan_small_kernel (images of at most 256 clusters) keeps the whole image
// in LDS; see its comment.  plan_kernel handles any size:
// one 1024-thread workgroup per image (every counter it touches belongs to
// its image, so no global zeroing pass and no cross-workgroup ordering are
// needed).  Phases, separated by workgroup barriers:
//   1. inv[token] = position of the token in q_idx (c*cs + m); zero counts.
//   2. per tile of query clusters: every slot looks up its key cluster
//      (jn = inv[token], staged in LDS); the first slot of cluster i that
//      points into key cluster j stages the entry (j, per-member
//      multiplicities) at its own slot position and counts it for j.
//   3. exclusive scan of the counts -> segment offsets.
//   4. staged entries are scattered into their segments (atomic cursor).
//   5. each segment is sorted by i, which fixes the summation order of the
//      key-major pass and makes it deterministic.
//   6. every entry gets the query tokens of its cluster i (the q_idx row),
//      so that the key-major pass gathers without a further lookup.
#include "common.h"

namespace ca {

namespace {

constexpr int kPlanThreads = 1024;
constexpr int kMaxNk = 64;
constexpr int kTileSlots = 12288;   // 48 KiB of LDS: 256 clusters of 48 slots

__global__ void __launch_bounds__(kPlanThreads)
plan_kernel(int N, int nk, const int32_t* __restrict__ q_idx, const int32_t* __restrict__ key_idx,
            int32_t* __restrict__ inv_all, int32_t* __restrict__ cnt_all,
            int32_t* __restrict__ off_all, int32_t* __restrict__ cur_all,
            RevEntry* __restrict__ stage_all, RevEntry* __restrict__ rev_all,
            int32_t* __restrict__ rtok_all) {
  __shared__ int32_t jn[kTileSlots];
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
  RevEntry* stage = stage_all + (int64_t)b * C * nk;
  RevEntry* rev = rev_all + (int64_t)b * C * nk;
  const int64_t slots = (int64_t)C * nk;

  // 1 (inv starts at -1 so that a q_idx that is not a permutation leaves
  //    unreached tokens marked invalid instead of holding stale values)
  for (int t = tid; t < N; t += kPlanThreads) inv[t] = -1;
  for (int j = tid; j < C; j += kPlanThreads) cnt[j] = 0;
  __syncthreads();
  for (int p = tid; p < N; p += kPlanThreads) inv[qi[p]] = p;
  __syncthreads();

  // 2
  const int tile_clusters = kTileSlots / nk;
  for (int i0 = 0; i0 < C; i0 += tile_clusters) {
    const int nc = min(tile_clusters, C - i0);
    const int ns = nc * nk;
    for (int x = tid; x < ns; x += kPlanThreads) {
      const int t = ki[(int64_t)i0 * nk + x];
      jn[x] = t >= 0 ? inv[t] : -1;          // (j << 3) | n
    }
    __syncthreads();
    for (int x = tid; x < ns; x += kPlanThreads) {
      const int il = x / nk, s = x - il * nk;
      const int* my = jn + il * nk;
      const int js = my[s];
      RevEntry e;
      e.i = -1;
      e.pad = 0;
      e.mult = 0;
      if (js >= 0) {
        const int j = js >> 3;
        bool first = true;
        for (int u = s - 1; u >= 0; --u)
          if (my[u] >= 0 && (my[u] >> 3) == j) { first = false; break; }
        if (first) {
          uint64_t mult = 0;
          for (int u = s; u < nk; ++u)
            if (my[u] >= 0 && (my[u] >> 3) == j) mult += 1ull << (8 * (my[u] & 7));
          e.i = j;   // key cluster while staged
          e.mult = mult;
          atomicAdd(&cnt[j], 1);
        }
      }
      stage[(int64_t)i0 * nk + x] = e;
    }
    __syncthreads();
  }

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
  __syncthreads();

  // 4
  for (int64_t x = tid; x < slots; x += kPlanThreads) {
    const RevEntry s = stage[x];
    if (s.i < 0) continue;
    const int pos = atomicAdd(&cur[s.i], 1);
    RevEntry r;
    r.i = (int32_t)(x / nk);
    r.pad = 0;
    r.mult = s.mult;
    rev[pos] = r;
  }
  __syncthreads();

  // 5
  for (int j = tid; j < C; j += kPlanThreads) {
    const int a = off[j], z = off[j + 1];
    for (int x = a + 1; x < z; ++x) {
      const RevEntry key = rev[x];
      int y = x - 1;
      while (y >= a && rev[y].i > key.i) {
        rev[y + 1] = rev[y];
        --y;
      }
      rev[y + 1] = key;
    }
  }
  __syncthreads();

  // 6
  int4* rt = reinterpret_cast<int4*>(rtok_all + (int64_t)b * C * nk * 8);
  const int total = off[C];
  for (int x = tid; x < total; x += kPlanThreads) {
    const int4* row = reinterpret_cast<const int4*>(qi + rev[x].i * 8);
    rt[2 * x] = row[0];
    rt[2 * x + 1] = row[1];
  }
}

// ---------------------------------------------------------------------------
// Images with at most 256 clusters and 12288 slots, one workgroup each, all
// in LDS.  A thread owns whole slot groups (8 consecutive slots of one
// cluster's list, loaded as two 16-byte vectors) and works on each distinct
// key cluster j its group points into (usually one, which is checked first):
// it sets bit i of row j in an LDS bitmap, and later adds the group's member
// counts for j into the multiplicity bytes of entry (i, j) with one LDS
// integer atomic (a list has at most 64 slots, so a byte never carries).
// Segment sizes are row popcounts and the entry of (i, j) sits at off[j] +
// (set bits of row j below i), so segments come out ordered by i and the
// sums are order independent: deterministic without a sort.  The thread
// that adds an entry's multiplicities also records its i, and the entries go
// out one thread each, together with the q_idx row of their i (the eight
// query tokens the key-major pass gathers), which the workgroup keeps in LDS.
// ---------------------------------------------------------------------------
constexpr int kPlanMaxC = 256;
constexpr int kPlanWords = kPlanMaxC / 32;
constexpr int kPlanMaxSlots = 12288;
constexpr int kGroupsPer = (kPlanMaxSlots / 8 + kPlanThreads - 1) / kPlanThreads;   // 2

__global__ void __launch_bounds__(kPlanThreads)
plan_small_kernel(int N, int nk, const int32_t* __restrict__ q_idx,
                  const int32_t* __restrict__ key_idx, int32_t* __restrict__ off_all,
                  RevEntry* __restrict__ rev_all, int32_t* __restrict__ rtok_all) {
  __shared__ int32_t inv[kSortChunk];                       // token -> position c*8 + m
  __shared__ __attribute__((aligned(16))) int32_t qp[kSortChunk];   // position -> token
  __shared__ uint32_t bits[kPlanMaxC][kPlanWords];
  __shared__ int32_t wo[kPlanMaxC][kPlanWords];
  __shared__ unsigned long long mult[kPlanMaxSlots];
  __shared__ uint8_t ent_i[kPlanMaxSlots];                  // entry -> its query cluster i
  __shared__ int32_t tmp[17];
  const int b = blockIdx.x;
  const int C = N / 8;
  const int tid = threadIdx.x;
  const int ns = C * nk;
  const int ngroups = ns / 8;
  const int32_t* qi = q_idx + (int64_t)b * N;
  const int32_t* ki = key_idx + (int64_t)b * ns;

  // this thread's slot groups gr = tid + r * 1024, loaded up front
  int tok[kGroupsPer][8];
#pragma unroll
  for (int r = 0; r < kGroupsPer; ++r) {
    const int gr = tid + r * kPlanThreads;
    int4 a = make_int4(-1, -1, -1, -1), c = a;
    if (gr < ngroups) {
      a = reinterpret_cast<const int4*>(ki)[2 * gr];
      c = reinterpret_cast<const int4*>(ki)[2 * gr + 1];
    }
    tok[r][0] = a.x; tok[r][1] = a.y; tok[r][2] = a.z; tok[r][3] = a.w;
    tok[r][4] = c.x; tok[r][5] = c.y; tok[r][6] = c.z; tok[r][7] = c.w;
  }
  const int q0 = tid < N ? qi[tid] : -1;                       // N <= 2048
  const int q1 = tid + kPlanThreads < N ? qi[tid + kPlanThreads] : -1;
  for (int t = tid; t < N; t += kPlanThreads) inv[t] = -1;
  for (int x = tid; x < kPlanMaxC * kPlanWords; x += kPlanThreads) (&bits[0][0])[x] = 0u;
  if (tid < N) qp[tid] = q0;
  if (tid + kPlanThreads < N) qp[tid + kPlanThreads] = q1;
  __syncthreads();
  if (q0 >= 0) inv[q0] = tid;
  if (q1 >= 0) inv[q1] = tid + kPlanThreads;
  __syncthreads();

  // key position (j << 3 | member) of every slot.  A group that holds the
  // whole cluster j in member order (as the neighbour build writes it) is
  // recognised from one lookup and the cluster's q_idx row; any other group
  // looks up all eight slots.
  int jn[kGroupsPer][8];
  bool one[kGroupsPer];
#pragma unroll
  for (int r = 0; r < kGroupsPer; ++r) {
    const int p0 = tok[r][0] >= 0 ? inv[tok[r][0]] : -1;
    bool same = p0 >= 0 && (p0 & 7) == 0;
    if (same) {
      const int4 a = reinterpret_cast<const int4*>(qp + p0)[0];
      const int4 c = reinterpret_cast<const int4*>(qp + p0)[1];
      same = a.y == tok[r][1] && a.z == tok[r][2] && a.w == tok[r][3] && c.x == tok[r][4] &&
             c.y == tok[r][5] && c.z == tok[r][6] && c.w == tok[r][7];
    }
    one[r] = same;
    jn[r][0] = p0;
    if (!same) {
#pragma unroll
      for (int m = 1; m < 8; ++m) jn[r][m] = tok[r][m] >= 0 ? inv[tok[r][m]] : -1;
    }
  }
  // bitmap rows
#pragma unroll
  for (int r = 0; r < kGroupsPer; ++r) {
    const int i = (tid + r * kPlanThreads) * 8 / nk;
    if (one[r]) {
      atomicOr(&bits[jn[r][0] >> 3][i >> 5], 1u << (i & 31));
      continue;
    }
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      if (jn[r][m] < 0) continue;
      bool seen = false;
#pragma unroll
      for (int u = 0; u < m; ++u) seen = seen || (jn[r][u] >= 0 && (jn[r][u] >> 3) == (jn[r][m] >> 3));
      if (!seen) atomicOr(&bits[jn[r][m] >> 3][i >> 5], 1u << (i & 31));
    }
  }
  __syncthreads();

  // segment sizes, offsets, per-word offsets (exclusive scan over j < C <= 256)
  int v = 0;
  if (tid < C) {
#pragma unroll
    for (int w = 0; w < kPlanWords; ++w) v += __popc(bits[tid][w]);
  }
  int total;
  const int ex = block_exclusive_scan(v, tmp, kPlanThreads, &total);
  if (tid < C) {
    int a = ex;
#pragma unroll
    for (int w = 0; w < kPlanWords; ++w) {
      wo[tid][w] = a;
      a += __popc(bits[tid][w]);
    }
  }
  int32_t* goff = off_all + (int64_t)b * (C + 1);
  if (tid <= C) goff[tid] = tid < C ? ex : total;
  for (int p = tid; p < total; p += kPlanThreads) mult[p] = 0ull;
  __syncthreads();

  // multiplicities: one LDS atomic per distinct key cluster of a group
#pragma unroll
  for (int r = 0; r < kGroupsPer; ++r) {
    const int i = (tid + r * kPlanThreads) * 8 / nk;
    const uint32_t below = (1u << (i & 31)) - 1u;
    if (one[r]) {   // members 0..7 once each
      const int jj = jn[r][0] >> 3;
      const uint64_t add = 0x0101010101010101ull;
      const int pos = wo[jj][i >> 5] + __popc(bits[jj][i >> 5] & below);
      atomicAdd(&mult[pos], (unsigned long long)add);
      ent_i[pos] = (uint8_t)i;
      continue;
    }
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      if (jn[r][m] < 0) continue;
      const int jj = jn[r][m] >> 3;
      bool seen = false;
#pragma unroll
      for (int u = 0; u < m; ++u) seen = seen || (jn[r][u] >= 0 && (jn[r][u] >> 3) == jj);
      if (seen) continue;
      uint64_t add = 0;
#pragma unroll
      for (int u = m; u < 8; ++u)
        if (jn[r][u] >= 0 && (jn[r][u] >> 3) == jj) add += 1ull << (8 * (jn[r][u] & 7));
      const int pos = wo[jj][i >> 5] + __popc(bits[jj][i >> 5] & below);
      atomicAdd(&mult[pos], (unsigned long long)add);
      ent_i[pos] = (uint8_t)i;   // groups of one i that share j store the same value
    }
  }
  __syncthreads();

  // entries out, one thread per entry (coalesced stores)
  RevEntry* rev = rev_all + (int64_t)b * ns;
  int4* rt = reinterpret_cast<int4*>(rtok_all + (int64_t)b * ns * 8);
  for (int p = tid; p < total; p += kPlanThreads) {
    const int i = ent_i[p];
    RevEntry e;
    e.i = i;
    e.pad = 0;
    e.mult = mult[p];
    rev[p] = e;
    const int4* row = reinterpret_cast<const int4*>(qp + i * 8);
    rt[2 * p] = row[0];
    rt[2 * p + 1] = row[1];
  }
}

}  // namespace

hipError_t launch_bwd_plan(int B, int N, int nk, const int32_t* q_idx, const int32_t* key_idx,
                           const BwdWorkspace& w, hipStream_t st) {
  if (nk > kMaxNk) return hipErrorInvalidValue;
  const int C = N / 8;
  if (N <= kSortChunk && C <= kPlanMaxC && C * nk <= kPlanMaxSlots && nk % 8 == 0) {
    hipLaunchKernelGGL(plan_small_kernel, dim3(B), dim3(kPlanThreads), 0, st, N, nk, q_idx, key_idx,
                       w.off, w.rev, w.rtok);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(plan_kernel, dim3(B), dim3(kPlanThreads), 0, st, N, nk, q_idx, key_idx,
                     w.inv, w.cnt, w.off, w.cursor, w.stage, w.rev, w.rtok);
  return hipGetLastError();
}

}  // namespace ca
