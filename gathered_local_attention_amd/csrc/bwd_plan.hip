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
// in LDS, one workgroup per image; see its comment.  Larger images go
// through six grid-wide kernels, each parallel over tokens, slots or
// clusters of the whole batch:
//   1. inv = -1, counts = 0
//   2. inv[token] = position of the token in q_idx (c*cs + m)
//   3. per query cluster i (one thread): every slot looks up its key cluster
//      (jn = inv[token]); the first slot of i that points into key cluster
//      j stages the entry (j, per-member multiplicities) in i's staging row
//      (compact, ended by a sentinel) and counts it for j (atomic)
//   4. per image, exclusive scan of the counts -> segment (start, end)
//      pairs, absolute in the entry arrays
//   5. per query cluster, its staged entries are placed in their segments
//      (atomic cursor)
//   6. per key cluster, its segment is sorted by i (which fixes the
//      summation order of the key-major pass and makes it deterministic) and
//      every entry gets the q_idx row of its i, so that the key-major pass
//      gathers without a further lookup.
#include "common.h"
#include "dpp_scan.h"

#include <algorithm>

namespace ca {

namespace {

constexpr int kPlanThreads = 1024;
constexpr int kMaxNk = 64;
constexpr int kGridThreads = 256;

__global__ void __launch_bounds__(kGridThreads)
plan_init_kernel(int64_t n_inv, int64_t n_cnt, int32_t* __restrict__ inv, int32_t* __restrict__ cnt) {
  const int64_t x = (int64_t)blockIdx.x * kGridThreads + threadIdx.x;
  if (x < n_inv) inv[x] = -1;
  if (x < n_cnt) cnt[x] = 0;
}

// one thread per q_idx position (c*8 + m) of the batch
__global__ void __launch_bounds__(kGridThreads)
plan_inv_kernel(int B, int N, int C, const int32_t* __restrict__ q_idx, int32_t* __restrict__ inv) {
  const int64_t x = (int64_t)blockIdx.x * kGridThreads + threadIdx.x;
  const int P = 8 * C;
  if (x >= (int64_t)B * P) return;
  const int64_t b = x / P;
  const int t = q_idx[x];
  if (t >= 0 && t < N) inv[b * N + t] = (int32_t)(x - b * P);
}

// Entry staging, per query cluster i: every distinct key cluster j that a
// slot of i points into becomes one entry (j, per-member multiplicities),
// staged compactly at stage[i*nk ...] (entry count in nent[i]) and counted
// for j (integer atomic).  Eight lanes per query cluster, lane g on slot
// group g: a group that holds the whole cluster j in member order (as the
// neighbour build writes it; absent members of a partial cluster are -1 on
// both sides) is recognised from one inverse lookup and j's q_idx row, and
// the groups' entries are merged by lane shuffles.  A cluster with any other
// group is staged by its lane 0 slot by slot (stage_serial).
constexpr int kCountThreads = 256;   // 32 query clusters per workgroup

__device__ void stage_serial(int64_t bc, int64_t b, int N, int C, int nk,
                             const int32_t* __restrict__ key_idx, const int32_t* __restrict__ inv,
                             int32_t* __restrict__ cnt, RevEntry* __restrict__ stage,
                             int32_t* __restrict__ nent, int32_t* my) {
  for (int s = 0; s < nk; ++s) {
    const int t = key_idx[bc * nk + s];
    my[s] = (t >= 0 && t < N) ? inv[b * N + t] : -1;   // (j << 3) | member, or -1
  }
  RevEntry* st = stage + bc * nk;
  int ne = 0;
  for (int s = 0; s < nk; ++s) {
    const int js = my[s];
    if (js < 0) continue;
    const int j = js >> 3;
    bool first = true;
    for (int u = s - 1; u >= 0; --u)
      if (my[u] >= 0 && (my[u] >> 3) == j) { first = false; break; }
    if (!first) continue;
    uint64_t mult = 0;
    for (int u = s; u < nk; ++u)
      if (my[u] >= 0 && (my[u] >> 3) == j) mult += 1ull << (8 * (my[u] & 7));
    RevEntry e;
    e.i = j;   // key cluster while staged
    e.pad = 0;
    e.mult = mult;
    st[ne++] = e;
    atomicAdd(&cnt[b * C + j], 1);
  }
  nent[bc] = ne;
}

__global__ void __launch_bounds__(kCountThreads)
plan_count_kernel(int B, int N, int C, int nk, const int32_t* __restrict__ key_idx,
                  const int32_t* __restrict__ q_idx, const int32_t* __restrict__ inv,
                  int32_t* __restrict__ cnt, RevEntry* __restrict__ stage,
                  int32_t* __restrict__ nent) {
  __shared__ int32_t jn[kCountThreads / 8][kMaxNk + 1];
  const int64_t bc = ((int64_t)blockIdx.x * kCountThreads + threadIdx.x) >> 3;
  const int g = threadIdx.x & 7;
  const int lane = threadIdx.x & 63;
  if (bc >= (int64_t)B * C) return;   // whole lane groups leave together
  const int64_t b = bc / C;
  const int ng = nk % 8 == 0 ? nk / 8 : 0;   // other list lengths: slot by slot
  int j = -1;
  uint64_t add = 0;
  bool reg = false;
  if (g < ng) {
    const int4* kr = reinterpret_cast<const int4*>(key_idx + bc * nk + 8 * g);
    const int4 a = kr[0], c = kr[1];
    const int t0 = a.x;
    const int p0 = (t0 >= 0 && t0 < N) ? inv[b * N + t0] : -1;
    reg = p0 >= 0 && (p0 & 7) == 0;
    if (reg) {
      const int4* qr = reinterpret_cast<const int4*>(q_idx + (b * C + (p0 >> 3)) * 8);
      const int4 qa = qr[0], qc = qr[1];
      reg = qa.y == a.y && qa.z == a.z && qa.w == a.w && qc.x == c.x && qc.y == c.y &&
            qc.z == c.z && qc.w == c.w;
      const int tk[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
#pragma unroll
      for (int m = 0; m < 8; ++m) add |= tk[m] >= 0 ? 1ull << (8 * m) : 0ull;
      j = p0 >> 3;
    }
  }
  const uint32_t irregular = (uint32_t)(__ballot(g < ng && !reg) >> (lane & ~7)) & 0xFFu;
  if (irregular || ng == 0) {   // the same for the 8 lanes of the cluster
    if (g == 0) stage_serial(bc, b, N, C, nk, key_idx, inv, cnt, stage, nent, jn[threadIdx.x >> 3]);
    return;
  }
  // merge groups that point into the same key cluster; the first one stages
  uint64_t mult = 0;
  bool first = g < ng;
#pragma unroll
  for (int o = 0; o < 8; ++o) {
    const int jo = __shfl(j, o, 8);
    const uint64_t ao = __shfl(add, o, 8);
    if (o < ng && jo == j && g < ng) {
      mult += ao;
      if (o < g) first = false;
    }
  }
  const uint32_t fb = (uint32_t)(__ballot(first) >> (lane & ~7)) & 0xFFu;
  if (first) {
    RevEntry e;
    e.i = j;
    e.pad = 0;
    e.mult = mult;
    stage[bc * nk + __popc(fb & ((1u << g) - 1u))] = e;
    atomicAdd(&cnt[b * C + j], 1);
  }
  if (g == 0) nent[bc] = __popc(fb);
}

// one workgroup per image: segment offsets from the counts.  Counts are
// staged through LDS in chunks of kScanChunk (coalesced), each thread scans
// a contiguous run of the chunk, one workgroup scan joins the runs.
constexpr int kScanChunk = 8192;

__global__ void __launch_bounds__(kPlanThreads)
plan_scan_kernel(int C, int nk, const int32_t* __restrict__ cnt_all, int2* __restrict__ seg_all,
                 int32_t* __restrict__ cur_all) {
  __shared__ int32_t v[kScanChunk];
  __shared__ int32_t tmp[17];
  const int64_t b = blockIdx.x;
  const int32_t* cnt = cnt_all + b * C;
  int2* seg = seg_all + b * C;
  int32_t* cur = cur_all + b * C;
  const int base = (int)(b * C * nk);   // the image's entries start here
  constexpr int kPer = kScanChunk / kPlanThreads;
  int carry = 0;
  for (int c0 = 0; c0 < C; c0 += kScanChunk) {
    const int n = min(kScanChunk, C - c0);
    for (int x = threadIdx.x; x < n; x += kPlanThreads) v[x] = cnt[c0 + x];
    __syncthreads();
    const int r0 = threadIdx.x * kPer;
    int run = 0;
#pragma unroll
    for (int r = 0; r < kPer; ++r) run += r0 + r < n ? v[r0 + r] : 0;
    int tot;
    int acc = carry + block_exclusive_scan_dpp(run, tmp, kPlanThreads, &tot);
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
      if (r0 + r < n) {
        const int c = v[r0 + r];
        v[r0 + r] = acc;
        acc += c;
      }
    }
    __syncthreads();
    for (int x = threadIdx.x; x < n; x += kPlanThreads) {
      seg[c0 + x] = make_int2(base + v[x], base + v[x] + cnt[c0 + x]);
      cur[c0 + x] = v[x];
    }
    carry += tot;
    __syncthreads();   // v and tmp are reused by the next chunk
  }
}

// Eight lanes per query cluster: its staged entries into their segments
// (atomic cursors; the order inside a segment is fixed by the sort after).
__global__ void __launch_bounds__(kGridThreads)
plan_place_kernel(int B, int C, int nk, const RevEntry* __restrict__ stage,
                  const int32_t* __restrict__ nent, int32_t* __restrict__ cur_all,
                  RevEntry* __restrict__ rev_all) {
  const int64_t bc = ((int64_t)blockIdx.x * kGridThreads + threadIdx.x) >> 3;
  const int g = threadIdx.x & 7;
  if (bc >= (int64_t)B * C) return;
  const int64_t b = bc / C;
  const int ne = nent[bc];
  for (int e = g; e < ne; e += 8) {
    const RevEntry s = stage[bc * nk + e];
    const int pos = atomicAdd(&cur_all[b * C + s.i], 1);
    RevEntry r;
    r.i = (int32_t)(bc - b * C);
    r.pad = 0;
    r.mult = s.mult;
    rev_all[b * C * nk + pos] = r;
  }
}

// One thread per key cluster: its segment ordered by query cluster i (in
// registers when it holds at most kSortRegs entries), which fixes the
// summation order of the key-major pass and makes it deterministic; then
// every entry gets the q_idx row of its i, so that the key-major pass
// gathers without a further lookup.  (Eight lanes per key cluster, each
// entry placed by counting the smaller i of its segment, measured slower:
// 17.5 against 11 us at high-res.)
constexpr int kSortRegs = 16;

__global__ void __launch_bounds__(kGridThreads)
plan_sort_kernel(int B, int C, int nk, const int32_t* __restrict__ q_idx,
                 const int2* __restrict__ seg_all, RevEntry* __restrict__ rev,
                 int32_t* __restrict__ rtok_all) {
  const int64_t bj = (int64_t)blockIdx.x * kGridThreads + threadIdx.x;
  if (bj >= (int64_t)B * C) return;
  const int64_t b = bj / C;
  const int2 sg = seg_all[bj];   // absolute entry range of key cluster j
  const int a = sg.x, z = sg.y;
  int4* rt = reinterpret_cast<int4*>(rtok_all);
  const int32_t* qi = q_idx + b * C * 8;
  if (z - a <= kSortRegs) {
    int ii[kSortRegs];
    uint64_t mm[kSortRegs];
#pragma unroll
    for (int x = 0; x < kSortRegs; ++x) {
      if (a + x < z) {
        const RevEntry e = rev[a + x];
        ii[x] = e.i;
        mm[x] = e.mult;
      } else {
        ii[x] = 0x7fffffff;
        mm[x] = 0;
      }
    }
    // odd-even transposition sort (the i are distinct)
#pragma unroll
    for (int r = 0; r < kSortRegs; ++r)
#pragma unroll
      for (int x = r & 1; x + 1 < kSortRegs; x += 2)
        if (ii[x] > ii[x + 1]) {
          const int ti = ii[x];
          ii[x] = ii[x + 1];
          ii[x + 1] = ti;
          const uint64_t tm = mm[x];
          mm[x] = mm[x + 1];
          mm[x + 1] = tm;
        }
#pragma unroll
    for (int x = 0; x < kSortRegs; ++x) {
      if (a + x >= z) break;
      RevEntry e;
      e.i = ii[x];
      e.pad = 0;
      e.mult = mm[x];
      rev[a + x] = e;
      const int4* row = reinterpret_cast<const int4*>(qi + ii[x] * 8);
      rt[2 * (a + x)] = row[0];
      rt[2 * (a + x) + 1] = row[1];
    }
    return;
  }
  for (int x = a + 1; x < z; ++x) {
    const RevEntry key = rev[x];
    int y = x - 1;
    while (y >= a && rev[y].i > key.i) {
      rev[y + 1] = rev[y];
      --y;
    }
    rev[y + 1] = key;
  }
  for (int x = a; x < z; ++x) {
    const int4* row = reinterpret_cast<const int4*>(qi + rev[x].i * 8);
    rt[2 * x] = row[0];
    rt[2 * x + 1] = row[1];
  }
}

// ---------------------------------------------------------------------------
// Images with at most MAXC clusters (256: up to 2048 tokens and 12288
// slots; 512: up to 4096 tokens), one workgroup each, all in LDS.  A thread
// owns whole slot groups (8 consecutive slots of one cluster's list, loaded
// as two 16-byte vectors) and works on each distinct key cluster j its
// group points into (usually one, which is checked first): it sets bit i of
// row j in an LDS bitmap, and later adds the group's member counts for j
// into the multiplicity bytes of entry (i, j) with one integer atomic (a
// list has at most 64 slots, so a byte never carries).  Segment sizes are
// row popcounts and the entry of (i, j) sits at seg[j] + (set bits of row j
// below i), so segments come out ordered by i and the sums are order
// independent: deterministic without a sort.  The thread that adds an
// entry's multiplicities also records its i, and the entries go out one
// thread each, together with the q_idx row of their i (the eight query
// tokens the key-major pass gathers), which the workgroup keeps in LDS.
// With MAXC = 512 the multiplicities are accumulated in the entry array in
// global memory (zeroed first) instead of LDS.  Packed batches (Geom with
// offsets) run one workgroup per image with batch-global token ids; image
// b's entries live at [c0 * nk, c1 * nk).
// ---------------------------------------------------------------------------
constexpr int kPlanMaxSlots = 12288;

template <int MAXC>
struct PlanLds;
template <>
struct PlanLds<256> {
  static constexpr int kWords = 8, kTok = 2048, kGroupsPer = 2;
  unsigned long long mult[kPlanMaxSlots];
  uint8_t ent_i[kPlanMaxSlots];   // entry -> its query cluster i
};
template <>
struct PlanLds<512> {
  static constexpr int kWords = 16, kTok = 4096, kGroupsPer = 3;
  uint16_t ent_i[512 * 48];
};

template <int MAXC>
__global__ void __launch_bounds__(kPlanThreads)
plan_small_kernel(Geom g, int nk, const int32_t* __restrict__ q_idx,
                  const int32_t* __restrict__ key_idx, int2* __restrict__ seg_all,
                  RevEntry* __restrict__ rev_all, int32_t* __restrict__ rtok_all) {
  typedef PlanLds<MAXC> L;
  constexpr int kWords = L::kWords, kGroupsPer = L::kGroupsPer, kQPer = L::kTok / kPlanThreads;
  constexpr bool kGlobalMult = MAXC > 256;
  __shared__ int32_t inv[L::kTok];                                  // token -> position c*8 + m
  __shared__ __attribute__((aligned(16))) int32_t qp[L::kTok];      // position -> token
  __shared__ uint32_t bits[MAXC][kWords];
  __shared__ int32_t wo[MAXC][kWords];
  __shared__ L lds;
  __shared__ int32_t tmp[17];
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  int t0, N, c0, C;
  g.image(b, t0, N, c0, C);
  if (C == 0) return;
  const int tb = g.tok_base(t0);                             // token id of the image's token 0
  const int cb = g.clu_base(c0);                             // cluster id of its cluster 0
  const int ns = C * nk;
  const int ngroups = ns / 8;
  const int P = 8 * C;                                       // q_idx positions
  const int32_t* qi = q_idx + (int64_t)c0 * 8;
  const int32_t* ki = key_idx + (int64_t)c0 * nk;
  const int64_t base = (int64_t)c0 * nk;                     // the image's entries

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
  int qv[kQPer];
#pragma unroll
  for (int r = 0; r < kQPer; ++r) {
    const int x = tid + r * kPlanThreads;
    qv[r] = x < P ? qi[x] : -1;                              // -1: absent member
  }
  for (int t = tid; t < N; t += kPlanThreads) inv[t] = -1;
  for (int x = tid; x < MAXC * kWords; x += kPlanThreads) (&bits[0][0])[x] = 0u;
#pragma unroll
  for (int r = 0; r < kQPer; ++r)
    if (tid + r * kPlanThreads < P) qp[tid + r * kPlanThreads] = qv[r];
  __syncthreads();
#pragma unroll
  for (int r = 0; r < kQPer; ++r)
    if (qv[r] >= 0) inv[qv[r] - tb] = tid + r * kPlanThreads;
  __syncthreads();

  // key position (j << 3 | member) of every slot.  A group that holds the
  // whole cluster j in member order (as the neighbour build writes it) is
  // recognised from one lookup and the cluster's q_idx row; any other group
  // looks up all eight slots.
  int jn[kGroupsPer][8];
  bool one[kGroupsPer];
#pragma unroll
  for (int r = 0; r < kGroupsPer; ++r) {
    const int p0 = tok[r][0] >= 0 ? inv[tok[r][0] - tb] : -1;
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
      for (int m = 1; m < 8; ++m) jn[r][m] = tok[r][m] >= 0 ? inv[tok[r][m] - tb] : -1;
    }
  }
  // bitmap rows
#pragma unroll
  for (int r = 0; r < kGroupsPer; ++r) {
    const int gr = tid + r * kPlanThreads;
    if (gr >= ngroups) continue;
    const int i = gr * 8 / nk;
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

  // segment sizes, starts, per-word starts (exclusive scan over j < C <= MAXC)
  static_assert(MAXC <= kPlanThreads, "one bitmap row per thread");
  int vsum = 0;
  if (tid < C) {
#pragma unroll
    for (int w = 0; w < kWords; ++w) vsum += __popc(bits[tid][w]);
  }
  int total;
  const int ex = block_exclusive_scan_dpp(vsum, tmp, kPlanThreads, &total);
  if (tid < C) {
    int a = ex;
#pragma unroll
    for (int w = 0; w < kWords; ++w) {
      wo[tid][w] = a;
      a += __popc(bits[tid][w]);
    }
    seg_all[c0 + tid] = make_int2((int)(base + ex), (int)(base + ex + vsum));
  }
  RevEntry* rev = rev_all + base;
  if constexpr (kGlobalMult) {
    for (int p = tid; p < total; p += kPlanThreads) rev[p].mult = 0ull;
    __threadfence_block();
  } else {
    for (int p = tid; p < total; p += kPlanThreads) lds.mult[p] = 0ull;
  }
  __syncthreads();

  // multiplicities: one integer atomic per distinct key cluster of a group
  auto add_mult = [&](int pos, uint64_t add, int i) {
    if constexpr (kGlobalMult) {
      atomicAdd(reinterpret_cast<unsigned long long*>(&rev[pos].mult), (unsigned long long)add);
      lds.ent_i[pos] = (uint16_t)i;
    } else {
      atomicAdd(&lds.mult[pos], (unsigned long long)add);
      lds.ent_i[pos] = (uint8_t)i;   // groups of one i that share j store the same value
    }
  };
#pragma unroll
  for (int r = 0; r < kGroupsPer; ++r) {
    const int gr = tid + r * kPlanThreads;
    if (gr >= ngroups) continue;
    const int i = gr * 8 / nk;
    const uint32_t below = (1u << (i & 31)) - 1u;
    if (one[r]) {   // the members of j once each (absent members: -1 slots)
      const int jj = jn[r][0] >> 3;
      uint64_t add = 0;
#pragma unroll
      for (int m = 0; m < 8; ++m) add |= tok[r][m] >= 0 ? 1ull << (8 * m) : 0ull;
      add_mult(wo[jj][i >> 5] + __popc(bits[jj][i >> 5] & below), add, i);
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
      add_mult(wo[jj][i >> 5] + __popc(bits[jj][i >> 5] & below), add, i);
    }
  }
  if constexpr (kGlobalMult) __threadfence_block();
  __syncthreads();

  // entries out, one thread per entry (coalesced stores)
  int4* rt = reinterpret_cast<int4*>(rtok_all + base * 8);
  for (int p = tid; p < total; p += kPlanThreads) {
    const int i = lds.ent_i[p];   // image-local; the entry records the batch-wide id
    if constexpr (kGlobalMult) {
      rev[p].i = cb + i;
      rev[p].pad = 0;
    } else {
      RevEntry e;
      e.i = cb + i;
      e.pad = 0;
      e.mult = lds.mult[p];
      rev[p] = e;
    }
    const int4* row = reinterpret_cast<const int4*>(qp + i * 8);
    rt[2 * p] = row[0];
    rt[2 * p + 1] = row[1];
  }
}

}  // namespace

hipError_t launch_bwd_plan(int B, int N, int C, int nk, const int32_t* q_idx,
                           const int32_t* key_idx, const BwdWorkspace& w, hipStream_t st,
                           const Geom* packed) {
  if (nk > kMaxNk) return hipErrorInvalidValue;
  // one workgroup per image, in LDS: equal-size images, or the images of a
  // packed batch (then every image must fit)
  const Geom g = packed ? *packed : Geom{nullptr, nullptr, N, C, 0};
  const int nimg = B;
  const int mn = g.N, mc = packed ? (g.N + 7) / 8 : C;
  if (nk % 8 == 0 && mn <= 2048 && mc <= 256 && mc * nk <= kPlanMaxSlots) {
    hipLaunchKernelGGL(plan_small_kernel<256>, dim3(nimg), dim3(kPlanThreads), 0, st, g, nk, q_idx,
                       key_idx, w.seg, w.rev, w.rtok);
    return hipGetLastError();
  }
  if (nk % 8 == 0 && nk <= 48 && mn <= 4096 && mc <= 512) {
    hipLaunchKernelGGL(plan_small_kernel<512>, dim3(nimg), dim3(kPlanThreads), 0, st, g, nk, q_idx,
                       key_idx, w.seg, w.rev, w.rtok);
    return hipGetLastError();
  }
  // grid-wide: a packed batch as one image of its N tokens and C clusters
  if (packed) B = 1;
  const int64_t tokens = (int64_t)B * N, clusters = (int64_t)B * C;
  auto grid = [](int64_t n) { return dim3((unsigned)((n + kGridThreads - 1) / kGridThreads)); };
  hipLaunchKernelGGL(plan_init_kernel, grid(std::max<int64_t>(tokens, 1)), dim3(kGridThreads), 0,
                     st, tokens, clusters, w.inv, w.cnt);
  hipLaunchKernelGGL(plan_inv_kernel, grid(clusters * 8), dim3(kGridThreads), 0, st, B, N, C,
                     q_idx, w.inv);
  hipLaunchKernelGGL(plan_count_kernel, grid(clusters * 8), dim3(kCountThreads), 0, st, B, N, C, nk,
                     key_idx, q_idx, (const int32_t*)w.inv, w.cnt, w.stage, w.nent);
  hipLaunchKernelGGL(plan_scan_kernel, dim3(B), dim3(kPlanThreads), 0, st, C, nk,
                     (const int32_t*)w.cnt, w.seg, w.cursor);
  hipLaunchKernelGGL(plan_place_kernel, grid(clusters * 8), dim3(kGridThreads), 0, st, B, C, nk,
                     (const RevEntry*)w.stage, (const int32_t*)w.nent, w.cursor, w.rev);
  hipLaunchKernelGGL(plan_sort_kernel, grid(clusters), dim3(kGridThreads), 0, st, B, C, nk, q_idx,
                     (const int2*)w.seg, w.rev, w.rtok);
  return hipGetLastError();
}

}  // namespace ca
