// Matrix-core (MFMA) cluster attention kernels for gfx950, bf16 / fp16,
// clusters of 8 and 48 key slots.
//
// What is computed: exact softmax attention of every query cluster over the
// 48 gathered key slots of its neighbour clusters, forward (O, LSE) and
// backward (dQ, dK, dV) - the local cluster attention of the English notes
// page "AFFMAE: Scalable Vision Pre-Training for High-Resolution Microscopy
// Segmentation on Desktop Hardware" ("Overall Architecture"), run as the
// numerically stable mixed-precision Flash-style kernels its arXiv abstract
// describes: bf16/fp16 operands, fp32 statistics and accumulation, logits in
// log2 units so every exponential is one v_exp_f32.
//
// Tiling (one 64-lane wavefront per item = (cluster, pair of heads)):
//  * v_mfma_f32_16x16x32 operand layout (checked on the hardware): lane
//    l = c + 16 g holds row/column c and reduction indices [8g, 8g+8); the
//    16x16 fp32 result puts rows 4g..4g+3 of column c in lane l.  Only this
//    one MFMA shape is used (16-deep products run on it with the upper half
//    of every lane's reduction slice zeroed); the MFMA units are far from
//    busy in these kernels, so a second shape would save little.
//  * A cluster has 8 queries, half a 16-wide tile, so the two heads of a
//    pair share one tile: columns 0-7 are head h0, 8-15 head h1.  Products
//    whose other operand differs per head run as two MFMAs, block-diagonal
//    over the heads, which keeps every lane of the softmax busy.
//  * Forward: the gathered rows go to a wavefront-private LDS tile through
//    direct-to-LDS loads (whole 128-byte rows per eight lanes); K is read
//    back in the MFMA layout and V through the transposing LDS read.
//  * Backward: the same staging; the query-major pass reads K transposed for
//    dQ, the key-major pass reads Q and dO transposed for dK and dV.  P and
//    dS are rounded once to the operand type for those products (relative
//    2^-8 in bf16, far below the bf16 rounding of the outputs).
//  * Workgroups are remapped so that each XCD (eight, dispatched
//    round-robin) walks one contiguous Morton range of clusters:
//    neighbouring clusters share their gathered rows in its L2.
//  * Partial clusters (images whose size is not a multiple of 8, packed
//    batches of images of different sizes): a -1 member of a q_idx row is
//    no query.  Its Q/dO/O rows are gathered from a clamped (valid) token
//    and nothing is stored for it; in the key-major pass it reads an
//    (LSE = +inf, Delta = 0) pair, so its P and dS are exactly 0.  Member 0
//    of every row is a token, so each store instruction keeps at least one
//    active lane (the pipelines count store instructions).
#include "common.h"
#include "mfma_util.h"

#include <algorithm>

namespace ca {

namespace {

constexpr int CS = 8;
constexpr int NK = 48;
constexpr int kWaves = 4;
__device__ __forceinline__ uint32_t swz(int s) { return (uint32_t)((s & 15) >> 1); }

// An output row of one head (32 dims) leaves the MFMA with lane group g
// holding dims 4g .. 4g+3 (lo) and 16+4g .. 16+4g+3 (hi).  Trading one half
// with the lane of group g ^ 1 (the same row) gives every lane 8
// consecutive dims, written with one 16-byte store at byte offset col.
// Every lane must take part (the exchange is a shuffle).
struct Row8 {
  uint4 v;
  uint32_t col;
};
__device__ __forceinline__ Row8 row8(uint2 lo, uint2 hi, int g) {
  const bool odd = (g & 1) != 0;
  const uint2 give = odd ? lo : hi;
  const uint2 got = make_uint2((uint32_t)__shfl_xor((int)give.x, 16, 64),
                               (uint32_t)__shfl_xor((int)give.y, 16, 64));
  Row8 r;
  // even g: dims 4g .. 4g+7; odd g: dims 12+4g .. 16+4g+3
  r.v = odd ? make_uint4(got.x, got.y, hi.x, hi.y) : make_uint4(lo.x, lo.y, got.x, got.y);
  r.col = odd ? 24u + 8u * (uint32_t)g : 8u * (uint32_t)g;
  return r;
}

// ---------------------------------------------------------------------------
// forward, LDS-staged gathers
// ---------------------------------------------------------------------------
// The gathered K and V rows of an item go to a wavefront-private LDS tile
// with direct-to-LDS 16-byte loads: eight consecutive lanes fetch the 128
// contiguous bytes of one slot's head pair, so every load instruction reads
// whole rows.  K is then read back in the MFMA A layout (ds_read_b128) and V
// transposed (ds_read_b64_tr_b16), which replaces the selection-matrix
// transposes.  Chunk c (16 bytes) of slot s sits at position c ^ F(s) with
// F(s) = (s & 15) >> 1, so that the 16 lanes of one K read hit 16 different
// bank groups.
constexpr int kSlotBytes = 2 * kRow;            // one slot: both heads of the pair
constexpr int kTileBytes = NK * kSlotBytes;     // 6 KiB per tensor
constexpr int kWaveLds = 2 * kTileBytes;        // K and V

// Position of an item (cluster bc of the batch, head pair hp), numbered
// item = bc * HP + hp; the forward steps it by a fixed stride without
// divisions after one initial division.
struct ItemPos {
  int bc, hp, cin, img;   // cluster (batch-wide), head pair, cluster in image, image base token
  __device__ void init(int item, int HP, int C, int N) {
    bc = item / HP;
    hp = item - bc * HP;
    const int b = bc / C;
    cin = bc - b * C;
    img = b * N;
  }
};


// LDS tile of one item's indices: ints 0..47 key tokens of the 48 slots,
// 48..55 the query tokens of the cluster, 56..63 unused (never written).
constexpr int kIdxBytes = 256;
// Wavefronts per workgroup: eight, i.e. four clusters with both head pairs
// (H=4) in one workgroup on one CU (LDS: one such workgroup per
// CU).  Against two per workgroup: high-res forward 84.0 -> 76.6 us,
// stage-1 23.8 -> 22.5 us, stage-3 unchanged.
constexpr int kFwdWaves = 8;
// Waves per CU the launch is sized for (one round over all 256 CUs); the
// measured optimum at the stage-1 shape.
constexpr int kFwdWavesPerCU = 8;
constexpr int kFwdWaveLds = 2 * kTileBytes + 1024 + kIdxBytes;

// One exec-masked 16-byte load with per-lane addresses: lanes 0..11 fetch
// the key_idx row of the cluster (ints 0..47 of the tile), lanes 12..13 its
// q_idx row (ints 48..55).  Counts as one vector-memory operation.
__device__ __forceinline__ void gather_idx(int bc, const int32_t* __restrict__ q_idx,
                                           const int32_t* __restrict__ key_idx, int lane,
                                           uint32_t lds) {
  if (lane < 14)
    dma16v(lane < 12 ? key_idx + (int64_t)bc * NK + 4 * lane : q_idx + (int64_t)bc * CS + 4 * (lane - 12),
           lds);
}

// Per-lane indices of one item, read from its LDS index tile.
struct FwdIdx2 {
  int tj[NK / 8];   // token of slot 8j + (lane >> 3)   (K/V gathers)
  int tq;           // query token (lane >> 3)          (Q gather)
  int tl;           // token of slot lane (lanes 48..63: slots 32..47)
  int qc;           // query token of column c16
};

__device__ __forceinline__ void read_idx(const char* t, int lane, FwdIdx2& x) {
  const int* ti = reinterpret_cast<const int*>(t);
#pragma unroll
  for (int j = 0; j < NK / 8; ++j) x.tj[j] = ti[8 * j + (lane >> 3)];
  x.tq = ti[NK + (lane >> 3)];
  x.tl = ti[lane < NK ? lane : lane - 16];
  x.qc = ti[NK + (lane & 7)];
}

// Byte offsets of one item's gathers.  Lane 8r + u fetches 16-byte chunk
// u ^ F(slot) of a slot row, which lands at chunk position u of the LDS
// tile: for slot 8j + r that is chunk u ^ F(8(j & 1) + r), so two column
// offsets per lane serve all six K/V instructions (K and V share the row
// offsets) and the query row r (F(r) = F(8 * 0 + r)).  With an odd head
// count the missing second head re-reads the first (never used).
struct FwdOffs {
  uint32_t kv[NK / 8];   // slot rows 8j + (lane >> 3)
  uint32_t qr;           // query row lane >> 3
};

// column offset (bytes within the token's row) of chunk position u of slot
// parity par, for the pair starting at head h0
__device__ __forceinline__ uint32_t chunk_col(int lane, int par, bool h1ok) {
  const uint32_t c = (uint32_t)(lane & 7) ^ swz(8 * par + (lane >> 3));
  return c < 4u ? 16u * c : (h1ok ? kRow : 0u) + 16u * (c - 4u);
}

__device__ __forceinline__ void item_offs(const FwdIdx2& x, int img, int h0, int H,
                                          uint32_t row_bytes, uint32_t col0, uint32_t col1,
                                          FwdOffs& o) {
  const uint32_t base = (uint32_t)(img * H + h0) * kRow;
#pragma unroll
  for (int j = 0; j < NK / 8; ++j)
    o.kv[j] = (uint32_t)__umul24((uint32_t)max(x.tj[j], 0), row_bytes) + base + ((j & 1) ? col1 : col0);
  o.qr = (uint32_t)__umul24((uint32_t)max(x.tq, 0), row_bytes) + base + col0;
}

// one tensor's 48 slot rows (both heads of the pair) into an LDS tile:
// instruction j fills slots 8j..8j+7
template <typename T>
__device__ __forceinline__ void gather_tile(const T* __restrict__ src, const FwdOffs& o,
                                            uint32_t lds_base) {
#pragma unroll
  for (int j = 0; j < NK / 8; ++j) dma16(src, o.kv[j], lds_base + (uint32_t)j * 1024u);
}

// Forward.  Each wavefront walks a run of `ipw` consecutive items (cluster,
// head pair) as a software pipeline in which every gather goes straight to
// LDS and every tile is refilled as soon as it has been consumed.  Memory
// operations are issued in this order in iteration t (vmcnt retires them in
// issue order):
//   idx(t+2) [1], K(t+1) [6], Q(t+1) [1], V(t+1) [6], O/LSE(t) stores [2]
// so at the top of iteration t, K(t), Q(t) and idx(t+1) are complete once
// at most V(t) + stores(t-1) = 8 newer operations remain, and V(t) is
// complete once at most stores(t-1) + idx(t+2) + K(t+1) = 9 remain.
template <typename T>
__global__ void __launch_bounds__(64 * kFwdWaves)
fwd_lds_kernel(int N, int C, int H, int HP, int n_items, int ipw, float scale_log2,
               const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
               const int32_t* __restrict__ q_idx, const int32_t* __restrict__ key_idx,
               T* __restrict__ o, float* __restrict__ lse) {
  __shared__ __attribute__((aligned(1024))) char lds[kFwdWaves * kFwdWaveLds];
  const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  // Items are dealt round-robin over the wavefronts (stride = all of them):
  // at any moment the wavefronts of one XCD work on one compact window of
  // consecutive clusters, whose gathered rows then stay in that XCD's L2.
  const int first = xcd_remap(blockIdx.x, gridDim.x) * kFwdWaves + wv;
  const int stride = gridDim.x * kFwdWaves;
  if (first >= n_items) return;
  (void)ipw;
  const int lane = threadIdx.x & 63;
  const int c16 = lane & 15, g = lane >> 4;
  const bool left = c16 < 8;
  char* tk = lds + wv * kFwdWaveLds;
  char* tv = tk + kTileBytes;
  char* tq = tv + kTileBytes;
  char* ti = tq + 1024;
  auto lds_addr = [](char* p) {
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)p;
  };
  const uint32_t ak = lds_addr(tk), av = lds_addr(tv), aq = lds_addr(tq), ai = lds_addr(ti);
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  const int e = c16 >> 2, qq = c16 & 3;
  const int CperImg = C;
  const bool neg = scale_log2 < 0.f;        // wave-uniform
  const float csl = fabsf(scale_log2);

  // Items are numbered item = bc * HP + hp: the head pairs of a cluster are
  // neighbouring items, so the wavefronts on one window read whole token
  // rows (all heads) at once rather than one head pair's half of each row
  // per pass over the batch (stage-3, 16 heads: 19.1 -> 18.1 us).
  // Positions advance by the fixed stride without divisions.
  const int st_bc = stride / HP, st_hp = stride - st_bc * HP;
  const int st_b = st_bc / CperImg, st_c = st_bc - st_b * CperImg;
  auto step = [&](ItemPos p) {
    p.hp += st_hp;
    int dbc = st_bc, dc = st_c;
    if (p.hp >= HP) {
      p.hp -= HP;
      ++dbc;
      ++dc;
    }
    p.bc += dbc;
    p.cin += dc;
    p.img += st_b * N;
    if (p.cin >= CperImg) {
      p.cin -= CperImg;
      p.img += N;
    }
    return p;
  };
  const uint32_t row_bytes = (uint32_t)H * kRow;   // one token, all heads
  // gather column offsets for a pair with / without a second head
  const uint32_t colA0 = chunk_col(lane, 0, true), colA1 = chunk_col(lane, 1, true);
  const uint32_t colB0 = chunk_col(lane, 0, false), colB1 = chunk_col(lane, 1, false);
  auto offs_of = [&](const FwdIdx2& x, const ItemPos& p, FwdOffs& o) {
    const bool two = 2 * p.hp + 1 < H;
    item_offs(x, p.img, 2 * p.hp, H, row_bytes, two ? colA0 : colB0, two ? colA1 : colB1, o);
  };

  // prologue: indices of `first`, then of `first + 1`, then the tiles of `first`
  ItemPos pc, pn, pnn;   // items it, it + stride, it + 2 * stride
  pc.init(first, HP, CperImg, N);
  pn = step(pc);
  pnn = step(pn);
  FwdIdx2 x, xn;
  FwdOffs ox, oxn;
  gather_idx(pc.bc, q_idx, key_idx, lane, ai);
  wait_vm<0>();
  read_idx(ti, lane, x);
  wait_lgkm0();
  if (first + stride < n_items) gather_idx(pn.bc, q_idx, key_idx, lane, ai);
  offs_of(x, pc, ox);
  gather_tile<T>(k, ox, ak);
  dma16_nt(q, ox.qr, aq);
  gather_tile<T>(v, ox, av);

  for (int it = first; it < n_items; it += stride) {
    const bool more = it + stride < n_items, more2 = it + 2 * stride < n_items;
    const bool prev = it > first;
    const int h0 = 2 * pc.hp, img = pc.img;
    const bool h1ok = h0 + 1 < H;
    const int hq = left ? h0 : h0 + 1;

    // K(t), Q(t) and idx(t+1) have landed
    if (prev) wait_vm<8>();
    else wait_vm<6>();
    if (more) {
      read_idx(ti, lane, xn);
      wait_lgkm0();
      if (more2) gather_idx(pnn.bc, q_idx, key_idx, lane, ai);
      offs_of(xn, pn, oxn);
    }

    // S^T = K Q^T: lane holds keys 16b+4g+i of column c16.  A negative scale
    // is applied as -|scale| with Q negated (exact), so that the row maximum
    // below is that of the scaled logits.
    const int qm = c16 & 7;
    uint4 qv = lds16(tq, (uint32_t)qm * kSlotBytes +
                             16u * ((uint32_t)((c16 >> 3) * 4 + g) ^ swz(qm)));
    if (neg) {
      qv.x ^= 0x80008000u;
      qv.y ^= 0x80008000u;
      qv.z ^= 0x80008000u;
      qv.w ^= 0x80008000u;
    }
    const uint4 qL = sel(left, qv), qR = sel(!left, qv);
    f32x4 s[3];
#pragma unroll
    for (int b = 0; b < 3; ++b) {
      const int sl = 16 * b + c16;
      const uint32_t row = (uint32_t)sl * kSlotBytes;
      const uint4 k0 = lds16(tk, row + 16u * ((uint32_t)g ^ swz(sl)));
      const uint4 k1 = lds16(tk, row + 16u * ((uint32_t)(4 + g) ^ swz(sl)));
      s[b] = Mfma<T>::mma(k0, qL, z);
      s[b] = Mfma<T>::mma(k1, qR, s[b]);
    }
    if (more) {   // K tile consumed: refill it for the next item
      wait_lgkm0();
      gather_tile<T>(k, oxn, ak);
    }

    // some slot of this list is empty: leave it out of the maximum, and
    // zero its probability below (exact for any finite scale, 0 included)
    const bool holes = __ballot(x.tl < 0) != 0ull;
    const uint64_t vb64 = __ballot(x.tl >= 0);
    if (holes) {
#pragma unroll
      for (int b = 0; b < 3; ++b) {
        const uint32_t vb = (uint32_t)(vb64 >> (16 * b));
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (!((vb >> (4 * g + i)) & 1u)) s[b][i] = -INFINITY;
      }
    }
    float mx = fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3]));
#pragma unroll
    for (int b = 1; b < 3; ++b)
      mx = fmaxf(mx, fmaxf(fmaxf(s[b][0], s[b][1]), fmaxf(s[b][2], s[b][3])));
    mx = shfl_max16_32(mx);
    const float mref = mx == -INFINITY ? 0.f : mx * csl;
    float p[3][4];
#pragma unroll
    for (int b = 0; b < 3; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) p[b][i] = __builtin_amdgcn_exp2f(fmaf(s[b][i], csl, -mref));
    if (holes) {
#pragma unroll
      for (int b = 0; b < 3; ++b) {
        const uint32_t vb = (uint32_t)(vb64 >> (16 * b));
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (!((vb >> (4 * g + i)) & 1u)) p[b][i] = 0.f;
      }
    }
    float l = 0.f;
#pragma unroll
    for (int b = 0; b < 3; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) l += p[b][i];
    l = shfl_sum16_32(l);
    uint2 ph[3];
#pragma unroll
    for (int b = 0; b < 3; ++b)
      ph[b] = make_uint2(pack2<T>(p[b][0], p[b][1]), pack2<T>(p[b][2], p[b][3]));
    const uint4 bp0 = cat(ph[0], ph[1]), bp1 = pad(ph[2]);

    // V(t) has landed
    if (prev && more2) wait_vm<9>();
    else wait_vm_n((prev ? 2 : 0) + (more2 ? 1 : 0) + (more ? 6 : 0));

    // O^T = V^T P^T per head.  Transposed read: lane c16 = 4e + qq of group g
    // addresses dims 16hf + 4qq.. of slot 16blk + 4g + e and receives dim
    // 16hf + c16 of the four slots 16blk + 4g + e, e = 0..3.
    f32x4 oacc[2][2] = {{z, z}, {z, z}};
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      if (hh == 1 && !h1ok) break;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        uint2 vt[3];
#pragma unroll
        for (int blk = 0; blk < 3; ++blk) {
          const int sl = 16 * blk + 4 * g + e;
          const uint32_t c = (uint32_t)(4 * hh + 2 * hf + (qq >> 1));
          vt[blk] = lds_tr8(tv, (uint32_t)sl * kSlotBytes + 16u * (c ^ swz(sl)) + 8u * (qq & 1));
        }
        oacc[hh][hf] = Mfma<T>::mma(cat(vt[0], vt[1]), bp0, oacc[hh][hf]);
        oacc[hh][hf] = Mfma<T>::mma(pad(vt[2]), bp1, oacc[hh][hf]);
      }
    }
    if (more) {   // Q and V tiles consumed: next item's
      wait_lgkm0();
      dma16_nt(q, oxn.qr, aq);
      gather_tile<T>(v, oxn, av);
    }

    // exactly two store instructions per item (the pipeline counts them);
    // 1/l through the hardware reciprocal (1 ulp)
    const float inv = l > 0.f ? __builtin_amdgcn_rcpf(l) : 0.f;
    const bool st = hq < H && x.qc >= 0;
    const uint32_t qrow = (uint32_t)__umul24((uint32_t)x.qc, (uint32_t)H) + (uint32_t)(img * H);
    const Row8 ov = row8(pack4<T>((left ? oacc[0][0] : oacc[1][0]) * inv),
                         pack4<T>((left ? oacc[0][1] : oacc[1][1]) * inv), g);
    if (st) stv<uint4>(o, (qrow + (uint32_t)hq) * kRow + ov.col, ov.v);
    if (st && g == 0)
      lse[qrow + hq] = l > 0.f ? (mref + __log2f(l)) * kLn2 : -INFINITY;
    x = xn;
    ox = oxn;
    pc = pn;
    pn = pnn;
    pnn = step(pnn);
  }
}

// (cluster of the batch, head pair, image, cluster in image) of an item
// numbered item = cluster * HP + pair, stepped by a fixed item stride
struct KvPos {
  int item, bj, hp, b, j;
};
struct KvStep {
  int s, s_bj, s_hp, s_b, s_j;
};
__device__ __forceinline__ KvPos kv_pos(int item, int HP, int C) {
  KvPos p;
  p.item = item;
  p.bj = item / HP;
  p.hp = item - p.bj * HP;
  p.b = p.bj / C;
  p.j = p.bj - p.b * C;
  return p;
}
__device__ __forceinline__ KvPos kv_next(KvPos p, const KvStep& st, int HP, int C) {
  p.item += st.s;
  p.hp += st.s_hp;
  p.bj += st.s_bj;
  p.j += st.s_j;
  p.b += st.s_b;
  if (p.hp >= HP) {
    p.hp -= HP;
    ++p.bj;
    ++p.j;
  }
  if (p.j >= C) {
    p.j -= C;
    ++p.b;
  }
  return p;
}

// ---------------------------------------------------------------------------
// backward pass A (query-major), LDS-staged gathers: Delta and dQ
// ---------------------------------------------------------------------------
// Per item (cluster, head pair), the 48 slot rows of K and V and the 8 query
// rows of Q and dO go to a wavefront-private LDS tile (direct-to-LDS loads,
// whole 128-byte rows).  S^T = K Q^T and dP^T = V dO^T read K and V in the A
// layout; dQ^T = K^T dS^T reads K through the transposing LDS read.  dS is
// rounded once to the operand type for that product.  Delta, the row sum of
// dO * O, equals the row sum of P * dP (O is the P-weighted sum of the V
// rows), so it is taken from the P and dP this pass computes anyway, in fp32
// before any rounding, and O is not read: a sixth of the pass's input bytes.
//
// Pipeline: at the top of item t every LDS operand of t is read into
// registers at once, which frees the tiles; the gathers of item t+1 are then
// issued and land while item t is computed from registers.  The index rows
// (key_idx and q_idx rows, as in the forward) run one item further ahead and
// the LSE values one item ahead, both through small LDS tiles, so that no
// register load crosses an iteration.  The two stores of an item are the
// last memory operations of its step: the wait at the top leaves exactly
// them in flight.
// four wavefronts per workgroup (two per workgroup: high-res backward
// 193.9 -> 183.3 us with four, stage-1 and stage-3 0.5-0.7 us faster)
constexpr int kQWaves = 4;
constexpr int kQWaveLds = 2 * kTileBytes + 2 * 1024 + kIdxBytes + 64;   // K, V, Q, dO, idx, LSE
constexpr int kQWavesPerCU = 8;

template <typename T>
__global__ void __launch_bounds__(64 * kQWaves)
bwd_q_lds_kernel(int N, int C, int H, int HP, int n_items, int ipw, float scale,
                 const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
                 const T* __restrict__ dout,
                 const float* __restrict__ lse, const int32_t* __restrict__ q_idx,
                 const int32_t* __restrict__ key_idx, T* __restrict__ dq,
                 float2* __restrict__ ld, float4* __restrict__ ld_none) {
  __shared__ __attribute__((aligned(1024))) char lds[kQWaves * kQWaveLds];
  // the (LSE*log2e, Delta) pair the key-major pass reads for an absent
  // query: P = exp2(s - inf) = 0 there (the first wait below covers it)
  if (blockIdx.x == 0 && threadIdx.x == 0) *ld_none = make_float4(INFINITY, 0.f, INFINITY, 0.f);
  const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  // items dealt round-robin over the wavefronts (see the forward)
  const int first = xcd_remap(blockIdx.x, gridDim.x) * kQWaves + wv;
  const int stride = gridDim.x * kQWaves;
  if (first >= n_items) return;
  (void)ipw;
  const int lane = threadIdx.x & 63;
  const int c16 = lane & 15, g = lane >> 4;
  const bool left = c16 < 8;
  char* tk = lds + wv * kQWaveLds;
  char* tv = tk + kTileBytes;
  char* tq = tv + kTileBytes;
  char* tdo = tq + 1024;
  char* ti = tdo + 1024;
  const float* tls = reinterpret_cast<const float*>(ti + kIdxBytes);
  auto lds_addr = [](const char* ptr) {
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)ptr;
  };
  const uint32_t ak = lds_addr(tk), av = lds_addr(tv), aq = lds_addr(tq), ado = lds_addr(tdo),
                 ai = lds_addr(ti), als = lds_addr(ti + kIdxBytes);
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  const int e = c16 >> 2, qq = c16 & 3;
  const float scale_log2 = scale * kLog2e;
  const uint32_t row_bytes = (uint32_t)H * kRow;   // one token, all heads
  const uint32_t colA0 = chunk_col(lane, 0, true), colA1 = chunk_col(lane, 1, true);
  const uint32_t colB0 = chunk_col(lane, 0, false), colB1 = chunk_col(lane, 1, false);

  KvStep st;
  st.s = stride;
  st.s_bj = stride / HP;
  st.s_hp = stride - st.s_bj * HP;
  st.s_b = st.s_bj / C;
  st.s_j = st.s_bj - st.s_b * C;
  // all gathers of an item (14 vector-memory operations)
  auto gather = [&](const KvPos& p, const FwdIdx2& x) {
    const bool two = 2 * p.hp + 1 < H;
    FwdOffs of;
    item_offs(x, p.b * N, 2 * p.hp, H, row_bytes, two ? colA0 : colB0, two ? colA1 : colB1, of);
    gather_tile<T>(k, of, ak);
    gather_tile<T>(v, of, av);
    dma16(q, of.qr, aq);
    dma16(dout, of.qr, ado);
  };
  // LSE of (query lane & 7, head h0 + (lane >> 3 & 1)) into the LSE tile
  // (lanes 0..15; one vector-memory operation)
  auto gather_lse = [&](const KvPos& p, const FwdIdx2& x) {
    if (lane < 16) {
      const int h = min(2 * p.hp + (lane >> 3), H - 1);
      dma4(lse, (uint32_t)((p.b * N + max(x.qc, 0)) * H + h) * 4u, als);
    }
  };

  // prologue: index rows of the first item, then its gathers and LSE, and
  // the index rows of the second
  KvPos pos = kv_pos(first, HP, C);
  KvPos pn = kv_next(pos, st, HP, C);
  FwdIdx2 x, xn;
  gather_idx(pos.bj, q_idx, key_idx, lane, ai);
  wait_vm<0>();
  read_idx(ti, lane, x);
  wait_lgkm0();
  gather(pos, x);
  gather_lse(pos, x);
  if (pn.item < n_items) gather_idx(pn.bj, q_idx, key_idx, lane, ai);

  for (;;) {
    const int h0 = 2 * pos.hp;
    const int img = pos.b * N;
    const bool h1ok = h0 + 1 < H;
    const int hq = left ? h0 : h0 + 1;
    const bool more = pn.item < n_items;
    const KvPos pnn = kv_next(pn, st, HP, C);

    // this item's gathers and LSE and the next item's index rows have
    // landed; the two stores of the previous item may still be in flight
    if (pos.item > first) wait_vm<2>();
    else wait_vm<0>();

    // every LDS operand of the item into registers
    const float lse2 = tls[c16] * kLog2e;   // (query c16 & 7, head hq)
    const int qm = c16 & 7;
    const uint32_t qoff = (uint32_t)qm * kSlotBytes +
                          16u * ((uint32_t)((c16 >> 3) * 4 + g) ^ swz(qm));
    const uint4 qv = lds16(tq, qoff), dov = lds16(tdo, qoff);
    uint4 k0[3], k1[3], v0[3], v1[3];
#pragma unroll
    for (int b = 0; b < 3; ++b) {
      const int sl = 16 * b + c16;
      const uint32_t row = (uint32_t)sl * kSlotBytes;
      k0[b] = lds16(tk, row + 16u * ((uint32_t)g ^ swz(sl)));
      k1[b] = lds16(tk, row + 16u * ((uint32_t)(4 + g) ^ swz(sl)));
      v0[b] = lds16(tv, row + 16u * ((uint32_t)g ^ swz(sl)));
      v1[b] = lds16(tv, row + 16u * ((uint32_t)(4 + g) ^ swz(sl)));
    }
    // K^T for dQ^T = K^T dS^T (transposed reads, as V in the forward)
    uint2 kt[2][2][3];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int blk = 0; blk < 3; ++blk) {
          const int sl = 16 * blk + 4 * g + e;
          const uint32_t c = (uint32_t)(4 * hh + 2 * hf + (qq >> 1));
          kt[hh][hf][blk] = lds_tr8(tk, (uint32_t)sl * kSlotBytes + 16u * (c ^ swz(sl)) + 8u * (qq & 1));
        }
    if (more) read_idx(ti, lane, xn);
    wait_lgkm0();

    // next item's gathers and LSE, and the index rows of the one after
    if (more) {
      gather(pn, xn);
      gather_lse(pn, xn);
      if (pnn.item < n_items) gather_idx(pnn.bj, q_idx, key_idx, lane, ai);
    }

    const uint4 qL = sel(left, qv), qR = sel(!left, qv);
    const uint4 dL = sel(left, dov), dR = sel(!left, dov);
    float p[3][4], dpv[3][4];
#pragma unroll
    for (int b = 0; b < 3; ++b) {
      f32x4 sv = Mfma<T>::mma(k0[b], qL, z);
      sv = Mfma<T>::mma(k1[b], qR, sv);
      f32x4 dp = Mfma<T>::mma(v0[b], dL, z);
      dp = Mfma<T>::mma(v1[b], dR, dp);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[b][i] = __builtin_amdgcn_exp2f(fmaf(sv[i], scale_log2, -lse2));
        dpv[b][i] = dp[i];
      }
    }
    if (__ballot(x.tl < 0) != 0ull) {   // empty slots of this list: P = 0 there
      const uint64_t vb64 = __ballot(x.tl >= 0);
#pragma unroll
      for (int b = 0; b < 3; ++b) {
        const uint32_t vb = (uint32_t)(vb64 >> (16 * b));
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (!((vb >> (4 * g + i)) & 1u)) p[b][i] = 0.f;
      }
    }
    // Delta of (query c16 & 7, head hq) = sum over the slots of P * dP
    float dl = 0.f;
#pragma unroll
    for (int b = 0; b < 3; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) dl = fmaf(p[b][i], dpv[b][i], dl);
    dl = shfl_sum16_32(dl);
    float ds[3][4];
#pragma unroll
    for (int b = 0; b < 3; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) ds[b][i] = p[b][i] * (dpv[b][i] - dl);
    uint2 dh[3];
#pragma unroll
    for (int b = 0; b < 3; ++b)
      dh[b] = make_uint2(pack2<T>(ds[b][0], ds[b][1]), pack2<T>(ds[b][2], ds[b][3]));
    const uint4 b0h = cat(dh[0], dh[1]), b1h = pad(dh[2]);

    f32x4 acc[2][2] = {{z, z}, {z, z}};
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      if (hh == 1 && !h1ok) break;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        acc[hh][hf] = Mfma<T>::mma(cat(kt[hh][hf][0], kt[hh][hf][1]), b0h, acc[hh][hf]);
        acc[hh][hf] = Mfma<T>::mma(pad(kt[hh][hf][2]), b1h, acc[hh][hf]);
      }
    }
    // exactly two store instructions per item (lane 0, member 0 of the
    // cluster, always stores)
    const uint32_t qrow = (uint32_t)__umul24((uint32_t)x.qc, (uint32_t)H) + (uint32_t)(img * H);
    const bool live = hq < H && x.qc >= 0;
    const Row8 dv8 = row8(pack4<T>((left ? acc[0][0] : acc[1][0]) * scale),
                          pack4<T>((left ? acc[0][1] : acc[1][1]) * scale), g);
    if (live && g == 0) ld[qrow + hq] = make_float2(lse2, dl);
    if (live) st16_nt(dq, (qrow + (uint32_t)hq) * kRow + dv8.col, dv8.v);
    if (!more) break;
    pos = pn;
    pn = pnn;
    x = xn;
  }
}

// ---------------------------------------------------------------------------
// backward pass B (key-major), LDS-staged gathers
// ---------------------------------------------------------------------------
// One wavefront per (key cluster j, head pair).  The entries of j (query
// clusters i reading j, with per-member multiplicities and the query tokens
// of i) are taken four at a time: their 32 query rows of Q and dO (both
// heads) are gathered into a wavefront-private LDS tile with direct-to-LDS
// loads (instruction u holds entry u's 8 rows).  S = Q K_j^T and
// dP = dO V_j^T read Q and dO in the MFMA A layout; dV^T += dO^T P and
// dK^T += Q^T dS read them transposed (ds_read_b64_tr_b16).  One accumulator
// set per head, so no operand needs zeroed columns.  Summation order is
// fixed by the entry order (sorted by i), so the result is bitwise
// reproducible.  A multiplicity m enters as exp2(s - LSE + log2 m), which is
// 0 for an entry past the end of a list (m = 0).
//
// The per-item lookups are prefetched one item ahead: when item t starts,
// the query tokens and multiplicities of the first eight entries of item
// t+1 go to a wavefront-private LDS block (direct-to-LDS loads; two blocks
// alternate), its own K/V rows and the segment bounds and key tokens of item
// t+2 are requested, all ahead of item t's first gathers, so that one wait
// per four entries covers them.  Loads for later items use clamped (always
// valid) addresses.  Item positions advance by the fixed stride without
// divisions.
constexpr int kKvRows = 32;                             // query rows per step
constexpr int kKvTile = kKvRows * kSlotBytes;           // 4 KiB per tensor
constexpr int kKvMeta = 2 * (64 * 4 + 8 * 8);           // two blocks of 8 entries' tokens, mults
constexpr int kKvWaveLds = 2 * kKvTile + kKvMeta;       // Q, dO, entry blocks
constexpr int kKvWavesPerCU = 16;                       // residency (VGPRs and LDS)

template <typename T>
__global__ void __launch_bounds__(64 * kWaves, kKvWavesPerCU / 4)
bwd_kv_lds_kernel(int N, int C, int H, int HP, int n_items, float scale, const T* __restrict__ q,
                  const T* __restrict__ k, const T* __restrict__ v, const T* __restrict__ dout,
                  const int32_t* __restrict__ q_idx, const float2* __restrict__ ld,
                  uint32_t ld_none,
                  const int2* __restrict__ seg_all, const RevEntry* __restrict__ rev_all,
                  const int32_t* __restrict__ rtok_all, int nk, T* __restrict__ dk,
                  T* __restrict__ dv) {
  __shared__ __attribute__((aligned(1024))) char lds[kWaves * kKvWaveLds];
  // (LSE*log2e, Delta) of both heads of the 32 query rows of a step
  __shared__ __attribute__((aligned(16))) float4 lds_ld[kWaves][32];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  // items dealt round-robin over the wavefronts (see the forward)
  const int first = xcd_remap(blockIdx.x, gridDim.x) * kWaves + wv;
  const int stride = gridDim.x * kWaves;
  if (first >= n_items) return;
  char* tq = lds + wv * kKvWaveLds;
  char* td = tq + kKvTile;
  char* tm = td + kKvTile;   // [2] x {int tok[64]; uint64 mult[8]}
  auto lds_addr = [](const void* ptr) {
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)ptr;
  };
  const uint32_t aq = lds_addr(tq), ad = lds_addr(td), am = lds_addr(tm);
  const float2* tl2 = reinterpret_cast<const float2*>(lds_ld[wv]);
  const uint32_t al = lds_addr(lds_ld[wv]);
  const int c16 = lane & 15, g = lane >> 4;
  const bool left = c16 < 8;
  const int kcol = c16 & 7;
  const int e = c16 >> 2, qq = c16 & 3;
  const int r8 = lane >> 3, u8 = lane & 7;
  const float scale_log2 = scale * kLog2e;
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  const uint32_t row_bytes = (uint32_t)H * kRow;   // one token, all heads

  KvStep st;
  st.s = stride;
  st.s_bj = stride / HP;
  st.s_hp = stride - st.s_bj * HP;
  st.s_b = st.s_bj / C;
  st.s_j = st.s_bj - st.s_b * C;

  // Segment bounds of an item as a vector load (every lane the same 8 bytes):
  // a scalar load would make every later LDS wait (lgkmcnt) wait for it too.
  // Its value is first used one item later, when the load is long complete.
  int vzero;
  asm volatile("v_mov_b32 %0, 0" : "=v"(vzero));
  auto seg_of = [&](const KvPos& p) {
    const int x = p.item < n_items ? p.bj : 0;
    return seg_all[x + vzero];
  };
  // absolute entry range [e0, e1) of an item (indices into rev / rtok)
  auto bounds = [&](const KvPos& p, int2 sg, int& e0, int& e1) {
    e0 = p.item < n_items ? __builtin_amdgcn_readfirstlane(sg.x) : 0;
    e1 = p.item < n_items ? __builtin_amdgcn_readfirstlane(sg.y) : 0;
  };
  // block of entries [x0, x0 + 8) (clamped to [x0, x1)) into LDS block `blk`:
  // int 8u + r = token of member r of entry u, uint64 u = its multiplicities
  // (two vector-memory operations)
  auto load_block = [&](int x0, int x1, int blk) {
    const uint32_t base = am + (uint32_t)blk * (kKvMeta / 2);
    const int xt = min(x0 + r8, x1 - 1);
    dma4(rtok_all, (uint32_t)((x1 > x0 ? xt : 0) * 8 + u8) * 4u, base);
    if (lane < 16) {
      const int xm = min(x0 + (lane >> 1), x1 - 1);
      dma4(rev_all, (uint32_t)(x1 > x0 ? xm : 0) * 16u + 8u + 4u * (lane & 1), base + 256u);
    }
  };
  auto key_row = [&](const KvPos& p, int ktok) {
    const int h0 = 2 * p.hp;
    const uint32_t h1off = h0 + 1 < H ? kRow : 0u;
    return (uint32_t)((p.b * N + max(ktok, 0)) * H + h0) * kRow + (left ? 0u : h1off) + 16u * g;
  };

  // prologue: item `first` and the lookups of the next two
  KvPos cur = kv_pos(first, HP, C);
  KvPos nx = kv_next(cur, st, HP, C);
  int e0, e1;
  bounds(cur, seg_of(cur), e0, e1);
  int2 sgn = seg_of(nx);
  int ktok = q_idx[cur.bj * CS + kcol];
  int ktok_n = q_idx[(nx.item < n_items ? nx.bj : cur.bj) * CS + kcol];
  uint4 kB = ld16(k, key_row(cur, ktok)), vB = ld16(v, key_row(cur, ktok));
  load_block(e0, e1, 0);
  wait_vm<0>();
  int blk = 0;

  for (;;) {
    const int h0 = 2 * cur.hp;
    const bool h1ok = h0 + 1 < H;
    const int hk = left ? h0 : h0 + 1;
    const uint32_t h1off = h1ok ? kRow : 0u;
    const int img = cur.b * N;

    // prefetch: next item (entry block, own K/V rows) and the one after
    // (segment bounds, key tokens)
    const KvPos nxx = kv_next(nx, st, HP, C);
    int e0n, e1n;
    bounds(nx, sgn, e0n, e1n);
    const int2 sgnn = seg_of(nxx);
    const int ktok_nn = q_idx[(nxx.item < n_items ? nxx.bj : cur.bj) * CS + kcol];
    load_block(e0n, e1n, blk ^ 1);
    const uint32_t krn = key_row(nx.item < n_items ? nx : cur, ktok_n);
    const uint4 kBn = ld16(k, krn), vBn = ld16(v, krn);

    const uint4 kL = sel(left, kB), kR = sel(!left, kB);
    const uint4 vL = sel(left, vB), vR = sel(!left, vB);
    // gather byte offsets: row of token t = t * row_bytes + gb[u & 1] for
    // instruction u (lane 8r + u8 fetches chunk u8 ^ F(8u + r) of its row)
    uint32_t gb[2];
#pragma unroll
    for (int par = 0; par < 2; ++par) {
      const uint32_t c = (uint32_t)u8 ^ swz(8 * par + r8);
      gb[par] = (uint32_t)(img * H + h0) * kRow + (c < 4u ? 16u * c : h1off + 16u * (c - 4u));
    }
    const uint32_t lb = (uint32_t)(img * H + h0) * 8u;
    f32x4 dka[2][2] = {{z, z}, {z, z}}, dva[2][2] = {{z, z}, {z, z}};   // [head][dim half]
    const int* btok = reinterpret_cast<const int*>(tm + blk * (kKvMeta / 2));
    const uint8_t* bmul = reinterpret_cast<const uint8_t*>(tm + blk * (kKvMeta / 2) + 256);

    for (int eb = e0; eb < e1; eb += 8) {
      const int ne = min(8, e1 - eb);
      if (eb > e0) {   // lists with more than eight entries: not prefetched
        load_block(eb, e1, blk);
        wait_vm<0>();
      }
      // A step takes four entries (32 query rows), or two (16 rows, one
      // MFMA row block) when at most two remain, so that a list of 4n + 2
      // entries carries no padding; the half step feeds zeros for the upper
      // 16 rows of the dK/dV products.
      for (int e4 = 0; e4 < ne; e4 += 4) {
        const bool half = ne - e4 <= 2;   // wave-uniform
        // gathers: instruction u holds entry e4 + u (an entry past the end
        // repeats the last one, with zero multiplicity); all offsets first,
        // then the loads (each load's asm block orders every LDS operation
        // before it)
        {
          uint32_t offs[4];
#pragma unroll
          for (int u = 0; u < 4; ++u)
            offs[u] = (uint32_t)max(btok[8 * min(e4 + u, ne - 1) + r8], 0) * row_bytes + gb[u & 1];
          const int lrow = lane & 31;
          const int tl_tok = btok[8 * min(e4 + (lrow >> 3), ne - 1) + (lrow & 7)];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            if (u == 2 && half) break;
            dma16(q, offs[u], aq + (uint32_t)u * 1024u);
            dma16(dout, offs[u], ad + (uint32_t)u * 1024u);
          }
          // (LSE*log2e, Delta) of both heads of query row `lane` (lanes < 32,
          // rows 16..31 only in a full step): 16 bytes at
          // ld[(img + t) * H + h0].  With an odd head count the second pair
          // belongs to the next token (or lies in the next workspace part);
          // it is never used then.  An absent query (-1) reads the
          // (+inf, 0) pairs at byte offset ld_none instead.
          const uint32_t lo_ = tl_tok >= 0 ? (uint32_t)tl_tok * (uint32_t)H * 8u + lb : ld_none;
          if (lane < (half ? 16 : 32)) dma16(ld, lo_, al);
        }
        // log2 of the multiplicity of this lane's output rows 4g+i of block
        // qb (entry e4 + 2qb + (g >> 1), key member kcol): -inf for 0
        float lm[2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const int ee = e4 + 2 * qb + (g >> 1);
          const float m = ee < ne ? (float)bmul[8 * min(ee, 7) + kcol] : 0.f;
          lm[qb] = __builtin_amdgcn_logf(m);
        }
        wait_vm<0>();

        uint2 ph[2] = {make_uint2(0u, 0u), make_uint2(0u, 0u)}, dh[2] = {ph[0], ph[1]};
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          if (qb == 1 && half) break;
          const int row = 16 * qb + c16;
          const uint32_t rb = (uint32_t)row * kSlotBytes;
          const uint4 q0 = lds16(tq, rb + 16u * ((uint32_t)g ^ swz(row)));
          const uint4 q1 = lds16(tq, rb + 16u * ((uint32_t)(4 + g) ^ swz(row)));
          const uint4 d0 = lds16(td, rb + 16u * ((uint32_t)g ^ swz(row)));
          const uint4 d1 = lds16(td, rb + 16u * ((uint32_t)(4 + g) ^ swz(row)));
          f32x4 sv = Mfma<T>::mma(q0, kL, z);
          sv = Mfma<T>::mma(q1, kR, sv);
          f32x4 dp = Mfma<T>::mma(d0, vL, z);
          dp = Mfma<T>::mma(d1, vR, dp);
          float p[4], ds[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            // (LSE*log2e, Delta) of row 16qb + 4g + i, head hk
            const float2 lv = tl2[2 * (16 * qb + 4 * g + i) + (left ? 0 : 1)];
            p[i] = __builtin_amdgcn_exp2f(fmaf(sv[i], scale_log2, lm[qb] - lv.x));
            ds[i] = p[i] * (dp[i] - lv.y);
          }
          ph[qb] = make_uint2(pack2<T>(p[0], p[1]), pack2<T>(p[2], p[3]));
          dh[qb] = make_uint2(pack2<T>(ds[0], ds[1]), pack2<T>(ds[2], ds[3]));
        }
        const uint4 bph = cat(ph[0], ph[1]), bdh = cat(dh[0], dh[1]);
        // transposed reads: lane c16 = 4e + qq of group g receives dim
        // 16hf + c16 of query rows 16qb + 4g + e, e = 0..3
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          if (hh == 1 && !h1ok) break;
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
            uint2 at_d[2] = {make_uint2(0u, 0u), make_uint2(0u, 0u)}, at_q[2] = {at_d[0], at_d[1]};
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
              if (qb == 1 && half) break;
              const int row = 16 * qb + 4 * g + e;
              const uint32_t c = (uint32_t)(4 * hh + 2 * hf + (qq >> 1));
              const uint32_t o = (uint32_t)row * kSlotBytes + 16u * (c ^ swz(row)) + 8u * (qq & 1);
              at_d[qb] = lds_tr8(td, o);
              at_q[qb] = lds_tr8(tq, o);
            }
            const uint4 ad4 = cat(at_d[0], at_d[1]), aq4 = cat(at_q[0], at_q[1]);
            dva[hh][hf] = Mfma<T>::mma(ad4, bph, dva[hh][hf]);
            dka[hh][hf] = Mfma<T>::mma(aq4, bdh, dka[hh][hf]);
          }
        }
        // the tiles are rewritten next step: all reads above must be complete
        wait_lgkm0();
      }
    }

    {
      const Row8 k8 = row8(pack4<T>((left ? dka[0][0] : dka[1][0]) * scale),
                           pack4<T>((left ? dka[0][1] : dka[1][1]) * scale), g);
      const Row8 v8 = row8(pack4<T>(left ? dva[0][0] : dva[1][0]),
                           pack4<T>(left ? dva[0][1] : dva[1][1]), g);
      if (hk < H && ktok >= 0) {   // -1: absent member of a partial key cluster
        const uint32_t orow = (uint32_t)((img + ktok) * H + hk) * kRow;
        st16_nt(dk, orow + k8.col, k8.v);
        st16_nt(dv, orow + v8.col, v8.v);
      }
    }
    if (nx.item >= n_items) break;
    cur = nx;
    nx = nxx;
    e0 = e0n;
    e1 = e1n;
    sgn = sgnn;
    ktok = ktok_n;
    ktok_n = ktok_nn;
    kB = kBn;
    vB = vBn;
    blk ^= 1;
  }
}

// Items per wavefront: enough wavefronts to give every SIMD of the 256 CUs
// about four, each pipelining its run of consecutive items.
// Items per wavefront for a kernel of which `per_cu` waves fit on a CU at
// once: just enough waves to fill all 256 CUs in one round.
int items_per_wave(int items, int per_cu) {
  const int target = 256 * per_cu;
  return std::max(1, std::min(16, (items + target - 1) / target));
}

template <typename T>
hipError_t fwd_t(int B, int N, int C, int H, float scale, const void* q, const void* k,
                 const void* v, const int32_t* q_idx, const int32_t* key_idx, void* o, float* lse,
                 hipStream_t st) {
  const int HP = (H + 1) / 2;
  const int items = B * C * HP;
  const int ipw = items_per_wave(items, kFwdWavesPerCU);
  const int waves = (items + ipw - 1) / ipw;
  const int wgs = (waves + kFwdWaves - 1) / kFwdWaves;
  hipLaunchKernelGGL((fwd_lds_kernel<T>), dim3(wgs), dim3(64 * kFwdWaves), 0, st, N, C, H, HP,
                     items, ipw, scale * kLog2e, (const T*)q, (const T*)k, (const T*)v, q_idx,
                     key_idx, (T*)o, lse);
  return hipGetLastError();
}

template <typename T>
hipError_t bwd_t(int pass, int B, int N, int C, int H, int nk, float scale, const void* q,
                 const void* k, const void* v, const void* o, const void* dout, const float* lse,
                 const int32_t* q_idx, const int32_t* key_idx, void* dq, void* dk, void* dv,
                 const BwdWorkspace& w, hipStream_t st) {
  (void)o;   // pass A takes Delta from P and dP; O is not read
  const int HP = (H + 1) / 2;
  const int items = B * C * HP;
  const int kv_waves = std::min(items, 256 * kKvWavesPerCU);
  const int kv_wgs = (kv_waves + kWaves - 1) / kWaves;
  if (pass & 1) {
    const int ipw = items_per_wave(items, kQWavesPerCU);
    const int waves = (items + ipw - 1) / ipw;
    hipLaunchKernelGGL((bwd_q_lds_kernel<T>), dim3((waves + kQWaves - 1) / kQWaves),
                       dim3(64 * kQWaves), 0, st, N, C, H, HP, items, ipw, scale, (const T*)q,
                       (const T*)k, (const T*)v, (const T*)dout, lse, q_idx, key_idx,
                       (T*)dq, w.ld, w.ld_none);
  }
  if (pass & 2) {
    const uint32_t ld_none = (uint32_t)((const char*)w.ld_none - (const char*)w.ld);
    hipLaunchKernelGGL((bwd_kv_lds_kernel<T>), dim3(kv_wgs), dim3(64 * kWaves), 0, st, N, C, H, HP,
                       items, scale, (const T*)q, (const T*)k, (const T*)v, (const T*)dout, q_idx,
                       (const float2*)w.ld, ld_none, (const int2*)w.seg,
                       (const RevEntry*)w.rev, (const int32_t*)w.rtok, nk, (T*)dk, (T*)dv);
  }
  return hipGetLastError();
}

}  // namespace

bool mfma_supported(int dt, int B, int N, int C, int H, int nk) {
  // 32-bit byte offsets (the workspace's LSE/Delta pairs included) and item counts
  const int64_t bytes = (int64_t)B * N * H * D * 2;
  const int64_t items = (int64_t)B * C * ((H + 1) / 2);
  return (dt == 1 || dt == 2) && nk == NK && bytes < (int64_t(1) << 31) &&
         items < (int64_t(1) << 30);
}

hipError_t launch_fwd_mfma(int dt, int B, int N, int C, int H, float scale, const void* q,
                           const void* k, const void* v, const int32_t* q_idx,
                           const int32_t* key_idx, void* o, float* lse, hipStream_t st) {
  if (dt == 1) return fwd_t<bf16>(B, N, C, H, scale, q, k, v, q_idx, key_idx, o, lse, st);
  if (dt == 2) return fwd_t<f16>(B, N, C, H, scale, q, k, v, q_idx, key_idx, o, lse, st);
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_mfma(int pass, int dt, int B, int N, int C, int H, int nk, float scale,
                           const void* q, const void* k, const void* v, const void* o,
                           const void* dout, const float* lse, const int32_t* q_idx,
                           const int32_t* key_idx, void* dq, void* dk, void* dv,
                           const BwdWorkspace& w, hipStream_t st) {
  if (dt == 1)
    return bwd_t<bf16>(pass, B, N, C, H, nk, scale, q, k, v, o, dout, lse, q_idx, key_idx, dq,
                       dk, dv, w, st);
  if (dt == 2)
    return bwd_t<f16>(pass, B, N, C, H, nk, scale, q, k, v, o, dout, lse, q_idx, key_idx, dq,
                      dk, dv, w, st);
  return hipErrorInvalidValue;
}

}  // namespace ca
