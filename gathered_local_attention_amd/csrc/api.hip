// C ABI of libclusterattn: argument validation and dispatch.
// Every entry point validates synchronously (no HIP call before validation
// has passed, so the checks also run on a machine without a GPU), then
// enqueues its kernels on the caller's stream and returns.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <new>

#include "../../include/cluster_attn.h"
#include "common.h"

namespace {

thread_local char g_last_error[512] = "";

ca_status fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return (ca_status)status;
}

ca_status ok() {
  g_last_error[0] = '\0';
  return CA_OK;
}

ca_status hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return ok();
  return fail(CA_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

size_t elem_size(int dt) { return dt == CA_F32 ? 4 : 2; }

struct Range {
  const void* p;
  size_t n;
};

bool overlaps(Range a, Range b) {
  if (!a.p || !b.p || a.n == 0 || b.n == 0) return false;
  const uintptr_t a0 = (uintptr_t)a.p, a1 = a0 + a.n;
  const uintptr_t b0 = (uintptr_t)b.p, b1 = b0 + b.n;
  return a0 < b1 && b0 < a1;
}

// outputs must not overlap each other or any input
ca_status check_alias(const Range* outs, int nout, const Range* ins, int nin) {
  for (int i = 0; i < nout; ++i) {
    for (int j = 0; j < nin; ++j)
      if (overlaps(outs[i], ins[j])) return fail(CA_ERR_ALIAS, "output %d overlaps input %d", i, j);
    for (int j = i + 1; j < nout; ++j)
      if (overlaps(outs[i], outs[j])) return fail(CA_ERR_ALIAS, "outputs %d and %d overlap", i, j);
  }
  return CA_OK;
}

using ca::kMaxTokensPerImage;   // 2^22: cluster ids of a (distance, index) key fit 19 bits

// Shape checks common to fwd and bwd.  Returns CA_OK or an error.
ca_status check_attn_shape(int dt, int B, int N, int H, int D, int cs, int nk) {
  if (dt != CA_F32 && dt != CA_BF16 && dt != CA_F16)
    return fail(CA_ERR_UNSUPPORTED, "dtype %d is not one of CA_F32, CA_BF16, CA_F16", dt);
  if (B < 0 || N < 0 || H < 1 || D < 1 || cs < 1 || nk < 1)
    return fail(CA_ERR_SHAPE, "bad sizes B=%d N=%d H=%d D=%d cs=%d nk=%d", B, N, H, D, cs, nk);
  if (cs != 8) return fail(CA_ERR_UNSUPPORTED, "cluster size %d (only 8 is supported)", cs);
  if (D != 32) return fail(CA_ERR_UNSUPPORTED, "head dim %d (only 32 is supported)", D);
  if (nk % cs != 0 || nk / cs > 8)
    return fail(CA_ERR_UNSUPPORTED, "nk=%d must be cs*k with 1 <= k <= 8", nk);
  if ((int64_t)B * N * H * D > (int64_t(1) << 40)) return fail(CA_ERR_SHAPE, "tensor too large");
  if ((int64_t)B * N > (int64_t(1) << 31) - 1) return fail(CA_ERR_SHAPE, "B*N above 2^31 - 1");
  return CA_OK;
}

int64_t clusters_of(int64_t N, int cs) { return (N + cs - 1) / cs; }


// Shape checks of the KNN sampler calls.
ca_status check_knn_shape(int B, int N, int M, int Cf, int G, int K) {
  if (B < 0 || N < 0 || M < 0) return fail(CA_ERR_SHAPE, "bad sizes B=%d N=%d M=%d", B, N, M);
  if (G < 1 || G > 2048) return fail(CA_ERR_SHAPE, "grid_side=%d outside [1, 2048]", G);
  if (K < 1 || K > 16) return fail(CA_ERR_UNSUPPORTED, "K=%d outside 1..16", K);
  if (Cf < 8 || Cf > 1024 || Cf % 8 != 0)
    return fail(CA_ERR_UNSUPPORTED, "channels %d: must be a multiple of 8 in [8, 1024]", Cf);
  if (N > (1 << 24) || M > (1 << 24)) return fail(CA_ERR_SHAPE, "N or M above 2^24");
  if ((int64_t)B * M * K > (int64_t(1) << 31) - 1 || (int64_t)M * K > (int64_t(1) << 31) - 1)
    return fail(CA_ERR_SHAPE, "B*M*K too large");
  return CA_OK;
}


ca_status check_merge_shape(int dt, int B, int N, int k, int C) {
  if (dt != CA_F32 && dt != CA_BF16 && dt != CA_F16)
    return fail(CA_ERR_UNSUPPORTED, "dtype %d is not one of CA_F32, CA_BF16, CA_F16", dt);
  if (B < 0 || N < 0 || k < 0) return fail(CA_ERR_SHAPE, "bad sizes B=%d N=%d k=%d", B, N, k);
  if (N > (1 << 24)) return fail(CA_ERR_SHAPE, "N=%d above 2^24", N);
  if ((int64_t)B * N > (int64_t(1) << 31) - 1) return fail(CA_ERR_SHAPE, "B*N above 2^31 - 1");
  if (k > N || (N > 0 && k < 1)) return fail(CA_ERR_SHAPE, "k=%d must be in [1, N=%d]", k, N);
  if (C < 8 || C > 1024 || C % 8 != 0)
    return fail(CA_ERR_UNSUPPORTED, "channels %d: must be a multiple of 8 in [8, 1024]", C);
  return CA_OK;
}

}  // namespace

extern "C" {

const char* cluster_attn_version(void) { return "clusterattn 0.1 (gfx950)"; }

const char* cluster_attn_status_string(int s) {
  switch (s) {
    case CA_OK: return "CA_OK";
    case CA_ERR_NULL: return "CA_ERR_NULL: a required pointer is NULL";
    case CA_ERR_SHAPE: return "CA_ERR_SHAPE: sizes out of range or inconsistent";
    case CA_ERR_UNSUPPORTED: return "CA_ERR_UNSUPPORTED: request outside the supported set";
    case CA_ERR_WORKSPACE: return "CA_ERR_WORKSPACE: workspace too small";
    case CA_ERR_ALIAS: return "CA_ERR_ALIAS: an output overlaps an input or another output";
    case CA_ERR_HIP: return "CA_ERR_HIP: the HIP runtime reported an error";
  }
  return "unknown status";
}

const char* cluster_attn_last_error(void) { return g_last_error; }

size_t cluster_attn_build_neighbors_workspace(int B, int N, int cs, int k) {
  if (B < 0 || N < 0 || cs != 8 || k < 1 || k > 8 || N > kMaxTokensPerImage) return 0;
  return ca::build_layout(nullptr, B, (int64_t)B * N, B * clusters_of(N, cs), N).bytes;
}

size_t cluster_attn_build_neighbors_varlen_workspace(int B, int T, int Ct, int max_n, int cs,
                                                     int k) {
  if (B < 0 || T < 0 || Ct < 0 || max_n < 0 || max_n > T || cs != 8 || k < 1 || k > 8 ||
      max_n > kMaxTokensPerImage)
    return 0;
  return ca::build_layout(nullptr, B, T, Ct, max_n).bytes;
}

}  // extern "C"

namespace {

// Equal-size images: coords [B, N, dims].
ca_status build_uniform(int dims, const float* coords, int B, int N, int grid_side, int cs, int k,
                  int32_t* perm, int32_t* nbr, int32_t* key_idx, void* ws, size_t ws_bytes,
                  void* hip_stream) {
  if (B < 0 || N < 0) return fail(CA_ERR_SHAPE, "bad sizes B=%d N=%d", B, N);
  if (cs != 8) return fail(CA_ERR_UNSUPPORTED, "cluster size %d (only 8 is supported)", cs);
  if (k < 1 || k > 8) return fail(CA_ERR_UNSUPPORTED, "k=%d outside 1..8", k);
  if (N > kMaxTokensPerImage) return fail(CA_ERR_SHAPE, "N=%d exceeds 2^22 tokens per image", N);
  if ((int64_t)B * N > (int64_t(1) << 31) - 1) return fail(CA_ERR_SHAPE, "B*N above 2^31 - 1");
  const int gmax = dims == 2 ? 65536 : 16384;
  if (grid_side < 1 || grid_side > gmax)
    return fail(CA_ERR_SHAPE, "grid_side=%d outside [1, %d]", grid_side, gmax);
  if (B == 0 || N == 0) return ok();
  if (!coords || !perm || !nbr || !key_idx) return fail(CA_ERR_NULL, "NULL tensor pointer");
  const int64_t C = clusters_of(N, cs);
  const size_t need = ca::build_layout(nullptr, B, (int64_t)B * N, B * C, N).bytes;
  if (need && !ws) return fail(CA_ERR_NULL, "NULL workspace (%zu bytes needed)", need);
  if (ws_bytes < need) return fail(CA_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  Range outs[] = {{perm, (size_t)(B * C * cs) * 4}, {nbr, (size_t)(B * C * k) * 4},
                  {key_idx, (size_t)(B * C * k * cs) * 4}, {ws, need}};
  Range ins[] = {{coords, (size_t)B * N * 4 * dims}};
  if (ca_status s = check_alias(outs, 4, ins, 1)) return s;
  const ca::Geom g{nullptr, nullptr, N, (int)C, 0};
  return hip_status(ca::launch_build_neighbors(coords, g, dims, B, (int64_t)B * N, B * C, grid_side,
                                               k, perm, nbr, key_idx, ws, (hipStream_t)hip_stream),
                    "build_neighbors launch");
}

// Packed images: coords [T, dims] with device offsets.
ca_status build_packed(int dims, const float* coords, int B, int T, int Ct, int max_n,
                 const int32_t* tok_off, const int32_t* clu_off, int grid_side, int cs, int k,
                 int32_t* q_idx, int32_t* nbr, int32_t* key_idx, void* ws, size_t ws_bytes,
                 void* hip_stream) {
  if (B < 0 || T < 0 || Ct < 0 || max_n < 0 || max_n > T)
    return fail(CA_ERR_SHAPE, "bad sizes B=%d T=%d Ct=%d max_n=%d", B, T, Ct, max_n);
  if (cs != 8) return fail(CA_ERR_UNSUPPORTED, "cluster size %d (only 8 is supported)", cs);
  if (k < 1 || k > 8) return fail(CA_ERR_UNSUPPORTED, "k=%d outside 1..8", k);
  if (max_n > kMaxTokensPerImage)
    return fail(CA_ERR_SHAPE, "max_n=%d exceeds 2^22 tokens per image", max_n);
  if (Ct < clusters_of(T, cs) || Ct > T || (int64_t)Ct * cs * k > (int64_t(1) << 31) - 1)
    return fail(CA_ERR_SHAPE, "Ct=%d is inconsistent with T=%d tokens", Ct, T);
  const int gmax = dims == 2 ? 65536 : 16384;
  if (grid_side < 1 || grid_side > gmax)
    return fail(CA_ERR_SHAPE, "grid_side=%d outside [1, %d]", grid_side, gmax);
  if (B == 0 || T == 0) return ok();
  if (!coords || !tok_off || !clu_off || !q_idx || !nbr || !key_idx)
    return fail(CA_ERR_NULL, "NULL tensor pointer");
  const size_t need = ca::build_layout(nullptr, B, T, Ct, max_n).bytes;
  if (need && !ws) return fail(CA_ERR_NULL, "NULL workspace (%zu bytes needed)", need);
  if (ws_bytes < need) return fail(CA_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  Range outs[] = {{q_idx, (size_t)Ct * cs * 4}, {nbr, (size_t)Ct * k * 4},
                  {key_idx, (size_t)Ct * k * cs * 4}, {ws, need}};
  Range ins[] = {{coords, (size_t)T * 4 * dims}, {tok_off, (size_t)(B + 1) * 4},
                 {clu_off, (size_t)(B + 1) * 4}};
  if (ca_status s = check_alias(outs, 4, ins, 3)) return s;
  const ca::Geom g{tok_off, clu_off, max_n, (int)clusters_of(max_n, cs), 0};
  return hip_status(ca::launch_build_neighbors(coords, g, dims, B, T, Ct, grid_side, k, q_idx, nbr,
                                               key_idx, ws, (hipStream_t)hip_stream),
                    "build_neighbors_varlen launch");
}

}  // namespace

extern "C" {

ca_status cluster_attn_build_neighbors(const float* coords, int B, int N, int grid_side, int cs, int k,
                                 int32_t* perm, int32_t* nbr, int32_t* key_idx, void* ws,
                                 size_t ws_bytes, void* hip_stream) {
  return build_uniform(2, coords, B, N, grid_side, cs, k, perm, nbr, key_idx, ws, ws_bytes,
                       hip_stream);
}

ca_status cluster_attn_build_neighbors_3d(const float* coords, int B, int N, int grid_side, int cs,
                                    int k, int32_t* perm, int32_t* nbr, int32_t* key_idx,
                                    void* ws, size_t ws_bytes, void* hip_stream) {
  return build_uniform(3, coords, B, N, grid_side, cs, k, perm, nbr, key_idx, ws, ws_bytes,
                       hip_stream);
}

ca_status cluster_attn_build_neighbors_varlen(const float* coords, int B, int T, int Ct, int max_n,
                                        const int32_t* tok_off, const int32_t* clu_off,
                                        int grid_side, int cs, int k, int32_t* q_idx,
                                        int32_t* nbr, int32_t* key_idx, void* ws,
                                        size_t ws_bytes, void* hip_stream) {
  return build_packed(2, coords, B, T, Ct, max_n, tok_off, clu_off, grid_side, cs, k, q_idx, nbr,
                      key_idx, ws, ws_bytes, hip_stream);
}

ca_status cluster_attn_build_neighbors_varlen_3d(const float* coords, int B, int T, int Ct, int max_n,
                                           const int32_t* tok_off, const int32_t* clu_off,
                                           int grid_side, int cs, int k, int32_t* q_idx,
                                           int32_t* nbr, int32_t* key_idx, void* ws,
                                           size_t ws_bytes, void* hip_stream) {
  return build_packed(3, coords, B, T, Ct, max_n, tok_off, clu_off, grid_side, cs, k, q_idx, nbr,
                      key_idx, ws, ws_bytes, hip_stream);
}

}  // extern "C"

namespace {

// Forward on B images of N tokens and C clusters each (q_idx [B, C, cs]).
ca_status attn_fwd(int dt, int B, int N, int64_t C, int H, int D, int cs, int nk, float scale,
             const void* q, const void* k, const void* v, const int32_t* q_idx,
             const int32_t* key_idx, void* o, float* lse, void* hip_stream) {
  if (!(scale == scale) || scale == INFINITY || scale == -INFINITY)
    return fail(CA_ERR_SHAPE, "scale is not finite");
  if (B == 0 || N == 0 || C == 0) return ok();
  if (!q || !k || !v || !q_idx || !key_idx || !o || !lse)
    return fail(CA_ERR_NULL, "NULL tensor pointer");
  const size_t tb = (size_t)B * N * H * D * elem_size(dt);
  Range outs[] = {{o, tb}, {lse, (size_t)B * N * H * 4}};
  Range ins[] = {{q, tb}, {k, tb}, {v, tb}, {q_idx, (size_t)(B * C * cs) * 4},
                 {key_idx, (size_t)(B * C * nk) * 4}};
  if (ca_status s = check_alias(outs, 2, ins, 5)) return s;
  hipStream_t st = (hipStream_t)hip_stream;
  if (ca::mfma_supported(dt, B, N, (int)C, H, nk))
    return hip_status(ca::launch_fwd_mfma(dt, B, N, (int)C, H, scale, q, k, v, q_idx, key_idx, o,
                                          lse, st),
                      "fwd launch");
  return hip_status(ca::launch_fwd_valu(dt, B, N, (int)C, H, nk, scale, q, k, v, q_idx, key_idx,
                                        o, lse, st),
                    "fwd launch");
}

// Backward; `plan` (nullptr: built here, in `ws` behind the per-call part)
// holds the transposed lists of a cluster_attn_bwd_plan call on the same
// q_idx / key_idx.
ca_status attn_bwd(int dt, int B, int N, int64_t C, int H, int D, int cs, int nk, float scale,
             const void* q, const void* k, const void* v, const void* o, const void* dout,
             const float* lse, const int32_t* q_idx, const int32_t* key_idx, const void* plan,
             size_t plan_bytes, void* dq, void* dk, void* dv, void* ws, size_t ws_bytes,
             void* hip_stream) {
  if (!(scale == scale) || scale == INFINITY || scale == -INFINITY)
    return fail(CA_ERR_SHAPE, "scale is not finite");
  if (B == 0 || N == 0 || C == 0) return ok();
  if (!q || !k || !v || !o || !dout || !lse || !q_idx || !key_idx || !dq || !dk || !dv)
    return fail(CA_ERR_NULL, "NULL tensor pointer");
  const size_t need = plan ? ca::call_layout(nullptr, B, N, H).bytes
                           : ca::bwd_layout(nullptr, B, N, H, C, nk).bytes;
  if (!ws) return fail(CA_ERR_NULL, "NULL workspace (%zu bytes needed)", need);
  if (ws_bytes < need) return fail(CA_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  const size_t pneed = ca::plan_layout(nullptr, B, N, C, nk).bytes;
  if (plan && plan_bytes < pneed)
    return fail(CA_ERR_WORKSPACE, "plan %zu < %zu bytes", plan_bytes, pneed);
  const size_t tb = (size_t)B * N * H * D * elem_size(dt);
  Range outs[] = {{dq, tb}, {dk, tb}, {dv, tb}, {ws, need}};
  Range ins[] = {{q, tb},
                 {k, tb},
                 {v, tb},
                 {o, tb},
                 {dout, tb},
                 {lse, (size_t)B * N * H * 4},
                 {q_idx, (size_t)(B * C * cs) * 4},
                 {key_idx, (size_t)(B * C * nk) * 4},
                 {plan, plan ? pneed : 0}};
  if (ca_status s = check_alias(outs, 4, ins, 9)) return s;
  ca::BwdWorkspace w;
  hipStream_t st = (hipStream_t)hip_stream;
  if (plan) {
    w = ca::plan_layout(const_cast<void*>(plan), B, N, C, nk);
    const ca::BwdWorkspace a = ca::call_layout(ws, B, N, H);
    w.ld = a.ld;
    w.ld_none = a.ld_none;
  } else {
    w = ca::bwd_layout(ws, B, N, H, C, nk);
    hipError_t e = ca::launch_bwd_plan(B, N, (int)C, nk, q_idx, key_idx, w, st);
    if (e != hipSuccess) return hip_status(e, "bwd plan launch");
  }
  if (ca::mfma_supported(dt, B, N, (int)C, H, nk))
    return hip_status(ca::launch_bwd_mfma(3, dt, B, N, (int)C, H, nk, scale, q, k, v, o, dout, lse,
                                          q_idx, key_idx, dq, dk, dv, w, st),
                      "bwd launch");
  return hip_status(ca::launch_bwd_valu(3, dt, B, N, (int)C, H, nk, scale, q, k, v, o, dout, lse,
                                        q_idx, key_idx, dq, dk, dv, w, st),
                    "bwd launch");
}

// (B, N, C) of a plan: C = ceil(N/cs) for equal-size images, or a packed
// batch as one image (B = 1) of N tokens in C clusters.
ca_status check_plan_sizes(int B, int N, int C, int cs, int nk) {
  if (B < 0 || N < 0 || C < 0) return fail(CA_ERR_SHAPE, "bad sizes B=%d N=%d C=%d", B, N, C);
  if (cs != 8) return fail(CA_ERR_UNSUPPORTED, "cluster size %d (only 8 is supported)", cs);
  if (nk % cs != 0 || nk / cs < 1 || nk / cs > 8)
    return fail(CA_ERR_UNSUPPORTED, "nk=%d must be cs*k with 1 <= k <= 8", nk);
  const int64_t cmin = clusters_of(N, cs);
  const bool ok_c = C == cmin || (B == 1 && C >= cmin && C <= N);
  if (!ok_c) return fail(CA_ERR_SHAPE, "C=%d is inconsistent with B=%d, N=%d", C, B, N);
  if ((int64_t)B * N > (int64_t(1) << 31) - 1 || (int64_t)B * C * nk * 8 > (int64_t(1) << 31) - 1)
    return fail(CA_ERR_SHAPE, "problem too large");
  return CA_OK;
}

// Packed batches run as one image of T tokens and Ct clusters.
ca_status check_varlen(int dt, int T, int Ct, int H, int D, int cs, int nk) {
  if (ca_status s = check_attn_shape(dt, 1, T, H, D, cs, nk)) return s;
  if (Ct < 0 || Ct < clusters_of(T, cs) || Ct > T)
    return fail(CA_ERR_SHAPE, "Ct=%d is inconsistent with T=%d tokens", Ct, T);
  return CA_OK;
}

}  // namespace

extern "C" {

ca_status cluster_attn_fwd(int dt, int B, int N, int H, int D, int cs, int nk, float scale,
                     const void* q, const void* k, const void* v, const int32_t* q_idx,
                     const int32_t* key_idx, void* o, float* lse, void* hip_stream) {
  if (ca_status s = check_attn_shape(dt, B, N, H, D, cs, nk)) return s;
  return attn_fwd(dt, B, N, clusters_of(N, cs), H, D, cs, nk, scale, q, k, v, q_idx, key_idx, o,
                  lse, hip_stream);
}

size_t cluster_attn_bwd_workspace(int dt, int B, int N, int H, int D, int cs, int nk) {
  const char saved = g_last_error[0];
  if (check_attn_shape(dt, B, N, H, D, cs, nk) != CA_OK) {
    g_last_error[0] = saved;
    return 0;
  }
  return ca::bwd_layout(nullptr, B, N, H, clusters_of(N, cs), nk).bytes;
}

ca_status cluster_attn_bwd(int dt, int B, int N, int H, int D, int cs, int nk, float scale,
                     const void* q, const void* k, const void* v, const void* o,
                     const void* dout, const float* lse, const int32_t* q_idx,
                     const int32_t* key_idx, void* dq, void* dk, void* dv, void* ws,
                     size_t ws_bytes, void* hip_stream) {
  if (ca_status s = check_attn_shape(dt, B, N, H, D, cs, nk)) return s;
  return attn_bwd(dt, B, N, clusters_of(N, cs), H, D, cs, nk, scale, q, k, v, o, dout, lse, q_idx,
                  key_idx, nullptr, 0, dq, dk, dv, ws, ws_bytes, hip_stream);
}

ca_status cluster_attn_fwd_varlen(int dt, int T, int Ct, int H, int D, int cs, int nk, float scale,
                            const void* q, const void* k, const void* v, const int32_t* q_idx,
                            const int32_t* key_idx, void* o, float* lse, void* hip_stream) {
  if (ca_status s = check_varlen(dt, T, Ct, H, D, cs, nk)) return s;
  return attn_fwd(dt, 1, T, Ct, H, D, cs, nk, scale, q, k, v, q_idx, key_idx, o, lse, hip_stream);
}

size_t cluster_attn_bwd_varlen_workspace(int dt, int T, int Ct, int H, int D, int cs, int nk) {
  const char saved = g_last_error[0];
  if (check_varlen(dt, T, Ct, H, D, cs, nk) != CA_OK) {
    g_last_error[0] = saved;
    return 0;
  }
  return ca::bwd_layout(nullptr, 1, T, H, Ct, nk).bytes;
}

ca_status cluster_attn_bwd_varlen(int dt, int T, int Ct, int H, int D, int cs, int nk, float scale,
                            const void* q, const void* k, const void* v, const void* o,
                            const void* dout, const float* lse, const int32_t* q_idx,
                            const int32_t* key_idx, void* dq, void* dk, void* dv, void* ws,
                            size_t ws_bytes, void* hip_stream) {
  if (ca_status s = check_varlen(dt, T, Ct, H, D, cs, nk)) return s;
  return attn_bwd(dt, 1, T, Ct, H, D, cs, nk, scale, q, k, v, o, dout, lse, q_idx, key_idx,
                  nullptr, 0, dq, dk, dv, ws, ws_bytes, hip_stream);
}

size_t cluster_attn_bwd_plan_workspace(int B, int N, int C, int cs, int nk) {
  const char saved = g_last_error[0];
  if (check_plan_sizes(B, N, C, cs, nk) != CA_OK) {
    g_last_error[0] = saved;
    return 0;
  }
  return ca::plan_layout(nullptr, B, N, C, nk).bytes;
}

ca_status cluster_attn_bwd_plan(int B, int N, int C, int cs, int nk, const int32_t* q_idx,
                          const int32_t* key_idx, void* plan, size_t plan_bytes,
                          void* hip_stream) {
  if (ca_status s = check_plan_sizes(B, N, C, cs, nk)) return s;
  if (B == 0 || N == 0 || C == 0) return ok();
  if (!q_idx || !key_idx || !plan) return fail(CA_ERR_NULL, "NULL pointer");
  const size_t need = ca::plan_layout(nullptr, B, N, C, nk).bytes;
  if (plan_bytes < need) return fail(CA_ERR_WORKSPACE, "plan %zu < %zu bytes", plan_bytes, need);
  Range outs[] = {{plan, need}};
  Range ins[] = {{q_idx, (size_t)B * C * cs * 4}, {key_idx, (size_t)B * C * nk * 4}};
  if (ca_status s = check_alias(outs, 1, ins, 2)) return s;
  const ca::BwdWorkspace w = ca::plan_layout(plan, B, N, C, nk);
  return hip_status(ca::launch_bwd_plan(B, N, C, nk, q_idx, key_idx, w, (hipStream_t)hip_stream),
                    "bwd plan launch");
}

ca_status cluster_attn_bwd_plan_varlen(int B, int T, int Ct, int max_n, const int32_t* tok_off,
                                 const int32_t* clu_off, int cs, int nk, const int32_t* q_idx,
                                 const int32_t* key_idx, void* plan, size_t plan_bytes,
                                 void* hip_stream) {
  if (ca_status s = check_plan_sizes(1, T, Ct, cs, nk)) return s;
  if (B < 0 || max_n < 0 || max_n > T)
    return fail(CA_ERR_SHAPE, "bad sizes B=%d T=%d max_n=%d", B, T, max_n);
  if (B == 0 || T == 0 || Ct == 0) return ok();
  if (!q_idx || !key_idx || !plan || !tok_off || !clu_off) return fail(CA_ERR_NULL, "NULL pointer");
  const size_t need = ca::plan_layout(nullptr, 1, T, Ct, nk).bytes;
  if (plan_bytes < need) return fail(CA_ERR_WORKSPACE, "plan %zu < %zu bytes", plan_bytes, need);
  Range outs[] = {{plan, need}};
  Range ins[] = {{q_idx, (size_t)Ct * cs * 4}, {key_idx, (size_t)Ct * nk * 4},
                 {tok_off, (size_t)(B + 1) * 4}, {clu_off, (size_t)(B + 1) * 4}};
  if (ca_status s = check_alias(outs, 1, ins, 4)) return s;
  const ca::BwdWorkspace w = ca::plan_layout(plan, 1, T, Ct, nk);
  const ca::Geom g{tok_off, clu_off, max_n, (int)clusters_of(max_n, cs), 0};
  return hip_status(ca::launch_bwd_plan(B, T, Ct, nk, q_idx, key_idx, w, (hipStream_t)hip_stream,
                                        &g),
                    "bwd plan launch");
}

size_t cluster_attn_bwd_planned_workspace(int dt, int B, int N, int H, int D) {
  if (dt < CA_F32 || dt > CA_F16 || B < 0 || N < 0 || H < 1 || D != 32) return 0;
  return ca::call_layout(nullptr, B, N, H).bytes;
}

ca_status cluster_attn_bwd_planned(int dt, int B, int N, int C, int H, int D, int cs, int nk,
                             float scale, const void* q, const void* k, const void* v,
                             const void* o, const void* dout, const float* lse,
                             const int32_t* q_idx, const int32_t* key_idx, const void* plan,
                             size_t plan_bytes, void* dq, void* dk, void* dv, void* ws,
                             size_t ws_bytes, void* hip_stream) {
  if (ca_status s = check_attn_shape(dt, B, N, H, D, cs, nk)) return s;
  if (ca_status s = check_plan_sizes(B, N, C, cs, nk)) return s;
  if (B > 0 && N > 0 && C > 0 && !plan) return fail(CA_ERR_NULL, "NULL plan");
  return attn_bwd(dt, B, N, C, H, D, cs, nk, scale, q, k, v, o, dout, lse, q_idx, key_idx, plan,
                  plan_bytes, dq, dk, dv, ws, ws_bytes, hip_stream);
}

}  // extern "C"

// ---- the backward without a caller workspace ------------------------------
// The (LSE log2 e, Delta) pairs that pass A hands to pass B live in this
// array (8 bytes per query row and head, plus one 16-byte (+inf, 0) pair):
// each GPU holds its own copy from module load until the process ends.
constexpr size_t kScratchBytes = size_t(32) << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
void* g_scratch[kMaxDevices] = {};   // device address of `scratch`, per device
std::mutex g_scratch_mu;

// The address of `scratch` on the current device, looked up once per device
// (host code never uses the array's own name, a host-side stand-in).
ca_status scratch_of_current_device(void** out) {
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(CA_ERR_UNSUPPORTED, "device %d outside 0..%d", dev, kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    const hipError_t r = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (r != hipSuccess) return hip_status(r, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(CA_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return ok();
}

}  // namespace

extern "C" {

size_t cluster_attn_bwd_planned_noalloc_max_rows(void) {
  // rows (query token x head) whose pairs fit the scratch with the extra pair
  return (kScratchBytes - 256) / sizeof(float2);
}

ca_status cluster_attn_bwd_planned_noalloc(int dt, int B, int N, int C, int H, int D, int cs,
                                           int nk, float scale, const void* q, const void* k,
                                           const void* v, const void* o, const void* dout,
                                           const float* lse, const int32_t* q_idx,
                                           const int32_t* key_idx, const void* plan,
                                           size_t plan_bytes, void* dq, void* dk, void* dv,
                                           void* hip_stream) {
  if (ca_status s = check_attn_shape(dt, B, N, H, D, cs, nk)) return s;
  if (ca_status s = check_plan_sizes(B, N, C, cs, nk)) return s;
  if (B == 0 || N == 0 || C == 0) return ok();
  if (!plan) return fail(CA_ERR_NULL, "NULL plan");
  const size_t need = ca::call_layout(nullptr, B, N, H).bytes;
  if (need > kScratchBytes)
    return fail(CA_ERR_WORKSPACE,
                "B*N*H = %lld query rows need %zu bytes of LSE/Delta pairs; the scratch of "
                "cluster_attn_bwd_planned_noalloc holds %zu (at most %zu rows)",
                (long long)B * N * H, need, kScratchBytes,
                cluster_attn_bwd_planned_noalloc_max_rows());
  void* ws = nullptr;
  if (ca_status s = scratch_of_current_device(&ws)) return s;
  return attn_bwd(dt, B, N, C, H, D, cs, nk, scale, q, k, v, o, dout, lse, q_idx, key_idx, plan,
                  plan_bytes, dq, dk, dv, ws, kScratchBytes, hip_stream);
}

size_t cluster_attn_knn_table_workspace(int B, int N, int grid_side) {
  if (B < 0 || N < 0 || N > (1 << 24) || grid_side < 1 || grid_side > 2048) return 0;
  return ca::knn_table_layout(nullptr, B, N).bytes;
}

ca_status cluster_attn_knn_table(const float* coords, int B, int N, int grid_side, int K,
                                 int32_t* table, void* ws, size_t ws_bytes, void* hip_stream) {
  if (B < 0 || N < 0) return fail(CA_ERR_SHAPE, "bad sizes B=%d N=%d", B, N);
  if (grid_side < 1 || grid_side > 2048)
    return fail(CA_ERR_UNSUPPORTED, "grid_side=%d: the table build supports 1..2048", grid_side);
  if (N > (1 << 24)) return fail(CA_ERR_SHAPE, "N=%d above 2^24", N);
  if ((int64_t)B * N > (int64_t(1) << 31) - 1) return fail(CA_ERR_SHAPE, "B*N above 2^31 - 1");
  if (K < 1 || K > 16) return fail(CA_ERR_UNSUPPORTED, "K=%d outside 1..16", K);
  if (B == 0) return ok();
  if (!table || (N > 0 && !coords)) return fail(CA_ERR_NULL, "NULL tensor pointer");
  const size_t need = ca::knn_table_layout(nullptr, B, N).bytes;
  if (need && !ws) return fail(CA_ERR_NULL, "NULL workspace (%zu bytes needed)", need);
  if (ws_bytes < need) return fail(CA_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  const size_t tb = (size_t)B * grid_side * grid_side * K * 4;
  Range outs[] = {{table, tb}, {ws, need}};
  Range ins[] = {{coords, (size_t)B * N * 8}};
  if (ca_status s = check_alias(outs, 2, ins, 1)) return s;
  return hip_status(ca::launch_knn_table(coords, B, N, grid_side, K, table, ws,
                                         (hipStream_t)hip_stream),
                    "knn table launch");
}

ca_status cluster_attn_knn_sample_fwd(int dt, int B, int N, int M, int C, int grid_side, int K, float p,
                                const float* coords, const void* feats, const float* queries,
                                const int32_t* table, void* out, void* hip_stream) {
  if (dt != CA_F32 && dt != CA_BF16 && dt != CA_F16)
    return fail(CA_ERR_UNSUPPORTED, "dtype %d is not one of CA_F32, CA_BF16, CA_F16", dt);
  if (ca_status s = check_knn_shape(B, N, M, C, grid_side, K)) return s;
  if (!(p == p) || p == INFINITY || p == -INFINITY) return fail(CA_ERR_SHAPE, "p is not finite");
  if (B == 0 || M == 0) return ok();
  if (!queries || !table || !out || (N > 0 && (!coords || !feats)))
    return fail(CA_ERR_NULL, "NULL tensor pointer");
  const size_t es = elem_size(dt);
  Range outs[] = {{out, (size_t)B * M * C * es}};
  Range ins[] = {{coords, (size_t)B * N * 8},
                 {feats, (size_t)B * N * C * es},
                 {queries, (size_t)B * M * 8},
                 {table, (size_t)B * grid_side * grid_side * K * 4}};
  if (ca_status s = check_alias(outs, 1, ins, 4)) return s;
  return hip_status(ca::launch_knn_fwd(dt, B, N, M, C, grid_side, K, p, coords, feats, queries,
                                       table, out, (hipStream_t)hip_stream),
                    "knn fwd launch");
}

size_t cluster_attn_knn_sample_bwd_workspace(int B, int N, int M, int K) {
  if (B < 0 || N < 0 || M < 0 || K < 1 || K > 16 || N > (1 << 24) || M > (1 << 24)) return 0;
  return ca::knn_layout(nullptr, B, N, M, K).bytes;
}

ca_status cluster_attn_knn_sample_bwd(int dt, int B, int N, int M, int C, int grid_side, int K, float p,
                                const float* coords, const void* feats, const float* queries,
                                const int32_t* table, const void* dout, void* dfeats, float* dq,
                                float* dp, void* ws, size_t ws_bytes, void* hip_stream) {
  if (dt != CA_F32 && dt != CA_BF16 && dt != CA_F16)
    return fail(CA_ERR_UNSUPPORTED, "dtype %d is not one of CA_F32, CA_BF16, CA_F16", dt);
  if (ca_status s = check_knn_shape(B, N, M, C, grid_side, K)) return s;
  if (!(p == p) || p == INFINITY || p == -INFINITY) return fail(CA_ERR_SHAPE, "p is not finite");
  if (!dp) return fail(CA_ERR_NULL, "NULL dp pointer");
  const bool some_q = B > 0 && M > 0, some_t = B > 0 && N > 0;
  if ((some_q && (!queries || !table || !dout || !dq)) ||
      (some_t && (!coords || !feats || !dfeats)))
    return fail(CA_ERR_NULL, "NULL tensor pointer");
  const size_t need = ca::knn_layout(nullptr, B, N, M, K).bytes;
  if (need && !ws) return fail(CA_ERR_NULL, "NULL workspace (%zu bytes needed)", need);
  if (ws_bytes < need) return fail(CA_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  const size_t es = elem_size(dt);
  Range outs[] = {{dfeats, (size_t)B * N * C * es}, {dq, (size_t)B * M * 8}, {dp, 4}, {ws, need}};
  Range ins[] = {{coords, (size_t)B * N * 8},
                 {feats, (size_t)B * N * C * es},
                 {queries, (size_t)B * M * 8},
                 {table, (size_t)B * grid_side * grid_side * K * 4},
                 {dout, (size_t)B * M * C * es}};
  if (ca_status s = check_alias(outs, 4, ins, 5)) return s;
  return hip_status(ca::launch_knn_bwd(dt, B, N, M, C, grid_side, K, p, coords, feats, queries,
                                       table, dout, dfeats, dq, dp, ws, (hipStream_t)hip_stream),
                    "knn bwd launch");
}

size_t cluster_attn_merge_plan_workspace(int B, int N, int k) {
  if (B < 0 || N < 0 || N > (1 << 24) || k < 0 || k > N) return 0;
  return ca::merge_layout(nullptr, B, N, k).bytes;
}

ca_status cluster_attn_merge_plan(const float* coords, const float* scores, int B, int N, int k,
                                  int grid_side, int32_t* anchors, int32_t* assign,
                                  int32_t* members, int32_t* offsets, void* ws, size_t ws_bytes,
                                  void* hip_stream) {
  if (B < 0 || N < 0 || k < 0) return fail(CA_ERR_SHAPE, "bad sizes B=%d N=%d k=%d", B, N, k);
  if (N > (1 << 24)) return fail(CA_ERR_SHAPE, "N=%d above 2^24", N);
  if ((int64_t)B * N > (int64_t(1) << 31) - 1) return fail(CA_ERR_SHAPE, "B*N above 2^31 - 1");
  if (k > N || (N > 0 && k < 1)) return fail(CA_ERR_SHAPE, "k=%d must be in [1, N=%d]", k, N);
  if (grid_side < 1 || grid_side > 65536)
    return fail(CA_ERR_SHAPE, "grid_side=%d outside [1, 65536]", grid_side);
  if (B == 0 || N == 0) return ok();
  if (!coords || !scores || !anchors || !assign || !members || !offsets)
    return fail(CA_ERR_NULL, "NULL tensor pointer");
  const size_t need = ca::merge_layout(nullptr, B, N, k).bytes;
  if (need && !ws) return fail(CA_ERR_NULL, "NULL workspace (%zu bytes needed)", need);
  if (ws_bytes < need) return fail(CA_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  Range outs[] = {{anchors, (size_t)B * k * 4}, {assign, (size_t)B * N * 4},
                  {members, (size_t)B * N * 4}, {offsets, (size_t)B * (k + 1) * 4}, {ws, need}};
  Range ins[] = {{coords, (size_t)B * N * 8}, {scores, (size_t)B * N * 4}};
  if (ca_status s = check_alias(outs, 5, ins, 2)) return s;
  return hip_status(ca::launch_merge_plan(coords, scores, B, N, k, grid_side, anchors, assign,
                                          members, offsets, ws, (hipStream_t)hip_stream),
                    "merge plan launch");
}

ca_status cluster_attn_merge_fwd(int dt, int B, int N, int k, int C, const void* feats,
                           const float* coords, const float* scores, const int32_t* members,
                           const int32_t* offsets, void* out_feats, float* out_coords,
                           void* hip_stream) {
  if (ca_status s = check_merge_shape(dt, B, N, k, C)) return s;
  if (B == 0 || N == 0) return ok();
  if (!feats || !coords || !scores || !members || !offsets || !out_feats || !out_coords)
    return fail(CA_ERR_NULL, "NULL tensor pointer");
  const size_t es = elem_size(dt);
  Range outs[] = {{out_feats, (size_t)B * k * C * es}, {out_coords, (size_t)B * k * 8}};
  Range ins[] = {{feats, (size_t)B * N * C * es}, {coords, (size_t)B * N * 8},
                 {scores, (size_t)B * N * 4}, {members, (size_t)B * N * 4},
                 {offsets, (size_t)B * (k + 1) * 4}};
  if (ca_status s = check_alias(outs, 2, ins, 5)) return s;
  return hip_status(ca::launch_merge_fwd(dt, B, N, k, C, feats, coords, scores, members, offsets,
                                         out_feats, out_coords, (hipStream_t)hip_stream),
                    "merge fwd launch");
}

ca_status cluster_attn_merge_bwd(int dt, int B, int N, int k, int C, const void* feats,
                           const float* coords, const float* scores, const int32_t* members,
                           const int32_t* offsets, const void* dout_feats,
                           const float* dout_coords, void* dfeats, float* dcoords,
                           float* dscores, void* hip_stream) {
  if (ca_status s = check_merge_shape(dt, B, N, k, C)) return s;
  if (B == 0 || N == 0) return ok();
  if (!feats || !coords || !scores || !members || !offsets || !dout_feats || !dout_coords ||
      !dfeats || !dcoords || !dscores)
    return fail(CA_ERR_NULL, "NULL tensor pointer");
  const size_t es = elem_size(dt);
  Range outs[] = {{dfeats, (size_t)B * N * C * es}, {dcoords, (size_t)B * N * 8},
                  {dscores, (size_t)B * N * 4}};
  Range ins[] = {{feats, (size_t)B * N * C * es},   {coords, (size_t)B * N * 8},
                 {scores, (size_t)B * N * 4},       {members, (size_t)B * N * 4},
                 {offsets, (size_t)B * (k + 1) * 4}, {dout_feats, (size_t)B * k * C * es},
                 {dout_coords, (size_t)B * k * 8}};
  if (ca_status s = check_alias(outs, 3, ins, 7)) return s;
  return hip_status(ca::launch_merge_bwd(dt, B, N, k, C, feats, coords, scores, members, offsets,
                                         dout_feats, dout_coords, dfeats, dcoords, dscores,
                                         (hipStream_t)hip_stream),
                    "merge bwd launch");
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Host-side validation of index lists (debug helper; no GPU involved).
// ---------------------------------------------------------------------------
extern "C" ca_status cluster_attn_check_lists(int B, int N, int C, int cs, int nk,
                                              const int32_t* q_idx, const int32_t* key_idx) {
  if (B < 0 || N < 0 || C < 0 || cs < 1 || nk < 0)
    return fail(CA_ERR_SHAPE, "bad sizes B=%d N=%d C=%d cs=%d nk=%d", B, N, C, cs, nk);
  if ((int64_t)C * cs < N || (B > 1 && C != clusters_of(N, cs)))
    return fail(CA_ERR_SHAPE, "C=%d clusters of %d cannot hold N=%d tokens per image", C, cs, N);
  if ((int64_t)B * C * (cs + nk) > (int64_t(1) << 40)) return fail(CA_ERR_SHAPE, "lists too large");
  if (B == 0 || C == 0) return ok();
  if (!q_idx || (nk && !key_idx)) return fail(CA_ERR_NULL, "NULL list pointer");
  char* seen = new (std::nothrow) char[N > 0 ? N : 1];
  if (!seen) return fail(CA_ERR_SHAPE, "out of host memory for N=%d", N);
  ca_status st = CA_OK;
  for (int b = 0; b < B && st == CA_OK; ++b) {
    memset(seen, 0, N > 0 ? N : 1);
    const int32_t* qb = q_idx + (int64_t)b * C * cs;
    const int32_t* kb = key_idx ? key_idx + (int64_t)b * C * nk : nullptr;
    int64_t tokens = 0;
    for (int64_t c = 0; c < C && st == CA_OK; ++c) {
      bool ended = false;
      for (int m = 0; m < cs; ++m) {
        const int32_t t = qb[c * cs + m];
        if (t == -1) {
          if (m == 0) {
            st = fail(CA_ERR_SHAPE, "q_idx[%d][%lld][0] is -1 (member 0 must be a token)", b,
                      (long long)c);
            break;
          }
          ended = true;
          continue;
        }
        if (t < 0 || t >= N) {
          st = fail(CA_ERR_SHAPE, "q_idx[%d][%lld][%d] = %d outside [-1, %d)", b, (long long)c, m,
                    t, N);
          break;
        }
        if (ended) {
          st = fail(CA_ERR_SHAPE, "q_idx[%d][%lld][%d] = %d follows a -1", b, (long long)c, m, t);
          break;
        }
        if (seen[t]) {
          st = fail(CA_ERR_SHAPE, "token %d appears twice in q_idx[%d]", t, b);
          break;
        }
        seen[t] = 1;
        ++tokens;
      }
      for (int s = 0; s < nk && st == CA_OK; ++s) {
        const int32_t t = kb[c * nk + s];
        if (t < -1 || t >= N)
          st = fail(CA_ERR_SHAPE, "key_idx[%d][%lld][%d] = %d outside [-1, %d)", b, (long long)c,
                    s, t, N);
      }
    }
    if (st == CA_OK && tokens != N)
      st = fail(CA_ERR_SHAPE, "q_idx[%d] holds %lld of the %d tokens", b, (long long)tokens, N);
  }
  delete[] seen;
  return st == CA_OK ? ok() : st;
}
