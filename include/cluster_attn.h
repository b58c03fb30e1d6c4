/*
 * cluster_attn.h - C ABI of the MI355X (gfx950) local cluster attention
 * library: neighbour-list build, gathered-KV forward, fused backward.
 *
 * What it computes.  The English notes page "AFFMAE: Scalable Vision
 * Pre-Training for High-Resolution Microscopy Segmentation on Desktop
 * Hardware" (en.papernotes.org), section "Overall Architecture", describes an
 * encoder in which every token keeps an explicit 2D coordinate and attention
 * is computed through local balanced clustering; the arXiv abstract of the
 * same paper (mlsanity.com page of that title) says the attention runs in
 * numerically stable, mixed-precision, Flash-style kernels, and the notes'
 * "Limitations & Future Work" name off-grid gather/scatter as the cost and
 * space-filling curves as the neighbourhood structure.  The pages fix no
 * interface; the calls below are this library's.  Readings of the open
 * points: Morton (Z-order, x in even bits) balanced clusters of cs = 8
 * tokens; each cluster attends to the keys of itself plus its k-1 = 5
 * nearest clusters by integer centroid-sum distance; plain scaled
 * dot-product softmax over those 48 key slots; LSE is the natural
 * log-sum-exp of the scaled logits.
 *
 * Conventions shared by every call.
 *  - Tensor pointers are DEVICE pointers (hipMalloc'd or torch CUDA tensors),
 *    owned by the caller; the library allocates nothing and keeps no state
 *    besides its loaded code objects.
 *  - Layouts are dense row-major.  Q, K, V, O, dO, dQ, dK, dV are
 *    [B, N, H, D] (token-major, heads inside a token); LSE is [B, N, H] f32.
 *    Index arrays are int32 and image-local: values in [0, N), -1 = empty
 *    slot.  A slot repeated in one key list counts once per occurrence.
 *  - q_idx [B, C, cs] (C = ceil(N/cs)) partitions each image's tokens into
 *    the query clusters: every token appears exactly once, and the cs - n
 *    unused places of a cluster of n < cs members hold -1 (after its
 *    members; member 0 of every row is a token).  When cs divides N this is
 *    a permutation of 0..N-1.  A -1 member is no query and no key: nothing
 *    is written for it.
 *  - Every call is asynchronous on `hip_stream` (a hipStream_t; NULL = the
 *    default stream): it validates its arguments synchronously, enqueues its
 *    kernels and returns.  Validation failures return before any launch and
 *    write nothing.  Out-of-range indices are a precondition the kernels do
 *    not check; cluster_attn_check_lists (host pointers) checks them.
 *  - Outputs are fully overwritten (dK and dV are not accumulated into);
 *    tokens no slot references get dK = dV = 0.  Outputs must not overlap
 *    inputs (CA_ERR_ALIAS where the ranges are visibly overlapping).
 *  - Supported set: cs = 8, D = 32, nk = cs*k with 1 <= k <= 8 (the MFMA
 *    kernels serve nk = 48 in bf16/f16; every other case runs on the
 *    vector-ALU kernels), H >= 1, any N >= 0, dtype f32 / bf16 / f16.
 *    Anything else: CA_ERR_SHAPE or CA_ERR_UNSUPPORTED.
 *  - No call throws across the ABI.  Launch or runtime failures return
 *    CA_ERR_HIP; cluster_attn_last_error() gives the text (thread-local).
 *    Entry points return ca_status (an int-sized enum; 0 = CA_OK).
 */
#ifndef CLUSTER_ATTN_H
#define CLUSTER_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CA_OK = 0,
  CA_ERR_NULL = 1,        /* a required pointer is NULL                        */
  CA_ERR_SHAPE = 2,       /* sizes out of range or inconsistent                */
  CA_ERR_UNSUPPORTED = 3, /* valid request outside the supported set           */
  CA_ERR_WORKSPACE = 4,   /* workspace smaller than the *_workspace() query    */
  CA_ERR_ALIAS = 5,       /* an output overlaps an input or another output     */
  CA_ERR_HIP = 6          /* the HIP runtime reported an error                 */
} ca_status;

typedef enum { CA_F32 = 0, CA_BF16 = 1, CA_F16 = 2 } ca_dtype;

/*
 * Workspace bytes needed by cluster_attn_build_neighbors for these sizes.
 * 0 for invalid sizes, and also for valid ones with N <= 4096: such an image
 * is built by one workgroup entirely in LDS and needs no workspace.
 * Supported: N <= 2^22 tokens per image.
 */
size_t cluster_attn_build_neighbors_workspace(int B, int N, int cs, int k);

/*
 * Neighbour-list build (notes page, "Overall Architecture": 2D coordinate per
 * token, local balanced clustering; "Limitations & Future Work": space-filling
 * curves).  Steps, all exact integer arithmetic after one fp64 quantisation:
 *   1. q = clamp(floor((c + 0.5) * 2^(16 - ceil(log2 G))), 0, 65535) per axis;
 *      Morton code with x in the even bits and y in the odd bits.
 *   2. per image, stable sort of tokens by (code, token index) -> order;
 *      cluster c = order[c*cs .. c*cs+cs-1], C = ceil(N/cs) clusters, the
 *      last one partial (N mod cs members) when cs does not divide N.
 *   3. centroids compared through their means: integer sums of the
 *      members' (qx, qy), scaled to a common multiple of the means (for
 *      cs = 8: sum * lcm(8, N mod 8) / members; plain sums when 8 | N).
 *   4. nbr[c] = c, then the k-1 clusters b != c with the smallest
 *      (squared centroid distance, b), ascending; -1 pads if C < k.
 *   5. key_idx[c][s*cs + m] = q_idx[nbr[c][s]][m] (-1 where nbr is -1 or
 *      the member is absent).
 * Arguments:
 *   coords    [B, N, 2] f32, (x = column, y = row) in patch units, device.
 *   grid_side G >= 1, the side of the patch grid the coordinates live on
 *             (only its ceil(log2) is used; coordinates outside [-0.5, G-0.5)
 *             clamp).
 *   cs        cluster size, must be 8.   k: clusters per list, 1..8.
 *   perm      [B, C*cs] int32 out: the q_idx rows [B, C, cs] (the token
 *             order itself when cs divides N; -1 after the members of a
 *             partial last cluster).
 *   nbr       [B, C, k] int32 out, slot 0 = self.
 *   key_idx   [B, C, cs*k] int32 out.
 *   ws        device workspace of at least
 *             cluster_attn_build_neighbors_workspace(B, N, cs, k) bytes
 *             (may be NULL when that is 0).  Contents on entry are ignored.
 * Deterministic: the output is the unique list defined above.
 */
ca_status cluster_attn_build_neighbors(const float* coords, int B, int N, int grid_side, int cs, int k,
                                 int32_t* perm, int32_t* nbr, int32_t* key_idx, void* ws,
                                 size_t ws_bytes, void* hip_stream);

/*
 * 3D tokens (notes page, "Limitations & Future Work": scaling to 3D voxels
 * is named as open; this is the library's reading).  The same steps as
 * cluster_attn_build_neighbors with three axes:
 *   1. q = clamp(floor((c + 0.5) * 2^(14 - ceil(log2 G))), 0, 16383) per
 *      axis (14 bits); Morton code with x, y, z in bits 3b, 3b+1, 3b+2
 *      (42 bits).
 *   2.-5. as in 2D (stable sort by (code, token), runs of cs, centroids as
 *      scaled means over three axes, k-1 nearest by (squared distance,
 *      index), key lists).
 *   coords    [B, N, 3] f32, (x = column, y = row, z = slice) in patch units.
 *   grid_side G in [1, 16384], the largest side of the patch grid.
 * Outputs, workspace (cluster_attn_build_neighbors_workspace) and errors as
 * for cluster_attn_build_neighbors.  The lists feed the same cluster_attn_fwd
 * / cluster_attn_bwd (the attention does not depend on the dimension).
 */
ca_status cluster_attn_build_neighbors_3d(const float* coords, int B, int N, int grid_side, int cs,
                                    int k, int32_t* perm, int32_t* nbr, int32_t* key_idx,
                                    void* ws, size_t ws_bytes, void* hip_stream);

/*
 * Packed batch of images of different sizes (ragged geometry).  Image b holds
 * tokens [tok_off[b], tok_off[b+1]) of the packed arrays and clusters
 * [clu_off[b], clu_off[b+1]), with clu_off[b+1] - clu_off[b] =
 * ceil((tok_off[b+1] - tok_off[b]) / cs).  Each image is built exactly as by
 * cluster_attn_build_neighbors on its own; the lists carry batch-global
 * ids (token ids offset by tok_off[b], cluster ids by clu_off[b]), so that
 * the packed batch can be handed to cluster_attn_fwd_varlen /
 * cluster_attn_bwd_varlen as one index space.
 *   coords    [T, 2] f32 device, the images one after another.
 *   B, T, Ct  images, total tokens (tok_off[B]), total clusters (clu_off[B]).
 *   max_n     the largest image's token count (sizes the launch; <= 2^22).
 *   tok_off, clu_off  [B + 1] int32 device, starting at 0, nondecreasing and
 *             consistent with T, Ct and max_n: a precondition, not checked
 *             (the Python binding computes them).
 *   q_idx     [Ct, cs], nbr [Ct, k], key_idx [Ct, cs*k] int32 out.
 *   ws        at least cluster_attn_build_neighbors_varlen_workspace(...)
 *             bytes (0 when max_n <= 4096).
 */
size_t cluster_attn_build_neighbors_varlen_workspace(int B, int T, int Ct, int max_n, int cs,
                                                     int k);
ca_status cluster_attn_build_neighbors_varlen(const float* coords, int B, int T, int Ct, int max_n,
                                        const int32_t* tok_off, const int32_t* clu_off,
                                        int grid_side, int cs, int k, int32_t* q_idx,
                                        int32_t* nbr, int32_t* key_idx, void* ws,
                                        size_t ws_bytes, void* hip_stream);
/* The same for packed 3D volumes: coords [T, 3] f32 (readings of
 * cluster_attn_build_neighbors_3d); same workspace query. */
ca_status cluster_attn_build_neighbors_varlen_3d(const float* coords, int B, int T, int Ct, int max_n,
                                           const int32_t* tok_off, const int32_t* clu_off,
                                           int grid_side, int cs, int k, int32_t* q_idx,
                                           int32_t* nbr, int32_t* key_idx, void* ws,
                                           size_t ws_bytes, void* hip_stream);

/*
 * Forward (notes page "Overall Architecture": local cluster attention; arXiv
 * abstract: Flash-style kernels).  For every image b, query cluster c and
 * head h, with K_s = K[b, key_idx[b,c,s], h, :] over the valid slots s:
 *   S_ms = scale * <Q[b, q_idx[b,c,m], h, :], K_s>
 *   O    = sum_s exp(S_ms - LSE_m) V_s,  LSE_m = ln sum_s exp(S_ms)
 * computed with fp32 max/sum statistics and fp32 accumulation (bf16/f16
 * operands of the matrix products; the unnormalised probabilities, all in
 * [0, 1], are rounded once to dt for the P*V product: relative error at most
 * 2^-8 (bf16) or 2^-11 (f16; absolute below 2^-25 in its subnormal range)
 * per probability; normalisation by the fp32 row sum happens after the
 * product).
 *   dt        element type of q, k, v and o.
 *   D         head dim, must be 32.  nk: slots per list (= cs*k).
 *   scale     logit scale (1/sqrt(D) for the plain reading).
 *   q, k, v   [B, N, H, D] dt.   q_idx [B, C, cs], key_idx [B, C, nk] int32.
 *   o         [B, N, H, D] dt out (RNE from fp32).
 *   lse       [B, N, H] f32 out.  A row whose list has no valid slot gets
 *             O = 0 and LSE = -inf.
 */
ca_status cluster_attn_fwd(int dt, int B, int N, int H, int D, int cs, int nk, float scale,
                     const void* q, const void* k, const void* v, const int32_t* q_idx,
                     const int32_t* key_idx, void* o, float* lse, void* hip_stream);

/* Workspace bytes needed by cluster_attn_bwd (0 for invalid sizes). */
size_t cluster_attn_bwd_workspace(int dt, int B, int N, int H, int D, int cs, int nk);

/*
 * Backward: gradients of L = sum(dO * O) with the index lists held fixed
 * (training through the kernels, notes page "Loss & Training").  With P the
 * forward's probabilities recomputed as exp(S - LSE):
 *   Delta_m = <dO_m, O_m>;  dP_ms = <dO_m, V_s>;  dS = P * (dP - Delta)
 * Since O_m = sum_s P_ms V_s, Delta_m also equals sum_s P_ms dP_ms; the
 * matrix-core kernels (bf16/f16 with nk = 48) take it in that form from the
 * fp32 P and dP they compute anyway, so they do not read o (the vector-ALU
 * kernels for f32 and other list lengths read it).
 *   dQ_m = scale sum_s dS_ms K_s
 *   dK_j = scale sum over every (cluster, slot) whose key is j of dS Q
 *   dV_j = sum over the same slots of P dO
 * Two passes: a query-major pass writes dQ and Delta, a key-major pass over a
 * transposed slot list (built in the workspace each call) writes dK and dV
 * directly, so no atomics touch the gradients and the result is bitwise
 * reproducible.  fp32 accumulation throughout; P and dS are rounded once to
 * dt as operands of the dV, dK and dQ products (bf16/f16); outputs RNE to dt.
 *   q, k, v, o, dout [B, N, H, D] dt (o as returned by the forward; not
 *             read by the matrix-core kernels, but always a valid pointer).
 *   lse       [B, N, H] f32 from the forward.
 *   dq, dk, dv [B, N, H, D] dt out.
 *   ws        device workspace of at least cluster_attn_bwd_workspace(...)
 *             bytes; contents on entry are ignored.  Two calls that overlap
 *             in time must not share a workspace.
 */
ca_status cluster_attn_bwd(int dt, int B, int N, int H, int D, int cs, int nk, float scale,
                     const void* q, const void* k, const void* v, const void* o,
                     const void* dout, const float* lse, const int32_t* q_idx,
                     const int32_t* key_idx, void* dq, void* dk, void* dv, void* ws,
                     size_t ws_bytes, void* hip_stream);

/*
 * The backward's transposed (key-major) slot lists depend on q_idx and
 * key_idx alone, like the lists themselves (which change only where tokens
 * are merged, so one build serves every attention layer of a stage).  A
 * caller that runs several backward passes on the same lists can build
 * them once:
 *   cluster_attn_bwd_plan      writes them into `plan` (device, at least
 *                              cluster_attn_bwd_plan_workspace bytes).
 *   cluster_attn_bwd_planned   is cluster_attn_bwd with that plan as an
 *                              input; its own workspace `ws` then only
 *                              holds the per-call LSE/Delta pairs
 *                              (cluster_attn_bwd_planned_workspace bytes).
 * Sizes: B images of N tokens and C clusters each, C = ceil(N/cs); a packed
 * batch (cluster_attn_*_varlen) is B = 1, N = T, C = Ct.  A plan must not
 * be used with lists other than the ones it was built from (not checked).
 * The result equals cluster_attn_bwd's bit for bit.
 */
size_t cluster_attn_bwd_plan_workspace(int B, int N, int C, int cs, int nk);
ca_status cluster_attn_bwd_plan(int B, int N, int C, int cs, int nk, const int32_t* q_idx,
                          const int32_t* key_idx, void* plan, size_t plan_bytes,
                          void* hip_stream);
/* The plan of a packed batch from its offsets (see
 * cluster_attn_build_neighbors_varlen): one workgroup per image when every
 * image has at most 4096 tokens, else the batch as one index space.  The
 * plan has the size cluster_attn_bwd_plan_workspace(1, T, Ct, cs, nk) and
 * feeds cluster_attn_bwd_planned with B = 1, N = T, C = Ct. */
ca_status cluster_attn_bwd_plan_varlen(int B, int T, int Ct, int max_n, const int32_t* tok_off,
                                 const int32_t* clu_off, int cs, int nk, const int32_t* q_idx,
                                 const int32_t* key_idx, void* plan, size_t plan_bytes,
                                 void* hip_stream);
size_t cluster_attn_bwd_planned_workspace(int dt, int B, int N, int H, int D);
ca_status cluster_attn_bwd_planned(int dt, int B, int N, int C, int H, int D, int cs, int nk,
                             float scale, const void* q, const void* k, const void* v,
                             const void* o, const void* dout, const float* lse,
                             const int32_t* q_idx, const int32_t* key_idx, const void* plan,
                             size_t plan_bytes, void* dq, void* dk, void* dv, void* ws,
                             size_t ws_bytes, void* hip_stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * cluster_attn_bwd_planned without the workspace argument.  The per-call
 * LSE/Delta pairs go to a scratch array compiled into the library (32 MiB,
 * one copy per GPU, resident from module load until the process ends, its
 * address looked up once per device with hipGetSymbolAddress); nothing is
 * allocated and nothing needs clearing (pass A writes every pair pass B
 * reads).  B*N*H may be at most cluster_attn_bwd_planned_noalloc_max_rows()
 * (4,194,272), else CA_ERR_WORKSPACE.  Every call on one GPU uses the same
 * scratch: calls that overlap on one GPU (different streams, or host
 * threads) race and must be serialised by the caller.  The stream must
 * belong to the current device.  Other arguments, outputs and results are
 * those of cluster_attn_bwd_planned, bit for bit. */
size_t cluster_attn_bwd_planned_noalloc_max_rows(void);
ca_status cluster_attn_bwd_planned_noalloc(int dt, int B, int N, int C, int H, int D, int cs,
                                           int nk, float scale, const void* q, const void* k,
                                           const void* v, const void* o, const void* dout,
                                           const float* lse, const int32_t* q_idx,
                                           const int32_t* key_idx, const void* plan,
                                           size_t plan_bytes, void* dq, void* dk, void* dv,
                                           void* hip_stream);

/*
 * Forward and backward of a packed batch (see
 * cluster_attn_build_neighbors_varlen): the same computation as
 * cluster_attn_fwd / cluster_attn_bwd with the whole batch as one index
 * space of T tokens and Ct clusters (lists never cross images, so nothing
 * mixes images).  q, k, v, o, dout, dq, dk, dv are [T, H, D] dt, lse
 * [T, H] f32, q_idx [Ct, cs] and key_idx [Ct, nk] int32 with batch-global
 * token ids; ceil(T / cs) <= Ct <= T.
 */
ca_status cluster_attn_fwd_varlen(int dt, int T, int Ct, int H, int D, int cs, int nk, float scale,
                            const void* q, const void* k, const void* v, const int32_t* q_idx,
                            const int32_t* key_idx, void* o, float* lse, void* hip_stream);
size_t cluster_attn_bwd_varlen_workspace(int dt, int T, int Ct, int H, int D, int cs, int nk);
ca_status cluster_attn_bwd_varlen(int dt, int T, int Ct, int H, int D, int cs, int nk, float scale,
                            const void* q, const void* k, const void* v, const void* o,
                            const void* dout, const float* lse, const int32_t* q_idx,
                            const int32_t* key_idx, void* dq, void* dk, void* dv, void* ws,
                            size_t ws_bytes, void* hip_stream);

/* ------------------------------------------------------------------------
 * KNN-cache point sampler of the point-wise decoder.
 *
 * Notes page, "Key Designs" item 2 (point-wise deformable cross-attention
 * decoder: a query samples at q = r + offset and aggregates its nearest
 * visible tokens with weights w_i = softmax_i(-p d_i), the stable
 * replacement of inverse-power weights) and item 3 (KNN cache lookup: an
 * H x W x K table holding, per grid cell, the K nearest visible tokens; a
 * query is quantised to its nearest cell so that neighbour retrieval is a
 * lookup plus a distance calculation, fused with the softmax weighting in
 * the forward and the backward).  Readings: H = W = G, the token grid;
 * cell (row i, column j) has its centre at (x, y) = (j, i); distances for
 * the table are those of the 16-bit fixed-point coordinates of the neighbour
 * build (ties to the lower token index); d_k of the weights is the Euclidean
 * distance of the f32 coordinates.  Coordinates and queries are
 * (x = column, y = row) in patch units, [B, N, 2] / [B, M, 2] f32.  Feature
 * tensors are read and written in 16-byte pieces: their pointers must be
 * 16-byte aligned (C is a multiple of 8).
 * ------------------------------------------------------------------------ */

/* Workspace bytes needed by cluster_attn_knn_table (0 for images of at most
 * 4096 tokens, and for invalid sizes). */
size_t cluster_attn_knn_table_workspace(int B, int N, int grid_side);

/*
 * Table: table[b, i, j, 0..K-1] = the K tokens of image b whose fixed-point
 * coordinates (q = clamp(floor((c + 0.5) * 2^(16 - ceil(log2 G))), 0,
 * 65535) per axis) are nearest to the cell centre ((j + 1/2) s, (i + 1/2) s),
 * s = 2^(16 - ceil(log2 G)), by (squared distance, token index) ascending;
 * -1 pads rows when N < K.  Exact integer arithmetic: the unique table.
 *   coords  [B, N, 2] f32 device.   G: 1..2048.   N: 0..2^24 (B*N < 2^31).
 *   K: 1..16.
 *   table   [B, G, G, K] int32 device out.
 *   ws      device workspace of cluster_attn_knn_table_workspace bytes
 *           (images above 4096 tokens are bucketed there; NULL when 0);
 *           two calls that overlap in time must not share it.
 */
ca_status cluster_attn_knn_table(const float* coords, int B, int N, int grid_side, int K,
                                 int32_t* table, void* ws, size_t ws_bytes, void* hip_stream);

/*
 * Forward: for query m of image b at q = queries[b, m], the cell is
 * (i, j) = (clamp(floor(q.y + 1/2), 0, G-1), clamp(floor(q.x + 1/2), 0, G-1))
 * (fp64); over the valid slots t_k = table[b, i, j, k] >= 0,
 *   d_k = |q - coords[b, t_k]|,  w = softmax(-p d) (fp32, max subtracted),
 *   out[b, m, :] = sum_k w_k feats[b, t_k, :]   (fp32 accumulation, RNE to dt);
 * a query whose row has no valid slot gets 0.
 *   dt     element type of feats and out.   C: channels, multiple of 8, <= 1024.
 *   p      finite real (one per level).     K: 1..16 (table's K).   G: 1..2048.
 *   N, M   up to 2^24 each (B*M*K < 2^31).
 *   feats  [B, N, C] dt.   table [B, G, G, K] int32 (any contents in [-1, N)).
 *   out    [B, M, C] dt out.
 */
ca_status cluster_attn_knn_sample_fwd(int dt, int B, int N, int M, int C, int grid_side, int K, float p,
                                const float* coords, const void* feats, const float* queries,
                                const int32_t* table, void* out, void* hip_stream);

/* Workspace bytes needed by cluster_attn_knn_sample_bwd (0 for invalid sizes). */
size_t cluster_attn_knn_sample_bwd_workspace(int B, int N, int M, int K);

/*
 * Backward of L = sum(dout * out) with the table held fixed: with
 * g_k = <dout[b, m], feats[b, t_k]> and ds_k = w_k (g_k - sum_j w_j g_j),
 *   dq[b, m]     = -p sum_k ds_k (q - x_k) / d_k   (terms with d_k = 0 are 0)
 *   dp           = -sum over all queries and slots of ds_k d_k
 *   dfeats[b, t] = sum over the (query, slot) pairs holding t of w_k dout[b, m]
 * The token coordinates are constants.  dfeats is built token-major from a
 * transposed slot list made in the workspace (entries ordered by query and
 * slot) and written once, with no atomics on floating-point values: the
 * result is bitwise reproducible.  fp32 accumulation; dfeats RNE to dt.
 *   dout    [B, M, C] dt.   dfeats [B, N, C] dt out (tokens no query reaches
 *           get 0).   dq [B, M, 2] f32 out.   dp: one f32 out (device).
 *   ws      device workspace of cluster_attn_knn_sample_bwd_workspace bytes;
 *           two calls that overlap in time must not share it.
 * Cost: for images above 4096 tokens the entries of tokens referenced up
 * to 256 times are ranked against their token's entries, those of more
 * referenced tokens radix-sorted (a workgroup per token), so the time stays
 * near linear in the entry count however the queries concentrate.
 */
ca_status cluster_attn_knn_sample_bwd(int dt, int B, int N, int M, int C, int grid_side, int K, float p,
                                const float* coords, const void* feats, const float* queries,
                                const int32_t* table, const void* dout, void* dfeats, float* dq,
                                float* dp, void* ws, size_t ws_bytes, void* hip_stream);

/* ------------------------------------------------------------------------
 * Adaptive off-grid token merging.
 *
 * Notes page, "Key Designs" item 1: every token keeps its 2D coordinate; a
 * lightweight MLP scores the tokens, the top-k by the retention rate are
 * kept as anchors, and the other tokens are merged, differentiably, into
 * their nearest anchors, features and spatial support alike ("A Complete
 * Example": retention 0.4, 2048 -> 819 -> 328 -> 131 tokens).  Readings: the
 * scores are an input; anchors are the k largest scores (ties to the lower
 * token index) in ascending token order; an anchor is assigned to itself and
 * every other token to the anchor nearest by squared distance of the 16-bit
 * fixed-point coordinates of the neighbour build (ties to the earlier
 * anchor); within a group the softmax of the members' scores weighs the
 * features and the coordinates.  N <= 2^24 tokens per image (B*N < 2^31);
 * scores finite.
 * ------------------------------------------------------------------------ */

/* Workspace bytes needed by cluster_attn_merge_plan (0 for images of at most
 * 4096 tokens, and for invalid sizes). */
size_t cluster_attn_merge_plan_workspace(int B, int N, int k);

/*
 * Plan (exact integers; the unique result of the rules above):
 *   coords [B, N, 2] f32, scores [B, N] f32.   1 <= k <= N.   grid_side: G.
 *   anchors [B, k] int32 out: token index of anchor a, ascending.
 *   assign  [B, N] int32 out: anchor position of every token.
 *   members [B, N] int32 out, offsets [B, k + 1] int32 out: the tokens of
 *           group a are members[offsets[a] .. offsets[a+1]), in token order.
 *   ws      device workspace of cluster_attn_merge_plan_workspace bytes
 *           (images above 4096 tokens are planned there; NULL when 0); two
 *           calls that overlap in time must not share it.
 * Cost: above 4096 tokens the members of groups of up to 256 tokens are
 * ranked against their group, larger groups are radix-sorted (a workgroup
 * per group), so the time stays near linear in N for any grouping.
 */
ca_status cluster_attn_merge_plan(const float* coords, const float* scores, int B, int N, int k,
                                  int grid_side, int32_t* anchors, int32_t* assign,
                                  int32_t* members, int32_t* offsets, void* ws, size_t ws_bytes,
                                  void* hip_stream);

/*
 * Forward: w_i = exp(s_i) / sum over the group of exp(s_j) (max subtracted,
 * fp32);  out_feats[b, a] = sum_i w_i feats[b, i]  (dt, RNE from fp32),
 * out_coords[b, a] = sum_i w_i coords[b, i]  (f32).
 *   feats [B, N, C] dt (16-byte aligned, C a multiple of 8 up to 1024);
 *   members/offsets as returned by cluster_attn_merge_plan.
 */
ca_status cluster_attn_merge_fwd(int dt, int B, int N, int k, int C, const void* feats,
                           const float* coords, const float* scores, const int32_t* members,
                           const int32_t* offsets, void* out_feats, float* out_coords,
                           void* hip_stream);

/*
 * Backward of L = sum(dout_feats * out_feats) + sum(dout_coords * out_coords)
 * with the plan held fixed: for token i of group a, with
 * g_i = <dout_feats[a], feats[i]> + <dout_coords[a], coords[i]>,
 *   dfeats[i] = w_i dout_feats[a],  dcoords[i] = w_i dout_coords[a],
 *   dscores[i] = w_i (g_i - sum_{j in a} w_j g_j).
 * Every token belongs to one group and is written once (no atomics):
 * bitwise reproducible.  dfeats dt; dcoords, dscores f32.
 */
ca_status cluster_attn_merge_bwd(int dt, int B, int N, int k, int C, const void* feats,
                           const float* coords, const float* scores, const int32_t* members,
                           const int32_t* offsets, const void* dout_feats,
                           const float* dout_coords, void* dfeats, float* dcoords,
                           float* dscores, void* hip_stream);

/*
 * Debug helper, HOST pointers: checks index lists before they reach a
 * kernel, which reads them unchecked (the conventions above make valid
 * lists a precondition of every attention call).  For B images of N
 * tokens in C clusters (C = ceil(N/cs); a packed batch is B = 1, N = T,
 * C = Ct), q_idx [B, C, cs] and key_idx [B, C, nk] (key_idx may be NULL
 * when nk = 0):
 *   - every q_idx value is a token in [0, N) or -1; member 0 of each row is
 *     a token and no token follows a -1 in its row;
 *   - every token of an image appears exactly once in its q_idx rows;
 *   - every key_idx value is in [-1, N).
 * Returns CA_OK, or CA_ERR_SHAPE with the first offending position in
 * cluster_attn_last_error().  Runs on the calling thread; allocates N bytes
 * of host memory for the duration of the call.
 */
ca_status cluster_attn_check_lists(int B, int N, int C, int cs, int nk, const int32_t* q_idx,
                                   const int32_t* key_idx);

/*
 * Measurement utility: copies `bytes` bytes from `src` to `dst` (device
 * pointers, 16-byte aligned, not overlapping) with a plain streaming kernel
 * of 16-byte loads and stores.  Timing it gives the HBM bandwidth this
 * device actually achieves, the second reference (beside the vendor peak)
 * for the attention kernels' effective bandwidth.  Asynchronous on
 * `hip_stream`.  CA_ERR_NULL / CA_ERR_UNSUPPORTED (misaligned) /
 * CA_ERR_ALIAS (overlap) / CA_ERR_HIP.
 */
ca_status cluster_attn_device_copy(void* dst, const void* src, size_t bytes, void* hip_stream);

/* Static text for a status code. */
const char* cluster_attn_status_string(int status);

/* Detail of the last error on the calling thread ("" if none). */
const char* cluster_attn_last_error(void);

/* Library version string. */
const char* cluster_attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CLUSTER_ATTN_H */
