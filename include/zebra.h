/*
 * zebra.h - C ABI of the MI355X (gfx950) library for Zebra3D's layerwise
 * hybrid global attention.
 *
 * Every global-attention stage of a feed-forward 3D backbone runs one of two
 * operators (Zebra3D paper page, thelatestinai.com: Abstract and Figure 1):
 *   - tile-sparse softmax attention: each query tile attends exactly to the
 *     tokens of its kept key tiles, and every omitted key tile enters as one
 *     mean-key/mean-value landmark;
 *   - linear attention with the feature map elu(x)+1, followed by a
 *     per-head, per-channel affine map fitted in closed form (news.hamidun.com
 *     article "Zebra3D speeds up 3D reconstruction...", section "How Zebra3D
 *     works"; paper page Table 3(a)).
 *
 * Conventions shared by every call:
 *   - Tensor arguments are DEVICE pointers owned by the caller. The library
 *     allocates nothing and keeps no state between calls. Scratch memory is
 *     a caller-provided device workspace whose size the *_workspace() query
 *     returns.
 *   - A token sequence is described by zebra_seq: element (h, n, c) of a
 *     tensor lives at base[h * stride_head + n * stride_token + c]. The
 *     channel dimension is contiguous. Strides are in elements; for bf16
 *     tensors the base must be 16-byte aligned and both strides multiples
 *     of 8.
 *   - head_dim must be 64 (ZEBRA_ERR_UNSUPPORTED otherwise).
 *   - `stream` is a hipStream_t passed as void*; NULL is the default stream.
 *     Calls enqueue work on that stream and return without synchronising.
 *   - Arguments are validated before any HIP call; a bad argument returns a
 *     status code and enqueues nothing. Launch failures return ZEBRA_ERR_HIP.
 *   - Outputs are fully overwritten and must not overlap any input.
 *     Non-finite inputs give undefined results.
 *   - Results are deterministic: the same inputs give bitwise identical
 *     outputs (no floating-point atomics).
 */
#ifndef ZEBRA_H_
#define ZEBRA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ZEBRA_ABI_VERSION 1

typedef enum zebra_status {
  ZEBRA_OK = 0,
  ZEBRA_ERR_INVALID_ARG = 1, /* null pointer, negative size, overlap, bad top_k */
  ZEBRA_ERR_UNSUPPORTED = 2, /* valid request outside the implemented shapes  */
  ZEBRA_ERR_WORKSPACE = 3,   /* workspace smaller than the query returned      */
  ZEBRA_ERR_HIP = 4          /* the HIP runtime rejected a launch              */
} zebra_status;

typedef enum zebra_dtype { ZEBRA_BF16 = 0, ZEBRA_F32 = 1 } zebra_dtype;

typedef struct zebra_seq {
  int64_t n_tokens;     /* N, tokens per head (0 allowed: nothing to do)   */
  int32_t n_heads;      /* H                                               */
  int32_t head_dim;     /* d, must be 64                                   */
  int64_t stride_token; /* elements between consecutive tokens of a head   */
  int64_t stride_head;  /* elements between consecutive heads              */
} zebra_seq;

/*
 * Tile pooling (landmarks). Zebra3D paper page, Figure 1 caption: omitted
 * key/value tiles are summarised by their mean key and mean value.
 *
 * x        bf16 sequence described by xs.
 * tile     tokens per tile, 1..1024. Tile t covers tokens
 *          [t*tile, min((t+1)*tile, N)); the last tile may be short and is
 *          averaged over its valid tokens only.
 * mean_out float32 [H][T][64], T = ceil(N / tile), contiguous.
 * The same call pools query tiles (for the tile scores) and key/value tiles
 * (the landmarks). Accumulation is in float32.
 */
zebra_status zebra_pool_landmarks(const void* x, zebra_seq xs, int32_t tile, float* mean_out,
                                  void* stream);

/*
 * Tile selection. The tile-sparse stage computes only selected blocks
 * (news.hamidun.com article, "How Zebra3D works"). Score of query tile i and
 * key tile j: s_ij = qbar_i . kbar_j (float32, unscaled). For each (head, i)
 * the top_k key tiles are kept under the order (s_ij descending, j ascending),
 * so equal scores go to the lower tile index.
 *
 * qbar     float32 [H][t_q][64], kbar float32 [H][t_k][64], contiguous
 *          (the outputs of zebra_pool_landmarks).
 * top_k    1..t_k; t_k at most 32768.
 * sel_out  int32 [H][t_q][top_k], each row in ascending tile order.
 * workspace at least zebra_select_tiles_workspace(H, t_q, t_k) bytes (the
 *          float32 score matrix, rows padded to a multiple of 32 scores).
 */
size_t zebra_select_tiles_workspace(int32_t n_heads, int32_t t_q, int32_t t_k);
zebra_status zebra_select_tiles(const float* qbar, const float* kbar, int32_t n_heads,
                                int32_t t_q, int32_t t_k, int32_t head_dim, int32_t top_k,
                                int32_t* sel_out, void* workspace, size_t workspace_bytes,
                                void* stream);

/*
 * Tile-sparse softmax attention with landmarks. Zebra3D paper page, Figure 1
 * caption: kept tiles retain full softmax interactions and omitted tiles
 * become mean-key/value landmarks. For each query q of query tile i:
 *   columns  = every token of every kept key tile j in sel[h][i][*]
 *              + one landmark (kbar_j, vbar_j) for each omitted tile j,
 *   o(q)     = softmax(scale * q . key over columns) . value over columns.
 * A landmark is one ordinary softmax column (no multiplicity weight).
 *
 * q        bf16 query sequence (qs); k, v bf16 key/value sequences sharing kvs.
 *          qs and kvs must have the same n_heads and head_dim; the query and
 *          key sequences may differ in length.
 * kbar     float32 [H][t_k][64] mean keys, vbar mean values (from
 *          zebra_pool_landmarks with k_tile); NULL iff top_k == t_k.
 * sel      int32 [H][t_q][top_k] kept tiles, each row strictly ascending
 *          (from zebra_select_tiles); NULL iff top_k == t_k, which is exact
 *          dense softmax attention.
 * q_tile   32, 64 or 128 query tokens per tile; t_q = ceil(Nq / q_tile).
 * k_tile   32 or 64 key tokens per tile; t_k = ceil(Nk / k_tile) <= 32768.
 * scale    softmax scale (1/sqrt(64) = 0.125 for the pages' backbones).
 * o        output sequence (os, same H and d as qs, n_tokens == qs.n_tokens),
 *          bf16 or float32 per o_dtype. Softmax statistics and accumulators
 *          are float32; products run on bf16 MFMA.
 * workspace at least zebra_tile_sparse_attn_workspace(Nq, Nk, H, 64, q_tile,
 *          k_tile, top_k) bytes, 16-byte aligned: the landmarks as bf16 (when
 *          top_k < t_k) and per-head maxima of the key norms and value
 *          magnitudes. For long key ranges with q_tile <= 64 (at least
 *          2 x 32768 keys, top_k < t_k) the keys are processed in chunks of
 *          32768 keys (65536 from 4 x 65536 keys on) and the workspace also
 *          holds float32 partial outputs, H x Nq x slots x 264 bytes, one
 *          slot per chunk plus, for 64-query and 64-key tiles with
 *          landmarks, one for the landmark columns; at most 64 GiB
 *          (33.2 GiB for 16 heads of 703,488 tokens). Never 0;
 *          the contents on return are unspecified.
 * The key/value token stride must be at most 2^24 elements
 * (ZEBRA_ERR_UNSUPPORTED otherwise).
 */
size_t zebra_tile_sparse_attn_workspace(int64_t n_q, int64_t n_kv, int32_t n_heads,
                                        int32_t head_dim, int32_t q_tile, int32_t k_tile,
                                        int32_t top_k);
zebra_status zebra_tile_sparse_attn(const void* q, zebra_seq qs, const void* k, const void* v,
                                    zebra_seq kvs, const float* kbar, const float* vbar,
                                    const int32_t* sel, int32_t q_tile, int32_t k_tile,
                                    int32_t top_k, float scale, void* o, zebra_seq os,
                                    zebra_dtype o_dtype, void* workspace,
                                    size_t workspace_bytes, void* stream);

/*
 * Variants of the sparse operator from the pages' ablations (Zebra3D paper
 * page, Table 3(b); appendix Tables 15-17 compare block/tile sparse attention
 * with and without landmarks). flags = 0 is zebra_tile_sparse_attn.
 *   ZEBRA_SPARSE_NO_LANDMARKS       omitted tiles are dropped: softmax over the
 *                                   kept tiles' tokens only; kbar and vbar are
 *                                   not read and may be NULL.
 *   ZEBRA_SPARSE_LANDMARK_LOG_COUNT a landmark stands for the n_j valid tokens
 *                                   of its tile: its logit gains ln(n_j).
 * The two flags are exclusive (ZEBRA_ERR_INVALID_ARG). Everything else,
 * including the workspace size, is as for zebra_tile_sparse_attn. With
 * top_k == t_k (dense attention) the flags have no effect.
 */
#define ZEBRA_SPARSE_NO_LANDMARKS 1u
#define ZEBRA_SPARSE_LANDMARK_LOG_COUNT 2u
zebra_status zebra_tile_sparse_attn_ex(const void* q, zebra_seq qs, const void* k, const void* v,
                                       zebra_seq kvs, const float* kbar, const float* vbar,
                                       const int32_t* sel, int32_t q_tile, int32_t k_tile,
                                       int32_t top_k, float scale, void* o, zebra_seq os,
                                       zebra_dtype o_dtype, uint32_t flags, void* workspace,
                                       size_t workspace_bytes, void* stream);

/*
 * zebra_tile_sparse_attn_ex that also writes each query's softmax normaliser,
 * for zebra_tile_sparse_attn_backward_lse (a training step keeps it from its
 * forward, as the refinement of a converted model would; Zebra3D paper page,
 * Tables 18-19). lse_out: float32 [H][Nq], contiguous, 4-byte aligned, caller
 * owned; lse[h][n] = log2 of sum_c 2^(w_c) over the columns c of query n, with
 * w_c = scale * log2(e) * q_n . key_c (+ log2 n_j for a landmark under
 * ZEBRA_SPARSE_LANDMARK_LOG_COUNT), the column weights of the forward's own
 * float32 sums. It must not overlap any other argument (ZEBRA_ERR_INVALID_ARG).
 * Output and workspace as for zebra_tile_sparse_attn_ex.
 */
zebra_status zebra_tile_sparse_attn_lse(const void* q, zebra_seq qs, const void* k, const void* v,
                                        zebra_seq kvs, const float* kbar, const float* vbar,
                                        const int32_t* sel, int32_t q_tile, int32_t k_tile,
                                        int32_t top_k, float scale, void* o, zebra_seq os,
                                        zebra_dtype o_dtype, uint32_t flags, float* lse_out,
                                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * Linear attention plus affine map. Tolerant stages run linear(-centered)
 * attention (Zebra3D paper page, Abstract; Table 3(a) "Linear-centered +
 * fit"). With phi(x) = elu(x) + 1 per channel:
 *   S = sum_n phi(k_n) v_n^T (64x64), z = sum_n phi(k_n),
 *   o_m = (phi(q_m)^T S) / (phi(q_m)^T z),  out_m = a (*) o_m + b.
 * q (qs) and k, v (kvs) bf16; the query sequence may differ in length from
 * the key/value sequence (the state comes from all of k, v).
 * aff_scale, aff_bias  float32 [H][64] or NULL (scale 1, bias 0).
 * o        output (os), bf16 or float32.
 * workspace at least zebra_linear_attn_workspace(Nk, H, 64) bytes (per-chunk
 *          partial states, reduced in a fixed order).
 */
size_t zebra_linear_attn_workspace(int64_t n_kv, int32_t n_heads, int32_t head_dim);
zebra_status zebra_linear_attn(const void* q, zebra_seq qs, const void* k, const void* v,
                               zebra_seq kvs, const float* aff_scale, const float* aff_bias,
                               void* o, zebra_seq os, zebra_dtype o_dtype, void* workspace,
                               size_t workspace_bytes, void* stream);

/*
 * zebra_linear_attn without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops or
 * harnesses that forbid hipMalloc). Same arguments, kernels and results as
 * zebra_linear_attn (bitwise), except that the partial and folded states live
 * in a fixed device array of zebra_linear_attn_noalloc_max_bytes() bytes
 * (40 MiB) that the library holds on each GPU it runs on until the process
 * ends; its device address is taken once per device on the first call there.
 * The call allocates nothing and frees nothing.
 *
 * Limit: zebra_linear_attn_workspace(Nk, H, 64) must not exceed that size
 * (true for up to 840 heads at any length); otherwise ZEBRA_ERR_WORKSPACE,
 * before any HIP call. Every call on one GPU shares that GPU's array and the
 * kernels overwrite it entirely (nothing must start at zero); calls that
 * overlap in time on one GPU (two streams, two threads) race on it and must
 * be serialised by the caller. ZEBRA_ERR_HIP if the array's address cannot be
 * taken on the current device.
 */
size_t zebra_linear_attn_noalloc_max_bytes(void);
zebra_status zebra_linear_attn_noalloc(const void* q, zebra_seq qs, const void* k, const void* v,
                                       zebra_seq kvs, const float* aff_scale,
                                       const float* aff_bias, void* o, zebra_seq os,
                                       zebra_dtype o_dtype, void* stream);

/*
 * Closed-form affine fit (news.hamidun.com article, "How Zebra3D works": the
 * linear components are fitted by a closed-form affine map, no gradient
 * descent). Per (head h, channel c), over the m samples:
 *   a = sum (x - xbar)(y - ybar) / sum (x - xbar)^2,  b = ybar - a xbar,
 * the least-squares solution of min sum (a x + b - y)^2. A channel with
 * sum (x - xbar)^2 <= 1e-30 * m gets a = 0, b = ybar. Statistics are
 * accumulated in float64.
 *
 * x, y     float32 [H][m][64], contiguous: x the linear output before the
 *          affine map, y the dense softmax output at the same m queries.
 * scale_out, bias_out  float32 [H][64].
 * n_degenerate_out     int32 [1] device counter of degenerate channels, or NULL.
 */
zebra_status zebra_fit_affine(const float* x, const float* y, int32_t m, int32_t n_heads,
                              int32_t head_dim, float* scale_out, float* bias_out,
                              int32_t* n_degenerate_out, void* stream);

/*
 * Gradients of one tile-sparse stage (for the optional refinement of a
 * converted model, Zebra3D paper page, Tables 18-19): for out of
 * zebra_tile_sparse_attn_ex with the same arguments and flags, the gradients
 * of sum(dout * out) with respect to q, k and v, the selection sel held fixed
 * (top-k is not differentiable). Per query row with columns c and
 * P = softmax over them:
 *   dP_c = dout . v_c,  D = dout . out,  dS_c = P_c (dP_c - D),
 *   dq = scale sum_c dS_c k_c,  dk_c = scale dS_c q,  dv_c = P_c dout,
 * and every token of tile j receives 1/n_j of its landmark column's dk and
 * dv (the landmark is the tile mean). The call runs the forward itself (its
 * float32 output and normaliser go to the workspace) and takes D from that
 * float32 output and the bf16-rounded dout; P comes from the normaliser as
 * the forward summed it (bf16-rounded probabilities). dout enters the bf16
 * MFMA products rounded to bf16, sums are float32 in a fixed order
 * (deterministic). sel is required (also when top_k == t_k).
 *
 * Arguments as zebra_tile_sparse_attn_ex, plus:
 * dout (dos)  output gradient [H][Nq][64], element type g_dtype.
 * dq (dqs), dk, dv (dkvs)  gradients, element type g_dtype (bf16 or float32).
 * workspace at least zebra_tile_sparse_attn_backward_workspace(Nq, Nk, H,
 *          64, q_tile, k_tile, top_k) bytes, 16-byte aligned (it includes the
 *          forward's workspace and 4 bytes per selection entry for the
 *          per-key-tile query lists). Outputs may not overlap the inputs or
 *          each other.
 */
size_t zebra_tile_sparse_attn_backward_workspace(int64_t n_q, int64_t n_kv, int32_t n_heads,
                                                 int32_t head_dim, int32_t q_tile, int32_t k_tile,
                                                 int32_t top_k);
zebra_status zebra_tile_sparse_attn_backward(
    const void* q, zebra_seq qs, const void* k, const void* v, zebra_seq kvs, const float* kbar,
    const float* vbar, const int32_t* sel, int32_t q_tile, int32_t k_tile, int32_t top_k,
    float scale, uint32_t flags, const void* dout, zebra_seq dos, zebra_dtype g_dtype, void* dq,
    zebra_seq dqs, void* dk, void* dv, zebra_seq dkvs, void* workspace, size_t workspace_bytes,
    void* stream);

/*
 * zebra_tile_sparse_attn_backward with the normaliser lse of an earlier
 * zebra_tile_sparse_attn_lse call on the same q, k, v, landmarks, selection,
 * tiles, scale and flags, for a forward whose output was bf16: the call
 * then does not run the forward itself (it packs the landmarks and copies lse
 * into its workspace). Without a float32 output at hand, a first pass over
 * every query's columns forms D = sum_c P_c dP_c and renormalises the copy of
 * lse so that the float32 P_c sum to one. The gradients agree with
 * zebra_tile_sparse_attn_backward to rounding (not bitwise). lse: float32
 * [H][Nq], contiguous, 4-byte aligned, read only. Workspace:
 * zebra_tile_sparse_attn_backward_workspace.
 */
zebra_status zebra_tile_sparse_attn_backward_lse(
    const void* q, zebra_seq qs, const void* k, const void* v, zebra_seq kvs, const float* kbar,
    const float* vbar, const int32_t* sel, int32_t q_tile, int32_t k_tile, int32_t top_k,
    float scale, uint32_t flags, const float* lse, const void* dout, zebra_seq dos,
    zebra_dtype g_dtype, void* dq, zebra_seq dqs, void* dk, void* dv, zebra_seq dkvs,
    void* workspace, size_t workspace_bytes, void* stream);

/*
 * zebra_tile_sparse_attn_backward from both saved results of an earlier
 * zebra_tile_sparse_attn_lse call with o_dtype ZEBRA_F32 on the same q, k, v,
 * landmarks, selection, tiles, scale and flags: its normaliser lse and its
 * float32 output out (os). The call does not run the forward; D comes from
 * out as in zebra_tile_sparse_attn_backward, so the gradients are bitwise
 * those of zebra_tile_sparse_attn_backward, with one pass over each query's
 * columns instead of the two of zebra_tile_sparse_attn_backward_lse (for a
 * training step that keeps the forward's output in float32; Zebra3D paper
 * page, Tables 18-19). lse: float32 [H][Nq], contiguous, 4-byte aligned.
 * out: float32 [H][Nq][64] with 16-byte aligned rows (ZEBRA_ERR_UNSUPPORTED
 * otherwise). Both are read only and must not overlap an output
 * (ZEBRA_ERR_INVALID_ARG); both are required unless Nq or H is 0. Workspace:
 * zebra_tile_sparse_attn_backward_workspace.
 */
zebra_status zebra_tile_sparse_attn_backward_saved(
    const void* q, zebra_seq qs, const void* k, const void* v, zebra_seq kvs, const float* kbar,
    const float* vbar, const int32_t* sel, int32_t q_tile, int32_t k_tile, int32_t top_k,
    float scale, uint32_t flags, const float* lse, const float* out, zebra_seq os,
    const void* dout, zebra_seq dos, zebra_dtype g_dtype, void* dq, zebra_seq dqs, void* dk,
    void* dv, zebra_seq dkvs, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Gradients of one linear stage (for the optional refinement of a converted
 * model, Zebra3D paper page, Tables 18-19): for out = a (*) o + b with o the
 * elu+1 linear attention of zebra_linear_attn, the gradients of
 * sum(dout * out) with respect to q, k, v, a and b. With num = phi(q) S,
 * den = phi(q) . z, do = a (*) dout:
 *   dq = (S dnum + z dden) (*) phi'(q),  dnum = do / den,
 *   dden = -(do . o) / den,  dS = sum phi(q) dnum^T,  dz = sum phi(q) dden,
 *   dv = dS^T phi(k),  dk = (dS v + dz) (*) phi'(k),
 *   da = sum dout (*) o,  db = sum dout,
 * phi'(x) = 1 for x > 0, e^x otherwise. All products and sums are float32
 * (partial sums over workgroups float64), deterministic.
 *
 * q (qs), k, v (kvs)  bf16 inputs of the forward call.
 * aff_scale   float32 [H][64], or NULL (a = 1). The bias does not enter.
 * dout (dos)  output gradient, [H][Nq][64], element type g_dtype.
 * dq (dqs), dk, dv (dkvs)  gradients, element type g_dtype (bf16 or float32).
 * d_scale, d_bias  float32 [H][64] gradients of a and b, or NULL (skipped).
 * workspace at least zebra_linear_attn_backward_workspace(Nq, Nk, H, 64)
 *          bytes, 16-byte aligned. Outputs may not overlap the inputs or
 *          each other.
 */
size_t zebra_linear_attn_backward_workspace(int64_t n_q, int64_t n_kv, int32_t n_heads,
                                            int32_t head_dim);
zebra_status zebra_linear_attn_backward(const void* q, zebra_seq qs, const void* k, const void* v,
                                        zebra_seq kvs, const float* aff_scale, const void* dout,
                                        zebra_seq dos, zebra_dtype g_dtype, void* dq,
                                        zebra_seq dqs, void* dk, void* dv, zebra_seq dkvs,
                                        float* d_scale, float* d_bias, void* workspace,
                                        size_t workspace_bytes, void* stream);

/*
 * Spatial tiles as a token permutation (Zebra3D paper page: softmax is kept
 * over selected spatial tiles, abstract; block- vs tile-sparse attention,
 * appendix Tables 15-17). Tiles are contiguous runs of the token order, so
 * spatial tiles come from a spatial order of the tokens: per view (n_special
 * leading tokens, then a grid_h x grid_w row-major patch grid; the VGGT-shaped
 * view is 5 + 37 x 37 = 1,374 tokens), the special tokens, then the patches
 * in block x block squares in raster order of squares, each square row-major
 * (squares at the right and bottom edges are smaller). Attention is
 * equivariant under a common permutation of queries and keys, so
 *   gather q, k, v by the order -> zebra_tile_sparse_attn -> scatter o back
 * is tile-sparse attention with spatial tiles, in the original token order.
 *
 * zebra_spatial_order: host function (no GPU, no stream). Writes
 *          order_out[i] = original index of the token at position i,
 *          order_len = n_views * (n_special + grid_h * grid_w) entries (host
 *          memory, owned by the caller). block >= 1.
 * zebra_permute_tokens: moves 64-channel rows on the device.
 *          inverse = 0: dst[h][i] = src[h][order[i]] (gather);
 *          inverse = 1: dst[h][order[i]] = src[h][i] (scatter, the inverse).
 *          src (ss) and dst (ds) have the same n_tokens and n_heads, element
 *          type dtype (bf16 or float32), 16-byte aligned rows; order is an
 *          int32 device vector of n_tokens entries, a permutation of
 *          [0, n_tokens): entries outside that range move nothing, repeated
 *          entries leave rows unwritten. dst may not overlap src or order.
 */
zebra_status zebra_spatial_order(int32_t n_views, int32_t n_special, int32_t grid_h,
                                 int32_t grid_w, int32_t block, int32_t* order_out,
                                 int64_t order_len);
zebra_status zebra_permute_tokens(const void* src, zebra_seq ss, const int32_t* order,
                                  int32_t inverse, zebra_dtype dtype, void* dst, zebra_seq ds,
                                  void* stream);

/*
 * Uncentered fit, the variant the Zebra3D paper page's Table 3(a) lists as
 * "Linear, uncentered fit": per (head h, channel c) the least-squares map
 * through the origin, min sum (a x - y)^2:
 *   a = sum x y / sum x^2,  b = 0.
 * A channel with sum x^2 <= 1e-30 * m gets a = 0. Arguments, layouts and
 * errors as zebra_fit_affine (bias_out is written with zeros).
 */
zebra_status zebra_fit_scale_only(const float* x, const float* y, int32_t m, int32_t n_heads,
                                  int32_t head_dim, float* scale_out, float* bias_out,
                                  int32_t* n_degenerate_out, void* stream);

/*
 * Selection-quality diagnostic: attention mass of every (query tile, key
 * tile) block under dense softmax. Zebra3D paper page, Figure 2 caption,
 * panel (b), and Figure 8 caption: the attention mass retained by the
 * highest-mass 20% of 64x64 token blocks. For query tile i and key tile j:
 *   mass[h][i][j] = (1/|Q_i|) sum_{q in Q_i} sum_{k in K_j} softmax_q(scale q . k),
 * so each row sums to one. Comparing sum_{j in sel_i} mass[h][i][j] with the
 * sum of the top_k largest entries of row i measures how much of the attention
 * mass the pooled-score selection keeps. Not on the forward path.
 *
 * q (qs) and k (ks) bf16 with the same n_heads; the sequences may differ in
 * length. q_tile 32, 64 or 128; k_tile 32 or 64; t_k = ceil(Nk / k_tile) at
 * most 32768. scale > 0.
 * mass_out float32 [H][t_q][t_k], contiguous. Row statistics (maximum and
 * sum per query) and masses are float32 from bf16 MFMA scores.
 * workspace at least zebra_block_mass_workspace(Nq, H) bytes, 16-byte aligned
 * (the per-query row statistics).
 */
size_t zebra_block_mass_workspace(int64_t n_q, int32_t n_heads);
zebra_status zebra_block_mass(const void* q, zebra_seq qs, const void* k, zebra_seq ks,
                              int32_t q_tile, int32_t k_tile, float scale, float* mass_out,
                              void* workspace, size_t workspace_bytes, void* stream);

/* Static strings; never NULL. */
const char* zebra_status_string(zebra_status status);
const char* zebra_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ZEBRA_H_ */
