/*
 * h3attn — TARA dense and pooled block-sparse attention for one packed
 * sequence, hand-written HIP for gfx950 (MI355X).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Rows:      one packed sequence [text | guide video | audio | output video]
 *            ("Flash Partitions for H3 native temporal alignment", section 1).
 * q, k, v, o [rows][heads][head_dim], contiguous, row stride heads*head_dim.
 * lse        [rows][heads] float32, natural log of the softmax normaliser.
 *            A row sub-range of q/o/lse is a plain pointer offset.
 * seg        [rows] uint8: 0 text (incl. padding), 1 guide video, 2 audio,
 *            3 output video.
 * t          [rows] float32 seconds (video frame k at k/6 s; 0 elsewhere).
 * dtype      H3_DTYPE_F32 (0) or H3_DTYPE_BF16 (1, raw bf16 bit patterns).
 * Pointers   named *_host are host memory; every other data pointer is device
 *            memory on the current HIP device.
 * stream     a hipStream_t (NULL = the null stream). Calls are stream-ordered
 *            and asynchronous: they never synchronise with the host, and
 *            results are valid once the stream has completed.
 * Ownership  the caller allocates every buffer, including workspaces sized by
 *            the *_workspace functions. The library allocates no device
 *            memory and keeps no global state; calls are re-entrant. Calls
 *            that share a workspace must be ordered on one stream.
 * Errors     every argument check runs before any HIP call, so a bad call
 *            returns without touching the device. Nothing throws across the
 *            boundary.
 * Forced     failure injection for a caller's dense fallback ("H3 SLA
 * failures   Attention", "Install": when the sparse kernel fails, the run
 *            degrades to plain dense attention). The environment variable
 *            H3ATTN_FORCE_FAIL holds a comma-separated list of call families:
 *            "dense" (attn_dense_tara, attn_dense_tara_via), "router" (the
 *            attn_block_router* calls) and "sparse" (the attn_block_sparse*
 *            calls). Entry points of a listed family return H3_EFORCED after
 *            their argument checks and before any HIP call. It is read on
 *            every call.
 */
#ifndef H3ATTN_H
#define H3ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define H3_OK            0
#define H3_EINVAL       (-1)  /* null pointer, bad size, non-finite or out-of-range knob */
#define H3_EUNSUPPORTED (-2)  /* dtype, head_dim not in {64,128}, block_size not in {32,64,128} */
#define H3_ELAUNCH      (-3)  /* a kernel launch failed (hipGetLastError) */
#define H3_EWORKSPACE   (-4)  /* workspace pointer null or smaller than required */
#define H3_ENOMEM       (-5)  /* host memory for a call's plan could not be allocated */
#define H3_EFORCED      (-6)  /* failure forced by H3ATTN_FORCE_FAIL (note above) */
#define H3_ESCRATCH     (-7)  /* larger than the static scratch of attn_block_router_static */

#define H3_DTYPE_F32  0
#define H3_DTYPE_BF16 1

#define H3_SEG_TEXT   0
#define H3_SEG_GUIDE  1
#define H3_SEG_AUDIO  2
#define H3_SEG_OUTPUT 3

/* Library version (major*10000 + minor*100 + patch). */
int h3attn_version(void);

/* Static text naming a status code. */
const char* h3attn_status_string(int status);

/*
 * Dense TARA attention.
 * Defined by "Flash Partitions for H3 native temporal alignment", section 1
 * (restated in "TARA : alignement temporel natif pour les références MiniMax
 * H3", "La règle temporelle"): for query row i and key row j of head h,
 *   s_ij = scale * (q_i . k_j) - p_ij,
 *   p_ij = min(strength * (max(|t_i - t_j| - window, 0) / falloff)^2, cap)
 *          when q_seg[i] == output video and k_seg[j] == guide video, else 0,
 *   o_i  = sum_j softmax_j(s_ij) v_j,   lse_i = ln sum_j exp(s_ij).
 * The penalty is evaluated in registers per score tile; no rows x rows bias
 * is ever formed. strength == 0 or cap == 0 gives plain attention (section 4).
 * Queries are nq rows of q (with q_seg/q_t), keys nk rows of k and v (with
 * k_seg/k_t); pass the same rows for self-attention or sub-ranges for
 * partition calls.
 * o_dtype: H3_DTYPE_F32 or H3_DTYPE_BF16 (bf16 rounding to nearest even).
 * head_dim 64 or 128. fp32 inputs run a float32 path (no bf16 rounding);
 * bf16 inputs use bf16 matrix cores with float32 accumulation.
 * Workspace: attn_dense_tara_workspace(nk, heads, head_dim, dtype) bytes
 * (0 for fp32); it holds a transposed copy of v used by the matrix cores.
 * Errors: H3_EINVAL for null pointers, nq/nk/heads <= 0, non-finite knobs,
 * strength/window/cap < 0, falloff <= 0, scale <= 0; H3_EUNSUPPORTED for a
 * dtype or head_dim outside the lists above, more than 65,535 heads, or bf16
 * inputs with more than 8,388,608 keys (32-bit addressing of the transposed v
 * copy); H3_EWORKSPACE; H3_ELAUNCH.
 */
size_t attn_dense_tara_workspace(int nk, int heads, int head_dim, int dtype);
int attn_dense_tara(const void* q, const void* k, const void* v, int dtype,
                    int nq, int nk, int heads, int head_dim,
                    const uint8_t* q_seg, const float* q_t,
                    const uint8_t* k_seg, const float* k_t,
                    float strength, float window, float falloff, float cap, float scale,
                    void* o, int o_dtype, float* lse,
                    void* ws, size_t ws_bytes, void* stream);

/*
 * Block size of the router and the block-sparse calls: 32, 64 or 128 rows
 * ("H3 SLA Attention", inputs table, block_size: the number of rows that share
 * one key selection). Query blocks and key blocks have the same size, and the
 * same rules hold at each size. A sequence may have at most 14,000 blocks of
 * that size and at most 896,000 rows.
 */

/*
 * Router plan (host only, no HIP call).
 * From "H3 SLA Attention" ("How it works", "The inputs that matter", inputs
 * table) and "H3 sparse-attention breakpoints" (the density is a fraction of
 * the video KV tiles; text and audio are not reduced): the sequence is cut
 * into nb = ceil(n / block_size) blocks (the last may be partial). A block is
 * protected when it overlaps rows [0, protected_prefix_len) or holds any text
 * or audio row; all other blocks are video tiles. The routed count is
 *   k = min(n_video, max(1, ceil((1 - sparsity_ratio) * n_video - 1e-9))),
 * k = n_video when sparsity_ratio == 0, and 0 when n_video == 0.
 * seg_host: [n] host segment ids. Outputs may be NULL when not wanted.
 * Errors: H3_EINVAL (seg_host null, n <= 0, protected_prefix_len not in
 * [0, n], sparsity_ratio not in [0, 1) or non-finite); H3_EUNSUPPORTED
 * (block_size not in {32, 64, 128}).
 */
int attn_router_plan(const uint8_t* seg_host, int n, int protected_prefix_len, int block_size,
                     double sparsity_ratio, int* nb, int* n_video, int* n_prot, int* k_sel);

/*
 * Reference protection ("H3 SLA Attention", inputs table, reference_protection). The
 * guide video is the visual reference of the packed sequence; a reference tile is a
 * video tile (see attn_router_plan) holding a guide row, and a reference range a
 * maximal run of reference tiles with consecutive block indices.
 *   H3_REF_OFF   no quota: reference tiles compete in the ordinary top-k.
 *   H3_REF_LIGHT the ordinary top-k over all video tiles, plus, for each reference
 *                range of m tiles, its best-scoring count(m, 0.85) tiles (a fixed
 *                reference sparsity of 0.85, i.e. 15% of the range); a query block
 *                attends the union.
 *   H3_REF_HEAVY every reference tile is protected (attended by every query block);
 *                the ordinary top-k runs over the other video tiles.
 * count(m, s) is the routed-count rule of attn_router_plan. Sparsity 0 still routes
 * every tile in every mode.
 */
#define H3_REF_OFF   0
#define H3_REF_LIGHT 1
#define H3_REF_HEAVY 2

/*
 * Router plan under a reference-protection mode (host only, no HIP call).
 * Outputs: nb; n_video = the routed candidates (the video tiles, without the
 * reference tiles under H3_REF_HEAVY); n_prot = the protected blocks (with the
 * reference tiles under H3_REF_HEAVY); k_sel = the list width
 * min(count(n_video, sparsity_ratio) + the sum of the Light quotas, n_video).
 * Errors: as attn_router_plan, plus H3_EUNSUPPORTED for an unknown mode or, under
 * H3_REF_LIGHT, more than 16 reference ranges.
 */
int attn_router_plan_ref(const uint8_t* seg_host, int n, int protected_prefix_len,
                         int block_size, double sparsity_ratio, int reference_protection,
                         int* nb, int* n_video, int* n_prot, int* k_sel);

/*
 * Pooled block router.
 * From "H3 SLA Attention", "How it works": one product of block-mean queries
 * with block-mean keys rates all (query block, key block) pairs; each query
 * block keeps its k highest-rated video tiles. Per head: qbar_b, kbar_b = mean
 * of the block's valid rows (float32 sums in row order from +0.0, then a
 * correctly rounded division by the row count); score(qb, kb) = sum over
 * d = 0..head_dim-1 of fl32(qbar[d] * kbar[d]) added in order, no fused
 * multiply-add, unscaled, over video tiles kb only; the k_sel highest scores are kept (ties to the lower block index,
 * NaN last) and written in ascending block order. Every query block is
 * routed, text and audio blocks included.
 * tiles: device int32 [heads][nb][k_sel], nb = ceil(n / block_size); entries
 *        past the device's video-tile count are -1.
 * prot:  device int32 [n_prot] ascending protected block indices; n_prot is the
 *        count from attn_router_plan on the same seg, and at most n_prot entries
 *        are written.
 * Workspace: attn_block_router_workspace(n, heads, head_dim, block_size).
 * Errors: as attn_router_plan, plus H3_EINVAL for null q/k/seg, null tiles
 * (k_sel > 0), null prot (n_prot > 0), k_sel < 0, k_sel > nb or n_prot < 0;
 * H3_EUNSUPPORTED for dtype/head_dim/block_size or more than 14,000 blocks;
 * H3_EWORKSPACE; H3_ELAUNCH.
 */
size_t attn_block_router_workspace(int n, int heads, int head_dim, int block_size);
int attn_block_router(const void* q, const void* k, int dtype, int n, int heads, int head_dim,
                      const uint8_t* seg, int protected_prefix_len, int block_size, int k_sel,
                      int32_t* tiles, int32_t* prot, int n_prot,
                      void* ws, size_t ws_bytes, void* stream);

/*
 * attn_block_router without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation). Its scratch (the block means, the video-tile list and counts) lives in a
 * static device array of H3_STATIC_SCRATCH_BYTES that the library holds on every GPU it
 * runs on until the process ends; the call allocates nothing. Inputs, outputs, rules and
 * results are those of attn_block_router.
 * Every call on one GPU shares that GPU's array: calls that overlap on one GPU (on
 * different streams, or from different threads) race and must be serialised by the
 * caller. Nothing in the array needs to start at zero.
 * Errors: as attn_block_router without H3_EWORKSPACE, plus H3_ESCRATCH when
 * attn_block_router_workspace(n, heads, head_dim, block_size) exceeds
 * H3_STATIC_SCRATCH_BYTES (checked before any HIP call).
 */
#define H3_STATIC_SCRATCH_BYTES (128u * 1024u * 1024u)
int attn_block_router_static(const void* q, const void* k, int dtype, int n, int heads,
                             int head_dim, const uint8_t* seg, int protected_prefix_len,
                             int block_size, int k_sel, int32_t* tiles, int32_t* prot,
                             int n_prot, void* stream);

/*
 * Pooled block router with reference protection (modes above). The scores, ranking,
 * ties and outputs are those of attn_block_router; each query block's list holds the
 * union of its selections in ascending order, padded with -1 to k_sel.
 * seg_host: host copy of seg (the reference ranges and quotas are planned on the host).
 * k_sel:    the list width from attn_router_plan_ref for the same arguments.
 * n_prot:   the protected count from attn_router_plan_ref (at most that many are
 *           written).
 * Workspace: attn_block_router_workspace(n, heads, head_dim, block_size).
 * Errors: as attn_block_router and attn_router_plan_ref, plus H3_EINVAL for a null
 * seg_host or a k_sel other than the plan's width.
 */
int attn_block_router_ref(const void* q, const void* k, int dtype, int n, int heads,
                          int head_dim, const uint8_t* seg, const uint8_t* seg_host,
                          int protected_prefix_len, int block_size, double sparsity_ratio,
                          int reference_protection, int k_sel, int32_t* tiles, int32_t* prot,
                          int n_prot, void* ws, size_t ws_bytes, void* stream);

/*
 * Block-sparse attention over routed tiles.
 * From "H3 SLA Attention", "How it works" and inputs table: query block qb of
 * head h attends the keys of the set of blocks formed by its protected blocks
 * prot[0..n_prot) and its routed blocks tiles[h][qb][0..k_sel), and nothing
 * else (a hard zero, no tail term). Blocks are block_size rows; tiles is
 * [heads][ceil(n / block_size)][k_sel]. Entries outside [0, ceil(n /
 * block_size)) are skipped and a block listed more than once counts once.
 * Inside those tiles the score is the dense TARA score of attn_dense_tara, so
 * the penalty applies to routed guide tiles of output-video queries when
 * strength > 0 and cap > 0.
 * Workspace: attn_block_sparse_workspace(n, heads, head_dim, dtype) bytes.
 * Errors: as attn_dense_tara, plus H3_EINVAL for k_sel < 0, n_prot < 0,
 * n_prot + k_sel == 0, null tiles (k_sel > 0) or prot (n_prot > 0);
 * H3_EUNSUPPORTED for block_size not in {32, 64, 128}, more than 14,000 blocks
 * or more than 896,000 rows.
 */
size_t attn_block_sparse_workspace(int n, int heads, int head_dim, int dtype);
int attn_block_sparse(const void* q, const void* k, const void* v, int dtype,
                      int n, int heads, int head_dim,
                      const uint8_t* seg, const float* t,
                      float strength, float window, float falloff, float cap, float scale,
                      int block_size, const int32_t* tiles, int k_sel,
                      const int32_t* prot, int n_prot,
                      void* o, int o_dtype, float* lse,
                      void* ws, size_t ws_bytes, void* stream);

/*
 * Routing with the pooled tail term.
 * From "H3 SLA Attention", inputs table (tail_correction): rather than dropping
 * the video tiles the top-k leaves out, one pooled term stands in for
 * all of them; its score reuses the block means that routing has formed.
 * Reading (the page gives no formula): for query block qb of head h and its
 * unrouted video tiles U,
 *   tail_lse[h][qb] = ln sum_{u in U} n_u * exp(scale * S[qb][u]),
 *   tail_v[h][qb][:] = sum_u n_u exp(scale * S[qb][u]) vbar_u / exp(tail_lse),
 * with S the float32 pooled score used for routing, n_u the rows of tile u and
 * vbar_u the float32 mean of its v rows; (-inf, 0) when U is empty.
 * Same routing outputs and rules as attn_block_router, plus:
 * v:        device [n][heads][head_dim] values (dtype as q/k);
 * scale:    the attention scale of the sparse call (> 0);
 * tail_lse: device float32 [heads][nb]; tail_v: device float32
 *           [heads][nb][head_dim], nb = ceil(n / block_size).
 * Workspace: attn_block_router_tail_workspace(n, heads, head_dim, block_size).
 * Errors: as attn_block_router, plus H3_EINVAL for null v/tail_lse/tail_v or a
 * non-finite or non-positive scale.
 */
size_t attn_block_router_tail_workspace(int n, int heads, int head_dim, int block_size);
int attn_block_router_tail(const void* q, const void* k, const void* v, int dtype, int n,
                           int heads, int head_dim, const uint8_t* seg, int protected_prefix_len,
                           int block_size, int k_sel, float scale, int32_t* tiles, int32_t* prot,
                           int n_prot, float* tail_lse, float* tail_v,
                           void* ws, size_t ws_bytes, void* stream);

/*
 * Block-sparse attention with the pooled tail term.
 * attn_block_sparse, where every query row of block qb also attends one extra
 * key with logit tail_lse[h][qb] and value tail_v[h][qb][:] (from
 * attn_block_router_tail with the same scale), so nothing leaves the softmax;
 * a -inf logit adds nothing. Workspace as attn_block_sparse.
 * Errors: as attn_block_sparse, plus H3_EINVAL for null tail_lse or tail_v.
 */
int attn_block_sparse_tail(const void* q, const void* k, const void* v, int dtype,
                           int n, int heads, int head_dim,
                           const uint8_t* seg, const float* t,
                           float strength, float window, float falloff, float cap, float scale,
                           int block_size, const int32_t* tiles, int k_sel,
                           const int32_t* prot, int n_prot,
                           const float* tail_lse, const float* tail_v,
                           void* o, int o_dtype, float* lse,
                           void* ws, size_t ws_bytes, void* stream);

/*
 * Block-sparse attention with sink query blocks.
 * From "Per-layer attention config LoRAs", section "Experimental: audio/text
 * protection": with sink_queries = audio, the audio queries see no sparsity.
 * attn_block_sparse, where a query block holding any row whose segment id s
 * has bit s set in sink_segments attends every key of the sequence (its list
 * is not read, and it takes no tail term: nothing is left out). The whole
 * block is dense, including its non-sink rows at a segment boundary.
 * sink_segments: bit mask over segment ids 0..3; 1 << H3_SEG_AUDIO gives the
 *           audio sink queries, 0 gives attn_block_sparse.
 * tail_lse, tail_v: both NULL (hard zero for left-out tiles) or both set (the
 *           tail term of attn_block_sparse_tail for the other blocks).
 * Workspace as attn_block_sparse.
 * Errors: as attn_block_sparse, plus H3_EINVAL for sink_segments bits above
 * bit 3 or only one of tail_lse and tail_v set.
 */
int attn_block_sparse_sinks(const void* q, const void* k, const void* v, int dtype,
                            int n, int heads, int head_dim,
                            const uint8_t* seg, const float* t,
                            float strength, float window, float falloff, float cap, float scale,
                            int block_size, const int32_t* tiles, int k_sel,
                            const int32_t* prot, int n_prot,
                            const float* tail_lse, const float* tail_v, unsigned sink_segments,
                            void* o, int o_dtype, float* lse,
                            void* ws, size_t ws_bytes, void* stream);

/*
 * Per-token int8 quantization.
 * From "H3 SLA Attention", inputs table (use_int8_qk): Q and K are quantized to
 * int8 per token with a dynamic scale. Reading (the page gives no formula): for
 * each (row, head) vector x of head_dim values, in float32 with correct
 * rounding, s = max|x| / 127 and x8 = clamp(rint(x / s), -127, 127), rounding
 * half to even; a zero vector gives s = 0 and zeros.
 * x:      device [rows][heads][head_dim], dtype H3_DTYPE_BF16 or H3_DTYPE_F32.
 * x8:     device int8 [rows][heads][head_dim]; scales: device float32 [rows][heads].
 * Errors: H3_EINVAL (null pointer, rows <= 0, heads <= 0); H3_EUNSUPPORTED
 * (dtype, head_dim); H3_ELAUNCH.
 */
int attn_quantize_int8(const void* x, int dtype, int rows, int heads, int head_dim,
                       int8_t* x8, float* scales, void* stream);

/*
 * Block-sparse attention with the int8 QK product.
 * From "H3 SLA Attention", inputs table (use_int8_qk): Q and K are quantized to
 * int8 per token (attn_quantize_int8) before the QK product on the attended
 * blocks; the PV product stays as in attn_block_sparse. Scores are
 * scale * s_q * s_k * sum_d q8 k8 - penalty, i.e. the score rule on the
 * dequantized q and k. Otherwise as attn_block_sparse_sinks (optional tail
 * terms, sink segments; pass 0 for none). bf16 inputs and block sizes 64 and
 * 128 only.
 * Workspace: attn_block_sparse_int8qk_workspace(n, heads, head_dim) bytes: the
 * attn_block_sparse workspace followed by the int8 copies of q and k and their
 * scales.
 * Errors: as attn_block_sparse_sinks, plus H3_EUNSUPPORTED for float32 inputs or
 * block_size 32.
 */
size_t attn_block_sparse_int8qk_workspace(int n, int heads, int head_dim);
int attn_block_sparse_int8qk(const void* q, const void* k, const void* v, int dtype,
                             int n, int heads, int head_dim,
                             const uint8_t* seg, const float* t,
                             float strength, float window, float falloff, float cap,
                             float scale, int block_size, const int32_t* tiles, int k_sel,
                             const int32_t* prot, int n_prot,
                             const float* tail_lse, const float* tail_v,
                             unsigned sink_segments, void* o, int o_dtype, float* lse,
                             void* ws, size_t ws_bytes, void* stream);

/*
 * Stable LSE merge of one partition result into an accumulator, in place.
 * From "Flash Partitions for H3 native temporal alignment", section 4:
 *   adjusted_L = lse_i + log_w (+ log_w_rows[row][h] when non-NULL),
 *   L = logaddexp(lse_acc, adjusted_L),
 *   o_acc = exp(lse_acc - L) * o_acc + exp(adjusted_L - L) * o_i,
 *   lse_acc = L.
 * All float32 device buffers: o_acc, o_i [rows][heads][head_dim]; lse_acc,
 * lse_i, log_w_rows [rows][heads]. Start an accumulator at o = 0 and
 * lse = -inf; -inf merged with -inf stays -inf with o unchanged. A part whose
 * adjusted normaliser is -inf (zero weight) is a no-op; log_w == -inf returns
 * H3_OK without a launch.
 * Errors: H3_EINVAL (null buffers, rows/heads <= 0, log_w NaN or +inf),
 * H3_EUNSUPPORTED (head_dim not in {64,128}), H3_ELAUNCH.
 */
int partition_lse_merge(float* o_acc, float* lse_acc, const float* o_i, const float* lse_i,
                        float log_w, const float* log_w_rows, int rows, int heads, int head_dim,
                        void* stream);

/*
 * Dense TARA attention through the positive-partition decomposition.
 * From "Flash Partitions for H3 native temporal alignment", sections 3-4:
 * exp(-p) = exp(-cap) + [exp(-p) - exp(-cap)]. Queries outside the output
 * video get one ordinary attention call over every key. For output-video
 * queries the library runs ordinary attention calls (with LSE) over: each
 * run of non-guide keys (multiplier 1); each run of guide keys (multiplier
 * exp(-cap)); and, per output frame f and guide frame g, the keys of g
 * (multiplier exp(-cap) * expm1(cap - p(|t_f - t_g|)), omitted when zero);
 * it merges them with partition_lse_merge. Frames are maximal runs of equal
 * timestamp within a guide or output run. The result equals attn_dense_tara
 * up to rounding order. Self-attention only (q, k, v share the n rows).
 * seg_host/t_host: host copies of seg/t (used to plan the calls).
 * Workspace: attn_dense_tara_via_workspace(seg_host, t_host, n, heads,
 * head_dim, dtype) bytes (0 for invalid arguments or when the plan cannot be
 * built). Errors: as attn_dense_tara, plus H3_ENOMEM when host memory for the
 * plan of calls cannot be allocated.
 */
size_t attn_dense_tara_via_workspace(const uint8_t* seg_host, const float* t_host, int n,
                                     int heads, int head_dim, int dtype);
int attn_dense_tara_via(const void* q, const void* k, const void* v, int dtype,
                        int n, int heads, int head_dim,
                        const uint8_t* seg, const float* t,
                        const uint8_t* seg_host, const float* t_host,
                        float strength, float window, float falloff, float cap, float scale,
                        void* o, int o_dtype, float* lse,
                        void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* H3ATTN_H */
