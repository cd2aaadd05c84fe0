/*
 * rbs.h - C ABI of librbs: RBS block-sparse causal prefill attention and
 * Block-attention's static RAG mask on AMD Instinct MI355X (gfx950).
 *
 * Sources (web pages, cited by title and section):
 *   [RBS]    "RBS-Attention: How a Geometric Rescue Branch Fixes Sparse Prefill
 *            for Long-Context LLMs" (techfordev.netlify.app/articles/4709260)
 *   [RBS-ID] "RBS-Attention Bikin Prefill LLM Gede 20x Lebih Cepat, Tanpa
 *            Training Lagi?" (news.captivela.com), section "Dual-Branch
 *            Selection: Centroid Base + Rescue Branch"
 *   [BA]     "Block-Attention for Efficient Prefilling"
 *            (paperlayer.ai/abs/2409.15355v5)
 *   [QUILT]  "QUILT: Rethinking Sparse-Attention Prefill through Shared Query
 *            Execution" (newx.sg)
 *
 * Conventions shared by every call
 * --------------------------------
 * - Batch is one sequence of S tokens. Q and O are [S][Hq][D], K and V are
 *   [S][Hkv][D], contiguous, token-major. Query head h reads KV head
 *   h / (Hq / Hkv). Blocks are B consecutive tokens; nb = ceil(S / B), the
 *   last block may be partial.
 * - Every tensor pointer is a DEVICE pointer owned by the caller and must be
 *   16-byte aligned. Host arrays are marked HOST. The library keeps no pointer
 *   after a call returns and allocates no device memory.
 * - Calls are asynchronous on `stream` (a hipStream_t passed as void*, NULL =
 *   the default stream) and never synchronise.
 * - All argument checks run on the host before anything is enqueued: a call
 *   that returns an error has enqueued nothing. RBS_E_HIP reports a failed
 *   launch (hipGetLastError); faults inside a kernel surface at the caller's
 *   next synchronisation. No exception crosses the ABI.
 * - S == 0 is valid and does nothing (rbs_select still writes row_ptr[0] = 0).
 */
#ifndef RBS_H_
#define RBS_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum rbs_status {
  RBS_OK = 0,
  RBS_E_ARG = 1,          /* null pointer, bad size, misalignment, bad ratio, bad segments */
  RBS_E_UNSUPPORTED = 2,  /* valid but not implemented: dtype/head_dim/block combination, sizes
                             (among them seqlen * n_q_heads * head_dim > 2^40) */
  RBS_E_CAPACITY = 3,     /* col_capacity or workspace too small */
  RBS_E_HIP = 4           /* a HIP runtime call or kernel launch failed */
} rbs_status;

typedef enum rbs_dtype { RBS_DT_BF16 = 0, RBS_DT_F32 = 1 } rbs_dtype;

/* rbs_select flag: always keep key block 0 (an attention sink). */
#define RBS_SEL_FORCE_SINK 0x1u

/* Short English name of a status code (static storage). */
const char* rbs_status_string(rbs_status s);

/*
 * rbs_block_stats - per-block statistics for dual-branch selection.
 *
 * [RBS] "The Standard Approach and Its Blind Spot": a key block is summarised
 * by its centroid (the mean of its keys) and its radius (the largest distance
 * from one of its keys to the centroid); [RBS] "The Fix" scores blocks with a
 * query q and its 2-norm. Computed here, for KV head g and block b:
 *   k_centroid[g][b][:] = mean over the block's tokens of K[t][g][:]
 *   k_radius[g][b]      = max over those tokens of ||K[t][g][:] - centroid||_2
 *   q_rep[g][b][:]      = mean over the block's tokens and over the query heads
 *                         of group g of Q[t][h][:] (one representative query
 *                         per KV head and query block)
 *   q_rep_norm[g][b]    = ||q_rep[g][b][:]||_2
 * Accumulation is fp32; outputs are fp32.
 *
 * dt:         element type of q and k (RBS_DT_BF16 or RBS_DT_F32).
 * q:          [seqlen][n_q_heads][head_dim]; k: [seqlen][n_kv_heads][head_dim].
 * head_dim:   64 or 128. block: 16..256, multiple of 16.
 * n_q_heads % n_kv_heads == 0.
 * Outputs (fp32, device): k_centroid [Hkv][nb][D], k_radius [Hkv][nb],
 *   q_rep [Hkv][nb][D], q_rep_norm [Hkv][nb].
 * Errors: RBS_E_ARG (null/misaligned pointer, size <= 0 other than seqlen == 0,
 *   n_q_heads % n_kv_heads != 0), RBS_E_UNSUPPORTED (head_dim/block outside
 *   the list above), RBS_E_HIP.
 */
rbs_status rbs_block_stats(rbs_dtype dt, const void* q, const void* k, int32_t seqlen,
                           int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim, int32_t block,
                           float* k_centroid, float* k_radius, float* q_rep, float* q_rep_norm,
                           void* stream);

/*
 * rbs_select - dual-branch key-block selection into CSR block lists.
 *
 * [RBS] "The Fix: A Radius-Adaptive Rescue Branch" and [RBS-ID] "Dual-Branch
 * Selection": for query block i of KV head g and every key block j <= i
 *   centroid branch  s_c(j) = q_rep[g][i] . k_centroid[g][j]
 *   rescue branch    s_r(j) = s_c(j) + q_rep_norm[g][i] * k_radius[g][j] * beta[g][j]
 * with beta in [0, 1]. Each branch is thresholded on its own: it keeps its
 * n = min(i+1, max(1, ceil(rho * (i+1) - 1e-6))) best blocks (rho = its keep
 * ratio, computed in double; ties go to the lower block index). The two sets
 * are OR-ed, block i (the causal diagonal) is always added, and block 0 too
 * when flags has RBS_SEL_FORCE_SINK. Scores and the ranking are fp32.
 *
 * beta: beta_in [Hkv][nb] if not NULL. Otherwise derived per KV head from the
 *   distribution of its radii over all nb blocks: with mu their mean and M
 *   their maximum, beta = clamp((r - mu) / (M - mu), 0, 1), and beta = 0 for
 *   every block when M - mu <= 1e-6 * M. (The pages give no formula; this is
 *   the reading the library takes.) beta_out [Hkv][nb] receives the betas used
 *   when not NULL.
 *
 * Output rows r = g * nb + i, ascending block indices:
 *   row_ptr [Hkv*nb + 1] int32, col_idx [row_ptr[Hkv*nb]] int32.
 * col_capacity must be >= rbs_select_capacity(...) for the same arguments.
 * workspace: device scratch of *workspace_bytes bytes, 256-byte aligned. Call
 *   with workspace == NULL to have *workspace_bytes set to the size needed
 *   (nothing else is checked or enqueued then). The workspace contents need
 *   no initialisation and are meaningless after the call.
 * Errors: RBS_E_ARG (null pointer, sizes <= 0, keep ratio outside (0, 1]),
 *   RBS_E_UNSUPPORTED (head_dim not 64/128, nb > 16384),
 *   RBS_E_CAPACITY (col_capacity or *workspace_bytes too small), RBS_E_HIP.
 */
rbs_status rbs_select(const float* k_centroid, const float* k_radius, const float* q_rep,
                      const float* q_rep_norm, const float* beta_in, int32_t n_kv_heads,
                      int32_t n_blocks, int32_t head_dim, double keep_ratio_centroid,
                      double keep_ratio_rescue, uint32_t flags, float* beta_out,
                      int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity,
                      void* workspace, size_t* workspace_bytes, void* stream);

/*
 * rbs_select_static - rbs_select without a workspace argument, for callers
 * that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc. It calls no allocator; its
 * scratch is a static device array of RBS_SELECT_STATIC_SCRATCH_BYTES per GPU,
 * held from the first call on that GPU until the process ends. Arguments,
 * outputs and errors as rbs_select, minus workspace/workspace_bytes; a call
 * whose workspace (as rbs_select's size query reports it) exceeds the array
 * returns RBS_E_CAPACITY and enqueues nothing. The GPU is the one that runs
 * `stream` (the current GPU for the null stream). Every call on one GPU
 * shares that GPU's array: calls that overlap on one GPU (several streams or
 * host threads at once) race and must be serialised by the caller.
 */
#define RBS_SELECT_STATIC_SCRATCH_BYTES ((size_t)16 << 20)
rbs_status rbs_select_static(const float* k_centroid, const float* k_radius,
                             const float* q_rep, const float* q_rep_norm, const float* beta_in,
                             int32_t n_kv_heads, int32_t n_blocks, int32_t head_dim,
                             double keep_ratio_centroid, double keep_ratio_rescue,
                             uint32_t flags, float* beta_out, int32_t* row_ptr,
                             int32_t* col_idx, int64_t col_capacity, void* stream);

/* Number of col_idx entries rbs_select may write for these arguments (host
 * only, no device work): Hkv * sum_i min(i+1, n_c(i) + n_r(i) + 1 + sink).
 * For rbs_select_per_head pass n_q_heads as the first argument (one list per
 * query head). Returns -1 on invalid arguments. */
int64_t rbs_select_capacity(int32_t n_kv_heads, int32_t n_blocks, double keep_ratio_centroid,
                            double keep_ratio_rescue, uint32_t flags);

/*
 * Per-query-head selection (the other reading of the representative query):
 * one representative per (query head, query block) instead of one per (GQA
 * group, query block), and one block list per query head. The rescue and
 * centroid scores of row (h, i) use q_rep_head[h][i] with the centroids,
 * radii and beta of KV head g = h / (Hq / Hkv); budgets, forced blocks, ties
 * and beta are as in rbs_select. A group's heads no longer share one list, so
 * fewer K/V tiles are shared between them in attention.
 *
 * rbs_block_stats_per_head: as rbs_block_stats, but instead of the group
 *   representative it writes, for query head h and block b,
 *     q_rep_head[h][b][:]    = mean over the block's tokens of Q[t][h][:]
 *     q_rep_head_norm[h][b]  = ||q_rep_head[h][b][:]||_2
 *   (fp32 [Hq][nb][D] and [Hq][nb]); k_centroid and k_radius as there. Q and K
 *   are read once. Same arguments, support and errors.
 * rbs_select_per_head: as rbs_select with rows r = h * nb + i for h < n_q_heads
 *   (row_ptr [Hq*nb + 1]); q_rep_head [Hq][nb][D], q_rep_head_norm [Hq][nb];
 *   k_centroid, k_radius, beta_in and beta_out stay per KV head. Errors as
 *   rbs_select, plus RBS_E_ARG when n_q_heads % n_kv_heads != 0.
 * blocksparse_attn_fwd_per_head: as blocksparse_attn_fwd, but query head h of
 *   block i attends to the blocks of CSR row h * nb + i.
 */
rbs_status rbs_block_stats_per_head(rbs_dtype dt, const void* q, const void* k, int32_t seqlen,
                                    int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                                    int32_t block, float* k_centroid, float* k_radius,
                                    float* q_rep_head, float* q_rep_head_norm, void* stream);

rbs_status rbs_select_per_head(const float* k_centroid, const float* k_radius,
                               const float* q_rep_head, const float* q_rep_head_norm,
                               const float* beta_in, int32_t n_q_heads, int32_t n_kv_heads,
                               int32_t n_blocks, int32_t head_dim, double keep_ratio_centroid,
                               double keep_ratio_rescue, uint32_t flags, float* beta_out,
                               int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity,
                               void* workspace, size_t* workspace_bytes, void* stream);

/*
 * blocksparse_attn_fwd - causal GQA attention over the selected key blocks.
 *
 * [RBS] "The Fix" (the combined mask runs through a standard block-sparse
 * attention) and [RBS-ID] "Dual-Branch Selection". For query token t of block
 * i and query head h (KV head g = h / G), the keys are the tokens u <= t of
 * the blocks listed in CSR row g * nb + i:
 *   out[t][h] = sum_u softmax_u(scale * q[t][h] . k[u][g]) v[u][g]
 *   lse[h][t] = log sum_u exp(scale * q[t][h] . k[u][g])   (natural log)
 * softmax_scale <= 0 selects 1/sqrt(head_dim). Arithmetic: bf16 inputs at
 * (head_dim, block) = (128, 128) use bf16 matrix-core products with fp32
 * accumulation and fp32 softmax; every other case computes in fp32 on the
 * vector ALUs (bf16 inputs widened exactly). out has the input dtype (a bf16
 * out is rounded to nearest even).
 *
 * Supported (dt, head_dim, block): dt BF16 or F32, head_dim 64 or 128,
 *   block 64 or 128.
 * row_ptr/col_idx: device CSR as rbs_select writes it. Entries outside 0..i
 *   are skipped; a row with no usable entry gives out 0 and lse -inf.
 * lse may be NULL.
 * Errors: RBS_E_ARG, RBS_E_UNSUPPORTED, RBS_E_HIP.
 */
rbs_status blocksparse_attn_fwd(rbs_dtype dt, const void* q, const void* k, const void* v,
                                int32_t seqlen, int32_t n_q_heads, int32_t n_kv_heads,
                                int32_t head_dim, int32_t block, const int32_t* row_ptr,
                                const int32_t* col_idx, float softmax_scale, void* out,
                                float* lse, void* stream);

/*
 * blocksparse_attn_fwd_shared_query - blocksparse_attn_fwd computed with
 * neighbouring query blocks processed together.
 *
 * [QUILT] "QUILT: Rethinking Sparse-Attention Prefill through Shared Query
 * Execution" (newx.sg), "Abstract" and "Innovation": neighbouring queries
 * select overlapping KV entries, so processing them jointly loads each
 * shared entry once. Here query blocks 2p and 2p + 1 of one query head run
 * in one workgroup over the union of their CSR rows: a key block listed in
 * both rows is moved into on-chip memory once and used by both, a block in
 * one row only by that row's queries. The result is blocksparse_attn_fwd's
 * definition and its arithmetic, unchanged (bit-identical output and lse for
 * the same CSR); only the execution order differs. Rows may be in any order
 * (ascending rows, as rbs_select writes them, share every common block).
 * Supported: bf16 with head_dim 128 and block 128 (else RBS_E_UNSUPPORTED);
 * group CSR rows g * nb + i. Arguments and errors as blocksparse_attn_fwd.
 */
rbs_status blocksparse_attn_fwd_shared_query(rbs_dtype dt, const void* q, const void* k,
                                             const void* v, int32_t seqlen, int32_t n_q_heads,
                                             int32_t n_kv_heads, int32_t head_dim, int32_t block,
                                             const int32_t* row_ptr, const int32_t* col_idx,
                                             float softmax_scale, void* out, float* lse,
                                             void* stream);

/* Per-query-head block lists (see rbs_select_per_head): row h * nb + i. */
rbs_status blocksparse_attn_fwd_per_head(rbs_dtype dt, const void* q, const void* k,
                                         const void* v, int32_t seqlen, int32_t n_q_heads,
                                         int32_t n_kv_heads, int32_t head_dim, int32_t block,
                                         const int32_t* row_ptr, const int32_t* col_idx,
                                         float softmax_scale, void* out, float* lse,
                                         void* stream);

/*
 * blocksparse_attn_fwd_fp8 - blocksparse_attn_fwd with fp8 Q, K and V.
 *
 * [RBS] "Integration with vLLM and Benchmark Results": the model the method is
 * measured on stores its weights in fp8. q, k and v hold OCP E4M3 bytes (sign,
 * 4 exponent bits with bias 7, 3 mantissa bits; largest finite value 448;
 * 0x7F and 0xFF are NaN) with one dequantisation factor per tensor: the real
 * inputs are q_descale * q, k_descale * k and v_descale * v. The result is
 * blocksparse_attn_fwd's definition on those real inputs (same CSR rows,
 * causal masking, softmax_scale and lse); out is bf16 [S][Hq][D], rounded to
 * nearest even.
 * Arithmetic: Q.K^T as fp8 x fp8 matrix-core products summed in fp32; softmax
 * in fp32; the probabilities are rounded to E4M3 with one power-of-two
 * scale per (query row, 32-key block), which puts each block's largest in
 * (128, 256] (nearest even: relative error <= 2^-4 down to 2^-13 of the
 * block's largest, absolute error <= 2^-17 of it below that), and the same
 * rounded values feed both the P.V product and the row sum, so out is a
 * weighted mean of the row's V rows whose weights are within
 * 2^-3 / (1 - 2^-4) relative of the exact softmax weights. Hence
 * |out - exact| <= 0.134 * max over the row's keys of |v_descale * v[u] - exact|
 * up to the small-probability term, fp32 and bf16 rounding; lse is the log
 * of that rounded row sum (within ln(1 + 2^-4) of the exact one).
 * Supported: head_dim 128 and block 128 (else RBS_E_UNSUPPORTED); group CSR
 * rows g * nb + i as rbs_select writes them.
 * Errors: RBS_E_ARG (also for a descale that is not finite and > 0),
 *   RBS_E_UNSUPPORTED, RBS_E_HIP.
 */
rbs_status blocksparse_attn_fwd_fp8(const void* q, const void* k, const void* v, int32_t seqlen,
                                    int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                                    int32_t block, const int32_t* row_ptr, const int32_t* col_idx,
                                    float softmax_scale, float q_descale, float k_descale,
                                    float v_descale, void* out, float* lse, void* stream);

/*
 * block_mask_attn_fwd - Block-attention prefill with position re-encoding.
 *
 * [BA] sections 1 and 2.1 "Main Idea": the input is split into blocks whose
 * key/value states are computed independently, and the final block attends to
 * all preceding blocks; section 2.4 "Block Fine-tune": non-final blocks attend
 * only within themselves; section 2.3 "Position Re-encoding": a cached block,
 * encoded from position 0, is rotated to its new position (RoPE); section 2.5
 * "Inference": cached blocks are re-encoded, then the final block is computed.
 *
 * Segments p = 0..n_segments-1 cover [seg_start[p], seg_start[p+1]); the last
 * one is the final block. Every key of segment p is first rotated by
 * k_rerotate[p] positions (rotate-half RoPE: pair (x_i, x_{i+D/2}) turned by
 * k_rerotate[p] * rope_theta^(-2i/D), angle formed in double precision). A
 * query t of a non-final segment p sees keys [seg_start[p], t]; a query of the
 * final segment sees keys [0, t]. Q is taken as already encoded at absolute
 * positions. Rows t < q_row_begin are not computed (out/lse untouched there):
 * q_row_begin = seg_start[n_segments-1] computes the final block only.
 *
 * seg_start:  HOST [n_segments+1], seg_start[0] = 0, strictly increasing,
 *             seg_start[n_segments] = seqlen; every start except the last
 *             entry a multiple of 128.
 * k_rerotate: HOST [n_segments], >= 0.
 * workspace:  device scratch, 256-byte aligned, caller-owned. It holds the
 *             re-encoded keys (S x Hkv x D bf16) and their cos/sin table when
 *             any k_rerotate[p] is nonzero, and, when the final block's rows
 *             see many key tiles, the partial results of the chunks their key
 *             range is cut into (merged by a second kernel). k_cached itself
 *             is never written. workspace == NULL is a size query:
 *             *workspace_bytes receives the bytes needed (0 when there is
 *             nothing to re-encode or split) and nothing is enqueued.
 *             Otherwise *workspace_bytes holds the workspace size
 *             (RBS_E_CAPACITY if too small). Concurrent calls need separate
 *             workspaces.
 * Supported: dt = BF16, head_dim = 128, 1 <= n_segments <= 256.
 * Errors: RBS_E_ARG, RBS_E_UNSUPPORTED, RBS_E_CAPACITY, RBS_E_HIP.
 */
rbs_status block_mask_attn_fwd(rbs_dtype dt, const void* q, const void* k_cached,
                               const void* v, int32_t seqlen, int32_t n_q_heads,
                               int32_t n_kv_heads, int32_t head_dim, int32_t n_segments,
                               const int32_t* seg_start, const int32_t* k_rerotate,
                               float rope_theta, int32_t q_row_begin, float softmax_scale,
                               void* out, float* lse, void* workspace, size_t* workspace_bytes,
                               void* stream);

#ifdef __cplusplus
}
#endif

#endif /* RBS_H_ */
