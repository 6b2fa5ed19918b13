/*
 * hattn.h -- C ABI of the hybrid compressed-attention library (libhattn.so).
 *
 * The library computes, on one gfx950 GPU, the steps of hybrid compressed
 * attention: sequence-dimension KV compression, lightning-indexer top-k
 * selection (flat and two-stage HISA), sparse MQA attention over the
 * selected entries plus a sliding window, and dense MQA attention over the
 * heavily compressed sequence plus the same window.
 *
 * Sources (cited by page title and section):
 *   [HYB]  process-cxr.github.io, "Hybrid Attention" (ai-library/architecture/attention)
 *   [HCA]  daiw.net, "前代 · HCA：128 倍压缩后再做稠密注意力" (deepseek-v4-flash/hca)
 *   [HISA] my.qihongyi.cn/?p=787, "DeepSeek速度狂飙4倍还不丢精度"
 *   [TRDM] trdm.cn/news/749237, section 2.1
 *
 * Conventions for every entry point:
 *   - Every array argument is a DEVICE pointer (memory from hipMalloc or a
 *     torch CUDA tensor), row-major and contiguous.  Sizes are element counts.
 *     Activation, cache, query, output and workspace arrays (the bf16/fp32
 *     data and the indexer head weights) must be 16-byte aligned: kernels
 *     move them in 16-byte vectors.  A misaligned one gives HATTN_ERR_ARG.
 *     Integer arrays (positions, counts, indices) need only 4-byte alignment.
 *   - The caller owns and allocates all inputs, outputs and workspaces.  The
 *     library allocates nothing and keeps no state between calls (except the
 *     optional kernel timer below).
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Calls only enqueue work on that stream and never synchronise; buffers
 *     must stay alive until the stream has passed the call.
 *   - Validation happens before anything is enqueued: on any status other
 *     than HATTN_OK nothing has been launched and no output was written.
 *     hattn_last_error() returns a thread-local message for the last failure.
 *     Faults inside kernels surface at the caller's next synchronisation.
 *   - Floating inputs are either all fp32 (HATTN_F32) or bf16 (HATTN_BF16,
 *     stored as raw 16-bit patterns) as stated per argument; accumulation is
 *     always fp32.  Non-finite inputs are not supported, nor are finite
 *     ones whose fp32 intermediates overflow (an indexer score or a scaled
 *     attention logit beyond about 3.4e38).  Finite V of any magnitude is
 *     handled (split-K partials are range-scaled).
 *   - Workspaces (device scratch for intermediate scores and partial
 *     results; contents need no initialisation and are meaningless after
 *     the call): with ws == NULL and ws_bytes != NULL the call stores the
 *     required byte count in *ws_bytes and returns HATTN_OK without
 *     launching anything.  With ws != NULL, *ws_bytes must hold the size of
 *     ws; a smaller size than required gives HATTN_ERR_WORKSPACE.
 *     ws_bytes == NULL means no workspace is given, which is accepted when
 *     the call needs none (required size 0) and gives HATTN_ERR_WORKSPACE
 *     otherwise.  Calls that overlap in time must not share a workspace.
 *   - Index lists are int32, ascending, padded with -1 at the end.
 */
#ifndef HATTN_H
#define HATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  HATTN_OK = 0,
  HATTN_ERR_ARG = 1,         /* bad size, NULL required pointer, inconsistent arguments */
  HATTN_ERR_UNSUPPORTED = 2, /* valid arguments with no kernel (e.g. a head size) */
  HATTN_ERR_WORKSPACE = 3,   /* workspace smaller than required */
  HATTN_ERR_HIP = 4          /* the HIP runtime reported an error at launch */
} hattn_status_t;

typedef enum { HATTN_F32 = 0, HATTN_BF16 = 1 } hattn_dtype_t;

/* Text for a status code (static storage). */
const char* hattn_status_string(int status);
/* Detail for the calling thread's last failing call (static thread storage). */
const char* hattn_last_error(void);
/* Version of this ABI (bumped on incompatible changes; 2: hattn_decode_desc gained csa_idx; 3: raw_rows
 * (raw K|V rings) in hattn_decode_desc, hattn_decode_append and the attention calls). */
int hattn_abi_version(void);

/*
 * hattn_compress -- sequence-dimension KV compression.
 * [HCA] section 怎么压: each compressed entry is the sum of a run of raw rows
 * weighted by a softmax over (per-token compression logit + learnable
 * position bias).  CSA uses runs of 8 at stride 4 (rate 4, [HCA] section
 * 它补的正是 CSA 的短板, [TRDM] 2.1); HCA uses disjoint runs of 128.
 *
 *   entry i of sequence b covers raw rows [i*stride, i*stride + w):
 *     a_j   = logits[b][i*stride + j] + pos_bias[j]          (j < w)
 *     y[b][i][c] = sum_j softmax(a)_j * x[b][i*stride + j][c]
 *
 *   x        [bt][L][C]  dtype (K and V of a row side by side: C = 2*d)
 *   logits   [bt][L]     fp32, or NULL for all-zero logits
 *   pos_bias [w]         fp32, or NULL for zero bias
 *   y        [bt][N][C]  dtype, N = (L - w)/stride + 1 complete windows
 *   Only entries e_begin <= i < e_end are (re)written, so a decode step can
 *   compress just the windows its new token completed.
 * Requires 1 <= w <= 4096, 1 <= stride, L >= w, C a multiple of 16 bytes'
 * worth of elements (8 for bf16, 4 for fp32), 0 <= e_begin <= e_end <= N.
 */
hattn_status_t hattn_compress(int dtype, const void* x, int64_t bt, int64_t L, int32_t C,
                              const float* logits, const float* pos_bias, int32_t w, int32_t stride,
                              int64_t e_begin, int64_t e_end, void* y, void* stream);

/*
 * hattn_compress_with_index -- compressed K|V entries and their indexer keys.
 * [TRDM] section 2.1 (the indexer picks the most important compressed KV
 * blocks: it scores the entries this call builds) and [HCA] section 怎么压
 * (the softmax(logit + position bias) merge): each entry's indexer key is
 * the merge of the raw indexer keys of its window with the entry's own
 * weights, the ones that merge its K|V rows:
 *   y[b][i]   = sum_j softmax(a)_j * x[b][i*stride + j]       (as hattn_compress)
 *   y_i[b][i] = sum_j softmax(a)_j * x_i[b][i*stride + j]     (same a)
 *   x   [bt][L][C]   dtype     x_i [bt][L][C_i] dtype (raw indexer keys)
 *   y   [bt][N][C]   dtype     y_i [bt][N][C_i] dtype (the entries' K_I)
 * Other arguments and limits as for hattn_compress (C_i a multiple of 16
 * bytes' worth of elements).  One pass computes both outputs.
 */
hattn_status_t hattn_compress_with_index(int dtype, const void* x, const void* x_i, int64_t bt, int64_t L, int32_t C,
                                         int32_t C_i, const float* logits, const float* pos_bias, int32_t w,
                                         int32_t stride, int64_t e_begin, int64_t e_end, void* y, void* y_i,
                                         void* stream);

/*
 * hattn_compress_channel_logits -- compression with a logit per channel.
 * The variant of hattn_compress whose compression weight ([HCA] section
 * 怎么压: one weight per raw entry, softmax over weight + position bias) is a
 * vector, one value per channel, so each channel has its own softmax:
 *   a_jc = logits[b][i*stride + j][c] + pos_bias[j]
 *   y[b][i][c] = sum_j softmax_j(a_.c)_j * x[b][i*stride + j][c]
 *   logits [bt][L][C] fp32 (required; 16-byte aligned), pos_bias [w] or NULL.
 * Other arguments and limits as for hattn_compress.
 */
hattn_status_t hattn_compress_channel_logits(int dtype, const void* x, int64_t bt, int64_t L, int32_t C,
                                             const float* logits, const float* pos_bias, int32_t w, int32_t stride,
                                             int64_t e_begin, int64_t e_end, void* y, void* stream);

/*
 * hattn_visible_count -- how many compressed entries each query may see.
 * Causal reading of [HYB] section 为什么长上下文需要新的 Attention (decode
 * reads only history): entry i is visible to a query at raw position p iff
 * its last raw row i*stride + w - 1 <= p, so
 *   n_vis = 0 if p < w - 1, else min(n_entries, (p - w + 1)/stride + 1).
 *   pos [count] int32 raw positions (>= 0) -> n_vis [count] int32.
 */
hattn_status_t hattn_visible_count(const int32_t* pos, int64_t count, int32_t w, int32_t stride,
                                   int64_t n_entries, int32_t* n_vis, void* stream);

/*
 * hattn_index_topk -- flat lightning-indexer selection.
 * [HISA] section 01: score every visible candidate of a query, keep the top k.
 * Score (the pages print no formula; ReLU-weighted head sum):
 *   S[q][i] = sum_h w_i[q][h] * max(0, q_i[q][h] . k_i[i])     for i < n_vis[q]
 * Selection: the k largest S (ties to the lower i), emitted in ascending i,
 * padded with -1 when n_vis[q] < k.  -0.0 and +0.0 are equal scores.
 *
 *   q_i   [bt][nq][h_i][d_i]  dtype       k_i [bt][n][d_i] dtype
 *   w_i   [bt][nq][h_i]       fp32        n_vis [bt][nq] int32 (clamped to [0, n])
 *   idx   [bt][nq][k]         int32 out   score [bt][nq][k] fp32 out or NULL
 *         (the selected scores; -inf where idx is -1)
 *   ws    workspace (size by query, see conventions)
 * Requires 1 <= k <= 8192, 1 <= h_i <= 64, 1 <= d_i <= 256, h_i * d_i <=
 * 8192 (HATTN_ERR_UNSUPPORTED above).  bf16 with h_i = 16 and d_i in
 * {32, 64, 128, 256} runs on MFMA; every other shape on the vector kernel.
 */
hattn_status_t hattn_index_topk(int dtype, const void* q_i, const void* k_i, const float* w_i,
                                const int32_t* n_vis, int64_t bt, int64_t nq, int32_t h_i, int32_t d_i,
                                int64_t n, int32_t k, int32_t* idx, float* score, void* ws,
                                size_t* ws_bytes, void* stream);

/*
 * hattn_hisa_pool -- HISA block representatives.
 * [HISA] section 第一阶段: the prefix is cut into blocks of B entries, each
 * summarised by one pooled vector; here the mean, with a short last block
 * zero-padded (divided by B, not by its own count).
 *   reps[b][j][c] = (1/B) * sum_{i in [jB, min(n, jB+B))} k_i[b][i][c]
 *   k_i [bt][n][d_i] dtype  ->  reps [bt][ceil(n/B)][d_i] fp32.
 * Only blocks j_begin <= j < j_end are written (a decode step refreshes the
 * last block alone).
 */
hattn_status_t hattn_hisa_pool(int dtype, const void* k_i, int64_t bt, int64_t n, int32_t d_i, int32_t B,
                               int64_t j_begin, int64_t j_end, float* reps, void* stream);

/*
 * hattn_hisa_topk -- two-stage HISA selection.
 * [HISA] section 第一阶段: score every block representative whose first entry
 * is visible with the same score form as above and keep the top m blocks
 * (ties to the lower block).  Section 第二阶段: run the token indexer only on
 * the visible entries of those blocks and keep the top k.  Section 05,
 * Step 3: the output has the flat indexer's form (ascending, -1 padded).
 *
 *   q_i, k_i, w_i, n_vis as for hattn_index_topk; reps from hattn_hisa_pool.
 *   idx [bt][nq][k] int32 out;  blk [bt][nq][m] int32 out (chosen blocks,
 *   ascending, -1 padded) or NULL.
 * Requires 1 <= B <= 1024, 1 <= m, m*B <= 16384, 1 <= k <= 8192, and the
 * indexer shape limits of hattn_index_topk.  With h_i = 16 the block scores
 * run on MFMA for d_i in {16, 32, 64, 128, 256} (bf16 or fp32 queries);
 * other shapes take the vector kernel.
 *
 * Departure from a compute-the-block-means mode: the block means are always
 * an input here (hattn_hisa_pool builds them once per prefix, and
 * hattn_decode_append keeps the last block current), so this call only reads
 * them.
 */
hattn_status_t hattn_hisa_topk(int dtype, const void* q_i, const void* k_i, const float* w_i,
                               const int32_t* n_vis, int64_t bt, int64_t nq, int32_t h_i, int32_t d_i,
                               int64_t n, const float* reps, int32_t B, int32_t m, int32_t k,
                               int32_t* idx, int32_t* blk, void* ws, size_t* ws_bytes, void* stream);

/*
 * hattn_block_sparse_topk -- block-sparse (MoBA/NSA-style) selection, the
 * baseline HISA is compared with.
 * [HISA] section 04: block-sparse methods select at block granularity and
 * every token of a chosen block takes part in attention; HISA's block level
 * is only a first filter.  The blocks are chosen exactly as
 * hattn_hisa_topk's first stage chooses them (same block means and score;
 * candidates are the blocks whose first entry is visible; ties to the lower
 * block), and the selection is every visible entry of the m chosen blocks:
 *   idx [bt][nq][m*B] int32 out, ascending, -1 padded (the attention budget
 *   of m blocks is m*B entries);  blk [bt][nq][m] int32 out or NULL.
 * Other arguments and limits as for hattn_hisa_topk (1 <= m, m*B <= 16384).
 */
hattn_status_t hattn_block_sparse_topk(int dtype, const void* q_i, const void* k_i, const float* w_i,
                                       const int32_t* n_vis, int64_t bt, int64_t nq, int32_t h_i, int32_t d_i,
                                       int64_t n, const float* reps, int32_t B, int32_t m, int32_t* idx,
                                       int32_t* blk, void* ws, size_t* ws_bytes, void* stream);

/*
 * hattn_sparse_attn -- CSA attention: selected entries plus sliding window.
 * [HYB] section Compressed Sparse Attention; [HCA] section 怎么压 (MQA: all
 * query heads share one K/V; a branch over the latest 128 raw tokens).
 * One softmax runs over the union U of {ckv[idx[q][j]] : idx != -1} and the
 * raw rows max(0, p - window + 1) .. p (no de-duplication):
 *   out[q][h] = sum_{u in U} softmax_u(scale * q[q][h] . K_u) * V_u
 *   lse[q][h] = log sum_{u in U} exp(scale * q[q][h] . K_u)
 *
 *   q      [bt][nq][h][d] dtype      ckv [bt][n][2d] dtype (K | V per entry)
 *   idx    [bt][nq][k] int32; entries < 0 or >= n are skipped
 *   raw_kv [bt][L][2d] dtype         q_pos [bt][nq] int32, 0 <= p < L
 *          or, with raw_rows = R > 0, a ring [bt][R][2d] of the newest
 *          rows (row r at slot r % R; window <= R <= L): it must hold every
 *          row a query reads, max(0, p - window + 1) .. p for each q_pos p
 *          of the sequence (the device cannot check this).  raw_rows = 0:
 *          all L rows.
 *   out    [bt][nq][h][d] fp32 out   lse [bt][nq][h] fp32 out or NULL
 * Requires window >= 1 and d a multiple of 8.  bf16 with d in {64, 128}
 * and h in {16, 32} or a multiple of 64 up to 1,024 runs on MFMA (64 heads
 * per workgroup); any other shape with h*d <= 8192 and d <= 256 takes the
 * vector path.  Arithmetic: fp32 accumulation; on the MFMA path the
 * softmax weights enter the PV product in bf16 and, when a query's key
 * list is split over several workgroups, each split's normalised output
 * O/l is kept in fp16 in the workspace until the merge, scaled down by a
 * power of two when its largest value reaches 2^15 (values beyond fp16's
 * range), with its max, sum and scale in fp32; the fp32 vector path keeps
 * fp32 throughout.  Layers that share one cache and one index list (CSA2's
 * cross-layer reuse, [HCA] section V4.1 为什么不要它了) are one call: with
 * MQA every head attends to the same keys, so layer g's head j is head
 * g*h_layer + j of q, out and lse.
 */
hattn_status_t hattn_sparse_attn(int dtype, const void* q, const void* ckv, int64_t n, const int32_t* idx,
                                 int32_t k, const void* raw_kv, int64_t L, int64_t raw_rows, const int32_t* q_pos,
                                 int32_t window, float scale, int64_t bt, int64_t nq, int32_t h, int32_t d,
                                 float* out, float* lse, void* ws, size_t* ws_bytes, void* stream);

/*
 * hattn_sparse_attn_noalloc -- hattn_sparse_attn for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments, result and errors as
 * hattn_sparse_attn, without a workspace: the split-K partials go to a
 * static device array of the library (32 MiB on each GPU it runs on, held
 * until the process ends).  The call allocates nothing.
 *   - A shape whose partials need more than 32 MiB (the size query of
 *     hattn_sparse_attn returns more than 33,554,432 bytes) gives
 *     HATTN_ERR_WORKSPACE and launches nothing.
 *   - Every call on one GPU shares that GPU's array: calls that overlap in
 *     time on one GPU (different streams, or graphs replayed concurrently)
 *     race on it and give undefined results.  Nothing needs clearing
 *     between calls (every partial is written before it is read).
 */
hattn_status_t hattn_sparse_attn_noalloc(int dtype, const void* q, const void* ckv, int64_t n, const int32_t* idx,
                                         int32_t k, const void* raw_kv, int64_t L, int64_t raw_rows,
                                         const int32_t* q_pos, int32_t window, float scale, int64_t bt, int64_t nq,
                                         int32_t h, int32_t d, float* out, float* lse, void* stream);

/*
 * hattn_dense_compressed_attn -- HCA attention: every visible entry plus window.
 * [HCA] sections 128 倍是什么概念 and 怎么压: no selection; each query attends
 * to all compressed entries it may see (ckv[0 .. n_vis[q]-1]) and to the
 * same window branch, in one softmax.  Arguments as for hattn_sparse_attn
 * with n_vis [bt][nq] int32 (clamped to [0, n]) in place of idx and k.
 */
hattn_status_t hattn_dense_compressed_attn(int dtype, const void* q, const void* ckv, int64_t n,
                                           const int32_t* n_vis, const void* raw_kv, int64_t L, int64_t raw_rows,
                                           const int32_t* q_pos, int32_t window, float scale, int64_t bt,
                                           int64_t nq, int32_t h, int32_t d, float* out, float* lse, void* ws,
                                           size_t* ws_bytes, void* stream);

/*
 * hattn_decode_append -- per-token maintenance of one compressed layer in a
 * decode step: one query per sequence, the sequence's newest token at
 * position q_pos[b].  In one launch:
 *   n_vis[b] = entries visible at q_pos[b] (exactly as hattn_visible_count);
 *   if that token completes entry e = (q_pos[b] - w + 1) / stride (the token
 *   is its window's last one and e < N), ckv[b][e] = the compression of
 *   that window (as hattn_compress over entries [e, e+1));
 *   if k_i and reps are given and an entry was completed, reps[b][e / B] =
 *   the mean of the HISA block holding e (as hattn_hisa_pool over it).
 * Sources: [HCA] section 怎么压 (each entry is a weighted merge of its run
 * of raw entries), [HISA] section 02, first stage (one pooled representative
 * per block), and the causal visibility of hattn_visible_count.
 *   raw_kv   [bt][L][C]      dtype; K|V rows as in hattn_compress, or, with
 *                            raw_rows = R > 0, a ring [bt][R][C] holding the
 *                            newest R rows: row r at slot r % R (the caller
 *                            writes each new token's row before the call;
 *                            w <= R <= L).  A decode step needs only the
 *                            rows of the newest windows, not the prefix.
 *   logits   [bt][L] fp32 or NULL ([bt][R] with a ring); pos_bias [w] or NULL
 *   q_pos    [bt] int32      any values (positions that complete no entry
 *                            only get their visible count)
 *   ckv      [bt][N][C]      N = (L - w) / stride + 1; entry e rewritten
 *   n_vis    [bt] int32      output
 *   k_i      [bt][N][d_i]    dtype, or NULL (then reps must be NULL)
 *   reps     [bt][ceil(N/B)][d_i] fp32; block e / B rewritten
 * Limits: 1 <= w <= 4096, L >= w; C and d_i multiples of 16/elem_bytes with
 * at most 256 16-byte pieces per row.  Errors: HATTN_ERR_ARG for bad sizes,
 * NULL required pointers or an inconsistent k_i / reps pair.
 */
hattn_status_t hattn_decode_append(int dtype, const void* raw_kv, int64_t bt, int64_t L, int64_t raw_rows,
                                   int32_t C, const float* logits, const float* pos_bias, int32_t w, int32_t stride,
                                   const int32_t* q_pos, void* ckv, int32_t* n_vis, const void* k_i, int32_t d_i,
                                   int32_t B, float* reps, void* stream);

/*
 * Decode step of a hybrid layer pair, as a reusable plan.
 * [HYB] section Compressed Sparse Attention and [HCA] section 它补的正是 CSA
 * 的短板 (a CSA branch and an HCA branch side by side); the steps are the
 * entry points above, for one new token per sequence (nq = 1) at q_pos[b]:
 *   CSA branch: hattn_decode_append (with block means) -> hattn_hisa_topk
 *               -> hattn_sparse_attn
 *   HCA branch: hattn_decode_append (no block means)
 *               -> hattn_dense_compressed_attn
 * A plan validates every argument once and keeps the launch parameters, so
 * running a step costs one host call, and everything runs on the caller's
 * stream: the HCA branch's work shares the CSA branch's launches (one
 * cache-maintenance launch for both layers, one attention launch, one merge
 * launch), so the two branches overlap on the GPU without any cross-stream
 * synchronisation.  For bf16 with h_i = 16 the cache-maintenance launch also
 * computes HISA's block scores (the first stage); the workgroup that scores
 * the block holding the new entry recomputes that block's mean itself.
 * Results equal those of the separate calls on the same arguments.
 *
 * hattn_decode_desc (all arrays as documented for the calls above; the two
 * branches share bt, L, h, d, window, scale and q_pos):
 *   dtype, bt, L, h, d, window, scale, q_pos [bt] int32
 *   raw_rows: 0 when csa_raw_kv / hca_raw_kv ([bt][L][2d]) and the logits
 *     ([bt][L]) hold every raw row; R > 0 when they are rings of the newest
 *     R rows ([bt][R][2d], [bt][R]; row r at slot r % R; R >= window and
 *     both compression windows): the caller writes the new token's rows and
 *     logits at slot q_pos[b] % R before each step
 *   csa_raw_kv, csa_logits, csa_pos_bias, csa_w, csa_stride, csa_ckv
 *     ([bt][N][2d], N = (L - csa_w) / csa_stride + 1; rewritten in place)
 *   k_i [bt][N][d_i], reps [bt][ceil(N/B)][d_i] fp32 (rewritten in place),
 *   q_i [bt][h_i][d_i], w_i [bt][h_i] fp32, h_i, d_i, B, m, k
 *   csa_q [bt][h][d], csa_out [bt][h][d] fp32, csa_lse [bt][h] fp32 or NULL
 *   csa_idx [bt][k] int32 or NULL: where given, the step leaves the CSA
 *     branch's selected entries there (hattn_hisa_topk's idx); otherwise
 *     they live in the workspace
 *   hca_raw_kv, hca_logits, hca_pos_bias, hca_w, hca_stride, hca_ckv,
 *   hca_q, hca_out, hca_lse     (as the CSA fields, for the HCA branch)
 *   ws, ws_bytes               workspace (size: hattn_decode_plan_ws_bytes);
 *                              holds visible counts, the selected indices and
 *                              the calls' own workspaces
 *
 *   hattn_decode_desc_size()        sizeof(hattn_decode_desc), for bindings
 *   hattn_decode_plan_ws_bytes(desc, &bytes)
 *   hattn_decode_plan_create(desc, &plan)  validates (HATTN_ERR_ARG /
 *       HATTN_ERR_UNSUPPORTED / HATTN_ERR_WORKSPACE as the separate calls
 *       would) and records the current device.  The plan keeps the
 *       pointers, not the data: every buffer must stay valid while the plan
 *       is used.
 *   hattn_decode_plan_run(plan, stream)  enqueues one step on `stream` (the
 *       current device must be the plan's).  Two runs of one plan must not
 *       overlap in time (they share the workspace).
 *   hattn_decode_plan_run_graph(plan, stream)  the same step as one launch:
 *       the first call captures the step's kernels into a HIP graph held by
 *       the plan (on a private stream; the kernel timer must be off, else
 *       HATTN_ERR_ARG), and every call launches that graph on `stream`.
 *       Results equal hattn_decode_plan_run's.  The graph reads the buffers
 *       when it runs, as run does, so inputs may change between steps.
 *   hattn_decode_plan_destroy(plan)  frees the plan and its graph; NULL is
 *       accepted.
 */
typedef struct hattn_decode_desc {
  int32_t dtype;
  int32_t h, d, window;
  int64_t bt, L;
  int64_t raw_rows;
  float scale;
  int32_t h_i, d_i, B, m, k;
  int32_t csa_w, csa_stride, hca_w, hca_stride;
  const int32_t* q_pos;
  const void* csa_raw_kv;
  const float* csa_logits;
  const float* csa_pos_bias;
  void* csa_ckv;
  const void* k_i;
  float* reps;
  const void* q_i;
  const float* w_i;
  const void* csa_q;
  float* csa_out;
  float* csa_lse;
  int32_t* csa_idx;
  const void* hca_raw_kv;
  const float* hca_logits;
  const float* hca_pos_bias;
  void* hca_ckv;
  const void* hca_q;
  float* hca_out;
  float* hca_lse;
  void* ws;
  size_t ws_bytes;
} hattn_decode_desc;

typedef struct hattn_decode_plan* hattn_decode_plan_t;

int64_t hattn_decode_desc_size(void);
hattn_status_t hattn_decode_plan_ws_bytes(const hattn_decode_desc* desc, size_t* ws_bytes);
hattn_status_t hattn_decode_plan_create(const hattn_decode_desc* desc, hattn_decode_plan_t* plan);
hattn_status_t hattn_decode_plan_run(hattn_decode_plan_t plan, void* stream);
hattn_status_t hattn_decode_plan_run_graph(hattn_decode_plan_t plan, void* stream);
hattn_status_t hattn_decode_plan_destroy(hattn_decode_plan_t plan);

/*
 * Kernel timer (profiling aid).  When enabled, every kernel the library
 * launches is bracketed by HIP events recorded on the same stream, and its
 * duration is accumulated per kernel name when hattn_timer_collect() is
 * called (which synchronises on those events).  Disabled by default; not
 * thread-safe; do not enable it while a HIP graph is being captured.
 *   hattn_timer_enable(1|0)     start / stop recording (start clears totals)
 *   hattn_timer_collect()       wait for recorded events, fold them into totals
 *   hattn_timer_query(name, &total_ms, &count) -> HATTN_OK or HATTN_ERR_ARG if
 *                               no kernel of that name was recorded
 *   hattn_timer_names(buf, len) writes the recorded kernel names, '\n'-separated
 */
hattn_status_t hattn_timer_enable(int on);
hattn_status_t hattn_timer_collect(void);
hattn_status_t hattn_timer_query(const char* name, double* total_ms, int64_t* count);
hattn_status_t hattn_timer_names(char* buf, int64_t len);

#ifdef __cplusplus
}
#endif

#endif /* HATTN_H */
