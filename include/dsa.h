/*
 * dsa.h -- C ABI of the DeepSeek Sparse Attention (DSA) forward path on
 * AMD Instinct MI355X (gfx950).
 *
 * The path has three stages (the two-stage data flow of the charlestar page
 * "DeepSeek V3.2 稀疏注意力", section "DSA 的两段式数据流"):
 *
 *   1. Lightning Indexer score ("详解DSA", Eq.(1)):
 *        I[t,s] = sum_{j<64} w[t,j] * ReLU(q[t,j] . k[s]),
 *      64 heads of dim 128, one key per cached token shared by all heads,
 *      fp8-e4m3fn keys with one fp32 scale per 128-element block (= per
 *      token); causal: only s <= pos(t) is scored.
 *   2. Per-query top-k over the valid positions ("详解DSA", Indexer code
 *      block: topk(min(index_topk, end_pos))), ties toward the lower index.
 *   3. Sparse MQA-mode MLA ("详解DSA" Eq.(2); MQA mode per the charlestar
 *      page "DSA 怎样嵌入 MLA" and the luowle page section 3.1): every query
 *      head attends to the same selected 576-wide latent entries (512 latent
 *      + 64 rope); the value is the first 512 dims; the softmax runs over the
 *      selected entries only.
 *
 * Geometry and positions.  B sequences, q_len new queries per sequence,
 * T = B*q_len query rows, row t = b*q_len + i.  seq_lens[b] is the number of
 * cached tokens of sequence b including its new ones (the end_pos of the
 * Indexer code block), so query i of sequence b sits at
 *     pos = seq_lens[b] - q_len + i
 * and sees the keys s <= pos (inclusive causal mask).  Kernels clamp
 * seq_lens[b] into [0, S_max]; a row whose pos is negative sees no key.
 *
 * Memory.  Every tensor pointer is DEVICE memory allocated and owned by the
 * caller; all tensors are dense row-major in the shapes given.  The library
 * never allocates or frees memory and keeps no pointer after the enqueued
 * work finishes; scratch memory comes in through (ws, ws_bytes), sized by
 * the matching *_workspace_size query.  Workspace pointers must be 256-byte
 * aligned, tensor pointers 16-byte aligned.
 *
 * Streams and errors.  Every call validates its arguments on the host before
 * enqueuing anything and returns DSA_ERR_INVALID_ARG (bad pointer, shape,
 * alignment or size), DSA_ERR_UNSUPPORTED (a dtype combination or size the
 * kernels do not implement) or DSA_ERR_WORKSPACE (ws too small) without
 * touching the device.  Otherwise the work is enqueued asynchronously on
 * `stream` (0 = the null stream) and the call returns DSA_OK, or DSA_ERR_HIP
 * if a launch failed.  No call synchronises, aborts or throws.  Calls share
 * no mutable library state; concurrent calls must use distinct workspaces.
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__) || defined(__clang__)
#define DSA_API __attribute__((visibility("default")))
#else
#define DSA_API
#endif

typedef enum {
  DSA_OK = 0,
  DSA_ERR_INVALID_ARG = 1,
  DSA_ERR_UNSUPPORTED = 2,
  DSA_ERR_WORKSPACE = 3,
  DSA_ERR_HIP = 4
} dsa_status;

typedef enum {
  DSA_F32 = 0,        /* IEEE binary32 */
  DSA_BF16 = 1,       /* bfloat16 */
  DSA_FP8_E4M3FN = 2  /* OCP fp8 e4m3 "fn" (the float8_e4m3fn cache dtype of the Indexer code block) */
} dsa_dtype;

/* Fixed indexer geometry: the public configuration printed on the luowle
 * page, section 3.2 (index_n_heads = 64, index_head_dim = 128). */
#define DSA_INDEX_HEADS 64
#define DSA_INDEX_DIM 128
/* Latent entry width and value width of MQA-mode MLA ("详解DSA": 576 = 512
 * latent + 64 rope; the value is the 512-wide latent). */
#define DSA_LATENT_DIM 576
#define DSA_VALUE_DIM 512

typedef struct {
  int32_t B;                /* sequences, >= 1 */
  int32_t q_len;            /* new queries per sequence, >= 1 */
  int32_t S_max;            /* cache capacity per sequence, >= 1 */
  const int32_t* seq_lens;  /* DEVICE [B]; intended q_len <= seq_lens[b] <= S_max */
} dsa_geom;

/* Lightning Indexer scores ("详解DSA" Eq.(1), with the fp8 scale handling of
 * its "DSA计算流" section: the q-scale multiplies each head's ReLU output and
 * the k-scale multiplies the sum over heads).
 *
 *   scores[r, s] = k_scale[b,s] * sum_j w[t,j]*q_scale[t,j]*ReLU(q[t,j,:].k[b,s,:])
 *                                              for s <= pos(t), s < S_max
 *   scores[r, s] = -inf                        for pos(t) < s < S_max
 * with t = row_begin + r, 0 <= r < row_count.  Columns S_max..ld-1 are not
 * written.
 *
 *   q        [T, 64, 128]   FP8_E4M3FN or F32
 *   q_scale  [T, 64] fp32 or NULL (= 1)
 *   w        [T, 64]        BF16 or F32, used as given (no extra factors)
 *   k        [B, S_max, 128] same dtype as q
 *   k_scale  [B, S_max] fp32 or NULL (= 1)
 *   scores   [row_count, ld] fp32, ld >= S_max
 * Supported: (q,k) FP8_E4M3FN with w BF16 or F32; (q,k,w) all F32.
 * fp8 dot products run on the fp8 matrix cores with fp32 accumulation. */
DSA_API dsa_status dsa_indexer_scores(const dsa_geom* geom,
                              const void* q, dsa_dtype q_dtype, const float* q_scale,
                              const void* w, dsa_dtype w_dtype,
                              const void* k, dsa_dtype k_dtype, const float* k_scale,
                              int32_t row_begin, int32_t row_count,
                              float* scores, int64_t ld, hipStream_t stream);

/* Top-k of precomputed scores ("详解DSA", Indexer code block:
 * topk(min(index_topk, end_pos)); ties go to the lower position).
 *
 * For row r (query t = row_begin + r) the valid set is V = {s : s <= pos(t)}.
 * If |V| <= k every valid position is selected; otherwise the k positions
 * that come first in the order (score descending, position ascending).
 * idx[r, :] holds the selected positions in ASCENDING order followed by -1
 * padding.  Only columns s <= pos(t) of `scores` are read.  Scores must not
 * be NaN (NaN rows give an unspecified but in-range selection).
 *
 *   scores [row_count, ld] fp32, ld >= S_max;  idx [row_count, k] int32
 *   k >= 1 (else DSA_ERR_INVALID_ARG); this build selects for k <= 4096
 *   and S_max <= 262144 and returns DSA_ERR_UNSUPPORTED beyond;
 *   ws >= dsa_topk_workspace_size(...) bytes. */
DSA_API dsa_status dsa_topk(const dsa_geom* geom, const float* scores, int64_t ld,
                    int32_t row_begin, int32_t row_count, int32_t k,
                    int32_t* idx, void* ws, size_t ws_bytes, hipStream_t stream);
DSA_API size_t dsa_topk_workspace_size(int32_t row_count, int32_t S_max, int32_t k);

/* Sparse MQA-mode MLA over selected latent entries ("详解DSA" Eq.(2) and the
 * masked MLA forward on that page: softmax in fp32 over the selected set).
 *
 * For each row t and head h, over M_t = {m : idx[t,m] valid}:
 *   z_m      = sm_scale * q[t,h,:] . kv[b, idx[t,m], :]          (576 dims)
 *   out[t,h] = sum_m softmax(z)_m * kv[b, idx[t,m], 0:512]
 *   lse[t,h] = log sum_m exp(z_m)      (natural log; -inf if M_t is empty)
 * An index is valid if 0 <= idx <= pos(t); -1 and any other value are skipped
 * (an empty set gives out = 0).  Duplicated indices count once per copy.
 *
 *   q   [T, H, 576]  BF16 or F32     kv [B, S_max, 576] same dtype
 *   idx [T, k] int32                 out [T, H, 512] same dtype as q
 *   lse [T, H] fp32 or NULL
 * H: BF16 needs H % 16 == 0 and H <= 128; F32 needs 1 <= H <= 128.
 * 1 <= k <= 16384.  ws >= dsa_sparse_mla_workspace_size(...) bytes. */
DSA_API dsa_status dsa_sparse_mla(const dsa_geom* geom, int32_t H, int32_t k, float sm_scale,
                          const void* q, dsa_dtype dtype, const void* kv,
                          const int32_t* idx, void* out, float* lse,
                          void* ws, size_t ws_bytes, hipStream_t stream);
DSA_API size_t dsa_sparse_mla_workspace_size(int32_t B, int32_t q_len, int32_t H, int32_t k,
                                     dsa_dtype dtype);

/* The whole forward path: indexer -> top-k -> sparse MLA, on one stream.
 * Arguments as in the three calls above (index_* = the indexer inputs,
 * mla_* = the attention inputs, both at the same geometry; H and topk in
 * the order of dsa_sparse_mla's H and k).  idx_out
 * [T, topk] int32 receives the selection (ascending, -1 padded); it may be
 * NULL, and the selection then lives in the workspace, which must hold
 * T * topk * 4 bytes (rounded up to 256) beyond the size query's value.
 *
 * Long prefills (q_len >= 64 with fp8 inputs) stream the indexer scores
 * through on-chip memory with a running per-row candidate set, so no T x S
 * score matrix is ever written; other shapes score into the workspace first.
 * When S_max <= topk no row can hold more than topk valid positions, so the
 * selection is every position ("详解DSA", DSA计算流: the indexer can be
 * bypassed) and neither the indexer nor the top-k runs; the index inputs are
 * still validated.
 * ws >= dsa_forward_workspace_size(...) bytes. */
DSA_API dsa_status dsa_forward(const dsa_geom* geom, int32_t H, int32_t topk, float sm_scale,
                       const void* index_q, dsa_dtype index_dtype, const float* index_q_scale,
                       const void* index_w, dsa_dtype index_w_dtype,
                       const void* index_k, const float* index_k_scale,
                       const void* mla_q, const void* mla_kv, dsa_dtype mla_dtype,
                       int32_t* idx_out, void* out, float* lse,
                       void* ws, size_t ws_bytes, hipStream_t stream);
DSA_API size_t dsa_forward_workspace_size(int32_t B, int32_t q_len, int32_t S_max, int32_t H,
                                  int32_t topk, dsa_dtype index_dtype, dsa_dtype mla_dtype);

/* The indexer and the top-k of dsa_forward without the attention: the
 * Indexer's forward, which returns topk_indices ("详解DSA", Indexer code
 * block: Eq.(1) scores, then topk(min(index_topk, end_pos))).  Arguments as
 * in dsa_forward; idx_out [T, topk] int32 (required, device memory)
 * receives exactly the selection dsa_forward computes for the same inputs:
 * ascending positions, -1 padded.  Long prefills (q_len >= 64 with fp8
 * inputs) stream the scores as dsa_forward does; other shapes score into the
 * workspace chunk by chunk; with S_max <= topk every position is selected
 * and the indexer does not run (its inputs are still validated).  Errors as
 * dsa_forward's (DSA_ERR_INVALID_ARG for a NULL idx_out).
 * ws >= dsa_indexer_topk_workspace_size(...) bytes (0 when S_max <= topk). */
DSA_API dsa_status dsa_indexer_topk(const dsa_geom* geom, int32_t topk,
                            const void* index_q, dsa_dtype index_dtype, const float* index_q_scale,
                            const void* index_w, dsa_dtype index_w_dtype,
                            const void* index_k, const float* index_k_scale,
                            int32_t* idx_out, void* ws, size_t ws_bytes, hipStream_t stream);
DSA_API size_t dsa_indexer_topk_workspace_size(int32_t B, int32_t q_len, int32_t S_max, int32_t topk,
                                       dsa_dtype index_dtype);

/* Per-block fp8 quantisation of indexer inputs (the act_quant step of the
 * "详解DSA" Indexer code block, applied there to q and to k before the key
 * cache stores k; the "DSA计算流" section of that page keeps each key's scale
 * in the cache and folds the q-scale into the head weights).  The pages do
 * not print act_quant; the reading implemented: for every block of 128
 * consecutive elements
 *   scale        = max(amax, 2^-126) / 448           (fp32, amax = max |x|)
 *   codes[e]     = e4m3fn(x[e] / scale)               (fp32 quotient)
 * where e4m3fn() rounds to the nearest value, ties to the even code, gives
 * 448 for a quotient beyond it and keeps the quotient's sign.
 *
 *   x      [rows, 128] BF16 or F32 (e.g. q as [T*64, 128])
 *   codes  [rows, 128] uint8 e4m3fn codes;  scales [rows] fp32
 * x must be 16-byte aligned, codes and scales 4-byte aligned; rows >= 0.
 * A q_scale produced here is the q_scale argument of dsa_indexer_scores. */
DSA_API dsa_status dsa_indexer_quantize(const void* x, dsa_dtype x_dtype, int64_t rows,
                                uint8_t* codes, float* scales, hipStream_t stream);

/* Indexer key-cache append (the k_cache[:bsz, start_pos:end_pos] = k_fp8
 * and k_scale_cache lines of the "详解DSA" Indexer code block): the q_len
 * new keys of sequence b are quantised as in dsa_indexer_quantize and
 * written at positions L_b - q_len + i, i < q_len, with
 * L_b = clamp(seq_lens[b], 0, S_max) (so end_pos = L_b, the convention of
 * the query positions); positions below zero are skipped and no other entry
 * of either cache is touched.
 *
 *   k_new          [B, q_len, 128] BF16 or F32 (16-byte aligned)
 *   k_cache        [B, S_max, 128] uint8 e4m3fn codes (4-byte aligned)
 *   k_scale_cache  [B, S_max] fp32 (4-byte aligned) */
DSA_API dsa_status dsa_indexer_cache_append(const dsa_geom* geom, const void* k_new, dsa_dtype k_dtype,
                                    uint8_t* k_cache, float* k_scale_cache, hipStream_t stream);

/* ---------------------------------------------------------------------
 * Paged caches.  The charlestar page ("DeepSeek V3.2 稀疏注意力") raises
 * paged KV twice: in "Prefill 与 decode 中发生了什么" (Decode), top-k
 * positions must be mapped to physical KV pages and the selected entries
 * spread over many pages; in "Top-k 是算法与 kernel 的交界面", a logical
 * position becomes a page and an offset.  Here a cache is a POOL of
 * num_pages pages of page_size tokens shared by all sequences, plus a block
 * table: token s of sequence b lives in row s % page_size of page
 * block_table[b * max_pages + s / page_size].  Every result equals the
 * contiguous call's on the cache that the table describes (same kernels,
 * same arithmetic); seq_lens, positions, the causal rule and idx stay
 * LOGICAL positions.
 *
 *   block_table  DEVICE [B, max_pages] int32 page ids (4-byte aligned)
 *   page_size    a power of two, 64 <= page_size <= 65536
 *   max_pages    >= 1 with max_pages * page_size >= S_max, B * max_pages < 2^31
 *   num_pages    >= 1 with num_pages * page_size < 2^31 (pool rows fit int32)
 * Only the table entries of pages holding tokens s < clamp(seq_lens[b], 0,
 * S_max) are read.  They should lie in [0, num_pages); the kernels clamp any
 * other id into that range, so a bad entry reads or writes a wrong page of
 * the pool but never memory outside it.  Pages may be shared or reordered
 * freely between sequences.  The library keeps no pointer to the table. */
typedef struct {
  const int32_t* block_table;
  int32_t max_pages;
  int32_t page_size;
  int64_t num_pages;
} dsa_pages;

/* dsa_indexer_scores on paged fp8 (or f32) key caches:
 *   k_pool        [num_pages, page_size, 128] same dtype as q
 *   k_scale_pool  [num_pages, page_size] fp32 or NULL (= 1)
 * Other arguments, results and errors as in dsa_indexer_scores; a NULL or
 * invalid `pages` gives DSA_ERR_INVALID_ARG. */
DSA_API dsa_status dsa_indexer_scores_paged(const dsa_geom* geom, const dsa_pages* pages,
                              const void* q, dsa_dtype q_dtype, const float* q_scale,
                              const void* w, dsa_dtype w_dtype,
                              const void* k_pool, dsa_dtype k_dtype, const float* k_scale_pool,
                              int32_t row_begin, int32_t row_count,
                              float* scores, int64_t ld, hipStream_t stream);

/* dsa_sparse_mla on a paged latent cache:
 *   kv_pool [num_pages, page_size, 576] BF16 or F32 (the dtype of q)
 * idx holds logical positions as in dsa_sparse_mla; they are translated to
 * pool rows inside the workspace before the gather, so the attention reads
 * the pool with no table look-up per entry.
 * ws >= dsa_sparse_mla_paged_workspace_size(...) bytes (256-byte aligned). */
DSA_API dsa_status dsa_sparse_mla_paged(const dsa_geom* geom, const dsa_pages* pages, int32_t H, int32_t k,
                          float sm_scale, const void* q, dsa_dtype dtype, const void* kv_pool,
                          const int32_t* idx, void* out, float* lse,
                          void* ws, size_t ws_bytes, hipStream_t stream);
DSA_API size_t dsa_sparse_mla_paged_workspace_size(int32_t B, int32_t q_len, int32_t H, int32_t k,
                                     dsa_dtype dtype);

/* dsa_forward on paged caches (index_k_pool / index_k_scale_pool as in
 * dsa_indexer_scores_paged, mla_kv_pool as in dsa_sparse_mla_paged).
 * Long prefills stream as in dsa_forward (the key tiles are read from their
 * pages); other shapes score into the workspace.
 * ws >= dsa_forward_paged_workspace_size(...) bytes. */
DSA_API dsa_status dsa_forward_paged(const dsa_geom* geom, const dsa_pages* pages, int32_t H, int32_t topk,
                       float sm_scale,
                       const void* index_q, dsa_dtype index_dtype, const float* index_q_scale,
                       const void* index_w, dsa_dtype index_w_dtype,
                       const void* index_k_pool, const float* index_k_scale_pool,
                       const void* mla_q, const void* mla_kv_pool, dsa_dtype mla_dtype,
                       int32_t* idx_out, void* out, float* lse,
                       void* ws, size_t ws_bytes, hipStream_t stream);
DSA_API size_t dsa_forward_paged_workspace_size(int32_t B, int32_t q_len, int32_t S_max, int32_t H,
                                  int32_t topk, dsa_dtype index_dtype, dsa_dtype mla_dtype);

/* dsa_indexer_cache_append into paged pools: the new key of position s of
 * sequence b goes to pool row s % page_size of its page.
 *   k_pool [num_pages, page_size, 128] uint8;  k_scale_pool [num_pages, page_size] fp32 */
DSA_API dsa_status dsa_indexer_cache_append_paged(const dsa_geom* geom, const dsa_pages* pages,
                                    const void* k_new, dsa_dtype k_dtype,
                                    uint8_t* k_pool, float* k_scale_pool, hipStream_t stream);

/* MHA-mode prefill for sequences no longer than top-k ("详解DSA", section
 * "DSA计算流 & 性能分析": prefill inside top-k runs in MHA mode, and a
 * sequence no longer than top-k keeps every position so the indexer can be
 * skipped; the MHA branch of the MLA forward code block on that page; the
 * charlestar page's short-prompt paragraph: a masked MHA stands in for DSA
 * when L <= k).  The latent rows are decompressed per head through wkv_b,
 *   [k_nope | v][b, s, h] = wkv_b[h] . kv[b, s, 0:512]      (128 + 128 dims)
 * and every query attends causally to all keys up to its position:
 *   k_s      = [k_nope[b,s,h] (128) | kv[b, s, 512:576] (64, shared)]
 *   z_s      = sm_scale * q[t, h, :] . k_s                    for s <= pos(t)
 *   out[t,h] = sum_s softmax(z)_s * v[b, s, h]     lse[t,h] = log sum_s exp(z_s)
 * This equals the DSA forward (MQA mode, dsa_forward) with weights absorbed
 * whenever every seq_lens[b] <= topk, the case it is meant for: there the
 * top-k keeps every position.  Longer sequences get dense causal attention,
 * not DSA.
 *
 *   q     [T, H, 192] BF16 (q_nope 128 | q_pe 64)
 *   kv    [B, S_max, 576] BF16 (the latent cache of dsa_sparse_mla)
 *   wkv_b [H, 256, 512] BF16 (per head: the 128 k_nope rows, then the 128 v rows)
 *   out   [T, H, 128] BF16;  lse [T, H] fp32 or NULL
 * 1 <= H <= 128; dtype must be DSA_BF16 (else DSA_ERR_UNSUPPORTED).
 * ws >= dsa_mha_prefill_workspace_size(B, S_max, H) bytes (holds the
 * decompressed keys and values, 512 bytes per (sequence, position, head)). */
DSA_API dsa_status dsa_mha_prefill(const dsa_geom* geom, int32_t H, float sm_scale,
                           const void* q, const void* kv, const void* wkv_b, dsa_dtype dtype,
                           void* out, float* lse, void* ws, size_t ws_bytes, hipStream_t stream);
DSA_API size_t dsa_mha_prefill_workspace_size(int32_t B, int32_t S_max, int32_t H);

/* Indexer KL objective, forward only ("详解DSA" Eq.(3)-(6): the dense
 * warm-up loss over every visible position, and the sparse-training loss
 * over the selected set S_t).  For each query row t over its set
 * (idx == NULL: every s <= pos(t); otherwise the entries 0 <= idx[t,m] <= pos(t),
 * other values skipped):
 *   v_s     = sum_h exp(sm_scale * q[t,h,:] . kv[b,s,:] - lse[t,h])   (the heads' attention weights, summed)
 *   p       = v / sum(v)                                  (Eq.(3): L1-normalised)
 *   p_hat   = softmax(scores[t, set])                     (Eq.(4))
 *   kl[t]   = sum_s p_s log(p_s / p_hat_s)                (Eq.(5) / (6); 0 for an empty set)
 *   *loss   = sum_t kl[t]                                 (if loss != NULL; rows summed in a fixed order)
 * lse is the attention's per-head natural-log normaliser over the same set
 * (the lse output of dsa_sparse_mla / dsa_forward for the selected set); any
 * per-head constant works, since Eq.(3) normalises the sum.
 *
 *   q [T, H, 576], kv [B, S_max, 576]: BF16 (the MQA-mode attention inputs)
 *   lse [T, H] fp32;  scores [T, ld] fp32 (ld >= S_max; only set positions read)
 *   idx [T, k] int32 or NULL;  kl [T] fp32;  loss: one fp32 or NULL
 * H a multiple of 32 up to 128; 1 <= k <= 16384 when idx is given.
 * ws >= dsa_indexer_kl_workspace_size(B, q_len, S_max, idx ? k : 0) bytes. */
DSA_API dsa_status dsa_indexer_kl(const dsa_geom* geom, int32_t H, float sm_scale,
                          const void* q, const void* kv, dsa_dtype dtype, const float* lse,
                          const float* scores, int64_t ld, const int32_t* idx, int32_t k,
                          float* kl, float* loss, void* ws, size_t ws_bytes, hipStream_t stream);
DSA_API size_t dsa_indexer_kl_workspace_size(int32_t B, int32_t q_len, int32_t S_max, int32_t k);

/* One workspace query for every call that takes a workspace.  Returns a
 * byte count that suffices for the named call at this geometry with ANY
 * dtype combination the call supports (the maximum of its own
 * *_workspace_size query over them), so a caller can size one buffer before
 * it knows the dtypes.  k is the top-k / selection width (dsa_topk's k,
 * dsa_sparse_mla's k, dsa_forward's and dsa_indexer_topk's topk,
 * dsa_indexer_kl's k with 0 = every
 * visible position); H the MLA heads.  For DSA_CALL_TOPK the rows are all
 * B*q_len rows.  The forward sizes assume idx_out != NULL (with NULL add
 * B*q_len*k*4 bytes rounded up to 256).  Returns 0 for calls that need no
 * workspace, for non-positive sizes and for an unknown which_call. */
typedef enum {
  DSA_CALL_TOPK = 0,
  DSA_CALL_SPARSE_MLA = 1,
  DSA_CALL_FORWARD = 2,
  DSA_CALL_SPARSE_MLA_PAGED = 3,
  DSA_CALL_FORWARD_PAGED = 4,
  DSA_CALL_MHA_PREFILL = 5,
  DSA_CALL_INDEXER_KL = 6,
  DSA_CALL_INDEXER_TOPK = 7
} dsa_call;
DSA_API size_t dsa_workspace_size(int32_t B, int32_t q_len, int32_t S_max, int32_t H, int32_t k,
                                  int which_call);

/* dsa_forward with no workspace argument, for callers that cannot allocate
 * device memory around the call: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation.  The scratch memory is a static
 * device array of DSA_NOALLOC_SCRATCH_BYTES owned by the library, one per GPU
 * (held from library load until the process ends); the call itself allocates
 * and frees nothing.  Arguments, results and errors as dsa_forward, minus
 * (ws, ws_bytes); the work runs on the stream's device.  Returns
 * DSA_ERR_WORKSPACE, before touching the device, when the call needs more
 * scratch than that: dsa_forward_workspace_size(...) bytes, plus
 * B*q_len*topk*4 rounded up to 256 when idx_out is NULL (decode steps fit,
 * e.g. 16 x 2 queries at context 131072 or 64 x 1 at 32768 with topk 2048
 * and 128 heads; long prefills do not).  Nothing in the array needs to start
 * at zero (the path clears what it counts into), so a call is unaffected by
 * what an earlier call left there.  Every call on one GPU shares that GPU's
 * array: calls that can overlap in time on one GPU (other streams, other
 * host threads) race and must be serialised by the caller. */
#define DSA_NOALLOC_SCRATCH_BYTES ((size_t)96 << 20)
DSA_API dsa_status dsa_forward_noalloc(const dsa_geom* geom, int32_t H, int32_t topk, float sm_scale,
                       const void* index_q, dsa_dtype index_dtype, const float* index_q_scale,
                       const void* index_w, dsa_dtype index_w_dtype,
                       const void* index_k, const float* index_k_scale,
                       const void* mla_q, const void* mla_kv, dsa_dtype mla_dtype,
                       int32_t* idx_out, void* out, float* lse, hipStream_t stream);

/* Static text for a status code. */
DSA_API const char* dsa_status_string(dsa_status status);

/* Library version "major.minor.patch". */
DSA_API const char* dsa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H */
