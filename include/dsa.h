/*
 * dsa.h — C ABI of the DeepSeek Sparse Attention (DSA) hot path on AMD Instinct MI355X (gfx950).
 *
 * The path has three steps per query token t of a causal sequence:
 *   1. lightning-indexer score  I[t,s] = sum_j w[t,j] * ReLU(q_I[t,j,:] . k_I[s,:]),  s <= t,
 *      FP8 operands, a few indexer heads (jdon.com "DeepSeek-V3.2-Exp" article, paragraph on
 *      the lightning indexer; openi.cn "DeepSeek-V3.2" page, section on the technology behind
 *      the model: the indexer scores the query against the preceding tokens);
 *   2. fine-grained selection of the top_k (2048) keys by that score, ties broken toward the
 *      lower position (jdon.com article, paragraph on fine-grained token selection);
 *   3. attention in MQA mode over only the selected shared latent KV rows: K is the whole
 *      row (D_k = 576 = 512 latent + 64 rope), V its first D_v (512) dims, shared by all
 *      query heads (openi.cn page, item on MLA run in MQA mode).
 * Decode reads the keys and KV rows through a page table (page size 64 in the serving
 * recipe on the mundobytes.com page, section "Quick guide to running locally"; paged indexer
 * kernels are named in its section "Open kernels and ecosystem support").
 *
 * Conventions shared by every entry point
 *  - Every pointer argument is a DEVICE pointer owned by the caller.  The library never
 *    allocates, frees or synchronises inside these calls; scratch memory is the caller's
 *    `workspace` (size from the matching *_workspace_size function, any alignment >= 256 B).
 *  - Work is enqueued on `stream` and the call returns; results are valid once the stream
 *    has reached that point.  Calls on different streams may run concurrently if they use
 *    different outputs and workspaces.
 *  - FP8 operands are OCP e4m3fn bytes with no scale factors.  bf16 operands/outputs are
 *    raw bf16 bit patterns (uint16_t), round-to-nearest-even on output.
 *  - Arguments are checked on the host before anything is launched.  On any non-zero status
 *    nothing has been enqueued, except DSA_ERR_HIP, which reports a launch failure.
 *  - Index rows hold the n = min(top_k, t+1) selected positions first, in ascending order,
 *    then -1.  The attention calls skip any index that is -1 or outside [0, t] (or outside
 *    [0, ctx) in decode, or whose page-table entry is outside [0, n_pages)), so a bad index
 *    can never cause an out-of-bounds read.  A query with no attended entry gets o = 0 and
 *    lse = -inf.
 *  - Supported shapes: d_I a multiple of 16 and <= 128; H_I <= 64; 1 <= top_k <= 2048;
 *    H <= 128; (D_k, D_v) in {(576, 512), (64, 64), (96, 64)}.  Other shapes return
 *    DSA_ERR_UNSUPPORTED_SHAPE.
 */
#ifndef DSA_H_
#define DSA_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSA_ABI_VERSION 1

typedef enum dsa_status {
  DSA_OK = 0,
  DSA_ERR_INVALID_ARG = -1,       /* null required pointer, negative size, bad page size... */
  DSA_ERR_UNSUPPORTED_SHAPE = -2, /* no kernel instance for this (H_I, d_I, H, D_k, D_v, k)  */
  DSA_ERR_WORKSPACE_TOO_SMALL = -3,
  DSA_ERR_HIP = -4,               /* a launch failed (hipGetLastError after the launch)     */
  DSA_ERR_SCRATCH_LIMIT = -5      /* the allocation-free entry point's scratch is too small */
} dsa_status;

/* ABI version of the loaded library (DSA_ABI_VERSION at build time). */
int dsa_abi_version(void);

/* Static, human-readable name of a status code (never NULL). */
const char* dsa_status_string(int status);

/* ---------------------------------------------------------------------------------------
 * Prefill indexer + top-k, one contiguous sequence.  Defines steps 1-2 above: the lightning
 * indexer's ReLU-activated, head-weighted FP8 score and the top_k selection (jdon.com
 * "DeepSeek-V3.2-Exp" article, paragraphs on the lightning indexer and on fine-grained token
 * selection; mundobytes.com page, section "Introduction of DeepSeek Sparse Attention (DSA)").
 *
 * q_idx   [n_q, H_I, d_I]  FP8   indexer queries of the n_q query rows
 * w       [n_q, H_I]       fp32  per-row head weights (any finite values, any sign)
 * k_idx   [n_keys, d_I]    FP8   indexer keys of positions 0..n_keys-1
 * q_pos   [n_q]            int32 position t of each query row; candidates are s in [0, t]
 *                                with t clamped to n_keys-1; a negative t selects nothing
 * out_idx [n_q, top_k]     int32 selection, ascending positions then -1 (see above)
 *
 * The n_q x n_keys score matrix is never stored: each workgroup streams key tiles and keeps
 * a per-row candidate list in the workspace.  The selection is the exact top_k of the scores
 * as computed, under (score desc, position asc), with -0 == +0.
 * Precision: scores are computed in fp32 from exact FP8 products, with ReLU applied as
 * w ReLU(x) = (w x + w |x|) / 2 (the |x| half by fma per head, the linear half as one product
 * with the weighted query sum).  When every product sum and weighted partial sum is exact in
 * fp32 (FP8 operands on a dyadic grid with power-of-two weights: the tested workloads) the
 * computed scores equal the definition's and the selection is bit-exact.  Otherwise each
 * computed score is within 2^-16 * M of the exact one, M = sum_j |w[t,j]| sum_i
 * |q_I[t,j,i]| |k_I[s,i]|; a key whose heads are all <= 0 scores within that bound of 0 rather
 * than exactly 0, so the order among such keys need not follow their positions.
 * ------------------------------------------------------------------------------------- */
size_t dsa_indexer_topk_workspace_size(int32_t n_q, int32_t top_k);

dsa_status dsa_indexer_topk(const uint8_t* q_idx, const float* w, const uint8_t* k_idx,
                            int32_t n_keys, const int32_t* q_pos, int32_t n_q, int32_t H_I,
                            int32_t d_I, int32_t top_k, int32_t* out_idx, void* workspace,
                            size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------------------
 * Decode indexer + top-k over a paged key cache: one new query per sequence at t = ctx-1.
 * Steps 1-2 for one query per sequence over the cached keys, read through the page table of
 * the serving recipe (mundobytes.com page, sections "Quick guide to running locally" and
 * "Open kernels and ecosystem support": paged indexer logits; jdon.com article, paragraph on
 * inference cost: decode revisits only the selected tokens).
 *
 * q_idx      [B, H_I, d_I]               FP8
 * w          [B, H_I]                    fp32
 * k_cache    [n_pages, page_size, d_I]   FP8   logical row s of sequence b lives at
 *                                              page page_table[b*max_pages + s/page_size],
 *                                              slot s % page_size
 * page_table [B, max_pages]              int32 entries beyond the context are not read;
 *                                              an entry outside [0, n_pages) inside the
 *                                              context is read as a page of all-zero keys
 *                                              (score 0), never out of bounds
 * ctx_lens   [B]                         int32 context length (>= 0, <= max_pages*page_size);
 *                                              candidates are s in [0, ctx)
 * out_idx    [B, top_k]                  int32 logical positions, ascending, then -1
 *
 * Scores are sum_j w_j max(x_j, 0) accumulated by fma in fp32 from the exact FP8 products: a
 * key whose heads are all <= 0 scores exactly 0; otherwise the same 2^-16 * M bound as the
 * prefill indexer holds, and on a dyadic grid with power-of-two weights the selection is
 * bit-exact.  The selection is the exact top_k of the computed scores (score desc, position
 * asc).
 * ------------------------------------------------------------------------------------- */
size_t dsa_indexer_topk_paged_workspace_size(int32_t B, int32_t max_pages, int32_t page_size);

dsa_status dsa_indexer_topk_paged(const uint8_t* q_idx, const float* w, const uint8_t* k_cache,
                                  const int32_t* page_table, const int32_t* ctx_lens, int32_t B,
                                  int32_t max_pages, int32_t n_pages, int32_t page_size,
                                  int32_t H_I, int32_t d_I, int32_t top_k, int32_t* out_idx,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------------------
 * Batched prefill indexer + top-k over paged key caches: many sequences per call, each query
 * row of any length of prefix (variable-length batches, and chunked prefill of a chunk of
 * queries against the prefix already in the cache).  The serving layout is the 64-token paged
 * cache of the mundobytes.com page (section "Quick guide to running locally"); the score and
 * the selection are those of dsa_indexer_topk (jdon.com article, paragraphs on the lightning
 * indexer and on fine-grained token selection).
 *
 * q_idx      [n_q, H_I, d_I]             FP8   indexer queries
 * w          [n_q, H_I]                  fp32  head weights
 * k_cache    [n_pages, page_size, d_I]   FP8   keys of all sequences (page_size a power of
 *                                              two >= 8, else DSA_ERR_UNSUPPORTED_SHAPE),
 *                                              written e.g. by dsa_cache_append
 * page_table [n_seq, max_pages]          int32 logical row s of sequence b at page
 *                                              page_table[b*max_pages + s/page_size]; an
 *                                              entry outside [0, n_pages) in a row's range
 *                                              reads as a page of zero keys
 * q_seq      [n_q]                       int32 sequence of each query row (NULL: all 0); a
 *                                              sequence outside [0, n_seq) selects nothing.
 *                                              Rows sorted by sequence run fastest (a group of
 *                                              16 consecutive rows streams the keys of each
 *                                              sequence it touches in turn)
 * q_pos      [n_q]                       int32 position t of each row in its sequence:
 *                                              candidates s in [0, t], t clamped to
 *                                              max_pages*page_size - 1; t < 0 selects nothing
 * out_idx    [n_q, top_k]                int32 logical positions, ascending, then -1
 * workspace: dsa_indexer_topk_workspace_size(n_q, top_k) bytes.  Precision and selection
 * rules are those of dsa_indexer_topk.
 * ------------------------------------------------------------------------------------- */
dsa_status dsa_indexer_topk_batched(const uint8_t* q_idx, const float* w,
                                    const uint8_t* k_cache, const int32_t* page_table,
                                    int32_t n_seq, int32_t max_pages, int32_t n_pages,
                                    int32_t page_size, const int32_t* q_seq,
                                    const int32_t* q_pos, int32_t n_q, int32_t H_I, int32_t d_I,
                                    int32_t top_k, int32_t* out_idx, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------------------
 * Batched sparse MQA over paged KV caches: row i (sequence q_seq[i], NULL: 0, position
 * q_pos[i]) attends the selected rows of its sequence through the page table, as
 * dsa_sparse_mqa_prefill does for one contiguous sequence (openi.cn page, MLA/MQA item;
 * mundobytes.com page, "Quick guide to running locally" for the paging).
 *
 * q [n_q, H, D_k] bf16, kv_cache [n_pages, page_size, D_k] bf16, page_table [n_seq,
 * max_pages], q_seq / q_pos [n_q], idx [n_q, top_k] logical positions (entries outside
 * [0, t], or on a page-table entry outside [0, n_pages), are skipped), out [n_q, H, D_v]
 * bf16, lse [n_q, H] fp32 or NULL.  A row of a sequence outside [0, n_seq) gets o = 0,
 * lse = -inf.
 * ------------------------------------------------------------------------------------- */
dsa_status dsa_sparse_mqa_batched(const uint16_t* q, const uint16_t* kv_cache,
                                  const int32_t* page_table, int32_t n_seq, int32_t max_pages,
                                  int32_t n_pages, int32_t page_size, const int32_t* q_seq,
                                  const int32_t* q_pos, const int32_t* idx, int32_t n_q,
                                  int32_t H, int32_t D_k, int32_t D_v, int32_t top_k,
                                  float scale, uint16_t* out, float* lse, hipStream_t stream);

/* ---------------------------------------------------------------------------------------
 * Sparse MQA prefill over the selected rows of one contiguous sequence.  Step 3: attention
 * in MQA mode over the selected shared latent rows only (openi.cn "DeepSeek-V3.2" page, item
 * on MLA run in MQA mode; jdon.com article, paragraph on fine-grained token selection).
 *
 * q      [n_q, H, D_k]     bf16  queries
 * kv     [n_kv, D_k]       bf16  shared latent KV rows; K = whole row, V = first D_v dims
 * idx    [n_q, top_k]      int32 selected positions (e.g. dsa_indexer_topk's output)
 * q_pos  [n_q]             int32 position t of each row (entries > t are skipped)
 * out    [n_q, H, D_v]     bf16  o[t,h] = sum_s softmax_s(scale * q[t,h].kv[s]) kv[s,:D_v]
 * lse    [n_q, H]          fp32  natural-log log-sum-exp of the scaled logits, or NULL
 * Accumulation is fp32; probabilities enter the value product as bf16.
 * ------------------------------------------------------------------------------------- */
dsa_status dsa_sparse_mqa_prefill(const uint16_t* q, const uint16_t* kv, int32_t n_kv,
                                  const int32_t* idx, const int32_t* q_pos, int32_t n_q,
                                  int32_t H, int32_t D_k, int32_t D_v, int32_t top_k,
                                  float scale, uint16_t* out, float* lse, hipStream_t stream);

/* ---------------------------------------------------------------------------------------
 * Sparse MQA decode over a paged KV cache: one query per sequence, t = ctx-1.  Step 3 for
 * the decode query through the page table (openi.cn page, MLA/MQA item; mundobytes.com page,
 * "Quick guide to running locally" for the 64-token pages).
 *
 * q        [B, H, D_k]                bf16
 * kv_cache [n_pages, page_size, D_k]  bf16  same paging as dsa_indexer_topk_paged
 * idx      [B, top_k]                 int32 logical positions (entries >= ctx are skipped)
 * out      [B, H, D_v] bf16, lse [B, H] fp32 or NULL
 * The selected rows of each sequence are split over n_split workgroups (1 <= n_split <= 16,
 * top_k rows divided evenly; pass 0 for the library's choice) whose partial results are
 * merged by their log-sum-exp; the workspace holds the partials (each split's output
 * normalised by its own softmax sum, in bf16, plus its running max and sum in fp32).
 * ------------------------------------------------------------------------------------- */
size_t dsa_sparse_mqa_decode_workspace_size(int32_t B, int32_t H, int32_t D_v, int32_t top_k,
                                            int32_t n_split);

dsa_status dsa_sparse_mqa_decode(const uint16_t* q, const uint16_t* kv_cache,
                                 const int32_t* page_table, const int32_t* ctx_lens,
                                 const int32_t* idx, int32_t B, int32_t max_pages,
                                 int32_t n_pages, int32_t page_size, int32_t H, int32_t D_k,
                                 int32_t D_v, int32_t top_k, float scale, int32_t n_split,
                                 uint16_t* out, float* lse, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------------------
 * Dense causal MLA/MQA attention: the baseline the selection is measured against.  Every
 * query row attends all positions 0..t (what DSA replaces by the top_k selected ones: the
 * O(L^2) -> O(L k) step of the jdon.com "DeepSeek-V3.2-Exp" article, and its paragraph on
 * inference cost comparing the two per token position).  Same shapes, layouts and numerics
 * as the sparse calls (bf16 MFMA, fp32 softmax and accumulation); the positions of a row are
 * split over workgroups of 2048 and merged by their log-sum-exp through the workspace.
 *
 * dsa_dense_mqa_prefill: q [n_q, H, D_k], kv [n_kv, D_k], q_pos [n_q] (t clamped to n_kv-1,
 *   t < 0 attends nothing), out [n_q, H, D_v], lse [n_q, H] or NULL;
 *   workspace >= dsa_dense_mqa_workspace_size(n_q, H, D_v, n_kv) bytes.
 * dsa_dense_mqa_decode: one query per sequence over its positions [0, ctx) through the page
 *   table (as dsa_sparse_mqa_decode; positions on a page-table entry outside [0, n_pages)
 *   are skipped); workspace >= dsa_dense_mqa_workspace_size(B, H, D_v,
 *   max_pages * page_size) bytes.
 * The workspace size is 0 when max_len <= 2048 (no split); more than 65535 splits
 * (max_len > 2^27) returns DSA_ERR_UNSUPPORTED_SHAPE.
 * ------------------------------------------------------------------------------------- */
size_t dsa_dense_mqa_workspace_size(int32_t n_q, int32_t H, int32_t D_v, int32_t max_len);

dsa_status dsa_dense_mqa_prefill(const uint16_t* q, const uint16_t* kv, int32_t n_kv,
                                 const int32_t* q_pos, int32_t n_q, int32_t H, int32_t D_k,
                                 int32_t D_v, float scale, uint16_t* out, float* lse,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream);

dsa_status dsa_dense_mqa_decode(const uint16_t* q, const uint16_t* kv_cache,
                                const int32_t* page_table, const int32_t* ctx_lens, int32_t B,
                                int32_t max_pages, int32_t n_pages, int32_t page_size, int32_t H,
                                int32_t D_k, int32_t D_v, float scale, uint16_t* out,
                                float* lse, void* workspace, size_t workspace_bytes,
                                hipStream_t stream);

/* ---------------------------------------------------------------------------------------
 * The indexer's training signal: KL divergence from the main attention's distribution to the
 * indexer's (the indexer is trained to reproduce how the main attention distributes itself,
 * with a KL-divergence loss: jdon.com "DeepSeek-V3.2-Exp" article, paragraph on the indexer's
 * warm-up; in the sparse stage the indexer's loss stays separate from the model's).  Forward
 * and the gradient with respect to the indexer scores, over each row's index list S (entries
 * that are -1 or outside [0, t] are not part of it; for the dense warm-up pass every position
 * as the list):
 *   target[t,e] = (1/H) sum_h softmax_S(scale q[t,h] . kv[s])[e]    (main attention)
 *   q_I[t,e]    = softmax_S(I[t, idx[t,e]])                          (indexer)
 *   loss[t]     = sum_e target (log target - log q_I),   grad[t,e] = q_I - target
 *
 * q [n_q, H, D_k] bf16, kv [n_kv, D_k] bf16, idx [n_q, top_k], q_pos [n_q], lse [n_q, H] fp32:
 * the forward's log-sum-exp over the same lists (dsa_sparse_mqa_prefill's lse output);
 * q_idx [n_q, H_I, d_I] FP8, w [n_q, H_I], k_idx [n_kv, d_I] FP8 (the indexer's inputs);
 * outputs (device, fp32): target [n_q, top_k] (0 for entries outside S), loss [n_q]
 * (0 for an empty list), grad [n_q, top_k] or NULL (0 outside S).  D_k in {576, 64, 96}.
 * The logits are recomputed with bf16 MFMAs and fp32 accumulation as in the forward; the
 * indexer scores are recomputed as the decode scorer forms them.
 * ------------------------------------------------------------------------------------- */
dsa_status dsa_indexer_kl(const uint16_t* q, const uint16_t* kv, int32_t n_kv,
                          const int32_t* idx, const int32_t* q_pos, const float* lse,
                          int32_t n_q, int32_t H, int32_t D_k, int32_t top_k, float scale,
                          const uint8_t* q_idx, const float* w, const uint8_t* k_idx,
                          int32_t H_I, int32_t d_I, float* target, float* loss, float* grad,
                          hipStream_t stream);

/* ---------------------------------------------------------------------------------------
 * Sparse MQA backward: the gradients of sum(d_out * out) with respect to q and the KV rows,
 * for the attention of dsa_sparse_mqa_prefill (the main model's loss in the sparse training
 * stage flows through the selected entries only: jdon.com "DeepSeek-V3.2-Exp" article,
 * sparse-training paragraph; MQA on the shared rows: openi.cn page, MLA/MQA item).  Per row t
 * and head h over the listed entries (the selection is not differentiated):
 *   P = exp(scale q.kv - lse), dP = d_out . v, dS = P (dP - sum_d d_out out),
 *   d_q[t,h]     = scale sum_e dS kv_e                       (written, fp32 [n_q, H, D_k])
 *   d_kv[s_e]   += scale sum_h dS q[t,h] + sum_h P d_out[t,h] (fp32 [n_kv, D_k], V part in the
 *                                                              first D_v dims; ACCUMULATED:
 *                                                              zero it before the first call)
 * q, kv, idx, q_pos as in dsa_sparse_mqa_prefill; out [n_q, H, D_v] bf16 and lse [n_q, H]
 * fp32 are that call's outputs; d_out [n_q, H, D_v] bf16.  workspace: P and dS in bf16,
 * dsa_sparse_mqa_backward_workspace_size(n_q, H, top_k) bytes.  d_kv takes fp32 atomic
 * adds, so its low-order bits depend on the order of the rows' contributions.
 * ------------------------------------------------------------------------------------- */
size_t dsa_sparse_mqa_backward_workspace_size(int32_t n_q, int32_t H, int32_t top_k);

dsa_status dsa_sparse_mqa_backward(const uint16_t* q, const uint16_t* kv, int32_t n_kv,
                                   const int32_t* idx, const int32_t* q_pos, const uint16_t* out,
                                   const float* lse, const uint16_t* d_out, int32_t n_q,
                                   int32_t H, int32_t D_k, int32_t D_v, int32_t top_k,
                                   float scale, float* d_q, float* d_kv, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------------------
 * Cache write: append new tokens to the paged caches the decode calls read.  Defines the step
 * just before the paged indexer and attention: the indexer keeps its keys in FP8 (jdon.com
 * "DeepSeek-V3.2-Exp" article, paragraph on the lightning indexer) in 64-token pages
 * (mundobytes.com page, sections "Quick guide to running locally" and "Open kernels and
 * ecosystem support"), next to the shared latent KV rows (openi.cn page, MLA/MQA item).
 *
 * k_new      [T, d_I]                   bf16  indexer keys of the new tokens, or NULL
 * kv_new     [T, D_k]                   bf16  latent KV rows of the new tokens, or NULL
 * seq        [T]                        int32 sequence of row r (page-table row), or NULL:
 *                                             row r belongs to sequence r
 * pos        [T]                        int32 logical position of row r in its sequence
 * page_table [B, max_pages]             int32 as in dsa_indexer_topk_paged
 * k_cache    [n_pages, page_size, d_I]  FP8   written at the rows' slots (if k_new)
 * kv_cache   [n_pages, page_size, D_k]  bf16  written at the rows' slots (if kv_new)
 *
 * Row r goes to page page_table[seq[r]*max_pages + pos[r]/page_size], slot pos[r] % page_size;
 * a row whose position is negative, whose page index is >= max_pages or whose page-table
 * entry is outside [0, n_pages) writes nothing.  The k_I values are quantised to e4m3fn by
 * rounding to nearest (ties to the even code), saturating finite values and infinities at
 * +-448, NaN to NaN; the KV rows are copied bit for bit.  Two rows with the same slot in one
 * call race (either may win).  Nothing else in the caches is touched.
 * Requires d_I a multiple of 16 (<= 128) and D_k a multiple of 8 (<= 1024), 16-byte aligned
 * rows in k_new / kv_new and 8-byte aligned caches.
 * ------------------------------------------------------------------------------------- */
dsa_status dsa_cache_append(const uint16_t* k_new, const uint16_t* kv_new, const int32_t* seq,
                            const int32_t* pos, const int32_t* page_table, int32_t T,
                            int32_t max_pages, int32_t n_pages, int32_t page_size, int32_t d_I,
                            int32_t D_k, uint8_t* k_cache, uint16_t* kv_cache,
                            hipStream_t stream);

/* ---------------------------------------------------------------------------------------
 * Allocation-free variant of dsa_sparse_mqa_decode, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 *
 * Same arguments, layouts, checks, kernels and results as dsa_sparse_mqa_decode, without the
 * workspace: the split partials live in a static device array of DSA_NOALLOC_SCRATCH_BYTES
 * that the library holds on every GPU it runs on until the process ends (its address on each
 * device is looked up once, on the first call there).  The call never allocates or frees.
 *  - A call whose partials need more than DSA_NOALLOC_SCRATCH_BYTES (the size
 *    dsa_sparse_mqa_decode_workspace_size reports for the same B, H, D_v, top_k, n_split)
 *    returns DSA_ERR_SCRATCH_LIMIT and enqueues nothing.  At H=128, D_v=512 the limit holds
 *    B * n_split <= 508 (e.g. B=64 with the library's 4 splits, or B=127 with 4).
 *  - Every call on one GPU shares that GPU's array: calls whose executions overlap on the
 *    same GPU (different streams, or host threads racing) race on it and give undefined
 *    results.  Calls ordered on one stream are safe: each writes every partial it reads, so
 *    nothing carries over from the previous call.
 * ------------------------------------------------------------------------------------- */
#define DSA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

dsa_status dsa_sparse_mqa_decode_noalloc(const uint16_t* q, const uint16_t* kv_cache,
                                         const int32_t* page_table, const int32_t* ctx_lens,
                                         const int32_t* idx, int32_t B, int32_t max_pages,
                                         int32_t n_pages, int32_t page_size, int32_t H,
                                         int32_t D_k, int32_t D_v, int32_t top_k, float scale,
                                         int32_t n_split, uint16_t* out, float* lse,
                                         hipStream_t stream);

/* ---------------------------------------------------------------------------------------
 * Measurement helpers (not part of the path).  They report what this GPU sustains on the
 * instruction shapes and the memory stream the path uses, so that roofline fractions can be
 * read against measured ceilings as well as against the published peaks.
 *
 * dsa_ceiling_mfma: n_wg workgroups of 512 threads each run `iters` iterations of independent
 *   MFMA chains on register operands: kind 0 = v_mfma_f32_32x32x16_bf16 (bf16), kind 1 =
 *   v_mfma_scale_f32_16x16x128_f8f6f4 with unscaled FP8 operands.  *flops (HOST pointer)
 *   receives the flop count of the launch; sink: device float[n_wg * 512], overwritten.
 * dsa_ceiling_read: streams `bytes` (a non-zero multiple of 16) from device memory `src` with
 *   16-byte non-temporal loads over n_wg workgroups of 256 threads; sink: device
 *   float[n_wg * 256], overwritten.
 * dsa_ceiling_gather: gathers rows of `row_bytes` bytes (a multiple of 16, at most 2048) from
 *   the device pool `pool` of n_rows rows along the index rows idx [n_q, top_k] int32 (device;
 *   top_k a multiple of 32; an entry outside [0, n_rows) reads row 0), 32 listed rows at a
 *   time by n_wg workgroups of 512 threads (8 waves, as the attention kernel): kind 0 moves
 *   them with the LDS DMA (global_load_lds_dwordx4), kind 1 with 16-byte loads into
 *   registers.  Bytes moved: n_q * top_k * row_bytes.  sink: device float[n_wg * 512],
 *   overwritten.
 * All return DSA_ERR_INVALID_ARG for out-of-range arguments (nothing launched).
 * ------------------------------------------------------------------------------------- */
dsa_status dsa_ceiling_mfma(int32_t kind, int32_t n_wg, int32_t iters, float* sink,
                            double* flops, hipStream_t stream);
dsa_status dsa_ceiling_read(const void* src, size_t bytes, int32_t n_wg, float* sink,
                            hipStream_t stream);
dsa_status dsa_ceiling_gather(int32_t kind, const void* pool, int64_t n_rows, int32_t row_bytes,
                              const int32_t* idx, int32_t n_q, int32_t top_k, int32_t n_wg,
                              float* sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* DSA_H_ */
