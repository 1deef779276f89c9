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
  DSA_ERR_HIP = -4                /* a launch failed (hipGetLastError after the launch)     */
} dsa_status;

/* ABI version of the loaded library (DSA_ABI_VERSION at build time). */
int dsa_abi_version(void);

/* Static, human-readable name of a status code (never NULL). */
const char* dsa_status_string(int status);

/* ---------------------------------------------------------------------------------------
 * Prefill indexer + top-k, one contiguous sequence.
 *
 * q_idx   [n_q, H_I, d_I]  FP8   indexer queries of the n_q query rows
 * w       [n_q, H_I]       fp32  per-row head weights (any finite values, any sign)
 * k_idx   [n_keys, d_I]    FP8   indexer keys of positions 0..n_keys-1
 * q_pos   [n_q]            int32 position t of each query row; candidates are s in [0, t]
 *                                with t clamped to n_keys-1; a negative t selects nothing
 * out_idx [n_q, top_k]     int32 selection, ascending positions then -1 (see above)
 *
 * Scores are computed in fp32 from exact FP8 products; the n_q x n_keys score matrix is
 * never stored: each workgroup streams key tiles and keeps a per-row candidate list in the
 * workspace.  Selection is exact under (score desc, position asc), with -0 == +0.
 * ------------------------------------------------------------------------------------- */
size_t dsa_indexer_topk_workspace_size(int32_t n_q, int32_t top_k);

dsa_status dsa_indexer_topk(const uint8_t* q_idx, const float* w, const uint8_t* k_idx,
                            int32_t n_keys, const int32_t* q_pos, int32_t n_q, int32_t H_I,
                            int32_t d_I, int32_t top_k, int32_t* out_idx, void* workspace,
                            size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------------------
 * Decode indexer + top-k over a paged key cache: one new query per sequence at t = ctx-1.
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
 * ------------------------------------------------------------------------------------- */
size_t dsa_indexer_topk_paged_workspace_size(int32_t B, int32_t max_pages, int32_t page_size);

dsa_status dsa_indexer_topk_paged(const uint8_t* q_idx, const float* w, const uint8_t* k_cache,
                                  const int32_t* page_table, const int32_t* ctx_lens, int32_t B,
                                  int32_t max_pages, int32_t n_pages, int32_t page_size,
                                  int32_t H_I, int32_t d_I, int32_t top_k, int32_t* out_idx,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------------------
 * Sparse MQA prefill over the selected rows of one contiguous sequence.
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
 * Sparse MQA decode over a paged KV cache: one query per sequence, t = ctx-1.
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
 * Both return DSA_ERR_INVALID_ARG for out-of-range arguments (nothing launched).
 * ------------------------------------------------------------------------------------- */
dsa_status dsa_ceiling_mfma(int32_t kind, int32_t n_wg, int32_t iters, float* sink,
                            double* flops, hipStream_t stream);
dsa_status dsa_ceiling_read(const void* src, size_t bytes, int32_t n_wg, float* sink,
                            hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* DSA_H_ */
