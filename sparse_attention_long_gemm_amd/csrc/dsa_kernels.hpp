// Internal launcher interface between the C ABI (dsa_api.cpp) and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dsa {

// indexer_topk.hip
int indexer_cap(int top_k);
size_t indexer_prefill_ws(int n_q, int top_k);
size_t indexer_paged_ws(int B, int max_pages, int page_size);
hipError_t launch_indexer_topk_prefill(const uint8_t* q_idx, const float* w, const uint8_t* k_idx,
                                       int n_keys, const int32_t* q_pos, int n_q, int H_I,
                                       int d_I, int top_k, int32_t* out_idx, void* ws,
                                       hipStream_t stream);
hipError_t launch_indexer_topk_batched(const uint8_t* q_idx, const float* w,
                                       const uint8_t* k_cache, const int32_t* page_table,
                                       int n_seq, int max_pages, int n_pages, int page_size,
                                       const int32_t* q_seq, const int32_t* q_pos, int n_q,
                                       int H_I, int d_I, int top_k, int32_t* out_idx, void* ws,
                                       hipStream_t stream);
hipError_t launch_indexer_kl(const uint8_t* q_idx, const float* w, const uint8_t* k_idx,
                             int n_keys, const int32_t* q_pos, const int32_t* idx, int n_q,
                             int top_k, int H_I, int d_I, const float* target, float* loss,
                             float* grad, hipStream_t stream);
hipError_t launch_indexer_topk_paged(const uint8_t* q_idx, const float* w, const uint8_t* k_cache,
                                     const int32_t* page_table, const int32_t* ctx_lens, int B,
                                     int max_pages, int n_pages, int page_size, int H_I, int d_I,
                                     int top_k, int32_t* out_idx, void* ws, hipStream_t stream);

// cache_write.hip
hipError_t launch_cache_append(const uint16_t* k_new, const uint16_t* kv_new, const int32_t* seq,
                               const int32_t* pos, const int32_t* page_table, int T,
                               int max_pages, int n_pages, int page_size, int d_I, int D_k,
                               uint8_t* k_cache, uint16_t* kv_cache, hipStream_t stream);

// sparse_mqa.hip
struct MqaArgs {
  const uint16_t* q;
  const uint16_t* kv;
  const int32_t* idx;
  const int32_t* qpos_or_ctx;  // prefill: q_pos; decode: ctx_lens
  const int32_t* page_table;   // nullptr: contiguous prefill
  const int32_t* q_seq;        // batched prefill: row -> sequence (nullptr: all sequence 0)
  int n_seq;                   // 0: decode (row qi = sequence qi); > 0: batched prefill rows
  int max_pages, n_pages, page_size;
  int n_kv;
  int n_q, H, D_k, D_v, top_k;
  float scale;
  int n_split, rows_per_split;
  uint16_t* out;
  float* lse;
  uint16_t* part_o;   // decode partials: o / l in bf16 [n_q, n_split, H, D_v]
  float* part_ml;     // running max (log2 units) and sum [n_q, n_split, H, 2]
};
bool mqa_shape_supported(int D_k, int D_v);
hipError_t launch_sparse_mqa(const MqaArgs& a, hipStream_t stream);
// Dense causal attention over positions 0..t (idx unused); n_split / rows_per_split set by the
// caller with rows_per_split = dense_rows_per_split().
hipError_t launch_dense_mqa(const MqaArgs& a, hipStream_t stream);
int dense_rows_per_split();
// Main-attention probabilities of each listed entry, summed over heads and divided by H
// (contiguous rows, n_split = 1), from the forward's natural-log lse.
hipError_t launch_mqa_probs(const MqaArgs& a, const float* lse_in, float* probs,
                            hipStream_t stream);
// Sparse MQA backward (contiguous rows): P / dS to the workspace, dQ (fp32, written), dKV
// (fp32, accumulated with atomics).
hipError_t launch_mqa_backward(const MqaArgs& a, const float* lse_in, const uint16_t* o_fwd,
                               const uint16_t* d_out, uint16_t* p_ws, uint16_t* ds_ws,
                               float* dq, float* dkv, hipStream_t stream);

// Bytes of the per-device static scratch array of the allocation-free decode entry point.
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
// Device address of the current GPU's scratch array (looked up once per device).
hipError_t noalloc_scratch(void** ptr);

}  // namespace dsa
