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
hipError_t launch_indexer_topk_paged(const uint8_t* q_idx, const float* w, const uint8_t* k_cache,
                                     const int32_t* page_table, const int32_t* ctx_lens, int B,
                                     int max_pages, int n_pages, int page_size, int H_I, int d_I,
                                     int top_k, int32_t* out_idx, void* ws, hipStream_t stream);

// sparse_mqa.hip
struct MqaArgs {
  const uint16_t* q;
  const uint16_t* kv;
  const int32_t* idx;
  const int32_t* qpos_or_ctx;  // prefill: q_pos; decode: ctx_lens
  const int32_t* page_table;   // nullptr: contiguous prefill
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

}  // namespace dsa
