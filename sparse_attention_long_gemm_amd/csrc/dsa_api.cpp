// C ABI of the DSA hot path: argument checks, workspace sizing and kernel dispatch.
// Every check happens on the host before any launch; see include/dsa.h for the contract.
#include "dsa.h"

#include <math.h>

#include "dsa_kernels.hpp"

namespace {

constexpr int kMaxTopK = 2048;
constexpr int kMaxHI = 64;
constexpr int kMaxDI = 128;
constexpr int kMaxH = 128;
constexpr int kMaxSplit = 16;
constexpr int kSplitRows = 32;  // a split boundary always falls on a 32-row chunk

bool indexer_shape_ok(int H_I, int d_I, int top_k) {
  return H_I >= 1 && H_I <= kMaxHI && d_I >= 16 && d_I <= kMaxDI && d_I % 16 == 0 &&
         top_k >= 1 && top_k <= kMaxTopK;
}

bool paging_ok(int max_pages, int n_pages, int page_size) {
  return max_pages >= 1 && n_pages >= 1 && page_size >= 1 &&
         (long long)max_pages * page_size <= 0x7fffffffLL &&
         (long long)n_pages * page_size <= 0x7fffffffLL;
}

dsa_status from_hip(hipError_t e) { return e == hipSuccess ? DSA_OK : DSA_ERR_HIP; }

// Rows per split and split count actually used for `requested` splits (0 = choose).
void decode_split(int B, int top_k, int requested, int* n_split, int* rows_per_split) {
  int ns = requested;
  if (ns <= 0) {
    // aim for >= 256 workgroups (one per CU) without splitting below 256 rows
    ns = B > 0 ? (256 + B - 1) / B : 1;
    int max_by_rows = (top_k + 255) / 256;
    if (ns > max_by_rows) ns = max_by_rows;
  }
  if (ns > kMaxSplit) ns = kMaxSplit;
  if (ns < 1) ns = 1;
  int rps = (top_k + ns - 1) / ns;
  rps = (rps + kSplitRows - 1) / kSplitRows * kSplitRows;
  *rows_per_split = rps;
  *n_split = (top_k + rps - 1) / rps;
}

}  // namespace

extern "C" {

int dsa_abi_version(void) { return DSA_ABI_VERSION; }

const char* dsa_status_string(int status) {
  switch (status) {
    case DSA_OK: return "DSA_OK";
    case DSA_ERR_INVALID_ARG: return "DSA_ERR_INVALID_ARG: invalid argument";
    case DSA_ERR_UNSUPPORTED_SHAPE: return "DSA_ERR_UNSUPPORTED_SHAPE: no kernel for this shape";
    case DSA_ERR_WORKSPACE_TOO_SMALL: return "DSA_ERR_WORKSPACE_TOO_SMALL: workspace too small";
    case DSA_ERR_HIP: return "DSA_ERR_HIP: kernel launch failed";
    case DSA_ERR_SCRATCH_LIMIT:
      return "DSA_ERR_SCRATCH_LIMIT: the call needs more scratch than the allocation-free entry "
             "point holds (DSA_NOALLOC_SCRATCH_BYTES); use the workspace variant";
    default: return "unknown dsa_status";
  }
}

size_t dsa_indexer_topk_workspace_size(int32_t n_q, int32_t top_k) {
  if (n_q < 0 || top_k < 1 || top_k > kMaxTopK) return 0;
  return dsa::indexer_prefill_ws(n_q, top_k);
}

dsa_status dsa_indexer_topk(const uint8_t* q_idx, const float* w, const uint8_t* k_idx,
                            int32_t n_keys, const int32_t* q_pos, int32_t n_q, int32_t H_I,
                            int32_t d_I, int32_t top_k, int32_t* out_idx, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
  if (n_q < 0 || n_keys < 0) return DSA_ERR_INVALID_ARG;
  if (!indexer_shape_ok(H_I, d_I, top_k)) return DSA_ERR_UNSUPPORTED_SHAPE;
  if (n_q == 0) return DSA_OK;
  if (!q_idx || !w || !q_pos || !out_idx || (n_keys > 0 && !k_idx) || !workspace)
    return DSA_ERR_INVALID_ARG;
  if (workspace_bytes < dsa::indexer_prefill_ws(n_q, top_k)) return DSA_ERR_WORKSPACE_TOO_SMALL;
  return from_hip(dsa::launch_indexer_topk_prefill(q_idx, w, k_idx, n_keys, q_pos, n_q, H_I, d_I,
                                                   top_k, out_idx, workspace, stream));
}

size_t dsa_indexer_topk_paged_workspace_size(int32_t B, int32_t max_pages, int32_t page_size) {
  if (B < 0 || max_pages < 1 || page_size < 1) return 0;
  return dsa::indexer_paged_ws(B, max_pages, page_size);
}

dsa_status dsa_indexer_topk_paged(const uint8_t* q_idx, const float* w, const uint8_t* k_cache,
                                  const int32_t* page_table, const int32_t* ctx_lens, int32_t B,
                                  int32_t max_pages, int32_t n_pages, int32_t page_size,
                                  int32_t H_I, int32_t d_I, int32_t top_k, int32_t* out_idx,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (B < 0 || !paging_ok(max_pages, n_pages, page_size)) return DSA_ERR_INVALID_ARG;
  if (!indexer_shape_ok(H_I, d_I, top_k)) return DSA_ERR_UNSUPPORTED_SHAPE;
  if (B == 0) return DSA_OK;
  if (B > 65535) return DSA_ERR_UNSUPPORTED_SHAPE;
  if (!q_idx || !w || !k_cache || !page_table || !ctx_lens || !out_idx || !workspace)
    return DSA_ERR_INVALID_ARG;
  if (workspace_bytes < dsa::indexer_paged_ws(B, max_pages, page_size))
    return DSA_ERR_WORKSPACE_TOO_SMALL;
  return from_hip(dsa::launch_indexer_topk_paged(q_idx, w, k_cache, page_table, ctx_lens, B,
                                                 max_pages, n_pages, page_size, H_I, d_I, top_k,
                                                 out_idx, workspace, stream));
}

dsa_status dsa_sparse_mqa_prefill(const uint16_t* q, const uint16_t* kv, int32_t n_kv,
                                  const int32_t* idx, const int32_t* q_pos, int32_t n_q,
                                  int32_t H, int32_t D_k, int32_t D_v, int32_t top_k,
                                  float scale, uint16_t* out, float* lse, hipStream_t stream) {
  if (n_q < 0 || n_kv < 1 || !isfinite(scale)) return DSA_ERR_INVALID_ARG;
  if (H < 1 || H > kMaxH || !dsa::mqa_shape_supported(D_k, D_v) || top_k < 1 ||
      top_k > kMaxTopK)
    return DSA_ERR_UNSUPPORTED_SHAPE;
  if (n_q == 0) return DSA_OK;
  if (!q || !kv || !idx || !q_pos || !out) return DSA_ERR_INVALID_ARG;
  dsa::MqaArgs a{};
  a.q = q; a.kv = kv; a.idx = idx; a.qpos_or_ctx = q_pos; a.page_table = nullptr;
  a.n_kv = n_kv; a.n_q = n_q; a.H = H; a.D_k = D_k; a.D_v = D_v; a.top_k = top_k;
  a.scale = scale; a.n_split = 1; a.rows_per_split = top_k; a.out = out; a.lse = lse;
  return from_hip(dsa::launch_sparse_mqa(a, stream));
}

dsa_status dsa_indexer_topk_batched(const uint8_t* q_idx, const float* w,
                                    const uint8_t* k_cache, const int32_t* page_table,
                                    int32_t n_seq, int32_t max_pages, int32_t n_pages,
                                    int32_t page_size, const int32_t* q_seq,
                                    const int32_t* q_pos, int32_t n_q, int32_t H_I, int32_t d_I,
                                    int32_t top_k, int32_t* out_idx, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream) {
  if (n_q < 0 || n_seq < 1 || !paging_ok(max_pages, n_pages, page_size))
    return DSA_ERR_INVALID_ARG;
  if (!indexer_shape_ok(H_I, d_I, top_k) || page_size < 8 || (page_size & (page_size - 1)) != 0)
    return DSA_ERR_UNSUPPORTED_SHAPE;
  if (n_q == 0) return DSA_OK;
  if (!q_idx || !w || !k_cache || !page_table || !q_pos || !out_idx || !workspace)
    return DSA_ERR_INVALID_ARG;
  if (workspace_bytes < dsa::indexer_prefill_ws(n_q, top_k)) return DSA_ERR_WORKSPACE_TOO_SMALL;
  return from_hip(dsa::launch_indexer_topk_batched(q_idx, w, k_cache, page_table, n_seq,
                                                   max_pages, n_pages, page_size, q_seq, q_pos,
                                                   n_q, H_I, d_I, top_k, out_idx, workspace,
                                                   stream));
}

dsa_status dsa_sparse_mqa_batched(const uint16_t* q, const uint16_t* kv_cache,
                                  const int32_t* page_table, int32_t n_seq, int32_t max_pages,
                                  int32_t n_pages, int32_t page_size, const int32_t* q_seq,
                                  const int32_t* q_pos, const int32_t* idx, int32_t n_q,
                                  int32_t H, int32_t D_k, int32_t D_v, int32_t top_k,
                                  float scale, uint16_t* out, float* lse, hipStream_t stream) {
  if (n_q < 0 || n_seq < 1 || !paging_ok(max_pages, n_pages, page_size) || !isfinite(scale))
    return DSA_ERR_INVALID_ARG;
  if (H < 1 || H > kMaxH || !dsa::mqa_shape_supported(D_k, D_v) || top_k < 1 ||
      top_k > kMaxTopK)
    return DSA_ERR_UNSUPPORTED_SHAPE;
  if (n_q == 0) return DSA_OK;
  if (n_q > 0x7fffffff / 2 || !q || !kv_cache || !page_table || !q_pos || !idx || !out)
    return DSA_ERR_INVALID_ARG;
  dsa::MqaArgs a{};
  a.q = q; a.kv = kv_cache; a.idx = idx; a.qpos_or_ctx = q_pos; a.page_table = page_table;
  a.q_seq = q_seq; a.n_seq = n_seq; a.max_pages = max_pages; a.n_pages = n_pages;
  a.page_size = page_size; a.n_kv = 0; a.n_q = n_q; a.H = H; a.D_k = D_k; a.D_v = D_v;
  a.top_k = top_k; a.scale = scale; a.n_split = 1; a.rows_per_split = top_k; a.out = out;
  a.lse = lse;
  return from_hip(dsa::launch_sparse_mqa(a, stream));
}

size_t dsa_dense_mqa_workspace_size(int32_t n_q, int32_t H, int32_t D_v, int32_t max_len) {
  if (n_q < 0 || H < 1 || D_v < 1 || max_len < 0) return 0;
  const int rps = dsa::dense_rows_per_split();
  const long long ns = ((long long)max_len + rps - 1) / rps;
  if (ns <= 1) return 0;
  return (size_t)n_q * (size_t)ns * H * ((size_t)D_v * sizeof(uint16_t) + 2 * sizeof(float));
}

namespace {

// Shared by the two dense entry points: split count, checks and launch.
dsa_status dense_launch(dsa::MqaArgs& a, int32_t max_len, void* workspace,
                        size_t workspace_bytes, hipStream_t stream) {
  const int rps = dsa::dense_rows_per_split();
  const long long ns = ((long long)max_len + rps - 1) / rps;
  if (ns > 65535) return DSA_ERR_UNSUPPORTED_SHAPE;
  a.n_split = ns < 1 ? 1 : (int)ns;
  a.rows_per_split = rps;
  const size_t need = dsa_dense_mqa_workspace_size(a.n_q, a.H, a.D_v, max_len);
  if (need > 0 && (!workspace || workspace_bytes < need)) return DSA_ERR_WORKSPACE_TOO_SMALL;
  if (a.n_split > 1) {
    a.part_o = reinterpret_cast<uint16_t*>(workspace);
    a.part_ml = reinterpret_cast<float*>(a.part_o + (size_t)a.n_q * a.n_split * a.H * a.D_v);
  }
  return from_hip(dsa::launch_dense_mqa(a, stream));
}

}  // namespace

dsa_status dsa_dense_mqa_prefill(const uint16_t* q, const uint16_t* kv, int32_t n_kv,
                                 const int32_t* q_pos, int32_t n_q, int32_t H, int32_t D_k,
                                 int32_t D_v, float scale, uint16_t* out, float* lse,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (n_q < 0 || n_kv < 1 || !isfinite(scale)) return DSA_ERR_INVALID_ARG;
  if (H < 1 || H > kMaxH || !dsa::mqa_shape_supported(D_k, D_v)) return DSA_ERR_UNSUPPORTED_SHAPE;
  if (n_q == 0) return DSA_OK;
  if (n_q > 0x7fffffff / 2 || !q || !kv || !q_pos || !out) return DSA_ERR_INVALID_ARG;
  dsa::MqaArgs a{};
  a.q = q; a.kv = kv; a.qpos_or_ctx = q_pos; a.n_kv = n_kv; a.n_q = n_q; a.H = H;
  a.D_k = D_k; a.D_v = D_v; a.scale = scale; a.out = out; a.lse = lse;
  return dense_launch(a, n_kv, workspace, workspace_bytes, stream);
}

dsa_status dsa_dense_mqa_decode(const uint16_t* q, const uint16_t* kv_cache,
                                const int32_t* page_table, const int32_t* ctx_lens, int32_t B,
                                int32_t max_pages, int32_t n_pages, int32_t page_size, int32_t H,
                                int32_t D_k, int32_t D_v, float scale, uint16_t* out,
                                float* lse, void* workspace, size_t workspace_bytes,
                                hipStream_t stream) {
  if (B < 0 || !paging_ok(max_pages, n_pages, page_size) || !isfinite(scale))
    return DSA_ERR_INVALID_ARG;
  if (H < 1 || H > kMaxH || !dsa::mqa_shape_supported(D_k, D_v)) return DSA_ERR_UNSUPPORTED_SHAPE;
  if (B == 0) return DSA_OK;
  if (B > 0x7fffffff / 2 || !q || !kv_cache || !page_table || !ctx_lens || !out)
    return DSA_ERR_INVALID_ARG;
  dsa::MqaArgs a{};
  a.q = q; a.kv = kv_cache; a.qpos_or_ctx = ctx_lens; a.page_table = page_table;
  a.max_pages = max_pages; a.n_pages = n_pages; a.page_size = page_size; a.n_q = B; a.H = H;
  a.D_k = D_k; a.D_v = D_v; a.scale = scale; a.out = out; a.lse = lse;
  return dense_launch(a, max_pages * page_size, workspace, workspace_bytes, stream);
}

dsa_status dsa_indexer_kl(const uint16_t* q, const uint16_t* kv, int32_t n_kv,
                          const int32_t* idx, const int32_t* q_pos, const float* lse,
                          int32_t n_q, int32_t H, int32_t D_k, int32_t top_k, float scale,
                          const uint8_t* q_idx, const float* w, const uint8_t* k_idx,
                          int32_t H_I, int32_t d_I, float* target, float* loss, float* grad,
                          hipStream_t stream) {
  if (n_q < 0 || n_kv < 1 || !isfinite(scale)) return DSA_ERR_INVALID_ARG;
  if (H < 1 || H > kMaxH || !(D_k == 576 || D_k == 64 || D_k == 96) ||
      !indexer_shape_ok(H_I, d_I, top_k))
    return DSA_ERR_UNSUPPORTED_SHAPE;
  if (n_q == 0) return DSA_OK;
  if (n_q > 0x7fffffff / 2 || !q || !kv || !idx || !q_pos || !lse || !q_idx || !w || !k_idx ||
      !target || !loss)
    return DSA_ERR_INVALID_ARG;
  dsa::MqaArgs a{};
  a.q = q; a.kv = kv; a.idx = idx; a.qpos_or_ctx = q_pos; a.n_kv = n_kv; a.n_q = n_q; a.H = H;
  a.D_k = D_k; a.D_v = D_k == 576 ? 512 : 64; a.top_k = top_k; a.scale = scale;
  a.n_split = 1; a.rows_per_split = top_k;
  hipError_t e = dsa::launch_mqa_probs(a, lse, target, stream);
  if (e != hipSuccess) return DSA_ERR_HIP;
  return from_hip(dsa::launch_indexer_kl(q_idx, w, k_idx, n_kv, q_pos, idx, n_q, top_k, H_I, d_I,
                                         target, loss, grad, stream));
}

size_t dsa_sparse_mqa_backward_workspace_size(int32_t n_q, int32_t H, int32_t top_k) {
  if (n_q < 0 || H < 1 || top_k < 1) return 0;
  return 2 * (size_t)n_q * H * top_k * sizeof(uint16_t);
}

dsa_status dsa_sparse_mqa_backward(const uint16_t* q, const uint16_t* kv, int32_t n_kv,
                                   const int32_t* idx, const int32_t* q_pos, const uint16_t* out,
                                   const float* lse, const uint16_t* d_out, int32_t n_q,
                                   int32_t H, int32_t D_k, int32_t D_v, int32_t top_k,
                                   float scale, float* d_q, float* d_kv, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream) {
  if (n_q < 0 || n_kv < 1 || !isfinite(scale)) return DSA_ERR_INVALID_ARG;
  if (H < 1 || H > kMaxH || !dsa::mqa_shape_supported(D_k, D_v) || top_k < 1 ||
      top_k > kMaxTopK)
    return DSA_ERR_UNSUPPORTED_SHAPE;
  if (n_q == 0) return DSA_OK;
  if (n_q > 0x7fffffff / 2 || !q || !kv || !idx || !q_pos || !out || !lse || !d_out || !d_q ||
      !d_kv)
    return DSA_ERR_INVALID_ARG;
  const size_t half = (size_t)n_q * H * top_k;
  if (!workspace || workspace_bytes < dsa_sparse_mqa_backward_workspace_size(n_q, H, top_k))
    return DSA_ERR_WORKSPACE_TOO_SMALL;
  dsa::MqaArgs a{};
  a.q = q; a.kv = kv; a.idx = idx; a.qpos_or_ctx = q_pos; a.n_kv = n_kv; a.n_q = n_q; a.H = H;
  a.D_k = D_k; a.D_v = D_v; a.top_k = top_k; a.scale = scale; a.n_split = 1;
  a.rows_per_split = top_k;
  uint16_t* p_ws = reinterpret_cast<uint16_t*>(workspace);
  return from_hip(dsa::launch_mqa_backward(a, lse, out, d_out, p_ws, p_ws + half, d_q, d_kv,
                                           stream));
}

dsa_status dsa_cache_append(const uint16_t* k_new, const uint16_t* kv_new, const int32_t* seq,
                            const int32_t* pos, const int32_t* page_table, int32_t T,
                            int32_t max_pages, int32_t n_pages, int32_t page_size, int32_t d_I,
                            int32_t D_k, uint8_t* k_cache, uint16_t* kv_cache,
                            hipStream_t stream) {
  if (T < 0 || !paging_ok(max_pages, n_pages, page_size)) return DSA_ERR_INVALID_ARG;
  if (k_new != nullptr && (d_I < 16 || d_I > kMaxDI || d_I % 16 != 0))
    return DSA_ERR_UNSUPPORTED_SHAPE;
  if (kv_new != nullptr && (D_k < 8 || D_k > 1024 || D_k % 8 != 0))
    return DSA_ERR_UNSUPPORTED_SHAPE;
  if (T == 0) return DSA_OK;
  if (T > 0x7fffffff / 2 || (!k_new && !kv_new) || !pos || !page_table ||
      (k_new && !k_cache) || (kv_new && !kv_cache))
    return DSA_ERR_INVALID_ARG;
  return from_hip(dsa::launch_cache_append(k_new, kv_new, seq, pos, page_table, T, max_pages,
                                           n_pages, page_size, d_I, D_k, k_cache, kv_cache,
                                           stream));
}

size_t dsa_sparse_mqa_decode_workspace_size(int32_t B, int32_t H, int32_t D_v, int32_t top_k,
                                            int32_t n_split) {
  if (B < 0 || H < 1 || D_v < 1 || top_k < 1 || top_k > kMaxTopK || n_split < 0) return 0;
  int ns, rps;
  decode_split(B, top_k, n_split, &ns, &rps);
  if (ns == 1) return 0;
  // bf16 normalised partial outputs, then (max, sum) pairs in fp32
  return (size_t)B * ns * H * ((size_t)D_v * sizeof(uint16_t) + 2 * sizeof(float));
}

}  // extern "C"

namespace {

// Checks shared by the two decode-attention entry points; fills the launch arguments except
// the partials.  *done is set when there is nothing to launch (B == 0).
dsa_status decode_args(const uint16_t* q, const uint16_t* kv_cache, const int32_t* page_table,
                       const int32_t* ctx_lens, const int32_t* idx, int32_t B,
                       int32_t max_pages, int32_t n_pages, int32_t page_size, int32_t H,
                       int32_t D_k, int32_t D_v, int32_t top_k, float scale, int32_t n_split,
                       uint16_t* out, float* lse, dsa::MqaArgs* a, bool* done) {
  *done = false;
  if (B < 0 || !paging_ok(max_pages, n_pages, page_size) || !isfinite(scale) || n_split < 0 ||
      n_split > kMaxSplit)
    return DSA_ERR_INVALID_ARG;
  if (H < 1 || H > kMaxH || !dsa::mqa_shape_supported(D_k, D_v) || top_k < 1 ||
      top_k > kMaxTopK)
    return DSA_ERR_UNSUPPORTED_SHAPE;
  if (B == 0) {
    *done = true;
    return DSA_OK;
  }
  if (B > 65535 * 16) return DSA_ERR_UNSUPPORTED_SHAPE;
  if (!q || !kv_cache || !page_table || !ctx_lens || !idx || !out) return DSA_ERR_INVALID_ARG;
  int ns, rps;
  decode_split(B, top_k, n_split, &ns, &rps);
  *a = dsa::MqaArgs{};
  a->q = q; a->kv = kv_cache; a->idx = idx; a->qpos_or_ctx = ctx_lens;
  a->page_table = page_table; a->max_pages = max_pages; a->n_pages = n_pages;
  a->page_size = page_size; a->n_kv = 0; a->n_q = B; a->H = H; a->D_k = D_k; a->D_v = D_v;
  a->top_k = top_k; a->scale = scale; a->n_split = ns; a->rows_per_split = rps; a->out = out;
  a->lse = lse;
  return DSA_OK;
}

void set_partials(dsa::MqaArgs* a, void* base) {
  if (a->n_split > 1) {
    a->part_o = reinterpret_cast<uint16_t*>(base);
    a->part_ml = reinterpret_cast<float*>(a->part_o + (size_t)a->n_q * a->n_split * a->H * a->D_v);
  }
}

}  // namespace

extern "C" {

dsa_status dsa_sparse_mqa_decode(const uint16_t* q, const uint16_t* kv_cache,
                                 const int32_t* page_table, const int32_t* ctx_lens,
                                 const int32_t* idx, int32_t B, int32_t max_pages,
                                 int32_t n_pages, int32_t page_size, int32_t H, int32_t D_k,
                                 int32_t D_v, int32_t top_k, float scale, int32_t n_split,
                                 uint16_t* out, float* lse, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
  dsa::MqaArgs a;
  bool done;
  dsa_status st = decode_args(q, kv_cache, page_table, ctx_lens, idx, B, max_pages, n_pages,
                              page_size, H, D_k, D_v, top_k, scale, n_split, out, lse, &a, &done);
  if (st != DSA_OK || done) return st;
  const size_t need = dsa_sparse_mqa_decode_workspace_size(B, H, D_v, top_k, n_split);
  if (need > 0 && (!workspace || workspace_bytes < need)) return DSA_ERR_WORKSPACE_TOO_SMALL;
  set_partials(&a, workspace);
  return from_hip(dsa::launch_sparse_mqa(a, stream));
}

dsa_status dsa_sparse_mqa_decode_noalloc(const uint16_t* q, const uint16_t* kv_cache,
                                         const int32_t* page_table, const int32_t* ctx_lens,
                                         const int32_t* idx, int32_t B, int32_t max_pages,
                                         int32_t n_pages, int32_t page_size, int32_t H,
                                         int32_t D_k, int32_t D_v, int32_t top_k, float scale,
                                         int32_t n_split, uint16_t* out, float* lse,
                                         hipStream_t stream) {
  static_assert(DSA_NOALLOC_SCRATCH_BYTES == dsa::kNoAllocScratchBytes, "scratch size");
  dsa::MqaArgs a;
  bool done;
  dsa_status st = decode_args(q, kv_cache, page_table, ctx_lens, idx, B, max_pages, n_pages,
                              page_size, H, D_k, D_v, top_k, scale, n_split, out, lse, &a, &done);
  if (st != DSA_OK || done) return st;
  const size_t need = dsa_sparse_mqa_decode_workspace_size(B, H, D_v, top_k, n_split);
  if (need > dsa::kNoAllocScratchBytes) return DSA_ERR_SCRATCH_LIMIT;
  if (need > 0) {
    void* base = nullptr;
    if (dsa::noalloc_scratch(&base) != hipSuccess) return DSA_ERR_HIP;
    set_partials(&a, base);
  }
  return from_hip(dsa::launch_sparse_mqa(a, stream));
}

}  // extern "C"
