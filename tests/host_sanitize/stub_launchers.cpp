// Host stand-ins for the kernel launchers, so that the C-ABI layer (dsa_api.cpp) can be built
// with g++ under AddressSanitizer / UndefinedBehaviorSanitizer and exercised without a GPU.
// Each launcher records what it was asked to launch; nothing touches device memory.
#include "stub_launchers.hpp"

namespace stub {
Launch last;
int launches = 0;
unsigned char scratch_stand_in[64];
}  // namespace stub

namespace dsa {

static hipError_t record(const char* what, const MqaArgs* a = nullptr) {
  stub::last = stub::Launch{};
  stub::last.what = what;
  if (a != nullptr) stub::last.mqa = *a;
  ++stub::launches;
  return hipSuccess;
}

int indexer_cap(int top_k) { return 2 * top_k + 128; }
size_t indexer_prefill_ws(int n_q, int top_k) { return (size_t)n_q * indexer_cap(top_k) * 8; }
size_t indexer_paged_ws(int B, int max_pages, int page_size) {
  return (size_t)B * max_pages * page_size * 12 + (size_t)B * 4096 * 4;
}
hipError_t launch_indexer_topk_prefill(const uint8_t*, const float*, const uint8_t*, int, const int32_t*,
                                       int n_q, int, int, int, int32_t*, void*, hipStream_t) {
  hipError_t e = record("indexer_topk_prefill");
  stub::last.n = n_q;
  return e;
}
hipError_t launch_indexer_topk_batched(const uint8_t*, const float*, const uint8_t*, const int32_t*, int n_seq,
                                       int, int, int page_size, const int32_t*, const int32_t*, int n_q, int,
                                       int, int, int32_t*, void*, hipStream_t) {
  hipError_t e = record("indexer_topk_batched");
  stub::last.n = n_q;
  stub::last.n_seq = n_seq;
  stub::last.page_size = page_size;
  return e;
}
hipError_t launch_indexer_kl(const uint8_t*, const float*, const uint8_t*, int, const int32_t*, const int32_t*,
                             int n_q, int, int, int, const float*, float*, float*, hipStream_t) {
  hipError_t e = record("indexer_kl");
  stub::last.n = n_q;
  return e;
}
hipError_t launch_indexer_topk_paged(const uint8_t*, const float*, const uint8_t*, const int32_t*, const int32_t*,
                                     int B, int, int, int, int, int, int, int32_t*, void*, hipStream_t) {
  hipError_t e = record("indexer_topk_paged");
  stub::last.n = B;
  return e;
}
hipError_t launch_cache_append(const uint16_t*, const uint16_t*, const int32_t*, const int32_t*, const int32_t*,
                               int T, int, int, int, int, int, uint8_t*, uint16_t*, hipStream_t) {
  hipError_t e = record("cache_append");
  stub::last.n = T;
  return e;
}
bool mqa_shape_supported(int D_k, int D_v) {
  return (D_k == 576 && D_v == 512) || (D_k == 64 && D_v == 64) || (D_k == 96 && D_v == 64);
}
hipError_t launch_sparse_mqa(const MqaArgs& a, hipStream_t) { return record("sparse_mqa", &a); }
hipError_t launch_dense_mqa(const MqaArgs& a, hipStream_t) { return record("dense_mqa", &a); }
int dense_rows_per_split() { return 2048; }
hipError_t launch_mqa_probs(const MqaArgs& a, const float*, float*, hipStream_t) {
  return record("mqa_probs", &a);
}
hipError_t launch_mqa_backward(const MqaArgs& a, const float*, const uint16_t*, const uint16_t*, uint16_t* p_ws,
                               uint16_t* ds_ws, float*, float*, hipStream_t) {
  hipError_t e = record("mqa_backward", &a);
  stub::last.p_ws = p_ws;
  stub::last.ds_ws = ds_ws;
  return e;
}
hipError_t noalloc_scratch(void** ptr) {
  *ptr = stub::scratch_stand_in;
  return hipSuccess;
}

}  // namespace dsa
