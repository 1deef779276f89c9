// Exercises every entry point of the C ABI on the host (argument checks, size arithmetic,
// workspace carving, split choice) with the launchers stubbed out; built with AddressSanitizer
// and UndefinedBehaviorSanitizer by tests/test_host_sanitizers.py.  Prints "ok" and returns 0
// when every expectation holds; any sanitizer report aborts the run.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "dsa.h"
#include "stub_launchers.hpp"

static int failures = 0;
#define EXPECT(cond)                                                      \
  do {                                                                    \
    if (!(cond)) {                                                        \
      fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                         \
    }                                                                     \
  } while (0)

// Distinct, never dereferenced addresses standing for device buffers.
static unsigned char arena[1 << 12];
#define P(i) ((void*)(arena + 16 * (i)))

static int launched_since(int before) { return stub::launches - before; }

static void status_strings() {
  const int codes[] = {DSA_OK, DSA_ERR_INVALID_ARG, DSA_ERR_UNSUPPORTED_SHAPE,
                       DSA_ERR_WORKSPACE_TOO_SMALL, DSA_ERR_HIP, DSA_ERR_SCRATCH_LIMIT, 7, -99};
  for (int c : codes) EXPECT(dsa_status_string(c) != nullptr && strlen(dsa_status_string(c)) > 0);
  EXPECT(dsa_abi_version() == DSA_ABI_VERSION);
}

static void indexer() {
  const size_t ws = dsa_indexer_topk_workspace_size(4096, 2048);
  EXPECT(ws > 0);
  EXPECT(dsa_indexer_topk_workspace_size(-1, 2048) == 0);
  EXPECT(dsa_indexer_topk_workspace_size(10, 0) == 0);
  int b = stub::launches;
  EXPECT(dsa_indexer_topk((uint8_t*)P(1), (float*)P(2), (uint8_t*)P(3), 131072, (int32_t*)P(4),
                          4096, 64, 128, 2048, (int32_t*)P(5), P(6), ws, nullptr) == DSA_OK);
  EXPECT(launched_since(b) == 1 && stub::last.n == 4096);
  b = stub::launches;
  EXPECT(dsa_indexer_topk((uint8_t*)P(1), (float*)P(2), (uint8_t*)P(3), 131072, (int32_t*)P(4),
                          4096, 64, 128, 2048, (int32_t*)P(5), P(6), ws - 1, nullptr) ==
         DSA_ERR_WORKSPACE_TOO_SMALL);
  EXPECT(dsa_indexer_topk(nullptr, (float*)P(2), (uint8_t*)P(3), 10, (int32_t*)P(4), 4, 64, 128,
                          32, (int32_t*)P(5), P(6), 1 << 20, nullptr) == DSA_ERR_INVALID_ARG);
  EXPECT(dsa_indexer_topk((uint8_t*)P(1), (float*)P(2), (uint8_t*)P(3), 10, (int32_t*)P(4), 4, 65,
                          128, 32, (int32_t*)P(5), P(6), 1 << 20, nullptr) == DSA_ERR_UNSUPPORTED_SHAPE);
  EXPECT(dsa_indexer_topk((uint8_t*)P(1), (float*)P(2), (uint8_t*)P(3), 10, (int32_t*)P(4),
                          INT32_MAX, 64, 128, 2048, (int32_t*)P(5), P(6), 16, nullptr) ==
         DSA_ERR_WORKSPACE_TOO_SMALL);
  EXPECT(dsa_indexer_topk(nullptr, nullptr, nullptr, 0, nullptr, 0, 64, 128, 32, nullptr, nullptr,
                          0, nullptr) == DSA_OK);
  EXPECT(launched_since(b) == 0);

  // paged decode indexer
  const size_t wp = dsa_indexer_topk_paged_workspace_size(64, 2048, 64);
  EXPECT(wp > 0 && dsa_indexer_topk_paged_workspace_size(64, 0, 64) == 0);
  b = stub::launches;
  EXPECT(dsa_indexer_topk_paged((uint8_t*)P(1), (float*)P(2), (uint8_t*)P(3), (int32_t*)P(4),
                                (int32_t*)P(5), 64, 2048, 70000, 64, 64, 128, 2048,
                                (int32_t*)P(6), P(7), wp, nullptr) == DSA_OK);
  EXPECT(launched_since(b) == 1 && stub::last.n == 64);
  EXPECT(dsa_indexer_topk_paged((uint8_t*)P(1), (float*)P(2), (uint8_t*)P(3), (int32_t*)P(4),
                                (int32_t*)P(5), 64, INT32_MAX, 70000, 64, 64, 128, 2048,
                                (int32_t*)P(6), P(7), wp, nullptr) == DSA_ERR_INVALID_ARG);
  EXPECT(dsa_indexer_topk_paged((uint8_t*)P(1), (float*)P(2), (uint8_t*)P(3), (int32_t*)P(4),
                                (int32_t*)P(5), 70000, 16, 70000, 64, 64, 128, 2048,
                                (int32_t*)P(6), P(7), (size_t)-1, nullptr) ==
         DSA_ERR_UNSUPPORTED_SHAPE);

  // batched prefill indexer: power-of-two page size >= 8, at least one sequence
  b = stub::launches;
  EXPECT(dsa_indexer_topk_batched((uint8_t*)P(1), (float*)P(2), (uint8_t*)P(3), (int32_t*)P(4), 3,
                                  100, 300, 64, nullptr, (int32_t*)P(5), 1000, 64, 128, 512,
                                  (int32_t*)P(6), P(7), dsa_indexer_topk_workspace_size(1000, 512),
                                  nullptr) == DSA_OK);
  EXPECT(launched_since(b) == 1 && stub::last.n_seq == 3 && stub::last.page_size == 64);
  EXPECT(dsa_indexer_topk_batched((uint8_t*)P(1), (float*)P(2), (uint8_t*)P(3), (int32_t*)P(4), 3,
                                  100, 300, 48, nullptr, (int32_t*)P(5), 1000, 64, 128, 512,
                                  (int32_t*)P(6), P(7), 1 << 30, nullptr) == DSA_ERR_UNSUPPORTED_SHAPE);
  EXPECT(dsa_indexer_topk_batched((uint8_t*)P(1), (float*)P(2), (uint8_t*)P(3), (int32_t*)P(4), 0,
                                  100, 300, 64, nullptr, (int32_t*)P(5), 1000, 64, 128, 512,
                                  (int32_t*)P(6), P(7), 1 << 30, nullptr) == DSA_ERR_INVALID_ARG);
}

static void attention() {
  int b = stub::launches;
  EXPECT(dsa_sparse_mqa_prefill((uint16_t*)P(1), (uint16_t*)P(2), 131072, (int32_t*)P(3),
                                (int32_t*)P(4), 4096, 128, 576, 512, 2048, 0.0416f,
                                (uint16_t*)P(5), nullptr, nullptr) == DSA_OK);
  EXPECT(launched_since(b) == 1 && stub::last.mqa.n_split == 1 && stub::last.mqa.page_table == nullptr);
  EXPECT(dsa_sparse_mqa_prefill((uint16_t*)P(1), (uint16_t*)P(2), 131072, (int32_t*)P(3),
                                (int32_t*)P(4), 4096, 128, 576, 256, 2048, 0.0416f,
                                (uint16_t*)P(5), nullptr, nullptr) == DSA_ERR_UNSUPPORTED_SHAPE);

  // decode: the library's split choice and the carving of the workspace
  const size_t wd = dsa_sparse_mqa_decode_workspace_size(64, 128, 512, 2048, 0);
  EXPECT(wd == (size_t)64 * 4 * 128 * (512 * 2 + 8));
  unsigned char* ws = (unsigned char*)P(40);
  b = stub::launches;
  EXPECT(dsa_sparse_mqa_decode((uint16_t*)P(1), (uint16_t*)P(2), (int32_t*)P(3), (int32_t*)P(4),
                               (int32_t*)P(5), 64, 2048, 70000, 64, 128, 576, 512, 2048, 0.04f, 0,
                               (uint16_t*)P(6), nullptr, ws, wd, nullptr) == DSA_OK);
  EXPECT(launched_since(b) == 1);
  EXPECT(stub::last.mqa.n_split == 4 && stub::last.mqa.rows_per_split == 512);
  EXPECT((unsigned char*)stub::last.mqa.part_o == ws);
  EXPECT((unsigned char*)stub::last.mqa.part_ml == ws + (size_t)64 * 4 * 128 * 512 * 2);
  EXPECT(stub::last.mqa.n_seq == 0 && stub::last.mqa.q_seq == nullptr);
  EXPECT(dsa_sparse_mqa_decode((uint16_t*)P(1), (uint16_t*)P(2), (int32_t*)P(3), (int32_t*)P(4),
                               (int32_t*)P(5), 64, 2048, 70000, 64, 128, 576, 512, 2048, 0.04f, 0,
                               (uint16_t*)P(6), nullptr, ws, wd - 1, nullptr) ==
         DSA_ERR_WORKSPACE_TOO_SMALL);
  EXPECT(dsa_sparse_mqa_decode((uint16_t*)P(1), (uint16_t*)P(2), (int32_t*)P(3), (int32_t*)P(4),
                               (int32_t*)P(5), 64, 2048, 70000, 64, 128, 576, 512, 2048, 0.04f, 17,
                               (uint16_t*)P(6), nullptr, ws, wd, nullptr) == DSA_ERR_INVALID_ARG);

  // allocation-free decode: partials in the static array; too large a call refused unlaunched
  b = stub::launches;
  EXPECT(dsa_sparse_mqa_decode_noalloc((uint16_t*)P(1), (uint16_t*)P(2), (int32_t*)P(3),
                                       (int32_t*)P(4), (int32_t*)P(5), 64, 2048, 70000, 64, 128,
                                       576, 512, 2048, 0.04f, 0, (uint16_t*)P(6), nullptr,
                                       nullptr) == DSA_OK);
  EXPECT(launched_since(b) == 1 && (unsigned char*)stub::last.mqa.part_o == stub::scratch_stand_in);
  b = stub::launches;
  EXPECT(dsa_sparse_mqa_decode_noalloc((uint16_t*)P(1), (uint16_t*)P(2), (int32_t*)P(3),
                                       (int32_t*)P(4), (int32_t*)P(5), 600, 2048, 70000, 64, 128,
                                       576, 512, 2048, 0.04f, 4, (uint16_t*)P(6), nullptr,
                                       nullptr) == DSA_ERR_SCRATCH_LIMIT);
  EXPECT(launched_since(b) == 0);

  // batched attention: the row -> sequence map reaches the launch
  b = stub::launches;
  EXPECT(dsa_sparse_mqa_batched((uint16_t*)P(1), (uint16_t*)P(2), (int32_t*)P(3), 5, 100, 600, 64,
                                (int32_t*)P(4), (int32_t*)P(5), (int32_t*)P(6), 3000, 128, 576,
                                512, 2048, 0.04f, (uint16_t*)P(7), nullptr, nullptr) == DSA_OK);
  EXPECT(launched_since(b) == 1 && stub::last.mqa.n_seq == 5 &&
         stub::last.mqa.q_seq == (int32_t*)P(4) && stub::last.mqa.n_split == 1);

  // dense: split count from the KV length, refused past 65535 splits
  const size_t wn = dsa_dense_mqa_workspace_size(256, 128, 512, 131072);
  EXPECT(wn == (size_t)256 * 64 * 128 * (512 * 2 + 8));
  EXPECT(dsa_dense_mqa_workspace_size(256, 128, 512, 2048) == 0);
  b = stub::launches;
  EXPECT(dsa_dense_mqa_prefill((uint16_t*)P(1), (uint16_t*)P(2), 131072, (int32_t*)P(3), 256, 128,
                               576, 512, 0.04f, (uint16_t*)P(4), nullptr, P(5), wn, nullptr) ==
         DSA_OK);
  EXPECT(launched_since(b) == 1 && stub::last.mqa.n_split == 64 &&
         stub::last.mqa.rows_per_split == 2048);
  EXPECT(dsa_dense_mqa_decode((uint16_t*)P(1), (uint16_t*)P(2), (int32_t*)P(3), (int32_t*)P(4), 64,
                              33554432, 1 << 20, 64, 128, 576, 512, 0.04f, (uint16_t*)P(5),
                              nullptr, P(6), (size_t)-1, nullptr) == DSA_ERR_INVALID_ARG);
  EXPECT(dsa_dense_mqa_decode((uint16_t*)P(1), (uint16_t*)P(2), (int32_t*)P(3), (int32_t*)P(4), 64,
                              4194304, 1 << 20, 512, 128, 576, 512, 0.04f, (uint16_t*)P(5),
                              nullptr, P(6), (size_t)-1, nullptr) == DSA_ERR_INVALID_ARG);
}

static void next_rows() {
  int b = stub::launches;
  EXPECT(dsa_indexer_kl((uint16_t*)P(1), (uint16_t*)P(2), 131072, (int32_t*)P(3), (int32_t*)P(4),
                        (float*)P(5), 4096, 128, 576, 2048, 0.04f, (uint8_t*)P(6), (float*)P(7),
                        (uint8_t*)P(8), 64, 128, (float*)P(9), (float*)P(10), nullptr,
                        nullptr) == DSA_OK);
  // two launches: the main attention's probabilities, then the per-row KL
  EXPECT(launched_since(b) == 2 && stub::last.n == 4096);
  EXPECT(dsa_indexer_kl((uint16_t*)P(1), (uint16_t*)P(2), 131072, (int32_t*)P(3), (int32_t*)P(4),
                        nullptr, 4096, 128, 576, 2048, 0.04f, (uint8_t*)P(6), (float*)P(7),
                        (uint8_t*)P(8), 64, 128, (float*)P(9), (float*)P(10), nullptr,
                        nullptr) == DSA_ERR_INVALID_ARG);

  const size_t wb = dsa_sparse_mqa_backward_workspace_size(4096, 128, 2048);
  EXPECT(wb == (size_t)2 * 4096 * 128 * 2048 * 2);
  unsigned char* ws = (unsigned char*)P(60);
  b = stub::launches;
  EXPECT(dsa_sparse_mqa_backward((uint16_t*)P(1), (uint16_t*)P(2), 131072, (int32_t*)P(3),
                                 (int32_t*)P(4), (uint16_t*)P(5), (float*)P(6), (uint16_t*)P(7),
                                 4096, 128, 576, 512, 2048, 0.04f, (float*)P(8), (float*)P(9), ws,
                                 wb, nullptr) == DSA_OK);
  EXPECT(launched_since(b) == 1 && (unsigned char*)stub::last.p_ws == ws &&
         (unsigned char*)stub::last.ds_ws == ws + wb / 2);
  EXPECT(dsa_sparse_mqa_backward((uint16_t*)P(1), (uint16_t*)P(2), 131072, (int32_t*)P(3),
                                 (int32_t*)P(4), (uint16_t*)P(5), (float*)P(6), (uint16_t*)P(7),
                                 4096, 128, 576, 512, 2048, 0.04f, (float*)P(8), (float*)P(9), ws,
                                 wb - 1, nullptr) == DSA_ERR_WORKSPACE_TOO_SMALL);

  b = stub::launches;
  EXPECT(dsa_cache_append((uint16_t*)P(1), (uint16_t*)P(2), nullptr, (int32_t*)P(3),
                          (int32_t*)P(4), 64, 2048, 70000, 64, 128, 576, (uint8_t*)P(5),
                          (uint16_t*)P(6), nullptr) == DSA_OK);
  EXPECT(launched_since(b) == 1 && stub::last.n == 64);
  EXPECT(dsa_cache_append(nullptr, nullptr, nullptr, (int32_t*)P(3), (int32_t*)P(4), 64, 2048,
                          70000, 64, 128, 576, (uint8_t*)P(5), (uint16_t*)P(6), nullptr) ==
         DSA_ERR_INVALID_ARG);
  EXPECT(dsa_cache_append((uint16_t*)P(1), nullptr, nullptr, (int32_t*)P(3), (int32_t*)P(4), 64,
                          2048, 70000, 64, 100, 576, (uint8_t*)P(5), nullptr, nullptr) ==
         DSA_ERR_UNSUPPORTED_SHAPE);
}

int main() {
  status_strings();
  indexer();
  attention();
  next_rows();
  if (failures != 0) {
    fprintf(stderr, "%d expectation(s) failed\n", failures);
    return 1;
  }
  printf("ok\n");
  return 0;
}
