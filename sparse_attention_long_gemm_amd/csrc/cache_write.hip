// Cache write: the step that feeds the paged decode path.  Each new token's indexer key k_I
// (bf16 from its projection) is quantised to FP8 e4m3fn and written with the token's latent KV
// row (bf16, copied as is) into the paged caches at its logical position, through the same page
// table the decode kernels read (page size 64 in the serving recipe of the mundobytes.com
// DeepSeek-V3.2-Exp page, section "Quick guide to running locally"; the indexer keeps its keys
// in FP8 per the jdon.com "DeepSeek-V3.2-Exp" article, paragraph on the lightning indexer).
//
// Quantisation: round to nearest, ties to the even code, saturating: a finite value at or past
// the largest e4m3fn magnitude (448) becomes +-448, infinities too; NaN stays NaN (0x7f with the
// sign).  The sign of zero is kept.
//
// One workgroup of 128 threads per row: thread i < D_k / 8 moves 16 bytes of the KV row, thread
// i < d_I / 8 converts 8 key values into 8 bytes.  Rows whose slot is invalid (negative
// position, page index past max_pages, page-table entry outside [0, n_pages)) write nothing.
#include "dsa_common.hpp"
#include "dsa_kernels.hpp"

namespace dsa {

namespace {

constexpr int CW_NT = 128;

// bf16 bit pattern -> e4m3fn code (see above).
__device__ __forceinline__ u32 bf16_to_e4m3fn(uint16_t b) {
  const u32 bits = (u32)b << 16;
  const u32 sign = (bits >> 24) & 0x80u;
  const u32 mag = bits & 0x7fffffffu;
  if (mag > 0x7f800000u) return sign | 0x7fu;             // NaN
  const float a = __uint_as_float(mag);
  if (a >= 448.0f) return sign | 0x7eu;                   // saturate (also +-inf)
  if (a < 0.015625f) {                                    // below 2^-6: subnormal step 2^-9
    const float m = __builtin_rintf(a * 512.0f);           // exact scaling, ties to even
    return sign | (u32)m;                                  // m == 8 is the code of 2^-6
  }
  // normal: keep 3 mantissa bits, round the other 20 to nearest even
  u32 r = mag + 0x7ffffu + ((mag >> 20) & 1u);
  r &= ~0xfffffu;
  const int e = (int)(r >> 23) - 127;                     // -6 .. 8
  u32 code = ((u32)(e + 7) << 3) | ((r >> 20) & 7u);
  if (code > 0x7eu) code = 0x7eu;                         // rounded up past 448
  return sign | code;
}

__global__ __launch_bounds__(CW_NT) void cache_append_kernel(
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ kv_new,
    const int32_t* __restrict__ seq, const int32_t* __restrict__ pos,
    const int32_t* __restrict__ page_table, int max_pages, int n_pages, int page_size, int d_I,
    int D_k, uint8_t* __restrict__ k_cache, uint16_t* __restrict__ kv_cache) {
  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  const int b = seq != nullptr ? seq[r] : r;
  const int p = pos[r];
  if (b < 0 || p < 0) return;
  const int pi = p / page_size;
  if (pi >= max_pages) return;
  const int page = page_table[(size_t)b * max_pages + pi];
  if (page < 0 || page >= n_pages) return;
  const size_t slot = (size_t)page * page_size + (p - pi * page_size);
  if (kv_new != nullptr && tid < D_k / 8) {
    const v4i v = *reinterpret_cast<const v4i*>(kv_new + (size_t)r * D_k + 8 * tid);
    *reinterpret_cast<v4i*>(kv_cache + slot * D_k + 8 * tid) = v;
  }
  if (k_new != nullptr && tid < d_I / 8) {
    const v4i v = *reinterpret_cast<const v4i*>(k_new + (size_t)r * d_I + 8 * tid);
    u32 lo = 0u, hi = 0u;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const u32 w = (u32)v[e];
      const u32 c0 = bf16_to_e4m3fn((uint16_t)(w & 0xffffu));
      const u32 c1 = bf16_to_e4m3fn((uint16_t)(w >> 16));
      const u32 pair = c0 | (c1 << 8);
      if (e < 2) lo |= pair << (16 * e);
      else hi |= pair << (16 * (e - 2));
    }
    *reinterpret_cast<uint2*>(k_cache + slot * d_I + 8 * tid) = uint2{lo, hi};
  }
}

}  // namespace

hipError_t launch_cache_append(const uint16_t* k_new, const uint16_t* kv_new, const int32_t* seq,
                               const int32_t* pos, const int32_t* page_table, int T,
                               int max_pages, int n_pages, int page_size, int d_I, int D_k,
                               uint8_t* k_cache, uint16_t* kv_cache, hipStream_t stream) {
  hipLaunchKernelGGL(cache_append_kernel, dim3(T), dim3(CW_NT), 0, stream, k_new, kv_new, seq,
                     pos, page_table, max_pages, n_pages, page_size, d_I, D_k, k_cache,
                     kv_cache);
  return hipGetLastError();
}

}  // namespace dsa
