// Measurement helpers: what this GPU sustains on the instruction shapes and the memory stream
// the path uses, so that roofline fractions can be read against measured ceilings as well as
// the published peaks.  Not part of the path.
#include "dsa.h"
#include "dsa_common.hpp"

namespace dsa {
namespace {

constexpr int CEIL_NT = 512;    // 8 waves per workgroup
constexpr int READ_NT = 256;

// Independent MFMA chains on register operands (no memory traffic inside the loop).
template <int KIND>
__global__ __launch_bounds__(CEIL_NT) void ceiling_mfma_kernel(int iters, float* __restrict__ sink) {
  v8bf a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(threadIdx.x * 1e-3f + i);
    b[i] = (__bf16)(i * 0.5f);
  }
  v8i ai, bi;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    ai[i] = (int)threadIdx.x + i;
    bi[i] = i;
  }
  float r;
  if (KIND == 0) {
    v16f c0 = {}, c1 = {};
    for (int it = 0; it < iters; ++it) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    }
    r = c0[0] + c1[5];
  } else {
    v4f c0 = {0.f, 0.f, 0.f, 0.f}, c1 = c0, c2 = c0, c3 = c0;
    for (int it = 0; it < iters; ++it) {
      c0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ai, bi, c0, 0, 0, 0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ai, bi, c1, 0, 0, 0, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ai, bi, c2, 0, 0, 0, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ai, bi, c3, 0, 0, 0, 0, 0, 0);
    }
    r = c0[0] + c1[1] + c2[2] + c3[3];
  }
  sink[(size_t)blockIdx.x * CEIL_NT + threadIdx.x] = r;
}

// Grid-stride stream of 16-byte non-temporal loads over [src, src + n16 * 16).
__global__ __launch_bounds__(READ_NT) void ceiling_read_kernel(const v4i* __restrict__ src,
                                                               size_t n16, float* __restrict__ sink) {
  v4i acc = {0, 0, 0, 0};
  const size_t stride = (size_t)gridDim.x * READ_NT;
  size_t i = (size_t)blockIdx.x * READ_NT + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const v4i x0 = __builtin_nontemporal_load(src + i);
    const v4i x1 = __builtin_nontemporal_load(src + i + stride);
    const v4i x2 = __builtin_nontemporal_load(src + i + 2 * stride);
    const v4i x3 = __builtin_nontemporal_load(src + i + 3 * stride);
    acc ^= x0 ^ x1 ^ x2 ^ x3;
  }
  for (; i < n16; i += stride) acc ^= __builtin_nontemporal_load(src + i);
  sink[(size_t)blockIdx.x * READ_NT + threadIdx.x] = (float)(acc[0] ^ acc[1] ^ acc[2] ^ acc[3]);
}

}  // namespace
}  // namespace dsa

extern "C" {

dsa_status dsa_ceiling_mfma(int32_t kind, int32_t n_wg, int32_t iters, float* sink,
                            double* flops, hipStream_t stream) {
  if ((kind != 0 && kind != 1) || n_wg < 1 || iters < 1 || !sink || !flops)
    return DSA_ERR_INVALID_ARG;
  const double per_iter = kind == 0 ? 2.0 * 32 * 32 * 16 * 2 : 4.0 * 16 * 16 * 128 * 2;
  *flops = (double)n_wg * (dsa::CEIL_NT / dsa::kWave) * iters * per_iter;
  if (kind == 0)
    hipLaunchKernelGGL(dsa::ceiling_mfma_kernel<0>, dim3(n_wg), dim3(dsa::CEIL_NT), 0, stream,
                       iters, sink);
  else
    hipLaunchKernelGGL(dsa::ceiling_mfma_kernel<1>, dim3(n_wg), dim3(dsa::CEIL_NT), 0, stream,
                       iters, sink);
  return hipGetLastError() == hipSuccess ? DSA_OK : DSA_ERR_HIP;
}

dsa_status dsa_ceiling_read(const void* src, size_t bytes, int32_t n_wg, float* sink,
                            hipStream_t stream) {
  if (!src || !sink || n_wg < 1 || bytes == 0 || bytes % 16 != 0) return DSA_ERR_INVALID_ARG;
  hipLaunchKernelGGL(dsa::ceiling_read_kernel, dim3(n_wg), dim3(dsa::READ_NT), 0, stream,
                     reinterpret_cast<const dsa::v4i*>(src), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? DSA_OK : DSA_ERR_HIP;
}

}  // extern "C"
