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

// Random-row gather along index rows, in the attention's shape: workgroups of 8 waves walk the
// index rows blockIdx.x, blockIdx.x + gridDim.x, ...; each chunk of 32 listed rows is
// row16 * 32 pieces of 16 bytes in row-major order, piece p loaded by thread p % 512.  An index
// outside [0, n_rows) loads row 0.  KIND 0: LDS DMA (global_load_lds_dwordx4, one instruction
// per wave-load with per-lane addresses) into two alternating 1 KB buffers per wave, at most
// one wave-load of the wave in flight behind the newest; KIND 1: plain 16-byte loads into
// registers, one chunk's loads of a thread in flight before they are folded into a checksum.
constexpr int GATH_NT = 512;
constexpr int GATH_CH = 32;
constexpr int GATH_MAXPER = 8;   // pieces per thread and chunk (rows up to 2048 bytes)

template <int KIND>
__global__ __launch_bounds__(GATH_NT) void ceiling_gather_kernel(
    const uint8_t* __restrict__ pool, int64_t n_rows, int row16, const int32_t* __restrict__ idx,
    int n_q, int top_k, float* __restrict__ sink) {
  __shared__ __attribute__((aligned(16))) uint8_t buf[GATH_NT / kWave][2][kWave * 16];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid & (kWave - 1);
  const int pieces = row16 * GATH_CH;
  const int per = (pieces + GATH_NT - 1) / GATH_NT;
  const size_t row_bytes = (size_t)row16 * 16;
  v4i acc = {0, 0, 0, 0};
  int n = 0;
  for (int qr = blockIdx.x; qr < n_q; qr += gridDim.x) {
    const int32_t* ir = idx + (size_t)qr * top_k;
    for (int c = 0; c + GATH_CH <= top_k; c += GATH_CH) {
      v4i x[GATH_MAXPER];
#pragma unroll
      for (int k = 0; k < GATH_MAXPER; ++k) {
        if (k >= per) break;
        const int p = tid + GATH_NT * k;
        const int pp = p < pieces ? p : 0;
        const int r = pp / row16, s = pp - r * row16;
        const int64_t row = ir[c + r];
        const uint8_t* src = pool + (size_t)(row >= 0 && row < n_rows ? row : 0) * row_bytes + 16 * s;
        if constexpr (KIND == 0) {
          const u32 lds = __builtin_amdgcn_readfirstlane(
              (u32)(uintptr_t)(__attribute__((address_space(3))) void*)(&buf[wave][n & 1][0]));
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
          asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off\n\t"
                       "s_waitcnt vmcnt(1)"
                       :
                       : "v"(src), "s"(lds)
                       : "memory", "m0");
#pragma clang diagnostic pop
          ++n;
        } else {
          x[k] = *reinterpret_cast<const v4i*>(src);
        }
      }
      if constexpr (KIND == 1) {
#pragma unroll
        for (int k = 0; k < GATH_MAXPER; ++k)
          if (k < per) acc ^= x[k];
      }
    }
  }
  if constexpr (KIND == 0) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    acc[0] = reinterpret_cast<const int*>(&buf[wave][0][0])[lane];
  }
  sink[(size_t)blockIdx.x * GATH_NT + tid] = (float)(acc[0] ^ acc[1] ^ acc[2] ^ acc[3]);
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

extern "C" dsa_status dsa_ceiling_gather(int32_t kind, const void* pool, int64_t n_rows,
                                         int32_t row_bytes, const int32_t* idx, int32_t n_q,
                                         int32_t top_k, int32_t n_wg, float* sink,
                                         hipStream_t stream) {
  if ((kind != 0 && kind != 1) || !pool || !idx || !sink || n_rows < 1 || row_bytes < 16 ||
      row_bytes % 16 != 0 || row_bytes / 16 * dsa::GATH_CH > dsa::GATH_MAXPER * dsa::GATH_NT ||
      n_q < 1 || top_k < dsa::GATH_CH || top_k % dsa::GATH_CH != 0 || n_wg < 1)
    return DSA_ERR_INVALID_ARG;
  const auto* src = reinterpret_cast<const uint8_t*>(pool);
  if (kind == 0)
    hipLaunchKernelGGL(dsa::ceiling_gather_kernel<0>, dim3(n_wg), dim3(dsa::GATH_NT), 0, stream,
                       src, n_rows, row_bytes / 16, idx, n_q, top_k, sink);
  else
    hipLaunchKernelGGL(dsa::ceiling_gather_kernel<1>, dim3(n_wg), dim3(dsa::GATH_NT), 0, stream,
                       src, n_rows, row_bytes / 16, idx, n_q, top_k, sink);
  return hipGetLastError() == hipSuccess ? DSA_OK : DSA_ERR_HIP;
}
