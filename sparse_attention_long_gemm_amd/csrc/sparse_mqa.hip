// Sparse MQA attention over the selected shared latent KV rows on gfx950.
//
// o[t,h] = sum_{s in S_t} softmax_s(scale * q[t,h] . kv[s]) * kv[s, :D_v]
// MQA mode: one shared KV row per token (K = the whole row, 512 latent + 64 rope dims;
// V = its first 512 dims) serves all 128 query heads (openi.cn "DeepSeek-V3.2" page, item on
// MLA run in MQA mode); only the selected entries are attended (jdon.com "DeepSeek-V3.2-Exp"
// article, paragraph on fine-grained token selection).
//
// One workgroup = one query row (all heads) x one slice of its selected rows, 8 waves.  Wave
// (hg, dh) owns heads 32hg..32hg+31 and half dh of the dimensions: its share of the queries
// (dims [D_k/2 * dh, +D_k/2)) stays in registers as the B operand of
// v_mfma_f32_32x32x16_bf16 and its fp32 output accumulators (dims [D_v/2 * dh, +D_v/2)) stay in
// registers for the whole slice.  Per chunk of 32 selected rows the workgroup gathers the rows
// (coalesced 16-byte pieces) into LDS twice: row-major (A operand of S^T = K Q^T, keys x
// heads) and transposed V^T (A operand of O^T += V^T P^T, dims x heads).  The two waves of a
// head group add their half-dimension partial logits through LDS (in a fixed order, so both
// hold the same sums).  With keys on the MFMA rows, each lane owns one head, so the
// online-softmax row max and sum stay in the lane (plus one exchange with the partner lane
// that holds the other 16 keys), and the probabilities already sit in the B-operand layout of
// the value product once packed to bf16; V^T's key order inside each 16-key group is
// permuted to match that layout.
//
// Decode (paged) splits each sequence's selected rows over n_split workgroups; partial
// (unnormalised o, running max, running sum) triples are merged by mqa_combine_kernel.
#include "dsa_common.hpp"
#include "dsa_kernels.hpp"

namespace dsa {

namespace {

constexpr int NW = 8;            // 4 head groups x 2 dimension halves
constexpr int NT = NW * kWave;
constexpr int HPW = 32;          // heads per wave
constexpr int CH = 32;           // selected rows per chunk
constexpr int VSTR = CH * 2 + 16; // V^T row stride in bytes (padded against bank conflicts)
constexpr int MAX_ROWS = 2048;   // selected rows per workgroup (top_k <= 2048)

__device__ __forceinline__ v4i ld16(const void* p) { return *reinterpret_cast<const v4i*>(p); }

__device__ __forceinline__ v16f mfma_bf16(const v8bf& a, const v8bf& b, const v16f& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ v8bf as_v8bf(const v4i& x) {
  v8bf r;
  __builtin_memcpy(&r, &x, 16);
  return r;
}

// Position of chunk-relative key r inside V^T: within each 16-key group, half h of the lanes
// reads positions 8h..8h+7, which must hold keys {4h..4h+3, 8+4h..8+4h+3} (the keys whose
// probabilities those lanes hold after the S^T product).
__device__ __forceinline__ int vt_pos_of_quad(int kq) {
  return 16 * (kq >> 2) + 8 * (kq & 1) + 4 * ((kq & 3) >> 1);
}

template <int DK, int DV>
struct MqaShared {
  static constexpr int KSTR = DK * 2 + 16;  // padded row stride (bytes) of the row-major tile
  alignas(16) uint8_t ks[CH * KSTR];
  alignas(16) uint8_t vt[DV * VSTR];
  alignas(16) float sx[NW][16][kWave];      // half-dimension partial logits of each wave
  int rows[MAX_ROWS];                       // physical row of each selected entry, or -1
};

template <int DK, int DV, bool PAGED>
__global__ __launch_bounds__(NT, 1) void sparse_mqa_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ qpos_or_ctx,
    const int32_t* __restrict__ page_table, int max_pages, int n_pages, int page_size, int n_kv,
    int H, int top_k, float scale_log2, int n_split, int rows_per_split,
    uint16_t* __restrict__ out, float* __restrict__ lse, float* __restrict__ part_o,
    float* __restrict__ part_ml) {
  static_assert(DK % 32 == 0 && DV % 64 == 0 && DV <= DK, "shape");
  using Sh = MqaShared<DK, DV>;
  constexpr int KSTR = Sh::KSTR;
  constexpr int NP = DK / 8;       // 16-byte pieces per row
  constexpr int NKS = DK / 32;     // k-steps of this wave's half of the S^T product
  constexpr int NDB = DV / 64;     // 32-dim blocks of this wave's half of the output
  __shared__ Sh sh;

  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int hg = wave & 3;          // head group
  const int dh = wave >> 2;         // dimension half
  const int lane = tid & (kWave - 1);
  const int c32 = lane & 31;
  const int hf = lane >> 5;
  const int qi = blockIdx.x;
  const int sp = blockIdx.y;
  const int head = hg * HPW + c32;
  const int kd0 = dh * (DK / 2);    // first key dim of this wave's logit half
  const int vd0 = dh * (DV / 2);    // first value dim of this wave's output half
  const bool head_ok = head < H;

  // last attendable position
  int t;
  if (PAGED) {
    t = qpos_or_ctx[qi] - 1;
    if (t > max_pages * page_size - 1) t = max_pages * page_size - 1;
  } else {
    t = qpos_or_ctx[qi];
    if (t > n_kv - 1) t = n_kv - 1;
  }

  const int r0 = sp * rows_per_split;
  int r1 = r0 + rows_per_split;
  if (r1 > top_k) r1 = top_k;
  const int nrows = r1 > r0 ? r1 - r0 : 0;

  // ---- translate the slice's selected positions to physical rows (invalid -> -1) ----
  for (int i = tid; i < nrows; i += NT) {
    const int s = idx[(size_t)qi * top_k + r0 + i];
    int row = -1;
    if (s >= 0 && s <= t) {
      if (PAGED) {
        const int pg = page_table[(size_t)qi * max_pages + s / page_size];
        if (pg >= 0 && pg < n_pages) row = pg * page_size + s % page_size;
      } else {
        row = s;
      }
    }
    sh.rows[i] = row;
  }

  // ---- queries of this wave's heads: B operand, k-step ks holds dims kd0 + 16ks + 8hf .. +8
  v8bf qf[NKS];
  {
    const uint16_t* qrow = q + ((size_t)qi * H + (head_ok ? head : 0)) * DK;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      v4i x = {0, 0, 0, 0};
      if (head_ok) x = ld16(qrow + kd0 + 16 * ks + 8 * hf);
      qf[ks] = as_v8bf(x);
    }
  }

  v16f o[NDB];
#pragma unroll
  for (int d = 0; d < NDB; ++d)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[d][i] = 0.f;
  float m_run = -__builtin_inff();
  float l_run = 0.f;
  __syncthreads();

  const int n_chunks = (nrows + CH - 1) / CH;
#pragma unroll 1
  for (int c = 0; c < n_chunks; ++c) {
    // ---- gather 32 selected rows: row-major tile + permuted V^T ----
#pragma unroll 1
    for (int task = tid; task < 8 * NP; task += NT) {
      const int kq = task / NP;
      const int p = task - kq * NP;
      v4i rv[4];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int e = c * CH + 4 * kq + rr;
        const int row = (e < nrows) ? sh.rows[e] : -1;
        rv[rr] = v4i{0, 0, 0, 0};
        if (row >= 0) rv[rr] = ld16(kv + (size_t)row * DK + 8 * p);
        *reinterpret_cast<v4i*>(&sh.ks[(4 * kq + rr) * KSTR + 16 * p]) = rv[rr];
      }
      if (8 * p < DV) {
        const int pos0 = vt_pos_of_quad(kq);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const u32 a0 = (u32)rv[0][m], a1 = (u32)rv[1][m], a2 = (u32)rv[2][m], a3 = (u32)rv[3][m];
          // dim 8p + 2m (low halves) and 8p + 2m + 1 (high halves), 4 keys each
          uint2 lo, hi;
          lo.x = (a0 & 0xffffu) | (a1 << 16);
          lo.y = (a2 & 0xffffu) | (a3 << 16);
          hi.x = (a0 >> 16) | (a1 & 0xffff0000u);
          hi.y = (a2 >> 16) | (a3 & 0xffff0000u);
          *reinterpret_cast<uint2*>(&sh.vt[(8 * p + 2 * m) * VSTR + 2 * pos0]) = lo;
          *reinterpret_cast<uint2*>(&sh.vt[(8 * p + 2 * m + 1) * VSTR + 2 * pos0]) = hi;
        }
      }
    }
    __syncthreads();

    // ---- S^T = K Q^T for 32 keys x this wave's 32 heads, over its half of the dims ----
    v16f sp_;
#pragma unroll
    for (int i = 0; i < 16; ++i) sp_[i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const v8bf a = as_v8bf(ld16(&sh.ks[c32 * KSTR + 2 * (kd0 + 16 * ks + 8 * hf)]));
      sp_ = mfma_bf16(a, qf[ks], sp_);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) sh.sx[wave][i][lane] = sp_[i];
    __syncthreads();
    float s[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = sh.sx[hg][i][lane] + sh.sx[hg + 4][i][lane];

    // ---- online softmax (lane = head; element i is key 8(i/4) + 4hf + i%4) ----
    float z[16];
    float cmax = -__builtin_inff();
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = 8 * (i >> 2) + 4 * hf + (i & 3);
      const int e = c * CH + key;
      const bool ok = (e < nrows) && (sh.rows[e] >= 0);
      z[i] = ok ? s[i] * scale_log2 : -__builtin_inff();
      cmax = fmaxf(cmax, z[i]);
    }
    cmax = fmaxf(cmax, __shfl_xor(cmax, 32));
    const float m_new = fmaxf(m_run, cmax);
    float alpha = 1.f;
    float psum = 0.f;
    float pr[16];
    if (m_new == -__builtin_inff()) {
#pragma unroll
      for (int i = 0; i < 16; ++i) pr[i] = 0.f;
    } else {
      alpha = exp2f(m_run - m_new);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        pr[i] = exp2f(z[i] - m_new);
        psum += pr[i];
      }
    }
    m_run = m_new;
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int d = 0; d < NDB; ++d)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[d][i] *= alpha;

    v8bf pb[2];
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
      for (int j = 0; j < 8; ++j) pb[k2][j] = (__bf16)pr[8 * k2 + j];

    // ---- O^T += V^T P^T ----
#pragma unroll
    for (int d = 0; d < NDB; ++d) {
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        const v8bf a =
            as_v8bf(ld16(&sh.vt[(vd0 + 32 * d + c32) * VSTR + 2 * (16 * k2 + 8 * hf)]));
        o[d] = mfma_bf16(a, pb[k2], o[d]);
      }
    }
    __syncthreads();
  }

  // ---- epilogue: lane holds head `head`, dims vd0 + 32d + 8(i/4) + 4hf + i%4 ----
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (n_split == 1) {
    if (!head_ok) return;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    uint16_t* orow = out + ((size_t)qi * H + head) * DV;
#pragma unroll
    for (int d = 0; d < NDB; ++d) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint2 v;
        v.x = pack_bf16x2(o[d][4 * j + 0] * inv, o[d][4 * j + 1] * inv);
        v.y = pack_bf16x2(o[d][4 * j + 2] * inv, o[d][4 * j + 3] * inv);
        *reinterpret_cast<uint2*>(orow + vd0 + 32 * d + 8 * j + 4 * hf) = v;
      }
    }
    if (lse != nullptr && hf == 0 && dh == 0)
      lse[(size_t)qi * H + head] =
          l_tot > 0.f ? (m_run + log2f(l_tot)) * 0.69314718055994531f : -__builtin_inff();
  } else {
    if (!head_ok) return;
    float* po = part_o + (((size_t)qi * n_split + sp) * H + head) * DV;
#pragma unroll
    for (int d = 0; d < NDB; ++d)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<v4f*>(po + vd0 + 32 * d + 8 * j + 4 * hf) =
            v4f{o[d][4 * j + 0], o[d][4 * j + 1], o[d][4 * j + 2], o[d][4 * j + 3]};
    if (hf == 0 && dh == 0) {
      float* pm = part_ml + (((size_t)qi * n_split + sp) * H + head) * 2;
      pm[0] = m_run;
      pm[1] = l_tot;
    }
  }
}

// Merge the n_split partial results of one (query, head): weights exp2(m_i - M).
// One workgroup per (query, head); each thread owns 4 consecutive dims.
template <int DV>
__global__ __launch_bounds__(DV / 4) void mqa_combine_kernel(const float* __restrict__ part_o,
                                                             const float* __restrict__ part_ml,
                                                             int H, int n_split,
                                                             uint16_t* __restrict__ out,
                                                             float* __restrict__ lse) {
  const int qi = blockIdx.x / H;
  const int h = blockIdx.x - qi * H;
  const size_t base = (size_t)qi * n_split * H + h;   // partial i lives at base + i*H
  float M = -__builtin_inff();
  for (int i = 0; i < n_split; ++i) M = fmaxf(M, part_ml[(base + (size_t)i * H) * 2]);
  float L = 0.f;
  v4f acc = {0.f, 0.f, 0.f, 0.f};
  const int d = 4 * threadIdx.x;
  if (M != -__builtin_inff()) {
    for (int i = 0; i < n_split; ++i) {
      const size_t b = base + (size_t)i * H;
      const float wgt = exp2f(part_ml[b * 2] - M);
      L += wgt * part_ml[b * 2 + 1];
      const v4f v = *reinterpret_cast<const v4f*>(part_o + b * DV + d);
      acc += wgt * v;
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  uint2 o;
  o.x = pack_bf16x2(acc[0] * inv, acc[1] * inv);
  o.y = pack_bf16x2(acc[2] * inv, acc[3] * inv);
  *reinterpret_cast<uint2*>(out + ((size_t)qi * H + h) * DV + d) = o;
  if (lse != nullptr && threadIdx.x == 0)
    lse[(size_t)qi * H + h] = L > 0.f ? (M + log2f(L)) * 0.69314718055994531f : -__builtin_inff();
}

template <int DK, int DV>
hipError_t launch_shape(const MqaArgs& a, hipStream_t stream) {
  const float scale_log2 = a.scale * 1.4426950408889634f;
  if (a.page_table == nullptr) {
    hipLaunchKernelGGL((sparse_mqa_kernel<DK, DV, false>), dim3(a.n_q, 1), dim3(NT), 0, stream,
                       a.q, a.kv, a.idx, a.qpos_or_ctx, nullptr, 0, 0, 1, a.n_kv, a.H, a.top_k,
                       scale_log2, 1, a.top_k, a.out, a.lse, nullptr, nullptr);
    return hipGetLastError();
  }
  const int rps = a.rows_per_split;
  hipLaunchKernelGGL((sparse_mqa_kernel<DK, DV, true>), dim3(a.n_q, a.n_split), dim3(NT), 0,
                     stream, a.q, a.kv, a.idx, a.qpos_or_ctx, a.page_table, a.max_pages,
                     a.n_pages, a.page_size, 0, a.H, a.top_k, scale_log2, a.n_split, rps, a.out,
                     a.lse, a.part_o, a.part_ml);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_split == 1) return e;
  hipLaunchKernelGGL((mqa_combine_kernel<DV>), dim3(a.n_q * a.H), dim3(DV / 4), 0, stream,
                     a.part_o, a.part_ml, a.H, a.n_split, a.out, a.lse);
  return hipGetLastError();
}

}  // namespace

bool mqa_shape_supported(int D_k, int D_v) {
  return (D_k == 576 && D_v == 512) || (D_k == 64 && D_v == 64) || (D_k == 96 && D_v == 64);
}

hipError_t launch_sparse_mqa(const MqaArgs& a, hipStream_t stream) {
  if (a.D_k == 576 && a.D_v == 512) return launch_shape<576, 512>(a, stream);
  if (a.D_k == 64 && a.D_v == 64) return launch_shape<64, 64>(a, stream);
  if (a.D_k == 96 && a.D_v == 64) return launch_shape<96, 64>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace dsa
