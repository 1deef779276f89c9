// Lightning indexer + exact top-k on gfx950.
//
// Score (jdon.com "DeepSeek-V3.2-Exp" article, paragraph on the lightning indexer):
//     I[t,s] = sum_j w[t,j] * ReLU(q_I[t,j,:] . k_I[s,:]),   s <= t,   FP8 operands.
// Selection (same article, paragraph on fine-grained token selection): keep the top_k keys
// under (score desc, position asc).
//
// Prefill kernel (one contiguous sequence)
//   One workgroup owns QB = 16 query rows and streams the keys 0..max(t) of its rows in tiles
//   of 64.  Each of its 4 waves holds the FP8 queries of 16 indexer heads for all 16 rows in
//   registers (the MFMA B operand, 8 VGPRs per head) and multiplies them with 16-key FP8
//   fragments of k_I (A operand) using v_mfma_f32_16x16x128_f8f6f4: the output lane owns one
//   query row, so ReLU and the head weights are applied and summed in registers with no
//   cross-lane traffic.  The 4 per-wave partial sums (16 heads each) meet in LDS, where the
//   causal mask and a per-row threshold filter run; rows' surviving (score, position) items
//   are appended in position order to a per-row candidate list in the workspace.  When a
//   list would overflow, it is cut to exactly top_k items by the block-wide radix select
//   (dsa_select.hpp), which also raises the row's threshold to the top_k-th score; only keys
//   scoring strictly above it can enter afterwards (a later key with an equal score has a
//   higher position, so it would lose the tie).  No n_q x L score matrix is ever stored.
//
// Decode kernels (paged cache, one query per sequence)
//   indexer_logits_paged: one wave scores 64 keys of one sequence; the A operand is the
//   query's 64 heads (4 fragments of 16), the B operand 16 keys read through the page table,
//   so the output lane owns one key and 4 heads; heads are summed in registers and across
//   the 4 lane groups.  Logits go to the workspace ([B, max_pages*page_size] fp32, 4 bytes
//   per key against 128 bytes of key read).  topk_rows then selects each row exactly.
#include "dsa_common.hpp"
#include "dsa_kernels.hpp"
#include "dsa_select.hpp"

namespace dsa {

namespace {

constexpr int QB = 16;       // query rows per workgroup
constexpr int NWAVE = 4;     // waves per workgroup, 16 indexer heads each
constexpr int NT = NWAVE * kWave;
constexpr int BK = 64;       // keys per tile
constexpr int HPW = 16;      // indexer heads per wave
constexpr int PSTR = BK + 4; // padded LDS row stride (floats) of the per-wave partial scores

__device__ __forceinline__ v4i load16(const uint8_t* p) { return *reinterpret_cast<const v4i*>(p); }

// 32 bytes [32g, 32g+32) of an FP8 row of d_I bytes (d_I a multiple of 16), zero past d_I.
__device__ __forceinline__ v8i load_row32(const uint8_t* row, int g, int d_I, bool ok) {
  v4i lo = {0, 0, 0, 0}, hi = {0, 0, 0, 0};
  if (ok) {
    if (32 * g < d_I) lo = load16(row + 32 * g);
    if (32 * g + 16 < d_I) hi = load16(row + 32 * g + 16);
  }
  v8i r;
  r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
  r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
  return r;
}

__device__ __forceinline__ v4f mfma_fp8(const v8i& a, const v8i& b) {
  const v4f z = {0.f, 0.f, 0.f, 0.f};
  // Scale operands 0 select the unscaled FP8 x FP8 form (formats 0/0 = e4m3 / e4m3).
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, z, 0, 0, 0, 0, 0, 0);
}

struct CandItem {
  u32 key;
  float score;
  int32_t pos;
};

struct PrefillShared {
  float part[NWAVE][QB][PSTR];
  float thr[QB];
  int cnt[QB];
  int need;
  SelectShared sel;
};

// Cut row q's candidate list (n > top_k items, position order) to its exact top_k, in place;
// returns the new threshold (the top_k-th score).
__device__ float compact_row(float* cs, int32_t* ci, int n, int top_k, SelectShared& sel) {
  u32 T;
  int r;
  block_radix_select<NT>([&](int i) { return ord_key(cs[i]); }, n, top_k, sel, T, r);
  block_stable_keep<NT>(
      [&](int i) { CandItem it; it.score = cs[i]; it.pos = ci[i]; it.key = ord_key(it.score); return it; },
      n, T, r,
      [&](const CandItem& it, int p) {
        if (p < top_k) {
          cs[p] = it.score;
          ci[p] = it.pos;
        }
      },
      sel);
  return key_to_float(T);
}

__global__ __launch_bounds__(NT, 1) void indexer_topk_prefill_kernel(
    const uint8_t* __restrict__ q_idx, const float* __restrict__ w,
    const uint8_t* __restrict__ k_idx, const int32_t* __restrict__ q_pos, int n_q, int n_keys,
    int H_I, int d_I, int top_k, int cap, float* __restrict__ cand_score,
    int32_t* __restrict__ cand_pos, int32_t* __restrict__ out_idx) {
  __shared__ PrefillShared sh;
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid & (kWave - 1);
  const int g = lane >> 4;     // lane group: bytes [32g, 32g+32) of a row; output rows 4g..4g+3
  const int c16 = lane & 15;   // output column = query row within the block
  const int q0 = blockIdx.x * QB;

  // ---- per-row state ----
  if (tid < QB) {
    sh.thr[tid] = -__builtin_inff();
    sh.cnt[tid] = 0;
  }
  // last candidate position of each row of the block, and of the block
  int t_lane = -1;
  {
    const int q = q0 + c16;
    if (q < n_q) t_lane = min(q_pos[q], n_keys - 1);
  }
  int t_max = t_lane;
  for (int o = 1; o < 16; o <<= 1) t_max = max(t_max, __shfl_xor(t_max, o));

  // ---- queries of this wave's 16 heads for the 16 rows (MFMA B operand) ----
  v8i qf[HPW];
  float wv[HPW];
  {
    const int q = q0 + c16;
#pragma unroll
    for (int j = 0; j < HPW; ++j) {
      const int h = wave * HPW + j;
      const bool ok = (q < n_q) && (h < H_I);
      qf[j] = load_row32(q_idx + ((size_t)q * H_I + h) * d_I, g, d_I, ok);
      wv[j] = ok ? w[(size_t)q * H_I + h] : 0.f;
    }
  }
  __syncthreads();

  const int n_tiles = (t_max + BK) / BK;  // tiles covering keys 0..t_max
#pragma unroll 1
  for (int tile = 0; tile < n_tiles; ++tile) {
    const int s0 = tile * BK;
    // ---- partial scores of this wave's heads: keys s0..s0+63 x 16 rows ----
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const int s = s0 + 16 * f + c16;
      const v8i a = load_row32(k_idx + (size_t)s * d_I, g, d_I, s < n_keys);
      float acc0 = 0.f, acc1 = 0.f, acc2 = 0.f, acc3 = 0.f;
#pragma unroll
      for (int j = 0; j < HPW; ++j) {
        const v4f x = mfma_fp8(a, qf[j]);
        acc0 = fmaf(wv[j], fmaxf(x[0], 0.f), acc0);
        acc1 = fmaf(wv[j], fmaxf(x[1], 0.f), acc1);
        acc2 = fmaf(wv[j], fmaxf(x[2], 0.f), acc2);
        acc3 = fmaf(wv[j], fmaxf(x[3], 0.f), acc3);
      }
      // lane holds keys 16f + 4g + (0..3) of query row c16
      float* dst = &sh.part[wave][c16][16 * f + 4 * g];
      *reinterpret_cast<v4f*>(dst) = v4f{acc0, acc1, acc2, acc3};
    }
    __syncthreads();
    // ---- head sum, causal mask, threshold filter, ordered append (wave owns 4 rows) ----
#pragma unroll 1
    for (int rr = 0; rr < QB / NWAVE; ++rr) {
      const int r = wave * (QB / NWAVE) + rr;
      const int q = q0 + r;
      if (q >= n_q) break;
      const int t = min(q_pos[q], n_keys - 1);
      if (s0 > t) continue;
      const int s = s0 + lane;
      const float sc = ((sh.part[0][r][lane] + sh.part[1][r][lane]) + sh.part[2][r][lane]) +
                       sh.part[3][r][lane];
      const bool pass = (s <= t) && (sc > sh.thr[r]);
      const uint64_t m = wave_ballot(pass);
      const int c = sh.cnt[r];
      if (pass) {
        const int p = c + lanes_below(m);
        cand_score[(size_t)q * cap + p] = (sc == 0.f) ? 0.f : sc;
        cand_pos[(size_t)q * cap + p] = s;
      }
      if (lane == 0) sh.cnt[r] = c + __builtin_popcountll(m);
    }
    __syncthreads();
    // ---- cut any list that could overflow on the next tile ----
    if (tile + 1 < n_tiles) {
      bool any = false;
#pragma unroll 1
      for (int r = 0; r < QB; ++r) any |= (sh.cnt[r] + BK > cap);
      if (any) {
#pragma unroll 1
        for (int r = 0; r < QB; ++r) {
          const int n = sh.cnt[r];
          if (n + BK <= cap) continue;
          const int q = q0 + r;
          const float T = compact_row(cand_score + (size_t)q * cap, cand_pos + (size_t)q * cap,
                                      n, top_k, sh.sel);
          __syncthreads();
          if (tid == 0) {
            sh.thr[r] = T;
            sh.cnt[r] = top_k;
          }
          __syncthreads();
        }
      }
    }
  }

  // ---- final exact selection of every row ----
#pragma unroll 1
  for (int r = 0; r < QB; ++r) {
    const int q = q0 + r;
    if (q >= n_q) break;
    const int n = sh.cnt[r];
    int32_t* orow = out_idx + (size_t)q * top_k;
    const float* cs = cand_score + (size_t)q * cap;
    const int32_t* ci = cand_pos + (size_t)q * cap;
    if (n <= top_k) {
      for (int i = tid; i < top_k; i += NT) orow[i] = (i < n) ? ci[i] : -1;
    } else {
      u32 T;
      int rr;
      block_radix_select<NT>([&](int i) { return ord_key(cs[i]); }, n, top_k, sh.sel, T, rr);
      block_stable_keep<NT>(
          [&](int i) { CandItem it; it.score = cs[i]; it.pos = ci[i]; it.key = ord_key(it.score); return it; },
          n, T, rr, [&](const CandItem& it, int p) { if (p < top_k) orow[p] = it.pos; }, sh.sel);
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------------------------------
// Decode: logits of one query per sequence over its paged keys.
// ------------------------------------------------------------------------------------------
constexpr int DEC_KEYS_PER_WAVE = 64;
constexpr int DEC_WAVES = 4;
constexpr int DEC_KEYS_PER_BLOCK = DEC_KEYS_PER_WAVE * DEC_WAVES;

__global__ __launch_bounds__(DEC_WAVES * kWave) void indexer_logits_paged_kernel(
    const uint8_t* __restrict__ q_idx, const float* __restrict__ w,
    const uint8_t* __restrict__ k_cache, const int32_t* __restrict__ page_table,
    const int32_t* __restrict__ ctx_lens, int max_pages, int n_pages, int page_size, int H_I,
    int d_I, int row_stride, float* __restrict__ logits) {
  const int b = blockIdx.y;
  const int ctx = ctx_lens[b];
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int g = lane >> 4, c16 = lane & 15;
  const int base = blockIdx.x * DEC_KEYS_PER_BLOCK + wave * DEC_KEYS_PER_WAVE;
  if (base >= ctx) return;

  // A operand: heads 16*hg + (lane & 15), bytes [32g, 32g+32)
  v8i qa[4];
  float wl[4][4];
#pragma unroll
  for (int hg = 0; hg < 4; ++hg) {
    const int h = 16 * hg + c16;
    qa[hg] = load_row32(q_idx + ((size_t)b * H_I + h) * d_I, g, d_I, h < H_I);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hh = 16 * hg + 4 * g + i;  // head of output row 4g+i
      wl[hg][i] = (hh < H_I) ? w[(size_t)b * H_I + hh] : 0.f;
    }
  }
  const int32_t* pt = page_table + (size_t)b * max_pages;
#pragma unroll
  for (int f = 0; f < DEC_KEYS_PER_WAVE / 16; ++f) {
    const int s = base + 16 * f + c16;
    bool ok = s < ctx && s < row_stride;
    int page = 0;
    if (ok) {
      page = pt[s / page_size];
      ok = (page >= 0) && (page < n_pages);
    }
    const uint8_t* row = k_cache + ((size_t)page * page_size + (ok ? s % page_size : 0)) * d_I;
    const v8i kb = load_row32(row, g, d_I, ok);
    float acc = 0.f;
#pragma unroll
    for (int hg = 0; hg < 4; ++hg) {
      const v4f x = mfma_fp8(qa[hg], kb);  // rows: heads 16hg+4g+i, column: key c16
      acc = fmaf(wl[hg][0], fmaxf(x[0], 0.f), acc);
      acc = fmaf(wl[hg][1], fmaxf(x[1], 0.f), acc);
      acc = fmaf(wl[hg][2], fmaxf(x[2], 0.f), acc);
      acc = fmaf(wl[hg][3], fmaxf(x[3], 0.f), acc);
    }
    acc += __shfl_xor(acc, 16);
    acc += __shfl_xor(acc, 32);
    if (g == 0 && s < ctx && s < row_stride) logits[(size_t)b * row_stride + s] = acc;
  }
}

constexpr int TOPK_NT = 1024;

struct PosItem {
  u32 key;
  int32_t pos;
};

__global__ __launch_bounds__(TOPK_NT) void topk_rows_kernel(const float* __restrict__ logits,
                                                            const int32_t* __restrict__ ctx_lens,
                                                            int row_stride, int top_k,
                                                            int32_t* __restrict__ out_idx) {
  __shared__ SelectShared sh;
  const int b = blockIdx.x;
  const int n = min(max(ctx_lens[b], 0), row_stride);
  const float* row = logits + (size_t)b * row_stride;
  int32_t* orow = out_idx + (size_t)b * top_k;
  if (n <= top_k) {
    for (int i = threadIdx.x; i < top_k; i += TOPK_NT) orow[i] = (i < n) ? i : -1;
    return;
  }
  u32 T;
  int r;
  block_radix_select<TOPK_NT>([&](int i) { return ord_key(row[i]); }, n, top_k, sh, T, r);
  block_stable_keep<TOPK_NT>(
      [&](int i) { PosItem it; it.key = ord_key(row[i]); it.pos = i; return it; }, n, T, r,
      [&](const PosItem& it, int p) { if (p < top_k) orow[p] = it.pos; }, sh);
}

}  // namespace

// ------------------------------------------------------------------------------------------
// Host launchers
// ------------------------------------------------------------------------------------------
int indexer_cap(int top_k) {
  int cap = 2 * top_k;
  if (cap < top_k + BK) cap = top_k + BK;
  return (cap + BK - 1) / BK * BK;
}

size_t indexer_prefill_ws(int n_q, int top_k) {
  return (size_t)n_q * (size_t)indexer_cap(top_k) * (sizeof(float) + sizeof(int32_t));
}

hipError_t launch_indexer_topk_prefill(const uint8_t* q_idx, const float* w, const uint8_t* k_idx,
                                       int n_keys, const int32_t* q_pos, int n_q, int H_I,
                                       int d_I, int top_k, int32_t* out_idx, void* ws,
                                       hipStream_t stream) {
  const int cap = indexer_cap(top_k);
  float* cs = reinterpret_cast<float*>(ws);
  int32_t* ci = reinterpret_cast<int32_t*>(cs + (size_t)n_q * cap);
  const int grid = (n_q + QB - 1) / QB;
  hipLaunchKernelGGL(indexer_topk_prefill_kernel, dim3(grid), dim3(NT), 0, stream, q_idx, w,
                     k_idx, q_pos, n_q, n_keys, H_I, d_I, top_k, cap, cs, ci, out_idx);
  return hipGetLastError();
}

size_t indexer_paged_ws(int B, int max_pages, int page_size) {
  return (size_t)B * (size_t)max_pages * (size_t)page_size * sizeof(float);
}

hipError_t launch_indexer_topk_paged(const uint8_t* q_idx, const float* w, const uint8_t* k_cache,
                                     const int32_t* page_table, const int32_t* ctx_lens, int B,
                                     int max_pages, int n_pages, int page_size, int H_I, int d_I,
                                     int top_k, int32_t* out_idx, void* ws, hipStream_t stream) {
  const int row_stride = max_pages * page_size;
  float* logits = reinterpret_cast<float*>(ws);
  dim3 grid((row_stride + DEC_KEYS_PER_BLOCK - 1) / DEC_KEYS_PER_BLOCK, B);
  hipLaunchKernelGGL(indexer_logits_paged_kernel, grid, dim3(DEC_WAVES * kWave), 0, stream, q_idx,
                     w, k_cache, page_table, ctx_lens, max_pages, n_pages, page_size, H_I, d_I,
                     row_stride, logits);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(topk_rows_kernel, dim3(B), dim3(TOPK_NT), 0, stream, logits, ctx_lens,
                     row_stride, top_k, out_idx);
  return hipGetLastError();
}

}  // namespace dsa
