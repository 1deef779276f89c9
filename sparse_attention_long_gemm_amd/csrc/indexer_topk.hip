// Lightning indexer + exact top-k on gfx950.
//
// Score (jdon.com "DeepSeek-V3.2-Exp" article, paragraph on the lightning indexer):
//     I[t,s] = sum_j w[t,j] * ReLU(q_I[t,j,:] . k_I[s,:]),   s <= t,   FP8 operands.
// Selection (same article, paragraph on fine-grained token selection): keep the top_k keys
// under (score desc, position asc).
//
// Prefill kernel (one contiguous sequence)
//   One workgroup (8 waves) owns QB = 16 query rows and streams the keys 0..max(t) of its rows,
//   128 keys per iteration, through a double-buffered LDS key tile (16-byte chunks
//   XOR-swizzled).  Wave (hg, kh) holds the FP8 queries of indexer heads 16hg..16hg+15 for the
//   16 rows in registers (the B operand of v_mfma_f32_16x16x128_f8f6f4, 8 VGPRs per head) and
//   scores the 64 keys of tile half kh: the output lane owns one query row, so the head sum
//   runs in registers.  ReLU is split as w ReLU(x) = (w x + w |x|) / 2: the |x| half costs one
//   fma per product (the abs is a free operand modifier), and the linear half is a single
//   product q_lin . k with q_lin[t] = sum_j w[t,j] q_I[t,j,:], run on bf16 MFMAs with q_lin
//   split exactly into three bf16 pieces (FP8 keys convert to bf16 exactly).  The per-wave
//   partial sums meet in LDS, where each wave applies the causal mask and a per-row threshold
//   filter to its 2 rows and appends the surviving (score, position) items, in position order,
//   to the row's candidate list in the workspace.  When lists near their capacity, every row
//   past half of its slack is cut at the next iteration (all waves together) to a threshold
//   that is at most its top_k-th score: from a per-row LDS histogram of the listed scores when
//   that leaves enough room, else by an exact radix select (dsa_select.hpp).  Only keys
//   scoring strictly above the row's threshold can enter afterwards (a later key with an equal
//   score has a higher position, so it would lose the tie).  A last exact select per row
//   writes the sorted top_k positions.  No n_q x L score matrix is ever stored.
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

constexpr int QB = 16;         // query rows per workgroup
constexpr int NWAVE = 8;       // 4 head groups x 2 key-tile parities
constexpr int NT = NWAVE * kWave;
constexpr int BK = 64;         // keys per tile; one iteration covers 2 tiles = 128 keys
constexpr int BK2 = 2 * BK;
constexpr int HPW = 16;        // indexer heads per wave
constexpr int PSTR = BK + 4;   // padded LDS row stride (floats) of the partial scores
constexpr int RPW = QB / NWAVE;  // query rows owned by each wave (filter + selection)

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
  float part[2][2][4][QB][PSTR];  // [buffer][tile parity][head group][row][key]: sum w|x|
  float plin[2][2][QB][PSTR];     // [buffer][tile parity][row][key]: sum w x (all heads)
  alignas(16) uint8_t ktile[2][BK2 * 128];  // [buffer][key][128 B], 16 B chunks XOR-swizzled
  alignas(16) __bf16 qlin[3][4][kWave][8];  // [bf16 piece][k-step][lane][8]: B operand of
                                            // the linear term (stored element-wise)
  u32 hist[NWAVE][256];           // per-wave radix histograms
  u32 rhist[QB][256];             // per-row histogram of the listed scores (see RowHist)
  int full[2][NWAVE];             // [iteration parity][wave]: a row of the wave is near full
};

// Physical 16-byte chunk of logical chunk c (0..7) of key row r in a key tile: the XOR spreads
// the 16 rows one fragment read touches over all 64 LDS banks.
__device__ __forceinline__ int kchunk(int r, int c) { return c ^ ((r >> 1) & 7); }

// Per-row histogram of the order keys of the listed candidates over [lo, hi_seen]: 256 bins
// of width 2^shift starting at lo (keys above the range land in the last bin).  Every listed
// key is >= lo, so the lower edge of any bin is a lower bound for the keys counted in it.
struct RowHist {
  u32 lo = 0u;
  int shift = 0;
  bool valid = false;
};

__device__ __forceinline__ int hbin(u32 key, const RowHist& h) {
  const u32 b = (key - h.lo) >> h.shift;
  return b > 255u ? 255 : (int)b;
}

__device__ __forceinline__ void hrange(RowHist& h, u32 lo, u32 hi) {
  h.lo = lo;
  const u32 span = hi > lo ? hi - lo : 0u;
  h.shift = span == 0u ? 0 : max(0, 32 - __builtin_clz(span) - 8);
  h.valid = true;
}

__device__ __forceinline__ u32 wave_max_u32(u32 v) {
  for (int o = 32; o >= 1; o >>= 1) v = max(v, (u32)__shfl_xor((int)v, o));
  return v;
}

// Cut a row's candidate list (n > top_k items in position order) in place.  Any threshold that
// is at most the top_k-th best key seen so far is valid: a later key must beat it strictly to
// enter (a later key with an equal score has a higher position, so it loses every tie).
//  * Histogram cut (one pass): the lower edge T of the highest bin b whose suffix count reaches
//    top_k; keeps every key >= T.  Used when the histogram is valid, b > 0 and the survivors
//    leave room for two more iterations of appends.
//  * Exact cut (radix select): keeps exactly the top_k; used otherwise (first cut, or scores
//    piled into one bin, e.g. massive ties).
// Both rebuild the row histogram over [T, hi_seen] from the survivors.  Returns the new
// threshold score; *n_out receives the survivor count.
__device__ float wave_cut(float* cs, int32_t* ci, int n, int top_k, int cap, u32 hi_seen,
                          RowHist& h, u32* rh, u32* hist, int* n_out) {
  const int lane = threadIdx.x & (kWave - 1);
  u32 T = 0u;
  bool exact = true;
  if (h.valid) {
    u32 c[4];
    int tot = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      c[b] = rh[4 * lane + b];
      tot += (int)c[b];
    }
    int incl = tot;  // suffix sum over lanes >= this lane
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int t = __shfl_down(incl, o);
      if (lane + o < kWave) incl += t;
    }
    // highest bin whose suffix count reaches top_k, and that count
    int bsel = -1, cnt_b = 0;
    const int excl = incl - tot;
    if (excl < top_k && top_k <= incl) {
      int cum = excl;
      for (int b = 3; b >= 0; --b) {
        cum += (int)c[b];
        if (cum >= top_k) {
          bsel = 4 * lane + b;
          cnt_b = cum;
          break;
        }
      }
    }
    const uint64_t who = wave_ballot(bsel >= 0);
    const int src = __builtin_ctzll(who | (1ull << 63));
    bsel = __builtin_amdgcn_readlane(bsel, src);
    cnt_b = __builtin_amdgcn_readlane(cnt_b, src);
    if (who != 0ull && bsel > 0 && cnt_b <= cap - 2 * BK2) {
      exact = false;
      T = h.lo + ((u32)bsel << h.shift);
    }
  }
  int r = 0;
  if (exact) wave_radix_select([&](int i) { return ord_key(cs[i]); }, n, top_k, hist, T, r);
  // rebuild the histogram for the survivors over [T, hi_seen]
#pragma unroll
  for (int b = 0; b < 4; ++b) rh[4 * lane + b] = 0u;
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  hrange(h, T, hi_seen);
  int kept;
  auto load = [&](int i) { CandItem it; it.score = cs[i]; it.pos = ci[i]; it.key = ord_key(it.score); return it; };
  auto emit = [&](const CandItem& it, int p) {
    if (p < cap) {
      cs[p] = it.score;
      ci[p] = it.pos;
      atomicAdd(&rh[hbin(it.key, h)], 1u);
    }
  };
  if (exact) {
    kept = wave_stable_keep(load, n, T, r, emit);
  } else {
    // keep every key >= T: "key > T - 1" with no ties to resolve (T >= 1 since bin b > 0)
    kept = wave_stable_keep(load, n, T - 1u, 0, emit);
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  *n_out = kept;
  return key_to_float(T);
}

// 8 FP8 bytes (ints 2ks, 2ks+1 of a 32-byte fragment) -> 8 bf16 (exact: e4m3 is a subset).
__device__ __forceinline__ v8bf fp8x8_to_bf16(int lo, int hi) {
  typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
  const v2bf a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((u32)lo, 1.0f, false);
  const v2bf b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((u32)lo, 1.0f, true);
  const v2bf c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((u32)hi, 1.0f, false);
  const v2bf d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((u32)hi, 1.0f, true);
  v8bf r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

// Linear term sum_j w_j (q_j . k) = q_lin . k for one 16-key fragment and the 16 rows.
// k-step ks of lane group g covers dims 32g + 8ks .. +8, like the FP8 fragments.
__device__ __forceinline__ v4f linear_term(const v8i& a, const PrefillShared& sh, int lane) {
  v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const v8bf ab = fp8x8_to_bf16(a[2 * ks], a[2 * ks + 1]);
#pragma unroll
    for (int pc = 0; pc < 3; ++pc)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          ab, *reinterpret_cast<const v8bf*>(&sh.qlin[pc][ks][lane][0]), acc, 0, 0, 0);
  }
  return acc;
}

// Key fragment (16 keys x 32 bytes per lane group) of tile row r0.. from the LDS key tile.
__device__ __forceinline__ v8i frag_from_tile(const uint8_t* tile, int r, int g) {
  const v4i lo = *reinterpret_cast<const v4i*>(tile + r * 128 + 16 * kchunk(r, 2 * g));
  const v4i hi = *reinterpret_cast<const v4i*>(tile + r * 128 + 16 * kchunk(r, 2 * g + 1));
  v8i a;
  a[0] = lo[0]; a[1] = lo[1]; a[2] = lo[2]; a[3] = lo[3];
  a[4] = hi[0]; a[5] = hi[1]; a[6] = hi[2]; a[7] = hi[3];
  return a;
}

__device__ __forceinline__ void epi_abs(float* acc, const v4f& x, float wj) {
  acc[0] = fmaf(wj, __builtin_fabsf(x[0]), acc[0]);
  acc[1] = fmaf(wj, __builtin_fabsf(x[1]), acc[1]);
  acc[2] = fmaf(wj, __builtin_fabsf(x[2]), acc[2]);
  acc[3] = fmaf(wj, __builtin_fabsf(x[3]), acc[3]);
}

__global__ __launch_bounds__(NT, 1) void indexer_topk_prefill_kernel(
    const uint8_t* __restrict__ q_idx, const float* __restrict__ w,
    const uint8_t* __restrict__ k_idx, const int32_t* __restrict__ q_pos, int n_q, int n_keys,
    int H_I, int d_I, int top_k, int cap, float* __restrict__ cand_score,
    int32_t* __restrict__ cand_pos, int32_t* __restrict__ out_idx) {
  __shared__ PrefillShared sh;
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int hg = wave & 3;       // head group: heads 16hg..16hg+15
  const int kh = wave >> 2;      // key-tile parity: tile 2i+kh of iteration i
  const int lane = tid & (kWave - 1);
  const int g = lane >> 4;       // lane group: bytes [32g, 32g+32) of a row; output rows 4g..4g+3
  const int c16 = lane & 15;     // output column = query row within the block
  const int q0 = blockIdx.x * QB;
  const bool heads_here = HPW * hg < H_I;

  // ---- last candidate position of each row (t clamped to the keys; -1: nothing) ----
  int t_lane = -1;
  {
    const int q = q0 + c16;
    if (q < n_q) t_lane = min(q_pos[q], n_keys - 1);
  }
  int t_max = t_lane;
  for (int o = 1; o < 16; o <<= 1) t_max = max(t_max, __shfl_xor(t_max, o));
  // rows owned by this wave, their state (wave-uniform)
  int t_own[RPW], cnt[RPW];
  float thr[RPW];
  u32 hi_seen[RPW];   // per lane: largest order key this lane ever listed for the row
  RowHist rowh[RPW];
#pragma unroll
  for (int rr = 0; rr < RPW; ++rr) {
    t_own[rr] = __shfl(t_lane, RPW * wave + rr);
    cnt[rr] = 0;
    thr[rr] = -__builtin_inff();
    hi_seen[rr] = 0u;
  }

  // ---- q_lin[row][d] = sum_j w[row][j] q_I[row][j][d] in fp32, split into 3 bf16 pieces
  // (hi + mid + lo == q_lin exactly) laid out as the B operand of the linear-term MFMA ----
  {
    const int row = tid >> 5;            // 16 rows x 32 threads, 4 dims each
    const int d0 = 4 * (tid & 31);
    const int q = q0 + row;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    if (q < n_q && d0 < d_I) {
      for (int j = 0; j < H_I; ++j) {
        const u32 b4 = *reinterpret_cast<const u32*>(q_idx + ((size_t)q * H_I + j) * d_I + d0);
        const float wj = w[(size_t)q * H_I + j];
        typedef float v2f __attribute__((ext_vector_type(2)));
        const v2f lo = __builtin_amdgcn_cvt_pk_f32_fp8(b4, false);
        const v2f hi = __builtin_amdgcn_cvt_pk_f32_fp8(b4, true);
        acc[0] = fmaf(wj, lo[0], acc[0]);
        acc[1] = fmaf(wj, lo[1], acc[1]);
        acc[2] = fmaf(wj, hi[0], acc[2]);
        acc[3] = fmaf(wj, hi[1], acc[3]);
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int d = d0 + e;
      const int gg = d >> 5, ks = (d & 31) >> 3, jj = d & 7;
      const int ln = 16 * gg + row;
      float v = acc[e];
#pragma unroll
      for (int pc = 0; pc < 3; ++pc) {
        const __bf16 b = (__bf16)v;             // round to nearest even
        sh.qlin[pc][ks][ln][jj] = b;
        v -= (float)b;                          // exact remainder
      }
    }
  }

  // ---- queries of this wave's 16 heads for the 16 rows (MFMA B operand) ----
  v8i qf[HPW];
  float wv[HPW];
  {
    const int q = q0 + c16;
#pragma unroll
    for (int j = 0; j < HPW; ++j) {
      const int h = hg * HPW + j;
      const bool ok = (q < n_q) && (h < H_I);
      qf[j] = load_row32(q_idx + ((size_t)q * H_I + h) * d_I, g, d_I, ok);
      wv[j] = ok ? w[(size_t)q * H_I + h] : 0.f;
    }
  }

  // ---- key tile loads: thread -> (key row lr = tid / 4, 32-byte half-pair hp = tid % 4) ----
  const int lr = tid >> 2, lc = 2 * (tid & 3);  // logical 16-byte chunks lc, lc+1
  auto load_tile = [&](int it_, v4i& c0, v4i& c1) {
    const int s = it_ * BK2 + lr;
    const bool ok = s < n_keys;
    c0 = v4i{0, 0, 0, 0};
    c1 = v4i{0, 0, 0, 0};
    if (ok && 16 * lc < d_I) c0 = load16(k_idx + (size_t)s * d_I + 16 * lc);
    if (ok && 16 * lc + 16 < d_I) c1 = load16(k_idx + (size_t)s * d_I + 16 * lc + 16);
  };
  auto store_tile = [&](int b, const v4i& c0, const v4i& c1) {
    *reinterpret_cast<v4i*>(&sh.ktile[b][lr * 128 + 16 * kchunk(lr, lc)]) = c0;
    *reinterpret_cast<v4i*>(&sh.ktile[b][lr * 128 + 16 * kchunk(lr, lc + 1)]) = c1;
  };

  const int n_iter = (t_max + BK2) / BK2;  // iterations covering keys 0..t_max
  {
    v4i c0, c1;
    load_tile(0, c0, c1);
    store_tile(0, c0, c1);
  }
  __syncthreads();

  // Iteration `it` computes the partial scores of keys [128 it, 128 it + 128) from key tile
  // buffer it%2 while the next tile is fetched, then filters that iteration's keys.
#pragma unroll 1
  for (int it = 0; it < n_iter; ++it) {
    const int buf = it & 1;

    // ---- cut candidate lists, all waves together (a cut stalls the whole workgroup at the
    // next barrier, so cuts are batched): when any row ended the previous filter with less
    // than one iteration of room, every row past half of its slack is cut ----
    if (it >= 1) {
      bool any_full = false;
#pragma unroll
      for (int v = 0; v < NWAVE; ++v) any_full |= sh.full[(it - 1) & 1][v] != 0;
      if (any_full) {
#pragma unroll
        for (int rr = 0; rr < RPW; ++rr) {
          const int q = q0 + RPW * wave + rr;
          if (q >= n_q || it * BK2 > t_own[rr] || 2 * cnt[rr] <= top_k + cap) continue;
          int kept;
          thr[rr] = wave_cut(cand_score + (size_t)q * cap, cand_pos + (size_t)q * cap, cnt[rr],
                             top_k, cap, wave_max_u32(hi_seen[rr]), rowh[rr],
                             sh.rhist[RPW * wave + rr], sh.hist[wave], &kept);
          cnt[rr] = kept;
        }
      }
    }

    // ---- fetch the next key tile into registers (stored to LDS after the MFMA work) ----
    v4i nc0 = {0, 0, 0, 0}, nc1 = {0, 0, 0, 0};
    if (it + 1 < n_iter) load_tile(it + 1, nc0, nc1);

    const uint8_t* tile = sh.ktile[buf] + kh * BK * 128;
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const v8i a = frag_from_tile(tile, 16 * f + c16, g);
      float acc[4] = {0.f, 0.f, 0.f, 0.f};
      if (heads_here) {
        // software-pipelined: MFMA j+1 is issued before the epilogue of MFMA j
        v4f x = mfma_fp8(a, qf[0]);
#pragma unroll
        for (int j = 1; j < HPW; ++j) {
          const v4f xn = mfma_fp8(a, qf[j]);
          epi_abs(acc, x, wv[j - 1]);
          x = xn;
        }
        epi_abs(acc, x, wv[HPW - 1]);
      }
      *reinterpret_cast<v4f*>(&sh.part[buf][kh][hg][c16][16 * f + 4 * g]) =
          v4f{acc[0], acc[1], acc[2], acc[3]};
      // linear term of fragment hg of this wave's tile (all heads at once)
      if (f == hg)
        *reinterpret_cast<v4f*>(&sh.plin[buf][kh][c16][16 * f + 4 * g]) = linear_term(a, sh, lane);
    }
    if (it + 1 < n_iter) store_tile(buf ^ 1, nc0, nc1);
    __syncthreads();

    // ---- this wave's rows: I = (sum_j w_j x_j + sum_j w_j |x_j|) / 2 = sum_j w_j ReLU(x_j);
    // causal mask, threshold filter, ordered append.  All LDS reads are issued first. ----
    float scv[RPW][2];
#pragma unroll
    for (int rr = 0; rr < RPW; ++rr) {
      const int r = RPW * wave + rr;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const float ab = ((sh.part[buf][half][0][r][lane] + sh.part[buf][half][1][r][lane]) +
                          sh.part[buf][half][2][r][lane]) + sh.part[buf][half][3][r][lane];
        scv[rr][half] = 0.5f * (sh.plin[buf][half][r][lane] + ab);
      }
    }
#pragma unroll
    for (int rr = 0; rr < RPW; ++rr) {
      const int r = RPW * wave + rr;
      const int q = q0 + r;
      const int t = t_own[rr];
      if (q >= n_q || it * BK2 > t) continue;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int s = it * BK2 + half * BK + lane;
        const float sc = scv[rr][half];
        const bool pass = (s <= t) && (sc > thr[rr]);
        const uint64_t m = wave_ballot(pass);
        if (m != 0ull) {
          if (pass) {
            const u32 key = ord_key(sc);
            hi_seen[rr] = max(hi_seen[rr], key);
            const int p = cnt[rr] + lanes_below(m);
            cand_score[(size_t)q * cap + p] = (sc == 0.f) ? 0.f : sc;
            cand_pos[(size_t)q * cap + p] = s;
            if (rowh[rr].valid) atomicAdd(&sh.rhist[r][hbin(key, rowh[rr])], 1u);
          }
          cnt[rr] += __builtin_popcountll(m);
        }
      }
    }
    // flag rows that could overflow in the next filter; they are cut after the next barrier
    bool full = false;
#pragma unroll
    for (int rr = 0; rr < RPW; ++rr)
      full |= (q0 + RPW * wave + rr < n_q) && cnt[rr] + BK2 > cap && (it + 1) * BK2 <= t_own[rr];
    if (lane == 0) sh.full[it & 1][wave] = full ? 1 : 0;
  }

  // ---- final exact selection of this wave's rows ----
#pragma unroll
  for (int rr = 0; rr < RPW; ++rr) {
    const int q = q0 + RPW * wave + rr;
    if (q >= n_q) continue;
    const int n = cnt[rr];
    int32_t* orow = out_idx + (size_t)q * top_k;
    const float* cs = cand_score + (size_t)q * cap;
    const int32_t* ci = cand_pos + (size_t)q * cap;
    if (n <= top_k) {
      for (int i = lane; i < top_k; i += kWave) orow[i] = (i < n) ? ci[i] : -1;
    } else {
      u32 T;
      int r;
      wave_radix_select([&](int i) { return ord_key(cs[i]); }, n, top_k, sh.hist[wave], T, r);
      wave_stable_keep(
          [&](int i) { CandItem it; it.score = cs[i]; it.pos = ci[i]; it.key = ord_key(it.score); return it; },
          n, T, r, [&](const CandItem& it, int p) { if (p < top_k) orow[p] = it.pos; });
    }
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
  // room for top_k kept items plus at least two iterations of appends
  int cap = 2 * top_k + BK2;
  if (cap < top_k + 2 * BK2) cap = top_k + 2 * BK2;
  return (cap + BK2 - 1) / BK2 * BK2;
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
