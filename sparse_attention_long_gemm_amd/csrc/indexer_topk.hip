// Lightning indexer + exact top-k on gfx950.
//
// Score (jdon.com "DeepSeek-V3.2-Exp" article, paragraph on the lightning indexer):
//     I[t,s] = sum_j w[t,j] * ReLU(q_I[t,j,:] . k_I[s,:]),   s <= t,   FP8 operands.
// Selection (same article, paragraph on fine-grained token selection): keep the top_k keys
// under (score desc, position asc).
//
// Prefill kernel (one contiguous sequence, or several through a paged cache)
//   One workgroup (8 waves) owns QB = 16 query rows and streams the keys 0..max(t) of its rows,
//   128 keys per step, through a double-buffered LDS key tile (16-byte chunks XOR-swizzled).
//   The waves have two roles; the two waves sharing a SIMD (w and w + 4) take one each.
//   * Scorer wave hg (0..3) holds the FP8 queries of indexer heads 16hg..16hg+15 for the 16
//     rows in registers (the B operand of v_mfma_f32_16x16x128_f8f6f4, 8 VGPRs per head) and
//     scores all 128 keys of the tile: the output lane owns one query row, so the sum over its
//     heads runs in registers.  ReLU is split as w ReLU(x) = (w x + w |x|) / 2: the |x| half
//     costs one fma per product (the abs is a free operand modifier), and the linear half is
//     a single product q_lin . k with q_lin[t] = sum_j w[t,j] q_I[t,j,:], run on bf16 MFMAs
//     with q_lin split exactly into three bf16 pieces (FP8 keys convert to bf16 exactly);
//     scorer hg computes it for 16-key fragments 2hg and 2hg+1, interleaved with its FP8
//     MFMAs.  Scorers touch only LDS and registers.
//   * Filter wave fw (0..3) owns rows 4fw..4fw+3: it issues the key-tile DMA, adds the four
//     head-group partial sums and the linear term from LDS, applies the causal mask and a
//     per-row threshold filter, and appends the surviving (score, position) items, in
//     position order, to the row's candidate list in the workspace.  Its memory latencies sit
//     beside the scorers' matrix work instead of in front of it.
//   When lists near their capacity, every row past half of its slack is cut at the next step
//   (all 8 waves, 2 rows each, with the rows' state passed through LDS) to a threshold that
//   is at most its top_k-th score: from a per-row LDS histogram of the listed scores when
//   that leaves enough room, else by an exact radix select (dsa_select.hpp).  Only keys
//   scoring strictly above the row's threshold can enter afterwards (a later key with an equal
//   score has a higher position, so it would lose the tie).  A last exact select per row
//   writes the sorted top_k positions.  No n_q x L score matrix is ever stored.
//
// Decode kernels (paged cache, one query per sequence)
//   indexer_logits_paged: persistent waves, each streaming an equal share of all rows' keys
//   (units of 32 positions) through the page table into its own LDS ring; the A operand is the
//   query's 64 heads (4 fragments of 16), the B operand 16 keys from the ring, so the output
//   lane owns one key and 4 heads; heads are summed in registers and across the 4 lane groups.
//   Scores go to the workspace (4 bytes per key against 128 bytes of key read; staged in LDS
//   and written in bursts of 32 units) and into a per-row histogram of their top 12 order-key
//   bits.  The histogram locates the
//   bin holding the top_k-th score; one pass over the scores, spread over many workgroups
//   (dec_collect), lists every key above that bin and every key inside it; dec_finish picks
//   the missing keys exactly among the latter and writes the row in position order.
#include "dsa_common.hpp"
#include "dsa_kernels.hpp"
#include "dsa_select.hpp"

namespace dsa {

namespace {

constexpr int QB = 16;         // query rows per workgroup
constexpr int NWAVE = 8;       // 4 scorer waves (head groups) + 4 filter waves
constexpr int NSC = 4;         // scorer waves
constexpr int NFW = NWAVE - NSC;   // filter waves
constexpr int NT = NWAVE * kWave;
constexpr int BK = 64;         // keys per filter lane pass (one key per lane)
constexpr int BK2 = 2 * BK;    // keys per step (one key tile)
constexpr int NFRAG = BK2 / 16;    // 16-key MFMA fragments per key tile
constexpr int HPW = 16;        // indexer heads per scorer wave
constexpr int PSTR = BK2 + 4;  // padded LDS row stride (floats) of the partial scores
constexpr int RPF = QB / NFW;  // query rows owned by each filter wave
constexpr int RPW = QB / NWAVE;  // rows each wave cuts and selects

__device__ __forceinline__ v4i load16(const uint8_t* p) { return *reinterpret_cast<const v4i*>(p); }

// The 32 bytes of an FP8 row of d_I bytes (d_I a multiple of 16) that lane group g feeds to a
// 128-deep FP8 MFMA: 16-byte chunks g and g + 4, i.e. dims [16g, 16g+16) and [64+16g, 80+16g),
// zero past d_I.  Any split of the 128 dims over lanes gives the same dot products as long as
// both operands use it; this one lets a 16-key operand read from a 128-byte-row LDS tile hit
// every bank once per pair of key rows.
__device__ __forceinline__ v8i load_row32(const uint8_t* row, int g, int d_I, bool ok) {
  v4i lo = {0, 0, 0, 0}, hi = {0, 0, 0, 0};
  if (ok) {
    if (16 * g < d_I) lo = load16(row + 16 * g);
    if (16 * g + 64 < d_I) hi = load16(row + 16 * g + 64);
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

// A row's selection state, published by its filter wave for a cut step and the final select.
struct RowState {
  int cnt;      // listed candidates
  float thr;    // strict threshold of the filter
  u32 hi;       // largest listed order key
  u32 lo_seen;  // smallest order key ever listed (the list's smallest until its first cut)
  u32 lo;       // row histogram: range start, bin width (log2), valid
  int shift;
  int valid;
  int t;        // last candidate position in the current segment (-1: none)
};

struct PrefillShared {
  float part[2][NSC][QB][PSTR];   // [buffer][head group][row][key]: sum w|x| of 16 heads
  float plin[2][QB][PSTR];        // [buffer][row][key]: sum w x (all heads)
  alignas(16) uint8_t ktile[2][BK2 * 128];  // [buffer][key][128 B], 16 B chunks XOR-swizzled
  alignas(16) __bf16 qlin[3][4][kWave][8];  // [bf16 piece][k-step][lane][8]: B operand of
                                            // the linear term (stored element-wise)
  u32 hist[NWAVE][256];           // per-wave radix histograms
  u32 rhist[QB][256];             // per-row histogram of the listed scores (see RowHist)
  RowState rs[QB];
  int full[2][NFW];               // [step parity][filter wave]: a row of the wave is near full
  int seg_seq[QB];                // paged: each row's sequence until its segment ran, then -1
  int seg_t[QB];                  // paged: each row's last candidate position
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

__device__ __forceinline__ u32 wave_min_u32(u32 v) {
  for (int o = 32; o >= 1; o >>= 1) v = min(v, (u32)__shfl_xor((int)v, o));
  return v;
}

// Keep, in place and in order, the listed items whose order key is > T, and (TIES) the first
// r items equal to T in list order: the histogram cut (T one below a bin edge, no ties), the
// exact cut and the final select.  Scores cs and positions ci of n items (rows 16-byte aligned)
// are read 4 consecutive items per lane with 16-byte loads (clamped to the last aligned quad,
// so no read leaves the row's items), all 16 items of a lane in a batch before any is written;
// an item's new slot is below its old one, so the writes never reach an unread item.  An
// item's slot (and a tied item's rank) counts the kept (tied) items before it: those of lower
// lanes (one ballot per quad slot) and those earlier in its own quad.  emit(item, slot) writes
// it.  Returns the kept count.
template <bool TIES, class Emit>
__device__ int wave_keep_quads(const float* cs, const int32_t* ci, int n, u32 T, int r, Emit emit) {
  const int lane = threadIdx.x & (kWave - 1);
  constexpr int V = kSelU / 4;
  const int last = (n - 1) & ~3;
  int out = 0, ties = 0;
  for (int base = 0; base < n; base += kWave * kSelU) {
    v4f f[V];
    v4i pq[V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int i0 = min(base + 256 * v + 4 * lane, last);
      f[v] = *reinterpret_cast<const v4f*>(cs + i0);
      pq[v] = *reinterpret_cast<const v4i*>(ci + i0);
    }
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int i0 = base + 256 * v + 4 * lane;
      u32 key[4];
      bool keep[4];
      uint64_t b[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        key[e] = ord_key(f[v][e]);
        keep[e] = i0 + e < n && key[e] > T;
      }
      if constexpr (TIES) {
        bool eq[4];
        uint64_t beq[4];
        int rank = ties;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          eq[e] = i0 + e < n && key[e] == T;
          beq[e] = wave_ballot(eq[e]);
          rank += lanes_below(beq[e]);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          keep[e] = keep[e] || (eq[e] && rank < r);
          rank += eq[e] ? 1 : 0;
          ties += __builtin_popcountll(beq[e]);
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) b[e] = wave_ballot(keep[e]);
      int at = out;
#pragma unroll
      for (int e = 0; e < 4; ++e) at += lanes_below(b[e]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (keep[e]) {
          CandItem it;
          it.key = key[e];
          it.score = f[v][e];
          it.pos = pq[v][e];
          emit(it, at);
        }
        at += keep[e] ? 1 : 0;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) out += __builtin_popcountll(b[e]);
    }
  }
  return out;
}

// Cut a row's candidate list (n > top_k items in position order) in place.  Any threshold that
// is at most the top_k-th best key seen so far is valid: a later key must beat it strictly to
// enter (a later key with an equal score has a higher position, so it loses every tie).
//  * Histogram cut: the lower edge T of the highest bin b whose suffix count reaches top_k;
//    keeps every key >= T.  The row's histogram serves (one pass); a row's first cut, which has
//    none yet, counts the listed keys over their range [lo_seen, hi_seen] (tracked by the
//    filter wave) in the wave's scratch histogram (one more pass).  Used when b > 0 and the
//    survivors leave room for two more iterations of appends.
//  * Exact cut (radix select): keeps exactly the top_k; used otherwise (scores piled into one
//    bin, e.g. massive ties).
// Both rebuild the row histogram over [T, hi_seen] from the survivors.  Returns the new
// threshold score; *n_out receives the survivor count.
__device__ float wave_cut(float* cs, int32_t* ci, int n, int top_k, int cap, u32 lo_seen,
                          u32 hi_seen, RowHist& h, u32* rh, u32* hist, int* n_out) {
  const int lane = threadIdx.x & (kWave - 1);
  u32 T = 0u;
  bool exact = true;
  // the histogram the threshold bin is chosen from: the row's own, or (first cut, when the
  // row has none yet) one built here over the listed keys' range in this wave's scratch
  RowHist hs = h;
  const u32* hsrc = rh;
  if (!h.valid) {
    // before its first cut a row's list holds every key appended to it, so the smallest and
    // largest listed keys are the ones its filter wave tracked
    const ScoreKeys ld{cs, n};
    hrange(hs, lo_seen, hi_seen);
#pragma unroll
    for (int b = 0; b < 4; ++b) hist[4 * lane + b] = 0u;
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    for (int base = 0; base < n; base += kWave * kSelU) {
      u32 kk[kSelU];
      bool in[kSelU];
      ld(base, kk, in);
#pragma unroll
      for (int u = 0; u < kSelU; ++u)
        if (in[u]) atomicAdd(&hist[hbin(kk[u], hs)], 1u);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    hsrc = hist;
  }
  if (hs.valid) {
    u32 c[4];
    int tot = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      c[b] = hsrc[4 * lane + b];
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
      T = hs.lo + ((u32)bsel << hs.shift);
    }
  }
  int r = 0;
  if (exact) wave_radix_select_scores(cs, n, top_k, hist, T, r);
  // rebuild the histogram for the survivors over [T, hi_seen]
#pragma unroll
  for (int b = 0; b < 4; ++b) rh[4 * lane + b] = 0u;
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  hrange(h, T, hi_seen);
  int kept;
  auto emit = [&](const CandItem& it, int p) {
    if (p < cap) {
      cs[p] = it.score;
      ci[p] = it.pos;
      atomicAdd(&rh[hbin(it.key, h)], 1u);
    }
  };
  if (exact) {
    kept = wave_keep_quads<true>(cs, ci, n, T, r, emit);
  } else {
    // keep every key >= T: "key > T - 1" with no ties to resolve (T >= 1 since bin b > 0)
    kept = wave_keep_quads<false>(cs, ci, n, T - 1u, 0, emit);
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

// Key fragment (16 keys x 32 bytes per lane group) of tile row r0.. from the LDS key tile.
__device__ __forceinline__ v8i frag_from_tile(const uint8_t* tile, int r, int g) {
  const v4i lo = *reinterpret_cast<const v4i*>(tile + r * 128 + 16 * kchunk(r, g));
  const v4i hi = *reinterpret_cast<const v4i*>(tile + r * 128 + 16 * kchunk(r, g + 4));
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

// PAGED: the keys come from a paged cache [n_pages, page_size, d_I] through the page table
// row of each query row's sequence (q_seq; NULL: every row is in sequence 0), page_size a
// power of two >= 8 (2^page_shift) so that every 8-row wave-load lies in one page and the page
// index is a shift; a page-table entry outside
// [0, n_pages) reads as a page of zero keys.  A workgroup whose rows belong to several
// sequences streams each sequence's keys in turn (rows of the other sequences masked).
// Otherwise the keys are the contiguous rows k_idx [n_keys, d_I].
template <bool PAGED>
__global__ __launch_bounds__(NT, 1) void indexer_topk_prefill_kernel(
    const uint8_t* __restrict__ q_idx, const float* __restrict__ w,
    const uint8_t* __restrict__ k_idx, const int32_t* __restrict__ q_pos, int n_q, int n_keys,
    const int32_t* __restrict__ page_table, const int32_t* __restrict__ q_seq, int n_seq,
    int max_pages, int n_pages, int page_shift, int H_I, int d_I, int top_k, int cap,
    float* __restrict__ cand_score, int32_t* __restrict__ cand_pos,
    int32_t* __restrict__ out_idx) {
  __shared__ PrefillShared sh;
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const bool scorer = wave < NSC;
  const int lane = tid & (kWave - 1);
  const int g = lane >> 4;       // lane group: 16-byte chunks g, g+4 of a row; output rows 4g..4g+3
  const int c16 = lane & 15;     // output column = query row within the block
  const int q0 = blockIdx.x * QB;

  // ---- last candidate position t of each row (clamped to the keys; -1: nothing) and the
  // sequence whose keys it reads (-1 for a row with nothing to score) ----
  int t_lane = -1, seq_lane = -1;
  {
    const int q = q0 + c16;
    if (q < n_q) {
      if (PAGED) {
        const int sq = q_seq != nullptr ? q_seq[q] : 0;
        if (sq >= 0 && sq < n_seq) {
          seq_lane = sq;
          t_lane = min(q_pos[q], (max_pages << page_shift) - 1);
        }
      } else {
        seq_lane = 0;
        t_lane = min(q_pos[q], n_keys - 1);
      }
    }
    if (t_lane < 0) seq_lane = -1;
  }

  // ---- rows with at most top_k candidates keep all of them whatever their scores: when that
  // holds for every row of the block (the first top_k positions of each sequence), write
  // positions 0..t in order, -1 padded, and score nothing.  Uniform over the workgroup: every
  // wave reduces the same 16 row positions. ----
  {
    int t_all = t_lane;
    for (int o = 1; o < 16; o <<= 1) t_all = max(t_all, __shfl_xor(t_all, o));
    if (t_all < top_k) {
#pragma unroll 1
      for (int rr = 0; rr < RPW; ++rr) {
        const int r = RPW * wave + rr;
        const int t_r = __shfl(t_lane, r);   // lane r (c16 == r) holds row r's position
        const int q = q0 + r;
        if (q >= n_q) continue;
        int32_t* orow = out_idx + (size_t)q * top_k;
        for (int i = lane; i < top_k; i += kWave) orow[i] = i <= t_r ? i : -1;
      }
      return;
    }
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
      const int gg = (d >> 4) & 3, ks = 2 * (d >> 6) + ((d >> 3) & 1), jj = d & 7;
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
  for (int i = tid; i < 2 * BK2 * 128 / 16; i += NT)
    reinterpret_cast<v4i*>(&sh.ktile[0][0])[i] = v4i{0, 0, 0, 0};
  if (PAGED && tid < QB) {
    sh.seg_seq[tid] = seq_lane;   // lanes 0..15 of wave 0 hold rows 0..15 (c16 == tid)
    sh.seg_t[tid] = t_lane;
  }
  __syncthreads();   // q_lin pieces, zeroed key tiles and the segment table are in place

  // ---- the segments: the rows of one sequence at a time (contiguous keys: one segment).
  // Every wave walks the same segments (read from LDS), so all waves meet the same barriers.
  // run(t_act, t_max): t_act is row c16's last position in this segment (-1: not in it).
  const int32_t* seg_pt = page_table;   // page-table row of the sequence being streamed
  auto segments = [&](auto&& run) __attribute__((always_inline)) {
    if constexpr (!PAGED) {
      int t_max = t_lane;
      for (int o = 1; o < 16; o <<= 1) t_max = max(t_max, __shfl_xor(t_max, o));
      run(t_lane, t_max);
    } else {
#pragma unroll 1
      for (;;) {
        const int pend = sh.seg_seq[c16];
        const uint64_t left = wave_ballot(pend >= 0) & 0xffffull;   // lanes 0..15: the 16 rows
        if (left == 0ull) break;
        const int cur = __shfl(pend, __builtin_ctzll(left));
        const bool act = pend == cur;
        const int t_act = act ? sh.seg_t[c16] : -1;
        int t_max = t_act;
        for (int o = 1; o < 16; o <<= 1) t_max = max(t_max, __shfl_xor(t_max, o));
        seg_pt = page_table + (size_t)cur * max_pages;
        __syncthreads();              // every wave has read seg_seq before it changes
        if (tid < QB && act) sh.seg_seq[tid] = -1;
        run(t_act, t_max);            // (its barriers publish the change)
      }
    }
  };

  // ---- cut step (every wave, between two barriers): a filter wave flagged a row that could
  // overflow in the next filter, so every row past half of its slack is cut.  The filter waves
  // publish their rows' state, each wave cuts RPW rows, the filter waves take the new state
  // back.  kf = the key tile the coming filter reads (a row whose keys end before it is done).
  auto cut_rows = [&](int kf) __attribute__((always_inline)) {
#pragma unroll 1
    for (int rr = 0; rr < RPW; ++rr) {
      const int r = RPW * wave + rr;
      const int q = q0 + r;
      const RowState s = sh.rs[r];
      if (q >= n_q || kf * BK2 > s.t || 2 * s.cnt <= top_k + cap) continue;
      RowHist h;
      h.lo = s.lo;
      h.shift = s.shift;
      h.valid = s.valid != 0;
      int kept;
      const float thr = wave_cut(cand_score + (size_t)q * cap, cand_pos + (size_t)q * cap, s.cnt,
                                 top_k, cap, s.lo_seen, s.hi, h, sh.rhist[r], sh.hist[wave],
                                 &kept);
      if (lane == 0) {
        sh.rs[r].cnt = kept;
        sh.rs[r].thr = thr;
        sh.rs[r].lo = h.lo;
        sh.rs[r].shift = h.shift;
        sh.rs[r].valid = h.valid ? 1 : 0;
      }
    }
  };
  auto any_full = [&](int it) __attribute__((always_inline)) {
    bool f = false;
#pragma unroll
    for (int v = 0; v < NFW; ++v) f |= sh.full[(it - 1) & 1][v] != 0;
    return f;
  };

  if (scorer) {
    // ================= scorer waves: head group hg, all 128 keys of each tile =================
    const int hg = wave;
    const bool heads_here = HPW * hg < H_I;
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
    // sum_{j in group} w_j |x_j| of key tile kt (buffer kt%2) into part[kt%2][hg], and the
    // linear term q_lin . k (all heads) of fragments 2hg, 2hg+1 into plin[kt%2]: the wave
    // scores those two fragments first, with the twelve bf16 MFMAs of each interleaved into
    // its FP8 MFMAs.  The next fragment's keys are read from LDS while one is scored.
    const int hg_s = __builtin_amdgcn_readfirstlane(hg);
    auto frag_row = [&](int i) __attribute__((always_inline)) { return 16 * ((2 * hg_s + i) & (NFRAG - 1)) + c16; };
    auto compute = [&](int kt) __attribute__((always_inline)) {
      const int buf = kt & 1;
      const uint8_t* tile = sh.ktile[buf];
      v8i a_next = frag_from_tile(tile, frag_row(0), g);
#pragma unroll
      for (int i = 0; i < NFRAG; ++i) {
        const int f = (2 * hg_s + i) & (NFRAG - 1);
        const v8i a = a_next;
        if (i + 1 < NFRAG) a_next = frag_from_tile(tile, frag_row(i + 1), g);
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
        constexpr int NL = 12;   // linear-term MFMAs of a fragment: 4 k-steps x 3 q_lin pieces
        v4f la[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
        v8bf ab;
        constexpr int LA = 3;
        v8bf qlb[LA];
        if (i < 2) {
#pragma unroll
          for (int m = 0; m < LA; ++m) qlb[m] = *reinterpret_cast<const v8bf*>(&sh.qlin[m % 3][m / 3][lane][0]);
        }
        auto lin_step = [&](int m) __attribute__((always_inline)) {
          if (m % 3 == 0) ab = fp8x8_to_bf16(a[2 * (m / 3)], a[2 * (m / 3) + 1]);
          la[m & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ab, qlb[m % LA], la[m & 1], 0, 0, 0);
          if (m + LA < NL) qlb[m % LA] = *reinterpret_cast<const v8bf*>(&sh.qlin[(m + LA) % 3][(m + LA) / 3][lane][0]);
        };
        if (heads_here) {
          // software-pipelined: the epilogue of MFMA j follows the issue of MFMA j+3, so the
          // wave does not stall on each result; the barrier keeps the compiler from pulling
          // the epilogues earlier
          constexpr int PD = 3;
          v4f x[PD + 1];
#pragma unroll
          for (int j = 0; j < HPW + PD; ++j) {
            if (j < HPW) x[j % (PD + 1)] = mfma_fp8(a, qf[j]);
            if (j >= PD) epi_abs(acc, x[(j - PD) % (PD + 1)], wv[j - PD]);
            if (i < 2 && j < NL) lin_step(j);
            __builtin_amdgcn_sched_barrier(0);
          }
        } else if (i < 2) {
#pragma unroll
          for (int m = 0; m < NL; ++m) lin_step(m);
        }
        *reinterpret_cast<v4f*>(&sh.part[buf][hg][c16][16 * f + 4 * g]) =
            v4f{acc[0], acc[1], acc[2], acc[3]};
        if (i < 2) *reinterpret_cast<v4f*>(&sh.plin[buf][c16][16 * f + 4 * g]) = la[0] + la[1];
      }
    };
    segments([&](int t_act, int t_max) __attribute__((always_inline)) {
      const int n_iter = (t_max + BK2) / BK2;   // key tiles covering keys 0..t_max
      __syncthreads();                           // the previous segment is done with the tiles
      __syncthreads();                           // key tile 0 has landed
#pragma unroll 1
      for (int it = 0; it <= n_iter; ++it) {
        if (it >= 2 && any_full(it)) {
          __syncthreads();                       // the filter waves' state is published
          cut_rows(it - 1);
          __syncthreads();                       // the new state is published
        }
        if (it < n_iter) compute(it);
        __syncthreads();
      }
    });
  } else {
    // ================= filter waves: rows RPF*fw.., the key-tile DMA =================
    const int fw = wave - NSC;
    int t_own[RPF], cnt[RPF];
    float thr[RPF];
    u32 hi_seen[RPF];   // per lane: largest order key this lane ever listed for the row
    u32 lo_seen[RPF];   // per lane: smallest order key this lane ever listed for the row
    RowHist rowh[RPF];
#pragma unroll
    for (int rr = 0; rr < RPF; ++rr) {
      t_own[rr] = -1;
      cnt[rr] = 0;
      thr[rr] = -__builtin_inff();
      hi_seen[rr] = 0u;
      lo_seen[rr] = 0xffffffffu;
    }

    // ---- key tiles straight from global memory into LDS (global_load_lds, 16 bytes per
    // lane): wave-load j (0..15) of a tile fills bytes [1024 j, 1024 j + 1024), i.e. rows
    // 8j .. 8j+7; lane L fills physical chunk L % 8 of row 8j + L / 8, which holds logical
    // chunk (L % 8) ^ ((row >> 1) & 7) (the kchunk swizzle).  Filter wave fw issues wave-loads
    // fw, fw + 4, fw + 8, fw + 12, whose rows have the same (row >> 1) & 7 pattern.  Keys past
    // n_keys and chunks past d_I are not loaded: the tiles were zeroed, so chunks past d_I stay
    // zero, and a key past n_keys (whose slot may hold an older key) is past every row's t.
    // Paged keys: wave-load j's 8 rows lie in one page; the wave looks the page up (a scalar
    // load), and a page-table entry outside [0, n_pages) fills its LDS slots with zero keys
    // instead.  Rows past the page table are not loaded (past every row's t). ----
    const int dl_row = lane >> 3;
    const int dl_chunk = (lane & 7) ^ ((4 * (fw & 1) + (dl_row >> 1)) & 7);
    const bool dl_chunk_ok = 16 * dl_chunk < d_I;
    const u32 dl_off = (u32)(dl_row * d_I + 16 * dl_chunk);
    auto dma_tile = [&](int it_, int b) __attribute__((always_inline)) {
      // the pages of this wave's four wave-loads, all read before the first key DMA: read
      // between two DMAs, each page would wait for the DMA before it (one memory round trip
      // per wave-load instead of one per tile)
      int pg4[4];
      if constexpr (PAGED) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int j = __builtin_amdgcn_readfirstlane(fw) + NFW * jj;
          const int pi = __builtin_amdgcn_readfirstlane(it_ * BK2 + 8 * j) >> page_shift;
          pg4[jj] = pi < max_pages ? seg_pt[pi] : -1;
        }
      }
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int j = __builtin_amdgcn_readfirstlane(fw) + NFW * jj;   // wave-uniform
        const int s0 = __builtin_amdgcn_readfirstlane(it_ * BK2 + 8 * j);
        const uint8_t* src = k_idx + (size_t)s0 * d_I;
        bool rows_ok = true;
        if (PAGED) {
          const int pi = s0 >> page_shift;        // page_size = 2^page_shift
          const int page = __builtin_amdgcn_readfirstlane(pg4[jj]);
          const bool page_ok = page >= 0 && page < n_pages;
          if (!page_ok) {
            if (pi < max_pages && dl_chunk_ok)   // inside the table: a page of zero keys
              *reinterpret_cast<v4i*>(sh.ktile[b] + 1024 * j + 16 * lane) = v4i{0, 0, 0, 0};
            continue;
          }
          src = k_idx + (((size_t)page << page_shift) + (s0 & ((1 << page_shift) - 1))) * d_I;
        } else {
          rows_ok = s0 + dl_row < n_keys;
        }
        // 64-bit base in scalar registers: each half through readfirstlane (which returns a
        // signed int), widened as unsigned so the low half is not sign-extended
        const uint64_t bp = (uint64_t)(uintptr_t)src;
        const uint64_t base =
            ((uint64_t)(u32)__builtin_amdgcn_readfirstlane((u32)(bp >> 32)) << 32) |
            (uint64_t)(u32)__builtin_amdgcn_readfirstlane((u32)bp);
        const u32 lds = __builtin_amdgcn_readfirstlane(
            (u32)(uintptr_t)(__attribute__((address_space(3))) void*)(sh.ktile[b] + 1024 * j));
        if (dl_chunk_ok && rows_ok) {
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
          asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %2"
                       :
                       : "v"(dl_off), "s"(lds), "s"(base)
                       : "memory", "m0");
#pragma clang diagnostic pop
        }
      }
    };

    // This wave's rows over key tile `kt`: I = (sum_j w_j x_j + sum_j w_j |x_j|) / 2 =
    // sum_j w_j ReLU(x_j); causal mask, threshold filter, ordered append.  All LDS reads are
    // issued first.  Rows that could overflow in the next filter are flagged in
    // full[(kt + 1) % 2] (read at the start of the next step).
    auto filter = [&](int kt) __attribute__((always_inline)) {
      const int buf = kt & 1;
      float scv[RPF][2];
#pragma unroll
      for (int rr = 0; rr < RPF; ++rr) {
        const int r = RPF * fw + rr;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int k = BK * half + lane;
          const float ab = ((sh.part[buf][0][r][k] + sh.part[buf][1][r][k]) +
                            sh.part[buf][2][r][k]) + sh.part[buf][3][r][k];
          scv[rr][half] = 0.5f * (sh.plin[buf][r][k] + ab);
        }
      }
      // Per row, one append pass covers both halves: a lane takes its first surviving key
      // there, and a second pass (rare) takes the second half's key of lanes where both
      // survive.  Each key's slot in the list is fixed by the ballots (position order), so
      // the stores may go in any order.  The row's list is addressed from a scalar base with
      // 32-bit lane offsets.
      const int kb = kt * BK2;
#pragma unroll
      for (int rr = 0; rr < RPF; ++rr) {
        const int r = RPF * fw + rr;
        const int q = q0 + r;
        const int t = t_own[rr];
        if (q >= n_q || kb > t) continue;   // uniform
        const bool p0 = (kb + lane <= t) && (scv[rr][0] > thr[rr]);
        const bool p1 = (kb + BK + lane <= t) && (scv[rr][1] > thr[rr]);
        const uint64_t m0 = wave_ballot(p0), m1 = wave_ballot(p1);
        if ((m0 | m1) == 0ull) continue;    // uniform
        const int c0 = __builtin_popcountll(m0);
        const size_t rbase = (size_t)__builtin_amdgcn_readfirstlane(q) * cap;
        char* srow = reinterpret_cast<char*>(cand_score + rbase);
        char* prow = reinterpret_cast<char*>(cand_pos + rbase);
        auto append = [&](float sc, int p, int pos) __attribute__((always_inline)) {
          const u32 key = ord_key(sc);
          hi_seen[rr] = max(hi_seen[rr], key);
          lo_seen[rr] = min(lo_seen[rr], key);
          const u32 off = 4u * (u32)p;
          *reinterpret_cast<float*>(srow + off) = sc;
          *reinterpret_cast<int32_t*>(prow + off) = pos;
          if (rowh[rr].valid) atomicAdd(&sh.rhist[r][hbin(key, rowh[rr])], 1u);
        };
        if (p0 || p1) {
          const int l0 = lanes_below(m0), l1 = c0 + lanes_below(m1);
          append(p0 ? scv[rr][0] : scv[rr][1], cnt[rr] + (p0 ? l0 : l1), kb + (p0 ? 0 : BK) + lane);
        }
        if ((m0 & m1) != 0ull) {            // uniform
          if (p0 && p1) append(scv[rr][1], cnt[rr] + c0 + lanes_below(m1), kb + BK + lane);
        }
        cnt[rr] += c0 + __builtin_popcountll(m1);
      }
      bool full = false;
#pragma unroll
      for (int rr = 0; rr < RPF; ++rr)
        full |= (q0 + RPF * fw + rr < n_q) && cnt[rr] + BK2 > cap && (kt + 1) * BK2 <= t_own[rr];
      if (lane == 0) sh.full[(kt + 1) & 1][fw] = full ? 1 : 0;
    };

    // the rows' state, for the cut step and the final selection
    auto publish = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int rr = 0; rr < RPF; ++rr) {
        const u32 hi = wave_max_u32(hi_seen[rr]);
        const u32 lo = wave_min_u32(lo_seen[rr]);
        if (lane == 0) {
          RowState& s = sh.rs[RPF * fw + rr];
          s.cnt = cnt[rr];
          s.thr = thr[rr];
          s.hi = hi;
          s.lo_seen = lo;
          s.lo = rowh[rr].lo;
          s.shift = rowh[rr].shift;
          s.valid = rowh[rr].valid ? 1 : 0;
          s.t = t_own[rr];
        }
      }
    };
    auto take_back = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int rr = 0; rr < RPF; ++rr) {
        const RowState s = sh.rs[RPF * fw + rr];
        cnt[rr] = s.cnt;
        thr[rr] = s.thr;
        rowh[rr].lo = s.lo;
        rowh[rr].shift = s.shift;
        rowh[rr].valid = s.valid != 0;
      }
    };

    segments([&](int t_act, int t_max) __attribute__((always_inline)) {
      const int n_iter = (t_max + BK2) / BK2;   // key tiles covering keys 0..t_max
#pragma unroll
      for (int rr = 0; rr < RPF; ++rr) t_own[rr] = __shfl(t_act, RPF * fw + rr);
      __syncthreads();                           // the previous segment is done with the tiles
      if (n_iter > 0) dma_tile(0, 0);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();                           // key tile 0 has landed
#pragma unroll 1
      for (int it = 0; it <= n_iter; ++it) {
        if (it >= 2 && any_full(it)) {
          publish();
          __syncthreads();
          cut_rows(it - 1);
          __syncthreads();
          take_back();
        }
        // Loads still pending from a cut are waited for first (vmcnt(0), nothing else): the
        // compiler does not see the DMA, so a wait it placed after the DMA for one of those
        // loads would also wait for the whole tile.
        __builtin_amdgcn_s_waitcnt(0x0f70);
        if (it + 1 < n_iter) dma_tile(it + 1, (it + 1) & 1);
        if (it >= 1) filter(it - 1);
        __builtin_amdgcn_s_waitcnt(0);   // this wave's part of the next key tile has landed
        __syncthreads();
      }
    });
    publish();
  }
  __syncthreads();   // every row's final state is published

  // The top_k-th key of a row whose list has a row histogram (it was cut at least once): the
  // histogram (every listed key, over [lo, ...)) gives the bin holding it and the count of keys
  // in higher bins; one pass over the list gathers that bin's keys into this wave's part of the
  // score buffers (free now that scoring is done) and the exact select runs on those alone.
  // Returns false (the caller selects over the whole list) when the row has no histogram or
  // the bin does not fit.  T_out / r_out as for wave_radix_select.
  constexpr int kSelBuf = (int)(sizeof(sh.part) / sizeof(u32)) / NWAVE;   // keys per wave
  u32* const selbuf = reinterpret_cast<u32*>(&sh.part[0][0][0][0]) + wave * kSelBuf;
  auto final_threshold_from_hist = [&](int r, const float* cs, int n, u32& T_out,
                                       int& r_out) -> bool {
    const RowState st = sh.rs[r];
    if (st.valid == 0) return false;
    RowHist h;
    h.lo = st.lo;
    h.shift = st.shift;
    h.valid = true;
    const u32* rh = sh.rhist[r];
    u32 c[4];
    int tot = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      c[b] = rh[4 * lane + b];
      tot += (int)c[b];
    }
    int incl = tot;   // suffix sum over lanes >= this lane
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int t = __shfl_down(incl, o);
      if (lane + o < kWave) incl += t;
    }
    int bsel = -1, above = 0;
    const int excl = incl - tot;
    if (excl < top_k && top_k <= incl) {
      int cum = excl;
      for (int b = 3; b >= 0; --b) {
        if (cum + (int)c[b] >= top_k) {
          bsel = 4 * lane + b;
          above = cum;
          break;
        }
        cum += (int)c[b];
      }
    }
    const uint64_t who = wave_ballot(bsel >= 0);
    if (who == 0ull) return false;
    const int src = __builtin_ctzll(who);
    bsel = __builtin_amdgcn_readlane(bsel, src);
    above = __builtin_amdgcn_readlane(above, src);
    const int nb = (int)rh[bsel];
    if (nb > kSelBuf) return false;
    // the keys of bin bsel, in any order
    int m = 0;
    const ScoreKeys ld{cs, n};
    for (int base = 0; base < n; base += kWave * kSelU) {
      u32 kk[kSelU];
      bool in[kSelU];
      ld(base, kk, in);
#pragma unroll
      for (int u = 0; u < kSelU; ++u) {
        const bool hit = in[u] && hbin(kk[u], h) == bsel;
        const uint64_t mm = wave_ballot(hit);
        const int p = m + lanes_below(mm);
        if (hit && p < kSelBuf) selbuf[p] = kk[u];
        m += __builtin_popcountll(mm);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    if (m != nb) return false;   // (the histogram counts every listed key: not expected)
    auto key_of = [&](int i) { return selbuf[i]; };
    wave_radix_select_batched(ScalarKeys<decltype(key_of)>{key_of, m}, m, top_k - above,
                              sh.hist[wave], T_out, r_out);
    return true;
  };

  // ---- final exact selection, RPW rows per wave ----
#pragma unroll 1
  for (int rr = 0; rr < RPW; ++rr) {
    const int r = RPW * wave + rr;
    const int q = q0 + r;
    if (q >= n_q) continue;
    const int n = sh.rs[r].cnt;
    int32_t* orow = out_idx + (size_t)q * top_k;
    const float* cs = cand_score + (size_t)q * cap;
    const int32_t* ci = cand_pos + (size_t)q * cap;
    if (n <= top_k) {
      for (int i = lane; i < top_k; i += kWave) orow[i] = (i < n) ? ci[i] : -1;
    } else {
      u32 T;
      int r2;
      if (!final_threshold_from_hist(r, cs, n, T, r2))
        wave_radix_select_scores(cs, n, top_k, sh.hist[wave], T, r2);
      wave_keep_quads<true>(cs, ci, n, T, r2,
                            [&](const CandItem& it, int p) { if (p < top_k) orow[p] = it.pos; });
    }
  }
}

// ------------------------------------------------------------------------------------------
// Decode: scores of one query per sequence over its paged keys, then an exact row top-k.
//
//  1. dec_zero_kernel clears the per-row histograms and list counters.
//  2. indexer_logits_paged_kernel (persistent, equal shares of all rows' keys per wave) writes
//     the fp32 scores of keys [0, n) of each row with n > top_k (n = min(ctx, max_pages *
//     page_size); a shorter row keeps all its keys and is not scored) and
//     counts them in a per-row histogram of the top HBITS bits of their order keys (LDS
//     histogram per wave, merged with atomics).
//  3. dec_collect_kernel: the histogram gives the bin b1 that holds the top_k-th best score;
//     workgroups over slices of the row list the positions of the keys above b1 and the keys
//     inside b1 (order key, position).
//  4. dec_finish_kernel, one workgroup per row: marks the keys above b1 in an LDS bitmap over
//     positions, chooses the missing keys exactly among the candidates (their next 12 key
//     bits from a histogram, the last 8 from one more pass, then the lowest positions among
//     keys tied with the threshold) and reads the bitmap out in position order.
// ------------------------------------------------------------------------------------------
constexpr int DEC_WAVES = 4;
constexpr int DEC_NT = DEC_WAVES * kWave;
constexpr int DEC_UNIT = 32;                                 // keys per scoring unit
constexpr int DEC_UNIT_LOADS = DEC_UNIT * 128 / 1024;        // wave-loads per unit
constexpr int DEC_NBUF = 2;                                  // units in LDS per wave
constexpr int DEC_WG_PER_CU = 1;                             // scoring workgroups per CU
constexpr int SC_WAVES = 8;                                  // waves per scoring workgroup
constexpr int SC_NT = SC_WAVES * kWave;
// per-wave histogram counts are 16 bits (two bins per LDS word): flushed at least every
// HIST16_UNITS units so that no count can carry into its neighbour
constexpr int HIST16_UNITS = 65535 / DEC_UNIT - 1;
// Scores of up to SC_STAGE consecutive units of one row wait in LDS and go to memory in one
// burst (32 units: 5% faster over a B = 64 decode step than a store per unit, 8 units: no
// faster; without any score stores the kernel would be 21% faster: the score writes, not the
// waits on them, cost the time; non-temporal stores are 1.7% faster than plain ones).  With the
// rings and histograms this fills the 160 KB of LDS.
constexpr int SC_STAGE = 32;
constexpr int HBITS = 12;                                    // histogram: top 12 key bits
constexpr int NBIN = 1 << HBITS;
constexpr int SEL_NT = 1024;
constexpr int SEL_U = 16;                                    // scores per thread (collect)
constexpr int COLLECT_CHUNK = SEL_NT * SEL_U;                // scores per collect workgroup
constexpr int SEL_CAND_LDS = 9216;                           // candidates kept on chip
constexpr int SEL_BITMAP_WORDS = 8192;                       // rows up to 2^18 positions
constexpr int kMaxK = 2048;

__device__ __forceinline__ int hist_bin(u32 key) { return (int)(key >> (32 - HBITS)); }

// Workspace of the paged indexer, carved from one caller buffer (offsets 256-byte aligned).
struct DecWs {
  float* logits;     // [B, row_stride]   scores
  u32* hist;         // [B, NBIN]         histogram of the scores' top HBITS order-key bits
  int32_t* cnt;      // [B, 4]            list sizes (keys above bin b1, keys in b1), b1, keys above b1
  int32_t* above;    // [B, kMaxK]        positions of the keys above bin b1
  u32* cand_key;     // [B, row_stride]   keys in bin b1: order key and position
  int32_t* cand_pos; // [B, row_stride]
};

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

inline size_t dec_ws_layout(int B, int row_stride, DecWs* w, char* base) {
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off = align256(off + bytes); return o; };
  const size_t o_log = take((size_t)B * row_stride * 4);
  const size_t o_hist = take((size_t)B * NBIN * 4);
  const size_t o_cnt = take((size_t)B * 4 * 4);
  const size_t o_above = take((size_t)B * kMaxK * 4);
  const size_t o_ck = take((size_t)B * row_stride * 4);
  const size_t o_cp = take((size_t)B * row_stride * 4);
  if (w != nullptr) {
    w->logits = reinterpret_cast<float*>(base + o_log);
    w->hist = reinterpret_cast<u32*>(base + o_hist);
    w->cnt = reinterpret_cast<int32_t*>(base + o_cnt);
    w->above = reinterpret_cast<int32_t*>(base + o_above);
    w->cand_key = reinterpret_cast<u32*>(base + o_ck);
    w->cand_pos = reinterpret_cast<int32_t*>(base + o_cp);
  }
  return off;
}

__global__ __launch_bounds__(DEC_NT) void dec_zero_kernel(u32* __restrict__ hist,
                                                          int32_t* __restrict__ cnt) {
  const int b = blockIdx.x;
  for (int i = threadIdx.x; i < NBIN; i += DEC_NT) hist[(size_t)b * NBIN + i] = 0u;
  if (threadIdx.x < 4) cnt[4 * b + threadIdx.x] = 0;
}

// n / d for 0 <= n < 2^31 and a divisor d >= 1 fixed for a launch, by one multiply-high
// (Granlund and Montgomery, "Division by Invariant Integers using Multiplication", 1994):
// with l = ceil(log2 d) and m = floor(2^32 (2^l - d) / d) + 1, n / d = (mulhi(n, m) + n) >> l.
struct FastDiv {
  u32 m;
  u32 l;
  int d;
};

inline FastDiv make_fastdiv(int d) {
  FastDiv f;
  f.d = d;
  f.l = 0;
  while ((1ull << f.l) < (unsigned long long)d) ++f.l;
  f.m = (u32)((((1ull << 32) * ((1ull << f.l) - (unsigned long long)d)) / (unsigned long long)d) + 1);
  return f;
}

__device__ __forceinline__ int fast_div(int n, const FastDiv& f) {
  return (int)((__umulhi((u32)n, f.m) + (u32)n) >> f.l);
}

// 16 bytes of an FP8 key row, streamed once: non-temporal load.
__device__ __forceinline__ v4i load16_nt(const uint8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const v4i*>(p));
}

// Persistent streaming scorer.  The keys of all rows are cut into units of DEC_UNIT
// consecutive positions (row b has ceil(n_b / DEC_UNIT) units); every wave of the grid takes
// an equal contiguous range of the flattened unit list, so rows of very different lengths load
// the machine evenly and each wave keeps DEC_NBUF - 1 units of loads in flight for its whole
// life instead of ramping up and down with short-lived workgroups.  The keys go straight from
// memory into a per-wave LDS ring (global_load_lds, 16 bytes per lane): 8 lanes cover one
// whole 128-byte key row, so each wave-load asks the memory system for 8 full cache lines (the
// per-CU limit on outstanding requests, not their size, bounds the stream, so full-line
// requests and 8 scoring waves per CU both count).  Waves are independent: each has its own
// LDS ring and its own LDS histogram (16-bit counts) of the row it is on, flushed into the
// row's global histogram (bins it touched only) when it moves to the next row, before a count
// could overflow, and at its end.
// Unit compute: the A operand is the row's query, 64 heads (4 fragments of 16 heads x 128
// bytes, kept in registers), the B operand 16 keys (lane group g holds chunks g and g + 4
// of key c16, read from the ring), so the output lane holds 4 heads of one key; heads are
// summed in registers and across the 4 lane groups.  Keys whose page-table entry is outside
// [0, n_pages) score as a zero key.  ALIGNED: the page size is a multiple of DEC_UNIT, so a
// unit lies in one page (one uniform lookup).
template <bool ALIGNED>
__global__ __launch_bounds__(SC_NT) void indexer_logits_paged_kernel(
    const uint8_t* __restrict__ q_idx, const float* __restrict__ w,
    const uint8_t* __restrict__ k_cache, const int32_t* __restrict__ page_table,
    const int32_t* __restrict__ ctx_lens, int B, int max_pages, int n_pages, FastDiv page,
    int H_I, int d_I, int row_stride, int top_k, float* __restrict__ logits,
    u32* __restrict__ hist) {
  const int page_size = page.d;
  __shared__ u32 lh_all[SC_WAVES][NBIN / 2];   // two 16-bit bins per word
  __shared__ float stage_all[SC_WAVES][SC_STAGE * DEC_UNIT];   // scores waiting for a burst
  // ring slot of chunk c (16 bytes) of key k of a unit: 8k + (c ^ ((k >> 1) & 7)); the swizzle
  // puts the 16 keys of an operand read on distinct LDS banks
  __shared__ __attribute__((aligned(16))) uint8_t ring_all[SC_WAVES][DEC_NBUF][DEC_UNIT * 128];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid & (kWave - 1);
  const int g = lane >> 4, c16 = lane & 15;
  u32* lh = lh_all[wave];
  const bool lo_ok = 16 * g < d_I, hi_ok = 16 * g + 64 < d_I;

  // keys of row bb that are scored: none when the row has at most top_k keys (it keeps them
  // all whatever their scores; the selection writes positions 0..n-1 for it)
  auto row_len = [&](int bb) {
    const int n = min(max(ctx_lens[bb], 0), row_stride);
    return n > top_k ? n : 0;
  };

  // ---- this wave's unit range [u0, u1) of the flattened list, and the row / unit it starts in
  auto units = [&](int bb) -> long long {
    return bb < B ? (row_len(bb) + DEC_UNIT - 1) / DEC_UNIT : 0;
  };
  long long total = 0;
  for (int b0 = 0; b0 < B; b0 += kWave) {
    long long u = units(b0 + lane);
    for (int o = 32; o >= 1; o >>= 1) u += __shfl_xor(u, o);
    total += u;
  }
  const long long n_waves = (long long)gridDim.x * SC_WAVES;
  const long long gw = (long long)blockIdx.x * SC_WAVES + wave;
  const long long u0 = total * gw / n_waves, u1 = total * (gw + 1) / n_waves;
  // (the reductions above leave the same value in every lane; make that visible to the
  // compiler so the loop control and the row cursors below live in scalar registers)
  const int my_units = __builtin_amdgcn_readfirstlane((int)(u1 - u0));
  int cb = 0, cj = 0;   // row and unit of u0
  if (my_units > 0) {
    long long before = 0;
    for (int b0 = 0; b0 < B; b0 += kWave) {
      const long long mine = units(b0 + lane);
      long long incl = mine;
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        const long long t = __shfl_up(incl, o);
        if (lane >= o) incl += t;
      }
      const uint64_t hit = wave_ballot(before + incl > u0);
      if (hit != 0) {
        const int l = __builtin_ctzll(hit);
        const long long excl = __shfl(incl - mine, l);
        cb = b0 + l;
        cj = (int)(u0 - before - excl);
        break;
      }
      before += __shfl(incl, kWave - 1);
    }
  }
  cb = __builtin_amdgcn_readfirstlane(cb);
  cj = __builtin_amdgcn_readfirstlane(cj);

  // A cursor over the unit list: row b (n keys, nu units), unit j of the row.
  struct Cursor {
    int b, j, n, nu;
  };
  auto cursor_at = [&](int b, int j) {
    Cursor c;
    c.b = b;
    c.j = j;
    c.n = b < B ? row_len(b) : 0;
    c.nu = (c.n + DEC_UNIT - 1) / DEC_UNIT;
    return c;
  };
  auto advance = [&](Cursor& c) {
    if (++c.j >= c.nu) {
      c.j = 0;
      do {
        ++c.b;
        c.n = c.b < B ? row_len(c.b) : 0;
        c.nu = (c.n + DEC_UNIT - 1) / DEC_UNIT;
      } while (c.b < B && c.nu == 0);
    }
  };

  // DMA of unit (c.b, c.j) into ring buffer nb: wave-load jj fills slots 64jj .. 64jj + 63,
  // i.e. lane l brings chunk (l % 8) ^ ((k >> 1) & 7) of key k = 8jj + l / 8.  Keys outside
  // the context or on an invalid page, chunks past d_I and every lane of a unit past the
  // wave's range load 16 harmless bytes from the start of the cache (masked or zeroed at
  // use).  Returns (uniform) whether the unit's page is valid (ALIGNED only; otherwise the
  // page is looked up again per key at use).
  auto dma_unit = [&](const Cursor& c, bool live, int nb) -> bool {
    const int32_t* pt = page_table + (size_t)(live ? c.b : 0) * max_pages;
    int gpage = 0, gslot = 0;
    if (ALIGNED) {
      const int s0 = DEC_UNIT * c.j;
      const int pi = fast_div(min(s0, max(c.n - 1, 0)), page);
      gslot = s0 - pi * page_size;
      gpage = live ? pt[pi < max_pages ? pi : max_pages - 1] : 0;
    }
    const u32 lds0 = (u32)(uintptr_t)(__attribute__((address_space(3))) void*)(ring_all[wave][nb]);
    // unaligned pages: every wave-load's page entries are read before the first key DMA and
    // unconditionally (a lane outside the row reads entry 0), so that waiting for them does not
    // wait for the DMAs issued between them
    int upg[DEC_UNIT_LOADS];
    if constexpr (!ALIGNED) {
#pragma unroll
      for (int jj = 0; jj < DEC_UNIT_LOADS; ++jj) {
        const int k = 8 * jj + (lane >> 3);
        const int ch = (lane & 7) ^ ((k >> 1) & 7);
        const int s = DEC_UNIT * c.j + k;
        const bool in = live && s < c.n && 16 * ch < d_I;
        upg[jj] = pt[fast_div(in ? s : 0, page)];
      }
    }
#pragma unroll
    for (int jj = 0; jj < DEC_UNIT_LOADS; ++jj) {
      const int k = 8 * jj + (lane >> 3);
      const int ch = (lane & 7) ^ ((k >> 1) & 7);
      const int s = DEC_UNIT * c.j + k;
      const bool in = live && s < c.n && 16 * ch < d_I;
      int pg, slot;
      if (ALIGNED) {
        pg = gpage;
        slot = gslot + k;
      } else {
        const int pi = fast_div(in ? s : 0, page);
        pg = in ? upg[jj] : 0;
        slot = s - pi * page_size;
      }
      const bool ok = in && pg >= 0 && pg < n_pages;
      const uint8_t* src = k_cache + (ok ? ((size_t)pg * page_size + slot) * d_I + 16 * ch : (size_t)0);
      // written out so that the compiler does not count it as an outstanding LDS access
      // (its waits are the explicit ones before each unit's use)
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
      asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt"
                   :
                   : "v"(src), "s"(lds0 + 1024 * jj)
                   : "memory", "m0");
#pragma clang diagnostic pop
    }
    return !ALIGNED || (gpage >= 0 && gpage < n_pages);
  };

  // query heads 16hg + c16 of row qb (A operand) and the head weights of output rows 4g + i
  v8i qa[4];
  float wl[4][4];
  auto load_query = [&](int qb) {
#pragma unroll
    for (int hg = 0; hg < 4; ++hg) {
      const int h = 16 * hg + c16;
      qa[hg] = load_row32(q_idx + ((size_t)qb * H_I + (h < H_I ? h : 0)) * d_I, g, d_I, h < H_I);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int hh = 16 * hg + 4 * g + i;
        wl[hg][i] = (hh < H_I) ? w[(size_t)qb * H_I + hh] : 0.f;
      }
    }
    // wait here (once per row) so that no query load is outstanding inside the unit loop: the
    // in-order load counter would otherwise make every unit's first product wait for the
    // units still in flight behind it
    __builtin_amdgcn_s_waitcnt(0);
  };

  // this wave's histogram: cleared once, then only the touched bin range [bmin, bmax] is
  // flushed and cleared again
#pragma unroll
  for (int i = 0; i < NBIN / 2 / kWave; ++i) lh[i * kWave + lane] = 0u;
  int bmin = NBIN, bmax = -1;
  auto flush = [&](int fb) {
    int lo = bmin, hi = bmax;
    for (int o = 32; o >= 1; o >>= 1) {
      lo = min(lo, __shfl_xor(lo, o));
      hi = max(hi, __shfl_xor(hi, o));
    }
    for (int i = (lo >> 1) + lane; i <= (hi >> 1); i += kWave) {   // two bins per word
      const u32 cnt = lh[i];
      if (cnt != 0u) {
        if (cnt & 0xffffu) atomicAdd(&hist[(size_t)fb * NBIN + 2 * i], cnt & 0xffffu);
        if (cnt >> 16) atomicAdd(&hist[(size_t)fb * NBIN + 2 * i + 1], cnt >> 16);
        lh[i] = 0u;
      }
    }
    bmin = NBIN;
    bmax = -1;
  };

  // staged scores: n_stage units of row st_b (st_n keys) from position st_s0 on, written out
  // when the row changes, the stage is full, and at the end
  int n_stage = 0, st_b = 0, st_n = 0, st_s0 = 0;
  auto store_stage = [&]() {
    if (n_stage == 0) return;
    const float* stg = stage_all[wave];
    float* dst = logits + (size_t)st_b * row_stride + st_s0;
    const int cnt = min(n_stage * DEC_UNIT, st_n - st_s0);
#pragma unroll
    for (int e = 0; e < SC_STAGE * DEC_UNIT / kWave; ++e) {
      const int k = e * kWave + lane;
      if (k < cnt) __builtin_nontemporal_store(stg[k], dst + k);   // streamed: read once, later
    }
    n_stage = 0;
  };

  // lane's ring offsets of chunks g and g+4 of key c16 of fragment 0 (fragment f: + 2048 f)
  static_assert(DEC_UNIT % 16 == 0 && DEC_UNIT <= 64, "unit size");
  const int hsw = (c16 >> 1) & 7;
  const int rd0 = 128 * c16 + 16 * (g ^ hsw), rd1 = 128 * c16 + 16 * ((g + 4) ^ hsw);
  auto compute_unit = [&](const Cursor& c, int nb, bool page_ok) {
    const __attribute__((address_space(3))) uint8_t* rb =
        (const __attribute__((address_space(3))) uint8_t*)ring_all[wave][nb];
    constexpr int NF = DEC_UNIT / 16;   // 16-key fragments per unit
    float tot[NF];
    // software-pipelined: the 4 MFMAs of fragment f+1 are issued before the epilogue of f
    v4f x[4], xn[4];
    // bytes past d_I are zeroed here, at the use (short rows only: a uniform branch), so the
    // loads stay in flight until the MFMA needs them
    auto frag = [&](int f) {
      const v4i lo = *reinterpret_cast<const __attribute__((address_space(3))) v4i*>(rb + rd0 + 2048 * f);
      const v4i hi = *reinterpret_cast<const __attribute__((address_space(3))) v4i*>(rb + rd1 + 2048 * f);
      v8i k = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      if (d_I < 128) {
        if (!lo_ok) k[0] = k[1] = k[2] = k[3] = 0;
        if (!hi_ok) k[4] = k[5] = k[6] = k[7] = 0;
      }
      return k;
    };
    {
      const v8i k0 = frag(0);
#pragma unroll
      for (int hg = 0; hg < 4; ++hg) x[hg] = mfma_fp8(qa[hg], k0);  // heads 16hg+4g+i, key c16
    }
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      if (f < NF - 1) {
        const v8i kf = frag(f + 1);
#pragma unroll
        for (int hg = 0; hg < 4; ++hg) xn[hg] = mfma_fp8(qa[hg], kf);
      }
      // four independent chains (one per output row of the fragment), summed at the end
      float a4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int hg = 0; hg < 4; ++hg)
#pragma unroll
        for (int i = 0; i < 4; ++i) a4[i] = fmaf(wl[hg][i], fmaxf(x[hg][i], 0.f), a4[i]);
      float acc = (a4[0] + a4[1]) + (a4[2] + a4[3]);
      acc += __shfl_xor(acc, 16);
      acc += __shfl_xor(acc, 32);
      tot[f] = acc;
#pragma unroll
      for (int hg = 0; hg < 4; ++hg) x[hg] = xn[hg];
    }
    // lane group g keeps key 16g + c16 of the unit; a key on an invalid page scores as a zero
    // key (0)
    float v = tot[0];
#pragma unroll
    for (int f = 1; f < NF; ++f) v = g == f ? tot[f] : v;
    const int s = DEC_UNIT * c.j + lane;
    bool ok = page_ok;
    if (!ALIGNED && lane < DEC_UNIT && s < c.n) {
      const int32_t* pt = page_table + (size_t)c.b * max_pages;
      const int pg = pt[fast_div(s, page)];
      ok = pg >= 0 && pg < n_pages;
    }
    if (!ok) v = 0.f;
    if (lane < DEC_UNIT && s < c.n) {
      const float sc = v == 0.f ? 0.f : v;
      stage_all[wave][DEC_UNIT * n_stage + lane] = sc;
      const int bin = hist_bin(ord_key(sc));
      atomicAdd(&lh[bin >> 1], 1u << (16 * (bin & 1)));
      bmin = min(bmin, bin);
      bmax = max(bmax, bin);
    }
  };

  if (my_units <= 0) return;
  Cursor lc = cursor_at(cb, cj);   // next unit to load
  Cursor cc = lc;                  // next unit to compute
  load_query(cc.b);
  // DEC_NBUF ring buffers: while unit i is computed, units i+1 .. i+DEC_NBUF-1 are in flight
  bool pok[DEC_NBUF];
  int since_flush = 0;   // units counted since the last flush
#pragma unroll
  for (int r = 0; r < DEC_NBUF - 1; ++r) {
    pok[r] = dma_unit(lc, r < my_units, r);
    if (r < my_units) advance(lc);
  }
  // wait until at most the newest (DEC_NBUF - 1) units' 8 wave-loads each are outstanding
  // (vmcnt bits 3:0 and 15:14, expcnt and lgkmcnt left at their no-wait values)
  constexpr int kVm = DEC_UNIT_LOADS * (DEC_NBUF - 1);
  constexpr int kWaitUnit = (kVm & 15) | ((kVm >> 4) << 14) | (7 << 4) | (15 << 8);
#pragma unroll 1
  for (int i = 0; i < my_units; i += DEC_NBUF) {
#pragma unroll
    for (int r = 0; r < DEC_NBUF; ++r) {
      const int nb = (r + DEC_NBUF - 1) % DEC_NBUF;
      const bool live = i + r + DEC_NBUF - 1 < my_units;
      pok[nb] = dma_unit(lc, live, nb);
      if (live) advance(lc);
      if (i + r < my_units) {
        __builtin_amdgcn_s_waitcnt(kWaitUnit);   // unit i + r has landed in buffer r
        if (n_stage == 0) {
          st_b = cc.b;
          st_n = cc.n;
          st_s0 = DEC_UNIT * cc.j;
        }
        compute_unit(cc, r, pok[r]);
        ++n_stage;
        const int ob = cc.b;
        advance(cc);
        ++since_flush;
        if (cc.b != ob || n_stage == SC_STAGE) store_stage();
        if (cc.b != ob) {          // next row: flush this one, fetch the next query
          flush(ob);
          since_flush = 0;
          if (i + r + 1 < my_units) load_query(cc.b);
        } else if (since_flush >= HIST16_UNITS) {
          flush(ob);
          since_flush = 0;
        }
      }
    }
  }
  store_stage();
  flush(cc.b);   // the row of the last unit, unless already flushed (then a no-op)
}

// Order key of a stored score.  The scores in the workspace hold no -0 (the logits kernel
// stores +0 for it), so the sign-flip form agrees with ord_key.
__device__ __forceinline__ u32 stored_key(float v) {
  const u32 u = __float_as_uint(v);
  return u ^ ((u32)((int)u >> 31) | 0x80000000u);
}

// The bin of an NB-bin histogram (bins ordered like the keys) that holds the k-th largest
// key, and the number of keys in higher bins.  Every thread of the block gets the result.
// Requires at least k counted keys.  h may be in global memory or LDS.
template <int NT, int NB>
__device__ void threshold_bin(const u32* h, int k, int* sh_scan, int& bin, int& above) {
  constexpr int PER = NB >= NT ? NB / NT : 1;
  constexpr int NW = NT / kWave;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const bool has = PER * tid < NB;
  int c[PER];
  int tot = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    c[i] = has ? (int)h[PER * tid + i] : 0;
    tot += c[i];
  }
  // inclusive suffix sum over threads >= tid: within the wave, then across waves
  int incl = tot;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int t = __shfl_down(incl, o);
    if (lane + o < kWave) incl += t;
  }
  if (lane == 0) sh_scan[wave] = incl;  // wave total
  __syncthreads();
  int after = 0;
#pragma unroll
  for (int v = 0; v < NW; ++v) after += (v > wave) ? sh_scan[v] : 0;
  incl += after;
  const int excl = incl - tot;   // keys in bins above this thread's range
  __syncthreads();
  if (has && excl < k && k <= incl) {
    int cum = excl;
    for (int i = PER - 1; i >= 0; --i) {
      if (cum + c[i] >= k) {
        sh_scan[NW] = PER * tid + i;
        sh_scan[NW + 1] = cum;
        break;
      }
      cum += c[i];
    }
  }
  __syncthreads();
  bin = sh_scan[NW];
  above = sh_scan[NW + 1];
}

constexpr int SEL_TIE_LDS = 1024;   // tied candidates ranked on chip


// One pass over a slice of the row's scores (COLLECT_CHUNK per workgroup): positions of keys
// above bin b1 go to the row's `above` list, keys inside b1 (order key, position) to its
// candidate list.  List space is reserved with one atomic per workgroup and list (device-wide
// atomics on one address serialise, so they are kept few).
__global__ __launch_bounds__(SEL_NT) void dec_collect_kernel(const int32_t* __restrict__ ctx_lens,
                                                             int row_stride, int top_k,
                                                             DecWs ws) {
  constexpr int NW = SEL_NT / kWave;
  __shared__ int sh_scan[NW + 2];
  __shared__ int sh_cnt[2][NW];
  __shared__ int sh_base[2];
  const int b = blockIdx.y;
  const int n = min(max(ctx_lens[b], 0), row_stride);
  const int base = blockIdx.x * COLLECT_CHUNK;
  if (n <= top_k || base >= n) return;                       // uniform over the workgroup
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const float* row = ws.logits + (size_t)b * row_stride;
  // clamped, unconditional loads, in flight while the histogram is scanned
  float v[SEL_U];
#pragma unroll
  for (int u = 0; u < SEL_U; ++u) v[u] = row[min(base + u * SEL_NT + tid, n - 1)];
  int b1, above;
  threshold_bin<SEL_NT, NBIN>(ws.hist + (size_t)b * NBIN, top_k, sh_scan, b1, above);
  if (blockIdx.x == 0 && threadIdx.x == 0) {   // for the finish: the bin and the count above it
    ws.cnt[4 * b + 2] = b1;
    ws.cnt[4 * b + 3] = above;
  }
  u32 key[SEL_U];
  int na = 0, nc = 0;
#pragma unroll
  for (int u = 0; u < SEL_U; ++u) {
    const bool in = base + u * SEL_NT + tid < n;
    key[u] = stored_key(v[u]);
    const int bin = hist_bin(key[u]);
    na += __builtin_popcountll(wave_ballot(in && bin > b1));
    nc += __builtin_popcountll(wave_ballot(in && bin == b1));
  }
  const int wave = tid / kWave;
  if (lane == 0) {
    sh_cnt[0][wave] = na;
    sh_cnt[1][wave] = nc;
  }
  __syncthreads();
  if (tid < 2) {
    int t = 0;
#pragma unroll
    for (int v = 0; v < NW; ++v) t += sh_cnt[tid][v];
    sh_base[tid] = t > 0 ? atomicAdd(&ws.cnt[4 * b + tid], t) : 0;
  }
  __syncthreads();
  int pa = sh_base[0], pc = sh_base[1];
  for (int v = 0; v < wave; ++v) {
    pa += sh_cnt[0][v];
    pc += sh_cnt[1][v];
  }
  int32_t* al = ws.above + (size_t)b * kMaxK;
  u32* ck = ws.cand_key + (size_t)b * row_stride;
  int32_t* cp = ws.cand_pos + (size_t)b * row_stride;
#pragma unroll
  for (int u = 0; u < SEL_U; ++u) {
    const int i = base + u * SEL_NT + tid;
    const bool in = i < n;
    const int bin = hist_bin(key[u]);
    const bool ab = in && bin > b1, ca = in && bin == b1;
    const uint64_t ma = wave_ballot(ab), mc = wave_ballot(ca);
    if (ab) {
      const int q = pa + lanes_below(ma);
      if (q < kMaxK) al[q] = i;
    }
    if (ca) {
      const int q = pc + lanes_below(mc);
      ck[q] = key[u];
      cp[q] = i;
    }
    pa += __builtin_popcountll(ma);
    pc += __builtin_popcountll(mc);
  }
  (void)above;
}

struct FinShared {
  SelectShared sel;
  int scan[SEL_NT / kWave + 2];
  int n_list;
  int n_tie;
  u32 bitmap[SEL_BITMAP_WORDS];   // selected positions (rows up to 2^18 keys)
  int32_t list[kMaxK];            // selected positions of longer rows (sorted at the end)
  u32 hsub[NBIN];                 // histogram of candidate key bits 19..8, then 7..0
  int32_t tie[SEL_TIE_LDS];       // positions of the candidates equal to the threshold
  u32 ck[SEL_CAND_LDS];           // candidates staged on chip (the rest read from global)
  int32_t cp[SEL_CAND_LDS];
};

// One workgroup per row: the keys above bin b1 are selected; the missing ones are chosen
// exactly among the candidates in b1, then the row is written in position order.
__global__ __launch_bounds__(SEL_NT) void dec_finish_kernel(const int32_t* __restrict__ ctx_lens,
                                                            int row_stride, int top_k, DecWs ws,
                                                            int32_t* __restrict__ out_idx) {
  __shared__ FinShared sh;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wave = tid / kWave;
  const int n = min(max(ctx_lens[b], 0), row_stride);
  int32_t* orow = out_idx + (size_t)b * top_k;
  if (n <= top_k) {
    for (int i = tid; i < top_k; i += SEL_NT) orow[i] = (i < n) ? i : -1;
    return;
  }
  // the bin holding the top_k-th score and the count of keys above it, as the collect pass
  // found them from the row's histogram
  const int b1 = ws.cnt[4 * b + 2], above = ws.cnt[4 * b + 3];
  const int c = ws.cnt[4 * b + 1];                 // candidates in bin b1
  const bool use_bitmap = n <= SEL_BITMAP_WORDS * 32;
  const int n_words = (n + 31) / 32;
  if (use_bitmap)
    for (int i = tid; i < n_words; i += SEL_NT) sh.bitmap[i] = 0u;
  for (int i = tid; i < NBIN; i += SEL_NT) sh.hsub[i] = 0u;
  if (tid == 0) { sh.n_list = 0; sh.n_tie = 0; }
  __syncthreads();
  auto mark = [&](int pos) {
    if (use_bitmap) {
      atomicOr(&sh.bitmap[pos >> 5], 1u << (pos & 31));
    } else {
      const int p = atomicAdd(&sh.n_list, 1);
      if (p < kMaxK) sh.list[p] = pos;
    }
  };
  const u32* gck = ws.cand_key + (size_t)b * row_stride;
  const int32_t* gcp = ws.cand_pos + (size_t)b * row_stride;
  // keys above b1; the candidates staged on chip, with the histogram of their bits 19..8
  const int32_t* al = ws.above + (size_t)b * kMaxK;
  for (int i = tid; i < above; i += SEL_NT) mark(al[i]);
  for (int i = tid; i < c; i += SEL_NT) {
    const u32 k = gck[i];
    const int32_t p = gcp[i];
    if (i < SEL_CAND_LDS) {
      sh.ck[i] = k;
      sh.cp[i] = p;
    }
    atomicAdd(&sh.hsub[(k >> 8) & (NBIN - 1)], 1u);
  }
  __syncthreads();
  const int need = top_k - above;                  // >= 1 keys to take from bin b1
  auto ckey = [&](int i) -> u32 { return i < SEL_CAND_LDS ? sh.ck[i] : gck[i]; };
  auto cpos = [&](int i) -> int32_t { return i < SEL_CAND_LDS ? sh.cp[i] : gcp[i]; };

  // ---- the need-th largest candidate key T (candidates share key bits 31..20): bits 19..8
  // from the histogram, bits 7..0 from one more pass ----
  u32 T = 0u, TP = 0u;
  const bool all = c <= need;
  if (!all) {
    int d2, above2, d3, above3;
    threshold_bin<SEL_NT, NBIN>(sh.hsub, need, sh.scan, d2, above2);
    const int need2 = need - above2;
    for (int i = tid; i < 256; i += SEL_NT) sh.hsub[i] = 0u;
    __syncthreads();
    const u32 pre = ((u32)b1 << 20) | ((u32)d2 << 8);
    for (int i = tid; i < c; i += SEL_NT) {
      const u32 k = ckey(i);
      if ((k & 0xffffff00u) == pre) atomicAdd(&sh.hsub[k & 255u], 1u);
    }
    __syncthreads();
    threshold_bin<SEL_NT, 256>(sh.hsub, need2, sh.scan, d3, above3);
    T = pre | (u32)d3;
    const int r = need2 - above3;                  // keys equal to T to take (>= 1)
    const int n_eq = (int)sh.hsub[d3];
    if (n_eq > r) {
      // ties at T: take the r lowest positions
      if (n_eq <= SEL_TIE_LDS) {
        for (int i = tid; i < c; i += SEL_NT) {
          if (ckey(i) == T) sh.tie[atomicAdd(&sh.n_tie, 1)] = cpos(i);
        }
        __syncthreads();
        // the r-th lowest tied position: the one with exactly r - 1 lower ones
        for (int i = tid; i < n_eq; i += SEL_NT) {
          const int pi = sh.tie[i];
          int lower = 0;
          for (int j = 0; j < n_eq; ++j) lower += sh.tie[j] < pi ? 1 : 0;
          if (lower == r - 1) sh.scan[0] = pi;
        }
        __syncthreads();
        TP = ~(u32)sh.scan[0];
      } else {
        int r2;
        block_radix_select<SEL_NT>(
            [&](int i) { return ckey(i) == T ? ~(u32)cpos(i) : 0u; }, c, r, sh.sel, TP, r2);
      }
    }
  }
  for (int i = tid; i < c; i += SEL_NT) {
    const u32 k = ckey(i);
    if (all || k > T || (k == T && ~(u32)cpos(i) >= TP)) mark(cpos(i));
  }
  __syncthreads();

  // ---- the selected positions in ascending order ----
  if (use_bitmap) {
    constexpr int WPT = SEL_BITMAP_WORDS / SEL_NT;
    const int w0 = tid * WPT;
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < WPT; ++j) cnt += w0 + j < n_words ? __builtin_popcount(sh.bitmap[w0 + j]) : 0;
    // exclusive prefix over threads
    int incl = cnt;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int t = __shfl_up(incl, o);
      if (lane >= o) incl += t;
    }
    if (lane == kWave - 1) sh.scan[wave] = incl;
    __syncthreads();
    int off = incl - cnt;
    for (int v = 0; v < wave; ++v) off += sh.scan[v];
#pragma unroll 1
    for (int j = 0; j < WPT; ++j) {
      if (w0 + j >= n_words) break;
      u32 bits = sh.bitmap[w0 + j];
      while (bits != 0u) {
        const int bit = __builtin_ctz(bits);
        if (off < top_k) orow[off] = 32 * (w0 + j) + bit;
        ++off;
        bits &= bits - 1u;
      }
    }
  } else {
    // bitonic sort of the listed positions, padded to a power of two
    int N = 1;
    while (N < top_k) N <<= 1;
    for (int i = top_k + tid; i < N; i += SEL_NT) sh.list[i] = 0x7fffffff;
    __syncthreads();
    for (int k2 = 2; k2 <= N; k2 <<= 1) {
      for (int j = k2 >> 1; j > 0; j >>= 1) {
        for (int i = tid; i < N; i += SEL_NT) {
          const int ixj = i ^ j;
          if (ixj > i) {
            const int a = sh.list[i], d = sh.list[ixj];
            const bool up = (i & k2) == 0;
            if ((a > d) == up) {
              sh.list[i] = d;
              sh.list[ixj] = a;
            }
          }
        }
        __syncthreads();
      }
    }
    for (int i = tid; i < top_k; i += SEL_NT) orow[i] = sh.list[i];
  }
}

// ------------------------------------------------------------------------------------------
// Indexer training signal (KL to the main attention), one workgroup per query row.
// The indexer is trained to reproduce the main attention's distribution with a KL-divergence
// loss (jdon.com "DeepSeek-V3.2-Exp" article, paragraph on the indexer's warm-up; in the
// sparse stage the indexer keeps its own loss, separate from the language-model gradients).
// Over the row's index list S (entries -1 or outside [0, t] are not part of it):
//   p[e] = target[e]                       main attention, summed over heads, / H (given)
//   q[e] = softmax_e(I[t, idx[e]])         the indexer's scores of the listed keys
//   loss = sum_e p[e] (log p[e] - log q[e]),  grad[e] = d loss / d I = q[e] - p[e]
// The scores are recomputed exactly as the decode scorer forms them (fp32 fma of
// w * max(x, 0) over the FP8 MFMA head products), so on a dyadic grid they are exact.
// ------------------------------------------------------------------------------------------
constexpr int KL_NT = 256;
constexpr int KL_WAVES = KL_NT / kWave;

__global__ __launch_bounds__(KL_NT) void indexer_kl_kernel(
    const uint8_t* __restrict__ q_idx, const float* __restrict__ w,
    const uint8_t* __restrict__ k_idx, int n_keys, const int32_t* __restrict__ q_pos,
    const int32_t* __restrict__ idx, int top_k, int H_I, int d_I,
    const float* __restrict__ target, float* __restrict__ loss, float* __restrict__ grad) {
  __shared__ float sc[kMaxK];
  __shared__ float red[KL_WAVES];
  const int row = blockIdx.x;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid & (kWave - 1);
  const int g = lane >> 4, c16 = lane & 15;
  const int t = min(q_pos[row], n_keys - 1);
  // A operand: the row's heads 16 hg + c16; weights of output rows 4g + i
  v8i qa[4];
  float wl[4][4];
#pragma unroll
  for (int hg = 0; hg < 4; ++hg) {
    const int h = 16 * hg + c16;
    qa[hg] = load_row32(q_idx + ((size_t)row * H_I + (h < H_I ? h : 0)) * d_I, g, d_I, h < H_I);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hh = 16 * hg + 4 * g + i;
      wl[hg][i] = hh < H_I ? w[(size_t)row * H_I + hh] : 0.f;
    }
  }
  const int n_frag = (top_k + 15) / 16;
  for (int f = wave; f < n_frag; f += KL_WAVES) {
    const int e = 16 * f + c16;
    const int s = e < top_k ? idx[(size_t)row * top_k + e] : -1;
    const bool ok = s >= 0 && s <= t;
    const v8i kf = load_row32(k_idx + (size_t)(ok ? s : 0) * d_I, g, d_I, ok);
    float a4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int hg = 0; hg < 4; ++hg) {
      if (16 * hg >= H_I) break;
      const v4f x = mfma_fp8(qa[hg], kf);
#pragma unroll
      for (int i = 0; i < 4; ++i) a4[i] = fmaf(wl[hg][i], fmaxf(x[i], 0.f), a4[i]);
    }
    float acc = (a4[0] + a4[1]) + (a4[2] + a4[3]);
    acc += __shfl_xor(acc, 16);
    acc += __shfl_xor(acc, 32);
    if (g == 0 && e < top_k) sc[e] = ok ? acc : -__builtin_inff();
  }
  __syncthreads();
  // softmax of the listed scores
  float m = -__builtin_inff();
  for (int e = tid; e < top_k; e += KL_NT) m = fmaxf(m, sc[e]);
  m = wave_max(m);
  if (lane == 0) red[wave] = m;
  __syncthreads();
  m = red[0];
#pragma unroll
  for (int v = 1; v < KL_WAVES; ++v) m = fmaxf(m, red[v]);
  __syncthreads();
  float z = 0.f;
  if (m != -__builtin_inff())
    for (int e = tid; e < top_k; e += KL_NT) z += expf(sc[e] - m);
  for (int o = 32; o >= 1; o >>= 1) z += __shfl_xor(z, o);
  if (lane == 0) red[wave] = z;
  __syncthreads();
  z = 0.f;
#pragma unroll
  for (int v = 0; v < KL_WAVES; ++v) z += red[v];
  __syncthreads();
  const float log_z = logf(z);
  float kl = 0.f;
  for (int e = tid; e < top_k; e += KL_NT) {
    const float p = target[(size_t)row * top_k + e];
    const bool listed = sc[e] != -__builtin_inff();
    const float log_q = sc[e] - m - log_z;
    if (listed && p > 0.f) kl += p * (logf(p) - log_q);
    if (grad != nullptr)
      grad[(size_t)row * top_k + e] = listed ? expf(log_q) - p : 0.f;
  }
  for (int o = 32; o >= 1; o >>= 1) kl += __shfl_xor(kl, o);
  if (lane == 0) red[wave] = kl;
  __syncthreads();
  if (tid == 0) {
    float tot = 0.f;
#pragma unroll
    for (int v = 0; v < KL_WAVES; ++v) tot += red[v];
    loss[row] = m == -__builtin_inff() ? 0.f : tot;
  }
}

}  // namespace

// ------------------------------------------------------------------------------------------
// Host launchers
// ------------------------------------------------------------------------------------------
hipError_t launch_indexer_kl(const uint8_t* q_idx, const float* w, const uint8_t* k_idx,
                             int n_keys, const int32_t* q_pos, const int32_t* idx, int n_q,
                             int top_k, int H_I, int d_I, const float* target, float* loss,
                             float* grad, hipStream_t stream) {
  hipLaunchKernelGGL(indexer_kl_kernel, dim3(n_q), dim3(KL_NT), 0, stream, q_idx, w, k_idx,
                     n_keys, q_pos, idx, top_k, H_I, d_I, target, loss, grad);
  return hipGetLastError();
}

int indexer_cap(int top_k) {
  // room for top_k kept items plus at least two iterations of appends; 3 top_k + 128 measured
  // fastest (cuts rarer than with 2 top_k + 128, thresholds fresher than with 4 top_k + 128)
  int cap = 3 * top_k + BK2;
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
  hipLaunchKernelGGL(indexer_topk_prefill_kernel<false>, dim3(grid), dim3(NT), 0, stream, q_idx,
                     w, k_idx, q_pos, n_q, n_keys, nullptr, nullptr, 1, 1, 1, 1, H_I, d_I,
                     top_k, cap, cs, ci, out_idx);
  return hipGetLastError();
}

hipError_t launch_indexer_topk_batched(const uint8_t* q_idx, const float* w,
                                       const uint8_t* k_cache, const int32_t* page_table,
                                       int n_seq, int max_pages, int n_pages, int page_size,
                                       const int32_t* q_seq, const int32_t* q_pos, int n_q,
                                       int H_I, int d_I, int top_k, int32_t* out_idx, void* ws,
                                       hipStream_t stream) {
  const int cap = indexer_cap(top_k);
  float* cs = reinterpret_cast<float*>(ws);
  int32_t* ci = reinterpret_cast<int32_t*>(cs + (size_t)n_q * cap);
  const int grid = (n_q + QB - 1) / QB;
  int shift = 0;
  while ((1 << shift) < page_size) ++shift;
  hipLaunchKernelGGL(indexer_topk_prefill_kernel<true>, dim3(grid), dim3(NT), 0, stream, q_idx,
                     w, k_cache, q_pos, n_q, 0, page_table, q_seq, n_seq, max_pages, n_pages,
                     shift, H_I, d_I, top_k, cap, cs, ci, out_idx);
  return hipGetLastError();
}

size_t indexer_paged_ws(int B, int max_pages, int page_size) {
  return dec_ws_layout(B, max_pages * page_size, nullptr, nullptr);
}

hipError_t launch_indexer_topk_paged(const uint8_t* q_idx, const float* w, const uint8_t* k_cache,
                                     const int32_t* page_table, const int32_t* ctx_lens, int B,
                                     int max_pages, int n_pages, int page_size, int H_I, int d_I,
                                     int top_k, int32_t* out_idx, void* ws, hipStream_t stream) {
  const int row_stride = max_pages * page_size;
  DecWs d;
  dec_ws_layout(B, row_stride, &d, reinterpret_cast<char*>(ws));
  hipLaunchKernelGGL(dec_zero_kernel, dim3(B), dim3(DEC_NT), 0, stream, d.hist, d.cnt);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // persistent scorer: a fixed number of workgroups per CU of the current device
  int dev = 0, n_cu = 0;
  if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
  if ((e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess)
    return e;
  const dim3 grid(DEC_WG_PER_CU * (n_cu > 0 ? n_cu : 1));
  const FastDiv pdiv = make_fastdiv(page_size);
  if (page_size % DEC_UNIT == 0)
    hipLaunchKernelGGL(indexer_logits_paged_kernel<true>, grid, dim3(SC_NT), 0, stream, q_idx,
                       w, k_cache, page_table, ctx_lens, B, max_pages, n_pages, pdiv, H_I, d_I,
                       row_stride, top_k, d.logits, d.hist);
  else
    hipLaunchKernelGGL(indexer_logits_paged_kernel<false>, grid, dim3(SC_NT), 0, stream, q_idx,
                       w, k_cache, page_table, ctx_lens, B, max_pages, n_pages, pdiv, H_I, d_I,
                       row_stride, top_k, d.logits, d.hist);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  dim3 cgrid((row_stride + COLLECT_CHUNK - 1) / COLLECT_CHUNK, B);
  hipLaunchKernelGGL(dec_collect_kernel, cgrid, dim3(SEL_NT), 0, stream, ctx_lens, row_stride,
                     top_k, d);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(dec_finish_kernel, dim3(B), dim3(SEL_NT), 0, stream, ctx_lens, row_stride,
                     top_k, d, out_idx);
  return hipGetLastError();
}

}  // namespace dsa
