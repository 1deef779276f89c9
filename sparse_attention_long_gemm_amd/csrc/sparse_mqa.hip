// Sparse MQA attention over the selected shared latent KV rows on gfx950.
//
// o[t,h] = sum_{s in S_t} softmax_s(scale * q[t,h] . kv[s]) * kv[s, :D_v]
// MQA mode: one shared KV row per token (K = the whole row, 512 latent + 64 rope dims;
// V = its first 512 dims) serves all 128 query heads (openi.cn "DeepSeek-V3.2" page, item on
// MLA run in MQA mode); only the selected entries are attended (jdon.com "DeepSeek-V3.2-Exp"
// article, paragraph on fine-grained token selection).
//
// One workgroup = one query row (all heads) x one slice of its selected rows, 8 waves.  Wave w
// owns heads 16w .. 16w+15 over all dimensions (v_mfma_f32_16x16x32_bf16): its queries stay
// in registers as the B operand of S^T = K Q^T (all 18 k-steps at DK = 576) and its fp32 output
// accumulators O^T stay in registers for the whole slice, so the waves never exchange partial
// results and every probability is computed once.  The selected rows are gathered 32 at a
// time straight from global memory into a ring of three LDS tiles (global_load_lds, 16 bytes
// per lane; two chunks' loads are in flight while one is computed, interleaved with the logit
// product); the waves meet once per chunk.  The tile is row-major with two 16-byte pad slots
// per row, which keeps both read patterns free of LDS bank conflicts and every address base +
// constant; it is the A operand of S^T = K Q^T as is, and the A operand of O^T += V^T P^T is
// read from the same tile with the transposing LDS read (ds_read_b64_tr_b16), so no
// transposed copy is stored.  With keys on the MFMA rows, each lane holds 8 keys of one head;
// the head's row max and sum need one exchange among its 4 lanes, and the probabilities
// already sit in the B-operand layout of the value product once packed to bf16 (the k slots
// of that product follow the lane's own keys).  The probabilities are formed in one pass
// against a lazily moved reference max; a chunk is redone in two passes only when one of its
// logits breaks the bound.
//
// Decode (paged) splits each sequence's selected rows over n_split workgroups; partial
// (output normalised by the split's own sum, running max, running sum) are merged by
// mqa_combine_kernel.
#include "dsa_common.hpp"
#include "dsa_kernels.hpp"

#include <mutex>
#include <type_traits>

namespace dsa {

namespace {

constexpr int NW = 8;            // waves: 16 heads each, all dimensions
constexpr int NT = NW * kWave;
constexpr int HPW = 16;          // heads per wave
constexpr int CH = 32;           // selected rows per chunk
constexpr int MAX_ROWS = 2048;   // selected rows per workgroup (top_k <= 2048)
constexpr int QPD = 2;           // k-steps of logit operands in flight

typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) v4s lds_v4s;

__device__ __forceinline__ v4i ld16(const void* p) { return *reinterpret_cast<const v4i*>(p); }

__device__ __forceinline__ v8bf as_v8bf(const v4i& x) {
  v8bf r;
  __builtin_memcpy(&r, &x, 16);
  return r;
}

// Wave-load jj of a wave's part of a chunk's gather is issued after logit product
// gather_slot(jj) of the chunk computed two steps earlier: evenly from the first product to
// the last but one.
template <int NKS, int GJ>
__device__ constexpr int gather_slot(int jj) {
  return GJ > 1 ? jj * (NKS > 2 ? NKS - 2 : 0) / (GJ - 1) : 0;
}
template <int NKS, int GJ>
__device__ constexpr int first_load_at(int ks) {   // first wave-load issued after product ks
  int jj = 0;
  while (jj < GJ && gather_slot<NKS, GJ>(jj) < ks) ++jj;
  return jj;
}


// Row tile of the head-split kernel: rows in entry order, two 16-byte pad slots per row.  For
// these read patterns (16 rows x one 16-byte column per lane group for the logit product, two
// 4-row x 32-byte groups per 32 lanes for the transposing value read) a stride of 74 slots
// measures free of LDS bank conflicts on gfx950 (73 slots conflicts on the logit read).
template <int DK>
struct Tile {
  static constexpr int NCH = DK / 8;
  static constexpr int SLOTS = NCH + 2;
  static constexpr int RS = 16 * SLOTS;
  static constexpr int LOADS = (CH * SLOTS + kWave - 1) / kWave;
  static constexpr int BYTES = LOADS * kWave * 16;
  static constexpr int GJ = (LOADS + NW - 1) / NW;
};

__device__ __forceinline__ v4f mfma16_bf16(const v8bf& a, const v8bf& b, const v4f& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

struct MqaShared {
  int rows[MAX_ROWS];   // physical row of each selected entry, or -1
  int last[NW];         // per wave: the last entry that is a valid row, or -1
};

// Byte offset, inside its KV row, of the 16-byte slot that this lane fills in wave-load jj of
// its wave's part of a chunk's gather (wave-load j = wave + NW jj covers 64 consecutive tile
// slots, lane i filling slot 64j + i), or 0 for a pad slot or a slot past the tile (those
// load the start of a row and are never read).  These depend only on the wave and lane, so
// they are computed once per workgroup.
template <int DK>
__device__ __forceinline__ void gather_plan(int wave, int lane, int (&slot_off)[Tile<DK>::GJ]) {
  using T = Tile<DK>;
#pragma unroll
  for (int jj = 0; jj < T::GJ; ++jj) {
    const int u = (wave + NW * jj) * kWave + lane;
    const int r = u / T::SLOTS;
    const int p = u - r * T::SLOTS;
    slot_off[jj] = (r < CH && p < T::NCH) ? 16 * p : 0;
  }
}

// Issue wave-loads jj0 <= jj < jj1 (compile-time constants once the caller's loop is unrolled)
// of this wave's part of one chunk's gather into `tile`.  `row` holds, in lane l (and l + 32),
// the physical row of entry l of the chunk or -1; each lane takes its slot's row from there.
// Entries that are not valid rows load row 0 (their keys are masked out of the softmax).  The
// load is written out
// (global_load_lds_dwordx4: 16 bytes per lane into LDS at M0 + 16 * lane) so that the compiler
// does not count it as an outstanding LDS access, which would make it wait for all LDS traffic
// wherever a tile read is consumed; its waits are the explicit ones at the end of each chunk.
template <int DK, bool NTG = false>
__device__ __forceinline__ void gather_chunk(uint8_t* tile, const uint16_t* __restrict__ kv,
                                             int row, int wave, int lane, int jj0, int jj1,
                                             const int (&slot_off)[Tile<DK>::GJ]) {
  using T = Tile<DK>;
  constexpr int GJ = T::GJ;
#pragma unroll
  for (int jj = 0; jj < GJ; ++jj) {
    if (jj < jj0 || jj >= jj1) continue;
    const int j = wave + NW * jj;
    if (GJ * NW > T::LOADS && j >= T::LOADS) break;     // wave-uniform
    const int so = slot_off[jj];
    const u32 lds = __builtin_amdgcn_readfirstlane(
        (u32)(uintptr_t)(__attribute__((address_space(3))) void*)(tile + 16 * kWave * j));
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
    if constexpr (T::SLOTS >= kWave) {
      // The 64 slots span rows rlo and rlo + 1 of the tile; lanes below `cut` fill the first.
      // Each row gets a 64-bit scalar base (row 0 for an entry that is not a valid row), and
      // the two lane ranges load in two instructions under scalar exec masks, so the address
      // work is scalar; a pad slot or a slot past the tile loads the start of its row.
      const int rlo = (j * kWave) / T::SLOTS;
      const int cut = (rlo + 1) * T::SLOTS - j * kWave;
      const int ra = __builtin_amdgcn_readlane(row, rlo < CH ? rlo : CH - 1);
      const int rb = __builtin_amdgcn_readlane(row, rlo + 1 < CH ? rlo + 1 : CH - 1);
      const uint16_t* base_a = kv + (size_t)(u32)(ra >= 0 ? ra : 0) * DK;
      const uint16_t* base_b = kv + (size_t)(u32)(rb >= 0 ? rb : 0) * DK;
      const uint64_t mask_a = cut >= kWave ? ~0ull : ((1ull << cut) - 1ull);
      uint64_t saved;
      if constexpr (NTG) {
        // non-temporal: rows of a pool far larger than the caches, read once per step
        asm volatile(
            "s_mov_b64 %[sv], exec\n\t"
            "s_and_b64 exec, %[sv], %[ma]\n\t"
            "s_mov_b32 m0, %[lds]\n\t"
            "s_nop 0\n\t"
            "global_load_lds_dwordx4 %[off], %[ba] nt\n\t"
            "s_andn2_b64 exec, %[sv], %[ma]\n\t"
            "global_load_lds_dwordx4 %[off], %[bb] nt\n\t"
            "s_mov_b64 exec, %[sv]"
            : [sv] "=&s"(saved)
            : [ma] "s"(mask_a), [lds] "s"(lds), [off] "v"(so), [ba] "s"(base_a), [bb] "s"(base_b)
            : "memory", "m0");
      } else {
        asm volatile(
            "s_mov_b64 %[sv], exec\n\t"
            "s_and_b64 exec, %[sv], %[ma]\n\t"
            "s_mov_b32 m0, %[lds]\n\t"
            "s_nop 0\n\t"
            "global_load_lds_dwordx4 %[off], %[ba]\n\t"
            "s_andn2_b64 exec, %[sv], %[ma]\n\t"
            "global_load_lds_dwordx4 %[off], %[bb]\n\t"
            "s_mov_b64 exec, %[sv]"
            : [sv] "=&s"(saved)
            : [ma] "s"(mask_a), [lds] "s"(lds), [off] "v"(so), [ba] "s"(base_a), [bb] "s"(base_b)
            : "memory", "m0");
      }
    } else {
      // short rows: several rows per wave-load, per-lane 64-bit addresses
      const int rw = __shfl(row, ((j * kWave + lane) / T::SLOTS) & (CH - 1));
      const size_t off = rw >= 0 ? (size_t)(u32)rw * DK + (u32)(so >> 1) : 0;
      asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                   :
                   : "v"(kv + off), "s"(lds)
                   : "memory", "m0");
    }
#pragma clang diagnostic pop
  }
}

// Load instructions per wave-load (two when a wave-load spans two rows of long rows).
template <int DK>
__device__ constexpr int gather_insts() { return Tile<DK>::SLOTS >= kWave ? 2 : 1; }

// Number of wave-loads of one chunk's gather that wave `wave` issues.
template <int DK>
__device__ constexpr int gather_count(int wave) {
  using T = Tile<DK>;
  int n = 0;
  for (int jj = 0; jj < T::GJ; ++jj) n += (wave + NW * jj < T::LOADS) ? 1 : 0;
  return n;
}

// s_waitcnt immediate: vmcnt = n, expcnt and lgkmcnt not waited for.
__host__ __device__ constexpr int vm_wait_imm(int n) {
  return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8);
}

// What a launch of the kernel computes.
enum MqaMode : int {
  MODE_FWD = 0,     // attention output (and lse)
  MODE_PROBS = 1,   // head-averaged probabilities of the listed entries (indexer KL target)
  MODE_BWDP = 2,    // backward, first pass: P and dS = P (dP - rowsum(dO o O)) per entry
  MODE_DQ = 3,      // backward, second pass: dQ = scale dS K over the listed rows
};

// Mode-specific operands.
struct MqaAux {
  float* probs;            // PROBS: out [n, top_k]
  const uint16_t* d_out;   // BWDP: dO [n, H, DV] bf16
  const uint16_t* o_fwd;   // BWDP: the forward's output O [n, H, DV] bf16
  uint16_t* p_ws;          // BWDP: out P [n, top_k, H] bf16
  uint16_t* ds_ws;         // BWDP: out scale * dS [n, top_k, H] bf16; DQ: in
  float* dq;               // DQ: out [n, H, DK] fp32
};

// PAGED rows read their KV rows through a page table: in decode (n_seq == 0) row qi is
// sequence qi with t = ctx[qi] - 1; in a batched prefill (n_seq > 0) row qi is sequence
// q_seq[qi] (0 when q_seq is NULL; a sequence outside [0, n_seq) attends nothing) with
// t = q_pos[qi].
// DENSE: the rows attended are all positions 0..t (dense causal attention, the baseline the
// selection is measured against); split sp takes positions [sp * rows_per_split, ...), and
// `idx` is not read.
// MODE_PROBS: no attention output; instead, for every entry of the row's index list, the main
// attention's probability summed over the heads and divided by H, from the logits recomputed
// here and the forward's log-sum-exp `lse` (read, natural log): probs[qi, e] =
// (1/H) sum_h exp(scale q_h . kv_s - lse_h), 0 for an entry that is not attended.
// MODE_BWDP: with the forward's lse (read) and output O, and the output gradient dO: per head
// and entry P = exp(scale q . kv - lse), dP = dO . v, dS = P (dP - sum_d dO O); P and scale dS
// go to the workspace in bf16, entry-major ([row][entry][head]; 0 for entries not attended).
// MODE_DQ: dQ[h] = sum_e (scale dS)[h, e] kv_e (all DK dims; instantiated with DV = DK), read
// from the workspace; fp32 output.
template <int DK, int DV, bool PAGED, bool DENSE, int MODE = MODE_FWD, bool NTG = false>
__global__ __launch_bounds__(NT, 1) void sparse_mqa_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ qpos_or_ctx,
    const int32_t* __restrict__ page_table, const int32_t* __restrict__ q_seq, int n_seq,
    int max_pages, int n_pages, int page_size, int n_kv,
    int H, int top_k, float scale_log2, int n_split, int rows_per_split,
    uint16_t* __restrict__ out, float* __restrict__ lse, uint16_t* __restrict__ part_o,
    float* __restrict__ part_ml, MqaAux aux) {
  static_assert(DK % 32 == 0 && DV % 16 == 0 && DV <= DK, "shape");
  constexpr bool PROBS = MODE == MODE_PROBS;
  constexpr bool BWDP = MODE == MODE_BWDP;
  constexpr bool DQM = MODE == MODE_DQ;
  static_assert(MODE == MODE_FWD || (!PAGED && !DENSE), "contiguous sparse rows only");
  static_assert(!DQM || DV == DK, "dQ mode covers every dimension");
  float* __restrict__ probs = aux.probs;
  using Sh = MqaShared;
  constexpr int NKS = DK / 32;           // k-steps of the S^T product
  constexpr int NDB = DV / 16;           // 16-dim blocks of the output
  constexpr int RS = Tile<DK>::RS;
  constexpr int GJ = Tile<DK>::GJ;
  __shared__ Sh sh;
  __shared__ float psh[2][CH];   // PROBS: head sums of the current / previous chunk
  __shared__ __attribute__((aligned(16))) uint8_t kt0[Tile<DK>::BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t kt1[Tile<DK>::BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t kt2[Tile<DK>::BYTES];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid & (kWave - 1);
  const int g = lane >> 4;          // lane group: k-slots 8g .. 8g+7, output rows 4g .. 4g+3
  const int h16 = lane & 15;        // head within the wave (MFMA column)
  const int c32 = lane & 31;
  const int qi = blockIdx.x;
  const int sp = blockIdx.y;
  const int head = wave * HPW + h16;
  const bool head_ok = head < H;

  int t;
  int prow = qi;   // page-table row
  if (PAGED) {
    if (n_seq > 0) {
      prow = q_seq != nullptr ? q_seq[qi] : 0;
      t = (prow >= 0 && prow < n_seq) ? qpos_or_ctx[qi] : -1;
    } else {
      t = qpos_or_ctx[qi] - 1;
    }
    if (t > max_pages * page_size - 1) t = max_pages * page_size - 1;
  } else {
    t = qpos_or_ctx[qi];
    if (t > n_kv - 1) t = n_kv - 1;
  }
  const int r0 = sp * rows_per_split;
  int r1 = r0 + rows_per_split;
  const int n_list = DENSE ? t + 1 : top_k;   // entries of the row's list
  if (r1 > n_list) r1 = n_list;
  const int nrows = r1 > r0 ? r1 - r0 : 0;

  // ---- queries: B operand of k-step ks = dims 32ks + 8g .. +8 of head `head` (issued first,
  // so that their latency overlaps the index and page-table reads below) ----
  v8bf qf[NKS];
  if constexpr (!DQM) {
    const uint16_t* qrow = q + ((size_t)qi * H + (head_ok ? head : 0)) * DK;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      v4i x = {0, 0, 0, 0};
      if (head_ok) x = ld16(qrow + 32 * ks + 8 * g);
      qf[ks] = as_v8bf(x);
    }
  }

  // ---- BWDP: the output gradient of this lane's head, as the B operand of dP^T = V dO^T
  // (the queries' layout over the first DV dims), and D = sum_d dO O of the head ----
  constexpr int NVS = DV / 32;
  v8bf dof[BWDP ? NVS : 1];
  float dlt = 0.f;
  if constexpr (BWDP) {
    static_assert(DV % 32 == 0, "dP k-steps");
    const size_t ro = ((size_t)qi * H + (head_ok ? head : 0)) * DV;
    float part = 0.f;
#pragma unroll
    for (int ks = 0; ks < NVS; ++ks) {
      v4i x = {0, 0, 0, 0}, y = {0, 0, 0, 0};
      if (head_ok) {
        x = ld16(aux.d_out + ro + 32 * ks + 8 * g);
        y = ld16(aux.o_fwd + ro + 32 * ks + 8 * g);
      }
      dof[ks] = as_v8bf(x);
      const v8bf yo = as_v8bf(y);
#pragma unroll
      for (int j = 0; j < 8; ++j) part = fmaf((float)dof[ks][j], (float)yo[j], part);
    }
    part += __shfl_xor(part, 16);
    part += __shfl_xor(part, 32);
    dlt = part;
  }

  // ---- physical row of every selected entry (-1: skipped); all index reads of a thread are
  // issued before any is used, then the page-table reads ----
  {
    constexpr int RPT = MAX_ROWS / NT;   // entries per thread
    static_assert(MAX_ROWS % NT == 0, "rows per thread");
    int sv[RPT];
#pragma unroll
    for (int k = 0; k < RPT; ++k) {
      const int i = tid + k * NT;
      if (DENSE) sv[k] = i < nrows ? r0 + i : -1;
      else sv[k] = i < nrows ? idx[(size_t)qi * top_k + r0 + i] : -1;
    }
    int pg[RPT];
#pragma unroll
    for (int k = 0; k < RPT; ++k) {
      const bool ok = sv[k] >= 0 && sv[k] <= t;
      if (PAGED) pg[k] = ok ? page_table[(size_t)prow * max_pages + sv[k] / page_size] : -1;
      else pg[k] = ok ? 0 : -1;
    }
    int last = -1;
#pragma unroll
    for (int k = 0; k < RPT; ++k) {
      const int i = tid + k * NT;
      if (i >= nrows) continue;
      int row = -1;
      if (PAGED) {
        if (pg[k] >= 0 && pg[k] < n_pages) row = pg[k] * page_size + sv[k] % page_size;
      } else if (pg[k] == 0) {
        row = sv[k];
      }
      sh.rows[i] = row;
      if (row >= 0) last = i;
    }
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) last = max(last, __shfl_xor(last, o));
    if (lane == 0) sh.last[wave] = last;
  }

  v4f o[NDB];
#pragma unroll
  for (int d = 0; d < NDB; ++d) o[d] = v4f{0.f, 0.f, 0.f, 0.f};
  float m_run = -__builtin_inff();   // per head (the 4 lanes of a head agree)
  float l_run = 0.f;                 // this lane's part of the head's sum

  int n_chunks = (nrows + CH - 1) / CH;
  auto chunk_row = [&](int cc) -> int {
    const int e = cc * CH + c32;
    const int v = sh.rows[e < MAX_ROWS ? e : MAX_ROWS - 1];
    return e < nrows ? v : -1;
  };
  // load instructions per chunk of the first waves, and of this wave
  constexpr int GW_HI = gather_count<DK>(0) * gather_insts<DK>();
  constexpr int GW_STEP = gather_insts<DK>();   // the other waves issue one wave-load fewer
  const int my_loads = gather_count<DK>(wave) * gather_insts<DK>();
  int slot_off[GJ];
  gather_plan<DK>(wave, lane, slot_off);
  if (PROBS && tid < 2 * CH) psh[tid / CH][tid % CH] = 0.f;
  __syncthreads();   // rows[] complete
  if constexpr (MODE == MODE_FWD) {
    // chunks after the last valid entry (the -1 padding of a row with fewer than top_k keys)
    // would add exactly nothing: they are not gathered or computed
    int last = -1;
#pragma unroll
    for (int v = 0; v < NW; ++v) last = max(last, sh.last[v]);
    n_chunks = (last + CH) / CH;
  }
  int row_nx = chunk_row(0);
  if (n_chunks > 0) gather_chunk<DK, NTG>(kt0, kv, row_nx, wave, lane, 0, GJ, slot_off);
  u32 vm_a = (u32)wave_ballot(row_nx >= 0);   // validity of the chunk being computed
  row_nx = chunk_row(1);
  if (n_chunks > 1) gather_chunk<DK, NTG>(kt1, kv, row_nx, wave, lane, 0, GJ, slot_off);
  u32 vm_b = (u32)wave_ballot(row_nx >= 0);   // validity of the next chunk
  row_nx = chunk_row(2);                       // rows of the chunk gathered during step 0
  // chunk 0 landed (chunk 1 may be in flight)
  if (n_chunks > 1) {
    if (my_loads == GW_HI) __builtin_amdgcn_s_waitcnt(vm_wait_imm(GW_HI));
    else __builtin_amdgcn_s_waitcnt(vm_wait_imm(GW_HI - GW_STEP));
  } else {
    __builtin_amdgcn_s_waitcnt(0);
  }
  __syncthreads();

  // per-lane byte offsets inside a tile:
  //  logit product, key block kb, k-step ks: entry 16kb + h16, dims 32ks + 8g .. +8
  //  ->  qk_off[kb] + 64 ks
  const int qk_off0 = h16 * RS + 16 * g;
  const int qk_off1 = (16 + h16) * RS + 16 * g;
  //  value read, input lane (m, q) of group g: entry 4g + m (k-slots 8g .. 8g+3; entry
  //  16 + 4g + m for k-slots 8g+4 .. 8g+7, 16 rows further), dims 16db + 4q
  const int tq = lane & 3, tm = (lane & 15) >> 2;
  const int tr_off = (4 * g + tm) * RS + 8 * tq;

  // PROBS: this lane's head's log-sum-exp in log2 units; the chunk sums are written out one
  // step later by wave 0 (the barrier at the end of each step separates the two buffers' uses)
  float lse2 = 0.f;
  if constexpr (PROBS || BWDP)
    lse2 = head_ok ? lse[(size_t)qi * H + head] * 1.4426950408889634f : 0.f;
  const float inv_h = 1.f / (float)H;
  auto flush_probs = [&](int cc) {
    if (wave == 0 && lane < CH) {
      const int e = cc * CH + lane;
      if (e < nrows) probs[(size_t)qi * top_k + r0 + e] = psh[cc & 1][lane] * inv_h;
      psh[cc & 1][lane] = 0.f;
    }
  };

  auto step = [&](const lds_u8* tile, uint8_t* gtile, int c) {
    const bool more = c + 2 < n_chunks;    // chunk c+2 is gathered during this step
    const u32 vmask = vm_a;
    if constexpr (PROBS) {
      if (c >= 1) flush_probs(c - 1);
    }

    // ---- S^T = K Q^T: 32 keys (two blocks of 16) x this wave's 16 heads ----
    v4f s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
    v4f dp0 = {0.f, 0.f, 0.f, 0.f}, dp1 = {0.f, 0.f, 0.f, 0.f};   // BWDP: dP^T
    const lds_u8* b0 = tile + qk_off0;
    const lds_u8* b1 = tile + qk_off1;
    v4i ka[QPD], kb[QPD];
    auto fetch = [&](int k) {
      ka[k % QPD] = *reinterpret_cast<const __attribute__((address_space(3))) v4i*>(b0 + 64 * k);
      kb[k % QPD] = *reinterpret_cast<const __attribute__((address_space(3))) v4i*>(b1 + 64 * k);
    };
    if constexpr (!DQM) {
#pragma unroll
      for (int ks = 0; ks < QPD && ks < NKS; ++ks) fetch(ks);
    }
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      if constexpr (!DQM) {
        const v4i a0 = ka[ks % QPD], a1 = kb[ks % QPD];
        const v8bf bq = qf[ks];
        if (ks + QPD < NKS) fetch(ks + QPD);
        s0 = mfma16_bf16(as_v8bf(a0), bq, s0);
        s1 = mfma16_bf16(as_v8bf(a1), bq, s1);
        if constexpr (BWDP) {
          if (ks < NVS) {   // the same key rows' first DV dims are V
            dp0 = mfma16_bf16(as_v8bf(a0), dof[ks < NVS ? ks : 0], dp0);
            dp1 = mfma16_bf16(as_v8bf(a1), dof[ks < NVS ? ks : 0], dp1);
          }
        }
      }
      const int j0 = first_load_at<NKS, GJ>(ks), j1 = first_load_at<NKS, GJ>(ks + 1);
      if (j0 < j1 && more) gather_chunk<DK, NTG>(gtile, kv, row_nx, wave, lane, j0, j1, slot_off);
      __builtin_amdgcn_sched_barrier(0);
    }

    if constexpr (PROBS) {
      // probabilities of this lane's 8 keys for its head, summed over the wave's 16 heads
      const u32 vmp = vmask >> (4 * g);
      float pv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float x = i < 4 ? s0[i & 3] : s1[i & 3];
        const bool ok = head_ok && ((vmp >> ((i < 4 ? 0 : 16) + (i & 3))) & 1u);
        pv[i] = ok ? __builtin_amdgcn_exp2f(fmaf(x, scale_log2, -lse2)) : 0.f;
      }
#pragma unroll
      for (int o = 1; o < 16; o <<= 1)
#pragma unroll
        for (int i = 0; i < 8; ++i) pv[i] += __shfl_xor(pv[i], o);
      if (h16 == 0) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
          atomicAdd(&psh[c & 1][(i < 4 ? 0 : 16) + 4 * g + (i & 3)], pv[i]);
      }
    } else if constexpr (BWDP) {
      // P and dS of this lane's 8 entries for its head, to the workspace (bf16, 0 for entries
      // that are not attended)
      const u32 vmp = vmask >> (4 * g);
      const float sc = scale_log2 * 0.69314718055994531f;   // the softmax scale
      const size_t wb = ((size_t)qi * top_k + r0 + c * CH) * H + head;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float x = i < 4 ? s0[i & 3] : s1[i & 3];
        const float dpv = i < 4 ? dp0[i & 3] : dp1[i & 3];
        const bool ok = head_ok && ((vmp >> ((i < 4 ? 0 : 16) + (i & 3))) & 1u);
        const float pv = ok ? __builtin_amdgcn_exp2f(fmaf(x, scale_log2, -lse2)) : 0.f;
        const float dsv = pv * (dpv - dlt) * sc;
        const int e = (i < 4 ? 0 : 16) + 4 * g + (i & 3);
        if (head_ok && c * CH + e < nrows) {
          aux.p_ws[wb + (size_t)e * H] = f32_to_bf16(pv);
          aux.ds_ws[wb + (size_t)e * H] = f32_to_bf16(dsv);
        }
      }
    } else {
    v8bf pb;
    if constexpr (DQM) {
      // dS of this lane's 8 entries (the value product's k slots follow them), from the
      // workspace; 0 past the row's entries
      const size_t wb = ((size_t)qi * top_k + r0 + c * CH) * H + (head_ok ? head : 0);
      uint16_t bits[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int e = (i < 4 ? 0 : 16) + 4 * g + (i & 3);
        bits[i] = 0;
        if (head_ok && c * CH + e < nrows) bits[i] = aux.ds_ws[wb + (size_t)e * H];
      }
      __builtin_memcpy(&pb, bits, 16);
    } else {
    // ---- online softmax: lane holds keys 4g + i (s0) and 16 + 4g + i (s1) of head h16 ----
    const u32 vml = vmask >> (4 * g);   // bit i: key 4g + i; bit 16 + i: key 16 + 4g + i
    float psum = 0.f;
    auto prob_pass = [&](float m_use, auto masked) {
      float mx = -__builtin_inff();
      psum = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float x = i < 4 ? s0[i & 3] : s1[i & 3];
        float nb = -m_use;
        if constexpr (decltype(masked)::value)
          nb = ((vml >> ((i < 4 ? 0 : 16) + (i & 3))) & 1u) ? -m_use : -__builtin_inff();
        const float y = fmaf(x, scale_log2, nb);
        mx = fmaxf(mx, y);
        const float pv = __builtin_amdgcn_exp2f(y);
        psum += pv;
        pb[i] = (__bf16)pv;
      }
      return mx;
    };
    const float over = vmask == 0xffffffffu ? prob_pass(m_run, std::false_type{})
                                            : prob_pass(m_run, std::true_type{});
    if (__ballot(!(over <= 8.f))) {
      float cmax = -__builtin_inff();
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float x = i < 4 ? s0[i & 3] : s1[i & 3];
        const float bias = ((vml >> ((i < 4 ? 0 : 16) + (i & 3))) & 1u) ? 0.f : -__builtin_inff();
        cmax = fmaxf(cmax, fmaf(x, scale_log2, bias));
      }
      cmax = fmaxf(cmax, __shfl_xor(cmax, 16));
      cmax = fmaxf(cmax, __shfl_xor(cmax, 32));
      float alpha = 1.f;
      if (cmax > m_run + 8.f) {
        alpha = m_run == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(m_run - cmax);
        m_run = cmax;
      }
      prob_pass(m_run == -__builtin_inff() ? 0.f : m_run, std::true_type{});
      l_run *= alpha;
      if (__ballot(alpha != 1.f)) {
#pragma unroll
        for (int d = 0; d < NDB; ++d) o[d] *= alpha;
      }
    }
    l_run += psum;
    }   // FWD softmax

    // ---- O^T += V^T P^T over the 32 keys, 16 dims per block (DQ: dQ^T += K^T dS^T) ----
    const lds_u8* tr_base = tile + tr_off;
    constexpr int VPD = 4;
    v4s fa[VPD], fb[VPD];
    auto vfetch = [&](int d) {
      fa[d % VPD] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(tr_base + 32 * d));
      fb[d % VPD] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(tr_base + 16 * RS + 32 * d));
    };
#pragma unroll
    for (int d = 0; d < VPD && d < NDB; ++d) vfetch(d);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int d = 0; d < NDB; ++d) {
      v8bf a;
      __builtin_memcpy(&a, &fa[d % VPD], 8);
      __builtin_memcpy(reinterpret_cast<char*>(&a) + 8, &fb[d % VPD], 8);
      if (d + VPD < NDB) vfetch(d + VPD);
      o[d] = mfma16_bf16(a, pb, o[d]);
      __builtin_amdgcn_sched_barrier(0);
    }
    }   // FWD / DQ
    vm_a = vm_b;
    vm_b = (u32)wave_ballot(row_nx >= 0);
    row_nx = chunk_row(c + 3);
    // chunk c+1 has landed: only this step's loads (chunk c+2) may still be in flight
    if (more) {
      if (my_loads == GW_HI) __builtin_amdgcn_s_waitcnt(vm_wait_imm(GW_HI));
      else __builtin_amdgcn_s_waitcnt(vm_wait_imm(GW_HI - GW_STEP));
    } else {
      __builtin_amdgcn_s_waitcnt(0);
    }
    __syncthreads();
  };

#pragma unroll 1
  for (int c = 0; c < n_chunks; c += 3) {
    step((const lds_u8*)kt0, kt2, c);
    if (c + 1 < n_chunks) step((const lds_u8*)kt1, kt0, c + 1);
    if (c + 2 < n_chunks) step((const lds_u8*)kt2, kt1, c + 2);
  }

  if constexpr (PROBS) {
    if (n_chunks > 0) flush_probs(n_chunks - 1);   // after the last step's barrier
    return;
  }
  if constexpr (BWDP) return;
  if constexpr (DQM) {
    // dQ = sum_e (scale dS) kv_e (the workspace holds dS already scaled)
    if (!head_ok) return;
    float* dqr = aux.dq + ((size_t)qi * H + head) * DK;
#pragma unroll
    for (int d = 0; d < NDB; ++d) *reinterpret_cast<v4f*>(dqr + 16 * d + 4 * g) = o[d];
    return;
  }

  // ---- epilogue: lane holds head `head`, dims 16d + 4g + i ----
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  if (!head_ok) return;
  if (n_split == 1) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    uint16_t* orow = out + ((size_t)qi * H + head) * DV;
#pragma unroll
    for (int d = 0; d < NDB; ++d) {
      uint2 v;
      v.x = pack_bf16x2(o[d][0] * inv, o[d][1] * inv);
      v.y = pack_bf16x2(o[d][2] * inv, o[d][3] * inv);
      *reinterpret_cast<uint2*>(orow + 16 * d + 4 * g) = v;
    }
    if (lse != nullptr && g == 0)
      lse[(size_t)qi * H + head] =
          l_tot > 0.f ? (m_run + log2f(l_tot)) * 0.69314718055994531f : -__builtin_inff();
  } else {
    // this split's output normalised by its own sum (bf16), merged by mqa_combine_kernel
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    uint16_t* po = part_o + (((size_t)qi * n_split + sp) * H + head) * DV;
#pragma unroll
    for (int d = 0; d < NDB; ++d) {
      uint2 v;
      v.x = pack_bf16x2(o[d][0] * inv, o[d][1] * inv);
      v.y = pack_bf16x2(o[d][2] * inv, o[d][3] * inv);
      *reinterpret_cast<uint2*>(po + 16 * d + 4 * g) = v;
    }
    if (g == 0) {
      float* pm = part_ml + (((size_t)qi * n_split + sp) * H + head) * 2;
      pm[0] = m_run;
      pm[1] = l_tot;
    }
  }
}

// Merge the n_split partial results of one (query, head): partial i holds o_i / l_i (bf16) with
// its running max m_i and sum l_i, so o = sum_i w_i (o_i / l_i) / sum_i w_i with
// w_i = exp2(m_i - M) l_i.  One workgroup per (query, head); each thread owns 4 consecutive dims
// and issues the reads of every partial before using any (one memory round trip).
// MAXS = 0: any number of partials, read in two passes (the maxima, then the weighted sum)
// with no per-partial registers.
template <int DV, int MAXS>
__global__ __launch_bounds__(DV / 4) void mqa_combine_kernel(const uint16_t* __restrict__ part_o,
                                                             const float* __restrict__ part_ml,
                                                             int H, int n_split,
                                                             uint16_t* __restrict__ out,
                                                             float* __restrict__ lse) {
  if constexpr (MAXS == 0) {
    const int qi = blockIdx.x / H;
    const int h = blockIdx.x - qi * H;
    const size_t base = (size_t)qi * n_split * H + h;
    const int d = 4 * threadIdx.x;
    float M = -__builtin_inff();
    for (int i = 0; i < n_split; ++i) M = fmaxf(M, part_ml[(base + (size_t)i * H) * 2]);
    float L = 0.f;
    v4f acc = {0.f, 0.f, 0.f, 0.f};
    if (M != -__builtin_inff()) {
#pragma unroll 4
      for (int i = 0; i < n_split; ++i) {
        const size_t b = base + (size_t)i * H;
        const float2 ml = *reinterpret_cast<const float2*>(part_ml + b * 2);
        const uint2 ov = *reinterpret_cast<const uint2*>(part_o + b * DV + d);
        const float wgt = exp2f(ml.x - M) * ml.y;
        L += wgt;
        acc[0] += wgt * bf16_to_f32((uint16_t)(ov.x & 0xffffu));
        acc[1] += wgt * bf16_to_f32((uint16_t)(ov.x >> 16));
        acc[2] += wgt * bf16_to_f32((uint16_t)(ov.y & 0xffffu));
        acc[3] += wgt * bf16_to_f32((uint16_t)(ov.y >> 16));
      }
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    uint2 o;
    o.x = pack_bf16x2(acc[0] * inv, acc[1] * inv);
    o.y = pack_bf16x2(acc[2] * inv, acc[3] * inv);
    *reinterpret_cast<uint2*>(out + ((size_t)qi * H + h) * DV + d) = o;
    if (lse != nullptr && threadIdx.x == 0)
      lse[(size_t)qi * H + h] = L > 0.f ? (M + log2f(L)) * 0.69314718055994531f : -__builtin_inff();
    return;
  } else {
  const int qi = blockIdx.x / H;
  const int h = blockIdx.x - qi * H;
  const size_t base = (size_t)qi * n_split * H + h;   // partial i lives at base + i*H
  const int d = 4 * threadIdx.x;
  float mv[MAXS], lv[MAXS];
  uint2 ov[MAXS];
#pragma unroll
  for (int i = 0; i < MAXS; ++i) {
    mv[i] = -__builtin_inff();
    lv[i] = 0.f;
    ov[i] = uint2{0u, 0u};
    if (i < n_split) {
      const size_t b = base + (size_t)i * H;
      const float2 ml = *reinterpret_cast<const float2*>(part_ml + b * 2);
      mv[i] = ml.x;
      lv[i] = ml.y;
      ov[i] = *reinterpret_cast<const uint2*>(part_o + b * DV + d);
    }
  }
  float M = -__builtin_inff();
#pragma unroll
  for (int i = 0; i < MAXS; ++i) M = fmaxf(M, mv[i]);
  float L = 0.f;
  v4f acc = {0.f, 0.f, 0.f, 0.f};
  if (M != -__builtin_inff()) {
#pragma unroll
    for (int i = 0; i < MAXS; ++i) {
      if (i >= n_split) break;
      const float wgt = exp2f(mv[i] - M) * lv[i];
      L += wgt;
      acc[0] += wgt * bf16_to_f32((uint16_t)(ov[i].x & 0xffffu));
      acc[1] += wgt * bf16_to_f32((uint16_t)(ov[i].x >> 16));
      acc[2] += wgt * bf16_to_f32((uint16_t)(ov[i].y & 0xffffu));
      acc[3] += wgt * bf16_to_f32((uint16_t)(ov[i].y >> 16));
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
}

template <int DV>
hipError_t launch_combine(const MqaArgs& a, hipStream_t stream) {
  if (a.n_split <= 4)
    hipLaunchKernelGGL((mqa_combine_kernel<DV, 4>), dim3(a.n_q * a.H), dim3(DV / 4), 0, stream,
                       a.part_o, a.part_ml, a.H, a.n_split, a.out, a.lse);
  else
    hipLaunchKernelGGL((mqa_combine_kernel<DV, 0>), dim3(a.n_q * a.H), dim3(DV / 4), 0, stream,
                       a.part_o, a.part_ml, a.H, a.n_split, a.out, a.lse);
  return hipGetLastError();
}

// Dense causal attention (every position 0..t): split over workgroups of up to MAX_ROWS
// positions, merged by the combine kernel.
template <int DK, int DV>
hipError_t launch_dense_shape(const MqaArgs& a, hipStream_t stream) {
  const float scale_log2 = a.scale * 1.4426950408889634f;
  const int rps = a.rows_per_split;
  if (a.page_table == nullptr)
    hipLaunchKernelGGL((sparse_mqa_kernel<DK, DV, false, true>), dim3(a.n_q, a.n_split),
                       dim3(NT), 0, stream, a.q, a.kv, nullptr, a.qpos_or_ctx, nullptr, nullptr,
                       0, 0, 0, 1, a.n_kv, a.H, 0, scale_log2, a.n_split, rps, a.out, a.lse,
                       a.part_o, a.part_ml, MqaAux{});
  else
    hipLaunchKernelGGL((sparse_mqa_kernel<DK, DV, true, true>), dim3(a.n_q, a.n_split),
                       dim3(NT), 0, stream, a.q, a.kv, nullptr, a.qpos_or_ctx, a.page_table,
                       nullptr, 0, a.max_pages, a.n_pages, a.page_size, 0, a.H, 0, scale_log2,
                       a.n_split, rps, a.out, a.lse, a.part_o, a.part_ml, MqaAux{});
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_split == 1) return e;
  return launch_combine<DV>(a, stream);
}

template <int DK, int DV>
hipError_t launch_shape(const MqaArgs& a, hipStream_t stream) {
  const float scale_log2 = a.scale * 1.4426950408889634f;
  if (a.page_table == nullptr) {
    hipLaunchKernelGGL((sparse_mqa_kernel<DK, DV, false, false>), dim3(a.n_q, 1), dim3(NT), 0, stream,
                       a.q, a.kv, a.idx, a.qpos_or_ctx, nullptr, nullptr, 0, 0, 0, 1, a.n_kv,
                       a.H, a.top_k, scale_log2, 1, a.top_k, a.out, a.lse, nullptr, nullptr,
                       MqaAux{});
    return hipGetLastError();
  }
  const int rps = a.rows_per_split;
  // decode (one query per sequence, no sequence map): the selected rows come from a cache
  // far larger than L2 and the Infinity Cache and are read once per step, so they are
  // gathered non-temporally (decode steps at batch 64 over contexts up to 128K: 7% faster when
  // the step follows a 512 MB write pass, unchanged when it follows the 128K prefill; the same
  // gathers in that prefill, whose 151 MB pool the Infinity Cache holds, ran 10% slower)
  if (a.n_seq == 0)
    hipLaunchKernelGGL((sparse_mqa_kernel<DK, DV, true, false, MODE_FWD, true>),
                       dim3(a.n_q, a.n_split), dim3(NT), 0, stream, a.q, a.kv, a.idx,
                       a.qpos_or_ctx, a.page_table, a.q_seq, a.n_seq, a.max_pages, a.n_pages,
                       a.page_size, 0, a.H, a.top_k, scale_log2, a.n_split, rps, a.out, a.lse,
                       a.part_o, a.part_ml, MqaAux{});
  else
    hipLaunchKernelGGL((sparse_mqa_kernel<DK, DV, true, false>), dim3(a.n_q, a.n_split),
                       dim3(NT), 0, stream, a.q, a.kv, a.idx, a.qpos_or_ctx, a.page_table,
                       a.q_seq, a.n_seq, a.max_pages, a.n_pages, a.page_size, 0, a.H, a.top_k,
                       scale_log2, a.n_split, rps, a.out, a.lse, a.part_o, a.part_ml, MqaAux{});
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_split == 1) return e;
  return launch_combine<DV>(a, stream);
}

}  // namespace

// ------------------------------------------------------------------------------------------
// Allocation-free decode: the split partials live in a static device array instead of a caller
// workspace.  Each GPU the library runs on holds its own copy (kNoAllocScratchBytes) until the
// process ends.  Host code never uses the array's name as an address: the device address of
// each GPU's copy is looked up once, with that GPU current, on the first call there.
// ------------------------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

bool mqa_shape_supported(int D_k, int D_v) {
  return (D_k == 576 && D_v == 512) || (D_k == 64 && D_v == 64) || (D_k == 96 && D_v == 64);
}

hipError_t launch_sparse_mqa(const MqaArgs& a, hipStream_t stream) {
  if (a.D_k == 576 && a.D_v == 512) return launch_shape<576, 512>(a, stream);
  if (a.D_k == 64 && a.D_v == 64) return launch_shape<64, 64>(a, stream);
  if (a.D_k == 96 && a.D_v == 64) return launch_shape<96, 64>(a, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_dense_mqa(const MqaArgs& a, hipStream_t stream) {
  if (a.D_k == 576 && a.D_v == 512) return launch_dense_shape<576, 512>(a, stream);
  if (a.D_k == 64 && a.D_v == 64) return launch_dense_shape<64, 64>(a, stream);
  if (a.D_k == 96 && a.D_v == 64) return launch_dense_shape<96, 64>(a, stream);
  return hipErrorInvalidValue;
}

int dense_rows_per_split() { return MAX_ROWS; }

// Backward, third pass: dKV.  For every listed entry e of row t (KV row s):
//   dKV[s, :] += sum_h (scale dS)[e, h] q[t, h, :] + sum_h P[e, h] dO[t, h, :DV] (0 past DV),
// i.e. per chunk of 32 entries the product C[entries x dims] = [scale dS | P] [q ; dO] with the
// 2H heads as the contraction, on bf16 MFMAs (16x16x32), added into fp32 dKV with atomics (a
// KV row is listed by many queries).  One workgroup (12 waves) per query row; wave w owns the
// output dims [16 BPW w, 16 BPW (w + 1)).  The B operands (q and dO over the wave's dims, 8
// heads per lane group) are gathered once per row and stay in registers; the A operands (8
// consecutive heads of one entry) are 16-byte loads from the entry-major workspace.  Each
// atomic instruction covers 16 consecutive dims of 4 KV rows.  The dims are split over
// gridDim.y workgroups per row (DKV_BPW blocks per wave keep the operands in registers).
constexpr int DKV_WAVES = 8;
constexpr int DKV_NT = DKV_WAVES * kWave;
constexpr int DKV_BPW = 3;                              // 16-dim blocks per wave
constexpr int DKV_BLOCKS = DKV_WAVES * DKV_BPW;         // 16-dim blocks per workgroup

template <int DK, int DV>
__global__ __launch_bounds__(DKV_NT) void mqa_dkv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ d_out,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ q_pos, int n_kv, int H,
    int top_k, const uint16_t* __restrict__ p_ws, const uint16_t* __restrict__ ds_ws,
    float* __restrict__ d_kv) {
  constexpr int NBLK = DK / 16;                                // 16-dim output blocks
  constexpr int BPW = DKV_BPW;
  constexpr int KS = 128 / 32;                                 // k-steps per part (H <= 128)
  const int qi = blockIdx.x;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid & (kWave - 1);
  const int g = lane >> 4, n16 = lane & 15;
  int t = q_pos[qi];
  if (t > n_kv - 1) t = n_kv - 1;
  const int blk0 = blockIdx.y * DKV_BLOCKS + wave * BPW;
  if (blk0 >= NBLK) return;                                    // wave-uniform
  const int nks = (H + 31) / 32;                               // k-steps actually used

  // ---- B operands: q[h, d] and dO[h, d] for d = 16 blk + n16, h = 32 ks + 8 g + j ----
  v8bf bq[BPW][KS], bo[BPW][KS];
#pragma unroll
  for (int b = 0; b < BPW; ++b) {
    const int d = 16 * (blk0 + b) + n16;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint16_t vq[8], vo[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int h = 32 * ks + 8 * g + j;
        const bool okh = ks < nks && h < H && blk0 + b < NBLK;
        vq[j] = okh ? q[((size_t)qi * H + h) * DK + d] : (uint16_t)0;
        vo[j] = (okh && d < DV) ? d_out[((size_t)qi * H + h) * DV + d] : (uint16_t)0;
      }
      __builtin_memcpy(&bq[b][ks], vq, 16);
      __builtin_memcpy(&bo[b][ks], vo, 16);
      __builtin_amdgcn_sched_barrier(0);   // 16 gathers in flight at a time, not all 128
    }
  }
  const bool heads8 = (H & 7) == 0;   // 8-head groups never straddle the row's end

  for (int c0 = 0; c0 < top_k; c0 += CH) {
    // rows of this lane's output entries 16 eb + 4 g + i (-1: not attended)
    int srow[2][4];
#pragma unroll
    for (int eb = 0; eb < 2; ++eb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = c0 + 16 * eb + 4 * g + i;
        const int sv = e < top_k ? idx[(size_t)qi * top_k + e] : -1;
        srow[eb][i] = (sv >= 0 && sv <= t) ? sv : -1;
      }
    v4f acc[BPW][2];
#pragma unroll
    for (int b = 0; b < BPW; ++b) acc[b][0] = acc[b][1] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int part = 0; part < 2; ++part) {
      const uint16_t* ws = part == 0 ? ds_ws : p_ws;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (ks >= nks) break;
        // A operands: entry 16 eb + n16, heads 32 ks + 8 g .. + 7
        v8bf a[2];
#pragma unroll
        for (int eb = 0; eb < 2; ++eb) {
          const int e = c0 + 16 * eb + n16;
          const int h0 = 32 * ks + 8 * g;
          v4i x = {0, 0, 0, 0};
          if (e < top_k && h0 < H) {
            const uint16_t* src = ws + ((size_t)qi * top_k + e) * H + h0;
            if (heads8) {
              x = *reinterpret_cast<const v4i*>(src);
            } else {
              uint16_t v[8];
#pragma unroll
              for (int j = 0; j < 8; ++j) v[j] = h0 + j < H ? src[j] : (uint16_t)0;
              __builtin_memcpy(&x, v, 16);
            }
          }
          __builtin_memcpy(&a[eb], &x, 16);
        }
#pragma unroll
        for (int b = 0; b < BPW; ++b) {
          if (part == 1 && 16 * (blk0 + b) >= DV) continue;   // no V part past DV
#pragma unroll
          for (int eb = 0; eb < 2; ++eb)
            acc[b][eb] = mfma16_bf16(a[eb], part == 0 ? bq[b][ks] : bo[b][ks], acc[b][eb]);
        }
      }
    }
    // lane holds C[entry 16 eb + 4 g + i][dim 16 blk + n16]
#pragma unroll
    for (int b = 0; b < BPW; ++b) {
      if (blk0 + b >= NBLK) continue;
      const int d = 16 * (blk0 + b) + n16;
#pragma unroll
      for (int eb = 0; eb < 2; ++eb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (srow[eb][i] >= 0) atomicAdd(&d_kv[(size_t)srow[eb][i] * DK + d], acc[b][eb][i]);
    }
  }
}

template <int DK, int DV>
hipError_t launch_backward_shape(const MqaArgs& a, const float* lse_in, const uint16_t* o_fwd,
                                 const uint16_t* d_out, uint16_t* p_ws, uint16_t* ds_ws,
                                 float* dq, float* dkv, hipStream_t stream) {
  const float scale_log2 = a.scale * 1.4426950408889634f;
  MqaAux aux{};
  aux.d_out = d_out;
  aux.o_fwd = o_fwd;
  aux.p_ws = p_ws;
  aux.ds_ws = ds_ws;
  aux.dq = dq;
  hipLaunchKernelGGL((sparse_mqa_kernel<DK, DV, false, false, MODE_BWDP>), dim3(a.n_q, 1),
                     dim3(NT), 0, stream, a.q, a.kv, a.idx, a.qpos_or_ctx, nullptr, nullptr, 0, 0,
                     0, 1, a.n_kv, a.H, a.top_k, scale_log2, 1, a.top_k, nullptr,
                     const_cast<float*>(lse_in), nullptr, nullptr, aux);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((sparse_mqa_kernel<DK, DK, false, false, MODE_DQ>), dim3(a.n_q, 1),
                     dim3(NT), 0, stream, a.q, a.kv, a.idx, a.qpos_or_ctx, nullptr, nullptr, 0, 0,
                     0, 1, a.n_kv, a.H, a.top_k, scale_log2, 1, a.top_k, nullptr, nullptr,
                     nullptr, nullptr, aux);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((mqa_dkv_kernel<DK, DV>), dim3(a.n_q, (DK / 16 + DKV_BLOCKS - 1) / DKV_BLOCKS),
                     dim3(DKV_NT), 0, stream, a.q, d_out,
                     a.idx, a.qpos_or_ctx, a.n_kv, a.H, a.top_k, p_ws, ds_ws, dkv);
  return hipGetLastError();
}

template <int DK, int DV>
hipError_t launch_probs_shape(const MqaArgs& a, const float* lse_in, float* probs,
                              hipStream_t stream) {
  const float scale_log2 = a.scale * 1.4426950408889634f;
  MqaAux aux{};
  aux.probs = probs;
  hipLaunchKernelGGL((sparse_mqa_kernel<DK, DV, false, false, MODE_PROBS>), dim3(a.n_q, 1),
                     dim3(NT), 0, stream, a.q, a.kv, a.idx, a.qpos_or_ctx, nullptr, nullptr, 0, 0,
                     0, 1, a.n_kv, a.H, a.top_k, scale_log2, 1, a.top_k, nullptr,
                     const_cast<float*>(lse_in), nullptr, nullptr, aux);
  return hipGetLastError();
}

hipError_t launch_mqa_backward(const MqaArgs& a, const float* lse_in, const uint16_t* o_fwd,
                               const uint16_t* d_out, uint16_t* p_ws, uint16_t* ds_ws,
                               float* dq, float* dkv, hipStream_t stream) {
  if (a.D_k == 576 && a.D_v == 512)
    return launch_backward_shape<576, 512>(a, lse_in, o_fwd, d_out, p_ws, ds_ws, dq, dkv, stream);
  if (a.D_k == 64 && a.D_v == 64)
    return launch_backward_shape<64, 64>(a, lse_in, o_fwd, d_out, p_ws, ds_ws, dq, dkv, stream);
  if (a.D_k == 96 && a.D_v == 64)
    return launch_backward_shape<96, 64>(a, lse_in, o_fwd, d_out, p_ws, ds_ws, dq, dkv, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_mqa_probs(const MqaArgs& a, const float* lse_in, float* probs,
                            hipStream_t stream) {
  if (a.D_k == 576) return launch_probs_shape<576, 512>(a, lse_in, probs, stream);
  if (a.D_k == 64) return launch_probs_shape<64, 64>(a, lse_in, probs, stream);
  if (a.D_k == 96) return launch_probs_shape<96, 64>(a, lse_in, probs, stream);
  return hipErrorInvalidValue;
}

}  // namespace dsa
