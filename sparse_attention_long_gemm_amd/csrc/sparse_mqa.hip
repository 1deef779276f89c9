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
// registers for the whole slice.  The selected rows are gathered 32 at a time straight from
// global memory into a double-buffered LDS tile (global_load_lds, 16 bytes per lane; the next
// chunk's loads are interleaved with the current chunk's logit product).  The tile is
// row-major with one 16-byte pad per row and the rows of each 16-row half permuted
// (tile_row), which puts both read patterns on disjoint LDS banks while keeping every address
// base + constant; it is the A operand of S^T = K Q^T as is, and the A operand of
// O^T += V^T P^T is read from the same tile with the transposing LDS read (ds_read_b64_tr_b16),
// so no transposed copy is stored.  The two waves of a head group add their half-dimension
// partial logits through LDS (in a fixed order, so both hold the same sums).  With keys on the
// MFMA rows, each lane owns one head, so the online-softmax row max and sum stay in the lane
// (plus one exchange with the partner lane that holds the other 16 keys), and the
// probabilities already sit in the B-operand layout of the value product once packed to bf16.
// The probabilities are formed in one pass against a lazily moved reference max; a chunk is
// redone in two passes only when one of its logits breaks the bound.
//
// Decode (paged) splits each sequence's selected rows over n_split workgroups; partial
// (unnormalised o, running max, running sum) triples are merged by mqa_combine_kernel.
#include "dsa_common.hpp"
#include "dsa_kernels.hpp"

#include <type_traits>

namespace dsa {

namespace {

constexpr int NW = 8;            // 4 head groups x 2 dimension halves
constexpr int NT = NW * kWave;
constexpr int HPW = 32;          // heads per wave
constexpr int CH = 32;           // selected rows per chunk
constexpr int MAX_ROWS = 2048;   // selected rows per workgroup (top_k <= 2048)
constexpr int QPD = 3;           // logit-product operands in flight per wave

typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) v4s lds_v4s;

__device__ __forceinline__ v4i ld16(const void* p) { return *reinterpret_cast<const v4i*>(p); }

// Workgroup barrier that orders LDS traffic only: it does not wait for outstanding global
// loads, so the asynchronous gather of the next chunk stays in flight across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ v16f mfma_bf16(const v8bf& a, const v8bf& b, const v16f& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ v8bf as_v8bf(const v4i& x) {
  v8bf r;
  __builtin_memcpy(&r, &x, 16);
  return r;
}

template <int DK>
struct Tile {
  static constexpr int NCH = DK / 8;                   // 16-byte chunks of a row
  static constexpr int SLOTS = NCH + 1;                // + one pad slot
  static constexpr int RS = 16 * SLOTS;                // row stride (bytes)
  static constexpr int LOADS = (CH * SLOTS + kWave - 1) / kWave;  // wave-loads per chunk
  static constexpr int GJ = (LOADS + NW - 1) / NW;                 // of them, per wave
  static constexpr int BYTES = LOADS * kWave * 16;
};

// Query fragments of the last QL k-steps of each wave live in LDS instead of registers (this
// keeps the 576-wide instance within 256 VGPRs per wave at 2 waves per SIMD).
template <int DK>
struct QSplit {
  static constexpr int NKS = DK / 32;
  static constexpr int QL = NKS >= 16 ? 4 : 0;
  static constexpr int QR = NKS - QL;
};

// (The two row-tile buffers are separate __shared__ objects: reads of one buffer then provably
// do not alias the asynchronous fill of the other, so no wait for that fill is inserted.)
template <int DK>
struct MqaShared {
  alignas(16) v4f sx[NW][4][kWave];          // half-dimension partial logits of each wave:
                                             // [wave][i/4][lane] holds elements 4(i/4)..+3
  alignas(16) v8bf qs[NW][QSplit<DK>::QL > 0 ? QSplit<DK>::QL : 1][kWave];  // LDS query part
  int rows[MAX_ROWS];                        // physical row of each selected entry, or -1
};

// Tile row of chunk entry e (and entry of tile row e: the map is its own inverse): inside each
// half of 16 rows, the 4x4 blocks (e = 4a + b -> 4b + a) are transposed.  The logit product
// reads entries 0..15 (16 lanes per LDS cycle) and the transposing value read reads entries
// 4a..4a+3 together; with a row stride of 73 16-byte slots, the permuted rows put both
// groups on disjoint LDS banks (unpermuted, the value read hits 2-way bank conflicts).
__host__ __device__ constexpr int tile_row(int e) {
  return (e & ~15) | ((e & 3) << 2) | ((e >> 2) & 3);
}

// Issue the gather of one chunk (32 rows) into `tile`: wave-load j covers 64 consecutive
// 16-byte tile slots; lane i fills slot 64j + i.  `row` holds, in lane l (and l + 32), the
// physical row of entry l of the chunk or -1; each lane takes its slot's row (that of entry
// tile_row(slot row)) from there.
// Pad slots, slots past the tile and entries that are not valid rows get a harmless load of
// the first 16 bytes of the KV array (their contents are never used: pad slots are never read
// and invalid keys are masked out of the softmax).
// Wave-load jj of a wave's part of the next chunk's gather is issued after logit product
// gather_slot(jj) of the current chunk: evenly from the first product to the last but one.
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

// Wave-loads jj0 <= jj < jj1 of this wave (compile-time constants at every call once the
// caller's loop is unrolled).  A chunk's gather is issued in parts spread over the logit
// product of the previous chunk, so that the CU's outstanding-miss capacity is not exceeded at
// once: a load that finds it full stalls its wave at issue.
template <int DK>
__device__ __forceinline__ void gather_chunk(uint8_t* tile, const uint16_t* __restrict__ kv,
                                             int row, int wave, int lane, int jj0, int jj1) {
  using T = Tile<DK>;
  constexpr int GJ = T::GJ;
  // The slot arithmetic below is the same for every chunk; recomputing it (a few VALU ops)
  // is cheaper than keeping it live across the loop, so hide the lane id from hoisting.
  int ln;
  asm volatile("v_mov_b32 %0, %1" : "=v"(ln) : "v"(lane));
#pragma unroll
  for (int jj = 0; jj < GJ; ++jj) {
    if (jj < jj0 || jj >= jj1) continue;
    const int j = wave + NW * jj;
    if (GJ * NW > T::LOADS && j >= T::LOADS) break;     // wave-uniform
    const int u = j * kWave + ln;
    const int r = u / T::SLOTS;
    const int p = u - r * T::SLOTS;
    int rw;
    if constexpr (T::SLOTS >= kWave) {
      // the wave-load spans at most two rows: two lane reads
      const int rlo = (j * kWave) / T::SLOTS;           // row of the wave-load's first slot
      const int ra = __builtin_amdgcn_readlane(row, tile_row(rlo < CH ? rlo : CH - 1));
      const int rb = __builtin_amdgcn_readlane(row, tile_row(rlo + 1 < CH ? rlo + 1 : CH - 1));
      rw = r == rlo ? ra : rb;
    } else {
      rw = __shfl(row, tile_row(r & (CH - 1)));         // short rows: one lane permute
    }
    const bool real = (r < CH) & (rw >= 0) & (p < T::NCH);
    const size_t off = (size_t)(u32)(real ? rw : 0) * DK + (u32)(real ? 8 * p : 0);
    // Written out (global_load_lds_dwordx4: 16 bytes per lane into LDS at M0 + 16 * lane) so
    // that the compiler does not count it as an outstanding LDS access: it would then wait
    // for all LDS traffic (lgkmcnt(0)) wherever a tile read is consumed instead of only for
    // that read.  It has no register result; its waits are the explicit full ones that end
    // each step (and the prologue).
    const u32 lds = (u32)(uintptr_t)(__attribute__((address_space(3))) void*)(tile + 16 * kWave * j);
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(kv + off), "s"(__builtin_amdgcn_readfirstlane(lds))
                 : "memory", "m0");
#pragma clang diagnostic pop
  }
}

template <int DK, int DV, bool PAGED>
__global__ __launch_bounds__(NT, 1) void sparse_mqa_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ qpos_or_ctx,
    const int32_t* __restrict__ page_table, int max_pages, int n_pages, int page_size, int n_kv,
    int H, int top_k, float scale_log2, int n_split, int rows_per_split,
    uint16_t* __restrict__ out, float* __restrict__ lse, float* __restrict__ part_o,
    float* __restrict__ part_ml) {
  static_assert(DK % 32 == 0 && DV % 64 == 0 && DV <= DK, "shape");
  using Sh = MqaShared<DK>;
  constexpr int NKS = DK / 32;           // k-steps of this wave's half of the S^T product
  constexpr int NDB = DV / 64;           // 32-dim blocks of this wave's half of the output
  constexpr int RS = Tile<DK>::RS;
  constexpr int GJ = Tile<DK>::GJ;
  __shared__ Sh sh;
  __shared__ __attribute__((aligned(16))) uint8_t kt0[Tile<DK>::BYTES];  // selected rows, buffer 0
  __shared__ __attribute__((aligned(16))) uint8_t kt1[Tile<DK>::BYTES];  // selected rows, buffer 1

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);   // uniform: lets the compiler
                                                                 // keep wave-derived values in SGPRs
  const int hg = wave & 3;          // head group
  const int dh = wave >> 2;         // dimension half
  const int lane = tid & (kWave - 1);
  const int c32 = lane & 31;
  const int hf = lane >> 5;
  const int qi = blockIdx.x;
  const int sp = blockIdx.y;
  const int head = hg * HPW + c32;
  const bool head_ok = head < H;
  const int kd0 = dh * (DK / 2);    // first key dim of this wave's logit half
  const int vd0 = dh * (DV / 2);    // first value dim of this wave's output half

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
  // (k-steps >= QR are kept in LDS)
  constexpr int QR = QSplit<DK>::QR;
  v8bf qf[QR];
  {
    const uint16_t* qrow = q + ((size_t)qi * H + (head_ok ? head : 0)) * DK;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      v4i x = {0, 0, 0, 0};
      if (head_ok) x = ld16(qrow + kd0 + 16 * ks + 8 * hf);
      if (ks < QR)
        qf[ks < QR ? ks : 0] = as_v8bf(x);
      else
        sh.qs[wave][ks - QR][lane] = as_v8bf(x);
    }
  }

  v16f o[NDB];
#pragma unroll
  for (int d = 0; d < NDB; ++d)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[d][i] = 0.f;
  float m_run = -__builtin_inff();
  float l_run = 0.f;

  const int n_chunks = (nrows + CH - 1) / CH;
  // physical row of entry c32 of chunk cc, or -1 (entries past the slice included)
  auto chunk_row = [&](int cc) -> int {
    const int e = cc * CH + c32;
    const int v = sh.rows[e < MAX_ROWS ? e : MAX_ROWS - 1];
    return e < nrows ? v : -1;
  };
  __syncthreads();   // rows[] complete
  int row_nx = chunk_row(0);                         // rows of the chunk gathered next
  if (n_chunks > 0) gather_chunk<DK>(kt0, kv, row_nx, wave, lane, 0, Tile<DK>::GJ);
  // bit k of vm_cur: key k of the current chunk is a valid selected row
  u32 vm_cur = (u32)wave_ballot(row_nx >= 0);
  row_nx = chunk_row(1);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // per-lane byte offsets inside a tile:
  //  S^T A operand, k-step ks: key c32 (tile row tile_row(c32)), dims kd0 + 16ks + 8hf .. +8
  //  ->  qk_off + 32 ks
  const int qk_off = tile_row(c32) * RS + 2 * (kd0 + 8 * hf);
  //  transposing read of the value product: input lane (m, q) of its 16-lane group points at
  //  dims D + 4q of key 16k2 + 4hf + m (tile row 16k2 + hf + 4m; key + 8, the second half of
  //  the k-slots, is tile row + 2), so output lane j holds dim D + j;
  //  D = vd0 + 32d + 16 * (group parity)
  const int tq = lane & 3, tm = (lane & 15) >> 2;
  const int tr_off = tile_row(4 * hf + tm) * RS + 2 * (vd0 + 16 * ((lane >> 4) & 1) + 4 * tq);
  static_assert(tile_row(8) - tile_row(0) == 2 && tile_row(12) - tile_row(4) == 2 &&
                tile_row(16) - tile_row(0) == 16, "tile-row offsets of the value read");

  auto step = [&](const lds_u8* tile, uint8_t* next_tile, int c) {
    // the next chunk is gathered into the other buffer during this chunk's logit product
    const bool more = c + 1 < n_chunks;
    const u32 vm_nx = (u32)wave_ballot(row_nx >= 0);
    const u32 vmask = vm_cur;

    // ---- S^T = K Q^T for 32 keys x this wave's 32 heads, over its half of the dims ----
    v16f sp_;
#pragma unroll
    for (int i = 0; i < 16; ++i) sp_[i] = 0.f;
    const lds_u8* qk_base = tile + qk_off;
    // LDS operands are fetched QPD k-steps ahead of their product
    v4i ka[QPD];
    v8bf kb[QPD];
    auto fetch = [&](int k) {
      ka[k % QPD] = *reinterpret_cast<const __attribute__((address_space(3))) v4i*>(qk_base + 32 * k);
      if (k >= QR) kb[k % QPD] = sh.qs[wave][k >= QR ? k - QR : 0][lane];
    };
#pragma unroll
    for (int ks = 0; ks < QPD; ++ks) fetch(ks);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const v4i av = ka[ks % QPD];
      const v8bf b = ks < QR ? qf[ks < QR ? ks : 0] : kb[ks % QPD];
      if (ks + QPD < NKS) fetch(ks + QPD);
      sp_ = mfma_bf16(as_v8bf(av), b, sp_);
      // after product ks: this wave's wave-loads jj with gather_slot(jj) == ks
      const int j0 = first_load_at<NKS, GJ>(ks), j1 = first_load_at<NKS, GJ>(ks + 1);
      if (j0 < j1 && more) gather_chunk<DK>(next_tile, kv, row_nx, wave, lane, j0, j1);
      __builtin_amdgcn_sched_barrier(0);   // keep the fetch distance as written
    }
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4)
      sh.sx[wave][i4][lane] = v4f{sp_[4 * i4], sp_[4 * i4 + 1], sp_[4 * i4 + 2], sp_[4 * i4 + 3]};
    lds_barrier();

    // ---- online softmax (lane = head; element i is key 8(i/4) + 4hf + i%4) ----
    // Lazy rescaling: the reference max m_run only moves when a logit exceeds it by more than
    // 8 (log2 units), so probabilities stay below 2^8 and the accumulators are rarely
    // rescaled.  The probabilities are first formed in one pass against the current m_run;
    // only if some logit of the wave breaks the bound is the chunk redone in two passes with
    // a new m_run.  Masked keys get a -inf bias (loads stay unconditional, no branches); a
    // chunk whose keys are all valid skips the bias.
    const u32 vml = vmask >> (4 * hf);   // bit 8a + b: key 8a + 4hf + b of the chunk
    float psum = 0.f;
    v8bf pb[2];
    auto prob_pass = [&](float m_use, auto masked) {
      float mx = -__builtin_inff();
      psum = 0.f;
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const v4f sa = sh.sx[hg][i4][lane], sb = sh.sx[hg + 4][i4][lane];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * i4 + e;
          float nb = -m_use;
          if constexpr (decltype(masked)::value)
            nb = ((vml >> (8 * (i >> 2) + (i & 3))) & 1u) ? -m_use : -__builtin_inff();
          const float y = fmaf(sa[e] + sb[e], scale_log2, nb);
          mx = fmaxf(mx, y);
          const float pv = __builtin_amdgcn_exp2f(y);
          psum += pv;
          pb[i >> 3][i & 7] = (__bf16)pv;
        }
      }
      return mx;
    };
    // (with m_run = -inf every valid logit is +inf here, which forces the second path)
    const float over = vmask == 0xffffffffu ? prob_pass(m_run, std::false_type{})
                                            : prob_pass(m_run, std::true_type{});
    if (__ballot(!(over <= 8.f))) {
      float cmax = -__builtin_inff();
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const v4f sa = sh.sx[hg][i4][lane], sb = sh.sx[hg + 4][i4][lane];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * i4 + e;
          const float bias = ((vml >> (8 * (i >> 2) + (i & 3))) & 1u) ? 0.f : -__builtin_inff();
          cmax = fmaxf(cmax, fmaf(sa[e] + sb[e], scale_log2, bias));
        }
      }
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
        for (int d = 0; d < NDB; ++d)
#pragma unroll
          for (int i = 0; i < 16; ++i) o[d][i] *= alpha;
      }
    }
    l_run += psum;

    // ---- O^T += V^T P^T; V^T slots j of half hf hold key 16k2 + 8(j/4) + 4hf + j%4 ----
    const lds_u8* tr_base = tile + tr_off;
#pragma unroll
    for (int d = 0; d < NDB; ++d) {
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        const lds_u8* pa = tr_base + 16 * k2 * RS + 64 * d;
        const v4s va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(pa));
        const v4s vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(pa + 2 * RS));
        v8bf a;
        __builtin_memcpy(&a, &va, 8);
        __builtin_memcpy(reinterpret_cast<char*>(&a) + 8, &vb, 8);
        o[d] = mfma_bf16(a, pb[k2], o[d]);
      }
    }
    row_nx = chunk_row(c + 2);
    vm_cur = vm_nx;
    __builtin_amdgcn_s_waitcnt(0);   // this wave's part of the next chunk has landed
    __syncthreads();
  };

#pragma unroll 1
  for (int c = 0; c < n_chunks; c += 2) {
    step((const lds_u8*)kt0, kt1, c);
    if (c + 1 < n_chunks) step((const lds_u8*)kt1, kt0, c + 1);
  }

  // ---- epilogue: lane holds head `head`, dims vd0 + 32d + 8(i/4) + 4hf + i%4 ----
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (!head_ok) return;
  if (n_split == 1) {
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
