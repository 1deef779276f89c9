// Exact block-wide top-k selection over a sequence of (score, position) items kept in
// position order.
//
// The selection keeps the k items that come first under (score descending, position
// ascending) — the fine-grained token selection of the jdon.com "DeepSeek-V3.2-Exp" article
// (paragraph on token selection: each query keeps its 2048 highest-scoring keys), with ties
// going to the lower position.  It is found in two steps:
//   1. a 4-pass radix select (8 bits per pass, most significant first) over the
//      order-preserving 32-bit keys of the scores finds the k-th largest key T and the number
//      r of items with key == T that belong to the top-k (count(key > T) == k - r);
//   2. a stable pass keeps every item with key > T and the first r items with key == T.
//      Because items are stored in position order, "first r" is "lowest r positions", and
//      the kept items come out in ascending position order.  (The prefill indexer's keep pass,
//      which reads 4 items per lane, sits beside its list cuts; the decode finish marks the
//      kept positions in a bitmap.)
#pragma once

#include "dsa_common.hpp"

namespace dsa {

struct SelectShared {
  u32 hist[256];
  int wave_a[16];
  int wave_b[16];
  int digit;
  int above;
};

// Step 1.  Requires n > k >= 1 and the same (n, k) in every thread of the block.
// key_of(i) must return the ord_key of item i; it is called several times per item.
template <int NT, class KeyOf>
__device__ void block_radix_select(KeyOf key_of, int n, int k, SelectShared& sh, u32& T_out,
                                   int& r_out) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  u32 prefix = 0u, pmask = 0u;
  int remaining = k;
#pragma unroll 1
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += NT) sh.hist[i] = 0u;
    __syncthreads();
    for (int i = tid; i < n; i += NT) {
      const u32 kk = key_of(i);
      const bool match = (kk & pmask) == prefix;
      const u32 d = (kk >> shift) & 255u;
      const uint64_t mm = wave_ballot(match);
      // All matching lanes of the wave on one digit (the common case for the leading
      // digits): one atomic for the whole wave instead of a 64-way conflict.
      const int first = __builtin_ctzll(mm | (1ull << 63));
      const u32 d0 = __builtin_amdgcn_readlane(d, first);
      const uint64_t same = wave_ballot(match && d == d0);
      if (same == mm) {
        if (lane == first && mm) atomicAdd(&sh.hist[d0], (u32)__builtin_popcountll(mm));
      } else if (match) {
        atomicAdd(&sh.hist[d], 1u);
      }
    }
    __syncthreads();
    if (tid < kWave) {
      // lane l owns digits 4l..4l+3; find the digit holding the remaining-th largest key.
      u32 c[4];
      int tot = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        c[b] = sh.hist[4 * lane + b];
        tot += (int)c[b];
      }
      int incl = tot;  // inclusive suffix sum over lanes >= this lane
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        const int t = __shfl_down(incl, o);
        if (lane + o < kWave) incl += t;
      }
      const int excl = incl - tot;
      if (excl < remaining && remaining <= incl) {
        int cum = excl;
#pragma unroll
        for (int b = 3; b >= 0; --b) {
          if (cum + (int)c[b] >= remaining) {
            sh.digit = 4 * lane + b;
            sh.above = cum;
            break;
          }
          cum += (int)c[b];
        }
      }
    }
    __syncthreads();
    const int d = sh.digit;
    remaining -= sh.above;
    prefix |= ((u32)d) << shift;
    pmask |= 255u << shift;
    __syncthreads();
  }
  T_out = prefix;
  r_out = remaining;
}

}  // namespace dsa

namespace dsa {

// ------------------------------------------------------------------------------------------
// Wave-level versions (one wave selects over one list; no block barriers).  `hist` is this
// wave's private 256-bin LDS histogram.  Lists live in global memory, so every pass loads
// U items per lane before using any of them, keeping U loads in flight.
// ------------------------------------------------------------------------------------------
constexpr int kSelU = 16;

// Batch loaders for wave_radix_select: load(base, kk, in) fills the order keys of items
// base .. base + 64 kSelU - 1 (any order) and whether each is below n.  Every load of a batch
// is issued before any of them is used.
template <class KeyOf>
struct ScalarKeys {
  KeyOf key_of;
  int n;
  __device__ void operator()(int base, u32 (&kk)[kSelU], bool (&in)[kSelU]) const {
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int u = 0; u < kSelU; ++u) kk[u] = key_of(min(base + u * kWave + lane, n - 1));
#pragma unroll
    for (int u = 0; u < kSelU; ++u) in[u] = base + u * kWave + lane < n;
  }
};

// fp32 scores stored contiguously (16-byte aligned, readable up to the next multiple of 4
// items): 16-byte loads, 4 items per load, so a batch takes kSelU / 4 loads per lane.
struct ScoreKeys {
  const float* cs;
  int n;
  __device__ void operator()(int base, u32 (&kk)[kSelU], bool (&in)[kSelU]) const {
    const int lane = threadIdx.x & (kWave - 1);
    constexpr int V = kSelU / 4;
    const int last = (n - 1) & ~3;                    // last 4-aligned item index below n
    v4f f[V];
#pragma unroll
    for (int v = 0; v < V; ++v)
      f[v] = *reinterpret_cast<const v4f*>(cs + min(base + 256 * v + 4 * lane, last));
#pragma unroll
    for (int v = 0; v < V; ++v)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kk[4 * v + e] = ord_key(f[v][e]);
        in[4 * v + e] = base + 256 * v + 4 * lane + e < n;
      }
  }
};

template <class Loader>
__device__ void wave_radix_select_batched(const Loader& load, int n, int k, u32* hist, u32& T_out,
                                          int& r_out) {
  const int lane = threadIdx.x & (kWave - 1);
  // bits on which all keys agree need no pass
  u32 kand = 0xffffffffu, kor = 0u;
  for (int base = 0; base < n; base += kWave * kSelU) {
    u32 kk[kSelU];
    bool in[kSelU];
    load(base, kk, in);
#pragma unroll
    for (int u = 0; u < kSelU; ++u) {
      kand &= in[u] ? kk[u] : 0xffffffffu;
      kor |= in[u] ? kk[u] : 0u;
    }
  }
  for (int o = 32; o >= 1; o >>= 1) {
    kand &= (u32)__shfl_xor((int)kand, o);
    kor |= (u32)__shfl_xor((int)kor, o);
  }
  const u32 diff = kand ^ kor;
  u32 prefix = kand & ~diff, pmask = ~diff;  // common bits are fixed from the start
  int remaining = k;
  if (diff != 0u) {
    const int top = 31 - __builtin_clz(diff);
#pragma unroll 1
    for (int hi = top; hi >= 0; hi -= 8) {
      const int shift = hi >= 7 ? hi - 7 : 0;
      const u32 dmask = (hi >= 7) ? 255u : ((1u << (hi + 1)) - 1u);
      if ((diff & (dmask << shift)) == 0u) continue;
#pragma unroll
      for (int b = 0; b < 4; ++b) hist[4 * lane + b] = 0u;
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
      for (int base = 0; base < n; base += kWave * kSelU) {
        u32 kk[kSelU];
        bool in[kSelU];
        load(base, kk, in);
#pragma unroll
        for (int u = 0; u < kSelU; ++u) {
          const bool match = in[u] && (kk[u] & pmask) == prefix;
          const u32 d = (kk[u] >> shift) & dmask;
          const uint64_t mm = wave_ballot(match);
          if (mm == 0ull) continue;
          // all matching lanes on one digit (the common case): one atomic for the wave
          const int first = __builtin_ctzll(mm);
          const u32 d0 = __builtin_amdgcn_readlane(d, first);
          const uint64_t same = wave_ballot(match && d == d0);
          if (same == mm) {
            if (lane == first) atomicAdd(&hist[d0], (u32)__builtin_popcountll(mm));
          } else if (match) {
            atomicAdd(&hist[d], 1u);
          }
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
      u32 c[4];
      int tot = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        c[b] = hist[4 * lane + b];
        tot += (int)c[b];
      }
      int incl = tot;
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        const int t = __shfl_down(incl, o);
        if (lane + o < kWave) incl += t;
      }
      const int excl = incl - tot;
      int dsel = 0, above = 0;
      const bool mine = (excl < remaining && remaining <= incl);
      if (mine) {
        int cum = excl;
        for (int b = 3; b >= 0; --b) {
          if (cum + (int)c[b] >= remaining) {
            dsel = 4 * lane + b;
            above = cum;
            break;
          }
          cum += (int)c[b];
        }
      }
      const uint64_t who = wave_ballot(mine);
      const int src = __builtin_ctzll(who | (1ull << 63));
      dsel = __builtin_amdgcn_readlane(dsel, src);
      above = __builtin_amdgcn_readlane(above, src);
      remaining -= above;
      prefix = (prefix & ~(dmask << shift)) | ((u32)dsel << shift);
      pmask |= dmask << shift;
    }
  }
  T_out = prefix;
  r_out = remaining;
}

// Step 1 over fp32 scores stored contiguously (see ScoreKeys).
__device__ inline void wave_radix_select_scores(const float* cs, int n, int k, u32* hist,
                                                u32& T_out, int& r_out) {
  wave_radix_select_batched(ScoreKeys{cs, n}, n, k, hist, T_out, r_out);
}

}  // namespace dsa
