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
//      the kept items come out in ascending position order.
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

// Step 2.  load(i) returns an item with a `.key` field; emit(item, pos) stores a kept item at
// output position pos.  In-place use (output aliasing the input) is safe: every item of a
// chunk is loaded before any item of that chunk is stored, and stores go below the chunk end.
// Returns the number of kept items (k when called with step 1's T and r).
template <int NT, class Load, class Emit>
__device__ int block_stable_keep(Load load, int n, u32 T, int r, Emit emit, SelectShared& sh) {
  constexpr int NW = NT / kWave;
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  int ties = 0, out = 0;
#pragma unroll 1
  for (int base = 0; base < n; base += NT) {
    const int i = base + tid;
    const bool in = i < n;
    auto item = load(in ? i : 0);
    const bool gt = in && item.key > T;
    const bool eq = in && item.key == T;
    const uint64_t beq = wave_ballot(eq);
    if ((tid & (kWave - 1)) == 0) sh.wave_a[wave] = __builtin_popcountll(beq);
    __syncthreads();
    int before = 0, tot = 0;
#pragma unroll
    for (int v = 0; v < NW; ++v) {
      const int c = sh.wave_a[v];
      before += (v < wave) ? c : 0;
      tot += c;
    }
    const int rank = ties + before + lanes_below(beq);
    const bool keep = gt || (eq && rank < r);
    const uint64_t bk = wave_ballot(keep);
    if ((tid & (kWave - 1)) == 0) sh.wave_b[wave] = __builtin_popcountll(bk);
    __syncthreads();
    int kbefore = 0, ktot = 0;
#pragma unroll
    for (int v = 0; v < NW; ++v) {
      const int c = sh.wave_b[v];
      kbefore += (v < wave) ? c : 0;
      ktot += c;
    }
    if (keep) emit(item, out + kbefore + lanes_below(bk));
    ties += tot;
    out += ktot;
    __syncthreads();
  }
  return out;
}

}  // namespace dsa
