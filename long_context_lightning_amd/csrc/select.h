// Exact block-level selection helpers shared by the top-k kernels.
//
// Keys are order-preserving uint32 images of fp32 scores.  Selection follows
// the top-k rule of the Indexer code block on the "详解DSA" page
// (topk(min(index_topk, end_pos))) with ties broken toward the lower
// position: the chosen set is {key > tau} plus the r_eq lowest positions among
// {key == tau}.
#pragma once

#include "block_scan.h"
#include "dsa_internal.h"

namespace dsa {

// Radix select, largest first, over the values produced by `for_each`
// (called once per pass with a visitor taking a uint32 value).  Values whose
// bits above `rem_bits` differ from `prefix` are ignored.  On return `prefix`
// holds the value v* such that count(v > v*) < want <= count(v >= v*) among
// the considered values, and `want` is reduced to the number of copies of v*
// still to take (want - count(v > v*)).  `whist` needs NT/64*256 words, `sm`
// needs 4 words.  Every thread of the block must call it.
template <int NT, class ForEach>
__device__ void radix_select_desc(ForEach&& for_each, uint32_t& prefix, int rem_bits, uint32_t& want,
                                  uint32_t* whist, uint32_t* sm) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  while (rem_bits > 0) {
    const int nb = rem_bits < 8 ? rem_bits : 8;
    const int shift = rem_bits - nb;
    const uint32_t dmask = (1u << nb) - 1u;
    for (int i = tid; i < NW * 256; i += NT) whist[i] = 0u;
    if (tid == 0) {
      sm[0] = 0u;
      sm[1] = 0u;
    }
    __syncthreads();
    const uint32_t hi = rem_bits >= 32 ? 0u : (prefix >> rem_bits);
    const int rb = rem_bits;
    uint32_t* mine = whist + wave * 256;
    for_each([&](uint32_t v) {
      if ((rb >= 32 ? 0u : (v >> rb)) == hi) atomicAdd(&mine[(v >> shift) & dmask], 1u);
    });
    __syncthreads();
    if (tid < 256) {
      uint32_t s = 0;
      for (int w = 0; w < NW; ++w) s += whist[w * 256 + tid];
      whist[tid] = s;  // column sums overwrite wave 0's row (only wave 0's row is read below)
    }
    __syncthreads();
    if (wave == 0) {
      // lane l owns digits 4*(63-l) .. 4*(63-l)+3, i.e. lanes walk digits high -> low
      const int d0 = 4 * (63 - lane);
      uint32_t c[4];
      uint32_t tot = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        c[j] = whist[d0 + 3 - j];  // descending digit order
        tot += c[j];
      }
      const uint32_t above = wave_inclusive_sum(tot) - tot;
      if (above < want && want <= above + tot) {
        uint32_t acc = above;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (acc < want && want <= acc + c[j]) {
            sm[0] = (uint32_t)(d0 + 3 - j);
            sm[1] = acc;
          }
          acc += c[j];
        }
      }
    }
    __syncthreads();
    prefix |= sm[0] << shift;
    want -= sm[1];
    rem_bits = shift;
    __syncthreads();
  }
}

// Write the set bits of `bitmap` (n bits, positions 0..n-1) as ascending
// positions to out[0..].  Returns the number written.  Block-wide.
template <int NT>
__device__ uint32_t bitmap_to_sorted(const uint32_t* bitmap, int n, int32_t* out, uint32_t limit, uint32_t* sm) {
  const int W = (n + 31) >> 5;
  const int per = (W + NT - 1) / NT;
  const int w0 = (int)threadIdx.x * per;
  const int w1 = min(w0 + per, W);
  uint32_t cnt = 0;
  for (int w = w0; w < w1; ++w) cnt += __popc(bitmap[w]);
  uint32_t total;
  uint32_t off = block_exclusive_sum<NT>(cnt, sm, &total);
  for (int w = w0; w < w1; ++w) {
    uint32_t bits = bitmap[w];
    while (bits) {
      const int b = __ffs(bits) - 1;
      if (off < limit) out[off] = 32 * w + b;
      ++off;
      bits &= bits - 1u;
    }
  }
  return total;
}

}  // namespace dsa
