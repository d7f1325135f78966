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
// (called once per pass with a visitor taking a uint32 value), DB bits per
// pass.  Values whose bits above `rem_bits` differ from `prefix` are ignored.
// On return `prefix` holds the value v* such that
// count(v > v*) < want <= count(v >= v*) among the considered values, and
// `want` is reduced to the number of copies of v* still to take
// (want - count(v > v*)).  `whist` needs NT/64 << DB words, `sm` 4 words.
// Every thread of the block must call it.
template <int NT, int DB, class ForEach>
__device__ void radix_select_desc(ForEach&& for_each, uint32_t& prefix, int rem_bits, uint32_t& want,
                                  uint32_t* whist, uint32_t* sm) {
  constexpr int NW = NT / 64;
  constexpr int NB = 1 << DB;
  constexpr int PER_LANE = NB / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  while (rem_bits > 0) {
    const int nb = rem_bits < DB ? rem_bits : DB;
    const int shift = rem_bits - nb;
    const uint32_t dmask = (1u << nb) - 1u;
    for (int i = tid; i < NW * NB; i += NT) whist[i] = 0u;
    if (tid == 0) {
      sm[0] = 0u;
      sm[1] = 0u;
    }
    __syncthreads();
    const uint32_t hi = rem_bits >= 32 ? 0u : (prefix >> rem_bits);
    const int rb = rem_bits;
    uint32_t* mine = whist + wave * NB;
    for_each([&](uint32_t v) {
      if ((rb >= 32 ? 0u : (v >> rb)) == hi) atomicAdd(&mine[(v >> shift) & dmask], 1u);
    });
    __syncthreads();
    for (int i = tid; i < NB; i += NT) {
      uint32_t c = 0;
      for (int w = 0; w < NW; ++w) c += whist[w * NB + i];
      whist[i] = c;  // column sums overwrite wave 0's row (each column read and written by one thread)
    }
    __syncthreads();
    if (wave == 0) {
      // lane l owns digits d0 .. d0+PER_LANE-1 with d0 = PER_LANE*(63-l): lanes walk digits high -> low
      const int d0 = PER_LANE * (63 - lane);
      uint32_t tot = 0;
      for (int j = 0; j < PER_LANE; ++j) tot += whist[d0 + j];
      const uint32_t above = wave_inclusive_sum(tot) - tot;
      if (above < want && want <= above + tot) {
        uint32_t acc = above;
        for (int j = PER_LANE - 1; j >= 0; --j) {
          const uint32_t cj = whist[d0 + j];
          if (acc < want && want <= acc + cj) {
            sm[0] = (uint32_t)(d0 + j);
            sm[1] = acc;
          }
          acc += cj;
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

// Bitmap tail of a selection.  `bitmap` holds the positions with key > tau,
// `tbits` the copies of tau; both cover n positions in W = ceil(n/32) words
// and are zero up to the next multiple of 4 words (they are read 16 bytes at
// a time).  Keeps the `want` lowest-position copies of tau (want >= 1),
// folds them into `bitmap`, and writes all set positions in ascending order
// to out[0..limit).  Thread t owns the contiguous words
// [t*per, (t+1)*per), per a multiple of 4.  Returns the number of set
// positions.  `sm` needs NT/64 + 4 words, and other threads may still read
// it on return: a barrier must come before it is written again.  Block-wide.
template <int NT>
__device__ uint32_t bitmap_select_emit(uint32_t* bitmap, const uint32_t* tbits, int n, uint32_t want, int32_t* out,
                                       uint32_t limit, uint32_t* sm) {
  constexpr int NW = NT / 64;
  const int W4 = (((n + 31) >> 5) + 3) >> 2;  // 16-byte groups
  const int per4 = (W4 + NT - 1) / NT;
  const int g0 = (int)threadIdx.x * per4, g1 = min(g0 + per4, W4);
  const v4i* t4 = reinterpret_cast<const v4i*>(tbits);
  v4i* b4 = reinterpret_cast<v4i*>(bitmap);
  // 1. the want-th set bit of tbits (in position order) is the last copy kept
  uint32_t c = 0;
  for (int gi = g0; gi < g1; ++gi) {
    const v4i t = t4[gi];
    c += __popc((uint32_t)t[0]) + __popc((uint32_t)t[1]) + __popc((uint32_t)t[2]) + __popc((uint32_t)t[3]);
  }
  if (threadIdx.x == 0) sm[NW + 2] = 0xFFFFFFFFu;
  uint32_t tot;
  uint32_t acc = block_exclusive_sum<NT>(c, sm, &tot);
  if (acc < want && want <= acc + c) {
    for (int gi = g0; gi < g1; ++gi) {
      const v4i t = t4[gi];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t bits = (uint32_t)t[j];
        const uint32_t pc = __popc(bits);
        if (acc < want && want <= acc + pc) {
          for (uint32_t r = want - acc; r > 1; --r) bits &= bits - 1u;
          sm[NW + 2] = 32u * (uint32_t)(4 * gi + j) + (uint32_t)(__ffs(bits) - 1);
        }
        acc += pc;
      }
    }
  }
  __syncthreads();
  const uint32_t cut = sm[NW + 2];
  const int cw = (int)(cut >> 5);
  const uint32_t cmask = (2u << (cut & 31)) - 1u;  // bits <= cut within word cw
  // 2. fold the kept copies into bitmap and count
  uint32_t cnt = 0;
  for (int gi = g0; gi < g1; ++gi) {
    const v4i t = t4[gi];
    v4i b = b4[gi];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int wi = 4 * gi + j;
      const uint32_t keep = wi < cw ? 0xFFFFFFFFu : (wi == cw ? cmask : 0u);
      b[j] = (int)((uint32_t)b[j] | ((uint32_t)t[j] & keep));
      cnt += __popc((uint32_t)b[j]);
    }
    b4[gi] = b;
  }
  uint32_t total;
  uint32_t off = block_exclusive_sum_once<NT>(cnt, sm, &total);  // sm is not written again here
  // 3. positions in ascending order
  for (int gi = g0; gi < g1; ++gi) {
    const v4i b = b4[gi];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t bits = (uint32_t)b[j];
      while (bits) {
        const int bb = __ffs(bits) - 1;
        if (off < limit) out[off] = 32 * (4 * gi + j) + bb;
        ++off;
        bits &= bits - 1u;
      }
    }
  }
  return total;
}

// Writes the set positions of `bitmap` (n positions, zero up to the next
// multiple of 4 words) in ascending order to out[0..limit).  Thread t owns
// the contiguous 16-byte groups [t*per, (t+1)*per).  Returns the number of
// set positions.  `sm` needs NT/64 + 4 words, and other threads may still
// read it on return: a barrier must come before it is written again.
// Block-wide.
template <int NT>
__device__ uint32_t bitmap_emit(const uint32_t* bitmap, int n, int32_t* out, uint32_t limit, uint32_t* sm) {
  const int W4 = (((n + 31) >> 5) + 3) >> 2;  // 16-byte groups
  const int per4 = (W4 + NT - 1) / NT;
  const int g0 = (int)threadIdx.x * per4, g1 = min(g0 + per4, W4);
  const v4i* b4 = reinterpret_cast<const v4i*>(bitmap);
  uint32_t cnt = 0;
  for (int gi = g0; gi < g1; ++gi) {
    const v4i b = b4[gi];
    cnt += __popc((uint32_t)b[0]) + __popc((uint32_t)b[1]) + __popc((uint32_t)b[2]) + __popc((uint32_t)b[3]);
  }
  uint32_t total;
  uint32_t off = block_exclusive_sum_once<NT>(cnt, sm, &total);  // sm is not written again here
  for (int gi = g0; gi < g1; ++gi) {
    const v4i b = b4[gi];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t bits = (uint32_t)b[j];
      while (bits) {
        const int bb = __ffs(bits) - 1;
        if (off < limit) out[off] = 32 * (4 * gi + j) + bb;
        ++off;
        bits &= bits - 1u;
      }
    }
  }
  return total;
}

}  // namespace dsa

