// Wave- and block-level scans used by the selection kernels (wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

// Value of lane (l - n) within the same 16-lane row for lanes of the rows
// in ROW_MASK (0 where that lane is outside the row), else 0; DPP CTRL.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_take(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xF, true);
}

// Inclusive prefix sum over the 64 lanes of a wave, with DPP: a
// Hillis-Steele scan inside each 16-lane row (row_shr 1, 2, 4, 8), then
// row_bcast:15 carries each even row's total into the next row and
// row_bcast:31 carries lanes 0..31's total into lanes 32..63.  Every lane of
// the wave must be active.
__device__ __forceinline__ uint32_t wave_inclusive_sum(uint32_t v) {
  v += dpp_take<0x111, 0xF>(v);  // row_shr:1
  v += dpp_take<0x112, 0xF>(v);  // row_shr:2
  v += dpp_take<0x114, 0xF>(v);  // row_shr:4
  v += dpp_take<0x118, 0xF>(v);  // row_shr:8
  v += dpp_take<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v += dpp_take<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}

// Exclusive prefix sum over a block of NT threads (NT a multiple of 64,
// NT <= 4096).  `sm` needs NT/64 + 1 words.  Returns the exclusive prefix of
// thread threadIdx.x; *total receives the block sum.  Contains barriers: call
// from every thread.
template <int NT>
__device__ __forceinline__ uint32_t block_exclusive_sum(uint32_t v, uint32_t* sm, uint32_t* total) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t inc = wave_inclusive_sum(v);
  if (lane == 63) sm[wave] = inc;
  __syncthreads();
  if (wave == 0) {
    uint32_t w = (lane < NW) ? sm[lane] : 0u;
    const uint32_t wi = wave_inclusive_sum(w);
    if (lane < NW) sm[lane] = wi - w;
    if (lane == NW - 1) sm[NW] = wi;
  }
  __syncthreads();
  const uint32_t res = sm[wave] + inc - v;
  *total = sm[NW];
  __syncthreads();
  return res;
}

// The same prefix sum with a single barrier: every wave reads all the wave
// totals.  `sm` needs NT/64 words; there is no trailing barrier, so the
// caller must not write sm[0 .. NT/64) again before a later barrier.
template <int NT>
__device__ __forceinline__ uint32_t block_exclusive_sum_once(uint32_t v, uint32_t* sm, uint32_t* total) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t inc = wave_inclusive_sum(v);
  if (lane == 63) sm[wave] = inc;
  __syncthreads();
  uint32_t base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint32_t t = sm[w];
    base += (w < wave) ? t : 0u;
    tot += t;
  }
  *total = tot;
  return base + inc - v;
}

}  // namespace dsa
