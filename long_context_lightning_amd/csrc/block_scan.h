// Wave- and block-level scans used by the selection kernels (wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ uint32_t wave_inclusive_sum(uint32_t v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t o = __shfl_up(v, d, 64);
    if (lane >= d) v += o;
  }
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

}  // namespace dsa
