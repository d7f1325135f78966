// Per-block fp8 quantisation of indexer inputs and the indexer key-cache
// append.
//
// The Indexer code block of "详解DSA" quantises q and k with act_quant(x,
// block_size) and stores the key codes and their scales in the fp8 key cache
// at the new positions (k_cache[:bsz, start_pos:end_pos] = k_fp8); its
// "DSA计算流" section adds that the key cache keeps each key's scale.  The
// pages do not print act_quant; the reading implemented here: one scale per
// 128-element block, scale = max(amax, 2^-126) / 448 in fp32, and each code
// the fp32 quotient x / scale rounded to the nearest e4m3fn value (ties to
// the even code, 448 for a quotient past it, the quotient's sign kept).
//
// HBM-bound streaming: a 32-lane half-wave owns one block; lane j loads
// elements 4j..4j+3 (8 bytes of bf16 or 16 of fp32), the block maximum comes
// from five xor-shuffles inside the half-wave, and each lane stores its four
// codes as one 4-byte word, so a block's 128 codes are one coalesced
// 128-byte store.  Grid-stride over blocks; every lane of a half-wave takes
// the same trip count, so the shuffles never see an inactive partner.
#include "dsa_internal.h"

namespace dsa {

namespace {

constexpr int kBlock = 128;
constexpr int kThreads = 256;
constexpr int kBlocksPerCta = kThreads / 32;

// fp32 -> e4m3fn code, round to nearest even, saturating at 448, sign kept.
// |v| < 2^-6 is the subnormal range (step 2^-9): the code is the rounded
// multiple of 2^-9 (8 meaning the smallest normal, whose code is also 8).
// Otherwise the 23-bit fp32 mantissa is rounded to 3 bits with the carry
// moving into the exponent.
__device__ __forceinline__ uint32_t e4m3fn_rne(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = fabsf(v);
  uint32_t code;
  if (!(a < 448.0f)) {
    code = 0x7Eu;
  } else if (a < 0.015625f) {
    code = (uint32_t)__builtin_rintf(a * 512.0f);
  } else {
    const uint32_t ua = __float_as_uint(a);
    uint32_t e = (ua >> 23) - 120u;  // biased e4m3 exponent: (e8 - 127) + 7
    uint32_t m = (ua >> 20) & 7u;
    const uint32_t rem = ua & 0xFFFFFu;
    m += (rem > 0x80000u || (rem == 0x80000u && (m & 1u))) ? 1u : 0u;
    if (m == 8u) {
      m = 0u;
      ++e;
    }
    code = min((e << 3) | m, 0x7Eu);
  }
  return code | sign;
}

template <bool BF16>
__device__ __forceinline__ void load4(const void* x, long long blk, int j, float (&v)[4]) {
  if (BF16) {
    const uint2 u = *(reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(x) + blk * kBlock) + j);
    v[0] = __uint_as_float(u.x << 16);
    v[1] = __uint_as_float(u.x & 0xFFFF0000u);
    v[2] = __uint_as_float(u.y << 16);
    v[3] = __uint_as_float(u.y & 0xFFFF0000u);
  } else {
    const float4 f = *(reinterpret_cast<const float4*>(static_cast<const float*>(x) + blk * kBlock) + j);
    v[0] = f.x;
    v[1] = f.y;
    v[2] = f.z;
    v[3] = f.w;
  }
}

// Quantises block blk in the calling half-wave; returns the lane's packed
// codes and (in every lane) the block scale.
template <bool BF16>
__device__ __forceinline__ uint32_t quant_block(const void* x, long long blk, int j, float& scale) {
  float v[4];
  load4<BF16>(x, blk, j, v);
  float amax = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
#pragma unroll
  for (int o = 16; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 32));
  amax = fmaxf(amax, 0x1p-126f);
  scale = __fdiv_rn(amax, 448.0f);
  uint32_t packed = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) packed |= e4m3fn_rne(__fdiv_rn(v[e], scale)) << (8 * e);
  return packed;
}

template <bool BF16>
__global__ __launch_bounds__(kThreads) void k_quantize(QuantArgs a) {
  const int j = threadIdx.x & 31;
  const long long first = (long long)blockIdx.x * kBlocksPerCta + (threadIdx.x >> 5);
  const long long stride = (long long)gridDim.x * kBlocksPerCta;
  for (long long blk = first; blk < a.rows; blk += stride) {
    float scale;
    const uint32_t packed = quant_block<BF16>(a.x, blk, j, scale);
    reinterpret_cast<uint32_t*>(a.codes + blk * kBlock)[j] = packed;
    if (j == 0) a.scales[blk] = scale;
  }
}

// Row blk = b * q_len + i of the new keys goes to position
// clamp(seq_lens[b], 0, S_max) - q_len + i of sequence b (skipped if negative).
template <bool BF16>
__global__ __launch_bounds__(kThreads) void k_cache_append(QuantArgs a) {
  const int j = threadIdx.x & 31;
  const long long first = (long long)blockIdx.x * kBlocksPerCta + (threadIdx.x >> 5);
  const long long stride = (long long)gridDim.x * kBlocksPerCta;
  for (long long blk = first; blk < a.rows; blk += stride) {
    const int b = (int)(blk / a.q_len), i = (int)(blk - (long long)b * a.q_len);
    const int s = clamped_len(a.seq_lens, b, a.S_max) - a.q_len + i;
    float scale;
    const uint32_t packed = quant_block<BF16>(a.x, blk, j, scale);
    if (s >= 0) {
      const long long dst = (long long)b * a.S_max + s;
      reinterpret_cast<uint32_t*>(a.codes + dst * kBlock)[j] = packed;
      if (j == 0) a.scales[dst] = scale;
    }
  }
}

unsigned grid_for(long long rows) {
  const long long ctas = (rows + kBlocksPerCta - 1) / kBlocksPerCta;
  return (unsigned)(ctas < 8192 ? ctas : 8192);  // grid-stride beyond 2048 resident blocks
}

}  // namespace

hipError_t launch_quantize(const QuantArgs& a, bool bf16, hipStream_t stream) {
  if (a.rows <= 0) return hipSuccess;
  const dim3 grid(grid_for(a.rows)), block(kThreads);
  if (bf16) hipLaunchKernelGGL(k_quantize<true>, grid, block, 0, stream, a);
  else hipLaunchKernelGGL(k_quantize<false>, grid, block, 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_cache_append(const QuantArgs& a, bool bf16, hipStream_t stream) {
  if (a.rows <= 0) return hipSuccess;
  const dim3 grid(grid_for(a.rows)), block(kThreads);
  if (bf16) hipLaunchKernelGGL(k_cache_append<true>, grid, block, 0, stream, a);
  else hipLaunchKernelGGL(k_cache_append<false>, grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace dsa
