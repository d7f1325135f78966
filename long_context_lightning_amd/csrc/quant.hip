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
// HBM-bound streaming: a 32-lane half-wave owns one block at a time; lane j
// loads elements 4j..4j+3 (8 bytes of bf16 or 16 of fp32), the block maximum
// comes from five xor-shuffles inside the half-wave, and each lane stores
// its four codes as one 4-byte word, so a block's 128 codes are one
// coalesced 128-byte store.  Grid-stride over blocks, kU blocks per trip;
// every lane of a half-wave takes the same trips and computes every block of
// a trip (the stores are what is skipped), so the shuffles never see an
// inactive partner.
#include "dsa_internal.h"

namespace dsa {

namespace {

constexpr int kBlock = 128;
constexpr int kThreads = 256;
constexpr int kBlocksPerCta = kThreads / 32;

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

// Codes of the lane's four elements of one block (its scale in every lane
// of the half-wave).  The quotients, clamped to +-448 (the fp32 rounding of
// the scale can put the block maximum a hair above it), go through the
// gfx950 packed fp32 -> e4m3fn conversion (round to nearest even), two per
// instruction.
__device__ __forceinline__ uint32_t quant4(const float (&v)[4], float& scale) {
  float amax = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
#pragma unroll
  for (int o = 16; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 32));
  amax = fmaxf(amax, 0x1p-126f);
  scale = __fdiv_rn(amax, 448.0f);
  float qv[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) qv[e] = __builtin_amdgcn_fmed3f(__fdiv_rn(v[e], scale), -448.0f, 448.0f);
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(qv[0], qv[1], 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(qv[2], qv[3], lo, true);
}

// Each half-wave takes kU blocks per trip (blk, blk + stride, ...), all
// loads issued first (indices clamped into range, out-of-range results not
// stored), so every lane keeps kU loads in flight.
constexpr int kU = 4;

template <bool BF16, bool APPEND>
__global__ __launch_bounds__(kThreads) void k_quant(QuantArgs a) {
  const int j = threadIdx.x & 31;
  const long long first = (long long)blockIdx.x * kBlocksPerCta + (threadIdx.x >> 5);
  const long long stride = (long long)gridDim.x * kBlocksPerCta;
  for (long long blk0 = first; blk0 < a.rows; blk0 += kU * stride) {
    float v[kU][4];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const long long blk = blk0 + u * stride;
      load4<BF16>(a.x, blk < a.rows ? blk : a.rows - 1, j, v[u]);
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const long long blk = blk0 + u * stride;
      float scale;
      const uint32_t packed = quant4(v[u], scale);
      if (blk >= a.rows) continue;
      long long dst = blk;
      if (APPEND) {
        // row b*q_len + i -> position clamp(seq_lens[b], 0, S_max) - q_len + i
        // (a pool row when the cache is paged)
        const int b = (int)(blk / a.q_len), i = (int)(blk - (long long)b * a.q_len);
        const int s = clamped_len(a.seq_lens, b, a.S_max) - a.q_len + i;
        if (s < 0) continue;
        dst = a.pages.table ? (long long)a.pages.row(b, s) : (long long)b * a.S_max + s;
      }
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
  if (bf16) hipLaunchKernelGGL((k_quant<true, false>), grid, block, 0, stream, a);
  else hipLaunchKernelGGL((k_quant<false, false>), grid, block, 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_cache_append(const QuantArgs& a, bool bf16, hipStream_t stream) {
  if (a.rows <= 0) return hipSuccess;
  const dim3 grid(grid_for(a.rows)), block(kThreads);
  if (bf16) hipLaunchKernelGGL((k_quant<true, true>), grid, block, 0, stream, a);
  else hipLaunchKernelGGL((k_quant<false, true>), grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace dsa
