// Lightning Indexer scores into a row-major score buffer ("详解DSA" Eq.(1)).
//
//   I[t,s] = k_scale[s] * sum_j w[t,j]*q_scale[t,j] * ReLU(q[t,j,:] . k[s,:])
//
// fp8 path: a block owns a 2048-key chunk of one sequence and up to NQ query
// rows of that sequence; its four waves step through the chunk 64 keys each
// per step, with the next step's key fragments loaded while the current step
// computes.  The 64x128 query tile of a row stays in
// registers as four A fragments of v_mfma_f32_16x16x128_f8f6f4 (16 heads x
// the full 128-deep dot each), each 16-key block of the fp8 key cache is
// loaded straight from HBM into a B fragment (four lanes per 128-byte key
// row, fully coalesced), and four MFMAs give D[64 heads, 16 keys].  The
// epilogue applies ReLU and the per-head weight in fp32 on the MFMA result
// registers, then reduces the 64 heads across the four 16-lane rows with the
// gfx950 row-swap permutes, arranged so that after four key blocks lane l
// holds the finished score of key (wave_base + l): the k-scale multiply, the
// causal mask and the store are one coalesced 256-byte row write.
#include "dsa_internal.h"

namespace dsa {

namespace {

constexpr int kWavesPerBlock = 4;
constexpr int kKeysPerWave = 64;                               // keys per wave per step
constexpr int kKeysPerBlock = kWavesPerBlock * kKeysPerWave;   // keys per block per step
// Keys streamed by one block.  At two blocks per CU a 128K decode launch has
// 1024 blocks, twice what is resident at once: blocks of the second round
// start where first-round blocks finish, which evens out the spread of
// finish times of a single round (measured: 47.6 -> 34.8 us per launch
// against 4096-key chunks, same box and data).
constexpr int kKeysPerChunk = 2048;

__device__ float g_unit_scale = 1.0f;  // k-scale read when the cache has none (never written)

__device__ __forceinline__ v8i load32(const uint8_t* p) {
  v4i lo = *reinterpret_cast<const v4i*>(p);
  v4i hi = *reinterpret_cast<const v4i*>(p + 16);
  return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// D[16 heads, 16 keys] = A (heads x 128 fp8) * B (128 fp8 x keys); fp32 accumulate.
__device__ __forceinline__ v4f mfma_fp8_16x16x128(v8i a, v8i b) {
  v4f z = {0.f, 0.f, 0.f, 0.f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, z, 0, 0, 0, 0, 0, 0);
}

// Row group handled by this block: up to NQ consecutive rows of one sequence.
struct RowGroup {
  int b, t0, nr;
};

template <int NQ>
__device__ __forceinline__ RowGroup row_group(const IndexerArgs& a) {
  const int row_end = a.row_begin + a.row_count;
  const int gps = (a.q_len + NQ - 1) / NQ;
  const int b = a.row_begin / a.q_len + (int)blockIdx.y / gps;
  const int j = (int)blockIdx.y % gps;
  int t0 = b * a.q_len + j * NQ;
  int t1 = min(t0 + NQ, (b + 1) * a.q_len);
  t0 = max(t0, a.row_begin);
  t1 = min(t1, row_end);
  return RowGroup{b, t0, t1 - t0};
}

// The zeroing side job (see IndexerArgs), spread over every block of the launch.
__device__ __forceinline__ void zero_side_job(const IndexerArgs& a) {
  if (!a.zero_base) return;
  const int nthreads = (int)(gridDim.x * gridDim.y * blockDim.x);
  const int total = a.zero_rows * a.zero_words;
  for (int i = (int)((blockIdx.y * gridDim.x + blockIdx.x) * blockDim.x + threadIdx.x); i < total; i += nthreads) {
    const int r = i / a.zero_words, j = i - r * a.zero_words;
    a.zero_base[(long long)r * a.zero_stride + j] = 0u;
  }
}

template <int NQ, bool WBF16, bool PAGED>
__global__ __launch_bounds__(256, 2) void k_indexer_fp8(IndexerArgs a) {
  zero_side_job(a);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4, c = lane & 15;
  const RowGroup rg = row_group<NQ>(a);
  if (rg.nr <= 0 || rg.b >= a.B) return;
  const int L = clamped_len(a.seq_lens, rg.b, a.S_max);
  const int qi0 = rg.t0 - rg.b * a.q_len;
  int pos[NQ];
#pragma unroll
  for (int r = 0; r < NQ; ++r) pos[r] = (r < rg.nr) ? L - a.q_len + qi0 + r : -1;
  const int maxpos = L - a.q_len + qi0 + rg.nr - 1;

  // This block streams keys [chunk0, chunk1); the four waves interleave
  // 64-key steps so the block reads one contiguous region at a time.
  const int chunk0 = (int)blockIdx.x * kKeysPerChunk;
  const int chunk1 = min(chunk0 + kKeysPerChunk, a.S_max);
  const int kend = min(chunk1, maxpos + 1);  // keys past this are masked for every row
  float* out = a.scores + (long long)(rg.t0 - a.row_begin) * a.ld;

  // Fully masked tail of the chunk: -inf, no scoring.
  for (int s = max(chunk0, kend) + (int)threadIdx.x; s < chunk1; s += 256)
    for (int r = 0; r < rg.nr; ++r) out[(long long)r * a.ld + s] = -INFINITY;
  if (kend <= chunk0) return;
  const int nsteps = (kend - chunk0 + kKeysPerBlock - 1) / kKeysPerBlock;

  const uint8_t* kb = static_cast<const uint8_t*>(a.k) + (PAGED ? 0 : (size_t)rg.b * a.S_max * kDI);
  const float* ksb = a.k_scale ? a.k_scale + (PAGED ? 0 : (size_t)rg.b * a.S_max) : nullptr;
  // Paged caches: a page holds a power of two >= 64 tokens, so the 64 keys
  // of one wave step never straddle a page, and a 2048-key chunk touches at
  // most 32 pages.  Lane i holds the id of the chunk's i-th page (read once),
  // and each step takes its page from the lane by a readlane: no table read
  // sits in front of a key load.
  int page_j0 = 0, lane_page = 0;
  if constexpr (PAGED) {
    page_j0 = chunk0 >> a.pages.shift;
    const int np = ((kend - 1) >> a.pages.shift) - page_j0 + 1;
    lane_page = a.pages.page(rg.b, page_j0 + min(lane, np - 1));
  }
  // Every key load is issued unconditionally (addresses clamped into
  // [chunk0, kend), a missing k-scale read from a unit constant), so the
  // compiler's memory-counter waits stay exact: the next step's keys stay in
  // flight while the current step computes.
  auto load_keys = [&](int step, v8i (&kf)[4], float& ks) {
    const int kw = chunk0 + step * kKeysPerBlock + wave * kKeysPerWave;
    const uint8_t* kwin = kb;
    const float* kswin = ksb;
    if constexpr (PAGED) {
      // the step's keys (clamped like the loads) lie in the 64-key window wb,
      // whose tokens are pool rows s + shift_rows
      const int wb = min(kw, kend - 1) & ~(kKeysPerWave - 1);
      const int pg = __builtin_amdgcn_readlane(lane_page, (wb >> a.pages.shift) - page_j0);
      const long long shift_rows =
          ((long long)pg << a.pages.shift) + (wb & ((1 << a.pages.shift) - 1)) - wb;
      kwin = kb + shift_rows * kDI;
      kswin = ksb ? ksb + shift_rows : nullptr;
    }
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) {
      const int s = min(kw + 16 * blk + c, kend - 1);  // keys past kend are never stored
      kf[blk] = load32(kwin + (size_t)s * kDI + 32 * g);
    }
    const int s_l = min(kw + lane, kend - 1);
    ks = *(kswin ? kswin + s_l : &g_unit_scale);
  };
  v8i kf_a[4], kf_b[4];
  float ks_a, ks_b;
  load_keys(0, kf_a, ks_a);

  // Query fragments (row = head 16m+c, bytes 32g..32g+31) and head weights of
  // the output rows this lane holds (heads 16m + 4g + i).
  const uint8_t* qb = static_cast<const uint8_t*>(a.q);
  v8i qf[NQ][4];
  float wv[NQ][4][4];
#pragma unroll
  for (int r = 0; r < NQ; ++r) {
    const int t = rg.t0 + r;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      qf[r][m] = (r < rg.nr) ? load32(qb + ((size_t)t * kHI + 16 * m + c) * kDI + 32 * g)
                             : v8i{0, 0, 0, 0, 0, 0, 0, 0};
    }
    if (r < rg.nr) {
      load_head_weights(a.w, WBF16, a.q_scale, (size_t)t, g, wv[r]);
    } else {
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) wv[r][m][i] = 0.f;
    }
  }
  // The row-dependent (conditional) loads above are complete before the
  // step loop, so no wait inside it has to cover them.
  __builtin_amdgcn_s_waitcnt(0);

  auto compute = [&](int step, const v8i (&kf)[4], float ks) {
    const int s_l = chunk0 + step * kKeysPerBlock + wave * kKeysPerWave + lane;
    float x[NQ][4];
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) {
#pragma unroll
      for (int r = 0; r < NQ; ++r) {
        float acc = 0.f;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const v4f d = mfma_fp8_16x16x128(qf[r][m], kf[blk]);
#pragma unroll
          for (int i = 0; i < 4; ++i) acc = fmaf(wv[r][m][i], relu(d[i]), acc);
        }
        x[r][blk] = acc;
      }
    }
#pragma unroll
    for (int r = 0; r < NQ; ++r) {
      // Transpose-reduce over the four 16-lane rows: afterwards lane (g, c)
      // holds the head sum of block g, key column c, i.e. key s_l.
      auto p01 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x[r][0]), __float_as_uint(x[r][1]), false, false);
      auto p23 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x[r][2]), __float_as_uint(x[r][3]), false, false);
      const float a01 = __uint_as_float(p01[0]) + __uint_as_float(p01[1]);
      const float a23 = __uint_as_float(p23[0]) + __uint_as_float(p23[1]);
      auto pf = __builtin_amdgcn_permlane32_swap(__float_as_uint(a01), __float_as_uint(a23), false, false);
      const float tot = __uint_as_float(pf[0]) + __uint_as_float(pf[1]);
      if (r < rg.nr && s_l < kend) {
        // a store the compiler does not track: otherwise its pending count
        // would force full memory waits in front of the next step's keys
        const float v = (s_l <= pos[r]) ? tot * ks : -INFINITY;
        store_u32_nowait(reinterpret_cast<uint32_t*>(out + (long long)r * a.ld + s_l), __float_as_uint(v));
      }
    }
  };

  // Two steps per trip with ping-pong key buffers (no register copies); the
  // next step's loads are pinned ahead of the current step's MFMAs, so the
  // waits in front of those MFMAs leave them in flight.  The trip body has
  // no branch around a load (an odd last step is peeled after the loop).
  int step = 0;
  for (; step + 1 < nsteps; step += 2) {
    load_keys(step + 1, kf_b, ks_b);
    __builtin_amdgcn_sched_barrier(0);
    compute(step, kf_a, ks_a);
    __builtin_amdgcn_sched_barrier(0);
    load_keys(step + 2, kf_a, ks_a);
    __builtin_amdgcn_sched_barrier(0);
    compute(step + 1, kf_b, ks_b);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (step < nsteps) compute(step, kf_a, ks_a);
}

// fp32 path (tiny configuration): one block per (row, 256-key tile), the query
// row staged in LDS, one thread per key.
__global__ __launch_bounds__(256) void k_indexer_f32(IndexerArgs a) {
  __shared__ float qs[kHI * kDI];
  __shared__ float wsh[kHI];
  zero_side_job(a);
  const int t = a.row_begin + (int)blockIdx.y;
  const int b = t / a.q_len;
  const int pos = row_pos(a.seq_lens, t, a.q_len, a.S_max);
  const int tile0 = (int)blockIdx.x * 256;
  const int s = tile0 + (int)threadIdx.x;
  float* out = a.scores + (long long)(t - a.row_begin) * a.ld;
  if (tile0 > pos) {
    if (s < a.S_max) out[s] = -INFINITY;
    return;
  }
  const float* qrow = static_cast<const float*>(a.q) + (size_t)t * kHI * kDI;
  for (int e = threadIdx.x; e < kHI * kDI; e += 256) qs[e] = qrow[e];
  if (threadIdx.x < kHI) {
    float wt = a.w_is_bf16 ? bf16_to_f32(static_cast<const uint16_t*>(a.w)[(size_t)t * kHI + threadIdx.x])
                           : static_cast<const float*>(a.w)[(size_t)t * kHI + threadIdx.x];
    if (a.q_scale) wt *= a.q_scale[(size_t)t * kHI + threadIdx.x];
    wsh[threadIdx.x] = wt;
  }
  __syncthreads();
  if (s >= a.S_max) return;
  if (s > pos) {
    out[s] = -INFINITY;
    return;
  }
  const size_t krow = a.pages.table ? (size_t)a.pages.row(b, s) : (size_t)b * a.S_max + s;
  const float4* kr = reinterpret_cast<const float4*>(static_cast<const float*>(a.k) + krow * kDI);
  float kreg[kDI];
#pragma unroll
  for (int d = 0; d < kDI / 4; ++d) {
    const float4 v = kr[d];
    kreg[4 * d] = v.x; kreg[4 * d + 1] = v.y; kreg[4 * d + 2] = v.z; kreg[4 * d + 3] = v.w;
  }
  float score = 0.f;
  for (int j = 0; j < kHI; ++j) {
    float dot = 0.f;
#pragma unroll
    for (int d = 0; d < kDI; ++d) dot = fmaf(qs[j * kDI + d], kreg[d], dot);
    score = fmaf(wsh[j], fmaxf(dot, 0.f), score);
  }
  const float ksc = a.k_scale ? a.k_scale[krow] : 1.0f;
  out[s] = score * ksc;
}

}  // namespace

template <int NQ, bool WBF16>
static void launch_fp8_variant(const IndexerArgs& a, dim3 grid, hipStream_t stream) {
  if (a.pages.table) hipLaunchKernelGGL((k_indexer_fp8<NQ, WBF16, true>), grid, dim3(256), 0, stream, a);
  else hipLaunchKernelGGL((k_indexer_fp8<NQ, WBF16, false>), grid, dim3(256), 0, stream, a);
}

hipError_t launch_indexer_fp8(const IndexerArgs& a, hipStream_t stream) {
  if (a.row_count <= 0) return hipSuccess;
  const int b0 = a.row_begin / a.q_len;
  const int b1 = (a.row_begin + a.row_count - 1) / a.q_len;
  const unsigned gx = (unsigned)((a.S_max + kKeysPerChunk - 1) / kKeysPerChunk);
  if (a.q_len == 1) {
    const dim3 grid(gx, (unsigned)(b1 - b0 + 1));
    if (a.w_is_bf16) launch_fp8_variant<1, true>(a, grid, stream);
    else launch_fp8_variant<1, false>(a, grid, stream);
  } else {
    const int gps = (a.q_len + 1) / 2;
    const dim3 grid(gx, (unsigned)((b1 - b0 + 1) * gps));
    if (a.w_is_bf16) launch_fp8_variant<2, true>(a, grid, stream);
    else launch_fp8_variant<2, false>(a, grid, stream);
  }
  return hipGetLastError();
}

hipError_t launch_indexer_f32(const IndexerArgs& a, hipStream_t stream) {
  if (a.row_count <= 0) return hipSuccess;
  const dim3 grid((unsigned)((a.S_max + 255) / 256), (unsigned)a.row_count);
  hipLaunchKernelGGL(k_indexer_f32, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace dsa
