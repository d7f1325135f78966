// Sparse MQA-mode MLA over the selected latent entries.
//
// "详解DSA" Eq.(2): u_t = Attn(h_t, {c_s : s in S_t}); MQA mode (charlestar
// page, "DSA 怎样嵌入 MLA"; luowle page section 3.1): all heads of a query
// share the selected 576-wide latent rows; the key is the whole row, the
// value its first 512 dims; the softmax covers the selected rows only.
//
// bf16 path.  A block owns one query row and one contiguous slice (split) of
// its selected indices, and all H heads: wave w owns heads 16w..16w+15.  The
// selected rows are gathered 32 at a time (1152 bytes each, 16-byte pieces,
// coalesced per row) into a padded LDS tile, double buffered with register
// prefetch so the next gather is in flight while the current tile computes.
// Per tile and wave:
//   S^T[32 keys x 16 heads] = K_tile[32 x 576] . Q^T[576 x 16]   (18 K-steps
//     of v_mfma_f32_16x16x32_bf16; Q^T lives in registers)
//   online softmax in fp32 (base-2 exponent), lane <-> head so the running
//     max / sum need no cross-lane traffic except one reduction per tile;
//   O^T[512 x 16] += V^T[512 x 32] . P^T[32 x 16]: the V^T operand is read
//     with the gfx950 LDS transpose load (ds_read_b64_tr_b16) straight from
//     the row-major tile, and P^T is the softmax result already sitting in
//     the right registers because the S^T rows were assigned to keys so that
//     lane row g holds keys 8g..8g+7.
// With one split the block writes bf16 output and the log-sum-exp; with
// several it writes fp32 partials (unnormalised O, running max, running sum)
// and a combine kernel merges them.
#include "dsa_internal.h"

namespace dsa {

namespace {

constexpr int kNT = 32;                 // keys per tile
constexpr int kRowBytes = kDQK * 2;     // 1152
constexpr int kRS = kRowBytes + 16;     // padded LDS row stride (bank spread)
constexpr int kPieces = kNT * (kRowBytes / 16);  // 16-byte pieces per tile (2304)
constexpr int kThreads = 512;
constexpr int kPPT = (kPieces + kThreads - 1) / kThreads;  // 5
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef __attribute__((address_space(3))) v4s lds_v4s;

__device__ __forceinline__ v4f mfma_bf16(v8bf a, v8bf b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ v8bf as_v8bf(v4i x) { return __builtin_bit_cast(v8bf, x); }

// Partition of one row's k indices into splits of whole tiles.
__host__ __device__ inline int mla_splits(int T, int k) {
  int ns = 256 / (T > 0 ? T : 1);
  if (ns < 1) ns = 1;
  if (ns > 8) ns = 8;
  const int max_ns = (k + 4 * kNT - 1) / (4 * kNT);  // at least 4 tiles per split
  if (ns > max_ns) ns = max_ns;
  return ns < 1 ? 1 : ns;
}
__host__ __device__ inline int mla_per_split(int k, int ns) {
  int per = (k + ns - 1) / ns;
  return (per + kNT - 1) / kNT * kNT;
}

struct Partials {
  float* o;   // [T][ns][H][512]
  float* ml;  // [T][ns][H][2]  (running max in log2 units, running sum)
};

__device__ __forceinline__ Partials partials(const MlaArgs& a, int ns) {
  Partials p;
  const size_t T = (size_t)a.row_count;
  p.o = static_cast<float*>(a.ws);
  p.ml = p.o + T * ns * a.H * kDV;
  return p;
}

__global__ __launch_bounds__(kThreads) void k_mla_bf16(MlaArgs a, int ns, int per_split) {
  __shared__ __attribute__((aligned(16))) unsigned char tile[2][kNT * kRS];
  __shared__ int vflag[2][kNT];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int r = (int)blockIdx.x / ns;       // row within this launch
  const int split = (int)blockIdx.x % ns;
  const int t = a.row_begin + r;
  const int b = t / a.q_len;
  const int pos = row_pos(a.seq_lens, t, a.q_len, a.S_max);
  const int m0 = split * per_split;
  const int m1 = min(a.k, m0 + per_split);
  const int ntiles = m1 > m0 ? (m1 - m0 + kNT - 1) / kNT : 0;
  const bool active = wave * 16 < a.H;
  const int head = wave * 16 + c;

  const int32_t* idx_row = a.idx + (size_t)t * a.k;
  const uint16_t* kvb = static_cast<const uint16_t*>(a.kv) + (size_t)b * a.S_max * kDQK;

  // ---- Q^T fragments: lane holds head (16w + c), dims 32ks + 8g .. +7
  v8bf qf[kDQK / 32];
  if (active) {
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) + ((size_t)t * a.H + head) * kDQK + 8 * g;
#pragma unroll
    for (int ks = 0; ks < kDQK / 32; ++ks) qf[ks] = as_v8bf(*reinterpret_cast<const v4i*>(qrow + 32 * ks));
  }

  // ---- gather helpers
  v4i pre[kPPT];
  auto gather = [&](int tile_i) {
    const int mb = m0 + tile_i * kNT;
#pragma unroll
    for (int j = 0; j < kPPT; ++j) {
      const int p = tid + j * kThreads;
      v4i v = {0, 0, 0, 0};
      if (p < kPieces) {
        const int row = p / (kRowBytes / 16), q = p % (kRowBytes / 16);
        const int m = mb + row;
        const int s = (m < m1) ? idx_row[m] : -1;
        if (s >= 0 && s <= pos) v = *reinterpret_cast<const v4i*>(kvb + (size_t)s * kDQK + 8 * q);
      }
      pre[j] = v;
    }
  };
  auto stage = [&](int tile_i, int buf) {
    const int mb = m0 + tile_i * kNT;
#pragma unroll
    for (int j = 0; j < kPPT; ++j) {
      const int p = tid + j * kThreads;
      if (p < kPieces) {
        const int row = p / (kRowBytes / 16), q = p % (kRowBytes / 16);
        *reinterpret_cast<v4i*>(&tile[buf][row * kRS + 16 * q]) = pre[j];
      }
    }
    if (tid < kNT) {
      const int m = mb + tid;
      const int s = (m < m1) ? idx_row[m] : -1;
      vflag[buf][tid] = (s >= 0 && s <= pos);
    }
  };

  // ---- running softmax state (per lane: head c; partial sum over own keys)
  float m_run = -INFINITY, l_part = 0.f;
  v4f acc_o[kDV / 16];
#pragma unroll
  for (int db = 0; db < kDV / 16; ++db) acc_o[db] = v4f{0.f, 0.f, 0.f, 0.f};
  const float qk_scale = a.sm_scale * kLog2e;

  if (ntiles > 0) {
    gather(0);
    stage(0, 0);
  }
  __syncthreads();
  for (int ti = 0; ti < ntiles; ++ti) {
    const int buf = ti & 1;
    if (ti + 1 < ntiles) gather(ti + 1);
    if (active) {
      const unsigned char* tb = tile[buf];
      // S^T blocks: block kb row rho <-> key 8*(rho/4) + 4*kb + rho%4
      v4f sacc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int rho = c;  // A-operand row of this lane
        const int key = 8 * (rho >> 2) + 4 * kb + (rho & 3);
        const unsigned char* arow = tb + key * kRS + 16 * g;
        v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < kDQK / 32; ++ks) {
          const v8bf av = as_v8bf(*reinterpret_cast<const v4i*>(arow + 64 * ks));
          acc = mfma_bf16(av, qf[ks], acc);
        }
        sacc[kb] = acc;
      }
      // lane (g, c): head c, keys 8g + 4kb + i
      float sv[8];
      float tmax = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = 8 * g + 4 * kb + i;
          const float v = vflag[buf][key] ? sacc[kb][i] * qk_scale : -INFINITY;
          sv[4 * kb + i] = v;
          tmax = fmaxf(tmax, v);
        }
      tmax = max_xor16(tmax);
      tmax = max_xor32(tmax);
      const float m_new = fmaxf(m_run, tmax);
      float alpha = 1.f;
      if (m_new != -INFINITY) {
        alpha = exp2f(m_run - m_new);  // m_run == -inf gives 0
        float psum = 0.f;
        uint16_t pb[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          // the normaliser sums the same bf16-rounded weights the PV product uses,
          // so the output stays an exact convex combination of the value rows
          pb[j] = f32_to_bf16_rne(exp2f(sv[j] - m_new));
          psum += bf16_to_f32(pb[j]);
        }
        l_part = l_part * alpha + psum;
        m_run = m_new;
        v4i pk;
        pk[0] = (int)((uint32_t)pb[0] | ((uint32_t)pb[1] << 16));
        pk[1] = (int)((uint32_t)pb[2] | ((uint32_t)pb[3] << 16));
        pk[2] = (int)((uint32_t)pb[4] | ((uint32_t)pb[5] << 16));
        pk[3] = (int)((uint32_t)pb[6] | ((uint32_t)pb[7] << 16));
        const v8bf pf = as_v8bf(pk);
        // O^T += V^T . P^T ; V^T fragment via transpose loads:
        // lane (g, j) supplies key 8g + j/4 (+4), dims 16db + 4*(j%4)
        const unsigned char* vbase0 = tb + (8 * g + (c >> 2)) * kRS + 2 * 4 * (c & 3);
        const unsigned char* vbase1 = vbase0 + 4 * kRS;
#pragma unroll
        for (int db = 0; db < kDV / 16; ++db) {
          const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(vbase0 + 32 * db));
          const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(vbase1 + 32 * db));
          const v8bf av = __builtin_bit_cast(v8bf, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          acc_o[db] = mfma_bf16(av, pf, acc_o[db] * alpha);
        }
      }
    }
    if (ti + 1 < ntiles) stage(ti + 1, buf ^ 1);
    __syncthreads();
  }

  if (!active) return;
  // Reduce the per-lane partial sums over the four lane rows (same head).
  float l_tot = sum_xor32(sum_xor16(l_part));
  if (ns == 1) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    uint16_t* orow = static_cast<uint16_t*>(a.out) + ((size_t)t * a.H + head) * kDV;
#pragma unroll
    for (int db = 0; db < kDV / 16; ++db) {
      const int d = 16 * db + 4 * g;
      v2i st;
      st[0] = (int)((uint32_t)f32_to_bf16_rne(acc_o[db][0] * inv) | ((uint32_t)f32_to_bf16_rne(acc_o[db][1] * inv) << 16));
      st[1] = (int)((uint32_t)f32_to_bf16_rne(acc_o[db][2] * inv) | ((uint32_t)f32_to_bf16_rne(acc_o[db][3] * inv) << 16));
      *reinterpret_cast<v2i*>(orow + d) = st;
    }
    if (a.lse && g == 0)
      a.lse[(size_t)t * a.H + head] = l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
  } else {
    const Partials P = partials(a, ns);
    float* po = P.o + (((size_t)r * ns + split) * a.H + head) * kDV;
#pragma unroll
    for (int db = 0; db < kDV / 16; ++db)
      *reinterpret_cast<v4f*>(po + 16 * db + 4 * g) = acc_o[db];
    if (g == 0) {
      float* pml = P.ml + (((size_t)r * ns + split) * a.H + head) * 2;
      pml[0] = m_run;
      pml[1] = l_tot;
    }
  }
}

// Merge split partials: out = sum_s 2^(m_s-M) O_s / sum_s 2^(m_s-M) l_s.
template <bool BF16>
__global__ __launch_bounds__(128) void k_mla_combine(MlaArgs a, int ns) {
  const int r = (int)blockIdx.x / a.H;
  const int h = (int)blockIdx.x % a.H;
  const int t = a.row_begin + r;
  const Partials P = partials(a, ns);
  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, P.ml[(((size_t)r * ns + s) * a.H + h) * 2]);
  float wsum = 0.f;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  const int d = 4 * threadIdx.x;
  for (int s = 0; s < ns; ++s) {
    const float* ml = P.ml + (((size_t)r * ns + s) * a.H + h) * 2;
    if (ml[0] == -INFINITY) continue;
    const float wgt = exp2f(ml[0] - M);
    wsum += wgt * ml[1];
    const v4f o = *reinterpret_cast<const v4f*>(P.o + (((size_t)r * ns + s) * a.H + h) * kDV + d);
    for (int i = 0; i < 4; ++i) acc[i] += wgt * o[i];
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  if (BF16) {
    uint16_t* orow = static_cast<uint16_t*>(a.out) + ((size_t)t * a.H + h) * kDV + d;
    v2i st;
    st[0] = (int)((uint32_t)f32_to_bf16_rne(acc[0] * inv) | ((uint32_t)f32_to_bf16_rne(acc[1] * inv) << 16));
    st[1] = (int)((uint32_t)f32_to_bf16_rne(acc[2] * inv) | ((uint32_t)f32_to_bf16_rne(acc[3] * inv) << 16));
    *reinterpret_cast<v2i*>(orow) = st;
  }
  if (a.lse && threadIdx.x == 0)
    a.lse[(size_t)t * a.H + h] = wsum > 0.f ? (M + log2f(wsum)) * kLn2 : -INFINITY;
}

// fp32 path: one block per (row, head); scores of the selected rows in LDS.
constexpr int kF32MaxK = 8192;
__global__ __launch_bounds__(256) void k_mla_f32(MlaArgs a) {
  __shared__ float qs[kDQK];
  __shared__ float zs[kF32MaxK];
  __shared__ float red[8];
  const int t = a.row_begin + (int)blockIdx.y;
  const int h = blockIdx.x;
  const int b = t / a.q_len;
  const int pos = row_pos(a.seq_lens, t, a.q_len, a.S_max);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* qrow = static_cast<const float*>(a.q) + ((size_t)t * a.H + h) * kDQK;
  for (int d = tid; d < kDQK; d += 256) qs[d] = qrow[d];
  __syncthreads();
  const float* kvb = static_cast<const float*>(a.kv) + (size_t)b * a.S_max * kDQK;
  const int32_t* idx_row = a.idx + (size_t)t * a.k;
  float lmax = -INFINITY;
  for (int m = tid; m < a.k; m += 256) {
    const int s = idx_row[m];
    float z = -INFINITY;
    if (s >= 0 && s <= pos) {
      const float* kr = kvb + (size_t)s * kDQK;
      float dot = 0.f;
      for (int d = 0; d < kDQK; ++d) dot = fmaf(qs[d], kr[d], dot);
      z = dot * a.sm_scale;
    }
    zs[m] = z;
    lmax = fmaxf(lmax, z);
  }
  for (int o = 32; o > 0; o >>= 1) lmax = fmaxf(lmax, __shfl_xor(lmax, o, 64));
  if (lane == 0) red[wave] = lmax;
  __syncthreads();
  const float M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  float lsum = 0.f;
  for (int m = tid; m < a.k; m += 256) {
    const float p = (zs[m] == -INFINITY) ? 0.f : expf(zs[m] - M);
    zs[m] = p;
    lsum += p;
  }
  for (int o = 32; o > 0; o >>= 1) lsum += __shfl_xor(lsum, o, 64);
  if (lane == 0) red[4 + wave] = lsum;
  __syncthreads();
  const float L = red[4] + red[5] + red[6] + red[7];
  const float inv = L > 0.f ? 1.f / L : 0.f;
  float* orow = static_cast<float*>(a.out) + ((size_t)t * a.H + h) * kDV;
  for (int d = tid; d < kDV; d += 256) {
    float acc = 0.f;
    for (int m = 0; m < a.k; ++m) {
      const float p = zs[m];
      if (p != 0.f) acc = fmaf(p, kvb[(size_t)idx_row[m] * kDQK + d], acc);
    }
    orow[d] = acc * inv;
  }
  if (a.lse && tid == 0) a.lse[(size_t)t * a.H + h] = L > 0.f ? M + logf(L) : -INFINITY;
}

}  // namespace

size_t mla_workspace_bytes(int T, int H, int k, int is_bf16) {
  if (!is_bf16 || T <= 0) return 0;
  const int ns = mla_splits(T, k);
  if (ns == 1) return 0;
  return (size_t)T * ns * H * (kDV + 2) * sizeof(float);
}

bool mla_f32_supported(int k) { return k <= kF32MaxK; }

hipError_t launch_mla_bf16(const MlaArgs& a, hipStream_t stream) {
  if (a.row_count <= 0) return hipSuccess;
  // Splits are sized from the whole launch so partial buffers match the workspace size query.
  const int ns = mla_splits(a.row_count, a.k);
  const int per = mla_per_split(a.k, ns);
  hipLaunchKernelGGL(k_mla_bf16, dim3((unsigned)(a.row_count * ns)), dim3(kThreads), 0, stream, a, ns, per);
  if (ns > 1)
    hipLaunchKernelGGL(k_mla_combine<true>, dim3((unsigned)(a.row_count * a.H)), dim3(128), 0, stream, a, ns);
  return hipGetLastError();
}

hipError_t launch_mla_f32(const MlaArgs& a, hipStream_t stream) {
  if (a.row_count <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_mla_f32, dim3((unsigned)a.H, (unsigned)a.row_count), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace dsa
