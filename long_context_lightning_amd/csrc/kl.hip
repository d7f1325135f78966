// Indexer KL objective, forward only ("详解DSA" Eq.(3)-(6)).
//
// For query t over a set of positions (Eq.(5): every s <= pos; Eq.(6): the
// selected S_t):
//   v_s   = sum_h exp(z_h,s - lse_h),  z_h,s = sm_scale * q[t,h] . c_s      (Eq.(3) before normalising)
//   p     = v / V,  V = sum_s v_s;   p_hat = Softmax(I[t, set])            (Eq.(3), (4))
//   KL_t  = sum_s p_s (log p_s - log p_hat_s)
//         = A / V - log V - C / V + lse_I,
// with A = sum_s v_s log v_s, C = sum_s v_s I_s, lse_I = log sum_s exp(I_s);
// the loss is sum_t KL_t (Eq.(5) / (6)).  lse_h is the attention's own
// normaliser (an input, as a training step has it from the attention
// forward); q and the 576-wide latent rows are the MQA-mode attention inputs.
//
// k_kl_partial: a block owns one query row and one split of its set, 4 waves,
// wave w on heads 32w..32w+31.  Per 32-entry tile the latent rows are copied
// global -> LDS (double buffered; dims 0..511 at a 1040-byte row stride so
// the 16 rows one fragment read covers fall on distinct banks, the rope dims
// XOR-swizzled), then D[heads x keys] = Q . K^T on
// v_mfma_f32_16x16x32_bf16 (Q fragments in registers): a lane holds heads
// 4g+i of one key column, so the head sum is in-lane plus two cross-row
// swaps, then across the 4 waves through LDS.  Wave 0 keeps the running
// (V, A, C) and the online log-sum-exp of I.  Per-split partials are merged
// per row by k_kl_combine; k_kl_sum adds the rows in a fixed order.
#include "dsa_internal.h"

namespace dsa {

namespace {

constexpr int kNT = 32;                       // entries per tile
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kMainRS = 1040;                 // LDS stride of dims 0..511 (1024 bytes + 16)
constexpr int kMainBytes = kNT * kMainRS;     // 33280
constexpr int kRopeRS = 128;                  // dims 512..575: 8 pieces, XOR-swizzled
constexpr int kSlotBytes = kMainBytes + kNT * kRopeRS;  // 37376
constexpr int kRows = kNT / kWaves;           // rows gathered per wave per tile (8)
constexpr int kKs = kDQK / 32;                // 18 k-steps (16 over dims 0..511, 2 rope)
constexpr int kKsMain = kDV / 32;
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kPartial = 5;                   // V, A, C, m_I, s_I

__device__ __forceinline__ v4f mfma_bf16(v8bf a, v8bf b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ v8bf as_v8bf(v4i x) { return __builtin_bit_cast(v8bf, x); }

__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Copies of tile rows into a slot: wave w moves rows 8w..8w+7 (positions
// s[r], an invalid entry given as row 0 of the sequence), one instruction per
// row for dims 0..511 and one for the rope dims of its eight rows (row r's
// logical piece p at p ^ ((r >> 1) & 7)).
__device__ __forceinline__ void gather_tile(const uint16_t* kvb, const int (&s)[kRows], uint32_t slot_off, int wave,
                                            int lane) {
  const int row0 = wave * kRows;
#pragma unroll
  for (int r = 0; r < kRows; ++r) dma16_lds_at(kvb + (size_t)s[r] * kDQK + 8 * lane, slot_off + (row0 + r) * kMainRS);
  const int rr = lane >> 3, sl = lane & 7;
  int sr = s[0];
#pragma unroll
  for (int r = 1; r < kRows; ++r) sr = rr == r ? s[r] : sr;
  const int piece = sl ^ (((row0 + rr) >> 1) & 7);
  dma16_lds_at(kvb + (size_t)sr * kDQK + kDV + 8 * piece, slot_off + kMainBytes + row0 * kRopeRS);
}

// DENSE: the set is positions 0, 1, ... (Eq.(5)); otherwise idx (Eq.(6)).
template <bool DENSE>
__global__ __launch_bounds__(kThreads, 2) void k_kl_partial(KlArgs a, int ns, int per_split) {
  __shared__ __attribute__((aligned(16))) unsigned char slots[2 * kSlotBytes];
  __shared__ float red[kWaves][kNT];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, c = lane & 15;
  const int r = blockIdx.x / ns, split = blockIdx.x % ns;
  const int t = a.row_begin + r;
  const int b = t / a.q_len;
  const int pos = row_pos(a.seq_lens, t, a.q_len, a.S_max);
  const int m0 = split * per_split;
  const int m1 = min(a.k, m0 + per_split);
  const int ntiles = (m1 > m0 && pos >= 0) ? (m1 - m0 + kNT - 1) / kNT : 0;
  const uint16_t* kvb = static_cast<const uint16_t*>(a.kv) + (size_t)b * a.S_max * kDQK;
  const int32_t* idx_row = DENSE ? nullptr : a.idx + (size_t)t * a.k;
  const uint32_t slot0 = lds_offset(slots);
  const bool heads_on = 32 * wave < a.H;  // this wave has heads (H is a multiple of 32)

  // Entry m of the set: its raw value is loaded branch-free (m clamped into
  // the split) and checked only where it is used, a tile later, so no load
  // is waited for right after it is issued.
  auto raw_at = [&](int m) -> int {
    const int mc = min(m, m1 - 1);
    return DENSE ? mc : idx_row[mc];
  };
  auto pos_of = [&](int m, int raw) -> int { return (m < m1 && raw >= 0 && raw <= pos) ? raw : -1; };
  auto rows_of = [&](int n, int (&raw)[kRows]) {
#pragma unroll
    for (int rr = 0; rr < kRows; ++rr) raw[rr] = raw_at(m0 + n * kNT + wave * kRows + rr);
  };
  auto gather = [&](int n, const int (&raw)[kRows], uint32_t slot_off) {
    int sp[kRows];
#pragma unroll
    for (int rr = 0; rr < kRows; ++rr) sp[rr] = max(pos_of(m0 + n * kNT + wave * kRows + rr, raw[rr]), 0);
    gather_tile(kvb, sp, slot_off, wave, lane);
  };
  // Every load has a whole tile of compute before its value is used: at the
  // top of tile n one full wait covers tile n's copies and the loads of the
  // step before; then tile n+1's copies go out, the entries of tile n+2 and
  // (wave 0) the scores I of tile n+1 are loaded, and tile n computes.
  // Wave 0 lane l < 32 accumulates entry l of every tile; every lane keeps
  // the raw entries of tiles n and n+1 and the score I of tile n (loaded by
  // all lanes, branch-free).
  const bool acc_lane = wave == 0 && lane < kNT;
  const int el = lane & (kNT - 1);
  const float* irow = a.scores + (size_t)t * a.ld;
  int raw_nx[kRows];
  int e_raw_c = 0, e_raw_n1 = 0;
  float e_i_c = 0.f;
  if (ntiles > 0) {
    int raw0[kRows];
    rows_of(0, raw0);
    rows_of(1, raw_nx);
    e_raw_c = raw_at(m0 + el);
    e_raw_n1 = raw_at(m0 + kNT + el);
    __builtin_amdgcn_s_waitcnt(0);
    gather(0, raw0, slot0);
    e_i_c = irow[max(pos_of(m0 + el, e_raw_c), 0)];
  }

  // Q fragments (A operand: row = head 32w + 16hb + c, dims 32ks + 8g .. +7)
  // and the normalisers of the heads this lane's results cover (4g + i).
  v8bf qf[2][kKs];
  float nl[2][4];
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    const int hq = heads_on ? 32 * wave + 16 * hb + c : 0;
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) + ((size_t)t * a.H + hq) * kDQK + 8 * g;
    // loads issued unconditionally (a wave without heads reads head 0 and
    // discards it), so they all go out before the first wait
#pragma unroll
    for (int ks = 0; ks < kKs; ++ks) qf[hb][ks] = as_v8bf(*reinterpret_cast<const v4i*>(qrow + 32 * ks));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hl = heads_on ? 32 * wave + 16 * hb + 4 * g + i : 0;
      nl[hb][i] = a.lse[(size_t)t * a.H + hl];
    }
  }
  // -lse in log2 units; a head with lse = -inf never weighs anything
#pragma unroll
  for (int hb = 0; hb < 2; ++hb)
#pragma unroll
    for (int i = 0; i < 4; ++i) nl[hb][i] = heads_on ? -nl[hb][i] * kLog2e : -INFINITY;

  const float qk = a.sm_scale * kLog2e;
  float accV = 0.f, accA = 0.f, accC = 0.f, mI = -INFINITY, sI = 0.f;

  for (int n = 0; n < ntiles; ++n) {
    __builtin_amdgcn_s_waitcnt(0);
    if (n + 1 < ntiles) gather(n + 1, raw_nx, slot0 + ((n + 1) & 1) * kSlotBytes);
    rows_of(n + 2, raw_nx);                        // clamped: always a valid address
    const float e_i_n1 = irow[max(pos_of(m0 + (n + 1) * kNT + el, e_raw_n1), 0)];
    const int e_raw_n2 = raw_at(m0 + (n + 2) * kNT + el);
    lds_barrier();  // tile n landed everywhere; slot (n+1)&1 was released after tile n-1
    const unsigned char* tb = slots + (n & 1) * kSlotBytes;
    if (heads_on) {
      // D[hb][kb]: heads 32w + 16hb + 4g + i x keys 16kb + c
      v4f d[2][2];
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) d[hb][0] = d[hb][1] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < kKs; ++ks) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const int row = 16 * kb + c;
          const unsigned char* p =
              ks < kKsMain ? tb + row * kMainRS + 64 * ks + 16 * g
                           : tb + kMainBytes + row * kRopeRS + 16 * ((4 * (ks - kKsMain) + g) ^ ((row >> 1) & 7));
          const v8bf kf = as_v8bf(*reinterpret_cast<const v4i*>(p));
          d[0][kb] = mfma_bf16(qf[0][ks], kf, d[0][kb]);
          d[1][kb] = mfma_bf16(qf[1][ks], kf, d[1][kb]);
        }
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        float e = 0.f;
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
#pragma unroll
          for (int i = 0; i < 4; ++i) e += __builtin_amdgcn_exp2f(fmaf(d[hb][kb][i], qk, nl[hb][i]));
        e += __shfl_xor(e, 16);
        e += __shfl_xor(e, 32);
        if (g == 0) red[wave][16 * kb + c] = e;
      }
    } else if (lane < kNT) {
      red[wave][lane] = 0.f;
    }
    lds_barrier();
    if (acc_lane && pos_of(m0 + n * kNT + el, e_raw_c) >= 0) {
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) v += red[w][lane];
      accV += v;
      if (v > 0.f) accA += v * __logf(v);
      accC += v * e_i_c;
      if (e_i_c > mI) {
        sI = sI * __expf(mI - e_i_c) + 1.f;
        mI = e_i_c;
      } else {
        sI += __expf(e_i_c - mI);
      }
    }
    e_raw_c = e_raw_n1;
    e_raw_n1 = e_raw_n2;
    e_i_c = e_i_n1;
  }

  // wave 0: reduce its 32 lanes and store the split's partial
  if (wave == 0) {
    float V = accV, A = accA, C = accC, m = mI, sm = sI;
#pragma unroll
    for (int o = 16; o > 0; o >>= 1) {
      V += __shfl_xor(V, o);
      A += __shfl_xor(A, o);
      C += __shfl_xor(C, o);
      const float m2 = __shfl_xor(m, o), s2 = __shfl_xor(sm, o);
      const float mm = fmaxf(m, m2);
      sm = (m == -INFINITY ? 0.f : sm * __expf(m - mm)) + (m2 == -INFINITY ? 0.f : s2 * __expf(m2 - mm));
      m = mm;
    }
    if (lane == 0) {
      float* out = a.ws + ((size_t)r * ns + split) * kPartial;
      out[0] = V;
      out[1] = A;
      out[2] = C;
      out[3] = m;
      out[4] = sm;
    }
  }
}

// One thread per row: merge the splits, KL = A/V - log V - C/V + lse_I.
__global__ __launch_bounds__(256) void k_kl_combine(KlArgs a, int ns) {
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r >= a.row_count) return;
  float V = 0.f, A = 0.f, C = 0.f, m = -INFINITY;
  for (int j = 0; j < ns; ++j) m = fmaxf(m, a.ws[((size_t)r * ns + j) * kPartial + 3]);
  float sI = 0.f;
  for (int j = 0; j < ns; ++j) {
    const float* p = a.ws + ((size_t)r * ns + j) * kPartial;
    V += p[0];
    A += p[1];
    C += p[2];
    if (p[3] > -INFINITY) sI += p[4] * __expf(p[3] - m);
  }
  float kl = 0.f;
  if (V > 0.f && sI > 0.f) {
    const float lseI = m + __logf(sI);
    kl = A / V - __logf(V) - C / V + lseI;
  }
  a.kl[r] = kl;
}

// The loss: sum of the per-row values in a fixed order (one block).
__global__ __launch_bounds__(1024) void k_kl_sum(const float* kl, int n, float* loss) {
  __shared__ float part[1024];
  float s = 0.f;
  for (int i = threadIdx.x; i < n; i += 1024) s += kl[i];
  part[threadIdx.x] = s;
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) *loss = part[0];
}

int kl_splits(int rows, int k) {
  int ns = (1024 + rows - 1) / (rows > 0 ? rows : 1);
  const int max_ns = (k + 4 * kNT - 1) / (4 * kNT);  // at least 4 tiles per split
  if (ns > max_ns) ns = max_ns;
  if (ns > 256) ns = 256;
  return ns < 1 ? 1 : ns;
}

}  // namespace

size_t kl_workspace_bytes(int rows, int k) { return (size_t)rows * kl_splits(rows, k) * kPartial * sizeof(float); }

hipError_t launch_indexer_kl(const KlArgs& a, hipStream_t stream) {
  if (a.row_count > 0) {
    const int ns = kl_splits(a.row_count, a.k);
    int per = (a.k + ns - 1) / ns;
    per = (per + kNT - 1) / kNT * kNT;
    if (a.idx)
      hipLaunchKernelGGL(k_kl_partial<false>, dim3((unsigned)(a.row_count * ns)), dim3(kThreads), 0, stream, a, ns, per);
    else
      hipLaunchKernelGGL(k_kl_partial<true>, dim3((unsigned)(a.row_count * ns)), dim3(kThreads), 0, stream, a, ns, per);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_kl_combine, dim3((unsigned)((a.row_count + 255) / 256)), dim3(256), 0, stream, a, ns);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.loss) {
    hipLaunchKernelGGL(k_kl_sum, dim3(1), dim3(1024), 0, stream, a.kl, a.row_count, a.loss);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace dsa
