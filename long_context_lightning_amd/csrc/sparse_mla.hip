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

constexpr int kNT = 32;                          // keys per tile
constexpr int kRowBytes = kDQK * 2;              // 1152
#ifndef DSA_MLA_PAD_SLOTS
#define DSA_MLA_PAD_SLOTS 1
#endif
constexpr int kSlots = kRowBytes / 16 + DSA_MLA_PAD_SLOTS;  // 72 data slots + padding per LDS row
constexpr int kRS = kSlots * 16;                 // 1168-byte LDS row stride
constexpr int kTileBytes = kNT * kRS;            // 37376
constexpr int kWaves = 4;                        // 32 heads per wave -> up to 128 heads
constexpr int kThreads = kWaves * 64;
constexpr int kRowsPerWave = kNT / kWaves;       // rows of a tile gathered by each wave
constexpr int kWaveSlots = kRowsPerWave * kSlots;
constexpr int kDma = (kWaveSlots + 63) / 64;     // gather instructions per wave per tile (10)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef __attribute__((address_space(3))) v4s lds_v4s;
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ v4f mfma_bf16(v8bf a, v8bf b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ v8bf as_v8bf(v4i x) { return __builtin_bit_cast(v8bf, x); }

// Wait until at most n of this wave's vector-memory operations are in flight.
__device__ __forceinline__ void vm_wait(int n) {
  // gfx9 s_waitcnt: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] << 14
  if (n >= 2 * kDma)
    __builtin_amdgcn_s_waitcnt(((2 * kDma) & 15) | (((2 * kDma) >> 4) << 14) | 0x70 | 0xF00);
  else if (n >= kDma)
    __builtin_amdgcn_s_waitcnt((kDma & 15) | ((kDma >> 4) << 14) | 0x70 | 0xF00);
  else
    __builtin_amdgcn_s_waitcnt(0x70 | 0xF00);
}

// Block barrier for the gather ring: LDS writes of this wave done (lgkmcnt),
// then s_barrier.  Unlike __syncthreads() it does not drain the vector-memory
// counter, so the gathers of later tiles stay in flight across it; each wave
// has already waited (vm_wait) for its own share of the tile being released.
__device__ __forceinline__ void ring_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

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
  uint16_t* o;  // [T][ns][H][512] bf16, normalised by the split's own sum
  float* ml;    // [T][ns][H][2]   (max in log2 units, sum)
};

__device__ __forceinline__ Partials partials(const MlaArgs& a, int ns) {
  Partials p;
  const size_t T = (size_t)a.row_count;
  p.ml = static_cast<float*>(a.ws);
  p.o = reinterpret_cast<uint16_t*>(p.ml + T * ns * a.H * 2);
  return p;
}

// Gather of one tile: wave w moves tile rows 8w..8w+7 (slots j = 0..583 of
// its region; slot 72 of each row is padding) straight into LDS, 16 bytes per
// lane per instruction.  Invalid rows read row 0 of the sequence so every
// instruction is issued with the same lanes (the wait counts stay exact); the
// row's validity bit masks its score.
struct TileSrc {
  const uint16_t* kvb;
  const int32_t* idx_row;
  int m1, pos;
};

__device__ __forceinline__ void gather_tile(const TileSrc& src, int mb, unsigned char* tile, int* vmask, int wave,
                                            int lane) {
  // The indices are wave-uniform: read them with scalar loads so they never
  // enter the vector-memory counter the tile waits are counted on.
  int sidx[kRowsPerWave];
  uint32_t vbits = 0;
#pragma unroll
  for (int rr = 0; rr < kRowsPerWave; ++rr) {
    const int m = __builtin_amdgcn_readfirstlane(mb + wave * kRowsPerWave + rr);
    const int mc = m < src.m1 ? m : src.m1 - 1;
    int s = __builtin_amdgcn_readfirstlane(src.idx_row[mc]);
    s = m < src.m1 ? s : -1;
    const bool ok = s >= 0 && s <= src.pos;
    sidx[rr] = ok ? s : 0;
    vbits |= (ok ? 1u : 0u) << rr;
  }
  if (lane == 0) vmask[wave] = (int)vbits;
  unsigned char* base = tile + wave * kRowsPerWave * kRS;
#pragma unroll
  for (int u = 0; u < kDma; ++u) {
    const int j = 64 * u + lane;
    const int r0 = (64 * u) / kSlots;  // the instruction's lanes fall in rows r0 and r0 + 1
    const int rr = j / kSlots;
    const int piece = j - rr * kSlots;
    const int s = (rr == r0) ? sidx[r0] : sidx[r0 + 1 < kRowsPerWave ? r0 + 1 : r0];
    const int pc = piece < kRowBytes / 16 ? piece : 0;
    const uint16_t* g = src.kvb + (size_t)s * kDQK + 8 * pc;
    if (j < kWaveSlots)
      __builtin_amdgcn_global_load_lds((const void*)g, (lds_void*)(base + 1024 * u), 16, 0, 0);
  }
}

// FULL: every wave owns two 16-head blocks (H a multiple of 32), so the
// second block needs no runtime guard.
template <bool FULL>
__global__ __launch_bounds__(kThreads, 1) void k_mla_bf16(MlaArgs a, const int32_t* __restrict__ idx, int ns,
                                                        int per_split, int per_xcd) {
  __shared__ __attribute__((aligned(16))) unsigned char tile0[kTileBytes];
  __shared__ __attribute__((aligned(16))) unsigned char tile1[kTileBytes];
  __shared__ __attribute__((aligned(16))) unsigned char tile2[kTileBytes];
  __shared__ __attribute__((aligned(16))) unsigned char tile3[kTileBytes];
  __shared__ int vmask[4][kWaves];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, c = lane & 15;
  // Blocks go round-robin over the 8 XCDs; give each XCD whole queries so the
  // splits of one query share that XCD's L2 (its query rows are read once).
  const int li = ((int)blockIdx.x % 8) * per_xcd + (int)blockIdx.x / 8;
  if (li >= a.row_count * ns) return;
  const int r = li / ns, split = li % ns;
  const int t = a.row_begin + r;
  const int b = t / a.q_len;
  const int pos = row_pos(a.seq_lens, t, a.q_len, a.S_max);
  const int m0 = split * per_split;
  const int m1 = min(a.k, m0 + per_split);
  const int ntiles = m1 > m0 ? (m1 - m0 + kNT - 1) / kNT : 0;
  const int h0 = 32 * wave;
  const bool hb0 = h0 < a.H, hb1 = FULL || (h0 + 16 < a.H);  // head blocks of this wave

  TileSrc src;
  src.kvb = static_cast<const uint16_t*>(a.kv) + (size_t)b * a.S_max * kDQK;
  src.idx_row = idx + (size_t)t * a.k;
  src.m1 = m1;
  src.pos = pos;

  // Q^T fragments: lane holds head h0 + 16*hb + c, dims 32ks + 8g .. +7.
  v8bf qf[2][kDQK / 32];
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    const bool on = hb ? hb1 : hb0;
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) + ((size_t)t * a.H + h0 + 16 * hb + c) * kDQK + 8 * g;
#pragma unroll
    for (int ks = 0; ks < kDQK / 32; ++ks)
      qf[hb][ks] = on ? as_v8bf(*reinterpret_cast<const v4i*>(qrow + 32 * ks)) : as_v8bf(v4i{0, 0, 0, 0});
  }

  // Q must be resident before the gather ring starts counting its own loads.
  __builtin_amdgcn_s_waitcnt(0x70 | 0xF00);  // vmcnt(0)

  // Zero the ring so rows never written hold finite values.
  {
    const v4i z = {0, 0, 0, 0};
    for (int i = tid; i < kTileBytes / 16; i += kThreads) {
      reinterpret_cast<v4i*>(tile0)[i] = z;
      reinterpret_cast<v4i*>(tile1)[i] = z;
      reinterpret_cast<v4i*>(tile2)[i] = z;
      reinterpret_cast<v4i*>(tile3)[i] = z;
    }
  }
  // Softmax reference: m_ref is fixed at the first tile with a valid key and
  // never moved, so the accumulators are never rescaled (they stay in the
  // MFMA accumulator registers).  Later scores may exceed it by up to 2^64,
  // which fp32 and bf16 carry exactly as ordinary numbers.  If a score goes
  // beyond that headroom the block reruns its split once with m_ref set to the
  // true maximum seen in the first run.
  float m_ref[2] = {-INFINITY, -INFINITY}, m_seen[2] = {-INFINITY, -INFINITY}, l_part[2] = {0.f, 0.f};
  v4f acc_o[kDV / 16][2];
  const float qk_scale = a.sm_scale * kLog2e;
  __shared__ int overflow_flag;
  bool overflow = false;

  auto compute = [&](const unsigned char* tb, uint32_t valid) {
    // S^T[key, head]: block kb row rho <-> key 4*(rho/4) + 16*kb + rho%4, so
    // lane row g holds keys 4g..4g+3 and 16+4g..16+4g+3 of the tile.
    v4f sacc[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int key = 4 * (c >> 2) + 16 * kb + (c & 3);
      const unsigned char* arow = tb + key * kRS + 16 * g;
      v4f s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < kDQK / 32; ++ks) {
        const v8bf av = as_v8bf(*reinterpret_cast<const v4i*>(arow + 64 * ks));
        s0 = mfma_bf16(av, qf[0][ks], s0);
        if (hb1) s1 = mfma_bf16(av, qf[1][ks], s1);
      }
      sacc[kb][0] = s0;
      sacc[kb][1] = s1;
    }
    v8bf pf[2];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      float sv[8];
      float tmax = -INFINITY;
      if (valid == 0xFFFFFFFFu) {  // full tile: no masking
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            sv[4 * kb + i] = sacc[kb][hb][i] * qk_scale;
            tmax = fmaxf(tmax, sv[4 * kb + i]);
          }
      } else {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = 4 * g + 16 * kb + i;
            const float v = ((valid >> key) & 1u) ? sacc[kb][hb][i] * qk_scale : -INFINITY;
            sv[4 * kb + i] = v;
            tmax = fmaxf(tmax, v);
          }
      }
      tmax = max_xor32(max_xor16(tmax));
      m_seen[hb] = fmaxf(m_seen[hb], tmax);
      if (m_ref[hb] == -INFINITY) m_ref[hb] = tmax;  // nothing accumulated yet
      if (tmax > m_ref[hb] + 64.f) overflow = true;
      // p = 2^(s - m_ref) rounded to bf16 (v_exp_f32 + v_cvt_pk_bf16_f32, RNE);
      // the normaliser sums the same rounded weights the PV product uses, so
      // the output is an exact convex combination of value rows.
      const float mr = m_ref[hb] == -INFINITY ? INFINITY : m_ref[hb];  // no reference yet: all p = 0
      v8bf pv;
      float psum = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        pv[j] = (__bf16)__builtin_amdgcn_exp2f(fminf(sv[j] - mr, 64.f));
        psum += (float)pv[j];
      }
      l_part[hb] += psum;
      pf[hb] = pv;
    }
    // O^T[dims, heads] += V^T[dims, keys] . P^T[keys, heads].  The V^T
    // fragment (16 dims x keys {4g..4g+3, 16+4g..16+4g+3} for lane row g) is
    // two LDS transpose loads: lane j of a 16-lane row supplies key
    // kbase + j/4, dims 16db + 4*(j%4) .. +3.
    const unsigned char* v0 = tb + (4 * g + (c >> 2)) * kRS + 8 * (c & 3);
    const unsigned char* v1 = v0 + 16 * kRS;
#pragma unroll
    for (int db = 0; db < kDV / 16; ++db) {
      const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(v0 + 32 * db));
      const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(v1 + 32 * db));
      const v8bf av = __builtin_bit_cast(v8bf, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      acc_o[db][0] = mfma_bf16(av, pf[0], acc_o[db][0]);
      if (hb1) acc_o[db][1] = mfma_bf16(av, pf[1], acc_o[db][1]);
    }
  };

  auto valid_of = [&](int q) -> uint32_t {
    return (uint32_t)vmask[q][0] | ((uint32_t)vmask[q][1] << 8) | ((uint32_t)vmask[q][2] << 16) |
           ((uint32_t)vmask[q][3] << 24);
  };
  // One ring step: wait for this wave's share of tile t, barrier (all shares
  // landed; everyone is done with tile t-1), refill the freed buffer with
  // tile t+3, compute tile t.
  auto step = [&](int tt, unsigned char* cur, int q, unsigned char* nxt, int qn) {
    vm_wait(kDma * min(2, ntiles - 1 - tt));
    ring_barrier();
    if (tt + 3 < ntiles) gather_tile(src, m0 + (tt + 3) * kNT, nxt, vmask[qn], wave, lane);
    if (hb0) compute(cur, valid_of(q));
  };

  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int db = 0; db < kDV / 16; ++db) acc_o[db][0] = acc_o[db][1] = v4f{0.f, 0.f, 0.f, 0.f};
    l_part[0] = l_part[1] = 0.f;
    if (tid == 0) overflow_flag = 0;
    __syncthreads();
    if (ntiles > 0) gather_tile(src, m0, tile0, vmask[0], wave, lane);
    if (ntiles > 1) gather_tile(src, m0 + kNT, tile1, vmask[1], wave, lane);
    if (ntiles > 2) gather_tile(src, m0 + 2 * kNT, tile2, vmask[2], wave, lane);
    for (int tt = 0; tt < ntiles; tt += 4) {
      step(tt, tile0, 0, tile3, 3);
      if (tt + 1 < ntiles) step(tt + 1, tile1, 1, tile0, 0);
      if (tt + 2 < ntiles) step(tt + 2, tile2, 2, tile1, 1);
      if (tt + 3 < ntiles) step(tt + 3, tile3, 3, tile2, 2);
    }
    if (overflow && lane == 0) overflow_flag = 1;
    __syncthreads();
    if (!overflow_flag) break;
    // rerun with the true maxima as references (no score can exceed them)
    m_ref[0] = m_seen[0];
    m_ref[1] = m_seen[1];
    overflow = false;
    __syncthreads();
  }

  if (!hb0) return;
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    if (hb == 1 && !hb1) break;
    const int head = h0 + 16 * hb + c;
    const float l_tot = sum_xor32(sum_xor16(l_part[hb]));
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    uint16_t* orow;
    if (ns == 1) {
      orow = static_cast<uint16_t*>(a.out) + ((size_t)t * a.H + head) * kDV;
      if (a.lse && g == 0)
        a.lse[(size_t)t * a.H + head] = l_tot > 0.f ? (m_ref[hb] + log2f(l_tot)) * kLn2 : -INFINITY;
    } else {
      const Partials P = partials(a, ns);
      orow = P.o + (((size_t)r * ns + split) * a.H + head) * kDV;
      if (g == 0) {
        float* pml = P.ml + (((size_t)r * ns + split) * a.H + head) * 2;
        pml[0] = l_tot > 0.f ? m_ref[hb] : -INFINITY;
        pml[1] = l_tot;
      }
    }
#pragma unroll
    for (int db = 0; db < kDV / 16; ++db) {
      const int d = 16 * db + 4 * g;
      v2i st;
      st[0] = (int)((uint32_t)f32_to_bf16_rne(acc_o[db][hb][0] * inv) |
                    ((uint32_t)f32_to_bf16_rne(acc_o[db][hb][1] * inv) << 16));
      st[1] = (int)((uint32_t)f32_to_bf16_rne(acc_o[db][hb][2] * inv) |
                    ((uint32_t)f32_to_bf16_rne(acc_o[db][hb][3] * inv) << 16));
      *reinterpret_cast<v2i*>(orow + d) = st;
    }
  }
}

// Merge split partials: each split stored its output normalised by its own
// sum l_s together with (m_s, l_s); out = sum_s 2^(m_s-M) l_s o_s / sum_s 2^(m_s-M) l_s.
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
    const float wgt = exp2f(ml[0] - M) * ml[1];
    wsum += wgt;
    const v2i o = *reinterpret_cast<const v2i*>(P.o + (((size_t)r * ns + s) * a.H + h) * kDV + d);
    acc[0] += wgt * bf16_to_f32((uint16_t)(o[0] & 0xFFFF));
    acc[1] += wgt * bf16_to_f32((uint16_t)((uint32_t)o[0] >> 16));
    acc[2] += wgt * bf16_to_f32((uint16_t)(o[1] & 0xFFFF));
    acc[3] += wgt * bf16_to_f32((uint16_t)((uint32_t)o[1] >> 16));
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  uint16_t* orow = static_cast<uint16_t*>(a.out) + ((size_t)t * a.H + h) * kDV + d;
  v2i st;
  st[0] = (int)((uint32_t)f32_to_bf16_rne(acc[0] * inv) | ((uint32_t)f32_to_bf16_rne(acc[1] * inv) << 16));
  st[1] = (int)((uint32_t)f32_to_bf16_rne(acc[2] * inv) | ((uint32_t)f32_to_bf16_rne(acc[3] * inv) << 16));
  *reinterpret_cast<v2i*>(orow) = st;
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
  return (size_t)T * ns * H * (2 * sizeof(float) + kDV * sizeof(uint16_t));
}

bool mla_f32_supported(int k) { return k <= kF32MaxK; }

hipError_t launch_mla_bf16(const MlaArgs& a, hipStream_t stream) {
  if (a.row_count <= 0) return hipSuccess;
  // Splits are sized from the whole launch so partial buffers match the workspace size query.
  const int ns = mla_splits(a.row_count, a.k);
  const int per = mla_per_split(a.k, ns);
  const int total = a.row_count * ns;
  const int per_xcd = (total + 7) / 8;
  if (a.H % 32 == 0)
    hipLaunchKernelGGL(k_mla_bf16<true>, dim3((unsigned)(8 * per_xcd)), dim3(kThreads), 0, stream, a, a.idx, ns,
                       per, per_xcd);
  else
    hipLaunchKernelGGL(k_mla_bf16<false>, dim3((unsigned)(8 * per_xcd)), dim3(kThreads), 0, stream, a, a.idx, ns,
                       per, per_xcd);
  if (ns > 1) hipLaunchKernelGGL(k_mla_combine, dim3((unsigned)(a.row_count * a.H)), dim3(128), 0, stream, a, ns);
  return hipGetLastError();
}

hipError_t launch_mla_f32(const MlaArgs& a, hipStream_t stream) {
  if (a.row_count <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_mla_f32, dim3((unsigned)a.H, (unsigned)a.row_count), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace dsa
