// Sparse MQA-mode MLA over the selected latent entries.
//
// "详解DSA" Eq.(2): u_t = Attn(h_t, {c_s : s in S_t}); MQA mode (charlestar
// page, "DSA 怎样嵌入 MLA"; luowle page section 3.1): all heads of a query
// share the selected 576-wide latent rows; the key is the whole row, the
// value its first 512 dims; the softmax covers the selected rows only.
//
// bf16 path.  A block owns one query row, one contiguous slice (split) of its
// selected indices and all H heads, with 8 waves, two per SIMD.  Heads come
// in groups of 32; the two waves of a group split the latent dims between
// them: wave half 0 takes score dims 0..287 and value dims 0..255, half 1
// the rest.  The selected rows are gathered 32 at a time (1152 bytes each, in
// 16-byte pieces, straight from global memory into LDS) through a ring of
// three padded tiles, so two tiles are in flight while one computes.
// Per tile and wave:
//   partial S^T[32 keys x 32 heads] = K_tile[32 x 288] . Q^T[288 x 32]
//     (9 K-steps of v_mfma_f32_16x16x32_bf16 per 16-head block; the Q^T
//     fragments live in registers);
//   the two halves swap their partial scores through LDS and add them, so
//     both hold the same full scores and the same softmax weights;
//   softmax in fp32 with base-2 exponents, lane <-> head;
//   O^T[256 dims x 32 heads] += V^T[256 x 32 keys] . P^T[32 keys x 32 heads]:
//     V^T is read with the gfx950 LDS transpose load (ds_read_b64_tr_b16)
//     straight from the row-major tile; P^T is already in the right
//     registers because the score rows of lane row g are keys 4g..4g+3 and
//     16+4g..16+4g+3.
// With one split the block writes the bf16 output and the log-sum-exp; with
// several each split writes its bf16 output normalised by its own sum plus
// (max, sum), and a combine kernel merges them.
#include "dsa_internal.h"

namespace dsa {

namespace {

constexpr int kNT = 32;                          // keys per tile
constexpr int kMainRS = 1056;                    // LDS stride of a row's dims 0..511 (1024 bytes + 32 pad)
constexpr int kMainBytes = kNT * kMainRS;        // 33792
constexpr int kRopeRS = 128;                     // dims 512..575 of a row: 8 pieces, XOR-swizzled
constexpr int kTileBytes = kMainBytes + kNT * kRopeRS;  // 37888
constexpr int kWaves = 8;                        // 4 head groups x 2 dim halves
constexpr int kThreads = kWaves * 64;
constexpr int kRowsPerWave = kNT / kWaves;       // rows of a tile gathered by each wave (4)
constexpr int kDma = kRowsPerWave + 1;           // gather instructions per wave per tile
constexpr int kKsMain = 8;                       // score K-steps per wave over dims 0..511
constexpr int kKsHalf = kKsMain + 1;             // ... plus one over the rope dims 512..575
constexpr int kDbHalf = kDV / 16 / 2;            // 16-dim value blocks per wave (16)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

static_assert(kRowsPerWave * 8 <= 64, "one instruction moves the rope pieces of a wave's rows");

typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v4s lds_v4s;
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ v4f mfma_bf16(v8bf a, v8bf b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ v8bf as_v8bf(v4i x) { return __builtin_bit_cast(v8bf, x); }

// Wait until at most n (0 or kDma) of this wave's vector-memory operations are in flight.
__device__ __forceinline__ void vm_wait(int n) {
  // gfx9 s_waitcnt: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] << 14
  if (n >= kDma)
    __builtin_amdgcn_s_waitcnt((kDma & 15) | ((kDma >> 4) << 14) | 0x70 | 0xF00);
  else
    __builtin_amdgcn_s_waitcnt(0x70 | 0xF00);
}

// Block barrier that leaves vector-memory operations in flight: LDS traffic
// of this wave done (lgkmcnt), then s_barrier.  __syncthreads() would also
// drain the vector-memory counter and stall the gather ring.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }


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

// Gather of one tile: wave w moves tile rows 4w..4w+3 straight into LDS,
// 16 bytes per lane per instruction: one instruction per row for its dims
// 0..511 (64 pieces, row stride kMainRS), and one more whose first 32 lanes
// move the rope pieces (dims 512..575) of the four rows.  Rope piece p of
// row r sits at position p ^ (r & 7) of the row's 128-byte slot, so the
// score reads of 8 consecutive rows hit distinct banks.  Rows past the split
// or not selectable read row 0 of the sequence (a real row whenever the query
// sees any key), so every instruction is issued with the same lanes and the
// wait counts stay exact; the row's validity bit masks its score.
struct TileSrc {
  const uint16_t* kvb;
  const int32_t* idx_row;
  int m1, pos;
};

__device__ __forceinline__ void gather_tile(const TileSrc& src, int mb, unsigned char* tile, unsigned char* vmask,
                                            int wave, int lane) {
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
  if (lane == 0) vmask[wave] = (unsigned char)vbits;  // byte w: validity of rows 4w..4w+3
  const int row0 = wave * kRowsPerWave;
#pragma unroll
  for (int rr = 0; rr < kRowsPerWave; ++rr)
    dma16_lds(src.kvb + (size_t)sidx[rr] * kDQK, 16u * lane, tile + (row0 + rr) * kMainRS);
  // rope pieces: lane l < 32 -> row row0 + l/8, slot l%8
  const int rr = (lane >> 3) & 3;
  const int s = rr == 0 ? sidx[0] : rr == 1 ? sidx[1] : rr == 2 ? sidx[2] : sidx[3];
  const int piece = 64 + ((lane & 7) ^ ((row0 + rr) & 7));
  if (lane < 8 * kRowsPerWave)
    dma16_lds(src.kvb, (uint32_t)s * (2 * kDQK) + 16u * piece, tile + kMainBytes + row0 * kRopeRS);
}

// FULL: H is a multiple of 32, so a wave's second 16-head block exists
// whenever its first does.
template <bool FULL>
__global__ __launch_bounds__(kThreads, 1) void k_mla_bf16(MlaArgs a, const int32_t* __restrict__ idx, int ns,
                                                        int per_split, int per_xcd) {
  __shared__ __attribute__((aligned(16))) unsigned char ring[3 * kTileBytes];
  __shared__ v4f xbuf[kWaves][4][64];  // partial scores swapped between the two halves of a head group
  __shared__ uint64_t vmask[3];  // per ring slot: byte w = validity bits of tile rows 4w..4w+3
  __shared__ int overflow_flag;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave & 3, half = wave >> 2;
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
  // a query that sees no key gathers nothing (its output is zero)
  const int ntiles = (m1 > m0 && pos >= 0) ? (m1 - m0 + kNT - 1) / kNT : 0;
  const int h0 = 32 * grp;
  const bool hb0 = h0 < a.H;                               // this wave has heads
  const bool hb1 = FULL ? hb0 : (h0 + 16 < a.H);           // ... and a second 16-head block

  // Per-lane LDS offsets within a tile (kept as single opaque values so the
  // compiler neither splits nor re-derives them inside the tile loop):
  // score-read row c of key block 0 (dims 0..511 and rope part) and the V^T
  // transpose-read position.
  int aoff = c * kMainRS + 16 * g + 512 * half;
  int roff = kMainBytes + c * kRopeRS + 16 * ((4 * half + g) ^ (c & 7));
  int voff = (4 * g + (c >> 2)) * kMainRS + 8 * (c & 3) + 32 * kDbHalf * half;
  asm volatile("" : "+v"(aoff), "+v"(roff), "+v"(voff));

  TileSrc src;
  src.kvb = static_cast<const uint16_t*>(a.kv) + (size_t)b * a.S_max * kDQK;
  src.idx_row = idx + (size_t)t * a.k;
  src.m1 = m1;
  src.pos = pos;

  // The first two tiles, then the Q^T fragments; the Q load overlaps the
  // gathers.  Lane holds head h0 + 16*hb + c, dims 32*(8*half + i) + 8g .. +7
  // for i < 8 and rope dims 32*(16 + half) + 8g .. +7 for i = 8.
  if (ntiles > 0) gather_tile(src, m0, ring, reinterpret_cast<unsigned char*>(&vmask[0]), wave, lane);
  if (ntiles > 1) gather_tile(src, m0 + kNT, ring + kTileBytes, reinterpret_cast<unsigned char*>(&vmask[1]), wave, lane);
  v8bf qf[2][kKsHalf];
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    const bool on = hb ? hb1 : hb0;
    const uint16_t* qrow =
        static_cast<const uint16_t*>(a.q) + ((size_t)t * a.H + (on ? h0 + 16 * hb + c : 0)) * kDQK + 8 * g;
#pragma unroll
    for (int i = 0; i < kKsHalf; ++i) {
      const int ks = i < kKsMain ? kKsMain * half + i : 2 * kKsMain + half;
      qf[hb][i] = on ? as_v8bf(*reinterpret_cast<const v4i*>(qrow + 32 * ks)) : as_v8bf(v4i{0, 0, 0, 0});
    }
  }
  vm_wait(0);  // Q and the first two tiles have landed

  // Softmax reference: m_ref is fixed at the first tile with a valid key and
  // never moved, so the accumulators are never rescaled.  Later scores may
  // exceed it by up to 2^64, which fp32 and bf16 carry exactly as ordinary
  // numbers.  If a score goes beyond that headroom the block reruns its split
  // once with m_ref set to the true maximum seen in the first run.
  float m_ref[2] = {-INFINITY, -INFINITY}, m_seen[2] = {-INFINITY, -INFINITY}, l_part[2] = {0.f, 0.f};
  v4f acc_o[kDbHalf][2];
  const float qk_scale = a.sm_scale * kLog2e;
  bool overflow = false;

  // The loops below are software-pipelined by hand: LDS reads run a few
  // steps ahead of the MFMAs that consume them, and sched_barrier fences keep
  // the scheduler from sinking them back next to their uses.
  auto compute = [&](const unsigned char* tb, int q) {
    // partial S^T[key, head] over this wave's share of the score dims; block
    // kb row rho is key 16*kb + rho, so lane row g holds keys 4g..4g+3
    // (kb = 0) and 16+4g..16+4g+3 (kb = 1).  Step n = 9*kb + i.
    v4f sacc[2][2];
    if (hb0) {
      // rows 16*kb + c: key block 1 is 16 rows further down; (row & 7) is c & 7 for both
      const unsigned char* arow = tb + aoff;
      const unsigned char* rrow = tb + roff;
      auto aload = [&](int n) -> v8bf {
        const int kb = n / kKsHalf, i = n % kKsHalf;
        const unsigned char* p = i < kKsMain ? arow + 16 * kMainRS * kb + 64 * i : rrow + 16 * kRopeRS * kb;
        return as_v8bf(*reinterpret_cast<const v4i*>(p));
      };
      constexpr int kAhead = 3;
      v8bf af[kAhead];
#pragma unroll
      for (int n = 0; n < kAhead; ++n) af[n] = aload(n);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) sacc[kb][0] = sacc[kb][1] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int n = 0; n < 2 * kKsHalf; ++n) {
        __builtin_amdgcn_sched_barrier(0);
        const int kb = n / kKsHalf, i = n % kKsHalf;
        sacc[kb][0] = mfma_bf16(af[n % kAhead], qf[0][i], sacc[kb][0]);
        if (hb1) sacc[kb][1] = mfma_bf16(af[n % kAhead], qf[1][i], sacc[kb][1]);
        if (n + kAhead < 2 * kKsHalf) af[n % kAhead] = aload(n + kAhead);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < 4; ++j) xbuf[wave][j][lane] = sacc[j >> 1][j & 1];
    }
    lds_barrier();  // both halves' partial scores are in LDS
    if (!hb0) return;
#pragma unroll
    for (int j = 0; j < 4; ++j) sacc[j >> 1][j & 1] += xbuf[wave ^ 4][j][lane];
    // Scores of lane row g: sv[4*kb + i] is key 4g + 16*kb + i, whose
    // validity bit is bit i of byte g + 4*kb of the slot's mask.  Masked keys
    // become -inf through a bit select (km[j] is all ones for a valid key).
    const uint64_t vm = vmask[q];
    const uint32_t vl[2] = {(uint32_t)vm >> (8 * g), (uint32_t)(vm >> 32) >> (8 * g)};
    uint32_t km[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) km[j] = (uint32_t)((int32_t)(vl[j >> 2] << (31 - (j & 3))) >> 31);
    v8bf pf[2];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      float sv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        sv[j] = __uint_as_float((km[j] & __float_as_uint(sacc[j >> 2][hb][j & 3])) | (~km[j] & 0xFF800000u));
      float tmax = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])), fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
      tmax = max_xor32(max_xor16(tmax)) * qk_scale;  // the scale is positive: max commutes with it
      m_seen[hb] = fmaxf(m_seen[hb], tmax);
      if (m_ref[hb] == -INFINITY) m_ref[hb] = tmax;  // nothing accumulated yet
      overflow = overflow || (tmax > m_ref[hb] + 64.f);
      // p = 2^(s*scale - m_ref) rounded to bf16 (RNE, two per conversion); the
      // normaliser sums the same rounded weights the PV product uses, so the
      // output is an exact convex combination of value rows.  Without a
      // reference yet every p is 0.  A score past the headroom may give inf
      // here; that pass is discarded and rerun.
      const float nmr = m_ref[hb] == -INFINITY ? -INFINITY : -m_ref[hb];
      uint32_t pk[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(sv[2 * j], qk_scale, nmr));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(sv[2 * j + 1], qk_scale, nmr));
        pk[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f){p0, p1}, v2bf));
      }
      float psum = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) psum += __uint_as_float(pk[j] << 16) + __uint_as_float(pk[j] & 0xFFFF0000u);
      l_part[hb] += psum;
      v4i pw = {(int)pk[0], (int)pk[1], (int)pk[2], (int)pk[3]};
      pf[hb] = as_v8bf(pw);
    }
    // O^T[dims, heads] += V^T[dims, keys] . P^T[keys, heads].  V^T fragments
    // (16 dims x keys {4g..4g+3, 16+4g..16+4g+3} for lane row g) are two LDS
    // transpose loads each: lane j of a 16-lane row supplies key kbase + j/4,
    // dims 16db + 4*(j%4) .. +3.
    const unsigned char* v0 = tb + voff;
    const unsigned char* v1 = v0 + 16 * kMainRS;
    constexpr int kVAhead = 4;
    v4s vlo[kVAhead], vhi[kVAhead];
#pragma unroll
    for (int db = 0; db < kVAhead; ++db) {
      vlo[db] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(v0 + 32 * db));
      vhi[db] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(v1 + 32 * db));
    }
#pragma unroll
    for (int db = 0; db < kDbHalf; ++db) {
      __builtin_amdgcn_sched_barrier(0);
      const int sl = db % kVAhead;
      const v8bf av =
          __builtin_bit_cast(v8bf, __builtin_shufflevector(vlo[sl], vhi[sl], 0, 1, 2, 3, 4, 5, 6, 7));
      acc_o[db][0] = mfma_bf16(av, pf[0], acc_o[db][0]);
      if (hb1) acc_o[db][1] = mfma_bf16(av, pf[1], acc_o[db][1]);
      if (db + kVAhead < kDbHalf) {
        vlo[sl] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(v0 + 32 * (db + kVAhead)));
        vhi[sl] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(v1 + 32 * (db + kVAhead)));
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  for (int pass = 0; pass < 2; ++pass) {
    if (pass == 1) {  // rerun with the true maxima as references (no score can exceed them)
      m_ref[0] = m_seen[0];
      m_ref[1] = m_seen[1];
      overflow = false;
      __syncthreads();
      if (ntiles > 0) gather_tile(src, m0, ring, reinterpret_cast<unsigned char*>(&vmask[0]), wave, lane);
      if (ntiles > 1) gather_tile(src, m0 + kNT, ring + kTileBytes, reinterpret_cast<unsigned char*>(&vmask[1]), wave, lane);
    }
#pragma unroll
    for (int db = 0; db < kDbHalf; ++db) acc_o[db][0] = acc_o[db][1] = v4f{0.f, 0.f, 0.f, 0.f};
    l_part[0] = l_part[1] = 0.f;
    if (tid == 0) overflow_flag = 0;
    // Ring step: wait for this wave's share of tile tt, barrier (all shares
    // landed; everyone is done with tile tt-1), refill the freed slot with
    // tile tt+2, compute tile tt.  Every wave takes both barriers of a step.
    int q = 0;  // ring slot of tile tt
    for (int tt = 0; tt < ntiles; ++tt) {
      vm_wait(tt + 1 < ntiles ? kDma : 0);
      lds_barrier();
      const int qn = q == 0 ? 2 : q - 1;  // slot of tile tt+2 (= slot of tile tt-1)
      if (tt + 2 < ntiles) gather_tile(src, m0 + (tt + 2) * kNT, ring + qn * kTileBytes, reinterpret_cast<unsigned char*>(&vmask[qn]), wave, lane);
      compute(ring + q * kTileBytes, q);
      q = q == 2 ? 0 : q + 1;
    }
    __syncthreads();
    if (overflow) overflow_flag = 1;
    __syncthreads();
    if (!overflow_flag) break;
  }

  if (!hb0) return;
  // Output through LDS (the ring is free now): each wave stages one 16-head
  // block at a time as rows of 256 dims, then stores whole 512-byte half rows.
  constexpr int kStageRS = 512 + 16;
  unsigned char* stage = ring + wave * 16 * kStageRS;
  const Partials P = partials(a, ns);
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    if (hb == 1 && !hb1) break;
    const int head = h0 + 16 * hb + c;
    const float l_tot = sum_xor32(sum_xor16(l_part[hb]));
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (g == 0 && half == 0) {
      if (ns == 1) {
        if (a.lse) a.lse[(size_t)t * a.H + head] = l_tot > 0.f ? (m_ref[hb] + log2f(l_tot)) * kLn2 : -INFINITY;
      } else {
        float* pml = P.ml + (((size_t)r * ns + split) * a.H + head) * 2;
        pml[0] = l_tot > 0.f ? m_ref[hb] : -INFINITY;
        pml[1] = l_tot;
      }
    }
#pragma unroll
    for (int db = 0; db < kDbHalf; ++db) {
      v2i st;
      st[0] = (int)((uint32_t)f32_to_bf16_rne(acc_o[db][hb][0] * inv) |
                    ((uint32_t)f32_to_bf16_rne(acc_o[db][hb][1] * inv) << 16));
      st[1] = (int)((uint32_t)f32_to_bf16_rne(acc_o[db][hb][2] * inv) |
                    ((uint32_t)f32_to_bf16_rne(acc_o[db][hb][3] * inv) << 16));
      *reinterpret_cast<v2i*>(stage + c * kStageRS + 2 * (16 * db + 4 * g)) = st;
    }
    // the stage is private to this wave: its own LDS writes complete in order
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int hr = 2 * j + (lane >> 5);
      const v4i v = *reinterpret_cast<const v4i*>(stage + hr * kStageRS + 16 * (lane & 31));
      const int hh = h0 + 16 * hb + hr;
      uint16_t* orow = ns == 1 ? static_cast<uint16_t*>(a.out) + ((size_t)t * a.H + hh) * kDV
                               : P.o + (((size_t)r * ns + split) * a.H + hh) * kDV;
      *reinterpret_cast<v4i*>(orow + 256 * half + 8 * (lane & 31)) = v;
    }
  }
}

// Merge split partials: each split stored its output normalised by its own
// sum l_s together with (m_s, l_s); out = sum_s 2^(m_s-M) l_s o_s / sum_s 2^(m_s-M) l_s.
// A block covers one row and 16 heads; 16 threads per head, 32 dims each.
// All of a thread's partial loads are issued before any is used.
constexpr int kCombineMaxSplits = 8;
__global__ __launch_bounds__(256) void k_mla_combine(MlaArgs a, int ns) {
  const int hg = a.H / 16;
  const int r = (int)blockIdx.x / hg;
  const int h = ((int)blockIdx.x % hg) * 16 + (int)threadIdx.x / 16;
  const int d = 32 * ((int)threadIdx.x % 16);
  const int t = a.row_begin + r;
  const Partials P = partials(a, ns);
  float ms[kCombineMaxSplits], ls[kCombineMaxSplits];
  v4i o[kCombineMaxSplits][4];
#pragma unroll
  for (int s = 0; s < kCombineMaxSplits; ++s) {
    if (s < ns) {
      const float* ml = P.ml + (((size_t)r * ns + s) * a.H + h) * 2;
      ms[s] = ml[0];
      ls[s] = ml[1];
      const v4i* src = reinterpret_cast<const v4i*>(P.o + (((size_t)r * ns + s) * a.H + h) * kDV + d);
#pragma unroll
      for (int i = 0; i < 4; ++i) o[s][i] = src[i];
    }
  }
  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < kCombineMaxSplits; ++s)
    if (s < ns) M = fmaxf(M, ms[s]);
  float wsum = 0.f;
  float acc[32];
#pragma unroll
  for (int e = 0; e < 32; ++e) acc[e] = 0.f;
#pragma unroll
  for (int s = 0; s < kCombineMaxSplits; ++s) {
    if (s < ns && ms[s] != -INFINITY) {
      const float wgt = exp2f(ms[s] - M) * ls[s];
      wsum += wgt;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t u = (uint32_t)o[s][i][j];
          acc[8 * i + 2 * j] += wgt * __uint_as_float(u << 16);
          acc[8 * i + 2 * j + 1] += wgt * __uint_as_float(u & 0xFFFF0000u);
        }
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  v4i* orow = reinterpret_cast<v4i*>(static_cast<uint16_t*>(a.out) + ((size_t)t * a.H + h) * kDV + d);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v4i st;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      st[j] = (int)((uint32_t)f32_to_bf16_rne(acc[8 * i + 2 * j] * inv) |
                    ((uint32_t)f32_to_bf16_rne(acc[8 * i + 2 * j + 1] * inv) << 16));
    orow[i] = st;
  }
  if (a.lse && (threadIdx.x % 16) == 0)
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
  if (ns > 1)
    hipLaunchKernelGGL(k_mla_combine, dim3((unsigned)(a.row_count * (a.H / 16))), dim3(256), 0, stream, a, ns);
  return hipGetLastError();
}

hipError_t launch_mla_f32(const MlaArgs& a, hipStream_t stream) {
  if (a.row_count <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_mla_f32, dim3((unsigned)a.H, (unsigned)a.row_count), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace dsa
