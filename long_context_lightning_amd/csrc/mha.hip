// MHA-mode MLA prefill for sequences no longer than top-k.
//
// "详解DSA", section "DSA计算流 & 性能分析": prefill inside top-k runs in MHA
// mode; the MLA forward code block there gives the MHA branch: wkv_b turns
// each latent row into per-head [k_nope | v], the key of head h is
// [k_nope_h, k_pe] with k_pe shared by the heads, softmax in fp32 over the
// scores plus the masks, output scores @ v.  With L <= k the top-k keeps
// every position (the charlestar page's short-prompt paragraph: nothing can
// be cut, a masked MHA stands in for DSA), so what remains is causal
// attention over the decompressed keys and values.  Per selected entry MHA
// mode costs 128 x (192 + 128) x 2 flops against 128 x (576 + 512) x 2 in
// MQA mode, which is why the pages take it for short prefills.
//
// Two kernels:
//
// k_mha_decompress: [k_nope | v] = latent . wkv_b^T per head, a bf16 GEMM on
//   v_mfma_f32_16x16x32_bf16.  A block computes 256 positions x the 256
//   output columns of one head (k_nope and v); 8 waves of 64 columns x 128
//   positions, so each copy instruction feeds 8 MFMAs.  64-deep K chunks of
//   both operands go global -> LDS by DMA (double buffered), 16-byte pieces
//   XOR-swizzled so the 16 rows one fragment read covers fall on distinct
//   banks.  Output head-major: k_nope[b][h][s][128], v[b][h][s][128] bf16,
//   staged through LDS so a block writes its two contiguous 64 KB regions in
//   whole 1 KB pieces.
//
// k_mha_attn: one block = one head x 256 consecutive queries of one
//   sequence, 8 waves (two per SIMD) of 32 queries.  Keys stream in 64-key
//   tiles through a 3-slot LDS ring (DMA; a K row is [k_nope_h | k_pe] =
//   384 bytes with XOR-swizzled pieces, a V row 256 bytes padded to 288 so
//   the 8 rows one transpose read covers fall on distinct banks).  Per tile
//   and wave:
//     S^T[64 keys x 32 queries] = K . Q^T   (Q^T fragments in registers),
//   so a lane holds one query column: the online softmax (fp32, base 2) and
//   its rescaling are per lane, and the bf16 weights stay in registers as the
//   B operand of
//     O^T[128 dims x 32 queries] += V^T . P^T
//   with V^T read by the LDS transpose load (keys in the order the score
//   fragments hold them).  The softmax reference moves only when a tile's
//   maximum passes it by more than 2^8, so the accumulators are rarely
//   rescaled; the normaliser sums the bf16-rounded weights the value product
//   uses.  Causal: keys past a query's position are -inf (diagonal tiles
//   only); tiles past a wave's last query are skipped by that wave.
#include "dsa_internal.h"

namespace dsa {

namespace {

typedef __attribute__((address_space(3))) v4s lds_v4s;
typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

constexpr int kDN = 128, kDR = 64, kDQh = kDN + kDR, kDVh = 128, kDL = 512;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ v4f mfma_bf16(v8bf a, v8bf b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ v8bf as_v8bf(v4i x) { return __builtin_bit_cast(v8bf, x); }

template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt has 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00);
}
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// four fp32 -> four bf16 (RNE), packed
__device__ __forceinline__ uint2 pack4_bf16(float x0, float x1, float x2, float x3) {
  const uint32_t lo = __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f){x0, x1}, v2bf));
  const uint32_t hi = __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f){x2, x3}, v2bf));
  return uint2{lo, hi};
}

// ------------------------------------------------------------ decompression

constexpr int kGT = 256;                 // positions per block
constexpr int kGN = 2 * kDVh;            // output columns per block: one head's k_nope and v rows
constexpr int kGK = 64;                  // K depth per stage
constexpr int kGRow = 2 * kGK;           // bytes of one row of a stage (128)
constexpr int kGW = kGN * kGRow;         // W part of a stage (32 KB)
constexpr int kGX = kGT * kGRow;         // latent part of a stage (32 KB)
constexpr int kGStage = kGW + kGX;
constexpr int kGSteps = kDL / kGK;       // 8
constexpr int kGWaves = 8;
constexpr int kGDma = kGStage / 1024 / kGWaves;  // DMA instructions per wave per stage (8)
constexpr int kGORow = 2 * kGN;          // bytes of one output position row in LDS (512)
static_assert(kGT * kGORow <= 2 * kGStage, "the staged output fits in the two stages");

// Stage kc of the block's operands: the head's 256 W rows (output columns)
// then 256 latent rows (positions), 128 bytes per row; lane l of instruction
// i fills 16-byte slot 64i + l of its part, i.e. row r = slot / 8, stored
// piece p = slot % 8, which holds the row's logical piece p ^ ((r >> 1) & 7).
__device__ __forceinline__ void gemm_stage(const MhaArgs& a, int b, int h, int s0, int L, int kc, uint32_t stage_off,
                                           int wave, int lane) {
#pragma unroll
  for (int u = 0; u < kGDma; ++u) {
    const int i = wave * kGDma + u;          // 0..63: 0..31 W, 32..63 latent
    const int slot = 64 * (i & 31) + lane;
    const int r = slot >> 3, p = slot & 7;
    const int piece = p ^ ((r >> 1) & 7);
    const char* src;
    if (i < 32) {
      src = reinterpret_cast<const char*>(a.wkv_b) + (((size_t)h * kGN + r) * kDL + (size_t)kc * kGK + 8 * piece) * 2;
    } else {
      const int s = min(s0 + r, L - 1);
      src = reinterpret_cast<const char*>(a.kv) + (((size_t)b * a.S_max + s) * kDQK + (size_t)kc * kGK + 8 * piece) * 2;
    }
    dma16_lds_at(src, stage_off + (i < 32 ? 0 : kGW) + 1024 * (i & 31));
  }
}

__global__ __launch_bounds__(kGWaves * 64, 1) void k_mha_decompress(MhaArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[2 * kGStage];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, c = lane & 15;
  const int b = blockIdx.z, h = blockIdx.y;
  const int L = clamped_len(a.seq_lens, b, a.S_max);
  const int s0 = blockIdx.x * kGT;
  if (s0 >= L) return;
  const uint32_t base = lds_offset(lds);
  const int wn = wave & 3, wsb = wave >> 2;  // 64-column block, 128-position block

  v4f acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  gemm_stage(a, b, h, s0, L, 0, base, wave, lane);
  for (int kc = 0; kc < kGSteps; ++kc) {
    if (kc + 1 < kGSteps) {
      gemm_stage(a, b, h, s0, L, kc + 1, base + ((kc + 1) & 1) * kGStage, wave, lane);
      vm_wait<kGDma>();
    } else {
      vm_wait<0>();
    }
    lds_barrier();
    const unsigned char* st = lds + (kc & 1) * kGStage;
#pragma unroll
    for (int kk = 0; kk < kGK / 32; ++kk) {
      const int pc = 4 * kk + g;  // logical piece
      v8bf wf[4], xf[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rw = 64 * wn + 16 * i + c;  // output column (W row)
        wf[i] = as_v8bf(*reinterpret_cast<const v4i*>(st + rw * kGRow + 16 * (pc ^ ((rw >> 1) & 7))));
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int rx = 128 * wsb + 16 * j + c;  // position (latent row)
        xf[j] = as_v8bf(*reinterpret_cast<const v4i*>(st + kGW + rx * kGRow + 16 * (pc ^ ((rx >> 1) & 7))));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = mfma_bf16(wf[i], xf[j], acc[i][j]);
    }
    lds_barrier();  // the next step refills this stage
  }
  // The output goes out through LDS (both stages are free after the last
  // step's barrier): position p's row of 256 bf16 columns (k_nope | v, 512
  // bytes) has its 16-byte chunk q at q ^ (p & 31), so the 16 positions one
  // register write covers fall on distinct banks.  The block's k_nope and v
  // outputs are each one contiguous region of the head-major workspace, so
  // the copy-out is whole 1 KB pieces, 16 bytes per lane.
  // acc[i][j][e]: column 64 wn + 16 i + 4 g + e of position 128 wsb + 16 j + c.
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int p = 128 * wsb + 16 * j + c;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int byte = 128 * wn + 32 * i + 8 * g;  // in the position's 512-byte row
      *reinterpret_cast<uint2*>(lds + p * kGORow + 16 * ((byte >> 4) ^ (p & 31)) + (byte & 15)) =
          pack4_bf16(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
    }
  }
  __syncthreads();
  const int nvalid = min(kGT, L - s0);  // positions past the sequence are not written
  const size_t obase = (((size_t)b * a.H + h) * a.S_max + s0) * kDVh;
  uint16_t* const kdst = static_cast<uint16_t*>(a.knope_ws) + obase;
  uint16_t* const vdst = static_cast<uint16_t*>(a.v_ws) + obase;
#pragma unroll 4
  for (int q = (int)threadIdx.x; q < 2 * kGT * 16; q += kGWaves * 64) {
    const int part = q / (kGT * 16), qq = q % (kGT * 16);  // part 0: k_nope, 1: v
    const int p = qq >> 4, cc = qq & 15;                  // position, 16-byte chunk of its 256-byte row
    if (p >= nvalid) continue;
    const v4i val = *reinterpret_cast<const v4i*>(lds + p * kGORow + 16 * ((cc + 16 * part) ^ (p & 31)));
    *reinterpret_cast<v4i*>((part ? vdst : kdst) + (size_t)p * kDVh + 8 * cc) = val;
  }
}

// ------------------------------------------------------------ attention

constexpr int kAW = 8;                    // waves per block (two per SIMD)
constexpr int kAQW = 32;                  // queries per wave
constexpr int kAQ = kAW * kAQW;           // queries per block
constexpr int kAK = 64;                   // keys per tile
constexpr int kKRow = 2 * kDQh;           // 384 bytes: [k_nope_h | k_pe]
constexpr int kKTile = kAK * kKRow;       // 24 KB
constexpr int kVPieces = 18;              // 16 pieces of 16 bytes + 32 bytes of padding
constexpr int kVRow = 16 * kVPieces;      // 288 bytes: consecutive rows 32 bytes apart mod 256
constexpr int kVTile = kAK * kVRow;       // 18 KB
constexpr int kAStage = kKTile + kVTile;  // 42 KB
constexpr int kASlots = 3;
constexpr int kKInstr = kKTile / 1024;    // 24
constexpr int kVInstr = kVTile / 1024;    // 18
constexpr int kAInstr = kKInstr + kVInstr;  // 42: waves 0, 1 issue 6 per tile, the others 5
constexpr float kRescaleMargin = 8.f;     // log2 units the running reference may lag the maximum

// Tile of keys s0 .. s0+63 into a ring slot; wave w issues instructions
// w, w + 8, ...  K slot 64i + l holds row r = slot / 24, stored piece
// p = slot % 24 = logical piece p ^ ((r >> 1) & 7) (pieces 0..15: k_nope of
// head h from the workspace, 16..23: k_pe from the latent cache).  V slot
// 64i' + l holds row r = slot / 18, piece slot % 18 (16, 17: padding, filled
// with a copy of piece 0).  Keys past the sequence read its last row
// (masked later).
__device__ __forceinline__ void attn_tile(const MhaArgs& a, const uint16_t* knope, const uint16_t* vv, int b,
                                          int s0, int L, uint32_t slot_off, int wave, int lane) {
#pragma unroll
  for (int u = 0; u < 6; ++u) {
    const int i = wave + kAW * u;
    if (i >= kAInstr) break;  // wave-uniform
    const char* src;
    uint32_t dst;
    if (i < kKInstr) {
      const int slot = 64 * i + lane;
      const int r = slot / 24, p = slot - 24 * r;
      const int piece = p ^ ((r >> 1) & 7);
      const int s = min(s0 + r, L - 1);
      src = piece < 16 ? reinterpret_cast<const char*>(knope + (size_t)s * kDN + 8 * piece)
                       : reinterpret_cast<const char*>(static_cast<const uint16_t*>(a.kv) +
                                                       ((size_t)b * a.S_max + s) * kDQK + kDL + 8 * (piece - 16));
      dst = slot_off + 1024 * i;
    } else {
      const int iv = i - kKInstr;
      const int slot = 64 * iv + lane;
      const int r = slot / kVPieces, p = slot - kVPieces * r;
      const int s = min(s0 + r, L - 1);
      src = reinterpret_cast<const char*>(vv + (size_t)s * kDVh + (p < 16 ? 8 * p : 0));
      dst = slot_off + kKTile + 1024 * iv;
    }
    dma16_lds_at(src, dst);
  }
}

__global__ __launch_bounds__(kAW * 64, 1) void k_mha_attn(MhaArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char ring[kASlots * kAStage];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, c = lane & 15;
  // Work items go longest query tile first, then (sequence, head).  Blocks
  // are dealt round-robin over the 8 XCDs by their linear index, so taking
  // items in that order gives every XCD an equal share of every query tile
  // (the query tile as the fastest block index would hand all blocks of one
  // tile length to one XCD and leave the short-tile XCDs idle most of the
  // launch).
  const int nbh = (int)(gridDim.y * gridDim.z);
  const int item = (int)(blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z));
  const int qt = (int)gridDim.x - 1 - item / nbh;
  const int h = (item % nbh) % (int)gridDim.y, b = (item % nbh) / (int)gridDim.y;
  const int L = clamped_len(a.seq_lens, b, a.S_max);
  const int i0 = qt * kAQ;                               // first query index within the sequence
  const int i1 = min(i0 + kAQ, a.q_len);
  if (i0 >= i1) return;
  const int pos0 = L - a.q_len;                          // position of query index 0
  const int maxpos = pos0 + i1 - 1;
  const int ntiles = maxpos < 0 ? 0 : maxpos / kAK + 1;
  const int wi0 = i0 + kAQW * wave;                      // this wave's first query index
  const int w_minpos = pos0 + wi0;
  const int w_maxpos = wi0 < i1 ? pos0 + min(wi0 + kAQW, i1) - 1 : -1;  // -1: the wave has no query
  const uint16_t* knope = static_cast<const uint16_t*>(a.knope_ws) + ((size_t)b * a.H + h) * a.S_max * kDN;
  const uint16_t* vv = static_cast<const uint16_t*>(a.v_ws) + ((size_t)b * a.H + h) * a.S_max * kDVh;
  const uint32_t ring_off = lds_offset(ring);

  if (ntiles > 0) attn_tile(a, knope, vv, b, 0, L, ring_off, wave, lane);
  if (ntiles > 1) attn_tile(a, knope, vv, b, kAK, L, ring_off + kAStage, wave, lane);

  // Q^T fragments: lane (g, c) supplies query wi0 + 16 qb + c, dims 32 ks + 8g .. +7.
  v8bf qf[2][kDQh / 32];
  int qpos[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int qi = wi0 + 16 * qb + c;
    const bool on = qi < i1;
    qpos[qb] = on ? pos0 + qi : -1;
    const uint16_t* qrow =
        static_cast<const uint16_t*>(a.q) + ((size_t)(b * a.q_len + (on ? qi : i0)) * a.H + h) * kDQh + 8 * g;
#pragma unroll
    for (int ks = 0; ks < kDQh / 32; ++ks)
      qf[qb][ks] = on ? as_v8bf(*reinterpret_cast<const v4i*>(qrow + 32 * ks)) : as_v8bf(v4i{0, 0, 0, 0});
  }

  // Per-lane LDS offsets inside a slot, kept opaque so every read below is
  // one base register plus an immediate.  K read of row 16 kb + c, logical
  // piece 4 ks + g, stored at piece (4 ks + g) ^ y with y = (c >> 1) & 7:
  // = 4 (ks ^ (y >> 2)) + (g ^ (y & 3)), so even and odd ks each need one
  // base.  V^T read of row 32 kk + 4g + c/4 (+16), bytes 32 db + 8 (c & 3).
  const int y = (c >> 1) & 7;
  int kbase0 = c * kKRow + 16 * (4 * (0 ^ (y >> 2)) + (g ^ (y & 3)));
  int kbase1 = c * kKRow + 16 * (4 * (1 ^ (y >> 2)) + (g ^ (y & 3)));
  int vbase = kKTile + (4 * g + (c >> 2)) * kVRow + 8 * (c & 3);
  asm volatile("" : "+v"(kbase0), "+v"(kbase1), "+v"(vbase));

  // The Q loads (and the first two tiles) complete before the loop, so the
  // compiler keeps no memory wait inside it: the only waits there are the
  // explicit ones that leave the next tile's copies in flight.
  vm_wait<0>();

  const float qk_scale = a.sm_scale * kLog2e;
  // m_ref: the reference the weights are taken against (log2 units); it
  // moves only when a tile's maximum passes it by more than kRescaleMargin,
  // so weights stay below 2^8 and the accumulators are rescaled rarely.
  float m_ref[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};
  v4f acc[kDVh / 16][2];
#pragma unroll
  for (int db = 0; db < kDVh / 16; ++db) acc[db][0] = acc[db][1] = v4f{0.f, 0.f, 0.f, 0.f};
  const v2bf ones = {(__bf16)1.0f, (__bf16)1.0f};

  for (int n = 0; n < ntiles; ++n) {
    if (n + 1 < ntiles) {
      if (wave < kAInstr - 5 * kAW) vm_wait<6>();
      else vm_wait<5>();
    } else {
      vm_wait<0>();
    }
    lds_barrier();  // tile n landed everywhere; every wave is done with tile n - 1
    if (n + 2 < ntiles) attn_tile(a, knope, vv, b, (n + 2) * kAK, L, ring_off + ((n + 2) % kASlots) * kAStage, wave, lane);
    const int s0 = n * kAK;
    if (s0 > w_maxpos) continue;  // every key of the tile is past this wave's queries
    const unsigned char* kt = ring + (n % kASlots) * kAStage;

    // scores S^T[key 16 kb + 4g + i][query 16 qb + c]; the four K fragments
    // of k-step ks + 1 are read while the MFMAs of k-step ks run
    v4f sa[4][2];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) sa[kb][0] = sa[kb][1] = v4f{0.f, 0.f, 0.f, 0.f};
    v8bf kf[2][4];
    auto kread = [&](int ks, v8bf (&dst)[4]) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        dst[kb] = as_v8bf(*reinterpret_cast<const v4i*>(kt + ((ks & 1) ? kbase1 : kbase0) + 16 * kKRow * kb +
                                                         128 * (ks >> 1)));
    };
    kread(0, kf[0]);
#pragma unroll
    for (int ks = 0; ks < kDQh / 32; ++ks) {
      __builtin_amdgcn_sched_barrier(0);
      if (ks + 1 < kDQh / 32) kread(ks + 1, kf[(ks + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        sa[kb][0] = mfma_bf16(kf[ks & 1][kb], qf[0][ks], sa[kb][0]);
        sa[kb][1] = mfma_bf16(kf[ks & 1][kb], qf[1][ks], sa[kb][1]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (s0 + kAK - 1 > w_minpos) {  // diagonal tile: keys past a query's position are -inf
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (s0 + 16 * kb + 4 * g + i > qpos[qb]) sa[kb][qb][i] = -INFINITY;
    }

    // weights 2^(s * scale - m_ref), rounded to bf16; k-slots 8g .. 8g+7 of
    // value step kk hold keys {4g..4g+3} of block 2kk and of block 2kk + 1
    v8bf pf[2][2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float tmax = fmaxf(fmaxf(sa[0][qb][0], sa[0][qb][1]), fmaxf(sa[0][qb][2], sa[0][qb][3]));
#pragma unroll
      for (int kb = 1; kb < 4; ++kb)
        tmax = fmaxf(tmax, fmaxf(fmaxf(sa[kb][qb][0], sa[kb][qb][1]), fmaxf(sa[kb][qb][2], sa[kb][qb][3])));
      tmax = max_xor32(max_xor16(tmax)) * qk_scale;  // the scale is positive
      if (tmax > m_ref[qb] + kRescaleMargin) {       // rare: move the reference
        const float alpha = __builtin_amdgcn_exp2f(m_ref[qb] - tmax);  // 0 while nothing is accumulated
        m_ref[qb] = tmax;
        l_run[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < kDVh / 16; ++db) acc[db][qb] *= alpha;
      }
      const float nm = m_ref[qb] == -INFINITY ? 0.f : -m_ref[qb];  // all -inf so far: weights 0
      uint32_t pk[8];
      float psum = l_run[qb];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(sa[j >> 1][qb][2 * (j & 1)], qk_scale, nm));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(sa[j >> 1][qb][2 * (j & 1) + 1], qk_scale, nm));
        const v2bf pb = __builtin_convertvector((v2f){p0, p1}, v2bf);
        pk[j] = __builtin_bit_cast(uint32_t, pb);
        psum = __builtin_amdgcn_fdot2_f32_bf16(pb, ones, psum, false);  // the rounded weights
      }
      l_run[qb] = psum;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
        pf[kk][qb] = __builtin_bit_cast(
            v8bf, v4i{(int)pk[4 * kk], (int)pk[4 * kk + 1], (int)pk[4 * kk + 2], (int)pk[4 * kk + 3]});
    }

    // values: the V^T fragment (16 dims x the 32 keys of step kk) feeds both
    // query blocks
    // V^T fragments are read two value blocks ahead of their MFMAs
    const unsigned char* vt = kt + vbase;
    constexpr int kVSteps = 2 * (kDVh / 16);  // (kk, db) pairs
    constexpr int kVAhead = 2;
    v4s vlo[kVAhead + 1], vhi[kVAhead + 1];
    auto vread = [&](int j) {
      const unsigned char* p0 = vt + 32 * (j / (kDVh / 16)) * kVRow + 32 * (j % (kDVh / 16));
      vlo[j % (kVAhead + 1)] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)p0);
      vhi[j % (kVAhead + 1)] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(p0 + 16 * kVRow));
    };
#pragma unroll
    for (int j = 0; j < kVAhead; ++j) vread(j);
#pragma unroll
    for (int j = 0; j < kVSteps; ++j) {
      __builtin_amdgcn_sched_barrier(0);
      if (j + kVAhead < kVSteps) vread(j + kVAhead);
      __builtin_amdgcn_sched_barrier(0);
      const int kk = j / (kDVh / 16), db = j % (kDVh / 16), sl = j % (kVAhead + 1);
      const v8bf vf = __builtin_bit_cast(v8bf, __builtin_shufflevector(vlo[sl], vhi[sl], 0, 1, 2, 3, 4, 5, 6, 7));
      acc[db][0] = mfma_bf16(vf, pf[kk][0], acc[db][0]);
      acc[db][1] = mfma_bf16(vf, pf[kk][1], acc[db][1]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  // Output rows out[t, h, :] (256 bytes each, consecutive queries H rows
  // apart) go out through the ring slot after the last tile's: every wave is
  // past the last tile barrier and no copy is in flight, so that slot is
  // free.  Each wave stages one 16-query block at a time in its own 4 KB
  // (query c's row, 16-byte chunk j at j ^ c, so a register write covers
  // 16 banks), then writes whole rows, 16 bytes per lane; the stage is
  // private to the wave, whose LDS accesses complete in order.  lse by the
  // g = 0 lanes.  Lane (g, c) holds dims 16 db + 4g .. +3 of query c.
  unsigned char* const ost = ring + (ntiles % kASlots) * kAStage + wave * (16 * 2 * kDVh);
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float l = sum_xor32(sum_xor16(l_run[qb]));
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int db = 0; db < kDVh / 16; ++db) {
      const v4f o = acc[db][qb];
      const int byte = 32 * db + 8 * g;  // in the query's 256-byte row
      *reinterpret_cast<uint2*>(ost + c * (2 * kDVh) + 16 * ((byte >> 4) ^ c) + (byte & 15)) =
          pack4_bf16(o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv);
    }
    const int qi = wi0 + 16 * qb + c;
    if (qi < i1 && a.lse && g == 0)
      a.lse[((size_t)b * a.q_len + qi) * a.H + h] = l > 0.f ? (m_ref[qb] + log2f(l)) * kLn2 : -INFINITY;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int row = 4 * it + (lane >> 4), j = lane & 15;
      const int qr = wi0 + 16 * qb + row;
      if (qr < i1) {
        const v4i v = *reinterpret_cast<const v4i*>(ost + row * (2 * kDVh) + 16 * (j ^ row));
        *reinterpret_cast<v4i*>(static_cast<uint16_t*>(a.out) + (((size_t)b * a.q_len + qr) * a.H + h) * kDVh + 8 * j) = v;
      }
    }
  }
}

}  // namespace

size_t mha_workspace_bytes(int B, int S_max, int H) { return (size_t)2 * B * H * S_max * kDVh * sizeof(uint16_t); }

hipError_t launch_mha_prefill(const MhaArgs& a, hipStream_t stream) {
  const dim3 g1((unsigned)((a.S_max + kGT - 1) / kGT), (unsigned)a.H, (unsigned)a.B);
  hipLaunchKernelGGL(k_mha_decompress, g1, dim3(kGWaves * 64), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 g2((unsigned)((a.q_len + kAQ - 1) / kAQ), (unsigned)a.H, (unsigned)a.B);
  hipLaunchKernelGGL(k_mha_attn, g2, dim3(kAW * 64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace dsa
