// Sparse MQA-mode MLA over the selected latent entries.
//
// "详解DSA" Eq.(2): u_t = Attn(h_t, {c_s : s in S_t}); MQA mode (charlestar
// page, "DSA 怎样嵌入 MLA"; luowle page section 3.1): all heads of a query
// share the selected 576-wide latent rows; the key is the whole row, the
// value its first 512 dims; the softmax covers the selected rows only.
//
// bf16 path.  A block owns one query row, one contiguous slice (split) of its
// selected indices and all H heads (or, for launches with few query rows,
// one 64-head half of them: see launch_mla_bf16), with 4 waves, one per SIMD (each wave has
// the SIMD's whole register file: 256 VGPRs plus 256 AGPRs).  The selected
// rows are gathered 32 at a time (1152 bytes each, in 16-byte pieces,
// straight from global memory into LDS) through a ring of three padded tiles,
// so two tiles are in flight while one computes.  Per tile:
//   scores: wave w takes heads 32w..32w+31 over all 576 dims,
//     S^T[32 keys x 32 heads] = K_tile[32 x 576] . Q^T[576 x 32]
//     (18 K-steps of v_mfma_f32_16x16x32_bf16 per 16-head block; each K
//     fragment read from LDS feeds both head blocks; the Q^T fragments live in
//     registers), then the softmax weights of those heads in fp32 with base-2
//     exponents, lane <-> head, rounded to bf16 and written to a shared
//     P[head][key] buffer in LDS;
//   values: wave w takes value dims 128w..128w+127 for all heads,
//     O^T[128 dims x 128 heads] += V^T[128 x 32 keys] . P^T[32 keys x 128 heads]:
//     V^T is read with the gfx950 LDS transpose load (ds_read_b64_tr_b16)
//     straight from the row-major tile, and every V^T fragment feeds all
//     eight head blocks, so each tile is read from LDS once for the scores'
//     K fragments per head pair and once for the values.  The accumulators
//     (256 per lane) stay in AGPRs.
// Keys inside a P row are stored in the order the MFMA contracts them: lane
// row g of a score block holds keys 4g..4g+3 and 16+4g..16+4g+3, which is
// the k-slice 8g..8g+7 of the value product.
// With one split the block writes the bf16 output and the log-sum-exp; with
// several each split writes its fp32 output normalised by its own sum plus
// (max, sum), and a combine kernel merges them (the output is rounded to
// bf16 once, after the merge).
#include "dsa_internal.h"

namespace dsa {

namespace {

constexpr int kNT = 32;                          // keys per tile
constexpr int kRowChunk = 16;                    // consecutive rows per XCD turn (one block per row)
constexpr int kMainRS = 1056;                    // LDS stride of a row's dims 0..511 (1024 bytes + 32 pad)
constexpr int kMainBytes = kNT * kMainRS;        // 33792
constexpr int kRopeRS = 128;                     // dims 512..575 of a row: 8 pieces, XOR-swizzled
constexpr int kTileBytes = kMainBytes + kNT * kRopeRS;  // 37888
constexpr int kWaves = 4;                        // one per SIMD
constexpr int kSlots = 4;                        // ring slots: values, scores, two tiles in flight
constexpr int kISlots = 4;                       // index slots per wave (indices arrive four tiles ahead)
constexpr int kThreads = kWaves * 64;
constexpr int kRowsPerWave = kNT / kWaves;       // rows of a tile gathered by each wave (8)
constexpr int kDma = kRowsPerWave + 1;           // gather instructions per wave per tile
constexpr int kKs = kDQK / 32;                   // score K-steps: 16 over dims 0..511, 2 over the rope dims
constexpr int kKsMain = kDV / 32;
constexpr int kMaxHB = 8;                        // 16-head blocks (H <= 128)
constexpr int kDbW = kDV / 16 / kWaves;          // 16-dim value blocks per wave (8)
constexpr int kPRow = 2 * kNT;                   // bytes of one head's P row (32 keys, bf16)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

static_assert(kRowsPerWave * 8 == 64, "one instruction moves the rope pieces of a wave's rows");
static_assert(kKs == kKsMain + 2, "two rope K-steps");

typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v4s lds_v4s;
typedef int v8i_a4 __attribute__((ext_vector_type(8), aligned(4)));

__device__ __forceinline__ v4f mfma_bf16(v8bf a, v8bf b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ v8bf as_v8bf(v4i x) { return __builtin_bit_cast(v8bf, x); }

// Wait until at most N of this wave's vector-memory operations are in flight.
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt has 6 bits");
  // gfx9 s_waitcnt: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] << 14
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00);
}

// vm_wait for the counts the prologue can leave in flight.
__device__ __forceinline__ void vm_wait_n(int n) {
  if (n >= 2 * kDma + 1) vm_wait<2 * kDma + 1>();
  else if (n >= 2 * kDma) vm_wait<2 * kDma>();
  else if (n >= kDma) vm_wait<kDma>();
  else vm_wait<0>();
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

// Decomposition of one launch: ns splits per row and nh blocks per
// (row, split).  With 128 heads and too few rows to fill the chip with one
// split each, every (row, split) gets two 64-head blocks, so the same block
// count needs half the splits (and half the split partials).
struct MlaPlan {
  int ns, nh;
};
__host__ inline MlaPlan mla_plan(int T, int H, int k) {
  const int ns1 = mla_splits(T, k);
  if (H == 128 && ns1 > 1) return MlaPlan{mla_splits(2 * T, k), 2};
  return MlaPlan{ns1, 1};
}

struct Partials {
  float* o;     // [T][ns][H][512] fp32, normalised by the split's own sum
  float* ml;    // [T][ns][H][2]   (max in log2 units, sum)
};

__device__ __forceinline__ Partials partials(const MlaArgs& a, int ns) {
  Partials p;
  const size_t T = (size_t)a.row_count;
  p.ml = static_cast<float*>(a.ws);
  p.o = p.ml + T * ns * a.H * 2;
  return p;
}

// Gather of one tile: wave w moves tile rows 8w..8w+7 straight into LDS,
// 16 bytes per lane per instruction: one instruction per row for its dims
// 0..511 (64 pieces, row stride kMainRS), and one more that moves the rope
// pieces (dims 512..575) of the eight rows.  Rope piece p of row r sits at
// position p ^ ((r >> 1) & 7) of the row's 128-byte slot: two consecutive
// rows share a 256-byte bank line, so the 16 rows one score read covers
// (16 lanes x 16 bytes per LDS cycle) fall on distinct banks.  Rows past the split or not
// selectable read row 0 of the sequence (a real row whenever the query sees
// any key), so every instruction is issued with the same lanes and the wait
// counts stay exact; the row's validity bit masks its score.
struct TileSrc {
  const uint16_t* kvb;
  const int32_t* idx_row;
  int m1, pos;
};

// The gather of one tile: prepare() takes the wave's eight indices (one per
// lane group: lane l works on row l & 7, and on row l >> 3 for the rope
// instruction) and their validity (one ballot gives the tile's mask byte),
// in vector registers, and leaves the row to read per lane (row 0 for an
// invalid entry); issue() takes each row's index from lane rr (a readlane),
// forms its base address in scalar registers and issues the nine copies.
// A copy instruction into LDS takes far longer to issue than the scalar
// arithmetic between two of them, and no compare/select chain per row sits
// in the issue stream.
struct TileGather {
  v4i lo, hi;         // raw indices of rows 0..3 / 4..7 (uniform; before the tile loop only)
  int raw, rraw;      // lane l: index of row l & 7 / of row l >> 3 (0 when invalid, after prepare)

  // indices of the eight rows from the wave's LDS slot (inside the tile loop)
  __device__ __forceinline__ void read_lds(const int32_t* slot, int lane) {
    raw = slot[lane & 7];
    rraw = slot[lane >> 3];
  }
  // ... or from the uniform values of a scalar load (before the loop)
  __device__ __forceinline__ void from_uniform(int lane) {
    const int i = lane & 7, j = lane >> 3;
    raw = lo[0];
    rraw = lo[0];
#pragma unroll
    for (int rr = 1; rr < kRowsPerWave; ++rr) {
      const int v = rr < 4 ? lo[rr] : hi[rr - 4];
      raw = i == rr ? v : raw;
      rraw = j == rr ? v : rraw;
    }
  }
  // Validity (entries at or past the split end, negative or past the query
  // position are invalid); byte w of vmask gets the validity of rows 8w..8w+7.
  __device__ __forceinline__ void prepare(const TileSrc& src, int mb, unsigned char* vmask, int wave, int lane) {
    const int mw = mb + wave * kRowsPerWave;
    const bool ok = mw + (lane & 7) < src.m1 && raw >= 0 && raw <= src.pos;
    const bool okr = mw + (lane >> 3) < src.m1 && rraw >= 0 && rraw <= src.pos;
    const uint32_t vbits = (uint32_t)__ballot(ok) & 0xFFu;  // lanes 0..7: rows 0..7
    if (lane == 0) vmask[wave] = (unsigned char)vbits;
    raw = ok ? raw : 0;
    rraw = okr ? rraw : 0;
  }
  // dims 0..511 of tile row 8w + rr (64 pieces; lane16 = 16 * lane)
  __device__ __forceinline__ void row(const TileSrc& src, int rr, uint32_t tile, int wave, uint32_t lane16) const {
    const int s = __builtin_amdgcn_readlane(raw, rr);
    dma16_lds_off(src.kvb + (size_t)s * kDQK, lane16, tile + (wave * kRowsPerWave + rr) * kMainRS);
  }
  // rope pieces: lane l -> row 8w + l/8, slot l%8
  __device__ __forceinline__ void rope(const TileSrc& src, uint32_t tile, int wave, int lane) const {
    const int row0 = wave * kRowsPerWave;
    const int piece = 64 + ((lane & 7) ^ (((row0 + (lane >> 3)) >> 1) & 7));
    dma16_lds_at(src.kvb + (size_t)rraw * kDQK + 8 * piece, tile + kMainBytes + row0 * kRopeRS);
  }
  __device__ __forceinline__ void issue(const TileSrc& src, uint32_t tile, int wave, int lane, uint32_t lane16) const {
#pragma unroll
    for (int rr = 0; rr < kRowsPerWave; ++rr) row(src, rr, tile, wave, lane16);
    rope(src, tile, wave, lane);
  }
};

// Indices read by scalar loads (used before the tile loop, so they stay off
// the vector-memory counter; a wave's eight indices are contiguous: one
// 32-byte load unless the split ends inside them).
__device__ __forceinline__ TileGather scalar_indices(const TileSrc& src, int mb, int wave) {
  const int mw = __builtin_amdgcn_readfirstlane(mb + wave * kRowsPerWave);
  int raw[kRowsPerWave];
  if (mw + kRowsPerWave <= src.m1) {
    const v8i_a4 v = *reinterpret_cast<const v8i_a4*>(src.idx_row + mw);
#pragma unroll
    for (int rr = 0; rr < kRowsPerWave; ++rr) raw[rr] = __builtin_amdgcn_readfirstlane(v[rr]);
  } else {
#pragma unroll
    for (int rr = 0; rr < kRowsPerWave; ++rr) {
      const int m = mw + rr;
      raw[rr] = __builtin_amdgcn_readfirstlane(src.idx_row[m < src.m1 ? m : src.m1 - 1]);
    }
  }
  TileGather tg;
  tg.lo = v4i{raw[0], raw[1], raw[2], raw[3]};
  tg.hi = v4i{raw[4], raw[5], raw[6], raw[7]};
  return tg;
}

// Inside the tile loop the indices arrive one tile ahead, by a 4-byte
// global -> LDS copy of the wave's eight entries (clamped into the split),
// so no scalar-load latency sits in front of a gather.
__device__ __forceinline__ void fetch_indices(const TileSrc& src, int mb, int32_t* slot, int wave, int lane) {
  asm volatile("" : "+v"(lane));  // formed here, not hoisted out of the loops (it would be spilled)
  if (lane < kRowsPerWave) {
    const int m = mb + wave * kRowsPerWave + lane;
    dma4_lds(src.idx_row, 4u * (uint32_t)(m < src.m1 ? m : src.m1 - 1), slot);
  }
}


// NHB 16-head blocks per block; wave w runs the scores and softmax of blocks
// SHB*w .. SHB*w + SHB-1 (those below NHB), and every wave's value product
// covers all NHB.  SHB = 2: all H heads per block (NHB = H / 16).  SHB = 1:
// a 64-head half per block (NHB = 4, one score block per wave), nh = 2 blocks
// per (row, split), so a launch with few rows fills the chip with half the
// splits (half the split partials).
template <int NHB, int SHB>
__global__ __launch_bounds__(kThreads, 1) void k_mla_bf16(MlaArgs a, const int32_t* __restrict__ idx, int ns,
                                                        int per_split, int per_xcd) {
  static_assert(SHB == 2 || (SHB == 1 && NHB == kWaves), "one score block per wave covers 64 heads");
  constexpr int nh = SHB == 1 ? 2 : 1;  // blocks per (row, split)
  __shared__ __attribute__((aligned(16))) unsigned char ring[kSlots * kTileBytes];
  // P[head][key] bf16; the 16-byte chunk j of head h's row sits at position
  // j ^ ((h >> 2) & 3), so 16 consecutive heads read or written at one chunk
  // fall on distinct banks.
  __shared__ __attribute__((aligned(16))) unsigned char pbuf[kMaxHB * 16 * kPRow];
  __shared__ uint32_t vmask[kSlots];  // per ring slot: bit r = validity of tile row r
  __shared__ __attribute__((aligned(16))) int32_t islot[kWaves][kISlots][kRowsPerWave];  // prefetched row indices
  __shared__ float hinv[kMaxHB * 16];
  __shared__ int overflow_flag;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, c = lane & 15;
  // Blocks go round-robin over the 8 XCDs.  With several blocks per row, an
  // XCD takes a contiguous range of whole rows, so the splits and halves of
  // one query share that XCD's L2 (its query rows are read once).  With one
  // block per row, the rows go to the XCDs in chunks of kRowChunk, dealt
  // round-robin and last rows first: every XCD gets an equal share of a
  // causal prefill's short early rows, which otherwise all fall on the first
  // XCD, and the long rows start first.
  int li;
  if (ns * nh == 1) {
    const int x = (int)blockIdx.x % 8, j = (int)blockIdx.x / 8;
    li = a.row_count - 1 - (((j / kRowChunk) * 8 + x) * kRowChunk + j % kRowChunk);
    if (li < 0) return;
  } else {
    li = ((int)blockIdx.x % 8) * per_xcd + (int)blockIdx.x / 8;
    if (li >= a.row_count * ns * nh) return;
  }
  const int r = li / (ns * nh), split = (li / nh) % ns;
  const int hoff = 64 * (li % nh);  // first head of this block
  const int t = a.row_begin + r;
  const int b = t / a.q_len;
  const int pos = row_pos(a.seq_lens, t, a.q_len, a.S_max);
  const int m0 = split * per_split;
  // with the forward's own selection the valid entries are the first
  // min(k, pos + 1): a causal row that sees fewer than k keys stops there
  // instead of gathering and masking -1 tiles
  const int kv_end = a.sel_prefix ? min(a.k, pos + 1) : a.k;
  const int m1 = min(kv_end, m0 + per_split);
  // a query that sees no key gathers nothing (its output is zero)
  const int ntiles = (m1 > m0 && pos >= 0) ? (m1 - m0 + kNT - 1) / kNT : 0;
  const bool sh0 = NHB >= SHB * kWaves - 1 || SHB * wave < NHB;                 // this wave has score heads
  const bool sh1 = SHB == 2 && (NHB >= 2 * kWaves || 2 * wave + 1 < NHB);      // ... and a second 16-head block

  // Per-lane LDS offsets within a tile (kept as single opaque values so the
  // compiler neither splits nor re-derives them inside the tile loop): score
  // read of row c over dims 0..511 and over the two rope K-steps, V^T
  // transpose-read position of this wave's value dims, and the P read.
  int aoff = c * kMainRS + 16 * g;
  int roff0 = kMainBytes + c * kRopeRS + 16 * (g ^ ((c >> 1) & 7));
  int roff1 = roff0 ^ 64;  // rope piece 4 + g: slot (g ^ ((c >> 1) & 7)) ^ 4
  int voff = (4 * g + (c >> 2)) * kMainRS + 8 * (c & 3) + 2 * (kDV / kWaves) * wave;
  int poff = c * kPRow + 16 * (g ^ ((c >> 2) & 3));
  // 16 * lane: the per-lane offset of every row copy (opaque, so no per-row
  // address is formed ahead of time)
  uint32_t lane16 = 16u * (uint32_t)lane;
  asm volatile("" : "+v"(aoff), "+v"(roff0), "+v"(roff1), "+v"(voff), "+v"(poff), "+v"(lane16));

  TileSrc src;
  src.kvb = static_cast<const uint16_t*>(a.kv) + (a.flat ? 0 : (size_t)b * a.S_max * kDQK);
  src.idx_row = idx + (size_t)t * a.k;
  src.m1 = m1;
  src.pos = a.flat ? 0x7FFFFFFF : pos;  // flat pool rows: the causal bound is already applied
  unsigned char* const vmb = reinterpret_cast<unsigned char*>(vmask);
  const uint32_t ring_off = lds_offset(ring);

  // Copies before the loop, in this order per wave: tile 0 (kDma), the Q^T
  // fragments (kQLoads), tile 1 (kDma), the indices of tile 3 (1), tile 2
  // (kDma).  The scores of tile 0 wait for tile 0 and Q only (the later
  // copies stay in flight).
  // Lane holds head 16*(2w + j) + c, dims 32*ks + 8g .. +7.
  TileGather g1, g2;
  auto prologue = [&]() {
    TileGather g0 = scalar_indices(src, m0, wave);
    if (ntiles > 1) g1 = scalar_indices(src, m0 + kNT, wave);
    if (ntiles > 2) g2 = scalar_indices(src, m0 + 2 * kNT, wave);
    if (ntiles > 0) {
      g0.from_uniform(lane);
      g0.prepare(src, m0, vmb, wave, lane);
      g0.issue(src, ring_off, wave, lane, lane16);
    }
  };
  auto prologue_rest = [&]() {
    if (ntiles > 1) {
      g1.from_uniform(lane);
      g1.prepare(src, m0 + kNT, vmb + 4, wave, lane);
      g1.issue(src, ring_off + kTileBytes, wave, lane, lane16);
    }
    if (ntiles > 3) fetch_indices(src, m0 + 3 * kNT, islot[wave][3], wave, lane);
    if (ntiles > 2) {
      g2.from_uniform(lane);
      g2.prepare(src, m0 + 2 * kNT, vmb + 8, wave, lane);
      g2.issue(src, ring_off + 2 * kTileBytes, wave, lane, lane16);
    }
  };
  prologue();
  v8bf qf[2][kKs];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const bool on = j ? sh1 : sh0;
    const uint16_t* qrow =
        static_cast<const uint16_t*>(a.q) + ((size_t)t * a.H + hoff + (on ? 16 * (SHB * wave + j) + c : 0)) * kDQK + 8 * g;
#pragma unroll
    for (int ks = 0; ks < kKs; ++ks)
      qf[j][ks] = on ? as_v8bf(*reinterpret_cast<const v4i*>(qrow + 32 * ks)) : as_v8bf(v4i{0, 0, 0, 0});
  }
  prologue_rest();

  // Softmax reference: m_ref is fixed at the first tile with a valid key and
  // never moved, so the accumulators are never rescaled.  Later scores may
  // exceed it by up to 2^64, which fp32 and bf16 carry exactly as ordinary
  // numbers.  If a score goes beyond that headroom the block reruns its split
  // once with m_ref set to the true maximum seen in the first run.
  float m_ref[2] = {-INFINITY, -INFINITY}, m_seen[2] = {-INFINITY, -INFINITY}, l_part[2] = {0.f, 0.f};
  v4f acc_o[kDbW][kMaxHB];
  const float qk_scale = a.sm_scale * kLog2e;
  bool overflow = false;

  // Scores of one tile: S^T[key, head] over all 576 dims; block kb row rho
  // is key 16*kb + rho, so lane row g holds keys 4g..4g+3 (kb = 0) and
  // 16+4g..16+4g+3 (kb = 1).  Step n = kKs*kb + ks.  LDS reads run kAhead
  // steps ahead of the MFMAs that consume them.
  constexpr int kAhead = 4;
  auto aload = [&](const unsigned char* tb, int n) -> v8bf {
    const int kb = n / kKs, ks = n % kKs;
    const unsigned char* p = ks < kKsMain ? tb + aoff + 16 * kMainRS * kb + 64 * ks
                                          : tb + (ks == kKsMain ? roff0 : roff1) + 16 * kRopeRS * kb;
    return as_v8bf(*reinterpret_cast<const v4i*>(p));
  };
  // hook(n) runs inside score step n (between fences), so other work can be
  // spread over the MFMAs.
  auto scores = [&](const unsigned char* tb, v4f (&sa)[2][2], auto&& hook) {
    v8bf af[kAhead];
#pragma unroll
    for (int n = 0; n < kAhead; ++n) af[n] = aload(tb, n);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) sa[kb][0] = sa[kb][1] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int n = 0; n < 2 * kKs; ++n) {
      __builtin_amdgcn_sched_barrier(0);
      const int kb = n / kKs, ks = n % kKs;
      sa[kb][0] = mfma_bf16(af[n % kAhead], qf[0][ks], sa[kb][0]);
      if (sh1) sa[kb][1] = mfma_bf16(af[n % kAhead], qf[1][ks], sa[kb][1]);
      if (n + kAhead < 2 * kKs) af[n % kAhead] = aload(tb, n + kAhead);
      hook(n);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  // Softmax weights of one tile's scores (vm: its row-validity bits), rounded
  // to bf16 and written to the P buffer, as kSoftSteps micro-steps so they
  // can ride on the next tile's score MFMAs.  sv[4*kb + i] is key
  // 16*kb + 4g + i; masked keys become -inf through a bit select.
  constexpr int kSoftSteps = 19;
  uint32_t vml;  // validity bits shifted so bit 16*kb + i is key 16*kb + 4g + i
  bool vfull;    // every key of the tile is valid (the common case: no masking)
  float sv[8], tmax, nmr;
  uint32_t pk[4];
  auto soft_step = [&](int k, const v4f (&sa)[2][2], uint32_t vm) {
    if (k == 0) {
      vml = vm >> (4 * g);
      vfull = vm == 0xFFFFFFFFu;
      return;
    }
    const int hb = (k - 1) / 9, st = (k - 1) % 9;
    if (hb == 1 && !sh1) return;
    if (st == 0) {
      if (vfull) {
#pragma unroll
        for (int j = 0; j < 8; ++j) sv[j] = sa[j >> 2][hb][j & 3];
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j)
          sv[j] = (vml >> (16 * (j >> 2) + (j & 3))) & 1u ? sa[j >> 2][hb][j & 3] : -INFINITY;
      }
    } else if (st == 1) {
      tmax = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])), fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
    } else if (st == 2) {
      tmax = max_xor16(tmax);
    } else if (st == 3) {
      tmax = max_xor32(tmax) * qk_scale;  // the scale is positive: max commutes with it
      m_seen[hb] = fmaxf(m_seen[hb], tmax);
      if (m_ref[hb] == -INFINITY) m_ref[hb] = tmax;  // nothing accumulated yet
      overflow = overflow || (tmax > m_ref[hb] + 64.f);
      // p = 2^(s*scale - m_ref) rounded to bf16 (RNE, two per conversion);
      // the normaliser sums the same rounded weights the value product
      // uses, so the output is an exact convex combination of value rows.
      // Without a reference yet every p is 0.  A score past the headroom
      // may give inf here; that pass is discarded and rerun.
      nmr = m_ref[hb] == -INFINITY ? -INFINITY : -m_ref[hb];
    } else if (st <= 7) {
      const int j = st - 4;
      const float p0 = __builtin_amdgcn_exp2f(fmaf(sv[2 * j], qk_scale, nmr));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(sv[2 * j + 1], qk_scale, nmr));
      pk[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f){p0, p1}, v2bf));
    } else {
      // sum of the rounded weights, a pair per dot instruction (exact products by one)
      float psum = 0.f;
      const v2bf ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
      for (int j = 0; j < 4; ++j) psum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(v2bf, pk[j]), ones, psum, false);
      l_part[hb] += psum;
      *reinterpret_cast<v4i*>(pbuf + (16 * (SHB * wave + hb)) * kPRow + poff) =
          v4i{(int)pk[0], (int)pk[1], (int)pk[2], (int)pk[3]};
    }
  };
  // O^T[dims, heads] += V^T[dims, keys] . P^T[keys, heads].  V^T fragments
  // (16 dims x keys {4g..4g+3, 16+4g..16+4g+3} for lane row g) are two LDS
  // transpose loads each: lane j of a 16-lane row supplies key kbase + j/4,
  // dims 16db + 4*(j%4) .. +3.  The first kVAhead fragments are read before
  // the barrier that publishes P (values_pre).
  constexpr int kVAhead = 3;
  v4s vlo[kVAhead], vhi[kVAhead];
  auto vaddr = [&](const unsigned char* tb, int db) { return tb + voff + 32 * db; };  // rows + 16: 16 * kMainRS further
  auto values_pre = [&](const unsigned char* tb) {
#pragma unroll
    for (int db = 0; db < kVAhead; ++db) {
      vlo[db] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)vaddr(tb, db));
      vhi[db] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(vaddr(tb, db) + 16 * kMainRS));
    }
  };
  auto values = [&](const unsigned char* tb) {
    v8bf pf[kMaxHB];
#pragma unroll
    for (int hb = 0; hb < kMaxHB; ++hb)
      if (hb < NHB) pf[hb] = as_v8bf(*reinterpret_cast<const v4i*>(pbuf + 16 * hb * kPRow + poff));
#pragma unroll
    for (int db = 0; db < kDbW; ++db) {
      __builtin_amdgcn_sched_barrier(0);
      const int sl = db % kVAhead;
      const v8bf av =
          __builtin_bit_cast(v8bf, __builtin_shufflevector(vlo[sl], vhi[sl], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int hb = 0; hb < kMaxHB; ++hb)
        if (hb < NHB) acc_o[db][hb] = mfma_bf16(av, pf[hb], acc_o[db][hb]);
      if (db + kVAhead < kDbW) {
        vlo[sl] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)vaddr(tb, db + kVAhead));
        vhi[sl] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(vaddr(tb, db + kVAhead) + 16 * kMainRS));
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  static_assert(kSoftSteps + 1 <= 2 * kKs, "softmax micro-steps fit into the score steps");

  for (int pass = 0; pass < 2; ++pass) {
    if (pass == 1) {  // rerun with the true maxima as references (no score can exceed them)
      m_ref[0] = m_seen[0];
      m_ref[1] = m_seen[1];
      overflow = false;
      __syncthreads();
      prologue();
      prologue_rest();
    }
#pragma unroll
    for (int db = 0; db < kDbW; ++db)
#pragma unroll
      for (int hb = 0; hb < kMaxHB; ++hb) acc_o[db][hb] = v4f{0.f, 0.f, 0.f, 0.f};
    l_part[0] = l_part[1] = 0.f;
    if (tid == 0) overflow_flag = 0;
    if (ntiles == 0) break;
    // Scores of tile 0 first: tile 0 and Q have landed once at most the
    // copies issued after them (tile 1, idx(3), tile 2) are in flight.
    vm_wait_n((ntiles > 1 ? kDma : 0) + (ntiles > 3 ? 1 : 0) + (ntiles > 2 ? kDma : 0));
    lds_barrier();
    v4f sacc[2][2];
    if (sh0) scores(ring, sacc, [](int) {});
    // Tile step tt: wait for tile tt+1 and the indices of tile tt+3, barrier
    // (all shares landed; everyone is done with tile tt-1 and with the P
    // buffer), copy burst (indices of tile tt+4, rows of tile tt+3 into the
    // slot tile tt-1 used), scores of tile tt+1 interleaved with the softmax
    // of tile tt, the first V^T reads, barrier (P complete), values of tile
    // tt.  Per wave the copies go out in the order ..., idx(tt+3), rows(tt+2),
    // idx(tt+4), rows(tt+3), so at most kDma copies in flight means rows(tt+1)
    // and idx(tt+3) landed.
    for (int tt = 0; tt < ntiles; ++tt) {
      if (tt + 2 < ntiles)
        vm_wait<kDma>();
      else
        vm_wait<0>();
      lds_barrier();
      if (tt + 4 < ntiles) fetch_indices(src, m0 + (tt + 4) * kNT, islot[wave][(tt + 4) % kISlots], wave, lane);
      if (tt + 3 < ntiles) {
        TileGather tg;
        tg.read_lds(islot[wave][(tt + 3) % kISlots], lane);
        tg.prepare(src, m0 + (tt + 3) * kNT, vmb + 4 * ((tt + 3) & 3), wave, lane);
        tg.issue(src, ring_off + ((tt + 3) & 3) * kTileBytes, wave, lane, lane16);
      }
      if (sh0) {
        const uint32_t vm = vmask[tt & 3];
        if (tt + 1 < ntiles) {
          // softmax micro-step k rides on score step k + 1
          v4f snext[2][2];
          scores(ring + ((tt + 1) & 3) * kTileBytes, snext, [&](int n) {
            if (n >= 1 && n <= kSoftSteps) soft_step(n - 1, sacc, vm);
          });
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
            sacc[kb][0] = snext[kb][0];
            sacc[kb][1] = snext[kb][1];
          }
        } else {
#pragma unroll
          for (int k = 0; k < kSoftSteps; ++k) soft_step(k, sacc, vm);
        }
      }
      values_pre(ring + (tt & 3) * kTileBytes);
      lds_barrier();  // P of every head is in LDS
      values(ring + (tt & 3) * kTileBytes);
    }
    __syncthreads();
    if (overflow) overflow_flag = 1;
    __syncthreads();
    if (!overflow_flag) break;
  }

  // Normalisers: the wave that ran a head's softmax publishes 1/l (and the
  // log-sum-exp or the split's (max, sum)).
  const Partials P = partials(a, ns);
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    if (!(hb ? sh1 : sh0)) break;
    const int head = 16 * (SHB * wave + hb) + c;  // within the block's heads
    const float l_tot = sum_xor32(sum_xor16(l_part[hb]));
    if (g == 0) {
      hinv[head] = l_tot > 0.f ? 1.f / l_tot : 0.f;
      if (ns == 1) {
        if (a.lse) a.lse[(size_t)t * a.H + hoff + head] = l_tot > 0.f ? (m_ref[hb] + log2f(l_tot)) * kLn2 : -INFINITY;
      } else {
        float* pml = P.ml + (((size_t)r * ns + split) * a.H + hoff + head) * 2;
        pml[0] = l_tot > 0.f ? m_ref[hb] : -INFINITY;
        pml[1] = l_tot;
      }
    }
  }
  __syncthreads();
  if (ns > 1) {
    // fp32 split partial straight from the accumulators: lane (c, g) holds
    // dims 128w + 16db + 4g .. +3 of head 16hb + c, one 16-byte store each
    // (each head's 16-dim piece is 64 contiguous bytes).
#pragma unroll
    for (int hb = 0; hb < kMaxHB; ++hb) {
      if (!(hb < NHB)) break;
      const int head = 16 * hb + c;
      const float inv = hinv[head];
      float* prow = P.o + (((size_t)r * ns + split) * a.H + hoff + head) * kDV + (kDV / kWaves) * wave + 4 * g;
#pragma unroll
      for (int db = 0; db < kDbW; ++db)
        *reinterpret_cast<v4f*>(prow + 16 * db) = acc_o[db][hb] * inv;
    }
    return;
  }
  // Output through LDS (the ring is free now): each wave stages four 16-head
  // blocks at a time as rows of its 128 dims, then stores whole 256-byte
  // pieces of the output rows.
  constexpr int kStageRS = 2 * (kDV / kWaves) + 16;
  unsigned char* stage = ring + wave * 64 * kStageRS;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    if (64 * half >= 16 * NHB) break;
#pragma unroll
    for (int hl = 0; hl < 4; ++hl) {
      const int hb = 4 * half + hl;
      if (!(hb < NHB)) break;
      const float inv = hinv[16 * hb + c];
#pragma unroll
      for (int db = 0; db < kDbW; ++db) {
        // hardware round-to-nearest-even, two values per conversion
        const v2bf lo = __builtin_convertvector((v2f){acc_o[db][hb][0] * inv, acc_o[db][hb][1] * inv}, v2bf);
        const v2bf hi = __builtin_convertvector((v2f){acc_o[db][hb][2] * inv, acc_o[db][hb][3] * inv}, v2bf);
        *reinterpret_cast<v2i*>(stage + (16 * hl + c) * kStageRS + 2 * (16 * db + 4 * g)) =
            v2i{__builtin_bit_cast(int, lo), __builtin_bit_cast(int, hi)};
      }
    }
    // the stage is private to this wave: its own LDS writes complete in order
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int hr = 4 * j + (lane >> 4);
      const int hh = 64 * half + hr;
      if (hh < 16 * NHB) {
        const v4i v = *reinterpret_cast<const v4i*>(stage + hr * kStageRS + 16 * (lane & 15));
        uint16_t* orow = static_cast<uint16_t*>(a.out) + ((size_t)t * a.H + hoff + hh) * kDV;
        *reinterpret_cast<v4i*>(orow + (kDV / kWaves) * wave + 8 * (lane & 15)) = v;
      }
    }
  }
}

// Merge split partials: each split stored its fp32 output normalised by its
// own sum l_s together with (m_s, l_s);
// out = sum_s 2^(m_s-M) l_s o_s / sum_s 2^(m_s-M) l_s, rounded to bf16 once.
// A wave merges one (row, head): lane l holds dims 8l..8l+7, so each split's
// partial row is one contiguous 2 KB load (all issued before any is used).
// Blocks for a row run on the XCD that ran its first split (the split
// kernel gives XCD x the flat (row, split, half) indices [x*per_xcd,
// (x+1)*per_xcd), upr = ns * nh of them per row), whose L2 saw the partials
// written.
constexpr int kCombineMaxSplits = 8;
constexpr int kCombineHeads = 4;  // heads (waves) per block
__global__ __launch_bounds__(64 * kCombineHeads) void k_mla_combine(MlaArgs a, int ns, int upr, int per_xcd) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int x = (int)blockIdx.x % 8, j = (int)blockIdx.x / 8;
  const int hpb = a.H / kCombineHeads;  // blocks per row
  const int r0 = (x * per_xcd + upr - 1) / upr;
  const int r1 = min(a.row_count, ((x + 1) * per_xcd + upr - 1) / upr);
  const int r = r0 + j / hpb;
  if (r >= r1) return;
  const int h = (j % hpb) * kCombineHeads + wave;
  const int t = a.row_begin + r;
  const Partials P = partials(a, ns);
  float ms[kCombineMaxSplits], ls[kCombineMaxSplits];
  v4f o[kCombineMaxSplits][2];
#pragma unroll
  for (int sp = 0; sp < kCombineMaxSplits; ++sp) {
    if (sp < ns) {
      const size_t rs = ((size_t)r * ns + sp) * a.H + h;
      ms[sp] = P.ml[rs * 2];
      ls[sp] = P.ml[rs * 2 + 1];
      o[sp][0] = *reinterpret_cast<const v4f*>(P.o + rs * kDV + 8 * lane);
      o[sp][1] = *reinterpret_cast<const v4f*>(P.o + rs * kDV + 8 * lane + 4);
    }
  }
  float M = -INFINITY;
#pragma unroll
  for (int sp = 0; sp < kCombineMaxSplits; ++sp)
    if (sp < ns) M = fmaxf(M, ms[sp]);
  float wsum = 0.f;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
  for (int sp = 0; sp < kCombineMaxSplits; ++sp) {
    if (sp < ns && ms[sp] != -INFINITY) {
      const float wgt = exp2f(ms[sp] - M) * ls[sp];
      wsum += wgt;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += wgt * o[sp][e >> 2][e & 3];
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  v4i st;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    st[e] = __builtin_bit_cast(int, __builtin_convertvector((v2f){acc[2 * e] * inv, acc[2 * e + 1] * inv}, v2bf));
  *reinterpret_cast<v4i*>(static_cast<uint16_t*>(a.out) + ((size_t)t * a.H + h) * kDV + 8 * lane) = st;
  if (a.lse && lane == 0) a.lse[(size_t)t * a.H + h] = wsum > 0.f ? (M + log2f(wsum)) * kLn2 : -INFINITY;
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
  const float* kvb = static_cast<const float*>(a.kv) + (a.flat ? 0 : (size_t)b * a.S_max * kDQK);
  const int32_t* idx_row = a.idx + (size_t)t * a.k;
  const int smax = a.flat ? 0x7FFFFFFF : pos;  // flat pool rows: the causal bound is already applied
  float lmax = -INFINITY;
  for (int m = tid; m < a.k; m += 256) {
    const int s = idx_row[m];
    float z = -INFINITY;
    if (s >= 0 && s <= smax && pos >= 0) {
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
  const int ns = mla_plan(T, H, k).ns;
  if (ns == 1) return 0;
  return (size_t)T * ns * H * (2 * sizeof(float) + kDV * sizeof(float));
}

bool mla_f32_supported(int k) { return k <= kF32MaxK; }

hipError_t launch_mla_bf16(const MlaArgs& a, hipStream_t stream) {
  if (a.row_count <= 0) return hipSuccess;
  // Splits are sized from the whole launch so partial buffers match the workspace size query.
  const MlaPlan plan = mla_plan(a.row_count, a.H, a.k);
  const int ns = plan.ns, upr = plan.ns * plan.nh;
  const int per = mla_per_split(a.k, ns);
  const int total = a.row_count * upr;
  // blocks per XCD: whole rows (several blocks per row), or whole row chunks
  const int per_xcd = upr == 1 ? ((total + kRowChunk - 1) / kRowChunk + 7) / 8 * kRowChunk : (total + 7) / 8;
  const dim3 grid((unsigned)(8 * per_xcd)), block(kThreads);
  if (plan.nh == 2) {
    hipLaunchKernelGGL((k_mla_bf16<4, 1>), grid, block, 0, stream, a, a.idx, ns, per, per_xcd);
  } else {
    switch (a.H / 16) {
      case 1: hipLaunchKernelGGL((k_mla_bf16<1, 2>), grid, block, 0, stream, a, a.idx, ns, per, per_xcd); break;
      case 2: hipLaunchKernelGGL((k_mla_bf16<2, 2>), grid, block, 0, stream, a, a.idx, ns, per, per_xcd); break;
      case 3: hipLaunchKernelGGL((k_mla_bf16<3, 2>), grid, block, 0, stream, a, a.idx, ns, per, per_xcd); break;
      case 4: hipLaunchKernelGGL((k_mla_bf16<4, 2>), grid, block, 0, stream, a, a.idx, ns, per, per_xcd); break;
      case 5: hipLaunchKernelGGL((k_mla_bf16<5, 2>), grid, block, 0, stream, a, a.idx, ns, per, per_xcd); break;
      case 6: hipLaunchKernelGGL((k_mla_bf16<6, 2>), grid, block, 0, stream, a, a.idx, ns, per, per_xcd); break;
      case 7: hipLaunchKernelGGL((k_mla_bf16<7, 2>), grid, block, 0, stream, a, a.idx, ns, per, per_xcd); break;
      case 8: hipLaunchKernelGGL((k_mla_bf16<8, 2>), grid, block, 0, stream, a, a.idx, ns, per, per_xcd); break;
      default: return hipErrorInvalidValue;
    }
  }
  if (ns > 1) {
    // per XCD at most ceil(per_xcd / upr) + 1 rows have their first block there
    const int cpx = ((per_xcd + upr - 1) / upr + 1) * (a.H / kCombineHeads);
    hipLaunchKernelGGL(k_mla_combine, dim3((unsigned)(8 * cpx)), dim3(64 * kCombineHeads), 0, stream, a, ns, upr,
                       per_xcd);
  }
  return hipGetLastError();
}

hipError_t launch_mla_f32(const MlaArgs& a, hipStream_t stream) {
  if (a.row_count <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_mla_f32, dim3((unsigned)a.H, (unsigned)a.row_count), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace dsa
