// Fused long-prefill indexer + streaming top-k.
//
// The charlestar page ("Prefill 与 decode 中发生了什么", Prefill) asks for
// tile-wise index scores with local candidates kept on chip, hierarchical
// merging into the final top-k, and no full L x L score matrix written to
// HBM.  This kernel does exactly that on gfx950:
//
//  * A block owns 8 consecutive query rows of one sequence (two per wave,
//    one wave per SIMD; two blocks share a CU, so one block's barrier waits
//    and list compactions overlap the other's MFMAs)
//    and walks the causal key range [0, max_pos] in 64-key tiles copied
//    straight from global memory into LDS one tile ahead (double buffered;
//    XOR-swizzled 16-byte chunks so the MFMA B-operand reads of consecutive
//    keys hit distinct banks).
//  * Scores: v_mfma_f32_16x16x128_f8f6f4 with the query rows' 64x128 fp8
//    tiles held in registers; ReLU, per-head weight and the reduction over
//    the 64 heads are fused on the MFMA result registers; the k-scale and
//    the causal mask are applied to the finished 64 scores (one per lane).
//  * Selection: each row keeps a running threshold theta (an order-preserving
//    uint32 image of an fp32 score) and a candidate list in the workspace.
//    A score is appended (in position order) only if it beats theta.  When
//    lists fill up, the owning waves compact them: an exact radix select
//    finds the k-th largest key tau of the list, the list keeps the entries
//    above tau plus the lowest-position copies of tau, and theta := tau.
//    Later scores equal to tau can never win (their positions are larger),
//    so the rule "score desc, position asc" is preserved exactly.  At the end
//    a last exact compaction leaves the top-k in ascending position order.
//  * Rows with pos + 1 <= k keep every position (no scoring needed); blocks
//    whose rows are all that short skip the GEMM.
//
// Blocks are issued longest-row-first so the causal triangle load-balances.
#include "block_scan.h"
#include "dsa_internal.h"

namespace dsa {

namespace {

constexpr int kRows = 8;          // query rows per block
constexpr int kWaves = 4;         // one per SIMD; two blocks share a CU
constexpr int kRowsPerWave = kRows / kWaves;
constexpr int kThreads = kWaves * 64;
constexpr int kNK = 64;           // keys per tile
constexpr int kMaxK = 4096;

// Candidate list capacity: k + max(k, 1024), and no more than the LDS
// staging area of a compaction when k leaves room for it (k = 2048: 3968).
constexpr int kLdsList = 3968;    // words of one wave's staged list keys
__host__ __device__ inline int cand_cap(int k) {
  int extra = k > 1024 ? k : 1024;
  const int cap = (k + extra + 63) / 64 * 64;
  return (cap > kLdsList && k + 1024 <= kLdsList) ? kLdsList : cap;
}

// Wait until this wave's vector-memory operations (loads, stores, global ->
// LDS copies) have completed, then barrier with the LDS traffic drained.
// The wait is the builtin so the compiler knows nothing is outstanding.
__device__ __forceinline__ void drain_barrier() {
  __builtin_amdgcn_s_waitcnt(0);
  asm volatile("s_barrier" ::: "memory");
}

__device__ __forceinline__ v8i lds_load32(const unsigned char* p) {
  const v4i lo = *reinterpret_cast<const v4i*>(p);
  const v4i hi = *reinterpret_cast<const v4i*>(p + 16);
  return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

__device__ __forceinline__ v8i glb_load32(const uint8_t* p) {
  const v4i lo = *reinterpret_cast<const v4i*>(p);
  const v4i hi = *reinterpret_cast<const v4i*>(p + 16);
  return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

__device__ __forceinline__ v4f mfma_fp8(v8i a, v8i b) {
  v4f z = {0.f, 0.f, 0.f, 0.f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, z, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ void wave_sync_mem() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
  __builtin_amdgcn_wave_barrier();
}

__device__ __forceinline__ uint32_t wave_min(uint32_t v) {
  for (int o = 32; o > 0; o >>= 1) v = min(v, (uint32_t)__shfl_xor((int)v, o, 64));
  return v;
}
__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
  for (int o = 32; o > 0; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o, 64));
  return v;
}

// Threshold-only compaction of one row's candidate list by one wave: one
// histogram pass over the 8 key bits below the list's common prefix finds
// the bin holding the want-th largest key; every entry at or above that
// bin's floor tau is kept (at least `want` of them), the rest dropped, in
// the original order.  No dropped entry can be among the final top `want`,
// and a later key can only enter if it is > tau: with >= want kept entries
// at or above tau, a later key equal to tau loses on position.  Returns tau.
__device__ uint32_t wave_trim(uint32_t* ekey, uint32_t* eidx, int& n, int want, uint32_t* hist);

// Exact compaction of one row's candidate list by one wave.
// Keeps the `want` best entries under (key desc, position asc), in the
// original (position-ascending) order.  Returns tau, the smallest kept key
// (0 if nothing was dropped).  `hist` is this wave's 256-word LDS area.
// Every pass over the list keeps kU loads per lane in flight.
constexpr int kU = 8;
__device__ uint32_t wave_compact(uint32_t* ekey, uint32_t* eidx, int& n, int want, uint32_t* hist) {
  const int lane = threadIdx.x & 63;
  const unsigned long long lt = (1ull << lane) - 1ull;
  if (n <= want) return 0u;
  __builtin_amdgcn_s_waitcnt(0);  // this wave's candidate stores have landed
  wave_sync_mem();
  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
  for (int base = 0; base < n; base += 64 * kU) {
    uint32_t u[kU];
#pragma unroll
    for (int j = 0; j < kU; ++j) {
      const int i = base + 64 * j + lane;
      u[j] = i < n ? ekey[i] : 0u;
    }
#pragma unroll
    for (int j = 0; j < kU; ++j)
      if (base + 64 * j + lane < n) {
        mn = min(mn, u[j]);
        mx = max(mx, u[j]);
      }
  }
  mn = wave_min(mn);
  mx = wave_max(mx);
  uint32_t tau = mn, rem = (uint32_t)want;
  if (mn != mx) {
    const int common = __clz(mn ^ mx);  // leading bits shared by every key
    int rem_bits = 32 - common;
    uint32_t prefix = common == 0 ? 0u : (mn & (0xFFFFFFFFu << rem_bits));
    while (rem_bits > 0) {
      const int nb = rem_bits < 8 ? rem_bits : 8;
      const int shift = rem_bits - nb;
      const uint32_t dmask = (1u << nb) - 1u;
      for (int i = lane; i < 256; i += 64) hist[i] = 0u;
      wave_sync_mem();
      const uint32_t hi = rem_bits >= 32 ? 0u : prefix >> rem_bits;
      for (int base = 0; base < n; base += 64 * kU) {
        uint32_t u[kU];
#pragma unroll
        for (int j = 0; j < kU; ++j) {
          const int i = base + 64 * j + lane;
          u[j] = i < n ? ekey[i] : 0u;
        }
#pragma unroll
        for (int j = 0; j < kU; ++j)
          if (base + 64 * j + lane < n && (rem_bits >= 32 ? 0u : u[j] >> rem_bits) == hi)
            atomicAdd(&hist[(u[j] >> shift) & dmask], 1u);
      }
      wave_sync_mem();
      const int d0 = 4 * (63 - lane);
      uint32_t c[4], tot = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        c[j] = hist[d0 + 3 - j];
        tot += c[j];
      }
      const uint32_t above = wave_inclusive_sum(tot) - tot;
      uint32_t dsel = 0, asel = 0;
      const bool mine = above < rem && rem <= above + tot;
      if (mine) {
        uint32_t acc = above;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (acc < rem && rem <= acc + c[j]) {
            dsel = (uint32_t)(d0 + 3 - j);
            asel = acc;
          }
          acc += c[j];
        }
      }
      const unsigned long long who = __ballot(mine);
      const int src = __ffsll((long long)who) - 1;
      dsel = (uint32_t)__shfl((int)dsel, src, 64);
      asel = (uint32_t)__shfl((int)asel, src, 64);
      prefix |= dsel << shift;
      rem -= asel;
      rem_bits = shift;
      wave_sync_mem();
    }
    tau = prefix;
  }
  // Stable in-place compaction: keep key > tau and the first `rem` copies of
  // tau.  Entries are read kU chunks of 64 ahead of the writes; writes never
  // pass the reads (w <= i), so in-place is safe.
  int w = 0;
  uint32_t eq_seen = 0;
  for (int base = 0; base < n; base += 64 * kU) {
    uint32_t u[kU], p[kU];
#pragma unroll
    for (int j = 0; j < kU; ++j) {
      const int i = base + 64 * j + lane;
      u[j] = i < n ? ekey[i] : 0u;
      p[j] = i < n ? eidx[i] : 0u;
    }
    wave_sync_mem();  // all reads of these chunks are done before any write
#pragma unroll
    for (int j = 0; j < kU; ++j) {
      const int i = base + 64 * j + lane;
      const bool eq = i < n && u[j] == tau;
      const unsigned long long eqb = __ballot(eq);
      const uint32_t eq_rank = eq_seen + (uint32_t)__popcll(eqb & lt);
      const bool keep = i < n && (u[j] > tau || (eq && eq_rank < rem));
      const unsigned long long kb = __ballot(keep);
      if (keep) {
        const int slot = w + __popcll(kb & lt);
        ekey[slot] = u[j];
        eidx[slot] = p[j];
      }
      w += __popcll(kb);
      eq_seen += (uint32_t)__popcll(eqb);
    }
  }
  n = w;
  wave_sync_mem();
  return tau;
}

__device__ uint32_t wave_trim(uint32_t* ekey, uint32_t* eidx, int& n, int want, uint32_t* hist) {
  const int lane = threadIdx.x & 63;
  const unsigned long long lt = (1ull << lane) - 1ull;
  if (n <= want) return 0u;
  __builtin_amdgcn_s_waitcnt(0);  // this wave's candidate stores have landed
  wave_sync_mem();
  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
  for (int base = 0; base < n; base += 64 * kU) {
    uint32_t u[kU];
#pragma unroll
    for (int j = 0; j < kU; ++j) {
      const int i = base + 64 * j + lane;
      u[j] = i < n ? ekey[i] : 0u;
    }
#pragma unroll
    for (int j = 0; j < kU; ++j)
      if (base + 64 * j + lane < n) {
        mn = min(mn, u[j]);
        mx = max(mx, u[j]);
      }
  }
  mn = wave_min(mn);
  mx = wave_max(mx);
  if (mn == mx) return 0u;  // all keys equal: nothing can be dropped by key
  const int rem_bits = 32 - __clz(mn ^ mx);
  const int nb = rem_bits < 8 ? rem_bits : 8;
  const int shift = rem_bits - nb;
  const uint32_t dmask = (1u << nb) - 1u;
  const uint32_t prefix = rem_bits >= 32 ? 0u : (mn & (0xFFFFFFFFu << rem_bits));
  for (int i = lane; i < 256; i += 64) hist[i] = 0u;
  wave_sync_mem();
  for (int base = 0; base < n; base += 64 * kU) {
    uint32_t u[kU];
#pragma unroll
    for (int j = 0; j < kU; ++j) {
      const int i = base + 64 * j + lane;
      u[j] = i < n ? ekey[i] : 0u;
    }
#pragma unroll
    for (int j = 0; j < kU; ++j)
      if (base + 64 * j + lane < n) atomicAdd(&hist[(u[j] >> shift) & dmask], 1u);
  }
  wave_sync_mem();
  const int d0 = 4 * (63 - lane);
  uint32_t c[4], tot = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    c[j] = hist[d0 + 3 - j];
    tot += c[j];
  }
  const uint32_t rem = (uint32_t)want;
  const uint32_t above = wave_inclusive_sum(tot) - tot;
  uint32_t dsel = 0;
  const bool mine = above < rem && rem <= above + tot;
  if (mine) {
    uint32_t acc = above;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (acc < rem && rem <= acc + c[j]) dsel = (uint32_t)(d0 + 3 - j);
      acc += c[j];
    }
  }
  const unsigned long long who = __ballot(mine);
  const int src = __ffsll((long long)who) - 1;
  dsel = (uint32_t)__shfl((int)dsel, src, 64);
  const uint32_t tau = prefix | (dsel << shift);  // floor of the bin holding the want-th key
  wave_sync_mem();
  int w = 0;
  for (int base = 0; base < n; base += 64 * kU) {
    uint32_t u[kU], p[kU];
#pragma unroll
    for (int j = 0; j < kU; ++j) {
      const int i = base + 64 * j + lane;
      u[j] = i < n ? ekey[i] : 0u;
      p[j] = i < n ? eidx[i] : 0u;
    }
    wave_sync_mem();  // all reads of these chunks are done before any write
#pragma unroll
    for (int j = 0; j < kU; ++j) {
      const int i = base + 64 * j + lane;
      const bool keep = i < n && u[j] >= tau;
      const unsigned long long kb = __ballot(keep);
      if (keep) {
        const int slot = w + __popcll(kb & lt);
        ekey[slot] = u[j];
        eidx[slot] = p[j];
      }
      w += __popcll(kb);
    }
  }
  n = w;
  wave_sync_mem();
  return tau;
}

// Exact compaction with the keys staged in LDS (lk: this wave's kLdsList
// words): the keys come in with one copy, the min/max and every radix pass
// read LDS, and the positions are read once, on the way out.  Same result
// as wave_compact.  A radix pass whose selected bin is taken whole ends the
// search: every key at or above the bin's floor is kept and tau is that
// floor (no dropped key reaches it, so later keys equal to it still lose).
// FINAL: the kept positions go to pout[0..want), -1 padded, instead of back
// into the list (a list of at most `want` entries is copied out as it is).
template <bool FINAL>
__device__ uint32_t wave_compact_lds(uint32_t* ekey, uint32_t* eidx, int& n, int want, int cap, uint32_t* hist,
                                     uint32_t* lk, int32_t* pout) {
  const int lane = threadIdx.x & 63;
  const unsigned long long lt = (1ull << lane) - 1ull;
  const int nn = n;
  if (!FINAL && nn <= want) return 0u;
  __builtin_amdgcn_s_waitcnt(0);  // this wave's candidate stores have landed
  wave_sync_mem();
  const bool select = nn > want;
  uint32_t tau = 0u, rem = (uint32_t)want;
  if (select) {
    // Lane l copies words 256b + 4l .. 256b + 4l + 3 of 1 KB block b, for
    // the words that hold entries (nn <= cap <= kLdsList, a multiple of 4).
    const int nblk = (nn + 255) / 256;
    for (int b = 0; b < nblk; ++b)
      if (256 * b + 4 * lane < nn) dma16_lds(ekey, 4u * (uint32_t)min(256 * b + 4 * lane, cap - 4), lk + 256 * b);
    __builtin_amdgcn_s_waitcnt(0);
    wave_sync_mem();
    uint32_t mn = 0xFFFFFFFFu, mx = 0u;
    for (int i = 4 * lane; i < nn; i += 256) {
      const v4i v = *reinterpret_cast<const v4i*>(lk + i);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (i + e < nn) {
          mn = min(mn, (uint32_t)v[e]);
          mx = max(mx, (uint32_t)v[e]);
        }
    }
    mn = wave_min(mn);
    mx = wave_max(mx);
    tau = mn;
    if (mn != mx) {
      const int common = __clz(mn ^ mx);  // leading bits shared by every key
      int rem_bits = 32 - common;
      uint32_t prefix = common == 0 ? 0u : (mn & (0xFFFFFFFFu << rem_bits));
      while (rem_bits > 0) {
        const int nb = rem_bits < 8 ? rem_bits : 8;
        const int shift = rem_bits - nb;
        const uint32_t dmask = (1u << nb) - 1u;
        for (int i = lane; i < 256; i += 64) hist[i] = 0u;
        wave_sync_mem();
        const uint32_t hi = rem_bits >= 32 ? 0u : prefix >> rem_bits;
        for (int i = 4 * lane; i < nn; i += 256) {
          const v4i v = *reinterpret_cast<const v4i*>(lk + i);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t u = (uint32_t)v[e];
            if (i + e < nn && (rem_bits >= 32 ? 0u : u >> rem_bits) == hi) atomicAdd(&hist[(u >> shift) & dmask], 1u);
          }
        }
        wave_sync_mem();
        const int d0 = 4 * (63 - lane);
        uint32_t c[4], tot = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          c[j] = hist[d0 + 3 - j];
          tot += c[j];
        }
        const uint32_t above = wave_inclusive_sum(tot) - tot;
        uint32_t dsel = 0, asel = 0, csel = 0;
        const bool mine = above < rem && rem <= above + tot;
        if (mine) {
          uint32_t acc = above;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if (acc < rem && rem <= acc + c[j]) {
              dsel = (uint32_t)(d0 + 3 - j);
              asel = acc;
              csel = c[j];
            }
            acc += c[j];
          }
        }
        const unsigned long long who = __ballot(mine);
        const int src = __ffsll((long long)who) - 1;
        dsel = (uint32_t)__shfl((int)dsel, src, 64);
        asel = (uint32_t)__shfl((int)asel, src, 64);
        csel = (uint32_t)__shfl((int)csel, src, 64);
        prefix |= dsel << shift;
        rem -= asel;
        rem_bits = shift;
        wave_sync_mem();
        if (csel == rem) break;  // the whole bin is kept
      }
      tau = prefix;
    }
  }
  // Keep key > tau and the first `rem` copies of tau, in list order, 64
  // entries a step (entry 64j + lane).  Kept entries only move down (slot <=
  // index) and a batch's positions are read before its writes: in place.
  int w = 0;
  uint32_t eq_seen = 0;
  const int nstr = (nn + 63) / 64;
  constexpr int kWB = 16;
  for (int j0 = 0; j0 < nstr; j0 += kWB) {
    uint32_t p[kWB];
#pragma unroll
    for (int jj = 0; jj < kWB; ++jj) p[jj] = eidx[min(64 * (j0 + jj) + lane, nn - 1)];
    wave_sync_mem();
#pragma unroll
    for (int jj = 0; jj < kWB; ++jj) {
      if (j0 + jj < nstr) {
        const int i = 64 * (j0 + jj) + lane;
        const uint32_t u = lk[min(i, kLdsList - 1)];
        const bool eq = select && i < nn && u == tau;
        const unsigned long long eqb = __ballot(eq);
        const uint32_t eq_rank = eq_seen + (uint32_t)__popcll(eqb & lt);
        const bool keep = i < nn && (!select || u > tau || (eq && eq_rank < rem));
        const unsigned long long kb = __ballot(keep);
        if (keep) {
          const int slot = w + __popcll(kb & lt);
          if (FINAL) {
            pout[slot] = (int32_t)p[jj];
          } else {
            ekey[slot] = u;
            eidx[slot] = p[jj];
          }
        }
        w += __popcll(kb);
        eq_seen += (uint32_t)__popcll(eqb);
      }
    }
  }
  if (FINAL)
    for (int j = w + lane; j < want; j += 64) pout[j] = -1;
  n = w;
  wave_sync_mem();
  return tau;
}

template <bool PAGED>
__global__ __launch_bounds__(kThreads, 2) void k_prefill(IndexerArgs a, int k, int32_t* idx_out, void* ws, int cap) {
  constexpr int R = kRowsPerWave;
  // K tiles: 128-byte rows, the 16-byte chunk ch of key j at slot ch ^ (j & 7)
  // (the MFMA operand reads of 8 consecutive keys then hit distinct banks).
  __shared__ __attribute__((aligned(16))) unsigned char ktile[2][kNK * kDI];
  __shared__ float ksc[2][kNK];
  __shared__ __attribute__((aligned(16))) uint32_t lkeys[kWaves][kLdsList];  // per-wave staged list keys
  // Two blocks share a CU's LDS (80 KB each): a compaction's per-wave
  // 256-word histograms live in the key buffer of the tile just consumed.
  static_assert(kWaves * 256 * 4 <= kNK * kDI, "compaction histograms fit one key buffer");
  auto hist_of = [&](int buf) { return reinterpret_cast<uint32_t*>(&ktile[buf][0]) + 256 * (threadIdx.x >> 6); };
  __shared__ int need_compact;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, c = lane & 15;
  const unsigned long long lt = (1ull << lane) - 1ull;

  // Longest rows first: block j -> query block nqb-1-j/B.  The B blocks of a
  // query block take the sequences in an order rotated once per round of 8
  // blocks: the XCDs take blocks round-robin, so with several sequences every
  // XCD sees all of them instead of a fixed subset.
  const int nqb = (a.q_len + kRows - 1) / kRows;
  const int grp = (int)blockIdx.x / a.B;
  const int b = ((int)blockIdx.x % a.B + grp / max(1, 8 / a.B)) % a.B;
  const int qb = nqb - 1 - grp;
  const int L = clamped_len(a.seq_lens, b, a.S_max);
  const int i0 = qb * kRows;                       // first query index in the sequence
  const int nrows = min(kRows, a.q_len - i0);
  const int t_base = b * a.q_len + i0;
  const int maxpos = L - a.q_len + i0 + nrows - 1;  // position of the last row

  // This wave's rows.
  int rpos[R];
  bool rvalid[R];
  int rt[R];
#pragma unroll
  for (int rr = 0; rr < R; ++rr) {
    const int ri = __builtin_amdgcn_readfirstlane(R * wave + rr);
    rvalid[rr] = ri < nrows;
    rt[rr] = t_base + ri;
    rpos[rr] = rvalid[rr] ? L - a.q_len + i0 + ri : -1;
  }

  if (maxpos + 1 <= k) {  // every row keeps all of its positions
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
      if (!rvalid[rr]) continue;
      int32_t* out = idx_out + (size_t)rt[rr] * k;
      for (int j = lane; j < k; j += 64) out[j] = (j <= rpos[rr]) ? j : -1;
    }
    return;
  }

  // Candidate lists of this wave's rows.
  uint32_t* ekey[R];
  uint32_t* eidx[R];
#pragma unroll
  for (int rr = 0; rr < R; ++rr) {
    uint32_t* base = static_cast<uint32_t*>(ws) + (size_t)(rt[rr] - a.row_begin) * 2 * cap;
    ekey[rr] = base;
    eidx[rr] = base + cap;
  }
  int n[R];
  uint32_t theta[R];  // below every real key: everything valid enters
#pragma unroll
  for (int rr = 0; rr < R; ++rr) {
    n[rr] = 0;
    theta[rr] = 0u;
  }

  // Query fragments and head weights (heads 16m + 4g + i of the MFMA output rows).
  const uint8_t* qb8 = static_cast<const uint8_t*>(a.q);
  v8i qf[R][4];
  float wv[R][4][4];
#pragma unroll
  for (int rr = 0; rr < R; ++rr) {
    const size_t t = (size_t)rt[rr];
#pragma unroll
    for (int m = 0; m < 4; ++m)
      qf[rr][m] = rvalid[rr] ? glb_load32(qb8 + (t * kHI + 16 * m + c) * kDI + 32 * g) : v8i{0, 0, 0, 0, 0, 0, 0, 0};
    if (rvalid[rr]) {
      load_head_weights(a.w, a.w_is_bf16, a.q_scale, t, g, wv[rr]);
    } else {
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) wv[rr][m][i] = 0.f;
    }
  }

  // Key tiles are copied straight from global memory into LDS, one tile
  // ahead: in copy j (of kNK / (8 kWaves)) wave w moves keys 8(kWaves j + w)
  // .. +7 of a tile (lane l: key + l/8, slot l%8); wave 0 also moves the
  // tile's 64 k-scales.  Keys past the last row's position read that
  // position's row (their scores are masked).
  const uint8_t* kb8 = static_cast<const uint8_t*>(a.k) + (PAGED ? 0 : (size_t)b * a.S_max * kDI);
  const float* ksb = a.k_scale ? a.k_scale + (PAGED ? 0 : (size_t)b * a.S_max) : nullptr;
  const int ntiles = (maxpos + kNK) / kNK;
  constexpr int kCopies = kNK / (8 * kWaves);
  static_assert(kCopies * 8 * kWaves == kNK, "whole 16-byte copies per lane per tile");
  // Paged caches: a page holds a power of two >= 64 tokens, so a 64-key
  // tile lies inside one page.  Lane i holds the id of page 64*pbatch + i of
  // this sequence (64 pages per batch, refilled when the tiles move past
  // them); a tile's page is a readlane, so no table read sits in front of its
  // copies except once per 64 pages.
  int pbatch = -1, lane_page = 0;
  const int last_j = PAGED ? maxpos >> a.pages.shift : 0;
  auto tile_rows = [&](int ti) -> long long {  // pool row of key ti*kNK
    if constexpr (PAGED) {
      const int s0 = ti * kNK, j = s0 >> a.pages.shift;
      if ((j >> 6) != pbatch) {
        pbatch = j >> 6;
        lane_page = a.pages.page(b, min(64 * pbatch + lane, last_j));
      }
      const int pg = __builtin_amdgcn_readlane(lane_page, j & 63);
      return ((long long)pg << a.pages.shift) | (s0 & ((1 << a.pages.shift) - 1));
    } else {
      return (long long)ti * kNK;
    }
  };
  auto issue = [&](int ti, int buf) {
    const long long row0 = tile_rows(ti);  // keys ti*kNK .. +63 are rows row0 .. +63
#pragma unroll
    for (int j = 0; j < kCopies; ++j) {
      const int kb0 = 8 * (kWaves * j + wave);  // first key of this copy within the tile
      const int key = ti * kNK + kb0 + (lane >> 3);
      const int kc = min(key, maxpos) - ti * kNK;
      const uint32_t chunk = (uint32_t)((lane & 7) ^ (key & 7));
      dma16_lds(kb8 + row0 * kDI, (uint32_t)kc * kDI + 16u * chunk, &ktile[buf][kb0 * kDI]);
    }
    if (wave == 0 && ksb) dma4_lds(ksb + row0, 4u * (uint32_t)(min(ti * kNK + lane, maxpos) - ti * kNK), &ksc[buf][0]);
  };

  // A tile's accepted candidates are stored at the start of the next tile
  // (next to that tile's copy), so the end-of-tile wait finds both long done.
  bool pend[R];
  uint32_t pu[R], ps[R];
  int pslot[R];
#pragma unroll
  for (int rr = 0; rr < R; ++rr) pend[rr] = false;
  auto flush = [&]() {
#pragma unroll
    for (int rr = 0; rr < R; ++rr)
      if (pend[rr]) {
        store_u32_nowait(ekey[rr] + pslot[rr], pu[rr]);
        store_u32_nowait(eidx[rr] + pslot[rr], ps[rr]);
        pend[rr] = false;
      }
  };

  if (tid == 0) need_compact = 0;
  if (!ksb && tid < 2 * kNK) ksc[tid / kNK][tid % kNK] = 1.f;
  issue(0, 0);
  drain_barrier();

  for (int ti = 0; ti < ntiles; ++ti) {
    const int buf = ti & 1;
    const int tile0 = ti * kNK;
    if (ti + 1 < ntiles) issue(ti + 1, buf ^ 1);
    flush();

    if (rpos[0] >= tile0 || rpos[R - 1] >= tile0) {  // positions grow with rr
      // Every row of the wave is computed (a row past its position only
      // masks its scores below).  Per key block: the two B-operand reads,
      // all eight MFMAs, then the ReLU / weight epilogue of both rows.
      float x[R][4];
#pragma unroll
      for (int blk = 0; blk < 4; ++blk) {
        const unsigned char* krow = &ktile[buf][(16 * blk + c) * kDI];
        const int sw = c & 7;
        const v4i lo = *reinterpret_cast<const v4i*>(krow + 16 * ((2 * g) ^ sw));
        const v4i hi = *reinterpret_cast<const v4i*>(krow + 16 * ((2 * g + 1) ^ sw));
        const v8i kf = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        v4f d[R][4];
#pragma unroll
        for (int rr = 0; rr < R; ++rr)
#pragma unroll
          for (int m = 0; m < 4; ++m) d[rr][m] = mfma_fp8(qf[rr][m], kf);
#pragma unroll
        for (int rr = 0; rr < R; ++rr) {
          float acc = 0.f;
#pragma unroll
          for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc = fmaf(wv[rr][m][i], relu(d[rr][m][i]), acc);
          x[rr][blk] = acc;
        }
        __builtin_amdgcn_sched_group_barrier(0x0100, 2, 0);        // the B-operand reads
        __builtin_amdgcn_sched_group_barrier(0x0008, 4 * R, 0);    // the MFMAs
        __builtin_amdgcn_sched_group_barrier(0x0002, 64 * R, 0);   // the epilogue
      }
      const float ks = ksc[buf][lane];
      const int s = tile0 + lane;
#pragma unroll
      for (int rr = 0; rr < R; ++rr) {
        auto p01 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x[rr][0]), __float_as_uint(x[rr][1]), false, false);
        auto p23 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x[rr][2]), __float_as_uint(x[rr][3]), false, false);
        const float a01 = __uint_as_float(p01[0]) + __uint_as_float(p01[1]);
        const float a23 = __uint_as_float(p23[0]) + __uint_as_float(p23[1]);
        auto pf = __builtin_amdgcn_permlane32_swap(__float_as_uint(a01), __float_as_uint(a23), false, false);
        const float score = (__uint_as_float(pf[0]) + __uint_as_float(pf[1])) * ks;
        const uint32_t u = order_key(score);
        const bool valid = s <= rpos[rr];
        const bool pred = valid && u > theta[rr];
        const unsigned long long ball = __ballot(pred);
        pend[rr] = pred;
        pu[rr] = u;
        ps[rr] = (uint32_t)s;
        pslot[rr] = n[rr] + __popcll(ball & lt);
        n[rr] += __popcll(ball);
      }
      bool full = false;
#pragma unroll
      for (int rr = 0; rr < R; ++rr) full = full || n[rr] > cap - kNK;
      if (lane == 0 && full) atomicOr(&need_compact, 1);
    }

    // This wave's copies of tile ti+1 (and its candidate stores) are done;
    // after the barrier every wave's are, and tile ti is free.
    drain_barrier();
    if (need_compact) {
      flush();
      // Batched: every wave trims its fuller lists so the trims overlap.
      // A trim keeps the keys at or above a threshold (>= k entries); if
      // that would leave the list nearly full, the exact compaction runs.
      const int trigger = k + (cap - k) / 2;
#pragma unroll
      for (int rr = 0; rr < R; ++rr)
        if (n[rr] > trigger) {
          uint32_t tau;
          if (cap <= kLdsList) {
            tau = wave_compact_lds<false>(ekey[rr], eidx[rr], n[rr], k, cap, hist_of(buf), lkeys[wave], nullptr);
          } else {
            tau = wave_trim(ekey[rr], eidx[rr], n[rr], k, hist_of(buf));
            if (n[rr] > trigger) tau = wave_compact(ekey[rr], eidx[rr], n[rr], k, hist_of(buf));
          }
          theta[rr] = max(theta[rr], tau);
        }
      __syncthreads();
      if (tid == 0) need_compact = 0;
      // nothing of the compaction stays in flight into the next tile (the
      // compiler would otherwise wait for it inside the MFMA sequence)
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
  }

  flush();

  // Final exact selection and output (ascending positions, -1 padded).
#pragma unroll
  for (int rr = 0; rr < R; ++rr) {
    if (!rvalid[rr]) continue;
    int32_t* out = idx_out + (size_t)rt[rr] * k;
    if (rpos[rr] + 1 <= k) {
      for (int j = lane; j < k; j += 64) out[j] = (j <= rpos[rr]) ? j : -1;
      continue;
    }
    if (cap <= kLdsList) {
      wave_compact_lds<true>(ekey[rr], eidx[rr], n[rr], k, cap, hist_of(0), lkeys[wave], out);
    } else {
      wave_compact(ekey[rr], eidx[rr], n[rr], k, hist_of(0));
      for (int j = lane; j < k; j += 64) out[j] = (j < n[rr]) ? (int32_t)eidx[rr][j] : -1;
    }
  }
}

}  // namespace

bool prefill_supported(int q_len, int S_max, int k) {
  (void)q_len;
  return k >= 1 && k <= kMaxK && S_max >= 1;
}

size_t prefill_workspace_bytes(int B, int q_len, int S_max, int k) {
  (void)S_max;
  return (size_t)B * q_len * 2 * cand_cap(k) * sizeof(uint32_t);
}

hipError_t launch_indexer_topk_prefill(const IndexerArgs& a, int k, int32_t* idx, void* ws, hipStream_t stream) {
  const int nqb = (a.q_len + kRows - 1) / kRows;
  const dim3 grid((unsigned)(nqb * a.B));
  if (a.pages.table)
    hipLaunchKernelGGL(k_prefill<true>, grid, dim3(kThreads), 0, stream, a, k, idx, ws, cand_cap(k));
  else
    hipLaunchKernelGGL(k_prefill<false>, grid, dim3(kThreads), 0, stream, a, k, idx, ws, cand_cap(k));
  return hipGetLastError();
}

}  // namespace dsa
