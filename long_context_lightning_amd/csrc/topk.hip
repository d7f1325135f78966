// Top-k over materialised score rows (decode / short rows).
//
// Rule ("详解DSA", Indexer code block: topk(min(index_topk, end_pos))):
// V = {s <= pos}; |V| <= k keeps V; otherwise the k positions first in the
// order (score desc, position asc).  Output: ascending positions, -1 padded.
//
// Four launches, all on the caller's stream:
//  1. zero   -- clear the per-row histograms and counters in the workspace.
//  2. hist   -- (row, 8192-score segment) blocks: LDS histogram of the top 12
//               bits of each score's order key, flushed with global atomics.
//  3. gather -- same blocks: every block finds the threshold bin b* (the bin
//               holding the k-th largest) from the row histogram and appends
//               the (key, position) of every score in bins >= b* to the row's
//               candidate list, reserving its range with one atomic; the keys
//               inside b* also go into a second histogram of their next 10
//               bits, and the first segment's block records b*, the count
//               above it and its size.
//  4. final  -- one 1024-thread block per row: the second histogram gives
//               the next 10 bits of the k-th key tau at once; the last 10
//               bits (when that digit bin is not taken whole) come from one
//               radix pass over the candidates; positions with key > tau and
//               the copies of tau go into two LDS bitmaps; the lower-position
//               tie rule keeps the copies up to the want-th set bit of the
//               second; both are written out in ascending order.  If the
//               candidate list would overflow (scores concentrated in one
//               bin) the block selects directly from the score row.
#include "dsa_internal.h"
#include "select.h"

namespace dsa {

namespace {

constexpr int kBins = 4096;     // histogram bins: top 12 bits of the order key (sign, exponent, 3 mantissa bits)
constexpr int kBinShift = 20;
constexpr int kBins2 = 1024;    // second histogram: the next 10 bits of the keys inside the threshold bin
constexpr int kBin2Shift = 10;
constexpr int kSeg = 8192;      // scores per hist/gather block
constexpr int kSegThreads = 512;
constexpr int kFinThreads = 1024;
constexpr int kDigitBits = 8;   // radix digit width of the selection from a score row
constexpr int kFinDigit = 10;   // radix digit width of the selection inside bin b*
constexpr int kMaxK = 4096;
constexpr int kMaxS = 262144;

__host__ __device__ inline size_t cap_for(int k) { return (size_t)2 * k + 4096; }
constexpr int kCapMax = 2 * kMaxK + 4096;  // candidate list bound (k = kMaxK)
__host__ __device__ inline size_t row_stride_bytes(int k) {
  size_t b = (size_t)kBins * 4 + 256 + (size_t)kBins2 * 4 + cap_for(k) * 8;
  return (b + 255) & ~(size_t)255;
}

struct RowWs {
  uint32_t* hist;   // [kBins]
  uint32_t* meta;   // [64]: 0 = candidate count; 1 = b*, 2 = count above b*, 3 = count in b* (gather)
  uint32_t* hist2;  // [kBins2]: next 10 bits of the keys in b*
  uint32_t* ekey;   // [cap]
  uint32_t* eidx;   // [cap]
};
constexpr int kZeroWords = kBins + 64 + kBins2;  // hist, meta and hist2 are contiguous

__device__ __forceinline__ RowWs row_ws(void* ws, int r, int k) {
  char* base = static_cast<char*>(ws) + (size_t)r * row_stride_bytes(k);
  RowWs w;
  w.hist = reinterpret_cast<uint32_t*>(base);
  w.meta = reinterpret_cast<uint32_t*>(base + kBins * 4);
  w.hist2 = reinterpret_cast<uint32_t*>(base + kBins * 4 + 256);
  w.ekey = w.hist2 + kBins2;
  w.eidx = w.ekey + cap_for(k);
  return w;
}

__device__ __forceinline__ int row_valid_count(const TopkArgs& a, int r) {
  const int pos = row_pos(a.seq_lens, a.row_begin + r, a.q_len, a.S_max);
  return pos < 0 ? 0 : pos + 1;
}

__global__ void k_topk_zero(TopkArgs a) {
  const size_t words = (size_t)kZeroWords;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < words * a.row_count;
       i += (size_t)gridDim.x * blockDim.x) {
    const size_t r = i / words, j = i % words;
    RowWs w = row_ws(a.ws, (int)r, a.k);
    w.hist[j] = 0u;  // hist, meta and hist2 are contiguous
  }
}

__global__ __launch_bounds__(kSegThreads) void k_topk_hist(TopkArgs a) {
  __shared__ uint32_t h[kBins];
  const int r = blockIdx.y;
  const int n = row_valid_count(a, r);
  const int seg0 = (int)blockIdx.x * kSeg;
  if (n <= a.k || seg0 >= n) return;
  for (int i = threadIdx.x; i < kBins; i += kSegThreads) h[i] = 0u;
  __syncthreads();
  const float* row = a.scores + (long long)r * a.ld;
  const int e1 = min(seg0 + kSeg, n);
  // all loads first (addresses clamped into the segment, so no branches)
  constexpr int kPer = kSeg / kSegThreads;
  uint32_t key[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int e = seg0 + (int)threadIdx.x + j * kSegThreads;
    key[j] = order_key(row[e < e1 ? e : e1 - 1]);
  }
#pragma unroll
  for (int j = 0; j < kPer; ++j)
    if (seg0 + (int)threadIdx.x + j * kSegThreads < e1) atomicAdd(&h[key[j] >> kBinShift], 1u);
  __syncthreads();
  RowWs w = row_ws(a.ws, r, a.k);
  for (int i = threadIdx.x; i < kBins; i += kSegThreads)
    if (h[i]) atomicAdd(&w.hist[i], h[i]);
}

// Threshold bin: the bin b* with count(bins > b*) < k <= count(bins >= b*).
// Thread t owns the bins [hi - per, hi), hi = kBins - per * t (threads walk
// the bins from the top; NT * per == kBins): load_bins reads them (c[j] is
// bin hi - 1 - j), threshold_from_bins finds b*, the count above it and the
// count in it.  `sm` needs NT/64 + 4 words; on return only sm[NT/64 + 1 ..
// NT/64 + 3] may still be read by other threads.
template <int NT>
__device__ __forceinline__ void load_bins(const uint32_t* hist, uint32_t (&c)[kBins / NT]) {
  constexpr int per = kBins / NT;
  static_assert(per % 4 == 0, "16-byte bin loads");
  const int lo = kBins - per * ((int)threadIdx.x + 1);
#pragma unroll
  for (int q = 0; q < per / 4; ++q) {
    const v4i v = *reinterpret_cast<const v4i*>(hist + lo + 4 * q);
#pragma unroll
    for (int e = 0; e < 4; ++e) c[per - 1 - (4 * q + e)] = (uint32_t)v[e];
  }
}

template <int NT>
__device__ void threshold_from_bins(const uint32_t (&c)[kBins / NT], uint32_t k, uint32_t* sm, uint32_t* out_bin,
                                    uint32_t* out_above, uint32_t* out_inbin) {
  constexpr int per = kBins / NT, NW = NT / 64;
  const int hi = kBins - per * (int)threadIdx.x;
  uint32_t tot = 0;
#pragma unroll
  for (int j = 0; j < per; ++j) tot += c[j];
  if (threadIdx.x == 0) {
    sm[NW + 1] = 0u;
    sm[NW + 2] = 0u;
    sm[NW + 3] = 0u;
  }
  uint32_t total;
  const uint32_t above = block_exclusive_sum_once<NT>(tot, sm, &total);
  if (above < k && k <= above + tot) {
    uint32_t acc = above;
#pragma unroll
    for (int j = 0; j < per; ++j) {
      if (acc < k && k <= acc + c[j]) {
        sm[NW + 1] = (uint32_t)(hi - 1 - j);
        sm[NW + 2] = acc;
        sm[NW + 3] = c[j];
      }
      acc += c[j];
    }
  }
  __syncthreads();
  *out_bin = sm[NW + 1];
  *out_above = sm[NW + 2];
  *out_inbin = sm[NW + 3];
}

__global__ __launch_bounds__(kSegThreads) void k_topk_gather(TopkArgs a) {
  constexpr int kPer = kSeg / kSegThreads;  // scores per thread
  __shared__ uint32_t sm[kSegThreads / 64 + 4];
  __shared__ uint32_t base_sh;
  __shared__ uint32_t h2[kBins2];
  const int r = blockIdx.y;
  const int n = row_valid_count(a, r);
  const int seg0 = (int)blockIdx.x * kSeg;
  if (n <= a.k || seg0 >= n) return;
  const float* row = a.scores + (long long)r * a.ld;
  const int e1 = min(seg0 + kSeg, n);
  RowWs w = row_ws(a.ws, r, a.k);
  // The row histogram's bins are loaded first, then the keys of this
  // thread's scores (kept in registers; addresses clamped into the segment,
  // no branches), so the threshold search waits only for the bins and
  // overlaps the score loads.  One reservation per block.
  uint32_t hb[kBins / kSegThreads];
  load_bins<kSegThreads>(w.hist, hb);
  uint32_t key[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int e = seg0 + (int)threadIdx.x + j * kSegThreads;
    key[j] = order_key(row[e < e1 ? e : e1 - 1]);
  }
  for (int i = threadIdx.x; i < kBins2; i += kSegThreads) h2[i] = 0u;  // cleared before the search's barriers
  uint32_t bstar, above, inbin;
  threshold_from_bins<kSegThreads>(hb, (uint32_t)a.k, sm, &bstar, &above, &inbin);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    w.meta[1] = bstar;
    w.meta[2] = above;
    w.meta[3] = inbin;
  }
  if ((size_t)above + inbin > cap_for(a.k)) return;  // final block takes the direct path
  uint32_t mine = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int e = seg0 + (int)threadIdx.x + j * kSegThreads;
    mine += (e < e1 && (key[j] >> kBinShift) >= bstar) ? 1u : 0u;
  }
  uint32_t total;
  uint32_t off = block_exclusive_sum<kSegThreads>(mine, sm, &total);
  if (total == 0) return;
  if (threadIdx.x == 0) base_sh = atomicAdd(&w.meta[0], total);
  __syncthreads();
  off += base_sh;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int e = seg0 + (int)threadIdx.x + j * kSegThreads;
    if (e < e1 && (key[j] >> kBinShift) >= bstar) {
      w.ekey[off] = key[j];
      w.eidx[off] = (uint32_t)e;
      ++off;
      if ((key[j] >> kBinShift) == bstar) atomicAdd(&h2[(key[j] >> kBin2Shift) & (kBins2 - 1)], 1u);
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < kBins2; i += kSegThreads)
    if (h2[i]) atomicAdd(&w.hist2[i], h2[i]);
}

// LDS of the selection tail (final_lds_bytes): two position bitmaps of
// Wmax words each (16-byte aligned), a digit histogram, per-wave digit
// histograms of the score-row path and a small scratch.
struct SelLds {
  uint32_t* bitmap;  // positions kept
  uint32_t* tbits;   // copies of tau, when ties need the position rule
  uint32_t* hist;    // 1 << kFinDigit
  uint32_t* whist;   // NW << kDigitBits
  uint32_t* sm;      // 64
};

__device__ __forceinline__ SelLds sel_lds(uint32_t* region, int S_max) {
  constexpr int NW = kFinThreads / 64;
  const int Wmax = (((S_max + 31) >> 5) + 3) & ~3;  // words, rounded up to 16 bytes
  SelLds L;
  L.bitmap = region;
  L.tbits = L.bitmap + Wmax;
  L.hist = L.tbits + Wmax;
  L.whist = L.hist + (1 << kFinDigit);
  L.sm = L.whist + (NW << kDigitBits);
  return L;
}

constexpr int kCPer = kCapMax / kFinThreads;  // candidates per thread at most
constexpr int kCPerSmall = 4;                 // ... in the common case (k <= 2048: at most 4096 candidates)

// The first `total` (<= NP * kFinThreads) candidates go to registers:
// thread t holds entries t + j * kFinThreads (slots past the list repeat
// its last entry and are never used).
template <int NP>
__device__ __forceinline__ void load_candidates(const uint32_t* ekey, const uint32_t* eidx, uint32_t total,
                                                uint32_t (&ck)[NP], uint32_t (&cp)[NP]) {
  const uint32_t last = total ? total - 1 : 0u;
#pragma unroll
  for (int j = 0; j < NP; ++j) {
    const uint32_t i = (uint32_t)((int)threadIdx.x + j * kFinThreads);
    const uint32_t ic = i < total ? i : last;
    ck[j] = ekey[ic];
    cp[j] = eidx[ic];
  }
}

__device__ __forceinline__ void clear_bitmaps(const SelLds& L, int W4) {
  for (int i = threadIdx.x; i < W4; i += kFinThreads) {
    L.bitmap[i] = 0u;
    L.tbits[i] = 0u;
  }
}

// Selection tail over the candidates held in registers (total of them, the
// keys and positions of every score at or above the current digit range).
// On entry: the keys whose bits above rem_bits equal prefix >> rem_bits are
// the open range; every candidate above it is kept, and `want` (>= 1) keys
// are still to take inside it; `whole` says the whole range is kept.  The
// bitmaps are cleared, and a barrier separates that from this call.  Each
// further digit (kFinDigit bits, one histogram bin per thread, the scan on
// 16-bin vector reads by one wave) narrows the range; a digit bin taken
// whole ends the search.  Then the kept positions are emitted in ascending
// order (ties to the lower position) and the rest of out is -1.
template <int NP>
__device__ void select_tail(const TopkArgs& a, int n, int32_t* out, const uint32_t (&ck)[NP], const uint32_t (&cp)[NP],
                            uint32_t total, uint32_t prefix, int rem_bits, uint32_t want, bool whole,
                            const SelLds& L) {
  static_assert(kFinThreads == 1 << kFinDigit, "one digit bin per thread");
  const int tid = threadIdx.x;
  while (!whole && rem_bits > 0) {
    const int nb = rem_bits < kFinDigit ? rem_bits : kFinDigit;
    const int shift = rem_bits - nb;
    const uint32_t dmask = (1u << nb) - 1u;
    L.hist[tid] = 0u;
    __syncthreads();
    const uint32_t hi = prefix >> rem_bits;
#pragma unroll
    for (int j = 0; j < NP; ++j)
      if ((uint32_t)(tid + j * kFinThreads) < total && (ck[j] >> rem_bits) == hi)
        atomicAdd(&L.hist[(ck[j] >> shift) & dmask], 1u);
    __syncthreads();
    if (tid < 64) {
      // lane l holds the 16 contiguous digits [d0, d0 + 16) and walks them
      // from the top; lanes go from the highest digits down (digits above
      // 1 << nb are empty)
      constexpr int kPer = (1 << kFinDigit) / 64;
      const int d0 = (1 << kFinDigit) - kPer * (tid + 1);
      uint32_t c[kPer];
#pragma unroll
      for (int q = 0; q < kPer / 4; ++q) {
        const v4i v = *reinterpret_cast<const v4i*>(&L.hist[d0 + 4 * q]);
#pragma unroll
        for (int e = 0; e < 4; ++e) c[4 * q + e] = (uint32_t)v[e];
      }
      uint32_t tot = 0;
#pragma unroll
      for (int j = 0; j < kPer; ++j) tot += c[j];
      const uint32_t abv = wave_inclusive_sum(tot) - tot;
      if (abv < want && want <= abv + tot) {
        uint32_t acc = abv;
#pragma unroll
        for (int j = kPer - 1; j >= 0; --j) {
          if (acc < want && want <= acc + c[j]) {
            L.sm[0] = (uint32_t)(d0 + j);
            L.sm[1] = acc;
            L.sm[2] = c[j];
          }
          acc += c[j];
        }
      }
    }
    __syncthreads();
    prefix |= L.sm[0] << shift;
    want -= L.sm[1];
    rem_bits = shift;
    whole = L.sm[2] == want;  // this digit bin is kept whole
  }
  // tau = prefix.  whole: keep key >= tau (every key of the open range).
  // Otherwise keep key > tau and the `want` lowest positions among the
  // copies of tau.
  const uint32_t tau = prefix;
#pragma unroll
  for (int j = 0; j < NP; ++j) {
    if ((uint32_t)(tid + j * kFinThreads) < total) {
      const uint32_t kk = ck[j], p = cp[j];
      if (kk > tau || (whole && kk == tau)) atomicOr(&L.bitmap[p >> 5], 1u << (p & 31));
      else if (kk == tau) atomicOr(&L.tbits[p >> 5], 1u << (p & 31));
    }
  }
  __syncthreads();
  const uint32_t written = whole ? bitmap_emit<kFinThreads>(L.bitmap, n, out, (uint32_t)a.k, L.sm)
                                 : bitmap_select_emit<kFinThreads>(L.bitmap, L.tbits, n, want, out, (uint32_t)a.k, L.sm);
  for (int j = (int)min(written, (uint32_t)a.k) + tid; j < a.k; j += kFinThreads) out[j] = -1;
}

// Selection of row r straight from its score row (the candidate list would
// overflow: scores concentrated in one bin): radix select of the k-th key
// with kDigitBits-bit digits over the row, then the bitmaps and the emit.
__device__ void select_direct(const TopkArgs& a, int r, int n, int32_t* out, const SelLds& L) {
  const int tid = threadIdx.x;
  const float* row = a.scores + (long long)r * a.ld;
  const int W4 = (((n + 31) >> 5) + 3) & ~3;  // words, rounded up to 16 bytes
  uint32_t tau = 0u, want = (uint32_t)a.k;
  radix_select_desc<kFinThreads, kDigitBits>(
      [&](auto f) {
        for (int e = tid; e < n; e += kFinThreads) f(order_key(row[e]));
      },
      tau, 32, want, L.whist, L.sm);
  clear_bitmaps(L, W4);
  __syncthreads();
  for (int e = tid; e < n; e += kFinThreads) {
    const uint32_t kk = order_key(row[e]);
    if (kk > tau) atomicOr(&L.bitmap[e >> 5], 1u << (e & 31));
    else if (kk == tau) atomicOr(&L.tbits[e >> 5], 1u << (e & 31));
  }
  __syncthreads();
  const uint32_t written = bitmap_select_emit<kFinThreads>(L.bitmap, L.tbits, n, want, out, (uint32_t)a.k, L.sm);
  for (int j = (int)min(written, (uint32_t)a.k) + tid; j < a.k; j += kFinThreads) out[j] = -1;
}

// Exact selection of row r (n > k valid positions) given its threshold bin
// b* (count(bins > b*) = above < k <= above + inbin) and its candidate list
// (ekey, eidx: the keys and positions of every score in the bins at or
// above b*, above + inbin of them, unless that exceeds cap_for(k), in which
// case the row is selected straight from the scores).  region: the LDS
// layout of final_lds_bytes.  Called by all kFinThreads threads of the block.
__device__ void select_row(const TopkArgs& a, int r, int n, int32_t* out, uint32_t bstar, uint32_t above,
                           uint32_t inbin, const uint32_t* ekey, const uint32_t* eidx, uint32_t* region) {
  const SelLds L = sel_lds(region, a.S_max);
  const uint32_t total = above + inbin;
  if (total > (uint32_t)cap_for(a.k)) {
    select_direct(a, r, n, out, L);
    return;
  }
  auto run = [&](auto np) {
    constexpr int NP = decltype(np)::value;
    uint32_t ck[NP], cp[NP];
    load_candidates<NP>(ekey, eidx, total, ck, cp);
    clear_bitmaps(L, (((n + 31) >> 5) + 3) & ~3);
    select_tail<NP>(a, n, out, ck, cp, total, bstar << kBinShift, kBinShift, (uint32_t)a.k - above, false, L);
  };
  if (total <= (uint32_t)(kCPerSmall * kFinThreads))
    run(std::integral_constant<int, kCPerSmall>());
  else
    run(std::integral_constant<int, kCPer>());
}

// With a.rows set, the row's selection (already in `out`, written by this
// block before the barrier) is also written as pool rows of a.pages, so a
// paged attention needs no translation launch of its own.
__device__ __forceinline__ void emit_pool_rows(const TopkArgs& a, int r, const int32_t* out) {
  if (!a.rows) return;
  __syncthreads();
  const int t = a.row_begin + r;
  const int pos = row_pos(a.seq_lens, t, a.q_len, a.S_max);
  const int b = t / a.q_len;
  int32_t* rows = a.rows + (long long)r * a.k;
  for (int j = threadIdx.x; j < a.k; j += blockDim.x) rows[j] = page_row(out[j], pos, b, a.pages);
}

// The final selection of a row whose candidates fit the list (total of
// them, at most NP per thread): the gather's histogram of bin b* gives the
// next 10 bits of tau, select_tail the rest.
// Wave 0's lane l reads the 16 contiguous second-histogram digits
// [kBins2 - 16 (l + 1), kBins2 - 16 l): c[j] is digit d0 + j.
__device__ __forceinline__ void load_hist2(const uint32_t* hist2, uint32_t (&c)[kBins2 / 64]) {
  constexpr int kPer = kBins2 / 64;
  const int d0 = kBins2 - kPer * ((int)threadIdx.x + 1);
#pragma unroll
  for (int q = 0; q < kPer / 4; ++q) {
    const v4i v = *reinterpret_cast<const v4i*>(&hist2[d0 + 4 * q]);
#pragma unroll
    for (int e = 0; e < 4; ++e) c[4 * q + e] = (uint32_t)v[e];
  }
}
template <int NP>
__device__ void final_from_candidates(const TopkArgs& a, int n, int32_t* out, uint32_t bstar, uint32_t above,
                                      uint32_t total, const uint32_t (&c)[kBins2 / 64], const RowWs& w,
                                      const SelLds& L) {
  uint32_t ck[NP], cp[NP];
  load_candidates<NP>(w.ekey, w.eidx, total, ck, cp);
  clear_bitmaps(L, (((n + 31) >> 5) + 3) & ~3);
  const uint32_t want = (uint32_t)a.k - above;
  // The next 10 bits of tau come from the gather's histogram of bin b*
  // (wave 0's c, from load_hist2): lane l holds the 16 contiguous digits
  // [d0, d0 + 16) and the lanes walk them from the top, as in the digit scan
  // of select_tail.
  if (threadIdx.x < 64) {
    constexpr int kPer = kBins2 / 64;
    const int d0 = kBins2 - kPer * ((int)threadIdx.x + 1);
    uint32_t tot = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) tot += c[j];
    const uint32_t abv = wave_inclusive_sum(tot) - tot;
    if (abv < want && want <= abv + tot) {
      uint32_t acc = abv;
#pragma unroll
      for (int j = kPer - 1; j >= 0; --j) {
        if (acc < want && want <= acc + c[j]) {
          L.sm[0] = (uint32_t)(d0 + j);
          L.sm[1] = acc;
          L.sm[2] = c[j];
        }
        acc += c[j];
      }
    }
  }
  __syncthreads();  // also orders the bitmap clears before the selection's bitmap writes
  const uint32_t want2 = want - L.sm[1];
  const uint32_t prefix = (bstar << kBinShift) | (L.sm[0] << kBin2Shift);
  select_tail<NP>(a, n, out, ck, cp, total, prefix, kBin2Shift, want2, L.sm[2] == want2, L);
}

__global__ __launch_bounds__(kFinThreads) void k_topk_final(TopkArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint32_t dyn[];
  const int r = blockIdx.x;
  const int n = row_valid_count(a, r);
  int32_t* out = a.idx + (long long)r * a.k;
  if (n <= a.k) {
    for (int j = threadIdx.x; j < a.k; j += kFinThreads) out[j] = (j < n) ? j : -1;
  } else {
    const RowWs w = row_ws(a.ws, r, a.k);
    // Wave 0 reads the second histogram before the counts that size the
    // candidate loads, so its digit scan overlaps those loads.
    uint32_t h2[kBins2 / 64];
    if (threadIdx.x < 64) load_hist2(w.hist2, h2);
    const uint32_t bstar = w.meta[1], above = w.meta[2], inbin = w.meta[3];
    const SelLds L = sel_lds(dyn, a.S_max);
    const uint32_t total = above + inbin;
    if (total > (uint32_t)cap_for(a.k)) {
      select_direct(a, r, n, out, L);
    } else {
      if (total <= (uint32_t)(kCPerSmall * kFinThreads))
        final_from_candidates<kCPerSmall>(a, n, out, bstar, above, total, h2, w, L);
      else
        final_from_candidates<kCPer>(a, n, out, bstar, above, total, h2, w, L);
    }
  }
  emit_pool_rows(a, r, out);
}

// One block per row does the whole selection (rows up to kRowMaxS scores,
// k up to kRowMaxK): the 12-bit histogram in LDS over one pass of the row,
// the threshold bin, the candidates (every score in the bins at or above it)
// compacted into LDS over a second pass, then select_row.  No workspace, no
// global atomics, one launch; the row's two passes read scores the indexer
// has just written (L2 / last-level cache).
// Longest row sent here.  Longer rows go to several blocks per row: at
// 131072 scores one block takes 47 us against 33 us for the multi-launch
// path: the per-score work of its two passes runs on one CU instead of
// sixteen (bins that spread the scores evenly were slower still).
constexpr int kRowMaxS = 32768;
constexpr int kRowMaxK = 2048;
constexpr int kRowCap = 2 * kRowMaxK + 4096;  // cap_for(kRowMaxK)
constexpr int kRowRegion = 2 * (kRowMaxS / 32) + (1 << kFinDigit) + ((kFinThreads / 64) << kDigitBits) + 64;
constexpr int kRowUnroll = 8;                 // score loads in flight per thread

// The scores of one pass over a row, kRowUnroll loads per thread in flight:
// f(key, position) for every valid position, in no particular order.  VEC:
// 16-byte loads of four scores (row start 16-byte aligned), so a 1024-thread
// block keeps 128 KB in flight; otherwise 4-byte loads.  Addresses are
// clamped into the row, so no load sits behind a branch.
template <bool VEC, typename F>
__device__ __forceinline__ void row_pass(const float* row, int n, F&& f) {
  const int tid = threadIdx.x;
  if constexpr (VEC) {
    const int last = (n - 1) & ~3;
    for (int e0 = 0; e0 < n; e0 += 4 * kFinThreads * kRowUnroll) {
      v4f v[kRowUnroll];
#pragma unroll
      for (int u = 0; u < kRowUnroll; ++u) {
        const int e = e0 + 4 * (u * kFinThreads + tid);
        v[u] = *reinterpret_cast<const v4f*>(row + (e < n ? e : last));
      }
#pragma unroll
      for (int u = 0; u < kRowUnroll; ++u) {
        const int e = e0 + 4 * (u * kFinThreads + tid);
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if (e + c < n) f(order_key(v[u][c]), e + c);
      }
    }
  } else {
    for (int e0 = 0; e0 < n; e0 += kFinThreads * kRowUnroll) {
      uint32_t key[kRowUnroll];
#pragma unroll
      for (int u = 0; u < kRowUnroll; ++u) {
        const int e = e0 + u * kFinThreads + tid;
        key[u] = order_key(row[e < n ? e : n - 1]);
      }
#pragma unroll
      for (int u = 0; u < kRowUnroll; ++u) {
        const int e = e0 + u * kFinThreads + tid;
        if (e < n) f(key[u], e);
      }
    }
  }
}

template <bool VEC>
__global__ __launch_bounds__(kFinThreads) void k_topk_row(TopkArgs a) {
  __shared__ __attribute__((aligned(16))) uint32_t region[kRowRegion];
  __shared__ __attribute__((aligned(16))) uint32_t hist12[kBins];
  __shared__ uint32_t ckey[kRowCap], cidx[kRowCap];
  __shared__ uint32_t ccount;
  const int r = blockIdx.x;
  const int n = row_valid_count(a, r);
  int32_t* out = a.idx + (long long)r * a.k;
  const int tid = threadIdx.x;
  if (n <= a.k) {
    for (int j = tid; j < a.k; j += kFinThreads) out[j] = (j < n) ? j : -1;
    emit_pool_rows(a, r, out);
    return;
  }
  for (int i = tid; i < kBins; i += kFinThreads) hist12[i] = 0u;
  if (tid == 0) ccount = 0u;
  __syncthreads();
  const float* row = a.scores + (long long)r * a.ld;
  // pass 1: histogram
  row_pass<VEC>(row, n, [&](uint32_t key, int) { atomicAdd(&hist12[key >> kBinShift], 1u); });
  __syncthreads();
  uint32_t hb[kBins / kFinThreads];
  load_bins<kFinThreads>(hist12, hb);
  uint32_t bstar, above, inbin;
  threshold_from_bins<kFinThreads>(hb, (uint32_t)a.k, sel_lds(region, a.S_max).sm, &bstar, &above, &inbin);
  if (above + inbin <= (uint32_t)kRowCap) {
    // pass 2: candidates (exactly above + hist12[bstar] of them)
    row_pass<VEC>(row, n, [&](uint32_t key, int e) {
      if ((key >> kBinShift) >= bstar) {
        const uint32_t slot = atomicAdd(&ccount, 1u);
        ckey[slot] = key;
        cidx[slot] = (uint32_t)e;
      }
    });
  }
  __syncthreads();
  select_row(a, r, n, out, bstar, above, inbin, ckey, cidx, region);
  emit_pool_rows(a, r, out);
}

size_t final_lds_bytes(int S_max, int k) {
  (void)k;
  return (2 * (size_t)((((S_max + 31) >> 5) + 3) & ~3) + ((size_t)1 << kFinDigit) +
          ((size_t)(kFinThreads / 64) << kDigitBits) + 64) * 4;
}

}  // namespace

bool topk_row_fused(int S_max, int k) { return S_max <= kRowMaxS && k <= kRowMaxK; }


// Rows whose valid set fits in k keep every valid position: idx = 0 .. pos,
// then -1.  Used when S_max <= k, where no score decides anything.
__global__ __launch_bounds__(256) void k_select_all(TopkArgs a) {
  const long long n = (long long)a.row_count * a.k;
  for (long long e = (long long)blockIdx.x * 256 + threadIdx.x; e < n; e += (long long)gridDim.x * 256) {
    const int r = (int)(e / a.k), j = (int)(e - (long long)r * a.k);
    a.idx[e] = j < row_valid_count(a, r) ? j : -1;
  }
}

hipError_t launch_select_all(const TopkArgs& a, hipStream_t stream) {
  const long long n = (long long)a.row_count * a.k;
  if (n <= 0) return hipSuccess;
  const long long blocks = (n + 255) / 256;
  hipLaunchKernelGGL(k_select_all, dim3((unsigned)(blocks < 8192 ? blocks : 8192)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

size_t topk_workspace_bytes(int row_count, int S_max, int k) {
  (void)S_max;
  if (row_count <= 0 || k <= 0) return 0;
  return (size_t)row_count * row_stride_bytes(k);
}

bool topk_supported(int S_max, int k) {
  return k >= 1 && k <= kMaxK && S_max >= 1 && S_max <= kMaxS && final_lds_bytes(S_max, k) <= 160 * 1024;
}

void topk_zero_region(void* ws, int rows, int k, uint32_t** base, long long* stride_words, int* words) {
  *base = static_cast<uint32_t*>(ws);
  *stride_words = (long long)(row_stride_bytes(k) / 4);
  *words = rows > 0 ? kZeroWords : 0;  // hist, meta and hist2 are contiguous
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t stream) {
  if (a.row_count <= 0) return hipSuccess;
  if (topk_row_fused(a.S_max, a.k)) {
    const bool vec = (a.ld % 4) == 0 && (reinterpret_cast<uintptr_t>(a.scores) & 15) == 0;
    if (vec)
      hipLaunchKernelGGL(k_topk_row<true>, dim3((unsigned)a.row_count), dim3(kFinThreads), 0, stream, a);
    else
      hipLaunchKernelGGL(k_topk_row<false>, dim3((unsigned)a.row_count), dim3(kFinThreads), 0, stream, a);
    return hipGetLastError();
  }
  const dim3 segs((unsigned)((a.S_max + kSeg - 1) / kSeg), (unsigned)a.row_count);
  if (!a.ws_zeroed) hipLaunchKernelGGL(k_topk_zero, dim3(256), dim3(256), 0, stream, a);
  hipLaunchKernelGGL(k_topk_hist, segs, dim3(kSegThreads), 0, stream, a);
  hipLaunchKernelGGL(k_topk_gather, segs, dim3(kSegThreads), 0, stream, a);
  const size_t lds = final_lds_bytes(a.S_max, a.k);
  hipLaunchKernelGGL(k_topk_final, dim3((unsigned)a.row_count), dim3(kFinThreads), lds, stream, a);
  return hipGetLastError();
}

}  // namespace dsa
