// Internal declarations shared by the HIP translation units of libdsa.
// Not part of the public ABI (include/dsa.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dsa.h"

namespace dsa {

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

// ReLU as one integer max on the bit pattern: a float with its sign bit set
// is a negative int32, so max(bits, 0) keeps every x >= +0 and maps every
// negative x (and -0) to +0.  fmaxf(x, 0.f) would also cost a canonicalising
// max per value in IEEE mode.  Differs from fmaxf only on NaN input (kept).
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef short v4s __attribute__((ext_vector_type(4)));

constexpr int kHI = DSA_INDEX_HEADS;   // indexer heads
constexpr int kDI = DSA_INDEX_DIM;     // indexer head dim
constexpr int kDQK = DSA_LATENT_DIM;   // latent entry width
constexpr int kDV = DSA_VALUE_DIM;     // value width

// ---------------------------------------------------------------- helpers

// Monotone map fp32 -> uint32: a < b (as floats, no NaN) <=> key(a) < key(b).
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Paged cache addressing: token s of sequence b lives in row s % P of page
// table[b * max_pages + s / P] of a pool of num_pages pages (P = 1 << shift
// tokens each).  Page ids are clamped into the pool, so a bad table entry
// reads or writes a wrong page of the pool, never memory outside it.  A null
// table means contiguous caches [B, S_max, ...].
struct PageMap {
  const int32_t* table;
  int max_pages, shift, last_page;  // last_page = num_pages - 1
  __device__ __forceinline__ int page(int b, int j) const {
    const int p = table[(long long)b * max_pages + j];
    return p < 0 ? 0 : (p > last_page ? last_page : p);
  }
  // pool row of token s of sequence b
  __device__ __forceinline__ int row(int b, int s) const {
    return (page(b, s >> shift) << shift) | (s & ((1 << shift) - 1));
  }
};

// Pool row of position s for a query of sequence b at position pos; -1 when
// the query may not select s (negative, or past pos).
__device__ __forceinline__ int32_t page_row(int32_t s, int pos, int b, const PageMap& pm) {
  return (s >= 0 && s <= pos) ? pm.row(b, s) : -1;
}

// Length of sequence b clamped into [0, S_max].
__device__ __forceinline__ int clamped_len(const int32_t* seq_lens, int b, int S_max) {
  int L = seq_lens[b];
  return L < 0 ? 0 : (L > S_max ? S_max : L);
}

// Position of query row t (may be negative: the row then sees no key).
__device__ __forceinline__ int row_pos(const int32_t* seq_lens, int t, int q_len, int S_max) {
  int b = t / q_len;
  return clamped_len(seq_lens, b, S_max) - q_len + (t - b * q_len);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(((uint32_t)h) << 16);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Sum of v over the lanes l and l^16 / l^32 using the gfx950 row-swap ops.
__device__ __forceinline__ float sum_xor16(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_xor16(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Head weights of the indexer output rows a lane holds: heads 16m + 4g + i
// (m, i = 0..3) of query row t, times the optional q-scale.  All loads are
// issued before any is used (no per-element branches).
__device__ __forceinline__ void load_head_weights(const void* w, int w_is_bf16, const float* q_scale, size_t t,
                                                  int g, float (&wv)[4][4]) {
  if (w_is_bf16) {
    const uint32_t* w32 = static_cast<const uint32_t*>(w) + (t * 64 + 4 * g) / 2;
    uint32_t raw[4][2];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      raw[m][0] = w32[8 * m];
      raw[m][1] = w32[8 * m + 1];
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      wv[m][0] = __uint_as_float(raw[m][0] << 16);
      wv[m][1] = __uint_as_float(raw[m][0] & 0xFFFF0000u);
      wv[m][2] = __uint_as_float(raw[m][1] << 16);
      wv[m][3] = __uint_as_float(raw[m][1] & 0xFFFF0000u);
    }
  } else {
    const float* wf = static_cast<const float*>(w) + t * 64 + 4 * g;
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) wv[m][i] = wf[16 * m + i];
  }
  if (q_scale) {
    const float* qs = q_scale + t * 64 + 4 * g;
    float sc[4][4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[m][i] = qs[16 * m + i];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) wv[m][i] *= sc[m][i];
  }
}

// ---------------------------------------------------------- async memory

typedef __attribute__((address_space(3))) void lds_void_t;

// One global -> LDS copy of 16 bytes per active lane (global_load_lds_dwordx4,
// address = uniform base + per-lane 32-bit offset): lane l's bytes land at
// lds_base + 16*l.  Issued from asm so the compiler does not make later LDS
// reads or its own memory waits depend on it (it cannot tell buffers apart
// and would drain every copy in flight); completion is tracked by the
// caller's explicit vmcnt waits and barriers.  gbase and lds_base must be
// the same for every lane of the wave.  No register result.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // m0 is reserved, but nothing else in these kernels uses it
__device__ __forceinline__ void dma16_lds(const void* gbase, uint32_t voff, const void* lds_base) {
  const uint32_t m = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const lds_void_t*)lds_base);  // uniform
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(gbase), "s"(m)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// As dma16_lds, but from a per-lane 64-bit address, into the LDS byte offset
// lds_off (the same for every lane of the wave).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16_lds_at(const void* gaddr, uint32_t lds_off) {
  const uint32_t m = __builtin_amdgcn_readfirstlane(lds_off);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gaddr), "s"(m)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// As dma16_lds, with the LDS destination given as a byte offset (the same
// for every lane of the wave).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16_lds_off(const void* gbase, uint32_t voff, uint32_t lds_off) {
  const uint32_t m = __builtin_amdgcn_readfirstlane(lds_off);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(gbase), "s"(m)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// LDS byte offset of a __shared__ object (its address in the LDS aperture).
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return (uint32_t)(uintptr_t)(const lds_void_t*)p;
}

// One global -> LDS copy of 4 bytes per active lane (lane l's word lands at
// lds_base + 4*l); otherwise as dma16_lds.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma4_lds(const void* gbase, uint32_t voff, const void* lds_base) {
  const uint32_t m = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const lds_void_t*)lds_base);  // uniform
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(gbase), "s"(m)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// A 4-byte global store issued from asm: the compiler keeps no wait for it
// (its data register is read at issue).  Visibility to later reads needs a
// vmcnt wait (a workgroup fence gives one).
__device__ __forceinline__ void store_u32_nowait(uint32_t* p, uint32_t v) {
  asm volatile("global_store_dword %0, %1, off" ::"v"(p), "v"(v) : "memory");
}

// ------------------------------------------------------------ launch args

struct IndexerArgs {
  int B, q_len, S_max;
  const int32_t* seq_lens;
  const void* q;          // [T,64,128] fp8 codes or f32
  const float* q_scale;   // [T,64] or null
  const void* w;          // [T,64] bf16 or f32
  int w_is_bf16;
  const void* k;          // [B,S_max,128] fp8 codes or f32
  const float* k_scale;   // [B,S_max] or null
  int row_begin, row_count;
  float* scores;          // [row_count, ld]
  long long ld;
  // Optional side job: zero zero_words words at zero_base + r * zero_stride
  // for r < zero_rows (the top-k counters of the same rows), so the top-k
  // that follows needs no clearing launch of its own.
  uint32_t* zero_base;
  long long zero_stride;
  int zero_words, zero_rows;
  PageMap pages;          // k / k_scale are page pools when pages.table is set
};

hipError_t launch_indexer_fp8(const IndexerArgs& a, hipStream_t s);
hipError_t launch_indexer_f32(const IndexerArgs& a, hipStream_t s);

struct TopkArgs {
  int B, q_len, S_max;
  const int32_t* seq_lens;
  const float* scores;    // [row_count, ld]
  long long ld;
  int row_begin, row_count, k;
  int32_t* idx;           // [row_count, k]
  void* ws;
  int ws_zeroed;          // the counters in ws are already zero (cleared by the indexer launch)
  int32_t* rows;          // optional [row_count, k]: the selection as pool rows of `pages` (-1 where idx is)
  PageMap pages;
};

// Per-block fp8 quantisation (launch_quantize: rows -> codes/scales;
// launch_cache_append: row b*q_len+i -> cache position
// clamp(seq_lens[b]) - q_len + i).
struct QuantArgs {
  const void* x;            // [rows, 128] bf16 or fp32
  long long rows;
  uint8_t* codes;           // [rows, 128], or the key cache [B, S_max, 128]
  float* scales;            // [rows], or the scale cache [B, S_max]
  const int32_t* seq_lens;  // cache append only
  int q_len, S_max;         // cache append only
  PageMap pages;            // cache append into page pools when pages.table is set
};
hipError_t launch_quantize(const QuantArgs& a, bool bf16, hipStream_t s);
hipError_t launch_cache_append(const QuantArgs& a, bool bf16, hipStream_t s);

size_t topk_workspace_bytes(int row_count, int S_max, int k);
// The words of a top-k workspace that must be zero before launch_topk.
void topk_zero_region(void* ws, int rows, int k, uint32_t** base, long long* stride_words, int* words);
hipError_t launch_topk(const TopkArgs& a, hipStream_t s);
// launch_topk selects each row in one block (no workspace use) for these sizes.
bool topk_row_fused(int S_max, int k);
// Every valid position (0 .. pos, then -1) for rows whose valid set fits in k.
hipError_t launch_select_all(const TopkArgs& a, hipStream_t s);

struct MlaArgs {
  int B, q_len, S_max, H, k;
  const int32_t* seq_lens;
  float sm_scale;
  const void* q;          // [T,H,576]
  const void* kv;         // [B,S_max,576]
  const int32_t* idx;     // [T,k]
  void* out;              // [T,H,512]
  float* lse;             // [T,H] or null
  void* ws;
  int row_begin, row_count;  // rows handled by this launch
  // idx holds rows of a flat pool (kv [rows, 576]) rather than positions of
  // sequence b: an entry is valid iff it is >= 0 (the causal bound was applied
  // when the positions were translated).
  int flat;
  // idx rows are the forward's own selection: ascending, every valid entry
  // before every -1, exactly min(k, pos + 1) of them, so a row's work can stop
  // there (a caller's idx may hold -1 anywhere and is read to the end).
  int sel_prefix;
};

// Positions idx[t, m] -> pool rows of the paged cache (-1 where the position
// is invalid for row t: negative or past its query position).
hipError_t launch_page_rows(const int32_t* idx, int32_t* rows, int T, int k, int q_len, int S_max,
                            const int32_t* seq_lens, const PageMap& pages, hipStream_t s);

size_t mla_workspace_bytes(int T, int H, int k, int is_bf16);
hipError_t launch_mla_bf16(const MlaArgs& a, hipStream_t s);
hipError_t launch_mla_f32(const MlaArgs& a, hipStream_t s);

// MHA-mode prefill (sequences within top-k): decompression of the latent
// rows through wkv_b into the workspace, then causal attention.
struct MhaArgs {
  int B, q_len, S_max, H;
  const int32_t* seq_lens;
  float sm_scale;
  const void* q;          // [T,H,192] bf16: q_nope | q_pe
  const void* kv;         // [B,S_max,576] bf16: latent | k_pe
  const void* wkv_b;      // [H,256,512] bf16: k_nope rows | v rows
  void* out;              // [T,H,128] bf16
  float* lse;             // [T,H] or null
  void* knope_ws;         // [B,H,S_max,128] bf16
  void* v_ws;             // [B,H,S_max,128] bf16
};
size_t mha_workspace_bytes(int B, int S_max, int H);
hipError_t launch_mha_prefill(const MhaArgs& a, hipStream_t s);

// Indexer KL objective (forward): per-row KL of the head-summed, normalised
// attention weights against Softmax(I) over a set of positions.
struct KlArgs {
  int B, q_len, S_max, H, k;  // k: entries per row (idx width, or S_max for every position)
  const int32_t* seq_lens;
  float sm_scale;
  const void* q;          // [T,H,576] bf16
  const void* kv;         // [B,S_max,576] bf16
  const float* lse;       // [T,H] natural log
  const float* scores;    // [T, ld] indexer scores I
  long long ld;
  const int32_t* idx;     // [T,k] or null (the set is 0 .. pos)
  float* kl;              // [row_count]
  float* loss;            // scalar or null
  float* ws;              // per-split partials
  int row_begin, row_count;
};
size_t kl_workspace_bytes(int rows, int k);
hipError_t launch_indexer_kl(const KlArgs& a, hipStream_t s);

}  // namespace dsa
