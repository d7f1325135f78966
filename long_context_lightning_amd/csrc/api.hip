// Host side of the C ABI declared in include/dsa.h: argument validation,
// workspace carving and the order of launches.  No allocation, no
// synchronisation, no exceptions across the boundary.
#include <atomic>
#include <mutex>

#include "dsa_internal.h"

namespace dsa {
bool topk_supported(int S_max, int k);
bool mla_f32_supported(int k);
bool prefill_supported(int q_len, int S_max, int k);
size_t prefill_workspace_bytes(int B, int q_len, int S_max, int k);
hipError_t launch_indexer_topk_prefill(const IndexerArgs& ia, int k, int32_t* idx, void* ws, hipStream_t s);
}  // namespace dsa

using namespace dsa;

namespace {

constexpr size_t kAlign = 256;
constexpr int kMaxRowsPerLaunch = 32768;
constexpr size_t kScoreChunkBytes = (size_t)256 << 20;
constexpr int kMaxMlaK = 16384;

inline size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }
inline bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }
inline dsa_status hip_status(hipError_t e) { return e == hipSuccess ? DSA_OK : DSA_ERR_HIP; }

bool geom_ok(const dsa_geom* g) {
  if (!g || g->B < 1 || g->q_len < 1 || g->S_max < 1 || !g->seq_lens) return false;
  if ((long long)g->B * g->q_len > 0x7FFFFFFFLL) return false;
  return g->q_len <= g->S_max;
}

long long rows_of(const dsa_geom* g) { return (long long)g->B * g->q_len; }

bool rows_ok(const dsa_geom* g, int32_t row_begin, int32_t row_count) {
  return row_begin >= 0 && row_count >= 0 && (long long)row_begin + row_count <= rows_of(g);
}

dsa_status check_indexer_inputs(const dsa_geom* g, const void* q, dsa_dtype q_dt, const float* q_scale,
                                const void* w, dsa_dtype w_dt, const void* k, dsa_dtype k_dt,
                                const float* k_scale) {
  if (!geom_ok(g) || !q || !w || !k) return DSA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(w, 4)) return DSA_ERR_INVALID_ARG;
  if ((q_scale && !aligned(q_scale, 4)) || (k_scale && !aligned(k_scale, 4))) return DSA_ERR_INVALID_ARG;
  if (q_dt != k_dt) return DSA_ERR_UNSUPPORTED;
  if (q_dt == DSA_FP8_E4M3FN) return (w_dt == DSA_BF16 || w_dt == DSA_F32) ? DSA_OK : DSA_ERR_UNSUPPORTED;
  if (q_dt == DSA_F32) return w_dt == DSA_F32 ? DSA_OK : DSA_ERR_UNSUPPORTED;
  return DSA_ERR_UNSUPPORTED;
}

IndexerArgs make_indexer_args(const dsa_geom* g, const void* q, const float* q_scale, const void* w,
                              dsa_dtype w_dt, const void* k, const float* k_scale) {
  IndexerArgs a;
  a.B = g->B;
  a.q_len = g->q_len;
  a.S_max = g->S_max;
  a.seq_lens = g->seq_lens;
  a.q = q;
  a.q_scale = q_scale;
  a.w = w;
  a.w_is_bf16 = (w_dt == DSA_BF16);
  a.k = k;
  a.k_scale = k_scale;
  a.row_begin = 0;
  a.row_count = 0;
  a.scores = nullptr;
  a.ld = 0;
  a.zero_base = nullptr;
  a.zero_stride = 0;
  a.zero_words = 0;
  a.zero_rows = 0;
  a.pages = PageMap{};
  return a;
}

// The score kernels launch at most kMaxRowsPerLaunch rows at a time.
hipError_t run_indexer(const IndexerArgs& a, bool fp8, hipStream_t stream) {
  const int end = a.row_begin + a.row_count;
  for (int r0 = a.row_begin; r0 < end; r0 += kMaxRowsPerLaunch) {
    IndexerArgs c = a;
    c.row_begin = r0;
    c.row_count = (end - r0 < kMaxRowsPerLaunch) ? end - r0 : kMaxRowsPerLaunch;
    c.scores = a.scores + (long long)(r0 - a.row_begin) * a.ld;
    const hipError_t e = fp8 ? launch_indexer_fp8(c, stream) : launch_indexer_f32(c, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Top-k over kMaxRowsPerLaunch-row chunks; each chunk reuses the same workspace.
hipError_t run_topk(const TopkArgs& a, hipStream_t stream) {
  const int end = a.row_begin + a.row_count;
  for (int r0 = a.row_begin; r0 < end; r0 += kMaxRowsPerLaunch) {
    TopkArgs c = a;
    c.row_begin = r0;
    c.row_count = (end - r0 < kMaxRowsPerLaunch) ? end - r0 : kMaxRowsPerLaunch;
    c.scores = a.scores + (long long)(r0 - a.row_begin) * a.ld;
    c.idx = a.idx + (long long)(r0 - a.row_begin) * a.k;
    if (a.rows) c.rows = a.rows + (long long)(r0 - a.row_begin) * a.k;
    c.ws_zeroed = r0 == a.row_begin ? a.ws_zeroed : 0;  // later chunks reuse the workspace
    const hipError_t e = launch_topk(c, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t run_mla(const MlaArgs& a, bool bf16, hipStream_t stream) {
  if (bf16) return launch_mla_bf16(a, stream);
  const int end = a.row_begin + a.row_count;
  for (int r0 = a.row_begin; r0 < end; r0 += kMaxRowsPerLaunch) {
    MlaArgs c = a;
    c.row_begin = r0;
    c.row_count = (end - r0 < kMaxRowsPerLaunch) ? end - r0 : kMaxRowsPerLaunch;
    const hipError_t e = launch_mla_f32(c, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

dsa_status check_mla(const dsa_geom* g, int32_t H, int32_t k, const void* q, dsa_dtype dt, const void* kv,
                     const int32_t* idx, const void* out, const float* lse) {
  if (!geom_ok(g) || !q || !kv || !idx || !out) return DSA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(kv, 16) || !aligned(out, 16) || !aligned(idx, 4)) return DSA_ERR_INVALID_ARG;
  if (lse && !aligned(lse, 4)) return DSA_ERR_INVALID_ARG;
  if (k < 1 || k > kMaxMlaK || H < 1 || H > 128) return DSA_ERR_INVALID_ARG;
  if (dt == DSA_BF16) return (H % 16 == 0) ? DSA_OK : DSA_ERR_UNSUPPORTED;
  if (dt == DSA_F32) return mla_f32_supported(k) ? DSA_OK : DSA_ERR_UNSUPPORTED;
  return DSA_ERR_UNSUPPORTED;
}

// A page table is usable with geometry g: power-of-two pages of 64..65536
// tokens, a table wide enough for S_max tokens, pool rows addressable by int32.
bool pages_ok(const dsa_geom* g, const dsa_pages* p) {
  if (!p || !p->block_table || !aligned(p->block_table, 4)) return false;
  if (p->max_pages < 1 || p->num_pages < 1) return false;
  if (p->page_size < 64 || p->page_size > 65536 || (p->page_size & (p->page_size - 1))) return false;
  if ((long long)p->max_pages * p->page_size < g->S_max) return false;
  if ((long long)g->B * p->max_pages > 0x7FFFFFFFLL) return false;
  return p->num_pages <= 0x7FFFFFFFLL / p->page_size;
}

PageMap page_map(const dsa_pages* p) {
  PageMap m{};
  if (!p) return m;
  m.table = p->block_table;
  m.max_pages = p->max_pages;
  m.shift = __builtin_ctz((unsigned)p->page_size);
  m.last_page = (int)(p->num_pages - 1);
  return m;
}

MlaArgs make_mla_args(const dsa_geom* g, int32_t H, int32_t k, float sm_scale, const void* q, const void* kv,
                      const int32_t* idx, void* out, float* lse, void* ws) {
  MlaArgs a;
  a.B = g->B;
  a.q_len = g->q_len;
  a.S_max = g->S_max;
  a.H = H;
  a.k = k;
  a.seq_lens = g->seq_lens;
  a.sm_scale = sm_scale;
  a.q = q;
  a.kv = kv;
  a.idx = idx;
  a.out = out;
  a.lse = lse;
  a.ws = ws;
  a.row_begin = 0;
  a.row_count = (int)rows_of(g);
  a.flat = 0;
  a.sel_prefix = 0;
  return a;
}

// Workspace plan of dsa_forward.  Paged caches add a buffer for the
// translated pool rows of the selection.
struct ForwardPlan {
  bool streaming;
  int chunk_rows;
  size_t scores_off, topk_off, mla_off, rows_off, total;
};

ForwardPlan plan_forward(int B, int q_len, int S_max, int H, int topk, dsa_dtype index_dt, dsa_dtype mla_dt,
                         bool paged) {
  ForwardPlan p{};
  const long long T = (long long)B * q_len;
  p.streaming = index_dt == DSA_FP8_E4M3FN && q_len >= 64 && prefill_supported(q_len, S_max, topk);
  size_t off = 0;
  if (p.streaming) {
    p.chunk_rows = 0;
    p.scores_off = p.topk_off = 0;
    off = align_up(prefill_workspace_bytes(B, q_len, S_max, topk));
  } else {
    long long rows = (long long)(kScoreChunkBytes / ((size_t)S_max * 4));
    if (rows < 1) rows = 1;
    if (rows > T) rows = T;
    if (rows > kMaxRowsPerLaunch) rows = kMaxRowsPerLaunch;
    p.chunk_rows = (int)rows;
    p.scores_off = 0;
    off = align_up((size_t)rows * S_max * 4);
    p.topk_off = off;
    off += align_up(topk_workspace_bytes((int)rows, S_max, topk));
  }
  p.mla_off = off;
  off += align_up(mla_workspace_bytes((int)T, H, topk, mla_dt == DSA_BF16));
  p.rows_off = off;
  if (paged) off += align_up((size_t)T * topk * sizeof(int32_t));
  p.total = off;
  return p;
}

size_t mla_paged_workspace_bytes(int T, int H, int k, dsa_dtype dt) {
  return align_up(mla_workspace_bytes(T, H, k, dt == DSA_BF16)) + align_up((size_t)T * k * sizeof(int32_t));
}

// ---- shared bodies of the contiguous and the paged entry points (pages null = contiguous)

dsa_status indexer_scores_impl(const dsa_geom* geom, const dsa_pages* pages, const void* q, dsa_dtype q_dtype,
                               const float* q_scale, const void* w, dsa_dtype w_dtype, const void* k,
                               dsa_dtype k_dtype, const float* k_scale, int32_t row_begin, int32_t row_count,
                               float* scores, int64_t ld, hipStream_t stream) {
  const dsa_status st = check_indexer_inputs(geom, q, q_dtype, q_scale, w, w_dtype, k, k_dtype, k_scale);
  if (st != DSA_OK) return st;
  if (pages && !pages_ok(geom, pages)) return DSA_ERR_INVALID_ARG;
  if (!rows_ok(geom, row_begin, row_count) || ld < geom->S_max) return DSA_ERR_INVALID_ARG;
  if (row_count == 0) return DSA_OK;
  if (!scores || !aligned(scores, 4)) return DSA_ERR_INVALID_ARG;
  IndexerArgs a = make_indexer_args(geom, q, q_scale, w, w_dtype, k, k_scale);
  a.pages = page_map(pages);
  a.row_begin = row_begin;
  a.row_count = row_count;
  a.scores = scores;
  a.ld = ld;
  return hip_status(run_indexer(a, q_dtype == DSA_FP8_E4M3FN, stream));
}

// The attention over translated pool rows (paged) or positions (contiguous).
// rows_ready: the top-k launch has already written the pool rows.
// sel_prefix: idx is the forward's own selection (valid entries first).
hipError_t mla_launches(const dsa_geom* geom, const dsa_pages* pages, int32_t H, int32_t k, float sm_scale,
                        const void* q, dsa_dtype dtype, const void* kv, const int32_t* idx, void* out, float* lse,
                        void* mla_ws, int32_t* rows, hipStream_t stream, bool rows_ready = false,
                        bool sel_prefix = false) {
  MlaArgs a = make_mla_args(geom, H, k, sm_scale, q, kv, idx, out, lse, mla_ws);
  a.sel_prefix = sel_prefix ? 1 : 0;
  if (pages) {
    const hipError_t e = rows_ready ? hipSuccess
                                    : launch_page_rows(idx, rows, (int)rows_of(geom), k, geom->q_len, geom->S_max,
                                                       geom->seq_lens, page_map(pages), stream);
    if (e != hipSuccess) return e;
    a.idx = rows;
    a.flat = 1;
  }
  return run_mla(a, dtype == DSA_BF16, stream);
}

dsa_status sparse_mla_impl(const dsa_geom* geom, const dsa_pages* pages, int32_t H, int32_t k, float sm_scale,
                           const void* q, dsa_dtype dtype, const void* kv, const int32_t* idx, void* out,
                           float* lse, void* ws, size_t ws_bytes, hipStream_t stream) {
  const dsa_status st = check_mla(geom, H, k, q, dtype, kv, idx, out, lse);
  if (st != DSA_OK) return st;
  if (pages && !pages_ok(geom, pages)) return DSA_ERR_INVALID_ARG;
  const int T = (int)rows_of(geom);
  const size_t mla_bytes = mla_workspace_bytes(T, H, k, dtype == DSA_BF16);
  const size_t need = pages ? mla_paged_workspace_bytes(T, H, k, dtype) : mla_bytes;
  if (ws_bytes < need || (need && (!ws || !aligned(ws, kAlign)))) return DSA_ERR_WORKSPACE;
  int32_t* rows = pages ? reinterpret_cast<int32_t*>(static_cast<char*>(ws) + align_up(mla_bytes)) : nullptr;
  return hip_status(mla_launches(geom, pages, H, k, sm_scale, q, dtype, kv, idx, out, lse, ws, rows, stream));
}

// The selection of dsa_forward (stages a1 and a2) into idx_out: the keep-all
// rows when S_max <= topk, the streamed indexer + top-k of long fp8
// prefills, else the indexer's score rows chunk by chunk into the workspace
// and the top-k over them.  With pages, the top-k of the chunked path also
// writes the selection as pool rows into rows (when rows is not null).
// The workspace layout is plan p's, below p.mla_off.
hipError_t select_impl(const dsa_geom* geom, const dsa_pages* pages, int32_t topk, const void* index_q,
                       dsa_dtype index_dtype, const float* index_q_scale, const void* index_w,
                       dsa_dtype index_w_dtype, const void* index_k, const float* index_k_scale, int32_t* idx_out,
                       char* wsb, const ForwardPlan& p, int32_t* rows, hipStream_t stream) {
  const int T = (int)rows_of(geom);
  if (geom->S_max <= topk) {
    // "详解DSA", DSA计算流: a sequence no longer than top-k keeps every
    // position, so the indexer's work is skipped; the selection is 0 .. pos.
    TopkArgs ta{};
    ta.B = geom->B;
    ta.q_len = geom->q_len;
    ta.S_max = geom->S_max;
    ta.seq_lens = geom->seq_lens;
    ta.row_begin = 0;
    ta.row_count = T;
    ta.k = topk;
    ta.idx = idx_out;
    return launch_select_all(ta, stream);
  }
  IndexerArgs ia = make_indexer_args(geom, index_q, index_q_scale, index_w, index_w_dtype, index_k, index_k_scale);
  ia.pages = page_map(pages);
  if (p.streaming) {
    ia.row_begin = 0;
    ia.row_count = T;
    return launch_indexer_topk_prefill(ia, topk, idx_out, wsb, stream);
  }
  hipError_t e = hipSuccess;
  float* scores = reinterpret_cast<float*>(wsb + p.scores_off);
  const bool fp8 = index_dtype == DSA_FP8_E4M3FN;
  for (int r0 = 0; r0 < T && e == hipSuccess; r0 += p.chunk_rows) {
    const int rc = (T - r0 < p.chunk_rows) ? T - r0 : p.chunk_rows;
    TopkArgs ta{};
    ta.B = geom->B;
    ta.q_len = geom->q_len;
    ta.S_max = geom->S_max;
    ta.seq_lens = geom->seq_lens;
    ta.scores = scores;
    ta.ld = geom->S_max;
    ta.row_begin = r0;
    ta.row_count = rc;
    ta.k = topk;
    ta.idx = idx_out + (long long)r0 * topk;
    ta.ws = wsb + p.topk_off;
    ta.ws_zeroed = 1;  // the indexer launch below clears the top-k counters
    if (pages && rows) {  // the top-k also writes the selection as pool rows
      ta.rows = rows + (long long)r0 * topk;
      ta.pages = page_map(pages);
    }
    ia.row_begin = r0;
    ia.row_count = rc;
    ia.scores = scores;
    ia.ld = geom->S_max;
    if (!topk_row_fused(geom->S_max, topk)) {  // the multi-launch top-k counts into cleared counters
      topk_zero_region(ta.ws, rc, topk, &ia.zero_base, &ia.zero_stride, &ia.zero_words);
      ia.zero_rows = rc;
    }
    e = run_indexer(ia, fp8, stream);
    if (e != hipSuccess) break;
    e = run_topk(ta, stream);
  }
  return e;
}

dsa_status forward_impl(const dsa_geom* geom, const dsa_pages* pages, int32_t H, int32_t topk, float sm_scale,
                        const void* index_q, dsa_dtype index_dtype, const float* index_q_scale,
                        const void* index_w, dsa_dtype index_w_dtype, const void* index_k,
                        const float* index_k_scale, const void* mla_q, const void* mla_kv, dsa_dtype mla_dtype,
                        int32_t* idx_out, void* out, float* lse, void* ws, size_t ws_bytes, hipStream_t stream) {
  dsa_status st = check_indexer_inputs(geom, index_q, index_dtype, index_q_scale, index_w, index_w_dtype, index_k,
                                       index_dtype, index_k_scale);
  if (st != DSA_OK) return st;
  if ((idx_out && !aligned(idx_out, 4)) || topk < 1) return DSA_ERR_INVALID_ARG;
  // any non-null placeholder for the MLA check; the real selection buffer is
  // idx_out or the workspace tail
  st = check_mla(geom, H, topk, mla_q, mla_dtype, mla_kv, idx_out ? idx_out : static_cast<int32_t*>(ws), out, lse);
  if (st != DSA_OK) return st;
  if (pages && !pages_ok(geom, pages)) return DSA_ERR_INVALID_ARG;
  const ForwardPlan p =
      plan_forward(geom->B, geom->q_len, geom->S_max, H, topk, index_dtype, mla_dtype, pages != nullptr);
  const bool keep_all = geom->S_max <= topk;  // no row can have more than topk valid positions
  if (!keep_all && !p.streaming && !topk_supported(geom->S_max, topk)) return DSA_ERR_UNSUPPORTED;
  const int T = (int)rows_of(geom);
  const size_t need = p.total + (idx_out ? 0 : align_up((size_t)T * topk * sizeof(int32_t)));
  if (ws_bytes < need || !ws || !aligned(ws, kAlign)) return DSA_ERR_WORKSPACE;
  char* wsb = static_cast<char*>(ws);
  if (!idx_out) idx_out = reinterpret_cast<int32_t*>(wsb + p.total);  // selection kept in the workspace
  int32_t* rows = reinterpret_cast<int32_t*>(wsb + p.rows_off);
  const hipError_t e = select_impl(geom, pages, topk, index_q, index_dtype, index_q_scale, index_w, index_w_dtype,
                                   index_k, index_k_scale, idx_out, wsb, p, rows, stream);
  if (e != hipSuccess) return DSA_ERR_HIP;
  // the chunked path's top-k already wrote the pool rows of a paged selection
  const bool rows_ready = !keep_all && !p.streaming;
  return hip_status(mla_launches(geom, pages, H, topk, sm_scale, mla_q, mla_dtype, mla_kv, idx_out, out, lse,
                                 wsb + p.mla_off, rows, stream, rows_ready, /*sel_prefix=*/true));
}

dsa_status cache_append_impl(const dsa_geom* geom, const dsa_pages* pages, const void* k_new, dsa_dtype k_dtype,
                             uint8_t* k_cache, float* k_scale_cache, hipStream_t stream) {
  if (!geom_ok(geom) || !k_new || !k_cache || !k_scale_cache) return DSA_ERR_INVALID_ARG;
  if (!aligned(k_new, 16) || !aligned(k_cache, 4) || !aligned(k_scale_cache, 4)) return DSA_ERR_INVALID_ARG;
  if (pages && !pages_ok(geom, pages)) return DSA_ERR_INVALID_ARG;
  if (k_dtype != DSA_BF16 && k_dtype != DSA_F32) return DSA_ERR_UNSUPPORTED;
  QuantArgs a{};
  a.x = k_new;
  a.rows = rows_of(geom);
  a.codes = k_cache;
  a.scales = k_scale_cache;
  a.seq_lens = geom->seq_lens;
  a.q_len = geom->q_len;
  a.S_max = geom->S_max;
  a.pages = page_map(pages);
  return hip_status(launch_cache_append(a, k_dtype == DSA_BF16, stream));
}

// ---- scratch memory of dsa_forward_noalloc
//
// A static device array: every GPU the library runs on holds its own copy
// from module load to process exit.  In host code `scratch` only names the
// symbol; its device address is looked up once per device with
// hipGetSymbolAddress (with that device current) and only that address is
// handed to kernels.
static __device__ __align__(256) unsigned char scratch[DSA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxScratchDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxScratchDevices];
std::mutex g_scratch_mu;

// Device address of device dev's copy of `scratch`.
hipError_t scratch_address(int dev, void** addr) {
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_addr[dev].load(std::memory_order_relaxed);
    if (!p) {
      int cur = 0;
      hipError_t e = hipGetDevice(&cur);
      if (e != hipSuccess) return e;
      if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (cur != dev) {
        const hipError_t back = hipSetDevice(cur);
        if (e == hipSuccess) e = back;
      }
      if (e != hipSuccess) return e;
      if (!p || ((uintptr_t)p & (kAlign - 1))) return hipErrorInvalidSymbol;
      g_scratch_addr[dev].store(p, std::memory_order_release);
    }
  }
  *addr = p;
  return hipSuccess;
}

}  // namespace

extern "C" {

dsa_status dsa_indexer_scores(const dsa_geom* geom, const void* q, dsa_dtype q_dtype, const float* q_scale,
                              const void* w, dsa_dtype w_dtype, const void* k, dsa_dtype k_dtype,
                              const float* k_scale, int32_t row_begin, int32_t row_count, float* scores,
                              int64_t ld, hipStream_t stream) {
  return indexer_scores_impl(geom, nullptr, q, q_dtype, q_scale, w, w_dtype, k, k_dtype, k_scale, row_begin,
                             row_count, scores, ld, stream);
}

dsa_status dsa_indexer_scores_paged(const dsa_geom* geom, const dsa_pages* pages, const void* q, dsa_dtype q_dtype,
                                    const float* q_scale, const void* w, dsa_dtype w_dtype, const void* k_pool,
                                    dsa_dtype k_dtype, const float* k_scale_pool, int32_t row_begin,
                                    int32_t row_count, float* scores, int64_t ld, hipStream_t stream) {
  if (!pages) return DSA_ERR_INVALID_ARG;
  return indexer_scores_impl(geom, pages, q, q_dtype, q_scale, w, w_dtype, k_pool, k_dtype, k_scale_pool,
                             row_begin, row_count, scores, ld, stream);
}

size_t dsa_topk_workspace_size(int32_t row_count, int32_t S_max, int32_t k) {
  if (row_count <= 0 || S_max <= 0 || k <= 0) return 0;
  const int rows = row_count < kMaxRowsPerLaunch ? row_count : kMaxRowsPerLaunch;
  return topk_workspace_bytes(rows, S_max, k);
}

dsa_status dsa_topk(const dsa_geom* geom, const float* scores, int64_t ld, int32_t row_begin, int32_t row_count,
                    int32_t k, int32_t* idx, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!geom_ok(geom) || !rows_ok(geom, row_begin, row_count) || ld < geom->S_max || k < 1)
    return DSA_ERR_INVALID_ARG;
  if (row_count == 0) return DSA_OK;
  if (!scores || !idx || !aligned(scores, 4) || !aligned(idx, 4)) return DSA_ERR_INVALID_ARG;
  if (!topk_supported(geom->S_max, k)) return DSA_ERR_UNSUPPORTED;
  const size_t need = dsa_topk_workspace_size(row_count, geom->S_max, k);
  if (ws_bytes < need || (need && (!ws || !aligned(ws, kAlign)))) return DSA_ERR_WORKSPACE;
  TopkArgs a{};
  a.B = geom->B;
  a.q_len = geom->q_len;
  a.S_max = geom->S_max;
  a.seq_lens = geom->seq_lens;
  a.scores = scores;
  a.ld = ld;
  a.row_begin = row_begin;
  a.row_count = row_count;
  a.k = k;
  a.idx = idx;
  a.ws = ws;
  a.ws_zeroed = 0;
  return hip_status(run_topk(a, stream));
}

size_t dsa_sparse_mla_workspace_size(int32_t B, int32_t q_len, int32_t H, int32_t k, dsa_dtype dtype) {
  if (B < 1 || q_len < 1 || H < 1 || k < 1) return 0;
  return mla_workspace_bytes(B * q_len, H, k, dtype == DSA_BF16);
}

dsa_status dsa_sparse_mla(const dsa_geom* geom, int32_t H, int32_t k, float sm_scale, const void* q,
                          dsa_dtype dtype, const void* kv, const int32_t* idx, void* out, float* lse, void* ws,
                          size_t ws_bytes, hipStream_t stream) {
  return sparse_mla_impl(geom, nullptr, H, k, sm_scale, q, dtype, kv, idx, out, lse, ws, ws_bytes, stream);
}

size_t dsa_sparse_mla_paged_workspace_size(int32_t B, int32_t q_len, int32_t H, int32_t k, dsa_dtype dtype) {
  if (B < 1 || q_len < 1 || H < 1 || k < 1) return 0;
  return mla_paged_workspace_bytes(B * q_len, H, k, dtype);
}

dsa_status dsa_sparse_mla_paged(const dsa_geom* geom, const dsa_pages* pages, int32_t H, int32_t k, float sm_scale,
                                const void* q, dsa_dtype dtype, const void* kv_pool, const int32_t* idx, void* out,
                                float* lse, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!pages) return DSA_ERR_INVALID_ARG;
  return sparse_mla_impl(geom, pages, H, k, sm_scale, q, dtype, kv_pool, idx, out, lse, ws, ws_bytes, stream);
}

size_t dsa_forward_workspace_size(int32_t B, int32_t q_len, int32_t S_max, int32_t H, int32_t topk,
                                  dsa_dtype index_dtype, dsa_dtype mla_dtype) {
  if (B < 1 || q_len < 1 || S_max < 1 || H < 1 || topk < 1) return 0;
  return plan_forward(B, q_len, S_max, H, topk, index_dtype, mla_dtype, false).total;
}

size_t dsa_forward_paged_workspace_size(int32_t B, int32_t q_len, int32_t S_max, int32_t H, int32_t topk,
                                        dsa_dtype index_dtype, dsa_dtype mla_dtype) {
  if (B < 1 || q_len < 1 || S_max < 1 || H < 1 || topk < 1) return 0;
  return plan_forward(B, q_len, S_max, H, topk, index_dtype, mla_dtype, true).total;
}

dsa_status dsa_forward(const dsa_geom* geom, int32_t H, int32_t topk, float sm_scale, const void* index_q,
                       dsa_dtype index_dtype, const float* index_q_scale, const void* index_w,
                       dsa_dtype index_w_dtype, const void* index_k, const float* index_k_scale,
                       const void* mla_q, const void* mla_kv, dsa_dtype mla_dtype, int32_t* idx_out, void* out,
                       float* lse, void* ws, size_t ws_bytes, hipStream_t stream) {
  return forward_impl(geom, nullptr, H, topk, sm_scale, index_q, index_dtype, index_q_scale, index_w, index_w_dtype,
                      index_k, index_k_scale, mla_q, mla_kv, mla_dtype, idx_out, out, lse, ws, ws_bytes, stream);
}

dsa_status dsa_forward_paged(const dsa_geom* geom, const dsa_pages* pages, int32_t H, int32_t topk, float sm_scale,
                             const void* index_q, dsa_dtype index_dtype, const float* index_q_scale,
                             const void* index_w, dsa_dtype index_w_dtype, const void* index_k_pool,
                             const float* index_k_scale_pool, const void* mla_q, const void* mla_kv_pool,
                             dsa_dtype mla_dtype, int32_t* idx_out, void* out, float* lse, void* ws,
                             size_t ws_bytes, hipStream_t stream) {
  if (!pages) return DSA_ERR_INVALID_ARG;
  return forward_impl(geom, pages, H, topk, sm_scale, index_q, index_dtype, index_q_scale, index_w, index_w_dtype,
                      index_k_pool, index_k_scale_pool, mla_q, mla_kv_pool, mla_dtype, idx_out, out, lse, ws,
                      ws_bytes, stream);
}

size_t dsa_indexer_topk_workspace_size(int32_t B, int32_t q_len, int32_t S_max, int32_t topk,
                                       dsa_dtype index_dtype) {
  if (B < 1 || q_len < 1 || S_max < 1 || topk < 1 || S_max <= topk) return 0;
  // the selection part of dsa_forward's plan (its size does not depend on H)
  return plan_forward(B, q_len, S_max, 16, topk, index_dtype, DSA_BF16, false).mla_off;
}

dsa_status dsa_indexer_topk(const dsa_geom* geom, int32_t topk, const void* index_q, dsa_dtype index_dtype,
                            const float* index_q_scale, const void* index_w, dsa_dtype index_w_dtype,
                            const void* index_k, const float* index_k_scale, int32_t* idx_out, void* ws,
                            size_t ws_bytes, hipStream_t stream) {
  const dsa_status st = check_indexer_inputs(geom, index_q, index_dtype, index_q_scale, index_w, index_w_dtype,
                                             index_k, index_dtype, index_k_scale);
  if (st != DSA_OK) return st;
  if (!idx_out || !aligned(idx_out, 4) || topk < 1) return DSA_ERR_INVALID_ARG;
  const ForwardPlan p = plan_forward(geom->B, geom->q_len, geom->S_max, 16, topk, index_dtype, DSA_BF16, false);
  const bool keep_all = geom->S_max <= topk;
  if (!keep_all && !p.streaming && !topk_supported(geom->S_max, topk)) return DSA_ERR_UNSUPPORTED;
  const size_t need = keep_all ? 0 : p.mla_off;
  if (ws_bytes < need || (need && (!ws || !aligned(ws, kAlign)))) return DSA_ERR_WORKSPACE;
  return hip_status(select_impl(geom, nullptr, topk, index_q, index_dtype, index_q_scale, index_w, index_w_dtype,
                                index_k, index_k_scale, idx_out, static_cast<char*>(ws), p, nullptr, stream));
}

dsa_status dsa_indexer_quantize(const void* x, dsa_dtype x_dtype, int64_t rows, uint8_t* codes, float* scales,
                                hipStream_t stream) {
  if (rows < 0) return DSA_ERR_INVALID_ARG;
  if (x_dtype != DSA_BF16 && x_dtype != DSA_F32) return DSA_ERR_UNSUPPORTED;
  if (rows == 0) return DSA_OK;
  if (!x || !codes || !scales || !aligned(x, 16) || !aligned(codes, 4) || !aligned(scales, 4))
    return DSA_ERR_INVALID_ARG;
  QuantArgs a{};
  a.x = x;
  a.rows = rows;
  a.codes = codes;
  a.scales = scales;
  return hip_status(launch_quantize(a, x_dtype == DSA_BF16, stream));
}

dsa_status dsa_indexer_cache_append(const dsa_geom* geom, const void* k_new, dsa_dtype k_dtype, uint8_t* k_cache,
                                    float* k_scale_cache, hipStream_t stream) {
  return cache_append_impl(geom, nullptr, k_new, k_dtype, k_cache, k_scale_cache, stream);
}

dsa_status dsa_indexer_cache_append_paged(const dsa_geom* geom, const dsa_pages* pages, const void* k_new,
                                          dsa_dtype k_dtype, uint8_t* k_pool, float* k_scale_pool,
                                          hipStream_t stream) {
  if (!pages) return DSA_ERR_INVALID_ARG;
  return cache_append_impl(geom, pages, k_new, k_dtype, k_pool, k_scale_pool, stream);
}

size_t dsa_mha_prefill_workspace_size(int32_t B, int32_t S_max, int32_t H) {
  if (B < 1 || S_max < 1 || H < 1) return 0;
  return mha_workspace_bytes(B, S_max, H) + kAlign;
}

dsa_status dsa_mha_prefill(const dsa_geom* geom, int32_t H, float sm_scale, const void* q, const void* kv,
                           const void* wkv_b, dsa_dtype dtype, void* out, float* lse, void* ws, size_t ws_bytes,
                           hipStream_t stream) {
  if (!geom_ok(geom) || !q || !kv || !wkv_b || !out) return DSA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(kv, 16) || !aligned(wkv_b, 16) || !aligned(out, 16)) return DSA_ERR_INVALID_ARG;
  if (lse && !aligned(lse, 4)) return DSA_ERR_INVALID_ARG;
  if (H < 1 || H > 128) return DSA_ERR_INVALID_ARG;
  if (dtype != DSA_BF16) return DSA_ERR_UNSUPPORTED;
  const size_t half = mha_workspace_bytes(geom->B, geom->S_max, H) / 2;
  if (ws_bytes < dsa_mha_prefill_workspace_size(geom->B, geom->S_max, H) || !ws || !aligned(ws, kAlign))
    return DSA_ERR_WORKSPACE;
  MhaArgs a;
  a.B = geom->B;
  a.q_len = geom->q_len;
  a.S_max = geom->S_max;
  a.H = H;
  a.seq_lens = geom->seq_lens;
  a.sm_scale = sm_scale;
  a.q = q;
  a.kv = kv;
  a.wkv_b = wkv_b;
  a.out = out;
  a.lse = lse;
  a.knope_ws = ws;
  a.v_ws = static_cast<char*>(ws) + align_up(half);
  return hip_status(launch_mha_prefill(a, stream));
}

size_t dsa_indexer_kl_workspace_size(int32_t B, int32_t q_len, int32_t S_max, int32_t k) {
  if (B < 1 || q_len < 1 || S_max < 1) return 0;
  return kl_workspace_bytes(B * q_len, k > 0 ? k : S_max);
}

dsa_status dsa_indexer_kl(const dsa_geom* geom, int32_t H, float sm_scale, const void* q, const void* kv,
                          dsa_dtype dtype, const float* lse, const float* scores, int64_t ld, const int32_t* idx,
                          int32_t k, float* kl, float* loss, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!geom_ok(geom) || !q || !kv || !lse || !scores || !kl) return DSA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(kv, 16) || !aligned(lse, 4) || !aligned(scores, 4) || !aligned(kl, 4))
    return DSA_ERR_INVALID_ARG;
  if ((loss && !aligned(loss, 4)) || (idx && !aligned(idx, 4)) || ld < geom->S_max) return DSA_ERR_INVALID_ARG;
  if (H < 32 || H > 128 || H % 32 != 0) return DSA_ERR_INVALID_ARG;
  if (idx && (k < 1 || k > kMaxMlaK)) return DSA_ERR_INVALID_ARG;
  if (dtype != DSA_BF16) return DSA_ERR_UNSUPPORTED;
  const int kk = idx ? k : geom->S_max;
  const size_t need = dsa_indexer_kl_workspace_size(geom->B, geom->q_len, geom->S_max, idx ? k : 0);
  if (ws_bytes < need || !ws || !aligned(ws, kAlign)) return DSA_ERR_WORKSPACE;
  KlArgs a;
  a.B = geom->B;
  a.q_len = geom->q_len;
  a.S_max = geom->S_max;
  a.H = H;
  a.k = kk;
  a.seq_lens = geom->seq_lens;
  a.sm_scale = sm_scale;
  a.q = q;
  a.kv = kv;
  a.lse = lse;
  a.scores = scores;
  a.ld = ld;
  a.idx = idx;
  a.kl = kl;
  a.loss = loss;
  a.ws = static_cast<float*>(ws);
  a.row_begin = 0;
  a.row_count = (int)rows_of(geom);
  return hip_status(launch_indexer_kl(a, stream));
}

size_t dsa_workspace_size(int32_t B, int32_t q_len, int32_t S_max, int32_t H, int32_t k, int which_call) {
  if (B < 1 || q_len < 1 || S_max < 1 || H < 1 || k < 0) return 0;
  if ((long long)B * q_len > 0x7FFFFFFFLL) return 0;
  const dsa_dtype mla_dts[2] = {DSA_BF16, DSA_F32};
  const dsa_dtype idx_dts[2] = {DSA_FP8_E4M3FN, DSA_F32};
  size_t best = 0;
  auto keep = [&](size_t v) { best = v > best ? v : best; };
  switch (which_call) {
    case DSA_CALL_TOPK:
      if (k >= 1) keep(dsa_topk_workspace_size(B * q_len, S_max, k));
      break;
    case DSA_CALL_SPARSE_MLA:
    case DSA_CALL_SPARSE_MLA_PAGED:
      if (k >= 1)
        for (dsa_dtype m : mla_dts)
          keep(which_call == DSA_CALL_SPARSE_MLA ? dsa_sparse_mla_workspace_size(B, q_len, H, k, m)
                                                 : dsa_sparse_mla_paged_workspace_size(B, q_len, H, k, m));
      break;
    case DSA_CALL_FORWARD:
    case DSA_CALL_FORWARD_PAGED:
      if (k >= 1)
        for (dsa_dtype i : idx_dts)
          for (dsa_dtype m : mla_dts)
            keep(which_call == DSA_CALL_FORWARD ? dsa_forward_workspace_size(B, q_len, S_max, H, k, i, m)
                                                : dsa_forward_paged_workspace_size(B, q_len, S_max, H, k, i, m));
      break;
    case DSA_CALL_MHA_PREFILL:
      keep(dsa_mha_prefill_workspace_size(B, S_max, H));
      break;
    case DSA_CALL_INDEXER_KL:
      keep(dsa_indexer_kl_workspace_size(B, q_len, S_max, k));
      break;
    case DSA_CALL_INDEXER_TOPK:
      if (k >= 1)
        for (dsa_dtype i : idx_dts) keep(dsa_indexer_topk_workspace_size(B, q_len, S_max, k, i));
      break;
    default:
      break;
  }
  return best;
}

dsa_status dsa_forward_noalloc(const dsa_geom* geom, int32_t H, int32_t topk, float sm_scale, const void* index_q,
                               dsa_dtype index_dtype, const float* index_q_scale, const void* index_w,
                               dsa_dtype index_w_dtype, const void* index_k, const float* index_k_scale,
                               const void* mla_q, const void* mla_kv, dsa_dtype mla_dtype, int32_t* idx_out,
                               void* out, float* lse, hipStream_t stream) {
  if (!geom_ok(geom) || H < 1 || topk < 1) return DSA_ERR_INVALID_ARG;
  size_t need = dsa_forward_workspace_size(geom->B, geom->q_len, geom->S_max, H, topk, index_dtype, mla_dtype);
  if (!idx_out) need += align_up((size_t)rows_of(geom) * topk * sizeof(int32_t));
  if (need > DSA_NOALLOC_SCRATCH_BYTES) return DSA_ERR_WORKSPACE;
  int dev = 0;
  if ((stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev)) != hipSuccess) return DSA_ERR_HIP;
  if (dev < 0 || dev >= kMaxScratchDevices) return DSA_ERR_UNSUPPORTED;
  void* ws = nullptr;
  if (scratch_address(dev, &ws) != hipSuccess) return DSA_ERR_HIP;
  return forward_impl(geom, nullptr, H, topk, sm_scale, index_q, index_dtype, index_q_scale, index_w, index_w_dtype,
                      index_k, index_k_scale, mla_q, mla_kv, mla_dtype, idx_out, out, lse, ws,
                      DSA_NOALLOC_SCRATCH_BYTES, stream);
}

const char* dsa_status_string(dsa_status s) {
  switch (s) {
    case DSA_OK: return "DSA_OK";
    case DSA_ERR_INVALID_ARG: return "DSA_ERR_INVALID_ARG: bad pointer, shape, alignment or size";
    case DSA_ERR_UNSUPPORTED: return "DSA_ERR_UNSUPPORTED: dtype combination or size not implemented";
    case DSA_ERR_WORKSPACE: return "DSA_ERR_WORKSPACE: workspace missing or too small";
    case DSA_ERR_HIP: return "DSA_ERR_HIP: a HIP launch failed";
  }
  return "unknown dsa_status";
}

const char* dsa_version(void) { return "0.1.0"; }

}  // extern "C"
