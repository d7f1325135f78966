// Selected positions -> rows of a paged latent pool.
//
// With a paged cache (the logical-position -> page mapping that the
// charlestar page raises in "Prefill 与 decode 中发生了什么" under Decode and
// in "Top-k 是算法与 kernel 的交界面"), the top-k positions of a query are
// translated once into rows of the page pool, so the attention kernel
// gathers from a flat [rows, 576] pool exactly as it gathers from one
// sequence's contiguous cache, with no table read in front of any gather.
// Positions the query may not select (negative, or past its query position)
// become -1, the value the attention kernel skips.
//
// One thread per four consecutive entries of one query row (k % 4 == 0), or
// per entry otherwise; grid-stride.
#include "dsa_internal.h"

namespace dsa {

namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void k_page_rows4(const int32_t* idx, int32_t* rows, long long nq, int k,
                                                         int q_len, int S_max, const int32_t* seq_lens,
                                                         PageMap pm) {
  const int kq = k >> 2;
  for (long long e = (long long)blockIdx.x * kThreads + threadIdx.x; e < nq; e += (long long)gridDim.x * kThreads) {
    const int t = (int)(e / kq);
    const int b = t / q_len;
    const int pos = row_pos(seq_lens, t, q_len, S_max);
    const v4i s = reinterpret_cast<const v4i*>(idx)[e];
    v4i r;
    r[0] = page_row(s[0], pos, b, pm);
    r[1] = page_row(s[1], pos, b, pm);
    r[2] = page_row(s[2], pos, b, pm);
    r[3] = page_row(s[3], pos, b, pm);
    reinterpret_cast<v4i*>(rows)[e] = r;
  }
}

__global__ __launch_bounds__(kThreads) void k_page_rows1(const int32_t* idx, int32_t* rows, long long n, int k,
                                                         int q_len, int S_max, const int32_t* seq_lens,
                                                         PageMap pm) {
  for (long long e = (long long)blockIdx.x * kThreads + threadIdx.x; e < n; e += (long long)gridDim.x * kThreads) {
    const int t = (int)(e / k);
    rows[e] = page_row(idx[e], row_pos(seq_lens, t, q_len, S_max), t / q_len, pm);
  }
}

unsigned grid_for(long long n) {
  const long long ctas = (n + kThreads - 1) / kThreads;
  return (unsigned)(ctas < 8192 ? ctas : 8192);
}

}  // namespace

hipError_t launch_page_rows(const int32_t* idx, int32_t* rows, int T, int k, int q_len, int S_max,
                            const int32_t* seq_lens, const PageMap& pages, hipStream_t stream) {
  const long long n = (long long)T * k;
  if (n <= 0) return hipSuccess;
  const bool vec = (k & 3) == 0 && ((uintptr_t)idx & 15) == 0 && ((uintptr_t)rows & 15) == 0;
  if (vec) {
    hipLaunchKernelGGL(k_page_rows4, dim3(grid_for(n / 4)), dim3(kThreads), 0, stream, idx, rows, n / 4, k, q_len,
                       S_max, seq_lens, pages);
  } else {
    hipLaunchKernelGGL(k_page_rows1, dim3(grid_for(n)), dim3(kThreads), 0, stream, idx, rows, n, k, q_len, S_max,
                       seq_lens, pages);
  }
  return hipGetLastError();
}

}  // namespace dsa
