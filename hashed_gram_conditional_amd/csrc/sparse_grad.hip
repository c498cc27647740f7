// Row-sparse gradient of the embedding tables (the backward pass of a training
// step; architecture walk-through, yaoyuxiang.cn/news/830577, section 4.4,
// trains the tables with the model).  A step reads at most N * H of the
// tables' rows -- 786432 of 480 million at B=1 T=32768 -- so instead of a dense
// float32 copy of the tables it returns those rows once each, in ascending
// order, with the sum of de over the (token, head) pairs that hashed to them.
//
// The rows are found without sorting: a bitmap of the stacked table's rows
// (one bit per row) marks every row a pair selects; per 64-word group of the
// bitmap a count of its set bits, scanned, gives each group's first rank; the
// rank of a row is then its group's first rank plus the set bits before it in
// the group.  Kernels:
//   k_bits_clear   bitmap = 0
//   k_bits_mark    bit of row(n, h) for every pair (atomic or)
//   k_bits_count   set bits per group
//   k_bits_scan    exclusive scan of the group counts (one workgroup), U = total
//   k_bits_rows    row ids in rank order
//   k_rows_zero    the U gradient rows cleared
//   k_pair_rank    rank of each pair's row
//   k_rows_add     d_rows[rank(row(n, h))] += de[n][h slice] (float32 atomics)
#include <algorithm>

#include "engram_internal.h"

namespace engram {
namespace {

constexpr int kGroupWords = 64;   // bitmap words (32 rows each) per counted group

__global__ void __launch_bounds__(256) k_bits_clear(uint32_t* __restrict__ bits, int64_t words) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < words; i += (int64_t)gridDim.x * 256) bits[i] = 0;
}

__device__ __forceinline__ int64_t pair_row(const HashConsts& hc, const int32_t* idx, int64_t p) {
  const int h = (int)(p % hc.n_heads);
  return hc.row_off[h] + idx[p];
}

__global__ void __launch_bounds__(256) k_bits_mark(HashConsts hc, const int32_t* __restrict__ idx, int64_t pairs,
                                                   uint32_t* __restrict__ bits) {
  const int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (p >= pairs) return;
  const int64_t r = pair_row(hc, idx, p);
  atomicOr(&bits[r >> 5], 1u << (r & 31));
}

__global__ void __launch_bounds__(256) k_bits_count(const uint32_t* __restrict__ bits, int64_t words,
                                                    int64_t groups, uint32_t* __restrict__ count) {
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (g >= groups) return;
  const int64_t w0 = g * kGroupWords, w1 = min(w0 + kGroupWords, words);
  uint32_t c = 0;
  for (int64_t w = w0; w < w1; w++) c += __popc(bits[w]);
  count[g] = c;
}

// Exclusive scan of count[0..groups) into first[], total into *n_rows, by one
// workgroup: each thread sums a contiguous run, the runs' sums are scanned in
// LDS, then each thread writes its run's prefixes.
__global__ void __launch_bounds__(1024) k_bits_scan(const uint32_t* __restrict__ count, int64_t groups,
                                                    uint32_t* __restrict__ first, int64_t* __restrict__ n_rows) {
  __shared__ uint32_t s[1024];
  const int t = threadIdx.x;
  const int64_t per = (groups + 1023) / 1024;
  const int64_t g0 = min((int64_t)t * per, groups), g1 = min(g0 + per, groups);
  uint32_t sum = 0;
  for (int64_t g = g0; g < g1; g++) sum += count[g];
  s[t] = sum;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {   // inclusive Hillis-Steele scan
    const uint32_t v = t >= o ? s[t - o] : 0;
    __syncthreads();
    s[t] += v;
    __syncthreads();
  }
  uint32_t run = s[t] - sum;
  for (int64_t g = g0; g < g1; g++) {
    first[g] = run;
    run += count[g];
  }
  if (t == 1023) *n_rows = (int64_t)s[1023];
}

// rank of row r: its group's first rank plus the set bits before it
__device__ __forceinline__ uint32_t row_rank(const uint32_t* bits, const uint32_t* first, int64_t r) {
  const int64_t w = r >> 5, g = w / kGroupWords;
  uint32_t k = first[g];
  for (int64_t v = g * kGroupWords; v < w; v++) k += __popc(bits[v]);
  return k + __popc(bits[w] & ((1u << (r & 31)) - 1u));
}

// one thread per group: the group's rows, in ascending order, at their ranks
__global__ void __launch_bounds__(256) k_bits_rows(const uint32_t* __restrict__ bits, const uint32_t* __restrict__ first,
                                                   int64_t words, int64_t groups, int64_t* __restrict__ row_index) {
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (g >= groups) return;
  uint32_t k = first[g];
  const int64_t w1 = min((g + 1) * kGroupWords, words);
  for (int64_t w = g * kGroupWords; w < w1; w++) {
    uint32_t m = bits[w];
    while (m) {
      const int b = __ffs(m) - 1;
      m &= m - 1;
      row_index[k++] = (w << 5) + b;
    }
  }
}

// the first *n_rows rows of d_rows cleared (the count is known on the device only)
__global__ void __launch_bounds__(256) k_rows_zero(float* __restrict__ d_rows, const int64_t* __restrict__ n_rows,
                                                   int32_t Dh) {
  const int64_t n = *n_rows * Dh;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) d_rows[i] = 0.f;
}

// rank of the row each (token, head) pair selects
__global__ void __launch_bounds__(256) k_pair_rank(HashConsts hc, const int32_t* __restrict__ idx, int64_t pairs,
                                                   const uint32_t* __restrict__ bits,
                                                   const uint32_t* __restrict__ first, uint32_t* __restrict__ rank) {
  const int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (p >= pairs) return;
  rank[p] = row_rank(bits, first, pair_row(hc, idx, p));
}

// one thread per (pair, element of the head's slice)
__global__ void __launch_bounds__(256) k_rows_add(const uint32_t* __restrict__ rank, const float* __restrict__ de,
                                                  int64_t total, int32_t Dh, float* __restrict__ d_rows) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  const int64_t p = i / Dh;
  atomicAdd(&d_rows[(int64_t)rank[p] * Dh + (i - p * Dh)], de[i]);
}

}  // namespace

int64_t sparse_bitmap_words(int64_t table_rows) { return (table_rows + 31) / 32; }
int64_t sparse_groups(int64_t table_rows) {
  return (sparse_bitmap_words(table_rows) + kGroupWords - 1) / kGroupWords;
}

hipError_t launch_sparse_rows(const SparseRowsArgs& a, hipStream_t s) {
  const int64_t words = sparse_bitmap_words(a.table_rows), groups = sparse_groups(a.table_rows);
  const int64_t pairs = a.n_tok * a.hc.n_heads;
  k_bits_clear<<<(unsigned)std::min<int64_t>((words + 255) / 256, 8192), 256, 0, s>>>(a.bits, words);
  if (pairs > 0) k_bits_mark<<<(unsigned)((pairs + 255) / 256), 256, 0, s>>>(a.hc, a.idx, pairs, a.bits);
  k_bits_count<<<(unsigned)((groups + 255) / 256), 256, 0, s>>>(a.bits, words, groups, a.count);
  k_bits_scan<<<1, 1024, 0, s>>>(a.count, groups, a.first, a.n_rows);
  k_bits_rows<<<(unsigned)((groups + 255) / 256), 256, 0, s>>>(a.bits, a.first, words, groups, a.row_index);
  const int64_t total = pairs * a.head_dim;   // de is [N][H * Dh]: pair p's slice starts at p * Dh
  k_rows_zero<<<(unsigned)std::min<int64_t>(std::max<int64_t>((total + 255) / 256, 1), 8192), 256, 0, s>>>(
      a.d_rows, a.n_rows, a.head_dim);
  if (pairs > 0) {
    k_pair_rank<<<(unsigned)((pairs + 255) / 256), 256, 0, s>>>(a.hc, a.idx, pairs, a.bits, a.first, a.pair_rank);
    k_rows_add<<<(unsigned)((total + 255) / 256), 256, 0, s>>>(a.pair_rank, a.de, total, a.head_dim, a.d_rows);
  }
  return hipGetLastError();
}

}  // namespace engram
