// Row-sparse gradient of the embedding tables (the backward pass of a training
// step; architecture walk-through, yaoyuxiang.cn/news/830577, section 4.4,
// trains the tables with the model).  A step reads at most N * H of the
// tables' rows -- 786432 of 480 million at B=1 T=32768 -- so instead of a dense
// float32 copy of the tables it returns those rows once each, in ascending
// order, with the sum of de over the (token, head) pairs that hashed to them.
//
// The rows are found without sorting: a bitmap of the stacked table's rows
// (one bit per row) marks every row a pair selects; per group of 64 bitmap
// words a count of its set bits, scanned (within blocks of 1024 groups, then
// over the blocks), gives each group's first rank; within a group a
// wavefront scans its 64 words' counts, which gives every word's first rank
// and each set bit its place in the row list.  The rank of a row is then its
// word's first rank plus the set bits below it in the word.  Kernels:
//   k_bits_clear   bitmap = 0
//   k_bits_mark    bit of row(n, h) for every pair (atomic or)
//   k_bits_count   set bits per group (a wavefront per group, a lane per word)
//   k_scan_local   exclusive scan of the group counts within blocks of 1024 groups, block totals
//   k_scan_top     exclusive scan of the block totals (one workgroup), U = total
//   k_scan_add     each group's block offset added
//   k_bits_rows    per word its first rank; row ids in rank order (a wavefront per group)
//   k_rows_zero    the U gradient rows cleared
//   k_pair_rank    rank of each pair's row
//   k_rows_add     d_rows[rank(row(n, h))] += de[n][h slice] (float32 atomics)
#include <algorithm>

#include "engram_internal.h"

namespace engram {
namespace {

constexpr int kGroupWords = 64;   // bitmap words (32 rows each) per group: one per lane of a wavefront
constexpr int kScanBlock = 1024;  // groups per block of the first scan level

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

__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// inclusive prefix sum over the 64 lanes of a wavefront
__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t u = __shfl_up(v, o, 64);
    if (lane >= o) v += u;
  }
  return v;
}

__global__ void __launch_bounds__(256) k_bits_count(const uint32_t* __restrict__ bits, int64_t words,
                                                    int64_t groups, uint32_t* __restrict__ count) {
  const int64_t g = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 6;
  if (g >= groups) return;   // whole wavefronts
  const int64_t w = g * kGroupWords + (threadIdx.x & 63);
  const uint32_t c = wave_sum_u32(w < words ? __popc(bits[w]) : 0u);
  if ((threadIdx.x & 63) == 0) count[g] = c;
}

// exclusive scan of count[] within each block of kScanBlock groups into
// first[], and each block's total into bsum[]
__global__ void __launch_bounds__(kScanBlock) k_scan_local(const uint32_t* __restrict__ count, int64_t groups,
                                                            uint32_t* __restrict__ first, uint32_t* __restrict__ bsum) {
  __shared__ uint32_t s[kScanBlock];
  const int t = threadIdx.x;
  const int64_t g = (int64_t)blockIdx.x * kScanBlock + t;
  const uint32_t c = g < groups ? count[g] : 0u;
  s[t] = c;
  __syncthreads();
  for (int o = 1; o < kScanBlock; o <<= 1) {   // inclusive Hillis-Steele scan
    const uint32_t v = t >= o ? s[t - o] : 0u;
    __syncthreads();
    s[t] += v;
    __syncthreads();
  }
  if (g < groups) first[g] = s[t] - c;
  if (t == kScanBlock - 1) bsum[blockIdx.x] = s[t];
}

// exclusive scan of bsum[0..nb) in place, total into *n_rows, by one
// workgroup: each thread sums a contiguous run, the runs' sums are scanned in
// LDS, then each thread writes its run's prefixes.
__global__ void __launch_bounds__(1024) k_scan_top(uint32_t* __restrict__ bsum, int64_t nb,
                                                   int64_t* __restrict__ n_rows) {
  __shared__ uint32_t s[1024];
  const int t = threadIdx.x;
  const int64_t per = (nb + 1023) / 1024;
  const int64_t b0 = min((int64_t)t * per, nb), b1 = min(b0 + per, nb);
  uint32_t sum = 0;
  for (int64_t b = b0; b < b1; b++) sum += bsum[b];
  s[t] = sum;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const uint32_t v = t >= o ? s[t - o] : 0u;
    __syncthreads();
    s[t] += v;
    __syncthreads();
  }
  uint32_t run = s[t] - sum;
  for (int64_t b = b0; b < b1; b++) {
    const uint32_t c = bsum[b];
    bsum[b] = run;
    run += c;
  }
  if (t == 1023) *n_rows = (int64_t)s[1023];
}

__global__ void __launch_bounds__(256) k_scan_add(uint32_t* __restrict__ first, int64_t groups,
                                                  const uint32_t* __restrict__ bsum) {
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (g < groups) first[g] += bsum[g / kScanBlock];
}

// a wavefront per group: each lane's word gets its first rank (wrank), and
// its set bits' rows go to row_index at consecutive ranks from there
__global__ void __launch_bounds__(256) k_bits_rows(const uint32_t* __restrict__ bits,
                                                   const uint32_t* __restrict__ first, int64_t words, int64_t groups,
                                                   uint32_t* __restrict__ wrank, int64_t* __restrict__ row_index) {
  const int64_t g = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 6;
  if (g >= groups) return;   // whole wavefronts
  const int64_t w = g * kGroupWords + (threadIdx.x & 63);
  uint32_t m = w < words ? bits[w] : 0u;
  const uint32_t c = __popc(m);
  uint32_t k = first[g] + wave_incl_scan_u32(c) - c;
  if (w < words) wrank[w] = k;
  while (m) {
    const int b = __ffs(m) - 1;
    m &= m - 1;
    row_index[k++] = (w << 5) + b;
  }
}

// the first *n_rows rows of d_rows cleared (the count is known on the device only)
__global__ void __launch_bounds__(256) k_rows_zero(float* __restrict__ d_rows, const int64_t* __restrict__ n_rows,
                                                   int32_t Dh) {
  const int64_t n = *n_rows * Dh;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) d_rows[i] = 0.f;
}

// rank of the row each (token, head) pair selects: its word's first rank plus
// the set bits below it in the word
__global__ void __launch_bounds__(256) k_pair_rank(HashConsts hc, const int32_t* __restrict__ idx, int64_t pairs,
                                                   const uint32_t* __restrict__ bits,
                                                   const uint32_t* __restrict__ wrank, uint32_t* __restrict__ rank) {
  const int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (p >= pairs) return;
  const int64_t r = pair_row(hc, idx, p), w = r >> 5;
  rank[p] = wrank[w] + __popc(bits[w] & ((1u << (r & 31)) - 1u));
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
int64_t sparse_scan_blocks(int64_t table_rows) { return (sparse_groups(table_rows) + kScanBlock - 1) / kScanBlock; }

hipError_t launch_sparse_rows(const SparseRowsArgs& a, hipStream_t s) {
  const int64_t words = sparse_bitmap_words(a.table_rows), groups = sparse_groups(a.table_rows);
  const int64_t nb = sparse_scan_blocks(a.table_rows);
  const int64_t pairs = a.n_tok * a.hc.n_heads;
  const unsigned wave_blocks = (unsigned)((groups + 3) / 4);   // 4 wavefronts (groups) per workgroup
  k_bits_clear<<<(unsigned)std::min<int64_t>((words + 255) / 256, 8192), 256, 0, s>>>(a.bits, words);
  if (pairs > 0) k_bits_mark<<<(unsigned)((pairs + 255) / 256), 256, 0, s>>>(a.hc, a.idx, pairs, a.bits);
  k_bits_count<<<wave_blocks, 256, 0, s>>>(a.bits, words, groups, a.count);
  k_scan_local<<<(unsigned)nb, kScanBlock, 0, s>>>(a.count, groups, a.first, a.bsum);
  k_scan_top<<<1, 1024, 0, s>>>(a.bsum, nb, a.n_rows);
  k_scan_add<<<(unsigned)((groups + 255) / 256), 256, 0, s>>>(a.first, groups, a.bsum);
  k_bits_rows<<<wave_blocks, 256, 0, s>>>(a.bits, a.first, words, groups, a.wrank, a.row_index);
  const int64_t total = pairs * a.head_dim;   // de is [N][H * Dh]: pair p's slice starts at p * Dh
  k_rows_zero<<<(unsigned)std::min<int64_t>(std::max<int64_t>((total + 255) / 256, 1), 8192), 256, 0, s>>>(
      a.d_rows, a.n_rows, a.head_dim);
  if (pairs > 0) {
    k_pair_rank<<<(unsigned)((pairs + 255) / 256), 256, 0, s>>>(a.hc, a.idx, pairs, a.bits, a.wrank, a.pair_rank);
    k_rows_add<<<(unsigned)((total + 255) / 256), 256, 0, s>>>(a.pair_rank, a.de, total, a.head_dim, a.d_rows);
  }
  return hipGetLastError();
}

}  // namespace engram
