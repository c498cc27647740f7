// K1: compressed-token remap, time shifts, multi-head n-gram hash and the
// gather of the hashed rows into e_t, fused in one kernel.
//
// Definitions: formula sheet (kwkr.cn/news/37585) section 1.2 steps 1-2 and
// the full formula in 1.3 (mix = xor of t_k * m_k, hash = mix mod p_{n,j}),
// section 4.2 (shift_k with pad_id); architecture walk-through
// (yaoyuxiang.cn/news/830577) sections 2.2-1 and 4.3 (concatenate the rows of
// all heads into e_t).
//
// Layout of the work: one 256-thread workgroup takes 16 consecutive tokens
// (flattened over batch and time; fewer when the call has too few tokens to
// give every CU two workgroups).  It stages the compressed ids of those
// tokens plus the max_order-1 tokens before them in LDS (one remap lookup per
// token instead of one per (token, head, offset)), hashes every (token, head)
// pair into a global table row kept in LDS, then copies the rows to e_t in
// 16-byte pieces: consecutive lanes take consecutive pieces of e_t, so a
// 128-byte bf16 row is one 8-lane load and every store is coalesced, and each
// lane keeps 8 independent row loads in flight before it stores.
//
// Tables in host memory (mapped into the device): each row load then waits on
// the host link for microseconds, and a workgroup per 16 tokens would hold
// every CU while it waits, starving whatever runs beside it.  The launch is
// then a small grid whose workgroups loop over the token tiles; a few of them
// keep enough loads in flight to fill the link.
#include "engram_internal.h"

namespace engram {
namespace {

constexpr int kThreads = 256;
constexpr int kTokens = 16;       // tokens per workgroup (at most)
constexpr int kUnroll = 8;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // one 16-byte piece

// Floored modulo of the int64 value with bit pattern u by p (numpy's `%` on
// int64): Barrett reduction of the unsigned value with magic = floor((2^64-1)/p)
// leaves a residue below 3p; if u is negative as int64 its value is u - 2^64,
// whose residue is (u mod p) - (2^64 mod p), brought back into [0, p).
__device__ __forceinline__ uint32_t floored_mod(uint64_t u, uint32_t p, uint64_t magic, uint32_t wrap) {
  const uint64_t q = __umul64hi(u, magic);
  uint64_t r = u - q * (uint64_t)p;
  if (r >= p) r -= p;
  if (r >= p) r -= p;
  if ((int64_t)u < 0) {
    r += (uint64_t)(p - wrap);
    if (r >= p) r -= p;
  }
  return (uint32_t)r;
}

// Staging of one tile's tokens (ends with a barrier):
//  - s_x: remapped ids of tokens n0-W .. n0+ntok-1 (W = max_order-1); ids before
//    the start of the flattened batch read as pad;
//  - s_hist[ti*W + k-1], for each token ti and offset k = 1..W that falls
//    before its sequence's position 0: the compressed id there, from the
//    state's token ring, or pad before the sequence start.
// The ids (id, then remap) and the ring (n_past, then the ring slot) are each
// two dependent loads; the first two waves take the ids and the last two the
// ring, so the two chains overlap (one decode step: every token's history is
// in the ring).
__device__ __forceinline__ void stage_window(const HashConsts& hc, const GatherArgs& a, int32_t* s_x, int32_t* s_hist,
                                             int64_t n0, int ntok) {
  static_assert(kTokens + ENGRAM_MAX_ORDERS - 1 <= kThreads / 2 && kTokens * (ENGRAM_MAX_ORDERS - 1) <= kThreads / 2,
                "one pass per half of the workgroup");
  const int W = hc.max_order - 1;
  const int tid = threadIdx.x;
  if (tid < ntok + W) {
    const int64_t n = n0 - W + tid;
    int32_t x = hc.pad_id;
    if (n >= 0) {
      const int32_t id = a.ids[n];
      if (id >= 0 && id < hc.vocab) x = a.remap ? a.remap[id] : id;
    }
    s_x[tid] = x;
  }
  const int j = tid - kThreads / 2;
  if (j >= 0 && j < ntok * W) {
    const int ti = j / W, k = 1 + j % W;
    const int64_t n = n0 + ti, b = n / a.seqlen;
    const int32_t t = (int32_t)(n - b * a.seqlen);
    if (t - k < 0) {
      const int64_t p = (a.n_past ? a.n_past[b] : 0) + t - k;
      s_hist[j] = p < 0 ? hc.pad_id : a.tok_ring[b * W + p % W];
    }
  }
  __syncthreads();
}

// Hash of token n = n0 + ti for head h with multipliers mult: the mix over the
// order's shifted tokens (from the staged window, or before position 0 of the
// sequence from the staged history), then the floored mod.
__device__ __forceinline__ uint32_t hash_one(const HashConsts& hc, const GatherArgs& a, const int32_t* s_x,
                                             const int32_t* s_hist, int64_t n0, int ti, int h, const uint64_t* mult) {
  const int W = hc.max_order - 1;
  const int64_t n = n0 + ti;
  const int32_t t = (int32_t)(n - n / a.seqlen * a.seqlen);
  const int order = hc.orders[h / hc.heads_per_order];
  uint64_t mix = 0;
  for (int k = 0; k < order; k++) {
    const int32_t tok = t - k >= 0 ? s_x[W + ti - k] : s_hist[ti * W + k - 1];
    mix ^= (uint64_t)(int64_t)tok * mult[k];
  }
  return floored_mod(mix, hc.prime[h], hc.magic[h], hc.wrap[h]);
}

// TOK tokens per workgroup: 16 on large calls; fewer on small ones (decode
// steps), so that the work spreads over more compute units
template <typename Chunk, int TOK>
__global__ void __launch_bounds__(kThreads) k_hash_gather(HashConsts hc, GatherArgs a, int compute_hash) {
  static_assert(TOK <= kTokens, "staging sized for kTokens");
  __shared__ int32_t s_x[TOK + ENGRAM_MAX_ORDERS];
  __shared__ int32_t s_hist[TOK * ENGRAM_MAX_ORDERS];
  __shared__ int64_t s_row[TOK * ENGRAM_MAX_HEADS];

  const int64_t N = (int64_t)a.batch * a.seqlen;
  const int H = hc.n_heads;
  const int tid = threadIdx.x;
  const int64_t n_tiles = (N + TOK - 1) / TOK;
  for (int64_t tile = blockIdx.x; tile < n_tiles; tile += gridDim.x) {
    const int64_t n0 = tile * TOK;
    const int ntok = (int)min((int64_t)TOK, N - n0);

    if (compute_hash) {
      if (a.past_out)   // n_past before this call, for kernels that advance the state later
        for (int ti = tid; ti < ntok; ti += kThreads) {
          const int64_t n = n0 + ti, b = n / a.seqlen;
          if (n - b * a.seqlen == 0) a.past_out[b] = a.n_past ? a.n_past[b] : 0;
        }
      stage_window(hc, a, s_x, s_hist, n0, ntok);
      for (int pr = tid; pr < ntok * H; pr += kThreads) {
        const int ti = pr / H, h = pr - ti * H;
        const uint32_t r = hash_one(hc, a, s_x, s_hist, n0, ti, h, hc.mult);
        if (a.idx_out) a.idx_out[(n0 + ti) * H + h] = (int32_t)r;
        s_row[ti * H + h] = hc.row_off[h] + r;
      }
    } else {
      for (int pr = tid; pr < ntok * H; pr += kThreads) {
        const int ti = pr / H, h = pr - ti * H;
        int32_t r = a.idx_in[(n0 + ti) * H + h];
        r = r < 0 ? 0 : (r >= (int32_t)hc.prime[h] ? (int32_t)hc.prime[h] - 1 : r);
        s_row[ti * H + h] = hc.row_off[h] + r;
      }
    }
    __syncthreads();
    if (a.e_out != nullptr) {
      const int cpr = a.row_bytes / (int)sizeof(Chunk);  // pieces per table row
      const int cpt = H * cpr;                           // pieces per token
      const int total = ntok * cpt;
      const Chunk* __restrict__ tab = reinterpret_cast<const Chunk*>(a.tables);
      Chunk* __restrict__ e = reinterpret_cast<Chunk*>(a.e_out) + n0 * cpt;
      auto src = [&](int c) -> const Chunk* {
        const int ti = c / cpt;
        const int r = c - ti * cpt;
        const int h = r / cpr;
        const int col = r - h * cpr;
        return tab + s_row[ti * H + h] * cpr + col;
      };
      // full rounds: kUnroll independent row loads in flight per lane, then
      // the stores; a last, partial round masks off the pieces past the tile
      // so that its loads are in flight together too (B=1 T=32768, 24 heads of
      // 160-byte rows: 15 pieces per lane, 61 -> 57-59 us on MI355X)
      int base = tid;
      for (; base + (kUnroll - 1) * kThreads < total; base += kThreads * kUnroll) {
        Chunk v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; u++) v[u] = *src(base + u * kThreads);
#pragma unroll
        for (int u = 0; u < kUnroll; u++) e[base + u * kThreads] = v[u];
      }
      if (base < total) {
        Chunk v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; u++)
          if (base + u * kThreads < total) v[u] = *src(base + u * kThreads);
#pragma unroll
        for (int u = 0; u < kUnroll; u++)
          if (base + u * kThreads < total) e[base + u * kThreads] = v[u];
      }
    }
    __syncthreads();   // s_x and s_row are rewritten by the next tile
  }
}

// Indices of several layers in one pass: the window is staged once per tile and
// each (token, head) is hashed with every layer's multipliers.
__global__ void __launch_bounds__(kThreads) k_hash_layers(HashConsts hc, LayerMults lm, GatherArgs a) {
  __shared__ int32_t s_x[kTokens + ENGRAM_MAX_ORDERS];
  __shared__ int32_t s_hist[kTokens * ENGRAM_MAX_ORDERS];
  const int64_t N = (int64_t)a.batch * a.seqlen;
  const int H = hc.n_heads;
  const int64_t n_tiles = (N + kTokens - 1) / kTokens;
  for (int64_t tile = blockIdx.x; tile < n_tiles; tile += gridDim.x) {
    const int64_t n0 = tile * kTokens;
    const int ntok = (int)min((int64_t)kTokens, N - n0);
    stage_window(hc, a, s_x, s_hist, n0, ntok);
    for (int pr = threadIdx.x; pr < ntok * H; pr += kThreads) {
      const int ti = pr / H, h = pr - ti * H;
      for (int l = 0; l < lm.n_layers; l++)
        a.idx_out[((int64_t)l * N + n0 + ti) * H + h] = (int32_t)hash_one(hc, a, s_x, s_hist, n0, ti, h, lm.mult[l]);
    }
    __syncthreads();   // s_x is rewritten by the next tile
  }
}

}  // namespace

hipError_t launch_hash_layers(const HashConsts& hc, const LayerMults& lm, const GatherArgs& a, hipStream_t s) {
  const int64_t N = (int64_t)a.batch * a.seqlen;
  if (N == 0) return hipSuccess;
  k_hash_layers<<<(unsigned)((N + kTokens - 1) / kTokens), kThreads, 0, s>>>(hc, lm, a);
  return hipGetLastError();
}

template <int TOK>
hipError_t hash_gather_tok(const HashConsts& hc, const GatherArgs& a, bool compute_hash, hipStream_t s,
                           int max_blocks) {
  const int64_t N = (int64_t)a.batch * a.seqlen;
  int64_t tiles = (N + TOK - 1) / TOK;
  if (max_blocks > 0 && tiles > max_blocks) tiles = max_blocks;
  const unsigned blocks = (unsigned)tiles;
  const int ch = compute_hash ? 1 : 0;
  if (a.row_bytes % 16 == 0)
    k_hash_gather<u32x4, TOK><<<blocks, kThreads, 0, s>>>(hc, a, ch);
  else if (a.row_bytes % 4 == 0)
    k_hash_gather<uint32_t, TOK><<<blocks, kThreads, 0, s>>>(hc, a, ch);
  else
    k_hash_gather<uint16_t, TOK><<<blocks, kThreads, 0, s>>>(hc, a, ch);
  return hipGetLastError();
}

hipError_t launch_hash_gather(const HashConsts& hc, const GatherArgs& a, bool compute_hash, hipStream_t s,
                              int max_blocks) {
  const int64_t N = (int64_t)a.batch * a.seqlen;
  if (N == 0) return hipSuccess;
  if (max_blocks > 0) return hash_gather_tok<kTokens>(hc, a, compute_hash, s, max_blocks);
  // the most tokens per workgroup that still leaves two workgroups per CU
  // (a decode step of 256 sequences: one token each; measured on MI355X, B=256
  // decode 7.4 -> 5.9 us, B=4 T=1024 8.3 -> 7.8 us)
  if (N >= 16 * 512) return hash_gather_tok<16>(hc, a, compute_hash, s, 0);
  if (N >= 8 * 512) return hash_gather_tok<8>(hc, a, compute_hash, s, 0);
  if (N >= 4 * 512) return hash_gather_tok<4>(hc, a, compute_hash, s, 0);
  if (N >= 2 * 512) return hash_gather_tok<2>(hc, a, compute_hash, s, 0);
  return hash_gather_tok<1>(hc, a, compute_hash, s, 0);
}

}  // namespace engram
