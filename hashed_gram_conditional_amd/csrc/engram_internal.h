// Internal declarations shared by the Engram HIP translation units: kernel
// argument blocks, launchers and small device helpers.  Not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/engram.h"

namespace engram {

// ----------------------------------------------------------------- helpers
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Round to nearest even; NaN stays NaN (quiet).  gfx950 converts in hardware
// (v_cvt_pk_bf16_f32, two values per instruction); on all 2^32 float patterns
// its result equals the integer rounding (u + 0x7FFF + bit 16 of u) >> 16, with
// NaNs quieted by setting bit 6 of the result.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// lo in bits 0-15, hi in bits 16-31
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

__device__ __forceinline__ float ld_elem(const void* p, int64_t i, bool bf16) {
  return bf16 ? bf16_to_f32(((const uint16_t*)p)[i]) : ((const float*)p)[i];
}

// The gate from the fused projection's partial sums of one (token, branch),
// computed by an aligned group of 8 lanes (lane l = lane % 8 adds partials l,
// l+8, ...; xor shuffles combine the 8 sums; every lane of the group returns
// g): rk = (sum K^2 / d + eps)^-1/2, rq alike, s = (sum K gk gq Q) rk rq / sqrt(d),
// g = sigmoid(sign(s) sqrt(max(|s|, clamp))).  All 8 lanes must call it.
__device__ __forceinline__ float gate_from_partials8(const float4* p, int n_part, bool ok, int d, float eps,
                                                     float clamp, float inv_sqrt_d, float4* st = nullptr) {
  const int l = threadIdx.x & 7;
  float kk = 0.f, qq = 0.f, kq = 0.f;
  if (ok)
    for (int t = l; t < n_part; t += 8) {
      const float4 v = p[t];
      kk += v.x;
      qq += v.y;
      kq += v.z;
    }
#pragma unroll
  for (int o = 1; o < 8; o <<= 1) {
    kk += __shfl_xor(kk, o, 64);
    qq += __shfl_xor(qq, o, 64);
    kq += __shfl_xor(kq, o, 64);
  }
  const float inv_d = 1.f / (float)d;
  const float rk = 1.f / sqrtf(kk * inv_d + eps);
  const float rq = 1.f / sqrtf(qq * inv_d + eps);
  const float s = kq * rk * rq * inv_sqrt_d;
  const float sgn = s > 0.f ? 1.f : (s < 0.f ? -1.f : 0.f);
  const float act = sgn * sqrtf(fmaxf(fabsf(s), clamp));
  const float g = 1.f / (1.f + expf(-act));
  if (st) *st = make_float4(g, s, rk, rq);   // the statistics the gradients read
  return g;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// --------------------------------------------------------------- hashing
// Everything the n-gram hash needs, passed by value (kernel arguments).
struct HashConsts {
  int32_t n_orders;
  int32_t heads_per_order;
  int32_t n_heads;
  int32_t max_order;
  int32_t pad_id;
  int32_t vocab;
  int32_t orders[ENGRAM_MAX_ORDERS];
  uint64_t mult[ENGRAM_MAX_ORDERS];
  uint32_t prime[ENGRAM_MAX_HEADS];
  uint32_t wrap[ENGRAM_MAX_HEADS];    // 2^64 mod p: turns an unsigned residue into the int64 floored one
  uint64_t magic[ENGRAM_MAX_HEADS];   // floor((2^64-1) / p) for Barrett reduction
  int64_t row_off[ENGRAM_MAX_HEADS];  // first stacked-table row of each head
};

struct GatherArgs {
  const int32_t* ids;       // [N] raw ids (hash mode)
  const int32_t* remap;     // [vocab] or null
  const int32_t* idx_in;    // [N][H] (gather-only mode)
  int32_t* idx_out;         // [N][H] or null
  const uint8_t* tables;    // stacked tables
  uint8_t* e_out;           // [N][E] or null
  const int32_t* tok_ring;  // [B][max_order-1] or null
  const int64_t* n_past;    // [B] or null
  int64_t* past_out;        // [B] or null: n_past of each sequence before this call
  int32_t batch, seqlen;
  int32_t row_bytes;        // head_dim * element size
};

// multipliers of several layers (layers share orders, heads and primes)
struct LayerMults {
  uint64_t mult[ENGRAM_MAX_LAYERS][ENGRAM_MAX_ORDERS];
  int32_t n_layers;
};
// idx_out of a: [n_layers][N][H]
hipError_t launch_hash_layers(const HashConsts& hc, const LayerMults& lm, const GatherArgs& a, hipStream_t s);

// max_blocks > 0 caps the grid (the workgroups then loop over the token tiles)
hipError_t launch_hash_gather(const HashConsts& hc, const GatherArgs& a, bool compute_hash, hipStream_t s,
                              int max_blocks = 0);

// ------------------------------------------------------------------ GEMM
// g from the fused GEMM's partial sums (per token and branch, one float4 per
// 128 channels)
struct GateFinalizeArgs {
  const float4* partials = nullptr;  // [N][hc][n_part]
  float* g_out = nullptr;            // [N][hc]
  float4* stats = nullptr;           // [N][hc] (g, s, rk, rq), or null
  int32_t n_tok = 0, hc = 0, d = 0, n_part = 0;
  float eps = 0.f, clamp = 0.f, inv_sqrt_d = 0.f;
};

// C[M][N] = A[M][K] * B[N][K]^T (both operands K-contiguous), fp32 accumulate.
struct GemmArgs {
  const void* A;   // e   [M][K]
  const void* B;   // w_kv [N][K]
  void* C;         // kv  [M][ldc]
  int32_t M, N, K;
  int64_t ldc = 0;  // bf16 output's row stride in elements (0: N)
  int32_t accumulate = 0;   // float32 outputs: C += A B^T instead of C = A B^T
  // float32 outputs only: `splits` independent products in one launch, the
  // s-th on A + s split_a, B + s split_b into C + s split_c (elements)
  int32_t splits = 1;
  int64_t split_a = 0, split_b = 0, split_c = 0;
};
// split-K count for a float32-output product of M x N over a long K (1 = none)
int gemm_k_splits(int64_t M, int64_t N, int64_t K);

// fin: also form these gates (from partials complete before the launch), each
// workgroup a share of them ahead of its K loop, so that no finalize kernel runs
hipError_t launch_gemm_bf16(const GemmArgs& a, hipStream_t s, const GateFinalizeArgs* fin = nullptr);
// bf16 operands, float32 result stored or accumulated into C (a.accumulate)
hipError_t launch_gemm_bf16_f32out(const GemmArgs& a, hipStream_t s);

// C[M][N] (float32) = sum_k A[k][m] B[k][n] over bf16 operands stored
// reduction-major (row k holds every m, resp. every n), in `splits` chunks of
// Ks rows: chunk s reduces rows [s Ks, min((s+1) Ks, K)) into C + s split_c.
struct GemmTnArgs {
  const void* A;        // [K][lda]
  const void* B;        // [K][ldb]
  float* C;             // [splits][M][N]
  int32_t M, N;
  int64_t K, Ks;        // rows in all, rows per chunk (a multiple of 64)
  int64_t lda, ldb;     // elements, multiples of 8
  int32_t splits = 1;
  int64_t split_c = 0;
  int32_t accumulate = 0;   // C += instead of C =
};
// false when the shapes leave the kernel's 32-bit buffer offsets (then use
// launch_gemm_bf16_f32out on transposed copies)
bool gemm_tn_fits(const GemmTnArgs& a);
hipError_t launch_gemm_tn_bf16_f32out(const GemmTnArgs& a, hipStream_t s);
hipError_t launch_gemm_f32(const GemmArgs& a, hipStream_t s);

// Projection GEMM with the gate reductions in its epilogue (bf16).  Key tiles
// are not stored: each writes, per token, the partial sums (sum K^2, sum Q^2,
// sum K gk gq Q) over its channels; value tiles are stored to v_out.
struct GemmGateArgs {
  GemmArgs g;             // C unused
  const void* hidden;     // [M][hc][d] queries
  const void* gamma_k;    // [hc][d]
  const void* gamma_q;    // [hc][d]
  void* v_out;            // [M][v_ld]
  float4* partials;       // [M][hc][d/128]: per 128 channels x = sum K^2, y = sum Q^2, z = sum K gk gq Q
  int32_t hc, d;
  int32_t tile_n;         // channel tile: 256 or 128 (from gemm_gate_plan)
  int64_t v_ld = 0;       // row stride of v_out in elements (0: d)
  void* k_out = nullptr;  // [M][k_ld], the keys in columns 0 .. hc d - 1, or null (not stored)
  int64_t k_ld = 0;
  GateFinalizeArgs fin;   // plain GEMM only: gates to form ahead of the K loop (partials null: none)
};

// How the fused projection runs for M tokens: `tile` is its channel tile (0:
// the fused path does not apply); `split`: the gate GEMM covers the key
// channels only and the value channels run as a plain GEMM after it.
struct GatePlan {
  int tile;
  bool split;
};
GatePlan gemm_gate_plan(int64_t M, int hc, int d);
hipError_t launch_gemm_gate_bf16(const GemmGateArgs& a, hipStream_t s);

// g[n][h] from the partial sums of the fused GEMM
hipError_t launch_gate_finalize(const GateFinalizeArgs& a, hipStream_t s);

// ------------------------------------------------------------- gate / conv
struct GateArgs {
  const void* kv;        // [N][hc+1][d]
  const void* hidden;    // [N][hc][d]
  const void* gamma_k;   // [hc][d]
  const void* gamma_q;   // [hc][d]
  float* g_out;          // [N][hc] or null
  float4* stats = nullptr;   // [N][hc] (g, s, rk, rq) or null: what the backward pass needs
  int32_t n_tok, hc, d;
  float eps, clamp, inv_sqrt_d;
  bool bf16;
};

hipError_t launch_gate(const GateArgs& a, hipStream_t s);

struct ConvArgs {
  const void* v;          // value rows, row stride v_stride elements
  int64_t v_stride;
  const float* g;         // [N][hc]
  const void* conv_w;     // [hc][d][K]
  void* out;              // [N][hc][d]
  const void* v_ring;     // [B][R][d] or null
  const float* g_ring;    // [B][R][hc] or null
  const int64_t* n_past;  // [B] or null
  int32_t batch, seqlen, hc, d, ksize, dil;
  bool bf16;
};

hipError_t launch_conv(const ConvArgs& a, hipStream_t s);

// ------------------------------------------------------------- backward
// dVg = dy + (conv taps applied ahead in time) and the taps' gradient (added)
struct ConvBwdArgs {
  const void* dy;          // [N][hc][d]
  const void* kv;          // [N][hc+1][d] (values in the last block)
  const float4* stats;     // [N][hc] (g, s, rk, rq)
  const void* conv_w;      // [hc][d][K]
  void* dvg;               // [N][hc][d] dtype (unfused)
  float* part;             // [conv_bwd_rows][hc][d][K]: tap sums of each block's positions
  // fused (conv_bwd_fused(hc)): dV into the value block of dkv [N][hc+1][d] and
  // dg partials [N][n_dgp][hc] (one per 64 channels of the lane order) instead of dvg
  void* dkv = nullptr;
  float* dgp = nullptr;
  int32_t n_dgp = 0;
  int32_t batch, seqlen, hc, d, ksize, dil;
  int32_t span;            // positions per thread (a block covers 4 spans of one sequence)
  bool bf16;
};
// positions per thread of the conv backward, and the partial rows it writes
int conv_bwd_span(int64_t n_tok);
bool conv_bwd_fused(int32_t hc);              // hc a power of two up to 16
int conv_bwd_dg_parts(int32_t hc, int32_t d);  // dg partials per (token, branch) of the fused kernel
int64_t conv_bwd_rows(int32_t batch, int32_t seqlen);
hipError_t launch_conv_bwd(const ConvBwdArgs& a, hipStream_t s);

// gate and RMSNorm gradients (dK, d hidden) and dV; the gammas' gradients as
// per-block partial sums S = sum_n coef K Q (d gamma_k = gamma_q S, d gamma_q = gamma_k S)
struct GateBwdArgs {
  const void* dvg;         // [N][hc][d] dtype, or null with dgp
  const float* dgp = nullptr;   // [N][n_dgp][hc] dg partials (fused conv kernel; dV already in dkv)
  int32_t n_dgp = 0;
  const void* kv;          // [N][hc+1][d]
  const void* hidden;      // [N][hc][d]
  const void* gamma_k;     // [hc][d]
  const void* gamma_q;
  const float4* stats;     // [N][hc]
  void* dkv;               // [N][hc+1][d]: dK blocks and dV
  void* d_hidden;          // [N][hc][d]
  float* part;             // [gate_bwd_rows][hc][d]
  int32_t n_tok, hc, d;
  int32_t tpb;             // tokens per block
  float clamp, inv_sqrt_d;
  bool bf16;
};
int gate_bwd_tpb(int64_t n_tok);
int64_t gate_bwd_rows(int64_t n_tok);
hipError_t launch_gate_bwd(const GateBwdArgs& a, hipStream_t s);

// out0[c] += scale0[c] * sum_r part[r][c] (scale0 NULL: 1), and the same sum
// into out1 with scale1 when out1 is not NULL; rows summed in a fixed order
hipError_t launch_colsum(const float* part, int64_t rows, int64_t cols, float* out0, const void* scale0,
                         float* out1, const void* scale1, bool bf16, hipStream_t s);
// dst[c][r] = src[r][c] for r < rows, 0 for rows <= r < ld_dst (elements of
// esz bytes; cols and ld_dst multiples of 16 / esz).  chunk > 0 (a multiple of
// 64 dividing ld_dst): the r axis in chunks, dst[r / chunk][c][r % chunk].
hipError_t launch_transpose(const void* src, void* dst, int64_t rows, int64_t cols, int64_t ld_dst, int esz,
                            hipStream_t s, int64_t chunk = 0);

// d_tables[row_off[h] + idx[n][h]][j] += de[n][h*Dh + j]
hipError_t launch_scatter_add(const HashConsts& hc, const int32_t* idx, const float* de, float* d_tables,
                              int64_t n_tok, int32_t head_dim, hipStream_t s);

// Row-sparse table gradient: the rows the pairs select, once each and
// ascending, with the sums of de over the pairs that selected them.
struct SparseRowsArgs {
  HashConsts hc;
  const int32_t* idx;    // [N][H]
  const float* de;       // [N][H * head_dim]
  int64_t n_tok;
  int32_t head_dim;
  int64_t table_rows;    // sum of the primes
  uint32_t* bits;        // [sparse_bitmap_words] scratch
  uint32_t* count;       // [sparse_groups] scratch
  uint32_t* first;       // [sparse_groups] scratch
  uint32_t* bsum;        // [sparse_scan_blocks] scratch
  uint32_t* wrank;       // [sparse_bitmap_words] scratch
  uint32_t* pair_rank;   // [N * H] scratch
  int64_t* row_index;    // [N * H] out: the rows, ascending (the first *n_rows valid)
  float* d_rows;         // [N * H][head_dim] out: their gradients
  int64_t* n_rows;       // [1] out
};
int64_t sparse_bitmap_words(int64_t table_rows);
int64_t sparse_groups(int64_t table_rows);
int64_t sparse_scan_blocks(int64_t table_rows);
hipError_t launch_sparse_rows(const SparseRowsArgs& a, hipStream_t s);

struct AdvanceArgs {
  const int32_t* ids;     // [B][T] raw
  const int32_t* remap;   // or null
  int32_t vocab, pad_id;
  const void* v;          // value rows, stride v_stride
  int64_t v_stride;
  const float* g;         // [N][hc]
  int32_t* tok_ring;
  void* v_ring;
  float* g_ring;
  int64_t* n_past;
  int32_t batch, seqlen, hc, d, tok_ring_len, ring_len;
  bool bf16;
};

hipError_t launch_advance(const AdvanceArgs& a, hipStream_t s);

// One decode step (T = 1) with a state after the fused projection: the gates
// from the partial sums, the conv over the rings' history and the state
// update, in one kernel (replaces gate_finalize, short_conv and advance_state).
struct DecodeTailArgs {
  const float4* partials;  // [B][hc][n_part]
  const void* v;           // [B][d] this step's value rows
  const void* conv_w;      // [hc][d][K]
  void* out;               // [B][hc][d]
  const int64_t* past;     // [B] n_past before the step (from the hash kernel)
  const int32_t* ids;      // [B] raw ids of the step
  const int32_t* remap;    // or null
  int32_t vocab, pad_id;
  int32_t* tok_ring;       // [B][tok_ring_len]
  void* v_ring;            // [B][ring_len][d]
  float* g_ring;           // [B][ring_len][hc]
  int64_t* n_past;         // [B]
  int32_t batch, hc, d, ksize, dil, n_part, ring_len, tok_ring_len;
  float eps, clamp, inv_sqrt_d;
  bool bf16;
};
hipError_t launch_decode_tail(const DecodeTailArgs& a, hipStream_t s);

}  // namespace engram
