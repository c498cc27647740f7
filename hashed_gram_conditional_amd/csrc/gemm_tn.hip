// Weight gradient of the projections, dW = dKV^T e: a reduction over the token
// axis of two token-major operands (dKV [tokens][(hc+1) d], e [tokens][E]),
// as the derivative of the projection K/V = W e (formula sheet,
// kwkr.cn/news/37585, section 2.2 steps 1 and 3) over all tokens.
//
// C[m][n] = sum_k A[k][m] B[k][n] with A and B stored reduction-major.  Each
// K step DMAs 64 rows of the A tile and of the B tile into LDS as they are
// stored, and gfx950's transposing LDS read (ds_read_b64_tr_b16) turns them
// into MFMA fragments.  Within each group of 16 lanes that read returns to lane
// j element j % 4 of the 8-byte blocks addressed by lanes j/4, j/4 + 4,
// j/4 + 8 and j/4 + 12.  A lane s that addresses row k0 + s/4, columns
// c0 + 4 (s % 4) .. + 3 therefore hands lane j the four values of column
// c0 + j in rows k0 .. k0 + 3; two such reads give the 8 consecutive k of one
// row of a 32x32x16 MFMA operand.  No transposed copies of dKV and e are made.
//
// Tiles: 256 x 256 per workgroup of 8 waves (4 x 2, 64 x 128 per wave) when
// there are at least two such tiles per CU, else 128 x 128 per workgroup of 4
// waves; two LDS stages, float32 result stored or added.
#include <algorithm>
#include <utility>

#include "gemm_common.h"

namespace engram {
namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kBK = 64;   // rows of the reduction axis per K step

// Physical 16-byte piece of logical piece p in LDS row r.  The transposing
// reads of one 32-lane pass touch 4 consecutive rows (r % 4 = 0..3) x 4
// consecutive pieces starting at a multiple of 4; the XOR moves each row's
// pieces to a different quarter of an aligned 16-piece span (256 bytes, the 64
// banks), so the pass hits 16 distinct bank groups.
__device__ __forceinline__ int tn_swz(int r, int p) { return p ^ ((r & 3) << 2); }

template <int BM, int BN, int WM, int WN>
__global__ void __launch_bounds__(64 * WM * WN, 1) k_gemm_tn(GemmTnArgs a) {
  constexpr int NW = WM * WN;
  constexpr int TM = BM / WM / 32, TN = BN / WN / 32;   // 32-wide fragments per wave along m and n
  constexpr int PA = BM / 8, PB = BN / 8;               // 16-byte pieces per LDS row of each operand
  constexpr int QA = kBK * PA / (64 * NW), QB = kBK * PB / (64 * NW);   // DMA instructions per wave per step
  constexpr int kPerStep = QA + QB;
  static_assert(QA * 64 * NW == kBK * PA && QB * 64 * NW == kBK * PB, "whole DMA instructions");
  static_assert(PA >= 16 && PB >= 16, "rows of at least 256 bytes: the swizzle spans 16 pieces");
  static_assert(kPerStep % 4 == 0, "the next step's loads are issued a quarter per k slice");
  // rows one DMA instruction of the whole workgroup covers: a multiple of 4, so
  // instruction x leaves a lane's swizzle unchanged
  constexpr int kRowsA = 64 * NW / PA, kRowsB = 64 * NW / PB;
  static_assert(kRowsA % 4 == 0 && kRowsB % 4 == 0, "swizzle period");
  constexpr int kStageA = kBK * PA, kStage = kBK * (PA + PB);   // u32x4 per A region / per stage
  __shared__ u32x4 smem[2 * kStage];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % WM, wn = wave / WM;
  const int m_tiles = (a.M + BM - 1) / BM, n_tiles = (a.N + BN - 1) / BN;
  int mt, nt;
  tile_of(blockIdx.x, a.splits * m_tiles, n_tiles, mt, nt);
  const int split = mt / m_tiles;
  mt -= split * m_tiles;
  const int m0 = mt * BM, n0 = nt * BN;
  const int64_t k_first = (int64_t)split * a.Ks;
  const int64_t rows = std::max((int64_t)0, std::min(a.Ks, a.K - k_first));   // rows of this chunk
  const int nk = (int)(a.Ks / kBK);
  // rows past the chunk, and offsets marked out of range, read zero
  const __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const uint16_t*)a.A + k_first * a.lda), (short)0, (int)(rows * a.lda * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t rB = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const uint16_t*)a.B + k_first * a.ldb), (short)0, (int)(rows * a.ldb * 2), 0x00020000);
  const int rowA = (int)(a.lda * 2), rowB = (int)(a.ldb * 2);   // bytes per stored row

  // This lane's slot in the 1 KB that one DMA instruction fills in lane order:
  // row (wave 64 + lane) / P of the instruction's rows, physical piece
  // (wave 64 + lane) % P, which holds the logical piece tn_swz(row, physical).
  // Columns past M (or N) read whatever follows in memory; they only feed
  // results that are not stored.
  const int voffA = [&] {
    const int q = wave * 64 + lane, r = q / PA;
    return r * rowA + (m0 + tn_swz(r, q % PA) * 8) * 2;
  }();
  const int voffB = [&] {
    const int q = wave * 64 + lane, r = q / PB;
    return r * rowB + (n0 + tn_swz(r, q % PB) * 8) * 2;
  }();

  // instruction x of this wave's share of step kt, into stage S
  auto issue_one = [&](auto stage_tag, int kt, auto x_tag) {
    constexpr int S = decltype(stage_tag)::value;
    constexpr int X = decltype(x_tag)::value;
    const bool in = kt < nk;
    if constexpr (X < QA) {
      const int soff = in ? (kt * kBK + X * kRowsA) * rowA : 0;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, LDS_PTR(&smem[S * kStage + (X * NW + wave) * 64]), 16,
                                               in ? voffA : kOutOfRange, soff, 0, 0);
    } else {
      const int soff = in ? (kt * kBK + (X - QA) * kRowsB) * rowB : 0;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rB, LDS_PTR(&smem[S * kStage + kStageA + ((X - QA) * NW + wave) * 64]),
                                               16, in ? voffB : kOutOfRange, soff, 0, 0);
    }
  };
  // quarter P of step kt's loads
  auto issue_part = [&](auto stage_tag, int kt, auto part_tag) {
    constexpr int P = decltype(part_tag)::value;
    constexpr int lo = P * kPerStep / 4, hi = (P + 1) * kPerStep / 4;
    [&]<int... X>(std::integer_sequence<int, X...>) {
      (issue_one(stage_tag, kt, std::integral_constant<int, lo + X>{}), ...);
    }(std::make_integer_sequence<int, hi - lo>{});
  };

  // Fragment reads: lane group g = lane / 16 takes fragment columns 16 (g % 2)
  // .. + 15 and the k half g / 2; lane j = lane % 16 of the group addresses
  // row j / 4 and columns 4 (j % 4) .. + 3 of its 4 x 16 block.
  const int j16 = lane & 15, grp = lane >> 4;
  const int fr_row = 8 * (grp >> 1) + (j16 >> 2);
  const int fr_col = 16 * (grp & 1) + 4 * (j16 & 3);
  auto frag = [&](u32x4* region, int P, int row0, int col0) {
    char* base = (char*)region;
    auto at = [&](int row) {
      const int col = col0 + fr_col;
      return (lds_s16x4*)(base + row * P * 16 + (tn_swz(row, col >> 3) << 4) + ((col & 7) << 1));
    };
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(at(row0 + fr_row));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(at(row0 + fr_row + 4));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; i++)
#pragma unroll
    for (int j = 0; j < TN; j++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[i][j][r] = 0.f;

  // One K step from stage S, while step kt + 1's loads go into the other
  // stage.  Every fragment of the step is read before the first of those
  // loads is issued: an LDS read after an LDS DMA waits for the DMA (the
  // compiler cannot tell the stages apart), so reads and DMA issues are not
  // interleaved; the MFMAs are.
  auto step = [&](auto stage_tag, int kt) {
    constexpr int S = decltype(stage_tag)::value;
    constexpr std::integral_constant<int, 1 - S> next{};
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));   // this step's loads have landed (this wave's) ...
    __builtin_amdgcn_s_barrier();               // ... and every wave's; the other stage is free
    u32x4* sa = &smem[S * kStage];
    u32x4* sb = sa + kStageA;
    bf16x8 fa[4][TM], fb[4][TN];
#pragma unroll
    for (int p = 0; p < 4; p++) {
#pragma unroll
      for (int i = 0; i < TM; i++) fa[p][i] = frag(sa, PA, 16 * p, wm * (BM / WM) + 32 * i);
#pragma unroll
      for (int j = 0; j < TN; j++) fb[p][j] = frag(sb, PB, 16 * p, wn * (BN / WN) + 32 * j);
    }
    __builtin_amdgcn_sched_barrier(0);
    auto slice = [&](auto part_tag) {
      constexpr int P = decltype(part_tag)::value;
      issue_part(next, kt + 1, part_tag);
#pragma unroll
      for (int i = 0; i < TM; i++)
#pragma unroll
        for (int j = 0; j < TN; j++)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[P][i], fb[P][j], acc[i][j], 0, 0, 0);
    };
    [&]<int... P>(std::integer_sequence<int, P...>) {
      (slice(std::integral_constant<int, P>{}), ...);
    }(std::make_integer_sequence<int, 4>{});
    __builtin_amdgcn_sched_barrier(0);
  };

  // prologue: step 0 into stage 0
  [&]<int... X>(std::integer_sequence<int, X...>) {
    (issue_one(std::integral_constant<int, 0>{}, 0, std::integral_constant<int, X>{}), ...);
  }(std::make_integer_sequence<int, kPerStep>{});
  for (int kt = 0; kt < nk; kt += 2) {
    step(std::integral_constant<int, 0>{}, kt);
    if (kt + 1 < nk) step(std::integral_constant<int, 1>{}, kt + 1);
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));   // the last (out-of-range) loads, before the LDS is released

  // accumulator r of fragment (i, j): row m = 8 (r / 4) + 4 (lane / 32) + r % 4,
  // column n = lane % 32 of the 32 x 32 block; 32 lanes store 128 bytes of a row
  float* __restrict__ C = a.C + split * a.split_c;
#pragma unroll
  for (int i = 0; i < TM; i++)
#pragma unroll
    for (int r = 0; r < 16; r++) {
      const int m = m0 + wm * (BM / WM) + 32 * i + 8 * (r / 4) + 4 * (lane / 32) + r % 4;
      if (m >= a.M) continue;
#pragma unroll
      for (int j = 0; j < TN; j++) {
        const int n = n0 + wn * (BN / WN) + 32 * j + (lane & 31);
        if (n < a.N) {
          float* c = C + (int64_t)m * a.N + n;
          *c = a.accumulate ? *c + acc[i][j][r] : acc[i][j][r];
        }
      }
    }
}

template <int BM, int BN, int WM, int WN>
hipError_t tn_launch(const GemmTnArgs& a, hipStream_t s) {
  const int64_t tiles = (int64_t)a.splits * ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  k_gemm_tn<BM, BN, WM, WN><<<(unsigned)tiles, 64 * WM * WN, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace

bool gemm_tn_fits(const GemmTnArgs& a) {
  // buffer offsets are 32-bit: a chunk's rows of either operand stay below 2 GB
  return a.Ks > 0 && a.Ks % kBK == 0 && a.lda % 8 == 0 && a.ldb % 8 == 0 && a.lda >= a.M && a.ldb >= a.N &&
         a.Ks * std::max(a.lda, a.ldb) * 2 < ((int64_t)1 << 31) && a.splits >= 1 &&
         (int64_t)a.splits * a.Ks >= a.K && a.K / a.Ks < ((int64_t)1 << 16);
}

hipError_t launch_gemm_tn_bf16_f32out(const GemmTnArgs& a, hipStream_t s) {
  if (a.M == 0 || a.N == 0) return hipSuccess;
  if (!gemm_tn_fits(a) || ((uintptr_t)a.A & 15) || ((uintptr_t)a.B & 15)) return hipErrorInvalidValue;
  // 256 x 256 tiles once they fill the chip twice over (fewer L2 requests per flop)
  if ((int64_t)a.splits * ((a.M + 255) / 256) * ((a.N + 255) / 256) >= 2 * 256)
    return tn_launch<256, 256, 4, 2>(a, s);
  return tn_launch<128, 128, 2, 2>(a, s);
}

}  // namespace engram
