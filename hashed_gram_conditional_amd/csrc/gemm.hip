// K2: key projections of every branch and the shared value projection
// (formula sheet, kwkr.cn/news/37585, section 2.2 steps 1 and 3; architecture
// walk-through, yaoyuxiang.cn/news/830577, section 2.2-4: one key projection
// per branch, one value projection shared by all), computed as one GEMM
//   kv[m][n] = sum_k e[m][k] * w_kv[n][k]
// over the concatenated weight [W_k,0; ...; W_k,hc-1; W_v].  It is the only
// dense contraction of the forward pass.
//
// bf16 path: v_mfma_f32_32x32x16_bf16 with float32 accumulation.  Both
// operands are K-contiguous, so an MFMA fragment (8 consecutive k of one row)
// is one 16-byte LDS read.  The MFMA "A" operand is the weight tile and the
// "B" operand the e tile, so each lane's accumulators hold 4 runs of 4
// consecutive output channels of one token and the epilogue stores 8 bytes at
// a time along the contiguous channel axis.
//
// Tiling: 256 tokens x 256 channels per workgroup of 8 waves (4 x 2, two per
// SIMD, 64 x 128 per wave) for large shapes, 128 x 128 per workgroup of 4
// waves for small ones, K step 64, two LDS stages filled by DMA.  LDS rows are
// 128 bytes; the 16-byte piece c of row r is stored at piece c ^ ((r >> 1) & 7),
// so the 16 lanes of a ds_read_b128 phase (16 rows, same logical piece) hit 16
// distinct bank groups.
#include <type_traits>
#include <utility>

#include <algorithm>

#include "gemm_common.h"

namespace engram {
namespace {

#ifndef ENGRAM_GEMM_BK
#define ENGRAM_GEMM_BK 64
#endif
constexpr int BK = ENGRAM_GEMM_BK;           // reduction step (bf16 elements)
constexpr int kPieces = BK / 8;              // 16-byte pieces per LDS row
constexpr int kRowsPerDma = 64 / kPieces;    // rows one 1 KB DMA instruction fills

// Physical 16-byte piece of logical piece `piece` in LDS row `row`.  LDS reads
// are served 256 bytes (64 banks) at a time, i.e. 16 lanes of a ds_read_b128;
// those lanes read 16 consecutive rows at the same logical piece, and the XOR
// spreads them over 16 distinct 16-byte bank groups (0 bank conflicts
// measured with SQ_LDS_BANK_CONFLICT).
__device__ __forceinline__ int swz(int row, int piece) {
  if constexpr (kPieces == 8) return piece ^ ((row >> 1) & 7);   // 128-byte rows: 2 rows per bank line
  else return piece ^ ((row >> 2) & 3);                          // 64-byte rows: 4 rows per bank line
}

// Buffer resource over rows [row0, row0 + rows) of a K-contiguous bf16 matrix:
// loads past the last valid row, or at an offset marked out of range, return
// zero, so ragged tiles and the K tail need no branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint16_t* base, int64_t row0, int64_t rows, int K) {
  const int64_t bytes = rows * (int64_t)K * 2;
  return __builtin_amdgcn_make_buffer_rsrc((void*)(base + row0 * K), (short)0, (int)(bytes > 0 ? bytes : 0),
                                           0x00020000);
}

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// 4 consecutive bf16 of a row as floats
__device__ __forceinline__ void load4(const uint16_t* p, float* v) {
  const uint2 u = *(const uint2*)p;
  v[0] = __uint_as_float(u.x << 16);
  v[1] = __uint_as_float(u.x & 0xFFFF0000u);
  v[2] = __uint_as_float(u.y << 16);
  v[3] = __uint_as_float(u.y & 0xFFFF0000u);
}

// BM tokens x BN channels per workgroup of WM x WN waves; each wave owns
// (BM/WM) x (BN/WN) as a grid of 32x32 MFMA tiles.  MFMA A = weight rows
// (channels), B = e rows (tokens), so accumulator r of tile (i, j) is channel
//   n0 + wn*BN/WN + 32 i + 8 (r/4) + 4 (lane/32) + r%4   of token   m0 + wm*BM/WM + 32 j + lane%32.
//
// Operands move global -> LDS by buffer_load_dwordx4 ... lds (no staging
// registers): one instruction of one wave fills 1 KB of LDS in lane order, so
// each lane fetches the global piece whose swizzled LDS slot is its own.  A
// ring of kStages LDS stages keeps kStages-1 K steps of loads in flight; every
// step issues exactly one more step of loads (past the end: out-of-range loads
// that only write zeros into a stage nobody reads again) so the wait before
// each step is one constant vmcnt, followed by a barrier that makes the other
// waves' loads visible.  The K steps are padded to a multiple of kStages with
// all-zero steps and the loop is unrolled over the ring, so every stage index
// is a constant and the compiler can tell the stage being filled from the one
// being read (it then inserts no wait of its own between them).  Within a step
// the fragments of slice kk+1 are read, and (in the first half of the step)
// half of the next step's loads issued, while the MFMAs of slice kk run.  With 8 waves (2 per SIMD)
// one wave's loads and barrier overlap the other wave's MFMAs.
//
// GATE = false: the tile is stored to C (bf16).
// STORE_K (with GATE): key tiles are also stored, to k_out (the gradients read them).
// GATE = true (fused gate): a tile of branch h's key channels is not stored;
// its epilogue reads the matching tile of the hidden state Q (the query of
// branch h) and the two RMSNorm scales, and writes per token and 128 channels
// the partial sums of K^2, Q^2 and K gk gq Q -- everything the gate needs
// from K (formula sheet, kwkr.cn/news/37585, section 2.2 step 1: the gate is
// the scaled dot of RMSNorm(K) and RMSNorm(Q), and RMSNorm only needs the mean
// square).  Value tiles are stored to v_out.  Writing K and reading it back
// is the largest traffic of the unfused path.
template <int BM, int BN, int WM, int WN, int kStages, bool GATE, bool F32OUT = false, bool STORE_K = false>
__global__ void __launch_bounds__(64 * WM * WN, 1) k_gemm_bf16(GemmGateArgs ga) {
  constexpr int NW = WM * WN;                          // waves
  constexpr int TM = BM / WM / 32, TN = BN / WN / 32;  // MFMA tiles per wave along tokens / channels
  constexpr int QA = BM / (NW * kRowsPerDma);          // DMA instructions per wave per K step
  constexpr int QB = BN / (NW * kRowsPerDma);
  constexpr int kPerStep = QA + QB;
  constexpr int KK = BK / 16;                          // MFMA k slices per step
  // Fused gate: the first PJ token blocks of the wave's Q tile (TN*16 values per
  // lane each) are loaded into registers before the first operand loads, so
  // they arrive under the K loop instead of in the epilogue -- the first
  // kPreI channel blocks of them, as many as the register budget left by the
  // K loop holds without spilling (24 VGPRs with 8 waves, 32 with 4).  (The
  // first step's vmcnt wait also covers these loads; they travel with the
  // prologue's operand loads.)
  constexpr int PJ = GATE ? (TM < 4 / TN ? TM : 4 / TN) : 0;
  constexpr bool kPreloadQ = PJ > 0;
  constexpr int kPreI = kPreloadQ ? ((NW >= 8 ? 24 : 32) / (8 * PJ) < TN ? (NW >= 8 ? 24 : 32) / (8 * PJ) : TN) : 1;
  // one LDS block of kStages stages, each an e tile then a weight tile; after
  // the K loop it holds the output tile on its way to memory.  The fused gate
  // adds, past the stages, the tile's gamma_k and gamma_q (1 KB each) and per
  // wave the Q pieces that are neither preloaded into registers nor brought in
  // by the last refill (token blocks j < PJ, channel blocks i >= kPreI); both
  // are loaded by DMA before the first operand step and read in the epilogue.
  constexpr int kStageElems = (BM + BN) * kPieces;
  constexpr int kGammaElems = GATE ? 128 : 0;
  constexpr bool kQ4 = GATE && PJ > 0 && kPreI < TN;
  constexpr int QP4 = (TN - kPreI) * 4;            // 16-byte pieces per row of those channel blocks
  constexpr int kQ4Elems = kQ4 ? PJ * 32 * QP4 : 0;
  static_assert(kQ4Elems % 64 == 0, "whole DMA instructions");
  constexpr int kGammaBase = kStages * kStageElems, kQ4Base = kGammaBase + kGammaElems;
  __shared__ u32x4 smem[kStages * kStageElems + kGammaElems + NW * kQ4Elems];
  static_assert(BM * BN * 2 <= kStages * kStageElems * 16, "output tile fits in the operand stages");
  const GemmArgs& a = ga.g;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: DMA LDS addresses stay scalar
  const int wm = wave % WM, wn = wave / WM;
  const int m_tiles = (a.M + BM - 1) / BM, n_tiles = (a.N + BN - 1) / BN;
  // split-K batches are stacked along M in the tile order
  int mt, nt;
  tile_of(blockIdx.x, a.splits * m_tiles, n_tiles, mt, nt);
  const int split = mt / m_tiles;
  mt -= split * m_tiles;
  const int64_t m0 = (int64_t)mt * BM, n0 = (int64_t)nt * BN;
  const int K = a.K;
  const int nk = (K + BK - 1) / BK;
  const int nk_pad = (nk + kStages - 1) / kStages * kStages;
  const __amdgpu_buffer_rsrc_t rA =
      tile_rsrc((const uint16_t*)a.A + split * a.split_a, m0, min((int64_t)BM, a.M - m0), K);
  const __amdgpu_buffer_rsrc_t rB =
      tile_rsrc((const uint16_t*)a.B + split * a.split_b, n0, min((int64_t)BN, a.N - n0), K);
  const int row_bytes = K * 2;

  // this lane's slot in the block of rows one DMA instruction fills: tile row
  // (q*NW + wave)*kRowsPerDma + drow for instruction q; the q term moves the
  // row by a multiple of 32, which leaves the swizzle unchanged
  static_assert((NW * kRowsPerDma) % 32 == 0, "swizzle period");
  const int drow = wave * kRowsPerDma + lane / kPieces;
  const int dlog = swz(drow, lane % kPieces);          // logical piece it fetches (swz is its own inverse)
  const int dvoff = drow * row_bytes + dlog * 16;

  // instruction x of one step's loads: x < QA fills e rows, the rest weight rows
  auto issue_one = [&](auto stage_tag, int voff, auto x_tag) {
    constexpr int S = decltype(stage_tag)::value;
    constexpr int X = decltype(x_tag)::value;
    if constexpr (X < QA)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, LDS_PTR(&smem[S * kStageElems + (X * NW + wave) * 64]), 16, voff,
                                               X * NW * kRowsPerDma * row_bytes, 0, 0);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rB, LDS_PTR(&smem[S * kStageElems + BM * kPieces + ((X - QA) * NW + wave) * 64]),
                                               16, voff,
                                               (X - QA) * NW * kRowsPerDma * row_bytes, 0, 0);
  };
  auto step_voff = [&](int kt) {
    return (kt < nk && kt * BK + dlog * 8 < K) ? dvoff + kt * BK * 2 : kOutOfRange;
  };
  // With two stages a step's loads go out over the first half of its slices:
  // slice P < KK/2 issues loads [P*kPerStep/(KK/2), (P+1)*kPerStep/(KK/2))
  // into stage S.  Spread over all four slices, the last quarter had almost
  // no time to land before the next step's wait; all in the first slice, they
  // queued behind its fragment reads (measured on MI355X, 32768 x 20480 x
  // 1920: 2393 / 2301 / 2216 us for four / one / two slices).  With four
  // stages the loads have three steps to land and go out over all four slices
  // (256 x 12800 x 1024 with the gate: 14.6 -> 14.1 us).
  constexpr int kDmaSlices = kStages > 2 ? KK : (KK / 2 > 0 ? KK / 2 : 1);
  auto issue_part = [&](auto stage_tag, int voff, auto part_tag) {
    constexpr int P = decltype(part_tag)::value;
    constexpr int lo = P < kDmaSlices ? P * kPerStep / kDmaSlices : kPerStep;
    constexpr int hi = P < kDmaSlices ? (P + 1) * kPerStep / kDmaSlices : kPerStep;
    [&]<int... X>(std::integer_sequence<int, X...>) {
      (issue_one(stage_tag, voff, std::integral_constant<int, lo + X>{}), ...);
    }(std::make_integer_sequence<int, hi - lo>{});
  };

  f32x16 acc[TN][TM];
#pragma unroll
  for (int i = 0; i < TN; i++)
#pragma unroll
    for (int j = 0; j < TM; j++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[i][j][r] = 0.f;

  const int lrow = lane & 31;
  const int lhalf = lane >> 5;
  // fragments of one 16-wide k slice: TN weight fragments, TM e fragments
  auto load_frags = [&](auto stage_tag, int kk, bf16x8* fa, bf16x8* fb) {
    constexpr int S = decltype(stage_tag)::value;
    const int piece = kk * 2 + lhalf;
#pragma unroll
    for (int i = 0; i < TN; i++) {
      const int r = wn * (BN / WN) + i * 32 + lrow;
      fa[i] = __builtin_bit_cast(bf16x8, smem[S * kStageElems + BM * kPieces + r * kPieces + swz(r, piece)]);
    }
#pragma unroll
    for (int j = 0; j < TM; j++) {
      const int r = wm * (BM / WM) + j * 32 + lrow;
      fb[j] = __builtin_bit_cast(bf16x8, smem[S * kStageElems + r * kPieces + swz(r, piece)]);
    }
  };
  auto mfmas = [&](const bf16x8* fa, const bf16x8* fb) {
#pragma unroll
    for (int i = 0; i < TN; i++)
#pragma unroll
      for (int j = 0; j < TM; j++)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
  };
  // The remaining token blocks of the Q tile come through LDS: the last K
  // step's refill (which would only write zeros) loads them instead, 16 bytes
  // per lane and whole 256-byte row runs per 16 lanes, into the stage no wave
  // reads any more; each wave gets a private region of kQRows rows x QP
  // pieces, piece c of row r stored at piece c ^ (r % QP).
  constexpr int QP = (BN / WN) / 8;           // 16-byte pieces of one wave's channel span
  constexpr int kQRows = (TM - PJ) * 32;
  constexpr int kQElems = kQRows * QP;        // u32x4 per wave region
  constexpr int kQStage = (kStages + kStages - 2) % kStages;   // the stage the last step refills
  // (taken when the regions are exactly one step's refill; otherwise those
  // token blocks are read from memory in the epilogue)
  constexpr bool kQInLds = GATE && PJ < TM && kQElems == kPerStep * 64 && NW * kQElems <= kStageElems;
  const bool key_tile = GATE && (int)(n0 / ga.d) < ga.hc;
  const int gate_h = GATE ? (int)(n0 / ga.d) : 0;
  const int gate_cw = GATE ? (int)(n0 - (int64_t)gate_h * ga.d) + wn * (BN / WN) + 4 * lhalf : 0;  // + 32 i + 8 q
  auto q_row = [&](int j) {
    // rows past M: any valid row, its sums are discarded
    const int64_t m = min(m0 + wm * (BM / WM) + j * 32 + lrow, (int64_t)a.M - 1);
    return (const uint16_t*)ga.hidden + (m * ga.hc + gate_h) * (int64_t)ga.d + gate_cw;
  };
  const int gate_c0 = GATE ? (int)(n0 - (int64_t)gate_h * ga.d) : 0;   // first channel of the tile in its branch
  const __amdgpu_buffer_rsrc_t rQ = [&] {
    // Q rows of the tile's tokens, branch gate_h; loads past the last token read zero
    const int64_t rows = min((int64_t)BM, a.M - m0);
    const bool use = (kQInLds || kQ4) && key_tile;
    const int64_t bytes = use ? (rows * ga.hc - gate_h) * (int64_t)ga.d * 2 : 0;
    const uint16_t* base = (const uint16_t*)ga.hidden + (use ? (m0 * ga.hc + gate_h) * (int64_t)ga.d : 0);
    return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)bytes, 0x00020000);
  }();
  auto issue_q_one = [&](auto x_tag) {
    constexpr int X = decltype(x_tag)::value;
    const int pi = X * 64 + lane;
    const int r = pi / QP, c = (pi % QP) ^ (r % QP);
    const int tok = wm * (BM / WM) + 32 * (PJ + r / 32) + r % 32;
    const int voff = (tok * ga.hc * ga.d + gate_c0 + wn * (BN / WN) + c * 8) * 2;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rQ, LDS_PTR(&smem[kQStage * kStageElems + wave * kQElems + X * 64]), 16,
                                             voff, 0, 0, 0);
  };
  auto issue_q_part = [&](auto part_tag) {
    constexpr int P = decltype(part_tag)::value;
    constexpr int lo = P < kDmaSlices ? P * kPerStep / kDmaSlices : kPerStep;
    constexpr int hi = P < kDmaSlices ? (P + 1) * kPerStep / kDmaSlices : kPerStep;
    [&]<int... X>(std::integer_sequence<int, X...>) {
      (issue_q_one(std::integral_constant<int, lo + X>{}), ...);
    }(std::make_integer_sequence<int, hi - lo>{});
  };

  // One K step; sched_barrier keeps the scheduler from regrouping the reads
  // and loads of a slice with their uses.
  auto step = [&](auto stage_tag, int kt) {
    constexpr int S = decltype(stage_tag)::value;
    constexpr std::integral_constant<int, (S + kStages - 1) % kStages> next{};
    // at most kStages-2 steps of this wave's loads may remain: step kt has landed
    __builtin_amdgcn_s_waitcnt(vmcnt_imm((kStages - 2) * kPerStep));
    __builtin_amdgcn_s_barrier();
    const int voff = step_voff(kt + kStages - 1);
    const bool q_refill = kQInLds && S == kStages - 1 && key_tile && kt + 1 == nk_pad;
    bf16x8 fa[2][TN], fb[2][TM];
    load_frags(stage_tag, 0, fa[0], fb[0]);
    // the stage being refilled was read by every wave before the barrier
    auto slice = [&](auto part_tag) {
      constexpr int P = decltype(part_tag)::value;
      if constexpr (P + 1 < KK) load_frags(stage_tag, P + 1, fa[(P + 1) & 1], fb[(P + 1) & 1]);
      if constexpr (kQInLds && S == kStages - 1) {
        if (q_refill) issue_q_part(part_tag);
        else issue_part(next, voff, part_tag);
      } else {
        issue_part(next, voff, part_tag);
      }
      __builtin_amdgcn_sched_barrier(0);
      mfmas(fa[P & 1], fb[P & 1]);
      __builtin_amdgcn_sched_barrier(0);
    };
    [&]<int... P>(std::integer_sequence<int, P...>) {
      (slice(std::integral_constant<int, P>{}), ...);
    }(std::make_integer_sequence<int, KK>{});
  };

  uint2 qpre[kPreI][4][kPreloadQ ? PJ : 1];
  if constexpr (kPreloadQ) {
    if (key_tile) {
#pragma unroll
      for (int j = 0; j < PJ; j++) {
        const uint16_t* qr = q_row(j);
#pragma unroll
        for (int i = 0; i < kPreI; i++)
#pragma unroll
          for (int q = 0; q < 4; q++) qpre[i][q][j] = *(const uint2*)(qr + 32 * i + 8 * q);
      }
    }
  }

  if constexpr (GATE) {
    // gamma_k and gamma_q of the tile's channels (value tiles: zeros)
    if (wave == 0) {
      const int64_t goff = key_tile ? (int64_t)gate_h * ga.d + gate_c0 : 0;
      const int gbytes = key_tile ? BN * 2 : 0;
      const int gv = lane < BN / 8 ? lane * 16 : kOutOfRange;
      const __amdgpu_buffer_rsrc_t rgk =
          __builtin_amdgcn_make_buffer_rsrc((void*)((const uint16_t*)ga.gamma_k + goff), (short)0, gbytes, 0x00020000);
      const __amdgpu_buffer_rsrc_t rgq =
          __builtin_amdgcn_make_buffer_rsrc((void*)((const uint16_t*)ga.gamma_q + goff), (short)0, gbytes, 0x00020000);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rgk, LDS_PTR(&smem[kGammaBase]), 16, gv, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rgq, LDS_PTR(&smem[kGammaBase + 64]), 16, gv, 0, 0, 0);
    }
  }
  if constexpr (kQ4) {
    // piece c of row r of this wave's region at piece c ^ ((r / 4) % QP4)
    [&]<int... X>(std::integer_sequence<int, X...>) {
      ([&] {
        const int pi = X * 64 + lane;
        const int r = pi / QP4, c = (pi % QP4) ^ ((r / 4) % QP4);
        const int tok = wm * (BM / WM) + 32 * (r / 32) + r % 32;
        const int voff = (tok * ga.hc * ga.d + gate_c0 + wn * (BN / WN) + kPreI * 32 + c * 8) * 2;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rQ, LDS_PTR(&smem[kQ4Base + wave * kQ4Elems + X * 64]), 16, voff,
                                                 0, 0, 0);
      }(), ...);
    }(std::make_integer_sequence<int, kQ4Elems / 64>{});
  }

  // prologue: steps 0 .. kStages-2 in flight
  auto issue_all = [&](auto stage_tag) {
    constexpr int S = decltype(stage_tag)::value;
    const int voff = step_voff(S);
    [&]<int... X>(std::integer_sequence<int, X...>) {
      (issue_one(stage_tag, voff, std::integral_constant<int, X>{}), ...);
    }(std::make_integer_sequence<int, kPerStep>{});
  };
  [&]<int... I>(std::integer_sequence<int, I...>) {
    (issue_all(std::integral_constant<int, I>{}), ...);
  }(std::make_integer_sequence<int, kStages - 1>{});
  // a plain GEMM that follows the fused key projection forms the gates from
  // its partial sums while the first operand steps are in flight; the loop
  // bound depends on the workgroup only, so each 8-lane group stays whole
  if constexpr (!GATE && !F32OUT) {
    const GateFinalizeArgs& f = ga.fin;
    if (f.partials != nullptr) {
      constexpr int kGroups = 64 * NW / 8;
      const int64_t n = (int64_t)f.n_tok * f.hc;
      for (int64_t i0 = (int64_t)blockIdx.x * kGroups; i0 < n; i0 += (int64_t)gridDim.x * kGroups) {
        const int64_t i = i0 + tid / 8;
        const bool ok = i < n;
        float4 st;
        const float g = gate_from_partials8(f.partials + (ok ? i : 0) * f.n_part, f.n_part, ok, f.d, f.eps, f.clamp,
                                            f.inv_sqrt_d, &st);
        if (ok && (tid & 7) == 0) {
          f.g_out[i] = g;
          if (f.stats) f.stats[i] = st;
        }
      }
    }
  }
  for (int kt = 0; kt < nk_pad; kt += kStages) {
    [&]<int... I>(std::integer_sequence<int, I...>) {
      (step(std::integral_constant<int, I>{}, kt + I), ...);
    }(std::make_integer_sequence<int, kStages>{});
  }
  // drain the trailing out-of-range loads before the workgroup's LDS is reused or released
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));

  // Store of a tile through LDS: the accumulators go to an LDS copy of the
  // bf16 tile (16-byte piece c of row r at piece c ^ (r % RP)), then each
  // lane stores one 16-byte piece, so a wave writes whole rows.
  auto store_tile = [&](uint16_t* __restrict__ C, int64_t ldc, int64_t col0, int64_t ncols) {
    constexpr int RP = BN / 8;        // 16-byte pieces per tile row
    constexpr int RPI = 64 / RP;      // tile rows per wave instruction
    static_assert(BM % (NW * RPI) == 0, "whole store rounds");
    uint16_t* t = reinterpret_cast<uint16_t*>(&smem[0]);
    __syncthreads();                  // every wave is done with the operand stages
#pragma unroll
    for (int j = 0; j < TM; j++) {
      const int row = wm * (BM / WM) + j * 32 + lrow;
#pragma unroll
      for (int i = 0; i < TN; i++)
#pragma unroll
        for (int q = 0; q < 4; q++) {
          const int pc = (wn * (BN / WN) + i * 32 + 8 * q) / 8;
          const bf16x4 v = {(__bf16)acc[i][j][4 * q + 0], (__bf16)acc[i][j][4 * q + 1],
                            (__bf16)acc[i][j][4 * q + 2], (__bf16)acc[i][j][4 * q + 3]};
          *(bf16x4*)(t + row * BN + (pc ^ (row % RP)) * 8 + 4 * lhalf) = v;
        }
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < BM / (NW * RPI); it++) {
      const int row = (it * NW + wave) * RPI + lane / RP, pc = lane % RP;
      const int64_t m = m0 + row, n = col0 + pc * 8;
      const u32x4 v = *(const u32x4*)(t + row * BN + (pc ^ (row % RP)) * 8);
      if (m < a.M && n < ncols) *(u32x4*)(C + m * ldc + n) = v;
    }
  };

  if constexpr (F32OUT) {
    // float32 result (gradients): 4 consecutive columns per lane, stored or added
    float* __restrict__ C = (float*)a.C + split * a.split_c;
#pragma unroll
    for (int j = 0; j < TM; j++) {
      const int64_t m = m0 + wm * (BM / WM) + j * 32 + lrow;
      if (m >= a.M) continue;
#pragma unroll
      for (int i = 0; i < TN; i++)
#pragma unroll
        for (int q = 0; q < 4; q++) {
          const int64_t n = n0 + wn * (BN / WN) + i * 32 + 8 * q + 4 * lhalf;
#pragma unroll
          for (int e = 0; e < 4; e++)
            if (n + e < a.N) {
              float* c = C + m * a.N + n + e;
              *c = a.accumulate ? *c + acc[i][j][4 * q + e] : acc[i][j][4 * q + e];
            }
        }
    }
  } else if constexpr (!GATE) {
    store_tile((uint16_t*)a.C, a.ldc ? a.ldc : a.N, n0, a.N);
  } else {
    const int d = ga.d, hc = ga.hc;
    const int h = (int)(n0 / d);
    if (h >= hc) {  // value tile
      store_tile((uint16_t*)ga.v_out, ga.v_ld ? ga.v_ld : d, n0 - (int64_t)hc * d, d);
      return;
    }
    // key tile of branch h: channels c0 .. c0+BN-1 of the branch
    const int c0 = (int)(n0 - (int64_t)h * d);
    const uint16_t* gks = reinterpret_cast<const uint16_t*>(&smem[kGammaBase]) + wn * (BN / WN) + 4 * lhalf;
    const uint16_t* gqs = reinterpret_cast<const uint16_t*>(&smem[kGammaBase + 64]) + wn * (BN / WN) + 4 * lhalf;
    // Partial sums are per 128 channels, whatever the tile: a wave of a
    // 128-wide tile covers 64 channels and the two waves of a row add theirs
    // in LDS; a wave of a 256-wide tile covers 128 channels, kept as two
    // 64-channel sums (kHalves) added once.  Either way each 128-channel sum is
    // (sum of the first 64) + (sum of the next 64), every term in the same
    // order, so the gates do not depend on the tile the call was planned with.
    constexpr int kHalves = BN / WN == 128 ? 2 : 1;
    static_assert(BN / WN == 128 || BN / WN == 64, "fused gate epilogue: 64 or 128 channels per wave");
    const uint16_t* q_rows[TM];
    float kk[kHalves][TM], qq[kHalves][TM], kq[kHalves][TM];
#pragma unroll
    for (int j = 0; j < TM; j++) {
      q_rows[j] = q_row(j);
#pragma unroll
      for (int hf = 0; hf < kHalves; hf++) kk[hf][j] = qq[hf][j] = kq[hf][j] = 0.f;
    }
    // per token: sums over this lane's runs of 4 channels
#pragma unroll
    for (int i = 0; i < TN; i++)
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const int hf = kHalves == 2 && i >= TN / 2 ? 1 : 0;
        float x[4], y[4], g[4];
        load4(gks + 32 * i + 8 * q, x);
        load4(gqs + 32 * i + 8 * q, y);
#pragma unroll
        for (int e = 0; e < 4; e++) g[e] = x[e] * y[e];
#pragma unroll
        for (int j = 0; j < TM; j++) {
          float qv[4];
          if (j < PJ && i < kPreI) {
            const uint2 u = qpre[i < kPreI ? i : 0][q][j < PJ ? j : 0];
            qv[0] = __uint_as_float(u.x << 16);
            qv[1] = __uint_as_float(u.x & 0xFFFF0000u);
            qv[2] = __uint_as_float(u.y << 16);
            qv[3] = __uint_as_float(u.y & 0xFFFF0000u);
          } else if (kQ4 && j < PJ) {
            const int r = j * 32 + lrow;
            const uint16_t* qs = reinterpret_cast<const uint16_t*>(&smem[kQ4Base + wave * kQ4Elems]);
            const uint2 u = *(const uint2*)(qs + (r * QP4 + (((i - kPreI) * 4 + q) ^ ((r / 4) % QP4))) * 8 + 4 * lhalf);
            qv[0] = __uint_as_float(u.x << 16);
            qv[1] = __uint_as_float(u.x & 0xFFFF0000u);
            qv[2] = __uint_as_float(u.y << 16);
            qv[3] = __uint_as_float(u.y & 0xFFFF0000u);
          } else if (kQInLds && j >= PJ) {
            const int r = (j - PJ) * 32 + lrow;
            const uint16_t* qs = reinterpret_cast<const uint16_t*>(&smem[kQStage * kStageElems + wave * kQElems]);
            const uint2 u = *(const uint2*)(qs + r * QP * 8 + (((4 * i + q) ^ (r % QP)) * 8) + 4 * lhalf);
            qv[0] = __uint_as_float(u.x << 16);
            qv[1] = __uint_as_float(u.x & 0xFFFF0000u);
            qv[2] = __uint_as_float(u.y << 16);
            qv[3] = __uint_as_float(u.y & 0xFFFF0000u);
          } else {
            load4(q_rows[j] + 32 * i + 8 * q, qv);
          }
#pragma unroll
          for (int e = 0; e < 4; e++) {
            const float k = acc[i][j][4 * q + e];
            kk[hf][j] = fmaf(k, k, kk[hf][j]);
            qq[hf][j] = fmaf(qv[e], qv[e], qq[hf][j]);
            kq[hf][j] = fmaf(k * g[e], qv[e], kq[hf][j]);
          }
        }
      }
#pragma unroll
    for (int hf = 0; hf < kHalves; hf++)
#pragma unroll
      for (int j = 0; j < TM; j++) {
        // lanes l and l+32 hold the other half of each 8-channel run of the same token
        kk[hf][j] += __shfl_xor(kk[hf][j], 32, 64);
        qq[hf][j] += __shfl_xor(qq[hf][j], 32, 64);
        kq[hf][j] += __shfl_xor(kq[hf][j], 32, 64);
      }
    const int n_part = d / 128;
    if constexpr (kHalves == 2) {
      if (lhalf == 0) {
        const int part = (c0 + wn * 128) / 128;
#pragma unroll
        for (int j = 0; j < TM; j++) {
          const int64_t m = m0 + wm * (BM / WM) + j * 32 + lrow;
          if (m < a.M)
            ga.partials[(m * hc + h) * n_part + part] =
                make_float4(kk[0][j] + kk[1][j], qq[0][j] + qq[1][j], kq[0][j] + kq[1][j], 0.f);
        }
      }
      if constexpr (STORE_K) store_tile((uint16_t*)ga.k_out, ga.k_ld, n0, (int64_t)hc * d);
      return;
    }
    // the WN waves of a token row meet in LDS; the operand stages are free now
    __syncthreads();
    float4* red = reinterpret_cast<float4*>(&smem[0]);   // [wn][wm][j][lrow]
    if (lhalf == 0)
#pragma unroll
      for (int j = 0; j < TM; j++)
        red[((wn * WM + wm) * TM + j) * 32 + lrow] = make_float4(kk[0][j], qq[0][j], kq[0][j], 0.f);
    __syncthreads();
    if (wn == 0 && lhalf == 0) {
      const int part = c0 / 128;
#pragma unroll
      for (int j = 0; j < TM; j++) {
        const int64_t m = m0 + wm * (BM / WM) + j * 32 + lrow;
        if (m >= a.M) continue;
        float4 o = red[(wm * TM + j) * 32 + lrow];
#pragma unroll
        for (int w2 = 1; w2 < WN; w2++) {
          const float4 t = red[((w2 * WM + wm) * TM + j) * 32 + lrow];
          o.x += t.x;
          o.y += t.y;
          o.z += t.z;
        }
        ga.partials[(m * hc + h) * n_part + part] = o;
      }
    }
    if constexpr (STORE_K) store_tile((uint16_t*)ga.k_out, ga.k_ld, n0, (int64_t)hc * d);
  }
}

// g from the fused GEMM's partial sums: 8 lanes per (token, branch)
// (gate_from_partials8), consecutive lanes on consecutive 16-byte partials.
__global__ void __launch_bounds__(256) k_gate_finalize(GateFinalizeArgs a) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 3;
  const bool ok = i < (int64_t)a.n_tok * a.hc;
  float4 st;
  const float g = gate_from_partials8(a.partials + (ok ? i : 0) * a.n_part, a.n_part, ok, a.d, a.eps, a.clamp,
                                      a.inv_sqrt_d, &st);
  if (ok && (threadIdx.x & 7) == 0) {
    a.g_out[i] = g;
    if (a.stats) a.stats[i] = st;
  }
}

// float32 path: v_mfma_f32_32x32x2_f32 with float32 accumulation.  An FT x FT
// tile per workgroup of 4 waves (FT = 128: each wave 64x64 as 2x2 blocks of
// 32x32; FT = 64 for small products: one block per wave); K
// steps of 16 staged through two LDS buffers, stored k-major (a row of 128
// tile rows per k, padded by 32 floats so that the two k of an MFMA operand
// fall in different bank halves), with the next step's global loads in
// registers while the current one is multiplied.  As in the bf16 kernel the
// MFMA "A" operand is the weight rows and "B" the token rows: lane l supplies
// row l % 32 at k = l / 32 of each pair of k, and accumulator r holds channel
// 8 (r/4) + 4 (l/32) + r%4 of token l % 32 of its block.
constexpr int FK = 16;

template <int FT, bool VEC>
__global__ void __launch_bounds__(256) k_gemm_f32(GemmArgs a) {
  constexpr int FP = FT + 32, NB = FT / 64, H = FT * 4 / 256;
  __shared__ float sA[2][FK][FP];   // k x token rows
  __shared__ float sB[2][FK][FP];   // k x weight rows
  const float* __restrict__ A = (const float*)a.A;
  const float* __restrict__ B = (const float*)a.B;
  float* __restrict__ C = (float*)a.C;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int64_t m0 = (int64_t)blockIdx.y * FT, n0 = (int64_t)blockIdx.x * FT;
  const int row = lane & 31, kh = lane >> 5;
  const int K = a.K, nk = (K + FK - 1) / FK;
  // this thread's share of a step: H runs of 4 k of one row per operand
  // (float4 index x: row x / 4, k 4 (x % 4)), tid, tid + 256, ...
  float ra[H][4], rb[H][4];
  auto fetch = [&](int k0) {
#pragma unroll
    for (int h = 0; h < H; h++) {
      const int x = tid + 256 * h, r = x >> 2, k = k0 + 4 * (x & 3);
      const int64_t m = m0 + r, n = n0 + r;
      if constexpr (VEC) {
        const float4 va = (m < a.M && k < K) ? *(const float4*)(A + m * K + k) : make_float4(0.f, 0.f, 0.f, 0.f);
        const float4 vb = (n < a.N && k < K) ? *(const float4*)(B + n * K + k) : make_float4(0.f, 0.f, 0.f, 0.f);
        ra[h][0] = va.x, ra[h][1] = va.y, ra[h][2] = va.z, ra[h][3] = va.w;
        rb[h][0] = vb.x, rb[h][1] = vb.y, rb[h][2] = vb.z, rb[h][3] = vb.w;
      } else {
#pragma unroll
        for (int e = 0; e < 4; e++) {
          ra[h][e] = (m < a.M && k + e < K) ? A[m * K + k + e] : 0.f;
          rb[h][e] = (n < a.N && k + e < K) ? B[n * K + k + e] : 0.f;
        }
      }
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int h = 0; h < H; h++) {
      const int x = tid + 256 * h, r = x >> 2, k = 4 * (x & 3);
#pragma unroll
      for (int e = 0; e < 4; e++) {
        sA[buf][k + e][r] = ra[h][e];
        sB[buf][k + e][r] = rb[h][e];
      }
    }
  };
  f32x16 acc[NB][NB];
#pragma unroll
  for (int i = 0; i < NB; i++)
#pragma unroll
    for (int j = 0; j < NB; j++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[i][j][r] = 0.f;
  fetch(0);
  stash(0);
  __syncthreads();
  for (int kt = 0; kt < nk; kt++) {
    const int cur = kt & 1;
    if (kt + 1 < nk) fetch((kt + 1) * FK);
#pragma unroll
    for (int kk = 0; kk < FK; kk += 2) {
      float fa[NB], fb[NB];
#pragma unroll
      for (int i = 0; i < NB; i++) fa[i] = sB[cur][kk + kh][wn * (FT / 2) + i * 32 + row];
#pragma unroll
      for (int j = 0; j < NB; j++) fb[j] = sA[cur][kk + kh][wm * (FT / 2) + j * 32 + row];
#pragma unroll
      for (int i = 0; i < NB; i++)
#pragma unroll
        for (int j = 0; j < NB; j++)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) stash(cur ^ 1);
    __syncthreads();
  }
#pragma unroll
  for (int j = 0; j < NB; j++) {
    const int64_t m = m0 + wm * (FT / 2) + j * 32 + row;
    if (m >= a.M) continue;
#pragma unroll
    for (int i = 0; i < NB; i++)
#pragma unroll
      for (int q = 0; q < 4; q++)
#pragma unroll
        for (int e = 0; e < 4; e++) {
          const int64_t n = n0 + wn * (FT / 2) + i * 32 + 8 * q + 4 * kh + e;
          if (n < a.N) {
            float* c = C + m * a.N + n;
            *c = a.accumulate ? *c + acc[i][j][4 * q + e] : acc[i][j][4 * q + e];
          }
        }
  }
}

}  // namespace

template <int BM, int BN, int WM, int WN, int ST, bool GATE, bool F32OUT = false, bool STORE_K = false>
hipError_t gemm_launch(const GemmGateArgs& a, hipStream_t s) {
  const int64_t tiles = (int64_t)a.g.splits * ((a.g.M + BM - 1) / BM) * ((a.g.N + BN - 1) / BN);
  k_gemm_bf16<BM, BN, WM, WN, ST, GATE, F32OUT, STORE_K><<<(unsigned)tiles, 64 * WM * WN, 0, s>>>(a);
  return hipGetLastError();
}

// Tile choice (measured on MI355X over the workloads' shapes): 256x256 with
// 4x2 waves (2 per SIMD) once there are at least 4 such tiles per CU, else
// 128x128 with 2x2 waves, whose 64 KB of LDS (two stages) lets two workgroups
// share a CU -- or, when there are no more tiles than CUs (decode-sized
// token counts), four stages in 128 KB: one workgroup per CU either way, and
// three K steps of loads in flight instead of one.
static int pick_tile_n(int64_t M, int N) {
  const int64_t big = ((M + 255) / 256) * ((N + 255) / 256);
  return big >= 4 * 256 ? 256 : 128;
}
static bool few_tiles(int64_t M, int N) { return ((M + 127) / 128) * ((N + 127) / 128) <= 256; }

hipError_t launch_gemm_bf16(const GemmArgs& a, hipStream_t s, const GateFinalizeArgs* fin) {
  if (a.M == 0 || a.N == 0) return fin ? launch_gate_finalize(*fin, s) : hipSuccess;
  GemmGateArgs ga = {};
  ga.g = a;
  if (fin) ga.fin = *fin;
  if (pick_tile_n(a.M, a.N) == 256) return gemm_launch<256, 256, 4, 2, 2, false>(ga, s);
  if (few_tiles(a.M, a.N)) return gemm_launch<128, 128, 2, 2, 4, false>(ga, s);
  return gemm_launch<128, 128, 2, 2, 2, false>(ga, s);
}

int gemm_k_splits(int64_t M, int64_t N, int64_t K) {
  // A long K over few output tiles: with S splits the time goes as the rounds
  // of 256-wide tiles over 256 CUs, ceil(S tiles / 256), times K / S.  Take
  // the S <= 8 that minimises it (each split at least 4096 deep, and whole
  // 256 x 256 tiles at least twice the CUs), if it beats one split by 10%.
  const int64_t tiles = ((M + 255) / 256) * ((N + 255) / 256);
  int best = 1;
  double best_cost = (double)((tiles + 255) / 256);
  for (int S = 2; S <= 8; S++) {
    if (K / S < 4096 || S * tiles < 2 * 256) continue;
    const double cost = (double)((S * tiles + 255) / 256) / S;
    if (cost < 0.9 * best_cost) {
      best = S;
      best_cost = cost;
    }
  }
  return best;
}

hipError_t launch_gemm_bf16_f32out(const GemmArgs& a, hipStream_t s) {
  if (a.M == 0 || a.N == 0) return hipSuccess;
  GemmGateArgs ga = {};
  ga.g = a;
  // 256 x 256 tiles once they fill the chip twice over (fewer L2 requests per flop)
  if ((int64_t)a.splits * ((a.M + 255) / 256) * ((a.N + 255) / 256) >= 2 * 256)
    return gemm_launch<256, 256, 4, 2, 2, false, true>(ga, s);
  if (a.splits != 1) return hipErrorInvalidValue;
  if (few_tiles(a.M, a.N)) return gemm_launch<128, 128, 2, 2, 4, false, true>(ga, s);
  return gemm_launch<128, 128, 2, 2, 2, false, true>(ga, s);
}

// Plan of the fused projection over M tokens and (hc+1) d channels, from a
// model of its time in rounds of 256x256 tiles over the 256 CUs (a round of
// 128x128 tiles, two per CU, costs ~0.34 of one: they move twice the operand
// bytes per flop; measured on MI355X):
//   one launch of 256x256 tiles (d % 256 == 0):   ceil(tiles / 256)
//   one launch of 128x128 tiles (d % 128 == 0):   0.34 max(1, tiles / 256)
//   split (d % 256 == 0): the key channels in 256x256 tiles with the gate
//     epilogue, then the value channels as a plain GEMM in 128x128 tiles
// B=4 T=1024 d=1024 hc=4: 320 large tiles are 2 rounds, 1280 small ones 1.7,
// the split 1 + 0.34 (256 key tiles, then 256 value tiles).
GatePlan gemm_gate_plan(int64_t M, int hc, int d) {
  const int64_t mt256 = (M + 255) / 256, mt128 = (M + 127) / 128;
  const double small = 0.34;
  GatePlan best = {0, false};
  double cost = 1e30;
  if (d % 256 == 0) {
    const double c = (double)((mt256 * ((int64_t)(hc + 1) * d / 256) + 255) / 256);
    if (c < cost) best = {256, false}, cost = c;
  }
  if (d % 128 == 0) {
    const double c = small * std::max(1.0, (double)(mt128 * ((int64_t)(hc + 1) * d / 128)) / 256.0);
    if (c < cost) best = {128, false}, cost = c;
  }
  if (d % 256 == 0) {
    const double c = (double)((mt256 * ((int64_t)hc * d / 256) + 255) / 256) +
                     small * std::max(1.0, (double)(mt128 * (d / 128)) / 256.0);
    if (c < 0.9 * cost) best = {256, true}, cost = c;
  }
  return best;
}

hipError_t launch_gemm_gate_bf16(const GemmGateArgs& a, hipStream_t s) {
  if (a.g.M == 0 || a.g.N == 0) return hipSuccess;
  const int bn = a.tile_n;
  if (a.k_out != nullptr) {   // the keys stored as well (training)
    if (bn == 256) return gemm_launch<256, 256, 4, 2, 2, true, false, true>(a, s);
    if (bn == 128 && few_tiles(a.g.M, a.g.N)) return gemm_launch<128, 128, 2, 2, 4, true, false, true>(a, s);
    if (bn == 128) return gemm_launch<128, 128, 2, 2, 2, true, false, true>(a, s);
    return hipErrorInvalidValue;
  }
  if (bn == 256) return gemm_launch<256, 256, 4, 2, 2, true>(a, s);
  if (bn == 128 && few_tiles(a.g.M, a.g.N)) return gemm_launch<128, 128, 2, 2, 4, true>(a, s);
  if (bn == 128) return gemm_launch<128, 128, 2, 2, 2, true>(a, s);
  return hipErrorInvalidValue;
}

hipError_t launch_gate_finalize(const GateFinalizeArgs& a, hipStream_t s) {
  const int64_t n = (int64_t)a.n_tok * a.hc;
  if (n == 0) return hipSuccess;
  k_gate_finalize<<<(unsigned)((n * 8 + 255) / 256), 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_gemm_f32(const GemmArgs& a, hipStream_t s) {
  if (a.M == 0 || a.N == 0) return hipSuccess;
  // float4 loads need every row 16-byte aligned; 64-wide tiles while the
  // 128-wide ones would not give every CU one
  const bool vec = a.K % 4 == 0 && (uintptr_t)a.A % 16 == 0 && (uintptr_t)a.B % 16 == 0;
  const bool big = ((int64_t)(a.M + 127) / 128) * ((a.N + 127) / 128) >= 256;
  const dim3 grid64((a.N + 63) / 64, (a.M + 63) / 64), grid128((a.N + 127) / 128, (a.M + 127) / 128);
  if (big && vec) k_gemm_f32<128, true><<<grid128, 256, 0, s>>>(a);
  else if (big) k_gemm_f32<128, false><<<grid128, 256, 0, s>>>(a);
  else if (vec) k_gemm_f32<64, true><<<grid64, 256, 0, s>>>(a);
  else k_gemm_f32<64, false><<<grid64, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace engram
