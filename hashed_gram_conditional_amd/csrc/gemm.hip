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
// Tiling: 128 tokens x 128 channels per 256-thread workgroup (2x2 waves of
// 64x64, each a 2x2 grid of 32x32 MFMA tiles), K step 64, double-buffered LDS
// (64 KB) with one barrier per K step.  LDS rows are 128 bytes; the 16-byte
// piece c of row r is stored at piece c ^ ((r >> 1) & 7), so the 16 lanes of a
// ds_read_b128 phase (16 rows, same logical piece) hit 16 distinct bank groups.
#include "engram_internal.h"

namespace engram {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BM = 128;  // tokens per tile
constexpr int BN = 128;  // output channels per tile
constexpr int BK = 64;   // reduction step
constexpr int kThreads = 256;
constexpr int kPieces = BK / 8;  // 16-byte pieces per LDS row

__device__ __forceinline__ int swz(int row, int piece) { return piece ^ ((row >> 1) & 7); }

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

__global__ void __launch_bounds__(kThreads, 2) k_gemm_bf16(GemmArgs a) {
  __shared__ uint4 sA[2][BM * kPieces];  // e tile
  __shared__ uint4 sB[2][BN * kPieces];  // weight tile

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave & 1;   // token half of the tile
  const int wn = wave >> 1;  // channel half of the tile
  const int64_t m0 = (int64_t)blockIdx.y * BM;
  const int64_t n0 = (int64_t)blockIdx.x * BN;
  const uint16_t* __restrict__ A = (const uint16_t*)a.A;
  const uint16_t* __restrict__ B = (const uint16_t*)a.B;
  const int K = a.K;
  const int nk = (K + BK - 1) / BK;

  // global -> register staging: 4 pieces of A and 4 of B per thread per K step
  uint4 ra[4], rb[4];
  auto load_tile = [&](int kt) {
    const int k0 = kt * BK;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int c = tid + i * kThreads;
      const int row = c >> 3, piece = c & 7;
      const int k = k0 + piece * 8;
      const int64_t m = m0 + row, n = n0 + row;
      ra[i] = (m < a.M && k < K) ? *(const uint4*)(A + m * K + k) : make_uint4(0, 0, 0, 0);
      rb[i] = (n < a.N && k < K) ? *(const uint4*)(B + n * K + k) : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int c = tid + i * kThreads;
      const int row = c >> 3, piece = c & 7;
      sA[buf][row * kPieces + swz(row, piece)] = ra[i];
      sB[buf][row * kPieces + swz(row, piece)] = rb[i];
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; i++)
#pragma unroll
    for (int j = 0; j < 2; j++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[i][j][r] = 0.f;

  load_tile(0);
  store_tile(0);
  __syncthreads();

  const int lrow = lane & 31;
  const int lhalf = lane >> 5;
  for (int kt = 0; kt < nk; kt++) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load_tile(kt + 1);
#pragma unroll
    for (int kk = 0; kk < BK / 16; kk++) {
      const int piece = kk * 2 + lhalf;
      bf16x8 fa[2], fb[2];
#pragma unroll
      for (int i = 0; i < 2; i++) {
        const int r = wn * 64 + i * 32 + lrow;
        fa[i] = as_bf16x8(sB[buf][r * kPieces + swz(r, piece)]);
      }
#pragma unroll
      for (int j = 0; j < 2; j++) {
        const int r = wm * 64 + j * 32 + lrow;
        fb[j] = as_bf16x8(sA[buf][r * kPieces + swz(r, piece)]);
      }
#pragma unroll
      for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) store_tile(buf ^ 1);
    __syncthreads();
  }

  // epilogue: accumulator r of tile (i, j) is output channel
  // n0 + wn*64 + i*32 + 8*(r/4) + 4*(lane/32) + r%4 of token m0 + wm*64 + j*32 + lane%32
  uint16_t* __restrict__ C = (uint16_t*)a.C;
#pragma unroll
  for (int j = 0; j < 2; j++) {
    const int64_t m = m0 + wm * 64 + j * 32 + lrow;
    if (m >= a.M) continue;
#pragma unroll
    for (int i = 0; i < 2; i++) {
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const int64_t n = n0 + wn * 64 + i * 32 + 8 * q + 4 * lhalf;
        if (n >= a.N) continue;
        uint2 pk;
        pk.x = (uint32_t)f32_to_bf16(acc[i][j][4 * q + 0]) | ((uint32_t)f32_to_bf16(acc[i][j][4 * q + 1]) << 16);
        pk.y = (uint32_t)f32_to_bf16(acc[i][j][4 * q + 2]) | ((uint32_t)f32_to_bf16(acc[i][j][4 * q + 3]) << 16);
        *(uint2*)(C + m * a.N + n) = pk;
      }
    }
  }
}

// float32 path: a plain LDS-tiled FMA GEMM, 64x64 tile, 4x4 outputs per thread.
constexpr int FT = 64, FK = 16;

__global__ void __launch_bounds__(256) k_gemm_f32(GemmArgs a) {
  __shared__ float sA[FK][FT + 1];
  __shared__ float sB[FK][FT + 1];
  const float* __restrict__ A = (const float*)a.A;
  const float* __restrict__ B = (const float*)a.B;
  float* __restrict__ C = (float*)a.C;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int64_t m0 = (int64_t)blockIdx.y * FT, n0 = (int64_t)blockIdx.x * FT;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < a.K; k0 += FK) {
    for (int i = threadIdx.x; i < FT * FK; i += 256) {
      const int r = i / FK, kk = i % FK;
      const int64_t m = m0 + r, n = n0 + r;
      const int k = k0 + kk;
      sA[kk][r] = (m < a.M && k < a.K) ? A[m * a.K + k] : 0.f;
      sB[kk][r] = (n < a.N && k < a.K) ? B[n * a.K + k] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < FK; kk++)
#pragma unroll
      for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++) acc[i][j] = fmaf(sA[kk][ty * 4 + i], sB[kk][tx * 4 + j], acc[i][j]);
    __syncthreads();
  }
  for (int i = 0; i < 4; i++) {
    const int64_t m = m0 + ty * 4 + i;
    if (m >= a.M) continue;
    for (int j = 0; j < 4; j++) {
      const int64_t n = n0 + tx * 4 + j;
      if (n < a.N) C[m * a.N + n] = acc[i][j];
    }
  }
}

}  // namespace

hipError_t launch_gemm_bf16(const GemmArgs& a, hipStream_t s) {
  if (a.M == 0 || a.N == 0) return hipSuccess;
  dim3 grid((a.N + BN - 1) / BN, (a.M + BM - 1) / BM);
  k_gemm_bf16<<<grid, kThreads, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_gemm_f32(const GemmArgs& a, hipStream_t s) {
  if (a.M == 0 || a.N == 0) return hipSuccess;
  dim3 grid((a.N + FT - 1) / FT, (a.M + FT - 1) / FT);
  k_gemm_f32<<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace engram
