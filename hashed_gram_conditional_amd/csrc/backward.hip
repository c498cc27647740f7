// Backward pass of the module (a training step; the walk-through,
// yaoyuxiang.cn/news/830577, section 4.4, trains the module).  The pages give
// the forward only; these kernels compute its exact derivatives:
//   conv + residual:  dVg[t] = dy[t] + sum_j w[j] dy[t + (K-1-j)D],
//                     dw[h][c][j] += sum_t dy[t][h][c] Vg[t - (K-1-j)D][h][c]
//   value fusion:     dV[t][c] = sum_h g dVg,  dg[t][h] = sum_c dVg V
//   gate:             ds = dg g (1-g) / (2 sqrt|s|) where |s| >= clamp and s != 0, else 0
//                     (sign(s) sqrt(max(|s|, clamp)) is flat in s inside the clamp)
//   score s = sum_c u v / sqrt(d), u = K rk gk, v = Q rq gq, rk = (mean K^2 + eps)^-1/2:
//                     du = ds v / sqrt(d),  dv = ds u / sqrt(d)
//                     dK = rk gk du - rk^3 K (sum du gk K) / d,  dgk += du K rk  (and Q alike)
// The projection and table gradients are GEMMs and a scatter-add, launched
// from the C ABI.  Accumulations across tokens (conv taps, gammas, table rows)
// use float32 atomics: their order, and so the last bits, vary between runs.
#include "engram_internal.h"

namespace engram {
namespace {

// 8 consecutive elements as floats
__device__ __forceinline__ void ld8(const void* p, int64_t i, bool bf16, float* v) {
  if (bf16) {
    const uint4 u = *(const uint4*)((const uint16_t*)p + i);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int k = 0; k < 4; k++) {
      v[2 * k] = __uint_as_float(w[k] << 16);
      v[2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
    }
  } else {
    const float4 a = *(const float4*)((const float*)p + i);
    const float4 b = *(const float4*)((const float*)p + i + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

__device__ __forceinline__ void st8(void* p, int64_t i, bool bf16, const float* v) {
  if (bf16) {
    uint4 u;
    u.x = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
    u.y = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
    u.z = (uint32_t)f32_to_bf16(v[4]) | ((uint32_t)f32_to_bf16(v[5]) << 16);
    u.w = (uint32_t)f32_to_bf16(v[6]) | ((uint32_t)f32_to_bf16(v[7]) << 16);
    *(uint4*)((uint16_t*)p + i) = u;
  } else {
    *(float4*)((float*)p + i) = make_float4(v[0], v[1], v[2], v[3]);
    *(float4*)((float*)p + i + 4) = make_float4(v[4], v[5], v[6], v[7]);
  }
}

constexpr int kRun = 32;   // positions per thread in the conv backward

// One thread: 8 channels of one branch over kRun consecutive positions.
template <bool BF16, int KS>
__global__ void __launch_bounds__(256) k_conv_bwd(ConvBwdArgs a) {
  const int groups = a.d >> 3;
  const int gx = blockIdx.x * 256 + threadIdx.x;
  if (gx >= a.hc * groups) return;
  const int h = gx / groups;
  const int c0 = (gx - h * groups) * 8;
  const int T = a.seqlen, D = a.dil;
  const int runs = (T + kRun - 1) / kRun;
  const int b = blockIdx.y / runs, run = blockIdx.y % runs;
  const int t_lo = run * kRun, t_hi = min(T, t_lo + kRun);
  const int64_t d = a.d, hcd = (int64_t)a.hc * d, O = (int64_t)(a.hc + 1) * d;

  float w[KS][8], dw[KS][8];
#pragma unroll
  for (int i = 0; i < 8; i++)
#pragma unroll
    for (int j = 0; j < KS; j++) {
      w[j][i] = ld_elem(a.conv_w, ((int64_t)h * d + c0 + i) * KS + j, BF16);
      dw[j][i] = 0.f;
    }
  for (int t = t_lo; t < t_hi; t++) {
    const int64_t n = (int64_t)b * T + t;
    float dyv[8], acc[8];
    ld8(a.dy, n * hcd + (int64_t)h * d + c0, BF16, dyv);
#pragma unroll
    for (int i = 0; i < 8; i++) acc[i] = dyv[i];
#pragma unroll
    for (int j = 0; j < KS; j++) {
      const int shift = (KS - 1 - j) * D;
      if (t + shift < T) {   // this position feeds y[t + shift] through tap j
        float da[8];
        ld8(a.dy, (n + shift) * hcd + (int64_t)h * d + c0, BF16, da);
#pragma unroll
        for (int i = 0; i < 8; i++) acc[i] = fmaf(w[j][i], da[i], acc[i]);
      }
      if (t - shift >= 0) {  // tap j of y[t] reads Vg[t - shift]
        const int64_t m = n - shift;
        const float g = a.stats[m * a.hc + h].x;
        float v[8];
        ld8(a.kv, m * O + hcd + c0, BF16, v);
#pragma unroll
        for (int i = 0; i < 8; i++) dw[j][i] = fmaf(dyv[i], g * v[i], dw[j][i]);
      }
    }
    st8(a.dvg, n * hcd + (int64_t)h * d + c0, false, acc);
  }
#pragma unroll
  for (int i = 0; i < 8; i++)
#pragma unroll
    for (int j = 0; j < KS; j++) atomicAdd(&a.d_conv_w[((int64_t)h * d + c0 + i) * KS + j], dw[j][i]);
}

// One wavefront per (token, branch): dg, the score's gradient, dK (into the
// key block of dkv), d hidden, and the gammas' gradients.
template <bool BF16>
__global__ void __launch_bounds__(256) k_gate_bwd(GateBwdArgs a) {
  const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (wid >= (int64_t)a.n_tok * a.hc) return;
  const int64_t n = wid / a.hc;
  const int h = (int)(wid - n * a.hc);
  const int64_t d = a.d, O = (int64_t)(a.hc + 1) * d;
  const float4 st = a.stats[n * a.hc + h];
  const float g = st.x, s = st.y, rk = st.z, rq = st.w;
  const int64_t k_off = n * O + (int64_t)h * d, v_off = n * O + (int64_t)a.hc * d;
  const int64_t q_off = (n * a.hc + h) * d, g_off = (int64_t)h * d;

  float dg = 0.f;
  for (int64_t c = lane * 8; c < d; c += 512) {
    float dv[8], V[8];
    ld8(a.dvg, q_off + c, false, dv);
    ld8(a.kv, v_off + c, BF16, V);
#pragma unroll
    for (int i = 0; i < 8; i++) dg = fmaf(dv[i], V[i], dg);
  }
  dg = wave_sum(dg);
  const float as = fabsf(s);
  const float ds = (s != 0.f && as >= a.clamp) ? dg * g * (1.f - g) / (2.f * sqrtf(as)) : 0.f;
  const float cu = ds * rq * a.inv_sqrt_d, cv = ds * rk * a.inv_sqrt_d;   // du = cu Q gq, dv = cv K gk

  float A = 0.f, B = 0.f;
  if (ds != 0.f) {
    for (int64_t c = lane * 8; c < d; c += 512) {
      float K[8], Q[8], gk[8], gq[8];
      ld8(a.kv, k_off + c, BF16, K);
      ld8(a.hidden, q_off + c, BF16, Q);
      ld8(a.gamma_k, g_off + c, BF16, gk);
      ld8(a.gamma_q, g_off + c, BF16, gq);
#pragma unroll
      for (int i = 0; i < 8; i++) {
        const float du = cu * Q[i] * gq[i], dv = cv * K[i] * gk[i];
        A = fmaf(du * gk[i], K[i], A);
        B = fmaf(dv * gq[i], Q[i], B);
        atomicAdd(&a.d_gamma_k[g_off + c + i], du * K[i] * rk);
        atomicAdd(&a.d_gamma_q[g_off + c + i], dv * Q[i] * rq);
      }
    }
    A = wave_sum(A);
    B = wave_sum(B);
  }
  const float inv_d = 1.f / (float)d;
  const float ak = rk * rk * rk * A * inv_d, bq = rq * rq * rq * B * inv_d;
  for (int64_t c = lane * 8; c < d; c += 512) {
    float K[8], Q[8], gk[8], gq[8], dK[8], dQ[8];
    ld8(a.kv, k_off + c, BF16, K);
    ld8(a.hidden, q_off + c, BF16, Q);
    ld8(a.gamma_k, g_off + c, BF16, gk);
    ld8(a.gamma_q, g_off + c, BF16, gq);
#pragma unroll
    for (int i = 0; i < 8; i++) {
      const float du = cu * Q[i] * gq[i], dv = cv * K[i] * gk[i];
      dK[i] = rk * gk[i] * du - ak * K[i];
      dQ[i] = rq * gq[i] * dv - bq * Q[i];
    }
    st8(a.dkv, k_off + c, BF16, dK);
    st8(a.d_hidden, q_off + c, BF16, dQ);
  }
}

// dV[n][c] = sum_h g[n][h] dVg[n][h][c], into the value block of dkv
template <bool BF16>
__global__ void __launch_bounds__(256) k_value_bwd(GateBwdArgs a) {
  const int groups = a.d >> 3;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)a.n_tok * groups) return;
  const int64_t n = i / groups;
  const int c0 = (int)(i - n * groups) * 8;
  const int64_t d = a.d, O = (int64_t)(a.hc + 1) * d;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int h = 0; h < a.hc; h++) {
    const float g = a.stats[n * a.hc + h].x;
    float v[8];
    ld8(a.dvg, (n * a.hc + h) * d + c0, false, v);
#pragma unroll
    for (int k = 0; k < 8; k++) acc[k] = fmaf(g, v[k], acc[k]);
  }
  st8(a.dkv, n * O + (int64_t)a.hc * d + c0, BF16, acc);
}

// 64 x 64 tiles through LDS; columns r of dst past the source rows are zero
template <typename Elem>
__global__ void __launch_bounds__(256) k_transpose(const Elem* __restrict__ src, Elem* __restrict__ dst,
                                                   int64_t rows, int64_t cols, int64_t ld_dst) {
  __shared__ Elem tile[64][65];
  const int64_t r0 = (int64_t)blockIdx.x * 64, c0 = (int64_t)blockIdx.y * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int k = ty; k < 64; k += 4) {
    const int64_t r = r0 + k, c = c0 + tx;
    tile[k][tx] = (r < rows && c < cols) ? src[r * cols + c] : Elem(0);
  }
  __syncthreads();
  for (int k = ty; k < 64; k += 4) {
    const int64_t c = c0 + k, r = r0 + tx;
    if (c < cols && r < ld_dst) dst[c * ld_dst + r] = tile[tx][k];
  }
}

__global__ void __launch_bounds__(256) k_scatter_add(HashConsts hc, const int32_t* __restrict__ idx,
                                                     const float* __restrict__ de, float* d_tables, int64_t n_tok,
                                                     int32_t Dh) {
  const int64_t E = (int64_t)hc.n_heads * Dh;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n_tok * E) return;
  const int64_t n = i / E;
  const int e = (int)(i - n * E);
  const int h = e / Dh, j = e - h * Dh;
  const int64_t row = hc.row_off[h] + idx[n * hc.n_heads + h];
  atomicAdd(&d_tables[row * Dh + j], de[i]);
}

template <bool BF16>
hipError_t conv_bwd_dispatch(const ConvBwdArgs& a, dim3 grid, hipStream_t s) {
  switch (a.ksize) {
    case 1: k_conv_bwd<BF16, 1><<<grid, 256, 0, s>>>(a); break;
    case 2: k_conv_bwd<BF16, 2><<<grid, 256, 0, s>>>(a); break;
    case 3: k_conv_bwd<BF16, 3><<<grid, 256, 0, s>>>(a); break;
    case 4: k_conv_bwd<BF16, 4><<<grid, 256, 0, s>>>(a); break;
    case 5: k_conv_bwd<BF16, 5><<<grid, 256, 0, s>>>(a); break;
    case 6: k_conv_bwd<BF16, 6><<<grid, 256, 0, s>>>(a); break;
    case 7: k_conv_bwd<BF16, 7><<<grid, 256, 0, s>>>(a); break;
    case 8: k_conv_bwd<BF16, 8><<<grid, 256, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_conv_bwd(const ConvBwdArgs& a, hipStream_t s) {
  if ((int64_t)a.batch * a.seqlen == 0) return hipSuccess;
  const int lanes = a.hc * (a.d / 8);
  const int runs = (a.seqlen + kRun - 1) / kRun;
  dim3 grid((unsigned)((lanes + 255) / 256), (unsigned)((int64_t)a.batch * runs));
  return a.bf16 ? conv_bwd_dispatch<true>(a, grid, s) : conv_bwd_dispatch<false>(a, grid, s);
}

hipError_t launch_gate_bwd(const GateBwdArgs& a, hipStream_t s) {
  const int64_t waves = (int64_t)a.n_tok * a.hc;
  if (waves == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((waves + 3) / 4);
  const unsigned vblocks = (unsigned)(((int64_t)a.n_tok * (a.d / 8) + 255) / 256);
  if (a.bf16) {
    k_gate_bwd<true><<<blocks, 256, 0, s>>>(a);
    k_value_bwd<true><<<vblocks, 256, 0, s>>>(a);
  } else {
    k_gate_bwd<false><<<blocks, 256, 0, s>>>(a);
    k_value_bwd<false><<<vblocks, 256, 0, s>>>(a);
  }
  return hipGetLastError();
}

hipError_t launch_transpose(const void* src, void* dst, int64_t rows, int64_t cols, int64_t ld_dst, int esz,
                            hipStream_t s) {
  if (rows == 0 || cols == 0) return hipSuccess;
  dim3 grid((unsigned)((ld_dst + 63) / 64), (unsigned)((cols + 63) / 64));
  if (esz == 2)
    k_transpose<uint16_t><<<grid, 256, 0, s>>>((const uint16_t*)src, (uint16_t*)dst, rows, cols, ld_dst);
  else
    k_transpose<float><<<grid, 256, 0, s>>>((const float*)src, (float*)dst, rows, cols, ld_dst);
  return hipGetLastError();
}

hipError_t launch_scatter_add(const HashConsts& hc, const int32_t* idx, const float* de, float* d_tables,
                              int64_t n_tok, int32_t head_dim, hipStream_t s) {
  const int64_t total = n_tok * hc.n_heads * head_dim;
  if (total == 0) return hipSuccess;
  k_scatter_add<<<(unsigned)((total + 255) / 256), 256, 0, s>>>(hc, idx, de, d_tables, n_tok, head_dim);
  return hipGetLastError();
}

}  // namespace engram
