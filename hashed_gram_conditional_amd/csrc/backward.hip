// Backward pass of the module (a training step; the walk-through,
// yaoyuxiang.cn/news/830577, section 4.4, trains the module).  The pages give
// the forward only; these kernels compute its exact derivatives:
//   conv + residual:  dVg[t] = dy[t] + sum_j w[j] dy[t + (K-1-j)D],
//                     dw[h][c][j] = sum_t dy[t][h][c] Vg[t - (K-1-j)D][h][c]
//   value fusion:     dV[t][c] = sum_h g dVg,  dg[t][h] = sum_c dVg V
//   gate:             ds = dg g (1-g) / (2 sqrt|s|) where |s| >= clamp and s != 0, else 0
//                     (sign(s) sqrt(max(|s|, clamp)) is flat in s inside the clamp)
//   score s = sum_c u v / sqrt(d), u = K rk gk, v = Q rq gq, rk = (mean K^2 + eps)^-1/2.
// With P = sum_c K gk gq Q = s sqrt(d) / (rk rq), the RMSNorm backward's two
// channel sums are both ds s / r, so per (token, branch) only dg needs a
// reduction, and with coef = ds rk rq / sqrt(d):
//                     dK = coef gk gq Q - (ds s rk^2 / d) K
//                     dQ = coef gk gq K - (ds s rq^2 / d) Q
//                     d gk = gq S,  d gq = gk S,  S[h][c] = sum_t coef K Q
// The sums over tokens (conv taps, S) are per-block partial rows reduced in a
// fixed order, so they do not vary between runs.  The projection and table
// gradients are GEMMs and a scatter-add launched from the C ABI.
#include "engram_internal.h"

namespace engram {
namespace {

constexpr int kGateBwdMaxTpb = 64;   // tokens per block of the gate backward (LDS: 12 B per token and branch)

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
    u.x = pack_bf16x2(v[0], v[1]);
    u.y = pack_bf16x2(v[2], v[3]);
    u.z = pack_bf16x2(v[4], v[5]);
    u.w = pack_bf16x2(v[6], v[7]);
    *(uint4*)((uint16_t*)p + i) = u;
  } else {
    *(float4*)((float*)p + i) = make_float4(v[0], v[1], v[2], v[3]);
    *(float4*)((float*)p + i + 4) = make_float4(v[4], v[5], v[6], v[7]);
  }
}

// 4 consecutive values at element i as floats, zeros when !ok (address clamped to 0)
__device__ __forceinline__ void ld4_or0(const void* p, int64_t i, bool ok, bool bf16, float* v) {
  if (bf16) {
    const uint2 u = *(const uint2*)((const uint16_t*)p + (ok ? i : 0));
    v[0] = __uint_as_float(u.x << 16);
    v[1] = __uint_as_float(u.x & 0xFFFF0000u);
    v[2] = __uint_as_float(u.y << 16);
    v[3] = __uint_as_float(u.y & 0xFFFF0000u);
  } else {
    const float4 f = *(const float4*)((const float*)p + (ok ? i : 0));
    v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
  }
#pragma unroll
  for (int k = 0; k < 4; k++) v[k] = ok ? v[k] : 0.f;
}

__device__ __forceinline__ void st4(void* p, int64_t i, bool bf16, const float* v) {
  if (bf16) {
    uint2 u;
    u.x = pack_bf16x2(v[0], v[1]);
    u.y = pack_bf16x2(v[2], v[3]);
    *(uint2*)((uint16_t*)p + i) = u;
  } else {
    *(float4*)((float*)p + i) = make_float4(v[0], v[1], v[2], v[3]);
  }
}

constexpr int kConvCh = 4;   // channels per thread of the conv backward

// v + v of another lane by a DPP move (no LDS): CTRL 0xB1 / 0x4E are the quad
// permutations of lane l ^ 1 / l ^ 2; 0x124 / 0x128 rotate a 16-lane row by 4 / 8
template <int CTRL>
__device__ __forceinline__ float add_dpp(float v) {
  return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}

// Sum over the lanes that share lane bits >= log2(hc) (the hc lanes of one
// channel group), hc a power of two up to 16.
__device__ __forceinline__ float sum_over_branches(float v, int hc) {
  if (hc > 1) v = add_dpp<0xB1>(v);
  if (hc > 2) v = add_dpp<0x4E>(v);
  for (int o = 4; o < hc; o <<= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Sum over the lanes with the same lane % hc (one branch, every channel group
// of the wave); the lanes with lane < hc hold it.  Rotations by multiples of
// hc within a row keep lane % hc, so they sum a branch's lanes of the row.
__device__ __forceinline__ float sum_over_channels(float v, int hc) {
  if (hc == 1) v = add_dpp<0xB1>(v);
  if (hc <= 2) v = add_dpp<0x4E>(v);
  if (hc <= 4) v = add_dpp<0x124>(v);
  if (hc <= 8) v = add_dpp<0x128>(v);
  v += __shfl_xor(v, 16, 64);
  v += __shfl_xor(v, 32, 64);
  return v;
}

// Block: 64 lanes over (branch, 4 channels) x 4 spans of `span` consecutive
// positions of one sequence.  A thread walks its span one residue r mod D at a
// time in steps of D, so the dy values ahead (dy[t + m D], m < K) and the
// gated values behind (Vg[t - m D]) are rings in registers: one new load of
// each per step.  The tap sums of the 4 spans are added in LDS in span order
// and stored as the block's partial row.
//
// FUSE (hc a power of two): lanes are ordered branch-minor (lane = channel
// group * hc + branch), so the dVg of a step never reaches memory: the hc
// lanes of a channel group add g dVg into dV (xor shuffles over the low lane
// bits) and the lanes of one branch add dVg . V over the wave's 64 channels
// into one partial of dg (shuffles over the high bits), both in a fixed order.
// Otherwise (lane = branch * groups + channel group) dVg is stored for the
// gate kernel.
template <bool BF16, int KS, bool FUSE>
__global__ void __launch_bounds__(256) k_conv_bwd(ConvBwdArgs a) {
  constexpr int CH = kConvCh;
  __shared__ float red[3][KS * CH][64];
  const int lane = threadIdx.x & 63, sp = threadIdx.x >> 6;
  const int groups = a.d / CH;
  const int gx = blockIdx.x * 64 + lane;
  const bool active = gx < a.hc * groups;
  int h, c0;
  if (FUSE) {
    h = gx % a.hc;
    c0 = active ? gx / a.hc * CH : 0;
  } else {
    h = active ? gx / groups : 0;
    c0 = active ? (gx - h * groups) * CH : 0;
  }
  const int T = a.seqlen, D = a.dil;
  const int blocks_per_seq = (T + 4 * a.span - 1) / (4 * a.span);
  const int b = blockIdx.y / blocks_per_seq;
  const int t_lo = (blockIdx.y - b * blocks_per_seq) * 4 * a.span + sp * a.span;
  const int t_hi = min(T, t_lo + a.span);
  const int64_t d = a.d, hcd = (int64_t)a.hc * d, O = (int64_t)(a.hc + 1) * d;
  const int64_t row0 = (int64_t)b * T;

  float dw[KS][CH];
#pragma unroll
  for (int j = 0; j < KS; j++)
#pragma unroll
    for (int i = 0; i < CH; i++) dw[j][i] = 0.f;

  // FUSE: every lane walks (inactive ones on zeros) so the shuffles see all 64
  if (FUSE || active) {
    float w[KS][CH];
#pragma unroll
    for (int i = 0; i < CH; i++)
#pragma unroll
      for (int j = 0; j < KS; j++) w[j][i] = active ? ld_elem(a.conv_w, ((int64_t)h * d + c0 + i) * KS + j, BF16) : 0.f;
    const int64_t dy_col = (int64_t)h * d + c0, v_col = hcd + c0;
    // 0 outside [0, T) (and for inactive lanes)
    auto load_dy = [&](int t, float* v) {
      ld4_or0(a.dy, (row0 + (t < T ? t : 0)) * hcd + dy_col, active && t < T, BF16, v);
    };
    auto load_v = [&](int t, float* v, float& g) {   // V at t and the gate of this branch
      const bool ok = active && t >= 0 && t < T;
      const int64_t n = row0 + (ok ? t : 0);
      ld4_or0(a.kv, n * O + v_col, ok, BF16, v);
      g = ok ? a.stats[n * a.hc + h].x : 0.f;
    };
    for (int r = 0; r < D; r++) {
      const int t0 = t_lo + r;
      if (t0 >= t_hi) break;
      const int n_steps = (t_hi - t0 + D - 1) / D;
      // rings: at step s, slot (s + m) % KS holds dy[t + m D] and slot
      // (s - m) mod KS holds g V at t - m D (m < KS), t = t0 + s D; the loop
      // is unrolled over the ring, so every slot index is a constant
      float F[KS][CH], P[KS][CH];
      // FUSE: results kept for a batched store (see below); n < 0: none held
      float keep_dv[CH] = {0.f, 0.f, 0.f, 0.f}, keep_g = 0.f;
      int64_t keep_dv_n = -1, keep_g_n = -1;
#pragma unroll
      for (int m = 0; m + 1 < KS; m++) load_dy(t0 + m * D, F[m]);
#pragma unroll
      for (int m = 1; m < KS; m++) {
        float g;
        load_v(t0 - m * D, P[KS - m], g);
#pragma unroll
        for (int i = 0; i < CH; i++) P[KS - m][i] *= g;
      }
      for (int s0 = 0; s0 < n_steps; s0 += KS) {
#pragma unroll
        for (int u = 0; u < KS; u++) {
          const int st = s0 + u;
          if (st >= n_steps) break;
          const int t = t0 + st * D;
          load_dy(t + (KS - 1) * D, F[(u + KS - 1) % KS]);   // the step's new dy (m = KS-1)
          float V[CH], g;                                    // and V, g at t (m = 0)
          load_v(t, V, g);
#pragma unroll
          for (int i = 0; i < CH; i++) P[u][i] = V[i] * g;
          float acc[CH];
#pragma unroll
          for (int i = 0; i < CH; i++) acc[i] = F[u][i];
#pragma unroll
          for (int j = 0; j < KS; j++)
#pragma unroll
            for (int i = 0; i < CH; i++) {
              acc[i] = fmaf(w[j][i], F[(u + KS - 1 - j) % KS][i], acc[i]);
              dw[j][i] = fmaf(F[u][i], P[(u + 1 + j) % KS][i], dw[j][i]);
            }
          if constexpr (FUSE) {
            float dv[CH], pg = 0.f;
#pragma unroll
            for (int i = 0; i < CH; i++) {
              dv[i] = g * acc[i];
              pg = fmaf(acc[i], V[i], pg);
            }
#pragma unroll
            for (int i = 0; i < CH; i++) dv[i] = sum_over_branches(dv[i], a.hc);
            pg = sum_over_channels(pg, a.hc);
            // Stores are batched: a store instruction costs about the same for
            // a few lanes as for the whole wave.  All hc lanes of a channel
            // group hold the same dV (a butterfly), so lane h keeps the dV of
            // steps st = h mod hc and the wave stores every hc steps; lane
            // u hc + h keeps branch h's dg partial of step u of each run of
            // 64/hc steps, stored once per run.
            const int64_t n = row0 + t;
            const int G = 64 / a.hc;
            if (st % a.hc == h) {
#pragma unroll
              for (int i = 0; i < CH; i++) keep_dv[i] = dv[i];
              keep_dv_n = n;
            }
            if (st % G == lane / a.hc) {
              keep_g = pg;
              keep_g_n = n;
            }
            const bool last = st + 1 == n_steps;
            if (st % a.hc == a.hc - 1 || last) {
              if (active && keep_dv_n >= 0) st4(a.dkv, keep_dv_n * O + hcd + c0, BF16, keep_dv);
              keep_dv_n = -1;
            }
            if (st % G == G - 1 || last) {
              if (keep_g_n >= 0) a.dgp[(keep_g_n * a.n_dgp + blockIdx.x) * a.hc + h] = keep_g;
              keep_g_n = -1;
            }
          } else {
            st4(a.dvg, (row0 + t) * hcd + dy_col, BF16, acc);
          }
        }
      }
    }
  }
  // spans 1..3 hand their sums to span 0, which adds them in order
  if (sp > 0) {
#pragma unroll
    for (int j = 0; j < KS; j++)
#pragma unroll
      for (int i = 0; i < CH; i++) red[sp - 1][j * CH + i][lane] = dw[j][i];
  }
  __syncthreads();
  if (sp == 0 && active) {
    float* out = a.part + (int64_t)blockIdx.y * hcd * KS + ((int64_t)h * d + c0) * KS;
#pragma unroll
    for (int i = 0; i < CH; i++)
#pragma unroll
      for (int j = 0; j < KS; j++)
        out[i * KS + j] = ((dw[j][i] + red[0][j * CH + i][lane]) + red[1][j * CH + i][lane]) + red[2][j * CH + i][lane];
  }
}

// Block: tpb consecutive tokens, all branches.
// Phase 1 (one wave per token): dg of every branch (V read once) and dV into
// the value block of dkv -- or, after the fused conv kernel, dg from its
// per-64-channel partials -- and per (token, branch) coef, ak = ds s rk^2 / d,
// bq = ds s rq^2 / d into LDS.  Phase 2 (a thread per 8 channels of one
// branch, looping over the block's tokens): dK, dQ and the partial S.
template <bool BF16, int HB>   // HB >= hc: bound of the per-branch arrays of phase 1
__global__ void __launch_bounds__(256) k_gate_bwd(GateBwdArgs a) {
  __shared__ float3 co[kGateBwdMaxTpb * ENGRAM_MAX_BRANCHES];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t n0 = (int64_t)blockIdx.x * a.tpb;
  const int nt = (int)min((int64_t)a.tpb, (int64_t)a.n_tok - n0);
  const int hc = a.hc;
  const int64_t d = a.d, hcd = (int64_t)hc * d, O = (int64_t)(hc + 1) * d;
  const float inv_d = 1.f / (float)d;

  for (int t = wave; t < nt; t += 4) {
    const int64_t n = n0 + t;
    float g[HB], dgp[HB];
#pragma unroll
    for (int h = 0; h < HB; h++) {
      g[h] = h < hc ? a.stats[n * hc + h].x : 0.f;
      dgp[h] = 0.f;
    }
    if (a.dgp) {   // dg partials per 64 channels from the conv kernel (dV is already stored)
#pragma unroll
      for (int h = 0; h < HB; h++)
        if (h < hc)
          for (int k = lane; k < a.n_dgp; k += 64) dgp[h] += a.dgp[(n * a.n_dgp + k) * hc + h];
    } else {
#pragma unroll 2
    for (int64_t c = lane * 8; c < d; c += 512) {
      float V[8], dV[8];
      ld8(a.kv, n * O + hcd + c, BF16, V);
#pragma unroll
      for (int i = 0; i < 8; i++) dV[i] = 0.f;
#pragma unroll
      for (int h = 0; h < HB; h++) {
        if (h < hc) {
          float dv[8];
          ld8(a.dvg, (n * hc + h) * d + c, BF16, dv);
#pragma unroll
          for (int i = 0; i < 8; i++) {
            dgp[h] = fmaf(dv[i], V[i], dgp[h]);
            dV[i] = fmaf(g[h], dv[i], dV[i]);
          }
        }
      }
      st8(a.dkv, n * O + hcd + c, BF16, dV);
    }
    }
#pragma unroll
    for (int h = 0; h < HB; h++) {
      if (h < hc) {
        const float dg = wave_sum(dgp[h]);
        const float4 st = a.stats[n * hc + h];
        const float s = st.y, rk = st.z, rq = st.w, as = fabsf(s);
        const float ds = (s != 0.f && as >= a.clamp) ? dg * g[h] * (1.f - g[h]) / (2.f * sqrtf(as)) : 0.f;
        if (lane == 0)
          co[t * hc + h] = make_float3(ds * rk * rq * a.inv_sqrt_d, ds * s * rk * rk * inv_d, ds * s * rq * rq * inv_d);
      }
    }
  }
  __syncthreads();

  const int groups = a.d >> 3;
  for (int j = threadIdx.x; j < hc * groups; j += 256) {
    const int h = j / groups;
    const int64_t col = (int64_t)h * d + (int64_t)(j - h * groups) * 8;
    float gk[8], gq[8], gg[8], S[8];
    ld8(a.gamma_k, col, BF16, gk);
    ld8(a.gamma_q, col, BF16, gq);
#pragma unroll
    for (int i = 0; i < 8; i++) {
      gg[i] = gk[i] * gq[i];
      S[i] = 0.f;
    }
#pragma unroll 2
    for (int t = 0; t < nt; t++) {
      const int64_t n = n0 + t;
      const float3 c3 = co[t * hc + h];
      float K[8], Q[8], dK[8], dQ[8];
      ld8(a.kv, n * O + col, BF16, K);
      ld8(a.hidden, n * hcd + col, BF16, Q);
#pragma unroll
      for (int i = 0; i < 8; i++) {
        dK[i] = c3.x * gg[i] * Q[i] - c3.y * K[i];
        dQ[i] = c3.x * gg[i] * K[i] - c3.z * Q[i];
        S[i] = fmaf(c3.x * K[i], Q[i], S[i]);
      }
      st8(a.dkv, n * O + col, BF16, dK);
      st8(a.d_hidden, n * hcd + col, BF16, dQ);
    }
    st8(a.part, (int64_t)blockIdx.x * hcd + col, false, S);
  }
}

// out0[c] += scale0[c] sum_r part[r][c] (and out1 with scale1).  Block: 64
// columns x 4 row groups; group q sums rows q, q+4, ... in order, then the
// four group sums are added in group order.
__global__ void __launch_bounds__(256) k_colsum(const float* __restrict__ part, int64_t rows, int64_t cols,
                                                float* out0, const void* scale0, float* out1, const void* scale1,
                                                bool bf16) {
  __shared__ float red[3][64];
  const int lane = threadIdx.x & 63, q = threadIdx.x >> 6;
  const int64_t c = (int64_t)blockIdx.x * 64 + lane;
  float acc = 0.f;
  if (c < cols) {
    int64_t r = q;
    for (; r + 28 < rows; r += 32) {   // 8 loads in flight, added in row order
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; i++) v[i] = part[(r + 4 * i) * cols + c];
#pragma unroll
      for (int i = 0; i < 8; i++) acc += v[i];
    }
    for (; r < rows; r += 4) acc += part[r * cols + c];
  }
  if (q > 0) red[q - 1][lane] = acc;
  __syncthreads();
  if (q == 0 && c < cols) {
    const float S = ((acc + red[0][lane]) + red[1][lane]) + red[2][lane];
    out0[c] += scale0 ? ld_elem(scale0, c, bf16) * S : S;
    if (out1) out1[c] += scale1 ? ld_elem(scale1, c, bf16) * S : S;
  }
}

// The same sum for few rows: 4 consecutive columns per thread, rows added in order.
__global__ void __launch_bounds__(256) k_colsum_short(const float* __restrict__ part, int64_t rows, int64_t cols,
                                                      float* out0, const void* scale0, float* out1,
                                                      const void* scale1, bool bf16) {
  const int64_t c = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (c >= cols) return;
  float4 S = *(const float4*)(part + c);
  for (int64_t r = 1; r < rows; r++) {
    const float4 v = *(const float4*)(part + r * cols + c);
    S.x += v.x;
    S.y += v.y;
    S.z += v.z;
    S.w += v.w;
  }
  const float s4[4] = {S.x, S.y, S.z, S.w};
  float4 o = *(float4*)(out0 + c);
  float o4[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
  for (int i = 0; i < 4; i++) o4[i] += scale0 ? ld_elem(scale0, c + i, bf16) * s4[i] : s4[i];
  *(float4*)(out0 + c) = make_float4(o4[0], o4[1], o4[2], o4[3]);
  if (out1) {
    o = *(float4*)(out1 + c);
    float p4[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
    for (int i = 0; i < 4; i++) p4[i] += scale1 ? ld_elem(scale1, c + i, bf16) * s4[i] : s4[i];
    *(float4*)(out1 + c) = make_float4(p4[0], p4[1], p4[2], p4[3]);
  }
}

// 64 x 64 tiles through LDS, 16 bytes per lane each way; columns r of dst past
// the source rows are zero.  rows, cols and ld_dst are multiples of 16 / sizeof(Elem).
template <typename Elem>
__global__ void __launch_bounds__(256) k_transpose(const Elem* __restrict__ src, Elem* __restrict__ dst,
                                                   int64_t rows, int64_t cols, int64_t ld_dst, int64_t chunk) {
  constexpr int V = 16 / sizeof(Elem);   // elements per 16-byte piece
  constexpr int PR = 64 / V;             // pieces per tile row
  __shared__ Elem tile[64][64 + 2];
  const int64_t r0 = (int64_t)blockIdx.x * 64, c0 = (int64_t)blockIdx.y * 64;
  for (int p = threadIdx.x; p < 64 * PR; p += 256) {
    const int k = p / PR, x = (p % PR) * V;
    const int64_t r = r0 + k, c = c0 + x;
    Elem v[V];
    if (r < rows && c < cols) {
      *(uint4*)v = *(const uint4*)(src + r * cols + c);
    } else {
#pragma unroll
      for (int i = 0; i < V; i++) v[i] = Elem(0);
    }
#pragma unroll
    for (int i = 0; i < V; i++) tile[k][x + i] = v[i];
  }
  __syncthreads();
  // chunked layout: the whole tile lies in chunk r0 / chunk
  const int64_t ch = chunk > 0 ? r0 / chunk : 0;
  Elem* const out = chunk > 0 ? dst + ch * cols * chunk : dst;
  const int64_t ld = chunk > 0 ? chunk : ld_dst, r_base = chunk > 0 ? r0 - ch * chunk : r0;
  for (int p = threadIdx.x; p < 64 * PR; p += 256) {
    const int k = p / PR, x = (p % PR) * V;   // dst row c0 + k, columns r0 + x ...
    const int64_t c = c0 + k;
    if (c < cols && r0 + x < ld_dst) {
      Elem v[V];
#pragma unroll
      for (int i = 0; i < V; i++) v[i] = tile[x + i][k];
      *(uint4*)(out + c * ld + r_base + x) = *(const uint4*)v;
    }
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

template <bool BF16, bool FUSE>
hipError_t conv_bwd_dispatch(const ConvBwdArgs& a, dim3 grid, hipStream_t s) {
  switch (a.ksize) {
    case 1: k_conv_bwd<BF16, 1, FUSE><<<grid, 256, 0, s>>>(a); break;
    case 2: k_conv_bwd<BF16, 2, FUSE><<<grid, 256, 0, s>>>(a); break;
    case 3: k_conv_bwd<BF16, 3, FUSE><<<grid, 256, 0, s>>>(a); break;
    case 4: k_conv_bwd<BF16, 4, FUSE><<<grid, 256, 0, s>>>(a); break;
    case 5: k_conv_bwd<BF16, 5, FUSE><<<grid, 256, 0, s>>>(a); break;
    case 6: k_conv_bwd<BF16, 6, FUSE><<<grid, 256, 0, s>>>(a); break;
    case 7: k_conv_bwd<BF16, 7, FUSE><<<grid, 256, 0, s>>>(a); break;
    case 8: k_conv_bwd<BF16, 8, FUSE><<<grid, 256, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

int conv_bwd_span(int64_t n_tok) { return n_tok >= 32768 ? 64 : n_tok >= 8192 ? 32 : 16; }

int64_t conv_bwd_rows(int32_t batch, int32_t seqlen) {
  const int span = conv_bwd_span((int64_t)batch * seqlen);
  return (int64_t)batch * ((seqlen + 4 * span - 1) / (4 * span));
}

bool conv_bwd_fused(int32_t hc) { return hc >= 1 && hc <= 16 && (hc & (hc - 1)) == 0; }

int conv_bwd_dg_parts(int32_t hc, int32_t d) { return (hc * (d / kConvCh) + 63) / 64; }

hipError_t launch_conv_bwd(const ConvBwdArgs& a, hipStream_t s) {
  if ((int64_t)a.batch * a.seqlen == 0) return hipSuccess;
  const int lanes = a.hc * (a.d / kConvCh);
  dim3 grid((unsigned)((lanes + 63) / 64), (unsigned)conv_bwd_rows(a.batch, a.seqlen));
  if (a.dgp != nullptr) {
    if (!conv_bwd_fused(a.hc) || a.n_dgp != (int)grid.x) return hipErrorInvalidValue;
    return a.bf16 ? conv_bwd_dispatch<true, true>(a, grid, s) : conv_bwd_dispatch<false, true>(a, grid, s);
  }
  return a.bf16 ? conv_bwd_dispatch<true, false>(a, grid, s) : conv_bwd_dispatch<false, false>(a, grid, s);
}

int gate_bwd_tpb(int64_t n_tok) {
  int t = 4;
  while (t < kGateBwdMaxTpb && n_tok >= (int64_t)2 * t * 1024) t *= 2;
  return t;
}

int64_t gate_bwd_rows(int64_t n_tok) {
  const int t = gate_bwd_tpb(n_tok);
  return (n_tok + t - 1) / t;
}

hipError_t launch_gate_bwd(const GateBwdArgs& a, hipStream_t s) {
  if (a.n_tok == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((a.n_tok + a.tpb - 1) / a.tpb);
  if (a.hc <= 4) {
    if (a.bf16)
      k_gate_bwd<true, 4><<<blocks, 256, 0, s>>>(a);
    else
      k_gate_bwd<false, 4><<<blocks, 256, 0, s>>>(a);
  } else {
    if (a.bf16)
      k_gate_bwd<true, ENGRAM_MAX_BRANCHES><<<blocks, 256, 0, s>>>(a);
    else
      k_gate_bwd<false, ENGRAM_MAX_BRANCHES><<<blocks, 256, 0, s>>>(a);
  }
  return hipGetLastError();
}

hipError_t launch_colsum(const float* part, int64_t rows, int64_t cols, float* out0, const void* scale0,
                         float* out1, const void* scale1, bool bf16, hipStream_t s) {
  if (cols == 0) return hipSuccess;
  const bool vec = cols % 4 == 0 && ((uintptr_t)part | (uintptr_t)out0 | (uintptr_t)out1) % 16 == 0;
  if (rows <= 16 && vec) {
    k_colsum_short<<<(unsigned)((cols / 4 + 255) / 256), 256, 0, s>>>(part, rows, cols, out0, scale0, out1, scale1,
                                                                      bf16);
    return hipGetLastError();
  }
  k_colsum<<<(unsigned)((cols + 63) / 64), 256, 0, s>>>(part, rows, cols, out0, scale0, out1, scale1, bf16);
  return hipGetLastError();
}

hipError_t launch_transpose(const void* src, void* dst, int64_t rows, int64_t cols, int64_t ld_dst, int esz,
                            hipStream_t s, int64_t chunk) {
  if (chunk < 0 || chunk % 64 != 0 || (chunk > 0 && ld_dst % chunk != 0)) return hipErrorInvalidValue;
  if (rows == 0 || cols == 0) return hipSuccess;
  dim3 grid((unsigned)((ld_dst + 63) / 64), (unsigned)((cols + 63) / 64));
  if (esz == 2)
    k_transpose<uint16_t><<<grid, 256, 0, s>>>((const uint16_t*)src, (uint16_t*)dst, rows, cols, ld_dst, chunk);
  else
    k_transpose<float><<<grid, 256, 0, s>>>((const float*)src, (float*)dst, rows, cols, ld_dst, chunk);
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
