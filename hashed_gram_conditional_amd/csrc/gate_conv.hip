// K3: context-aware gate, value fusion, short causal conv and residual, plus
// the decode-state update.
//
// Gate (formula sheet, kwkr.cn/news/37585, section 2.2 steps 1-2 and the full
// formula in 2.3): per token and branch h, with K_h the key and Q_h the hidden
// state of that branch,
//   s = sum_c (K_c rk gk_c) (Q_c rq gq_c) / sqrt(d),  rk = (mean K^2 + eps)^-1/2
//   g = sigmoid(sign(s) sqrt(max(|s|, clamp)))
// One wavefront per (token, branch); each lane reads 16 bytes of K, Q and both
// gammas per step and the three sums (K.K, Q.Q, K gk Q gq) are reduced across
// the wavefront, so K and Q stream through once.
//
// Value fusion, conv and residual (formula sheet 2.2 step 3 and 3.2;
// walk-through, yaoyuxiang.cn/news/830577, section 2.2-3: depthwise causal
// conv, kernel 4, dilation = largest order):
//   y_h[t] = Vg_h[t] + sum_j w_h[j] Vg_h[t - (K-1-j) D],  Vg_h = g_h V
// A wavefront walks the positions t0+r, t0+r+D, t0+r+2D, ... of one residue
// r mod D over 256 channels, for every branch: every conv tap of the next
// position is a position already visited, so the history stays in registers,
// and each value slice is loaded once for all branches.
#include <type_traits>

#include "engram_internal.h"

namespace engram {
namespace {

// 8 consecutive elements of a real array as floats
__device__ __forceinline__ void load8(const void* p, int64_t i, bool bf16, float* v) {
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

// 8 outputs of the module, stored non-temporally: the output is written once
// and not read again here, so it should not evict the table rows that the
// next call's gather finds in the last-level cache (B=8 T=4096: gather 37 ->
// 30 us; B=4 T=1024: conv 16.4 -> 14.7 us).
__device__ __forceinline__ void store8(void* p, int64_t i, bool bf16, const float* v) {
  typedef uint32_t w4 __attribute__((ext_vector_type(4)));
  if (bf16) {
    const w4 u = {pack_bf16x2(v[0], v[1]),
                  pack_bf16x2(v[2], v[3]),
                  pack_bf16x2(v[4], v[5]),
                  pack_bf16x2(v[6], v[7])};
    __builtin_nontemporal_store(u, (w4*)((uint16_t*)p + i));
  } else {
    const w4 a = {__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])};
    const w4 b = {__float_as_uint(v[4]), __float_as_uint(v[5]), __float_as_uint(v[6]), __float_as_uint(v[7])};
    __builtin_nontemporal_store(a, (w4*)((float*)p + i));
    __builtin_nontemporal_store(b, (w4*)((float*)p + i + 4));
  }
}

__device__ __forceinline__ float gate_activation(float s, float clamp) {
  const float sgn = s > 0.f ? 1.f : (s < 0.f ? -1.f : 0.f);
  const float a = sgn * sqrtf(fmaxf(fabsf(s), clamp));
  return 1.f / (1.f + expf(-a));
}

template <bool BF16>
__global__ void __launch_bounds__(256) k_gate(GateArgs a) {
  const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (wid >= (int64_t)a.n_tok * a.hc) return;
  const int64_t n = wid / a.hc;
  const int h = (int)(wid - n * a.hc);
  const int64_t d = a.d;
  const int64_t k_off = (n * (a.hc + 1) + h) * d;
  const int64_t q_off = (n * a.hc + h) * d;
  const int64_t g_off = (int64_t)h * d;
  float kk = 0.f, qq = 0.f, kq = 0.f;
  for (int64_t c = lane * 8; c < d; c += 512) {
    float K[8], Q[8], gk[8], gq[8];
    load8(a.kv, k_off + c, BF16, K);
    load8(a.hidden, q_off + c, BF16, Q);
    load8(a.gamma_k, g_off + c, BF16, gk);
    load8(a.gamma_q, g_off + c, BF16, gq);
#pragma unroll
    for (int i = 0; i < 8; i++) {
      kk = fmaf(K[i], K[i], kk);
      qq = fmaf(Q[i], Q[i], qq);
      kq = fmaf(K[i] * gk[i], Q[i] * gq[i], kq);
    }
  }
  kk = wave_sum(kk);
  qq = wave_sum(qq);
  kq = wave_sum(kq);
  if (lane == 0) {
    const float inv_d = 1.f / (float)d;
    const float rk = 1.f / sqrtf(kk * inv_d + a.eps);
    const float rq = 1.f / sqrtf(qq * inv_d + a.eps);
    const float s = kq * rk * rq * a.inv_sqrt_d;
    const float g = gate_activation(s, a.clamp);
    if (a.g_out) a.g_out[n * a.hc + h] = g;
    if (a.stats) a.stats[n * a.hc + h] = make_float4(g, s, rk, rq);
  }
}

// Positions one walk visits (stride D), measured on MI355X inside the forward
// pass: 16 for calls of at least 16384 tokens (B=8 T=4096: 8 -> 162 us,
// 16 -> 142-154 us, 24 -> 169 us; B=1 T=32768 D=4: 262, 245-257, 265 us),
// where longer walks re-read less history and reload the taps less often;
// 8 for smaller calls, where more walks fill the GPU (B=4 T=1024: 11.7 us at 8,
// 16.9 us at 16).
constexpr int conv_walk(int64_t n_tok) { return n_tok >= 16384 ? 16 : 8; }

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// 8 consecutive elements as raw words (bf16: one 16-byte piece in lo; f32:
// two pieces, lo and hi)
template <bool BF16>
__device__ __forceinline__ void load_raw8(const void* p, int64_t i, u32x4& lo, u32x4& hi) {
  if constexpr (BF16) {
    lo = *(const u32x4*)((const uint16_t*)p + i);
  } else {
    lo = *(const u32x4*)((const float*)p + i);
    hi = *(const u32x4*)((const float*)p + i + 4);
  }
}

template <bool BF16>
__device__ __forceinline__ void unpack8(const u32x4& lo, const u32x4& hi, float scale, float* v) {
  if constexpr (BF16) {
#pragma unroll
    for (int k = 0; k < 4; k++) {
      v[2 * k] = __uint_as_float(lo[k] << 16) * scale;
      v[2 * k + 1] = __uint_as_float(lo[k] & 0xFFFF0000u) * scale;
    }
  } else {
#pragma unroll
    for (int k = 0; k < 4; k++) {
      v[k] = __uint_as_float(lo[k]) * scale;
      v[4 + k] = __uint_as_float(hi[k]) * scale;
    }
  }
}

// 4 consecutive elements as raw words: 8 bytes of bf16 or 16 bytes of f32
template <bool BF16>
using Raw4 = typename std::conditional<BF16, u32x2, u32x4>::type;

template <bool BF16>
__device__ __forceinline__ void unpack4(const Raw4<BF16>& r, float scale, float* v) {
  if constexpr (BF16) {
    v[0] = __uint_as_float(r[0] << 16) * scale;
    v[1] = __uint_as_float(r[0] & 0xFFFF0000u) * scale;
    v[2] = __uint_as_float(r[1] << 16) * scale;
    v[3] = __uint_as_float(r[1] & 0xFFFF0000u) * scale;
  } else {
#pragma unroll
    for (int k = 0; k < 4; k++) v[k] = __uint_as_float(r[k]) * scale;
  }
}

// Workgroup order: workgroups are dispatched round-robin over the 8 XCDs, so
// workgroup b runs on XCD b % 8; each XCD is given a contiguous range of
// logical workgroups.  Neighbouring logical workgroups then share one XCD's L2.
__device__ __forceinline__ int xcd_contiguous(int bid, int total) {
  const int xcd = bid & 7, local = bid >> 3;
  const int per = total >> 3, rem = total & 7;
  return xcd < rem ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
}

// Gates are read through the constant address space: every lane of a
// wavefront needs the same gate, which then comes through the scalar cache.
// The gate arrays are not written while the conv runs.
typedef const __attribute__((address_space(4))) float const_float;

__device__ __forceinline__ const const_float* as_const(const float* p) { return (const const_float*)p; }

// A wavefront takes one walk: positions t_first, t_first + D, ... (W of them)
// of one residue mod D, over 256 consecutive channels (4 per lane), for every
// branch.  Every conv tap of a position is either an earlier position of the
// walk or one of the K-1 positions before it, so the walk loads those K-1 + W
// value slices once, keeps them in registers, and then takes the branches one
// after the other, each with its own taps (4 channels x K, reloaded per branch
// from the cache) and gates.  The value rows are thus read once for all
// branches instead of once per branch (B=8 T=4096 d=2560 hc=4, inside the
// forward pass: 222 -> 142-154 us).  Positions before the call come from the
// decode rings, or are zero before the sequence start.
template <bool BF16, int KS, int W>
__global__ void __launch_bounds__(256) k_conv(ConvArgs a) {
  constexpr int kCh = 4;              // channels per lane
  constexpr int kWaveCh = 64 * kCh;   // channels per wavefront
  constexpr int NP = KS - 1 + W;
  constexpr int NH = KS > 1 ? KS - 1 : 1;
  const int64_t d = a.d;
  const int D = a.dil, T = a.seqlen, hc = a.hc;
  const int nch = (a.d + kWaveCh - 1) / kWaveCh;
  const int runs = (T + W * D - 1) / (W * D);
  const int L = xcd_contiguous(blockIdx.x, gridDim.x);
  int w = __builtin_amdgcn_readfirstlane(L * 4 + (int)(threadIdx.x >> 6));
  const int cc = w % nch;
  w /= nch;
  const int r = w % D;
  w /= D;
  const int run = w % runs;
  const int b = w / runs;
  const int c0 = cc * kWaveCh + (int)(threadIdx.x & 63) * kCh;
  const int t_first = run * W * D + r;
  if (b >= a.batch || t_first >= T || c0 >= a.d) return;
  const int n_it = min(W, (T - t_first + D - 1) / D);   // positions of the walk inside the call
  const int64_t R = (KS - 1) * D + 1;   // ring length of the state (history plus the slot a decode step fills)
  const int64_t past = a.n_past ? a.n_past[b] : 0;

  // slot k holds position t_first + (k - (KS-1)) D: its raw value slice and
  // its row of gates (null for a zero position)
  Raw4<BF16> raw[NP];
  const const_float* grow[NP];
#pragma unroll
  for (int k = 0; k < NP; k++) {
    const int t = t_first + (k - (KS - 1)) * D;
    raw[k] = Raw4<BF16>{};
    grow[k] = nullptr;
    if (t >= 0) {
      if (k - (KS - 1) < n_it) {
        const int64_t n = (int64_t)b * T + t;
        raw[k] = *(const Raw4<BF16>*)((const char*)a.v + (n * a.v_stride + c0) * (BF16 ? 2 : 4));
        grow[k] = as_const(a.g + n * hc);
      }
    } else if (a.v_ring != nullptr && past + t >= 0) {
      const int64_t slot = (int64_t)b * R + (past + t) % R;
      raw[k] = *(const Raw4<BF16>*)((const char*)a.v_ring + (slot * d + c0) * (BF16 ? 2 : 4));
      grow[k] = as_const(a.g_ring + slot * hc);
    }
  }

#pragma unroll 1
  for (int h = 0; h < hc; h++) {
    // taps of channels c0..c0+3: conv_w[h][c0+i][0..KS), 4 KS consecutive
    // elements, loaded 4 at a time (the array is 16-byte aligned and c0 % 4 == 0)
    float wt[KS][kCh];
    const int64_t e0 = ((int64_t)h * d + c0) * KS;
#pragma unroll
    for (int q = 0; q < KS; q++) {
      float f[4];
      unpack4<BF16>(*(const Raw4<BF16>*)((const char*)a.conv_w + (e0 + 4 * q) * (BF16 ? 2 : 4)), 1.f, f);
#pragma unroll
      for (int m = 0; m < 4; m++) wt[(4 * q + m) % KS][(4 * q + m) / KS] = f[m];
    }
    float hist[NH][kCh];
#pragma unroll
    for (int k = 0; k < NP; k++) {
      float cur[kCh];
      unpack4<BF16>(raw[k], grow[k] != nullptr ? grow[k][h] : 0.f, cur);
      const int it = k - (KS - 1);
      if (it >= 0 && it < n_it) {
        float out[kCh];
#pragma unroll
        for (int i = 0; i < kCh; i++) {
          float acc = fmaf(wt[KS - 1][i], cur[i], cur[i]);
#pragma unroll
          for (int j = 0; j < KS - 1; j++) acc = fmaf(wt[j][i], hist[j][i], acc);
          out[i] = acc;
        }
        const int64_t o = (((int64_t)b * T + t_first + it * D) * hc + h) * d + c0;
        if constexpr (BF16) {
          const u32x2 u = {pack_bf16x2(out[0], out[1]), pack_bf16x2(out[2], out[3])};
          __builtin_nontemporal_store(u, (u32x2*)((uint16_t*)a.out + o));
        } else {
          const u32x4 u = {__float_as_uint(out[0]), __float_as_uint(out[1]), __float_as_uint(out[2]),
                           __float_as_uint(out[3])};
          __builtin_nontemporal_store(u, (u32x4*)((float*)a.out + o));
        }
      }
      if constexpr (KS > 1) {
#pragma unroll
        for (int j = 0; j + 1 < NH; j++)
#pragma unroll
          for (int i = 0; i < kCh; i++) hist[j][i] = hist[j + 1][i];
#pragma unroll
        for (int i = 0; i < kCh; i++) hist[NH - 1][i] = cur[i];
      }
    }
  }
}

// One workgroup per sequence: copy the newest positions of this call into the
// rings, then advance n_past.  Runs after every kernel that reads the rings.
template <bool BF16>
__global__ void __launch_bounds__(256) k_advance(AdvanceArgs a) {
  const int b = blockIdx.x;
  const int T = a.seqlen;
  const int64_t past = a.n_past[b];
  const int64_t d = a.d;
  const int esz = BF16 ? 2 : 4;
  // value and gate rings: last min(T, R) positions
  if (a.ring_len > 0) {
    const int cnt = T < a.ring_len ? T : a.ring_len;
    const int t_lo = T - cnt;
    const int64_t words = (int64_t)cnt * d * esz / 4;   // d % 8 == 0, so rows are whole 32-bit words
    const int64_t row_words = d * esz / 4;
    for (int64_t i = threadIdx.x; i < words; i += 256) {
      const int tt = (int)(i / row_words);
      const int64_t wd = i - tt * row_words;
      const int t = t_lo + tt;
      const int64_t slot = (int64_t)b * a.ring_len + (past + t) % a.ring_len;
      const int64_t n = (int64_t)b * T + t;
      const uint32_t* src = (const uint32_t*)((const uint8_t*)a.v + n * a.v_stride * esz);
      ((uint32_t*)((uint8_t*)a.v_ring + slot * d * esz))[wd] = src[wd];
    }
    for (int i = threadIdx.x; i < cnt * a.hc; i += 256) {
      const int tt = i / a.hc, h = i - tt * a.hc;
      const int t = t_lo + tt;
      const int64_t slot = (int64_t)b * a.ring_len + (past + t) % a.ring_len;
      a.g_ring[slot * a.hc + h] = a.g[((int64_t)b * T + t) * a.hc + h];
    }
  }
  if (a.tok_ring_len > 0) {
    const int cnt = T < a.tok_ring_len ? T : a.tok_ring_len;
    for (int i = threadIdx.x; i < cnt; i += 256) {
      const int t = T - cnt + i;
      const int32_t id = a.ids[(int64_t)b * T + t];
      int32_t x = a.pad_id;
      if (id >= 0 && id < a.vocab) x = a.remap ? a.remap[id] : id;
      a.tok_ring[(int64_t)b * a.tok_ring_len + (past + t) % a.tok_ring_len] = x;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) a.n_past[b] = past + T;
}

// One decode step (T = 1) with a state, after the fused projection.  Block
// (channel block cb, sequence b) of hc wavefronts: wavefront h takes branch h
// of 64 groups of 8 channels, so the branches of the same channels run on one
// CU and their reads of the value row and its history taps are served once
// from memory (branches in other workgroups would land on other XCDs and
// fetch them again).  The gates of all branches come from the partial sums (8
// lanes each, as gate_finalize); the output is the conv over the rings'
// history with k_conv's arithmetic; then the new position enters the rings at
// slot past % R.  The rings hold R = (K-1) D + 1 positions, so that slot is
// never one the history reads (those are past - m D, 0 < m D < R), and the
// block may write it while other blocks still read the history.  Every block
// reads n_past from the hash kernel's snapshot; one thread then advances
// n_past and the token ring.
template <bool BF16, int KS>
__global__ void __launch_bounds__(64 * ENGRAM_MAX_BRANCHES) k_decode_tail(DecodeTailArgs a) {
  __shared__ float sg[ENGRAM_MAX_BRANCHES];
  const int cb = blockIdx.x, b = blockIdx.y;
  const int h = threadIdx.x >> 6;
  const int gx = cb * 64 + (threadIdx.x & 63);   // 8-channel group of this lane
  const bool active = gx < (a.d >> 3);
  const int c0 = gx * 8;
  const int64_t past = a.past[b];
  const int64_t d = a.d, R = a.ring_len;
  const int64_t new_slot = (int64_t)b * R + past % R;

  if ((int)threadIdx.x < 8 * a.hc) {   // one 8-lane group per branch
    const int hh = threadIdx.x >> 3;
    const float g = gate_from_partials8(a.partials + ((int64_t)b * a.hc + hh) * a.n_part, a.n_part, true, a.d, a.eps,
                                        a.clamp, a.inv_sqrt_d);
    if ((threadIdx.x & 7) == 0) {
      sg[hh] = g;
      if (cb == 0) a.g_ring[new_slot * a.hc + hh] = g;
    }
  }
  __syncthreads();
  if (active) {
    // taps of channels c0..c0+7: conv_w[h][c0+i][0..KS), 8 KS consecutive
    // elements, loaded 4 at a time (c0 % 8 == 0 keeps every load aligned)
    float w[KS][8];
    const int64_t e0 = ((int64_t)h * d + c0) * KS;
#pragma unroll
    for (int q = 0; q < 2 * KS; q++) {
      float f[4];
      unpack4<BF16>(*(const Raw4<BF16>*)((const char*)a.conv_w + (e0 + 4 * q) * (BF16 ? 2 : 4)), 1.f, f);
#pragma unroll
      for (int m = 0; m < 4; m++) w[(4 * q + m) % KS][(4 * q + m) / KS] = f[m];
    }
    u32x4 lo, hi = u32x4{0, 0, 0, 0};
    load_raw8<BF16>(a.v, (int64_t)b * d + c0, lo, hi);
    float cur[8];
    unpack8<BF16>(lo, hi, sg[h], cur);
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; i++) acc[i] = fmaf(w[KS - 1][i], cur[i], cur[i]);
#pragma unroll
    for (int j = 0; j < KS - 1; j++) {
      const int64_t p = past - (int64_t)(KS - 1 - j) * a.dil;   // history position of tap j
      float hv[8];
      if (p < 0) {
#pragma unroll
        for (int i = 0; i < 8; i++) hv[i] = 0.f;
      } else {
        const int64_t slot = (int64_t)b * R + p % R;
        u32x4 l, u = u32x4{0, 0, 0, 0};
        load_raw8<BF16>(a.v_ring, slot * d + c0, l, u);
        unpack8<BF16>(l, u, a.g_ring[slot * a.hc + h], hv);
      }
#pragma unroll
      for (int i = 0; i < 8; i++) acc[i] = fmaf(w[j][i], hv[i], acc[i]);
    }
    store8(a.out, ((int64_t)b * a.hc + h) * d + c0, BF16, acc);
    if (h == 0) {   // the value row enters the ring (branch 0's lanes cover every channel once)
      if constexpr (BF16) {
        *(u32x4*)((uint16_t*)a.v_ring + new_slot * d + c0) = lo;
      } else {
        *(u32x4*)((float*)a.v_ring + new_slot * d + c0) = lo;
        *(u32x4*)((float*)a.v_ring + new_slot * d + c0 + 4) = hi;
      }
    }
  }
  if (cb == 0 && threadIdx.x == 0) {
    if (a.tok_ring_len > 0) {
      const int32_t id = a.ids[b];
      int32_t x = a.pad_id;
      if (id >= 0 && id < a.vocab) x = a.remap ? a.remap[id] : id;
      a.tok_ring[(int64_t)b * a.tok_ring_len + past % a.tok_ring_len] = x;
    }
    a.n_past[b] = past + 1;
  }
}

template <bool BF16>
hipError_t decode_tail_dispatch(const DecodeTailArgs& a, dim3 grid, hipStream_t s) {
  switch (a.ksize) {
    case 1: k_decode_tail<BF16, 1><<<grid, 64 * a.hc, 0, s>>>(a); break;
    case 2: k_decode_tail<BF16, 2><<<grid, 64 * a.hc, 0, s>>>(a); break;
    case 3: k_decode_tail<BF16, 3><<<grid, 64 * a.hc, 0, s>>>(a); break;
    case 4: k_decode_tail<BF16, 4><<<grid, 64 * a.hc, 0, s>>>(a); break;
    case 5: k_decode_tail<BF16, 5><<<grid, 64 * a.hc, 0, s>>>(a); break;
    case 6: k_decode_tail<BF16, 6><<<grid, 64 * a.hc, 0, s>>>(a); break;
    case 7: k_decode_tail<BF16, 7><<<grid, 64 * a.hc, 0, s>>>(a); break;
    case 8: k_decode_tail<BF16, 8><<<grid, 64 * a.hc, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <bool BF16, int W>
hipError_t conv_dispatch(const ConvArgs& a, dim3 grid, hipStream_t s) {
  switch (a.ksize) {
    case 1: k_conv<BF16, 1, W><<<grid, 256, 0, s>>>(a); break;
    case 2: k_conv<BF16, 2, W><<<grid, 256, 0, s>>>(a); break;
    case 3: k_conv<BF16, 3, W><<<grid, 256, 0, s>>>(a); break;
    case 4: k_conv<BF16, 4, W><<<grid, 256, 0, s>>>(a); break;
    case 5: k_conv<BF16, 5, W><<<grid, 256, 0, s>>>(a); break;
    case 6: k_conv<BF16, 6, W><<<grid, 256, 0, s>>>(a); break;
    case 7: k_conv<BF16, 7, W><<<grid, 256, 0, s>>>(a); break;
    case 8: k_conv<BF16, 8, W><<<grid, 256, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gate(const GateArgs& a, hipStream_t s) {
  const int64_t waves = (int64_t)a.n_tok * a.hc;
  if (waves == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((waves + 3) / 4);
  if (a.bf16)
    k_gate<true><<<blocks, 256, 0, s>>>(a);
  else
    k_gate<false><<<blocks, 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_conv(const ConvArgs& a, hipStream_t s) {
  const int64_t n_tok = (int64_t)a.batch * a.seqlen;
  if (n_tok == 0) return hipSuccess;
  if (a.dil < 1 || a.d % 8 != 0) return hipErrorInvalidValue;
  // one wavefront per (sequence, run of W D positions, residue mod D, 256 channels)
  const int W = conv_walk(n_tok);
  const int64_t runs = (a.seqlen + (int64_t)W * a.dil - 1) / ((int64_t)W * a.dil);
  const int64_t waves = (int64_t)a.batch * runs * a.dil * ((a.d + 255) / 256);
  if ((waves + 3) / 4 > INT32_MAX / 4) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((waves + 3) / 4));
  if (W == 16) return a.bf16 ? conv_dispatch<true, 16>(a, grid, s) : conv_dispatch<false, 16>(a, grid, s);
  return a.bf16 ? conv_dispatch<true, 8>(a, grid, s) : conv_dispatch<false, 8>(a, grid, s);
}

hipError_t launch_decode_tail(const DecodeTailArgs& a, hipStream_t s) {
  if (a.batch == 0) return hipSuccess;
  if (a.ring_len < 1) return hipErrorInvalidValue;
  dim3 grid((unsigned)((a.d / 8 + 63) / 64), (unsigned)a.batch);
  return a.bf16 ? decode_tail_dispatch<true>(a, grid, s) : decode_tail_dispatch<false>(a, grid, s);
}

hipError_t launch_advance(const AdvanceArgs& a, hipStream_t s) {
  if (a.batch == 0 || a.seqlen == 0) return hipSuccess;
  if (a.bf16)
    k_advance<true><<<a.batch, 256, 0, s>>>(a);
  else
    k_advance<false><<<a.batch, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace engram
