// Pieces shared by the bf16 MFMA GEMM kernels (gemm.hip: operands contiguous
// along the reduction axis; gemm_tn.hip: operands stored reduction-major).
#pragma once

#include "engram_internal.h"

namespace engram {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

// Logical tile of a workgroup.  Workgroups are dispatched round-robin over the
// 8 XCDs, so workgroup b runs on XCD b % 8; each XCD is given a contiguous
// range of logical tiles, ordered GROUP m-tiles at a time with the n tiles
// innermost, so the tiles resident on one XCD share a few operand slabs in
// that XCD's L2.
__device__ __forceinline__ void tile_of(int bid, int m_tiles, int n_tiles, int& mt, int& nt) {
  constexpr int GROUP = 4;
  const int total = m_tiles * n_tiles;
  const int xcd = bid & 7, local = bid >> 3;
  const int per = total >> 3, rem = total & 7;
  const int L = xcd < rem ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
  const int span = GROUP * n_tiles;
  const int first_m = (L / span) * GROUP;
  const int gsz = min(m_tiles - first_m, GROUP);
  const int r = L - (L / span) * span;
  mt = first_m + r % gsz;
  nt = r / gsz;
}

// a buffer offset past every resource's record count: the load returns zero
constexpr int kOutOfRange = (int)0x80000000;

// s_waitcnt immediate that waits for vmcnt <= n only (gfx9 encoding: vmcnt
// bits [3:0] and [15:14], expcnt [6:4] and lgkmcnt [11:8] left at their maxima).
constexpr int vmcnt_imm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

}  // namespace
}  // namespace engram
