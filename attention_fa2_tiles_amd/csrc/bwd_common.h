// Pieces of the attention backward kernels: launch parameters, the
// piecewise distance rule and pair masks, and the LDS addressing of the
// transposing operand reads.
// Everything here has internal linkage in each translation unit.
#pragma once

#include <type_traits>

#include "common.h"

namespace fa {
namespace {

constexpr int kBwdLdsBytes = 160 * 1024;

struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* q2;
  const void* k2;
  const void* dout;
  const float* lse;
  const float* delta;
  // dQ pass only: when delta_out is set, the pass forms each row's Delta from
  // o, dout and dlse itself and writes it there (delta is then unused)
  const void* o;
  const float* dlse;
  float* delta_out;
  void* dq;
  void* dk;
  void* dv;
  void* dq2;
  void* dk2;
  int BH, M, N, nblk;
  float scale2;
  float sm_scale;
  int w;
};

// LSE in log2 units; a row that saw no key (LSE = -inf) gets +inf so that
// exp2(s - lse2) is exactly 0 for it.
__device__ __forceinline__ float lse_to_log2(float lse) {
  return lse == kNegInf ? __builtin_huge_valf() : lse * kLog2e;
}

__device__ __forceinline__ bool pw_near(int dist, int w) { return dist <= w && dist >= -w; }

// Block classification for the piecewise rule, rows [r_lo, r_hi] x keys
// [c_lo, c_hi]: every pair near, every pair far, or mixed.
__device__ __forceinline__ void pw_classify(int r_lo, int r_hi, int c_lo, int c_hi, int pshift, int w,
                                            bool& all_near, bool& all_far) {
  const int dmax = r_hi + pshift - c_lo;
  const int dmin = r_lo + pshift - c_hi;
  all_near = (dmax <= w) && (dmin >= -w);
  all_far = (w < 0) || (dmin > w) || (dmax < -w);
}

// Pair masks of a score tile: none, the causal one (dist >= 0), or one side
// of the piecewise rule (near: |dist| <= w; far: the rest), each side also
// under the causal mask when CAUSAL.  dist = query + (N - M) - key.
constexpr int kMaskNone = 0, kMaskCausal = 1, kMaskNear = 2, kMaskFar = 3;

template <int MODE, bool CAUSAL>
__device__ __forceinline__ bool pair_kept(int dist, int w) {
  if constexpr (MODE == kMaskNone) {
    return true;
  } else if constexpr (MODE == kMaskCausal) {
    return dist >= 0;
  } else {
    const bool side = (MODE == kMaskNear) == pw_near(dist, w);
    return CAUSAL ? side && dist >= 0 : side;
  }
}

// Compile-time choice between two operand sets (registers or accumulators).
template <int SEL, typename A, typename B>
__device__ __forceinline__ auto& pick(A& a, B& b) {
  if constexpr (SEL == 0)
    return a;
  else
    return b;
}

// 16-byte row reads of a DTile: row m, chunk c, as a byte offset.
template <int D>
__device__ __forceinline__ uint32_t row_chunk_ofs(int m, int c) {
  return (uint32_t)((m * D + ((c ^ swz<D>(m)) * 8)) * 2);
}

// Byte offsets of the transposing reads (TrOps::issue_at) of d-tile dt,
// halves s = 0, 1, key/query group 0 of a swap23 DTile.
template <int D>
__device__ __forceinline__ void tr_offsets(const TrLane& tl, uint32_t (&ofs)[D / 32][2]) {
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const int m = swap23(8 * tl.hh + 4 * s2 + tl.r);
      const int d = 32 * dt + tl.dcol;
      ofs[dt][s2] = (uint32_t)((m * D + (((d >> 3) ^ swz<D>(m)) * 8) + (d & 7)) * 2);
    }
  }
}

template <int V>
using ic = std::integral_constant<int, V>;

// Per-lane LDS addresses of the transposing reads: allocation base + the
// lane's offsets (tr_offsets).
template <int D>
struct TrAddr {
  uint32_t lo[D / 32][2];
  __device__ __forceinline__ void init(const void* alloc, const TrLane& tl) {
    uint32_t ofs[D / 32][2];
    tr_offsets<D>(tl, ofs);
    const uint32_t b = lds_addr(alloc);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      lo[dt][0] = b + ofs[dt][0];
      lo[dt][1] = b + ofs[dt][1];
    }
  }
};

template <int D, int NOPS, int OFF>
constexpr bool tr_fits() {
  return OFF + (NOPS - 1) * 16 * D * 2 <= 65535;
}

// Issue the transposing reads of d-tile dt of the tile at byte offset OFF
// inside the LDS allocation (tiles beyond the 16-bit immediate use the
// addresses plus 32 KiB).
template <typename T, int D, int NOPS, int OFF>
__device__ __forceinline__ void tr_issue(TrOps<T, NOPS>& x, const TrAddr<D>& a, int dt) {
  if constexpr (tr_fits<D, NOPS, OFF>()) {
    x.template issue_imm<D, OFF>(a.lo[dt]);
  } else {
    static_assert(tr_fits<D, NOPS, OFF - 32768>(), "tile beyond the 96 KiB reach of the hi addresses");
    const uint32_t hi[2] = {a.lo[dt][0] + 32768u, a.lo[dt][1] + 32768u};
    x.template issue_imm<D, OFF - 32768>(hi);
  }
}

}  // namespace
}  // namespace fa
