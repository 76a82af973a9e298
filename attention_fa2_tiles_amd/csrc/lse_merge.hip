// N-way online-softmax merge of (y_s, lse_s) partials, forward and backward.
//
// What is computed: the combine step of the block-residual merge
// (flash_attn_res 0.1.11, slop/backward_phase_2.txt: reference_forward),
// with S inputs whose logits are given instead of one of two being computed
// from x and the pseudo-query.  It is how attention partials over disjoint
// key ranges (split-KV, ring partials, the O/LSE pairs of fa_fwd) combine
// into attention over all keys.  Per row:
//   lse = log sum_s e^(lse_s),   y = sum_s w_s y_s,   w_s = e^(lse_s - lse)
// backward for <gy, y> + <gl, lse>:
//   gy_s = w_s gy,   glse_s = w_s (gl + gy . (y_s - y))
// A row whose logits are all -inf merges to y = 0, lse = -inf, and gets zero
// gradients.
//
// CDNA4 mapping: bandwidth-bound, no MFMA.  LPR lanes (a power of two) own
// one row, each holding CPL 16-byte chunks of 8 elements, interleaved so
// that the RPW = 64 / LPR rows of a wavefront are read and written as one
// contiguous run per (input, chunk) instruction.  The S logits of a row are
// read by its lanes directly (they hit the cache after the first lane).  The
// backward keeps y and gy in registers, forms the dot products
// gy . (y_s - y), reduces them over the row's lanes with butterflies, and
// writes gy_s and glse_s.  Rows of at most 64 chunks with at most 8 partials
// (the split-KV combine of attention heads) take kernels that issue every
// load of the row first and keep the S chunks in registers; wider rows or
// more partials read each y_s a second time for the dot product (a cache hit
// for rows of a few KiB, mostly).  Every row is owned by one group of lanes,
// so nothing is shared between wavefronts and results do not depend on
// timing.
#include "common.h"
#include "kernels.h"

namespace fa {
namespace {

constexpr int kLmWaves = 4;  // wavefronts per workgroup

template <typename T>
struct alignas(16) Ch8 {
  T e[8];
};

// 8 elements; stores as 16-byte vectors with the non-temporal hint (the
// outputs are written once; measured 5% faster forward, 14% faster
// backward).  Loads keep the default policy: the backward reads each input
// chunk twice, and with the hint on the loads both passes were 15% slower.
template <typename T>
__device__ __forceinline__ void load8(const T* p, float (&f)[8]) {
  const Ch8<T> c = *reinterpret_cast<const Ch8<T>*>(p);
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = (float)c.e[i];
}

template <typename T>
__device__ __forceinline__ void store8(T* p, const float (&f)[8]) {
  constexpr int NV = (int)sizeof(Ch8<T>) / 16;
  Ch8<T> c;
#pragma unroll
  for (int i = 0; i < 8; ++i) c.e[i] = (T)f[i];
  u32x4 raw[NV];
  __builtin_memcpy(raw, &c, sizeof(c));
#pragma unroll
  for (int v = 0; v < NV; ++v) __builtin_nontemporal_store(raw[v], reinterpret_cast<u32x4*>(p) + v);
}

// Row maximum and normaliser of the S logits of one row (logits at
// lses[s * rows + row]).  Z = 0 marks a row whose logits are all -inf.
__device__ __forceinline__ void row_stats(const float* __restrict__ lses, int S, int64_t rows, int64_t row,
                                          float& mx, float& Z) {
  mx = -__builtin_huge_valf();
  for (int s = 0; s < S; ++s) mx = fmaxf(mx, lses[s * rows + row]);
  Z = 0.f;
  if (mx == -__builtin_huge_valf()) return;
  for (int s = 0; s < S; ++s) Z += __expf(lses[s * rows + row] - mx);
}

template <typename T, int LPR, int CPL>
__global__ __launch_bounds__(64 * kLmWaves) void lse_merge_fwd_kernel(const T* __restrict__ ys,
                                                                      const float* __restrict__ lses,
                                                                      T* __restrict__ y, float* __restrict__ lse,
                                                                      int S, int64_t rows, int D) {
  constexpr int RPW = 64 / LPR;
  const int lane = threadIdx.x & 63;
  const int64_t row = ((int64_t)blockIdx.x * kLmWaves + (threadIdx.x >> 6)) * RPW + lane / LPR;
  const int sub = lane % LPR;
  const int C = D / 8;
  if (row >= rows) return;
  float mx, Z;
  row_stats(lses, S, rows, row, mx, Z);
  float acc[CPL][8];
#pragma unroll
  for (int c = 0; c < CPL; ++c)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[c][i] = 0.f;
  if (Z > 0.f) {
    const float inv = 1.f / Z;
#pragma unroll 4
    for (int s = 0; s < S; ++s) {
      const float w = __expf(lses[s * rows + row] - mx) * inv;
      const T* src = ys + (s * rows + row) * (int64_t)D;
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const int ch = sub + c * LPR;
        if (ch < C) {
          float f[8];
          load8(src + ch * 8, f);
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[c][i] = fmaf(w, f[i], acc[c][i]);
        }
      }
    }
  }
  T* dst = y + row * (int64_t)D;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int ch = sub + c * LPR;
    if (ch < C) store8(dst + ch * 8, acc[c]);
  }
  if (sub == 0) lse[row] = Z > 0.f ? mx + __logf(Z) : -__builtin_huge_valf();
}

// The forward for rows of at most 64 chunks and at most SM <= 8 partials:
// every load of the row is issued before any arithmetic (the general kernel
// above loads, waits and accumulates one partial at a time).  Same
// operations in the same order, so the results are bitwise equal.
template <typename T, int LPR, int SM>
__global__ __launch_bounds__(64 * kLmWaves) void lse_merge_fwd_small_kernel(const T* __restrict__ ys,
                                                                            const float* __restrict__ lses,
                                                                            T* __restrict__ y, float* __restrict__ lse,
                                                                            int S, int64_t rows, int D) {
  constexpr int RPW = 64 / LPR;
  const int lane = threadIdx.x & 63;
  const int64_t row = ((int64_t)blockIdx.x * kLmWaves + (threadIdx.x >> 6)) * RPW + lane / LPR;
  const int sub = lane % LPR;
  const bool has_ch = sub < D / 8;
  if (row >= rows) return;
  float ls[SM];
  Ch8<T> cy[SM];
#pragma unroll
  for (int s = 0; s < SM; ++s) {
    ls[s] = s < S ? lses[s * rows + row] : -__builtin_huge_valf();
    if (s < S && has_ch) cy[s] = *reinterpret_cast<const Ch8<T>*>(ys + (s * rows + row) * (int64_t)D + sub * 8);
  }
  float mx = -__builtin_huge_valf();
#pragma unroll
  for (int s = 0; s < SM; ++s)
    if (s < S) mx = fmaxf(mx, ls[s]);
  const bool has = mx != -__builtin_huge_valf();
  float Z = 0.f;
  if (has) {
#pragma unroll
    for (int s = 0; s < SM; ++s)
      if (s < S) Z += __expf(ls[s] - mx);
  }
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  if (has && has_ch) {
    const float inv = 1.f / Z;
#pragma unroll
    for (int s = 0; s < SM; ++s)
      if (s < S) {
        const float w = __expf(ls[s] - mx) * inv;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = fmaf(w, (float)cy[s].e[i], acc[i]);
      }
  }
  if (has_ch) store8(y + row * (int64_t)D + sub * 8, acc);
  if (sub == 0) lse[row] = has ? mx + __logf(Z) : -__builtin_huge_valf();
}

template <int LPR>
__device__ __forceinline__ float row_sum(float x) {
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

template <typename T, int LPR, int CPL>
__global__ __launch_bounds__(64 * kLmWaves) void lse_merge_bwd_kernel(
    const T* __restrict__ ys, const float* __restrict__ lses, const T* __restrict__ gy,
    const float* __restrict__ gl, T* __restrict__ gys, float* __restrict__ glses, int S, int64_t rows, int D) {
  constexpr int RPW = 64 / LPR;
  const int lane = threadIdx.x & 63;
  const int64_t row = ((int64_t)blockIdx.x * kLmWaves + (threadIdx.x >> 6)) * RPW + lane / LPR;
  const int sub = lane % LPR;
  const int C = D / 8;
  // A row's lanes are consecutive and leave together, so the butterflies
  // below only ever combine lanes of one live row.
  if (row >= rows) return;
  float mx, Z;
  row_stats(lses, S, rows, row, mx, Z);
  const bool has = Z > 0.f;
  const float inv = has ? 1.f / Z : 0.f;
  // merged y (fp32, as the forward forms it) and gy, in registers
  float yv[CPL][8], g[CPL][8];
#pragma unroll
  for (int c = 0; c < CPL; ++c)
#pragma unroll
    for (int i = 0; i < 8; ++i) yv[c][i] = 0.f;
  if (has) {
#pragma unroll 4
    for (int s = 0; s < S; ++s) {
      const float w = __expf(lses[s * rows + row] - mx) * inv;
      const T* src = ys + (s * rows + row) * (int64_t)D;
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const int ch = sub + c * LPR;
        if (ch < C) {
          float f[8];
          load8(src + ch * 8, f);
#pragma unroll
          for (int i = 0; i < 8; ++i) yv[c][i] = fmaf(w, f[i], yv[c][i]);
        }
      }
    }
  }
  const T* gsrc = gy + row * (int64_t)D;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int ch = sub + c * LPR;
    if (ch < C)
      load8(gsrc + ch * 8, g[c]);
    else
#pragma unroll
      for (int i = 0; i < 8; ++i) g[c][i] = 0.f;
  }
  const float glr = gl ? gl[row] : 0.f;
  for (int s = 0; s < S; ++s) {
    const float w = has ? __expf(lses[s * rows + row] - mx) * inv : 0.f;
    const T* src = ys + (s * rows + row) * (int64_t)D;
    T* dst = gys + (s * rows + row) * (int64_t)D;
    float dot = 0.f;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int ch = sub + c * LPR;
      if (ch < C) {
        float f[8], o[8];
        if (has) {
          load8(src + ch * 8, f);
#pragma unroll
          for (int i = 0; i < 8; ++i) dot = fmaf(g[c][i], f[i] - yv[c][i], dot);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] = w * g[c][i];
        store8(dst + ch * 8, o);
      }
    }
    dot = row_sum<LPR>(dot);
    if (sub == 0) glses[s * rows + row] = w * (glr + dot);
  }
}

// The backward for rows of at most 64 chunks (one chunk per lane) and at
// most SM <= 8 partials: every load of the row (the S chunks, gy, the
// logits) is issued before any arithmetic, the chunks stay in registers for
// both the merged y and the dot products (no second read), and the S
// butterflies run side by side.  Same operations in the same order as
// lse_merge_bwd_kernel, so the results are bitwise equal.
template <typename T, int LPR, int SM>
__global__ __launch_bounds__(64 * kLmWaves) void lse_merge_bwd_small_kernel(
    const T* __restrict__ ys, const float* __restrict__ lses, const T* __restrict__ gy,
    const float* __restrict__ gl, T* __restrict__ gys, float* __restrict__ glses, int S, int64_t rows, int D) {
  constexpr int RPW = 64 / LPR;
  const int lane = threadIdx.x & 63;
  const int64_t row = ((int64_t)blockIdx.x * kLmWaves + (threadIdx.x >> 6)) * RPW + lane / LPR;
  const int sub = lane % LPR;
  const bool has_ch = sub < D / 8;
  if (row >= rows) return;
  float ls[SM];
  Ch8<T> cy[SM], cg;
#pragma unroll
  for (int s = 0; s < SM; ++s) {
    ls[s] = s < S ? lses[s * rows + row] : -__builtin_huge_valf();
    if (s < S && has_ch) cy[s] = *reinterpret_cast<const Ch8<T>*>(ys + (s * rows + row) * (int64_t)D + sub * 8);
  }
  if (has_ch) cg = *reinterpret_cast<const Ch8<T>*>(gy + row * (int64_t)D + sub * 8);
  const float glr = gl ? gl[row] : 0.f;
  float mx = -__builtin_huge_valf();
#pragma unroll
  for (int s = 0; s < SM; ++s)
    if (s < S) mx = fmaxf(mx, ls[s]);
  const bool has = mx != -__builtin_huge_valf();
  float Z = 0.f;
  if (has) {
#pragma unroll
    for (int s = 0; s < SM; ++s)
      if (s < S) Z += __expf(ls[s] - mx);
  }
  const float inv = has ? 1.f / Z : 0.f;
  float w[SM], g[8], yv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    g[i] = has_ch ? (float)cg.e[i] : 0.f;
    yv[i] = 0.f;
  }
#pragma unroll
  for (int s = 0; s < SM; ++s) w[s] = (has && s < S) ? __expf(ls[s] - mx) * inv : 0.f;
  if (has && has_ch) {
#pragma unroll
    for (int s = 0; s < SM; ++s)
      if (s < S) {
#pragma unroll
        for (int i = 0; i < 8; ++i) yv[i] = fmaf(w[s], (float)cy[s].e[i], yv[i]);
      }
  }
  float dot[SM];
#pragma unroll
  for (int s = 0; s < SM; ++s) {
    dot[s] = 0.f;
    if (has && has_ch && s < S) {
#pragma unroll
      for (int i = 0; i < 8; ++i) dot[s] = fmaf(g[i], (float)cy[s].e[i] - yv[i], dot[s]);
    }
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) {
#pragma unroll
    for (int s = 0; s < SM; ++s) dot[s] += __shfl_xor(dot[s], off, 64);
  }
#pragma unroll
  for (int s = 0; s < SM; ++s) {
    if (s >= S) continue;
    if (has_ch) {
      float o[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] = w[s] * g[i];
      store8(gys + (s * rows + row) * (int64_t)D + sub * 8, o);
    }
    if (sub == 0) glses[s * rows + row] = w[s] * (glr + dot[s]);
  }
}

// Lanes per row and chunks per lane for rows of C chunks: rows of at most
// 64 chunks take the next power of two of lanes and one chunk each; wider
// rows take a whole wavefront and up to 8 chunks per lane.
template <typename T, bool BWD>
hipError_t launch_lm(const LseMergeArgs& a, hipStream_t s) {
  const int C = a.D / 8;
  int lpr = 1;
  while (lpr < C && lpr < 64) lpr *= 2;
  const int cpl = (C + lpr - 1) / lpr;
  const int64_t rpw = 64 / lpr;
  const int64_t rows_per_block = rpw * kLmWaves;
  dim3 grid((unsigned)((a.rows + rows_per_block - 1) / rows_per_block)), block(64 * kLmWaves);
  if constexpr (!BWD) {
    if (cpl == 1 && a.S <= 8) {
#define FA_LM_SMALL(L)                                                                                      \
  if (lpr == L) {                                                                                           \
    if (a.S <= 2)                                                                                           \
      hipLaunchKernelGGL((lse_merge_fwd_small_kernel<T, L, 2>), grid, block, 0, s, (const T*)a.ys, a.lses,  \
                         (T*)a.y, a.lse, a.S, a.rows, a.D);                                                 \
    else if (a.S <= 4)                                                                                      \
      hipLaunchKernelGGL((lse_merge_fwd_small_kernel<T, L, 4>), grid, block, 0, s, (const T*)a.ys, a.lses,  \
                         (T*)a.y, a.lse, a.S, a.rows, a.D);                                                 \
    else                                                                                                    \
      hipLaunchKernelGGL((lse_merge_fwd_small_kernel<T, L, 8>), grid, block, 0, s, (const T*)a.ys, a.lses,  \
                         (T*)a.y, a.lse, a.S, a.rows, a.D);                                                 \
    return hipGetLastError();                                                                               \
  }
      FA_LM_SMALL(1)
      FA_LM_SMALL(2)
      FA_LM_SMALL(4)
      FA_LM_SMALL(8)
      FA_LM_SMALL(16)
      FA_LM_SMALL(32)
      FA_LM_SMALL(64)
#undef FA_LM_SMALL
    }
  }
  if constexpr (BWD) {
    if (cpl == 1 && a.S <= 8) {
#define FA_LM_SMALL(L)                                                                                      \
  if (lpr == L) {                                                                                           \
    if (a.S <= 2)                                                                                           \
      hipLaunchKernelGGL((lse_merge_bwd_small_kernel<T, L, 2>), grid, block, 0, s, (const T*)a.ys, a.lses,  \
                         (const T*)a.gy, a.gl, (T*)a.gys, a.glses, a.S, a.rows, a.D);                       \
    else if (a.S <= 4)                                                                                      \
      hipLaunchKernelGGL((lse_merge_bwd_small_kernel<T, L, 4>), grid, block, 0, s, (const T*)a.ys, a.lses,  \
                         (const T*)a.gy, a.gl, (T*)a.gys, a.glses, a.S, a.rows, a.D);                       \
    else                                                                                                    \
      hipLaunchKernelGGL((lse_merge_bwd_small_kernel<T, L, 8>), grid, block, 0, s, (const T*)a.ys, a.lses,  \
                         (const T*)a.gy, a.gl, (T*)a.gys, a.glses, a.S, a.rows, a.D);                       \
    return hipGetLastError();                                                                               \
  }
      FA_LM_SMALL(1)
      FA_LM_SMALL(2)
      FA_LM_SMALL(4)
      FA_LM_SMALL(8)
      FA_LM_SMALL(16)
      FA_LM_SMALL(32)
      FA_LM_SMALL(64)
#undef FA_LM_SMALL
    }
  }
#define FA_LM_CASE(L, CP)                                                                                   \
  if (lpr == L && cpl <= CP) {                                                                              \
    if constexpr (BWD)                                                                                      \
      hipLaunchKernelGGL((lse_merge_bwd_kernel<T, L, CP>), grid, block, 0, s, (const T*)a.ys, a.lses,       \
                         (const T*)a.gy, a.gl, (T*)a.gys, a.glses, a.S, a.rows, a.D);                       \
    else                                                                                                    \
      hipLaunchKernelGGL((lse_merge_fwd_kernel<T, L, CP>), grid, block, 0, s, (const T*)a.ys, a.lses,       \
                         (T*)a.y, a.lse, a.S, a.rows, a.D);                                                 \
    return hipGetLastError();                                                                               \
  }
  FA_LM_CASE(1, 1)
  FA_LM_CASE(2, 1)
  FA_LM_CASE(4, 1)
  FA_LM_CASE(8, 1)
  FA_LM_CASE(16, 1)
  FA_LM_CASE(32, 1)
  FA_LM_CASE(64, 1)
  FA_LM_CASE(64, 2)
  FA_LM_CASE(64, 4)
  FA_LM_CASE(64, 8)
#undef FA_LM_CASE
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_lse_merge_fwd(const LseMergeArgs& a, hipStream_t s) {
  if (a.dtype == 0) return launch_lm<float, false>(a, s);
  if (a.dtype == 1) return launch_lm<_Float16, false>(a, s);
  if (a.dtype == 2) return launch_lm<__bf16, false>(a, s);
  return hipErrorInvalidValue;
}

hipError_t launch_lse_merge_bwd(const LseMergeArgs& a, hipStream_t s) {
  if (a.dtype == 0) return launch_lm<float, true>(a, s);
  if (a.dtype == 1) return launch_lm<_Float16, true>(a, s);
  if (a.dtype == 2) return launch_lm<__bf16, true>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace fa
