// Generic attention (forward, JVP, piecewise, backward) without matrix
// cores: every storage dtype, every head dim the pages allow.
//
// It serves fp32 inputs, which are computed in true fp32 arithmetic end to
// end (no reduced-precision MFMA), and the one 16-bit shape the MFMA kernels
// do not cover: piecewise attention at head dim 256.  The
// computation is the same as the MFMA kernels' -- the Triton tutorial's
// online-softmax forward and recompute backward, the JVP recurrences of its
// ENABLE_JVP path, FlagAttention's piecewise score selection -- in fp32, with
// P (and P * Sdot, dS) rounded to the storage dtype before the products that
// consume them, as the 16-bit kernels do (a no-op for fp32).  A group of RL
// lanes (RL = min(D, 64), at least 16) owns one query row (forward, dQ) or
// one key row (dK/dV), so a wavefront holds 64 / RL rows; lane l of a group
// holds head-dimension elements l, l + RL, ..., every dot product is a
// butterfly reduction across the group, and keys (or queries) are taken
// four at a time: four independent reductions, one online-softmax rescale
// per four keys.  Correct for any shape, not fast: the large 16-bit
// workloads run on the MFMA kernels.
#include "common.h"
#include "kernels.h"

namespace fa {
namespace {

__device__ __forceinline__ bool near_pair(int dist, int w) { return dist <= w && dist >= -w; }

// Lanes per row and elements per lane.
template <int D>
constexpr int row_lanes() {
  return D >= 64 ? 64 : (D >= 32 ? 32 : 16);
}
template <int D>
constexpr int per_lane() {
  return D / row_lanes<D>();
}
constexpr int kChunk = 4;  // keys (or queries) per step

// x of the lane that DPP control CTRL names (all rows and banks enabled).
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}

// Sum over the RL lanes of this lane's group, in every lane of the group,
// without the LDS crossbar: the pair and quad partners inside each group of
// four lanes (DPP quad permutations), the quads of a 16-lane row (rotations
// of the row by 4 and 8 lanes), then the partner rows (16 lanes apart) and
// halves (32 apart) by the register swaps across rows.
template <int RL>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(RL == 16 || RL == 32 || RL == 64, "group of 16, 32 or 64 lanes");
  x += dpp<0xB1>(x);   // quad_perm [1, 0, 3, 2]
  x += dpp<0x4E>(x);   // quad_perm [2, 3, 0, 1]
  x += dpp<0x124>(x);  // row_ror:4
  x += dpp<0x128>(x);  // row_ror:8
  if constexpr (RL >= 32) {
    const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(int, x), __builtin_bit_cast(int, x), false, false);
    x = __builtin_bit_cast(float, (int)r[0]) + __builtin_bit_cast(float, (int)r[1]);
  }
  if constexpr (RL >= 64) {
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, x), __builtin_bit_cast(int, x), false, false);
    x = __builtin_bit_cast(float, (int)r[0]) + __builtin_bit_cast(float, (int)r[1]);
  }
  return x;
}
// Maximum / minimum over the whole wavefront (a loop bound its groups share).
__device__ __forceinline__ int wave_max(int x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x = max(x, __shfl_xor(x, off, 64));
  return x;
}
__device__ __forceinline__ int wave_min(int x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x = min(x, __shfl_xor(x, off, 64));
  return x;
}

template <int D, typename T>
__device__ __forceinline__ void load_row(const T* p, int sl, float (&x)[per_lane<D>()]) {
#pragma unroll
  for (int e = 0; e < per_lane<D>(); ++e) x[e] = (float)p[sl + row_lanes<D>() * e];
}
template <int D, typename T>
__device__ __forceinline__ void store_row(T* p, int sl, const float (&x)[per_lane<D>()], float scale) {
#pragma unroll
  for (int e = 0; e < per_lane<D>(); ++e) p[sl + row_lanes<D>() * e] = (T)(x[e] * scale);
}

// x rounded to the storage dtype and back (the operand precision of the
// 16-bit kernels' second products); exact for fp32.
template <typename T>
__device__ __forceinline__ float rnd(float x) {
  return (float)(T)x;
}

// This lane's part of a . (row b) (the caller takes the group sum).
template <int D, typename T>
__device__ __forceinline__ float dot_part(const float (&a)[per_lane<D>()], const T* b, int sl) {
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < per_lane<D>(); ++e) s = fmaf(a[e], (float)b[sl + row_lanes<D>() * e], s);
  return s;
}

// A group per query row.
template <typename T, int D, int VAR>
__global__ __launch_bounds__(256) void fwd_gen_kernel(FwdArgs a, float scale, int64_t rows) {
  constexpr int RL = row_lanes<D>(), E = per_lane<D>(), RPW = 64 / RL;
  const int lane = threadIdx.x & 63, sl = lane % RL;
  const int64_t row_raw = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * RPW + lane / RL;
  const bool valid = row_raw < rows;
  const int64_t row = valid ? row_raw : rows - 1;  // (a clamped row computes, never stores)
  const int bh = (int)(row / a.M), i = (int)(row % a.M);
  const int pshift = a.N - a.M;
  const int64_t qoff = row * D, kbase = (int64_t)bh * a.N * D;
  float q[E], q2[E], tq[E], acc[E], accg[E];
  load_row<D>((const T*)a.q + qoff, sl, q);
#pragma unroll
  for (int e = 0; e < E; ++e) q2[e] = tq[e] = acc[e] = accg[e] = 0.f;
  if (VAR == PW) load_row<D>((const T*)a.q2 + qoff, sl, q2);
  if (VAR == JVP) load_row<D>((const T*)a.tq + qoff, sl, tq);
  float m = kNegInf, l = 0.f, mu = 0.f;
  const int jend = a.causal ? max(0, min(a.N, i + pshift + 1)) : a.N;
  const int jmax = wave_max(jend);
  for (int j0 = 0; j0 < jmax; j0 += kChunk) {
    float sc[kChunk], sd[kChunk];
    const T* vr[kChunk];
    const T* tvr[kChunk];
#pragma unroll
    for (int c = 0; c < kChunk; ++c) {
      const int j = j0 + c;
      const int jc = j < a.N ? j : a.N - 1;  // (addresses stay inside the keys)
      const int64_t ko = kbase + (int64_t)jc * D;
      vr[c] = (const T*)a.v + ko;
      tvr[c] = VAR == JVP ? (const T*)a.tv + ko : vr[c];
      const bool far = VAR == PW && !near_pair(i + pshift - j, a.w);
      const float part = far ? dot_part<D>(q2, (const T*)a.k2 + ko, sl) : dot_part<D>(q, (const T*)a.k + ko, sl);
      sc[c] = group_sum<RL>(part);
      sd[c] = 0.f;
      if (VAR == JVP)
        sd[c] = group_sum<RL>(dot_part<D>(tq, (const T*)a.k + ko, sl) + dot_part<D>(q, (const T*)a.tk + ko, sl));
      sc[c] = j < jend ? sc[c] * scale : kNegInf;
    }
    float m_new = m;
#pragma unroll
    for (int c = 0; c < kChunk; ++c) m_new = fmaxf(m_new, sc[c]);
    if (m_new == kNegInf) continue;  // nothing visible yet in this row
    const float alpha = expf(m - m_new);  // m = -inf -> 0
    l *= alpha;
    mu *= alpha;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      acc[e] *= alpha;
      accg[e] *= alpha;
    }
#pragma unroll
    for (int c = 0; c < kChunk; ++c) {
      const float pv = rnd<T>(expf(sc[c] - m_new));  // a masked key: exp(-inf) = 0
      l += pv;
      if (VAR == JVP) {
        const float ps = sc[c] == kNegInf ? 0.f : pv * sd[c] * scale;
        mu += ps;
        const float psr = rnd<T>(ps);
#pragma unroll
        for (int e = 0; e < E; ++e)
          accg[e] += psr * (float)vr[c][sl + RL * e] + pv * (float)tvr[c][sl + RL * e];
      }
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] = fmaf(pv, (float)vr[c][sl + RL * e], acc[e]);
    }
    m = m_new;
  }
  if (!valid) return;
  const bool has = l > 0.f;
  const float inv = has ? 1.f / l : 0.f;
  store_row<D>((T*)a.o + qoff, sl, acc, inv);
  if (sl == 0) a.lse[row] = has ? m + logf(l) : kNegInf;
  if (VAR == JVP) {
    const float c = mu * inv;
    float tv[E];
#pragma unroll
    for (int e = 0; e < E; ++e) tv[e] = accg[e] - c * acc[e];
    store_row<D>((T*)a.to + qoff, sl, tv, inv);
    // LSE tangent: sum_j P_ij Sdot_ij (0 for a row with no visible key)
    if (sl == 0 && a.tlse) a.tlse[row] = c;
  }
}

// A group per query row: dQ (piecewise: dQ1 and dQ2).
template <typename T, int D, int VAR>
__global__ __launch_bounds__(256) void dq_gen_kernel(BwdArgs a, int64_t rows) {
  constexpr int RL = row_lanes<D>(), E = per_lane<D>(), RPW = 64 / RL;
  const int lane = threadIdx.x & 63, sl = lane % RL;
  const int64_t row_raw = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * RPW + lane / RL;
  const bool valid = row_raw < rows;
  const int64_t row = valid ? row_raw : rows - 1;
  const int bh = (int)(row / a.M), i = (int)(row % a.M);
  const int pshift = a.N - a.M;
  const int64_t qoff = row * D, kbase = (int64_t)bh * a.N * D;
  float q[E], q2[E], dO[E], dq[E], dq2[E];
  load_row<D>((const T*)a.q + qoff, sl, q);
  load_row<D>((const T*)a.dout + qoff, sl, dO);
#pragma unroll
  for (int e = 0; e < E; ++e) q2[e] = dq[e] = dq2[e] = 0.f;
  if (VAR == PW) load_row<D>((const T*)a.q2 + qoff, sl, q2);
  const float lse = a.lse[row], dl = a.delta[row];
  const int jend = (lse == kNegInf) ? 0 : (a.causal ? max(0, min(a.N, i + pshift + 1)) : a.N);
  const int jmax = wave_max(jend);
  for (int j0 = 0; j0 < jmax; j0 += kChunk) {
    float ds[kChunk];
    bool far[kChunk];
    const T* kr[kChunk];
#pragma unroll
    for (int c = 0; c < kChunk; ++c) {
      const int j = j0 + c;
      const int jc = j < a.N ? j : a.N - 1;
      const int64_t ko = kbase + (int64_t)jc * D;
      far[c] = VAR == PW && !near_pair(i + pshift - j, a.w);
      kr[c] = far[c] ? (const T*)a.k2 + ko : (const T*)a.k + ko;
      const float s = group_sum<RL>(dot_part<D>(far[c] ? q2 : q, kr[c], sl)) * a.sm_scale;
      const float dp = group_sum<RL>(dot_part<D>(dO, (const T*)a.v + ko, sl));
      ds[c] = j < jend ? rnd<T>(expf(s - lse) * (dp - dl)) : 0.f;
    }
#pragma unroll
    for (int c = 0; c < kChunk; ++c) {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float kv = (float)kr[c][sl + RL * e];
        if (VAR == PW && far[c])
          dq2[e] = fmaf(ds[c], kv, dq2[e]);
        else
          dq[e] = fmaf(ds[c], kv, dq[e]);
      }
    }
  }
  if (!valid) return;
  store_row<D>((T*)a.dq + qoff, sl, dq, a.sm_scale);
  if (VAR == PW) store_row<D>((T*)a.dq2 + qoff, sl, dq2, a.sm_scale);
}

// A group per key row: dK, dV (piecewise: dK1, dK2, dV).
template <typename T, int D, int VAR>
__global__ __launch_bounds__(256) void dkdv_gen_kernel(BwdArgs a, int64_t rows) {
  constexpr int RL = row_lanes<D>(), E = per_lane<D>(), RPW = 64 / RL;
  const int lane = threadIdx.x & 63, sl = lane % RL;
  const int64_t row_raw = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * RPW + lane / RL;
  const bool valid = row_raw < rows;
  const int64_t row = valid ? row_raw : rows - 1;
  const int bh = (int)(row / a.N), j = (int)(row % a.N);
  const int pshift = a.N - a.M;
  const int64_t koff = row * D, qbase = (int64_t)bh * a.M * D, lbase = (int64_t)bh * a.M;
  float k[E], k2[E], v[E], dk[E], dk2[E], dv[E];
  load_row<D>((const T*)a.k + koff, sl, k);
  load_row<D>((const T*)a.v + koff, sl, v);
#pragma unroll
  for (int e = 0; e < E; ++e) k2[e] = dk[e] = dk2[e] = dv[e] = 0.f;
  if (VAR == PW) load_row<D>((const T*)a.k2 + koff, sl, k2);
  const int ibeg = a.causal ? min(a.M, max(0, j - pshift)) : 0;
  const int imin = wave_min(ibeg) / kChunk * kChunk;
  for (int i0 = imin; i0 < a.M; i0 += kChunk) {
    float ds[kChunk], pr[kChunk];
    bool far[kChunk];
    const T* qr[kChunk];
    const T* dor[kChunk];
#pragma unroll
    for (int c = 0; c < kChunk; ++c) {
      const int i = i0 + c;
      const int ii = i < a.M ? i : a.M - 1;
      const int64_t qo = qbase + (int64_t)ii * D;
      const float lse = a.lse[lbase + ii];
      far[c] = VAR == PW && !near_pair(i + pshift - j, a.w);
      qr[c] = far[c] ? (const T*)a.q2 + qo : (const T*)a.q + qo;
      dor[c] = (const T*)a.dout + qo;
      const float s = group_sum<RL>(dot_part<D>(far[c] ? k2 : k, qr[c], sl)) * a.sm_scale;
      const float dp = group_sum<RL>(dot_part<D>(v, dor[c], sl));
      const bool on = i >= ibeg && i < a.M && lse != kNegInf;
      const float pv = on ? expf(s - lse) : 0.f;
      ds[c] = rnd<T>(pv * (dp - a.delta[lbase + ii]));
      pr[c] = rnd<T>(pv);
    }
#pragma unroll
    for (int c = 0; c < kChunk; ++c) {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        dv[e] = fmaf(pr[c], (float)dor[c][sl + RL * e], dv[e]);
        const float qv = (float)qr[c][sl + RL * e];
        if (VAR == PW && far[c])
          dk2[e] = fmaf(ds[c], qv, dk2[e]);
        else
          dk[e] = fmaf(ds[c], qv, dk[e]);
      }
    }
  }
  if (!valid) return;
  store_row<D>((T*)a.dv + koff, sl, dv, 1.f);
  store_row<D>((T*)a.dk + koff, sl, dk, a.sm_scale);
  if (VAR == PW) store_row<D>((T*)a.dk2 + koff, sl, dk2, a.sm_scale);
}

template <typename T, int D>
hipError_t fwd_e(const FwdArgs& a, hipStream_t s) {
  const int64_t rows = (int64_t)a.B * a.H * a.M;
  constexpr int RPB = 4 * (64 / row_lanes<D>());  // rows per workgroup
  dim3 grid((unsigned)((rows + RPB - 1) / RPB)), block(256);
  switch (a.variant) {
    case PLAIN: hipLaunchKernelGGL((fwd_gen_kernel<T, D, PLAIN>), grid, block, 0, s, a, a.sm_scale, rows); break;
    case JVP: hipLaunchKernelGGL((fwd_gen_kernel<T, D, JVP>), grid, block, 0, s, a, a.sm_scale, rows); break;
    case PW: hipLaunchKernelGGL((fwd_gen_kernel<T, D, PW>), grid, block, 0, s, a, a.sm_scale, rows); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T, int D>
hipError_t dq_e(const BwdArgs& a, hipStream_t s) {
  const int64_t rows = (int64_t)a.B * a.H * a.M;
  constexpr int RPB = 4 * (64 / row_lanes<D>());
  dim3 grid((unsigned)((rows + RPB - 1) / RPB)), block(256);
  if (a.variant == PW)
    hipLaunchKernelGGL((dq_gen_kernel<T, D, PW>), grid, block, 0, s, a, rows);
  else
    hipLaunchKernelGGL((dq_gen_kernel<T, D, PLAIN>), grid, block, 0, s, a, rows);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t dkdv_e(const BwdArgs& a, hipStream_t s) {
  const int64_t rows = (int64_t)a.B * a.H * a.N;
  constexpr int RPB = 4 * (64 / row_lanes<D>());
  dim3 grid((unsigned)((rows + RPB - 1) / RPB)), block(256);
  if (a.variant == PW)
    hipLaunchKernelGGL((dkdv_gen_kernel<T, D, PW>), grid, block, 0, s, a, rows);
  else
    hipLaunchKernelGGL((dkdv_gen_kernel<T, D, PLAIN>), grid, block, 0, s, a, rows);
  return hipGetLastError();
}

// Head dim and storage dtype -> instantiation.
template <template <typename, int> class L, typename A>
hipError_t by_d_t(const A& a, hipStream_t s) {
  auto by_d = [&](auto tag) -> hipError_t {
    using T = decltype(tag);
    switch (a.D) {
      case 16: return L<T, 16>::run(a, s);
      case 32: return L<T, 32>::run(a, s);
      case 64: return L<T, 64>::run(a, s);
      case 128: return L<T, 128>::run(a, s);
      case 256: return L<T, 256>::run(a, s);
    }
    return hipErrorInvalidValue;
  };
  if (a.dtype == 0) return by_d(float{});
  if (a.dtype == 1) return by_d(_Float16{});
  if (a.dtype == 2) return by_d(__bf16{});
  return hipErrorInvalidValue;
}

template <typename T, int D>
struct FwdL {
  static hipError_t run(const FwdArgs& a, hipStream_t s) { return fwd_e<T, D>(a, s); }
};
template <typename T, int D>
struct DqL {
  static hipError_t run(const BwdArgs& a, hipStream_t s) { return dq_e<T, D>(a, s); }
};
template <typename T, int D>
struct DkdvL {
  static hipError_t run(const BwdArgs& a, hipStream_t s) { return dkdv_e<T, D>(a, s); }
};

}  // namespace

hipError_t launch_attn_fwd_generic(const FwdArgs& a, hipStream_t s) { return by_d_t<FwdL>(a, s); }
hipError_t launch_attn_dq_generic(const BwdArgs& a, hipStream_t s) { return by_d_t<DqL>(a, s); }
hipError_t launch_attn_dkdv_generic(const BwdArgs& a, hipStream_t s) { return by_d_t<DkdvL>(a, s); }

}  // namespace fa
