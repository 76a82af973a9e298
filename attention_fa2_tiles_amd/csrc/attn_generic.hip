// Generic attention (forward, JVP, piecewise, backward) without matrix
// cores: every storage dtype, every head dim the pages allow.
//
// It serves fp32 inputs, which are computed in true fp32 arithmetic end to
// end (no reduced-precision MFMA), and the 16-bit shapes the MFMA kernels do
// not cover: head dim 16, and head dim 256 outside the plain forward.  The
// computation is the same as the MFMA kernels' -- the Triton tutorial's
// online-softmax forward and recompute backward, the JVP recurrences of its
// ENABLE_JVP path, FlagAttention's piecewise score selection -- in fp32, with
// P (and P * Sdot, dS) rounded to the storage dtype before the products that
// consume them, as the 16-bit kernels do (a no-op for fp32).  One wavefront
// owns one query row (forward, dQ) or one key row (dK/dV): lane l holds
// head-dimension elements l, l + 64, ... (E of them; for D < 64 the lanes
// past D hold none) and every dot product is a butterfly reduction across
// the wavefront.  It is correct for any shape, not fast: the large 16-bit
// workloads run on the MFMA kernels.
#include "common.h"
#include "kernels.h"

namespace fa {
namespace {

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

__device__ __forceinline__ bool near_pair(int dist, int w) { return dist <= w && dist >= -w; }

// Head-dimension elements per lane, and whether lane holds element
// lane + 64 e of a row of D (rows of 32 leave the upper half-wave idle).
template <int D>
constexpr int elems() {
  return (D + 63) / 64;
}
template <int D>
__device__ __forceinline__ bool has_col(int lane, int e) {
  return D % 64 == 0 || lane + 64 * e < D;
}
template <int D, typename T>
__device__ __forceinline__ float ld_col(const T* p, int lane, int e) {
  return has_col<D>(lane, e) ? (float)p[lane + 64 * e] : 0.f;
}
template <int D, typename T>
__device__ __forceinline__ void st_col(T* p, int lane, int e, float v) {
  if (has_col<D>(lane, e)) p[lane + 64 * e] = (T)v;
}

// x rounded to the storage dtype and back (the operand precision of the
// 16-bit kernels' second products); exact for fp32.
template <typename T>
__device__ __forceinline__ float rnd(float x) {
  return (float)(T)x;
}

template <int D, int E, typename T>
__device__ __forceinline__ float dot_row(const float (&a)[E], const T* b, int lane) {
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) s += a[e] * ld_col<D>(b, lane, e);
  return wave_sum(s);
}

// One wave per query row.
template <typename T, int D, int VAR>
__global__ __launch_bounds__(256) void fwd_gen_kernel(FwdArgs a, float scale, int64_t rows) {
  constexpr int E = elems<D>();
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int bh = (int)(row / a.M), i = (int)(row % a.M);
  const int pshift = a.N - a.M;
  const int64_t qoff = row * D, kbase = (int64_t)bh * a.N * D;
  const T* Q = (const T*)a.q + qoff;
  float q[E], q2[E], tq[E], acc[E], accg[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    q[e] = ld_col<D>(Q, lane, e);
    q2[e] = VAR == PW ? ld_col<D>((const T*)a.q2 + qoff, lane, e) : 0.f;
    tq[e] = VAR == JVP ? ld_col<D>((const T*)a.tq + qoff, lane, e) : 0.f;
    acc[e] = 0.f;
    accg[e] = 0.f;
  }
  float m = kNegInf, l = 0.f, mu = 0.f;
  const int jend = a.causal ? min(a.N, i + pshift + 1) : a.N;
  for (int j = 0; j < jend; ++j) {
    const int64_t ko = kbase + (int64_t)j * D;
    float s;
    if (VAR == PW && !near_pair(i + pshift - j, a.w))
      s = dot_row<D>(q2, (const T*)a.k2 + ko, lane) * scale;
    else
      s = dot_row<D>(q, (const T*)a.k + ko, lane) * scale;
    const float m_new = fmaxf(m, s);
    const float alpha = expf(m - m_new);  // m = -inf on the first key -> 0
    const float pv = rnd<T>(expf(s - m_new));
    l = alpha * l + pv;
    const T* V = (const T*)a.v + ko;
    if (VAR == JVP) {
      const float sd = dot_row<D>(tq, (const T*)a.k + ko, lane) + dot_row<D>(q, (const T*)a.tk + ko, lane);
      const float ps = pv * sd * scale;
      mu = alpha * mu + ps;
      const float psr = rnd<T>(ps);
      const T* TV = (const T*)a.tv + ko;
#pragma unroll
      for (int e = 0; e < E; ++e) accg[e] = alpha * accg[e] + psr * ld_col<D>(V, lane, e) + pv * ld_col<D>(TV, lane, e);
    }
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = alpha * acc[e] + pv * ld_col<D>(V, lane, e);
    m = m_new;
  }
  const bool has = l > 0.f;
  const float inv = has ? 1.f / l : 0.f;
  T* O = (T*)a.o + qoff;
#pragma unroll
  for (int e = 0; e < E; ++e) st_col<D>(O, lane, e, acc[e] * inv);
  if (lane == 0) a.lse[row] = has ? m + logf(l) : kNegInf;
  if (VAR == JVP) {
    T* TO = (T*)a.to + qoff;
    const float c = mu * inv;
#pragma unroll
    for (int e = 0; e < E; ++e) st_col<D>(TO, lane, e, (accg[e] - c * acc[e]) * inv);
    // LSE tangent: sum_j P_ij Sdot_ij (0 for a row with no visible key)
    if (lane == 0 && a.tlse) a.tlse[row] = c;
  }
}

// One wave per query row: dQ (piecewise: dQ1 and dQ2).
template <typename T, int D, int VAR>
__global__ __launch_bounds__(256) void dq_gen_kernel(BwdArgs a, int64_t rows) {
  constexpr int E = elems<D>();
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int bh = (int)(row / a.M), i = (int)(row % a.M);
  const int pshift = a.N - a.M;
  const int64_t qoff = row * D, kbase = (int64_t)bh * a.N * D;
  float q[E], q2[E], dO[E], dq[E], dq2[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    q[e] = ld_col<D>((const T*)a.q + qoff, lane, e);
    q2[e] = VAR == PW ? ld_col<D>((const T*)a.q2 + qoff, lane, e) : 0.f;
    dO[e] = ld_col<D>((const T*)a.dout + qoff, lane, e);
    dq[e] = 0.f;
    dq2[e] = 0.f;
  }
  const float lse = a.lse[row], dl = a.delta[row];
  const int jend = (lse == kNegInf) ? 0 : (a.causal ? min(a.N, i + pshift + 1) : a.N);
  for (int j = 0; j < jend; ++j) {
    const int64_t ko = kbase + (int64_t)j * D;
    const bool far = VAR == PW && !near_pair(i + pshift - j, a.w);
    const T* Kr = far ? (const T*)a.k2 + ko : (const T*)a.k + ko;
    const float s = dot_row<D>(far ? q2 : q, Kr, lane) * a.sm_scale;
    const float pv = expf(s - lse);
    const float dp = dot_row<D>(dO, (const T*)a.v + ko, lane);
    const float ds = rnd<T>(pv * (dp - dl));
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if (far)
        dq2[e] += ds * ld_col<D>(Kr, lane, e);
      else
        dq[e] += ds * ld_col<D>(Kr, lane, e);
    }
  }
#pragma unroll
  for (int e = 0; e < E; ++e) {
    st_col<D>((T*)a.dq + qoff, lane, e, dq[e] * a.sm_scale);
    if (VAR == PW) st_col<D>((T*)a.dq2 + qoff, lane, e, dq2[e] * a.sm_scale);
  }
}

// One wave per key row: dK, dV (piecewise: dK1, dK2, dV).
template <typename T, int D, int VAR>
__global__ __launch_bounds__(256) void dkdv_gen_kernel(BwdArgs a, int64_t rows) {
  constexpr int E = elems<D>();
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int bh = (int)(row / a.N), j = (int)(row % a.N);
  const int pshift = a.N - a.M;
  const int64_t koff = row * D, qbase = (int64_t)bh * a.M * D, lbase = (int64_t)bh * a.M;
  float k[E], k2[E], v[E], dk[E], dk2[E], dv[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    k[e] = ld_col<D>((const T*)a.k + koff, lane, e);
    k2[e] = VAR == PW ? ld_col<D>((const T*)a.k2 + koff, lane, e) : 0.f;
    v[e] = ld_col<D>((const T*)a.v + koff, lane, e);
    dk[e] = dk2[e] = dv[e] = 0.f;
  }
  const int ibeg = a.causal ? max(0, j - pshift) : 0;
  for (int i = ibeg; i < a.M; ++i) {
    const int64_t qo = qbase + (int64_t)i * D;
    const float lse = a.lse[lbase + i];
    const bool far = VAR == PW && !near_pair(i + pshift - j, a.w);
    const T* Qr = far ? (const T*)a.q2 + qo : (const T*)a.q + qo;
    const float s = dot_row<D>(far ? k2 : k, Qr, lane) * a.sm_scale;
    const float pv = (lse == kNegInf) ? 0.f : expf(s - lse);
    const T* dOr = (const T*)a.dout + qo;
    const float dp = dot_row<D>(v, dOr, lane);
    const float ds = rnd<T>(pv * (dp - a.delta[lbase + i]));
    const float pr = rnd<T>(pv);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      dv[e] += pr * ld_col<D>(dOr, lane, e);
      if (far)
        dk2[e] += ds * ld_col<D>(Qr, lane, e);
      else
        dk[e] += ds * ld_col<D>(Qr, lane, e);
    }
  }
#pragma unroll
  for (int e = 0; e < E; ++e) {
    st_col<D>((T*)a.dv + koff, lane, e, dv[e]);
    st_col<D>((T*)a.dk + koff, lane, e, dk[e] * a.sm_scale);
    if (VAR == PW) st_col<D>((T*)a.dk2 + koff, lane, e, dk2[e] * a.sm_scale);
  }
}

template <typename T, int D>
hipError_t fwd_e(const FwdArgs& a, hipStream_t s) {
  const int64_t rows = (int64_t)a.B * a.H * a.M;
  dim3 grid((unsigned)((rows + 3) / 4)), block(256);
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
  dim3 grid((unsigned)((rows + 3) / 4)), block(256);
  if (a.variant == PW)
    hipLaunchKernelGGL((dq_gen_kernel<T, D, PW>), grid, block, 0, s, a, rows);
  else
    hipLaunchKernelGGL((dq_gen_kernel<T, D, PLAIN>), grid, block, 0, s, a, rows);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t dkdv_e(const BwdArgs& a, hipStream_t s) {
  const int64_t rows = (int64_t)a.B * a.H * a.N;
  dim3 grid((unsigned)((rows + 3) / 4)), block(256);
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
