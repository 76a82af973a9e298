// Block-residual two-way online-softmax merge (forward and backward).
//
// What is computed (flash_attn_res 0.1.11, slop/backward_phase_2.txt:
// reference_forward and the phase-2 merge backward kernel), per row of
// x, y0 ([rows, D]):
//   rho = (mean x^2 + eps)^-1/2,  l1 = rho (x . q),  m = max(l0, l1)
//   a = e^(l0-m)/Z,  b = e^(l1-m)/Z,  Z = e^(l0-m) + e^(l1-m)
//   y = a y0 + b x,  lse = m + log Z
// backward, with s = gy . (y0 - x):
//   gy0 = a gy,  gl0 = a gl + a b s,  gl1 = b gl - a b s
//   gx  = b gy + gl1 (rho q - (x.q) rho^3 x / D),   gq = sum_rows gl1 rho x
//
// CDNA4 mapping: the merge is bandwidth-bound (about one flop per byte), so
// there is no MFMA.  One wavefront owns one row at a time; each lane holds
// D/64 elements as 16-byte chunks (lane-interleaved, so every load and store
// instruction moves 1 KiB of contiguous memory).  The row stays in registers
// between the reductions (x.x, x.q, gy.(y0-x): butterfly shuffles across the
// wavefront) and the output pass, so every input byte is read from HBM once.
// The pseudo-query q is loaded once per wavefront and reused for all of its
// rows (grid-stride loop).  gq is reduced deterministically: each wavefront
// accumulates its rows in registers, the 8 wavefronts of a workgroup are
// summed in LDS in fixed order into one partial row per workgroup, and a
// second kernel adds the partial rows in index order.  The page's kernel
// uses relaxed float atomics there instead, whose result depends on timing.
#include "common.h"
#include "kernels.h"

namespace fa {
namespace {

constexpr int kWPB = 8;           // wavefronts per workgroup
constexpr int kNTM = 64 * kWPB;
constexpr int kMaxWG = 512;       // cap on workgroups (= gq partial rows)

template <typename T>
struct alignas(16) Chunk {
  T e[8];
};

template <typename T>
__device__ __forceinline__ void to_f32(const Chunk<T>& c, float (&f)[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = (float)c.e[i];
}

template <typename T>
__device__ __forceinline__ Chunk<T> from_f32(const float (&f)[8]) {
  Chunk<T> c;
#pragma unroll
  for (int i = 0; i < 8; ++i) c.e[i] = (T)f[i];
  return c;
}

__device__ __forceinline__ float wsum(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

struct Mix {
  float rho, xq, alpha, beta, m, Z;
};

__device__ __forceinline__ Mix mix(float sxx, float sxq, float l0, int D, float eps) {
  Mix r;
  r.rho = 1.0f / sqrtf(sxx / (float)D + eps);
  r.xq = sxq;
  const float l1 = r.rho * sxq;
  r.m = fmaxf(l0, l1);
  const float w0 = expf(l0 - r.m);  // l0 = -inf -> 0
  const float w1 = expf(l1 - r.m);
  r.Z = w0 + w1;
  r.alpha = w0 / r.Z;
  r.beta = w1 / r.Z;
  return r;
}

// ------------------------------------------------------- register path ----
// NC = D / 512 chunks of 8 elements per lane.
template <typename T, int NC>
__global__ __launch_bounds__(kNTM) void merge_fwd_kernel(MergeArgs a) {
  const int lane = threadIdx.x & 63;
  const int gw = blockIdx.x * kWPB + (threadIdx.x >> 6);
  const int nw = gridDim.x * kWPB;
  const int D = a.D;
  const Chunk<T>* qc = reinterpret_cast<const Chunk<T>*>(a.q);
  Chunk<T> qr[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) qr[c] = qc[c * 64 + lane];
  for (int row = gw; row < a.rows; row += nw) {
    const int64_t base = (int64_t)row * (D / 8);
    const Chunk<T>* xc = reinterpret_cast<const Chunk<T>*>(a.x) + base;
    const Chunk<T>* yc = reinterpret_cast<const Chunk<T>*>(a.y0) + base;
    Chunk<T> xr[NC], yr[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      xr[c] = xc[c * 64 + lane];
      yr[c] = yc[c * 64 + lane];
    }
    const float l0 = a.l0[row];
    float sxx = 0.f, sxq = 0.f;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      float xf[8], qf[8];
      to_f32(xr[c], xf);
      to_f32(qr[c], qf);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        sxx += xf[i] * xf[i];
        sxq += xf[i] * qf[i];
      }
    }
    sxx = wsum(sxx);
    sxq = wsum(sxq);
    const Mix mx = mix(sxx, sxq, l0, D, a.eps);
    Chunk<T>* oc = reinterpret_cast<Chunk<T>*>(a.y) + base;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      float xf[8], yf[8], of[8];
      to_f32(xr[c], xf);
      to_f32(yr[c], yf);
#pragma unroll
      for (int i = 0; i < 8; ++i) of[i] = mx.alpha * yf[i] + mx.beta * xf[i];
      oc[c * 64 + lane] = from_f32<T>(of);
    }
    if (lane == 0) a.lse[row] = mx.m + logf(mx.Z);
  }
}

template <typename T, int NC>
__global__ __launch_bounds__(kNTM) void merge_bwd_kernel(MergeArgs a) {
  __shared__ float red[512 * NC];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int gw = blockIdx.x * kWPB + wid;
  const int nw = gridDim.x * kWPB;
  const int D = a.D;
  const Chunk<T>* qc = reinterpret_cast<const Chunk<T>*>(a.q);
  Chunk<T> qr[NC];
  float gq[NC][8];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    qr[c] = qc[c * 64 + lane];
#pragma unroll
    for (int i = 0; i < 8; ++i) gq[c][i] = 0.f;
  }
  for (int row = gw; row < a.rows; row += nw) {
    const int64_t base = (int64_t)row * (D / 8);
    const Chunk<T>* xc = reinterpret_cast<const Chunk<T>*>(a.x) + base;
    const Chunk<T>* yc = reinterpret_cast<const Chunk<T>*>(a.y0) + base;
    const Chunk<T>* gc = reinterpret_cast<const Chunk<T>*>(a.gy) + base;
    Chunk<T> xr[NC], yr[NC], gr[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      xr[c] = xc[c * 64 + lane];
      yr[c] = yc[c * 64 + lane];
      gr[c] = gc[c * 64 + lane];
    }
    const float l0 = a.l0[row];
    const float gl = a.gl ? a.gl[row] : 0.f;
    float sxx = 0.f, sxq = 0.f, s = 0.f;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      float xf[8], yf[8], gf[8], qf[8];
      to_f32(xr[c], xf);
      to_f32(yr[c], yf);
      to_f32(gr[c], gf);
      to_f32(qr[c], qf);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        sxx += xf[i] * xf[i];
        sxq += xf[i] * qf[i];
        s += gf[i] * (yf[i] - xf[i]);
      }
    }
    sxx = wsum(sxx);
    sxq = wsum(sxq);
    s = wsum(s);
    const Mix mx = mix(sxx, sxq, l0, D, a.eps);
    const float ab = mx.alpha * mx.beta;
    const float gl1 = mx.beta * gl - ab * s;
    const float cq = gl1 * mx.rho;                                   // coefficient of q
    const float cx = -gl1 * mx.xq * mx.rho * mx.rho * mx.rho / (float)D;  // coefficient of x
    const float cg = gl1 * mx.rho;                                   // gq += cg * x
    Chunk<T>* gxc = reinterpret_cast<Chunk<T>*>(a.gx) + base;
    Chunk<T>* gyc = reinterpret_cast<Chunk<T>*>(a.gy0) + base;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      float xf[8], gf[8], qf[8], gx[8], gy0[8];
      to_f32(xr[c], xf);
      to_f32(gr[c], gf);
      to_f32(qr[c], qf);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        gy0[i] = mx.alpha * gf[i];
        gx[i] = mx.beta * gf[i] + cq * qf[i] + cx * xf[i];
        gq[c][i] += cg * xf[i];
      }
      gxc[c * 64 + lane] = from_f32<T>(gx);
      gyc[c * 64 + lane] = from_f32<T>(gy0);
    }
    if (lane == 0) a.gl0[row] = mx.alpha * gl + ab * s;
  }
  // Workgroup partial of gq: wavefronts add into LDS one after another.
  for (int w = 0; w < kWPB; ++w) {
    if (wid == w) {
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int d = (c * 64 + lane) * 8 + i;
          red[d] = (w == 0 ? 0.f : red[d]) + gq[c][i];
        }
    }
    __syncthreads();
  }
  float* part = a.partial + (int64_t)blockIdx.x * D;
  for (int d = threadIdx.x; d < D; d += kNTM) part[d] = red[d];
}

// --------------------------------------------------------- generic path ----
// Any D that is a multiple of 8: each lane walks the row's chunks twice (the
// second pass re-reads the row, which is then normally served by the cache).
template <typename T>
__global__ __launch_bounds__(kNTM) void merge_fwd_generic(MergeArgs a) {
  const int lane = threadIdx.x & 63;
  const int gw = blockIdx.x * kWPB + (threadIdx.x >> 6);
  const int nw = gridDim.x * kWPB;
  const int D = a.D, nch = D / 8;
  const Chunk<T>* qc = reinterpret_cast<const Chunk<T>*>(a.q);
  for (int row = gw; row < a.rows; row += nw) {
    const int64_t base = (int64_t)row * nch;
    const Chunk<T>* xc = reinterpret_cast<const Chunk<T>*>(a.x) + base;
    const Chunk<T>* yc = reinterpret_cast<const Chunk<T>*>(a.y0) + base;
    float sxx = 0.f, sxq = 0.f;
    for (int c = lane; c < nch; c += 64) {
      float xf[8], qf[8];
      to_f32(xc[c], xf);
      to_f32(qc[c], qf);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        sxx += xf[i] * xf[i];
        sxq += xf[i] * qf[i];
      }
    }
    sxx = wsum(sxx);
    sxq = wsum(sxq);
    const Mix mx = mix(sxx, sxq, a.l0[row], D, a.eps);
    Chunk<T>* oc = reinterpret_cast<Chunk<T>*>(a.y) + base;
    for (int c = lane; c < nch; c += 64) {
      float xf[8], yf[8], of[8];
      to_f32(xc[c], xf);
      to_f32(yc[c], yf);
#pragma unroll
      for (int i = 0; i < 8; ++i) of[i] = mx.alpha * yf[i] + mx.beta * xf[i];
      oc[c] = from_f32<T>(of);
    }
    if (lane == 0) a.lse[row] = mx.m + logf(mx.Z);
  }
}

// Generic backward: each wavefront owns one partial row of gq in the
// workspace (partial rows = all wavefronts of the grid).
template <typename T>
__global__ __launch_bounds__(kNTM) void merge_bwd_generic(MergeArgs a) {
  const int lane = threadIdx.x & 63;
  const int gw = blockIdx.x * kWPB + (threadIdx.x >> 6);
  const int nw = gridDim.x * kWPB;
  const int D = a.D, nch = D / 8;
  const Chunk<T>* qc = reinterpret_cast<const Chunk<T>*>(a.q);
  float* part = a.partial + (int64_t)gw * D;
  for (int c = lane; c < nch; c += 64)
#pragma unroll
    for (int i = 0; i < 8; ++i) part[c * 8 + i] = 0.f;
  for (int row = gw; row < a.rows; row += nw) {
    const int64_t base = (int64_t)row * nch;
    const Chunk<T>* xc = reinterpret_cast<const Chunk<T>*>(a.x) + base;
    const Chunk<T>* yc = reinterpret_cast<const Chunk<T>*>(a.y0) + base;
    const Chunk<T>* gc = reinterpret_cast<const Chunk<T>*>(a.gy) + base;
    float sxx = 0.f, sxq = 0.f, s = 0.f;
    for (int c = lane; c < nch; c += 64) {
      float xf[8], qf[8], yf[8], gf[8];
      to_f32(xc[c], xf);
      to_f32(qc[c], qf);
      to_f32(yc[c], yf);
      to_f32(gc[c], gf);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        sxx += xf[i] * xf[i];
        sxq += xf[i] * qf[i];
        s += gf[i] * (yf[i] - xf[i]);
      }
    }
    sxx = wsum(sxx);
    sxq = wsum(sxq);
    s = wsum(s);
    const float gl = a.gl ? a.gl[row] : 0.f;
    const Mix mx = mix(sxx, sxq, a.l0[row], D, a.eps);
    const float ab = mx.alpha * mx.beta;
    const float gl1 = mx.beta * gl - ab * s;
    const float cq = gl1 * mx.rho;
    const float cx = -gl1 * mx.xq * mx.rho * mx.rho * mx.rho / (float)D;
    const float cg = gl1 * mx.rho;
    Chunk<T>* gxc = reinterpret_cast<Chunk<T>*>(a.gx) + base;
    Chunk<T>* gyc = reinterpret_cast<Chunk<T>*>(a.gy0) + base;
    for (int c = lane; c < nch; c += 64) {
      float xf[8], qf[8], gf[8], gx[8], gy0[8];
      to_f32(xc[c], xf);
      to_f32(qc[c], qf);
      to_f32(gc[c], gf);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        gy0[i] = mx.alpha * gf[i];
        gx[i] = mx.beta * gf[i] + cq * qf[i] + cx * xf[i];
        part[c * 8 + i] += cg * xf[i];
      }
      gxc[c] = from_f32<T>(gx);
      gyc[c] = from_f32<T>(gy0);
    }
    if (lane == 0) a.gl0[row] = mx.alpha * gl + ab * s;
  }
}

// gq[d] = sum over partial rows p = 0 .. np-1 of partial[p][d], in order.
__global__ __launch_bounds__(256) void gq_reduce_kernel(const float* __restrict__ partial, float* __restrict__ gq,
                                                        int np, int D) {
  const int d = blockIdx.x * 256 + threadIdx.x;
  if (d >= D) return;
  float s = 0.f;
  for (int p = 0; p < np; ++p) s += partial[(int64_t)p * D + d];
  gq[d] = s;
}

int grid_for(int rows) {
  int g = (rows + kWPB - 1) / kWPB;
  return g < kMaxWG ? g : kMaxWG;
}

// Rows are kept in registers when they fit: D a multiple of 512 with
// D/512 chunks per lane a power of two, at most max_nc of them.
bool register_path(int D, int max_nc) {
  if (D % 512 != 0) return false;
  const int nc = D / 512;
  return nc <= max_nc && (nc & (nc - 1)) == 0;
}

template <typename T>
hipError_t fwd_t(const MergeArgs& a, hipStream_t s) {
  dim3 grid(grid_for(a.rows)), block(kNTM);
  if (register_path(a.D, sizeof(T) == 2 ? 16 : 8)) {
    switch (a.D / 512) {
      case 1: hipLaunchKernelGGL((merge_fwd_kernel<T, 1>), grid, block, 0, s, a); break;
      case 2: hipLaunchKernelGGL((merge_fwd_kernel<T, 2>), grid, block, 0, s, a); break;
      case 4: hipLaunchKernelGGL((merge_fwd_kernel<T, 4>), grid, block, 0, s, a); break;
      case 8: hipLaunchKernelGGL((merge_fwd_kernel<T, 8>), grid, block, 0, s, a); break;
      case 16:
        if constexpr (sizeof(T) == 2) hipLaunchKernelGGL((merge_fwd_kernel<T, 16>), grid, block, 0, s, a);
        break;
    }
  } else {
    hipLaunchKernelGGL((merge_fwd_generic<T>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

template <typename T>
hipError_t bwd_t(const MergeArgs& a, hipStream_t s) {
  const int g = grid_for(a.rows);
  dim3 grid(g), block(kNTM);
  int np;
  if (register_path(a.D, sizeof(T) == 2 ? 8 : 4)) {
    switch (a.D / 512) {
      case 1: hipLaunchKernelGGL((merge_bwd_kernel<T, 1>), grid, block, 0, s, a); break;
      case 2: hipLaunchKernelGGL((merge_bwd_kernel<T, 2>), grid, block, 0, s, a); break;
      case 4: hipLaunchKernelGGL((merge_bwd_kernel<T, 4>), grid, block, 0, s, a); break;
      case 8:
        if constexpr (sizeof(T) == 2) hipLaunchKernelGGL((merge_bwd_kernel<T, 8>), grid, block, 0, s, a);
        break;
    }
    np = g;
  } else {
    hipLaunchKernelGGL((merge_bwd_generic<T>), grid, block, 0, s, a);
    np = g * kWPB;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 rgrid((a.D + 255) / 256), rblock(256);
  hipLaunchKernelGGL(gq_reduce_kernel, rgrid, rblock, 0, s, a.partial, a.gq, np, a.D);
  return hipGetLastError();
}

}  // namespace

int merge_bwd_partial_rows(int rows, int D) {
  // upper bound over both paths: one partial row per wavefront
  (void)D;
  return grid_for(rows) * kWPB;
}

hipError_t launch_merge_fwd(const MergeArgs& a, hipStream_t s) {
  if (a.dtype == 0) return fwd_t<float>(a, s);
  if (a.dtype == 1) return fwd_t<_Float16>(a, s);
  if (a.dtype == 2) return fwd_t<__bf16>(a, s);
  return hipErrorInvalidValue;
}

hipError_t launch_merge_bwd(const MergeArgs& a, hipStream_t s) {
  if (a.dtype == 0) return bwd_t<float>(a, s);
  if (a.dtype == 1) return bwd_t<_Float16>(a, s);
  if (a.dtype == 2) return bwd_t<__bf16>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace fa
