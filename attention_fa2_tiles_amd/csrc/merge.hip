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
// there is no MFMA.  A row is owned by a team of four wavefronts (one
// wavefront for narrow rows); each thread holds a few 16-byte chunks of x,
// y0 (and gy), lane-interleaved so that every load and store instruction
// moves 1 KiB of contiguous memory, and loads the next row's chunks while
// the current row is reduced and written.  The row stays in registers
// between the reductions (x.x, x.q, gy.(y0-x): butterflies across the
// wavefront, then the team's partial sums in LDS in wavefront order) and the
// output pass, so every input byte is read from HBM once.  Cache policy, as
// measured at 32768 x 4096 bf16: the forward's row loads carry the
// non-temporal hint and its stores do not (153 -> 125 us; with the hint on
// the stores as well, 140 us), the backward's loads and its gy0 stores
// carry it and its gx stores do not (266 -> 232 us; loads only 264 us,
// loads and both stores 251 us, gx instead of gy0 233 us).  The N-way merge, whose
// backward reads its inputs twice, takes it on its stores only.  The
// pseudo-query q is loaded once per thread.  gq is reduced deterministically: each thread
// accumulates its columns over the rows of its workgroup, the workgroup
// writes one partial row, and a second kernel adds the partial rows in index
// order.  The page's kernel uses relaxed float atomics there instead, whose
// result depends on timing.  Rows whose width does not split into whole
// chunks per thread take a generic path that reads each row twice.
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
// A team of WPR wavefronts (WPR = 1 or 4; a workgroup is 4 wavefronts) owns
// one row at a time.  Team thread t holds NCH 16-byte chunks of the row,
// chunk j at index t + j * 64 * WPR, so every load and store instruction of
// a wavefront moves 1 KiB of contiguous memory.  The next row's inputs are
// loaded while the current row is reduced and written.  Row sums are reduced
// across the wavefront with butterflies and, for WPR = 4, across the team
// through LDS in wavefront order.
constexpr int kTeamWG = 256;  // threads per workgroup on this path

template <typename T>
struct Elems {
  static constexpr int N = 16 / sizeof(T);
};

template <typename T>
__device__ __forceinline__ void chunk_f32(const u32x4& c, float (&f)[Elems<T>::N]) {
  const T* e = reinterpret_cast<const T*>(&c);
#pragma unroll
  for (int i = 0; i < Elems<T>::N; ++i) f[i] = (float)e[i];
}

template <typename T>
__device__ __forceinline__ u32x4 f32_chunk(const float (&f)[Elems<T>::N]) {
  u32x4 c;
  T* e = reinterpret_cast<T*>(&c);
#pragma unroll
  for (int i = 0; i < Elems<T>::N; ++i) e[i] = (T)f[i];
  return c;
}

template <int WPR>
struct Team {
  int lane, wave, sub, t;
  __device__ __forceinline__ Team() {
    lane = threadIdx.x & 63;
    wave = threadIdx.x >> 6;
    sub = wave / WPR;            // which of the workgroup's rows
    t = (wave % WPR) * 64 + lane;  // thread index inside the team
  }
};

// Sum of NV per-thread values over the team; red is 2 x 4 x 4 floats of LDS
// (double-buffered by row parity, one barrier per row).
template <int WPR, int NV>
__device__ __forceinline__ void team_sum(float (&v)[NV], float* red, int parity, const Team<WPR>& tm) {
#pragma unroll
  for (int k = 0; k < NV; ++k) v[k] = wsum(v[k]);
  if constexpr (WPR > 1) {
    float* slot = red + parity * 16;
    if (tm.lane == 0) {
#pragma unroll
      for (int k = 0; k < NV; ++k) slot[tm.wave * 4 + k] = v[k];
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      float acc = 0.f;
#pragma unroll
      for (int w = 0; w < WPR; ++w) acc += slot[(tm.sub * WPR + w) * 4 + k];
      v[k] = acc;
    }
  }
}

template <typename T, int WPR, int NCH>
__global__ __launch_bounds__(kTeamWG) void merge_fwd_kernel(MergeArgs a) {
  constexpr int E = Elems<T>::N;
  constexpr int RPI = 4 / WPR;  // rows per workgroup iteration
  __shared__ float red[32];
  const Team<WPR> tm;
  const int D = a.D;
  const int64_t cpr = D / E;    // chunks per row
  const u32x4* qc = reinterpret_cast<const u32x4*>(a.q);
  float qf[NCH][E];
#pragma unroll
  for (int j = 0; j < NCH; ++j) chunk_f32<T>(qc[tm.t + j * 64 * WPR], qf[j]);
  const int stride = gridDim.x * RPI;
  int row = blockIdx.x * RPI + tm.sub;
  u32x4 xr[NCH], yr[NCH];
  auto load = [&](int r) {
    const u32x4* xc = reinterpret_cast<const u32x4*>(a.x) + (int64_t)r * cpr;
    const u32x4* yc = reinterpret_cast<const u32x4*>(a.y0) + (int64_t)r * cpr;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      xr[j] = __builtin_nontemporal_load(&xc[tm.t + j * 64 * WPR]);
      yr[j] = __builtin_nontemporal_load(&yc[tm.t + j * 64 * WPR]);
    }
  };
  if (row < a.rows) load(row);
  for (int parity = 0; row < a.rows; row += stride, parity ^= 1) {
    u32x4 xc[NCH], yc[NCH];
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      xc[j] = xr[j];
      yc[j] = yr[j];
    }
    if (row + stride < a.rows) load(row + stride);
    float v[2] = {0.f, 0.f};  // x.x, x.q
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      float xf[E];
      chunk_f32<T>(xc[j], xf);
#pragma unroll
      for (int i = 0; i < E; ++i) {
        v[0] += xf[i] * xf[i];
        v[1] += xf[i] * qf[j][i];
      }
    }
    team_sum<WPR, 2>(v, red, parity, tm);
    const Mix mx = mix(v[0], v[1], a.l0[row], D, a.eps);
    u32x4* oc = reinterpret_cast<u32x4*>(a.y) + (int64_t)row * cpr;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      float xf[E], yf[E], of[E];
      chunk_f32<T>(xc[j], xf);
      chunk_f32<T>(yc[j], yf);
#pragma unroll
      for (int i = 0; i < E; ++i) of[i] = mx.alpha * yf[i] + mx.beta * xf[i];
      oc[tm.t + j * 64 * WPR] = f32_chunk<T>(of);
    }
    if (tm.t == 0) a.lse[row] = mx.m + logf(mx.Z);
  }
}

template <typename T, int WPR, int NCH>
__global__ __launch_bounds__(kTeamWG) void merge_bwd_kernel(MergeArgs a) {
  constexpr int E = Elems<T>::N;
  constexpr int RPI = 4 / WPR;
  __shared__ float red[32];
  __shared__ float gqs[WPR == 1 ? 64 * NCH * E : 1];
  const Team<WPR> tm;
  const int D = a.D;
  const int64_t cpr = D / E;
  const u32x4* qc = reinterpret_cast<const u32x4*>(a.q);
  float qf[NCH][E], gq[NCH][E];
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    chunk_f32<T>(qc[tm.t + j * 64 * WPR], qf[j]);
#pragma unroll
    for (int i = 0; i < E; ++i) gq[j][i] = 0.f;
  }
  const int stride = gridDim.x * RPI;
  int row = blockIdx.x * RPI + tm.sub;
  u32x4 xr[NCH], yr[NCH], gr[NCH];
  auto load = [&](int r) {
    const u32x4* xc = reinterpret_cast<const u32x4*>(a.x) + (int64_t)r * cpr;
    const u32x4* yc = reinterpret_cast<const u32x4*>(a.y0) + (int64_t)r * cpr;
    const u32x4* gc = reinterpret_cast<const u32x4*>(a.gy) + (int64_t)r * cpr;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      xr[j] = __builtin_nontemporal_load(&xc[tm.t + j * 64 * WPR]);
      yr[j] = __builtin_nontemporal_load(&yc[tm.t + j * 64 * WPR]);
      gr[j] = __builtin_nontemporal_load(&gc[tm.t + j * 64 * WPR]);
    }
  };
  if (row < a.rows) load(row);
  for (int parity = 0; row < a.rows; row += stride, parity ^= 1) {
    u32x4 xc[NCH], yc[NCH], gc[NCH];
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      xc[j] = xr[j];
      yc[j] = yr[j];
      gc[j] = gr[j];
    }
    if (row + stride < a.rows) load(row + stride);
    float v[3] = {0.f, 0.f, 0.f};  // x.x, x.q, gy.(y0 - x)
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      float xf[E], yf[E], gf[E];
      chunk_f32<T>(xc[j], xf);
      chunk_f32<T>(yc[j], yf);
      chunk_f32<T>(gc[j], gf);
#pragma unroll
      for (int i = 0; i < E; ++i) {
        v[0] += xf[i] * xf[i];
        v[1] += xf[i] * qf[j][i];
        v[2] += gf[i] * (yf[i] - xf[i]);
      }
    }
    team_sum<WPR, 3>(v, red, parity, tm);
    const float gl = a.gl ? a.gl[row] : 0.f;
    const Mix mx = mix(v[0], v[1], a.l0[row], D, a.eps);
    const float s = v[2];
    const float ab = mx.alpha * mx.beta;
    const float gl1 = mx.beta * gl - ab * s;
    const float cq = gl1 * mx.rho;                                        // coefficient of q
    const float cx = -gl1 * mx.xq * mx.rho * mx.rho * mx.rho / (float)D;  // coefficient of x
    const float cg = gl1 * mx.rho;                                        // gq += cg * x
    u32x4* gxc = reinterpret_cast<u32x4*>(a.gx) + (int64_t)row * cpr;
    u32x4* gyc = reinterpret_cast<u32x4*>(a.gy0) + (int64_t)row * cpr;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      float xf[E], gf[E], gx[E], gy0[E];
      chunk_f32<T>(xc[j], xf);
      chunk_f32<T>(gc[j], gf);
#pragma unroll
      for (int i = 0; i < E; ++i) {
        gy0[i] = mx.alpha * gf[i];
        gx[i] = mx.beta * gf[i] + cq * qf[j][i] + cx * xf[i];
        gq[j][i] += cg * xf[i];
      }
      if (a.accumulate) {  // add into the caller's gradient (one rounding)
        float old[E];
        chunk_f32<T>(gxc[tm.t + j * 64 * WPR], old);
#pragma unroll
        for (int i = 0; i < E; ++i) gx[i] += old[i];
      }
      gxc[tm.t + j * 64 * WPR] = f32_chunk<T>(gx);
      __builtin_nontemporal_store(f32_chunk<T>(gy0), &gyc[tm.t + j * 64 * WPR]);
    }
    if (tm.t == 0) a.gl0[row] = mx.alpha * gl + ab * s;
  }
  // Workgroup partial of gq.  WPR = 4: each column belongs to one thread.
  // WPR = 1: the 4 wavefronts hold the same columns; they are added in LDS
  // one after another.
  float* part = a.partial + (int64_t)blockIdx.x * D;
  if constexpr (WPR == 4) {
#pragma unroll
    for (int j = 0; j < NCH; ++j)
#pragma unroll
      for (int i = 0; i < E; ++i) part[(tm.t + j * 256) * E + i] = gq[j][i];
  } else {
    for (int w = 0; w < 4; ++w) {
      if (tm.wave == w) {
#pragma unroll
        for (int j = 0; j < NCH; ++j)
#pragma unroll
          for (int i = 0; i < E; ++i) {
            const int d = (tm.lane + j * 64) * E + i;
            gqs[d] = (w == 0 ? 0.f : gqs[d]) + gq[j][i];
          }
      }
      __syncthreads();
    }
    for (int d = threadIdx.x; d < D; d += kTeamWG) part[d] = gqs[d];
  }
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
      if (a.accumulate) {
        float old[8];
        to_f32(gxc[c], old);
#pragma unroll
        for (int i = 0; i < 8; ++i) gx[i] += old[i];
      }
      gxc[c] = from_f32<T>(gx);
      gyc[c] = from_f32<T>(gy0);
    }
    if (lane == 0) a.gl0[row] = mx.alpha * gl + ab * s;
  }
}

// gq[d] = sum over the np partial rows, in a fixed order, in two steps.
// Step 1: slice s (a fixed contiguous range of partial rows) of a 128-column
// block: thread (r, c) sums rows r, r + 8, ... of the range for 4 columns,
// and the 8 row groups are added in order through LDS.  Step 2 adds the
// kRedSlices slice rows in order.
constexpr int kRedSlices = 8;

__global__ __launch_bounds__(256) void gq_reduce_slices(const float* __restrict__ partial,
                                                        float* __restrict__ slices, int np, int D) {
  __shared__ f32x4 red[8][32];
  const int c = threadIdx.x & 31, r = threadIdx.x >> 5;
  const int d = blockIdx.x * 128 + 4 * c;
  const int sl = blockIdx.y;
  const int p0 = (int)((int64_t)np * sl / kRedSlices);
  const int p1 = (int)((int64_t)np * (sl + 1) / kRedSlices);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if (d < D) {
    for (int p = p0 + r; p < p1; p += 8) acc += *reinterpret_cast<const f32x4*>(partial + (int64_t)p * D + d);
  }
  red[r][c] = acc;
  __syncthreads();
  if (r == 0 && d < D) {
    f32x4 t = red[0][c];
#pragma unroll
    for (int k = 1; k < 8; ++k) t += red[k][c];
    *reinterpret_cast<f32x4*>(slices + (int64_t)sl * D + d) = t;
  }
}

__global__ __launch_bounds__(256) void gq_reduce_final(const float* __restrict__ slices, float* __restrict__ gq,
                                                       int D, int accumulate) {
  const int d = blockIdx.x * 256 + threadIdx.x;
  if (d >= D) return;
  float t = 0.f;
#pragma unroll
  for (int sl = 0; sl < kRedSlices; ++sl) t += slices[(int64_t)sl * D + d];
  gq[d] = accumulate ? gq[d] + t : t;
}

int grid_for(int rows) {
  int g = (rows + kWPB - 1) / kWPB;
  return g < kMaxWG ? g : kMaxWG;
}

// Register path shape: 16-byte chunks per row C = D * sizeof(T) / 16 split as
// C = 64 * WPR * NCH with WPR in {4, 1} and NCH in {1, 2, 4, 8}; else the
// generic path (returns false).
struct RegShape {
  int wpr, nch;
};
bool reg_shape(int D, int elem_bytes, RegShape& r) {
  if ((D * elem_bytes) % 16 != 0) return false;
  const int C = D * elem_bytes / 16;
  for (int wpr : {4, 1}) {
    if (C % (64 * wpr) != 0) continue;
    const int nch = C / (64 * wpr);
    if (nch == 1 || nch == 2 || nch == 4 || nch == 8) {
      r.wpr = wpr;
      r.nch = nch;
      return true;
    }
  }
  return false;
}

constexpr int kMaxTeamWG = 1024;  // cap on register-path workgroups (= gq partial rows)

// Workgroups that fit on the device at once for a register-path kernel.
int resident_wgs(const void* kernel) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kTeamWG, 0) != hipSuccess || cus <= 0 ||
      per_cu <= 0) {
    cus = 256;
    per_cu = 2;
  }
  return cus * per_cu;
}

// Workgroups of the register path: one per row group, but no more than fit
// on the device at once (the kernels loop over rows, so a second partial
// wave of workgroups would only add a tail) and, for the backward, no more
// than kMaxTeamWG.
int team_grid(int resident, int rows, int wpr, bool capped) {
  const int rpi = 4 / wpr;
  int g = (rows + rpi - 1) / rpi;
  if (g > resident) g = resident;
  if (capped && g > kMaxTeamWG) g = kMaxTeamWG;
  return g;
}

template <typename T, int WPR, int NCH>
void fwd_launch(const MergeArgs& a, hipStream_t s) {
  static const int resident = resident_wgs((const void*)merge_fwd_kernel<T, WPR, NCH>);
  hipLaunchKernelGGL((merge_fwd_kernel<T, WPR, NCH>), dim3(team_grid(resident, a.rows, WPR, false)),
                     dim3(kTeamWG), 0, s, a);
}

template <typename T, int WPR, int NCH>
int bwd_launch(const MergeArgs& a, hipStream_t s) {
  static const int resident = resident_wgs((const void*)merge_bwd_kernel<T, WPR, NCH>);
  const int g = team_grid(resident, a.rows, WPR, true);
  hipLaunchKernelGGL((merge_bwd_kernel<T, WPR, NCH>), dim3(g), dim3(kTeamWG), 0, s, a);
  return g;
}

// WPR = 1 is only chosen for rows of 64 or 128 chunks (NCH = 1, 2): wider
// rows that split into whole chunks per thread go to WPR = 4.
template <typename T, int WPR>
void launch_fwd_nch(const MergeArgs& a, int nch, hipStream_t s) {
  switch (nch) {
    case 1: fwd_launch<T, WPR, 1>(a, s); break;
    case 2: fwd_launch<T, WPR, 2>(a, s); break;
    case 4: if constexpr (WPR == 4) fwd_launch<T, WPR, 4>(a, s); break;
    case 8: if constexpr (WPR == 4) fwd_launch<T, WPR, 8>(a, s); break;
  }
}

template <typename T, int WPR>
int launch_bwd_nch(const MergeArgs& a, int nch, hipStream_t s) {
  switch (nch) {
    case 1: return bwd_launch<T, WPR, 1>(a, s);
    case 2: return bwd_launch<T, WPR, 2>(a, s);
    case 4: if constexpr (WPR == 4) return bwd_launch<T, WPR, 4>(a, s); break;
    case 8: if constexpr (WPR == 4) return bwd_launch<T, WPR, 8>(a, s); break;
  }
  return 0;
}

template <typename T>
hipError_t fwd_t(const MergeArgs& a, hipStream_t s) {
  RegShape r;
  if (reg_shape(a.D, sizeof(T), r)) {
    if (r.wpr == 4)
      launch_fwd_nch<T, 4>(a, r.nch, s);
    else
      launch_fwd_nch<T, 1>(a, r.nch, s);
  } else {
    dim3 grid(grid_for(a.rows)), block(kNTM);
    hipLaunchKernelGGL((merge_fwd_generic<T>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

template <typename T>
hipError_t bwd_t(const MergeArgs& a, hipStream_t s) {
  RegShape r;
  int np;
  if (reg_shape(a.D, sizeof(T), r)) {
    np = (r.wpr == 4) ? launch_bwd_nch<T, 4>(a, r.nch, s) : launch_bwd_nch<T, 1>(a, r.nch, s);
  } else {
    const int g = grid_for(a.rows);
    hipLaunchKernelGGL((merge_bwd_generic<T>), dim3(g), dim3(kNTM), 0, s, a);
    np = g * kWPB;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // the slice rows follow the np partial rows in the workspace
  float* slices = a.partial + (int64_t)np * a.D;
  hipLaunchKernelGGL(gq_reduce_slices, dim3((a.D + 127) / 128, kRedSlices), dim3(256), 0, s, a.partial, slices, np,
                     a.D);
  hipLaunchKernelGGL(gq_reduce_final, dim3((a.D + 255) / 256), dim3(256), 0, s, slices, a.gq, a.D, a.accumulate);
  return hipGetLastError();
}

}  // namespace

int merge_bwd_partial_rows(int rows, int D) {
  // upper bound over both paths and every dtype: one partial row per
  // wavefront of the generic path (min(rows rounded up to 8, 4096)), which is
  // at least the register path's one per workgroup (min(rows, 1024)), plus
  // the kRedSlices rows of the reduction's first step
  (void)D;
  return grid_for(rows) * kWPB + kRedSlices;
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
