// Attention forward for fp16/bf16 on gfx950 MFMA: plain, fused JVP, and
// piecewise variants of one tiled online-softmax kernel.
//
// What is computed: the FlashAttention-2 forward of the Triton fused-attention
// tutorial (_attn_fwd, _attn_fwd_inner): per query block, stream K/V blocks,
// keep a running row max m and row sum l, rescale the running output by
// exp2(m_old - m_new), and finish with O = acc / l and LSE = m + log l.
// The JVP variant adds the tangent recurrences of the same tutorial's
// ENABLE_JVP path; the piecewise variant takes its scores from (q1, k1) or
// (q2, k2) by query-key distance (FlagAttention piecewise.py, _fwd_kernel).
//
// How it maps to CDNA4: 4 waves per workgroup, 32 query rows per wave
// (BM = 128), K/V blocks of 64 keys staged in LDS, double-buffered, loaded
// with 16-byte global loads.  Scores are formed transposed, S^t = K Q^t, so
// that each lane owns one query row: row max and row sum are in-lane
// reductions plus one exchange with the other half-wave, and the rescale of
// the output accumulator is lane-local because that accumulator is also kept
// transposed (O^t = V^t P^t).  K sits in LDS row-major (swap23 rows) and V
// transposed, so both products read 16-byte MFMA operands straight from LDS
// and the scores feed the second product without leaving registers.
#include "common.h"
#include "kernels.h"

namespace fa {
namespace {

constexpr int kWaves = 4;
constexpr int kNT = 64 * kWaves;
constexpr int kBM = 32 * kWaves;  // query rows per workgroup
constexpr int kBN = 64;           // keys per K/V block

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* q2;
  const void* k2;
  const void* tq;
  const void* tk;
  const void* tv;
  void* o;
  float* lse;
  void* to;
  int BH, M, N, nmb;
  float scale2;    // sm_scale * log2(e)
  float sm_scale;
  int w;
};

template <typename T, int D, int VAR>
struct alignas(16) FwdStage {
  using RT = RowTile<T, kBN, D, kNT>;
  using TT = TransTile<T, kBN, D, kNT>;
  static constexpr int NRM = (VAR == PLAIN) ? 1 : 2;  // K (+ tK or K2)
  static constexpr int NTR = (VAR == JVP) ? 2 : 1;    // V^t (+ tV^t)
  T rm[NRM][RT::ELEMS];
  T tr[NTR][TT::ELEMS];
};

template <typename T, int D, int VAR, bool CAUSAL>
__global__ __launch_bounds__(kNT) void attn_fwd_kernel(const FwdParams p) {
  using V8 = typename Vec8<T>::type;
  using St = FwdStage<T, D, VAR>;
  using RT = typename St::RT;
  using TT = typename St::TT;
  constexpr int KK = D / 16;     // 16-wide k steps over the head dim
  constexpr int DT = D / 32;     // 32-wide tiles of the output's head dim
  constexpr int ST = kBN / 32;   // 32-key score tiles per block
  constexpr int PT = kBN / 16;   // 16-key operand slices per block
  constexpr bool kJvp = VAR == JVP;
  constexpr bool kPw = VAR == PW;

  __shared__ St smem[2];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int li = lane & 31, h = lane >> 5;

  // Workgroup -> (head, query block).  Heads vary fastest so every query
  // block of one head lands on the same XCD (the dispatcher deals workgroups
  // round-robin over the 8 XCDs and BH is a multiple of 8 in practice), which
  // keeps that head's K/V in one L2.  Causal: longest query blocks first.
  const int bh = blockIdx.x % p.BH;
  int mb = blockIdx.x / p.BH;
  if (CAUSAL) mb = p.nmb - 1 - mb;
  const int m0 = mb * kBM;
  const int row0 = m0 + 32 * wave;
  const bool wave_valid = row0 < p.M;
  const int qi = row0 + li;
  const int pshift = p.N - p.M;
  const int64_t qbase = (int64_t)bh * p.M * D;
  const int64_t kbase = (int64_t)bh * p.N * D;

  const T* Kp = (const T*)p.k + kbase;
  const T* Vp = (const T*)p.v + kbase;
  const T* K2p = kPw ? (const T*)p.k2 + kbase : nullptr;
  const T* TKp = kJvp ? (const T*)p.tk + kbase : nullptr;
  const T* TVp = kJvp ? (const T*)p.tv + kbase : nullptr;

  int n_end = p.N;
  const int wg_last_row = min(p.M, m0 + kBM) - 1;
  if (CAUSAL) n_end = min(p.N, wg_last_row + pshift + 1);
  const int nblk = n_end > 0 ? (n_end + kBN - 1) / kBN : 0;

  // Query-side operands stay in registers for the whole pass.
  V8 qf[KK], q2f[kPw ? KK : 1], tqf[kJvp ? KK : 1];
  if (wave_valid) {
    const T* qrow = (const T*)p.q + qbase + (int64_t)qi * D + 8 * h;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) qf[kk] = *reinterpret_cast<const V8*>(qrow + 16 * kk);
    if constexpr (kPw) {
      const T* q2row = (const T*)p.q2 + qbase + (int64_t)qi * D + 8 * h;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) q2f[kk] = *reinterpret_cast<const V8*>(q2row + 16 * kk);
    }
    if constexpr (kJvp) {
      const T* tqrow = (const T*)p.tq + qbase + (int64_t)qi * D + 8 * h;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) tqf[kk] = *reinterpret_cast<const V8*>(tqrow + 16 * kk);
    }
  }

  f32x16 acc[DT];
  f32x16 accg[kJvp ? DT : 1];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = zero16();
  if constexpr (kJvp) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) accg[dt] = zero16();
  }
  float m_i = kNegInf;  // running max, log2 units
  float l_i = 0.f;      // running sum, this half-wave's keys
  float mu_i = 0.f;     // JVP: running sum of P * Sdot, this half-wave's keys

  RT ldk, ldk2;
  TT ldv, ldtv;

  // Piecewise: which score pairs a block needs, for a row range.
  auto pw_class = [&](int r_lo, int r_hi, int n0, bool& all_near, bool& all_far) {
    const int dmax = r_hi + pshift - n0;
    const int dmin = r_lo + pshift - (n0 + kBN - 1);
    all_near = (dmax <= p.w) && (dmin >= -p.w);
    all_far = (p.w < 0) || (dmin > p.w) || (dmax < -p.w);
  };

  bool ld_k1 = true, ld_k2 = true;  // piecewise: tiles staged for the next block
  auto issue = [&](int jb) {
    const int64_t off = (int64_t)jb * kBN * D;
    if constexpr (kPw) {
      bool an, af;
      pw_class(m0, wg_last_row, jb * kBN, an, af);
      ld_k1 = !af;
      ld_k2 = !an;
      if (ld_k1) ldk.load(Kp + off, tid);
      if (ld_k2) ldk2.load(K2p + off, tid);
    } else {
      ldk.load(Kp + off, tid);
      if constexpr (kJvp) ldk2.load(TKp + off, tid);
    }
    ldv.load(Vp + off, tid);
    if constexpr (kJvp) ldtv.load(TVp + off, tid);
  };
  auto commit = [&](St& s) {
    if constexpr (kPw) {
      if (ld_k1) ldk.store(s.rm[0], tid);
      if (ld_k2) ldk2.store(s.rm[1], tid);
    } else {
      ldk.store(s.rm[0], tid);
      if constexpr (kJvp) ldk2.store(s.rm[1], tid);
    }
    ldv.store(s.tr[0], tid);
    if constexpr (kJvp) ldtv.store(s.tr[1], tid);
  };

  if (nblk > 0) {
    issue(0);
    commit(smem[0]);
  }
  __syncthreads();

  for (int jb = 0; jb < nblk; ++jb) {
    St& cur = smem[jb & 1];
    if (jb + 1 < nblk) issue(jb + 1);
    const int n0 = jb * kBN;
    const bool active = wave_valid && (!CAUSAL || n0 <= row0 + 31 + pshift);
    if (active) {
      const bool need_mask = CAUSAL && (n0 + kBN - 1 > row0 + pshift);
      f32x16 s[ST];
      f32x16 sd[kJvp ? ST : 1];
      // ---- scores S^t = K Q^t (and tangents) ------------------------------
      if constexpr (kPw) {
        bool an, af;
        pw_class(row0, row0 + 31, n0, an, af);
#pragma unroll
        for (int st = 0; st < ST; ++st) {
          f32x16 s1 = zero16(), s2 = zero16();
          const T* k1row = cur.rm[0] + (32 * st + li) * RT::PITCH + 8 * h;
          const T* k2row = cur.rm[1] + (32 * st + li) * RT::PITCH + 8 * h;
          if (!af) {
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) s1 = mfma32x32x16(lds_read8(k1row + 16 * kk), qf[kk], s1);
          }
          if (!an) {
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) s2 = mfma32x32x16(lds_read8(k2row + 16 * kk), q2f[kk], s2);
          }
          if (an) {
            s[st] = s1;
          } else if (af) {
            s[st] = s2;
          } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = n0 + 32 * st + perm_row(r, h);
              const int dist = qi + pshift - key;
              s[st][r] = (dist <= p.w && dist >= -p.w) ? s1[r] : s2[r];
            }
          }
        }
      } else {
#pragma unroll
        for (int st = 0; st < ST; ++st) {
          s[st] = zero16();
          if constexpr (kJvp) sd[st] = zero16();
          const T* krow = cur.rm[0] + (32 * st + li) * RT::PITCH + 8 * h;
#pragma unroll
          for (int kk = 0; kk < KK; ++kk) {
            const V8 a = lds_read8(krow + 16 * kk);
            s[st] = mfma32x32x16(a, qf[kk], s[st]);
            if constexpr (kJvp) sd[st] = mfma32x32x16(a, tqf[kk], sd[st]);
          }
          if constexpr (kJvp) {
            const T* tkrow = cur.rm[1] + (32 * st + li) * RT::PITCH + 8 * h;
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) sd[st] = mfma32x32x16(lds_read8(tkrow + 16 * kk), qf[kk], sd[st]);
          }
        }
      }
      // ---- online softmax (log2 units) ------------------------------------
      float mloc = kNegInf;
#pragma unroll
      for (int st = 0; st < ST; ++st) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float x = s[st][r] * p.scale2;
          if (need_mask) {
            const int key = n0 + 32 * st + perm_row(r, h);
            if (key > qi + pshift) x = kNegInf;
          }
          s[st][r] = x;
          mloc = fmaxf(mloc, x);
        }
      }
      mloc = fmaxf(mloc, xor32(mloc));
      const float m_new = fmaxf(m_i, mloc);
      const float m_use = (m_new == kNegInf) ? 0.f : m_new;
      const float alpha = exp2_fast(m_i - m_use);
      float lsum = 0.f, musum = 0.f;
#pragma unroll
      for (int st = 0; st < ST; ++st) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pv = exp2_fast(s[st][r] - m_use);
          s[st][r] = pv;
          lsum += pv;
          if constexpr (kJvp) {
            const float ps = pv * sd[st][r] * p.sm_scale;
            sd[st][r] = ps;
            musum += ps;
          }
        }
      }
      l_i = alpha * l_i + lsum;
      m_i = m_new;
      if constexpr (kJvp) mu_i = alpha * mu_i + musum;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[dt][r] *= alpha;
        if constexpr (kJvp) {
#pragma unroll
          for (int r = 0; r < 16; ++r) accg[dt][r] *= alpha;
        }
      }
      // ---- O^t += V^t P^t (and the tangent accumulator) --------------------
      V8 pb[PT];
      V8 psb[kJvp ? PT : 1];
#pragma unroll
      for (int t = 0; t < PT; ++t) {
        pb[t] = pack8<T>(s[t >> 1], 8 * (t & 1));
        if constexpr (kJvp) psb[t] = pack8<T>(sd[t >> 1], 8 * (t & 1));
      }
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const T* vrow = cur.tr[0] + (32 * dt + li) * TT::PITCH + 8 * h;
#pragma unroll
        for (int t = 0; t < PT; ++t) {
          const V8 a = lds_read8(vrow + 16 * t);
          acc[dt] = mfma32x32x16(a, pb[t], acc[dt]);
          if constexpr (kJvp) accg[dt] = mfma32x32x16(a, psb[t], accg[dt]);
        }
        if constexpr (kJvp) {
          const T* tvrow = cur.tr[1] + (32 * dt + li) * TT::PITCH + 8 * h;
#pragma unroll
          for (int t = 0; t < PT; ++t) accg[dt] = mfma32x32x16(lds_read8(tvrow + 16 * t), pb[t], accg[dt]);
        }
      }
    }
    if (jb + 1 < nblk) commit(smem[(jb + 1) & 1]);
    __syncthreads();
  }

  // ---- epilogue: O = acc / l, LSE = (m + log2 l) ln 2 ----------------------
  if (!wave_valid) return;
  const float l = l_i + xor32(l_i);
  const bool has = l > 0.f;
  const float inv = has ? 1.f / l : 0.f;
  T* orow = (T*)p.o + qbase + (int64_t)qi * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) store_acc_t<T>(orow, acc[dt], 32 * dt, h, inv);
  if (h == 0) p.lse[(int64_t)bh * p.M + qi] = has ? (m_i + log2f(l)) * kLn2 : kNegInf;
  if constexpr (kJvp) {
    const float mu = mu_i + xor32(mu_i);
    const float c = mu * inv;  // mu / l
    T* torow = (T*)p.to + qbase + (int64_t)qi * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      f32x16 t;
#pragma unroll
      for (int r = 0; r < 16; ++r) t[r] = (accg[dt][r] - c * acc[dt][r]) * inv;
      store_acc_t<T>(torow, t, 32 * dt, h, 1.f);
    }
  }
}

template <typename T, int D, int VAR>
hipError_t launch_t(const FwdArgs& a, hipStream_t s) {
  FwdParams p;
  p.q = a.q;
  p.k = a.k;
  p.v = a.v;
  p.q2 = a.q2;
  p.k2 = a.k2;
  p.tq = a.tq;
  p.tk = a.tk;
  p.tv = a.tv;
  p.o = a.o;
  p.lse = a.lse;
  p.to = a.to;
  p.BH = a.B * a.H;
  p.M = a.M;
  p.N = a.N;
  p.nmb = (a.M + kBM - 1) / kBM;
  p.scale2 = a.sm_scale * kLog2e;
  p.sm_scale = a.sm_scale;
  p.w = a.w;
  dim3 grid(p.nmb * p.BH), block(kNT);
  if (a.causal)
    hipLaunchKernelGGL((attn_fwd_kernel<T, D, VAR, true>), grid, block, 0, s, p);
  else
    hipLaunchKernelGGL((attn_fwd_kernel<T, D, VAR, false>), grid, block, 0, s, p);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_var(const FwdArgs& a, hipStream_t s) {
  switch (a.variant) {
    case PLAIN: return launch_t<T, D, PLAIN>(a, s);
    case JVP: return launch_t<T, D, JVP>(a, s);
    case PW: return launch_t<T, D, PW>(a, s);
  }
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t launch_d(const FwdArgs& a, hipStream_t s) {
  if (a.D == 64) return launch_var<T, 64>(a, s);
  if (a.D == 128) return launch_var<T, 128>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_attn_fwd(const FwdArgs& a, hipStream_t s) {
  if (a.dtype == 1) return launch_d<_Float16>(a, s);
  if (a.dtype == 2) return launch_d<__bf16>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace fa
