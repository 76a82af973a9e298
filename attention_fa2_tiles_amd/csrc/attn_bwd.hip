// Attention backward for fp16/bf16 on gfx950 MFMA (plain and piecewise).
//
// What is computed: the recompute-based FlashAttention-2 backward of the
// Triton fused-attention tutorial (_attn_bwd_preprocess, _attn_bwd_dkdv,
// _attn_bwd_dq) and of FlagAttention piecewise.py (_bwd_preprocess,
// _bwd_kv_kernel, _bwd_q_kernel):
//   Delta_i = sum_d O_id dO_id
//   P_ij    = exp(sm_scale q_i.k_j - LSE_i)      (recomputed from LSE)
//   dV      = P^t dO,    dP = dO V^t,    dS = P * (dP - Delta)
//   dK      = sm_scale dS^t Q,           dQ = sm_scale dS K
// Non-causal passes visit every block (the correction from the tutorial's
// comment thread); causal passes start or stop at the diagonal.  In the
// piecewise variant dS is split by the distance rule into the (q1, k1) and
// (q2, k2) parts.
//
// Layout on CDNA4:
//  * dK/dV pass: 4 waves x 32 keys per workgroup with K and V resident in
//    registers; query blocks of 32 rows stream through LDS both row-major
//    (swap23, for S = Q K^t and dP = dO V^t) and transposed (for the
//    accumulations dV^t += dO^t P and dK^t += Q^t dS).  Each lane owns one
//    key column, so P and dS leave the score product already laid out as the
//    B operand of the accumulation products.
//  * dQ pass: 4 waves x 32 queries per workgroup with Q and dO resident;
//    64-key blocks of K, V (row-major) and K^t stream through LDS.  Each lane
//    owns one query, so LSE and Delta are per-lane scalars.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace fa {
namespace {

constexpr int kWaves = 4;
constexpr int kNT = 64 * kWaves;

// ------------------------------------------------------------------ Delta --
template <typename T>
struct Row8 {
  T e[8];
};

template <typename T, int D>
__global__ __launch_bounds__(256) void delta_kernel(const T* __restrict__ o, const T* __restrict__ dout,
                                                    float* __restrict__ delta, int64_t rows) {
  constexpr int TPR = D / 8;      // threads per row
  constexpr int RPB = 256 / TPR;  // rows per block
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
  const int c = threadIdx.x % TPR;
  float sum = 0.f;
  if (row < rows) {
    const Row8<T> a = *reinterpret_cast<const Row8<T>*>(o + row * D + 8 * c);
    const Row8<T> b = *reinterpret_cast<const Row8<T>*>(dout + row * D + 8 * c);
#pragma unroll
    for (int e = 0; e < 8; ++e) sum += (float)a.e[e] * (float)b.e[e];
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) sum += __shfl_xor(sum, off, 64);
  if (row < rows && c == 0) delta[row] = sum;
}

template <typename T>
hipError_t launch_delta_t(const void* o, const void* dout, float* delta, int64_t rows, int D,
                          hipStream_t s) {
  const int64_t rpb = 256 / (D / 8);
  dim3 grid((unsigned)((rows + rpb - 1) / rpb)), block(256);
  if (D == 64)
    hipLaunchKernelGGL((delta_kernel<T, 64>), grid, block, 0, s, (const T*)o, (const T*)dout, delta, rows);
  else if (D == 128)
    hipLaunchKernelGGL((delta_kernel<T, 128>), grid, block, 0, s, (const T*)o, (const T*)dout, delta, rows);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* q2;
  const void* k2;
  const void* dout;
  const float* lse;
  const float* delta;
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

// ------------------------------------------------------------- dK/dV pass --
constexpr int kQB = 32;            // query rows per streamed block
constexpr int kKB = 32 * kWaves;   // keys per workgroup

template <typename T, int D, int VAR>
struct alignas(16) DkdvStage {
  using RT = RowTile<T, kQB, D, kNT>;
  using TT = TransTile<T, kQB, D, kNT>;
  static constexpr int NQ = (VAR == PW) ? 2 : 1;
  T qrm[NQ][RT::ELEMS];
  T dorm[RT::ELEMS];
  T qtr[NQ][TT::ELEMS];
  T dotr[TT::ELEMS];
  alignas(16) float lse2[kQB];
  alignas(16) float delta[kQB];
};

template <typename T, int D, int VAR, bool CAUSAL>
__global__ __launch_bounds__(kNT) void attn_dkdv_kernel(const BwdParams p) {
  using V8 = typename Vec8<T>::type;
  using St = DkdvStage<T, D, VAR>;
  using RT = typename St::RT;
  using TT = typename St::TT;
  constexpr int KK = D / 16;
  constexpr int DT = D / 32;
  constexpr int ST = kQB / 32;
  constexpr int PT = kQB / 16;
  constexpr bool kPw = VAR == PW;
  constexpr int NQ = St::NQ;

  __shared__ St smem[2];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int li = lane & 31, h = lane >> 5;

  // Heads vary fastest (one head's Q/dO stay in one XCD's L2).  Causal: key
  // block 0 is seen by every query, so natural order already runs the
  // longest workgroups first.
  const int bh = blockIdx.x % p.BH;
  const int kb = blockIdx.x / p.BH;
  const int n0 = kb * kKB;
  const int kw0 = n0 + 32 * wave;
  const bool wave_valid = kw0 < p.N;
  const int kj = kw0 + li;  // this lane's key
  const int pshift = p.N - p.M;
  const int64_t qbase = (int64_t)bh * p.M * D;
  const int64_t kbase = (int64_t)bh * p.N * D;
  const int64_t lbase = (int64_t)bh * p.M;

  const T* Qp = (const T*)p.q + qbase;
  const T* Q2p = kPw ? (const T*)p.q2 + qbase : nullptr;
  const T* DOp = (const T*)p.dout + qbase;

  // K and V columns stay in registers: lane li feeds key kj as B operand.
  V8 kf[KK], k2f[kPw ? KK : 1], vf[KK];
  if (wave_valid) {
    const int64_t off = kbase + (int64_t)kj * D + 8 * h;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      kf[kk] = *reinterpret_cast<const V8*>((const T*)p.k + off + 16 * kk);
      vf[kk] = *reinterpret_cast<const V8*>((const T*)p.v + off + 16 * kk);
      if constexpr (kPw) k2f[kk] = *reinterpret_cast<const V8*>((const T*)p.k2 + off + 16 * kk);
    }
  }

  f32x16 dvt[DT], dkt[DT], dk2t[kPw ? DT : 1];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    dvt[dt] = zero16();
    dkt[dt] = zero16();
    if constexpr (kPw) dk2t[dt] = zero16();
  }

  // Query blocks to visit.
  int q_begin = 0;
  if (CAUSAL) q_begin = max(0, n0 - pshift) / kQB * kQB;
  const int nq = p.M > q_begin ? (p.M - q_begin + kQB - 1) / kQB : 0;
  const int wg_key_hi = min(p.N, n0 + kKB) - 1;

  RT ldq[NQ], lddo;
  TT ldqt[NQ], lddot;
  float ld_lse = 0.f, ld_delta = 0.f;
  bool ld_q[2] = {true, true};

  auto issue = [&](int qb) {
    const int i0 = q_begin + qb * kQB;
    const int64_t off = (int64_t)i0 * D;
    if constexpr (kPw) {
      bool an, af;
      pw_classify(i0, i0 + kQB - 1, n0, wg_key_hi, pshift, p.w, an, af);
      ld_q[0] = !af;
      ld_q[1] = !an;
      if (ld_q[0]) {
        ldq[0].load(Qp + off, tid);
        ldqt[0].load(Qp + off, tid);
      }
      if (ld_q[1]) {
        ldq[1].load(Q2p + off, tid);
        ldqt[1].load(Q2p + off, tid);
      }
    } else {
      ldq[0].load(Qp + off, tid);
      ldqt[0].load(Qp + off, tid);
    }
    lddo.load(DOp + off, tid);
    lddot.load(DOp + off, tid);
    if (tid < kQB) {
      ld_lse = lse_to_log2(p.lse[lbase + i0 + tid]);
      ld_delta = p.delta[lbase + i0 + tid];
    }
  };
  auto commit = [&](St& s) {
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      if (!kPw || ld_q[j]) {
        ldq[j].store(s.qrm[j], tid);
        ldqt[j].store(s.qtr[j], tid);
      }
    }
    lddo.store(s.dorm, tid);
    lddot.store(s.dotr, tid);
    if (tid < kQB) {
      s.lse2[tid] = ld_lse;
      s.delta[tid] = ld_delta;
    }
  };

  if (nq > 0) {
    issue(0);
    commit(smem[0]);
  }
  __builtin_amdgcn_s_waitcnt(0);  // resident K/V loads and the first block
  __syncthreads();

  // One query block for this wave; MASK selects the causal-diagonal path.
  auto block = [&](const St& cur, int i0, auto mask_tag) {
      constexpr bool need_mask = decltype(mask_tag)::value;
      bool an = true, af = false;
      if constexpr (kPw) pw_classify(i0, i0 + kQB - 1, kw0, kw0 + 31, pshift, p.w, an, af);
      f32x16 s[ST], dp[ST], dsf[kPw ? ST : 1];
#pragma unroll
      for (int st = 0; st < ST; ++st) {
        const int roff = (32 * st + li);
        // scores S = Q K^t (rows: queries, swap23 order; column: this key)
        if constexpr (kPw) {
          f32x16 s1 = zero16(), s2 = zero16();
          if (!af) {
            const T* qrow = cur.qrm[0] + roff * RT::PITCH + 8 * h;
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) s1 = mfma32x32x16(lds_read8(qrow + 16 * kk), kf[kk], s1);
          }
          if (!an) {
            const T* qrow = cur.qrm[1] + roff * RT::PITCH + 8 * h;
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) s2 = mfma32x32x16(lds_read8(qrow + 16 * kk), k2f[kk], s2);
          }
          if (an) {
            s[st] = s1;
          } else if (af) {
            s[st] = s2;
          } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int qrow_i = i0 + 32 * st + perm_row(r, h);
              s[st][r] = pw_near(qrow_i + pshift - kj, p.w) ? s1[r] : s2[r];
            }
          }
        } else {
          s[st] = zero16();
          const T* qrow = cur.qrm[0] + roff * RT::PITCH + 8 * h;
#pragma unroll
          for (int kk = 0; kk < KK; ++kk) s[st] = mfma32x32x16(lds_read8(qrow + 16 * kk), kf[kk], s[st]);
        }
        // dP = dO V^t
        dp[st] = zero16();
        const T* dorow = cur.dorm + roff * RT::PITCH + 8 * h;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) dp[st] = mfma32x32x16(lds_read8(dorow + 16 * kk), vf[kk], dp[st]);
        // P and dS
        const f32x4* l4 = reinterpret_cast<const f32x4*>(cur.lse2 + 32 * st + 8 * h);
        const f32x4* d4 = reinterpret_cast<const f32x4*>(cur.delta + 32 * st + 8 * h);
        f32x4 lv[4] = {l4[0], l4[1], l4[4], l4[5]};
        f32x4 dv4[4] = {d4[0], d4[1], d4[4], d4[5]};
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float l2 = lv[r >> 2][r & 3];
          const float dl = dv4[r >> 2][r & 3];
          float pv = exp2_fast(fmaf(s[st][r], p.scale2, -l2));
          if constexpr (need_mask) {
            const int qrow_i = i0 + 32 * st + perm_row(r, h);
            if (kj > qrow_i + pshift) pv = 0.f;
          }
          const float ds = pv * (dp[st][r] - dl);
          s[st][r] = pv;
          if constexpr (kPw) {
            if (an) {
              dp[st][r] = ds;
            } else if (af) {
              dp[st][r] = 0.f;
              dsf[st][r] = ds;
            } else {
              const int qrow_i = i0 + 32 * st + perm_row(r, h);
              const bool nr = pw_near(qrow_i + pshift - kj, p.w);
              dp[st][r] = nr ? ds : 0.f;
              dsf[st][r] = nr ? 0.f : ds;
            }
          } else {
            dp[st][r] = ds;
          }
        }
      }
      // dV^t += dO^t P ;  dK^t += Q^t dS
      V8 pb[PT], dsb[PT], dsfb[kPw ? PT : 1];
#pragma unroll
      for (int t = 0; t < PT; ++t) {
        pb[t] = pack8<T>(s[t >> 1], 8 * (t & 1));
        if (!kPw || !af) dsb[t] = pack8<T>(dp[t >> 1], 8 * (t & 1));
        if constexpr (kPw) {
          if (!an) dsfb[t] = pack8<T>(dsf[t >> 1], 8 * (t & 1));
        }
      }
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const T* dotrow = cur.dotr + (32 * dt + li) * TT::PITCH + 8 * h;
#pragma unroll
        for (int t = 0; t < PT; ++t) dvt[dt] = mfma32x32x16(lds_read8(dotrow + 16 * t), pb[t], dvt[dt]);
        if (!kPw || !af) {
          const T* qtrow = cur.qtr[0] + (32 * dt + li) * TT::PITCH + 8 * h;
#pragma unroll
          for (int t = 0; t < PT; ++t) dkt[dt] = mfma32x32x16(lds_read8(qtrow + 16 * t), dsb[t], dkt[dt]);
        }
        if constexpr (kPw) {
          if (!an) {
            const T* qtrow = cur.qtr[1] + (32 * dt + li) * TT::PITCH + 8 * h;
#pragma unroll
            for (int t = 0; t < PT; ++t) dk2t[dt] = mfma32x32x16(lds_read8(qtrow + 16 * t), dsfb[t], dk2t[dt]);
          }
        }
      }
  };

  for (int qb = 0; qb < nq; ++qb) {
    const St& cur = smem[qb & 1];
    if (qb + 1 < nq) issue(qb + 1);
    const int i0 = q_begin + qb * kQB;
    if (wave_valid && (!CAUSAL || i0 + kQB - 1 + pshift >= kw0)) {
      if (CAUSAL && (i0 + pshift < kw0 + 31))
        block(cur, i0, std::true_type{});
      else
        block(cur, i0, std::false_type{});
    }
    if (qb + 1 < nq) commit(smem[(qb + 1) & 1]);
    __syncthreads();
  }

  if (!wave_valid) return;
  const int64_t orow = kbase + (int64_t)kj * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    store_acc_t<T>((T*)p.dv + orow, dvt[dt], 32 * dt, h, 1.f);
    store_acc_t<T>((T*)p.dk + orow, dkt[dt], 32 * dt, h, p.sm_scale);
    if constexpr (kPw) store_acc_t<T>((T*)p.dk2 + orow, dk2t[dt], 32 * dt, h, p.sm_scale);
  }
}

// ---------------------------------------------------------------- dQ pass --
constexpr int kQW = 32 * kWaves;  // queries per workgroup

template <int D, int VAR>
struct DqCfg {
  // keys per streamed block; the piecewise D=128 stage is halved to fit LDS
  static constexpr int BN = (VAR == PW && D == 128) ? 32 : 64;
};

template <typename T, int D, int VAR>
struct alignas(16) DqStage {
  static constexpr int BN = DqCfg<D, VAR>::BN;
  using RT = RowTile<T, BN, D, kNT>;
  using TT = TransTile<T, BN, D, kNT>;
  static constexpr int NK = (VAR == PW) ? 2 : 1;
  T krm[NK][RT::ELEMS];
  T vrm[RT::ELEMS];
  T ktr[NK][TT::ELEMS];
};

template <typename T, int D, int VAR, bool CAUSAL>
__global__ __launch_bounds__(kNT) void attn_dq_kernel(const BwdParams p) {
  using V8 = typename Vec8<T>::type;
  using St = DqStage<T, D, VAR>;
  using RT = typename St::RT;
  using TT = typename St::TT;
  constexpr int BN = St::BN;
  constexpr int KK = D / 16;
  constexpr int DT = D / 32;
  constexpr int ST = BN / 32;
  constexpr int PT = BN / 16;
  constexpr bool kPw = VAR == PW;
  constexpr int NK = St::NK;

  __shared__ St smem[2];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int li = lane & 31, h = lane >> 5;

  const int bh = blockIdx.x % p.BH;
  int mb = blockIdx.x / p.BH;
  if (CAUSAL) mb = p.nblk - 1 - mb;
  const int m0 = mb * kQW;
  const int row0 = m0 + 32 * wave;
  const bool wave_valid = row0 < p.M;
  const int qi = row0 + li;
  const int pshift = p.N - p.M;
  const int64_t qbase = (int64_t)bh * p.M * D;
  const int64_t kbase = (int64_t)bh * p.N * D;

  const T* Kp = (const T*)p.k + kbase;
  const T* K2p = kPw ? (const T*)p.k2 + kbase : nullptr;
  const T* Vp = (const T*)p.v + kbase;

  V8 qf[KK], q2f[kPw ? KK : 1], dof[KK];
  float lse2 = __builtin_huge_valf(), dl = 0.f;
  if (wave_valid) {
    const int64_t off = qbase + (int64_t)qi * D + 8 * h;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      qf[kk] = *reinterpret_cast<const V8*>((const T*)p.q + off + 16 * kk);
      dof[kk] = *reinterpret_cast<const V8*>((const T*)p.dout + off + 16 * kk);
      if constexpr (kPw) q2f[kk] = *reinterpret_cast<const V8*>((const T*)p.q2 + off + 16 * kk);
    }
    lse2 = lse_to_log2(p.lse[(int64_t)bh * p.M + qi]);
    dl = p.delta[(int64_t)bh * p.M + qi];
  }

  f32x16 dqt[DT], dq2t[kPw ? DT : 1];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    dqt[dt] = zero16();
    if constexpr (kPw) dq2t[dt] = zero16();
  }

  const int wg_last_row = min(p.M, m0 + kQW) - 1;
  int n_end = p.N;
  if (CAUSAL) n_end = min(p.N, wg_last_row + pshift + 1);
  const int nkb = n_end > 0 ? (n_end + BN - 1) / BN : 0;

  RT ldk[NK], ldv;
  TT ldkt[NK];
  bool ld_k[2] = {true, true};

  auto issue = [&](int jb) {
    const int64_t off = (int64_t)jb * BN * D;
    if constexpr (kPw) {
      bool an, af;
      pw_classify(m0, wg_last_row, jb * BN, jb * BN + BN - 1, pshift, p.w, an, af);
      ld_k[0] = !af;
      ld_k[1] = !an;
      if (ld_k[0]) {
        ldk[0].load(Kp + off, tid);
        ldkt[0].load(Kp + off, tid);
      }
      if (ld_k[1]) {
        ldk[1].load(K2p + off, tid);
        ldkt[1].load(K2p + off, tid);
      }
    } else {
      ldk[0].load(Kp + off, tid);
      ldkt[0].load(Kp + off, tid);
    }
    ldv.load(Vp + off, tid);
  };
  auto commit = [&](St& s) {
#pragma unroll
    for (int j = 0; j < NK; ++j) {
      if (!kPw || ld_k[j]) {
        ldk[j].store(s.krm[j], tid);
        ldkt[j].store(s.ktr[j], tid);
      }
    }
    ldv.store(s.vrm, tid);
  };

  if (nkb > 0) {
    issue(0);
    commit(smem[0]);
  }
  __builtin_amdgcn_s_waitcnt(0);  // resident Q/dO loads and the first block
  __syncthreads();

  // One key block for this wave; MASK selects the causal-diagonal path.
  auto block = [&](const St& cur, int n0, auto mask_tag) {
      constexpr bool need_mask = decltype(mask_tag)::value;
      bool an = true, af = false;
      if constexpr (kPw) pw_classify(row0, row0 + 31, n0, n0 + BN - 1, pshift, p.w, an, af);
      f32x16 s[ST], dp[ST], dsf[kPw ? ST : 1];
#pragma unroll
      for (int st = 0; st < ST; ++st) {
        const int roff = 32 * st + li;
        if constexpr (kPw) {
          f32x16 s1 = zero16(), s2 = zero16();
          if (!af) {
            const T* krow = cur.krm[0] + roff * RT::PITCH + 8 * h;
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) s1 = mfma32x32x16(lds_read8(krow + 16 * kk), qf[kk], s1);
          }
          if (!an) {
            const T* krow = cur.krm[1] + roff * RT::PITCH + 8 * h;
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) s2 = mfma32x32x16(lds_read8(krow + 16 * kk), q2f[kk], s2);
          }
          if (an) {
            s[st] = s1;
          } else if (af) {
            s[st] = s2;
          } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = n0 + 32 * st + perm_row(r, h);
              s[st][r] = pw_near(qi + pshift - key, p.w) ? s1[r] : s2[r];
            }
          }
        } else {
          s[st] = zero16();
          const T* krow = cur.krm[0] + roff * RT::PITCH + 8 * h;
#pragma unroll
          for (int kk = 0; kk < KK; ++kk) s[st] = mfma32x32x16(lds_read8(krow + 16 * kk), qf[kk], s[st]);
        }
        dp[st] = zero16();
        const T* vrow = cur.vrm + roff * RT::PITCH + 8 * h;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) dp[st] = mfma32x32x16(lds_read8(vrow + 16 * kk), dof[kk], dp[st]);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = n0 + 32 * st + perm_row(r, h);
          float pv = exp2_fast(fmaf(s[st][r], p.scale2, -lse2));
          if constexpr (need_mask) {
            if (key > qi + pshift) pv = 0.f;
          }
          const float ds = pv * (dp[st][r] - dl);
          if constexpr (kPw) {
            if (an) {
              dp[st][r] = ds;
            } else if (af) {
              dp[st][r] = 0.f;
              dsf[st][r] = ds;
            } else {
              const bool nr = pw_near(qi + pshift - key, p.w);
              dp[st][r] = nr ? ds : 0.f;
              dsf[st][r] = nr ? 0.f : ds;
            }
          } else {
            dp[st][r] = ds;
          }
        }
      }
      V8 dsb[PT], dsfb[kPw ? PT : 1];
#pragma unroll
      for (int t = 0; t < PT; ++t) {
        if (!kPw || !af) dsb[t] = pack8<T>(dp[t >> 1], 8 * (t & 1));
        if constexpr (kPw) {
          if (!an) dsfb[t] = pack8<T>(dsf[t >> 1], 8 * (t & 1));
        }
      }
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        if (!kPw || !af) {
          const T* ktrow = cur.ktr[0] + (32 * dt + li) * TT::PITCH + 8 * h;
#pragma unroll
          for (int t = 0; t < PT; ++t) dqt[dt] = mfma32x32x16(lds_read8(ktrow + 16 * t), dsb[t], dqt[dt]);
        }
        if constexpr (kPw) {
          if (!an) {
            const T* ktrow = cur.ktr[1] + (32 * dt + li) * TT::PITCH + 8 * h;
#pragma unroll
            for (int t = 0; t < PT; ++t) dq2t[dt] = mfma32x32x16(lds_read8(ktrow + 16 * t), dsfb[t], dq2t[dt]);
          }
        }
      }
  };

  for (int jb = 0; jb < nkb; ++jb) {
    const St& cur = smem[jb & 1];
    if (jb + 1 < nkb) issue(jb + 1);
    const int n0 = jb * BN;
    if (wave_valid && (!CAUSAL || n0 <= row0 + 31 + pshift)) {
      if (CAUSAL && (n0 + BN - 1 > row0 + pshift))
        block(cur, n0, std::true_type{});
      else
        block(cur, n0, std::false_type{});
    }
    if (jb + 1 < nkb) commit(smem[(jb + 1) & 1]);
    __syncthreads();
  }

  if (!wave_valid) return;
  const int64_t orow = qbase + (int64_t)qi * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    store_acc_t<T>((T*)p.dq + orow, dqt[dt], 32 * dt, h, p.sm_scale);
    if constexpr (kPw) store_acc_t<T>((T*)p.dq2 + orow, dq2t[dt], 32 * dt, h, p.sm_scale);
  }
}

BwdParams make_params(const BwdArgs& a) {
  BwdParams p;
  p.q = a.q;
  p.k = a.k;
  p.v = a.v;
  p.q2 = a.q2;
  p.k2 = a.k2;
  p.dout = a.dout;
  p.lse = a.lse;
  p.delta = a.delta;
  p.dq = a.dq;
  p.dk = a.dk;
  p.dv = a.dv;
  p.dq2 = a.dq2;
  p.dk2 = a.dk2;
  p.BH = a.B * a.H;
  p.M = a.M;
  p.N = a.N;
  p.nblk = 0;
  p.scale2 = a.sm_scale * kLog2e;
  p.sm_scale = a.sm_scale;
  p.w = a.w;
  return p;
}

template <typename T, int D, int VAR>
hipError_t dkdv_t(const BwdArgs& a, hipStream_t s) {
  BwdParams p = make_params(a);
  p.nblk = (a.N + kKB - 1) / kKB;
  dim3 grid(p.nblk * p.BH), block(kNT);
  if (a.causal)
    hipLaunchKernelGGL((attn_dkdv_kernel<T, D, VAR, true>), grid, block, 0, s, p);
  else
    hipLaunchKernelGGL((attn_dkdv_kernel<T, D, VAR, false>), grid, block, 0, s, p);
  return hipGetLastError();
}

template <typename T, int D, int VAR>
hipError_t dq_t(const BwdArgs& a, hipStream_t s) {
  BwdParams p = make_params(a);
  p.nblk = (a.M + kQW - 1) / kQW;
  dim3 grid(p.nblk * p.BH), block(kNT);
  if (a.causal)
    hipLaunchKernelGGL((attn_dq_kernel<T, D, VAR, true>), grid, block, 0, s, p);
  else
    hipLaunchKernelGGL((attn_dq_kernel<T, D, VAR, false>), grid, block, 0, s, p);
  return hipGetLastError();
}

template <typename T, bool DKDV>
hipError_t dispatch(const BwdArgs& a, hipStream_t s) {
  const bool pw = a.variant == PW;
  if (a.D == 64) {
    if (DKDV) return pw ? dkdv_t<T, 64, PW>(a, s) : dkdv_t<T, 64, PLAIN>(a, s);
    return pw ? dq_t<T, 64, PW>(a, s) : dq_t<T, 64, PLAIN>(a, s);
  }
  if (a.D == 128) {
    if (DKDV) return pw ? dkdv_t<T, 128, PW>(a, s) : dkdv_t<T, 128, PLAIN>(a, s);
    return pw ? dq_t<T, 128, PW>(a, s) : dq_t<T, 128, PLAIN>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_attn_delta(int dtype, const void* o, const void* dout, float* delta, int64_t rows, int D,
                             hipStream_t s) {
  if (dtype == 0) return launch_delta_t<float>(o, dout, delta, rows, D, s);
  if (dtype == 1) return launch_delta_t<_Float16>(o, dout, delta, rows, D, s);
  if (dtype == 2) return launch_delta_t<__bf16>(o, dout, delta, rows, D, s);
  return hipErrorInvalidValue;
}

hipError_t launch_attn_dkdv(const BwdArgs& a, hipStream_t s) {
  if (a.dtype == 1) return dispatch<_Float16, true>(a, s);
  if (a.dtype == 2) return dispatch<__bf16, true>(a, s);
  return hipErrorInvalidValue;
}

hipError_t launch_attn_dq(const BwdArgs& a, hipStream_t s) {
  if (a.dtype == 1) return dispatch<_Float16, false>(a, s);
  if (a.dtype == 2) return dispatch<__bf16, false>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace fa
