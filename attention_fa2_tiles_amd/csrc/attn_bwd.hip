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
// (q2, k2) parts: a block wholly on one side of the rule runs the plain pass
// on that side's operands, a block that straddles it runs it twice, once
// per side with the other side's pairs masked (dV collects P from both).
//
// Layout on CDNA4 (both passes stream tiles through a three-stage LDS ring
// filled by direct global -> LDS loads, prefetching two blocks ahead; a
// two-stage ring at D = 256, whose passes run one wave per SIMD with the
// accumulators in AGPRs; head dim 16 runs the D = 32 kernels over rows
// zero-padded to 32 columns, template parameter G = 16):
//  * dK/dV pass: 32 keys per wave, 8 waves (4 for piecewise at D = 128 and
//    for D = 32, 256) per workgroup.
//    K stays in registers (B operand of S = Q K^t), each wave's 32 rows of V
//    stay in LDS (B operand of dP = dO V^t).  Query blocks of Q, dO and their
//    LSE / Delta rows stream through the ring.  Each lane owns one key, so P
//    and dS leave the score products already laid out as the B operands of
//    dV^t += dO^t P and dK^t += Q^t dS, whose A operands (dO^t, Q^t) are
//    transposing LDS reads of the same row-major tiles.
//  * dQ pass: 32 queries per wave, 8 waves (4 for piecewise at D = 128 and
//    for D = 32, 256) per workgroup,
//    Q and dO resident in registers; 64-key blocks of K and V stream through
//    the ring.  S^t = K Q^t and dP^t = V dO^t put one query per lane (LSE and
//    Delta are per-lane scalars) and dQ^t += K^t dS^t reads K^t with
//    transposing LDS reads of the K tile.
#include <type_traits>

#include "bwd_common.h"
#include "common.h"
#include "kernels.h"

namespace fa {

// The 16-bit D = 256 passes, in translation units of their own: one wave per
// SIMD with the accumulators in AGPRs (the other units keep MFMA results in
// VGPRs).
hipError_t bwd_dkdv_d256_f16(const BwdArgs& a, hipStream_t s);
hipError_t bwd_dkdv_d256_bf16(const BwdArgs& a, hipStream_t s);
hipError_t bwd_dq_d256_f16(const BwdArgs& a, hipStream_t s);
hipError_t bwd_dq_d256_bf16(const BwdArgs& a, hipStream_t s);

namespace {

constexpr int kLdsBytes = kBwdLdsBytes;

// ------------------------------------------------------------------ Delta --
template <typename T>
struct Row8 {
  T e[8];
};

template <typename T, int D>
__global__ __launch_bounds__(256) void delta_kernel(const T* __restrict__ o, const T* __restrict__ dout,
                                                    const float* __restrict__ dlse, float* __restrict__ delta,
                                                    int64_t rows) {
  constexpr int TPR = D / 8;      // threads per row
  constexpr int RPB = 256 / TPR;  // rows per block
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
  const int c = threadIdx.x % TPR;
  float sum = 0.f;
  if (row < rows) {
    const Row8<T> a = *reinterpret_cast<const Row8<T>*>(o + row * D + 8 * c);
    const Row8<T> b = *reinterpret_cast<const Row8<T>*>(dout + row * D + 8 * c);
#pragma unroll
    for (int e = 0; e < 8; ++e) sum = fmaf((float)a.e[e], (float)b.e[e], sum);
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) sum += __shfl_xor(sum, off, 64);
  // (the dQ pass that forms Delta itself sums in this same order)
  // A gradient reaching LSE adds P * dLSE to dS, i.e. it lowers Delta.
  if (row < rows && c == 0) delta[row] = dlse ? sum - dlse[row] : sum;
}

template <typename T>
hipError_t launch_delta_t(const void* o, const void* dout, const float* dlse, float* delta, int64_t rows,
                          int D, hipStream_t s) {
  const int64_t rpb = 256 / (D / 8);
  dim3 grid((unsigned)((rows + rpb - 1) / rpb)), block(256);
  if (D == 64)
    hipLaunchKernelGGL((delta_kernel<T, 64>), grid, block, 0, s, (const T*)o, (const T*)dout, dlse, delta, rows);
  else if (D == 128)
    hipLaunchKernelGGL((delta_kernel<T, 128>), grid, block, 0, s, (const T*)o, (const T*)dout, dlse, delta,
                       rows);
  else if (D == 32)
    hipLaunchKernelGGL((delta_kernel<T, 32>), grid, block, 0, s, (const T*)o, (const T*)dout, dlse, delta, rows);
  else if (D == 16)
    hipLaunchKernelGGL((delta_kernel<T, 16>), grid, block, 0, s, (const T*)o, (const T*)dout, dlse, delta, rows);
  else if (D == 256)
    hipLaunchKernelGGL((delta_kernel<T, 256>), grid, block, 0, s, (const T*)o, (const T*)dout, dlse, delta,
                       rows);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

// ============================================================ dK/dV pass ==
template <int D, int VAR>
struct DkdvShape {
  // D = 32 tiles are too small to split their loads over 8 waves; the
  // piecewise operand pairs fit 8 waves' registers only up to D = 64.
  // D = 256: the dV / dK accumulators alone take 256 registers, so one wave
  // per SIMD holds them (in AGPRs), and the ring has two stages (three
  // stages of 32 x 256 Q and dO tiles and the four waves' V rows would need
  // 160.75 KiB).
  static constexpr int WAVES = ((VAR == PW && D > 64) || D == 32 || D == 256) ? 4 : 8;
  static constexpr int NT = 64 * WAVES;
  static constexpr int KB = 32 * WAVES;                        // keys per workgroup
  static constexpr int QB = (D == 64 || D == 32) ? 64 : 32;    // query rows per streamed block
  static constexpr int NS = D == 256 ? 2 : 3;                  // ring stages
};

template <typename T, int D, int VAR>
struct alignas(16) DkdvStage {
  using Sh = DkdvShape<D, VAR>;
  using Tile = DTile<T, Sh::QB, D, Sh::WAVES>;
  static constexpr int NQ = (VAR == PW) ? 2 : 1;
  T dout[Tile::ELEMS];
  T q[NQ][Tile::ELEMS];       // Q (piecewise: Q1, Q2)
  float stats[2 * Sh::QB];    // LSE of the block's rows, then their Delta
};

template <typename T, int D, int VAR>
struct alignas(256) DkdvSmem {
  using Sh = DkdvShape<D, VAR>;
  using VTile = DTile<T, 32, D, 1, false>;  // natural key order
  DkdvStage<T, D, VAR> st[Sh::NS];
  T v[Sh::WAVES][VTile::ELEMS];
  // piecewise: each wave's 32 rows of K2 (the far side's B operand), read
  // from LDS like V to leave their registers to the accumulators
  T k2[(VAR == PW) ? Sh::WAVES * VTile::ELEMS : 1];
};

template <int D, int VAR>
constexpr int dkdv_waves_per_eu() {
  return DkdvShape<D, VAR>::WAVES / 4;
}

// RAGGED: M or N is not a multiple of 64 (the tail handling is compiled only
// into these instantiations).  G: the row length of the tensors (normally D;
// head dim 16 runs the D = 32 tiles with G = 16, the upper 16 columns zero
// in every operand and not stored).
template <typename T, int D, int VAR, bool CAUSAL, bool RAGGED, int G = D>
__global__ __launch_bounds__((DkdvShape<D, VAR>::NT))
__attribute__((amdgpu_waves_per_eu(dkdv_waves_per_eu<D, VAR>(), dkdv_waves_per_eu<D, VAR>())))
void attn_dkdv_kernel(const BwdParams p) {
  using Sh = DkdvShape<D, VAR>;
  constexpr int kWaves = Sh::WAVES;
  constexpr int QB = Sh::QB;
  constexpr int KB = Sh::KB;
  constexpr int NS = Sh::NS;
  using V8 = typename Vec8<T>::type;
  using Sm = DkdvSmem<T, D, VAR>;
  using St = DkdvStage<T, D, VAR>;
  using Tile = typename St::Tile;
  using VTile = DTile<T, 32, D, 1, false, G>;  // the layout of Sm::VTile, loaded from G-wide rows
  using Dma = DmaTile<T, QB, D, kWaves, true, G>;
  static_assert(G <= D, "rows no longer than the tile");
  constexpr int KK = D / 16;   // 16-wide k steps over the head dim
  constexpr int DT = D / 32;   // 32-wide d tiles of dK^t / dV^t
  constexpr int ST = QB / 32;  // 32-query score tiles per block
  constexpr int PT = QB / 16;  // 16-query operand slices per block
  constexpr bool kPw = VAR == PW;
  static_assert(sizeof(Sm) <= kLdsBytes, "LDS budget");
  static_assert(NS == 2 || NS == 3, "ring of two or three stages");

  __shared__ Sm smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int li = lane & 31, h = lane >> 5;

  // Heads vary fastest (one head's Q/dO stay in one XCD's L2).  Causal: key
  // block 0 is seen by every query, so natural order runs the longest
  // workgroups first.
  const int bh = blockIdx.x % p.BH;
  const int kb = blockIdx.x / p.BH;
  const int n0 = kb * KB;
  const int kw0 = n0 + 32 * wave;
  const bool wave_valid = kw0 < p.N;
  const int kj = kw0 + li;  // this lane's key
  const int pshift = p.N - p.M;
  const int64_t qbase = (int64_t)bh * p.M * G;
  const int64_t kbase = (int64_t)bh * p.N * G;
  const int64_t lbase = (int64_t)bh * p.M;

  // Resident operands: this wave's 32 rows of V (piecewise: and of K2) in
  // LDS, K (K1) columns in registers (lane li feeds key kj).  Keys past the
  // last one read the last key; their columns are not stored.
  V8 kf[KK];
  if (wave_valid) {
    const T* vsrc = (const T*)p.v + kbase + (int64_t)kw0 * G;
    const T* k2src = kPw ? (const T*)p.k2 + kbase + (int64_t)kw0 * G : vsrc;
    T* k2dst = smem.k2 + (kPw ? wave * VTile::ELEMS : 0);
    if (!RAGGED || p.N - kw0 >= 32) {
      VTile::load(smem.v[wave], vsrc, 0, lane);
      if constexpr (kPw) VTile::load(k2dst, k2src, 0, lane);
    } else {
      VTile::load_lim(smem.v[wave], vsrc, 0, lane, p.N - kw0);
      if constexpr (kPw) VTile::load_lim(k2dst, k2src, 0, lane, p.N - kw0);
    }
    const int64_t off = kbase + (int64_t)(RAGGED ? min(kj, p.N - 1) : kj) * G + 8 * h;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)  // (G < D: zero past the row's G columns)
      kf[kk] = (G >= D || 16 * kk + 8 * h < G) ? *reinterpret_cast<const V8*>((const T*)p.k + off + 16 * kk) : V8{};
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
  if (CAUSAL) q_begin = max(0, n0 - pshift) / QB * QB;
  const int nq = p.M > q_begin ? (p.M - q_begin + QB - 1) / QB : 0;
  const int wg_key_hi = min(p.N, n0 + KB) - 1;

  const T* gq = (const T*)p.q + qbase;
  const T* gq2 = kPw ? (const T*)p.q2 + qbase : gq;
  const T* gdo = (const T*)p.dout + qbase;
  Dma dma;
  dma.lane_offsets(wave, lane);

  // LSE / Delta rows of a block: 2 QB floats loaded with 4-byte direct loads,
  // E of them per wave, so every wave issues exactly one such load.  A
  // wave's E elements lie all in the LSE half or all in the Delta half (E
  // divides QB), so the source array is the same for the whole wave.
  constexpr int E = 2 * QB / kWaves;
  static_assert(64 % E == 0 && QB % E == 0, "row statistics split");
  const int st_first = wave * E;
  const int st_ins = st_first / 64;
  const bool st_lane = lane >= st_first % 64 && lane < st_first % 64 + E;
  const float* st_src = (st_first < QB ? p.lse : p.delta) + lbase;
  const int st_row = lane + (st_first < QB ? st_ins * 64 : st_ins * 64 - QB);  // row within a block

  // Issue the direct loads of query block qb into stage st; returns the
  // number of vector-memory instructions this wave issued.
  auto tload = [&](const T* g, T* lds, int nr) {
    if constexpr (RAGGED)
      dma.load_rows(g, lds, wave, lane, nr);
    else
      dma.load(g, lds, wave);
  };
  auto issue = [&](St& st, int qb) -> int {
    const int i0 = q_begin + qb * QB;
    const int64_t off = (int64_t)i0 * G;
    int n = Dma::PER_WAVE + 1;
    const int nr = p.M - i0;  // rows of this block that exist
    if constexpr (kPw) {
      bool an, af;
      pw_classify(i0, i0 + QB - 1, n0, wg_key_hi, pshift, p.w, an, af);
      if (!af) {
        tload(gq + off, st.q[0], nr);
        n += Dma::PER_WAVE;
      }
      if (!an) {
        tload(gq2 + off, st.q[kPw ? 1 : 0], nr);
        n += Dma::PER_WAVE;
      }
    } else {
      tload(gq + off, st.q[0], nr);
      n += Dma::PER_WAVE;
    }
    tload(gdo + off, st.dout, nr);
    // (a row past the last one gets LSE = +inf, so P = 0 for all of it, and
    // Delta = 0; its Q and dO rows load as zeros)
    const float* st_ptr = (!RAGGED || i0 + st_row < p.M)
                              ? st_src + (i0 + st_row)
                              : (st_first < QB ? &kPosInfF : reinterpret_cast<const float*>(kZero16));
    if (st_lane)
      __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)st_ptr,
                                       (void __attribute__((address_space(3)))*)(st.stats + st_ins * 64), 4, 0,
                                       0);
    return n;
  };
  // Wait until the loads of every block but the newest (n instructions)
  // have landed.  (Two stages: the newest block is the one needed next, so
  // every load is waited for.)
  auto wait_all_but = [&](int n) {
    if constexpr (NS == 2)
      wait_vmcnt0();
    else if constexpr (kPw)
      wait_vmcnt_any<3 * Dma::PER_WAVE + 1, 2 * Dma::PER_WAVE + 1>(n);
    else
      wait_vmcnt<2 * Dma::PER_WAVE + 1>();
  };

  // Prologue: resident loads, blocks 0 .. NS-2 in flight, block 0 landed.
  int n_new = 0;
#pragma unroll
  for (int j = 0; j < NS - 1; ++j)
    if (j < nq) n_new = issue(smem.st[j], j);
  if (nq > 1)
    wait_all_but(n_new);
  else
    wait_vmcnt0();
  // The resident V tile is stored negated (each wave flips the sign bits of
  // its own rows), so that the dP accumulator can start at +Delta:
  // Delta + dO (-V)^t = -(dP - Delta), i.e. the pass computes -dS, and dK is
  // stored with scale -sm_scale.
  if (wave_valid) {
    constexpr int kChunks = VTile::ELEMS * 2 / 16 / 64;
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      u32x4* c = reinterpret_cast<u32x4*>(smem.v[wave]) + i * 64 + lane;
      *c = *c ^ 0x80008000u;
    }
  }
  lds_barrier();

  // Loop-invariant LDS byte offsets.  Row reads: row li, chunk 2 kk + h of a
  // Q/dO tile (swap23 rows) or of this wave's V tile (natural rows).
  uint32_t rofs[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) rofs[kk] = row_chunk_ofs<D>(li, 2 * kk + h);
  TrAddr<D> tra;
  tra.init(&smem, TrLane(lane));
  const char* sbase = reinterpret_cast<const char*>(&smem);
  auto rd8 = [&](int off, int kk) -> V8 {
    return *reinterpret_cast<const V8*>(sbase + off + rofs[kk]);
  };
  const int voff = (int)(reinterpret_cast<const char*>(smem.v[wave]) - sbase);
  const int k2off = (int)(reinterpret_cast<const char*>(smem.k2 + (kPw ? wave * VTile::ELEMS : 0)) - sbase);
  const float neg_inv_scale = -1.f / p.sm_scale;

  // One query block for this wave from stage S.  SEL picks the score
  // operands and the dK accumulator: 0 = (Q tile, K, dK), 1 = (Q2 tile, K2,
  // dK2) (piecewise only); dV takes P from either.  MODE masks pairs: none,
  // the causal diagonal, or one side of the piecewise rule on a block that
  // straddles it (each side also under the causal mask).  A masked pair's
  // score starts at -inf, so its P and dS are 0; rows with LSE = -inf (no
  // visible key) only occur in causal blocks whose every pair is masked.
  auto sub = [&](auto stage_c, int i0, auto sel_c, auto mode_c) {
    constexpr int S = decltype(stage_c)::value;
    constexpr int SEL = decltype(sel_c)::value;
    constexpr int MODE = decltype(mode_c)::value;
    constexpr int kSt = (int)(__builtin_offsetof(Sm, st) + S * sizeof(St));
    constexpr int kDo = kSt + (int)__builtin_offsetof(St, dout);
    constexpr int kQs = kSt + (int)__builtin_offsetof(St, q) + SEL * Tile::ELEMS * 2;
    const St& cur = smem.st[S];
    auto& dks = pick<SEL>(dkt, dk2t);
    // B operand of the score product: K from registers, K2 from LDS
    auto kop = [&](int kk) -> V8 {
      if constexpr (SEL == 0)
        return kf[kk];
      else
        return rd8(k2off, kk);
    };
    f32x16 s[ST], dp[ST];
#pragma unroll
    for (int st = 0; st < ST; ++st) {
      // The score accumulator starts at -LSE / sm_scale and the dP one at
      // +Delta (this lane's 16 rows): scale2 * S is then the exponent of P
      // and the second product gives -(dP - Delta).
      {
        const f32x4* l4 = reinterpret_cast<const f32x4*>(cur.stats + 32 * st + 8 * h);
        const f32x4* d4 = reinterpret_cast<const f32x4*>(cur.stats + QB + 32 * st + 8 * h);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 lv = l4[(g & 1) + 4 * (g >> 1)];
          const f32x4 dv = d4[(g & 1) + 4 * (g >> 1)];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            s[st][4 * g + e] = lv[e] * neg_inv_scale;
            dp[st][4 * g + e] = dv[e];
          }
        }
      }
      if constexpr (MODE != kMaskNone) {
        // row i0 + 32 st + perm_row(r, h) sits at distance perm_row(r, 0) - c0
        // from key kj
        const int c0 = kj - pshift - i0 - 32 * st - 8 * h;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (!pair_kept<MODE, CAUSAL>(perm_row(r, 0) - c0, p.w)) s[st][r] = kNegInf;
      }
      // S = Q K^t and Delta - dP = Delta + dO (-V)^t, interleaved
      const int so = st * 32 * D * 2;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        s[st] = mfma32x32x16(rd8(kQs + so, kk), kop(kk), s[st]);
        dp[st] = mfma32x32x16(rd8(kDo + so, kk), rd8(voff, kk), dp[st]);
      }
    }
    V8 pb[PT], dsb[PT];
    // P and -dS of operand slot t (8 rows of the score tile): exponent,
    // product with Delta - dP, packing.  Element e of slot t is formed right after
    // the e-th product of the accumulation of slot t - 1: a wave's vector
    // work overlaps matrix work best when it sits between its own products
    // (with two waves per SIMD); slot 0 has nothing before it to hide under.
    constexpr int kPer = 8 / (2 * DT) > 0 ? 8 / (2 * DT) : 1;  // elements per product
    static_assert(8 % (2 * DT) == 0 || 2 * DT % 8 == 0, "slot split");
    auto element = [&](auto tc, auto ec) {
      constexpr int t = decltype(tc)::value, e = decltype(ec)::value;
      constexpr int st = t >> 1, r = 8 * (t & 1) + e;
      const float pv = exp2_fast(s[st][r] * p.scale2);
      dp[st][r] = pv * dp[st][r];  // -dS
      s[st][r] = pv;
      if constexpr (e == 7) {
        pb[t] = pack8<T>(s[st], 8 * (t & 1));
        dsb[t] = pack8<T>(dp[st], 8 * (t & 1));
      }
    };
    static_for<8>([&](auto ec) { element(ic<0>{}, ec); });
    // dV^t += dO^t P ;  -dK^t += Q^t (-dS), slot by slot, d-tile by d-tile;
    // the two transposing operands of step k + 1 are read during step k.
    TrOps<T, 1> xo[2], yo[2];
    auto rd = [&](auto kc) {
      constexpr int k = decltype(kc)::value, t = k / DT, dt = k % DT;
      tr_issue<T, D, 1, kDo + t * 16 * D * 2>(xo[k & 1], tra, dt);
      tr_issue<T, D, 1, kQs + t * 16 * D * 2>(yo[k & 1], tra, dt);
    };
    rd(ic<0>{});
    static_for<PT * DT>([&](auto kc) {
      constexpr int k = decltype(kc)::value, t = k / DT, dt = k % DT;
      if constexpr (k + 1 < PT * DT) {
        rd(ic<k + 1>{});
        asm volatile("s_waitcnt lgkmcnt(4)" : "+v"(xo[k & 1].op[0]), "+v"(yo[k & 1].op[0]));
      } else {
        asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(xo[k & 1].op[0]), "+v"(yo[k & 1].op[0]));
      }
      // elements of slot t + 1 placed after this step's two products (D =
      // 256: one after each of the first eight products)
      constexpr int e0 = 2 * dt * kPer;
      dvt[dt] = mfma32x32x16(xo[k & 1].op[0], pb[t], dvt[dt]);
      if constexpr (t + 1 < PT) {
        static_for<kPer>([&](auto uc) {
          if constexpr (e0 + decltype(uc)::value < 8) element(ic<t + 1>{}, ic<e0 + decltype(uc)::value>{});
        });
      }
      __builtin_amdgcn_sched_barrier(0);
      dks[dt] = mfma32x32x16(yo[k & 1].op[0], dsb[t], dks[dt]);
      if constexpr (t + 1 < PT) {
        static_for<kPer>([&](auto uc) {
          if constexpr (e0 + kPer + decltype(uc)::value < 8)
            element(ic<t + 1>{}, ic<e0 + kPer + decltype(uc)::value>{});
        });
      }
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  // One query block for this wave from stage S; MASK: a causal-diagonal
  // block.  Piecewise: a block wholly on one side of the rule is one pass
  // with that side's operands; a block that straddles it is two passes, each
  // masked to its side.
  auto block = [&](auto stage_c, int i0, auto mask_tag) {
    constexpr int M0 = decltype(mask_tag)::value ? kMaskCausal : kMaskNone;
    if constexpr (!kPw) {
      sub(stage_c, i0, ic<0>{}, ic<M0>{});
    } else {
      bool an, af;
      pw_classify(i0, i0 + QB - 1, kw0, kw0 + 31, pshift, p.w, an, af);
      if (an) {
        sub(stage_c, i0, ic<0>{}, ic<M0>{});
      } else if (af) {
        sub(stage_c, i0, ic<1>{}, ic<M0>{});
      } else {
        sub(stage_c, i0, ic<0>{}, ic<kMaskNear>{});
        sub(stage_c, i0, ic<1>{}, ic<kMaskFar>{});
      }
    }
  };

  // Block qb is computed from stage qb % NS while block qb + NS - 1 is being
  // loaded into the stage freed by block qb - 1.  The stage index is a
  // compile-time constant in each of the three unrolled steps, so every LDS
  // address is a per-lane register plus an immediate.
  auto step = [&](auto stage_c, int qb) {
    constexpr int S = decltype(stage_c)::value;
    constexpr int LD = (S + NS - 1) % NS;
    const int ahead = qb + NS - 1;
    const bool issued = ahead < nq;
    if (issued) n_new = issue(smem.st[LD], ahead);
    const int i0 = q_begin + qb * QB;
    const bool active = wave_valid && (!CAUSAL || i0 + QB - 1 + pshift >= kw0);
    if (active) {
      if (CAUSAL && (kw0 + 31 > i0 + pshift))
        block(stage_c, i0, std::true_type{});
      else
        block(stage_c, i0, std::false_type{});
    }
    if (issued)
      wait_all_but(n_new);
    else
      wait_vmcnt0();
    lds_barrier();
  };
  for (int qb = 0; qb < nq; qb += NS) {
    static_for<NS>([&](auto sc) {
      if (qb + decltype(sc)::value < nq) step(sc, qb + decltype(sc)::value);
    });
  }

  // The LDS is free after the last barrier: each wave stages its dV and dK
  // tiles through its own part of it and stores whole rows (keys past the
  // last one are not stored).
  if (!wave_valid) return;
  const float dk_scale = -p.sm_scale;
  static_assert(kWaves * RowStage<D>::kStageBytes <= (int)sizeof(Sm), "output staging fits in the LDS");
  char* stage = reinterpret_cast<char*>(&smem) + wave * RowStage<D>::kStageBytes;
  const int nrows = RAGGED ? p.N - kw0 : 32;
  const int64_t orow = kbase + (int64_t)kw0 * G;
  store_tile_rows<T, D, G>((T*)p.dv + orow, nrows, dvt, 1.f, stage, lane);
  store_tile_rows<T, D, G>((T*)p.dk + orow, nrows, dkt, dk_scale, stage, lane);
  if constexpr (kPw) store_tile_rows<T, D, G>((T*)p.dk2 + orow, nrows, dk2t, dk_scale, stage, lane);
}

// =============================================================== dQ pass ==
template <int D, int VAR>
struct DqShape {
  // D = 256: Q, dO (128 registers) and the dQ accumulators (128) fill one
  // wave per SIMD; two ring stages of 64 x 256 K and V tiles (128 KiB)
  static constexpr int WAVES = ((VAR == PW && D > 64) || D == 32 || D == 256) ? 4 : 8;
  static constexpr int NT = 64 * WAVES;
  static constexpr int BM = 32 * WAVES;  // queries per workgroup
  static constexpr int BN = 64;          // keys per streamed block
  static constexpr int NS = D == 256 ? 2 : 3;  // ring stages
};

// Ring of K (K1), K2 and V tiles, grouped by kind so that the transposing
// reads of the K tiles have small immediate offsets.
template <typename T, int D, int VAR>
struct alignas(256) DqSmem {
  using Sh = DqShape<D, VAR>;
  using Tile = DTile<T, Sh::BN, D, Sh::WAVES>;
  static constexpr int NK = (VAR == PW) ? 2 : 1;
  T k[NK][Sh::NS][Tile::ELEMS];  // K (piecewise: K1, K2)
  T v[Sh::NS][Tile::ELEMS];
};

template <int D, int VAR>
constexpr int dq_waves_per_eu() {
  return DqShape<D, VAR>::WAVES / 4;
}

template <typename T, int D, int VAR, bool CAUSAL, bool RAGGED, int G = D>
__global__ __launch_bounds__((DqShape<D, VAR>::NT))
__attribute__((amdgpu_waves_per_eu(dq_waves_per_eu<D, VAR>(), dq_waves_per_eu<D, VAR>())))
void attn_dq_kernel(const BwdParams p) {
  using Sh = DqShape<D, VAR>;
  constexpr int kWaves = Sh::WAVES;
  constexpr int BM = Sh::BM;
  constexpr int BN = Sh::BN;
  constexpr int NS = Sh::NS;
  using V8 = typename Vec8<T>::type;
  using Sm = DqSmem<T, D, VAR>;
  using Tile = typename Sm::Tile;
  using Dma = DmaTile<T, BN, D, kWaves, true, G>;
  static_assert(G <= D, "rows no longer than the tile");
  constexpr int KK = D / 16;
  constexpr int DT = D / 32;
  constexpr int ST = BN / 32;
  constexpr int PT = BN / 16;
  constexpr bool kPw = VAR == PW;
  static_assert(sizeof(Sm) <= kLdsBytes, "LDS budget");
  static_assert(NS == 2 || NS == 3, "ring of two or three stages");

  __shared__ Sm smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int li = lane & 31, h = lane >> 5;

  // Heads vary fastest; causal: the longest query blocks (last rows) first.
  const int bh = blockIdx.x % p.BH;
  int mb = blockIdx.x / p.BH;
  if (CAUSAL) mb = p.nblk - 1 - mb;
  const int m0 = mb * BM;
  const int row0 = m0 + 32 * wave;
  const bool wave_valid = row0 < p.M;
  const int qi = row0 + li;
  const int pshift = p.N - p.M;
  const int64_t qbase = (int64_t)bh * p.M * G;
  const int64_t kbase = (int64_t)bh * p.N * G;

  const T* gk = (const T*)p.k + kbase;
  const T* gk2 = kPw ? (const T*)p.k2 + kbase : gk;
  const T* gv = (const T*)p.v + kbase;
  Dma dma;
  dma.lane_offsets(wave, lane);

  // Query-side operands stay in registers for the whole pass.
  // (lanes past the last query row read that row; their results are not stored)
  V8 qf[KK], q2f[kPw ? KK : 1], dof[KK];
  V8 of[KK];  // this row's O chunks, when the pass forms Delta
  float lse2 = __builtin_huge_valf(), dl = 0.f;
  const int qr = RAGGED ? min(qi, p.M - 1) : qi;
  // chunk 2 kk + h of a row (G < D: zero past the row's G columns)
  auto chunk = [&](const void* base, int64_t off, int kk) -> V8 {
    if (G >= D || 16 * kk + 8 * h < G) return *reinterpret_cast<const V8*>((const T*)base + off + 16 * kk);
    return V8{};
  };
  if (wave_valid) {
    const int64_t off = qbase + (int64_t)qr * G + 8 * h;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      qf[kk] = chunk(p.q, off, kk);
      dof[kk] = chunk(p.dout, off, kk);
      if constexpr (kPw) q2f[kk] = chunk(p.q2, off, kk);
    }
    lse2 = lse_to_log2(p.lse[(int64_t)bh * p.M + qr]);
    if (p.delta_out) {
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) of[kk] = chunk(p.o, off, kk);
    } else {
      dl = p.delta[(int64_t)bh * p.M + qr];
    }
  }

  f32x16 dqt[DT], dq2t[kPw ? DT : 1];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    dqt[dt] = zero16();
    if constexpr (kPw) dq2t[dt] = zero16();
  }

  const int wg_last_row = min(p.M, m0 + BM) - 1;
  int n_end = p.N;
  if (CAUSAL) n_end = min(p.N, wg_last_row + pshift + 1);
  const int nkb = n_end > 0 ? (n_end + BN - 1) / BN : 0;

  // Issue the direct loads of key block jb into ring stage S; returns the
  // number of load instructions this wave issued.
  auto tload = [&](const T* g, T* lds, int nr) {
    if constexpr (RAGGED)
      dma.load_rows(g, lds, wave, lane, nr);
    else
      dma.load(g, lds, wave);
  };
  auto issue = [&](int S, int jb) -> int {
    const int64_t off = (int64_t)jb * BN * G;
    const int nr = p.N - jb * BN;  // rows of this block that exist
    int n = Dma::PER_WAVE;
    if constexpr (kPw) {
      bool an, af;
      pw_classify(m0, wg_last_row, jb * BN, jb * BN + BN - 1, pshift, p.w, an, af);
      if (!af) {
        tload(gk + off, smem.k[0][S], nr);
        n += Dma::PER_WAVE;
      }
      if (!an) {
        tload(gk2 + off, smem.k[kPw ? 1 : 0][S], nr);
        n += Dma::PER_WAVE;
      }
    } else {
      tload(gk + off, smem.k[0][S], nr);
      n += Dma::PER_WAVE;
    }
    tload(gv + off, smem.v[S], nr);
    return n;
  };
  // (two stages: every load is waited for, as in the dK/dV pass)
  auto wait_all_but = [&](int n) {
    if constexpr (NS == 2)
      wait_vmcnt0();
    else if constexpr (kPw)
      wait_vmcnt_any<3 * Dma::PER_WAVE, 2 * Dma::PER_WAVE>(n);
    else
      wait_vmcnt<2 * Dma::PER_WAVE>();
  };

  // Prologue: blocks 0 .. NS-2 are issued right behind the query operands
  // (all but the newest block's loads, the query operands included, have
  // landed after the wait).
  int n_new = 0;
#pragma unroll
  for (int j = 0; j < NS - 1; ++j)
    if (j < nkb) n_new = issue(j, j);
  if (nkb > 1)
    wait_all_but(n_new);
  else
    wait_vmcnt0();
  lds_barrier();

  if (wave_valid && p.delta_out) {
    // Delta_i = sum_d O_id dO_id - dLSE_i, in the delta kernel's order: fma
    // chains over 16-byte chunks, then the chunk sums pairwise with stride
    // half the chunk count (chunk 2 kk + h sits in slot kk of half h)
    float cs[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      cs[kk] = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) cs[kk] = fmaf((float)of[kk][e], (float)dof[kk][e], cs[kk]);
    }
#pragma unroll
    for (int half = KK / 2; half >= 1; half /= 2) {
#pragma unroll
      for (int kk = 0; kk < half; ++kk) cs[kk] += cs[kk + half];
    }
    dl = halves_sum(cs[0]);
    if (p.dlse) dl -= p.dlse[(int64_t)bh * p.M + qr];
    if (h == 0 && (!RAGGED || qi < p.M)) p.delta_out[(int64_t)bh * p.M + qi] = dl;
  }

  uint32_t rofs[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) rofs[kk] = row_chunk_ofs<D>(li, 2 * kk + h);
  TrAddr<D> tra;
  tra.init(&smem, TrLane(lane));
  const char* sbase = reinterpret_cast<const char*>(&smem);
  auto rd8 = [&](int off, int kk) -> V8 {
    return *reinterpret_cast<const V8*>(sbase + off + rofs[kk]);
  };

  // One key block for this wave from stage S.  SEL picks the score operands
  // and the accumulator: 0 = (K tile, Q, dQ), 1 = (K2 tile, Q2, dQ2)
  // (piecewise only).  MODE masks pairs: none, the causal diagonal, or one
  // side of the piecewise rule on a block that straddles it (each side also
  // under the causal mask); a masked pair's score starts at -inf, so P = 0.
  // The vector work of each score tile is spread between matrix products
  // that do not depend on it (a wave's vector work overlaps matrix work best
  // when it sits between its own products, with two waves per SIMD): tile
  // 0's P / dS between tile 1's score products, tile 1's between the dQ
  // products of tile 0.
  auto sub = [&](auto stage_c, int n0, auto sel_c, auto mode_c) {
    constexpr int S = decltype(stage_c)::value;
    constexpr int SEL = decltype(sel_c)::value;
    constexpr int MODE = decltype(mode_c)::value;
    constexpr int kKs = (int)(__builtin_offsetof(Sm, k) + (SEL * NS + S) * Tile::ELEMS * 2);
    constexpr int kV = (int)(__builtin_offsetof(Sm, v) + S * Tile::ELEMS * 2);
    static_assert(ST == 2 && PT == 4, "two score tiles of 32 keys");
    auto& qs = pick<SEL>(qf, q2f);
    auto& acc = pick<SEL>(dqt, dq2t);
    V8 dsb[PT];
    f32x16 s[ST], dp[ST];
#pragma unroll
    for (int st = 0; st < ST; ++st) {
      s[st] = zero16();
      dp[st] = zero16();
      if constexpr (MODE != kMaskNone) {
        // key n0 + 32 st + perm_row(r, h) sits at distance c1 - perm_row(r, 0)
        // from this query
        const int c1 = qi + pshift - n0 - 32 * st - 8 * h;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (!pair_kept<MODE, CAUSAL>(c1 - perm_row(r, 0), p.w)) s[st][r] = kNegInf;
      }
    }
    // element r of tile st: P, dS = P (dP - Delta), packed per 8 rows.  The
    // exponent is at most 0 for every key that exists (LSE bounds each of
    // its row's scores); with ragged lengths it is clamped there, so that a
    // zero-filled key past the last one (S = 0) cannot overflow P when LSE
    // is very negative (its dS then meets a zero K row).
    auto element = [&](auto stc, auto rc) {
      constexpr int st = decltype(stc)::value, r = decltype(rc)::value;
      const float x = fmaf(s[st][r], p.scale2, -lse2);
      const float pv = exp2_fast(RAGGED ? fminf(x, 0.f) : x);
      dp[st][r] = pv * (dp[st][r] - dl);
      if constexpr (r % 8 == 7) dsb[2 * st + r / 8] = pack8<T>(dp[st], r - 7);
    };
    // S^t = K Q^t (rows: keys in swap23 order; column: this query) and
    // dP^t = V dO^t of tile st; after product pair kk, between(kk)
    auto products = [&](auto stc, auto&& between) {
      constexpr int st = decltype(stc)::value;
      constexpr int so = st * 32 * D * 2;
      static_for<KK>([&](auto kc) {
        constexpr int kk = decltype(kc)::value;
        s[st] = mfma32x32x16(rd8(kKs + so, kk), qs[kk], s[st]);
        dp[st] = mfma32x32x16(rd8(kV + so, kk), dof[kk], dp[st]);
        between(kc);
        __builtin_amdgcn_sched_barrier(0);
      });
    };
    products(ic<0>{}, [](auto) {});
    constexpr int kPerKK = 16 / KK;  // tile-0 elements per product pair
    products(ic<1>{}, [&](auto kc) {
      constexpr int kk = decltype(kc)::value;
      static_for<kPerKK>([&](auto uc) { element(ic<0>{}, ic<kk * kPerKK + decltype(uc)::value>{}); });
    });
    // dQ^t += K^t dS^t slot by slot, d-tile by d-tile; the transposing
    // operand of step k + 1 is read during step k; tile 1's elements sit
    // between the products of slots 0 and 1.
    TrOps<T, 1> ko[2];
    auto rd = [&](auto kc) {
      constexpr int k = decltype(kc)::value, t = k / DT, dt = k % DT;
      tr_issue<T, D, 1, kKs + t * 16 * D * 2>(ko[k & 1], tra, dt);
    };
    constexpr int kPerStep = 16 / (2 * DT);  // tile-1 elements per product of slots 0, 1
    rd(ic<0>{});
    static_for<PT * DT>([&](auto kc) {
      constexpr int k = decltype(kc)::value, t = k / DT, dt = k % DT;
      if constexpr (k + 1 < PT * DT) {
        rd(ic<k + 1>{});
        asm volatile("s_waitcnt lgkmcnt(2)" : "+v"(ko[k & 1].op[0]));
      } else {
        asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(ko[k & 1].op[0]));
      }
      acc[dt] = mfma32x32x16(ko[k & 1].op[0], dsb[t], acc[dt]);
      if constexpr (t < 2) {
        static_for<kPerStep>([&](auto uc) { element(ic<1>{}, ic<k * kPerStep + decltype(uc)::value>{}); });
      }
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  // One key block for this wave from stage S; MASK: a causal-diagonal
  // block.  Piecewise: a block wholly on one side of the rule is one pass
  // with that side's operands; a block that straddles it is two passes, each
  // masked to its side.
  auto block = [&](auto stage_c, int n0, auto mask_tag) {
    constexpr int M0 = decltype(mask_tag)::value ? kMaskCausal : kMaskNone;
    if constexpr (!kPw) {
      sub(stage_c, n0, ic<0>{}, ic<M0>{});
    } else {
      bool an, af;
      pw_classify(row0, row0 + 31, n0, n0 + BN - 1, pshift, p.w, an, af);
      if (an) {
        sub(stage_c, n0, ic<0>{}, ic<M0>{});
      } else if (af) {
        sub(stage_c, n0, ic<1>{}, ic<M0>{});
      } else {
        sub(stage_c, n0, ic<0>{}, ic<kMaskNear>{});
        sub(stage_c, n0, ic<1>{}, ic<kMaskFar>{});
      }
    }
  };

  auto step = [&](auto stage_c, int jb) {
    constexpr int S = decltype(stage_c)::value;
    constexpr int LD = (S + NS - 1) % NS;
    const int ahead = jb + NS - 1;
    const bool issued = ahead < nkb;
    if (issued) n_new = issue(LD, ahead);
    const int n0 = jb * BN;
    const bool active = wave_valid && (!CAUSAL || n0 <= row0 + 31 + pshift);
    if (active) {
      if (CAUSAL && (n0 + BN - 1 > row0 + pshift))
        block(stage_c, n0, std::true_type{});
      else
        block(stage_c, n0, std::false_type{});
    }
    if (issued)
      wait_all_but(n_new);
    else
      wait_vmcnt0();
    lds_barrier();
  };
  for (int jb = 0; jb < nkb; jb += NS) {
    static_for<NS>([&](auto sc) {
      if (jb + decltype(sc)::value < nkb) step(sc, jb + decltype(sc)::value);
    });
  }

  // The ring is free after the last barrier: each wave stages its dQ tile
  // through its own part of it and stores whole rows (rows past the last one
  // are not stored).
  if (!wave_valid) return;
  static_assert(kWaves * RowStage<D>::kStageBytes <= (int)sizeof(Sm), "output staging fits in the LDS");
  char* stage = reinterpret_cast<char*>(&smem) + wave * RowStage<D>::kStageBytes;
  const int nrows = RAGGED ? p.M - row0 : 32;
  const int64_t orow = qbase + (int64_t)row0 * G;
  store_tile_rows<T, D, G>((T*)p.dq + orow, nrows, dqt, p.sm_scale, stage, lane);
  if constexpr (kPw) store_tile_rows<T, D, G>((T*)p.dq2 + orow, nrows, dq2t, p.sm_scale, stage, lane);
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
  p.o = a.o;
  p.dlse = a.dlse;
  p.delta_out = a.delta_out;
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

template <typename T, int D, int VAR, int G = D>
hipError_t dkdv_t(const BwdArgs& a, hipStream_t s) {
  using Sh = DkdvShape<D, VAR>;
  BwdParams p = make_params(a);
  p.nblk = (a.N + Sh::KB - 1) / Sh::KB;
  dim3 grid(p.nblk * p.BH), block(Sh::NT);
  const bool ragged = a.M % 64 != 0 || a.N % 64 != 0;
  if (a.causal && ragged)
    hipLaunchKernelGGL((attn_dkdv_kernel<T, D, VAR, true, true, G>), grid, block, 0, s, p);
  else if (a.causal)
    hipLaunchKernelGGL((attn_dkdv_kernel<T, D, VAR, true, false, G>), grid, block, 0, s, p);
  else if (ragged)
    hipLaunchKernelGGL((attn_dkdv_kernel<T, D, VAR, false, true, G>), grid, block, 0, s, p);
  else
    hipLaunchKernelGGL((attn_dkdv_kernel<T, D, VAR, false, false, G>), grid, block, 0, s, p);
  return hipGetLastError();
}

template <typename T, int D, int VAR, int G = D>
hipError_t dq_t(const BwdArgs& a, hipStream_t s) {
  using Sh = DqShape<D, VAR>;
  BwdParams p = make_params(a);
  p.nblk = (a.M + Sh::BM - 1) / Sh::BM;
  dim3 grid(p.nblk * p.BH), block(Sh::NT);
  const bool ragged = a.M % 64 != 0 || a.N % 64 != 0;
  if (a.causal && ragged)
    hipLaunchKernelGGL((attn_dq_kernel<T, D, VAR, true, true, G>), grid, block, 0, s, p);
  else if (a.causal)
    hipLaunchKernelGGL((attn_dq_kernel<T, D, VAR, true, false, G>), grid, block, 0, s, p);
  else if (ragged)
    hipLaunchKernelGGL((attn_dq_kernel<T, D, VAR, false, true, G>), grid, block, 0, s, p);
  else
    hipLaunchKernelGGL((attn_dq_kernel<T, D, VAR, false, false, G>), grid, block, 0, s, p);
  return hipGetLastError();
}

template <typename T, bool DKDV>
hipError_t dispatch(const BwdArgs& a, hipStream_t s) {
  const bool pw = a.variant == PW;
  if (a.D == 64) {
    if constexpr (DKDV) return pw ? dkdv_t<T, 64, PW>(a, s) : dkdv_t<T, 64, PLAIN>(a, s);
    else return pw ? dq_t<T, 64, PW>(a, s) : dq_t<T, 64, PLAIN>(a, s);
  }
  if (a.D == 128) {
    if constexpr (DKDV) return pw ? dkdv_t<T, 128, PW>(a, s) : dkdv_t<T, 128, PLAIN>(a, s);
    else return pw ? dq_t<T, 128, PW>(a, s) : dq_t<T, 128, PLAIN>(a, s);
  }
  if (a.D == 32) {
    if constexpr (DKDV) return pw ? dkdv_t<T, 32, PW>(a, s) : dkdv_t<T, 32, PLAIN>(a, s);
    else return pw ? dq_t<T, 32, PW>(a, s) : dq_t<T, 32, PLAIN>(a, s);
  }
  if (a.D == 16) {  // the D = 32 kernels over zero-padded tiles
    if constexpr (DKDV) return pw ? dkdv_t<T, 32, PW, 16>(a, s) : dkdv_t<T, 32, PLAIN, 16>(a, s);
    else return pw ? dq_t<T, 32, PW, 16>(a, s) : dq_t<T, 32, PLAIN, 16>(a, s);
  }
  if (a.D == 256 && !pw) {
    constexpr bool kF16 = std::is_same<T, _Float16>::value;
    if constexpr (DKDV) return kF16 ? bwd_dkdv_d256_f16(a, s) : bwd_dkdv_d256_bf16(a, s);
    else return kF16 ? bwd_dq_d256_f16(a, s) : bwd_dq_d256_bf16(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

// The kernels of this file are compiled in parts, so that the build can run
// them in parallel: FA_BWD_PART selects which launcher (pass x dtype) this
// translation unit instantiates; 0 holds Delta and the dispatch, and an
// undefined FA_BWD_PART builds everything in one unit.
#ifndef FA_BWD_PART
#define FA_BWD_ALL 1
#define FA_BWD_PART 0
#else
#define FA_BWD_ALL 0
#endif

#if FA_BWD_ALL || FA_BWD_PART == 1
hipError_t bwd_dkdv_f16(const BwdArgs& a, hipStream_t s) { return dispatch<_Float16, true>(a, s); }
#endif
#if FA_BWD_ALL || FA_BWD_PART == 2
hipError_t bwd_dkdv_bf16(const BwdArgs& a, hipStream_t s) { return dispatch<__bf16, true>(a, s); }
#endif
#if FA_BWD_ALL || FA_BWD_PART == 3
hipError_t bwd_dq_f16(const BwdArgs& a, hipStream_t s) { return dispatch<_Float16, false>(a, s); }
#endif
#if FA_BWD_ALL || FA_BWD_PART == 4
hipError_t bwd_dq_bf16(const BwdArgs& a, hipStream_t s) { return dispatch<__bf16, false>(a, s); }
#endif
#if FA_BWD_ALL || FA_BWD_PART == 5
hipError_t bwd_dkdv_d256_f16(const BwdArgs& a, hipStream_t s) { return dkdv_t<_Float16, 256, PLAIN>(a, s); }
#endif
#if FA_BWD_ALL || FA_BWD_PART == 6
hipError_t bwd_dkdv_d256_bf16(const BwdArgs& a, hipStream_t s) { return dkdv_t<__bf16, 256, PLAIN>(a, s); }
#endif
#if FA_BWD_ALL || FA_BWD_PART == 7
hipError_t bwd_dq_d256_f16(const BwdArgs& a, hipStream_t s) { return dq_t<_Float16, 256, PLAIN>(a, s); }
#endif
#if FA_BWD_ALL || FA_BWD_PART == 8
hipError_t bwd_dq_d256_bf16(const BwdArgs& a, hipStream_t s) { return dq_t<__bf16, 256, PLAIN>(a, s); }
#endif

#if FA_BWD_PART == 0
hipError_t bwd_dkdv_f16(const BwdArgs& a, hipStream_t s);
hipError_t bwd_dkdv_bf16(const BwdArgs& a, hipStream_t s);
hipError_t bwd_dq_f16(const BwdArgs& a, hipStream_t s);
hipError_t bwd_dq_bf16(const BwdArgs& a, hipStream_t s);

hipError_t launch_attn_delta(int dtype, const void* o, const void* dout, const float* dlse, float* delta,
                             int64_t rows, int D, hipStream_t s) {
  if (dtype == 0) return launch_delta_t<float>(o, dout, dlse, delta, rows, D, s);
  if (dtype == 1) return launch_delta_t<_Float16>(o, dout, dlse, delta, rows, D, s);
  if (dtype == 2) return launch_delta_t<__bf16>(o, dout, dlse, delta, rows, D, s);
  return hipErrorInvalidValue;
}

hipError_t launch_attn_dkdv(const BwdArgs& a, hipStream_t s) {
  if (a.dtype == 1) return bwd_dkdv_f16(a, s);
  if (a.dtype == 2) return bwd_dkdv_bf16(a, s);
  return hipErrorInvalidValue;
}

hipError_t launch_attn_dq(const BwdArgs& a, hipStream_t s) {
  if (a.dtype == 1) return bwd_dq_f16(a, s);
  if (a.dtype == 2) return bwd_dq_bf16(a, s);
  return hipErrorInvalidValue;
}
#endif

}  // namespace fa
