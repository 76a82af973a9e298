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
// How it maps to CDNA4: 8 waves per workgroup (4 for the JVP variant at
// D = 128, for causal JVP at D = 64, and for D = 32 and 256), 32 query rows
// per wave, K/V blocks of 64 keys (32 for the D = 256 JVP, which splits the
// output columns over two workgroups) streamed through a three-stage LDS
// ring (two blocks prefetched) filled by direct global -> LDS loads (no
// staging registers).  Head dim 16 runs the D = 32 kernels over rows
// zero-padded to 32 columns (template parameter G = 16).  Scores are formed
// transposed, S^t = K Q^t, so that each lane owns one query row: row max and
// row sum are in-lane reductions plus one exchange with the other half-wave,
// and the rescale of the output accumulator is lane-local because that
// accumulator is also kept transposed (O^t = V^t P^t).  K is read with
// 16-byte row reads, V^t with transposing LDS reads of the same row-major
// tile layout, and the scores feed the second product without leaving
// registers (swap23 row order).
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace fa {

// The 16-bit D = 256 fused JVP, in translation units of their own (they
// compile separately from the other kernels of each dtype).
hipError_t fwd_jvp_d256_f16(const FwdArgs& a, hipStream_t s);
hipError_t fwd_jvp_d256_bf16(const FwdArgs& a, hipStream_t s);

namespace {

template <int V>
using ic = std::integral_constant<int, V>;

constexpr int kBN = 64;           // keys per K/V block
constexpr float kRescaleSlack = 8.0f;  // log2 units: P may reach 2^8 before a rescale

// The slack a variant may use.  The fp16 JVP packs P * Sdot into fp16 (max
// 65504): with P up to 2^8 a tangent score above 256 would overflow, so that
// variant rescales at every new maximum (P <= 1).
template <typename T, int VAR>
constexpr float rescale_slack() {
  return (VAR == JVP && std::is_same<T, _Float16>::value) ? 0.0f : kRescaleSlack;
}
constexpr int kLdsBytes = 160 * 1024;

// Launch shape per variant.  Variants whose per-lane state fits in 256
// registers run 8 waves (256 query rows) per workgroup, i.e. two waves per
// SIMD sharing each K/V block; the others (JVP with D = 128) run 4 waves.
// Causal JVP at D = 64 runs 4 waves over a two-stage ring (64 KiB), so that
// two workgroups share a CU: twice as many, shorter query blocks balance
// the causal triangle's uneven work better (12% faster at 1024, 4% slower
// than 8 waves without the mask).  Each wave owns 32 query rows.
//
// JVP at D = 256: the output and tangent accumulators of all 256 columns
// (256 registers) next to Q and the tangent Q (128) do not fit one wave's
// 512, so the output columns are split over two workgroups (SPLIT), each
// forming the full scores and accumulating 128 columns of O and its tangent
// (one wave per SIMD, AGPRs holding what the VGPRs cannot); its blocks are
// 32 keys (K and tK of 32 x 256, V and tV of 32 x 128: 48 KiB per ring
// stage).
template <int VAR, int D, bool CAUSAL>
struct FwdShape {
  static constexpr bool kSmall = VAR == JVP && D == 64 && CAUSAL;
  static constexpr int WAVES = (D == 32 || D == 256 || (VAR == JVP && D == 128) || kSmall) ? 4 : 8;
  static constexpr int NT = 64 * WAVES;
  static constexpr int BM = 32 * WAVES;
  static constexpr int BN = (VAR == JVP && D == 256) ? 32 : kBN;  // keys per K/V block
  static constexpr int SPLIT = (VAR == JVP && D == 256) ? 2 : 1;  // workgroups per query block
  static constexpr int DV = D / SPLIT;                            // output columns per workgroup
};

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
  float* tlse;     // may be NULL
  int BH, M, N, nmb;
  int fold;        // causal: row blocks 0 .. fold-1 of the grid run the longest
                   // query blocks, longest first; the rest the shortest first
  float scale2;    // sm_scale * log2(e)
  float sm_scale;
  int w;
};

template <typename T, int D, int VAR, bool CAUSAL>
struct alignas(16) FwdStage {
  using Sh = FwdShape<VAR, D, CAUSAL>;
  using Tile = DTile<T, Sh::BN, D, Sh::WAVES>;
  using VTile = DTile<T, Sh::BN, Sh::DV, Sh::WAVES, true, D>;  // this workgroup's V columns
  static constexpr int NK = (VAR == PLAIN) ? 1 : 2;  // K (+ tK or K2)
  static constexpr int NV = (VAR == JVP) ? 2 : 1;    // V (+ tV)
  T k[NK][Tile::ELEMS];
  T v[NV][VTile::ELEMS];
};

// K/V stages in the LDS ring: three (prefetch two blocks ahead) when they fit
// in the CU's LDS, else two (and two for the shape that shares a CU).
template <typename T, int D, int VAR, bool CAUSAL>
constexpr int fwd_stages() {
  if (FwdShape<VAR, D, CAUSAL>::kSmall) return 2;
  return 3 * (int)sizeof(FwdStage<T, D, VAR, CAUSAL>) <= kLdsBytes ? 3 : 2;
}

template <int VAR, int D, bool CAUSAL>
constexpr int fwd_waves_per_eu() {
  return FwdShape<VAR, D, CAUSAL>::kSmall ? 2 : FwdShape<VAR, D, CAUSAL>::WAVES / 4;
}

// RAGGED: M or N is not a multiple of 64 (the tail handling is compiled only
// into these instantiations, so the common case runs none of it).  G: the
// row length of the tensors (normally D; head dim 16 runs the D = 32 tiles
// with G = 16, the upper 16 columns zero in every operand and not stored).
template <typename T, int D, int VAR, bool CAUSAL, bool RAGGED, int G = D>
__global__ __launch_bounds__((FwdShape<VAR, D, CAUSAL>::NT))
__attribute__((amdgpu_waves_per_eu(fwd_waves_per_eu<VAR, D, CAUSAL>(), fwd_waves_per_eu<VAR, D, CAUSAL>())))
void attn_fwd_kernel(const FwdParams p) {
  constexpr int BN = FwdShape<VAR, D, CAUSAL>::BN;
  constexpr int SPLIT = FwdShape<VAR, D, CAUSAL>::SPLIT;
  constexpr int DV = FwdShape<VAR, D, CAUSAL>::DV;
  constexpr int kWaves = FwdShape<VAR, D, CAUSAL>::WAVES;
  constexpr int kBM = FwdShape<VAR, D, CAUSAL>::BM;
  constexpr int NS = fwd_stages<T, D, VAR, CAUSAL>();
  using V8 = typename Vec8<T>::type;
  using St = FwdStage<T, D, VAR, CAUSAL>;
  constexpr int KK = D / 16;     // 16-wide k steps over the head dim
  constexpr int DT = DV / 32;    // 32-wide tiles of this workgroup's output columns
  constexpr int ST = BN / 32;   // 32-key score tiles per block
  constexpr int PT = BN / 16;   // 16-key operand slices per block
  constexpr bool kJvp = VAR == JVP;
  constexpr bool kPw = VAR == PW;

  __shared__ St smem[NS];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int li = lane & 31, h = lane >> 5;

  // Workgroup -> (head, query block).  Heads vary fastest so every query
  // block of one head lands on the same XCD (the dispatcher deals workgroups
  // round-robin over the 8 XCDs and BH is a multiple of 8 in practice), which
  // keeps that head's K/V in one L2.  Causal: longest query blocks first;
  // when the whole grid is resident at once (two workgroups per CU), the
  // second half runs the shortest first, so that the workgroup dispatched
  // beside the longest one on a CU is the shortest.
  // (SPLIT > 1: the workgroups of one query block are adjacent; half is
  // the share of the output columns this one accumulates)
  const int half = SPLIT > 1 ? (int)(blockIdx.x % SPLIT) : 0;
  const int wg = SPLIT > 1 ? (int)(blockIdx.x / SPLIT) : (int)blockIdx.x;
  const int bh = wg % p.BH;
  int mb = wg / p.BH;
  if (CAUSAL) mb = mb < p.fold ? p.nmb - 1 - mb : mb - p.fold;
  const int m0 = mb * kBM;
  const int row0 = m0 + 32 * wave;
  const bool wave_valid = row0 < p.M;
  const int qi = row0 + li;
  const int pshift = p.N - p.M;
  const int64_t qbase = (int64_t)bh * p.M * G;
  const int64_t kbase = (int64_t)bh * p.N * G;

  // Direct loads of this head's K/V (and tK/tV or K2): uniform block base
  // pointer plus in-tile lane offsets computed once.
  const T* gk = (const T*)p.k + kbase;
  const T* gv = (const T*)p.v + kbase + half * DV;
  const T* gk2 = kPw ? (const T*)p.k2 + kbase : kJvp ? (const T*)p.tk + kbase : gk;
  const T* gv2 = kJvp ? (const T*)p.tv + kbase + half * DV : gv;
  static_assert(SPLIT == 1 || G == D, "split output columns of full rows");
  using DmaK = DmaTile<T, BN, D, kWaves, true, G>;
  using DmaV = DmaTile<T, BN, DV, kWaves, true, G>;
  DmaK dma;
  dma.lane_offsets(wave, lane);
  DmaV dmav;
  if constexpr (SPLIT > 1) dmav.lane_offsets(wave, lane);

  int n_end = p.N;
  const int wg_last_row = min(p.M, m0 + kBM) - 1;
  if (CAUSAL) n_end = min(p.N, wg_last_row + pshift + 1);
  const int nblk = n_end > 0 ? (n_end + BN - 1) / BN : 0;
  // Non-causal with a partial last key block: that block is visited first,
  // in a peeled iteration, so that the loop never needs the mask (causal:
  // the diagonal mask already hides every key past the last one).
  const bool tail_first = RAGGED && !CAUSAL && p.N % BN != 0;
  auto key_block = [&](int jb) { return tail_first ? (jb == 0 ? nblk - 1 : jb - 1) : jb; };

  // Query-side operands stay in registers for the whole pass.
  // (lanes past the last query row read that row; their results are not stored)
  V8 qf[KK], q2f[kPw ? KK : 1], tqf[kJvp ? KK : 1];
  const int qr = RAGGED ? min(qi, p.M - 1) : qi;
  // chunk 2 kk + h of a row (G < D: zero past the row's G columns)
  auto qchunk = [&](const T* row, int kk) -> V8 {
    if (G >= D || 16 * kk + 8 * h < G) return *reinterpret_cast<const V8*>(row + 16 * kk);
    return V8{};
  };
  if (wave_valid) {
    const T* qrow = (const T*)p.q + qbase + (int64_t)qr * G + 8 * h;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) qf[kk] = qchunk(qrow, kk);
    if constexpr (kPw) {
      const T* q2row = (const T*)p.q2 + qbase + (int64_t)qr * G + 8 * h;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) q2f[kk] = qchunk(q2row, kk);
    }
    if constexpr (kJvp) {
      const T* tqrow = (const T*)p.tq + qbase + (int64_t)qr * G + 8 * h;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) tqf[kk] = qchunk(tqrow, kk);
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
  float m_i = kNegInf;  // running max (possibly stale, see block()), log2 units
  float l_i = 0.f;      // running sum, this half-wave's keys
  float mu_i = 0.f;     // JVP: running sum of P * Sdot, this half-wave's keys

  // Loop-invariant LDS byte offsets inside a tile.  K row reads: row li,
  // chunk 2 kk + h (the 32-row sub-tile adds a constant).  V^t transposing
  // reads: (d-tile dt, half s) for key group 0 (key groups add constants).
  uint32_t kofs[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) kofs[kk] = (uint32_t)((li * D + (((2 * kk + h) ^ swz<D>(li)) * 8)) * 2);
  const TrLane tl(lane);
  uint32_t vofs[DT][2];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const int m = swap23(8 * tl.hh + 4 * s2 + tl.r);
      const int d = 32 * dt + tl.dcol;
      vofs[dt][s2] = (uint32_t)((m * DV + (((d >> 3) ^ swz<DV>(m)) * 8) + (d & 7)) * 2);
    }
  }

  // Piecewise: which score pairs a block needs, for a row range.
  auto pw_class = [&](int r_lo, int r_hi, int n0, bool& all_near, bool& all_far) {
    const int dmax = r_hi + pshift - n0;
    const int dmin = r_lo + pshift - (n0 + BN - 1);
    all_near = (dmax <= p.w) && (dmin >= -p.w);
    all_far = (p.w < 0) || (dmin > p.w) || (dmax < -p.w);
  };

  // Issue the direct loads of K/V block jb into stage st (completion:
  // vmcnt); returns the number of load instructions this wave issued.
  constexpr int kTileLoads = DmaK::PER_WAVE;
  constexpr int kVLoads = DmaV::PER_WAVE;
  auto tload = [&](const T* g, T* lds, int nr) {
    if constexpr (RAGGED)
      dma.load_rows(g, lds, wave, lane, nr);
    else
      dma.load(g, lds, wave);
  };
  auto vload = [&](const T* g, T* lds, int nr) {
    if constexpr (SPLIT == 1)
      tload(g, lds, nr);
    else if constexpr (RAGGED)
      dmav.load_rows(g, lds, wave, lane, nr);
    else
      dmav.load(g, lds, wave);
  };
  auto issue = [&](St& st, int jb) -> int {
    const int kb = key_block(jb);
    const int64_t off = (int64_t)kb * BN * G;
    const int nr = p.N - kb * BN;  // rows of this block that exist
    int n = kVLoads * St::NV;
    if constexpr (kPw) {
      bool an, af;
      pw_class(m0, wg_last_row, kb * BN, an, af);
      if (!af) {
        tload(gk + off, st.k[0], nr);
        n += kTileLoads;
      }
      if (!an) {
        tload(gk2 + off, st.k[1], nr);
        n += kTileLoads;
      }
    } else {
      tload(gk + off, st.k[0], nr);
      if constexpr (kJvp) tload(gk2 + off, st.k[1], nr);
      n += kTileLoads * St::NK;
    }
    vload(gv + off, st.v[0], nr);
    if constexpr (kJvp) vload(gv2 + off, st.v[1], nr);
    return n;
  };
  // Wait until every load but the newest n (one block's) has landed; loads
  // complete in issue order.  A piecewise block may skip one K tile.
  auto wait_all_but = [&](int n) {
    if constexpr (kPw)
      wait_vmcnt_any<3 * kTileLoads, 2 * kTileLoads>(n);
    else
      wait_vmcnt<kTileLoads * St::NK + kVLoads * St::NV>();
  };

  // Prologue: blocks 0 .. NS-2 are issued right behind the query operands;
  // block 0 (and the query operands) have landed after the wait.
  int n_new = 0;
#pragma unroll
  for (int j = 0; j < NS - 1; ++j)
    if (j < nblk) n_new = issue(smem[j], j);
  if (NS == 3 && nblk > 1)
    wait_all_but(n_new);
  else
    wait_vmcnt0();
  lds_barrier();

  auto krow8 = [&](const T* tile, int st, int kk) -> V8 {
    return *reinterpret_cast<const V8*>(reinterpret_cast<const char*>(tile) + kofs[kk] + st * 32 * D * 2);
  };

  // One K/V block for this wave.  Scores are raw Q.K in the loop; the scale
  // (sm_scale * log2 e) is folded into the exponent's FMA.  The running max
  // m_i is in log2 units and is only raised when a row's block max exceeds
  // it by more than kRescaleSlack: otherwise P = exp2(s - m_i) <= 2^slack is
  // accumulated against the stale max, which leaves O = acc / l and
  // LSE = m_i + log2 l exact and skips the rescale of the accumulators.
  auto block = [&](const St& cur, int n0, auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    f32x16 s[ST];
    f32x16 sd[kJvp ? ST : 1];
    // ---- scores S^t = K Q^t (and tangents) ------------------------------
    if constexpr (kPw) {
      bool an, af;
      pw_class(row0, row0 + 31, n0, an, af);
#pragma unroll
      for (int st = 0; st < ST; ++st) {
        f32x16 s1 = zero16(), s2 = zero16();
        if (!af) {
#pragma unroll
          for (int kk = 0; kk < KK; ++kk) s1 = mfma32x32x16(krow8(cur.k[0], st, kk), qf[kk], s1);
        }
        if (!an) {
#pragma unroll
          for (int kk = 0; kk < KK; ++kk) s2 = mfma32x32x16(krow8(cur.k[1], st, kk), q2f[kk], s2);
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
    } else if constexpr (!kJvp && ST * KK <= 16) {
      // All ST * KK row reads of the K tile are put in flight first; product
      // i then waits only for read i.  Reads and products alternate between
      // the ST score tiles (independent accumulation chains).
      static_assert(ST * KK <= 16, "row reads in flight");
      RowReads<ST * KK> kr;
      const uint32_t kb = lds_addr(cur.k[0]);
      static_for<ST * KK>([&](auto ic) {
        constexpr int I = decltype(ic)::value;
        kr.template issue<I, (I % ST) * 32 * D * 2>(kb + kofs[I / ST]);
      });
#pragma unroll
      for (int st = 0; st < ST; ++st) s[st] = zero16();
      static_for<ST * KK>([&](auto ic) {
        constexpr int I = decltype(ic)::value;
        kr.template wait<I>();
        s[I % ST] = mfma32x32x16(kr.template get<V8>(I), qf[I / ST], s[I % ST]);
        __builtin_amdgcn_sched_barrier(0);
      });
    } else if constexpr (!kJvp) {
      // wide heads: one row read per product
#pragma unroll
      for (int st = 0; st < ST; ++st) {
        s[st] = zero16();
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) s[st] = mfma32x32x16(krow8(cur.k[0], st, kk), qf[kk], s[st]);
      }
    } else if constexpr (SPLIT == 1) {
#pragma unroll
      for (int st = 0; st < ST; ++st) {
        s[st] = zero16();
        sd[st] = zero16();
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          const V8 a = krow8(cur.k[0], st, kk);
          s[st] = mfma32x32x16(a, qf[kk], s[st]);
          sd[st] = mfma32x32x16(a, tqf[kk], sd[st]);
        }
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) sd[st] = mfma32x32x16(krow8(cur.k[1], st, kk), qf[kk], sd[st]);
      }
    } else {
      // (one 32-key tile) the K rows, then the tK rows, read in a rolling
      // window of four: row i + 4 is read right after the products of row
      // i, so that few reads hold registers (Q and the tangent Q take 128)
      static_assert(ST == 1, "one score tile");
      constexpr int kW = 4;
      auto kread = [&](auto i_c) -> V8 {
        constexpr int I = decltype(i_c)::value;
        return krow8(cur.k[I / KK], 0, I % KK);
      };
      V8 kr[kW];
      static_for<kW>([&](auto ic) { kr[decltype(ic)::value] = kread(ic); });
      s[0] = zero16();
      sd[0] = zero16();
      static_for<2 * KK>([&](auto ic) {
        constexpr int I = decltype(ic)::value, kk = I % KK;
        const V8 a = kr[I % kW];
        if constexpr (I < KK) {
          s[0] = mfma32x32x16(a, qf[kk], s[0]);
          sd[0] = mfma32x32x16(a, tqf[kk], sd[0]);
        } else {
          sd[0] = mfma32x32x16(a, qf[kk], sd[0]);
        }
        if constexpr (I + kW < 2 * KK) kr[I % kW] = kread(std::integral_constant<int, I + kW>{});
        __builtin_amdgcn_sched_barrier(0);
      });
    }
    // ---- online softmax ---------------------------------------------------
    if constexpr (MASK) {
#pragma unroll
      for (int st = 0; st < ST; ++st) {
        // key n0 + 32 st + perm_row(r, h) is beyond this query (causal) or
        // beyond the last key
        const int thr = (CAUSAL ? (RAGGED ? min(qi + pshift, p.N - 1) : qi + pshift) : p.N - 1) - n0 - 32 * st - 8 * h;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          if (perm_row(r, 0) > thr) s[st][r] = kNegInf;
        }
      }
    }
    // row max over this lane's 16 * ST scores: four independent chains
    float mx[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) mx[c] = kNegInf;
#pragma unroll
    for (int st = 0; st < ST; ++st) {
#pragma unroll
      for (int r = 0; r < 16; ++r) mx[(r >> 1) & 3] = fmaxf(mx[(r >> 1) & 3], s[st][r]);
    }
    const float mloc = halves_max(fmaxf(fmaxf(mx[0], mx[1]), fmaxf(mx[2], mx[3]))) * p.scale2;
    if (__ballot(mloc > m_i + rescale_slack<T, VAR>()) != 0) {
      const float m_new = fmaxf(m_i, mloc);
      const float alpha = (m_new == kNegInf) ? 1.f : exp2_fast(m_i - m_new);  // m_i = -inf -> 0
      l_i *= alpha;
      if constexpr (kJvp) mu_i *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[dt][r] *= alpha;
        if constexpr (kJvp) {
#pragma unroll
          for (int r = 0; r < 16; ++r) accg[dt][r] *= alpha;
        }
      }
      m_i = m_new;
    }
    const float neg_m = (m_i == kNegInf) ? 0.f : -m_i;
    float mus[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < ST; ++st) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pv = exp2_fast(fmaf(s[st][r], p.scale2, neg_m));
        s[st][r] = pv;
        if constexpr (kJvp) {
          const float ps = pv * sd[st][r] * p.sm_scale;
          sd[st][r] = ps;
          mus[r & 3] += ps;
        }
      }
    }
    if constexpr (kJvp) mu_i += (mus[0] + mus[1]) + (mus[2] + mus[3]);
    // ---- O^t += V^t P^t (and the tangent accumulator) ----------------------
    // The row sum is taken over P as rounded for the product (pair dot
    // products with 1), so O = acc / l is normalised with the same weights.
    V8 pb[PT];
    V8 psb[kJvp ? PT : 1];
    float ls = 0.f;
#pragma unroll
    for (int t = 0; t < PT; ++t) {
      pb[t] = pack8<T>(s[t >> 1], 8 * (t & 1));
      ls = add_sum8(ls, pb[t]);
      if constexpr (kJvp) psb[t] = pack8<T>(sd[t >> 1], 8 * (t & 1));
    }
    l_i += ls;
    // V^t operands come from transposing LDS reads issued as inline asm
    // (see TrOps): the reads of d-tile dt + 1 are in flight while the
    // products of d-tile dt run.
    const uint32_t vbase = lds_addr(cur.v[0]);
    const uint32_t vbase2 = kJvp ? lds_addr(cur.v[kJvp ? 1 : 0]) : 0u;
    TrOps<T, PT> va, vb;
    TrOps<T, kJvp ? PT : 1> ta, tb;
    va.template issue_at<DV>(vbase, vofs[0]);
    if constexpr (kJvp) ta.template issue_at<DV>(vbase2, vofs[0]);
    va.wait();
    if constexpr (kJvp) ta.wait();
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      TrOps<T, PT>& cv = (dt & 1) ? vb : va;
      TrOps<T, PT>& nv = (dt & 1) ? va : vb;
      TrOps<T, kJvp ? PT : 1>& ct = (dt & 1) ? tb : ta;
      TrOps<T, kJvp ? PT : 1>& nt = (dt & 1) ? ta : tb;
      if (dt + 1 < DT) {
        nv.template issue_at<DV>(vbase, vofs[dt + 1]);
        if constexpr (kJvp) nt.template issue_at<DV>(vbase2, vofs[dt + 1]);
      }
#pragma unroll
      for (int t = 0; t < PT; ++t) {
        acc[dt] = mfma32x32x16(cv.op[t], pb[t], acc[dt]);
        if constexpr (kJvp) accg[dt] = mfma32x32x16(cv.op[t], psb[t], accg[dt]);
      }
      if constexpr (kJvp) {
#pragma unroll
        for (int t = 0; t < PT; ++t) accg[dt] = mfma32x32x16(ct.op[t], pb[t], accg[dt]);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (dt + 1 < DT) {
        nv.wait();
        if constexpr (kJvp) nt.wait();
      }
    }
  };

  // Block jb is computed from stage jb % NS while block jb + NS - 1 is being
  // loaded into the stage freed by block jb - 1.  Before the barrier each
  // wave waits until its loads of block jb + 1 have landed, leaving those of
  // the newest block in flight (loads complete in issue order).
  int cur_stage = 0;
  auto iteration = [&](int jb, auto tail_tag) {
    const int ahead = jb + NS - 1;
    int ld_stage = cur_stage + NS - 1;
    if (ld_stage >= NS) ld_stage -= NS;
    const bool issued = ahead < nblk;
    if (issued) n_new = issue(smem[ld_stage], ahead);
    const int n0 = key_block(jb) * BN;
    const bool active = wave_valid && (!CAUSAL || n0 <= row0 + 31 + pshift);
    if (active) {
      if (decltype(tail_tag)::value || (CAUSAL && (n0 + BN - 1 > row0 + pshift)))
        block(smem[cur_stage], n0, std::true_type{});
      else
        block(smem[cur_stage], n0, std::false_type{});
    }
    if (NS == 3 && issued)
      wait_all_but(n_new);
    else
      wait_vmcnt0();
    lds_barrier();
    cur_stage = (cur_stage + 1 == NS) ? 0 : cur_stage + 1;
  };
  int jb0 = 0;
  if constexpr (RAGGED) {
    if (tail_first && nblk > 0) {
      iteration(0, std::true_type{});
      jb0 = 1;
    }
  }
  for (int jb = jb0; jb < nblk; ++jb) iteration(jb, std::false_type{});

  // ---- epilogue: O = acc / l, LSE = (m + log2 l) ln 2 ----------------------
  // Waves whose rows lie beyond M (last query block of a head) store nothing.
  // The ring is free after the last barrier: each wave stages its output
  // tiles through its own part of it and stores whole rows.
  if (!wave_valid) return;
  const float l = halves_sum(l_i);
  const bool has = l > 0.f;
  const float inv = has ? 1.f / l : 0.f;
  static_assert(kWaves * RowStage<DV>::kStageBytes <= (int)sizeof(smem), "output staging fits in the ring");
  char* stage = reinterpret_cast<char*>(&smem[0]) + wave * RowStage<DV>::kStageBytes;
  const int nrows = RAGGED ? p.M - row0 : 32;
  const int64_t orow = qbase + (int64_t)row0 * G + half * DV;
  store_tile_rows<T, DV, G>((T*)p.o + orow, nrows, acc, inv, stage, lane);
  float c = 0.f;
  if constexpr (kJvp) {
    const float mu = halves_sum(mu_i);
    c = mu * inv;  // mu / l
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) accg[dt][r] = accg[dt][r] - c * acc[dt][r];
    }
    store_tile_rows<T, DV, G>((T*)p.to + orow, nrows, accg, inv, stage, lane);
  }
  if (RAGGED && qi >= p.M) return;  // lanes past the last query row
  if (half != 0) return;            // (every share forms the same row statistics)
  if (h == 0) p.lse[(int64_t)bh * p.M + qi] = has ? (m_i + log2f(l)) * kLn2 : kNegInf;
  // LSE tangent: sum_j P_ij Sdot_ij (0 for a row with no visible key)
  if (kJvp && h == 0 && p.tlse) p.tlse[(int64_t)bh * p.M + qi] = c;
}

// ---------------------------------------------------------------------------
// Software-pipelined forward, plain variant.
//
// Iteration j works on two K/V blocks.  The 16 (D = 128) or 8 (D = 64) score
// products of block j + 1 are issued one at a time, each followed by the
// exponent work of a few scores of block j, so the matrix core and the vector
// ALU of a SIMD work side by side; then the products P_j V_j are issued, each
// followed by a step of block j + 1's row max.  The K tile of block j + 1 is
// needed one iteration earlier than in the single-block loop, so the LDS ring
// has four stages: block j (V read), j + 1 (K read), j + 2 (landed) and j + 3
// (loading).  The loop is unrolled by the four stages so every LDS address is
// a per-lane register plus an immediate.
//
// Piecewise variant (D = 64): each stage also holds a K2 tile; a block is
// loaded with the K tiles its workgroup needs, and a wave forms the scores
// of a block wholly on one side of the distance rule from that side's
// operands, or, on a block that straddles it, takes the (q1, k1) scores and
// replaces the far pairs by (q2, k2) scores formed after them.
// ---------------------------------------------------------------------------
constexpr int kPipeNS = 4;
constexpr int kPipeWaves = 8;

// Transposing LDS read as inline asm, completed by an explicit lgkmcnt wait
// tied to its result (the compiler would otherwise wait for the direct loads
// of the ring that are still in flight).
template <int IMM>
__device__ __forceinline__ void tr_read_imm(std::integral_constant<int, IMM>, uint32_t a, u32x2& r) {
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(a), "i"(IMM));
}
template <int N>
__device__ __forceinline__ void lgkm_wait_pair(std::integral_constant<int, N>, u32x2& r0, u32x2& r1) {
  asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(r0), "+v"(r1) : "n"(N));
}

template <typename T, int D, int VAR>
struct alignas(256) PipeSmem {
  using Tile = DTile<T, kBN, D, kPipeWaves>;
  static constexpr int NK = (VAR == PW) ? 2 : 1;
  T k[NK][kPipeNS][Tile::ELEMS];  // K (piecewise: K1, then K2)
  T v[kPipeNS][Tile::ELEMS];
};

template <typename T, int D, int VAR, bool CAUSAL, bool RAGGED>
__global__ __launch_bounds__(64 * kPipeWaves) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_pipe_kernel(const FwdParams p) {
  constexpr int kWaves = kPipeWaves;
  constexpr int kBM = 32 * kWaves;
  constexpr int NS = kPipeNS;
  constexpr bool kPw = VAR == PW;
  using V8 = typename Vec8<T>::type;
  using Sm = PipeSmem<T, D, VAR>;
  using Tile = typename Sm::Tile;
  using Dma = DmaTile<T, kBN, D, kWaves>;
  constexpr int KK = D / 16;
  constexpr int DT = D / 32;
  constexpr int ST = kBN / 32;
  constexpr int PT = kBN / 16;
  constexpr int NR = ST * KK;        // K row reads (= score products) per block
  constexpr int NSC = 16 * ST;       // scores per lane per block
  constexpr int EPM = NSC / NR;      // scores whose exponent follows each product
  constexpr int NPV = DT * PT;       // P V products per block
  constexpr int MPP = NSC / NPV;     // scores folded into the max per P V product
  constexpr int kTileBytes = Tile::ELEMS * 2;
  static_assert(sizeof(Sm) <= kLdsBytes, "LDS budget");
  static_assert(NSC % NR == 0 && NSC % NPV == 0 && MPP % 2 == 0, "interleave shape");
  constexpr int kK2Bytes = NS * kTileBytes;  // K2 tiles follow the K tiles
  static_assert((kPw ? kK2Bytes : 0) + (NS - 1) * kTileBytes + (ST - 1) * 32 * D * 2 <= 65535,
                "K read immediates");
  static_assert((NS - 1) * kTileBytes + (PT - 1) * 16 * D * 2 <= 65535, "V read immediates");

  __shared__ Sm smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = wave_id();
  const int li = lane & 31, h = lane >> 5;

  // Workgroup -> (head, query block): heads vary fastest (one head's K/V in
  // one XCD's L2); causal: longest query blocks first.
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
  const T* gk = (const T*)p.k + kbase;
  const T* gv = (const T*)p.v + kbase;
  Dma dma;
  dma.lane_offsets(wave, lane);

  int n_end = p.N;
  const int wg_last_row = min(p.M, m0 + kBM) - 1;
  if (CAUSAL) n_end = min(p.N, wg_last_row + pshift + 1);
  const int nblk = n_end > 0 ? (n_end + kBN - 1) / kBN : 0;
  // A partial last key block.  Non-causal: it is visited first (its mask is
  // applied in the prologue, never in the loop).  Causal: its tile is the
  // 64 keys ending at key N - 1 (all of them exist, so the loads need no
  // per-lane tail code); the keys it shares with the block before are masked
  // from below, and the diagonal mask hides every key past the last one.
  const bool tail_first = RAGGED && !CAUSAL && p.N % kBN != 0;
  auto key_block = [&](int jb) { return tail_first ? (jb == 0 ? nblk - 1 : jb - 1) : jb; };
  auto tile_start = [&](int kb) {
    return (RAGGED && CAUSAL && kb * kBN + kBN > p.N && p.N >= kBN) ? p.N - kBN : kb * kBN;
  };

  // (lanes past the last query row read that row; their results are not stored)
  V8 qf[KK], q2f[kPw ? KK : 1];
  if (wave_valid) {
    const int64_t qoff = qbase + (int64_t)(RAGGED ? min(qi, p.M - 1) : qi) * D + 8 * h;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) qf[kk] = *reinterpret_cast<const V8*>((const T*)p.q + qoff + 16 * kk);
    if constexpr (kPw) {
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) q2f[kk] = *reinterpret_cast<const V8*>((const T*)p.q2 + qoff + 16 * kk);
    }
  }
  const T* gk2 = kPw ? (const T*)p.k2 + kbase : gk;

  f32x16 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = zero16();
  float m_i = kNegInf;  // running max, log2 units (raised lazily, see kRescaleSlack)
  float l_i = 0.f;      // running sum, this half-wave's keys

  // Per-lane LDS addresses.  K row reads: row li, chunk 2 kk + h of a K tile
  // (stage and 32-row sub-tile are immediates).  V^t transposing reads of
  // d-tile dt, halves 0 and 1, key group 0 of a V tile.
  const uint32_t lbase = lds_addr(&smem);
  uint32_t kaddr[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk)
    kaddr[kk] = lbase + (uint32_t)((li * D + (((2 * kk + h) ^ swz<D>(li)) * 8)) * 2);
  const TrLane tl(lane);
  uint32_t vaddr[DT][2];
  const uint32_t vb = lbase + (uint32_t)__builtin_offsetof(Sm, v);
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const int m = swap23(8 * tl.hh + 4 * s2 + tl.r);
      const int d = 32 * dt + tl.dcol;
      vaddr[dt][s2] = vb + (uint32_t)((m * D + (((d >> 3) ^ swz<D>(m)) * 8) + (d & 7)) * 2);
    }
  }

  // Piecewise: is every pair of rows [r_lo, r_hi] x keys [t0, t0 + 63] near
  // (|dist| <= w), or every pair far?
  auto pw_class = [&](int r_lo, int r_hi, int t0, bool& all_near, bool& all_far) {
    const int dmax = r_hi + pshift - t0;
    const int dmin = r_lo + pshift - (t0 + kBN - 1);
    all_near = (dmax <= p.w) && (dmin >= -p.w);
    all_far = (p.w < 0) || (dmin > p.w) || (dmax < -p.w);
  };

  // Issue the direct loads of block jb; returns this wave's number of load
  // instructions.  (CHK: the tile may lack rows: only in the prologue, since
  // in the loop every tile lies inside the keys)
  auto issue = [&](int jb, auto chk) -> int {
    const int st = jb % NS;
    const int kb = key_block(jb);
    const int t0 = tile_start(kb);
    const int64_t off = (int64_t)t0 * D;
    bool need_k = true, need_k2 = false;
    if constexpr (kPw) {
      bool an, af;
      pw_class(m0, wg_last_row, t0, an, af);
      need_k = !af;
      need_k2 = !an;
    }
    if constexpr (RAGGED && decltype(chk)::value) {
      const int nr = p.N - t0;  // rows of this tile that exist
      if (need_k) dma.load_rows(gk + off, smem.k[0][st], wave, lane, nr);
      if (kPw && need_k2) dma.load_rows(gk2 + off, smem.k[kPw ? 1 : 0][st], wave, lane, nr);
      dma.load_rows(gv + off, smem.v[st], wave, lane, nr);
    } else {
      if (need_k) dma.load(gk + off, smem.k[0][st], wave);
      if (kPw && need_k2) dma.load(gk2 + off, smem.k[kPw ? 1 : 0][st], wave);
      dma.load(gv + off, smem.v[st], wave);
    }
    return Dma::PER_WAVE * (1 + (int)need_k + (int)(kPw && need_k2));
  };
  // Wait until every load but the newest n (one block's) has landed; loads
  // complete in issue order.  A piecewise block may skip one K tile.
  auto wait_all_but = [&](int n) {
    if constexpr (kPw)
      wait_vmcnt_any<3 * Dma::PER_WAVE, 2 * Dma::PER_WAVE>(n);
    else
      wait_vmcnt<2 * Dma::PER_WAVE>();
  };
  auto active = [&](int jb) { return wave_valid && (!CAUSAL || jb * kBN <= row0 + 31 + pshift); };
  auto needs_mask = [&](int jb) { return CAUSAL && (jb * kBN + kBN - 1 > row0 + pshift); };

  // K row read i of stage S (i = kk * ST + st) from tile set KS (0: K,
  // 1: K2), as inline asm.
  auto kread = [&](auto stage_c, auto i_c, u32x4& r, auto set_c) {
    constexpr int S = decltype(stage_c)::value;
    constexpr int I = decltype(i_c)::value;
    constexpr int KS = decltype(set_c)::value;
    const uint32_t a = kaddr[I / ST];
    asm volatile("ds_read_b128 %0, %1 offset:%2"
                 : "=v"(r)
                 : "v"(a), "i"(KS * kK2Bytes + S * kTileBytes + (I % ST) * 32 * D * 2));
  };
  // Wait for K read i.  Reads are kept kWin deep: 0 .. kWin-1 are issued
  // first and read i + kWin right after product i (reads complete in issue
  // order).
  constexpr int kWin = 4;
  auto kwait = [&](auto i_c, u32x4& r) {
    constexpr int I = decltype(i_c)::value;
    constexpr int CNT = (NR - 1 - I < kWin - 1) ? (NR - 1 - I) : (kWin - 1);
    asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(r) : "n"(CNT));
  };

  // Score products of tile set KS (query operands qs) of the block in
  // stage S into sn; after product i, run between(i) (exponent work of the
  // previous block, or nothing).
  auto scores_set = [&](auto stage_c, auto set_c, const V8 (&qs)[KK], f32x16 (&sn)[ST], auto&& between) {
    u32x4 kr[NR];
    static_for<kWin>([&](auto ic) { kread(stage_c, ic, kr[decltype(ic)::value], set_c); });
#pragma unroll
    for (int st = 0; st < ST; ++st) sn[st] = zero16();
    static_for<NR>([&](auto ic) {
      constexpr int I = decltype(ic)::value;
      kwait(ic, kr[I]);
      sn[I % ST] = mfma32x32x16(__builtin_bit_cast(V8, kr[I]), qs[I / ST], sn[I % ST]);
      if constexpr (I + kWin < NR) kread(stage_c, std::integral_constant<int, I + kWin>{}, kr[I + kWin], set_c);
      between(ic);
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  // Scores of block jb (in stage S) into sn.  Piecewise: from the side of
  // the rule the wave's pairs lie on; a straddling block takes the (q1, k1)
  // scores, then forms the (q2, k2) ones one 32-key tile at a time and
  // replaces the far pairs (key t0 + 32 st + perm_row(r, h) is at distance
  // c1 - perm_row(r, 0) from this lane's query).
  auto scores = [&](auto stage_c, int jb, f32x16 (&sn)[ST], auto&& between) {
    if constexpr (!kPw) {
      scores_set(stage_c, ic<0>{}, qf, sn, between);
    } else {
      const int t0 = tile_start(key_block(jb));
      bool an, af;
      pw_class(row0, row0 + 31, t0, an, af);
      if (af) {
        scores_set(stage_c, ic<1>{}, q2f, sn, between);
      } else {
        scores_set(stage_c, ic<0>{}, qf, sn, between);
        if (!an) {
          static_for<ST>([&](auto stc) {
            constexpr int st = decltype(stc)::value;
            u32x4 kr[KK];
            static_for<KK>([&](auto kc) {
              kread(stage_c, ic<decltype(kc)::value * ST + st>{}, kr[decltype(kc)::value], ic<1>{});
            });
            f32x16 s2 = zero16();
            static_for<KK>([&](auto kc) {
              constexpr int kk = decltype(kc)::value;
              asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(kr[kk]) : "n"(KK - 1 - kk));
              s2 = mfma32x32x16(__builtin_bit_cast(V8, kr[kk]), q2f[kk], s2);
            });
            const int c1 = qi + pshift - t0 - 32 * st - 8 * h;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int dist = c1 - perm_row(r, 0);
              if (!(dist <= p.w && dist >= -p.w)) sn[st][r] = s2[r];
            }
          });
        }
      }
    }
  };

  // Mask of the raw scores of key block kb (tile from key t0): keys beyond
  // this query (causal) or beyond the last key (non-causal), and keys of the
  // block before (a causal tail tile starts before kb * kBN) -> -inf.
  auto apply_mask = [&](f32x16 (&sc)[ST], int kb) {
    const int t0 = tile_start(kb);
#pragma unroll
    for (int st = 0; st < ST; ++st) {
      const int thr = (CAUSAL ? qi + pshift : p.N - 1) - t0 - 32 * st - 8 * h;
      const int lo = kb * kBN - t0 - 32 * st - 8 * h;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (perm_row(r, 0) > thr || (RAGGED && CAUSAL && perm_row(r, 0) < lo)) sc[st][r] = kNegInf;
    }
  };

  // Exponent work on scores [I*EPM, (I+1)*EPM) of sc against neg_m.
  auto exp_step = [&](f32x16 (&sc)[ST], float neg_m, auto i_c) {
    constexpr int I = decltype(i_c)::value;
#pragma unroll
    for (int u = 0; u < EPM; ++u) {
      const int e = I * EPM + u;
      sc[e / 16][e % 16] = exp2_fast(fmaf(sc[e / 16][e % 16], p.scale2, neg_m));
    }
  };
  // Lazy rescale after the row max mloc (log2 units) of the next block.
  auto rescale = [&](float mloc) {
    if (__ballot(mloc > m_i + kRescaleSlack) != 0) {
      const float m_new = fmaxf(m_i, mloc);
      const float alpha = (m_new == kNegInf) ? 1.f : exp2_fast(m_i - m_new);
      l_i *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[dt][r] *= alpha;
      }
      m_i = m_new;
    }
  };
  // O^t += V^t P^t for the V tile of stage S; after product i, between(i).
  // (V^t operands in a rolling window of kVWin: operand i + kVWin is read
  // right after product i; each operand is two transposing reads, which
  // complete in issue order)
  constexpr int kVWin = 3;
  auto pv = [&](auto stage_c, const V8 (&pb)[PT], auto&& between) {
    constexpr int S = decltype(stage_c)::value;
    constexpr int IMM = S * kTileBytes;
    // product I: key slice TI = I / DT (P operand), d-tile DTI = I % DT, so
    // consecutive products feed different accumulators and slice t's P is
    // first needed by product t * DT
    u32x2 vr[NPV][2];
    auto vread = [&](auto i_c) {
      constexpr int I = decltype(i_c)::value, DTI = I % DT, TI = I / DT;
      tr_read_imm(std::integral_constant<int, IMM + TI * 16 * D * 2>{}, vaddr[DTI][0], vr[I][0]);
      tr_read_imm(std::integral_constant<int, IMM + TI * 16 * D * 2>{}, vaddr[DTI][1], vr[I][1]);
    };
    static_for<kVWin>([&](auto ic) { vread(ic); });
    static_for<NPV>([&](auto ic) {
      constexpr int I = decltype(ic)::value, DTI = I % DT, TI = I / DT;
      constexpr int AFTER = (NPV - 1 - I < kVWin - 1) ? (NPV - 1 - I) : (kVWin - 1);
      lgkm_wait_pair(std::integral_constant<int, 2 * AFTER>{}, vr[I][0], vr[I][1]);
      u32x4 w;
      w[0] = vr[I][0][0];
      w[1] = vr[I][0][1];
      w[2] = vr[I][1][0];
      w[3] = vr[I][1][1];
      acc[DTI] = mfma32x32x16(__builtin_bit_cast(V8, w), pb[TI], acc[DTI]);
      if constexpr (I + kVWin < NPV) vread(std::integral_constant<int, I + kVWin>{});
      between(ic);
      __builtin_amdgcn_sched_barrier(0);
    });
  };


  // Prologue: blocks 0, 1, 2 are issued right behind the query operands;
  // blocks 0 and 1 (and the query operands) have landed; the scores of
  // block 0 and its max are taken.
  int n_new = 0;  // load instructions of the newest block issued
#pragma unroll
  for (int j = 0; j < NS - 1; ++j)
    if (j < nblk) n_new = issue(j, std::true_type{});
  if (nblk > NS - 2)
    wait_all_but(n_new);
  else
    wait_vmcnt0();
  lds_barrier();

  f32x16 sa[ST], sb[ST];  // raw scores of the current / next block (ping-pong across stages)
#pragma unroll
  for (int st = 0; st < ST; ++st) {
    sa[st] = zero16();
    sb[st] = zero16();
  }
  if (nblk > 0 && active(0)) {
    scores(std::integral_constant<int, 0>{}, 0, sa, [](auto) {});
    if (tail_first || needs_mask(0)) apply_mask(sa, key_block(0));
    float mx = kNegInf;
#pragma unroll
    for (int st = 0; st < ST; ++st)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sa[st][r]);
    rescale(halves_max(mx) * p.scale2);
  }

  // One iteration: block jb's V tile in stage S, block jb + 1's K tile in
  // stage S + 1.  sc holds block jb's raw scores, sn receives block jb + 1's.
  auto step = [&](auto stage_c, int jb, f32x16 (&sc)[ST], f32x16 (&sn)[ST]) {
    constexpr int S = decltype(stage_c)::value;
    constexpr int SN = (S + 1) % NS;
    if (jb + NS - 1 < nblk) n_new = issue(jb + NS - 1, std::false_type{});
    const bool a_c = active(jb);
    const bool a_n = jb + 1 < nblk && active(jb + 1);
    const float neg_m = (m_i == kNegInf) ? 0.f : -m_i;
    if (a_c) {
      // scores of block jb + 1 || exponents of block jb
      if (a_n)
        scores(std::integral_constant<int, SN>{}, jb + 1, sn, [&](auto ic) { exp_step(sc, neg_m, ic); });
      else
        static_for<NR>([&](auto ic) { exp_step(sc, neg_m, ic); });
      // P of block jb packed into the operands of P V: slice 0 now, slice
      // t + 1 after product t; the row sum over the packed P after products
      // PT - 1 .. 2 PT - 2 (same order as a sum right after packing)
      V8 pb[PT];
      pb[0] = pack8<T>(sc[0], 0);
      if (a_n && needs_mask(jb + 1)) apply_mask(sn, jb + 1);
      // P V of block jb || row max of block jb + 1 (taken whether or not
      // that block is active; only used when it is)
      float mx[2] = {kNegInf, kNegInf};
      float ls = 0.f;
      pv(stage_c, pb, [&](auto ic) {
        constexpr int I = decltype(ic)::value;
        if constexpr (I + 1 < PT) pb[I + 1] = pack8<T>(sc[(I + 1) >> 1], 8 * ((I + 1) & 1));
        if constexpr (I >= PT - 1 && I < 2 * PT - 1) ls = add_sum8(ls, pb[I - (PT - 1)]);
        if constexpr (I == 2 * PT - 2) l_i += ls;
#pragma unroll
        for (int u = 0; u < MPP; u += 2) {
          const int e = I * MPP + u;
          mx[u / 2 % 2] = fmaxf(fmaxf(mx[u / 2 % 2], sn[e / 16][e % 16]), sn[(e + 1) / 16][(e + 1) % 16]);
        }
      });
      if (a_n) rescale(halves_max(fmaxf(mx[0], mx[1])) * p.scale2);
    }
    if (jb + NS - 1 < nblk)
      wait_all_but(n_new);
    else
      wait_vmcnt0();
    lds_barrier();
  };
  for (int jb = 0; jb < nblk; jb += NS) {
    step(std::integral_constant<int, 0>{}, jb, sa, sb);
    if (jb + 1 < nblk) step(std::integral_constant<int, 1>{}, jb + 1, sb, sa);
    if (jb + 2 < nblk) step(std::integral_constant<int, 2>{}, jb + 2, sa, sb);
    if (jb + 3 < nblk) step(std::integral_constant<int, 3>{}, jb + 3, sb, sa);
  }

  // Epilogue: O = acc / l, LSE = (m + log2 l) ln 2.  The ring is free after
  // the last barrier: each wave stages its O tile through its own part of it
  // and stores whole rows.
  if (!wave_valid) return;
  const float l = halves_sum(l_i);
  const bool has = l > 0.f;
  const float inv = has ? 1.f / l : 0.f;
  static_assert(kWaves * RowStage<D>::kStageBytes <= (int)sizeof(Sm), "O staging fits in the ring");
  store_tile_rows<T, D>((T*)p.o + qbase + (int64_t)row0 * D, RAGGED ? p.M - row0 : 32, acc, inv,
                        reinterpret_cast<char*>(&smem) + wave * RowStage<D>::kStageBytes, lane);
  if (RAGGED && qi >= p.M) return;  // lanes past the last query row
  if (h == 0) p.lse[(int64_t)bh * p.M + qi] = has ? (m_i + log2f(l)) * kLn2 : kNegInf;
}

template <typename T, int D, int VAR, int G = D>
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
  p.tlse = a.tlse;
  p.BH = a.B * a.H;
  p.M = a.M;
  p.N = a.N;
  const int bm = a.causal ? FwdShape<VAR, D, true>::BM : FwdShape<VAR, D, false>::BM;
  p.nmb = (a.M + bm - 1) / bm;
  p.fold = p.nmb;
  if constexpr (FwdShape<VAR, D, true>::kSmall) {
    // two workgroups per CU: one round when the grid fits twice the CUs
    int dev = 0, cus = 0;
    if (a.causal && hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cus > 0 &&
        (int64_t)p.nmb * p.BH <= 2 * (int64_t)cus)
      p.fold = p.nmb / 2;
  }
  p.scale2 = a.sm_scale * kLog2e;
  p.sm_scale = a.sm_scale;
  p.w = a.w;
  static_assert(FwdShape<VAR, D, true>::SPLIT == FwdShape<VAR, D, false>::SPLIT, "one split per variant");
  dim3 grid(p.nmb * p.BH * FwdShape<VAR, D, true>::SPLIT),
      block(a.causal ? FwdShape<VAR, D, true>::NT : FwdShape<VAR, D, false>::NT);
  const bool ragged = a.M % 64 != 0 || a.N % 64 != 0;
  if constexpr (G == D && ((VAR == PLAIN && (D == 64 || D == 128)) || (VAR == PW && D == 64))) {
    static_assert(FwdShape<VAR, D, true>::NT == 64 * kPipeWaves && FwdShape<VAR, D, false>::NT == 64 * kPipeWaves,
                  "same launch shape");
    if (a.causal && ragged)
      hipLaunchKernelGGL((attn_fwd_pipe_kernel<T, D, VAR, true, true>), grid, block, 0, s, p);
    else if (a.causal)
      hipLaunchKernelGGL((attn_fwd_pipe_kernel<T, D, VAR, true, false>), grid, block, 0, s, p);
    else if (ragged)
      hipLaunchKernelGGL((attn_fwd_pipe_kernel<T, D, VAR, false, true>), grid, block, 0, s, p);
    else
      hipLaunchKernelGGL((attn_fwd_pipe_kernel<T, D, VAR, false, false>), grid, block, 0, s, p);
  } else {
    if (a.causal && ragged)
      hipLaunchKernelGGL((attn_fwd_kernel<T, D, VAR, true, true, G>), grid, block, 0, s, p);
    else if (a.causal)
      hipLaunchKernelGGL((attn_fwd_kernel<T, D, VAR, true, false, G>), grid, block, 0, s, p);
    else if (ragged)
      hipLaunchKernelGGL((attn_fwd_kernel<T, D, VAR, false, true, G>), grid, block, 0, s, p);
    else
      hipLaunchKernelGGL((attn_fwd_kernel<T, D, VAR, false, false, G>), grid, block, 0, s, p);
  }
  return hipGetLastError();
}

template <typename T, int D, int G = D>
hipError_t launch_var(const FwdArgs& a, hipStream_t s) {
  switch (a.variant) {
    case PLAIN: return launch_t<T, D, PLAIN, G>(a, s);
    case JVP: return launch_t<T, D, JVP, G>(a, s);
    case PW: return launch_t<T, D, PW, G>(a, s);
  }
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t launch_d(const FwdArgs& a, hipStream_t s) {
  if (a.D == 64) return launch_var<T, 64>(a, s);
  if (a.D == 128) return launch_var<T, 128>(a, s);
  if (a.D == 32) return launch_var<T, 32>(a, s);
  // D = 16: the D = 32 kernels over zero-padded tiles (a 16-wide row is one
  // 32-byte piece, below the 16 x 32 operand of the products)
  if (a.D == 16) return launch_var<T, 32, 16>(a, s);
  // D = 256: plain attention here, the JVP in its own translation units
  // (piecewise runs on the generic kernels)
  if (a.D == 256 && a.variant == PLAIN) return launch_t<T, 256, PLAIN>(a, s);
  if (a.D == 256 && a.variant == JVP)
    return std::is_same<T, _Float16>::value ? fwd_jvp_d256_f16(a, s) : fwd_jvp_d256_bf16(a, s);
  return hipErrorInvalidValue;
}

}  // namespace

// Compiled in parts (one per dtype) so that the build runs them in
// parallel; FA_FWD_PART 0 holds the dispatch, an undefined FA_FWD_PART
// builds everything in one unit.
#ifndef FA_FWD_PART
#define FA_FWD_ALL 1
#define FA_FWD_PART 0
#else
#define FA_FWD_ALL 0
#endif

#if FA_FWD_ALL || FA_FWD_PART == 1
hipError_t fwd_f16(const FwdArgs& a, hipStream_t s) { return launch_d<_Float16>(a, s); }
#endif
#if FA_FWD_ALL || FA_FWD_PART == 2
hipError_t fwd_bf16(const FwdArgs& a, hipStream_t s) { return launch_d<__bf16>(a, s); }
#endif
#if FA_FWD_ALL || FA_FWD_PART == 3
hipError_t fwd_jvp_d256_f16(const FwdArgs& a, hipStream_t s) { return launch_t<_Float16, 256, JVP>(a, s); }
#endif
#if FA_FWD_ALL || FA_FWD_PART == 4
hipError_t fwd_jvp_d256_bf16(const FwdArgs& a, hipStream_t s) { return launch_t<__bf16, 256, JVP>(a, s); }
#endif

#if FA_FWD_PART == 0
hipError_t fwd_f16(const FwdArgs& a, hipStream_t s);
hipError_t fwd_bf16(const FwdArgs& a, hipStream_t s);

hipError_t launch_attn_fwd(const FwdArgs& a, hipStream_t s) {
  if (a.dtype == 1) return fwd_f16(a, s);
  if (a.dtype == 2) return fwd_bf16(a, s);
  return hipErrorInvalidValue;
}
#endif

}  // namespace fa
