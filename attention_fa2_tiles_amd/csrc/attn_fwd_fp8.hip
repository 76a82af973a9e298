// Attention forward with FP8 (e5m2) inputs on gfx950 MFMA.
//
// What is computed: the forward of the Triton fused-attention tutorial with
// its FP8 path (_attn_fwd with q, k, v in float8 e5m2 and v supplied
// transposed), i.e. O = softmax(sm_scale Q K^T) V and the natural-log LSE,
// causal or not, with the online softmax of the 16-bit kernels.  Both
// products run on v_mfma_scale_f32_32x32x64_f8f6f4 (unit scales), the
// gfx950 instruction that gives FP8 twice the bf16 matrix rate: S^t = K Q^t
// with e5m2 operands, and O^t = V^t P^t with V^t in e5m2 and P rounded to
// e4m3 (one more mantissa bit than the tutorial's e5m2 P; P <= 2^8 under the
// lazy rescale, inside e4m3's range).  The softmax runs in fp32; O and the
// LSE are normalised by the sum of the unrounded P (summing the rounded
// ones would cost a decode per score).  The weights' rounding moves each
// p by at most 2^-4 p where p >= 2^-6 (e4m3 normal range) and by at most
// 2^-10 in absolute terms below it (subnormal spacing 2^-9, values under
// 2^-10 flush to 0); divided by the row sum, which is at least the sum
// taken against the row's true maximum, that bounds the error of O.  O is
// written in fp16 or bf16.
//
// CDNA4 mapping: 4 waves x 32 query rows, 64-key blocks through a 3-stage
// LDS ring filled by direct global -> LDS loads.  The f8f6f4 product takes
// 32 bytes of k per lane; the byte -> k assignment inside an instruction
// only has to agree between A and B, so lane half h simply feeds bytes
// [32h, 32h + 32) of each 64-byte k step of both operands.  The K tile's LDS
// rows are permuted (key = bits h, st, r of the LDS row, see key_of_row) so
// that the 32 scores a lane receives from the two 32-key score tiles are
// keys 32h .. 32h + 31 in order: they pack straight into the lane's B
// operand of the P V product, whose A operand (V^t, keys contiguous) is then
// two plain 16-byte row reads of the transposed V tile.  The scores stay in
// registers, as in the 16-bit kernels.
#include "common.h"
#include "kernels.h"

namespace fa {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));

constexpr int kF8BN = 64;     // keys per block
constexpr int kF8Waves = 4;   // waves per workgroup, 32 query rows each (three workgroups per CU)
constexpr int kF8BM = 32 * kF8Waves;
constexpr int kF8NS = 3;      // ring stages
constexpr int kFmtE4M3 = 0, kFmtE5M2 = 1;  // f8f6f4 operand format codes

struct Fp8Params {
  const uint8_t* q;   // [BH, M, D] e5m2
  const uint8_t* k;   // [BH, N, D] e5m2
  const uint8_t* vt;  // [BH, D, N] e5m2 (V transposed)
  void* o;            // [BH, M, D] fp16 / bf16
  float* lse;         // [BH, M]
  int BH, M, N, nmb;
  float scale2;       // sm_scale * log2(e)
};

// LDS row m of a K tile holds key key_of_row(m): with m = 32 st + 8 a + 4 h
// + b (a = r / 4, b = r % 4 of the accumulator register r that receives it),
// key = 32 h + 16 st + 4 a + b.
__device__ __forceinline__ constexpr int key_of_row(int m) {
  return (((m >> 2) & 1) << 5) | (((m >> 5) & 1) << 4) | (((m >> 3) & 3) << 2) | (m & 3);
}

// 16-byte chunk swizzle for rows of C chunks (C = 8: 128-byte rows, two per
// 256-byte bank window; C = 4: 64-byte rows, four per window): 16 lanes
// reading one chunk of 16 consecutive rows hit 16 distinct bank slots.
template <int C>
__device__ __forceinline__ int swz8(int m) {
  static_assert(C == 4 || C == 8, "chunks per row");
  return (m / (16 / C)) % C;
}

template <int D>
struct alignas(256) Fp8Stage {
  uint8_t k[kF8BN * D];   // K tile, rows permuted (key_of_row)
  uint8_t vt[D * kF8BN];  // V^t tile: row d holds keys n0 .. n0 + 63
};

// 32 x 32 x 64 product, A in format FA and B in format FB, unit block scales
// (127 is 2^0 in the e8m0 scale encoding).
template <int FA, int FB>
__device__ __forceinline__ f32x16 mfma_f8(const i32x8& a, const i32x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FA, FB, 0, 127, 0, 127);
}

__device__ __forceinline__ i32x8 read32(const uint8_t* lds_row, int c0, int c1) {
  const u32x4v x = *reinterpret_cast<const u32x4v*>(lds_row + 16 * c0);
  const u32x4v y = *reinterpret_cast<const u32x4v*>(lds_row + 16 * c1);
  i32x8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r[i] = (int)x[i];
    r[4 + i] = (int)y[i];
  }
  return r;
}

template <typename TO, int D, bool CAUSAL, bool RAGGED>
__global__ __launch_bounds__(64 * kF8Waves) void attn_fwd_fp8_kernel(const Fp8Params p) {
  constexpr int KS = D / 64;          // 64-wide k steps over the head dim
  constexpr int DT = D / 32;          // 32-wide tiles of the output's head dim
  constexpr int KC = D / 16;          // 16-byte chunks per K row
  constexpr int VC = kF8BN / 16;      // 16-byte chunks per V^t row (4)
  constexpr int KI = kF8BN * KC / 64; // load instructions of a K tile
  constexpr int VI = D * VC / 64;     // load instructions of a V^t tile
  constexpr int LPW = (KI + VI) / kF8Waves;
  static_assert((KI + VI) % kF8Waves == 0, "tile loads split over the waves");
  using St = Fp8Stage<D>;
  static_assert(kF8NS * sizeof(St) <= 160 * 1024, "LDS budget");
  __shared__ St smem[kF8NS];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int li = lane & 31, h = lane >> 5;
  const int bh = blockIdx.x % p.BH;
  int mb = blockIdx.x / p.BH;
  if (CAUSAL) mb = p.nmb - 1 - mb;
  const int m0 = mb * kF8BM;
  const int row0 = m0 + 32 * wave;
  const bool wave_valid = row0 < p.M;
  const int qi = row0 + li;
  const int pshift = p.N - p.M;

  const uint8_t* gk = p.k + (int64_t)bh * p.N * D;
  const uint8_t* gvt = p.vt + (int64_t)bh * D * p.N;

  int n_end = p.N;
  const int wg_last_row = min(p.M, m0 + kF8BM) - 1;
  if (CAUSAL) n_end = min(p.N, wg_last_row + pshift + 1);
  const int nblk = n_end > 0 ? (n_end + kF8BN - 1) / kF8BN : 0;
  const bool tail_first = RAGGED && !CAUSAL && p.N % kF8BN != 0;
  auto key_block = [&](int jb) { return tail_first ? (jb == 0 ? nblk - 1 : jb - 1) : jb; };

  // Q operand (B of the score product): lane (query li, half h) holds bytes
  // [64 ks + 32 h, + 32) of its row.
  i32x8 qf[KS];
  const int qr = RAGGED ? min(qi, p.M - 1) : qi;
  if (wave_valid) {
    const uint8_t* qrow = p.q + ((int64_t)bh * p.M + qr) * D + 32 * h;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = *reinterpret_cast<const i32x8*>(qrow + 64 * ks);
  }

  f32x16 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = zero16();
  float m_i = kNegInf;  // running max, log2 units (possibly stale)
  float l_x = 0.f;      // running sum of the unrounded P

  // Direct loads of block jb into stage st: instruction j of this wave
  // covers 64 chunks of the K tile (first KI instructions) or of the V^t
  // tile.  Rows past the last key read zeros.
  auto issue = [&](St& st, int jb) {
    const int n0 = key_block(jb) * kF8BN;
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
      const int ins = wave * LPW + j;
      const uint8_t* src;
      uint8_t* dst;
      if (ins < KI) {
        const int pch = ins * 64 + lane;
        const int m = pch / KC, slot = pch % KC;
        const int key = n0 + key_of_row(m);
        src = (!RAGGED || key < p.N) ? gk + (int64_t)key * D + 16 * (slot ^ swz8<KC>(m))
                                     : reinterpret_cast<const uint8_t*>(kZero16);
        dst = st.k + ins * 1024;
      } else {
        const int pch = (ins - KI) * 64 + lane;
        const int d = pch / VC, slot = pch % VC;
        const int key = n0 + 16 * (slot ^ swz8<VC>(d));  // first of the chunk's 16 keys
        src = (!RAGGED || key < p.N) ? gvt + (int64_t)d * p.N + key : reinterpret_cast<const uint8_t*>(kZero16);
        dst = st.vt + (ins - KI) * 1024;
      }
      __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)src,
                                       (void __attribute__((address_space(3)))*)dst, 16, 0, 0);
    }
  };

  wait_vmcnt0();
#pragma unroll
  for (int j = 0; j < kF8NS - 1; ++j)
    if (j < nblk) issue(smem[j], j);
  if (nblk > 1)
    wait_vmcnt<LPW>();
  else
    wait_vmcnt0();
  lds_barrier();

  auto block = [&](const St& cur, int n0, auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    // ---- scores S^t = K Q^t: two 32-key tiles ---------------------------
    f32x16 s[2];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      s[st] = zero16();
      const int m = 32 * st + li;
      const uint8_t* krow = cur.k + m * D;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int c0 = 4 * ks + 2 * h;
        const i32x8 a = read32(krow, c0 ^ swz8<KC>(m), (c0 + 1) ^ swz8<KC>(m));
        s[st] = mfma_f8<kFmtE5M2, kFmtE5M2>(a, qf[ks], s[st]);
      }
    }
    // register r of tile st holds key n0 + 32 h + 16 st + r
    if constexpr (MASK) {
      const int thr = (CAUSAL ? (RAGGED ? min(qi + pshift, p.N - 1) : qi + pshift) : p.N - 1) - n0 - 32 * h;
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (16 * st + r > thr) s[st][r] = kNegInf;
    }
    float mx = kNegInf;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[st][r]);
    const float mloc = halves_max(mx) * p.scale2;
    if (__ballot(mloc > m_i + 8.0f) != 0) {
      const float m_new = fmaxf(m_i, mloc);
      const float alpha = (m_new == kNegInf) ? 1.f : exp2_fast(m_i - m_new);
      l_x *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[dt][r] *= alpha;
      m_i = m_new;
    }
    const float neg_m = (m_i == kNegInf) ? 0.f : -m_i;
    // P = exp2(s scale2 - m), rounded to e4m3 and packed: byte j of the
    // operand is key 32 h + j.
    i32x8 pb;
    float sx = 0.f;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const int st = w >> 2, r0 = 4 * (w & 3);
      float e[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        e[i] = exp2_fast(fmaf(s[st][r0 + i], p.scale2, neg_m));
        sx += e[i];
      }
      int word = __builtin_amdgcn_cvt_pk_fp8_f32(e[0], e[1], 0, false);
      word = __builtin_amdgcn_cvt_pk_fp8_f32(e[2], e[3], word, true);
      pb[w] = word;
    }
    l_x += sx;
    // ---- O^t += V^t P^t ---------------------------------------------------
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int d = 32 * dt + li;
      const uint8_t* vrow = cur.vt + d * kF8BN;
      const i32x8 a = read32(vrow, (2 * h) ^ swz8<VC>(d), (2 * h + 1) ^ swz8<VC>(d));
      acc[dt] = mfma_f8<kFmtE5M2, kFmtE4M3>(a, pb, acc[dt]);
    }
  };

  int cur_stage = 0;
  auto iteration = [&](int jb, auto tail_tag) {
    const int ahead = jb + kF8NS - 1;
    int ld_stage = cur_stage + kF8NS - 1;
    if (ld_stage >= kF8NS) ld_stage -= kF8NS;
    const bool issued = ahead < nblk;
    if (issued) issue(smem[ld_stage], ahead);
    const int n0 = key_block(jb) * kF8BN;
    const bool active = wave_valid && (!CAUSAL || n0 <= row0 + 31 + pshift);
    if (active) {
      if (decltype(tail_tag)::value || (CAUSAL && (n0 + kF8BN - 1 > row0 + pshift)))
        block(smem[cur_stage], n0, std::true_type{});
      else
        block(smem[cur_stage], n0, std::false_type{});
    }
    if (issued)
      wait_vmcnt<LPW>();
    else
      wait_vmcnt0();
    lds_barrier();
    cur_stage = (cur_stage + 1 == kF8NS) ? 0 : cur_stage + 1;
  };
  int jb0 = 0;
  if constexpr (RAGGED) {
    if (tail_first && nblk > 0) {
      iteration(0, std::true_type{});
      jb0 = 1;
    }
  }
  for (int jb = jb0; jb < nblk; ++jb) iteration(jb, std::false_type{});

  if (!wave_valid) return;
  const float lx = halves_sum(l_x);
  const bool has = lx > 0.f;
  const float inv = has ? 1.f / lx : 0.f;
  if (RAGGED && qi >= p.M) return;
  TO* orow = (TO*)p.o + ((int64_t)bh * p.M + qi) * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) store_acc_t<TO>(orow, acc[dt], 32 * dt, h, inv);
  if (h == 0) p.lse[(int64_t)bh * p.M + qi] = has ? (m_i + log2f(lx)) * kLn2 : kNegInf;
}

template <typename TO, int D>
hipError_t launch_fp8_t(const Fp8Args& a, hipStream_t s) {
  Fp8Params p;
  p.q = (const uint8_t*)a.q;
  p.k = (const uint8_t*)a.k;
  p.vt = (const uint8_t*)a.vt;
  p.o = a.o;
  p.lse = a.lse;
  p.BH = a.B * a.H;
  p.M = a.M;
  p.N = a.N;
  p.nmb = (a.M + kF8BM - 1) / kF8BM;
  p.scale2 = a.sm_scale * kLog2e;
  dim3 grid(p.nmb * p.BH), block(64 * kF8Waves);
  const bool ragged = a.M % 64 != 0 || a.N % 64 != 0;
  if (a.causal && ragged)
    hipLaunchKernelGGL((attn_fwd_fp8_kernel<TO, D, true, true>), grid, block, 0, s, p);
  else if (a.causal)
    hipLaunchKernelGGL((attn_fwd_fp8_kernel<TO, D, true, false>), grid, block, 0, s, p);
  else if (ragged)
    hipLaunchKernelGGL((attn_fwd_fp8_kernel<TO, D, false, true>), grid, block, 0, s, p);
  else
    hipLaunchKernelGGL((attn_fwd_fp8_kernel<TO, D, false, false>), grid, block, 0, s, p);
  return hipGetLastError();
}

template <typename TO>
hipError_t launch_fp8_d(const Fp8Args& a, hipStream_t s) {
  if (a.D == 64) return launch_fp8_t<TO, 64>(a, s);
  if (a.D == 128) return launch_fp8_t<TO, 128>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_attn_fwd_fp8(const Fp8Args& a, hipStream_t s) {
  if (a.out_dtype == 1) return launch_fp8_d<_Float16>(a, s);
  if (a.out_dtype == 2) return launch_fp8_d<__bf16>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace fa
