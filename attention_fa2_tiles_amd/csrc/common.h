// Device-side building blocks shared by the gfx950 attention kernels.
//
// MFMA operand convention used throughout (v_mfma_f32_32x32x16_{bf16,f16}):
//   A is 32 x 16 (rows x k), B is 16 x 32 (k x cols), C/D is 32 x 32 fp32.
//   Lane l (li = l % 32, h = l / 32) supplies row li of A and column li of B,
//   each as 8 consecutive k values (k = 8h .. 8h+7).  It receives 16 results
//   of column li, rows 8*(r/4) + 4h + (r%4) for r = 0..15.
// A lane therefore always owns one column of the product.  The kernels
// choose which matrix goes in A so that the index they reduce over in the
// softmax lives in that lane's registers ("lane = query" in the forward and
// the dQ pass, "lane = key" in the dK/dV pass).
//
// Row-major tiles in LDS are stored with bits 2 and 3 of the row index
// swapped (swap23).  Then the 16 results a lane receives from a product whose
// A operand came from such a tile belong to A rows 16*(r/8) + 8h + (r%8):
// registers 0..7 cover 8 consecutive rows and 8..15 the next run.  That is
// exactly the k-slice the same lane must feed as B operand to the next
// product (contracting over those rows), so scores become operands without
// any cross-lane traffic.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

template <typename T> struct Vec8;
template <> struct Vec8<__bf16> { typedef bf16x8 type; };
template <> struct Vec8<_Float16> { typedef f16x8 type; };

// acc + (sum of the 8 elements of v), as four pair dot products with (1, 1)
// in fp32 (v_dot2c_f32_{bf16,f16}).
__device__ __forceinline__ float add_sum8(float acc, const bf16x8& v) {
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bf16x2 pr = {v[2 * i], v[2 * i + 1]};
    acc = __builtin_amdgcn_fdot2_f32_bf16(pr, one, acc, false);
  }
  return acc;
}
__device__ __forceinline__ float add_sum8(float acc, const f16x8& v) {
  const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f16x2 pr = {v[2 * i], v[2 * i + 1]};
    acc = __builtin_amdgcn_fdot2(pr, one, acc, false);
  }
  return acc;
}

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32x32x16(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// 8 fp32 values (registers base..base+7 of an accumulator) -> MFMA operand.
template <typename T>
__device__ __forceinline__ typename Vec8<T>::type pack8(const f32x16& v, int base) {
  typename Vec8<T>::type r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (T)v[base + e];
  return r;
}

// s_waitcnt vmcnt(N) with the LDS and export counters left alone (gfx9
// encoding: vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}
__device__ __forceinline__ void wait_vmcnt0() { wait_vmcnt<0>(); }

// Wait until at most n vector-memory operations of this wave are
// outstanding, where n (wave-uniform) is one of the listed counts.  List the
// counts in decreasing order: a value matching none of them waits for the
// last (smallest), which is always safe.
template <int A, int... Rest>
__device__ __forceinline__ void wait_vmcnt_any(int n) {
  if constexpr (sizeof...(Rest) == 0) {
    wait_vmcnt<A>();
  } else {
    if (n == A)
      wait_vmcnt<A>();
    else
      wait_vmcnt_any<Rest...>(n);
  }
}

// Workgroup barrier without the release/acquire fences of __syncthreads():
// those make the compiler wait for every outstanding load (including the
// direct LDS loads of stages still being prefetched) before the barrier.
// Callers make LDS data visible themselves (wait_vmcnt for direct loads,
// lgkmcnt for LDS stores); the empty asm statements keep the compiler from
// moving memory accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Index of this wavefront in the workgroup, as a value the compiler knows to
// be the same for every lane (branches on it become scalar branches rather
// than exec-masked regions).
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6); }

__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32, 64); }

__device__ __forceinline__ constexpr int swap23(int r) {
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

// Key/query offset (within a 32-row group) of accumulator register r held
// by lane half h, for products whose A operand came from a swap23 tile.
__device__ __forceinline__ constexpr int perm_row(int r, int h) {
  return 16 * (r >> 3) + 8 * h + (r & 7);
}

// Row offset (within a 32 x 32 output tile) of accumulator register r for
// lane half h, natural MFMA layout (A operand not permuted).
__device__ __forceinline__ constexpr int nat_row(int r, int h) {
  return 8 * (r >> 2) + 4 * h + (r & 3);
}

template <typename T>
__device__ __forceinline__ typename Vec8<T>::type lds_read8(const T* p) {
  return *reinterpret_cast<const typename Vec8<T>::type*>(p);
}

// ---------------------------------------------------------------------------
// Cooperative global -> register -> LDS staging of one R x C tile (row-major
// in global memory, row stride C elements, C*sizeof(T) a multiple of 16).
// ---------------------------------------------------------------------------

// Row-major destination, rows stored swap23-permuted, row pitch C + 8.
template <typename T, int R, int C, int NT>
struct RowTile {
  static constexpr int PITCH = C + 8;
  static constexpr int CHUNKS = R * C / 8;            // 16-byte chunks
  static constexpr int PER_THREAD = (CHUNKS + NT - 1) / NT;
  static constexpr int ELEMS = R * PITCH;
  u32x4 r[PER_THREAD];

  __device__ __forceinline__ void load(const T* g, int tid) {
#pragma unroll
    for (int i = 0; i < PER_THREAD; ++i) {
      int c = tid + i * NT;
      if (CHUNKS % NT == 0 || c < CHUNKS) {
        int row = c / (C / 8), col = (c % (C / 8)) * 8;
        r[i] = *reinterpret_cast<const u32x4*>(g + (int64_t)row * C + col);
      }
    }
  }
  __device__ __forceinline__ void store(T* s, int tid) const {
#pragma unroll
    for (int i = 0; i < PER_THREAD; ++i) {
      int c = tid + i * NT;
      if (CHUNKS % NT == 0 || c < CHUNKS) {
        int row = c / (C / 8), col = (c % (C / 8)) * 8;
        *reinterpret_cast<u32x4*>(s + swap23(row) * PITCH + col) = r[i];
      }
    }
  }
};

// Transposed destination: LDS holds T^t, i.e. C rows of R elements, pitch
// R + 8.  Each thread moves an RB x 8 block (RB rows of 8 columns).
template <typename T, int R, int C, int NT>
struct TransTile {
  static constexpr int PITCH = R + 8;
  static constexpr int RB = (R * C / 8 >= 4 * NT) ? 4 : 2;   // rows per block
  static constexpr int BLOCKS = (R / RB) * (C / 8);
  static constexpr int PER_THREAD = (BLOCKS + NT - 1) / NT;
  static constexpr int ELEMS = C * PITCH;
  u32x4 r[PER_THREAD][RB];

  __device__ __forceinline__ void load(const T* g, int tid) {
#pragma unroll
    for (int i = 0; i < PER_THREAD; ++i) {
      int b = tid + i * NT;
      if (BLOCKS % NT == 0 || b < BLOCKS) {
        int rg = b % (R / RB), cg = b / (R / RB);
#pragma unroll
        for (int j = 0; j < RB; ++j)
          r[i][j] = *reinterpret_cast<const u32x4*>(g + (int64_t)(rg * RB + j) * C + cg * 8);
      }
    }
  }
  __device__ __forceinline__ void store(T* s, int tid) const {
#pragma unroll
    for (int i = 0; i < PER_THREAD; ++i) {
      int b = tid + i * NT;
      if (BLOCKS % NT == 0 || b < BLOCKS) {
        int rg = b % (R / RB), cg = b / (R / RB);
        const uint16_t* src[RB];
#pragma unroll
        for (int j = 0; j < RB; ++j) src[j] = reinterpret_cast<const uint16_t*>(&r[i][j]);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          T* dst = s + (cg * 8 + e) * PITCH + rg * RB;
          if constexpr (RB == 4) {
            u32x2 w;
            w[0] = (uint32_t)src[0][e] | ((uint32_t)src[1][e] << 16);
            w[1] = (uint32_t)src[2][e] | ((uint32_t)src[3][e] << 16);
            *reinterpret_cast<u32x2*>(dst) = w;
          } else {
            uint32_t w = (uint32_t)src[0][e] | ((uint32_t)src[1][e] << 16);
            *reinterpret_cast<uint32_t*>(dst) = w;
          }
        }
      }
    }
  }
};

// ---------------------------------------------------------------------------
// LDS tiles filled by direct global -> LDS loads (gfx950 global_load_lds of
// 16 bytes: lane l's 16 bytes land at the instruction's LDS base + 16 * l).
//
// A tile holds R rows of D 2-byte elements, row-major with no padding.  LDS
// row m holds global row swap23(m) of the tile (global row m when PERM is
// false), and 16-byte chunk c of LDS row m sits at chunk slot c ^ swz<D>(m).  The XOR pattern makes both ways
// the kernels read a tile free of bank conflicts:
//  * row reads (ds_read_b128): 16 lanes read one chunk of 16 consecutive
//    rows -> 16 distinct 16-byte slots of the 256-byte bank window;
//  * transposing reads (ds_read_b64_tr_b16): 32 lanes read a 4-row x
//    4-chunk block -> 16 distinct slots.
// ---------------------------------------------------------------------------

template <int D>
__device__ __forceinline__ int swz(int m) {
  static_assert(D == 32 || D == 64 || D == 128 || D == 256, "head dim");
  if constexpr (D >= 128) return ((m & 3) << 2) | ((m >> 2) & 3);
  else if constexpr (D == 64) return (((m >> 1) & 1) << 2) | ((m >> 2) & 3);
  else return (m >> 2) & 3;
}

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ constexpr int tile_row(int m, bool perm) { return perm ? swap23(m) : m; }

// 16 zero bytes (source of the lanes of a direct tile load whose row lies
// past the end of the tensor) and a +inf (the LSE of such a row).
static __device__ __attribute__((aligned(16))) uint32_t kZero16[4] = {0u, 0u, 0u, 0u};
static __device__ float kPosInfF = __builtin_huge_valf();

// G: the row stride of the tensor the tile is loaded from, in elements.
// Normally G = D; G > D: a tile of D columns out of wider rows; G < D: rows
// of G elements zero-padded to the tile's D columns (chunks from column G on
// are loaded from kZero16).
template <typename T, int R, int D, int NW, bool PERM = true, int G = D>
struct DTile {
  static constexpr int CPR = D / 8;                 // 16-byte chunks per row
  static constexpr int ROWS_PER_INSTR = 64 / CPR;   // rows per wave instruction
  static constexpr int INSTR = R / ROWS_PER_INSTR;  // wave instructions per tile
  static constexpr int PER_WAVE = INSTR / NW;
  static constexpr int ELEMS = R * D;
  static constexpr int DATA_CHUNKS = (G < D ? G : D) / 8;  // chunks of a row that exist in memory
  static_assert(INSTR % NW == 0, "tile must split evenly over the waves");
  static_assert(G % 8 == 0, "rows of whole 16-byte chunks");

  // Issue this wave's share of the direct loads of the R x D tile at g
  // (row stride G elements) into lds.  Completion is tracked by vmcnt.
  __device__ static __forceinline__ void load(T* lds, const T* g, int wave, int lane) {
#pragma unroll
    for (int j = 0; j < PER_WAVE; ++j) {
      const int ins = wave * PER_WAVE + j;
      const int p = ins * 64 + lane;
      const int m = p / CPR, slot = p % CPR;
      const int c = slot ^ swz<D>(m);
      const T* src = (G >= D || c < DATA_CHUNKS) ? g + tile_row(m, PERM) * G + c * 8
                                                 : reinterpret_cast<const T*>(kZero16);
      __builtin_amdgcn_global_load_lds(
          (const void __attribute__((address_space(1)))*)src,
          (void __attribute__((address_space(3)))*)(lds + ins * 512), 16, 0, 0);
    }
  }

  // As load, for a tile of which only rows 0 .. nrows-1 exist in memory:
  // the rows beyond are filled with zeros (a lane whose source row lies
  // beyond reads 16 zero bytes of kZero16 instead).  Same instruction count
  // as load.
  __device__ static __forceinline__ void load_lim(T* lds, const T* g, int wave, int lane, int nrows) {
#pragma unroll
    for (int j = 0; j < PER_WAVE; ++j) {
      const int ins = wave * PER_WAVE + j;
      const int p = ins * 64 + lane;
      const int m = p / CPR, slot = p % CPR;
      const int src = tile_row(m, PERM);
      const int c = slot ^ swz<D>(m);
      const T* src_ptr = (src < nrows && (G >= D || c < DATA_CHUNKS)) ? g + src * G + c * 8
                                                                      : reinterpret_cast<const T*>(kZero16);
      __builtin_amdgcn_global_load_lds(
          (const void __attribute__((address_space(1)))*)src_ptr,
          (void __attribute__((address_space(3)))*)(lds + ins * 512), 16, 0, 0);
    }
  }

  // 8 consecutive elements (chunk c) of LDS row m: one ds_read_b128.
  __device__ static __forceinline__ typename Vec8<T>::type row8(const T* lds, int m, int c) {
    return *reinterpret_cast<const typename Vec8<T>::type*>(lds + m * D + ((c ^ swz<D>(m)) * 8));
  }
};

// Direct loads of an R x D tile with loop-invariant per-lane byte offsets
// inside the tile (computed once by lane_offsets): a tile is issued from a
// uniform base pointer plus those 32-bit offsets, which the compiler can
// encode with a scalar base register, so issuing costs no vector arithmetic.
template <typename T, int R, int D, int NW, bool PERM = true, int G = D>
struct DmaTile {
  using Tile = DTile<T, R, D, NW, PERM, G>;
  static constexpr int PER_WAVE = Tile::PER_WAVE;
  uint32_t voff[PER_WAVE];
  uint32_t live = ~0u;  // G < D: bit j set when this lane's chunk of load j exists in memory

  __device__ __forceinline__ void lane_offsets(int wave, int lane) {
#pragma unroll
    for (int j = 0; j < PER_WAVE; ++j) {
      const int ins = wave * PER_WAVE + j;
      const int p = ins * 64 + lane;
      const int m = p / Tile::CPR, slot = p % Tile::CPR;
      const int c = slot ^ swz<D>(m);
      voff[j] = (uint32_t)((tile_row(m, PERM) * G + c * 8) * 2);
      if constexpr (G < D) {
        if (c >= Tile::DATA_CHUNKS) live &= ~(1u << j);
      }
    }
  }
  // Load the tile whose first row is at g (row stride G) into lds (G < D:
  // the padding chunks from kZero16).
  __device__ __forceinline__ void load(const T* g, T* lds, int wave) const {
#pragma unroll
    for (int j = 0; j < PER_WAVE; ++j) {
      const int ins = wave * PER_WAVE + j;
      const char* src = reinterpret_cast<const char*>(g) + voff[j];
      if constexpr (G < D) src = ((live >> j) & 1u) ? src : reinterpret_cast<const char*>(kZero16);
      __builtin_amdgcn_global_load_lds(
          (const void __attribute__((address_space(1)))*)src,
          (void __attribute__((address_space(3)))*)(lds + ins * 512), 16, 0, 0);
    }
  }
  // As load, when only rows 0 .. nrows-1 of the tile exist (see
  // DTile::load_lim); nrows >= R is the same as load.
  __device__ __forceinline__ void load_rows(const T* g, T* lds, int wave, int lane, int nrows) const {
    if (nrows >= R)
      load(g, lds, wave);
    else
      Tile::load_lim(lds, g, wave, lane, nrows);
  }
};

// Combine the two half-wave partial values of a row (lanes l and l ^ 32).
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, x), __builtin_bit_cast(int, x), false, false);
  return fmaxf(__builtin_bit_cast(float, (int)r[0]), __builtin_bit_cast(float, (int)r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, x), __builtin_bit_cast(int, x), false, false);
  return __builtin_bit_cast(float, (int)r[0]) + __builtin_bit_cast(float, (int)r[1]);
}

// Per-lane part of a transposing operand read.  The operand is the 32 x 16
// block X^t[d][j] of a tile X[j][d] (j = tile row: key or query, natural
// order), d in [32 dt, 32 dt + 32), j in [j0, j0 + 16): lane l receives
// X[j0 + 8 (l/32) + e][32 dt + l%32] for e = 0..7, i.e. exactly the MFMA
// operand "row = l%32, 8 consecutive k from 8 (l/32)".  Built from two
// ds_read_b64_tr_b16: inside each 16-lane group, lane 4r + c supplies row
// j_r, columns d0 + 4c .. d0 + 4c + 3, and lane i receives column d0 + i of
// the four rows.
struct TrLane {
  int r;      // row within the 4-row group this lane addresses
  int dcol;   // column offset (within a 32-wide d tile) this lane addresses
  int hh;     // operand k-group (l / 32)
  __device__ __forceinline__ explicit TrLane(int lane) {
    const int g = lane >> 4, i = lane & 15;
    r = i >> 2;
    dcol = 16 * (g & 1) + 4 * (i & 3);
    hh = g >> 1;
  }
};

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Column offset of d-tile dt (for TrOps::issue).
__device__ __forceinline__ constexpr int dt_base(int dt) { return 32 * dt; }

// NOPS transposing operand reads X^t[d0 + (0..31)][16 t + (0..15)], t = 0..
// NOPS-1, of an R x D tile X (see DTile / TrLane).  Each operand is two
// ds_read_b64_tr_b16 issued as inline asm: the compiler's wait-count pass
// cannot tell these reads apart from the direct loads of the next stage
// that are in flight (it has no alias scope for them) and would otherwise
// wait for all of those loads before every such read.  The results are only
// valid after wait(), which waits for all outstanding LDS reads and ties the
// result registers to that wait.
template <typename T, int NOPS>
struct TrOps {
  typename Vec8<T>::type op[NOPS];

  template <int D>
  __device__ __forceinline__ void issue(const T* lds, const TrLane& tl, int d0) {
    const int d = d0 + tl.dcol;
#pragma unroll
    for (int t = 0; t < NOPS; ++t) {
      u32x2 part[2];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int m = swap23(16 * t + 8 * tl.hh + 4 * s + tl.r);
        const uint32_t a = lds_addr(lds + m * D + (((d >> 3) ^ swz<D>(m)) * 8) + (d & 7));
        asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(part[s]) : "v"(a));
      }
      u32x4 w;
      w[0] = part[0][0];
      w[1] = part[0][1];
      w[2] = part[1][0];
      w[3] = part[1][1];
      op[t] = __builtin_bit_cast(typename Vec8<T>::type, w);
    }
  }
  // Same reads from precomputed per-lane offsets: ofs[s] is the byte offset
  // (inside the tile) of this lane's half-s read for key group 0; key group
  // t adds t * 16 rows, folded into the instruction's immediate offset.
  template <int D>
  __device__ __forceinline__ void issue_at(uint32_t base, const uint32_t (&ofs)[2]) {
    const uint32_t a0 = base + ofs[0], a1 = base + ofs[1];
#pragma unroll
    for (int t = 0; t < NOPS; ++t) {
      u32x2 part[2];
      asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(part[0]) : "v"(a0), "i"(t * 16 * D * 2));
      asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(part[1]) : "v"(a1), "i"(t * 16 * D * 2));
      u32x4 w;
      w[0] = part[0][0];
      w[1] = part[0][1];
      w[2] = part[1][0];
      w[3] = part[1][1];
      op[t] = __builtin_bit_cast(typename Vec8<T>::type, w);
    }
  }
  // Same reads from per-lane LDS byte addresses a[s] (allocation base plus
  // the lane's half-s offset for key group 0) with the tile's byte offset
  // inside the allocation, IMM, folded into the instruction's immediate.
  template <int D, int IMM>
  __device__ __forceinline__ void issue_imm(const uint32_t (&a)[2]) {
    static_assert(IMM >= 0 && IMM + (NOPS - 1) * 16 * D * 2 <= 65535, "LDS immediate offset range");
#pragma unroll
    for (int t = 0; t < NOPS; ++t) {
      u32x2 part[2];
      asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(part[0]) : "v"(a[0]), "i"(IMM + t * 16 * D * 2));
      asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(part[1]) : "v"(a[1]), "i"(IMM + t * 16 * D * 2));
      u32x4 w;
      w[0] = part[0][0];
      w[1] = part[0][1];
      w[2] = part[1][0];
      w[3] = part[1][1];
      op[t] = __builtin_bit_cast(typename Vec8<T>::type, w);
    }
  }
  __device__ __forceinline__ void wait() {
    if constexpr (NOPS == 1) {
      asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(op[0]));
    } else if constexpr (NOPS == 2) {
      asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(op[0]), "+v"(op[1]));
    } else if constexpr (NOPS == 4) {
      asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(op[0]), "+v"(op[1]), "+v"(op[2]), "+v"(op[3]));
    } else {
      static_assert(NOPS == 1 || NOPS == 2 || NOPS == 4, "operand count");
    }
  }
};

// f(std::integral_constant<int, I>{}) for I = 0 .. N-1, unrolled.
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// N 16-byte LDS reads (ds_read_b128) issued back to back as inline asm, so
// that they are all in flight together; wait<I>() makes results 0 .. I valid
// (LDS reads of one wave complete in issue order) and ties them to that wait.
// As with TrOps, inline asm keeps the compiler's wait-count pass from
// waiting for the direct loads of later stages before these reads.
template <int N>
struct RowReads {
  static_assert(N >= 1 && N <= 16, "lgkmcnt counts up to 15 outstanding reads");
  u32x4 r[N];
  template <int I, int IMM>
  __device__ __forceinline__ void issue(uint32_t addr) {
    static_assert(I >= 0 && I < N && IMM >= 0 && IMM <= 65535, "read slot / immediate offset");
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r[I]) : "v"(addr), "i"(IMM));
  }
  template <int I>
  __device__ __forceinline__ void wait() {
    asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(r[I]) : "n"(N - 1 - I));
  }
  template <typename V>
  __device__ __forceinline__ V get(int i) const {
    return __builtin_bit_cast(V, r[i]);
  }
};

// Store 4 consecutive fp32 values (converted to T) as one 8-byte write.
template <typename T>
__device__ __forceinline__ void store4(T* dst, float a, float b, float c, float d) {
  T t0 = (T)a, t1 = (T)b, t2 = (T)c, t3 = (T)d;
  u32x2 w;
  w[0] = (uint32_t)__builtin_bit_cast(uint16_t, t0) | ((uint32_t)__builtin_bit_cast(uint16_t, t1) << 16);
  w[1] = (uint32_t)__builtin_bit_cast(uint16_t, t2) | ((uint32_t)__builtin_bit_cast(uint16_t, t3) << 16);
  *reinterpret_cast<u32x2*>(dst) = w;
}

// Store one lane's share of a transposed accumulator tile: acc holds the
// 32 x 32 block X^t[d][c] (rows d = natural MFMA rows, column c = this lane).
// Writes X[c][d0 + ...] of a row-major [., ld] matrix, scaled by s.
template <typename T>
__device__ __forceinline__ void store_acc_t(T* row_ptr, const f32x16& acc, int d0, int h, float s) {
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    int d = d0 + 8 * g + 4 * h;
    store4<T>(row_ptr + d, acc[4 * g] * s, acc[4 * g + 1] * s, acc[4 * g + 2] * s, acc[4 * g + 3] * s);
  }
}

// One wave's 32 x D output tile, held transposed in MFMA accumulators
// (acc[dt] holds X^t[d][c] with d = 32 dt + nat_row(r, h) and column c = this
// lane's row li), stored as 32 rows of a row-major [., D] matrix.  Stored
// straight from the accumulators, each 8-byte store instruction would touch
// 32 rows; staged through LDS, each 16-byte store instruction writes whole
// consecutive rows (64 / (D / 8) of them).
//   lds: this wave's private region of kStageBytes (32 rows, pitch 2 D + 16
//        bytes: the padding staggers the rows over the banks);
//   g:   row 0 of the tile in global memory (row stride G, normally D; G
//        < D: only the first G columns are stored);
//   s:   this lane's scale (its row's);
//   nrows: rows of the tile that exist (rows from nrows on are not stored).
// The caller makes sure no other wave uses the region.
template <int D>
struct RowStage {
  static constexpr int PITCH = 2 * D + 16;
  static constexpr int kStageBytes = 32 * PITCH;
};

template <typename T, int D, int G = D>
__device__ __forceinline__ void store_tile_rows(T* g, int nrows, const f32x16 (&acc)[D / 32], float s, char* lds,
                                                int lane) {
  static_assert(G % 8 == 0, "rows of whole 16-byte chunks");
  constexpr int PITCH = RowStage<D>::PITCH;
  constexpr int CPR = D / 8;        // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;     // rows per store instruction
  const int li = lane & 31, h = lane >> 5;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int d = 32 * dt + 8 * gq + 4 * h;
      T t0 = (T)(acc[dt][4 * gq] * s), t1 = (T)(acc[dt][4 * gq + 1] * s);
      T t2 = (T)(acc[dt][4 * gq + 2] * s), t3 = (T)(acc[dt][4 * gq + 3] * s);
      u32x2 w;
      w[0] = (uint32_t)__builtin_bit_cast(uint16_t, t0) | ((uint32_t)__builtin_bit_cast(uint16_t, t1) << 16);
      w[1] = (uint32_t)__builtin_bit_cast(uint16_t, t2) | ((uint32_t)__builtin_bit_cast(uint16_t, t3) << 16);
      *reinterpret_cast<u32x2*>(lds + li * PITCH + 2 * d) = w;
    }
  }
  // the region is this wave's own: its LDS writes complete in order before
  // its reads, which wait for them
#pragma unroll
  for (int i = 0; i < 32 / RPI; ++i) {
    const int row = RPI * i + lane / CPR, c = lane % CPR;
    const u32x4 v = *reinterpret_cast<const u32x4*>(lds + row * PITCH + 16 * c);
    if (row < nrows && (G >= D || 8 * c < G)) *reinterpret_cast<u32x4*>(g + (int64_t)row * G + 8 * c) = v;
  }
}

}  // namespace fa
