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

template <typename T> struct Vec8;
template <> struct Vec8<__bf16> { typedef bf16x8 type; };
template <> struct Vec8<_Float16> { typedef f16x8 type; };

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

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32, 64); }

__device__ __forceinline__ int swap23(int r) {
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

}  // namespace fa
