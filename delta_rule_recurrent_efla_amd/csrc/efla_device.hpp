// Device-side building blocks for the gfx950 EFLA kernels: the fp32
// exact-flow gate and 16x16 MFMA fragment helpers for bf16 (16x16x32) and
// fp32 (16x16x4) operands.
//
// Fragment conventions (wave64). Lane l has i = l & 15 and g = l >> 4.
//   * Accumulator tile (floatx4): lane holds rows 4g + e (e = 0..3) of
//     column i of a 16x16 fp32 tile.
//   * A operand: lane supplies row i of A; B operand: lane supplies column i
//     of B. Both carry the same set of k indices per (g, slot), so the k
//     order inside one MFMA is free: the helpers below choose it so that an
//     accumulator tile can be fed back as a B operand without leaving
//     registers (k slot (g, e) <-> row 4g + e of each 16-row tile).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace efla {

typedef __bf16 bf16;
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Exact-flow coefficient alpha = (1 - e^{-beta*lambda}) / lambda, in fp32,
// with lambda floored at 1e-12 and the numerator formed by expm1 (rank-1
// collapse: papernotes note, 关键设计 item 2; floor and expm1: 损失函数 / 训练策略).
__device__ __forceinline__ float gate_alpha(float beta, float lam) {
  const float lamc = fmaxf(lam, 1e-12f);
  return -expm1f(-beta * lamc) / lamc;
}

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }

template <typename CT>
__device__ __forceinline__ CT from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

// ---------------------------------------------------------------------------
// MFMA traits. All pointers are LDS pointers already offset to the lane's
// row (A) or column (B), k running contiguously.
template <typename CT>
struct Mma;

template <>
struct Mma<bf16> {
  static constexpr int PAD = 8;  // 16-byte row padding in elements
  typedef bf16x8 Pack;           // B operand covering two 16-row tiles

  __device__ __forceinline__ static floatx4 mfma(bf16x8 a, bf16x8 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  __device__ __forceinline__ static bf16x4 cvt4(floatx4 v) {
    return __builtin_convertvector(v, bf16x4);
  }
  __device__ __forceinline__ static bf16x8 cat(bf16x4 lo, bf16x4 hi) {
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }

  // c += A[16 x K] * B[K x 16]; A row and B column both from LDS, k contiguous.
  // K is a multiple of 16.
  template <int K>
  __device__ __forceinline__ static void ll(floatx4& c, const bf16* arow, const bf16* bcol) {
    const int g = lane_id() >> 4;
#pragma unroll
    for (int k0 = 0; k0 + 32 <= K; k0 += 32) {
      bf16x8 a = *(const bf16x8*)(arow + k0 + 8 * g);
      bf16x8 b = *(const bf16x8*)(bcol + k0 + 8 * g);
      c = mfma(a, b, c);
    }
    if constexpr (K % 32 == 16) {
      constexpr int k0 = K - 16;
      bf16x8 a = {}, b = {};
      if (g < 2) {
        a = *(const bf16x8*)(arow + k0 + 8 * g);
        b = *(const bf16x8*)(bcol + k0 + 8 * g);
      }
      c = mfma(a, b, c);
    }
  }

  // Pack NR accumulator row tiles (rows 16r + 4g + e) into B operands.
  template <int NR>
  __device__ __forceinline__ static void pack(const floatx4* t, Pack* p) {
#pragma unroll
    for (int r = 0; r < NR; r += 2) {
      bf16x4 lo = cvt4(t[r]);
      bf16x4 hi = {};
      if (r + 1 < NR) hi = cvt4(t[r + 1]);
      p[r / 2] = cat(lo, hi);
    }
  }

  // c += A[16 x 16*NR] * B where B's 16-row tiles come packed from registers.
  // A is read with the matching k order (4 contiguous per 16-row tile).
  template <int NR>
  __device__ __forceinline__ static void lp(floatx4& c, const bf16* arow, const Pack* p) {
    const int g = lane_id() >> 4;
#pragma unroll
    for (int r = 0; r < NR; r += 2) {
      bf16x4 lo = *(const bf16x4*)(arow + 16 * r + 4 * g);
      bf16x4 hi = {};
      if (r + 1 < NR) hi = *(const bf16x4*)(arow + 16 * (r + 1) + 4 * g);
      c = mfma(cat(lo, hi), p[r / 2], c);
    }
  }

  // Accumulator tile -> LDS, transposed: lane writes its 4 rows as 4
  // consecutive elements of row (lane's column) of dst.
  __device__ __forceinline__ static void store_t(bf16* dst_row, floatx4 v) {
    const int g = lane_id() >> 4;
    *(bf16x4*)(dst_row + 4 * g) = cvt4(v);
  }
};

template <>
struct Mma<float> {
  static constexpr int PAD = 4;
  typedef floatx4 Pack;  // one 16-row tile, kept in fp32

  __device__ __forceinline__ static floatx4 mfma(float a, float b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }

  template <int K>
  __device__ __forceinline__ static void ll(floatx4& c, const float* arow, const float* bcol) {
    const int g = lane_id() >> 4;
#pragma unroll
    for (int k0 = 0; k0 < K; k0 += 4) c = mfma(arow[k0 + g], bcol[k0 + g], c);
  }

  template <int NR>
  __device__ __forceinline__ static void pack(const floatx4* t, Pack* p) {
#pragma unroll
    for (int r = 0; r < NR; ++r) p[r] = t[r];
  }

  template <int NR>
  __device__ __forceinline__ static void lp(floatx4& c, const float* arow, const Pack* p) {
    const int g = lane_id() >> 4;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
#pragma unroll
      for (int s = 0; s < 4; ++s) c = mfma(arow[16 * r + 4 * g + s], p[r][s], c);
    }
  }

  __device__ __forceinline__ static void store_t(float* dst_row, floatx4 v) {
    const int g = lane_id() >> 4;
    *(floatx4*)(dst_row + 4 * g) = v;
  }
};

// Number of packs needed for NR row tiles.
template <typename CT, int NR>
struct PackCount {
  static constexpr int value = sizeof(CT) == 2 ? (NR + 1) / 2 : NR;
};

}  // namespace efla
