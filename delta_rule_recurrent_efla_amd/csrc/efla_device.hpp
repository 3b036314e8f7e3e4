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

// Scalar c of the rank-1 step S_t = (I - c k k^T) S_{t-1} + c k v^T for each
// step rule, x = beta lambda (the efla_coef values of the C interface):
//   0 exact flow (above); 1 explicit Euler, c = beta (papernotes note,
//   关键设计 item 1); 2 one classical RK4 step, c = beta (1 - x/2 + x^2/6 -
//   x^3/24), the matrix polynomial of the jsqmd.com article, section 5.3,
//   collapsed by A^n = lambda^(n-1) A; 3 that series cut after the
//   second-order term, c = beta (1 - x/2).
__device__ __forceinline__ float gate_coef(int coef, float beta, float lam) {
  if (coef == 0) return gate_alpha(beta, lam);
  if (coef == 1) return beta;
  const float x = beta * lam;
  if (coef == 2) return beta * (1.f + x * (-0.5f + x * (1.f / 6.f - x * (1.f / 24.f))));
  return beta * (1.f - 0.5f * x);
}

// Raw buffer access (gfx9 buffer descriptor, stride 0, range checked): a load
// whose per-lane byte offset is at or past `bytes` returns zeros and touches
// no memory. Descriptors are wave-uniform (scalar registers); per-lane offsets
// are 32-bit, so loads need no 64-bit address arithmetic.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, long long bytes) {
  const int n = bytes <= 0 ? 0 : (bytes > 0x7fffffffLL ? 0x7fffffff : (int)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}
__device__ __forceinline__ void buf_load(__amdgpu_buffer_rsrc_t r, unsigned off, bf16x8& v) {
  v = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ void buf_load(__amdgpu_buffer_rsrc_t r, unsigned off, floatx4& v) {
  v = __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ void buf_load(__amdgpu_buffer_rsrc_t r, unsigned off, bf16& v) {
  v = __builtin_bit_cast(bf16, __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0));
}
__device__ __forceinline__ void buf_load(__amdgpu_buffer_rsrc_t r, unsigned off, float& v) {
  v = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

// x plus x of lane l ^ 16 (xor16_sum) or l ^ 32 (xor32_sum), in every lane.
// gfx950's row swaps exchange 16-lane rows (the odd rows of one operand with
// the even rows of the other) or 32-lane halves inside the VALU, with no LDS
// round trip: given x as both operands, the two results hold the two rows
// (halves) that meet in each lane. The results are copied out of the returned
// vector before the bit cast: a bit cast of a vector element reads element 0
// with this compiler. Every lane must be active.
__device__ __forceinline__ float xor16_sum(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const unsigned lo = r[0], hi = r[1];
  return __builtin_bit_cast(float, lo) + __builtin_bit_cast(float, hi);
}
__device__ __forceinline__ float xor32_sum(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const unsigned lo = r[0], hi = r[1];
  return __builtin_bit_cast(float, lo) + __builtin_bit_cast(float, hi);
}

// Inclusive prefix sum over the 64 lanes (lane l receives x_0 + ... + x_l):
// DPP right shifts by 1, 2, 4, 8 inside each 16-lane row (lanes shifted in
// from outside the row add 0), then the totals of the rows below, read from
// lanes 15, 31 and 47. Every lane must be active.
__device__ __forceinline__ float wave_prefix_sum(float x) {
  auto shr = [](float v, auto n) {  // row_shr:n is DPP control 0x110 + n
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                 0x110 + decltype(n)::value, 0xf, 0xf, false));
  };
  x += shr(x, std::integral_constant<int, 1>{});
  x += shr(x, std::integral_constant<int, 2>{});
  x += shr(x, std::integral_constant<int, 4>{});
  x += shr(x, std::integral_constant<int, 8>{});
  const float t0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 15));
  const float t1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 31));
  const float t2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 47));
  const int row = lane_id() >> 4;
  const float below = row == 0 ? 0.f : (row == 1 ? t0 : (row == 2 ? t0 + t1 : (t0 + t1) + t2));
  return x + below;
}

// Sum over aligned groups of N consecutive lanes (N = 1, 2, 4, 8, 16, 32),
// every lane of a group receiving the group's sum. Within a 16-lane row the
// exchange uses DPP (quad permutes, then half-row and row mirrors), across
// rows the row swap. Every lane must be active.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  auto dpp = [](float v, auto ctrl) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v),
                                                              decltype(ctrl)::value, 0xf, 0xf,
                                                              false));
  };
  if constexpr (N >= 2) x += dpp(x, std::integral_constant<int, 0xB1>{});   // quad_perm 1,0,3,2
  if constexpr (N >= 4) x += dpp(x, std::integral_constant<int, 0x4E>{});   // quad_perm 2,3,0,1
  if constexpr (N >= 8) x += dpp(x, std::integral_constant<int, 0x141>{});  // row_half_mirror
  if constexpr (N >= 16) x += dpp(x, std::integral_constant<int, 0x140>{}); // row_mirror
  if constexpr (N >= 32) x = xor16_sum(x);
  static_assert(N <= 32, "group size");
  return x;
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
// MFMA traits.
//
// A "fragment" is one lane's share of an MFMA operand for a k-step covering
// KT 16-row tiles: bf16 MFMAs (16x16x32) cover two tiles per instruction, fp32
// MFMAs (16x16x4) one tile in four instructions. Inside a tile, k slot
// (g, e) is row 4g + e, so an accumulator tile (rows 4g + e per lane) turns
// into a fragment with no data movement across lanes:
//   * as the B operand of A*X (k running over X's rows), or
//   * as the A operand of X^T*B (k running over X's rows again).
// LDS rows are read with the same k order: 4 contiguous elements at
// column (16 t + 4 g) ^ swz, where swz (a multiple of 4) is the row's XOR
// swizzle (0 for unswizzled arrays).
template <typename CT>
struct Mma;

template <>
struct Mma<bf16> {
  static constexpr int PAD = 4;   // row padding (elements) of unpermuted tiles
  static constexpr int PADP = 8;  // row padding of column-permuted tiles (16-byte rows)
  static constexpr int KT = 2;    // 16-row tiles per fragment
  typedef bf16x8 Frag;

  // Column-permuted LDS layout (used by the pipelined kernel): inside every
  // 32-column block, column 16h + 4g + e is stored at position 8g + 4h + e,
  // so the 8 elements lane group g needs for one fragment (columns 4g..4g+3
  // of both 16-column tiles) are one 16-byte read.
  __device__ __forceinline__ static constexpr int pcol(int c) {
    return (c & ~31) | ((c & 12) << 1) | ((c & 16) >> 2) | (c & 3);
  }

  __device__ __forceinline__ static floatx4 mma(floatx4 c, Frag a, Frag b) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  __device__ __forceinline__ static bf16x4 cvt4(floatx4 v) {
    return __builtin_convertvector(v, bf16x4);
  }
  __device__ __forceinline__ static bf16x8 cat(bf16x4 lo, bf16x4 hi) {
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
  // Fragment f (tiles 2f, 2f+1) of NR accumulator tiles.
  template <int NR>
  __device__ __forceinline__ static Frag acc(const floatx4* t, int f) {
    bf16x4 hi = {};
    if (2 * f + 1 < NR) hi = cvt4(t[2 * f + 1]);
    return cat(cvt4(t[2 * f]), hi);
  }
  // Fragment f of an unpermuted LDS row (k contiguous), restricted to NR tiles:
  // columns 32f + 4g.. and 32f + 16 + 4g.., XOR-swizzled by swz.
  template <int NR>
  __device__ __forceinline__ static Frag lds(const bf16* row, int f, int swz) {
    const int g = lane_id() >> 4;
    bf16x4 lo = *(const bf16x4*)(row + ((32 * f + 4 * g) ^ swz));
    bf16x4 hi = {};
    if (2 * f + 1 < NR) hi = *(const bf16x4*)(row + ((32 * f + 16 + 4 * g) ^ swz));
    return cat(lo, hi);
  }
  // Fragment f of a column-permuted LDS row (16-byte aligned), NR tiles.
  template <int NR>
  __device__ __forceinline__ static Frag ldp(const bf16* row, int f) {
    const int g = lane_id() >> 4;
    if (2 * f + 1 < NR) return *(const bf16x8*)(row + 32 * f + 8 * g);
    return cat(*(const bf16x4*)(row + 32 * f + 8 * g), bf16x4{});
  }
  // c += A[16 x K] * B[K x 16] with A row and B column from LDS, natural k
  // order (8 contiguous elements per lane, 8-byte aligned). K % 16 == 0.
  template <int K>
  __device__ __forceinline__ static void ll(floatx4& c, const bf16* arow, const bf16* bcol) {
    const int g = lane_id() >> 4;
#pragma unroll
    for (int k0 = 0; k0 + 32 <= K; k0 += 32) c = mma(c, ld8(arow + k0 + 8 * g), ld8(bcol + k0 + 8 * g));
    if constexpr (K % 32 == 16) {
      constexpr int k0 = K - 16;
      bf16x8 a = {}, b = {};
      if (g < 2) {
        a = ld8(arow + k0 + 8 * g);
        b = ld8(bcol + k0 + 8 * g);
      }
      c = mma(c, a, b);
    }
  }
  // Same product for two column-permuted rows (16-byte reads; the k order is
  // the permuted one, identical for both operands).
  template <int K>
  __device__ __forceinline__ static void llp(floatx4& c, const bf16* arow, const bf16* bcol) {
#pragma unroll
    for (int f = 0; f < (K + 31) / 32; ++f)
      c = mma(c, ldp<K / 16>(arow, f), ldp<K / 16>(bcol, f));
  }
  // 8 contiguous elements from an 8-byte aligned LDS address (two 8-byte reads).
  __device__ __forceinline__ static bf16x8 ld8(const bf16* p) {
    return cat(*(const bf16x4*)p, *(const bf16x4*)(p + 4));
  }
  // Accumulator tile -> 4 contiguous elements at dst_row + 4g.
  __device__ __forceinline__ static void store_t(bf16* dst_row, floatx4 v) {
    const int g = lane_id() >> 4;
    *(bf16x4*)(dst_row + 4 * g) = cvt4(v);
  }
  // Accumulator tile -> columns 16 J + 4g .. + 3 of a column-permuted row.
  __device__ __forceinline__ static void store_tp(bf16* row, int J, floatx4 v) {
    const int g = lane_id() >> 4;
    *(bf16x4*)(row + pcol(16 * J + 4 * g)) = cvt4(v);
  }
  // Swizzled form of the column-permuted layout, for tiles that are stored
  // from accumulators (lane (g, i) writes row i) and read as fragments: in
  // row r the 16-byte group g of every 32-column block sits at g ^ sw(r),
  // sw(r) = (r >> 2) & 3. Measured on gfx950 at row strides of 160 and 288
  // bytes, this halves the cycles of the tile stores (a 2-way bank conflict
  // without it) and keeps the fragment and transposed reads conflict-free.
  // Callers pass the row of lane i of a 16-row tile, so sw = (i >> 2) & 3.
  __device__ __forceinline__ static int sw() { return (lane_id() >> 2) & 3; }
  __device__ __forceinline__ static void store_tps(bf16* row, int J, floatx4 v) {
    const int g = lane_id() >> 4;
    *(bf16x4*)(row + 32 * (J >> 1) + 8 * (g ^ sw()) + 4 * (J & 1)) = cvt4(v);
  }
  template <int NR>
  __device__ __forceinline__ static Frag ldps(const bf16* row, int f) {
    const int g = lane_id() >> 4;
    const bf16* p = row + 32 * f + 8 * (g ^ sw());
    if (2 * f + 1 < NR) return *(const bf16x8*)p;
    return cat(*(const bf16x4*)p, bf16x4{});
  }
  __device__ __forceinline__ static floatx4 load4(const bf16* p) {
    return __builtin_convertvector(*(const bf16x4*)p, floatx4);
  }
};

template <>
struct Mma<float> {
  static constexpr int PAD = 4;
  static constexpr int PADP = 4;
  static constexpr int KT = 1;
  typedef floatx4 Frag;  // the four k-slices of one tile

  // fp32 fragments are already one 16-byte read: no column permutation.
  __device__ __forceinline__ static constexpr int pcol(int c) { return c; }

  __device__ __forceinline__ static floatx4 mma(floatx4 c, Frag a, Frag b) {
#pragma unroll
    for (int s = 0; s < 4; ++s) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s], c, 0, 0, 0);
    return c;
  }
  template <int NR>
  __device__ __forceinline__ static Frag acc(const floatx4* t, int f) {
    return t[f];
  }
  template <int NR>
  __device__ __forceinline__ static Frag lds(const float* row, int f, int swz) {
    const int g = lane_id() >> 4;
    return *(const floatx4*)(row + ((16 * f + 4 * g) ^ swz));
  }
  template <int K>
  __device__ __forceinline__ static void ll(floatx4& c, const float* arow, const float* bcol) {
    const int g = lane_id() >> 4;
#pragma unroll
    for (int k0 = 0; k0 < K; k0 += 4)
      c = __builtin_amdgcn_mfma_f32_16x16x4f32(arow[k0 + g], bcol[k0 + g], c, 0, 0, 0);
  }
  template <int NR>
  __device__ __forceinline__ static Frag ldp(const float* row, int f) {
    const int g = lane_id() >> 4;
    return *(const floatx4*)(row + 16 * f + 4 * g);
  }
  template <int K>
  __device__ __forceinline__ static void llp(floatx4& c, const float* arow, const float* bcol) {
    ll<K>(c, arow, bcol);
  }
  __device__ __forceinline__ static void store_t(float* dst_row, floatx4 v) {
    const int g = lane_id() >> 4;
    *(floatx4*)(dst_row + 4 * g) = v;
  }
  __device__ __forceinline__ static void store_tp(float* row, int J, floatx4 v) {
    const int g = lane_id() >> 4;
    *(floatx4*)(row + 16 * J + 4 * g) = v;
  }
  // Same swizzle as the bf16 form: 16-byte group g of row i at g ^ ((i >> 2) & 3).
  __device__ __forceinline__ static int sw() { return (lane_id() >> 2) & 3; }
  __device__ __forceinline__ static void store_tps(float* row, int J, floatx4 v) {
    const int g = lane_id() >> 4;
    *(floatx4*)(row + 16 * J + 4 * (g ^ sw())) = v;
  }
  template <int NR>
  __device__ __forceinline__ static Frag ldps(const float* row, int f) {
    const int g = lane_id() >> 4;
    return *(const floatx4*)(row + 16 * f + 4 * (g ^ sw()));
  }
  __device__ __forceinline__ static floatx4 load4(const float* p) { return *(const floatx4*)p; }
};

// 16-byte register vector <-> LDS at 8-byte alignment (bf16 rows are padded
// by 8 bytes, so a 16-byte LDS access is issued as two 8-byte ones).
__device__ __forceinline__ void st16(bf16* p, bf16x8 v) {
  *(bf16x4*)p = __builtin_shufflevector(v, v, 0, 1, 2, 3);
  *(bf16x4*)(p + 4) = __builtin_shufflevector(v, v, 4, 5, 6, 7);
}
__device__ __forceinline__ bf16x8 ld16(const bf16* p) { return Mma<bf16>::ld8(p); }
__device__ __forceinline__ void st16(float* p, floatx4 v) { *(floatx4*)p = v; }
// Sum of squares of a 16-byte vector, in fp32 (bf16 pairs by packed dot
// products: the products are exact in fp32).
__device__ __forceinline__ float sumsq(bf16x8 v) {
  typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bf16x2 p = {v[2 * i], v[2 * i + 1]};
    s = __builtin_amdgcn_fdot2_f32_bf16(p, p, s, false);
  }
  return s;
}
__device__ __forceinline__ float sumsq(floatx4 v) { return v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3]; }
// Four fp32 values -> 4 consecutive elements at p (8 bytes as bf16, rounded to
// nearest even; 16 bytes as fp32).
__device__ __forceinline__ void store4(bf16* p, floatx4 v) { *(bf16x4*)p = __builtin_convertvector(v, bf16x4); }
__device__ __forceinline__ void store4(float* p, floatx4 v) { *(floatx4*)p = v; }
__device__ __forceinline__ floatx4 ld16(const float* p) { return *(const floatx4*)p; }

// Four consecutive rows row0 .. row0+3 of column col0 + (lane & 15) of a
// row-major LDS tile with leading dimension ld (elements). row0 may differ
// between the four 16-lane groups; col0 is a multiple of 16.
//   bf16: one ds_read_b64_tr_b16. Within each 16-lane group, lane a + 4m
//   addresses row row0 + m, columns col0 + 4a .. col0 + 4a + 3, and the
//   instruction returns to lane 4a + b column col0 + 4a + b of those four rows.
//   fp32: four 4-byte reads.
template <bool PERM = false>
__device__ __forceinline__ bf16x4 ldtr4(const bf16* base, int ld, int row0, int col0) {
  const int li = lane_id() & 15;
  const int col = col0 + 4 * (li & 3);
  const bf16* p = base + (row0 + (li >> 2)) * ld + (PERM ? Mma<bf16>::pcol(col) : col);
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (__attribute__((address_space(3))) bf16x4*)(p));
}
template <bool PERM = false>
__device__ __forceinline__ floatx4 ldtr4(const float* base, int ld, int row0, int col0) {
  const int li = lane_id() & 15;
  const float* p = base + row0 * ld + col0 + li;
  return floatx4{p[0], p[ld], p[2 * ld], p[3 * ld]};
}
__device__ __forceinline__ floatx4 to_f32x4(bf16x4 v) { return __builtin_convertvector(v, floatx4); }
__device__ __forceinline__ floatx4 to_f32x4(floatx4 v) { return v; }

// Fragment f (k over rows 32f.. or 16f.. of a row-major tile) of the
// transposed tile, for a 16-column block at col0: lane i gets column col0 + i.
// NR bounds the row tiles present.
template <int NR, bool PERM = false>
__device__ __forceinline__ bf16x8 tr_frag(const bf16* base, int ld, int f, int col0) {
  const int g = lane_id() >> 4;
  bf16x4 lo = ldtr4<PERM>(base, ld, 32 * f + 4 * g, col0);
  bf16x4 hi = {};
  if (2 * f + 1 < NR) hi = ldtr4<PERM>(base, ld, 32 * f + 16 + 4 * g, col0);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}
template <int NR, bool PERM = false>
__device__ __forceinline__ floatx4 tr_frag(const float* base, int ld, int f, int col0) {
  const int g = lane_id() >> 4;
  return ldtr4<PERM>(base, ld, 16 * f + 4 * g, col0);
}

// 16-byte register vector of 8 (bf16) or 4 (fp32) consecutive columns
// starting at c0 (a multiple of 8, or 4) -> column-permuted LDS row.
__device__ __forceinline__ void st_perm(bf16* row, int c0, bf16x8 v) {
  *(bf16x4*)(row + Mma<bf16>::pcol(c0)) = __builtin_shufflevector(v, v, 0, 1, 2, 3);
  *(bf16x4*)(row + Mma<bf16>::pcol(c0 + 4)) = __builtin_shufflevector(v, v, 4, 5, 6, 7);
}
__device__ __forceinline__ void st_perm(float* row, int c0, floatx4 v) { *(floatx4*)(row + c0) = v; }

// Number of fragments covering NR 16-row tiles.
template <typename CT, int NR>
struct NFrag {
  static constexpr int value = (NR + Mma<CT>::KT - 1) / Mma<CT>::KT;
};

}  // namespace efla
