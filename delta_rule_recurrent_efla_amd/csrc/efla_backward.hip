// Backward of the chunk-parallel EFLA forward for gfx950: gradients of a loss
// of o and S_T with respect to q, k, v, beta and S0.
//
// The pages give no gradient formulas (papernotes.org note "Exact Flow Linear
// Attention: Exact Solution from Continuous-Time Dynamics" states the forward;
// its 实验 sections train with it). This is reverse mode through the chunk
// form of the forward (整体框架: WY/UT chunks). Per chunk with start state S,
// D = diag(c) (the step scalars), A = strictly-lower(D K K^T),
// T = (I + A)^{-1}, Yh = V - K S, U = T D Yh, M = lower-incl-diag(Q K^T):
//   forward   O = Q S + M U,  S' = S + K^T U
//   backward  dU = M^T dO + K dS',  G = T^T dU,  dV = D G
//             dS = dS' + Q^T dO - K^T D G
//             dM = lower-incl-diag(dO U^T),  E = strictly-lower(-G U^T)
//             dc = rowsum(G * Yh) + rowsum(E * K K^T)
//             dQ = dO S^T + dM K
//             dK = dM^T Q + U dS'^T - D G S^T + D E K + E^T D K + 2 dc c_lambda k
//             dbeta = dc c_beta
// Four launches:
//   1. the forward again (pipelined kernel, pass mode 2): the state at the
//      start of every chunk;
//   2. efla_bwd_prep_kernel, one workgroup per (head, chunk): c, c_beta,
//      c_lambda, K K^T, T (by forward substitution in fp32), T^T and M^T;
//   3. efla_bwd_state_kernel, one workgroup per (head, 64-column slice),
//      chunks last to first: the dS recurrence (the only serial part), dV,
//      G and the dS' of every chunk;
//   4. efla_bwd_grad_kernel, one workgroup per (head, chunk) (in the bf16
//      form one persistent workgroup per CU over those items): dq, dk, dbeta.
// Numerics: fp32 inputs run every product as v_mfma_f32_16x16x4_f32 with fp32
// storage. bf16 inputs with C and d multiples of 32 (the "bf16 form":
// efla_bwd_state_kernel_bf, efla_bwd_grad_kernel_bf) take bf16 MFMA operands
// (v_mfma_f32_16x16x32_bf16) and keep the chunk-start states, T^T, M^T, dS'
// and G as bf16 in the workspace, accumulating in fp32 (G's one fp32 use, the
// row sum of G * Yh in dc, then takes the rounded G); the gradient kernel
// forms K K^T itself instead of reading it. The other bf16 shapes run the
// fp32 form. The gate and its derivatives are fp32 everywhere.

#include <hip/hip_runtime.h>

#include "efla_device.hpp"

namespace efla {

// acc += A B over k in [0, 16 nkb) for one 16x16 tile. fa(kb) returns
// A(row li, 16 kb + 4 g + e), e = 0..3; fb(kb) returns B(16 kb + 4 g + e,
// col li). Step e of block kb lets lane (g, li) supply k = 16 kb + 4 g + e to
// v_mfma_f32_16x16x4_f32 (whose k index is g), so a row-major A and a
// column-major B each give their four values as one 16-byte read. The result
// holds rows 4 g + e, column li.
template <class FA, class FB>
__device__ __forceinline__ floatx4 mm16(floatx4 acc, int nkb, FA fa, FB fb) {
  for (int kb = 0; kb < nkb; ++kb) {
    const floatx4 a = fa(kb), b = fb(kb);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], acc, 0, 0, 0);
  }
  return acc;
}

// acc += A B over k in [0, KD) for one 16x16 tile, with the operands given
// as fa(k0) = A(row li, k0 .. k0 + 3) and fb(k0) = B(k0 .. k0 + 3, col li).
// BF (bf16 inputs, KD a multiple of 32): v_mfma_f32_16x16x32_bf16 with lane
// (g, li) supplying k = 32 kb + 4 g + {0..3} and 32 kb + 16 + 4 g + {0..3}
// (the same slots for A and B), operands rounded to bf16; otherwise the fp32
// product of mm16.
template <int KD, bool BF, class FA, class FB>
__device__ __forceinline__ floatx4 mmk(floatx4 acc, FA fa, FB fb) {
  const int g = (threadIdx.x & 63) >> 4;
  if constexpr (BF && KD % 32 == 0) {
#pragma unroll 2
    for (int kb = 0; kb < KD / 32; ++kb) {
      const int k0 = 32 * kb + 4 * g;
      const bf16x4 a0 = __builtin_convertvector(fa(k0), bf16x4), a1 = __builtin_convertvector(fa(k0 + 16), bf16x4);
      const bf16x4 b0 = __builtin_convertvector(fb(k0), bf16x4), b1 = __builtin_convertvector(fb(k0 + 16), bf16x4);
      const bf16x8 a8 = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
      const bf16x8 b8 = __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a8, b8, acc, 0, 0, 0);
    }
    return acc;
  } else {
    for (int kb = 0; kb < KD / 16; ++kb) {
      const int k0 = 16 * kb + 4 * g;
      const floatx4 a = fa(k0), b = fb(k0);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], acc, 0, 0, 0);
    }
    return acc;
  }
}

// bf16 operand fragments of mmk's layout for all KD / 32 blocks, formed once
// and reused across tiles: out[kb] holds f(32 kb + 4 g .. + 3) and
// f(32 kb + 16 + 4 g .. + 3).
template <int KD, class F>
__device__ __forceinline__ void bf_frags(bf16x8* out, F f) {
  const int g = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int kb = 0; kb < KD / 32; ++kb) {
    const bf16x4 x0 = __builtin_convertvector(f(32 * kb + 4 * g), bf16x4);
    const bf16x4 x1 = __builtin_convertvector(f(32 * kb + 16 + 4 * g), bf16x4);
    out[kb] = __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7);
  }
}
// acc += A B with B (fb == nullptr: A) given as precomputed fragments
template <int KD, class FA>
__device__ __forceinline__ floatx4 mm_fb(floatx4 acc, FA fa, const bf16x8* bfr) {
  bf16x8 afr[KD / 32];
  bf_frags<KD>(afr, fa);
#pragma unroll
  for (int kb = 0; kb < KD / 32; ++kb) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr[kb], bfr[kb], acc, 0, 0, 0);
  return acc;
}
template <int KD, class FB>
__device__ __forceinline__ floatx4 mm_fa(floatx4 acc, const bf16x8* afr, FB fb) {
  bf16x8 bfr[KD / 32];
  bf_frags<KD>(bfr, fb);
#pragma unroll
  for (int kb = 0; kb < KD / 32; ++kb) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr[kb], bfr[kb], acc, 0, 0, 0);
  return acc;
}

__device__ __forceinline__ float ld1(const float* p) { return *p; }
__device__ __forceinline__ float ld1(const bf16* p) { return (float)*p; }
// four consecutive elements (8- or 16-byte aligned)
__device__ __forceinline__ floatx4 ld4(const float* p) { return *(const floatx4*)p; }
__device__ __forceinline__ floatx4 ld4(const bf16* p) { return __builtin_convertvector(*(const bf16x4*)p, floatx4); }

// dc/dbeta and dc/dlambda of gate_coef, in fp32.
__device__ __forceinline__ void gate_coef_grad(int coef, float beta, float lam, float& db, float& dl) {
  if (coef == 1) {
    db = 1.f;
    dl = 0.f;
    return;
  }
  const float x = beta * lam;
  if (coef == 2) {
    db = 1.f + x * (-1.f + x * (0.5f - x * (1.f / 6.f)));
    dl = beta * beta * (-0.5f + x * (1.f / 3.f - x * (1.f / 8.f)));
    return;
  }
  if (coef == 3) {
    db = 1.f - x;
    dl = -0.5f * beta * beta;
    return;
  }
  const float lamc = fmaxf(lam, 1e-12f);
  const float xc = beta * lamc;
  const float ex = expf(-xc);
  db = ex;
  if (!(lam > 1e-12f)) {
    dl = 0.f;  // the floor makes the scalar constant in lambda
  } else if (fabsf(xc) < 0.1f) {
    // (beta e^{-x} - c)/lambda = beta^2 sum_{n>=1} (-1)^n n x^{n-1}/(n+1)!
    dl = beta * beta *
         (-0.5f + xc * (1.f / 3.f + xc * (-1.f / 8.f + xc * (1.f / 30.f + xc * (-1.f / 144.f + xc * (1.f / 840.f))))));
  } else {
    dl = (beta * ex - gate_alpha(beta, lam)) / lamc;
  }
}

struct BwdArgs {
  const void *q, *k, *v, *beta, *dout;
  const float *s0, *dsT;
  void *dq, *dk, *dv, *dbeta;
  float* ds0;
  int T, nc, coef, nh;
  // workspace (fp32, except sc, dsc and gw in the bf16 form: bf16 inputs with
  // C and d multiples of 32)
  const float* sc;  // [head][chunk][d_v][d_k] state at the start of each chunk
  const float* scn; // the same states, [head][chunk][d_k][d_v]
  float* dsc;       // [head][chunk][d_k][d_v] gradient of the state at each chunk's end
  float* gw;        // [head][nc C][d_v] G rows
  float *al, *fb, *fl;        // [head][nc C] c, dc/dbeta, dc/dlambda (0 past T)
  float *gram, *tn, *tt, *mt;  // [head][chunk][C][C]: K K^T (fp32 form only), T, T^T, M^T
};

// ---------------------------------------------------------------------------
// 2. Per (head, chunk): scalars, K K^T, T = (I + A)^{-1}, T^T, M^T.
template <typename CT, int D, int C>
__global__ __launch_bounds__(256) void efla_bwd_prep_kernel(BwdArgs a) {
  // M^T and T^T are stored as bf16 where their only reader rounds them to bf16
  // (the bf16 form of the state pass), else as fp32
  constexpr bool MBF = sizeof(CT) == 2 && C % 32 == 0 && D % 32 == 0;
  // K and Q rows are staged in the input type where the products take them as
  // bf16 MFMA operands (the smaller footprint lets more workgroups share a
  // CU), else in fp32; A and T (fp32, row stride LC) reuse their space
  using LT = std::conditional_t<MBF, bf16, float>;
  constexpr int LC = C + 4;
  constexpr int LK = MBF ? D + 16 : D + 4;  // bf16 rows: 32 bytes mod 64
  constexpr int LQ = LK * (int)sizeof(LT) >= LC * 4 ? LK : (LC * 4 + (int)sizeof(LT) - 1) / (int)sizeof(LT);
  // K rows, then (after the Gram tiles) T
  __shared__ __attribute__((aligned(16))) LT Kf[C][LQ];
  // Q rows, then (after the Q K^T tiles) strictly-lower D K K^T
  __shared__ __attribute__((aligned(16))) LT Qf[C][LQ];
  auto Am = [&](int i, int j) -> float& { return ((float*)&Qf[0][0])[i * LC + j]; };
  auto Ts = [&](int i, int j) -> float& { return ((float*)&Kf[0][0])[i * LC + j]; };
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, li = lane & 15, g = lane >> 4;
  const int h = blockIdx.x / a.nc, ch = blockIdx.x % a.nc;
  const int t0 = ch * C, nval = min(C, a.T - t0);
  const CT* kg = (const CT*)a.k + ((size_t)h * a.T + t0) * D;
  const CT* qg = (const CT*)a.q + ((size_t)h * a.T + t0) * D;
  constexpr int VE = 16 / (int)sizeof(LT);  // elements per 16-byte piece
  using Piece = std::conditional_t<MBF, bf16x8, floatx4>;
  // every load is issued before the first LDS write (rows past T are read
  // clamped to the last row and staged as zeros; no load behind a branch,
  // which would make the compiler wait for each in turn); beta of row
  // tid / 4 with them
  constexpr int NP = C * D / VE, NPT = (NP + 255) / 256;
  constexpr bool EXP = NPT * 256 == NP;
  Piece kx[NPT], qx[NPT];
#pragma unroll
  for (int it = 0; it < NPT; ++it) {
    const int i = min(tid + 256 * it, NP - 1), r = min(i / (D / VE), nval - 1), c = VE * (i % (D / VE));
    if constexpr (MBF) {
      kx[it] = *(const bf16x8*)(kg + (size_t)r * D + c);
      qx[it] = *(const bf16x8*)(qg + (size_t)r * D + c);
    } else {
      kx[it] = ld4(kg + (size_t)r * D + c);
      qx[it] = ld4(qg + (size_t)r * D + c);
    }
  }
  const float bq = ld1((const CT*)a.beta + (size_t)h * a.T + t0 + min(tid >> 2, nval - 1));
#pragma unroll
  for (int it = 0; it < NPT; ++it) {
    const int i = tid + 256 * it, r = i / (D / VE), c = VE * (i % (D / VE));
    if (EXP || i < NP) {
      *(Piece*)&Kf[r][c] = r < nval ? kx[it] : Piece{};
      *(Piece*)&Qf[r][c] = r < nval ? qx[it] : Piece{};
    }
  }
  __syncthreads();
  const size_t rb = (size_t)h * a.nc * C + t0;  // row base of this chunk
  __shared__ float cs[C];
  {
    // lambda of row tid / 4: four lanes sum every fourth 16-byte piece
    const int r = tid >> 2, part = tid & 3;
    float lam = 0.f;
    if (r < C) {
      for (int pc = part; pc < D / VE; pc += 4) {
        const Piece x = *(const Piece*)&Kf[r][VE * pc];
#pragma unroll
        for (int e = 0; e < VE; ++e) lam = fmaf((float)x[e], (float)x[e], lam);
      }
    }
    lam = group_sum<4>(lam);
    if (r < C && part == 0) {
      float c = 0.f, db = 0.f, dl = 0.f;
      if (r < nval) {
        c = gate_coef(a.coef, bq, lam);
        gate_coef_grad(a.coef, bq, lam, db, dl);
      }
      cs[r] = c;
      a.al[rb + r] = c;
      a.fb[rb + r] = db;
      a.fl[rb + r] = dl;
    }
  }
  __syncthreads();
  const size_t mb = ((size_t)h * a.nc + ch) * C * C;
  constexpr int NT = C / 16;
  const floatx4 z = {0.f, 0.f, 0.f, 0.f};
  // M^T tiles (J, I) as Q K^T products: A = rows of Q, B = rows of K; lane
  // (g, li) holds M[16I + 4g + e][16J + li] = M^T[16J + li][16I + 4g + e],
  // 4 consecutive entries of one row of M^T, stored together
  for (int tl = w; tl < NT * NT; tl += 4) {
    const int I = tl / NT, J = tl % NT;
    // bf16 inputs: products of bf16 values are exact in fp32, so the bf16 MFMA
    // gives the same K K^T and Q K^T as the fp32 one
    const floatx4 qk = mmk<D, sizeof(CT) == 2>(z, [&](int k0) { return ld4(&Qf[16 * I + li][k0]); },
                                               [&](int k0) { return ld4(&Kf[16 * J + li][k0]); });
    const int j = 16 * J + li, i0 = 16 * I + 4 * g;
    floatx4 m;
#pragma unroll
    for (int e = 0; e < 4; ++e) m[e] = j <= i0 + e ? qk[e] : 0.f;  // M[i][j] = q_i . k_j for j <= i
    if constexpr (MBF) *(bf16x4*)&((bf16*)a.mt)[mb + (size_t)j * C + i0] = __builtin_convertvector(m, bf16x4);
    else *(floatx4*)&a.mt[mb + (size_t)j * C + i0] = m;
  }
  __syncthreads();  // Q is dead: its space takes A
  // K K^T tiles (I, J): lane (g, li) holds row 16I + li, columns
  // 16J + 4g .. + 3 (operands swapped), stored 16 bytes at a time
  for (int tl = w; tl < NT * NT; tl += 4) {
    const int I = tl / NT, J = tl % NT;
    const floatx4 gk = mmk<D, sizeof(CT) == 2>(z, [&](int k0) { return ld4(&Kf[16 * J + li][k0]); },
                                               [&](int k0) { return ld4(&Kf[16 * I + li][k0]); });
    const int i = 16 * I + li, j0 = 16 * J + 4 * g;
    // the bf16 form's gradient kernel forms these tiles itself from the same
    // bf16 keys, with the same products in the same order
    if constexpr (!MBF) *(floatx4*)&a.gram[mb + (size_t)i * C + j0] = gk;
    const float ci = cs[i];
    floatx4 am;
#pragma unroll
    for (int e = 0; e < 4; ++e) am[e] = j0 + e < i ? ci * gk[e] : 0.f;
    *(floatx4*)&Am(i, j0) = am;
  }
  __syncthreads();  // K is dead: its space takes T
  // T = (I + A)^{-1} by blocks. Diagonal blocks: lane (b, c) solves column c
  // of (I + A_bb) t = e_c by forward substitution in fp32 (all blocks at once)
  if (w == 0 && lane < C) {
    const int bb = lane >> 4, c = lane & 15;
    float t[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float sum = (r == c) ? 1.f : 0.f;
#pragma unroll
      for (int m4 = 0; m4 < r; m4 += 4) {
        const floatx4 a4 = *(const floatx4*)&Am(16 * bb + r, 16 * bb + m4);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (m4 + e < r) sum = fmaf(-a4[e], t[m4 + e], sum);
      }
      t[r] = sum;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) Ts(16 * bb + r, 16 * bb + c) = t[r];
  }
  // blocks above the diagonal are zero
  for (int i = tid; i < C * C; i += 256)
    if ((i % C) / 16 > (i / C) / 16) Ts(i / C, i % C) = 0.f;
  __syncthreads();
  // block rows below: T_ij = -T_ii sum_{j <= m < i} A_im T_mj, on fp32 MFMA;
  // block row i needs the rows above it (one barrier per block row)
  for (int i = 1; i < NT; ++i) {
    const int j = w;  // block column of this wave
    if (j < i) {
      floatx4 p = z;
      for (int k0 = 16 * j + 4 * g; k0 < 16 * i; k0 += 16) {
        const floatx4 a4 = *(const floatx4*)&Am(16 * i + li, k0);
#pragma unroll
        for (int e = 0; e < 4; ++e) p = __builtin_amdgcn_mfma_f32_16x16x4f32(a4[e], Ts(k0 + e, 16 * j + li), p, 0, 0, 0);
      }
      // -T_ii P: B from the accumulator (rows 4 g + e of P)
      const floatx4 t4 = *(const floatx4*)&Ts(16 * i + li, 16 * i + 4 * g);
      floatx4 x = z;
#pragma unroll
      for (int e = 0; e < 4; ++e) x = __builtin_amdgcn_mfma_f32_16x16x4f32(-t4[e], p[e], x, 0, 0, 0);
#pragma unroll
      for (int e = 0; e < 4; ++e) Ts(16 * i + 4 * g + e, 16 * j + li) = x[e];
    }
    __syncthreads();
  }
  // T (in the bf16 form T D, the only form its reader takes: rounded to bf16,
  // columns permuted so a fragment is one 16-byte read) and T^T to the
  // workspace
  for (int i = tid; i < C * C / 4; i += 256) {
    const int r = i / (C / 4), c4 = 4 * (i % (C / 4));
    if constexpr (MBF) {
      const floatx4 td = *(const floatx4*)&Ts(r, c4) * *(const floatx4*)&cs[c4];
      *(bf16x4*)&((bf16*)a.tn)[mb + (size_t)r * C + Mma<bf16>::pcol(c4)] = __builtin_convertvector(td, bf16x4);
    } else {
      *(floatx4*)&a.tn[mb + (size_t)r * C + c4] = *(const floatx4*)&Ts(r, c4);
    }
    floatx4 x;
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = Ts(c4 + e, r);
    if constexpr (MBF) *(bf16x4*)&((bf16*)a.tt)[mb + (size_t)r * C + c4] = __builtin_convertvector(x, bf16x4);
    else *(floatx4*)&a.tt[mb + (size_t)r * C + c4] = x;
  }
}

// Workgroups are dealt to the 8 XCDs round robin. This index keeps the column
// slices of one head on one XCD: they read the same K, Q, M^T and T^T rows,
// so the second read hits that XCD's L2.
__device__ __forceinline__ int bwd_xcd_slot(int nvt) {
  const int n = gridDim.x;
  if (n % 8 == 0 && (n / 8) % nvt == 0) return (blockIdx.x % 8) * (n / 8) + blockIdx.x / 8;
  return blockIdx.x;
}

// ---------------------------------------------------------------------------
// 3. Per (head, BV-column slice), chunks last to first: the dS recurrence.
// Wave w < BV/16 owns columns 16 w .. 16 w + 15 of the slice; its d_k x 16
// block of dS stays in MFMA accumulator registers.
template <int D, int C, int BV>
struct StateSmem {
  static constexpr int LD = D + 4, LC = C + 4;
  float Kf[C][LD];    // K rows
  float KT[D][LC];    // K^T
  float QT[D][LC];    // Q^T
  float MT[C][LC];    // M^T
  float TT[C][LC];    // T^T
  float dOT[BV][LC];  // dO^T (slice columns)
  float al[C];
};

template <typename CT, int D, int C, int BV>
__global__ __launch_bounds__(256) void efla_bwd_state_kernel(BwdArgs a) {
  using Sm = StateSmem<D, C, BV>;
  __shared__ __attribute__((aligned(16))) Sm sm;
  constexpr int NKT = D / 16, NB = C / 16, NW = BV / 16;
  const int tid = threadIdx.x, lane = tid & 63, li = lane & 15, g = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nvt = D / BV;
  const int L = bwd_xcd_slot(nvt);
  const int h = L / nvt, v0 = (L % nvt) * BV;
  const int col = v0 + 16 * w + li;  // this lane's state column (when w < NW)
  const bool owner = w < NW;
  floatx4 ds[NKT];
#pragma unroll
  for (int rt = 0; rt < NKT; ++rt) ds[rt] = floatx4{0.f, 0.f, 0.f, 0.f};
  if (owner && a.dsT) {
#pragma unroll
    for (int rt = 0; rt < NKT; ++rt)
#pragma unroll
      for (int e = 0; e < 4; ++e) ds[rt][e] = a.dsT[((size_t)h * D + 16 * rt + 4 * g + e) * D + col];
  }
  const CT* kg = (const CT*)a.k + (size_t)h * a.T * D;
  const CT* qg = (const CT*)a.q + (size_t)h * a.T * D;
  const CT* dog = (const CT*)a.dout + (size_t)h * a.T * D;
  // The next chunk's inputs (chunks run last to first) are requested into
  // registers while this chunk computes, then written to LDS.
  constexpr int NLK = (C * D / 4 + 255) / 256, NLO = (C * BV / 4 + 255) / 256, NLM = (C * C / 4 + 255) / 256;
  floatx4 rk[NLK], rq[NLK], ro[NLO], rm[NLM], rt4[NLM];
  float ral = 0.f;
  auto fetch = [&](int ch) {
    const int t0 = ch * C, nval = min(C, a.T - t0);
    const size_t mb = ((size_t)h * a.nc + ch) * C * C;
    const floatx4 z4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < NLK; ++j) {
      const int i = tid + 256 * j, r = i / (D / 4), c4 = 4 * (i % (D / 4));
      const bool ok = i < C * D / 4 && r < nval;
      rk[j] = ok ? ld4(kg + (size_t)(t0 + r) * D + c4) : z4;
      rq[j] = ok ? ld4(qg + (size_t)(t0 + r) * D + c4) : z4;
    }
#pragma unroll
    for (int j = 0; j < NLO; ++j) {
      const int i = tid + 256 * j, r = i / (BV / 4), c4 = 4 * (i % (BV / 4));
      ro[j] = (i < C * BV / 4 && r < nval) ? ld4(dog + (size_t)(t0 + r) * D + v0 + c4) : z4;
    }
#pragma unroll
    for (int j = 0; j < NLM; ++j) {
      const int i = tid + 256 * j;
      if (i < C * C / 4) {
        rm[j] = ld4(a.mt + mb + 4 * (size_t)i);
        rt4[j] = ld4(a.tt + mb + 4 * (size_t)i);
      }
    }
    if (tid < C) ral = a.al[(size_t)h * a.nc * C + t0 + tid];
  };
  fetch(a.nc - 1);
  for (int ch = a.nc - 1; ch >= 0; --ch) {
    const int t0 = ch * C, nval = min(C, a.T - t0);
    // dS' of this chunk (natural layout [d_k][d_v])
    if (owner) {
      float* dst = a.dsc + ((size_t)h * a.nc + ch) * D * D;
#pragma unroll
      for (int rt = 0; rt < NKT; ++rt)
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[(size_t)(16 * rt + 4 * g + e) * D + col] = ds[rt][e];
    }
    __syncthreads();  // the previous chunk's reads of LDS are done
#pragma unroll
    for (int j = 0; j < NLK; ++j) {
      const int i = tid + 256 * j, r = i / (D / 4), c4 = 4 * (i % (D / 4));
      if (i < C * D / 4) {
        *(floatx4*)&sm.Kf[r][c4] = rk[j];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sm.KT[c4 + e][r] = rk[j][e];
          sm.QT[c4 + e][r] = rq[j][e];
        }
      }
    }
#pragma unroll
    for (int j = 0; j < NLO; ++j) {
      const int i = tid + 256 * j, r = i / (BV / 4), c4 = 4 * (i % (BV / 4));
      if (i < C * BV / 4) {
#pragma unroll
        for (int e = 0; e < 4; ++e) sm.dOT[c4 + e][r] = ro[j][e];
      }
    }
#pragma unroll
    for (int j = 0; j < NLM; ++j) {
      const int i = tid + 256 * j, r = i / (C / 4), c4 = 4 * (i % (C / 4));
      if (i < C * C / 4) {
        *(floatx4*)&sm.MT[r][c4] = rm[j];
        *(floatx4*)&sm.TT[r][c4] = rt4[j];
      }
    }
    if (tid < C) sm.al[tid] = ral;
    // always issued (the first chunk's again at the end): a conditional load
    // would make the compiler copy the registers at the loop latch
    fetch(ch > 0 ? ch - 1 : 0);
    __syncthreads();
    if (owner) {
      const floatx4 z = {0.f, 0.f, 0.f, 0.f};
      // dU = M^T dO + K dS'
      floatx4 du[NB];
#pragma unroll
      for (int I = 0; I < NB; ++I) {
        floatx4 acc = mm16(z, NB, [&](int kb) { return *(const floatx4*)&sm.MT[16 * I + li][16 * kb + 4 * g]; },
                           [&](int kb) { return *(const floatx4*)&sm.dOT[16 * w + li][16 * kb + 4 * g]; });
#pragma unroll
        for (int rt = 0; rt < NKT; ++rt) {
          const floatx4 a4 = *(const floatx4*)&sm.Kf[16 * I + li][16 * rt + 4 * g];
#pragma unroll
          for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a4[e], ds[rt][e], acc, 0, 0, 0);
        }
        du[I] = acc;
      }
      // G = T^T dU; D G is dV
      floatx4 dy[NB];
      float* grow = a.gw + ((size_t)h * a.nc * C + t0) * D;
      CT* dvg = (CT*)a.dv + ((size_t)h * a.T + t0) * D;
#pragma unroll
      for (int I = 0; I < NB; ++I) {
        floatx4 acc = z;
#pragma unroll
        for (int kb = 0; kb < NB; ++kb) {
          const floatx4 a4 = *(const floatx4*)&sm.TT[16 * I + li][16 * kb + 4 * g];
#pragma unroll
          for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a4[e], du[kb][e], acc, 0, 0, 0);
        }
        const floatx4 al4 = *(const floatx4*)&sm.al[16 * I + 4 * g];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * I + 4 * g + e;
          grow[(size_t)r * D + col] = acc[e];
          dy[I][e] = al4[e] * acc[e];
          if (r < nval) dvg[(size_t)r * D + col] = from_f32<CT>(dy[I][e]);
        }
      }
      // dS = dS' + Q^T dO - K^T D G
#pragma unroll
      for (int rt = 0; rt < NKT; ++rt) {
        floatx4 acc = mm16(ds[rt], NB, [&](int kb) { return *(const floatx4*)&sm.QT[16 * rt + li][16 * kb + 4 * g]; },
                           [&](int kb) { return *(const floatx4*)&sm.dOT[16 * w + li][16 * kb + 4 * g]; });
#pragma unroll
        for (int kb = 0; kb < NB; ++kb) {
          const floatx4 a4 = *(const floatx4*)&sm.KT[16 * rt + li][16 * kb + 4 * g];
#pragma unroll
          for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(-a4[e], dy[kb][e], acc, 0, 0, 0);
        }
        ds[rt] = acc;
      }
    }
  }
  if (owner && a.ds0) {
#pragma unroll
    for (int rt = 0; rt < NKT; ++rt)
#pragma unroll
      for (int e = 0; e < 4; ++e) a.ds0[((size_t)h * D + 16 * rt + 4 * g + e) * D + col] = ds[rt][e];
  }
}

// bf16 form of the same pass (bf16 inputs, C and d multiples of 32): the
// chunk's operands sit in LDS as bf16 and every product is
// v_mfma_f32_16x16x32_bf16. Lane (g, li) supplies k = 32 kb + 4 g + {0..3}
// and 32 kb + 16 + 4 g + {0..3}: for an operand held in accumulators these
// are rows 4 g + e of tiles 2 kb and 2 kb + 1, so dS', dU and D G feed the
// next product without lane exchange. K, Q and the dO slice are staged
// row-major with 16-byte writes; the operands that run over their columns
// (K^T, Q^T as A, dO as B) are read with ds_read_b64_tr_b16. Every row
// stride is an odd multiple of 32 bytes, which keeps both the 16-byte writes
// and the transposed reads free of bank conflicts. T and M are rounded to
// bf16, as in the forward; accumulation and the dS state stay fp32.
template <int D, int C, int BV>
struct StateSmemBf {
  static constexpr int LD = D + 16, LO = BV + ((32 - 2 * BV % 64 + 64) % 64) / 2, LC = C + 8;
  bf16 Kf[C][LD];
  bf16 Qf[C][LD];
  bf16 dOf[C][LO];
  bf16 MT[C][LC];
  bf16 TT[C][LC];
  float al[C];
};

__device__ __forceinline__ bf16x8 pk8(bf16x4 a, bf16x4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ bf16x4 cv4(floatx4 x) { return __builtin_convertvector(x, bf16x4); }

template <int D, int C, int BV>
__global__ __launch_bounds__(256) void efla_bwd_state_kernel_bf(BwdArgs a) {
  using Sm = StateSmemBf<D, C, BV>;
  static_assert((Sm::LD * 2) % 64 == 32 && (Sm::LO * 2) % 64 == 32, "row strides");
  __shared__ __attribute__((aligned(16))) Sm sm;
  constexpr int NKT = D / 16, NB = C / 16, NW = BV / 16;
  const int tid = threadIdx.x, lane = tid & 63, li = lane & 15, g = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nvt = D / BV;
  const int L = bwd_xcd_slot(nvt);
  const int h = L / nvt, v0 = (L % nvt) * BV;
  const int col = v0 + 16 * w + li;
  const bool owner = w < NW;
  floatx4 ds[NKT];
#pragma unroll
  for (int rt = 0; rt < NKT; ++rt) ds[rt] = floatx4{0.f, 0.f, 0.f, 0.f};
  if (owner && a.dsT) {
#pragma unroll
    for (int rt = 0; rt < NKT; ++rt)
#pragma unroll
      for (int e = 0; e < 4; ++e) ds[rt][e] = a.dsT[((size_t)h * D + 16 * rt + 4 * g + e) * D + col];
  }
  const bf16* kg = (const bf16*)a.k + (size_t)h * a.T * D;
  const bf16* qg = (const bf16*)a.q + (size_t)h * a.T * D;
  const bf16* dog = (const bf16*)a.dout + (size_t)h * a.T * D;
  // 16-byte pieces per thread: K and Q rows, the dO slice, M^T and T^T (fp32)
  constexpr int NLK = (C * D / 8 + 255) / 256, NLO = (C * BV / 8 + 255) / 256, NLM = (C * C / 4 + 255) / 256;
  bf16x8 rk[NLK], rq[NLK], ro[NLO];
  bf16x4 rm[NLM], rt4[NLM];  // M^T and T^T, stored as bf16 for this form
  float ral = 0.f;
  auto fetch = [&](int ch) {
    const int t0 = ch * C, nval = min(C, a.T - t0);
    const size_t mb = ((size_t)h * a.nc + ch) * C * C;
    const bf16x8 z8 = {};
#pragma unroll
    for (int j = 0; j < NLK; ++j) {
      const int i = tid + 256 * j, r = i / (D / 8), c8 = 8 * (i % (D / 8));
      const bool ok = i < C * D / 8 && r < nval;
      rk[j] = ok ? *(const bf16x8*)(kg + (size_t)(t0 + r) * D + c8) : z8;
      rq[j] = ok ? *(const bf16x8*)(qg + (size_t)(t0 + r) * D + c8) : z8;
    }
#pragma unroll
    for (int j = 0; j < NLO; ++j) {
      const int i = tid + 256 * j, r = i / (BV / 8), c8 = 8 * (i % (BV / 8));
      ro[j] = (i < C * BV / 8 && r < nval) ? *(const bf16x8*)(dog + (size_t)(t0 + r) * D + v0 + c8) : z8;
    }
#pragma unroll
    for (int j = 0; j < NLM; ++j) {
      const int i = tid + 256 * j;
      if (i < C * C / 4) {
        rm[j] = *(const bf16x4*)((const bf16*)a.mt + mb + 4 * (size_t)i);
        rt4[j] = *(const bf16x4*)((const bf16*)a.tt + mb + 4 * (size_t)i);
      }
    }
    if (tid < C) ral = a.al[(size_t)h * a.nc * C + t0 + tid];
  };
  auto ld_a = [&](const bf16* row, int kb) {  // A(row, 32 kb + 4 g + ..) and (.. + 16)
    return pk8(*(const bf16x4*)(row + 32 * kb + 4 * g), *(const bf16x4*)(row + 32 * kb + 16 + 4 * g));
  };
  fetch(a.nc - 1);
  for (int ch = a.nc - 1; ch >= 0; --ch) {
    const int t0 = ch * C, nval = min(C, a.T - t0);
    if (owner) {
      bf16* dst = (bf16*)a.dsc + ((size_t)h * a.nc + ch) * D * D;
#pragma unroll
      for (int rt = 0; rt < NKT; ++rt)
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[(size_t)(16 * rt + 4 * g + e) * D + col] = (bf16)ds[rt][e];
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < NLK; ++j) {
      const int i = tid + 256 * j, r = i / (D / 8), c8 = 8 * (i % (D / 8));
      if (i < C * D / 8) {
        *(bf16x8*)&sm.Kf[r][c8] = rk[j];
        *(bf16x8*)&sm.Qf[r][c8] = rq[j];
      }
    }
#pragma unroll
    for (int j = 0; j < NLO; ++j) {
      const int i = tid + 256 * j, r = i / (BV / 8), c8 = 8 * (i % (BV / 8));
      if (i < C * BV / 8) *(bf16x8*)&sm.dOf[r][c8] = ro[j];
    }
#pragma unroll
    for (int j = 0; j < NLM; ++j) {
      const int i = tid + 256 * j, r = i / (C / 4), c4 = 4 * (i % (C / 4));
      if (i < C * C / 4) {
        *(bf16x4*)&sm.MT[r][c4] = rm[j];
        *(bf16x4*)&sm.TT[r][c4] = rt4[j];
      }
    }
    if (tid < C) sm.al[tid] = ral;
    fetch(ch > 0 ? ch - 1 : 0);  // always issued (see the fp32 form)
    __syncthreads();
    if (owner) {
      const floatx4 z = {0.f, 0.f, 0.f, 0.f};
      // dO columns of this wave as B fragments (k = tokens)
      bf16x8 dof[NB / 2];
#pragma unroll
      for (int kb = 0; kb < NB / 2; ++kb) dof[kb] = tr_frag<NB>(&sm.dOf[0][0], Sm::LO, kb, 16 * w);
      // Q^T dO: no dependence on dS', so it runs ahead of the chain
      floatx4 qd[NKT];
#pragma unroll
      for (int rt = 0; rt < NKT; ++rt) {
        floatx4 acc = ds[rt];
#pragma unroll
        for (int kb = 0; kb < NB / 2; ++kb)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(tr_frag<NB>(&sm.Qf[0][0], Sm::LD, kb, 16 * rt), dof[kb], acc,
                                                        0, 0, 0);
        qd[rt] = acc;
      }
      // dU = M^T dO + K dS'
      floatx4 du[NB];
#pragma unroll
      for (int I = 0; I < NB; ++I) {
        floatx4 acc = z;
#pragma unroll
        for (int kb = 0; kb < NB / 2; ++kb)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ld_a(&sm.MT[16 * I + li][0], kb), dof[kb], acc, 0, 0, 0);
#pragma unroll
        for (int kb = 0; kb < NKT / 2; ++kb)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ld_a(&sm.Kf[16 * I + li][0], kb),
                                                        pk8(cv4(ds[2 * kb]), cv4(ds[2 * kb + 1])), acc, 0, 0, 0);
        du[I] = acc;
      }
      // G = T^T dU; D G is dV. G is stored as bf16: the gradient kernel
      // takes it as a bf16 MFMA operand, and in one fp32 row sum (dc)
      floatx4 dy[NB];
      bf16* grow = (bf16*)a.gw + ((size_t)h * a.nc * C + t0) * D;
      bf16* dvg = (bf16*)a.dv + ((size_t)h * a.T + t0) * D;
#pragma unroll
      for (int I = 0; I < NB; ++I) {
        floatx4 acc = z;
#pragma unroll
        for (int kb = 0; kb < NB / 2; ++kb)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ld_a(&sm.TT[16 * I + li][0], kb),
                                                        pk8(cv4(du[2 * kb]), cv4(du[2 * kb + 1])), acc, 0, 0, 0);
        const floatx4 al4 = *(const floatx4*)&sm.al[16 * I + 4 * g];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * I + 4 * g + e;
          grow[(size_t)r * D + col] = (bf16)acc[e];
          dy[I][e] = al4[e] * acc[e];
          if (r < nval) dvg[(size_t)r * D + col] = (bf16)dy[I][e];
        }
      }
      // dS = dS' + Q^T dO - K^T D G
#pragma unroll
      for (int rt = 0; rt < NKT; ++rt) {
        floatx4 acc = qd[rt];
#pragma unroll
        for (int kb = 0; kb < NB / 2; ++kb)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(tr_frag<NB>(&sm.Kf[0][0], Sm::LD, kb, 16 * rt),
                                                        pk8(cv4(-dy[2 * kb]), cv4(-dy[2 * kb + 1])), acc, 0, 0, 0);
        ds[rt] = acc;
      }
    }
  }
  if (owner && a.ds0) {
#pragma unroll
    for (int rt = 0; rt < NKT; ++rt)
#pragma unroll
      for (int e = 0; e < 4; ++e) a.ds0[((size_t)h * D + 16 * rt + 4 * g + e) * D + col] = ds[rt][e];
  }
}

// The same dS recurrence with the chunk operands staged by four loader waves
// into a double-buffered copy of the LDS tiles: the four column waves compute
// chunk ch from one buffer while the loaders stage chunk ch - 1 into the
// other, from registers fetched one chunk step earlier, and then fetch chunk
// ch - 2. One workgroup barrier per chunk; the column waves' arithmetic is
// that of efla_bwd_state_kernel_bf, bit for bit.
template <int D, int C, int BV>
__global__ __launch_bounds__(512) void efla_bwd_state_kernel_bfp(BwdArgs a) {
  using Sm = StateSmemBf<D, C, BV>;
  static_assert((Sm::LD * 2) % 64 == 32 && (Sm::LO * 2) % 64 == 32, "row strides");
  __shared__ __attribute__((aligned(16))) Sm sm[2];
  constexpr int NKT = D / 16, NB = C / 16, NW = BV / 16;
  static_assert(NW <= 4, "four column waves");
  const int tid = threadIdx.x, lane = tid & 63, li = lane & 15, g = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nvt = D / BV;
  const int L = bwd_xcd_slot(nvt);
  const int h = L / nvt, v0 = (L % nvt) * BV;
  const bf16* kg = (const bf16*)a.k + (size_t)h * a.T * D;
  const bf16* qg = (const bf16*)a.q + (size_t)h * a.T * D;
  const bf16* dog = (const bf16*)a.dout + (size_t)h * a.T * D;
  if (w >= 4) {
    // ======== loaders (waves 4..7): loader thread lt = tid - 256
    const int lt = tid - 256;
    constexpr int NLK = (C * D / 8 + 255) / 256, NLO = (C * BV / 8 + 255) / 256, NLM = (C * C / 4 + 255) / 256;
    bf16x8 rk[NLK], rq[NLK], ro[NLO];
    bf16x4 rm[NLM], rt4[NLM];
    float ral = 0.f;
    auto fetch = [&](int ch) {
      const int t0 = ch * C, nval = min(C, a.T - t0);
      const size_t mb = ((size_t)h * a.nc + ch) * C * C;
      const bf16x8 z8 = {};
#pragma unroll
      for (int j = 0; j < NLK; ++j) {
        const int i = lt + 256 * j, r = i / (D / 8), c8 = 8 * (i % (D / 8));
        const bool ok = i < C * D / 8 && r < nval;
        rk[j] = ok ? *(const bf16x8*)(kg + (size_t)(t0 + r) * D + c8) : z8;
        rq[j] = ok ? *(const bf16x8*)(qg + (size_t)(t0 + r) * D + c8) : z8;
      }
#pragma unroll
      for (int j = 0; j < NLO; ++j) {
        const int i = lt + 256 * j, r = i / (BV / 8), c8 = 8 * (i % (BV / 8));
        ro[j] = (i < C * BV / 8 && r < nval) ? *(const bf16x8*)(dog + (size_t)(t0 + r) * D + v0 + c8) : z8;
      }
#pragma unroll
      for (int j = 0; j < NLM; ++j) {
        const int i = lt + 256 * j;
        if (i < C * C / 4) {
          rm[j] = *(const bf16x4*)((const bf16*)a.mt + mb + 4 * (size_t)i);
          rt4[j] = *(const bf16x4*)((const bf16*)a.tt + mb + 4 * (size_t)i);
        }
      }
      if (lt < C) ral = a.al[(size_t)h * a.nc * C + t0 + lt];
    };
    auto stage = [&](Sm& S) {
#pragma unroll
      for (int j = 0; j < NLK; ++j) {
        const int i = lt + 256 * j, r = i / (D / 8), c8 = 8 * (i % (D / 8));
        if (i < C * D / 8) {
          *(bf16x8*)&S.Kf[r][c8] = rk[j];
          *(bf16x8*)&S.Qf[r][c8] = rq[j];
        }
      }
#pragma unroll
      for (int j = 0; j < NLO; ++j) {
        const int i = lt + 256 * j, r = i / (BV / 8), c8 = 8 * (i % (BV / 8));
        if (i < C * BV / 8) *(bf16x8*)&S.dOf[r][c8] = ro[j];
      }
#pragma unroll
      for (int j = 0; j < NLM; ++j) {
        const int i = lt + 256 * j, r = i / (C / 4), c4 = 4 * (i % (C / 4));
        if (i < C * C / 4) {
          *(bf16x4*)&S.MT[r][c4] = rm[j];
          *(bf16x4*)&S.TT[r][c4] = rt4[j];
        }
      }
      if (lt < C) S.al[lt] = ral;
    };
    fetch(a.nc - 1);
    stage(sm[(a.nc - 1) & 1]);
    fetch(a.nc > 1 ? a.nc - 2 : 0);  // always issued (the last one repeats)
    __syncthreads();
    for (int ch = a.nc - 1; ch >= 0; --ch) {
      if (ch > 0) {
        stage(sm[(ch - 1) & 1]);
        fetch(ch > 1 ? ch - 2 : 0);
      }
      __syncthreads();
    }
    return;
  }
  // ======== column waves (0..3): wave w < BV / 16 owns columns v0 + 16 w ..
  const int col = v0 + 16 * w + li;
  const bool owner = w < NW;
  floatx4 ds[NKT];
#pragma unroll
  for (int rt = 0; rt < NKT; ++rt) ds[rt] = floatx4{0.f, 0.f, 0.f, 0.f};
  if (owner && a.dsT) {
#pragma unroll
    for (int rt = 0; rt < NKT; ++rt)
#pragma unroll
      for (int e = 0; e < 4; ++e) ds[rt][e] = a.dsT[((size_t)h * D + 16 * rt + 4 * g + e) * D + col];
  }
  auto ld_a = [&](const bf16* row, int kb) {  // A(row, 32 kb + 4 g + ..) and (.. + 16)
    return pk8(*(const bf16x4*)(row + 32 * kb + 4 * g), *(const bf16x4*)(row + 32 * kb + 16 + 4 * g));
  };
  __syncthreads();  // the last chunk is staged
  for (int ch = a.nc - 1; ch >= 0; --ch) {
    const int t0 = ch * C, nval = min(C, a.T - t0);
    Sm& S = sm[ch & 1];
    if (owner) {
      bf16* dst = (bf16*)a.dsc + ((size_t)h * a.nc + ch) * D * D;
#pragma unroll
      for (int rt = 0; rt < NKT; ++rt)
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[(size_t)(16 * rt + 4 * g + e) * D + col] = (bf16)ds[rt][e];
    }
    if (owner) {
      const floatx4 z = {0.f, 0.f, 0.f, 0.f};
      // dO columns of this wave as B fragments (k = tokens)
      bf16x8 dof[NB / 2];
#pragma unroll
      for (int kb = 0; kb < NB / 2; ++kb) dof[kb] = tr_frag<NB>(&S.dOf[0][0], Sm::LO, kb, 16 * w);
      // Q^T dO: no dependence on dS', so it runs ahead of the chain
      floatx4 qd[NKT];
#pragma unroll
      for (int rt = 0; rt < NKT; ++rt) {
        floatx4 acc = ds[rt];
#pragma unroll
        for (int kb = 0; kb < NB / 2; ++kb)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(tr_frag<NB>(&S.Qf[0][0], Sm::LD, kb, 16 * rt), dof[kb], acc,
                                                        0, 0, 0);
        qd[rt] = acc;
      }
      // dU = M^T dO + K dS'
      floatx4 du[NB];
#pragma unroll
      for (int I = 0; I < NB; ++I) {
        floatx4 acc = z;
#pragma unroll
        for (int kb = 0; kb < NB / 2; ++kb)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ld_a(&S.MT[16 * I + li][0], kb), dof[kb], acc, 0, 0, 0);
#pragma unroll
        for (int kb = 0; kb < NKT / 2; ++kb)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ld_a(&S.Kf[16 * I + li][0], kb),
                                                        pk8(cv4(ds[2 * kb]), cv4(ds[2 * kb + 1])), acc, 0, 0, 0);
        du[I] = acc;
      }
      // G = T^T dU; D G is dV. G is stored as bf16: the gradient kernel
      // takes it as a bf16 MFMA operand, and in one fp32 row sum (dc)
      floatx4 dy[NB];
      bf16* grow = (bf16*)a.gw + ((size_t)h * a.nc * C + t0) * D;
      bf16* dvg = (bf16*)a.dv + ((size_t)h * a.T + t0) * D;
#pragma unroll
      for (int I = 0; I < NB; ++I) {
        floatx4 acc = z;
#pragma unroll
        for (int kb = 0; kb < NB / 2; ++kb)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ld_a(&S.TT[16 * I + li][0], kb),
                                                        pk8(cv4(du[2 * kb]), cv4(du[2 * kb + 1])), acc, 0, 0, 0);
        const floatx4 al4 = *(const floatx4*)&S.al[16 * I + 4 * g];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * I + 4 * g + e;
          grow[(size_t)r * D + col] = (bf16)acc[e];
          dy[I][e] = al4[e] * acc[e];
          if (r < nval) dvg[(size_t)r * D + col] = (bf16)dy[I][e];
        }
      }
      // dS = dS' + Q^T dO - K^T D G
#pragma unroll
      for (int rt = 0; rt < NKT; ++rt) {
        floatx4 acc = qd[rt];
#pragma unroll
        for (int kb = 0; kb < NB / 2; ++kb)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(tr_frag<NB>(&S.Kf[0][0], Sm::LD, kb, 16 * rt),
                                                        pk8(cv4(-dy[2 * kb]), cv4(-dy[2 * kb + 1])), acc, 0, 0, 0);
        ds[rt] = acc;
      }
    }
    __syncthreads();
  }
  if (owner && a.ds0) {
#pragma unroll
    for (int rt = 0; rt < NKT; ++rt)
#pragma unroll
      for (int e = 0; e < 4; ++e) a.ds0[((size_t)h * D + 16 * rt + 4 * g + e) * D + col] = ds[rt][e];
  }
}

// ---------------------------------------------------------------------------
// 4. Per (head, chunk): dq, dk, dbeta from S, dS', G and the chunk's inputs.
// Every MFMA operand is a 16-byte read: rows of K, dO, V, G and of the two
// stored layouts of S and dS' from global memory (L2), the rest from LDS.
template <int D, int C>
struct GradSmem {
  static constexpr int LD = D + 4, LC = C + 4;
  union {
    float YT[D][LC];  // Yh^T = (V - K S)^T, until U and dc are formed
    float KT[D][LC];  // then K^T
  };
  float QT[D][LC];  // Q^T
  float Uf[C][LD];  // U = T D Yh
  float dM[C][LC];  // lower-incl-diag(dO U^T)
  float E[C][LC];   // strictly-lower(-G U^T)
  float al[C], dc[C];
};

template <typename CT, int D, int C>
__global__ __launch_bounds__(512) void efla_bwd_grad_kernel(BwdArgs a) {
  using Sm = GradSmem<D, C>;
  __shared__ __attribute__((aligned(16))) Sm sm;
  constexpr int NKT = D / 16, NB = C / 16, NWV = 8;  // waves
  constexpr bool BF = sizeof(CT) == 2;
  const int tid = threadIdx.x, lane = tid & 63, li = lane & 15, g = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = blockIdx.x / a.nc, ch = blockIdx.x % a.nc;
  const int t0 = ch * C, nval = min(C, a.T - t0);
  const size_t mb = ((size_t)h * a.nc + ch) * C * C;
  const size_t rb = (size_t)h * a.nc * C + t0;
  const float* St = a.sc + ((size_t)h * a.nc + ch) * D * D;   // [v][k]
  const float* Sn = a.scn + ((size_t)h * a.nc + ch) * D * D;  // [k][v]
  const float* dS = a.dsc + ((size_t)h * a.nc + ch) * D * D;  // [k][v]
  const bf16* Stb = (const bf16*)a.sc + ((size_t)h * a.nc + ch) * D * D;   // bf16 form
  const bf16* dSb = (const bf16*)a.dsc + ((size_t)h * a.nc + ch) * D * D;  // bf16 form
  const float* G = a.gw + rb * D;                             // [row][v]
  const CT* kg = (const CT*)a.k + ((size_t)h * a.T + t0) * D;
  const CT* qg = (const CT*)a.q + ((size_t)h * a.T + t0) * D;
  const CT* vg = (const CT*)a.v + ((size_t)h * a.T + t0) * D;
  const CT* dog = (const CT*)a.dout + ((size_t)h * a.T + t0) * D;
  // four consecutive row entries of an input, zero past T
  auto row4 = [&](const CT* base, int r, int c) -> floatx4 {
    return r < nval ? ld4(base + (size_t)r * D + c) : floatx4{0.f, 0.f, 0.f, 0.f};
  };
  // X^T of a C x D input into LDS (zero rows past T). Consecutive lanes take
  // consecutive rows of X, so each transposed write of a wave covers
  // consecutive words of one row of X^T (a lane per row of X would put a
  // wave's writes on a few LDS banks).
  auto stage_t = [&](float (*XT)[Sm::LC], const CT* base) {
    for (int i = tid; i < C * D / 4; i += 64 * NWV) {
      const int r = i % C, c4 = 4 * (i / C);
      const floatx4 x = row4(base, r, c4);
#pragma unroll
      for (int e = 0; e < 4; ++e) XT[c4 + e][r] = x[e];
    }
  };
  if (tid < C) sm.al[tid] = a.al[rb + tid];
  stage_t(sm.QT, qg);
  // K rows in the space U takes later (read by every Yh tile)
  for (int i = tid; i < C * D / 4; i += 64 * NWV) {
    const int r = i / (D / 4), c4 = 4 * (i % (D / 4));
    *(floatx4*)&sm.Uf[r][c4] = row4(kg, r, c4);
  }
  __syncthreads();
  const floatx4 z = {0.f, 0.f, 0.f, 0.f};
  // Yh^T tiles (v, i) = V[i][v] - sum_k S[k][v] K[i][k]: A(v, k) = S[k][v], a
  // row of S^T; B(k, i) = K[i][k], a row of K
  // with bf16 products each wave keeps one v tile I (NWV is a multiple of
  // NKT) and forms its S^T fragments once
  constexpr bool BFK = BF && D % 32 == 0 && C % 32 == 0;
  bf16x8 stf[BFK ? D / 32 : 1];
  if constexpr (BFK) bf_frags<D>(stf, [&](int k0) { return -ld4(&Stb[(size_t)(16 * (w % NKT) + li) * D + k0]); });
  for (int tl = w; tl < NKT * NB; tl += NWV) {
    const int I = tl % NKT, J = tl / NKT;  // I: v tile, J: row tile
    floatx4 acc;
    if constexpr (BFK) {
      acc = mm_fa<D>(z, stf, [&](int k0) { return *(const floatx4*)&sm.Uf[16 * J + li][k0]; });
    } else {
      acc = mmk<D, BF>(z, [&](int k0) { return -ld4(&St[(size_t)(16 * I + li) * D + k0]); },
                       [&](int k0) { return *(const floatx4*)&sm.Uf[16 * J + li][k0]; });
    }
    const floatx4 vv = row4(vg, 16 * J + li, 16 * I + 4 * g);  // V[row][v], v = 16 I + 4 g + e
#pragma unroll
    for (int e = 0; e < 4; ++e) sm.YT[16 * I + 4 * g + e][16 * J + li] = acc[e] + vv[e];
  }
  __syncthreads();
  // U = (T D) Yh: A(i, j) = T[i][j] c_j; B(j, v) = Yh[j][v], a row of Yh^T
  const float* Tn = a.tn + mb;
  // with bf16 products each wave keeps one row tile I (NWV is a multiple of
  // NB) and forms its T D fragments once
  bf16x8 tdf[BFK ? C / 32 : 1];
  if constexpr (BFK)
    bf_frags<C>(tdf, [&](int k0) {
      return ld4(&Tn[(size_t)(16 * (w % NB) + li) * C + k0]) * *(const floatx4*)&sm.al[k0];
    });
  for (int tl = w; tl < NB * NKT; tl += NWV) {
    const int I = tl % NB, J = tl / NB;  // I: row tile, J: v tile
    floatx4 acc;
    if constexpr (BFK) {
      acc = mm_fa<C>(z, tdf, [&](int k0) { return *(const floatx4*)&sm.YT[16 * J + li][k0]; });
    } else {
      acc = mmk<C, BF>(z,
                       [&](int k0) {
                         return ld4(&Tn[(size_t)(16 * I + li) * C + k0]) * *(const floatx4*)&sm.al[k0];
                       },
                       [&](int k0) { return *(const floatx4*)&sm.YT[16 * J + li][k0]; });
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) sm.Uf[16 * I + 4 * g + e][16 * J + li] = acc[e];
  }
  __syncthreads();
  // dM = lower-incl-diag(dO U^T), E = strictly-lower(-G U^T): k = v;
  // B(v, j) = U[j][v], a row of U
  // with bf16 products each wave keeps one row tile I and forms its dO and G
  // fragments once
  bf16x8 dof[BFK ? D / 32 : 1], gf[BFK ? D / 32 : 1];
  if constexpr (BFK) {
    bf_frags<D>(dof, [&](int k0) { return row4(dog, 16 * (w % NB) + li, k0); });
    bf_frags<D>(gf, [&](int k0) { return -ld4(&G[(size_t)(16 * (w % NB) + li) * D + k0]); });
  }
  for (int tl = w; tl < NB * NB; tl += NWV) {
    const int I = tl % NB, J = tl / NB;
    floatx4 m, e4;
    if constexpr (BFK) {
      m = mm_fa<D>(z, dof, [&](int k0) { return *(const floatx4*)&sm.Uf[16 * J + li][k0]; });
      e4 = mm_fa<D>(z, gf, [&](int k0) { return *(const floatx4*)&sm.Uf[16 * J + li][k0]; });
    } else {
      m = mmk<D, BF>(z, [&](int k0) { return row4(dog, 16 * I + li, k0); },
                     [&](int k0) { return *(const floatx4*)&sm.Uf[16 * J + li][k0]; });
      e4 = mmk<D, BF>(z, [&](int k0) { return -ld4(&G[(size_t)(16 * I + li) * D + k0]); },
                      [&](int k0) { return *(const floatx4*)&sm.Uf[16 * J + li][k0]; });
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 16 * I + 4 * g + e, j = 16 * J + li;
      sm.dM[i][j] = j <= i ? m[e] : 0.f;
      sm.E[i][j] = j < i ? e4[e] : 0.f;
    }
  }
  __syncthreads();
  // dc = rowsum(G * Yh) + rowsum(E * K K^T): four lanes per row
  {
    const int i = tid >> 2, part = tid & 3;
    float s = 0.f;
    if (i < C) {
      for (int v = part; v < D; v += 4) s = fmaf(G[(size_t)i * D + v], sm.YT[v][i], s);
      const float* gr = a.gram + mb + (size_t)i * C;
      for (int j = part; j < i; j += 4) s = fmaf(sm.E[i][j], gr[j], s);
    }
    s = group_sum<4>(s);
    if (i < C && part == 0) {
      sm.dc[i] = s;
      if (i < nval) ((CT*)a.dbeta)[(size_t)h * a.T + t0 + i] = from_f32<CT>(s * a.fb[rb + i]);
    }
  }
  __syncthreads();  // Yh^T is dead: its space takes K^T
  stage_t(sm.KT, kg);
  __syncthreads();
  // dQ and dK tiles (row tile I, key tile J)
  CT* dqg = (CT*)a.dq + ((size_t)h * a.T + t0) * D;
  CT* dkg = (CT*)a.dk + ((size_t)h * a.T + t0) * D;
  // with bf16 products each wave keeps one key tile J and forms the
  // fragments of its rows of S, dS', K^T and Q^T once
  bf16x8 snf[BFK ? D / 32 : 1], dsf[BFK ? D / 32 : 1], ktf[BFK ? C / 32 : 1], qtf[BFK ? C / 32 : 1];
  if constexpr (BFK) {
    const int cj = 16 * (w % NKT) + li;
    // row cj of S from the transposed copy (once per wave: the natural copy is
    // not written for this form)
    bf_frags<D>(snf, [&](int k0) {
      floatx4 x;
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = ld1(&Stb[(size_t)(k0 + e) * D + cj]);
      return x;
    });
    bf_frags<D>(dsf, [&](int k0) { return ld4(&dSb[(size_t)cj * D + k0]); });
    bf_frags<C>(ktf, [&](int k0) { return *(const floatx4*)&sm.KT[cj][k0]; });
    bf_frags<C>(qtf, [&](int k0) { return *(const floatx4*)&sm.QT[cj][k0]; });
  }
  // K^T and Q^T now live in registers: their LDS takes the rows of dO and G
  // (when C x (d + 4) fits in d x (C + 4), i.e. d >= C)
  constexpr bool STAGE = BFK && D >= C;
  float(*dOs)[D + 4] = reinterpret_cast<float(*)[D + 4]>(&sm.KT[0][0]);
  float(*Gs)[D + 4] = reinterpret_cast<float(*)[D + 4]>(&sm.QT[0][0]);
  if constexpr (STAGE) {
    __syncthreads();
    for (int i = tid; i < C * D / 4; i += 64 * NWV) {
      const int r = i / (D / 4), c4 = 4 * (i % (D / 4));
      *(floatx4*)&dOs[r][c4] = row4(dog, r, c4);
      *(floatx4*)&Gs[r][c4] = ld4(&G[(size_t)r * D + c4]);
    }
    __syncthreads();
  }
  for (int tl = w; tl < NB * NKT; tl += NWV) {
    const int J = tl % NKT, I = tl / NKT;
    const int ci = 16 * J + li;  // key dimension of this lane's column
    if constexpr (BFK) {
      const float cr = sm.al[16 * I + li];
      floatx4 dq = mm_fb<D>(z,
                            [&](int k0) {
                              if constexpr (STAGE) return *(const floatx4*)&dOs[16 * I + li][k0];
                              else return row4(dog, 16 * I + li, k0);
                            },
                            snf);
      dq = mm_fb<C>(dq, [&](int k0) { return *(const floatx4*)&sm.dM[16 * I + li][k0]; }, ktf);
      floatx4 dk = mm_fb<C>(z,
                            [&](int k0) {
                              floatx4 x;
#pragma unroll
                              for (int e = 0; e < 4; ++e) x[e] = sm.dM[k0 + e][16 * I + li];
                              return x;
                            },
                            qtf);
      dk = mm_fb<D>(dk, [&](int k0) { return *(const floatx4*)&sm.Uf[16 * I + li][k0]; }, dsf);
      dk = mm_fb<D>(dk,
                    [&](int k0) {
                      if constexpr (STAGE) return -cr * *(const floatx4*)&Gs[16 * I + li][k0];
                      else return -cr * ld4(&G[(size_t)(16 * I + li) * D + k0]);
                    },
                    snf);
      dk = mm_fb<C>(dk,
                    [&](int k0) {
                      floatx4 x;
#pragma unroll
                      for (int e = 0; e < 4; ++e) {
                        const int j = k0 + e;
                        x[e] = cr * sm.E[16 * I + li][j] + sm.E[j][16 * I + li] * sm.al[j];
                      }
                      return x;
                    },
                    ktf);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * I + 4 * g + e;
        if (r < nval) {
          const float kv = STAGE ? ld1(kg + (size_t)r * D + ci) : sm.KT[ci][r];
          dqg[(size_t)r * D + ci] = from_f32<CT>(dq[e]);
          dkg[(size_t)r * D + ci] = from_f32<CT>(dk[e] + 2.f * sm.dc[r] * a.fl[rb + r] * kv);
        }
      }
      continue;
    }
    // dQ = dO S^T + dM K: B(v, k) = S[k][v], a row of S; B(j, k) = K[j][k], a row of K^T
    floatx4 dq = mmk<D, BF>(z, [&](int k0) { return row4(dog, 16 * I + li, k0); },
                      [&](int k0) { return ld4(&Sn[(size_t)ci * D + k0]); });
    dq = mmk<C, BF>(dq, [&](int k0) { return *(const floatx4*)&sm.dM[16 * I + li][k0]; },
              [&](int k0) { return *(const floatx4*)&sm.KT[ci][k0]; });
    // dK = dM^T Q + U dS'^T - D G S^T + D E K + E^T D K
    floatx4 dk = mmk<C, BF>(z,
                      [&](int k0) {
                        floatx4 x;
#pragma unroll
                        for (int e = 0; e < 4; ++e) x[e] = sm.dM[k0 + e][16 * I + li];
                        return x;
                      },
                      [&](int k0) { return *(const floatx4*)&sm.QT[ci][k0]; });
    dk = mmk<D, BF>(dk, [&](int k0) { return *(const floatx4*)&sm.Uf[16 * I + li][k0]; },
              [&](int k0) { return ld4(&dS[(size_t)ci * D + k0]); });
    {
      const float cr = sm.al[16 * I + li];  // row scale of this lane's A row
      dk = mmk<D, BF>(dk, [&](int k0) { return -cr * ld4(&G[(size_t)(16 * I + li) * D + k0]); },
                [&](int k0) { return ld4(&Sn[(size_t)ci * D + k0]); });
      dk = mmk<C, BF>(dk,
                [&](int k0) {
                  floatx4 x;
#pragma unroll
                  for (int e = 0; e < 4; ++e) {
                    const int j = k0 + e;
                    x[e] = cr * sm.E[16 * I + li][j] + sm.E[j][16 * I + li] * sm.al[j];
                  }
                  return x;
                },
                [&](int k0) { return *(const floatx4*)&sm.KT[ci][k0]; });
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 16 * I + 4 * g + e;
      if (r < nval) {
        const float kv = sm.KT[ci][r];
        dqg[(size_t)r * D + ci] = from_f32<CT>(dq[e]);
        dkg[(size_t)r * D + ci] = from_f32<CT>(dk[e] + 2.f * sm.dc[r] * a.fl[rb + r] * kv);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// 4, bf16 form (bf16 inputs, C and d multiples of 32). Every tile the products
// share sits in LDS as bf16 with column-permuted rows (the forward kernel's
// layout): a fragment along a row is one 16-byte read and a fragment along a
// column a pair of ds_read_b64_tr_b16. Each product is formed in the
// orientation whose accumulator holds 4 consecutive columns of one row of the
// tile it is stored to (8-byte writes). dc is summed from the fp32
// accumulators of Yh and E as they are formed. Every global read is 8 or 16
// bytes per lane: the state is staged whole and its columns are read from LDS
// (with 2-byte column reads from global memory instead, the kernel took
// 1.5x as long). With X = D E:
//   Yh tiles    = V - (S^T K^T)^T     A = rows of S^T (as stored), B = rows of K
//   U^T tiles   = Yh^T (T D)^T        A = columns of Yh, B = rows of T D
//   dM, E       from U dO^T, -U G^T   A = rows of U, B = rows of dO, G
//   dQ = dO S^T + dM K
//   dK = dM^T Q + U dS'^T - D (G S^T) + X K + X^T K
template <int D, int C>
struct GradSmemBf {
  static constexpr int LD = D + 16, LC = C + 16;  // row strides: 32 bytes mod 64
  bf16 Kb[C][LD];
  bf16 Qb[C][LD];
  bf16 dOb[C][LD];
  bf16 Gb[C][LD];
  bf16 Ub[C][LD];  // U = T D Yh
  bf16 Sb[D][LD];  // the chunk-start state as stored, [v][k]
  union {
    bf16 Yb[C][LD];  // Yh, until U is formed
    struct {
      bf16 dMb[C][LC];  // lower-incl-diag(dO U^T)
      bf16 Xb[C][LC];   // D E
    } m;
  };
  float al[C], dc[C], fl[C];
  float dcp[C][D / 16 + 1];   // rowsum(G * Yh) over one 16-column tile of v
  float dcp2[C][C / 16 + 1];  // rowsum(E * K K^T) over one 16-column tile
};

template <int D, int C>
__global__ __launch_bounds__(512) void efla_bwd_grad_kernel_bf(BwdArgs a) {
  using Sm = GradSmemBf<D, C>;
  using MM = Mma<bf16>;
  static_assert(D % 32 == 0 && C % 32 == 0, "bf16 form");
  static_assert((Sm::LD * 2) % 64 == 32 && (Sm::LC * 2) % 64 == 32, "row strides");
  __shared__ __attribute__((aligned(16))) Sm sm;
  constexpr int NKT = D / 16, NB = C / 16, NWV = 8, KD = D / 32, KC = C / 32;
  // lane indices: passed through an empty asm at every item (step below),
  // so the addresses formed from them are recomputed per item rather than
  // held in registers across the whole loop
  int tid = threadIdx.x, lane = tid & 63, li = lane & 15, g = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const floatx4 z = {0.f, 0.f, 0.f, 0.f};
  auto mma = [](bf16x8 x, bf16x8 y, floatx4 c) { return __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, y, c, 0, 0, 0); };

  static_assert(NKT <= NWV, "one v tile per wave in the Yh and dQ/dK phases");
  // The workgroups are persistent: each takes the (head, chunk) items
  // blockIdx.x, blockIdx.x + gridDim.x, ... and requests the operands that
  // open its next item (K rows, the state, V and G at (token, v), the
  // scalars) during the current one, right after its Yh phase, so their
  // latency overlaps most of an item's products (one workgroup fills a CU's
  // LDS, so no second workgroup could). The rest of an item's operands are requested when the
  // item starts: its first phases run while they arrive. (Holding all of
  // the next item's operands would take more registers than a wave has.)
  //
  // The operands of an item are requested in the order its phases first need
  // them, and each is staged or used only where that phase starts:
  // Yh phase: K rows, the chunk-start state (staged whole: its columns are
  // read from LDS, transposed, where a fragment runs along v), V and G at
  // (token 16 J + li, v 16 w + 4g .. + 3); U^T phase (token tile w % NB): row
  // 16 I2 + li of T D; dM/E phase: dO and G rows; dQ/dK phase (key tile w): Q
  // rows and rows of dS'.
  // No load sits behind a branch: rows past T are read clamped to the last
  // row and zeroed where they are used, and the last round requests its own
  // item again instead of none, so every wave issues the same loads and each
  // wait counts exactly the loads it needs.
  constexpr int NIT = (C * D / 8 + 64 * NWV - 1) / (64 * NWV);
  constexpr int NIS = (D * D / 8 + 64 * NWV - 1) / (64 * NWV);
  // when the threads cover a tile exactly, its staging has no bounds test
  // (the compiler would otherwise move the guarded row loads behind it)
  constexpr bool EXR = NIT * 64 * NWV == C * D / 8, EXS = NIS * 64 * NWV == D * D / 8;
  constexpr int JS = NWV / NB, NJ3 = (NB + JS - 1) / JS;
  const bool vt = w < NKT;
  const int I1 = w, I2 = w % NB;
  int vw = 16 * (w % NKT) + 4 * g;  // v columns of this lane in the Yh phase
  int tc = min(tid, C - 1);
  struct Ops {  // requested one item ahead
    bf16x8 kx[NIT], sx[NIS];
    bf16x4 vq[NB], gq[NB];
    float alt, flt, fbt;
  };
  struct Late {  // requested when the item starts
    bf16x8 qx[NIT], ox[NIT], gx[NIT], dsf[KD], tdf[KC];
  };
  auto item_rows = [&](int item, auto f) {
    const int h = item / a.nc, ch = item % a.nc;
    const int t0 = ch * C, rlast = min(C, a.T - t0) - 1;
    auto load_rows = [&](bf16x8* x, const bf16* src) {
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
        const int i = min(tid + 64 * NWV * it, C * D / 8 - 1), r = i / (D / 8), c8 = 8 * (i % (D / 8));
        x[it] = *(const bf16x8*)(src + (size_t)min(r, rlast) * D + c8);
      }
    };
    f(h, ch, t0, rlast, load_rows);
  };
  auto request_late = [&](int item, Late& o) {
    item_rows(item, [&](int h, int ch, int t0, int rlast, auto load_rows) {
      const size_t mb = ((size_t)h * a.nc + ch) * C * C;
      const size_t rb = (size_t)h * a.nc * C + t0;
      const size_t tok = ((size_t)h * a.T + t0) * D;
      const bf16* Tn = (const bf16*)a.tn + mb;  // column-permuted by the prep kernel
#pragma unroll
      for (int kb = 0; kb < KC; ++kb) o.tdf[kb] = *(const bf16x8*)&Tn[(size_t)(16 * I2 + li) * C + 32 * kb + 8 * g];
      load_rows(o.ox, (const bf16*)a.dout + tok);
      load_rows(o.gx, (const bf16*)a.gw + rb * D);
      load_rows(o.qx, (const bf16*)a.q + tok);
      const bf16* dS = (const bf16*)a.dsc + ((size_t)h * a.nc + ch) * D * D;  // [k][v]
      const int cj = 16 * (w % NKT) + li;
      bf_frags<D>(o.dsf, [&](int k0) { return ld4(&dS[(size_t)cj * D + k0]); });
    });
  };
  auto request = [&](int item, Ops& o) {
    item_rows(item, [&](int h, int ch, int t0, int rlast, auto load_rows) {
      const size_t rb = (size_t)h * a.nc * C + t0;
      const bf16* St = (const bf16*)a.sc + ((size_t)h * a.nc + ch) * D * D;  // [v][k]
      const size_t tok = ((size_t)h * a.T + t0) * D;
      load_rows(o.kx, (const bf16*)a.k + tok);
#pragma unroll
      for (int it = 0; it < NIS; ++it)
        o.sx[it] = *(const bf16x8*)(St + (size_t)8 * min(tid + 64 * NWV * it, D * D / 8 - 1));
      o.alt = a.al[rb + tc];
      o.flt = a.fl[rb + tc];
      o.fbt = a.fb[rb + tc];
#pragma unroll
      for (int J = 0; J < NB; ++J) {
        const size_t r = (size_t)min(16 * J + li, rlast) * D + vw;
        o.vq[J] = *(const bf16x4*)((const bf16*)a.v + tok + r);
        o.gq[J] = *(const bf16x4*)((const bf16*)a.gw + rb * D + r);
      }
    });
  };
  auto process = [&](int item, const Ops& o, const Late& l, auto after_yh) {
    const int h = item / a.nc, ch = item % a.nc;
    const int t0 = ch * C, nval = min(C, a.T - t0);
    const auto& vq = o.vq;
    const auto& gq = o.gq;
    const auto& tdf = l.tdf;
    const auto& dsf = l.dsf;
    const float fbt = o.fbt;
    auto stage_rows = [&](bf16 (*dst)[Sm::LD], const bf16x8* x) {
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
        const int i = tid + 64 * NWV * it, r = i / (D / 8);
        if (EXR || i < C * D / 8) st_perm(&dst[r][0], 8 * (i % (D / 8)), r < nval ? x[it] : bf16x8{});
      }
    };
    const auto& ox = l.ox;
    const auto& gx = l.gx;
    const auto& qx = l.qx;
    stage_rows(sm.Kb, o.kx);
#pragma unroll
    for (int it = 0; it < NIS; ++it) {
      const int i = tid + 64 * NWV * it;
      if (EXS || i < D * D / 8) st_perm(&sm.Sb[i / (D / 8)][0], 8 * (i % (D / 8)), o.sx[it]);
    }
    // every thread stores (those past C repeat row C - 1 with its own
    // values): behind a tid < C test the compiler would move these loads
    // after the rest
    sm.al[tc] = o.alt;
    sm.fl[tc] = o.flt;
    __syncthreads();

    // ---- Yh tiles (token tile J, v tile I), formed transposed (S as the
    //      first operand): acc[e] = (K S)[16 J + li][16 I + 4g + e], so a lane
    //      holds 4 consecutive v of one token; Yh = V - K S, rowsum(G * Yh)
    //      over the tile's 16 v, stored as rows of Yh
    if (vt) {
      const int I = I1;
      bf16x8 stf[KD];
#pragma unroll
      for (int kb = 0; kb < KD; ++kb) stf[kb] = MM::template ldp<NKT>(&sm.Sb[16 * I + li][0], kb);
#pragma unroll
      for (int J = 0; J < NB; ++J) {
        floatx4 acc = z;
#pragma unroll
        for (int kb = 0; kb < KD; ++kb) acc = mma(stf[kb], MM::template ldp<NKT>(&sm.Kb[16 * J + li][0], kb), acc);
        const bool ok = 16 * J + li < nval;
        acc = (ok ? __builtin_convertvector(vq[J], floatx4) : z) - acc;
        const floatx4 gg = ok ? __builtin_convertvector(gq[J], floatx4) : z;
        float p = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) p += gg[e] * acc[e];
        p = xor32_sum(xor16_sum(p));
        if (g == 0) sm.dcp[16 * J + li][I] = p;
        MM::store_tp(&sm.Yb[16 * J + li][0], I, acc);
      }
    }
    __syncthreads();
    after_yh();  // this item's opening registers are free now

    // ---- U^T tiles (token tile I, v tile J): acc[e] = U[16 I + li][16 J + 4g + e];
    //      B(j, i) = T[i][j] c_j, row i of T D (read once per wave)
    {
      const int I = I2;
      for (int J = w / NB; J < NKT; J += NWV / NB) {
        floatx4 acc = z;
#pragma unroll
        for (int kb = 0; kb < KC; ++kb) acc = mma(tr_frag<NB, true>(&sm.Yb[0][0], Sm::LD, kb, 16 * J), tdf[kb], acc);
        MM::store_tp(&sm.Ub[16 * I + li][0], J, acc);
      }
    }
    stage_rows(sm.dOb, ox);
    stage_rows(sm.Gb, gx);
    __syncthreads();

    // ---- dM and E tiles (token tiles I >= J; the others are zero): acc[e] =
    //      (dO U^T)[16 I + li][16 J + 4g + e], and the same with -G; X = D E;
    //      rowsum(E * K K^T) over the tile's 16 columns, with the K K^T tile
    //      formed here in the same orientation
    {
      const int I = I2;
      const float ci = sm.al[16 * I + li];
      bf16x8 dof[KD], gf[KD];
#pragma unroll
      for (int kb = 0; kb < KD; ++kb) {
        dof[kb] = MM::template ldp<NKT>(&sm.dOb[16 * I + li][0], kb);
        gf[kb] = MM::template ldp<NKT>(&sm.Gb[16 * I + li][0], kb);
      }
#pragma unroll
      for (int jm = 0; jm < NJ3; ++jm) {
        const int J = w / NB + JS * jm;
        if (J >= NB) break;
        floatx4 m = z, e4 = z;
        float s = 0.f;
        if (J <= I) {
#pragma unroll
          for (int kb = 0; kb < KD; ++kb) {
            const bf16x8 u = MM::template ldp<NKT>(&sm.Ub[16 * J + li][0], kb);
            m = mma(u, dof[kb], m);
            e4 = mma(u, gf[kb], e4);
          }
          floatx4 gr = z;
#pragma unroll
          for (int kb = 0; kb < KD; ++kb)
            gr = mma(MM::template ldp<NKT>(&sm.Kb[16 * J + li][0], kb), MM::template ldp<NKT>(&sm.Kb[16 * I + li][0], kb), gr);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = 16 * I + li, j = 16 * J + 4 * g + e;
            m[e] = j <= i ? m[e] : 0.f;
            e4[e] = j < i ? -e4[e] : 0.f;
            s += e4[e] * gr[e];
            e4[e] *= ci;
          }
        }
        s = xor32_sum(xor16_sum(s));
        if (g == 0) sm.dcp2[16 * I + li][J] = s;
        MM::store_tp(&sm.m.dMb[16 * I + li][0], J, m);
        MM::store_tp(&sm.m.Xb[16 * I + li][0], J, e4);
      }
    }
    __syncthreads();

    // ---- dc, dbeta
    if (tid < C) {
      float s = 0.f;
#pragma unroll
      for (int I = 0; I < NKT; ++I) s += sm.dcp[tid][I];
#pragma unroll
      for (int J = 0; J < NB; ++J) s += sm.dcp2[tid][J];
      sm.dc[tid] = s;
      if (tid < nval) ((bf16*)a.dbeta)[(size_t)h * a.T + t0 + tid] = (bf16)(s * fbt);
    }
    stage_rows(sm.Qb, qx);
    __syncthreads();

    // ---- dQ and dK tiles (token tile I, key tile J): acc[e] at row 16 I + 4g + e,
    //      column 16 J + li; wave w takes key tile J and forms the fragments of
    //      row J of S, dS' (over v) and of columns J of K, Q (over tokens) once
    bf16* dqg = (bf16*)a.dq + ((size_t)h * a.T + t0) * D;
    bf16* dkg = (bf16*)a.dk + ((size_t)h * a.T + t0) * D;
    if (vt) {
      const int J = I1;
      bf16x8 ktf[KC], qtf[KC], snf[KD];
#pragma unroll
      for (int kb = 0; kb < KC; ++kb) {
        ktf[kb] = tr_frag<NB, true>(&sm.Kb[0][0], Sm::LD, kb, 16 * J);
        qtf[kb] = tr_frag<NB, true>(&sm.Qb[0][0], Sm::LD, kb, 16 * J);
      }
      // row J of S over v: column 16 J + li of the stored [v][k] tile
#pragma unroll
      for (int kb = 0; kb < KD; ++kb) snf[kb] = tr_frag<NKT, true>(&sm.Sb[0][0], Sm::LD, kb, 16 * J);
      // the products are formed transposed (operands swapped): lane (g, li)
      // holds token 16 I + li, keys 16 J + 4g .. + 3, stored as 8 bytes
      for (int I = 0; I < NB; ++I) {
        floatx4 dq = z, dk = z, dg = z;
#pragma unroll
        for (int kb = 0; kb < KD; ++kb) {
          dq = mma(snf[kb], MM::template ldp<NKT>(&sm.dOb[16 * I + li][0], kb), dq);
          dk = mma(dsf[kb], MM::template ldp<NKT>(&sm.Ub[16 * I + li][0], kb), dk);
          dg = mma(snf[kb], MM::template ldp<NKT>(&sm.Gb[16 * I + li][0], kb), dg);
        }
#pragma unroll
        for (int kb = 0; kb < KC; ++kb) {
          dq = mma(ktf[kb], MM::template ldp<NB>(&sm.m.dMb[16 * I + li][0], kb), dq);
          dk = mma(qtf[kb], tr_frag<NB, true>(&sm.m.dMb[0][0], Sm::LC, kb, 16 * I), dk);
          dk = mma(ktf[kb], MM::template ldp<NB>(&sm.m.Xb[16 * I + li][0], kb), dk);
          dk = mma(ktf[kb], tr_frag<NB, true>(&sm.m.Xb[0][0], Sm::LC, kb, 16 * I), dk);
        }
        const int r = 16 * I + li, k4 = 16 * J + 4 * g;
        if (r < nval) {
          // pcol keeps 4-aligned runs of 4 columns together
          const floatx4 kv = __builtin_convertvector(*(const bf16x4*)&sm.Kb[r][MM::pcol(k4)], floatx4);
          const float ar = sm.al[r], fr = 2.f * sm.dc[r] * sm.fl[r];
          floatx4 dkr;
#pragma unroll
          for (int e = 0; e < 4; ++e) dkr[e] = dk[e] - ar * dg[e] + fr * kv[e];
          *(bf16x4*)&dqg[(size_t)r * D + k4] = cv4(dq);
          *(bf16x4*)&dkg[(size_t)r * D + k4] = cv4(dkr);
        }
      }
    }
  };
  const int nitems = a.nh * a.nc;
  int item = blockIdx.x;  // the grid holds at most nitems workgroups
  // one item: its late operands, its products, and after its Yh phase (when
  // its own opening registers are dead) the next item's opening operands;
  // false after the last item. Two register sets alternate (the loop body
  // takes two items), so nothing is copied and no wait covers this item's
  // stores
  auto step = [&](const Ops& cur, Ops& nx) {
    asm volatile("" : "+v"(tid), "+v"(lane), "+v"(li), "+v"(g), "+v"(vw), "+v"(tc));
    const int nxt = item + (int)gridDim.x;
    Late late;
    request_late(item, late);
    process(item, cur, late, [&] { request(nxt < nitems ? nxt : item, nx); });
    if (nxt >= nitems) return false;
    __syncthreads();  // the LDS reads of this item are done before the next staging
    item = nxt;
    return true;
  };
  Ops A, B;
  request(item, A);
  while (step(A, B) && step(B, A)) {
  }
  // the last round's requests (its own item again) are drained before the
  // waves end
  __builtin_amdgcn_s_waitcnt(0);
}

// Compute units of the current device (the persistent gradient kernel runs
// one workgroup per CU), cached per device.
static int device_cus() {
  static int cus[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] <= 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

// ---------------------------------------------------------------------------
template <typename CT, int D, int C>
static hipError_t launch_bwd(const BwdArgs& a, int NH, hipStream_t stream) {
  constexpr int BV = D < 64 ? D : 64;
  hipLaunchKernelGGL((efla_bwd_prep_kernel<CT, D, C>), dim3((unsigned)(NH * a.nc)), dim3(256), 0, stream, a);
  if constexpr (sizeof(CT) == 2 && C % 32 == 0 && D % 32 == 0) {
    if constexpr (2 * sizeof(StateSmemBf<D, C, BV>) <= 160 * 1024) {
      hipLaunchKernelGGL((efla_bwd_state_kernel_bfp<D, C, BV>), dim3((unsigned)(NH * (D / BV))), dim3(512), 0,
                         stream, a);
    } else {
      hipLaunchKernelGGL((efla_bwd_state_kernel_bf<D, C, BV>), dim3((unsigned)(NH * (D / BV))), dim3(256), 0,
                         stream, a);
    }
  } else {
    hipLaunchKernelGGL((efla_bwd_state_kernel<CT, D, C, BV>), dim3((unsigned)(NH * (D / BV))), dim3(256), 0,
                       stream, a);
  }
  if constexpr (sizeof(CT) == 2 && C % 32 == 0 && D % 32 == 0) {
    const int items = NH * a.nc;
    hipLaunchKernelGGL((efla_bwd_grad_kernel_bf<D, C>), dim3((unsigned)min(items, device_cus())), dim3(512), 0, stream, a);
  } else {
    hipLaunchKernelGGL((efla_bwd_grad_kernel<CT, D, C>), dim3((unsigned)(NH * a.nc)), dim3(512), 0, stream, a);
  }
  return hipGetLastError();
}

template <typename CT, int D>
static hipError_t bwd_chunk(const BwdArgs& a, int NH, int chunk, hipStream_t s) {
  switch (chunk) {
    case 16: return launch_bwd<CT, D, 16>(a, NH, s);
    case 32: return launch_bwd<CT, D, 32>(a, NH, s);
    case 64: return launch_bwd<CT, D, 64>(a, NH, s);
    default: return hipErrorInvalidValue;
  }
}

template <typename CT>
static hipError_t bwd_d(const BwdArgs& a, int NH, int d, int chunk, hipStream_t s) {
  switch (d) {
    case 16: return bwd_chunk<CT, 16>(a, NH, chunk, s);
    case 32: return bwd_chunk<CT, 32>(a, NH, chunk, s);
    case 64: return bwd_chunk<CT, 64>(a, NH, chunk, s);
    case 128: return bwd_chunk<CT, 128>(a, NH, chunk, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace efla

hipError_t efla_internal_launch_states(const void* q, const void* k, const void* v, const void* beta,
                                       const float* s0, void* o, float* s_final, float* s_chunks,
                                       float* s_chunks_n, int NH, int T, int d, int chunk, int coef, int is_bf16,
                                       hipStream_t stream);
hipError_t efla_internal_launch_chunked(const void* q, const void* k, const void* v, const void* beta,
                                        const float* s0, void* o, float* s_final, void* workspace, int NH, int T,
                                        int d, int chunk, int coef, int is_bf16, hipStream_t stream);
bool efla_internal_states_supported(int d, int chunk, int is_bf16);

// Chunk size the backward runs with for a requested forward chunk.
static int bwd_chunk_for(int d, int chunk, int is_bf16) {
  int c = chunk;
  if (!efla_internal_states_supported(d, c, is_bf16)) c = 32;
  if (!efla_internal_states_supported(d, c, is_bf16)) return 0;
  return c;
}

size_t efla_internal_bwd_workspace_bytes(int NH, int T, int d, int chunk, int is_bf16) {
  const int c = bwd_chunk_for(d, chunk, is_bf16);
  if (c == 0) return 0;
  const size_t nc = (size_t)((T + c - 1) / c), Tp = nc * c;
  const size_t per_head = 3 * nc * d * d + Tp * d + 3 * Tp + 4 * nc * c * c;
  return (size_t)NH * per_head * sizeof(float);
}

// The backward's workspace starts with the chunk-start states: [head][chunk]
// [d_v][d_k] (bf16 in the bf16 form of the gradient kernel, else fp32), then,
// where the fp32 form needs them, the same states as [head][chunk][d_k][d_v].
static bool bwd_needs_kv_states(int d, int c, int is_bf16) { return !(is_bf16 && c % 32 == 0 && d % 32 == 0); }

// Forward of a training step: o and s_final as the plain forward, plus the
// chunk-start states in the backward's workspace. Where the pipelined kernel
// serves the requested chunk one pass writes all of it; otherwise the states
// pass (at the backward's chunk) runs first and the forward after it, so that
// s_final may alias s0 in both cases.
hipError_t efla_internal_launch_fwd_save(const void* q, const void* k, const void* v, const void* beta,
                                         const float* s0, void* o, float* s_final, void* workspace, int NH, int T,
                                         int d, int chunk, int coef, int is_bf16, hipStream_t stream) {
  const int c = bwd_chunk_for(d, chunk, is_bf16);
  if (c == 0) return hipErrorInvalidValue;
  const size_t nc = (size_t)((T + c - 1) / c);
  float* sc = (float*)workspace;
  float* scn = bwd_needs_kv_states(d, c, is_bf16) ? sc + (size_t)NH * nc * d * d : nullptr;
  if (c == chunk)
    return efla_internal_launch_states(q, k, v, beta, s0, o, s_final, sc, scn, NH, T, d, c, coef, is_bf16, stream);
  const hipError_t e =
      efla_internal_launch_states(q, k, v, beta, s0, nullptr, nullptr, sc, scn, NH, T, d, c, coef, is_bf16, stream);
  if (e != hipSuccess) return e;
  return efla_internal_launch_chunked(q, k, v, beta, s0, o, s_final, nullptr, NH, T, d, chunk, coef, is_bf16,
                                      stream);
}

hipError_t efla_internal_launch_bwd(const void* q, const void* k, const void* v, const void* beta,
                                    const float* s0, const void* dout, const float* dsT, void* dq, void* dk,
                                    void* dv, void* dbeta, float* ds0, void* workspace, int NH, int T, int d,
                                    int chunk, int coef, int is_bf16, int states_saved, hipStream_t stream) {
  const int c = bwd_chunk_for(d, chunk, is_bf16);
  if (c == 0) return hipErrorInvalidValue;
  const size_t nc = (size_t)((T + c - 1) / c), Tp = nc * c;
  float* p = (float*)workspace;
  efla::BwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.beta = beta;
  a.dout = dout;
  a.s0 = s0;
  a.dsT = dsT;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dbeta = dbeta;
  a.ds0 = ds0;
  a.T = T;
  a.nc = (int)nc;
  a.nh = NH;
  a.coef = coef;
  float* sc = p;
  p += (size_t)NH * nc * d * d;
  float* scn = p;
  p += (size_t)NH * nc * d * d;
  a.sc = sc;
  a.scn = scn;
  a.dsc = p;
  p += (size_t)NH * nc * d * d;
  a.gw = p;
  p += (size_t)NH * Tp * d;
  a.al = p;
  p += (size_t)NH * Tp;
  a.fb = p;
  p += (size_t)NH * Tp;
  a.fl = p;
  p += (size_t)NH * Tp;
  a.gram = p;
  p += (size_t)NH * nc * c * c;
  a.tn = p;
  p += (size_t)NH * nc * c * c;
  a.tt = p;
  p += (size_t)NH * nc * c * c;
  a.mt = p;
  // the bf16 form of the gradient kernel (C and d multiples of 32) reads the
  // transposed states only
  if (!states_saved) {
    const hipError_t e = efla_internal_launch_states(q, k, v, beta, s0, nullptr, nullptr, sc,
                                                     bwd_needs_kv_states(d, c, is_bf16) ? scn : nullptr, NH, T, d,
                                                     c, coef, is_bf16, stream);
    if (e != hipSuccess) return e;
  }
  return is_bf16 ? efla::bwd_d<efla::bf16>(a, NH, d, c, stream) : efla::bwd_d<float>(a, NH, d, c, stream);
}
