// Chunk-parallel EFLA forward for gfx950 (WY/UT form).
//
// Method: papernotes.org note "Exact Flow Linear Attention: Exact Solution
// from Continuous-Time Dynamics". The update S_t = (I - a_t k_t k_t^T) S_{t-1}
// + a_t k_t v_t^T with a_t the exact-flow coefficient (关键设计 item 2) has the
// same algebraic form as the delta rule, so the chunkwise WY/UT algorithm of
// DeltaNet applies unchanged (整体框架 and 亮点 sections). Per chunk of C tokens
// with start state S:
//   A  = strictly-lower(diag(a) K K^T)          Gram, fp32 accumulate
//   T  = (I + A)^{-1}                           unit lower triangular
//   W  = T diag(a) K,  U = T diag(a) V          WY factors
//   U' = U - W S
//   O  = Q S + lower-incl-diag(Q K^T) U'        read out after each update
//   S <- S + K^T U'
// It reproduces the token-serial recurrence exactly up to rounding.
//
// One workgroup (4 wave64s) owns one (head, BV-column slice of the state)
// and walks the chunks in order; the d_k x BV fp32 state never leaves the
// MFMA accumulator registers of the waves that own its columns (32 columns
// per wave; columns of S evolve independently, so the slice split is exact).
// Chunk tiles are staged in LDS; T is never formed: its 16x16 diagonal blocks
// are inverted by forward substitution in fp32 and W, U come from a blocked
// forward solve whose right-hand sides stay in registers. The next chunk's
// loads are issued before the current chunk's compute.

#include "efla_device.hpp"

// Waves per workgroup that hold the state slice (2: 32 columns each; 4: 16).
#ifndef EFLA_STATE_WAVES
#define EFLA_STATE_WAVES 2
#endif

namespace efla {

struct ChunkedArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* beta;
  const float* s0;
  void* o;
  float* s_final;
  int T;
  int nvt;  // state column slices per head
};

template <typename CT>
struct Vec16;
template <>
struct Vec16<bf16> { typedef bf16x8 type; };
template <>
struct Vec16<float> { typedef floatx4 type; };

template <typename CT, int D, int C, int BV>
struct __attribute__((aligned(16))) ChunkedSmem {
  static constexpr int P = Mma<CT>::PAD;
  static constexpr int NB = C / 16;
  CT K[C][D + P];         // keys, row-major
  CT Kt[D][C + P];        // keys, transposed, XOR-swizzled columns (see tsw)
  CT Q[C][D + P];         // queries
  CT Vt[BV][C + P];       // value slice, transposed, swizzled like Kt
  CT Wn[C][D + P];        // -W
  CT An[C][C + P];        // -A (only the strictly lower part is read)
  CT M[C][C + P];         // lower-incl-diag(Q K^T) (only J <= I blocks are read)
  CT O[C][BV + P];        // output staging
  float Adt[NB][16][20];  // fp32 diagonal blocks of A, transposed
  CT Td[NB][16][16 + P];  // (I + diagonal block of A)^{-1}
  float alpha[C];
};

template <typename CT, int D, int C, int BV>
constexpr size_t chunked_smem_bytes() {
  return sizeof(ChunkedSmem<CT, D, C, BV>);
}

template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (N > 0) {
    static_for<N - 1>(f);
    f(std::integral_constant<int, N - 1>{});
  }
}

// Work split of the blocked solve: every wave advances a fixed list of
// 16-column tiles of [K | V_slice] through the row blocks. A state wave's
// first CPW slots are its own value tiles (their solution U stays in its
// registers); key tiles go to the least-loaded wave; spare slots repeat key
// tile 0 and store nothing.
template <int NW, int SW, int CPW, int NKT>
struct SolvePlan {
  static constexpr int NVT = SW * CPW;
  static constexpr int NTW = (NKT + NVT + NW - 1) / NW > CPW ? (NKT + NVT + NW - 1) / NW : CPW;
  int kind[NW][NTW];  // 0 value tile, 1 key tile, 2 spare
  int idx[NW][NTW];
  constexpr SolvePlan() : kind(), idx() {
    int n[NW] = {};
    for (int w = 0; w < NW; ++w)
      for (int t = 0; t < NTW; ++t) kind[w][t] = 2, idx[w][t] = 0;
    for (int w = 0; w < SW; ++w)
      for (int c = 0; c < CPW; ++c) kind[w][n[w]] = 0, idx[w][n[w]] = w * CPW + c, ++n[w];
    for (int m = 0; m < NKT; ++m) {
      int best = 0;
      for (int w = 1; w < NW; ++w)
        if (n[w] < n[best]) best = w;
      kind[best][n[best]] = 1, idx[best][n[best]] = m, ++n[best];
    }
  }
};

template <typename CT, int D, int C, int BV, int SWQ>
__global__ __launch_bounds__(256, 1) void efla_chunked_kernel(ChunkedArgs a) {
  using MM = Mma<CT>;
  using Frag = typename MM::Frag;
  using Vec = typename Vec16<CT>::type;
  constexpr int NB = C / 16;    // 16-token blocks per chunk
  constexpr int NKT = D / 16;   // 16-row tiles of the state (key dimension)
  constexpr int NVT = BV / 16;  // 16-column tiles of the state slice
  constexpr int NW = 4;
  constexpr int SW = SWQ < NVT ? SWQ : NVT;   // waves that own state columns
  constexpr int CPW = NVT / SW;               // column tiles per state wave
  constexpr int VE = 16 / sizeof(CT);
  constexpr int NFK = NFrag<CT, NKT>::value;  // fragments over the key dim
  constexpr int NFB = NFrag<CT, NB>::value;   // fragments over a chunk
  static_assert(C % 16 == 0 && D % 16 == 0 && BV % 16 == 0 && SW <= NW, "tile sizes");
  constexpr SolvePlan<NW, SW, CPW, NKT> plan{};
  constexpr int NTW = plan.NTW;

  __shared__ ChunkedSmem<CT, D, C, BV> sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int li = lane & 15;
  const int g = lane >> 4;

  // Transposed tiles (rows = feature index d, columns = tokens) XOR their
  // column index with tsw(d) in 4-element groups: the staging writes, where
  // the lanes of a wave hold 16 different d, then spread over the LDS banks,
  // while every reader still gets 4 contiguous tokens.
  auto tsw = [](int d) { return ((d / VE) & (C / 4 - 1)) * 4; };

  // Workgroups are dispatched round-robin over the 8 XCDs; remap so that the
  // column slices of one head are adjacent on one XCD and share its L2.
  int L = blockIdx.x;
  const int total = gridDim.x;
  if (total % 8 == 0 && ((total / 8) % a.nvt) == 0)
    L = (blockIdx.x % 8) * (total / 8) + blockIdx.x / 8;
  const int head = L / a.nvt;
  const int v0 = (L % a.nvt) * BV;
  const int T = a.T;

  const CT* qg = (const CT*)a.q + (size_t)head * T * D;
  const CT* kg = (const CT*)a.k + (size_t)head * T * D;
  const CT* vg = (const CT*)a.v + (size_t)head * T * D;
  const CT* bg = (const CT*)a.beta + (size_t)head * T;
  CT* og = (CT*)a.o + (size_t)head * T * D;

  // ---- state slice: wave w < SW owns columns v0 + 16 (w CPW + c) + [0, 16)
  const bool owner = w < SW;
  floatx4 sacc[CPW][NKT];
#pragma unroll
  for (int c = 0; c < CPW; ++c)
#pragma unroll
    for (int rt = 0; rt < NKT; ++rt) sacc[c][rt] = floatx4{0.f, 0.f, 0.f, 0.f};
  if (owner && a.s0) {
    const float* s0 = a.s0 + (size_t)head * D * D;
#pragma unroll
    for (int c = 0; c < CPW; ++c)
#pragma unroll
      for (int rt = 0; rt < NKT; ++rt)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          sacc[c][rt][e] = s0[(size_t)(16 * rt + 4 * g + e) * D + v0 + 16 * (w * CPW + c) + li];
  }
  // Retire the initial-state loads here: left pending, they make the compiler
  // wait on every outstanding load (the next chunk's prefetch included)
  // inside the chunk loop.
#pragma unroll
  for (int c = 0; c < CPW; ++c)
#pragma unroll
    for (int rt = 0; rt < NKT; ++rt) asm volatile("" : "+v"(sacc[c][rt]));
  floatx4 uacc[CPW][NB];

  // ---- register prefetch of one chunk (coalesced 16-byte loads)
  constexpr int VPR = D / VE;    // 16-byte vectors per K/Q row
  constexpr int VPRV = BV / VE;  // 16-byte vectors per V-slice row
  constexpr int NLK = (C * VPR + 255) / 256;
  constexpr int NLV = (C * VPRV + 255) / 256;
  Vec kreg[NLK], qreg[NLK], vreg[NLV];
  CT breg[NLK];  // raw: converting here would make the prefetch wait for its loads
  auto prefetch = [&](int chunk) {
    const int t0 = chunk * C;
    const int nval = min(C, T - t0);
#pragma unroll
    for (int j = 0; j < NLK; ++j) {
      const int idx = tid + 256 * j;
      const int r = idx / VPR, cv = idx % VPR;
      kreg[j] = Vec{};
      qreg[j] = Vec{};
      breg[j] = from_f32<CT>(0.f);
      if (idx < C * VPR && r < nval) {
        kreg[j] = *(const Vec*)(kg + (size_t)(t0 + r) * D + cv * VE);
        qreg[j] = *(const Vec*)(qg + (size_t)(t0 + r) * D + cv * VE);
        breg[j] = bg[t0 + r];
      }
    }
#pragma unroll
    for (int j = 0; j < NLV; ++j) {
      const int idx = tid + 256 * j;
      const int r = idx / VPRV, cv = idx % VPRV;
      vreg[j] = Vec{};
      if (idx < C * VPRV && r < nval) vreg[j] = *(const Vec*)(vg + (size_t)(t0 + r) * D + v0 + cv * VE);
    }
  };

  const int nchunks = (T + C - 1) / C;
  prefetch(0);
  for (int ch = 0; ch < nchunks; ++ch) {
    const int t0 = ch * C;
    const int nval = min(C, T - t0);

    // ---- chunk ch (prefetched) -> LDS; lambda = ||k||^2 and alpha per row
    {
#pragma unroll
      for (int j = 0; j < NLK; ++j) {
        const int idx = tid + 256 * j;
        if (idx < C * VPR) {
          const int r = idx / VPR, cv = idx % VPR;
          st16(&sm.K[r][cv * VE], kreg[j]);
          st16(&sm.Q[r][cv * VE], qreg[j]);
          float ss = 0.f;
#pragma unroll
          for (int e = 0; e < VE; ++e) {
            const int d = cv * VE + e;
            sm.Kt[d][r ^ tsw(d)] = kreg[j][e];
            const float x = to_f32(kreg[j][e]);
            ss += x * x;
          }
          ss = group_sum<VPR>(ss);
          if (cv == 0) sm.alpha[r] = gate_alpha(to_f32(breg[j]), ss);
        }
      }
#pragma unroll
      for (int j = 0; j < NLV; ++j) {
        const int idx = tid + 256 * j;
        if (idx < C * VPRV) {
          const int r = idx / VPRV, cv = idx % VPRV;
#pragma unroll
          for (int e = 0; e < VE; ++e) {
            const int d = cv * VE + e;
            sm.Vt[d][r ^ tsw(d)] = vreg[j][e];
          }
        }
      }
    }
    // issue the global loads of the next chunk; they land during this one
    if (ch + 1 < nchunks) prefetch(ch + 1);
    __syncthreads();

    // ---- Gram, diagonal-block inverses and Q K^T, one barrier.
    //      Wave w first computes diagonal Gram block w, writes its scaled
    //      strictly-lower part (fp32, transposed) to LDS and inverts
    //      I + A_ww by column-parallel right-looking forward substitution
    //      (lane i owns column i; once t_j is final, column j of A is
    //      eliminated from the rows below, all independently). The remaining
    //      lower-triangle tiles of K K^T (-> -A) and Q K^T (-> M) are then
    //      shared out. Tile (I, J) is computed as X_J Y_I^T so that a lane
    //      ends up with 4 consecutive columns of row 16 I + li.
    {
      auto gram_store = [&](int I, int J, floatx4 acc) {
        const int r = 16 * I + li;
        const int cb = 16 * J + 4 * g;
        const float al = sm.alpha[r];
        floatx4 ad;
#pragma unroll
        for (int e = 0; e < 4; ++e) ad[e] = (cb + e < r) ? al * acc[e] : 0.f;
        MM::store_t(&sm.An[r][16 * J], -ad);
        return ad;
      };
      if (w < NB) {
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
        MM::template ll<D>(acc, &sm.K[16 * w + li][0], &sm.K[16 * w + li][0]);
        const floatx4 ad = gram_store(w, w, acc);
#pragma unroll
        for (int e = 0; e < 4; ++e) sm.Adt[w][4 * g + e][li] = ad[e];
        // the block is private to this wave: order its LDS writes before the
        // reads below without a workgroup barrier
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        float t[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) t[r] = (r == li) ? 1.f : 0.f;
#pragma unroll
        for (int j = 0; j < 15; ++j) {
          floatx4 a4[4];
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) a4[q4] = *(const floatx4*)&sm.Adt[w][j][4 * q4];
#pragma unroll
          for (int r = j + 1; r < 16; ++r) t[r] -= a4[r >> 2][r & 3] * t[j];
        }
        // lane groups g = 0..3 hold identical columns; group g writes rows 4g..4g+3
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if ((r >> 2) == g) sm.Td[w][r][li] = from_f32<CT>(t[r]);
      }
      constexpr int NOFF = NB * (NB - 1) / 2;   // strictly-lower Gram tiles
      constexpr int NQK = NB * (NB + 1) / 2;    // lower-incl-diag Q K^T tiles
      for (int job = w; job < NOFF + NQK; job += NW) {
        const bool isq = job >= NOFF;
        const int jj = isq ? job - NOFF : job;
        int I, J;
        if (isq) {
          I = 0;
          while ((I + 1) * (I + 2) / 2 <= jj) ++I;
          J = jj - I * (I + 1) / 2;
        } else {
          I = 1;
          while (I * (I + 1) / 2 <= jj) ++I;
          J = jj - I * (I - 1) / 2;
        }
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
        MM::template ll<D>(acc, &sm.K[16 * J + li][0],
                           isq ? &sm.Q[16 * I + li][0] : &sm.K[16 * I + li][0]);
        if (!isq) {
          gram_store(I, J, acc);
        } else {
          const int r = 16 * I + li;
          const int cb = 16 * J + 4 * g;
          floatx4 m;
#pragma unroll
          for (int e = 0; e < 4; ++e) m[e] = (cb + e <= r) ? acc[e] : 0.f;
          MM::store_t(&sm.M[r][16 * J], m);
        }
      }
    }
    __syncthreads();

    // ---- blocked forward solve (I + A) X = diag(a) [K | V_slice]:
    //      Y_i = diag(a_i) B_i - sum_{j<i} A_ij X_j,  X_i = (I + A_ii)^{-1} Y_i,
    //      all of this wave's tiles advancing together so their MFMA chains
    //      overlap. A value tile's X (= U) stays in registers. A key tile's X
    //      (= W) is also formed transposed, X_i^T = Y_i^T (I + A_ii)^{-T}, whose
    //      accumulator holds 4 consecutive columns of a row of W: it is
    //      stored negated and row-major with 8-byte writes.
    {
      const CT* rhs[NTW];
      int swz[NTW];
#pragma unroll
      for (int t = 0; t < NTW; ++t) {
        const int row = 16 * plan.idx[w][t] + li;
        rhs[t] = plan.kind[w][t] == 0 ? &sm.Vt[row][0] : &sm.Kt[row][0];
        swz[t] = tsw(row);
      }
      floatx4 x[NTW][NB];
      Frag xf[NTW][NFB];
      static_for<NB>([&](auto ib) {
        constexpr int i = decltype(ib)::value;
        const floatx4 al = *(const floatx4*)&sm.alpha[16 * i + 4 * g];
        const Frag td = MM::template lds<1>(&sm.Td[i][li][0], 0, 0);
        Frag an[NFrag<CT, (i > 0 ? i : 1)>::value];
        if constexpr (i > 0) {
#pragma unroll
          for (int f = 0; f < NFrag<CT, i>::value; ++f)
            an[f] = MM::template lds<i>(&sm.An[16 * i + li][0], f, 0);
        }
#pragma unroll
        for (int t = 0; t < NTW; ++t) {
          floatx4 y = al * MM::load4(rhs[t] + ((16 * i + 4 * g) ^ swz[t]));
          if constexpr (i > 0) {
#pragma unroll
            for (int f = 0; f < NFrag<CT, i>::value; ++f) {
              // fragment f of X_{<i}; its upper tile exists only once block 2f+1 < i
              Frag xin = xf[t][f];
              if constexpr (Mma<CT>::KT == 2) {
                if (2 * f + 1 >= i) xin = MM::template acc<1>(&x[t][2 * f], 0);
              }
              y = MM::mma(y, an[f], xin);
            }
          }
          const Frag yf = MM::template acc<1>(&y, 0);
          x[t][i] = MM::mma(floatx4{0.f, 0.f, 0.f, 0.f}, td, yf);
          if constexpr (Mma<CT>::KT == 2) {
            if constexpr (i % 2 == 1) xf[t][i / 2] = MM::template acc<2>(&x[t][i - 1], 0);
          } else {
            xf[t][i] = MM::template acc<1>(&x[t][i], 0);
          }
          if (plan.kind[w][t] == 1) {
            const floatx4 xt = MM::mma(floatx4{0.f, 0.f, 0.f, 0.f}, yf, td);
            MM::store_t(&sm.Wn[16 * i + li][16 * plan.idx[w][t]], -xt);
          }
        }
      });
#pragma unroll
      for (int t = 0; t < NTW; ++t) {
        if (plan.kind[w][t] == 0) {
          const int c = plan.idx[w][t] - w * CPW;
#pragma unroll
          for (int cc = 0; cc < CPW; ++cc)
            if (cc == c) {
#pragma unroll
              for (int i = 0; i < NB; ++i) uacc[cc][i] = x[t][i];
            }
        }
      }
    }
    __syncthreads();

    // ---- serial part, per state wave and column tile c:
    //      U' = U - W S;  O^T = S^T Q^T + U'^T M^T;  S += K^T U'
    if (owner) {
      Frag sf[CPW][NFK];
#pragma unroll
      for (int c = 0; c < CPW; ++c)
#pragma unroll
        for (int f = 0; f < NFK; ++f) sf[c][f] = MM::template acc<NKT>(sacc[c], f);
      floatx4 oacc[CPW][NB];
#pragma unroll
      for (int ut = 0; ut < NB; ++ut) {
#pragma unroll
        for (int c = 0; c < CPW; ++c) oacc[c][ut] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int f = 0; f < NFK; ++f) {
          const Frag wf = MM::template lds<NKT>(&sm.Wn[16 * ut + li][0], f, 0);
          const Frag qf = MM::template lds<NKT>(&sm.Q[16 * ut + li][0], f, 0);
#pragma unroll
          for (int c = 0; c < CPW; ++c) {
            uacc[c][ut] = MM::mma(uacc[c][ut], wf, sf[c][f]);
            oacc[c][ut] = MM::mma(oacc[c][ut], sf[c][f], qf);
          }
        }
      }
      Frag uf[CPW][NFB];
#pragma unroll
      for (int c = 0; c < CPW; ++c)
#pragma unroll
        for (int f = 0; f < NFB; ++f) uf[c][f] = MM::template acc<NB>(uacc[c], f);
      static_for<NB>([&](auto ub) {
        constexpr int ut = decltype(ub)::value;
#pragma unroll
        for (int f = 0; f < NFrag<CT, ut + 1>::value; ++f) {
          const Frag mf = MM::template lds<ut + 1>(&sm.M[16 * ut + li][0], f, 0);
#pragma unroll
          for (int c = 0; c < CPW; ++c) oacc[c][ut] = MM::mma(oacc[c][ut], uf[c][f], mf);
        }
      });
#pragma unroll
      for (int rt = 0; rt < NKT; ++rt) {
        const int row = 16 * rt + li;
#pragma unroll
        for (int f = 0; f < NFB; ++f) {
          const Frag kf = MM::template lds<NB>(&sm.Kt[row][0], f, tsw(row));
#pragma unroll
          for (int c = 0; c < CPW; ++c) sacc[c][rt] = MM::mma(sacc[c][rt], kf, uf[c][f]);
        }
      }
      // O^T tile (c, ut): lane holds O[16 ut + li][16 (w CPW + c) + 4 g + e]
#pragma unroll
      for (int c = 0; c < CPW; ++c)
#pragma unroll
        for (int ut = 0; ut < NB; ++ut) MM::store_t(&sm.O[16 * ut + li][16 * (w * CPW + c)], oacc[c][ut]);
    }
    __syncthreads();

    // ---- write the chunk's outputs (coalesced 16-byte stores)
    {
      constexpr int VPRO = BV / VE;
      for (int idx = tid; idx < C * VPRO; idx += 256) {
        const int r = idx / VPRO, cv = idx % VPRO;
        if (r < nval) *(Vec*)(og + (size_t)(t0 + r) * D + v0 + cv * VE) = ld16(&sm.O[r][cv * VE]);
      }
    }
  }

  if (owner && a.s_final) {
    float* sf = a.s_final + (size_t)head * D * D;
#pragma unroll
    for (int c = 0; c < CPW; ++c)
#pragma unroll
      for (int rt = 0; rt < NKT; ++rt)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          sf[(size_t)(16 * rt + 4 * g + e) * D + v0 + 16 * (w * CPW + c) + li] = sacc[c][rt][e];
  }
}

// ===========================================================================
// Pipelined variant: 8 waves per workgroup. Waves 0-3 (state group) run the
// serial state pass of chunk c while waves 4-7 (prep group) prepare chunk c+1,
// so on every SIMD one wave's MFMA stream overlaps the other's latency-bound
// prep. The prep produces, per chunk, A = strictly-lower(diag(a) K K^T),
// T = (I + A)^{-1} (full, lower triangular), M = lower-incl-diag(Q K^T) and a;
// the state pass then needs no WY factor:
//   Y  = diag(a) (V - K S)
//   U' = T Y                       (= U - W S with W = T diag(a) K, U = T diag(a) V)
//   O^T = S^T Q^T + U'^T M^T       (read out after each update)
//   S <- S + K^T U'
// K, Q, V, T, M and a are double-buffered in LDS; K^T and the columns of V
// are read with ds_read_b64_tr_b16 straight from the row-major tiles. Both
// groups pass three workgroup barriers per chunk.
template <typename CT, int D, int C, int BV>
struct __attribute__((aligned(16))) PipeSmem {
  static constexpr int P = Mma<CT>::PAD;
  static constexpr int PK = 16 / sizeof(CT);  // K, Q rows padded by 16 bytes
  static constexpr int NB = C / 16;
  struct Buf {
    CT K[C][D + PK];
    CT Q[C][D + PK];
    CT V[C][BV + P];   // value slice
    CT T[C][C + P];    // (I + A)^{-1}; only the lower block triangle is read
    CT M[C][C + P];    // lower-incl-diag(Q K^T); only J <= I blocks are read
    float alpha[C];
  } buf[2];
  CT An[C][C + P];        // -A, strictly lower part (prep-private)
  float Adt[NB][16][20];  // fp32 diagonal blocks of A, transposed (prep-private)
  CT Td[NB][16][16 + P];  // (I + A_bb)^{-1} (prep-private)
  CT O[C][BV + P];        // output staging (state group)
};

template <typename CT, int D, int C, int BV>
constexpr size_t pipe_smem_bytes() {
  return sizeof(PipeSmem<CT, D, C, BV>);
}

// Strictly-lower Gram tiles and lower-incl-diag Q K^T tiles, enumerated
// (I, J) row by row; job j goes to prep wave j % 4.
template <int NB>
struct PrepJobs {
  static constexpr int NOFF = NB * (NB - 1) / 2;
  static constexpr int NQK = NB * (NB + 1) / 2;
  static constexpr int N = NOFF + NQK;
  static constexpr int is_qk(int j) { return j >= NOFF; }
  static constexpr int I(int j) {
    if (j < NOFF) { int i = 1; while (i * (i + 1) / 2 <= j) ++i; return i; }
    j -= NOFF; int i = 0; while ((i + 1) * (i + 2) / 2 <= j) ++i; return i;
  }
  static constexpr int J(int j) {
    const int i = I(j);
    return j < NOFF ? j - i * (i - 1) / 2 : (j - NOFF) - i * (i + 1) / 2;
  }
};

template <typename CT, int D, int C, int BV>
__global__ __launch_bounds__(512, 1) void efla_chunked_pipe_kernel(ChunkedArgs a) {
  using MM = Mma<CT>;
  using Frag = typename MM::Frag;
  using Vec = typename Vec16<CT>::type;
  using Sm = PipeSmem<CT, D, C, BV>;
  constexpr int NB = C / 16;
  constexpr int NKT = D / 16;
  constexpr int NVT = BV / 16;
  constexpr int VE = 16 / sizeof(CT);
  constexpr int NFK = NFrag<CT, NKT>::value;
  constexpr int NFB = NFrag<CT, NB>::value;
  constexpr int LDK = D + Sm::PK;
  constexpr int LDV = BV + Sm::P;
  static_assert(NVT <= 4 && NB <= 4 && C % 16 == 0 && D % 16 == 0, "tile sizes");

  __shared__ Sm sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;  // 0-3 state group, 4-7 prep group
  const int li = lane & 15;
  const int g = lane >> 4;

  int L = blockIdx.x;
  const int total = gridDim.x;
  if (total % 8 == 0 && ((total / 8) % a.nvt) == 0)
    L = (blockIdx.x % 8) * (total / 8) + blockIdx.x / 8;
  const int head = L / a.nvt;
  const int v0 = (L % a.nvt) * BV;
  const int T = a.T;
  const int nchunks = (T + C - 1) / C;

  if (w < 4) {
    // ======================= state group =======================
    const bool owner = w < NVT;
    const int scol = v0 + 16 * w + li;
    CT* og = (CT*)a.o + (size_t)head * T * D;
    floatx4 sacc[NKT];
#pragma unroll
    for (int rt = 0; rt < NKT; ++rt) sacc[rt] = floatx4{0.f, 0.f, 0.f, 0.f};
    if (owner && a.s0) {
      const float* s0 = a.s0 + (size_t)head * D * D;
#pragma unroll
      for (int rt = 0; rt < NKT; ++rt)
#pragma unroll
        for (int e = 0; e < 4; ++e) sacc[rt][e] = s0[(size_t)(16 * rt + 4 * g + e) * D + scol];
    }
#pragma unroll
    for (int rt = 0; rt < NKT; ++rt) asm volatile("" : "+v"(sacc[rt]));

    auto store_out = [&](int chunk) {
      const int t0 = chunk * C;
      const int nval = min(C, T - t0);
      constexpr int VPRO = BV / VE;
      for (int idx = tid; idx < C * VPRO; idx += 256) {
        const int r = idx / VPRO, cv = idx % VPRO;
        if (r < nval) *(Vec*)(og + (size_t)(t0 + r) * D + v0 + cv * VE) = ld16(&sm.O[r][cv * VE]);
      }
    };

    for (int c = -1; c < nchunks; ++c) {
      const bool act = c >= 0 && owner;
      const auto& B = sm.buf[c & 1];
      floatx4 oacc[NB], y[NB];
      Frag sf[NFK], uf[NFB];
      // ---- phase A: K S, S^T Q^T, Y = diag(a)(V - K S); store outputs of c-1
      if (c >= 1) store_out(c - 1);
      if (act) {
#pragma unroll
        for (int f = 0; f < NFK; ++f) sf[f] = MM::template acc<NKT>(sacc, f);
#pragma unroll
        for (int ut = 0; ut < NB; ++ut) {
          floatx4 p = {0.f, 0.f, 0.f, 0.f};
          oacc[ut] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int f = 0; f < NFK; ++f) {
            p = MM::mma(p, MM::template lds<NKT>(&B.K[16 * ut + li][0], f, 0), sf[f]);
            oacc[ut] = MM::mma(oacc[ut], sf[f], MM::template lds<NKT>(&B.Q[16 * ut + li][0], f, 0));
          }
          const floatx4 al = *(const floatx4*)&B.alpha[16 * ut + 4 * g];
          const floatx4 vv = to_f32x4(ldtr4(&B.V[0][0], LDV, 16 * ut + 4 * g, 16 * w));
          y[ut] = al * (vv - p);
        }
      }
      __syncthreads();
      // ---- phase B: U' = T Y, O^T += U'^T M^T
      if (act) {
        Frag yf[NFB];
#pragma unroll
        for (int f = 0; f < NFB; ++f) yf[f] = MM::template acc<NB>(y, f);
        floatx4 u[NB];
        static_for<NB>([&](auto ub) {
          constexpr int ut = decltype(ub)::value;
          u[ut] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int f = 0; f < NFrag<CT, ut + 1>::value; ++f)
            u[ut] = MM::mma(u[ut], MM::template lds<ut + 1>(&B.T[16 * ut + li][0], f, 0), yf[f]);
        });
#pragma unroll
        for (int f = 0; f < NFB; ++f) uf[f] = MM::template acc<NB>(u, f);
        static_for<NB>([&](auto ub) {
          constexpr int ut = decltype(ub)::value;
#pragma unroll
          for (int f = 0; f < NFrag<CT, ut + 1>::value; ++f)
            oacc[ut] = MM::mma(oacc[ut], uf[f], MM::template lds<ut + 1>(&B.M[16 * ut + li][0], f, 0));
        });
      }
      __syncthreads();
      // ---- phase C: S += K^T U'; stage O^T
      if (act) {
#pragma unroll
        for (int rt = 0; rt < NKT; ++rt)
#pragma unroll
          for (int f = 0; f < NFB; ++f)
            sacc[rt] = MM::mma(sacc[rt], tr_frag<NB>(&B.K[0][0], LDK, f, 16 * rt), uf[f]);
#pragma unroll
        for (int ut = 0; ut < NB; ++ut) MM::store_t(&sm.O[16 * ut + li][16 * w], oacc[ut]);
      }
      __syncthreads();
    }
    store_out(nchunks - 1);
    if (owner && a.s_final) {
      float* sf = a.s_final + (size_t)head * D * D;
#pragma unroll
      for (int rt = 0; rt < NKT; ++rt)
#pragma unroll
        for (int e = 0; e < 4; ++e) sf[(size_t)(16 * rt + 4 * g + e) * D + scol] = sacc[rt][e];
    }
  } else {
    // ======================= prep group =======================
    const int pw = w - 4;        // prep wave 0..3
    const int ptid = tid - 256;  // 0..255
    const CT* qg = (const CT*)a.q + (size_t)head * T * D;
    const CT* kg = (const CT*)a.k + (size_t)head * T * D;
    const CT* vg = (const CT*)a.v + (size_t)head * T * D;
    const CT* bg = (const CT*)a.beta + (size_t)head * T;

    constexpr int VPR = D / VE;
    constexpr int VPRV = BV / VE;
    constexpr int NLK = (C * VPR + 255) / 256;
    constexpr int NLV = (C * VPRV + 255) / 256;
    Vec kreg[NLK], qreg[NLK], vreg[NLV];
    CT breg[NLK];
    auto prefetch = [&](int chunk) {
      const int t0 = chunk * C;
      const int nval = min(C, T - t0);
#pragma unroll
      for (int j = 0; j < NLK; ++j) {
        const int idx = ptid + 256 * j;
        const int r = idx / VPR, cv = idx % VPR;
        kreg[j] = Vec{};
        qreg[j] = Vec{};
        breg[j] = from_f32<CT>(0.f);
        if (idx < C * VPR && r < nval) {
          kreg[j] = *(const Vec*)(kg + (size_t)(t0 + r) * D + cv * VE);
          qreg[j] = *(const Vec*)(qg + (size_t)(t0 + r) * D + cv * VE);
          breg[j] = bg[t0 + r];
        }
      }
#pragma unroll
      for (int j = 0; j < NLV; ++j) {
        const int idx = ptid + 256 * j;
        const int r = idx / VPRV, cv = idx % VPRV;
        vreg[j] = Vec{};
        if (idx < C * VPRV && r < nval) vreg[j] = *(const Vec*)(vg + (size_t)(t0 + r) * D + v0 + cv * VE);
      }
    };
    prefetch(0);

    for (int c = -1; c < nchunks; ++c) {
      const int n = c + 1;  // chunk being prepared
      const bool act = n < nchunks;
      auto& B = sm.buf[n & 1];
      // ---- phase A: stage chunk n; a = -expm1(-beta lambda)/lambda per row
      if (act) {
#pragma unroll
        for (int j = 0; j < NLK; ++j) {
          const int idx = ptid + 256 * j;
          if (idx < C * VPR) {
            const int r = idx / VPR, cv = idx % VPR;
            st16(&B.K[r][cv * VE], kreg[j]);
            st16(&B.Q[r][cv * VE], qreg[j]);
            float ss = 0.f;
#pragma unroll
            for (int e = 0; e < VE; ++e) {
              const float x = to_f32(kreg[j][e]);
              ss += x * x;
            }
            ss = group_sum<VPR>(ss);
            if (cv == 0) B.alpha[r] = gate_alpha(to_f32(breg[j]), ss);
          }
        }
#pragma unroll
        for (int j = 0; j < NLV; ++j) {
          const int idx = ptid + 256 * j;
          if (idx < C * VPRV) {
            const int r = idx / VPRV, cv = idx % VPRV;
            st16(&B.V[r][cv * VE], vreg[j]);
          }
        }
        if (n + 1 < nchunks) prefetch(n + 1);
      }
      __syncthreads();
      // ---- phase B: diagonal Gram block + its inverse (wave pw = block), then
      //      the remaining Gram (-> -A) and Q K^T (-> M) tiles.
      if (act) {
        auto gram_scaled = [&](int I, int J, floatx4 acc) {
          const int r = 16 * I + li;
          const int cb = 16 * J + 4 * g;
          const float al = B.alpha[r];
          floatx4 ad;
#pragma unroll
          for (int e = 0; e < 4; ++e) ad[e] = (cb + e < r) ? al * acc[e] : 0.f;
          MM::store_t(&sm.An[r][16 * J], -ad);
          return ad;
        };
        auto tile_jobs = [&](auto pwc) {
          constexpr int PW = decltype(pwc)::value;
          using JB = PrepJobs<NB>;
          constexpr int NJ = (JB::N - PW + 3) / 4;  // jobs PW, PW+4, ...
          floatx4 acc[NJ > 0 ? NJ : 1];
          static_for<NJ>([&](auto jc) {
            constexpr int j = PW + 4 * decltype(jc)::value;
            constexpr int I = JB::I(j), J = JB::J(j);
            acc[decltype(jc)::value] = floatx4{0.f, 0.f, 0.f, 0.f};
            MM::template ll<D>(acc[decltype(jc)::value], &B.K[16 * J + li][0],
                               JB::is_qk(j) ? &B.Q[16 * I + li][0] : &B.K[16 * I + li][0]);
          });
          static_for<NJ>([&](auto jc) {
            constexpr int j = PW + 4 * decltype(jc)::value;
            constexpr int I = JB::I(j), J = JB::J(j);
            const floatx4 v = acc[decltype(jc)::value];
            if constexpr (JB::is_qk(j)) {
              const int r = 16 * I + li;
              const int cb = 16 * J + 4 * g;
              floatx4 m;
#pragma unroll
              for (int e = 0; e < 4; ++e) m[e] = (cb + e <= r) ? v[e] : 0.f;
              MM::store_t(&B.M[r][16 * J], m);
            } else {
              gram_scaled(I, J, v);
            }
          });
        };
        if (pw < NB) {
          floatx4 acc = {0.f, 0.f, 0.f, 0.f};
          MM::template ll<D>(acc, &B.K[16 * pw + li][0], &B.K[16 * pw + li][0]);
          const floatx4 ad = gram_scaled(pw, pw, acc);
#pragma unroll
          for (int e = 0; e < 4; ++e) sm.Adt[pw][4 * g + e][li] = ad[e];
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
        switch (pw) {
          case 0: tile_jobs(std::integral_constant<int, 0>{}); break;
          case 1: tile_jobs(std::integral_constant<int, 1>{}); break;
          case 2: tile_jobs(std::integral_constant<int, 2>{}); break;
          default: tile_jobs(std::integral_constant<int, 3>{}); break;
        }
        if (pw < NB) {
          // column-parallel right-looking forward substitution in fp32 (lane
          // li owns column li; once t_j is final, column j of A is eliminated
          // from the rows below, all independently)
          float t[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) t[r] = (r == li) ? 1.f : 0.f;
#pragma unroll
          for (int j = 0; j < 15; ++j) {
            floatx4 a4[4];
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) a4[q4] = *(const floatx4*)&sm.Adt[pw][j][4 * q4];
#pragma unroll
            for (int r = j + 1; r < 16; ++r) t[r] -= a4[r >> 2][r & 3] * t[j];
          }
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if ((r >> 2) == g) sm.Td[pw][r][li] = from_f32<CT>(t[r]);
        }
      }
      __syncthreads();
      // ---- phase C: column tile m = pw of T = (I + A)^{-1}:
      //      X_i = (I + A_ii)^{-1} (E_i - sum_{m<=j<i} A_ij X_j), i >= m, where
      //      E is the identity; X_i^T is also formed so T is written
      //      row-major with 8-byte stores.
      if (act && pw < NB) {
        auto col_tile = [&](auto mc) {
          constexpr int m = decltype(mc)::value;
          floatx4 x[NB];
          static_for<NB>([&](auto ib) {
            constexpr int i = decltype(ib)::value;
            if constexpr (i >= m) {
              floatx4 yv;
#pragma unroll
              for (int e = 0; e < 4; ++e) yv[e] = (i == m && 4 * g + e == li) ? 1.f : 0.f;
              if constexpr (i > m) {
#pragma unroll
                for (int f = 0; f < NFrag<CT, i>::value; ++f) {
                  if constexpr (MM::KT == 2) {
                    if (2 * f + 1 < m) continue;  // both tiles of the fragment are zero
                  } else {
                    if (f < m) continue;
                  }
                  floatx4 xin[2] = {x[MM::KT * f], MM::KT == 2 && 2 * f + 1 < i ? x[2 * f + 1] : x[MM::KT * f]};
                  yv = MM::mma(yv, MM::template lds<i>(&sm.An[16 * i + li][0], f, 0),
                               MM::template acc<(MM::KT == 2 ? 2 : 1)>(xin, 0));
                }
              }
              const Frag td = MM::template lds<1>(&sm.Td[i][li][0], 0, 0);
              const Frag yf = MM::template acc<1>(&yv, 0);
              x[i] = MM::mma(floatx4{0.f, 0.f, 0.f, 0.f}, td, yf);
              const floatx4 xt = MM::mma(floatx4{0.f, 0.f, 0.f, 0.f}, yf, td);
              MM::store_t(&B.T[16 * i + li][16 * m], xt);
            } else {
              x[i] = floatx4{0.f, 0.f, 0.f, 0.f};
            }
          });
        };
        switch (pw) {
          case 0: col_tile(std::integral_constant<int, 0>{}); break;
          case 1: if constexpr (NB > 1) col_tile(std::integral_constant<int, (NB > 1 ? 1 : 0)>{}); break;
          case 2: if constexpr (NB > 2) col_tile(std::integral_constant<int, (NB > 2 ? 2 : 0)>{}); break;
          default: if constexpr (NB > 3) col_tile(std::integral_constant<int, (NB > 3 ? 3 : 0)>{}); break;
        }
      }
      __syncthreads();
    }
  }
}

// ---------------------------------------------------------------------------
// Host-side launch. Returns hipSuccess or the launch error.
template <typename CT, int D, int C>
static hipError_t launch_chunked(const ChunkedArgs& in, int NH, hipStream_t stream) {
  constexpr int BV = D < 64 ? D : 64;
  ChunkedArgs a = in;
  a.nvt = D / BV;
  dim3 grid((unsigned)(NH * a.nvt));
  if constexpr (pipe_smem_bytes<CT, D, C, BV>() <= 160 * 1024) {
    hipLaunchKernelGGL((efla_chunked_pipe_kernel<CT, D, C, BV>), grid, dim3(512), 0, stream, a);
  } else {
    static_assert(chunked_smem_bytes<CT, D, C, BV>() <= 160 * 1024, "LDS budget");
    hipLaunchKernelGGL((efla_chunked_kernel<CT, D, C, BV, EFLA_STATE_WAVES>), grid, dim3(256), 0,
                       stream, a);
  }
  return hipGetLastError();
}

template <typename CT, int D>
static hipError_t dispatch_chunk(const ChunkedArgs& a, int NH, int chunk, hipStream_t s) {
  switch (chunk) {
    case 16: return launch_chunked<CT, D, 16>(a, NH, s);
    case 32: return launch_chunked<CT, D, 32>(a, NH, s);
    case 64:
      if constexpr (sizeof(CT) == 4 && D == 128) return hipErrorInvalidValue;
      else return launch_chunked<CT, D, 64>(a, NH, s);
    default: return hipErrorInvalidValue;
  }
}

template <typename CT>
static hipError_t dispatch_d(const ChunkedArgs& a, int NH, int d, int chunk, hipStream_t s) {
  switch (d) {
    case 16: return dispatch_chunk<CT, 16>(a, NH, chunk, s);
    case 32: return dispatch_chunk<CT, 32>(a, NH, chunk, s);
    case 64: return dispatch_chunk<CT, 64>(a, NH, chunk, s);
    case 128: return dispatch_chunk<CT, 128>(a, NH, chunk, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace efla

// Internal entry used by the C ABI layer (arguments already validated).
hipError_t efla_internal_launch_chunked(const void* q, const void* k, const void* v,
                                        const void* beta, const float* s0, void* o,
                                        float* s_final, int NH, int T, int d, int chunk,
                                        int is_bf16, hipStream_t stream) {
  efla::ChunkedArgs a{q, k, v, beta, s0, o, s_final, T, 1};
  if (is_bf16) return efla::dispatch_d<efla::bf16>(a, NH, d, chunk, stream);
  return efla::dispatch_d<float>(a, NH, d, chunk, stream);
}
