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

#include <algorithm>

#include "efla_device.hpp"

// Waves per workgroup that hold the state slice (2: 32 columns each; 4: 16),
// for the 4-wave kernel and for the state group of the pipelined kernel.
#ifndef EFLA_STATE_WAVES
#define EFLA_STATE_WAVES 2
#endif
#ifndef EFLA_PIPE_STATE_WAVES
#define EFLA_PIPE_STATE_WAVES 2
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
  // Time-segmented passes (pipelined kernel only), over nseg segments of
  // seg_len tokens. mode 0: one pass over the whole sequence per head.
  // mode 1 (pass mode 1): the affine maps S_end = P_g S_start + R_g of
  // segments g = 1 .. nseg - 2; virtual head h nrun + j (nrun = nseg - 2)
  // handles segment j + 1 and stores R_g to seg_out[(h nrun + j) 2] and P_g
  // to seg_out[(h nrun + j) 2 + 1]. mode 2: virtual head h nrun + j runs
  // segment g = seg_first + j from its start state (S0 for g = 0, else
  // seg_s0[h nseg + g]) and writes its outputs; segment 0 stores its end
  // state to seg_s0[h nseg + 1], the last segment writes s_final.
  int mode;
  int seg_len;
  int nseg;
  float* seg_s0;  // segment start states (workspace; segment 0 writes slot 1)
  float* seg_out;
  int coef;  // step coefficient rule (gate_coef)
  // pass mode 2 of the pipelined kernel (states for the backward): the state
  // at the start of every chunk, [head][chunk][d_v][d_k] (transposed; bf16
  // for bf16 inputs with C and d multiples of 32, else fp32) and, when
  // s_chunks_n is not null, [head][chunk][d_k][d_v] fp32 (natural)
  float* s_chunks;
  float* s_chunks_n;
  int seg_first;  // mode 2: first segment of this launch
  int nrun;       // modes 1 and 2: segments per head in this launch
  // gated variant (4-wave kernel): per-token log-decay [head][T], fp32
  const float* log_g;
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
  float lg[C];            // gated variant: b_r, the log-decay summed over rows 0..r
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

// GATED: the gated variant S_t = g_t (I - c k k^T) S_{t-1} + c k v^T,
// g_t = exp(log_g_t) (the reading taken of the papernotes note's "Gated
// EFLA": Gated DeltaNet's update with the exact-flow coefficient). With
// b_r = log_g summed over the chunk's rows 0..r and Gamma_r = exp(b_r), the
// chunk's rows satisfy (I + A) U = diag(c) (V - diag(Gamma) K S) with
// A = strictly-lower(diag(c) K K^T * exp(b_r - b_i)), so:
//   W  = T diag(c Gamma) K,  U = T diag(c) V,  U' = U - W S
//   O  = diag(Gamma) Q S + (lower-incl-diag(Q K^T) * exp(b_r - b_i)) U'
//   S <- Gamma_C S + K^T diag(Gamma_C / Gamma) U'
// Every exponent b_r - b_i (i <= r) and b_C - b_r is <= 0 for decays g <= 1;
// a decay factor is only formed where the recurrence carries it.
template <typename CT, int D, int C, int BV, int SWQ, bool GATED = false>
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
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: role branches stay scalar
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
  float lgreg = 0.f;  // gated: wave 0, lane r holds log_g of the chunk's row r
  const float* lgg = GATED ? a.log_g + (size_t)head * T : nullptr;
  auto prefetch = [&](int chunk) {
    const int t0 = chunk * C;
    const int nval = min(C, T - t0);
    if constexpr (GATED) lgreg = (tid < nval) ? lgg[t0 + tid] : 0.f;
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
          if (cv == 0) sm.alpha[r] = gate_coef(a.coef, to_f32(breg[j]), ss);
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
    if constexpr (GATED) {
      // b_r: inclusive prefix sum of the chunk's log-decays (rows past T
      // carry 0, so the last row holds b of the last valid token)
      if (w == 0) {
        float x = lgreg;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const float y = __shfl_up(x, off);
          if (lane >= off) x += y;
        }
        if (lane < C) sm.lg[lane] = x;
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
        if constexpr (GATED) {
          // the decay factor is formed only below the diagonal, where its
          // exponent b_r - b_i is what the recurrence carries
          const float br = sm.lg[r];
#pragma unroll
          for (int e = 0; e < 4; ++e) ad[e] = (cb + e < r) ? al * acc[e] * __expf(br - sm.lg[cb + e]) : 0.f;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) ad[e] = (cb + e < r) ? al * acc[e] : 0.f;
        }
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
          if constexpr (GATED) {
            const float br = sm.lg[r];
#pragma unroll
            for (int e = 0; e < 4; ++e) m[e] = (cb + e <= r) ? acc[e] * __expf(br - sm.lg[cb + e]) : 0.f;
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) m[e] = (cb + e <= r) ? acc[e] : 0.f;
          }
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
        // gated: the key right-hand sides take diag(c Gamma), the values diag(c)
        floatx4 alk = al;
        if constexpr (GATED) {
#pragma unroll
          for (int e = 0; e < 4; ++e) alk[e] = al[e] * __expf(sm.lg[16 * i + 4 * g + e]);
        }
        const Frag td = MM::template lds<1>(&sm.Td[i][li][0], 0, 0);
        Frag an[NFrag<CT, (i > 0 ? i : 1)>::value];
        if constexpr (i > 0) {
#pragma unroll
          for (int f = 0; f < NFrag<CT, i>::value; ++f)
            an[f] = MM::template lds<i>(&sm.An[16 * i + li][0], f, 0);
        }
#pragma unroll
        for (int t = 0; t < NTW; ++t) {
          floatx4 y = (plan.kind[w][t] == 1 ? alk : al) * MM::load4(rhs[t] + ((16 * i + 4 * g) ^ swz[t]));
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
      if constexpr (GATED) {
        // O^T tile column li is token 16 ut + li: the Q S part takes Gamma
#pragma unroll
        for (int ut = 0; ut < NB; ++ut) {
          const float gm = __expf(sm.lg[16 * ut + li]);
#pragma unroll
          for (int c = 0; c < CPW; ++c) oacc[c][ut] = oacc[c][ut] * gm;
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
      if constexpr (GATED) {
        // S <- Gamma_C S + K^T diag(Gamma_C / Gamma) U': rows 4g + e of U'
        // tile ut are tokens 16 ut + 4g + e
        const float bl = sm.lg[C - 1];
#pragma unroll
        for (int c = 0; c < CPW; ++c) {
#pragma unroll
          for (int ut = 0; ut < NB; ++ut)
#pragma unroll
            for (int e = 0; e < 4; ++e) uacc[c][ut][e] *= __expf(bl - sm.lg[16 * ut + 4 * g + e]);
#pragma unroll
          for (int f = 0; f < NFB; ++f) uf[c][f] = MM::template acc<NB>(uacc[c], f);
        }
        const float gc = __expf(bl);
#pragma unroll
        for (int c = 0; c < CPW; ++c)
#pragma unroll
          for (int rt = 0; rt < NKT; ++rt) sacc[c][rt] = sacc[c][rt] * gc;
      }
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
// Pipelined variant: NSW state waves plus four prep waves per workgroup. The
// state waves run the serial state pass of chunk c while the prep waves
// prepare chunk c+1. The prep produces, per chunk, a, the diagonal-block
// inverses, T = (I + A)^{-1} with A = strictly-lower(diag(a) K K^T) (full,
// lower triangular) and M = lower-incl-diag(Q K^T); the state pass then needs
// no WY factor:
//   Y  = V - K S
//   U' = T diag(a) Y               (= U - W S with W = T diag(a) K, U = T diag(a) V)
//   O^T = S^T Q^T + U'^T M^T       (read out after each update)
//   S <- S + K^T U'
// In the output and summary passes the state waves hold N = -S and the
// solvers store T' = -T diag(a) (a applied in fp32), so Y = V + K N comes out
// of the MFMAs with the values as the accumulator's start, -U' = T' Y,
// N <- N + K^T (-U') and -O^T = N^T Q^T + (-U')^T M^T: no per-element gate or
// subtraction in the serial pass; outputs and the final state are negated
// back when stored. The state-saving pass (for the backward), which stores
// the state at every chunk, keeps S and forms Y = diag(a) (V - K S) in the
// state waves with T unscaled.
// Two workgroup barriers per chunk split it into phases A and B. While the
// state waves run chunk c:
//   state waves    A: K S, Y, U' = T Y           B: S^T Q^T, K^T U', U'^T M^T;
//                                                    store O
//   prep 0, 1      A: (I+A_bb)^-1 of c+1 (with   B: Gram tiles below the diagonal,
//   ("solvers")       four 16-row blocks the         the column tiles of T and
//                     loaders formed A_bb)           (four blocks) row block 3 of
//                                                    M, of c+1
//   prep 2..5      A: stage K, Q, V of c+1;      B: the other Q K^T tiles of
//   ("loaders")       one Q K^T tile of c (with      c+1 (with four blocks:
//                     four blocks: loaders 2, 3);    loaders 2, 3); a (and with
//                     load the keys of c+2 (with     four blocks the diagonal
//                     four blocks: keys, betas,      Gram blocks) of c+2; load
//                     queries and values of c+3)     Q, V of c+2
// Waves are placed on the SIMDs round robin: the two state waves and the two
// solvers get a SIMD each, and every SIMD also runs one loader. Every global
// load is issued as soon as its registers are free and consumed one chunk
// (with four blocks two chunk steps) later; loads are never conditional (the
// last chunk is fetched again), so the compiler keeps no copy at the loop
// latch.
// K, Q, V, T, M and a are double-buffered in LDS; K^T and the columns of V
// are read with ds_read_b64_tr_b16 straight from the row-major tiles.
template <typename CT, int D, int C, int BV>
struct __attribute__((aligned(16))) PipeSmem {
  static constexpr int NB = C / 16;
  // Row strides: on gfx950 the 16-byte fragment reads and the transposed
  // 8-byte reads of a tile are free of bank conflicts when the row stride is
  // 32 bytes modulo 64 (measured: an odd multiple of 32 bytes halves their
  // LDS cycles against the other strides). The column permutation acts
  // inside 32-column blocks, so permuted rows hold at least 32 positions.
  static constexpr int RP = 32 / (int)sizeof(CT);
  static constexpr int DP = (D < 32 ? 32 : D) + RP;
  static constexpr int CP = (C < 32 ? 32 : C) + RP;
  static constexpr int VS = BV + ((32 - (int)sizeof(CT) * BV % 64 + 64) % 64) / (int)sizeof(CT);
  static constexpr int TDS = 32 / (int)sizeof(CT) + (sizeof(CT) == 4 ? 16 : 0);  // 32 or 96 bytes
  struct Buf {
    CT K[C][DP];       // keys, row-major (column-permuted for bf16, d = 16)
    CT Q[C][DP];       // queries, likewise
    CT V[C][VS];       // value slice, natural layout
    CT T[C][CP];       // (I + A)^{-1}, permuted; only the lower block triangle is read
    CT M[C][CP];       // lower-incl-diag(Q K^T), permuted; only J <= I blocks are read
    float alpha[C];
  } buf[2];
  CT An[2][C][CP];        // -(K K^T) blocks below the diagonal, permuted, one copy per solver
  float Adt[NB][17][20];  // fp32 diagonal blocks of A, transposed; the 17th row
                          // staggers the blocks over the LDS banks
  CT Td[NB][16][TDS];     // (I + A_bb)^{-1}, transposed: row c holds column c
};

template <typename CT, int D, int C, int BV>
constexpr size_t pipe_smem_bytes() {
  return sizeof(PipeSmem<CT, D, C, BV>);
}

// Gram tiles below the diagonal blocks and lower-incl-diag Q K^T tiles,
// enumerated (I, J) row by row.
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

// Column tile m of T goes to solver 0 when it is the first or (with four
// tiles) the last one, else to solver 1: with NB = 4 the dependent chains are
// 3 + 0 and 2 + 1 block steps.
template <int NB>
__host__ __device__ constexpr int t_owner(int m) {
  return NB == 4 ? ((m == 0 || m == 3) ? 0 : 1) : (m == 0 ? 0 : 1);
}
template <int NB>
__host__ __device__ constexpr int t_first(int pw) {
  int f = NB;
  for (int m = NB - 1; m >= 0; --m)
    if (t_owner<NB>(m) == pw) f = m;
  return f;
}


// Loader waves of a pass mode: the segment summaries (mode 1) form no M, so
// two loaders serve them and the other waves hold state columns.
template <int PM>
constexpr int pipe_loaders() {
  return PM == 1 ? 2 : 4;
}

// The pipelined chunk pass of one workgroup: L is its index among the
// workgroups of the pass (head-major, column slices adjacent).
template <typename CT, int D, int C, int BV, int NSW, int PM, bool GATED = false>
__device__ __forceinline__ void pipe_body(const ChunkedArgs& a, PipeSmem<CT, D, C, BV>& sm, const int L) {
  using MM = Mma<CT>;
  using Frag = typename MM::Frag;
  using Vec = typename Vec16<CT>::type;
  using Sm = PipeSmem<CT, D, C, BV>;
  constexpr int NB = C / 16;
  constexpr int NKT = D / 16;
  constexpr int NVT = BV / 16;
  // Pass mode PM: 0 outputs (one pass, or one segment of a time-segmented
  // pass); 1 segment summaries, no outputs: the first half of the state waves
  // runs the slice's columns from S = I with zero values (the segment's
  // transition), the second half from S = 0 with the values (its offset),
  // both on one prep of the keys; 2 chunk-start states for the backward, no
  // outputs; 3 outputs and the chunk-start states (the forward of a training
  // step, whose backward then skips its own state pass). All compile-time.
  constexpr bool SUMMARY = PM == 1;
  constexpr bool SAVE = PM == 2 || PM == 3;
  constexpr bool outs = PM == 0 || PM == 3;
  // negated form (state N = -S, T' = -T diag(a) from the solvers) where the
  // state is not stored every chunk; the state-saving passes keep S and
  // apply a in the state waves, so their stores need no sign flips
  constexpr bool NEG = !SAVE;
  // the query fragments of the output products are requested in phase A,
  // except with outputs and state saving together (pass mode 3), whose plain
  // state form holds more registers there, and in the gated pass: then in
  // phase B, before their use
  constexpr bool QA = outs && NEG && !GATED;
  constexpr int NSP = SUMMARY ? NSW / 2 : NSW;  // state waves per column set
  constexpr int SW = NSP < NVT ? NSP : NVT;  // state waves holding columns
  constexpr int CPW = NVT / SW;              // 16-column tiles per state wave
  constexpr int VE = 16 / sizeof(CT);
  constexpr int NFK = NFrag<CT, NKT>::value;
  constexpr int NFB = NFrag<CT, NB>::value;
  constexpr int LDK = Sm::DP;
  constexpr int LDV = Sm::VS;
  constexpr int NST = 64 * NSW;  // state-group threads
  // Key order of the state rows. bf16 MFMA operands take 8 k values per lane
  // in the order (4 rows of accumulator tile 2f, 4 rows of tile 2f + 1), so
  // a state tile feeds the next product straight from its registers only if
  // the keys it multiplies come in that same order. With d >= 32 the state
  // row r holds key pcol(r) (a permutation inside each 32-key block): the K
  // and Q tiles can then stay in natural column order in LDS, staged with
  // whole 16-byte stores, and K^T is read transposed at pcol-mapped
  // addresses. With d = 16 (one 16-row tile) pcol is no permutation of the
  // keys; there the state rows are natural and K, Q are stored permuted. The
  // state-saving passes (modes 2, 3) keep natural rows as well: they store
  // the state every chunk, and the permuted store addresses cost them the
  // register that keeps the pass without spills.
  constexpr bool SROWP = sizeof(CT) == 2 && D >= 32 && !SAVE;
#define skey(r) (SROWP ? MM::pcol(r) : (r))
  // Where the chunk has four 16-row blocks (bf16, C = 64, d >= 32), each
  // loader fetches the key rows of its blocks straight into MFMA operand
  // layout: block L for loader L of the four, blocks L and L + 2 for the
  // summaries' two loaders. It then forms, one chunk ahead, the gate of those
  // rows and the diagonal Gram blocks a_r (K_b K_b^T)_{rc}, c < r, and leaves
  // them in LDS: the solvers' phase A starts at the forward substitution,
  // with no key fetch, no Gram product and no LDS round trip of their own.
  constexpr bool LGRAM = sizeof(CT) == 2 && NB == 4 && D >= 32;
  // With four 16-row blocks and outputs, the solvers form row block 3 of
  // M = tril(Q K^T): their key fragments of blocks 0..3 are in registers
  // for the Gram tiles, so each adds only the query fragments of block 3
  // and two tiles, and the loaders keep the six tiles of rows 0..2.
  constexpr bool SM3 = outs && NB == 4;
  constexpr int NQKL = SM3 ? 6 : PrepJobs<NB>::NQK;  // Q K^T jobs the loaders form
  // GATED (outputs pass, bf16, four 16-row blocks): per-token decays
  // g = exp(log_g), S_t = g_t (I - c k k^T) S_{t-1} + c k v^T. With b_r the
  // chunk's log-decays summed over rows 0..r, Gamma_r = exp(b_r) and
  // E_rs = exp(b_r - b_s):
  //   A    = strictly-lower(diag(c) K K^T * E)   (loaders: diagonal blocks;
  //                                               solvers: the tiles below)
  //   M    = lower-incl-diag(Q K^T) * E
  //   Y    = V + diag(Gamma) K N,  -U' = T' Y     (N = -S, T' = -T diag(c))
  //   -O^T = N^T Q^T diag(Gamma) + (-U')^T M^T
  //   N   <- Gamma_C N + K^T diag(Gamma_C / Gamma) (-U')
  // The loaders form b, Gamma and Gamma_C / Gamma = exp(b_C - b) of a chunk
  // with its gate, two chunk steps before its state pass, and leave them in
  // a three-slot table in LDS. E is formed per element where the recurrence
  // carries it (never as a ratio), so no log-decay overflows it.
  static_assert(!GATED || (PM == 0 && LGRAM && SROWP && SM3), "gated pipelined pass");
  // the table lives in rows 0..31 of solver 1's Gram-tile copy, which that
  // solver never touches (its tiles (i, j) have i > j >= 1)
  static_assert(!GATED || (t_first<NB>(1) >= 1 && 9 * C * 4 <= 32 * Sm::CP * (int)sizeof(CT)), "decay table");
  float* const gdec = (float*)&sm.An[1][0][0];
  // [b | Gamma | Gamma_C / Gamma] of a chunk
  auto gslot = [&](int chunk) { return gdec + (chunk % 3) * (3 * C); };
  // tile (I, J) in accumulator layout (lane (g, li): row r = 16 I + li,
  // columns s = 16 J + 4g + e) times E_rs, zero above the diagonal (or on it
  // when STRICT); gb is the chunk's b
  auto decay_tile = [&](const float* gb, int I, int J, floatx4 v, auto strictc) {
    constexpr bool STRICT = decltype(strictc)::value;
    const int ln = lane_id() & 15, gg = lane_id() >> 4;
    const int r = 16 * I + ln, s0 = 16 * J + 4 * gg;
    const float br = gb[r];
    const floatx4 bs = *(const floatx4*)&gb[s0];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool keep = STRICT ? (s0 + e < r) : (s0 + e <= r);
      v[e] = keep ? v[e] * __expf(br - bs[e]) : 0.f;
    }
    return v;
  };
  static_assert(NVT % SW == 0 && NB <= 4 && C % 16 == 0 && D % 16 == 0, "tile sizes");
  static_assert(!SUMMARY || NSW % 2 == 0, "summary state waves come in pairs");
  static_assert((Sm::DP * sizeof(CT)) % 64 == 32 && (Sm::CP * sizeof(CT)) % 64 == 32 &&
                    (Sm::VS * sizeof(CT)) % 64 == 32 && (Sm::TDS * sizeof(CT)) % 64 == 32,
                "row strides");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave-uniform (scalar), so role dispatch compiles to scalar branches
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // 0..NSW-1 state, then 2 solvers, the loaders
  const int li = lane & 15;
  const int g = lane >> 4;

  const int vh = L / a.nvt;  // virtual head
  const int v0 = (L % a.nvt) * BV;
  int hd = vh, t_begin = 0, T = a.T;
  // the transition half of the summary state waves (wave-uniform)
  const bool ident = SUMMARY && w < NSP;
  const float* s0p = a.s0 ? a.s0 + (size_t)hd * D * D : nullptr;
  float* sfp = a.s_final ? a.s_final + (size_t)hd * D * D : nullptr;
  if constexpr (SUMMARY) {
    // segments 1 .. nseg - 2 (whole segments), summary j = segment j + 1
    const int j = vh % a.nrun;
    hd = vh / a.nrun;
    t_begin = (j + 1) * a.seg_len;
    T = a.seg_len;
    s0p = nullptr;
    sfp = a.seg_out + ((size_t)(hd * a.nrun + j) * 2 + (ident ? 1 : 0)) * D * D;
  } else if (a.mode == 2) {
    // segments seg_first .. seg_first + nrun - 1; segment 0 starts from S0
    // and leaves its end state as the start of segment 1, the last segment
    // writes S_T
    const int sg = a.seg_first + vh % a.nrun;
    hd = vh / a.nrun;
    t_begin = sg * a.seg_len;
    T = min(a.seg_len, a.T - t_begin);
    s0p = sg == 0 ? (a.s0 ? a.s0 + (size_t)hd * D * D : nullptr)
                  : a.seg_s0 + (size_t)(hd * a.nseg + sg) * D * D;
    sfp = sg == a.nseg - 1 ? (a.s_final ? a.s_final + (size_t)hd * D * D : nullptr)
                           : (sg == 0 ? a.seg_s0 + (size_t)(hd * a.nseg + 1) * D * D : nullptr);
  }
  const size_t tok0 = (size_t)hd * a.T + t_begin;  // first token of this sequence piece
  const int nchunks = (T + C - 1) / C;

  if (w < NSW) {
    // ======================= state waves =======================
    const int wl = SUMMARY ? w % NSP : w;  // wave within its column set
    const bool owner = wl < SW;
    floatx4 sacc[CPW][NKT];
#pragma unroll
    for (int c = 0; c < CPW; ++c)
#pragma unroll
      for (int rt = 0; rt < NKT; ++rt) sacc[c][rt] = floatx4{0.f, 0.f, 0.f, 0.f};
    if (owner && s0p) {
#pragma unroll
      for (int c = 0; c < CPW; ++c)
#pragma unroll
        for (int rt = 0; rt < NKT; ++rt)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            sacc[c][rt][e] = NEG ? -s0p[(size_t)skey(16 * rt + 4 * g + e) * D + v0 + 16 * (wl * CPW + c) + li]
                                 : s0p[(size_t)skey(16 * rt + 4 * g + e) * D + v0 + 16 * (wl * CPW + c) + li];
    }
    if (SUMMARY && owner && ident) {
#pragma unroll
      for (int c = 0; c < CPW; ++c)
#pragma unroll
        for (int rt = 0; rt < NKT; ++rt)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            sacc[c][rt][e] = (skey(16 * rt + 4 * g + e) == v0 + 16 * (wl * CPW + c) + li) ? -1.f : 0.f;
    }
#pragma unroll
    for (int c = 0; c < CPW; ++c)
#pragma unroll
      for (int rt = 0; rt < NKT; ++rt) asm volatile("" : "+v"(sacc[c][rt]));

    __syncthreads();  // a of the first chunk
    for (int c = -1; c < nchunks; ++c) {
      const bool act = c >= 0 && owner;
      const auto& B = sm.buf[c & 1];
      floatx4 oacc[CPW][NB];
      Frag sf[CPW][NFK], uf[CPW][NFB], kt[NKT][NFB], qf[NB][NFK];
      const float* gb = GATED && act ? gslot(c) : nullptr;
      // ---- phase A: Y = V + K N; -U' = T' Y (T' of this chunk is ready one
      //      phase early). The K, V and T' fragments are requested first, the
      //      Q fragments (for phase B) while the K N products run
      if (act) {
        if constexpr (SAVE) {
          // lane (g, li) holds rows 16 rt + 4g .. + 3 of one column: 4
          // contiguous elements of the transposed state, stored as bf16 where
          // the backward takes them only as bf16 MFMA operands (bf16 inputs,
          // C and d multiples of 32), else as fp32
          constexpr bool SBF = sizeof(CT) == 2 && C % 32 == 0 && D % 32 == 0;
          float* dst = a.s_chunks + ((size_t)hd * nchunks + c) * D * D;
          bf16* dsb = (bf16*)a.s_chunks + ((size_t)hd * nchunks + c) * D * D;
          float* dsn = a.s_chunks_n + ((size_t)hd * nchunks + c) * D * D;
#pragma unroll
          for (int cc = 0; cc < CPW; ++cc)
#pragma unroll
            for (int rt = 0; rt < NKT; ++rt) {
              const int col = v0 + 16 * (wl * CPW + cc) + li;
              // rows 16 rt + 4g + e, e = 0..3: 4 consecutive keys (the saving
              // passes keep the state rows in natural key order)
              static_assert(!SROWP, "saving passes keep natural state rows");
              if constexpr (SBF) *(bf16x4*)&dsb[(size_t)col * D + 16 * rt + 4 * g] = Mma<bf16>::cvt4(sacc[cc][rt]);
              else *(floatx4*)&dst[(size_t)col * D + 16 * rt + 4 * g] = sacc[cc][rt];
              if (a.s_chunks_n) {
#pragma unroll
                for (int e = 0; e < 4; ++e) dsn[(size_t)(16 * rt + 4 * g + e) * D + col] = sacc[cc][rt][e];
              }
            }
        }
#pragma unroll
        for (int cc = 0; cc < CPW; ++cc)
#pragma unroll
          for (int f = 0; f < NFK; ++f) sf[cc][f] = MM::template acc<NKT>(sacc[cc], f);
        if constexpr (GATED) {
          // N <- Gamma_C N + ...: the decay of the carried state, applied
          // once its fragments for this chunk are formed
          const float gC = gb[2 * C - 1];
#pragma unroll
          for (int cc = 0; cc < CPW; ++cc)
#pragma unroll
            for (int rt = 0; rt < NKT; ++rt) sacc[cc][rt] = sacc[cc][rt] * gC;
        }
        Frag kf[NB][NFK];
        floatx4 al[NB], y[CPW][NB];
        // the value columns stay in their storage type until Y: converting
        // them here would make the wave wait for every read before the first
        // product (a transition run ignores them: its value buffer holds keys)
        std::conditional_t<sizeof(CT) == 2, bf16x4, floatx4> vraw[CPW][NB];
#pragma unroll
        for (int ut = 0; ut < NB; ++ut)
#pragma unroll
          for (int f = 0; f < NFK; ++f) kf[ut][f] = MM::template ldp<NKT>(&B.K[16 * ut + li][0], f);
#pragma unroll
        for (int ut = 0; ut < NB; ++ut) {
          if constexpr (!NEG) al[ut] = *(const floatx4*)&B.alpha[16 * ut + 4 * g];
          if constexpr (!GATED) {
#pragma unroll
            for (int cc = 0; cc < CPW; ++cc) vraw[cc][ut] = ldtr4(&B.V[0][0], LDV, 16 * ut + 4 * g, 16 * (wl * CPW + cc));
          }
        }
        // T of this chunk is ready since phase B of the previous one: its
        // fragments are requested now so T Y finds them in registers
        Frag tf[NB][NFB];
        static_for<NB>([&](auto ub) {
          constexpr int ut = decltype(ub)::value;
#pragma unroll
          for (int f = 0; f < NFrag<CT, ut + 1>::value; ++f) tf[ut][f] = MM::template ldps<ut + 1>(&B.T[16 * ut + li][0], f);
        });
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ut = 0; ut < NB; ++ut) {
          // negated form: Y = V - K S = V + K N, with the values as the
          // accumulator's start; else Y = diag(a) (V - K S)
#pragma unroll
          for (int cc = 0; cc < CPW; ++cc)
            y[cc][ut] = (!NEG || (SUMMARY && ident) || GATED) ? floatx4{0.f, 0.f, 0.f, 0.f} : to_f32x4(vraw[cc][ut]);
#pragma unroll
          for (int f = 0; f < NFK; ++f) {
#pragma unroll
            for (int cc = 0; cc < CPW; ++cc) y[cc][ut] = MM::mma(y[cc][ut], kf[ut][f], sf[cc][f]);
            if constexpr (QA) qf[ut][f] = MM::template ldp<NKT>(&B.Q[16 * ut + li][0], f);
          }
          if constexpr (!NEG) {
#pragma unroll
            for (int cc = 0; cc < CPW; ++cc) y[cc][ut] = al[ut] * (to_f32x4(vraw[cc][ut]) - y[cc][ut]);
          }
          if constexpr (GATED) {
            // Y = V + diag(Gamma) K N: rows 4g + e of tile ut are tokens
            // 16 ut + 4g + e (the value columns are read here: kept from the
            // start of the phase they would cost the registers of a spill)
            const floatx4 gm = *(const floatx4*)&gb[C + 16 * ut + 4 * g];
#pragma unroll
            for (int cc = 0; cc < CPW; ++cc)
              y[cc][ut] = to_f32x4(ldtr4(&B.V[0][0], LDV, 16 * ut + 4 * g, 16 * (wl * CPW + cc))) + gm * y[cc][ut];
          }
        }
        Frag yf[CPW][NFB];
#pragma unroll
        for (int cc = 0; cc < CPW; ++cc)
#pragma unroll
          for (int f = 0; f < NFB; ++f) yf[cc][f] = MM::template acc<NB>(y[cc], f);
        __builtin_amdgcn_sched_barrier(0);
        floatx4 u[CPW][NB];
        static_for<NB>([&](auto ub) {
          constexpr int ut = decltype(ub)::value;
#pragma unroll
          for (int cc = 0; cc < CPW; ++cc) u[cc][ut] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int f = 0; f < NFrag<CT, ut + 1>::value; ++f) {
#pragma unroll
            for (int cc = 0; cc < CPW; ++cc) u[cc][ut] = MM::mma(u[cc][ut], tf[ut][f], yf[cc][f]);
          }
        });
#pragma unroll
        for (int cc = 0; cc < CPW; ++cc)
#pragma unroll
          for (int f = 0; f < NFB; ++f) uf[cc][f] = MM::template acc<NB>(u[cc], f);
        // T Y only reads registers once its fragments are in, so the
        // compiler would sink it below the barrier into phase B; consuming
        // U' here keeps it in phase A
#pragma unroll
        for (int cc = 0; cc < CPW; ++cc)
#pragma unroll
          for (int f = 0; f < NFB; ++f) asm volatile("" : "+v"(uf[cc][f]));
      }
      __syncthreads();
      // ---- phase B: O^T = S^T Q^T (S before this chunk's update, Q from
      //      phase A), each row block followed by the requests for its share
      //      of K^T fragments; S += K^T U'; O^T += U'^T M^T; store O. M
      //      fragments while K^T U' runs
      if (act) {
        static_for<NB>([&](auto ub) {
          constexpr int ut = decltype(ub)::value;
          if constexpr (outs) {
            if constexpr (!QA) {
#pragma unroll
              for (int f = 0; f < NFK; ++f) qf[ut][f] = MM::template ldp<NKT>(&B.Q[16 * ut + li][0], f);
            }
            // register-only products would otherwise be hoisted above the
            // barrier; tying their inputs to this point keeps them in phase B
#pragma unroll
            for (int f = 0; f < NFK; ++f) asm volatile("" : "+v"(qf[ut][f]));
#pragma unroll
            for (int cc = 0; cc < CPW; ++cc) oacc[cc][ut] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int f = 0; f < NFK; ++f) {
#pragma unroll
              for (int cc = 0; cc < CPW; ++cc) oacc[cc][ut] = MM::mma(oacc[cc][ut], sf[cc][f], qf[ut][f]);
            }
            if constexpr (GATED) {
              // column li of O^T tile ut is token 16 ut + li: N^T Q^T diag(Gamma)
              const float gm = gb[C + 16 * ut + li];
#pragma unroll
              for (int cc = 0; cc < CPW; ++cc) oacc[cc][ut] = oacc[cc][ut] * gm;
              // this row tile's outputs now: O^T += (-U')^T M^T with -U' as
              // formed (it is scaled for the state update afterwards), then
              // the store; one tile's M fragments are live at a time
              Frag mf[NFrag<CT, ut + 1>::value];
#pragma unroll
              for (int f = 0; f < NFrag<CT, ut + 1>::value; ++f) mf[f] = MM::template ldps<ut + 1>(&B.M[16 * ut + li][0], f);
#pragma unroll
              for (int f = 0; f < NFrag<CT, ut + 1>::value; ++f) {
#pragma unroll
                for (int cc = 0; cc < CPW; ++cc) oacc[cc][ut] = MM::mma(oacc[cc][ut], uf[cc][f], mf[f]);
              }
              if (16 * ut + li < min(C, T - c * C)) {
                CT* orow = (CT*)a.o + (tok0 + (size_t)c * C + 16 * ut + li) * D + v0 + 4 * g;
#pragma unroll
                for (int cc = 0; cc < CPW; ++cc) store4(orow + 16 * (wl * CPW + cc), -oacc[cc][ut]);
              }
            }
          }
#pragma unroll
          for (int rt = ut * NKT / NB; rt < (ut + 1) * NKT / NB; ++rt)
#pragma unroll
            for (int f = 0; f < NFB; ++f) kt[rt][f] = tr_frag<NB, true>(&B.K[0][0], LDK, f, 16 * rt);
        });
        if constexpr (GATED) {
          // -U' with row r scaled in place by Gamma_C / Gamma_r =
          // exp(b_C - b_r) (elements 0..3 of fragment f are rows
          // 32 f + 4g + e, elements 4..7 rows 32 f + 16 + 4g + e), then the
          // state update
          static_assert(2 * NFB == NB && NEG, "whole fragments, negated form");
#pragma unroll
          for (int f = 0; f < NFB; ++f) {
            const floatx4 d0 = *(const floatx4*)&gb[2 * C + 32 * f + 4 * g];
            const floatx4 d1 = *(const floatx4*)&gb[2 * C + 32 * f + 16 + 4 * g];
#pragma unroll
            for (int cc = 0; cc < CPW; ++cc) {
              const Frag x = uf[cc][f];
              const floatx4 lo = __builtin_convertvector(__builtin_shufflevector(x, x, 0, 1, 2, 3), floatx4);
              const floatx4 hi = __builtin_convertvector(__builtin_shufflevector(x, x, 4, 5, 6, 7), floatx4);
              uf[cc][f] = MM::cat(MM::cvt4(lo * d0), MM::cvt4(hi * d1));
            }
          }
#pragma unroll
          for (int rt = 0; rt < NKT; ++rt)
#pragma unroll
            for (int f = 0; f < NFB; ++f)
#pragma unroll
              for (int cc = 0; cc < CPW; ++cc) sacc[cc][rt] = MM::mma(sacc[cc][rt], kt[rt][f], uf[cc][f]);
        } else {
        Frag mf[NB][NFB];
#pragma unroll
        for (int rt = 0; rt < NKT; ++rt) {
#pragma unroll
          for (int f = 0; f < NFB; ++f) {
#pragma unroll
            for (int cc = 0; cc < CPW; ++cc) sacc[cc][rt] = MM::mma(sacc[cc][rt], kt[rt][f], uf[cc][f]);
          }
          if (outs && rt < NB) {  // constant after unrolling
            static_for<NB>([&](auto ub) {
              constexpr int ut = decltype(ub)::value;
              if (ut == rt) {
#pragma unroll
                for (int f = 0; f < NFrag<CT, ut + 1>::value; ++f) mf[ut][f] = MM::template ldps<ut + 1>(&B.M[16 * ut + li][0], f);
              }
            });
          }
        }
        if constexpr (outs) {
        static_for<NB>([&](auto ub) {  // row tiles past the K^T loop (NKT < NB)
          constexpr int ut = decltype(ub)::value;
          if constexpr (ut >= NKT) {
#pragma unroll
            for (int f = 0; f < NFrag<CT, ut + 1>::value; ++f) mf[ut][f] = MM::template ldps<ut + 1>(&B.M[16 * ut + li][0], f);
          }
        });
        static_for<NB>([&](auto ub) {
          constexpr int ut = decltype(ub)::value;
#pragma unroll
          for (int f = 0; f < NFrag<CT, ut + 1>::value; ++f) {
#pragma unroll
            for (int cc = 0; cc < CPW; ++cc) oacc[cc][ut] = MM::mma(oacc[cc][ut], uf[cc][f], mf[ut][f]);
          }
        });
        // lane (g, li) holds columns 4g..4g+3 of token row 16 ut + li of its
        // 16-column tile: 4 contiguous outputs, a 32-byte row segment per tile
        const int nval = min(C, T - c * C);
        CT* orow = (CT*)a.o + (tok0 + (size_t)c * C + li) * D + v0 + 4 * g;
#pragma unroll
        for (int ut = 0; ut < NB; ++ut)
          if (16 * ut + li < nval) {
#pragma unroll
            for (int cc = 0; cc < CPW; ++cc)
              store4(orow + (size_t)16 * ut * D + 16 * (wl * CPW + cc), NEG ? -oacc[cc][ut] : oacc[cc][ut]);
          }
        }
        }
      }
      __syncthreads();
    }
    if (owner && sfp) {
      float* sf = sfp;
#pragma unroll
      for (int cc = 0; cc < CPW; ++cc)
#pragma unroll
        for (int rt = 0; rt < NKT; ++rt)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            sf[(size_t)skey(16 * rt + 4 * g + e) * D + v0 + 16 * (wl * CPW + cc) + li] = NEG ? -sacc[cc][rt][e] : sacc[cc][rt][e];
    }
  } else if (w < NSW + 2) {
    // ======================= solvers (prep waves 0, 1) =======================
    const int pw = w - NSW;
    const CT* kg = (const CT*)a.k + tok0 * D;
    auto solver = [&](auto pwc) {
      constexpr int PW = decltype(pwc)::value;
      constexpr int NDB = NB > PW ? (NB - PW + 1) / 2 : 0;  // diagonal blocks PW, PW + 2
      // Rows of the diagonal blocks in MFMA operand layout, straight from
      // HBM: lane (g, li) holds row 16 b + li, 16-byte pieces at columns
      // 32 f + 8 g (bf16) or 16 f + 4 g (fp32). Both Gram operands are these
      // same registers, so the k order only has to be consistent.
      constexpr int NPC = sizeof(CT) == 2 ? (D + 31) / 32 : D / 16;  // pieces per row
      constexpr int PST = sizeof(CT) == 2 ? 32 : 16;                 // column stride of pieces
      Vec kd[NDB > 0 ? NDB : 1][NPC];
      // rows past T are clamped here; their a is zero
      auto load_rows = [&](int chunk) {
        const int t0 = chunk * C;
#pragma unroll
        for (int i = 0; i < NDB; ++i) {
          const int t = min(t0 + 16 * (PW + 2 * i) + li, T - 1);
#pragma unroll
          for (int f = 0; f < NPC; ++f) {
            const int col = PST * f + VE * g;
            if (col < D) kd[i][f] = *(const Vec*)(kg + (size_t)t * D + col);
            else kd[i][f] = Vec{};
          }
        }
      };
      if constexpr (NDB > 0 && !LGRAM) load_rows(0);
      // blocks of this solver's An copy left of its first column tile are
      // never computed; they are read only against zero blocks of X, so they
      // must hold zeros, not stale bits
      if constexpr (t_first<NB>(PW) > 0 && t_first<NB>(PW) < NB) {
        // (only rows of blocks below its first column tile are ever read)
        constexpr int R0 = 16 * (t_first<NB>(PW) + 1);
        constexpr int NZ = (int)(sizeof(CT) * (C - R0) * Sm::CP / 16);
        floatx4* z = (floatx4*)&sm.An[PW][R0][0];
        for (int i = lane; i < NZ; i += 64) z[i] = floatx4{0.f, 0.f, 0.f, 0.f};
      }
      __syncthreads();  // a of the first chunk

      for (int c = -1; c < nchunks; ++c) {
        const int n = c + 1;  // chunk being prepared
        const bool act = n < nchunks;
        auto& B = sm.buf[n & 1];
        int li = lane & 15, g = lane >> 4;
        asm volatile("" : "+v"(li), "+v"(g));
        // ---- phase A: (I + A_bb)^{-1} for the diagonal blocks (a of this
        //      chunk was written by the loaders one chunk ahead; it is zero for
        //      rows past T, which clears their rows of A)
        if constexpr (NDB > 0) {
          if (act) {
           if constexpr (!LGRAM) {
            float al[NDB];
#pragma unroll
            for (int i = 0; i < NDB; ++i) al[i] = B.alpha[16 * (PW + 2 * i) + li];
            floatx4 dg[NDB];
#pragma unroll
            for (int i = 0; i < NDB; ++i) {
              dg[i] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
              for (int f = 0; f < NPC; ++f) dg[i] = MM::mma(dg[i], kd[i][f], kd[i][f]);
            }
            // the row registers are free again: fetch the next chunk's rows now,
            // so their latency is covered by the rest of this chunk (always
            // issued, the last chunk's again at the end: a conditional load
            // would make the compiler copy the registers at the loop latch and
            // wait there for every load in flight)
            load_rows(min(n + 1, nchunks - 1));
            // lane (g, li) holds G[4g + e][li] = G[li][4g + e]: row li of A_bb
            // is a_li G[li][c], c < li, stored transposed
#pragma unroll
            for (int i = 0; i < NDB; ++i) {
#pragma unroll
              for (int e = 0; e < 4; ++e)
                sm.Adt[PW + 2 * i][4 * g + e][li] = (4 * g + e < li) ? al[i] * dg[i][e] : 0.f;
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
           }
            if (g < NDB) {
              // column-parallel right-looking forward substitution in fp32:
              // lane group g = block PW + 2g, lane li = column li; once t_j is
              // final, column j is eliminated from the rows below. The
              // 4-groups of column j below the diagonal are read in two batches
              // (columns 0-6, then 7-14, issued after three elimination steps):
              // two LDS round trips instead of fifteen.
              const float* Ab = &sm.Adt[PW + 2 * g][0][0];
              floatx4 acol[15][4];
              float t[16];
#pragma unroll
              for (int j = 0; j < 7; ++j)
#pragma unroll
                for (int q4 = (j + 1) >> 2; q4 < 4; ++q4) acol[j][q4] = *(const floatx4*)&Ab[20 * j + 4 * q4];
#pragma unroll
              for (int r = 0; r < 16; ++r) t[r] = (r == li) ? 1.f : 0.f;
#pragma unroll
              for (int j = 0; j < 15; ++j) {
                if (j == 3) {
                  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                  for (int jj = 7; jj < 15; ++jj)
#pragma unroll
                    for (int q4 = (jj + 1) >> 2; q4 < 4; ++q4)
                      acol[jj][q4] = *(const floatx4*)&Ab[20 * jj + 4 * q4];
                  __builtin_amdgcn_sched_barrier(0);
                }
#pragma unroll
                for (int r = j + 1; r < 16; ++r) t[r] -= acol[j][r >> 2][r & 3] * t[j];
              }
              // lane li holds column li of the inverse: stored as row li of
              // its transpose, in 16-byte pieces (two LDS stores for bf16
              // instead of sixteen 2-byte ones)
              CT* Tb = &sm.Td[PW + 2 * g][li][0];
              constexpr int VE16 = 16 / (int)sizeof(CT);
#pragma unroll
              for (int p = 0; p < 16 / VE16; ++p) {
                Vec tv;
#pragma unroll
                for (int e = 0; e < VE16; ++e) tv[e] = from_f32<CT>(t[VE16 * p + e]);
                *(Vec*)&Tb[VE16 * p] = tv;
              }
            }
          }
        }
        __syncthreads();
        // ---- phase B: the Gram tiles below the diagonal that this solver's
        //      column tiles of T need (stored as -K K^T, unscaled: a is
        //      applied in the solve), then those column tiles:
        //        X_m = -(I + A_mm)^{-1} diag(a_m),
        //        X_i = (I + A_ii)^{-1} diag(a_i) sum_{m<=j<i} (-K_i K_j^T) X_j, i > m,
        //      the column tile m of T' = -T diag(a); X_i^T is formed too so T'
        //      is written row-major.
        constexpr int M0 = t_first<NB>(PW);
        if constexpr (M0 < NB) {
          if (act) {
            auto& An = sm.An[PW];
            // K row blocks M0.. read once into registers, then every Gram tile
            // (i, j), i > j >= M0, from them
            Frag kf[NB][NFK];
            static_for<NB>([&](auto ib) {
              constexpr int i = decltype(ib)::value;
              if constexpr (i >= M0) {
#pragma unroll
                for (int f = 0; f < NFK; ++f) kf[i][f] = MM::template ldp<NKT>(&B.K[16 * i + li][0], f);
              }
            });
            Frag q3[SM3 ? NFK : 1];
            if constexpr (SM3) {
              static_assert(t_first<NB>(0) == 0 && t_first<NB>(1) <= 2, "key blocks 2 PW, 2 PW + 1 in registers");
#pragma unroll
              for (int f = 0; f < NFK; ++f) q3[f] = MM::template ldp<NKT>(&B.Q[48 + li][0], f);
            }
            static_for<NB>([&](auto ib) {
              constexpr int i = decltype(ib)::value;
              static_for<i>([&](auto jb) {
                constexpr int j = decltype(jb)::value;
                if constexpr (j >= M0) {
                  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                  for (int f = 0; f < NFK; ++f) acc = MM::mma(acc, kf[j][f], kf[i][f]);
                  if constexpr (GATED) acc = decay_tile(gslot(n), i, j, acc, std::true_type{});
                  MM::store_tps(&An[16 * i + li][0], j, -acc);
                }
              });
            });
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            static_for<NB>([&](auto mb) {
              constexpr int m = decltype(mb)::value;
              if constexpr (t_owner<NB>(m) == PW) {
                floatx4 x[NB];
                static_for<NB>([&](auto ib) {
                  constexpr int i = decltype(ib)::value;
                  if constexpr (i >= m) {
                    floatx4 yv;
                    if constexpr (i == m) {
#pragma unroll
                      for (int e = 0; e < 4; ++e) yv[e] = (4 * g + e == li) ? 1.f : 0.f;
                    } else {
                      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                      for (int f = 0; f < NFrag<CT, i>::value; ++f) {
                        if constexpr (MM::KT == 2) {
                          if (2 * f + 1 < m) continue;  // both tiles of the fragment are zero
                        } else {
                          if (f < m) continue;
                        }
                        floatx4 xin[2] = {x[MM::KT * f],
                                          MM::KT == 2 && 2 * f + 1 < i ? x[2 * f + 1] : x[MM::KT * f]};
                        acc = MM::mma(acc, MM::template ldps<i>(&An[16 * i + li][0], f),
                                      MM::template acc<(MM::KT == 2 ? 2 : 1)>(xin, 0));
                      }
                      yv = *(const floatx4*)&B.alpha[16 * i + 4 * g] * acc;
                    }
                    // row li of (I + A_ii)^{-1}, columns 4g..4g+3, from the
                    // transposed store: one transposed read
                    Frag td{};
                    {
                      const auto t4 = ldtr4(&sm.Td[i][0][0], Sm::TDS, 4 * g, 0);
#pragma unroll
                      for (int e = 0; e < 4; ++e) td[e] = t4[e];
                    }
                    const Frag yf = MM::template acc<1>(&yv, 0);
                    x[i] = MM::mma(floatx4{0.f, 0.f, 0.f, 0.f}, td, yf);
                    floatx4 xt = MM::mma(floatx4{0.f, 0.f, 0.f, 0.f}, yf, td);
                    if constexpr (i == m && NEG) {
                      // T' = -T diag(a) for the negated form of the state
                      // pass: the columns of tile m are scaled by -a in fp32
                      // here; the tiles below inherit it through the solve,
                      // which is linear in X_m
                      const float ac = -B.alpha[16 * m + li];
                      const floatx4 ar = -*(const floatx4*)&B.alpha[16 * m + 4 * g];
                      x[i] = x[i] * ac;
                      xt = xt * ar;
                    }
                    MM::store_tps(&B.T[16 * i + li][0], m, xt);
                  } else {
                    x[i] = floatx4{0.f, 0.f, 0.f, 0.f};
                  }
                });
              }
            });
            if constexpr (SM3) {
              // tiles (3, 2 PW) and (3, 2 PW + 1) of M, lower-incl-diagonal;
              // the same fragments and product order as the loaders' tiles
              static_for<2>([&](auto tc) {
                constexpr int J = 2 * PW + decltype(tc)::value;
                floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int f = 0; f < NFK; ++f) acc = MM::mma(acc, kf[J][f], q3[f]);
                if constexpr (GATED) {
                  acc = decay_tile(gslot(n), 3, J, acc, std::false_type{});
                } else if constexpr (J == 3) {
#pragma unroll
                  for (int e = 0; e < 4; ++e) acc[e] = (4 * g + e <= li) ? acc[e] : 0.f;
                }
                MM::store_tps(&B.M[48 + li][0], J, acc);
              });
            }
          }
        }
        __syncthreads();
      }
    };
    if (pw == 0) solver(std::integral_constant<int, 0>{});
    else solver(std::integral_constant<int, 1>{});
  } else {
    // ======================= loaders (prep waves 2, 3) =======================
    const int lt = tid - NST - 128;  // loader thread
    const CT* kg = (const CT*)a.k + tok0 * D;
    // without outputs the queries are not needed: those loads read the key
    // rows instead (same lines, no extra HBM traffic; measured, skipping
    // them altogether made the state-saving pass slower) and are not used
    const CT* qg = outs ? (const CT*)a.q + tok0 * D : kg;
    const CT* vg = (const CT*)a.v + tok0 * D;
    constexpr int NLT = 64 * pipe_loaders<PM>();
    constexpr int VPR = D / VE;
    constexpr int VPRV = BV / VE;
    constexpr int NLK = (C * VPR + NLT - 1) / NLT;
    constexpr int NLV = (C * VPRV + NLT - 1) / NLT;
    // every loader thread has a piece in every slot: the slot tests drop
    // out, so no load is conditional and the compiler's count of loads in
    // flight is exact (a test it cannot fold makes it wait for the most
    // recent requests as well)
    constexpr bool KFULL = NLT * NLK == C * VPR;
    constexpr bool VFULL = NLT * NLV == C * VPRV;
    const CT* bg = (const CT*)a.beta + tok0;
    Vec kreg[NLK], qreg[NLK], vreg[NLV];
    CT breg;
    // Loads go through buffer descriptors that start at the chunk's first
    // token and end with this sequence piece: rows past T read as zeros, so
    // the ragged tail needs no clamping and no masking. The per-lane byte
    // offsets are the same for every chunk.
    auto chunk_rsrc = [&](const CT* base, int chunk, int col0) {
      const long long tok = (long long)chunk * C;
      return buf_rsrc(base + tok * D + col0, ((long long)(T - tok) * D - col0) * (long long)sizeof(CT));
    };
    unsigned koff[NLK], voff[NLV];
#pragma unroll
    for (int j = 0; j < NLK; ++j) {
      const int idx = lt + NLT * j;
      koff[j] = (unsigned)(((idx / VPR) * D + (idx % VPR) * VE) * (int)sizeof(CT));
    }
#pragma unroll
    for (int j = 0; j < NLV; ++j) {
      const int idx = lt + NLT * j;
      voff[j] = (unsigned)(((idx / VPRV) * D + (idx % VPRV) * VE) * (int)sizeof(CT));
    }
    // Row-sum layout of the key slots: slot j, lane (q, p) = (lane / VPR,
    // lane % VPR) holds piece p of row (64 w' + NLT j) / VPR + q of this wave
    // w'. Lane (q, p < NLK) computes a for slot p's row q and loads its beta.
    const int lw = lt >> 6;        // loader wave
    const int lq = lane / VPR, lp = lane % VPR;
    const int arow = (64 * lw + NLT * lp) / VPR + lq;  // row of this lane's a (when lp < NLK)
    // coalesced 16-byte loads of one chunk
    auto load_k = [&](int chunk) {
      const auto rk = chunk_rsrc(kg, chunk, 0);
#pragma unroll
      for (int j = 0; j < NLK; ++j)
        if (KFULL || lt + NLT * j < C * VPR) buf_load(rk, koff[j], kreg[j]);
      const long long tok = (long long)chunk * C;
      buf_load(buf_rsrc(bg + tok, (long long)(T - tok) * (long long)sizeof(CT)),
               (unsigned)(min(arow, C - 1) * (int)sizeof(CT)), breg);
    };
    // lambda = ||k||^2 per row by a DPP row sum over the row's VPR lanes, then
    // a = -expm1(-beta lambda)/lambda for the chunk whose keys are in kreg, into
    // that chunk's buffer; zero for rows past T
    auto gate_rows = [&](int chunk, float* alpha) {
      float lam[NLK];
#pragma unroll
      for (int j = 0; j < NLK; ++j) lam[j] = group_sum<VPR>(sumsq(kreg[j]));
      float l = lam[0];
#pragma unroll
      for (int j = 1; j < NLK; ++j) l = lp == j ? lam[j] : l;
      const int nval = min(C, T - chunk * C);
      if (lp < NLK && arow < C) alpha[arow] = arow < nval ? gate_coef(a.coef, to_f32(breg), l) : 0.f;
    };
    auto load_qv = [&](int chunk) {
      const auto rq = chunk_rsrc(qg, chunk, 0);
      const auto rv = chunk_rsrc(vg, chunk, v0);
#pragma unroll
      for (int j = 0; j < NLK; ++j)
        if (KFULL || lt + NLT * j < C * VPR) buf_load(rq, koff[j], qreg[j]);
#pragma unroll
      for (int j = 0; j < NLV; ++j)
        if (VFULL || lt + NLT * j < C * VPRV) buf_load(rv, voff[j], vreg[j]);
    };
    auto loader = [&](auto pwc) {
      constexpr int PW = decltype(pwc)::value;  // loader 0..3
      using JB = PrepJobs<NB>;
      // Q K^T jobs of this wave, in the order of PrepJobs (jobs 0..5 of rows
      // 0..2 are tiles (0,0) (1,0) (1,1) (2,0) (2,1) (2,2)). The first of a
      // wave's jobs runs in phase A of the chunk's own state pass (its K and
      // Q were staged one phase before, the state reads M only in phase B);
      // the others one chunk ahead in phase B. With the solvers on row block
      // 3 (six jobs left), loaders 0 and 1, which share their SIMDs with the
      // state waves, form no tile: the state waves' products have those
      // SIMDs' MFMA pipes to themselves. Loaders 2 and 3 take (0,0), (1,1),
      // (2,1) and (1,0), (2,0), (2,2), the first in phase A (measured, same
      // box: 1.3B layer 149 -> 141 us, 340M layer 73 -> 68 us against one
      // tile per loader). Otherwise jobs PW, PW + 4, ... with the first in
      // phase A except on loaders 2 and 3 next to the solvers' row block 3.
      constexpr bool XJ = NQKL == 6 && outs;
      constexpr int NJ = XJ ? (PW < 2 ? 0 : 3) : (NQKL > PW ? (NQKL - PW + 3) / 4 : 0);
      auto ljob = [](int t) constexpr { return XJ ? PW - 2 + 2 * t : PW + 4 * t; };
      constexpr int NA = XJ ? (PW < 2 ? 0 : 1) : ((outs && NJ > 0 && !(SM3 && PW >= 2)) ? 1 : 0);
      // jobs [J0, J1) of this wave on buffer Bm: every fragment first, then
      // the products (one exposed LDS round trip)
      auto mtiles = [&](auto& Bm, auto j0c, auto j1c, const float* gb) {
        constexpr int J0 = decltype(j0c)::value, J1 = decltype(j1c)::value;
        if constexpr (outs && J1 > J0) {
          const int li = lane & 15, g = lane >> 4;
          Frag kfr[J1 - J0][NFK], qfr[J1 - J0][NFK];
          static_for<J1 - J0>([&](auto jc) {
            constexpr int j = JB::NOFF + ljob(J0 + decltype(jc)::value);
            constexpr int I = JB::I(j), J = JB::J(j);
#pragma unroll
            for (int f = 0; f < NFK; ++f) {
              kfr[decltype(jc)::value][f] = MM::template ldp<NKT>(&Bm.K[16 * J + li][0], f);
              qfr[decltype(jc)::value][f] = MM::template ldp<NKT>(&Bm.Q[16 * I + li][0], f);
            }
          });
          __builtin_amdgcn_sched_barrier(0);
          floatx4 acc[J1 - J0];
          static_for<J1 - J0>([&](auto jc) {
            acc[decltype(jc)::value] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int f = 0; f < NFK; ++f)
              acc[decltype(jc)::value] =
                  MM::mma(acc[decltype(jc)::value], kfr[decltype(jc)::value][f], qfr[decltype(jc)::value][f]);
          });
          static_for<J1 - J0>([&](auto jc) {
            constexpr int j = JB::NOFF + ljob(J0 + decltype(jc)::value);
            constexpr int I = JB::I(j), J = JB::J(j);
            floatx4 v = acc[decltype(jc)::value];
            if constexpr (GATED) {
              v = decay_tile(gb, I, J, v, std::false_type{});
            } else if constexpr (I == J) {
#pragma unroll
              for (int e = 0; e < 4; ++e) v[e] = (4 * g + e <= li) ? v[e] : 0.f;
            }
            MM::store_tps(&Bm.M[16 * I + li][0], J, v);
          });
        }
      };
      // LGRAM: this loader's blocks PW, PW + NLW, ... of key rows (one with
      // four loaders, two with the summaries' two) in MFMA operand layout:
      // lane (g, li) holds row 16 b + li of block b, 16-byte pieces at
      // columns 32 f + 8 g (the pieces' k order only has to agree between
      // the two Gram operands, which are these same registers), and that
      // row's beta
      const int li0 = lane & 15, g0 = lane >> 4;
      constexpr int NLW = pipe_loaders<PM>();
      constexpr int NKB = LGRAM ? NFK : 1;
      constexpr int NBL = LGRAM ? NB / NLW : 1;  // key blocks of this loader
      static_assert(!LGRAM || NB % NLW == 0, "key blocks per loader");
      static_assert(!GATED || NBL == 1, "gated pass: one key block per loader");
      unsigned kboff[NBL][NKB];
      if constexpr (LGRAM) {
#pragma unroll
        for (int i = 0; i < NBL; ++i)
#pragma unroll
          for (int f = 0; f < NFK; ++f)
            kboff[i][f] = (unsigned)(((16 * (PW + NLW * i) + li0) * D + 32 * f + 8 * g0) * (int)sizeof(CT));
      }
      if constexpr (LGRAM) {
        // Two register sets, each holding one chunk's keys (in the layout
        // above), betas, queries and values. A chunk's data is requested in
        // phase A two chunk steps before it is staged, and one and a half
        // before its gate and Gram block are formed from it.
        struct LB {
          Vec kb[NBL][NKB];
          CT kbeta[NBL];
          Vec q[NLK];
          Vec v[NLV];
          float lgv;  // gated: log-decay of the chunk's row `lane`
        };
        LB b0, b1;
        auto load_all = [&](LB& b, int chunk) {
          const auto rk = chunk_rsrc(kg, chunk, 0);
#pragma unroll
          for (int i = 0; i < NBL; ++i)
#pragma unroll
            for (int f = 0; f < NKB; ++f) buf_load(rk, kboff[i][f], b.kb[i][f]);
          const long long tok = (long long)chunk * C;
          const auto rb = buf_rsrc(bg + tok, (long long)(T - tok) * (long long)sizeof(CT));
#pragma unroll
          for (int i = 0; i < NBL; ++i) buf_load(rb, (unsigned)((16 * (PW + NLW * i) + li0) * (int)sizeof(CT)), b.kbeta[i]);
          const auto rq = chunk_rsrc(qg, chunk, 0);
          const auto rv = chunk_rsrc(vg, chunk, v0);
#pragma unroll
          for (int j = 0; j < NLK; ++j)
            if (KFULL || lt + NLT * j < C * VPR) buf_load(rq, koff[j], b.q[j]);
#pragma unroll
          for (int j = 0; j < NLV; ++j)
            if (VFULL || lt + NLT * j < C * VPRV) buf_load(rv, voff[j], b.v[j]);
          if constexpr (GATED)
            buf_load(buf_rsrc(a.log_g + tok0 + tok, (long long)(T - tok) * 4), (unsigned)(lane * 4), b.lgv);
        };
        // a of rows 16 b + li of `chunk` (zero past T) and the strictly
        // lower a_r G_rc of the Gram matrix of each of this loader's blocks
        // b, stored transposed for the solvers' column-parallel forward
        // substitution
        auto gate_gram = [&](LB& b, int chunk, float* alpha) {
#pragma unroll
         for (int i = 0; i < NBL; ++i) {
          const int blk = PW + NLW * i;
          float lam = 0.f;
#pragma unroll
          for (int f = 0; f < NKB; ++f) lam += sumsq(b.kb[i][f]);
          lam = xor32_sum(xor16_sum(lam));
          const int row = 16 * blk + li0;
          const float al = row < min(C, T - chunk * C) ? gate_coef(a.coef, to_f32(b.kbeta[i]), lam) : 0.f;
          if (g0 == 0) alpha[row] = al;
          floatx4 dg = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int f = 0; f < NKB; ++f) dg = MM::mma(dg, b.kb[i][f], b.kb[i][f]);
          if constexpr (GATED) {
            // b over the chunk's rows (lane l: row l; rows past T add 0),
            // this block's rows of [b | Gamma | Gamma_C / Gamma] into the
            // chunk's slot of the table, then the block's Gram entries times E
            const float bsc = wave_prefix_sum(b.lgv);
            const float bC = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, bsc), C - 1));
            float* gb = gslot(chunk);
            if (g0 == PW) {
              gb[lane] = bsc;
              gb[C + lane] = __expf(bsc);
              gb[2 * C + lane] = __expf(bC - bsc);
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            const floatx4 de = decay_tile(gb, PW, PW, dg, std::true_type{});
#pragma unroll
            for (int e = 0; e < 4; ++e) sm.Adt[PW][4 * g0 + e][li0] = al * de[e];
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) sm.Adt[blk][4 * g0 + e][li0] = (4 * g0 + e < li0) ? al * dg[e] : 0.f;
          }
         }
        };
        // one chunk step: cur holds chunk n = c + 1, nxt holds chunk n + 1
        auto step = [&](int c, LB& cur, LB& nxt) {
          const int n = c + 1;
          const bool act = n < nchunks;
          auto& B = sm.buf[n & 1];
          int li = lane & 15, g = lane >> 4;
          asm volatile("" : "+v"(li), "+v"(g));
          // the fragments of this wave's phase-A M job (chunk c, the other
          // buffer) are requested before the staging writes, so that their
          // LDS round trip overlaps the staging
          using JA = std::integral_constant<int, JB::NOFF + ljob(0)>;
          Frag akf[NA > 0 ? NFK : 1], aqf[NA > 0 ? NFK : 1];
          if constexpr (NA > 0) {
            if (c >= 0) {
              auto& Bc = sm.buf[c & 1];
#pragma unroll
              for (int f = 0; f < NFK; ++f) {
                akf[f] = MM::template ldp<NKT>(&Bc.K[16 * JB::J(JA::value) + li][0], f);
                aqf[f] = MM::template ldp<NKT>(&Bc.Q[16 * JB::I(JA::value) + li][0], f);
              }
            }
          }
          // ---- phase A: stage chunk n (rows past T arrived as zeros), keys
          //      and queries in the key layout of this pass (natural, or
          //      column-permuted)
          if (act) {
#pragma unroll
            for (int i = 0; i < NBL; ++i)
#pragma unroll
              for (int f = 0; f < NKB; ++f) {
                if constexpr (SROWP) *(Vec*)&B.K[16 * (PW + NLW * i) + li][32 * f + 8 * g] = cur.kb[i][f];
                else st_perm(&B.K[16 * (PW + NLW * i) + li][0], 32 * f + 8 * g, cur.kb[i][f]);
              }
#pragma unroll
            for (int j = 0; j < NLK; ++j) {
              const int idx = lt + NLT * j;
              if (KFULL || idx < C * VPR) {
                const int r = idx / VPR, cv = idx % VPR;
                if constexpr (SROWP) *(Vec*)&B.Q[r][cv * VE] = cur.q[j];
                else st_perm(&B.Q[r][0], cv * VE, cur.q[j]);
              }
            }
#pragma unroll
            for (int j = 0; j < NLV; ++j) {
              const int idx = lt + NLT * j;
              if (VFULL || idx < C * VPRV) {
                const int r = idx / VPRV, cv = idx % VPRV;
                *(Vec*)&B.V[r][cv * VE] = cur.v[j];  // 16-byte aligned rows
              }
            }
          }
          // first M job of the chunk whose state pass runs now
          if constexpr (NA > 0) {
            static_assert(NA == 1, "one phase-A job");
            if (c >= 0) {
              constexpr int I = JB::I(JA::value), J = JB::J(JA::value);
              floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
              for (int f = 0; f < NFK; ++f) acc = MM::mma(acc, akf[f], aqf[f]);
              if constexpr (GATED) {
                acc = decay_tile(gslot(c), I, J, acc, std::false_type{});
              } else if constexpr (I == J) {
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[e] = (4 * g + e <= li) ? acc[e] : 0.f;
              }
              MM::store_tps(&sm.buf[c & 1].M[16 * I + li][0], J, acc);
            }
          }
          // cur is free again: chunk n + 2 into it (clamped, never skipped)
          load_all(cur, min(n + 2, nchunks - 1));
          __syncthreads();
          // ---- phase B: the rest of this wave's lower-incl-diag Q K^T tiles
          //      of chunk n (-> M); a and the diagonal Gram block of chunk
          //      n + 1, which the solvers invert in the next phase
          if constexpr (NJ > NA) {
            if (act) mtiles(B, std::integral_constant<int, NA>{}, std::integral_constant<int, NJ>{}, GATED ? gslot(n) : nullptr);
          }
          if (n + 1 < nchunks) gate_gram(nxt, n + 1, sm.buf[(n + 1) & 1].alpha);
          __syncthreads();
        };
        load_all(b0, 0);
        load_all(b1, min(1, nchunks - 1));
        gate_gram(b0, 0, sm.buf[0].alpha);
        __syncthreads();
        // steps c = -1 .. nchunks - 1 (b0 holds the even chunks, b1 the odd),
        // two per trip so that the register sets keep fixed names
        int c = -1;
        for (; c + 1 < nchunks; c += 2) {
          step(c, b0, b1);
          step(c + 1, b1, b0);
        }
        if (c < nchunks) step(c, b0, b1);
      } else {
        load_k(0);
        load_qv(0);
        gate_rows(0, sm.buf[0].alpha);
        __syncthreads();
        for (int c = -1; c < nchunks; ++c) {
          const int n = c + 1;  // chunk being prepared
          const bool act = n < nchunks;
          auto& B = sm.buf[n & 1];
          // ---- phase A: stage chunk n (keys, queries, value slice); rows
          //      past T arrived as zeros
          if (act) {
#pragma unroll
            for (int j = 0; j < NLK; ++j) {
              const int idx = lt + NLT * j;
              if (KFULL || idx < C * VPR) {
                const int r = idx / VPR, cv = idx % VPR;
                if constexpr (SROWP) {
                  *(Vec*)&B.K[r][cv * VE] = kreg[j];  // 16-byte aligned rows
                  *(Vec*)&B.Q[r][cv * VE] = qreg[j];
                } else {
                  st_perm(&B.K[r][0], cv * VE, kreg[j]);
                  st_perm(&B.Q[r][0], cv * VE, qreg[j]);
                }
              }
            }
#pragma unroll
            for (int j = 0; j < NLV; ++j) {
              const int idx = lt + NLT * j;
              if (VFULL || idx < C * VPRV) {
                const int r = idx / VPRV, cv = idx % VPRV;
                *(Vec*)&B.V[r][cv * VE] = vreg[j];  // 16-byte aligned rows
              }
            }
          }
          // first M job of the chunk whose state pass runs now
          if constexpr (NA > 0) {
            if (c >= 0) mtiles(sm.buf[c & 1], std::integral_constant<int, 0>{}, std::integral_constant<int, NA>{}, nullptr);
          }
          load_k(min(n + 1, nchunks - 1));
          __syncthreads();
          // ---- phase B: load the queries and values of chunk n + 1; the rest
          //      of this wave's lower-incl-diag Q K^T tiles of chunk n (-> M)
          load_qv(min(n + 1, nchunks - 1));
          if constexpr (NJ > NA) {
            if (act) mtiles(B, std::integral_constant<int, NA>{}, std::integral_constant<int, NJ>{}, nullptr);
          }
          // a of chunk n + 1 (its keys arrived during this phase)
          if (n + 1 < nchunks) gate_rows(n + 1, sm.buf[(n + 1) & 1].alpha);
          __syncthreads();
        }
      }
    };
    switch (w - NSW - 2) {
      case 0: loader(std::integral_constant<int, 0>{}); break;
      case 1: loader(std::integral_constant<int, 1>{}); break;
      case 2: loader(std::integral_constant<int, 2>{}); break;
      default: loader(std::integral_constant<int, 3>{}); break;
    }
  }
}

#undef skey

// Workgroup -> pass index with the column slices of a head on one XCD (the
// hardware deals workgroups to the 8 XCDs round robin): the slices read the
// same keys and queries, which then come from that XCD's L2.
__device__ __forceinline__ int xcd_slot(int nvt) {
  const int total = gridDim.x;
  if (total % 8 == 0 && ((total / 8) % nvt) == 0) return (blockIdx.x % 8) * (total / 8) + blockIdx.x / 8;
  return blockIdx.x;
}

template <typename CT, int D, int C, int BV, int NSW, int PM, bool GATED = false>
__global__ __launch_bounds__(64 * (NSW + 2 + pipe_loaders<PM>()), 1) void efla_chunked_pipe_kernel(ChunkedArgs a) {
  __shared__ PipeSmem<CT, D, C, BV> sm;
  pipe_body<CT, D, C, BV, NSW, PM, GATED>(a, sm, xcd_slot(a.nvt));
}

// First launch of the time-segmented forward: the summaries of segments
// 1 .. nseg - 2 (pass mode 1, first nsum workgroups) and the outputs of
// segment 0, which starts from S0 and needs no carry (pass mode 0, the rest).
// Both run 8 waves of 64 lanes on one shared-memory layout.
template <typename CT, int D, int C, int BV>
__global__ __launch_bounds__(512, 1) void efla_seg_first_kernel(ChunkedArgs summ, ChunkedArgs first, int nsum) {
  __shared__ PipeSmem<CT, D, C, BV> sm;
  const int L = xcd_slot(summ.nvt);
  if (L < nsum) pipe_body<CT, D, C, BV, 4, 1>(summ, sm, L);
  else pipe_body<CT, D, C, BV, 2, 0>(first, sm, L - nsum);
}

// ---------------------------------------------------------------------------
// Carry of the time-segmented forward: per head, the start state of every
// segment from the second on, S_start(1) = the end state of segment 0 (left
// in seg_s0 by the first launch) and S_start(g + 1) = P_g S_start(g) + R_g
// for g = 1 .. nseg - 2, in fp32. One workgroup per (head, 16-column slice
// of S): the columns of S evolve independently, so the slices need no
// exchange. P_g is staged in LDS each step.
template <int D>
__global__ __launch_bounds__(256) void efla_seg_carry_kernel(const float* seg_out, float* seg_s0, int nseg) {
  // fp32 MFMA (16x16x4): lane (g, i) of a 16x16 tile product takes
  // A[i][k] and B[k][i] for the four k values 16q + 4g + s of k-block q
  // (s = 0..3: one MFMA each) from one 16-byte read of a row of P and of a
  // row of S^T; the result holds rows 4g + e of column i. Rows are padded to
  // an odd multiple of 32 bytes (conflict-free 16-byte reads).
  constexpr int LD = D + 8;
  __shared__ __attribute__((aligned(16))) float P[D][LD];
  __shared__ __attribute__((aligned(16))) float St[16][LD];  // S^T of this 16-column slice
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int li = lane & 15, g = lane >> 4;
  const int h = blockIdx.x / (D / 16);
  const int j0 = (blockIdx.x % (D / 16)) * 16;
  for (int i = tid; i < D * 16; i += 256) {
    const int r = i / 16, c = i % 16;
    St[c][r] = seg_s0[((size_t)(h * nseg + 1) * D + r) * D + j0 + c];
  }
  __syncthreads();
  // P_g and this lane's R_g values are fetched into registers one step ahead
  constexpr int NPL = (D * D / 4 + 255) / 256;  // 16-byte pieces of P per thread
  constexpr int NT = (D / 16 + 3) / 4;  // 16-row tiles per wave
  floatx4 pr[NPL], rr[NT];
  // maps of segments 1 .. nseg - 2, map j = segment j + 1
  auto fetch = [&](int m) {
    const float* R = seg_out + ((size_t)(h * (nseg - 2) + m) * 2) * D * D;
    const float* Pg = R + (size_t)D * D;
#pragma unroll
    for (int j = 0; j < NPL; ++j)
      if (tid + 256 * j < D * D / 4) pr[j] = *(const floatx4*)&Pg[4 * (tid + 256 * j)];
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
      const int t = w + 4 * tt;
      if (t < D / 16) {
#pragma unroll
        for (int e = 0; e < 4; ++e) rr[tt][e] = R[(size_t)(16 * t + 4 * g + e) * D + j0 + li];
      }
    }
  };
  fetch(0);
  for (int gs = 1; gs < nseg; ++gs) {
    if (gs > 1) {
      float* dst = seg_s0 + ((size_t)h * nseg + gs) * D * D;
      for (int i = tid; i < D * 16; i += 256) {
        const int r = i / 16, c = i % 16;
        dst[(size_t)r * D + j0 + c] = St[c][r];
      }
    }
    if (gs == nseg - 1) break;
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      const int e4 = 4 * (tid + 256 * j);
      if (e4 < D * D) *(floatx4*)&P[e4 / D][e4 % D] = pr[j];
    }
    floatx4 acc[NT];
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) acc[tt] = rr[tt];
    __syncthreads();
    if (gs + 1 < nseg - 1) fetch(gs);
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
      const int t = w + 4 * tt;
      if (t < D / 16) {
        floatx4 c4 = acc[tt];
#pragma unroll
        for (int q = 0; q < D / 16; ++q) {
          const floatx4 a4 = *(const floatx4*)&P[16 * t + li][16 * q + 4 * g];
          const floatx4 b4 = *(const floatx4*)&St[li][16 * q + 4 * g];
#pragma unroll
          for (int sidx = 0; sidx < 4; ++sidx) c4 = __builtin_amdgcn_mfma_f32_16x16x4f32(a4[sidx], b4[sidx], c4, 0, 0, 0);
        }
        acc[tt] = c4;
      }
    }
    __syncthreads();
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
      const int t = w + 4 * tt;
      if (t < D / 16) *(floatx4*)&St[li][16 * t + 4 * g] = acc[tt];
    }
    __syncthreads();
  }
}

// When a plain pass would leave most of the GPU idle (few heads, long
// sequences), the forward runs as three launches over nseg time segments:
// the affine maps of segments 1 .. nseg - 2 together with the outputs of
// segment 0 (which starts from S0), the carry, then the outputs of segments
// 1 .. nseg - 1 from their true start states. About three times the state
// arithmetic of one pass, spread over ~nseg times more workgroups; with W
// workgroups per pass both big launches have W (nseg - 1) workgroups.
struct SegPlan {
  int nseg = 1;
  int seg_len = 0;
};

static SegPlan seg_plan(int NH, int T, int d, int C, bool pipelined) {
  SegPlan p;
  if (!pipelined) return p;
  const long long W = (long long)NH * (d / (d < 64 ? d : 64));  // workgroups of one pass
  const int nchunks = (T + C - 1) / C;
  if (W >= 128 || nchunks < 64) return p;
  // Segments of >= 8 chunks (measured on fp32_d64, 32 heads x 128 chunks of
  // 16 tokens: at least 32 chunks per segment gave 4 segments and 162.7 us,
  // at least 16 gave 8 and 95 us, at least 8 gave 9 and 89.5 us), and at
  // most sqrt(nchunks) + 1 of them: the two big launches take about
  // 2 nchunks / G chunk steps, the carry G steps of its own (each about
  // 1.5 chunk steps), which this bound balances for very few heads.
  long long rt = 1;
  while ((rt + 1) * (rt + 1) <= nchunks) ++rt;
  const long long G = std::min<long long>(std::min<long long>(256 / W + 1, nchunks / 8), rt + 1);
  if (G < 2) return p;
  const int cps = (int)((nchunks + G - 1) / G);  // chunks per segment
  p.seg_len = cps * C;
  p.nseg = (T + p.seg_len - 1) / p.seg_len;
  if (p.nseg < 2) p = SegPlan{};
  return p;
}

// Workspace: the maps (R_g, P_g) of segments 1 .. nseg - 2, then the start
// states of all segments (slot 0 unused).
static size_t seg_workspace_bytes(const SegPlan& p, int NH, int d) {
  if (p.nseg < 2) return 0;
  return (size_t)NH * (3 * (size_t)p.nseg - 4) * d * d * sizeof(float);
}

// ---------------------------------------------------------------------------
// Host-side launch. Returns hipSuccess or the launch error.
template <typename CT, int D, int C>
constexpr bool pipelined() {
  return pipe_smem_bytes<CT, D, C, (D < 64 ? D : 64)>() <= 160 * 1024;
}

template <typename CT, int D, int C>
static hipError_t launch_chunked(const ChunkedArgs& in, int NH, void* ws, hipStream_t stream) {
  constexpr int BV = D < 64 ? D : 64;
  ChunkedArgs a = in;
  a.nvt = D / BV;
  dim3 grid((unsigned)(NH * a.nvt));
  if constexpr (pipelined<CT, D, C>()) {
    constexpr int NSW = EFLA_PIPE_STATE_WAVES;
    const SegPlan sp = seg_plan(NH, a.T, D, C, true);
    if (sp.nseg >= 2) {
      static_assert(NSW == 2, "the first segmented launch runs the two-state-wave output pass");
      const int ns = sp.nseg;
      float* seg_out = (float*)ws;
      float* seg_s0 = seg_out + (size_t)NH * (ns - 2) * 2 * D * D;
      ChunkedArgs m1 = a;  // maps of segments 1 .. ns - 2
      m1.mode = 1;
      m1.seg_len = sp.seg_len;
      m1.nseg = ns;
      m1.nrun = ns - 2;
      m1.seg_out = seg_out;
      ChunkedArgs m0 = a;  // outputs of segment 0
      m0.mode = 2;
      m0.seg_len = sp.seg_len;
      m0.nseg = ns;
      m0.seg_first = 0;
      m0.nrun = 1;
      m0.seg_s0 = seg_s0;
      const int nsum = NH * (ns - 2) * a.nvt;
      hipLaunchKernelGGL((efla_seg_first_kernel<CT, D, C, BV>), dim3((unsigned)(nsum + NH * a.nvt)), dim3(512), 0,
                         stream, m1, m0, nsum);
      if (const hipError_t e = hipGetLastError(); e != hipSuccess) return e;
      if (ns >= 3) {
        hipLaunchKernelGGL((efla_seg_carry_kernel<D>), dim3((unsigned)(NH * (D / 16))), dim3(256), 0, stream,
                           (const float*)seg_out, seg_s0, ns);
        if (const hipError_t e = hipGetLastError(); e != hipSuccess) return e;
      }
      ChunkedArgs m2 = a;  // outputs of segments 1 .. ns - 1
      m2.mode = 2;
      m2.seg_len = sp.seg_len;
      m2.nseg = ns;
      m2.seg_first = 1;
      m2.nrun = ns - 1;
      m2.seg_s0 = seg_s0;
      hipLaunchKernelGGL((efla_chunked_pipe_kernel<CT, D, C, BV, NSW, 0>),
                         dim3((unsigned)(NH * (ns - 1) * a.nvt)), dim3(64 * (NSW + 6)), 0, stream, m2);
      return hipGetLastError();
    }
    hipLaunchKernelGGL((efla_chunked_pipe_kernel<CT, D, C, BV, NSW, 0>), grid, dim3(64 * (NSW + 6)), 0,
                       stream, a);
  } else {
    // 4-wave kernel. When a pass of 64-column slices would leave CUs idle,
    // 16-column slices give 4x the workgroups (the key-only work of a chunk
    // is then repeated per slice, on CUs that would otherwise idle):
    // fp32, 32 heads, d = 64, T = 2048, C = 64: 477 -> 341 us.
    static_assert(chunked_smem_bytes<CT, D, C, BV>() <= 160 * 1024, "LDS budget");
    if (NH * a.nvt < 256 && BV > 16) {
      a.nvt = D / 16;
      hipLaunchKernelGGL((efla_chunked_kernel<CT, D, C, 16, EFLA_STATE_WAVES>), dim3((unsigned)(NH * a.nvt)),
                         dim3(256), 0, stream, a);
    } else {
      hipLaunchKernelGGL((efla_chunked_kernel<CT, D, C, BV, EFLA_STATE_WAVES>), grid, dim3(256), 0, stream,
                         a);
    }
  }
  return hipGetLastError();
}

// Chunk length the forward runs with. fp32 tiles of 64 tokens do not fit the
// pipelined kernel's double-buffered LDS (and at d = 128 no kernel's), so
// fp32 with chunk 64 runs the pipelined kernel with 32-token chunks when one
// pass fills the GPU (>= 128 workgroups) and with 16-token chunks otherwise,
// where the time-segmented schedule then has twice the chunks to split into
// segments. Measured on MI355X (fp32, T = 2048): 32 heads at d = 64 340 ->
// 166 us, 256 heads at d = 64 474 -> 294 us, 32 heads at d = 128 476 ->
// 284 us. The chunk length changes the rounding order only: the chunked
// form is exact algebra for any length.
static int effective_chunk(int NH, int d, int chunk, bool is_bf16) {
  if (is_bf16 || chunk != 64) return chunk;
  const long long W = (long long)NH * (d / (d < 64 ? d : 64));
  return W >= 128 ? 32 : 16;
}

template <typename CT, int D>
static hipError_t dispatch_chunk(const ChunkedArgs& a, int NH, int chunk, void* ws, hipStream_t s) {
  switch (chunk) {
    case 16: return launch_chunked<CT, D, 16>(a, NH, ws, s);
    case 32: return launch_chunked<CT, D, 32>(a, NH, ws, s);
    case 64:
      if constexpr (sizeof(CT) == 4 && D == 128) return launch_chunked<CT, D, 32>(a, NH, ws, s);
      else return launch_chunked<CT, D, 64>(a, NH, ws, s);
    default: return hipErrorInvalidValue;
  }
}

// Gated variant. bf16 with 64-token chunks and d >= 32 runs the pipelined
// kernel's gated outputs pass (one pass per head and 64-column slice, no
// time segments); the other shapes the 4-wave kernel with the decay terms,
// in slices of 16 state columns when 64-column slices would leave CUs idle.
template <typename CT, int D, int C>
static hipError_t launch_chunked_gated(const ChunkedArgs& in, int NH, hipStream_t stream) {
  constexpr int BV = D < 64 ? D : 64;
  static_assert(chunked_smem_bytes<CT, D, C, BV>() <= 160 * 1024, "LDS budget");
  ChunkedArgs a = in;
  a.nvt = D / BV;
  if constexpr (sizeof(CT) == 2 && C == 64 && D >= 32 && pipelined<CT, D, C>()) {
    constexpr int NSW = EFLA_PIPE_STATE_WAVES;
    hipLaunchKernelGGL((efla_chunked_pipe_kernel<CT, D, C, BV, NSW, 0, true>), dim3((unsigned)(NH * a.nvt)),
                       dim3(64 * (NSW + 6)), 0, stream, a);
    return hipGetLastError();
  }
  if (NH * a.nvt < 256 && BV > 16) {
    a.nvt = D / 16;
    hipLaunchKernelGGL((efla_chunked_kernel<CT, D, C, 16, EFLA_STATE_WAVES, true>), dim3((unsigned)(NH * a.nvt)),
                       dim3(256), 0, stream, a);
  } else {
    hipLaunchKernelGGL((efla_chunked_kernel<CT, D, C, BV, EFLA_STATE_WAVES, true>), dim3((unsigned)(NH * a.nvt)),
                       dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

template <typename CT, int D>
static hipError_t dispatch_chunk_gated(const ChunkedArgs& a, int NH, int chunk, hipStream_t s) {
  switch (chunk) {
    case 16: return launch_chunked_gated<CT, D, 16>(a, NH, s);
    case 32: return launch_chunked_gated<CT, D, 32>(a, NH, s);
    case 64:
      if constexpr (sizeof(CT) == 4 && D == 128) return launch_chunked_gated<CT, D, 32>(a, NH, s);
      else return launch_chunked_gated<CT, D, 64>(a, NH, s);
    default: return hipErrorInvalidValue;
  }
}

template <typename CT>
static hipError_t dispatch_d_gated(const ChunkedArgs& a, int NH, int d, int chunk, hipStream_t s) {
  switch (d) {
    case 16: return dispatch_chunk_gated<CT, 16>(a, NH, chunk, s);
    case 32: return dispatch_chunk_gated<CT, 32>(a, NH, chunk, s);
    case 64: return dispatch_chunk_gated<CT, 64>(a, NH, chunk, s);
    case 128: return dispatch_chunk_gated<CT, 128>(a, NH, chunk, s);
    default: return hipErrorInvalidValue;
  }
}

template <typename CT, int D>
static bool pipelined_chunk(int chunk) {
  switch (chunk) {
    case 16: return pipelined<CT, D, 16>();
    case 32: return pipelined<CT, D, 32>();
    case 64:
      if constexpr (sizeof(CT) == 4 && D == 128) return false;
      else return pipelined<CT, D, 64>();
    default: return false;
  }
}

template <typename CT>
static bool pipelined_d(int d, int chunk) {
  switch (d) {
    case 16: return pipelined_chunk<CT, 16>(chunk);
    case 32: return pipelined_chunk<CT, 32>(chunk);
    case 64: return pipelined_chunk<CT, 64>(chunk);
    case 128: return pipelined_chunk<CT, 128>(chunk);
    default: return false;
  }
}

template <typename CT>
static hipError_t dispatch_d(const ChunkedArgs& a, int NH, int d, int chunk, void* ws, hipStream_t s) {
  switch (d) {
    case 16: return dispatch_chunk<CT, 16>(a, NH, chunk, ws, s);
    case 32: return dispatch_chunk<CT, 32>(a, NH, chunk, ws, s);
    case 64: return dispatch_chunk<CT, 64>(a, NH, chunk, ws, s);
    case 128: return dispatch_chunk<CT, 128>(a, NH, chunk, ws, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace efla

// Internal entries used by the C ABI layer (arguments already validated).
size_t efla_internal_chunked_workspace_bytes(int NH, int T, int d, int chunk, int is_bf16) {
  const int c = efla::effective_chunk(NH, d, chunk, is_bf16 != 0);
  const bool pipe = is_bf16 ? efla::pipelined_d<efla::bf16>(d, c) : efla::pipelined_d<float>(d, c);
  return efla::seg_workspace_bytes(efla::seg_plan(NH, T, d, c, pipe), NH, d);
}

// Gated forward: one pass of the 4-wave kernel per (head, column slice); no
// workspace.
hipError_t efla_internal_launch_chunked_gated(const void* q, const void* k, const void* v, const void* beta,
                                              const float* log_g, const float* s0, void* o, float* s_final,
                                              int NH, int T, int d, int chunk, int coef, int is_bf16,
                                              hipStream_t stream) {
  efla::ChunkedArgs a{q, k, v, beta, s0, o, s_final, T, 1, 0, 0, 1, nullptr, nullptr, coef, nullptr, nullptr};
  a.log_g = log_g;
  if (is_bf16) return efla::dispatch_d_gated<efla::bf16>(a, NH, d, chunk, stream);
  return efla::dispatch_d_gated<float>(a, NH, d, chunk, stream);
}

hipError_t efla_internal_launch_chunked(const void* q, const void* k, const void* v,
                                        const void* beta, const float* s0, void* o,
                                        float* s_final, void* workspace, int NH, int T, int d,
                                        int chunk, int coef, int is_bf16, hipStream_t stream) {
  efla::ChunkedArgs a{q, k, v, beta, s0, o, s_final, T, 1, 0, 0, 1, nullptr, nullptr, coef, nullptr, nullptr};
  const int c = efla::effective_chunk(NH, d, chunk, is_bf16 != 0);
  if (is_bf16) return efla::dispatch_d<efla::bf16>(a, NH, d, c, workspace, stream);
  return efla::dispatch_d<float>(a, NH, d, c, workspace, stream);
}

// Pass mode 2 of the pipelined kernel: one plain pass that stores the state at
// the start of every chunk (for the backward). Only where the pipelined kernel
// serves the shape.
namespace efla {
template <typename CT, int D, int C, int PM>
static hipError_t launch_states_pm(const ChunkedArgs& in, int NH, hipStream_t stream) {
  if constexpr (pipelined<CT, D, C>()) {
    constexpr int BV = D < 64 ? D : 64;
    constexpr int NSW = EFLA_PIPE_STATE_WAVES;
    ChunkedArgs a = in;
    a.nvt = D / BV;
    hipLaunchKernelGGL((efla_chunked_pipe_kernel<CT, D, C, BV, NSW, PM>), dim3((unsigned)(NH * a.nvt)),
                       dim3(64 * (NSW + 6)), 0, stream, a);
    return hipGetLastError();
  } else {
    return hipErrorInvalidValue;
  }
}

// pass mode 2 (states only) or 3 (outputs and states)
template <typename CT, int D>
static hipError_t states_chunk(const ChunkedArgs& a, int NH, int chunk, hipStream_t s) {
  const bool o = a.o != nullptr;
  switch (chunk) {
    case 16: return o ? launch_states_pm<CT, D, 16, 3>(a, NH, s) : launch_states_pm<CT, D, 16, 2>(a, NH, s);
    case 32: return o ? launch_states_pm<CT, D, 32, 3>(a, NH, s) : launch_states_pm<CT, D, 32, 2>(a, NH, s);
    case 64:
      if constexpr (sizeof(CT) == 4 && D == 128) return hipErrorInvalidValue;
      else return o ? launch_states_pm<CT, D, 64, 3>(a, NH, s) : launch_states_pm<CT, D, 64, 2>(a, NH, s);
    default: return hipErrorInvalidValue;
  }
}

template <typename CT>
static hipError_t states_d(const ChunkedArgs& a, int NH, int d, int chunk, hipStream_t s) {
  switch (d) {
    case 16: return states_chunk<CT, 16>(a, NH, chunk, s);
    case 32: return states_chunk<CT, 32>(a, NH, chunk, s);
    case 64: return states_chunk<CT, 64>(a, NH, chunk, s);
    case 128: return states_chunk<CT, 128>(a, NH, chunk, s);
    default: return hipErrorInvalidValue;
  }
}
}  // namespace efla

bool efla_internal_states_supported(int d, int chunk, int is_bf16) {
  if (d != 16 && d != 32 && d != 64 && d != 128) return false;
  if (chunk != 16 && chunk != 32 && chunk != 64) return false;
  return is_bf16 ? efla::pipelined_d<efla::bf16>(d, chunk) : efla::pipelined_d<float>(d, chunk);
}

// The chunk-start states for the backward; with o (and optionally s_final)
// the same pass also writes the outputs (pass mode 3).
hipError_t efla_internal_launch_states(const void* q, const void* k, const void* v, const void* beta,
                                       const float* s0, void* o, float* s_final, float* s_chunks,
                                       float* s_chunks_n, int NH, int T, int d, int chunk, int coef, int is_bf16,
                                       hipStream_t stream) {
  efla::ChunkedArgs a{q, k, v, beta, s0, o, o ? s_final : nullptr, T, 1, 0, 0, 1, nullptr, nullptr, coef,
                      s_chunks, s_chunks_n};
  if (is_bf16) return efla::states_d<efla::bf16>(a, NH, d, chunk, stream);
  return efla::states_d<float>(a, NH, d, chunk, stream);
}
