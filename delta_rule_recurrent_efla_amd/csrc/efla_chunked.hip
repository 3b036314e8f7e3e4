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
// MFMA accumulator registers of the wave that owns its 16 columns (columns
// of S evolve independently, so the slice split is exact). Chunk tiles are
// staged in LDS; T is never formed: its 16x16 diagonal blocks are inverted
// by forward substitution in fp32 and W, U come from a blocked forward solve
// whose right-hand sides stay in registers.

#include "efla_device.hpp"

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
  CT K[C][D + P];      // keys, row-major
  CT Kt[D][C + P];     // keys, transposed
  CT Q[C][D + P];      // queries
  CT Vt[BV][C + P];    // value slice, transposed
  CT Wn[C][D + P];     // -W
  CT An[C][C + P];     // -A (strictly lower part only is meaningful)
  CT M[C][C + P];      // lower-incl-diag(Q K^T)
  CT O[C][BV + P];     // output staging
  float Adt[NB][16][20]; // fp32 diagonal blocks of A, transposed (row j = column j)
  CT Td[NB][16][16 + P]; // inverses of I + diagonal blocks
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

template <typename CT, int D, int C, int BV>
__global__ __launch_bounds__(256, 1) void efla_chunked_kernel(ChunkedArgs a) {
  using MM = Mma<CT>;
  using Pack = typename MM::Pack;
  using Vec = typename Vec16<CT>::type;
  constexpr int NB = C / 16;    // 16-row blocks per chunk
  constexpr int NKT = D / 16;   // 16-row tiles of the state
  constexpr int NVT = BV / 16;  // 16-column tiles of the slice (one per wave)
  constexpr int NW = 4;
  constexpr int VE = 16 / sizeof(CT);
  static_assert(NVT <= NW, "one state column tile per wave");
  constexpr int KPW = (NKT + NW - 1) / NW;  // key tiles per wave in the solve
  constexpr int NTW = 1 + KPW;              // solve tiles per wave
  static_assert(C % 16 == 0 && D % 16 == 0 && BV % 16 == 0, "tile sizes");

  __shared__ ChunkedSmem<CT, D, C, BV> sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int li = lane & 15;
  const int g = lane >> 4;

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

  const bool owner = w < NVT;
  const int kfirst = (w + NW - (NVT % NW)) % NW;  // first key tile of this wave
  const int scol = v0 + 16 * w + li;  // state column held by this lane
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
  // Retire the initial-state loads here: left pending, they make the compiler
  // wait on every outstanding load (the next chunk's prefetch included)
  // inside the chunk loop.
#pragma unroll
  for (int rt = 0; rt < NKT; ++rt) asm volatile("" : "+v"(sacc[rt]));
  floatx4 uacc[NB];

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

    // ---- chunk ch (prefetched in registers) -> LDS: K (both layouts), Q and
    //      the V slice; lambda = ||k||^2 and alpha per row
    {
#pragma unroll
      for (int j = 0; j < NLK; ++j) {
        const int idx = tid + 256 * j;
        if (idx < C * VPR) {
          const int r = idx / VPR, cv = idx % VPR;
          *(Vec*)&sm.K[r][cv * VE] = kreg[j];
          *(Vec*)&sm.Q[r][cv * VE] = qreg[j];
          float ss = 0.f;
#pragma unroll
          for (int e = 0; e < VE; ++e) {
            sm.Kt[cv * VE + e][r] = kreg[j][e];
            const float x = to_f32(kreg[j][e]);
            ss += x * x;
          }
#pragma unroll
          for (int off = 1; off < VPR; off <<= 1) ss += __shfl_xor(ss, off);
          if (cv == 0) sm.alpha[r] = gate_alpha(to_f32(breg[j]), ss);
        }
      }
#pragma unroll
      for (int j = 0; j < NLV; ++j) {
        const int idx = tid + 256 * j;
        if (idx < C * VPRV) {
          const int r = idx / VPRV, cv = idx % VPRV;
#pragma unroll
          for (int e = 0; e < VE; ++e) sm.Vt[cv * VE + e][r] = vreg[j][e];
        }
      }
    }
    // issue the global loads of the next chunk; they land during this one
    if (ch + 1 < nchunks) prefetch(ch + 1);
    __syncthreads();

    // ---- Gram and Q K^T on the lower block triangle
    {
      constexpr int NT = NB * (NB + 1) / 2;
      for (int job = w; job < 2 * NT; job += NW) {
        const bool isq = job >= NT;
        const int jj = isq ? job - NT : job;
        int I = 0;
        while ((I + 1) * (I + 2) / 2 <= jj) ++I;
        const int J = jj - I * (I + 1) / 2;
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
        // (K_J X_I^T)[4g+e][li] = x_{16I+li} . k_{16J+4g+e}
        MM::template ll<D>(acc, &sm.K[16 * J + li][0],
                           isq ? &sm.Q[16 * I + li][0] : &sm.K[16 * I + li][0]);
        const int r = 16 * I + li;
        const int cb = 16 * J + 4 * g;
        if (!isq) {
          const float al = sm.alpha[r];
          floatx4 ad;
#pragma unroll
          for (int e = 0; e < 4; ++e) ad[e] = (cb + e < r) ? al * acc[e] : 0.f;
          MM::store_t(&sm.An[r][16 * J], -ad);
          if (I == J) {
#pragma unroll
            for (int e = 0; e < 4; ++e) sm.Adt[I][4 * g + e][li] = ad[e];
          }
        } else {
          floatx4 m;
#pragma unroll
          for (int e = 0; e < 4; ++e) m[e] = (cb + e <= r) ? acc[e] : 0.f;
          MM::store_t(&sm.M[r][16 * J], m);
        }
      }
    }
    __syncthreads();

    // ---- (I + A_bb)^{-1} for each 16x16 diagonal block: column-parallel,
    //      right-looking forward substitution in fp32 (lane group g takes
    //      block g, lane i its column i; after t_j is final, column j of A
    //      is eliminated from the rows below, so the updates are independent).
    if (w == 0 && g < NB) {
      float t[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) t[r] = (r == li) ? 1.f : 0.f;
#pragma unroll
      for (int j = 0; j < 15; ++j) {
        floatx4 a4[4];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) a4[q4] = *(const floatx4*)&sm.Adt[g][j][4 * q4];
#pragma unroll
        for (int r = j + 1; r < 16; ++r) t[r] -= a4[r >> 2][r & 3] * t[j];
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) sm.Td[g][r][li] = from_f32<CT>(t[r]);
    }
    __syncthreads();

    // ---- blocked forward solve (I + A) X = diag(a) [K | V_slice] over
    //      16-column tiles. Each wave takes its value tile (kept in registers
    //      as U) and KPW key tiles (written to LDS as -W); the tiles advance
    //      through the row blocks together so their MFMA chains overlap.
    {
      const CT* rhs[NTW];
      int kt[NTW];  // key tile index, or -1 for the value tile, -2 for padding
#pragma unroll
      for (int t = 0; t < NTW; ++t) {
        int m;
        if (t == 0 && owner) {
          kt[t] = -1;
          rhs[t] = &sm.Vt[16 * w + li][0];
          continue;
        }
        m = kfirst + NW * (owner ? t - 1 : t);
        kt[t] = m < NKT ? m : -2;  // padding slots recompute tile 0 and store nothing
        rhs[t] = &sm.Kt[16 * (m < NKT ? m : 0) + li][0];
      }
      floatx4 x[NTW][NB];
      static_for<NB>([&](auto ib) {
        constexpr int i = decltype(ib)::value;
#pragma unroll
        for (int t = 0; t < NTW; ++t) {
          floatx4 acc;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 16 * i + 4 * g + e;
            acc[e] = sm.alpha[r] * to_f32(rhs[t][r]);
          }
          if constexpr (i > 0) {
            Pack p[PackCount<CT, i>::value];
            MM::template pack<i>(x[t], p);
            MM::template lp<i>(acc, &sm.An[16 * i + li][0], p);
          }
          Pack pa[PackCount<CT, 1>::value];
          MM::template pack<1>(&acc, pa);
          floatx4 xi = {0.f, 0.f, 0.f, 0.f};
          MM::template lp<1>(xi, &sm.Td[i][li][0], pa);
          x[t][i] = xi;
        }
      });
#pragma unroll
      for (int t = 0; t < NTW; ++t) {
        if (kt[t] == -1) {
#pragma unroll
          for (int i = 0; i < NB; ++i) uacc[i] = x[t][i];
        } else if (kt[t] >= 0) {
#pragma unroll
          for (int i = 0; i < NB; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              sm.Wn[16 * i + 4 * g + e][16 * kt[t] + li] = from_f32<CT>(-x[t][i][e]);
        }
      }
    }
    __syncthreads();

    // ---- serial part: U' = U - W S, O = Q S + M U', S += K^T U'
    if (owner) {
      Pack spk[PackCount<CT, NKT>::value];
      MM::template pack<NKT>(sacc, spk);
      floatx4 oacc[NB];
#pragma unroll
      for (int ut = 0; ut < NB; ++ut) {
        MM::template lp<NKT>(uacc[ut], &sm.Wn[16 * ut + li][0], spk);
        oacc[ut] = floatx4{0.f, 0.f, 0.f, 0.f};
        MM::template lp<NKT>(oacc[ut], &sm.Q[16 * ut + li][0], spk);
      }
      Pack upk[PackCount<CT, NB>::value];
      MM::template pack<NB>(uacc, upk);
      static_for<NB>([&](auto ub) {
        constexpr int ut = decltype(ub)::value;
        MM::template lp<ut + 1>(oacc[ut], &sm.M[16 * ut + li][0], upk);
      });
#pragma unroll
      for (int rt = 0; rt < NKT; ++rt) MM::template lp<NB>(sacc[rt], &sm.Kt[16 * rt + li][0], upk);
#pragma unroll
      for (int ut = 0; ut < NB; ++ut)
#pragma unroll
        for (int e = 0; e < 4; ++e) sm.O[16 * ut + 4 * g + e][16 * w + li] = from_f32<CT>(oacc[ut][e]);
    }
    __syncthreads();

    // ---- write the chunk's outputs (coalesced 16-byte stores)
    {
      constexpr int VPRO = BV / VE;
      for (int idx = tid; idx < C * VPRO; idx += 256) {
        const int r = idx / VPRO, cv = idx % VPRO;
        if (r < nval) *(Vec*)(og + (size_t)(t0 + r) * D + v0 + cv * VE) = *(const Vec*)&sm.O[r][cv * VE];
      }
    }
  }

  if (owner && a.s_final) {
    float* sf = a.s_final + (size_t)head * D * D;
#pragma unroll
    for (int rt = 0; rt < NKT; ++rt)
#pragma unroll
      for (int e = 0; e < 4; ++e) sf[(size_t)(16 * rt + 4 * g + e) * D + scol] = sacc[rt][e];
  }
}

// ---------------------------------------------------------------------------
// Host-side launch. Returns hipSuccess or the launch error.
template <typename CT, int D, int C>
static hipError_t launch_chunked(const ChunkedArgs& in, int NH, hipStream_t stream) {
  constexpr int BV = D < 64 ? D : 64;
  static_assert(chunked_smem_bytes<CT, D, C, BV>() <= 160 * 1024, "LDS budget");
  ChunkedArgs a = in;
  a.nvt = D / BV;
  dim3 grid((unsigned)(NH * a.nvt)), block(256);
  hipLaunchKernelGGL((efla_chunked_kernel<CT, D, C, BV>), grid, block, 0, stream, a);
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
