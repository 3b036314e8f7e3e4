// Single-token EFLA step (the recurrent decode form; papernotes.org note
// "Exact Flow Linear Attention: Exact Solution from Continuous-Time
// Dynamics", 整体框架 last paragraph, with the update of 关键设计 item 2).
//
// Per head, with S the fp32 state [d_k, d_v]:
//   lambda = k.k,  a = -expm1(-beta*max(lambda,1e-12)) / max(lambda,1e-12)
//                  (or the Euler / RK4 / second-order scalar: gate_coef)
//   p = S^T k,  r = S^T q                  (one read pass over S)
//   u = a (v - p)                          (S_new = S + k u^T)
//   o = S_new^T q = r + (k.q) u
//   S <- S + k u^T                         (one write pass over S)
// The step is HBM-bound (0.75 flop per state byte) and, at serving batch
// sizes, latency-bound: one read of the state, a reduction, one write. Each
// workgroup is a single wave64 that owns a VB-column slice of one head and
// keeps it in registers between the read and the write; every reduction is
// a cross-lane exchange inside the wave, so the step has no LDS round trip
// and no workgroup barrier.

#include "efla_device.hpp"

namespace efla {

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* beta;
  float* state;
  void* o;
  int nvt;
  int coef;            // step coefficient rule (gate_coef)
  const float* log_g;  // gated variant: [NH] per-head log-decay of this token
};

// RPT consecutive elements of a d-vector starting at element e0 (a multiple
// of RPT), upcast to fp32: 16-byte loads when the run is a multiple of 16
// bytes, else element loads.
template <typename CT, int RPT>
__device__ __forceinline__ void load_run(const CT* p, int e0, float (&x)[RPT]) {
  constexpr int VE = 16 / (int)sizeof(CT);
  if constexpr ((RPT * (int)sizeof(CT)) % 16 == 0) {
    typedef typename std::conditional<sizeof(CT) == 2, bf16x8, floatx4>::type V;
#pragma unroll
    for (int j = 0; j < RPT / VE; ++j) {
      const V w = *(const V*)(p + e0 + VE * j);
#pragma unroll
      for (int e = 0; e < VE; ++e) x[VE * j + e] = to_f32(w[e]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < RPT; ++i) x[i] = to_f32(p[e0 + i]);
  }
}

// Sum over the lanes that share lane % CG (the row groups of one column
// group); every lane receives its column group's total. Inside a 16-lane row
// a DPP rotation by off (a power of two, 8 at most) adds lane i + off mod 16,
// which keeps the lanes of one column group together; across rows the row
// swaps. No exchange goes through the LDS.
template <int CG>
__device__ __forceinline__ float rowgroup_sum(float x) {
  static_assert(CG == 1 || CG == 2 || CG == 4 || CG == 8 || CG == 16 || CG == 32, "column groups");
  auto ror = [](float v, auto ctrl) {  // row_ror:n is DPP control 0x120 + n
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x120 + decltype(ctrl)::value,
                                                              0xf, 0xf, false));
  };
  if constexpr (CG <= 1) x += ror(x, std::integral_constant<int, 1>{});
  if constexpr (CG <= 2) x += ror(x, std::integral_constant<int, 2>{});
  if constexpr (CG <= 4) x += ror(x, std::integral_constant<int, 4>{});
  if constexpr (CG <= 8) x += ror(x, std::integral_constant<int, 8>{});
  if constexpr (CG <= 16) x = xor16_sum(x);
  return xor32_sum(x);
}

// GATED: the gated variant, S_new = g (I - c k k^T) S + c k v^T with
// g = exp(log_g) per head (the plain reading of the papernotes note's
// "Gated EFLA": Gated DeltaNet's update with the exact-flow coefficient).
// Then u = c (v - g p), S_new = g S + k u^T and o = g r + (k.q) u.
template <typename CT, int D, int VB, bool GATED>
__global__ __launch_bounds__(64) void efla_decode_kernel(DecodeArgs a) {
  // lane = rg * CG + cg: column group cg holds columns v0 + 4 cg .. + 3,
  // row group rg holds the RPT consecutive rows rg * RPT ..
  constexpr int CG = VB / 4;
  constexpr int RG = 64 / CG;
  constexpr int RPT = D / RG;
  static_assert(VB % 4 == 0 && 64 % CG == 0 && D % RG == 0 && RPT >= 1, "slice shape");
  const int lane = threadIdx.x;
  const int cg = lane % CG, rg = lane / CG;
  const int head = blockIdx.x / a.nvt;
  const int v0 = (blockIdx.x % a.nvt) * VB;
  const int r0 = rg * RPT;

  float* S = a.state + (size_t)head * D * D + (size_t)r0 * D + v0 + 4 * cg;
  floatx4 s[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) s[i] = *(const floatx4*)(S + (size_t)i * D);
  float kr[RPT], qr[RPT];
  load_run<CT, RPT>((const CT*)a.k + (size_t)head * D, r0, kr);
  load_run<CT, RPT>((const CT*)a.q + (size_t)head * D, r0, qr);
  float vv[4];
  load_run<CT, 4>((const CT*)a.v + (size_t)head * D, v0 + 4 * cg, vv);
  const float b = to_f32(((const CT*)a.beta)[head]);
  const float gd = GATED ? __expf(a.log_g[head]) : 1.f;

  // lambda = k.k and k.q: partial sums over this lane's rows, completed
  // across the row groups
  float lam = 0.f, kq = 0.f;
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    lam += kr[i] * kr[i];
    kq += kr[i] * qr[i];
  }
  // p = S^T k and r = S^T q for this lane's four columns
  floatx4 p = {0.f, 0.f, 0.f, 0.f}, r = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    p += kr[i] * s[i];
    r += qr[i] * s[i];
  }
  lam = rowgroup_sum<CG>(lam);
  kq = rowgroup_sum<CG>(kq);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    p[e] = rowgroup_sum<CG>(p[e]);
    r[e] = rowgroup_sum<CG>(r[e]);
  }
  // u = a (v - p): S_new = S + k u^T; o = S_new^T q = r + (k.q) u
  const float al = gate_coef(a.coef, b, lam);
  floatx4 u;
  if constexpr (GATED) {
#pragma unroll
    for (int e = 0; e < 4; ++e) u[e] = al * (vv[e] - gd * p[e]);
    if (rg == 0) store4((CT*)a.o + (size_t)head * D + v0 + 4 * cg, gd * r + kq * u);
#pragma unroll
    for (int i = 0; i < RPT; ++i) *(floatx4*)(S + (size_t)i * D) = gd * s[i] + kr[i] * u;
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) u[e] = al * (vv[e] - p[e]);
    if (rg == 0) store4((CT*)a.o + (size_t)head * D + v0 + 4 * cg, r + kq * u);
#pragma unroll
    for (int i = 0; i < RPT; ++i) *(floatx4*)(S + (size_t)i * D) = s[i] + kr[i] * u;
  }
}

// State columns per wave. Measured on MI355X (128 heads, d = 128, kernel
// trace): 32 columns 4.86 us per step, 64 columns 5.31 us, 16 columns 8.12 us
// (each row piece is then half a 128-byte line).
#ifndef EFLA_DECODE_VB
#define EFLA_DECODE_VB 32
#endif
template <typename CT, int D>
static hipError_t launch_decode(const DecodeArgs& in, int NH, hipStream_t stream) {
  constexpr int VB = D < EFLA_DECODE_VB ? D : EFLA_DECODE_VB;
  DecodeArgs a = in;
  a.nvt = D / VB;
  if (a.log_g)
    hipLaunchKernelGGL((efla_decode_kernel<CT, D, VB, true>), dim3((unsigned)(NH * a.nvt)), dim3(64), 0, stream, a);
  else
    hipLaunchKernelGGL((efla_decode_kernel<CT, D, VB, false>), dim3((unsigned)(NH * a.nvt)), dim3(64), 0, stream, a);
  return hipGetLastError();
}

template <typename CT>
static hipError_t dispatch_decode(const DecodeArgs& a, int NH, int d, hipStream_t s) {
  switch (d) {
    case 16: return launch_decode<CT, 16>(a, NH, s);
    case 32: return launch_decode<CT, 32>(a, NH, s);
    case 64: return launch_decode<CT, 64>(a, NH, s);
    case 128: return launch_decode<CT, 128>(a, NH, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace efla

hipError_t efla_internal_launch_decode(const void* q, const void* k, const void* v,
                                       const void* beta, const float* log_g, float* state, void* o,
                                       int NH, int d, int coef, int is_bf16, hipStream_t stream) {
  efla::DecodeArgs a{q, k, v, beta, state, o, 1, coef, log_g};
  if (is_bf16) return efla::dispatch_decode<efla::bf16>(a, NH, d, stream);
  return efla::dispatch_decode<float>(a, NH, d, stream);
}
