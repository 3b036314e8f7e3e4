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
// The step is HBM-bound (0.75 flop per state byte), so the kernel is a
// single coalesced read and write of the state: each workgroup owns a
// 32-column slice of one head, holds it in registers between the two passes
// and reduces the column partial sums by lane exchanges inside each wave and
// through LDS across the four waves.

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
  int coef;  // step coefficient rule (gate_coef)
};

template <typename CT, int D, int VB>
__global__ __launch_bounds__(256) void efla_decode_kernel(DecodeArgs a) {
  // Thread layout: lane l of wave wv reads float4 column group cg = l % CG
  // of rows rg + RG i, rg = l / CG + (64 / CG) wv. The column partial sums
  // are reduced over the row groups of a wave by lane exchanges, then over
  // the four waves through LDS.
  constexpr int CG = VB / 4;               // float4 column groups per row
  constexpr int RG = 256 / CG;             // row groups
  constexpr int RPT = (D + RG - 1) / RG;   // rows per thread
  __shared__ float sk[D], sq[D], sv[VB], su[VB];
  __shared__ floatx4 sp[4][CG], sr[4][CG];
  __shared__ float slam, skq;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int head = blockIdx.x / a.nvt;
  const int v0 = (blockIdx.x % a.nvt) * VB;
  const int cg = tid % CG, rg = tid / CG;

  const CT* qg = (const CT*)a.q + (size_t)head * D;
  const CT* kg = (const CT*)a.k + (size_t)head * D;
  const CT* vg = (const CT*)a.v + (size_t)head * D;
  float* S = a.state + (size_t)head * D * D;

  floatx4 s[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int r = rg + RG * i;
    if (r < D) s[i] = *(const floatx4*)(S + (size_t)r * D + v0 + 4 * cg);
  }
  if (tid < D) {
    sk[tid] = to_f32(kg[tid]);
    sq[tid] = to_f32(qg[tid]);
  }
  if (tid < VB) sv[tid] = to_f32(vg[v0 + tid]);
  __syncthreads();

  if (wv == 0) {
    float l = 0.f, kq = 0.f;
    for (int j = lane; j < D; j += 64) {
      l += sk[j] * sk[j];
      kq += sk[j] * sq[j];
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      l += __shfl_xor(l, off);
      kq += __shfl_xor(kq, off);
    }
    if (lane == 0) {
      slam = l;
      skq = kq;
    }
  }
  floatx4 p = {0.f, 0.f, 0.f, 0.f}, rr = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int r = rg + RG * i;
    if (r < D) {
      p += sk[r] * s[i];
      rr += sq[r] * s[i];
    }
  }
  // sum over the row groups of this wave: lanes that differ in the bits
  // above the column-group bits
#pragma unroll
  for (int off = CG; off < 64; off <<= 1) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      p[e] += __shfl_xor(p[e], off);
      rr[e] += __shfl_xor(rr[e], off);
    }
  }
  if (lane < CG) {
    sp[wv][lane] = p;
    sr[wv][lane] = rr;
  }
  __syncthreads();

  if (tid < VB) {
    const int j = tid;
    float pj = 0.f, rj = 0.f;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      pj += sp[x][j >> 2][j & 3];
      rj += sr[x][j >> 2][j & 3];
    }
    const float al = gate_coef(a.coef, to_f32(((const CT*)a.beta)[head]), slam);
    const float u = al * (sv[j] - pj);
    su[j] = u;
    ((CT*)a.o)[(size_t)head * D + v0 + j] = from_f32<CT>(rj + skq * u);
  }
  __syncthreads();

  const floatx4 u4 = *(const floatx4*)&su[4 * cg];
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int r = rg + RG * i;
    if (r < D) *(floatx4*)(S + (size_t)r * D + v0 + 4 * cg) = s[i] + sk[r] * u4;
  }
}

template <typename CT, int D>
static hipError_t launch_decode(const DecodeArgs& in, int NH, hipStream_t stream) {
  constexpr int VB = D < 32 ? D : 32;
  DecodeArgs a = in;
  a.nvt = D / VB;
  dim3 grid((unsigned)(NH * a.nvt)), block(256);
  hipLaunchKernelGGL((efla_decode_kernel<CT, D, VB>), grid, block, 0, stream, a);
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
                                       const void* beta, float* state, void* o, int NH, int d,
                                       int coef, int is_bf16, hipStream_t stream) {
  efla::DecodeArgs a{q, k, v, beta, state, o, 1, coef};
  if (is_bf16) return efla::dispatch_decode<efla::bf16>(a, NH, d, stream);
  return efla::dispatch_decode<float>(a, NH, d, stream);
}
