// Measurement-only kernels for the benchmark: the achievable MFMA rate and
// HBM streaming bandwidth of the GPU the benchmark runs on, so that roofline
// fractions can be given against measured peaks as well as the vendor's.
// Built into libefla_bench.so, which only bench.py loads; nothing of the
// EFLA path calls it.

#include <hip/hip_runtime.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

// NCH independent accumulation chains of v_mfma_f32_32x32x16_bf16 per wave,
// iters steps each; the operands are loop-invariant registers, so the loop
// is MFMA issue only. The sums are written out so nothing is removed.
template <int NCH>
__global__ __launch_bounds__(256) void mfma_bf16_loop(float* out, int iters) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(0.001f * (lane + e));
    b[e] = (__bf16)(0.002f * (lane - e));
  }
  floatx16 c[NCH];
  for (int i = 0; i < NCH; ++i) c[i] = floatx16{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) c[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[i], 0, 0, 0);
  }
  float s = 0.f;
  for (int i = 0; i < NCH; ++i)
    for (int e = 0; e < 16; ++e) s += c[i][e];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

template <int NCH>
__global__ __launch_bounds__(256) void mfma_f32_loop(float* out, int iters) {
  const int lane = threadIdx.x & 63;
  const float a = 0.001f * lane, b = 0.002f * (64 - lane);
  floatx4 c[NCH];
  for (int i = 0; i < NCH; ++i) c[i] = floatx4{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) c[i] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c[i], 0, 0, 0);
  }
  float s = 0.f;
  for (int i = 0; i < NCH; ++i)
    for (int e = 0; e < 4; ++e) s += c[i][e];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// dst[i] = src[i] over n float4 elements, 16-byte accesses: each thread
// issues four loads before its four stores (four requests in flight), then
// moves on by four grid strides.
__global__ __launch_bounds__(256) void stream_copy(const floatx4* __restrict__ src, floatx4* __restrict__ dst,
                                                   long long n) {
  const long long stride = (long long)gridDim.x * blockDim.x;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += 4 * stride) {
    floatx4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (i + u * stride < n) v[u] = __builtin_nontemporal_load(&src[i + u * stride]);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (i + u * stride < n) __builtin_nontemporal_store(v[u], &dst[i + u * stride]);
  }
}

}  // namespace

// Each returns the runtime status of the launch; the caller times the
// launch with events on `stream`. `out` must hold blocks * 256 floats.
extern "C" int efla_bench_mfma_bf16(float* out, int blocks, int iters, void* stream) {
  hipLaunchKernelGGL((mfma_bf16_loop<4>), dim3(blocks), dim3(256), 0, (hipStream_t)stream, out, iters);
  return (int)hipGetLastError();
}
// flops of one launch: blocks * 4 waves * 4 chains * iters * 2*32*32*16
extern "C" double efla_bench_mfma_bf16_flops(int blocks, int iters) {
  return (double)blocks * 4 * 4 * iters * 2.0 * 32 * 32 * 16;
}

extern "C" int efla_bench_mfma_f32(float* out, int blocks, int iters, void* stream) {
  hipLaunchKernelGGL((mfma_f32_loop<4>), dim3(blocks), dim3(256), 0, (hipStream_t)stream, out, iters);
  return (int)hipGetLastError();
}
extern "C" double efla_bench_mfma_f32_flops(int blocks, int iters) {
  return (double)blocks * 4 * 4 * iters * 2.0 * 16 * 16 * 4;
}

// n16: number of 16-byte elements; src and dst must each hold n16 * 16 bytes.
extern "C" int efla_bench_copy(const void* src, void* dst, long long n16, int blocks, void* stream) {
  hipLaunchKernelGGL(stream_copy, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (const floatx4*)src,
                     (floatx4*)dst, n16);
  return (int)hipGetLastError();
}
