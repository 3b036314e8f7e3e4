// C ABI of the EFLA forward library: argument validation on the host, then
// dispatch to the gfx950 kernels. Nothing here allocates, frees or
// synchronises; every launch goes to the caller's stream.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "efla.h"

hipError_t efla_internal_launch_chunked(const void* q, const void* k, const void* v,
                                        const void* beta, const float* s0, void* o,
                                        float* s_final, void* workspace, int NH, int T, int d,
                                        int chunk, int coef, int is_bf16, hipStream_t stream);
size_t efla_internal_chunked_workspace_bytes(int NH, int T, int d, int chunk, int is_bf16);
hipError_t efla_internal_launch_decode(const void* q, const void* k, const void* v,
                                       const void* beta, const float* log_g, float* state, void* o,
                                       int NH, int d, int coef, int is_bf16, hipStream_t stream);
hipError_t efla_internal_launch_chunked_gated(const void* q, const void* k, const void* v, const void* beta,
                                              const float* log_g, const float* s0, void* o, float* s_final,
                                              int NH, int T, int d, int chunk, int coef, int is_bf16,
                                              hipStream_t stream);

size_t efla_internal_bwd_workspace_bytes(int NH, int T, int d, int chunk, int is_bf16);
hipError_t efla_internal_launch_bwd(const void* q, const void* k, const void* v, const void* beta,
                                    const float* s0, const void* dout, const float* dsT, void* dq, void* dk,
                                    void* dv, void* dbeta, float* ds0, void* workspace, int NH, int T, int d,
                                    int chunk, int coef, int is_bf16, int states_saved, hipStream_t stream);
hipError_t efla_internal_launch_fwd_save(const void* q, const void* k, const void* v, const void* beta,
                                         const float* s0, void* o, float* s_final, void* workspace, int NH, int T,
                                         int d, int chunk, int coef, int is_bf16, hipStream_t stream);

namespace {

bool aligned16(const void* p) { return p == nullptr || (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool elem_aligned(const void* p, efla_dtype dt) {
  const uintptr_t m = dt == EFLA_DTYPE_F32 ? 3u : 1u;
  return (reinterpret_cast<uintptr_t>(p) & m) == 0;
}

bool coef_ok(efla_coef c) {
  return c == EFLA_COEF_EXACT || c == EFLA_COEF_EULER || c == EFLA_COEF_RK4 ||
         c == EFLA_COEF_ORDER2;
}

bool head_dim_ok(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }

bool chunked_supported(int d, int chunk, efla_dtype) {
  if (!head_dim_ok(d)) return false;
  return chunk == 16 || chunk == 32 || chunk == 64;
}

}  // namespace

extern "C" size_t efla_fwd_chunked_workspace_bytes(int B, int H, int T, int d_k, int d_v,
                                                   int chunk, efla_dtype dt) {
  if (B < 1 || H < 1 || T < 1 || d_k != d_v) return 0;
  if (dt != EFLA_DTYPE_F32 && dt != EFLA_DTYPE_BF16) return 0;
  if (!chunked_supported(d_k, chunk, dt)) return 0;
  if ((long long)B * H > (1LL << 30) || (long long)T > (1LL << 30)) return 0;
  // nonzero only for the time-segmented schedule (few heads, long sequences):
  // per head and segment, the segment's affine map and its start state
  return efla_internal_chunked_workspace_bytes(B * H, T, d_k, chunk, dt == EFLA_DTYPE_BF16);
}

extern "C" efla_status efla_fwd_chunked(const void* q, const void* k, const void* v,
                                        const void* beta, const float* s0, void* o,
                                        float* s_final, void* workspace, size_t workspace_bytes,
                                        int B, int H, int T, int d_k, int d_v, int chunk,
                                        efla_coef coef, efla_dtype dt, void* stream) {
  if (!q || !k || !v || !beta || !o) return EFLA_ERR_NULL_POINTER;
  if (B < 1 || H < 1 || T < 1 || d_k != d_v) return EFLA_ERR_BAD_SHAPE;
  if (dt != EFLA_DTYPE_F32 && dt != EFLA_DTYPE_BF16) return EFLA_ERR_UNSUPPORTED;
  if (!chunked_supported(d_k, chunk, dt) || !coef_ok(coef)) return EFLA_ERR_UNSUPPORTED;
  if ((long long)B * H > (1LL << 30) || (long long)T > (1LL << 30)) return EFLA_ERR_BAD_SHAPE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(s0) ||
      !aligned16(s_final) || !aligned16(workspace) || !elem_aligned(beta, dt))
    return EFLA_ERR_MISALIGNED;
  const size_t need = efla_fwd_chunked_workspace_bytes(B, H, T, d_k, d_v, chunk, dt);
  if (workspace_bytes < need || (need > 0 && workspace == nullptr)) return EFLA_ERR_WORKSPACE;
  const hipError_t e = efla_internal_launch_chunked(q, k, v, beta, s0, o, s_final, workspace,
                                                    B * H, T, d_k, chunk, (int)coef,
                                                    dt == EFLA_DTYPE_BF16,
                                                    static_cast<hipStream_t>(stream));
  return e == hipSuccess ? EFLA_OK : EFLA_ERR_HIP;
}

extern "C" efla_status efla_fwd_recurrent_step(const void* q, const void* k, const void* v,
                                               const void* beta, float* state, void* o, int B,
                                               int H, int d_k, int d_v, efla_coef coef,
                                               efla_dtype dt, void* stream) {
  if (!q || !k || !v || !beta || !state || !o) return EFLA_ERR_NULL_POINTER;
  if (B < 1 || H < 1 || d_k != d_v) return EFLA_ERR_BAD_SHAPE;
  if (dt != EFLA_DTYPE_F32 && dt != EFLA_DTYPE_BF16) return EFLA_ERR_UNSUPPORTED;
  if (!head_dim_ok(d_k) || !coef_ok(coef)) return EFLA_ERR_UNSUPPORTED;
  if ((long long)B * H > (1LL << 30)) return EFLA_ERR_BAD_SHAPE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(state) ||
      !elem_aligned(beta, dt))
    return EFLA_ERR_MISALIGNED;
  const hipError_t e = efla_internal_launch_decode(q, k, v, beta, nullptr, state, o, B * H, d_k,
                                                   (int)coef, dt == EFLA_DTYPE_BF16,
                                                   static_cast<hipStream_t>(stream));
  return e == hipSuccess ? EFLA_OK : EFLA_ERR_HIP;
}

extern "C" efla_status efla_fwd_recurrent_step_gated(const void* q, const void* k, const void* v,
                                                     const void* beta, const float* log_g, float* state,
                                                     void* o, int B, int H, int d_k, int d_v,
                                                     efla_coef coef, efla_dtype dt, void* stream) {
  if (!q || !k || !v || !beta || !log_g || !state || !o) return EFLA_ERR_NULL_POINTER;
  if (B < 1 || H < 1 || d_k != d_v) return EFLA_ERR_BAD_SHAPE;
  if (dt != EFLA_DTYPE_F32 && dt != EFLA_DTYPE_BF16) return EFLA_ERR_UNSUPPORTED;
  if (!head_dim_ok(d_k) || !coef_ok(coef)) return EFLA_ERR_UNSUPPORTED;
  if ((long long)B * H > (1LL << 30)) return EFLA_ERR_BAD_SHAPE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(state) ||
      !elem_aligned(beta, dt) || !elem_aligned(log_g, EFLA_DTYPE_F32))
    return EFLA_ERR_MISALIGNED;
  const hipError_t e = efla_internal_launch_decode(q, k, v, beta, log_g, state, o, B * H, d_k, (int)coef,
                                                   dt == EFLA_DTYPE_BF16, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? EFLA_OK : EFLA_ERR_HIP;
}

extern "C" efla_status efla_fwd_chunked_gated(const void* q, const void* k, const void* v, const void* beta,
                                              const float* log_g, const float* s0, void* o, float* s_final,
                                              int B, int H, int T, int d_k, int d_v, int chunk, efla_coef coef,
                                              efla_dtype dt, void* stream) {
  if (!q || !k || !v || !beta || !log_g || !o) return EFLA_ERR_NULL_POINTER;
  if (B < 1 || H < 1 || T < 1 || d_k != d_v) return EFLA_ERR_BAD_SHAPE;
  if (dt != EFLA_DTYPE_F32 && dt != EFLA_DTYPE_BF16) return EFLA_ERR_UNSUPPORTED;
  if (!chunked_supported(d_k, chunk, dt) || !coef_ok(coef)) return EFLA_ERR_UNSUPPORTED;
  if ((long long)B * H > (1LL << 30) || (long long)T > (1LL << 30)) return EFLA_ERR_BAD_SHAPE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(s0) ||
      !aligned16(s_final) || !elem_aligned(beta, dt) || !elem_aligned(log_g, EFLA_DTYPE_F32))
    return EFLA_ERR_MISALIGNED;
  const hipError_t e = efla_internal_launch_chunked_gated(q, k, v, beta, log_g, s0, o, s_final, B * H, T, d_k,
                                                          chunk, (int)coef, dt == EFLA_DTYPE_BF16,
                                                          static_cast<hipStream_t>(stream));
  return e == hipSuccess ? EFLA_OK : EFLA_ERR_HIP;
}

extern "C" size_t efla_bwd_chunked_workspace_bytes(int B, int H, int T, int d_k, int d_v, int chunk,
                                                  efla_dtype dt) {
  if (B < 1 || H < 1 || T < 1 || d_k != d_v) return 0;
  if (dt != EFLA_DTYPE_F32 && dt != EFLA_DTYPE_BF16) return 0;
  if (!chunked_supported(d_k, chunk, dt)) return 0;
  if ((long long)B * H > (1LL << 30) || (long long)T > (1LL << 30)) return 0;
  return efla_internal_bwd_workspace_bytes(B * H, T, d_k, chunk, dt == EFLA_DTYPE_BF16);
}

namespace {
efla_status bwd_common(const void* q, const void* k, const void* v, const void* beta, const float* s0,
                       const void* dout, const float* ds_final, void* dq, void* dk, void* dv, void* dbeta,
                       float* ds0, void* workspace, size_t workspace_bytes, int B, int H, int T, int d_k, int d_v,
                       int chunk, efla_coef coef, efla_dtype dt, int states_saved, void* stream) {
  if (!q || !k || !v || !beta || !dout || !dq || !dk || !dv || !dbeta) return EFLA_ERR_NULL_POINTER;
  if (B < 1 || H < 1 || T < 1 || d_k != d_v) return EFLA_ERR_BAD_SHAPE;
  if (dt != EFLA_DTYPE_F32 && dt != EFLA_DTYPE_BF16) return EFLA_ERR_UNSUPPORTED;
  if (!chunked_supported(d_k, chunk, dt) || !coef_ok(coef)) return EFLA_ERR_UNSUPPORTED;
  if ((long long)B * H > (1LL << 30) || (long long)T > (1LL << 30)) return EFLA_ERR_BAD_SHAPE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dout) || !aligned16(s0) ||
      !aligned16(ds_final) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned16(ds0) ||
      !aligned16(workspace) || !elem_aligned(beta, dt) || !elem_aligned(dbeta, dt))
    return EFLA_ERR_MISALIGNED;
  const size_t need = efla_bwd_chunked_workspace_bytes(B, H, T, d_k, d_v, chunk, dt);
  if (need == 0 || workspace == nullptr || workspace_bytes < need) return EFLA_ERR_WORKSPACE;
  const hipError_t e = efla_internal_launch_bwd(q, k, v, beta, s0, dout, ds_final, dq, dk, dv, dbeta, ds0,
                                                workspace, B * H, T, d_k, chunk, (int)coef,
                                                dt == EFLA_DTYPE_BF16, states_saved,
                                                static_cast<hipStream_t>(stream));
  return e == hipSuccess ? EFLA_OK : EFLA_ERR_HIP;
}
}  // namespace

extern "C" efla_status efla_bwd_chunked(const void* q, const void* k, const void* v, const void* beta,
                                        const float* s0, const void* dout, const float* ds_final, void* dq,
                                        void* dk, void* dv, void* dbeta, float* ds0, void* workspace,
                                        size_t workspace_bytes, int B, int H, int T, int d_k, int d_v,
                                        int chunk, efla_coef coef, efla_dtype dt, void* stream) {
  return bwd_common(q, k, v, beta, s0, dout, ds_final, dq, dk, dv, dbeta, ds0, workspace, workspace_bytes, B, H,
                    T, d_k, d_v, chunk, coef, dt, 0, stream);
}

extern "C" efla_status efla_bwd_chunked_saved(const void* q, const void* k, const void* v, const void* beta,
                                              const void* dout, const float* ds_final, void* dq, void* dk,
                                              void* dv, void* dbeta, float* ds0, void* workspace,
                                              size_t workspace_bytes, int B, int H, int T, int d_k, int d_v,
                                              int chunk, efla_coef coef, efla_dtype dt, void* stream) {
  return bwd_common(q, k, v, beta, nullptr, dout, ds_final, dq, dk, dv, dbeta, ds0, workspace, workspace_bytes,
                    B, H, T, d_k, d_v, chunk, coef, dt, 1, stream);
}

extern "C" efla_status efla_fwd_chunked_train(const void* q, const void* k, const void* v, const void* beta,
                                              const float* s0, void* o, float* s_final, void* bwd_workspace,
                                              size_t bwd_workspace_bytes, int B, int H, int T, int d_k, int d_v,
                                              int chunk, efla_coef coef, efla_dtype dt, void* stream) {
  if (!q || !k || !v || !beta || !o) return EFLA_ERR_NULL_POINTER;
  if (B < 1 || H < 1 || T < 1 || d_k != d_v) return EFLA_ERR_BAD_SHAPE;
  if (dt != EFLA_DTYPE_F32 && dt != EFLA_DTYPE_BF16) return EFLA_ERR_UNSUPPORTED;
  if (!chunked_supported(d_k, chunk, dt) || !coef_ok(coef)) return EFLA_ERR_UNSUPPORTED;
  if ((long long)B * H > (1LL << 30) || (long long)T > (1LL << 30)) return EFLA_ERR_BAD_SHAPE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(s0) ||
      !aligned16(s_final) || !aligned16(bwd_workspace) || !elem_aligned(beta, dt))
    return EFLA_ERR_MISALIGNED;
  const size_t need = efla_bwd_chunked_workspace_bytes(B, H, T, d_k, d_v, chunk, dt);
  if (need == 0 || bwd_workspace == nullptr || bwd_workspace_bytes < need) return EFLA_ERR_WORKSPACE;
  const hipError_t e = efla_internal_launch_fwd_save(q, k, v, beta, s0, o, s_final, bwd_workspace, B * H, T, d_k,
                                                     chunk, (int)coef, dt == EFLA_DTYPE_BF16,
                                                     static_cast<hipStream_t>(stream));
  return e == hipSuccess ? EFLA_OK : EFLA_ERR_HIP;
}

extern "C" const char* efla_status_string(efla_status s) {
  switch (s) {
    case EFLA_OK: return "EFLA_OK";
    case EFLA_ERR_NULL_POINTER: return "EFLA_ERR_NULL_POINTER: a required pointer is NULL";
    case EFLA_ERR_BAD_SHAPE: return "EFLA_ERR_BAD_SHAPE: B, H, T < 1, sizes too large, or d_k != d_v";
    case EFLA_ERR_UNSUPPORTED: return "EFLA_ERR_UNSUPPORTED: head dim, chunk size, dtype or coefficient not supported";
    case EFLA_ERR_MISALIGNED: return "EFLA_ERR_MISALIGNED: tensor pointer not 16-byte aligned";
    case EFLA_ERR_WORKSPACE: return "EFLA_ERR_WORKSPACE: workspace too small";
    case EFLA_ERR_HIP: return "EFLA_ERR_HIP: the HIP runtime reported a launch error";
    case EFLA_ERR_SCRATCH_LIMIT:
      return "EFLA_ERR_SCRATCH_LIMIT: the sizes need more workspace than the no-allocation entry's fixed scratch";
  }
  return "EFLA_ERR_UNKNOWN";
}
