/*
 * efla.h — C ABI of the MI355X (gfx950) Exact Flow Linear Attention forward.
 *
 * The operation (papernotes.org note "Exact Flow Linear Attention: Exact
 * Solution from Continuous-Time Dynamics"):
 *   - section 关键设计 item 2: with lambda_t = ||k_t||^2, the exact-flow
 *     coefficient alpha_t = (1 - exp(-beta_t lambda_t)) / lambda_t and the
 *     update S_t = (I - alpha_t k_t k_t^T) S_{t-1} + alpha_t k_t v_t^T;
 *   - section 损失函数 / 训练策略: lambda is floored at 1e-12 and the numerator
 *     is -expm1(-beta lambda), evaluated in fp32 here;
 *   - section 整体框架 (flowchart node F): the output o_t = S_t^T q_t is read
 *     after the update;
 *   - section 整体框架 (last paragraph): the same recurrence runs either token
 *     by token (decode) or chunk-parallel in the WY/UT form of DeltaNet.
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are DEVICE pointers, contiguous, row-major, 16-byte
 *     aligned. The caller owns every buffer; the library never allocates,
 *     frees or synchronises, keeps no per-call state and is safe to call from
 *     several host threads.
 *   - q, k: [B, H, T, d_k]; v, o: [B, H, T, d_v]; beta: [B, H, T]; all in the
 *     element type `dt` (fp32 or bf16). The state is always fp32, laid out
 *     [B, H, d_k, d_v] with the row index running over the key dimension.
 *     Only d_k == d_v is supported.
 *   - No scaling is applied to q; o_t = S_t^T q_t exactly. bf16 outputs are
 *     rounded to nearest even from fp32 accumulators.
 *   - beta may be any finite real; NaN and Inf in the inputs propagate to the
 *     outputs and are not sanitised.
 *   - `stream` is a hipStream_t (NULL = the default stream). EFLA_OK means the
 *     work was enqueued on that stream; completion is observed through the
 *     stream (event or synchronise).
 *   - Argument errors are detected on the host before any launch; such a
 *     call returns the error code and writes nothing. A launch failure
 *     reported by the HIP runtime returns EFLA_ERR_HIP. No C++ exception
 *     crosses this interface.
 */
#ifndef EFLA_H
#define EFLA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * The enumerations below have int as their underlying type in C++ as well
 * (EFLA_ENUM), so any int a C or foreign-language caller passes is a valid
 * value of the parameter's type and reaches the validation, which rejects it
 * with EFLA_ERR_UNSUPPORTED; in C an enumeration already holds any int.
 */
#ifdef __cplusplus
#define EFLA_ENUM(name) enum name : int
#else
#define EFLA_ENUM(name) enum name
#endif

typedef EFLA_ENUM(efla_dtype_e) { EFLA_DTYPE_F32 = 0, EFLA_DTYPE_BF16 = 1 } efla_dtype;

/*
 * Scalar of the rank-1 step S_t = (I - c k k^T) S_{t-1} + c k v^T, with
 * x = beta lambda, lambda = ||k||^2 (every choice keeps the same update form,
 * so every kernel serves all four):
 *   EXACT   c = -expm1(-beta lambda~)/lambda~, lambda~ = max(lambda, 1e-12):
 *           the exact flow (papernotes note, 关键设计 item 2; default).
 *   EULER   c = beta: one explicit Euler step, the delta rule (same note,
 *           关键设计 item 1).
 *   RK4     c = beta (1 - x/2 + x^2/6 - x^3/24): one classical RK4 step; the
 *           matrix polynomial of the jsqmd.com article "EFLA注意力机制：优化挑战
 *           与训练策略解析", section 5.3, collapsed by A^n = lambda^(n-1) A.
 *   ORDER2  c = beta (1 - x/2): the same series cut after the second-order
 *           term, the second-order approximation that section names.
 * All four are evaluated in fp32. Only EXACT floors lambda.
 */
typedef EFLA_ENUM(efla_coef_e) {
  EFLA_COEF_EXACT = 0,
  EFLA_COEF_EULER = 1,
  EFLA_COEF_RK4 = 2,
  EFLA_COEF_ORDER2 = 3
} efla_coef;

typedef EFLA_ENUM(efla_status_e) {
  EFLA_OK = 0,
  EFLA_ERR_NULL_POINTER = 1, /* a required pointer is NULL */
  EFLA_ERR_BAD_SHAPE = 2,    /* B, H or T < 1, or d_k != d_v */
  EFLA_ERR_UNSUPPORTED = 3,  /* head dim, chunk size, dtype or coefficient outside the supported set */
  EFLA_ERR_MISALIGNED = 4,   /* a tensor pointer is not 16-byte aligned */
  EFLA_ERR_WORKSPACE = 5,    /* workspace smaller than efla_fwd_chunked_workspace_bytes() */
  EFLA_ERR_HIP = 6,          /* the HIP runtime reported an error at launch */
  EFLA_ERR_SCRATCH_LIMIT = 7 /* efla_fwd_chunked_noalloc: the sizes need more than its fixed scratch */
} efla_status;

/*
 * Bytes of device workspace efla_fwd_chunked needs for these sizes. It is 0
 * when one pass over the sequence fills the GPU. For few heads and long
 * sequences (fewer than 128 workgroups of 64 state columns, and at least 64
 * chunks; segments of at least 8 chunks, at most sqrt(chunks) + 1 of
 * them) the forward runs over nseg time
 * segments: the first segment from S0 beside the affine maps S -> P S + R of
 * segments 1 .. nseg - 2, then their composition, then every later segment
 * from its true start state (the chunk recurrence is affine in S, section
 * 整体框架 of the papernotes note); the workspace then holds, per head, those
 * maps (P, R) and a start state per segment: B H (3 nseg - 4) d_k d_v fp32
 * values.
 * Returns 0 for unsupported sizes as well; efla_fwd_chunked reports those.
 */
size_t efla_fwd_chunked_workspace_bytes(int B, int H, int T, int d_k, int d_v, int chunk,
                                        efla_dtype dt);

/*
 * Chunk-parallel EFLA forward over a whole sequence (WY/UT form; section
 * 整体框架 of the papernotes note).
 *   q, k, v   inputs as above, element type dt.
 *   beta      [B, H, T] step sizes, element type dt.
 *   s0        [B, H, d_k, d_v] fp32 initial state, or NULL for zeros.
 *   o         [B, H, T, d_v] output, element type dt.
 *   s_final   [B, H, d_k, d_v] fp32 final state S_T, or NULL to skip it. It
 *             may alias s0 (the state is then advanced in place).
 *   workspace, workspace_bytes   caller-owned device scratch of at least
 *             efla_fwd_chunked_workspace_bytes() bytes, 16-byte aligned (may
 *             be NULL/0 when that is 0). Its contents on entry do not matter
 *             and are overwritten; calls sharing one workspace must not
 *             overlap in time.
 *   chunk     tokens per chunk, one of 16, 32, 64. T need not be a multiple.
 *   coef      step coefficient (efla_coef; EFLA_COEF_EXACT for EFLA itself).
 * Supported (d, chunk, dtype): d in {16, 32, 64, 128}; chunk in {16, 32, 64}.
 * fp32 with chunk 64 runs with 32-token chunks when B H d / min(d, 64) >=
 * 128 and with 16-token chunks otherwise (64-token fp32 tiles do not fit the
 * pipelined kernel's LDS); the chunk length changes only the rounding order.
 * Anything else: EFLA_ERR_UNSUPPORTED.
 */
efla_status efla_fwd_chunked(const void* q, const void* k, const void* v, const void* beta,
                             const float* s0, void* o, float* s_final, void* workspace,
                             size_t workspace_bytes, int B, int H, int T, int d_k, int d_v,
                             int chunk, efla_coef coef, efla_dtype dt, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * efla_fwd_chunked with no workspace argument. Arguments, layouts, results
 * and errors are those of efla_fwd_chunked. Where efla_fwd_chunked needs a
 * workspace (the time-segmented path), this call uses a fixed device array
 * of EFLA_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, held until
 * the process ends; every size the segmented path takes fits (at most
 * 383 d^2 fp32 values), and a size that would not returns
 * EFLA_ERR_SCRATCH_LIMIT before any launch. The call itself allocates
 * nothing (no hipMalloc, hipFree or allocating library routine); its first
 * call on a device that needs the array looks up its device address. All
 * calls on one GPU share that array: calls that overlap in time on one GPU
 * (other streams, other host threads) must not be made.
 */
#define EFLA_NOALLOC_SCRATCH_BYTES (24u << 20)
efla_status efla_fwd_chunked_noalloc(const void* q, const void* k, const void* v, const void* beta,
                                     const float* s0, void* o, float* s_final, int B, int H, int T,
                                     int d_k, int d_v, int chunk, efla_coef coef, efla_dtype dt,
                                     void* stream);

/*
 * One token per head, token-serial (the recurrent decode form; section 整体框架
 * of the papernotes note).
 *   q, k      [B, H, d_k], element type dt.
 *   v         [B, H, d_v], element type dt.
 *   beta      [B, H], element type dt.
 *   state     [B, H, d_k, d_v] fp32; read, then overwritten with S_t.
 *   o         [B, H, d_v] output S_t^T q_t, element type dt.
 *   coef      step coefficient (efla_coef), as in efla_fwd_chunked.
 * Supported: d in {16, 32, 64, 128}, fp32 or bf16.
 */
efla_status efla_fwd_recurrent_step(const void* q, const void* k, const void* v,
                                    const void* beta, float* state, void* o, int B, int H,
                                    int d_k, int d_v, efla_coef coef, efla_dtype dt,
                                    void* stream);

/*
 * Gated EFLA. The papernotes note lists a gated variant ("Gated EFLA", main
 * results table) and states that the exact flow upgrades Gated DeltaNet and
 * any other delta-rule variant (key findings), without printing its update.
 * The reading implemented: Gated DeltaNet's update with the exact-flow
 * coefficient,
 *   S_t = g_t (I - c_t k_t k_t^T) S_{t-1} + c_t k_t v_t^T,  o_t = S_t^T q_t,
 * with the per-token decay g_t = exp(log_g_t) given as its natural log.
 * log_g = 0 everywhere gives efla_fwd_chunked's recurrence.
 *   log_g     [B, H, T] fp32 log-decays (4-byte aligned); values <= 0 keep
 *             every decay factor the kernel forms at most 1.
 * Every other argument, layout, supported size and error as in
 * efla_fwd_chunked; no workspace is needed (one pass per head and column
 * slice).
 */
efla_status efla_fwd_chunked_gated(const void* q, const void* k, const void* v, const void* beta,
                                   const float* log_g, const float* s0, void* o, float* s_final,
                                   int B, int H, int T, int d_k, int d_v, int chunk, efla_coef coef,
                                   efla_dtype dt, void* stream);

/*
 * One gated token per head (the decode form of efla_fwd_chunked_gated):
 * log_g is [B, H] fp32; every other argument as in efla_fwd_recurrent_step.
 */
efla_status efla_fwd_recurrent_step_gated(const void* q, const void* k, const void* v,
                                          const void* beta, const float* log_g, float* state,
                                          void* o, int B, int H, int d_k, int d_v, efla_coef coef,
                                          efla_dtype dt, void* stream);

/*
 * Bytes of device workspace efla_bwd_chunked needs: per head, the state at
 * the start of every chunk in two layouts and the state gradient at the end
 * of every chunk (3 nchunks d^2 fp32), one d-wide fp32 row per token, three
 * scalars per token and four C x C fp32 matrices per chunk. Never 0 for supported sizes; 0 for
 * unsupported ones.
 */
size_t efla_bwd_chunked_workspace_bytes(int B, int H, int T, int d_k, int d_v, int chunk,
                                        efla_dtype dt);

/*
 * Backward of efla_fwd_chunked: the gradients of a loss L(o, S_T) with
 * respect to q, k, v, beta and s0, given dout = dL/do and ds_final = dL/dS_T.
 * The pages give no gradient formulas; this is reverse mode through the
 * forward as defined above (the chunk form of section 整体框架 of the
 * papernotes note, with the step scalar of coef and its derivatives in beta
 * and lambda; the exact flow's lambda floor makes its scalar constant in
 * lambda below 1e-12).
 *   q, k, v, beta, s0, chunk, coef, dt   exactly as passed to the forward.
 *   dout      [B, H, T, d_v], element type dt.
 *   ds_final  [B, H, d_k, d_v] fp32, or NULL for zero.
 *   dq, dk    [B, H, T, d_k], dv [B, H, T, d_v], dbeta [B, H, T]: outputs,
 *             element type dt (RNE from fp32). They must not alias inputs.
 *   ds0       [B, H, d_k, d_v] fp32 output dL/dS0, or NULL to skip it.
 *   workspace, workspace_bytes   caller-owned, 16-byte aligned, at least
 *             efla_bwd_chunked_workspace_bytes() bytes (required); contents
 *             on entry do not matter; calls sharing one must not overlap.
 * The forward is recomputed inside (the chunk-start states go to the
 * workspace). Numerics: for fp32 inputs every product is fp32 MFMA with fp32
 * storage. For bf16 inputs with chunk and d multiples of 32, the products
 * take bf16 MFMA operands (the saved chunk-start states, T^T, M^T, T diag(c)
 * and the state gradients are stored as bf16, which is exactly the rounding
 * their consumers apply; so is G = T^T dU, whose one fp32 use, a row sum in
 * dc, then takes the rounded value) and accumulate in fp32; other bf16
 * shapes run the fp32 form. The gate, its derivatives and every accumulator are fp32. Supported sizes are
 * the forward's; where the forward's pipelined kernel does not serve the
 * chunk size, the backward runs with chunk 32 (same result up to rounding).
 * Errors as for efla_fwd_chunked; a missing or short workspace is
 * EFLA_ERR_WORKSPACE.
 */
efla_status efla_bwd_chunked(const void* q, const void* k, const void* v, const void* beta,
                             const float* s0, const void* dout, const float* ds_final, void* dq,
                             void* dk, void* dv, void* dbeta, float* ds0, void* workspace,
                             size_t workspace_bytes, int B, int H, int T, int d_k, int d_v, int chunk,
                             efla_coef coef, efla_dtype dt, void* stream);

/*
 * Forward of a training step: exactly the outputs of efla_fwd_chunked (o and,
 * if not NULL, s_final; equal up to rounding order), and in the same call the
 * state at the start of every chunk, written into the backward's workspace,
 * so that efla_bwd_chunked_saved can skip the forward that efla_bwd_chunked
 * recomputes. The chunk form and the state update are those of
 * efla_fwd_chunked (section 整体框架 of the papernotes note).
 *   q, k, v, beta, s0, o, s_final, chunk, coef, dt   as for efla_fwd_chunked
 *             (s_final may alias s0).
 *   bwd_workspace, bwd_workspace_bytes   caller-owned device memory of at
 *             least efla_bwd_chunked_workspace_bytes() bytes for the same
 *             sizes, 16-byte aligned (required). On return it holds the
 *             chunk-start states; pass it unchanged to efla_bwd_chunked_saved.
 * Where the pipelined kernel serves the chunk size this is one pass; otherwise
 * the states pass runs first and the plain forward after it. Errors as for
 * efla_fwd_chunked; a missing or short workspace is EFLA_ERR_WORKSPACE.
 */
efla_status efla_fwd_chunked_train(const void* q, const void* k, const void* v, const void* beta,
                                   const float* s0, void* o, float* s_final, void* bwd_workspace,
                                   size_t bwd_workspace_bytes, int B, int H, int T, int d_k, int d_v,
                                   int chunk, efla_coef coef, efla_dtype dt, void* stream);

/*
 * efla_bwd_chunked without the recomputed forward: the chunk-start states are
 * taken from `workspace`, which efla_fwd_chunked_train filled for the same
 * q, k, v, beta, s0, sizes, chunk, coef and dt (s0 itself is not read again).
 * All other arguments, outputs and errors are those of efla_bwd_chunked; the
 * gradients are the same. The workspace must not have been used by another
 * call in between.
 */
efla_status efla_bwd_chunked_saved(const void* q, const void* k, const void* v, const void* beta,
                                   const void* dout, const float* ds_final, void* dq, void* dk, void* dv,
                                   void* dbeta, float* ds0, void* workspace, size_t workspace_bytes, int B,
                                   int H, int T, int d_k, int d_v, int chunk, efla_coef coef, efla_dtype dt,
                                   void* stream);

/* Static, human-readable name of a status code. Never NULL. */
const char* efla_status_string(efla_status s);

#ifdef __cplusplus
}
#endif

#endif /* EFLA_H */
