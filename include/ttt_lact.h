/*
 * ttt_lact.h -- C ABI of the MI355X (gfx950) chunked TTT-KVB fast-weight library.
 *
 * Three forward entry points, one per form of the layer:
 *
 *   ttt_lact_forward          the chunked LaCT layer: SwiGLU fast weight, gradient of the
 *                             eta-weighted negative inner-product loss, optional heavy-ball
 *                             momentum, optional Newton-Schulz-5 orthogonalisation, optional
 *                             input-dim weight renormalisation, apply-then-update or
 *                             update-then-apply order.
 *   ttt_linattn_forward       the last-layer-only linear-attention form: a chunk-level prefix
 *                             scan of phi(K)^T (eta * V) with the static map
 *                             phi(x) = silu(x W0) * (x W2), and O = phi(Q) S.
 *   ttt_inplace_down_forward  the In-Place TTT MLP down-projection update.
 *
 * Conventions common to all entry points
 * --------------------------------------
 * - Row-vector convention. All arrays are dense, contiguous, row-major, in device memory.
 * - "I/O dtype" (TTT_BF16 or TTT_FP32) is the element type of the token tensors (Q, K, V, O,
 *   H, Vbar) and of the In-Place slow weights. Fast-weight state, momentum and step sizes are
 *   always float32. Accumulation is always float32.
 * - Ownership: the caller owns every buffer. The entry points never allocate, free or
 *   synchronise device memory; apart from the optional timing recorder (ttt_timing_*) the
 *   library keeps no mutable global state and is re-entrant for calls with distinct
 *   workspaces. Inputs are read only. Outputs are fully overwritten and must not alias inputs.
 * - Workspace: pass workspace == NULL to query; the required size in bytes is written to
 *   *workspace_bytes, TTT_OK is returned and nothing is launched. Otherwise *workspace_bytes
 *   must hold the size of the buffer (at least the queried size, 256-byte aligned base).
 * - Validation happens before any launch: NULL required pointers, negative sizes or a bad
 *   enum give TTT_ERR_ARG; inconsistent shapes give TTT_ERR_SHAPE; combinations this build
 *   does not implement give TTT_ERR_UNSUPPORTED; a short workspace gives TTT_ERR_WORKSPACE.
 *   A failed HIP launch gives TTT_ERR_HIP. Execution is asynchronous on `stream` (a
 *   hipStream_t passed as void*; NULL is the null stream); device faults surface at the
 *   caller's next synchronisation. NaN/Inf inputs propagate and are not checked.
 * - Zero-length sequences (N == 0) and empty batches are valid: nothing is computed and the
 *   final-state outputs receive the initial state.
 * - No exception or abort crosses this ABI.
 */
#ifndef TTT_LACT_H
#define TTT_LACT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t ttt_status;
#define TTT_OK 0
#define TTT_ERR_ARG (-1)
#define TTT_ERR_SHAPE (-2)
#define TTT_ERR_UNSUPPORTED (-3)
#define TTT_ERR_WORKSPACE (-4)
#define TTT_ERR_HIP (-5)

/* Order of the fast-weight operations within a chunk. The language-model layer applies the
 * history state to the chunk's queries and then writes the chunk ("Test-Time Training Done
 * Right" reading notes, section 2.3, autoregressive row); set / view-synthesis layers write
 * first and then read (same section, full-set row). */
#define TTT_APPLY_THEN_UPDATE 0
#define TTT_UPDATE_THEN_APPLY 1

/* I/O element type. */
#define TTT_FP32 0
#define TTT_BF16 1

/* Which fast-weight matrices a LaCT call writes (bit mask). Writing only W1 is the
 * "update the last layer only" simplification of the KV-binding paper (summary page,
 * "Method step details", step 1). */
#define TTT_UPD_W0 1u
#define TTT_UPD_W1 2u
#define TTT_UPD_W2 4u

/* ------------------------------------------------------------------------------------------
 * ttt_lact_forward
 *
 * Defined by: the KV-binding paper's summary page, "Prerequisites -> LaCT" (bias-free SwiGLU
 * fast weight f(x) = (silu(x W0) * (x W2)) W1, loss -<f(k), v>, per-token eta, momentum,
 * Muon-style orthogonalisation); "Test-Time Training Done Right" reading notes, sections 2.1
 * (symbols h, r, b, eta), 2.2 (gradient / Muon write, five Newton-Schulz rounds with
 * coefficients 3.4445, -4.7750, 2.0315, input-dim renormalisation back to the original norm,
 * momentum fed to the operator) and 2.3 (order); "In-Place Test-Time Training" notes,
 * section 3.1 (all tokens of a chunk take their gradient at the chunk-start weights).
 *
 * Per (sequence b, head) pair and chunk c, with rh = r*h and Vt = diag(eta_c) V_c:
 *   apply   O_c = (silu(Q_c W0) * (Q_c W2)) W1
 *   grads   A = K_c W0, Bm = K_c W2, D = Vt W1^T,
 *           G1 = -(silu(A)*Bm)^T Vt, G0 = -K_c^T (D*Bm*silu'(A)), G2 = -K_c^T (D*silu(A))
 *   write   for each matrix X in update_mask:
 *             U = G_X; if momentum != 0: M_X = momentum*M_X + G_X, U = M_X
 *             if muon: U = NS5(U)  (U/(||U||_F + eps_ns), five rounds on the wide orientation)
 *             W_X = W_X - U
 *             if weight_norm: W_X[:, j] *= nu_j / (||W_X[:, j]||_2 + eps_norm), nu = the
 *             column norms (over the input axis) of W_X at the start of the call
 * Order per `order`.
 *
 * Arguments (all device pointers):
 *   Q       [B, H, Nq, h]   I/O dtype        queries
 *   K, V    [B, H, Nk, h]   I/O dtype        keys, values
 *   eta     [B, H, Nk]      float32          per-token step sizes
 *   W0, W2  [H, h, rh]      float32          initial fast weights; if w_batch_stride != 0 the
 *   W1      [H, rh, h]      float32          arrays are [B, H, ...] (per sequence) and
 *                                            w_batch_stride is the element stride between
 *                                            sequences of W0 (= H*h*rh); W1/W2 use the same
 *   M_in    [B, H, 3, h*rh] float32, nullable: initial momentum for (W0 [h,rh], W1 [rh,h],
 *                                            W2 [h,rh]); NULL means zeros
 *   O       [B, H, Nq, h]   I/O dtype        output
 *   W0_out, W2_out [B, H, h, rh], W1_out [B, H, rh, h] float32, nullable: final fast weights
 *   M_out   [B, H, 3, h*rh] float32, nullable: final momentum
 * Shape rules: Nq/chunk_q == Nk/chunk_kv (number of chunks); a ragged last chunk is rejected
 * (TTT_ERR_SHAPE); h a multiple of 32 and r >= 1 with r*h a multiple of 64, r*h <= 1024;
 * this build implements h <= 192 in TTT_BF16 mode and h <= 64 in TTT_FP32 mode
 * (TTT_ERR_UNSUPPORTED otherwise).
 * Precision: in TTT_BF16 mode the per-chunk products use fp16 MFMA operands (bf16 inputs
 * convert exactly) and Newton-Schulz uses split-bf16 operands; fp32 state throughout. In
 * TTT_FP32 mode all operands are fp32.
 * ---------------------------------------------------------------------------------------- */
typedef struct {
  int32_t B, H;
  int32_t Nq, Nk;
  int32_t h, r;
  int32_t chunk_q, chunk_kv;
  int32_t order;         /* TTT_APPLY_THEN_UPDATE or TTT_UPDATE_THEN_APPLY */
  int32_t dtype;         /* TTT_FP32 or TTT_BF16 */
  uint32_t update_mask;  /* TTT_UPD_* bits; default all three */
  int32_t weight_norm;   /* 0 or 1; default 1 */
  int32_t muon;          /* 0 or 1; default 0 */
  float momentum;        /* heavy-ball coefficient; 0 disables the momentum buffer */
  float eps_norm;        /* default 1e-5 */
  float eps_ns;          /* default 1e-7 */
  int64_t w_batch_stride;/* 0: weights shared by the batch; else element stride per sequence */
} ttt_lact_params;

ttt_status ttt_lact_forward(const ttt_lact_params* p,
                            const void* Q, const void* K, const void* V, const float* eta,
                            const float* W0, const float* W1, const float* W2, const float* M_in,
                            void* O, float* W0_out, float* W1_out, float* W2_out, float* M_out,
                            void* workspace, size_t* workspace_bytes, void* stream);

/* ------------------------------------------------------------------------------------------
 * ttt_linattn_forward
 *
 * Defined by: the KV-binding paper's summary page, "Prerequisites -> Linear attention"
 * (o = phi(q) S, S = S0 + sum_i phi(k_i)^T v_i) and "Method step details" (Theorem 5.2: the
 * unrolled last-layer write W_{t+1} = W_0 + sum_i phi_i(k_i)^T g_i(k_i), g = eta v); the press
 * article on the same paper, section 4 (with a static kernel and no renormalisation the state
 * update is associative and becomes a prefix scan over chunks).
 *
 * Per pair and chunk c: phi(X) = silu(X W0) * (X W2), dS_c = phi(K_c)^T diag(eta_c) V_c,
 *   S_c = W1 + sum_{j<c} dS_j (TTT_APPLY_THEN_UPDATE) or sum_{j<=c} (TTT_UPDATE_THEN_APPLY),
 *   O_c = phi(Q_c) S_c.
 * With momentum alpha (same summary page, Theorem 5.3, read as one heavy-ball step per chunk
 * with a constant coefficient): chunk j's write enters S_c with the cumulative coefficient
 * sum_{i=j}^{last} alpha^(i-j), last = c-1 (apply-then-update) or c (update-then-apply);
 * equivalently M_j = alpha M_{j-1} + dS_j, W_{j+1} = W_j + M_j. 0 <= momentum < 1, else
 * TTT_ERR_ARG; momentum 0 is the plain scan. With momentum the workspace holds one more
 * [B*H, N/chunk, rh, h] float32 region on the single-pass path.
 * Arguments: Q, K, V [B, H, N, h] I/O dtype; eta [B, H, N] float32; W0, W2 [H, h, rh] and
 * W1 [H, rh, h] float32 (or [B, H, ...] with w_batch_stride as above); O [B, H, N, h] I/O
 * dtype; S_out [B, H, rh, h] float32, nullable: the state after the last chunk.
 * Shape rules: N % chunk == 0; h a multiple of 32, 32 <= h <= 256; r*h a multiple of 64,
 * r*h <= 1024. Operands are bf16 (TTT_BF16) or fp32 (TTT_FP32), fp32 accumulation and state.
 * ---------------------------------------------------------------------------------------- */
typedef struct {
  int32_t B, H, N, h, r, chunk;
  int32_t order;
  int32_t dtype;
  int64_t w_batch_stride;
  float momentum;        /* heavy-ball coefficient alpha per chunk; 0: none */
} ttt_linattn_params;

ttt_status ttt_linattn_forward(const ttt_linattn_params* p,
                               const void* Q, const void* K, const void* V, const float* eta,
                               const float* W0, const float* W2, const float* W1,
                               void* O, float* S_out,
                               void* workspace, size_t* workspace_bytes, void* stream);

/* ------------------------------------------------------------------------------------------
 * ttt_inplace_down_forward
 *
 * Defined by: "In-Place Test-Time Training" reading notes, section 3.1 / Eq. 2 (gated MLP
 * with frozen W_gate, W_up and the fast weight W_down; chunk-wise apply then update),
 * section 3.2 / Eq. 4 (with the loss -<., .>_F: W_down += eta Vbar_[i]^T Z_[i]) and
 * section 3.4 (the update is associative). Transposes read as O = Z W_down^T.
 *
 * Per sequence and chunk i of `chunk` tokens:
 *   Z_i = silu(H_i W_gate^T) * (H_i W_up^T);  O_i = Z_i W_down^T;  W_down += eta Vbar_i^T Z_i.
 * Arguments: Hs, Vbar [B, N, d_model] bf16 (Vbar is the target, e.g. the next-token shift of
 * the embeddings, built by the caller); W_gate, W_up [d_hidden, d_model] bf16; W_down
 * [d_model, d_hidden] float32 (shared, or [B, ...] with wdown_batch_stride); O [B, N, d_model]
 * bf16; W_down_out [B, d_model, d_hidden] float32, nullable.
 * Shape rules: N % chunk == 0; d_model and d_hidden multiples of 256; chunk a multiple of 64.
 * Only TTT_BF16 is implemented (TTT_FP32 gives TTT_ERR_UNSUPPORTED).
 * ---------------------------------------------------------------------------------------- */
typedef struct {
  int32_t B, N, d_model, d_hidden, chunk;
  float eta;
  int32_t dtype;
  int64_t wdown_batch_stride;
} ttt_inplace_params;

ttt_status ttt_inplace_down_forward(const ttt_inplace_params* p,
                                    const void* Hs, const void* W_gate, const void* W_up,
                                    const float* W_down, const void* Vbar,
                                    void* O, float* W_down_out,
                                    void* workspace, size_t* workspace_bytes, void* stream);

/* ------------------------------------------------------------------------------------------
 * Kernel timing (instrumentation; off by default)
 *
 * For callers that need per-kernel durations (the benchmark's roofline figures). While
 * enabled, every kernel launched by the entry points above is bracketed by two HIP events
 * recorded on the stream it is launched on, grouped by kernel class. ttt_timing_collect waits
 * for the recorded events, writes one entry per class that ran (name: static string,
 * launches, summed milliseconds) and clears the record. The recorder is process-wide state
 * owned by the library; it is not meant for concurrent use from several host threads.
 * Returns TTT_ERR_HIP if an event cannot be created or read.
 * ---------------------------------------------------------------------------------------- */
typedef struct {
  const char* name;
  int32_t launches;
  float total_ms;
} ttt_kernel_time;

ttt_status ttt_timing_enable(int32_t on);
ttt_status ttt_timing_collect(ttt_kernel_time* out, int32_t capacity, int32_t* count);

/* Human-readable name of a status code (static string). */
const char* ttt_status_string(ttt_status s);

#ifdef __cplusplus
}
#endif
#endif /* TTT_LACT_H */
