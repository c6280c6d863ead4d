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
 *   synchronise device memory, create no streams or events, and launch only on `stream`;
 *   apart from the optional timing recorder (ttt_timing_*) the library keeps no mutable
 *   global state and is re-entrant for calls with distinct workspaces (concurrent calls on
 *   different streams give the same results as sequential calls). Inputs are read only.
 *   Outputs are fully overwritten and must not alias inputs.
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
 * this build implements h <= 192 in TTT_BF16 mode and h <= 64 in TTT_FP32 mode. Wider heads
 * (the LaCT notes' d = 768 defaults, section 2.5) run a slower composed path in TTT_BF16 mode:
 * 192 < h <= 1024 with h, r*h, chunk_q and chunk_kv multiples of 128, r*h <= 2048 and
 * r*h*h <= 2^21, without chunk_flags, inner_steps > 1 or eta_per_matrix (TTT_ERR_SHAPE or
 * TTT_ERR_UNSUPPORTED otherwise; TTT_ERR_UNSUPPORTED for other unbuilt combinations). 0 <= momentum < 1 and finite eps_norm, eps_ns >= 0, else
 * TTT_ERR_ARG (NaN included).
 * Precision: in TTT_BF16 mode the per-chunk products use fp16 MFMA operands (bf16 inputs
 * convert exactly) and Newton-Schulz uses split-bf16 operands; fp32 state throughout. In
 * TTT_FP32 mode all operands are fp32, Newton-Schulz included.
 * Range (TTT_BF16 mode): because the product operands are fp16, Q, K, V and the fast weights
 * must lie within the fp16 range, |x| <= 65504 (the step-size-scaled intermediates are rescaled
 * by a power of two per token segment and are not limited). Larger values are not representable
 * as operands and give undefined results; the library does not read the inputs on the host and
 * does not check this.
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
  /* Loop variants. A zero-initialised tail gives the plain loop above. */
  const uint8_t* chunk_flags; /* device [B, Nk/chunk_kv] or NULL: TTT_CHUNK_* bits per sequence and chunk */
  int32_t inner_steps;   /* writes per chunk; 0 or 1: one */
  int32_t eta_per_matrix;/* 0: eta [B, H, Nk]; 1: eta [B, H, 3, Nk], one row per matrix W0, W1, W2 */
} ttt_lact_params;

/* Per-chunk flags (chunk_flags), shared by the heads of a sequence:
 *   TTT_CHUNK_NO_UPDATE  the chunk is applied with the current weights and writes nothing:
 *                        weights and momentum are left as they are (apply-only chunks, e.g.
 *                        the noisy chunks of autoregressive video: "Test-Time Training Done
 *                        Right" notes, section 2.3 update-order table and section 2.4);
 *   TTT_CHUNK_RESET      before the chunk is applied or written, the weights return to the
 *                        call's initial weights (W0, W1, W2 of this sequence) and the momentum
 *                        to zero, as if a new call started there (a document boundary inside a
 *                        packed sequence: "In-Place Test-Time Training" notes, section 3.4).
 * Both may be set (reset, then apply only). The flags live on the device and are read by the
 * kernels only (not validated on the host); other bits are ignored. The array must stay valid
 * until the call's work on the stream has finished.
 * inner_steps (KV-binding summary page, "Motivation": more inner-loop iterations per chunk)
 * repeats the chunk's write that many times on the same tokens (gradient
 * at the current weights, momentum, Newton-Schulz, subtract, renorm); apply-then-update applies
 * before the first write, update-then-apply after the last. 1 <= inner_steps <= 64 (0 means 1),
 * else TTT_ERR_ARG. eta_per_matrix (notes, section 2.1: eta may be predicted separately for the
 * three matrices): matrix X takes the gradient of the chunk loss weighted by its own row eta_X. */
enum { TTT_CHUNK_NO_UPDATE = 1, TTT_CHUNK_RESET = 2 };

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
 * r*h <= 1024. fp32 accumulation and state. Operands: in TTT_FP32 mode fp32; in TTT_BF16 mode
 * bf16, except on the single-pass path (h = 32 with r*h in {64, 128}, h = 64 with r*h = 128),
 * whose operands are fp16: there Q, K, eta*V, the fast weights and the states must lie within
 * the fp16 range, |x| <= 65504 (not checked; larger values give undefined results).
 * The single-pass path runs on devices with 8 XCDs (hipDeviceAttributeNumberOfXccs); other
 * devices take the multi-launch path (same results, more launches). Test hook: when the
 * environment variable TTT_LOOKBACK_STRESS holds a nonzero integer at call time, every group of
 * the single-pass path waits a pseudo-random time (seeded by it, up to about 0.1 ms) before each
 * publication, so the chunk-prefix lookback meets other arrival orders; results are unchanged
 * bit for bit.
 * feature_map = TTT_PHI_IDENTITY (the same summary page's simplification ladder, "Method step
 * details", step 3: the fast weight is one linear layer f(x) = x W): phi(X) = X, so
 * dS_c = K_c^T diag(eta_c) V_c, S_c as above and O_c = Q_c S_c, with the h x h state W1 = S_0
 * [H, h, h] (or [B, H, h, h]); r must be 1 (else TTT_ERR_ARG); W0 and W2 are not read and may be
 * NULL; S_out is [B, H, h, h]. It runs on the single-pass path only: TTT_BF16 with h in {64, 128}
 * on an 8-XCD device (fp16 operands as above); anything else returns TTT_ERR_UNSUPPORTED.
 * chunk_flags (the per-chunk flags of ttt_lact_forward, read for the scan form): an apply-only
 * chunk writes nothing and takes no momentum step; a reset chunk starts from W1 with zero
 * momentum, as a fresh call would. Calls with flags take the multi-launch path (the SwiGLU map;
 * with the identity map they return TTT_ERR_UNSUPPORTED); ttt_linattn_backward does not take
 * flags (TTT_ERR_UNSUPPORTED).
 * ---------------------------------------------------------------------------------------- */
typedef enum {
  TTT_PHI_SWIGLU = 0,    /* phi(x) = silu(x W0) * (x W2), state [rh, h] */
  TTT_PHI_IDENTITY = 1   /* phi(x) = x: one linear fast-weight layer, state [h, h] (r = 1) */
} ttt_feature_map;

typedef struct {
  int32_t B, H, N, h, r, chunk;
  int32_t order;
  int32_t dtype;
  int64_t w_batch_stride;
  float momentum;        /* heavy-ball coefficient alpha per chunk; 0: none */
  int32_t feature_map;   /* ttt_feature_map; 0 (zero-initialised struct): TTT_PHI_SWIGLU */
  const uint8_t* chunk_flags; /* device [B, N/chunk] or NULL: TTT_CHUNK_* bits, as for ttt_lact_forward */
} ttt_linattn_params;

ttt_status ttt_linattn_forward(const ttt_linattn_params* p,
                               const void* Q, const void* K, const void* V, const float* eta,
                               const float* W0, const float* W2, const float* W1,
                               void* O, float* S_out,
                               void* workspace, size_t* workspace_bytes, void* stream);

/* ------------------------------------------------------------------------------------------
 * ttt_linattn_backward
 *
 * Defined by: the same pages as ttt_linattn_forward (the parallel form is what the model trains
 * through: KV-binding summary page, "Experimental results", end-to-end training with the
 * parallel form; press article, section 4). Gradients of sum(O * dO) with respect to every
 * input of ttt_linattn_forward, for the same parameters:
 *   G_c = phi(Q_c)^T dO_c,  R_j = sum_c w(c, j) G_c (w: the forward's coefficient of chunk j's
 *   write in the state chunk c reads), dW1 = sum_c G_c;
 *   query side: dphi(Q_c) = dO_c S_c^T;  key side: dphi(K_j) = diag(eta_j) V_j R_j^T,
 *   d(eta V)_j = phi(K_j) R_j, dV = eta d(eta V), deta_t = <d(eta V)_t, V_t>;
 *   through phi: dA = dphi * Bm * silu'(A), dBm = dphi * silu(A) (A = X W0, Bm = X W2),
 *   dX = dA W0^T + dBm W2^T, dW0 = sum X^T dA, dW2 = sum X^T dBm over queries and keys.
 * Arguments: Q, K, V, eta, W0, W2, W1 as for ttt_linattn_forward; dO [B, H, N, h] bf16 (the
 * gradient of the output); dQ, dK, dV [B, H, N, h] bf16; deta [B, H, N] float32; dW0, dW2
 * [H, h, rh] and dW1 [H, rh, h] float32, summed over the batch when the weights are shared
 * (w_batch_stride 0), else [B, H, ...] per sequence (dW0/dW2/dW1 nullable: not written).
 * Built for TTT_BF16 with the SwiGLU map and (h, r*h) in {(32, 64), (32, 128), (64, 128)}, any
 * order and momentum; other combinations return TTT_ERR_UNSUPPORTED. fp32 accumulation, fp16
 * MFMA operands (the fp16 range note of ttt_linattn_forward applies, to dO too). Weight
 * gradients are reduced in a fixed order: repeated calls give identical bits. Workspace and
 * errors as for ttt_linattn_forward.
 * ---------------------------------------------------------------------------------------- */
ttt_status ttt_linattn_backward(const ttt_linattn_params* p,
                                const void* Q, const void* K, const void* V, const float* eta,
                                const float* W0, const float* W2, const float* W1, const void* dO,
                                void* dQ, void* dK, void* dV, float* deta,
                                float* dW0, float* dW2, float* dW1,
                                void* workspace, size_t* workspace_bytes, void* stream);

/* ------------------------------------------------------------------------------------------
 * ttt_linattn_forward_noalloc
 *
 * For callers that cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc. Same operation, arguments, layouts and results as
 * ttt_linattn_forward, without a workspace: the scratch (chunk aggregates, prefixes, flags and
 * ticket counters) lives in a device array inside the library, TTT_NOALLOC_SCRATCH_BYTES per GPU,
 * created with the library's code object on each GPU it runs on and held until the process ends.
 * The entry point calls no allocating routine. A call that needs more scratch than that (the
 * size ttt_linattn_forward's workspace query reports) returns TTT_ERR_WORKSPACE before any
 * launch, with the sizes in ttt_last_error(). Every call on a GPU uses that GPU's one array and
 * leaves its contents behind (what must start at zero is cleared by a kernel at the start of
 * each call): calls that overlap in time on one GPU race and give undefined results, so issue
 * them on one stream or otherwise one after another. The first call on a device looks up the
 * array's address (one hipGetSymbolAddress per device, then cached).
 * ---------------------------------------------------------------------------------------- */
#define TTT_NOALLOC_SCRATCH_BYTES (64u << 20)

ttt_status ttt_linattn_forward_noalloc(const ttt_linattn_params* p,
                                       const void* Q, const void* K, const void* V, const float* eta,
                                       const float* W0, const float* W2, const float* W1,
                                       void* O, float* S_out, void* stream);

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
 * Shape rules: N % chunk == 0; d_model and d_hidden multiples of 256; chunk a multiple of 128.
 * Only TTT_BF16 is implemented (TTT_FP32 gives TTT_ERR_UNSUPPORTED). Every launch goes to
 * `stream`; the next chunk's Z is formed in the same launch as the current chunk's apply.
 * LM-aligned target (section 3.2 / Eq. 3: Vbar = Conv1D(X0) W_target): when X0 is set the
 * library builds Vbar itself and the Vbar argument must be NULL (else TTT_ERR_ARG). Per sequence,
 *   Vbar_t = (sum_{tau < conv_k} conv_taps[tau] * X0_{t+tau}) W_target^T
 * a depthwise convolution over the sequence (tap tau weights the token tau positions ahead,
 * tau = 0 the token itself; rows past the end read zero) followed by the projection. X0
 * [B, N, d_model] bf16; conv_taps [conv_k, d_model] float32, 1 <= conv_k <= 16 (else
 * TTT_ERR_ARG); W_target [d_model(out), d_model(in)] bf16 in nn.Linear layout, or NULL for the
 * identity. conv_k = 2 with taps (0, 1) and no W_target is the next-token target. The
 * convolution accumulates in float32 and rounds Vbar to bf16, as a given Vbar would be.
 * ---------------------------------------------------------------------------------------- */
typedef struct {
  int32_t B, N, d_model, d_hidden, chunk;
  float eta;
  int32_t dtype;
  int64_t wdown_batch_stride;
  /* LM-aligned target; a zero-initialised tail means Vbar is given */
  const void* X0;          /* [B, N, d_model] bf16 or NULL */
  const float* conv_taps;  /* [conv_k, d_model] float32 */
  const void* W_target;    /* [d_model, d_model] bf16 (nn.Linear layout) or NULL: identity */
  int32_t conv_k;
} ttt_inplace_params;

ttt_status ttt_inplace_down_forward(const ttt_inplace_params* p,
                                    const void* Hs, const void* W_gate, const void* W_up,
                                    const float* W_down, const void* Vbar,
                                    void* O, float* W_down_out,
                                    void* workspace, size_t* workspace_bytes, void* stream);

/* ------------------------------------------------------------------------------------------
 * ttt_inplace_down_backward
 *
 * Defined by: the same notes as ttt_inplace_down_forward (sections 3.1, 3.2 / Eq. 4 and 3.4: the
 * chunked update is what the model trains through). Gradients of sum(O * dO) of
 * ttt_inplace_down_forward with respect to Hs, W_gate, W_up, W_down and Vbar, for the same
 * parameters. With G_i = dO_i^T Z_i and R_i = sum_{k > i} G_k: dW_down = sum_i G_i;
 * dZ_i = dO_i W_i + eta Vbar_i R_i; dVbar_i = eta Z_i R_i^T; through the gate,
 * dA = dZ * U * silu'(A), dU = dZ * silu(A) (A = H W_gate^T, U = H W_up^T), dHs = dA W_gate +
 * dU W_up, dW_gate = sum dA^T H, dW_up = sum dU^T H.
 * Arguments: Hs, W_gate, W_up, W_down, Vbar as for ttt_inplace_down_forward; dO [B, N, d_model]
 * bf16; dHs, dVbar [B, N, d_model] bf16; dW_gate, dW_up [d_hidden, d_model] float32 (summed over
 * the batch); dW_down [d_model, d_hidden] float32 (summed over the batch) or [B, d_model,
 * d_hidden] when wdown_batch_stride != 0. Shape rules as for the forward. TTT_BF16 only; a
 * target built from X0 (the LM-aligned target) returns TTT_ERR_UNSUPPORTED here: build Vbar with
 * ttt_inplace_target_forward, pass it, and take dVbar through ttt_inplace_target_backward. The workspace holds,
 * per sequence in turn, every chunk's Z (both orientations), gate and up products, the
 * transposed dA and dU, and every chunk's state W_i^T, all bf16: about
 * 6 N d_hidden + (N / chunk) d_model d_hidden bf16 elements plus a few d_model x d_hidden
 * buffers (11.3 GB at d_model 4096, d_hidden 14336, N 32768, chunk 1024).
 * ---------------------------------------------------------------------------------------- */
ttt_status ttt_inplace_down_backward(const ttt_inplace_params* p, const void* Hs, const void* W_gate,
                                     const void* W_up, const float* W_down, const void* Vbar, const void* dO,
                                     void* dHs, float* dW_gate, float* dW_up, float* dW_down, void* dVbar,
                                     void* workspace, size_t* workspace_bytes, void* stream);

/* ------------------------------------------------------------------------------------------
 * ttt_inplace_target_forward / ttt_inplace_target_backward
 *
 * Defined by: "In-Place Test-Time Training" reading notes, section 3.2 / Eq. 3 (the LM-aligned
 * target; the same readings as ttt_inplace_down_forward with X0 given). The target on its own, so
 * that its inputs can be trained: ttt_inplace_target_forward writes Vbar [B, N, d_model] bf16
 * (token-major) from p->X0, p->conv_taps, p->conv_k and p->W_target (NULL: identity); pass it to
 * ttt_inplace_down_backward as Vbar. ttt_inplace_target_backward takes that call's dVbar
 * [B, N, d_model] bf16 and writes the gradients of sum(Vbar * dVbar): dX0 [B, N, d_model] bf16,
 * dtaps [conv_k, d_model] float32 and dW_target [d_model, d_model] float32 (both summed over the
 * batch; dW_target must be NULL exactly when p->W_target is). With C = Conv1D(X0):
 * dC = dVbar W_target, dW_target = sum dVbar^T C, dX0[s] = sum_tau taps[tau] * dC[s - tau],
 * dtaps[tau] = sum_t dC[t] * X0[t + tau]. Fields used: B, N, d_model, dtype (TTT_BF16 only, else
 * TTT_ERR_UNSUPPORTED), X0, conv_taps, conv_k (1..16), W_target; d_model a multiple of 256 and N
 * a multiple of 128 (TTT_ERR_SHAPE). Workspace: one sequence's Conv1D (forward, with a
 * projection); C^T, dVbar^T, dC and W_target^T (backward, with a projection) and the per-tile tap
 * partials, B * N / 64 * conv_k * d_model float32.
 * ---------------------------------------------------------------------------------------- */
ttt_status ttt_inplace_target_forward(const ttt_inplace_params* p, void* Vbar, void* workspace,
                                      size_t* workspace_bytes, void* stream);
ttt_status ttt_inplace_target_backward(const ttt_inplace_params* p, const void* dVbar, void* dX0,
                                       float* dtaps, float* dW_target, void* workspace,
                                       size_t* workspace_bytes, void* stream);

/* ------------------------------------------------------------------------------------------
 * Kernel timing (instrumentation; off by default)
 *
 * For callers that need per-kernel durations (the benchmark's roofline figures). While
 * enabled, every kernel launched by the entry points above is bracketed by two HIP events
 * recorded on the stream it is launched on, grouped by kernel class. ttt_timing_collect waits
 * for the recorded events, writes one entry per class that ran (name: static string,
 * launches, summed milliseconds) and clears the record. The recorder is process-wide state
 * owned by the library; it is not meant for concurrent use from several host threads.
 * ttt_timing_enable(0) also destroys the events the recorder holds (call it after the last
 * ttt_timing_collect, so that no HIP object of the library outlives the caller's use of it).
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

/* Diagnostic text of the last HIP failure an entry point of this library met on the calling
 * host thread (the failing HIP call, its error name and the source location), or "" if none.
 * The string is owned by the library and stays valid until the next failure on the thread. */
const char* ttt_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* TTT_LACT_H */
