/*
 * ssm_scan.h — C ABI of the MI355X (gfx950) selective state-space scan library
 * (libssm_scan.so).
 *
 * What it computes, per batch b, channel d (of `dim`), state n (of `dstate`),
 * time step l (of `seqlen`):
 *
 *   dt      = softplus(delta[b,l,d] + delta_bias[d])   (or no softplus)
 *   h[n]    = exp(dt * A[d,n]) * h[n] + k * B[b,l,n] * u[b,l,d]
 *   k       = dt (default), or (exp(dt * A[d,n]) - 1) / A[d,n] (exact
 *             zero-order hold; k = dt where A[d,n] = 0)
 *   y[b,l,d] = (sum_n C[b,l,n] * h[n] + D[d] * u[b,l,d]) * silu(z[b,l,d])
 *
 * Sources (page title and section; the same pages throughout this library):
 *   - "从 Transformer 到 Mamba：状态空间模型如何重塑序列计算的效率边界" (ybb.press):
 *     section 2 (discrete recurrence), section 3 (input-dependent delta, B, C;
 *     softplus), section 3.1 (the selective_scan(u, delta, A, B, C, D)
 *     statement, shapes and discretisation), section 5 (SelectiveScan loop,
 *     step-size bias before softplus, D skip, MambaBlock gate), section 6.3
 *     (decode: fixed work per token, state in, new state out).
 *   - "Mamba" study notes (lyirs.cc): "Selective State Space" (y_t = C_t h_t +
 *     D x_t), "block structure" (gate branch), and the fixed-size ssm_state
 *     kept between tokens.
 *   - "Mamba架构：突破Transformer瓶颈的序列建模新范式" (intelliparadigm.com),
 *     section 6.2: very long sequences are processed in chunks with the state
 *     carried from chunk to chunk (h0 in, h_final out).
 *   - "Mamba新突破：SSM架构挑战注意力机制，引领推理新范式" (ruibaoantu.com),
 *     section 二.3: the continuous system is discretised by a zero-order hold,
 *     whose input coefficient for a diagonal A is the closed form above.
 *
 * Readings where the pages disagree: the transition is exp(dt * A) with A <= 0
 * passed in directly (not A_log, and no extra minus sign); the input term is
 * dt * B * u; the gate multiplies after the D skip.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers on the current HIP device,
 *     dense row-major with the shapes given. The caller owns every buffer; the
 *     library never allocates, frees or synchronises, and keeps no mutable
 *     global state.
 *   - `stream` is a hipStream_t (NULL = the null stream). Calls enqueue work
 *     and return at once; a status of 0 means the launch was accepted.
 *   - dtype codes: 0 = float32, 1 = bfloat16. u, delta, B, C and z share
 *     `in_dtype`; y has `out_dtype`; A, D, delta_bias, h0, h_final and the
 *     decode state are always float32. bfloat16 outputs round to nearest even.
 *   - Optional pointers may be NULL: D (= 0), z (no gate), delta_bias (= 0),
 *     h0 (= zero state), h_final (not written).
 *   - Errors: arguments are validated on the host before anything is launched.
 *     A failed check returns its status and touches no memory. A launch error
 *     returns SSM_E_HIP. Nothing throws across the ABI.
 *   - Alignment: u, delta, z, y, B, C must be 16-byte aligned (SSM_E_ALIGN);
 *     float32 arrays 4-byte aligned.
 */
#ifndef SSM_SCAN_H
#define SSM_SCAN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* 2: the workspace must be 16-byte aligned; the forward with checkpoints and
 * the backward from them were added. */
#define SSM_ABI_VERSION 2

/* Status codes. */
#define SSM_OK 0
#define SSM_E_NULLPTR 1     /* a required pointer is NULL                        */
#define SSM_E_SHAPE 2       /* negative or inconsistent size                     */
#define SSM_E_DTYPE 3       /* dtype code other than 0 or 1                      */
#define SSM_E_ALIGN 4       /* pointer not aligned as documented                 */
#define SSM_E_WORKSPACE 5   /* workspace missing or smaller than required        */
#define SSM_E_ALIAS 6       /* an output overlaps an input it may not overlap    */
#define SSM_E_UNSUPPORTED 7 /* a size or an option outside the supported range */
#define SSM_E_HIP 8         /* the HIP runtime reported an error at launch       */

/* Bits of the `flags` argument of the scan and decode entry points. Any other
 * bit set returns SSM_E_UNSUPPORTED. */
#define SSM_FLAG_SOFTPLUS 1 /* dt = softplus(delta + delta_bias), else delta + delta_bias */
#define SSM_FLAG_ZOH 2      /* input coefficient k = (exp(dt A) - 1) / A, else k = dt   */

/* Version of this ABI (SSM_ABI_VERSION of the header the library was built from). */
int ssm_abi_version(void);

/* Static, NUL-terminated description of a status code. Never NULL. */
const char* ssm_status_string(int status);

/*
 * Bytes of device workspace ssm_selective_scan_fwd needs for this shape. It
 * holds B and C repacked time-major per state (read by the kernels as
 * wave-uniform rows) and, when the sequence is split into chunks that run in
 * parallel (see ssm_scan_chunks), each chunk's summary: the sum of its step
 * sizes, [B, d] float32 (its transition product is exp(A * that sum)), and
 * its final state from a zero start, [B, d, N] float32. The summaries are
 * joined in order with the recurrence's own combine rule, the associative
 * operator (A_i, b_i) (+) (A_j, b_j) = (A_j A_i, A_j b_i + b_j) of
 * "Mamba的隐藏代价" (kongchang.com), section on sequential gradients, and the
 * chunked processing with a carried state of intelliparadigm.com section 6.2.
 * With N > 32 (padded to 64 or 128 states) and 65 to 128 blocks of 64
 * channels (B * ceil(d / 64)) in a single pass, each channel's states are
 * split over two blocks of half the padded states, so that the device fills;
 * the workspace then also holds
 * the two float32 partial readouts sum_n C h over each half of the states
 * (the first with the skip D u), [2][B, L, d] (rounded up), which a combine
 * pass adds before the gate. It depends only on the four sizes. Returns 0 for
 * invalid or unsupported sizes, and for batch, dim or seqlen 0.
 */
size_t ssm_scan_workspace_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate);

/*
 * Number of sequence chunks the scan of this shape runs in (1: one pass over
 * the whole sequence; 0: invalid or unsupported sizes). Chunking is chosen
 * when the batch has too few 64-channel blocks to occupy the device
 * (L >= 2048 and B * ceil(d / 64) <= 128 for N <= 32, <= 64 for N >= 33), or
 * when one batch row's [L, d] plane exceeds 2^30 bytes at 4 bytes per element.
 * Results of a chunked and a single-pass scan agree to rounding; each is
 * deterministic.
 */
int64_t ssm_scan_chunks(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate);

/*
 * Selective scan forward (the selective_scan(u, delta, A, B, C, D) statement
 * of ybb.press section 3.1 with the loop of section 5; gate from section 5's
 * MambaBlock; h0/h_final per intelliparadigm.com section 6.2).
 *
 *   batch, seqlen, dim, dstate : B >= 0, 0 <= L < 2^30, 0 <= d < 2^24,
 *                                1 <= N <= 128 (else SSM_E_UNSUPPORTED).
 *   in_dtype, out_dtype        : 0 float32, 1 bfloat16.
 *   flags                      : SSM_FLAG_SOFTPLUS and/or SSM_FLAG_ZOH.
 *   u, delta  [B, L, d]  in_dtype   input and raw step size
 *   A         [d, N]     float32    diagonal state matrix (expected <= 0)
 *   B, C      [B, L, N]  in_dtype   input and output projections
 *   D         [d]        float32    skip (optional)
 *   z         [B, L, d]  in_dtype   gate branch (optional)
 *   delta_bias[d]        float32    step-size bias (optional)
 *   h0        [B, d, N]  float32    initial state (optional)
 *   y         [B, L, d]  out_dtype  output; must not overlap any input
 *   h_final   [B, d, N]  float32    final state (optional); may equal h0
 *   workspace, workspace_bytes      device scratch of at least
 *                                   ssm_scan_workspace_bytes() bytes, 16-byte
 *                                   aligned (may be NULL when that is 0)
 *   stream                          hipStream_t
 *
 * L = 0 writes h_final = h0 (or zeros) and nothing else. Results are
 * bitwise deterministic from run to run (fixed combine order, no atomics on
 * floating-point data). NaN/Inf propagate without clamping.
 */
int ssm_selective_scan_fwd(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                           int in_dtype, int out_dtype, int flags,
                           const void* u, const void* delta, const float* A,
                           const void* B, const void* C, const float* D, const void* z,
                           const float* delta_bias, const float* h0,
                           void* y, float* h_final,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * For callers that cannot allocate device memory at the time of the call
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): ssm_selective_scan_fwd with the same arguments except the
 * workspace, which here is a device array of SSM_NOALLOC_SCRATCH_BYTES that
 * the library owns, one per GPU, reserved from the first use of this entry
 * point's code on that GPU until the process ends. The call allocates nothing.
 *   - Shapes whose ssm_scan_workspace_bytes() exceeds SSM_NOALLOC_SCRATCH_BYTES
 *     return SSM_E_WORKSPACE (checked before any launch).
 *   - Every call on one GPU uses that GPU's single array: calls that may
 *     overlap in time on one GPU (other streams, other threads) race and
 *     must be serialised by the caller. Nothing in the array needs to start
 *     at zero; a call keeps no state in it for the next one.
 *   - A shape whose states ssm_selective_scan_fwd splits over two blocks
 *     (see ssm_scan_workspace_bytes), with partial readouts too large for the
 *     array, runs here with one block per channel instead: its results then
 *     agree with ssm_selective_scan_fwd to rounding, not bitwise.
 *   - Otherwise as ssm_selective_scan_fwd (same validation, results bitwise
 *     equal to it for the same inputs).
 */
#define SSM_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int ssm_selective_scan_fwd_noalloc(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                                   int in_dtype, int out_dtype, int flags,
                                   const void* u, const void* delta, const float* A,
                                   const void* B, const void* C, const float* D, const void* z,
                                   const float* delta_bias, const float* h0,
                                   void* y, float* h_final, void* stream);

/*
 * Decode: one token's state update in place (ybb.press section 6.3; the
 * fixed-size ssm_state of the lyirs.cc notes). The step is the scan's step
 * for L = 1 with h0 = state and h_final = state:
 *
 *   batch, dim, dstate         : B >= 0, d >= 0, 1 <= N <= 256.
 *   flags                      : SSM_FLAG_SOFTPLUS and/or SSM_FLAG_ZOH.
 *   state     [B, d, N]  float32    read, then overwritten with the new state
 *   x, delta  [B, d]     in_dtype   token input and raw step size
 *   A         [d, N]     float32
 *   B, C      [B, N]     in_dtype
 *   D         [d]        float32    (optional)
 *   z         [B, d]     in_dtype   gate branch (optional)
 *   delta_bias[d]        float32    (optional)
 *   y         [B, d]     out_dtype  output; must not overlap state or inputs
 *   stream                          hipStream_t
 */
int ssm_selective_state_update(int64_t batch, int64_t dim, int64_t dstate,
                               int in_dtype, int out_dtype, int flags,
                               float* state, const void* x, const void* delta,
                               const float* A, const void* B, const void* C,
                               const float* D, const void* z, const float* delta_bias,
                               void* y, void* stream);

/*
 * Bytes of device workspace ssm_selective_scan_bwd needs for this shape: B and
 * C repacked per state, the states at every tile start ([B][Lp/T][N'][d]
 * float32, N' = N rounded up to a power of two, Lp = L rounded up to 16, and
 * tiles of T = 16 steps for N' <= 8, 128 / N' steps from N' = 16 on), and
 * per-block / per-batch partial sums of dB, dC, dA, dD and the bias gradient.
 * Returns 0 for invalid or unsupported sizes (N > 64, and rows too long for
 * 32-bit offsets into the packed B/C or the dB/dC partials).
 */
size_t ssm_scan_bwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate);

/*
 * Selective scan backward: gradients of a loss through ssm_selective_scan_fwd
 * with the same inputs, given dy = dL/dy and optionally dh_final = dL/dh_final.
 * Reverse-mode steps of the forward recurrence (its gradient flows back
 * through every later state: "Mamba的隐藏代价" (kongchang.com), section on the
 * optimisation problems of sequential gradients):
 *
 *   lam_l   = dp_l C_l + exp(dt_{l+1} A) lam_{l+1},  dp = dy * silu(z) (or dy)
 *   du      = dp D + sum_n lam dt B          ddelta = softplus'(x) sum_n lam (A exp(dt A) h_{l-1} + B u)
 *   dA      = sum_{b,l} lam dt exp(dt A) h_{l-1}      dB_l = sum_d lam dt u,  dC_l = sum_d dp h_l
 *   dD      = sum_{b,l} dp u                 dz = dy p silu'(z), p = sum_n C h + D u
 *   ddelta_bias = sum_{b,l} ddelta           dh0 = exp(dt_0 A) lam_0
 *
 *   batch, seqlen, dim, dstate : as the forward, with 1 <= N <= 64 (else
 *                                SSM_E_UNSUPPORTED).
 *   in_dtype, flags, u, delta, A, B, C, D, z, delta_bias, h0 : the
 *                                forward's inputs (same layouts and rules);
 *                                with SSM_FLAG_ZOH the gradients of the exact
 *                                zero-order-hold forward: k = (a - 1) / A in
 *                                place of dt in front of B u, dk/ddt = a and
 *                                dk/dA = dt^2 phi'(dt A), phi(x) = expm1(x)/x
 *                                (ruibaoantu.com, section 二.3).
 *   dy        [B, L, d]  float32    gradient of the loss w.r.t. y
 *   dh_final  [B, d, N]  float32    gradient w.r.t. h_final (optional, 0)
 *   du, ddelta [B, L, d] float32    outputs (ddelta w.r.t. the raw delta)
 *   dA        [d, N]     float32    output
 *   dB, dC    [B, L, N]  float32    outputs
 *   dD [d], dz [B, L, d], ddelta_bias [d] : float32 outputs, optional; written
 *                                only when D, z, delta_bias are given
 *   dh0       [B, d, N]  float32    output (optional)
 *   workspace, workspace_bytes      at least ssm_scan_bwd_workspace_bytes()
 * No output may overlap an input, another output or the workspace. Results
 * are bitwise deterministic from run to run (sums over channels and batches
 * in a fixed order; no floating-point atomics).
 */
int ssm_selective_scan_bwd(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                           int in_dtype, int flags,
                           const void* u, const void* delta, const float* A,
                           const void* B, const void* C, const float* D, const void* z,
                           const float* delta_bias, const float* h0,
                           const float* dy, const float* dh_final,
                           float* du, float* ddelta, float* dA, float* dB, float* dC,
                           float* dD, float* dz, float* ddelta_bias, float* dh0,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * A training step that keeps the forward's states instead of recomputing
 * them ("Mamba的隐藏代价" (kongchang.com), section on the optimisation
 * problems of sequential gradients, names storing or recomputing each step's
 * local terms as the two options). For 1 <= N <= 16 only.
 *
 * ssm_scan_checkpoint_bytes: bytes of the checkpoints, the states at every
 * tile start of the backward, [B][Lp/T][N'][d] float32 (N' = N rounded up to
 * a power of two, Lp = L rounded up to 16, T = 16 steps for N' <= 8 and 8
 * for N' = 16). Returns 0 for sizes the backward does not run or N > 16.
 *
 * ssm_selective_scan_fwd_ckpt: ssm_selective_scan_fwd (same arguments, rules
 * and results, bitwise) that also writes the checkpoints (caller-owned,
 * ssm_scan_checkpoint_bytes() bytes, 4-byte aligned, overlapping no input,
 * output or the workspace; may be NULL only for L = 0). A single-pass scan
 * writes them from its own recurrence; where the sequence runs in chunks
 * (ssm_scan_chunks() > 1) they are computed by a recurrence pass before the
 * scan. N > 16, or sizes ssm_selective_scan_bwd does not run, give
 * SSM_E_UNSUPPORTED.
 *
 * ssm_selective_scan_bwd_ckpt: ssm_selective_scan_bwd (same arguments, rules
 * and results, bitwise, and the same workspace) with the states taken from
 * the checkpoints that ssm_selective_scan_fwd_ckpt wrote for the same inputs
 * and h0, instead of a recurrence pass of its own. The checkpoints are an
 * input: no output may overlap them.
 */
size_t ssm_scan_checkpoint_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate);
int ssm_selective_scan_fwd_ckpt(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                                int in_dtype, int out_dtype, int flags,
                                const void* u, const void* delta, const float* A,
                                const void* B, const void* C, const float* D, const void* z,
                                const float* delta_bias, const float* h0,
                                void* y, float* h_final, float* checkpoints,
                                void* workspace, size_t workspace_bytes, void* stream);
int ssm_selective_scan_bwd_ckpt(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                                int in_dtype, int flags,
                                const void* u, const void* delta, const float* A,
                                const void* B, const void* C, const float* D, const void* z,
                                const float* delta_bias, const float* h0,
                                const float* dy, const float* dh_final,
                                float* du, float* ddelta, float* dA, float* dB, float* dC,
                                float* dD, float* dz, float* ddelta_bias, float* dh0,
                                const float* checkpoints,
                                void* workspace, size_t workspace_bytes, void* stream);

/*
 * Causal depthwise conv1d (+ SiLU) over a sequence: the short local
 * convolution that precedes the selective scan in the block ("从 Transformer
 * 到 Mamba", ybb.press, section 5: depthwise Conv1d of width d_conv padded by
 * width-1 and cut to the first L outputs, then SiLU; lyirs.cc notes, "Mamba
 * block 的结构" and the fixed-size conv_state kept between tokens).
 *
 *   out[b,l,d] = bias[d] + sum_{k<K} weight[d,k] * x[b, l-(K-1)+k, d]
 *   y[b,l,d]   = silu(out) if silu_activation, else out
 *
 * Inputs before step 0 are state_in[b,d,j] = x[b, j-(K-1), d] (oldest first),
 * or zero when state_in is NULL. state_out receives the last K-1 inputs the
 * same way (some from state_in when L < K-1), ready for the next call or for
 * ssm_causal_conv1d_update.
 *
 *   batch, seqlen, dim, width  : B >= 0, 0 <= L <= 4194240, d >= 0,
 *                                1 <= K <= 8; B <= 65535 (else
 *                                SSM_E_UNSUPPORTED).
 *   in_dtype, out_dtype        : 0 float32, 1 bfloat16 (x / y).
 *   x         [B, L, d]  in_dtype   input (may be NULL when L = 0)
 *   weight    [d, K]     float32    filter; weight[d, K-1] meets the newest input
 *   bias      [d]        float32    (optional, 0)
 *   state_in  [B, d, K-1] float32   (optional, zeros)
 *   y         [B, L, d]  out_dtype  output; must not overlap any input
 *   state_out [B, d, K-1] float32   (optional); must not overlap y or any
 *                                   input, state_in included
 *   stream                          hipStream_t
 * x and y must be 16-byte aligned; float32 arrays 4-byte aligned.
 */
int ssm_causal_conv1d_fwd(int64_t batch, int64_t seqlen, int64_t dim, int64_t width,
                          int in_dtype, int out_dtype, int silu_activation,
                          const void* x, const float* weight, const float* bias,
                          const float* state_in, void* y, float* state_out, void* stream);

/*
 * Decode: one token through the convolution, updating the carried state in
 * place (the conv_state of the lyirs.cc notes; the per-token step of ybb.press
 * section 6.3). Equal to ssm_causal_conv1d_fwd with L = 1, state_in = state
 * and state_out = state.
 *
 *   batch, dim, width          : B >= 0, d >= 0, 1 <= K <= 8.
 *   state     [B, d, K-1] float32   read, then overwritten (may be NULL when K = 1)
 *   x         [B, d]     in_dtype
 *   weight    [d, K], bias [d] (optional)   float32
 *   y         [B, d]     out_dtype  must not overlap state or inputs
 */
int ssm_causal_conv1d_update(int64_t batch, int64_t dim, int64_t width,
                             int in_dtype, int out_dtype, int silu_activation,
                             float* state, const void* x, const float* weight, const float* bias,
                             void* y, void* stream);

/*
 * Mamba-2 SSD layer, forward ("Mamba的隐藏代价", kongchang.com, section on the
 * value and limits of the argument: the selective SSM recast as a structured
 * state-space duality, y = M o (Q K^T) V with M lower triangular and
 * semiseparable, Q from C and K from B, computed with matrix products;
 * "从 Transformer 到 Mamba", ybb.press, section 9.1: diagonal state matrix).
 * One scalar decay per head, B and C shared by all heads. Per batch b, step t,
 * head h, head channel p, state n:
 *
 *   dt      = softplus(dt_raw[b,t,h] + dt_bias[h])     (or without softplus)
 *   H[n,p]  = exp(dt * A[h]) * H[n,p] + dt * B[b,t,n] * x[b,t,h,p]
 *   y[b,t,h,p] = (sum_n C[b,t,n] * H[n,p] + D[h] * x[b,t,h,p]) * silu(z[b,t,h,p])
 *
 * which is the selective scan above with d = H * P channels, A[h*P+p, n] =
 * A[h] for every n and delta[b,t,h*P+p] = dt_raw[b,t,h]. It is computed in
 * chunks of 64 steps as dense products on the matrix cores (see the source).
 *
 *   batch, seqlen, nheads, headdim, dstate : B >= 0, L >= 0, H >= 0,
 *                                1 <= P <= 64, 1 <= N <= 128 (else
 *                                SSM_E_UNSUPPORTED); B * H < 2^31,
 *                                H * P < 2^23.
 *   in_dtype, out_dtype        : 0 float32, 1 bfloat16.
 *   flags                      : SSM_FLAG_SOFTPLUS or 0 (SSM_FLAG_ZOH and any
 *                                other bit: SSM_E_UNSUPPORTED).
 *   x         [B, L, H, P]  in_dtype   input
 *   dt        [B, L, H]     in_dtype   raw step size per head
 *   A         [H]           float32    decay per head (expected <= 0)
 *   B, C      [B, L, N]     in_dtype   input and output projections
 *   D         [H]           float32    skip per head (optional)
 *   z         [B, L, H, P]  in_dtype   gate branch (optional)
 *   dt_bias   [H]           float32    step-size bias (optional)
 *   h0        [B, H, P, N]  float32    initial state (optional)
 *   y         [B, L, H, P]  out_dtype  output; must not overlap any input
 *   h_final   [B, H, P, N]  float32    final state (optional); may equal h0
 *   stream                             hipStream_t
 *
 * Alignment and NULL rules as for the scan (x, dt, B, C, z, y 16-byte
 * aligned). No workspace. L = 0 writes h_final = h0 (or zeros). Bitwise
 * deterministic.
 */
int ssm_ssd_fwd(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim, int64_t dstate,
                int in_dtype, int out_dtype, int flags,
                const void* x, const void* dt, const float* A, const void* B, const void* C,
                const float* D, const void* z, const float* dt_bias, const float* h0,
                void* y, float* h_final, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SSM_SCAN_H */
