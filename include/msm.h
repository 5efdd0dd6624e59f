/*
 * msm.h -- C ABI of the Momentum-Mamba selective scan for AMD Instinct MI355X (gfx950).
 *
 * The operation (Momentum Mamba README, "Momentum Mamba Recurrence"; its plain-Mamba special
 * case beta = 0, alpha = 1 is "Standard Mamba Recurrence" on the same page).  For every batch
 * row b, channel d and state n, starting from v = h = 0:
 *
 *     a_t = exp(delta[b,t,d] * A[d,n])                               (exact Abar, first-order Bbar:
 *     v_t = beta * v_{t-1} + alpha * delta[b,t,d] * B[b,t,n] * x[b,t,d]   "Discretization Note")
 *     h_t = a_t * h_{t-1} + v_t
 *     y[b,t,d] = sum_n C[b,t,n] * h_t  (+ Dskip[d] * x[b,t,d] when Dskip is given)
 *
 * B and C carry N values per position shared by all channels, delta one value per channel and
 * A one value per (channel, state) -- the selection layout of "Mamba: Choosing What to Remember
 * Based on the Input", section "From input features to update coefficients".  The skip term is
 * the per-channel D weight of the Mamba block ("Where the state computation sits in a Mamba
 * block" on the same page); alpha does not scale it.
 *
 * The backward returns the gradients of sum(dy * y) with respect to every input (README,
 * "Gradient Flow" / "Gradient Formulas"; the velocity adjoint also receives the hidden-state
 * adjoint because v_t enters h_t directly).  dB, dC sum over channels, dA over batch and time.
 *
 * Conventions for every entry point
 *   - All array pointers are DEVICE pointers to contiguous row-major buffers owned by the
 *     caller.  The library allocates no memory and keeps no mutable global state.
 *   - Shapes: x, delta, y, dy, dx, ddelta: (Bt, L, D).  A, dA: (D, N) fp32.
 *             B, C, dB, dC: (Bt, L, N).  Dskip, dDskip: (D,) fp32.  last_h, last_v: (Bt, D, N) fp32.
 *   - io selects the element type of x, delta, B, C, y, dy, dx, ddelta, dB, dC:
 *     MSM_F32 (IEEE binary32) or MSM_BF16 (bfloat16, outputs rounded to nearest even).
 *     A, Dskip, dA, dDskip, last_h, last_v are always fp32.  All arithmetic and every state
 *     is fp32 inside the kernels.  A is in natural-log units (the kernels rescale it to base 2).
 *   - stream is a hipStream_t (NULL = the null stream).  Work is enqueued asynchronously; the
 *     function returns once it is enqueued.
 *   - workspace is caller-owned device scratch of at least the size returned by the matching
 *     *_workspace_bytes query for the same shape and io (may be NULL when that size is 0).
 *     Its contents on entry do not matter and are undefined on exit.  Two calls in flight at
 *     the same time must not share a workspace.
 *   - Argument errors are detected before anything is enqueued and reported as a status; no
 *     exception crosses the ABI and nothing is printed.  A launch failure reported by the HIP
 *     runtime is returned as MSM_ERR_LAUNCH.  Non-finite inputs are not checked: NaN/Inf
 *     propagate to the outputs.
 */
#ifndef MSM_H_
#define MSM_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MSM_OK = 0,
  MSM_ERR_INVALID_ARG = 1, /* null required pointer, bad size, beta outside [0,1), alpha not
                              finite or negative, an output overlapping an input */
  MSM_ERR_UNSUPPORTED = 2, /* valid by the method but outside this build (N > 64, io value) */
  MSM_ERR_WORKSPACE = 3,   /* workspace smaller than the query result */
  MSM_ERR_LAUNCH = 4       /* the HIP runtime rejected a kernel launch */
} msm_status;

typedef enum { MSM_F32 = 0, MSM_BF16 = 1 } msm_dtype;

/* Optional launch plan.  0 in a field means "choose automatically".
 *   states_per_wave : 1, 2, 4, 8 or 16 -- how many of the N states one lane keeps in registers.
 *                     N pads to 4, 16, 32 or 64 states.  Forward: a 64-lane wavefront serves
 *                     64 channels and a workgroup holds padded-N / states_per_wave wavefronts
 *                     (allowed: 1, 2, 4 at 4 states; 1-16 at 16; 4, 8 at 32; 4, 8, 16 at 64).
 *                     Backward: each 32-lane half of a wavefront holds states_per_wave states of
 *                     32 channels (allowed: 1, 2 at 4 states; 1, 2, 4 at 16; 2 at 32); at 64
 *                     states 2 runs two launches of 32 states and 4 the 64-channel kernel.
 *                     Other values return MSM_ERR_UNSUPPORTED.
 *   chunks          : number of time chunks the sequence is cut into (1..64, forward only);
 *                     chunks > 1 adds a pass that summarises each chunk as an affine map of its
 *                     start state.
 * A plan never changes results beyond fp32 rounding order. */
typedef struct {
  int32_t states_per_wave;
  int32_t chunks;
} msm_plan;

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int32_t msm_version(void);

/* Human-readable name of a status code (static string, never NULL). */
const char* msm_status_string(msm_status s);

/* Workspace sizes in bytes.  Valid for every plan the library may choose (automatic or
 * explicit).  Return 0 for invalid sizes. */
size_t msm_scan_fwd_workspace_bytes(int64_t Bt, int64_t L, int64_t D, int64_t N, msm_dtype io);
size_t msm_scan_bwd_workspace_bytes(int64_t Bt, int64_t L, int64_t D, int64_t N, msm_dtype io);

/* The plan msm_scan_fwd / msm_scan_bwd would use for this shape (written to *plan).  The fused
 * backward (msm_selective_scan_bwd with any extra) takes two states per wavefront half at 5-16
 * states instead.  At 64 states with D >= 2^23 the backward takes the 64-channel kernel (4). */
msm_status msm_scan_fwd_plan(int64_t Bt, int64_t L, int64_t D, int64_t N, msm_dtype io,
                             float beta, msm_plan* plan);
msm_status msm_scan_bwd_plan(int64_t Bt, int64_t L, int64_t D, int64_t N, msm_dtype io,
                             float beta, msm_plan* plan);

/* Forward scan.  y is overwritten.  last_h / last_v (the states after the final step) are
 * written when non-NULL.  Dskip may be NULL.  Requirements: Bt, L, D >= 1; 1 <= N <= 64;
 * 0 <= beta < 1; alpha finite and >= 0.  Outputs must not overlap any input. */
msm_status msm_scan_fwd(const void* x, const void* delta, const float* A, const void* B,
                        const void* C, const float* Dskip, void* y, float* last_h,
                        float* last_v, int64_t Bt, int64_t L, int64_t D, int64_t N, float beta,
                        float alpha, msm_dtype io, void* workspace, size_t workspace_bytes,
                        void* stream);

/* Forward scan with an explicit plan (NULL plan = automatic, identical to msm_scan_fwd). */
msm_status msm_scan_fwd_with_plan(const void* x, const void* delta, const float* A,
                                  const void* B, const void* C, const float* Dskip, void* y,
                                  float* last_h, float* last_v, int64_t Bt, int64_t L, int64_t D,
                                  int64_t N, float beta, float alpha, msm_dtype io,
                                  void* workspace, size_t workspace_bytes, void* stream,
                                  const msm_plan* plan);

/* Forward scan started at a given state: h0, v0 are (Bt, D, N) fp32, NULL meaning zero.  This
 * continues a sequence from the last_h / last_v a previous call returned for its first part
 * (the README's last_state outputs; chunked prefill and streaming).  The result equals one call
 * over the whole sequence up to rounding.  h0 and v0 must not overlap any output (continue
 * with a second pair of state buffers rather than in place).  plan may be NULL (automatic).
 * Everything else as msm_scan_fwd_with_plan, which is this call with h0 = v0 = NULL. */
msm_status msm_scan_fwd_state(const void* x, const void* delta, const float* A, const void* B,
                              const void* C, const float* Dskip, const float* h0,
                              const float* v0, void* y, float* last_h, float* last_v, int64_t Bt,
                              int64_t L, int64_t D, int64_t N, float beta, float alpha,
                              msm_dtype io, void* workspace, size_t workspace_bytes, void* stream,
                              const msm_plan* plan);

/* Allocation-free forward scan, for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same arguments, checks
 * and results as msm_scan_fwd, without the workspace: the chunk summaries of a chunked plan
 * live in a static device array owned by the library, MSM_NOALLOC_SCRATCH_BYTES (32 MiB) per
 * GPU, held until the process ends.  The call allocates nothing (no hipMalloc, no library
 * allocation); the first call on a device looks up that device's copy of the array.  A shape
 * whose summaries exceed the array returns MSM_ERR_WORKSPACE before anything is enqueued (use
 * msm_scan_fwd with a workspace for it).  Every call on one GPU shares that GPU's array: two
 * calls in flight on one GPU at the same time (different streams, or host threads) race and
 * must be ordered by the caller.  Nothing in the array needs to start at zero: every summary is
 * written before it is read within the call. */
#define MSM_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
msm_status msm_scan_fwd_noalloc(const void* x, const void* delta, const float* A, const void* B,
                                const void* C, const float* Dskip, void* y, float* last_h,
                                float* last_v, int64_t Bt, int64_t L, int64_t D, int64_t N,
                                float beta, float alpha, msm_dtype io, void* stream);

/* Backward scan: gradients of sum(dy * y).  dx, ddelta, dB, dC, dA are overwritten (not
 * accumulated).  dDskip is required exactly when Dskip is non-NULL.  The forward is recomputed
 * inside; no saved activations are needed.  Same requirements as msm_scan_fwd, and L < 2^30
 * (a longer sequence returns MSM_ERR_UNSUPPORTED: split it with msm_scan_bwd_state) and
 * 64 * D * (element size) < 2^31 (D < 2^23 channels with fp32 I/O). */
msm_status msm_scan_bwd(const void* x, const void* delta, const float* A, const void* B,
                        const void* C, const float* Dskip, const void* dy, void* dx,
                        void* ddelta, float* dA, void* dB, void* dC, float* dDskip, int64_t Bt,
                        int64_t L, int64_t D, int64_t N, float beta, float alpha, msm_dtype io,
                        void* workspace, size_t workspace_bytes, void* stream);

msm_status msm_scan_bwd_with_plan(const void* x, const void* delta, const float* A,
                                  const void* B, const void* C, const float* Dskip,
                                  const void* dy, void* dx, void* ddelta, float* dA, void* dB,
                                  void* dC, float* dDskip, int64_t Bt, int64_t L, int64_t D,
                                  int64_t N, float beta, float alpha, msm_dtype io,
                                  void* workspace, size_t workspace_bytes, void* stream,
                                  const msm_plan* plan);

/* Backward of a scan started at (h0, v0) (NULL: zero), for the loss
 *   sum(dy * y) + <dlast_h, last_h> + <dlast_v, last_v>
 * (dlast_h, dlast_v: (Bt, D, N) fp32 adjoints of the final state, NULL meaning zero).  Besides
 * the gradients of msm_scan_bwd it writes the adjoints of the initial state, dh0 = a_0 gh_0 and
 * dv0 = beta gv_0 ((Bt, D, N) fp32), when dh0 / dv0 are non-NULL.  A sequence split in two is
 * differentiated by running the second part first and passing its dh0 / dv0 as the first
 * part's dlast_h / dlast_v (Momentum Mamba README, "Gradient Flow", read with the terminal
 * terms of a split sequence).  msm_scan_bwd_with_plan is this call with every state pointer
 * NULL. */
msm_status msm_scan_bwd_state(const void* x, const void* delta, const float* A, const void* B,
                              const void* C, const float* Dskip, const void* dy, const float* h0,
                              const float* v0, const float* dlast_h, const float* dlast_v,
                              void* dx, void* ddelta, float* dA, void* dB, void* dC,
                              float* dDskip, float* dh0, float* dv0, int64_t Bt, int64_t L,
                              int64_t D, int64_t N, float beta, float alpha, msm_dtype io,
                              void* workspace, size_t workspace_bytes, void* stream,
                              const msm_plan* plan);

/* The full selective-scan operation: the function of the Momentum Mamba README ("Low-Level
 * Functions": u, delta, A, B, C, D, z, delta_bias, delta_softplus, beta, alpha, with last
 * states) plus the initial state of msm_scan_fwd_state.  Read as in the Mamba block of
 * "Where the state computation sits in a Mamba block":
 *     delta_eff[b,t,d] = softplus(delta[b,t,d] + delta_bias[d])   when delta_softplus == 1
 *                      = delta[b,t,d] + delta_bias[d]             when delta_softplus == 0
 *     (softplus(u) = log(1 + e^u); a NULL delta_bias is zero),
 *     the scan of msm_scan_fwd_state runs on delta_eff, giving y_raw (skip term included),
 *     y = y_raw * silu(z)  with silu(z) = z / (1 + e^-z), when z (Bt, L, D, io dtype) is given.
 * delta_bias is (D,) fp32.  delta_softplus must be 0 or 1.
 * zero_order_hold (0 or 1) selects the write coefficient: 0 keeps the first-order delta of the
 * README's "Discretization Note"; 1 uses the zero-order hold Bbar = (exp(delta_eff A) - 1) A^{-1} B
 * of the glossary and complextorch pages ("The diagonal SSM"), i.e.
 *     v_t = beta v_{t-1} + alpha ((exp(delta_eff A) - 1) / A) B_t x_t   (delta_eff at A = 0).
 * With z, delta_bias NULL and delta_softplus = zero_order_hold = 0 this is msm_scan_fwd_state.
 * The bias, softplus and gate are applied inside the scan kernels (no extra pass over memory).  Everything else as msm_scan_fwd_state; z and
 * delta_bias are inputs and must not overlap an output. */
msm_status msm_selective_scan_fwd(const void* x, const void* delta, const float* A,
                                  const void* B, const void* C, const float* Dskip, const void* z,
                                  const float* delta_bias, int32_t delta_softplus,
                                  int32_t zero_order_hold, const float* h0, const float* v0,
                                  void* y, float* last_h,
                                  float* last_v, int64_t Bt, int64_t L, int64_t D, int64_t N,
                                  float beta, float alpha, msm_dtype io, void* workspace,
                                  size_t workspace_bytes, void* stream, const msm_plan* plan);

/* Backward of msm_selective_scan_fwd for the loss of msm_scan_bwd_state.  ddelta is the
 * gradient of the raw delta (through the bias and softplus); dz (Bt, L, D, io dtype) is
 * required exactly when z is given and ddelta_bias ((D,) fp32, summed over batch and time)
 * exactly when delta_bias is given.  The output before the gate, which dz needs, is recomputed
 * inside: nothing from the forward is saved.  zero_order_hold as in msm_selective_scan_fwd.
 * With z, delta_bias NULL and delta_softplus = zero_order_hold = 0 this is msm_scan_bwd_state. */
msm_status msm_selective_scan_bwd(const void* x, const void* delta, const float* A,
                                  const void* B, const void* C, const float* Dskip, const void* z,
                                  const float* delta_bias, int32_t delta_softplus,
                                  int32_t zero_order_hold, const void* dy,
                                  const float* h0, const float* v0, const float* dlast_h,
                                  const float* dlast_v, void* dx, void* ddelta, float* dA,
                                  void* dB, void* dC, float* dDskip, void* dz,
                                  float* ddelta_bias, float* dh0, float* dv0, int64_t Bt,
                                  int64_t L, int64_t D, int64_t N, float beta, float alpha,
                                  msm_dtype io, void* workspace, size_t workspace_bytes,
                                  void* stream, const msm_plan* plan);

/* Single-token decode step (the README's Mamba `step`: hidden_states of one position plus the
 * ssm_state and velocity_state caches, "Low-Level Functions" / `allocate_inference_cache`),
 * for the scan part of the block.  x, delta, z, y: (Bt, D) io dtype -- the token's input, raw
 * step size, gate and output; B, C: (Bt, N) io; A (D, N), Dskip (D,), delta_bias (D,) fp32;
 * h, v: (Bt, D, N) fp32 ssm and velocity states, read and overwritten IN PLACE with the states
 * after this token.  Computes, per (b, d, n), with delta_eff as in msm_selective_scan_fwd:
 *     v <- beta v + alpha delta_eff B x,  h <- exp(delta_eff A) h + v,
 *     y  = (sum_n C h + Dskip x) * silu(z)        (gate only when z is non-NULL)
 * which is msm_selective_scan_fwd over a sequence of length one started at (h, v), up to fp32
 * rounding.  Zero-initialised h, v start a new sequence; the last_h / last_v of a prefill call
 * continue one.  z, Dskip and delta_bias may be NULL; delta_softplus and zero_order_hold
 * (as in msm_selective_scan_fwd) are 0 or 1.  h and v must
 * not overlap each other, an input or y.  Needs no workspace.  Same requirements on Bt, D, N,
 * beta, alpha and io as msm_scan_fwd. */
msm_status msm_scan_step(const void* x, const void* delta, const float* A, const void* B,
                         const void* C, const float* Dskip, const void* z,
                         const float* delta_bias, int32_t delta_softplus,
                         int32_t zero_order_hold, float* h, float* v, void* y, int64_t Bt,
                         int64_t D, int64_t N, float beta, float alpha, msm_dtype io,
                         void* stream);

/* Complex-valued scan (Momentum Mamba README, "Complex Number Support": the same recurrence
 * with A, B and C complex; complextorch, "The diagonal SSM", for the complex diagonal state).
 * x, delta, y, dy, dx, ddelta are real (Bt, L, D) io arrays as above; for every (b, d, n):
 *     a_t = exp(delta[b,t,d] * A[d,n])                 (complex exponential)
 *     v_t = beta * v_{t-1} + alpha * delta[b,t,d] * x[b,t,d] * B[b,t,n]
 *     h_t = a_t * h_{t-1} + v_t
 *     y[b,t,d] = Re(sum_n C[b,t,n] * h_t)  (+ Dskip[d] * x[b,t,d])
 * Complex arrays are interleaved (re, im) pairs, i.e. an extra trailing dimension of 2:
 *   A, dA: (D, N, 2) fp32; B, C, dB, dC: (Bt, L, N, 2) in the io dtype (for MSM_F32 the memory
 *   of a complex64 array); h0, v0, last_h, last_v, dlast_h, dlast_v, dh0, dv0: (Bt, D, N, 2) fp32.
 * The real part of C h is the readout (a conjugate-pair convention, C h + conj(C h), would be
 * twice this).  h0, v0 (NULL = zero) start the scan; last_h, last_v (may be NULL) receive the
 * final state.  Requirements as msm_scan_fwd, L < 2^30 (else MSM_ERR_UNSUPPORTED), and
 * 17 * N * D * 8 < 2^31 (the kernels address 17 rows of the state history with 32-bit
 * offsets); B and C must be aligned to a whole complex
 * element (8 bytes for MSM_F32, 4 for MSM_BF16), else MSM_ERR_INVALID_ARG.
 * Needs no workspace. */
msm_status msm_scan_complex_fwd(const void* x, const void* delta, const float* A, const void* B,
                                const void* C, const float* Dskip, const float* h0,
                                const float* v0, void* y, float* last_h, float* last_v,
                                int64_t Bt, int64_t L, int64_t D, int64_t N, float beta,
                                float alpha, msm_dtype io, void* stream);

/* Workspace of msm_scan_complex_bwd: the state history Bt * (L + 1) * N * D * 8 bytes plus the
 * per-block partial sums.  Returns 0 for invalid sizes. */
size_t msm_scan_complex_bwd_workspace_bytes(int64_t Bt, int64_t L, int64_t D, int64_t N,
                                            msm_dtype io);

/* Backward of msm_scan_complex_fwd for the real loss
 *     sum(dy * y) + <dlast_h, last_h> + <dlast_v, last_v>,   <u, w> = Re sum conj(u) w
 * (dlast_h, dlast_v NULL = zero).  The gradient of a complex input is written as
 * dL/dRe + i dL/dIm (the convention of PyTorch's complex autograd for a real loss): dA (summed
 * over batch and time), dB, dC (summed over channels), and dh0, dv0 when non-NULL.  dx, ddelta
 * are real; dDskip is required exactly when Dskip is given.  A forward pass that records every
 * state into the workspace runs first; nothing from an earlier forward call is needed.  The
 * workspace must be 16-byte aligned (MSM_ERR_INVALID_ARG otherwise).
 * Everything else as msm_scan_complex_fwd. */
msm_status msm_scan_complex_bwd(const void* x, const void* delta, const float* A, const void* B,
                                const void* C, const float* Dskip, const float* h0,
                                const float* v0, const void* dy, const float* dlast_h,
                                const float* dlast_v, void* dx, void* ddelta, float* dA,
                                void* dB, void* dC, float* dDskip, float* dh0, float* dv0,
                                int64_t Bt, int64_t L, int64_t D, int64_t N, float beta,
                                float alpha, msm_dtype io, void* workspace,
                                size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MSM_H_ */
