/*
 * linattn.h -- C ABI of liblinattn.so: chunkwise causal linear attention on AMD
 * Instinct MI355X (gfx950), hand-written HIP kernels.
 *
 * What the library computes (per batch b, head h, in the recurrent form the
 * prefill reproduces exactly up to rounding):
 *
 *   S_t = gamma_h S_{t-1} + psi(k_t) v_t^T        (n_psi x d_v, fp32)
 *   Z_t = gamma_h Z_{t-1} + psi(k_t)              (n_psi, fp32)
 *   o_t = psi(q_t)^T S_t / (psi(q_t) . Z_t + eps)  if normalize
 *   o_t = psi(q_t)^T S_t                           otherwise
 *
 * Sources (page title, section):
 *  - "Log-Depth Chunked Linear-Attention Scan", Mathematical statement and
 *    Implementation notes: states S_t and Z_t summed over i <= t, chunk summaries
 *    S_c^loc, Z_c^loc, their additive monoid, the exclusive prefix over chunks,
 *    the three kernels (local pass, scan, output), eps in the denominator, fp32
 *    summaries, zero contribution from padded positions.
 *  - "Linear Attention and Retentive Networks": elu(x)+1 feature map (The
 *    Associative Property and Linear Kernel Formulation), the recurrent dual
 *    (The Recurrent Dual), per-head decay gamma and the decayed recurrent and
 *    chunkwise forms (Retentive Networks, Multi-Scale Decay Formulation, B, C).
 *  - "Linearized 2-Simplicial Attention", section 3.2 and appendix Feature
 *    scaling: positive random features psi(x)_p = exp(w_p . x - |x|^2/2)/sqrt(m).
 *
 * Conventions for every entry point
 *  - Ownership: the caller allocates and owns every buffer. The library never
 *    allocates, frees or synchronises device memory and never changes the
 *    current device; it only enqueues kernels on `stream`.
 *  - Pointers marked "device" are device addresses on the current device and
 *    must be 16-byte aligned; "host" pointers are read before the call returns.
 *  - Layouts are dense row-major (C order) with the stated shapes.
 *  - Errors: every argument is validated on the host before anything is
 *    enqueued; an invalid call returns a status != LA_OK and enqueues nothing.
 *    LA_ERR_HIP reports a launch error (hipGetLastError); faults inside a
 *    kernel surface at the caller's next synchronisation.
 *  - Results are deterministic: the same inputs give bitwise-identical outputs
 *    (fixed reduction orders, no floating-point atomics).
 *  - Functions are re-entrant and thread-safe; calls that share output or
 *    workspace buffers must not overlap in time.
 */
#ifndef LINATTN_H_
#define LINATTN_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LA_OK = 0,
  LA_ERR_NULL = 1,        /* a required pointer is NULL                        */
  LA_ERR_SHAPE = 2,       /* a size is out of range or inconsistent            */
  LA_ERR_UNSUPPORTED = 3, /* a valid combination this build has no kernel for  */
  LA_ERR_WORKSPACE = 4,   /* workspace missing or smaller than required        */
  LA_ERR_ALIGN = 5,       /* a device pointer is not 16-byte aligned           */
  LA_ERR_VALUE = 6,       /* eps < 0, gamma outside (0, 1], bad enum value     */
  LA_ERR_HIP = 7          /* the HIP runtime reported an error at launch       */
} la_status;

/* Feature map psi. */
typedef enum {
  LA_PSI_IDENTITY = 0, /* psi(x) = x; requires n_psi == d_k                        */
  LA_PSI_ELU1 = 1,     /* psi(x)_j = x_j + 1 if x_j > 0 else exp(x_j); n_psi == d_k */
  LA_PSI_PRF = 2,      /* psi(x)_p = exp(w_p . x - |x|^2/2) / sqrt(n_psi)           */
  LA_PSI_PRF_QSHIFT = 3 /* the same features with the log-space shift of the query
                         * row ("Linearized 2-Simplicial Attention", appendix B.2):
                         * psi(q)_p = exp(l_p - max_r l_r) / sqrt(n_psi), l_p = w_p . q
                         * - |q|^2/2; keys unshifted. The shift depends on the query
                         * row only and scales numerator and denominator alike, so the
                         * output equals LA_PSI_PRF's with eps weighted by exp(max_r l_r);
                         * it keeps psi(q) . S finite for large-magnitude queries.
                         * Requires normalize == 1 (LA_ERR_UNSUPPORTED otherwise):
                         * without the denominator nothing cancels the shift.        */
} la_psi;

typedef enum { LA_BF16 = 0, LA_F32 = 1 } la_dtype;

/* Layout of the token tensors q, k, v and o of lin_attn_prefill (d is d_k or d_v). */
typedef enum {
  LA_LAYOUT_BHTD = 0, /* [B, H, T, d]: each head's tokens contiguous                  */
  LA_LAYOUT_BTHD = 1  /* [B, T, H, d]: heads interleaved per token, the layout of a   *
                       * projection output viewed as (B, T, H, d), no transpose needed */
} la_layout;

/* Prefill (training / prompt) problem description. All fields are int32 so the
 * struct has the same layout from C, C++ and ctypes. */
typedef struct {
  int32_t B, H, T;       /* batch, heads, sequence length (T >= 1, any value:
                            the last chunk may be ragged)                        */
  int32_t d_k, d_v;      /* key/query and value widths                           */
  int32_t n_psi;         /* feature width: == d_k unless psi is a PRF map        */
  int32_t chunk;         /* chunk size C: the token block of the method; segment
                            boundaries (where the scanned states apply) fall on
                            multiples of C. Within a chunk the kernels may group
                            tokens differently (the bf16 kernels walk 64-token
                            steps, and with C = 32 a segment holds an even number
                            of chunks); the result is the same function,
                            C-invariant up to rounding                           */
  int32_t psi;           /* la_psi                                               */
  int32_t normalize;     /* 1: divide by psi(q).Z + eps; 0: numerator only       */
  float eps;             /* >= 0; used only when normalize == 1                  */
  int32_t in_dtype;      /* la_dtype of q, k, v and prf_w                        */
  int32_t out_dtype;     /* la_dtype of o: LA_F32, or LA_BF16 = the fp32 result
                            rounded to nearest even (in_dtype LA_BF16 only)      */
  int32_t layout;        /* la_layout of q, k, v, o (0 = [B, H, T, d]); states
                            are [B, H, n_psi, d_v] in every layout               */
} la_prefill_desc;

/* Supported sizes in this build (anything else: LA_ERR_UNSUPPORTED):
 *   in_dtype LA_BF16: psi identity/elu1: d_k == d_v == n_psi in {64, 128},
 *                     chunk in {32, 64, 128};
 *                     psi PRF, PRF_QSHIFT: d_k == d_v == 128, n_psi in {128, 256},
 *                     chunk in {32, 64, 128}.
 *   in_dtype LA_F32 : d_k, d_v <= 128, d_k a multiple of 4, n_psi <= 256 (LDS permitting),
 *                     chunk in {16, 32, 64}, any psi.
 *   always: d_v and n_psi multiples of 4 (16-byte state rows in the workspace).
 *   out_dtype LA_BF16 with in_dtype LA_BF16 only.
 *   gamma: when given, at most LA_MAX_DECAY_HEADS heads.                        */
#define LA_MAX_DECAY_HEADS 256

/* Device workspace bytes lin_attn_prefill needs for `d` (0 is possible).
 * Pure host function. Returns LA_OK and writes *bytes, or a validation error. */
la_status lin_attn_prefill_workspace_size(const la_prefill_desc* d, size_t* bytes);

/* The same for lin_attn_prefill_varlen with this `d` (B = number of sequences,
 * T = longest length) and total_tokens >= 0 packed tokens: segments are sized from
 * the total, so the workspace depends on it. */
la_status lin_attn_prefill_varlen_workspace_size(const la_prefill_desc* d, int32_t total_tokens, size_t* bytes);

/*
 * Chunkwise causal linear attention over whole sequences ("Log-Depth Chunked
 * Linear-Attention Scan", Implementation notes: a chunk-local pass that emits
 * chunk summaries, an exclusive associative scan over them, and an output pass;
 * with decay, the chunkwise recurrent representation of "Linear Attention and
 * Retentive Networks", section C, whose summaries combine as
 * (a1, S1) (+) (a2, S2) = (a1 a2, a2 S1 + S2)).
 *
 *   q, k      device [B, H, T, d_k] in_dtype ([B, T, H, d_k] for LA_LAYOUT_BTHD)
 *   v         device [B, H, T, d_v] in_dtype (likewise)
 *   gamma     host   [H] fp32 per-head decay, 0 < gamma <= 1; NULL means 1
 *   prf_w     device [H, n_psi, d_k] in_dtype (the PRF bank, one per head,
 *             shared over the batch); required iff psi is LA_PSI_PRF or
 *             LA_PSI_PRF_QSHIFT
 *   init_S    device [B, H, n_psi, d_v] fp32 state before token 1, or NULL (zero)
 *   init_Z    device [B, H, n_psi] fp32, or NULL (zero); ignored when normalize == 0
 *   o         device [B, H, T, d_v] out_dtype ([B, T, H, d_v] for LA_LAYOUT_BTHD),
 *             written for every t < T
 *   final_S   device [B, H, n_psi, d_v] fp32 state after token T, or NULL
 *   final_Z   device [B, H, n_psi] fp32, or NULL; not written when normalize == 0
 *             (without a denominator the normaliser is not maintained)
 *   workspace device buffer of at least lin_attn_prefill_workspace_size bytes
 *             (contents on entry ignored; NULL allowed when that size is 0)
 * Outputs must not alias inputs. Asynchronous on `stream`.
 */
la_status lin_attn_prefill(const la_prefill_desc* d, const void* q, const void* k, const void* v,
                           const float* gamma, const void* prf_w, const float* init_S,
                           const float* init_Z, void* o, float* final_S, float* final_Z,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * lin_attn_prefill over a batch of sequences of different lengths packed end to end
 * (the variable-length batches of serving, where prompts of many lengths are
 * prefilled together; "Log-Depth Chunked Linear-Attention Scan", Implementation
 * notes: every sequence's ragged tail contributes zero). Each sequence is an
 * independent problem with its own state; no token attends across a boundary.
 *
 *   d           as for lin_attn_prefill with B = number of sequences and
 *               T = the longest sequence length (host value, >= every length);
 *               layout must be LA_LAYOUT_BTHD (tokens of all heads interleaved)
 *   cu_seqlens  device [B + 1] int32: sequence b is tokens
 *               [cu_seqlens[b], cu_seqlens[b+1]) of the packed tensors;
 *               cu_seqlens[0] = 0, non-decreasing, cu_seqlens[B] = total_tokens.
 *               Lengths may be 0 (no output; final state = initial state).
 *               Offsets outside these rules give unspecified outputs but are
 *               clamped, so no access falls outside the tensors.
 *   total_tokens host, >= 0: tokens in the packed tensors
 *   q, k        device [total_tokens, H, d_k];  v device [total_tokens, H, d_v]
 *   o           device [total_tokens, H, d_v] out_dtype
 *   init_S, init_Z, final_S, final_Z: per sequence, [B, H, n_psi, d_v] / [B, H, n_psi]
 *   workspace   at least lin_attn_prefill_varlen_workspace_size(d, total_tokens) bytes
 *   other arguments as for lin_attn_prefill.
 */
la_status lin_attn_prefill_varlen(const la_prefill_desc* d, const int32_t* cu_seqlens, int32_t total_tokens,
                                  const void* q, const void* k, const void* v, const float* gamma,
                                  const void* prf_w, const float* init_S, const float* init_Z, void* o,
                                  float* final_S, float* final_Z, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream);

/*
 * lin_attn_prefill with phase timing for profilers and benchmarks: identical work
 * and results, plus four events recorded on `stream` -- events[0] before the
 * segment-summary kernel, events[1] after it, events[2] after the segment scan,
 * events[3] after the output kernel. `events` is a host array of 4 events created
 * by the caller on the current device; NULL entries are skipped.
 */
la_status lin_attn_prefill_profiled(const la_prefill_desc* d, const void* q, const void* k,
                                    const void* v, const float* gamma, const void* prf_w,
                                    const float* init_S, const float* init_Z, void* o,
                                    float* final_S, float* final_Z, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream,
                                    hipEvent_t* events);

/* Per-device scratch of lin_attn_prefill_noalloc (its summary records), in bytes. */
#define LA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * lin_attn_prefill for callers that cannot allocate device memory: code under HIP graph
 * capture, serving loops and harnesses that forbid hipMalloc. Same arguments, results and
 * errors as lin_attn_prefill minus the workspace, which is replaced by a library-owned scratch
 * array of LA_NOALLOC_SCRATCH_BYTES on each device (reserved when the library's code object
 * is loaded on that device, held until the process ends). The call allocates nothing.
 *   - When the usual segment plan's summary records exceed the scratch, the call uses fewer,
 *     longer segments (the same function; results agree with lin_attn_prefill's to rounding).
 *     When not even one record per sequence fits -- B * H * (n_psi * d_v + n_psi) * 4 bytes
 *     above LA_NOALLOC_SCRATCH_BYTES -- it returns LA_ERR_WORKSPACE before touching the device.
 *   - Every call on a device uses that device's one array and leaves its contents behind;
 *     nothing in it needs to start at zero. Calls that overlap in time on one device (other
 *     streams or threads) race on the array: the caller serialises them.
 *   - The first call on each device looks the array's address up (hipGetSymbolAddress):
 *     LA_ERR_HIP if that fails. Fixed-length batches only (no varlen or gated form).
 */
la_status lin_attn_prefill_noalloc(const la_prefill_desc* d, const void* q, const void* k, const void* v,
                                   const float* gamma, const void* prf_w, const float* init_S,
                                   const float* init_Z, void* o, float* final_S, float* final_Z,
                                   hipStream_t stream);

/*
 * Chunkwise causal linear attention with data-dependent forget gates ("Linear Attention
 * and Retentive Networks", Data-Dependent Gating Mechanism: S_t = G_t . S_{t-1} + k_t^T v_t
 * with G_t = alpha_t 1^T, one gate per state row and token):
 *   S_t[p][:] = alpha_t[p] S_{t-1}[p][:] + psi(k_t)[p] v_t^T,   alpha_t = exp(log_gate_t)
 *   Z_t[p]    = alpha_t[p] Z_{t-1}[p]    + psi(k_t)[p]
 *   o_t       = psi(q_t)^T S_t / (psi(q_t) . Z_t + eps)   (numerator alone if !normalize)
 * The gates replace gamma. Chunks combine under (a1, X1) (+) (a2, X2) = (a1 a2,
 * diag(a2) X1 + X2) with a the per-row product of a chunk's gates.
 *
 *   d         as for lin_attn_prefill; supported: psi identity or elu1, d_k == d_v ==
 *             n_psi in {64, 128}, chunk 32, in_dtype LA_BF16 or LA_F32, either layout
 *   log_gate  device fp32, laid out like k ([B, H, T, d_k] or [B, T, H, d_k]): the log of
 *             each token's gate per state row, <= 0 (gates in (0, 1]). Values must be
 *             finite; an exact reset between documents is a sequence boundary (separate
 *             batch entries), not a gate.
 *   workspace at least lin_attn_prefill_gated_workspace_size bytes
 *   other arguments as for lin_attn_prefill (no gamma, no PRF bank).
 * bf16 inputs run on the matrix cores with every gate-scaled operand carried as a two-term
 * (hi + lo) bf16 pair, since the gate factors make them inexact in one bf16; fp32 inputs
 * run on the vector ALUs in fp32.
 */
la_status lin_attn_prefill_gated_workspace_size(const la_prefill_desc* d, size_t* bytes);
la_status lin_attn_prefill_gated(const la_prefill_desc* d, const void* q, const void* k, const void* v,
                                 const float* log_gate, const float* init_S, const float* init_Z, void* o,
                                 float* final_S, float* final_Z, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream);

/*
 * Backward pass of lin_attn_prefill: for L = sum_t dout_t . o_t, the gradients of L with
 * respect to q, k, v and the initial state of the same prefill (same d, q, k, v, gamma,
 * init_S, init_Z). Two sweeps ("Linearized 2-Simplicial Attention", 4.2 Custom Triton
 * kernel, Backward, and the appendix's backward query and state sweeps): a query sweep that
 * recomputes the prefix state (and, with a denominator, dout_t . o_t from it, so no forward
 * output is needed) and gives dq, then a state sweep over the adjoint state
 * R_t = sum_{u >= t} gamma^(u-t) psi(q_u) dnum_u^T (dnum_u = dout_u / den_u) that gives dk and dv;
 * across segments the adjoint state is the forward scan's monoid run in reverse order.
 * gamma, eps and the feature map's bank are constants (no gradient for them). With random
 * features the feature map's Jacobian follows ("Linearized 2-Simplicial Attention", 3.2):
 * dx = sum_p a_p w_p - (sum_p a_p) x with a_p = dL/dpsi_p psi_p(x), where under the query-row
 * shift the last term of dq takes the row of the bank that attains the shift (the argmax).
 *
 *   d         as for lin_attn_prefill; supported:
 *               in_dtype LA_BF16 on the matrix cores, chunk 32, 64 or 128 (walked in steps of
 *               64 tokens: the gradient does not depend on the grouping):
 *                 psi identity or elu1: d_k == d_v == n_psi == 128;
 *                 psi PRF or PRF_QSHIFT: d_k == d_v == 128, n_psi 128 or 256;
 *               in fp32 on the vector ALUs (steps of 16 tokens, the same segment records):
 *                 in_dtype LA_BF16, psi identity or elu1, d_k == d_v == n_psi == 64, chunk 32,
 *                 64 or 128;
 *                 in_dtype LA_F32 (out_dtype LA_F32), every psi, wherever lin_attn_prefill
 *                 takes the shape (chunk 16, 32 or 64) and the state plus one step's rows fit
 *                 in 160 KiB of LDS with n_psi * d_v <= 16384 (d = 128 with n_psi 128; d = 64
 *                 with n_psi up to 256);
 *             either layout. out_dtype is the type of dout (LA_F32, or LA_BF16 with bf16
 *             inputs).
 *   prf_w     device [H, n_psi, d_k] bf16, the forward call's bank; required iff psi is a
 *             random-feature map
 *   dout      device, dL/do, laid out like lin_attn_prefill's o, out_dtype
 *   dq, dk    device fp32, laid out like q and k
 *   dv        device fp32, laid out like v
 *   dinit_S   device fp32 [B, H, n_psi, d_v] or NULL; dinit_Z [B, H, n_psi] or NULL (not
 *             written when normalize == 0)
 *   workspace at least lin_attn_prefill_backward_workspace_size bytes: two segment-summary
 *             regions (random features: one record per 64-token step), 8 bytes per token-head
 *             when normalize == 1, and for random features a transposed copy of the bank
 * Errors as for lin_attn_prefill. Rows past T are neither read nor written.
 */
la_status lin_attn_prefill_backward_workspace_size(const la_prefill_desc* d, size_t* bytes);
la_status lin_attn_prefill_backward(const la_prefill_desc* d, const void* q, const void* k, const void* v,
                                    const float* gamma, const void* prf_w, const float* init_S, const float* init_Z,
                                    const void* dout, float* dq, float* dk, float* dv, float* dinit_S,
                                    float* dinit_Z, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * lin_attn_prefill_backward over a packed batch of variable-length sequences: the backward
 * pass of lin_attn_prefill_varlen with the same d, cu_seqlens, total_tokens, q, k, v, gamma,
 * init_S and init_Z. Each sequence's gradients depend only on its own tokens and initial state.
 *
 *   d, cu_seqlens, total_tokens  as for lin_attn_prefill_varlen (layout LA_LAYOUT_BTHD),
 *                subject to lin_attn_prefill_backward's support limits, identity or elu1
 *                features only (random features: LA_ERR_UNSUPPORTED; their per-step records
 *                would scale with the longest sequence times the batch)
 *   prf_w        as for lin_attn_prefill_backward (NULL here)
 *   dout         device [total_tokens, H, d_v] out_dtype
 *   dq, dk       device fp32 [total_tokens, H, d_k];  dv device fp32 [total_tokens, H, d_v]
 *   dinit_S, dinit_Z  per sequence, [B, H, n_psi, d_v] / [B, H, n_psi], or NULL; an empty
 *                sequence's are zero
 *   workspace    at least lin_attn_prefill_backward_varlen_workspace_size(d, total_tokens) bytes
 * Errors as for lin_attn_prefill_varlen. Token rows outside every sequence are not written.
 */
la_status lin_attn_prefill_backward_varlen_workspace_size(const la_prefill_desc* d, int32_t total_tokens,
                                                          size_t* bytes);
la_status lin_attn_prefill_backward_varlen(const la_prefill_desc* d, const int32_t* cu_seqlens, int32_t total_tokens,
                                           const void* q, const void* k, const void* v, const float* gamma,
                                           const void* prf_w, const float* init_S, const float* init_Z,
                                           const void* dout, float* dq, float* dk, float* dv, float* dinit_S,
                                           float* dinit_Z, void* workspace, size_t workspace_bytes,
                                           hipStream_t stream);

/* Batched single-token decode description: N independent streams x H heads. */
typedef struct {
  int32_t N, H;
  int32_t d_k, d_v, n_psi;
  int32_t psi;       /* la_psi */
  int32_t normalize;
  float eps;
  int32_t in_dtype;  /* la_dtype of q, k, v, prf_w */
  int32_t out_dtype; /* la_dtype of o: LA_F32, or LA_BF16 with bf16 inputs (the fp32
                        result rounded to nearest even)                          */
} la_decode_desc;

/* Supported: in_dtype LA_BF16 or LA_F32; d_k == d_v in {64, 128}; psi identity
 * or elu1 (n_psi == d_k), or PRF with n_psi in {64, 128, 256}.                  */

/*
 * One recurrent decode step for every (stream, head), updating the state in
 * place ("Linear Attention and Retentive Networks", The Recurrent Dual and
 * recurrent representation B: O(1) memory per step, no token-level cache):
 *   S <- gamma S + psi(k) v^T;  Z <- gamma Z + psi(k);
 *   o  = psi(q)^T S / (psi(q) . Z + eps)   (numerator only if normalize == 0)
 * The update comes first, so o includes the new token.
 *
 *   q, k  device [N, H, d_k] in_dtype;  v device [N, H, d_v] in_dtype
 *   gamma host [H] fp32 or NULL (1);  prf_w device [H, n_psi, d_k] or NULL
 *   S     device [N, H, n_psi, d_v] fp32, read and written in place
 *   Z     device [N, H, n_psi] fp32, in place; when normalize == 0 it is neither
 *         read nor written and may be NULL
 *   o     device [N, H, d_v] out_dtype
 */
la_status lin_attn_decode_step(const la_decode_desc* d, const void* q, const void* k, const void* v,
                               const float* gamma, const void* prf_w, float* S, float* Z, void* o,
                               hipStream_t stream);

/*
 * lin_attn_decode_step with per-row forget gates in place of gamma (same page, Data-
 * Dependent Gating Mechanism): S[p][:] <- alpha[p] S[p][:] + psi(k)[p] v^T, Z[p] <- alpha[p]
 * Z[p] + psi(k)[p], alpha = exp(log_gate), then o as above. log_gate: device fp32
 * [N, H, n_psi], <= 0, finite. Other arguments as for lin_attn_decode_step (no gamma).
 */
la_status lin_attn_decode_step_gated(const la_decode_desc* d, const void* q, const void* k, const void* v,
                                     const float* log_gate, const void* prf_w, float* S, float* Z, void* o,
                                     hipStream_t stream);

/* Diagnostic: the segment scan and its depth ("Log-Depth Chunked Linear-Attention Scan",
 * Verification: the scan's round count is the check of its log depth). Runs the scan the
 * prefill runs on one sequence of n_seg segments with 4 x 4 states and no decay, replacing
 * each record with its exclusive prefix, and raises *rounds to the number of dependent (+)
 * levels the kernel executed:
 *   n_seg <= 128: W waves (a power of two <= 16) fold runs of up to ceil(n_seg / W) segments
 *     in sequence, a Blelloch tree takes log2 W levels up and log2 W down, one step carries
 *     the initial state and each run is rewritten: 2 ceil(n_seg / W) + 2 log2 W + 1;
 *   n_seg > 128: lanes hold segments; per block of 64 NW segments (NW = 4, 8 or 16 waves)
 *     6 lane-shift rounds, log2 NW levels up and down, and 2 combines with the carried
 *     prefix: ceil(n_seg / (64 NW)) (8 + 2 log2 NW).
 *   ws:     device fp32, n_seg records of 20 floats (S row-major 4 x 4, then Z), 16-byte
 *           aligned; on return record s holds the sum of records 0 .. s-1.
 *   rounds: device int32, set by the caller (e.g. to 0) before the call; raised by atomic max.
 * Errors: LA_ERR_NULL, LA_ERR_SHAPE (n_seg outside 1 .. 65535), LA_ERR_ALIGN, LA_ERR_HIP.
 * Asynchronous on `stream`. */
la_status lin_attn_scan_depth(int32_t n_seg, float* ws, int32_t* rounds, hipStream_t stream);

/* Static, NUL-terminated description of a status code. */
const char* lin_attn_status_string(la_status s);

/* Library version as "major.minor.patch". */
const char* lin_attn_version(void);

#ifdef __cplusplus
}
#endif
#endif /* LINATTN_H_ */
