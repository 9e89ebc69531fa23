/*
 * ssmvjp.h -- C ABI of libssmvjp: the backward pass (VJP) of the selective
 * state-space scan on AMD Instinct MI355X (gfx950).
 *
 * The operation.  The forward scan keeps a state s_t[h,p,n] per (batch, head):
 *     delta_t,h = softplus(dt_t,h)                  (dt is the raw, pre-softplus value)
 *     a_t       = exp(delta_t,h * A)                (A = A_h: Mamba-2, one decay per head;
 *                                                    A = A_h,n: Mamba-1, one decay per state)
 *     s_t       = a_t * s_{t-1} + delta_t,h * x_t[h,p] * B_t[g,n]
 *     y_t[h,p]  = sum_n C_t[g,n] * s_t[h,p,n]       (reads the state after the update)
 * with s_{-1} = s0 and head h reading group g = h / (H/G).  Given the upstream
 * gradients dy (of y) and ds_final (of the final state s_{T-1}), the library
 * returns the five gradients dx, d_dt, dB, dC, d_s0 of
 *     J = <dy, y> + <ds_final, s_{T-1}>.
 * This is the reverse-time recurrence of llama.cpp PR "S1-31: SSM_SCAN_BACK --
 * Mamba has a backward" (the op paragraph: five gradients from one op, both the
 * per-head and the per-state decay branch), seeded at t = T with the non-zero
 * final-state gradient (its point 1) and needing s_{t-1} for the decay path of
 * d_dt (its point 2).
 *
 * The chunked entry point computes the same gradients with the chunked SSD
 * algorithm of burn-mamba "combined_backward.rs" (combined_backward: K1..K4
 * recompute, reverse chunk loop over the BLUE / ORANGE / K4 backwards, batched
 * K3 / K2 / K1 backwards), including the fused L*M length of the MIMO form.
 * The delta-rule entry point is the KDA backward of the K3 notes section
 * "反向传播推导" (forward F1..F6, BPTT steps 1..6, GVA view+sum).
 *
 * Conventions shared by every entry point
 *  - All tensors are dense, row-major, innermost axis last, and live in device
 *    memory of the current HIP device.  The caller allocates every input,
 *    output and workspace buffer; the library allocates nothing and keeps no
 *    state between calls, so concurrent calls on different streams are safe.
 *  - `stream` is a hipStream_t (NULL = the null stream).  Work is enqueued
 *    asynchronously; the caller synchronises.
 *  - Outputs are overwritten, never accumulated into.  Inputs, outputs and the
 *    workspace must not overlap.
 *  - Validation errors (SSMVJP_EINVAL, SSMVJP_EUNSUPPORTED, SSMVJP_EWORKSPACE)
 *    are returned before anything is enqueued.  SSMVJP_EHIP means a launch
 *    failed; outputs are then undefined.
 *  - Results are deterministic: the same inputs give bitwise-identical outputs
 *    on every call (all reductions run in a fixed order, no float atomics).
 *  - "big" tensors (x or v, B, C, dy and their gradients) are float32 or
 *    bfloat16 as selected by `dtype`; everything else is float32.
 *  - Debug finiteness mode: with the environment variable SSMVJP_CHECK_FINITE
 *    set (to anything but "0") when a call is made, every entry point scans
 *    the outputs it wrote for NaN and infinite values after its launches,
 *    synchronises the stream and returns SSMVJP_ENONFINITE if it found one
 *    (the outputs are still written).  While the mode is on, the *_workspace
 *    queries report 256 more bytes, which hold the scan's flag (burn-mamba's
 *    combined_backward checks its intermediates for NaNs in the same spirit;
 *    here the intermediates stay inside the kernels, so the outputs are
 *    checked).  Off by default: the normal calls neither scan nor synchronise.
 */
#ifndef SSMVJP_H
#define SSMVJP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SSMVJP_OK = 0,
  SSMVJP_EINVAL = 1,        /* bad descriptor, NULL required pointer, misaligned pointer */
  SSMVJP_EUNSUPPORTED = 2,  /* valid arguments outside what the kernels implement */
  SSMVJP_EWORKSPACE = 3,    /* workspace NULL or smaller than the *_workspace query */
  SSMVJP_EHIP = 4,          /* a HIP launch or runtime call failed */
  SSMVJP_ENONFINITE = 5     /* debug mode only: an output holds a NaN or an infinity */
} ssmvjp_status;

enum { SSMVJP_F32 = 0, SSMVJP_BF16 = 1 };                         /* dtype of the big tensors */
enum { SSMVJP_DECAY_PER_HEAD = 0, SSMVJP_DECAY_PER_STATE = 1 };   /* Mamba-2 / Mamba-1 */
enum { SSMVJP_FORM_MAMBA2 = 0, SSMVJP_FORM_RAW = 1 };             /* (x, dt, A) or (v, da) */

/* ------------------------------------------------------------------------ */
/* ssm_scan_bwd: sequential reverse recurrence                               */
/* ------------------------------------------------------------------------ */

typedef struct {
  int64_t batch, seqlen, nheads, headdim, dstate, ngroups; /* b, T, H, P, N, G */
  int32_t decay;      /* SSMVJP_DECAY_PER_HEAD (A is [H]) or SSMVJP_DECAY_PER_STATE (A is [H,N]) */
  int32_t dtype;      /* SSMVJP_F32 or SSMVJP_BF16 for x, B, C, dy, dx, dB, dC */
  int32_t ckpt_every; /* K: states are checkpointed every K steps and recomputed per
                         segment (llama.cpp PR, point 2: checkpoint-every-K against
                         store-all).  0 = library default.  Outputs are bitwise
                         identical for every K. */
  int32_t reserved;   /* must be 0 */
} ssmvjp_scan_desc;

/* Bytes of device workspace ssm_scan_bwd needs for `desc` (0 is valid). */
ssmvjp_status ssm_scan_bwd_workspace(const ssmvjp_scan_desc* desc, size_t* bytes);

/* Backward of the sequential selective scan.
 *   x [b,T,H,P] (dtype)   dt [b,T,H] f32 (raw)   A [H] or [H,N] f32
 *   B, C [b,T,G,N] (dtype)   s0 [b,H,P,N] f32 (NULL = zeros)
 *   dy [b,T,H,P] (dtype)   ds_final [b,H,P,N] f32 (NULL = zeros)
 * Outputs:
 *   dx [b,T,H,P] (dtype)   d_dt [b,T,H] f32   dB, dC [b,T,G,N] (dtype)
 *   d_s0 [b,H,P,N] f32
 * Constraints: b, T >= 0 (an empty batch or sequence enqueues nothing except
 * d_s0 = ds_final for T = 0); H % G == 0 (SSMVJP_EINVAL otherwise).  One
 * workgroup per (batch, head) holds the head's state in LDS, so with
 * Q = ceil(P / min(P, 16)) groups of p values
 *     N <= 1024,  P*N <= 32768,  Q*N <= 1024  and
 *     4 * (P*(N+1) + 2*Q*N + ceil(Q*N / 64)) <= 65536 bytes of LDS
 * (SSMVJP_EUNSUPPORTED otherwise; e.g. P = N = 128 needs 74,304 bytes and is
 * refused, P = 64, N = 128 fits).
 * Pointers must be 4-byte aligned (f32) or 2-byte aligned (bf16). */
ssmvjp_status ssm_scan_bwd(const ssmvjp_scan_desc* desc,
                           const void* x, const float* dt, const float* A,
                           const void* B, const void* C, const float* s0,
                           const void* dy, const float* ds_final,
                           void* dx, float* d_dt, void* dB, void* dC, float* d_s0,
                           void* workspace, size_t workspace_bytes, void* stream);

/* ssm_scan_bwd plus dA, the gradient of the decay coefficients A: dA [H]
 * (per-head decay) or [H,N] (per-state decay), float32, written (not
 * accumulated).  With a_t = exp(delta_t A) the state update gives
 * d s_t / d A = delta_t a_t s_{t-1}, so dA = sum over the batch and time of
 * delta_t a_t <dS_t, s_{t-1}> (per state: per column n).  burn-mamba's
 * combined_backward returns the decay gradient d_da; dA is its sum
 * sum_{b,t} d_da * delta, the gradient training needs for A.  The other
 * arguments and outputs are exactly those of ssm_scan_bwd; dA must not be NULL
 * when batch > 0.  The sums over the batch run in a fixed order (deterministic). */
ssmvjp_status ssm_scan_bwd_dA(const ssmvjp_scan_desc* desc,
                              const void* x, const float* dt, const float* A,
                              const void* B, const void* C, const float* s0,
                              const void* dy, const float* ds_final,
                              void* dx, float* d_dt, void* dB, void* dC, float* d_s0, float* dA,
                              void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* ssd_chunk_bwd: chunked SSD backward (Mamba-2 and Mamba-3 MIMO)            */
/* ------------------------------------------------------------------------ */

typedef struct {
  int64_t batch, seqlen, nheads, headdim, dstate, ngroups; /* b, T, H, P, N, G */
  int64_t mimo_rank;  /* M: rank of the per-step input (1 for Mamba-2) */
  int64_t chunk_len;  /* L: steps per chunk; the fused chunk length is L*M */
  int32_t form;       /* SSMVJP_FORM_MAMBA2: inputs x, dt, A (requires M == 1);
                         SSMVJP_FORM_RAW: pre-scaled inputs v, da (burn-mamba's
                         combined_backward arguments) */
  int32_t dtype;      /* SSMVJP_F32 or SSMVJP_BF16 for x/v, B, C, dy and their gradients */
} ssmvjp_ssd_desc;

ssmvjp_status ssd_chunk_bwd_workspace(const ssmvjp_ssd_desc* desc, size_t* bytes);

/* Chunked backward.  Layouts (all row-major):
 *   FORM_MAMBA2: x_or_v = x [b,T,H,P], dt_or_da = dt [b,T,H] (raw), A [H]
 *   FORM_RAW:    x_or_v = v [b,T,M,H,P], dt_or_da = da [b,T,H] (= delta*A), A = NULL
 *   B, C [b,T,M,G,N]   s0, ds_final, d_s0 [b,H,P,N] f32 (s0/ds_final NULL = zeros)
 *   dy, dx_or_dv like x_or_v;  d_dt_or_dda like dt_or_da;  dB, dC like B.
 * A last chunk shorter than L (T % L != 0) is handled as a shorter chunk.
 * Constraints (SSMVJP_EUNSUPPORTED otherwise): H % G == 0; P % 16 == 0,
 * N % 16 == 0, P <= 128, N <= 128; (P/16) * (N/16) <= 32 unless N is a
 * multiple of 32; and the fused chunk length L*M is either
 *   - a multiple of 16 up to 64 (one kernel holds the whole chunk): its
 *     working set must fit 160 KiB of LDS (P*N <= 8192 with bf16 at
 *     L*M = 64; P*N <= 4096 more or less with float32), or
 *   - a multiple of 64 above 64 with L <= 64 and M dividing 64 (row-blocked
 *     kernels, e.g. the rank-4 MIMO form with L = 64): 64 rows of B, C, x and
 *     dy plus one state must fit 160 KiB of LDS (any P, N <= 128 with bf16;
 *     P*N <= 8192 more or less with float32).
 * Alignment (SSMVJP_EINVAL otherwise): x_or_v, B, C, dy, dx_or_dv, dB and dC
 * 16-byte aligned (the kernels move them in 16-byte vectors); the float32
 * tensors 4-byte aligned; the workspace 256-byte aligned. */
ssmvjp_status ssd_chunk_bwd(const ssmvjp_ssd_desc* desc,
                            const void* x_or_v, const float* dt_or_da, const float* A,
                            const void* B, const void* C, const float* s0,
                            const void* dy, const float* ds_final,
                            void* dx_or_dv, float* d_dt_or_dda, void* dB, void* dC, float* d_s0,
                            void* workspace, size_t workspace_bytes, void* stream);

/* ssd_chunk_bwd plus dA [H] (FORM_MAMBA2 only, SSMVJP_EINVAL otherwise):
 * dA_h = sum over the batch and time of d_da * delta for head h, with d_da the
 * decay gradient the chunked backward forms on the way to d_dt (burn-mamba
 * combined_backward's d_da).  Each chunk's per-head sum is formed in the
 * chunk kernel, and the sums over (batch, chunk) run in a fixed order.  The
 * other arguments and outputs are exactly those of ssd_chunk_bwd (same
 * workspace size, same shape limits and 16-byte alignment of the big
 * tensors); dA must not be NULL when batch > 0. */
ssmvjp_status ssd_chunk_bwd_dA(const ssmvjp_ssd_desc* desc,
                               const void* x, const float* dt, const float* A,
                               const void* B, const void* C, const float* s0,
                               const void* dy, const float* ds_final,
                               void* dx, float* d_dt, void* dB, void* dC, float* d_s0, float* dA,
                               void* workspace, size_t workspace_bytes, void* stream);

/* The two stages of ssd_chunk_bwd as separate calls, for callers that want to
 * schedule or time them apart.  ssd_chunk_bwd_states followed by
 * ssd_chunk_bwd_grads on the same stream, with the same descriptor, inputs and
 * workspace, is exactly ssd_chunk_bwd.
 *  - ssd_chunk_bwd_states: the forward and reverse state passing over chunks
 *    (burn-mamba combined_backward's K1..K4 recompute and the K4 backward with
 *    the BLUE state gradient).  Writes d_s0 and leaves the chunk-input states
 *    and the chunk-output state gradients in the workspace.
 *  - ssd_chunk_bwd_grads: the per-chunk BLUE / ORANGE / K3 / K2 / K1 backwards
 *    and the Mamba-2 chain, reading the states the previous call left in the
 *    workspace.  The workspace must not be modified in between.
 * Arguments mean what they mean for ssd_chunk_bwd, with the same shape limits
 * and the same alignment (the big tensors 16-byte aligned, the workspace 256). */
ssmvjp_status ssd_chunk_bwd_states(const ssmvjp_ssd_desc* desc,
                                   const void* x_or_v, const float* dt_or_da, const float* A,
                                   const void* B, const void* C, const float* s0,
                                   const void* dy, const float* ds_final, float* d_s0,
                                   void* workspace, size_t workspace_bytes, void* stream);
ssmvjp_status ssd_chunk_bwd_grads(const ssmvjp_ssd_desc* desc,
                                  const void* x_or_v, const float* dt_or_da, const float* A,
                                  const void* B, const void* C, const void* dy,
                                  void* dx_or_dv, float* d_dt_or_dda, void* dB, void* dC,
                                  void* workspace, size_t workspace_bytes, void* stream);

/* ssd_chunk_bwd without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  The workspace is a device array of
 * SSMVJP_NOALLOC_SCRATCH_BYTES (96 MiB) that the library owns: each device
 * holds its own copy from the first call on that device until the process
 * ends.  The call allocates nothing (no hipMalloc, no hipFree); the caller
 * still passes every input and output.  Arguments, layouts, limits, alignment
 * and results are exactly those of ssd_chunk_bwd; a shape whose
 * ssd_chunk_bwd_workspace size exceeds SSMVJP_NOALLOC_SCRATCH_BYTES returns
 * SSMVJP_EWORKSPACE before anything is enqueued (the Mamba-2 head shape
 * H = 32, P = 64, N = 128 in bf16 fits up to b*T = 4096 tokens, e.g. one
 * sequence of 4096).  Every call on one device shares that device's array:
 * calls whose work overlaps on one device (other streams, other host threads)
 * race and must be serialised by the caller. */
#define SSMVJP_NOALLOC_SCRATCH_BYTES (96u << 20)
ssmvjp_status ssd_chunk_bwd_noalloc(const ssmvjp_ssd_desc* desc,
                                    const void* x_or_v, const float* dt_or_da, const float* A,
                                    const void* B, const void* C, const float* s0,
                                    const void* dy, const float* ds_final,
                                    void* dx_or_dv, float* d_dt_or_dda, void* dB, void* dC, float* d_s0,
                                    void* stream);

/* ------------------------------------------------------------------------ */
/* ssd_chunk_fwd: chunked SSD forward (the step before the backward)         */
/* ------------------------------------------------------------------------ */

/* The forward scan in the chunked SSD form of burn-mamba's chunked forward
 * (K1 chunk cumsum, K2 C.B^T, K3 intra-chunk state, K4 state passing, K5
 * output = BLUE inter-chunk term + ORANGE causal intra-chunk term): returns
 * y and the final state s_{T-1} (s0 when T = 0).
 *   Inputs as for ssd_chunk_bwd (FORM_MAMBA2: x, dt, A; FORM_RAW: v, da).
 *   y like x_or_v ([b,T,H,P] or [b,T,M,H,P], dtype); s_final [b,H,P,N] f32
 *   (NULL: not written); s0 NULL = zeros.
 * The running state of each (batch, head) stays on chip; with bf16 the
 * workspace holds the scores C.B^T of every chunk (from ssd_chunk_fwd_workspace;
 * none with float32).  The kernel walks chunks of chunk_len steps when
 * chunk_len * M <= 64, else of 64 / M steps; the results do not depend on the
 * chunk length apart from rounding.
 * Constraints (SSMVJP_EUNSUPPORTED otherwise): P % 16 == 0, N % 16 == 0,
 * N <= 128, M <= 64.  x_or_v, B, C and y 16-byte aligned. */
ssmvjp_status ssd_chunk_fwd_workspace(const ssmvjp_ssd_desc* desc, size_t* bytes);
ssmvjp_status ssd_chunk_fwd(const ssmvjp_ssd_desc* desc,
                            const void* x_or_v, const float* dt_or_da, const float* A,
                            const void* B, const void* C, const float* s0,
                            void* y, float* s_final,
                            void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* delta_rule_bwd: KDA gated delta rule backward                             */
/* ------------------------------------------------------------------------ */

typedef struct {
  int64_t batch, seqlen, nqk_heads, nv_heads, dk, dv; /* b, T, H, HV, K, V */
  float scale;        /* q enters the output as scale * q */
  int32_t reserved;   /* must be 0 */
} ssmvjp_delta_desc;

ssmvjp_status delta_rule_bwd_workspace(const ssmvjp_delta_desc* desc, size_t* bytes);

/* KDA backward (all float32), K3 notes section "反向传播推导": the forward
 *   S_dec = exp(g_t) (.) S_{t-1};  r = v_t - k_t^T S_dec;  S_t = S_dec + (beta_t k_t) (x) r;
 *   o_t = (scale q_t)^T S_t
 * (F1..F6) with S_{-1} = S0, and its reverse-time backward (BPTT steps 1..5)
 * seeded with dS_final, followed by the GVA sum of dq and dk over the value
 * heads of each qk head (step 6).  The gradients are those of
 *     J = <d_o, o> + <dS_final, S_{T-1}>.
 *   q, k [b,T,H,K]   v [b,T,HV,V]   beta [b,T,HV]   g [b,T,HV,K] (log gate)
 *   S0 [b,HV,K,V] (NULL = zeros)   d_o [b,T,HV,V]   dS_final [b,HV,K,V] (NULL = zeros)
 * Outputs: dq, dk [b,T,H,K]   dv [b,T,HV,V]   dg [b,T,HV,K]   dbeta [b,T,HV]
 *   dS0 [b,HV,K,V] (NULL = not written).
 * Value head hv reads qk head hv / (HV/H).
 * Constraints: HV % H == 0 (SSMVJP_EINVAL otherwise); K == 128 and V a
 * multiple of 32 (SSMVJP_EUNSUPPORTED otherwise).  Every pointer must be
 * 16-byte aligned.  T = 0 writes dS0 = dS_final only. */
ssmvjp_status delta_rule_bwd(const ssmvjp_delta_desc* desc,
                             const float* q, const float* k, const float* v, const float* beta,
                             const float* g, const float* S0, const float* d_o, const float* dS_final,
                             float* dq, float* dk, float* dv, float* dg, float* dbeta, float* dS0,
                             void* workspace, size_t workspace_bytes, void* stream);

/* The three stages of delta_rule_bwd as separate calls, for callers that
 * schedule or time them apart.  `stages` is a non-empty bit mask of
 *  - SSMVJP_DELTA_CKPT:   forward walk that leaves the state at the start of
 *                         every checkpoint segment in the workspace;
 *  - SSMVJP_DELTA_BWD:    reverse walk (recompute from the checkpoints, BPTT
 *                         steps 1..5): writes dv and dS0 and leaves per-slice
 *                         partial sums of the per-key outputs in the workspace;
 *  - SSMVJP_DELTA_REDUCE: slice sums and the GVA sum: writes dq, dk, dg, dbeta.
 * The stages run in that order; calls for the three stages in order on one
 * stream, with the same descriptor, arguments and workspace, are exactly
 * delta_rule_bwd (the workspace must not be modified in between).  Arguments
 * mean what they mean for delta_rule_bwd and are validated the same way. */
enum { SSMVJP_DELTA_CKPT = 1, SSMVJP_DELTA_BWD = 2, SSMVJP_DELTA_REDUCE = 4, SSMVJP_DELTA_ALL = 7 };
ssmvjp_status delta_rule_bwd_stages(const ssmvjp_delta_desc* desc, int32_t stages,
                                    const float* q, const float* k, const float* v, const float* beta,
                                    const float* g, const float* S0, const float* d_o, const float* dS_final,
                                    float* dq, float* dk, float* dv, float* dg, float* dbeta, float* dS0,
                                    void* workspace, size_t workspace_bytes, void* stream);

/* Human-readable name of a status code (static storage). */
const char* ssmvjp_status_str(ssmvjp_status status);

/* Library version, e.g. "0.1.0" (static storage). */
const char* ssmvjp_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SSMVJP_H */
