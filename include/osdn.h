/*
 * osdn.h -- C ABI of the OSDN forward library (libosdn.so, AMD gfx950).
 *
 * Online Scaled DeltaNet (OSDN) is the delta rule with a diagonal
 * preconditioner d_t on the write side, learned online by descent on a
 * closed-form hypergradient surrogate.  Source of every definition below: the
 * gist.science technical summary of "OSDN: Improving Delta Rule with Provable
 * Online Preconditioning in Linear Attention" (arXiv 2605.13473), cited as
 * [summary §N].
 *
 * Per (batch b, head h), tokens t = 0..T-1, keys/queries in R^dk, values in
 * R^dv, state S in R^{dv x dk}, preconditioner d in R^dk:
 *   kt_t    = d_t (.) k_t                                   [summary §2.1]
 *   S_t     = S_{t-1} + beta_t (v_t - S_{t-1} k_t) kt_t^T    [summary §2.1]
 *   o_t     = S_t q_t           (readout after the write; the pages give none)
 *   a_t     = <d_t, k_t (.) k_t>,  rho_t = (1 - beta_t a_t)^2  [summary §2.2, §3]
 *   d_{t+1} = r_t d_t + eta beta_t (1 - beta_t a_t) (k_t (.) k_t) / ||k_t||^2
 *             (descent on the surrogate of [summary §2.2]; r_t = 1 without the
 *              APF retention gate of [summary §2.3]; the step is 0 when k_t = 0)
 * Phase 1 (osdn_precond_scan) is the O(dk) walk over the key stream that
 * produces kt; phase 2 (osdn_chunk_fwd) is the chunkwise delta-rule pass with
 * kt in place of k in the chunk gram, the intra-chunk scores and the state
 * update [summary §2.2, two-phase implementation].  osdn_forward does both.
 *
 * Conventions shared by every entry point
 *  - Layout: every tensor is dense, row-major, contiguous:
 *      q, k, kt  [B][H][T][dk]     v, o [B][H][T][dv]
 *      beta, r   [B][H][T]  fp32   d0, d_final [B][H][dk] fp32
 *      S0, S_final [B][H][dv][dk] fp32 (row j of S is value channel j)
 *  - dtype (q, k, v, kt, o): OSDN_BF16 (bfloat16) or OSDN_F32.  beta, r, d and
 *    S are always fp32; arithmetic is fp32 on the device.
 *  - Pointers are device pointers (any memory the GPU can address) except where
 *    stated.  The caller owns every buffer; the library never allocates, frees
 *    or synchronises on these calls.  Outputs must not overlap inputs.
 *  - stream is a hipStream_t (NULL = the default stream).  Work is enqueued on
 *    it and the call returns; device faults surface at the caller's next sync.
 *  - Sizes: B, H, T >= 0 (any zero makes the call a no-op apart from copying
 *    the initial state to the final-state outputs when T = 0); dk, dv in
 *    {16, 32, 64, 128}; chunk in {16, 32, 64}.  T need not be a multiple of
 *    chunk (the last chunk is short).
 *  - Errors: every argument is checked before anything is enqueued; on error
 *    nothing is enqueued and a negative OSDN_ERR_* code is returned.
 *  - State gate (osdn_chunk_fwd, osdn_forward, osdn_step): alpha [B][H][T]
 *    fp32, or NULL for none.  The pages run OSDN on a Gated DeltaNet backbone
 *    [summary §4] without printing its update; the plainest reading, used
 *    here, decays the state before each token's read and write:
 *      S_t = alpha_t S_{t-1} + beta_t (v_t - alpha_t S_{t-1} k_t) kt_t^T.
 *    alpha acts on S only; the preconditioner walk does not see it.  alpha = 1
 *    gives the ungated results; alpha in [0, 1] is the intended range (decays
 *    below 2^-126 over a chunk are flushed to zero).
 *  - Per-channel gate (osdn_chunk_fwd, osdn_forward, osdn_step with
 *    OSDN_GATE_PER_CHANNEL): alpha is [B][H][T][dk] fp32 (step: [B][H][dk]), one gate per key
 *    dimension.  The pages also run OSDN on a Kimi Delta Attention backbone
 *    [summary §4] without printing its update; the reading used here
 *    generalises the scalar gate:
 *      S_t = S_{t-1} D_t + beta_t (v_t - S_{t-1} D_t k_t) kt_t^T,  D_t = diag(alpha_t),
 *    i.e. column i of S (key dimension i) decays by alpha_t[i].
 *  - Results are deterministic run to run (no floating-point atomics).
 *  - Non-finite inputs propagate; they are not checked.
 */
#ifndef OSDN_H
#define OSDN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define OSDN_OK 0
#define OSDN_ERR_NULL (-1)        /* a required pointer is NULL */
#define OSDN_ERR_SHAPE (-2)       /* a size is negative or the sizes overflow */
#define OSDN_ERR_UNSUPPORTED (-3) /* dtype, dk, dv or chunk outside the supported set */
#define OSDN_ERR_WORKSPACE (-4)   /* workspace NULL or smaller than required */
#define OSDN_ERR_HIP (-5)         /* the HIP runtime rejected a launch */
#define OSDN_ERR_TOO_LARGE (-6)   /* osdn_forward_noalloc: more scratch than its fixed array holds */

/* Size in bytes of osdn_forward_noalloc's fixed scratch array (one per GPU). */
#define OSDN_NOALLOC_MAX_BYTES ((size_t)64 << 20)

#define OSDN_BF16 0
#define OSDN_F32 1

/* osdn_forward flag: run the plain delta rule (kt = k, [summary §1]); d0, r and
 * eta are ignored, d_final is not written, rho_t = (1 - beta_t ||k_t||^2)^2. */
#define OSDN_PRECOND_OFF 1u

/* Input transforms done inside the kernels as the inputs are staged, so no
 * separate elementwise pass over them is needed (osdn_forward, osdn_step):
 *   OSDN_NORM_QK      q and k arrive unnormalised; every q_t and k_t is divided
 *                     by its L2 norm (fp32; a zero vector stays zero)
 *   OSDN_GATE_LOGITS  beta and r arrive as logits; the kernels use
 *                     1 / (1 + exp(-x)).  alpha is not transformed.
 * The measured workloads apply exactly these transforms to their draws.
 * osdn_forward takes them on the multi-launch path (bf16, dk = dv = 128,
 * chunk 64, enough workspace) and on the two-phase path; where the
 * single fused kernel would run it returns OSDN_ERR_UNSUPPORTED. */
#define OSDN_NORM_QK 2u
#define OSDN_GATE_LOGITS 4u

/* osdn_chunk_fwd, osdn_forward, osdn_step flag: alpha holds one gate per key
 * dimension (the per-channel gate above; required with this flag).  Given the
 * workspace osdn_forward_workspace_bytes (osdn_chunk_fwd_workspace_bytes)
 * reports for these flags, the matrix-core shapes run the multi-launch
 * pipeline; otherwise the forward runs the two-phase path (which needs the
 * write-key buffer) and osdn_chunk_fwd the vector chunk kernel.  The single
 * fused kernel does not take it. */
#define OSDN_GATE_PER_CHANNEL 8u

/*
 * Phase 1: the preconditioner scan over the key stream [summary §2.2 phase 1,
 * §2.3 APF].
 *   k         [B,H,T,dk] dtype   keys (required if T > 0)
 *   beta      [B,H,T]    fp32    write gates (required if T > 0)
 *   r         [B,H,T]    fp32    APF retention gates; NULL means r = 1
 *   d0        [B,H,dk]   fp32    initial preconditioner; NULL means all ones
 *   eta                          meta step size
 *   k_tilde   [B,H,T,dk] dtype   out: kt_t = d_t (.) k_t, rounded to dtype
 *                                (required if T > 0)
 *   d_final   [B,H,dk]   fp32    out: d_T (optional, NULL to skip)
 *   d_all     [B,H,T,dk] fp32    out: d_t, the value used at token t (optional)
 *   log_ratio [B,H,T]    fp32    out: log rho_t (optional; -inf where rho_t = 0)
 *   workspace  optional device scratch.  With at least
 *              osdn_precond_scan_workspace_bytes(...) bytes (positive for bf16
 *              keys with dk = 128) the walk runs in one launch: some
 *              workgroups prepare the d-independent part of every chunk (the
 *              (I + M)^-1 of the chunked walk) while one workgroup per (b,h)
 *              walks the chunks as they become ready, and the preparing
 *              workgroups then write the keys of each chunk the walk has
 *              passed (handed over through two 8-byte flags per chunk at the
 *              end of the workspace).  When B*H exceeds half the device's
 *              compute units, or with 16 * B * H * ceil(T / 64) bytes less,
 *              the three run as launches of their own.  NULL, or less,
 *              selects a single kernel per (b,h).  Results are bitwise the
 *              same on all the multi-launch forms.
 */
int osdn_precond_scan(const void *k, const float *beta, const float *r, const float *d0,
                      float eta, int B, int H, int T, int dk, int dtype,
                      void *k_tilde, float *d_final, float *d_all, float *log_ratio,
                      void *workspace, size_t workspace_bytes, void *stream);

/* Scratch bytes that select osdn_precond_scan's fastest multi-launch walk (0
 * when no such path exists for these arguments); (size_t)-1 if they are
 * invalid. */
size_t osdn_precond_scan_workspace_bytes(int B, int H, int T, int dk, int dtype);

/*
 * Phase 2: the chunkwise delta-rule pass with a given write key kt
 * [summary §2.1: kt replaces k in the chunk gram and intra-chunk scores].
 * Within a chunk with entry state S, A = strict_lower(diag(beta) K Kt^T),
 * (I + A) X = diag(beta) (V - K S^T), O = Q S^T + lower(Q Kt^T) X,
 * S <- S + X^T Kt.  Same result as the token recurrence up to rounding.
 *   q, k      [B,H,T,dk] dtype   queries; read-side keys (required if T > 0)
 *   k_tilde   [B,H,T,dk] dtype   write-side keys (required if T > 0)
 *   v         [B,H,T,dv] dtype   values (required if T > 0)
 *   beta      [B,H,T]    fp32    (required if T > 0)
 *   alpha     [B,H,T]    fp32    state gate; NULL means none.  With it, gamma_t
 *                                the product of alpha over the chunk up to t:
 *                                A_ts and the scores take gamma_t / gamma_s,
 *                                K S^T and Q S^T take gamma_t, and
 *                                S <- gamma_L S + sum_s (gamma_L / gamma_s) x_s kt_s^T
 *   S0        [B,H,dv,dk] fp32   initial state; NULL means zero
 *   chunk                        chunk length
 *   o         [B,H,T,dv] dtype   out: o_t = S_t q_t (required if T > 0)
 *   S_final   [B,H,dv,dk] fp32   out: S_T (optional)
 *   flags      0 or OSDN_GATE_PER_CHANNEL (alpha [B,H,T,dk], one gate per key
 *              dimension, as for osdn_forward); the input transforms are not
 *              taken here (OSDN_ERR_UNSUPPORTED)
 *   workspace  optional device scratch.  When it holds at least
 *              osdn_chunk_fwd_workspace_bytes(...) bytes (a positive number),
 *              the per-chunk work runs chunk-parallel ahead of the sequential
 *              pass (faster); NULL selects the single-kernel pass (the vector
 *              chunk kernel with the per-channel gate).
 */
int osdn_chunk_fwd(const void *q, const void *k, const void *k_tilde, const void *v,
                   const float *beta, const float *alpha, const float *S0, int B, int H,
                   int T, int dk, int dv, int chunk, int dtype, unsigned flags, void *o,
                   float *S_final, void *workspace, size_t workspace_bytes, void *stream);

/* Scratch bytes that let osdn_chunk_fwd run its chunk-parallel path for these
 * flags (0 when no path for these arguments uses scratch); (size_t)-1 if the
 * arguments are invalid. */
size_t osdn_chunk_fwd_workspace_bytes(int B, int H, int T, int dk, int dv, int chunk, int dtype,
                                      unsigned flags);

/*
 * Both phases end to end [summary §2.2 two-phase implementation].
 *   q, k, v, beta, r, alpha, d0, S0, eta   as above; with OSDN_PRECOND_OFF and
 *                  alpha this is Gated DeltaNet itself
 *   flags          OSDN_PRECOND_OFF, OSDN_NORM_QK, OSDN_GATE_LOGITS,
 *                  OSDN_GATE_PER_CHANNEL, or'd
 *   o              [B,H,T,dv] dtype out (required if T > 0)
 *   S_final        [B,H,dv,dk] fp32 out (optional)
 *   d_final        [B,H,dk] fp32 out (optional)
 *   log_ratio_sum  [B,H] fp32 out: sum_t log rho_t (optional) -- the per-head
 *                  log of the product of token-local residual ratios of
 *                  [summary §3]; its mean over tokens gives log q_geo [summary §4.2]
 *   workspace      device scratch.  With at least osdn_forward_workspace_bytes(...)
 *                  bytes the fastest path runs; for bf16, dk = dv = 128, chunk 64
 *                  that is a pipeline of launches (walk, chunk-parallel pass,
 *                  sequential state pass; the walk and the preparation of its
 *                  chunks share one launch when B*H is at most half the
 *                  device's compute units).  With at most 32 heads (B*H) and
 *                  neither a state gate nor OSDN_NORM_QK, on a device with at
 *                  least 8 B*H compute units, the whole forward runs as one
 *                  launch; the scratch then holds the walk's records apart
 *                  (17.3 KiB more per chunk).  Less scratch (or
 *                  NULL) selects the single fused kernel.  Other shapes need the
 *                  scratch: the walk hands kt to the chunk pass through it, in
 *                  fp32 whatever the data type (a bf16 kt would cost up to 2^-9
 *                  relative per element before the chunk pass), followed for
 *                  bf16 keys with dk = 128 by the chunked walk's records.
 *
 * The path follows from the shapes and the scratch alone, silently;
 * osdn_forward_path names it.  What each costs, measured on MI355X for
 * B = 4, H = 16, T = 4096, dk = dv = 128, chunk 64, bf16:
 *   "split"      about 0.27 ms (the scratch of osdn_forward_workspace_bytes:
 *                about 137 MB there, 32.75 KiB per (b, h, 64-token chunk))
 *   "fused"      about 0.5 ms: one kernel redoes each chunk's preparation for
 *                every 32-channel tile of the values
 *   "two-phase"  for the per-channel gate (OSDN_GATE_PER_CHANNEL) with less
 *                scratch than "split" needs (65.25 KiB per chunk): about 22 ms,
 *                some 50 times the 0.45 ms of its split path, because the chunk
 *                pass then runs on vector kernels; give such calls the scratch.
 *                Other shapes run only here (vector kernels, fp32 kt).
 */
int osdn_forward(const void *q, const void *k, const void *v, const float *beta,
                 const float *r, const float *alpha, const float *d0, const float *S0,
                 float eta, int B, int H, int T, int dk, int dv, int chunk, int dtype,
                 unsigned flags, void *o, float *S_final, float *d_final,
                 float *log_ratio_sum, void *workspace, size_t workspace_bytes, void *stream);

/*
 * One decoding step with persistent state [summary §2.1-§2.3, §3; the
 * efficiency claims concern this per-token update]: for one token per (b,h),
 *   kt = d (.) k,  S <- alpha S (if gated),  S <- S + beta (v - S k) kt^T,
 *   o = S q  (after the write),
 *   rho = (1 - beta <d, k (.) k>)^2,
 *   d <- r d + eta beta (1 - beta <d, k (.) k>) (k (.) k) / ||k||^2  (0 if k = 0).
 * Running it for t = 0..T-1 gives the same o, S and d as osdn_forward over the
 * T tokens, up to rounding.
 *   q, k      [B,H,dk] dtype     query and key of the token (required)
 *   v         [B,H,dv] dtype     value (required)
 *   beta      [B,H]    fp32      write gate (required)
 *   r         [B,H]    fp32      APF retention gate; NULL means r = 1
 *   alpha     [B,H]    fp32      state gate; NULL means none
 *   S         [B,H,dv,dk] fp32   state, read and updated in place (required)
 *   d         [B,H,dk] fp32      preconditioner, read and updated in place (required)
 *   o         [B,H,dv] dtype     out: the readout (required)
 *   log_ratio [B,H]    fp32      out: log rho (optional)
 *   flags     0, OSDN_NORM_QK, OSDN_GATE_LOGITS, OSDN_GATE_PER_CHANNEL, or'd
 * S, d and o must not overlap each other or the inputs.
 */
int osdn_step(const void *q, const void *k, const void *v, const float *beta, const float *r,
              const float *alpha, float eta, int B, int H, int dk, int dv, int dtype,
              unsigned flags, float *S, float *d, void *o, float *log_ratio, void *stream);

/*
 * osdn_forward for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.  Same
 * arguments, kernels and results as osdn_forward given the workspace of
 * osdn_forward_workspace_bytes, but the scratch is a fixed array of
 * OSDN_NOALLOC_MAX_BYTES (64 MiB) that the library keeps in
 * device memory, one per GPU, for the life of the process: nothing is
 * allocated, freed or cleared on the call.  A call needing more (more than
 * about 2,000 (b, h, 64-token chunk) triples on the split pipeline, e.g. 16
 * heads x 8,000 tokens) returns OSDN_ERR_TOO_LARGE before anything is
 * enqueued.  The first call on a device resolves the array's address there
 * (hipGetSymbolAddress); the stream must belong to the current device.  Every
 * call on one GPU uses the same array: calls that overlap on that GPU (other
 * streams, other host threads) race and must be serialised by the caller.
 */
int osdn_forward_noalloc(const void *q, const void *k, const void *v, const float *beta,
                         const float *r, const float *alpha, const float *d0, const float *S0,
                         float eta, int B, int H, int T, int dk, int dv, int chunk, int dtype,
                         unsigned flags, void *o, float *S_final, float *d_final,
                         float *log_ratio_sum, void *stream);

/* Scratch bytes that select osdn_forward's fastest path for these arguments
 * (required on the two-phase path, optional on the matrix-core shapes);
 * (size_t)-1 if the arguments are invalid. */
size_t osdn_forward_workspace_bytes(int B, int H, int T, int dk, int dv, int chunk, int dtype,
                                    unsigned flags);

/* Static, NUL-terminated description of a status code (host pointer). */
const char *osdn_status_str(int status);

/* Name of the kernel family osdn_forward would launch for these arguments and
 * the workspace size (every family takes the state gate): "split"
 * (the multi-launch pipeline), "fused" (one kernel), "two-phase", "none", or
 * "unsupported" (input transforms where only the fused kernel could run);
 * static host string, "invalid" on bad arguments.  Lets callers and tests
 * know which path they exercised. */
const char *osdn_forward_path(int B, int H, int T, int dk, int dv, int chunk, int dtype,
                              unsigned flags, size_t workspace_bytes);

#ifdef __cplusplus
}
#endif

#endif /* OSDN_H */
