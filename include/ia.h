/*
 * ia.h — C ABI of the Interdomain Attention (IA) token-mixer library, libia.so (gfx950).
 *
 * Sources for what is computed.  Two web pages describe the method:
 *   [summary]  "Interdomain Attention: Beyond Token-Level Key-Value Memory", paper summary
 *              page (paperlayer.ai), organised by the paper's sections;
 *   [podcast]  "Interdomain Attention: Beyond Token-Level Key-Value Memory", AI Radio episode
 *              page (montaan.com), whose "Key Components and Derivation" and "Implementation
 *              Details" paragraphs carry the derivation and the matrix form of the readout.
 *
 * The operation, per batch row b and head h (all quantities of one (b,h) slice):
 *   feature map        phi(x) = elu(x) + 1, applied elementwise to q_t and k_t   [podcast, derivation]
 *   state recurrence   U_t[m,:]   = lambda_m U_{t-1}[m,:]   + beta_m phi(k_t)     [summary §3.2]
 *                      Gam_t[m,:] = lambda_m Gam_{t-1}[m,:] + beta_m v_t          [podcast, derivation]
 *                      eta_t[m]   = lambda_m eta_{t-1}[m]   + beta_m              (a value channel of ones)
 *   readout            a_t[m] = sum_r phi(q_t)[r] U_t[m,r]   (plain transpose, no conjugate)
 *                      o_t    = Re(sum_m a_t[m] Gam_t[m,:]) / max(Re(sum_m a_t[m] eta_t[m]), clamp)
 *   This is the matrix form O = Fq U^T Gamma / Fq U^T eta with element-wise division
 *   [podcast, derivation], the states U, Gamma, eta of fixed size [summary §3.1], with M
 *   complex-diagonal modes lambda_m (S4D) [summary §3.2].  The readout at step t includes
 *   token t.  The clamp (default 1e-6) is one-sided: a negative real part is raised to it.
 *
 * Layouts (all row-major, innermost index last, no padding; ia_prefill_fwd_strided also takes
 * q, k, v with element strides):
 *   q, k        [B][N][H][F]   in_dtype (IA_F32 or IA_BF16)
 *   v           [B][N][H][Dv]  in_dtype
 *   o           [B][N][H][Dv]  out_dtype
 *   lambda,beta [H][M]         complex64: interleaved (re, im) float pairs
 *   state U     [B][H][M][F]   complex64 interleaved
 *   state Gamma [B][H][M][Dv]  complex64 interleaved
 *   state eta   [B][H][M]      complex64 interleaved
 *   decode q_t,k_t [B][H][F], v_t and o_t [B][H][Dv]
 * The state holds 2(F+Dv)M + 2M reals per (b,h): the 2(d_feat + d_h)M of [summary §D.2] plus
 * the normaliser eta.
 *
 * Conventions for every call:
 *   - All pointers except `desc`, `st` (the struct) are DEVICE pointers, 16-byte aligned.
 *   - The caller owns every buffer.  The library allocates nothing and keeps no global state.
 *   - Work is enqueued on `stream` (a hipStream_t passed as void*; NULL = the null stream);
 *     the call returns without synchronising.  Results are visible after the stream syncs.
 *   - Validation happens on the host before anything is enqueued.  On any error nothing is
 *     enqueued and no output is touched.  A launch failure returns IA_ERR_LAUNCH.  A device
 *     fault surfaces at the caller's next synchronisation, as in HIP.
 *   - No call prints, aborts or throws.
 *   - Results are bitwise reproducible run to run (no floating-point atomics).
 */
#ifndef IA_H
#define IA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  IA_OK = 0,
  IA_ERR_NULL = 1,         /* a required pointer is NULL */
  IA_ERR_SHAPE = 2,        /* a size is out of range (B,H,N,F,Dv,M <= 0, or too large) */
  IA_ERR_DTYPE = 3,        /* unknown dtype code */
  IA_ERR_ALIGN = 4,        /* a device pointer is not 16-byte aligned */
  IA_ERR_ALIAS = 5,        /* an output overlaps an input or another output */
  IA_ERR_DOMAIN = 6,       /* lambda outside the supported domain (see ia_prefill_fwd) */
  IA_ERR_UNSUPPORTED = 7,  /* a combination the library does not implement */
  IA_ERR_LAUNCH = 8,       /* the HIP runtime refused a launch */
  IA_ERR_WORKSPACE = 9     /* workspace NULL or smaller than the *_workspace_bytes query */
} ia_status;

typedef enum { IA_F32 = 0, IA_BF16 = 1 } ia_dtype;

/* Bidirectional layer: o = IA(x) + flip_t(IA(flip_t x)), each direction from a zero state and
 * normalised separately, same lambda, beta, q, k, v (the Caduceus-style genomic models of
 * [summary §5.2, §A.1] run the token mixer over the sequence and its reversal). */
#define IA_FLAG_BIDIR 1u

/* Readout without the normaliser: o = Re(phi(q) U^T Gamma), no division by Re(phi(q) U^T eta)
 * and no clamp (the practical readout that drops the denominator [summary §3.1]).  Prefill
 * (either direction) and decode. */
#define IA_FLAG_NO_DEN 2u

/* q and k already hold features: no feature map is applied (phi = identity), for callers that
 * form phi(q), phi(k) themselves.  Prefill and decode. */
#define IA_FLAG_IDENTITY_FEATURES 4u

typedef struct ia_desc {
  int B;             /* batch rows */
  int H;             /* heads */
  int N;             /* tokens (prefill); ignored by ia_decode_step */
  int F;             /* feature dim of q and k (R = d_h on the pages); multiple of 16, <= 256 */
  int Dv;            /* value dim; multiple of 16, <= 256 */
  int M;             /* complex modes; multiple of 16, <= 128 */
  /* B, H, N, F, Dv, M <= 0: IA_ERR_SHAPE.  F, Dv or M not a multiple of 16 or above the
   * maximum: IA_ERR_UNSUPPORTED. */
  int in_dtype;      /* ia_dtype of q, k, v */
  int out_dtype;     /* ia_dtype of o */
  float den_clamp;   /* lower clamp of Re(den); finite and > 0 (the method uses 1e-6), else
                        IA_ERR_DOMAIN */
  unsigned flags;    /* IA_FLAG_BIDIR | IA_FLAG_NO_DEN | IA_FLAG_IDENTITY_FEATURES, or 0; other
                        bits: IA_ERR_UNSUPPORTED */
  int chunk;         /* chunk length of the chunked prefill: 0 (= 64 [summary §A.2]), 32 or
                        64; other values: IA_ERR_UNSUPPORTED */
} ia_desc;

/* Recurrent state of all (b,h) slices; three device pointers, layouts above. */
typedef struct ia_state {
  void* U;
  void* Gamma;
  void* eta;
} ia_state;

/* Zero the state (the recurrence starts from U = Gamma = eta = 0).  Enqueues a fill kernel
 * (no memset node), so it may be captured in a graph.  Errors: IA_ERR_NULL, IA_ERR_SHAPE,
 * IA_ERR_ALIGN, IA_ERR_LAUNCH. */
ia_status ia_state_init(const ia_desc* desc, ia_state* st, void* stream);

/* Bytes of device workspace ia_prefill_fwd needs for `desc` (may be 0); 0 also if the desc
 * is invalid.  The workspace holds the per-head tables and per-segment state summaries of the
 * chunked scan, or a state for state-less fp32 calls.  Its contents need no initialisation
 * and are scratch between calls.  (The bidirectional layer accumulates its two directions in
 * o itself, in o's dtype.) */
size_t ia_prefill_workspace_bytes(const ia_desc* desc);

/* Host-side check of the mode domain for `desc` (lambda_host: [H][M] complex64 in HOST
 * memory).  lambda lives in device memory in the other calls, which therefore cannot check
 * it without a synchronisation and do not; callers that build lambda call this once.
 * IA_ERR_DOMAIN unless every 0 < |lambda| <= 1 + 1e-6 and, for bf16 inputs (the chunked MFMA
 * path, whose per-chunk decay factorises lambda^(i-j) = lambda^i lambda^(-j)),
 * |lambda|^(chunk-1) >= 2^-8 (|lambda| >= 0.916 at chunk 64, 0.836 at chunk 32).  Outside
 * that domain the chunked path stays finite but may miss the bf16 tolerance. */
ia_status ia_check_lambda(const ia_desc* desc, const void* lambda_host);

/* Causal (or, with IA_FLAG_BIDIR, bidirectional) forward of one IA layer over N tokens.
 *
 * Runs the chunkwise form of the recurrence: work inside each chunk of `chunk` tokens is done
 * as dense contractions, the state is passed across chunk boundaries, and a second pass
 * recomputes each segment from its corrected initial state [summary §3.2, §A.2].  Results
 * equal the token-by-token recurrence up to rounding and do not depend on `chunk`.
 *
 *   q, k, v    inputs, layouts above, read only.
 *   lambda     [H][M] complex64 in the domain of ia_check_lambda (not checked here).
 *   beta       [H][M] complex64 input vector of the S4D recurrence (B on the pages).
 *   st         NULL: start from zero and do not return a state.  Otherwise st->U/Gamma/eta
 *              hold the initial state on entry and the state after token N-1 on return
 *              (resume point for a later prefill or decode).  Must be NULL with BIDIR.
 *   o          [B][N][H][Dv] out_dtype, or NULL: state-only prefill that builds the decoding
 *              state and writes no outputs [summary §F.2].  o == NULL with st == NULL is an
 *              error (nothing to compute).
 *   workspace  device scratch of at least ia_prefill_workspace_bytes(desc) bytes.
 * Errors: IA_ERR_NULL, IA_ERR_SHAPE, IA_ERR_DTYPE, IA_ERR_ALIGN, IA_ERR_ALIAS (o overlapping
 * an input, lambda/beta or the state, or state buffers overlapping inputs or each other),
 * IA_ERR_DOMAIN (den_clamp), IA_ERR_UNSUPPORTED (BIDIR with st != NULL, sizes, chunk),
 * IA_ERR_WORKSPACE, IA_ERR_LAUNCH. */
ia_status ia_prefill_fwd(const ia_desc* desc,
                         const void* q, const void* k, const void* v,
                         const void* lambda, const void* beta,
                         ia_state* st, void* o,
                         void* workspace, size_t ws_bytes, void* stream);

/* ia_prefill_fwd with q, k, v in strided layouts, e.g. views of one fused projection
 * [B][N][3][H][F] (no copy needed).  strides[i] = {b, n, h} element strides of q (i = 0),
 * k (1) and v (2): element (b, n, h, x) of q lies at q + b*s[0] + n*s[1] + h*s[2] + x, the
 * feature (value) axis contiguous.  strides == NULL: the dense layouts above (this is what
 * ia_prefill_fwd does).  o, the state, lambda and beta keep their dense layouts, and the
 * workspace size is ia_prefill_workspace_bytes(desc) as before.  Ownership and aliasing as
 * for ia_prefill_fwd, with the inputs' extents taken from the strides.
 * Errors, besides those of ia_prefill_fwd: IA_ERR_SHAPE (a stride <= 0), IA_ERR_ALIGN (a
 * stride times the element size not a multiple of 16 bytes), IA_ERR_UNSUPPORTED (q and k
 * with different strides; with bf16 inputs, 64 token rows of q/k or of v spanning more than
 * 1 GiB). */
ia_status ia_prefill_fwd_strided(const ia_desc* desc,
                                 const void* q, const void* k, const void* v,
                                 const long long strides[3][3],
                                 const void* lambda, const void* beta,
                                 ia_state* st, void* o,
                                 void* workspace, size_t ws_bytes, void* stream);

/* Profiling variant of ia_prefill_fwd: identical work and results, and in addition, for its
 * i-th kernel launch (i < max_launches, in launch order), records events[2i] before and
 * events[2i+1] after the kernel on `stream` and stores the kernel's kind in kinds[i]
 * (2 decay tables, launched on their own only when a sequence is one segment; 3 segment end
 * states, whose launch also computes the tables when there are several segments; 4 segment
 * carry; 5 chunked prefill with outputs; 0 zero fill; 1 token-sequential prefill).  events: 2*max_launches hipEvent_t handles
 * created by the caller.  *n_launches receives the number of launches recorded.  Errors: as
 * ia_prefill_fwd, and IA_ERR_NULL for missing events/kinds/n_launches. */
ia_status ia_prefill_fwd_profiled(const ia_desc* desc,
                                  const void* q, const void* k, const void* v,
                                  const void* lambda, const void* beta,
                                  ia_state* st, void* o,
                                  void* workspace, size_t ws_bytes, void* stream,
                                  void** events, int* kinds, int max_launches,
                                  int* n_launches);

/* One autoregressive step for every (b,h): updates the state in place with token t and
 * writes o_t (the recurrence and readout above with N = 1).  The per-step work and the
 * state are independent of how many tokens came before [summary §3.2, §F.3].
 *   q_t, k_t  [B][H][F] in_dtype;  v_t [B][H][Dv] in_dtype;  o_t [B][H][Dv] out_dtype.
 *   st        required; updated in place.
 * desc->N, desc->chunk and IA_FLAG_BIDIR are ignored (BIDIR has no causal decode: error
 * IA_ERR_UNSUPPORTED if set).  No workspace.  Errors as ia_prefill_fwd. */
ia_status ia_decode_step(const ia_desc* desc,
                         const void* q_t, const void* k_t, const void* v_t,
                         const void* lambda, const void* beta,
                         ia_state* st, void* o_t, void* stream);

/* Workspace bytes ia_prefill_bwd needs for this descriptor: state checkpoints every 32 tokens
 * (B*H*ceil(N/32)*M*(F+Dv+1) complex64), per-token partial denominators (B*H*N*M/2 complex64),
 * per-mode-group gradient rows (M/16 * B*H*N*(2F+Dv) float), per-slice lambda/beta gradients,
 * the recompute's a = phi(q) U^T per token (B*H*N*M complex64) and, when a long sequence is
 * cut into segments, their start states and entering adjoints, each region 256-byte aligned.
 * 0 on an invalid descriptor. */
size_t ia_prefill_bwd_workspace_bytes(const ia_desc* desc);

/* Gradients of the causal layer (ia_prefill_fwd's outputs o) for a real loss L, given
 * dO = dL/do: reverse-mode differentiation of the recurrence and readout above, as the
 * training step of [summary §G] needs.  The states are recomputed from st0 (not read from a
 * forward call), checkpointed every 32 tokens, and rebuilt backward inside each interval by
 * U_{t-1} = (U_t - beta phi(k_t)) / lambda, in fp32.
 *   q, k, v, lambda, beta   as in ia_prefill_fwd (dense layout, in_dtype).
 *   st0      initial state the forward started from, or NULL for zeros; read only.
 *   dO       [B][N][H][Dv] out_dtype.
 *   dq, dk   [B][N][H][F] in_dtype; dv [B][N][H][Dv] in_dtype (overwritten).
 *   dlambda, dbeta  [H][M] complex64: dL/dRe + i dL/dIm, summed over the batch.
 *   dst0     receives dL/d(st0) in the ia_state layout, or NULL.
 * Readout gradient: dnum = dO / c and, where den >= den_clamp (the branch the forward takes
 * for den itself), dden = -sum_j dO_j num_j / c^2, with c = max(den, den_clamp); below the
 * clamp den has no gradient.  IA_FLAG_NO_DEN: dnum = dO, dden = 0.  IA_FLAG_IDENTITY_FEATURES:
 * phi' = 1.  IA_FLAG_BIDIR: gradients of o = IA(x) + flip_t(IA(flip_t x)) (both directions from
 * zero), the reversed walk's added onto the forward's; st0 and dst0 must then be NULL
 * (IA_ERR_UNSUPPORTED otherwise).
 * Accuracy: the rebuild grows fp32 rounding by at most |lambda|^-31 inside an interval; for
 * |lambda| >= 0.9 that is below 30x (an S4D-Lin lambda = exp(dt(-1/2 + i pi m)) with
 * dt <= 0.1 has |lambda| >= 0.95).
 * lambda = 0 gives non-finite gradients.
 * Errors: as ia_prefill_fwd (IA_ERR_NULL for a missing required pointer, IA_ERR_ALIGN for
 * pointers not 16-byte aligned, IA_ERR_ALIAS when an output overlaps an input, another
 * output or the workspace, IA_ERR_WORKSPACE when ws_bytes is below
 * ia_prefill_bwd_workspace_bytes); nothing is launched on error. */
ia_status ia_prefill_bwd(const ia_desc* desc,
                         const void* q, const void* k, const void* v,
                         const void* lambda, const void* beta,
                         const ia_state* st0, const void* dO,
                         void* dq, void* dk, void* dv, void* dlambda, void* dbeta,
                         ia_state* dst0, void* workspace, size_t ws_bytes, void* stream);

/* Readout matrix variants.  A learned complex M x M matrix R per head mixes the modes of
 * a = phi(q_t) U^T before both readouts (the full readout matrix listed with the practical
 * layer's dimensions [summary §A.3], the M^2 term of the decode cost [summary §3.2]):
 *   a'[n] = sum_m a[m] R[m][n],  o_t = Re(a' Gamma) / max(Re(a' eta), den_clamp)
 * (or Re(a' Gamma) with IA_FLAG_NO_DEN).  R = identity gives the plain layer.
 *   readout  [H][M][M] complex64 (row m, column n), device, read only; NULL: IA_ERR_NULL.
 * Both run the token-sequential fp32 kernels (bf16 inputs included): the chunked factorisation
 * keeps modes separate.  Other arguments, layouts and errors as ia_prefill_fwd /
 * ia_decode_step; readout must be 16-byte aligned and must not overlap an output. */

/* Workspace bytes ia_prefill_fwd_readout needs at most: one state,
 * B*H*M*(F+Dv+1) complex64 rounded up to 256 bytes (used when st is NULL or IA_FLAG_BIDIR is
 * set; otherwise the workspace may be NULL).  0 on an invalid descriptor. */
size_t ia_prefill_readout_workspace_bytes(const ia_desc* desc);

ia_status ia_prefill_fwd_readout(const ia_desc* desc,
                                 const void* q, const void* k, const void* v,
                                 const void* lambda, const void* beta, const void* readout,
                                 ia_state* st, void* o,
                                 void* workspace, size_t ws_bytes, void* stream);

ia_status ia_decode_step_readout(const ia_desc* desc,
                                 const void* q_t, const void* k_t, const void* v_t,
                                 const void* lambda, const void* beta, const void* readout,
                                 ia_state* st, void* o_t, void* stream);

/* Static string naming a status code. */
const char* ia_status_string(ia_status s);

/* Static string: the HIP runtime's text for the error behind the calling thread's most recent
 * IA_ERR_LAUNCH ("no launch error" if there was none).  The one piece of per-thread state
 * the library keeps. */
const char* ia_last_launch_error(void);

#ifdef __cplusplus
}
#endif

#endif /* IA_H */
