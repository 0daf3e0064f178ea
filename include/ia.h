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
 *   - The caller owns every buffer.  The library allocates nothing at run time.  Its state:
 *     per thread, the text behind the last IA_ERR_LAUNCH (ia_last_launch_error) and, for the
 *     duration of an ia_prefill_fwd_profiled call, a pointer to that call's event list; per
 *     device, the fixed workspace array of ia_prefill_fwd_noalloc (part of the loaded code).
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

/* ia_prefill_bwd only (ignored elsewhere): which of its two implementations runs.  Without
 * either flag the chunked kernels run where they exist (F == Dv in {32, 64, 128}) unless the
 * (b,h) slices and mode groups are so few that the token-sequential sweeps would cut each
 * sequence into more than eight segments; IA_FLAG_SEQUENTIAL_BWD forces the token-sequential
 * kernels, IA_FLAG_CHUNKED_BWD the chunked ones (IA_ERR_UNSUPPORTED on other shapes, and with
 * both flags).  Both give the same gradients up to fp32 rounding. */
#define IA_FLAG_SEQUENTIAL_BWD 8u
#define IA_FLAG_CHUNKED_BWD 16u

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
  unsigned flags;    /* IA_FLAG_BIDIR | IA_FLAG_NO_DEN | IA_FLAG_IDENTITY_FEATURES |
                        IA_FLAG_SEQUENTIAL_BWD | IA_FLAG_CHUNKED_BWD, or 0; other bits:
                        IA_ERR_UNSUPPORTED */
  int chunk;         /* chunk length of the chunked prefill: 0 (= 64 [summary §A.2]), 32 or
                        64; other values: IA_ERR_UNSUPPORTED */
} ia_desc;

/* Recurrent state of all (b,h) slices; three device pointers, layouts above. */
typedef struct ia_state {
  void* U;
  void* Gamma;
  void* eta;
} ia_state;

/* Zero the state: U = Gamma = eta = 0, the state of the recurrence before its first token
 * (the fixed-size memory U, Gamma, eta of [summary §3.1], updated token by token by the S4D
 * recurrence of [summary §3.2]; a chunked prefill that builds only this state [summary §F.2]
 * or a decode step then continue from it).  Enqueues a fill kernel (no memset node), so it
 * may be captured in a graph.  Errors: IA_ERR_NULL, IA_ERR_SHAPE, IA_ERR_ALIGN,
 * IA_ERR_LAUNCH. */
ia_status ia_state_init(const ia_desc* desc, ia_state* st, void* stream);

/* Bytes of device workspace ia_prefill_fwd needs for `desc` (may be 0); 0 also if the desc
 * is invalid or has no kernel (bf16 shapes outside the chunked path).  The workspace holds the
 * per-head tables, the per-segment state summaries and one state (the caller's initial state
 * copied there when several segments run, or the fp32 route's working state) of the chunked
 * scan (for IA_FLAG_BIDIR a second set of summaries, the reverse walk's), or, for the fp32
 * token-sequential path, a state (state-less or bidirectional calls) and the slots of its
 * sequence segments (see below).  Its contents need no initialisation and are scratch between
 * calls.  (The bidirectional layer accumulates its two directions in o itself, in o's dtype.)
 *
 * Sequence segments of the token-sequential path (F, Dv in {32, 64, 128}): when the B*H slices
 * leave compute units idle, each sequence is cut into up to CUs / (B*H) segments of at least
 * 64 tokens, each walked by its own workgroup from its start state (a state-only pass from
 * zero per segment, then a carry of the starts).  The query returns the bytes of the full
 * count: per segment one state of all slices, B*H*M*(F+Dv+1) complex64, plus B*H*M complex64
 * of decay products; a call runs as many segments as its ws_bytes holds, down to one (then
 * the workspace may be NULL when st is given and IA_FLAG_BIDIR is not set).  The results
 * agree with one walk to rounding. */
size_t ia_prefill_workspace_bytes(const ia_desc* desc);

/* Host-side check of the modes for `desc` (lambda_host: [H][M] complex64 in HOST memory).
 * Returns IA_ERR_DOMAIN unless every 0 < |lambda| <= 1 + 1e-6 (stable S4D modes
 * [summary §3.2]; the prefill and decode calls do not reject other values, which they cannot
 * see without a synchronisation: they compute the recurrence as written).
 * fp32_heads (may be NULL) receives, for bf16 inputs, the number of heads that the chunked
 * MFMA prefill runs on the fp32 route instead (0 for fp32 inputs).  A head takes that route
 * when any of its modes has |lambda| outside (0, 1 + 1e-6], |lambda|^(chunk-1) < 2^-8 (the
 * chunk's decay tables hold beta lambda^-j for j < chunk with one fp16 scale per head), or
 * |1 - lambda|^2 > 1000 (1 - |lambda|^2): a mode (nearly) undamped far from lambda = 1, whose
 * state is an oscillating sum in which the mean feature (about 1) cancels while the bf16
 * rounding of the features does not.  S4D-Lin modes exp(dt(-1/2 + i pi m)), m < 64, never do
 * for dt <= 0.17 at chunk 64.
 * The route is decided on the device from lambda, with this same test, in the prefill's own
 * launches: the head's first workgroup runs the token-by-token fp32 recurrence over the whole
 * sequence (about as slow per head as the fp32 prefill below); the other heads are
 * unaffected. */
ia_status ia_check_lambda(const ia_desc* desc, const void* lambda_host, int* fp32_heads);

/* Causal (or, with IA_FLAG_BIDIR, bidirectional) forward of one IA layer over N tokens.
 *
 * bf16 inputs: the chunkwise form of the recurrence on MFMA.  Work inside each chunk of
 * `chunk` tokens is done as dense contractions, the state is passed across chunk boundaries,
 * and a second pass recomputes each segment from its corrected initial state [summary §3.2,
 * §A.2].  Results equal the token-by-token recurrence up to rounding and do not depend on
 * `chunk`.  Shapes: F = Dv in {32, 64, 128}, M in {16, 32, 64}, and 64 token rows of one
 * tensor within 1 GiB; other bf16 shapes return IA_ERR_UNSUPPORTED.  Heads with modes the
 * chunk factorisation does not resolve run the fp32 recurrence in the same launches (see
 * ia_check_lambda).  Accuracy: about 1e-2 row-wise relative error with the S4D-Lin modes and
 * beta = 1; like any finite-precision evaluation of o = num / max(den, clamp), a row whose
 * Re(den) nearly cancels (terms of both signs, e.g. with complex beta) or lies near the clamp
 * loses accuracy in proportion, about 2^-8 times the ratio of its terms' size to den.
 * fp32 inputs: the token-by-token recurrence in fp32, one workgroup per (b,h) slice (a
 * reference path: about 300x slower than the chunked path at the 1.3B-shaped layer).
 *
 *   q, k, v    inputs, layouts above, read only.
 *   lambda     [H][M] complex64 modes (see ia_check_lambda), read on the device only.
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
 * IA_ERR_DOMAIN (den_clamp), IA_ERR_UNSUPPORTED (BIDIR with st != NULL, sizes, chunk, bf16
 * shapes without a chunk kernel), IA_ERR_WORKSPACE, IA_ERR_LAUNCH. */
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

/* Bytes of the device array that ia_prefill_fwd_noalloc uses as its workspace. */
#define IA_NOALLOC_SCRATCH_BYTES (32u << 20)

/* ia_prefill_fwd with no workspace argument that allocates nothing, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation.  Its workspace is a fixed array of IA_NOALLOC_SCRATCH_BYTES bytes inside
 * the library, one per device, which each device holds until the process ends (the first call
 * on a device looks its address up; that lookup failing returns IA_ERR_LAUNCH).
 *   - A call whose workspace (ia_prefill_workspace_bytes) exceeds the array returns
 *     IA_ERR_WORKSPACE and enqueues nothing (the 1.3B-shaped layer, B=4 H=16 N=2048 F=Dv=128
 *     M=64, needs 21 MiB).
 *   - All calls on one device share the array.  Calls ordered on one stream are safe; calls
 *     that can overlap in time on one device (other streams, other threads) race on it.
 *   - The array's contents are scratch: nothing in it needs to start at zero, and it keeps
 *     whatever the last call left.
 * Other arguments, results and errors as ia_prefill_fwd. */
ia_status ia_prefill_fwd_noalloc(const ia_desc* desc,
                                 const void* q, const void* k, const void* v,
                                 const void* lambda, const void* beta,
                                 ia_state* st, void* o, void* stream);

/* Profiling variant of ia_prefill_fwd: identical work and results, and in addition, for its
 * i-th kernel launch (i < max_launches, in launch order), records events[2i] before and
 * events[2i+1] after the kernel on `stream` and stores the kernel's kind in kinds[i]
 * (2 decay tables, launched on their own only when a sequence is one segment; 3 segment end
 * states, whose launch also computes the tables when there are several segments; 4 segment
 * carry; 5 chunked prefill with outputs; 0 zero fill; 1 token-sequential prefill; 10 copy of
 * the caller's initial state into the workspace).  events: 2*max_launches hipEvent_t handles
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

/* Workspace bytes ia_prefill_bwd needs for this descriptor, each region 256-byte aligned; 0 on
 * an invalid descriptor (or a backward flag combination it refuses).
 * Chunked kernels: every 16-token chunk's start state per group of 16 modes
 * (B*H*ceil(N/16)*M*(F+Dv+1) complex64), per-token den and dL/do.num partials per group
 * (B*H*N*M/16 float pairs), per-mode-group gradient rows (M/16 * B*H*N*(2F+Dv) float) and
 * per-slice lambda/beta gradients.
 * Token-sequential kernels: state checkpoints every 32 tokens (B*H*ceil(N/32)*M*(F+Dv+1)
 * complex64), per-token partial denominators (B*H*N*M/2 complex64), the gradient rows as above,
 * per-slice lambda/beta gradients, the recompute's a = phi(q) U^T per token (B*H*N*M complex64)
 * and, when a long sequence is cut into segments, their start states and entering adjoints. */
size_t ia_prefill_bwd_workspace_bytes(const ia_desc* desc);

/* Gradients of the causal layer (ia_prefill_fwd's outputs o) for a real loss L, given
 * dO = dL/do: reverse-mode differentiation of the recurrence and readout above, as the
 * training step of [summary §G] needs, in fp32 throughout.  The states are recomputed from st0
 * (not read from a forward call).  Chunked kernels (the flags above pick them): 16-token
 * chunks per (b, h, group of 16 modes), every contraction on fp32 MFMA, each chunk's start
 * state stored by a forward sweep and the state adjoints carried chunk by chunk backward
 * [summary §A.2].  Token-sequential kernels: checkpoints every 32 tokens, the states rebuilt
 * backward inside each interval by U_{t-1} = (U_t - beta phi(k_t)) / lambda.
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
 * Accuracy: the chunked kernels' chunk-local powers lambda^e (|e| <= 9) stay inside fp32's
 * range for |lambda| above about 1e-4.  The gradients then carry fp32 rounding amplified by the
 * layer's own conditioning: with the denominator and |lambda| well below 1, o_t tends to v_t
 * and dq, dk are differences of nearly equal terms; dlambda's distance-weighted sums lose
 * about log10(1/|lambda|) + 2 digits (tested to |lambda| = 0.01).  In the
 * token-sequential kernels the rebuild grows fp32 rounding by at most |lambda|^-31 inside an
 * interval; for |lambda| >= 0.9 that is below 30x (an S4D-Lin lambda = exp(dt(-1/2 + i pi m))
 * with dt <= 0.1 has |lambda| >= 0.95).
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
 * The decode step runs its fp32 kernels.  The prefill with bf16 inputs on the chunk kernels'
 * shapes (ia_prefill_fwd's) runs the chunked path: the readouts' query-mode rows a (C x M per
 * chunk) take a R on MFMA before both readouts, the state pass unchanged [summary §A.2, §A.3].
 * Its chunk length is desc->chunk, or with chunk 0 64, except F = Dv = 128 with M = 64, whose
 * 64-token layout has no room for R in LDS: there 32, and an explicit chunk 64 returns
 * IA_ERR_UNSUPPORTED.  The same accuracy note as ia_prefill_fwd applies, with the denominator's
 * conditioning that of Re(a R eta): a strongly mixing R can raise the terms over the
 * denominator.  fp32 inputs, and bf16 shapes without chunk kernels, run the token-sequential
 * fp32 kernel.  Other arguments, layouts and errors as ia_prefill_fwd / ia_decode_step;
 * readout must be 16-byte aligned and must not overlap an output. */

/* Workspace bytes ia_prefill_fwd_readout needs at most: on the chunked path its plan (as
 * ia_prefill_workspace_bytes, at its chunk length) plus each head's readout-matrix operand,
 * 8*M*M bytes and a scale, 256-byte aligned; otherwise that of the token-sequential path
 * (ia_prefill_workspace_bytes: a state and the segments' slots).  0 on an invalid
 * descriptor. */
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

/* The block's edges around the layer: the pieces the pages place before and after the IA
 * mixer in their model blocks, named there without formulas.  Readings taken:
 *   - short convolutions on q, k (summary §5.3, the ablations of §B.1) and on v: causal and
 *     depthwise along time, conv_width taps per channel (tap 0 on the current token), the
 *     conv_width-1 raw tokens before token 0 taken from conv_state_in (zeros if NULL), then
 *     SiLU (x * sigmoid(x));
 *   - RoPE on q and k (the language models of summary §A.1): feature pairs (2i, 2i+1) turned
 *     by the angle p * rope_base^(-2i/F) at position p = pos0 + n;
 *   - the feature map elu+1 on q and k, after the two steps above;
 *   - the SSM input z = [phi(k), v] (F + Dv entries) normalised per token and head, as the
 *     episode page's implementation details describe it (an RMS normalisation with a learned
 *     per-head bias): z' = g * z / sqrt(mean(z^2) + norm_eps) + b;
 *   - the output gate (summary §3.3): out = o * SiLU(gate), gate the caller's projection.
 * ia_block_prologue writes phi(q'), phi(k')'s and v''s normalised values: the inputs of
 * ia_prefill_fwd / ia_decode_step with IA_FLAG_IDENTITY_FEATURES.  It streams each input once
 * (one workgroup per 64 tokens of a (b,h) slice).  For decode, call it with N = 1 and the
 * token's position in pos0, carrying the convolution state from call to call.
 *   desc          B, H, N, F, Dv and in_dtype (inputs and outputs; M unused but checked).
 *   p->conv_width 0 (no convolution, no SiLU) to 8; p->conv_q, p->conv_k [H][F][conv_width],
 *                 p->conv_v [H][Dv][conv_width] float, tap tau weighting the token tau steps
 *                 back, required with conv_width > 0.
 *   p->rope_base  > 0: RoPE with that base; 0: none.  p->pos0 >= 0, pos0 + N - 1 (the
 *                 last position) at most 2^31 - 1.
 *   p->norm_gain, p->norm_bias  [H][F+Dv] float each, both or neither (no normalisation);
 *                 p->norm_eps >= 0.
 *   q, k, v       raw [B][N][H][F|Dv] in_dtype, read only.
 *   conv_state_in, conv_state_out  [B][H][conv_width-1][2F+Dv] float (q, k, v channels side
 *                 by side, oldest token first): the raw tokens before token 0, and those
 *                 ending at token N-1 (NULL: none); distinct buffers; unused for
 *                 conv_width <= 1.
 *   fq, fk, vo    [B][N][H][F|Dv] in_dtype outputs.
 * Parameter arrays 16-byte aligned; outputs must not overlap any input or each other.
 * Errors as ia_prefill_fwd, IA_ERR_UNSUPPORTED for conv_width > 8 or a token row of one
 * tensor (H * max(F, Dv) elements) of 16 MiB or more, IA_ERR_DOMAIN for a negative or
 * non-finite rope_base or norm_eps, or positions outside 0 .. 2^31 - 1. */
typedef struct ia_block_params {
  int conv_width;
  const void *conv_q, *conv_k, *conv_v;
  float rope_base;
  int pos0;
  const void *norm_gain, *norm_bias;
  float norm_eps;
} ia_block_params;

ia_status ia_block_prologue(const ia_desc* desc, const ia_block_params* p,
                            const void* q, const void* k, const void* v,
                            const void* conv_state_in, void* conv_state_out,
                            void* fq, void* fk, void* vo, void* stream);

/* out = o * SiLU(gate) elementwise over [B][N][H][Dv] (desc->N = 1 for a decode step's o_t);
 * o, gate and out in desc->out_dtype; out may be o itself (in place), and must not overlap
 * gate.  Errors as ia_prefill_fwd. */
ia_status ia_block_gate(const ia_desc* desc, const void* o, const void* gate, void* out,
                        void* stream);

/* One decode step of the whole block, in one kernel: ia_block_prologue of the token (N = 1,
 * position p->pos0, the convolution state carried from conv_state_in to conv_state_out), the
 * layer's step as ia_decode_step on its outputs, then the output gate, out = o * SiLU(gate).
 * The prologue's outputs stay in fp32 inside the kernel (ia_block_prologue followed by
 * ia_decode_step rounds them to in_dtype in between), so the two routes agree to rounding.
 * For callers that run a stack of layers token by token, one kernel node per layer.
 *   desc        as ia_decode_step (N unused); IA_FLAG_BIDIR and IA_FLAG_IDENTITY_FEATURES
 *               return IA_ERR_UNSUPPORTED (the prologue applies the feature map itself).
 *   p           as ia_block_prologue, pos0 the token's position.
 *   q_t, k_t, v_t  raw [B][H][F|Dv] in_dtype.
 *   conv_state_in, conv_state_out  as ia_block_prologue ([B][H][conv_width-1][2F+Dv] float).
 *   gate_t      [B][H][Dv] in_dtype, or NULL for no gate.
 *   lambda, beta, st  as ia_decode_step; st updated in place.
 *   out_t       [B][H][Dv] out_dtype.
 * Outputs (out_t, the state, conv_state_out) must not overlap any input or each other.
 * Errors as ia_decode_step and ia_block_prologue. */
ia_status ia_block_decode_step(const ia_desc* desc, const ia_block_params* p,
                               const void* q_t, const void* k_t, const void* v_t,
                               const void* conv_state_in, void* conv_state_out,
                               const void* gate_t, const void* lambda, const void* beta,
                               ia_state* st, void* out_t, void* stream);

/* Selective writing and memory decay.  Input-dependent gates, computed by the caller for every
 * token, control what the memory stores and how fast it forgets (the optional enhancement of
 * [summary §3.3], ablated as selective vs non-selective in [summary §B.3, Table 7]).  The pages
 * give no formula; the reading implemented, with a write gate w and a decay gate a per token
 * and head:
 *   U[m,:]   <- a_t lambda_m U[m,:]   + w_t beta_m phi(k_t)
 *   Gam[m,:] <- a_t lambda_m Gam[m,:] + w_t beta_m v_t
 *   eta[m]   <- a_t lambda_m eta[m]   + w_t beta_m
 * and the readout unchanged (w = a = 1 is the plain layer; 0 < a <= 1 forgets faster).
 *   wgate, dgate  float, device, read only: [B][N][H] for the prefill (dense, element
 *                 (b, n, h) at (b N + n) H + h), [B][H] for the decode step; NULL:
 *                 IA_ERR_NULL; 16-byte aligned; must not overlap an output.
 * Paths: bf16 inputs on the shapes of the chunked kernels (as ia_prefill_fwd's) run the
 * chunked MFMA prefill with the gates folded into each chunk (per token, the running sum of
 * log2|a| and the sign of the running product of a within the chunk; a decay gate with
 * |a| < 2^-64, zero included, counts as 2^-64 there, so the carried state falls to 2^-64 of
 * itself instead of to zero); fp32 inputs, and bf16 inputs on other shapes, run the
 * token-sequential fp32 kernels with sequence segments as the fp32 prefill.  Gates may take any
 * real value; rows whose readout sums cancel are resolved to the precision of each path.
 * IA_FLAG_BIDIR: both directions use the gates of the positions they walk.  Other arguments,
 * layouts and errors as ia_prefill_fwd / ia_decode_step.  The workspace (the chunked plan's,
 * or the fp32 path's: a state and the segments' slots) is
 * ia_prefill_gated_workspace_bytes(desc) bytes. */
size_t ia_prefill_gated_workspace_bytes(const ia_desc* desc);

ia_status ia_prefill_fwd_gated(const ia_desc* desc,
                               const void* q, const void* k, const void* v,
                               const void* wgate, const void* dgate,
                               const void* lambda, const void* beta,
                               ia_state* st, void* o,
                               void* workspace, size_t ws_bytes, void* stream);

ia_status ia_decode_step_gated(const ia_desc* desc,
                               const void* q_t, const void* k_t, const void* v_t,
                               const void* wgate, const void* dgate,
                               const void* lambda, const void* beta,
                               ia_state* st, void* o_t, void* stream);

/* Static string naming a status code. */
const char* ia_status_string(ia_status s);

/* Static string: the HIP runtime's text for the error behind the calling thread's most recent
 * IA_ERR_LAUNCH ("no launch error" if there was none), kept per thread. */
const char* ia_last_launch_error(void);

#ifdef __cplusplus
}
#endif

#endif /* IA_H */
