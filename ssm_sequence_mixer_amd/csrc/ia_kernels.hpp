// ia_kernels.hpp — internal launch interface between the C ABI (ia_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include <cmath>

namespace ia {

// Kernel kinds reported by the profiling entry point, in launch order.
enum LaunchKind {
  kKindFill = 0,       // state / workspace zero fill
  kKindScan = 1,       // token-sequential prefill
  kKindTables = 2,     // per-head decay tables of the chunked prefill
  kKindSummary = 3,    // chunked prefill, segment end states (no outputs)
  kKindCarry = 4,      // segment carry (many segments)
  kKindChunk = 5,      // chunked prefill with outputs (or the last segment's state)
  kKindDecode = 6,
  kKindBwdForward = 7,   // backward: state recompute and checkpoints
  kKindBwdReverse = 8,   // backward: reverse sweep
  kKindBwdReduce = 9,    // backward: sum of the mode groups' partials
  kKindCopy = 10,        // copy of the caller's initial state into the workspace
  kKindBlock = 11,       // the block's edges: input prologue, output gate
};

// While set (only inside ia_prefill_fwd_profiled), every launch records events[2i] before
// and events[2i+1] after its i-th kernel on the launch stream, and notes its kind.
struct ProfileSink {
  void** events;
  int* kinds;
  int max_launches;
  int used;
};
extern thread_local ProfileSink* g_profile;

inline void prof_begin(hipStream_t st) {
  if (g_profile && g_profile->used < g_profile->max_launches)
    (void)hipEventRecord(static_cast<hipEvent_t>(g_profile->events[2 * g_profile->used]), st);
}
inline void prof_end(hipStream_t st, int kind) {
  if (g_profile && g_profile->used < g_profile->max_launches) {
    (void)hipEventRecord(static_cast<hipEvent_t>(g_profile->events[2 * g_profile->used + 1]),
                         st);
    g_profile->kinds[g_profile->used++] = kind;
  }
}

constexpr int kMaxDim = 256;    // largest F and Dv
constexpr int kMaxModes = 128;  // largest M

// Readout options (the desc's flags, as kernels take them): kOptNoDen, o = Re num with no
// denominator; kOptIdentity, q and k arrive as features (no feature map).
constexpr int kOptNoDen = 1, kOptIdentity = 2;

// Element strides of a [B][N][H][X] tensor along b, n and h (X contiguous).
struct RowStrides {
  long long b, n, h;
};
inline RowStrides dense_strides(int N, int H, int X) {
  return RowStrides{(long long)N * H * X, (long long)H * X, X};
}

// One token of the block's prologue and the output gate around a decode step
// (ia_block_decode_step): q, k, v of the step are then the raw projections.
struct BlockStepArgs {
  const float *conv_q, *conv_k, *conv_v;   // [H][F|D][W] or NULL (conv_width 0)
  const float* state_in;                   // [B][H][W-1][2F+D] raw tokens before, or NULL
  float* state_out;                        // the same ending at this token, or NULL
  const float *norm_gain, *norm_bias;      // [H][F+D] or NULL
  float norm_eps, rope_base;               // rope_base 0: no RoPE
  int pos, conv_width;                     // the token's position; taps (0..kMaxConvTaps)
  const void* gate;                        // [B][H][D] in the input dtype, or NULL
};

struct DecodeArgs {
  const void *q, *k, *v;
  const float2 *lam, *beta;
  float2 *U, *G, *E;
  void* o;
  int B, H, F, D, M;
  int in_bf16, out_bf16;
  float clamp;
  int opt;   // kOptNoDen | kOptIdentity
  const float2* readout = nullptr;   // [H][M][M] readout matrix, or NULL
  const float *wgate = nullptr, *dgate = nullptr;   // [B][H] write / decay gates, or NULL
  int block = 0;          // q, k, v raw: the block prologue runs first (blk), the gate after
  BlockStepArgs blk{};
};

// The block's edges (ia_block.hip): short convolutions of up to kMaxConvTaps taps.
constexpr int kMaxConvTaps = 8;

struct BlockArgs {
  const void *q, *k, *v;          // raw [B][N][H][F|D], bf16 or f32 (bf16 flag)
  void *fq, *fk, *vo;             // outputs, same dtype and layout
  const float *conv_q, *conv_k, *conv_v;   // [H][F|D][W] or NULL (conv_width 0)
  const float* state_in;          // [B][H][W-1][2F+D] raw tokens before token 0, or NULL
  float* state_out;               // the same for the last W-1 tokens, or NULL
  const float *norm_gain, *norm_bias;      // [H][F+D] or NULL
  float norm_eps, rope_base;
  int B, H, N, F, D, conv_width, pos0, bf16;
};
hipError_t launch_block_prologue(const BlockArgs& a, hipStream_t st);
// out = o * SiLU(g) over n elements (n even), bf16 or f32
hipError_t launch_block_gate(const void* o, const void* g, void* out, size_t n, int bf16,
                             hipStream_t st);

struct ScanArgs {
  const void *q, *k, *v;   // element strides sqk (q and k) and sv; o dense
  RowStrides sqk, sv;
  const float2 *lam, *beta;
  float2 *U, *G, *E;
  void* o;
  int accumulate;   // add to the values already in o (second direction of the bidirectional layer)
  int B, H, N, F, D, M;
  int in_bf16, out_bf16;
  float clamp;
  int reverse;
  int opt;   // kOptNoDen | kOptIdentity
  const float2* readout = nullptr;   // [H][M][M] readout matrix, or NULL
  const float *wgate = nullptr, *dgate = nullptr;   // [B][N][H] write / decay gates, or NULL
  // Sequence segments of the register-resident kernel (n_seg > 1, shapes it takes): each
  // segment's end state from zero and its decay product (state-only pass), the segment
  // starts (carry), then every segment from its start with outputs.  slots: n_seg states of
  // all B*H slices (the slice layout of U, Gamma, eta side by side), dec: (n_seg - 1) * B*H*M.
  int n_seg = 1, seg_len = 0;
  float2 *slots = nullptr, *dec = nullptr;
};
// Whether the register-resident kernel takes a shape (F, D in {32, 64, 128}).
bool scan_rows_supported(int F, int D);
// Complex floats of one slice's state, M (F + D + 1).
__host__ __device__ inline long scan_slot_float2(int F, int D, int M) { return (long)M * (F + D + 1); }

// Chunked MFMA prefill of one direction (bf16 inputs).  The sequence is cut into `segments`
// runs of `seg_chunks` chunks; with more than one, the end states of all but the last segment
// go through `slots` (B*H*(segments-1) slots of chunk_slot_floats(F, D, M) floats), from
// which each segment's workgroup assembles its initial state.  `tables` holds
// H * chunk_table_bytes(chunk, M) bytes.  U0/G0/E0: initial state or NULL (zeros);
// U1/G1/E1: final state or NULL (with a caller state both are the caller's buffers).
// wU/wG/wE: one state in the workspace ([B][H][M][F], [B][H][M][D], [B][H][M]): with several
// segments and a caller state, the initial state is copied there first, so that no
// workgroup reads the caller's buffers while the last segment writes the final state into
// them; heads that take the fp32 route without a caller state run in it.  o NULL: state only.
// accumulate: add to the values already in o (in o's dtype).
struct ChunkPrefillArgs {
  const void *q, *k, *v;   // element strides sqk (q and k) and sv; o dense
  RowStrides sqk, sv;
  const float2 *lam, *beta;
  void* o;
  int accumulate;
  const float2 *U0, *G0, *E0;
  float2 *U1, *G1, *E1;
  float* slots;                 // (B*H) x (segments-1) segment end states
  float* slots_rev;             // bidirectional, both walks in one call: the reverse walk's
                                // slots (same size); NULL otherwise
  unsigned char* tables;
  float2 *wU, *wG, *wE;         // workspace state
  const float2* readout;        // [H][M][M] readout matrix, or NULL (plain layer)
  unsigned char* rtab;          // its per-head MFMA operand (readout_table_bytes(M) each)
  const float *wgate, *dgate;   // gated layer: [B][N][H] write / decay gates, or NULL
  int B, H, N, F, D, M;
  int chunk, segments, seg_chunks;
  int reverse, out_bf16;
  float clamp;
  int opt;   // kOptNoDen | kOptIdentity
};

// Whether the bf16 chunk factorisation does NOT resolve mode lam = (lx, ly) at chunk length C
// (its head then runs the fp32 recurrence inside the chunked launches): for
//   - |lam| outside (0, 1 + 1e-6], or not finite: outside the S4D modes' domain, computed
//     literally by the fp32 recurrence;
//   - |lam|^(C-1) < 2^-8: the per-chunk decay tables hold beta lam^-j for j < C with one fp16
//     scale per head;
//   - |1 - lam|^2 > 1000 (1 - |lam|^2): a mode (nearly) undamped far from lam = 1.  Its state
//     is an oscillating sum over ~1/(1 - |lam|^2) tokens in which the mean of phi(k) = elu+1
//     (about 1) cancels while the bf16 rounding of the features does not: a few percent of
//     the sum at inputs of scale 1/sqrt(F).  S4D-Lin modes exp(dt(-1/2 + i pi m)) stay below
//     300 for any dt when m < 64 (the ratio peaks near 4/dt where the argument reaches pi).
// fp64 keeps the digits of 1 - |lam|^2 near the unit circle (every product below is exact).
// The device computes it with the tables; ia_check_lambda runs the same function on the host.
__host__ __device__ inline bool chunk_unresolved(float lx, float ly, int C) {
  const double x = lx, y = ly;
  const double mag2 = x * x + y * y;
  if (!(mag2 > 0.0) || !(mag2 <= (1.0 + 1e-6) * (1.0 + 1e-6))) return true;
  if (0.5 * (C - 1) * log(mag2) < -8.0 * 0.6931471805599453) return true;
  const double one_minus = (1.0 - x) * (1.0 + x) - y * y;   // 1 - |lam|^2
  const double dist2 = (1.0 - x) * (1.0 - x) + y * y;       // |1 - lam|^2
  return dist2 > 1000.0 * one_minus;
}

bool chunk_supported(int F, int D, int M);
long chunk_table_bytes(int chunk, int M);
// Shapes and chunk lengths with a readout-matrix instantiation of the output pass, and the
// bytes of one head's readout-matrix operand.
bool chunk_rm_supported(int chunk, int F, int D, int M);
long readout_table_bytes(int M);
long chunk_slot_floats(int F, int D, int M);
// Backward pass (ia_backward.hip).  States are checkpointed every kBwdCheckpoint tokens.
constexpr int kBwdCheckpoint = 32;
constexpr int kBwdPrefetch = 2;   // 16-byte loads per thread that stage a block of token rows
constexpr int kBwdMinSegment = 256;   // shortest sequence segment of the backward sweeps

struct BwdArgs {
  const void *q, *k, *v, *dO;
  const float2 *lam, *beta;
  const float2 *U0, *G0, *E0;     // initial state, or all NULL (zeros)
  void *dq, *dk, *dv;             // in dtype
  float2 *dlam, *dbeta;           // [H][M]
  float2 *dU0, *dG0, *dE0;        // gradient of the initial state, or all NULL
  float2* ckpt;                   // workspace regions (BwdLayout)
  float2* dpart;
  float* gpart;
  float2* lpart;
  float2* apart;                  // a[m] per token, from the recompute sweep
  int B, H, N, F, D, M;
  int in_bf16, out_bf16, opt;
  float clamp;
  int tb;                         // tokens per staged block (bwd_block_tokens)
  int dir;                        // 1: walk index t is position N-1-t (reversed sequence)
  int accumulate;                 // 1: add the gradients onto dq, dk, dv, dlam, dbeta
  int nseg, seg_len;              // sequence segments swept side by side (bwd_segments)
  int local;                      // 1: the segment-local pass that feeds a carry
  float2 *cstate, *cadj;          // segment start states and entering adjoints (nseg > 1)
};

struct BwdLayout {
  size_t ckpt_off, dpart_off, gpart_off, lpart_off, apart_off, cstate_off, cadj_off, bytes;
};
int bwd_segments(int B, int H, int N, int M, int* seg_len);
BwdLayout bwd_layout(int B, int H, int N, int F, int D, int M);
int bwd_block_tokens(int F, int D, int M, int in_bf16, int out_bf16);
size_t bwd_lds_bytes(int F, int D, int M, int in_bf16, int out_bf16, int tb, bool rev);
hipError_t launch_prefill_bwd(const BwdArgs& a, hipStream_t st);
// The sum of the mode groups' partial rows (gpart) and of the lambda/beta partials (lpart).
hipError_t launch_bwd_reduce(const BwdArgs& a, hipStream_t st);
// Chunked backward on fp32 MFMA (ia_backward_chunk.hip): F == Dv in {32, 64, 128}, M a
// multiple of 16, no sequence segments.  Its workspace: chunk start states (ckpt), per-token
// den and g.num partials (dpart), gpart and lpart as the token-sequential path.
bool bwd_chunked_supported(int F, int D, int M);
BwdLayout bwd_chunked_layout(int B, int H, int N, int F, int D, int M);
hipError_t launch_prefill_bwd_chunked(const BwdArgs& a, hipStream_t st);

int chunk_wgs_per_cu(int chunk, int F, int D, int M, bool rm = false,
                     bool gated = false);   // 0 if unknown (no device)
int device_cus();                                        // compute units of the current device
hipError_t launch_chunk_prefill(const ChunkPrefillArgs& a, hipStream_t st);

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t st);
// dst[i] <- src[i] for up to three (dst, src, bytes) pairs (bytes multiples of 16; a pair
// with bytes 0 is skipped), one launch.
hipError_t launch_copy3(void* d0, const void* s0, size_t n0, void* d1, const void* s1,
                        size_t n1, void* d2, const void* s2, size_t n2, hipStream_t st);
hipError_t launch_decode_step(const DecodeArgs& a, hipStream_t st);
hipError_t launch_scan_prefill(const ScanArgs& a, hipStream_t st);

}  // namespace ia
