// ia_kernels.hpp — internal launch interface between the C ABI (ia_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

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
};

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
};

// Chunked MFMA prefill of one direction (bf16 inputs).  The sequence is cut into `segments`
// runs of `seg_chunks` chunks; with more than one, the end states of all but the last segment
// go through `slots` (B*H*(segments-1) slots of chunk_slot_floats(F, D, M) floats), from
// which each segment's workgroup assembles its initial state.  `tables` holds
// H * chunk_table_bytes(chunk, M) bytes.  U0/G0/E0: initial state or NULL (zeros);
// U1/G1/E1: final state or NULL.  o NULL: state only.  accumulate: add to the values already
// in o (in o's dtype).
struct ChunkPrefillArgs {
  const void *q, *k, *v;   // element strides sqk (q and k) and sv; o dense
  RowStrides sqk, sv;
  const float2 *lam, *beta;
  void* o;
  int accumulate;
  const float2 *U0, *G0, *E0;
  float2 *U1, *G1, *E1;
  float* slots;                 // (B*H) x (segments-1) segment end states
  unsigned char* tables;
  int B, H, N, F, D, M;
  int chunk, segments, seg_chunks;
  int reverse, out_bf16;
  float clamp;
  int opt;   // kOptNoDen | kOptIdentity
};

bool chunk_supported(int F, int D, int M);
long chunk_table_bytes(int chunk, int M);
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

int chunk_wgs_per_cu(int chunk, int F, int D, int M);   // 0 if unknown (no device)
int device_cus();                                        // compute units of the current device
hipError_t launch_chunk_prefill(const ChunkPrefillArgs& a, hipStream_t st);

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t st);
hipError_t launch_decode_step(const DecodeArgs& a, hipStream_t st);
hipError_t launch_scan_prefill(const ScanArgs& a, hipStream_t st);

}  // namespace ia
