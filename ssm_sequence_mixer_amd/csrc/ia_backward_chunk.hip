// ia_backward_chunk.hip — chunked gradients of the causal IA layer on fp32 MFMA
// (v_mfma_f32_16x16x4_f32): the reverse mode of the recurrence taken chunk by chunk, so that
// every sum over a chunk's tokens, features or modes is a matrix product, in fp32 throughout.
// The training-time figures of "Interdomain Attention: Beyond Token-Level Key-Value Memory"
// (summary page §G) count this pass beside the forward; the recurrence and readout are those
// of summary page §3.1-§3.2 and the episode page's derivation; the chunkwise form is summary
// page §A.2.
//
// Layer, per mode m (lam, beta complex; phi = elu + 1 or the identity):
//   U_t = lam U_{t-1} + beta phi(k_t),  G_t = lam G_{t-1} + beta v_t,  e_t = lam e_{t-1} + beta
//   a_t = phi(q_t) . U_t,  num_t = Re sum_m a_t G_t,  den_t = Re sum_m a_t e_t,
//   o_t = num_t / c_t with c_t = max(den_t, clamp).
// With g_t = dL/do_t / c_t and dd_t = -(dL/do_t . o_t) / c_t where den_t >= clamp (0 below it;
// g = dL/do, dd = 0 without a denominator), every gradient follows from
//   A_t[m] = g_t . G_t[m] + dd_t e_t[m]          (dL/da_t = conj(A_t))
// and the forward a_t (dL/dG_t = g_t conj(a_t), dL/de_t = dd_t conj(a_t)).
// In a chunk of C tokens (local index i, start states U_c, G_c, e_c, and S^U, S^G, S^e the
// adjoints the chunk's last state receives from later tokens), with S = phi(Q) phi(K)^T,
// S' = g V^T + dd 1^T, both causal (j <= i), and P[i,j] = Re sum_m a_i beta lam^(i-j),
// Pg[i,j] = Re sum_m A_i beta lam^(i-j):
//   a_i  = beta sum_j lam^(i-j) S[i,j]  + lam^(i+1) phi(q_i) . U_c
//   A_i  = beta sum_j lam^(i-j) S'[i,j] + lam^(i+1) (g_i . G_c + dd_i e_c)
//   dphi(q_i) = sum_j Pg[i,j] phi(k_j) + Re sum_m lam^(i+1) A_i U_c
//   dphi(k_j) = sum_i Pg[i,j] phi(q_i) + Re sum_m conj(beta lam^(C-1-j)) S^U
//   dv_j      = sum_i P[i,j] g_i      + Re sum_m conj(beta lam^(C-1-j)) S^G
//   S^U <- conj(lam^C) S^U + conj(sum_i lam^(i+1) A_i phi(q_i))   (likewise S^G with a_i g_i,
//   S^e with a_i dd_i), which is the adjoint of the chunk's start state;
// dbeta and dlam add, per mode, the products of each token's state adjoint with its input and
// with the previous state.  The distance-weighted sums that dlam needs,
// sum_j (i-j) lam^(i-j-1) S[i,j], split into lam^(i-1-o) (i T0 - T1) with
// T0 = sum_j lam^(o-j) S[i,j] and T1 = sum_j j lam^(o-j) S[i,j]: two more products with fixed
// per-mode tables.  The powers are centred (o = C/2), so with C = 16 they stay inside fp32's
// range for |lam| above about 1e-4.
//
// Launches (one workgroup per (b, h, group of 16 modes), chunks walked in order):
//  1. bwdc_forward_kernel: from the initial state, stores every chunk's start state and, per
//     token, the group's partial sums of den_t and of dL/do_t . num_t (the readout gradient
//     needs both over all modes before any chunk runs backward).
//  2. bwdc_reverse_kernel: chunks from last to first with the adjoints in LDS; per chunk the
//     contractions above on MFMA, the per-(token, mode) terms of dlam and dbeta, and the
//     group's partial rows of dq, dk (through phi'), dv.
//  3. the reduce kernel of ia_backward.hip sums the groups' partial rows in group order and the
//     lambda and beta gradients over the batch.
//
// MFMA operands.  v_mfma_f32_16x16x4_f32 takes, in lane l, A[l % 16][k] and B[k][l % 16] for one
// k of four (k = l / 16) and leaves D[4 (l / 16) + r][l % 16] in accumulator r.  Every product
// here walks K in blocks of 16 with lane l holding k = 4 (l / 16) + s in step s (the same on both
// sides), so an operand stored with K contiguous is one 16-byte LDS read per four steps.
#include <algorithm>

#include "ia_device.hpp"
#include "ia_kernels.hpp"

namespace ia {

namespace {

constexpr int kC = 16;          // chunk length
constexpr int kMG = 16;         // modes per workgroup
constexpr int kM2 = 2 * kMG;    // real rows of a group's complex state (Re rows, then Im rows)
constexpr int kO = kC / 2;      // centre of the chunk-local powers
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kPwLo = kC + 1;           // PW[e + kPwLo] = lam^e, e in [-kC-1, kC+1]
constexpr int kPwN = 2 * kC + 3;
constexpr int LC = kC + 4;              // leading dims (floats): rows stay 16-byte aligned
constexpr int L2M = kM2 + 4;
constexpr int L4M = 2 * kM2 + 4;
constexpr int LA = kC + kM2 + 4;

typedef float f4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f4 mfma4(float a, float b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// acc += A B over K (a multiple of 16) for one 16 x 16 tile.  A points at the tile's first row
// (AK: A(r,k) = A[r*lda + k], else A(r,k) = A[k*lda + r]); B at its first column (BK:
// B(k,n) = B[n*ldb + k], else B(k,n) = B[k*ldb + n]).
// Operands of one K block of 16 (four MFMA steps) into registers.
template <bool AK, bool BK>
__device__ __forceinline__ void tile_operands(float (&a)[4], float (&b)[4], const float* A,
                                              int lda, const float* B, int ldb, int rc, int kk) {
  if constexpr (AK) {
    const float4 x = *reinterpret_cast<const float4*>(A + rc * lda + kk);
    a[0] = x.x; a[1] = x.y; a[2] = x.z; a[3] = x.w;
  } else {
#pragma unroll
    for (int s = 0; s < 4; ++s) a[s] = A[(kk + s) * lda + rc];
  }
  if constexpr (BK) {
    const float4 x = *reinterpret_cast<const float4*>(B + rc * ldb + kk);
    b[0] = x.x; b[1] = x.y; b[2] = x.z; b[3] = x.w;
  } else {
#pragma unroll
    for (int s = 0; s < 4; ++s) b[s] = B[(kk + s) * ldb + rc];
  }
}

// PIPE: the next block's operands are read from LDS before the current block's MFMAs issue
// (eight more registers; for kernels with registers to spare).
template <int K, bool AK, bool BK, bool PIPE = false>
__device__ __forceinline__ void tile_mma(f4& acc, const float* A, int lda, const float* B,
                                         int ldb, int lane) {
  static_assert(K % 16 == 0, "K in blocks of 16");
  const int rc = lane & 15, kq = 4 * (lane >> 4);
  // blocks of 16 alternate between two accumulators (two dependent chains in flight)
  f4 acc2 = f4{0.f, 0.f, 0.f, 0.f};
  if constexpr (PIPE) {
    float a[2][4], b[2][4];
    tile_operands<AK, BK>(a[0], b[0], A, lda, B, ldb, rc, kq);
#pragma unroll
    for (int blk = 0; blk < K / 16; ++blk) {
      if (blk + 1 < K / 16)
        tile_operands<AK, BK>(a[(blk + 1) & 1], b[(blk + 1) & 1], A, lda, B, ldb, rc,
                              16 * (blk + 1) + kq);
      f4& t = blk & 1 ? acc2 : acc;
#pragma unroll
      for (int s = 0; s < 4; ++s) t = mfma4(a[blk & 1][s], b[blk & 1][s], t);
    }
  } else {
#pragma unroll
    for (int blk = 0; blk < K / 16; ++blk) {
      float a[4], b[4];
      tile_operands<AK, BK>(a, b, A, lda, B, ldb, rc, 16 * blk + kq);
      f4& t = blk & 1 ? acc2 : acc;
#pragma unroll
      for (int s = 0; s < 4; ++s) t = mfma4(a[s], b[s], t);
    }
  }
  if constexpr (K > 16) acc += acc2;
}

__device__ __forceinline__ f4 zero4() { return f4{0.f, 0.f, 0.f, 0.f}; }

// Row and column of accumulator r in lane l.
__device__ __forceinline__ int acc_row(int lane, int r) { return 4 * (lane >> 4) + r; }
__device__ __forceinline__ int acc_col(int lane) { return lane & 15; }

__device__ __forceinline__ float2 cconj(float2 a) { return make_float2(a.x, -a.y); }
__device__ __forceinline__ float2 cadd2(float2 a, float2 b) { return make_float2(a.x + b.x, a.y + b.y); }
__device__ __forceinline__ float2 csc(float s, float2 a) { return make_float2(s * a.x, s * a.y); }
// a * conj(b)
__device__ __forceinline__ float2 cmulc2(float2 a, float2 b) {
  return make_float2(a.x * b.x + a.y * b.y, a.y * b.x - a.x * b.y);
}

// Sum over the 16 lanes of a row (lanes 16r .. 16r+15), left in every lane of the row: two
// sums at once through DPP moves (row_totals: quad swaps, then half-row and row mirrors), no
// LDS round trip.
__device__ __forceinline__ void row16_sum2(float& x, float& y) {
  float v[2] = {x, y};
  row_totals<16, 2>(v);
  x = v[0];
  y = v[1];
}

// lam^e for integer e (negative allowed), in fp64 by binary exponentiation, rounded once.
__device__ float2 cpow_i(float2 z, int e) {
  double br = z.x, bi = z.y;
  if (e < 0) {   // 1/z
    const double n = br * br + bi * bi;
    br = br / n;
    bi = -bi / n;
    e = -e;
  }
  double ar = 1.0, ai = 0.0;
  for (; e > 0; e >>= 1) {
    if (e & 1) {
      const double tr = ar * br - ai * bi;
      ai = ar * bi + ai * br;
      ar = tr;
    }
    const double qr = br * br - bi * bi;
    bi = 2.0 * br * bi;
    br = qr;
  }
  return make_float2((float)ar, (float)ai);
}

// The workgroup's (slice, group) and its per-mode constants.  Workgroups are dispatched to the
// eight XCDs in turn (block b to XCD b % 8); with the grid a multiple of 8, block b takes
// position (b % 8) (grid / 8) + b / 8, so every XCD holds whole slices, and the mode groups of
// a slice, which read the same token rows chunk by chunk, share that XCD's L2.
struct Wg {
  int slice, b, h, group, m0;
};
__device__ __forceinline__ Wg wg_of(const BwdArgs& a) {
  const int groups = a.M / kMG;
  const int nb = gridDim.x;
  const int p = nb % 8 ? (int)blockIdx.x : (blockIdx.x % 8) * (nb / 8) + blockIdx.x / 8;
  Wg w;
  w.slice = p / groups;
  w.group = p % groups;
  w.b = w.slice / a.H;
  w.h = w.slice % a.H;
  w.m0 = w.group * kMG;
  return w;
}

// Element (walk position t, column f) of a [B][N][H][W] array.
__device__ __forceinline__ size_t row_index(const BwdArgs& a, const Wg& w, int t, int W) {
  const size_t pos = a.dir ? (size_t)(a.N - 1 - t) : (size_t)t;
  return (((size_t)w.b * a.N + pos) * a.H + w.h) * W;
}

// Per-mode power table PW[e + kPwLo][m] = lam_m^e and beta, in LDS.
__device__ void build_powers(const BwdArgs& a, const Wg& w, float2* PW, float2* BETA) {
  for (int e = threadIdx.x; e < kPwN * kMG; e += kThreads) {
    const int m = e % kMG, p = e / kMG - kPwLo;
    PW[e] = cpow_i(a.lam[w.h * a.M + w.m0 + m], p);
  }
  for (int m = threadIdx.x; m < kMG; m += kThreads) BETA[m] = a.beta[w.h * a.M + w.m0 + m];
}

// Floats of one stored chunk start state of a group: U (Re rows, Im rows) [kM2][F], G [kM2][D],
// e [kM2].
__device__ __forceinline__ size_t cks_floats(int F, int D) { return (size_t)kM2 * (F + D + 1); }

// ------------------------------------------------------------------ forward (recompute) sweep

template <int F, int D>
struct FwdLds {
  static constexpr int LF = F + 4, LD = D + 4;
  static constexpr int XQ = 0;
  static constexpr int XK = XQ + kC * LF;
  static constexpr int XV = XK + kC * LF;
  static constexpr int XD = XV + kC * LD;
  static constexpr int UC = XD + kC * LD;
  static constexpr int GC = UC + kM2 * LF;
  static constexpr int S1 = GC + kM2 * LD;
  static constexpr int SD1 = S1 + kC * LC;
  static constexpr int T0 = SD1 + kC * LC;
  static constexpr int T0D = T0 + kC * L2M;
  static constexpr int T2 = T0D + kC * L2M;
  static constexpr int T2D = T2 + kC * L2M;
  static constexpr int W0 = T2D + kC * L2M;      // [kC][L2M]: lam^(o-j), Re | Im
  static constexpr int AW0E = W0 + kC * L2M;     // [kM2][LC]: lam^(C-1-j), Re rows | Im rows
  static constexpr int EC = AW0E + kM2 * LC;     // [2][kMG] float2 (parity)
  static constexpr int PW = EC + 4 * kMG;        // [kPwN][kMG] float2
  static constexpr int BETA = PW + 2 * kPwN * kMG;
  static constexpr int E0T = BETA + 2 * kMG;     // [kC][kMG] float2: sum_{j<=i} lam^(i-j)
  static constexpr int floats = E0T + 2 * kC * kMG;
  static constexpr size_t bytes = (size_t)floats * 4;
};

// A chunk's rows of a [B][N][H][W] array (bf16 if BF, else fp32) as 16-byte vectors, PT per
// thread, held in registers between the load and the write into LDS; rows past N read as zero.
template <int W, bool BF>
struct Rows {
  static constexpr int E = BF ? 8 : 4;             // elements per vector
  static constexpr int VPR = W / E;                // vectors per row
  static constexpr int NV = kC * VPR;
  static constexpr int PT = (NV + kThreads - 1) / kThreads;
  uint4 r[PT];
  long long off0[PT];   // element offset of this thread's vector at walk position 0
  long long step;       // elements from one walk position to the next (negative backwards)

  // Offsets once per kernel; a chunk's fetch then adds its walk position times the step.
  __device__ __forceinline__ void init(const BwdArgs& a, const Wg& w) {
    step = (long long)(a.dir ? -1 : 1) * a.H * W;
#pragma unroll
    for (int p = 0; p < PT; ++p) {
      const int n = threadIdx.x + kThreads * p;
      off0[p] = (long long)row_index(a, w, 0, W) + (n % VPR) * E;
    }
  }
  __device__ __forceinline__ void fetch(const void* base, const BwdArgs& a, const Wg& w, int t0) {
#pragma unroll
    for (int p = 0; p < PT; ++p) {
      const int n = threadIdx.x + kThreads * p, i = n / VPR, t = t0 + i;
      r[p] = make_uint4(0u, 0u, 0u, 0u);
      if (n < NV && t < a.N)
        r[p] = *reinterpret_cast<const uint4*>(static_cast<const char*>(base) +
                                               (off0[p] + t * step) * (BF ? 2 : 4));
    }
  }
  // into X ([kC][ld] floats); fmap: the feature map (rows past N stay zero)
  __device__ __forceinline__ void put(float* X, int ld, int t0, int N, bool fmap, int opt) const {
#pragma unroll
    for (int p = 0; p < PT; ++p) {
      const int n = threadIdx.x + kThreads * p, i = n / VPR;
      if (n >= NV) continue;
      float v[E];
      const uint32_t u[4] = {r[p].x, r[p].y, r[p].z, r[p].w};
      if constexpr (BF) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[2 * e] = __uint_as_float(u[e] << 16);
          v[2 * e + 1] = __uint_as_float(u[e] & 0xffff0000u);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = __uint_as_float(u[e]);
      }
      if (fmap) {
        const bool ok = t0 + i < N;
#pragma unroll
        for (int e = 0; e < E; ++e) v[e] = ok ? feat(v[e], opt) : 0.f;
      }
      float* dst = X + i * ld + (n % VPR) * E;
#pragma unroll
      for (int e = 0; e < E; e += 4)
        *reinterpret_cast<float4*>(dst + e) = make_float4(v[e], v[e + 1], v[e + 2], v[e + 3]);
    }
  }
};

// The four token-row inputs of a chunk: q, k, v (bf16 if BI) and dL/do (bf16 if BO).
template <int F, int D, bool BI, bool BO>
struct ChunkRows {
  Rows<F, BI> q, k;
  Rows<D, BI> v;
  Rows<D, BO> g;
  __device__ __forceinline__ void init(const BwdArgs& a, const Wg& w) {
    q.init(a, w);
    k.init(a, w);
    v.init(a, w);
    g.init(a, w);
  }
  __device__ __forceinline__ void fetch(const BwdArgs& a, const Wg& w, int t0) {
    q.fetch(a.q, a, w, t0);
    k.fetch(a.k, a, w, t0);
    v.fetch(a.v, a, w, t0);
    g.fetch(a.dO, a, w, t0);
  }
  __device__ __forceinline__ void put(const BwdArgs& a, int t0, float* XQ, float* XK, float* XV,
                                      float* XG) const {
    q.put(XQ, F + 4, t0, a.N, true, a.opt);
    k.put(XK, F + 4, t0, a.N, true, a.opt);
    v.put(XV, D + 4, t0, a.N, false, 0);
    g.put(XG, D + 4, t0, a.N, false, 0);
  }
};

template <int F, int D, bool BI, bool BO>
__global__ void __launch_bounds__(kThreads) bwdc_forward_kernel(const BwdArgs a) {
  using L = FwdLds<F, D>;
  constexpr int LF = L::LF, LD = L::LD;
  extern __shared__ __align__(16) float sm[];
  float *XQ = sm + L::XQ, *XK = sm + L::XK, *XV = sm + L::XV, *XD = sm + L::XD;
  float *UC = sm + L::UC, *GC = sm + L::GC;
  float *S1 = sm + L::S1, *SD1 = sm + L::SD1, *T0 = sm + L::T0, *T0D = sm + L::T0D;
  float *T2 = sm + L::T2, *T2D = sm + L::T2D, *W0 = sm + L::W0, *AW0E = sm + L::AW0E;
  float2* EC = reinterpret_cast<float2*>(sm + L::EC);
  float2* PW = reinterpret_cast<float2*>(sm + L::PW);
  float2* BETA = reinterpret_cast<float2*>(sm + L::BETA);
  float2* E0T = reinterpret_cast<float2*>(sm + L::E0T);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const Wg w = wg_of(a);
  const int groups = a.M / kMG;
  const int nch = (a.N + kC - 1) / kC;

  build_powers(a, w, PW, BETA);
  // initial state (the caller's, or zeros), planar
  for (int e = tid; e < kMG * F; e += kThreads) {
    const int m = e / F, f = e % F;
    float2 u = make_float2(0.f, 0.f);
    if (a.U0) u = a.U0[((size_t)w.slice * a.M + w.m0 + m) * F + f];
    UC[m * LF + f] = u.x;
    UC[(kMG + m) * LF + f] = u.y;
  }
  for (int e = tid; e < kMG * D; e += kThreads) {
    const int m = e / D, d = e % D;
    float2 g = make_float2(0.f, 0.f);
    if (a.G0) g = a.G0[((size_t)w.slice * a.M + w.m0 + m) * D + d];
    GC[m * LD + d] = g.x;
    GC[(kMG + m) * LD + d] = g.y;
  }
  if (tid < kMG) EC[tid] = a.E0 ? a.E0[(size_t)w.slice * a.M + w.m0 + tid] : make_float2(0.f, 0.f);
  __syncthreads();
  // tables from the powers
  for (int e = tid; e < kC * kMG; e += kThreads) {
    const int j = e / kMG, m = e % kMG;
    const float2 p = PW[(kO - j + kPwLo) * kMG + m];
    W0[j * L2M + m] = p.x;
    W0[j * L2M + kMG + m] = p.y;
    const float2 pe = PW[(kC - 1 - j + kPwLo) * kMG + m];
    AW0E[m * LC + j] = pe.x;
    AW0E[(kMG + m) * LC + j] = pe.y;
  }
  if (tid < kMG) {
    double sr = 0.0, si = 0.0;
    for (int i = 0; i < kC; ++i) {
      const float2 p = PW[(i + kPwLo) * kMG + tid];
      sr += p.x;
      si += p.y;
      E0T[i * kMG + tid] = make_float2((float)sr, (float)si);
    }
  }
  float2* cks_base = reinterpret_cast<float2*>(a.ckpt);
  float* cks = reinterpret_cast<float*>(cks_base) +
               ((size_t)w.slice * groups + w.group) * nch * cks_floats(F, D);

  // start state of chunk cc (U, G planar in LDS, e in EC[par]) into its workspace block, by half
  // the workgroup (t: the thread's index among them; threads with t outside [0, nt) return)
  auto store_state = [&](int cc, int par, int t) {
    constexpr int nt = kThreads / 2;
    if (t < 0 || t >= nt) return;
    float* dst = cks + (size_t)cc * cks_floats(F, D);
    for (int e = 4 * t; e < kM2 * F; e += 4 * nt)
      *reinterpret_cast<float4*>(dst + e) =
          *reinterpret_cast<const float4*>(UC + (e / F) * LF + e % F);
    for (int e = 4 * t; e < kM2 * D; e += 4 * nt)
      *reinterpret_cast<float4*>(dst + kM2 * F + e) =
          *reinterpret_cast<const float4*>(GC + (e / D) * LD + e % D);
    if (t < kMG) {
      dst[kM2 * (F + D) + t] = EC[par * kMG + t].x;
      dst[kM2 * (F + D) + kMG + t] = EC[par * kMG + t].y;
    }
  };
  // chunk c's rows arrive in registers one chunk ahead and stay in flight across its compute
  ChunkRows<F, D, BI, BO> rows;
  rows.init(a, w);
  rows.fetch(a, w, 0);
  for (int c = 0; c < nch; ++c) {
    const int t0 = c * kC, par = c & 1;
    rows.put(a, t0, XQ, XK, XV, XD);
    if (c + 1 < nch) rows.fetch(a, w, t0 + kC);
    __syncthreads();
    // ---- phase B: S, S_d, T2, T2_d, and the chunk's state contributions (kept in registers
    // until the update); chunk 0's start state is stored here, every later one in the previous
    // chunk's phase D
    if (c == 0) store_state(0, 0, tid);
    // big tiles: 0 S, 1 S_d, 2-3 T2, 4-5 T2_d
    if (wv < 6) {
      f4 acc = zero4();
      if (wv == 0) {
        tile_mma<F, true, true, true>(acc, XQ, LF, XK, LF, lane);
      } else if (wv == 1) {
        tile_mma<D, true, true, true>(acc, XD, LD, XV, LD, lane);
      } else if (wv < 4) {
        tile_mma<F, true, true, true>(acc, XQ, LF, UC + 16 * (wv - 2) * LF, LF, lane);
      } else {
        tile_mma<D, true, true, true>(acc, XD, LD, GC + 16 * (wv - 4) * LD, LD, lane);
      }
      const int col = acc_col(lane);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = acc_row(lane, r);
        if (wv < 2) {
          (wv == 0 ? S1 : SD1)[row * LC + col] = col <= row ? acc[r] : 0.f;
        } else if (wv < 4) {
          T2[row * L2M + 16 * (wv - 2) + col] = acc[r];
        } else {
          T2D[row * L2M + 16 * (wv - 4) + col] = acc[r];
        }
      }
    }
    // state contributions: tile pairs (Re rows, Im rows) of K0 = lam^(C-1-j) phi(K) (F/16
    // column blocks) and V0 = lam^(C-1-j) V (D/16)
    constexpr int NPAIR = F / 16 + D / 16;
    constexpr int PPW = (NPAIR + kWaves - 1) / kWaves;
    f4 kre[PPW], kim[PPW];
#pragma unroll
    for (int p = 0; p < PPW; ++p) {
      const int pr = wv + kWaves * p;
      kre[p] = zero4();
      kim[p] = zero4();
      if (pr < F / 16) {
        tile_mma<kC, true, false, true>(kre[p], AW0E, LC, XK + 16 * pr, LF, lane);
        tile_mma<kC, true, false, true>(kim[p], AW0E + kMG * LC, LC, XK + 16 * pr, LF, lane);
      } else if (pr < NPAIR) {
        const int dc = pr - F / 16;
        tile_mma<kC, true, false, true>(kre[p], AW0E, LC, XV + 16 * dc, LD, lane);
        tile_mma<kC, true, false, true>(kim[p], AW0E + kMG * LC, LC, XV + 16 * dc, LD, lane);
      }
    }
    __syncthreads();
    // ---- phase C: T0 = S W0, T0_d = S_d W0; the state update
    if (wv < 4) {
      f4 acc = zero4();
      const float* Sx = wv < 2 ? S1 : SD1;
      const int nb = 16 * (wv & 1);
      tile_mma<kC, true, false, true>(acc, Sx, LC, W0 + nb, L2M, lane);
      float* Tx = wv < 2 ? T0 : T0D;
      const int col = acc_col(lane);
#pragma unroll
      for (int r = 0; r < 4; ++r) Tx[acc_row(lane, r) * L2M + nb + col] = acc[r];
    }
#pragma unroll
    for (int p = 0; p < PPW; ++p) {
      const int pr = wv + kWaves * p;
      if (pr < NPAIR) {
        const bool isu = pr < F / 16;
        float* X = isu ? UC : GC;
        const int ld = isu ? LF : LD;
        const int col = 16 * (isu ? pr : pr - F / 16) + acc_col(lane);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = acc_row(lane, r);
          const float2 x = make_float2(X[m * ld + col], X[(kMG + m) * ld + col]);
          const float2 nx = cadd2(cmul(PW[(kC + kPwLo) * kMG + m], x),
                                  cmul(BETA[m], make_float2(kre[p][r], kim[p][r])));
          X[m * ld + col] = nx.x;
          X[(kMG + m) * ld + col] = nx.y;
        }
      }
    }
    if (tid < kMG)
      EC[(par ^ 1) * kMG + tid] = cadd2(cmul(PW[(kC + kPwLo) * kMG + tid], EC[par * kMG + tid]),
                                       cmul(BETA[tid], E0T[(kC - 1) * kMG + tid]));
    __syncthreads();
    // ---- phase D: per (token i, mode m) the readout terms, summed over the group's modes
    // (waves 0-3); waves 4-7 store the updated state, the next chunk's start state
    if (c + 1 < nch) store_state(c + 1, par ^ 1, tid - kThreads / 2);
    if (tid < kC * kMG) {
      const int i = tid >> 4, m = tid & 15;
      const float2 li = PW[(i - kO + kPwLo) * kMG + m], l1 = PW[(i + 1 + kPwLo) * kMG + m];
      const float2 b = BETA[m];
      const float2 t0v = make_float2(T0[i * L2M + m], T0[i * L2M + kMG + m]);
      const float2 t0d = make_float2(T0D[i * L2M + m], T0D[i * L2M + kMG + m]);
      const float2 t2 = make_float2(T2[i * L2M + m], T2[i * L2M + kMG + m]);
      const float2 t2d = make_float2(T2D[i * L2M + m], T2D[i * L2M + kMG + m]);
      const float2 av = cadd2(cmul(b, cmul(li, t0v)), cmul(l1, t2));       // a_i
      const float2 xv = cadd2(cmul(b, cmul(li, t0d)), cmul(l1, t2d));      // dL/do_i . G_i
      const float2 ev = cadd2(cmul(l1, EC[par * kMG + m]), cmul(b, E0T[i * kMG + m]));   // e_i
      float den = av.x * ev.x - av.y * ev.y;
      float gn = av.x * xv.x - av.y * xv.y;
      row16_sum2(den, gn);
      const int t = t0 + i;
      if (m == 0 && t < a.N)
        a.dpart[((size_t)w.slice * a.N + t) * groups + w.group] = make_float2(den, gn);
    }
  }
}

// ------------------------------------------------------------------ reverse sweep

template <int F, int D>
struct RevLds {
  static constexpr int LF = F + 4, LD = D + 4;
  // [XQ; SU], [XK; UC], [XG; SG] adjacent: the B operands of dphi(k), dphi(q), dv
  static constexpr int XQ = 0;
  static constexpr int SU = XQ + kC * LF;
  static constexpr int XK = SU + kM2 * LF;
  static constexpr int UC = XK + kC * LF;
  static constexpr int XG = UC + kM2 * LF;
  static constexpr int SG = XG + kC * LD;
  static constexpr int XV = SG + kM2 * LD;
  static constexpr int GC = XV + kC * LD;
  static constexpr int S1 = GC + kM2 * LD;
  static constexpr int SG1 = S1 + kC * LC;
  static constexpr int T01 = SG1 + kC * LC;      // [kC][L4M]: T0 Re | Im, T1 Re | Im
  static constexpr int T01G = T01 + kC * L4M;
  static constexpr int T2 = T01G + kC * L4M;     // [kC][L2M]
  static constexpr int T2G = T2 + kC * L2M;
  static constexpr int Z = T2G + kC * L2M;       // [kM2][LC]
  static constexpr int ZG = Z + kM2 * LC;
  static constexpr int APA = ZG + kM2 * LC;      // [kC][L2M]
  static constexpr int APG = APA + kC * L2M;
  static constexpr int AQ = APG + kC * L2M;      // [kC][LA]
  static constexpr int AK = AQ + kC * LA;
  static constexpr int AV = AK + kC * LA;
  static constexpr int AYU = AV + kC * LA;       // [kM2][LC]
  static constexpr int AYG = AYU + kM2 * LC;
  static constexpr int W01 = AYG + kM2 * LC;     // [kC][L4M]: lam^(o-j) Re | Im, j lam^(o-j) Re | Im
  static constexpr int WT = W01 + kC * L4M;      // [kC][L2M]: beta lam^(o-j) Re | Im
  static constexpr int PW = WT + kC * L2M;       // [kPwN][kMG] float2
  static constexpr int BETA = PW + 2 * kPwN * kMG;
  static constexpr int EC = BETA + 2 * kMG;      // [kMG] float2
  static constexpr int SE = EC + 2 * kMG;        // [2][kMG] float2 (parity)
  static constexpr int CT = SE + 4 * kMG;        // [kC]: 1 / c_t
  static constexpr int DD = CT + kC;             // [kC]: dd_t
  static constexpr int LSUM = DD + kC;           // [kMG] float2 x 2: dlam, dbeta of waves 4-7
  static constexpr int floats = LSUM + 4 * kMG;
  static constexpr size_t bytes = (size_t)floats * 4;
};

template <int F, int D, bool BI, bool BO>
__global__ void __launch_bounds__(kThreads) bwdc_reverse_kernel(const BwdArgs a) {
  using L = RevLds<F, D>;
  constexpr int LF = L::LF, LD = L::LD;
  extern __shared__ __align__(16) float sm[];
  float *XQ = sm + L::XQ, *SU = sm + L::SU, *XK = sm + L::XK, *UC = sm + L::UC;
  float *XG = sm + L::XG, *SG = sm + L::SG, *XV = sm + L::XV, *GC = sm + L::GC;
  float *S1 = sm + L::S1, *SG1 = sm + L::SG1, *T01 = sm + L::T01, *T01G = sm + L::T01G;
  float *T2 = sm + L::T2, *T2G = sm + L::T2G, *Z = sm + L::Z, *ZG = sm + L::ZG;
  float *APA = sm + L::APA, *APG = sm + L::APG, *AQ = sm + L::AQ, *AK = sm + L::AK;
  float *AV = sm + L::AV, *AYU = sm + L::AYU, *AYG = sm + L::AYG, *W01 = sm + L::W01;
  float* WT = sm + L::WT;
  float2* PW = reinterpret_cast<float2*>(sm + L::PW);
  float2* BETA = reinterpret_cast<float2*>(sm + L::BETA);
  float2* EC = reinterpret_cast<float2*>(sm + L::EC);
  float2* SE = reinterpret_cast<float2*>(sm + L::SE);
  float *CT = sm + L::CT, *DD = sm + L::DD;
  float2* LSUM = reinterpret_cast<float2*>(sm + L::LSUM);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const Wg w = wg_of(a);
  const int groups = a.M / kMG;
  const int nch = (a.N + kC - 1) / kC;
  const int W = 2 * F + D;
  const size_t S = (size_t)a.B * a.H;
  const bool no_den = a.opt & kOptNoDen, ident = a.opt & kOptIdentity;

  build_powers(a, w, PW, BETA);
  for (int e = tid; e < kM2 * LF; e += kThreads) SU[e] = 0.f;
  for (int e = tid; e < kM2 * LD; e += kThreads) SG[e] = 0.f;
  if (tid < 2 * kMG) SE[tid] = make_float2(0.f, 0.f);
  __syncthreads();
  for (int e = tid; e < kC * kMG; e += kThreads) {
    const int j = e / kMG, m = e % kMG;
    const float2 p = PW[(kO - j + kPwLo) * kMG + m];
    W01[j * L4M + m] = p.x;
    W01[j * L4M + kMG + m] = p.y;
    W01[j * L4M + kM2 + m] = j * p.x;
    W01[j * L4M + kM2 + kMG + m] = j * p.y;
    const float2 wb = cmul(BETA[m], p);
    WT[j * L2M + m] = wb.x;
    WT[j * L2M + kMG + m] = wb.y;
    const float2 we = cmul(BETA[m], PW[(kC - 1 - j + kPwLo) * kMG + m]);
    AK[j * LA + kC + m] = we.x;
    AK[j * LA + kC + kMG + m] = we.y;
    AV[j * LA + kC + m] = we.x;
    AV[j * LA + kC + kMG + m] = we.y;
  }

  // per-thread (token i, mode m) accumulators of dlam and dbeta: thread m*16 + i
  const int em = tid >> 4, ei = tid & 15;
  float2 dlam = make_float2(0.f, 0.f), dbet = make_float2(0.f, 0.f);

  const float* cks = reinterpret_cast<const float*>(a.ckpt) +
                     ((size_t)w.slice * groups + w.group) * nch * cks_floats(F, D);
  float* gp = a.gpart + (size_t)w.group * S * a.N * W + (size_t)w.slice * a.N * W;

  // Y tile pairs of the adjoint update, kept in registers across the barrier after phase F
  constexpr int NYP = F / 16 + D / 16;
  constexpr int YPW = (NYP + kWaves - 1) / kWaves;

  // Chunk c's rows, start state and den partials arrive in registers one chunk ahead.
  constexpr int NS4 = kM2 * (F + D) / 4;                 // float4s of U and G per stored state
  constexpr int PTS = (NS4 + kThreads - 1) / kThreads;
  constexpr int kMaxGroups = kMaxModes / kMG;
  static_assert(kMaxGroups <= 8, "den partials staged 8 groups per token");
  ChunkRows<F, D, BI, BO> rows;
  float4 sv[PTS];
  float2 ev = make_float2(0.f, 0.f), dp = make_float2(0.f, 0.f);
  auto fetch = [&](int c) {
    const int t0 = c * kC;
    rows.fetch(a, w, t0);
    const float* src = cks + (size_t)c * cks_floats(F, D);
#pragma unroll
    for (int p = 0; p < PTS; ++p) {
      const int n = tid + kThreads * p;
      sv[p] = n < NS4 ? reinterpret_cast<const float4*>(src)[n] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    if (tid < kMG) ev = make_float2(src[kM2 * (F + D) + tid], src[kM2 * (F + D) + kMG + tid]);
    if (tid < kC * 8) {   // token tid / 8, group tid % 8 (groups <= 8)
      const int t = t0 + (tid >> 3), g = tid & 7;
      dp = g < groups && t < a.N ? a.dpart[((size_t)w.slice * a.N + t) * groups + g]
                                 : make_float2(0.f, 0.f);
    }
  };
  rows.init(a, w);
  f4 yre[YPW], yim[YPW];
  // S^U <- conj(lam^C) S^U + conj(Y_U), S^G likewise, from the Y tiles of the chunk just done
  auto update_adjoints = [&]() {
#pragma unroll
    for (int p = 0; p < YPW; ++p) {
      const int pr = wv + kWaves * p;
      if (pr < NYP) {
        const bool isu = pr < F / 16;
        float* X = isu ? SU : SG;
        const int ld = isu ? LF : LD;
        const int col = 16 * (isu ? pr : pr - F / 16) + acc_col(lane);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = acc_row(lane, r);
          const float2 x = make_float2(X[m * ld + col], X[(kMG + m) * ld + col]);
          const float2 nx = cadd2(cmulc2(x, PW[(kC + kPwLo) * kMG + m]),
                                  make_float2(yre[p][r], -yim[p][r]));
          X[m * ld + col] = nx.x;
          X[(kMG + m) * ld + col] = nx.y;
        }
      }
    }
  };

  fetch(nch - 1);
  for (int c = nch - 1; c >= 0; --c) {
    const int t0 = c * kC, par = c & 1;
    // ---- phase A: the adjoint update of chunk c+1; chunk c's inputs, start state, 1/c_t and
    // dd_t into LDS; chunk c-1's loads issued
    if (c + 1 < nch) update_adjoints();
    rows.put(a, t0, XQ, XK, XV, XG);   // XG: dL/do, scaled by 1/c_t in phase C
#pragma unroll
    for (int p = 0; p < PTS; ++p) {
      const int e = 4 * (tid + kThreads * p);
      if (e < kM2 * F)
        *reinterpret_cast<float4*>(UC + (e / F) * LF + e % F) = sv[p];
      else if (e < kM2 * (F + D))
        *reinterpret_cast<float4*>(GC + ((e - kM2 * F) / D) * LD + (e - kM2 * F) % D) = sv[p];
    }
    if (tid < kMG) EC[tid] = ev;
    if (tid < kC * 8) {   // 1/c_t and dd_t: the groups' partials of token tid / 8 summed
      float den = dp.x, gn = dp.y;
#pragma unroll
      for (int off = 4; off > 0; off >>= 1) {
        den += __shfl_xor(den, off, 64);
        gn += __shfl_xor(gn, off, 64);
      }
      const int i = tid >> 3;
      if ((tid & 7) == 0) {
        float inv = 0.f, dd = 0.f;
        if (t0 + i < a.N) {
          if (no_den) {
            inv = 1.f;
          } else {
            const float cc = clamp_den(den, a.clamp);
            inv = 1.f / cc;
            dd = den >= a.clamp ? -gn * inv * inv : 0.f;
          }
        }
        CT[i] = inv;
        DD[i] = dd;
      }
    }
    if (c > 0) fetch(c - 1);
    __syncthreads();
    // ---- phase B: S, S', T2, T2', Z, Z' (K = F or D)
    for (int tk = wv; tk < 10; tk += kWaves) {
      f4 acc = zero4();
      if (tk == 0) tile_mma<F, true, true, true>(acc, XQ, LF, XK, LF, lane);
      else if (tk == 1) tile_mma<D, true, true, true>(acc, XG, LD, XV, LD, lane);
      else if (tk < 4) tile_mma<F, true, true, true>(acc, XQ, LF, UC + 16 * (tk - 2) * LF, LF, lane);
      else if (tk < 6) tile_mma<D, true, true, true>(acc, XG, LD, GC + 16 * (tk - 4) * LD, LD, lane);
      else if (tk < 8) tile_mma<F, true, true, true>(acc, SU + 16 * (tk - 6) * LF, LF, XK, LF, lane);
      else tile_mma<D, true, true, true>(acc, SG + 16 * (tk - 8) * LD, LD, XV, LD, lane);
      const int col = acc_col(lane);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = acc_row(lane, r);
        if (tk == 0) S1[row * LC + col] = col <= row ? acc[r] : 0.f;
        else if (tk == 1) SG1[row * LC + col] = col <= row ? CT[row] * acc[r] + DD[row] : 0.f;
        else if (tk < 4) T2[row * L2M + 16 * (tk - 2) + col] = acc[r];
        else if (tk < 6) T2G[row * L2M + 16 * (tk - 4) + col] = CT[row] * acc[r];
        else if (tk < 8) Z[(16 * (tk - 6) + row) * LC + col] = acc[r];
        else ZG[(16 * (tk - 8) + row) * LC + col] = acc[r];
      }
    }
    __syncthreads();
    // ---- phase C: T01 = S W01, T01' = S' W01 (K = C); the rows of G scaled to dL/do / c_t
    for (int e = 4 * tid; e < kC * D; e += 4 * kThreads) {
      float4* x = reinterpret_cast<float4*>(XG + (e / D) * LD + e % D);
      const float sc = CT[e / D];
      const float4 y = *x;
      *x = make_float4(sc * y.x, sc * y.y, sc * y.z, sc * y.w);
    }
    {
      const float* Sx = wv < 4 ? S1 : SG1;
      float* Tx = wv < 4 ? T01 : T01G;
      const int nb = 16 * (wv & 3);
      f4 acc = zero4();
      tile_mma<kC, true, false>(acc, Sx, LC, W01 + nb, L4M, lane);
      const int col = acc_col(lane);
#pragma unroll
      for (int r = 0; r < 4; ++r) Tx[acc_row(lane, r) * L4M + nb + col] = acc[r];
    }
    __syncthreads();
    // ---- phase D: per (token i, mode m); waves 0-3 the readout terms, waves 4-7 the terms of
    // the carried adjoints
    if (tid < kC * kMG) {
      const int i = ei, m = em;
      const float2 li = PW[(i - kO + kPwLo) * kMG + m], l1 = PW[(i + 1 + kPwLo) * kMG + m];
      const float2 li0 = PW[(i + kPwLo) * kMG + m], lq1 = PW[(i - 1 - kO + kPwLo) * kMG + m];
      const float2 b = BETA[m];
      const float2 t0v = make_float2(T01[i * L4M + m], T01[i * L4M + kMG + m]);
      const float2 t1v = make_float2(T01[i * L4M + kM2 + m], T01[i * L4M + kM2 + kMG + m]);
      const float2 t0g = make_float2(T01G[i * L4M + m], T01G[i * L4M + kMG + m]);
      const float2 t1g = make_float2(T01G[i * L4M + kM2 + m], T01G[i * L4M + kM2 + kMG + m]);
      const float2 t2 = make_float2(T2[i * L2M + m], T2[i * L2M + kMG + m]);
      const float2 ecm = EC[m];
      const float ddi = DD[i];
      const float2 t2g =
          cadd2(make_float2(T2G[i * L2M + m], T2G[i * L2M + kMG + m]), csc(ddi, ecm));
      const float2 E = cmul(li, t0v), Eg = cmul(li, t0g);
      const float2 av = cadd2(cmul(b, E), cmul(l1, t2));     // a_i
      const float2 Ag = cadd2(cmul(b, Eg), cmul(l1, t2g));   // A_i
      const float2 La = cmul(li, av), LAg = cmul(li, Ag);
      APA[i * L2M + m] = La.x;
      APA[i * L2M + kMG + m] = -La.y;
      APG[i * L2M + m] = LAg.x;
      APG[i * L2M + kMG + m] = -LAg.y;
      const float2 l1A = cmul(l1, Ag), l1a = cmul(l1, av);
      AQ[i * LA + kC + m] = l1A.x;
      AQ[i * LA + kC + kMG + m] = -l1A.y;
      AYU[m * LC + i] = l1A.x;
      AYU[(kMG + m) * LC + i] = l1A.y;
      AYG[m * LC + i] = l1a.x;
      AYG[(kMG + m) * LC + i] = l1a.y;
      // dbeta: sum_i conj(A_i E_i + a_i E'_i)
      dbet = cadd2(dbet, cconj(cadd2(cmul(Ag, E), cmul(av, Eg))));
      // dlam, within the chunk: conj(beta A_i D1_i + beta a_i D1'_i + (i+1) lam^i (A_i T2_i +
      // a_i T2'_i))
      const float fi = (float)i;
      const float2 D1 = cmul(lq1, make_float2(fi * t0v.x - t1v.x, fi * t0v.y - t1v.y));
      const float2 D1g = cmul(lq1, make_float2(fi * t0g.x - t1g.x, fi * t0g.y - t1g.y));
      float2 sx = cmul(b, cadd2(cmul(Ag, D1), cmul(av, D1g)));
      sx = cadd2(sx, csc(fi + 1.f, cmul(li0, cadd2(cmul(Ag, t2), cmul(av, t2g)))));
      dlam = cadd2(dlam, cconj(sx));
      // the eta adjoint: S^e <- conj(lam^C) S^e + conj(sum_i lam^(i+1) a_i dd_i)
      const float2 sev = SE[par * kMG + m];
      float sr = ddi * l1a.x, si = ddi * l1a.y;
      row16_sum2(sr, si);
      if (i == 0)
        SE[(par ^ 1) * kMG + m] =
            cadd2(cmulc2(sev, PW[(kC + kPwLo) * kMG + m]), make_float2(sr, -si));
    } else {
      const int i = ei, m = em - kMG;
      const float2 b = BETA[m];
      // carried adjoints, token j = i: Z[m,j] = S^U . phi(k_j), Z'[m,j] = S^G . v_j + S^e
      const float2 sev = SE[par * kMG + m];
      const float2 zz = cadd2(make_float2(Z[m * LC + i], Z[(kMG + m) * LC + i]),
                              cadd2(make_float2(ZG[m * LC + i], ZG[(kMG + m) * LC + i]), sev));
      dbet = cadd2(dbet, cmulc2(zz, PW[(kC - 1 - i + kPwLo) * kMG + m]));
      // dlam: (C-1-j) conj(beta lam^(C-2-j)) Z_total[m,j] and C conj(lam^(C-1)) (S^U . conj(U_c)
      // + S^G . conj(G_c) + S^e conj(e_c)), the dot products spread over the mode's 16 threads
      float2 sx = make_float2(0.f, 0.f);
      if (i < kC - 1)
        sx = csc((float)(kC - 1 - i),
                 cconj(cmul(cconj(zz), cmul(b, PW[(kC - 2 - i + kPwLo) * kMG + m]))));
      float2 dotv = make_float2(0.f, 0.f);
#pragma unroll 2
      for (int f = i; f < F; f += 16)
        dotv = cadd2(dotv, cmulc2(make_float2(SU[m * LF + f], SU[(kMG + m) * LF + f]),
                                  make_float2(UC[m * LF + f], UC[(kMG + m) * LF + f])));
#pragma unroll 2
      for (int d = i; d < D; d += 16)
        dotv = cadd2(dotv, cmulc2(make_float2(SG[m * LD + d], SG[(kMG + m) * LD + d]),
                                  make_float2(GC[m * LD + d], GC[(kMG + m) * LD + d])));
      if (i == 0) dotv = cadd2(dotv, cmulc2(sev, EC[m]));
      dlam = cadd2(dlam, cadd2(sx, csc((float)kC, cmulc2(dotv, PW[(kC - 1 + kPwLo) * kMG + m]))));
    }
    __syncthreads();
    // ---- phase E: P and Pg (K = 2 MG), causal, into the operands of phase F
    if (wv < 2) {
      f4 acc = zero4();
      tile_mma<kM2, true, true>(acc, wv == 0 ? APA : APG, L2M, WT, L2M, lane);
      const int col = acc_col(lane);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = acc_row(lane, r);   // i = row, j = col
        const float x = col <= row ? acc[r] : 0.f;
        if (wv == 0) {
          AV[col * LA + row] = x;
        } else {
          AQ[row * LA + col] = x;
          AK[col * LA + row] = x;
        }
      }
    }
    __syncthreads();
    // ---- phase F: dphi(q) = AQ [phi(K); UC], dphi(k) = AK [phi(Q); SU], dv = AV [G; SG]
    // (K = C + 2 MG), and the adjoint updates Y_U = AYU phi(Q), Y_G = AYG G (K = C)
    constexpr int NT = 2 * (F / 16) + D / 16;
    for (int tk = wv; tk < NT; tk += kWaves) {
      f4 acc = zero4();
      int col0, kind;
      if (tk < F / 16) {
        kind = 0;
        col0 = 16 * tk;
        tile_mma<kC + kM2, true, false, true>(acc, AQ, LA, XK + col0, LF, lane);
      } else if (tk < 2 * (F / 16)) {
        kind = 1;
        col0 = 16 * (tk - F / 16);
        tile_mma<kC + kM2, true, false, true>(acc, AK, LA, XQ + col0, LF, lane);
      } else {
        kind = 2;
        col0 = 16 * (tk - 2 * (F / 16));
        tile_mma<kC + kM2, true, false, true>(acc, AV, LA, XG + col0, LD, lane);
      }
      const int col = col0 + acc_col(lane);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = acc_row(lane, r), t = t0 + i;
        float x = acc[r];
        if (kind == 0 && !ident) x *= fminf(1.f, XQ[i * LF + col]);
        if (kind == 1 && !ident) x *= fminf(1.f, XK[i * LF + col]);
        if (t < a.N) gp[(size_t)t * W + (kind == 0 ? 0 : kind == 1 ? F : 2 * F) + col] = x;
      }
    }
#pragma unroll
    for (int p = 0; p < YPW; ++p) {
      const int pr = wv + kWaves * p;
      yre[p] = zero4();
      yim[p] = zero4();
      if (pr < F / 16) {
        tile_mma<kC, true, false>(yre[p], AYU, LC, XQ + 16 * pr, LF, lane);
        tile_mma<kC, true, false>(yim[p], AYU + kMG * LC, LC, XQ + 16 * pr, LF, lane);
      } else if (pr < NYP) {
        const int dc = pr - F / 16;
        tile_mma<kC, true, false>(yre[p], AYG, LC, XG + 16 * dc, LD, lane);
        tile_mma<kC, true, false>(yim[p], AYG + kMG * LC, LC, XG + 16 * dc, LD, lane);
      }
    }
    __syncthreads();
  }
  update_adjoints();   // chunk 0's
  __syncthreads();

  // gradient of the initial state: the adjoints left after chunk 0
  if (a.dU0) {
    for (int e = tid; e < kMG * F; e += kThreads) {
      const int m = e / F, f = e % F;
      a.dU0[((size_t)w.slice * a.M + w.m0 + m) * F + f] =
          make_float2(SU[m * LF + f], SU[(kMG + m) * LF + f]);
    }
    for (int e = tid; e < kMG * D; e += kThreads) {
      const int m = e / D, d = e % D;
      a.dG0[((size_t)w.slice * a.M + w.m0 + m) * D + d] =
          make_float2(SG[m * LD + d], SG[(kMG + m) * LD + d]);
    }
    // chunk 0 (parity 0) wrote the eta adjoint into parity slot 1
    if (tid < kMG) a.dE0[(size_t)w.slice * a.M + w.m0 + tid] = SE[kMG + tid];
  }
  // dlam, dbeta: sum over the 16 token threads of each mode, then over the two wave halves
  {
    float lr = dlam.x, lim = dlam.y, br = dbet.x, bim = dbet.y;
    row16_sum2(lr, lim);
    row16_sum2(br, bim);
    if (ei == 0 && tid >= kC * kMG) {
      LSUM[em - kMG] = make_float2(lr, lim);
      LSUM[em] = make_float2(br, bim);
    }
    __syncthreads();
    if (ei == 0 && tid < kC * kMG) {
      const size_t i = (size_t)w.slice * a.M + w.m0 + em;
      a.lpart[2 * i] = cadd2(make_float2(lr, lim), LSUM[em]);
      a.lpart[2 * i + 1] = cadd2(make_float2(br, bim), LSUM[kMG + em]);
    }
  }
}

hipError_t allow_lds_c(const void* kernel, size_t bytes, size_t& allowed) {
  if (bytes <= allowed) return hipSuccess;
  hipError_t e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)bytes);
  if (e == hipSuccess) allowed = bytes;
  return e;
}

template <int F, int D, bool BI, bool BO>
hipError_t launch_bwdc(const BwdArgs& a, hipStream_t st) {
  static size_t allowed_f = 65536, allowed_r = 65536;
  const size_t lf = FwdLds<F, D>::bytes, lr = RevLds<F, D>::bytes;
  hipError_t e = allow_lds_c(reinterpret_cast<const void*>(&bwdc_forward_kernel<F, D, BI, BO>),
                             lf, allowed_f);
  if (e == hipSuccess)
    e = allow_lds_c(reinterpret_cast<const void*>(&bwdc_reverse_kernel<F, D, BI, BO>), lr,
                    allowed_r);
  if (e != hipSuccess) return e;
  const unsigned grid = (unsigned)((size_t)a.B * a.H * (a.M / kMG));
  prof_begin(st);
  hipLaunchKernelGGL((bwdc_forward_kernel<F, D, BI, BO>), dim3(grid), dim3(kThreads), lf, st, a);
  prof_end(st, kKindBwdForward);
  prof_begin(st);
  hipLaunchKernelGGL((bwdc_reverse_kernel<F, D, BI, BO>), dim3(grid), dim3(kThreads), lr, st, a);
  prof_end(st, kKindBwdReverse);
  return hipGetLastError();
}

template <int F>
hipError_t launch_bwdc_f(const BwdArgs& a, hipStream_t st) {
  if (a.in_bf16) return a.out_bf16 ? launch_bwdc<F, F, true, true>(a, st)
                                   : launch_bwdc<F, F, true, false>(a, st);
  return a.out_bf16 ? launch_bwdc<F, F, false, true>(a, st)
                    : launch_bwdc<F, F, false, false>(a, st);
}

}  // namespace

bool bwd_chunked_supported(int F, int D, int M) {
  return F == D && (F == 32 || F == 64 || F == 128) && M % kMG == 0;
}

BwdLayout bwd_chunked_layout(int B, int H, int N, int F, int D, int M) {
  auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
  const size_t S = (size_t)B * H;
  const size_t nch = ((size_t)N + kC - 1) / kC;
  const size_t groups = (size_t)M / kMG;
  BwdLayout l{};
  l.ckpt_off = 0;
  l.dpart_off = up(S * groups * nch * kM2 * (F + D + 1) * 4);
  l.gpart_off = l.dpart_off + up(S * N * groups * 8);
  l.lpart_off = l.gpart_off + up(groups * S * N * (2 * F + D) * 4);
  l.apart_off = l.lpart_off + up(S * M * 2 * 8);
  l.cstate_off = l.cadj_off = l.bytes = l.apart_off;
  return l;
}

hipError_t launch_prefill_bwd_chunked(const BwdArgs& a, hipStream_t st) {
  (void)hipGetLastError();
  hipError_t e = hipErrorInvalidValue;
  if (a.F == 32 && a.D == 32) e = launch_bwdc_f<32>(a, st);
  else if (a.F == 64 && a.D == 64) e = launch_bwdc_f<64>(a, st);
  else if (a.F == 128 && a.D == 128) e = launch_bwdc_f<128>(a, st);
  if (e != hipSuccess) return e;
  return launch_bwd_reduce(a, st);
}

}  // namespace ia
