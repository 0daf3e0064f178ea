// ia_backward.hip — gradients of the causal IA layer: reverse-mode differentiation of the
// token recurrence, in fp32, token-sequential within each (b,h) slice and parallel over slices
// and modes.  The training-time figures of "Interdomain Attention: Beyond Token-Level
// Key-Value Memory" (summary page §G) count this pass beside the forward.
//
// The recurrence per mode m (summary page §3.1-§3.2; episode page, derivation):
//   U_t = lam U_{t-1} + beta phi(k_t),  Gam_t = lam Gam_{t-1} + beta v_t,  eta_t = lam eta_{t-1} + beta
//   a_t[m] = phi(q_t) . U_t[m],  num_t = Re sum_m a_t[m] Gam_t[m],  den_t = Re sum_m a_t[m] eta_t[m]
//   o_t = num_t / max(den_t, clamp)
// Reverse mode carries the state adjoints Ubar_t = (readout at t) + conj(lam) Ubar_{t+1} (the
// same for Gam and eta); complex gradients are dL/dRe + i dL/dIm.
//
// Launches:
//  1. bwd_forward_kernel: recompute the states from the initial state, store them every
//     kBwdCheckpoint tokens (and after the last token), and per token the partial sums over
//     this wave's modes of den_t and of g_t . num_t (g = dL/do), which the readout gradient
//     needs in full before any mode can run backward, and a_t[m], which the reverse sweep
//     reuses.
//  2. bwd_reverse_kernel: walk each checkpoint interval backward from its end state,
//     rebuilding U_{t-1} = (U_t - beta phi(k_t)) / lam (the interval is short, so the growth of
//     rounding by |lam|^-1 per step stays bounded), carrying the adjoints, and collecting the
//     gradients of q, k, v (summed over this workgroup's modes), lambda and beta.
//  3. bwd_reduce_kernel: sum the per-mode-group partials of dq, dk, dv in a fixed order and
//     store them in the input dtype; sum lambda and beta gradients over the batch (and over
//     sequence segments).
// When slices x mode groups leave compute units idle, each sequence is cut into segments that
// run side by side; both sweeps are linear recurrences, so each gets a local pass from zero
// and bwd_carry_kernel (lam^L for the states, conj(lam)^L for the adjoints, across segments)
// before its full pass.  The bidirectional layer runs all of it twice, the second time on the
// reversed walk, adding onto the first.
//
// Layout: a workgroup is 8 waves x 2 modes (16 modes, a block of one slice's modes); lane l of
// a wave owns state columns l, l + 64, ... of U (F wide) and Gam (D wide) for both of its
// modes, so every sum over modes of a column is a lane's own, and every sum over a mode's
// columns is a wave reduction (DPP moves) per token.  Token rows reach LDS in double-buffered
// blocks.
#include <algorithm>

#include "ia_device.hpp"
#include "ia_kernels.hpp"

namespace ia {

namespace {

constexpr int kModesPerWave = 2;
constexpr int kWaves = 8;
constexpr int kRed = 4 * kModesPerWave;   // values a wave sums per token: 4 per mode
constexpr int kModesPerWg = kModesPerWave * kWaves;
constexpr int kThreads = 64 * kWaves;

__device__ __forceinline__ float2 cadd(float2 a, float2 b) { return make_float2(a.x + b.x, a.y + b.y); }
__device__ __forceinline__ float2 cscale(float s, float2 a) { return make_float2(s * a.x, s * a.y); }
__device__ __forceinline__ float2 conjf2(float2 a) { return make_float2(a.x, -a.y); }
// a * conj(b)
__device__ __forceinline__ float2 cmulc(float2 a, float2 b) {
  return make_float2(a.x * b.x + a.y * b.y, a.y * b.x - a.x * b.y);
}
// Re(a * conj(b))
__device__ __forceinline__ float cdotr(float2 a, float2 b) { return a.x * b.x + a.y * b.y; }

__device__ __forceinline__ float uniform(float x, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}

// Wave total of v as a wave-uniform scalar, through DPP moves (no LDS round trip): swaps
// within quads (lane ^ 1, lane ^ 2), then mirrors within half-rows and rows, leave every lane
// of a 16-lane row with the row's sum; row_bcast:15 and row_bcast:31 then fold rows 0-1 into
// 1 and rows 0-3 into 3, so lane 63 holds the total.
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ float dpp_plus(float v) {
  return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROWS, 0xF,
                                                        false));
}
__device__ __forceinline__ float wave_total(float v) {
  v = dpp_plus<0xB1>(v);         // quad_perm [1,0,3,2]
  v = dpp_plus<0x4E>(v);         // quad_perm [2,3,0,1]
  v = dpp_plus<0x141>(v);        // row_half_mirror
  v = dpp_plus<0x140>(v);        // row_mirror
  v = dpp_plus<0x142, 0xA>(v);   // row_bcast:15 into rows 1 and 3
  v = dpp_plus<0x143, 0xC>(v);   // row_bcast:31 into rows 2 and 3
  return uniform(v, 63);
}
template <int NV>
__device__ __forceinline__ void wave_totals(float (&v)[NV]) {
#pragma unroll
  for (int i = 0; i < NV; ++i) v[i] = wave_total(v[i]);
}

struct Slice {
  int lane, wave, slice, grp, seg, b, h, m0, groups;
  int lo, hi;   // the segment's tokens [lo, hi)
};

// Workgroups are dispatched to the eight XCDs in turn (block b to XCD b % 8); with the grid a
// multiple of 8, block b takes position (b % 8) (grid / 8) + b / 8, so the mode groups of a
// slice, which read the same token rows, run on one XCD and share its L2.
__device__ __forceinline__ Slice slice_of(const BwdArgs& a) {
  Slice s;
  s.lane = threadIdx.x & 63;
  s.wave = threadIdx.x >> 6;
  s.groups = a.M / kModesPerWg;
  const int nb = gridDim.x;
  const int p = nb % 8 ? (int)blockIdx.x : (blockIdx.x % 8) * (nb / 8) + blockIdx.x / 8;
  s.seg = p % a.nseg;
  s.slice = p / a.nseg / s.groups;
  s.grp = p / a.nseg % s.groups;
  s.lo = s.seg * a.seg_len;
  s.hi = min(a.N, s.lo + a.seg_len);
  s.b = s.slice / a.H;
  s.h = s.slice % a.H;
  s.m0 = s.grp * kModesPerWg + s.wave * kModesPerWave;
  return s;
}

// The state of this wave's modes at the lane's columns.
template <int NF, int ND>
struct State {
  float2 U[kModesPerWave][NF], G[kModesPerWave][ND], E[kModesPerWave];

  __device__ void zero() {
#pragma unroll
    for (int i = 0; i < kModesPerWave; ++i) {
#pragma unroll
      for (int j = 0; j < NF; ++j) U[i][j] = make_float2(0.f, 0.f);
#pragma unroll
      for (int j = 0; j < ND; ++j) G[i][j] = make_float2(0.f, 0.f);
      E[i] = make_float2(0.f, 0.f);
    }
  }
  // From a caller's state ([slice][M][F], [slice][M][D], [slice][M]); zeros when absent.
  __device__ void load_state(const BwdArgs& a, const float2* U0, const float2* G0,
                             const float2* E0, const Slice& s) {
    if (!U0) {
      zero();
      return;
    }
#pragma unroll
    for (int i = 0; i < kModesPerWave; ++i) {
      const size_t m = (size_t)s.slice * a.M + s.m0 + i;
#pragma unroll
      for (int j = 0; j < NF; ++j) {
        const int r = s.lane + 64 * j;
        U[i][j] = r < a.F ? U0[m * a.F + r] : make_float2(0.f, 0.f);
      }
#pragma unroll
      for (int j = 0; j < ND; ++j) {
        const int c = s.lane + 64 * j;
        G[i][j] = c < a.D ? G0[m * a.D + c] : make_float2(0.f, 0.f);
      }
      E[i] = E0[m];
    }
  }
  // Row block `idx` of a [..][M][F + D + 1] array: per mode, F values of U, D of Gam, then
  // eta (checkpoints: idx = slice * checkpoints + k; segment carries: slice * nseg + seg).
  __device__ static float2* row_at(const BwdArgs& a, float2* base, size_t idx, const Slice& s,
                                   int i) {
    return base + (idx * a.M + s.m0 + i) * (a.F + a.D + 1);
  }
  __device__ static size_t ckpt_idx(const BwdArgs& a, const Slice& s, int ck) {
    return (size_t)s.slice * ((a.N + kBwdCheckpoint - 1) / kBwdCheckpoint) + ck;
  }
  __device__ static size_t seg_idx(const BwdArgs& a, const Slice& s) {
    return (size_t)s.slice * a.nseg + s.seg;
  }
  __device__ void store_ckpt(const BwdArgs& a, const Slice& s, int ck) const {
    store_rows(a, a.ckpt, ckpt_idx(a, s, ck), s);
  }
  __device__ void load_ckpt(const BwdArgs& a, const Slice& s, int ck) {
    load_rows(a, a.ckpt, ckpt_idx(a, s, ck), s);
  }
  __device__ void store_rows(const BwdArgs& a, float2* base, size_t idx, const Slice& s) const {
#pragma unroll
    for (int i = 0; i < kModesPerWave; ++i) {
      float2* row = row_at(a, base, idx, s, i);
#pragma unroll
      for (int j = 0; j < NF; ++j)
        if (s.lane + 64 * j < a.F) row[s.lane + 64 * j] = U[i][j];
#pragma unroll
      for (int j = 0; j < ND; ++j)
        if (s.lane + 64 * j < a.D) row[a.F + s.lane + 64 * j] = G[i][j];
      if (s.lane == 0) row[a.F + a.D] = E[i];
    }
  }
  __device__ void load_rows(const BwdArgs& a, float2* base, size_t idx, const Slice& s) {
#pragma unroll
    for (int i = 0; i < kModesPerWave; ++i) {
      const float2* row = row_at(a, base, idx, s, i);
#pragma unroll
      for (int j = 0; j < NF; ++j)
        U[i][j] = s.lane + 64 * j < a.F ? row[s.lane + 64 * j] : make_float2(0.f, 0.f);
#pragma unroll
      for (int j = 0; j < ND; ++j)
        G[i][j] = s.lane + 64 * j < a.D ? row[a.F + s.lane + 64 * j] : make_float2(0.f, 0.f);
      E[i] = row[a.F + a.D];
    }
  }
};

// Token rows staged in LDS, as raw bytes in the inputs' own dtypes: one token's q[F], k[F],
// v[D], g[D] (g = dL/do) and, for the reverse sweep, the per-wave partials of den and g . num
// of that token (M/2 float pairs), each segment a multiple of 16 bytes.  Blocks of
// BwdArgs::tb rows are double-buffered: the 16-byte loads of the next block are issued
// before the current block is processed and land in LDS after it, so their latency hides
// behind a block of tokens.
// 16-byte loads per thread that stage one block; the block length (BwdArgs::tb) is chosen on
// the host so that a block of the reverse sweep's rows fits them.
constexpr int kPrefetch = kBwdPrefetch;

struct RowLayout {
  int q, k, v, g, p, a, bytes;   // byte offsets of the segments in a row, and its length
};

__device__ __forceinline__ RowLayout row_layout(const BwdArgs& a, bool with_den) {
  const int ei = a.in_bf16 ? 2 : 4, eo = a.out_bf16 ? 2 : 4;
  RowLayout l;
  l.q = 0;
  l.k = a.F * ei;
  l.v = 2 * a.F * ei;
  l.g = l.v + a.D * ei;
  l.p = l.g + a.D * eo;
  l.a = l.p + (with_den ? 8 * (a.M / kModesPerWave) : 0);
  l.bytes = l.a + (with_den ? 8 * kModesPerWg : 0);   // the workgroup's a[m] of the token
  return l;
}

// Issues the loads of the block of rows for tokens t_first, t_first + step, ... (rows of
// tokens outside [0, N) are not read).
template <int P>
__device__ __forceinline__ void stage_issue(const BwdArgs& a, const Slice& s, const RowLayout& l,
                                            int t_first, int step, int tb, uint4 (&pre)[P]) {
  const int vec_row = l.bytes / 16, n = tb * vec_row;
  const int ei = a.in_bf16 ? 2 : 4, eo = a.out_bf16 ? 2 : 4;
#pragma unroll
  for (int i = 0; i < P; ++i) {
    const int e = threadIdx.x + kThreads * i;
    uint4 x = make_uint4(0u, 0u, 0u, 0u);
    if (e < n) {
      const int j = e / vec_row, o = 16 * (e - j * vec_row);
      const int t = t_first + step * j;
      if (t >= 0 && t < a.N) {
        // walk index t is position t, or N-1-t for the reverse direction
        const size_t row = ((size_t)s.b * a.N + (a.dir ? a.N - 1 - t : t)) * a.H + s.h;
        const char* src;
        if (o < l.k)
          src = static_cast<const char*>(a.q) + row * a.F * ei + o;
        else if (o < l.v)
          src = static_cast<const char*>(a.k) + row * a.F * ei + (o - l.k);
        else if (o < l.g)
          src = static_cast<const char*>(a.v) + row * a.D * ei + (o - l.v);
        else if (o < l.p)
          src = static_cast<const char*>(a.dO) + row * a.D * eo + (o - l.g);
        else if (o < l.a)
          src = reinterpret_cast<const char*>(a.dpart) +
                ((size_t)s.slice * a.N + t) * (a.M / kModesPerWave) * 8 + (o - l.p);
        else
          src = reinterpret_cast<const char*>(a.apart) +
                (((size_t)s.slice * a.N + t) * a.M + s.grp * kModesPerWg) * 8 + (o - l.a);
        x = *reinterpret_cast<const uint4*>(src);
      }
    }
    pre[i] = x;
  }
}

template <int P>
__device__ __forceinline__ void stage_store(const RowLayout& l, int tb, const uint4 (&pre)[P],
                                            unsigned char* buf) {
  const int n = tb * (l.bytes / 16);
#pragma unroll
  for (int i = 0; i < P; ++i) {
    const int e = threadIdx.x + kThreads * i;
    if (e < n) reinterpret_cast<uint4*>(buf)[e] = pre[i];
  }
}

__device__ __forceinline__ float lds_in(const unsigned char* seg, int i, int bf16) {
  // bf16: the 16 bits at 2i, widened; fp32: the word at 4i (bf16 is wave-uniform)
  if (bf16) return bf16_to_f32(reinterpret_cast<const uint16_t*>(seg)[i]);
  return reinterpret_cast<const float*>(seg)[i];
}

// One token's inputs at the lane's columns, from its staged row: features of q and k (zero
// past F), their derivatives, v and g (zero past D).
template <int NF, int ND>
struct Token {
  float fq[NF], fk[NF], dq[NF], dk[NF], v[ND], g[ND];

  __device__ void load(const BwdArgs& a, const Slice& s, const RowLayout& l,
                       const unsigned char* row) {
    const bool ident = a.opt & kOptIdentity;
#pragma unroll
    for (int j = 0; j < NF; ++j) {
      // columns past F read column F-1 (no branch) and are then zeroed
      const bool ok = s.lane + 64 * j < a.F;
      const int r = min(s.lane + 64 * j, a.F - 1);
      const float x = ok ? lds_in(row + l.q, r, a.in_bf16) : 0.f;
      const float y = ok ? lds_in(row + l.k, r, a.in_bf16) : 0.f;
      // phi(x) = x + 1 above 0, exp(x) at or below; phi'(x) = 1 above 0, exp(x) at or below
      const float ex = __expf(fminf(x, 0.f)), ey = __expf(fminf(y, 0.f));
      fq[j] = !ok ? 0.f : ident ? x : (x > 0.f ? x + 1.f : ex);
      fk[j] = !ok ? 0.f : ident ? y : (y > 0.f ? y + 1.f : ey);
      dq[j] = ident || x > 0.f ? 1.f : ex;
      dk[j] = ident || y > 0.f ? 1.f : ey;
    }
#pragma unroll
    for (int j = 0; j < ND; ++j) {
      const bool ok = s.lane + 64 * j < a.D;
      const int c = min(s.lane + 64 * j, a.D - 1);
      v[j] = ok ? lds_in(row + l.v, c, a.in_bf16) : 0.f;
      g[j] = ok ? lds_in(row + l.g, c, a.out_bf16) : 0.f;
    }
  }
};

template <int NF, int ND>
__global__ void __launch_bounds__(kThreads) bwd_forward_kernel(const BwdArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];   // two blocks of staged token rows
  const int TB = a.tb;
  constexpr int P = kPrefetch;
  const Slice s = slice_of(a);
  const RowLayout L = row_layout(a, false);
  const int R = L.bytes;
  float2 lam[kModesPerWave], bet[kModesPerWave];
#pragma unroll
  for (int i = 0; i < kModesPerWave; ++i) {
    lam[i] = a.lam[(size_t)s.h * a.M + s.m0 + i];
    bet[i] = a.beta[(size_t)s.h * a.M + s.m0 + i];
  }
  // the segment's start state: zeros for the local pass (its end state from zero feeds the
  // carry), else the caller's state for segment 0 and the carried state after it
  State<NF, ND> st;
  if (a.local)
    st.zero();
  else if (s.seg == 0)
    st.load_state(a, a.U0, a.G0, a.E0, s);
  else
    st.load_rows(a, a.cstate, State<NF, ND>::seg_idx(a, s), s);
  const int parts = a.M / kModesPerWave;
  const int nblk = (s.hi - s.lo + TB - 1) / TB;
  uint4 pre[P];
  stage_issue(a, s, L, s.lo, 1, TB, pre);
  stage_store(L, TB, pre, smem);
  __syncthreads();
  for (int blk = 0; blk < nblk; ++blk) {
    const unsigned char* rows = smem + (blk & 1) * TB * R;
    if (blk + 1 < nblk) stage_issue(a, s, L, s.lo + (blk + 1) * TB, 1, TB, pre);
    for (int j = 0; j < TB; ++j) {
      const int t = s.lo + blk * TB + j;
      if (t >= s.hi) break;
      Token<NF, ND> x;
      x.load(a, s, L, rows + j * R);
      float red[kRed];
#pragma unroll
      for (int i = 0; i < kModesPerWave; ++i) {
        float2 ap = make_float2(0.f, 0.f), sp = make_float2(0.f, 0.f);
#pragma unroll
        for (int j2 = 0; j2 < NF; ++j2) {
          st.U[i][j2] = cadd(cmul(lam[i], st.U[i][j2]), cscale(x.fk[j2], bet[i]));
          ap = cadd(ap, cscale(x.fq[j2], st.U[i][j2]));
        }
#pragma unroll
        for (int j2 = 0; j2 < ND; ++j2) {
          st.G[i][j2] = cadd(cmul(lam[i], st.G[i][j2]), cscale(x.v[j2], bet[i]));
          sp = cadd(sp, cscale(x.g[j2], st.G[i][j2]));
        }
        st.E[i] = cadd(cmul(lam[i], st.E[i]), bet[i]);
        red[4 * i + 0] = ap.x;
        red[4 * i + 1] = ap.y;
        red[4 * i + 2] = sp.x;
        red[4 * i + 3] = sp.y;
      }
      if (a.local) continue;   // the local pass only carries the state
      wave_totals(red);
      // den_t and g_t . num_t over this wave's modes: Re(a eta) and Re(a sum_j g_j Gam_j)
      float den = 0.f, gn = 0.f;
#pragma unroll
      for (int i = 0; i < kModesPerWave; ++i) {
        const float2 am = make_float2(red[4 * i], red[4 * i + 1]);
        const float2 sm = make_float2(red[4 * i + 2], red[4 * i + 3]);
        den += am.x * st.E[i].x - am.y * st.E[i].y;
        gn += am.x * sm.x - am.y * sm.y;
      }
      if (s.lane == 0) {
        a.dpart[((size_t)s.slice * a.N + t) * parts + s.m0 / kModesPerWave] = make_float2(den, gn);
#pragma unroll
        for (int i = 0; i < kModesPerWave; ++i)   // a[m], which the reverse sweep reuses
          a.apart[((size_t)s.slice * a.N + t) * a.M + s.m0 + i] =
              make_float2(red[4 * i], red[4 * i + 1]);
      }
      if (t % kBwdCheckpoint == kBwdCheckpoint - 1 || t == a.N - 1)
        st.store_ckpt(a, s, t / kBwdCheckpoint);
    }
    if (blk + 1 < nblk) {
      // the other buffer was last read in the previous block, which every wave has left
      stage_store(L, TB, pre, smem + ((blk + 1) & 1) * TB * R);
      __syncthreads();
    }
  }
  if (a.local) st.store_rows(a, a.cstate, State<NF, ND>::seg_idx(a, s), s);
}

template <int NF, int ND>
__global__ void __launch_bounds__(kThreads) bwd_reverse_kernel(const BwdArgs a) {
  // two blocks of staged token rows, then [token][wave][2F + D] gradient rows before the mode
  // sum
  extern __shared__ __align__(16) unsigned char smem[];
  const int TB = a.tb;
  constexpr int P = kPrefetch;
  const Slice s = slice_of(a);
  const RowLayout L = row_layout(a, true);
  const int R = L.bytes;
  const int W = 2 * a.F + a.D;
  float* part = reinterpret_cast<float*>(smem + 2 * TB * R);
  float2 lam[kModesPerWave], bet[kModesPerWave], linv[kModesPerWave];
#pragma unroll
  for (int i = 0; i < kModesPerWave; ++i) {
    lam[i] = a.lam[(size_t)s.h * a.M + s.m0 + i];
    bet[i] = a.beta[(size_t)s.h * a.M + s.m0 + i];
    const float n2 = lam[i].x * lam[i].x + lam[i].y * lam[i].y;
    linv[i] = make_float2(lam[i].x / n2, -lam[i].y / n2);
  }
  const bool noden = a.opt & kOptNoDen;
  const int parts = a.M / kModesPerWave;
  // adjoints of U, Gam, eta (eta's is wave-uniform), and the lane's share of the lambda and
  // beta gradients of each mode
  // Adjoints entering the segment's last token: zeros for the last segment and for the local
  // pass (whose adjoints leaving the segment feed the carry), else the carried ones.
  State<NF, ND> adj;
  if (a.local || s.seg == a.nseg - 1)
    adj.zero();
  else
    adj.load_rows(a, a.cadj, State<NF, ND>::seg_idx(a, s), s);
  float2 gl[kModesPerWave], gb[kModesPerWave];
#pragma unroll
  for (int i = 0; i < kModesPerWave; ++i) gl[i] = gb[i] = make_float2(0.f, 0.f);
  const int nblk = (s.hi - s.lo + TB - 1) / TB;
  uint4 pre[P];
  stage_issue(a, s, L, s.hi - 1, -1, TB, pre);
  stage_store(L, TB, pre, smem);
  State<NF, ND> cur;
  cur.load_ckpt(a, s, (s.hi - 1) / kBwdCheckpoint);   // the state after the segment's last token
  __syncthreads();
  for (int blk = 0; blk < nblk; ++blk) {
    const unsigned char* rows = smem + (blk & 1) * TB * R;
    const int t_hi = s.hi - 1 - blk * TB;   // tokens t_hi, t_hi - 1, ... of this block
    if (blk + 1 < nblk) stage_issue(a, s, L, t_hi - TB, -1, TB, pre);
    // The readout's gradient factors of the block's tokens, dnum = g rc and dden (0 below the
    // clamp, and without a denominator): the 8 lanes 8j..8j+7 sum token j's partials of den
    // and g . num, and lane 8j keeps its factors.
    float blk_rc = 1.f, blk_dd = 0.f;
    if (!noden) {
      const int jt = s.lane >> 3, sub = s.lane & 7;
      float2 p = make_float2(0.f, 0.f);
      if (jt < TB && t_hi - jt >= s.lo) {
        const float2* dp = reinterpret_cast<const float2*>(rows + jt * R + L.p);
#pragma unroll
        for (int k = 0; k < kMaxModes / kModesPerWave / 8; ++k)
          if (sub + 8 * k < parts) p = cadd(p, dp[sub + 8 * k]);
      }
#pragma unroll
      for (int bit = 4; bit >= 1; bit >>= 1) {
        p.x += __shfl_xor(p.x, bit, 64);
        p.y += __shfl_xor(p.y, bit, 64);
      }
      const float cl = p.x < a.clamp ? a.clamp : p.x;   // NaN stays NaN
      blk_rc = 1.f / cl;
      blk_dd = p.x >= a.clamp ? -p.y * blk_rc * blk_rc : 0.f;
    }
    for (int j = 0; j < TB; ++j) {
      const int t = t_hi - j;
      if (t < s.lo) break;
      const unsigned char* row = rows + j * R;
      Token<NF, ND> x;
      x.load(a, s, L, row);
      const float rc = uniform(blk_rc, 8 * j), dd = uniform(blk_dd, 8 * j);
      // h[m] = sum_j g_j conj(Gam_mj) over the wave; a[m] as the recompute sweep formed it
      float red[2 * kModesPerWave];
#pragma unroll
      for (int i = 0; i < kModesPerWave; ++i) {
        float2 hp = make_float2(0.f, 0.f);
#pragma unroll
        for (int j2 = 0; j2 < ND; ++j2) hp = cadd(hp, cscale(x.g[j2], conjf2(cur.G[i][j2])));
        red[2 * i + 0] = hp.x;
        red[2 * i + 1] = hp.y;
      }
      wave_totals(red);
      const float2* arow = reinterpret_cast<const float2*>(row + L.a) + s.wave * kModesPerWave;
      float dfq[NF], dfk[NF], dv[ND];
#pragma unroll
      for (int j2 = 0; j2 < NF; ++j2) dfq[j2] = dfk[j2] = 0.f;
#pragma unroll
      for (int j2 = 0; j2 < ND; ++j2) dv[j2] = 0.f;
#pragma unroll
      for (int i = 0; i < kModesPerWave; ++i) {
        const float2 am = arow[i];
        const float2 hm = make_float2(red[2 * i], red[2 * i + 1]);
        // gradient of a[m]: sum_j dnum_j conj(Gam_mj) + dden conj(eta_m)
        const float2 ga = cadd(cscale(rc, hm), cscale(dd, conjf2(cur.E[i])));
        const float2 ca = conjf2(am);
#pragma unroll
        for (int j2 = 0; j2 < NF; ++j2) {
          adj.U[i][j2] = cadd(adj.U[i][j2], cscale(x.fq[j2], ga));
          dfq[j2] += cdotr(ga, cur.U[i][j2]);
          dfk[j2] += cdotr(adj.U[i][j2], bet[i]);
          gb[i] = cadd(gb[i], cscale(x.fk[j2], adj.U[i][j2]));
        }
#pragma unroll
        for (int j2 = 0; j2 < ND; ++j2) {
          adj.G[i][j2] = cadd(adj.G[i][j2], cscale(rc * x.g[j2], ca));
          dv[j2] += cdotr(adj.G[i][j2], bet[i]);
          gb[i] = cadd(gb[i], cscale(x.v[j2], adj.G[i][j2]));
        }
        adj.E[i] = cadd(adj.E[i], cscale(dd, ca));
        if (s.lane == 0 && !a.local) gb[i] = cadd(gb[i], adj.E[i]);
      }
      // the state before token t, in place: rebuilt inside a checkpoint interval, read from
      // the previous checkpoint (or the initial state) at its start
      if (t % kBwdCheckpoint != 0) {
#pragma unroll
        for (int i = 0; i < kModesPerWave; ++i) {
#pragma unroll
          for (int j2 = 0; j2 < NF; ++j2)
            cur.U[i][j2] = cmul(make_float2(cur.U[i][j2].x - x.fk[j2] * bet[i].x,
                                            cur.U[i][j2].y - x.fk[j2] * bet[i].y), linv[i]);
#pragma unroll
          for (int j2 = 0; j2 < ND; ++j2)
            cur.G[i][j2] = cmul(make_float2(cur.G[i][j2].x - x.v[j2] * bet[i].x,
                                            cur.G[i][j2].y - x.v[j2] * bet[i].y), linv[i]);
          cur.E[i] = cmul(make_float2(cur.E[i].x - bet[i].x, cur.E[i].y - bet[i].y), linv[i]);
        }
      } else if (t > 0) {
        cur.load_ckpt(a, s, t / kBwdCheckpoint - 1);
      } else {
        cur.load_state(a, a.U0, a.G0, a.E0, s);
      }
#pragma unroll
      for (int i = 0; i < kModesPerWave; ++i) {
        const float2 cl = conjf2(lam[i]);
#pragma unroll
        for (int j2 = 0; j2 < NF; ++j2) {
          gl[i] = cadd(gl[i], cmulc(adj.U[i][j2], cur.U[i][j2]));
          adj.U[i][j2] = cmul(cl, adj.U[i][j2]);
        }
#pragma unroll
        for (int j2 = 0; j2 < ND; ++j2) {
          gl[i] = cadd(gl[i], cmulc(adj.G[i][j2], cur.G[i][j2]));
          adj.G[i][j2] = cmul(cl, adj.G[i][j2]);
        }
        if (s.lane == 0 && !a.local) gl[i] = cadd(gl[i], cmulc(adj.E[i], cur.E[i]));
        adj.E[i] = cmul(cl, adj.E[i]);
      }
      if (a.local) continue;   // the local pass only carries the adjoints
      // this wave's gradient row of token t
      float* out = part + (size_t)(j * kWaves + s.wave) * W;
#pragma unroll
      for (int j2 = 0; j2 < NF; ++j2) {
        const int r = s.lane + 64 * j2;
        if (r < a.F) {
          out[r] = dfq[j2] * x.dq[j2];
          out[a.F + r] = dfk[j2] * x.dk[j2];
        }
      }
#pragma unroll
      for (int j2 = 0; j2 < ND; ++j2)
        if (s.lane + 64 * j2 < a.D) out[2 * a.F + s.lane + 64 * j2] = dv[j2];
    }
    __syncthreads();
    // the waves' rows summed: this workgroup's partial for the block's tokens; then the
    // next block's rows land in the buffer just used
    const int ntok = a.local ? 0 : min(TB, t_hi - s.lo + 1);
    for (int e = threadIdx.x; e < ntok * W; e += kThreads) {
      const int jj = e / W, col = e - jj * W;
      float sum = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) sum += part[(size_t)(jj * kWaves + w) * W + col];
      a.gpart[(((size_t)s.grp * a.B * a.H + s.slice) * a.N + (t_hi - jj)) * W + col] = sum;
    }
    if (blk + 1 < nblk) stage_store(L, TB, pre, smem + ((blk + 1) & 1) * TB * R);
    __syncthreads();
  }
  if (a.local) {
    adj.store_rows(a, a.cadj, State<NF, ND>::seg_idx(a, s), s);
    return;
  }
  // gradients of lambda and beta of this wave's modes, for this slice and segment
  float red[kRed];
#pragma unroll
  for (int i = 0; i < kModesPerWave; ++i) {
    red[4 * i + 0] = gl[i].x;
    red[4 * i + 1] = gl[i].y;
    red[4 * i + 2] = gb[i].x;
    red[4 * i + 3] = gb[i].y;
  }
  wave_totals(red);
#pragma unroll
  for (int i = 0; i < kModesPerWave; ++i) {
    const size_t m = (size_t)s.slice * a.M + s.m0 + i;
    const size_t ms = State<NF, ND>::seg_idx(a, s) * a.M + s.m0 + i;
    const float2 l = make_float2(red[4 * i], red[4 * i + 1]);
    const float2 bb = make_float2(red[4 * i + 2], red[4 * i + 3]);
    if (s.lane == 0) {
      a.lpart[2 * ms] = l;
      a.lpart[2 * ms + 1] = bb;
    }
    // what is left in segment 0's adjoints is the gradient of the initial state
    if (a.dU0 && s.seg == 0) {
#pragma unroll
      for (int j = 0; j < NF; ++j)
        if (s.lane + 64 * j < a.F) a.dU0[m * a.F + s.lane + 64 * j] = adj.U[i][j];
#pragma unroll
      for (int j = 0; j < ND; ++j)
        if (s.lane + 64 * j < a.D) a.dG0[m * a.D + s.lane + 64 * j] = adj.G[i][j];
      if (s.lane == 0) a.dE0[m] = adj.E[i];
    }
  }
}

// dq, dk, dv: the mode groups' partials summed in group order, stored in the input dtype;
// lambda and beta gradients summed over the batch in b order.  Four consecutive columns per
// thread (F and Dv are multiples of 16, so the four lie in one of dq, dk, dv).
__global__ void __launch_bounds__(256) bwd_reduce_kernel(const BwdArgs a) {
  const int W = 2 * a.F + a.D;
  const int groups = a.M / kModesPerWg;
  const size_t S = (size_t)a.B * a.H;
  const size_t n = S * a.N * W;
  for (size_t e = 4 * (blockIdx.x * (size_t)blockDim.x + threadIdx.x); e < n;
       e += 4 * (size_t)gridDim.x * blockDim.x) {
    float4 sum = *reinterpret_cast<const float4*>(a.gpart + e);
    for (int g = 1; g < groups; ++g) {
      const float4 x = *reinterpret_cast<const float4*>(a.gpart + (size_t)g * n + e);
      sum.x += x.x;
      sum.y += x.y;
      sum.z += x.z;
      sum.w += x.w;
    }
    const size_t sl = e / ((size_t)a.N * W);
    const size_t rem = e - sl * a.N * W;
    const size_t t = rem / W;
    const int col = (int)(rem - t * W);
    const size_t b = sl / a.H, h = sl % a.H;
    const size_t row = (b * a.N + (a.dir ? a.N - 1 - t : t)) * a.H + h;
    void* dst;
    size_t i;
    if (col < a.F) {
      dst = a.dq;
      i = row * a.F + col;
    } else if (col < 2 * a.F) {
      dst = a.dk;
      i = row * a.F + col - a.F;
    } else {
      dst = a.dv;
      i = row * a.D + col - 2 * a.F;
    }
    float v[4] = {sum.x, sum.y, sum.z, sum.w};
    if (a.in_bf16) {
      uint2* p = reinterpret_cast<uint2*>(static_cast<uint16_t*>(dst) + i);
      if (a.accumulate) {
        const uint2 o = *p;
        v[0] += __uint_as_float(o.x << 16);
        v[1] += __uint_as_float(o.x & 0xffff0000u);
        v[2] += __uint_as_float(o.y << 16);
        v[3] += __uint_as_float(o.y & 0xffff0000u);
      }
      *p = make_uint2((uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16),
                      (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16));
    } else {
      float4* p = reinterpret_cast<float4*>(static_cast<float*>(dst) + i);
      if (a.accumulate) {
        const float4 o = *p;
        v[0] += o.x;
        v[1] += o.y;
        v[2] += o.z;
        v[3] += o.w;
      }
      *p = make_float4(v[0], v[1], v[2], v[3]);
    }
  }
  const size_t hm = (size_t)a.H * a.M;
  for (size_t e = blockIdx.x * (size_t)blockDim.x + threadIdx.x; e < hm;
       e += (size_t)gridDim.x * blockDim.x) {
    float2 l = make_float2(0.f, 0.f), bb = make_float2(0.f, 0.f);
    const size_t h = e / a.M, m = e % a.M;
    for (int b = 0; b < a.B; ++b)
      for (int g = 0; g < a.nseg; ++g) {
        const size_t i = (((size_t)b * a.H + h) * a.nseg + g) * a.M + m;
        l = cadd(l, a.lpart[2 * i]);
        bb = cadd(bb, a.lpart[2 * i + 1]);
      }
    if (a.accumulate) {
      l = cadd(l, a.dlam[e]);
      bb = cadd(bb, a.dbeta[e]);
    }
    a.dlam[e] = l;
    a.dbeta[e] = bb;
  }
}

// Dynamic LDS above the default limit needs the kernel's attribute raised first.
hipError_t allow_lds(const void* kernel, size_t bytes, size_t& allowed) {
  if (bytes <= allowed) return hipSuccess;
  hipError_t e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)bytes);
  if (e == hipSuccess) allowed = bytes;
  return e;
}

// z^n for complex z in fp64 by binary exponentiation, rounded once to fp32.
__device__ __forceinline__ float2 cpow_n(float2 z, int n) {
  double ar = 1.0, ai = 0.0, sr = z.x, si = z.y;
  for (; n > 0; n >>= 1) {
    if (n & 1) {
      const double tr = ar * sr - ai * si;
      ai = ar * si + ai * sr;
      ar = tr;
    }
    const double qr = sr * sr - si * si;
    si = 2.0 * sr * si;
    sr = qr;
  }
  return make_float2((float)ar, (float)ai);
}

// Segment carry of the state, one thread per (slice, mode, column): the local pass left each
// segment's end state from zero in `cstate`; replace it by the segment's start state,
// start(0) = the initial state, start(g + 1) = lam^L(g) start(g) + end(g).  With `adjoint`,
// the same for the adjoints from the last segment down, with conj(lam): the local reverse
// pass left in `cadj` what each segment passes on from zero, and the carried adjoints entering
// segment g are conj(lam)^L(g+1) (those entering g + 1) + what g + 1 passes on.
__global__ void __launch_bounds__(256) bwd_carry_kernel(const BwdArgs a, int adjoint) {
  const int C = a.F + a.D + 1;
  const size_t n = (size_t)a.B * a.H * a.M * C;
  for (size_t e = blockIdx.x * (size_t)blockDim.x + threadIdx.x; e < n;
       e += (size_t)gridDim.x * blockDim.x) {
    const int col = (int)(e % C);
    const size_t sm = e / C;
    const int m = (int)(sm % a.M);
    const size_t slice = sm / a.M;
    float2 lam = a.lam[(slice % a.H) * a.M + m];
    float2* buf = adjoint ? a.cadj : a.cstate;
    auto at = [&](int g) -> float2& {
      return buf[(((size_t)slice * a.nseg + g) * a.M + m) * C + col];
    };
    auto len = [&](int g) { return min(a.N, (g + 1) * a.seg_len) - g * a.seg_len; };
    float2 x = make_float2(0.f, 0.f);
    if (!adjoint) {
      const size_t sm0 = slice * a.M + m;
      if (a.U0)
        x = col < a.F ? a.U0[sm0 * a.F + col]
                      : col < a.F + a.D ? a.G0[sm0 * a.D + col - a.F] : a.E0[sm0];
      for (int g = 0; g < a.nseg; ++g) {
        const float2 end = at(g);
        at(g) = x;
        x = cadd(cmul(cpow_n(lam, len(g)), x), end);
      }
    } else {
      lam.y = -lam.y;
      for (int g = a.nseg - 1; g >= 0; --g) {
        const float2 out = at(g);
        at(g) = x;
        x = cadd(cmul(cpow_n(lam, len(g)), x), out);
      }
    }
  }
}

template <int NF, int ND>
hipError_t launch_bwd_nf_nd(const BwdArgs& a, hipStream_t st) {
  static size_t allowed_fwd = 65536, allowed_rev = 65536;
  const unsigned grid = (unsigned)((size_t)a.B * a.H * (a.M / kModesPerWg) * a.nseg);
  const size_t lds_fwd = bwd_lds_bytes(a.F, a.D, a.M, a.in_bf16, a.out_bf16, a.tb, false);
  const size_t lds_rev = bwd_lds_bytes(a.F, a.D, a.M, a.in_bf16, a.out_bf16, a.tb, true);
  hipError_t e = allow_lds(reinterpret_cast<const void*>(&bwd_forward_kernel<NF, ND>), lds_fwd,
                           allowed_fwd);
  if (e == hipSuccess)
    e = allow_lds(reinterpret_cast<const void*>(&bwd_reverse_kernel<NF, ND>), lds_rev,
                  allowed_rev);
  if (e != hipSuccess) return e;
  const size_t carry_n = (size_t)a.B * a.H * a.M * (a.F + a.D + 1);
  const unsigned carry_grid = (unsigned)std::min<size_t>((carry_n + 255) / 256, 4096);
  BwdArgs loc = a;
  loc.local = 1;
  if (a.nseg > 1) {   // segment end states from zero, then the carry
    hipLaunchKernelGGL((bwd_forward_kernel<NF, ND>), dim3(grid), dim3(kThreads), lds_fwd, st,
                       loc);
    hipLaunchKernelGGL(bwd_carry_kernel, dim3(carry_grid), dim3(256), 0, st, a, 0);
  }
  prof_begin(st);
  hipLaunchKernelGGL((bwd_forward_kernel<NF, ND>), dim3(grid), dim3(kThreads), lds_fwd, st, a);
  prof_end(st, kKindBwdForward);
  if (a.nseg > 1) {   // what each segment's adjoints pass on from zero, then the carry
    hipLaunchKernelGGL((bwd_reverse_kernel<NF, ND>), dim3(grid), dim3(kThreads), lds_rev, st,
                       loc);
    hipLaunchKernelGGL(bwd_carry_kernel, dim3(carry_grid), dim3(256), 0, st, a, 1);
  }
  prof_begin(st);
  hipLaunchKernelGGL((bwd_reverse_kernel<NF, ND>), dim3(grid), dim3(kThreads), lds_rev, st, a);
  prof_end(st, kKindBwdReverse);
  return hipGetLastError();
}

}  // namespace

int bwd_segments(int B, int H, int N, int M, int* seg_len) {
  // Segments of at least kBwdMinSegment tokens (a multiple of the checkpoint interval) while
  // slices x mode groups leave compute units idle: the walk of one long sequence is cut so
  // its pieces run side by side.
  const long wgs = (long)B * H * (M / kModesPerWg);
  long n = wgs >= device_cus() ? 1 : device_cus() / wgs;
  const long most = ((long)N + kBwdMinSegment - 1) / kBwdMinSegment;
  if (n > most) n = most;
  if (n < 1) n = 1;
  long len = ((long)N + n - 1) / n;
  len = (len + kBwdCheckpoint - 1) / kBwdCheckpoint * kBwdCheckpoint;
  *seg_len = (int)len;
  return (int)((N + len - 1) / len);
}

BwdLayout bwd_layout(int B, int H, int N, int F, int D, int M) {
  auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
  const size_t S = (size_t)B * H;
  const size_t nck = ((size_t)N + kBwdCheckpoint - 1) / kBwdCheckpoint;
  int seg_len;
  const size_t nseg = bwd_segments(B, H, N, M, &seg_len);
  const size_t carry = nseg > 1 ? up(S * nseg * M * (F + D + 1) * 8) : 0;
  BwdLayout l{};
  l.ckpt_off = 0;
  l.dpart_off = up(S * nck * M * (F + D + 1) * 8);
  l.gpart_off = l.dpart_off + up(S * N * (M / kModesPerWave) * 8);
  l.lpart_off = l.gpart_off + up((size_t)(M / kModesPerWg) * S * N * (2 * F + D) * 4);
  l.apart_off = l.lpart_off + up(S * nseg * M * 2 * 8);
  l.cstate_off = l.apart_off + up(S * N * M * 8);
  l.cadj_off = l.cstate_off + carry;
  l.bytes = l.cadj_off + carry;
  return l;
}

// Bytes of a staged token row (q, k, v in the input dtype, g in the output dtype and, for the
// reverse sweep, the per-wave den partials).
static size_t bwd_row_bytes(int F, int D, int M, int in_bf16, int out_bf16, bool rev) {
  return (size_t)(2 * F + D) * (in_bf16 ? 2 : 4) + (size_t)D * (out_bf16 ? 2 : 4) +
         (rev ? (size_t)8 * (M / kModesPerWave) + 8 * kModesPerWg : 0);
}

size_t bwd_lds_bytes(int F, int D, int M, int in_bf16, int out_bf16, int tb, bool rev) {
  return 2 * (size_t)tb * bwd_row_bytes(F, D, M, in_bf16, out_bf16, rev) +
         (rev ? (size_t)tb * kWaves * (2 * F + D) * sizeof(float) : 0);
}

int bwd_block_tokens(int F, int D, int M, int in_bf16, int out_bf16) {
  // as many tokens (up to 8) as the prefetch registers stage and 150 KiB of LDS holds
  const size_t vec = bwd_row_bytes(F, D, M, in_bf16, out_bf16, true) / 16;
  int tb = (int)((size_t)kPrefetch * kThreads / vec);
  if (tb > 8) tb = 8;
  while (tb > 1 && bwd_lds_bytes(F, D, M, in_bf16, out_bf16, tb, true) > 150 * 1024) --tb;
  return tb < 1 ? 1 : tb;
}

hipError_t launch_prefill_bwd(const BwdArgs& a, hipStream_t st) {
  (void)hipGetLastError();
  const int nf = (a.F + 63) / 64, nd = (a.D + 63) / 64;
  hipError_t e = hipErrorInvalidValue;
#define IA_BWD(X, Y) \
  if (nf == X && nd == Y) e = launch_bwd_nf_nd<X, Y>(a, st); else
  IA_BWD(1, 1) IA_BWD(1, 2) IA_BWD(1, 3) IA_BWD(1, 4)
  IA_BWD(2, 1) IA_BWD(2, 2) IA_BWD(2, 3) IA_BWD(2, 4)
  IA_BWD(3, 1) IA_BWD(3, 2) IA_BWD(3, 3) IA_BWD(3, 4)
  IA_BWD(4, 1) IA_BWD(4, 2) IA_BWD(4, 3) IA_BWD(4, 4)
  {}
#undef IA_BWD
  if (e != hipSuccess) return e;
  return launch_bwd_reduce(a, st);
}

hipError_t launch_bwd_reduce(const BwdArgs& a, hipStream_t st) {
  const size_t n = (size_t)a.B * a.H * a.N * (2 * a.F + a.D) / 4;
  size_t blocks = (n + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) blocks = 1;
  prof_begin(st);
  hipLaunchKernelGGL(bwd_reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, st, a);
  prof_end(st, kKindBwdReduce);
  return hipGetLastError();
}

}  // namespace ia
