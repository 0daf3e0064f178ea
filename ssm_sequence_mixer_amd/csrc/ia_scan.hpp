// ia_scan.hpp — the token-by-token recurrence of one (b,h) slice by one workgroup of NW waves
// (fp32 VALU), shared by the decode step, the token-sequential prefill and the chunked
// prefill's fp32 route (heads whose modes the bf16 chunk factorisation does not resolve).
//
// One step is the recurrence and readout of the layer ("Interdomain Attention: Beyond
// Token-Level Key-Value Memory": summary page §3.2 for the complex-diagonal S4D recurrence and
// the O(M(R+d)) per-step decode; episode page, "Key Components and Derivation", for the
// feature map and the matrix form Fq U^T Gamma / Fq U^T eta):
//     U[m,:] <- lam_m U[m,:] + beta_m phi(k_t),   a[m] = phi(q_t) . U[m,:]
//     G[m,:] <- lam_m G[m,:] + beta_m v_t,        eta[m] <- lam_m eta[m] + beta_m
//     o_t = Re(sum_m a[m] G[m,:]) / max(Re(sum_m a[m] eta[m]), clamp)
// The state stays in global memory (HBM or L2) and is streamed once per token: each wave takes
// every NW-th mode and its lanes cover a state row with 16-byte accesses, so a row of F
// complex values is one coalesced access.
#pragma once

#include "ia_device.hpp"
#include "ia_kernels.hpp"

namespace ia {

__device__ __forceinline__ float2 cadd2(float2 a, float2 b) {
  return make_float2(a.x + b.x, a.y + b.y);
}

// Shared memory of one step: the token's features and values, the modes, a = phi(q) U^T (and
// a R with a readout matrix), eta, and the per-wave numerator partial sums.  MF, MD, MM bound
// F, Dv and M; WR: room for the readout matrix's partial sums.
template <int NW, int MF, int MD, int MM, bool WR>
struct SeqSmem {
  float fq[MF];
  float fk[MF];
  float v[MD];
  float2 lam[MM];
  float2 beta[MM];
  float2 a[MM];
  float2 ar[WR ? MM : 1];          // a R
  float2 rp[WR ? 64 * NW : 1];     // partial sums of a R
  float2 eta[MM];
  float num[NW][MD];
  float den;
};

// State rows are float2 arrays; lanes take two complex values (one float4) at a time.
// F and D are multiples of 16, so a row is a whole number of float4 pairs.
// R: this head's readout matrix [M][M] (row m, column n), or NULL for none: the readouts then
// use (a R)[n] = sum_m a[m] R[m][n] in place of a.
// wg, dg: this token's write and decay gates (1 and 1 without gating): every lambda_m is
// taken times dg and every beta_m times wg.
template <int NW, int MF, int MD, int MM, bool WR>
__device__ __forceinline__ void seq_step(SeqSmem<NW, MF, MD, MM, WR>& s, float2* __restrict__ U,
                                         float2* __restrict__ G, float2* __restrict__ E, int F,
                                         int D, int M, const float2* __restrict__ R,
                                         float wg = 1.f, float dg = 1.f) {
  constexpr int NT = 64 * NW;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;

  // U rows: update in place and contract with phi(q_t).  Each wave takes rows wave, wave+NW,
  // ...: every row's lane partials first, then their wave totals together (DPP, the rows'
  // chains interleaved), lane 63 holding them.
  constexpr int RW = (MM + NW - 1) / NW;   // rows per wave at most
  float ar[RW], ai[RW];
#pragma unroll
  for (int i = 0; i < RW; ++i) {
    const int m = wave + NW * i;
    ar[i] = ai[i] = 0.f;
    if (m < M) {
      const float2 l = make_float2(dg * s.lam[m].x, dg * s.lam[m].y);
      const float2 b = make_float2(wg * s.beta[m].x, wg * s.beta[m].y);
      float4* row = reinterpret_cast<float4*>(U + (size_t)m * F);
      for (int p = lane; p < F / 2; p += 64) {
        float4 u = row[p];
        const float k0 = s.fk[2 * p], k1 = s.fk[2 * p + 1];
        float2 u0 = cfma(l, make_float2(u.x, u.y), make_float2(b.x * k0, b.y * k0));
        float2 u1 = cfma(l, make_float2(u.z, u.w), make_float2(b.x * k1, b.y * k1));
        row[p] = make_float4(u0.x, u0.y, u1.x, u1.y);
        const float q0 = s.fq[2 * p], q1 = s.fq[2 * p + 1];
        ar[i] += q0 * u0.x + q1 * u1.x;
        ai[i] += q0 * u0.y + q1 * u1.y;
      }
    }
  }
  row_totals<64>(ar);
  row_totals<64>(ai);
  if (lane == 63) {
#pragma unroll
    for (int i = 0; i < RW; ++i) {
      const int m = wave + NW * i;
      if (m < M) s.a[m] = make_float2(ar[i], ai[i]);
    }
  }
  // eta: one mode per thread.
  for (int m = threadIdx.x; m < M; m += NT) {
    float2 e = cfma(make_float2(dg * s.lam[m].x, dg * s.lam[m].y), E[m],
                    make_float2(wg * s.beta[m].x, wg * s.beta[m].y));
    E[m] = e;
    s.eta[m] = e;
  }
  __syncthreads();
  if constexpr (WR) {
    if (R) {
      // thread t sums the modes m = t / M, t / M + parts, ... of column n = t % M
      const int parts = NT / M, n = threadIdx.x % M, part = threadIdx.x / M;
      if (part < parts) {
        float2 acc = make_float2(0.f, 0.f);
        for (int m = part; m < M; m += parts) acc = cfma(s.a[m], R[(size_t)m * M + n], acc);
        s.rp[threadIdx.x] = acc;
      }
      __syncthreads();
      if (threadIdx.x < M) {
        float2 acc = make_float2(0.f, 0.f);
        for (int p = 0; p < parts; ++p) acc = cadd2(acc, s.rp[p * M + threadIdx.x]);
        s.ar[threadIdx.x] = acc;
      }
      __syncthreads();
    }
  }
  const float2* A = (WR && R) ? s.ar : s.a;

  // Gamma rows: update in place, accumulate Re(a[m] G[m,:]) per lane.
  constexpr int NP = (MD + 127) / 128;   // float4 pairs per lane and row
  float acc[2 * NP];
#pragma unroll
  for (int i = 0; i < 2 * NP; ++i) acc[i] = 0.f;
  for (int m = wave; m < M; m += NW) {
    const float2 l = make_float2(dg * s.lam[m].x, dg * s.lam[m].y);
    const float2 b = make_float2(wg * s.beta[m].x, wg * s.beta[m].y), a = A[m];
    float4* row = reinterpret_cast<float4*>(G + (size_t)m * D);
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int p = lane + 64 * i;
      if (p < D / 2) {
        float4 g = row[p];
        const float v0 = s.v[2 * p], v1 = s.v[2 * p + 1];
        float2 g0 = cfma(l, make_float2(g.x, g.y), make_float2(b.x * v0, b.y * v0));
        float2 g1 = cfma(l, make_float2(g.z, g.w), make_float2(b.x * v1, b.y * v1));
        row[p] = make_float4(g0.x, g0.y, g1.x, g1.y);
        acc[2 * i] += a.x * g0.x - a.y * g0.y;
        acc[2 * i + 1] += a.x * g1.x - a.y * g1.y;
      }
    }
  }
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int p = lane + 64 * i;
    if (p < D / 2) {
      s.num[wave][2 * p] = acc[2 * i];
      s.num[wave][2 * p + 1] = acc[2 * i + 1];
    }
  }
  if (wave == 0) {
    float d = 0.f;
    for (int m = lane; m < M; m += 64) d += A[m].x * s.eta[m].x - A[m].y * s.eta[m].y;
    d = wave_sum(d);
    if (lane == 0) s.den = d;
  }
  __syncthreads();
}

// phi(q), phi(k), v of one token into shared memory (BF: bf16 inputs, else f32).  Each thread
// issues its loads before converting any of them.
template <bool BF, int NW, int MF, int MD, int MM, bool WR>
__device__ __forceinline__ void seq_load_token(SeqSmem<NW, MF, MD, MM, WR>& s, const void* q,
                                               const void* k, const void* v, size_t qk_off,
                                               size_t v_off, int F, int D, int opt) {
  for (int i = threadIdx.x; i < F || i < D; i += 64 * NW) {
    float xq = 0.f, xk = 0.f, xv = 0.f;
    if (i < F) {
      xq = load_t<BF>(q, qk_off + i);
      xk = load_t<BF>(k, qk_off + i);
    }
    if (i < D) xv = load_t<BF>(v, v_off + i);
    if (i < F) {
      s.fq[i] = feat(xq, opt);
      s.fk[i] = feat(xk, opt);
    }
    if (i < D) s.v[i] = xv;
  }
}

template <int NW, int MF, int MD, int MM, bool WR>
__device__ __forceinline__ void seq_load_modes(SeqSmem<NW, MF, MD, MM, WR>& s,
                                               const float2* lam, const float2* beta, int h,
                                               int M) {
  for (int m = threadIdx.x; m < M; m += 64 * NW) {
    s.lam[m] = lam[(size_t)h * M + m];
    s.beta[m] = beta[(size_t)h * M + m];
  }
}

// Numerator of output column j: the per-wave partial sums added in a fixed order.
template <int NW, int MF, int MD, int MM, bool WR>
__device__ __forceinline__ float seq_num(const SeqSmem<NW, MF, MD, MM, WR>& s, int j) {
  float n = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) n += s.num[w][j];
  return n;
}

// The whole sequence of slice (b, h) from the state (U, G, E) (updated in place to the state
// after the last token), walking positions N-1 .. 0 when `reverse` is set, with the write and
// decay gates of each position when given (selective writing and memory decay, summary page
// §3.3: lambda_m -> dg lambda_m, beta_m -> wg beta_m at that token).  q, k and v are
// addressed through their element strides; o is dense [B][N][H][D] (o + value with
// `accumulate`), or NULL for a state-only walk.
struct SeqScanArgs {
  const void *q, *k, *v;
  RowStrides sqk, sv;
  const float2 *lam, *beta;
  void* o;
  int accumulate;
  int N, H, F, D, M;
  int in_bf16, out_bf16;
  float clamp;
  int reverse;
  int opt;
  const float2* readout;   // [H][M][M] or NULL
  const float *wgate = nullptr, *dgate = nullptr;   // [B][N][H] write / decay gates, or NULL
};

template <bool BF, int NW, int MF, int MD, int MM, bool WR>
__device__ __forceinline__ void seq_scan_t(SeqSmem<NW, MF, MD, MM, WR>& s, const SeqScanArgs& a,
                                           int b, int h, float2* U, float2* G, float2* E) {
  seq_load_modes(s, a.lam, a.beta, h, a.M);
  const float2* R = a.readout ? a.readout + (size_t)h * a.M * a.M : nullptr;
  for (int t = 0; t < a.N; ++t) {
    const int pos = a.reverse ? a.N - 1 - t : t;
    const size_t tok = ((size_t)b * a.N + pos) * a.H + h;
    seq_load_token<BF>(s, a.q, a.k, a.v, (size_t)(b * a.sqk.b + pos * a.sqk.n + h * a.sqk.h),
                       (size_t)(b * a.sv.b + pos * a.sv.n + h * a.sv.h), a.F, a.D, a.opt);
    const size_t gi = ((size_t)b * a.N + pos) * a.H + h;
    const float wg = a.wgate ? a.wgate[gi] : 1.f, dg = a.dgate ? a.dgate[gi] : 1.f;
    __syncthreads();
    seq_step(s, U, G, E, a.F, a.D, a.M, R, wg, dg);
    if (a.o) {
      for (int j = threadIdx.x; j < a.D; j += 64 * NW) {
        float val = readout(seq_num(s, j), s.den, a.clamp, a.opt);
        if (a.accumulate) val += load_in(a.o, tok * a.D + j, a.out_bf16);
        store_out(a.o, tok * a.D + j, val, a.out_bf16);
      }
    }
    __syncthreads();
  }
}

template <int NW, int MF, int MD, int MM, bool WR>
__device__ __forceinline__ void seq_scan(SeqSmem<NW, MF, MD, MM, WR>& s, const SeqScanArgs& a,
                                         int b, int h, float2* U, float2* G, float2* E) {
  if (a.in_bf16)
    seq_scan_t<true>(s, a, b, h, U, G, E);
  else
    seq_scan_t<false>(s, a, b, h, U, G, E);
}

}  // namespace ia
