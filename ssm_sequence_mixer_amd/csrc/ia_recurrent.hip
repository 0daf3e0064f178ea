// ia_recurrent.hip — token-by-token IA kernels (fp32 VALU): the decode step, the
// token-sequential fp32 prefill, and the state fill and copy.
//
// The step is the recurrence and readout of the layer ("Interdomain Attention: Beyond
// Token-Level Key-Value Memory": summary page §3.2 for the complex-diagonal S4D recurrence and
// the O(M(R+d)) per-step decode; episode page, "Key Components and Derivation", for the
// feature map and the matrix form Fq U^T Gamma / Fq U^T eta), written once in ia_scan.hpp.
// One workgroup owns one (b,h) slice.
#include "ia_block_step.hpp"
#include "ia_device.hpp"
#include "ia_kernels.hpp"
#include "ia_scan.hpp"

namespace ia {

constexpr int kStepThreads = 256;
constexpr int kStepWaves = kStepThreads / 64;
// MM: the largest M a kernel instance takes (64 or kMaxModes; the smaller set keeps the per-wave
// row partials, and so the registers, small for the common sizes).
template <int MM>
using StepSmem = SeqSmem<kStepWaves, kMaxDim, kMaxDim, MM, true>;

// ---------------------------------------------------------------- kernels

// Decode: one step for every (b,h).  grid = B*H.  BF: bf16 inputs; M <= MM.  PRO: q, k, v
// are the raw projections, the block's prologue (blk) makes the step's inputs and its output
// gate scales the readout.
template <bool BF, int MM, bool PRO>
__global__ void __launch_bounds__(kStepThreads)
decode_step_kernel(const void* __restrict__ q, const void* __restrict__ k,
                   const void* __restrict__ v, const float2* __restrict__ lam,
                   const float2* __restrict__ beta, float2* __restrict__ U,
                   float2* __restrict__ G, float2* __restrict__ E, void* __restrict__ o,
                   int H, int F, int D, int M, int out_bf16, float clamp,
                   int opt, const float2* __restrict__ rmat, const float* __restrict__ wgate,
                   const float* __restrict__ dgate, const BlockStepArgs blk) {
  __shared__ StepSmem<MM> s;
  __shared__ float s_red[kStepWaves];
  __shared__ __align__(16) float s_w[PRO ? 3 * kMaxDim * kMaxConvTaps : 4];
  const int bh = blockIdx.x;
  const int h = bh % H;
  seq_load_modes(s, lam, beta, h, M);
  if constexpr (PRO) {
    static_assert(2 * kStepThreads >= kMaxDim + kMaxDim / 2, "two channel pairs per thread");
    constexpr int NW4 = (3 * kMaxDim * kMaxConvTaps / 4 + kStepThreads - 1) / kStepThreads;
    BlockToken<2, NW4> tok;
    tok.template load<BF>(blk, q, k, v, bh, h, F, D);
    tok.finish(blk, bh, F, D, s.fq, s.fk, s.v, s_w, s_red);
  } else {
    seq_load_token<BF>(s, q, k, v, (size_t)bh * F, (size_t)bh * D, F, D, opt);
  }
  __syncthreads();
  seq_step(s, U + (size_t)bh * M * F, G + (size_t)bh * M * D, E + (size_t)bh * M, F, D, M,
           rmat ? rmat + (size_t)h * M * M : nullptr, wgate ? wgate[bh] : 1.f,
           dgate ? dgate[bh] : 1.f);
  for (int j = threadIdx.x; j < D; j += kStepThreads) {
    float y = readout(seq_num(s, j), s.den, clamp, opt);
    if (PRO && blk.gate) y *= silu_f(load_t<BF>(blk.gate, (size_t)bh * D + j));
    store_out(o, (size_t)bh * D + j, y, out_bf16);
  }
}

// The row sums a[m] = (sum of ar, sum of ai over the RU lanes holding row m's columns) of the
// rows m = ru + SU i (i < IU) into s_a[m].  With 64-lane rows (RU = 64: a wave holds rows ru +
// SU i of one set of columns) the 2 IU values reduce-scatter over the wave (scatter_totals16,
// 16 values at a time) and one lane of each group of eight writes its row; otherwise each row's
// lanes sum by DPP moves (row_totals), all rows' chains interleaved, and the row's last lane
// writes it.
template <int RU, int SU, int IU>
__device__ __forceinline__ void row_sums_to_lds(float (&ar)[IU], float (&ai)[IU], int ru, int M,
                                                float2* s_a) {
  const int lane = threadIdx.x & 63;
  if constexpr (RU == 64 && IU % 8 == 0) {
#pragma unroll
    for (int i0 = 0; i0 < IU; i0 += 8) {
      float v[16];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        v[2 * i] = ar[i0 + i];
        v[2 * i + 1] = ai[i0 + i];
      }
      float z0, z1;
      scatter_totals16(v, z0, z1);
      if ((lane & 7) == 0) {   // this group holds values T, T + 1: row i0 + T / 2
        const int i = i0 + ((lane >> 3) & 1) + 2 * ((lane >> 4) & 1) + 4 * (lane >> 5);
        const int m = ru + SU * i;
        if (m < M) s_a[m] = make_float2(z0, z1);
      }
    }
  } else {
    row_totals<RU>(ar);
    row_totals<RU>(ai);
    if (threadIdx.x % RU == RU - 1) {
#pragma unroll
      for (int i = 0; i < IU; ++i) {
        const int m = ru + SU * i;
        if (m < M) s_a[m] = make_float2(ar[i], ai[i]);
      }
    }
  }
}

// Decode with the whole state of a slice in flight at once.  grid = B*H; NT threads per slice.
// A state row of F complex values is F/2 float4 (2 complex each); thread t owns float4 column
// pu = t % (F/2) of the U rows m = t / (F/2) + (NT/(F/2)) i, and likewise column pd of the
// Gamma rows, so its inputs are two entries each of phi(q), phi(k) and v.  Every row load is
// issued before any arithmetic; a[m] needs all of row m (a reduction over the F/2 lanes that
// share it), then the Gamma rows, whose column sums over rows go through LDS in a fixed order.
// PRO: as decode_step_kernel; the prologue's loads go out before the state's.
template <int F, int D, int MM, bool BF, bool PRO>
__global__ void __launch_bounds__(512)
decode_step_rows_kernel(const void* __restrict__ q, const void* __restrict__ k,
                        const void* __restrict__ v, const float2* __restrict__ lam,
                        const float2* __restrict__ beta, float2* __restrict__ U,
                        float2* __restrict__ G, float2* __restrict__ E, void* __restrict__ o,
                        int H, int M, int out_bf16, float clamp, int opt,
                        const float2* __restrict__ rmat, const float* __restrict__ wgate,
                        const float* __restrict__ dgate, const BlockStepArgs blk) {
  constexpr int NT = 512, NWV = NT / 64;
  constexpr int RU = F / 2, RD = D / 2;
  static_assert(RU <= 64 && RD <= 64 && NT % RU == 0 && NT % RD == 0, "row width");
  constexpr int SU = NT / RU, SD = NT / RD;                  // rows per pass
  constexpr int IU = (MM + SU - 1) / SU, ID = (MM + SD - 1) / SD;   // M <= MM
  __shared__ float2 s_lam[kMaxModes], s_beta[kMaxModes], s_a[kMaxModes], s_ar[kMaxModes];
  __shared__ float2 s_rp[NT];   // partial sums of a R
  __shared__ float s_num[SD][D];
  __shared__ float s_den[NWV];
  __shared__ float s_pro[PRO ? 2 * F + D : 1];   // phi(q'), then the normalised phi(k'), v'
  __shared__ __align__(16) float s_w[PRO ? (2 * F + D) * kMaxConvTaps : 4];   // the taps

  const int bh = blockIdx.x, h = bh % H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int pu = tid % RU, ru = tid / RU, pd = tid % RD, rd = tid / RD;
  float4* Ub = reinterpret_cast<float4*>(U + (size_t)bh * M * F);
  float4* Gb = reinterpret_cast<float4*>(G + (size_t)bh * M * D);
  float2* Eb = E + (size_t)bh * M;
  // this token's inputs first: the state loads below stay in flight behind them
  float2 kk, qq, vv;
  BlockToken<1, ((2 * F + D) * kMaxConvTaps / 4 + NT - 1) / NT> tok;
  float gt = 0.f;
  if constexpr (PRO) {
    static_assert(NT >= F + D / 2, "one channel pair per thread");
    tok.template load<BF>(blk, q, k, v, bh, h, F, D);
    // the gate of output tid (tid < D), loaded unconditionally from a valid address (q's own
    // row without a gate) so that no branch holds the loads above waiting
    gt = blk.gate ? load_t<BF>(blk.gate, (size_t)bh * D + min(tid, D - 1))
                  : load_t<BF>(q, (size_t)bh * F + min(tid, F - 1));
  } else {
    kk = load_pair_t<BF>(k, (size_t)bh * F + 2 * pu);
    qq = load_pair_t<BF>(q, (size_t)bh * F + 2 * pu);
    vv = load_pair_t<BF>(v, (size_t)bh * D + 2 * pd);
  }
  // lambda, beta, eta and the gates: loads without branches (indices clamped, lambda standing
  // in for a missing gate) so that none of them waits before the state's loads go out
  const int mt = min(tid, M - 1);
  const float2 lv = lam[(size_t)h * M + mt], bv = beta[(size_t)h * M + mt];
  float2 e = Eb[mt];   // used by threads tid < M only
  const float wgv = *(wgate ? wgate + bh : reinterpret_cast<const float*>(lam));
  const float dgv = *(dgate ? dgate + bh : reinterpret_cast<const float*>(lam));

  // the whole state, U and Gamma rows together; unconditional (rows past M read row M-1 and
  // go unused) so that the compiler keeps them here, ahead of any arithmetic, and waits for
  // the earlier loads only where those are used
  float4 u[IU], g[ID];
#pragma unroll
  for (int i = 0; i < IU; ++i) u[i] = Ub[(size_t)min(ru + SU * i, M - 1) * RU + pu];
#pragma unroll
  for (int i = 0; i < ID; ++i) g[i] = Gb[(size_t)min(rd + SD * i, M - 1) * RD + pd];
  float fk0, fk1, fq0, fq1, v0, v1;
  if constexpr (PRO) {
    tok.finish(blk, bh, F, D, s_pro, s_pro + F, s_pro + 2 * F, s_w, s_den);
    fq0 = s_pro[2 * pu];
    fq1 = s_pro[2 * pu + 1];
    fk0 = s_pro[F + 2 * pu];
    fk1 = s_pro[F + 2 * pu + 1];
    v0 = s_pro[2 * F + 2 * pd];
    v1 = s_pro[2 * F + 2 * pd + 1];
  } else {
    fk0 = feat(kk.x, opt);
    fk1 = feat(kk.y, opt);
    fq0 = feat(qq.x, opt);
    fq1 = feat(qq.y, opt);
    v0 = vv.x;
    v1 = vv.y;
  }
  // with gates, lambda_m and beta_m of this slice's step times its decay and write gate
  const float wg = wgate ? wgv : 1.f, dg = dgate ? dgv : 1.f;
  if (tid < M) {
    s_lam[tid] = make_float2(dg * lv.x, dg * lv.y);
    s_beta[tid] = make_float2(wg * bv.x, wg * bv.y);
  }
  __syncthreads();   // lam, beta

  if (tid < M) {
    e = cfma(s_lam[tid], e, s_beta[tid]);
    Eb[tid] = e;
  }
  // U rows: update, store, contract with phi(q) over the row's lanes.
  float ar[IU], ai[IU];
#pragma unroll
  for (int i = 0; i < IU; ++i) {
    const int m = ru + SU * i;
    if (m < M) {
      const float2 l = s_lam[m], bt = s_beta[m];
      const float2 u0 = cfma(l, make_float2(u[i].x, u[i].y), make_float2(bt.x * fk0, bt.y * fk0));
      const float2 u1 = cfma(l, make_float2(u[i].z, u[i].w), make_float2(bt.x * fk1, bt.y * fk1));
      Ub[(size_t)m * RU + pu] = make_float4(u0.x, u0.y, u1.x, u1.y);
      ar[i] = fq0 * u0.x + fq1 * u1.x;
      ai[i] = fq0 * u0.y + fq1 * u1.y;
    } else {
      ar[i] = ai[i] = 0.f;
    }
  }
  // each row's RU lane partials summed (row_sums_to_lds), a[m] into LDS
  row_sums_to_lds<RU, SU, IU>(ar, ai, ru, M, s_a);
  __syncthreads();   // a[m]
  // with a readout matrix R ([H][M][M]), the readouts use (a R)[n] = sum_m a[m] R[m][n]
  if (rmat) {
    // thread t sums the modes m = t / M, t / M + parts, ... of column n = t % M (coalesced
    // rows of R), then M threads add the parts
    const float2* Rh = rmat + (size_t)h * M * M;
    const int parts = NT / M, n = tid % M, part = tid / M;
    if (part < parts) {
      float2 acc = make_float2(0.f, 0.f);
      for (int m = part; m < M; m += parts) acc = cfma(s_a[m], Rh[(size_t)m * M + n], acc);
      s_rp[tid] = acc;
    }
    __syncthreads();
    if (tid < M) {
      float2 acc = make_float2(0.f, 0.f);
      for (int p = 0; p < parts; ++p) acc = cadd2(acc, s_rp[p * M + tid]);
      s_ar[tid] = acc;
    }
    __syncthreads();
  }
  const float2* A = rmat ? s_ar : s_a;

  float dn = tid < M ? A[tid].x * e.x - A[tid].y * e.y : 0.f;
  dn = wave_sum(dn);
  if (lane == 0) s_den[wave] = dn;
  // Gamma rows: update, store, accumulate Re(a[m] G[m, 2pd..2pd+1]).
  float n0 = 0.f, n1 = 0.f;
#pragma unroll
  for (int i = 0; i < ID; ++i) {
    const int m = rd + SD * i;
    if (m < M) {
      const float2 l = s_lam[m], bt = s_beta[m], am = A[m];
      const float2 g0 = cfma(l, make_float2(g[i].x, g[i].y), make_float2(bt.x * v0, bt.y * v0));
      const float2 g1 = cfma(l, make_float2(g[i].z, g[i].w), make_float2(bt.x * v1, bt.y * v1));
      Gb[(size_t)m * RD + pd] = make_float4(g0.x, g0.y, g1.x, g1.y);
      n0 += am.x * g0.x - am.y * g0.y;
      n1 += am.x * g1.x - am.y * g1.y;
    }
  }
  s_num[rd][2 * pd] = n0;
  s_num[rd][2 * pd + 1] = n1;
  __syncthreads();
  if (tid < D) {
    float n = 0.f;
#pragma unroll
    for (int r = 0; r < SD; ++r) n += s_num[r][tid];
    float den = 0.f;
#pragma unroll
    for (int w = 0; w < NWV; ++w) den += s_den[w];
    float y = readout(n, den, clamp, opt);
    if (PRO && blk.gate) y *= silu_f(gt);
    store_out(o, (size_t)bh * D + tid, y, out_bf16);
  }
}

// Token-sequential prefill with the slice's whole state in registers: one 512-thread
// workgroup per (b,h) slice walks its N tokens (positions N-1..0 with `reverse`) in the layout
// of decode_step_rows_kernel -- thread t holds float4 column pu of the U rows ru + SU i and
// column pd of the Gamma rows rd + SD i -- reading the state once before the first token and
// writing it once after the last.  Each token's q, k, v pairs and gates are loaded one token
// ahead.  Per token: the U rows' update and their a[m] (DPP row totals, LDS), a barrier, the
// readout matrix if any, the Gamma rows' update and their column sums (LDS), a barrier, the
// output.  Arithmetic as seq_step (gates: lambda times the decay gate, beta times the write
// gate), with its own summation order.
// Segments (a.n_seg > 1): blockIdx.y is the segment, walk steps [y L, min(N, (y+1) L)).
// LOCAL: the state-only pass of segments 0..n_seg-2 from a zero state: their end states go to
// slots y+1 and the products of the per-token decays (decay gate times lambda, per mode) to
// dec; no output.  Otherwise segment y starts from slot y (n_seg > 1) or from U, Gamma, eta,
// and the last segment writes the final state to U, Gamma, eta.
template <int F, int D, int MM, bool BF, bool LOCAL>
__global__ void __launch_bounds__(512)
scan_rows_kernel(const ScanArgs a) {
  constexpr int NT = 512, NWV = NT / 64;
  constexpr int RU = F / 2, RD = D / 2;
  static_assert(RU <= 64 && RD <= 64 && NT % RU == 0 && NT % RD == 0, "row width");
  constexpr int SU = NT / RU, SD = NT / RD;
  constexpr int IU = (MM + SU - 1) / SU, ID = (MM + SD - 1) / SD;
  __shared__ float2 s_lam[kMaxModes], s_beta[kMaxModes], s_a[kMaxModes], s_ar[kMaxModes];
  __shared__ float2 s_rp[NT];
  __shared__ float s_num[SD][D];
  __shared__ float s_den[NWV];

  const int M = a.M, N = a.N, H = a.H;
  const int bh = blockIdx.x, b = bh / H, h = bh % H, BH = a.B * H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int pu = tid % RU, ru = tid / RU, pd = tid % RD, rd = tid / RD;
  const int seg = blockIdx.y, segmented = a.n_seg > 1;
  const int t_begin = segmented ? seg * a.seg_len : 0;
  const int t_end = segmented ? min(N, t_begin + a.seg_len) : N;
  // where this workgroup's state starts and ends
  const long slot = scan_slot_float2(F, D, M);
  auto slot_of = [&](int g) { return a.slots + ((size_t)g * BH + bh) * slot; };
  float2* const in = LOCAL ? nullptr
                           : (segmented ? slot_of(seg) : nullptr);
  float2* const out = LOCAL ? slot_of(seg + 1) : nullptr;
  const bool last = !LOCAL && (!segmented || seg == a.n_seg - 1);
  float4* Ub = reinterpret_cast<float4*>(in ? in : a.U + (size_t)bh * M * F);
  float4* Gb = reinterpret_cast<float4*>(in ? in + (size_t)M * F : a.G + (size_t)bh * M * D);
  float2* Eb = in ? in + (size_t)M * (F + D) : a.E + (size_t)bh * M;
  const float2* R = a.readout ? a.readout + (size_t)h * M * M : nullptr;
  const float* dummy = reinterpret_cast<const float*>(a.lam);   // a valid address

  // one token's inputs: the thread's pairs and the gates (loads without branches)
  struct Tok {
    float2 q, k, v;
    float wg, dg;
  };
  auto load_tok = [&](int t) {
    const int pos = a.reverse ? N - 1 - t : t;
    const size_t qk = (size_t)(b * a.sqk.b + pos * a.sqk.n + h * a.sqk.h);
    const size_t vo = (size_t)(b * a.sv.b + pos * a.sv.n + h * a.sv.h);
    const size_t gi = ((size_t)b * N + pos) * H + h;
    Tok x;
    x.k = load_pair_t<BF>(a.k, qk + 2 * pu);
    x.q = load_pair_t<BF>(a.q, qk + 2 * pu);
    x.v = load_pair_t<BF>(a.v, vo + 2 * pd);
    x.wg = *(a.wgate ? a.wgate + gi : dummy);
    x.dg = *(a.dgate ? a.dgate + gi : dummy);
    return x;
  };
  Tok nxt = load_tok(t_begin);

  // the state (zero for the state-only pass), unconditional loads (rows past M read row M-1
  // and stay unused)
  float4 u[IU], g[ID];
  const int mt = min(tid, M - 1);
  float2 e;   // used by threads tid < M only
  if constexpr (LOCAL) {
#pragma unroll
    for (int i = 0; i < IU; ++i) u[i] = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int i = 0; i < ID; ++i) g[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    e = make_float2(0.f, 0.f);
  } else {
#pragma unroll
    for (int i = 0; i < IU; ++i) u[i] = Ub[(size_t)min(ru + SU * i, M - 1) * RU + pu];
#pragma unroll
    for (int i = 0; i < ID; ++i) g[i] = Gb[(size_t)min(rd + SD * i, M - 1) * RD + pd];
    e = Eb[mt];
  }
  float2 dprod = make_float2(1.f, 0.f);   // LOCAL: product of the decays, mode tid
  const float2 lv = a.lam[(size_t)h * M + mt], bv = a.beta[(size_t)h * M + mt];
  if (tid < M) {
    s_lam[tid] = lv;
    s_beta[tid] = bv;
  }
  __syncthreads();

  for (int t = t_begin; t < t_end; ++t) {
    const Tok cur = nxt;
    nxt = load_tok(min(t + 1, t_end - 1));
    const float wg = a.wgate ? cur.wg : 1.f, dg = a.dgate ? cur.dg : 1.f;
    const float fk0 = feat(cur.k.x, a.opt), fk1 = feat(cur.k.y, a.opt);
    const float fq0 = feat(cur.q.x, a.opt), fq1 = feat(cur.q.y, a.opt);
    const float v0 = cur.v.x, v1 = cur.v.y;

    if (tid < M) {
      const float2 l = s_lam[tid], bt = s_beta[tid];
      const float2 ld = make_float2(dg * l.x, dg * l.y);
      e = cfma(ld, e, make_float2(wg * bt.x, wg * bt.y));
      if constexpr (LOCAL) dprod = cmul(ld, dprod);
    }
    if constexpr (LOCAL) {
      // the state update alone: no readout, so no barrier
#pragma unroll
      for (int i = 0; i < IU; ++i) {
        const int m = ru + SU * i;
        if (m < M) {
          const float2 l0 = s_lam[m], b0 = s_beta[m];
          const float2 l = make_float2(dg * l0.x, dg * l0.y);
          const float2 bt = make_float2(wg * b0.x, wg * b0.y);
          const float2 u0 =
              cfma(l, make_float2(u[i].x, u[i].y), make_float2(bt.x * fk0, bt.y * fk0));
          const float2 u1 =
              cfma(l, make_float2(u[i].z, u[i].w), make_float2(bt.x * fk1, bt.y * fk1));
          u[i] = make_float4(u0.x, u0.y, u1.x, u1.y);
        }
      }
#pragma unroll
      for (int i = 0; i < ID; ++i) {
        const int m = rd + SD * i;
        if (m < M) {
          const float2 l0 = s_lam[m], b0 = s_beta[m];
          const float2 l = make_float2(dg * l0.x, dg * l0.y);
          const float2 bt = make_float2(wg * b0.x, wg * b0.y);
          const float2 g0 = cfma(l, make_float2(g[i].x, g[i].y), make_float2(bt.x * v0, bt.y * v0));
          const float2 g1 = cfma(l, make_float2(g[i].z, g[i].w), make_float2(bt.x * v1, bt.y * v1));
          g[i] = make_float4(g0.x, g0.y, g1.x, g1.y);
        }
      }
      continue;
    }
    // U rows: update in registers, contract with phi(q) over the row's lanes
    float ar[IU], ai[IU];
#pragma unroll
    for (int i = 0; i < IU; ++i) {
      const int m = ru + SU * i;
      if (m < M) {
        const float2 l0 = s_lam[m], b0 = s_beta[m];
        const float2 l = make_float2(dg * l0.x, dg * l0.y), bt = make_float2(wg * b0.x, wg * b0.y);
        const float2 u0 = cfma(l, make_float2(u[i].x, u[i].y), make_float2(bt.x * fk0, bt.y * fk0));
        const float2 u1 = cfma(l, make_float2(u[i].z, u[i].w), make_float2(bt.x * fk1, bt.y * fk1));
        u[i] = make_float4(u0.x, u0.y, u1.x, u1.y);
        ar[i] = fq0 * u0.x + fq1 * u1.x;
        ai[i] = fq0 * u0.y + fq1 * u1.y;
      } else {
        ar[i] = ai[i] = 0.f;
      }
    }
    row_sums_to_lds<RU, SU, IU>(ar, ai, ru, M, s_a);
    __syncthreads();   // a[m]
    if (R) {   // (a R)[n] = sum_m a[m] R[m][n], as the decode step
      const int parts = NT / M, n = tid % M, part = tid / M;
      if (part < parts) {
        float2 acc = make_float2(0.f, 0.f);
        for (int m = part; m < M; m += parts) acc = cfma(s_a[m], R[(size_t)m * M + n], acc);
        s_rp[tid] = acc;
      }
      __syncthreads();
      if (tid < M) {
        float2 acc = make_float2(0.f, 0.f);
        for (int p = 0; p < parts; ++p) acc = cadd2(acc, s_rp[p * M + tid]);
        s_ar[tid] = acc;
      }
      __syncthreads();
    }
    const float2* A = R ? s_ar : s_a;
    float dn = tid < M ? A[tid].x * e.x - A[tid].y * e.y : 0.f;
    dn = wave_sum(dn);
    if (lane == 0) s_den[wave] = dn;
    // Gamma rows: update in registers, accumulate Re(a[m] G[m, 2pd..2pd+1])
    float n0 = 0.f, n1 = 0.f;
#pragma unroll
    for (int i = 0; i < ID; ++i) {
      const int m = rd + SD * i;
      if (m < M) {
        const float2 l0 = s_lam[m], b0 = s_beta[m], am = A[m];
        const float2 l = make_float2(dg * l0.x, dg * l0.y), bt = make_float2(wg * b0.x, wg * b0.y);
        const float2 g0 = cfma(l, make_float2(g[i].x, g[i].y), make_float2(bt.x * v0, bt.y * v0));
        const float2 g1 = cfma(l, make_float2(g[i].z, g[i].w), make_float2(bt.x * v1, bt.y * v1));
        g[i] = make_float4(g0.x, g0.y, g1.x, g1.y);
        n0 += am.x * g0.x - am.y * g0.y;
        n1 += am.x * g1.x - am.y * g1.y;
      }
    }
    s_num[rd][2 * pd] = n0;
    s_num[rd][2 * pd + 1] = n1;
    __syncthreads();   // numerator parts, den
    if (a.o && tid < D) {
      float n = 0.f;
#pragma unroll
      for (int r = 0; r < SD; ++r) n += s_num[r][tid];
      float den = 0.f;
#pragma unroll
      for (int w = 0; w < NWV; ++w) den += s_den[w];
      const int pos = a.reverse ? N - 1 - t : t;
      const size_t oi = (((size_t)b * N + pos) * H + h) * D + tid;
      float val = readout(n, den, a.clamp, a.opt);
      if (a.accumulate) val += load_in(a.o, oi, a.out_bf16);
      store_out(a.o, oi, val, a.out_bf16);
    }
  }

  // the state after the segment's last token: the slot of the next segment's start (LOCAL),
  // or the final state (the last segment)
  if (!LOCAL && !last) return;
  float4* Uo = reinterpret_cast<float4*>(LOCAL ? out : a.U + (size_t)bh * M * F);
  float4* Go = reinterpret_cast<float4*>(LOCAL ? out + (size_t)M * F : a.G + (size_t)bh * M * D);
  float2* Eo = LOCAL ? out + (size_t)M * (F + D) : a.E + (size_t)bh * M;
#pragma unroll
  for (int i = 0; i < IU; ++i) {
    const int m = ru + SU * i;
    if (m < M) Uo[(size_t)m * RU + pu] = u[i];
  }
#pragma unroll
  for (int i = 0; i < ID; ++i) {
    const int m = rd + SD * i;
    if (m < M) Go[(size_t)m * RD + pd] = g[i];
  }
  if (tid < M) {
    Eo[tid] = e;
    if constexpr (LOCAL) a.dec[((size_t)seg * BH + bh) * M + tid] = dprod;
  }
}

// The segment starts: slot 0 takes the initial state (U, Gamma, eta), then slot g+1 (holding
// segment g's end state from zero) becomes dec_g * slot g + slot g+1, per complex entry and its
// mode.  One thread per complex entry of all slices' states, the segments in order.
__global__ void __launch_bounds__(256)
scan_carry_kernel(const ScanArgs a) {
  const int M = a.M, F = a.F, D = a.D, BH = a.B * a.H;
  const long per = scan_slot_float2(F, D, M);
  const long x = blockIdx.x * 256L + threadIdx.x;
  if (x >= per * BH) return;
  const int bh = (int)(x / per);
  const long r = x % per;
  const int m = r < (long)M * F ? (int)(r / F)
                : r < (long)M * (F + D) ? (int)((r - (long)M * F) / D)
                                        : (int)(r - (long)M * (F + D));
  float2 s = r < (long)M * F ? a.U[(size_t)bh * M * F + r]
             : r < (long)M * (F + D) ? a.G[(size_t)bh * M * D + (r - (long)M * F)]
                                     : a.E[(size_t)bh * M + (r - (long)M * (F + D))];
  a.slots[(size_t)bh * per + r] = s;
  for (int g = 0; g + 1 < a.n_seg; ++g) {
    float2* nx = a.slots + ((size_t)(g + 1) * BH + bh) * per + r;
    s = cfma(a.dec[((size_t)g * BH + bh) * M + m], s, *nx);
    *nx = s;
  }
}

// Token-sequential prefill (the fp32 path).  M <= MM.  grid = B*H; one workgroup walks all N tokens of
// its slice, in reverse when `reverse` is set (then token t of the walk is position N-1-t).
// q, k and v are addressed through their element strides sqk, sv; o is dense.
// o (out dtype) receives value, or o + value with `accumulate` (the second direction of the
// bidirectional layer adds onto the first); o may be NULL (state only).
template <int MM>
__global__ void __launch_bounds__(kStepThreads)
scan_prefill_kernel(const void* __restrict__ q, const void* __restrict__ k,
                    const void* __restrict__ v, const float2* __restrict__ lam,
                    const float2* __restrict__ beta, float2* __restrict__ U,
                    float2* __restrict__ G, float2* __restrict__ E, void* __restrict__ o,
                    int accumulate, int N, int H, int F, int D, int M,
                    int in_bf16, int out_bf16, float clamp, int reverse, RowStrides sqk,
                    RowStrides sv, int opt, const float2* __restrict__ rmat,
                    const float* __restrict__ wgate, const float* __restrict__ dgate) {
  __shared__ StepSmem<MM> s;
  const int bh = blockIdx.x;
  const int b = bh / H, h = bh % H;
  const SeqScanArgs a{q, k, v, sqk, sv, lam, beta, o, accumulate, N, H, F, D, M,
                      in_bf16, out_bf16, clamp, reverse, opt, rmat, wgate, dgate};
  seq_scan(s, a, b, h, U + (size_t)bh * M * F, G + (size_t)bh * M * D, E + (size_t)bh * M);
}

__global__ void fill_zero_kernel(float4* __restrict__ p, size_t n4) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n4;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

// Copy of up to three buffers (16-byte units), in one launch.
__global__ void copy3_kernel(float4* __restrict__ d0, const float4* __restrict__ s0, size_t n0,
                             float4* __restrict__ d1, const float4* __restrict__ s1, size_t n1,
                             float4* __restrict__ d2, const float4* __restrict__ s2, size_t n2) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n0 + n1 + n2; i += stride) {
    if (i < n0) d0[i] = s0[i];
    else if (i < n0 + n1) d1[i - n0] = s1[i - n0];
    else d2[i - n0 - n1] = s2[i - n0 - n1];
  }
}

// ---------------------------------------------------------------- launchers

hipError_t launch_copy3(void* d0, const void* s0, size_t n0, void* d1, const void* s1,
                        size_t n1, void* d2, const void* s2, size_t n2, hipStream_t st) {
  const size_t n = (n0 + n1 + n2) / 16;
  if (n == 0) return hipSuccess;
  unsigned grid = static_cast<unsigned>(n / 256 + 1 < 4096 ? n / 256 + 1 : 4096);
  (void)hipGetLastError();
  prof_begin(st);
  hipLaunchKernelGGL(copy3_kernel, dim3(grid), dim3(256), 0, st, static_cast<float4*>(d0),
                     static_cast<const float4*>(s0), n0 / 16, static_cast<float4*>(d1),
                     static_cast<const float4*>(s1), n1 / 16, static_cast<float4*>(d2),
                     static_cast<const float4*>(s2), n2 / 16);
  prof_end(st, kKindCopy);
  return hipGetLastError();
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t st) {
  // bytes is a multiple of 16 for every state buffer (F, Dv, M multiples of 16).
  size_t n4 = bytes / 16;
  if (n4 == 0) return hipSuccess;
  unsigned grid = static_cast<unsigned>(n4 / 256 + 1 < 4096 ? n4 / 256 + 1 : 4096);
  (void)hipGetLastError();
  prof_begin(st);
  hipLaunchKernelGGL(fill_zero_kernel, dim3(grid), dim3(256), 0, st,
                     static_cast<float4*>(p), n4);
  prof_end(st, kKindFill);
  return hipGetLastError();
}

template <int F, int D, bool BF, bool PRO>
static void launch_decode_rows_t(const DecodeArgs& a, hipStream_t st) {
  // The per-thread row registers are sized for M <= 64 or M <= 128: the smaller set lets two
  // workgroups share a CU.
  if (a.M <= 64)
    hipLaunchKernelGGL((decode_step_rows_kernel<F, D, 64, BF, PRO>), dim3(a.B * a.H), dim3(512),
                       0, st, a.q, a.k, a.v, a.lam, a.beta, a.U, a.G, a.E, a.o, a.H, a.M,
                       a.out_bf16, a.clamp, a.opt, a.readout, a.wgate, a.dgate, a.blk);
  else
    hipLaunchKernelGGL((decode_step_rows_kernel<F, D, kMaxModes, BF, PRO>), dim3(a.B * a.H),
                       dim3(512), 0, st, a.q, a.k, a.v, a.lam, a.beta, a.U, a.G, a.E, a.o, a.H,
                       a.M, a.out_bf16, a.clamp, a.opt, a.readout, a.wgate, a.dgate, a.blk);
}

template <int F, int D>
static void launch_decode_rows(const DecodeArgs& a, hipStream_t st) {
  if (a.in_bf16) {
    if (a.block) launch_decode_rows_t<F, D, true, true>(a, st);
    else launch_decode_rows_t<F, D, true, false>(a, st);
  } else {
    if (a.block) launch_decode_rows_t<F, D, false, true>(a, st);
    else launch_decode_rows_t<F, D, false, false>(a, st);
  }
}

// Compute units of the current device (cached per device; 256 when there is none).
int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

hipError_t launch_decode_step(const DecodeArgs& a, hipStream_t st) {
  (void)hipGetLastError();
  prof_begin(st);
  // Row-parallel kernel (row widths up to 64 float4: F, Dv in {32, 64, 128}) while there are
  // fewer than eight slices per CU; with more, the small mode-looping kernel keeps every slice
  // resident at once.  (Measured on MI355X at H=16, F=Dv=128, M=64, graph-captured: rows
  // 39.5 us against 41.7 us at B=64; the row kernel's loads and reductions were since made
  // latency-lean, which moved the crossover up from four slices per CU.)
  const bool rows = (long)a.B * a.H < 8L * device_cus();
#define IA_DEC(FF, DD) \
  if (rows && a.F == FF && a.D == DD) { launch_decode_rows<FF, DD>(a, st); } else
  IA_DEC(32, 32) IA_DEC(32, 64) IA_DEC(32, 128)
  IA_DEC(64, 32) IA_DEC(64, 64) IA_DEC(64, 128)
  IA_DEC(128, 32) IA_DEC(128, 64) IA_DEC(128, 128)
#undef IA_DEC
#define IA_DSK(BF, MM, PRO)                                                                \
  hipLaunchKernelGGL((decode_step_kernel<BF, MM, PRO>), dim3(a.B * a.H), dim3(kStepThreads), 0, \
                     st, a.q, a.k, a.v, a.lam, a.beta, a.U, a.G, a.E, a.o, a.H, a.F, a.D, a.M,  \
                     a.out_bf16, a.clamp, a.opt, a.readout, a.wgate, a.dgate, a.blk)
#define IA_DSK_M(BF, PRO) \
  if (a.M <= 64) IA_DSK(BF, 64, PRO); else IA_DSK(BF, kMaxModes, PRO);
  if (a.in_bf16) {
    if (a.block) { IA_DSK_M(true, true) } else { IA_DSK_M(true, false) }
  } else {
    if (a.block) { IA_DSK_M(false, true) } else { IA_DSK_M(false, false) }
  }
#undef IA_DSK_M
#undef IA_DSK
  prof_end(st, kKindDecode);
  return hipGetLastError();
}

template <int F, int D, bool LOCAL>
static void launch_scan_rows_t(const ScanArgs& a, dim3 grid, hipStream_t st) {
  if (a.in_bf16) {
    if (a.M <= 64)
      hipLaunchKernelGGL((scan_rows_kernel<F, D, 64, true, LOCAL>), grid, dim3(512), 0, st, a);
    else
      hipLaunchKernelGGL((scan_rows_kernel<F, D, kMaxModes, true, LOCAL>), grid, dim3(512), 0,
                         st, a);
  } else {
    if (a.M <= 64)
      hipLaunchKernelGGL((scan_rows_kernel<F, D, 64, false, LOCAL>), grid, dim3(512), 0, st, a);
    else
      hipLaunchKernelGGL((scan_rows_kernel<F, D, kMaxModes, false, LOCAL>), grid, dim3(512), 0,
                         st, a);
  }
}

// One segment: the walk.  Several: the state-only pass, the carry, the walk of every segment.
template <int F, int D>
static void launch_scan_rows(const ScanArgs& a, hipStream_t st) {
  const int BH = a.B * a.H;
  if (a.n_seg > 1) {
    launch_scan_rows_t<F, D, true>(a, dim3(BH, a.n_seg - 1), st);
    const long n = scan_slot_float2(F, D, a.M) * BH;
    hipLaunchKernelGGL(scan_carry_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                       a);
  }
  launch_scan_rows_t<F, D, false>(a, dim3(BH, a.n_seg > 1 ? a.n_seg : 1), st);
}

bool scan_rows_supported(int F, int D) {
  return (F == 32 || F == 64 || F == 128) && (D == 32 || D == 64 || D == 128);
}

hipError_t launch_scan_prefill(const ScanArgs& a, hipStream_t st) {
  (void)hipGetLastError();
  prof_begin(st);
  // the state in registers (scan_rows_kernel) for row widths up to 64 float4; the mode-looping
  // kernel with the state in memory otherwise
#define IA_SR(FF, DD)                         \
  if (a.F == FF && a.D == DD) {               \
    launch_scan_rows<FF, DD>(a, st);          \
    prof_end(st, kKindScan);                  \
    return hipGetLastError();                 \
  }
  IA_SR(32, 32) IA_SR(32, 64) IA_SR(32, 128)
  IA_SR(64, 32) IA_SR(64, 64) IA_SR(64, 128)
  IA_SR(128, 32) IA_SR(128, 64) IA_SR(128, 128)
#undef IA_SR
#define IA_SCAN(MM)                                                                          \
  hipLaunchKernelGGL((scan_prefill_kernel<MM>), dim3(a.B * a.H), dim3(kStepThreads), 0, st,    \
                     a.q, a.k, a.v, a.lam, a.beta, a.U, a.G, a.E, a.o, a.accumulate, a.N, a.H, \
                     a.F, a.D, a.M, a.in_bf16, a.out_bf16, a.clamp, a.reverse, a.sqk, a.sv,   \
                     a.opt, a.readout, a.wgate, a.dgate)
  if (a.M <= 64)
    IA_SCAN(64);
  else
    IA_SCAN(kMaxModes);
#undef IA_SCAN
  prof_end(st, kKindScan);
  return hipGetLastError();
}

}  // namespace ia
