// ia_tables.hpp — per-head tables of the chunked IA prefill, and the per-mode powers of lam
// that the state-only pass computes for itself.  Included by ia_chunk_state.hpp (whose
// launch also carries the table workgroups) and by ia_chunk.hip (the standalone launch).
//
// The tables take every power of a mode's lam from its log-polar form, lam^n =
// exp(n log|lam|) (cos n arg lam, sin n arg lam), which holds for any exponent; the state-only
// pass needs only lam^n for n <= C and takes them by binary exponentiation in fp64
// ("Interdomain Attention: Beyond Token-Level Key-Value Memory", summary page §A.2 for the
// chunk factorisation both serve).
#pragma once

#include "ia_chunk.hpp"

namespace ia {

// One mode's lam in log-polar form, with its beta.
struct LamPow {
  float lr, th;   // log |lam|, arg lam
  float2 bt;      // beta
  __device__ LamPow(float2 l, float2 b)
      : lr(0.5f * logf(l.x * l.x + l.y * l.y)), th(atan2f(l.y, l.x)), bt(b) {}
  __device__ float2 pw(float n) const {   // lam^n
    const float mag = expf(n * lr);
    float sn, cs;
    sincosf(n * th, &sn, &cs);
    return make_float2(mag * cs, mag * sn);
  }
  __device__ float2 cexpm1(float n) const {   // lam^-n - 1 = exp(-n log lam) - 1
    const float ar = -n * lr, ai = -n * th;
    const float e = expm1f(ar);
    float sn, cs, sh, ch;
    sincosf(ai, &sn, &cs);
    sincosf(0.5f * ai, &sh, &ch);
    return make_float2(e * cs - 2.f * sh * sh, (1.f + e) * sn);   // cos - 1 = -2 sin^2(x/2)
  }
  // beta sum_{j<n} lam^-j in closed form, (lam^-n - 1) / (lam^-1 - 1), numerator and
  // denominator as expm1 (no cancellation for lam near 1); lam = 1 gives n beta.
  __device__ float2 geo_sum(float n) const {
    const float2 den = cexpm1(1.f);
    const float dd = den.x * den.x + den.y * den.y;
    if (!(dd > 0.f)) return make_float2(n * bt.x, n * bt.y);
    const float2 num = cexpm1(n);
    const float2 r = make_float2((num.x * den.x + num.y * den.y) / dd,
                                 (num.y * den.x - num.x * den.y) / dd);
    return cmul(bt, r);
  }
};

// Small powers of one mode's lam by binary exponentiation in fp64 (fp64 VALU runs at the
// unpacked fp32 rate): lam^n for 1 <= n < C and, from the same squarings, lam^C, each within
// an ulp or so once rounded to fp32.  The state-only pass takes its chunk table from these.
struct LamSmallPow {
  double lr, li;   // lam
  __device__ explicit LamSmallPow(float2 l) : lr(l.x), li(l.y) {}
  // lam^n (0 <= n < 2^LOGC) into pn, lam^(2^LOGC) into pc.
  template <int LOGC>
  __device__ void pow_and_top(int n, float2& pn, float2& pc) const {
    double ar = 1.0, ai = 0.0, sr = lr, si = li;
#pragma unroll
    for (int k = 0; k < LOGC; ++k) {
      const double tr = ar * sr - ai * si, ti = ar * si + ai * sr;
      const bool take = (n >> k) & 1;
      ar = take ? tr : ar;
      ai = take ? ti : ai;
      const double qr = sr * sr - si * si, qi = 2.0 * sr * si;
      sr = qr;
      si = qi;
    }
    pn = make_float2((float)ar, (float)ai);
    pc = make_float2((float)sr, (float)si);
  }
  // beta sum_{n=1..C} lam^n = beta lam (1 - lam^C) / (1 - lam), lam^C given in fp64 parts; in
  // fp64 the differences lose nothing that matters in fp32.  lam = 1 gives C beta.
  __device__ float2 geo(float2 beta, int C, double cr, double ci) const {
    const double dr = 1.0 - lr, di = -li;
    const double dd = dr * dr + di * di;
    if (!(dd > 0.0)) return make_float2((float)C * beta.x, (float)C * beta.y);
    const double nr = 1.0 - cr, ni = -ci;
    const double qr = (nr * dr + ni * di) / dd, qi = (ni * dr - nr * di) / dd;   // n / d
    const double gr = lr * qr - li * qi, gi = lr * qi + li * qr;                  // lam n / d
    return make_float2((float)(beta.x * gr - beta.y * gi), (float)(beta.x * gi + beta.y * gr));
  }
  template <int LOGC>
  __device__ void top(double& cr, double& ci) const {   // lam^(2^LOGC) in fp64
    double sr = lr, si = li;
#pragma unroll
    for (int k = 0; k < LOGC; ++k) {
      const double qr = sr * sr - si * si, qi = 2.0 * sr * si;
      sr = qr;
      si = qi;
    }
    cr = sr;
    ci = si;
  }
};

// Table run `run` of head h, thread t < 4M: mode m = t % M, exponent j = 4 run + t / M.
// Written in the LDS form the prefill kernel copies verbatim: beta lam^-j in bf16 ([Re;Im]
// rows, j in K-slot order) and in scaled fp16 (row j, modes in K-slot order), both swizzled.
// Runs 0..3 also write the factors lam^(2i), i < 16, run 4 the factors lam^(32r) (with
// `half`, for the readout-matrix variant: lam^i and lam^(16r)); run 0 per
// mode lam^C, sum_{j<C} beta lam^-j, the same two for the last chunk's length Lt, lam^Ls for
// the segment length Ls, and 1/lam, the four threads of a mode splitting that work, and the
// head's route flag (chunk_unresolved for any of its modes).  The
// fp16 scale comes from max_m |beta| |lam|^-(C-1), reduced over the mode lanes of each wave:
// every wave of every run of the head reduces the same values, so all agree on it.
template <int C, int M>
__device__ __forceinline__ void table_run(const float2* __restrict__ lam,
                                          const float2* __restrict__ beta,
                                          unsigned char* tables, long table_bytes, int Lt,
                                          int Ls, int h, int run, int t, int half) {
  using TL = TableLayout<C, M>;
  constexpr int M2 = 2 * M;
  constexpr int JB = 4;            // exponents per run
  constexpr int RUNS = C / 16;     // rows of lam^(32r)
  constexpr int L2S = M + 2;
  static_assert(C / JB > 16 / JB, "a run for the lam^(32r) rows");
  static_assert((4 * M) % 64 == 0, "a run is whole waves");
  unsigned char* tab = tables + (size_t)h * table_bytes;
  uint16_t* WT = reinterpret_cast<uint16_t*>(tab + TL::oW);
  uint16_t* Wb = WT + M2 * C;
  float2* L2lo = reinterpret_cast<float2*>(tab + TL::oL2);
  float2* L2hi = L2lo + 16 * L2S;
  const int m = t % M, jj = t / M;
  const int j = JB * run + jj;
  const LamPow lp(lam[(size_t)h * M + m], beta[(size_t)h * M + m]);

  float mx = hypotf(lp.bt.x, lp.bt.y) * expf(-(float)(C - 1) * lp.lr);
  const float2 lm = lam[(size_t)h * M + m];
  int route = chunk_unresolved(lm.x, lm.y, C);
#pragma unroll
  for (int o = 1; o < (M < 64 ? M : 64); o <<= 1) {
    mx = fmaxf(mx, __shfl_xor(mx, o, 64));
    route |= __shfl_xor(route, o, 64);
  }
  const float wscale = pow2_scale(mx);

  const float2 w = cmul(lp.bt, lp.pw(-(float)j));   // beta lam^-j
  WT[soff<C>(m, kpos(j))] = __builtin_bit_cast(uint16_t, (__bf16)w.x);
  WT[soff<C>(M + m, kpos(j))] = __builtin_bit_cast(uint16_t, (__bf16)w.y);
  Wb[soff<M2>(j, kpos(m))] = __builtin_bit_cast(uint16_t, (_Float16)(w.x * wscale));
  Wb[soff<M2>(j, kpos(M + m))] = __builtin_bit_cast(uint16_t, (_Float16)(w.y * wscale));
  const float fe = half ? 1.f : 2.f;   // factor exponent: lam^(2i), or lam^i with `half`
  if (run < 16 / JB) L2lo[j * L2S + m] = lp.pw(fe * j);                    // i = j
  if (run == 16 / JB && jj < RUNS) L2hi[jj * M + m] = lp.pw(16.f * fe * jj);   // i = 16r
  if (run != 0) return;

  float2* const out = reinterpret_cast<float2*>(tab);
  if (jj == 0) {
    out[TL::oGeo / 8 + m] = lp.geo_sum((float)C);
  } else if (jj == 1) {
    out[TL::oGeoT / 8 + m] = lp.geo_sum((float)Lt);
  } else if (jj == 2) {
    out[TL::oPow / 8 + m] = lp.pw((float)C);
    out[TL::oPowT / 8 + m] = lp.pw((float)Lt);
  } else {
    out[TL::oPowS / 8 + m] = lp.pw((float)Ls);
    out[TL::oInv / 8 + m] = lp.pw(-1.f);
    if (m == 0) {
      *reinterpret_cast<float*>(tab + TL::oSc) = 1.f / wscale;
      *reinterpret_cast<int*>(tab + TL::oRoute) = route;
    }
  }
}

// The readout-matrix operand of head h (ReadoutTable), by threads tid < nt (nt a multiple of
// 64, at most 1024) of one workgroup: the power-of-two scale from the largest |Re| or |Im|
// of R's entries (NaN entries do not count: they reach the output through the products), then
// the four fp16 entries each R[m][n] gives.
template <int M>
__device__ __forceinline__ void readout_table_run(const float2* __restrict__ R,
                                                  unsigned char* rtab, long rtab_bytes, int h,
                                                  int tid, int nt) {
  constexpr int M2 = 2 * M;
  __shared__ float red[16];
  const float2* Rh = R + (size_t)h * M * M;
  float mx = 0.f;
  for (int i = tid; i < M * M; i += nt) {
    const float2 r = Rh[i];
    mx = fmaxf(mx, fmaxf(fabsf(r.x), fabsf(r.y)));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
  if ((tid & 63) == 0) red[tid >> 6] = mx;
  __syncthreads();
  mx = 0.f;
  for (int w = 0; w < nt / 64; ++w) mx = fmaxf(mx, red[w]);
  const float sc = pow2_scale(mx);
  uint16_t* T = reinterpret_cast<uint16_t*>(rtab + (size_t)h * rtab_bytes);
  for (int i = tid; i < M * M; i += nt) {
    const int m = i / M, n = i % M;
    const float2 r = Rh[i];
    const uint16_t re = __builtin_bit_cast(uint16_t, (_Float16)(r.x * sc));
    const uint16_t im = __builtin_bit_cast(uint16_t, (_Float16)(r.y * sc));
    T[soff<M2>(n, kpos(m))] = re;
    T[soff<M2>(n, kpos(M + m))] = im;
    T[soff<M2>(M + n, kpos(m))] = im;
    T[soff<M2>(M + n, kpos(M + m))] = re ^ 0x8000u;   // -Re
  }
  if (tid == 0)
    *reinterpret_cast<float*>(rtab + (size_t)h * rtab_bytes + ReadoutTable<M>::oScale) = 1.f / sc;
}

}  // namespace ia
