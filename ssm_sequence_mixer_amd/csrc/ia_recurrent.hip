// ia_recurrent.hip — token-by-token IA kernels (fp32 VALU): the decode step, the
// token-sequential fp32 prefill, and the state fill.
//
// The step is the recurrence and readout of the layer ("Interdomain Attention: Beyond
// Token-Level Key-Value Memory": summary page §3.2 for the complex-diagonal S4D recurrence and
// the O(M(R+d)) per-step decode; episode page, "Key Components and Derivation", for the
// feature map and the matrix form Fq U^T Gamma / Fq U^T eta):
//     U[m,:] <- lam_m U[m,:] + beta_m phi(k_t),   a[m] = phi(q_t) . U[m,:]
//     G[m,:] <- lam_m G[m,:] + beta_m v_t,        eta[m] <- lam_m eta[m] + beta_m
//     o_t = Re(sum_m a[m] G[m,:]) / max(Re(sum_m a[m] eta[m]), clamp)
// One workgroup owns one (b,h) slice.  The state stays in global memory (HBM or L2) and is
// streamed once per token: each wave takes every 4th mode and its lanes cover a state row
// with 16-byte accesses, so a row of F complex values is one coalesced access.
#include "ia_device.hpp"
#include "ia_kernels.hpp"

namespace ia {

constexpr int kStepThreads = 256;
constexpr int kStepWaves = kStepThreads / 64;

__device__ __forceinline__ float2 cadd2(float2 a, float2 b) {
  return make_float2(a.x + b.x, a.y + b.y);
}

struct StepSmem {
  float fq[kMaxDim];
  float fk[kMaxDim];
  float v[kMaxDim];
  float2 lam[kMaxModes];
  float2 beta[kMaxModes];
  float2 a[kMaxModes];
  float2 ar[kMaxModes];   // a R, with a readout matrix R
  float2 rp[kStepThreads];   // partial sums of a R
  float2 eta[kMaxModes];
  float num[kStepWaves][kMaxDim];
  float den[kStepWaves];
};

// State rows are float2 arrays; lanes take two complex values (one float4) at a time.
// F and D are multiples of 16, so a row is a whole number of float4 pairs.
// R: this head's readout matrix [M][M] (row m, column n), or NULL for none: the readouts then
// use (a R)[n] = sum_m a[m] R[m][n] in place of a.
__device__ __forceinline__ void step_one(StepSmem& s, float2* __restrict__ U,
                                         float2* __restrict__ G, float2* __restrict__ E,
                                         int F, int D, int M, const float2* __restrict__ R) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;

  // U rows: update in place and contract with phi(q_t).
  for (int m = wave; m < M; m += kStepWaves) {
    const float2 l = s.lam[m], b = s.beta[m];
    float4* row = reinterpret_cast<float4*>(U + (size_t)m * F);
    float ar = 0.f, ai = 0.f;
    for (int p = lane; p < F / 2; p += 64) {
      float4 u = row[p];
      const float k0 = s.fk[2 * p], k1 = s.fk[2 * p + 1];
      float2 u0 = cfma(l, make_float2(u.x, u.y), make_float2(b.x * k0, b.y * k0));
      float2 u1 = cfma(l, make_float2(u.z, u.w), make_float2(b.x * k1, b.y * k1));
      row[p] = make_float4(u0.x, u0.y, u1.x, u1.y);
      const float q0 = s.fq[2 * p], q1 = s.fq[2 * p + 1];
      ar += q0 * u0.x + q1 * u1.x;
      ai += q0 * u0.y + q1 * u1.y;
    }
    ar = wave_sum(ar);
    ai = wave_sum(ai);
    if (lane == 0) s.a[m] = make_float2(ar, ai);
  }
  // eta: one mode per thread.
  for (int m = threadIdx.x; m < M; m += kStepThreads) {
    float2 e = cfma(s.lam[m], E[m], s.beta[m]);
    E[m] = e;
    s.eta[m] = e;
  }
  __syncthreads();
  if (R) {
    // thread t sums the modes m = t / M, t / M + parts, ... of column n = t % M
    const int parts = kStepThreads / M, n = threadIdx.x % M, part = threadIdx.x / M;
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
  const float2* A = R ? s.ar : s.a;

  // Gamma rows: update in place, accumulate Re(a[m] G[m,:]) per lane.
  float acc[kMaxDim / 64];
#pragma unroll
  for (int i = 0; i < kMaxDim / 64; ++i) acc[i] = 0.f;
  for (int m = wave; m < M; m += kStepWaves) {
    const float2 l = s.lam[m], b = s.beta[m], a = A[m];
    float4* row = reinterpret_cast<float4*>(G + (size_t)m * D);
#pragma unroll
    for (int i = 0; i < kMaxDim / 128; ++i) {
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
  for (int i = 0; i < kMaxDim / 128; ++i) {
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
    if (lane == 0) s.den[0] = d;
  }
  __syncthreads();
}

// Load phi(q), phi(k), v of one token into shared memory.
__device__ __forceinline__ void load_token(StepSmem& s, const void* q, const void* k,
                                           const void* v, size_t qk_off, size_t v_off, int F,
                                           int D, int bf16, int opt) {
  for (int i = threadIdx.x; i < F; i += kStepThreads) {
    s.fq[i] = feat(load_in(q, qk_off + i, bf16), opt);
    s.fk[i] = feat(load_in(k, qk_off + i, bf16), opt);
  }
  for (int i = threadIdx.x; i < D; i += kStepThreads) s.v[i] = load_in(v, v_off + i, bf16);
}

__device__ __forceinline__ void load_modes(StepSmem& s, const float2* lam, const float2* beta,
                                           int h, int M) {
  for (int m = threadIdx.x; m < M; m += kStepThreads) {
    s.lam[m] = lam[(size_t)h * M + m];
    s.beta[m] = beta[(size_t)h * M + m];
  }
}

// ---------------------------------------------------------------- kernels

// Decode: one step for every (b,h).  grid = B*H.
__global__ void __launch_bounds__(kStepThreads)
decode_step_kernel(const void* __restrict__ q, const void* __restrict__ k,
                   const void* __restrict__ v, const float2* __restrict__ lam,
                   const float2* __restrict__ beta, float2* __restrict__ U,
                   float2* __restrict__ G, float2* __restrict__ E, void* __restrict__ o,
                   int H, int F, int D, int M, int in_bf16, int out_bf16, float clamp,
                   int opt, const float2* __restrict__ rmat) {
  __shared__ StepSmem s;
  const int bh = blockIdx.x;
  const int h = bh % H;
  load_modes(s, lam, beta, h, M);
  load_token(s, q, k, v, (size_t)bh * F, (size_t)bh * D, F, D, in_bf16, opt);
  __syncthreads();
  step_one(s, U + (size_t)bh * M * F, G + (size_t)bh * M * D, E + (size_t)bh * M, F, D, M,
           rmat ? rmat + (size_t)h * M * M : nullptr);
  for (int j = threadIdx.x; j < D; j += kStepThreads) {
    float n = 0.f;
#pragma unroll
    for (int w = 0; w < kStepWaves; ++w) n += s.num[w][j];
    store_out(o, (size_t)bh * D + j, readout(n, s.den[0], clamp, opt), out_bf16);
  }
}

// Decode with the whole state of a slice in flight at once.  grid = B*H; NT threads per slice.
// A state row of F complex values is F/2 float4 (2 complex each); thread t owns float4 column
// pu = t % (F/2) of the U rows m = t / (F/2) + (NT/(F/2)) i, and likewise column pd of the
// Gamma rows, so its inputs are two entries each of phi(q), phi(k) and v.  Every row load is
// issued before any arithmetic; a[m] needs all of row m (a reduction over the F/2 lanes that
// share it), then the Gamma rows, whose column sums over rows go through LDS in a fixed order.
template <int F, int D, int MM>
__global__ void __launch_bounds__(512)
decode_step_rows_kernel(const void* __restrict__ q, const void* __restrict__ k,
                        const void* __restrict__ v, const float2* __restrict__ lam,
                        const float2* __restrict__ beta, float2* __restrict__ U,
                        float2* __restrict__ G, float2* __restrict__ E, void* __restrict__ o,
                        int H, int M, int in_bf16, int out_bf16, float clamp, int opt,
                        const float2* __restrict__ rmat) {
  constexpr int NT = 512, NWV = NT / 64;
  constexpr int RU = F / 2, RD = D / 2;
  static_assert(RU <= 64 && RD <= 64 && NT % RU == 0 && NT % RD == 0, "row width");
  constexpr int SU = NT / RU, SD = NT / RD;                  // rows per pass
  constexpr int IU = (MM + SU - 1) / SU, ID = (MM + SD - 1) / SD;   // M <= MM
  __shared__ float2 s_lam[kMaxModes], s_beta[kMaxModes], s_a[kMaxModes], s_ar[kMaxModes];
  __shared__ float2 s_rp[NT];   // partial sums of a R
  __shared__ float s_num[SD][D];
  __shared__ float s_den[NWV];

  const int bh = blockIdx.x, h = bh % H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int pu = tid % RU, ru = tid / RU, pd = tid % RD, rd = tid / RD;
  float4* Ub = reinterpret_cast<float4*>(U + (size_t)bh * M * F);
  float4* Gb = reinterpret_cast<float4*>(G + (size_t)bh * M * D);
  float2* Eb = E + (size_t)bh * M;

  float4 u[IU], g[ID];
#pragma unroll
  for (int i = 0; i < IU; ++i) {
    const int m = ru + SU * i;
    if (m < M) u[i] = Ub[(size_t)m * RU + pu];
  }
#pragma unroll
  for (int i = 0; i < ID; ++i) {
    const int m = rd + SD * i;
    if (m < M) g[i] = Gb[(size_t)m * RD + pd];
  }
  float2 e = make_float2(0.f, 0.f);
  if (tid < M) {
    s_lam[tid] = lam[(size_t)h * M + tid];
    s_beta[tid] = beta[(size_t)h * M + tid];
    e = Eb[tid];
  }
  const float fk0 = feat(load_in(k, (size_t)bh * F + 2 * pu, in_bf16), opt);
  const float fk1 = feat(load_in(k, (size_t)bh * F + 2 * pu + 1, in_bf16), opt);
  const float fq0 = feat(load_in(q, (size_t)bh * F + 2 * pu, in_bf16), opt);
  const float fq1 = feat(load_in(q, (size_t)bh * F + 2 * pu + 1, in_bf16), opt);
  const float v0 = load_in(v, (size_t)bh * D + 2 * pd, in_bf16);
  const float v1 = load_in(v, (size_t)bh * D + 2 * pd + 1, in_bf16);
  __syncthreads();   // lam, beta

  if (tid < M) {
    e = cfma(s_lam[tid], e, s_beta[tid]);
    Eb[tid] = e;
  }
  // U rows: update, store, contract with phi(q) over the row's lanes.
#pragma unroll
  for (int i = 0; i < IU; ++i) {
    const int m = ru + SU * i;
    if (m < M) {   // uniform over the row's F/2 lanes, which the shuffles below combine
      const float2 l = s_lam[m], bt = s_beta[m];
      const float2 u0 = cfma(l, make_float2(u[i].x, u[i].y), make_float2(bt.x * fk0, bt.y * fk0));
      const float2 u1 = cfma(l, make_float2(u[i].z, u[i].w), make_float2(bt.x * fk1, bt.y * fk1));
      Ub[(size_t)m * RU + pu] = make_float4(u0.x, u0.y, u1.x, u1.y);
      float ar = fq0 * u0.x + fq1 * u1.x, ai = fq0 * u0.y + fq1 * u1.y;
#pragma unroll
      for (int off = RU / 2; off > 0; off >>= 1) {
        ar += __shfl_xor(ar, off, 64);
        ai += __shfl_xor(ai, off, 64);
      }
      if (pu == 0) s_a[m] = make_float2(ar, ai);
    }
  }
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
    store_out(o, (size_t)bh * D + tid, readout(n, den, clamp, opt), out_bf16);
  }
}

// Token-sequential prefill (the fp32 path).  grid = B*H; one workgroup walks all N tokens of
// its slice, in reverse when `reverse` is set (then token t of the walk is position N-1-t).
// q, k and v are addressed through their element strides sqk, sv; o is dense.
// o (out dtype) receives value, or o + value with `accumulate` (the second direction of the
// bidirectional layer adds onto the first); o may be NULL (state only).
__global__ void __launch_bounds__(kStepThreads)
scan_prefill_kernel(const void* __restrict__ q, const void* __restrict__ k,
                    const void* __restrict__ v, const float2* __restrict__ lam,
                    const float2* __restrict__ beta, float2* __restrict__ U,
                    float2* __restrict__ G, float2* __restrict__ E, void* __restrict__ o,
                    int accumulate, int N, int H, int F, int D, int M,
                    int in_bf16, int out_bf16, float clamp, int reverse, RowStrides sqk,
                    RowStrides sv, int opt, const float2* __restrict__ rmat) {
  __shared__ StepSmem s;
  const int bh = blockIdx.x;
  const int b = bh / H, h = bh % H;
  load_modes(s, lam, beta, h, M);
  float2* Ub = U + (size_t)bh * M * F;
  float2* Gb = G + (size_t)bh * M * D;
  float2* Eb = E + (size_t)bh * M;
  for (int t = 0; t < N; ++t) {
    const int pos = reverse ? N - 1 - t : t;
    const size_t tok = ((size_t)b * N + pos) * H + h;
    load_token(s, q, k, v, (size_t)(b * sqk.b + pos * sqk.n + h * sqk.h),
               (size_t)(b * sv.b + pos * sv.n + h * sv.h), F, D, in_bf16, opt);
    __syncthreads();
    step_one(s, Ub, Gb, Eb, F, D, M, rmat ? rmat + (size_t)h * M * M : nullptr);
    if (o) {
      for (int j = threadIdx.x; j < D; j += kStepThreads) {
        float n = 0.f;
#pragma unroll
        for (int w = 0; w < kStepWaves; ++w) n += s.num[w][j];
        float val = readout(n, s.den[0], clamp, opt);
        if (accumulate) val += load_in(o, tok * D + j, out_bf16);
        store_out(o, tok * D + j, val, out_bf16);
      }
    }
    __syncthreads();
  }
}

__global__ void fill_zero_kernel(float4* __restrict__ p, size_t n4) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n4;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

// ---------------------------------------------------------------- launchers

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

template <int F, int D>
static void launch_decode_rows(const DecodeArgs& a, hipStream_t st) {
  // The per-thread row registers are sized for M <= 64 or M <= 128: the smaller set lets two
  // workgroups share a CU.
  if (a.M <= 64)
    hipLaunchKernelGGL((decode_step_rows_kernel<F, D, 64>), dim3(a.B * a.H), dim3(512), 0, st,
                       a.q, a.k, a.v, a.lam, a.beta, a.U, a.G, a.E, a.o, a.H, a.M, a.in_bf16,
                       a.out_bf16, a.clamp, a.opt, a.readout);
  else
    hipLaunchKernelGGL((decode_step_rows_kernel<F, D, kMaxModes>), dim3(a.B * a.H), dim3(512),
                       0, st, a.q, a.k, a.v, a.lam, a.beta, a.U, a.G, a.E, a.o, a.H, a.M,
                       a.in_bf16, a.out_bf16, a.clamp, a.opt, a.readout);
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
  // fewer than four slices per CU; with more, the small mode-looping kernel keeps every slice
  // resident at once and streams better (measured on MI355X at H=16, F=Dv=128, M=64: rows
  // 11.1 us vs 20.9 us at B=16, 46.0 us vs 42.8 us at B=64).
  const bool rows = (long)a.B * a.H < 4L * device_cus();
#define IA_DEC(FF, DD) \
  if (rows && a.F == FF && a.D == DD) { launch_decode_rows<FF, DD>(a, st); } else
  IA_DEC(32, 32) IA_DEC(32, 64) IA_DEC(32, 128)
  IA_DEC(64, 32) IA_DEC(64, 64) IA_DEC(64, 128)
  IA_DEC(128, 32) IA_DEC(128, 64) IA_DEC(128, 128)
#undef IA_DEC
  hipLaunchKernelGGL(decode_step_kernel, dim3(a.B * a.H), dim3(kStepThreads), 0, st, a.q, a.k,
                     a.v, a.lam, a.beta, a.U, a.G, a.E, a.o, a.H, a.F, a.D, a.M, a.in_bf16,
                     a.out_bf16, a.clamp, a.opt, a.readout);
  prof_end(st, kKindDecode);
  return hipGetLastError();
}

hipError_t launch_scan_prefill(const ScanArgs& a, hipStream_t st) {
  (void)hipGetLastError();
  prof_begin(st);
  hipLaunchKernelGGL(scan_prefill_kernel, dim3(a.B * a.H), dim3(kStepThreads), 0, st, a.q,
                     a.k, a.v, a.lam, a.beta, a.U, a.G, a.E, a.o, a.accumulate, a.N, a.H, a.F, a.D,
                     a.M, a.in_bf16, a.out_bf16, a.clamp, a.reverse, a.sqk, a.sv, a.opt,
                     a.readout);
  prof_end(st, kKindScan);
  return hipGetLastError();
}

}  // namespace ia
