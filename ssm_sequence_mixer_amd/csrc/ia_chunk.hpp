// ia_chunk.hpp — chunked IA prefill on gfx950 MFMA (bf16 inputs): the kernel.  Included by
// the per-feature-width translation units that instantiate it.
//
// The layer ("Interdomain Attention: Beyond Token-Level Key-Value Memory": summary page §3.2
// and §A.2 for the complex-diagonal S4D recurrence run chunkwise — dense work inside a
// chunk, the state passed across chunk boundaries, and a second pass that recomputes each
// chunk from its corrected initial state; episode page, "Key Components and Derivation", for
// the readout O = Fq U^T Gamma / Fq U^T eta) is evaluated per chunk of C tokens.  With the
// chunk's starting state (U_c, G_c, eta_c), local positions i, j in [0, C) and
// S[i,j] = phi(q_i).phi(k_j) masked to j <= i, unrolling the recurrence gives
//   A[i,m]   = lam^i A'[i,m],  A' = S (beta lam^-j) + Fq (lam U_c)^T      (query-mode matrix)
//   P[i,j]   = Re sum_m A[i,m] beta_m lam_m^(i-j)   = Re (lam^i A)(beta lam^-j)^T, j <= i
//   num[i,:] = P V + Re (lam^i A)(lam G_c)          den[i] = sum_j P[i,j] + Re (lam^i A)(lam eta_c)
//   o[i,:]   = num[i,:] / max(den[i], clamp)
//   U_{c+1}  = lam^(L-1) (lam U_c + sum_j beta lam^-j phi(k_j)), same for G with v, eta with 1.
// Complex matrices enter real MFMAs as [Re | Im] blocks of 2M real columns.
//
// Workgroup = one (b, h, segment, direction); 64*(C/16 + 4) threads:
//   readout waves r < C/16 own the 16 queries [16r, 16r+16) of each chunk and chain
//     S^T -> A'^T -> P^T -> num^T through MFMA accumulators (an accumulator tile of X is the
//     operand of X^T, with the K index permuted identically on both operands).  They also
//     fetch the next chunk's q, k, v into registers while the current chunk computes;
//   state waves own columns of the fp32 state, kept in MFMA accumulators for the whole
//     segment, update it with two MFMA contractions per chunk, and publish operand copies of
//     the new state (bf16 lam U, fp16 lam G scaled per column) to LDS.
// Operand precision: features, S, the decay table, U, P and v in bf16; A, beta lam^-j and G
// in fp16 after exact power-of-two scaling (per query row for A; per value column for G; per
// head for the table), which keeps the readout's cancelling sums within the bf16 tolerance.
// Every LDS matrix row is padded by 16 bytes so that the 16 rows an MFMA operand read
// touches fall in distinct banks.
#pragma once

#include <utility>

#include "ia_device.hpp"
#include "ia_kernels.hpp"

namespace ia {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

union Frag {
  uint4 u;
  bf16x8 b;
  f16x8 h;
};

__device__ __forceinline__ f32x4 mma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma_f16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// 8 consecutive 16-bit values.
__device__ __forceinline__ Frag lds8(const uint16_t* p) {
  Frag f;
  f.u = *reinterpret_cast<const uint4*>(p);
  return f;
}
// 4 + 4 values from two places (the permuted K order of an accumulator-sourced partner).
__device__ __forceinline__ Frag lds44(const uint16_t* p0, const uint16_t* p1) {
  Frag f;
  const uint2 a = *reinterpret_cast<const uint2*>(p0);
  const uint2 b = *reinterpret_cast<const uint2*>(p1);
  f.u = make_uint4(a.x, a.y, b.x, b.y);
  return f;
}

__device__ __forceinline__ bf16x8 pack_bf16(f32x4 a, f32x4 b) {
  bf16x8 r;
  r[0] = (__bf16)a[0]; r[1] = (__bf16)a[1]; r[2] = (__bf16)a[2]; r[3] = (__bf16)a[3];
  r[4] = (__bf16)b[0]; r[5] = (__bf16)b[1]; r[6] = (__bf16)b[2]; r[7] = (__bf16)b[3];
  return r;
}

__device__ __forceinline__ uint2 pack4_bf16(float a, float b, float c, float d) {
  return make_uint2(uint32_t(f32_to_bf16(a)) | (uint32_t(f32_to_bf16(b)) << 16),
                    uint32_t(f32_to_bf16(c)) | (uint32_t(f32_to_bf16(d)) << 16));
}

__device__ __forceinline__ uint16_t f16_bits(float x) {
  _Float16 h = (_Float16)x;
  return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ uint2 pack4_f16(float a, float b, float c, float d) {
  return make_uint2(uint32_t(f16_bits(a)) | (uint32_t(f16_bits(b)) << 16),
                    uint32_t(f16_bits(c)) | (uint32_t(f16_bits(d)) << 16));
}

// Power of two s with s * mx in [2^14, 2^15): maps the largest magnitude of a row or column
// near the top of the fp16 range.  mx == 0 or not finite: 1.
__device__ __forceinline__ float pow2_scale(float mx) {
  if (!(mx > 0.f) || !(mx < 3.0e38f)) return 1.f;
  const int e = ilogbf(mx);               // mx in [2^e, 2^(e+1))
  return ldexpf(1.f, 14 - e);
}

__device__ __forceinline__ float xor_sum16_32(float v) {
  v += __shfl_xor(v, 16, 64);
  v += __shfl_xor(v, 32, 64);
  return v;
}
__device__ __forceinline__ float xor_max16_32(float v) {
  v = fmaxf(v, __shfl_xor(v, 16, 64));
  v = fmaxf(v, __shfl_xor(v, 32, 64));
  return v;
}

// Complex power lam^n = exp(n log|lam|) (cos n arg, sin n arg), lam != 0.
__device__ __forceinline__ float2 cpow_f(float2 lam, float n) {
  const float lr = 0.5f * logf(lam.x * lam.x + lam.y * lam.y);
  const float th = atan2f(lam.y, lam.x);
  const float mag = expf(n * lr);
  float sn, cs;
  sincosf(n * th, &sn, &cs);
  return make_float2(mag * cs, mag * sn);
}

// ---------------------------------------------------------------- LDS layout

template <int C, int F, int D, int M>
struct Layout {
  static constexpr int M2 = 2 * M;
  // padded row lengths, in 16-bit elements
  static constexpr int RF = F + 8, RC = C + 8, RM = M2 + 8;
  // 16-bit element offsets (all multiples of 8 -> 16-byte aligned)
  static constexpr int oFk = 0;                    // [C][RF]   bf16 phi(k), row j
  static constexpr int oFkT = oFk + C * RF;        // [F][RC]   bf16 phi(k)^T
  static constexpr int oVT = oFkT + F * RC;        // [D][RC]   bf16 v^T
  static constexpr int oWT = oVT + D * RC;         // [2M][RC]  bf16 beta lam^-j, [Re;Im] rows
  static constexpr int oWb = oWT + M2 * RC;        // [C][RM]   fp16 scaled beta lam^-j, row j
  static constexpr int oLU = oWb + C * RM;         // [2M][RF]  bf16 lam U_c, [Re;Im] rows
  static constexpr int oGT = oLU + M2 * RF;        // [D][RM]   fp16 c_d lam G_c, row d
  static constexpr int n16 = oGT + D * RM;
  // fp32 arrays after the 16-bit block (byte offsets)
  static constexpr int bC = n16 * 2;               // [D]  float  c_d
  static constexpr int bLE = bC + D * 4;           // [M]  float2 lam eta_c
  static constexpr int bLam = bLE + M * 8;         // [M]  float2 lam
  static constexpr int bPowL = bLam + M * 8;       // [M]  float2 lam^(L-1) of the current chunk
  static constexpr int bGeo = bPowL + M * 8;       // [M]  float2 sum_{j<L} beta lam^-j
  static constexpr int bytes = bGeo + M * 8;
};

struct ChunkArgs {
  const uint16_t *q, *k, *v;   // bf16 [B][N][H][F|D]
  const float2 *lam, *beta;    // [H][M]
  void* o;                     // [B][N][H][D] or NULL (state only)
  const float* acc_in;         // fp32 [B][N][H][D] added to the output, or NULL
  int N, H;
  int seg_chunks;              // chunks per segment
  int seg_first;               // first segment index handled by this launch
  int n_seg;                   // segments in this launch, per sequence
  int dir;                     // 1: the walk runs from position N-1 down to 0
  int out_bf16;
  float clamp;
  // Initial state: workspace slot `seg` of the sequence when `initc` is set, else (one
  // segment) the caller's state `init0` or zeros.  Final state: with `fin_seg` set, segment
  // g writes slot g+1; otherwise the segment holding the last token writes the caller's
  // `fin` (if set).  Slot components: U at 0, G at M*F, eta at M*(F+D) (complex elements).
  const float2 *init0_U, *init0_G, *init0_E;   // caller layout: [seq][M][F] etc.
  const float2* initc;
  float2 *fin_U, *fin_G, *fin_E;               // caller layout
  float2* fin_seg;
  long slot;                                   // complex elements per slot
  int slots_per_seq;
  const unsigned char* tables;                 // per-head tables (chunk_tables_kernel)
  long table_bytes;                            // bytes per head
};

// Per-head tables, computed once per call by chunk_tables_kernel (byte offsets).  The two
// decay tables are stored with the padded LDS row lengths, adjacent, as in LDS.
template <int C, int M>
struct TableLayout {
  static constexpr int RC = C + 8, RM = 2 * M + 8;
  static constexpr long oW = 0;                       // bf16 [2M][RC] then fp16 [C][RM]
  static constexpr long nW = 2L * (2L * M * RC + (long)C * RM);
  static constexpr long oL2 = oW + nW;                // float2 [C][M]: lam^(2i)
  static constexpr long oPow = oL2 + 8L * C * M;      // float2 [M]: lam^(C-1)
  static constexpr long oGeo = oPow + 8L * M;         // float2 [M]: sum_{j<C} beta lam^-j
  static constexpr long oPowT = oGeo + 8L * M;        // float2 [M]: lam^(Lt-1), last chunk
  static constexpr long oGeoT = oPowT + 8L * M;       // float2 [M]: sum_{j<Lt} beta lam^-j
  static constexpr long oPowS = oGeoT + 8L * M;       // float2 [M]: lam^(segment length)
  static constexpr long oSc = oPowS + 8L * M;         // float: 1 / fp16 table scale
  static constexpr long bytes = (oSc + 16 + 255) / 256 * 256;
};

// Per-workgroup context shared by the two wave roles.
template <int C, int F, int D, int M>
struct Ctx {
  uint16_t *sFk, *sFkT, *sVT, *sWT, *sWb, *sLU, *sGT;
  float* sC;
  float2 *sLE, *sLam, *sPowL, *sGeo;
  const unsigned char* tab;
  int lane, il, g, wave;
  int seq, seg, b, h, c_begin, c_end;
  bool last_seg, want_out;
  float wb_unscale;
  __device__ int pos_of(const ChunkArgs& a, int t) const { return a.dir ? a.N - 1 - t : t; }
  __device__ size_t tok_index(const ChunkArgs& a, int pos) const {
    return ((size_t)b * a.N + pos) * a.H + h;
  }
};

// ---------------------------------------------------------------- readout waves
// Wave r owns queries [16r, 16r+16) of every chunk.  It also loads tokens [16r, 16r+16) of
// k and v for everyone (phi(k) rows, phi(k)^T and v^T in LDS), one chunk ahead.
template <int C, int F, int D, int M, int R>
__device__ __forceinline__ void readout_main(const ChunkArgs& a, const Ctx<C, F, D, M>& x) {
  using Lay = Layout<C, F, D, M>;
  using TL = TableLayout<C, M>;
  constexpr int NR = C / 16;
  constexpr int MH = M / 16;
  constexpr int TM = 2 * M / 16;
  constexpr int KF = F / 32;
  constexpr int KM = 2 * M / 32;
  constexpr int KC = C / 32;
  constexpr int TD = D / 16;
  constexpr int RF = Lay::RF, RC = Lay::RC, RM = Lay::RM;
  constexpr int NK = 4 * (F / 8);   // load items of k: 4 token quads x F/8 column octets
  constexpr int NV = 4 * (D / 8);
  static_assert(NK <= 64 && NV <= 64, "one load item per lane");
  constexpr int r = R;   // compile-time: causal trip counts below are constants
  const int lane = x.lane, il = x.il, g = x.g;

  float2 lam2i[MH][4];   // lam_m^(2i), i = 16r + il, modes 16mt + 4g + q
  {
    const float2* l2 = reinterpret_cast<const float2*>(x.tab + TL::oL2) + (16 * r + il) * M;
#pragma unroll
    for (int mt = 0; mt < MH; ++mt)
#pragma unroll
      for (int q = 0; q < 4; ++q) lam2i[mt][q] = l2[16 * mt + 4 * g + q];
  }

  // Raw bf16 inputs of the next chunk (issued before the current chunk's compute).
  uint4 rk[4], rv[4], rq[KF];
  const int iq4 = lane & 3, io = lane >> 2;   // this lane's load item: token quad, octet
  auto prefetch = [&](int c) {
    const int t0 = c * C + 16 * r + 4 * iq4;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const int t = t0 + tt;
      const bool ok = t < a.N;
      const size_t ti = ok ? x.tok_index(a, x.pos_of(a, t)) : 0;
      rk[tt] = make_uint4(0, 0, 0, 0);
      rv[tt] = make_uint4(0, 0, 0, 0);
      if (ok && lane < NK) rk[tt] = *reinterpret_cast<const uint4*>(a.k + ti * F + 8 * io);
      if (ok && lane < NV) rv[tt] = *reinterpret_cast<const uint4*>(a.v + ti * D + 8 * io);
    }
    if (x.want_out) {
      const int t = c * C + 16 * r + il;
      const bool ok = t < a.N;
      const size_t qoff = ok ? x.tok_index(a, x.pos_of(a, t)) * F : 0;
#pragma unroll
      for (int s = 0; s < KF; ++s)
        rq[s] = ok ? *reinterpret_cast<const uint4*>(a.q + qoff + 32 * s + 8 * g)
                   : make_uint4(0, 0, 0, 0);
    }
  };
  bf16x8 fq[KF];
  // phi(k) rows and columns, v columns, and this wave's phi(q) operands from the raw data.
  // Tokens past N have zero features and values (zeros, not phi(0)).
  auto write_lds = [&](int c) {
    const int j0 = 16 * r + 4 * iq4;
    const int L = min(C, a.N - c * C);
    if (lane < NK) {
      float f[4][8];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const uint16_t* e16 = reinterpret_cast<const uint16_t*>(&rk[tt]);
        const bool ok = j0 + tt < L;
#pragma unroll
        for (int e = 0; e < 8; ++e) f[tt][e] = ok ? feature(bf16_to_f32(e16[e])) : 0.f;
        if (x.want_out)
          *reinterpret_cast<uint4*>(x.sFk + (j0 + tt) * RF + 8 * io) = make_uint4(
              f32_to_bf16(f[tt][0]) | (uint32_t(f32_to_bf16(f[tt][1])) << 16),
              f32_to_bf16(f[tt][2]) | (uint32_t(f32_to_bf16(f[tt][3])) << 16),
              f32_to_bf16(f[tt][4]) | (uint32_t(f32_to_bf16(f[tt][5])) << 16),
              f32_to_bf16(f[tt][6]) | (uint32_t(f32_to_bf16(f[tt][7])) << 16));
      }
#pragma unroll
      for (int e = 0; e < 8; ++e)
        *reinterpret_cast<uint2*>(x.sFkT + (8 * io + e) * RC + j0) =
            pack4_bf16(f[0][e], f[1][e], f[2][e], f[3][e]);
    }
    if (lane < NV) {
      const uint16_t* e0 = reinterpret_cast<const uint16_t*>(&rv[0]);
      const uint16_t* e1 = reinterpret_cast<const uint16_t*>(&rv[1]);
      const uint16_t* e2 = reinterpret_cast<const uint16_t*>(&rv[2]);
      const uint16_t* e3 = reinterpret_cast<const uint16_t*>(&rv[3]);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        *reinterpret_cast<uint2*>(x.sVT + (8 * io + e) * RC + j0) =
            make_uint2(uint32_t(e0[e]) | (uint32_t(e1[e]) << 16),
                       uint32_t(e2[e]) | (uint32_t(e3[e]) << 16));
    }
    if (x.want_out) {
#pragma unroll
      for (int s = 0; s < KF; ++s) {
        const uint16_t* e16 = reinterpret_cast<const uint16_t*>(&rq[s]);
        bf16x8 v;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (__bf16)feature(bf16_to_f32(e16[e]));
        fq[s] = v;
      }
    }
  };

  __syncthreads();  // tables visible
  if (x.c_begin < x.c_end) {
    prefetch(x.c_begin);
    write_lds(x.c_begin);
  }
  __syncthreads();

  for (int c = x.c_begin; c < x.c_end; ++c) {
    if (c + 1 < x.c_end) prefetch(c + 1);
    if (x.want_out) {
      // ---- S^T tiles (rows j, columns i), causal: tiles jt <= r
      f32x4 accS[NR];
#pragma unroll
      for (int jt = 0; jt < NR; ++jt) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        if (jt <= r) {
#pragma unroll
          for (int s = 0; s < KF; ++s)
            acc = mma_bf16(lds8(x.sFk + (16 * jt + il) * RF + 32 * s + 8 * g).b, fq[s], acc);
          if (jt == r) {
#pragma unroll
            for (int q = 0; q < 4; ++q)
              if (4 * g + q > il) acc[q] = 0.f;
          }
        }
        accS[jt] = acc;
      }
      bf16x8 Sf[KC];
#pragma unroll
      for (int kb = 0; kb < KC; ++kb) Sf[kb] = pack_bf16(accS[2 * kb], accS[2 * kb + 1]);

      // ---- A'^T tiles (rows k, columns i)
      f32x4 accA[TM];
#pragma unroll
      for (int kt = 0; kt < TM; ++kt) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        const uint16_t* wrow = x.sWT + (16 * kt + il) * RC;
#pragma unroll
        for (int kb = 0; kb < KC; ++kb)
          if (32 * kb <= 16 * r + 15)
            acc = mma_bf16(lds44(wrow + 32 * kb + 4 * g, wrow + 32 * kb + 16 + 4 * g).b,
                           Sf[kb], acc);
        const uint16_t* urow = x.sLU + (16 * kt + il) * RF;
#pragma unroll
        for (int s = 0; s < KF; ++s) acc = mma_bf16(lds8(urow + 32 * s + 8 * g).b, fq[s], acc);
        accA[kt] = acc;
      }

      // ---- lam^(2i) A' (fp32), den_inter, per-query scale, fp16 operands [Re | -Im]
      float den_inter = 0.f, amax = 0.f;
#pragma unroll
      for (int mt = 0; mt < MH; ++mt)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float xr = accA[mt][q], yi = accA[mt + MH][q];
          const float2 L2 = lam2i[mt][q];
          const float ar = xr * L2.x - yi * L2.y, ai = xr * L2.y + yi * L2.x;
          accA[mt][q] = ar;
          accA[mt + MH][q] = -ai;
          const float2 le = x.sLE[16 * mt + 4 * g + q];
          den_inter += ar * le.x - ai * le.y;
          amax = fmaxf(amax, fmaxf(fabsf(ar), fabsf(ai)));
        }
      den_inter = xor_sum16_32(den_inter);
      amax = xor_max16_32(amax);
      const float si = pow2_scale(amax);
      f16x8 Af[KM];
#pragma unroll
      for (int kb = 0; kb < KM; ++kb)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          Af[kb][q] = (_Float16)(si * accA[2 * kb][q]);
          Af[kb][4 + q] = (_Float16)(si * accA[2 * kb + 1][q]);
        }

      // ---- P^T tiles (rows j, columns i), causal
      f32x4 accP[NR];
      float den_intra = 0.f;
#pragma unroll
      for (int jt = 0; jt < NR; ++jt) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        if (jt <= r) {
          const uint16_t* wrow = x.sWb + (16 * jt + il) * RM;
#pragma unroll
          for (int kb = 0; kb < KM; ++kb)
            acc = mma_f16(lds44(wrow + 32 * kb + 4 * g, wrow + 32 * kb + 16 + 4 * g).h, Af[kb],
                          acc);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            acc[q] *= x.wb_unscale;
            if (jt == r && 4 * g + q > il) acc[q] = 0.f;
            den_intra += acc[q];
          }
        }
        accP[jt] = acc;
      }
      den_intra = xor_sum16_32(den_intra);
      const float den = den_intra + si * den_inter;   // in units of si
      const float dcl = clamp_den(den, si * a.clamp);
      bf16x8 Pf[KC];
#pragma unroll
      for (int kb = 0; kb < KC; ++kb) Pf[kb] = pack_bf16(accP[2 * kb], accP[2 * kb + 1]);

      // ---- num^T tiles (rows d, columns i): P V (accI) + c_d-scaled Re(A lam G) (accX)
      const int t = c * C + 16 * r + il;
      const bool ok = t < a.N;
      const size_t obase = ok ? x.tok_index(a, x.pos_of(a, t)) * D : 0;
#pragma unroll
      for (int dt = 0; dt < TD; ++dt) {
        f32x4 accI = {0.f, 0.f, 0.f, 0.f}, accX = {0.f, 0.f, 0.f, 0.f};
        const uint16_t* vrow = x.sVT + (16 * dt + il) * RC;
#pragma unroll
        for (int kb = 0; kb < KC; ++kb)
          if (32 * kb <= 16 * r + 15)
            accI = mma_bf16(lds44(vrow + 32 * kb + 4 * g, vrow + 32 * kb + 16 + 4 * g).b,
                            Pf[kb], accI);
        const uint16_t* grow = x.sGT + (16 * dt + il) * RM;
#pragma unroll
        for (int kb = 0; kb < KM; ++kb)
          accX = mma_f16(lds44(grow + 32 * kb + 4 * g, grow + 32 * kb + 16 + 4 * g).h, Af[kb],
                         accX);
        if (ok) {
          const float4 cd = *reinterpret_cast<const float4*>(x.sC + 16 * dt + 4 * g);
          const float rd = 1.f / dcl;
          float val[4] = {(accI[0] + accX[0] / cd.x) * rd, (accI[1] + accX[1] / cd.y) * rd,
                          (accI[2] + accX[2] / cd.z) * rd, (accI[3] + accX[3] / cd.w) * rd};
          const size_t oi = obase + 16 * dt + 4 * g;
          if (a.acc_in) {
            const float4 prev = *reinterpret_cast<const float4*>(a.acc_in + oi);
            val[0] += prev.x; val[1] += prev.y; val[2] += prev.z; val[3] += prev.w;
          }
          if (a.out_bf16)
            *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.o) + oi) =
                pack4_bf16(val[0], val[1], val[2], val[3]);
          else
            *reinterpret_cast<float4*>(static_cast<float*>(a.o) + oi) =
                make_float4(val[0], val[1], val[2], val[3]);
        }
      }
    }
    __syncthreads();
    if (c + 1 < x.c_end) write_lds(c + 1);
    __syncthreads();
  }
}

// ---------------------------------------------------------------- state waves
// State wave u owns feature tiles ft = u, u+4, ... of U^T and value tiles dt = u, u+4, ...
// of G, in fp32 MFMA accumulators for the whole segment; wave 0 also owns eta.
template <int C, int F, int D, int M, int U>
__device__ __forceinline__ void state_main(const ChunkArgs& a, const Ctx<C, F, D, M>& x) {
  using Lay = Layout<C, F, D, M>;
  using TL = TableLayout<C, M>;
  constexpr int MH = M / 16;
  constexpr int TM = 2 * M / 16;
  constexpr int KC = C / 32;
  constexpr int TD = D / 16;
  constexpr int NFT = (F / 16 + 3) / 4;
  constexpr int NDT = (D / 16 + 3) / 4;
  constexpr int RF = Lay::RF, RC = Lay::RC, RM = Lay::RM;
  constexpr int u = U;   // compile-time: owned tiles below are constants
  const int lane = x.lane, il = x.il, g = x.g;

  f32x4 accU[NFT][TM];   // U^T tiles: rows f = 16ft + 4g + q, columns k = 16kt + il
  f32x4 accG[NDT][TM];   // G tiles:   rows k = 16kt + 4g + q, columns d = 16dt + il
  float2 eta = make_float2(0.f, 0.f);  // wave 0, lane m < M
#pragma unroll
  for (int fi = 0; fi < NFT; ++fi)
#pragma unroll
    for (int kt = 0; kt < TM; ++kt) accU[fi][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int di = 0; di < NDT; ++di)
#pragma unroll
    for (int kt = 0; kt < TM; ++kt) accG[di][kt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Initial state.
  const float2 *iU = nullptr, *iG = nullptr, *iE = nullptr;
  if (a.initc) {
    const float2* base = a.initc + ((size_t)x.seq * a.slots_per_seq + x.seg) * a.slot;
    iU = base;
    iG = base + (size_t)M * F;
    iE = base + (size_t)M * (F + D);
  } else if (x.seg == 0 && a.init0_U) {
    iU = a.init0_U + (size_t)x.seq * M * F;
    iG = a.init0_G + (size_t)x.seq * M * D;
    iE = a.init0_E + (size_t)x.seq * M;
  }
  if (iU) {
#pragma unroll
    for (int fi = 0; fi < NFT; ++fi) {
      const int ft = u + 4 * fi;
      if (ft < F / 16) {
#pragma unroll
        for (int mt = 0; mt < MH; ++mt) {
          const int m = 16 * mt + il;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float2 v = iU[(size_t)m * F + 16 * ft + 4 * g + q];
            accU[fi][mt][q] = v.x;
            accU[fi][mt + MH][q] = v.y;
          }
        }
      }
    }
#pragma unroll
    for (int di = 0; di < NDT; ++di) {
      const int dt = u + 4 * di;
      if (dt < TD) {
#pragma unroll
        for (int mt = 0; mt < MH; ++mt)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float2 v = iG[(size_t)(16 * mt + 4 * g + q) * D + 16 * dt + il];
            accG[di][mt][q] = v.x;
            accG[di][mt + MH][q] = v.y;
          }
      }
    }
    if (u == 0 && lane < M) eta = iE[lane];
  }

  // Operand copies of the state for the readout of chunk c: lam U (bf16), c_d lam G (fp16,
  // c_d a power of two per value column), lam eta; and chunk c's decay factors if it is the
  // last, partial chunk.
  auto publish = [&](int c) {
#pragma unroll
    for (int fi = 0; fi < NFT; ++fi) {
      const int ft = u + 4 * fi;
      if (ft < F / 16) {
#pragma unroll
        for (int mt = 0; mt < MH; ++mt) {
          const int m = 16 * mt + il;
          const float2 l = x.sLam[m];
          float re[4], im[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float xr = accU[fi][mt][q], yi = accU[fi][mt + MH][q];
            re[q] = l.x * xr - l.y * yi;
            im[q] = l.x * yi + l.y * xr;
          }
          *reinterpret_cast<uint2*>(x.sLU + m * RF + 16 * ft + 4 * g) =
              pack4_bf16(re[0], re[1], re[2], re[3]);
          *reinterpret_cast<uint2*>(x.sLU + (M + m) * RF + 16 * ft + 4 * g) =
              pack4_bf16(im[0], im[1], im[2], im[3]);
        }
      }
    }
#pragma unroll
    for (int di = 0; di < NDT; ++di) {
      const int dt = u + 4 * di;
      if (dt < TD) {
        const int d = 16 * dt + il;
        // Column max of |lam G| first, then the scaled copy (lam G recomputed, not held).
        float mx = 0.f;
#pragma unroll
        for (int mt = 0; mt < MH; ++mt)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float2 l = x.sLam[16 * mt + 4 * g + q];
            const float xr = accG[di][mt][q], yi = accG[di][mt + MH][q];
            mx = fmaxf(mx, fmaxf(fabsf(l.x * xr - l.y * yi), fabsf(l.x * yi + l.y * xr)));
          }
        mx = xor_max16_32(mx);
        const float cd = pow2_scale(mx);
        if (g == 0) x.sC[d] = cd;
#pragma unroll
        for (int mt = 0; mt < MH; ++mt) {
          float re[4], im[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float2 l = x.sLam[16 * mt + 4 * g + q];
            const float xr = accG[di][mt][q], yi = accG[di][mt + MH][q];
            re[q] = cd * (l.x * xr - l.y * yi);
            im[q] = cd * (l.x * yi + l.y * xr);
          }
          *reinterpret_cast<uint2*>(x.sGT + d * RM + 16 * mt + 4 * g) =
              pack4_f16(re[0], re[1], re[2], re[3]);
          *reinterpret_cast<uint2*>(x.sGT + d * RM + M + 16 * mt + 4 * g) =
              pack4_f16(im[0], im[1], im[2], im[3]);
        }
      }
    }
    if (u == 0 && lane < M) {
      const float2 l = x.sLam[lane];
      x.sLE[lane] = make_float2(l.x * eta.x - l.y * eta.y, l.x * eta.y + l.y * eta.x);
      if (a.N - c * C < C) {
        x.sPowL[lane] = reinterpret_cast<const float2*>(x.tab + TL::oPowT)[lane];
        x.sGeo[lane] = reinterpret_cast<const float2*>(x.tab + TL::oGeoT)[lane];
      }
    }
  };

  __syncthreads();  // tables visible
  if (x.c_begin < x.c_end) publish(x.c_begin);
  __syncthreads();

  for (int c = x.c_begin; c < x.c_end; ++c) {
    // U^T <- lam^(L-1) (lam U^T + phi(K)^T (beta lam^-j)),  G <- lam^(L-1) (lam G + W^T V)
    bf16x8 afk[NFT][KC], bv[NDT][KC];
#pragma unroll
    for (int fi = 0; fi < NFT; ++fi) {
      const int ft = u + 4 * fi;
      if (ft < F / 16) {
#pragma unroll
        for (int kb = 0; kb < KC; ++kb)
          afk[fi][kb] = lds8(x.sFkT + (16 * ft + il) * RC + 32 * kb + 8 * g).b;
#pragma unroll
        for (int mt = 0; mt < MH; ++mt) {
          const float2 l = x.sLam[16 * mt + il];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float xr = accU[fi][mt][q], yi = accU[fi][mt + MH][q];
            accU[fi][mt][q] = l.x * xr - l.y * yi;
            accU[fi][mt + MH][q] = l.x * yi + l.y * xr;
          }
        }
      }
    }
#pragma unroll
    for (int di = 0; di < NDT; ++di) {
      const int dt = u + 4 * di;
      if (dt < TD) {
#pragma unroll
        for (int kb = 0; kb < KC; ++kb)
          bv[di][kb] = lds8(x.sVT + (16 * dt + il) * RC + 32 * kb + 8 * g).b;
#pragma unroll
        for (int mt = 0; mt < MH; ++mt)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float2 l = x.sLam[16 * mt + 4 * g + q];
            const float xr = accG[di][mt][q], yi = accG[di][mt + MH][q];
            accG[di][mt][q] = l.x * xr - l.y * yi;
            accG[di][mt + MH][q] = l.x * yi + l.y * xr;
          }
      }
    }
#pragma unroll
    for (int kt = 0; kt < TM; ++kt) {
#pragma unroll
      for (int kb = 0; kb < KC; ++kb) {
        const bf16x8 w = lds8(x.sWT + (16 * kt + il) * RC + 32 * kb + 8 * g).b;
#pragma unroll
        for (int fi = 0; fi < NFT; ++fi)
          if (u + 4 * fi < F / 16) accU[fi][kt] = mma_bf16(afk[fi][kb], w, accU[fi][kt]);
#pragma unroll
        for (int di = 0; di < NDT; ++di)
          if (u + 4 * di < TD) accG[di][kt] = mma_bf16(w, bv[di][kb], accG[di][kt]);
      }
    }
#pragma unroll
    for (int fi = 0; fi < NFT; ++fi)
      if (u + 4 * fi < F / 16) {
#pragma unroll
        for (int mt = 0; mt < MH; ++mt) {
          const float2 p = x.sPowL[16 * mt + il];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float xr = accU[fi][mt][q], yi = accU[fi][mt + MH][q];
            accU[fi][mt][q] = p.x * xr - p.y * yi;
            accU[fi][mt + MH][q] = p.x * yi + p.y * xr;
          }
        }
      }
#pragma unroll
    for (int di = 0; di < NDT; ++di)
      if (u + 4 * di < TD) {
#pragma unroll
        for (int mt = 0; mt < MH; ++mt)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float2 p = x.sPowL[16 * mt + 4 * g + q];
            const float xr = accG[di][mt][q], yi = accG[di][mt + MH][q];
            accG[di][mt][q] = p.x * xr - p.y * yi;
            accG[di][mt + MH][q] = p.x * yi + p.y * xr;
          }
      }
    if (u == 0 && lane < M) {
      const float2 l = x.sLam[lane], p = x.sPowL[lane], ge = x.sGeo[lane];
      const float2 t = make_float2(l.x * eta.x - l.y * eta.y + ge.x,
                                   l.x * eta.y + l.y * eta.x + ge.y);
      eta = make_float2(p.x * t.x - p.y * t.y, p.x * t.y + p.y * t.x);
    }
    __syncthreads();
    if (c + 1 < x.c_end) publish(c + 1);
    __syncthreads();
  }

  // Final state.
  float2 *fU = nullptr, *fG = nullptr, *fE = nullptr;
  if (a.fin_seg) {
    float2* base = a.fin_seg + ((size_t)x.seq * a.slots_per_seq + x.seg + 1) * a.slot;
    fU = base;
    fG = base + (size_t)M * F;
    fE = base + (size_t)M * (F + D);
  } else if (x.last_seg && a.fin_U) {
    fU = a.fin_U + (size_t)x.seq * M * F;
    fG = a.fin_G + (size_t)x.seq * M * D;
    fE = a.fin_E + (size_t)x.seq * M;
  }
  if (fU) {
#pragma unroll
    for (int fi = 0; fi < NFT; ++fi) {
      const int ft = u + 4 * fi;
      if (ft < F / 16) {
#pragma unroll
        for (int mt = 0; mt < MH; ++mt) {
          const int m = 16 * mt + il;
#pragma unroll
          for (int q = 0; q < 4; ++q)
            fU[(size_t)m * F + 16 * ft + 4 * g + q] =
                make_float2(accU[fi][mt][q], accU[fi][mt + MH][q]);
        }
      }
    }
#pragma unroll
    for (int di = 0; di < NDT; ++di) {
      const int dt = u + 4 * di;
      if (dt < TD) {
#pragma unroll
        for (int mt = 0; mt < MH; ++mt)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            fG[(size_t)(16 * mt + 4 * g + q) * D + 16 * dt + il] =
                make_float2(accG[di][mt][q], accG[di][mt + MH][q]);
      }
    }
    if (u == 0 && lane < M) fE[lane] = eta;
  }
}

template <int C, int F, int D, int M, int W>
__device__ __forceinline__ void run_role(const ChunkArgs& a, const Ctx<C, F, D, M>& x) {
  if constexpr (W < C / 16)
    readout_main<C, F, D, M, W>(a, x);
  else
    state_main<C, F, D, M, W - C / 16>(a, x);
}

template <int C, int F, int D, int M, int... Ws>
__device__ __forceinline__ void dispatch_role(const ChunkArgs& a, const Ctx<C, F, D, M>& x,
                                              int w, std::integer_sequence<int, Ws...>) {
  ((w == Ws ? (run_role<C, F, D, M, Ws>(a, x), 0) : 0), ...);
}

template <int C, int F, int D, int M>
__global__ void __launch_bounds__(64 * (C / 16 + 4))
chunk_prefill_kernel(const ChunkArgs a) {
  using Lay = Layout<C, F, D, M>;
  using TL = TableLayout<C, M>;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  uint16_t* s16 = reinterpret_cast<uint16_t*>(smem_raw);

  Ctx<C, F, D, M> x;
  x.sFk = s16 + Lay::oFk;
  x.sFkT = s16 + Lay::oFkT;
  x.sVT = s16 + Lay::oVT;
  x.sWT = s16 + Lay::oWT;
  x.sWb = s16 + Lay::oWb;
  x.sLU = s16 + Lay::oLU;
  x.sGT = s16 + Lay::oGT;
  x.sC = reinterpret_cast<float*>(smem_raw + Lay::bC);
  x.sLE = reinterpret_cast<float2*>(smem_raw + Lay::bLE);
  x.sLam = reinterpret_cast<float2*>(smem_raw + Lay::bLam);
  x.sPowL = reinterpret_cast<float2*>(smem_raw + Lay::bPowL);
  x.sGeo = reinterpret_cast<float2*>(smem_raw + Lay::bGeo);
  const int tid = threadIdx.x;
  x.lane = tid & 63;
  x.wave = tid >> 6;
  x.il = x.lane & 15;
  x.g = x.lane >> 4;
  x.seq = blockIdx.x / a.n_seg;
  x.seg = a.seg_first + blockIdx.x % a.n_seg;
  x.b = x.seq / a.H;
  x.h = x.seq % a.H;
  const int n_chunks_total = (a.N + C - 1) / C;
  x.c_begin = x.seg * a.seg_chunks;
  x.c_end = min(x.c_begin + a.seg_chunks, n_chunks_total);
  x.last_seg = x.c_end == n_chunks_total;
  x.want_out = a.o != nullptr;
  x.tab = a.tables + (size_t)x.h * a.table_bytes;

  // Per-head tables -> LDS (sWT and sWb are adjacent, padded alike, in LDS and the table).
  static_assert(Lay::oWb == Lay::oWT + 2 * M * Lay::RC, "tables adjacent");
  {
    const uint4* src = reinterpret_cast<const uint4*>(x.tab + TL::oW);
    uint4* dst = reinterpret_cast<uint4*>(x.sWT);
    for (int e = tid; e < (int)(TL::nW / 16); e += blockDim.x) dst[e] = src[e];
  }
  x.wb_unscale = *reinterpret_cast<const float*>(x.tab + TL::oSc);
  const float2* lamh = a.lam + (size_t)x.h * M;
  for (int m = tid; m < M; m += blockDim.x) {
    x.sLam[m] = lamh[m];
    x.sPowL[m] = reinterpret_cast<const float2*>(x.tab + TL::oPow)[m];
    x.sGeo[m] = reinterpret_cast<const float2*>(x.tab + TL::oGeo)[m];
  }
  // Both roles run the same sequence of block barriers.  Each wave runs code specialised
  // for its index, so trip counts and owned tiles are compile-time constants.
  dispatch_role<C, F, D, M>(a, x, x.wave, std::make_integer_sequence<int, C / 16 + 4>{});
}

template <int C, int F, int D, int M>
hipError_t launch_chunk_t(const ChunkArgs& a, int n_wg, hipStream_t st, int kind) {
  constexpr int threads = 64 * (C / 16 + 4);
  constexpr int bytes = Layout<C, F, D, M>::bytes;
  static_assert(bytes <= 160 * 1024, "LDS budget");
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&chunk_prefill_kernel<C, F, D, M>),
        hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  (void)hipGetLastError();
  prof_begin(st);
  hipLaunchKernelGGL((chunk_prefill_kernel<C, F, D, M>), dim3(n_wg), dim3(threads), bytes, st,
                     a);
  prof_end(st, kind);
  return hipGetLastError();
}

}  // namespace ia
