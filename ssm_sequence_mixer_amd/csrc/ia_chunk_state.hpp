// ia_chunk_state.hpp — state-only pass of the chunked IA prefill on gfx950 MFMA: the end state
// of a full segment of Ls = nc*C tokens from a zero state.  Included by the per-feature-width
// translation units that instantiate it.
//
// In the frame the prefill carries (X = lam U, lam Gamma, lam eta; "Interdomain Attention:
// Beyond Token-Level Key-Value Memory", summary page §3.2 for the recurrence, §A.2 for the
// chunkwise form), the end state of a segment started from zero is a plain contraction over
// its tokens t:
//   X[k,f] = sum_t beta_k lam_k^(Ls-t) phi(k_t)[f],   lam G likewise with v_t,
//   lam eta = sum_t beta lam^(Ls-t).
// With t = c C + j this is, per chunk c, the table T_c[k,j] = lam^((nc-1-c) C) beta lam^(C-j)
// against the chunk's features: no per-chunk decay of the accumulators.  Chunks are walked
// from the segment's last to its first, so the chunk factor pw = lam^(i C) (i = nc-1-c) only
// shrinks and underflows exactly where the contribution vanishes.
//
// Workgroup = one (b, h, segment); NS waves with the tile ownership of the output pass's
// state waves, so the final accumulators are already in the workspace slot layout.  LDS holds
// two stages of (phi(k), v, T); each wave keeps three chunks of raw inputs in flight in
// registers, one barrier per chunk.  (Splitting each wave's U and G tiles over two waves was
// measured slower: the table is then read twice per chunk.)
#pragma once

#include <type_traits>

#include "ia_chunk.hpp"
#include "ia_tables.hpp"

namespace ia {

template <int C, int F, int D, int M, bool GT = false>
struct StateLayout {
  static constexpr int M2 = 2 * M;
  // 16-bit element offsets within a stage; every matrix swizzled by row (see soff).
  static constexpr int oFk = 0;            // [C][F]   bf16 phi(k)
  static constexpr int oV = C * F;         // [C][D]   bf16 v
  static constexpr int oT = oV + C * D;    // [2M][C]  bf16 T_c (j in K-slot order)
  static constexpr int stage = oT + M2 * C;
  // Gated layer: three buffers of per-token gate factors (walk iteration i in buffer i % 3).
  static constexpr int bFac = 2 * stage * 2;
  static constexpr int bytes = bFac + (GT ? 3 * C * 4 : 0);
};

// Gated layer (GT): token j of the chunk of walk iteration i enters the segment's end state
// with the factor w_j prod_{s > j in the segment} a_s = E_i[j] P_i (GateRec's E of that chunk,
// P_i the decay product of the chunks walked before it, which lie after it), folded into the
// chunk's table T_i; lam eta is the sum of the tables' fp32 entries; the slot also receives
// the segment's decay product.
template <int C, int F, int D, int M, bool GT>
__global__ void __launch_bounds__((64 * StateWaves<F, D, M>::NS))
chunk_state_kernel(const ChunkArgs a) {
  using SL = SlotLayout<F, D, M>;
  using Lay = StateLayout<C, F, D, M, GT>;
  constexpr int NS = StateWaves<F, D, M>::NS;
  constexpr int NFT = SL::NFT, NDT = SL::NDT, TM = SL::TM;
  constexpr int KC = C / 32;
  constexpr int TD = D / 16;
  constexpr int VF = F / 8, VD = D / 8;
  constexpr int NL = 64 * NS;
  constexpr int NLK = (C * VF + NL - 1) / NL, NLV = (C * VD + NL - 1) / NL;
  constexpr int GROUPS = M * C / 4;          // table groups: 4 consecutive j of one mode
  constexpr int NGR = (GROUPS + NL - 1) / NL;
  constexpr int ST = Lay::stage;
  constexpr int LOGC = C == 64 ? 6 : 5;
  static_assert(C == 1 << LOGC, "chunk a power of two");
  static_assert((NL / VF) % 16 == 0 && (NL / VD) % 16 == 0, "loader rows keep the swizzle");
  static_assert(Lay::bytes <= 160 * 1024, "LDS budget");

  extern __shared__ __align__(16) unsigned char smem_raw[];
  uint16_t* const s16 = reinterpret_cast<uint16_t*>(smem_raw);
  const int tid = threadIdx.x, lane = tid & 63, u = tid >> 6;
  if (a.tables_out && (int)blockIdx.x >= a.n_sum_wg) {
    // Table workgroup of head blockIdx.x - n_sum_wg: its C/4 table runs, RPP at a time.  The
    // state-only workgroups below do not read these tables; the output pass does.
    constexpr int RPP = 64 * NS / (4 * M);
    static_assert(RPP >= 1 && (C / 4) % RPP == 0, "whole table runs per pass");
    const int h = blockIdx.x - a.n_sum_wg;
    for (int r0 = 0; r0 < C / 4; r0 += RPP)
      table_run<C, M>(a.lam, a.beta, a.tables_out, a.table_bytes, a.Lt, a.seg_chunks * C, h,
                      r0 + tid / (4 * M), tid % (4 * M), a.tables_half);
    if (a.rtab_out) readout_table_run<M>(a.readout, a.rtab_out, a.rtab_bytes, h, tid, 64 * NS);
    return;
  }
  const int il = lane & 15, g = lane >> 4;
  // Both walks of a bidirectional call in one launch (seg_end_rev set): workgroups from
  // n_dir_wg on take the reverse walk and its slots.
  int wg = blockIdx.x, dir = a.dir;
  float* seg_end = a.seg_end;
  if (a.seg_end_rev && wg >= a.n_dir_wg) {
    wg -= a.n_dir_wg;
    dir = 1;
    seg_end = a.seg_end_rev;
  }
  int seq, seg;
  if (!pair_wg(wg, a.H * a.B, a.n_seg, a.pair_heads, seq, seg)) return;
  seg += a.seg_first;
  const int b = seq / a.H, h = seq % a.H;
  const int nc = a.seg_chunks;               // a full segment
  const int c_first = seg * nc;

  // ---- per-lane LDS offsets (stage 0; stage 1 adds the constant ST)
  int offT[KC], trF[NFT], trD[NDT];
#pragma unroll
  for (int kb = 0; kb < KC; ++kb) offT[kb] = opaque(Lay::oT + lane_off<C>(il, 4 * kb + g));
#pragma unroll
  for (int fi = 0; fi < NFT; ++fi) trF[fi] = opaque(Lay::oFk + tr_off<F>(u + NS * fi, lane));
#pragma unroll
  for (int di = 0; di < NDT; ++di) trD[di] = opaque(Lay::oV + tr_off<D>(u + NS * di, lane));

  // ---- loader: 16-byte vectors n = n0 + NL t of the row-major chunk matrices k ([C][F]) and
  // v ([C][D]); token rows are sqk.n (sv.n) elements apart, backwards in the reverse
  // direction.
  const int n0 = 64 * u + lane;
  const int rowK0 = n0 / VF, rowV0 = n0 / VD;
  const int sgn = dir ? -1 : 1;
  const int snK = (int)a.sqk.n, snV = (int)a.sv.n;   // < 2^23 (the host checks)
  const int lofK = sgn * rowK0 * snK + 8 * (n0 % VF);
  const int lofV = sgn * rowV0 * snV + 8 * (n0 % VD);
  const int stepK = sgn * (NL / VF) * snK, stepV = sgn * (NL / VD) * snV;
  const int stK = opaque(Lay::oFk + soff<F>(rowK0, 8 * (n0 % VF)));
  const int stV = opaque(Lay::oV + soff<D>(rowV0, 8 * (n0 % VD)));
  uint4 rk[3][NLK], rv[3][NLV];
  // Walk chunk of iteration i: the segment's chunks from last to first.
  auto chunk_of = [&](int i) { return c_first + nc - 1 - i; };
  auto fetch = [&](auto R, int i) {
    constexpr int r = decltype(R)::value;
    const int t0 = chunk_of(i) * C;
    const long long pos = dir ? a.N - 1 - t0 : t0;
    const uint16_t* kb = a.k + b * a.sqk.b + pos * a.sqk.n + h * a.sqk.h + lofK;
    const uint16_t* vb = a.v + b * a.sv.b + pos * a.sv.n + h * a.sv.h + lofV;
#pragma unroll
    for (int t = 0; t < NLK; ++t)
      rk[r][t] = n0 + NL * t < C * VF ? *reinterpret_cast<const uint4*>(kb + t * stepK)
                                      : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int t = 0; t < NLV; ++t)
      rv[r][t] = n0 + NL * t < C * VD ? *reinterpret_cast<const uint4*>(vb + t * stepV)
                                      : make_uint4(0, 0, 0, 0);
  };
  // phi(k) in place (k itself with kOptIdentity), then both into the stage.
  const float fT = feature_t(a.opt), fC = feature_c(a.opt);
  auto write_inputs = [&](auto R, auto S) {
    constexpr int r = decltype(R)::value, so = decltype(S)::value * ST;
#pragma unroll
    for (int t = 0; t < NLK; ++t)
      if (n0 + NL * t < C * VF) {
        const uint32_t w[4] = {rk[r][t].x, rk[r][t].y, rk[r][t].z, rk[r][t].w};
        uint32_t o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          o[e] = pk_bf16(feature_tc(__uint_as_float(w[e] << 16), fT, fC),
                         feature_tc(__uint_as_float(w[e] & 0xffff0000u), fT, fC));
        *reinterpret_cast<uint4*>(s16 + stK + so + t * (NL / VF) * F) =
            make_uint4(o[0], o[1], o[2], o[3]);
      }
#pragma unroll
    for (int t = 0; t < NLV; ++t)
      if (n0 + NL * t < C * VD)
        *reinterpret_cast<uint4*>(s16 + stV + so + t * (NL / VD) * D) = rv[r][t];
  };

  // ---- chunk table T_i = pw_i beta lam^(C-j), pw_i = lam^(i C): this thread's groups of 4
  // consecutive j of one mode, beta lam^(C-j) held in registers for the whole segment.  The
  // powers are computed here from lam and beta (binary exponentiation in fp64), while the
  // first chunks load (init_tables, after those loads are issued), so this pass does not wait
  // for the per-head tables.
  float2 tl[NGR][4], pw[NGR], pc[NGR];
  int tRe[NGR], tIm[NGR];
  auto init_tables = [&]() {
#pragma unroll
    for (int q = 0; q < NGR; ++q) {
      const int gi = tid + NL * q;
      const int m = gi < GROUPS ? gi / (C / 4) : 0, j0 = 4 * (gi % (C / 4));
      const float2 l = a.lam[(size_t)h * M + m];
      float2 base;   // lam^(C-j0-3), the group's smallest exponent (>= 1)
      LamSmallPow(l).pow_and_top<LOGC>(C - j0 - 3, base, pc[q]);
      tl[q][3] = cmul(a.beta[(size_t)h * M + m], base);
#pragma unroll
      for (int e = 2; e >= 0; --e) tl[q][e] = cmul(tl[q][e + 1], l);
      pw[q] = make_float2(1.f, 0.f);
      tRe[q] = opaque(Lay::oT + soff<C>(m, kpos(j0)));
      tIm[q] = opaque(Lay::oT + soff<C>(M + m, kpos(j0)));
    }
  };
  // Gated: per-token factors of walk iteration i in buffer i % 3 (wave 0 writes iteration
  // i + 2's during iteration i), and this thread's share of lam eta: the fp32 sum of its groups'
  // table entries over the 16-lane row's C/4 groups of one mode, kept by the row's first lane.
  float* const fac = reinterpret_cast<float*>(smem_raw + Lay::bFac);
  float2 eta_g[NGR];
#pragma unroll
  for (int q = 0; q < NGR; ++q) eta_g[q] = make_float2(0.f, 0.f);
  auto write_table = [&](auto S, int i) {
    constexpr int so = decltype(S)::value * ST;
#pragma unroll
    for (int q = 0; q < NGR; ++q) {
      float2 w[4];
      const bool own = tid + NL * q < GROUPS;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = cmul(pw[q], tl[q][e]);
      if constexpr (GT) {
        const int j0 = 4 * ((tid + NL * q) % (C / 4));
        const float4 f4 = *reinterpret_cast<const float4*>(fac + (i % 3) * C + j0);
        const float f[4] = {f4.x, f4.y, f4.z, f4.w};
        float2 sum = make_float2(0.f, 0.f);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          w[e].x *= f[e];
          w[e].y *= f[e];
          sum.x += w[e].x;
          sum.y += w[e].y;
        }
        // over the C/4 lanes of the mode (DPP: quad swaps, then half-row and row mirrors)
        sum.x = dpp_add<0x141>(dpp_add<0x4E>(dpp_add<0xB1>(sum.x)));
        sum.y = dpp_add<0x141>(dpp_add<0x4E>(dpp_add<0xB1>(sum.y)));
        if constexpr (C / 4 == 16) {
          sum.x = dpp_add<0x140>(sum.x);
          sum.y = dpp_add<0x140>(sum.y);
        }
        static_assert(C / 4 == 8 || C / 4 == 16, "8 or 16 groups per mode");
        eta_g[q].x += sum.x;
        eta_g[q].y += sum.y;
      }
      if (own) {
        *reinterpret_cast<uint2*>(s16 + tRe[q] + so) = pack4_bf16(w[0].x, w[1].x, w[2].x, w[3].x);
        *reinterpret_cast<uint2*>(s16 + tIm[q] + so) = pack4_bf16(w[0].y, w[1].y, w[2].y, w[3].y);
      }
    }
  };
  // Gated: wave 0 turns the gates of walk iteration k into its factors (buffer k % 3), keeping
  // P (the decay product of the iterations before) and the raw gates of the next iteration.
  // (Gate loads go out before the same iteration's input loads, so waiting for them does not
  // wait for those.)
  float2 graw = make_float2(1.f, 0.f);
  float gP = 1.f;
  auto gate_load = [&](int k) {
    return u == 0 ? gate_fetch(a, b, h, dir, chunk_of(k), C, lane) : make_float2(1.f, 0.f);
  };
  auto gate_factors = [&](float2 raw, int k) {
    if (u == 0) {
      const GateScan gs = gate_scan(raw, lane < C);   // segments hold full chunks
      if (lane < C) fac[(k % 3) * C + lane] = gs.e * gP;
      gP *= gs.d;
    }
  };
  auto advance_table = [&]() {
#pragma unroll
    for (int q = 0; q < NGR; ++q) pw[q] = cmul(pw[q], pc[q]);
  };

  // ---- accumulators (lam U)^T and lam G in the output pass's state-wave layout; lam eta in
  // wave 0, lane m < M.
  f32x4 accU[NFT][TM], accG[NDT][TM];
#pragma unroll
  for (int fi = 0; fi < NFT; ++fi)
#pragma unroll
    for (int kt = 0; kt < TM; ++kt) accU[fi][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int di = 0; di < NDT; ++di)
#pragma unroll
    for (int kt = 0; kt < TM; ++kt) accG[di][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float2 eta = make_float2(0.f, 0.f), epw = make_float2(1.f, 0.f), epc = epw, egeo = eta;
  auto init_eta = [&]() {
    if (u == 0 && lane < M) {   // lam^C and sum_j beta lam^(C-j) of mode `lane`
      const LamSmallPow lp(a.lam[(size_t)h * M + lane]);
      double cr, ci;
      lp.top<LOGC>(cr, ci);
      epc = make_float2((float)cr, (float)ci);
      egeo = lp.geo(a.beta[(size_t)h * M + lane], C, cr, ci);
    }
  };

  auto update = [&](auto S) {
    constexpr int so = decltype(S)::value * ST;
#pragma unroll
    for (int kb = 0; kb < KC; ++kb) {
      bf16x8 afk[NFT], bv[NDT];
#pragma unroll
      for (int fi = 0; fi < NFT; ++fi)
        if (u + NS * fi < F / 16) afk[fi] = ldtr<F>(s16, trF[fi] + so, kb).b;
#pragma unroll
      for (int di = 0; di < NDT; ++di)
        if (u + NS * di < TD) bv[di] = ldtr<D>(s16, trD[di] + so, kb).b;
#pragma unroll
      for (int kt = 0; kt < TM; ++kt) {
        const bf16x8 w = lds8(s16 + offT[kb] + so + 16 * kt * C).b;
#pragma unroll
        for (int fi = 0; fi < NFT; ++fi)
          if (u + NS * fi < F / 16) accU[fi][kt] = mma_bf16(afk[fi], w, accU[fi][kt]);
#pragma unroll
        for (int di = 0; di < NDT; ++di)
          if (u + NS * di < TD) accG[di][kt] = mma_bf16(w, bv[di], accG[di][kt]);
      }
    }
    if constexpr (!GT) {
      if (u == 0 && lane < M) {
        eta = cfma(epw, egeo, eta);
        epw = cmul(epw, epc);
      }
    }
  };

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  // Iteration i: update from stage i%2; convert chunk i+1 (ring set (i+1)%3, loaded two
  // iterations ago) into stage (i+1)%2 with its table; load chunk i+3 into set i%3.
  auto step = [&](auto Rc, auto Rf, auto Sr, auto Sw, int i) {
    update(Sr);
    if (i + 1 < nc) {
      advance_table();
      write_inputs(Rc, Sw);
      write_table(Sw, i + 1);
      if constexpr (GT) {
        if (i + 2 < nc) gate_factors(graw, i + 2);
        if (i + 3 < nc) graw = gate_load(i + 3);
      }
      if (i + 3 < nc) fetch(Rf, i + 3);
    }
    __syncthreads();
  };

  float2 g0 = graw, g1 = graw;
  if constexpr (GT) {
    g0 = gate_load(0);
    if (nc > 1) g1 = gate_load(1);
    if (nc > 2) graw = gate_load(2);
  }
  fetch(I0{}, 0);
  if (nc > 1) fetch(I1{}, 1);
  if (nc > 2) fetch(I2{}, 2);
  if constexpr (GT) {
    gate_factors(g0, 0);
    if (nc > 1) gate_factors(g1, 1);
  }
  init_tables();
  if constexpr (!GT) init_eta();
  write_inputs(I0{}, I0{});
  if constexpr (GT) __syncthreads();   // iteration 0's factors visible
  write_table(I0{}, 0);
  __syncthreads();
  for (int i = 0; i < nc; i += 6) {
    step(I1{}, I0{}, I0{}, I1{}, i);
    if (i + 1 < nc) step(I2{}, I1{}, I1{}, I0{}, i + 1);
    if (i + 2 < nc) step(I0{}, I2{}, I0{}, I1{}, i + 2);
    if (i + 3 < nc) step(I1{}, I0{}, I1{}, I0{}, i + 3);
    if (i + 4 < nc) step(I2{}, I1{}, I0{}, I1{}, i + 4);
    if (i + 5 < nc) step(I0{}, I2{}, I1{}, I0{}, i + 5);
  }

  // ---- end state into the segment's slot (fp16 tile pairs, see SlotLayout).  The row maxima
  // of all the wave's pairs are reduced together, so their shuffles overlap.
  float* sl = seg_end + ((size_t)seq * a.slots_per_seq + seg) * a.slot_floats;
  constexpr int MH = M / 16;
  constexpr int NPW = (NFT + NDT) * MH;   // tile pairs of this wave, SlotLayout order
  auto pair_vals = [&](int p, float (&re)[4], float (&im)[4]) {
    const int ts = p / MH, mt = p % MH;
    const f32x4& r = ts < NFT ? accU[ts][mt] : accG[ts - NFT][mt];
    const f32x4& m = ts < NFT ? accU[ts][mt + MH] : accG[ts - NFT][mt + MH];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      re[q] = r[q];
      im[q] = m[q];
    }
  };
  auto owned = [&](int p) {
    const int ts = p / MH;
    return ts < NFT ? u + NS * ts < F / 16 : u + NS * (ts - NFT) < TD;
  };
  float mx[NPW];
#pragma unroll
  for (int p = 0; p < NPW; ++p) {
    float re[4], im[4];
    pair_vals(p, re, im);
    float v = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) v = fmaxf(v, fmaxf(fabsf(re[q]), fabsf(im[q])));
    mx[p] = v;
  }
#pragma unroll
  for (int o = 1; o < 16; o <<= 1)
#pragma unroll
    for (int p = 0; p < NPW; ++p) mx[p] = fmaxf(mx[p], __shfl_xor(mx[p], o, 16));
#pragma unroll
  for (int p = 0; p < NPW; ++p)
    if (owned(p)) {
      float re[4], im[4];
      pair_vals(p, re, im);
      const float sc = pow2_scale(mx[p]);
      const uint2 r = pack4_f16(re[0] * sc, re[1] * sc, re[2] * sc, re[3] * sc);
      const uint2 m = pack4_f16(im[0] * sc, im[1] * sc, im[2] * sc, im[3] * sc);
      *reinterpret_cast<uint4*>(sl + SL::pair(u, p, lane)) = make_uint4(r.x, r.y, m.x, m.y);
      if (il == 0) sl[SL::scale_of(u, p, lane)] = 1.f / sc;
    }
  if constexpr (GT) {
#pragma unroll
    for (int q = 0; q < NGR; ++q) {
      const int gi = tid + NL * q;
      if (gi < GROUPS && gi % (C / 4) == 0)
        reinterpret_cast<float2*>(sl + SL::eta)[gi / (C / 4)] = eta_g[q];
    }
    if (tid == 0) sl[SL::dseg] = gP;
  } else {
    if (u == 0 && lane < M) reinterpret_cast<float2*>(sl + SL::eta)[lane] = eta;
  }
}

template <int C, int F, int D, int M, bool GT = false>
hipError_t launch_state_t(const ChunkArgs& a, int n_wg, hipStream_t st, int kind) {
  constexpr int threads = 64 * StateWaves<F, D, M>::NS;
  constexpr int bytes = StateLayout<C, F, D, M, GT>::bytes;
  static_assert(bytes <= 160 * 1024, "LDS budget");
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&chunk_state_kernel<C, F, D, M, GT>),
        hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  (void)hipGetLastError();
  prof_begin(st);
  hipLaunchKernelGGL((chunk_state_kernel<C, F, D, M, GT>), dim3(n_wg), dim3(threads), bytes, st,
                     a);
  prof_end(st, kind);
  return hipGetLastError();
}

}  // namespace ia
