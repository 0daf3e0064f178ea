// ia_block_step.hpp — the block's prologue for one token inside a decode workgroup
// ("Interdomain Attention: Beyond Token-Level Key-Value Memory": summary page §5.3 and §B.1 for
// the short convolutions, §A.1 for RoPE, §3.3 for the output gate; AI Radio episode page,
// "Implementation Details", for the normalised SSM input).  The same readings as the prologue
// kernel of ia_block.hip: causal depthwise convolution (tap 0 on the current token, the W-1
// earlier raw tokens from the carried state) and SiLU, RoPE on q and k, the feature map, then
// z = [phi(k), v] scaled to unit RMS with a per-head gain and bias.
//
// Split in two so that a decode kernel can issue its state loads between them: load() issues
// every global load of the token's inputs, finish() computes and writes phi(q') and the
// normalised phi(k') and v' to LDS, and the new convolution state to memory.  The SiLU and
// RoPE helpers here serve the prefill prologue of ia_block.hip too.
#pragma once

#include "ia_device.hpp"
#include "ia_kernels.hpp"

namespace ia {

__device__ __forceinline__ float silu_f(float y) {
  return y * __builtin_amdgcn_rcpf(1.f + __expf(-y));
}

// RoPE: pair i of F features turns by base^(-2i/F) / (2 pi) turns per position (fp64).
__device__ __forceinline__ double rope_rate(float base, int i, int F) {
  return pow((double)base, -2.0 * i / F) * 0.15915494309189535;
}
// (cos, sin) of the angle pos * rate turns: reduced to [0, 1) turns in fp64, then the
// hardware cosine and sine, which take turns.
__device__ __forceinline__ float2 rope_cs(double pos, double rate) {
  const float tr = (float)__builtin_amdgcn_fract(pos * rate);
  return make_float2(__builtin_amdgcn_cosf(tr), __builtin_amdgcn_sinf(tr));
}

// RoPE angles stepped from anchors.  Positions that are multiples of kRopeAnchor take their
// (cos, sin) from rope_cs; a position after an anchor multiplies the anchor's value by the
// one-position turn (rope_cs(1, rate)) once per position, in order.  A position's value thus
// depends on the position alone, so a call split into pieces gives the same bits, while 15 of
// 16 positions cost a complex multiplication instead of a sine and a cosine (the products
// drift by a few fp32 ulps at most).
constexpr int kRopeAnchor = 16;
__device__ __forceinline__ float2 rope_step(double rate) { return rope_cs(1.0, rate); }
// c times the step, with its roundings spelled out (explicit fmaf: the same bits wherever it
// is inlined, which plain a*b - c*d, left to the compiler's contraction, does not promise)
__device__ __forceinline__ float2 rope_advance(float2 c, float2 step) {
  return make_float2(fmaf(c.x, step.x, -(c.y * step.y)), fmaf(c.x, step.y, c.y * step.x));
}
__device__ __forceinline__ float2 rope_cs_at(int pos, double rate, float2 step) {
  float2 c = rope_cs((double)(pos & ~(kRopeAnchor - 1)), rate);
  for (int k = 0; k < (pos & (kRopeAnchor - 1)); ++k) c = rope_advance(c, step);
  return c;
}

// Channel pair c of the head's [q | k | v]: kind (0 q, 1 k, 2 v) and pair index in its tensor.
struct PairIndex {
  int kind, i, width;
  __device__ PairIndex(int c, int F, int D)
      : kind(c < F / 2 ? 0 : (c < F ? 1 : 2)),
        i(c < F / 2 ? c : (c < F ? c - F / 2 : c - F)),
        width(c < F ? F : D) {}
};

// Pairs c = threadIdx.x + r * blockDim.x, r < NP, of slice bh; the head's taps arrive as
// NW4 float4 per thread (coalesced: the q, k and v weight blocks of the head side by side,
// channel ch's W taps at ch W) and reach the pairs through LDS.
template <int NP, int NW4>
struct BlockToken {
  static constexpr int WM = kMaxConvTaps;
  // (a native vector: HIP's float4 struct copies as bytes, through memory)
  typedef float f4 __attribute__((ext_vector_type(4)));
  float x0[NP], x1[NP];         // the token's raw pair
  f4 wv[NW4];                   // this thread's share of the head's taps
  float2 sv[NP][WM - 1];        // sv[j]: the carried raw pair j + 1 steps back
  float2 gv[NP], bv[NP];        // normalisation gain and bias of k and v pairs

  template <bool BF>
  __device__ void load(const BlockStepArgs& p, const void* q, const void* k, const void* v,
                       int bh, int h, int F, int D) {
    const int W = p.conv_width, CH = F + D / 2;
    const size_t srow = 2 * F + D;
#pragma unroll
    for (int r = 0; r < NP; ++r) {
      const int c = min((int)(threadIdx.x + r * blockDim.x), CH - 1);   // in bounds
      const PairIndex pi(c, F, D);
      const float2 x = load_pair_t<BF>(pi.kind == 0 ? q : (pi.kind == 1 ? k : v),
                                       (size_t)bh * pi.width + 2 * pi.i);
      x0[r] = x.x;
      x1[r] = x.y;
      if (W > 1 && p.state_in) {   // state rows oldest first: j + 1 steps back is row W-2-j
        const float* si = p.state_in + (size_t)bh * (W - 1) * srow + 2 * c;
#pragma unroll
        for (int j = 0; j < WM - 1; ++j)
          sv[r][j] = *reinterpret_cast<const float2*>(si + (size_t)max(W - 2 - j, 0) * srow);
      }
      if (p.norm_gain && pi.kind != 0) {
        const size_t e = (size_t)h * (F + D) + (pi.kind == 1 ? 2 * pi.i : F + 2 * pi.i);
        gv[r] = *reinterpret_cast<const float2*>(p.norm_gain + e);
        bv[r] = *reinterpret_cast<const float2*>(p.norm_bias + e);
      }
    }
    if (W > 0) {
      const int nq = F * W / 4, n4 = (2 * F + D) * W / 4;   // float4 of q's block, of all
#pragma unroll
      for (int r = 0; r < NW4; ++r) {
        const int j = min((int)(threadIdx.x + r * blockDim.x), n4 - 1);
        const float* src = j < nq       ? p.conv_q + (size_t)h * F * W + 4 * j
                           : j < 2 * nq ? p.conv_k + (size_t)h * F * W + 4 * (j - nq)
                                        : p.conv_v + (size_t)h * D * W + 4 * (j - 2 * nq);
        wv[r] = *reinterpret_cast<const f4*>(src);
      }
    }
  }

  // phi(q') into fq[F], the normalised phi(k') and v' into fk[F], fv[D] (LDS), the new
  // convolution state; s_w: (2F + D) kMaxConvTaps floats of LDS for the taps, red: one float
  // per wave.  Ends with a barrier.
  __device__ void finish(const BlockStepArgs& p, int bh, int F, int D, float* fq, float* fk,
                         float* fv, float* s_w, float* red) {
    const int W = p.conv_width, CH = F + D / 2;
    const size_t srow = 2 * F + D;
    if (W > 0) {
      const int n4 = (2 * F + D) * W / 4;
#pragma unroll
      for (int r = 0; r < NW4; ++r) {
        const int j = threadIdx.x + r * blockDim.x;
        if (j < n4) reinterpret_cast<f4*>(s_w)[j] = wv[r];
      }
      __syncthreads();
    }
    float y0[NP], y1[NP], sq = 0.f;
#pragma unroll
    for (int r = 0; r < NP; ++r) {
      const int c = threadIdx.x + r * blockDim.x;
      const PairIndex pi(min(c, CH - 1), F, D);
      float a0 = x0[r], a1 = x1[r];
      if (W > 0) {
        // tap tau on the token tau steps back (zero without a state); the pair's channels are
        // 2c and 2c + 1 of [q | k | v]
        const float* w0 = s_w + (size_t)(2 * min(c, CH - 1)) * W;
        const float* w1 = w0 + W;
        const bool st = W > 1 && p.state_in;
        float c0 = w0[0] * a0, c1 = w1[0] * a1;
#pragma unroll
        for (int tau = 1; tau < WM; ++tau)
          if (tau < W) {
            const float2 pv = st ? sv[r][tau - 1] : make_float2(0.f, 0.f);
            c0 += w0[tau] * pv.x;
            c1 += w1[tau] * pv.y;
          }
        if (W > 1 && p.state_out && c < CH) {   // this token is the last row, W-2
          float* so = p.state_out + (size_t)bh * (W - 1) * srow + 2 * c;
          *reinterpret_cast<float2*>(so + (size_t)(W - 2) * srow) = make_float2(x0[r], x1[r]);
#pragma unroll
          for (int tau = 1; tau < WM - 1; ++tau)   // tau steps back moves to row W-2-tau
            if (tau <= W - 2)
              *reinterpret_cast<float2*>(so + (size_t)(W - 2 - tau) * srow) =
                  st ? sv[r][tau - 1] : make_float2(0.f, 0.f);
        }
        a0 = silu_f(c0);
        a1 = silu_f(c1);
      }
      if (pi.kind != 2) {
        if (p.rope_base > 0.f) {
          const double rate = rope_rate(p.rope_base, pi.i, F);
          const float2 cs = rope_cs_at(p.pos, rate, rope_step(rate));
          const float r0 = a0 * cs.x - a1 * cs.y, r1 = a0 * cs.y + a1 * cs.x;
          a0 = r0;
          a1 = r1;
        }
        a0 = feature(a0);
        a1 = feature(a1);
      }
      y0[r] = a0;
      y1[r] = a1;
      if (pi.kind != 0 && c < CH) sq += a0 * a0 + a1 * a1;
    }
    float rn = 1.f;
    if (p.norm_gain) {
      sq = wave_sum(sq);
      if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = sq;
      __syncthreads();
      float tot = 0.f;
      for (int w = 0; w < (int)(blockDim.x >> 6); ++w) tot += red[w];
      rn = __builtin_amdgcn_rsqf(tot * (1.f / (float)(F + D)) + p.norm_eps);
    }
#pragma unroll
    for (int r = 0; r < NP; ++r) {
      const int c = threadIdx.x + r * blockDim.x;
      if (c < CH) {
        const PairIndex pi(c, F, D);
        float a0 = y0[r], a1 = y1[r];
        if (p.norm_gain && pi.kind != 0) {
          a0 = a0 * (gv[r].x * rn) + bv[r].x;
          a1 = a1 * (gv[r].y * rn) + bv[r].y;
        }
        float* dst = pi.kind == 0 ? fq : (pi.kind == 1 ? fk : fv);
        dst[2 * pi.i] = a0;
        dst[2 * pi.i + 1] = a1;
      }
    }
    __syncthreads();
  }
};

}  // namespace ia
