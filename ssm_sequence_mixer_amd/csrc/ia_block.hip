// ia_block.hip — the IA block's edges around the layer: the input prologue (short causal
// convolutions with SiLU on q, k, v; rotary position embedding on q and k; the feature map;
// the RMS normalisation with a per-head bias of the SSM input z = [phi(k), v]) and the output
// gate.  ("Interdomain Attention: Beyond Token-Level Key-Value Memory": summary page §5.3 and
// §B.1 for the query/key and value convolutions, §A.1 for RoPE in the language models, §3.3
// for the output gate; AI Radio episode page, "Implementation Details", for the normalised
// SSM input.  The pages give no formulas; the readings are those of include/ia.h.)
//
// The prologue writes the layer's inputs in the form the layer takes with
// IA_FLAG_IDENTITY_FEATURES: phi(q'), the normalised phi(k') and v'.  It is a streaming pass
// (each input read once, each output written once), one workgroup per (block of 64 tokens,
// b, h), one thread per pair of adjacent channels: the q pairs, then the k pairs, then the
// v pairs of the head, so a RoPE pair (2i, 2i+1) sits in one thread and the convolution keeps
// its window of the W-1 previous raw tokens in that thread's registers.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ia_block_step.hpp"
#include "ia_device.hpp"
#include "ia_kernels.hpp"

namespace ia {

namespace {

constexpr int kBlockTokens = 64;   // tokens per workgroup
constexpr int kNormGroup = 16;     // tokens whose normalisation sums are reduced together

// A channel pair: bf16 as one packed word, fp32 as two words.
template <bool BF>
struct PairIO;
template <>
struct PairIO<true> {
  static constexpr int kBytes = 4;
  __device__ static float2 load(const char* p) {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(p);
    return make_float2(__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u));
  }
  __device__ static void store(char* p, float a, float b) {   // round to nearest even
    typedef float f2v __attribute__((ext_vector_type(2)));
    typedef __bf16 b2v __attribute__((ext_vector_type(2)));
    *reinterpret_cast<uint32_t*>(p) =
        __builtin_bit_cast(uint32_t, __builtin_convertvector((f2v){a, b}, b2v));
  }
};
template <>
struct PairIO<false> {
  static constexpr int kBytes = 8;
  __device__ static float2 load(const char* p) { return *reinterpret_cast<const float2*>(p); }
  __device__ static void store(char* p, float a, float b) {
    *reinterpret_cast<float2*>(p) = make_float2(a, b);
  }
};

// Thread c of a (b, h) token block: channel pair c of [q | k | v] (channels 2c, 2c+1 of the
// head's 2F + Dv); W taps of convolution (0: none).  Window x[tau] = raw input tau tokens
// back.  Every load of a group of tokens is unconditional (token indices clamped into the
// call) so that the group's loads are in flight together; what a clamped load brings is
// neither stored nor summed.
template <bool BF, int W>
__global__ void __launch_bounds__(512)
block_prologue_kernel(const BlockArgs a) {
  using IO = PairIO<BF>;
  constexpr int WX = W > 1 ? W - 1 : 1;   // window entries before the current token
  const int F = a.F, D = a.D, H = a.H, N = a.N;
  const int CH = F + D / 2;   // channel pairs: F/2 of q, F/2 of k, D/2 of v
  const int bh = blockIdx.y, b = bh / H, h = bh % H;
  const int n0 = blockIdx.x * kBlockTokens, n1 = min(N, n0 + kBlockTokens);
  const bool active = (int)threadIdx.x < CH;
  const int c = active ? (int)threadIdx.x : F;   // threads past the pairs shadow v pair 0
  const int kind = c < F / 2 ? 0 : (c < F ? 1 : 2);          // q, k, v
  const int i = kind == 0 ? c : (kind == 1 ? c - F / 2 : c - F);   // pair index in its tensor
  const int width = kind == 2 ? D : F;
  // element (b, 0, h, 2i) of the tensor, and the bytes from one token to the next
  const size_t e0 = ((size_t)b * N * H + h) * width + 2 * i;
  const char* sp = static_cast<const char*>(kind == 0 ? a.q : (kind == 1 ? a.k : a.v)) +
                   e0 * (IO::kBytes / 2);
  char* dp = static_cast<char*>(kind == 0 ? a.fq : (kind == 1 ? a.fk : a.vo)) +
             e0 * (IO::kBytes / 2);
  const uint32_t tsb = (uint32_t)H * width * (IO::kBytes / 2);   // < 2^24 (host check)
  auto in_at = [&](int t) { return IO::load(sp + (size_t)t * tsb); };
  const size_t srow = 2 * F + D;   // floats per state row
  // this thread's channels in the state before the call (rows oldest first)
  const float* sin_ =
      a.state_in && W > 1 ? a.state_in + (size_t)bh * (W - 1) * srow + 2 * c : nullptr;

  float w0[W > 0 ? W : 1], w1[W > 0 ? W : 1], x0[WX], x1[WX];
#pragma unroll
  for (int tau = 0; tau < WX; ++tau) x0[tau] = x1[tau] = 0.f;
  if constexpr (W > 0) {
    const float* wt = kind == 0 ? a.conv_q : (kind == 1 ? a.conv_k : a.conv_v);
    const float* wr = wt + ((size_t)h * width + 2 * i) * W;
#pragma unroll
    for (int tau = 0; tau < W; ++tau) {
      w0[tau] = wr[tau];
      w1[tau] = wr[W + tau];
    }
  }
  // the window before token n0 (x[j] = raw token n0 - 1 - j): raw tokens of this call
  // (n0 >= 64 > W), or the state before it
  if constexpr (W > 1) {
    if (n0 > 0) {
      float2 xv[WX];
#pragma unroll
      for (int tau = 0; tau < WX; ++tau) xv[tau] = in_at(n0 - 1 - tau);
#pragma unroll
      for (int tau = 0; tau < WX; ++tau) {
        x0[tau] = xv[tau].x;
        x1[tau] = xv[tau].y;
      }
    } else if (sin_) {
#pragma unroll
      for (int tau = 0; tau < WX; ++tau) {   // token -1 - tau is state row W - 2 - tau
        const float* s = sin_ + (size_t)(W - 2 - tau) * srow;
        x0[tau] = s[0];
        x1[tau] = s[1];
      }
    }
  }
  float g0 = 1.f, g1 = 1.f, c0 = 0.f, c1 = 0.f;
  const bool norm = a.norm_gain != nullptr;
  if (norm && kind != 0) {
    const int e = kind == 1 ? 2 * i : F + 2 * i;   // entry of z = [phi(k), v]
    const float* gp = a.norm_gain + (size_t)h * (F + D) + e;
    const float* bp = a.norm_bias + (size_t)h * (F + D) + e;
    g0 = gp[0];
    g1 = gp[1];
    c0 = bp[0];
    c1 = bp[1];
  }
  // RoPE: the pair turns by base^(-2i/F) / (2 pi) turns per position, its angles stepped from
  // anchors (rope_cs_at), so that a call's split into pieces does not change them
  const bool rope = a.rope_base > 0.f && kind != 2;
  const double rev = rope ? rope_rate(a.rope_base, i, F) : 0.0;
  const float2 step = rope ? rope_step(rev) : make_float2(1.f, 0.f);
  const float inv_e = 1.f / (float)(F + D);
  const bool summed = active && kind != 0;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwave = (blockDim.x + 63) >> 6;
  const bool wave_sums = (wave + 1) * 64 > F / 2;   // the wave holds k or v pairs

  __shared__ __align__(16) float s_red[2][8][kNormGroup];   // per-wave sums, groups in turn
  int parity = 0;
  for (int t0 = n0; t0 < n1; t0 += kNormGroup) {
    const int jmax = n1 - 1 - t0;   // tokens past it are clamped to it
    const char* gp = sp + (size_t)t0 * tsb;
    float2 xin[kNormGroup];
#pragma unroll
    for (int j = 0; j < kNormGroup; ++j)
      xin[j] = IO::load(gp + (uint32_t)__umul24((uint32_t)min(j, jmax), tsb));
    // (cos, sin) of token t0's angle, and of the next anchor, where the group may cross one
    const int p0 = a.pos0 + t0;   // < 2^31
    float2 rc = make_float2(1.f, 0.f), rc_next = rc;
    if (rope) {
      rc = rope_cs_at(p0, rev, step);
      rc_next = rope_cs((double)(p0 | (kRopeAnchor - 1)) + 1.0, rev);
    }
    float y0[kNormGroup], y1[kNormGroup], sq[kNormGroup];
#pragma unroll
    for (int j = 0; j < kNormGroup; ++j) {
      float a0 = xin[j].x, a1 = xin[j].y;
      if constexpr (W > 0) {
        float s0 = w0[0] * a0, s1 = w1[0] * a1;
#pragma unroll
        for (int tau = 1; tau < W; ++tau) {
          s0 += w0[tau] * x0[tau - 1];
          s1 += w1[tau] * x1[tau - 1];
        }
        if constexpr (W > 1) {
#pragma unroll
          for (int tau = WX - 1; tau > 0; --tau) {
            x0[tau] = x0[tau - 1];
            x1[tau] = x1[tau - 1];
          }
          x0[0] = a0;
          x1[0] = a1;
        }
        a0 = silu_f(s0);
        a1 = silu_f(s1);
      }
      if (kind != 2) {
        if (rope) {
          const float r0 = a0 * rc.x - a1 * rc.y, r1 = a0 * rc.y + a1 * rc.x;
          a0 = r0;
          a1 = r1;
          // the next position's angle: an anchor's own, else one more step
          const bool anchor = (((uint32_t)p0 + j + 1) & (kRopeAnchor - 1)) == 0;
          rc = anchor ? rc_next : rope_advance(rc, step);
        }
        a0 = feature(a0);
        a1 = feature(a1);
      }
      y0[j] = a0;
      y1[j] = a1;
      sq[j] = summed && j <= jmax ? a0 * a0 + a1 * a1 : 0.f;
    }
    if (norm) {
      // the wave's totals of the 16 tokens, two per group of eight lanes
      float z0 = 0.f, z1 = 0.f;
      if (wave_sums) scatter_totals16(sq, z0, z1);
      if ((lane & 7) == 0) {
        const int T = 2 * ((lane >> 3) & 1) + 4 * ((lane >> 4) & 1) + 8 * (lane >> 5);
        *reinterpret_cast<float2*>(&s_red[parity][wave][T]) = make_float2(z0, z1);
      }
      __syncthreads();   // (the next group writes the other half of s_red)
      // lane j of every wave: token j's total and 1 / rms; then read out lane by lane
      float rj = 0.f;
      if (lane < kNormGroup) {
        float s = 0.f;
        for (int w2 = 0; w2 < nwave; ++w2) s += s_red[parity][w2][lane];
        rj = __builtin_amdgcn_rsqf(s * inv_e + a.norm_eps);
      }
      if (kind != 0) {
#pragma unroll
        for (int j = 0; j < kNormGroup; ++j) {
          const float r = __builtin_bit_cast(
              float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, rj), j));
          y0[j] = y0[j] * (g0 * r) + c0;
          y1[j] = y1[j] * (g1 * r) + c1;
        }
      }
      parity ^= 1;
    }
    if (active) {
      char* gd = dp + (size_t)t0 * tsb;
#pragma unroll
      for (int j = 0; j < kNormGroup; ++j)
        if (j <= jmax) IO::store(gd + (uint32_t)__umul24((uint32_t)j, tsb), y0[j], y1[j]);
    }
  }

  // the new state: the last W-1 raw tokens (oldest first), written by the blocks that hold the
  // last token; tokens before this call come from the state before it
  if constexpr (W > 1) {
    if (active && a.state_out && n1 == N) {
      float* so = a.state_out + (size_t)bh * (W - 1) * srow + 2 * c;
      float xv0[WX], xv1[WX];
      if (N >= W - 1) {
#pragma unroll
        for (int tau = 0; tau < WX; ++tau) {
          const float2 xv = in_at(N - 1 - tau);
          xv0[tau] = xv.x;
          xv1[tau] = xv.y;
        }
      } else {
#pragma unroll
        for (int tau = 0; tau < WX; ++tau) {
          const int t = N - 1 - tau;
          float2 xv = make_float2(0.f, 0.f);
          if (t >= 0) {
            xv = in_at(t);
          } else if (sin_) {
            const float* s = sin_ + (size_t)(W - 1 + t) * srow;   // row >= 0: t >= 1 - W
            xv = make_float2(s[0], s[1]);
          }
          xv0[tau] = xv.x;
          xv1[tau] = xv.y;
        }
      }
#pragma unroll
      for (int tau = 0; tau < WX; ++tau) {
        const size_t row = (size_t)(W - 2 - tau) * srow;
        so[row] = xv0[tau];
        so[row + 1] = xv1[tau];
      }
    }
  }
}

// out = o * SiLU(g), elementwise (out may be o).
template <bool BF>
__global__ void __launch_bounds__(256)
block_gate_kernel(const void* o, const void* __restrict__ g, void* out, size_t n) {
  for (size_t p = 2 * (blockIdx.x * (size_t)blockDim.x + threadIdx.x); p < n;
       p += 2 * (size_t)gridDim.x * blockDim.x) {
    using IO = PairIO<BF>;
    const size_t off = p * (IO::kBytes / 2);
    const float2 ov = IO::load(static_cast<const char*>(o) + off);
    const float2 gv = IO::load(static_cast<const char*>(g) + off);
    IO::store(static_cast<char*>(out) + off, ov.x * silu_f(gv.x), ov.y * silu_f(gv.y));
  }
}

}  // namespace

template <bool BF>
void launch_prologue_w(const BlockArgs& a, dim3 grid, dim3 block, hipStream_t st) {
  switch (a.conv_width) {
    case 0: hipLaunchKernelGGL((block_prologue_kernel<BF, 0>), grid, block, 0, st, a); break;
    case 1: hipLaunchKernelGGL((block_prologue_kernel<BF, 1>), grid, block, 0, st, a); break;
    case 2: hipLaunchKernelGGL((block_prologue_kernel<BF, 2>), grid, block, 0, st, a); break;
    case 3: hipLaunchKernelGGL((block_prologue_kernel<BF, 3>), grid, block, 0, st, a); break;
    case 4: hipLaunchKernelGGL((block_prologue_kernel<BF, 4>), grid, block, 0, st, a); break;
    case 5: hipLaunchKernelGGL((block_prologue_kernel<BF, 5>), grid, block, 0, st, a); break;
    case 6: hipLaunchKernelGGL((block_prologue_kernel<BF, 6>), grid, block, 0, st, a); break;
    case 7: hipLaunchKernelGGL((block_prologue_kernel<BF, 7>), grid, block, 0, st, a); break;
    default: hipLaunchKernelGGL((block_prologue_kernel<BF, 8>), grid, block, 0, st, a); break;
  }
}

hipError_t launch_block_prologue(const BlockArgs& a, hipStream_t st) {
  static_assert(kMaxConvTaps == 8, "one instantiation per tap count");
  const int CH = a.F + a.D / 2;
  const int threads = (CH + 63) / 64 * 64;   // at most 384 (F, Dv <= 256)
  const long row_bytes = (long)a.H * (a.F > a.D ? a.F : a.D) * (a.bf16 ? 2 : 4);
  if (threads > 512 || a.conv_width < 0 || a.conv_width > kMaxConvTaps ||
      row_bytes >= (1L << 24))   // token strides are 24-bit products in the kernel
    return hipErrorInvalidValue;
  if (a.N == 0 || a.B == 0) return hipSuccess;
  const dim3 grid((a.N + kBlockTokens - 1) / kBlockTokens, a.B * a.H);
  (void)hipGetLastError();
  prof_begin(st);
  if (a.bf16)
    launch_prologue_w<true>(a, grid, dim3(threads), st);
  else
    launch_prologue_w<false>(a, grid, dim3(threads), st);
  prof_end(st, kKindBlock);
  return hipGetLastError();
}

hipError_t launch_block_gate(const void* o, const void* g, void* out, size_t n, int bf16,
                             hipStream_t st) {
  if (n == 0) return hipSuccess;
  const size_t pairs = n / 2;
  const unsigned grid = static_cast<unsigned>(pairs / 256 + 1 < 8192 ? pairs / 256 + 1 : 8192);
  (void)hipGetLastError();
  prof_begin(st);
  if (bf16)
    hipLaunchKernelGGL(block_gate_kernel<true>, dim3(grid), dim3(256), 0, st, o, g, out, n);
  else
    hipLaunchKernelGGL(block_gate_kernel<false>, dim3(grid), dim3(256), 0, st, o, g, out, n);
  prof_end(st, kKindBlock);
  return hipGetLastError();
}

}  // namespace ia
