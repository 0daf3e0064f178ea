// ia_device.hpp — device-side helpers shared by the IA kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ia_kernels.hpp"

namespace ia {

// ---------------------------------------------------------------- scalar conversions

// bf16 bits -> float (exact).
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// float -> bf16 bits, round to nearest even; NaN stays NaN (quiet bit forced).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Load element i of a q/k/v-like array whose dtype is a runtime flag (0 = f32, 1 = bf16).
__device__ __forceinline__ float load_in(const void* p, size_t i, int bf16) {
  return bf16 ? bf16_to_f32(static_cast<const uint16_t*>(p)[i])
              : static_cast<const float*>(p)[i];
}

__device__ __forceinline__ void store_out(void* p, size_t i, float x, int bf16) {
  if (bf16)
    static_cast<uint16_t*>(p)[i] = f32_to_bf16(x);
  else
    static_cast<float*>(p)[i] = x;
}

// Feature map of the layer: elu(x) + 1 (x + 1 above zero, exp(x) at or below).
__device__ __forceinline__ float feature(float x) { return x > 0.f ? x + 1.f : __expf(x); }

// The feature map as x > t ? x + c : exp(x), with (t, c) uniform: (0, 1) is elu(x)+1 and
// (-inf, 0) the identity (kOptIdentity), the same instructions for both.
__device__ __forceinline__ float feature_tc(float x, float t, float c) {
  return x > t ? x + c : __expf(x);
}
__device__ __forceinline__ float feature_t(int opt) { return (opt & kOptIdentity) ? -INFINITY : 0.f; }
__device__ __forceinline__ float feature_c(int opt) { return (opt & kOptIdentity) ? 0.f : 1.f; }

// Feature map, or none with kOptIdentity (ia_kernels.hpp).
__device__ __forceinline__ float feat(float x, int opt) {
  return (opt & kOptIdentity) ? x : feature(x);
}

// Denominator clamp: one-sided, NaN passes through unchanged.
__device__ __forceinline__ float clamp_den(float d, float c) { return d < c ? c : d; }
// Output of a readout: num / max(den, clamp), or num with kOptNoDen.
__device__ __forceinline__ float readout(float num, float den, float clamp, int opt) {
  return (opt & kOptNoDen) ? num : num / clamp_den(den, clamp);
}

// ---------------------------------------------------------------- complex (float2)

__device__ __forceinline__ float2 cmul(float2 a, float2 b) {
  return make_float2(a.x * b.x - a.y * b.y, a.x * b.y + a.y * b.x);
}

// a*x + b (complex a, b; complex x)
__device__ __forceinline__ float2 cfma(float2 a, float2 x, float2 b) {
  return make_float2(a.x * x.x - a.y * x.y + b.x, a.x * x.y + a.y * x.x + b.y);
}

// ---------------------------------------------------------------- wave reductions (wave64)

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

}  // namespace ia
