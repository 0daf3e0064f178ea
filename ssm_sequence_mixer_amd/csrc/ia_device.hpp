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

// Input element i with the dtype a compile-time flag (BF: bf16, else f32).  Kernels that
// take their dtype as a template parameter load without branches, so the compiler can keep
// later loads in flight behind these instead of waiting for every outstanding load.
template <bool BF>
__device__ __forceinline__ float load_t(const void* p, size_t i) {
  if constexpr (BF) return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
  else return static_cast<const float*>(p)[i];
}
// Elements i and i+1 (i even) in one load.
template <bool BF>
__device__ __forceinline__ float2 load_pair_t(const void* p, size_t i) {
  if constexpr (BF) {
    const uint32_t w = static_cast<const uint32_t*>(p)[i / 2];
    return make_float2(__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u));
  } else {
    return static_cast<const float2*>(p)[i / 2];
  }
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

// Lane-group totals of N values at once through DPP moves (VALU, no LDS round trip), the N
// chains interleaved stage by stage so their hazards overlap: swaps within quads (lane ^ 1,
// lane ^ 2) and mirrors within half-rows and rows leave every lane of a 16-lane row with the
// row's sum; row_bcast:15 then folds rows 0-1 into 1 and 2-3 into 3 (32-lane totals in lanes
// 31 and 63), row_bcast:31 rows 0-3 into 3 (the wave total in lane 63).
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ float dpp_add(float v) {
  return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROWS, 0xF,
                                                        false));
}
// Inclusive prefix sum over the wave's 64 lanes through DPP moves: row_shr 1, 2, 4, 8 (a lane
// whose source lies before its 16-lane row adds zero) give prefix sums within each row;
// row_bcast:15 then adds row 0's total to row 1 and row 2's to row 3, and row_bcast:31 the
// total of rows 0-1 to rows 2 and 3.
__device__ __forceinline__ float wave_scan_incl(float v) {
  v = dpp_add<0x111>(v);        // row_shr:1
  v = dpp_add<0x112>(v);        // row_shr:2
  v = dpp_add<0x114>(v);        // row_shr:4
  v = dpp_add<0x118>(v);        // row_shr:8
  v = dpp_add<0x142, 0xA>(v);   // row_bcast:15 into rows 1 and 3
  v = dpp_add<0x143, 0xC>(v);   // row_bcast:31 into rows 2 and 3
  return v;
}

// Sums over aligned groups of W lanes (W = 16, 32 or 64) of N values at once; the group's last
// lane ends with each total (W = 16: every lane of the 16-lane row).
template <int W, int N>
__device__ __forceinline__ void row_totals(float (&v)[N]) {
  static_assert(W == 16 || W == 32 || W == 64, "16, 32 or 64 lanes");
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = dpp_add<0xB1>(v[i]);         // quad_perm [1,0,3,2]
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = dpp_add<0x4E>(v[i]);         // quad_perm [2,3,0,1]
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = dpp_add<0x141>(v[i]);        // row_half_mirror
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = dpp_add<0x140>(v[i]);        // row_mirror
  if constexpr (W >= 32) {
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = dpp_add<0x142, 0xA>(v[i]);   // row_bcast:15
  }
  if constexpr (W == 64) {
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = dpp_add<0x143, 0xC>(v[i]);   // row_bcast:31
  }
}

// Totals over the 64 lanes of a wave of 16 values v[0..15], scattered over the lanes: lane l
// ends with the totals of values T and T + 1 in z0 and z1, T = 2 b + 4 (r & 1) + 8 (r >> 1),
// r = l / 16 and b = (l / 8) & 1 (all eight lanes of a group hold the same two).  The first
// two rounds pair lane halves and then rows with the cross-row swaps (each instruction serves
// two values), the third pairs lanes l, l ^ 8 by a row rotation, the last three sum within
// groups of eight by DPP: 36 instructions where a full reduction of every value takes 96.
__device__ __forceinline__ void scatter_totals16(const float (&v)[16], float& z0, float& z1) {
  float u[8], w[4];
#pragma unroll
  for (int j = 0; j < 8; ++j) {   // u[j]: lanes 0-31 value j, 32-63 value j + 8
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[j]),
                                                    __float_as_uint(v[j + 8]), false, false);
    u[j] = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {   // w[j], row r: value j + 4 (r & 1) + 8 (r >> 1)
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(u[j]),
                                                    __float_as_uint(u[j + 4]), false, false);
    w[j] = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  }
  const bool hi = threadIdx.x & 8;
  float z[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {   // lanes l, l ^ 8: each keeps one value and sends the other
    const float keep = hi ? w[j + 2] : w[j], send = hi ? w[j] : w[j + 2];
    z[j] = keep + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(send), 0x128,
                                                             0xF, 0xF, false));   // row_ror:8
    z[j] = dpp_add<0xB1>(z[j]);    // quad_perm [1,0,3,2]
    z[j] = dpp_add<0x4E>(z[j]);    // quad_perm [2,3,0,1]
    z[j] = dpp_add<0x141>(z[j]);   // row_half_mirror
  }
  z0 = z[0];
  z1 = z[1];
}

}  // namespace ia
