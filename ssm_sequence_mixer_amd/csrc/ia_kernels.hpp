// ia_kernels.hpp — internal launch interface between the C ABI (ia_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace ia {

constexpr int kMaxDim = 256;    // largest F and Dv
constexpr int kMaxModes = 128;  // largest M

struct DecodeArgs {
  const void *q, *k, *v;
  const float2 *lam, *beta;
  float2 *U, *G, *E;
  void* o;
  int B, H, F, D, M;
  int in_bf16, out_bf16;
  float clamp;
};

struct ScanArgs {
  const void *q, *k, *v;
  const float2 *lam, *beta;
  float2 *U, *G, *E;
  void* o;
  const float* acc_in;
  int B, H, N, F, D, M;
  int in_bf16, out_bf16;
  float clamp;
  int reverse;
};

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t st);
hipError_t launch_decode_step(const DecodeArgs& a, hipStream_t st);
hipError_t launch_scan_prefill(const ScanArgs& a, hipStream_t st);

}  // namespace ia
