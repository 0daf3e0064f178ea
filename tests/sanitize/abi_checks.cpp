// Host-side validation paths of libia under AddressSanitizer and UndefinedBehaviorSanitizer.
// The library's sources are compiled host-only (no device code): every call below fails
// validation before anything would be enqueued, so fake device addresses are never touched.
// Exit status 0 when every call returns its expected status.
#include <cstdio>
#include <cstdint>
#include <vector>

#include "ia.h"

namespace {

void* addr(int i, std::uintptr_t off = 0) {
  return reinterpret_cast<void*>((std::uintptr_t(1) << 32) + std::uintptr_t(i) * (1u << 28) + off);
}

ia_desc desc(int B = 2, int H = 3, int N = 70, int F = 32, int Dv = 32, int M = 16,
             int in_dtype = IA_BF16) {
  ia_desc d{};
  d.B = B; d.H = H; d.N = N; d.F = F; d.Dv = Dv; d.M = M;
  d.in_dtype = in_dtype; d.out_dtype = IA_F32; d.den_clamp = 1e-6f; d.flags = 0; d.chunk = 0;
  return d;
}

int failures = 0;
void expect(const char* what, int got, int want) {
  if (got != want) {
    std::printf("FAIL %s: status %d, expected %d\n", what, got, want);
    ++failures;
  }
}

}  // namespace

int main() {
  ia_state st{addr(10), addr(11), addr(12)};
  ia_state st_alias{addr(10), addr(10, 256), addr(12)};
  const size_t big = size_t(1) << 40;
  // descriptor fields
  {
    ia_desc d = desc(0);
    expect("B = 0", ia_prefill_fwd(&d, addr(0), addr(1), addr(2), addr(3), addr(4), &st, addr(5),
                                   addr(6), big, nullptr), IA_ERR_SHAPE);
    d = desc(2, 3, 70, 24);
    expect("F = 24", ia_decode_step(&d, addr(0), addr(1), addr(2), addr(3), addr(4), &st,
                                    addr(5), nullptr), IA_ERR_UNSUPPORTED);
    d = desc(); d.in_dtype = 7;
    expect("dtype", ia_state_init(&d, &st, nullptr), IA_ERR_DTYPE);
    d = desc(); d.den_clamp = -1.f;
    expect("clamp", ia_prefill_workspace_bytes(&d) == 0 ? IA_ERR_DOMAIN : IA_OK, IA_ERR_DOMAIN);
    d = desc(); d.flags = 32;
    expect("flags", ia_prefill_fwd(&d, addr(0), addr(1), addr(2), addr(3), addr(4), &st,
                                   addr(5), addr(6), big, nullptr), IA_ERR_UNSUPPORTED);
    expect("null desc", ia_prefill_fwd(nullptr, addr(0), addr(1), addr(2), addr(3), addr(4), &st,
                                       addr(5), addr(6), big, nullptr), IA_ERR_NULL);
  }
  ia_desc d = desc();
  expect("null q", ia_prefill_fwd(&d, nullptr, addr(1), addr(2), addr(3), addr(4), &st, addr(5),
                                  addr(6), big, nullptr), IA_ERR_NULL);
  expect("misaligned v", ia_prefill_fwd(&d, addr(0), addr(1), addr(2, 8), addr(3), addr(4), &st,
                                        addr(5), addr(6), big, nullptr), IA_ERR_ALIGN);
  expect("o aliases k", ia_prefill_fwd(&d, addr(0), addr(1), addr(2), addr(3), addr(4), &st,
                                       addr(1, 16), addr(6), big, nullptr), IA_ERR_ALIAS);
  expect("state aliases", ia_prefill_fwd(&d, addr(0), addr(1), addr(2), addr(3), addr(4),
                                         &st_alias, addr(5), addr(6), big, nullptr),
         IA_ERR_ALIAS);
  expect("workspace missing", ia_prefill_fwd(&d, addr(0), addr(1), addr(2), addr(3), addr(4),
                                             nullptr, addr(5), nullptr, 0, nullptr),
         IA_ERR_WORKSPACE);
  {
    ia_desc u = desc(2, 3, 70, 32, 16);   // bf16 without a chunk kernel
    expect("bf16 F != Dv", ia_prefill_fwd(&u, addr(0), addr(1), addr(2), addr(3), addr(4), &st,
                                          addr(5), addr(6), big, nullptr), IA_ERR_UNSUPPORTED);
  }
  {
    const long long s[3][3] = {{70 * 3 * 32, 3 * 32, 36}, {70 * 3 * 32, 3 * 32, 36},
                               {70 * 3 * 32, 3 * 32, 32}};
    expect("strided misaligned", ia_prefill_fwd_strided(&d, addr(0), addr(1), addr(2), s, addr(3),
                                                        addr(4), &st, addr(5), addr(6), big,
                                                        nullptr), IA_ERR_ALIGN);
  }
  // lambda check on host memory
  {
    ia_desc l = desc(2, 2, 70, 32, 32, 16);
    std::vector<float> lam(2 * 2 * 16, 0.f);
    for (int i = 0; i < 2 * 16; ++i) lam[2 * i] = 0.99f;
    int routed = -1;
    expect("lambda ok", ia_check_lambda(&l, lam.data(), &routed), IA_OK);
    expect("no routed heads", routed, 0);
    lam[2 * 5] = -1.f;
    expect("lambda -1 in domain", ia_check_lambda(&l, lam.data(), &routed), IA_OK);
    expect("one routed head", routed, 1);
    lam[2 * 20] = 1.5f;
    expect("lambda 1.5", ia_check_lambda(&l, lam.data(), nullptr), IA_ERR_DOMAIN);
  }
  // backward, readout, gated
  {
    const size_t need = ia_prefill_bwd_workspace_bytes(&d);
    expect("bwd small workspace",
           ia_prefill_bwd(&d, addr(0), addr(1), addr(2), addr(3), addr(4), nullptr, addr(5),
                          addr(6), addr(7), addr(8), addr(9), addr(13), nullptr, addr(14),
                          need - 1, nullptr), IA_ERR_WORKSPACE);
    // both backward kernel choices, and the chunked kernels on a shape they do not serve
    ia_desc db = d;
    db.flags = IA_FLAG_SEQUENTIAL_BWD | IA_FLAG_CHUNKED_BWD;
    expect("bwd both kernel flags",
           ia_prefill_bwd(&db, addr(0), addr(1), addr(2), addr(3), addr(4), nullptr, addr(5),
                          addr(6), addr(7), addr(8), addr(9), addr(13), nullptr, addr(14), big,
                          nullptr), IA_ERR_UNSUPPORTED);
    db.flags = IA_FLAG_CHUNKED_BWD;
    db.Dv = 48;
    expect("bwd chunked on Dv 48",
           ia_prefill_bwd(&db, addr(0), addr(1), addr(2), addr(3), addr(4), nullptr, addr(5),
                          addr(6), addr(7), addr(8), addr(9), addr(13), nullptr, addr(14), big,
                          nullptr), IA_ERR_UNSUPPORTED);
    expect("bwd chunked workspace bytes", ia_prefill_bwd_workspace_bytes(&db) == 0 ? 0 : 1, 0);
    expect("readout null", ia_prefill_fwd_readout(&d, addr(0), addr(1), addr(2), addr(3),
                                                  addr(4), nullptr, &st, addr(5), addr(6), big,
                                                  nullptr), IA_ERR_NULL);
    expect("gated null", ia_prefill_fwd_gated(&d, addr(0), addr(1), addr(2), nullptr, addr(21),
                                              addr(3), addr(4), &st, addr(5), addr(6), big,
                                              nullptr), IA_ERR_NULL);
    const size_t gneed = ia_prefill_gated_workspace_bytes(&d);   // the chunked plan's
    expect("gated small workspace",
           ia_prefill_fwd_gated(&d, addr(0), addr(1), addr(2), addr(20), addr(21), addr(3),
                                addr(4), &st, addr(5), addr(6), gneed - 1, nullptr),
           IA_ERR_WORKSPACE);
    expect("gated decode alias", ia_decode_step_gated(&d, addr(0), addr(1), addr(2), addr(20),
                                                      addr(21), addr(3), addr(4), &st,
                                                      addr(21, 16), nullptr), IA_ERR_ALIAS);
  }
  // the block's edges
  {
    ia_block_params p{};
    p.conv_width = 4;
    p.conv_q = addr(20); p.conv_k = addr(21); p.conv_v = addr(22);
    p.rope_base = 1e4f; p.pos0 = 0;
    p.norm_gain = addr(23); p.norm_bias = addr(24); p.norm_eps = 1e-6f;
    expect("prologue taps", [&] { ia_block_params b = p; b.conv_width = 9;
      return ia_block_prologue(&d, &b, addr(0), addr(1), addr(2), nullptr, nullptr, addr(5),
                               addr(6), addr(7), nullptr); }(), IA_ERR_UNSUPPORTED);
    expect("prologue positions", [&] { ia_block_params b = p; b.pos0 = 2147483647 - 68;
      return ia_block_prologue(&d, &b, addr(0), addr(1), addr(2), nullptr, nullptr, addr(5),
                               addr(6), addr(7), nullptr); }(), IA_ERR_DOMAIN);
    expect("prologue state alias", ia_block_prologue(&d, &p, addr(0), addr(1), addr(2), addr(30),
                                                     addr(30), addr(5), addr(6), addr(7),
                                                     nullptr), IA_ERR_ALIAS);
    expect("gate alias", ia_block_gate(&d, addr(0), addr(1), addr(1, 64), nullptr),
           IA_ERR_ALIAS);
    expect("block step null gain", [&] { ia_block_params b = p; b.norm_gain = nullptr;
      return ia_block_decode_step(&d, &b, addr(0), addr(1), addr(2), nullptr, nullptr, nullptr,
                                  addr(3), addr(4), &st, addr(5), nullptr); }(), IA_ERR_NULL);
    expect("block step alias", ia_block_decode_step(&d, &p, addr(0), addr(1), addr(2), addr(30),
                                                    addr(5), nullptr, addr(3), addr(4), &st,
                                                    addr(5), nullptr), IA_ERR_ALIAS);
  }
  for (int s = 0; s <= IA_ERR_WORKSPACE; ++s)
    if (!ia_status_string(static_cast<ia_status>(s))) ++failures;
  std::printf("%s (%d failure(s))\n", failures ? "FAILED" : "ok", failures);
  return failures ? 1 : 0;
}
