// ia_api.cpp — the C ABI of libia.so: host-side validation, workspace layout and dispatch.
// Every check runs before anything is enqueued; no call synchronises, allocates or prints.
#include "ia.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "ia_kernels.hpp"

namespace {

size_t esize(int dt) { return dt == IA_BF16 ? 2 : 4; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

// The bytes [p, p + bytes) of an argument; a NULL argument covers nothing.
Range rng(const void* p, size_t bytes) {
  uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return {a, p ? a + bytes : a};
}

bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi && a.lo != a.hi && b.lo != b.hi; }

// Checks shared by every call on the descriptor's sizes and codes.
ia_status check_desc(const ia_desc* d, bool need_n) {
  if (!d) return IA_ERR_NULL;
  if (d->B <= 0 || d->H <= 0 || d->F <= 0 || d->Dv <= 0 || d->M <= 0) return IA_ERR_SHAPE;
  if (need_n && d->N <= 0) return IA_ERR_SHAPE;
  if (d->F % 16 || d->Dv % 16 || d->M % 16) return IA_ERR_UNSUPPORTED;
  if (d->F > ia::kMaxDim || d->Dv > ia::kMaxDim || d->M > ia::kMaxModes)
    return IA_ERR_UNSUPPORTED;
  if ((d->in_dtype != IA_F32 && d->in_dtype != IA_BF16) ||
      (d->out_dtype != IA_F32 && d->out_dtype != IA_BF16))
    return IA_ERR_DTYPE;
  if (!(std::isfinite(d->den_clamp) && d->den_clamp > 0.f)) return IA_ERR_DOMAIN;
  if (d->flags & ~(IA_FLAG_BIDIR | IA_FLAG_NO_DEN | IA_FLAG_IDENTITY_FEATURES |
                   IA_FLAG_SEQUENTIAL_BWD | IA_FLAG_CHUNKED_BWD))
    return IA_ERR_UNSUPPORTED;
  if (d->chunk != 0 && d->chunk != 32 && d->chunk != 64) return IA_ERR_UNSUPPORTED;
  // Index arithmetic in the kernels is 64-bit for element offsets; keep grid sizes sane.
  const double slices = double(d->B) * d->H;
  if (slices > 1e7 || (need_n && double(d->N) * slices * (d->F + d->Dv) > 9e18))
    return IA_ERR_SHAPE;
  return IA_OK;
}

size_t state_u_bytes(const ia_desc* d) { return size_t(d->B) * d->H * d->M * d->F * 8; }
size_t state_g_bytes(const ia_desc* d) { return size_t(d->B) * d->H * d->M * d->Dv * 8; }
size_t state_e_bytes(const ia_desc* d) { return size_t(d->B) * d->H * d->M * 8; }
size_t state_bytes(const ia_desc* d) {
  return state_u_bytes(d) + state_g_bytes(d) + state_e_bytes(d);
}

size_t round_up(size_t x) { return (x + 255) & ~size_t(255); }

ia_status check_state(const ia_desc* d, const ia_state* st) {
  if (!st || !st->U || !st->Gamma || !st->eta) return IA_ERR_NULL;
  if (!aligned16(st->U) || !aligned16(st->Gamma) || !aligned16(st->eta)) return IA_ERR_ALIGN;
  Range u = rng(st->U, state_u_bytes(d)), g = rng(st->Gamma, state_g_bytes(d)),
        e = rng(st->eta, state_e_bytes(d));
  if (overlap(u, g) || overlap(u, e) || overlap(g, e)) return IA_ERR_ALIAS;
  return IA_OK;
}

// Workspace of the token-sequential prefill path: a state when the caller passes none (or the
// call is bidirectional), and, for the register-resident kernel, the slots and decay products
// of its sequence segments.  Segments give every compute unit one slice's workgroup
// (B*H*segments up to the CU count), at least kMinScanSegment tokens each; their count is the
// largest whose bytes fit `avail` (the workspace queries pass no limit, a call its ws_bytes),
// so a smaller workspace runs fewer segments, down to one.
constexpr int kMinScanSegment = 64;
struct ScanWorkspace {
  size_t state_off, bytes;
  int n_seg, seg_len;
  size_t slots_off, dec_off;
};

ScanWorkspace scan_workspace(const ia_desc* d, bool have_state, size_t avail = SIZE_MAX) {
  ScanWorkspace w{0, 0, 1, d->N, 0, 0};
  const bool bidir = d->flags & IA_FLAG_BIDIR;
  if (!have_state || bidir) {
    w.state_off = 0;
    w.bytes = round_up(state_bytes(d));
  }
  if (!ia::scan_rows_supported(d->F, d->Dv)) return w;
  const long bh = long(d->B) * d->H;
  long S = std::min<long>(ia::device_cus() / bh, d->N / kMinScanSegment);
  for (; S > 1; --S) {
    const int len = int((d->N + S - 1) / S);
    const int n = (d->N + len - 1) / len;
    const size_t slots = round_up(size_t(n) * bh * ia::scan_slot_float2(d->F, d->Dv, d->M) * 8);
    const size_t dec = round_up(size_t(n - 1) * bh * d->M * 8);
    if (w.bytes + slots + dec <= avail) {
      w.n_seg = n;
      w.seg_len = len;
      w.slots_off = w.bytes;
      w.dec_off = w.bytes + slots;
      w.bytes += slots + dec;
      break;
    }
  }
  return w;
}

// Workspace and segmentation of the chunked (bf16, MFMA) path.  Segments cut each sequence so
// that B*H*segments output-pass workgroups fill the device once: as many as its compute units
// hold at the same time (their count times the kernel's workgroups per CU), rounded down, so
// no second, partial round of workgroups follows.

struct ChunkPlan {
  int C, G, seg_chunks;
  size_t tables_off, slots_off, slots_rev_off, state_off, rtab_off, bytes;
};

// Readout options of the desc's flags, in the kernels' encoding.
int kernel_opt(const ia_desc* d) {
  return (d->flags & IA_FLAG_NO_DEN ? ia::kOptNoDen : 0) |
         (d->flags & IA_FLAG_IDENTITY_FEATURES ? ia::kOptIdentity : 0);
}

bool use_chunk_path(const ia_desc* d) {
  // The chunk kernels address a chunk's token rows with 32-bit byte offsets, rows outside a
  // chunk wrapping to large ones: 64 rows of H * F bf16 values must span at most 1 GiB.
  // bf16 calls outside these shapes are refused (IA_ERR_UNSUPPORTED), not sent to the
  // token-sequential kernel.
  return d->in_dtype == IA_BF16 && ia::chunk_supported(d->F, d->Dv, d->M) &&
         64L * d->H * std::max(d->F, d->Dv) * 2 <= (1L << 30);
}

// Chunk length of a call: the descriptor's, else 64, or 32 for a readout matrix whose
// 64-token layout does not fit the LDS.
int chunk_len(const ia_desc* d, bool rm) {
  if (d->chunk) return d->chunk;
  return rm && !ia::chunk_rm_supported(64, d->F, d->Dv, d->M) ? 32 : 64;
}

// The chunked path serves a call: bf16 chunk shapes (use_chunk_path), with a readout matrix a
// chunk length that has its instantiation (no gates: the gated entry point takes no matrix).
bool chunk_path_for(const ia_desc* d, bool rm, bool gated) {
  if ((rm && gated) || !use_chunk_path(d)) return false;
  return !rm || ia::chunk_rm_supported(chunk_len(d, true), d->F, d->Dv, d->M);
}

ChunkPlan chunk_plan(const ia_desc* d, bool rm = false, bool gated = false) {
  ChunkPlan p{};
  p.C = chunk_len(d, rm);
  const int n_chunks = (d->N + p.C - 1) / p.C;
  const long seqs = long(d->B) * d->H;
  int per_cu = ia::chunk_wgs_per_cu(p.C, d->F, d->Dv, d->M, rm, gated);
  if (per_cu <= 0) per_cu = 1;
  long G = long(ia::device_cus()) * per_cu / seqs;
  if (G > n_chunks) G = n_chunks;
  if (G < 1) G = 1;
  p.seg_chunks = int((n_chunks + G - 1) / G);
  p.G = (n_chunks + p.seg_chunks - 1) / p.seg_chunks;
  p.tables_off = 0;
  p.bytes = round_up(size_t(d->H) * ia::chunk_table_bytes(p.C, d->M));
  p.slots_off = p.bytes;
  const size_t slot_bytes =
      p.G > 1 ? round_up(size_t(seqs) * (p.G - 1) * ia::chunk_slot_floats(d->F, d->Dv, d->M) * 4)
              : 0;
  p.bytes += slot_bytes;
  // bidirectional: the reverse walk's slots (both walks' state-only passes run in one launch)
  p.slots_rev_off = p.bytes;
  if (d->flags & IA_FLAG_BIDIR) p.bytes += slot_bytes;
  // one state: the copy of a caller's initial state (several segments), or the working state
  // of heads on the fp32 route when the caller passes none
  p.state_off = p.bytes;
  p.bytes += round_up(state_bytes(d));
  p.rtab_off = p.bytes;
  if (rm) p.bytes += round_up(size_t(d->H) * ia::readout_table_bytes(d->M));
  return p;
}

// Text of the HIP error behind the calling thread's most recent IA_ERR_LAUNCH.
thread_local const char* t_launch_error = "no launch error";

ia_status launch_status(hipError_t e) {
  if (e == hipSuccess) return IA_OK;
  t_launch_error = hipGetErrorString(e);
  return IA_ERR_LAUNCH;
}

}  // namespace

namespace ia {
thread_local ProfileSink* g_profile = nullptr;
}

extern "C" {

const char* ia_status_string(ia_status s) {
  switch (s) {
    case IA_OK: return "IA_OK";
    case IA_ERR_NULL: return "IA_ERR_NULL: a required pointer is NULL";
    case IA_ERR_SHAPE: return "IA_ERR_SHAPE: a size is out of range";
    case IA_ERR_DTYPE: return "IA_ERR_DTYPE: unknown dtype code";
    case IA_ERR_ALIGN: return "IA_ERR_ALIGN: a device pointer is not 16-byte aligned";
    case IA_ERR_ALIAS: return "IA_ERR_ALIAS: an output overlaps an input or another output";
    case IA_ERR_DOMAIN: return "IA_ERR_DOMAIN: a parameter is outside its domain";
    case IA_ERR_UNSUPPORTED: return "IA_ERR_UNSUPPORTED: combination not implemented";
    case IA_ERR_LAUNCH: return "IA_ERR_LAUNCH: the HIP runtime refused a launch";
    case IA_ERR_WORKSPACE: return "IA_ERR_WORKSPACE: workspace missing or too small";
  }
  return "unknown ia_status";
}

const char* ia_last_launch_error(void) { return t_launch_error; }

ia_status ia_check_lambda(const ia_desc* d, const void* lambda_host, int* fp32_heads) {
  ia_status s = check_desc(d, false);
  if (s != IA_OK) return s;
  if (!lambda_host) return IA_ERR_NULL;
  const float* l = static_cast<const float*>(lambda_host);
  const int chunk = d->chunk ? d->chunk : 64;
  const bool chunked = d->in_dtype == IA_BF16;
  int routed = 0;
  ia_status st = IA_OK;
  for (long h = 0; h < d->H; ++h) {
    bool route = false;
    for (long m = 0; m < d->M; ++m) {
      const float x = l[2 * (h * d->M + m)], y = l[2 * (h * d->M + m) + 1];
      const double mag = std::hypot(double(x), double(y));
      if (!(mag > 0.0 && mag <= 1.0 + 1e-6)) st = IA_ERR_DOMAIN;
      route = route || ia::chunk_unresolved(x, y, chunk);
    }
    routed += chunked && route;
  }
  if (fp32_heads) *fp32_heads = routed;
  return st;
}

ia_status ia_state_init(const ia_desc* d, ia_state* st, void* stream) {
  ia_status s = check_desc(d, false);
  if (s != IA_OK) return s;
  if ((s = check_state(d, st)) != IA_OK) return s;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  hipError_t e = ia::launch_fill_zero(st->U, state_u_bytes(d), hs);
  if (e == hipSuccess) e = ia::launch_fill_zero(st->Gamma, state_g_bytes(d), hs);
  if (e == hipSuccess) e = ia::launch_fill_zero(st->eta, state_e_bytes(d), hs);
  return launch_status(e);
}

size_t ia_prefill_workspace_bytes(const ia_desc* d) {
  if (check_desc(d, true) != IA_OK) return 0;
  if (use_chunk_path(d)) return chunk_plan(d).bytes;
  if (d->in_dtype == IA_BF16) return 0;   // no bf16 kernel for this shape
  // The state-less case needs the larger workspace; callers size for it.
  return scan_workspace(d, false).bytes;
}

// The prefill behind every prefill entry point: optional (b, n, h) strides of q, k, v, an
// optional readout matrix ([H][M][M] complex64), and optional write / decay gates ([B][N][H]
// float).
static ia_status prefill_impl(const ia_desc* d, const void* q, const void* k, const void* v,
                              const long long strides[3][3], const void* lambda,
                              const void* beta, const void* readout, ia_state* st, void* o,
                              void* workspace, size_t ws_bytes, void* stream,
                              const float* wgate = nullptr, const float* dgate = nullptr) {
  ia_status s = check_desc(d, true);
  if (s != IA_OK) return s;
  const bool gated = wgate || dgate;
  // Element strides (b, n, h) of q, k, v; the feature axis is contiguous.
  ia::RowStrides sq = ia::dense_strides(d->N, d->H, d->F), sk = sq;
  ia::RowStrides sv = ia::dense_strides(d->N, d->H, d->Dv);
  if (strides) {
    sq = ia::RowStrides{strides[0][0], strides[0][1], strides[0][2]};
    sk = ia::RowStrides{strides[1][0], strides[1][1], strides[1][2]};
    sv = ia::RowStrides{strides[2][0], strides[2][1], strides[2][2]};
    for (const ia::RowStrides& r : {sq, sk, sv}) {
      if (r.b <= 0 || r.n <= 0 || r.h <= 0) return IA_ERR_SHAPE;
      const long long es = esize(d->in_dtype);
      if ((r.b * es) % 16 || (r.n * es) % 16 || (r.h * es) % 16) return IA_ERR_ALIGN;
    }
    if (sq.b != sk.b || sq.n != sk.n || sq.h != sk.h) return IA_ERR_UNSUPPORTED;
    // The chunk kernels address a chunk's rows with 32-bit byte offsets (as for the dense
    // layout in use_chunk_path).
    if (!readout && use_chunk_path(d) &&
        (64LL * sq.n * 2 > (1LL << 30) || 64LL * sv.n * 2 > (1LL << 30)))
      return IA_ERR_UNSUPPORTED;
  }
  const bool bidir = d->flags & IA_FLAG_BIDIR;
  if (!q || !k || !v || !lambda || !beta) return IA_ERR_NULL;
  if (!o && !st) return IA_ERR_NULL;
  if (bidir && st) return IA_ERR_UNSUPPORTED;
  if (bidir && !o) return IA_ERR_NULL;
  for (const void* p : {q, k, v, lambda, beta})
    if (!aligned16(p)) return IA_ERR_ALIGN;
  if (o && !aligned16(o)) return IA_ERR_ALIGN;
  if (readout && !aligned16(readout)) return IA_ERR_ALIGN;
  if ((wgate && !aligned16(wgate)) || (dgate && !aligned16(dgate))) return IA_ERR_ALIGN;
  if (st && (s = check_state(d, st)) != IA_OK) return s;

  const size_t tok = size_t(d->B) * d->N * d->H;
  auto extent = [&](const ia::RowStrides& r, int width) {   // bytes from the base pointer
    return size_t((d->B - 1) * r.b + (d->N - 1) * r.n + (d->H - 1) * r.h + width) *
           esize(d->in_dtype);
  };
  const Range rq = rng(q, extent(sq, d->F));
  const Range rk = rng(k, extent(sk, d->F));
  const Range rv = rng(v, extent(sv, d->Dv));
  const Range rl = rng(lambda, size_t(d->H) * d->M * 8);
  const Range rb = rng(beta, size_t(d->H) * d->M * 8);
  const Range rr = rng(readout, readout ? size_t(d->H) * d->M * d->M * 8 : 0);
  const Range rwg = rng(wgate, wgate ? tok * 4 : 0), rdg = rng(dgate, dgate ? tok * 4 : 0);
  const Range ins[] = {rq, rk, rv, rl, rb, rr, rwg, rdg};
  if (o) {
    const Range ro = rng(o, tok * d->Dv * esize(d->out_dtype));
    for (const Range& r : ins)
      if (overlap(ro, r)) return IA_ERR_ALIAS;
    if (st && (overlap(ro, rng(st->U, state_u_bytes(d))) ||
               overlap(ro, rng(st->Gamma, state_g_bytes(d))) ||
               overlap(ro, rng(st->eta, state_e_bytes(d)))))
      return IA_ERR_ALIAS;
  }
  if (st) {
    const Range sr[] = {rng(st->U, state_u_bytes(d)), rng(st->Gamma, state_g_bytes(d)),
                        rng(st->eta, state_e_bytes(d))};
    for (const Range& a : sr)
      for (const Range& r : ins)
        if (overlap(a, r)) return IA_ERR_ALIAS;
  }

  hipStream_t hs = static_cast<hipStream_t>(stream);

  if (chunk_path_for(d, readout != nullptr, gated)) {
    const ChunkPlan pl = chunk_plan(d, readout != nullptr, gated);
    if (!workspace || ws_bytes < pl.bytes) return IA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return IA_ERR_ALIGN;
    const Range rw = rng(workspace, pl.bytes);
    for (const Range& r : ins)
      if (overlap(rw, r)) return IA_ERR_ALIAS;
    if (o && overlap(rw, rng(o, tok * d->Dv * esize(d->out_dtype)))) return IA_ERR_ALIAS;
    if (st && (overlap(rw, rng(st->U, state_u_bytes(d))) ||
               overlap(rw, rng(st->Gamma, state_g_bytes(d))) ||
               overlap(rw, rng(st->eta, state_e_bytes(d)))))
      return IA_ERR_ALIAS;
    char* ws = static_cast<char*>(workspace);
    ia::ChunkPrefillArgs a{};
    a.wU = reinterpret_cast<float2*>(ws + pl.state_off);
    a.wG = reinterpret_cast<float2*>(ws + pl.state_off + state_u_bytes(d));
    a.wE = reinterpret_cast<float2*>(ws + pl.state_off + state_u_bytes(d) + state_g_bytes(d));
    a.q = q;
    a.k = k;
    a.v = v;
    a.sqk = sq;
    a.sv = sv;
    a.lam = static_cast<const float2*>(lambda);
    a.beta = static_cast<const float2*>(beta);
    a.o = o;
    if (st) {
      a.U0 = a.U1 = static_cast<float2*>(st->U);
      a.G0 = a.G1 = static_cast<float2*>(st->Gamma);
      a.E0 = a.E1 = static_cast<float2*>(st->eta);
    }
    a.slots = reinterpret_cast<float*>(ws + pl.slots_off);
    a.tables = reinterpret_cast<unsigned char*>(ws + pl.tables_off);
    a.readout = static_cast<const float2*>(readout);
    a.rtab = readout ? reinterpret_cast<unsigned char*>(ws + pl.rtab_off) : nullptr;
    a.wgate = wgate;
    a.dgate = dgate;
    a.B = d->B; a.H = d->H; a.N = d->N; a.F = d->F; a.D = d->Dv; a.M = d->M;
    a.chunk = pl.C;
    a.segments = pl.G;
    a.seg_chunks = pl.seg_chunks;
    a.out_bf16 = d->out_dtype == IA_BF16;
    a.clamp = d->den_clamp;
    a.opt = kernel_opt(d);
    // Bidirectional: both walks in one call; the forward one writes o, the reverse one adds
    // onto it.
    if (bidir) a.slots_rev = pl.G > 1 ? reinterpret_cast<float*>(ws + pl.slots_rev_off) : nullptr;
    if (bidir && pl.G == 1) {
      hipError_t e = ia::launch_chunk_prefill(a, hs);
      if (e == hipSuccess) {
        a.accumulate = 1;
        a.reverse = 1;
        e = ia::launch_chunk_prefill(a, hs);
      }
      return launch_status(e);
    }
    return launch_status(ia::launch_chunk_prefill(a, hs));
  }

  // bf16 inputs on shapes without a chunk kernel are refused rather than run 300x slower by
  // the token-sequential kernel (fp32 inputs take that path, as do gated calls on shapes
  // without a chunk kernel).  A readout
  // matrix with bf16 inputs runs the token-sequential kernel only on shapes the chunk kernels
  // do not take at all; a chunk shape whose requested chunk length has no readout-matrix
  // instantiation is refused.
  if (!gated && d->in_dtype == IA_BF16 && (!readout || use_chunk_path(d)))
    return IA_ERR_UNSUPPORTED;

  // fp32 path: token-sequential recurrence.
  const ScanWorkspace w = scan_workspace(d, st != nullptr, workspace ? ws_bytes : 0);
  if (w.bytes) {
    if (!workspace || ws_bytes < w.bytes) return IA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return IA_ERR_ALIGN;
    const Range rw = rng(workspace, w.bytes);
    for (const Range& r : ins)
      if (overlap(rw, r)) return IA_ERR_ALIAS;
    if (o && overlap(rw, rng(o, tok * d->Dv * esize(d->out_dtype)))) return IA_ERR_ALIAS;
  }
  char* ws = static_cast<char*>(workspace);
  float2 *U, *G, *E;
  if (st && !bidir) {
    U = static_cast<float2*>(st->U);
    G = static_cast<float2*>(st->Gamma);
    E = static_cast<float2*>(st->eta);
  } else {
    U = reinterpret_cast<float2*>(ws + w.state_off);
    G = reinterpret_cast<float2*>(ws + w.state_off + state_u_bytes(d));
    E = reinterpret_cast<float2*>(ws + w.state_off + state_u_bytes(d) + state_g_bytes(d));
    hipError_t e = ia::launch_fill_zero(ws + w.state_off, state_bytes(d), hs);
    if (e != hipSuccess) return launch_status(e);
  }
  ia::ScanArgs a{q, k, v, sq, sv, static_cast<const float2*>(lambda),
                 static_cast<const float2*>(beta), U, G, E, o, 0, d->B, d->H, d->N, d->F, d->Dv,
                 d->M, d->in_dtype == IA_BF16, d->out_dtype == IA_BF16, d->den_clamp, 0};
  a.opt = kernel_opt(d);
  a.readout = static_cast<const float2*>(readout);
  a.wgate = wgate;
  a.dgate = dgate;
  if (w.n_seg > 1) {
    a.n_seg = w.n_seg;
    a.seg_len = w.seg_len;
    a.slots = reinterpret_cast<float2*>(ws + w.slots_off);
    a.dec = reinterpret_cast<float2*>(ws + w.dec_off);
  }
  if (!bidir) return launch_status(ia::launch_scan_prefill(a, hs));

  // Bidirectional: the forward direction writes o, the reverse direction (from a zero state
  // again) adds onto it.
  hipError_t e = ia::launch_scan_prefill(a, hs);
  if (e == hipSuccess) e = ia::launch_fill_zero(ws + w.state_off, state_bytes(d), hs);
  if (e == hipSuccess) {
    a.accumulate = 1;
    a.reverse = 1;
    e = ia::launch_scan_prefill(a, hs);
  }
  return launch_status(e);
}

ia_status ia_prefill_fwd(const ia_desc* d, const void* q, const void* k, const void* v,
                         const void* lambda, const void* beta, ia_state* st, void* o,
                         void* workspace, size_t ws_bytes, void* stream) {
  return prefill_impl(d, q, k, v, nullptr, lambda, beta, nullptr, st, o, workspace, ws_bytes,
                      stream);
}

}  // extern "C"

namespace ia {
// Status of a HIP error, keeping its text for ia_last_launch_error.
ia_status status_of(hipError_t e) { return launch_status(e); }

// ia_prefill_fwd on a workspace the caller does not pass (the no-allocation entry point).
ia_status prefill_on_workspace(const ia_desc* d, const void* q, const void* k, const void* v,
                               const void* lambda, const void* beta, ia_state* st, void* o,
                               void* workspace, size_t ws_bytes, void* stream) {
  return prefill_impl(d, q, k, v, nullptr, lambda, beta, nullptr, st, o, workspace, ws_bytes,
                      stream);
}
}  // namespace ia

extern "C" {

ia_status ia_prefill_fwd_strided(const ia_desc* d, const void* q, const void* k, const void* v,
                                 const long long strides[3][3], const void* lambda,
                                 const void* beta, ia_state* st, void* o, void* workspace,
                                 size_t ws_bytes, void* stream) {
  return prefill_impl(d, q, k, v, strides, lambda, beta, nullptr, st, o, workspace, ws_bytes,
                      stream);
}

size_t ia_prefill_readout_workspace_bytes(const ia_desc* d) {
  if (check_desc(d, true) != IA_OK) return 0;
  if (chunk_path_for(d, true, false)) return chunk_plan(d, true).bytes;
  return scan_workspace(d, false).bytes;
}

ia_status ia_prefill_fwd_readout(const ia_desc* d, const void* q, const void* k, const void* v,
                                 const void* lambda, const void* beta, const void* readout,
                                 ia_state* st, void* o, void* workspace, size_t ws_bytes,
                                 void* stream) {
  if (!readout) return IA_ERR_NULL;
  return prefill_impl(d, q, k, v, nullptr, lambda, beta, readout, st, o, workspace, ws_bytes,
                      stream);
}

size_t ia_prefill_gated_workspace_bytes(const ia_desc* d) {
  if (check_desc(d, true) != IA_OK) return 0;
  if (chunk_path_for(d, false, true)) return chunk_plan(d, false, true).bytes;
  return scan_workspace(d, false).bytes;
}

ia_status ia_prefill_fwd_gated(const ia_desc* d, const void* q, const void* k, const void* v,
                               const void* wgate, const void* dgate, const void* lambda,
                               const void* beta, ia_state* st, void* o, void* workspace,
                               size_t ws_bytes, void* stream) {
  if (!wgate || !dgate) return IA_ERR_NULL;
  return prefill_impl(d, q, k, v, nullptr, lambda, beta, nullptr, st, o, workspace, ws_bytes,
                      stream, static_cast<const float*>(wgate), static_cast<const float*>(dgate));
}

// Which backward serves a call: the flag's, else the chunked one where it exists, unless the
// slices and mode groups are too few to fill the device: the token-sequential sweeps then cut
// each sequence into segments that run side by side, which the chunked walk does not.
static bool bwd_chunked(const ia_desc* d) {
  if (d->flags & IA_FLAG_SEQUENTIAL_BWD) return false;
  if (d->flags & IA_FLAG_CHUNKED_BWD) return true;
  int seg_len;
  return ia::bwd_chunked_supported(d->F, d->Dv, d->M) &&
         ia::bwd_segments(d->B, d->H, d->N, d->M, &seg_len) <= 8;
}

static ia_status check_bwd_path(const ia_desc* d) {
  const unsigned both = IA_FLAG_SEQUENTIAL_BWD | IA_FLAG_CHUNKED_BWD;
  if ((d->flags & both) == both) return IA_ERR_UNSUPPORTED;
  if ((d->flags & IA_FLAG_CHUNKED_BWD) && !ia::bwd_chunked_supported(d->F, d->Dv, d->M))
    return IA_ERR_UNSUPPORTED;
  return IA_OK;
}

static ia::BwdLayout bwd_plan(const ia_desc* d) {
  return bwd_chunked(d) ? ia::bwd_chunked_layout(d->B, d->H, d->N, d->F, d->Dv, d->M)
                        : ia::bwd_layout(d->B, d->H, d->N, d->F, d->Dv, d->M);
}

size_t ia_prefill_bwd_workspace_bytes(const ia_desc* d) {
  if (check_desc(d, true) != IA_OK || check_bwd_path(d) != IA_OK) return 0;
  return bwd_plan(d).bytes;
}

ia_status ia_prefill_bwd(const ia_desc* d, const void* q, const void* k, const void* v,
                         const void* lambda, const void* beta, const ia_state* st0,
                         const void* dO, void* dq, void* dk, void* dv, void* dlambda,
                         void* dbeta, ia_state* dst0, void* workspace, size_t ws_bytes,
                         void* stream) {
  ia_status s = check_desc(d, true);
  if (s != IA_OK) return s;
  if ((s = check_bwd_path(d)) != IA_OK) return s;
  const bool bidir = d->flags & IA_FLAG_BIDIR;
  if (!q || !k || !v || !lambda || !beta || !dO || !dq || !dk || !dv || !dlambda || !dbeta)
    return IA_ERR_NULL;
  if (bidir && (st0 || dst0)) return IA_ERR_UNSUPPORTED;   // both directions start from zero
  for (const void* p : {q, k, v, lambda, beta, dO, static_cast<const void*>(dq),
                        static_cast<const void*>(dk), static_cast<const void*>(dv),
                        static_cast<const void*>(dlambda), static_cast<const void*>(dbeta)})
    if (!aligned16(p)) return IA_ERR_ALIGN;
  if (st0 && (s = check_state(d, st0)) != IA_OK) return s;
  if (dst0 && (s = check_state(d, dst0)) != IA_OK) return s;
  const bool chunked = bwd_chunked(d);
  const ia::BwdLayout L = bwd_plan(d);
  if (!workspace || ws_bytes < L.bytes) return IA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return IA_ERR_ALIGN;

  const size_t tok = size_t(d->B) * d->N * d->H;
  const size_t ein = esize(d->in_dtype);
  Range ins[9] = {rng(q, tok * d->F * ein), rng(k, tok * d->F * ein),
                  rng(v, tok * d->Dv * ein), rng(lambda, size_t(d->H) * d->M * 8),
                  rng(beta, size_t(d->H) * d->M * 8),
                  rng(dO, tok * d->Dv * esize(d->out_dtype))};
  int n_ins = 6;
  if (st0) {
    ins[n_ins++] = rng(st0->U, state_u_bytes(d));
    ins[n_ins++] = rng(st0->Gamma, state_g_bytes(d));
    ins[n_ins++] = rng(st0->eta, state_e_bytes(d));
  }
  Range outs[9] = {rng(dq, tok * d->F * ein), rng(dk, tok * d->F * ein),
                   rng(dv, tok * d->Dv * ein), rng(dlambda, size_t(d->H) * d->M * 8),
                   rng(dbeta, size_t(d->H) * d->M * 8), rng(workspace, L.bytes)};
  int n_outs = 6;
  if (dst0) {
    outs[n_outs++] = rng(dst0->U, state_u_bytes(d));
    outs[n_outs++] = rng(dst0->Gamma, state_g_bytes(d));
    outs[n_outs++] = rng(dst0->eta, state_e_bytes(d));
  }
  for (int i = 0; i < n_outs; ++i) {
    for (int j = 0; j < n_ins; ++j)
      if (overlap(outs[i], ins[j])) return IA_ERR_ALIAS;
    for (int j = i + 1; j < n_outs; ++j)
      if (overlap(outs[i], outs[j])) return IA_ERR_ALIAS;
  }

  char* ws = static_cast<char*>(workspace);
  ia::BwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.dO = dO;
  a.lam = static_cast<const float2*>(lambda);
  a.beta = static_cast<const float2*>(beta);
  if (st0) {
    a.U0 = static_cast<const float2*>(st0->U);
    a.G0 = static_cast<const float2*>(st0->Gamma);
    a.E0 = static_cast<const float2*>(st0->eta);
  }
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dlam = static_cast<float2*>(dlambda);
  a.dbeta = static_cast<float2*>(dbeta);
  if (dst0) {
    a.dU0 = static_cast<float2*>(dst0->U);
    a.dG0 = static_cast<float2*>(dst0->Gamma);
    a.dE0 = static_cast<float2*>(dst0->eta);
  }
  a.ckpt = reinterpret_cast<float2*>(ws + L.ckpt_off);
  a.dpart = reinterpret_cast<float2*>(ws + L.dpart_off);
  a.gpart = reinterpret_cast<float*>(ws + L.gpart_off);
  a.lpart = reinterpret_cast<float2*>(ws + L.lpart_off);
  a.apart = reinterpret_cast<float2*>(ws + L.apart_off);
  a.cstate = reinterpret_cast<float2*>(ws + L.cstate_off);
  a.cadj = reinterpret_cast<float2*>(ws + L.cadj_off);
  if (chunked) {
    a.nseg = 1;
    a.seg_len = d->N;
  } else {
    a.nseg = ia::bwd_segments(d->B, d->H, d->N, d->M, &a.seg_len);
  }
  a.B = d->B; a.H = d->H; a.N = d->N; a.F = d->F; a.D = d->Dv; a.M = d->M;
  a.in_bf16 = d->in_dtype == IA_BF16;
  a.out_bf16 = d->out_dtype == IA_BF16;
  a.opt = kernel_opt(d);
  a.clamp = d->den_clamp;
  a.tb = ia::bwd_block_tokens(d->F, d->Dv, d->M, a.in_bf16, a.out_bf16);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  auto launch = chunked ? ia::launch_prefill_bwd_chunked : ia::launch_prefill_bwd;
  hipError_t e = launch(a, hs);
  if (e == hipSuccess && bidir) {
    // o = IA(x) + flip(IA(flip x)): the reversed walk's gradients are added on (the workspace
    // is reused in stream order)
    a.dir = 1;
    a.accumulate = 1;
    e = launch(a, hs);
  }
  return launch_status(e);
}

// The decode step behind both decode entry points; readout: [H][M][M] complex64 or NULL.
static ia_status decode_impl(const ia_desc* d, const void* q_t, const void* k_t,
                             const void* v_t, const void* lambda, const void* beta,
                             const void* readout, ia_state* st, void* o_t, void* stream,
                             const float* wgate = nullptr, const float* dgate = nullptr) {
  ia_status s = check_desc(d, false);
  if (s != IA_OK) return s;
  if (d->flags & IA_FLAG_BIDIR) return IA_ERR_UNSUPPORTED;
  if (!q_t || !k_t || !v_t || !lambda || !beta || !o_t) return IA_ERR_NULL;
  if ((s = check_state(d, st)) != IA_OK) return s;
  for (const void* p : {q_t, k_t, v_t, lambda, beta, static_cast<const void*>(o_t)})
    if (!aligned16(p)) return IA_ERR_ALIGN;
  if (readout && !aligned16(readout)) return IA_ERR_ALIGN;
  if ((wgate && !aligned16(wgate)) || (dgate && !aligned16(dgate))) return IA_ERR_ALIGN;
  const size_t bh = size_t(d->B) * d->H;
  const Range ins[] = {rng(q_t, bh * d->F * esize(d->in_dtype)),
                       rng(k_t, bh * d->F * esize(d->in_dtype)),
                       rng(v_t, bh * d->Dv * esize(d->in_dtype)),
                       rng(lambda, size_t(d->H) * d->M * 8), rng(beta, size_t(d->H) * d->M * 8),
                       rng(readout, readout ? size_t(d->H) * d->M * d->M * 8 : 0),
                       rng(wgate, wgate ? bh * 4 : 0), rng(dgate, dgate ? bh * 4 : 0)};
  const Range outs[] = {rng(o_t, bh * d->Dv * esize(d->out_dtype)),
                        rng(st->U, state_u_bytes(d)), rng(st->Gamma, state_g_bytes(d)),
                        rng(st->eta, state_e_bytes(d))};
  for (const Range& a : outs)
    for (const Range& r : ins)
      if (overlap(a, r)) return IA_ERR_ALIAS;
  for (int i = 1; i < 4; ++i)
    if (overlap(outs[0], outs[i])) return IA_ERR_ALIAS;
  ia::DecodeArgs a{q_t, k_t, v_t, static_cast<const float2*>(lambda),
                   static_cast<const float2*>(beta), static_cast<float2*>(st->U),
                   static_cast<float2*>(st->Gamma), static_cast<float2*>(st->eta), o_t,
                   d->B, d->H, d->F, d->Dv, d->M, d->in_dtype == IA_BF16,
                   d->out_dtype == IA_BF16, d->den_clamp};
  a.opt = kernel_opt(d);
  a.readout = static_cast<const float2*>(readout);
  a.wgate = wgate;
  a.dgate = dgate;
  return launch_status(ia::launch_decode_step(a, static_cast<hipStream_t>(stream)));
}

ia_status ia_decode_step(const ia_desc* d, const void* q_t, const void* k_t, const void* v_t,
                         const void* lambda, const void* beta, ia_state* st, void* o_t,
                         void* stream) {
  return decode_impl(d, q_t, k_t, v_t, lambda, beta, nullptr, st, o_t, stream);
}

ia_status ia_decode_step_gated(const ia_desc* d, const void* q_t, const void* k_t,
                               const void* v_t, const void* wgate, const void* dgate,
                               const void* lambda, const void* beta, ia_state* st, void* o_t,
                               void* stream) {
  if (!wgate || !dgate) return IA_ERR_NULL;
  return decode_impl(d, q_t, k_t, v_t, lambda, beta, nullptr, st, o_t, stream,
                     static_cast<const float*>(wgate), static_cast<const float*>(dgate));
}

ia_status ia_decode_step_readout(const ia_desc* d, const void* q_t, const void* k_t,
                                 const void* v_t, const void* lambda, const void* beta,
                                 const void* readout, ia_state* st, void* o_t, void* stream) {
  if (!readout) return IA_ERR_NULL;
  return decode_impl(d, q_t, k_t, v_t, lambda, beta, readout, st, o_t, stream);
}

// ---------------------------------------------------------------- the block's edges

// Checks of ia_block_params shared by the prologue and the fused decode step: the tap count,
// the weight and normalisation arrays, RoPE's base and the positions pos0 .. pos0 + n - 1.
static ia_status check_block_params(const ia_block_params* p, long n) {
  const int W = p->conv_width;
  if (W < 0 || W > ia::kMaxConvTaps) return IA_ERR_UNSUPPORTED;
  if (W > 0 && (!p->conv_q || !p->conv_k || !p->conv_v)) return IA_ERR_NULL;
  if (!(std::isfinite(p->rope_base) && p->rope_base >= 0.f) || p->pos0 < 0 ||
      (long long)p->pos0 + n - 1 > 2147483647LL)
    return IA_ERR_DOMAIN;
  if ((p->norm_gain == nullptr) != (p->norm_bias == nullptr)) return IA_ERR_NULL;
  if (p->norm_gain && !(std::isfinite(p->norm_eps) && p->norm_eps >= 0.f)) return IA_ERR_DOMAIN;
  for (const void* x : {p->conv_q, p->conv_k, p->conv_v, p->norm_gain, p->norm_bias})
    if (x && !aligned16(x)) return IA_ERR_ALIGN;
  return IA_OK;
}

// The parameter arrays of p (five ranges) and the convolution state's bytes.
static void block_param_ranges(const ia_desc* d, const ia_block_params* p, Range* r) {
  const int W = p->conv_width;
  r[0] = rng(p->conv_q, W ? size_t(d->H) * d->F * W * 4 : 0);
  r[1] = rng(p->conv_k, W ? size_t(d->H) * d->F * W * 4 : 0);
  r[2] = rng(p->conv_v, W ? size_t(d->H) * d->Dv * W * 4 : 0);
  r[3] = rng(p->norm_gain, p->norm_gain ? size_t(d->H) * (d->F + d->Dv) * 4 : 0);
  r[4] = rng(p->norm_bias, p->norm_bias ? size_t(d->H) * (d->F + d->Dv) * 4 : 0);
}
static size_t conv_state_bytes(const ia_desc* d, int W) {
  return W > 1 ? size_t(d->B) * d->H * (W - 1) * (2 * d->F + d->Dv) * 4 : 0;
}

ia_status ia_block_prologue(const ia_desc* d, const ia_block_params* p, const void* q,
                            const void* k, const void* v, const void* conv_state_in,
                            void* conv_state_out, void* fq, void* fk, void* vo, void* stream) {
  ia_status s = check_desc(d, true);
  if (s != IA_OK) return s;
  if (!p || !q || !k || !v || !fq || !fk || !vo) return IA_ERR_NULL;
  if ((s = check_block_params(p, d->N)) != IA_OK) return s;
  if ((long long)d->H * (d->F > d->Dv ? d->F : d->Dv) * esize(d->in_dtype) >= (1LL << 24))
    return IA_ERR_UNSUPPORTED;   // a token's row of one tensor: under 16 MiB
  const int W = p->conv_width;
  for (const void* x : {q, k, v, static_cast<const void*>(fq), static_cast<const void*>(fk),
                        static_cast<const void*>(vo)})
    if (!aligned16(x)) return IA_ERR_ALIGN;
  const bool st_used = W > 1;
  if (st_used && ((conv_state_in && !aligned16(conv_state_in)) ||
                  (conv_state_out && !aligned16(conv_state_out))))
    return IA_ERR_ALIGN;
  const size_t tok = size_t(d->B) * d->N * d->H, es = esize(d->in_dtype);
  const size_t st_bytes = conv_state_bytes(d, W);
  Range ins[9] = {rng(q, tok * d->F * es), rng(k, tok * d->F * es), rng(v, tok * d->Dv * es)};
  block_param_ranges(d, p, ins + 3);
  ins[8] = rng(st_used ? conv_state_in : nullptr, st_bytes);
  const Range outs[] = {rng(fq, tok * d->F * es), rng(fk, tok * d->F * es),
                        rng(vo, tok * d->Dv * es),
                        rng(st_used ? conv_state_out : nullptr, st_bytes)};
  for (const Range& a : outs)
    for (const Range& r : ins)
      if (overlap(a, r)) return IA_ERR_ALIAS;
  for (int i = 0; i < 4; ++i)
    for (int j = i + 1; j < 4; ++j)
      if (overlap(outs[i], outs[j])) return IA_ERR_ALIAS;
  ia::BlockArgs a{};
  a.q = q; a.k = k; a.v = v; a.fq = fq; a.fk = fk; a.vo = vo;
  a.conv_q = static_cast<const float*>(p->conv_q);
  a.conv_k = static_cast<const float*>(p->conv_k);
  a.conv_v = static_cast<const float*>(p->conv_v);
  a.state_in = st_used ? static_cast<const float*>(conv_state_in) : nullptr;
  a.state_out = st_used ? static_cast<float*>(conv_state_out) : nullptr;
  a.norm_gain = static_cast<const float*>(p->norm_gain);
  a.norm_bias = static_cast<const float*>(p->norm_bias);
  a.norm_eps = p->norm_eps;
  a.rope_base = p->rope_base;
  a.B = d->B; a.H = d->H; a.N = d->N; a.F = d->F; a.D = d->Dv;
  a.conv_width = W;
  a.pos0 = p->pos0;
  a.bf16 = d->in_dtype == IA_BF16;
  return launch_status(ia::launch_block_prologue(a, static_cast<hipStream_t>(stream)));
}

ia_status ia_block_decode_step(const ia_desc* d, const ia_block_params* p, const void* q_t,
                               const void* k_t, const void* v_t, const void* conv_state_in,
                               void* conv_state_out, const void* gate_t, const void* lambda,
                               const void* beta, ia_state* st, void* out_t, void* stream) {
  ia_status s = check_desc(d, false);
  if (s != IA_OK) return s;
  if (d->flags & (IA_FLAG_BIDIR | IA_FLAG_IDENTITY_FEATURES)) return IA_ERR_UNSUPPORTED;
  if (!p || !q_t || !k_t || !v_t || !lambda || !beta || !out_t) return IA_ERR_NULL;
  if ((s = check_state(d, st)) != IA_OK) return s;
  if ((s = check_block_params(p, 1)) != IA_OK) return s;
  const int W = p->conv_width;
  for (const void* x : {q_t, k_t, v_t, lambda, beta, static_cast<const void*>(out_t)})
    if (!aligned16(x)) return IA_ERR_ALIGN;
  if (gate_t && !aligned16(gate_t)) return IA_ERR_ALIGN;
  const bool st_used = W > 1;
  if (st_used && ((conv_state_in && !aligned16(conv_state_in)) ||
                  (conv_state_out && !aligned16(conv_state_out))))
    return IA_ERR_ALIGN;
  const size_t bh = size_t(d->B) * d->H, es = esize(d->in_dtype);
  const size_t st_bytes = conv_state_bytes(d, W);
  Range ins[12] = {rng(q_t, bh * d->F * es), rng(k_t, bh * d->F * es),
                   rng(v_t, bh * d->Dv * es), rng(gate_t, gate_t ? bh * d->Dv * es : 0),
                   rng(lambda, size_t(d->H) * d->M * 8), rng(beta, size_t(d->H) * d->M * 8),
                   rng(st_used ? conv_state_in : nullptr, st_bytes)};
  block_param_ranges(d, p, ins + 7);
  const Range outs[] = {rng(out_t, bh * d->Dv * esize(d->out_dtype)),
                        rng(st->U, state_u_bytes(d)), rng(st->Gamma, state_g_bytes(d)),
                        rng(st->eta, state_e_bytes(d)),
                        rng(st_used ? conv_state_out : nullptr, st_bytes)};
  for (const Range& a : outs)
    for (const Range& r : ins)
      if (overlap(a, r)) return IA_ERR_ALIAS;
  for (int i = 0; i < 5; ++i)
    for (int j = i + 1; j < 5; ++j)
      if (overlap(outs[i], outs[j])) return IA_ERR_ALIAS;
  ia::DecodeArgs a{q_t, k_t, v_t, static_cast<const float2*>(lambda),
                   static_cast<const float2*>(beta), static_cast<float2*>(st->U),
                   static_cast<float2*>(st->Gamma), static_cast<float2*>(st->eta), out_t,
                   d->B, d->H, d->F, d->Dv, d->M, d->in_dtype == IA_BF16,
                   d->out_dtype == IA_BF16, d->den_clamp};
  a.opt = kernel_opt(d);
  a.block = 1;
  a.blk.conv_q = static_cast<const float*>(p->conv_q);
  a.blk.conv_k = static_cast<const float*>(p->conv_k);
  a.blk.conv_v = static_cast<const float*>(p->conv_v);
  a.blk.state_in = st_used ? static_cast<const float*>(conv_state_in) : nullptr;
  a.blk.state_out = st_used ? static_cast<float*>(conv_state_out) : nullptr;
  a.blk.norm_gain = static_cast<const float*>(p->norm_gain);
  a.blk.norm_bias = static_cast<const float*>(p->norm_bias);
  a.blk.norm_eps = p->norm_eps;
  a.blk.rope_base = p->rope_base;
  a.blk.pos = p->pos0;
  a.blk.conv_width = W;
  a.blk.gate = gate_t;
  return launch_status(ia::launch_decode_step(a, static_cast<hipStream_t>(stream)));
}

ia_status ia_block_gate(const ia_desc* d, const void* o, const void* g, void* out,
                        void* stream) {
  ia_status s = check_desc(d, true);
  if (s != IA_OK) return s;
  if (!o || !g || !out) return IA_ERR_NULL;
  for (const void* x : {o, g, static_cast<const void*>(out)})
    if (!aligned16(x)) return IA_ERR_ALIGN;
  const size_t n = size_t(d->B) * d->N * d->H * d->Dv;
  const size_t bytes = n * esize(d->out_dtype);
  const Range ro = rng(o, bytes), rg = rng(g, bytes), rout = rng(out, bytes);
  // out may be o itself (each element is read, then written, by one thread), not part of it
  if (overlap(rout, rg) || (overlap(rout, ro) && out != o)) return IA_ERR_ALIAS;
  return launch_status(ia::launch_block_gate(o, g, out, n, d->out_dtype == IA_BF16,
                                             static_cast<hipStream_t>(stream)));
}

ia_status ia_prefill_fwd_profiled(const ia_desc* d, const void* q, const void* k,
                                  const void* v, const void* lambda, const void* beta,
                                  ia_state* st, void* o, void* workspace, size_t ws_bytes,
                                  void* stream, void** events, int* kinds, int max_launches,
                                  int* n_launches) {
  if (!events || !kinds || !n_launches || max_launches < 0) return IA_ERR_NULL;
  for (int i = 0; i < 2 * max_launches; ++i)
    if (!events[i]) return IA_ERR_NULL;
  ia::ProfileSink sink{events, kinds, max_launches, 0};
  ia::g_profile = &sink;
  const ia_status s = ia_prefill_fwd(d, q, k, v, lambda, beta, st, o, workspace, ws_bytes,
                                     stream);
  ia::g_profile = nullptr;
  *n_launches = sink.used;
  return s;
}

}  // extern "C"
