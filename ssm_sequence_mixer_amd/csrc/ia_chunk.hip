// ia_chunk.hip — chunked IA prefill: per-head tables and the host-side dispatch over the
// kernel instantiations (which live in ia_chunk_f*.hip).
#include "ia_chunk.hpp"
#include "ia_chunk_state.hpp"
#include "ia_tables.hpp"

namespace ia {

#define IA_EXTERN(C, FF, MM)                                                              \
  extern template hipError_t launch_chunk_t<C, FF, FF, MM>(const ChunkArgs&, int, hipStream_t, \
                                                           int);                          \
  extern template hipError_t launch_state_t<C, FF, FF, MM>(const ChunkArgs&, int, hipStream_t, \
                                                           int);                          \
  extern template int chunk_occupancy_t<C, FF, FF, MM>();
// The gated layer's kernels (ia_chunk_g*.hip).
#define IA_EXTERN_G(C, FF, MM)                                                            \
  extern template hipError_t launch_chunk_t<C, FF, FF, MM, false, true>(                   \
      const ChunkArgs&, int, hipStream_t, int);                                           \
  extern template hipError_t launch_state_t<C, FF, FF, MM, true>(const ChunkArgs&, int,    \
                                                                 hipStream_t, int);       \
  extern template int chunk_occupancy_t<C, FF, FF, MM, false, true>();
#define IA_EXTERN_C(C)                                                                    \
  IA_EXTERN(C, 32, 16) IA_EXTERN(C, 32, 32) IA_EXTERN(C, 32, 64)                          \
  IA_EXTERN(C, 64, 16) IA_EXTERN(C, 64, 32) IA_EXTERN(C, 64, 64)                          \
  IA_EXTERN(C, 128, 16) IA_EXTERN(C, 128, 32) IA_EXTERN(C, 128, 64)                       \
  IA_EXTERN_G(C, 32, 16) IA_EXTERN_G(C, 32, 32) IA_EXTERN_G(C, 32, 64)                    \
  IA_EXTERN_G(C, 64, 16) IA_EXTERN_G(C, 64, 32) IA_EXTERN_G(C, 64, 64)                    \
  IA_EXTERN_G(C, 128, 16) IA_EXTERN_G(C, 128, 32) IA_EXTERN_G(C, 128, 64)
IA_EXTERN_C(32)
IA_EXTERN_C(64)
#undef IA_EXTERN_C
#undef IA_EXTERN_G
#undef IA_EXTERN
// The readout-matrix variant, for every shape whose LDS layout fits (all but C = 64 with
// F = Dv = 128 and M = 64).
#define IA_EXTERN_RM(C, FF, MM)                                                           \
  extern template hipError_t launch_chunk_t<C, FF, FF, MM, true>(const ChunkArgs&, int,    \
                                                                 hipStream_t, int);       \
  extern template int chunk_occupancy_t<C, FF, FF, MM, true>();
IA_EXTERN_RM(32, 32, 16) IA_EXTERN_RM(32, 32, 32) IA_EXTERN_RM(32, 32, 64)
IA_EXTERN_RM(32, 64, 16) IA_EXTERN_RM(32, 64, 32) IA_EXTERN_RM(32, 64, 64)
IA_EXTERN_RM(32, 128, 16) IA_EXTERN_RM(32, 128, 32) IA_EXTERN_RM(32, 128, 64)
IA_EXTERN_RM(64, 32, 16) IA_EXTERN_RM(64, 32, 32) IA_EXTERN_RM(64, 32, 64)
IA_EXTERN_RM(64, 64, 16) IA_EXTERN_RM(64, 64, 32) IA_EXTERN_RM(64, 64, 64)
IA_EXTERN_RM(64, 128, 16) IA_EXTERN_RM(64, 128, 32)
#undef IA_EXTERN_RM

bool chunk_rm_supported(int chunk, int F, int D, int M) {
  return chunk_supported(F, D, M) && (chunk == 32 || chunk == 64) &&
         !(chunk == 64 && F == 128 && D == 128 && M == 64);
}

long readout_table_bytes(int M) {
  switch (M) {
    case 16: return ReadoutTable<16>::bytes;
    case 32: return ReadoutTable<32>::bytes;
    case 64: return ReadoutTable<64>::bytes;
  }
  return 0;
}

// ---------------------------------------------------------------- per-head tables
// Once per call, when no state-only pass carries them: block (h, run) is one table run
// (table_run), C/4 small blocks per head, so the transcendental work spreads over the CUs.
// Block (h, 0) also writes the head's readout-matrix operand when rtab is set.
template <int C, int M>
__global__ void __launch_bounds__(4 * M) chunk_tables_kernel(const float2* __restrict__ lam,
                                    const float2* __restrict__ beta, unsigned char* tables,
                                    long table_bytes, int Lt, int Ls, int half,
                                    const float2* __restrict__ R, unsigned char* rtab,
                                    long rtab_bytes) {
  table_run<C, M>(lam, beta, tables, table_bytes, Lt, Ls, blockIdx.x, blockIdx.y, threadIdx.x,
                  half);
  if (rtab && blockIdx.y == 0)
    readout_table_run<M>(R, rtab, rtab_bytes, blockIdx.x, threadIdx.x, 4 * M);
}

// ---------------------------------------------------------------- segment carry
// Turns the end states of segments 0..G-2 (each from a zero state, in the slot layout) into
// the states entering segments 1..G-1, in place:
//   slot 0 <- lam^Ls (lam init) + slot 0,   slot g <- lam^Ls slot g-1 + slot g
// (gated: lam^Ls times segment g's decay product, held by slot g).
// One thread per lane of a tile pair (4 Re, 4 Im values; a wave per pair, whose 16-lane rows
// requantise it: SlotLayout) or per mode of lam eta; segments in order, the carried state in fp32.  Used
// when the output pass would otherwise combine many slots per workgroup.  With slots_rev set
// (a bidirectional call, no initial state) rows y >= nseq of the grid carry the reverse walk's
// slots.
template <int F, int D, int M>
__global__ void __launch_bounds__(256)
carry_slots_kernel(float* __restrict__ slots, float* __restrict__ slots_rev, int nseq,
                   const float2* __restrict__ U0,
                   const float2* __restrict__ G0, const float2* __restrict__ E0,
                   const float2* __restrict__ lam, const unsigned char* __restrict__ tables,
                   long table_bytes, long pows_off, int H, int nslots, long slot_floats,
                   int gated) {
  using SL = SlotLayout<F, D, M>;
  constexpr int NS = SL::NS, NFT = SL::NFT, NDT = SL::NDT, MH = M / 16;
  constexpr int PAIRS = NS * (NFT + NDT) * MH * 64;
  int seq = blockIdx.y;
  float* walk_slots = slots;
  if (slots_rev && seq >= nseq) {
    seq -= nseq;
    walk_slots = slots_rev;
  }
  const int h = seq % H;
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= PAIRS + M) return;
  float* base = walk_slots + (size_t)seq * nslots * slot_floats;
  const float2* lamh = lam + (size_t)h * M;
  const float2* pows =
      reinterpret_cast<const float2*>(tables + (size_t)h * table_bytes + pows_off);
  // Slots are loaded KB at a time ahead of their combination, so the loads of a batch are in
  // flight together instead of one round trip per slot.
  constexpr int KB = 8;
  if (e >= PAIRS) {   // lam eta, mode m
    const int m = e - PAIRS;
    const float2 p = pows[m];
    float2 c = E0 ? cmul(lamh[m], E0[(size_t)seq * M + m]) : make_float2(0.f, 0.f);
    for (int g0 = 0; g0 < nslots; g0 += KB) {
      float2 x[KB];
      float ds[KB];
#pragma unroll
      for (int k = 0; k < KB; ++k)
        if (g0 + k < nslots) {
          const float* sl = base + (size_t)(g0 + k) * slot_floats;
          x[k] = reinterpret_cast<const float2*>(sl + SL::eta)[m];
          ds[k] = gated ? sl[SL::dseg] : 1.f;
        }
#pragma unroll
      for (int k = 0; k < KB; ++k)
        if (g0 + k < nslots) {
          c = cfma(make_float2(p.x * ds[k], p.y * ds[k]), c, x[k]);
          reinterpret_cast<float2*>(base + (size_t)(g0 + k) * slot_floats + SL::eta)[m] = c;
        }
    }
    return;
  }
  const int lane = e & 63, il = lane & 15, gq = lane >> 4;
  const int mt = (e >> 6) % MH;
  const int ts = (e >> 6) / MH % (NFT + NDT);   // tile set: f tiles, then d tiles
  const int u = (e >> 6) / MH / (NFT + NDT);
  const bool is_u = ts < NFT;
  const int tile = is_u ? u + NS * ts : u + NS * (ts - NFT);
  if (tile >= (is_u ? F / 16 : D / 16)) return;   // a tile no wave owns
  float cr[4], ci[4];
  for (int q = 0; q < 4; ++q) {
    cr[q] = 0.f;
    ci[q] = 0.f;
    if (U0) {
      const int m = is_u ? 16 * mt + il : 16 * mt + 4 * gq + q;
      const float2 v = is_u ? U0[((size_t)seq * M + m) * F + 16 * tile + 4 * gq + q]
                            : G0[((size_t)seq * M + m) * D + 16 * tile + il];
      const float2 w = cmul(lamh[m], v);
      cr[q] = w.x;
      ci[q] = w.y;
    }
  }
  const long po = SL::pair(u, ts * MH + mt, lane), so = SL::scale_of(u, ts * MH + mt, lane);
  float2 pq[4];
  for (int q = 0; q < 4; ++q) pq[q] = pows[is_u ? 16 * mt + il : 16 * mt + 4 * gq + q];
  for (int g0 = 0; g0 < nslots; g0 += KB) {
    uint4 v[KB];
    float is[KB], ds[KB];
#pragma unroll
    for (int k = 0; k < KB; ++k)
      if (g0 + k < nslots) {
        const float* sl = base + (size_t)(g0 + k) * slot_floats;
        v[k] = *reinterpret_cast<const uint4*>(sl + po);
        is[k] = sl[so];
        ds[k] = gated ? sl[SL::dseg] : 1.f;
      }
    // Carried states of the batch in fp32, then their row maxima reduced together (the
    // shuffles overlap), then each quantised to its slot.
    float vr[KB][4], vi[KB][4], mx[KB];
#pragma unroll
    for (int k = 0; k < KB; ++k) {
      mx[k] = 0.f;
      if (g0 + k < nslots) {   // uniform over the wave
        float rr[4], ii[4];
        slot_unpack(v[k], is[k], rr, ii);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float xr = cr[q], yi = ci[q];
          const float px = pq[q].x * ds[k], py = pq[q].y * ds[k];
          cr[q] = px * xr - py * yi + rr[q];
          ci[q] = px * yi + py * xr + ii[q];
          vr[k][q] = cr[q];
          vi[k][q] = ci[q];
          mx[k] = fmaxf(mx[k], fmaxf(fabsf(cr[q]), fabsf(ci[q])));
        }
      }
    }
#pragma unroll
    for (int o = 1; o < 16; o <<= 1)
#pragma unroll
      for (int k = 0; k < KB; ++k) mx[k] = fmaxf(mx[k], __shfl_xor(mx[k], o, 16));
#pragma unroll
    for (int k = 0; k < KB; ++k)
      if (g0 + k < nslots) {
        float* sl = base + (size_t)(g0 + k) * slot_floats;
        const float sc = pow2_scale(mx[k]);
        const uint2 r = pack4_f16(vr[k][0] * sc, vr[k][1] * sc, vr[k][2] * sc, vr[k][3] * sc);
        const uint2 i = pack4_f16(vi[k][0] * sc, vi[k][1] * sc, vi[k][2] * sc, vi[k][3] * sc);
        *reinterpret_cast<uint4*>(sl + po) = make_uint4(r.x, r.y, i.x, i.y);
        if (il == 0) sl[so] = 1.f / sc;
      }
  }
}

template <int F, int D, int M>
static hipError_t launch_carry_t(const ChunkPrefillArgs& p, long tb, long pows_off, int nslots,
                                 long slot_floats, hipStream_t st) {
  using SL = SlotLayout<F, D, M>;
  constexpr int n = SL::NS * (SL::NFT + SL::NDT) * (M / 16) * 64 + M;
  const int seqs = p.B * p.H;
  (void)hipGetLastError();
  prof_begin(st);
  hipLaunchKernelGGL((carry_slots_kernel<F, D, M>),
                     dim3((n + 255) / 256, p.slots_rev ? 2 * seqs : seqs), dim3(256), 0, st,
                     p.slots, p.slots_rev, seqs, p.U0, p.G0, p.E0, p.lam, p.tables, tb, pows_off,
                     p.H, nslots, slot_floats, p.wgate != nullptr);
  prof_end(st, kKindCarry);
  return hipGetLastError();
}

static hipError_t launch_carry(const ChunkPrefillArgs& p, long tb, long pows_off, int nslots,
                               long slot_floats, hipStream_t st) {
#define IA_CARRY(FF, MM) \
  if (p.F == FF && p.D == FF && p.M == MM)   \
    return launch_carry_t<FF, FF, MM>(p, tb, pows_off, nslots, slot_floats, st);
  IA_CARRY(32, 16) IA_CARRY(32, 32) IA_CARRY(32, 64)
  IA_CARRY(64, 16) IA_CARRY(64, 32) IA_CARRY(64, 64)
  IA_CARRY(128, 16) IA_CARRY(128, 32) IA_CARRY(128, 64)
#undef IA_CARRY
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------- launch

template <int C>
static hipError_t dispatch_fdm(const ChunkArgs& a, int F, int D, int M, int n_wg,
                               hipStream_t st, int kind) {
  const bool gt = a.wgate != nullptr;
#define IA_CASE(FF, MM)                                                                 \
  if (F == FF && D == FF && M == MM)                                                    \
    return gt ? launch_chunk_t<C, FF, FF, MM, false, true>(a, n_wg, st, kind)           \
              : launch_chunk_t<C, FF, FF, MM>(a, n_wg, st, kind);
  IA_CASE(32, 16) IA_CASE(32, 32) IA_CASE(32, 64)
  IA_CASE(64, 16) IA_CASE(64, 32) IA_CASE(64, 64)
  IA_CASE(128, 16) IA_CASE(128, 32) IA_CASE(128, 64)
#undef IA_CASE
  return hipErrorInvalidValue;
}

template <int C>
static hipError_t dispatch_fdm_rm(const ChunkArgs& a, int F, int D, int M, int n_wg,
                                  hipStream_t st, int kind) {
#define IA_CASE(FF, MM)                                   \
  if (F == FF && D == FF && M == MM) return launch_chunk_t<C, FF, FF, MM, true>(a, n_wg, st, kind);
  IA_CASE(32, 16) IA_CASE(32, 32) IA_CASE(32, 64)
  IA_CASE(64, 16) IA_CASE(64, 32) IA_CASE(64, 64)
  IA_CASE(128, 16) IA_CASE(128, 32)
  if constexpr (C == 32) {
    IA_CASE(128, 64)
  }
#undef IA_CASE
  return hipErrorInvalidValue;
}

template <int C>
static hipError_t dispatch_state_fdm(const ChunkArgs& a, int F, int D, int M, int n_wg,
                                     hipStream_t st, int kind) {
  const bool gt = a.wgate != nullptr;
#define IA_CASE(FF, MM)                                                                 \
  if (F == FF && D == FF && M == MM)                                                    \
    return gt ? launch_state_t<C, FF, FF, MM, true>(a, n_wg, st, kind)                  \
              : launch_state_t<C, FF, FF, MM>(a, n_wg, st, kind);
  IA_CASE(32, 16) IA_CASE(32, 32) IA_CASE(32, 64)
  IA_CASE(64, 16) IA_CASE(64, 32) IA_CASE(64, 64)
  IA_CASE(128, 16) IA_CASE(128, 32) IA_CASE(128, 64)
#undef IA_CASE
  return hipErrorInvalidValue;
}

template <int C, int M>
static hipError_t launch_tables_cm(const ChunkPrefillArgs& p, long tb, hipStream_t st) {
  const int Lt = p.N % C == 0 ? C : p.N % C;
  (void)hipGetLastError();
  prof_begin(st);
  hipLaunchKernelGGL((chunk_tables_kernel<C, M>), dim3(p.H, C / 4), dim3(4 * M), 0, st,
                     p.lam, p.beta, p.tables, tb, Lt, p.seg_chunks * C, p.readout ? 1 : 0,
                     p.readout, p.rtab, readout_table_bytes(M));
  prof_end(st, kKindTables);
  return hipGetLastError();
}

template <int C>
static hipError_t launch_tables_c(const ChunkPrefillArgs& p, long tb, hipStream_t st) {
  switch (p.M) {
    case 16: return launch_tables_cm<C, 16>(p, tb, st);
    case 32: return launch_tables_cm<C, 32>(p, tb, st);
    case 64: return launch_tables_cm<C, 64>(p, tb, st);
  }
  return hipErrorInvalidValue;
}

bool chunk_supported(int F, int D, int M) {
  return F == D && (F == 32 || F == 64 || F == 128) && (M == 16 || M == 32 || M == 64);
}

long chunk_table_bytes(int chunk, int M) {
  switch (chunk * 1000 + M) {
    case 32016: return TableLayout<32, 16>::bytes;
    case 32032: return TableLayout<32, 32>::bytes;
    case 32064: return TableLayout<32, 64>::bytes;
    case 64016: return TableLayout<64, 16>::bytes;
    case 64032: return TableLayout<64, 32>::bytes;
    case 64064: return TableLayout<64, 64>::bytes;
  }
  return 0;
}

int chunk_wgs_per_cu(int chunk, int F, int D, int M, bool rm, bool gated) {
  if (gated) {
#define IA_OCC(CC, FF, MM) \
  if (chunk == CC && F == FF && D == FF && M == MM) return chunk_occupancy_t<CC, FF, FF, MM, false, true>();
    IA_OCC(32, 32, 16) IA_OCC(32, 32, 32) IA_OCC(32, 32, 64)
    IA_OCC(32, 64, 16) IA_OCC(32, 64, 32) IA_OCC(32, 64, 64)
    IA_OCC(32, 128, 16) IA_OCC(32, 128, 32) IA_OCC(32, 128, 64)
    IA_OCC(64, 32, 16) IA_OCC(64, 32, 32) IA_OCC(64, 32, 64)
    IA_OCC(64, 64, 16) IA_OCC(64, 64, 32) IA_OCC(64, 64, 64)
    IA_OCC(64, 128, 16) IA_OCC(64, 128, 32) IA_OCC(64, 128, 64)
#undef IA_OCC
    return 0;
  }
  if (rm) {
#define IA_OCC(CC, FF, MM) \
  if (chunk == CC && F == FF && D == FF && M == MM) return chunk_occupancy_t<CC, FF, FF, MM, true>();
    IA_OCC(32, 32, 16) IA_OCC(32, 32, 32) IA_OCC(32, 32, 64)
    IA_OCC(32, 64, 16) IA_OCC(32, 64, 32) IA_OCC(32, 64, 64)
    IA_OCC(32, 128, 16) IA_OCC(32, 128, 32) IA_OCC(32, 128, 64)
    IA_OCC(64, 32, 16) IA_OCC(64, 32, 32) IA_OCC(64, 32, 64)
    IA_OCC(64, 64, 16) IA_OCC(64, 64, 32) IA_OCC(64, 64, 64)
    IA_OCC(64, 128, 16) IA_OCC(64, 128, 32)
#undef IA_OCC
    return 0;
  }
#define IA_OCC(CC, FF, MM) \
  if (chunk == CC && F == FF && D == FF && M == MM) return chunk_occupancy_t<CC, FF, FF, MM>();
  IA_OCC(32, 32, 16) IA_OCC(32, 32, 32) IA_OCC(32, 32, 64)
  IA_OCC(32, 64, 16) IA_OCC(32, 64, 32) IA_OCC(32, 64, 64)
  IA_OCC(32, 128, 16) IA_OCC(32, 128, 32) IA_OCC(32, 128, 64)
  IA_OCC(64, 32, 16) IA_OCC(64, 32, 32) IA_OCC(64, 32, 64)
  IA_OCC(64, 64, 16) IA_OCC(64, 64, 32) IA_OCC(64, 64, 64)
  IA_OCC(64, 128, 16) IA_OCC(64, 128, 32) IA_OCC(64, 128, 64)
#undef IA_OCC
  return 0;
}

static long pows_offset(int chunk, int M) {
  switch (chunk * 1000 + M) {
    case 32016: return TableLayout<32, 16>::oPowS;
    case 32032: return TableLayout<32, 32>::oPowS;
    case 32064: return TableLayout<32, 64>::oPowS;
    case 64016: return TableLayout<64, 16>::oPowS;
    case 64032: return TableLayout<64, 32>::oPowS;
    case 64064: return TableLayout<64, 64>::oPowS;
  }
  return 0;
}

long chunk_slot_floats(int F, int D, int M) {
#define IA_SLOT(FF, MM) \
  if (F == FF && D == FF && M == MM) return SlotLayout<FF, FF, MM>::floats;
  IA_SLOT(32, 16) IA_SLOT(32, 32) IA_SLOT(32, 64)
  IA_SLOT(64, 16) IA_SLOT(64, 32) IA_SLOT(64, 64)
  IA_SLOT(128, 16) IA_SLOT(128, 32) IA_SLOT(128, 64)
#undef IA_SLOT
  return 0;
}

// Up to this many predecessor slots an output workgroup combines itself (Horner); beyond, a
// carry kernel writes inclusive states first.
constexpr int kHornerSlots = 3;

// Full chunked prefill for one direction (or, with p.slots_rev set, both walks of a
// bidirectional call): tables; the end states of segments 0..G-2 from a zero state; every
// segment (or, state only, the last) from its initial state, which each workgroup assembles
// from the caller's state and the earlier segments' end states.  With several segments the
// tables are computed by extra workgroups of the state-only launch (which itself does not read
// them), so they cost no launch of their own on the way to the output pass.  A bidirectional
// call runs one state-only launch and one carry for both walks (the tables serve both), then
// the forward output pass, which writes o, and the reverse one, which adds onto it.
hipError_t launch_chunk_prefill(const ChunkPrefillArgs& p, hipStream_t st) {
  const int C = p.chunk;
  const int n_chunks = (p.N + C - 1) / C;
  const int seqs = p.B * p.H;
  const int G = p.segments;
  const int seg_chunks = p.seg_chunks;
  const long tb = chunk_table_bytes(C, p.M);
  const bool both = p.slots_rev != nullptr;
  if (G < 1 || (G - 1) * seg_chunks >= n_chunks || G * seg_chunks < n_chunks)
    return hipErrorInvalidValue;
  if (both && (p.reverse || p.accumulate || p.U0 || !p.o)) return hipErrorInvalidValue;

  hipError_t e = hipSuccess;
  if (G == 1) {
    e = C == 64 ? launch_tables_c<64>(p, tb, st) : launch_tables_c<32>(p, tb, st);
    if (e != hipSuccess) return e;
  }

  ChunkArgs a{};
  a.q = static_cast<const uint16_t*>(p.q);
  a.k = static_cast<const uint16_t*>(p.k);
  a.v = static_cast<const uint16_t*>(p.v);
  a.sqk = p.sqk;
  a.sv = p.sv;
  a.lam = p.lam;
  a.beta = p.beta;
  a.N = p.N;
  a.H = p.H;
  a.B = p.B;
  // token rows of 32 bf16 features are half a cache line: order the workgroups so neighbouring
  // heads share each line's fetch (pair_wg)
  const bool pairs = (p.F < 64 || p.D < 64) && p.H % 2 == 0;
  a.pair_heads = pairs;
  a.seg_chunks = seg_chunks;
  a.dir = p.reverse;
  a.out_bf16 = p.out_bf16;
  a.clamp = p.clamp;
  a.opt = p.opt;
  a.den_w = (p.opt & kOptNoDen) ? 0.f : 1.f;
  a.den_c = (p.opt & kOptNoDen) ? 1.f : p.clamp;
  a.slot_floats = chunk_slot_floats(p.F, p.D, p.M);
  a.slots_per_seq = G - 1;
  a.tables = p.tables;
  a.table_bytes = tb;
  a.tables_half = p.readout ? 1 : 0;
  a.readout = p.readout;
  a.rtab = p.rtab;
  a.rtab_bytes = readout_table_bytes(p.M);
  a.wU = p.wU;
  a.wG = p.wG;
  a.wE = p.wE;
  a.wgate = p.wgate;
  a.dgate = p.dgate;

  auto go = [&](const ChunkArgs& x, int n_wg, int kind) -> hipError_t {
    if (p.readout)
      return C == 64 ? dispatch_fdm_rm<64>(x, p.F, p.D, p.M, n_wg, st, kind)
                     : dispatch_fdm_rm<32>(x, p.F, p.D, p.M, n_wg, st, kind);
    return C == 64 ? dispatch_fdm<64>(x, p.F, p.D, p.M, n_wg, st, kind)
                   : dispatch_fdm<32>(x, p.F, p.D, p.M, n_wg, st, kind);
  };

  bool inclusive = false;
  if (G > 1) {
    // Pass 1: end state of segments 0..G-2 from a zero state (both walks in one launch for a
    // bidirectional call).  The launch also computes the tables: one more workgroup per head.
    ChunkArgs s = a;
    s.seg_first = 0;
    s.n_seg = G - 1;
    s.seg_end = p.slots;
    s.seg_end_rev = p.slots_rev;
    s.n_dir_wg = pair_wg_count(seqs, G - 1, pairs);
    s.tables_out = p.tables;
    s.rtab_out = p.readout ? p.rtab : nullptr;
    s.n_sum_wg = s.n_dir_wg * (both ? 2 : 1);
    s.Lt = p.N % C == 0 ? C : p.N % C;
    const int n_wg = s.n_sum_wg + p.H;
    e = C == 64 ? dispatch_state_fdm<64>(s, p.F, p.D, p.M, n_wg, st, kKindSummary)
                : dispatch_state_fdm<32>(s, p.F, p.D, p.M, n_wg, st, kKindSummary);
    if (e != hipSuccess) return e;
    // With many segments, carry once (each slot read and written once) instead of letting
    // every output workgroup combine all of its predecessors' slots.
    if (G - 1 > kHornerSlots) {
      e = launch_carry(p, tb, pows_offset(C, p.M), G - 1, a.slot_floats, st);
      if (e != hipSuccess) return e;
      inclusive = true;
    }
  }
  // Pass 2: every segment from its initial state, with outputs; the last segment returns the
  // final state.  State-only calls run just the last segment.  With several segments each
  // running, the caller's initial state is read from a copy in the workspace: the last
  // segment's workgroup writes the final state into the caller's buffers while the others may
  // still be reading their initial state.
  ChunkArgs o = a;
  o.seg_prev = G > 1 ? p.slots : nullptr;
  o.seg_inclusive = inclusive;
  o.init0_U = p.U0;
  o.init0_G = p.G0;
  o.init0_E = p.E0;
  if (p.U0 && p.o && G > 1) {
    const size_t bh = (size_t)p.B * p.H;
    e = launch_copy3(p.wU, p.U0, bh * p.M * p.F * 8, p.wG, p.G0, bh * p.M * p.D * 8, p.wE, p.E0,
                     bh * p.M * 8, st);
    if (e != hipSuccess) return e;
    o.init0_U = p.wU;
    o.init0_G = p.wG;
    o.init0_E = p.wE;
  }
  o.o = p.o;
  o.accumulate = p.accumulate;
  o.fin_U = p.U1;
  o.fin_G = p.G1;
  o.fin_E = p.E1;
  o.seg_first = p.o ? 0 : G - 1;
  o.n_seg = p.o ? G : 1;
  const int n_out = pair_wg_count(seqs, o.n_seg, pairs);
  e = go(o, n_out, kKindChunk);
  if (e != hipSuccess || !both) return e;
  // The reverse walk: its slots, adding onto the forward walk's outputs.
  o.dir = 1;
  o.accumulate = 1;
  o.seg_prev = G > 1 ? p.slots_rev : nullptr;
  return go(o, n_out, kKindChunk);
}

}  // namespace ia
