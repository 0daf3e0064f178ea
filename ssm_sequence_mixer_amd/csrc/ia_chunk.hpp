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
//   lam U_{c+1} = lam^L (lam U_c + sum_j beta lam^-j phi(k_j)), same for G with v, eta with 1.
// Complex matrices enter real MFMAs as [Re | Im] blocks of 2M real columns.
//
// Workgroup = one (b, h, segment, direction); 64*(C/16 + NS) threads:
//   readout waves r < C/16 own the 16 queries [16r, 16r+16) of each chunk and chain
//     S^T -> A'^T -> P^T -> num^T through MFMA accumulators (an accumulator tile of X is the
//     operand of X^T, with the K index permuted identically on both operands);
//   state waves own columns of the fp32 state (held as lam U, lam G), kept in MFMA
//     accumulators for the whole segment, update it with two MFMA contractions per chunk,
//     publish operand copies of the new state (bf16 lam U, fp16 lam G scaled per column), and
//     fetch the next chunk's q, k into registers while the current chunk computes (the
//     readout waves fetch v).  Two barriers per chunk separate a first phase (S, A' and the
//     lam U update) from a second (P, the numerator and the lam G update).
// Operand precision: features, S, the decay table, U, P and v in bf16; A, beta lam^-j and G
// in fp16 after exact power-of-two scaling (per query row for A; per value column for G; per
// head for the table), which keeps the readout's cancelling sums within the bf16 tolerance.
// LDS operands are read as one 16-byte access per lane, or as two transposing 8-byte reads
// (ds_read_b64_tr_b16) for phi(k) and v, which are stored once, row-major: the transposing
// read returns 4 consecutive rows of one column per lane, exactly the K-slot order of an
// accumulator-sourced partner.  Tables paired with such a partner store their K axis in that
// slot order, and 16-byte blocks are XOR-swizzled by row so one read hits distinct banks.
#pragma once

#include <utility>

#include "ia_device.hpp"
#include "ia_kernels.hpp"
#include "ia_scan.hpp"

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
__device__ __forceinline__ bf16x8 pack_bf16(f32x4 a, f32x4 b) {
  bf16x8 r;
  r[0] = (__bf16)a[0]; r[1] = (__bf16)a[1]; r[2] = (__bf16)a[2]; r[3] = (__bf16)a[3];
  r[4] = (__bf16)b[0]; r[5] = (__bf16)b[1]; r[6] = (__bf16)b[2]; r[7] = (__bf16)b[3];
  return r;
}

// Two floats -> packed bf16 / fp16 pair (hardware round-to-nearest-even conversions).
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
  typedef __bf16 v2 __attribute__((ext_vector_type(2)));
  const v2 r = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ uint32_t pk_f16(float a, float b) {
  typedef _Float16 v2 __attribute__((ext_vector_type(2)));
  const v2 r = {(_Float16)a, (_Float16)b};
  return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ uint2 pack4_bf16(float a, float b, float c, float d) {
  return make_uint2(pk_bf16(a, b), pk_bf16(c, d));
}
__device__ __forceinline__ uint2 pack4_f16(float a, float b, float c, float d) {
  return make_uint2(pk_f16(a, b), pk_f16(c, d));
}

// K-slot order of an operand built from two 16x16 accumulator tiles: slot 8g+e of a 32-wide K
// block holds index 4g+e (e < 4, first tile) or 16+4g+e-4 (second tile).  kpos maps an index
// to its slot; four consecutive indices starting at a multiple of 4 stay consecutive.
__host__ __device__ constexpr int kpos(int l) {
  return (l & ~31) | (8 * ((l & 15) >> 2) + 4 * ((l >> 4) & 1) + (l & 3));
}

// XOR swizzle of the 16-byte blocks of a row of RL 16-bit elements: rows 0..15 of one
// operand read (same logical block) land in 16 distinct 16-byte bank groups.
template <int RL>
__host__ __device__ constexpr int swz(int row) {
  constexpr int nb = RL / 8;
  static_assert(nb == 4 || nb == 8 || nb == 16, "row of 32, 64 or 128 elements");
  if constexpr (nb == 16) return row & 15;
  else if constexpr (nb == 8) return (row >> 1) & 7;
  else return (row >> 2) & 3;
}
// Element offset of (row, col) in a swizzled [rows][RL] matrix (col already in slot order).
template <int RL>
__host__ __device__ constexpr int soff(int row, int col) {
  return row * RL + ((((col >> 3) ^ swz<RL>(row)) << 3) | (col & 7));
}

// Scheduling fence: keeps the loads of later unrolled steps from being hoisted above it, so
// register use stays per step (latency is covered by the other waves on the SIMD instead).
#define IA_STEP_FENCE() __builtin_amdgcn_sched_barrier(0)

// Offset of row `row` (0..15), 8-element block `blk` in a swizzled [..][RL] matrix.  Rows
// 16t + row for any t have the same swizzle, so tile t of a 16-row operand is this offset
// plus the compile-time constant 16 t RL: per-lane address registers stay few (one per
// K step), the tile offsets become instruction immediates.
template <int RL>
__device__ __forceinline__ int lane_off(int row, int blk) {
  return row * RL + ((blk ^ swz<RL>(row)) << 3);
}

// Keeps a per-lane LDS offset out of constant folding.  Several matrices start past 64 KiB,
// beyond the 16-bit immediate of ds_read/ds_write; folded with a tile offset into one constant
// the sum no longer fits the immediate and costs a register per tile.  With the matrix base
// inside the opaque value, tile offsets (< 64 KiB) stay immediates.
__device__ __forceinline__ int opaque(int v) {
  asm volatile("" : "+v"(v));
  return v;
}

typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s* lds_v4s_ptr;

// Operand of a contraction over the rows of a row-major swizzled [K][RL] matrix, in the K-slot
// order of an accumulator-sourced partner: lane (il, g) gets column 16ct + il at rows
// 32kb + 4g + {0..3} (slots 0..3) and 32kb + 16 + 4g + {0..3} (slots 4..7).  Each
// ds_read_b64_tr_b16 of a 16-lane group reads a 4-row x 16-column block (lane l: row l/4,
// columns 4(l%4)..+3) and hands lane l column l of it.  tr_off gives the per-lane part for
// column tile ct; row blocks kb add 32 kb RL (the swizzle of row r depends on r mod 16 only).
template <int RL>
__device__ __forceinline__ int tr_off(int ct, int lane) {
  const int g = lane >> 4, lam = lane & 15;
  const int row = 4 * g + (lam >> 2);
  const int col = 16 * ct + 4 * (lam & 3);
  return row * RL + ((((col >> 3) ^ swz<RL>(row)) << 3) | (col & 7));
}
template <int RL>
__device__ __forceinline__ Frag ldtr(const uint16_t* base, int off, int kb) {
  const v4s a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_v4s_ptr)(base + off + 32 * kb * RL));
  const v4s b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_v4s_ptr)(base + off + (32 * kb + 16) * RL));
  Frag f;
  f.u = make_uint4(uint32_t(uint16_t(a[0])) | (uint32_t(uint16_t(a[1])) << 16),
                   uint32_t(uint16_t(a[2])) | (uint32_t(uint16_t(a[3])) << 16),
                   uint32_t(uint16_t(b[0])) | (uint32_t(uint16_t(b[1])) << 16),
                   uint32_t(uint16_t(b[2])) | (uint32_t(uint16_t(b[3])) << 16));
  return f;
}

// Power of two s with s * mx in [2^14, 2^15): maps the largest magnitude of a row or column
// near the top of the fp16 range.  mx == 0 or not finite: 1.
__device__ __forceinline__ float pow2_scale(float mx) {
  if (!(mx > 0.f) || !(mx < 3.0e38f)) return 1.f;
  const int e = ilogbf(mx);               // mx in [2^e, 2^(e+1))
  return ldexpf(1.f, 14 - e);
}

// Sum (max) of a value over lanes l, l^16, l^32, l^48 (one column of the four 16-lane rows), in
// every lane, by two cross-row swaps on the VALU instead of LDS permutes: permlane16_swap(v, v)
// returns v with rows 1, 3 replaced by rows 0, 2 and v with rows 0, 2 replaced by rows 1, 3,
// whose sum pairs rows 0+1 and 2+3; permlane32_swap(v, v) likewise pairs the two halves.  Each
// lane adds the same two values in the same order as with shuffles, so results are unchanged.
__device__ __forceinline__ float xor_sum16_32(float v) {
  const unsigned b = __float_as_uint(v);
  const auto p = __builtin_amdgcn_permlane16_swap(b, b, false, false);
  const unsigned c = __float_as_uint(__uint_as_float(p[0]) + __uint_as_float(p[1]));
  const auto q = __builtin_amdgcn_permlane32_swap(c, c, false, false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}
__device__ __forceinline__ float xor_max16_32(float v) {
  const unsigned b = __float_as_uint(v);
  const auto p = __builtin_amdgcn_permlane16_swap(b, b, false, false);
  const unsigned c = __float_as_uint(fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1])));
  const auto q = __builtin_amdgcn_permlane32_swap(c, c, false, false);
  return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
}

// ---------------------------------------------------------------- wave roles
// C/16 readout waves and NS state waves.  The widest shapes use 8 state waves (12 waves per
// workgroup, 3 per SIMD) so that each state wave's share of the fp32 state plus its share of
// the next chunk's inputs fits its registers; the others use 4.
template <int F, int D, int M>
struct StateWaves {
  static constexpr int NS = (F + D >= 256 && M >= 64) ? 8 : 4;
};

// Workspace slot of one segment's end state (times lam), in the state waves' accumulator
// layout and in fp16: for wave u and tile pair p = (tile set ts, mode tile mt) -- accumulator
// tiles ts TM + mt (Re) and ts TM + mt + M/16 (Im), tile sets f tiles then d tiles -- lane l
// holds 16 bytes at float offset pair(u, p, l): its 4 Re then 4 Im values times 2^s, one
// power of two per (u, p) and 16-lane row l/16 that puts the row's largest magnitude in
// [2^14, 2^15).  Then 2^-s per (u, p, row) (fp32) and lam eta (complex fp32, per mode).
// fp16 halves the bytes every workgroup of a later segment reads; its relative rounding
// (2^-11 of the row's largest value) is finer than the bf16 / scaled-fp16 operands the
// readout forms from the state.
template <int F, int D, int M>
struct SlotLayout {
  static constexpr int NS = StateWaves<F, D, M>::NS;
  static constexpr int NFT = (F / 16 + NS - 1) / NS, NDT = (D / 16 + NS - 1) / NS;
  static constexpr int TM = 2 * M / 16, MH = M / 16;
  static constexpr int NP = (NFT + NDT) * MH;           // tile pairs per wave
  static constexpr long scale = (long)NS * NP * 64 * 4;  // float offset of the 2^-s
  static constexpr long eta = scale + NS * NP * 4;       // float offset of lam eta
  static constexpr long dseg = eta + 2L * M;             // gated layer: the segment's decay
                                                         // product (prod of its a_t)
  static constexpr long floats = dseg + 4;
  static_assert(scale % 4 == 0 && eta % 4 == 0 && floats % 4 == 0, "16-byte aligned slots");
  __device__ static long pair(int u, int p, int lane) {
    return ((long)(u * NP + p) * 64 + lane) * 4;
  }
  __device__ static long scale_of(int u, int p, int lane) {
    return scale + (u * NP + p) * 4 + (lane >> 4);
  }
};

// Largest |value| over the 8 values of every lane of this lane's 16-lane row (all 16 active).
__device__ __forceinline__ float row_absmax8(const float (&re)[4], const float (&im)[4]) {
  float mx = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) mx = fmaxf(mx, fmaxf(fabsf(re[q]), fabsf(im[q])));
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 16));
  return mx;
}

// One tile pair of a slot, written by whole 16-lane rows: pair_off = SlotLayout::pair(u, p,
// lane), scale_off = SlotLayout::scale_of(u, p, lane).
__device__ __forceinline__ void slot_put(float* slot, long pair_off, long scale_off, int lane,
                                         const float (&re)[4], const float (&im)[4]) {
  const float s = pow2_scale(row_absmax8(re, im));
  const uint2 r = pack4_f16(re[0] * s, re[1] * s, re[2] * s, re[3] * s);
  const uint2 i = pack4_f16(im[0] * s, im[1] * s, im[2] * s, im[3] * s);
  *reinterpret_cast<uint4*>(slot + pair_off) = make_uint4(r.x, r.y, i.x, i.y);
  if ((lane & 15) == 0) slot[scale_off] = 1.f / s;
}

__device__ __forceinline__ float f16_lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// One tile pair of a slot (its 16 bytes v and inverse scale is), back in fp32.
__device__ __forceinline__ void slot_unpack(uint4 v, float is, float (&re)[4], float (&im)[4]) {
  re[0] = f16_lo(v.x) * is;
  re[1] = f16_hi(v.x) * is;
  re[2] = f16_lo(v.y) * is;
  re[3] = f16_hi(v.y) * is;
  im[0] = f16_lo(v.z) * is;
  im[1] = f16_hi(v.z) * is;
  im[2] = f16_lo(v.w) * is;
  im[3] = f16_hi(v.w) * is;
}

// One tile pair of a slot, back in fp32.
__device__ __forceinline__ void slot_get(const float* slot, long pair_off, long scale_off,
                                         float (&re)[4], float (&im)[4]) {
  slot_unpack(*reinterpret_cast<const uint4*>(slot + pair_off), slot[scale_off], re, im);
}

// ---------------------------------------------------------------- LDS layout

template <int C, int F, int D, int M, int NR, bool RM = false, bool GT = false>
struct Layout {
  static constexpr int M2 = 2 * M;
  // 16-bit element offsets; every matrix is swizzled by row (see soff).
  static constexpr int oFk = 0;                    // [C][F]   bf16 phi(k)           (f order)
  static constexpr int oFq = oFk + C * F;          // [C][F]   bf16 phi(q)           (f order)
  static constexpr int oV = oFq + C * F;           // [C][D]   bf16 v                (d order)
  static constexpr int oWT = oV + C * D;           // [2M][C]  bf16 beta lam^-j      (j slots)
  static constexpr int oWb = oWT + M2 * C;         // [C][2M]  fp16 scaled beta lam^-j (k slots)
  static constexpr int oLU = oWb + C * M2;         // [2M][F]  bf16 lam U_c          (f order)
  static constexpr int oGT = oLU + M2 * F;         // [D][2M]  fp16 c_d lam G_c      (k slots)
  static constexpr int oR = oGT + D * M2;          // [2M][2M] fp16 scaled readout matrix
                                                   //          (k slots; RM only)
  static constexpr int n16 = oR + (RM ? M2 * M2 : 0);
  // 32-bit arrays (byte offsets)
  static constexpr int bC = n16 * 2;               // [D]  float  c_d
  static constexpr int bCi = bC + D * 4;           // [D]  float  1 / c_d
  static constexpr int bLE = bCi + D * 4;          // [M]  float2 lam eta_c
  static constexpr int bPowL = bLE + M * 8;        // [M]  float2 lam^C
  static constexpr int bGeo = bPowL + M * 8;       // [M]  float2 sum_{j<C} beta lam^-j
  static constexpr int bPowT = bGeo + M * 8;       // [M]  float2 lam^Lt, last (partial) chunk
  static constexpr int bGeoT = bPowT + M * 8;      // [M]  float2 sum_{j<Lt} beta lam^-j
  static constexpr int kTail = bPowT - bPowL;      // offset of the last chunk's pair
  static constexpr int bPowS = bGeoT + M * 8;      // [M]  float2 lam^Ls, segment length Ls
  static constexpr int L2S = M + 2;                // row stride of the lam^(2i) factor table
  static constexpr int bL2lo = bPowS + M * 8;      // [16][L2S] float2 lam^(2i), i = 0..15
  static constexpr int bL2hi = bL2lo + 16 * L2S * 8;  // [NR][M] float2 lam^(32r)
  static constexpr int bL2end = bL2hi + NR * M * 8;
  // Gated layer: two buffers of a chunk's gate records (GateRec), chunk c in buffer c % 2.
  static constexpr int bRec = bL2end;
  static constexpr int recBytes = (3 * C + 4) * 4;
  static constexpr int bytes = bRec + (GT ? 2 * recBytes : 0);
};

// Gate records of one chunk (gated layer), float offsets within a record buffer.  With a_s, w_s
// the decay and write gates of the chunk's tokens s = 0..C-1 in walk order (a = 1, w = 0 past
// the sequence end), L_j = sum_{s<=j} log2|a_s| and sigma_j the sign of prod_{s<=j} a_s:
//   L[j] = L_j,   W[j] = sigma_j w_j,
//   E[j] = w_j prod_{s=j+1}^{C-1} a_s = sigma_{C-1} W[j] 2^(L_{C-1} - L_j),
//   D    = prod_s a_s = sigma_{C-1} 2^(L_{C-1}).
// Then w_j prod_{s=j+1}^{i} a_s = sigma_i W[j] 2^(L_i - L_j) and prod_{s<=i} a_s =
// sigma_i 2^(L_i); the factor sigma_i of query i multiplies its numerator and denominator
// alike and is dropped.  |a| below 2^-64 counts as 2^-64 (the log stays finite).
template <int C>
struct GateRec {
  static constexpr int L = 0, W = C, E = 2 * C, D = 3 * C, floats = 3 * C + 4;
};

struct ChunkArgs {
  const uint16_t *q, *k, *v;   // bf16, element (b, n, h) strides sqk (q and k) and sv; the
  RowStrides sqk, sv;          // feature axis contiguous
  const float2 *lam, *beta;    // [H][M]
  void* o;                     // [B][N][H][D] or NULL (state only)
  int accumulate;              // add to the values o holds (second bidirectional direction)
  int N, H;
  int seg_chunks;              // chunks per segment
  int seg_first;               // first segment index handled by this launch
  int n_seg;                   // segments in this launch, per sequence
  int pair_heads;              // workgroup order pairs heads 2j, 2j+1 (pair_wg)
  int dir;                     // 1: the walk runs from position N-1 down to 0
  int out_bf16;
  float clamp;
  int opt;                     // kOptNoDen | kOptIdentity
  float den_w, den_c;          // 1 and clamp; with kOptNoDen 0 and 1 (the readout divisor)
  // Initial state of segment g: the caller's state init0 (or zeros) carried across segments
  // 0..g-1, whose end states (each computed from a zero state) are the workspace slots
  // seg_prev[seq][0..g-1]: state <- lam^Ls state + slot, Ls the segment length (with
  // seg_inclusive, slot seg_prev[seq][g-1] is already that state).  Final state:
  // with seg_end set, segment g writes slot seg_end[seq][g]; otherwise the segment holding
  // the last token writes the caller's fin (if set).  Slots hold lam U, lam G and lam eta in
  // the state waves' accumulator layout (SlotLayout).
  const float2 *init0_U, *init0_G, *init0_E;   // caller layout: [seq][M][F] etc.
  float2 *fin_U, *fin_G, *fin_E;               // caller layout
  // Heads whose tables carry the route flag run the fp32 recurrence instead: the first
  // workgroup of the head in this launch walks the whole sequence, in place on fin_* (which
  // then hold the initial state) or, without a caller state, on the zeroed workspace state
  // wU/wG/wE (same layout).
  float2 *wU, *wG, *wE;
  // Gated layer: write and decay gates, float [B][N][H] (element (b, n, h) at (b N + n) H + h).
  const float *wgate, *dgate;
  const float* seg_prev;
  int seg_inclusive;                           // seg_prev[g] already holds the state entering
                                               // segment g+1 (caller state included)
  float* seg_end;
  // State-only pass of a bidirectional call: the reverse walk's slots, and the workgroups per
  // walk (the first n_dir_wg walk forward, the next n_dir_wg backward into seg_end_rev).
  float* seg_end_rev;
  int n_dir_wg;
  long slot_floats;                            // floats per slot
  int slots_per_seq;
  const unsigned char* tables;                 // per-head tables (chunk_tables_kernel)
  long table_bytes;                            // bytes per head
  int tables_half;                             // factor tables of lam^i (readout matrix)
                                               // instead of lam^(2i)
  // Readout matrix (kernels instantiated with RM): R [H][M][M] for the fp32 route, and its
  // per-head MFMA operand (readout_table_kernel): fp16 [2M][2M], then 1 / its scale.
  const float2* readout;
  const unsigned char* rtab;
  long rtab_bytes;
  unsigned char* rtab_out;   // state-only pass: its table workgroups also write rtab
  // State-only pass: workgroups past the first n_sum_wg compute the per-head tables (one
  // workgroup per head, table_run) into tables_out, Lt the last chunk's length.
  unsigned char* tables_out;
  int n_sum_wg;
  int B;                                       // batch (sequences = B H)
  int Lt;
};

// Per-head tables, computed once per call by table_run, in the state-only pass's launch or in
// chunk_tables_kernel (byte offsets).  The two decay tables and the two lam^(2i) factor
// tables are stored exactly as in LDS.
template <int C, int M>
struct TableLayout {
  static constexpr int NR = C / 16;
  static constexpr long oW = 0;                       // bf16 [2M][C] then fp16 [C][2M]
  static constexpr long nW = 2L * (2L * M * C + (long)C * 2 * M);
  static constexpr long oL2 = oW + nW;                // [16][M+2] then [NR][M] float2
  static constexpr long nL2 = 8L * (16L * (M + 2) + (long)NR * M);
  static constexpr long oPow = oL2 + nL2;             // float2 [M]: lam^C
  static constexpr long oGeo = oPow + 8L * M;         // float2 [M]: sum_{j<C} beta lam^-j
  static constexpr long oPowT = oGeo + 8L * M;        // float2 [M]: lam^Lt, last chunk
  static constexpr long oGeoT = oPowT + 8L * M;       // float2 [M]: sum_{j<Lt} beta lam^-j
  static constexpr long oPowS = oGeoT + 8L * M;       // float2 [M]: lam^(segment length)
  static constexpr long oInv = oPowS + 8L * M;        // float2 [M]: 1 / lam
  static constexpr long oSc = oInv + 8L * M;          // float: 1 / fp16 table scale
  static constexpr long oRoute = oSc + 4;             // int: 1 = the head takes the fp32 route
  static constexpr long bytes = (oSc + 16 + 255) / 256 * 256;
};

// Per-head MFMA operand of the readout matrix R (readout_table_kernel).  With the query-mode
// row a = lam^i A' held as the operand [Re a | -Im a] (the same convention as every other
// contraction here), (a R)^T = R_op [Re a | -Im a]^T for the real 2M x 2M matrix
//   row n     (Re (aR)_n):  Re R[m][n] at column m,  Im R[m][n] at column M + m
//   row M + n (Im (aR)_n):  Im R[m][n] at column m, -Re R[m][n] at column M + m,
// stored in fp16 times a power-of-two scale (max |entry| in [2^14, 2^15)), columns in K-slot
// order, 16-byte blocks swizzled by row as in LDS; then the float 1 / scale.
template <int M>
struct ReadoutTable {
  static constexpr long oScale = 8L * M * M;
  static constexpr long bytes = (oScale + 4 + 255) / 256 * 256;
};

// Word 3 of a CDNA buffer resource for raw (untyped) loads: 32-bit data format, no swizzle,
// no index stride; offsets at or past the range read as zeros.
constexpr int kBufferFlags = 0x00020000;

// The L valid token rows of chunk c (C tokens) of one sequence of a bf16 tensor, whose token
// 0 is at `seq` and whose token rows are sn elements apart, as a buffer: based at the
// lowest-addressed valid row (row 0 walking forward, row L-1 walking backward), L row strides
// long.  Row r (walk order) column e lies at row_off(r, e) - shift; rows at or past the
// sequence end fall outside the range (past its end forward, below its base, wrapping to
// large offsets, backward) and read as zeros.  (C sn 2 bytes fit 32 bits; the host checks.)
template <int C>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t chunk_rows(const ChunkArgs& a,
                                                             const uint16_t* seq, int sn,
                                                             int c, uint32_t& shift) {
  const int L = min(C, a.N - c * C);
  const uint32_t stride = (uint32_t)sn * 2u;
  shift = a.dir ? (uint32_t)(C - L) * stride : 0u;
  const int pos = a.dir ? a.N - c * C - L : c * C;
  const uint16_t* p = seq + (long long)pos * sn;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p), (short)0,
                                           (int)((uint32_t)L * stride), kBufferFlags);
}

// Byte offset of chunk row r (0 = the chunk's first token in walk order), column e, from the
// lowest-addressed row of a full chunk.
template <int C>
__device__ __forceinline__ uint32_t row_off(const ChunkArgs& a, int sn, int r, int e) {
  return (uint32_t)((a.dir ? C - 1 - r : r) * (uint32_t)sn + e) * 2u;
}

// Workgroup w of a launch over (sequence, segment) pairs, n_seg segments per sequence: the
// plain order is w = seq n_seg + seg.  With `pairs` (H even, bf16 token rows of 32 features:
// 64 bytes, half a 128-byte cache line shared with the neighbouring head) heads 2j and 2j+1 of
// one segment run as workgroups 8 apart, on the same XCD (workgroups go round-robin over the 8)
// at about the same time, so the line comes from HBM once and the second head reads it from
// that XCD's L2: w = 16 (p / 8) + 8 (h & 1) + p % 8 for pair p = (seq / 2) n_seg + seg.  The
// host launches pair_wg_count workgroups; false: a padding workgroup (no work).
__host__ __device__ inline int pair_wg_count(int seqs, int n_seg, bool pairs) {
  return pairs ? 16 * ((seqs / 2 * n_seg + 7) / 8) : seqs * n_seg;
}
// heads > 0 (the output pass, plain order): block w takes position
// p = (w % 8) (grid / 8) + w / 8 of a head-major order p = (h B + b) n_seg + seg, so each XCD
// runs whole heads: the workgroups that copy one head's tables and fold the same sequences'
// segment slots find them in that XCD's L2 after the first.
__device__ inline bool pair_wg(int w, int seqs, int n_seg, bool pairs, int& seq, int& seg,
                               int heads = 0) {
  if (!pairs) {
    const int nb = seqs * n_seg;
    if (heads > 0 && nb % 8 == 0) {
      const int p = (w % 8) * (nb / 8) + w / 8;
      const int rows = seqs / heads, hb = p / n_seg;
      seq = (hb % rows) * heads + hb / rows;
      seg = p % n_seg;
      return true;
    }
    seq = w / n_seg;
    seg = w % n_seg;
    return true;
  }
  const int p = 8 * (w / 16) + w % 8;
  if (p >= seqs / 2 * n_seg) return false;
  seq = 2 * (p / n_seg) + (w / 8) % 2;
  seg = p % n_seg;
  return true;
}

// Per-workgroup context shared by the two wave roles.
template <int C, int F, int D, int M>
struct Ctx {
  uint16_t *s16, *sFk, *sFq, *sV, *sWT, *sWb, *sLU, *sGT;
  float *sC, *sCi;
  float2 *sLE, *sPowL, *sGeo, *sL2lo, *sL2hi;
  const unsigned char* tab;
  int lane, il, g, wave;
  int seq, seg, b, h, c_begin, c_end;
  bool last_seg, want_out;
  float wb_unscale;
  float r_unscale;   // 1 / scale of the readout-matrix operand (RM)
  __device__ int pos_of(const ChunkArgs& a, int t) const { return a.dir ? a.N - 1 - t : t; }
  __device__ size_t tok_index(const ChunkArgs& a, int pos) const {
    return ((size_t)b * a.N + pos) * a.H + h;
  }
  // This sequence's token 0 in q, k and v, and their token-row strides (elements).
  const uint16_t *q0, *k0, *v0;
  int snqk, snv;
  __device__ __amdgpu_buffer_rsrc_t chunk_rows(const ChunkArgs& a, const uint16_t* seq, int sn,
                                               int c, uint32_t& shift) const {
    return ia::chunk_rows<C>(a, seq, sn, c, shift);
  }
  __device__ static uint32_t row_off(const ChunkArgs& a, int sn, int r, int e) {
    return ia::row_off<C>(a, sn, r, e);
  }
};

// 16 bytes through a buffer resource (zeros outside its range).
__device__ __forceinline__ uint4 load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  typedef __attribute__((ext_vector_type(4))) unsigned v4u;
  const v4u v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// n16 16-byte vectors from global memory straight into LDS (no registers), spread over the
// waves in blocks of 64: lane l of block b moves vector 64 b + l.  Completion is
// counted with the wave's vector-memory loads (vmcnt), which complete in issue order.
__device__ __forceinline__ void lds_dma(const unsigned char* src, unsigned char* dst, int n16,
                                        int wave, int lane, int nwaves) {
  for (int b = wave; 64 * b < n16; b += nwaves) {
    const int e = 64 * b + lane;
    if (e < n16)
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)(src + 16 * (size_t)e),
          (__attribute__((address_space(3))) void*)(dst + 1024 * b), 16, 0, 0);
  }
}

// Wait until none of this wave's vector-memory loads, LDS DMA included, is outstanding
// (vmcnt 0; expcnt and lgkmcnt left at their maxima, i.e. not waited on).
__device__ __forceinline__ void wait_vm_zero() {
  __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));
}

// ---------------------------------------------------------------- gate records (gated layer)
// Raw gates (decay, write) of token `lane` of chunk c in walk order for one wave; tokens past
// the sequence end read its last token, and gate_scan clears them.
__device__ __forceinline__ float2 gate_fetch(const ChunkArgs& a, int b, int h, int dir, int c,
                                             int C, int lane) {
  const int t = min(c * C + lane, a.N - 1);
  const size_t gi = ((size_t)b * a.N + (dir ? a.N - 1 - t : t)) * a.H + h;
  return make_float2(a.dgate[gi], a.wgate[gi]);
}

// Lane j of a wave, token j of a chunk (valid: inside the chunk and the sequence): the
// records of GateRec by inclusive scans over the wave's lanes (padding tokens a = 1, w = 0, so
// lane 63 holds the chunk's totals whatever C).
struct GateScan {
  float l;     // L_j
  float w;     // sigma_j w_j
  float e;     // w_j prod_{s=j+1}^{C-1} a_s
  float d;     // prod_s a_s (every lane)
};
__device__ __forceinline__ GateScan gate_scan(float2 raw, bool valid) {
  const float av = valid ? raw.x : 1.f, wv = valid ? raw.y : 0.f;
  const float mag = fabsf(av);
  // log2 (NaN stays NaN); the count of negative gates is scanned as a float (exact to 2^24)
  const float l = wave_scan_incl(mag < 0x1p-64f ? -64.f : __builtin_amdgcn_logf(mag));
  const int neg = (int)wave_scan_incl(av < 0.f ? 1.f : 0.f);
  const float l_last = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(l), 63));
  const float s_last = (__builtin_amdgcn_readlane(neg, 63) & 1) ? -1.f : 1.f;
  GateScan r;
  r.l = l;
  r.w = (neg & 1) ? -wv : wv;
  r.e = s_last * r.w * __builtin_amdgcn_exp2f(l_last - l);
  r.d = s_last * __builtin_amdgcn_exp2f(l_last);
  return r;
}

// A chunk's gate records into one record buffer (GateRec).
template <int C>
__device__ __forceinline__ void gate_records(float2 raw, bool valid, int lane, float* rec) {
  using GR = GateRec<C>;
  const GateScan g = gate_scan(raw, valid);
  if (lane < C) {
    rec[GR::L + lane] = g.l;
    rec[GR::W + lane] = g.w;
    rec[GR::E + lane] = g.e;
  }
  if (lane == 0) rec[GR::D] = g.d;
}

// Gate factors of one 16 x 16 accumulator tile whose rows are keys j = j0 + q (q = 0..3, this
// lane's entries) and whose column is query i (this lane): S[i,j] and P[i,j] times
// W[j] 2^(L_i - L_j), zero past the causal diagonal (diag: the tile holding j = i).
template <int C>
__device__ __forceinline__ void gate_tile(f32x4& t, const float* rec, float li, int j0,
                                          bool diag, int g, int il) {
  using GR = GateRec<C>;
  const float4 L4 = *reinterpret_cast<const float4*>(rec + GR::L + j0);
  const float4 W4 = *reinterpret_cast<const float4*>(rec + GR::W + j0);
  const float lj[4] = {L4.x, L4.y, L4.z, L4.w}, wj[4] = {W4.x, W4.y, W4.z, W4.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float f = __builtin_amdgcn_exp2f(li - lj[q]) * wj[q];
    t[q] *= (!diag || 4 * g + q <= il) ? f : 0.f;
  }
}

// A state operand fragment whose K slots are keys 32kb + 4g + (0..3) (slots 0..3) and
// 32kb + 16 + 4g + (0..3) (slots 4..7), times those keys' end factors E[j] (GateRec).
template <int C>
__device__ __forceinline__ bf16x8 gate_frag(bf16x8 f, const float* rec, int kb, int g) {
  using GR = GateRec<C>;
  const float4 e0 = *reinterpret_cast<const float4*>(rec + GR::E + 32 * kb + 4 * g);
  const float4 e1 = *reinterpret_cast<const float4*>(rec + GR::E + 32 * kb + 16 + 4 * g);
  const float e[8] = {e0.x, e0.y, e0.z, e0.w, e1.x, e1.y, e1.z, e1.w};
  bf16x8 r;
#pragma unroll
  for (int k = 0; k < 8; ++k) r[k] = (__bf16)((float)f[k] * e[k]);
  return r;
}

// ---------------------------------------------------------------- readout waves
// Wave R owns queries [16R, 16R+16) of every chunk.
template <int C, int F, int D, int M, int R, bool RM, bool GT>
__device__ __forceinline__ void readout_main(const ChunkArgs& a, const Ctx<C, F, D, M>& x) {
  using Lay = Layout<C, F, D, M, C / 16, RM, GT>;
  using GR = GateRec<C>;
  constexpr int NR = C / 16;
  constexpr int M2 = 2 * M;
  constexpr int MH = M / 16;
  constexpr int TM = M2 / 16;
  constexpr int KF = F / 32;
  constexpr int KM = M2 / 32;
  constexpr int KC = C / 32;
  constexpr int TD = D / 16;
  constexpr int r = R;   // compile-time: causal trip counts below are constants
  const int lane = x.lane, il = x.il, g = x.g;
  // Per-lane LDS offsets, one per K step (row il, block 4 step + g); tiles add constants.
  // Offsets from the LDS base (matrix start included, see opaque): phi(k) / phi(q) (one set,
  // phi(q) is at a constant distance below 64 KiB), lam U, the two decay tables, lam G, v.
  int oF[KF], oLU[KF], oWT[KC], oWb[KM], oGT[KM], oV[TD], oRm[RM ? KM : 1];
#pragma unroll
  for (int s = 0; s < KF; ++s) {
    oF[s] = opaque(Lay::oFk + lane_off<F>(il, 4 * s + g));
    oLU[s] = opaque(Lay::oLU + lane_off<F>(il, 4 * s + g));
  }
#pragma unroll
  for (int kb = 0; kb < KC; ++kb) oWT[kb] = opaque(Lay::oWT + lane_off<C>(il, 4 * kb + g));
#pragma unroll
  for (int kb = 0; kb < KM; ++kb) {
    oWb[kb] = opaque(Lay::oWb + lane_off<M2>(il, 4 * kb + g));
    oGT[kb] = opaque(Lay::oGT + lane_off<M2>(il, 4 * kb + g));
    if constexpr (RM) oRm[kb] = opaque(Lay::oR + lane_off<M2>(il, 4 * kb + g));
  }
#pragma unroll
  for (int dt = 0; dt < TD; ++dt) oV[dt] = opaque(Lay::oV + tr_off<D>(dt, lane));
  const uint16_t* s16 = x.s16;
  static_assert(Lay::oFq - Lay::oFk + C * F < 32768, "phi(q) within the immediate range");
  // fp32 tables past 64 KiB likewise: lam^(2i) rows (il), then lam^(32r), lam eta and 1/c_d
  // (lane group g).
  const unsigned char* sb = reinterpret_cast<const unsigned char*>(x.s16);
  const int oLo = opaque(Lay::bL2lo + 8 * (il * Lay::L2S + 4 * g));
  const int oG = opaque(Lay::bLE + 32 * g);
  const int oCi = opaque(Lay::bCi + 16 * g);
  static_assert(Lay::bL2hi + 8 * (NR * M) - Lay::bLE < 65536, "tables within the immediate range");

  // ---- v loader: this wave moves rows 16r + il of the chunk's v, 16-byte blocks g + 4t, from
  // HBM to LDS (raw bf16).  Token rows are H*D elements apart, backwards in reverse.
  constexpr int VD = D / 8, NV = VD / 4;
  int stV[NV];
#pragma unroll
  for (int t = 0; t < NV; ++t) stV[t] = opaque(Lay::oV + soff<D>(16 * r + il, 8 * (g + 4 * t)));
  const uint32_t lofV = x.row_off(a, x.snv, 16 * r + il, 8 * g);
  uint4 rv[NV];
  auto fetch_v = [&](int c) {   // rows past N read as zeros
    uint32_t shift;
    const __amdgpu_buffer_rsrc_t vb = x.chunk_rows(a, x.v0, x.snv, c, shift);
#pragma unroll
    for (int t = 0; t < NV; ++t) rv[t] = load16(vb, lofV - shift + 64 * t);
  };
  auto write_v = [&]() {
#pragma unroll
    for (int t = 0; t < NV; ++t) *reinterpret_cast<uint4*>(x.s16 + stV[t]) = rv[t];
  };

  // Gated layer: wave 0 turns each chunk's gates into its records (GateRec), chunk c into
  // buffer c % 2: the first chunk's before the loop, chunk c+1's in chunk c's second phase
  // (chunk c-1, the buffer's last reader, is done), from gates loaded at chunk c's start.
  float* const recb = reinterpret_cast<float*>(reinterpret_cast<unsigned char*>(x.s16) + Lay::bRec);
  auto rec_of = [&](int c) { return recb + (c & 1) * GR::floats; };
  float2 graw = make_float2(1.f, 0.f);
  auto gate_valid = [&](int c) { return lane < C && c * C + lane < a.N; };

  // The first chunk's v loads go out before the barrier and land while the state waves copy
  // the tables.
  if (x.c_begin < x.c_end) {
    fetch_v(x.c_begin);
    if constexpr (GT && r == 0) graw = gate_fetch(a, x.b, x.h, a.dir, x.c_begin, C, lane);
  }
  __syncthreads();  // tables visible
  if constexpr (GT && r == 0)
    if (x.c_begin < x.c_end) gate_records<C>(graw, gate_valid(x.c_begin), lane, rec_of(x.c_begin));
  // lam^(2i) for this lane's queries i = 16r + il and modes m = 16mt + 4g + q, for the whole
  // segment: the product of the two factor tables, formed once.  With a readout matrix the
  // tables hold lam^i factors instead: A = lam^i A' before the mixing, lam^i (A R) after it.
  float2 l2[MH][4];
#pragma unroll
  for (int mt = 0; mt < MH; ++mt)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int mo = 8 * (16 * mt + q);
      l2[mt][q] = cmul(*reinterpret_cast<const float2*>(sb + oLo + mo),
                       *reinterpret_cast<const float2*>(sb + oG + (Lay::bL2hi - Lay::bLE) +
                                                        8 * r * M + mo));
    }
  __syncthreads();  // first chunk's inputs in LDS

  // The second walk of a bidirectional call adds onto the first walk's outputs: with narrow
  // values (D <= 32, a few registers) this lane's o entries of the chunk are loaded at the
  // chunk's start, their latency covered by the chunk's work instead of stalling the output.
  constexpr bool kEarlyO = D <= 32;
  uint4 o_prev[kEarlyO ? TD : 1];
  for (int c = x.c_begin; c < x.c_end; ++c) {
    // v of chunk c into LDS (its readers run after the mid-chunk barrier), the next chunk's
    // loads out.
    write_v();
    if (c + 1 < x.c_end) fetch_v(c + 1);
    const float* const rec = rec_of(c);
    if constexpr (kEarlyO) {
      const int t = c * C + 16 * r + il;
      if (a.accumulate && x.want_out && t < a.N) {
        const size_t ob = x.tok_index(a, x.pos_of(a, t)) * D + 4 * g;
#pragma unroll
        for (int dt = 0; dt < TD; ++dt) {
          if (a.out_bf16) {
            const uint2 w = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(a.o) +
                                                            ob + 16 * dt);
            o_prev[dt] = make_uint4(w.x, w.y, 0u, 0u);
          } else {
            o_prev[dt] = *reinterpret_cast<const uint4*>(static_cast<const float*>(a.o) + ob +
                                                         16 * dt);
          }
        }
      }
    }
    // Live across the mid-chunk barrier: the fp16 operand of lam^(2i) A', its per-query
    // scale and the inter-chunk denominator.
    f16x8 Af[KM];
    float si = 1.f, den_inter = 0.f;
    if (x.want_out) {
      // phi(q) of this wave's queries as B operands (K = f)
      bf16x8 fq[KF];
#pragma unroll
      for (int s = 0; s < KF; ++s) fq[s] = lds8(s16 + oF[s] + (Lay::oFq - Lay::oFk) + 16 * r * F).b;
      // ---- S^T tiles (rows j, columns i), causal: tiles jt <= r.  Their results are read
      // only after the inter-chunk MFMAs below, which cover the latency.
      f32x4 accS[NR];
#pragma unroll
      for (int jt = 0; jt < NR; ++jt) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        if (jt <= r) {
#pragma unroll
          for (int s = 0; s < KF; ++s)
            acc = mma_bf16(lds8(s16 + oF[s] + 16 * jt * F).b, fq[s], acc);
        }
        accS[jt] = acc;
      }
      IA_STEP_FENCE();

      // ---- A'^T tiles (rows k, columns i): the inter-chunk term (lam U_c) Fq^T first
      f32x4 accA[TM];
#pragma unroll
      for (int kt = 0; kt < TM; ++kt) accA[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KF; ++s) {
#pragma unroll
        for (int kt = 0; kt < TM; ++kt)
          accA[kt] = mma_bf16(lds8(s16 + oLU[s] + 16 * kt * F).b, fq[s], accA[kt]);
        IA_STEP_FENCE();
      }
      // Gated: the inter-chunk term times the decay since the chunk start, 2^(L_i), and each
      // S[i,j] times the gate factor W[j] 2^(L_i - L_j) (zero past the diagonal).
      if constexpr (GT) {
        const float li = rec[GR::L + 16 * r + il];
        const float di = __builtin_amdgcn_exp2f(li);
#pragma unroll
        for (int kt = 0; kt < TM; ++kt)
#pragma unroll
          for (int q = 0; q < 4; ++q) accA[kt][q] *= di;
#pragma unroll
        for (int jt = 0; jt <= r; ++jt) gate_tile<C>(accS[jt], rec, li, 16 * jt + 4 * g, jt == r, g, il);
      }
      // causal mask of the diagonal S tile, then S as the bf16 operand of WT^T S
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (4 * g + q > il) accS[r][q] = 0.f;
      bf16x8 Sf[KC];
#pragma unroll
      for (int kb = 0; kb < KC; ++kb) Sf[kb] = pack_bf16(accS[2 * kb], accS[2 * kb + 1]);
#pragma unroll
      for (int kb = 0; kb < KC; ++kb)
        if (32 * kb <= 16 * r + 15) {
#pragma unroll
          for (int kt = 0; kt < TM; ++kt)
            accA[kt] = mma_bf16(lds8(s16 + oWT[kb] + 16 * kt * C).b, Sf[kb], accA[kt]);
          IA_STEP_FENCE();
        }

      // ---- readout matrix: A = lam^i A' as the fp16 operand [Re | -Im] (scaled per query),
      // then (A R)^T = R_op A^T on MFMA into the same accumulators, whose [Re; Im] rows the
      // step below takes as it takes A' (times 1 / both scales).
      float ru = 1.f;
      if constexpr (RM) {
        float xmax = 0.f;
#pragma unroll
        for (int mt = 0; mt < MH; ++mt)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float2 L = l2[mt][q];
            const float xr = accA[mt][q], yi = accA[mt + MH][q];
            const float ar = xr * L.x - yi * L.y, ai = xr * L.y + yi * L.x;
            accA[mt][q] = ar;
            accA[mt + MH][q] = -ai;
            xmax = fmaxf(xmax, fmaxf(fabsf(ar), fabsf(ai)));
          }
        const float sx = pow2_scale(xor_max16_32(xmax));
        ru = x.r_unscale / sx;
        f16x8 Xf[KM];
#pragma unroll
        for (int kb = 0; kb < KM; ++kb)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            Xf[kb][q] = (_Float16)(sx * accA[2 * kb][q]);
            Xf[kb][4 + q] = (_Float16)(sx * accA[2 * kb + 1][q]);
          }
#pragma unroll
        for (int nt = 0; nt < TM; ++nt) {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kb = 0; kb < KM; ++kb)
            acc = mma_f16(lds8(s16 + oRm[kb] + 16 * nt * M2).h, Xf[kb], acc);
          accA[nt] = acc;
        }
        IA_STEP_FENCE();
      }

      // ---- lam^(2i) A' (fp32), den_inter, per-query scale, fp16 operands [Re | -Im]
      float amax = 0.f;
#pragma unroll
      for (int mt = 0; mt < MH; ++mt) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          // m = 16 mt + 4 g + q
          const int mo = 8 * (16 * mt + q);
          const float2 le = *reinterpret_cast<const float2*>(sb + oG + mo);
          float2 L2 = l2[mt][q];
          if constexpr (RM) {
            L2.x *= ru;
            L2.y *= ru;
          }
          const float xr = accA[mt][q], yi = accA[mt + MH][q];
          const float ar = xr * L2.x - yi * L2.y, ai = xr * L2.y + yi * L2.x;
          accA[mt][q] = ar;
          accA[mt + MH][q] = -ai;
          den_inter += ar * le.x - ai * le.y;
          amax = fmaxf(amax, fmaxf(fabsf(ar), fabsf(ai)));
        }
        IA_STEP_FENCE();
      }
      den_inter = xor_sum16_32(den_inter);
      if constexpr (GT)   // eta_c decays by 2^(L_i) as well
        den_inter *= __builtin_amdgcn_exp2f(rec[GR::L + 16 * r + il]);
      amax = xor_max16_32(amax);
      si = pow2_scale(amax);
#pragma unroll
      for (int kb = 0; kb < KM; ++kb)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          Af[kb][q] = (_Float16)(si * accA[2 * kb][q]);
          Af[kb][4 + q] = (_Float16)(si * accA[2 * kb + 1][q]);
        }
    }
    // Mid-chunk barrier: S, A' and its decay are done, so phi(q), phi(k) and lam U of chunk c
    // are no longer read and the state waves overwrite them with chunk c+1's.
    __syncthreads();
    // (gated: chunk c+1's gates load during this second phase, whose registers are fewer)
    if constexpr (GT && r == 0)
      if (c + 1 < x.c_end) graw = gate_fetch(a, x.b, x.h, a.dir, c + 1, C, lane);
    if (x.want_out) {
      // gated: L_i and 2^(L_i) again (the records stay until chunk c+1's second phase)
      const float li = GT ? rec[GR::L + 16 * r + il] : 0.f;
      const float di = GT ? __builtin_amdgcn_exp2f(li) : 1.f;

      // ---- P^T tiles (rows j, columns i), causal; their results are read after the
      // inter-chunk numerator MFMAs below
      f32x4 accP[NR];
#pragma unroll
      for (int jt = 0; jt < NR; ++jt) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        if (jt <= r) {
#pragma unroll
          for (int kb = 0; kb < KM; ++kb)
            acc = mma_f16(lds8(s16 + oWb[kb] + 16 * jt * M2).h, Af[kb], acc);
        }
        accP[jt] = acc;
      }
      IA_STEP_FENCE();
      if constexpr (GT) {
#pragma unroll
        for (int jt = 0; jt <= r; ++jt) gate_tile<C>(accP[jt], rec, li, 16 * jt + 4 * g, jt == r, g, il);
      }
      // ---- c_d-scaled Re(A lam G) per value tile (rows d, columns i)
      f32x4 accX[TD];
#pragma unroll
      for (int dt = 0; dt < TD; ++dt) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < KM; ++kb)
          acc = mma_f16(lds8(s16 + oGT[kb] + 16 * dt * M2).h, Af[kb], acc);
        accX[dt] = acc;
        IA_STEP_FENCE();
      }
      float den_intra = 0.f;
#pragma unroll
      for (int jt = 0; jt < NR; ++jt)
        if (jt <= r) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            float p = accP[jt][q] * x.wb_unscale;
            if (jt == r && 4 * g + q > il) p = 0.f;
            accP[jt][q] = p;
            den_intra += p;
          }
        }
      den_intra = xor_sum16_32(den_intra);
      const float den = den_intra + si * den_inter;   // in units of si
      // num and den are in units of si (the fp16 scale of A).  Without a denominator
      // (kOptNoDen) den_w = 0 and den_c = 1: the divisor is max(0, si) = si and o = num.
      const float rd = 1.f / clamp_den(den * a.den_w, si * a.den_c);
      bf16x8 Pf[KC];
#pragma unroll
      for (int kb = 0; kb < KC; ++kb) Pf[kb] = pack_bf16(accP[2 * kb], accP[2 * kb + 1]);

      // ---- num^T tiles (rows d, columns i): P V (accI) + the inter-chunk part (accX)
      const int t = c * C + 16 * r + il;
      const bool ok = t < a.N;
      // Output row of query t from this lane's column 4g: dt tiles are constant offsets.
      const size_t obase = ok ? x.tok_index(a, x.pos_of(a, t)) * D + 4 * g : 0;
      uint16_t* const o16 = static_cast<uint16_t*>(a.o) + obase;
      float* const o32 = static_cast<float*>(a.o) + obase;
#pragma unroll
      for (int dt = 0; dt < TD; ++dt) {
        f32x4 accI = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < KC; ++kb)
          if (32 * kb <= 16 * r + 15)
            accI = mma_bf16(ldtr<D>(s16, oV[dt], kb).b, Pf[kb], accI);
        const f32x4 accXd = accX[dt];
        if (ok) {
          float4 ci = *reinterpret_cast<const float4*>(sb + oCi + 64 * dt);
          if constexpr (GT) {   // G_c decays by 2^(L_i) as well
            ci.x *= di; ci.y *= di; ci.z *= di; ci.w *= di;
          }
          float val[4] = {(accI[0] + accXd[0] * ci.x) * rd, (accI[1] + accXd[1] * ci.y) * rd,
                          (accI[2] + accXd[2] * ci.z) * rd, (accI[3] + accXd[3] * ci.w) * rd};
          if (a.out_bf16) {
            if (a.accumulate) {   // the element's other direction, same lane, read then written
              uint2 p;
              if constexpr (kEarlyO) p = make_uint2(o_prev[dt].x, o_prev[dt].y);
              else p = *reinterpret_cast<const uint2*>(o16 + 16 * dt);
              val[0] += __uint_as_float(p.x << 16);
              val[1] += __uint_as_float(p.x & 0xffff0000u);
              val[2] += __uint_as_float(p.y << 16);
              val[3] += __uint_as_float(p.y & 0xffff0000u);
            }
            *reinterpret_cast<uint2*>(o16 + 16 * dt) = pack4_bf16(val[0], val[1], val[2], val[3]);
          } else {
            if (a.accumulate) {
              float4 p;
              if constexpr (kEarlyO) p = __builtin_bit_cast(float4, o_prev[dt]);
              else p = *reinterpret_cast<const float4*>(o32 + 16 * dt);
              val[0] += p.x; val[1] += p.y; val[2] += p.z; val[3] += p.w;
            }
            *reinterpret_cast<float4*>(o32 + 16 * dt) = make_float4(val[0], val[1], val[2], val[3]);
          }
        }
        IA_STEP_FENCE();
      }
    }
    if constexpr (GT && r == 0)
      if (c + 1 < x.c_end) gate_records<C>(graw, gate_valid(c + 1), lane, rec_of(c + 1));
    __syncthreads();   // chunk c read by every wave
  }
}

// ---------------------------------------------------------------- state waves
// State wave U owns feature tiles ft = U, U+NS, ... of (lam U)^T and value tiles dt = U,
// U+NS, ... of lam G, in fp32 MFMA accumulators for the whole segment; wave 0 also owns
// lam eta.
template <int C, int F, int D, int M, int U, bool RM, bool GT>
__device__ __forceinline__ void state_main(const ChunkArgs& a, const Ctx<C, F, D, M>& x) {
  using TL = TableLayout<C, M>;
  using Lay = Layout<C, F, D, M, C / 16, RM, GT>;
  using GR = GateRec<C>;
  constexpr int M2 = 2 * M;
  constexpr int MH = M / 16;
  constexpr int TM = M2 / 16;
  constexpr int KC = C / 32;
  constexpr int TD = D / 16;
  constexpr int NS = StateWaves<F, D, M>::NS;
  constexpr int NFT = (F / 16 + NS - 1) / NS;
  constexpr int NDT = (D / 16 + NS - 1) / NS;
  constexpr int u = U;   // compile-time: owned tiles below are constants
  const int lane = x.lane, il = x.il, g = x.g;
  // Loader share of this wave: 16-byte vectors n = 64u + lane + 64 NS t of the row-major
  // chunk matrices q, k ([C][F]) and v ([C][D]).
  constexpr int VF = F / 8;
  constexpr int NL = 64 * NS;
  constexpr int NLF = (C * VF + NL - 1) / NL;
  // Per-lane LDS offsets (tiles add compile-time constants).
  // Offsets from the LDS base, matrix start included (see opaque).
  int offC[KC], trF[NFT], trD[NDT], pubU[NFT], pubG[TM / 2];
#pragma unroll
  for (int kb = 0; kb < KC; ++kb) offC[kb] = opaque(Lay::oWT + lane_off<C>(il, 4 * kb + g));
#pragma unroll
  for (int fi = 0; fi < NFT; ++fi) {
    trF[fi] = opaque(Lay::oFk + tr_off<F>(u + NS * fi, lane));
    // lam U row m = 16mt + il (Re) or M + 16mt + il (Im), columns 16ft + 4g .. +3
    pubU[fi] = opaque(Lay::oLU + lane_off<F>(il, 2 * (u + NS * fi) + (g >> 1)) + 4 * (g & 1));
  }
#pragma unroll
  for (int di = 0; di < NDT; ++di) trD[di] = opaque(Lay::oV + tr_off<D>(u + NS * di, lane));
  // c_d lam G row d = 16dt + il, columns kpos(16kt + 4g) = 32 (kt/2) + 8g + 4 (kt%2) .. +3
#pragma unroll
  for (int k2 = 0; k2 < TM / 2; ++k2) pubG[k2] = opaque(Lay::oGT + lane_off<M2>(il, 4 * k2 + g));
  uint16_t* const s16 = x.s16;
  // fp32 tables past 64 KiB: lam^L by mode row il / group g, c_d by value row il, per-lane
  // vectors (lam eta, lam^L, the geometric sums) by lane.
  unsigned char* const sb = reinterpret_cast<unsigned char*>(x.s16);
  const int oPl = opaque(Lay::bPowL + 8 * il);
  const int oPg = opaque(Lay::bPowL + 32 * g);
  const int oCd = opaque(Lay::bC + 4 * il);
  const int oLn = opaque(Lay::bLE + 8 * lane);
  auto f2 = [&](int off) -> float2& { return *reinterpret_cast<float2*>(sb + off); };

  f32x4 accU[NFT][TM];   // (lam U)^T tiles: rows f = 16ft + 4g + q, columns k = 16kt + il
  f32x4 accG[NDT][TM];   // lam G tiles:     rows k = 16kt + 4g + q, columns d = 16dt + il
  float2 eta = make_float2(0.f, 0.f);  // lam eta; wave 0, lane m < M
#pragma unroll
  for (int fi = 0; fi < NFT; ++fi)
#pragma unroll
    for (int kt = 0; kt < TM; ++kt) accU[fi][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int di = 0; di < NDT; ++di)
#pragma unroll
    for (int kt = 0; kt < TM; ++kt) accG[di][kt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- chunk inputs q, k: this wave loads 16-byte vectors n = 64u + lane + NL t of the
  // row-major chunk matrices ([C][F]); vector n0 + NL t is row row0 + t NL/VF.  Token rows are
  // H*F elements apart in memory, walking backwards for the reverse direction; per chunk the
  // wave-uniform base moves, the per-lane offsets stay.  (The readout waves load v.)
  const int n0 = 64 * u + lane;
  const int rowF0 = n0 / VF;
  uint32_t lofF[NLF];
#pragma unroll
  for (int t = 0; t < NLF; ++t)
    lofF[t] = x.row_off(a, x.snqk, rowF0 + t * (NL / VF), 8 * (n0 % VF));
  // LDS rows row0 + t NL/VF share the swizzle of row0 (NL/VF is a multiple of 16).
  static_assert((NL / VF) % 16 == 0, "loader rows keep the swizzle");
  const int stF = opaque(Lay::oFk + soff<F>(rowF0, 8 * (n0 % VF)));
  // Raw bf16 q, k of a chunk, then (convert) phi(q), phi(k) as packed bf16.
  uint4 rq[NLF], rk[NLF];
  auto fetch = [&](int c) {   // rows past N (and past the chunk) read as zeros
    uint32_t shift;
    const __amdgpu_buffer_rsrc_t kb = x.chunk_rows(a, x.k0, x.snqk, c, shift);
    const __amdgpu_buffer_rsrc_t qb = x.chunk_rows(a, x.q0, x.snqk, c, shift);
#pragma unroll
    for (int t = 0; t < NLF; ++t) {
      rk[t] = load16(kb, lofF[t] - shift);
      if (x.want_out) rq[t] = load16(qb, lofF[t] - shift);
    }
  };
  // Features in place (the values themselves with kOptIdentity).  Rows past N get zero
  // features (not phi(0)); their values are zero.
  const float fT = feature_t(a.opt), fC = feature_c(a.opt);
  auto phi8 = [&](uint4& r, bool ok) {
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)   // bf16 pair -> two floats -> features -> bf16 pair
      o[i] = pk_bf16(feature_tc(__uint_as_float(w[i] << 16), fT, fC),
                     feature_tc(__uint_as_float(w[i] & 0xffff0000u), fT, fC));
    r = ok ? make_uint4(o[0], o[1], o[2], o[3]) : make_uint4(0, 0, 0, 0);
  };
  auto convert = [&](int c) {
    const int L = a.N - c * C;
#pragma unroll
    for (int t = 0; t < NLF; ++t) {
      const bool ok = rowF0 + t * (NL / VF) < L;
      phi8(rk[t], ok);
      if (x.want_out) phi8(rq[t], ok);
    }
  };
  auto write_inputs = [&]() {
#pragma unroll
    for (int t = 0; t < NLF; ++t)
      if (n0 + NL * t < C * VF) {
        const int so = stF + t * (NL / VF) * F;
        *reinterpret_cast<uint4*>(s16 + so) = rk[t];
        if (x.want_out) *reinterpret_cast<uint4*>(s16 + so + (Lay::oFq - Lay::oFk)) = rq[t];
      }
  };

  // Initial state (times lam): the caller's state, then the end states of the earlier
  // segments of this sequence.
  using SL = SlotLayout<F, D, M>;
  const float2 *iU = nullptr, *iG = nullptr, *iE = nullptr;
  const bool from_slot = a.seg_prev && a.seg_inclusive && x.seg > 0;
  if (a.init0_U && !from_slot) {
    iU = a.init0_U + (size_t)x.seq * M * F;
    iG = a.init0_G + (size_t)x.seq * M * D;
    iE = a.init0_E + (size_t)x.seq * M;
  }
  const float2* lamh = a.lam + (size_t)x.h * M;
  if (iU) {
#pragma unroll
    for (int fi = 0; fi < NFT; ++fi) {
      const int ft = u + NS * fi;
      if (ft < F / 16) {
#pragma unroll
        for (int mt = 0; mt < MH; ++mt) {
          const int m = 16 * mt + il;
          const float2 l = lamh[m];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float2 v = cmul(l, iU[(size_t)m * F + 16 * ft + 4 * g + q]);
            accU[fi][mt][q] = v.x;
            accU[fi][mt + MH][q] = v.y;
          }
        }
      }
    }
#pragma unroll
    for (int di = 0; di < NDT; ++di) {
      const int dt = u + NS * di;
      if (dt < TD) {
#pragma unroll
        for (int mt = 0; mt < MH; ++mt)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int m = 16 * mt + 4 * g + q;
            const float2 v = cmul(lamh[m], iG[(size_t)m * D + 16 * dt + il]);
            accG[di][mt][q] = v.x;
            accG[di][mt + MH][q] = v.y;
          }
      }
    }
    if (u == 0 && lane < M) eta = cmul(lamh[lane], iE[lane]);
  }
  // The state waves copy the tables straight into LDS, so the readout waves carry no pending
  // LDS-DMA writes and their first chunk's loads stay in flight across the barrier.
  {
    unsigned char* const sb = reinterpret_cast<unsigned char*>(x.s16);
    lds_dma(x.tab + TL::oW, sb + 2 * Lay::oWT, (int)(TL::nW / 16), u, lane, NS);
    lds_dma(x.tab + TL::oL2, sb + Lay::bL2lo, (int)(TL::nL2 / 16), u, lane, NS);
    lds_dma(x.tab + TL::oPow, sb + Lay::bPowL, 40 * M / 16, (u + 1) % NS, lane, NS);
    if constexpr (RM)
      lds_dma(a.rtab + (size_t)x.h * a.rtab_bytes, sb + 2 * Lay::oR, 8 * M * M / 16,
              (u + 2) % NS, lane, NS);
  }
  wait_vm_zero();
  __syncthreads();  // tables visible (the Horner step reads lam^Ls from LDS)
  if (a.seg_prev && x.seg > 0) {
    // Horner over the earlier segments; an inclusive slot is the state itself (zero state
    // times lam^Ls plus the slot).  lam^Ls comes from LDS, so a slot's loads can all be in
    // flight before any of it is combined.
    constexpr int dS = Lay::bPowS - Lay::bPowL;   // lam^Ls beside lam^C (oPl, oPg offsets)
    for (int sp = a.seg_inclusive ? x.seg - 1 : 0; sp < x.seg; ++sp) {
      const float* sl = a.seg_prev + ((size_t)x.seq * a.slots_per_seq + sp) * a.slot_floats;
      float2 e = make_float2(0.f, 0.f);
      if (u == 0 && lane < M) e = reinterpret_cast<const float2*>(sl + SL::eta)[lane];
      // gated: the state entering segment sp also decays by the segment's gate product
      const float ds = GT ? sl[SL::dseg] : 1.f;
      auto pws = [&](float2 p) { return GT ? make_float2(p.x * ds, p.y * ds) : p; };
      // lam U tile pairs: this wave's MH pairs loaded together, then combined
#pragma unroll
      for (int fi = 0; fi < NFT; ++fi)
        if (u + NS * fi < F / 16) {
          uint4 v[MH];
          float is[MH];
#pragma unroll
          for (int mt = 0; mt < MH; ++mt) {
            v[mt] = *reinterpret_cast<const uint4*>(sl + SL::pair(u, fi * MH + mt, lane));
            is[mt] = sl[SL::scale_of(u, fi * MH + mt, lane)];
          }
#pragma unroll
          for (int mt = 0; mt < MH; ++mt) {
            const float2 pw = pws(f2(oPl + dS + 128 * mt));
            float er[4], ei[4];
            slot_unpack(v[mt], is[mt], er, ei);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const float xr = accU[fi][mt][q], yi = accU[fi][mt + MH][q];
              accU[fi][mt][q] = pw.x * xr - pw.y * yi + er[q];
              accU[fi][mt + MH][q] = pw.x * yi + pw.y * xr + ei[q];
            }
          }
        }
      // lam G tile pairs likewise
#pragma unroll
      for (int di = 0; di < NDT; ++di)
        if (u + NS * di < TD) {
          uint4 v[MH];
          float is[MH];
#pragma unroll
          for (int mt = 0; mt < MH; ++mt) {
            const int pp = (NFT + di) * MH + mt;
            v[mt] = *reinterpret_cast<const uint4*>(sl + SL::pair(u, pp, lane));
            is[mt] = sl[SL::scale_of(u, pp, lane)];
          }
#pragma unroll
          for (int mt = 0; mt < MH; ++mt) {
            float er[4], ei[4];
            slot_unpack(v[mt], is[mt], er, ei);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const float2 pw = pws(f2(oPg + dS + 8 * (16 * mt + q)));
              const float xr = accG[di][mt][q], yi = accG[di][mt + MH][q];
              accG[di][mt][q] = pw.x * xr - pw.y * yi + er[q];
              accG[di][mt + MH][q] = pw.x * yi + pw.y * xr + ei[q];
            }
          }
        }
      if (u == 0 && lane < M) {
        eta = cmul(pws(f2(oLn + (Lay::bPowS - Lay::bLE))), eta);
        eta.x += e.x;
        eta.y += e.y;
      }
    }
  }

  // ---- operand copies of the state for the readout: lam U (bf16) and lam eta of chunk c+1,
  // written in chunk c's second phase (the readout reads them in the first); c_d lam G (fp16,
  // c_d a power of two per value column) and the column scales of chunk c, written in chunk
  // c's first phase (the readout reads them in the second).
  uint2 pG[NDT][TM];       // c_d lam G, 4 fp16 each
  float pC[NDT];
  auto pack_state = [&]() {
#pragma unroll
    for (int di = 0; di < NDT; ++di)
      if (u + NS * di < TD) {
        float mx = 0.f;
#pragma unroll
        for (int kt = 0; kt < TM; ++kt)
#pragma unroll
          for (int q = 0; q < 4; ++q) mx = fmaxf(mx, fabsf(accG[di][kt][q]));
        mx = xor_max16_32(mx);
        const float cd = pow2_scale(mx);
        pC[di] = cd;
#pragma unroll
        for (int kt = 0; kt < TM; ++kt)
          pG[di][kt] = pack4_f16(cd * accG[di][kt][0], cd * accG[di][kt][1],
                                 cd * accG[di][kt][2], cd * accG[di][kt][3]);
      }
  };
  auto write_lam_u = [&]() {
#pragma unroll
    for (int fi = 0; fi < NFT; ++fi)
      if (u + NS * fi < F / 16) {
#pragma unroll
        for (int mt = 0; mt < MH; ++mt) {
          *reinterpret_cast<uint2*>(s16 + pubU[fi] + 16 * mt * F) = pack4_bf16(
              accU[fi][mt][0], accU[fi][mt][1], accU[fi][mt][2], accU[fi][mt][3]);
          *reinterpret_cast<uint2*>(s16 + pubU[fi] + (M + 16 * mt) * F) =
              pack4_bf16(accU[fi][mt + MH][0], accU[fi][mt + MH][1], accU[fi][mt + MH][2],
                         accU[fi][mt + MH][3]);
        }
      }
  };
  auto write_g = [&]() {   // lam G copy and its column scales
#pragma unroll
    for (int di = 0; di < NDT; ++di) {
      const int dt = u + NS * di;
      if (dt < TD) {
        if (g == 0) {
          *reinterpret_cast<float*>(sb + oCd + 64 * dt) = pC[di];
          *reinterpret_cast<float*>(sb + oCd + (Lay::bCi - Lay::bC) + 64 * dt) = 1.f / pC[di];
        }
#pragma unroll
        for (int kt = 0; kt < TM; ++kt)
          *reinterpret_cast<uint2*>(s16 + pubG[kt >> 1] + 4 * (kt & 1) + 16 * dt * M2) =
              pG[di][kt];
      }
    }
  };
  auto write_eta = [&]() {
    if (u == 0 && lane < M) f2(oLn) = eta;
  };
  // lam G <- lam^L lam G with chunk cc's pair (the full-chunk pair, or the last chunk's)
  auto decay_g = [&](int cc) {
    const int ts = a.N - cc * C < C ? Lay::kTail : 0;
#pragma unroll
    for (int di = 0; di < NDT; ++di)
      if (u + NS * di < TD) {
#pragma unroll
        for (int mt = 0; mt < MH; ++mt)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float2 p = f2(oPg + ts + 8 * (16 * mt + q));
            const float xr = accG[di][mt][q], yi = accG[di][mt + MH][q];
            accG[di][mt][q] = p.x * xr - p.y * yi;
            accG[di][mt + MH][q] = p.x * yi + p.y * xr;
          }
      }
  };

  if (x.c_begin < x.c_end) {
    fetch(x.c_begin);
    convert(x.c_begin);
    if (x.want_out) {
      write_lam_u();
      pack_state();   // written in the first chunk's first phase
      write_eta();
    }
    write_inputs();
    if (x.c_begin + 1 < x.c_end) fetch(x.c_begin + 1);
  }
  __syncthreads();

  // Two phases per chunk.  First: the lam G copy of chunk c (lam G of chunk c-1, updated in
  // the previous second phase, is decayed and packed here), then
  // lam U^T <- lam^L (lam U^T + phi(K)^T (beta lam^-j)).  Second, once v of chunk c is in
  // LDS: lam G <- lam G + W^T V (its decay waits for the next first phase), and chunk c+1's
  // copies and inputs.
  // Gated: this chunk's records (GateRec; buffer c % 2, written by readout wave 0).
  const float* const recb =
      reinterpret_cast<const float*>(reinterpret_cast<const unsigned char*>(x.s16) + Lay::bRec);
  for (int c = x.c_begin; c < x.c_end; ++c) {
    const float* const rec = recb + (c & 1) * GR::floats;
    const float dl = GT ? rec[GR::D] : 1.f;   // gated: the chunk's decay product
    if (c > x.c_begin) {
      decay_g(c - 1);
      if (x.want_out) pack_state();
    }
    if (x.want_out) write_g();
    // Gated: lam U_{c+1} = lam^L (D lam U_c + sum_j beta lam^-j E[j] phi(k_j)).
    if constexpr (GT) {
#pragma unroll
      for (int fi = 0; fi < NFT; ++fi)
        if (u + NS * fi < F / 16) {
#pragma unroll
          for (int kt = 0; kt < TM; ++kt)
#pragma unroll
            for (int q = 0; q < 4; ++q) accU[fi][kt][q] *= dl;
        }
    }
#pragma unroll
    for (int kb = 0; kb < KC; ++kb) {
      bf16x8 afk[NFT];
#pragma unroll
      for (int fi = 0; fi < NFT; ++fi)
        if (u + NS * fi < F / 16) {
          afk[fi] = ldtr<F>(s16, trF[fi], kb).b;
          if constexpr (GT) afk[fi] = gate_frag<C>(afk[fi], rec, kb, g);
        }
#pragma unroll
      for (int kt = 0; kt < TM; ++kt) {
        const bf16x8 w = lds8(s16 + offC[kb] + 16 * kt * C).b;
#pragma unroll
        for (int fi = 0; fi < NFT; ++fi)
          if (u + NS * fi < F / 16) accU[fi][kt] = mma_bf16(afk[fi], w, accU[fi][kt]);
        IA_STEP_FENCE();
      }
    }
    // lam^L and the geometric sum of chunk c: the full-chunk pair, or the last chunk's
    const int tsel = a.N - c * C < C ? Lay::kTail : 0;
#pragma unroll
    for (int fi = 0; fi < NFT; ++fi)
      if (u + NS * fi < F / 16) {
#pragma unroll
        for (int mt = 0; mt < MH; ++mt) {
          const float2 p = f2(oPl + tsel + 128 * mt);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float xr = accU[fi][mt][q], yi = accU[fi][mt + MH][q];
            accU[fi][mt][q] = p.x * xr - p.y * yi;
            accU[fi][mt + MH][q] = p.x * yi + p.y * xr;
          }
        }
      }
    if constexpr (!GT) {
      if (u == 0 && lane < M) {
        const float2 ge = f2(oLn + tsel + (Lay::bGeo - Lay::bLE));
        eta = cmul(f2(oLn + tsel + (Lay::bPowL - Lay::bLE)),
                   make_float2(eta.x + ge.x, eta.y + ge.y));
      }
    }
    const bool more = c + 1 < x.c_end;
    __syncthreads();    // mid-chunk: phi(q), phi(k), lam U of chunk c no longer read
    // Gated: lam G <- D lam G + W^T (E V) (lam G_c was packed for the readout in phase one).
    if constexpr (GT) {
#pragma unroll
      for (int di = 0; di < NDT; ++di)
        if (u + NS * di < TD) {
#pragma unroll
          for (int kt = 0; kt < TM; ++kt)
#pragma unroll
            for (int q = 0; q < 4; ++q) accG[di][kt][q] *= dl;
        }
    }
#pragma unroll
    for (int kb = 0; kb < KC; ++kb) {
      bf16x8 bv[NDT];
#pragma unroll
      for (int di = 0; di < NDT; ++di)
        if (u + NS * di < TD) {
          bv[di] = ldtr<D>(s16, trD[di], kb).b;
          if constexpr (GT) bv[di] = gate_frag<C>(bv[di], rec, kb, g);
        }
#pragma unroll
      for (int kt = 0; kt < TM; ++kt) {
        const bf16x8 w = lds8(s16 + offC[kb] + 16 * kt * C).b;
#pragma unroll
        for (int di = 0; di < NDT; ++di)
          if (u + NS * di < TD) accG[di][kt] = mma_bf16(w, bv[di], accG[di][kt]);
        IA_STEP_FENCE();
      }
    }
    // Gated: lam eta <- lam^L D lam eta + lam beta sum_{j<L} lam^(L-1-j) E[j] (Horner in
    // fp32), in the second phase, whose registers are fewer.
    if constexpr (GT) {
      if (u == 0 && lane < M) {
        // Four tokens per Horner step, hs <- lam^4 hs + (lam^3 E[j] + lam^2 E[j+1] +
        // lam E[j+2] + E[j+3]), the four products independent; the padding tokens past the
        // sequence end (E = 0) would still multiply by lam, so a last, partial chunk takes the
        // one-token steps.
        const int Lc = min(C, a.N - c * C);
        const float2 l1 = lamh[lane];   // (loaded here: not held across the chunk loop)
        const float2 lb_m = cmul(l1, a.beta[(size_t)x.h * M + lane]);
        float2 hs = make_float2(0.f, 0.f);
        if (Lc == C) {
          const float2 l2 = cmul(l1, l1), l3 = cmul(l2, l1), l4 = cmul(l2, l2);
#pragma unroll 4
          for (int j4 = 0; j4 < C; j4 += 4) {
            const float4 e4 = *reinterpret_cast<const float4*>(rec + GR::E + j4);
            const float2 t = make_float2(l3.x * e4.x + l2.x * e4.y + l1.x * e4.z + e4.w,
                                         l3.y * e4.x + l2.y * e4.y + l1.y * e4.z);
            hs = cfma(l4, hs, t);
          }
        } else {
          for (int j = 0; j < Lc; ++j) hs = cfma(l1, hs, make_float2(rec[GR::E + j], 0.f));
        }
        const float2 pl = f2(oLn + tsel + (Lay::bPowL - Lay::bLE));
        eta = cfma(lb_m, hs, cmul(pl, make_float2(dl * eta.x, dl * eta.y)));
      }
    }
    if (more) {
      if (x.want_out) {
        write_lam_u();
        write_eta();
      }
      convert(c + 1);   // waits for the loads issued one chunk ago
      write_inputs();
      if (c + 2 < x.c_end) fetch(c + 2);
    }
    __syncthreads();    // chunk c read by every wave
  }
  if (x.c_begin < x.c_end) decay_g(x.c_end - 1);

  // Final state (divided by lam) in the caller's layout.
  float2 *fU = nullptr, *fG = nullptr, *fE = nullptr;
  if (x.last_seg && a.fin_U) {
    fU = a.fin_U + (size_t)x.seq * M * F;
    fG = a.fin_G + (size_t)x.seq * M * D;
    fE = a.fin_E + (size_t)x.seq * M;
  }
  if (fU) {
    const float2* inv = reinterpret_cast<const float2*>(x.tab + TL::oInv);
#pragma unroll
    for (int fi = 0; fi < NFT; ++fi) {
      const int ft = u + NS * fi;
      if (ft < F / 16) {
#pragma unroll
        for (int mt = 0; mt < MH; ++mt) {
          const int m = 16 * mt + il;
          const float2 li = inv[m];
#pragma unroll
          for (int q = 0; q < 4; ++q)
            fU[(size_t)m * F + 16 * ft + 4 * g + q] =
                cmul(li, make_float2(accU[fi][mt][q], accU[fi][mt + MH][q]));
        }
      }
    }
#pragma unroll
    for (int di = 0; di < NDT; ++di) {
      const int dt = u + NS * di;
      if (dt < TD) {
#pragma unroll
        for (int mt = 0; mt < MH; ++mt)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int m = 16 * mt + 4 * g + q;
            fG[(size_t)m * D + 16 * dt + il] =
                cmul(inv[m], make_float2(accG[di][mt][q], accG[di][mt + MH][q]));
          }
      }
    }
    if (u == 0 && lane < M) fE[lane] = cmul(inv[lane], eta);
  }
}

// The fp32 route of a head whose modes the bf16 chunk factorisation does not resolve
// (chunk_unresolved): the token-by-token recurrence of slice (b, h) over all N tokens by this
// workgroup, from the caller's state (updated in place) or from zero in the workspace state.
template <int C, int F, int D, int M, bool RM, bool GT>
__device__ __forceinline__ void fp32_route(const ChunkArgs& a, int b, int h, unsigned char* smem) {
  constexpr int NW = C / 16 + StateWaves<F, D, M>::NS;
  using S = SeqSmem<NW, F, D, M, RM>;
  static_assert(sizeof(S) <= Layout<C, F, D, M, C / 16, RM, GT>::bytes, "fits the kernel's LDS");
  S& s = *reinterpret_cast<S*>(smem);
  const size_t seq = (size_t)b * a.H + h;
  float2 *U, *G, *E;
  if (a.fin_U) {
    U = a.fin_U + seq * M * F;
    G = a.fin_G + seq * M * D;
    E = a.fin_E + seq * M;
  } else {
    U = a.wU + seq * M * F;
    G = a.wG + seq * M * D;
    E = a.wE + seq * M;
    for (int i = threadIdx.x; i < M * F; i += 64 * NW) U[i] = make_float2(0.f, 0.f);
    for (int i = threadIdx.x; i < M * D; i += 64 * NW) G[i] = make_float2(0.f, 0.f);
    for (int i = threadIdx.x; i < M; i += 64 * NW) E[i] = make_float2(0.f, 0.f);
    __syncthreads();
  }
  SeqScanArgs sa{a.q, a.k, a.v, a.sqk, a.sv, a.lam, a.beta, a.o, a.accumulate, a.N, a.H,
                 F, D, M, 1, a.out_bf16, a.clamp, a.dir, a.opt,
                 RM ? a.readout : nullptr};
  if constexpr (GT) {
    sa.wgate = a.wgate;
    sa.dgate = a.dgate;
  }
  seq_scan(s, sa, b, h, U, G, E);
}

template <int C, int F, int D, int M, bool RM, bool GT, int W>
__device__ __forceinline__ void run_role(const ChunkArgs& a, const Ctx<C, F, D, M>& x) {
  if constexpr (W < C / 16)
    readout_main<C, F, D, M, W, RM, GT>(a, x);
  else
    state_main<C, F, D, M, W - C / 16, RM, GT>(a, x);
}

template <int C, int F, int D, int M, bool RM, bool GT, int... Ws>
__device__ __forceinline__ void dispatch_role(const ChunkArgs& a, const Ctx<C, F, D, M>& x,
                                              int w, std::integer_sequence<int, Ws...>) {
  ((w == Ws ? (run_role<C, F, D, M, RM, GT, Ws>(a, x), 0) : 0), ...);
}
// RM: the readout matrix variant (a R in place of a before both readouts).  GT: the gated
// layer (write and decay gates per token, GateRec).
template <int C, int F, int D, int M, bool RM, bool GT>
__global__ void __launch_bounds__(64 * (C / 16 + StateWaves<F, D, M>::NS))
chunk_prefill_kernel(const ChunkArgs a) {
  using Lay = Layout<C, F, D, M, C / 16, RM, GT>;
  using TL = TableLayout<C, M>;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  uint16_t* s16 = reinterpret_cast<uint16_t*>(smem_raw);

  Ctx<C, F, D, M> x;
  x.s16 = s16;
  x.sFk = s16 + Lay::oFk;
  x.sFq = s16 + Lay::oFq;
  x.sV = s16 + Lay::oV;
  x.sWT = s16 + Lay::oWT;
  x.sWb = s16 + Lay::oWb;
  x.sLU = s16 + Lay::oLU;
  x.sGT = s16 + Lay::oGT;
  x.sC = reinterpret_cast<float*>(smem_raw + Lay::bC);
  x.sCi = reinterpret_cast<float*>(smem_raw + Lay::bCi);
  x.sLE = reinterpret_cast<float2*>(smem_raw + Lay::bLE);
  x.sPowL = reinterpret_cast<float2*>(smem_raw + Lay::bPowL);
  x.sGeo = reinterpret_cast<float2*>(smem_raw + Lay::bGeo);
  x.sL2lo = reinterpret_cast<float2*>(smem_raw + Lay::bL2lo);
  x.sL2hi = reinterpret_cast<float2*>(smem_raw + Lay::bL2hi);
  const int tid = threadIdx.x;
  x.lane = tid & 63;
  x.wave = tid >> 6;
  x.il = x.lane & 15;
  x.g = x.lane >> 4;
  {
    int seq, seg;
    if (!pair_wg(blockIdx.x, a.H * a.B, a.n_seg, a.pair_heads, seq, seg, a.H)) return;
    x.seq = seq;
    x.seg = a.seg_first + seg;
  }
  x.b = x.seq / a.H;
  x.h = x.seq % a.H;
  x.q0 = a.q + x.b * a.sqk.b + x.h * a.sqk.h;
  x.k0 = a.k + x.b * a.sqk.b + x.h * a.sqk.h;
  x.v0 = a.v + x.b * a.sv.b + x.h * a.sv.h;
  x.snqk = (int)a.sqk.n;
  x.snv = (int)a.sv.n;
  const int n_chunks_total = (a.N + C - 1) / C;
  x.c_begin = x.seg * a.seg_chunks;
  x.c_end = min(x.c_begin + a.seg_chunks, n_chunks_total);
  x.last_seg = x.c_end == n_chunks_total;
  x.want_out = a.o != nullptr;
  x.tab = a.tables + (size_t)x.h * a.table_bytes;
  if (__builtin_amdgcn_readfirstlane(*reinterpret_cast<const int*>(x.tab + TL::oRoute))) {
    if (x.seg == a.seg_first) fp32_route<C, F, D, M, RM, GT>(a, x.b, x.h, smem_raw);
    return;
  }

  x.wb_unscale = *reinterpret_cast<const float*>(x.tab + TL::oSc);
  x.r_unscale = RM ? *reinterpret_cast<const float*>(a.rtab + (size_t)x.h * a.rtab_bytes +
                                                     ReadoutTable<M>::oScale)
                   : 1.f;
  // Both roles run the same sequence of block barriers.  Each wave runs code specialised
  // for its index, so trip counts and owned tiles are compile-time constants.
  // The state waves copy the per-head tables to LDS as three contiguous runs: the decay
  // tables, the two lam^(2i) factor tables, and the per-mode pairs (decay and geometric sum of
  // a full and of the last chunk, then lam^Ls).  The layouts below make each run contiguous
  // on both sides.
  static_assert(Lay::oWb == Lay::oWT + 2 * M * C, "decay tables adjacent");
  static_assert(Lay::bL2hi == Lay::bL2lo + 16 * Lay::L2S * 8, "factor tables adjacent");
  static_assert(TL::nW == 2L * (Lay::oLU - Lay::oWT), "decay table size");
  static_assert(TL::nL2 == Lay::bL2end - Lay::bL2lo, "factor table size");
  static_assert(Lay::bGeoT - Lay::bGeo == Lay::kTail, "tail pair at one offset");
  static_assert(Lay::bPowS == Lay::bPowL + 4 * 8 * M, "lam^Ls after the decay pairs");
  static_assert(TL::oPowT - TL::oPow == 2 * 8 * M && TL::oGeoT - TL::oGeo == 2 * 8 * M,
                "decay pairs adjacent in the table");
  static_assert(Lay::bGeo == Lay::bPowL + 8 * M && Lay::bPowT == Lay::bGeo + 8 * M &&
                Lay::bGeoT == Lay::bPowT + 8 * M && Lay::bPowS == Lay::bGeoT + 8 * M,
                "per-mode arrays adjacent in LDS");
  static_assert(TL::oGeo == TL::oPow + 8 * M && TL::oPowT == TL::oGeo + 8 * M &&
                TL::oGeoT == TL::oPowT + 8 * M && TL::oPowS == TL::oGeoT + 8 * M,
                "per-mode arrays adjacent in the table");
  static_assert((Lay::oWT * 2) % 16 == 0 && Lay::bL2lo % 16 == 0 && Lay::bPowL % 16 == 0 &&
                TL::nW % 16 == 0 && TL::nL2 % 16 == 0 && (40 * M) % 16 == 0, "16-byte copies");
  dispatch_role<C, F, D, M, RM, GT>(
      a, x, x.wave, std::make_integer_sequence<int, C / 16 + StateWaves<F, D, M>::NS>{});
}

template <int C, int F, int D, int M, bool RM, bool GT>
hipError_t chunk_kernel_attr() {
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&chunk_prefill_kernel<C, F, D, M, RM, GT>),
        hipFuncAttributeMaxDynamicSharedMemorySize, Layout<C, F, D, M, C / 16, RM, GT>::bytes);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  return hipSuccess;
}

// Workgroups of the output-pass kernel one CU holds at once (LDS, registers, waves), or 0 if
// the runtime cannot say (no device).
template <int C, int F, int D, int M, bool RM = false, bool GT = false>
int chunk_occupancy_t() {
  if (chunk_kernel_attr<C, F, D, M, RM, GT>() != hipSuccess) return 0;
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &n, reinterpret_cast<const void*>(&chunk_prefill_kernel<C, F, D, M, RM, GT>),
          64 * (C / 16 + StateWaves<F, D, M>::NS), Layout<C, F, D, M, C / 16, RM, GT>::bytes) !=
      hipSuccess)
    return 0;
  return n;
}

template <int C, int F, int D, int M, bool RM = false, bool GT = false>
hipError_t launch_chunk_t(const ChunkArgs& a, int n_wg, hipStream_t st, int kind) {
  constexpr int threads = 64 * (C / 16 + StateWaves<F, D, M>::NS);
  constexpr int bytes = Layout<C, F, D, M, C / 16, RM, GT>::bytes;
  static_assert(bytes <= 160 * 1024, "LDS budget");
  {
    hipError_t e = chunk_kernel_attr<C, F, D, M, RM, GT>();
    if (e != hipSuccess) return e;
  }
  (void)hipGetLastError();
  prof_begin(st);
  hipLaunchKernelGGL((chunk_prefill_kernel<C, F, D, M, RM, GT>), dim3(n_wg), dim3(threads), bytes,
                     st, a);
  prof_end(st, kind);
  return hipGetLastError();
}

}  // namespace ia
