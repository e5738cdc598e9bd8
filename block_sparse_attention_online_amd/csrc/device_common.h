// Device helpers shared by the gfx950 kernels: vector types for the bf16 MFMA
// operands, bf16 packing, wave reductions, and the key-tile visit order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace ssattn {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2_t;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kTile = 128;  // keys per tile, query rows per prefill decision block

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }
__device__ __forceinline__ float pos_inf() { return __builtin_inff(); }

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t u) {
  return __builtin_bit_cast(bf16x8_t, u);
}

__device__ __forceinline__ float bf16_lo(unsigned int w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(unsigned int w) { return __uint_as_float(w & 0xffff0000u); }

// Two fp32 values -> packed bf16 pair (round to nearest even, v_cvt_pk_bf16_f32).
__device__ __forceinline__ unsigned int pack_bf16x2(float lo, float hi) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
  bf16x2_t r;
  r[0] = (__bf16)lo;
  r[1] = (__bf16)hi;
  return __builtin_bit_cast(unsigned int, r);
}

// acc + lo + hi of a packed bf16 pair, one v_dot2c_f32_bf16 against (1, 1): a
// row sum of probabilities taken from the very bf16 values the P*V product
// uses, at half the vector instructions of two fp32 adds.
__device__ __forceinline__ float add_bf16x2(unsigned int w, float acc) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
  const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w), ones, acc, false);
}

// 2^x on the hardware exponential unit.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---- cross-lane helpers -------------------------------------------------------

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, true));
}
constexpr int kDppXor1 = 0xB1;          // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;          // quad_perm [2,3,0,1]
constexpr int kDppRor4 = 0x124;         // row_ror:4
constexpr int kDppRor8 = 0x128;         // row_ror:8
constexpr int kDppHalfMirror = 0x141;   // row_half_mirror

// Sum over each aligned group of N lanes (N = 8 or 16); every lane of the
// group receives the total.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 8 || N == 16, "group size");
  if constexpr (N == 16) {
    x += dpp<kDppRor8>(x);
    x += dpp<kDppRor4>(x);
  } else {
    x += dpp<kDppHalfMirror>(x);
  }
  x += dpp<kDppXor2>(x);
  x += dpp<kDppXor1>(x);
  return x;
}

__device__ __forceinline__ float shfl_xor_f(float x, int mask) { return __shfl_xor(x, mask, 64); }

// The lane index, computed afresh at each use (the asm keeps the compiler from
// merging it with other copies): lets code deep in a loop derive lane-dependent
// offsets in two instructions instead of holding them in registers all along.
__device__ __forceinline__ int lane_id_fresh() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// Lane l combined with lane l ^ 32, without LDS or an address register:
// v_permlane32_swap with x as both operands returns lanes 0..31 of x in both
// halves of its first result and lanes 32..63 in both halves of the second.
// Both lanes of a pair get the same value (same operand order).
__device__ __forceinline__ float max_xor32(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Max over all 64 lanes, returned to every lane: DPP within each row of 16
// lanes, then the four row results through readlane (no LDS round trips).
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp<kDppXor1>(x));
  x = fmaxf(x, dpp<kDppXor2>(x));
  x = fmaxf(x, dpp<kDppRor4>(x));
  x = fmaxf(x, dpp<kDppRor8>(x));
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// Workgroup order for L2 sharing.  The hardware hands workgroup p to XCD
// p % 8; this returns the logical work index for physical index p such that
// each XCD owns one contiguous range of logical indices, so work items that
// are adjacent in logical order (and read the same key/value tiles at the same
// time) run on the same XCD, behind the same L2.  A bijection on [0, n).
__device__ __forceinline__ int xcd_local_order(int p, int n) {
  const int x = p & 7, s = p >> 3;
  const int per = n >> 3, rem = n & 7;
  return x * per + min(x, rem) + s;
}

// Max over lanes whose index differs only in bits [lo_bit, 6).
template <int LO>
__device__ __forceinline__ float lanes_max_from(float x) {
#pragma unroll
  for (int m = 32; m >= LO; m >>= 1) x = fmaxf(x, shfl_xor_f(x, m));
  return x;
}
template <int LO>
__device__ __forceinline__ float lanes_sum_from(float x) {
#pragma unroll
  for (int m = 32; m >= LO; m >>= 1) x += shfl_xor_f(x, m);
  return x;
}


// ---- direct-to-LDS rings ------------------------------------------------------

// s_waitcnt with vmcnt = N and no wait on the other counters (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Workgroup barrier for the ring.  __syncthreads (and any release fence that
// covers LDS) waits for every outstanding direct-to-LDS load, which would
// leave one step in flight instead of two; this barrier waits only for the
// wave's own LDS operations (lgkmcnt), and the "memory" clobber keeps the
// compiler from moving memory accesses across it.  Direct-to-LDS loads are
// waited for explicitly (wait_vmcnt) before it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// One direct global -> LDS load of 16 bytes per lane: lane l's bytes at
// gbase + goff land at LDS address lds + 16 l.  Written out rather than through
// the compiler builtin: with the builtin in a loop the compiler waits for every
// outstanding LDS read (lgkmcnt 0) before each use of one, which defeats the
// read-ahead of the MFMA operands.  The ring waits for these loads itself
// (wait_vmcnt); the compiler's own vmcnt waits count only the loads it knows,
// which can only make them stricter.  M0 holds the LDS address and is
// restored; the wait states after each M0 write are the ones the hardware
// needs before a read of M0.
__device__ __forceinline__ void dma16(const void* gbase, unsigned goff, const unsigned char* lds) {
  const unsigned la =
      (unsigned)(uintptr_t)(const __attribute__((address_space(3))) unsigned char*)lds;
  unsigned saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %2, %3\n\ts_mov_b32 m0, %0\n\ts_nop 0"
      : "=&s"(saved)
      : "s"(la), "v"(goff), "s"(gbase)
      : "memory");
}

// Four such loads whose global and LDS addresses step by 1024 bytes: load x
// (0..3) brings lane l's bytes at gbase + goff[x] + 1024 x to LDS address
// lds + 1024 x + 16 l.  The instruction offset of a direct-to-LDS load moves
// its global and its LDS address alike (observed on gfx950), so M0 is
// written once for the four instead of twice per load.
__device__ __forceinline__ void dma16_run4(const void* gbase, const unsigned (&goff)[4],
                                           const unsigned char* lds) {
  const unsigned la =
      (unsigned)(uintptr_t)(const __attribute__((address_space(3))) unsigned char*)lds;
  unsigned saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %2, %6\n\t"
      "global_load_lds_dwordx4 %3, %6 offset:1024\n\t"
      "global_load_lds_dwordx4 %4, %6 offset:2048\n\t"
      "global_load_lds_dwordx4 %5, %6 offset:3072\n\t"
      "s_mov_b32 m0, %0\n\ts_nop 0"
      : "=&s"(saved)
      : "s"(la), "v"(goff[0]), "v"(goff[1]), "v"(goff[2]), "v"(goff[3]), "s"(gbase)
      : "memory");
}

// ---- LDS tile swizzle for row and transpose reads --------------------------------

// Physical 16-byte chunk of logical chunk c in row r of a tile image with
// D bf16 elements per row, for an image read two ways (the backward's Q, dO,
// K and V; the forward's V), conflict-free for both:
//  * row reads (MFMA operand with k along the row): one chunk of 16
//    consecutive rows per LDS cycle, so the XOR term must take 16 different
//    values over r & 15;
//  * transpose reads (ds_read_b64_tr_b16, k across rows): 64 bytes (4 chunks)
//    of 4 consecutive rows per 32 lanes, so those 4 rows must land on 4
//    different 64-byte bank groups.
// D = 128: a row is one 256-byte bank line; chunk bits 2-3 take r & 3, bits
// 0-1 take (r >> 2) & 3.  D = 64: two rows per bank line (r & 1 picks the
// half); chunk bit 2 takes bit 1 of r, bits 0-1 take (r >> 2) & 3.  Either
// term is a bijection on r & 15, and XOR with it is its own inverse.
template <int D>
__device__ __forceinline__ int dual_slot(int r, int c) {
  return D == 128 ? c ^ (((r & 3) << 2) | ((r >> 2) & 3))
                  : c ^ ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}

// Per-lane offset of a row read: the A operand of a 32x32x16 MFMA whose rows
// are tile rows 32 blk + l % 32 and whose k-step ks covers elements
// 16 ks + 8 (l / 32) .. + 8 of the row.  The swizzle sees r & 15 only, so the
// 32-row block is an immediate offset (blk * 32 * ROW).
template <int D>
__device__ __forceinline__ int dual_row_off(int lane, int ks) {
  const int l32 = lane & 31, g = lane >> 5;
  return l32 * 2 * D + (dual_slot<D>(l32, 2 * ks + g) << 4);
}

// Per-lane offset of a transpose read: the A operand (rows = tile columns
// 32 mb + l % 32, k = tile rows) of a 16-row k-step, in the row order that the
// MFMA accumulator layout gives its B operand: lane half g takes rows
// 4 g .. 4 g + 3 (hi = 0) and 8 + 4 g .. 8 + 4 g + 3 (hi = 1) of the step.
// Each 16-lane group reads 4 rows x 16 columns (lane: row r16 / 4, columns
// 4 (r16 % 4) .. + 4 of its 16) and receives one column's 4 rows.
template <int D>
__device__ __forceinline__ int dual_tr_off(int lane, int mb, int hi) {
  const int g = lane >> 5, r16 = lane & 15;
  const int R = 4 * g + (r16 >> 2) + 8 * hi;
  const int c = 4 * mb + 2 * ((lane >> 4) & 1) + ((r16 & 3) >> 1);
  return R * 2 * D + (dual_slot<D>(R, c) << 4) + (r16 & 1) * 8;
}

// The swizzle is an XOR of chunk bits with row bits, so the offsets of the
// other k-steps (row reads) and column blocks / halves (transpose reads)
// follow from the first by XOR with constants: one register per kind.
//   dual_row_off<D>(l, ks)     == dual_row_off<D>(l, 0) ^ (ks << 5)
//   dual_tr_off<D>(l, mb, hi)  == dual_tr_off<D>(l, 0, 0) ^ dual_tr_xor<D>(mb, hi)
template <int D>
__device__ __forceinline__ constexpr int dual_tr_xor(int mb, int hi) {
  // hi moves the rows by 8 (bit 11 of the offset for D = 128, bit 10 for
  // D = 64) and flips bit 1 of the swizzle term ((R >> 2) & 3 gains 2)
  return (mb << 6) ^ (hi << 5) ^ (hi << (D == 128 ? 11 : 10));
}

template <class F, int... E>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, E...>) {
  (f(std::integral_constant<int, E>{}), ...);
}
// f(integral_constant<int, 0>), ..., f(integral_constant<int, N - 1>)
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// ---- key-tile visit order ---------------------------------------------------------

// Tiles visited by one query tile of a prefill call: `count` tiles starting at
// `first`; the t-th visited tile is tile_at(t).  Causal keeps only tiles with
// a key visible to some row (key c visible to row r iff c <= r + Lk - Lq).
struct VisitPlan {
  int count;  // number of visited tiles
  int last;   // causal: highest visited tile
  int start;  // non-causal diag_first: first tile
  int nK;
  int causal;
  int diag_first;
  // tile_at(t) = base + t, or base - t when `down`, less nK past the end
  // (only a non-causal diag_first visit wraps): no branch on the order.
  int base;
  int down;

  __device__ __forceinline__ int tile_at(int t) const {
    const int j = base + (down ? -t : t);
    return j >= nK ? j - nK : j;
  }
};

__device__ __forceinline__ VisitPlan make_visit_plan(int qtile, int Lq, int Lk, int causal,
                                                     int diag_first) {
  VisitPlan p;
  p.nK = (Lk + kTile - 1) / kTile;
  p.causal = causal;
  p.diag_first = diag_first;
  const int r0 = qtile * kTile;
  const int r1 = min(r0 + kTile, Lq) - 1;
  if (causal) {
    const long last_key = (long)r1 + Lk - Lq;
    if (last_key < 0) {
      p.count = 0;
      p.last = -1;
    } else {
      p.last = min(p.nK - 1, (int)(last_key / kTile));
      p.count = p.last + 1;
    }
    p.start = 0;
  } else {
    p.count = p.nK;
    p.last = p.nK - 1;
    long s = ((long)r0 + Lk - Lq) / kTile;
    if ((long)r0 + Lk - Lq < 0) s = 0;
    p.start = (int)min((long)(p.nK - 1), s);
  }
  // visit orders: causal diag_first last, last - 1, ..., 0; non-causal
  // diag_first start, ..., nK - 1, 0, ..., start - 1; ascending 0, 1, ...
  p.down = causal && diag_first;
  p.base = causal ? (diag_first ? p.last : 0) : (diag_first ? p.start : 0);
  return p;
}

}  // namespace ssattn
