// Device helpers shared by the two backward kernels of the skip-softmax
// prefill (prefill_bwd_dkdv.hip, prefill_bwd_dq.hip): the LDS image of a
// 128-row tile, its direct-to-LDS loads, and its row and transpose reads.
#pragma once

#include "device_common.h"

namespace ssattn {

typedef __attribute__((ext_vector_type(4))) short bw_s16x4_t;
typedef __attribute__((address_space(3))) bw_s16x4_t bw_lds_s16x4_t;

// Entries of the work lists a backward workgroup compacts from the skip mask
// (one refill; longer lists are walked in several refills).
constexpr int kBwdListCap = 2048;
constexpr int kMaskKept = 0;  // skip-mask byte of a tile the forward computed

// Physical 16-byte chunk of logical chunk c in row r of a tile image with
// D bf16 elements per row.  Every backward tile is read two ways:
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
__device__ __forceinline__ int bw_slot(int r, int c) {
  return D == 128 ? c ^ (((r & 3) << 2) | ((r >> 2) & 3))
                  : c ^ ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}

// Direct-to-LDS loads of one 128-row tile (rows of D bf16 elements starting
// at `src`) into the image at `dst`, swizzled by bw_slot.  The NW waves of the
// workgroup share the tile's 1024-byte load instructions; lane l of a load
// writes physical chunk l % (D / 8) of its row and so fetches the logical
// chunk that bw_slot puts there.  Rows past `rlast` (>= 0) re-read row rlast.
template <int D, int NW>
__device__ __forceinline__ void bw_issue_tile(const unsigned char* src, int rlast,
                                              unsigned char* dst, int w) {
  constexpr int ROW = 2 * D, KCH = D / 8, RPL = 64 / KCH, LOADS = kTile / RPL / NW;
  static_assert(LOADS >= 1 && LOADS * RPL * NW == kTile, "tile split");
  const int ln = lane_id_fresh();
  const int lr = ln / KCH, pc = ln % KCH;
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int r = (w * LOADS + i) * RPL + lr;
    const unsigned go = (unsigned)min(r, rlast) * ROW + ((unsigned)bw_slot<D>(r, pc) << 4);
    __builtin_amdgcn_global_load_lds(
        (const void __attribute__((address_space(1)))*)(src + go),
        (void __attribute__((address_space(3)))*)(dst + (w * LOADS + i) * RPL * ROW), 16, 0, 0);
  }
}

// Per-lane offset of a row read: the A operand of a 32x32x16 MFMA whose rows
// are tile rows 32 blk + l % 32 and whose k-step ks covers elements
// 16 ks + 8 (l / 32) .. + 8 of the row.  The swizzle sees r & 15 only, so the
// 32-row block is an immediate offset (blk * 32 * ROW).
template <int D>
__device__ __forceinline__ int bw_row_off(int lane, int ks) {
  const int l32 = lane & 31, g = lane >> 5;
  return l32 * 2 * D + (bw_slot<D>(l32, 2 * ks + g) << 4);
}

// Per-lane offset of a transpose read: the A operand (rows = tile columns
// 32 mb + l % 32, k = tile rows) of a 16-row k-step, in the row order that the
// MFMA accumulator layout gives its B operand: lane half g takes rows
// 4 g .. 4 g + 3 (hi = 0) and 8 + 4 g .. 8 + 4 g + 3 (hi = 1) of the step.
// Each 16-lane group reads 4 rows x 16 columns (lane: row r16 / 4, columns
// 4 (r16 % 4) .. + 4 of its 16) and receives one column's 4 rows.
template <int D>
__device__ __forceinline__ int bw_tr_off(int lane, int mb, int hi) {
  const int g = lane >> 5, r16 = lane & 15;
  const int R = 4 * g + (r16 >> 2) + 8 * hi;
  const int c = 4 * mb + 2 * ((lane >> 4) & 1) + ((r16 & 3) >> 1);
  return R * 2 * D + (bw_slot<D>(R, c) << 4) + (r16 & 1) * 8;
}

// The swizzle is an XOR of chunk bits with row bits, so the offsets of the
// other k-steps (row reads) and column blocks / halves (transpose reads)
// follow from the first by XOR with constants: one register per kind.
//   bw_row_off<D>(l, ks)     == bw_row_off<D>(l, 0) ^ (ks << 5)
//   bw_tr_off<D>(l, mb, hi)  == bw_tr_off<D>(l, 0, 0) ^ bw_tr_xor<D>(mb, hi)
template <int D>
__device__ __forceinline__ constexpr int bw_tr_xor(int mb, int hi) {
  // hi moves the rows by 8 (bit 11 of the offset for D = 128, bit 10 for
  // D = 64) and flips bit 1 of the swizzle term ((R >> 2) & 3 gains 2)
  return (mb << 6) ^ (hi << 5) ^ (hi << (D == 128 ? 11 : 10));
}

// Transpose read of 8 rows (lo and hi halves) at `p + off_lo` / `p + off_hi`.
__device__ __forceinline__ bf16x8_t bw_tr_read(const unsigned char* p, int off_lo, int off_hi) {
  const bw_s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((bw_lds_s16x4_t*)(p + off_lo));
  const bw_s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((bw_lds_s16x4_t*)(p + off_hi));
  const u32x2_t l2 = __builtin_bit_cast(u32x2_t, lo);
  const u32x2_t h2 = __builtin_bit_cast(u32x2_t, hi);
  return as_bf16x8(u32x4_t{l2[0], l2[1], h2[0], h2[1]});
}

// Sixteen fp32 accumulator values of one 32-row (or 32-key) block as the two
// bf16 B operands of the 16-wide k-steps that follow in the accumulator's
// row order.
__device__ __forceinline__ void bw_pack_b(const float (&x)[16], bf16x8_t (&out)[2]) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    u32x4_t u;
#pragma unroll
    for (int e = 0; e < 4; ++e) u[e] = pack_bf16x2(x[8 * h + 2 * e], x[8 * h + 2 * e + 1]);
    out[h] = as_bf16x8(u);
  }
}

}  // namespace ssattn
