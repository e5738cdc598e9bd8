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

// Direct-to-LDS loads of one 128-row tile (rows of D bf16 elements starting
// at `src`, a wave-uniform address) into the image at `dst`, swizzled by
// dual_slot.  Written out (dma16, dma16_run4), not through the compiler
// builtin, which makes the compiler wait for every outstanding LDS read
// (lgkmcnt 0) before each use of one; the kernels wait for these loads
// themselves (s_waitcnt 0 before the ring's barrier).  The NW waves of the
// workgroup share the tile's 1024-byte load instructions; lane l of a load
// writes physical chunk l % (D / 8) of its row and so fetches the logical
// chunk that dual_slot puts there.  Rows past `rlast` (>= 0) re-read row rlast.
//
// `go0` is the lane's source offset for load 0 (bw_issue_off0), formed once
// per workgroup: load i of a full tile covers rows i * (64 / (D / 8)) further
// on, 1024 bytes for D = 64 and 128, and the swizzle of its rows differs from
// load 0's by XOR with chunk bits -- (i & 3) << 4 bytes for D = 128, (i & 1)
// << 5 for D = 64 -- because dual_slot reads row bits 0-3 only and the
// wave's first row is a multiple of 16.  Formed at each load, the offsets
// cost about a fifth of the dK/dV kernel's vector instructions.
template <int D, int NW>
struct BwLoads {
  static constexpr int ROW = 2 * D, KCH = D / 8, RPL = 64 / KCH, LOADS = kTile / RPL / NW;
  static_assert(LOADS >= 1 && LOADS * RPL * NW == kTile, "tile split");
  static_assert(RPL * ROW == 1024 && LOADS % 4 == 0, "offset step of a load, runs of four");
};

template <int D, int NW>
__device__ __forceinline__ unsigned bw_issue_off0(int w) {
  using L = BwLoads<D, NW>;
  const int ln = lane_id_fresh();
  const int r = w * L::LOADS * L::RPL + ln / L::KCH;
  return (unsigned)r * L::ROW + ((unsigned)dual_slot<D>(r, ln % L::KCH) << 4);
}

template <int D, int NW>
__device__ __forceinline__ void bw_issue_tile(const unsigned char* src, int rlast,
                                              unsigned char* dst, int w, unsigned go0) {
  using L = BwLoads<D, NW>;
  if (rlast >= kTile - 1) {
    // load 4 h + x: 4096 h in the addresses, 1024 x in the instruction offset,
    // which moves the global and the LDS address alike (one M0 per four)
    unsigned gx[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) gx[x] = go0 ^ (unsigned)(D == 128 ? x << 4 : (x & 1) << 5);
    unsigned char* d0 = dst + w * L::LOADS * L::RPL * L::ROW;
#pragma unroll
    for (int h = 0; h < L::LOADS / 4; ++h) dma16_run4(src + h * 4096, gx, d0 + h * 4096);
    return;
  }
  const int ln = lane_id_fresh();
  const int lr = ln / L::KCH, pc = ln % L::KCH;
#pragma unroll
  for (int i = 0; i < L::LOADS; ++i) {
    const int r = (w * L::LOADS + i) * L::RPL + lr;
    const unsigned go = (unsigned)min(r, rlast) * L::ROW + ((unsigned)dual_slot<D>(r, pc) << 4);
    dma16(src, go, dst + (w * L::LOADS + i) * L::RPL * L::ROW);
  }
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
