// Skip-softmax (BLASST) prefill, bf16 inputs, fp32 accumulation, gfx950.
//
// Method: vLLM-Omni design page "Skip-Softmax" -- section "The online-softmax
// pass" (per-row running max m, denominator l and numerator O, rescaled when m
// grows; one streaming pass over 128-key tiles) and section "The skip test"
// (a tile whose exp(tile_max - running_max) is below the threshold
// contributes nothing: no exponentials, no P.V).  Section "What this bounds":
// the score product Q.K^T always runs.  BLASST summary page, section
// "Kernel-ontwerp": the prefill kernel skips both the softmax and the matrix
// multiply of skipped blocks.
//
// Design (one workgroup = one 128-row query tile of NH query heads that share
// a KV head -- NH = 2 when the group size is even, else 1 -- with 4 waves of
// 32 rows per head, one workgroup per compute unit):
//  * The NH heads visit the same key/value tiles in the same order, so every
//    tile brought into LDS serves all of them; each head keeps its own
//    128-row skip decision and its own running state.  With NH = 2 every SIMD
//    runs two waves, which cover each other's LDS and memory waits (they
//    step through the same phases together, so one wave's exponentials do
//    not run beside the other's MFMAs).
//  * K and V tiles move from global memory straight into LDS
//    (global_load_lds, 16 bytes per lane, no registers), into a two-stage
//    ring: the next tile's loads are in flight while the current tile is
//    multiplied.  Which lane fetches which 16-byte chunk is permuted so the
//    LDS image is XOR-swizzled for conflict-free operand reads.
//  * Scores are computed transposed, S^T = K Q^T with
//    v_mfma_f32_32x32x16_bf16: K is the A operand (16-byte LDS reads), Q^T the
//    B operand held in registers for the whole pass.  The accumulator layout
//    gives every lane one query row and 16 keys per 32-key block, so the row
//    max, the running state and the exponentials stay in the lane that owns
//    the row.
//  * The output is accumulated transposed too, O^T += V^T P^T: the lane's bf16
//    exponentials are already the B operand (its row, 8 keys); the V^T A
//    operand comes from the row-major V tile through ds_read_b64_tr_b16
//    transpose reads (each 16-lane group turns 4 keys x 16 value columns into
//    4 keys per column).
//  * The skip decision: per row delta = tile_max - m (log2 units); skip when
//    the max of delta over the head's 128 rows is below log2(threshold), i.e.
//    when no row passes its own test -- a ballot over each wave's rows, an OR
//    over the head's 4 waves through LDS.  The branch is uniform over the
//    head's waves, so a skipped tile issues no exp and no P.V MFMA at all.
//    With per-row decisions the tile is still skipped exactly when every row
//    fails the test; in a kept tile a row that fails it takes +inf as its
//    exponent reference, so its P is 0 and it adds nothing.

#include "device_common.h"
#include "launch.h"

namespace ssattn {
namespace {

constexpr int kRowWaves = 4;  // waves per head: 4 x 32 rows

typedef __attribute__((ext_vector_type(4))) short s16x4_t;
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

// Physical 16-byte chunk of logical chunk c in row r of the K image.  The
// A-operand reads take the same logical chunk of 16 consecutive rows in one
// LDS cycle (16 lanes x 16 bytes over 64 four-byte banks), so those 16 chunks
// must sit in 16 different 16-byte bank groups: with 256-byte rows (D = 128)
// every row starts at bank 0 and the chunk is XORed with four row bits; with
// 128-byte rows (D = 64) two rows share a bank line and the chunk is XORed
// with the pair index.
template <int D>
__device__ __forceinline__ int k_slot(int r, int c) {
  return D == 128 ? c ^ (r & 15) : c ^ ((r >> 1) & 7);
}

// QP = false: the NH = 2 row sets are two query heads of one KV group on one
// query tile.  QP = true (group sizes that are odd, e.g. one query head per KV
// head): the two row sets are two neighbouring query tiles of one head, and the
// workgroup streams the key tiles both visit -- each set takes exactly its own
// visit order out of the shared stream and sits out the steps it has no tile
// in (a causal tile's sequence is one tile shorter than its upper
// neighbour's; in diag_first order without causality the two rotations are
// one tile apart, so the stream is one tile longer than either).
template <int D, int NH, bool QP>
__global__ __launch_bounds__(64 * kRowWaves * NH, 1) void prefill_bf16_kernel(PrefillArgs a) {
  static_assert(!QP || NH == 2, "query-tile pairs need two row sets");
  constexpr int NW = kRowWaves * NH;         // waves in the workgroup
  constexpr int KCH = D / 8;                 // 16-byte chunks per row
  constexpr int KS = D / 16;                 // MFMA k-steps over the head dimension
  constexpr int MB = D / 32;                 // 32-wide value-column blocks
  constexpr int ROW = D * 2;                 // bytes per row
  constexpr int TILE_BYTES = kTile * ROW;    // one K or V tile
  constexpr int ROWS_PER_LOAD = 64 / KCH;    // rows one wave instruction covers
  // The tile loads are issued by the waves of row set 0 only (one per SIMD):
  // the loads a wave issues slow its own MFMA and vector work, so each SIMD
  // keeps one wave that issues none (measured faster than spreading the loads
  // over all waves or between the score blocks).
  constexpr int LW = kRowWaves;                      // loading waves: 0 .. LW-1
  constexpr int LOADS = kTile / ROWS_PER_LOAD / LW;  // per loading wave per tile (each of K, V)
  static_assert(LOADS >= 1 && LOADS * ROWS_PER_LOAD * LW == kTile, "tile split");

  // Two-stage ring.  Its loads are direct-to-LDS loads written out in
  // assembly (dma16_run4, dma16), which the compiler does not track: one loop body serves
  // both stages through a runtime stage base (no duplicated body, no copies of
  // the accumulators between two register assignments), and the ring waits
  // for its loads itself (vmcnt 0 before the barrier at the top of a step).
  __shared__ __attribute__((aligned(1024))) unsigned char kst[2][TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char vst[2][TILE_BYTES];
  __shared__ int red[NH][kRowWaves];  // per wave: some row of it passes its own test

  const int nQ = (a.Lq + kTile - 1) / kTile;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = w / kRowWaves;              // this wave's row set
  const int wr = w % kRowWaves;              // this wave's 32-row block
  // Logical order: (batch, KV head, query tile, head set within the group) --
  // QP: (batch, KV head, head within the group, query-tile pair) -- so work
  // items that read the same key/value tiles at the same time are adjacent
  // and, through xcd_local_order, share an XCD's L2.  Heaviest query tiles
  // first when causal.
  const int grp_sz = a.Hq / a.Hkv;
  const int L = xcd_local_order(blockIdx.x, gridDim.x);
  int hk, b, head, qtile, qpair = 0;
  if constexpr (QP) {
    const int nQP = (nQ + 1) / 2;
    const int pi = L % nQP;
    const int hin = (L / nQP) % grp_sz;
    hk = (L / (nQP * grp_sz)) % a.Hkv;
    b = L / (nQP * grp_sz * a.Hkv);
    qpair = a.causal ? nQP - 1 - pi : pi;
    head = hk * grp_sz + hin;
    qtile = 2 * qpair + hh;
  } else {
    const int sets = grp_sz / NH;
    const int hs = L % sets;
    const int qi = (L / sets) % nQ;
    hk = (L / (sets * nQ)) % a.Hkv;
    b = L / (sets * nQ * a.Hkv);
    qtile = a.causal ? nQ - 1 - qi : qi;
    head = hk * grp_sz + hs * NH + hh;
  }
  const bool qtile_ok = qtile < nQ;  // QP with an odd tile count: the last pair's upper set is empty
  const int l32 = lane & 31;
  const int g = lane >> 5;  // MFMA k-group of this lane
  const int row0 = qtile * kTile;
  const int rq = row0 + wr * 32 + l32;  // the query row this lane owns
  const bool row_ok = rq < a.Lq;
  const int shift = a.Lk - a.Lq;

  const unsigned short* kp =
      static_cast<const unsigned short*>(a.k) + ((size_t)(b * a.Hkv + hk) * a.Lk) * D;
  const unsigned short* vp =
      static_cast<const unsigned short*>(a.v) + ((size_t)(b * a.Hkv + hk) * a.Lk) * D;

  const VisitPlan plan = make_visit_plan(qtile_ok ? qtile : nQ - 1, a.Lq, a.Lk, a.causal, a.order);
  const int nK = plan.nK;
  const int count = qtile_ok ? plan.count : 0;  // tiles this row set visits
  // The stream of key tiles the workgroup loads: U steps; this row set takes
  // its visit t at stream step u0 + t.
  int U = count, u0 = 0;
  VisitPlan pl0 = plan, pl1 = plan;
  int c0 = count, c1 = count, s0 = 0, s1 = 0;
  if constexpr (QP) {
    const int q0 = 2 * qpair, q1 = 2 * qpair + 1;
    pl0 = make_visit_plan(q0, a.Lq, a.Lk, a.causal, a.order);
    pl1 = make_visit_plan(q1 < nQ ? q1 : q0, a.Lq, a.Lk, a.causal, a.order);
    c0 = pl0.count;
    c1 = q1 < nQ ? pl1.count : 0;
    if (a.causal) {
      // both end on tile 0 (diag_first) or start on it (ascending)
      U = max(c0, c1);
      if (a.order == SS_ORDER_DIAG_FIRST) {
        s0 = U - c0;
        s1 = U - c1;
      }
    } else if (a.order == SS_ORDER_DIAG_FIRST && c1 > 0 && pl1.start != pl0.start) {
      // rotations one tile apart: start_1 = start_0 + 1
      U = c0 + 1;
      s1 = 1;
    } else {
      U = max(c0, c1);
    }
    u0 = hh == 0 ? s0 : s1;
  }
  // the key tile of stream step u
  auto stream_tile = [&](int u) __attribute__((always_inline)) {
    if constexpr (QP) {
      const int t0 = u - s0;
      return (t0 >= 0 && t0 < c0) ? pl0.tile_at(t0) : pl1.tile_at(u - s1);
    } else {
      return plan.tile_at(u);
    }
  };
  // this head's mask row; its first wave writes it
  uint8_t* const mrow =
      a.mask && qtile_ok ? a.mask + ((size_t)(b * a.Hq + head) * nQ + qtile) * nK : nullptr;
  const bool mask_writer = mrow && wr == 0;
  if (mask_writer && plan.causal)
    for (int j = plan.last + 1 + lane; j < nK; j += 64) mrow[j] = 2;
  // per-row decisions: this lane's row of the row mask (lane half 0 writes)
  // (its address is formed where it is written, not held across the tiles)
  const bool row_writer = a.row_mask && g == 0 && row_ok;
  auto rrow = [&]() __attribute__((always_inline)) {
    return a.row_mask + ((size_t)(b * a.Hq + head) * a.Lq + rq) * nK;
  };
  if (row_writer && plan.causal)
    for (int j = plan.last + 1; j < nK; ++j) rrow()[j] = 2;

  // Issue the direct-to-LDS loads of tile j into ring stage st.  Loading wave
  // w covers rows [w * LOADS * ROWS_PER_LOAD, ...); lane l of load i writes LDS row
  // (base row + l / KCH), physical chunk l % KCH, and fetches the logical
  // chunk that the swizzle puts there.  Rows past Lk read the last key row
  // (their scores are masked to -inf, their P is 0).
  // Addresses: the tile's first row is a wave-uniform base; the lane's offset
  // within a full tile follows from its offset for load 0 (kgo0, vgo0): load i
  // covers rows 1024 i / ROW further on, and the swizzle of its rows differs
  // from load 0's by XOR with chunk bits -- K (k_slot): bits 2-3, (i & 3) << 2
  // for D = 128, (i & 1) << 2 for D = 64; V (dual_slot): bits 0-1, i & 3 for
  // D = 128, (i & 1) << 1 for D = 64.  kgo0 and vgo0 are formed once and held
  // across the tile loop, like the operand offsets below: every vector
  // instruction taken out of the loop shortens it, since the vector work
  // does not run beside the MFMAs.  A full tile's loads go out in runs of
  // four that share one M0 write (dma16_run4), each run's 1024-byte steps
  // in the instruction offsets.  Only the last tile clamps rows.
  unsigned kgo0, vgo0;
  {
    const int ln = lane_id_fresh();
    const int lr = ln / KCH, pc = ln % KCH;
    const int r = w * LOADS * ROWS_PER_LOAD + lr;
    kgo0 = (unsigned)r * ROW + ((unsigned)k_slot<D>(r, pc) << 4);     // an involution
    vgo0 = (unsigned)r * ROW + ((unsigned)dual_slot<D>(r, pc) << 4);  // likewise
  }
  auto issue_tile = [&](int j, int st) {
    if (w >= LW) return;
    const int j0 = j * kTile;
    const unsigned char* kt = reinterpret_cast<const unsigned char*>(kp) + (size_t)j0 * ROW;
    const unsigned char* vt = reinterpret_cast<const unsigned char*>(vp) + (size_t)j0 * ROW;
    unsigned char* kd = kst[st] + w * LOADS * ROWS_PER_LOAD * ROW;
    unsigned char* vd = vst[st] + w * LOADS * ROWS_PER_LOAD * ROW;
    if (j0 + kTile <= a.Lk) {
      // loads 4 h + x: offsets 4096 h in the bases, 1024 x in the instruction
      static_assert(LOADS % 4 == 0 && ROWS_PER_LOAD * ROW == 1024, "load runs of four");
      unsigned ko[4], vo[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        ko[x] = kgo0 ^ (unsigned)((D == 128 ? x : (x & 1)) << 6);
        vo[x] = vgo0 ^ (unsigned)(D == 128 ? x << 4 : (x & 1) << 5);
      }
#pragma unroll
      for (int h = 0; h < LOADS / 4; ++h) {
        dma16_run4(kt + h * 4096, ko, kd + h * 4096);
        dma16_run4(vt + h * 4096, vo, vd + h * 4096);
      }
    } else {
      const int rlast = a.Lk - 1 - j0;  // last valid row of this tile
      const int ln = lane_id_fresh();
      const int lr = ln / KCH, pc = ln % KCH;
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        const int r = (w * LOADS + i) * ROWS_PER_LOAD + lr;
        const unsigned ro = (unsigned)min(r, rlast) * ROW;
        dma16(kt, ro + ((unsigned)k_slot<D>(r, pc) << 4), kd + i * ROWS_PER_LOAD * ROW);
        dma16(vt, ro + ((unsigned)dual_slot<D>(r, pc) << 4), vd + i * ROWS_PER_LOAD * ROW);
      }
    }
  };

  // Q^T operands: lane holds row rq, head dims [16 ks + 8 g, +8) for every k-step
  bf16x8_t qf[KS];
  {
    const unsigned short* qp =
        static_cast<const unsigned short*>(a.q) + ((size_t)(b * a.Hq + head) * a.Lq) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4_t u = {0u, 0u, 0u, 0u};
      if (row_ok) u = *reinterpret_cast<const u32x4_t*>(qp + (size_t)rq * D + ks * 16 + g * 8);
      qf[ks] = as_bf16x8(u);
    }
  }

  f32x16_t oacc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[mb][i] = 0.f;

  const float c = a.scale * kLog2e;  // raw score -> log2 units
  float m2 = neg_inf();              // running max of row rq (log2 units): the skip test
  // Exponent reference of row rq (log2 units): l and O hold sums of
  // exp2(s c - mref).  It follows m2 only once m2 has risen more than
  // kRefMargin above it (p = exp2(s c - mref) < 2^kRefMargin, exact in fp32
  // and bf16 alike), so l and O are rescaled rarely, not whenever a row's max
  // grows a little.
  constexpr float kRefMargin = 8.f;
  float mref = neg_inf();
  float lpart = 0.f;                 // this lane's half of the row's denominator

  // Per-lane LDS offsets (the parts of the addresses that depend on the
  // swizzle), formed once from the lane index and held across the tile loop
  // (koff0, voff0 below; formed at each use they cost ~30 vector
  // instructions per tile, 4 % of the dense time).
  // K: row kb * 32 + l32, logical chunk 2 ks + g; the swizzle depends on the
  // row only through l32 (the row block is an immediate offset), and k-step
  // ks's offset is koff(0) ^ (ks << 5) (chunk 2 ks + g differs from chunk g in
  // bits 1-3 only).
  auto koff_now = [&]() __attribute__((always_inline)) {
    const int ln = lane_id_fresh();
    const int r = ln & 31;
    return (k_slot<D>(r, ln >> 5) << 4) + r * ROW;
  };
  // V^T: the transpose reads of dual_tr_off (keys {4g..4g+3} and
  // {8+4g..8+4g+3} of each 16-key step, one value column per lane); the V
  // image uses dual_slot, which keeps 32 lanes of a transpose read on
  // different banks (the swizzle it replaced did so for 16 lanes only).

  const int koff0 = koff_now();
  const int voff0 = dual_tr_off<D>(lane_id_fresh(), 0, 0);
  if (U > 0) issue_tile(stream_tile(0), 0);

  // one stream step, from ring stage u & 1; the row set works on it when it
  // holds one of its own visits (always, unless QP)
  for (int u = 0; u < U; ++u) {
    const int st = u & 1;
    const unsigned char* Ks = kst[st];
    const unsigned char* Vs = vst[st];
    const int t = u - u0;  // this row set's visit
    const bool active = !QP || (t >= 0 && t < count);
    const int j = active ? plan.tile_at(t) : 0;
    const int j0 = j * kTile;
    // this tile's loads have landed (own wave), and every wave is past tile t-1
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    // the stage of tile t-1 is free: start tile t+1
    if (u + 1 < U) issue_tile(stream_tile(u + 1), st ^ 1);

    f32x16_t sacc[4];
    float tmax2 = neg_inf();
    bool row_skip = false;
    if (active) {
    // ---- S^T = K Q^T: 4 blocks of 32 keys x 32 rows
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[kb][i] = 0.f;
      // K operands four k-steps at a time (register budget of two waves per SIMD)
#pragma unroll
      for (int k4 = 0; k4 < KS; k4 += 4) {
        u32x4_t kop[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          kop[ks] = *reinterpret_cast<const u32x4_t*>(Ks + kb * 32 * ROW + (koff0 ^ ((k4 + ks) << 5)));
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kop[ks]), qf[k4 + ks],
                                                            sacc[kb], 0, 0, 0);
      }
    }
    {
      // K operand reads issued RA MFMAs ahead of their use: each MFMA then
      // waits only for the read RA back, long since landed (four ahead,
      // the compiler's own order, left every MFMA waiting on LDS)
      constexpr int RA = 8;
      __builtin_amdgcn_sched_group_barrier(0x100, RA, 0);
#pragma unroll
      for (int i = 0; i < 4 * KS - RA; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, RA, 0);
    }

    // ---- mask: keys past Lk, and causal keys past row + shift
    const bool need_mask = (j0 + kTile > a.Lk) || (a.causal && j0 + kTile - 1 > row0 + shift);
    if (need_mask) {
      const int lim = a.causal ? min(a.Lk - 1, rq + shift) : a.Lk - 1;
      const int kg = j0 + (lane_id_fresh() >> 5) * 4;  // this lane half's first key
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kg + kb * 32 + (i >> 2) * 8 + (i & 3);
          if (key > lim) sacc[kb][i] = neg_inf();
        }
    }

    // ---- tile max of the row (raw units), both lane halves
    float tmax = neg_inf();
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, sacc[kb][i]);
    tmax = max_xor32(tmax);
    tmax2 = tmax * c;

    float delta = neg_inf();
    if (row_ok && tmax2 != neg_inf()) delta = (m2 == neg_inf()) ? pos_inf() : tmax2 - m2;
    row_skip = delta < a.log2_thr;  // this row's own test
    if (row_writer) rrow()[j] = row_skip ? 1 : 0;
    // The tile is skipped iff the max over the head's rows of delta is below
    // log2(threshold), i.e. iff no row passes its own test: one ballot per
    // wave, an OR over the head's waves (no max reduction across lanes).
    const bool wave_keeps = __builtin_amdgcn_ballot_w64(!row_skip) != 0;
    if (lane == 0) red[hh][wr] = wave_keeps ? 1 : 0;
    }
    __syncthreads();  // red[] visible
    if (active) {
    int keeps = red[hh][0];
#pragma unroll
    for (int i = 1; i < kRowWaves; ++i) keeps |= red[hh][i];
    const bool skip = keeps == 0;
    if (mask_writer && lane == 0) mrow[j] = skip ? 1 : 0;

    const float m2n = fmaxf(m2, tmax2);
    // Move the exponent reference (and rescale l and O by the factor, exactly
    // 1 for every other row) when some row's max has risen more than
    // kRefMargin above it.  A kept tile can raise m; a skipped one only when
    // threshold > 1 (with threshold <= 1 a skipped tile lies below every
    // row's m).  One place for both, so the accumulators keep one register
    // assignment through the loop.  A row that has seen no key yet keeps
    // mref = -inf (its l and O are 0; the first key moves it).
    const bool up = m2n > mref + kRefMargin;
    if (__builtin_amdgcn_ballot_w64(up) != 0) {
      const float alpha = up ? fast_exp2(mref - m2n) : 1.f;  // mref = -inf: 0
      lpart *= alpha;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) oacc[mb] *= alpha;
      if (up) mref = m2n;
    }
    if (!skip) {
      // per-row decisions: a row that failed its own test gets P = 0
      const float mexp = (a.per_row && row_skip) ? pos_inf() : (mref == neg_inf() ? 0.f : mref);
      // ---- per 32-key block: exponentials, then O^T += V^T P^T (two 16-key
      // steps, V^T operands from transpose reads).
      auto read_v = [&](int kb, int half, u32x4_t (&dst)[MB]) {
        const unsigned char* va = Vs + (kb * 32 + half * 16) * ROW;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_s16x4_t*)(va + (voff0 ^ dual_tr_xor<D>(mb, 0))));
          const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_s16x4_t*)(va + (voff0 ^ dual_tr_xor<D>(mb, 1))));
          const u32x2_t l2 = __builtin_bit_cast(u32x2_t, lo);
          const u32x2_t h2 = __builtin_bit_cast(u32x2_t, hi);
          dst[mb] = u32x4_t{l2[0], l2[1], h2[0], h2[1]};
        }
      };
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        bf16x8_t pb[2];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          unsigned int pw[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float p0 = fast_exp2(fmaf(sacc[kb][half * 8 + 2 * e], c, -mexp));
            const float p1 = fast_exp2(fmaf(sacc[kb][half * 8 + 2 * e + 1], c, -mexp));
            lpart += p0 + p1;
            pw[e] = pack_bf16x2(p0, p1);
          }
          u32x4_t pu = {pw[0], pw[1], pw[2], pw[3]};
          pb[half] = as_bf16x8(pu);
        }
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          u32x4_t vop[MB];
          read_v(kb, half, vop);
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
            oacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vop[mb]), pb[half],
                                                              oacc[mb], 0, 0, 0);
        }
      }
    }
    m2 = m2n;
    }
  }

  // ---- epilogue: O / l, lane holds columns 32 mb + 8 (i/4) + 4 g + i%4 of row rq
  const float l = sum_xor32(lpart);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  if (a.lse && row_ok && g == 0)
    a.lse[(size_t)(b * a.Hq + head) * a.Lq + rq] = l > 0.f ? (mref + __log2f(l)) * kLn2 : neg_inf();
  unsigned short* op = static_cast<unsigned short*>(a.out) + ((size_t)(b * a.Hq + head) * a.Lq) * D;
  if (row_ok) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int col = mb * 32 + i4 * 8 + g * 4;
        u32x2_t pk = {pack_bf16x2(oacc[mb][i4 * 4 + 0] * inv, oacc[mb][i4 * 4 + 1] * inv),
                      pack_bf16x2(oacc[mb][i4 * 4 + 2] * inv, oacc[mb][i4 * 4 + 3] * inv)};
        *reinterpret_cast<u32x2_t*>(op + (size_t)rq * D + col) = pk;
      }
  }
}

}  // namespace

bool prefill_bf16_supported(int D, int Dv) { return D == Dv && (D == 64 || D == 128); }

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t s) {
  const int nQ = (a.Lq + kTile - 1) / kTile;
  // two heads of a KV group per workgroup when the group size is even, else
  // two neighbouring query tiles of one head
  const bool pairs_of_heads = (a.Hq / a.Hkv) % 2 == 0;
  const dim3 block(64 * kRowWaves * 2);
  const dim3 grid(pairs_of_heads ? (unsigned)((size_t)nQ * (a.Hq / 2) * a.B)
                                 : (unsigned)((size_t)((nQ + 1) / 2) * a.Hq * a.B));
  if (a.D == 64) {
    if (pairs_of_heads)
      hipLaunchKernelGGL((prefill_bf16_kernel<64, 2, false>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((prefill_bf16_kernel<64, 2, true>), grid, block, 0, s, a);
  } else {
    if (pairs_of_heads)
      hipLaunchKernelGGL((prefill_bf16_kernel<128, 2, false>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((prefill_bf16_kernel<128, 2, true>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace ssattn
