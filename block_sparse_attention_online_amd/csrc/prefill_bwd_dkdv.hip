// Skip-aware backward of the skip-softmax prefill: key and value gradients,
// bf16 inputs, fp32 accumulation, gfx950.
//
// Method.  The pages train models with the sparsity switched on (BLASST
// summary page, "Belangrijkste Bijdragen": sparsity-aware training) and print
// no backward pass.  This is the derivative of the forward with its skip
// decisions held fixed (a threshold test: constant between its switching
// points).  With them fixed, row r of query tile i attends by plain softmax to
// the visible keys of the key tiles the forward kept for (head, i) (design
// page "Skip-Softmax", "The online-softmax pass": the streaming pass is exact
// over the keys it keeps), so with lse the forward's log-sum-exp:
//     P = exp(scale Q K^T - lse),  dP = dO V^T,  Delta_r = dO_r . O_r,
//     dS = P * (dP - Delta),  dV = P^T dO,  dK = scale dS^T Q.
// A (query tile, key tile) pair that the forward skipped contributes nothing,
// so none of its four products runs here.
//
// Design: one workgroup per (batch, KV head, 128-key tile), four waves of 32
// keys, one wave per SIMD (the dK^T and dV^T accumulators of 32 keys take 128
// registers per lane, beside 64 of K and V operands).
//  * K and V of the wave's 32 keys are loaded once, into registers, as the
//    B operands of S = Q K^T and dP = dO V^T (v_mfma_f32_32x32x16_bf16).
//  * The workgroup compacts, from the skip mask, the list of (query head of
//    the KV group, query tile) pairs that kept its key tile, and walks it:
//    Q_i, dO_i and the rows' (lse, Delta) stream through a two-stage ring of
//    direct-to-LDS loads; dK^T and dV^T accumulate in registers across all
//    pairs (no atomics; each gradient row is written once, at the end).
//  * S and dP are computed untransposed (query rows x keys): the accumulator
//    gives each lane one key and 16 rows, so P and dS, rounded to bf16, are
//    directly the B operands of dV^T += dO^T P and dK^T += Q^T dS (k = query
//    rows); their A operands come from transpose reads of the dO and Q tiles.

#include "bwd_common.h"
#include "launch.h"

namespace ssattn {
namespace {

constexpr int kDkdvWaves = 4;

// S = Q K^T and dP = dO V^T in the MFMA's VGPR form.  The kernel needs more
// than 256 registers per lane, so its builtin MFMAs accumulate in the
// accumulation registers (AGPRs); S and dP are read by the vector ALU, and
// from AGPRs every element would first take a v_accvgpr_read (128 per tile
// pair).  These two chains are therefore written out (taking K and V as AGPR
// operands instead spilled: both register files then filled up).  Gradients
// are bitwise those of the builtin form; dense 4 % faster.  The hardware
// forwards an accumulator from one MFMA to the next that names it (no wait); the first
// MFMA of a chain starts from 0, two wait states after any vector write of
// its operands; mfma_v_drain gives the 24 wait states an MFMA result needs
// before a vector ALU instruction reads it, and ties the chain so that
// nothing reads it earlier.
__device__ __forceinline__ void mfma_v_first(f32x16_t& acc, u32x4_t a, bf16x8_t b) {
  asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_v(f32x16_t& acc, u32x4_t a, bf16x8_t b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_v_drain(f32x16_t& x) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(x));
}

template <int D>
__global__ __launch_bounds__(64 * kDkdvWaves, 1) void bwd_dkdv_kernel(PrefillBwdArgs a) {
  constexpr int NW = kDkdvWaves;
  constexpr int ROW = 2 * D;            // bytes per row (D == Dv)
  constexpr int TB = kTile * ROW;       // bytes per tile
  constexpr int KS = D / 16;            // k-steps of S and dP over the head dimension
  constexpr int MB = D / 32;            // 32-wide blocks of dK^T / dV^T rows

  // Two-stage ring; the step loop is unrolled by two so every access names its
  // stage at compile time.
  __shared__ __attribute__((aligned(1024))) unsigned char qs0[TB];
  __shared__ __attribute__((aligned(1024))) unsigned char ds0[TB];
  __shared__ __attribute__((aligned(1024))) unsigned char qs1[TB];
  __shared__ __attribute__((aligned(1024))) unsigned char ds1[TB];
  __shared__ __attribute__((aligned(16))) float rs0[2 * kTile];
  __shared__ __attribute__((aligned(16))) float rs1[2 * kTile];
  __shared__ int plist[kBwdListCap];
  __shared__ int wcnt[NW];

  const int G = a.Hq / a.Hkv;
  const int nQ = (a.Lq + kTile - 1) / kTile;
  const int nK = (a.Lk + kTile - 1) / kTile;
  // Logical order (batch, KV head, key tile): neighbouring key tiles walk the
  // same query tiles in the same order and, through xcd_local_order, share an
  // XCD's L2.  Causal: key tile 0 has the most query tiles, so it goes first.
  const int L = xcd_local_order(blockIdx.x, gridDim.x);
  const int j = L % nK;
  const int hk = (L / nK) % a.Hkv;
  const int b = L / (nK * a.Hkv);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int g = lane >> 5;
  const int j0 = j * kTile;
  const int key = j0 + w * 32 + l32;  // the key this lane owns
  const bool key_ok = key < a.Lk;
  const int shift = a.Lk - a.Lq;

  // Query tiles that see key tile j: i >= i_min (the last query row sees
  // every key, so i = nQ - 1 always does).
  int i_min = 0;
  if (a.causal) {
    const long num = (long)j0 - shift - (kTile - 1);
    i_min = num <= 0 ? 0 : min(nQ - 1, (int)((num + kTile - 1) / kTile));
  }
  const int nI = nQ - i_min;
  const int total = G * nI;  // candidate pairs p = head_in_group * nI + (i - i_min)

  // K and V of this lane's key: B operands, elements 16 ks + 8 g .. + 8.
  bf16x8_t kf[KS], vf[KS];
  {
    const size_t kr = ((size_t)(b * a.Hkv + hk) * a.Lk + (key_ok ? key : 0)) * D;
    const unsigned short* kp = static_cast<const unsigned short*>(a.k) + kr;
    const unsigned short* vp = static_cast<const unsigned short*>(a.v) + kr;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4_t uk = {0u, 0u, 0u, 0u}, uv = {0u, 0u, 0u, 0u};
      if (key_ok) {
        uk = *reinterpret_cast<const u32x4_t*>(kp + ks * 16 + g * 8);
        uv = *reinterpret_cast<const u32x4_t*>(vp + ks * 16 + g * 8);
      }
      kf[ks] = as_bf16x8(uk);
      vf[ks] = as_bf16x8(uv);
    }
  }

  f32x16_t dka[MB], dva[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      dka[mb][i] = 0.f;
      dva[mb][i] = 0.f;
    }

  // LDS offsets of this lane's row and transpose reads, one register each
  // (forming them from the first by XOR would cost a VALU instruction per read)
  int roff[KS], toff[MB][2];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) roff[ks] = dual_row_off<D>(lane, ks);
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) toff[mb][hi] = dual_tr_off<D>(lane, mb, hi);

  const float c2 = a.scale * kLog2e;

  // Loads of pair p into one ring stage: Q_i and dO_i by all waves, the rows'
  // statistics (1 KiB) by wave 0.
  const unsigned go0 = bw_issue_off0<D, NW>(w);
  auto issue = [&](int p, unsigned char* qd, unsigned char* dd, float* rd) {
    const int hl = p / nI;
    const int i = i_min + (p - hl * nI);
    const size_t bh = (size_t)b * a.Hq + hk * G + hl;
    const size_t r0 = bh * a.Lq + (size_t)i * kTile;
    const int rlast = a.Lq - 1 - i * kTile;
    bw_issue_tile<D, NW>(static_cast<const unsigned char*>(a.q) + r0 * ROW, rlast, qd, w, go0);
    bw_issue_tile<D, NW>(static_cast<const unsigned char*>(a.dout) + r0 * ROW, rlast, dd, w, go0);
    if (w == 0)
      dma16(a.rowstat + (bh * nQ + i) * (2 * kTile), 16u * (unsigned)lane_id_fresh(),
            reinterpret_cast<const unsigned char*>(rd));
  };

  // Rows of a tile that do not see this lane's key: r < rmin (causal: the key
  // is visible to row r iff key <= r + shift), every row when the key lies
  // past Lk.  The +-2^30 sentinels leave room to subtract a row index
  // (< 2^24) without overflow.
  const int rmin = !key_ok ? (1 << 30) : (a.causal ? key - shift : -(1 << 30));

  // The products of one pair from its ring stage, as a software pipeline over
  // the tile's four 32-row blocks.  With one wave per SIMD nothing else hides
  // latency, so every block runs four stages of eight MFMAs, each interleaved
  // with the work the next stage needs:
  //   S  = Q K^T    | LDS reads: dO rows, the rows' lse2
  //   dP = dO V^T   | VALU: P = exp2(S c2 - lse2) -> bf16; LDS: dO^T, Delta
  //   dV^T += dO^T P| VALU: dS = P (dP - Delta) -> bf16; LDS: Q^T
  //   dK^T += Q^T dS| LDS: Q rows of the next block
  // Scheduling barriers keep the compiler from hoisting a stage's reads
  // further (their registers would not fit).  `tlim`: the row offset within
  // the tile, minus 4 g, below which this lane's P is 0; `masked`: some row
  // of the tile does not see some key of the wave's block.
  auto pair_body = [&](bool masked, int tlim, const unsigned char* Qs, const unsigned char* Ds,
                       const float* Rs) {
    u32x4_t qa[KS], da[KS];
    bf16x8_t tv[2][MB], tq[2][MB];
    f32x4_t l4[4], d4[4];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qa[ks] = *reinterpret_cast<const u32x4_t*>(Qs + roff[ks]);
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      // ---- stage 1: S for rows 32 rb .. + 32 (accumulator: column = key,
      // rows 8 (e / 4) + 4 g + e % 4)
      f32x16_t sacc;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (ks == 0)
          mfma_v_first(sacc, qa[0], kf[0]);
        else
          mfma_v(sacc, qa[ks], kf[ks]);
        da[ks] = *reinterpret_cast<const u32x4_t*>(Ds + rb * 32 * ROW + roff[ks]);
        if (ks < 4) l4[ks] = *reinterpret_cast<const f32x4_t*>(Rs + rb * 32 + 8 * ks + 4 * g);
        __builtin_amdgcn_sched_barrier(0);
      }
      mfma_v_drain(sacc);

      // Rows that do not see this lane's key: their scores become -inf, so
      // P is exactly 0 there (the scale is positive).  A uniform branch, so
      // the pairs that need no mask run no per-element test (the empty asm
      // keeps the compiler from turning it into selects every pair runs).
      if (masked) {
        asm volatile("");
#pragma unroll
        for (int ii = 0; ii < 16; ++ii)
          if (rb * 32 + 8 * (ii >> 2) + (ii & 3) < tlim) sacc[ii] = neg_inf();
      }

      // ---- stage 2: dP; P from S
      // one dP MFMA, 16 / KS of P's elements and the next reads per step
      // (KS k-steps: 2 h x MB transpose reads and the 4 Delta reads fit them)
      static_assert(16 % KS == 0 && 2 * MB == KS && KS >= 4, "stage 2 layout");
      f32x16_t dacc;
      float pv[16];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (ks == 0)
          mfma_v_first(dacc, da[0], vf[0]);
        else
          mfma_v(dacc, da[ks], vf[ks]);
#pragma unroll
        for (int ii = (16 / KS) * ks; ii < (16 / KS) * (ks + 1); ++ii)
          pv[ii] = fast_exp2(fmaf(sacc[ii], c2, -l4[ii >> 2][ii & 3]));
        tv[ks / MB][ks % MB] =
            bw_tr_read(Ds + (rb * 32 + 16 * (ks / MB)) * ROW, toff[ks % MB][0], toff[ks % MB][1]);
        if (ks < 4) d4[ks] = *reinterpret_cast<const f32x4_t*>(Rs + kTile + rb * 32 + 8 * ks + 4 * g);
        __builtin_amdgcn_sched_barrier(0);
      }
      bf16x8_t pb[2];
      bw_pack_b(pv, pb);
      mfma_v_drain(dacc);

      // ---- stage 3: dV^T += dO^T P; dS from dP
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          dva[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tv[h][mb], pb[h], dva[mb], 0, 0, 0);
      float sv[16];
#pragma unroll
      for (int ii = 0; ii < 16; ++ii) sv[ii] = pv[ii] * (dacc[ii] - d4[ii >> 2][ii & 3]);
      bf16x8_t sb[2];
      bw_pack_b(sv, sb);
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          tq[h][mb] = bw_tr_read(Qs + (rb * 32 + 16 * h) * ROW, toff[mb][0], toff[mb][1]);
#pragma unroll
      for (int x = 0; x < 2 * MB; ++x) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);  // VALU
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // DS read
      }
      __builtin_amdgcn_sched_barrier(0);

      // ---- stage 4: dK^T += Q^T dS; Q rows of the next block
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          dka[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tq[h][mb], sb[h], dka[mb], 0, 0, 0);
      if (rb < 3) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          qa[ks] = *reinterpret_cast<const u32x4_t*>(Qs + (rb + 1) * 32 * ROW + roff[ks]);
      }
#pragma unroll
      for (int x = 0; x < 2 * MB; ++x) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // One pair; Qs/Ds/Rs: its stage, Qn/Dn/Rn: the other stage.
  auto step = [&](int t, int n, const unsigned char* Qs, const unsigned char* Ds, const float* Rs,
                  unsigned char* Qn, unsigned char* Dn, float* Rn) {
    // this pair's loads have landed (own wave), and every wave is past pair t-1
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (t + 1 < n) issue(__builtin_amdgcn_readfirstlane(plist[t + 1]), Qn, Dn, Rn);
    const int p = __builtin_amdgcn_readfirstlane(plist[t]);
    const int r0 = (i_min + p % nI) * kTile;
    // every key of this wave's block visible to every row of the tile?
    const bool full = (j0 + w * 32 + 32 <= a.Lk) && (!a.causal || j0 + w * 32 + 31 <= r0 + shift);
    pair_body(!full, rmin - r0 - 4 * g, Qs, Ds, Rs);
  };

  int next = 0;  // first candidate pair not yet scanned
  for (;;) {
    // ---- refill the list: compact kept pairs, 256 candidates per round
    int n = 0;
    while (next < total && n + 64 * NW <= kBwdListCap) {
      const int p = next + tid;
      bool kept = false;
      if (p < total) {
        kept = true;
        if (a.mask) {
          const int hl = p / nI;
          const int i = i_min + (p - hl * nI);
          kept = a.mask[(((size_t)b * a.Hq + hk * G + hl) * nQ + i) * nK + j] == kMaskKept;
        }
      }
      const unsigned long long bal = __builtin_amdgcn_ballot_w64(kept);
      if (lane == 0) wcnt[w] = __builtin_popcountll(bal);
      __syncthreads();
      int before = n, sum = n;
#pragma unroll
      for (int x = 0; x < NW; ++x) {
        const int cx = wcnt[x];
        before += x < w ? cx : 0;
        sum += cx;
      }
      if (kept) {
        const int rank = __builtin_amdgcn_mbcnt_hi((unsigned)(bal >> 32),
                                                   __builtin_amdgcn_mbcnt_lo((unsigned)bal, 0));
        plist[before + rank] = p;
      }
      n = __builtin_amdgcn_readfirstlane(sum);
      next += 64 * NW;
      __syncthreads();  // list entries visible; wcnt free again
    }
    if (n == 0) break;
    issue(__builtin_amdgcn_readfirstlane(plist[0]), qs0, ds0, rs0);
    for (int t = 0; t < n; t += 2) {
      step(t, n, qs0, ds0, rs0, qs1, ds1, rs1);
      if (t + 1 < n) step(t + 1, n, qs1, ds1, rs1, qs0, ds0, rs0);
    }
    __syncthreads();  // every wave is done with the ring and the list
  }

  // ---- epilogue: lane holds rows 32 mb + 8 q4 + 4 g + e of dK^T / dV^T for its key
  if (key_ok) {
    const size_t kr = ((size_t)(b * a.Hkv + hk) * a.Lk + key) * D;
    unsigned short* dkp = static_cast<unsigned short*>(a.dk) + kr;
    unsigned short* dvp = static_cast<unsigned short*>(a.dv) + kr;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int col = mb * 32 + q4 * 8 + g * 4;
        const u32x2_t k2 = {pack_bf16x2(dka[mb][4 * q4] * a.scale, dka[mb][4 * q4 + 1] * a.scale),
                            pack_bf16x2(dka[mb][4 * q4 + 2] * a.scale,
                                        dka[mb][4 * q4 + 3] * a.scale)};
        const u32x2_t v2 = {pack_bf16x2(dva[mb][4 * q4], dva[mb][4 * q4 + 1]),
                            pack_bf16x2(dva[mb][4 * q4 + 2], dva[mb][4 * q4 + 3])};
        *reinterpret_cast<u32x2_t*>(dkp + col) = k2;
        *reinterpret_cast<u32x2_t*>(dvp + col) = v2;
      }
  }
}

}  // namespace

bool prefill_bwd_supported(int D, int Dv) { return D == Dv && (D == 64 || D == 128); }

hipError_t launch_prefill_bwd_dkdv(const PrefillBwdArgs& a, hipStream_t s) {
  const int nK = (a.Lk + kTile - 1) / kTile;
  const dim3 grid((unsigned)((size_t)nK * a.Hkv * a.B));
  if (a.D == 64)
    hipLaunchKernelGGL((bwd_dkdv_kernel<64>), grid, dim3(64 * kDkdvWaves), 0, s, a);
  else
    hipLaunchKernelGGL((bwd_dkdv_kernel<128>), grid, dim3(64 * kDkdvWaves), 0, s, a);
  return hipGetLastError();
}

}  // namespace ssattn
