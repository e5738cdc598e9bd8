// Skip-aware backward of the skip-softmax prefill: per-row statistics and
// query gradients, bf16 inputs, fp32 accumulation, gfx950.
//
// Method: the derivative of the forward with its skip decisions held fixed
// (BLASST summary page, "Belangrijkste Bijdragen", trains with the sparsity
// on; design page "Skip-Softmax", "The online-softmax pass": the pass is
// exact softmax attention over the keys it keeps).  For the rows of query
// tile i and the key tiles the forward kept for (head, i):
//     P = exp(scale Q K^T - lse),  dP = dO V^T,  Delta_r = dO_r . O_r,
//     dS = P * (dP - Delta),  dQ = scale dS K.
// Skipped and unvisited key tiles add nothing; their products do not run.
//
// rowstat: one workgroup per (batch, head, query tile) writes the tile's
// 128 values of lse * log2(e) (+inf for a row that kept no key or lies past
// Lq, so its weights come out 0) and of Delta, 1 KiB, which one wave-wide
// direct-to-LDS load brings into the dK/dV kernel.
//
// dQ: one workgroup per (batch, 128-row query tile, NH query heads sharing a
// KV head -- NH = 2 when the group size is even, else 1), four waves of 32 rows
// per head, as the forward.  The heads walk the union of the key tiles either
// kept; K and V tiles stream through a two-stage ring of direct-to-LDS loads
// and serve both heads; a head whose own tile pair was skipped runs nothing
// on it.  Per kept tile (v_mfma_f32_32x32x16_bf16):
//  * S^T = K Q^T and dP^T = V dO^T, with Q^T and dO^T of the lane's row held
//    in registers (B operands) and K, V read as rows from LDS: the
//    accumulator gives each lane one query row and 16 keys per 32-key block;
//  * P and dS in that lane, then dQ^T += K^T dS^T: dS^T (bf16) is the B
//    operand as it stands, K^T comes from transpose reads of the K tile.
// S and dP of a kept pair are computed here and again in the dK/dV kernel:
// two more products per pair in exchange for writing every gradient once,
// without atomics.

#include "bwd_common.h"
#include "launch.h"

namespace ssattn {
namespace {

constexpr int kDqRowWaves = 4;  // waves per head: 4 x 32 rows

template <int DV>
__global__ __launch_bounds__(256) void bwd_rowstat_kernel(PrefillBwdArgs a) {
  constexpr int LPR = DV / 8;          // lanes per row (16 bytes of O and dO each)
  constexpr int RPP = 256 / LPR;       // rows per pass of the workgroup
  const int nQ = (a.Lq + kTile - 1) / kTile;
  const size_t tile = blockIdx.x;      // (b * Hq + h) * nQ + qt
  const int qt = (int)(tile % nQ);
  const size_t bh = tile / nQ;
  const int tid = threadIdx.x;
  const int sub = tid % LPR;
  float* rs = a.rowstat + tile * (2 * kTile);
#pragma unroll
  for (int pass = 0; pass < kTile / RPP; ++pass) {
    const int rl = pass * RPP + tid / LPR;
    const int r = qt * kTile + rl;
    float d = 0.f;
    if (r < a.Lq) {
      const size_t off = (bh * a.Lq + r) * DV + sub * 8;
      const u32x4_t o = *reinterpret_cast<const u32x4_t*>(
          static_cast<const unsigned short*>(a.out) + off);
      const u32x4_t go = *reinterpret_cast<const u32x4_t*>(
          static_cast<const unsigned short*>(a.dout) + off);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        d = fmaf(bf16_lo(o[e]), bf16_lo(go[e]), fmaf(bf16_hi(o[e]), bf16_hi(go[e]), d));
    }
    d = group_sum<LPR>(d);
    if (sub == 0) {
      float l2 = pos_inf();
      if (r < a.Lq) {
        const float l = a.lse[bh * a.Lq + r];
        l2 = l == neg_inf() ? pos_inf() : l * kLog2e;
      }
      rs[rl] = l2;
      rs[kTile + rl] = r < a.Lq ? d : 0.f;
    }
  }
}

template <int D, int NH>
__global__ __launch_bounds__(64 * kDqRowWaves * NH, 1) void bwd_dq_kernel(PrefillBwdArgs a) {
  constexpr int NW = kDqRowWaves * NH;
  constexpr int ROW = 2 * D;
  constexpr int TB = kTile * ROW;
  constexpr int KS = D / 16;  // k-steps of S^T and dP^T over the head dimension
  constexpr int MB = D / 32;  // 32-wide blocks of dQ^T rows

  __shared__ __attribute__((aligned(1024))) unsigned char kst0[TB];
  __shared__ __attribute__((aligned(1024))) unsigned char vst0[TB];
  __shared__ __attribute__((aligned(1024))) unsigned char kst1[TB];
  __shared__ __attribute__((aligned(1024))) unsigned char vst1[TB];
  __shared__ int tlist[kBwdListCap];
  __shared__ int wcnt[NW];

  const int G = a.Hq / a.Hkv;
  const int sets = G / NH;
  const int nQ = (a.Lq + kTile - 1) / kTile;
  const int nK = (a.Lk + kTile - 1) / kTile;
  // Logical order as the forward: (batch, KV head, query tile, head set),
  // heaviest query tiles first when causal.
  const int L = xcd_local_order(blockIdx.x, gridDim.x);
  const int hs = L % sets;
  const int qi = (L / sets) % nQ;
  const int hk = (L / (sets * nQ)) % a.Hkv;
  const int b = L / (sets * nQ * a.Hkv);
  const int qtile = a.causal ? nQ - 1 - qi : qi;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = w / kDqRowWaves;
  const int wr = w % kDqRowWaves;
  const int head0 = hk * G + hs * NH;
  const int head = head0 + hh;
  const int l32 = lane & 31;
  const int g = lane >> 5;
  const int row0 = qtile * kTile;
  const int rq = row0 + wr * 32 + l32;  // the query row this lane owns
  const bool row_ok = rq < a.Lq;
  const int shift = a.Lk - a.Lq;
  const VisitPlan plan = make_visit_plan(qtile, a.Lq, a.Lk, a.causal, 0);
  const int total = plan.count;  // candidate key tiles 0 .. count - 1

  // Q^T and dO^T operands of row rq: elements 16 ks + 8 g .. + 8
  bf16x8_t qf[KS], of[KS];
  {
    const size_t off = ((size_t)(b * a.Hq + head) * a.Lq + (row_ok ? rq : 0)) * D;
    const unsigned short* qp = static_cast<const unsigned short*>(a.q) + off;
    const unsigned short* op = static_cast<const unsigned short*>(a.dout) + off;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4_t uq = {0u, 0u, 0u, 0u}, uo = {0u, 0u, 0u, 0u};
      if (row_ok) {
        uq = *reinterpret_cast<const u32x4_t*>(qp + ks * 16 + g * 8);
        uo = *reinterpret_cast<const u32x4_t*>(op + ks * 16 + g * 8);
      }
      qf[ks] = as_bf16x8(uq);
      of[ks] = as_bf16x8(uo);
    }
  }
  float lse2, delta;
  {
    const float* rs = a.rowstat + ((size_t)(b * a.Hq + head) * nQ + qtile) * (2 * kTile);
    lse2 = rs[wr * 32 + l32];
    delta = rs[kTile + wr * 32 + l32];
  }

  f32x16_t dqa[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int i = 0; i < 16; ++i) dqa[mb][i] = 0.f;

  // LDS offsets of this lane's row and transpose reads (k-step 0, column
  // block 0); the others follow by XOR with constants
  const int roff0 = dual_row_off<D>(lane, 0);
  const int toff0 = dual_tr_off<D>(lane, 0, 0);

  const float c2 = a.scale * kLog2e;
  const unsigned char* kbase = static_cast<const unsigned char*>(a.k) +
                               (size_t)(b * a.Hkv + hk) * a.Lk * ROW;
  const unsigned char* vbase = static_cast<const unsigned char*>(a.v) +
                               (size_t)(b * a.Hkv + hk) * a.Lk * ROW;

  // With two waves per SIMD, the waves of the first head issue the loads (one
  // per SIMD), so each SIMD keeps one wave that issues none: the loads a wave
  // issues slow its own MFMA and vector work (as in the forward kernel).
  constexpr int LW = NW > kDqRowWaves ? kDqRowWaves : NW;  // loading waves
  const unsigned go0 = bw_issue_off0<D, LW>(w < LW ? w : 0);
  auto issue = [&](int e, unsigned char* kd, unsigned char* vd) {
    if (w >= LW) return;
    const int j = e >> 2;
    const int rlast = a.Lk - 1 - j * kTile;
    bw_issue_tile<D, LW>(kbase + (size_t)j * kTile * ROW, rlast, kd, w, go0);
    bw_issue_tile<D, LW>(vbase + (size_t)j * kTile * ROW, rlast, vd, w, go0);
  };

  // One key tile (list entry t: tile << 2 | bit hh set when head hh kept it).
  auto step = [&](int t, int n, const unsigned char* Ks, const unsigned char* Vs,
                  unsigned char* Kn, unsigned char* Vn) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (t + 1 < n) issue(__builtin_amdgcn_readfirstlane(tlist[t + 1]), Kn, Vn);
    const int e = __builtin_amdgcn_readfirstlane(tlist[t]);
    if (!((e >> hh) & 1)) return;  // this head skipped the tile (uniform over its waves)
    const int j0 = (e >> 2) * kTile;
    const bool need_mask = (j0 + kTile > a.Lk) || (a.causal && j0 + kTile - 1 > row0 + shift);
    const int lim = a.causal ? min(a.Lk - 1, rq + shift) : a.Lk - 1;
    // one 32-key block at a time (register budget of two waves per SIMD)
#pragma unroll 1
    for (int kb = 0; kb < 4; ++kb) {
      // ---- S^T and dP^T for keys 32 kb .. + 32 (accumulator: column = row rq,
      // keys 8 (i / 4) + 4 g + i % 4)
      f32x16_t st, dpt;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        st[i] = 0.f;
        dpt[i] = 0.f;
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const u32x4_t ka = *reinterpret_cast<const u32x4_t*>(Ks + kb * 32 * ROW + (roff0 ^ (ks << 5)));
        st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ka), qf[ks], st, 0, 0, 0);
      }
      // keep the V operand reads from being hoisted above the S^T products
      // (their registers would not fit beside the K operands)
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const u32x4_t va = *reinterpret_cast<const u32x4_t*>(Vs + kb * 32 * ROW + (roff0 ^ (ks << 5)));
        dpt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(va), of[ks], dpt, 0, 0, 0);
      }
      // Keys past the row's limit: their scores become -inf, so their
      // exponentials are exactly 0 (the scale is positive).  A uniform
      // branch: the tiles that need no mask run no per-element test (the
      // empty asm keeps the compiler from turning the branch into selects
      // that every tile would run).
      if (need_mask) {
        asm volatile("");
        const int kg = j0 + kb * 32 + 4 * g;
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (kg + (i >> 2) * 8 + (i & 3) > lim) st[i] = neg_inf();
      }
      float sv[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) sv[i] = fast_exp2(fmaf(st[i], c2, -lse2)) * (dpt[i] - delta);
      bf16x8_t sb[2];
      bw_pack_b(sv, sb);
      // ---- dQ^T += K^T dS^T over the block's two 16-key steps
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const unsigned char* kt = Ks + (kb * 32 + 16 * h) * ROW;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          dqa[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              bw_tr_read(kt, toff0 ^ dual_tr_xor<D>(mb, 0), toff0 ^ dual_tr_xor<D>(mb, 1)), sb[h], dqa[mb], 0, 0, 0);
      }
    }
  };

  int next = 0;
  for (;;) {
    // ---- refill the list: key tiles kept by either head, 64 NW candidates per round
    int n = 0;
    while (next < total && n + 64 * NW <= kBwdListCap) {
      const int j = next + tid;
      int bits = 0;
      if (j < total) {
#pragma unroll
        for (int x = 0; x < NH; ++x) {
          const bool kept =
              !a.mask ||
              a.mask[(((size_t)b * a.Hq + head0 + x) * nQ + qtile) * nK + j] == kMaskKept;
          bits |= kept ? 1 << x : 0;
        }
      }
      const unsigned long long bal = __builtin_amdgcn_ballot_w64(bits != 0);
      if (lane == 0) wcnt[w] = __builtin_popcountll(bal);
      __syncthreads();
      int before = n, sum = n;
#pragma unroll
      for (int x = 0; x < NW; ++x) {
        const int cx = wcnt[x];
        before += x < w ? cx : 0;
        sum += cx;
      }
      if (bits) {
        const int rank = __builtin_amdgcn_mbcnt_hi((unsigned)(bal >> 32),
                                                   __builtin_amdgcn_mbcnt_lo((unsigned)bal, 0));
        tlist[before + rank] = (j << 2) | bits;
      }
      n = __builtin_amdgcn_readfirstlane(sum);
      next += 64 * NW;
      __syncthreads();
    }
    if (n == 0) break;
    issue(__builtin_amdgcn_readfirstlane(tlist[0]), kst0, vst0);
    for (int t = 0; t < n; t += 2) {
      step(t, n, kst0, vst0, kst1, vst1);
      if (t + 1 < n) step(t + 1, n, kst1, vst1, kst0, vst0);
    }
    __syncthreads();
  }

  // ---- epilogue: lane holds columns 32 mb + 8 (i / 4) + 4 g + i % 4 of row rq
  if (row_ok) {
    unsigned short* dqp = static_cast<unsigned short*>(a.dq) + ((size_t)(b * a.Hq + head) * a.Lq + rq) * D;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int col = mb * 32 + q4 * 8 + g * 4;
        const u32x2_t pk = {
            pack_bf16x2(dqa[mb][4 * q4] * a.scale, dqa[mb][4 * q4 + 1] * a.scale),
            pack_bf16x2(dqa[mb][4 * q4 + 2] * a.scale, dqa[mb][4 * q4 + 3] * a.scale)};
        *reinterpret_cast<u32x2_t*>(dqp + col) = pk;
      }
  }
}

}  // namespace

hipError_t launch_prefill_bwd_rowstat(const PrefillBwdArgs& a, hipStream_t s) {
  const int nQ = (a.Lq + kTile - 1) / kTile;
  const dim3 grid((unsigned)((size_t)nQ * a.Hq * a.B));
  if (a.Dv == 64)
    hipLaunchKernelGGL((bwd_rowstat_kernel<64>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((bwd_rowstat_kernel<128>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_prefill_bwd_dq(const PrefillBwdArgs& a, hipStream_t s) {
  const int nQ = (a.Lq + kTile - 1) / kTile;
  const int nh = ((a.Hq / a.Hkv) % 2 == 0) ? 2 : 1;
  const dim3 grid((unsigned)((size_t)nQ * (a.Hq / nh) * a.B));
  const dim3 block(64 * kDqRowWaves * nh);
  if (a.D == 64) {
    if (nh == 2)
      hipLaunchKernelGGL((bwd_dq_kernel<64, 2>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((bwd_dq_kernel<64, 1>), grid, block, 0, s, a);
  } else {
    if (nh == 2)
      hipLaunchKernelGGL((bwd_dq_kernel<128, 2>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((bwd_dq_kernel<128, 1>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace ssattn
