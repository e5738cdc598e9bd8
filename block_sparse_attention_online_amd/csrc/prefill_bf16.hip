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
// Design (one workgroup = one 128-row query tile of one head, 4 waves of 32
// rows; two workgroups share a compute unit):
//  * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//    K is the A operand read from LDS, Q^T the B operand held in registers for
//    the whole pass.  The accumulator layout then gives every lane one query
//    row and 16 keys per 32-key block, so the row max, the running state and
//    the exponentials stay in the lane that owns the row.
//  * The output is accumulated transposed too, O^T += V^T P^T: the lane's
//    exponentials P are already laid out as the B operand (its row, 8 keys);
//    V^T is the A operand, staged in LDS transposed with the 4-key groups of
//    every 16 keys ordered so that each lane's 8 keys are one 16-byte read.
//  * LDS tiles use an XOR swizzle of 16-byte chunks so the MFMA operand reads
//    (8 lanes on 8 different rows, same column) hit distinct banks.
//  * The skip decision: per row delta = tile_max - m (log2 units), the max over
//    the wave's 32 rows by shuffles, the max over the 4 waves through LDS;
//    skip when it is below log2(threshold).  The branch is uniform over the
//    workgroup, so a skipped tile issues no exp and no P.V MFMA at all.
//  * K for the next tile is prefetched into registers during the current one.

#include "device_common.h"
#include "launch.h"

namespace ssattn {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

// Byte offset of 16-byte chunk `c` of row `r` in a swizzled LDS tile whose
// rows are `row_bytes` long.
__device__ __forceinline__ int swz(int r, int c, int row_bytes) {
  return r * row_bytes + ((c ^ (r & 7)) << 4);
}
// V^T rows are the value columns; both the transposing writes (8 rows 8
// apart) and the operand reads (8 consecutive rows) must spread over chunks.
__device__ __forceinline__ int vt_swz(int dv, int c) {
  return dv * (kTile * 2) + ((c ^ ((dv ^ (dv >> 3)) & 7)) << 4);
}
// Slot of 4-key group `a` (0..3) inside its 16-key group in the V^T layout:
// groups 1 and 2 trade places, so MFMA lane half g reads keys
// {4g..4g+3, 8+4g..8+4g+3} of the group as one contiguous 16-byte chunk.
__device__ __forceinline__ int quad_slot(int a) { return (a == 1) ? 2 : (a == 2 ? 1 : a); }

template <int D>
__global__ __launch_bounds__(kThreads, 1) void prefill_bf16_kernel(PrefillArgs a) {
  constexpr int KCH = D / 8;        // 16-byte chunks per K row
  constexpr int KS = D / 16;        // MFMA k-steps over the head dimension
  constexpr int MB = D / 32;        // 32-wide value-column blocks
  constexpr int KROW = D * 2;       // bytes per K row in LDS
  constexpr int K_LOADS = (kTile * KCH) / kThreads;       // 16-byte K loads per thread
  constexpr int V_UNITS = (kTile / 4) * KCH / kThreads;   // (4 keys x 8 cols) units per thread
  static_assert(K_LOADS >= 1 && V_UNITS >= 1, "tile split");

  __shared__ __attribute__((aligned(16))) unsigned char Ks[kTile * KROW];
  __shared__ __attribute__((aligned(16))) unsigned char Vt[D * kTile * 2];
  __shared__ float red[kWaves];

  const int nQ = (a.Lq + kTile - 1) / kTile;
  // heaviest (most tiles) query tiles first when causal
  const int qi = blockIdx.x % nQ;
  const int qtile = a.causal ? nQ - 1 - qi : qi;
  const int h = (blockIdx.x / nQ) % a.Hq;
  const int b = blockIdx.x / (nQ * a.Hq);
  const int hk = h / (a.Hq / a.Hkv);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int l32 = lane & 31;
  const int g = lane >> 5;  // MFMA k-group of this lane
  const int row0 = qtile * kTile;
  const int rq = row0 + w * 32 + l32;  // the query row this lane owns
  const bool row_ok = rq < a.Lq;
  const int shift = a.Lk - a.Lq;

  const unsigned short* qp =
      static_cast<const unsigned short*>(a.q) + ((size_t)(b * a.Hq + h) * a.Lq) * D;
  const unsigned short* kp =
      static_cast<const unsigned short*>(a.k) + ((size_t)(b * a.Hkv + hk) * a.Lk) * D;
  const unsigned short* vp =
      static_cast<const unsigned short*>(a.v) + ((size_t)(b * a.Hkv + hk) * a.Lk) * D;
  unsigned short* op = static_cast<unsigned short*>(a.out) + ((size_t)(b * a.Hq + h) * a.Lq) * D;

  const VisitPlan plan = make_visit_plan(qtile, a.Lq, a.Lk, a.causal, a.order);
  const int nK = plan.nK;
  uint8_t* mrow = a.mask ? a.mask + ((size_t)(b * a.Hq + h) * nQ + qtile) * nK : nullptr;
  if (mrow && plan.causal) {
    for (int j = plan.last + 1 + tid; j < nK; j += kThreads) mrow[j] = 2;
  }

  // Q^T operand: lane holds row rq, head dims [16 ks + 8 g, +8) for every k-step
  bf16x8_t qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    u32x4_t u = {0u, 0u, 0u, 0u};
    if (row_ok) u = *reinterpret_cast<const u32x4_t*>(qp + (size_t)rq * D + ks * 16 + g * 8);
    qf[ks] = as_bf16x8(u);
  }

  f32x16_t oacc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[mb][i] = 0.f;

  const float c = a.scale * kLog2e;  // raw score -> log2 units
  float m2 = neg_inf();             // running max of this lane's row (log2 units)
  float lpart = 0.f;                // this lane's half of the row's denominator

  // K prefetch registers: thread loads chunk (row, col) = divmod(tid + 256 i, KCH)
  u32x4_t kreg[K_LOADS];
  auto load_k = [&](int j) {
    const int j0 = j * kTile;
#pragma unroll
    for (int i = 0; i < K_LOADS; ++i) {
      const int u = tid + kThreads * i;
      const int r = u / KCH, cc = u % KCH;
      u32x4_t val = {0u, 0u, 0u, 0u};
      if (j0 + r < a.Lk) val = *reinterpret_cast<const u32x4_t*>(kp + (size_t)(j0 + r) * D + cc * 8);
      kreg[i] = val;
    }
  };

  if (plan.count > 0) load_k(plan.tile_at(0));

  for (int t = 0; t < plan.count; ++t) {
    const int j = plan.tile_at(t);
    const int j0 = j * kTile;
    __syncthreads();  // previous tile's LDS reads are done
#pragma unroll
    for (int i = 0; i < K_LOADS; ++i) {
      const int u = tid + kThreads * i;
      const int r = u / KCH, cc = u % KCH;
      *reinterpret_cast<u32x4_t*>(Ks + swz(r, cc, KROW)) = kreg[i];
    }
    // V of this tile, 4 keys x 8 value columns per unit
    u32x4_t vreg[V_UNITS][4];
#pragma unroll
    for (int i = 0; i < V_UNITS; ++i) {
      const int u = tid + kThreads * i;
      const int oc = u % KCH, quad = u / KCH;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int key = j0 + quad * 4 + kk;
        u32x4_t val = {0u, 0u, 0u, 0u};
        if (key < a.Lk) val = *reinterpret_cast<const u32x4_t*>(vp + (size_t)key * D + oc * 8);
        vreg[i][kk] = val;
      }
    }
    __syncthreads();  // K tile visible

    // ---- S^T = K Q^T: 4 blocks of 32 keys x 32 rows
    f32x16_t sacc[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[kb][i] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int kr = kb * 32 + l32;
        const u32x4_t kv = *reinterpret_cast<const u32x4_t*>(Ks + swz(kr, ks * 2 + g, KROW));
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kv), qf[ks], sacc[kb], 0, 0, 0);
      }
    }

    // ---- mask: keys past Lk, and causal keys past row + shift
    const bool need_mask = (j0 + kTile > a.Lk) || (a.causal && j0 + kTile - 1 > row0 + shift);
    if (need_mask) {
      const int lim = a.causal ? min(a.Lk - 1, rq + shift) : a.Lk - 1;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = j0 + kb * 32 + (i >> 2) * 8 + g * 4 + (i & 3);
          if (key > lim) sacc[kb][i] = neg_inf();
        }
    }

    // ---- tile max of the row (raw units), both lane halves
    float tmax = neg_inf();
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, sacc[kb][i]);
    tmax = fmaxf(tmax, shfl_xor_f(tmax, 32));
    const float tmax2 = tmax * c;

    float delta = neg_inf();
    if (row_ok && tmax2 != neg_inf()) delta = (m2 == neg_inf()) ? pos_inf() : tmax2 - m2;
    delta = lanes_max_from<1>(delta);
    if (lane == 0) red[w] = delta;

    // V^T tile: for each of the 8 columns of a unit, the unit's 4 keys as 8 bytes
#pragma unroll
    for (int i = 0; i < V_UNITS; ++i) {
      const int u = tid + kThreads * i;
      const int oc = u % KCH, quad = u / KCH;
      const int grp = quad >> 2;                    // 16-key group
      const int slot = grp * 4 + quad_slot(quad & 3);  // 4-key slot in the row
      const int chunk = slot >> 1, within = (slot & 1) * 8;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int word = e >> 1;
        const bool hi = e & 1;
        unsigned int x[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) x[kk] = hi ? (vreg[i][kk][word] >> 16) : (vreg[i][kk][word] & 0xffffu);
        u32x2_t pk = {x[0] | (x[1] << 16), x[2] | (x[3] << 16)};
        const int dv = oc * 8 + e;
        *reinterpret_cast<u32x2_t*>(Vt + vt_swz(dv, chunk) + within) = pk;
      }
    }
    // next K tile in flight during the decision, the exponentials and P.V
    if (t + 1 < plan.count) load_k(plan.tile_at(t + 1));
    __syncthreads();  // red[] and V^T visible

    const float dblk = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const bool skip = dblk < a.log2_thr;
    if (mrow && tid == 0) mrow[j] = skip ? 1 : 0;

    const float m2_new = fmaxf(m2, tmax2);
    if (!skip) {
      const float mref = (m2_new == neg_inf()) ? 0.f : m2_new;
      const float alpha = fast_exp2(m2 - mref);
      float lsum = 0.f;
      bf16x8_t pb[4][2];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          unsigned int pw[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float p0 = fast_exp2(fmaf(sacc[kb][hh * 8 + 2 * e], c, -mref));
            const float p1 = fast_exp2(fmaf(sacc[kb][hh * 8 + 2 * e + 1], c, -mref));
            lsum += p0 + p1;
            pw[e] = pack_bf16x2(p0, p1);
          }
          u32x4_t pu = {pw[0], pw[1], pw[2], pw[3]};
          pb[kb][hh] = as_bf16x8(pu);
        }
      }
      lpart = fmaf(alpha, lpart, lsum);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[mb][i] *= alpha;
      // ---- O^T += V^T P^T
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
            const int dv = mb * 32 + l32;
            const u32x4_t vv = *reinterpret_cast<const u32x4_t*>(Vt + vt_swz(dv, kb * 4 + hh * 2 + g));
            oacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vv), pb[kb][hh], oacc[mb], 0, 0, 0);
          }
    } else if (a.thr_above_1 && m2_new > m2) {
      const float alpha = fast_exp2(m2 - m2_new);
      lpart *= alpha;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[mb][i] *= alpha;
    }
    m2 = m2_new;
  }

  // ---- epilogue: O / l, lane holds columns 32 mb + 8 (i/4) + 4 g + i%4 of row rq
  const float l = lpart + shfl_xor_f(lpart, 32);
  const float inv = l > 0.f ? 1.f / l : 0.f;
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
  const dim3 grid((unsigned)((size_t)nQ * a.Hq * a.B));
  if (a.D == 64)
    hipLaunchKernelGGL(prefill_bf16_kernel<64>, grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(prefill_bf16_kernel<128>, grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace ssattn
