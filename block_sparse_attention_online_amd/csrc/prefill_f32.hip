// fp32 debug path of skip-softmax prefill: the same streaming pass and skip
// rule as the bf16 MFMA kernel, computed in fp32 on the vector ALUs with no
// bf16 rounding anywhere, so its output can be held to a tight tolerance.
//
// Method: vLLM-Omni design page "Skip-Softmax", sections "The online-softmax
// pass" (per-row running max m, denominator l, numerator O, rescaled when m
// grows) and "The skip test" (skip a tile when exp(tile_max - running_max) <
// threshold; it adds nothing to l or O).  The decision is uniform over the
// 128 rows of a query tile, or (per-row mode) each row decides alone and a
// row that fails its own test adds nothing from a kept tile.
//
// One workgroup per (batch, query head, 128-row query tile); 256 threads:
// thread t owns query row t % 128 and half t / 128 of the value columns.  The
// key and value tiles are staged in LDS as fp32.  Scores are recomputed for
// the exponentials instead of being held, which keeps registers low; speed
// is not a goal of this path.

#include "device_common.h"
#include "launch.h"

namespace ssattn {
namespace {

template <int D>
__global__ __launch_bounds__(256) void prefill_f32_kernel(PrefillArgs a) {
  constexpr int DH = D / 2;  // value columns per thread
  __shared__ float Ks[kTile][D];
  __shared__ float Vs[kTile][D];
  __shared__ float red[4];

  const int nQ = (a.Lq + kTile - 1) / kTile;
  const int qtile = blockIdx.x % nQ;
  const int h = (blockIdx.x / nQ) % a.Hq;
  const int b = blockIdx.x / (nQ * a.Hq);
  const int hk = h / (a.Hq / a.Hkv);
  const int tid = threadIdx.x;
  const int rloc = tid & (kTile - 1);
  const int half = tid >> 7;
  const int row = qtile * kTile + rloc;
  const bool row_ok = row < a.Lq;
  const int shift = a.Lk - a.Lq;  // causal: key c visible to row r iff c <= r + shift

  const float* qp = static_cast<const float*>(a.q) + ((size_t)(b * a.Hq + h) * a.Lq) * D;
  const float* kp = static_cast<const float*>(a.k) + ((size_t)(b * a.Hkv + hk) * a.Lk) * D;
  const float* vp = static_cast<const float*>(a.v) + ((size_t)(b * a.Hkv + hk) * a.Lk) * D;
  float* op = static_cast<float*>(a.out) + ((size_t)(b * a.Hq + h) * a.Lq) * D;

  const VisitPlan plan = make_visit_plan(qtile, a.Lq, a.Lk, a.causal, a.order);
  const int nK = plan.nK;
  uint8_t* mrow = a.mask ? a.mask + ((size_t)(b * a.Hq + h) * nQ + qtile) * nK : nullptr;
  if (mrow) {
    for (int j = tid; j < nK; j += blockDim.x) {
      const bool visited = plan.causal ? (j <= plan.last) : true;
      if (!visited) mrow[j] = 2;
    }
  }

  // per-row decisions: this thread's row of the row mask (half 0 writes)
  uint8_t* const rrow = (a.row_mask && half == 0 && row_ok)
                            ? a.row_mask + ((size_t)(b * a.Hq + h) * a.Lq + row) * nK
                            : nullptr;
  if (rrow && plan.causal)
    for (int j = plan.last + 1; j < nK; ++j) rrow[j] = 2;

  float q[D];
#pragma unroll
  for (int d = 0; d < D; ++d) q[d] = row_ok ? qp[(size_t)row * D + d] : 0.f;
  float o[DH];
#pragma unroll
  for (int d = 0; d < DH; ++d) o[d] = 0.f;

  const float c = a.scale * kLog2e;  // raw dot product -> log2 units
  float m2 = neg_inf();
  float l = 0.f;

  for (int t = 0; t < plan.count; ++t) {
    const int j = plan.tile_at(t);
    const int j0 = j * kTile;
    const int nkeys = min(kTile, a.Lk - j0);
    __syncthreads();
    for (int e = tid; e < kTile * D; e += blockDim.x) {
      const int kr = e / D, d = e % D;
      Ks[kr][d] = kr < nkeys ? kp[(size_t)(j0 + kr) * D + d] : 0.f;
      Vs[kr][d] = kr < nkeys ? vp[(size_t)(j0 + kr) * D + d] : 0.f;
    }
    __syncthreads();

    // scores (log2 units) and the row's tile max
    const int lim = a.causal ? row + shift - j0 : nkeys - 1;  // last visible key in tile
    const int nvis = min(nkeys - 1, lim) + 1;                 // visible keys [0, nvis)
    float tmax = neg_inf();
    for (int kr = 0; kr < nvis; ++kr) {
      float s = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) s = fmaf(q[d], Ks[kr][d], s);
      tmax = fmaxf(tmax, s * c);
    }
    float delta = neg_inf();
    if (row_ok && nvis > 0) delta = (m2 == neg_inf()) ? pos_inf() : tmax - m2;
    const bool row_skip = delta < a.log2_thr;  // this row's own test
    if (rrow) rrow[j] = row_skip ? 1 : 0;
    delta = lanes_max_from<1>(delta);
    if ((tid & 63) == 0) red[tid >> 6] = delta;
    __syncthreads();
    const float dblk = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const bool skip = dblk < a.log2_thr;
    if (mrow && tid == 0) mrow[j] = skip ? 1 : 0;

    const float m2_new = fmaxf(m2, tmax);
    const float mref = m2_new == neg_inf() ? 0.f : m2_new;
    const float alpha = exp2f(m2 - mref);
    if (!skip) {
      l *= alpha;
#pragma unroll
      for (int d = 0; d < DH; ++d) o[d] *= alpha;
      // per-row decisions: a row that failed its own test adds nothing
      const int nacc = (a.per_row && row_skip) ? 0 : nvis;
      for (int kr = 0; kr < nacc; ++kr) {
        float s = 0.f;
#pragma unroll
        for (int d = 0; d < D; ++d) s = fmaf(q[d], Ks[kr][d], s);
        const float p = exp2f(s * c - mref);
        l += p;
#pragma unroll
        for (int d = 0; d < DH; ++d) o[d] = fmaf(p, Vs[kr][half * DH + d], o[d]);
      }
    } else if (a.thr_above_1 && m2_new > m2) {
      l *= alpha;
#pragma unroll
      for (int d = 0; d < DH; ++d) o[d] *= alpha;
    }
    m2 = m2_new;
  }

  if (row_ok && half == 0 && a.lse)
    a.lse[(size_t)(b * a.Hq + h) * a.Lq + row] = l > 0.f ? (m2 + __log2f(l)) * kLn2 : neg_inf();
  if (row_ok) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int d = 0; d < DH; ++d) op[(size_t)row * D + half * DH + d] = o[d] * inv;
  }
}

}  // namespace

bool prefill_f32_supported(int D, int Dv) { return D == Dv && (D == 64 || D == 128); }

hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t s) {
  const int nQ = (a.Lq + kTile - 1) / kTile;
  const dim3 grid((unsigned)((size_t)nQ * a.Hq * a.B));
  if (a.D == 64)
    hipLaunchKernelGGL(prefill_f32_kernel<64>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(prefill_f32_kernel<128>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace ssattn
