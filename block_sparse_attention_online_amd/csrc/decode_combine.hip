// Log-sum-exp merge of split-KV decode partials.
//
// Each split s of a row produced O_s = (sum over its kept keys of
// exp(s_c - m_s) v_c) / l_s and lse_s = m_s + ln l_s (-inf when it kept no
// key).  The whole row is
//   lse = ln sum_s exp(lse_s),   O = sum_s exp(lse_s - lse) O_s,
// which is what a single streaming pass over all the splits' kept keys would
// return (the same rescaling identity that keeps the online-softmax pass exact,
// vLLM-Omni design page "Skip-Softmax", section "The online-softmax pass").
//
// One workgroup per (batch, query head).  The split weights are formed once
// (all lse values loaded at the same time, a workgroup max, the exponentials)
// and kept in LDS; then every thread sums its value columns over the splits
// with independent loads.  When each thread owns one value column and there
// are at most 32 splits, the column's partials are loaded into registers
// before the weights are formed, so the whole merge waits on memory about
// once instead of once per few splits.

#include "device_common.h"
#include "launch.h"

namespace ssattn {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxSplitsInLds = 4096;
constexpr int kRegSplits = 32;  // splits whose partials one thread holds in registers

__global__ __launch_bounds__(kThreads) void decode_combine_kernel(DecodeArgs a) {
  __shared__ float wsplit[kMaxSplitsInLds];
  __shared__ float red[kThreads / 64];
  const int bh = blockIdx.x;  // b * Hq + h
  const int S = a.num_splits;
  const size_t rows = (size_t)a.B * a.Hq;
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;

  // fast path: one column per thread, partials loaded ahead of the weights
  const bool in_regs = a.Dv <= kThreads && S <= kRegSplits;
  const size_t step = rows * a.Dv;
  float ov[kRegSplits];
  if (in_regs) {
    const float* po = a.part_o + (size_t)bh * a.Dv + (tid < a.Dv ? tid : 0);
#pragma unroll
    for (int s = 0; s < kRegSplits; ++s)  // past S: the last split again, not used
      ov[s] = po[(size_t)(s < S ? s : S - 1) * step];
  }

  float mx = neg_inf();
  for (int s = tid; s < S; s += kThreads) {
    const float v = a.part_lse[s * rows + bh];
    if (s < kMaxSplitsInLds) wsplit[s] = v;
    mx = fmaxf(mx, v);
  }
  mx = lanes_max_from<1>(mx);
  if (lane == 0) red[w] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float mref = mx == neg_inf() ? 0.f : mx;
  float wsum = 0.f;
  for (int s = tid; s < S; s += kThreads) {
    const float e = __expf((s < kMaxSplitsInLds ? wsplit[s] : a.part_lse[s * rows + bh]) - mref);
    if (s < kMaxSplitsInLds) wsplit[s] = e;
    wsum += e;
  }
  wsum = lanes_sum_from<1>(wsum);
  __syncthreads();  // everyone has read red[] (max) and written the weights
  if (lane == 0) red[w] = wsum;
  __syncthreads();
  wsum = red[0] + red[1] + red[2] + red[3];
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;

  unsigned short* op = static_cast<unsigned short*>(a.out) + (size_t)bh * a.Dv;
  if (in_regs) {
    if (tid < a.Dv) {
      float o0 = 0.f, o1 = 0.f;
#pragma unroll
      for (int s = 0; s < kRegSplits; s += 2) {
        if (s < S) o0 = fmaf(wsplit[s], ov[s], o0);
        if (s + 1 < S) o1 = fmaf(wsplit[s + 1], ov[s + 1], o1);
      }
      op[tid] = (unsigned short)(pack_bf16x2((o0 + o1) * inv, 0.f) & 0xffffu);
    }
    return;
  }
  for (int dv = tid; dv < a.Dv; dv += kThreads) {
    float o0 = 0.f, o1 = 0.f, o2 = 0.f, o3 = 0.f;
    const float* po = a.part_o + (size_t)bh * a.Dv + dv;
    const int Sl = S < kMaxSplitsInLds ? S : kMaxSplitsInLds;
    int s = 0;
    for (; s + 4 <= Sl; s += 4) {
      o0 = fmaf(wsplit[s], po[(size_t)s * step], o0);
      o1 = fmaf(wsplit[s + 1], po[(size_t)(s + 1) * step], o1);
      o2 = fmaf(wsplit[s + 2], po[(size_t)(s + 2) * step], o2);
      o3 = fmaf(wsplit[s + 3], po[(size_t)(s + 3) * step], o3);
    }
    for (; s < Sl; ++s) o0 = fmaf(wsplit[s], po[(size_t)s * step], o0);
    for (; s < S; ++s)  // splits beyond the LDS table: weights recomputed
      o0 = fmaf(__expf(a.part_lse[s * rows + bh] - mref), po[(size_t)s * step], o0);
    const float r = ((o0 + o1) + (o2 + o3)) * inv;
    op[dv] = (unsigned short)(pack_bf16x2(r, 0.f) & 0xffffu);
  }
}

}  // namespace

hipError_t launch_decode_combine(const DecodeArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(decode_combine_kernel, dim3((unsigned)((size_t)a.B * a.Hq)), dim3(kThreads),
                     0, s, a);
  return hipGetLastError();
}

}  // namespace ssattn
