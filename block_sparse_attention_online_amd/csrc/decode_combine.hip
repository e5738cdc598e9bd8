// Log-sum-exp merge of split-KV decode partials.
//
// Each split s of a row produced O_s = (sum over its kept keys of
// exp(s_c - m_s) v_c) / l_s and lse_s = m_s + ln l_s.  The whole row is
//   lse = ln sum_s exp(lse_s),   O = sum_s exp(lse_s - lse) O_s,
// which is what a single streaming pass over all the splits' kept keys would
// return (the same rescaling identity that keeps the online-softmax pass exact,
// vLLM-Omni design page "Skip-Softmax", section "The online-softmax pass").
//
// One workgroup per (batch, query head); thread t writes value column t.

#include "device_common.h"
#include "launch.h"

namespace ssattn {
namespace {

__global__ __launch_bounds__(512) void decode_combine_kernel(DecodeArgs a) {
  const int bh = blockIdx.x;  // b * Hq + h
  const int S = a.num_splits;
  const size_t rows = (size_t)a.B * a.Hq;
  float mx = neg_inf();
  for (int s = 0; s < S; ++s) mx = fmaxf(mx, a.part_lse[s * rows + bh]);
  const float mref = mx == neg_inf() ? 0.f : mx;
  float wsum = 0.f;
  for (int s = 0; s < S; ++s) wsum += __expf(a.part_lse[s * rows + bh] - mref);
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  unsigned short* op = static_cast<unsigned short*>(a.out) + (size_t)bh * a.Dv;
  for (int dv = threadIdx.x; dv < a.Dv; dv += blockDim.x) {
    float o = 0.f;
    for (int s = 0; s < S; ++s) {
      const float wt = __expf(a.part_lse[s * rows + bh] - mref);
      o = fmaf(wt, a.part_o[(s * rows + bh) * a.Dv + dv], o);
    }
    const float r = o * inv;
    op[dv] = (unsigned short)(pack_bf16x2(r, 0.f) & 0xffffu);
  }
}

}  // namespace

hipError_t launch_decode_combine(const DecodeArgs& a, hipStream_t s) {
  const int threads = a.Dv >= 512 ? 512 : (a.Dv >= 256 ? 256 : 128);
  hipLaunchKernelGGL(decode_combine_kernel, dim3((unsigned)((size_t)a.B * a.Hq)), dim3(threads), 0,
                     s, a);
  return hipGetLastError();
}

}  // namespace ssattn
