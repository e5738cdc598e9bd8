// Internal interface between the C-ABI host code (api.cpp) and the kernel
// translation units.  Not installed; callers use include/ss_attn.h.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

namespace ssattn {

// Arguments of one prefill launch, already validated by the host code.
struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  uint8_t* mask;  // may be null
  int B, Hq, Hkv, Lq, Lk, D, Dv;
  float scale;      // softmax scale (> 0)
  float log2_thr;   // log2(threshold); -inf for threshold 0
  int thr_above_1;  // threshold > 1: a skipped tile may raise m
  int causal;
  int order;  // ss_order
};

// Arguments of one split-KV decode launch.
struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;  // null: value row = first Dv columns of the key row
  void* out;
  uint8_t* mask;  // may be null
  float* part_o;    // [S, B, Hq, Dv] split outputs O_s / l_s
  float* part_lse;  // [S, B, Hq]     split log-sum-exp (natural log)
  int B, Hq, Hkv, Lk, D, Dv;
  int num_splits;       // effective number of non-empty splits
  int tiles_per_split;  // ceil(nK / requested splits)
  float scale;
  float log2_thr;
  int thr_above_1;
};

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t s);
hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t s);
bool prefill_bf16_supported(int D, int Dv);
bool prefill_f32_supported(int D, int Dv);

hipError_t launch_decode_gqa(const DecodeArgs& a, hipStream_t s);
bool decode_gqa_supported(int D, int Dv, int group, bool latent);
hipError_t launch_decode_mla(const DecodeArgs& a, hipStream_t s);
bool decode_mla_supported(int D, int Dv, int group, bool latent);
hipError_t launch_decode_combine(const DecodeArgs& a, hipStream_t s);

}  // namespace ssattn
