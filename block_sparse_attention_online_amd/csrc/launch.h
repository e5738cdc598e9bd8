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
  // Per-row decisions: rows that fail the test add nothing from a kept tile;
  // row_mask (may be null) is u8 [B, Hq, Lq, nK].
  int per_row;
  uint8_t* row_mask;
  float* lse;  // may be null: [B, Hq, Lq] ln of the row's kept exponential sum
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
  int num_splits;       // sub-splits per (batch, KV head), one workgroup each
  int tiles_per_split;  // tiles per sub-split (the last of a chain may be shorter)
  int chain_tiles;      // tiles per chain (a user split; the whole sequence if chained)
  int subs_per_chain;   // sub-splits per chain
  float scale;
  float log2_thr;
  int thr_above_1;
  // Every sub-split publishes its per-row maxima and folds in those of the
  // earlier sub-splits of its chain before deciding.
  unsigned lb_tag;                 // nonzero, unique per launch (wraps after 2^31)
  unsigned long long* lb_slot;     // [B][Hkv][S][G] (tag << 32) | float bits
  unsigned int* lb_timeouts;       // count of look-back waits that gave up
  // Paged caches: k, v point at [num_blocks, Hkv, 2^block_log2, D] caches (a
  // latent cache: k alone, v null), sequence b has seq_lens[b] keys (Lk is
  // their upper bound) whose
  // blocks are block_table[b][...] ([B][max_blocks]), and its threshold is
  // thresholds[b], or factor / seq_lens[b] when thresholds is null.  The mask
  // has mask_tiles entries per (batch, KV head).
  const int* block_table;
  const int* seq_lens;
  const float* thresholds;
  float factor;
  int block_log2;
  int max_blocks;
  int num_blocks;
  int mask_tiles;
  // Per-row decisions (contiguous GQA decode): rows that fail the test add
  // nothing from a kept tile; row_mask (may be null) is u8 [B, Hq, nK].
  int per_row;
  uint8_t* row_mask;
  // Latent decode with a threshold: stage 1 scores every tile, decides and
  // records each sub-split's kept tiles (kept_bits, bit t = its tile t,
  // [B * Hkv][S]); a planning launch shares each sequence's kept tiles out
  // evenly (share_tiles [B * Hkv][S][64] absolute tile indices, share_count
  // [B * Hkv][S], share_mref [B * Hq] the heads' max over the sequence, log2
  // units); stage 2 runs them.  Stage 0: one launch (threshold 0).
  int mla_stage;
  unsigned long long* kept_bits;
  int* share_tiles;
  int* share_count;
  float* share_mref;
};

// Arguments of the backward launches of a bf16 prefill.
struct PrefillBwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* out;   // forward output O [B, Hq, Lq, Dv]
  const void* dout;  // dL/dO           [B, Hq, Lq, Dv]
  const float* lse;  // forward log-sum-exp (natural log) [B, Hq, Lq]
  const uint8_t* mask;  // forward skip mask [B, Hq, nQ, nK], or null: every visible tile
  void* dq;
  void* dk;
  void* dv;
  float* rowstat;  // workspace [B, Hq, nQ, 2, 128]: lse * log2(e) (+inf: no kept key), dO . O
  int B, Hq, Hkv, Lq, Lk, D, Dv;
  float scale;
  int causal;
};

// Sets the thread-local message ss_last_error() returns; returns code.
int report_error(int code, const char* msg);
}  // namespace ssattn

#include "ss_attn.h"

namespace ssattn {
// Every host-side check of a decode call (the split stage's), workspace size
// included; touches no device and launches nothing.
int validate_decode(const ss_decode_params* p);

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t s);
hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t s);
bool prefill_bf16_supported(int D, int Dv);
bool prefill_f32_supported(int D, int Dv);

bool prefill_bwd_supported(int D, int Dv);
hipError_t launch_prefill_bwd_rowstat(const PrefillBwdArgs& a, hipStream_t s);
hipError_t launch_prefill_bwd_dkdv(const PrefillBwdArgs& a, hipStream_t s);
hipError_t launch_prefill_bwd_dq(const PrefillBwdArgs& a, hipStream_t s);

hipError_t launch_decode_gqa(const DecodeArgs& a, hipStream_t s);
hipError_t launch_decode_gqa_paged(const DecodeArgs& a, hipStream_t s);
bool decode_gqa_supported(int D, int Dv, int group, bool latent);
int decode_gqa_max_tiles(int group);  // tiles a split may hold in chained mode
hipError_t launch_decode_mla(const DecodeArgs& a, hipStream_t s);
hipError_t launch_decode_mla_paged(const DecodeArgs& a, hipStream_t s);
bool decode_mla_supported(int D, int Dv, int group, bool latent);
int decode_mla_max_tiles(int group);
int decode_mla_workgroups_per_split(int group);
hipError_t launch_decode_combine(const DecodeArgs& a, hipStream_t s);

}  // namespace ssattn
