// C ABI of the skip-softmax attention library: argument checks, the operating
// point (factor, threshold, timestep gate), the decode split policy and the
// kernel launches.  Every public function is declared in include/ss_attn.h.

#include "ss_attn.h"

#include <atomic>
#include <chrono>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <limits>

#include "launch.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return SS_OK;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(SS_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Threshold as the kernels consume it: log2(thr), -inf at thr = 0.
float log2_threshold(float thr) {
  return thr > 0.f ? std::log2(thr) : -std::numeric_limits<float>::infinity();
}

int check_threshold(float thr) {
  if (!(thr >= 0.f) || !std::isfinite(thr))
    return fail(SS_ERR_INVALID_ARG, "threshold must be finite and >= 0 (got %g)", (double)thr);
  return SS_OK;
}

int check_scale(float scale) {
  if (!(scale > 0.f) || !std::isfinite(scale))
    return fail(SS_ERR_INVALID_ARG, "scale must be finite and > 0 (got %g)", (double)scale);
  return SS_OK;
}

// Largest sequence length accepted; keeps every index product in 64 bits and
// every per-row tile index in 32 bits.
constexpr int kMaxLen = 1 << 24;

struct SplitPlan {
  int requested;  // after clamping to [1, nK]
  int per;        // tiles per split
  int count;      // non-empty splits
};

SplitPlan plan_splits(int nK, int num_splits) {
  SplitPlan p;
  p.requested = num_splits < 1 ? 1 : (num_splits > nK ? nK : num_splits);
  p.per = (int)ceil_div(nK, p.requested);
  p.count = (int)ceil_div(nK, p.per);
  return p;
}

bool is_latent_decode(int D, int Dv, const void* v) { return v == nullptr && Dv <= D; }

// Which kernel serves a decode shape, and how many tiles one split of it may
// hold when splits are chained (its score buffer in LDS).
enum class DecodeKernel { kNone, kGqa, kMla };

DecodeKernel decode_kernel(int D, int Dv, int group, bool latent) {
  if (ssattn::decode_gqa_supported(D, Dv, group, latent)) return DecodeKernel::kGqa;
  if (ssattn::decode_mla_supported(D, Dv, group, latent)) return DecodeKernel::kMla;
  return DecodeKernel::kNone;
}

int chained_max_tiles(int D, int Dv, int group, bool latent) {
  switch (decode_kernel(D, Dv, group, latent)) {
    case DecodeKernel::kGqa: return ssattn::decode_gqa_max_tiles(group);
    case DecodeKernel::kMla: return ssattn::decode_mla_max_tiles(group);
    default: return 1 << 30;
  }
}

// Automatic split count: enough workgroups to keep all 256 compute units
// streaming, with no split longer than a chained split may be.  GQA: about 11
// workgroups per compute unit (3 resident at a time); on the 32K Llama-shape
// decode this measured 6 % faster at 70 % skip than 8 per unit, and anything
// from 9 to 14 per unit within 1 %.  Latent: one resident workgroup per
// compute unit, one workgroup per sub-split, one round (at 131072 keys, 8
// sequences: 32 sub-splits of 32 tiles measured 296 us plus a 15 us merge,
// against 318 + 26 us for two rounds; more splits cost more in the merge).
// Chained decisions do not depend on the count.
int auto_splits(int B, int Hq, int Hkv, int Lk, int D, int Dv, bool latent) {
  const int64_t nK = ceil_div(Lk, SS_TILE_KEYS);
  const int64_t units = (int64_t)B * Hkv;
  const int group = Hq / Hkv;
  const int64_t want = decode_kernel(D, Dv, group, latent) == DecodeKernel::kMla
                           ? 256 / ssattn::decode_mla_workgroups_per_split(group)
                           : 11 * 256;
  int64_t per = ceil_div(nK * units, want);
  const int64_t cap = chained_max_tiles(D, Dv, Hq / Hkv, latent);
  if (per > cap) per = cap;
  if (per < 1) per = 1;
  return (int)ceil_div(nK, per);
}

struct DecodePlan {
  int subs;            // sub-splits (workgroups) per (batch, KV head)
  int tiles_per_sub;   // tiles per sub-split
  int chain_tiles;     // tiles per chain
  int subs_per_chain;  // sub-splits per chain
  size_t o_off, lse_off, slot_off, timeout_off, bytes;
  // latent decode with a threshold: kept tiles per sub-split, their share-out
  size_t kept_off, share_tiles_off, share_count_off, share_mref_off;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Cut a chain of `tiles` tiles into sub-splits of at most `cap` tiles.
void cut_chain(int tiles, int cap, int* per, int* count) {
  const int n = (int)ceil_div(tiles, cap);
  *per = (int)ceil_div(tiles, n);
  *count = (int)ceil_div(tiles, *per);
}

// Split partition and workspace layout.  Chained: one chain over the whole
// sequence, cut into `num_splits` sub-splits (raised where a sub-split would
// exceed the kernel's capacity).  Independent: `num_splits` chains (user
// splits of ceil(nK/S) tiles), each cut into sub-splits within capacity.
DecodePlan plan_decode(int B, int Hq, int Hkv, int Lk, int D, int Dv, bool latent,
                       int num_splits, bool chained) {
  const int nK = (int)ceil_div(Lk, SS_TILE_KEYS);
  const int req = num_splits == 0 ? auto_splits(B, Hq, Hkv, Lk, D, Dv, latent) : num_splits;
  const int cap = chained_max_tiles(D, Dv, Hq / Hkv, latent);
  DecodePlan p;
  int subs_chained = 0;
  {
    const SplitPlan sp = plan_splits(nK, req);
    int per = sp.per, cnt = sp.count;
    if (per > cap) cut_chain(nK, cap, &per, &cnt);
    subs_chained = cnt;
    if (chained) {
      p.subs = cnt;
      p.tiles_per_sub = per;
      p.chain_tiles = nK;
      p.subs_per_chain = cnt;
    }
  }
  int subs_indep = 0;
  {
    const SplitPlan sp = plan_splits(nK, req);
    int per = 0, cnt = 0;
    cut_chain(sp.per, cap, &per, &cnt);
    subs_indep = sp.count * cnt;
    if (!chained) {
      p.subs = subs_indep;
      p.tiles_per_sub = per;
      p.chain_tiles = sp.per;
      p.subs_per_chain = cnt;
    }
  }
  const int subs_max = subs_chained > subs_indep ? subs_chained : subs_indep;
  const size_t rows = (size_t)subs_max * B * Hq;
  const size_t slots = (size_t)subs_max * B * Hkv;
  p.o_off = 0;
  p.lse_off = align256(rows * (size_t)Dv * sizeof(float));
  p.slot_off = p.lse_off + align256(rows * sizeof(float));
  const size_t after_slots =
      p.slot_off + align256(slots * (size_t)(Hq / Hkv) * sizeof(unsigned long long));
  p.kept_off = after_slots;
  p.share_tiles_off = p.kept_off + align256(slots * sizeof(unsigned long long));
  p.share_count_off = p.share_tiles_off + align256(slots * 64 * sizeof(int));
  p.share_mref_off = p.share_count_off + align256(slots * sizeof(int));
  // the timeout counter block stays the last 256 bytes
  p.timeout_off =
      latent ? p.share_mref_off + align256((size_t)B * Hq * sizeof(float)) : after_slots;
  p.bytes = p.timeout_off + 256;
  return p;
}

// Launch tags: nonzero and different for consecutive decode launches of this
// process, so values published by an earlier launch (or stale workspace
// bytes) are not read as current.  They start from a process-specific value.
std::atomic<unsigned> g_tag{0};

unsigned next_tag() {
  unsigned t = g_tag.fetch_add(2u) + 2u;
  if (t == 2u) {  // first use
    const unsigned seed = (unsigned)(std::chrono::steady_clock::now().time_since_epoch().count() *
                                     0x9E3779B97F4A7C15ull >> 32);
    g_tag.store(seed | 1u);
    t = g_tag.fetch_add(2u) + 2u;
  }
  return t | 1u;
}

int check_granularity(int granularity, const uint8_t* row_mask_out) {
  if (granularity != SS_SKIP_TILE && granularity != SS_SKIP_ROW)
    return fail(SS_ERR_INVALID_ARG, "unknown granularity %d", granularity);
  if (row_mask_out && granularity != SS_SKIP_ROW)
    return fail(SS_ERR_INVALID_ARG, "row_mask_out needs granularity SS_SKIP_ROW");
  return SS_OK;
}

int validate_prefill(const ss_prefill_params* p) {
  if (!p) return fail(SS_ERR_INVALID_ARG, "params is null");
  if (!p->q || !p->k || !p->v || !p->out)
    return fail(SS_ERR_INVALID_ARG, "q, k, v and out must be non-null");
  if (p->B <= 0 || p->Hq <= 0 || p->Hkv <= 0 || p->Lq <= 0 || p->Lk <= 0 || p->D <= 0 ||
      p->Dv <= 0)
    return fail(SS_ERR_INVALID_ARG, "sizes must be positive");
  if (p->Lq > kMaxLen || p->Lk > kMaxLen)
    return fail(SS_ERR_INVALID_ARG, "sequence lengths above %d are not supported", kMaxLen);
  if (p->Hq % p->Hkv) return fail(SS_ERR_INVALID_ARG, "Hq (%d) must be a multiple of Hkv (%d)",
                                  p->Hq, p->Hkv);
  if (int rc = check_scale(p->scale)) return rc;
  if (int rc = check_threshold(p->threshold)) return rc;
  if (p->order != SS_ORDER_ASCENDING && p->order != SS_ORDER_DIAG_FIRST)
    return fail(SS_ERR_INVALID_ARG, "unknown order %d", p->order);
  if (p->dtype == SS_DTYPE_BF16) {
    if (!ssattn::prefill_bf16_supported(p->D, p->Dv))
      return fail(SS_ERR_UNSUPPORTED, "bf16 prefill supports D == Dv in {64, 128} (got %d, %d)",
                  p->D, p->Dv);
  } else if (p->dtype == SS_DTYPE_F32) {
    if (!ssattn::prefill_f32_supported(p->D, p->Dv))
      return fail(SS_ERR_UNSUPPORTED, "fp32 prefill supports D == Dv in {64, 128} (got %d, %d)",
                  p->D, p->Dv);
  } else {
    return fail(SS_ERR_INVALID_ARG, "unknown dtype %d", p->dtype);
  }
  if (int rc = check_granularity(p->granularity, p->row_mask_out)) return rc;
  return SS_OK;
}

}  // namespace

namespace ssattn {
int report_error(int code, const char* msg) { return fail(code, "%s", msg); }
}  // namespace ssattn

extern "C" {

const char* ss_last_error(void) { return g_err; }

const char* ss_version(void) { return "ssattn 0.1.0 (gfx950)"; }

int ss_attn_prefill_ex(const ss_prefill_params* p, hipStream_t stream) {
  if (int rc = validate_prefill(p)) return rc;
  ssattn::PrefillArgs a{};
  a.q = p->q;
  a.k = p->k;
  a.v = p->v;
  a.out = p->out;
  a.mask = p->skip_mask_out;
  a.B = p->B;
  a.Hq = p->Hq;
  a.Hkv = p->Hkv;
  a.Lq = p->Lq;
  a.Lk = p->Lk;
  a.D = p->D;
  a.Dv = p->Dv;
  a.scale = p->scale;
  a.log2_thr = log2_threshold(p->threshold);
  a.thr_above_1 = p->threshold > 1.f;
  a.causal = p->causal != 0;
  a.order = p->order;
  a.per_row = p->granularity == SS_SKIP_ROW;
  a.row_mask = p->row_mask_out;
  a.lse = p->lse_out;
  hipError_t e = p->dtype == SS_DTYPE_BF16 ? ssattn::launch_prefill_bf16(a, stream)
                                           : ssattn::launch_prefill_f32(a, stream);
  if (e != hipSuccess) return hip_fail(e, "prefill launch");
  return ok();
}

int ss_attn_prefill(const void* q, const void* k, const void* v, void* out, int B, int Hq,
                    int Hkv, int Lq, int Lk, int D, int Dv, float scale, int causal,
                    float threshold, uint8_t* skip_mask_out, hipStream_t stream) {
  ss_prefill_params p{q, k, v, out, B, Hq, Hkv, Lq, Lk, D, Dv, scale, threshold,
                      causal, SS_DTYPE_BF16, SS_ORDER_ASCENDING, skip_mask_out};
  return ss_attn_prefill_ex(&p, stream);
}

int ss_attn_prefill_f32(const float* q, const float* k, const float* v, float* out, int B,
                        int Hq, int Hkv, int Lq, int Lk, int D, int Dv, float scale, int causal,
                        float threshold, uint8_t* skip_mask_out, hipStream_t stream) {
  ss_prefill_params p{q, k, v, out, B, Hq, Hkv, Lq, Lk, D, Dv, scale, threshold,
                      causal, SS_DTYPE_F32, SS_ORDER_ASCENDING, skip_mask_out};
  return ss_attn_prefill_ex(&p, stream);
}

int ss_decode_num_splits(int B, int Hq, int Hkv, int Lk, int D, int Dv) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Lk <= 0 || D <= 0 || Dv <= 0 || Hq % Hkv ||
      Lk > kMaxLen)
    return 0;
  const bool latent = decode_kernel(D, Dv, Hq / Hkv, false) == DecodeKernel::kNone && Dv <= D;
  return auto_splits(B, Hq, Hkv, Lk, D, Dv, latent);
}

size_t ss_attn_prefill_backward_workspace_bytes(int B, int Hq, int Lq) {
  if (B <= 0 || Hq <= 0 || Lq <= 0 || Lq > kMaxLen) return 0;
  const size_t nQ = ((size_t)Lq + SS_TILE_ROWS - 1) / SS_TILE_ROWS;
  return align256((size_t)B * Hq * nQ * 2 * SS_TILE_ROWS * sizeof(float));
}

int ss_attn_prefill_backward(const ss_prefill_bwd_params* p, hipStream_t stream) {
  if (!p) return fail(SS_ERR_INVALID_ARG, "params is null");
  if (!p->q || !p->k || !p->v || !p->out || !p->dout || !p->lse || !p->dq || !p->dk || !p->dv)
    return fail(SS_ERR_INVALID_ARG, "q, k, v, out, dout, lse, dq, dk and dv must be non-null");
  if (p->B <= 0 || p->Hq <= 0 || p->Hkv <= 0 || p->Lq <= 0 || p->Lk <= 0 || p->D <= 0 ||
      p->Dv <= 0)
    return fail(SS_ERR_INVALID_ARG, "sizes must be positive");
  if (p->Lq > kMaxLen || p->Lk > kMaxLen)
    return fail(SS_ERR_INVALID_ARG, "sequence lengths above %d are not supported", kMaxLen);
  if (p->Hq % p->Hkv) return fail(SS_ERR_INVALID_ARG, "Hq (%d) must be a multiple of Hkv (%d)",
                                  p->Hq, p->Hkv);
  if (int rc = check_scale(p->scale)) return rc;
  if (p->dtype != SS_DTYPE_BF16)
    return fail(p->dtype == SS_DTYPE_F32 ? SS_ERR_UNSUPPORTED : SS_ERR_INVALID_ARG,
                "the prefill backward supports dtype bf16 only (got %d)", p->dtype);
  if (!ssattn::prefill_bwd_supported(p->D, p->Dv))
    return fail(SS_ERR_UNSUPPORTED, "the prefill backward supports D == Dv in {64, 128} (got %d, %d)",
                p->D, p->Dv);
  const size_t need = ss_attn_prefill_backward_workspace_bytes(p->B, p->Hq, p->Lq);
  if (!p->workspace || p->workspace_bytes < need)
    return fail(SS_ERR_WORKSPACE, "prefill backward workspace needs %zu bytes (got %zu%s)", need,
                p->workspace_bytes, p->workspace ? "" : ", null");
  ssattn::PrefillBwdArgs a{};
  a.q = p->q;
  a.k = p->k;
  a.v = p->v;
  a.out = p->out;
  a.dout = p->dout;
  a.lse = p->lse;
  a.mask = p->skip_mask;
  a.dq = p->dq;
  a.dk = p->dk;
  a.dv = p->dv;
  a.rowstat = static_cast<float*>(p->workspace);
  a.B = p->B;
  a.Hq = p->Hq;
  a.Hkv = p->Hkv;
  a.Lq = p->Lq;
  a.Lk = p->Lk;
  a.D = p->D;
  a.Dv = p->Dv;
  a.scale = p->scale;
  a.causal = p->causal != 0;
  hipError_t e = ssattn::launch_prefill_bwd_rowstat(a, stream);
  if (e != hipSuccess) return hip_fail(e, "prefill backward row statistics launch");
  e = ssattn::launch_prefill_bwd_dkdv(a, stream);
  if (e != hipSuccess) return hip_fail(e, "prefill backward dK/dV launch");
  e = ssattn::launch_prefill_bwd_dq(a, stream);
  if (e != hipSuccess) return hip_fail(e, "prefill backward dQ launch");
  return ok();
}

size_t ss_attn_decode_workspace_bytes(int B, int Hq, int Hkv, int Lk, int D, int Dv,
                                      int num_splits) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Lk <= 0 || D <= 0 || Dv <= 0 || Hq % Hkv ||
      num_splits < 0 || Lk > kMaxLen)
    return 0;
  const bool latent = decode_kernel(D, Dv, Hq / Hkv, false) == DecodeKernel::kNone && Dv <= D;
  return plan_decode(B, Hq, Hkv, Lk, D, Dv, latent, num_splits, true).bytes;
}

}  // extern "C"

namespace {

// Validate a decode call and fill the launch arguments.  `stage_partial`
// checks the inputs of the split kernel; the combine stage needs only sizes,
// the workspace and out.
int prepare_decode(const ss_decode_params* p, bool stage_partial, ssattn::DecodeArgs* a,
                   DecodeKernel* kernel) {
  if (!p) return fail(SS_ERR_INVALID_ARG, "params is null");
  if (stage_partial && (!p->q || !p->k)) return fail(SS_ERR_INVALID_ARG, "q and k must be non-null");
  if (p->B <= 0 || p->Hq <= 0 || p->Hkv <= 0 || p->Lk <= 0 || p->D <= 0 || p->Dv <= 0)
    return fail(SS_ERR_INVALID_ARG, "sizes must be positive");
  if (p->Lk > kMaxLen) return fail(SS_ERR_INVALID_ARG, "Lk above %d is not supported", kMaxLen);
  if (p->Hq % p->Hkv)
    return fail(SS_ERR_INVALID_ARG, "Hq (%d) must be a multiple of Hkv (%d)", p->Hq, p->Hkv);
  if (p->num_splits < 0) return fail(SS_ERR_INVALID_ARG, "num_splits must be >= 0");
  if (p->split_mode != SS_SPLIT_CHAINED && p->split_mode != SS_SPLIT_INDEPENDENT)
    return fail(SS_ERR_INVALID_ARG, "unknown split_mode %d", p->split_mode);
  const bool latent = is_latent_decode(p->D, p->Dv, p->v);
  if (stage_partial) {
    if (!p->v && p->Dv > p->D) return fail(SS_ERR_INVALID_ARG, "v == NULL needs Dv <= D");
    if (int rc = check_scale(p->scale)) return rc;
    if (int rc = check_threshold(p->threshold)) return rc;
  }
  const int group = p->Hq / p->Hkv;
  // the combine stage sees no v pointer: any kernel that serves the shape will do
  DecodeKernel k = decode_kernel(p->D, p->Dv, group, stage_partial ? latent : false);
  if (k == DecodeKernel::kNone && !stage_partial) k = decode_kernel(p->D, p->Dv, group, true);
  if (k == DecodeKernel::kNone)
    return fail(SS_ERR_UNSUPPORTED, "no decode kernel for D=%d Dv=%d group=%d %s", p->D, p->Dv,
                group, latent ? "(latent V)" : "(separate V)");
  *kernel = k;
  if (int rc = check_granularity(p->granularity, p->row_mask_out)) return rc;
  if (stage_partial && p->granularity == SS_SKIP_ROW && k != DecodeKernel::kGqa)
    return fail(SS_ERR_UNSUPPORTED, "per-row skip decisions need the separate-V decode");
  const bool chained = p->split_mode == SS_SPLIT_CHAINED;
  const DecodePlan pl = plan_decode(p->B, p->Hq, p->Hkv, p->Lk, p->D, p->Dv,
                                    k == DecodeKernel::kMla, p->num_splits, chained);
  if (!p->workspace || p->workspace_bytes < pl.bytes)
    return fail(SS_ERR_WORKSPACE, "decode workspace needs %zu bytes (got %zu%s)", pl.bytes,
                p->workspace_bytes, p->workspace ? "" : ", null");
  char* ws = static_cast<char*>(p->workspace);
  a->q = p->q;
  a->k = p->k;
  a->v = p->v;
  a->out = p->out;
  a->mask = p->skip_mask_out;
  a->part_o = reinterpret_cast<float*>(ws + pl.o_off);
  a->part_lse = reinterpret_cast<float*>(ws + pl.lse_off);
  a->lb_slot = reinterpret_cast<unsigned long long*>(ws + pl.slot_off);
  a->lb_timeouts = reinterpret_cast<unsigned int*>(ws + pl.timeout_off);
  if (k == DecodeKernel::kMla) {
    a->kept_bits = reinterpret_cast<unsigned long long*>(ws + pl.kept_off);
    a->share_tiles = reinterpret_cast<int*>(ws + pl.share_tiles_off);
    a->share_count = reinterpret_cast<int*>(ws + pl.share_count_off);
    a->share_mref = reinterpret_cast<float*>(ws + pl.share_mref_off);
  }
  a->B = p->B;
  a->Hq = p->Hq;
  a->Hkv = p->Hkv;
  a->Lk = p->Lk;
  a->D = p->D;
  a->Dv = p->Dv;
  a->num_splits = pl.subs;
  a->tiles_per_split = pl.tiles_per_sub;
  a->chain_tiles = pl.chain_tiles;
  a->subs_per_chain = pl.subs_per_chain;
  a->scale = p->scale;
  a->log2_thr = log2_threshold(p->threshold);
  a->thr_above_1 = p->threshold > 1.f;
  a->lb_tag = 0;
  a->per_row = p->granularity == SS_SKIP_ROW;
  a->row_mask = p->row_mask_out;
  return SS_OK;
}

}  // namespace

namespace ssattn {
int validate_decode(const ss_decode_params* p) {
  DecodeArgs a{};
  DecodeKernel k;
  return prepare_decode(p, true, &a, &k);
}
}  // namespace ssattn

extern "C" {

int ss_attn_decode_partial(const ss_decode_params* p, hipStream_t stream) {
  ssattn::DecodeArgs a{};
  DecodeKernel k;
  if (int rc = prepare_decode(p, true, &a, &k)) return rc;
  a.lb_tag = next_tag();
  hipError_t e = k == DecodeKernel::kGqa ? ssattn::launch_decode_gqa(a, stream)
                                         : ssattn::launch_decode_mla(a, stream);
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  return ok();
}

int ss_attn_decode_combine(const ss_decode_params* p, hipStream_t stream) {
  ssattn::DecodeArgs a{};
  DecodeKernel k;
  if (int rc = prepare_decode(p, false, &a, &k)) return rc;
  if (!p->out) return fail(SS_ERR_INVALID_ARG, "out must be non-null");
  hipError_t e = ssattn::launch_decode_combine(a, stream);
  if (e != hipSuccess) return hip_fail(e, "combine launch");
  return ok();
}

int ss_attn_decode_paged(const ss_decode_paged_params* p, hipStream_t stream) {
  if (!p) return fail(SS_ERR_INVALID_ARG, "params is null");
  if (!p->q || !p->k_cache || !p->block_table || !p->seq_lens || !p->out)
    return fail(SS_ERR_INVALID_ARG, "q, k_cache, block_table, seq_lens and out must be non-null");
  // v_cache == NULL: a latent cache, the value row is the first Dv columns of the key row
  const bool latent = p->v_cache == nullptr;
  if (p->B <= 0 || p->Hq <= 0 || p->Hkv <= 0 || p->D <= 0 || p->Dv <= 0 ||
      p->max_blocks_per_seq <= 0 || p->num_blocks <= 0 || p->max_seq_len <= 0)
    return fail(SS_ERR_INVALID_ARG, "sizes must be positive");
  if (p->max_seq_len > kMaxLen)
    return fail(SS_ERR_INVALID_ARG, "max_seq_len above %d is not supported", kMaxLen);
  if (p->Hq % p->Hkv)
    return fail(SS_ERR_INVALID_ARG, "Hq (%d) must be a multiple of Hkv (%d)", p->Hq, p->Hkv);
  int block_log2 = -1;
  for (int l = 4; l <= 7; ++l)
    if (p->block_size == (1 << l)) block_log2 = l;
  if (block_log2 < 0)
    return fail(SS_ERR_INVALID_ARG, "block_size must be 16, 32, 64 or 128 (got %d)",
                p->block_size);
  if ((int64_t)p->max_blocks_per_seq * p->block_size < p->max_seq_len)
    return fail(SS_ERR_INVALID_ARG, "max_seq_len %d exceeds %d blocks of %d keys",
                p->max_seq_len, p->max_blocks_per_seq, p->block_size);
  if (p->num_splits < 0) return fail(SS_ERR_INVALID_ARG, "num_splits must be >= 0");
  if (int rc = check_scale(p->scale)) return rc;
  if (!(p->factor >= 0.f) || !std::isfinite(p->factor))
    return fail(SS_ERR_INVALID_ARG, "factor must be finite and >= 0 (got %g)", (double)p->factor);
  const int group = p->Hq / p->Hkv;
  const DecodeKernel kern = decode_kernel(p->D, p->Dv, group, latent);
  if (!latent && kern != DecodeKernel::kGqa)
    return fail(SS_ERR_UNSUPPORTED, "paged decode supports D == Dv in {64, 128} and Hq/Hkv in "
                "1..8, 16 or 32 (got D=%d Dv=%d group=%d)", p->D, p->Dv, group);
  if (latent && kern != DecodeKernel::kMla)
    return fail(SS_ERR_UNSUPPORTED, "paged latent decode supports D = 576, Dv = 512 and Hq/Hkv "
                "in {64, 128} (got D=%d Dv=%d group=%d)", p->D, p->Dv, group);
  if (latent && p->block_size < 32)
    return fail(SS_ERR_UNSUPPORTED, "paged latent decode needs block_size 32, 64 or 128 (got %d)",
                p->block_size);
  const DecodePlan pl =
      plan_decode(p->B, p->Hq, p->Hkv, p->max_seq_len, p->D, p->Dv, latent, p->num_splits, true);
  if (!p->workspace || p->workspace_bytes < pl.bytes)
    return fail(SS_ERR_WORKSPACE, "decode workspace needs %zu bytes (got %zu%s)", pl.bytes,
                p->workspace_bytes, p->workspace ? "" : ", null");
  char* ws = static_cast<char*>(p->workspace);
  ssattn::DecodeArgs a{};
  a.q = p->q;
  a.k = p->k_cache;
  a.v = p->v_cache;
  a.out = p->out;
  a.mask = p->skip_mask_out;
  a.part_o = reinterpret_cast<float*>(ws + pl.o_off);
  a.part_lse = reinterpret_cast<float*>(ws + pl.lse_off);
  a.lb_slot = reinterpret_cast<unsigned long long*>(ws + pl.slot_off);
  a.lb_timeouts = reinterpret_cast<unsigned int*>(ws + pl.timeout_off);
  a.B = p->B;
  a.Hq = p->Hq;
  a.Hkv = p->Hkv;
  a.Lk = p->max_seq_len;
  a.D = p->D;
  a.Dv = p->Dv;
  a.num_splits = pl.subs;
  a.tiles_per_split = pl.tiles_per_sub;
  a.chain_tiles = pl.chain_tiles;
  a.subs_per_chain = pl.subs_per_chain;
  a.scale = p->scale;
  a.log2_thr = 0.f;  // per sequence on the device
  a.thr_above_1 = 0;
  a.lb_tag = next_tag();
  a.block_table = p->block_table;
  a.seq_lens = p->seq_lens;
  a.thresholds = p->thresholds;
  a.factor = p->factor;
  a.block_log2 = block_log2;
  a.max_blocks = p->max_blocks_per_seq;
  a.num_blocks = p->num_blocks;
  a.mask_tiles = (int)ceil_div(p->max_seq_len, SS_TILE_KEYS);
  hipError_t e = latent ? ssattn::launch_decode_mla_paged(a, stream)
                        : ssattn::launch_decode_gqa_paged(a, stream);
  if (e != hipSuccess) return hip_fail(e, "paged decode launch");
  e = ssattn::launch_decode_combine(a, stream);
  if (e != hipSuccess) return hip_fail(e, "combine launch");
  return ok();
}

int ss_attn_decode_lookback_timeouts(const ss_decode_params* p, unsigned int* count_out,
                                     int reset, hipStream_t stream) {
  if (!count_out) return fail(SS_ERR_INVALID_ARG, "count_out is null");
  ssattn::DecodeArgs a{};
  DecodeKernel k;
  if (int rc = prepare_decode(p, false, &a, &k)) return rc;
  unsigned int v = 0;
  hipError_t e = hipMemcpyAsync(&v, a.lb_timeouts, sizeof(v), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e, "reading the look-back counter");
  if (reset) {
    static const unsigned int zero = 0;
    e = hipMemcpyAsync(a.lb_timeouts, &zero, sizeof(zero), hipMemcpyHostToDevice, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return hip_fail(e, "clearing the look-back counter");
  }
  *count_out = v;
  return ok();
}

int ss_attn_decode_ex(const ss_decode_params* p, hipStream_t stream) {
  if (!p) return fail(SS_ERR_INVALID_ARG, "params is null");
  if (!p->out) return fail(SS_ERR_INVALID_ARG, "out must be non-null");
  if (int rc = ss_attn_decode_partial(p, stream)) return rc;
  return ss_attn_decode_combine(p, stream);
}

int ss_attn_decode(const void* q, const void* k, const void* v, void* out, int B, int Hq,
                   int Hkv, int Lk, int D, int Dv, float scale, float threshold, int num_splits,
                   uint8_t* skip_mask_out, void* workspace, size_t workspace_bytes,
                   hipStream_t stream) {
  ss_decode_params p{q, k, v, out, B, Hq, Hkv, Lk, D, Dv, scale, threshold, num_splits,
                     SS_SPLIT_CHAINED, skip_mask_out, workspace, workspace_bytes};
  return ss_attn_decode_ex(&p, stream);
}

int ss_factor(ss_factor_mode mode, double a, double b, double target_sparsity,
              double threshold, int64_t seqlen, double* factor_out) {
  if (!factor_out) return fail(SS_ERR_INVALID_ARG, "factor_out is null");
  if (seqlen <= 0) return fail(SS_ERR_INVALID_ARG, "seqlen must be positive");
  if (mode == SS_FACTOR_CALIBRATED) {
    if (!std::isfinite(a) || !std::isfinite(b) || !std::isfinite(target_sparsity))
      return fail(SS_ERR_INVALID_ARG, "a, b and target_sparsity must be finite");
    if (target_sparsity < 0.0 || target_sparsity > 1.0)
      return fail(SS_ERR_INVALID_ARG, "target_sparsity must be in [0, 1]");
    const double f = a * std::exp(b * target_sparsity);
    if (!std::isfinite(f) || f < 0.0)
      return fail(SS_ERR_INVALID_ARG, "calibrated factor is negative or not finite");
    *factor_out = f;
    return ok();
  }
  if (mode == SS_FACTOR_DIRECT) {
    if (!std::isfinite(threshold) || threshold < 0.0)
      return fail(SS_ERR_INVALID_ARG, "threshold must be finite and >= 0");
    *factor_out = threshold * (double)seqlen;
    return ok();
  }
  return fail(SS_ERR_INVALID_ARG, "unknown factor mode %d", (int)mode);
}

int ss_threshold(double factor, int64_t seqlen, double* threshold_out) {
  if (!threshold_out) return fail(SS_ERR_INVALID_ARG, "threshold_out is null");
  if (seqlen <= 0) return fail(SS_ERR_INVALID_ARG, "seqlen must be positive");
  if (!std::isfinite(factor) || factor < 0.0)
    return fail(SS_ERR_INVALID_ARG, "factor must be finite and >= 0");
  *threshold_out = factor / (double)seqlen;
  return ok();
}

int ss_gate_enabled(int has_timestep, double t, int has_disabled_until, double disabled_until) {
  if (!has_disabled_until) return 1;
  if (!has_timestep) return 0;
  return t <= disabled_until ? 1 : 0;
}

int ss_resolve_threshold(ss_factor_mode mode, double a, double b, double target_sparsity,
                         double threshold, int64_t seqlen, int has_timestep, double t,
                         int has_disabled_until, double disabled_until, float* threshold_out) {
  if (!threshold_out) return fail(SS_ERR_INVALID_ARG, "threshold_out is null");
  double f = 0.0;
  if (int rc = ss_factor(mode, a, b, target_sparsity, threshold, seqlen, &f)) return rc;
  if (!ss_gate_enabled(has_timestep, t, has_disabled_until, disabled_until)) {
    *threshold_out = 0.f;
    return ok();
  }
  double thr = threshold;
  if (mode == SS_FACTOR_CALIBRATED) {
    if (int rc = ss_threshold(f, seqlen, &thr)) return rc;
  }
  *threshold_out = (float)thr;
  return ok();
}

}  // extern "C"
