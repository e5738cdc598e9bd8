// C ABI of the skip-softmax attention library: argument checks, the operating
// point (factor, threshold, timestep gate), the decode split policy and the
// kernel launches.  Every public function is declared in include/ss_attn.h.

#include "ss_attn.h"

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

int auto_splits(int B, int Hq, int Hkv, int Lk, int D, int Dv) {
  const int nK = (int)ceil_div(Lk, SS_TILE_KEYS);
  const int64_t units = (int64_t)B * Hkv;
  // Workgroups wanted to keep all 256 compute units streaming: the GQA kernel
  // is light per tile, so aim for ~4 resident workgroups per CU; the
  // latent-cache kernel carries 128 rows of MFMA work per tile, so one per CU.
  const int64_t want = (D >= 256) ? 256 : 1024;
  int64_t s = ceil_div(want, units);
  // A split restarts the running max, so keep at least 8 tiles per split.
  int64_t cap = nK / 8;
  if (cap < 1) cap = 1;
  if (s > cap) s = cap;
  if (s < 1) s = 1;
  return (int)s;
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
  return SS_OK;
}

}  // namespace

extern "C" {

const char* ss_last_error(void) { return g_err; }

const char* ss_version(void) { return "ssattn 0.1.0 (gfx950)"; }

int ss_attn_prefill_ex(const ss_prefill_params* p, hipStream_t stream) {
  if (int rc = validate_prefill(p)) return rc;
  ssattn::PrefillArgs a;
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
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Lk <= 0 || D <= 0 || Dv <= 0 || Hq % Hkv) return 0;
  return auto_splits(B, Hq, Hkv, Lk, D, Dv);
}

size_t ss_attn_decode_workspace_bytes(int B, int Hq, int Hkv, int Lk, int D, int Dv,
                                      int num_splits) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Lk <= 0 || D <= 0 || Dv <= 0 || Hq % Hkv ||
      num_splits < 0 || Lk > kMaxLen)
    return 0;
  const int nK = (int)ceil_div(Lk, SS_TILE_KEYS);
  const int req = num_splits == 0 ? auto_splits(B, Hq, Hkv, Lk, D, Dv) : num_splits;
  const SplitPlan sp = plan_splits(nK, req);
  const size_t rows = (size_t)sp.count * B * Hq;
  // split outputs, then split lse; both fp32, the lse block 256-byte aligned
  size_t o_bytes = rows * (size_t)Dv * sizeof(float);
  o_bytes = (o_bytes + 255) & ~(size_t)255;
  return o_bytes + rows * sizeof(float);
}

}  // extern "C"

namespace {

// Validate a decode call and fill the launch arguments (out may be null for
// the partial stage).  Returns SS_OK or an error code.
int prepare_decode(const void* q, const void* k, const void* v, int B, int Hq, int Hkv, int Lk,
                   int D, int Dv, float scale, float threshold, int num_splits,
                   const void* workspace, size_t workspace_bytes, bool check_inputs,
                   ssattn::DecodeArgs* a, bool* use_gqa) {
  if (check_inputs && (!q || !k)) return fail(SS_ERR_INVALID_ARG, "q and k must be non-null");
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Lk <= 0 || D <= 0 || Dv <= 0)
    return fail(SS_ERR_INVALID_ARG, "sizes must be positive");
  if (Lk > kMaxLen) return fail(SS_ERR_INVALID_ARG, "Lk above %d is not supported", kMaxLen);
  if (Hq % Hkv)
    return fail(SS_ERR_INVALID_ARG, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
  if (num_splits < 0) return fail(SS_ERR_INVALID_ARG, "num_splits must be >= 0");
  if (check_inputs) {
    if (!v && Dv > D) return fail(SS_ERR_INVALID_ARG, "v == NULL needs Dv <= D");
    if (int rc = check_scale(scale)) return rc;
    if (int rc = check_threshold(threshold)) return rc;
    const int group = Hq / Hkv;
    const bool latent = is_latent_decode(D, Dv, v);
    const bool gqa = ssattn::decode_gqa_supported(D, Dv, group, latent);
    const bool mla = !gqa && ssattn::decode_mla_supported(D, Dv, group, latent);
    if (!gqa && !mla)
      return fail(SS_ERR_UNSUPPORTED, "no decode kernel for D=%d Dv=%d group=%d %s", D, Dv,
                  group, latent ? "(latent V)" : "(separate V)");
    *use_gqa = gqa;
  }
  const size_t need = ss_attn_decode_workspace_bytes(B, Hq, Hkv, Lk, D, Dv, num_splits);
  if (!workspace || workspace_bytes < need)
    return fail(SS_ERR_WORKSPACE, "decode workspace needs %zu bytes (got %zu%s)", need,
                workspace_bytes, workspace ? "" : ", null");
  const int nK = (int)ceil_div(Lk, SS_TILE_KEYS);
  const int req = num_splits == 0 ? auto_splits(B, Hq, Hkv, Lk, D, Dv) : num_splits;
  const SplitPlan sp = plan_splits(nK, req);
  a->q = q;
  a->k = k;
  a->v = v;
  a->out = nullptr;
  a->mask = nullptr;
  const size_t rows = (size_t)sp.count * B * Hq;
  size_t o_bytes = rows * (size_t)Dv * sizeof(float);
  o_bytes = (o_bytes + 255) & ~(size_t)255;
  char* ws = static_cast<char*>(const_cast<void*>(workspace));
  a->part_o = reinterpret_cast<float*>(ws);
  a->part_lse = reinterpret_cast<float*>(ws + o_bytes);
  a->B = B;
  a->Hq = Hq;
  a->Hkv = Hkv;
  a->Lk = Lk;
  a->D = D;
  a->Dv = Dv;
  a->num_splits = sp.count;
  a->tiles_per_split = sp.per;
  a->scale = scale;
  a->log2_thr = log2_threshold(threshold);
  a->thr_above_1 = threshold > 1.f;
  return SS_OK;
}

}  // namespace

extern "C" {

int ss_attn_decode_partial(const void* q, const void* k, const void* v, int B, int Hq, int Hkv,
                           int Lk, int D, int Dv, float scale, float threshold, int num_splits,
                           uint8_t* skip_mask_out, void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
  ssattn::DecodeArgs a;
  bool gqa = false;
  if (int rc = prepare_decode(q, k, v, B, Hq, Hkv, Lk, D, Dv, scale, threshold, num_splits,
                              workspace, workspace_bytes, true, &a, &gqa))
    return rc;
  a.mask = skip_mask_out;
  hipError_t e = gqa ? ssattn::launch_decode_gqa(a, stream) : ssattn::launch_decode_mla(a, stream);
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  return ok();
}

int ss_attn_decode_combine(void* out, int B, int Hq, int Hkv, int Lk, int D, int Dv,
                           int num_splits, const void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
  if (!out) return fail(SS_ERR_INVALID_ARG, "out must be non-null");
  ssattn::DecodeArgs a;
  bool gqa = false;
  if (int rc = prepare_decode(nullptr, nullptr, nullptr, B, Hq, Hkv, Lk, D, Dv, 1.f, 0.f,
                              num_splits, workspace, workspace_bytes, false, &a, &gqa))
    return rc;
  a.out = out;
  hipError_t e = ssattn::launch_decode_combine(a, stream);
  if (e != hipSuccess) return hip_fail(e, "combine launch");
  return ok();
}

int ss_attn_decode(const void* q, const void* k, const void* v, void* out, int B, int Hq,
                   int Hkv, int Lk, int D, int Dv, float scale, float threshold, int num_splits,
                   uint8_t* skip_mask_out, void* workspace, size_t workspace_bytes,
                   hipStream_t stream) {
  if (!out) return fail(SS_ERR_INVALID_ARG, "out must be non-null");
  if (int rc = ss_attn_decode_partial(q, k, v, B, Hq, Hkv, Lk, D, Dv, scale, threshold,
                                      num_splits, skip_mask_out, workspace, workspace_bytes,
                                      stream))
    return rc;
  return ss_attn_decode_combine(out, B, Hq, Hkv, Lk, D, Dv, num_splits, workspace,
                                workspace_bytes, stream);
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
