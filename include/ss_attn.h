/*
 * ss_attn.h -- C ABI of the skip-softmax (BLASST) attention library for
 * AMD Instinct MI355X (gfx950).
 *
 * The method.  Attention is computed in one streaming online-softmax pass
 * over key tiles of 128 keys.  Per query row the pass keeps the running max m,
 * the running denominator l = sum exp(s - m) and the running numerator
 * O = sum exp(s - m) v, rescaling l and O when m grows, and returns O / l
 * (vLLM-Omni design page "Skip-Softmax", section "The online-softmax pass").
 * Each tile's scores S = Q K_j^T * scale are always computed; the tile is then
 * skipped -- no exponentials, no P.V accumulation, and in decode no V read --
 * when exp(tile_max - running_max) < threshold (same page, "The skip test";
 * BLASST summary page of arXiv 2512.12087, sections "Kerninzicht" and
 * "Kernel-ontwerp").  The threshold is normalised by the sequence length,
 * threshold = factor / seqlen, with a calibrated or a direct factor (design
 * page, "The threshold"), and the mode can be gated off during early
 * diffusion timesteps (design page, "Timestep gating").
 *
 * Conventions shared by every entry point:
 *  - Tensors are dense, contiguous, head-major device buffers owned by the
 *    caller; the library allocates no device memory and keeps no state other
 *    than a thread-local error string and a counter that numbers decode
 *    launches.
 *  - Kernels are enqueued on `stream` and the call returns without
 *    synchronising.  A NULL stream is the default stream.
 *  - A tile is skipped iff  max over the rows of its decision block of
 *    (tile_max_r - m_r)  <  ln(threshold), where m_r is the running max of
 *    row r before the tile.  A row that has seen no key yet never lets its
 *    first visible tile be skipped; a row that sees no key of the tile does
 *    not hold the tile.  The comparison is strict, so threshold 0 is exactly
 *    dense attention.  A skipped tile still updates m (its scores were
 *    computed); when threshold > 1 lets a skipped tile raise m, l and O are
 *    rescaled so the result stays exact over the kept keys.
 *  - Skip-mask bytes: 0 = tile computed, 1 = tile skipped, 2 = tile not
 *    visited (entirely above the causal diagonal).
 *  - Every function returns an ss_status.  On failure nothing is launched and
 *    ss_last_error() describes the problem.
 */
#ifndef SS_ATTN_H
#define SS_ATTN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SS_TILE_KEYS 128 /* keys per tile (design page, "The online-softmax pass") */
#define SS_TILE_ROWS 128 /* query rows per prefill decision block */

typedef enum {
  SS_OK = 0,
  SS_ERR_INVALID_ARG = -1, /* null pointer, bad size, bad threshold, Hq % Hkv != 0 */
  SS_ERR_UNSUPPORTED = -2, /* head dimensions or grouping without a kernel */
  SS_ERR_HIP = -3,         /* a HIP launch failed; see ss_last_error() */
  SS_ERR_WORKSPACE = -4    /* workspace missing or too small */
} ss_status;

typedef enum { SS_FACTOR_DIRECT = 0, SS_FACTOR_CALIBRATED = 1 } ss_factor_mode;
typedef enum { SS_DTYPE_BF16 = 0, SS_DTYPE_F32 = 1 } ss_dtype;

/* Key-tile visit order of a prefill query tile.  ASCENDING walks tiles
 * 0, 1, ...  DIAG_FIRST starts at the query tile's diagonal: causal goes from
 * the last visible tile down to tile 0; non-causal goes from the query tile's
 * own key tile upwards and wraps to tile 0.  The pages describe a single
 * streaming pass and do not fix the order. */
typedef enum { SS_ORDER_ASCENDING = 0, SS_ORDER_DIAG_FIRST = 1 } ss_order;

enum { SS_MASK_COMPUTED = 0, SS_MASK_SKIPPED = 1, SS_MASK_UNVISITED = 2 };

/* Who decides a skip.  The pages keep the running max per query row (design
 * page, "The online-softmax pass") and state the test per key tile ("The
 * skip test"); which query rows share one decision is left open.
 *   SS_SKIP_TILE (default): one decision per (row block, key tile) -- the
 *     128-row query tile of one head in prefill, the Hq/Hkv heads of one KV
 *     head in decode -- taken when every row of the block passes the test.
 *   SS_SKIP_ROW: every row decides alone: a row whose own
 *     exp(tile_max_r - m_r) is below the threshold adds nothing from the tile
 *     (its running max still moves).  A tile where every row skips runs no
 *     exponentials and no P.V (decode: reads no V); those tiles, and so the
 *     tile-level skip_mask_out, are the same as with SS_SKIP_TILE.  The
 *     per-row decisions go to row_mask_out when given.
 * Supported with SS_SKIP_ROW: prefill (bf16 and fp32) and the separate-V
 * decode of ss_attn_decode_ex / ss_attn_decode_partial. */
typedef enum { SS_SKIP_TILE = 0, SS_SKIP_ROW = 1 } ss_granularity;

/* ------------------------------------------------------------------ prefill */

/*
 * Skip-softmax prefill (design page, "The online-softmax pass" and "The skip
 * test"; BLASST summary, "Kernel-ontwerp": the prefill kernel skips the
 * exponentials and the P.V matrix multiply of skipped tiles).
 *
 *   q   [B, Hq,  Lq, D ]  bf16     k [B, Hkv, Lk, D]  bf16
 *   v   [B, Hkv, Lk, Dv]  bf16   out [B, Hq,  Lq, Dv] bf16 (written)
 *   skip_mask_out  u8 [B, Hq, ceil(Lq/128), ceil(Lk/128)] or NULL (written)
 *
 * Query head h reads KV head h / (Hq / Hkv).  The skip decision for key tile
 * j is uniform over each 128-row query tile of one head.  `causal` masks key
 * c from query row r when c > r + Lk - Lq (bottom-right alignment); rows that
 * see no key produce 0.  Supported: D == Dv in {64, 128}.  `scale` > 0 and
 * finite; `threshold` finite and >= 0.  Key tiles are visited in ascending
 * order.
 */
int ss_attn_prefill(const void* q, const void* k, const void* v, void* out, int B, int Hq,
                    int Hkv, int Lq, int Lk, int D, int Dv, float scale, int causal,
                    float threshold, uint8_t* skip_mask_out, hipStream_t stream);

/* fp32 debug path: the same operation and arguments with fp32 q, k, v, out,
 * computed in fp32 throughout (no bf16 rounding of P). */
int ss_attn_prefill_f32(const float* q, const float* k, const float* v, float* out, int B,
                        int Hq, int Hkv, int Lq, int Lk, int D, int Dv, float scale, int causal,
                        float threshold, uint8_t* skip_mask_out, hipStream_t stream);

/* Full form: the two calls above are this one with dtype BF16 / F32, order
 * ASCENDING and granularity SS_SKIP_TILE.  row_mask_out (SS_SKIP_ROW only,
 * else it must be NULL): u8 [B, Hq, Lq, ceil(Lk/128)], every row's decision
 * per key tile (2 for tiles its query tile does not visit), or NULL.
 * lse_out: fp32 [B, Hq, Lq] or NULL; row r receives ln of its sum of
 * exp(scale q_r . k_c) over the keys it kept (-inf when it kept none), what
 * ss_attn_prefill_backward needs to rebuild the row's weights. */
typedef struct {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  int B, Hq, Hkv, Lq, Lk, D, Dv;
  float scale;
  float threshold;
  int causal;
  int dtype; /* ss_dtype */
  int order; /* ss_order */
  uint8_t* skip_mask_out;
  int granularity;       /* ss_granularity */
  uint8_t* row_mask_out; /* SS_SKIP_ROW: u8 [B, Hq, Lq, ceil(Lk/128)] or NULL */
  float* lse_out;        /* fp32 [B, Hq, Lq] or NULL */
} ss_prefill_params;

int ss_attn_prefill_ex(const ss_prefill_params* p, hipStream_t stream);

/*
 * Skip-aware backward of the prefill.  The pages train with the sparsity on
 * (BLASST summary, "Belangrijkste Bijdragen": sparsity-aware training) and
 * give no backward pass; this is the derivative of the forward with its skip
 * decisions held fixed.  With them fixed, row r of query tile i attends by
 * plain softmax (design page, "The online-softmax pass") to the visible keys
 * of the key tiles j whose skip_mask byte for (b, h, i, j) is 0:
 *     P = exp(scale Q K^T - lse),  dV = P^T dO,  dP = dO V^T,
 *     Delta_r = dO_r . O_r,  dS = P (dP - Delta),
 *     dQ = scale dS K,  dK = scale dS^T Q
 * (dK and dV of a KV head sum over the query heads that read it).  Pairs the
 * forward skipped or did not visit contribute nothing and run no product.
 *
 *   q, k, v, out, dout   as the forward: q [B,Hq,Lq,D], k [B,Hkv,Lk,D],
 *                        v [B,Hkv,Lk,Dv]; out = the forward's output and
 *                        dout = dL/dout, both [B,Hq,Lq,Dv]; bf16
 *   lse        fp32 [B,Hq,Lq], the forward's lse_out
 *   skip_mask  u8 [B,Hq,ceil(Lq/128),ceil(Lk/128)], the forward's
 *              skip_mask_out (SS_SKIP_TILE), or NULL for every visible tile
 *              (the derivative of dense attention)
 *   dq [B,Hq,Lq,D], dk [B,Hkv,Lk,D], dv [B,Hkv,Lk,Dv]  bf16 (written; every
 *              element, zeros where no kept pair reaches it)
 *   workspace  caller-owned device memory of at least
 *              ss_attn_prefill_backward_workspace_bytes(B, Hq, Lq) bytes
 *              (per-row statistics; contents on entry do not matter)
 *
 * scale, causal and the sizes must be those of the forward call.  Supported:
 * dtype SS_DTYPE_BF16, D == Dv in {64, 128}.  Three kernels on `stream`
 * (row statistics, then dK/dV, then dQ); no atomics, so the result is the
 * same bit for bit on every run.
 */
typedef struct {
  const void* q;
  const void* k;
  const void* v;
  const void* out;
  const void* dout;
  const float* lse;
  const uint8_t* skip_mask;
  void* dq;
  void* dk;
  void* dv;
  int B, Hq, Hkv, Lq, Lk, D, Dv;
  float scale;
  int causal;
  int dtype; /* ss_dtype: SS_DTYPE_BF16 */
  void* workspace;
  size_t workspace_bytes;
} ss_prefill_bwd_params;

size_t ss_attn_prefill_backward_workspace_bytes(int B, int Hq, int Lq);
int ss_attn_prefill_backward(const ss_prefill_bwd_params* p, hipStream_t stream);

/* ------------------------------------------------------------------ decode */

/* How the key tiles of one sequence are split across workgroups.
 * CHAINED (the default): the splits run in parallel, but every split first
 *   publishes its tile maxima and takes the running max of all earlier splits
 *   into its decisions, so the skip decisions are exactly those of one
 *   streaming pass over the whole sequence -- the method as the pages state
 *   it -- whatever the split count.
 * INDEPENDENT: every split is its own streaming pass with its own running max
 *   (a split restarts at -inf), so decisions depend on the split count. */
typedef enum { SS_SPLIT_CHAINED = 0, SS_SPLIT_INDEPENDENT = 1 } ss_split_mode;

/*
 * Split-KV skip-softmax decode of one query token per sequence (BLASST
 * summary, "Kerninzicht" and "Kernel-ontwerp": in decode a skipped tile also
 * skips its V load from HBM, and V loads of surviving tiles are issued
 * together).
 *
 *   q   [B, Hq, D]  bf16           k [B, Hkv, Lk, D] bf16
 *   v   [B, Hkv, Lk, Dv] bf16, or NULL: the value row of key c is then the
 *       first Dv columns of key row c (a shared latent cache, Dv <= D)
 *   out [B, Hq, Dv] bf16 (written)
 *   skip_mask_out  u8 [B, Hkv, ceil(Lk/128)] or NULL (written)
 *
 * The key tiles are cut into num_splits contiguous splits of
 * ceil(nK / num_splits) tiles each (the last may be shorter; num_splits is
 * clamped to [1, nK] and empty trailing splits are dropped).  In CHAINED mode
 * the count is raised where a split would exceed what one workgroup can hold
 * (decisions do not depend on it).  A second kernel merges the splits with a
 * log-sum-exp combine.  The skip decision is uniform over the Hq/Hkv query
 * heads that share a KV head.  num_splits = 0 selects ss_decode_num_splits().
 *
 * `workspace` is caller-owned device memory of at least
 * ss_attn_decode_workspace_bytes() bytes; its contents on entry do not
 * matter, and two calls that overlap in time must not share one.  Supported:
 * (D, Dv) = (64, 64) or (128, 128) with Hq/Hkv in 1..8, 16 or 32 (multi-head,
 * grouped-query and multi-query attention: the BLASST summary, "Belangrijkste
 * Bijdragen", names MHA, GQA, MQA and MLA); (576, 512) with v == NULL and
 * Hq/Hkv in {64, 128} (a shared latent cache).
 *
 * With a latent cache the value is part of the key row, so a skipped tile
 * saves its exponentials and its P.V work but no bytes.  CHAINED splits score
 * every tile of a sequence before any decision and then read the kept tiles
 * again; INDEPENDENT splits (and a single split) run one streaming pass per
 * split, which decides each tile as it is scored and reads a kept tile once
 * more from the last-level cache, not from HBM.
 *
 * ss_attn_decode is ss_attn_decode_ex with split_mode CHAINED.
 */
int ss_attn_decode(const void* q, const void* k, const void* v, void* out, int B, int Hq,
                   int Hkv, int Lk, int D, int Dv, float scale, float threshold, int num_splits,
                   uint8_t* skip_mask_out, void* workspace, size_t workspace_bytes,
                   hipStream_t stream);

typedef struct {
  const void* q;
  const void* k;
  const void* v; /* NULL: latent cache, value = first Dv columns of the key row */
  void* out;
  int B, Hq, Hkv, Lk, D, Dv;
  float scale;
  float threshold;
  int num_splits; /* 0 = automatic */
  int split_mode; /* ss_split_mode */
  uint8_t* skip_mask_out;
  void* workspace;
  size_t workspace_bytes;
  int granularity;       /* ss_granularity; SS_SKIP_ROW needs a separate v */
  uint8_t* row_mask_out; /* SS_SKIP_ROW: u8 [B, Hq, ceil(Lk/128)] or NULL */
} ss_decode_params;

int ss_attn_decode_ex(const ss_decode_params* p, hipStream_t stream);

/* The two stages of ss_attn_decode_ex, for callers that time or schedule them
 * separately.  ss_attn_decode_partial runs every split (p->out is not used)
 * and leaves in the workspace, at offset 0, O_s / l_s as fp32 [S][B][Hq][Dv]
 * and, at the next 256-byte boundary, lse_s = m_s + ln l_s as fp32
 * [S][B][Hq] (-inf for a split whose tiles were all skipped), S being the
 * effective split count.  ss_attn_decode_combine merges them into p->out
 * (p->q, p->k, p->v are not used); the other fields must equal those of the
 * partial call. */
int ss_attn_decode_partial(const ss_decode_params* p, hipStream_t stream);
int ss_attn_decode_combine(const ss_decode_params* p, hipStream_t stream);

/* Look-back give-ups of chained splits.  A chained split waits for the
 * running maxima that the earlier splits of its sequence publish.  Those
 * splits are dispatched earlier -- the hardware starts workgroups in order of
 * their index, which forward progress relies on -- so the wait is short; it
 * is still bounded (about 2^21 polls), and a wait that gives up decides
 * without that split's maxima (it keeps tiles the exact rule might skip: the
 * output stays a valid softmax over the kept keys, but the mask can differ
 * from the oracle's) and adds 1 to a 32-bit counter in the last 256 bytes of
 * the workspace.  The counter is cumulative over the calls that use one
 * workspace and starts at whatever the workspace held: zero the workspace
 * once when allocating it, or call this with reset = 1 before the calls to
 * be checked.
 *
 * Reads the counter into *count_out after the work already queued on
 * `stream` (it synchronizes the stream, so do not call it under graph
 * capture) and, with reset != 0, sets it back to 0.  p locates the counter
 * exactly as the decode call does: pass the fields of that call (sizes,
 * num_splits, split_mode, workspace, workspace_bytes; q, k, v, out and the
 * masks are not read).  For ss_attn_decode_paged pass Lk = max_seq_len and
 * a non-null v. */
int ss_attn_decode_lookback_timeouts(const ss_decode_params* p, unsigned int* count_out,
                                     int reset, hipStream_t stream);

/*
 * Allocation-free decode, for callers that cannot allocate device memory
 * (code under graph capture, tight serving loops, hosts that forbid it):
 * ss_attn_decode without the workspace arguments.  The split workspace is a
 * fixed array of SS_DECODE_NOALLOC_SCRATCH_BYTES inside this library, one per
 * GPU, held from the library's first use on that GPU until the process ends;
 * this call allocates nothing and frees nothing.
 *
 * Arguments, layouts, splits and results are those of ss_attn_decode
 * (CHAINED splits).  With num_splits = 0 the automatic count is lowered, if
 * needed, to the largest one whose workspace fits the array (chained
 * decisions do not depend on the count).  A call whose workspace does not
 * fit even so -- or an explicit num_splits whose workspace does not fit --
 * returns SS_ERR_WORKSPACE without launching.
 *
 * Every call on one GPU shares that GPU's array: calls that overlap in time on
 * one GPU (different streams, or different host threads, without ordering
 * between them) race and give wrong results.  Calls on one stream are
 * ordered and safe.  The look-back give-up counter of this array is not
 * exposed.
 */
#define SS_DECODE_NOALLOC_SCRATCH_BYTES (48u << 20)

int ss_attn_decode_noalloc(const void* q, const void* k, const void* v, void* out, int B,
                           int Hq, int Hkv, int Lk, int D, int Dv, float scale, float threshold,
                           int num_splits, uint8_t* skip_mask_out, hipStream_t stream);

/*
 * Decode over a block-paged KV cache, one query token per sequence, sequences
 * of different lengths, each with its own threshold (design page "The
 * threshold": the threshold is a factor over the sequence length, so every
 * sequence of a batch gets factor / L_b).  Splits are CHAINED: the decisions
 * of sequence b are those of one streaming pass over its L_b keys.
 *
 *   q            [B, Hq, D] bf16
 *   k_cache      [num_blocks, Hkv, block_size, D] bf16
 *   v_cache      [num_blocks, Hkv, block_size, Dv] bf16, or NULL: a latent
 *                cache, the value row of a key is the first Dv columns of
 *                its key row (D = 576, Dv = 512, Hq/Hkv in {64, 128})
 *   block_table  int32 [B, max_blocks_per_seq]: cache block of each
 *                block_size-key block of a sequence (device memory)
 *   seq_lens     int32 [B]: keys of each sequence (device memory)
 *   thresholds   fp32 [B] (device memory), or NULL: sequence b then uses
 *                factor / seq_lens[b]; factor 0 is dense
 *   out          [B, Hq, Dv] bf16 (written)
 *   skip_mask_out u8 [B, Hkv, ceil(max_seq_len/128)] or NULL (written; 2 marks
 *                tiles past a sequence's end)
 *
 * Host-side checks: shapes as for ss_attn_decode (Dv = D with a v_cache),
 * block_size in {16, 32, 64, 128} ({32, 64, 128} for a latent cache: the 32
 * keys of one latent load step lie in one block), max_seq_len <=
 * max_blocks_per_seq * block_size, factor
 * finite and >= 0, workspace of ss_attn_decode_workspace_bytes(B, Hq, Hkv,
 * max_seq_len, D, Dv, num_splits) bytes.  The device arrays are trusted up to
 * clamping: a sequence length is clamped into [0, max_seq_len] (0 writes a
 * zero output row) and a block id into [0, num_blocks).  Thresholds from the
 * array must be >= 0.
 */
typedef struct {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const float* thresholds;
  void* out;
  int B, Hq, Hkv, D, Dv;
  int block_size;
  int max_blocks_per_seq;
  int num_blocks;
  int max_seq_len;
  float scale;
  float factor;
  int num_splits; /* 0 = automatic, as ss_decode_num_splits(..., max_seq_len, ...) */
  uint8_t* skip_mask_out;
  void* workspace;
  size_t workspace_bytes;
} ss_decode_paged_params;

int ss_attn_decode_paged(const ss_decode_paged_params* p, hipStream_t stream);

/* Bytes of decode workspace for these sizes (num_splits as for
 * ss_attn_decode, 0 = automatic), enough for either split mode.  Returns 0
 * for invalid sizes. */
size_t ss_attn_decode_workspace_bytes(int B, int Hq, int Hkv, int Lk, int D, int Dv,
                                      int num_splits);

/* The automatic split count: deterministic in the sizes, exported so that a
 * reference can reproduce the same partition.  Returns a value in [1, nK], or
 * 0 for invalid sizes. */
int ss_decode_num_splits(int B, int Hq, int Hkv, int Lk, int D, int Dv);

/* ------------------------------------------------------------------ host helpers */

/*
 * factor of the per-tile threshold (design page, "The threshold"):
 *   SS_FACTOR_CALIBRATED: factor = a * exp(b * target_sparsity), with a, b
 *                         fitted per model; target_sparsity in [0, 1].
 *   SS_FACTOR_DIRECT:     factor = threshold * seqlen (calibration free).
 * Rejects seqlen <= 0 and non-finite inputs.  Writes *factor_out.
 */
int ss_factor(ss_factor_mode mode, double a, double b, double target_sparsity,
              double threshold, int64_t seqlen, double* factor_out);

/* threshold = factor / seqlen (design page, "The threshold"; BLASST summary,
 * "Calibratie en Thresholding": inversely proportional to the context
 * length).  Rejects seqlen <= 0 and a negative or non-finite factor. */
int ss_threshold(double factor, int64_t seqlen, double* threshold_out);

/*
 * Timestep gating (design page, "Timestep gating"): returns 1 (sparse) or 0
 * (dense).  Without disabled_until the mode is always on; with it, the mode
 * is on once a published timestep t satisfies t <= disabled_until, and a
 * pipeline that publishes no timestep stays dense.
 */
int ss_gate_enabled(int has_timestep, double t, int has_disabled_until, double disabled_until);

/*
 * The kernel threshold for one call: dense (0) when the gate is off;
 * otherwise the direct user threshold unchanged (no factor round trip), or
 * factor / seqlen with the calibrated factor.  Writes *threshold_out.
 */
int ss_resolve_threshold(ss_factor_mode mode, double a, double b, double target_sparsity,
                         double threshold, int64_t seqlen, int has_timestep, double t,
                         int has_disabled_until, double disabled_until, float* threshold_out);

/* Thread-local description of the last failure ("" if none). */
const char* ss_last_error(void);

/* Library version string. */
const char* ss_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SS_ATTN_H */
