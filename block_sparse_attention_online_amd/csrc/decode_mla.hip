// Split-KV skip-softmax decode over a shared latent cache: many query heads
// (64 or 128) read one 576-wide latent key row, whose first 512 columns are
// also the value row.  bf16 inputs, fp32 accumulation, gfx950.
//
// Method: vLLM-Omni design page "Skip-Softmax", sections "The online-softmax
// pass" and "The skip test"; BLASST summary page, sections "Kerninzicht" and
// "Kernel-ontwerp".  The skip is decided once per 128-key tile for the whole
// group of query heads that share the latent row, from each head's tile max
// against its running max.  Since the value is a slice of the key row, a
// skipped tile saves the exponentials and the P.V product, not HBM bytes.
//
// Work split: one workgroup per (batch, sub-split of at most 64 tiles) with
// all G query heads: G / 32 waves, wave w owns heads [32 w, 32 w + 32).  MFMA
// v_mfma_f32_32x32x16_bf16 throughout, transposed products so the heads are
// the MFMA columns:
//   S^T [32 keys x 32 heads] = K [32 x 576] . Q^T [576 x 32]
//   O^T [512 x 32 heads]    += V^T [512 x 32 keys] . P^T [32 keys x 32 heads]
// Q^T lives in registers for the whole call (36 k-steps), O^T in the
// accumulation registers (16 blocks of 32 value columns).  The lane that owns
// a head's scores also holds them in the layout of the P^T operand, so the
// exponentials never leave the lane.  The decision (a max over heads) crosses
// waves through LDS once per sub-split; no other workgroup is involved.
//
// Keys move through a three-slot LDS ring in steps of 32 keys x 576 columns
// (direct global -> LDS loads).  One step serves both products: the score
// reads take 16-byte chunks of each key row, the value reads take the same
// image through ds_read_b64_tr_b16 transpose reads, so every byte comes into
// the workgroup once per pass.  Columns 0..511 are stored as four blocks of
// [32 keys x 128 columns] (256-byte rows), columns 512..575 as a block of
// [32 keys x 64 columns] (128-byte rows); chunks are XOR-swizzled by row so
// both read patterns hit distinct banks.
//
//  * threshold 0: one online pass whose exponent reference trails the
//    running max by at most 2^64 (see kRefMargin); the pass starts over only
//    for a head whose scores climb further.
//  * threshold > 0, sub-splits that are whole chains (independent splits, or
//    one split): a single streaming pass (stream mode below).  Each tile is
//    scored and decided against the running max of the tiles before it in
//    the chain; a kept tile is read once more a few steps later, while its
//    bytes are still in the device's last-level cache, scored again and
//    multiplied by V.  No tile is read from HBM twice.
//  * threshold > 0, chains cut into several sub-splits: a score pass over
//    the sub-split records every head's tile maxima (LDS table); the decision
//    folds in the maxima of the earlier sub-splits of the chain (published
//    per head, each read with a launch tag), so the decisions are those of
//    one streaming pass over the chain; then the kept tiles are read again,
//    scored, exponentiated against the sub-split's own per-head max (no
//    rescaling) and multiplied by V.
//
// The split's O / l and lse go to the workspace; decode_combine merges splits.

#include "device_common.h"
#include "launch.h"

namespace ssattn {
namespace {

constexpr int kDqk = 576;                 // latent key width
constexpr int kDv = 512;                  // value width (leading columns of the key row)
constexpr int kHeadsPerWave = 32;
constexpr int kTmax = 64;                 // tiles per sub-split
constexpr int kShareMinTiles = 16;        // tiles per sub-split from which the kept tiles are shared out
constexpr int kStepKeys = 32;             // keys per ring step
constexpr int kStepsPerTile = kTile / kStepKeys;
constexpr int kBlkBytes = kStepKeys * 256;               // [32 keys x 128 columns] bf16
constexpr int kRopeOff = 4 * kBlkBytes;                  // [32 keys x 64 columns] block
constexpr int kStepBytes = kRopeOff + kStepKeys * 128;   // 36 KB
constexpr int kUnits = kStepBytes / 1024;                // 1 KB wave load instructions per step
constexpr int kQk = kDqk / 16;                           // 36 MFMA k-steps over the key width
constexpr int kVb = kDv / 32;                            // 16 value-column blocks
// How far (log2 units) a head's scores may rise above its exponent reference
// before a pass starts over: p = exp2(s - ref) then stays below 2^64, and its
// sums over a sequence (at most 2^24 keys, |v| bf16) stay far below fp32's
// 2^128; fp32 and bf16 carry such p with the same relative precision as p <= 1.
constexpr float kRefMargin = 64.f;
constexpr int kSpinCap = 1 << 21;

typedef __attribute__((ext_vector_type(4))) short s16x4_t;
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

// Physical 16-byte chunk = logical chunk ^ swizzle(row).
//  * 256-byte rows (16 chunks): score reads take one chunk of 16 consecutive
//    rows -> 16 distinct values over r & 15; value transpose reads take
//    64 bytes (4 chunks) of 4 consecutive rows per 32 lanes -> the 4 rows on
//    4 different 64-byte bank groups: chunk bits 2-3 take r & 3, bits 0-1
//    (r >> 2) & 3 (the dual_slot swizzle for D = 128).
//  * 128-byte rows (8 chunks, two rows per 256 bytes): score reads only.
__device__ __forceinline__ int swz256(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
__device__ __forceinline__ int swz128(int r) { return (r >> 1) & 7; }

__device__ __forceinline__ unsigned long long tagged(unsigned tag, float x) {
  return ((unsigned long long)tag << 32) | __float_as_uint(x);
}

// Relaxed device-scope poll of a tagged value; gives up after kSpinCap polls
// (counted in *timeouts, value -inf).
__device__ __forceinline__ float poll_tagged(unsigned long long* p, unsigned tag,
                                             unsigned* timeouts) {
  int spins = 0;
  unsigned long long v;
  while (((v = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) >> 32) != tag &&
         spins < kSpinCap) {
    __builtin_amdgcn_s_sleep(1);
    ++spins;
  }
  if (spins >= kSpinCap) {
    atomicAdd(timeouts, 1u);
    return neg_inf();
  }
  return __uint_as_float((unsigned)v);
}

// The score MFMAs in their VGPR form.  Every builtin MFMA of this kernel is
// compiled to the accumulation-register form (the [512 x 32] output blocks
// fill all 256 of them), so the score products, whose results the vector ALU
// reads, are written out here.  The hardware forwards an accumulator from one
// MFMA to the next that names it as its own (no wait); the first MFMA of a
// chain starts from 0 and is preceded by two wait states for a vector ALU
// write of its operands; mfma_vgpr_drain gives the 24 wait states an MFMA
// result needs before a vector ALU instruction may read it, and ties the
// chains so that nothing reads them earlier.
__device__ __forceinline__ void mfma_vgpr_first(f32x16_t& acc, u32x4_t a, bf16x8_t b) {
  asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_vgpr(f32x16_t& acc, u32x4_t a, bf16x8_t b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_vgpr_drain(f32x16_t& x, f32x16_t& y) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(x), "+v"(y));
}

// Kernel modes.  kModeSplit: stage 0 or 1 (a.mla_stage); kModeShare: stage 2
// of a thresholded decode (this workgroup's share of the sequence's kept
// tiles, from the planning launch); kModeStream: the single streaming pass of
// a thresholded decode whose sub-splits are whole chains.
//
// PAGED (kModeSplit, stage 0 only): the latent rows come from a
// [num_blocks, Hkv, 2^block_log2, 576] cache through a per-sequence block
// table (block size 32 or more, so the 32 keys of a ring step lie in one
// block); sequence b has seq_lens[b] keys (a.Lk is their upper bound) and the
// threshold thresholds[b], or factor / seq_lens[b].
constexpr int kModeSplit = 0;
constexpr int kModeShare = 1;
constexpr int kModeStream = 2;

template <int NW, int MODE, bool PAGED = false>
__global__ __launch_bounds__(64 * NW, 1) void decode_mla_kernel(DecodeArgs a) {
  static_assert(!PAGED || MODE == kModeSplit, "paged caches: one launch per decode");
  constexpr bool SHARE = MODE == kModeShare;
  constexpr int G = NW * kHeadsPerWave;  // heads per latent head
  constexpr int kThreads = 64 * NW;
  constexpr int LPW = kUnits / NW;       // load instructions per wave per step
  static_assert(LPW * NW == kUnits, "step loads");
  __shared__ __attribute__((aligned(1024))) unsigned char slot0[kStepBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char slot1[kStepBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char slot2[kStepBytes];
  __shared__ __attribute__((aligned(16))) float tmaxs[kTmax * G];  // [tile][head]
  __shared__ float part_red[2][G];
  __shared__ float s_mref[G];
  __shared__ float s_dtile[kTmax];
  __shared__ int s_surv[kTmax];
  __shared__ int s_nsurv;
  __shared__ int s_restart;
  __shared__ int s_blk[PAGED ? kTmax * kTile / 32 : 1];  // paged: this sub-split's cache blocks

  // block -> (batch, sub-split): sub-splits in order, so every look-back
  // waits only on lower blocks (dispatched first)
  const int S = a.num_splits;
  const int usub = blockIdx.x;
  const int sub = usub % S;
  const int pair = usub / S;  // b * Hkv + hk
  const int hk = pair % a.Hkv;
  const int b = pair / a.Hkv;
  // the sequence's length and threshold (paged: per sequence)
  int Lk = a.Lk;
  float log2_thr = a.log2_thr;
  if constexpr (PAGED) {
    Lk = min(max(a.seq_lens[b], 0), a.Lk);
    const float thr = a.thresholds ? a.thresholds[b]
                                   : (Lk > 0 ? (float)((double)a.factor / (double)Lk) : 0.f);
    log2_thr = thr > 0.f ? (float)log2((double)thr) : neg_inf();
  }
  const int nK = (Lk + kTile - 1) / kTile;
  const int mstride = PAGED ? a.mask_tiles : nK;  // mask entries per (batch, latent head)
  const int chain = sub / a.subs_per_chain;
  const int link = sub % a.subs_per_chain;
  const int chain_t0 = chain * a.chain_tiles;
  const int chain_t1 = min(chain_t0 + a.chain_tiles, nK);
  const int t0 = chain_t0 + link * a.tiles_per_split;
  const int T = max(0, min(t0 + a.tiles_per_split, chain_t1) - t0);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave index as a scalar: everything derived from it stays in scalar registers
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int g = lane >> 5;                    // MFMA k-group of this lane
  const int head0 = hk * G;                   // first query head of the group
  const int myhead = w * kHeadsPerWave + l32;  // head within the group owned by this lane

  // 0: one launch; 1: scores, decisions, kept tiles recorded (no output);
  // 2: this workgroup's share of the sequence's kept tiles (the output)
  const int stage = a.mla_stage;
  if constexpr (PAGED) {
    // tiles of this sub-split's range past the sequence's end: not visited
    const int t_end = min(min(t0 + a.tiles_per_split, chain_t0 + a.chain_tiles), a.mask_tiles);
    if (a.mask)
      for (int t = max(t0, t0 + T) + tid; t < t_end; t += kThreads)
        a.mask[(size_t)pair * mstride + t] = 2;
  }
  if (T == 0 && !SHARE && stage == 1) {  // an empty trailing link: no tile kept, nothing published
    if (tid == 0) a.kept_bits[(size_t)pair * S + sub] = 0ull;
    return;
  }
  if (T == 0 && !SHARE && stage == 0) {  // an empty trailing link: nothing to publish, nobody waits on it
    for (int idx = tid; idx < G * kDv; idx += kThreads) {
      const size_t rowid = ((size_t)sub * a.B + b) * a.Hq + head0 + idx / kDv;
      a.part_o[rowid * kDv + idx % kDv] = 0.f;
      if (idx % kDv == 0) a.part_lse[rowid] = neg_inf();
    }
    return;
  }

  const unsigned char* kp = static_cast<const unsigned char*>(a.k) +
                           (PAGED ? 0 : (size_t)pair * a.Lk * (kDqk * 2));
  const float c = a.scale * kLog2e;
  const bool dense = log2_thr == neg_inf();
  // paged: the cache blocks of keys [t0 * 128, min((t0 + T) * 128, Lk)), block
  // ids clamped into the cache
  const int blk0 = PAGED ? (t0 * kTile) >> a.block_log2 : 0;
  if constexpr (PAGED) {
    const int nb = ((min((t0 + T) * kTile, Lk) - 1) >> a.block_log2) - blk0 + 1;
    for (int i = tid; i < nb; i += kThreads)
      s_blk[i] = min(max(a.block_table[(size_t)b * a.max_blocks + blk0 + i], 0), a.num_blocks - 1);
    __syncthreads();
  }

  // Q^T operands: lane holds head myhead, dims [16 ks + 8 g, +8) for ks < 36
  bf16x8_t qf[kQk];
  {
    const unsigned short* qp =
        static_cast<const unsigned short*>(a.q) + ((size_t)b * a.Hq + head0 + myhead) * kDqk;
#pragma unroll
    for (int ks = 0; ks < kQk; ++ks)
      qf[ks] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(qp + ks * 16 + g * 8));
    // Q has landed before the ring starts: the compiler's waits for these
    // loads would otherwise also count (and wait for) the ring's loads
    wait_vmcnt<0>();
  }

  auto slot = [&](auto I) __attribute__((always_inline)) -> unsigned char* {
    constexpr int i = decltype(I)::value % 3;
    if constexpr (i == 0) return slot0;
    else if constexpr (i == 1) return slot1;
    else return slot2;
  };

  auto issue = [&](int tile, int st, unsigned char* dst) __attribute__((always_inline)) {
    // a step that starts past Lk (tail tile) reads the last key row throughout
    const int key0 = min(tile * kTile + st * kStepKeys, Lk - 1);
    const int rlast = Lk - 1 - key0;  // last valid row of this step (>= 0)
    const unsigned char* src;
    if constexpr (PAGED) {
      // the step's rows are consecutive rows of one cache block
      const int blk = s_blk[(key0 >> a.block_log2) - blk0];
      const size_t r = (((size_t)blk * a.Hkv + hk) << a.block_log2) +
                       (key0 & ((1 << a.block_log2) - 1));
      src = kp + r * (kDqk * 2);
    } else {
      src = kp + (size_t)key0 * (kDqk * 2);
    }
    const int ln = lane_id_fresh();
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int ui = i * NW;  // compile-time part of the unit
      int row, col_byte, dst_off;
      if (ui < 32) {
        const int cb = ui / 8;
        row = 4 * (ui % 8 + w) + (ln >> 4);
        const int lc = (ln & 15) ^ swz256(row);
        col_byte = cb * 256 + lc * 16;
        dst_off = cb * kBlkBytes + (ui % 8 + w) * 1024;
      } else {
        const int up = ui - 32 + w;
        row = 8 * up + (ln >> 3);
        const int lc = (ln & 7) ^ swz128(row);
        col_byte = 1024 + lc * 16;
        dst_off = kRopeOff + up * 1024;
      }
      const unsigned ro = (unsigned)min(row, rlast) * (kDqk * 2) + col_byte;
      dma16(src, ro, dst + dst_off);
    }
  };

  // Per-lane LDS offsets of the score operand reads (row l32; k-step ks reads
  // logical chunk 2 (ks % 8) + g of block ks / 8, or chunk 2 (ks - 32) + g of
  // the 128-byte block): the block is an immediate offset.
  int koff[8], koff4[4];
#pragma unroll
  for (int k8 = 0; k8 < 8; ++k8) koff[k8] = l32 * 256 + (((2 * k8 + g) ^ swz256(l32)) << 4);
#pragma unroll
  for (int k4 = 0; k4 < 4; ++k4)
    koff4[k4] = kRopeOff + l32 * 128 + (((2 * k4 + g) ^ swz128(l32)) << 4);
  // ... of the value transpose reads.  Value block vb (columns 32 vb ..),
  // 16-key k-step t, half hi: lane l reads row 16 t + 8 hi + 4 g + (l & 15) / 4,
  // 8 bytes at column 32 vb + 16 ((l >> 4) & 1) + 4 (l & 3).  The swizzle of
  // that row does not depend on t, and vb % 4 enters only through chunk
  // bits 2..3 (XORed with the row's), so 8 offsets (hi, vb % 4) cover every
  // read.
  int voff[2][4];
  {
    const int r16 = lane & 15;
    const int x = 2 * ((lane >> 4) & 1) + ((r16 & 3) >> 1);  // chunk bits 0..1
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) {
      const int row = 8 * hi + 4 * g + (r16 >> 2);
      const int sw = swz256(row);
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4)
        voff[hi][v4] = row * 256 + (((4 * v4 + x) ^ sw) << 4) + (r16 & 1) * 8;
    }
  }

  // S^T = K Q^T over one step, two accumulation chains (even and odd
  // k-steps) so that consecutive MFMAs are independent.  Operand reads run
  // kPre k-steps ahead of their MFMA; the scheduling barriers keep that order.
  // Lane l ends up with head l32, keys 8 j + 4 g + r in element 4 j + r.
  auto scores = [&](const unsigned char* sl) __attribute__((always_inline)) -> f32x16_t {
    constexpr int kPre = 4;
    auto read = [&](int ks) __attribute__((always_inline)) {
      const int off = ks < 32 ? (ks / 8) * kBlkBytes + koff[ks % 8] : koff4[ks - 32];
      return *reinterpret_cast<const u32x4_t*>(sl + off);
    };
    u32x4_t kv[kPre];
#pragma unroll
    for (int p = 0; p < kPre; ++p) kv[p] = read(p);
    f32x16_t acc[2];
#pragma unroll
    for (int ks = 0; ks < kQk; ++ks) {
      const u32x4_t cur = kv[ks % kPre];
      if (ks + kPre < kQk) kv[ks % kPre] = read(ks + kPre);
      __builtin_amdgcn_sched_barrier(0);
      if (ks < 2)
        mfma_vgpr_first(acc[ks & 1], cur, qf[ks]);
      else
        mfma_vgpr(acc[ks & 1], cur, qf[ks]);
      __builtin_amdgcn_sched_barrier(0);
    }
    mfma_vgpr_drain(acc[0], acc[1]);
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[0][i] += acc[1][i];
    return acc[0];
  };

  // raw scores of keys past Lk -> -inf (only the tail step of a sequence;
  // the lane's key offset is computed there, not kept live across the loop)
  auto mask_tail = [&](f32x16_t& s, int key0) __attribute__((always_inline)) {
    if (key0 + kStepKeys > Lk) {
      const int k0 = key0 + 4 * (lane_id_fresh() >> 5);
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (k0 + 8 * (i >> 2) + (i & 3) >= Lk) s[i] = neg_inf();
    }
  };

  // the head's max over the step in log2 units (c > 0 keeps the order)
  auto head_max = [&](const f32x16_t& s) __attribute__((always_inline)) {
    float m = neg_inf();
#pragma unroll
    for (int i = 0; i < 16; ++i) m = fmaxf(m, s[i]);
    return max_xor32(m) * c;  // lanes l and l ^ 32 hold the same head
  };

  // O^T accumulators: block vb holds value columns 32 vb + 8 j + 4 g + r of head l32
  f32x16_t oacc[kVb];
#pragma unroll
  for (int vb = 0; vb < kVb; ++vb)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[vb][i] = 0.f;
  float lpart = 0.f;  // this lane's share of the head's denominator

  // p = exp2(s c - mref) from raw scores s, lpart += bf16(p), then O^T += V^T P^T
  // over the step's keys
  auto accumulate = [&](const f32x16_t& s, float mref, const unsigned char* sl)
                        __attribute__((always_inline)) {
    // O^T += V^T P^T: 32 MFMAs (k-step t, value block vb); the two transpose
    // reads of each run kPre MFMAs ahead, the first ones under the exponentials
    constexpr int kPre = 4;
    auto read = [&](int n) __attribute__((always_inline)) {
      const int t = n / kVb, vb = n % kVb;
      const unsigned char* base = sl + (vb / 4) * kBlkBytes + t * 16 * 256;
      const s16x4_t lo =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(base + voff[0][vb % 4]));
      const s16x4_t hi =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(base + voff[1][vb % 4]));
      const u32x2_t l2 = __builtin_bit_cast(u32x2_t, lo);
      const u32x2_t h2 = __builtin_bit_cast(u32x2_t, hi);
      return u32x4_t{l2[0], l2[1], h2[0], h2[1]};
    };
    u32x4_t vv[kPre];
#pragma unroll
    for (int p = 0; p < kPre; ++p) vv[p] = read(p);
    __builtin_amdgcn_sched_barrier(0);
    bf16x8_t pb[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      unsigned pw[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p0 = fast_exp2(fmaf(s[8 * t + 2 * e], c, -mref));
        const float p1 = fast_exp2(fmaf(s[8 * t + 2 * e + 1], c, -mref));
        pw[e] = pack_bf16x2(p0, p1);
        lpart = add_bf16x2(pw[e], lpart);
      }
      pb[t] = as_bf16x8(u32x4_t{pw[0], pw[1], pw[2], pw[3]});
    }
#pragma unroll
    for (int n = 0; n < 2 * kVb; ++n) {
      const u32x4_t cur = vv[n % kPre];
      if (n + kPre < 2 * kVb) vv[n % kPre] = read(n + kPre);
      __builtin_amdgcn_sched_barrier(0);
      oacc[n % kVb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(cur), pb[n / kVb],
                                                             oacc[n % kVb], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Run `nsteps` ring steps; step e covers keys 32 (e % 4) .. of tile
  // tile_of(e / 4).  Every step issues the loads of the step two ahead (past
  // the end: the last step again); the loop is unrolled by three so every
  // step names its slot at compile time.  The waits, barriers and loads of
  // the three steps run unconditionally (steps past the end, up to the next
  // multiple of three, load and compute nothing new), so the loads in flight
  // at every wait are the same on every path: this step's and the next one's.
  // stop() is read after each step's barrier (so it may read LDS written in
  // the step before) and ends the pass early, uniformly over the workgroup.
  auto pipeline = [&](int nsteps, auto&& tile_of, auto&& body, auto&& stop)
                      __attribute__((always_inline)) {
    auto load = [&](int e, unsigned char* dst) __attribute__((always_inline)) {
      const int ec = min(e, nsteps - 1);
      issue(tile_of(ec >> 2), ec & 3, dst);
    };
    load(0, slot0);
    load(1, slot1);
    bool done = false;
    for (int e0 = 0; e0 < nsteps && !done; e0 += 3) {
      static_for<3>([&](auto I) __attribute__((always_inline)) {
        constexpr int i = decltype(I)::value;
        const int e = e0 + i;
        wait_vmcnt<LPW>();  // this step's loads have landed, the next one's may not
        lds_barrier();      // everyone's have, and everyone is done with step e - 1
        if (!done && stop()) done = true;
        load(e + 2, slot(std::integral_constant<int, i + 2>{}));
        if (!done && e < nsteps) body(slot(I), tile_of(e >> 2), e & 3);
      });
    }
    wait_vmcnt<0>();
    __syncthreads();
  };
  auto never = []() __attribute__((always_inline)) { return false; };

  const unsigned tag = a.lb_tag;
  const size_t lbslot = (size_t)pair * S + sub;
  float mref = neg_inf();  // exponent reference of head myhead (log2 units)
  int nkept = T;

  if constexpr (MODE == kModeStream) {
    // ---------------------------------------------------------- stream pass
    // The sub-split is a whole chain.  Steps, in the order they run:
    //   K(u, 0..3)  tile u's four score steps; K(u, 3) decides tile u from
    //               every head's tile max against its running max and folds
    //               the tile max into it
    //   R(u, 0..3)  only for a kept tile u, right after K(u + 1, 2): the tile
    //               is read again (from the last-level cache: it came from
    //               HBM four to seven steps earlier), scored, exponentiated
    //               and multiplied by V
    //   after the last tile: three empty steps, then its R steps if kept.
    // Loads run three steps ahead in a four-slot ring, so the step after
    // K(u + 1, 2) is issued at the barrier of K(u + 1, 0): the first point
    // at which every wave can read tile u's decision, written to LDS (one
    // value per wave, the max over its heads) in K(u, 3).
    constexpr int kRing = 4;
    constexpr int kAhead = kRing - 1;
    static_assert(kStepsPerTile == kRing, "a round of steps starts at slot 0");
    __shared__ __attribute__((aligned(1024))) unsigned char ring[kRing * kStepBytes];
    __shared__ float s_dmax[2][NW];  // per tile parity: each wave's max statistic
    enum : int { kStepK = 0, kStepR = 1, kStepNop = 2, kStepEnd = 3 };
    // step descriptor: kind | st << 2 | (tile - t0) << 4 (loads only)

    // The step sequence, produced kAhead steps before each step runs; all
    // waves produce the same sequence (scalar state, the decision read from
    // LDS made scalar).  kept_bits collects the decisions (T <= 64).
    int gu = 0, gj = 0, gkept = 0;
    unsigned long long kept_bits = 0;
    auto next_step = [&]() __attribute__((always_inline)) -> int {
      if (gu > T) return kStepEnd;
      if (gj < 3) {
        const int d = gu < T ? (kStepK | (gj << 2) | (gu << 4)) : kStepNop;
        ++gj;
        return d;
      }
      if (gj == 3 && gu >= 1) {
        float dm = s_dmax[(gu - 1) & 1][0];
#pragma unroll
        for (int j = 1; j < NW; ++j) dm = fmaxf(dm, s_dmax[(gu - 1) & 1][j]);
        gkept = __builtin_amdgcn_readfirstlane(!(dm < log2_thr) ? 1 : 0);
        if (gkept) kept_bits |= 1ull << (gu - 1);
      } else if (gj == 3) {
        gkept = 0;
      }
      if (gkept && gj < 7) {
        const int d = kStepR | ((gj - 3) << 2) | ((gu - 1) << 4);
        ++gj;
        return d;
      }
      const int d = gu < T ? (kStepK | (3 << 2) | (gu << 4)) : kStepEnd;
      ++gu;
      gj = 0;
      return d;
    };
    auto load_step = [&](int d, int slot_i) __attribute__((always_inline)) {
      // empty and end steps load the last step again (from L2), so every
      // step issues the same loads and the waits below count them alike
      const bool real = (d & 3) < kStepNop;
      issue(t0 + (real ? d >> 4 : T - 1), real ? (d >> 2) & 3 : kStepsPerTile - 1,
            ring + slot_i * kStepBytes);
    };

    float mrun = neg_inf();  // running max of head myhead over the decided tiles (log2 units)
    float tmax = neg_inf();  // its max over the current tile's score steps
    auto score_step = [&](const unsigned char* sl, int u, int st) __attribute__((always_inline)) {
      f32x16_t s = scores(sl);
      mask_tail(s, (t0 + u) * kTile + st * kStepKeys);
      tmax = fmaxf(tmax, head_max(s));
      if (st == kStepsPerTile - 1) {
        float dh = neg_inf();
        if (tmax != neg_inf()) dh = mrun == neg_inf() ? pos_inf() : tmax - mrun;
        mrun = fmaxf(mrun, tmax);
        tmax = neg_inf();
        dh = wave_max(dh);
        if (lane == 0) s_dmax[u & 1][w] = dh;
      }
    };
    auto reread_step = [&](const unsigned char* sl, int u, int st) __attribute__((always_inline)) {
      f32x16_t s = scores(sl);
      mask_tail(s, (t0 + u) * kTile + st * kStepKeys);
      accumulate(s, mref == neg_inf() ? 0.f : mref, sl);
    };

    // One ring step at slot I: wait for its loads, barrier, issue the loads
    // of the step kAhead later, run it.  The slot's offset is hidden from the
    // optimiser: as a constant, every slot's lane addresses would be hoisted
    // out of the loop, four sets of them live at once.
    auto step = [&](auto I, auto&& run) __attribute__((always_inline)) {
      constexpr int i = decltype(I)::value;
      wait_vmcnt<(kAhead - 1) * LPW>();  // this step's loads have landed
      lds_barrier();  // everyone's have, and everyone is done with the step before
      load_step(next_step(), (i + kAhead) % kRing);
      int off = i * kStepBytes;
      asm volatile("" : "+s"(off));
      run(ring + off);
    };
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using S2 = std::integral_constant<int, 2>;
    using S3 = std::integral_constant<int, 3>;

    // The exponent reference of a head is its running max at the first kept
    // tile (tile 0); p = exp2(s - mref) then stays below 2^kRefMargin while
    // the running max (which bounds every kept score) stays within that
    // margin of it.  A head whose running max climbs
    // further sets s_restart: the pass runs again with every head's max over
    // the chain as its reference (same decisions, no p above 1).
    for (bool preset = false;; preset = true) {
      if (tid == 0) s_restart = 0;
#pragma unroll
      for (int vb = 0; vb < kVb; ++vb)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[vb][i] = 0.f;
      lpart = 0.f;
      gu = gj = gkept = 0;
      kept_bits = 0;
      mrun = tmax = neg_inf();
      __syncthreads();
      load_step(next_step(), 0);
      load_step(next_step(), 1);
      load_step(next_step(), 2);
      // Round u (u <= T) runs K(u, 0..2) (empty steps for u = T), then R(u - 1,
      // 0..3) if tile u - 1 was kept, then K(u, 3) (u < T).  A round takes 4 or
      // 8 steps, so it always starts at slot 0.
      for (int u = 0; u <= T; ++u) {
        const bool real = u < T;
        step(S0{}, [&](const unsigned char* sl) __attribute__((always_inline)) {
          if (real) score_step(sl, u, 0);
        });
        step(S1{}, [&](const unsigned char* sl) __attribute__((always_inline)) {
          if (real) score_step(sl, u, 1);
        });
        step(S2{}, [&](const unsigned char* sl) __attribute__((always_inline)) {
          if (real) score_step(sl, u, 2);
        });
        // gkept: tile u - 1's decision, read by next_step at the barrier of
        // this round's first step
        if (gkept) {
          if (!preset && mref == neg_inf()) mref = mrun;
          if (__builtin_amdgcn_ballot_w64(mrun > mref + kRefMargin) != 0 && lane == 0)
            s_restart = 1;
          step(S3{}, [&](const unsigned char* sl) __attribute__((always_inline)) {
            reread_step(sl, u - 1, 0);
          });
          step(S0{}, [&](const unsigned char* sl) __attribute__((always_inline)) {
            reread_step(sl, u - 1, 1);
          });
          step(S1{}, [&](const unsigned char* sl) __attribute__((always_inline)) {
            reread_step(sl, u - 1, 2);
          });
          step(S2{}, [&](const unsigned char* sl) __attribute__((always_inline)) {
            reread_step(sl, u - 1, 3);
          });
        }
        if (real)
          step(S3{}, [&](const unsigned char* sl) __attribute__((always_inline)) {
            score_step(sl, u, 3);
          });
      }
      wait_vmcnt<0>();
      __syncthreads();
      if (s_restart == 0) break;
      mref = mrun;      // the head's max over the chain
      __syncthreads();  // everyone has read s_restart before it is cleared
    }
    if (a.mask && tid < T) a.mask[(size_t)pair * mstride + t0 + tid] = (kept_bits >> tid) & 1ull ? 0 : 1;
  } else {
  if constexpr (SHARE) {
    // the share the planning launch gave this workgroup
    const size_t us = (size_t)pair * S + sub;
    if (tid == 0) s_nsurv = a.share_count[us];
    if (tid < kTmax) s_surv[tid] = a.share_tiles[us * kTmax + tid];
    if (tid < G) s_mref[tid] = a.share_mref[(size_t)b * a.Hq + head0 + tid];
    __syncthreads();
  } else if (!dense) {
    // ---------------------------------------------------------- 1. score pass
    float tmax = neg_inf();
    pipeline(kStepsPerTile * T, [&](int t) __attribute__((always_inline)) { return t0 + t; },
             [&](const unsigned char* sl, int tile, int st) __attribute__((always_inline)) {
               f32x16_t s = scores(sl);
               mask_tail(s, tile * kTile + st * kStepKeys);
               tmax = fmaxf(tmax, head_max(s));
               if (st == kStepsPerTile - 1) {
                 if (g == 0) tmaxs[(tile - t0) * G + myhead] = tmax;
                 tmax = neg_inf();
               }
             },
             never);

    // ---------------------------------------------------------- 2. decision
    // thread (part, h): head h, tiles / earlier links of parity `part`
    const int h = tid % G, part = tid / G;  // part in {0, 1}
    float cm = neg_inf();
    for (int t = part; t < T; t += 2) cm = fmaxf(cm, tmaxs[t * G + h]);
    part_red[part][h] = cm;
    __syncthreads();
    cm = fmaxf(part_red[0][h], part_red[1][h]);
    if (part == 0) {
      s_mref[h] = cm;
      if (a.subs_per_chain > 1 || stage == 1)
        __hip_atomic_store(&a.lb_slot[lbslot * G + h], tagged(tag, cm), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
    // earlier links of the chain: eight reads in flight at a time (by then
    // the earlier links have usually published), a poll only for a value
    // not yet published
    float pv = neg_inf();
    const size_t chain_slot0 = (size_t)pair * S + (sub - link);
    for (int lk0 = part; lk0 < link; lk0 += 16) {
      unsigned long long v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int lk = lk0 + 2 * j;
        v[j] = lk < link ? __hip_atomic_load(&a.lb_slot[(chain_slot0 + lk) * G + h],
                                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                         : tagged(tag, neg_inf());
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int lk = lk0 + 2 * j;
        const float x = (v[j] >> 32) == tag
                            ? __uint_as_float((unsigned)v[j])
                            : poll_tagged(&a.lb_slot[(chain_slot0 + lk) * G + h], tag,
                                          a.lb_timeouts);
        pv = fmaxf(pv, x);
      }
    }
    __syncthreads();  // part_red reads above are done
    part_red[part][h] = pv;
    __syncthreads();
    if (part == 0) {
      // running max before each tile, and each tile's statistic for head h
      // (written over its tile max)
      float M = fmaxf(part_red[0][h], part_red[1][h]);
      for (int t = 0; t < T; ++t) {
        const float tm = tmaxs[t * G + h];
        float d = neg_inf();
        if (tm != neg_inf()) d = (M == neg_inf()) ? pos_inf() : tm - M;
        tmaxs[t * G + h] = d;
        M = fmaxf(M, tm);
      }
    }
    __syncthreads();
    // max over heads per tile: wave w reduces the tiles t = w (mod NW)
    for (int t = w; t < T; t += NW) {
      float d = neg_inf();
#pragma unroll
      for (int j = 0; j < G / 64; ++j) d = fmaxf(d, tmaxs[t * G + j * 64 + lane]);
      d = wave_max(d);
      if (lane == 0) s_dtile[t] = d;
    }
    __syncthreads();
    if (w == 0) {
      const bool valid = lane < T;
      const float d = valid ? s_dtile[lane] : neg_inf();
      const bool kept = valid && !(d < log2_thr);
      const unsigned long long bits = __ballot(kept);
      const int idx = __popcll(bits & ((1ull << lane) - 1ull));
      if (kept) s_surv[idx] = t0 + lane;
      if (lane == 0) s_nsurv = __popcll(bits);
      if (lane == 0 && stage == 1) a.kept_bits[(size_t)pair * S + sub] = bits;
      if (valid && a.mask) a.mask[(size_t)pair * mstride + t0 + lane] = kept ? 0 : 1;
    }
    __syncthreads();
    if (stage == 1) return;  // the planning launch and stage 2 run the kept tiles
  }
  if (SHARE || !dense) {
    nkept = s_nsurv;
    mref = s_mref[myhead];

    // ---------------------------------------------------------- 3. kept tiles
    // (s_surv: absolute tile indices)
    if (nkept > 0) {
      const float mr = mref == neg_inf() ? 0.f : mref;
      pipeline(kStepsPerTile * nkept,
               [&](int t) __attribute__((always_inline)) { return s_surv[t]; },
               [&](const unsigned char* sl, int tile, int st) __attribute__((always_inline)) {
                 f32x16_t s = scores(sl);
                 mask_tail(s, tile * kTile + st * kStepKeys);
                 accumulate(s, mr, sl);
               },
               never);
    }
  } else {
    // ---------------------------------------------------------- online pass
    // The exponent reference of each head is its max over the first step;
    // p = exp2(s - mref) may reach 2^kRefMargin.  When some head's scores
    // rise further above it, the pass starts over with every head's running
    // max as its reference (rewriting the accumulators in place would cost a
    // copy of all 256 of them through the vector ALU; with a reference 2^8
    // wide, keys whose scores are i.i.d. Gumbel made every long pass start
    // over, 456 against 279 us at 131072 keys).
    if (a.mask)
      for (int t = tid; t < T; t += kThreads) a.mask[(size_t)pair * mstride + t0 + t] = 0;
    float mrun = neg_inf();  // running max of head myhead over the steps seen
    for (;;) {
#pragma unroll
      for (int vb = 0; vb < kVb; ++vb)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[vb][i] = 0.f;
      lpart = 0.f;
      if (tid == 0) s_restart = 0;
      __syncthreads();
      pipeline(kStepsPerTile * T, [&](int t) __attribute__((always_inline)) { return t0 + t; },
               [&](const unsigned char* sl, int tile, int st) __attribute__((always_inline)) {
                 f32x16_t s = scores(sl);
                 mask_tail(s, tile * kTile + st * kStepKeys);
                 const float sm = head_max(s);
                 mrun = fmaxf(mrun, sm);
                 if (mref == neg_inf()) mref = sm;  // first step (always has a valid key)
                 if (__builtin_amdgcn_ballot_w64(sm > mref + kRefMargin) != 0) {
                   if (lane == 0) s_restart = 1;
                 } else {
                   accumulate(s, mref, sl);
                 }
               },
               [&]() __attribute__((always_inline)) { return s_restart != 0; });
      if (s_restart == 0) break;
      mref = mrun;
      __syncthreads();  // everyone has read s_restart
    }
  }
  }

  // ------------------------------------------------------------ write O / l and lse
  const float l = sum_xor32(lpart);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const size_t rowid = ((size_t)sub * a.B + b) * a.Hq + head0 + myhead;
  float* op = a.part_o + rowid * kDv;
#pragma unroll
  for (int vb = 0; vb < kVb; ++vb)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<f32x4_t*>(op + vb * 32 + j * 8 + g * 4) =
          f32x4_t{oacc[vb][4 * j] * inv, oacc[vb][4 * j + 1] * inv, oacc[vb][4 * j + 2] * inv,
                  oacc[vb][4 * j + 3] * inv};
  if (g == 0) a.part_lse[rowid] = l > 0.f ? (mref + __log2f(l)) * kLn2 : neg_inf();
}

// Planning launch of a thresholded decode: one workgroup per sequence (batch,
// latent head).  Its kept tiles, in (sub-split, tile) order, are numbered
// 0 .. K-1; workgroup o of stage 2 takes ranks [o K / S, (o + 1) K / S)
// (at most 64, since no sub-split holds more than 64 tiles).  The heads'
// exponent reference is their max over the whole sequence: the maxima every
// non-empty sub-split published in stage 1.
__global__ __launch_bounds__(256) void decode_mla_plan_kernel(DecodeArgs a) {
  const int S = a.num_splits;
  const int pair = blockIdx.x;  // b * Hkv + hk
  const int b = pair / a.Hkv, hk = pair % a.Hkv;
  const int G = a.Hq / a.Hkv;
  const int nK = (a.Lk + kTile - 1) / kTile;
  const int tid = threadIdx.x;
  __shared__ int s_base[1024];  // exclusive prefix of the kept counts (S <= 1024)
  __shared__ int s_total;
  auto first_tile = [&](int s2) {
    const int c2 = s2 / a.subs_per_chain, k2 = s2 % a.subs_per_chain;
    return c2 * a.chain_tiles + k2 * a.tiles_per_split;
  };
  auto tiles_of = [&](int s2) {
    const int c2 = s2 / a.subs_per_chain;
    const int a0 = first_tile(s2);
    return max(0, min(a0 + a.tiles_per_split, min(c2 * a.chain_tiles + a.chain_tiles, nK)) - a0);
  };
  const unsigned long long* bits = a.kept_bits + (size_t)pair * S;
  // Stage 1 has finished before this launch, so every non-empty sub-split's
  // published maxima and kept tiles are in memory: plain loads, all issued
  // together, no polling.  A value without this launch's tag where a
  // sub-split had tiles would be a lost publish; it is counted with the
  // look-back timeouts and left out of the max.
  __shared__ float s_part[256];
  // this thread's kept masks first (sub-splits 4t .. 4t+3; past S the last
  // again, not used), so their loads overlap those of the maxima
  unsigned long long kw[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) kw[i] = bits[min(4 * tid + i, S - 1)];
  {
    const int per = 256 / G;  // threads per head
    const int h = tid % G;
    float m = neg_inf();
    unsigned bad = 0;
#pragma unroll 16
    for (int s2 = tid / G; s2 < S; s2 += per) {
      const unsigned long long v = a.lb_slot[((size_t)pair * S + s2) * G + h];
      const bool use = tiles_of(s2) > 0;
      const bool fresh = (unsigned)(v >> 32) == a.lb_tag;
      m = use && fresh ? fmaxf(m, __uint_as_float((unsigned)v)) : m;
      bad += use && !fresh;
    }
    if (bad) atomicAdd(a.lb_timeouts, bad);
    s_part[tid] = m;
  }
  // kept counts: thread t holds sub-splits 4t .. 4t+3; exclusive scan over
  // the 256 threads' sums in LDS
  __shared__ int s_scan[2][256];
  __shared__ unsigned long long s_bits[1024];
  int cnt[4], own = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int s2 = 4 * tid + i;
    cnt[i] = s2 < S ? __popcll(kw[i]) : 0;
    own += cnt[i];
    if (s2 < S) s_bits[s2] = kw[i];
  }
  s_scan[0][tid] = own;
  __syncthreads();
  if (tid < G) {
    float m = s_part[tid];
    for (int p2 = 1; p2 < 256 / G; ++p2) m = fmaxf(m, s_part[p2 * G + tid]);
    a.share_mref[(size_t)b * a.Hq + hk * G + tid] = m;
  }
  int src = 0;
#pragma unroll
  for (int d = 1; d < 256; d <<= 1) {
    const int v = s_scan[src][tid] + (tid >= d ? s_scan[src][tid - d] : 0);
    s_scan[src ^ 1][tid] = v;
    src ^= 1;
    __syncthreads();
  }
  {
    int run = s_scan[src][tid] - own;  // exclusive
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int s2 = 4 * tid + i;
      if (s2 < S) s_base[s2] = run;
      run += cnt[i];
    }
    if (tid == 255) s_total = s_scan[src][255];
  }
  __syncthreads();
  // Products of a rank or a count with S stay below 64 S^2 <= 2^26: 32-bit.
  const int K = s_total;
  for (int o = tid; o < S; o += 256)
    a.share_count[(size_t)pair * S + o] = ((o + 1) * K) / S - (o * K) / S;
  // one thread per (sub-split, tile) position: a kept tile's rank is its
  // sub-split's base plus the kept tiles before it in the mask
  for (int g = tid; g < S * kTmax; g += 256) {
    const int s2 = g / kTmax, t = g % kTmax;
    const unsigned long long m = s_bits[s2];
    if (!((m >> t) & 1ull)) continue;
    const int r = s_base[s2] + __popcll(m & ((1ull << t) - 1ull));
    const int o = ((r + 1) * S - 1) / K;  // the workgroup whose range holds rank r
    const int pos = r - (o * K) / S;
    a.share_tiles[((size_t)pair * S + o) * kTmax + pos] = first_tile(s2) + t;
  }
}

}  // namespace

bool decode_mla_supported(int D, int Dv, int group, bool latent) {
  return latent && D == kDqk && Dv == kDv && (group == 64 || group == 128);
}

int decode_mla_max_tiles(int) { return kTmax; }

int decode_mla_workgroups_per_split(int) { return 1; }

// A threshold and sub-splits that are whole chains: one launch in stream
// mode.  Threshold 0, or few tiles per sub-split: one launch.  Otherwise three on
// the same stream: stage 1 scores every tile and decides (each sub-split
// publishes its per-head maxima and its kept tiles), the planning launch
// spreads each sequence's kept tiles evenly over its workgroups, stage 2 runs
// them.  With chained decisions the
// first sub-splits of a sequence keep most of their tiles (the running max is
// still low there), so if each ran its own kept tiles the whole launch would
// wait on them.
hipError_t launch_decode_mla(const DecodeArgs& args, hipStream_t s) {
  const int G = args.Hq / args.Hkv;
  if (G != 128 && G != 64) return hipErrorInvalidValue;
  if (args.num_splits > 1024) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((size_t)args.num_splits * args.B * args.Hkv));
  DecodeArgs a = args;
  // The share-out pays where a sub-split holds many tiles: chained decisions
  // then leave the first sub-splits of a sequence with most of theirs and
  // the rest with few.  With few tiles per sub-split that imbalance is small
  // and the two extra launches and the second pass's start-up cost more than
  // they save; one launch then scores, decides and runs each sub-split's own
  // kept tiles (on 8 sequences of 16K / 32K keys, 4 / 8 tiles per
  // sub-split: 100 / 150 us in one launch, 121 / 164 us shared out; of
  // 64K / 128K keys, 16 / 32 tiles: 256 / 456 us against 229 / 365 us).
  const bool thresholded = a.log2_thr != -__builtin_inff();
  if (thresholded && a.subs_per_chain == 1 && a.tiles_per_split <= kTmax) {
    // every sub-split is a whole chain: one streaming pass, no look-back
    a.mla_stage = 0;
    if (G == 128)
      hipLaunchKernelGGL((decode_mla_kernel<4, kModeStream>), grid, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((decode_mla_kernel<2, kModeStream>), grid, dim3(128), 0, s, a);
    return hipGetLastError();
  }
  const bool share = a.tiles_per_split >= kShareMinTiles;
  if (!thresholded || !share) {
    a.mla_stage = 0;
    if (G == 128)
      hipLaunchKernelGGL((decode_mla_kernel<4, kModeSplit>), grid, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((decode_mla_kernel<2, kModeSplit>), grid, dim3(128), 0, s, a);
    return hipGetLastError();
  }
  a.mla_stage = 1;
  if (G == 128)
    hipLaunchKernelGGL((decode_mla_kernel<4, kModeSplit>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((decode_mla_kernel<2, kModeSplit>), grid, dim3(128), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_mla_plan_kernel, dim3((unsigned)(args.B * args.Hkv)), dim3(256), 0, s,
                     a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  a.mla_stage = 2;
  if (G == 128)
    hipLaunchKernelGGL((decode_mla_kernel<4, kModeShare>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((decode_mla_kernel<2, kModeShare>), grid, dim3(128), 0, s, a);
  return hipGetLastError();
}

// Paged, variable-length latent decode: one launch (chained sub-splits score,
// decide and run their own kept tiles; each sequence its own length and
// threshold), then the merge.
hipError_t launch_decode_mla_paged(const DecodeArgs& args, hipStream_t s) {
  const int G = args.Hq / args.Hkv;
  if (G != 128 && G != 64) return hipErrorInvalidValue;
  if (args.block_log2 < 5 || args.block_log2 > 7) return hipErrorInvalidValue;
  if (args.tiles_per_split > kTmax) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((size_t)args.num_splits * args.B * args.Hkv));
  DecodeArgs a = args;
  a.mla_stage = 0;
  if (G == 128)
    hipLaunchKernelGGL((decode_mla_kernel<4, kModeSplit, true>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((decode_mla_kernel<2, kModeSplit, true>), grid, dim3(128), 0, s, a);
  return hipGetLastError();
}
}  // namespace ssattn
