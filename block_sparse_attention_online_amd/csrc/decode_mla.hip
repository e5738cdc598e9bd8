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
// Work split: one workgroup per (batch, sub-split of at most 64 tiles, half of
// the head group); a half is 64 query heads.  4 waves; wave w owns heads
// [16 w, 16 w + 16) of the half and the whole 128-key tile, so each wave has
// full tiles for its heads: tile maxima, exponentials and P stay in its
// registers.  MFMA v_mfma_f32_16x16x32_bf16 throughout; Q stays in registers
// as the B operand for the whole call.
//
// Tiles move through a three-slot LDS ring (direct global -> LDS loads,
// 16-byte chunks swizzled by row so the operand reads are conflict free).
//
//  1. Score pass (thresholds > 0 only), 6 steps of 96 columns per tile:
//     S^T = K Q^T for every tile of the sub-split; each head's tile max goes
//     to an LDS table.
//  2. Decision: each half publishes its heads' maxima for later sub-splits of
//     its chain and folds in those of the earlier ones (the look-back of the
//     GQA decode), computes its heads' part of every tile's statistic
//     max_r (tile_max - running_max), and exchanges it with the other half, so
//     both halves take the same decision for the whole group.
//  3. Kept tiles, 9 steps of [128 keys x 128 columns] per tile: 5 score steps
//     (columns 0..511, then the 64 rope columns), p = exp2(s - m) with m the
//     sub-split's own per-head max (no rescaling), then 4 value steps that
//     reload columns 0..511 (from L2: the score steps have just read them),
//     O^T += V^T P^T with V^T from ds_read_b64_tr_b16 transpose reads.
// With threshold 0 nothing can be skipped: phases 1 and 2 are left out and
// phase 3 runs over every tile as an online pass (running max, rescale when
// it grows).
//
// The split's O / l and lse go to the workspace; decode_combine merges splits.

#include <type_traits>
#include <utility>

#include "device_common.h"
#include "launch.h"

namespace ssattn {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kDqk = 576;              // latent key width
constexpr int kDv = 512;               // value width (leading columns of the key row)
constexpr int kHalf = 64;              // query heads per workgroup
constexpr int kTmax = 64;              // tiles per sub-split
constexpr int kSlotBytes = kTile * 256;  // [128 keys x 128 columns] bf16
constexpr int kQk = kDqk / 32;         // 18 MFMA k-steps over the key width
constexpr int kSpinCap = 1 << 21;

typedef __attribute__((ext_vector_type(4))) short s16x4_t;
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

// Physical 16-byte chunk of logical chunk c in row r of a ring step, per
// step kind, so that each kind's operand reads hit 16 different chunk
// positions (all banks) per 16 lanes:
//  * score step, 128 columns (16 chunks, 256-byte rows): 16 consecutive rows
//    read the same logical chunk -> c ^ (r & 15);
//  * score step, 64 columns (8 chunks, 128-byte rows, two rows per 256
//    bytes) -> c ^ ((r >> 1) & 7);
//  * value step (transpose reads: 4 consecutive rows x 2 adjacent chunks
//    per 16 lanes) -> c ^ ((r & 7) << 1).
__device__ __forceinline__ int swz_score128(int r) { return r & 15; }
__device__ __forceinline__ int swz_score64(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int swz_value(int r) { return (r & 7) << 1; }

// s_waitcnt with vmcnt = N and no wait on the other counters (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Workgroup barrier for the ring.  __syncthreads (and any release fence that
// covers LDS) waits for every outstanding direct-to-LDS load, which would
// leave one step in flight instead of two; this barrier waits only for the
// wave's own LDS operations (lgkmcnt), and the "memory" clobber keeps the
// compiler from moving memory accesses across it.  Direct-to-LDS loads are
// waited for explicitly (wait_vmcnt) before it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

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

template <class F, int... E>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, E...>) {
  (f(std::integral_constant<int, E>{}), ...);
}
// f(integral_constant<int, 0>), ..., f(integral_constant<int, N - 1>)
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Step plans: the columns each step of a tile brings into the ring.
struct ScorePlan {  // score pass: all 576 columns
  static constexpr int P = 6;
  static constexpr int col[P] = {0, 128, 256, 384, 448, 512};
  static constexpr int width[P] = {128, 128, 128, 64, 64, 64};
  static constexpr bool value[P] = {false, false, false, false, false, false};
};
struct KeptPlan {  // kept tile: 576 score columns, then the 512 value columns again
  static constexpr int P = 9;
  static constexpr int col[P] = {0, 128, 256, 384, 512, 0, 128, 256, 384};
  static constexpr int width[P] = {128, 128, 128, 128, 64, 128, 128, 128, 128};
  static constexpr bool value[P] = {false, false, false, false, false, true, true, true, true};
  static constexpr int kLastScore = 4;
};

template <int NHALF>
__global__ __launch_bounds__(kThreads, 1) void decode_mla_kernel(DecodeArgs a) {
  constexpr int G = NHALF * kHalf;  // heads per latent head
  __shared__ __attribute__((aligned(1024))) unsigned char slot0[kSlotBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char slot1[kSlotBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char slot2[kSlotBytes];
  __shared__ __attribute__((aligned(16))) float tmaxs[kTmax * kHalf];  // [tile][head]
  __shared__ float prevred[kWaves][kHalf];
  __shared__ float s_mref[kHalf];
  __shared__ float s_dtile[kTmax];
  __shared__ int s_surv[kTmax];
  __shared__ int s_nsurv;

  // block -> (batch, sub-split, half): sub-splits in order (every look-back
  // waits only on lower blocks); the two halves of a sub-split are 8 blocks
  // apart, on the same XCD (blocks go to XCDs round robin), so both read the
  // same tiles through one L2.
  const int S = a.num_splits;
  int half, usub;
  if (NHALF == 2) {
    const int grp16 = blockIdx.x >> 4, in16 = blockIdx.x & 15;
    half = in16 >> 3;
    usub = grp16 * 8 + (in16 & 7);
  } else {
    half = 0;
    usub = blockIdx.x;
  }
  const bool live = usub < S * a.B * a.Hkv;
  const int sub = usub % S;
  const int pair = usub / S;  // b * Hkv + hk
  const int hk = pair % a.Hkv;
  const int b = pair / a.Hkv;
  const int nK = (a.Lk + kTile - 1) / kTile;
  const int chain = sub / a.subs_per_chain;
  const int link = sub % a.subs_per_chain;
  const int chain_t0 = chain * a.chain_tiles;
  const int chain_t1 = min(chain_t0 + a.chain_tiles, nK);
  const int t0 = chain_t0 + link * a.tiles_per_split;
  const int T = live ? max(0, min(t0 + a.tiles_per_split, chain_t1) - t0) : 0;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave index as a scalar: everything derived from it (ring destinations,
  // row bases) stays in scalar registers
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15;
  const int q = lane >> 4;                   // MFMA k-group of this lane
  const int head0 = hk * G + half * kHalf;   // first query head of this half
  const int myhead = w * 16 + l16;           // head within the half owned by this lane

  if (!live) return;  // padding block of the half-interleaved grid
  if (T == 0) {       // an empty trailing link: nothing to publish, nobody waits on it
    for (int idx = tid; idx < kHalf * kDv; idx += kThreads) {
      const size_t rowid = ((size_t)sub * a.B + b) * a.Hq + head0 + idx / kDv;
      a.part_o[rowid * kDv + idx % kDv] = 0.f;
      if (idx % kDv == 0) a.part_lse[rowid] = neg_inf();
    }
    return;
  }

  const unsigned short* kp =
      static_cast<const unsigned short*>(a.k) + ((size_t)pair * a.Lk) * kDqk;
  const float c = a.scale * kLog2e;
  const bool dense = a.log2_thr == neg_inf();

  // Q^T operands: lane holds head myhead, dims 32 j + 8 q .. + 8 for j < 18
  bf16x8_t qf[kQk];
  {
    const unsigned short* qp =
        static_cast<const unsigned short*>(a.q) + ((size_t)b * a.Hq + head0 + myhead) * kDqk;
#pragma unroll
    for (int j = 0; j < kQk; ++j)
      qf[j] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(qp + j * 32 + q * 8));
    // keep these loads ahead of the ring's first loads, so waiting for Q
    // does not wait for the ring
    asm volatile("" ::: "memory");
  }

  // ---- the ring: three LDS slots.  A tile is a fixed number of steps (6 in
  // the score pass, 9 for a kept tile), a multiple of three, so step e of
  // every tile uses slot e % 3: the slot and the step kind are compile-time
  // constants, and so is every register-array index below.
  auto slot = [&](auto I) __attribute__((always_inline)) -> unsigned char* {
    constexpr int i = decltype(I)::value % 3;
    if constexpr (i == 0) return slot0;
    else if constexpr (i == 1) return slot1;
    else return slot2;
  };

  // A step holds W = 128 or 64 columns from column C of the tile's 128 keys:
  // rows of 2 W bytes, 16-byte chunks swizzled by the step kind's rule above.
  // Wave w loads rows [32 w, 32 w + 32), 1024 bytes per instruction.  Keys
  // past Lk read the last key row (their scores are masked, their p is 0).
  auto issue = [&](auto C_, auto W_, auto V_, int tile, unsigned char* dst)
                   __attribute__((always_inline)) {
    constexpr int C = decltype(C_)::value, W = decltype(W_)::value;
    constexpr bool V = decltype(V_)::value;
    constexpr int CPR = W / 8;         // chunks per row
    constexpr int RPI = 64 / CPR;      // rows per instruction
    constexpr int NI = 32 / RPI;       // instructions per wave
    const int lr = lane / CPR, pc = lane % CPR;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int r = (w * NI + i) * RPI + lr;
      const int key = min(tile * kTile + r, a.Lk - 1);
      const int lc = pc ^ (V ? swz_value(r) : (W == 128 ? swz_score128(r) : swz_score64(r)));
      __builtin_amdgcn_global_load_lds(
          (const void __attribute__((address_space(1)))*)(kp + (size_t)key * kDqk + C + lc * 8),
          (void __attribute__((address_space(3)))*)(dst + (w * NI + i) * 1024), 16, 0, 0);
    }
  };

  // S^T blocks [16 keys x 16 heads], block kb = keys 16 kb .. of the tile;
  // lane holds head l16, keys 16 kb + 4 q + i
  f32x4_t sacc[8];
  // scores over the step's columns: k-step ks (32 columns) reads logical
  // chunk 4 ks + q of row 16 kb + l16
  auto score = [&](auto C_, auto W_, const unsigned char* sl) __attribute__((always_inline)) {
    constexpr int C = decltype(C_)::value, W = decltype(W_)::value;
    constexpr int NKS = W / 32;
    if constexpr (C == 0) {
#pragma unroll
      for (int kb = 0; kb < 8; ++kb) sacc[kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    // rows 16 kb + l16: the swizzle depends on l16 only, the row block is an
    // immediate offset
    const int sw = W == 128 ? swz_score128(l16) : swz_score64(l16);
    const unsigned char* base = sl + l16 * (2 * W);
    auto read = [&](int ks, u32x4_t (&kv)[8]) __attribute__((always_inline)) {
      const int off = ((4 * ks + q) ^ sw) << 4;
#pragma unroll
      for (int kb = 0; kb < 8; ++kb)
        kv[kb] = *reinterpret_cast<const u32x4_t*>(base + kb * 16 * (2 * W) + off);
    };
    // operands of k-step ks + 1 are read while the MFMAs of k-step ks run
    u32x4_t kv[2][8];
    read(0, kv[0]);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      if (ks + 1 < NKS) read(ks + 1, kv[(ks + 1) & 1]);
#pragma unroll
      for (int kb = 0; kb < 8; ++kb)
        sacc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kv[ks & 1][kb]),
                                                          qf[C / 32 + ks], sacc[kb], 0, 0, 0);
    }
    // schedule: the first k-step's reads, then one MFMA per read of the next
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
    for (int i = 0; i < 8 * (NKS - 1); ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
  };

  // scores of the tile in log2 units, keys past Lk at -inf; returns the tile
  // max of head myhead (every lane of the head agrees)
  auto finish_scores = [&](int tile) __attribute__((always_inline)) {
    const int kbase = tile * kTile + q * 4;
    float m = neg_inf();
#pragma unroll
    for (int kb = 0; kb < 8; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float s = sacc[kb][i] * c;
        if (kbase + kb * 16 + i >= a.Lk) s = neg_inf();
        sacc[kb][i] = s;
        m = fmaxf(m, s);
      }
    m = fmaxf(m, shfl_xor_f(m, 16));
    return fmaxf(m, shfl_xor_f(m, 32));
  };

  // Run `nt` tiles through the ring, PLAN::P steps each.  Every step issues the
  // loads of the step two ahead; past the last tile it repeats the same step
  // kind of the last tile, so the loads in flight at every wait are known:
  // this step's and the next step's.
  auto pipeline = [&](int nt, auto plan, auto&& tile_of, auto&& body) __attribute__((always_inline)) {
    using PL = decltype(plan);
    constexpr int P = PL::P;
    static_assert(P % 3 == 0, "steps per tile");
    auto load = [&](int t, auto E, unsigned char* dst) __attribute__((always_inline)) {
      constexpr int e = decltype(E)::value;
      issue(std::integral_constant<int, PL::col[e]>{}, std::integral_constant<int, PL::width[e]>{},
            std::integral_constant<bool, PL::value[e]>{}, tile_of(min(t, nt - 1)), dst);
    };
    load(0, std::integral_constant<int, 0>{}, slot0);
    load(0, std::integral_constant<int, 1>{}, slot1);
    for (int t = 0; t < nt; ++t) {
      const int tile = tile_of(t);
      static_for<P>([&](auto E) __attribute__((always_inline)) {
        constexpr int e = decltype(E)::value;
        constexpr int en = (e + 1) % P;
        wait_vmcnt<PL::width[en] / 16>();  // this step's loads have landed, the next one's may not
        lds_barrier();  // everyone's have, and everyone is done with the previous step
        constexpr int e2 = e + 2;
        if constexpr (e2 < P)
          load(t, std::integral_constant<int, e2>{}, slot(std::integral_constant<int, e2>{}));
        else
          load(t + 1, std::integral_constant<int, e2 - P>{}, slot(std::integral_constant<int, e2>{}));
        body(E, std::integral_constant<int, PL::col[e]>{},
             std::integral_constant<int, PL::width[e]>{}, tile, slot(E));
      });
    }
    wait_vmcnt<0>();
    __syncthreads();
  };

  // ------------------------------------------------------------ 1. score pass
  if (!dense) {
    pipeline(T, ScorePlan{}, [&](int t) __attribute__((always_inline)) { return t0 + t; },
             [&](auto E, auto C_, auto W_, int tile, const unsigned char* sl)
                 __attribute__((always_inline)) {
               score(C_, W_, sl);
               if constexpr (decltype(E)::value == ScorePlan::P - 1) {
                 const float m = finish_scores(tile);
                 if (q == 0) tmaxs[(tile - t0) * kHalf + myhead] = m;
               }
             });
  }

  // ------------------------------------------------------------ 2. decision
  const unsigned tag = a.lb_tag;
  const size_t lbslot = (size_t)pair * S + sub;
  if (!dense) {
    // the sub-split's own per-head max
    const int h = tid & 63;
    float cm = neg_inf();
    for (int t = tid >> 6; t < T; t += kWaves) cm = fmaxf(cm, tmaxs[t * kHalf + h]);
    prevred[w][h] = cm;
    __syncthreads();
    if (w == 0) {
      cm = fmaxf(fmaxf(prevred[0][h], prevred[1][h]), fmaxf(prevred[2][h], prevred[3][h]));
      s_mref[h] = cm;
      if (a.subs_per_chain > 1)
        __hip_atomic_store(&a.lb_slot[lbslot * G + half * kHalf + h], tagged(tag, cm),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    // earlier links of the chain: every thread polls some (link, head) pairs
    float pv = neg_inf();
    for (int lk = tid >> 6; lk < link; lk += kWaves) {
      const size_t ps = (size_t)pair * S + (sub - link) + lk;
      pv = fmaxf(pv, poll_tagged(&a.lb_slot[ps * G + half * kHalf + h], tag, a.lb_timeouts));
    }
    __syncthreads();  // the reads of prevred above are done
    prevred[w][h] = pv;
    __syncthreads();
    // every wave scans all tiles for head h and reduces over heads for the
    // tiles t = w (mod 4)
    {
      float M = fmaxf(fmaxf(prevred[0][h], prevred[1][h]), fmaxf(prevred[2][h], prevred[3][h]));
      for (int t = 0; t < T; ++t) {
        const float tm = tmaxs[t * kHalf + h];
        float d = neg_inf();
        if (tm != neg_inf()) d = (M == neg_inf()) ? pos_inf() : tm - M;
        if ((t & 3) == w) {
          d = wave_max(d);
          if (lane == 0) s_dtile[t] = d;
        }
        M = fmaxf(M, tm);
      }
    }
    __syncthreads();
    if (w == 0) {
      const bool valid = lane < T;
      float d = valid ? s_dtile[lane] : neg_inf();
      if (NHALF == 2) {  // the other half's heads
        const size_t xs = (lbslot * 2 + half) * kTmax + lane;
        const size_t xo = (lbslot * 2 + (half ^ 1)) * kTmax + lane;
        if (valid) {
          __hip_atomic_store(&a.lb_xchg[xs], tagged(tag, d), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
          d = fmaxf(d, poll_tagged(&a.lb_xchg[xo], tag, a.lb_timeouts));
        }
      }
      const bool kept = valid && !(d < a.log2_thr);
      const unsigned long long bits = __ballot(kept);
      const int idx = __popcll(bits & ((1ull << lane) - 1ull));
      if (kept) s_surv[idx] = lane;
      if (lane == 0) s_nsurv = __popcll(bits);
      if (valid && half == 0 && a.mask) a.mask[(size_t)pair * nK + t0 + lane] = kept ? 0 : 1;
    }
    __syncthreads();
  } else {
    if (half == 0 && a.mask)
      for (int t = tid; t < T; t += kThreads) a.mask[(size_t)pair * nK + t0 + t] = 0;
  }

  // ------------------------------------------------------------ 3. kept tiles
  f32x4_t oacc[32];  // O^T blocks [16 value columns x 16 heads]: columns 16 i + 4 q + j
#pragma unroll
  for (int i = 0; i < 32; ++i) oacc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float mrun = dense ? neg_inf() : s_mref[myhead];
  float lpart = 0.f;  // this lane's keys of the kept tiles
  unsigned int pw[4][4];  // P of the tile as the P.V B operand, per 32-key step
  const int nkept = dense ? T : s_nsurv;

  auto kept_step = [&](auto E, auto C_, auto W_, int tile, const unsigned char* sl)
                       __attribute__((always_inline)) {
    constexpr int e = decltype(E)::value;
    constexpr int C = decltype(C_)::value;
    if constexpr (!KeptPlan::value[e]) {
      score(C_, W_, sl);
      if constexpr (e == KeptPlan::kLastScore) {
        const float m = finish_scores(tile);
        if (dense) {  // online pass
          const float mnew = fmaxf(mrun, m);
          if (__builtin_amdgcn_ballot_w64(mnew != mrun) != 0) {
            const float alpha = fast_exp2(mrun - (mnew == neg_inf() ? 0.f : mnew));
            lpart *= alpha;
#pragma unroll
            for (int i = 0; i < 32; ++i)
#pragma unroll
              for (int j = 0; j < 4; ++j) oacc[i][j] *= alpha;
          }
          mrun = mnew;
        }
        const float mref = mrun == neg_inf() ? 0.f : mrun;
        // 32-key step j takes blocks 2 j and 2 j + 1: k-elements 0..3 are the
        // lane's keys of the first, 4..7 those of the second
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int hb = 0; hb < 2; ++hb) {
            const float p0 = fast_exp2(sacc[2 * j + hb][0] - mref);
            const float p1 = fast_exp2(sacc[2 * j + hb][1] - mref);
            const float p2 = fast_exp2(sacc[2 * j + hb][2] - mref);
            const float p3 = fast_exp2(sacc[2 * j + hb][3] - mref);
            lpart += (p0 + p1) + (p2 + p3);
            pw[j][hb * 2] = pack_bf16x2(p0, p1);
            pw[j][hb * 2 + 1] = pack_bf16x2(p2, p3);
          }
      }
    } else {
      // value columns C + 16 cb + l16 for cb < 8.  The A operand V^T of
      // 32-key step j: rows 32 j + 4 q + (l16 >> 2) and + 16 (the keys of P's
      // k-elements), 4 columns from 4 (l16 & 3) of the block.
      const int rr = q * 4 + (l16 >> 2);  // row within the 16-key block
      const int sw = swz_value(rr);       // rows 32 j + rr and + 16 share it
      const int cq = (l16 & 3) * 4;       // first of the lane's 4 columns
      const unsigned char* base = sl + rr * 256 + (cq & 7) * 2;
      auto read = [&](int j, u32x4_t (&vv)[8]) __attribute__((always_inline)) {
#pragma unroll
        for (int cb = 0; cb < 8; ++cb) {
          const int off = ((2 * cb + (cq >> 3)) ^ sw) << 4;
          const s16x4_t lo =
              __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(base + 32 * j * 256 + off));
          const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_s16x4_t*)(base + (32 * j + 16) * 256 + off));
          const u32x2_t l2 = __builtin_bit_cast(u32x2_t, lo);
          const u32x2_t h2 = __builtin_bit_cast(u32x2_t, hi);
          vv[cb] = u32x4_t{l2[0], l2[1], h2[0], h2[1]};
        }
      };
      // V^T operands of 32-key step j + 1 are read while the MFMAs of step j run
      u32x4_t vv[2][8];
      read(0, vv[0]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (j + 1 < 4) read(j + 1, vv[(j + 1) & 1]);
        const bf16x8_t pb = as_bf16x8(u32x4_t{pw[j][0], pw[j][1], pw[j][2], pw[j][3]});
#pragma unroll
        for (int cb = 0; cb < 8; ++cb) {
          constexpr int ob = C / 16;
          oacc[ob + cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(vv[j & 1][cb]), pb,
                                                                 oacc[ob + cb], 0, 0, 0);
        }
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);
#pragma unroll
      for (int i = 0; i < 24; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    }
  };
  if (nkept > 0)
    pipeline(nkept, KeptPlan{},
             [&](int t) __attribute__((always_inline)) { return dense ? t0 + t : t0 + s_surv[t]; },
             kept_step);

  // ------------------------------------------------------------ write O / l and lse
  const float l = lpart + shfl_xor_f(lpart, 16) + shfl_xor_f(lpart + shfl_xor_f(lpart, 16), 32);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const size_t rowid = ((size_t)sub * a.B + b) * a.Hq + head0 + myhead;
  float* op = a.part_o + rowid * kDv;
#pragma unroll
  for (int i = 0; i < 32; ++i)
    *reinterpret_cast<f32x4_t*>(op + i * 16 + q * 4) =
        f32x4_t{oacc[i][0] * inv, oacc[i][1] * inv, oacc[i][2] * inv, oacc[i][3] * inv};
  if (q == 0) a.part_lse[rowid] = l > 0.f ? (mrun + __log2f(l)) * kLn2 : neg_inf();
}

}  // namespace

bool decode_mla_supported(int D, int Dv, int group, bool latent) {
  return latent && D == kDqk && Dv == kDv && (group == 64 || group == 128);
}

int decode_mla_max_tiles(int) { return kTmax; }

int decode_mla_workgroups_per_split(int group) { return group / kHalf; }

hipError_t launch_decode_mla(const DecodeArgs& a, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  const size_t units = (size_t)a.num_splits * a.B * a.Hkv;
  if (G == 128) {
    // halves interleaved in groups of 16 blocks: pad to a multiple of 8 sub-splits
    const size_t blocks = (units + 7) / 8 * 16;
    hipLaunchKernelGGL((decode_mla_kernel<2>), dim3((unsigned)blocks), dim3(kThreads), 0, s, a);
  } else if (G == 64) {
    hipLaunchKernelGGL((decode_mla_kernel<1>), dim3((unsigned)units), dim3(kThreads), 0, s, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace ssattn
