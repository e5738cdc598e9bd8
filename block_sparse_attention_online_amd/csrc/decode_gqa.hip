// Split-KV skip-softmax decode for grouped-query attention (a few query heads
// per KV head), bf16 K/V, fp32 accumulation, gfx950.
//
// Method: vLLM-Omni design page "Skip-Softmax", sections "The online-softmax
// pass" and "The skip test"; BLASST summary page, sections "Kerninzicht" (a
// skipped block also skips loading its V block from HBM) and "Kernel-ontwerp"
// (decode is memory bound; V loads of blocks that pass the test are issued in
// batches so the pipeline does not stall).
//
// One workgroup per (batch, KV head, sub-split of at most 64/G tiles), 4
// waves; wave w owns keys [32w, 32w + 32) of every 128-key tile.  Sub-splits
// form chains: in chained mode the whole sequence is one chain, in
// independent mode each user split is one.  Three phases per workgroup:
//
//  1. K pass.  Scores S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (16 keys x 16
//     query columns, G of them real).  K is loaded fully coalesced (16 lanes
//     per 256-byte row, whole rows per wave instruction, two tiles ahead),
//     passed 16 rows at a time through a per-wave XOR-swizzled LDS stage and
//     read back in the MFMA operand layout.  Scores (log2 units) go to LDS; each wave's per-row
//     maximum of every tile goes to LDS too.
//  2. Decision.  One wave scans the chunk's tile maxima: lane t holds tile t,
//     an exclusive prefix max over lanes gives every tile its running max, and
//     the tile is skipped iff max over rows of (tile_max - running_max) <
//     log2(threshold).  Kept tiles are compacted into a survivor list.  With
//     per-row decisions the tile is kept under the same rule (some row passes)
//     and each kept tile also records which rows passed; the others get P = 0.
//     Every sub-split first publishes its local maxima and reads those of the
//     earlier sub-splits of its chain, so the decisions are exactly those of
//     one streaming pass over the chain; the sub-splits still run in parallel
//     and only this step waits.
//  3. V pass.  Only survivors: lane (key, 16-byte chunk of the value row)
//     loads whole 256-byte V rows per wave instruction, two survivor tiles in
//     flight while one is accumulated, exponentials read back the
//     stored scores.  The exponent reference is the sub-split's own maximum,
//     so no rescale is needed at all.
//
// The split's O / l and lse go to the workspace; decode_combine merges splits.

#include "device_common.h"
#include "launch.h"

namespace ssattn {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kKeysPerWave = kTile / kWaves;  // 32
constexpr int kSpinCap = 1 << 21;             // look-back polls before giving up
constexpr int kWavesPerSimd = 3;              // occupancy target: 3 workgroups per CU

// Score area: 128 keys x G rows x 4 bytes per tile, 32 KB (64 KB past eight
// rows, where one workgroup holds the compute unit anyway).
template <int G>
constexpr int max_tiles() { return (G <= 8 ? 64 : 128) / G; }
// Query-head columns of one 16x16x32 MFMA block, and the rows one V-pass
// round accumulates (a lane holds 8 value columns of each).
template <int G>
constexpr int col_blocks() { return (G + 15) / 16; }
template <int G>
constexpr int v_rows() { return G < 16 ? G : 16; }
// Workgroups per compute unit the registers allow.
template <int D, int G>
constexpr int wg_per_cu() { return G <= 4 ? kWavesPerSimd : G <= 8 ? (D == 128 ? 2 : kWavesPerSimd) : 1; }

typedef __attribute__((ext_vector_type(4))) float f4_t;

template <int D, int G, bool PAGED>
__global__ __launch_bounds__(kThreads, (wg_per_cu<D, G>())) void decode_gqa_kernel(DecodeArgs a) {
  constexpr int TMAX = max_tiles<G>();
  constexpr int CB = col_blocks<G>();  // K pass: MFMA column blocks
  constexpr int GR = v_rows<G>();      // V pass: rows per round
  constexpr int RH = G / GR;           // V pass: rounds
  constexpr unsigned kAllRows = G == 32 ? ~0u : (1u << G) - 1u;
  constexpr int KS = D / 32;          // MFMA k-steps over the head dimension
  constexpr int KL = 2 * KS;          // 16-byte K loads per lane per tile
  constexpr int KCH = D / 8;          // V pass: lanes per value row
  constexpr int KPI = 64 / KCH;       // V pass: keys per wave instruction
  constexpr int IT = kKeysPerWave / KPI;
  static_assert(G >= 1 && G <= 32 && TMAX <= 64 && RH * GR == G, "group");
  static_assert(RH > 1 || kWaves * GR * D <= TMAX * kTile * G, "reduction reuses the score area");

  __shared__ __attribute__((aligned(16))) float sc[TMAX * kTile * G];  // [tile][key][row]
  __shared__ __attribute__((aligned(16))) unsigned char kstage[kWaves][16 * D * 2];
  __shared__ float tpart[kWaves][TMAX][G];
  __shared__ float s_mref[G];
  __shared__ float s_lred[kWaves][GR];
  // several V rounds read the scores again: their reduction area is separate
  __shared__ __attribute__((aligned(16))) float red_sep[RH > 1 ? kWaves * GR * D : 1];
  __shared__ int s_surv[TMAX];
  __shared__ unsigned s_rowkeep[TMAX];  // per kept tile: bit r = row r adds its P
  __shared__ int s_nsurv;
  __shared__ int s_blk[PAGED ? TMAX * kTile / 16 : 1];  // paged: this sub-split's cache blocks

  const int S = a.num_splits;  // sub-splits per (batch, KV head)
  const int sub = blockIdx.x % S;
  const int pair = blockIdx.x / S;  // b * Hkv + hk
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
  const int chain = sub / a.subs_per_chain;
  const int link = sub % a.subs_per_chain;
  const int chain_t0 = chain * a.chain_tiles;
  const int chain_t1 = min(chain_t0 + a.chain_tiles, nK);
  const int t0 = chain_t0 + link * a.tiles_per_split;
  const int T = max(0, min(t0 + a.tiles_per_split, chain_t1) - t0);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int l16 = lane & 15;
  const int grp = lane >> 4;

  if constexpr (PAGED) {
    // tiles of this sub-split's range past the sequence's end: not visited
    const int mask_tiles = a.mask_tiles;
    const int t_end = min(min(t0 + a.tiles_per_split, chain_t0 + a.chain_tiles), mask_tiles);
    if (a.mask)
      for (int t = max(t0, t0 + T) + threadIdx.x; t < t_end; t += kThreads)
        a.mask[(size_t)pair * mask_tiles + t] = 2;
  }
  if (T == 0) {  // an empty trailing link: nothing to publish, nobody waits on it
    for (int idx = tid; idx < G * D; idx += kThreads) {
      const size_t rowid = ((size_t)sub * a.B + b) * a.Hq + hk * G + idx / D;
      a.part_o[rowid * D + idx % D] = 0.f;
      if (idx % D == 0) a.part_lse[rowid] = neg_inf();
    }
    return;
  }

  const unsigned short* qp =
      static_cast<const unsigned short*>(a.q) + ((size_t)b * a.Hq + hk * G) * D;
  const unsigned short* kp =
      static_cast<const unsigned short*>(a.k) + (PAGED ? 0 : ((size_t)pair * a.Lk) * D);
  const unsigned short* vp =
      static_cast<const unsigned short*>(a.v) + (PAGED ? 0 : ((size_t)pair * a.Lk) * D);
  // paged: the cache blocks of keys [t0 * 128, min((t0 + T) * 128, Lk)), block
  // ids clamped into the cache
  const int blk0 = PAGED ? (t0 * kTile) >> a.block_log2 : 0;
  if constexpr (PAGED) {
    const int nb = ((min((t0 + T) * kTile, Lk) - 1) >> a.block_log2) - blk0 + 1;
    for (int i = tid; i < nb; i += kThreads)
      s_blk[i] = min(max(a.block_table[(size_t)b * a.max_blocks + blk0 + i], 0), a.num_blocks - 1);
    __syncthreads();
  }
  // first element of key row `key` (Lk > key >= t0 * 128) of K, or of V
  auto row = [&](const unsigned short* base, int key) -> const unsigned short* {
    if constexpr (PAGED) {
      const int blk = s_blk[(key >> a.block_log2) - blk0];
      const size_t r = (((size_t)blk * a.Hkv + hk) << a.block_log2) +
                       (key & ((1 << a.block_log2) - 1));
      return base + r * D;
    } else {
      return base + (size_t)key * D;
    }
  };
  const float c = a.scale * kLog2e;

  // ---------------------------------------------------------------- 1. K pass
  {
    // Q^T as the MFMA B operand: in column block cb lane holds row
    // 16 cb + l16 (zero past G), dims 32 ks + 8 grp
    bf16x8_t qb[CB][KS];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int r = cb * 16 + l16;
        u32x4_t u = {0u, 0u, 0u, 0u};
        if (r < G) u = *reinterpret_cast<const u32x4_t*>(qp + (size_t)r * D + ks * 32 + grp * 8);
        qb[cb][ks] = as_bf16x8(u);
      }
    // coalesced K loads: load i covers rows [i*RPI, (i+1)*RPI) of the wave's 32
    constexpr int RPI = 64 / KCH;  // key rows per wave instruction
    const int lrow = lane / KCH, lch = lane % KCH;
    // Loads are unconditional (no branch around them, so the compiler's wait
    // counts stay exact and the prefetch stays in flight): keys past Lk read
    // the last key row, and their scores are masked to -inf below.
    auto load_k = [&](int tl, u32x4_t (&dst)[KL]) {
      const int j0 = (t0 + tl) * kTile + w * kKeysPerWave;
#pragma unroll
      for (int i = 0; i < KL; ++i) {
        const int key = min(j0 + i * RPI + lrow, Lk - 1);
        dst[i] = *reinterpret_cast<const u32x4_t*>(row(kp, key) + lch * 8);
      }
    };
    unsigned char* stage = kstage[w];
    auto score_tile = [&](int tl, const u32x4_t (&src)[KL]) {
      // the wave's 32 rows go through the stage 16 at a time (one MFMA block);
      // 16-byte chunk c of stage row r sits at chunk c ^ (r & 7)
      f32x4_t acc[CB][2];
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
        for (int i = blk * (KL / 2); i < (blk + 1) * (KL / 2); ++i) {
          const int r = i * RPI + lrow - blk * 16;
          *reinterpret_cast<u32x4_t*>(stage + r * (D * 2) + ((lch ^ (r & 7)) << 4)) = src[i];
        }
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) acc[cb][blk] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const int ch = ks * 4 + grp;
          const u32x4_t kv =
              *reinterpret_cast<const u32x4_t*>(stage + l16 * (D * 2) + ((ch ^ (l16 & 7)) << 4));
#pragma unroll
          for (int cb = 0; cb < CB; ++cb)
            acc[cb][blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kv), qb[cb][ks],
                                                                  acc[cb][blk], 0, 0, 0);
        }
        __builtin_amdgcn_wave_barrier();
      }
      const int jw = (t0 + tl) * kTile + w * kKeysPerWave;  // first key of this wave
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const int r = cb * 16 + l16;  // this lane's query row
        float pm = neg_inf();
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int kin = blk * 16 + grp * 4 + i;  // key within the wave's 32
            float s = acc[cb][blk][i] * c;
            if (jw + kin >= Lk) s = neg_inf();
            if (r < G) sc[(tl * kTile + w * kKeysPerWave + kin) * G + r] = s;
            pm = fmaxf(pm, s);
          }
        pm = fmaxf(pm, shfl_xor_f(pm, 16));
        pm = fmaxf(pm, shfl_xor_f(pm, 32));
        if (lane < 16 && r < G) tpart[w][tl][r] = pm;
      }
    };
    // three tiles of K in flight per wave; prefetches past the last tile
    // re-read the last tile (cache hits) and are not used
    u32x4_t kA[KL], kB[KL], kC[KL];
    load_k(0, kA);
    load_k(min(1, T - 1), kB);
    for (int tl = 0; tl < T; tl += 3) {
      load_k(min(tl + 2, T - 1), kC);
      score_tile(tl, kA);
      load_k(min(tl + 3, T - 1), kA);
      if (tl + 1 < T) score_tile(tl + 1, kB);
      load_k(min(tl + 4, T - 1), kB);
      if (tl + 2 < T) score_tile(tl + 2, kC);
    }
  }
  __syncthreads();

  // ---------------------------------------------------------------- 2. decision
  if (w == 0) {
    const bool valid = lane < T;
    float tm[G], cmax[G];
#pragma unroll
    for (int r = 0; r < G; ++r) {
      float x = neg_inf();
      if (valid) {
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) x = fmaxf(x, tpart[ww][lane][r]);
      }
      tm[r] = x;
      cmax[r] = lanes_max_from<1>(x);
    }
    // Publish this link's per-row maxima and fold in those of the earlier
    // links of the chain.  Every published value is one 64-bit relaxed
    // device-scope atomic holding (launch tag, float bits): a reader takes a
    // value only once its tag is this launch's, so no ordering between
    // locations (and no cache write-back fence) is needed.
    const unsigned tag = a.lb_tag;
    const size_t slot = (size_t)pair * S + sub;
    if (a.subs_per_chain > 1) {
#pragma unroll
      for (int r = 0; r < G; ++r)
        if (lane == r)
          __hip_atomic_store(&a.lb_slot[slot * G + r],
                             ((unsigned long long)tag << 32) | __float_as_uint(cmax[r]),
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    float prev[G];
#pragma unroll
    for (int r = 0; r < G; ++r) prev[r] = neg_inf();
    for (int base = 0; base < link; base += 64) {
      const int lk = base + lane;
      if (lk < link) {
        const size_t ps = (size_t)pair * S + (sub - link) + lk;
#pragma unroll
        for (int r = 0; r < G; ++r) {
          int spins = 0;
          unsigned long long v;
          while (((v = __hip_atomic_load(&a.lb_slot[ps * G + r], __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT)) >> 32) != tag &&
                 spins < kSpinCap) {
            __builtin_amdgcn_s_sleep(1);
            ++spins;
          }
          if (spins < kSpinCap)
            prev[r] = fmaxf(prev[r], __uint_as_float((unsigned)v));
          else
            atomicAdd(a.lb_timeouts, 1u);
        }
      }
    }
    // running max before each tile: earlier links, then an exclusive prefix
    // max over this link's tiles (lane t = tile t)
    float dmax = neg_inf();
    unsigned rowkeep = 0;  // bit r: row r passes its own test on this lane's tile
#pragma unroll
    for (int r = 0; r < G; ++r) {
      const float mstart = lanes_max_from<1>(prev[r]);
      float incl = tm[r];
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float up = __shfl_up(incl, off, 64);
        if (lane >= off) incl = fmaxf(incl, up);
      }
      float excl = __shfl_up(incl, 1, 64);
      if (lane == 0) excl = neg_inf();
      const float M = fmaxf(mstart, excl);
      float dr = neg_inf();
      if (tm[r] != neg_inf()) dr = (M == neg_inf()) ? pos_inf() : tm[r] - M;
      dmax = fmaxf(dmax, dr);
      if (!(dr < log2_thr)) rowkeep |= 1u << r;
    }
    const bool skip = dmax < log2_thr;
    const bool kept = valid && !skip;
    const unsigned long long bits = __ballot(kept);
    const int idx = __popcll(bits & ((1ull << lane) - 1ull));
    if (kept) s_surv[idx] = lane;
    if constexpr (!PAGED) {
      if (valid) s_rowkeep[lane] = a.per_row ? rowkeep : kAllRows;
      if (valid && a.row_mask) {
#pragma unroll
        for (int r = 0; r < G; ++r)
          a.row_mask[((size_t)b * a.Hq + hk * G + r) * nK + t0 + lane] = (rowkeep >> r) & 1u ? 0 : 1;
      }
    }
    if (lane == 0) s_nsurv = __popcll(bits);
    if (valid && a.mask)
      a.mask[(size_t)pair * (PAGED ? a.mask_tiles : nK) + t0 + lane] = skip ? 1 : 0;
#pragma unroll
    for (int r = 0; r < G; ++r)
      if (lane == r) s_mref[r] = cmax[r];
  }
  __syncthreads();

  // ---------------------------------------------------------------- 3. V pass
  // rows [rb, rb + GR) per round; more than one round (past 16 rows) reads
  // the kept V rows again, from L2
  const int kq = lane / KCH;
  const int cc = lane % KCH;
  const int nsurv = s_nsurv;
#pragma unroll
  for (int rh = 0; rh < RH; ++rh) {
    const int rb = rh * GR;
    float mref[GR], o[GR][8], lp[GR];
#pragma unroll
    for (int r = 0; r < GR; ++r) {
      mref[r] = s_mref[rb + r];
      lp[r] = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[r][e] = 0.f;
    }
    {
      // unconditional loads as in the K pass; keys past Lk carry p = 0
      auto load_v = [&](int si, u32x4_t (&dst)[IT]) {
        const int j0 = (t0 + s_surv[si]) * kTile + w * kKeysPerWave;
#pragma unroll
        for (int it = 0; it < IT; ++it) {
          const int key = min(j0 + it * KPI + kq, Lk - 1);
          dst[it] = *reinterpret_cast<const u32x4_t*>(row(vp, key) + cc * 8);
        }
      };
      auto accum_v = [&](int si, const u32x4_t (&src)[IT]) {
        const int tl = s_surv[si];
        // rows that did not pass on this tile (per-row decisions) take +inf
        // as their exponent reference: P = 0
        const unsigned keep = PAGED ? kAllRows : s_rowkeep[tl];
        float mx[GR];
#pragma unroll
        for (int r = 0; r < GR; ++r) mx[r] = (keep >> (rb + r)) & 1u ? mref[r] : pos_inf();
#pragma unroll
        for (int it = 0; it < IT; ++it) {
          const int kin = w * kKeysPerWave + it * KPI + kq;
          const float* srow = sc + (tl * kTile + kin) * G + rb;
          float p[GR];
          if constexpr (G == 4) {
            const f4_t s4 = *reinterpret_cast<const f4_t*>(srow);
#pragma unroll
            for (int r = 0; r < 4; ++r) p[r] = fast_exp2(s4[r] - mx[r]);
          } else {
#pragma unroll
            for (int r = 0; r < GR; ++r) p[r] = fast_exp2(srow[r] - mx[r]);
          }
          float vf[8];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            vf[2 * e] = bf16_lo(src[it][e]);
            vf[2 * e + 1] = bf16_hi(src[it][e]);
          }
#pragma unroll
          for (int r = 0; r < GR; ++r) {
            lp[r] += p[r];
#pragma unroll
            for (int e = 0; e < 8; ++e) o[r][e] = fmaf(p[r], vf[e], o[r][e]);
          }
        }
      };
      if constexpr (G <= 8) {
        if (nsurv > 0) {  // three survivor tiles of V in flight per wave
          u32x4_t vA[IT], vB[IT], vC[IT];
          load_v(0, vA);
          load_v(min(1, nsurv - 1), vB);
          for (int si = 0; si < nsurv; si += 3) {
            load_v(min(si + 2, nsurv - 1), vC);
            accum_v(si, vA);
            load_v(min(si + 3, nsurv - 1), vA);
            if (si + 1 < nsurv) accum_v(si + 1, vB);
            load_v(min(si + 4, nsurv - 1), vB);
            if (si + 2 < nsurv) accum_v(si + 2, vC);
          }
        }
      } else {
        if (nsurv > 0) {  // the accumulators of 16 rows leave room for two tiles in flight
          u32x4_t vA[IT], vB[IT];
          load_v(0, vA);
          for (int si = 0; si < nsurv; si += 2) {
            load_v(min(si + 1, nsurv - 1), vB);
            accum_v(si, vA);
            load_v(min(si + 2, nsurv - 1), vA);
            if (si + 1 < nsurv) accum_v(si + 1, vB);
          }
        }
      }
    }
    // ------------------------------------------------------------ merge and write
    float* red = RH > 1 ? red_sep : sc;  // [wave][row][D]
    __syncthreads();  // a single round's reduction overwrites the score area; the previous round's is read
#pragma unroll
    for (int r = 0; r < GR; ++r) {
      const float lr = lanes_sum_from<KCH>(lp[r]);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[r][e] = lanes_sum_from<KCH>(o[r][e]);
      if (kq == 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) red[(w * GR + r) * D + cc * 8 + e] = o[r][e];
      }
      if (lane == 0) s_lred[w][r] = lr;
    }
    __syncthreads();
    for (int idx = tid; idx < GR * D; idx += kThreads) {
      const int r = idx / D, dv = idx % D;
      float ov = 0.f, l = 0.f;
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) {
        ov += red[(ww * GR + r) * D + dv];
        l += s_lred[ww][r];
      }
      const size_t rowid = ((size_t)sub * a.B + b) * a.Hq + hk * G + rb + r;
      a.part_o[rowid * D + dv] = l > 0.f ? ov / l : 0.f;
      if (dv == 0) a.part_lse[rowid] = l > 0.f ? (s_mref[rb + r] + __log2f(l)) * kLn2 : neg_inf();
    }
  }
}

template <int D, bool PAGED>
hipError_t launch_d(const DecodeArgs& a, hipStream_t s, int G) {
  const dim3 grid((unsigned)((size_t)a.num_splits * a.Hkv * a.B));
#define SSATTN_DECODE_CASE(g) \
  case g: hipLaunchKernelGGL((decode_gqa_kernel<D, g, PAGED>), grid, dim3(kThreads), 0, s, a); break;
  switch (G) {
    SSATTN_DECODE_CASE(1)
    SSATTN_DECODE_CASE(2)
    SSATTN_DECODE_CASE(3)
    SSATTN_DECODE_CASE(4)
    SSATTN_DECODE_CASE(5)
    SSATTN_DECODE_CASE(6)
    SSATTN_DECODE_CASE(7)
    SSATTN_DECODE_CASE(8)
    SSATTN_DECODE_CASE(16)
    SSATTN_DECODE_CASE(32)
    default: return hipErrorInvalidValue;
  }
#undef SSATTN_DECODE_CASE
  return hipGetLastError();
}

}  // namespace

bool decode_gqa_supported(int D, int Dv, int group, bool latent) {
  return !latent && D == Dv && (D == 64 || D == 128) &&
         ((group >= 1 && group <= 8) || group == 16 || group == 32);
}

int decode_gqa_max_tiles(int group) { return (group <= 8 ? 64 : 128) / group; }

hipError_t launch_decode_gqa(const DecodeArgs& a, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  return a.D == 64 ? launch_d<64, false>(a, s, G) : launch_d<128, false>(a, s, G);
}

hipError_t launch_decode_gqa_paged(const DecodeArgs& a, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  return a.D == 64 ? launch_d<64, true>(a, s, G) : launch_d<128, true>(a, s, G);
}

}  // namespace ssattn
