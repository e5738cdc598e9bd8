// Split-KV skip-softmax decode for grouped-query attention (a few query heads
// per KV head), bf16 K/V, fp32 accumulation, gfx950.
//
// Method: vLLM-Omni design page "Skip-Softmax", sections "The online-softmax
// pass" and "The skip test"; BLASST summary page, section "Kerninzicht" (a
// skipped block also skips loading its V block from HBM) and
// "Kernel-ontwerp" (decode is memory bound; the saving is V bandwidth).
//
// One workgroup per (batch, KV head, split); 8 waves, each owning 16 keys of
// every 128-key tile.  The group's G query rows are tiny, so the dot products
// run on the vector ALUs: lane (key k, chunk c) multiplies 8 head dims of key
// k by the same 8 dims of all G rows, and the 16 lanes of one key (8 for
// D = 64) sum their partials with DPP row operations.  Every K load is one
// 16-byte load per lane with 16 consecutive lanes on one 256-byte key row, so
// a wave instruction reads whole rows.  The decision is taken for the whole
// group (max over rows and over the 8 waves through LDS) before any V byte of
// the tile is requested: a skipped tile's V is never loaded.  K of the next
// tile is requested before the current tile is reduced.

#include "device_common.h"
#include "launch.h"

namespace ssattn {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kKeysPerWave = kTile / kWaves;  // 16

template <int D, int G>
__global__ __launch_bounds__(kThreads) void decode_gqa_kernel(DecodeArgs a) {
  constexpr int KCH = D / 8;               // lanes per key row (16-byte chunks)
  constexpr int KPI = 64 / KCH;            // keys per wave instruction
  constexpr int IT = kKeysPerWave / KPI;   // instructions per wave per tile
  static_assert(IT >= 1, "layout");

  __shared__ float redm[2][kWaves][G];
  __shared__ float sred[kWaves][G][D];
  __shared__ float lred[kWaves][G];

  const int S = a.num_splits;
  const int split = blockIdx.x % S;
  const int hk = (blockIdx.x / S) % a.Hkv;
  const int b = blockIdx.x / (S * a.Hkv);
  const int nK = (a.Lk + kTile - 1) / kTile;
  const int t0 = split * a.tiles_per_split;
  const int t1 = min(t0 + a.tiles_per_split, nK);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int cch = lane % KCH;  // head-dim chunk of this lane
  const int kq = lane / KCH;   // key slot within one instruction

  const unsigned short* qp = static_cast<const unsigned short*>(a.q) + ((size_t)b * a.Hq + hk * G) * D;
  const unsigned short* kp =
      static_cast<const unsigned short*>(a.k) + ((size_t)(b * a.Hkv + hk) * a.Lk) * D;
  const unsigned short* vp =
      static_cast<const unsigned short*>(a.v) + ((size_t)(b * a.Hkv + hk) * a.Lk) * D;

  const float c = a.scale * kLog2e;
  float qv[G][8];
#pragma unroll
  for (int r = 0; r < G; ++r) {
    const u32x4_t u = *reinterpret_cast<const u32x4_t*>(qp + (size_t)r * D + cch * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      qv[r][2 * e] = bf16_lo(u[e]) * c;
      qv[r][2 * e + 1] = bf16_hi(u[e]) * c;
    }
  }

  float m2[G], lpart[G], opart[G][8];
#pragma unroll
  for (int r = 0; r < G; ++r) {
    m2[r] = neg_inf();
    lpart[r] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) opart[r][e] = 0.f;
  }

  auto key_of = [&](int j, int it) { return j * kTile + w * kKeysPerWave + it * KPI + kq; };
  u32x4_t kcur[IT];
  auto load_k = [&](u32x4_t (&dst)[IT], int j) {
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int key = key_of(j, it);
      u32x4_t val = {0u, 0u, 0u, 0u};
      if (key < a.Lk) val = *reinterpret_cast<const u32x4_t*>(kp + (size_t)key * D + cch * 8);
      dst[it] = val;
    }
  };
  load_k(kcur, t0);

  for (int j = t0; j < t1; ++j) {
    const int par = (j - t0) & 1;
    u32x4_t knext[IT];
    if (j + 1 < t1) load_k(knext, j + 1);

    // scores in log2 units, every lane of a key row holds its key's score
    float s2[IT][G];
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      float kf[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kf[2 * e] = bf16_lo(kcur[it][e]);
        kf[2 * e + 1] = bf16_hi(kcur[it][e]);
      }
      const bool valid = key_of(j, it) < a.Lk;
#pragma unroll
      for (int r = 0; r < G; ++r) {
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) d = fmaf(qv[r][e], kf[e], d);
        d = group_sum<KCH>(d);
        s2[it][r] = valid ? d : neg_inf();
      }
    }

    // tile max per row: over this lane's keys, the wave's key slots, the waves
#pragma unroll
    for (int r = 0; r < G; ++r) {
      float tm = s2[0][r];
#pragma unroll
      for (int it = 1; it < IT; ++it) tm = fmaxf(tm, s2[it][r]);
      tm = lanes_max_from<KCH>(tm);
      if (lane == 0) redm[par][w][r] = tm;
    }
    __syncthreads();
    float tmax2[G];
    float dblk = neg_inf();
#pragma unroll
    for (int r = 0; r < G; ++r) {
      float tm = redm[par][0][r];
#pragma unroll
      for (int ww = 1; ww < kWaves; ++ww) tm = fmaxf(tm, redm[par][ww][r]);
      tmax2[r] = tm;
      float dr = neg_inf();
      if (tm != neg_inf()) dr = (m2[r] == neg_inf()) ? pos_inf() : tm - m2[r];
      dblk = fmaxf(dblk, dr);
    }
    const bool skip = dblk < a.log2_thr;
    if (a.mask && tid == 0) a.mask[(size_t)(b * a.Hkv + hk) * nK + j] = skip ? 1 : 0;

    if (!skip) {
      u32x4_t vreg[IT];
#pragma unroll
      for (int it = 0; it < IT; ++it) {
        const int key = key_of(j, it);
        u32x4_t val = {0u, 0u, 0u, 0u};
        if (key < a.Lk) val = *reinterpret_cast<const u32x4_t*>(vp + (size_t)key * D + cch * 8);
        vreg[it] = val;
      }
#pragma unroll
      for (int r = 0; r < G; ++r) {
        const float m2n = fmaxf(m2[r], tmax2[r]);
        const float alpha = fast_exp2(m2[r] - m2n);  // 0 when m2 = -inf (m2n finite here)
        lpart[r] *= alpha;
#pragma unroll
        for (int e = 0; e < 8; ++e) opart[r][e] *= alpha;
        m2[r] = m2n;
      }
#pragma unroll
      for (int it = 0; it < IT; ++it) {
        float vf[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          vf[2 * e] = bf16_lo(vreg[it][e]);
          vf[2 * e + 1] = bf16_hi(vreg[it][e]);
        }
#pragma unroll
        for (int r = 0; r < G; ++r) {
          const float p = fast_exp2(s2[it][r] - m2[r]);
          lpart[r] += p;
#pragma unroll
          for (int e = 0; e < 8; ++e) opart[r][e] = fmaf(p, vf[e], opart[r][e]);
        }
      }
    } else {
#pragma unroll
      for (int r = 0; r < G; ++r) {
        const float m2n = fmaxf(m2[r], tmax2[r]);
        if (a.thr_above_1 && m2n > m2[r]) {
          const float alpha = fast_exp2(m2[r] - m2n);
          lpart[r] *= alpha;
#pragma unroll
          for (int e = 0; e < 8; ++e) opart[r][e] *= alpha;
        }
        m2[r] = m2n;
      }
    }
    if (j + 1 < t1) {
#pragma unroll
      for (int it = 0; it < IT; ++it) kcur[it] = knext[it];
    }
  }

  // ---- merge lanes of different key slots, then the waves, and write the split
#pragma unroll
  for (int r = 0; r < G; ++r) {
    float lr = lanes_sum_from<KCH>(lpart[r]);
#pragma unroll
    for (int e = 0; e < 8; ++e) opart[r][e] = lanes_sum_from<KCH>(opart[r][e]);
    if (lane < KCH) {
#pragma unroll
      for (int e = 0; e < 8; ++e) sred[w][r][cch * 8 + e] = opart[r][e];
    }
    if (lane == 0) lred[w][r] = lr;
  }
  __syncthreads();
  for (int idx = tid; idx < G * D; idx += kThreads) {
    const int r = idx / D, dv = idx % D;
    float o = 0.f, l = 0.f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
      o += sred[ww][r][dv];
      l += lred[ww][r];
    }
    const size_t rowid = ((size_t)split * a.B + b) * a.Hq + hk * G + r;
    a.part_o[rowid * D + dv] = o / l;
    if (dv == 0) a.part_lse[rowid] = (m2[r] + __log2f(l)) * kLn2;
  }
}

template <int D>
hipError_t launch_d(const DecodeArgs& a, hipStream_t s, int G) {
  const dim3 grid((unsigned)((size_t)a.num_splits * a.Hkv * a.B));
  switch (G) {
    case 1: hipLaunchKernelGGL((decode_gqa_kernel<D, 1>), grid, dim3(kThreads), 0, s, a); break;
    case 2: hipLaunchKernelGGL((decode_gqa_kernel<D, 2>), grid, dim3(kThreads), 0, s, a); break;
    case 4: hipLaunchKernelGGL((decode_gqa_kernel<D, 4>), grid, dim3(kThreads), 0, s, a); break;
    case 8: hipLaunchKernelGGL((decode_gqa_kernel<D, 8>), grid, dim3(kThreads), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

bool decode_gqa_supported(int D, int Dv, int group, bool latent) {
  return !latent && D == Dv && (D == 64 || D == 128) &&
         (group == 1 || group == 2 || group == 4 || group == 8);
}

hipError_t launch_decode_gqa(const DecodeArgs& a, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  return a.D == 64 ? launch_d<64>(a, s, G) : launch_d<128>(a, s, G);
}

}  // namespace ssattn
