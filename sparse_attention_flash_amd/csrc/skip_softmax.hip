// skip_softmax.hip -- skip-softmax (BLASST-style) flash-attention forward for gfx950.
//
// Method: Model-Optimizer "Skip-Softmax Sparse Attention for Diffusion Models" README
// (introduction; "Threshold Modes"): during the FlashAttention loop a key tile whose scores are
// negligible is skipped, which saves its exponentials, its V load and its P.V product; the kernel
// works with log2(lambda).  Decision rule (the reading stated in sa.h): with t = c*q.k in the log2
// domain, tile j is skipped when every valid row r of the query tile has
//     M_j[r] < fl32(m[r] + log2(lambda)),
// m[r] being the fp32 running max of the tiles kept so far; a skipped tile leaves (m, l, O) alone.
//
// One workgroup = one (batch, query head, query tile of 32*QB*NW rows); each wavefront owns 32*QB
// rows.
// The pipelined loop (mainloop.h) computes S^T = K.Q^T on MFMA, masks, takes the row max (in-lane
// plus one permlane32 swap), and each wavefront votes "some row not negligible" with a ballot; the
// votes meet in LDS at the barrier that also publishes the previous V tile.  Only a kept tile has
// its V tile fetched and runs exp2 + P.V.
#include "kernels.h"
#include "mainloop.h"

namespace sa {
namespace {

template <int D, int NW, int QB>
struct SkipPolicy {
  static constexpr bool kDecide = true, kFilter = false, kWeighted = false;
  static constexpr int RW = 32 * QB;   // rows per wave
  static constexpr int BR = NW * RW;
  const __bf16* kslab;
  const __bf16* vslab;
  int k_stride_b, v_stride_b, k_bytes, v_bytes;
  int Sq, Sk, causal, wrow0, nvis, nKT, h, r32;
  float L32;
  uint8_t* tile_state;
  float* rowmax;
  int64_t unit;
  int nskip;

  __device__ __forceinline__ int steps() const { return nvis; }

  __device__ __forceinline__ TileSrc src(int j) const {
    const int k0 = j * kKeysPerTile;
    return TileSrc{kslab + (int64_t)k0 * (k_stride_b / 2), vslab + (int64_t)k0 * (v_stride_b / 2),
                   max(0, k_bytes - k0 * k_stride_b), max(0, v_bytes - k0 * v_stride_b),
                   k_stride_b, v_stride_b};
  }

  // key = k0 + 4*h + off(kb, r) with off a compile-time constant; masked when off >= lim
  __device__ __forceinline__ void mask(int j, f32x16 (&s)[2][QB], int lane) const {
    const int k0 = j * kKeysPerTile;
    if (!((k0 + kKeysPerTile > Sk) || (causal && k0 + kKeysPerTile - 1 > wrow0))) return;
    const int klim = Sk - k0 - 4 * h;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      int lim = klim;
      if (causal) lim = min(lim, wrow0 + qb * 32 + r32 - k0 - 4 * h + 1);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) mask_block(s[kb][qb], kb, lim);
    }
  }

  // true when every valid row this lane holds is negligible: M < fl32(m + log2(lambda))
  __device__ __forceinline__ bool negligible(const float (&M)[QB], const float (&mt)[QB],
                                             int lane) const {
    bool negl = true;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float thr = mt[qb] + L32;
      if (wrow0 + qb * 32 + r32 < Sq && !(M[qb] < thr)) negl = false;
    }
    return negl;
  }

  __device__ __forceinline__ void record(int j, bool keep, const float (&M)[QB], int wave,
                                         int lane, int tid) {
    if (!keep) ++nskip;
    if (tid == 0 && tile_state != nullptr) tile_state[unit * nKT + j] = keep ? 0 : 1;
    if (rowmax != nullptr && h == 0) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
        rowmax[(unit * nKT + j) * BR + wave * RW + qb * 32 + r32] = M[qb];
    }
  }

  __device__ __forceinline__ void filter(int, const f32x16 (&)[2][QB], uint32_t (&)[QB], int) const {}
};

template <int D, int NW, int QB>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(kWavesPerSimd<QB>)))
void skip_softmax_kernel(SkipArgs a) {
  constexpr int RW = 32 * QB;
  constexpr int BR = NW * RW;
  constexpr int NT = NW * 64;
  __shared__ __attribute__((aligned(1024))) Smem<D, NW> sm;

  const AttnGeom& g = a.g;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, r32 = lane & 31;
  const int nQT = (g.Sq + BR - 1) / BR;
  const int nKT = (g.Sk + kKeysPerTile - 1) / kKeysPerTile;
  const int G = g.Hq / g.Hkv;
  const int total = g.B * g.Hq * nQT;

  // Work item order: KV head major, then query tile, then the G query heads sharing the KV head,
  // so that concurrently running workgroups of one XCD read the same K/V tiles.  Causal: the
  // longest rows first.
  int item = xcd_remap(blockIdx.x, total);
  const int gq = item % G;
  item /= G;
  int qt = item % nQT;
  item /= nQT;
  const int hk = item % g.Hkv;
  const int b = item / g.Hkv;
  if (g.causal) qt = nQT - 1 - qt;
  const int hq = hk * G + gq;

  const int row0 = qt * BR;
  const int wrow0 = row0 + wave * RW;
  const int last_row = min(row0 + BR, g.Sq) - 1;
  const int nvis = g.causal ? min(nKT, last_row / kKeysPerTile + 1) : nKT;

  const __bf16* qslab = (const __bf16*)g.q + b * g.qs[0] + hq * g.qs[2];
  const auto qsrc = slab_rsrc(qslab, g.qs[1], g.Sq, D);
  bf16x8 qf[QB][D / 16];
  load_q_frags<D, QB>(qf, qsrc, g.qs[1], wrow0, lane);

  SkipPolicy<D, NW, QB> pol;
  pol.kslab = (const __bf16*)g.k + b * g.ks[0] + hk * g.ks[2];
  pol.vslab = (const __bf16*)g.v + b * g.vs[0] + hk * g.vs[2];
  pol.k_stride_b = (int)(g.ks[1] * 2);
  pol.v_stride_b = (int)(g.vs[1] * 2);
  pol.k_bytes = (int)(((int64_t)(g.Sk - 1) * g.ks[1] + D) * 2);
  pol.v_bytes = (int)(((int64_t)(g.Sk - 1) * g.vs[1] + D) * 2);
  pol.Sq = g.Sq;
  pol.Sk = g.Sk;
  pol.causal = g.causal;
  pol.wrow0 = wrow0;
  pol.nvis = nvis;
  pol.nKT = nKT;
  pol.h = h;
  pol.r32 = r32;
  pol.L32 = a.L32;
  pol.tile_state = a.tile_state;
  pol.rowmax = a.rowmax;
  pol.unit = ((int64_t)b * g.Hq + hq) * nQT + qt;
  pol.nskip = 0;

  f32x16 o[D / 32][QB];
  float mref[QB], l[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o[db][qb] = f32x16{};
    mref[qb] = -INFINITY;
    l[qb] = 0.f;
  }
  run_mainloop<D, NW, QB>(pol, sm, qf, o, mref, l, g.c32, wave, lane, tid);

  // Epilogue: normalise, store O and the natural-log LSE.
  float inv[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lt = half_sum(l[qb]);
    inv[qb] = lt > 0.f ? 1.f / lt : 0.f;
    const int row = wrow0 + qb * 32 + r32;
    if (a.lse != nullptr && h == 0 && row < g.Sq)
      a.lse[((int64_t)b * g.Hq + hq) * g.Sq + row] =
          lt > 0.f ? (mref[qb] + __log2f(lt)) * 0.69314718055994531f : -INFINITY;
  }
  __bf16* op = (__bf16*)g.o + b * g.os[0] + (int64_t)wrow0 * g.os[1] + hq * g.os[2];
  store_o<D, QB>(op, g.os[1], g.Sq - wrow0, o, inv, lane);

  const int64_t unit = pol.unit;
  if (a.tile_state != nullptr)
    for (int j = nvis + tid; j < nKT; j += NT) a.tile_state[unit * nKT + j] = 2;
  if (a.rowmax != nullptr)
    for (int64_t i = (int64_t)nvis * BR + tid; i < (int64_t)nKT * BR; i += NT)
      a.rowmax[unit * nKT * BR + i] = -INFINITY;
  if (tid == 0 && a.counters != nullptr) {
    atomicAdd(&a.counters[2 * (b * g.Hq + hq)], (unsigned)nvis);
    atomicAdd(&a.counters[2 * (b * g.Hq + hq) + 1], (unsigned)pol.nskip);
  }
}

template <int D, int NW, int QB>
hipError_t launch_t(const SkipArgs& a, hipStream_t stream) {
  constexpr int BR = NW * 32 * QB;
  const int nQT = (a.g.Sq + BR - 1) / BR;
  const int total = a.g.B * a.g.Hq * nQT;
  hipLaunchKernelGGL((skip_softmax_kernel<D, NW, QB>), dim3(total), dim3(NW * 64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

// Query tiles of block_q rows run as block_q/32 wavefronts of 32 rows each (kQueryBlocksPerWave =
// 1): the per-wave state then fits in half the register file, so two workgroups share each CU and
// one's MFMA work overlaps the other's softmax arithmetic.
hipError_t launch_skip_softmax(const SkipArgs& a, hipStream_t stream) {
  constexpr int QB = kQueryBlocksPerWave;
  const bool q128 = a.g.block_q == 128;
  if (a.g.D == 128)
    return q128 ? launch_t<128, 4 / QB, QB>(a, stream) : launch_t<128, 2 / QB, QB>(a, stream);
  return q128 ? launch_t<64, 4 / QB, QB>(a, stream) : launch_t<64, 2 / QB, QB>(a, stream);
}

}  // namespace sa
