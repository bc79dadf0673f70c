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
// One workgroup = one (batch, query head, query tile of 64*NW rows); each wavefront owns 64 rows.
// Per visited key tile: stage K in LDS -> S^T = K.Q^T on MFMA -> mask -> row max (in-lane +
// permlane32 swap) -> per-wave ballot of "some row not negligible" -> one LDS flag per wave ->
// workgroup-uniform keep/skip.  Only a kept tile stages V and runs exp2 + P.V.
#include "kernels.h"
#include "tile_core.h"

namespace sa {
namespace {

template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void skip_softmax_kernel(SkipArgs a) {
  constexpr int BR = NW * kRowsPerWave;
  constexpr int NT = NW * 64;
  __shared__ __attribute__((aligned(16))) char ldsK[kKeysPerTile * D * 2];
  __shared__ __attribute__((aligned(16))) char ldsV[kKeysPerTile * D * 2];
  __shared__ int keep_flag[NW];

  const AttnGeom& g = a.g;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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
  const int wrow0 = row0 + wave * kRowsPerWave;
  const int wrows = g.Sq - wrow0;                 // valid rows of this wave (may exceed 64)
  const int last_row = min(row0 + BR, g.Sq) - 1;
  const int nvis = g.causal ? min(nKT, last_row / kKeysPerTile + 1) : nKT;
  const int64_t unit = ((int64_t)b * g.Hq + hq) * nQT + qt;

  const auto qsrc = slab_rsrc((const __bf16*)g.q + b * g.qs[0] + hq * g.qs[2], g.qs[1], g.Sq, D);
  const auto ksrc = slab_rsrc((const __bf16*)g.k + b * g.ks[0] + hk * g.ks[2], g.ks[1], g.Sk, D);
  const auto vsrc = slab_rsrc((const __bf16*)g.v + b * g.vs[0] + hk * g.vs[2], g.vs[1], g.Sk, D);

  bf16x8 qf[2][D / 16];
  load_q_frags<D>(qf, qsrc, g.qs[1], wrow0, lane);

  f32x16 o[D / 32][2];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) o[db][0] = o[db][1] = f32x16{};
  float m[2] = {-INFINITY, -INFINITY};
  float l[2] = {0.f, 0.f};
  int nskip = 0;

  for (int j = 0; j < nvis; ++j) {
    const int k0 = j * kKeysPerTile;
    stage_tile<D, NT>(ldsK, ksrc, g.ks[1], k0, tid);
    __syncthreads();

    f32x16 s[2][2];
    qk_tile<D>(ldsK, qf, s, lane);

    const bool need_mask = (k0 + kKeysPerTile > g.Sk) ||
                           (g.causal && k0 + kKeysPerTile - 1 > wrow0);
    if (need_mask) {
      // key = k0 + 4*h + off(kb, r) with off a compile-time constant; a key is masked when
      // off >= lim[qb] (beyond Sk, or beyond the row under causal masking).
      const int klim = g.Sk - k0 - 4 * h;
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        int lim = klim;
        if (g.causal) lim = min(lim, wrow0 + qb * 32 + r32 - k0 - 4 * h + 1);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (kb * 32 + (r >> 2) * 8 + (r & 3) >= lim) s[kb][qb][r] = -INFINITY;
      }
    }

    // Tile row maxima in the log2 domain and the negligibility test.
    float M[2];
    bool negligible = true;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][qb][r]);
      M[qb] = half_max(mx) * g.c32;
      const float thr = m[qb] + a.L32;
      if (wrow0 + qb * 32 + r32 < g.Sq && !(M[qb] < thr)) negligible = false;
    }
    const bool wave_keep = __builtin_amdgcn_ballot_w64(!negligible) != 0ull;
    if (lane == 0) keep_flag[wave] = wave_keep ? 1 : 0;
    if (a.rowmax != nullptr && h == 0) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
        a.rowmax[(unit * nKT + j) * BR + wave * kRowsPerWave + qb * 32 + r32] = M[qb];
    }
    __syncthreads();
    int keep = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) keep |= keep_flag[w];
    if (tid == 0 && a.tile_state != nullptr) a.tile_state[unit * nKT + j] = keep ? 0 : 1;
    if (!keep) {
      ++nskip;
      continue;
    }

    stage_tile<D, NT>(ldsV, vsrc, g.vs[1], k0, tid);

    // Online softmax update with the kept tile.
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const float m_new = fmaxf(m[qb], M[qb]);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m[qb] - m_use);
      l[qb] *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) o[db][qb] *= alpha;
      m[qb] = m_new;
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = __builtin_amdgcn_exp2f(s[kb][qb][r] * g.c32 - m_use);
          s[kb][qb][r] = p;
          rs += p;
        }
      l[qb] += rs;
    }
    bf16x8 pb[2][2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) pb[kb][c][qb] = p_operand(s[kb][qb], c);

    __syncthreads();   // V tile staged
    pv_tile<D>(ldsV, pb, o, lane);
  }

  // Epilogue: normalise, store O and the natural-log LSE.
  float inv[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float lt = half_sum(l[qb]);
    inv[qb] = lt > 0.f ? 1.f / lt : 0.f;
    const int row = wrow0 + qb * 32 + r32;
    if (a.lse != nullptr && h == 0 && row < g.Sq)
      a.lse[((int64_t)b * g.Hq + hq) * g.Sq + row] =
          lt > 0.f ? (m[qb] + __log2f(lt)) * 0.69314718055994531f : -INFINITY;
  }
  __bf16* op = (__bf16*)g.o + b * g.os[0] + (int64_t)wrow0 * g.os[1] + hq * g.os[2];
  store_o<D>(op, g.os[1], wrows, o, inv, lane);

  if (a.tile_state != nullptr)
    for (int j = nvis + tid; j < nKT; j += NT) a.tile_state[unit * nKT + j] = 2;
  if (a.rowmax != nullptr)
    for (int64_t i = (int64_t)nvis * BR + tid; i < (int64_t)nKT * BR; i += NT)
      a.rowmax[unit * nKT * BR + i] = -INFINITY;
  if (tid == 0 && a.counters != nullptr) {
    atomicAdd(&a.counters[2 * (b * g.Hq + hq)], (unsigned)nvis);
    atomicAdd(&a.counters[2 * (b * g.Hq + hq) + 1], (unsigned)nskip);
  }
}

template <int D, int NW>
hipError_t launch_t(const SkipArgs& a, hipStream_t stream) {
  constexpr int BR = NW * kRowsPerWave;
  const int nQT = (a.g.Sq + BR - 1) / BR;
  const int total = a.g.B * a.g.Hq * nQT;
  hipLaunchKernelGGL((skip_softmax_kernel<D, NW>), dim3(total), dim3(NW * 64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_skip_softmax(const SkipArgs& a, hipStream_t stream) {
  const bool q128 = a.g.block_q == 128;
  if (a.g.D == 128) return q128 ? launch_t<128, 2>(a, stream) : launch_t<128, 1>(a, stream);
  return q128 ? launch_t<64, 2>(a, stream) : launch_t<64, 1>(a, stream);
}

}  // namespace sa
