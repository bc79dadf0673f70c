// proxy.hip -- proxy-compensated block-sparse flash-attention forward for gfx950.
//
// Method: FlashInfer block-sparse proxy description quoted in the TensorRT-LLM "add VisualGen SOL
// sparse attention" PR ("Description", "Bitmask format"): selected KV blocks are attended exactly;
// every omitted KV block is approximated by one arithmetic-mean K summary and one summed-V summary,
// and the softmax denominator is corrected by the token mass the summary represents, including the
// true length of the final partial block.  For a query q:
//     O = [sum_t e^{s_t} v_t + sum_j e^{s^_j} Vsum_j] / [sum_t e^{s_t} + sum_j c_j e^{s^_j}],
//     s = scale * q.k,  c_j = min(Bk, Sk - j*Bk).
//
// One workgroup = one (batch, query head, query block).  The exact part walks the route stream
// (n_exact, exact_idx) of the query block's (batch, KV head) row: each exact block is one or two
// 64-key tiles of raw K/V.  The proxy part, when enabled, treats the summary rows as keys: tiles of
// 64 summaries (K = k_mean rows, V = v_sum rows), rows whose proxy_keep bit is clear masked to
// -inf, and the row sum weighted by c_j.  Both parts share the online softmax state.
#include "kernels.h"
#include "tile_core.h"

namespace sa {
namespace {

template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void proxy_kernel(ProxyArgs a) {
  constexpr int BR = NW * kRowsPerWave;
  constexpr int NT = NW * 64;
  __shared__ __attribute__((aligned(16))) char ldsK[kKeysPerTile * D * 2];
  __shared__ __attribute__((aligned(16))) char ldsV[kKeysPerTile * D * 2];

  const AttnGeom& g = a.g;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, r32 = lane & 31;
  const int Bk = g.block_k;
  const int nQB = (g.Sq + BR - 1) / BR;
  const int nKB = (g.Sk + Bk - 1) / Bk;
  const int Wd = (nKB + 31) / 32;
  const int G = g.Hq / g.Hkv;
  const int total = g.B * g.Hq * nQB;

  int item = xcd_remap(blockIdx.x, total);
  const int gq = item % G;
  item /= G;
  const int qb_blk = item % nQB;
  item /= nQB;
  const int hk = item % g.Hkv;
  const int b = item / g.Hkv;
  const int hq = hk * G + gq;

  const int row0 = qb_blk * BR;
  const int wrow0 = row0 + wave * kRowsPerWave;
  const int wrows = g.Sq - wrow0;
  const int64_t route_row = ((int64_t)b * g.Hkv + hk) * nQB + qb_blk;
  const int n_exact = min(max(a.n_exact[route_row], 0), nKB);   // never index past the row
  const int32_t* exact = a.exact_idx + route_row * nKB;
  const uint32_t* keep_bits = a.proxy_keep + route_row * Wd;

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

  const int sub = Bk / kKeysPerTile;                       // 64-key tiles per semantic block
  const int n_proxy_tiles = a.use_proxy ? (nKB + kKeysPerTile - 1) / kKeysPerTile : 0;
  const int n_steps = n_exact * sub + n_proxy_tiles;
  const int last_len = g.Sk - (nKB - 1) * Bk;              // tokens in the final (partial) block

  for (int step = 0; step < n_steps; ++step) {
    const bool proxy = step >= n_exact * sub;
    int k0;
    if (!proxy) {
      k0 = exact[step / sub] * Bk + (step % sub) * kKeysPerTile;
      stage_tile<D, NT>(ldsK, ksrc, g.ks[1], k0, tid);
      stage_tile<D, NT>(ldsV, vsrc, g.vs[1], k0, tid);
    } else {
      k0 = (step - n_exact * sub) * kKeysPerTile;           // first summary row of the tile
      const int64_t sbase = ((int64_t)b * g.Hkv + hk) * nKB * D;
      const auto kmsrc = slab_rsrc((const __bf16*)a.k_mean + sbase, D, nKB, D);
      const auto vssrc = slab_rsrc((const __bf16*)a.v_sum + sbase, D, nKB, D);
      stage_tile<D, NT>(ldsK, kmsrc, D, k0, tid);
      stage_tile<D, NT>(ldsV, vssrc, D, k0, tid);
    }
    __syncthreads();

    f32x16 s[2][2];
    qk_tile<D>(ldsK, qf, s, lane);

    if (!proxy) {
      // keys past Sk (final partial block) -> -inf
      if (k0 + kKeysPerTile > g.Sk) {
        const int lim = g.Sk - k0 - 4 * h;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (kb * 32 + (r >> 2) * 8 + (r & 3) >= lim) s[kb][qb][r] = -INFINITY;
      }
    } else {
      // summaries not selected by proxy_keep (or past nKB) -> -inf
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int wd = (k0 >> 5) + kb;
        uint32_t bits = 0u;
        if (wd < Wd) {
          const int nbits = nKB - 32 * wd;   // >= 1; clears stray padding bits
          bits = keep_bits[wd] & (nbits >= 32 ? 0xFFFFFFFFu : ((1u << nbits) - 1u));
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int bit = (r >> 2) * 8 + 4 * h + (r & 3);
          if (!((bits >> bit) & 1u)) {
            s[kb][0][r] = -INFINITY;
            s[kb][1][r] = -INFINITY;
          }
        }
      }
    }

    float M_[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][qb][r]);
      M_[qb] = half_max(mx) * g.c32;
    }
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const float m_new = fmaxf(m[qb], M_[qb]);
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
          if (!proxy) {
            rs += p;
          } else {
            // token mass of summary row j: the full block, or the final block's true length
            const int j = k0 + tile_key(kb, r, lane);
            rs += p * (float)(j == nKB - 1 ? last_len : Bk);
          }
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
    pv_tile<D>(ldsV, pb, o, lane);
    __syncthreads();
  }

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
}

template <int D, int NW>
hipError_t launch_t(const ProxyArgs& a, hipStream_t stream) {
  constexpr int BR = NW * kRowsPerWave;
  const int nQB = (a.g.Sq + BR - 1) / BR;
  const int total = a.g.B * a.g.Hq * nQB;
  hipLaunchKernelGGL((proxy_kernel<D, NW>), dim3(total), dim3(NW * 64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_proxy(const ProxyArgs& a, hipStream_t stream) {
  const bool q128 = a.g.block_q == 128;
  if (a.g.D == 128) return q128 ? launch_t<128, 2>(a, stream) : launch_t<128, 1>(a, stream);
  return q128 ? launch_t<64, 2>(a, stream) : launch_t<64, 1>(a, stream);
}

}  // namespace sa
