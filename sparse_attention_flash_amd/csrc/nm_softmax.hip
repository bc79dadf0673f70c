// nm_softmax.hip -- N:M sparse softmax flash-attention forward for gfx950.
//
// Method: Model-Optimizer "Attention Sparsity for HuggingFace Models", "N:M Sparse Softmax": for
// every M consecutive key positions keep the top-N attention scores and set the rest to -inf
// before the softmax; the first dense_sink_tokens keys and a window of dense_recent_tokens recent
// keys stay dense; M = 4 (N = 1..3) or M = 8 (N = 1..7); prefill only.  Readings (stated in sa.h):
// groups aligned to key 0, ranking by the raw score q.k among all members of the group (masked
// keys rank last), ties to the lower key index, "recent" = 0 <= row - key < R.
//
// Same tile skeleton as the skip-softmax kernel, every visited tile kept.  In the S^T register
// layout a lane holds, for one query, keys 8g + 4h + {0..3} in elements 4g..4g+3 (h = lane/32), so
// an M = 4 group is four consecutive elements of one lane and an M = 8 group is those four plus the
// same four elements of lane ^ 32 (one v_permlane32_swap).  Dropped keys get weight 0 in P.  The
// running max needs no change: the group maximum always survives (rank 0 < N), so the max over
// kept keys equals the max over allowed keys.
#include "kernels.h"
#include "tile_core.h"

namespace sa {
namespace {

// Number of elements of the group that beat element i (higher score, or equal score and lower key
// index).  own[0..3] are this lane's four keys in ascending key order; for M = 8, oth[0..3] are the
// lane ^ 32 half of the group, whose keys all come before ours when own_first is false.
template <int M>
__device__ __forceinline__ void group_ranks(const float (&own)[4], const float (&oth)[4],
                                            bool own_first, int (&rank)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int rk = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (j == i) continue;
      rk += (j < i) ? (own[j] >= own[i]) : (own[j] > own[i]);
    }
    if constexpr (M == 8) {
#pragma unroll
      for (int j = 0; j < 4; ++j) rk += own_first ? (oth[j] > own[i]) : (oth[j] >= own[i]);
    }
    rank[i] = rk;
  }
}

template <int D, int NW, int M>
__global__ __launch_bounds__(NW * 64) void nm_softmax_kernel(NmArgs a) {
  constexpr int BR = NW * kRowsPerWave;
  constexpr int NT = NW * 64;
  __shared__ __attribute__((aligned(16))) char ldsK[kKeysPerTile * D * 2];
  __shared__ __attribute__((aligned(16))) char ldsV[kKeysPerTile * D * 2];

  const AttnGeom& g = a.g;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, r32 = lane & 31;
  const int nQT = (g.Sq + BR - 1) / BR;
  const int nKT = (g.Sk + kKeysPerTile - 1) / kKeysPerTile;
  const int G = g.Hq / g.Hkv;
  const int total = g.B * g.Hq * nQT;

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
  const int wrows = g.Sq - wrow0;
  const int last_row = min(row0 + BR, g.Sq) - 1;
  const int nvis = g.causal ? min(nKT, last_row / kKeysPerTile + 1) : nKT;
  const int W = (g.Sk + 31) / 32;

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

  for (int j = 0; j < nvis; ++j) {
    const int k0 = j * kKeysPerTile;
    stage_tile<D, NT>(ldsK, ksrc, g.ks[1], k0, tid);
    stage_tile<D, NT>(ldsV, vsrc, g.vs[1], k0, tid);
    __syncthreads();

    f32x16 s[2][2];
    qk_tile<D>(ldsK, qf, s, lane);

    // causal / out-of-range keys -> -inf (same limit form as the skip kernel)
    const bool need_mask = (k0 + kKeysPerTile > g.Sk) ||
                           (g.causal && k0 + kKeysPerTile - 1 > wrow0);
    if (need_mask) {
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

    // keep mask: bit (kb*16 + r) of keep[qb]
    uint32_t keep[2] = {0u, 0u};
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int row = wrow0 + qb * 32 + r32;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int gi = 0; gi < 4; ++gi) {
          float own[4], oth[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            own[e] = s[kb][qb][4 * gi + e];
            oth[e] = own[e];
            if constexpr (M == 8) oth[e] = other_half(own[e], lane);
          }
          int rank[4];
          group_ranks<M>(own, oth, h == 0, rank);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int key = k0 + kb * 32 + gi * 8 + 4 * h + e;
            const bool dense = key < a.sink || (row - key >= 0 && row - key < a.recent);
            const bool masked = key >= g.Sk || (g.causal && key > row);
            if (!masked && (dense || rank[e] < a.n)) keep[qb] |= 1u << (kb * 16 + 4 * gi + e);
          }
        }
      }
    }

    if (a.keep_bits != nullptr || a.scores != nullptr) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const int row = wrow0 + qb * 32 + r32;
        if (row >= g.Sq) continue;
        const int64_t rbase = ((int64_t)b * g.Hq + hq) * g.Sq + row;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          // this lane's 16 bits of the 32-key word k0/32 + kb, merged with the other half's
          uint32_t word = 0u;
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if ((keep[qb] >> (kb * 16 + r)) & 1u) word |= 1u << ((r >> 2) * 8 + 4 * h + (r & 3));
          word |= __float_as_uint(other_half(__uint_as_float(word), lane));
          if (a.keep_bits != nullptr && h == 0 && k0 + kb * 32 < g.Sk)
            a.keep_bits[rbase * W + k0 / 32 + kb] = word;
          if (a.scores != nullptr) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = k0 + tile_key(kb, r, lane);
              if (key < g.Sk) a.scores[rbase * g.Sk + key] = s[kb][qb][r];
            }
          }
        }
      }
    }

    // online softmax; dropped keys contribute exactly 0
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
          const float e = __builtin_amdgcn_exp2f(s[kb][qb][r] * g.c32 - m_use);
          const float p = ((keep[qb] >> (kb * 16 + r)) & 1u) ? e : 0.f;
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
    pv_tile<D>(ldsV, pb, o, lane);
    __syncthreads();   // all waves done with this K/V tile before it is overwritten
  }

  // keep-bit words of tiles never visited (causal): all zero
  if (a.keep_bits != nullptr) {
    const int wfirst = nvis * (kKeysPerTile / 32);
    for (int rr = tid; rr < BR; rr += NT) {
      const int row = row0 + rr;
      if (row >= g.Sq) continue;
      const int64_t rbase = ((int64_t)b * g.Hq + hq) * g.Sq + row;
      for (int w = wfirst; w < W; ++w) a.keep_bits[rbase * W + w] = 0u;
    }
  }
  if (a.scores != nullptr) {
    const int kfirst = nvis * kKeysPerTile;
    for (int rr = 0; rr < BR; ++rr) {
      const int row = row0 + rr;
      if (row >= g.Sq) break;
      const int64_t rbase = ((int64_t)b * g.Hq + hq) * g.Sq + row;
      for (int key = kfirst + tid; key < g.Sk; key += NT) a.scores[rbase * g.Sk + key] = -INFINITY;
    }
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

template <int D, int NW, int M>
hipError_t launch_t(const NmArgs& a, hipStream_t stream) {
  constexpr int BR = NW * kRowsPerWave;
  const int nQT = (a.g.Sq + BR - 1) / BR;
  const int total = a.g.B * a.g.Hq * nQT;
  hipLaunchKernelGGL((nm_softmax_kernel<D, NW, M>), dim3(total), dim3(NW * 64), 0, stream, a);
  return hipGetLastError();
}

template <int D, int NW>
hipError_t launch_m(const NmArgs& a, hipStream_t stream) {
  return a.m == 8 ? launch_t<D, NW, 8>(a, stream) : launch_t<D, NW, 4>(a, stream);
}

}  // namespace

hipError_t launch_nm_softmax(const NmArgs& a, hipStream_t stream) {
  const bool q128 = a.g.block_q == 128;
  if (a.g.D == 128) return q128 ? launch_m<128, 2>(a, stream) : launch_m<128, 1>(a, stream);
  return q128 ? launch_m<64, 2>(a, stream) : launch_m<64, 1>(a, stream);
}

}  // namespace sa
