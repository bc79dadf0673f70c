// nm_softmax.hip -- N:M sparse softmax flash-attention forward for gfx950.
//
// Method: Model-Optimizer "Attention Sparsity for HuggingFace Models", "N:M Sparse Softmax": for
// every M consecutive key positions keep the top-N attention scores and set the rest to -inf
// before the softmax; the first dense_sink_tokens keys and a window of dense_recent_tokens recent
// keys stay dense; M = 4 (N = 1..3) or M = 8 (N = 1..7); prefill only.  Readings (stated in sa.h):
// groups aligned to key 0, ranking by the raw score q.k among all members of the group (masked
// keys rank last), ties to the lower key index, "recent" = 0 <= row - key < R.
//
// Same pipelined loop as the skip-softmax kernel (mainloop.h), every visited tile kept.  In the S^T register
// layout a lane holds, for one query, keys 8g + 4h + {0..3} in elements 4g..4g+3 (h = lane/32), so
// an M = 4 group is four consecutive elements of one lane and an M = 8 group is those four plus the
// same four elements of lane ^ 32 (one v_permlane32_swap).  Dropped keys get weight 0 in P.  The
// running max needs no change: the group maximum always survives (rank 0 < N), so the max over
// kept keys equals the max over allowed keys.
#include "kernels.h"
#include "mainloop.h"

namespace sa {
namespace {

// 1 when d < 0, else 0, for d the fp32 difference of two finite scores normalised by "+ 0.0f"
// (so that equal scores give +0): the sign bit, read without a compare (a compare per pair would
// park a lane mask in SGPRs).
__device__ __forceinline__ int neg01(float d) { return (int)(__float_as_uint(d + 0.0f) >> 31); }

// rank[i] = number of group members that beat own[i]: a higher score, or an equal score at a lower
// key index.  own[0..3] are this lane's four keys in ascending key order; for M = 8, oth[0..3] are
// the lane ^ 32 half of the group, whose keys all come after ours when own_first is true.  Scores
// are finite here (masked keys enter as -FLT_MAX, which still ties only with other masked keys).
template <int M>
__device__ __forceinline__ void group_ranks(const float (&own)[4], const float (&oth)[4],
                                            bool own_first, int (&rank)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) rank[i] = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = i + 1; j < 4; ++j) {
      // j comes after i: j beats i iff own[j] > own[i], otherwise i beats j
      const int jgt = neg01(own[i] - own[j]);
      rank[i] += jgt;
      rank[j] += 1 - jgt;
    }
  if constexpr (M == 8) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // other half after ours: it beats own[i] iff strictly greater; before ours: iff >=
        const int gt = neg01(own[i] - oth[j]);   // oth[j] > own[i]
        const int lt = neg01(oth[j] - own[i]);   // oth[j] < own[i]
        rank[i] += own_first ? gt : 1 - lt;
      }
  }
}

// This lane's 32 keys of a 64-key tile, bit b = kb*16 + r, sit at key offsets
// p(b) = kb*32 + (r/4)*8 + 4h + r%4, which increase with b: the keys with offset < T are the
// low bits, as many as there are such offsets.
__device__ __forceinline__ uint32_t bits_below(int T, int h) {
  int cnt = 0;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int q = 0; q < 4; ++q) cnt += min(max(T - (kb * 32 + q * 8 + 4 * h), 0), 4);
  return cnt >= 32 ? 0xFFFFFFFFu : ((1u << cnt) - 1u);
}

template <int D, int NW, int QB, int M>
struct NmPolicy {
  static constexpr bool kDecide = false, kFilter = true, kWeighted = false;
  static constexpr int RW = 32 * QB;   // rows per wave
  const __bf16* kslab;
  const __bf16* vslab;
  int k_stride_b, v_stride_b, k_bytes, v_bytes;
  int Sq, Sk, causal, wrow0, nvis, h, r32, n, sink, recent, W;
  uint32_t* keep_bits;
  float* scores;
  int64_t row_base;   // (b*Hq + hq)*Sq

  __device__ __forceinline__ int steps() const { return nvis; }

  __device__ __forceinline__ TileSrc src(int j) const {
    const int k0 = j * kKeysPerTile;
    return TileSrc{kslab + (int64_t)k0 * (k_stride_b / 2), vslab + (int64_t)k0 * (v_stride_b / 2),
                   max(0, k_bytes - k0 * k_stride_b), max(0, v_bytes - k0 * v_stride_b),
                   k_stride_b, v_stride_b};
  }

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

  // keep bit (kb*16 + r) of bits[qb]: key not masked and (dense, or top-n of its group).  The
  // ranks are sign-bit arithmetic per element; the sink/recent windows and masked keys are key
  // ranges, turned into bit ranges (bits_below) on the few tiles per row that touch them.
  __device__ __forceinline__ void filter(int j, const f32x16 (&s)[2][QB], uint32_t (&bits)[QB],
                                         int lane) const {
    const int k0 = j * kKeysPerTile;
    const bool any_masked = (k0 + kKeysPerTile > Sk) || (causal && k0 + kKeysPerTile - 1 > wrow0);
    const bool any_dense = k0 < sink ||
        (recent > 0 && k0 <= wrow0 + RW - 1 && k0 + kKeysPerTile - 1 > wrow0 - recent);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int row = wrow0 + qb * 32 + r32;
      uint32_t kb_bits = 0u;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int gi = 0; gi < 4; ++gi) {
          float own[4], oth[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            own[e] = fmaxf(s[kb][qb][4 * gi + e], -3.402823466e38f);   // masked: finite sentinel
            oth[e] = own[e];
            if constexpr (M == 8) oth[e] = other_half(own[e], lane);
          }
          int rank[4];
          group_ranks<M>(own, oth, h == 0, rank);
#pragma unroll
          for (int e = 0; e < 4; ++e)   // top-n: rank - n < 0
            kb_bits |= ((uint32_t)(rank[e] - n) >> 31) << (kb * 16 + 4 * gi + e);
          // one group at a time: the scheduler would otherwise interleave all eight groups'
          // comparisons and run out of registers
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if (any_dense) {   // key < sink, or row - recent < key <= row
        kb_bits |= bits_below(sink - k0, h);
        if (recent > 0) kb_bits |= bits_below(row - k0 + 1, h) & ~bits_below(row - recent - k0 + 1, h);
      }
      if (any_masked)    // key < Sk and (causal) key <= row
        kb_bits &= bits_below(causal ? min(Sk, row + 1) - k0 : Sk - k0, h);
      bits[qb] = kb_bits;
      if (keep_bits != nullptr || scores != nullptr) export_row(k0, row, qb, kb_bits, s, lane);
    }
  }

  // debug exports of one query row: keep-bit words and raw scores
  __device__ __forceinline__ void export_row(int k0, int row, int qb, uint32_t kb_bits,
                                             const f32x16 (&s)[2][QB], int lane) const {
    // lanes l and l^32 hold the same row: both stay active through the swap
    const int64_t rbase = row_base + row;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      // this lane's 16 bits sit at key offsets (r/4)*8 + 4h + r%4: spread the nibbles 8 apart,
      // then shift by 4h; merged with lane^32's half
      const uint32_t x = (kb_bits >> (kb * 16)) & 0xFFFFu;
      uint32_t word = ((x & 0xFu) | ((x & 0xF0u) << 4) | ((x & 0xF00u) << 8) |
                       ((x & 0xF000u) << 12)) << (4 * h);
      word |= __float_as_uint(other_half(__uint_as_float(word), lane));
      if (row < Sq) {
        if (keep_bits != nullptr && h == 0 && k0 + kb * 32 < Sk)
          keep_bits[rbase * W + k0 / 32 + kb] = word;
        if (scores != nullptr) {
          int kbase = k0 + 4 * h;   // key = kbase + c, c a compile-time constant
          asm volatile("" : "+v"(kbase));
          float* dst = scores + rbase * Sk + kbase;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int c = kb * 32 + (r >> 2) * 8 + (r & 3);
            if (kbase + c < Sk) dst[c] = s[kb][qb][r];
          }
        }
      }
    }
  }

  __device__ __forceinline__ bool negligible(const float (&)[QB], const float (&)[QB], int) const {
    return false;
  }
  __device__ __forceinline__ void record(int, bool, const float (&)[QB], int, int, bool) {}
};

template <int D, int NW, int QB, int M>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(kWavesPerSimd<QB>)))
void nm_softmax_kernel(NmArgs a) {
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
  const int W = (g.Sk + 31) / 32;

  const auto qsrc = slab_rsrc((const __bf16*)g.q + b * g.qs[0] + hq * g.qs[2], g.qs[1], g.Sq, D);
  bf16x8 qf[QB][D / 16];
  load_q_frags<D, QB>(qf, qsrc, g.qs[1], wrow0, lane);

  NmPolicy<D, NW, QB, M> pol;
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
  pol.h = h;
  pol.r32 = r32;
  pol.n = a.n;
  pol.sink = a.sink;
  pol.recent = a.recent;
  pol.W = W;
  pol.keep_bits = a.keep_bits;
  pol.scores = a.scores;
  pol.row_base = ((int64_t)b * g.Hq + hq) * g.Sq;

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

  // keep-bit words and scores of tiles never visited (causal): zero / -inf
  if (a.keep_bits != nullptr) {
    const int wfirst = nvis * (kKeysPerTile / 32);
    for (int rr = tid; rr < BR; rr += NT) {
      const int row = row0 + rr;
      if (row >= g.Sq) continue;
      const int64_t rbase = pol.row_base + row;
      for (int w = wfirst; w < W; ++w) a.keep_bits[rbase * W + w] = 0u;
    }
  }
  if (a.scores != nullptr) {
    const int kfirst = nvis * kKeysPerTile;
    for (int rr = 0; rr < BR; ++rr) {
      const int row = row0 + rr;
      if (row >= g.Sq) break;
      const int64_t rbase = pol.row_base + row;
      for (int key = kfirst + tid; key < g.Sk; key += NT) a.scores[rbase * g.Sk + key] = -INFINITY;
    }
  }

  float inv[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lt = half_sum(l[qb]);
    inv[qb] = lt > 0.f ? 1.f / lt : 0.f;
    const int row = wrow0 + qb * 32 + r32;
    if (a.lse != nullptr && h == 0 && row < g.Sq)
      a.lse[pol.row_base + row] =
          lt > 0.f ? (mref[qb] + __log2f(lt)) * 0.69314718055994531f : -INFINITY;
  }
  __bf16* op = (__bf16*)g.o + b * g.os[0] + (int64_t)wrow0 * g.os[1] + hq * g.os[2];
  store_o<D, QB>(op, g.os[1], g.Sq - wrow0, o, inv, lane);
}

template <int D, int NW, int QB, int M>
hipError_t launch_t(const NmArgs& a, hipStream_t stream) {
  constexpr int BR = NW * 32 * QB;
  const int nQT = (a.g.Sq + BR - 1) / BR;
  const int total = a.g.B * a.g.Hq * nQT;
  hipLaunchKernelGGL((nm_softmax_kernel<D, NW, QB, M>), dim3(total), dim3(NW * 64), 0, stream, a);
  return hipGetLastError();
}

template <int D, int NW, int QB>
hipError_t launch_m(const NmArgs& a, hipStream_t stream) {
  return a.m == 8 ? launch_t<D, NW, QB, 8>(a, stream) : launch_t<D, NW, QB, 4>(a, stream);
}

}  // namespace

hipError_t launch_nm_softmax(const NmArgs& a, hipStream_t stream) {
  constexpr int QB = kQueryBlocksPerWave;
  const bool q128 = a.g.block_q == 128;
  if (a.g.D == 128)
    return q128 ? launch_m<128, 4 / QB, QB>(a, stream) : launch_m<128, 2 / QB, QB>(a, stream);
  return q128 ? launch_m<64, 4 / QB, QB>(a, stream) : launch_m<64, 2 / QB, QB>(a, stream);
}

}  // namespace sa
