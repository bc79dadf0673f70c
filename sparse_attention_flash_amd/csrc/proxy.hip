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
// One workgroup = one (batch, query head, query block), on the pipelined loop of mainloop.h.  The
// steps are first the exact blocks of the route stream (n_exact, exact_idx) of the query block's
// (batch, KV head) row, each one or two 64-key tiles of raw K/V, then, when enabled, the proxy
// tiles: 64 summary rows at a time (K = k_mean rows, V = v_sum rows), rows whose proxy_keep bit is
// clear masked to -inf, and the row sum weighted by c_j.  Both parts share the online softmax.
#include "kernels.h"
#include "mainloop.h"

namespace sa {
namespace {

// Exact steps (pipelined main loop): the 64-key tiles of the exact blocks, in ascending order.
template <int D, int NW, int QB>
struct ExactPolicy {
  static constexpr bool kDecide = false, kFilter = false, kWeighted = false;
  const __bf16* kslab;
  const __bf16* vslab;
  const int32_t* exact;  // ascending exact block indices of this query block
  int k_stride_b, v_stride_b, k_bytes, v_bytes;
  int Sk, Bk, sub, n_exact, nKB, h;

  // the route row of query block route_row of (b, KV head hk); a row that is not present (the
  // missing half of a 64-row pair) has no steps
  __device__ __forceinline__ void init(const ProxyArgs& a, int b, int hk, int64_t route_row,
                                       int nKB, int lane_half, bool present = true) {
    const AttnGeom& g = a.g;
    kslab = (const __bf16*)g.k + b * g.ks[0] + hk * g.ks[2];
    vslab = (const __bf16*)g.v + b * g.vs[0] + hk * g.vs[2];
    exact = a.exact_idx + route_row * nKB;
    k_stride_b = (int)(g.ks[1] * 2);
    v_stride_b = (int)(g.vs[1] * 2);
    k_bytes = (int)(((int64_t)(g.Sk - 1) * g.ks[1] + D) * 2);
    v_bytes = (int)(((int64_t)(g.Sk - 1) * g.vs[1] + D) * 2);
    Sk = g.Sk;
    Bk = g.block_k;
    sub = Bk / kKeysPerTile;
    // never index past the route row, whatever the caller passed
    n_exact = present ? min(max(__builtin_amdgcn_readfirstlane(a.n_exact[route_row]), 0), nKB) : 0;
    this->nKB = nKB;
    h = lane_half;
  }

  __device__ __forceinline__ int steps() const { return n_exact * sub; }

  // A block index outside [0, nKB) (the -1 fill after a route's real entries, read when the
  // caller's n_exact exceeds them, or any other bad value) becomes an empty step: it is placed at
  // block nKB, past the last key, so its copies read no bytes and mask() drops every key.
  __device__ __forceinline__ int first_key(int step) const {
    int blk = __builtin_amdgcn_readfirstlane(exact[step / sub]);
    if ((unsigned)blk >= (unsigned)nKB) blk = nKB;
    return blk * Bk + (step % sub) * kKeysPerTile;
  }

  __device__ __forceinline__ TileSrc src(int step) const {
    const int k0 = first_key(step);
    return TileSrc{kslab + (int64_t)k0 * (k_stride_b / 2), vslab + (int64_t)k0 * (v_stride_b / 2),
                   max(0, k_bytes - k0 * k_stride_b), max(0, v_bytes - k0 * v_stride_b),
                   k_stride_b, v_stride_b};
  }

  // keys past Sk exist only in the final partial block
  __device__ __forceinline__ void mask(int step, f32x16 (&s)[2][QB], int) const {
    const int k0 = first_key(step);
    if (k0 + kKeysPerTile <= Sk) return;
    const int lim = Sk - k0 - 8 * h;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) mask_block(s[kb][qb], kb, lim);
  }

  __device__ __forceinline__ bool negligible(const float (&)[QB], const float (&)[QB], int) const {
    return false;
  }
  __device__ __forceinline__ void filter(int, f32x16 (&)[2][QB], int) const {}
  __device__ __forceinline__ void record(int, bool, const float (&)[QB], int, int, bool) {}
};

// Proxy tiles: 64 summary rows at a time; rows whose proxy_keep bit is clear (or past nKB) are
// masked, and each kept row's row-sum term is weighted by its token mass c_j.
template <int QB>
struct SummaryPolicy {
  static constexpr bool kFilter = false, kWeighted = true;
  const uint32_t* keep;  // proxy_keep words of this query block
  int Bk, nKB, Wd, last_len, h;

  __device__ __forceinline__ void init(const ProxyArgs& a, int64_t route_row, int nKB_,
                                       int lane_half) {
    Bk = a.g.block_k;
    nKB = nKB_;
    Wd = (nKB + 31) / 32;
    keep = a.proxy_keep + route_row * Wd;
    last_len = a.g.Sk - (nKB - 1) * Bk;
    h = lane_half;
  }

  __device__ __forceinline__ bool weighted(int) const { return true; }

  __device__ __forceinline__ void mask(int t, f32x16 (&s)[2][QB]) const {
    const int r0 = t * kKeysPerTile;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int wd = (r0 >> 5) + kb;
      uint32_t bits = 0u;
      if (wd < Wd) {
        const int nbits = nKB - 32 * wd;   // >= 1; clears stray padding bits
        bits = keep[wd] & (nbits >= 32 ? 0xFFFFFFFFu : ((1u << nbits) - 1u));
      }
      const uint32_t lane_bits = bits >> (8 * h);   // element r holds bit (r/8)*16 + r%8 of these
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const uint32_t m = ((lane_bits >> ((r >> 3) * 16 + (r & 7))) & 1u) - 1u;   // ~0: drop
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[kb][qb][r] = select_neg_inf(s[kb][qb][r], m);
      }
    }
  }

  // token mass of summary row j: the full block, or the final block's true length
  __device__ __forceinline__ float weight(int t, int kb, int r, int lane) const {
    const int j = t * kKeysPerTile + tile_key(kb, r, lane);
    return (float)(j == nKB - 1 ? last_len : Bk);
  }
};

// Normalise and store this wave's rows of O and their natural-log LSE.
template <int D, int QB>
__device__ __forceinline__ void store_rows(const ProxyArgs& a, int b, int hq, int wrow0,
                                           const f32x16 (&o)[D / 32][QB], const float (&mref)[QB],
                                           const float (&l)[QB], int lane) {
  const AttnGeom& g = a.g;
  const int h = lane >> 5, r32 = lane & 31;
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
}

template <int D, int NW, int QB>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(kWavesPerSimd<QB>)))
void proxy_kernel(ProxyArgs a) {
  constexpr int RW = 32 * QB;
  constexpr int BR = NW * RW;
  __shared__ __attribute__((aligned(1024))) Smem<D, NW> sm;

  const AttnGeom& g = a.g;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5;
  const int Bk = g.block_k;
  const int nQB = (g.Sq + BR - 1) / BR;
  const int nKB = (g.Sk + Bk - 1) / Bk;
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
  const int wrow0 = row0 + wave * RW;
  const int64_t route_row = ((int64_t)b * g.Hkv + hk) * nQB + qb_blk;

  const auto qsrc = slab_rsrc((const __bf16*)g.q + b * g.qs[0] + hq * g.qs[2], g.qs[1], g.Sq, D);
  bf16x8 qf[QB][D / 16];
  load_q_frags<D, QB>(qf, qsrc, g.qs[1], wrow0, lane);

  ExactPolicy<D, NW, QB> pol;
  pol.init(a, b, hk, route_row, nKB, h);

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

  // proxy tiles: summaries as keys, one tile at a time
  if (a.use_proxy) {
    SummaryPolicy<QB> sp;
    sp.init(a, route_row, nKB, h);
    const int64_t sbase = ((int64_t)b * g.Hkv + hk) * nKB * D;
    const __bf16* kmean = (const __bf16*)a.k_mean + sbase;
    const __bf16* vsum = (const __bf16*)a.v_sum + sbase;
    const int n_tiles = (nKB + kKeysPerTile - 1) / kKeysPerTile;
    const auto sklo = Dma<KLayout<D>, NW>::lane_offsets(D * 2, wave, lane);
    const auto svlo = Dma<VLayout<D>, NW>::lane_offsets(D * 2, wave, lane);
    for (int t = 0; t < n_tiles; ++t) {
      const int r0 = t * kKeysPerTile;
      const int bytes = (nKB - r0) * D * 2;
      lds_barrier();   // every wave is done with the buffers the loop above (or tile t-1) used
      Dma<KLayout<D>, NW>::copy(sm.k[0], kmean + (int64_t)r0 * D, bytes, D * 2, sklo, wave);
      Dma<VLayout<D>, NW>::copy(sm.v[0], vsum + (int64_t)r0 * D, bytes, D * 2, svlo, wave);
      wait_vmcnt<0>();
      lds_barrier();
      f32x16 s[2][QB];
      qk_tile<D, QB>(sm.k[0], qf, s, lane);
      sp.mask(t, s);
      TileState<QB> ts;
      tile_row_max<QB>(s, g.c32, ts.M);
      ts.keep = true;
      softmax_pv<D, QB>(sp, t, s, ts, mref, l, o, sm.v[0], g.c32, lane);
    }
  }

  store_rows<D, QB>(a, b, hq, wrow0, o, mref, l, lane);
}

// ---- 64-row query blocks: copy waves and compute waves ------------------------------------------
// A 64-row block has two compute waves, and on those the K/V copies of every tile (16 per wave)
// took a large share of the time: each copy stalls its wave at issue while the vector-memory path
// is busy.  Here a workgroup of 8 waves takes two query blocks of the same (batch, query head),
// each with its own double-buffered K/V tiles (2 x 68 KB of LDS, one workgroup per CU).  Waves 0-3
// compute (two per query block) and waves 4-7 only copy (two per query block); waves w and w + 4
// share a SIMD, so every SIMD holds one compute wave and one copy wave.  Both blocks advance in
// lockstep through two barriers per step; the block with fewer exact tiles idles at the end.
//
//   copy waves:    K(0), V(0), K(1), V(1); wait K(0); barrier;
//                  step j: wait V(j), K(j+1); barrier A(j); request K(j+2);
//                          barrier B(j); request V(j+2)
//   compute waves: barrier; S(0);
//                  step j: barrier A(j); softmax(j) + O += P(j) V(j); barrier B(j); S(j+1)
// At A(j) the compute waves are done with K(j) (S(j) ran before it), at B(j) with V(j): each
// buffer is refilled as soon as it is free, so every copy has about one and a half steps to land.
// (With one barrier per step, V(j+1) was requested only at the start of step j and arrived late:
// the kernel waited on its copies.)  The summary tiles (proxy on) follow in a loop of the same
// shape.
constexpr int kPcGroups = 2;   // query blocks per workgroup
constexpr int kPcWaves = 2;    // compute (and copy) waves per query block

template <int D>
__global__ __launch_bounds__(2 * kPcGroups * kPcWaves * 64) __attribute__((amdgpu_waves_per_eu(2)))
void proxy_pc_kernel(ProxyArgs a) {
  constexpr int QB = 1;
  constexpr int BR = kPcWaves * 32;   // rows per query block
  using DmaK = Dma<KLayout<D>, kPcWaves>;
  using DmaV = Dma<VLayout<D>, kPcWaves>;
  constexpr int kN = DmaK::kPerWave;
  static_assert(DmaV::kPerWave == kN, "K and V tiles take the same number of copies");
  __shared__ __attribute__((aligned(1024))) Smem<D, kPcWaves> sms[kPcGroups];

  const AttnGeom& g = a.g;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool copier = wave >= kPcGroups * kPcWaves;
  const int cw = copier ? wave - kPcGroups * kPcWaves : wave;
  const int grp = cw / kPcWaves, rank = cw % kPcWaves;
  Smem<D, kPcWaves>& sm = sms[grp];
  const int h = lane >> 5;
  const int Bk = g.block_k;
  const int nQB = (g.Sq + BR - 1) / BR;
  const int nPair = (nQB + kPcGroups - 1) / kPcGroups;
  const int nKB = (g.Sk + Bk - 1) / Bk;
  const int G = g.Hq / g.Hkv;
  const int total = g.B * g.Hq * nPair;

  int item = xcd_remap(blockIdx.x, total);
  const int gq = item % G;
  item /= G;
  const int pair = item % nPair;
  item /= nPair;
  const int hk = item % g.Hkv;
  const int b = item / g.Hkv;
  const int hq = hk * G + gq;

  const int qblk = pair * kPcGroups + grp;
  const bool present = qblk < nQB;   // the last pair may have one block
  const int row0 = qblk * BR;
  const int wrow0 = row0 + rank * 32;
  const int64_t route_row = ((int64_t)b * g.Hkv + hk) * nQB + min(qblk, nQB - 1);

  ExactPolicy<D, kPcWaves, QB> pol;
  pol.init(a, b, hk, route_row, nKB, h, present);
  const int n = pol.steps();
  // steps of the other query block of the pair (both walk max(n, n_other) barriers)
  int n_other = 0;
  {
    const int oblk = pair * kPcGroups + (grp ^ 1);
    if (oblk < nQB) {
      const int64_t orow = ((int64_t)b * g.Hkv + hk) * nQB + oblk;
      n_other = min(max(__builtin_amdgcn_readfirstlane(a.n_exact[orow]), 0), nKB) * pol.sub;
    }
  }
  const int N = max(n, n_other);
  const int n_sum = a.use_proxy ? (nKB + kKeysPerTile - 1) / kKeysPerTile : 0;

  if (copier) {
    auto issue_k = [&](int step) {
      const TileSrc t = pol.src(step);
      DmaK::copy(sm.k[step & 1], t.k, t.k_bytes, t.k_stride_b,
                 DmaK::lane_offsets(t.k_stride_b, rank, lane), rank);
    };
    auto issue_v = [&](int step) {
      const TileSrc t = pol.src(step);
      DmaV::copy(sm.v[step & 1], t.v, t.v_bytes, t.v_stride_b,
                 DmaV::lane_offsets(t.v_stride_b, rank, lane), rank);
    };
    if (n > 0) {
      issue_k(0);
      issue_v(0);
    }
    if (n > 1) {
      issue_k(1);
      issue_v(1);
      wait_vmcnt<3 * kN>();   // K(0) landed
    } else {
      wait_vmcnt<kN>();
    }
    lds_barrier();
    for (int j = 0; j < N; ++j) {
      // V(j) and K(j+1) landed; V(j+1), requested after K(j+1), may still be in flight
      if (j + 1 < n) wait_vmcnt<kN>(); else wait_vmcnt<0>();
      lds_barrier();   // A(j): S(j) is done, K(j)'s buffer is free
      if (j + 2 < n) issue_k(j + 2);
      lds_barrier();   // B(j): P.V(j) is done, V(j)'s buffer is free
      if (j + 2 < n) issue_v(j + 2);
    }
    if (n_sum > 0) {
      // summary tile t (64 rows of k_mean / v_sum) into buffer t&1
      const int64_t sbase = ((int64_t)b * g.Hkv + hk) * nKB * D;
      const auto sklo = DmaK::lane_offsets(D * 2, rank, lane);
      const auto svlo = DmaV::lane_offsets(D * 2, rank, lane);
      // rows past nKB read as zeros (and are masked); a missing query block copies nothing
      auto issue_sk = [&](int t) {
        const int r0 = t * kKeysPerTile;
        DmaK::copy(sm.k[t & 1], (const __bf16*)a.k_mean + sbase + (int64_t)r0 * D,
                   present ? (nKB - r0) * D * 2 : 0, D * 2, sklo, rank);
      };
      auto issue_sv = [&](int t) {
        const int r0 = t * kKeysPerTile;
        DmaV::copy(sm.v[t & 1], (const __bf16*)a.v_sum + sbase + (int64_t)r0 * D,
                   present ? (nKB - r0) * D * 2 : 0, D * 2, svlo, rank);
      };
      lds_barrier();   // the compute waves are done with every exact tile
      issue_sk(0);
      issue_sv(0);
      if (n_sum > 1) {
        issue_sk(1);
        issue_sv(1);
        wait_vmcnt<3 * kN>();   // K(0) landed
      } else {
        wait_vmcnt<kN>();
      }
      lds_barrier();
      // the exact loop's schedule over the summary tiles
      for (int t = 0; t < n_sum; ++t) {
        if (t + 1 < n_sum) wait_vmcnt<kN>(); else wait_vmcnt<0>();
        lds_barrier();   // A(t)
        if (t + 2 < n_sum) issue_sk(t + 2);
        lds_barrier();   // B(t)
        if (t + 2 < n_sum) issue_sv(t + 2);
      }
    }
    return;
  }

  const auto qsrc = slab_rsrc((const __bf16*)g.q + b * g.qs[0] + hq * g.qs[2], g.qs[1], g.Sq, D);
  bf16x8 qf[QB][D / 16];
  load_q_frags<D, QB>(qf, qsrc, g.qs[1], wrow0, lane);

  f32x16 o[D / 32][QB];
  float mref[QB], l[QB];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) o[db][0] = f32x16{};
  mref[0] = -INFINITY;
  l[0] = 0.f;

  f32x16 s[2][QB];
  TileState<QB> ts;
  auto scores = [&](int step) {
    qk_tile<D, QB>(sm.k[step & 1], qf, s, lane);
    pol.mask(step, s, lane);
    tile_row_max<QB>(s, g.c32, ts.M);
    ts.keep = true;
  };
  lds_barrier();
  if (n > 0) scores(0);
  for (int j = 0; j < N; ++j) {
    lds_barrier();   // A(j)
    if (j < n) softmax_pv<D, QB>(pol, j, s, ts, mref, l, o, sm.v[j & 1], g.c32, lane);
    lds_barrier();   // B(j)
    if (j + 1 < n) scores(j + 1);
  }

  if (n_sum > 0) {
    SummaryPolicy<QB> sp;
    sp.init(a, route_row, nKB, h);
    auto summary_scores = [&](int t) {
      qk_tile<D, QB>(sm.k[t & 1], qf, s, lane);
      sp.mask(t, s);
      tile_row_max<QB>(s, g.c32, ts.M);
      ts.keep = true;
    };
    lds_barrier();   // every exact tile is done
    lds_barrier();   // summary K(0) has landed
    if (present) summary_scores(0);
    for (int t = 0; t < n_sum; ++t) {
      lds_barrier();   // A(t)
      if (present) softmax_pv<D, QB>(sp, t, s, ts, mref, l, o, sm.v[t & 1], g.c32, lane);
      lds_barrier();   // B(t)
      if (present && t + 1 < n_sum) summary_scores(t + 1);
    }
  }
  if (!present) return;

  store_rows<D, QB>(a, b, hq, wrow0, o, mref, l, lane);
}

template <int D>
hipError_t launch_pc(const ProxyArgs& a, hipStream_t stream) {
  constexpr int BR = kPcWaves * 32;
  const int nQB = (a.g.Sq + BR - 1) / BR;
  const int nPair = (nQB + kPcGroups - 1) / kPcGroups;
  const int total = a.g.B * a.g.Hq * nPair;
  hipLaunchKernelGGL((proxy_pc_kernel<D>), dim3(total), dim3(2 * kPcGroups * kPcWaves * 64), 0,
                     stream, a);
  return hipGetLastError();
}

template <int D, int NW, int QB>
hipError_t launch_t(const ProxyArgs& a, hipStream_t stream) {
  constexpr int BR = NW * 32 * QB;
  const int nQB = (a.g.Sq + BR - 1) / BR;
  const int total = a.g.B * a.g.Hq * nQB;
  hipLaunchKernelGGL((proxy_kernel<D, NW, QB>), dim3(total), dim3(NW * 64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_proxy(const ProxyArgs& a, hipStream_t stream) {
  constexpr int QB = kQueryBlocksPerWave;
  const bool q128 = a.g.block_q == 128;
  if (a.g.D == 128) return q128 ? launch_t<128, 4 / QB, QB>(a, stream) : launch_pc<128>(a, stream);
  return q128 ? launch_t<64, 4 / QB, QB>(a, stream) : launch_pc<64>(a, stream);
}

}  // namespace sa
