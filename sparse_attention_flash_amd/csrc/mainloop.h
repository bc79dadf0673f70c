// mainloop.h -- the pipelined key-tile loop shared by the skip-softmax, N:M, combined and proxy
// kernels.
//
// One workgroup of NW wavefronts, each owning QB blocks of 32 query rows, walks a sequence of
// 64-key tiles ("steps") given by a policy object.  K and V tiles are copied HBM/L2 -> LDS with
// buffer loads that write LDS directly (no staging registers), double-buffered.  Scores run two
// tiles ahead of the softmax and every tile's votes are published one barrier before its V tile
// is requested, so each iteration needs a single barrier:
//
//   iteration j (S(j) in registers and decided; S(j+1) in registers, votes written)
//     1  wait for V(j), K(j+2); barrier (also publishes the votes of j+1)
//     2  keep(j+1) = OR of its votes; [kept] raise mt, request V(j+1)
//     3  request K(j+3)
//     4  [kept(j)]  softmax(j) fused with O += P(j) V(j), 16 keys at a time (VALU || MFMA)
//     5  S(j+2) = QK^T(j+2) into the registers S(j) used; mask; row max; wave votes for j+2
//
// A skipped tile costs its QK^T, row max and vote only: no exponentials, no V traffic, no P.V.
// Every load of iteration j-1 is complete at step 1 of iteration j (s_waitcnt vmcnt(0)).
// Cross-wave barriers are "s_waitcnt lgkmcnt(0); s_barrier" (vote stores must land, prefetches
// must not drain).
//
// Exponent reference: P = 2^(t - m_ref), m_ref raised (and O, l rescaled) only when a kept tile's
// row max exceeds it by more than kRescaleSlack, so P <= 2^kRescaleSlack; numerator and
// denominator share the reference.  The skip decision uses the exact fp32 running max mt of the
// kept tiles' row maxima, updated as soon as a tile is decided.
#pragma once

#include "tile_core.h"

namespace sa {

constexpr float kRescaleSlack = 8.f;

// Query blocks of 32 rows per wavefront.  With one block a wave's registers (O 64, Q^T 32, two score
// tiles 64, operands) fit in 256, so two waves share each SIMD; with two they need the whole file.
constexpr int kQueryBlocksPerWave = 1;
template <int QB>
constexpr int kWavesPerSimd = QB == 1 ? 2 : 1;

template <int D, int NW>
struct Smem {
  char k[2][KLayout<D>::kBytes];
  char v[2][VLayout<D>::kBytes];
  int vote[2][NW];
};

// One step's K and V sources: buffer-resource bases already offset to the tile's first row, and
// the number of valid bytes from those bases (rows past the end read as zeros).
struct TileSrc {
  const __bf16* k;
  const __bf16* v;
  int k_bytes, v_bytes;
  int k_stride_b, v_stride_b;
};

__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// s_waitcnt vmcnt(N), leaving expcnt and lgkmcnt alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

template <class L, int NW>
struct Dma {
  static constexpr int kPerWave = L::kBlocks / NW;   // one block (1 KiB) per wave-wide instruction
  static_assert(kPerWave >= 1 && L::kBlocks % NW == 0, "tile must split over the waves");

  // Lane byte offset of a block copy relative to the block's first row (the same for every block;
  // the copy adds the block's row shift).
  struct LaneOffsets {
    int off;
  };
  static __device__ __forceinline__ LaneOffsets lane_offsets(int stride_b, int, int lane) {
    return LaneOffsets{L::dma_lane(stride_b, lane)};
  }

  // Copy a 64-row tile whose first row starts at `base` (`bytes` valid bytes from there; rows past
  // them arrive as zeros) into the LDS tile at `lds` (layout L): wave w copies blocks w, w + NW, ...
  //
  // Issued from inline asm: the compiler, seeing an LDS-writing load it cannot disambiguate,
  // would otherwise wait for every outstanding copy (vmcnt(0)) before each later LDS read and
  // drain the prefetches.  The explicit s_waitcnt vmcnt + barrier pairs in the loop are what
  // order these copies against the reads.  M0 carries the LDS destination (no other use of M0
  // remains in these kernels).
  static __device__ __forceinline__ void copy(char* lds, const __bf16* base, int bytes,
                                              int stride_b, const LaneOffsets& lo, int wave) {
    const unsigned lds0 = (unsigned)(uintptr_t)(__attribute__((address_space(3))) char*)lds;
    const auto rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, max(0, bytes),
                                                        0x00020000);
    // One resource per tile; a block's row shift goes into the lane offset, so the per-lane
    // range check still zero-fills rows past the end.  The empty asm makes the block offsets
    // look loop-variant: hoisted out of the key loop they would hold about 30 SGPRs, which the
    // compiler then spills to VGPR lanes and reloads (v_readlane) in front of every copy.
    int w = wave, sb = stride_b;
    asm volatile("" : "+s"(w), "+s"(sb));
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      const int blk = w + i * NW;
      const int voff = lo.off + blk * L::kRowShiftPerBlock * sb;
      const unsigned dst = lds0 + blk * L::kPitch;
      asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                   :
                   : "s"(dst), "v"(voff), "s"(rsrc)
                   : "memory", "m0");
    }
  }
};

template <int QB>
__device__ __forceinline__ void tile_row_max(const f32x16 (&s)[2][QB], float c32, float (&M)[QB]) {
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][qb][r]);
    M[qb] = half_max(mx) * c32;
  }
}

// Per-step state: row maxima (log2 domain) and the decision.
template <int QB>
struct TileState {
  float M[QB];
  bool keep;      // this wave runs the step's softmax and P.V
  bool fetched;   // the step's V tile was requested
  bool own;       // this wave's published vote
};

// Softmax of a kept tile fused with its P.V product.  For each 16-key chunk: exponentials of the
// chunk (VALU), then the MFMAs that consume them, so the VALU work of one chunk overlaps the MFMAs
// of the previous one.  Keys a filter dropped (N:M) arrive as -inf and get weight 0; Pol::weight
// (proxy) scales each key's row-sum term.  The row sum adds the fp32 weights (before their
// rounding to bf16 for P.V), which keeps the LSE at fp32 accuracy.
template <int D, int QB, class Pol>
__device__ __forceinline__ void softmax_pv(const Pol& pol, int step, const f32x16 (&s)[2][QB],
                                           const TileState<QB>& ts, float (&mref)[QB],
                                           float (&l)[QB], f32x16 (&o)[D / 32][QB],
                                           const char* ldsV, float c32, int lane) {
  bool need = false;
  float cand[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    cand[qb] = fmaxf(mref[qb], ts.M[qb]);
    need |= cand[qb] > mref[qb] + kRescaleSlack;   // also true when mref = -inf, M finite
  }
  if (__builtin_amdgcn_ballot_w64(need) != 0ull) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float alpha = mref[qb] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mref[qb] - cand[qb]);
      l[qb] *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) o[db][qb] *= alpha;
      mref[qb] = cand[qb];
    }
  }
  float muse[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) muse[qb] = mref[qb] == -INFINITY ? 0.f : mref[qb];
  bool weighted = false;
  if constexpr (Pol::kWeighted) weighted = pol.weighted(step);

  // V^T operands of chunk n (16 keys: kb = n/2, c = n%2) for each 32-wide d block: two transpose
  // reads each, issued one chunk ahead of the MFMAs that consume them.
  auto vt = [&](int n, bf16x8 (&a)[D / 32]) {
    const int kb = n >> 1, c = n & 1;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_i16x4*)(ldsV + VLayout<D>::v_off(lane, kb, c, 0, db)));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_i16x4*)(ldsV + VLayout<D>::v_off(lane, kb, c, 1, db)));
      a[db] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  };
  // P of chunk n into pb (bf16 operands) and its row sums into l
  auto make_p = [&](int n, bf16x8 (&pb)[QB]) {
    const int kb = n >> 1, c = n & 1;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float rs = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int r = 8 * c + e;
        float p = __builtin_amdgcn_exp2f(s[kb][qb][r] * c32 - muse[qb]);
        if constexpr (Pol::kWeighted) {
          rs += weighted ? p * pol.weight(step, kb, r, lane) : p;
        } else {
          rs += p;
        }
        pb[qb][e] = (__bf16)p;
      }
      l[qb] += rs;
    }
  };
  // Chunk n's MFMAs run while the exponentials of chunk n+1 are computed: the scheduling groups
  // alternate one MFMA with a share of that VALU work.
  constexpr int kMfma = (D / 32) * QB;
  constexpr int kValu = (28 * QB + kMfma - 1) / kMfma;
  bf16x8 va[2][D / 32];
  bf16x8 pb[2][QB];
  vt(0, va[0]);
  make_p(0, pb[0]);
  vt(1, va[1]);
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) o[db][qb] = mfma32(va[n & 1][db], pb[n & 1][qb], o[db][qb]);
    if (n + 1 < 4) {
      make_p(n + 1, pb[(n + 1) & 1]);
#pragma unroll
      for (int i = 0; i < kMfma; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, kValu, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (n + 2 < 4) vt(n + 2, va[n & 1]);
  }
}

// The step loop.  Pol provides (arrays indexed by the wave's 32-row query blocks qb < QB):
//   int steps() const;  TileSrc src(int step) const;
//   void mask(int step, f32x16 (&s)[2][QB], int lane) const;        -inf for masked keys
//   static constexpr bool kDecide, kFilter, kWeighted;
//   static constexpr bool kWave, kPair;                                            [kDecide]
//   bool negligible(const float (&M)[QB], const float (&mt)[QB], int lane) const;   [kDecide]
//   bool visible(int step) const;   the step holds an unmasked key of this wave's rows [kDecide]
//   void filter(int step, f32x16 (&s)[2][QB], int lane) const;  dropped keys -> -inf   [kFilter]
//   bool exports() const;  the filter's debug exports are on: filter every visited step
//                                                                   [kFilter and kDecide]
//   bool weighted(int step) const; float weight(int step, int kb, int r, int lane) const; [kWeighted]
//   void record(int tile, bool keep, const float (&M)[QB], int wave, int lane, bool leader);
// On return o, mref and l hold the unnormalised accumulator, exponent reference and row-sum
// partials of this lane (l still to be summed over the two lane halves).
//
// Decisions (kDecide).  Every wave publishes one vote per step in LDS; after the next barrier:
//   - tile granularity (!kWave): the step is kept for every wave when any wave voted "some row
//     not negligible";
//   - wave granularity (kWave): each wave keeps the step on its own vote (its 32 rows alone) and
//     the V tile is fetched when any wave keeps it.
// A kept step raises the wave's decision max mt at once.  With kPair the decision tile is 128 keys,
// two consecutive 64-key steps (2p, 2p+1) decided together against the running max from before
// the pair: the pair is skipped only when both halves are negligible (max over the 128 keys below
// the threshold is the same as both halves below it).  Half a is decided first; when it is kept
// the pair is kept.  Otherwise half b's vote decides, and a pair kept only through half b ("late"
// keep) requests V of half a then, waiting for it before that half's softmax.
template <int D, int NW, int QB, class Pol>
struct Mainloop {
  using DmaK = Dma<KLayout<D>, NW>;
  using DmaV = Dma<VLayout<D>, NW>;
  using TS = TileState<QB>;
  static constexpr int kN = DmaK::kPerWave;   // loads per tile per lane
  static_assert(DmaK::kPerWave == DmaV::kPerWave, "K and V tiles take the same number of copies");

  Pol& pol;
  Smem<D, NW>& sm;
  typename DmaK::LaneOffsets klo;
  typename DmaV::LaneOffsets vlo;
  const bf16x8 (&qf)[QB][D / 16];
  f32x16 (&o)[D / 32][QB];
  float (&mref)[QB];
  float (&l)[QB];
  float c32;
  int wave, lane, tid, n;
  float mt[QB];         // running max of kept tiles' maxima (decision state)
  bool pair_own = false;       // kPair: this wave keeps the pair being decided (from half a)
  bool pair_fetched = false;   // kPair: V of half a was requested

  __device__ __forceinline__ void issue_k(int step) {
    const TileSrc t = pol.src(step);
    DmaK::copy(sm.k[step & 1], t.k, t.k_bytes, t.k_stride_b, klo, wave);
  }
  __device__ __forceinline__ void issue_v(int step) {
    const TileSrc t = pol.src(step);
    DmaV::copy(sm.v[step & 1], t.v, t.v_bytes, t.v_stride_b, vlo, wave);
  }

  // S(step) from the K tile in LDS, masked, with its row maxima; without decisions a filtering
  // policy (N:M) then sets the scores of the keys it drops to -inf.  With decisions the filter runs
  // once the step is decided, on kept steps only (the tile maxima it leaves unchanged are already
  // taken: the rule keeps every group maximum).
  __device__ __forceinline__ void scores(int step, f32x16 (&s)[2][QB], TS& ts) {
    qk_tile<D, QB>(sm.k[step & 1], qf, s, lane);
    pol.mask(step, s, lane);
    tile_row_max<QB>(s, c32, ts.M);
    if constexpr (Pol::kFilter && !Pol::kDecide) pol.filter(step, s, lane);
  }

  // Each wave publishes "some row of this tile is not negligible" in LDS (for the second half of a
  // pair: "this wave keeps the pair"); the votes are read after the next barrier.
  __device__ __forceinline__ void vote(int step, TS& ts) {
    if constexpr (Pol::kDecide) {
      bool own = __builtin_amdgcn_ballot_w64(!pol.negligible(ts.M, mt, lane)) != 0ull;
      if constexpr (Pol::kWave) own = own && pol.visible(step);
      if constexpr (Pol::kPair) {
        if (step & 1) own = own || pair_own;
      }
      ts.own = own;
      if (lane == 0) sm.vote[step & 1][wave] = own ? 1 : 0;
    }
  }

  __device__ __forceinline__ void raise_mt(const float (&M)[QB]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) mt[qb] = fmaxf(mt[qb], M[qb]);
  }

  // After a barrier that follows every wave's vote(step): the decision.  A kept step raises the
  // decision max mt at once and has its V tile fetched.  `other` is the state of the pair's other
  // half (kPair).  Returns true for a late keep: V of half a was requested only now.
  __device__ __forceinline__ bool resolve(int step, TS& ts, TS& other) {
    int any = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) any |= sm.vote[step & 1][w];
    const bool fetch = any != 0;
    const bool mine = Pol::kWave ? ts.own : fetch;
    ts.keep = mine;
    ts.fetched = fetch;
    if constexpr (!Pol::kPair) {
      if (mine) raise_mt(ts.M);
      if (fetch) issue_v(step);
      pol.record(step, mine, ts.M, wave, lane, tid == 0);
      return false;
    } else {
      if (!(step & 1)) {   // half a
        pair_own = mine;
        pair_fetched = fetch;
        if (mine) raise_mt(ts.M);
        if (fetch) issue_v(step);
        if (step + 1 >= n) pol.record(step >> 1, mine, ts.M, wave, lane, tid == 0);
        return false;
      }
      // half b: `mine` already includes half a's keep (the published vote ORs it in)
      if (mine) {
        if (!pair_own) {   // kept through half b only: half a is kept too
          raise_mt(other.M);
          other.keep = true;
        }
        raise_mt(ts.M);
      }
      const bool late = fetch && !pair_fetched;
      if (late) {
        issue_v(step - 1);
        other.fetched = true;
      }
      if (fetch) issue_v(step);
      float Mp[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) Mp[qb] = fmaxf(other.M[qb], ts.M[qb]);
      pol.record(step >> 1, mine, Mp, wave, lane, tid == 0);
      return late;
    }
  }

  // iteration j.  On entry S(j) is in sa with keep(j) resolved (V(j) requested when kept), S(j+1)
  // is in sb (state tb) with its votes written, K(j+2) is requested.  One barrier per iteration.
  __device__ __forceinline__ void iteration(int j, f32x16 (&sa)[2][QB], TS& ta, TS& tb) {
    // 1: V(j), K(j+2) and the votes of j+1 are complete and visible to every wave
    wait_vmcnt<0>();
    lds_barrier();
    // 2: decide j+1 and request its V tile (the buffer V(j-1) used)
    bool late = false;
    if (j + 1 < n) late = resolve(j + 1, tb, ta);
    // 3: request K(j+3) (the buffer K(j+1) used)
    if (j + 3 < n) issue_k(j + 3);
    if constexpr (Pol::kPair) {
      // a late keep requested V(j) just now (into the buffer V(j-2) used, free since the barrier of
      // iteration j-1), ahead of V(j+1) and K(j+3): wait for it alone
      if (late) {
        if (j + 3 < n) wait_vmcnt<2 * kN>(); else wait_vmcnt<kN>();
        lds_barrier();
      }
    }
    // 4: the filter of a kept step j (of every step while the filter's exports are on), then
    // softmax(j) fused with O += P(j) V(j)
    if constexpr (Pol::kFilter) {
      if (ta.keep || pol.exports()) pol.filter(j, sa, lane);
    }
    if (ta.keep) softmax_pv<D, QB>(pol, j, sa, ta, mref, l, o, sm.v[j & 1], c32, lane);
    // 5: S(j+2) into sa, its row maxima and votes (mt already holds every kept tile up to j+1)
    if (j + 2 < n) {
      scores(j + 2, sa, ta);
      vote(j + 2, ta);
    }
  }

  // Without decisions (N:M, exact routes) every V tile is fetched, so the scores need only one
  // step of lookahead and a single S tile:
  //   iteration j: wait for V(j), K(j+1); barrier; request V(j+1), K(j+2);
  //                softmax(j) + O += P(j) V(j); S(j+1) = QK^T(j+1) into the same registers.
  __device__ __forceinline__ void run_dense() {
    f32x16 s[2][QB];
    TS ts;
    issue_k(0);
    issue_v(0);
    if (n > 1) issue_k(1);
    if (n > 1) wait_vmcnt<2 * kN>(); else wait_vmcnt<kN>();   // K(0) landed
    lds_barrier();
    scores(0, s, ts);
    for (int j = 0; j < n; ++j) {
      wait_vmcnt<0>();   // V(j), K(j+1)
      lds_barrier();
      if (j + 1 < n) issue_v(j + 1);   // the buffer V(j-1) used
      if (j + 2 < n) issue_k(j + 2);   // the buffer K(j) used
      pol.record(j, true, ts.M, wave, lane, tid == 0);
      softmax_pv<D, QB>(pol, j, s, ts, mref, l, o, sm.v[j & 1], c32, lane);
      if (j + 1 < n) scores(j + 1, s, ts);
    }
  }

  __device__ __forceinline__ void run() {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) mt[qb] = -INFINITY;
    if (n <= 0) return;
    {
      const TileSrc t = pol.src(0);
      klo = DmaK::lane_offsets(t.k_stride_b, wave, lane);
      vlo = DmaV::lane_offsets(t.v_stride_b, wave, lane);
    }
    if constexpr (!Pol::kDecide) {
      run_dense();
    } else {
      run_decide();
    }
  }

  // The decision pipeline: scores two steps ahead of the softmax.
  __device__ __forceinline__ void run_decide() {
    f32x16 sa[2][QB], sb[2][QB];
    TS ta, tb;
    // prologue: K(0), K(1); S(0) and keep(0) (V(0) requested); S(1) and its votes; K(2)
    issue_k(0);
    if (n > 1) issue_k(1);
    if (n > 1) wait_vmcnt<kN>(); else wait_vmcnt<0>();
    lds_barrier();
    scores(0, sa, ta);
    vote(0, ta);
    lds_barrier();
    resolve(0, ta, tb);
    if (n > 1) {
      // K(1) landed: only V(0) (if requested) was requested after it
      if (ta.fetched) wait_vmcnt<kN>(); else wait_vmcnt<0>();
      lds_barrier();
      scores(1, sb, tb);
      vote(1, tb);
      if (n > 2) issue_k(2);   // K(0)'s buffer: every wave passed a barrier after QK(0)
    }
    for (int j = 0; j < n; j += 2) {
      iteration(j, sa, ta, tb);
      if (j + 1 < n) iteration(j + 1, sb, tb, ta);
    }
  }
};

template <int D, int NW, int QB, class Pol>
__device__ __forceinline__ void run_mainloop(Pol& pol, Smem<D, NW>& sm,
                                             const bf16x8 (&qf)[QB][D / 16],
                                             f32x16 (&o)[D / 32][QB], float (&mref)[QB],
                                             float (&l)[QB], float c32, int wave, int lane,
                                             int tid) {
  Mainloop<D, NW, QB, Pol> ml{pol, sm, {}, {}, qf, o, mref, l, c32, wave, lane, tid, pol.steps()};
  ml.run();
}

}  // namespace sa
