// policies.h -- the per-method parts of the key-tile loop (mainloop.h) and the kernel body shared
// by the dense-walk kernels (skip-softmax, N:M, and the two combined).
//
//   KeyTiles      walks every visited 64-key tile of the query tile in order; causal and
//                 out-of-range keys are masked to -inf.
//   SkipDecision  the skip-softmax rule (Model-Optimizer "Skip-Softmax Sparse Attention for
//                 Diffusion Models": a key tile whose scores are negligible under lambda is
//                 skipped, saving its exponentials, V load and P.V; the kernel works with
//                 log2(lambda)): tile j is skipped when every valid row r has
//                 M_j[r] < fl32(m[r] + log2(lambda)), m the fp32 running max of the kept tiles.
//   NmFilter      the N:M rule (Model-Optimizer "Attention Sparsity for HuggingFace Models",
//                 "N:M Sparse Softmax": per query, of every M consecutive keys keep the top N,
//                 the others -inf; sink and recent windows stay dense).
//
// A policy is KeyTiles plus any of the two rules; attention_tile() is the kernel body around it.
#pragma once

#include "kernels.h"
#include "mainloop.h"

namespace sa {

// Where one workgroup sits: (batch, query head, query tile), and this wave's first row.
struct TileUnit {
  int b, hq, hk, qt, row0, wrow0, nvis, nQT, nKT;
  int64_t unit;   // (b*Hq + hq)*nQT + qt
};

// Work item order: KV head major, then query tile, then the G query heads sharing the KV head, so
// that concurrently running workgroups of one XCD read the same K/V tiles.
//
// Causal rows differ in length, so the longest go first.  The items are cut into blocks of hb KV
// heads (hb = the KV heads in one XCD's share of the items, at least 1), and inside a block the
// order is query tile (longest first), then KV head, then query head: each XCD then runs its
// share longest-first, and the workgroups of one head still walk the same K/V tiles together.
// With one KV head per block this is the plain order above.
template <int NW, int QB>
__device__ __forceinline__ TileUnit tile_unit(const AttnGeom& g, int wave) {
  constexpr int BR = NW * 32 * QB;
  TileUnit u;
  u.nQT = (g.Sq + BR - 1) / BR;
  u.nKT = (g.Sk + kKeysPerTile - 1) / kKeysPerTile;
  const int G = g.Hq / g.Hkv;
  const int total = g.B * g.Hq * u.nQT;
  int item = xcd_remap(blockIdx.x, total);
  int gq, qt, bh;
  if (!g.causal) {
    gq = item % G;
    item /= G;
    qt = item % u.nQT;
    bh = item / u.nQT;
  } else {
    const int per = u.nQT * G;   // items of one KV head
    const int BH = g.B * g.Hkv;
    const int hb = max(1, min(BH, (total >> 3) / per));
    const int h0 = item / (hb * per) * hb;   // first KV head of this item's block
    const int nh = min(hb, BH - h0);          // KV heads in the block
    const int c = item - h0 * per;            // position inside the block, < nh * per
    qt = u.nQT - 1 - c / (nh * G);
    const int r = c % (nh * G);
    bh = h0 + r / G;
    gq = r % G;
  }
  u.hk = bh % g.Hkv;
  u.b = bh / g.Hkv;
  u.qt = qt;
  u.hq = u.hk * G + gq;
  u.row0 = qt * BR;
  u.wrow0 = u.row0 + wave * 32 * QB;
  const int last_row = min(u.row0 + BR, g.Sq) - 1;
  u.nvis = g.causal ? min(u.nKT, last_row / kKeysPerTile + 1) : u.nKT;
  u.unit = ((int64_t)u.b * g.Hq + u.hq) * u.nQT + qt;
  return u;
}

template <int QB>
struct KeyTiles {
  static constexpr int RW = 32 * QB;   // rows per wave
  const __bf16* kslab;
  const __bf16* vslab;
  int k_stride_b, v_stride_b, k_bytes, v_bytes;
  int Sq, Sk, causal, wrow0, nvis, h, r32;

  __device__ __forceinline__ void init_tiles(const AttnGeom& g, const TileUnit& u, int D,
                                             int lane) {
    kslab = (const __bf16*)g.k + u.b * g.ks[0] + u.hk * g.ks[2];
    vslab = (const __bf16*)g.v + u.b * g.vs[0] + u.hk * g.vs[2];
    k_stride_b = (int)(g.ks[1] * 2);
    v_stride_b = (int)(g.vs[1] * 2);
    k_bytes = (int)(((int64_t)(g.Sk - 1) * g.ks[1] + D) * 2);
    v_bytes = (int)(((int64_t)(g.Sk - 1) * g.vs[1] + D) * 2);
    Sq = g.Sq;
    Sk = g.Sk;
    causal = g.causal;
    wrow0 = u.wrow0;
    nvis = u.nvis;
    h = lane >> 5;
    r32 = lane & 31;
  }

  __device__ __forceinline__ int steps() const { return nvis; }

  __device__ __forceinline__ TileSrc src(int j) const {
    const int k0 = j * kKeysPerTile;
    return TileSrc{kslab + (int64_t)k0 * (k_stride_b / 2), vslab + (int64_t)k0 * (v_stride_b / 2),
                   max(0, k_bytes - k0 * k_stride_b), max(0, v_bytes - k0 * v_stride_b),
                   k_stride_b, v_stride_b};
  }

  // key = k0 + 8*h + elem_key(kb, r), a compile-time offset; masked when it reaches lim
  __device__ __forceinline__ void mask(int j, f32x16 (&s)[2][QB], int) const {
    const int k0 = j * kKeysPerTile;
    if (!((k0 + kKeysPerTile > Sk) || (causal && k0 + kKeysPerTile - 1 > wrow0))) return;
    const int klim = Sk - k0 - 8 * h;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      int lim = klim;
      if (causal) lim = min(lim, wrow0 + qb * 32 + r32 - k0 - 8 * h + 1);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) mask_block(s[kb][qb], kb, lim);
    }
  }

  // defaults for a policy without the rule
  __device__ __forceinline__ bool negligible(const float (&)[QB], const float (&)[QB], int) const {
    return false;
  }
  __device__ __forceinline__ void filter(int, f32x16 (&)[2][QB], int) const {}
  __device__ __forceinline__ void record(int, bool, const float (&)[QB], int, int, bool) {}
};

// ---- the skip rule --------------------------------------------------------------------------------
//
// Decision tiles are block_k = 64 keys (one step) or 128 keys (kPair: two steps decided together).
// Decision rows are the whole query tile (tile granularity) or each wavefront's 32 rows alone
// (kWave, wave granularity: a 32-row block is decided exactly as a query tile of 32 rows would
// be, and the V tile is fetched for the workgroup when any wave keeps it).  The state, counter and
// maxima exports are per decision block of rows: tile_state [B, Hq, nR, nKTd] with nR =
// ceil(Sq/R), R = block_q or 32, nKTd = ceil(Sk/block_k); rowmax [.., nKTd, R].

template <int D, int NW, int QB, bool kWaveGran = false, bool kPairTiles = false>
struct SkipDecision : KeyTiles<QB> {
  static constexpr bool kDecide = true, kFilter = false, kWeighted = false;
  static constexpr bool kWave = kWaveGran, kPair = kPairTiles;
  static_assert(!kWave || QB == 1, "wave granularity decides 32-row blocks");
  static constexpr int RW = 32 * QB;
  static constexpr int BR = NW * RW;
  static constexpr int R = kWave ? RW : BR;        // decision rows
  static constexpr int kSub = kPair ? 2 : 1;       // steps per decision tile
  float L32;
  uint8_t* tile_state;
  float* rowmax;
  int64_t unit;      // decision row block: (b*Hq + hq)*nR + (qt*NW + wave when kWave, else qt)
  int nKTd;          // decision tiles per row block
  int nvis_w;        // steps with an unmasked key of this wave's rows (kWave), else of the tile
  bool exists;       // this decision block has a row < Sq
  int nskip;

  // Args: SkipArgs or SkipNmArgs
  template <class Args>
  __device__ __forceinline__ void init(const Args& a, const TileUnit& u, int lane) {
    this->init_tiles(a.g, u, D, lane);
    nKTd = (a.g.Sk + kSub * kKeysPerTile - 1) / (kSub * kKeysPerTile);
    L32 = a.L32;
    tile_state = a.tile_state;
    rowmax = a.rowmax;
    nskip = 0;
    if constexpr (kWave) {
      const int wave = (u.wrow0 - u.row0) / RW;
      const int n32 = (a.g.Sq + RW - 1) / RW;
      unit = ((int64_t)u.b * a.g.Hq + u.hq) * n32 + (int64_t)u.qt * NW + wave;
      exists = u.wrow0 < a.g.Sq;
      const int last = min(u.wrow0 + RW, a.g.Sq) - 1;
      nvis_w = !exists ? 0 : (a.g.causal ? min(u.nKT, last / kKeysPerTile + 1) : u.nKT);
    } else {
      unit = u.unit;
      exists = true;
      nvis_w = u.nvis;
    }
  }

  // true when every valid row this lane holds is negligible: M < fl32(m + log2(lambda))
  __device__ __forceinline__ bool negligible(const float (&M)[QB], const float (&mt)[QB],
                                             int) const {
    bool negl = true;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float thr = mt[qb] + L32;
      if (this->wrow0 + qb * 32 + this->r32 < this->Sq && !(M[qb] < thr)) negl = false;
    }
    return negl;
  }

  // the step holds an unmasked key of this wave's rows (wave granularity)
  __device__ __forceinline__ bool visible(int step) const { return step < nvis_w; }

  // decision tiles this block of rows visits
  __device__ __forceinline__ int nvis_d() const { return (nvis_w + kSub - 1) / kSub; }

  // the final decision of decision tile j (M: its row maxima over all of its keys)
  __device__ __forceinline__ void record(int j, bool keep, const float (&M)[QB], int wave,
                                         int lane, bool leader) {
    if constexpr (kWave) {
      if (!exists || j >= nvis_d()) return;   // not part of this block's visited tiles
      leader = lane == 0;
    }
    if (!keep) ++nskip;
    if (leader && tile_state != nullptr) tile_state[unit * nKTd + j] = keep ? 0 : 1;
    if (rowmax != nullptr && this->h == 0) {
      const int r0 = kWave ? 0 : wave * RW;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
        rowmax[(unit * nKTd + j) * R + r0 + qb * 32 + this->r32] = M[qb];
    }
  }

  // tiles never visited (causal): state 2, maxima -inf; the head counters
  template <class Args>
  __device__ __forceinline__ void finish(const Args& a, const TileUnit& u, int tid) const {
    if (!exists) return;
    // tile granularity: the workgroup's threads share the row block; wave granularity: the wave's
    constexpr int NT = kWave ? 64 : NW * 64;
    const int t = kWave ? (tid & 63) : tid;
    const int nv = nvis_d();
    if (a.tile_state != nullptr)
      for (int j = nv + t; j < nKTd; j += NT) a.tile_state[unit * nKTd + j] = 2;
    if (a.rowmax != nullptr)
      for (int64_t i = (int64_t)nv * R + t; i < (int64_t)nKTd * R; i += NT)
        a.rowmax[unit * nKTd * R + i] = -INFINITY;
    if (t == 0 && a.counters != nullptr) {
      atomicAdd(&a.counters[2 * (u.b * a.g.Hq + u.hq)], (unsigned)nv);
      atomicAdd(&a.counters[2 * (u.b * a.g.Hq + u.hq) + 1], (unsigned)nskip);
    }
  }
};

// ---- the N:M rule ---------------------------------------------------------------------------------
// In the S^T register layout (tile_core.h, "Key order") element r of a lane's block kb holds, for
// one query, key 32*kb + 16*(r/8) + 8*h + r%8 (h = lane/32): every run of 8 elements r = 8c..8c+7
// is 8 consecutive keys.  A group of M = 4 consecutive keys is elements 4g..4g+3 and a group of
// M = 8 is elements 8c..8c+7, both inside one lane, with keys increasing with the element index.
// Dropped keys get weight 0 in P.  The running max needs no change: the group maximum always
// survives (rank 0 < N), so the max over kept keys equals the max over allowed keys -- which is
// also why the skip rule may be decided on the unfiltered tile maxima.

// 1 when d < 0, else 0, for d the fp32 difference of two finite scores normalised by "+ 0.0f"
// (so that equal scores give +0): the sign bit, read without a compare (a compare per pair would
// park a lane mask in SGPRs).
__device__ __forceinline__ int neg01(float d) { return (int)(__float_as_uint(d + 0.0f) >> 31); }

// rank[i] = number of group members that beat x[i]: a higher score, or an equal score at a lower
// key index.  x[0..M-1] are the group's scores in ascending key order; they are finite (masked
// keys enter as -FLT_MAX, which ties only with other masked keys and ranks below every score).
template <int M>
__device__ __forceinline__ void group_ranks(const float (&x)[M], int (&rank)[M]) {
#pragma unroll
  for (int i = 0; i < M; ++i) rank[i] = 0;
#pragma unroll
  for (int i = 0; i < M; ++i)
#pragma unroll
    for (int j = i + 1; j < M; ++j) {
      // j comes after i: j beats i iff x[j] > x[i], otherwise i beats j
      const int jgt = neg01(x[i] - x[j]);
      rank[i] += jgt;
      rank[j] += 1 - jgt;
    }
}

// This lane's 32 keys of a 64-key tile, bit b = kb*16 + r, sit at key offsets
// p(b) = kb*32 + 16*(r/8) + 8h + r%8, which increase with b: the keys with offset < T are the
// low bits, as many as there are such offsets.
__device__ __forceinline__ uint32_t bits_below(int T, int h) {
  int cnt = 0;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int c = 0; c < 2; ++c) cnt += min(max(T - (kb * 32 + c * 16 + 8 * h), 0), 8);
  return cnt >= 32 ? 0xFFFFFFFFu : ((1u << cnt) - 1u);
}

template <int NW, int QB, int M>
struct NmFilter {
  static constexpr int RW = 32 * QB;
  static constexpr int BR = NW * RW;
  static constexpr int kGroups = 16 / M;   // groups per block of 16 elements
  int n, sink, recent, W;
  uint32_t* keep_bits;
  float* scores;
  int64_t row_base;   // (b*Hq + hq)*Sq

  // Args: NmArgs or SkipNmArgs
  template <class Args>
  __device__ __forceinline__ void init(const Args& a, const TileUnit& u) {
    n = a.n;
    sink = a.sink;
    recent = a.recent;
    W = (a.g.Sk + 31) / 32;
    keep_bits = a.keep_bits;
    scores = a.scores;
    row_base = ((int64_t)u.b * a.g.Hq + u.hq) * a.g.Sq;
  }

  // some row of this wave has a sink or recent-window key in the tile
  __device__ __forceinline__ bool dense_tile(const KeyTiles<QB>& kt, int k0) const {
    return k0 < sink ||
           (recent > 0 && k0 <= kt.wrow0 + RW - 1 && k0 + kKeysPerTile - 1 > kt.wrow0 - recent);
  }

  // The window bits of query block qb (key < sink, or row - recent < key <= row), as bits
  // b = kb*16 + r of this lane's elements.
  __device__ __forceinline__ uint32_t window(const KeyTiles<QB>& kt, int k0, int qb) const {
    const int row = kt.wrow0 + qb * 32 + kt.r32;
    uint32_t win = bits_below(sink - k0, kt.h);
    if (recent > 0)
      win |= bits_below(row - k0 + 1, kt.h) & ~bits_below(row - recent - k0 + 1, kt.h);
    return win;
  }

  // The exact rank pass: a key is dropped (-inf) unless it is among the top n of its group or lies
  // in the sink/recent window.  The ranks are sign-bit arithmetic per pair, exact for ties.
  // Masked keys are -inf already and stay so.
  __device__ __forceinline__ void rank_apply(const KeyTiles<QB>& kt, int j, f32x16 (&s)[2][QB],
                                             int) const {
    const int k0 = j * kKeysPerTile;
    const bool any_dense = dense_tile(kt, k0);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const uint32_t win = any_dense ? window(kt, k0, qb) : 0u;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int g = 0; g < kGroups; ++g) {
          float x[M];
#pragma unroll
          for (int e = 0; e < M; ++e)
            x[e] = fmaxf(s[kb][qb][M * g + e], -3.402823466e38f);   // masked: finite sentinel
          int rank[M];
          group_ranks<M>(x, rank);
#pragma unroll
          for (int e = 0; e < M; ++e) {
            const int r = M * g + e;
            const bool keep = rank[e] < n || ((win >> (kb * 16 + r)) & 1u);
            s[kb][qb][r] = keep ? s[kb][qb][r] : -INFINITY;
          }
          // one group at a time: the scheduler would otherwise interleave all groups'
          // comparisons and run out of registers
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  }

  // The N-th and (N+1)-th largest of a group of four, t and u.  With a <= b <= c the first three
  // sorted (min3, med3, max3) and d the fourth: the largest is max(c, d), the 2nd largest
  // max(b, min(c, d)), the 3rd min(b, max(a, d)) and the smallest min(a, d).
  template <int N>
  static __device__ __forceinline__ void nth_largest4(float x0, float x1, float x2, float x3,
                                                      float& t, float& u) {
    const float hi = fmaxf(fmaxf(x0, x1), x2);
    const float lo = fminf(fminf(x0, x1), x2);
    const float md = __builtin_amdgcn_fmed3f(x0, x1, x2);
    if constexpr (N == 1) {
      t = fmaxf(hi, x3);
      u = fmaxf(md, fminf(hi, x3));
    } else if constexpr (N == 2) {
      t = fmaxf(md, fminf(hi, x3));
      u = fminf(md, fmaxf(lo, x3));
    } else {
      t = fminf(md, fmaxf(lo, x3));
      u = fminf(lo, x3);
    }
  }

  // The four values sorted, largest first (the same max3 / med3 / min3 construction).
  static __device__ __forceinline__ void sort4_desc(float x0, float x1, float x2, float x3,
                                                    float (&a)[4]) {
    const float hi = fmaxf(fmaxf(x0, x1), x2);
    const float lo = fminf(fminf(x0, x1), x2);
    const float md = __builtin_amdgcn_fmed3f(x0, x1, x2);
    a[0] = fmaxf(hi, x3);
    a[1] = fmaxf(md, fminf(hi, x3));
    a[2] = fminf(md, fmaxf(lo, x3));
    a[3] = fminf(lo, x3);
  }

  // The K-th largest of the eight values in two lists of four sorted largest first: the maximum
  // over i of min(a[i-1], b[K-1-i]), with a[-1] = b[-1] = +inf and i from max(0, K-4) to min(K, 4)
  // (i of the K largest come from a and the rest from b).
  template <int K>
  static __device__ __forceinline__ float kth_largest8(const float (&a)[4], const float (&b)[4]) {
    float t = -INFINITY;
#pragma unroll
    for (int i = (K > 4 ? K - 4 : 0); i <= (K < 4 ? K : 4); ++i) {
      const float x = i == 0 ? INFINITY : a[i > 0 ? i - 1 : 0];
      const float y = K - 1 - i < 0 ? INFINITY : b[K - 1 - i >= 0 ? K - 1 - i : 0];
      t = fmaxf(t, fminf(x, y));
    }
    return t;
  }

  // Keys of a group below its N-th largest t are dropped unless they lie in a window.  This keeps
  // every key that reaches t, which is exactly the top N unless the (N+1)-th largest u equals t (a
  // tie at the threshold, decided by the lower key index); such groups set `tie`.
  template <bool kWin>
  static __device__ __forceinline__ void drop_below(f32x16& v, int r0, int cnt, float t, float u,
                                                    uint32_t win, bool& tie) {
    tie = tie || (u == t && t != -INFINITY);
#pragma unroll
    for (int e = 0; e < cnt; ++e) {
      const int r = r0 + e;
      if constexpr (kWin) {
        const bool keep = !(v[r] < t) || ((win >> r) & 1u);
        v[r] = keep ? v[r] : -INFINITY;
      } else {
        v[r] = v[r] < t ? -INFINITY : v[r];
      }
    }
  }

  // Threshold pass.  M = 4: each group's N-th and (N+1)-th largest by the max3/med3/min3
  // construction.  M = 8: the two halves of a group sorted, then the N-th and (N+1)-th largest of
  // the union.  Window keys (kWin) are kept whatever their rank.
  template <int N, bool kWin>
  static __device__ __forceinline__ void threshold_apply(f32x16 (&s)[2][QB],
                                                         const uint32_t (&win)[QB], bool& tie) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int g = 0; g < kGroups; ++g) {
          f32x16& v = s[kb][qb];
          const uint32_t wb = kWin ? (win[qb] >> (kb * 16)) : 0u;
          float t, u;
          if constexpr (M == 4) {
            nth_largest4<N>(v[4 * g], v[4 * g + 1], v[4 * g + 2], v[4 * g + 3], t, u);
          } else {
            float a[4], b[4];
            sort4_desc(v[8 * g], v[8 * g + 1], v[8 * g + 2], v[8 * g + 3], a);
            sort4_desc(v[8 * g + 4], v[8 * g + 5], v[8 * g + 6], v[8 * g + 7], b);
            t = kth_largest8<N>(a, b);
            u = kth_largest8<N + 1>(a, b);
          }
          drop_below<kWin>(v, M * g, M, t, u, wb, tie);
          __builtin_amdgcn_sched_barrier(0);   // one group at a time (register pressure)
        }
  }

  template <bool kWin>
  __device__ __forceinline__ void threshold_n(f32x16 (&s)[2][QB], const uint32_t (&win)[QB],
                                              bool& tie) const {
    if constexpr (M == 4) {
      switch (n) {
        case 1: threshold_apply<1, kWin>(s, win, tie); break;
        case 2: threshold_apply<2, kWin>(s, win, tie); break;
        case 3: threshold_apply<3, kWin>(s, win, tie); break;
        default: break;   // n >= M keeps every allowed key
      }
    } else {
      switch (n) {
        case 1: threshold_apply<1, kWin>(s, win, tie); break;
        case 2: threshold_apply<2, kWin>(s, win, tie); break;
        case 3: threshold_apply<3, kWin>(s, win, tie); break;
        case 4: threshold_apply<4, kWin>(s, win, tie); break;
        case 5: threshold_apply<5, kWin>(s, win, tie); break;
        case 6: threshold_apply<6, kWin>(s, win, tie); break;
        case 7: threshold_apply<7, kWin>(s, win, tie); break;
        default: break;
      }
    }
  }

  // Drops the keys the rule does not keep by setting their scores to -inf (masked keys already
  // are): the threshold pass, with the window bits on the tiles that touch a window, then, only if
  // some group of the wave had a tie at its threshold, the rank pass over the result.  That is
  // exact: the keys the threshold pass dropped lie below the N-th largest and outside the windows,
  // so the rule drops them too, and the rank pass ranks the surviving keys as it would rank them
  // among all.
  __device__ __forceinline__ void filter(const KeyTiles<QB>& kt, int j, f32x16 (&s)[2][QB],
                                         int lane) const {
    const int k0 = j * kKeysPerTile;
    if (scores != nullptr) export_scores(kt, k0, s);
    bool tie = false;
    if (dense_tile(kt, k0)) {
      uint32_t win[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) win[qb] = window(kt, k0, qb);
      threshold_n<true>(s, win, tie);
    } else {
      const uint32_t none[QB] = {};
      threshold_n<false>(s, none, tie);
    }
    if (__builtin_amdgcn_ballot_w64(tie) != 0ull) rank_apply(kt, j, s, lane);
    if (keep_bits != nullptr) export_bits(kt, k0, s, lane);
  }

  // debug export: the raw scores the ranking used (before any key is dropped)
  __device__ __forceinline__ void export_scores(const KeyTiles<QB>& kt, int k0,
                                                const f32x16 (&s)[2][QB]) const {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int row = kt.wrow0 + qb * 32 + kt.r32;
      if (row >= kt.Sq) continue;
      int kbase = k0 + 8 * kt.h;   // key = kbase + elem_key(kb, r), a compile-time offset
      asm volatile("" : "+v"(kbase));
      float* dst = scores + (row_base + row) * kt.Sk + kbase;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int c = elem_key(kb, r);
          if (kbase + c < kt.Sk) dst[c] = s[kb][qb][r];
        }
    }
  }

  // debug export: keep-bit words of one tile (a key is kept when its score survived as finite)
  __device__ __forceinline__ void export_bits(const KeyTiles<QB>& kt, int k0,
                                              const f32x16 (&s)[2][QB], int lane) const {
    const int h = kt.h;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int row = kt.wrow0 + qb * 32 + kt.r32;
      uint32_t kb_bits = 0u;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          kb_bits |= (s[kb][qb][r] != -INFINITY ? 1u : 0u) << (kb * 16 + r);
      // lanes l and l^32 hold the same row: both stay active through the swap
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        // this lane's 16 bits sit at key offsets 16*(r/8) + 8h + r%8: the two bytes 16 apart,
        // then shifted by 8h; merged with lane^32's half
        const uint32_t x = (kb_bits >> (kb * 16)) & 0xFFFFu;
        uint32_t word = ((x & 0xFFu) | ((x & 0xFF00u) << 8)) << (8 * h);
        word |= __float_as_uint(other_half(__uint_as_float(word), lane));
        if (row < kt.Sq && h == 0 && k0 + kb * 32 < kt.Sk)
          keep_bits[(row_base + row) * W + k0 / 32 + kb] = word;
      }
    }
  }

  // keep-bit words and scores of tiles never visited (causal): zero / -inf
  template <class Args>
  __device__ __forceinline__ void finish(const Args& a, const TileUnit& u, int tid) const {
    constexpr int NT = NW * 64;
    const AttnGeom& g = a.g;
    if (keep_bits != nullptr) {
      const int wfirst = u.nvis * (kKeysPerTile / 32);
      for (int rr = tid; rr < BR; rr += NT) {
        const int row = u.row0 + rr;
        if (row >= g.Sq) continue;
        const int64_t rbase = row_base + row;
        for (int w = wfirst; w < W; ++w) keep_bits[rbase * W + w] = 0u;
      }
    }
    if (scores != nullptr) {
      const int kfirst = u.nvis * kKeysPerTile;
      for (int rr = 0; rr < BR; ++rr) {
        const int row = u.row0 + rr;
        if (row >= g.Sq) break;
        const int64_t rbase = row_base + row;
        for (int key = kfirst + tid; key < g.Sk; key += NT) scores[rbase * g.Sk + key] = -INFINITY;
      }
    }
  }
};

// ---- the policies -----------------------------------------------------------------------------------

template <int D, int NW, int QB, bool kWave = false, bool kPair = false>
using SkipPolicy = SkipDecision<D, NW, QB, kWave, kPair>;

template <int D, int NW, int QB, int M>
struct NmPolicy : KeyTiles<QB> {
  static constexpr bool kDecide = false, kFilter = true, kWeighted = false;
  NmFilter<NW, QB, M> nm;

  __device__ __forceinline__ void init(const NmArgs& a, const TileUnit& u, int lane) {
    this->init_tiles(a.g, u, D, lane);
    nm.init(a, u);
  }
  __device__ __forceinline__ void filter(int j, f32x16 (&s)[2][QB], int lane) const {
    nm.filter(*this, j, s, lane);
  }
  __device__ __forceinline__ void finish(const NmArgs& a, const TileUnit& u, int tid) const {
    nm.finish(a, u, tid);
  }
};

// Both rules: the skip decision on the tile maxima (equal to the maxima over the N:M-kept keys),
// the N:M bits inside every kept tile (a skipped tile needs none: the filter runs after the
// decision, on kept tiles).
template <int D, int NW, int QB, int M, bool kPair = false>
struct SkipNmPolicy : SkipDecision<D, NW, QB, false, kPair> {
  using Skip = SkipDecision<D, NW, QB, false, kPair>;
  static constexpr bool kDecide = true, kFilter = true, kWeighted = false;
  NmFilter<NW, QB, M> nm;

  __device__ __forceinline__ void init(const SkipNmArgs& a, const TileUnit& u, int lane) {
    Skip::init(a, u, lane);
    nm.init(a, u);
  }
  __device__ __forceinline__ void filter(int j, f32x16 (&s)[2][QB], int lane) const {
    nm.filter(*this, j, s, lane);
  }
  // the raw scores or keep bits are exported: every visited tile is filtered, kept or not
  __device__ __forceinline__ bool exports() const {
    return nm.scores != nullptr || nm.keep_bits != nullptr;
  }
  __device__ __forceinline__ void finish(const SkipNmArgs& a, const TileUnit& u, int tid) const {
    Skip::finish(a, u, tid);
    nm.finish(a, u, tid);
  }
};

// ---- the kernel body ----------------------------------------------------------------------------------
// One workgroup = one (batch, query head, query tile of 32*QB*NW rows); each wavefront owns 32*QB
// rows.  Load Q, run the key-tile loop with the policy, then normalise and store O and the
// natural-log LSE.
template <int D, int NW, int QB, class Pol, class Args>
__device__ __forceinline__ void attention_tile(const Args& a, Smem<D, NW>& sm) {
  const AttnGeom& g = a.g;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, r32 = lane & 31;
  const TileUnit u = tile_unit<NW, QB>(g, wave);

  const auto qsrc = slab_rsrc((const __bf16*)g.q + u.b * g.qs[0] + u.hq * g.qs[2], g.qs[1], g.Sq, D);
  bf16x8 qf[QB][D / 16];
  load_q_frags<D, QB>(qf, qsrc, g.qs[1], u.wrow0, lane);

  Pol pol;
  pol.init(a, u, lane);

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
  pol.finish(a, u, tid);

  float inv[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lt = half_sum(l[qb]);
    inv[qb] = lt > 0.f ? 1.f / lt : 0.f;
    const int row = u.wrow0 + qb * 32 + r32;
    if (a.lse != nullptr && h == 0 && row < g.Sq)
      a.lse[((int64_t)u.b * g.Hq + u.hq) * g.Sq + row] =
          lt > 0.f ? (mref[qb] + __log2f(lt)) * 0.69314718055994531f : -INFINITY;
  }
  __bf16* op = (__bf16*)g.o + u.b * g.os[0] + (int64_t)u.wrow0 * g.os[1] + u.hq * g.os[2];
  store_o<D, QB>(op, g.os[1], g.Sq - u.wrow0, o, inv, lane);
}

}  // namespace sa
