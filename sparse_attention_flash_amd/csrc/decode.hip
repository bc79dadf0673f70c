// decode.hip -- decode-phase skip-softmax forward for gfx950: one query token per (batch, query
// head) against a KV cache of up to Sk keys, the key axis split over workgroups.
//
// Method: the skip-softmax rule of Model-Optimizer "Skip-Softmax Sparse Attention for Diffusion
// Models" (a key tile whose scores are negligible under lambda is skipped: no exponentials, no V
// load, no P.V), applied in the decode phase with its own threshold (Model-Optimizer "Attention
// Sparsity for HuggingFace Models", custom configuration: phase-specific thresholds, decode
// 1e-4).  With one query row, tile j of head h is skipped when M_j < fl32(m + log2(lambda)), m the
// fp32 running max of the tiles kept so far, M_j the tile's max of t = c*q.k.
//
// Splitting the key axis keeps the sequential decisions exactly when lambda <= 1: a skipped tile
// has M_j < m + log2(lambda) <= m, so it could not have raised the running max, and the running
// max of the kept tiles before j equals the prefix max of ALL tiles before j.  A split therefore
// starts from the max of the earlier splits' tile maxima.  (lambda > 1 runs as one split.)
//
// Decode reads every K row once and each kept V row once for G query heads: about 4 flops per
// byte, so the kernels are bound by the K/V stream.  K and V are read straight into registers
// with 16-byte loads, and each 64-key chunk's loads are in flight while the previous chunk is used:
//   1 decode_scores   q.k for the G heads of a KV head on MFMA (the heads as the columns of
//                     S^T = K.Q^T), written to a small fp32 workspace, and each tile's maximum;
//   2 decode_attend   per split: the decisions (for lambda <= 1 a wave-wide prefix-max scan over
//                     64 tiles at a time, else the running max in order), then P.V over the kept
//                     tiles only: per 64 keys one lane per key computes P = 2^(t - r) for the G
//                     heads into LDS (r = the split's max over its kept tiles, so no rescaling),
//                     and the key-row lanes accumulate P.V from it;
//   3 decode_combine  the splits' (r, l, O) merged into O and the natural-log LSE.
#include "kernels.h"
#include "tile_core.h"

namespace sa {
namespace {

constexpr int kDecWaves = 4;
constexpr int kDecThreads = 64 * kDecWaves;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// The (batch, KV head, split) of this workgroup and its key range.
struct DecUnit {
  int b, hk, s, len, nvis, t0, t1;
};

__device__ __forceinline__ DecUnit dec_unit(const DecodeArgs& a) {
  DecUnit u;
  int item = blockIdx.x;
  u.s = item % a.nsplit;
  item /= a.nsplit;
  u.hk = item % a.g.Hkv;
  u.b = item / a.g.Hkv;
  u.len = a.g.Sk;
  if (a.seqlens_k != nullptr) u.len = min(max(a.seqlens_k[u.b], 0), a.g.Sk);
  u.nvis = (u.len + a.block_k - 1) / a.block_k;
  const int nKT = (a.g.Sk + a.block_k - 1) / a.block_k;
  u.t0 = u.s * a.tiles_per_split;
  u.t1 = min(u.t0 + a.tiles_per_split, nKT);
  return u;
}

// ---- 1: scores and tile maxima --------------------------------------------------------------------
// S^T = K.Q^T on v_mfma_f32_32x32x16_bf16, one 32-key block at a time: A = 32 K rows (lane l: key
// l%32, the 8 values at d = 16ks + 8(l/32)), B = Q^T with the G heads as columns (columns past G
// are zero).  Only G of the 32 columns do useful work, but the matrix cores still need about an
// eighth of the issue cycles of the same dot products on the VALU, so the kernel stays bound by
// the K stream.  Lane l then holds, for head l%32, keys 8i + 4(l/32) + {0..3} in elements
// 4i..4i+3.  Scores go to the workspace head-major, [GM][nKT*block_k] per (batch, KV head).
template <int D, int GM>
__global__ __launch_bounds__(kDecThreads) void decode_scores(DecodeArgs a) {
  constexpr int KS = D / 16;   // MFMA k-steps per key block
  const AttnGeom& g = a.g;
  const DecUnit u = dec_unit(a);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 31, hl = lane >> 5;
  const int G = g.Hq / g.Hkv;
  const int BC = a.block_k;
  const int64_t row_len = (int64_t)a.nKT * BC;   // scores row stride (a multiple of 64 keys)

  bf16x8 qf[KS];
  {
    const __bf16* qp = (const __bf16*)g.q + u.b * g.qs[0] + (u.hk * G + min(col, G - 1)) * g.qs[2];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bf16x8 x = *(const bf16x8*)(qp + 16 * ks + 8 * hl);
      if (col >= G) x = bf16x8{};
      qf[ks] = x;
    }
  }
  const __bf16* kslab = (const __bf16*)g.k + u.b * g.ks[0] + u.hk * g.ks[2];
  const auto krs = slab_rsrc(kslab, g.ks[1], u.len, D);
  const int kstride_b = (int)(g.ks[1] * 2);
  float* sc = a.scores + ((int64_t)u.b * g.Hkv + u.hk) * GM * row_len;
  // A chunk's scores go through LDS so that the whole wave stores them with full 16-byte lanes
  // (the lanes holding them are only 2*GM of 64).
  __shared__ __attribute__((aligned(16))) float sbuf[kDecWaves][GM][64];
  float (*sw)[64] = sbuf[wave];

  // Tiles past this sequence's keys are not visited.
  for (int t = u.t0 + wave; t < u.t1; t += kDecWaves) {
    if (t >= u.nvis && lane < G)
      a.tmax[((int64_t)u.b * g.Hq + u.hk * G + lane) * a.nKT + t] = -INFINITY;
  }

  // This wave's visited tiles t = t0 + wave + 4i as a stream of 64-key chunks; chunk q+1 is loaded
  // while chunk q is multiplied (two register buffers).  The prefetches are unconditional (the
  // index is clamped, so the tail re-reads the last chunk): a prefetch under a branch would make
  // every later use wait for all loads in flight.
  const int t_end = min(u.t1, u.nvis);
  const int ntile = t_end > u.t0 + wave ? (t_end - (u.t0 + wave) + kDecWaves - 1) / kDecWaves : 0;
  const int cpt = BC / 64;   // chunks per tile
  const int nq = ntile * cpt;
  auto chunk_key0 = [&](int q) { return (u.t0 + wave + kDecWaves * (q / cpt)) * BC + (q % cpt) * 64; };
  auto load_chunk = [&](bf16x8 (&kv)[2][KS], int q) {
    const int key0 = chunk_key0(q);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int off = (key0 + 32 * kb + col) * kstride_b + 16 * hl;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        kv[kb][ks] = __builtin_bit_cast(bf16x8, load16(krs, off + 32 * ks));
    }
  };
  float mx = -INFINITY;   // running max of this lane's keys in the current tile (its head)
  auto consume = [&](const bf16x8 (&kv)[2][KS], int q) {
    const int key0 = chunk_key0(q);
    f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) s[kb] = mfma32(kv[kb][ks], qf[ks], s[kb]);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      // keys past the sequence: -inf (their rows read as zeros)
      mask_block(s[kb], kb, u.len - key0 - 4 * hl);
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
      if (col < GM) {
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4)
          *(f32x4*)&sw[col][32 * kb + 8 * i4 + 4 * hl] =
              f32x4{s[kb][4 * i4], s[kb][4 * i4 + 1], s[kb][4 * i4 + 2], s[kb][4 * i4 + 3]};
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): the chunk's scores are in LDS
    __builtin_amdgcn_wave_barrier();
    // GM rows of 64 keys = GM*16 lanes of 16 bytes
#pragma unroll
    for (int r = 0; r < (GM * 16 + 63) / 64; ++r) {
      const int e = 64 * r + lane;
      if (e < GM * 16) {
        const int hh = e >> 4, k4 = (e & 15) * 4;
        *(f32x4*)(sc + hh * row_len + key0 + k4) = *(const f32x4*)&sw[hh][k4];
      }
    }
    __builtin_amdgcn_wave_barrier();   // read before the next chunk rewrites the buffer
    if (q % cpt == cpt - 1) {
      // tile max of head col over both lane halves, in the log2 domain
      const int t = u.t0 + wave + kDecWaves * (q / cpt);
      const float m = half_max(mx);
      if (hl == 0 && col < G)
        a.tmax[((int64_t)u.b * g.Hq + u.hk * G + col) * a.nKT + t] = m * g.c32;
      mx = -INFINITY;
    }
  };
  bf16x8 kva[2][KS], kvb[2][KS];
  if (nq > 0) {
    load_chunk(kva, 0);
    for (int q = 0; q < nq; q += 2) {
      load_chunk(kvb, min(q + 1, nq - 1));
      consume(kva, q);
      load_chunk(kva, min(q + 2, nq - 1));
      if (q + 1 < nq) consume(kvb, q + 1);
    }
  }
}

// ---- 2: decisions and P.V over kept tiles ---------------------------------------------------------
// Decisions (wave 0).  For lambda <= 1 the running max of the kept tiles before j is the prefix max
// of all tile maxima before j, so the tiles of a split are decided 64 at a time with a wave-wide
// prefix-max scan.  For lambda > 1 each head walks its tiles in order (maxima staged through LDS).
// keepbits[j - t0] bit h: tile j kept by head h.
template <int GM>
__device__ __forceinline__ void decide_tiles(const DecodeArgs& a, const DecUnit& u, int lane,
                                             const float (&pre)[kDecWaves][GM],
                                             uint32_t* keepbits, float (&ref_s)[GM],
                                             float (&stage)[GM][64]) {
  const AttnGeom& g = a.g;
  const int G = g.Hq / g.Hkv;
  const float* tmax = a.tmax + ((int64_t)u.b * g.Hq + u.hk * G) * a.nKT;
  const int64_t unit0 = (int64_t)u.b * g.Hq + u.hk * G;
  float carry[GM], ref[GM];
  unsigned vis_n[GM], skip_n[GM];
#pragma unroll
  for (int h = 0; h < GM; ++h) {
    carry[h] = -INFINITY;
    for (int w = 0; w < kDecWaves; ++w) carry[h] = fmaxf(carry[h], pre[w][h]);
    ref[h] = -INFINITY;
    vis_n[h] = skip_n[h] = 0u;
  }
  if (a.L32 <= 0.f) {
    for (int j0 = u.t0; j0 < u.t1; j0 += 64) {
      const int j = j0 + lane;
      const bool in = j < u.t1, vis = in && j < u.nvis;
      uint32_t bits = 0u;
#pragma unroll
      for (int h = 0; h < GM; ++h) {
        if (h >= G) break;
        const float M = vis ? tmax[(int64_t)h * a.nKT + j] : -INFINITY;
        float incl = M;   // inclusive prefix max over the lanes
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
          const float up = __shfl_up(incl, d, 64);
          if (lane >= d) incl = fmaxf(incl, up);
        }
        float excl = __shfl_up(incl, 1, 64);
        excl = lane == 0 ? carry[h] : fmaxf(carry[h], excl);
        const bool keep = vis && !(M < excl + a.L32);
        bits |= (keep ? 1u : 0u) << h;
        carry[h] = fmaxf(carry[h], __shfl(incl, 63, 64));
        ref[h] = fmaxf(ref[h], keep ? M : -INFINITY);
        vis_n[h] += __popcll(__ballot(vis));
        skip_n[h] += __popcll(__ballot(vis && !keep));
        if (in && a.tile_state != nullptr)
          a.tile_state[(unit0 + h) * a.nKT + j] = vis ? (keep ? 0 : 1) : 2;
      }
      if (in) keepbits[j - u.t0] = bits;
    }
#pragma unroll
    for (int h = 0; h < GM; ++h)
      for (int d = 1; d < 64; d <<= 1) ref[h] = fmaxf(ref[h], __shfl_xor(ref[h], d, 64));
  } else {
    // lane h walks head h; the maxima of 64 tiles at a time come through LDS
    const int h = lane;
    float m = -INFINITY, rf = -INFINITY;
    unsigned vn = 0u, sn = 0u;
#pragma unroll
    for (int hh = 0; hh < GM; ++hh)
      if (h == hh) m = carry[hh];
    for (int j0 = u.t0; j0 < u.t1; j0 += 64) {
      const int j = j0 + lane;
#pragma unroll
      for (int hh = 0; hh < GM; ++hh)
        stage[hh][lane] = (hh < G && j < u.nvis && j < u.t1) ? tmax[(int64_t)hh * a.nKT + j]
                                                              : -INFINITY;
      __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): the staged maxima are in LDS
      __builtin_amdgcn_wave_barrier();
      const int n = min(64, u.t1 - j0);
      for (int jj = 0; jj < n; ++jj) {
        const int jt = j0 + jj;
        bool keep = false;
        if (h < G && jt < u.nvis) {
          const float M = stage[h][jj];
          keep = !(M < m + a.L32);
          if (keep) {
            m = fmaxf(m, M);
            rf = fmaxf(rf, M);
          }
          ++vn;
          sn += keep ? 0u : 1u;
          if (a.tile_state != nullptr) a.tile_state[(unit0 + h) * a.nKT + jt] = keep ? 0 : 1;
        } else if (h < G && a.tile_state != nullptr) {
          a.tile_state[(unit0 + h) * a.nKT + jt] = 2;
        }
        const uint64_t kb = __ballot(keep);
        if (lane == 0) keepbits[jt - u.t0] = (uint32_t)kb;
      }
      __builtin_amdgcn_wave_barrier();
    }
#pragma unroll
    for (int hh = 0; hh < GM; ++hh) {
      ref[hh] = __shfl(rf, hh, 64);
      vis_n[hh] = __shfl(vn, hh, 64);
      skip_n[hh] = __shfl(sn, hh, 64);
    }
  }
  if (lane < GM) {
    float r = -INFINITY;
#pragma unroll
    for (int hh = 0; hh < GM; ++hh)
      if (lane == hh) r = ref[hh];
    ref_s[lane] = r;
  }
  if (lane < G && a.counters != nullptr) {
    unsigned vn = 0u, sn = 0u;
#pragma unroll
    for (int hh = 0; hh < GM; ++hh)
      if (lane == hh) {
        vn = vis_n[hh];
        sn = skip_n[hh];
      }
    atomicAdd(&a.counters[2 * (unit0 + lane)], vn);
    atomicAdd(&a.counters[2 * (unit0 + lane) + 1], sn);
  }
}

template <int D, int GM>
__global__ __launch_bounds__(kDecThreads) void decode_attend(DecodeArgs a) {
  constexpr int LPK = D / 8;
  constexpr int KPI = 64 / LPK;
  constexpr int kIt = 64 / KPI;
  constexpr int GQ = (GM + 3) / 4;   // 16-byte groups of P per key
  const AttnGeom& g = a.g;
  const DecUnit u = dec_unit(a);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int sub = lane / LPK, c = lane % LPK;
  const int G = g.Hq / g.Hkv;
  const int BC = a.block_k;

  __shared__ float pre[kDecWaves][GM];
  __shared__ float ref_s[GM];
  __shared__ uint32_t keepbits[kMaxTilesPerSplit];
  __shared__ float stage[GM][64];
  __shared__ __attribute__((aligned(16))) float pbuf[kDecWaves][64][4 * GQ];
  __shared__ uint16_t klist[kDecWaves][kMaxTilesPerSplit / kDecWaves];
  __shared__ float red[kDecWaves][GM][D];
  __shared__ float lred[kDecWaves][GM];

  const float* tmax = a.tmax + ((int64_t)u.b * g.Hq + u.hk * G) * a.nKT;

  // prefix max of every tile before this split, per head
  for (int h = 0; h < G; ++h) {
    float m = -INFINITY;
    for (int j = tid; j < u.t0; j += kDecThreads) m = fmaxf(m, tmax[(int64_t)h * a.nKT + j]);
    for (int d = 1; d < 64; d <<= 1) m = fmaxf(m, __shfl_xor(m, d, 64));
    if (lane == 0) pre[wave][h] = m;
  }
  __syncthreads();
  if (wave == 0) decide_tiles<GM>(a, u, lane, pre, keepbits, ref_s, stage);
  __syncthreads();

  float ref[GM];
#pragma unroll
  for (int h = 0; h < GM; ++h) ref[h] = ref_s[h];
  float acc[GM][8];
  float ls[GM];
#pragma unroll
  for (int h = 0; h < GM; ++h) {
    ls[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
  }
  const __bf16* vslab = (const __bf16*)g.v + u.b * g.vs[0] + u.hk * g.vs[2];
  const auto vrs = slab_rsrc(vslab, g.vs[1], u.len, D);
  const int vstride_b = (int)(g.vs[1] * 2);
  const int64_t row_len = (int64_t)a.nKT * BC;   // scores row stride
  const float* sc = a.scores + ((int64_t)u.b * g.Hkv + u.hk) * GM * row_len;
  float (*pw)[4 * GQ] = pbuf[wave];

  // This wave's kept tiles t = t0 + wave + 4i (kept by some head) listed in LDS, then walked as
  // 64-key chunks; the V rows and scores of chunk q+1 are loaded while chunk q is reduced.  The
  // prefetches are unconditional (clamped index), so the compiler's waits leave them in flight.
  uint16_t* list = klist[wave];
  int nkept = 0;
  for (int i0 = 0; u.t0 + wave + kDecWaves * i0 < u.t1; i0 += 64) {
    const int t = u.t0 + wave + kDecWaves * (i0 + lane);
    const bool kept = t < u.t1 && keepbits[t - u.t0] != 0u;
    const uint64_t m = __ballot(kept);
    if (kept) list[nkept + __popcll(m & ((1ull << lane) - 1ull))] = (uint16_t)(t - u.t0);
    nkept += __popcll(m);
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): the list is in LDS for the whole wave
  __builtin_amdgcn_wave_barrier();
  const int cpt = BC / 64;
  const int nq = nkept * cpt;
  auto chunk_key0 = [&](int q) { return (u.t0 + list[q / cpt]) * BC + (q % cpt) * 64; };
  auto load_chunk = [&](u32x4 (&vv)[kIt], float (&sv)[GM], int q) {
    const int key0 = chunk_key0(q);
#pragma unroll
    for (int it = 0; it < kIt; ++it)
      vv[it] = load16(vrs, (key0 + sub + it * KPI) * vstride_b + c * 16);
#pragma unroll
    for (int h = 0; h < GM; ++h) sv[h] = sc[h * row_len + key0 + lane];   // one key per lane
  };
  auto reduce_chunk = [&](const u32x4 (&vv)[kIt], const float (&sv)[GM], int q) {
    const int key0 = chunk_key0(q);
    const uint32_t kb = keepbits[key0 / BC - u.t0];
    // P of the 64 keys, one key per lane, into this wave's LDS slot; l from the same values
    const bool valid = key0 + lane < u.len;
#pragma unroll
    for (int h = 0; h < 4 * GQ; ++h) {
      float p = 0.f;
      if (h < GM && ((kb >> h) & 1u) && valid)
        p = __builtin_amdgcn_exp2f(sv[h < GM ? h : 0] * g.c32 - ref[h < GM ? h : 0]);
      if (h < GM) ls[h] += p;
      pw[lane][h] = p;
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): P is in LDS for the whole wave
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int it = 0; it < kIt; ++it) {
      const int kl = sub + it * KPI;   // key within the 64
      float vf[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t w = vv[it][i];
        vf[2 * i] = bf16_lo(w);
        vf[2 * i + 1] = bf16_hi(w);
      }
#pragma unroll
      for (int q4 = 0; q4 < GQ; ++q4) {
        const f32x4 p4 = *(const f32x4*)&pw[kl][4 * q4];
#pragma unroll
        for (int hh = 0; hh < 4; ++hh) {
          const int h = 4 * q4 + hh;
          if (h >= GM) break;
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[h][e] += p4[hh] * vf[e];
        }
      }
    }
    __builtin_amdgcn_wave_barrier();   // every lane has read P before the next chunk rewrites it
  };
  if (nq > 0) {
    u32x4 vva[kIt], vvb[kIt];
    float sva[GM], svb[GM];
    load_chunk(vva, sva, 0);
    for (int q = 0; q < nq; q += 2) {
      load_chunk(vvb, svb, min(q + 1, nq - 1));
      reduce_chunk(vva, sva, q);
      load_chunk(vva, sva, min(q + 2, nq - 1));
      if (q + 1 < nq) reduce_chunk(vvb, svb, q + 1);
    }
  }

  // sum over the key slots of the wave, then over the waves
#pragma unroll
  for (int h = 0; h < GM; ++h) {
    for (int d = LPK; d < 64; d <<= 1) {
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] += __shfl_xor(acc[h][e], d, 64);
    }
    float l = ls[h];
    for (int d = 1; d < 64; d <<= 1) l += __shfl_xor(l, d, 64);
    if (sub == 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) red[wave][h][8 * c + e] = acc[h][e];
    }
    if (lane == 0) lred[wave][h] = l;
  }
  __syncthreads();
  for (int i = tid; i < G * D; i += kDecThreads) {
    const int h = i / D, d = i % D;
    float o = 0.f;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) o += red[w][h][d];
    const int64_t part = ((int64_t)u.b * g.Hq + u.hk * G + h) * a.nsplit + u.s;
    a.part_o[part * D + d] = o;
    if (d == 0) {
      float l = 0.f;
#pragma unroll
      for (int w = 0; w < kDecWaves; ++w) l += lred[w][h];
      a.part_l[part] = l;
      a.part_m[part] = ref_s[h];
    }
  }
}

// ---- 3: merge the splits --------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(64) void decode_combine(DecodeArgs a) {
  const AttnGeom& g = a.g;
  const int lane = threadIdx.x;
  const int64_t bh = blockIdx.x;   // b*Hq + hq
  const int b = (int)(bh / g.Hq), hq = (int)(bh % g.Hq);
  const float* pm = a.part_m + bh * a.nsplit;
  const float* pl = a.part_l + bh * a.nsplit;
  const float* po = a.part_o + bh * a.nsplit * D;
  float M = -INFINITY;
  for (int s = 0; s < a.nsplit; ++s) M = fmaxf(M, pm[s]);
  float L = 0.f;
  float o[D / 64];
#pragma unroll
  for (int i = 0; i < D / 64; ++i) o[i] = 0.f;
  if (M != -INFINITY) {
    for (int s = 0; s < a.nsplit; ++s) {
      if (pm[s] == -INFINITY) continue;
      const float w = __builtin_amdgcn_exp2f(pm[s] - M);
      L += w * pl[s];
#pragma unroll
      for (int i = 0; i < D / 64; ++i) o[i] += w * po[(int64_t)s * D + lane + 64 * i];
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  __bf16* op = (__bf16*)g.o + b * g.os[0] + hq * g.os[2];
#pragma unroll
  for (int i = 0; i < D / 64; ++i) op[lane + 64 * i] = (__bf16)(o[i] * inv);
  if (a.lse != nullptr && lane == 0)
    a.lse[bh] = L > 0.f ? (M + __log2f(L)) * 0.69314718055994531f : -INFINITY;
}

template <int D, int GM>
hipError_t launch_dg(const DecodeArgs& a, hipStream_t stream) {
  const int units = a.g.B * a.g.Hkv * a.nsplit;
  hipLaunchKernelGGL((decode_scores<D, GM>), dim3(units), dim3(kDecThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_attend<D, GM>), dim3(units), dim3(kDecThreads), 0, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_combine<D>), dim3(a.g.B * a.g.Hq), dim3(64), 0, stream, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const DecodeArgs& a, hipStream_t stream) {
  const int G = a.g.Hq / a.g.Hkv;
  if (G <= 1) return launch_dg<D, 1>(a, stream);
  if (G <= 2) return launch_dg<D, 2>(a, stream);
  if (G <= 4) return launch_dg<D, 4>(a, stream);
  if constexpr (D == 128) {
    if (G <= 8) return launch_dg<D, 8>(a, stream);
    return launch_dg<D, 16>(a, stream);
  } else {
    return launch_dg<D, 8>(a, stream);
  }
}

}  // namespace

hipError_t launch_skip_decode(const DecodeArgs& a, hipStream_t stream) {
  if (a.g.D == 128) return launch_d<128>(a, stream);
  return launch_d<64>(a, stream);
}

}  // namespace sa
