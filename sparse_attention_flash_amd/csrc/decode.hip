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
// byte, far below what MFMA needs, so the three kernels are VALU code that streams K/V with
// coalesced 16-byte loads (LPK = D/8 lanes per key row, 64/LPK rows per wave instruction):
//   1 decode_scores   q.k for the G heads of a KV head (v_dot2 on packed bf16, LPK-lane sums),
//                     written to a small fp32 workspace, and each tile's maximum;
//   2 decode_attend   per split: the decisions (prefix max of earlier splits, then the running
//                     max in order), then P.V over the kept tiles only, with P = 2^(t - r) for the
//                     split's own reference r = max over its kept tiles (so no rescaling);
//   3 decode_combine  the splits' (r, l, O) merged into O and the natural-log LSE.
#include "kernels.h"
#include "tile_core.h"

namespace sa {
namespace {

constexpr int kDecWaves = 4;
constexpr int kDecThreads = 64 * kDecWaves;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

template <int Ctrl>
__device__ __forceinline__ float dpp_f(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), Ctrl, 0xF, 0xF, true));
}

// Sum over the LPK (16 or 8) lanes of one key row, with identical bits in every lane: xor-1 and
// xor-2 swaps within quads, the 8-lane half mirror, then the 16-lane mirror (each step adds two
// equal-by-construction halves in both orders, and fp32 addition commutes).
template <int LPK>
__device__ __forceinline__ float row_sum(float x) {
  x += dpp_f<0xB1>(x);    // quad_perm [1,0,3,2]
  x += dpp_f<0x4E>(x);    // quad_perm [2,3,0,1]
  x += dpp_f<0x141>(x);   // row_half_mirror
  if constexpr (LPK == 16) x += dpp_f<0x140>(x);   // row_mirror
  return x;
}

// Each word is copied out of the vector before the bit cast: a __builtin_bit_cast applied to a
// vector element expression itself compiles to a read of element 0.
__device__ __forceinline__ float dot8(const u32x4& a, const u32x4& b, float acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t x = a[i], y = b[i];
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, x),
                                          __builtin_bit_cast(bf16x2_t, y), acc, false);
  }
  return acc;
}

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
template <int D, int GM>
__global__ __launch_bounds__(kDecThreads) void decode_scores(DecodeArgs a) {
  constexpr int LPK = D / 8;         // lanes per key row (16 B each)
  constexpr int KPI = 64 / LPK;      // key rows per wave instruction
  constexpr int kIt = 64 / KPI;      // instructions per 64 keys
  static_assert(GM <= LPK, "one writer lane per head");
  const AttnGeom& g = a.g;
  const DecUnit u = dec_unit(a);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int sub = lane / LPK, c = lane % LPK;
  const int G = g.Hq / g.Hkv;
  const int BC = a.block_k;

  // q of the G heads: 8 values of chunk c each (zeros for padding heads h >= G)
  u32x4 qv[GM];
#pragma unroll
  for (int h = 0; h < GM; ++h) {
    qv[h] = u32x4{0u, 0u, 0u, 0u};
    if (h < G) {
      const __bf16* qp = (const __bf16*)g.q + u.b * g.qs[0] + (u.hk * G + h) * g.qs[2];
      qv[h] = *(const u32x4*)(qp + 8 * c);
    }
  }
  const __bf16* kslab = (const __bf16*)g.k + u.b * g.ks[0] + u.hk * g.ks[2];
  const auto krs = slab_rsrc(kslab, g.ks[1], u.len, D);
  const int kstride_b = (int)(g.ks[1] * 2);
  float* sc = a.scores + ((int64_t)u.b * g.Hkv + u.hk) * g.Sk * GM;

  for (int t = u.t0 + wave; t < u.t1; t += kDecWaves) {
    float* tm = a.tmax + ((int64_t)u.b * g.Hq + u.hk * G) * a.nKT + t;
    if (t >= u.nvis) {   // beyond this sequence's keys: not visited
      if (sub == 0 && c < G) tm[(int64_t)c * a.nKT] = -INFINITY;
      continue;
    }
    float mx[GM];
#pragma unroll
    for (int h = 0; h < GM; ++h) mx[h] = -INFINITY;
    for (int k64 = 0; k64 < BC; k64 += 64) {
      const int kbase = t * BC + k64 + sub;
      u32x4 kv[kIt];
#pragma unroll
      for (int it = 0; it < kIt; ++it)
        kv[it] = load16(krs, (kbase + it * KPI) * kstride_b + c * 16);
#pragma unroll
      for (int it = 0; it < kIt; ++it) {
        const int key = kbase + it * KPI;
        float sv = -INFINITY;
#pragma unroll
        for (int h = 0; h < GM; ++h) {
          float s = row_sum<LPK>(dot8(qv[h], kv[it], 0.f));
          s = key < u.len ? s : -INFINITY;
          mx[h] = fmaxf(mx[h], s);
          sv = c == h ? s : sv;
        }
        if (c < GM && key < g.Sk) sc[(int64_t)key * GM + c] = sv;
      }
    }
    // tile max over the key slots, in the log2 domain; lane (slot 0, chunk h) writes head h
    float out = -INFINITY;
#pragma unroll
    for (int h = 0; h < GM; ++h) {
      float m = mx[h];
      for (int d = LPK; d < 64; d <<= 1) m = fmaxf(m, __shfl_xor(m, d, 64));
      out = c == h ? m * g.c32 : out;
    }
    if (sub == 0 && c < G) tm[(int64_t)c * a.nKT] = out;
  }
}

// ---- 2: decisions and P.V over kept tiles ---------------------------------------------------------
template <int D, int GM>
__global__ __launch_bounds__(kDecThreads) void decode_attend(DecodeArgs a) {
  constexpr int LPK = D / 8;
  constexpr int KPI = 64 / LPK;
  constexpr int kIt = 64 / KPI;
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

  // decisions, in key order: lane h of wave 0 walks head h
  if (wave == 0) {
    const int h = lane;
    float m = -INFINITY, ref = -INFINITY;
    if (h < G)
      for (int w = 0; w < kDecWaves; ++w) m = fmaxf(m, pre[w][h]);
    unsigned visited = 0, skipped = 0;
    const int64_t unit = (int64_t)u.b * g.Hq + u.hk * G + h;
    for (int j = u.t0; j < u.t1; ++j) {
      bool keep = false;
      if (h < G && j < u.nvis) {
        const float M = tmax[(int64_t)h * a.nKT + j];
        keep = !(M < m + a.L32);
        if (keep) {
          m = fmaxf(m, M);
          ref = fmaxf(ref, M);
        }
        ++visited;
        skipped += keep ? 0u : 1u;
        if (a.tile_state != nullptr) a.tile_state[unit * a.nKT + j] = keep ? 0 : 1;
      } else if (h < G && a.tile_state != nullptr) {
        a.tile_state[unit * a.nKT + j] = 2;
      }
      const uint64_t kb = __ballot(keep);
      if (lane == 0) keepbits[j - u.t0] = (uint32_t)kb;
    }
    if (h < GM) ref_s[h] = ref;
    if (h < G && a.counters != nullptr) {
      atomicAdd(&a.counters[2 * unit], visited);
      atomicAdd(&a.counters[2 * unit + 1], skipped);
    }
  }
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
  const float* sc = a.scores + ((int64_t)u.b * g.Hkv + u.hk) * g.Sk * GM;

  for (int t = u.t0 + wave; t < u.t1; t += kDecWaves) {
    const uint32_t kb = keepbits[t - u.t0];
    if (kb == 0u) continue;   // skipped by every head: no V traffic
    for (int k64 = 0; k64 < BC; k64 += 64) {
      const int kbase = t * BC + k64 + sub;
      u32x4 vv[kIt];
#pragma unroll
      for (int it = 0; it < kIt; ++it)
        vv[it] = load16(vrs, (kbase + it * KPI) * vstride_b + c * 16);
#pragma unroll
      for (int it = 0; it < kIt; ++it) {
        const int key = kbase + it * KPI;
        if (key >= u.len) break;   // the rest of this tile is past the sequence
        const float* sk = sc + (int64_t)key * GM;
        float vf[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          vf[2 * i] = bf16_lo(vv[it][i]);
          vf[2 * i + 1] = bf16_hi(vv[it][i]);
        }
#pragma unroll
        for (int h = 0; h < GM; ++h) {
          const float p = ((kb >> h) & 1u) ? __builtin_amdgcn_exp2f(sk[h] * g.c32 - ref[h]) : 0.f;
          ls[h] += c == 0 ? p : 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[h][e] += p * vf[e];
        }
      }
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
