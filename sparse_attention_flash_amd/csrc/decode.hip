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
// byte, so the kernels are bound by the K/V stream.  Each 64-key chunk's loads are in flight while
// the previous chunk is used:
//   1 decode_scores   q.k for the G heads of a KV head on MFMA (the heads as the columns of
//                     S^T = K.Q^T), written to a small fp32 workspace, and each tile's maximum;
//   2 decode_attend   per split: the decisions (for lambda <= 1 a wave-wide prefix-max scan over
//                     64 tiles at a time, else the running max in order), then P.V over the kept
//                     tiles only: per 64 keys one lane per key computes P = 2^(t - r) for the G
//                     heads into LDS (r = the split's max over its kept tiles, so no rescaling),
//                     and the key-row lanes accumulate P.V from it;
//   3 decode_combine  the splits' (r, l, O) merged into O and the natural-log LSE.
#include <atomic>
#include <mutex>

#include "kernels.h"
#include "mainloop.h"

// The allocation-free decode entry point keeps its workspace here (scores, tile maxima, split
// partials).  Host code never uses this name as an address: it is a host-side stand-in for the
// device symbol, so every kernel argument, copy or fill takes the pointer decode_scratch() looks
// up on the current device instead.
static __device__ __attribute__((aligned(256))) char scratch[sa::kDecodeScratchBytes];

namespace sa {

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;
}  // namespace

hipError_t decode_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    // first call on this device (with it current): the device address of its copy of the array
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (p == nullptr) return hipErrorInvalidSymbol;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return hipSuccess;
}

namespace {

constexpr int kDecWaves = 4;
constexpr int kDecThreads = 64 * kDecWaves;

// P.V of one 64-key chunk for the heads of a KV head, on the VALU (a rank-GM update with no
// contraction depth to fill an MFMA).  A V row is D/8 lanes of 16 bytes; lane (sub, c) loads keys
// sub + KPI*it (it < kIt) at d = 8c..8c+7.  Keys sub + KPI*2j and sub + KPI*(2j+1) are paired:
// v_perm_b32 puts their values at one d into one word and v_dot2_f32_bf16 adds both products to
// the fp32 accumulator, half the instructions of a multiply-add per key.  P goes through LDS as
// bf16 (as in the prefill P.V), in the pairing's layout: word [pair][h] holds head h's P of the
// pair's first key in its low half and of its second key in its high half.
template <int D, int GM>
struct PvChunk {
  static constexpr int LPK = D / 8;       // lanes per V row
  static constexpr int KPI = 64 / LPK;    // keys per load instruction
  static constexpr int kIt = 64 / KPI;    // load instructions per chunk
  static constexpr int GQ = (GM + 3) / 4; // 16-byte groups of heads
  static constexpr int kPairs = 32;
  typedef uint32_t Buf[kPairs][4 * GQ];

  // lane = key kl of the chunk writes its heads' P (p[h] for h < 4*GQ, zero past the group)
  static __device__ __forceinline__ void write_p(Buf& pw, int kl, const float (&p)[4 * GQ]) {
    const int it = kl / KPI, sub = kl % KPI;
    uint16_t* dst = reinterpret_cast<uint16_t*>(&pw[sub + KPI * (it >> 1)][0]) + (it & 1);
#pragma unroll
    for (int h = 0; h < 4 * GQ; ++h) dst[2 * h] = __builtin_bit_cast(uint16_t, (__bf16)p[h]);
  }

  static __device__ __forceinline__ void accumulate(const Buf& pw, const u32x4 (&vv)[kIt], int sub,
                                                    float (&acc)[GM][8]) {
#pragma unroll
    for (int j = 0; j < kIt / 2; ++j) {
      uint32_t pp[4 * GQ];
#pragma unroll
      for (int q4 = 0; q4 < GQ; ++q4) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(&pw[sub + KPI * j][4 * q4]);
#pragma unroll
        for (int e = 0; e < 4; ++e) pp[4 * q4 + e] = w[e];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t w1 = vv[2 * j][i], w2 = vv[2 * j + 1][i];
        const bf16x2 lo = __builtin_bit_cast(bf16x2, __builtin_amdgcn_perm(w2, w1, 0x05040100u));
        const bf16x2 hi = __builtin_bit_cast(bf16x2, __builtin_amdgcn_perm(w2, w1, 0x07060302u));
#pragma unroll
        for (int h = 0; h < GM; ++h) {
          const bf16x2 ph = __builtin_bit_cast(bf16x2, pp[h]);
          acc[h][2 * i] = __builtin_amdgcn_fdot2_f32_bf16(lo, ph, acc[h][2 * i], false);
          acc[h][2 * i + 1] = __builtin_amdgcn_fdot2_f32_bf16(hi, ph, acc[h][2 * i + 1], false);
        }
      }
    }
  }
};

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

// Elements r of a lane's s[kb] whose key 32*kb + (r/4)*8 + r%4 (+ 4*(lane/32), in lim) is at
// or past lim become -inf.  Here the MFMA rows are the K rows in order (no key permutation: the
// rows come straight from global memory), so element r holds row (r/4)*8 + 4*(lane/32) + r%4.
__device__ __forceinline__ void mask_rows(f32x16& s, int kb, int lim) {
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int off = kb * 32 + (r >> 2) * 8 + (r & 3);
    s[r] = select_neg_inf(s[r], (uint32_t)((lim - 1 - off) >> 31));
  }
}

// ---- 1: scores and tile maxima --------------------------------------------------------------------
// S^T = K.Q^T on v_mfma_f32_32x32x16_bf16 with the G heads as the columns of Q^T (columns past G
// are zero).  Only G of the 32 columns do useful work, but the matrix cores still need about an
// eighth of the issue cycles of the same dot products on the VALU, so the kernel stays bound by
// the K stream.
//
// Each wave streams its own 64-key chunks (tiles t0 + wave + kDecWaves*i) HBM -> LDS with the
// direct-to-LDS copies of the prefill kernels, 16 lanes on each 256-byte row, one chunk in flight
// while the previous one is multiplied, and reads the MFMA operands from LDS.  Loading K straight
// into operand registers instead makes every instruction touch 32 rows at 32 bytes each, so each
// 128-byte line is fetched by four instructions and, with two chunks in flight per wave, can fall
// out of the 32 KB L1 between them (measured on 16 x 8 KV heads x 8192 keys: 63.4 us per pass that
// way, 56.5 us through LDS).  Scores go to the workspace head-major and in key order,
// [GM][nKT*block_k] per (batch, KV head).
//
// The K copies carry the non-temporal hint (nt): the key stream is read once, and without the hint
// it runs through L2 and evicts the score lines the stores leave there, which then go out to HBM in
// the middle of the read stream.  With it the scores stay in L2 for decode_attend, and both
// kernels run near the part's read rate (16 x 8 KV heads x 8192 keys: 57.0 -> 52.8 us for this
// kernel and 55.6 -> 45.9 us for decode_attend).  The hint only suits streams read once: the
// prefill kernels re-read every K/V tile from L2 for many query tiles.
template <class L>
__device__ __forceinline__ void copy_k_stream(char* lds, const __bf16* base, int bytes,
                                              int stride_b, int lane_off) {
  const unsigned lds0 = (unsigned)(uintptr_t)(__attribute__((address_space(3))) char*)lds;
  const auto rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, max(0, bytes),
                                                      0x00020000);
  int sb = stride_b;
  asm volatile("" : "+s"(sb));   // keep the block offsets out of SGPRs across the loop
#pragma unroll
  for (int blk = 0; blk < L::kBlocks; ++blk) {
    const int voff = lane_off + blk * L::kRowShiftPerBlock * sb;
    const unsigned dst = lds0 + blk * L::kPitch;
    // as Dma::copy (M0 = LDS destination, rows past `bytes` arrive as zeros), plus nt
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds"
                 :
                 : "s"(dst), "v"(voff), "s"(rsrc)
                 : "memory", "m0");
  }
}

template <int D, int GM, int CPT>
__global__ __launch_bounds__(kDecThreads) void decode_scores(DecodeArgs a) {
  constexpr int KS = D / 16;   // MFMA k-steps per key block
  using L = KLayout<D>;
  using DmaK = Dma<L, 1>;      // lane offsets of a one-wave copy of a whole chunk
  const AttnGeom& g = a.g;
  const DecUnit u = dec_unit(a);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 31, hl = lane >> 5;
  const int G = g.Hq / g.Hkv;
  constexpr int BC = 64 * CPT;
  const int64_t row_len = (int64_t)a.nKT * BC;   // scores row stride (a multiple of 64 keys)

  bf16x8 qf[1][KS];
  {
    const __bf16* qp = (const __bf16*)g.q + u.b * g.qs[0] + (u.hk * G + min(col, G - 1)) * g.qs[2];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bf16x8 x = *(const bf16x8*)(qp + 16 * ks + 8 * hl);
      if (col >= G) x = bf16x8{};
      qf[0][ks] = x;
    }
  }
  const __bf16* kslab = (const __bf16*)g.k + u.b * g.ks[0] + u.hk * g.ks[2];
  const int kstride_b = (int)(g.ks[1] * 2);
  float* sc = a.scores + ((int64_t)u.b * g.Hkv + u.hk) * GM * row_len;
  __shared__ __attribute__((aligned(1024))) char kbuf[kDecWaves][2][L::kBytes];
  // A chunk's scores go through LDS so that the whole wave stores them with full 16-byte lanes
  // (the lanes holding them are only 2*GM of 64).
  __shared__ __attribute__((aligned(16))) float sbuf[kDecWaves][GM][64];
  float (*sw)[64] = sbuf[wave];

  // Tiles past this sequence's keys are not visited.
  for (int t = u.t0 + wave; t < u.t1; t += kDecWaves) {
    if (t >= u.nvis && lane < G)
      a.tmax[((int64_t)u.b * g.Hq + u.hk * G + lane) * a.nKT + t] = -INFINITY;
  }

  const int t_end = min(u.t1, u.nvis);
  const int ntile = t_end > u.t0 + wave ? (t_end - (u.t0 + wave) + kDecWaves - 1) / kDecWaves : 0;
  constexpr int cpt = CPT;   // chunks per tile
  const int nq = ntile * cpt;
  auto chunk_key0 = [&](int q) { return (u.t0 + wave + kDecWaves * (q / cpt)) * BC + (q % cpt) * 64; };
  const auto lo = DmaK::lane_offsets(kstride_b, 0, lane);
  // Chunk q into LDS buffer q%2: rows past the sequence are outside the copy's byte range and
  // arrive as zeros (the range covers at most the chunk's 64 rows).
  auto issue = [&](int q) {
    const int key0 = chunk_key0(q);
    const int rows = min(u.len - key0, 64);
    const int bytes = rows > 0 ? (rows - 1) * kstride_b + D * 2 : 0;
    copy_k_stream<L>(kbuf[wave][q & 1], kslab + (int64_t)key0 * g.ks[1], bytes, kstride_b, lo.off);
  };
  float mx = -INFINITY;     // running max of this lane's keys in the current tile (its head)
  float tile_m = -INFINITY; // the last finished tile's max of head col, in the log2 domain
  // The global stores of chunk q: its scores from the LDS staging buffer and, when it ends a tile,
  // the tile's max.  They are issued one iteration late, just before the next copy, so that the
  // wait for that copy never waits on stores younger than it.
  auto flush = [&](int q) {
    const int key0 = chunk_key0(q);
    // GM rows of 64 keys = GM*16 lanes of 16 bytes
#pragma unroll
    for (int r = 0; r < (GM * 16 + 63) / 64; ++r) {
      const int e = 64 * r + lane;
      if (e < GM * 16) {
        const int hh = e >> 4, k4 = (e & 15) * 4;
        *(f32x4*)(sc + hh * row_len + key0 + k4) = *(const f32x4*)&sw[hh][k4];
      }
    }
    if (q % cpt == cpt - 1 && hl == 0 && col < G) {
      const int t = u.t0 + wave + kDecWaves * (q / cpt);
      a.tmax[((int64_t)u.b * g.Hq + u.hk * G + col) * a.nKT + t] = tile_m;
    }
  };
  if (nq > 0) issue(0);
  for (int q = 0; q < nq; ++q) {
    // chunk q is in LDS (the stores of chunk q-2, issued before it, are done too)
    wait_vmcnt<0>();
    if (q > 0) {
      flush(q - 1);
      __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): the staging buffer is read
      __builtin_amdgcn_wave_barrier();
    }
    // chunk q+1 into the other buffer, whose operands the MFMAs of chunk q-1 read
    if (q + 1 < nq) issue(q + 1);
    const int key0 = chunk_key0(q);
    f32x16 s[2][1];
    qk_tile<D, 1>(kbuf[wave][q & 1], qf, s, lane);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      // keys past the sequence (only in its last chunk): -inf
      if (key0 + 64 > u.len) mask_block(s[kb][0], kb, u.len - key0 - 8 * hl);
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][0][i]);
      // element r holds key 32kb + 16(r/8) + 8hl + r%8: two runs of 8 consecutive keys
      if (col < GM) {
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4)
          *(f32x4*)&sw[col][32 * kb + 16 * (i4 >> 1) + 8 * hl + 4 * (i4 & 1)] =
              f32x4{s[kb][0][4 * i4], s[kb][0][4 * i4 + 1], s[kb][0][4 * i4 + 2],
                    s[kb][0][4 * i4 + 3]};
      }
    }
    if (q % cpt == cpt - 1) {
      tile_m = half_max(mx) * g.c32;   // tile max of head col over both lane halves
      mx = -INFINITY;
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): the chunk's scores are in LDS
    __builtin_amdgcn_wave_barrier();
  }
  if (nq > 0) flush(nq - 1);
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

template <int D, int GM, int CPT>
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
  constexpr int BC = 64 * CPT;

  __shared__ float pre[kDecWaves][GM];
  __shared__ float ref_s[GM];
  __shared__ uint32_t keepbits[kMaxTilesPerSplit];
  __shared__ float stage[GM][64];
  __shared__ __attribute__((aligned(16))) typename PvChunk<D, GM>::Buf pbuf[kDecWaves];
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
  typename PvChunk<D, GM>::Buf& pw = pbuf[wave];

  // This wave's kept tiles t = t0 + wave + kDecWaves*i (kept by some head) listed in LDS, then
  // walked as 64-key chunks; the V rows and scores of chunk q+1 are loaded while chunk q is
  // reduced.  The prefetches are unconditional (clamped index), so the compiler's waits leave them
  // in flight.
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
  constexpr int cpt = CPT;
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
    float p[4 * GQ];
#pragma unroll
    for (int h = 0; h < 4 * GQ; ++h) {
      p[h] = 0.f;
      if (h < GM && ((kb >> h) & 1u) && valid)
        p[h] = __builtin_amdgcn_exp2f(sv[h < GM ? h : 0] * g.c32 - ref[h < GM ? h : 0]);
      if (h < GM) ls[h] += p[h];
    }
    PvChunk<D, GM>::write_p(pw, lane, p);
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): P is in LDS for the whole wave
    __builtin_amdgcn_wave_barrier();
    PvChunk<D, GM>::accumulate(pw, vv, sub, acc);
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

// ---- whole-sequence decode: one workgroup per (batch, KV head) -------------------------------------
// When one workgroup owns every key of its (batch, KV head), the decisions need no exchange between
// workgroups and the scores of the G heads can stay in LDS from the K pass to the V pass:
//   1 scores: the waves stride over 64-key chunks (K rows straight into MFMA operands, the next
//     chunk loaded while the current one is multiplied) and write S and each chunk's max per head
//     into LDS;
//   2 decisions: one wave per head walks the tiles in order -- a wave-wide prefix-max scan 64 tiles
//     at a time for lambda <= 1 (a skipped tile cannot raise the running max), the running max for
//     lambda > 1 -- writing the keep bits, tile states, counters and the head's exponent reference
//     r (the max of its kept tile maxima, so that P = 2^(t - r) <= 1 needs no rescaling);
//   3 P.V: the waves stride over the chunks of tiles some head keeps (the V rows of the next chunk
//     loaded while the current one is reduced), with P from the LDS scores; the waves' partial sums
//     are then added in LDS (reusing the score buffer) and O and the natural-log LSE written.
// K and V are each read once; nothing goes through device memory between the passes.
constexpr int kFusedWaves = 8;
constexpr int kFusedThreads = 64 * kFusedWaves;

template <int D, int GM>
__global__ __launch_bounds__(kFusedThreads) void decode_fused(DecodeArgs a) {
  constexpr int KS = D / 16;
  constexpr int LPK = D / 8;          // lanes per V row (16 bytes each)
  constexpr int KPI = 64 / LPK;       // V rows per wave-wide load
  constexpr int kIt = 64 / KPI;
  constexpr int GQ = (GM + 3) / 4;    // 16-byte groups of P per key
  constexpr int kMaxChunks = kFusedScoreBytes / (4 * 64);   // GM * chunks <= this (host check)
  const AttnGeom& g = a.g;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, hl = lane >> 5;
  const int G = g.Hq / g.Hkv;
  const int BC = a.block_k, cpt = BC / 64;
  const int hk = (int)(blockIdx.x % g.Hkv), b = (int)(blockIdx.x / g.Hkv);
  int len = g.Sk;
  if (a.seqlens_k != nullptr) len = min(max(a.seqlens_k[b], 0), g.Sk);
  const int nKT = a.nKT;
  const int nvis = (len + BC - 1) / BC;   // tiles holding a key of the sequence
  const int nch = nvis * cpt;             // their 64-key chunks
  const int row_len = nKT * BC;           // LDS score row stride (keys)
  const int cstride = nKT * cpt;          // chunk-maxima row stride

  __shared__ __attribute__((aligned(16))) float sc[kFusedScoreBytes / 4];   // [GM][row_len]
  __shared__ float cmax[kMaxChunks];        // [G][cstride] chunk maxima, log2 domain
  __shared__ uint32_t kbits[kMaxChunks];    // per tile: bit h set when head h keeps it
  __shared__ uint16_t klist[kMaxChunks];    // tiles kept by some head, ascending
  __shared__ int nkept_s;
  __shared__ float ref_s[GM];
  __shared__ __attribute__((aligned(16))) typename PvChunk<D, GM>::Buf pbuf[kFusedWaves];
  __shared__ float lred[kFusedWaves][GM];

  for (int t = tid; t < nKT; t += kFusedThreads) kbits[t] = 0u;

  // ---- 1: scores into LDS ----
  bf16x8 qf[KS];
  {
    const __bf16* qp = (const __bf16*)g.q + b * g.qs[0] + (hk * G + min(col, G - 1)) * g.qs[2];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bf16x8 x = *(const bf16x8*)(qp + 16 * ks + 8 * hl);
      if (col >= G) x = bf16x8{};
      qf[ks] = x;
    }
  }
  {
    const __bf16* kslab = (const __bf16*)g.k + b * g.ks[0] + hk * g.ks[2];
    const auto krs = slab_rsrc(kslab, g.ks[1], len, D);
    const int kstride_b = (int)(g.ks[1] * 2);
    // this wave's chunks c = wave + kFusedWaves * i; the prefetch index is clamped (unconditional
    // loads keep the compiler's waits from draining them)
    const int nq = nch > wave ? (nch - wave + kFusedWaves - 1) / kFusedWaves : 0;
    auto key_of = [&](int i) { return (wave + kFusedWaves * i) * 64; };
    auto load_chunk = [&](bf16x8 (&kv)[2][KS], int i) {
      const int key0 = key_of(i);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int off = (key0 + 32 * kb + col) * kstride_b + 16 * hl;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          kv[kb][ks] = __builtin_bit_cast(bf16x8, load16(krs, off + 32 * ks));
      }
    };
    auto consume = [&](const bf16x8 (&kv)[2][KS], int i) {
      const int key0 = key_of(i);
      f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) s[kb] = mfma32(kv[kb][ks], qf[ks], s[kb]);
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        mask_rows(s[kb], kb, len - key0 - 4 * hl);   // keys past the sequence: -inf
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
        if (col < G) {
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4)
            *(f32x4*)&sc[col * row_len + key0 + 32 * kb + 8 * i4 + 4 * hl] =
                f32x4{s[kb][4 * i4], s[kb][4 * i4 + 1], s[kb][4 * i4 + 2], s[kb][4 * i4 + 3]};
        }
      }
      const float m = half_max(mx);
      if (hl == 0 && col < G) cmax[col * cstride + key0 / 64] = m * g.c32;
    };
    bf16x8 kva[2][KS], kvb[2][KS];
    if (nq > 0) {
      load_chunk(kva, 0);
      for (int i = 0; i < nq; i += 2) {
        load_chunk(kvb, min(i + 1, nq - 1));
        consume(kva, i);
        load_chunk(kva, min(i + 2, nq - 1));
        if (i + 1 < nq) consume(kvb, i + 1);
      }
    }
  }
  __syncthreads();

  // ---- 2: decisions, one wave per head ----
  for (int h = wave; h < G; h += kFusedWaves) {
    const int64_t unit = (int64_t)b * g.Hq + hk * G + h;
    auto tile_max = [&](int t) {   // t < nvis
      float m = cmax[h * cstride + t * cpt];
      if (cpt == 2) m = fmaxf(m, cmax[h * cstride + t * cpt + 1]);
      return m;
    };
    float ref = -INFINITY;
    unsigned vis_n = 0u, skip_n = 0u;
    if (a.L32 <= 0.f) {
      float carry = -INFINITY;
      for (int j0 = 0; j0 < nKT; j0 += 64) {
        const int j = j0 + lane;
        const bool in = j < nKT, vis = j < nvis;
        const float M = vis ? tile_max(j) : -INFINITY;
        float incl = M;   // inclusive prefix max over the lanes
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
          const float up = __shfl_up(incl, d, 64);
          if (lane >= d) incl = fmaxf(incl, up);
        }
        float excl = __shfl_up(incl, 1, 64);
        excl = lane == 0 ? carry : fmaxf(carry, excl);
        const bool keep = vis && !(M < excl + a.L32);
        if (keep) atomicOr(&kbits[j], 1u << h);
        ref = fmaxf(ref, keep ? M : -INFINITY);
        vis_n += __popcll(__ballot(vis));
        skip_n += __popcll(__ballot(vis && !keep));
        if (in && a.tile_state != nullptr) a.tile_state[unit * nKT + j] = vis ? (keep ? 0 : 1) : 2;
        if (in && a.dbg_tmax != nullptr) a.dbg_tmax[unit * nKT + j] = M;
        carry = fmaxf(carry, __shfl(incl, 63, 64));
      }
      for (int d = 1; d < 64; d <<= 1) ref = fmaxf(ref, __shfl_xor(ref, d, 64));
    } else {
      // the running max of the kept tiles, in order (every lane walks the same sequence)
      float m = -INFINITY;
      for (int j0 = 0; j0 < nKT; j0 += 64) {
        const int jl = j0 + lane;
        const float Ml = jl < nvis ? tile_max(jl) : -INFINITY;
        if (jl < nKT && a.dbg_tmax != nullptr) a.dbg_tmax[unit * nKT + jl] = Ml;
        const int n = min(64, nKT - j0);
        for (int jj = 0; jj < n; ++jj) {
          const int jt = j0 + jj;
          const float M = __shfl(Ml, jj, 64);
          const bool vis = jt < nvis;
          const bool keep = vis && !(M < m + a.L32);
          if (keep) {
            m = fmaxf(m, M);
            ref = fmaxf(ref, M);
          }
          vis_n += vis ? 1u : 0u;
          skip_n += (vis && !keep) ? 1u : 0u;
          if (lane == 0) {
            if (keep) atomicOr(&kbits[jt], 1u << h);
            if (a.tile_state != nullptr) a.tile_state[unit * nKT + jt] = vis ? (keep ? 0 : 1) : 2;
          }
        }
      }
    }
    if (lane == 0) {
      ref_s[h] = ref;
      if (a.counters != nullptr) {
        atomicAdd(&a.counters[2 * unit], vis_n);
        atomicAdd(&a.counters[2 * unit + 1], skip_n);
      }
    }
  }
  __syncthreads();
  if (wave == 0) {   // the tiles kept by some head, in order
    int n = 0;
    for (int t0 = 0; t0 < nvis; t0 += 64) {
      const int t = t0 + lane;
      const bool kept = t < nvis && kbits[t] != 0u;
      const uint64_t m = __ballot(kept);
      if (kept) klist[n + __popcll(m & ((1ull << lane) - 1ull))] = (uint16_t)t;
      n += __popcll(m);
    }
    if (lane == 0) nkept_s = n;
  }
  __syncthreads();

  // ---- 3: P.V over the kept chunks ----
  const int sub = lane / LPK, c = lane % LPK;
  float ref[GM];
#pragma unroll
  for (int h = 0; h < GM; ++h) ref[h] = h < G ? ref_s[h] : -INFINITY;
  float acc[GM][8];
  float ls[GM];
#pragma unroll
  for (int h = 0; h < GM; ++h) {
    ls[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
  }
  {
    const __bf16* vslab = (const __bf16*)g.v + b * g.vs[0] + hk * g.vs[2];
    const auto vrs = slab_rsrc(vslab, g.vs[1], len, D);
    const int vstride_b = (int)(g.vs[1] * 2);
    typename PvChunk<D, GM>::Buf& pw = pbuf[wave];
    const int nq_all = nkept_s * cpt;
    const int nq = nq_all > wave ? (nq_all - wave + kFusedWaves - 1) / kFusedWaves : 0;
    auto chunk_of = [&](int i) { return wave + kFusedWaves * i; };   // index into the kept chunks
    auto key_of = [&](int i) {
      const int q = chunk_of(i);
      return (int)klist[q / cpt] * BC + (q % cpt) * 64;
    };
    auto load_chunk = [&](u32x4 (&vv)[kIt], int i) {
      const int key0 = key_of(i);
#pragma unroll
      for (int it = 0; it < kIt; ++it)
        vv[it] = load16(vrs, (key0 + sub + it * KPI) * vstride_b + c * 16);
    };
    auto reduce_chunk = [&](const u32x4 (&vv)[kIt], int i) {
      const int q = chunk_of(i);
      const int key0 = key_of(i);
      const uint32_t kb = kbits[klist[q / cpt]];
      // P of the 64 keys, one key per lane, into this wave's LDS slot; l from the same values
      const bool valid = key0 + lane < len;
      float p[4 * GQ];
#pragma unroll
      for (int h = 0; h < 4 * GQ; ++h) {
        p[h] = 0.f;
        if (h < G && ((kb >> h) & 1u) && valid)
          p[h] = __builtin_amdgcn_exp2f(sc[(h < GM ? h : 0) * row_len + key0 + lane] * g.c32 -
                                        ref[h < GM ? h : 0]);
        if (h < GM) ls[h < GM ? h : 0] += p[h];
      }
      PvChunk<D, GM>::write_p(pw, lane, p);
      __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): P is in LDS for the whole wave
      __builtin_amdgcn_wave_barrier();
      PvChunk<D, GM>::accumulate(pw, vv, sub, acc);
      __builtin_amdgcn_wave_barrier();   // every lane has read P before the next chunk rewrites it
    };
    if (nq > 0) {
      u32x4 vva[kIt], vvb[kIt];
      load_chunk(vva, 0);
      for (int i = 0; i < nq; i += 2) {
        load_chunk(vvb, min(i + 1, nq - 1));
        reduce_chunk(vva, i);
        load_chunk(vva, min(i + 2, nq - 1));
        if (i + 1 < nq) reduce_chunk(vvb, i + 1);
      }
    }
  }

  // sum over the key slots of each wave, then over the waves (the score buffer is free now)
  __syncthreads();
  float* red = sc;   // [kFusedWaves][GM][D]
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
      for (int e = 0; e < 8; ++e) red[(wave * GM + h) * D + 8 * c + e] = acc[h][e];
    }
    if (lane == 0) lred[wave][h] = l;
  }
  __syncthreads();
  for (int i = tid; i < G * D; i += kFusedThreads) {
    const int h = i / D, d = i % D;
    float o = 0.f, l = 0.f;
#pragma unroll
    for (int w = 0; w < kFusedWaves; ++w) {
      o += red[(w * GM + h) * D + d];
      l += lred[w][h];
    }
    const int hq = hk * G + h;
    __bf16* op = (__bf16*)g.o + b * g.os[0] + hq * g.os[2];
    op[d] = (__bf16)(l > 0.f ? o / l : 0.f);
    if (d == 0 && a.lse != nullptr)
      a.lse[(int64_t)b * g.Hq + hq] = l > 0.f ? (ref_s[h] + __log2f(l)) * 0.69314718055994531f
                                              : -INFINITY;
  }
}

template <int D, int GM>
hipError_t launch_fused(const DecodeArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((decode_fused<D, GM>), dim3(a.g.B * a.g.Hkv), dim3(kFusedThreads), 0, stream,
                     a);
  return hipGetLastError();
}

template <int D, int GM>
hipError_t launch_dg(const DecodeArgs& a, hipStream_t stream) {
  if constexpr (GM <= kFusedMaxGM) {
    if (a.fused) return launch_fused<D, GM>(a, stream);
  }
  const int units = a.g.B * a.g.Hkv * a.nsplit;
  if (a.block_k == 128)
    hipLaunchKernelGGL((decode_scores<D, GM, 2>), dim3(units), dim3(kDecThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((decode_scores<D, GM, 1>), dim3(units), dim3(kDecThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.block_k == 128)
    hipLaunchKernelGGL((decode_attend<D, GM, 2>), dim3(units), dim3(kDecThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((decode_attend<D, GM, 1>), dim3(units), dim3(kDecThreads), 0, stream, a);
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
