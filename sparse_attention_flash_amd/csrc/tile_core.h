// tile_core.h -- device building blocks shared by the gfx950 attention kernels.
//
// One wavefront owns 64 query rows and walks the keys in tiles of 64.  Both contractions run on
// v_mfma_f32_32x32x16_bf16 in the "keys on MFMA rows" orientation:
//
//   S^T[key][query] = K . Q^T      A = K rows from LDS, B = Q^T held in registers for the kernel
//   O^T[d][query]  += V^T . P^T    A = V^T from LDS via transpose reads, B = P^T straight from
//                                  the S^T accumulator registers (no shuffles)
//
// With this orientation a lane holds ONE query and 16 keys of each 32x32 block, so a row max is
// an in-lane max plus one cross-half exchange (v_permlane32_swap), and the softmax weights leave
// the QK accumulator already in the B-operand layout of the PV product.
//
// MFMA 32x32x16 bf16 register layout (verified on gfx950 with an in-bounds probe):
//   A[i][k]: lane i + 32*(k/8), element k%8      B[k][j]: lane j + 32*(k/8), element k%8
//   C[i][j]: lane j + 32*h holds rows i = (r/4)*8 + 4*h + r%4 in element r (r = 0..15)
// Transpose read ds_read_b64_tr_b16 (verified likewise): in each group of 16 lanes, source lane j
// points at 4 consecutive 16-bit elements; output lane i receives element i%4 of source lanes
// i/4, i/4+4, i/4+8, i/4+12.  Pointing source lane j at V[kb + j/4][db + 4*(j%4)] hands output
// lane i the column V[kb..kb+3][db + i], i.e. a 4-key x 16-d transpose per 16 lanes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr int kKeysPerTile = 64;    // key tile
constexpr int kRowsPerWave = 64;    // query rows owned by one wavefront
constexpr float kLog2e = 1.4426950408889634f;

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// ------------------------------------------------------------------------------------------------
// LDS tile of 64 rows x D bf16, row pitch D*2 bytes, 16-byte chunks permuted per row.  The
// permutation makes (a) 16 consecutive rows at one chunk index (the K reads of QK^T) hit 16
// different chunks, and (b) the 4 aligned rows x 2 neighbouring chunks read by one transpose-read
// group land on 8 different chunks.
// ------------------------------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ int chunk_swizzle(int row, int chunk) {
  int f = ((row & 3) << 1) | ((row >> 2) & 1);
  if constexpr (D == 128) f |= ((row >> 3) & 1) << 3;
  return chunk ^ f;
}

template <int D>
__device__ __forceinline__ int tile_offset(int row, int col) {   // byte offset of element (row, col)
  return row * (D * 2) + chunk_swizzle<D>(row, col >> 3) * 16 + (col & 7) * 2;
}

// Buffer resource over one (batch, head) slab of a [rows, D] bf16 tensor with the given row stride
// (elements).  num_records covers exactly the valid rows, so buffer loads beyond the last row
// return zeros (padded keys then contribute 0 * 0, padded queries produce unused rows).  Offsets
// are 32-bit: the host rejects slabs of 2 GiB or more.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t slab_rsrc(const __bf16* base, int64_t row_stride,
                                                             int rows, int D) {
  const int64_t bytes = rows > 0 ? ((int64_t)(rows - 1) * row_stride + D) * 2 : 0;
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ u32x4 load16(__amdgpu_buffer_rsrc_t r, int byte_offset) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_offset, 0, 0));
}

// Copy key rows [k0, k0 + 64) of a slab into an LDS tile (rows past the slab arrive as zeros).
template <int D, int NT>
__device__ __forceinline__ void stage_tile(char* lds, __amdgpu_buffer_rsrc_t src,
                                           int64_t row_stride, int k0, int tid) {
  constexpr int kChunksPerRow = D / 8;
  constexpr int kIters = kKeysPerTile * kChunksPerRow / NT;
  constexpr int kRowStep = NT / kChunksPerRow;
  static_assert(kKeysPerTile * kChunksPerRow % NT == 0, "tile must split evenly over threads");
  const int row = tid / kChunksPerRow, ch = tid % kChunksPerRow;
  const int stride_b = (int)(row_stride * 2);
  const int off0 = (k0 + row) * stride_b + ch * 16;
  u32x4 val[kIters];
#pragma unroll
  for (int i = 0; i < kIters; ++i) val[i] = load16(src, off0 + i * kRowStep * stride_b);
#pragma unroll
  for (int i = 0; i < kIters; ++i) {
    const int r = row + i * kRowStep;
    *reinterpret_cast<u32x4*>(lds + r * (D * 2) + chunk_swizzle<D>(r, ch) * 16) = val[i];
  }
}

// Q^T fragments (B operand of S^T = K.Q^T) for the wave's 64 rows starting at slab row row0:
// qf[qb][ks] holds Q[row0 + 32*qb + lane%32][16*ks + 8*(lane/32) .. +7]; rows past the slab are 0.
template <int D>
__device__ __forceinline__ void load_q_frags(bf16x8 (&qf)[2][D / 16], __amdgpu_buffer_rsrc_t q,
                                             int64_t row_stride, int row0, int lane) {
  const int h = lane >> 5, r32 = lane & 31;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int off = (row0 + qb * 32 + r32) * (int)(row_stride * 2) + h * 16;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) qf[qb][ks] = __builtin_bit_cast(bf16x8, load16(q, off + ks * 32));
  }
}

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Register classes of the two contractions are fixed by hand (inline asm): the Q^T operand and the
// O accumulator live in AGPRs, the score accumulators in VGPRs where the softmax arithmetic reads
// them.  The compiler's hazard recognizer does not see inside inline asm, so the wait states it
// would insert are written out: qk_result_guard() between the last QK MFMA and the first VALU read
// of the scores, a leading s_nop before MFMAs whose operands VALU code just wrote.

// Move the Q^T fragments into AGPRs (they are only ever MFMA operands).
template <int D>
__device__ __forceinline__ void park_q_in_agprs(bf16x8 (&qf)[2][D / 16]) {
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) asm volatile("" : "+a"(qf[qb][ks]));
}

// The MFMA asm statements are volatile with a memory clobber: LDS reads stay where the code puts
// them relative to the MFMAs, which is how the operand prefetches below are scheduled.
__device__ __forceinline__ void mfma32_qk_first(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "a"(b) : "memory");
}
__device__ __forceinline__ void mfma32_qk(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "a"(b) : "memory");
}
// Wait states between the QK MFMAs writing the scores and VALU code reading them (a 32x32x16 MFMA
// has 8 passes; 20 wait states cover it with margin).  Tied to the score registers so that it sits
// exactly between the last MFMA and the first read.
__device__ __forceinline__ void qk_result_guard(f32x16 (&s)[2][2]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3"
               : "+v"(s[0][0]), "+v"(s[0][1]), "+v"(s[1][0]), "+v"(s[1][1]));
}

// S^T for one 64-key tile: s[kb][qb] is the 32x32 block keys 32*kb.., queries 32*qb..
// Element r of lane l: key 32*kb + (r/4)*8 + 4*(l/32) + r%4, query 32*qb + l%32.
// S^T for one 64-key tile: s[kb][qb] is the 32x32 block keys 32*kb.., queries 32*qb..
// Element r of lane l: key 32*kb + (r/4)*8 + 4*(l/32) + r%4, query 32*qb + l%32.
// K fragments are read from LDS kPrefetch steps ahead of the MFMAs that use them.
template <int D>
__device__ __forceinline__ void qk_tile(const char* ldsK, const bf16x8 (&qf)[2][D / 16],
                                        f32x16 (&s)[2][2], int lane) {
  constexpr int KS = D / 16;        // 16-wide k steps per 32-key block
  constexpr int NF = 2 * KS;        // fragments per tile
  constexpr int kPrefetch = 4;
  const int h = lane >> 5, r32 = lane & 31;
  auto frag = [&](int i) {
    const int kb = i / KS, ks = i % KS, row = kb * 32 + r32;
    return *reinterpret_cast<const bf16x8*>(ldsK + row * (D * 2) +
                                            chunk_swizzle<D>(row, 2 * ks + h) * 16);
  };
  bf16x8 f[NF];
#pragma unroll
  for (int i = 0; i < kPrefetch; ++i) f[i] = frag(i);
#pragma unroll
  for (int i = 0; i < NF; ++i) {
    if (i + kPrefetch < NF) f[i + kPrefetch] = frag(i + kPrefetch);
    const int kb = i / KS, ks = i % KS;
    if (ks == 0) {
      mfma32_qk_first(s[kb][0], f[i], qf[0][ks]);
      mfma32_qk_first(s[kb][1], f[i], qf[1][ks]);
    } else {
      mfma32_qk(s[kb][0], f[i], qf[0][ks]);
      mfma32_qk(s[kb][1], f[i], qf[1][ks]);
    }
  }
  qk_result_guard(s);
}

// Set element r of s to -inf when off(r) >= lim, off(r) = kb*32 + (r/4)*8 + r%4 being the key's
// offset inside the tile minus 4*(lane/32).  Pure VGPR arithmetic (shift mask + bitfield insert):
// a compare per element would park 64 lane masks in SGPRs.
__device__ __forceinline__ void mask_block(f32x16& s, int kb, int lim) {
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int off = kb * 32 + (r >> 2) * 8 + (r & 3);
    const int m = (lim - 1 - off) >> 31;   // all ones when off >= lim
    float out;
    asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(out) : "v"(m), "v"(-INFINITY), "v"(s[r]));
    s[r] = out;
  }
}

// Key index (0..63 inside the tile) held in element r of this lane's s[kb][*] block.
__device__ __forceinline__ int tile_key(int kb, int r, int lane) {
  return kb * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
}

// Value of x held by the lane in the other half of the wavefront (lane ^ 32).
__device__ __forceinline__ float other_half(float x, int lane) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                   false);
  return __uint_as_float(lane < 32 ? sw[1] : sw[0]);
}

__device__ __forceinline__ float half_max(float x) {   // max over lanes l and l^32
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                   false);
  return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}

__device__ __forceinline__ float half_sum(float x) {   // sum over lanes l and l^32
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                   false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

// P^T operands: the 16-key chunk c (keys 16c..16c+15 of the 32-key block kb) of query block qb,
// taken as elements 8c..8c+7 of s[kb][qb].  Element e stands for key 16c + 4*(l/32) + e (e < 4)
// or 16c + 8 + 4*(l/32) + e - 4 (e >= 4); pv_tile reads V in the same key order.
__device__ __forceinline__ bf16x8 p_operand(const f32x16& p, int c) {
  bf16x8 out;
#pragma unroll
  for (int e = 0; e < 8; ++e) out[e] = (__bf16)p[8 * c + e];
  return out;
}

// MFMA accumulating in AGPRs.  The P.V accumulator O (128 registers per lane at head_dim 128) is
// kept in the accumulation registers so that the score tiles S(j), S(j+1) and P(j) fit in the
// VGPRs beside it; the builtin would put every accumulator in one register class.  The leading
// s_nop covers the VALU-write -> MFMA-read wait states (the operands are produced by VALU); reads
// of the accumulator by VALU code must be preceded by agpr_read_guard(o).
__device__ __forceinline__ void mfma32_agpr(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
               : "+a"(acc) : "v"(a), "v"(b) : "memory");
}

// Wait states between an MFMA writing the accumulator O and VALU code reading or rewriting it.  The
// asm takes every accumulator as an in/out operand, so the compiler can place it neither before the
// last MFMA that writes O nor after the first instruction that reads it.
template <int D>
__device__ __forceinline__ void agpr_read_guard(f32x16 (&o)[D / 32][2]) {
  if constexpr (D == 128) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
                 : "+a"(o[0][0]), "+a"(o[0][1]), "+a"(o[1][0]), "+a"(o[1][1]), "+a"(o[2][0]),
                   "+a"(o[2][1]), "+a"(o[3][0]), "+a"(o[3][1]));
  } else {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
                 : "+a"(o[0][0]), "+a"(o[0][1]), "+a"(o[1][0]), "+a"(o[1][1]));
  }
}

// Wait states between VALU code rewriting O and the next MFMA reading it as the accumulator input.
template <int D>
__device__ __forceinline__ void agpr_write_guard(f32x16 (&o)[D / 32][2]) {
  if constexpr (D == 128) {
    asm volatile("s_nop 4"
                 : "+a"(o[0][0]), "+a"(o[0][1]), "+a"(o[1][0]), "+a"(o[1][1]), "+a"(o[2][0]),
                   "+a"(o[2][1]), "+a"(o[3][0]), "+a"(o[3][1]));
  } else {
    asm volatile("s_nop 4" : "+a"(o[0][0]), "+a"(o[0][1]), "+a"(o[1][0]), "+a"(o[1][1]));
  }
}

// O^T[d][q] += V^T . P^T over one 64-key tile; o[db][qb] is the 32x32 block d 32*db.., queries
// 32*qb..; pb[kb][c][qb] from p_operand.
template <int D>
__device__ __forceinline__ void pv_tile(const char* ldsV, const bf16x8 (&pb)[2][2][2],
                                        f32x16 (&o)[D / 32][2], int lane) {
  const int g = lane >> 4, j = lane & 15, h = lane >> 5;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int row = kb * 32 + c * 16 + 4 * h + (j >> 2);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const int col = db * 32 + 16 * (g & 1) + 4 * (j & 3);
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(ldsV + tile_offset<D>(row, col)));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(ldsV + tile_offset<D>(row + 8, col)));
        const bf16x8 a = __builtin_bit_cast(
            bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        mfma32_agpr(o[db][0], a, pb[kb][c][0]);
        mfma32_agpr(o[db][1], a, pb[kb][c][1]);
      }
    }
  }
}

// Store the wave's normalised output rows: o[db][qb] element r is d = 32*db + (r/4)*8 + 4*h + r%4.
template <int D>
__device__ __forceinline__ void store_o(__bf16* out, int64_t row_stride, int rows_valid,
                                        const f32x16 (&o)[D / 32][2], const float (&inv)[2],
                                        int lane) {
  const int h = lane >> 5, r32 = lane & 31;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int row = qb * 32 + r32;
    if (row >= rows_valid) continue;
    __bf16* dst = out + (int64_t)row * row_stride;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (__bf16)(o[db][qb][4 * g4 + e] * inv[qb]);
        *reinterpret_cast<bf16x4*>(dst + db * 32 + g4 * 8 + h * 4) = v;
      }
    }
  }
}

// Bijective remap of workgroup ids so that consecutive logical work items run on the same XCD
// (workgroups are dispatched round-robin over the 8 XCDs, each with its own L2).
__device__ __forceinline__ int xcd_remap(int wg, int n) {
  const int x = wg & 7, i = wg >> 3, q = n >> 3, r = n & 7;
  return x * q + (x < r ? x : r) + i;
}

}  // namespace sa
