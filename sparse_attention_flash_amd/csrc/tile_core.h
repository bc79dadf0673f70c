// tile_core.h -- device building blocks shared by the gfx950 attention kernels.
//
// One wavefront owns QB blocks of 32 query rows (QB = 1 or 2) and walks the keys in tiles of 64.
// Both contractions run on v_mfma_f32_32x32x16_bf16 in the "keys on MFMA rows" orientation:
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
//
// Key order.  MFMA row i of a 32-key block is fed key kappa(i) = i with bits 2 and 3 exchanged,
// so element r of lane j + 32*h holds key 16*(r/8) + 8*h + r%8 of the block: every lane holds
// runs of 8 consecutive keys (two per block), which keeps groups of 4 and of 8 consecutive keys
// inside one lane.  For P.V the 16-key chunk c of a block is then simply key 16*c + k at the
// B-operand index k = 8*h + e of element 8*c + e.
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
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr int kKeysPerTile = 64;    // key tile
constexpr float kLog2e = 1.4426950408889634f;

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// ------------------------------------------------------------------------------------------------
// LDS layouts of a 64-key x D bf16 tile.  A tile is a run of blocks; a direct-to-LDS copy writes
// one 1 KiB block per wave-wide instruction (lane l -> bytes 16l..16l+15 of the block) and each
// lane may fetch any 16-byte chunk, so placement inside and between blocks is free.  The copies
// keep 16 consecutive lanes on 16 consecutive chunks of one key row (coalesced 256-byte rows).
//
// head_dim 128: block b (b < 16) holds rows b, b+16, b+32, b+48 row-major (chunk q of row
// b + 16*rho at 16-byte slot 16*rho + q); blocks sit kPitch bytes apart.  A lane's LDS reads
// are then base(lane) + a compile-time offset (immediate offsets, no per-step address registers),
// and both read patterns are conflict-free through the block pitch alone:
//   K (ds_read_b128, 16 rows at one chunk per quarter wave): rows 0..15 are in blocks 0..15 and
//     a pitch of 65 slots puts them on 16 different 16-byte bank groups;
//   V (ds_read_b64_tr_b16, 4 rows x 4 chunks per half wave): 4 consecutive rows are in 4
//     consecutive blocks and a pitch of 68 slots moves each by 4 bank groups.
//
// head_dim 64 (one layout for K and V): 8 blocks of 8 rows x 8 chunks, row-major, chunk q of row r
// stored at q ^ f(r) (f a bijection on 8 rows) so 8 consecutive rows at one chunk hit 8 chunks.
// ------------------------------------------------------------------------------------------------
// The key fed to MFMA row i of a 32-key block: bits 2 and 3 of i exchanged (see "Key order").
__device__ __forceinline__ int key_of_row(int i) {
  return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1);
}

template <int D, bool kV>
struct TileLayout;

template <bool kV>
struct TileLayout<128, kV> {
  static constexpr int kPitch = kV ? 1088 : 1040;   // bytes per block
  static constexpr int kBlocks = 16;
  static constexpr int kBytes = kBlocks * kPitch;
  // A copy of block b: lane l fetches row b + 16*(l/16), chunk l%16 (dma_lane plus the row shift
  // of b).
  static constexpr int kRowShiftPerBlock = 1;
  static __device__ __forceinline__ int dma_lane(int stride_b, int lane) {
    return (lane >> 4) * 16 * stride_b + (lane & 15) * 16;
  }
  // byte offset of chunk q of row r
  static __device__ __forceinline__ int chunk_off(int r, int q) {
    return (r & 15) * kPitch + ((r >> 4) * 16 + q) * 16;
  }
  // K rows as MFMA A operands: row 32kb + kappa(lane%32), chunk 2ks + lane/32 (rows 0..15 of a
  // quarter wave are a permutation of 16 consecutive rows: still one per block)
  static __device__ __forceinline__ int k_off(int lane, int kb, int ks) {
    return chunk_off(key_of_row(lane & 31) + 32 * kb, 2 * ks + (lane >> 5));
  }
  // transpose-read source of lane (g = lane/16, j = lane%16): row 32kb + 16c + 8(lane/32) + j/4
  // + 4hi, columns 32db + 16(g%2) + 4(j%4) .. +3
  static __device__ __forceinline__ int v_off(int lane, int kb, int c, int hi, int db) {
    const int g = lane >> 4, j = lane & 15, h = lane >> 5;
    const int r = kb * 32 + c * 16 + 8 * h + (j >> 2) + 4 * hi;
    return chunk_off(r, db * 4 + 2 * (g & 1) + ((j & 3) >> 1)) + (j & 1) * 8;
  }
};

template <bool kV>
struct TileLayout<64, kV> {
  static constexpr int kPitch = 1024;
  static constexpr int kBlocks = 8;
  static constexpr int kBytes = kBlocks * kPitch;
  static constexpr int kRowShiftPerBlock = 8;   // block b holds rows 8b..8b+7
  static __device__ __forceinline__ int swz(int row, int chunk) {
    return chunk ^ (((row & 3) << 1) | ((row >> 2) & 1));
  }
  static __device__ __forceinline__ int elem(int row, int col) {   // byte offset of (row, col)
    return row * 128 + swz(row, col >> 3) * 16 + (col & 7) * 2;
  }
  static __device__ __forceinline__ int dma_lane(int stride_b, int lane) {
    return (lane >> 3) * stride_b + swz(lane >> 3, lane & 7) * 16;
  }
  static __device__ __forceinline__ int k_off(int lane, int kb, int ks) {
    const int row = kb * 32 + key_of_row(lane & 31);
    return row * 128 + swz(row, 2 * ks + (lane >> 5)) * 16;
  }
  static __device__ __forceinline__ int v_off(int lane, int kb, int c, int hi, int db) {
    const int g = lane >> 4, j = lane & 15, h = lane >> 5;
    return elem(kb * 32 + c * 16 + 8 * h + (j >> 2) + 4 * hi, db * 32 + 16 * (g & 1) + 4 * (j & 3));
  }
};

template <int D>
using KLayout = TileLayout<D, false>;
template <int D>
using VLayout = TileLayout<D, true>;

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

// Q^T fragments (B operand of S^T = K.Q^T) for the wave's 32*QB rows starting at slab row row0:
// qf[qb][ks] holds Q[row0 + 32*qb + lane%32][16*ks + 8*(lane/32) .. +7]; rows past the slab are 0.
template <int D, int QB>
__device__ __forceinline__ void load_q_frags(bf16x8 (&qf)[QB][D / 16], __amdgpu_buffer_rsrc_t q,
                                             int64_t row_stride, int row0, int lane) {
  const int h = lane >> 5, r32 = lane & 31;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int off = (row0 + qb * 32 + r32) * (int)(row_stride * 2) + h * 16;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) qf[qb][ks] = __builtin_bit_cast(bf16x8, load16(q, off + ks * 32));
  }
}

// Both contractions use the compiler's MFMA builtin with accumulators in VGPRs (built with
// -amdgpu-mfma-vgpr-form): with one 32-row query block per wave the Q^T operand (32), O (64 at
// head_dim 128), two score tiles (64) and the operand prefetches fit in 256 VGPRs, so the softmax
// reads the scores and rescales O with plain VALU code and the compiler inserts every MFMA wait
// state itself.
__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// S^T for one 64-key tile: s[kb][qb] is the 32x32 block keys 32*kb.., queries 32*qb..
// Element r of lane l: key 32*kb + (r/8)*16 + 8*(l/32) + r%8, query 32*qb + l%32.
// K fragments are read from LDS kPrefetch steps ahead of the MFMAs that use them.
template <int D, int QB>
__device__ __forceinline__ void qk_tile(const char* ldsK, const bf16x8 (&qf)[QB][D / 16],
                                        f32x16 (&s)[2][QB], int lane) {
  constexpr int KS = D / 16;        // 16-wide k steps per 32-key block
  constexpr int NF = 2 * KS;        // fragments per tile
  constexpr int kPrefetch = 4;
  auto frag = [&](int i) {
    return *reinterpret_cast<const bf16x8*>(ldsK + KLayout<D>::k_off(lane, i / KS, i % KS));
  };
  bf16x8 f[NF];
#pragma unroll
  for (int i = 0; i < kPrefetch; ++i) f[i] = frag(i);
  // The scheduler would otherwise sink each read next to its MFMA (fewest live registers) and
  // expose the full LDS latency on every step; the scheduling barriers keep the reads kPrefetch
  // steps ahead.
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < NF; ++i) {
    if (i + kPrefetch < NF) f[i + kPrefetch] = frag(i + kPrefetch);
    const int kb = i / KS, ks = i % KS;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) s[kb][qb] = mfma32(f[i], qf[qb][ks], ks == 0 ? f32x16{} : s[kb][qb]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Set element r of s to -inf when off(r) >= lim, off(r) = kb*32 + (r/8)*16 + r%8 being the key's
// offset inside the tile minus 8*(lane/32).  Pure VGPR arithmetic (shift mask + bitfield select,
// one v_bfi_b32): a compare per element would park 64 lane masks in SGPRs.
__device__ __forceinline__ float select_neg_inf(float x, uint32_t m) {   // m: all ones -> -inf
  return __uint_as_float((0xFF800000u & m) | (__float_as_uint(x) & ~m));
}

// offset of element r of a lane's s[kb] inside the tile, less 8*(lane/32)
__device__ __forceinline__ constexpr int elem_key(int kb, int r) {
  return kb * 32 + (r >> 3) * 16 + (r & 7);
}

__device__ __forceinline__ void mask_block(f32x16& s, int kb, int lim) {
#pragma unroll
  for (int r = 0; r < 16; ++r)
    s[r] = select_neg_inf(s[r], (uint32_t)((lim - 1 - elem_key(kb, r)) >> 31));   // off >= lim
}

// Key index (0..63 inside the tile) held in element r of this lane's s[kb][*] block.
__device__ __forceinline__ int tile_key(int kb, int r, int lane) {
  return elem_key(kb, r) + (lane >> 5) * 8;
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

// Store the wave's normalised output rows: o[db][qb] element r is d = 32*db + (r/4)*8 + 4*h + r%4.
template <int D, int QB>
__device__ __forceinline__ void store_o(__bf16* out, int64_t row_stride, int rows_valid,
                                        const f32x16 (&o)[D / 32][QB], const float (&inv)[QB],
                                        int lane) {
  const int h = lane >> 5, r32 = lane & 31;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
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
