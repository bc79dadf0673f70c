// peak_probes.hip -- microbenchmarks that re-measure the bf16 MFMA rate and the HBM read rate of
// the part (libsa_probes.so; declared in include/sa_probes.h).
#include <hip/hip_runtime.h>

#include "sa_probes.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Four independent chains per wave: each MFMA depends only on its own chain's previous result, so
// the matrix core always has independent work in flight.  With random_operands the chains take two
// sets of random bf16 operands (magnitudes in [0.5, 1), random signs) in turn, so every issue
// changes the multiplier inputs as attention's data does; the power that draws lowers the clock
// under sustained load.  Without it the operands are small constants that never change.
__device__ __forceinline__ unsigned mix(unsigned h) {
  h ^= h >> 16;
  h *= 0x7feb352du;
  h ^= h >> 15;
  h *= 0x846ca68bu;
  return h ^ (h >> 16);
}

__global__ __launch_bounds__(256) void mfma_loop(float* out, int iters, int random_operands) {
  const int lane = threadIdx.x & 63;
  bf16x8 a0, b0, a1, b1;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    if (random_operands) {
      const unsigned h = mix((unsigned)(threadIdx.x * 8 + e) ^ (blockIdx.x * 0x9e3779b9u));
      a0[e] = __builtin_bit_cast(__bf16, (unsigned short)((h & 0x807Fu) | 0x3F00u));
      b0[e] = __builtin_bit_cast(__bf16, (unsigned short)(((h >> 8) & 0x807Fu) | 0x3F00u));
      a1[e] = __builtin_bit_cast(__bf16, (unsigned short)(((h >> 16) & 0x807Fu) | 0x3F00u));
      b1[e] = __builtin_bit_cast(__bf16, (unsigned short)(((h >> 4) & 0x807Fu) | 0x3F00u));
    } else {
      a0[e] = a1[e] = (__bf16)(0.001f * (float)((lane + e) & 7));
      b0[e] = b1[e] = (__bf16)(0.001f * (float)((lane * 3 + e) & 7));
    }
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b0, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b1, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b0, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b1, c3, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) s += c0[e] + c1[e] + c2[e] + c3[e];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

constexpr int kReadWaves = 8;
constexpr int kReadDepth = 4;
constexpr int kChunkVec = 16384 / 16;   // 16-byte vectors per chunk

// Chunk c of the buffer is read by wave (c mod (grid*8)) in rounds of kReadDepth chunks; indices
// past the last chunk are clamped to it (a few repeated reads at the very end).
__global__ __launch_bounds__(64 * kReadWaves) void read_stream(const u32x4* __restrict__ x,
                                                                size_t nch, unsigned* out) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const size_t step = (size_t)gridDim.x * kReadWaves;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (size_t c = (size_t)blockIdx.x * kReadWaves + wave; c < nch; c += step * kReadDepth) {
    u32x4 v[kReadDepth][16];
#pragma unroll
    for (int d = 0; d < kReadDepth; ++d) {
      const size_t cc = c + d * step < nch ? c + d * step : nch - 1;
#pragma unroll
      for (int i = 0; i < 16; ++i) v[d][i] = x[cc * kChunkVec + i * 64 + lane];
    }
#pragma unroll
    for (int d = 0; d < kReadDepth; ++d)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc ^= v[d][i];
  }
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

}  // namespace

extern "C" double sa_probe_mfma_bf16_flops(int workgroups, int iters) {
  return (double)workgroups * 4.0 * (double)iters * 4.0 * 32768.0;
}

extern "C" int sa_probe_mfma_bf16(float* out, int workgroups, int iters, int random_operands,
                                  void* stream) {
  if (out == nullptr || workgroups < 1 || iters < 1) return 1;
  hipLaunchKernelGGL(mfma_loop, dim3(workgroups), dim3(256), 0, (hipStream_t)stream, out, iters,
                     random_operands != 0 ? 1 : 0);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

extern "C" int sa_probe_read(const void* buf, size_t bytes, unsigned* out, int workgroups,
                             void* stream) {
  if (buf == nullptr || out == nullptr || workgroups < 1 || bytes == 0 || bytes % 16384 != 0 ||
      ((size_t)buf & 15) != 0)
    return 1;
  hipLaunchKernelGGL(read_stream, dim3(workgroups), dim3(64 * kReadWaves), 0, (hipStream_t)stream,
                     (const u32x4*)buf, bytes / 16384, out);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
