// route_prep.hip -- bitmask route preparation for the block-sparse proxy path (gfx950).
//
// FlashInfer block-sparse proxy description ("Bitmask format"): exact KV blocks arrive as packed
// UInt32 bitmaps, one per (batch, KV head, query block); out-of-range padding bits in the final
// word are ignored; the bitmap is prepared into one route stream plus score-keep metadata so a
// block covered by an exact route is not also counted by its proxy.
//
// Our route stream: n_exact, the exact block indices in ascending order (-1 after them) and
// proxy_keep = the complement of the exact bits over the valid blocks.  One wavefront per bitmap
// row: each lane takes one 32-bit word, popcounts it, a wavefront prefix sum gives its output
// offset, and the lane then writes its set-bit positions in ascending order.
#include "kernels.h"

namespace sa {
namespace {

constexpr int kWavesPerBlock = 4;

__global__ __launch_bounds__(kWavesPerBlock * 64) void route_prep_kernel(RouteArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (row >= a.rows) return;   // whole wavefront leaves together
  const uint32_t* bits = a.bitmask + row * a.W;
  uint32_t* keep = a.proxy_keep + row * a.W;
  int32_t* idx = a.exact_idx + row * a.nKB;

  int base = 0;   // exact blocks found in earlier 64-word chunks
  for (int w0 = 0; w0 < a.W; w0 += 64) {
    const int w = w0 + lane;
    uint32_t word = 0u, valid = 0u;
    if (w < a.W) {
      const int nbits = a.nKB - 32 * w;   // >= 1 for every w < W
      valid = nbits >= 32 ? 0xFFFFFFFFu : ((1u << nbits) - 1u);
      word = bits[w] & valid;
      keep[w] = ~word & valid;
    }
    const int cnt = __popc(word);
    int incl = cnt;   // inclusive prefix sum over the wavefront
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int up = __shfl_up(incl, d, 64);
      if (lane >= d) incl += up;
    }
    int pos = base + incl - cnt;
    while (word != 0u) {
      const int bit = __ffs(word) - 1;
      idx[pos++] = 32 * w + bit;
      word &= word - 1u;
    }
    base += __shfl(incl, 63, 64);
  }
  for (int j = base + lane; j < a.nKB; j += 64) idx[j] = -1;
  if (lane == 0) a.n_exact[row] = base;
}

}  // namespace

hipError_t launch_route_prep(const RouteArgs& a, hipStream_t stream) {
  if (a.rows == 0) return hipSuccess;
  const int blocks = (int)((a.rows + kWavesPerBlock - 1) / kWavesPerBlock);
  hipLaunchKernelGGL(route_prep_kernel, dim3(blocks), dim3(kWavesPerBlock * 64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace sa
