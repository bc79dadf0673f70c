// route_prep.hip -- route preparation for the block-sparse proxy path (gfx950).
//
// FlashInfer block-sparse proxy description ("Bitmask format"): exact KV blocks arrive either as
// packed UInt32 bitmaps, one per (batch, KV head, query block), whose out-of-range padding bits in
// the final word are ignored, or as canonical BSR (block_indptr / block_indices); both are prepared
// into one route stream plus score-keep metadata, so a block covered by an exact route is not also
// counted by its proxy, and the two formats give bitwise-identical results.
//
// Our route stream: n_exact, the exact block indices in ascending order (-1 after them) and
// proxy_keep = the complement of the exact bits over the valid blocks.  One wavefront per row: each
// lane takes one 32-bit word of the row's bitmap, popcounts it, a wavefront prefix sum gives its
// output offset, and the lane then writes its set-bit positions in ascending order.  A BSR row is
// first turned into that bitmap in LDS, so both formats share the emission step.
#include "kernels.h"

namespace sa {
namespace {

constexpr int kWavesPerBlock = 4;

// Writes one row's route stream from its bitmap; word(w) returns word w (w < W) of the row.
template <class WordFn>
__device__ __forceinline__ void emit_route(int lane, int W, int nKB, WordFn word_of,
                                           uint32_t* keep, int32_t* idx, int32_t* n_exact) {
  int base = 0;   // exact blocks found in earlier 64-word chunks
  for (int w0 = 0; w0 < W; w0 += 64) {
    const int w = w0 + lane;
    uint32_t word = 0u;
    if (w < W) {
      const int nbits = nKB - 32 * w;   // >= 1 for every w < W
      const uint32_t valid = nbits >= 32 ? 0xFFFFFFFFu : ((1u << nbits) - 1u);
      word = word_of(w) & valid;
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
  for (int j = base + lane; j < nKB; j += 64) idx[j] = -1;
  if (lane == 0) *n_exact = base;
}

__global__ __launch_bounds__(kWavesPerBlock * 64) void route_prep_kernel(RouteArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (row >= a.rows) return;   // whole wavefront leaves together
  const uint32_t* bits = a.bitmask + row * a.W;
  emit_route(lane, a.W, a.nKB, [&](int w) { return bits[w]; }, a.proxy_keep + row * a.W,
             a.exact_idx + row * a.nKB, a.n_exact + row);
}

// One wavefront (= one workgroup) per BSR row: the row's entries are OR-ed into an LDS bitmap, so
// duplicates collapse and order does not matter; entries outside [0, nKB) are dropped.  Pointer
// ranges are clamped to [0, nnz], so nothing past the index array is read.
__global__ __launch_bounds__(64) void bsr_route_prep_kernel(BsrRouteArgs a) {
  __shared__ uint32_t bm[kBsrMaxWords];
  const int lane = threadIdx.x;
  const int64_t row = blockIdx.x;
  for (int w = lane; w < a.W; w += 64) bm[w] = 0u;
  __syncthreads();

  const int64_t p0 = a.indptr[row], p1 = a.indptr[row + 1];
  const int64_t start = min(max(p0, (int64_t)0), a.nnz);
  const int64_t end = min(max(p1, start), a.nnz);
  bool bad = p0 < 0 || p1 < p0 || p1 > a.nnz;
  for (int64_t e = start + lane; e < end; e += 64) {
    const int32_t j = a.indices[e];
    if (j < 0 || j >= a.nKB) bad = true;
    else atomicOr(&bm[j >> 5], 1u << (j & 31));
    if (e > start && a.indices[e - 1] >= j) bad = true;
  }
  __syncthreads();
  if (a.bad_rows != nullptr && __ballot(bad) != 0ull && lane == 0) atomicAdd(a.bad_rows, 1u);
  emit_route(lane, a.W, a.nKB, [&](int w) { return bm[w]; }, a.proxy_keep + row * a.W,
             a.exact_idx + row * a.nKB, a.n_exact + row);
}

}  // namespace

hipError_t launch_route_prep(const RouteArgs& a, hipStream_t stream) {
  if (a.rows == 0) return hipSuccess;
  const int blocks = (int)((a.rows + kWavesPerBlock - 1) / kWavesPerBlock);
  hipLaunchKernelGGL(route_prep_kernel, dim3(blocks), dim3(kWavesPerBlock * 64), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_bsr_route_prep(const BsrRouteArgs& a, hipStream_t stream) {
  if (a.rows == 0) return hipSuccess;
  hipLaunchKernelGGL(bsr_route_prep_kernel, dim3((unsigned)a.rows), dim3(64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace sa
