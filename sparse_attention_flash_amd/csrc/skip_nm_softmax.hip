// skip_nm_softmax.hip -- skip-softmax and N:M sparse softmax in one flash-attention forward.
//
// Method: the combined configuration of Model-Optimizer "Attention Sparsity for HuggingFace
// Models" (skip_softmax_calib_sparse24: calibrated skip-softmax together with 2:4 sparse softmax),
// each rule as in skip_softmax.hip and nm_softmax.hip.  Reading (stated in sa.h): the N:M rule
// fixes which keys of each query row may enter the softmax, and the skip loop runs over the tiles
// of those masked scores.  Because top-N keeps every group maximum, the masked tile maxima equal
// the unmasked ones, so the skip decision is taken exactly as in the skip-softmax kernel and the
// N:M bits only gate P inside kept tiles (SkipNmPolicy, policies.h).
#include "policies.h"

namespace sa {
namespace {

template <int D, int NW, int QB, int M, bool kPair>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(kWavesPerSimd<QB>)))
void skip_nm_softmax_kernel(SkipNmArgs a) {
  __shared__ __attribute__((aligned(1024))) Smem<D, NW> sm;
  attention_tile<D, NW, QB, SkipNmPolicy<D, NW, QB, M, kPair>>(a, sm);
}

template <int D, int NW, int QB, int M, bool kPair>
hipError_t launch_t(const SkipNmArgs& a, hipStream_t stream) {
  constexpr int BR = NW * 32 * QB;
  const int nQT = (a.g.Sq + BR - 1) / BR;
  const int total = a.g.B * a.g.Hq * nQT;
  hipLaunchKernelGGL((skip_nm_softmax_kernel<D, NW, QB, M, kPair>), dim3(total), dim3(NW * 64), 0,
                     stream, a);
  return hipGetLastError();
}

template <int D, int NW, int QB>
hipError_t launch_m(const SkipNmArgs& a, hipStream_t stream) {
  const bool pair = a.g.block_k == 128;   // 128-key decision tiles: two 64-key steps together
  if (a.m == 8)
    return pair ? launch_t<D, NW, QB, 8, true>(a, stream) : launch_t<D, NW, QB, 8, false>(a, stream);
  return pair ? launch_t<D, NW, QB, 4, true>(a, stream) : launch_t<D, NW, QB, 4, false>(a, stream);
}

}  // namespace

hipError_t launch_skip_nm_softmax(const SkipNmArgs& a, hipStream_t stream) {
  constexpr int QB = kQueryBlocksPerWave;
  const bool q128 = a.g.block_q == 128;
  if (a.g.D == 128)
    return q128 ? launch_m<128, 4 / QB, QB>(a, stream) : launch_m<128, 2 / QB, QB>(a, stream);
  return q128 ? launch_m<64, 4 / QB, QB>(a, stream) : launch_m<64, 2 / QB, QB>(a, stream);
}

}  // namespace sa
