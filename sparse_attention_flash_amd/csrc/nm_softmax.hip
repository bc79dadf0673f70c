// nm_softmax.hip -- N:M sparse softmax flash-attention forward for gfx950.
//
// Method: Model-Optimizer "Attention Sparsity for HuggingFace Models", "N:M Sparse Softmax": for
// every M consecutive key positions keep the top-N attention scores and set the rest to -inf
// before the softmax; the first dense_sink_tokens keys and a window of dense_recent_tokens recent
// keys stay dense; M = 4 (N = 1..3) or M = 8 (N = 1..7); prefill only.  Readings (stated in sa.h):
// groups aligned to key 0, ranking by the raw score q.k among all members of the group (masked
// keys rank last), ties to the lower key index, "recent" = 0 <= row - key < R.
//
// Same pipelined loop as the skip-softmax kernel (mainloop.h), every visited tile kept; the rule
// is NmFilter (policies.h).  Nothing here depends on the key tile: block_k 64 and 128 run the same
// kernel and give the same result.
#include "policies.h"

namespace sa {
namespace {

template <int D, int NW, int QB, int M>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(kWavesPerSimd<QB>)))
void nm_softmax_kernel(NmArgs a) {
  __shared__ __attribute__((aligned(1024))) Smem<D, NW> sm;
  attention_tile<D, NW, QB, NmPolicy<D, NW, QB, M>>(a, sm);
}

template <int D, int NW, int QB, int M>
hipError_t launch_t(const NmArgs& a, hipStream_t stream) {
  constexpr int BR = NW * 32 * QB;
  const int nQT = (a.g.Sq + BR - 1) / BR;
  const int total = a.g.B * a.g.Hq * nQT;
  hipLaunchKernelGGL((nm_softmax_kernel<D, NW, QB, M>), dim3(total), dim3(NW * 64), 0, stream, a);
  return hipGetLastError();
}

template <int D, int NW, int QB>
hipError_t launch_m(const NmArgs& a, hipStream_t stream) {
  return a.m == 8 ? launch_t<D, NW, QB, 8>(a, stream) : launch_t<D, NW, QB, 4>(a, stream);
}

}  // namespace

hipError_t launch_nm_softmax(const NmArgs& a, hipStream_t stream) {
  constexpr int QB = kQueryBlocksPerWave;
  const bool q128 = a.g.block_q == 128;
  if (a.g.D == 128)
    return q128 ? launch_m<128, 4 / QB, QB>(a, stream) : launch_m<128, 2 / QB, QB>(a, stream);
  return q128 ? launch_m<64, 4 / QB, QB>(a, stream) : launch_m<64, 2 / QB, QB>(a, stream);
}

}  // namespace sa
