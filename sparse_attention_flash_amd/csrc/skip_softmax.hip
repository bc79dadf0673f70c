// skip_softmax.hip -- skip-softmax (BLASST-style) flash-attention forward for gfx950.
//
// Method: Model-Optimizer "Skip-Softmax Sparse Attention for Diffusion Models" README
// (introduction; "Threshold Modes"): during the FlashAttention loop a key tile whose scores are
// negligible is skipped, which saves its exponentials, its V load and its P.V product; the kernel
// works with log2(lambda).  Decision rule (the reading stated in sa.h): with t = c*q.k in the log2
// domain, tile j is skipped when every valid row r of the query tile has
//     M_j[r] < fl32(m[r] + log2(lambda)),
// m[r] being the fp32 running max of the tiles kept so far; a skipped tile leaves (m, l, O) alone.
//
// The pipelined loop (mainloop.h) computes S^T = K.Q^T on MFMA, masks, takes the row max (in-lane
// plus one permlane32 swap), and each wavefront votes "some row not negligible" with a ballot; the
// votes meet in LDS at the barrier that also publishes the previous V tile.  Only a kept tile has
// its V tile fetched and runs exp2 + P.V.  The rule itself is SkipDecision (policies.h).
// Decision granularity (Model-Optimizer "Attention Sparsity for HuggingFace Models", "Custom
// Configuration": the br x bc blocks): the whole query tile, or each 32-row wavefront on its own.
#include "policies.h"

namespace sa {
namespace {

template <int D, int NW, int QB, bool kWave, bool kPair>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(kWavesPerSimd<QB>)))
void skip_softmax_kernel(SkipArgs a) {
  __shared__ __attribute__((aligned(1024))) Smem<D, NW> sm;
  attention_tile<D, NW, QB, SkipPolicy<D, NW, QB, kWave, kPair>>(a, sm);
}

template <int D, int NW, int QB, bool kWave, bool kPair>
hipError_t launch_t(const SkipArgs& a, hipStream_t stream) {
  constexpr int BR = NW * 32 * QB;
  const int nQT = (a.g.Sq + BR - 1) / BR;
  const int total = a.g.B * a.g.Hq * nQT;
  hipLaunchKernelGGL((skip_softmax_kernel<D, NW, QB, kWave, kPair>), dim3(total), dim3(NW * 64),
                     0, stream, a);
  return hipGetLastError();
}

// decision granularity (tile or 32-row wave) and decision tile (64 or 128 keys)
template <int D, int NW, int QB>
hipError_t launch_d(const SkipArgs& a, hipStream_t stream) {
  const bool pair = a.g.block_k == 128;
  if (a.wave_gran)
    return pair ? launch_t<D, NW, QB, true, true>(a, stream)
                : launch_t<D, NW, QB, true, false>(a, stream);
  return pair ? launch_t<D, NW, QB, false, true>(a, stream)
              : launch_t<D, NW, QB, false, false>(a, stream);
}

}  // namespace

// Query tiles of block_q rows run as block_q/32 wavefronts of 32 rows each (kQueryBlocksPerWave =
// 1): the per-wave state then fits in half the register file, so two workgroups share each CU and
// one's MFMA work overlaps the other's softmax arithmetic.  A 128-key decision tile runs as two
// 64-key steps decided together.
hipError_t launch_skip_softmax(const SkipArgs& a, hipStream_t stream) {
  constexpr int QB = kQueryBlocksPerWave;
  const bool q128 = a.g.block_q == 128;
  if (a.g.D == 128)
    return q128 ? launch_d<128, 4 / QB, QB>(a, stream) : launch_d<128, 2 / QB, QB>(a, stream);
  return q128 ? launch_d<64, 4 / QB, QB>(a, stream) : launch_d<64, 2 / QB, QB>(a, stream);
}

}  // namespace sa
