// kernels.h -- internal launch interface between the C-ABI host layer and the gfx950 kernels.
// Host code fills these plain structs after validating the call; launchers enqueue on `stream`
// and return the hipGetLastError() status of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sa {

struct AttnGeom {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  int64_t qs[3], ks[3], vs[3], os[3];   // batch, seq, head strides (elements)
  int B, Hq, Hkv, Sq, Sk, D, causal, block_q, block_k;
  float c32;                            // softmax_scale * log2(e), rounded to fp32
};

struct SkipArgs {
  AttnGeom g;
  float L32;                            // log2(lambda) in fp32; -inf when lambda == 0
  int wave_gran;                        // 1: each 32-row wavefront decides alone
  uint8_t* tile_state;
  uint32_t* counters;
  float* lse;
  float* rowmax;
};

struct NmArgs {
  AttnGeom g;
  int n, m, sink, recent;
  float* lse;
  uint32_t* keep_bits;
  float* scores;
};

// skip-softmax with the N:M rule inside kept tiles: the fields of SkipArgs and NmArgs
struct SkipNmArgs {
  AttnGeom g;
  float L32;
  uint8_t* tile_state;
  uint32_t* counters;
  float* lse;
  float* rowmax;
  int n, m, sink, recent;
  uint32_t* keep_bits;
  float* scores;
};

// Decode-phase skip-softmax (one query token per head, key axis split over workgroups).
constexpr int kMaxTilesPerSplit = 4096;

// Whole-sequence decode: one workgroup per (batch, KV head) keeps the scores of its G heads over
// the whole key range in LDS, when they fit in this many bytes (GM <= kFusedMaxGM).
constexpr int kFusedScoreBytes = 128 * 1024;
constexpr int kFusedMaxGM = 8;

struct DecodeArgs {
  AttnGeom g;                           // Sq == 1, non-causal
  float L32;
  const int32_t* seqlens_k;             // optional [B], keys per sequence (clamped to [0, Sk])
  int block_k;                          // 64 or 128: the decision tile
  int nKT, nsplit, tiles_per_split;
  int fused;                            // 1: one whole-sequence kernel (nsplit == 1, no workspace)
  float* dbg_tmax;                      // optional [B, Hq, nKT] export of the tile maxima (fused)
  float* scores;                        // workspace [B, Hkv, GM, nKT*block_k] raw q.k (GM >= G)
  float* tmax;                          // [B, Hq, nKT] tile maxima, log2 domain
  float* part_m;                        // [B, Hq, nsplit] split reference (max of kept maxima)
  float* part_l;                        // [B, Hq, nsplit]
  float* part_o;                        // [B, Hq, nsplit, D]
  uint8_t* tile_state;                  // optional [B, Hq, nKT]
  uint32_t* counters;                   // optional [B, Hq, 2]
  float* lse;                           // optional [B, Hq]
};

struct RouteArgs {
  const uint32_t* bitmask;
  int32_t* n_exact;
  int32_t* exact_idx;
  uint32_t* proxy_keep;
  int64_t rows;                         // B * Hkv * nQB
  int nKB, W;
};

// BSR rows are expanded into an LDS bitmap of at most this many words (nKB <= 32 * kBsrMaxWords).
constexpr int kBsrMaxWords = 2048;

struct BsrRouteArgs {
  const int32_t* indptr;                // [rows + 1]
  const int32_t* indices;               // [nnz]
  int64_t nnz;
  int32_t* n_exact;
  int32_t* exact_idx;
  uint32_t* proxy_keep;
  uint32_t* bad_rows;                   // optional
  int64_t rows;                         // B * Hkv * nQB
  int nKB, W;
};

struct ProxyArgs {
  AttnGeom g;
  const void* k_mean;
  const void* v_sum;
  const int32_t* n_exact;
  const int32_t* exact_idx;
  const uint32_t* proxy_keep;
  int use_proxy;
  float* lse;
};

hipError_t launch_skip_softmax(const SkipArgs& a, hipStream_t stream);
hipError_t launch_nm_softmax(const NmArgs& a, hipStream_t stream);
hipError_t launch_skip_nm_softmax(const SkipNmArgs& a, hipStream_t stream);
hipError_t launch_skip_decode(const DecodeArgs& a, hipStream_t stream);

// Device scratch of the allocation-free decode entry point: a fixed file-scope device array (one
// copy per GPU, held until the process ends).  decode_scratch() returns the current device's
// address of it, looked up once per device.
constexpr size_t kDecodeScratchBytes = (size_t)32 << 20;
hipError_t decode_scratch(void** ptr);
hipError_t launch_route_prep(const RouteArgs& a, hipStream_t stream);
hipError_t launch_bsr_route_prep(const BsrRouteArgs& a, hipStream_t stream);
hipError_t launch_proxy(const ProxyArgs& a, hipStream_t stream);

}  // namespace sa
