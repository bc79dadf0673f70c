// api.hip -- the extern "C" entry points of libsa_hip.so (declared and documented in sa.h).
//
// Every argument check runs here, on the host, before any HIP call: a rejected call enqueues and
// writes nothing, which also lets the checks be exercised on a machine without a GPU.  Accepted
// calls are lowered into the plain launch structs of kernels.h (the user-facing description is
// not passed to the kernels) and enqueued on the caller's stream.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <vector>

#include "kernels.h"
#include "sa.h"

static_assert(sa::kDecodeScratchBytes == SA_DECODE_SCRATCH_BYTES,
              "the scratch size sa.h states is the array's");

namespace {

constexpr double kLog2eD = 1.4426950408889634074;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool strides_ok(const int64_t (&s)[3]) {
  for (int i = 0; i < 3; ++i)
    if (s[i] < 0 || s[i] % 8 != 0) return false;
  return true;
}

// Checks shared by the three attention entry points.
sa_status check_attention(const sa_attn_desc* d, const void* q, const void* k, const void* v,
                          const void* o) {
  if (d == nullptr || q == nullptr || k == nullptr || v == nullptr || o == nullptr)
    return SA_ERR_NULL;
  if (d->batch < 1 || d->heads_q < 1 || d->heads_kv < 1 || d->seqlen_q < 1 || d->seqlen_k < 1 ||
      d->head_dim < 1 || d->block_q < 1 || d->block_k < 1)
    return SA_ERR_SHAPE;
  if (d->heads_q % d->heads_kv != 0) return SA_ERR_SHAPE;
  if (d->causal != 0 && d->causal != 1) return SA_ERR_VALUE;
  if (d->causal && d->seqlen_q != d->seqlen_k) return SA_ERR_SHAPE;
  if (!(d->softmax_scale > 0.f) || !std::isfinite(d->softmax_scale)) return SA_ERR_VALUE;
  if (d->head_dim != 64 && d->head_dim != 128) return SA_ERR_UNSUPPORTED;
  if (d->block_q != 64 && d->block_q != 128) return SA_ERR_UNSUPPORTED;
  // grid and row indices are 32-bit inside the kernels
  const int64_t n_qt = (d->seqlen_q + 63) / 64;
  if ((int64_t)d->batch * d->heads_q * n_qt > INT32_MAX || d->seqlen_q > INT32_MAX - 256 ||
      d->seqlen_k > INT32_MAX - 256)
    return SA_ERR_SHAPE;
  // Q/K/V are read through buffer resources with 32-bit byte offsets (tile reads may run up to
  // 256 rows past the end of a slab)
  const auto slab_fits = [&](int64_t rows, int64_t row_stride) {
    return (rows + 256) * row_stride * 2 + (int64_t)d->head_dim * 2 < (int64_t)INT32_MAX;
  };
  if (!slab_fits(d->seqlen_q, d->q_stride[1]) || !slab_fits(d->seqlen_k, d->k_stride[1]) ||
      !slab_fits(d->seqlen_k, d->v_stride[1]))
    return SA_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return SA_ERR_ALIGN;
  if (!strides_ok(d->q_stride) || !strides_ok(d->k_stride) || !strides_ok(d->v_stride) ||
      !strides_ok(d->o_stride))
    return SA_ERR_ALIGN;
  return SA_OK;
}

sa::AttnGeom geometry(const sa_attn_desc* d, const void* q, const void* k, const void* v,
                      void* o) {
  sa::AttnGeom g{};
  g.q = q;
  g.k = k;
  g.v = v;
  g.o = o;
  for (int i = 0; i < 3; ++i) {
    g.qs[i] = d->q_stride[i];
    g.ks[i] = d->k_stride[i];
    g.vs[i] = d->v_stride[i];
    g.os[i] = d->o_stride[i];
  }
  g.B = d->batch;
  g.Hq = d->heads_q;
  g.Hkv = d->heads_kv;
  g.Sq = d->seqlen_q;
  g.Sk = d->seqlen_k;
  g.D = d->head_dim;
  g.causal = d->causal;
  g.block_q = d->block_q;
  g.block_k = d->block_k;
  g.c32 = (float)((double)d->softmax_scale * kLog2eD);
  return g;
}

sa_status from_hip(hipError_t e) { return e == hipSuccess ? SA_OK : SA_ERR_HIP; }

// Decode: split plan and workspace layout, the same for the size query and the call.
struct DecodePlan {
  int GM, nKT, nsplit, tps, fused;
  size_t off_scores, off_tmax, off_pm, off_pl, off_po, bytes;
};

sa_status plan_decode(const sa_attn_desc* d, float lambda, int32_t num_splits, DecodePlan* p) {
  if (d->seqlen_q != 1 || d->causal != 0) return SA_ERR_UNSUPPORTED;
  if (d->block_k != 64 && d->block_k != 128) return SA_ERR_UNSUPPORTED;
  if (!(lambda >= 0.f) || !std::isfinite(lambda)) return SA_ERR_VALUE;
  if (num_splits < 0) return SA_ERR_VALUE;
  const int G = d->heads_q / d->heads_kv;
  const int gmax = d->head_dim == 128 ? 16 : 8;   // one writer lane per head in a key row
  if (G > gmax) return SA_ERR_UNSUPPORTED;
  p->GM = G <= 1 ? 1 : G <= 2 ? 2 : G <= 4 ? 4 : G <= 8 ? 8 : 16;
  p->nKT = (int)(((int64_t)d->seqlen_k + d->block_k - 1) / d->block_k);
  const int64_t units = (int64_t)d->batch * d->heads_kv;
  // One workgroup per (batch, KV head) holding its heads' scores for the whole cache in LDS, when
  // they fit: no workspace and no exchange between workgroups.  Chosen whenever the call runs one
  // split -- asked for, or lambda > 1, whose decisions depend on the order of the kept tiles.
  // With several splits the key axis spreads over more workgroups than there are (batch, KV head)
  // units, which streams faster when those units are fewer than the CUs (measured on the
  // 16 x 8-KV-head decode workload: 119 us per step with two splits against 136 us whole-sequence).
  const bool fits = p->GM <= sa::kFusedMaxGM &&
                    (int64_t)p->GM * p->nKT * d->block_k * 4 <= sa::kFusedScoreBytes;
  p->fused = fits && (num_splits == 1 || (num_splits == 0 && lambda > 1.f));
  if (p->fused) {
    p->nsplit = 1;
    p->tps = p->nKT;
    p->off_scores = p->off_tmax = p->off_pm = p->off_pl = p->off_po = 0;
    p->bytes = 256;   // no workspace is used; the callers' contract keeps a non-empty buffer
    return SA_OK;
  }
  int ns;
  if (lambda > 1.f) {
    // decisions depend on the order of the kept tiles: one split walks them all
    if (num_splits > 1) return SA_ERR_UNSUPPORTED;
    ns = 1;
  } else if (num_splits > 0) {
    ns = num_splits;
  } else {
    // about one workgroup per compute unit: a longer key range per wave hides the start-up of
    // its load stream better than more, shorter workgroups do
    ns = (int)std::min<int64_t>(std::max<int64_t>(1, (256 + units - 1) / units), p->nKT);
  }
  ns = std::min(ns, p->nKT);
  int tps = (p->nKT + ns - 1) / ns;
  if (tps > sa::kMaxTilesPerSplit) {
    if (lambda > 1.f || num_splits > 0) return SA_ERR_UNSUPPORTED;
    tps = sa::kMaxTilesPerSplit;
  }
  p->tps = tps;
  p->nsplit = (p->nKT + tps - 1) / tps;
  if (units * p->nsplit > INT32_MAX) return SA_ERR_SHAPE;
  const auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t heads = (size_t)d->batch * d->heads_q;
  size_t off = 0;
  p->off_scores = off;
  off += up((size_t)units * p->GM * p->nKT * d->block_k * sizeof(float));
  p->off_tmax = off;
  off += up(heads * p->nKT * sizeof(float));
  p->off_pm = off;
  off += up(heads * p->nsplit * sizeof(float));
  p->off_pl = off;
  off += up(heads * p->nsplit * sizeof(float));
  p->off_po = off;
  off += up(heads * p->nsplit * d->head_dim * sizeof(float));
  p->bytes = off;
  return SA_OK;
}



// Enqueue the three decode kernels over the workspace at `ws` laid out by the plan (every region
// is written before it is read, so nothing needs clearing).
sa_status decode_run(const sa_attn_desc& d, const DecodePlan& p, const void* q, const void* k,
                     const void* v, void* o, float lambda, const int32_t* seqlens_k, char* ws,
                     uint8_t* tile_state, uint32_t* head_counters, float* lse,
                     float* dbg_tile_rowmax, void* stream) {
  sa::DecodeArgs a{};
  a.g = geometry(&d, q, k, v, o);
  a.L32 = lambda == 0.f ? -INFINITY : (float)std::log2((double)lambda);
  a.seqlens_k = seqlens_k;
  a.block_k = d.block_k;
  a.nKT = p.nKT;
  a.nsplit = p.nsplit;
  a.tiles_per_split = p.tps;
  a.fused = p.fused;
  a.dbg_tmax = dbg_tile_rowmax;
  a.scores = reinterpret_cast<float*>(ws + p.off_scores);
  a.tmax = dbg_tile_rowmax != nullptr ? dbg_tile_rowmax : reinterpret_cast<float*>(ws + p.off_tmax);
  a.part_m = reinterpret_cast<float*>(ws + p.off_pm);
  a.part_l = reinterpret_cast<float*>(ws + p.off_pl);
  a.part_o = reinterpret_cast<float*>(ws + p.off_po);
  a.tile_state = tile_state;
  a.counters = head_counters;
  a.lse = lse;
  return from_hip(sa::launch_skip_decode(a, (hipStream_t)stream));
}

}  // namespace

extern "C" {

const char* sa_status_str(sa_status status) {
  switch (status) {
    case SA_OK: return "SA_OK";
    case SA_ERR_NULL: return "SA_ERR_NULL: a required pointer is NULL";
    case SA_ERR_SHAPE: return "SA_ERR_SHAPE: inconsistent or out-of-range sizes";
    case SA_ERR_UNSUPPORTED: return "SA_ERR_UNSUPPORTED: configuration not implemented";
    case SA_ERR_ALIGN: return "SA_ERR_ALIGN: pointer or stride not 16-byte aligned";
    case SA_ERR_VALUE: return "SA_ERR_VALUE: invalid scalar argument";
    case SA_ERR_HIP: return "SA_ERR_HIP: the HIP runtime reported an error";
    case SA_ERR_SCRATCH:
      return "SA_ERR_SCRATCH: the call needs more device scratch than the fixed buffer holds";
  }
  return "unknown sa_status";
}

sa_status sa_skip_softmax_fwd_ex(const sa_attn_desc* desc, const void* q, const void* k,
                                 const void* v, void* o, float lambda, int32_t granularity,
                                 uint8_t* tile_state, uint32_t* head_counters, float* lse,
                                 float* dbg_tile_rowmax, void* stream) {
  sa_status st = check_attention(desc, q, k, v, o);
  if (st != SA_OK) return st;
  if (desc->block_k != 64 && desc->block_k != 128) return SA_ERR_UNSUPPORTED;
  if (granularity != SA_SKIP_GRAN_TILE && granularity != SA_SKIP_GRAN_WAVE) return SA_ERR_VALUE;
  if (!(lambda >= 0.f) || !std::isfinite(lambda)) return SA_ERR_VALUE;
  sa::SkipArgs a{};
  a.g = geometry(desc, q, k, v, o);
  a.L32 = lambda == 0.f ? -INFINITY : (float)std::log2((double)lambda);
  a.wave_gran = granularity == SA_SKIP_GRAN_WAVE;
  a.tile_state = tile_state;
  a.counters = head_counters;
  a.lse = lse;
  a.rowmax = dbg_tile_rowmax;
  return from_hip(sa::launch_skip_softmax(a, (hipStream_t)stream));
}

sa_status sa_skip_softmax_fwd(const sa_attn_desc* desc, const void* q, const void* k,
                              const void* v, void* o, float lambda, uint8_t* tile_state,
                              uint32_t* head_counters, float* lse, float* dbg_tile_rowmax,
                              void* stream) {
  return sa_skip_softmax_fwd_ex(desc, q, k, v, o, lambda, SA_SKIP_GRAN_TILE, tile_state,
                                head_counters, lse, dbg_tile_rowmax, stream);
}

sa_status sa_nm_softmax_fwd(const sa_attn_desc* desc, const void* q, const void* k,
                            const void* v, void* o, int32_t n, int32_t m,
                            int32_t dense_sink_tokens, int32_t dense_recent_tokens, float* lse,
                            uint32_t* dbg_keep_bits, float* dbg_scores, void* stream) {
  sa_status st = check_attention(desc, q, k, v, o);
  if (st != SA_OK) return st;
  if (desc->block_k != 64 && desc->block_k != 128) return SA_ERR_UNSUPPORTED;
  if (!((m == 4 && n >= 1 && n <= 4) || (m == 8 && n >= 1 && n <= 8))) return SA_ERR_UNSUPPORTED;
  if (dense_sink_tokens < 0 || dense_recent_tokens < 0) return SA_ERR_VALUE;
  sa::NmArgs a{};
  a.g = geometry(desc, q, k, v, o);
  a.n = n;
  a.m = m;
  a.sink = dense_sink_tokens;
  a.recent = dense_recent_tokens;
  a.lse = lse;
  a.keep_bits = dbg_keep_bits;
  a.scores = dbg_scores;
  return from_hip(sa::launch_nm_softmax(a, (hipStream_t)stream));
}

sa_status sa_skip_nm_softmax_fwd(const sa_attn_desc* desc, const void* q, const void* k,
                                 const void* v, void* o, float lambda, int32_t n, int32_t m,
                                 int32_t dense_sink_tokens, int32_t dense_recent_tokens,
                                 uint8_t* tile_state, uint32_t* head_counters, float* lse,
                                 float* dbg_tile_rowmax, uint32_t* dbg_keep_bits,
                                 float* dbg_scores, void* stream) {
  sa_status st = check_attention(desc, q, k, v, o);
  if (st != SA_OK) return st;
  if (desc->block_k != 64 && desc->block_k != 128) return SA_ERR_UNSUPPORTED;
  if (!((m == 4 && n >= 1 && n <= 4) || (m == 8 && n >= 1 && n <= 8))) return SA_ERR_UNSUPPORTED;
  if (dense_sink_tokens < 0 || dense_recent_tokens < 0) return SA_ERR_VALUE;
  if (!(lambda >= 0.f) || !std::isfinite(lambda)) return SA_ERR_VALUE;
  sa::SkipNmArgs a{};
  a.g = geometry(desc, q, k, v, o);
  a.L32 = lambda == 0.f ? -INFINITY : (float)std::log2((double)lambda);
  a.tile_state = tile_state;
  a.counters = head_counters;
  a.lse = lse;
  a.rowmax = dbg_tile_rowmax;
  a.n = n;
  a.m = m;
  a.sink = dense_sink_tokens;
  a.recent = dense_recent_tokens;
  a.keep_bits = dbg_keep_bits;
  a.scores = dbg_scores;
  return from_hip(sa::launch_skip_nm_softmax(a, (hipStream_t)stream));
}

sa_status sa_skip_softmax_decode_workspace(const sa_attn_desc* desc, float lambda,
                                           int32_t num_splits, size_t* workspace_bytes,
                                           int32_t* num_splits_used) {
  if (desc == nullptr || workspace_bytes == nullptr) return SA_ERR_NULL;
  if (desc->batch < 1 || desc->heads_q < 1 || desc->heads_kv < 1 || desc->seqlen_k < 1 ||
      desc->head_dim < 1 || desc->heads_q % desc->heads_kv != 0)
    return SA_ERR_SHAPE;
  if (desc->head_dim != 64 && desc->head_dim != 128) return SA_ERR_UNSUPPORTED;
  DecodePlan p;
  const sa_status st = plan_decode(desc, lambda, num_splits, &p);
  if (st != SA_OK) return st;
  *workspace_bytes = p.bytes;
  if (num_splits_used != nullptr) *num_splits_used = p.nsplit;
  return SA_OK;
}

sa_status sa_skip_softmax_decode_fwd(const sa_attn_desc* desc, const void* q, const void* k,
                                     const void* v, void* o, float lambda,
                                     const int32_t* seqlens_k, int32_t num_splits,
                                     void* workspace, size_t workspace_bytes,
                                     uint8_t* tile_state, uint32_t* head_counters, float* lse,
                                     float* dbg_tile_rowmax, void* stream) {
  if (desc == nullptr) return SA_ERR_NULL;
  // the query tile is the single query row: block_q plays no part
  sa_attn_desc d = *desc;
  d.block_q = 64;
  sa_status st = check_attention(&d, q, k, v, o);
  if (st != SA_OK) return st;
  DecodePlan p;
  st = plan_decode(&d, lambda, num_splits, &p);
  if (st != SA_OK) return st;
  if (workspace == nullptr) return SA_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return SA_ERR_ALIGN;
  if (workspace_bytes < p.bytes) return SA_ERR_SHAPE;
  return decode_run(d, p, q, k, v, o, lambda, seqlens_k, static_cast<char*>(workspace), tile_state,
                    head_counters, lse, dbg_tile_rowmax, stream);
}

sa_status sa_skip_softmax_decode_fwd_noalloc(const sa_attn_desc* desc, const void* q,
                                             const void* k, const void* v, void* o, float lambda,
                                             const int32_t* seqlens_k, int32_t num_splits,
                                             uint8_t* tile_state, uint32_t* head_counters,
                                             float* lse, float* dbg_tile_rowmax, void* stream) {
  if (desc == nullptr) return SA_ERR_NULL;
  sa_attn_desc d = *desc;
  d.block_q = 64;
  sa_status st = check_attention(&d, q, k, v, o);
  if (st != SA_OK) return st;
  DecodePlan p;
  st = plan_decode(&d, lambda, num_splits, &p);
  if (st != SA_OK) return st;
  if (p.bytes > sa::kDecodeScratchBytes) return SA_ERR_SCRATCH;
  void* ws = nullptr;
  if (sa::decode_scratch(&ws) != hipSuccess) return SA_ERR_HIP;
  return decode_run(d, p, q, k, v, o, lambda, seqlens_k, static_cast<char*>(ws), tile_state,
                    head_counters, lse, dbg_tile_rowmax, stream);
}

sa_status sa_bitmask_route_prep(const sa_attn_desc* desc, const uint32_t* bitmask,
                                int32_t* n_exact, int32_t* exact_idx, uint32_t* proxy_keep,
                                void* stream) {
  if (desc == nullptr || bitmask == nullptr || n_exact == nullptr || exact_idx == nullptr ||
      proxy_keep == nullptr)
    return SA_ERR_NULL;
  if (desc->batch < 1 || desc->heads_kv < 1 || desc->seqlen_q < 1 || desc->seqlen_k < 1 ||
      desc->block_q < 1 || desc->block_k < 1)
    return SA_ERR_SHAPE;
  sa::RouteArgs a{};
  const int64_t nQB = ((int64_t)desc->seqlen_q + desc->block_q - 1) / desc->block_q;
  a.nKB = (int)(((int64_t)desc->seqlen_k + desc->block_k - 1) / desc->block_k);
  a.W = (a.nKB + 31) / 32;
  a.rows = (int64_t)desc->batch * desc->heads_kv * nQB;
  if (a.rows > INT32_MAX) return SA_ERR_SHAPE;
  a.bitmask = bitmask;
  a.n_exact = n_exact;
  a.exact_idx = exact_idx;
  a.proxy_keep = proxy_keep;
  return from_hip(sa::launch_route_prep(a, (hipStream_t)stream));
}

sa_status sa_bsr_route_prep(const sa_attn_desc* desc, const int32_t* block_indptr,
                            const int32_t* block_indices, int64_t nnz, int32_t* n_exact,
                            int32_t* exact_idx, uint32_t* proxy_keep, uint32_t* bad_rows,
                            void* stream) {
  if (desc == nullptr || block_indptr == nullptr || n_exact == nullptr || exact_idx == nullptr ||
      proxy_keep == nullptr || (nnz > 0 && block_indices == nullptr))
    return SA_ERR_NULL;
  if (desc->batch < 1 || desc->heads_kv < 1 || desc->seqlen_q < 1 || desc->seqlen_k < 1 ||
      desc->block_q < 1 || desc->block_k < 1 || nnz < 0)
    return SA_ERR_SHAPE;
  sa::BsrRouteArgs a{};
  const int64_t nQB = ((int64_t)desc->seqlen_q + desc->block_q - 1) / desc->block_q;
  const int64_t nKB = ((int64_t)desc->seqlen_k + desc->block_k - 1) / desc->block_k;
  if (nKB > 32 * (int64_t)sa::kBsrMaxWords) return SA_ERR_UNSUPPORTED;
  a.nKB = (int)nKB;
  a.W = (a.nKB + 31) / 32;
  a.rows = (int64_t)desc->batch * desc->heads_kv * nQB;
  if (a.rows > INT32_MAX) return SA_ERR_SHAPE;
  a.indptr = block_indptr;
  a.indices = block_indices;
  a.nnz = nnz;
  a.n_exact = n_exact;
  a.exact_idx = exact_idx;
  a.proxy_keep = proxy_keep;
  a.bad_rows = bad_rows;
  return from_hip(sa::launch_bsr_route_prep(a, (hipStream_t)stream));
}

sa_status sa_proxy_block_sparse_fwd(const sa_attn_desc* desc, const void* q, const void* k,
                                    const void* v, const void* k_mean, const void* v_sum,
                                    const int32_t* n_exact, const int32_t* exact_idx,
                                    const uint32_t* proxy_keep, int32_t use_proxy, void* o,
                                    float* lse, void* stream) {
  sa_status st = check_attention(desc, q, k, v, o);
  if (st != SA_OK) return st;
  if (n_exact == nullptr || exact_idx == nullptr || proxy_keep == nullptr) return SA_ERR_NULL;
  if (use_proxy && (k_mean == nullptr || v_sum == nullptr)) return SA_ERR_NULL;
  if (desc->causal) return SA_ERR_UNSUPPORTED;
  if (desc->block_k != 64 && desc->block_k != 128) return SA_ERR_UNSUPPORTED;
  if (use_proxy && (!aligned16(k_mean) || !aligned16(v_sum))) return SA_ERR_ALIGN;
  sa::ProxyArgs a{};
  a.g = geometry(desc, q, k, v, o);
  a.k_mean = k_mean;
  a.v_sum = v_sum;
  a.n_exact = n_exact;
  a.exact_idx = exact_idx;
  a.proxy_keep = proxy_keep;
  a.use_proxy = use_proxy != 0;
  a.lse = lse;
  return from_hip(sa::launch_proxy(a, (hipStream_t)stream));
}

sa_status sa_threshold_from_calib(double a, double b, double target_sparsity, int64_t seq_k,
                                  double* scale_factor_out, float* lambda_out,
                                  float* log2_lambda_out) {
  if (!(a > 0.0) || !std::isfinite(a) || !std::isfinite(b) || !(target_sparsity >= 0.0) ||
      !(target_sparsity < 1.0) || seq_k < 1)
    return SA_ERR_VALUE;
  const double sf = a * std::exp(b * target_sparsity);
  const double lam = sf / (double)seq_k;
  const float lam32 = (float)lam;
  if (!std::isfinite(sf) || !std::isfinite(lam32) || !(lam32 > 0.f)) return SA_ERR_VALUE;
  if (scale_factor_out != nullptr) *scale_factor_out = sf;
  if (lambda_out != nullptr) *lambda_out = lam32;
  if (log2_lambda_out != nullptr) *log2_lambda_out = (float)std::log2((double)lam32);
  return SA_OK;
}

sa_status sa_skip_softmax_calibrate(const sa_attn_desc* desc, const void* q, const void* k,
                                    const void* v, void* o, const float* trial_lambdas,
                                    int32_t n_trials, uint32_t* head_counters,
                                    double* sparsities_out, void* stream) {
  if (trial_lambdas == nullptr || sparsities_out == nullptr || head_counters == nullptr)
    return SA_ERR_NULL;
  if (n_trials < 1) return SA_ERR_VALUE;
  for (int32_t i = 0; i < n_trials; ++i)
    if (!(trial_lambdas[i] >= 0.f) || !std::isfinite(trial_lambdas[i])) return SA_ERR_VALUE;
  sa_status st = check_attention(desc, q, k, v, o);
  if (st != SA_OK) return st;
  if (desc->block_k != 64 && desc->block_k != 128) return SA_ERR_UNSUPPORTED;
  const hipStream_t s = (hipStream_t)stream;
  const size_t n_heads = (size_t)desc->batch * desc->heads_q;
  std::vector<uint32_t> host(2 * n_heads);
  for (int32_t i = 0; i < n_trials; ++i) {
    if (hipMemsetAsync(head_counters, 0, host.size() * sizeof(uint32_t), s) != hipSuccess)
      return SA_ERR_HIP;
    st = sa_skip_softmax_fwd(desc, q, k, v, o, trial_lambdas[i], nullptr, head_counters, nullptr,
                             nullptr, stream);
    if (st != SA_OK) return st;
    if (hipMemcpyAsync(host.data(), head_counters, host.size() * sizeof(uint32_t),
                       hipMemcpyDeviceToHost, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
      return SA_ERR_HIP;
    uint64_t visited = 0, skipped = 0;
    for (size_t h = 0; h < n_heads; ++h) {
      visited += host[2 * h];
      skipped += host[2 * h + 1];
    }
    sparsities_out[i] = visited ? (double)skipped / (double)visited : 0.0;
  }
  return SA_OK;
}

sa_status sa_fit_threshold_calib(const double* trial_lambdas, const double* sparsities,
                                 int32_t n_trials, int64_t seq_k, double* a_out, double* b_out,
                                 double* min_sparsity_out, double* max_sparsity_out) {
  if (trial_lambdas == nullptr || sparsities == nullptr || a_out == nullptr || b_out == nullptr)
    return SA_ERR_NULL;
  if (n_trials < 0 || seq_k < 1) return SA_ERR_VALUE;
  // a trial tells where the curve lies only when some but not all tiles were skipped
  auto usable = [&](int32_t i) {
    return trial_lambdas[i] > 0.0 && std::isfinite(trial_lambdas[i]) && sparsities[i] > 0.0 &&
           sparsities[i] < 1.0;
  };
  int used = 0;
  double sx = 0.0, sy = 0.0, lo = INFINITY, hi = -INFINITY;
  for (int32_t i = 0; i < n_trials; ++i) {
    if (!usable(i)) continue;
    ++used;
    sx += sparsities[i];
    sy += std::log(trial_lambdas[i] * (double)seq_k);
    lo = std::fmin(lo, sparsities[i]);
    hi = std::fmax(hi, sparsities[i]);
  }
  if (used < 2 || !(hi > lo)) return SA_ERR_VALUE;
  const double mx = sx / used, my = sy / used;
  double cov = 0.0, var = 0.0;
  for (int32_t i = 0; i < n_trials; ++i) {
    if (!usable(i)) continue;
    const double dx = sparsities[i] - mx;
    cov += dx * (std::log(trial_lambdas[i] * (double)seq_k) - my);
    var += dx * dx;
  }
  const double b = cov / var, a = std::exp(my - b * mx);
  if (!std::isfinite(a) || !std::isfinite(b) || !(a > 0.0)) return SA_ERR_VALUE;
  *a_out = a;
  *b_out = b;
  if (min_sparsity_out != nullptr) *min_sparsity_out = lo;
  if (max_sparsity_out != nullptr) *max_sparsity_out = hi;
  return SA_OK;
}

}  // extern "C"
