// api.hip -- the extern "C" entry points of libsa_hip.so (declared and documented in sa.h).
//
// Every argument check runs here, on the host, before any HIP call: a rejected call enqueues and
// writes nothing, which also lets the checks be exercised on a machine without a GPU.  Accepted
// calls are lowered into the plain launch structs of kernels.h (the user-facing description is
// not passed to the kernels) and enqueued on the caller's stream.
#include <cmath>
#include <cstdint>

#include "kernels.h"
#include "sa.h"

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
  }
  return "unknown sa_status";
}

sa_status sa_skip_softmax_fwd(const sa_attn_desc* desc, const void* q, const void* k,
                              const void* v, void* o, float lambda, uint8_t* tile_state,
                              uint32_t* head_counters, float* lse, float* dbg_tile_rowmax,
                              void* stream) {
  sa_status st = check_attention(desc, q, k, v, o);
  if (st != SA_OK) return st;
  if (desc->block_k != 64) return SA_ERR_UNSUPPORTED;
  if (!(lambda >= 0.f) || !std::isfinite(lambda)) return SA_ERR_VALUE;
  sa::SkipArgs a{};
  a.g = geometry(desc, q, k, v, o);
  a.L32 = lambda == 0.f ? -INFINITY : (float)std::log2((double)lambda);
  a.tile_state = tile_state;
  a.counters = head_counters;
  a.lse = lse;
  a.rowmax = dbg_tile_rowmax;
  return from_hip(sa::launch_skip_softmax(a, (hipStream_t)stream));
}

sa_status sa_nm_softmax_fwd(const sa_attn_desc* desc, const void* q, const void* k,
                            const void* v, void* o, int32_t n, int32_t m,
                            int32_t dense_sink_tokens, int32_t dense_recent_tokens, float* lse,
                            uint32_t* dbg_keep_bits, float* dbg_scores, void* stream) {
  sa_status st = check_attention(desc, q, k, v, o);
  if (st != SA_OK) return st;
  if (desc->block_k != 64) return SA_ERR_UNSUPPORTED;
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

}  // extern "C"
