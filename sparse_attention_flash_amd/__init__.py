"""Python binding of libsa_hip.so, the gfx950 sparse flash-attention forward library.

The functions here carry the C ABI's names (``include/sa.h``) and only marshal arguments: tensor
shapes and strides become an ``sa_attn_desc``, tensors become device pointers, and the current
torch stream becomes the ``hipStream_t``.  Every step of the computation runs in the HIP kernels of
``libsa_hip.so``; there is no fallback path.  Importing this package fails if the library has not
been built (``python sparse_attention_flash_amd/build.py``).

Tensors: Q/O ``[B, Sq, Hq, D]`` and K/V ``[B, Sk, Hkv, D]`` bf16 on the GPU with a unit stride on
D; optional outputs are preallocated by the caller with the shapes given in ``sa.h``.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_DIR = os.path.dirname(os.path.abspath(__file__))
# SA_HIP_LIB names another build of the same library (the host-sanitizer build, for instance).
LIB_PATH = os.environ.get("SA_HIP_LIB") or os.path.join(_DIR, "libsa_hip.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python sparse_attention_flash_amd/build.py`")

_lib = ctypes.CDLL(LIB_PATH)

SA_SKIP_GRAN_TILE, SA_SKIP_GRAN_WAVE = 0, 1
GRANULARITY = {"tile": SA_SKIP_GRAN_TILE, "wave": SA_SKIP_GRAN_WAVE}
WAVE_ROWS = 32   # decision rows at wave granularity

(SA_OK, SA_ERR_NULL, SA_ERR_SHAPE, SA_ERR_UNSUPPORTED, SA_ERR_ALIGN, SA_ERR_VALUE, SA_ERR_HIP,
 SA_ERR_SCRATCH) = range(8)
STATUS_NAMES = {0: "SA_OK", 1: "SA_ERR_NULL", 2: "SA_ERR_SHAPE", 3: "SA_ERR_UNSUPPORTED",
                4: "SA_ERR_ALIGN", 5: "SA_ERR_VALUE", 6: "SA_ERR_HIP", 7: "SA_ERR_SCRATCH"}
SA_DECODE_SCRATCH_BYTES = 32 << 20


class sa_attn_desc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads_q", ctypes.c_int32),
                ("heads_kv", ctypes.c_int32), ("seqlen_q", ctypes.c_int32),
                ("seqlen_k", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("causal", ctypes.c_int32), ("block_q", ctypes.c_int32),
                ("block_k", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
                ("q_stride", ctypes.c_int64 * 3), ("k_stride", ctypes.c_int64 * 3),
                ("v_stride", ctypes.c_int64 * 3), ("o_stride", ctypes.c_int64 * 3)]


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_F = ctypes.c_float
_D = ctypes.c_double
_DESC = ctypes.POINTER(sa_attn_desc)

_lib.sa_status_str.argtypes = [ctypes.c_int]
_lib.sa_status_str.restype = ctypes.c_char_p
_lib.sa_skip_softmax_fwd.argtypes = [_DESC, _P, _P, _P, _P, _F, _P, _P, _P, _P, _P]
_lib.sa_skip_softmax_fwd.restype = ctypes.c_int
_lib.sa_skip_softmax_fwd_ex.argtypes = [_DESC, _P, _P, _P, _P, _F, _I32, _P, _P, _P, _P, _P]
_lib.sa_skip_softmax_fwd_ex.restype = ctypes.c_int
_lib.sa_nm_softmax_fwd.argtypes = [_DESC, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _P, _P, _P, _P]
_lib.sa_nm_softmax_fwd.restype = ctypes.c_int
_lib.sa_skip_nm_softmax_fwd.argtypes = [_DESC, _P, _P, _P, _P, _F, _I32, _I32, _I32, _I32, _P, _P,
                                        _P, _P, _P, _P, _P]
_lib.sa_skip_nm_softmax_fwd.restype = ctypes.c_int
_lib.sa_skip_softmax_decode_workspace.argtypes = [_DESC, _F, _I32, _P, _P]
_lib.sa_skip_softmax_decode_workspace.restype = ctypes.c_int
_lib.sa_skip_softmax_decode_fwd.argtypes = [_DESC, _P, _P, _P, _P, _F, _P, _I32, _P, ctypes.c_size_t,
                                            _P, _P, _P, _P, _P]
_lib.sa_skip_softmax_decode_fwd.restype = ctypes.c_int
_lib.sa_skip_softmax_decode_fwd_noalloc.argtypes = [_DESC, _P, _P, _P, _P, _F, _P, _I32, _P, _P,
                                                    _P, _P, _P]
_lib.sa_skip_softmax_decode_fwd_noalloc.restype = ctypes.c_int
_lib.sa_bitmask_route_prep.argtypes = [_DESC, _P, _P, _P, _P, _P]
_lib.sa_bitmask_route_prep.restype = ctypes.c_int
_lib.sa_bsr_route_prep.argtypes = [_DESC, _P, _P, ctypes.c_int64, _P, _P, _P, _P, _P]
_lib.sa_bsr_route_prep.restype = ctypes.c_int
_lib.sa_proxy_block_sparse_fwd.argtypes = [_DESC, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _P, _P, _P]
_lib.sa_proxy_block_sparse_fwd.restype = ctypes.c_int
_lib.sa_threshold_from_calib.argtypes = [_D, _D, _D, ctypes.c_int64, _P, _P, _P]
_lib.sa_threshold_from_calib.restype = ctypes.c_int
_lib.sa_skip_softmax_calibrate.argtypes = [_DESC, _P, _P, _P, _P, _P, _I32, _P, _P, _P]
_lib.sa_skip_softmax_calibrate.restype = ctypes.c_int
_lib.sa_fit_threshold_calib.argtypes = [_P, _P, _I32, ctypes.c_int64, _P, _P, _P, _P]
_lib.sa_fit_threshold_calib.restype = ctypes.c_int

raw = _lib   # the ctypes handle, for callers that pass raw pointers


class SaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {sa_status_str(status)}")


def sa_status_str(status: int) -> str:
    return _lib.sa_status_str(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != SA_OK:
        raise SaError(status, where)


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError("tensor must live on the GPU")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _bsh_strides(t, name):
    if t.dim() != 4:
        raise ValueError(f"{name} must be [batch, seq, heads, head_dim]")
    if t.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be bfloat16")
    if t.stride(3) != 1:
        raise ValueError(f"{name} needs a unit stride on head_dim")
    return (t.stride(0), t.stride(1), t.stride(2))


_U8 = (torch.uint8,)
_U32 = (torch.int32, torch.uint32)
_F32 = (torch.float32,)


def _need(t, name, numel, dtypes):
    """An optional output or route buffer (None passes): a contiguous tensor of one of ``dtypes``
    with exactly ``numel`` elements, the size sa.h gives for it."""
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} must be {' or '.join(str(d) for d in dtypes)}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() != numel:
        raise ValueError(f"{name} must hold {numel} elements, got {t.numel()}")


def make_desc(q, k, v=None, o=None, *, causal=False, block_q=128, block_k=64, scale=None):
    """sa_attn_desc from tensor shapes/strides (v and o default to the strides of k and q).

    Checks that the tensors agree: v has k's shape, o has q's, and q, k share batch and
    head_dim."""
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q and k must be [batch, seq, heads, head_dim]")
    B, Sq, Hq, D = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    if k.shape[0] != B or k.shape[3] != D:
        raise ValueError(f"k {tuple(k.shape)} does not match q {tuple(q.shape)} in batch/head_dim")
    if v is not None and v.shape != k.shape:
        raise ValueError(f"v {tuple(v.shape)} must have k's shape {tuple(k.shape)}")
    if o is not None and o.shape != q.shape:
        raise ValueError(f"o {tuple(o.shape)} must have q's shape {tuple(q.shape)}")
    d = sa_attn_desc()
    d.batch, d.heads_q, d.heads_kv, d.seqlen_q, d.seqlen_k, d.head_dim = B, Hq, Hkv, Sq, Sk, D
    d.causal = int(bool(causal))
    d.block_q, d.block_k = int(block_q), int(block_k)
    d.softmax_scale = float(scale) if scale is not None else 1.0 / math.sqrt(D)
    qs = _bsh_strides(q, "q")
    ks = _bsh_strides(k, "k")
    vs = _bsh_strides(v, "v") if v is not None else ks
    os_ = _bsh_strides(o, "o") if o is not None else qs
    for i in range(3):
        d.q_stride[i], d.k_stride[i], d.v_stride[i], d.o_stride[i] = qs[i], ks[i], vs[i], os_[i]
    return d


def _skip_outputs(d, rows, tile_state, head_counters, lse, rowmax):
    """Sizes of the skip-softmax outputs for decision blocks of ``rows`` query rows."""
    if min(rows, d.block_k, d.seqlen_q, d.seqlen_k) < 1:
        return   # the library rejects the sizes themselves
    nR, nKT = -(-d.seqlen_q // rows), -(-d.seqlen_k // d.block_k)
    BH = d.batch * d.heads_q
    _need(tile_state, "tile_state", BH * nR * nKT, _U8)
    _need(head_counters, "head_counters", BH * 2, _U32)
    _need(lse, "lse", BH * d.seqlen_q, _F32)
    _need(rowmax, "dbg_tile_rowmax", BH * nR * nKT * rows, _F32)


def _nm_outputs(d, lse, keep_bits, scores):
    BH = d.batch * d.heads_q
    _need(lse, "lse", BH * d.seqlen_q, _F32)
    _need(keep_bits, "dbg_keep_bits", BH * d.seqlen_q * (-(-d.seqlen_k // 32)), _U32)
    _need(scores, "dbg_scores", BH * d.seqlen_q * d.seqlen_k, _F32)


def sa_skip_softmax_fwd(q, k, v, o, lam, *, causal=False, block_q=128, block_k=64, scale=None,
                        tile_state=None, head_counters=None, lse=None, dbg_tile_rowmax=None,
                        stream=None):
    d = make_desc(q, k, v, o, causal=causal, block_q=block_q, block_k=block_k, scale=scale)
    _skip_outputs(d, d.block_q, tile_state, head_counters, lse, dbg_tile_rowmax)
    _check(_lib.sa_skip_softmax_fwd(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                    float(lam), _ptr(tile_state), _ptr(head_counters), _ptr(lse),
                                    _ptr(dbg_tile_rowmax), _stream(stream)),
           "sa_skip_softmax_fwd")


def sa_skip_softmax_fwd_ex(q, k, v, o, lam, granularity="tile", *, causal=False, block_q=128,
                           block_k=64, scale=None, tile_state=None, head_counters=None, lse=None,
                           dbg_tile_rowmax=None, stream=None):
    """Skip-softmax with decisions per query tile ("tile") or per 32-row wavefront ("wave");
    tile_state / dbg_tile_rowmax are per decision block of rows (sa.h)."""
    gran = GRANULARITY[granularity] if isinstance(granularity, str) else int(granularity)
    d = make_desc(q, k, v, o, causal=causal, block_q=block_q, block_k=block_k, scale=scale)
    rows = WAVE_ROWS if gran == SA_SKIP_GRAN_WAVE else d.block_q
    _skip_outputs(d, rows, tile_state, head_counters, lse, dbg_tile_rowmax)
    _check(_lib.sa_skip_softmax_fwd_ex(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                       float(lam), gran, _ptr(tile_state), _ptr(head_counters),
                                       _ptr(lse), _ptr(dbg_tile_rowmax), _stream(stream)),
           "sa_skip_softmax_fwd_ex")


def sa_nm_softmax_fwd(q, k, v, o, n, m, dense_sink_tokens=0, dense_recent_tokens=0, *,
                      causal=False, block_q=128, block_k=64, scale=None, lse=None,
                      dbg_keep_bits=None, dbg_scores=None, stream=None):
    d = make_desc(q, k, v, o, causal=causal, block_q=block_q, block_k=block_k, scale=scale)
    _nm_outputs(d, lse, dbg_keep_bits, dbg_scores)
    _check(_lib.sa_nm_softmax_fwd(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(o), int(n),
                                  int(m), int(dense_sink_tokens), int(dense_recent_tokens),
                                  _ptr(lse), _ptr(dbg_keep_bits), _ptr(dbg_scores),
                                  _stream(stream)),
           "sa_nm_softmax_fwd")


def sa_skip_nm_softmax_fwd(q, k, v, o, lam, n, m, dense_sink_tokens=0, dense_recent_tokens=0, *,
                           causal=False, block_q=128, block_k=64, scale=None, tile_state=None,
                           head_counters=None, lse=None, dbg_tile_rowmax=None, dbg_keep_bits=None,
                           dbg_scores=None, stream=None):
    d = make_desc(q, k, v, o, causal=causal, block_q=block_q, block_k=block_k, scale=scale)
    _skip_outputs(d, d.block_q, tile_state, head_counters, None, dbg_tile_rowmax)
    _nm_outputs(d, lse, dbg_keep_bits, dbg_scores)
    _check(_lib.sa_skip_nm_softmax_fwd(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                       float(lam), int(n), int(m), int(dense_sink_tokens),
                                       int(dense_recent_tokens), _ptr(tile_state),
                                       _ptr(head_counters), _ptr(lse), _ptr(dbg_tile_rowmax),
                                       _ptr(dbg_keep_bits), _ptr(dbg_scores), _stream(stream)),
           "sa_skip_nm_softmax_fwd")


def sa_skip_softmax_decode_workspace(q, k, lam, *, block_k=64, num_splits=0, scale=None):
    """(workspace bytes, splits used) for a decode call with these shapes."""
    d = make_desc(q, k, block_q=64, block_k=block_k, scale=scale)
    nbytes, used = ctypes.c_size_t(), ctypes.c_int32()
    _check(_lib.sa_skip_softmax_decode_workspace(ctypes.byref(d), float(lam), int(num_splits),
                                                 ctypes.addressof(nbytes), ctypes.addressof(used)),
           "sa_skip_softmax_decode_workspace")
    return nbytes.value, used.value


def sa_skip_softmax_decode_fwd(q, k, v, o, lam, *, block_k=64, seqlens_k=None, num_splits=0,
                               workspace=None, scale=None, tile_state=None, head_counters=None,
                               lse=None, dbg_tile_rowmax=None, stream=None):
    """q, o [B, 1, Hq, D]; k, v [B, Sk, Hkv, D].  Without a workspace one is allocated."""
    d = make_desc(q, k, v, o, block_q=64, block_k=block_k, scale=scale)
    BH, nKT = d.batch * d.heads_q, -(-d.seqlen_k // max(1, d.block_k))
    _need(seqlens_k, "seqlens_k", d.batch, (torch.int32,))
    _need(tile_state, "tile_state", BH * nKT, _U8)
    _need(head_counters, "head_counters", BH * 2, _U32)
    _need(lse, "lse", BH, _F32)
    _need(dbg_tile_rowmax, "dbg_tile_rowmax", BH * nKT, _F32)
    if workspace is not None and not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    if workspace is None:
        nbytes, _ = sa_skip_softmax_decode_workspace(q, k, lam, block_k=block_k,
                                                     num_splits=num_splits, scale=scale)
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    _check(_lib.sa_skip_softmax_decode_fwd(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                           float(lam), _ptr(seqlens_k), int(num_splits),
                                           _ptr(workspace), workspace.numel() * workspace.element_size(),
                                           _ptr(tile_state), _ptr(head_counters), _ptr(lse),
                                           _ptr(dbg_tile_rowmax), _stream(stream)),
           "sa_skip_softmax_decode_fwd")


def _nkb(d):
    return -(-d.seqlen_k // d.block_k)


def _route_rows(d):
    return d.batch * d.heads_kv * (-(-d.seqlen_q // d.block_q))


def _sizes_ok(d):
    return min(d.batch, d.heads_kv, d.seqlen_q, d.seqlen_k, d.block_q, d.block_k) >= 1


def _route_outputs(d, n_exact, exact_idx, proxy_keep):
    for t, name in ((n_exact, "n_exact"), (exact_idx, "exact_idx"), (proxy_keep, "proxy_keep")):
        if t is None:
            raise ValueError(f"{name} is required")
    if not _sizes_ok(d):
        return   # the library rejects the sizes themselves
    rows, nKB = _route_rows(d), _nkb(d)
    _need(n_exact, "n_exact", rows, _U32)
    _need(exact_idx, "exact_idx", rows * nKB, _U32)
    _need(proxy_keep, "proxy_keep", rows * (-(-nKB // 32)), _U32)


def sa_skip_softmax_decode_fwd_noalloc(q, k, v, o, lam, *, block_k=64, seqlens_k=None,
                                       num_splits=0, scale=None, tile_state=None,
                                       head_counters=None, lse=None, dbg_tile_rowmax=None,
                                       stream=None):
    """sa_skip_softmax_decode_fwd with its workspace in the library's fixed device array (no
    allocation anywhere; calls that overlap on one GPU race, see sa.h)."""
    d = make_desc(q, k, v, o, block_q=64, block_k=block_k, scale=scale)
    BH, nKT = d.batch * d.heads_q, -(-d.seqlen_k // max(1, d.block_k))
    _need(seqlens_k, "seqlens_k", d.batch, (torch.int32,))
    _need(tile_state, "tile_state", BH * nKT, _U8)
    _need(head_counters, "head_counters", BH * 2, _U32)
    _need(lse, "lse", BH, _F32)
    _need(dbg_tile_rowmax, "dbg_tile_rowmax", BH * nKT, _F32)
    _check(_lib.sa_skip_softmax_decode_fwd_noalloc(
        ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(o), float(lam), _ptr(seqlens_k),
        int(num_splits), _ptr(tile_state), _ptr(head_counters), _ptr(lse), _ptr(dbg_tile_rowmax),
        _stream(stream)), "sa_skip_softmax_decode_fwd_noalloc")


def sa_bitmask_route_prep(bitmask, n_exact, exact_idx, proxy_keep, *, batch, heads_kv, seqlen_q,
                          seqlen_k, block_q, block_k, stream=None):
    d = sa_attn_desc()
    d.batch, d.heads_kv, d.heads_q = batch, heads_kv, heads_kv
    d.seqlen_q, d.seqlen_k, d.block_q, d.block_k = seqlen_q, seqlen_k, block_q, block_k
    _route_outputs(d, n_exact, exact_idx, proxy_keep)
    if _sizes_ok(d):
        _need(bitmask, "bitmask", _route_rows(d) * (-(-_nkb(d) // 32)), _U32)
    _check(_lib.sa_bitmask_route_prep(ctypes.byref(d), _ptr(bitmask), _ptr(n_exact),
                                      _ptr(exact_idx), _ptr(proxy_keep), _stream(stream)),
           "sa_bitmask_route_prep")


def sa_bsr_route_prep(block_indptr, block_indices, n_exact, exact_idx, proxy_keep, *, batch,
                      heads_kv, seqlen_q, seqlen_k, block_q, block_k, bad_rows=None, stream=None):
    d = sa_attn_desc()
    d.batch, d.heads_kv, d.heads_q = batch, heads_kv, heads_kv
    d.seqlen_q, d.seqlen_k, d.block_q, d.block_k = seqlen_q, seqlen_k, block_q, block_k
    _route_outputs(d, n_exact, exact_idx, proxy_keep)
    if _sizes_ok(d):
        _need(block_indptr, "block_indptr", _route_rows(d) + 1, (torch.int32,))
    _need(block_indices, "block_indices", block_indices.numel(), (torch.int32,))
    _need(bad_rows, "bad_rows", 1, _U32)
    nnz = block_indices.numel()
    _check(_lib.sa_bsr_route_prep(ctypes.byref(d), _ptr(block_indptr),
                                  _ptr(block_indices) if nnz else None, nnz, _ptr(n_exact),
                                  _ptr(exact_idx), _ptr(proxy_keep), _ptr(bad_rows),
                                  _stream(stream)),
           "sa_bsr_route_prep")


def sa_proxy_block_sparse_fwd(q, k, v, k_mean, v_sum, n_exact, exact_idx, proxy_keep, use_proxy,
                              o, *, block_q=128, block_k=128, scale=None, lse=None, stream=None):
    d = make_desc(q, k, v, o, causal=False, block_q=block_q, block_k=block_k, scale=scale)
    if _sizes_ok(d):
        summ = d.batch * d.heads_kv * _nkb(d) * d.head_dim
        _need(k_mean, "k_mean", summ, (torch.bfloat16,))
        _need(v_sum, "v_sum", summ, (torch.bfloat16,))
    _route_outputs(d, n_exact, exact_idx, proxy_keep)
    _need(lse, "lse", d.batch * d.heads_q * d.seqlen_q, _F32)
    _check(_lib.sa_proxy_block_sparse_fwd(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v),
                                          _ptr(k_mean), _ptr(v_sum), _ptr(n_exact),
                                          _ptr(exact_idx), _ptr(proxy_keep), int(use_proxy),
                                          _ptr(o), _ptr(lse), _stream(stream)),
           "sa_proxy_block_sparse_fwd")


def sa_threshold_from_calib(a, b, target_sparsity, seq_k):
    """(scale_factor, lambda, log2_lambda) with lambda and log2_lambda as the kernel sees them."""
    sf, lam, l2 = ctypes.c_double(), ctypes.c_float(), ctypes.c_float()
    _check(_lib.sa_threshold_from_calib(float(a), float(b), float(target_sparsity), int(seq_k),
                                        ctypes.addressof(sf), ctypes.addressof(lam),
                                        ctypes.addressof(l2)),
           "sa_threshold_from_calib")
    return sf.value, lam.value, l2.value


def sa_skip_softmax_calibrate(q, k, v, o, trial_lambdas, head_counters, *, causal=False,
                              block_q=128, block_k=64, scale=None, stream=None):
    """Tile sparsity of each trial threshold (a list of floats); blocks until done."""
    d = make_desc(q, k, v, o, causal=causal, block_q=block_q, block_k=block_k, scale=scale)
    _need(head_counters, "head_counters", d.batch * d.heads_q * 2, _U32)
    trials = (ctypes.c_float * len(trial_lambdas))(*map(float, trial_lambdas))
    out = (ctypes.c_double * len(trial_lambdas))()
    _check(_lib.sa_skip_softmax_calibrate(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                          ctypes.addressof(trials), len(trial_lambdas),
                                          _ptr(head_counters), ctypes.addressof(out),
                                          _stream(stream)),
           "sa_skip_softmax_calibrate")
    return list(out)


def sa_fit_threshold_calib(trial_lambdas, sparsities, seq_k):
    """(a, b, min_sparsity, max_sparsity) of the log-space fit."""
    n = len(trial_lambdas)
    if len(sparsities) != n:
        raise ValueError("one sparsity per trial")
    lam = (ctypes.c_double * n)(*map(float, trial_lambdas))
    sp = (ctypes.c_double * n)(*map(float, sparsities))
    out = [ctypes.c_double() for _ in range(4)]
    _check(_lib.sa_fit_threshold_calib(ctypes.addressof(lam), ctypes.addressof(sp), n, int(seq_k),
                                       *[ctypes.addressof(o) for o in out]),
           "sa_fit_threshold_calib")
    return tuple(o.value for o in out)


def tile_counts(seqlen_q, seqlen_k, block_q, block_k):
    """(nQT, nKT) tile counts for a call."""
    return -(-seqlen_q // block_q), -(-seqlen_k // block_k)
