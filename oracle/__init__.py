"""CPU oracle for the sparse flash-attention forward paths (test infrastructure only).

Only the tests, the package smoke check and the benchmark's CPU-baseline leg may import this
module.  It wraps ``sa_oracle.c`` (plain C, double-precision accumulation, OpenMP over independent
units) through ctypes; it imports nothing from the HIP package and shares no code with it.  Inputs
are contiguous bf16 bit patterns (numpy ``uint16``) in the layout ``[B, S, H, D]``.

Each wrapper returns results in natural layouts:

* ``skip_softmax``: ``o [B,Sq,Hq,D]`` (float64), ``lse [B,Hq,Sq]``, ``tile_state [B,Hq,nQT,nKT]``
  (0 kept, 1 skipped, 2 not visited), ``rowmax [B,Hq,nQT,nKT,Br]`` (log2 domain, float64).
* ``nm_softmax``: ``o``, ``lse``, ``keep_bits [B,Hq,Sq,ceil(Sk/32)]`` (uint32, LSB first).
* ``skip_nm_softmax``: ``o``, ``lse``, ``tile_state``, ``rowmax`` as skip_softmax, plus
  ``keep_bits`` as nm_softmax.
* ``skip_softmax_wave``: skip_softmax with every 32-row block deciding alone (block_q = 32).
* ``skip_replay``: ``tile_state`` alone, replayed from given fp32 tile maxima (no dot products).
* ``nm_keep_replay``: N:M keep bits alone, replayed from given fp32 scores (no dot products).
* ``route_prep``: ``n_exact``, ``exact_idx`` (ascending, -1 padded), ``proxy_keep``.
* ``bsr_route_prep``: the same triple from BSR rows, plus the count of non-canonical rows.
* ``proxy_fwd``: ``o``, ``lse``.
* ``threshold``: ``(scale_factor, lambda, log2_lambda)`` as Python floats.
* ``fit_threshold``: ``(a, b, s_min, s_max)`` of the log-space calibration fit.

When ``units`` (linear (b, hq, query-tile) indices) is given, only those units are computed and
the results come back per unit: ``o [n, Br, D]``, ``lse [n, Br]``, ``tile_state [n, nKT]`` ...
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_DIR = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_DIR, "sa_oracle.c")
_DEFAULT_LIB = os.path.join(_DIR, "libsa_oracle.so")
# SA_ORACLE_LIB names another build of the oracle (the sanitizer build, for instance).
_LIB_PATH = os.environ.get("SA_ORACLE_LIB") or _DEFAULT_LIB
_lib = None

GCC_FLAGS = ["-O2", "-std=gnu11", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
             "-fno-fast-math", "-Wall", "-Wextra"]

# AddressSanitizer + UndefinedBehaviorSanitizer build with ROCm's clang, whose shared ASan runtime
# the HIP library's sanitizer build uses too (one runtime per process).
SAN_LIB = os.path.join(_DIR, "libsa_oracle_san.so")
CLANG = "/opt/rocm/llvm/bin/clang"
SAN_FLAGS = ["-O1", "-g", "-std=gnu11", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
             "-fno-fast-math", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
             "-shared-libasan", "-Wl,-rpath,/opt/rocm/llvm/lib"]


def build(force: bool = False, sanitize: bool = False) -> str:
    """Compile sa_oracle.c into libsa_oracle.so with gcc (host code only); with sanitize=True into
    libsa_oracle_san.so with clang and ASan/UBSan."""
    out = SAN_LIB if sanitize else _LIB_PATH
    sanitize = out == SAN_LIB
    if force or not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(_SRC):
        if out not in (_DEFAULT_LIB, SAN_LIB):
            raise RuntimeError(f"{out} (SA_ORACLE_LIB) is missing or older than {_SRC}")
        tmp = out + f".tmp{os.getpid()}"
        cmd = [CLANG, *SAN_FLAGS] if sanitize else ["gcc", *GCC_FLAGS]
        subprocess.run([*cmd, _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, out)
    return out


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        I = ctypes.c_int
        D = ctypes.c_double
        I64 = ctypes.c_int64
        lib.oracle_num_threads.restype = I
        lib.oracle_skip_softmax.argtypes = [I] * 9 + [D, D, P, P, P, I, P, P, P, I64, P, P, P, P]
        lib.oracle_skip_softmax.restype = I
        lib.oracle_nm_softmax.argtypes = [I] * 8 + [D, I, I, I, I, P, P, P, I, P, P, P, I64, P, P, P]
        lib.oracle_nm_softmax.restype = I
        lib.oracle_skip_nm_softmax.argtypes = ([I] * 9 + [D, D] + [I] * 4 + [P, P, P, I] +
                                               [P] * 5 + [I64] + [P] * 5)
        lib.oracle_skip_nm_softmax.restype = I
        lib.oracle_skip_replay.argtypes = [I] * 7 + [D, P, I64, P, P]
        lib.oracle_skip_replay.restype = I
        lib.oracle_nm_keep_replay.argtypes = [I] * 7 + [P, I64, P, P]
        lib.oracle_nm_keep_replay.restype = I
        lib.oracle_route_prep.argtypes = [I64, I, P, P, P, P]
        lib.oracle_route_prep.restype = I
        lib.oracle_bsr_route_prep.argtypes = [I64, I, P, I64, P, P, P, P, P]
        lib.oracle_bsr_route_prep.restype = I
        lib.oracle_proxy_fwd.argtypes = [I] * 8 + [D, P, P, P, P, P, P, I, P, I64, P, P]
        lib.oracle_proxy_fwd.restype = I
        lib.oracle_threshold.argtypes = [D, D, D, I64, P, P, P]
        lib.oracle_threshold.restype = I
        lib.oracle_fit_threshold.argtypes = [I, P, P, I64, P, P, P, P]
        lib.oracle_fit_threshold.restype = I
        _lib = lib
    return _lib


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _bf16(a, name):
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError(f"{name} must hold bf16 bit patterns as uint16, got {a.dtype}")
    return a


def _units(units, total):
    if units is None:
        return None, total
    u = np.ascontiguousarray(np.asarray(units, dtype=np.int64))
    return u, int(u.size)


def skip_softmax(q, k, v, *, causal, block_q, block_k, scale, lam, mode=0, rowmax_in=None,
                 state_in=None, units=None):
    q, k, v = _bf16(q, "q"), _bf16(k, "k"), _bf16(v, "v")
    B, Sq, Hq, D = q.shape
    _, Sk, Hkv, _ = k.shape
    nQT, nKT = -(-Sq // block_q), -(-Sk // block_k)
    u, n = _units(units, B * Hq * nQT)
    if mode == 1:
        rowmax_in = np.ascontiguousarray(rowmax_in, dtype=np.float32)
        assert rowmax_in.size == B * Hq * nQT * nKT * block_q
    if mode == 2:
        state_in = np.ascontiguousarray(state_in, dtype=np.uint8)
        assert state_in.size == B * Hq * nQT * nKT
    o = np.zeros((n, block_q, D))
    lse = np.zeros((n, block_q))
    st = np.zeros((n, nKT), np.uint8)
    rm = np.zeros((n, nKT, block_q))
    rc = _load().oracle_skip_softmax(B, Hq, Hkv, Sq, Sk, D, int(causal), block_q, block_k,
                                     float(scale), float(lam), _ptr(q), _ptr(k), _ptr(v), int(mode),
                                     _ptr(rowmax_in), _ptr(state_in), _ptr(u), n, _ptr(o),
                                     _ptr(lse), _ptr(st), _ptr(rm))
    if rc:
        raise ValueError("oracle_skip_softmax rejected its arguments")
    if units is not None:
        return o, lse, st, rm
    o = o.reshape(B, Hq, nQT * block_q, D)[:, :, :Sq].transpose(0, 2, 1, 3)
    lse = lse.reshape(B, Hq, nQT * block_q)[:, :, :Sq]
    return (np.ascontiguousarray(o), np.ascontiguousarray(lse), st.reshape(B, Hq, nQT, nKT),
            rm.reshape(B, Hq, nQT, nKT, block_q))


def nm_softmax(q, k, v, *, causal, scale, n, m, sink, recent, block_q=64, mode=0, scores_in=None,
               keep_in=None, units=None):
    q, k, v = _bf16(q, "q"), _bf16(k, "k"), _bf16(v, "v")
    B, Sq, Hq, D = q.shape
    _, Sk, Hkv, _ = k.shape
    nQT, W = -(-Sq // block_q), -(-Sk // 32)
    u, cnt = _units(units, B * Hq * nQT)
    if mode == 1:
        scores_in = np.ascontiguousarray(scores_in, dtype=np.float32)
        assert scores_in.size == B * Hq * Sq * Sk
    if mode == 2:
        keep_in = np.ascontiguousarray(keep_in, dtype=np.uint32)
        assert keep_in.size == B * Hq * Sq * W
    o = np.zeros((cnt, block_q, D))
    lse = np.zeros((cnt, block_q))
    kb = np.zeros((cnt, block_q, W), np.uint32)
    rc = _load().oracle_nm_softmax(B, Hq, Hkv, Sq, Sk, D, int(causal), block_q, float(scale),
                                   int(n), int(m), int(sink), int(recent), _ptr(q), _ptr(k),
                                   _ptr(v), int(mode), _ptr(scores_in), _ptr(keep_in), _ptr(u),
                                   cnt, _ptr(o), _ptr(lse), _ptr(kb))
    if rc:
        raise ValueError("oracle_nm_softmax rejected its arguments")
    if units is not None:
        return o, lse, kb
    o = o.reshape(B, Hq, nQT * block_q, D)[:, :, :Sq].transpose(0, 2, 1, 3)
    lse = lse.reshape(B, Hq, nQT * block_q)[:, :, :Sq]
    kb = kb.reshape(B, Hq, nQT * block_q, W)[:, :, :Sq]
    return np.ascontiguousarray(o), np.ascontiguousarray(lse), np.ascontiguousarray(kb)


def skip_nm_softmax(q, k, v, *, causal, block_q, block_k, scale, lam, n, m, sink, recent, mode=0,
                    rowmax_in=None, state_in=None, scores_in=None, keep_in=None, units=None):
    q, k, v = _bf16(q, "q"), _bf16(k, "k"), _bf16(v, "v")
    B, Sq, Hq, D = q.shape
    _, Sk, Hkv, _ = k.shape
    nQT, nKT, W = -(-Sq // block_q), -(-Sk // block_k), -(-Sk // 32)
    u, cnt = _units(units, B * Hq * nQT)
    if mode == 1:
        rowmax_in = np.ascontiguousarray(rowmax_in, dtype=np.float32)
        assert rowmax_in.size == B * Hq * nQT * nKT * block_q
        scores_in = np.ascontiguousarray(scores_in, dtype=np.float32)
        assert scores_in.size == B * Hq * Sq * Sk
    if mode == 2:
        state_in = np.ascontiguousarray(state_in, dtype=np.uint8)
        assert state_in.size == B * Hq * nQT * nKT
        keep_in = np.ascontiguousarray(keep_in, dtype=np.uint32)
        assert keep_in.size == B * Hq * Sq * W
    o = np.zeros((cnt, block_q, D))
    lse = np.zeros((cnt, block_q))
    st = np.zeros((cnt, nKT), np.uint8)
    rm = np.zeros((cnt, nKT, block_q))
    kb = np.zeros((cnt, block_q, W), np.uint32)
    rc = _load().oracle_skip_nm_softmax(
        B, Hq, Hkv, Sq, Sk, D, int(causal), block_q, block_k, float(scale), float(lam), int(n),
        int(m), int(sink), int(recent), _ptr(q), _ptr(k), _ptr(v), int(mode), _ptr(rowmax_in),
        _ptr(state_in), _ptr(scores_in), _ptr(keep_in), _ptr(u), cnt, _ptr(o), _ptr(lse), _ptr(st),
        _ptr(rm), _ptr(kb))
    if rc:
        raise ValueError("oracle_skip_nm_softmax rejected its arguments")
    if units is not None:
        return o, lse, st, rm, kb
    o = o.reshape(B, Hq, nQT * block_q, D)[:, :, :Sq].transpose(0, 2, 1, 3)
    lse = lse.reshape(B, Hq, nQT * block_q)[:, :, :Sq]
    kb = kb.reshape(B, Hq, nQT * block_q, W)[:, :, :Sq]
    return (np.ascontiguousarray(o), np.ascontiguousarray(lse), st.reshape(B, Hq, nQT, nKT),
            rm.reshape(B, Hq, nQT, nKT, block_q), np.ascontiguousarray(kb))


def skip_softmax_wave(q, k, v, *, causal, block_k, scale, lam, mode=0, rowmax_in=None,
                      state_in=None, units=None):
    """Skip-softmax at wave granularity: every block of 32 query rows decides on its own, with its
    own running max -- by definition the tile rule on 32-row query tiles (the reading of a
    per-wave decision; the HuggingFace attention-sparsity page's "Custom Configuration" sets the
    br x bc decision block).  Same outputs as skip_softmax with block_q = 32."""
    return skip_softmax(q, k, v, causal=causal, block_q=32, block_k=block_k, scale=scale, lam=lam,
                        mode=mode, rowmax_in=rowmax_in, state_in=state_in, units=units)


def skip_replay(rowmax, *, batch, heads_q, seqlen_q, seqlen_k, causal, block_q, block_k, lam,
                units=None):
    """Skip decisions alone, replayed from fp32 tile maxima (no attention arithmetic).

    ``rowmax`` holds the listed units' maxima, ``[n_units, nKT, block_q]`` float32 (all units in
    order when ``units`` is None); returns ``tile_state [n_units, nKT]`` (0 kept, 1 skipped,
    2 not visited)."""
    nQT, nKT = -(-seqlen_q // block_q), -(-seqlen_k // block_k)
    u, n = _units(units, batch * heads_q * nQT)
    rm = np.ascontiguousarray(rowmax, dtype=np.float32)
    assert rm.size == n * nKT * block_q, (rm.shape, n, nKT, block_q)
    st = np.zeros((n, nKT), np.uint8)
    rc = _load().oracle_skip_replay(batch, heads_q, seqlen_q, seqlen_k, int(causal), block_q,
                                    block_k, float(lam), _ptr(u), n, _ptr(rm), _ptr(st))
    if rc:
        raise ValueError("oracle_skip_replay rejected its arguments")
    return st


def nm_keep_replay(scores, row_pos, *, seqlen_q, causal, n, m, sink, recent):
    """N:M keep bits alone, replayed from fp32 score rows ``[n_rows, Sk]`` whose query positions
    are ``row_pos``; returns ``keep [n_rows, ceil(Sk/32)]`` uint32 (LSB first)."""
    sc = np.ascontiguousarray(scores, dtype=np.float32)
    rp = np.ascontiguousarray(np.asarray(row_pos, dtype=np.int32)).ravel()
    n_rows, Sk = sc.shape
    assert rp.size == n_rows
    keep = np.zeros((n_rows, -(-Sk // 32)), np.uint32)
    rc = _load().oracle_nm_keep_replay(int(seqlen_q), Sk, int(causal), int(n), int(m), int(sink),
                                       int(recent), _ptr(rp), n_rows, _ptr(sc), _ptr(keep))
    if rc:
        raise ValueError("oracle_nm_keep_replay rejected its arguments")
    return keep


def route_prep(bitmask, n_kv_blocks):
    bm = np.ascontiguousarray(bitmask, dtype=np.uint32)
    W = -(-n_kv_blocks // 32)
    assert bm.shape[-1] == W
    lead = bm.shape[:-1]
    rows = int(np.prod(lead)) if lead else 1
    n_exact = np.zeros(rows, np.int32)
    idx = np.zeros((rows, n_kv_blocks), np.int32)
    keep = np.zeros((rows, W), np.uint32)
    rc = _load().oracle_route_prep(rows, n_kv_blocks, _ptr(bm), _ptr(n_exact), _ptr(idx),
                                   _ptr(keep))
    if rc:
        raise ValueError("oracle_route_prep rejected its arguments")
    return (n_exact.reshape(lead), idx.reshape(*lead, n_kv_blocks), keep.reshape(*lead, W))


def bsr_route_prep(indptr, indices, n_kv_blocks):
    """Route stream from BSR rows (indptr of rows+1 entries, indices); returns the route_prep
    triple plus the number of non-canonical rows."""
    ip = np.ascontiguousarray(indptr, dtype=np.int32).ravel()
    ix = np.ascontiguousarray(indices, dtype=np.int32).ravel()
    rows = ip.size - 1
    W = -(-n_kv_blocks // 32)
    n_exact = np.zeros(rows, np.int32)
    idx = np.zeros((rows, n_kv_blocks), np.int32)
    keep = np.zeros((rows, W), np.uint32)
    bad = np.zeros(1, np.int64)
    rc = _load().oracle_bsr_route_prep(rows, n_kv_blocks, _ptr(ip), ix.size, _ptr(ix),
                                       _ptr(n_exact), _ptr(idx), _ptr(keep), _ptr(bad))
    if rc:
        raise ValueError("oracle_bsr_route_prep rejected its arguments")
    return n_exact, idx, keep, int(bad[0])


def proxy_fwd(q, k, v, k_mean, v_sum, bitmask, *, block_q, block_k, scale, use_proxy,
              units=None):
    q, k, v = _bf16(q, "q"), _bf16(k, "k"), _bf16(v, "v")
    km, vs = _bf16(k_mean, "k_mean"), _bf16(v_sum, "v_sum")
    B, Sq, Hq, D = q.shape
    _, Sk, Hkv, _ = k.shape
    nQB, nKB = -(-Sq // block_q), -(-Sk // block_k)
    W = -(-nKB // 32)
    bm = np.ascontiguousarray(bitmask, dtype=np.uint32)
    assert bm.shape == (B, Hkv, nQB, W), bm.shape
    assert km.shape == (B, Hkv, nKB, D) and vs.shape == (B, Hkv, nKB, D)
    u, cnt = _units(units, B * Hq * nQB)
    o = np.zeros((cnt, block_q, D))
    lse = np.zeros((cnt, block_q))
    rc = _load().oracle_proxy_fwd(B, Hq, Hkv, Sq, Sk, D, block_q, block_k, float(scale), _ptr(q),
                                  _ptr(k), _ptr(v), _ptr(km), _ptr(vs), _ptr(bm), int(use_proxy),
                                  _ptr(u), cnt, _ptr(o), _ptr(lse))
    if rc:
        raise ValueError("oracle_proxy_fwd rejected its arguments")
    if units is not None:
        return o, lse
    o = o.reshape(B, Hq, nQB * block_q, D)[:, :, :Sq].transpose(0, 2, 1, 3)
    lse = lse.reshape(B, Hq, nQB * block_q)[:, :, :Sq]
    return np.ascontiguousarray(o), np.ascontiguousarray(lse)


def threshold(a, b, target_sparsity, seq_k):
    sf, lam, l2 = ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
    rc = _load().oracle_threshold(float(a), float(b), float(target_sparsity), int(seq_k),
                                  ctypes.addressof(sf), ctypes.addressof(lam),
                                  ctypes.addressof(l2))
    if rc:
        raise ValueError("oracle_threshold rejected its arguments")
    return sf.value, lam.value, l2.value


def fit_threshold(lambdas, sparsities, seq_k):
    lam = np.ascontiguousarray(lambdas, dtype=np.float64)
    sp = np.ascontiguousarray(sparsities, dtype=np.float64)
    assert lam.shape == sp.shape
    out = [ctypes.c_double() for _ in range(4)]
    rc = _load().oracle_fit_threshold(lam.size, _ptr(lam), _ptr(sp), int(seq_k),
                                      *[ctypes.addressof(o) for o in out])
    if rc:
        raise ValueError("oracle_fit_threshold: fewer than two usable trials")
    return tuple(o.value for o in out)
