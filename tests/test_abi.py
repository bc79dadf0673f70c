"""C-ABI checks that need no GPU: the library loads, exports every entry point sa.h declares, and
rejects every invalid call on the host before any HIP call (all calls here are invalid, so no
kernel is ever launched; the pointers are dummies)."""
import ctypes
import math
import os
import re

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

sa = pytest.importorskip("sparse_attention_flash_amd")

FAKE = 0x10000          # 16-byte aligned dummy address, never dereferenced
FAKE_MIS = 0x10008      # misaligned dummy address


def declared_entry_points(header="sa.h"):
    text = open(os.path.join(ROOT, "include", header)).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sa_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = declared_entry_points()
    assert {"sa_skip_softmax_fwd", "sa_nm_softmax_fwd", "sa_skip_nm_softmax_fwd",
            "sa_bitmask_route_prep", "sa_bsr_route_prep", "sa_skip_softmax_calibrate",
            "sa_fit_threshold_calib", "sa_skip_softmax_decode_workspace",
            "sa_skip_softmax_decode_fwd",
            "sa_proxy_block_sparse_fwd", "sa_threshold_from_calib", "sa_status_str"} <= set(names)
    lib = ctypes.CDLL(sa.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_probe_library_exports_its_header_and_rejects_bad_arguments():
    """libsa_probes.so (the peak-rate microbenchmarks bench.py --peak-probes runs) exports what
    sa_probes.h declares, and rejects bad arguments on the host before any launch."""
    names = declared_entry_points("sa_probes.h")
    assert names == ["sa_probe_mfma_bf16", "sa_probe_mfma_bf16_flops", "sa_probe_read"]
    lib = ctypes.CDLL(os.path.join(ROOT, "sparse_attention_flash_amd", "libsa_probes.so"))
    for n in names:
        assert hasattr(lib, n), n
    lib.sa_probe_mfma_bf16_flops.restype = ctypes.c_double
    assert lib.sa_probe_mfma_bf16_flops(3, 5) == 3 * 4 * 5 * 4 * 32768
    V, I, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.sa_probe_mfma_bf16.argtypes = [V, I, I, I, V]
    lib.sa_probe_read.argtypes = [V, Z, V, I, V]
    assert lib.sa_probe_mfma_bf16(None, 1, 1, 1, None) == 1
    assert lib.sa_probe_mfma_bf16(FAKE, 0, 1, 1, None) == 1
    assert lib.sa_probe_mfma_bf16(FAKE, 1, 0, 0, None) == 1
    assert lib.sa_probe_read(FAKE, 16384 + 16, FAKE, 1, None) == 1    # not whole chunks
    assert lib.sa_probe_read(FAKE, 0, FAKE, 1, None) == 1
    assert lib.sa_probe_read(FAKE_MIS, 16384, FAKE, 1, None) == 1     # misaligned
    assert lib.sa_probe_read(FAKE, 16384, FAKE, 0, None) == 1


def test_status_strings():
    for code in range(8):
        assert sa.sa_status_str(code).startswith(sa.STATUS_NAMES[code])


def _desc(**kw):
    d = sa.sa_attn_desc()
    base = dict(batch=1, heads_q=4, heads_kv=2, seqlen_q=256, seqlen_k=256, head_dim=128,
                causal=0, block_q=128, block_k=64, softmax_scale=1 / math.sqrt(128))
    base.update({k: v for k, v in kw.items() if not k.endswith("stride")})
    for k, v in base.items():
        setattr(d, k, v)
    for name in ("q_stride", "k_stride", "v_stride", "o_stride"):
        default = (256 * 4 * 128, 4 * 128, 128) if name[0] in "qo" else (256 * 2 * 128, 256, 128)
        s = kw.get(name, default)
        for i in range(3):
            getattr(d, name)[i] = s[i]
    return d


def _skip(d, q=FAKE, k=FAKE, v=FAKE, o=FAKE, lam=0.1):
    return sa.raw.sa_skip_softmax_fwd(ctypes.byref(d), q, k, v, o, lam, None, None, None, None, None)


@pytest.mark.parametrize("change,code", [
    (dict(batch=0), sa.SA_ERR_SHAPE),
    (dict(seqlen_k=0), sa.SA_ERR_SHAPE),
    (dict(heads_q=3), sa.SA_ERR_SHAPE),
    (dict(causal=1, seqlen_q=128), sa.SA_ERR_SHAPE),
    (dict(causal=2), sa.SA_ERR_VALUE),
    (dict(head_dim=96), sa.SA_ERR_UNSUPPORTED),
    (dict(block_q=32), sa.SA_ERR_UNSUPPORTED),
    (dict(block_k=32), sa.SA_ERR_UNSUPPORTED),
    (dict(block_k=256), sa.SA_ERR_UNSUPPORTED),
    (dict(softmax_scale=0.0), sa.SA_ERR_VALUE),
    (dict(softmax_scale=float("nan")), sa.SA_ERR_VALUE),
    (dict(q_stride=(256 * 4 * 128, 4 * 128, 4)), sa.SA_ERR_ALIGN),
    (dict(k_stride=(-256, 256, 128)), sa.SA_ERR_ALIGN),
])
def test_skip_rejects_bad_desc(change, code):
    assert _skip(_desc(**change)) == code


@pytest.mark.parametrize("lam", [-1.0, float("nan"), float("inf")])
def test_skip_rejects_bad_lambda(lam):
    assert _skip(_desc(), lam=lam) == sa.SA_ERR_VALUE


def test_skip_rejects_null_and_misaligned():
    assert _skip(_desc(), q=None) == sa.SA_ERR_NULL
    assert sa.raw.sa_skip_softmax_fwd(None, FAKE, FAKE, FAKE, FAKE, 0.1, None, None, None, None,
                                      None) == sa.SA_ERR_NULL
    assert _skip(_desc(), v=FAKE_MIS) == sa.SA_ERR_ALIGN


@pytest.mark.parametrize("n,m,sink,recent,code", [
    (0, 4, 0, 0, sa.SA_ERR_UNSUPPORTED), (5, 4, 0, 0, sa.SA_ERR_UNSUPPORTED),
    (2, 6, 0, 0, sa.SA_ERR_UNSUPPORTED), (9, 8, 0, 0, sa.SA_ERR_UNSUPPORTED),
    (2, 4, -1, 0, sa.SA_ERR_VALUE), (2, 4, 0, -5, sa.SA_ERR_VALUE),
])
def test_nm_rejects(n, m, sink, recent, code):
    d = _desc(causal=1)
    assert sa.raw.sa_nm_softmax_fwd(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, n, m, sink, recent,
                                    None, None, None, None) == code


def test_route_prep_rejects():
    d = _desc(block_k=128)
    assert sa.raw.sa_bitmask_route_prep(ctypes.byref(d), None, FAKE, FAKE, FAKE, None) == sa.SA_ERR_NULL
    assert sa.raw.sa_bitmask_route_prep(None, FAKE, FAKE, FAKE, FAKE, None) == sa.SA_ERR_NULL
    d0 = _desc(block_k=0)
    assert sa.raw.sa_bitmask_route_prep(ctypes.byref(d0), FAKE, FAKE, FAKE, FAKE, None) == sa.SA_ERR_SHAPE


def test_bsr_route_prep_rejects():
    d = _desc(block_k=128)
    f = sa.raw.sa_bsr_route_prep
    assert f(ctypes.byref(d), None, FAKE, 4, FAKE, FAKE, FAKE, None, None) == sa.SA_ERR_NULL
    assert f(ctypes.byref(d), FAKE, None, 4, FAKE, FAKE, FAKE, None, None) == sa.SA_ERR_NULL
    assert f(None, FAKE, FAKE, 4, FAKE, FAKE, FAKE, None, None) == sa.SA_ERR_NULL
    assert f(ctypes.byref(d), FAKE, FAKE, -1, FAKE, FAKE, FAKE, None, None) == sa.SA_ERR_SHAPE
    d0 = _desc(block_k=0)
    assert f(ctypes.byref(d0), FAKE, FAKE, 4, FAKE, FAKE, FAKE, None, None) == sa.SA_ERR_SHAPE
    big = _desc(block_k=1)
    big.seqlen_k = 32 * 2048 + 1
    assert f(ctypes.byref(big), FAKE, FAKE, 4, FAKE, FAKE, FAKE, None, None) == sa.SA_ERR_UNSUPPORTED


def _proxy(d, use_proxy=1, km=FAKE, vs=FAKE, routes=FAKE):
    return sa.raw.sa_proxy_block_sparse_fwd(ctypes.byref(d), FAKE, FAKE, FAKE, km, vs, routes,
                                            FAKE, FAKE, use_proxy, FAKE, None, None)


def test_proxy_rejects():
    assert _proxy(_desc(block_k=128, causal=1)) == sa.SA_ERR_UNSUPPORTED
    assert _proxy(_desc(block_k=32)) == sa.SA_ERR_UNSUPPORTED
    assert _proxy(_desc(block_k=128), km=None) == sa.SA_ERR_NULL
    assert _proxy(_desc(block_k=128), routes=None) == sa.SA_ERR_NULL
    assert _proxy(_desc(block_k=128), vs=FAKE_MIS) == sa.SA_ERR_ALIGN


def test_threshold_matches_oracle_and_rejects():
    for s in (0.0, 0.5, 0.7, 0.95):
        for seq_k in (256, 8192, 16257, 32760):
            sf, lam, l2 = sa.sa_threshold_from_calib(1443.49, 4.30, s, seq_k)
            osf, olam, ol2 = oracle.threshold(1443.49, 4.30, s, seq_k)
            assert sf == pytest.approx(osf, rel=1e-15)
            assert lam == pytest.approx(olam, rel=6e-8)       # float32 rounding of lambda
            assert l2 == pytest.approx(math.log2(lam), abs=1e-6)
    for args in [(0.0, 4.3, 0.5, 10), (1443.49, float("nan"), 0.5, 10), (1443.49, 4.3, 1.0, 10),
                 (1443.49, 4.3, -0.1, 10), (1443.49, 4.3, 0.5, 0)]:
        with pytest.raises(sa.SaError) as e:
            sa.sa_threshold_from_calib(*args)
        assert e.value.status == sa.SA_ERR_VALUE


def test_fit_threshold_matches_oracle_and_rejects():
    import numpy as np
    rng = np.random.default_rng(11)
    s = np.concatenate([np.sort(rng.uniform(0.25, 0.85, 10)), [0.0, 1.0]])
    lam = 1443.49 * np.exp(4.30 * s + rng.normal(0, 0.2, s.size)) / 32760
    got = sa.sa_fit_threshold_calib(lam, s, 32760)
    ref = oracle.fit_threshold(lam, s, 32760)
    for g, r in zip(got, ref):
        assert g == pytest.approx(r, rel=1e-12)
    for lams, sps in [([0.1, 0.2], [0.5, 0.5]), ([0.1, 0.2], [0.0, 0.4]), ([0.0, 0.2], [0.3, 0.4])]:
        with pytest.raises(sa.SaError) as e:
            sa.sa_fit_threshold_calib(lams, sps, 100)
        assert e.value.status == sa.SA_ERR_VALUE
    assert sa.raw.sa_fit_threshold_calib(None, FAKE, 2, 10, FAKE, FAKE, None, None) == sa.SA_ERR_NULL


def test_calibrate_rejects():
    d = _desc()
    f = sa.raw.sa_skip_softmax_calibrate

    def call(trials, n=None, counters=FAKE, out=True, desc=d):
        arr = (ctypes.c_float * max(1, len(trials)))(*trials)
        res = (ctypes.c_double * max(1, len(trials)))()
        return f(ctypes.byref(desc) if desc is not None else None, FAKE, FAKE, FAKE, FAKE,
                 ctypes.addressof(arr), len(trials) if n is None else n, counters,
                 ctypes.addressof(res) if out else None, None)

    assert call([0.1], counters=None) == sa.SA_ERR_NULL
    assert call([0.1], out=False) == sa.SA_ERR_NULL
    assert call([0.1], n=0) == sa.SA_ERR_VALUE
    assert call([0.1, -1.0]) == sa.SA_ERR_VALUE
    assert call([float("nan")]) == sa.SA_ERR_VALUE
    assert call([0.1], desc=None) == sa.SA_ERR_NULL
    assert call([0.1], desc=_desc(block_k=32)) == sa.SA_ERR_UNSUPPORTED


@pytest.mark.parametrize("lam,n,m,sink,recent,code", [
    (-1.0, 2, 4, 0, 0, "VALUE"), (float("inf"), 2, 4, 0, 0, "VALUE"),
    (0.1, 5, 4, 0, 0, "UNSUPPORTED"), (0.1, 0, 4, 0, 0, "UNSUPPORTED"), (0.1, 2, 6, 0, 0, "UNSUPPORTED"),
    (0.1, 2, 4, -1, 0, "VALUE"), (0.1, 2, 4, 0, -1, "VALUE")])
def test_skip_nm_rejects(lam, n, m, sink, recent, code):
    d = _desc()
    f = sa.raw.sa_skip_nm_softmax_fwd
    got = f(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, lam, n, m, sink, recent, None, None, None,
            None, None, None, None)
    assert got == getattr(sa, "SA_ERR_" + code)
    assert f(None, FAKE, FAKE, FAKE, FAKE, 0.1, 2, 4, 0, 0, None, None, None, None, None, None,
             None) == sa.SA_ERR_NULL
    d64 = _desc(block_k=32)
    assert f(ctypes.byref(d64), FAKE, FAKE, FAKE, FAKE, 0.1, 2, 4, 0, 0, None, None, None, None,
             None, None, None) == sa.SA_ERR_UNSUPPORTED


def _dec_desc(**kw):
    base = dict(seqlen_q=1, seqlen_k=1024, heads_q=8, heads_kv=2, block_k=64,
                q_stride=(8 * 128, 8 * 128, 128), o_stride=(8 * 128, 8 * 128, 128),
                k_stride=(1024 * 2 * 128, 2 * 128, 128), v_stride=(1024 * 2 * 128, 2 * 128, 128))
    base.update(kw)
    return _desc(**base)


def test_decode_workspace_plan():
    nbytes, splits = ctypes.c_size_t(), ctypes.c_int32()
    f = sa.raw.sa_skip_softmax_decode_workspace
    d = _dec_desc()
    assert f(ctypes.byref(d), ctypes.c_float(0.5), 0, ctypes.byref(nbytes), ctypes.byref(splits)) == sa.SA_OK
    assert 1 <= splits.value <= 16 and nbytes.value % 256 == 0
    # scores (B*Hkv*Sk*4 heads) + maxima + partials, each padded to 256 bytes
    assert nbytes.value >= 1 * 2 * 1024 * 4 * 4 + 8 * 16 * 4
    assert f(ctypes.byref(d), ctypes.c_float(0.5), 3, ctypes.byref(nbytes), ctypes.byref(splits)) == sa.SA_OK
    assert splits.value == 3
    # lambda > 1: one split, and an explicit larger count is refused
    assert f(ctypes.byref(d), ctypes.c_float(2.0), 0, ctypes.byref(nbytes), ctypes.byref(splits)) == sa.SA_OK
    assert splits.value == 1
    assert f(ctypes.byref(d), ctypes.c_float(2.0), 4, ctypes.byref(nbytes), None) == sa.SA_ERR_UNSUPPORTED
    assert f(ctypes.byref(_dec_desc(seqlen_q=2, causal=0)), ctypes.c_float(0.5), 0, ctypes.byref(nbytes), None) == sa.SA_ERR_UNSUPPORTED
    assert f(ctypes.byref(_dec_desc(block_k=32)), ctypes.c_float(0.5), 0, ctypes.byref(nbytes), None) == sa.SA_ERR_UNSUPPORTED
    assert f(ctypes.byref(_dec_desc(heads_q=64, heads_kv=2)), ctypes.c_float(0.5), 0, ctypes.byref(nbytes), None) == sa.SA_ERR_UNSUPPORTED
    assert f(ctypes.byref(d), ctypes.c_float(-1.0), 0, ctypes.byref(nbytes), None) == sa.SA_ERR_VALUE
    assert f(ctypes.byref(d), ctypes.c_float(0.5), -1, ctypes.byref(nbytes), None) == sa.SA_ERR_VALUE
    assert f(None, ctypes.c_float(0.5), 0, ctypes.byref(nbytes), None) == sa.SA_ERR_NULL


def test_decode_rejects():
    d = _dec_desc()
    f = sa.raw.sa_skip_softmax_decode_fwd

    def call(desc=d, lam=0.5, ws=0x100000, ws_bytes=1 << 30, splits=0):
        return f(ctypes.byref(desc) if desc is not None else None, FAKE, FAKE, FAKE, FAKE,
                 ctypes.c_float(lam), None, splits, ws, ws_bytes, None, None, None, None, None)

    assert call(desc=None) == sa.SA_ERR_NULL
    assert call(ws=None) == sa.SA_ERR_NULL
    assert call(ws=0x100010) == sa.SA_ERR_ALIGN          # not 256-byte aligned
    assert call(ws_bytes=1024) == sa.SA_ERR_SHAPE
    assert call(lam=float("nan")) == sa.SA_ERR_VALUE
    assert call(lam=2.0, splits=2) == sa.SA_ERR_UNSUPPORTED
    assert call(desc=_dec_desc(seqlen_q=4)) == sa.SA_ERR_UNSUPPORTED
    assert call(desc=_dec_desc(causal=1, seqlen_k=1)) == sa.SA_ERR_UNSUPPORTED


# ---- the Python binding's own checks (run before any pointer is taken, so CPU tensors serve) ----

def _bf(*shape):
    import torch
    return torch.zeros(shape, dtype=torch.bfloat16)


def test_binding_rejects_mismatched_tensors():
    q, k = _bf(1, 128, 2, 64), _bf(1, 256, 2, 64)
    with pytest.raises(ValueError, match="v .* must have k's shape"):
        sa.make_desc(q, k, _bf(1, 255, 2, 64), q)
    with pytest.raises(ValueError, match="o .* must have q's shape"):
        sa.make_desc(q, k, k, _bf(1, 128, 2, 128))
    with pytest.raises(ValueError, match="batch/head_dim"):
        sa.make_desc(q, _bf(2, 256, 2, 64))
    with pytest.raises(ValueError, match="batch/head_dim"):
        sa.make_desc(q, _bf(1, 256, 2, 128))


def test_binding_checks_output_sizes():
    import torch
    q, k = _bf(1, 128, 2, 64), _bf(1, 256, 2, 64)
    o = _bf(1, 128, 2, 64)
    # nQT = 1 (block_q 128), nKT = 4
    bad = [dict(tile_state=torch.zeros(1, 2, 1, 3, dtype=torch.uint8)),
           dict(tile_state=torch.zeros(1, 2, 1, 4, dtype=torch.int32)),
           dict(head_counters=torch.zeros(1, 2, 3, dtype=torch.int32)),
           dict(lse=torch.zeros(1, 2, 127)),
           dict(dbg_tile_rowmax=torch.zeros(1, 2, 1, 4, 64))]
    for kw in bad:
        with pytest.raises((ValueError, TypeError), match="must (hold|be)"):
            sa.sa_skip_softmax_fwd(q, k, k, o, 0.5, **kw)
    with pytest.raises(ValueError, match="must hold"):
        sa.sa_nm_softmax_fwd(q, k, k, o, 2, 4, dbg_keep_bits=torch.zeros(1, 2, 128, 7,
                                                                           dtype=torch.int32))
    with pytest.raises(ValueError, match="must hold"):
        sa.sa_nm_softmax_fwd(q, k, k, o, 2, 4, dbg_scores=torch.zeros(1, 2, 128, 255))
    with pytest.raises(ValueError, match="must be contiguous"):
        sa.sa_skip_softmax_fwd(q, k, k, o, 0.5, lse=torch.zeros(1, 128, 2).transpose(1, 2))
    # correctly sized outputs pass the checks and only then meet the GPU-pointer check
    with pytest.raises(ValueError, match="must live on the GPU"):
        sa.sa_skip_softmax_fwd(q, k, k, o, 0.5,
                               tile_state=torch.zeros(1, 2, 1, 4, dtype=torch.uint8),
                               head_counters=torch.zeros(1, 2, 2, dtype=torch.int32),
                               lse=torch.zeros(1, 2, 128), dbg_tile_rowmax=torch.zeros(2, 4, 128))


def test_binding_checks_route_sizes():
    import torch
    kw = dict(batch=1, heads_kv=2, seqlen_q=300, seqlen_k=300, block_q=128, block_k=64)
    # rows = 1*2*3 = 6, nKB = 5, W = 1
    i32 = lambda *s: torch.zeros(s, dtype=torch.int32)   # noqa: E731
    with pytest.raises(ValueError, match="exact_idx must hold"):
        sa.sa_bitmask_route_prep(i32(6, 1), i32(6), i32(6, 4), i32(6, 1), **kw)
    with pytest.raises(ValueError, match="bitmask must hold"):
        sa.sa_bitmask_route_prep(i32(5, 1), i32(6), i32(6, 5), i32(6, 1), **kw)
    with pytest.raises(ValueError, match="block_indptr must hold"):
        sa.sa_bsr_route_prep(i32(6), i32(3), i32(6), i32(6, 5), i32(6, 1), **kw)
    q, k = _bf(1, 300, 2, 64), _bf(1, 300, 2, 64)
    with pytest.raises(ValueError, match="k_mean must hold"):
        sa.sa_proxy_block_sparse_fwd(q, k, k, _bf(1, 2, 4, 64), _bf(1, 2, 5, 64), i32(6),
                                     i32(6, 5), i32(6, 1), 1, q, block_q=128, block_k=64)


@pytest.mark.parametrize("gran", [-1, 2, 7])
def test_skip_ex_rejects_bad_granularity(gran):
    d = _desc()
    assert sa.raw.sa_skip_softmax_fwd_ex(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, 0.1, gran, None,
                                         None, None, None, None) == sa.SA_ERR_VALUE


def test_skip_ex_shares_the_descriptor_checks():
    d = _desc(block_k=32)
    assert sa.raw.sa_skip_softmax_fwd_ex(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, 0.1, 1, None,
                                         None, None, None, None) == sa.SA_ERR_UNSUPPORTED
    assert sa.raw.sa_skip_softmax_fwd_ex(ctypes.byref(_desc()), None, FAKE, FAKE, FAKE, 0.1, 1,
                                         None, None, None, None, None) == sa.SA_ERR_NULL


def test_binding_wave_granularity_output_sizes():
    import torch
    q, k = _bf(1, 100, 2, 64), _bf(1, 256, 2, 64)
    o = _bf(1, 100, 2, 64)
    # wave granularity: nR = ceil(100/32) = 4 blocks of 32 rows, nKT = 2 at block_k 128
    with pytest.raises(ValueError, match="tile_state must hold"):
        sa.sa_skip_softmax_fwd_ex(q, k, k, o, 0.5, "wave", block_k=128,
                                  tile_state=torch.zeros(1, 2, 1, 2, dtype=torch.uint8))
    with pytest.raises(ValueError, match="must live on the GPU"):
        sa.sa_skip_softmax_fwd_ex(q, k, k, o, 0.5, "wave", block_k=128,
                                  tile_state=torch.zeros(1, 2, 4, 2, dtype=torch.uint8),
                                  dbg_tile_rowmax=torch.zeros(1, 2, 4, 2, 32))


def test_decode_noalloc_rejects_on_the_host():
    f = sa.raw.sa_skip_softmax_decode_fwd_noalloc
    d = _desc(seqlen_q=1, seqlen_k=8192, heads_q=32, heads_kv=8, batch=16)
    assert f(None, FAKE, FAKE, FAKE, FAKE, 0.1, None, 0, None, None, None, None, None) == sa.SA_ERR_NULL
    assert f(ctypes.byref(d), None, FAKE, FAKE, FAKE, 0.1, None, 0, None, None, None, None,
             None) == sa.SA_ERR_NULL
    assert f(ctypes.byref(_desc()), FAKE, FAKE, FAKE, FAKE, 0.1, None, 0, None, None, None, None,
             None) == sa.SA_ERR_UNSUPPORTED                         # seqlen_q != 1
    assert f(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, -1.0, None, 0, None, None, None, None,
             None) == sa.SA_ERR_VALUE
    # a workspace larger than the fixed buffer: 4x the decode workload's cache
    big = _desc(seqlen_q=1, seqlen_k=4 * 8192, heads_q=32, heads_kv=8, batch=16)
    need = ctypes.c_size_t()
    assert sa.raw.sa_skip_softmax_decode_workspace(ctypes.byref(big), ctypes.c_float(0.1), 0,
                                                   ctypes.byref(need), None) == sa.SA_OK
    assert need.value > sa.SA_DECODE_SCRATCH_BYTES
    assert f(ctypes.byref(big), FAKE, FAKE, FAKE, FAKE, 0.1, None, 0, None, None, None, None,
             None) == sa.SA_ERR_SCRATCH
