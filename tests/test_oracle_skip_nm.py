"""Pins for the oracle's skip-softmax + N:M combined forward (CPU only).

The combined configuration of the HuggingFace attention-sparsity page (skip_softmax_calib_sparse24:
calibrated skip-softmax together with 2:4 sparse softmax) uses the two methods at once.  The oracle
is checked against the separately pinned skip-softmax and N:M oracles and against textbook
attention:

* the N:M rule keeps every group maximum, so the tile decisions and tile maxima equal those of
  skip-softmax alone, for every N:M;
* lambda = 0 never skips: the result is the N:M oracle's;
* N = M keeps everything: the result is the skip-softmax oracle's;
* whatever is decided, the output is softmax attention (torch SDPA, float64) over the keys that
  are both N:M-kept and in a kept tile;
* replay and forced modes reproduce the independent run when fed its own decisions.
"""
import math

import numpy as np
import pytest

import oracle
import refs
import workloads as W

CASES = [
    # (B, S, Hq, Hkv, D, causal, Br, Bc, n, m, sink, recent)
    (1, 256, 2, 2, 64, False, 64, 64, 2, 4, 0, 0),
    (1, 200, 4, 2, 32, True, 64, 64, 2, 4, 4, 32),     # ragged, GQA, sink + recent
    (2, 130, 2, 1, 16, True, 128, 64, 3, 8, 4, 16),    # 2-row last tile, M = 8
    (1, 190, 2, 2, 32, False, 64, 64, 1, 4, 0, 64),    # partial last group
]


def _unpack(kb, Sk):
    by = np.ascontiguousarray(kb).view(np.uint8).reshape(*kb.shape[:-1], kb.shape[-1] * 4)
    return np.unpackbits(by, axis=-1, bitorder="little")[..., :Sk].astype(bool)


def _inputs(seed, case):
    B, S, Hq, Hkv, D, causal, Br, Bc, n, m, sink, recent = case
    return W.gen_llm(seed, B, S, Hq, Hkv, D)


def _combined(q, k, v, case, lam, **kw):
    B, S, Hq, Hkv, D, causal, Br, Bc, n, m, sink, recent = case
    return oracle.skip_nm_softmax(q, k, v, causal=causal, block_q=Br, block_k=Bc,
                                  scale=1 / math.sqrt(D), lam=lam, n=n, m=m, sink=sink,
                                  recent=recent, **kw)


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("lam", [0.3, 1.0, 4.0])
def test_decisions_equal_skip_alone_and_output_is_masked_attention(case, lam):
    B, S, Hq, Hkv, D, causal, Br, Bc, n, m, sink, recent = case
    q, k, v = _inputs(61, case)
    scale = 1 / math.sqrt(D)
    o, lse, st, rm, kb = _combined(q, k, v, case, lam)
    _, _, st_s, rm_s = oracle.skip_softmax(q, k, v, causal=causal, block_q=Br, block_k=Bc,
                                           scale=scale, lam=lam)
    assert np.array_equal(st, st_s)
    fin = np.isfinite(rm_s)
    assert np.array_equal(np.isfinite(rm), fin) and np.array_equal(rm[fin], rm_s[fin])
    _, _, kb_nm = oracle.nm_softmax(q, k, v, causal=causal, scale=scale, n=n, m=m, sink=sink,
                                    recent=recent)
    assert np.array_equal(kb, kb_nm)
    mask = refs.tile_key_mask(st, S, S, Br, Bc, causal) & _unpack(kb, S)
    ref = refs.sdpa(q, k, v, scale, mask=mask)
    assert np.abs(o - ref).max() < 1e-12
    assert np.abs(lse - refs.lse(q, k, scale, mask)).max() < 1e-12


@pytest.mark.parametrize("case", CASES)
def test_lambda_zero_is_nm_softmax(case):
    B, S, Hq, Hkv, D, causal, Br, Bc, n, m, sink, recent = case
    q, k, v = _inputs(62, case)
    o, lse, st, _, kb = _combined(q, k, v, case, 0.0)
    o_nm, lse_nm, kb_nm = oracle.nm_softmax(q, k, v, causal=causal, scale=1 / math.sqrt(D), n=n,
                                            m=m, sink=sink, recent=recent)
    assert set(np.unique(st)) <= {0, 2}
    assert np.abs(o - o_nm).max() < 1e-12 and np.abs(lse - lse_nm).max() < 1e-12
    assert np.array_equal(kb, kb_nm)


@pytest.mark.parametrize("case", CASES)
def test_n_equal_m_is_skip_softmax(case):
    B, S, Hq, Hkv, D, causal, Br, Bc, n, m, sink, recent = case
    case = case[:8] + (m, m, sink, recent)
    q, k, v = _inputs(63, case)
    o, lse, st, rm, _ = _combined(q, k, v, case, 0.5)
    o_s, lse_s, st_s, rm_s = oracle.skip_softmax(q, k, v, causal=causal, block_q=Br, block_k=Bc,
                                                 scale=1 / math.sqrt(D), lam=0.5)
    assert np.array_equal(st, st_s)
    assert np.abs(o - o_s).max() < 1e-12 and np.abs(lse - lse_s).max() < 1e-12


def test_replay_and_forced_modes_reproduce_their_inputs():
    case = CASES[1]
    B, S, Hq, Hkv, D, causal, Br, Bc, n, m, sink, recent = case
    q, k, v = _inputs(64, case)
    o, lse, st, rm, kb = _combined(q, k, v, case, 1.0)
    sc = refs.scores(q, k).astype(np.float32)
    # replay on the oracle's own maxima and scores, rounded to fp32
    _, _, st1, _, kb1 = _combined(q, k, v, case, 1.0, mode=1, rowmax_in=rm.astype(np.float32),
                                  scores_in=sc)
    assert np.array_equal(kb1, kb)
    assert (st1 == st).mean() > 0.99
    o2, lse2, st2, _, kb2 = _combined(q, k, v, case, 1.0, mode=2, state_in=st, keep_in=kb)
    assert np.array_equal(st2, st) and np.array_equal(kb2, kb)
    assert np.abs(o2 - o).max() < 1e-12


@pytest.mark.parametrize("case", CASES)
def test_replay_mode_decides_from_the_given_maxima_alone(case):
    """Mode 1 decides from the fp32 maxima it is handed, exactly as the separately pinned
    decisions-only replay does: on maxima that are not the true ones (perturbed), the two agree on
    every tile, while the keep bits still come from the given scores."""
    B, S, Hq, Hkv, D, causal, Br, Bc, n, m, sink, recent = case
    q, k, v = _inputs(66, case)
    _, _, _, rm, kb = _combined(q, k, v, case, 0.0)
    rm32 = rm.astype(np.float32)
    fin = np.isfinite(rm32)
    rm32[fin] += np.random.default_rng(67).normal(0, 0.5, int(fin.sum())).astype(np.float32)
    sc = refs.scores(q, k).astype(np.float32)
    nQT, nKT = rm.shape[2], rm.shape[3]
    skipped = 0
    for lam in (0.5, 1.0, 3.0):
        _, _, st, _, kb1 = _combined(q, k, v, case, lam, mode=1, rowmax_in=rm32, scores_in=sc)
        ref = oracle.skip_replay(rm32.reshape(-1, nKT, Br), batch=B, heads_q=Hq, seqlen_q=S,
                                 seqlen_k=S, causal=causal, block_q=Br, block_k=Bc, lam=lam)
        assert np.array_equal(st.reshape(-1, nKT), ref)
        assert np.array_equal(kb1, kb)
        skipped += int((ref == 1).sum())
    assert skipped > 0


def test_replay_mode_threshold_is_rounded_to_fp32():
    """As in the skip-softmax replay: the threshold is fl32(m + L32), so with a running max m for
    which that sum rounds down, a tile whose max equals it is kept and one just below is skipped."""
    def find():
        for lam in np.linspace(0.3, 0.95, 14):
            L32 = np.float32(math.log2(np.float64(np.float32(lam))))
            for m in (np.float32(3.0), np.float32(5.0), np.float32(10.0), np.float32(20.0)):
                thr = np.float32(m + L32)
                if np.float64(thr) < np.float64(m) + np.float64(L32):
                    return float(lam), m, thr
        raise AssertionError("no rounding-down case")
    lam, m, thr = find()
    q, k, v = W.gen_iid(68, 1, 1, 3, 1, 1, 16)
    rm = np.array([m, thr, np.nextafter(thr, np.float32(-np.inf))], np.float32)
    _, _, st, _, _ = oracle.skip_nm_softmax(q, k, v, causal=False, block_q=1, block_k=1,
                                            scale=0.25, lam=lam, n=1, m=1, sink=0, recent=0,
                                            mode=1, rowmax_in=rm,
                                            scores_in=np.zeros((1, 1, 1, 3), np.float32))
    assert st.ravel().tolist() == [0, 0, 1]


def test_rejects_bad_arguments():
    q, k, v = W.gen_iid(65, 1, 64, 64, 1, 1, 16)
    with pytest.raises(ValueError):
        oracle.skip_nm_softmax(q, k, v, causal=False, block_q=64, block_k=64, scale=0.25, lam=-1.0,
                               n=2, m=4, sink=0, recent=0)
    with pytest.raises(ValueError):
        oracle.skip_nm_softmax(q, k, v, causal=False, block_q=64, block_k=64, scale=0.25, lam=0.1,
                               n=5, m=4, sink=0, recent=0)
