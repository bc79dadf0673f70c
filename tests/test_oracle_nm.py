"""Pins for the oracle's N:M sparse softmax (CPU only).

The Model-Optimizer HuggingFace attention-sparsity page ("N:M Sparse Softmax") fixes the method:
in every M consecutive key positions keep the top-N scores and set the rest to -inf before the
softmax; the first ``dense_sink_tokens`` and the last ``dense_recent_tokens`` stay dense;
M=4 with N=1..3 and M=8 with N=1..7; prefill only.  Checked here against independent routes:

* N = M, a sink covering every key, or a recent window covering every key give dense attention
  (torch SDPA, float64);
* the keep mask equals a numpy stable-argsort top-N per group (ties to the lower index), which is
  a different computation from the oracle's rank count;
* N = 1 keeps exactly the per-group argmax;
* with no sink/recent, non-causal and M dividing Sk, every row keeps exactly N*Sk/M keys;
* with recent >= M (causal), every group straddling the diagonal is fully kept;
* given its mask, the output is masked softmax attention (SDPA).
"""
import math

import numpy as np
import pytest

import oracle
import refs
import workloads as W

NM_PAIRS = [(n, 4) for n in (1, 2, 3)] + [(n, 8) for n in range(1, 8)]


def _run(q, k, v, causal, n, m, sink=0, recent=0, **kw):
    D = q.shape[-1]
    return oracle.nm_softmax(q, k, v, causal=causal, scale=1 / math.sqrt(D), n=n, m=m, sink=sink,
                             recent=recent, **kw)


def _bits_to_mask(bits, Sk):
    B, H, Sq, Wd = bits.shape
    by = bits.view(np.uint8).reshape(B, H, Sq, Wd * 4)
    return np.unpackbits(by, axis=-1, bitorder="little")[..., :Sk].astype(bool)


def _argsort_mask(q, k, n, m, causal, sink, recent):
    """Top-n of every m consecutive keys by numpy stable argsort, plus sink/recent, causal."""
    s = refs.scores(q, k)
    B, H, Sq, Sk = s.shape
    allowed = np.ones((Sq, Sk), bool)
    if causal:
        allowed = np.tril(allowed)
    s = np.where(allowed, s, -np.inf)
    keep = np.zeros_like(s, dtype=bool)
    for g0 in range(0, Sk, m):
        g1 = min(Sk, g0 + m)
        order = np.argsort(-s[..., g0:g1], axis=-1, kind="stable")
        top = np.zeros(order.shape, bool)
        np.put_along_axis(top, order[..., :n], True, axis=-1)
        keep[..., g0:g1] = top
    r = np.arange(Sq)[:, None]
    kk = np.arange(Sk)[None, :]
    dense = (kk < sink) | ((r - kk >= 0) & (r - kk < recent))
    return (keep | dense) & allowed


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("m", [4, 8])
def test_n_equals_m_is_dense(causal, m):
    q, k, v = W.gen_iid(31, 1, 100, 100, 2, 1, 32)
    o, lse, bits = _run(q, k, v, causal, m, m)
    assert np.abs(o - refs.sdpa(q, k, v, 1 / math.sqrt(32), causal=causal)).max() < 1e-12
    allowed = np.ones((100, 100), bool)
    if causal:
        allowed = np.tril(allowed)
    assert (_bits_to_mask(bits, 100) == allowed).all()


def test_sink_or_recent_covering_all_keys_is_dense():
    q, k, v = W.gen_iid(32, 1, 96, 96, 2, 2, 16)
    ref = refs.sdpa(q, k, v, 0.25, causal=True)
    o1, _, _ = _run(q, k, v, True, 1, 8, sink=96)
    o2, _, _ = _run(q, k, v, True, 1, 8, recent=96)
    assert np.abs(o1 - ref).max() < 1e-12 and np.abs(o2 - ref).max() < 1e-12


@pytest.mark.parametrize("n,m", NM_PAIRS)
@pytest.mark.parametrize("causal,sink,recent", [(True, 4, 16), (False, 0, 0), (False, 3, 5)])
def test_mask_matches_stable_argsort(n, m, causal, sink, recent):
    S = 70   # ragged last group for both M
    q, k, v = W.gen_llm(33, 1, S, 2, 1, 16)
    o, lse, bits = _run(q, k, v, causal, n, m, sink, recent)
    mask = _argsort_mask(q, k, n, m, causal, sink, recent)
    assert (_bits_to_mask(bits, S) == mask).all()
    assert np.abs(o - refs.sdpa(q, k, v, 0.25, mask=mask)).max() < 1e-12
    assert np.abs(lse - refs.lse(q, k, 0.25, mask)).max() < 1e-12


def test_ties_go_to_lower_index():
    # keys 0..3 identical, keys 4..7 identical: every score in a group ties
    k = np.repeat(W.gen_iid(34, 1, 1, 2, 1, 1, 16)[1], 4, axis=1)
    q, _, v = W.gen_iid(34, 1, 5, 8, 1, 1, 16)
    _, _, bits = _run(q, k, v, False, 2, 4)
    mask = _bits_to_mask(bits, 8)
    assert (mask == np.array([1, 1, 0, 0, 1, 1, 0, 0], bool)).all()


def test_n1_is_group_argmax():
    q, k, v = W.gen_iid(35, 1, 64, 64, 1, 1, 32)
    _, _, bits = _run(q, k, v, False, 1, 8)
    mask = _bits_to_mask(bits, 64)[0, 0]
    s = refs.scores(q, k)[0, 0]
    for g in range(8):
        am = np.argmax(s[:, g * 8:(g + 1) * 8], axis=-1)
        expect = np.zeros((64, 8), bool)
        expect[np.arange(64), am] = True
        assert (mask[:, g * 8:(g + 1) * 8] == expect).all()


@pytest.mark.parametrize("n,m", NM_PAIRS)
def test_kept_count_without_windows(n, m):
    q, k, v = W.gen_iid(36, 1, 16, 64, 1, 1, 16)
    _, _, bits = _run(q, k, v, False, n, m)
    assert (_bits_to_mask(bits, 64).sum(-1) == n * 64 // m).all()


@pytest.mark.parametrize("m", [4, 8])
def test_groups_straddling_diagonal_dense_with_recent(m):
    S = 64
    q, k, v = W.gen_iid(37, 1, S, S, 1, 1, 16)
    _, _, bits = _run(q, k, v, True, 1, m, recent=m)
    mask = _bits_to_mask(bits, S)[0, 0]
    for r in range(S):
        g0 = (r // m) * m
        assert mask[r, g0:r + 1].all()
        assert not mask[r, r + 1:].any()


def test_replay_and_forced_modes():
    q, k, v = W.gen_llm(38, 1, 64, 2, 2, 32)
    s32 = refs.scores(q, k).astype(np.float32)
    o, _, bits = _run(q, k, v, True, 2, 4, 4, 8)
    _, _, bits_r = _run(q, k, v, True, 2, 4, 4, 8, mode=1, scores_in=s32)
    assert (bits_r == bits).mean() > 0.99
    o_f, _, bits_f = _run(q, k, v, True, 2, 4, 4, 8, mode=2, keep_in=bits)
    assert (bits_f == bits).all() and np.abs(o_f - o).max() < 1e-14


def test_rejects_bad_arguments():
    q, k, v = W.gen_iid(1, 1, 16, 16, 1, 1, 16)
    for n, m in [(0, 4), (5, 4), (1, 0)]:
        with pytest.raises(ValueError):
            _run(q, k, v, False, n, m)
    with pytest.raises(ValueError):
        _run(q, k, v, False, 1, 4, sink=-1)


# ---- keep bits alone, replayed from given scores (oracle.nm_keep_replay) ------------------------

@pytest.mark.parametrize("n,m", NM_PAIRS + [(4, 4), (8, 8)])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("sink,recent", [(3, 9), (0, 0)])
def test_keep_replay_matches_argsort(n, m, causal, sink, recent):
    """Keep bits from fp32 scores equal a numpy stable-argsort top-n over the same scores.  With
    no windows (0, 0) the group holding the diagonal is ranked too, which checks the causal mask
    of the replay's own inputs (a window of M or more keys keeps that whole group dense)."""
    Sq, Hq, D = 150, 2, 32
    q, k, _ = W.gen_llm(41, 1, Sq, Hq, Hq, D)
    s32 = refs.scores(q, k).astype(np.float32)[0]               # [H, Sq, Sk]
    allowed = np.tril(np.ones((Sq, Sq), bool)) if causal else np.ones((Sq, Sq), bool)
    rows = s32.reshape(Hq * Sq, Sq)
    pos = np.tile(np.arange(Sq), Hq)
    got = oracle.nm_keep_replay(rows, pos, seqlen_q=Sq, causal=causal, n=n, m=m, sink=sink,
                                recent=recent)
    s = np.where(allowed[None], s32.astype(np.float64), -np.inf)
    keep = np.zeros_like(s, dtype=bool)
    for g0 in range(0, Sq, m):
        g1 = min(Sq, g0 + m)
        order = np.argsort(-s[..., g0:g1], axis=-1, kind="stable")
        top = np.zeros(order.shape, bool)
        np.put_along_axis(top, order[..., :n], True, axis=-1)
        keep[..., g0:g1] = top
    r = np.arange(Sq)[:, None]
    kk = np.arange(Sq)[None, :]
    keep = (keep | (kk < sink) | ((r - kk >= 0) & (r - kk < recent))) & allowed
    mask = _bits_to_mask(got.reshape(1, Hq, Sq, -1), Sq)[0]
    assert np.array_equal(mask, keep)


def test_keep_replay_equals_full_oracle_replay():
    Sq, H, D = 200, 2, 32
    q, k, v = W.gen_llm(42, 1, Sq, H, H, D)
    s32 = refs.scores(q, k).astype(np.float32)
    for n, m in ((2, 4), (5, 8)):
        _, _, kb = _run(q, k, v, True, n, m, 4, 16, mode=1, scores_in=s32)
        got = oracle.nm_keep_replay(s32.reshape(H * Sq, Sq), np.tile(np.arange(Sq), H),
                                    seqlen_q=Sq, causal=True, n=n, m=m, sink=4, recent=16)
        assert np.array_equal(got, kb.reshape(H * Sq, -1))
