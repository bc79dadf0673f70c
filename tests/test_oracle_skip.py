"""Pins for the oracle's skip-softmax forward (CPU only).

What fixes the method, from the Model-Optimizer skip-softmax pages (README introduction and
"Threshold Modes"): KV tiles whose scores are negligible under lambda are skipped during the
FlashAttention loop, and the kernel works with log2(lambda).  The oracle is checked against
consequences of that definition that it does not itself compute:

* lambda = 0 never skips, so the result is textbook softmax attention (torch SDPA, float64);
* a huge lambda keeps only the first visited tile of every row block;
* for lambda <= 1 a skipped tile can never raise the running max, so keep(j) holds exactly when
  some valid row reaches the dense prefix max of the earlier tiles plus log2(lambda) -- computed
  here from numpy logits, independently of the oracle's loop;
* decisions are monotone in lambda (lambda <= 1);
* whatever is kept, the output is softmax attention restricted to the kept tiles' keys;
* hand-built cases with exact logits fix the strict test, the untouched state on skip and the
  all-rows rule.
"""
import math

import numpy as np
import pytest

import oracle
import refs
import workloads as W


def _run(q, k, v, causal, Br, Bc, lam, scale=None, **kw):
    D = q.shape[-1]
    scale = scale if scale is not None else 1.0 / math.sqrt(D)
    return oracle.skip_softmax(q, k, v, causal=causal, block_q=Br, block_k=Bc, scale=scale,
                               lam=lam, **kw)


CASES = [
    # (B, Sq, Sk, Hq, Hkv, D, causal, Br, Bc)
    (1, 256, 256, 2, 2, 64, False, 64, 64),
    (1, 200, 200, 4, 2, 32, True, 64, 32),     # ragged tail, GQA, Br != Bc
    (2, 96, 160, 2, 1, 16, False, 32, 64),     # Sq != Sk non-causal, ragged K tile
    (1, 130, 130, 2, 2, 16, True, 128, 64),    # 2-row last Q tile
    (2, 1, 300, 4, 2, 32, False, 1, 64),       # decode: one query row per head, ragged K tile
    (1, 1, 640, 2, 2, 16, False, 1, 128),      # decode with 128-key tiles
]


@pytest.mark.parametrize("case", CASES)
def test_lambda_zero_is_dense_attention(case):
    B, Sq, Sk, Hq, Hkv, D, causal, Br, Bc = case
    q, k, v = W.gen_iid(11, B, Sq, Sk, Hq, Hkv, D)
    o, lse, st, _ = _run(q, k, v, causal, Br, Bc, 0.0)
    ref = refs.sdpa(q, k, v, 1 / math.sqrt(D), causal=causal)
    assert np.abs(o - ref).max() < 1e-12
    assert set(np.unique(st)) <= {0, 2}
    if causal:
        nQT, nKT = st.shape[2:]
        for i in range(nQT):
            last_row = min((i + 1) * Br, Sq) - 1
            for j in range(nKT):
                assert st[0, 0, i, j] == (0 if j * Bc <= last_row else 2)
    mask = np.ones((B, Hq, Sq, Sk), bool)
    if causal:
        mask &= np.tril(np.ones((Sq, Sk), bool))
    assert np.abs(lse - refs.lse(q, k, 1 / math.sqrt(D), mask)).max() < 1e-12


@pytest.mark.parametrize("case", CASES)
def test_huge_lambda_keeps_only_first_tile(case):
    B, Sq, Sk, Hq, Hkv, D, causal, Br, Bc = case
    q, k, v = W.gen_iid(12, B, Sq, Sk, Hq, Hkv, D)
    o, _, st, _ = _run(q, k, v, causal, Br, Bc, 1e30)
    assert (st[..., 0] == 0).all()
    assert set(np.unique(st[..., 1:])) <= {1, 2}
    mask = np.zeros((B, Hq, Sq, Sk), bool)
    mask[..., :Bc] = True
    ref = refs.sdpa(q, k, v, 1 / math.sqrt(D), mask=mask, causal=causal)
    assert np.abs(o - ref).max() < 1e-12


def _closed_form_keep(q, k, causal, Br, Bc, lam, scale, dtype=np.float64):
    """keep(j) for lambda <= 1 from the dense prefix max of tile row maxima (numpy logits)."""
    c = scale * math.log2(math.e)
    t = (c * refs.scores(q, k)).astype(dtype)
    B, Hq, Sq, Sk = t.shape
    if causal:
        t = np.where(np.tril(np.ones((Sq, Sk), bool)), t, -np.inf)
    nQT, nKT = -(-Sq // Br), -(-Sk // Bc)
    L = dtype(math.log2(lam))
    keep = np.zeros((B, Hq, nQT, nKT), np.int8)
    margin = np.full((B, Hq, nQT, nKT), np.inf)
    for i in range(nQT):
        rows = slice(i * Br, min(Sq, (i + 1) * Br))
        prefix = np.full(t[:, :, rows, 0].shape, -np.inf, dtype)
        for j in range(nKT):
            Mj = t[:, :, rows, j * Bc:min(Sk, (j + 1) * Bc)].max(axis=-1)
            visited = (not causal) or j * Bc <= min(Sq, (i + 1) * Br) - 1
            if not visited:
                keep[:, :, i, j] = -1
                continue
            thr = (prefix + L).astype(dtype)
            keep[:, :, i, j] = (Mj >= thr).any(axis=-1)
            with np.errstate(invalid="ignore"):
                gap = np.abs(Mj - thr)
            margin[:, :, i, j] = np.nanmin(np.where(np.isfinite(gap), gap, np.inf), axis=-1)
            prefix = np.maximum(prefix, Mj)
    return keep, margin


@pytest.mark.parametrize("Br,Bc", [(32, 32), (128, 128), (64, 128)])
@pytest.mark.parametrize("lam", [0.25, 0.5, 0.8, 1.0])
@pytest.mark.parametrize("causal", [True, False])
def test_closed_form_decisions_for_lambda_at_most_one(lam, causal, Br, Bc):
    S, D = 512, 128
    q, k, v = W.gen_llm(21, 1, S, 2, 1, D)
    _, _, st, _ = _run(q, k, v, causal, Br, Bc, lam)
    keep, margin = _closed_form_keep(q, k, causal, Br, Bc, lam, 1 / math.sqrt(D))
    visited = keep >= 0
    assert ((st == 2) == ~visited).all()
    clear = visited & (margin > 1e-9)
    assert (st[clear] == 1 - keep[clear]).all()
    assert clear.sum() >= 0.99 * visited.sum()


def test_closed_form_case_is_not_vacuous():
    S, Br, Bc, D = 512, 32, 32, 128
    q, k, v = W.gen_llm(21, 1, S, 2, 1, D)
    _, _, st, _ = _run(q, k, v, True, Br, Bc, 0.8)
    assert (st == 1).sum() > 10 and (st == 0).sum() > 10


@pytest.mark.parametrize("causal", [True, False])
def test_decisions_monotone_in_lambda(causal):
    q, k, v = W.gen_llm(22, 1, 384, 2, 2, 128)
    prev = None
    for lam in [1e-3, 0.1, 0.3, 0.6, 0.9, 1.0]:
        _, _, st, _ = _run(q, k, v, causal, 64, 64, lam)
        skipped = st == 1
        if prev is not None:
            assert (skipped | ~prev).all(), "a tile skipped at a smaller lambda was kept"
        prev = skipped


@pytest.mark.parametrize("lam", [0.5, 1.0, 1.5, 3.0])
@pytest.mark.parametrize("case", CASES[:2])
def test_output_is_attention_over_kept_tiles(case, lam):
    B, Sq, Sk, Hq, Hkv, D, causal, Br, Bc = case
    q, k, v = W.gen_llm(23, B, Sq, Hq, Hkv, D)
    o, lse, st, _ = _run(q, k, v, causal, Br, Bc, lam)
    mask = refs.tile_key_mask(st, Sq, Sk, Br, Bc, causal)
    ref = refs.sdpa(q, k, v, 1 / math.sqrt(D), mask=mask)
    assert np.abs(o - ref).max() < 1e-12
    assert np.abs(lse - refs.lse(q, k, 1 / math.sqrt(D), mask)).max() < 1e-12
    first = np.argmax(st != 2, axis=-1)
    assert (np.take_along_axis(st, first[..., None], -1) == 0).all()


def _exact_case(q_scalars, key_values):
    """Query r is q_scalars[r] * e0 and key j is key_values[j] * e0, so with scale = ln 2 the
    log2-domain logit of (r, j) is exactly q_scalars[r] * key_values[j].  V is one-hot per key, so
    an output row is the attention weight vector itself."""
    n = len(key_values)
    q = np.zeros((1, len(q_scalars), 1, n), np.float32)
    q[0, :, 0, 0] = q_scalars
    k = np.zeros((1, n, 1, n), np.float32)
    k[0, :, 0, 0] = key_values
    v = np.eye(n, dtype=np.float32).reshape(1, n, 1, n)
    return W.to_bf16_bits(q), W.to_bf16_bits(k), W.to_bf16_bits(v)


LN2 = math.log(2.0)   # scale*log2(e) == 1 exactly in double, so logits equal q.k


@pytest.mark.parametrize("lam,state,weights", [
    # logits [0, 2, 1, 3.5], one key per tile.  m after tile 0 is 0.
    (0.0, [0, 0, 0, 0], [1, 4, 2, 2 ** 3.5]),
    (2.0, [0, 0, 1, 0], [1, 4, 0, 2 ** 3.5]),    # L=1: 2<1 no; 1<3 skip; 3.5<3 no
    (4.0, [0, 0, 1, 1], [1, 4, 0, 0]),           # L=2: 2<2 is false (strict) -> kept, m=2
    (8.0, [0, 1, 1, 0], [1, 0, 0, 2 ** 3.5]),    # L=3: skipped tiles leave m=0, so 3.5<3 no
])
def test_hand_built_sequence(lam, state, weights):
    q, k, v = _exact_case([1.0], [0.0, 2.0, 1.0, 3.5])
    o, lse, st, rm = _run(q, k, v, False, 1, 1, lam, scale=LN2)
    assert st[0, 0, 0].tolist() == state
    w = np.asarray(weights, float)
    assert np.abs(o[0, 0, 0] - w / w.sum()).max() < 1e-15
    assert abs(lse[0, 0, 0] - math.log(w.sum())) < 1e-14   # ln sum 2^t (natural log)
    assert rm[0, 0, 0, :, 0].tolist() == [0.0, 2.0, 1.0, 3.5]


def test_tile_kept_if_any_row_not_negligible():
    # two query rows (+e0, -e0) in one tile; keys [0, -3]: row 0 sees -3 after 0 (negligible at
    # lambda 0.5, L=-1), row 1 sees +3 after 0 (not negligible), so the 2x1 tile is kept.
    q, k, v = _exact_case([1.0, -1.0], [0.0, -3.0])
    _, _, st, _ = _run(q, k, v, False, 2, 1, 0.5, scale=LN2)
    assert st[0, 0, 0].tolist() == [0, 0]
    # a single-row tile holding only row 0 skips the second key tile
    _, _, st1, _ = _run(q, k, v, False, 1, 1, 0.5, scale=LN2)
    assert st1[0, 0, 0].tolist() == [0, 1] and st1[0, 0, 1].tolist() == [0, 0]


def test_replay_mode_fp32_decisions():
    """Replay in fp32 agrees with the fp32 closed form computed from the same maxima."""
    q, k, v = W.gen_llm(24, 1, 512, 2, 2, 64)
    lam = 0.7
    _, _, st64, rm = _run(q, k, v, True, 64, 64, lam)
    rm32 = rm.astype(np.float32)
    _, _, st32, _ = _run(q, k, v, True, 64, 64, lam, mode=1, rowmax_in=rm32)
    L32 = np.float32(math.log2(np.float64(np.float32(lam))))
    B, Hq, nQT, nKT, Br = rm32.shape
    for h in range(Hq):
        for i in range(nQT):
            m = np.full(Br, -np.inf, np.float32)
            nr = min(512, (i + 1) * Br) - i * Br
            for j in range(nKT):
                if st32[0, h, i, j] == 2:
                    continue
                M = rm32[0, h, i, j, :nr]
                skip = bool((M < (m[:nr] + L32)).all())
                assert st32[0, h, i, j] == int(skip)
                if not skip:
                    m[:nr] = np.maximum(m[:nr], M)
    assert (st32 == st64).mean() > 0.99


def test_forced_mode_follows_given_states():
    q, k, v = W.gen_iid(25, 1, 128, 128, 1, 1, 16)
    st_in = np.array([[[[0, 1], [0, 0]]]], np.uint8)
    o, _, st, _ = _run(q, k, v, False, 64, 64, 0.0, mode=2, state_in=st_in)
    assert (st == st_in).all()
    mask = refs.tile_key_mask(st_in, 128, 128, 64, 64, False)
    assert np.abs(o - refs.sdpa(q, k, v, 0.25, mask=mask)).max() < 1e-12


def test_forced_mode_with_every_tile_skipped_is_empty():
    # A row that attends to nothing has O = 0 and LSE = log 0 = -inf (the convention every path
    # shares); only forced states can produce it, since a free run always keeps a row's first
    # tile.  Rows past Sq keep LSE 0 (they are padding, not rows).
    q, k, v = W.gen_iid(27, 1, 100, 128, 1, 1, 16)
    st_in = np.ones((1, 1, 2, 2), np.uint8)
    o, lse, st, _ = _run(q, k, v, False, 64, 64, 0.0, mode=2, state_in=st_in)
    assert (st == 1).all() and (o == 0).all()
    assert np.isneginf(lse).all()
    ou, lu, _, _ = _run(q, k, v, False, 64, 64, 0.0, mode=2, state_in=st_in, units=[1])
    assert np.isneginf(lu[0, :36]).all() and (lu[0, 36:] == 0).all()


def test_units_subset_matches_full_run():
    q, k, v = W.gen_llm(26, 1, 256, 4, 2, 32)
    o, lse, st, rm = _run(q, k, v, True, 64, 64, 0.9)
    units = [0, 5, 15]
    ou, lu, su, ru = _run(q, k, v, True, 64, 64, 0.9, units=units)
    for n, u in enumerate(units):
        h, i = divmod(u, 4)
        assert np.array_equal(ou[n], o[0, i * 64:(i + 1) * 64, h])
        assert np.array_equal(su[n], st[0, h, i])


def test_rejects_bad_arguments():
    q, k, v = W.gen_iid(1, 1, 64, 64, 2, 2, 16)
    with pytest.raises(ValueError):
        _run(q, k, v, False, 64, 64, -1.0)
    with pytest.raises(ValueError):
        _run(q, k, v, False, 64, 64, float("nan"))
    with pytest.raises(ValueError):
        _run(q, k[:, :32], v[:, :32], True, 64, 64, 0.1)   # causal needs Sq == Sk


# ---- decisions-only replay (oracle.skip_replay) -------------------------------------------------

def _fp32_closed_form_states(rm32, Sq, Br, Bc, causal, lam):
    """For lambda <= 1: a skipped tile has M < fl32(m + L) <= m, so it never raises the running
    max and m is the fp32 prefix max of every earlier visited tile; keep(j) holds exactly when
    some valid row has M_j >= fl32(prefix + L32).  Vectorised numpy over [units, nKT, Br]."""
    n, nKT, _ = rm32.shape
    L32 = np.float32(math.log2(np.float64(np.float32(lam))))
    st = np.zeros((n, nKT), np.uint8)
    qt = np.arange(n) % (-(-Sq // Br))
    nr = np.minimum(Br, Sq - qt * Br)
    valid = np.arange(Br)[None, :] < nr[:, None]
    prefix = np.full((n, Br), -np.inf, np.float32)
    for j in range(nKT):
        visited = (j * Bc <= qt * Br + nr - 1) if causal else np.ones(n, bool)
        M = rm32[:, j, :]
        keep = ((M >= (prefix + L32)) & valid).any(axis=1)
        st[:, j] = np.where(visited, np.where(keep, 0, 1), 2)
        prefix = np.where(visited[:, None], np.maximum(prefix, M), prefix)
    return st


@pytest.mark.parametrize("lam", [0.1, 0.4, 0.8, 1.0])
@pytest.mark.parametrize("causal,Sq,Br,Bc", [(True, 512, 128, 64), (False, 300, 64, 64),
                                             (True, 200, 32, 128), (False, 257, 32, 64),
                                             # the last query row is the first key of a tile
                                             (True, 257, 64, 64), (True, 129, 128, 128)])
def test_skip_replay_matches_fp32_closed_form(lam, causal, Sq, Br, Bc):
    """Replay from maxima of numpy fp32 logits equals the fp32 closed form (lambda <= 1)."""
    D, H = 64, 3
    q, k, _ = W.gen_llm(31, 1, Sq, H, H, D)
    c = (1 / math.sqrt(D)) * math.log2(math.e)
    t = (c * refs.scores(q, k)).astype(np.float32)[0]          # [H, Sq, Sk]
    if causal:
        t = np.where(np.tril(np.ones((Sq, Sq), bool)), t, -np.inf).astype(np.float32)
    nQT, nKT = -(-Sq // Br), -(-Sq // Bc)
    rm = np.full((H, nQT, nKT, Br), -np.inf, np.float32)
    for i in range(nQT):
        for j in range(nKT):
            blk = t[:, i * Br:(i + 1) * Br, j * Bc:(j + 1) * Bc]
            rm[:, i, j, :blk.shape[1]] = blk.max(axis=-1)
    rm = rm.reshape(H * nQT, nKT, Br)
    st = oracle.skip_replay(rm, batch=1, heads_q=H, seqlen_q=Sq, seqlen_k=Sq, causal=causal,
                            block_q=Br, block_k=Bc, lam=lam)
    ref = _fp32_closed_form_states(rm, Sq, Br, Bc, causal, lam)
    assert np.array_equal(st, ref)
    vis = st != 2
    if (causal, Sq, Br, Bc) == (False, 257, 32, 64):   # not vacuous: this case skips 22-67 tiles
        assert (st[vis] == 1).sum() >= 20


def test_skip_replay_threshold_is_rounded_to_fp32():
    """The threshold is fl32(m + L32), not the exact sum: with a running max m for which the fp32
    sum rounds down, a tile whose max equals fl32(m + L32) is kept (the exact sum would skip it).
    Inside one binade of m the bits of the sum below m's last place come from L32 alone, so the
    case is searched over lambda and the binade of m."""
    def find():
        for lam in np.linspace(0.3, 0.95, 14):
            L32 = np.float32(math.log2(np.float64(np.float32(lam))))
            for m in (np.float32(3.0), np.float32(5.0), np.float32(10.0), np.float32(20.0)):
                thr = np.float32(m + L32)
                if np.float64(thr) < np.float64(m) + np.float64(L32):
                    return float(lam), m, thr
        raise AssertionError("no rounding-down case")
    lam, m, thr = find()
    rm = np.array([[[m], [thr], [np.nextafter(thr, np.float32(-np.inf))]]], np.float32)
    st = oracle.skip_replay(rm, batch=1, heads_q=1, seqlen_q=1, seqlen_k=3, causal=False,
                            block_q=1, block_k=1, lam=lam)
    assert st[0].tolist() == [0, 0, 1]


@pytest.mark.parametrize("lam,state", [(0.0, [0, 0, 0, 0]), (2.0, [0, 0, 1, 0]),
                                       (4.0, [0, 0, 1, 1]), (8.0, [0, 1, 1, 0])])
def test_skip_replay_hand_built_sequence(lam, state):
    """Maxima [0, 2, 1, 3.5] of one row over four one-key tiles: the strict test and the
    untouched running max on a skip (lambda > 1), as in the hand-built oracle case above."""
    rm = np.array([[[0.0], [2.0], [1.0], [3.5]]], np.float32)
    st = oracle.skip_replay(rm, batch=1, heads_q=1, seqlen_q=1, seqlen_k=4, causal=False,
                            block_q=1, block_k=1, lam=lam)
    assert st[0].tolist() == state


@pytest.mark.parametrize("lam", [0.0, 0.5, 1.0, 1.5, 3.0, 1e30])
@pytest.mark.parametrize("case", CASES)
def test_skip_replay_equals_full_oracle_replay(case, lam):
    """On any maxima, the decisions-only replay equals mode 1 of the full oracle."""
    B, Sq, Sk, Hq, Hkv, D, causal, Br, Bc = case
    q, k, v = W.gen_llm(32, B, Sq, Hq, Hkv, D) if Sq == Sk else W.gen_iid(32, B, Sq, Sk, Hq, Hkv, D)
    _, _, _, rm = _run(q, k, v, causal, Br, Bc, 0.0)
    rm32 = rm.astype(np.float32)
    _, _, st_full, _ = _run(q, k, v, causal, Br, Bc, lam, mode=1, rowmax_in=rm32)
    nQT, nKT = st_full.shape[2:]
    st = oracle.skip_replay(rm32.reshape(-1, nKT, Br), batch=B, heads_q=Hq, seqlen_q=Sq,
                            seqlen_k=Sk, causal=causal, block_q=Br, block_k=Bc, lam=lam)
    assert np.array_equal(st, st_full.reshape(-1, nKT))
    units = np.array([0, B * Hq * nQT - 1])
    st_u = oracle.skip_replay(rm32.reshape(-1, nKT, Br)[units], batch=B, heads_q=Hq, seqlen_q=Sq,
                              seqlen_k=Sk, causal=causal, block_q=Br, block_k=Bc, lam=lam,
                              units=units)
    assert np.array_equal(st_u, st_full.reshape(-1, nKT)[units])



# ---- decision granularity: each 32-row block on its own (oracle.skip_softmax_wave) ---------------

@pytest.mark.parametrize("causal", [True, False])
def test_wave_granularity_is_the_tile_rule_on_32_row_tiles(causal):
    q, k, v = W.gen_llm(71, 1, 300, 2, 2, 64)
    for lam in (0.0, 0.7, 2.0):
        a = oracle.skip_softmax_wave(q, k, v, causal=causal, block_k=64, scale=0.125, lam=lam)
        b = _run(q, k, v, causal, 32, 64, lam)
        for x, y in zip(a, b):
            assert np.array_equal(x, y)


@pytest.mark.parametrize("Bc", [64, 128])
def test_wave_granularity_lambda_zero_is_dense(Bc):
    q, k, v = W.gen_llm(72, 1, 256, 2, 1, 64)
    o, lse, st, _ = oracle.skip_softmax_wave(q, k, v, causal=True, block_k=Bc, scale=0.125,
                                             lam=0.0)
    assert (st != 1).all()
    assert np.abs(o - refs.sdpa(q, k, v, 0.125, causal=True)).max() < 1e-12


@pytest.mark.parametrize("lam", [0.3, 0.6, 0.9])
@pytest.mark.parametrize("Bc", [64, 128])
def test_wave_sparsity_at_least_tile_sparsity(lam, Bc):
    """For lambda <= 1 every row's running max is the dense prefix max at either granularity, so a
    tile that 128 rows skip together is skipped by each 32-row block that visits it: wave sparsity
    (over the pairs a block visits) is at least tile sparsity.  Closed-form consequence, checked
    on the oracle's decisions."""
    q, k, v = W.gen_llm(73, 1, 1024, 2, 2, 128)
    _, _, st_t, _ = _run(q, k, v, True, 128, Bc, lam)
    _, _, st_w, _ = oracle.skip_softmax_wave(q, k, v, causal=True, block_k=Bc,
                                             scale=1 / math.sqrt(128), lam=lam)
    tile_skip = np.repeat(st_t == 1, 4, axis=2)
    assert (st_w[tile_skip] != 0).all()
    vis = st_w != 2
    assert (st_w[vis] == 1).sum() >= tile_skip[vis].sum()
