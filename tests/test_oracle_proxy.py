"""Pins for the oracle's route preparation and proxy-compensated block-sparse forward (CPU only).

The FlashInfer block-sparse proxy description (quoted in the TensorRT-LLM "add VisualGen SOL
sparse attention" PR, "Description" and "Bitmask format") fixes: packed UInt32 exact-block bitmaps
per (batch, KV head, Q block) with padding bits ignored; omitted blocks approximated by one
arithmetic-mean K and one summed-V summary; the denominator corrected by the token mass each
summary represents, including the true length of the final partial block; all-exact parity with
dense attention; mixed-proxy cases at 256/257 tokens.  Checked here:

* route prep equals numpy ``unpackbits(bitorder="little")``, with garbage in the padding bits;
* an all-ones bitmap gives dense attention (SDPA, float64);
* K constant inside every block (with exactly representable V sums) gives dense attention for
  ANY bitmap -- this fixes the mean-K logit, the summed-V numerator and c_j = true block length,
  including a 1-token last block;
* block size 1 gives dense attention for any bitmap;
* use_proxy = 0 gives attention restricted to the exact blocks;
* a row with no exact block and no proxy gives O = 0, lse = -inf.
"""
import math

import numpy as np
import pytest

import oracle
import refs
import workloads as W


def _unpack(bm, nKB):
    by = np.ascontiguousarray(bm).view(np.uint8).reshape(*bm.shape[:-1], bm.shape[-1] * 4)
    return np.unpackbits(by, axis=-1, bitorder="little")[..., :nKB].astype(bool)


@pytest.mark.parametrize("nKB", [1, 5, 32, 33, 128, 255])
def test_route_prep_matches_unpackbits(nKB):
    bm = W.gen_bitmask(41, 2, 3, 7, nKB, max(1, nKB // 4), garbage_padding=True)
    n_exact, idx, keep = oracle.route_prep(bm, nKB)
    bits = _unpack(bm, nKB)
    assert (n_exact == bits.sum(-1)).all()
    for pos in np.ndindex(bits.shape[:-1]):
        expect = np.flatnonzero(bits[pos])
        assert (idx[pos][:expect.size] == expect).all() and (idx[pos][expect.size:] == -1).all()
    assert (_unpack(keep, nKB) == ~bits).all()
    pad = keep.shape[-1] * 32 - nKB
    if pad:
        assert ((keep[..., -1] >> np.uint32(32 - pad)) == 0).all()


def test_route_prep_padding_ignored_and_all_ones():
    nKB = 37
    bm = W.gen_bitmask(42, 1, 2, 4, nKB, 9)
    junk = bm.copy()
    junk[..., -1] |= np.uint32((0xFFFFFFFF << (nKB - 32)) & 0xFFFFFFFF)
    a, b = oracle.route_prep(bm, nKB), oracle.route_prep(junk, nKB)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))
    ones = np.full_like(bm, 0xFFFFFFFF)
    n_exact, idx, keep = oracle.route_prep(ones, nKB)
    assert (n_exact == nKB).all() and (idx == np.arange(nKB)).all() and (keep == 0).all()


@pytest.mark.parametrize("nKB", [1, 31, 33, 128, 255])
def test_bsr_route_matches_bitmask_route(nKB):
    # "Bitmask format": BSR and bitmap inputs prepare into the same route stream and give
    # bitwise-identical results.
    bm = W.gen_bitmask(44, 2, 3, 5, nKB, max(1, nKB // 4), garbage_padding=True)
    indptr, indices = W.bitmask_to_bsr(bm, nKB)
    ref = oracle.route_prep(bm, nKB)
    n_exact, idx, keep, bad = oracle.bsr_route_prep(indptr, indices, nKB)
    assert bad == 0
    for x, y in zip(ref, (n_exact, idx, keep)):
        assert np.array_equal(x.reshape(y.shape), y)


def test_bsr_route_worked_example():
    # Three rows over nKB = 40 blocks (W = 2 words, 8 valid bits in the second):
    #   row 0: {0, 5, 39}, canonical;  row 1: empty;  row 2: [33, 2, 2, 40, -1] -> {2, 33}, not
    #   canonical (unsorted, duplicate, two entries out of range).
    indptr = np.array([0, 3, 3, 8], np.int32)
    indices = np.array([0, 5, 39, 33, 2, 2, 40, -1], np.int32)
    n_exact, idx, keep, bad = oracle.bsr_route_prep(indptr, indices, 40)
    assert n_exact.tolist() == [3, 0, 2]
    assert idx[0, :4].tolist() == [0, 5, 39, -1] and (idx[1] == -1).all()
    assert idx[2, :3].tolist() == [2, 33, -1] and (idx[:, 3:] == -1).all()
    assert keep.tolist() == [[0xFFFFFFDE, 0x7F], [0xFFFFFFFF, 0xFF], [0xFFFFFFFB, 0xFD]]
    assert bad == 1


def test_bsr_route_rows_are_sets():
    # Shuffling a row, repeating an entry or adding out-of-range entries leaves its route unchanged;
    # exactly those rows are reported as non-canonical.
    nKB = 70
    bm = W.gen_bitmask(45, 1, 4, 9, nKB, 20)
    indptr, indices = W.bitmask_to_bsr(bm, nKB)
    ref = oracle.bsr_route_prep(indptr, indices, nKB)
    ip2, ix2, scrambled = W.scramble_bsr(46, indptr, indices, nKB)
    got = oracle.bsr_route_prep(ip2, ix2, nKB)
    assert scrambled.any() and not scrambled.all()
    assert got[3] == int(scrambled.sum())
    for x, y in zip(ref[:3], got[:3]):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("indptr,indices,exact", [
    ([0, 3], [1, 1, 4], [1, 4]),     # ascending, one entry repeated
    ([0, 2], [2, 8], [2]),           # ascending, the last entry one past the final block
    ([0, 2], [-1, 3], [3]),          # ascending, a negative entry
    ([0, 2], [5, 2], [2, 5]),        # distinct and in range, but descending
    ([-1, 2], [3, 6], [3, 6]),       # a negative start pointer, clamped to 0
])
def test_bsr_route_each_defect_alone_makes_the_row_non_canonical(indptr, indices, exact):
    # "Bitmask format": a canonical row is strictly ascending and in range, so each defect on its
    # own is counted, while the route is that of the set the row names.
    got = oracle.bsr_route_prep(np.array(indptr, np.int32), np.array(indices, np.int32), 8)
    ref = oracle.bsr_route_prep(np.array([0, len(exact)], np.int32), np.array(exact, np.int32), 8)
    assert got[3] == 1 and ref[3] == 0
    assert got[0].tolist() == [len(exact)] and got[1][0, :len(exact)].tolist() == exact
    for x, y in zip(ref[:3], got[:3]):
        assert np.array_equal(x, y)


def test_bsr_route_bad_pointers_are_clamped():
    # A reversed pointer pair is an empty row; a range past nnz is cut at nnz.  Both are counted.
    indptr = np.array([0, 2, 1, 4], np.int32)
    indices = np.array([1, 3, 5], np.int32)
    n_exact, idx, keep, bad = oracle.bsr_route_prep(indptr, indices, 8)
    assert n_exact.tolist() == [2, 0, 2]
    assert idx[0, :2].tolist() == [1, 3] and idx[2, :2].tolist() == [3, 5]
    assert bad == 2


def _proxy(q, k, v, bm, Bq, Bk, use_proxy, km=None, vs=None):
    if km is None:
        km, vs = W.block_summaries(k, v, Bk)
    D = q.shape[-1]
    return oracle.proxy_fwd(q, k, v, km, vs, bm, block_q=Bq, block_k=Bk, scale=1 / math.sqrt(D),
                            use_proxy=use_proxy)


@pytest.mark.parametrize("S", [256, 257])
def test_all_ones_bitmap_is_dense(S):
    Bq = Bk = 64
    q, k, v = W.gen_iid(43, 1, S, S, 2, 1, 32)
    nQB, nKB = -(-S // Bq), -(-S // Bk)
    bm = np.full((1, 1, nQB, -(-nKB // 32)), 0xFFFFFFFF, np.uint32)
    ref = refs.sdpa(q, k, v, 1 / math.sqrt(32))
    for use_proxy in (0, 1):
        o, lse = _proxy(q, k, v, bm, Bq, Bk, use_proxy)
        assert np.abs(o - ref).max() < 1e-12
        assert np.abs(lse - refs.lse(q, k, 1 / math.sqrt(32), np.ones((1, 2, S, S), bool))).max() < 1e-12


@pytest.mark.parametrize("S,Bk", [(257, 64), (256, 64), (255, 1), (300, 128)])
def test_block_constant_keys_make_proxy_exact(S, Bk):
    """With K constant over each block and V sums exact in bf16, proxies are exact."""
    rng = np.random.default_rng(44)
    Bq, Hq, Hkv, D = 64, 2, 1, 16
    nKB = -(-S // Bk)
    kb = rng.standard_normal((1, nKB, Hkv, D)).astype(np.float32)
    k = W.to_bf16_bits(np.repeat(kb, Bk, axis=1)[:, :S])
    v = W.to_bf16_bits(rng.integers(-1, 2, (1, S, Hkv, D)).astype(np.float32))
    q = W.to_bf16_bits(rng.standard_normal((1, S, Hq, D)).astype(np.float32))
    km, vs = W.block_summaries(k, v, Bk)
    assert np.array_equal(km, W.to_bf16_bits(kb.transpose(0, 2, 1, 3)))
    nQB = -(-S // Bq)
    bm = W.gen_bitmask(45, 1, Hkv, nQB, nKB, max(1, nKB // 4))
    o, lse = _proxy(q, k, v, bm, Bq, Bk, 1, km, vs)
    ref = refs.sdpa(q, k, v, 1 / math.sqrt(D))
    assert np.abs(o - ref).max() < 1e-12
    assert np.abs(lse - refs.lse(q, k, 1 / math.sqrt(D), np.ones((1, Hq, S, S), bool))).max() < 1e-12


def test_block_size_one_is_dense():
    S = 70
    q, k, v = W.gen_iid(46, 1, S, S, 2, 2, 16)
    bm = W.gen_bitmask(46, 1, 2, -(-S // 16), S, 10)
    o, _ = _proxy(q, k, v, bm, 16, 1, 1)
    assert np.abs(o - refs.sdpa(q, k, v, 0.25)).max() < 1e-12


@pytest.mark.parametrize("S", [256, 257])
def test_proxy_off_is_exact_blocks_only(S):
    Bq = Bk = 64
    q, k, v = W.gen_iid(47, 1, S, S, 2, 2, 32)
    nQB, nKB = -(-S // Bq), -(-S // Bk)
    bm = W.gen_bitmask(47, 1, 2, nQB, nKB, 2, garbage_padding=True)
    o, lse = _proxy(q, k, v, bm, Bq, Bk, 0)
    bits = _unpack(bm, nKB)                       # [1, Hkv, nQB, nKB]
    mask = bits[:, :, np.arange(S) // Bq][:, :, :, np.arange(S) // Bk]
    ref = refs.sdpa(q, k, v, 1 / math.sqrt(32), mask=mask)
    assert np.abs(o - ref).max() < 1e-12
    assert np.abs(lse - refs.lse(q, k, 1 / math.sqrt(32), mask)).max() < 1e-12


def test_proxy_off_never_reads_the_summaries():
    # "Description": omitted blocks are approximated only when the proxy is on.  With it off the
    # output is the exact blocks' attention whatever the summaries hold -- here summaries whose
    # logits would dwarf every exact score, so using them anywhere (even for the reference max)
    # changes the result.
    S, Bq, Bk = 200, 64, 64
    q, k, v = W.gen_iid(48, 1, S, S, 2, 2, 32)
    nQB, nKB = -(-S // Bq), -(-S // Bk)
    bm = W.gen_bitmask(48, 1, 2, nQB, nKB, 2, garbage_padding=True)
    km, vs = W.block_summaries(k, v, Bk)
    qsum = refs.f64(q).sum(axis=(0, 1, 2))            # a direction every query leans along
    huge = np.broadcast_to(np.sign(qsum) * 2000.0, km.shape)
    km_big = W.to_bf16_bits(huge)
    vs_big = W.to_bf16_bits(np.full(vs.shape, 1000.0))
    o_a, lse_a = _proxy(q, k, v, bm, Bq, Bk, 0, km, vs)
    o_b, lse_b = _proxy(q, k, v, bm, Bq, Bk, 0, km_big, vs_big)
    assert np.array_equal(o_a, o_b) and np.array_equal(lse_a, lse_b)
    assert np.isfinite(lse_a).all()


def test_proxy_changes_output_and_padding_is_ignored():
    S, Bq, Bk = 257, 64, 64
    q, k, v = W.gen_iid(48, 1, S, S, 1, 1, 32)
    nQB, nKB = -(-S // Bq), -(-S // Bk)
    bm = W.gen_bitmask(48, 1, 1, nQB, nKB, 2)
    junk = bm.copy()
    junk[..., -1] |= np.uint32((0xFFFFFFFF << nKB) & 0xFFFFFFFF)
    o1, _ = _proxy(q, k, v, bm, Bq, Bk, 1)
    o2, _ = _proxy(q, k, v, junk, Bq, Bk, 1)
    o0, _ = _proxy(q, k, v, bm, Bq, Bk, 0)
    assert np.array_equal(o1, o2)
    assert np.abs(o1 - o0).max() > 1e-3


def test_empty_row_without_proxy():
    S = 128
    q, k, v = W.gen_iid(49, 1, S, S, 1, 1, 16)
    bm = np.zeros((1, 1, 2, 1), np.uint32)
    bm[0, 0, 1, 0] = 1
    o, lse = _proxy(q, k, v, bm, 64, 64, 0)
    assert (o[0, :64] == 0).all() and np.isneginf(lse[0, 0, :64]).all()
    assert np.isfinite(lse[0, 0, 64:]).all()
