"""Parity at the full sizes of the benchmarked workloads, in the launch configuration bench.py
times (same shapes, tiles, thresholds and exports), on an MI355X.

The GPU computes every query tile.
  * replay, over the WHOLE tensor: fed the GPU's fp32 tile maxima (skip) or scores (N:M), the
    oracle's decisions-only replay must reproduce every tile state and every keep bit;
the float64 oracle recomputes a seeded sample of query tiles (plus the first and the last, which
holds the ragged tail) in two more ways:
  * independent: its own float64 decisions agree with the GPU's on >= 99.9 % of the sample;
  * forced: given the GPU's decisions, its O matches within max-abs 2e-2 / mean-abs 2e-3 and its
    LSE within 2e-3.
Properties that hold at any size are checked on everything: tile_state values, head counters
equal to the tile_state histogram, route prep bit-exact on every bitmap row.

The exported maxima and scores are copied to the host a chunk (of units, or of one head) at a
time.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import announce, assert_output_parity, err, from_dev_bf16, to_dev

pytestmark = pytest.mark.gpu

sa = pytest.importorskip("sparse_attention_flash_amd")

N_SAMPLE = 32   # query tiles recomputed by the oracle per case (plus the first and the last)


def sample_units(total, seed):
    rng = np.random.default_rng(seed)
    pick = rng.choice(total, size=min(N_SAMPLE, total), replace=False)
    return np.unique(np.concatenate([[0, total - 1], pick])).astype(np.int64)


def o_rows(o, units, Hq, nQT, Br, Sq):
    """GPU output rows of the sampled units as [n, Br, D] (rows past Sq left at 0)."""
    D = o.shape[-1]
    out = np.zeros((units.size, Br, D))
    for i, u in enumerate(units):
        b, rest = divmod(int(u), Hq * nQT)
        h, qt = divmod(rest, nQT)
        r0, r1 = qt * Br, min(Sq, qt * Br + Br)
        out[i, : r1 - r0] = o[b, r0:r1, h]
    return out


def row_valid(units, Hq, nQT, Br, Sq):
    qt = units % nQT
    rows = qt[:, None] * Br + np.arange(Br)[None, :]
    return rows < Sq


def replay_all_skip_states(rm, state, *, B, Hq, Sq, Sk, causal, Br, Bc, lam, chunk=1024):
    """Replay the skip decisions of EVERY unit from the GPU's exported fp32 tile maxima (the
    oracle's decisions-only replay, no dot products), a chunk of units at a time; returns the
    number of visited tiles replayed."""
    nQT, nKT = -(-Sq // Br), -(-Sk // Bc)
    total = B * Hq * nQT
    flat = state.reshape(total, nKT)
    replayed = 0
    for u0 in range(0, total, chunk):
        units = np.arange(u0, min(total, u0 + chunk), dtype=np.int64)
        rm_h = rm[u0:u0 + units.size].cpu().numpy()
        st = oracle.skip_replay(rm_h, batch=B, heads_q=Hq, seqlen_q=Sq, seqlen_k=Sk,
                                causal=causal, block_q=Br, block_k=Bc, lam=lam, units=units)
        bad = np.argwhere(st != flat[units])
        assert bad.size == 0, f"replayed decisions differ at (unit, tile) {bad[:5] + [u0, 0]}"
        replayed += int((st != 2).sum())
    return replayed


def replay_all_nm_bits(sc, bits, *, B, Hq, Sq, causal, n, m, sink, recent):
    """Replay the N:M keep bits of EVERY row from the GPU's exported fp32 scores, one (batch,
    head) at a time (the oracle's keep rule alone, no dot products)."""
    pos = np.arange(Sq, dtype=np.int32)
    for b in range(B):
        for h in range(Hq):
            kb = oracle.nm_keep_replay(sc[b, h].cpu().numpy(), pos, seqlen_q=Sq, causal=causal,
                                       n=n, m=m, sink=sink, recent=recent)
            got = bits[b, h].cpu().numpy().view(np.uint32)
            assert np.array_equal(kb, got), f"replayed keep bits differ at batch {b} head {h}"


@pytest.mark.parametrize("name,target", [("video_dit_s32760", 0.5), ("video_dit_s32760", 0.7),
                                         ("video_dit_s32760", None),
                                         ("llm_prefill_gqa_s8192", 0.5),
                                         ("llm_prefill_gqa_s8192", None)])
def test_skip_softmax_full_size(name, target):
    """target None: lambda = 0, the dense arm the benchmark times beside each threshold."""
    wl = W.WORKLOADS[name]
    announce(f"skip full size {name} target={target}")
    q, k, v = wl.generate()
    B, Sq, Hq, D = q.shape
    Sk = k.shape[1]
    Br, Bc = wl.block_q, wl.block_k
    nQT, nKT = -(-Sq // Br), -(-Sk // Bc)
    lam = 0.0 if target is None else sa.sa_threshold_from_calib(W.CALIB_A, W.CALIB_B, target,
                                                                 Sk)[1]
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    o = torch.empty_like(qd)
    st = torch.full((B, Hq, nQT, nKT), 255, dtype=torch.uint8, device="cuda")
    cnt = torch.zeros((B, Hq, 2), dtype=torch.int32, device="cuda")
    lse = torch.empty((B, Hq, Sq), device="cuda")
    rm = torch.empty((B * Hq * nQT, nKT, Br), device="cuda")
    sa.sa_skip_softmax_fwd(qd, kd, vd, o, lam, causal=wl.causal, block_q=Br, block_k=Bc,
                           tile_state=st, head_counters=cnt, lse=lse, dbg_tile_rowmax=rm)
    torch.cuda.synchronize()
    state = st.cpu().numpy()
    counts = cnt.cpu().numpy()
    assert set(np.unique(state)) <= {0, 1, 2}
    assert (counts[..., 0] == (state != 2).sum((-1, -2))).all()
    assert (counts[..., 1] == (state == 1).sum((-1, -2))).all()
    visited = (state != 2).sum()
    if target is None:
        assert (state == 1).sum() == 0, "lambda = 0 never skips"
    else:
        assert 0 < (state == 1).sum() < visited, "the calibrated threshold skips some tiles, not all"

    # every visited tile of the tensor, replayed bit for bit
    replayed = replay_all_skip_states(rm, state, B=B, Hq=Hq, Sq=Sq, Sk=Sk, causal=wl.causal,
                                      Br=Br, Bc=Bc, lam=lam)
    assert replayed == visited
    del rm

    units = sample_units(B * Hq * nQT, wl.seed)
    kw = dict(causal=wl.causal, block_q=Br, block_k=Bc, scale=wl.scale, lam=lam, units=units)
    flat = state.reshape(-1, nKT)[units]
    _, _, st_ind, _ = oracle.skip_softmax(q, k, v, mode=0, **kw)
    vis = flat != 2
    assert np.array_equal(st_ind != 2, vis)
    agree = (st_ind[vis] == flat[vis]).mean()
    assert agree >= 0.999, f"independent decision agreement {agree:.5f}"

    o_ref, lse_ref, _, _ = oracle.skip_softmax(q, k, v, mode=2, state_in=state, **kw)
    valid = row_valid(units, Hq, nQT, Br, Sq)
    got = o_rows(from_dev_bf16(o), units, Hq, nQT, Br, Sq)
    assert_output_parity(got[valid], o_ref[valid], f"{name} O")
    lse_h = lse.cpu().numpy().reshape(B * Hq, Sq)
    lse_got = np.zeros((units.size, Br))
    for i, u in enumerate(units):
        bh, qt = divmod(int(u), nQT)
        r0, r1 = qt * Br, min(Sq, qt * Br + Br)
        lse_got[i, : r1 - r0] = lse_h[bh, r0:r1]
    assert err(lse_got[valid], lse_ref[valid])[0] < 2e-3
    assert np.isfinite(lse.cpu().numpy()).all()


def sampled_bits(keep_all, units, Hq, nQT, Br, Sq, Wd):
    gpu_bits = np.zeros((units.size, Br, Wd), np.uint32)
    for i, u in enumerate(units):
        bh, qt = divmod(int(u), nQT)
        b, h = divmod(bh, Hq)
        r0, r1 = qt * Br, min(Sq, qt * Br + Br)
        gpu_bits[i, : r1 - r0] = keep_all[b, h, r0:r1]
    return gpu_bits


def lse_rows(lse_h, units, Hq, nQT, Br, Sq):
    lse_got = np.zeros((units.size, Br))
    for i, u in enumerate(units):
        bh, qt = divmod(int(u), nQT)
        b, h = divmod(bh, Hq)
        r0, r1 = qt * Br, min(Sq, qt * Br + Br)
        lse_got[i, : r1 - r0] = lse_h[b, h, r0:r1]
    return lse_got


# every (n, m) the benchmark times on this workload, and 3:8
@pytest.mark.parametrize("n,m", [(2, 4), (4, 4), (1, 4), (3, 4), (1, 8), (3, 8), (4, 8), (7, 8)])
def test_nm_softmax_full_size(n, m):
    wl = W.WORKLOADS["llm_prefill_nm_s4096"]
    announce(f"nm full size {n}:{m}")
    q, k, v = wl.generate()
    B, Sq, Hq, D = q.shape
    Sk = k.shape[1]
    Br = wl.block_q
    nQT, Wd = -(-Sq // Br), -(-Sk // 32)
    sink, recent = wl.param("sink"), wl.param("recent")
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    o = torch.empty_like(qd)
    lse = torch.empty((B, Hq, Sq), device="cuda")
    bits = torch.empty((B, Hq, Sq, Wd), dtype=torch.int32, device="cuda")
    sc = torch.empty((B, Hq, Sq, Sk), device="cuda")
    sa.sa_nm_softmax_fwd(qd, kd, vd, o, n, m, sink, recent, causal=True, block_q=Br,
                         block_k=wl.block_k, lse=lse, dbg_keep_bits=bits, dbg_scores=sc)
    torch.cuda.synchronize()
    # every row of the tensor, replayed bit for bit
    replay_all_nm_bits(sc, bits, B=B, Hq=Hq, Sq=Sq, causal=True, n=n, m=m, sink=sink,
                       recent=recent)
    del sc

    units = sample_units(B * Hq * nQT, wl.seed + n * 10 + m)
    keep_all = bits.cpu().numpy().view(np.uint32)
    kw = dict(causal=True, scale=wl.scale, n=n, m=m, sink=sink, recent=recent, block_q=Br,
              units=units)
    valid = row_valid(units, Hq, nQT, Br, Sq)
    gpu_bits = sampled_bits(keep_all, units, Hq, nQT, Br, Sq, Wd)
    _, _, kb_ind = oracle.nm_softmax(q, k, v, mode=0, **kw)
    agree = (np.unpackbits(kb_ind[valid].view(np.uint8)) ==
             np.unpackbits(gpu_bits[valid].view(np.uint8))).mean()
    assert agree >= 0.999, f"independent keep agreement {agree:.5f}"
    o_ref, lse_ref, _ = oracle.nm_softmax(q, k, v, mode=2, keep_in=keep_all, **kw)
    got = o_rows(from_dev_bf16(o), units, Hq, nQT, Br, Sq)
    assert_output_parity(got[valid], o_ref[valid], f"N:M {n}:{m} O")
    lse_got = lse_rows(lse.cpu().numpy(), units, Hq, nQT, Br, Sq)
    assert err(lse_got[valid], lse_ref[valid])[0] < 2e-3


@pytest.mark.parametrize("target", [0.5, None])
def test_skip_nm_full_size(target):
    """Skip-softmax with 2:4 inside kept tiles on the N:M workload at the two thresholds the
    benchmark times: target 0.5 lowered through the pages' model, and lambda = 0 (None)."""
    wl = W.WORKLOADS["llm_prefill_nm_s4096"]
    announce(f"skip + 2:4 full size target={target}")
    q, k, v = wl.generate()
    B, Sq, Hq, D = q.shape
    Sk = k.shape[1]
    Br, Bc = wl.block_q, wl.block_k
    nQT, nKT, Wd = -(-Sq // Br), -(-Sk // Bc), -(-Sk // 32)
    sink, recent = wl.param("sink"), wl.param("recent")
    lam = 0.0 if target is None else sa.sa_threshold_from_calib(W.CALIB_A, W.CALIB_B, target,
                                                                 Sk)[1]
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    o = torch.empty_like(qd)
    st = torch.full((B, Hq, nQT, nKT), 255, dtype=torch.uint8, device="cuda")
    cnt = torch.zeros((B, Hq, 2), dtype=torch.int32, device="cuda")
    lse = torch.empty((B, Hq, Sq), device="cuda")
    rm = torch.empty((B * Hq * nQT, nKT, Br), device="cuda")
    bits = torch.empty((B, Hq, Sq, Wd), dtype=torch.int32, device="cuda")
    sc = torch.empty((B, Hq, Sq, Sk), device="cuda")
    sa.sa_skip_nm_softmax_fwd(qd, kd, vd, o, lam, 2, 4, sink, recent, causal=True, block_q=Br,
                              block_k=Bc, tile_state=st, head_counters=cnt, lse=lse,
                              dbg_tile_rowmax=rm, dbg_keep_bits=bits, dbg_scores=sc)
    torch.cuda.synchronize()
    state = st.cpu().numpy()
    counts = cnt.cpu().numpy()
    assert (counts[..., 0] == (state != 2).sum((-1, -2))).all()
    assert (counts[..., 1] == (state == 1).sum((-1, -2))).all()
    if target is None:
        assert (state == 1).sum() == 0
    else:
        assert 0 < (state == 1).sum() < (state != 2).sum()
    # every visited tile and every row, replayed bit for bit (the combined rule decides tiles on
    # the same maxima as skip-softmax alone and gates keys by the N:M bits)
    replay_all_skip_states(rm, state, B=B, Hq=Hq, Sq=Sq, Sk=Sk, causal=True, Br=Br, Bc=Bc,
                           lam=lam)
    replay_all_nm_bits(sc, bits, B=B, Hq=Hq, Sq=Sq, causal=True, n=2, m=4, sink=sink,
                       recent=recent)
    del rm, sc

    # the launch the benchmark times: no debug exports, so the N:M filter runs on kept tiles only;
    # its decisions and outputs are those of the exporting run, bit for bit
    o_run = torch.empty_like(qd)
    st_run = torch.full_like(st, 255)
    lse_run = torch.empty_like(lse)
    sa.sa_skip_nm_softmax_fwd(qd, kd, vd, o_run, lam, 2, 4, sink, recent, causal=True,
                              block_q=Br, block_k=Bc, tile_state=st_run, lse=lse_run)
    torch.cuda.synchronize()
    assert np.array_equal(st_run.cpu().numpy(), state)
    assert torch.equal(o_run.view(torch.int16), o.view(torch.int16))
    assert torch.equal(lse_run, lse)

    units = sample_units(B * Hq * nQT, wl.seed + 77)
    keep_all = bits.cpu().numpy().view(np.uint32)
    kw = dict(causal=True, block_q=Br, block_k=Bc, scale=wl.scale, lam=lam, n=2, m=4, sink=sink,
              recent=recent, units=units)
    flat = state.reshape(-1, nKT)[units]
    valid = row_valid(units, Hq, nQT, Br, Sq)
    _, _, st_i, _, _ = oracle.skip_nm_softmax(q, k, v, mode=0, **kw)
    vis = flat != 2
    assert (st_i[vis] == flat[vis]).mean() >= 0.999
    o_ref, lse_ref, _, _, _ = oracle.skip_nm_softmax(q, k, v, mode=2, state_in=state,
                                                     keep_in=keep_all, **kw)
    got = o_rows(from_dev_bf16(o_run), units, Hq, nQT, Br, Sq)
    assert_output_parity(got[valid], o_ref[valid], "skip + 2:4 O")
    lse_got = lse_rows(lse_run.cpu().numpy(), units, Hq, nQT, Br, Sq)
    assert err(lse_got[valid], lse_ref[valid])[0] < 2e-3


@pytest.mark.parametrize("name", ["proxy_bitmask_s16257", "proxy_page_s32760"])
def test_proxy_full_size(name):
    wl = W.WORKLOADS[name]
    announce(f"proxy full size {name}")
    q, k, v = wl.generate()
    B, S, H, D = q.shape
    Bq, Bk = wl.block_q, wl.block_k
    nQB, nKB = -(-S // Bq), -(-S // Bk)
    Wd = -(-nKB // 32)
    bm = W.gen_bitmask(wl.seed, B, H, nQB, nKB, int(round(wl.param("density") * nKB)))
    km, vs = W.block_summaries(k, v, Bk)
    bmd = torch.from_numpy(bm.view(np.int32)).to("cuda")
    n_exact = torch.empty((B, H, nQB), dtype=torch.int32, device="cuda")
    idx = torch.empty((B, H, nQB, nKB), dtype=torch.int32, device="cuda")
    keep = torch.empty((B, H, nQB, Wd), dtype=torch.int32, device="cuda")
    sa.sa_bitmask_route_prep(bmd, n_exact, idx, keep, batch=B, heads_kv=H, seqlen_q=S, seqlen_k=S,
                             block_q=Bq, block_k=Bk)
    torch.cuda.synchronize()
    r_ne, r_ix, r_kp = oracle.route_prep(bm, nKB)
    assert np.array_equal(n_exact.cpu().numpy(), r_ne)
    assert np.array_equal(idx.cpu().numpy(), r_ix)
    assert np.array_equal(keep.cpu().numpy().view(np.uint32), r_kp)

    qd, kd, vd, kmd, vsd = to_dev(q), to_dev(k), to_dev(v), to_dev(km), to_dev(vs)
    units = sample_units(B * H * nQB, wl.seed)
    valid = row_valid(units, H, nQB, Bq, S)
    for use in (0, 1):
        o = torch.empty_like(qd)
        lse = torch.empty((B, H, S), device="cuda")
        sa.sa_proxy_block_sparse_fwd(qd, kd, vd, kmd, vsd, n_exact, idx, keep, use, o,
                                     block_q=Bq, block_k=Bk, lse=lse)
        torch.cuda.synchronize()
        o_ref, lse_ref = oracle.proxy_fwd(q, k, v, km, vs, bm, block_q=Bq, block_k=Bk,
                                          scale=1 / math.sqrt(D), use_proxy=use, units=units)
        got = o_rows(from_dev_bf16(o), units, H, nQB, Bq, S)
        assert_output_parity(got[valid], o_ref[valid], f"proxy use={use} O")
        lse_h = lse.cpu().numpy().reshape(B * H, S)
        lse_got = np.zeros((units.size, Bq))
        for i, u in enumerate(units):
            bh, qb = divmod(int(u), nQB)
            r0, r1 = qb * Bq, min(S, qb * Bq + Bq)
            lse_got[i, : r1 - r0] = lse_h[bh, r0:r1]
        assert err(lse_got[valid], lse_ref[valid])[0] < 2e-3
