"""GPU parity of sa_skip_softmax_decode_fwd against the oracle (needs an MI355X).

The decode step is the skip-softmax forward with one query row per head: the oracle runs
oracle.skip_softmax with seqlen_q = 1 and block_q = 1 on each sequence's own keys.  For every case:
  * replay: fed the GPU's fp32 tile maxima, the oracle's decisions equal the GPU's tile states bit
    for bit (this also shows the key-axis split reproduces the sequential running max);
  * independent: the oracle's float64 decisions agree on >= 99.9 % of visited tiles;
  * the exported tile maxima match the oracle's float64 maxima;
  * output: the oracle, forced onto the GPU's tile states, matches O within max-abs 2e-2 /
    mean-abs 2e-3 and the LSE within 2e-3;
  * tiles past a sequence's end are state 2, counters equal the tile_state histogram, and the tile
    states do not depend on the number of splits.
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


def run_gpu(q, k, v, lens, lam, BC, num_splits=0):
    B, _, Hq, D = q.shape
    S = k.shape[1]
    nKT = -(-S // BC)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    o = torch.full((B, 1, Hq, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    st = torch.full((B, Hq, nKT), 255, dtype=torch.uint8, device="cuda")
    cnt = torch.zeros((B, Hq, 2), dtype=torch.int32, device="cuda")
    lse = torch.full((B, Hq), float("nan"), device="cuda")
    rm = torch.full((B, Hq, nKT), float("nan"), device="cuda")
    ln = None if lens is None else torch.from_numpy(lens.astype(np.int32)).to("cuda")
    sa.sa_skip_softmax_decode_fwd(qd, kd, vd, o, lam, block_k=BC, seqlens_k=ln,
                                  num_splits=num_splits, tile_state=st, head_counters=cnt,
                                  lse=lse, dbg_tile_rowmax=rm)
    torch.cuda.synchronize()
    return dict(o=from_dev_bf16(o), st=st.cpu().numpy(), cnt=cnt.cpu().numpy(),
                lse=lse.cpu().numpy(), rm=rm.cpu().numpy())


def check(q, k, v, lens, lam, BC, tag, num_splits=0):
    announce(f"decode {tag} lam={lam} BC={BC} splits={num_splits}")
    B, _, Hq, D = q.shape
    S = k.shape[1]
    g = run_gpu(q, k, v, lens, lam, BC, num_splits)
    st = g["st"]
    assert (g["cnt"][..., 0] == (st != 2).sum(-1)).all()
    assert (g["cnt"][..., 1] == (st == 1).sum(-1)).all()
    kw = dict(causal=False, block_q=1, block_k=BC, scale=1 / math.sqrt(D), lam=lam)
    n_vis = n_agree = 0
    for b in range(B):
        L = S if lens is None else int(lens[b])
        nkt = -(-L // BC)
        assert (st[b, :, nkt:] == 2).all()
        if L == 0:
            assert (g["o"][b] == 0).all() and np.isneginf(g["lse"][b]).all()
            continue
        qb, kb, vb = q[b:b + 1], k[b:b + 1, :L], v[b:b + 1, :L]
        stb = st[b:b + 1, :, None, :nkt]
        _, _, st_r, _ = oracle.skip_softmax(qb, kb, vb, mode=1,
                                            rowmax_in=g["rm"][b:b + 1, :, :nkt], **kw)
        assert np.array_equal(st_r, stb), f"replayed decisions differ (sequence {b})"
        _, _, st_i, rm_i = oracle.skip_softmax(qb, kb, vb, **kw)
        # the exported tile maxima against the oracle's float64 maxima
        rm_g = g["rm"][b, :, :nkt]
        rm_o = rm_i[0, :, 0, :, 0]
        assert np.abs(rm_g - rm_o).max() < 2e-3 * max(1.0, np.abs(rm_o).max()), \
            f"tile maxima differ (sequence {b}): {np.abs(rm_g - rm_o).max():.3e}"
        n_vis += st_i.size
        n_agree += int((st_i == stb).sum())
        o_ref, lse_ref, _, _ = oracle.skip_softmax(qb, kb, vb, mode=2, state_in=stb, **kw)
        assert_output_parity(g["o"][b:b + 1], o_ref, f"{tag} sequence {b}")
        assert err(g["lse"][b], lse_ref[0, :, 0])[0] < 2e-3
    if n_vis:
        assert n_agree / n_vis >= 0.999, f"independent agreement {n_agree / n_vis:.5f}"
    return g


# num_splits 1 takes the whole-sequence kernel (one workgroup per batch and KV head, scores in
# LDS) wherever its scores fit; 0 lets the library choose: the key-axis split (three kernels) for
# lambda <= 1, the whole-sequence kernel for lambda > 1.
@pytest.mark.parametrize("splits", [0, 1])
@pytest.mark.parametrize("lam", [0.0, 0.3, 1.0, 3.0])
@pytest.mark.parametrize("BC", [64, 128])
def test_llm_decode_ragged(lam, BC, splits):
    q, k, v, lens = W.gen_llm_decode(31, 4, 1500, 8, 2, 128)
    lens[1] = 1          # a one-key sequence
    lens[2] = 700        # a ragged last tile
    g = check(q, k, v, lens, lam, BC, "llm gqa 8/2 cap 1500", num_splits=splits)
    if lam >= 1.0:
        assert (g["st"] == 1).sum() > 0


@pytest.mark.parametrize("splits", [1, 3, 7])
def test_split_count_does_not_change_decisions(splits):
    q, k, v, lens = W.gen_llm_decode(32, 2, 2000, 8, 2, 128)
    ref = run_gpu(q, k, v, lens, 0.6, 64, num_splits=1)
    g = check(q, k, v, lens, 0.6, 64, "split invariance", num_splits=splits)
    assert np.array_equal(g["st"], ref["st"])
    assert np.array_equal(g["rm"], ref["rm"])


@pytest.mark.parametrize("splits", [0, 1])
@pytest.mark.parametrize("Hq,Hkv,D", [(4, 4, 128), (16, 2, 128), (32, 2, 128), (8, 1, 64),
                                      (6, 2, 64), (5, 1, 128)])
def test_head_groups_and_head_dims(Hq, Hkv, D, splits):
    q, k, v, lens = W.gen_llm_decode(33, 2, 900, Hq, Hkv, D)
    check(q, k, v, lens, 0.8, 64, f"G={Hq // Hkv} D={D}", num_splits=splits)


@pytest.mark.parametrize("splits", [0, 1])
def test_empty_sequence_and_no_lengths(splits):
    q, k, v, lens = W.gen_llm_decode(34, 3, 300, 4, 2, 128)
    lens[0] = 0
    check(q, k, v, lens, 0.5, 64, "empty sequence", num_splits=splits)
    check(q, k, v, None, 0.5, 64, "no seqlens", num_splits=splits)


def test_whole_sequence_kernel_at_its_size_limit():
    """The largest cache whose scores still fit in LDS (G 4, 8192 keys; G 1, 32768 keys at 128-key
    tiles), one split: the whole-sequence kernel; the split path on the same inputs decides
    identically."""
    for Hq, Hkv, S, BC in ((8, 2, 8192, 64), (2, 2, 32768, 128)):
        q, k, v, lens = W.gen_llm_decode(35, 2, S, Hq, Hkv, 128)
        g = check(q, k, v, lens, 0.7, BC, f"limit G={Hq // Hkv} S={S}", num_splits=1)
        ref = run_gpu(q, k, v, lens, 0.7, BC, num_splits=4)
        assert np.array_equal(g["st"], ref["st"])
        assert np.array_equal(g["rm"], ref["rm"])


def test_full_size_decode_workload():
    wl = W.WORKLOADS["llm_decode_gqa_kv8192"]
    q, k, v, lens = wl.generate()
    for lam in (wl.param("lambda"), 0.5):
        check(q, k, v, lens, lam, wl.block_k, f"{wl.name}")
