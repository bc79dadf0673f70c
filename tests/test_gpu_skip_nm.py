"""GPU parity of sa_skip_nm_softmax_fwd (skip-softmax with N:M inside kept tiles) against the
oracle (needs an MI355X).

For every case the GPU runs with all exports on, then:
  * the tile states equal those of sa_skip_softmax_fwd and the keep bits those of
    sa_nm_softmax_fwd on the same inputs (the group maximum survives top-N, so the combined
    kernel decides exactly as the skip kernel does);
  * replay: fed the GPU's fp32 tile maxima and scores, the oracle's tile states and keep bits
    equal the GPU's bit for bit;
  * independent: the oracle's float64 tile decisions agree on >= 99.9 % of visited tiles;
  * output: the oracle, forced onto the GPU's tile states and keep bits, matches O within max-abs
    2e-2 / mean-abs 2e-3 and the LSE within 2e-3; counters equal the tile_state histogram;
  * the same call without the debug exports (the N:M filter then runs on kept tiles only) gives
    the same tile states and matches the same oracle output.
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


def run_gpu(q, k, v, causal, Br, lam, n, m, sink, recent, Bc=64):
    B, Sq, Hq, D = q.shape
    Sk = k.shape[1]
    nQT, nKT, Wd = -(-Sq // Br), -(-Sk // Bc), -(-Sk // 32)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    o = torch.full((B, Sq, Hq, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    st = torch.full((B, Hq, nQT, nKT), 255, dtype=torch.uint8, device="cuda")
    cnt = torch.zeros((B, Hq, 2), dtype=torch.int32, device="cuda")
    lse = torch.full((B, Hq, Sq), float("nan"), device="cuda")
    rm = torch.empty((B, Hq, nQT, nKT, Br), device="cuda")
    bits = torch.full((B, Hq, Sq, Wd), -1, dtype=torch.int32, device="cuda")
    sc = torch.full((B, Hq, Sq, Sk), float("nan"), device="cuda")
    sa.sa_skip_nm_softmax_fwd(qd, kd, vd, o, lam, n, m, sink, recent, causal=causal, block_q=Br,
                              block_k=Bc, tile_state=st, head_counters=cnt, lse=lse, dbg_tile_rowmax=rm,
                              dbg_keep_bits=bits, dbg_scores=sc)
    # the two separate kernels on the same inputs
    st_skip = torch.full_like(st, 255)
    sa.sa_skip_softmax_fwd(qd, kd, vd, torch.empty_like(o), lam, causal=causal, block_q=Br,
                           block_k=Bc, tile_state=st_skip)
    bits_nm = torch.full_like(bits, -1)
    sa.sa_nm_softmax_fwd(qd, kd, vd, torch.empty_like(o), n, m, sink, recent, causal=causal,
                         block_q=Br, dbg_keep_bits=bits_nm)
    torch.cuda.synchronize()
    return dict(o=from_dev_bf16(o), st=st.cpu().numpy(), cnt=cnt.cpu().numpy(),
                lse=lse.cpu().numpy(), rm=rm.cpu().numpy(),
                bits=bits.cpu().numpy().view(np.uint32), sc=sc.cpu().numpy(),
                st_skip=st_skip.cpu().numpy(), bits_nm=bits_nm.cpu().numpy().view(np.uint32))


def run_gpu_plain(q, k, v, causal, Br, lam, n, m, sink, recent, Bc=64):
    """The combined kernel with no debug exports: O, tile states and LSE only."""
    B, Sq, Hq, D = q.shape
    nQT, nKT = -(-Sq // Br), -(-k.shape[1] // Bc)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    o = torch.full((B, Sq, Hq, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    st = torch.full((B, Hq, nQT, nKT), 255, dtype=torch.uint8, device="cuda")
    lse = torch.full((B, Hq, Sq), float("nan"), device="cuda")
    sa.sa_skip_nm_softmax_fwd(qd, kd, vd, o, lam, n, m, sink, recent, causal=causal, block_q=Br,
                              block_k=Bc, tile_state=st, lse=lse)
    torch.cuda.synchronize()
    return from_dev_bf16(o), st.cpu().numpy(), lse.cpu().numpy()


def check(q, k, v, causal, Br, lam, n, m, sink, recent, tag, Bc=64):
    announce(f"skip+nm {tag} lam={lam} {n}:{m} sink={sink} recent={recent} Bc={Bc}")
    D = q.shape[-1]
    g = run_gpu(q, k, v, causal, Br, lam, n, m, sink, recent, Bc)
    st = g["st"]
    assert np.array_equal(st, g["st_skip"]), "tile states differ from the skip kernel's"
    assert np.array_equal(g["bits"], g["bits_nm"]), "keep bits differ from the N:M kernel's"
    assert (g["cnt"][..., 0] == (st != 2).sum(-1).sum(-1)).all()
    assert (g["cnt"][..., 1] == (st == 1).sum(-1).sum(-1)).all()
    kw = dict(causal=causal, block_q=Br, block_k=Bc, scale=1 / math.sqrt(D), lam=lam, n=n, m=m,
              sink=sink, recent=recent)
    _, _, st_r, _, kb_r = oracle.skip_nm_softmax(q, k, v, mode=1, rowmax_in=g["rm"],
                                                 scores_in=g["sc"], **kw)
    assert np.array_equal(st_r, st), "replayed tile states differ"
    assert np.array_equal(kb_r, g["bits"]), "replayed keep bits differ"
    _, _, st_i, _, _ = oracle.skip_nm_softmax(q, k, v, **kw)
    visited = st != 2
    assert np.array_equal(st_i == 2, ~visited)
    agree = (st_i[visited] == st[visited]).mean()
    assert agree >= 0.999, f"independent agreement {agree:.5f}"
    o_ref, lse_ref, _, _, _ = oracle.skip_nm_softmax(q, k, v, mode=2, state_in=st,
                                                     keep_in=g["bits"], **kw)
    assert_output_parity(g["o"], o_ref, tag)
    lmx, _ = err(g["lse"], lse_ref)
    assert lmx < 2e-3, f"lse {lmx}"
    # without the debug exports the N:M filter runs on kept tiles only (the production launch):
    # the same decisions, and the oracle's output on them
    o2, st2, lse2 = run_gpu_plain(q, k, v, causal, Br, lam, n, m, sink, recent, Bc)
    assert np.array_equal(st2, st), "tile states differ without the exports"
    assert_output_parity(o2, o_ref, tag + " (no exports)")
    lmx, _ = err(lse2, lse_ref)
    assert lmx < 2e-3, f"lse without exports {lmx}"
    return st


@pytest.mark.parametrize("n,m", [(2, 4), (1, 4), (3, 8)])
@pytest.mark.parametrize("lam", [0.0, 1.0, 1.5127145])
def test_llm_causal_gqa(n, m, lam):
    q, k, v = W.gen_llm(21, 1, 1024, 4, 2, 128)
    st = check(q, k, v, True, 128, lam, n, m, 4, 128, "llm causal gqa s1024")
    if lam >= 1.0:
        assert (st == 1).sum() > 0


@pytest.mark.parametrize("shape", [
    # (B, Sq, Sk, Hq, Hkv, D, causal, Br)
    (1, 200, 300, 2, 2, 128, False, 128),    # ragged tiles, Sq != Sk, partial last group
    (2, 130, 130, 4, 1, 128, True, 128),     # 2-row last tile, GQA 4:1
    (1, 257, 257, 2, 2, 64, True, 64),       # D 64, Br 64, 1-row last tile
    (1, 1, 1, 1, 1, 128, True, 128),         # single token
    (2, 200, 200, 20, 10, 64, True, 128),    # causal work order in blocks of 2 KV heads, GQA 2:1
])
@pytest.mark.parametrize("n,m", [(2, 4), (5, 8)])
def test_edge_shapes(shape, n, m):
    B, Sq, Sk, Hq, Hkv, D, causal, Br = shape
    if causal:
        q, k, v = W.gen_llm(22, B, Sq, Hq, Hkv, D)
    else:
        q, k, v = W.gen_iid(22, B, Sq, Sk, Hq, Hkv, D)
    check(q, k, v, causal, Br, 0.9, n, m, 4, 16, f"edge {shape}")


def test_video_non_causal():
    q, k, v = W.gen_video(23, 1, 2, 128, grid=(3, 10, 20))
    st = check(q, k, v, False, 128, 0.378, 2, 4, 0, 0, "video grid 3x10x20")
    assert (st == 1).sum() > 0


@pytest.mark.parametrize("n,m", [(2, 4), (3, 8)])
@pytest.mark.parametrize("lam", [0.0, 1.0, 3.0])
@pytest.mark.parametrize("Br", [64, 128])
def test_block_k_128(n, m, lam, Br):
    """The pages' bc = 128: 128-key decision tiles over the N:M-masked logits."""
    q, k, v = W.gen_llm(24, 1, 1000, 4, 2, 128)
    st = check(q, k, v, True, Br, lam, n, m, 4, 128, "llm causal gqa s1000", Bc=128)
    if lam >= 3.0:
        assert (st == 1).sum() > 0
