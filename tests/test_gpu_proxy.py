"""GPU parity of sa_bitmask_route_prep and sa_bsr_route_prep (bit-exact) and
sa_proxy_block_sparse_fwd (max-abs 2e-2, mean-abs 2e-3 against the float64 oracle), needs an
MI355X."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import announce, assert_output_parity, err, from_dev_bf16, to_dev

pytestmark = pytest.mark.gpu

sa = pytest.importorskip("sparse_attention_flash_amd")


def i32(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int32)).to("cuda")


def route_gpu(bm, B, Hkv, Sq, Sk, Bq, Bk):
    nQB, nKB = -(-Sq // Bq), -(-Sk // Bk)
    Wd = -(-nKB // 32)
    bmd = i32(bm)
    n_exact = torch.full((B, Hkv, nQB), -7, dtype=torch.int32, device="cuda")
    idx = torch.full((B, Hkv, nQB, nKB), -7, dtype=torch.int32, device="cuda")
    keep = torch.full((B, Hkv, nQB, Wd), -7, dtype=torch.int32, device="cuda")
    sa.sa_bitmask_route_prep(bmd, n_exact, idx, keep, batch=B, heads_kv=Hkv, seqlen_q=Sq,
                             seqlen_k=Sk, block_q=Bq, block_k=Bk)
    return n_exact, idx, keep


@pytest.mark.parametrize("S,Bk", [(64, 64), (257, 64), (16257, 128), (16257, 64), (32760, 64),
                                  (300000, 64)])
def test_route_prep_bit_exact(S, Bk):
    announce(f"route prep S={S} Bk={Bk}")
    B, Hkv, Bq = 2, 3, 128
    nQB, nKB = -(-S // Bq), -(-S // Bk)
    nQB = min(nQB, 40)          # rows are independent; a prefix of query blocks suffices
    Sq = nQB * Bq
    bm = W.gen_bitmask(51, B, Hkv, nQB, nKB, max(1, nKB // 4), garbage_padding=True)
    ne, ix, kp = route_gpu(bm, B, Hkv, Sq, S, Bq, Bk)
    torch.cuda.synchronize()
    r_ne, r_ix, r_kp = oracle.route_prep(bm, nKB)
    assert np.array_equal(ne.cpu().numpy(), r_ne)
    assert np.array_equal(ix.cpu().numpy(), r_ix)
    assert np.array_equal(kp.cpu().numpy().view(np.uint32), r_kp)


def bsr_route_gpu(indptr, indices, B, Hkv, Sq, Sk, Bq, Bk):
    nQB, nKB = -(-Sq // Bq), -(-Sk // Bk)
    Wd = -(-nKB // 32)
    n_exact = torch.full((B, Hkv, nQB), -7, dtype=torch.int32, device="cuda")
    idx = torch.full((B, Hkv, nQB, nKB), -7, dtype=torch.int32, device="cuda")
    keep = torch.full((B, Hkv, nQB, Wd), -7, dtype=torch.int32, device="cuda")
    bad = torch.zeros(1, dtype=torch.int32, device="cuda")
    sa.sa_bsr_route_prep(i32(indptr), i32(indices), n_exact, idx, keep, batch=B, heads_kv=Hkv,
                         seqlen_q=Sq, seqlen_k=Sk, block_q=Bq, block_k=Bk, bad_rows=bad)
    return n_exact, idx, keep, bad


@pytest.mark.parametrize("S,Bk", [(64, 64), (257, 64), (16257, 128), (32760, 64), (300000, 64)])
def test_bsr_route_prep_matches_bitmask(S, Bk):
    # "Bitmask format": BSR and bitmap routes are bitwise identical.
    announce(f"bsr route prep S={S} Bk={Bk}")
    B, Hkv, Bq = 2, 3, 128
    nQB, nKB = min(-(-S // Bq), 40), -(-S // Bk)
    Sq = nQB * Bq
    bm = W.gen_bitmask(53, B, Hkv, nQB, nKB, max(1, nKB // 4), garbage_padding=True)
    indptr, indices = W.bitmask_to_bsr(bm, nKB)
    got = bsr_route_gpu(indptr, indices, B, Hkv, Sq, S, Bq, Bk)
    ref = route_gpu(bm, B, Hkv, Sq, S, Bq, Bk)
    torch.cuda.synchronize()
    for x, y in zip(got[:3], ref):
        assert torch.equal(x, y)
    assert int(got[3].item()) == 0


def test_bsr_route_prep_non_canonical_rows():
    announce("bsr route prep, non-canonical rows")
    B, Hkv, Bq, Bk, S = 1, 4, 128, 64, 4500
    nQB, nKB = -(-S // Bq), -(-S // Bk)
    bm = W.gen_bitmask(54, B, Hkv, nQB, nKB, 20)
    indptr, indices = W.bitmask_to_bsr(bm, nKB)
    ip2, ix2, scrambled = W.scramble_bsr(55, indptr, indices, nKB)
    ip2[5], ip2[6] = ip2[6], ip2[5]          # one reversed pointer pair (rows 4 and 5 change)
    ip2[-1] = ix2.size + 3                   # last row runs past nnz: clamped
    ne, ix, kp, bad = bsr_route_gpu(ip2, ix2, B, Hkv, S, S, Bq, Bk)
    torch.cuda.synchronize()
    r_ne, r_ix, r_kp, r_bad = oracle.bsr_route_prep(ip2, ix2, nKB)
    assert np.array_equal(ne.cpu().numpy().ravel(), r_ne)
    assert np.array_equal(ix.cpu().numpy().reshape(r_ix.shape), r_ix)
    assert np.array_equal(kp.cpu().numpy().view(np.uint32).reshape(r_kp.shape), r_kp)
    assert int(bad.item()) == r_bad and r_bad >= int(scrambled.sum())


def run_proxy(q, k, v, bm, Bq, Bk, use_proxy):
    B, S, Hq, D = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    km, vs = W.block_summaries(k, v, Bk)
    ne, ix, kp = route_gpu(bm, B, Hkv, S, Sk, Bq, Bk)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    o = torch.full((B, S, Hq, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, Hq, S), float("nan"), device="cuda")
    sa.sa_proxy_block_sparse_fwd(qd, kd, vd, to_dev(km), to_dev(vs), ne, ix, kp, use_proxy, o,
                                 block_q=Bq, block_k=Bk, lse=lse)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.proxy_fwd(q, k, v, km, vs, bm, block_q=Bq, block_k=Bk,
                                      scale=1 / math.sqrt(D), use_proxy=use_proxy)
    return from_dev_bf16(o), lse.cpu().numpy(), o_ref, lse_ref


@pytest.mark.parametrize("use_proxy", [0, 1])
@pytest.mark.parametrize("cfg", [
    # (B, S, Hq, Hkv, D, Bq, Bk, density)
    (1, 256, 2, 2, 128, 128, 128, 0.5),
    (1, 257, 2, 1, 128, 128, 128, 0.5),     # 1-token final block, GQA
    (1, 257, 2, 2, 128, 64, 64, 0.4),
    (2, 1000, 2, 2, 64, 128, 64, 0.25),
    (1, 2049, 4, 2, 128, 128, 128, 0.25),
    (1, 1000, 2, 2, 64, 64, 64, 0.25),      # head_dim 64, 64-row blocks, even block count
    (2, 777, 4, 2, 128, 64, 128, 0.3),      # 64-row blocks over 128-key blocks, odd block count
])
def test_proxy_parity(cfg, use_proxy):
    B, S, Hq, Hkv, D, Bq, Bk, dens = cfg
    announce(f"proxy {cfg} use_proxy={use_proxy}")
    q, k, v = W.gen_iid(52, B, S, S, Hq, Hkv, D)
    nQB, nKB = -(-S // Bq), -(-S // Bk)
    bm = W.gen_bitmask(52, B, Hkv, nQB, nKB, max(1, int(round(dens * nKB))), garbage_padding=True)
    o, lse, o_ref, lse_ref = run_proxy(q, k, v, bm, Bq, Bk, use_proxy)
    assert_output_parity(o, o_ref, f"proxy {cfg}")
    lmx, _ = err(lse, lse_ref)
    assert lmx < 2e-3


@pytest.mark.parametrize("use_proxy", [0, 1])
@pytest.mark.parametrize("D", [64, 128])
def test_proxy_uneven_routes(D, use_proxy):
    """64-row query blocks run two to a workgroup in lockstep: rows of very different exact-block
    counts (none, one, two, a few, all) side by side, and an odd number of query blocks."""
    B, S, H, Bq, Bk = 1, 1100, 2, 64, 64
    announce(f"proxy uneven routes D={D} use_proxy={use_proxy}")
    q, k, v = W.gen_iid(56, B, S, S, H, H, D)
    nQB, nKB = -(-S // Bq), -(-S // Bk)
    rng = np.random.default_rng(56)
    bits = np.zeros((B, H, nQB, nKB), bool)
    for hh in range(H):
        for qb in range(nQB):
            kind = (qb + hh) % 4
            if kind == 1:   # one or two exact blocks: the shortest step counts
                bits[0, hh, qb, rng.choice(nKB, 1 + (qb // 4) % 2, replace=False)] = True
            elif kind == 2:
                bits[0, hh, qb] = True
            elif kind == 3:
                bits[0, hh, qb, rng.choice(nKB, int(rng.integers(3, nKB)), replace=False)] = True
    W_ = -(-nKB // 32)
    bm = np.zeros((B, H, nQB, W_), np.uint32)
    for j in range(nKB):
        bm[..., j // 32] |= bits[..., j].astype(np.uint32) << np.uint32(j % 32)
    o, lse, o_ref, lse_ref = run_proxy(q, k, v, bm, Bq, Bk, use_proxy)
    fin = np.isfinite(lse_ref)
    assert_output_parity(o, o_ref, f"proxy uneven D={D}")
    assert (np.isneginf(lse) == ~fin).all()
    lmx, _ = err(lse[fin], lse_ref[fin])
    assert lmx < 2e-3


@pytest.mark.parametrize("Bq,Bk", [(128, 64), (64, 64), (128, 128)])
def test_all_ones_is_dense_and_empty_rows_are_zero(Bq, Bk):
    """"Current integration stack": with every block exact, the proxy path is dense attention.  The
    GPU result is compared with the oracle's proxy result and with the oracle's dense attention
    (skip-softmax at lambda = 0, which never skips)."""
    announce(f"proxy all-ones / empty Bq={Bq} Bk={Bk}")
    B, S, H, D = 1, 300, 2, 128
    q, k, v = W.gen_iid(53, B, S, S, H, H, D)
    nQB, nKB = -(-S // Bq), -(-S // Bk)
    ones = np.full((B, H, nQB, 1), 0xFFFFFFFF, np.uint32)
    o1, lse1, o_ref, lse_ref = run_proxy(q, k, v, ones, Bq, Bk, 1)
    assert_output_parity(o1, o_ref, "proxy all-ones")
    assert err(lse1, lse_ref)[0] < 2e-3
    o_dense, lse_dense, _, _ = oracle.skip_softmax(q, k, v, causal=False, block_q=Bq, block_k=64,
                                                   scale=1 / math.sqrt(D), lam=0.0)
    assert_output_parity(o1, o_dense, "proxy all-ones vs dense oracle")
    assert err(lse1, lse_dense)[0] < 2e-3
    empty = np.zeros((B, H, nQB, 1), np.uint32)
    empty[:, :, 1:] = 1
    o0, lse0, _, _ = run_proxy(q, k, v, empty, Bq, Bk, 0)
    assert (o0[:, :Bq] == 0).all() and np.isneginf(lse0[:, :, :Bq]).all()


@pytest.mark.parametrize("use_proxy", [0, 1])
@pytest.mark.parametrize("Bq,Bk", [(128, 128), (128, 64), (64, 64)])
def test_inflated_n_exact_reads_nothing_past_the_route(Bq, Bk, use_proxy):
    """A caller n_exact larger than the route's real count makes the kernel read the -1 fill after
    the real exact_idx entries: such entries must contribute nothing (the result equals the one
    with the true counts).  Only rows of batch 1 are inflated, so the K/V rows an unguarded kernel
    would fetch in front of batch 1's slab still lie inside the allocation (batch 0)."""
    announce(f"proxy inflated n_exact Bq={Bq} Bk={Bk} use_proxy={use_proxy}")
    B, S, H, D = 2, 700, 2, 128
    q, k, v = W.gen_iid(57, B, S, S, H, H, D)
    nQB, nKB = -(-S // Bq), -(-S // Bk)
    bm = W.gen_bitmask(57, B, H, nQB, nKB, max(1, nKB // 3))
    km, vs = W.block_summaries(k, v, Bk)
    ne, ix, kp = route_gpu(bm, B, H, S, S, Bq, Bk)
    qd, kd, vd, kmd, vsd = to_dev(q), to_dev(k), to_dev(v), to_dev(km), to_dev(vs)
    ne_bad = ne.clone()
    ne_bad[1] = nKB + 5                       # past the real entries and past the row
    ix_bad = ix.clone()
    ix_bad[1, :, :, -1] = 1 << 20             # a far out-of-range entry inside the counted range
    outs = []
    for n_e, idx in ((ne, ix), (ne_bad, ix_bad)):
        o = torch.full((B, S, H, D), float("nan"), dtype=torch.bfloat16, device="cuda")
        lse = torch.full((B, H, S), float("nan"), device="cuda")
        sa.sa_proxy_block_sparse_fwd(qd, kd, vd, kmd, vsd, n_e, idx, kp, use_proxy, o,
                                     block_q=Bq, block_k=Bk, lse=lse)
        torch.cuda.synchronize()
        outs.append((from_dev_bf16(o), lse.cpu().numpy()))
    assert np.array_equal(outs[0][0], outs[1][0])
    assert np.array_equal(outs[0][1], outs[1][1])
    o_ref, lse_ref = oracle.proxy_fwd(q, k, v, km, vs, bm, block_q=Bq, block_k=Bk,
                                      scale=1 / math.sqrt(D), use_proxy=use_proxy)
    assert_output_parity(outs[1][0], o_ref, "inflated n_exact")
    assert err(outs[1][1], lse_ref)[0] < 2e-3
