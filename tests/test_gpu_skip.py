"""GPU parity of sa_skip_softmax_fwd against the oracle (needs an MI355X).

For every case the GPU runs with all exports on, then:
  * replay: the oracle re-decides every tile from the GPU's exported fp32 tile maxima in fp32;
    the skip decisions must equal the GPU's tile_state bit for bit;
  * independent: the oracle's own float64 decisions agree on >= 99.9 % of visited tiles;
  * output: the oracle, forced onto the GPU's kept tiles, matches O within max-abs 2e-2 and
    mean-abs 2e-3, and the LSE within 2e-3;
  * the exported maxima match the oracle's float64 maxima, and the head counters equal the
    tile_state histogram.
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


def run_gpu(q, k, v, causal, Br, lam, *, dbg=True, q_dev=None, k_dev=None, v_dev=None, Bc=64,
            gran="tile"):
    """Runs the GPU with every export on.  Decision blocks are R = Br rows (tile granularity) or
    R = 32 rows (wave granularity), so states and maxima are [B, Hq, ceil(Sq/R), nKT(, R)]."""
    B, Sq, Hq, D = q.shape
    Sk = k.shape[1]
    R = 32 if gran == "wave" else Br
    nR, nKT = -(-Sq // R), -(-Sk // Bc)
    qd = q_dev if q_dev is not None else to_dev(q)
    kd = k_dev if k_dev is not None else to_dev(k)
    vd = v_dev if v_dev is not None else to_dev(v)
    o = torch.full((B, Sq, Hq, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    st = torch.full((B, Hq, nR, nKT), 255, dtype=torch.uint8, device="cuda")
    cnt = torch.zeros((B, Hq, 2), dtype=torch.int32, device="cuda")
    lse = torch.full((B, Hq, Sq), float("nan"), device="cuda")
    rm = torch.empty((B, Hq, nR, nKT, R), device="cuda") if dbg else None
    kw = dict(causal=causal, block_q=Br, block_k=Bc, tile_state=st, head_counters=cnt, lse=lse,
              dbg_tile_rowmax=rm)
    if gran == "tile":
        sa.sa_skip_softmax_fwd(qd, kd, vd, o, lam, **kw)
    else:
        sa.sa_skip_softmax_fwd_ex(qd, kd, vd, o, lam, gran, **kw)
    torch.cuda.synchronize()
    return dict(o=from_dev_bf16(o), st=st.cpu().numpy(), cnt=cnt.cpu().numpy(),
                lse=lse.cpu().numpy(), rm=None if rm is None else rm.cpu().numpy())


def check_case(q, k, v, causal, Br, lam, tag, *, Bc=64, gran="tile"):
    """Wave granularity is checked against the oracle's tile rule on 32-row query tiles: each
    32-row block has its own running max and its own decisions."""
    announce(f"skip {tag} lam={lam} Bc={Bc} gran={gran}")
    D = q.shape[-1]
    scale = 1 / math.sqrt(D)
    g = run_gpu(q, k, v, causal, Br, lam, Bc=Bc, gran=gran)
    st = g["st"]
    assert set(np.unique(st)) <= {0, 1, 2}
    # counters = histogram of tile_state
    assert (g["cnt"][..., 0] == (st != 2).sum(-1).sum(-1)).all()
    assert (g["cnt"][..., 1] == (st == 1).sum(-1).sum(-1)).all()
    R = 32 if gran == "wave" else Br
    kw = dict(causal=causal, block_q=R, block_k=Bc, scale=scale, lam=lam)
    # replay: decisions bit-exact given the GPU's maxima
    _, _, st_replay, _ = oracle.skip_softmax(q, k, v, mode=1, rowmax_in=g["rm"], **kw)
    assert np.array_equal(st_replay, st), "replayed decisions differ from the GPU's"
    # independent float64 decisions
    o_ind, _, st_ind, rm_ind = oracle.skip_softmax(q, k, v, **kw)
    visited = st != 2
    assert np.array_equal(st_ind == 2, ~visited)
    agree = (st_ind[visited] == st[visited]).mean()
    assert agree >= 0.999, f"independent agreement {agree:.5f}"
    # exported maxima vs float64 maxima (valid rows of visited tiles)
    fin = np.isfinite(rm_ind)
    assert np.array_equal(np.isfinite(g["rm"]) & fin, fin)
    assert np.abs(g["rm"][fin] - rm_ind[fin]).max() < 2e-3 * max(1.0, np.abs(rm_ind[fin]).max())
    # output on the GPU's kept-tile set
    o_ref, lse_ref, _, _ = oracle.skip_softmax(q, k, v, mode=2, state_in=st, **kw)
    mx, mean = assert_output_parity(g["o"], o_ref, tag)
    lmx, _ = err(g["lse"], lse_ref)
    assert lmx < 2e-3, f"lse max err {lmx}"
    return st, mx, mean


LAMBDAS_C1 = [1e-3, 0.0, 0.5, 1.0, 1.5, 3.0, 1e30]


@pytest.mark.parametrize("lam", LAMBDAS_C1)
def test_iid_s256_d64(lam):
    """The small non-causal case: B1, 2 heads, S 256, D 64, 64x64 tiles."""
    wl = W.WORKLOADS["iid_s256_d64"]
    q, k, v = wl.generate()
    st, _, _ = check_case(q, k, v, False, 64, lam, "iid_s256_d64")
    if lam in (0.0, 1e-3):
        assert (st == 0).all()
    if lam == 1e30:
        assert (st[..., 0] == 0).all() and (st[..., 1:] == 1).all()


@pytest.mark.parametrize("lam", [0.0, 0.5, 1.0, 1.5127145])
def test_llm_causal_gqa_reduced(lam):
    """Causal GQA on the LLM generator at a reduced size (8 query / 2 KV heads, S 1024)."""
    q, k, v = W.gen_llm(2, 1, 1024, 8, 2, 128)
    st, _, _ = check_case(q, k, v, True, 128, lam, "llm_causal_gqa_s1024")
    if lam >= 1.0:
        assert (st == 1).sum() > 0


@pytest.mark.parametrize("shape", [
    # (B, Sq, Sk, Hq, Hkv, D, causal, Br)
    (1, 200, 300, 2, 2, 128, False, 128),    # ragged Q and K tiles, Sq != Sk
    (2, 130, 130, 4, 1, 128, True, 128),     # 2-row last Q tile, batch 2, GQA 4:1
    (1, 257, 257, 2, 2, 64, True, 64),       # 1-row last tile, D 64, Br 64
    (1, 192, 192, 2, 2, 128, True, 64),      # D 128 with Br 64
    (1, 1, 1, 1, 1, 128, True, 128),         # single token
    (1, 65, 64, 3, 3, 64, False, 128),       # D 64 with Br 128
    # causal work order in blocks of several KV heads (longest rows first inside a block):
    (1, 300, 300, 31, 31, 64, True, 128),    # blocks of 3 heads, the last one holding 1
    (2, 200, 200, 20, 10, 64, True, 128),    # blocks of 2 KV heads, GQA 2:1
])
@pytest.mark.parametrize("lam", [0.0, 0.9])
def test_edge_shapes(shape, lam):
    B, Sq, Sk, Hq, Hkv, D, causal, Br = shape
    if causal:
        q, k, v = W.gen_llm(5, B, Sq, Hq, Hkv, D)
    else:
        q, k, v = W.gen_iid(5, B, Sq, Sk, Hq, Hkv, D)
    check_case(q, k, v, causal, Br, lam, f"edge {shape}")


def test_strided_views_match_contiguous():
    """Q/K/V/O as non-contiguous views (head stride 2*D) give the same bits as contiguous."""
    announce("skip strided views")
    B, S, H, D = 1, 256, 2, 128
    q, k, v = W.gen_llm(6, B, S, H, H, D)
    ref = run_gpu(q, k, v, True, 128, 0.8, dbg=False)

    def padded(x):
        big = torch.zeros((x.shape[0], x.shape[1], x.shape[2], 2 * D), dtype=torch.bfloat16,
                          device="cuda")
        big[..., :D] = to_dev(x)
        return big[..., :D]

    qv, kv, vv = padded(q), padded(k), padded(v)
    assert not qv.is_contiguous()
    o_big = torch.zeros((B, S, H, 2 * D), dtype=torch.bfloat16, device="cuda")
    o = o_big[..., :D]
    st = torch.zeros((B, H, 2, 4), dtype=torch.uint8, device="cuda")
    sa.sa_skip_softmax_fwd(qv, kv, vv, o, 0.8, causal=True, block_q=128, tile_state=st)
    torch.cuda.synchronize()
    assert np.array_equal(from_dev_bf16(o), ref["o"])
    assert np.array_equal(st.cpu().numpy(), ref["st"])
    assert (o_big[..., D:] == 0).all()


def test_debug_exports_do_not_change_results():
    announce("skip dbg on/off")
    q, k, v = W.gen_llm(7, 1, 512, 4, 2, 128)
    a = run_gpu(q, k, v, True, 128, 1.2, dbg=True)
    b = run_gpu(q, k, v, True, 128, 1.2, dbg=False)
    assert np.array_equal(a["o"], b["o"]) and np.array_equal(a["st"], b["st"])


def test_counters_accumulate_and_stream_order():
    announce("skip counters accumulate")
    q, k, v = W.gen_llm(8, 1, 512, 2, 2, 128)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    o = torch.empty_like(qd)
    cnt = torch.zeros((1, 2, 2), dtype=torch.int32, device="cuda")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        for _ in range(3):
            sa.sa_skip_softmax_fwd(qd, kd, vd, o, 1.0, causal=True, head_counters=cnt)
    s.synchronize()
    one = run_gpu(q, k, v, True, 128, 1.0, dbg=False)["cnt"]
    assert np.array_equal(cnt.cpu().numpy(), 3 * one)


# ---- 128-key decision tiles: two 64-key steps decided together ---------------------------------

def late_keeps(q, k, causal, Br, lam, st128):
    """Kept 128-key tiles whose first 64 keys alone are negligible against the running max before
    the tile (the tile is kept only through its second half: the kernel then fetches the first
    half's V late).  Computed in float64 from the oracle's 64-key maxima, to show the path runs."""
    D = q.shape[-1]
    _, _, _, rm64 = oracle.skip_softmax(q, k, k, causal=causal, block_q=Br, block_k=64,
                                        scale=1 / math.sqrt(D), lam=0.0)
    L = math.log2(lam) if lam > 0 else -math.inf
    B, H, nQT, nKT128 = st128.shape
    nKT64 = rm64.shape[3]
    Sq = q.shape[1]
    count = 0
    for b in range(B):
        for h in range(H):
            for i in range(nQT):
                nr = min(Br, Sq - i * Br)
                m = np.full(nr, -np.inf)
                for j in range(nKT128):
                    if st128[b, h, i, j] != 0:
                        continue
                    a = rm64[b, h, i, 2 * j, :nr]
                    bm = rm64[b, h, i, 2 * j + 1, :nr] if 2 * j + 1 < nKT64 else np.full(nr, -np.inf)
                    if (a < m + L).all():
                        count += 1
                    m = np.maximum(m, np.maximum(a, bm))
    return count


@pytest.mark.parametrize("shape", [
    # (B, Sq, Sk, Hq, Hkv, D, causal, Br)
    (1, 256, 256, 2, 2, 64, False, 64),      # the small case at the pages' bc = 128
    (1, 1000, 1000, 4, 2, 128, True, 64),    # causal with Br 64: the last 128-key tile of odd
                                             # query tiles holds one 64-key step
    (1, 1000, 1000, 2, 2, 128, True, 128),   # br = bc = 128
    (1, 200, 300, 2, 2, 128, False, 128),    # last 128-key tile is 44 keys (one step)
    (2, 130, 130, 4, 1, 64, True, 128),      # 2-row last query tile, GQA 4:1
])
@pytest.mark.parametrize("lam", [0.0, 0.5, 1.0, 1.5, 3.0, 1e30])
def test_block_k_128(shape, lam):
    B, Sq, Sk, Hq, Hkv, D, causal, Br = shape
    if causal:
        q, k, v = W.gen_llm(61, B, Sq, Hq, Hkv, D)
    else:
        q, k, v = W.gen_iid(61, B, Sq, Sk, Hq, Hkv, D)
    st, _, _ = check_case(q, k, v, causal, Br, lam, f"bk128 {shape}", Bc=128)
    if lam == 0.0:
        assert (st != 1).all()
    if lam == 1e30:
        assert (st[..., 0] == 0).all()


def test_block_k_128_late_keeps_happen():
    """The sweep above runs the late-keep path (tiles kept through their second half only)."""
    q, k, v = W.gen_iid(61, 1, 256, 256, 2, 2, 64)
    seen = 0
    for lam in (1.0, 1.5, 3.0):
        g = run_gpu(q, k, v, False, 64, lam, dbg=False, Bc=128)
        seen += late_keeps(q, k, False, 64, lam, g["st"])
    assert seen > 0


def test_block_k_128_llm_causal_gqa():
    """The causal GQA prefill generator at a reduced size with the pages' br = bc = 128."""
    q, k, v = W.gen_llm(2, 1, 2048, 8, 2, 128)
    st, _, _ = check_case(q, k, v, True, 128, 1.5127145, "llm_causal_gqa_s2048", Bc=128)
    assert 0 < (st == 1).sum() < (st != 2).sum()


# ---- wave granularity: each 32-row wavefront decides alone ----------------------------------------

@pytest.mark.parametrize("shape", [
    # (B, Sq, Sk, Hq, Hkv, D, causal, Br)
    (1, 256, 256, 2, 2, 64, False, 64),
    (1, 1000, 1000, 4, 2, 128, True, 128),   # causal: the waves of a tile visit different tiles
    (1, 200, 300, 2, 2, 128, False, 128),    # ragged: a wave with 8 rows, a wave with none
    (2, 130, 130, 4, 1, 64, True, 64),
])
@pytest.mark.parametrize("Bc", [64, 128])
@pytest.mark.parametrize("lam", [0.0, 0.5, 1.0, 3.0])
def test_wave_granularity(shape, Bc, lam):
    B, Sq, Sk, Hq, Hkv, D, causal, Br = shape
    if causal:
        q, k, v = W.gen_llm(62, B, Sq, Hq, Hkv, D)
    else:
        q, k, v = W.gen_iid(62, B, Sq, Sk, Hq, Hkv, D)
    st, _, _ = check_case(q, k, v, causal, Br, lam, f"wave {shape}", Bc=Bc, gran="wave")
    if lam == 0.0:
        assert (st != 1).all()


@pytest.mark.parametrize("lam", [0.3, 0.6, 1.0])
def test_wave_sparsity_at_least_tile_sparsity(lam):
    """For lambda <= 1 a skipped tile never raises the running max, so every row's running max is
    the dense prefix max under both granularities: a tile skipped by the whole query tile is
    skipped by each of its waves, and the wave sparsity is at least the tile sparsity."""
    announce(f"wave vs tile sparsity lam={lam}")
    q, k, v = W.gen_llm(63, 1, 2048, 4, 4, 128)
    t = run_gpu(q, k, v, True, 128, lam, dbg=False)
    w = run_gpu(q, k, v, True, 128, lam, dbg=False, gran="wave")
    ts, ws = t["st"], w["st"]              # [1, H, 16, nKT] and [1, H, 64, nKT]
    tile_skip = np.repeat(ts == 1, 4, axis=2)
    # skipped by each wave that visits it (a wave below the diagonal may not visit it at all)
    assert (ws[tile_skip] != 0).all()
    # and over the (wave, tile) pairs a wave visits, at least as many skips
    vis = ws != 2
    assert (ws[vis] == 1).sum() >= tile_skip[vis].sum()
    if lam >= 0.6:
        assert (ws[vis] == 1).sum() > tile_skip[vis].sum()   # the finer rule skips more
