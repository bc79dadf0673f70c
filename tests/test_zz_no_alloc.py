"""The allocation-free decode entry point (needs an MI355X): sa_skip_softmax_decode_fwd_noalloc
keeps its workspace in the library's fixed device array.  Called through the C ABI, its outputs
must equal those of sa_skip_softmax_decode_fwd with a caller workspace bit for bit (the same
kernels: within the parity bar a fortiori), on two calls in a row, the second with a smaller input
(the array keeps the first call's contents), and also after a call with a different head group."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import announce, to_dev

pytestmark = pytest.mark.gpu

sa = pytest.importorskip("sparse_attention_flash_amd")


def both(q, k, v, lens, lam, BC, num_splits=0):
    B, _, Hq, D = q.shape
    S = k.shape[1]
    nKT = -(-S // BC)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    ln = torch.from_numpy(lens.astype(np.int32)).to("cuda")
    res = []
    for noalloc in (False, True):
        o = torch.full((B, 1, Hq, D), float("nan"), dtype=torch.bfloat16, device="cuda")
        st = torch.full((B, Hq, nKT), 255, dtype=torch.uint8, device="cuda")
        cnt = torch.zeros((B, Hq, 2), dtype=torch.int32, device="cuda")
        lse = torch.full((B, Hq), float("nan"), device="cuda")
        kw = dict(block_k=BC, seqlens_k=ln, num_splits=num_splits, tile_state=st,
                  head_counters=cnt, lse=lse)
        if noalloc:
            sa.sa_skip_softmax_decode_fwd_noalloc(qd, kd, vd, o, lam, **kw)
        else:
            sa.sa_skip_softmax_decode_fwd(qd, kd, vd, o, lam, **kw)
        torch.cuda.synchronize()
        res.append([t.cpu() for t in (o.view(torch.int16), st, cnt, lse)])
    for a, b in zip(*res):
        assert torch.equal(a, b)
    return res[1]


@pytest.mark.parametrize("lam", [0.1, 2.0])
def test_noalloc_matches_workspace_entry_point(lam):
    announce(f"decode noalloc lam={lam}: large call, then a smaller one")
    # first call: the decode workload's head layout (G = 4, head_dim 128) on a 4096-key cache
    q, k, v, lens = W.gen_llm_decode(81, 8, 4096, 32, 8, 128)
    out = both(q, k, v, lens, lam, 64)
    assert (out[1] == 1).sum() > 0 or lam < 1.0
    # second call, smaller in every dimension (head_dim 64, G = 2, 128-key tiles)
    q2, k2, v2, lens2 = W.gen_llm_decode(82, 3, 700, 4, 2, 64)
    both(q2, k2, v2, lens2, lam, 128)
    # and the first shape again after the smaller one
    both(q, k, v, lens, lam, 64)


def test_noalloc_explicit_splits_and_full_workload_size():
    announce("decode noalloc: explicit splits, decode workload size")
    wl = W.WORKLOADS["llm_decode_gqa_kv8192"]
    q, k, v, lens = wl.generate()
    both(q, k, v, lens, 0.1146, wl.block_k)
    q2, k2, v2, lens2 = W.gen_llm_decode(83, 2, 1000, 8, 8, 128)
    both(q2, k2, v2, lens2, 0.5, 64, num_splits=3)


@pytest.mark.parametrize("num_splits", [0, 1])
def test_noalloc_under_graph_capture(num_splits):
    """The callers the entry point is for: one eager call (which looks up the array's address),
    then the same call captured in a HIP graph and replayed three times, with eager work that
    overwrites the outputs between the replays; every replay must reproduce the eager outputs bit
    for bit.  The decode path enqueues no memset, so nothing in the graph depends on one.
    num_splits 0 runs the key-axis split (three kernels), 1 the whole-sequence kernel."""
    announce(f"decode noalloc under graph capture splits={num_splits}")
    q, k, v, lens = W.gen_llm_decode(83, 4, 2048, 16, 4, 128)
    B, _, Hq, D = q.shape
    BC = 64
    nKT = -(-k.shape[1] // BC)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    ln = torch.from_numpy(lens.astype(np.int32)).to("cuda")
    o = torch.empty((B, 1, Hq, D), dtype=torch.bfloat16, device="cuda")
    st = torch.empty((B, Hq, nKT), dtype=torch.uint8, device="cuda")
    lse = torch.empty((B, Hq), device="cuda")
    kw = dict(block_k=BC, seqlens_k=ln, num_splits=num_splits, tile_state=st, lse=lse)
    sa.sa_skip_softmax_decode_fwd_noalloc(qd, kd, vd, o, 0.1, **kw)
    torch.cuda.synchronize()
    ref = [t.clone() for t in (o.view(torch.int16), st, lse)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sa.sa_skip_softmax_decode_fwd_noalloc(qd, kd, vd, o, 0.1, **kw)
    for _ in range(3):
        o.fill_(float("nan"))
        st.fill_(255)
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip((o.view(torch.int16), st, lse), ref):
            assert torch.equal(a, b)
