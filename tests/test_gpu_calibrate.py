"""GPU checks of the calibration sweep (sa_skip_softmax_calibrate) and the log-space fit
(sa_fit_threshold_calib), needs an MI355X.

Model-Optimizer diffusion README ("Calibrated threshold"; "Known Issues") and the HuggingFace
attention-sparsity page (calibration.threshold_trials): trial thresholds are run, the tile sparsity
each reaches is measured, and scale_factor = a*exp(b*sparsity) is fitted in log space.  Checked:
  * each trial's sparsity equals the tile_state histogram of a direct sa_skip_softmax_fwd call at
    that threshold, and the oracle's independent float64 decisions give the same sparsity to
    within 0.1 % of the visited tiles;
  * sparsity never falls as the threshold rises (every trial is <= 1, where a skipped tile could
    not have raised the running max, so each decision only tightens with lambda);
  * the C-ABI fit of the measured sparsities equals the oracle's fit of them;
  * lowering a target inside the fitted range and running at that threshold lands near the target.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import announce, to_dev

pytestmark = pytest.mark.gpu

sa = pytest.importorskip("sparse_attention_flash_amd")

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _trials():
    with open(os.path.join(GOLDEN, "page_constants.json")) as f:
        return json.load(f)["threshold_trials"]["values"]


def test_calibration_sweep_and_fit():
    announce("calibration sweep on a reduced video grid")
    grid = (5, 16, 26)
    B, H, D, Br = 1, 2, 128, 128
    q, k, v = W.gen_video(6, B, H, D, grid=grid)
    S = q.shape[1]
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    o = torch.empty((B, S, H, D), dtype=torch.bfloat16, device="cuda")
    cnt = torch.zeros((B, H, 2), dtype=torch.int32, device="cuda")
    trials = _trials()
    sp = sa.sa_skip_softmax_calibrate(qd, kd, vd, o, trials, cnt, block_q=Br)
    assert all(b >= a for a, b in zip(sp, sp[1:])), sp
    nQT, nKT = sa.tile_counts(S, S, Br, 64)
    scale = 1 / math.sqrt(D)
    for lam, s in zip(trials, sp):
        st = torch.full((B, H, nQT, nKT), 255, dtype=torch.uint8, device="cuda")
        sa.sa_skip_softmax_fwd(qd, kd, vd, o, lam, block_q=Br, tile_state=st)
        torch.cuda.synchronize()
        st = st.cpu().numpy()
        visited = int((st != 2).sum())
        assert s == (st == 1).sum() / visited
        _, _, st_ref, _ = oracle.skip_softmax(q, k, v, causal=False, block_q=Br, block_k=64,
                                              scale=scale, lam=lam)
        assert abs(int((st_ref == 1).sum()) - int((st == 1).sum())) <= max(1, visited // 1000)
    a, b, lo, hi = sa.sa_fit_threshold_calib(trials, sp, S)
    ra, rb, rlo, rhi = oracle.fit_threshold(trials, sp, S)
    assert a == pytest.approx(ra, rel=1e-12) and b == pytest.approx(rb, rel=1e-12)
    assert (lo, hi) == (rlo, rhi)
    target = 0.5 * (lo + hi)
    _, lam_t, _ = sa.sa_threshold_from_calib(a, b, target, S)
    got = sa.sa_skip_softmax_calibrate(qd, kd, vd, o, [lam_t], cnt, block_q=Br)[0]
    announce(f"fit a={a:.4g} b={b:.4g} range [{lo:.3f}, {hi:.3f}]; target {target:.3f} -> {got:.3f}")
    assert abs(got - target) < 0.15


def test_calibration_sweep_at_128_key_tiles():
    """The sweep at the pages' 128 x 128 tiles (Model-Optimizer HuggingFace page, "Custom
    Configuration"): each trial's sparsity is the tile_state histogram of the forward kernel at
    block_k = 128, and the oracle's float64 decisions on 128-key tiles agree to within 0.1 % of the
    visited tiles."""
    announce("calibration sweep at 128 x 128 tiles")
    q, k, v = W.gen_video(7, 1, 2, 128, grid=(5, 16, 26))
    B, S, H, D = q.shape
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    o = torch.empty((B, S, H, D), dtype=torch.bfloat16, device="cuda")
    cnt = torch.zeros((B, H, 2), dtype=torch.int32, device="cuda")
    trials = _trials()
    sp = sa.sa_skip_softmax_calibrate(qd, kd, vd, o, trials, cnt, block_q=128, block_k=128)
    assert all(b >= a for a, b in zip(sp, sp[1:])), sp
    assert 0.0 < max(sp) < 1.0   # the sweep reaches sparsity on this input
    nQT, nKT = sa.tile_counts(S, S, 128, 128)
    for lam, s in zip(trials, sp):
        st = torch.full((B, H, nQT, nKT), 255, dtype=torch.uint8, device="cuda")
        sa.sa_skip_softmax_fwd(qd, kd, vd, o, lam, block_q=128, block_k=128, tile_state=st)
        torch.cuda.synchronize()
        st = st.cpu().numpy()
        visited = int((st != 2).sum())
        assert s == (st == 1).sum() / visited
        _, _, st_ref, _ = oracle.skip_softmax(q, k, v, causal=False, block_q=128, block_k=128,
                                              scale=1 / math.sqrt(D), lam=lam)
        assert abs(int((st_ref == 1).sum()) - int((st == 1).sum())) <= max(1, visited // 1000)
