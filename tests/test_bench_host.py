"""Host-side pieces of bench.py (no GPU): the algorithmic-work accounting behind `value` and
`roofline.achieved`, the profile-digest guard on `roofline.traffic`, and the one-GPU refusal."""
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def brute_pairs(Sq, Sk, Br, Bc, causal):
    nQT, nKT = -(-Sq // Br), -(-Sk // Bc)
    P = np.zeros((nQT, nKT), np.int64)
    for r in range(Sq):
        for k in range(Sk):
            if not causal or k <= r:
                P[r // Br, k // Bc] += 1
    return P


@pytest.mark.parametrize("Sq,Sk,Br,Bc,causal", [
    (256, 256, 64, 64, False),
    (257, 257, 128, 64, True),    # ragged last tiles, causal
    (100, 300, 64, 64, False),    # Sq != Sk
    (130, 130, 128, 64, True),
])
def test_tile_pairs_brute_force(Sq, Sk, Br, Bc, causal):
    assert np.array_equal(bench.tile_pairs(Sq, Sk, Br, Bc, causal),
                          brute_pairs(Sq, Sk, Br, Bc, causal))


def test_skip_flops_counts_qk_on_visited_and_pv_on_kept():
    P = bench.tile_pairs(200, 200, 64, 64, True)
    D = 128
    rng = np.random.default_rng(0)
    st = rng.integers(0, 3, size=(2, 3) + P.shape).astype(np.uint8)   # 0 kept, 1 skipped, 2 unvisited
    computed, dense = bench.skip_flops(st, P, D)
    flat = st.reshape(-1, *P.shape)
    expect = sum(2 * D * int(P[i, j]) * (int(s[i, j] != 2) + int(s[i, j] == 0))
                 for s in flat for i in range(P.shape[0]) for j in range(P.shape[1]))
    assert computed == expect
    assert dense == 4 * D * int(P.sum()) * flat.shape[0]
    # every tile kept: computed == dense
    c0, d0 = bench.skip_flops(np.zeros_like(st), P, D)
    assert c0 == d0


def test_measured_traffic_only_for_the_profiled_source(tmp_path, monkeypatch):
    digest = bench.source_digest(bench.SKIP_SOURCES)
    good = tmp_path / "good.txt"
    good.write_text(f"hbm_bytes_per_launch: 6.0e+10\nsource_digest: {digest}\n")
    stale = tmp_path / "stale.txt"
    stale.write_text("hbm_bytes_per_launch: 6.0e+10\nsource_digest: 0000000000000000\n")
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    assert bench.measured_traffic("good.txt") == 6.0e10
    assert bench.measured_traffic("stale.txt") is None
    assert bench.measured_traffic("missing.txt") is None
    # each kernel's profile is checked against its own sources
    nm_good = tmp_path / "nm.txt"
    nm_good.write_text(f"hbm_bytes_per_launch: 1.0e+9\nsource_digest: "
                       f"{bench.source_digest(bench.KERNEL_SOURCES['nm'])}\n")
    assert bench.measured_traffic("nm.txt", "nm") == 1.0e9
    assert bench.measured_traffic("nm.txt", "skip") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_wave_flops_count_qk_per_tile_and_pv_per_wave_block():
    S, D = 256, 64
    P_tile = bench.tile_pairs(S, S, 128, 64, False)
    P_wave = bench.tile_pairs(S, S, 32, 64, False)
    st = np.zeros((1, 1, S // 32, S // 64), np.uint8)
    st[0, 0, 1, 2] = 1                          # one 32-row block skips one key tile
    got = bench.wave_skip_flops(st, P_tile, P_wave, D)
    assert got == 4 * D * S * S - 2 * D * 32 * 64
    # every block keeps every tile: the dense flops
    assert bench.wave_skip_flops(np.zeros_like(st), P_tile, P_wave, D) == 4 * D * S * S


def test_roofline_block_fields():
    r = bench.roofline("mfma", 1250.0)
    assert r["frac"] == 0.5 and r["peak"] == 2500.0 and r["unit"] == "TFLOP/s"
    h = bench.roofline("hbm", 4000.0)
    assert h["frac"] == 0.5 and h["unit"] == "GB/s" and h["traffic"] is None


def test_unknown_leg_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--only", "nope"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0 and "unknown leg" in r.stderr
