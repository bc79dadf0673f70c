#!/usr/bin/env python
"""Benchmark of the sparse flash-attention forward library on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-paths]
    python bench.py --only LEG [--steps K] [--warmup W]       (one leg, for profiler runs)
    python bench.py --cpu-full-runs                           (the oracle's full-run times)
    python bench.py --peak-probes                             (attainable HBM / GEMM rates)

One step is one pass of the skip-softmax hot path over the headline workload: the calibrated
threshold lowering (host, a*exp(b*0.5)/seq_k) followed by the skip-softmax forward with its tile
state and per-head counters, on the video-DiT self-attention shape (batch 1, 40 heads, 32760
tokens = 21x30x52, head_dim 128, non-causal, 128x64 tiles), inputs seeded and synthetic and
resident in HBM before timing.  W untimed steps, then exactly K steps between two
torch.cuda.synchronize() calls, timed with HIP events on the launch stream.  Afterwards (untimed
for the headline) the same kernel at lambda = 0, and the sibling paths at their own workloads,
are timed the same way and reported under "paths", each with its own roofline block.

Prints ONE JSON line.  value = computed TFLOP/s of the skip-softmax kernel (QK^T flops of every
visited tile + P.V flops of every kept tile, unmasked pairs only); dense_equiv_tflops counts the
full attention's flops over the same time.

Legs (--only): headline, skip_gqa, nm:N:M (e.g. nm:2:4), skip_nm, decode,
proxy_bitmask_s16257, proxy_page_s32760, video_bk128, video_wave.  A leg run alone launches
only its main arm: warmup + steps launches of one kernel (decode: of its three kernels).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA (no sparsity)
PEAK_HBM_GBPS = 8000.0         # MI355X HBM3E
HEADLINE = "video_dit_s32760"
PROFILES = os.path.join(ROOT, "profiles")
LEGS = ("headline", "skip_gqa", "nm", "skip_nm", "decode", "proxy_bitmask_s16257",
        "proxy_page_s32760", "video_bk128", "video_wave")


def parse_args(argv=None):
    p = argparse.ArgumentParser(description=__doc__.split("\n")[1])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-paths", action="store_true", help="only the headline workload")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="target wall time of the CPU-oracle sample")
    p.add_argument("--only", default="", metavar="LEG",
                   help="run one leg only (main arm, warmup + steps launches) and print its "
                        "record as one JSON line; for profiler runs")
    p.add_argument("--profile", action="store_true", help="same as --only headline")
    p.add_argument("--cpu-full-runs", action="store_true",
                   help="time the CPU oracle over the whole of the small, causal-GQA, N:M and "
                        "proxy workloads (minutes of CPU time) and print the times")
    p.add_argument("--peak-probes", action="store_true",
                   help="only measure the attainable HBM read / copy rates and a library bf16 "
                        "GEMM rate on this part, and print them")
    p.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                   help="only run 5 device-to-device copies of BYTES bytes (a plain copy kernel "
                        "of known size, used to scale the HBM byte counters) and exit")
    return p.parse_args(argv)


def peak_probes():
    """Attainable rates on this part, for the roofline's context (the roofline itself uses the
    published peaks), from libsa_probes.so (include/sa_probes.h) and torch:
      * the bf16 matrix-core rate: four independent v_mfma_f32_32x32x16_bf16 chains per wave,
        16 waves per CU, register operands only, once with random operands that change from
        issue to issue (the switching power of real data) and once with constant ones;
      * the HBM read rate: 16 KiB contiguous chunks, four in flight per wave, over four 268 MB
        buffers read in rotation (1.07 GB in all, more than the 256 MB last-level cache, so no
        launch finds its data there);
      * a read+write stream (torch copy of 1 GiB, both directions counted);
      * a library bf16 GEMM (torch.matmul, 8192^3, hipBLASLt)."""
    import ctypes
    import torch
    lib = probe_lib()
    dev = torch.device("cuda:0")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    out = {
        "mfma_bf16_tflops_random_operands": mfma_probe(torch, lib, True),
        "mfma_bf16_tflops_constant_operands": mfma_probe(torch, lib, False),
    }

    g = torch.Generator(device=dev)
    g.manual_seed(0)
    nbytes, rwgs = 1 << 28, 512
    bufs = [torch.randint(0, 1 << 15, (nbytes // 2,), generator=g, dtype=torch.int16, device=dev)
            for _ in range(4)]
    sink = torch.empty(rwgs * 512, dtype=torch.int32, device=dev)
    turn = [0]

    def read():
        x = bufs[turn[0] % len(bufs)]
        turn[0] += 1
        if lib.sa_probe_read(ctypes.c_void_p(x.data_ptr()), nbytes, ctypes.c_void_p(sink.data_ptr()),
                             rwgs, stream) != 0:
            raise RuntimeError("sa_probe_read failed")
    ms = time_steps(torch, read, 12, 4)
    out["read_stream_gbps"] = round(nbytes / ms / 1e6, 1)
    del bufs, sink

    a = torch.rand(1 << 28, generator=g, device=dev)             # 1 GiB
    b = torch.empty_like(a)
    ms = time_steps(torch, lambda: b.copy_(a), 10, 3)
    out["copy_read_plus_write_gbps"] = round(2 * a.numel() * 4 / ms / 1e6, 1)
    del a, b
    out["bf16_gemm_8192_tflops"] = gemm_probe(torch)
    torch.cuda.empty_cache()
    return out


def probe_lib():
    """libsa_probes.so (include/sa_probes.h), with its ctypes signatures."""
    import ctypes
    path = os.path.join(ROOT, "sparse_attention_flash_amd", "libsa_probes.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with sparse_attention_flash_amd/build.py")
    lib = ctypes.CDLL(path)
    lib.sa_probe_mfma_bf16_flops.restype = ctypes.c_double
    lib.sa_probe_mfma_bf16_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.sa_probe_mfma_bf16.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_void_p]
    lib.sa_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                  ctypes.c_void_p]
    return lib


def mfma_probe(torch, lib, random_operands):
    """TFLOP/s of sa_probe_mfma_bf16: 1024 workgroups (16 waves per CU) x 20000 rounds of four
    32x32x16 bf16 MFMA chains, about 5 ms per launch."""
    import ctypes
    wgs, iters = 1024, 20000
    buf = torch.empty(wgs * 256, dtype=torch.float32, device="cuda:0")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def run():
        if lib.sa_probe_mfma_bf16(ctypes.c_void_p(buf.data_ptr()), wgs, iters,
                                  1 if random_operands else 0, stream):
            raise RuntimeError("sa_probe_mfma_bf16 failed")
    ms = time_steps(torch, run, 10, 3)
    return round(lib.sa_probe_mfma_bf16_flops(wgs, iters) / ms / 1e9, 1)


def gemm_probe(torch):
    """TFLOP/s of torch.matmul (hipBLASLt) on two 8192 x 8192 bf16 matrices: the part's own
    library bf16 GEMM rate."""
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(1)
    n = 8192
    ma = torch.randn(n, n, generator=g, device=dev).to(torch.bfloat16)
    mb = torch.randn(n, n, generator=g, device=dev).to(torch.bfloat16)
    ms = time_steps(torch, lambda: torch.matmul(ma, mb), 20, 5)
    del ma, mb
    return round(2 * n ** 3 / ms / 1e9, 1)


def copy_probe(nbytes):
    import torch
    x = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
    y = torch.empty_like(x)
    for _ in range(5):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": nbytes, "dispatches": 5}))


# ------------------------------------------------------------------------------------------------
# algorithmic work
# ------------------------------------------------------------------------------------------------
def tile_pairs(Sq, Sk, Br, Bc, causal):
    """Unmasked (query, key) pairs of every (query tile, key tile): int64 [nQT, nKT]."""
    nQT, nKT = -(-Sq // Br), -(-Sk // Bc)
    P = np.zeros((nQT, nKT), np.int64)
    for i in range(nQT):
        r0, r1 = i * Br, min(Sq, (i + 1) * Br)
        for j in range(nKT):
            k0, k1 = j * Bc, min(Sk, (j + 1) * Bc)
            if not causal:
                P[i, j] = (r1 - r0) * (k1 - k0)
            else:
                # sum over rows r of #keys k in [k0, k1) with k <= r
                rows = np.arange(r0, r1)
                P[i, j] = np.clip(np.minimum(rows + 1, k1) - k0, 0, None).sum()
    return P


def skip_flops(tile_state, P, D):
    """(computed, dense-equivalent) flops: QK on visited tiles + PV on kept tiles, unmasked."""
    st = tile_state.reshape(-1, *P.shape)
    visited = (st != 2)
    kept = (st == 0)
    computed = 2 * D * (P[None] * visited).sum() + 2 * D * (P[None] * kept).sum()
    dense = 4 * D * P.sum() * st.shape[0]
    return int(computed), int(dense)


def wave_skip_flops(wave_state, P_tile, P_wave, D):
    """Computed flops at wave granularity: QK^T of every tile the query tile visits (all its rows
    are computed whatever each wave decides) + P.V of every (32-row block, key tile) kept.
    wave_state [B*Hq, nR32, nKT]; P_tile [nQT, nKT] (block_q rows); P_wave [nR32, nKT]."""
    st = wave_state.reshape(-1, *P_wave.shape)
    BH = st.shape[0]
    qk = 2 * D * int(P_tile.sum()) * BH          # non-causal: every tile is visited
    pv = 2 * D * int((P_wave[None] * (st == 0)).sum())
    return qk + pv


def sparsity(st):
    return round(float((st == 1).sum() / max(1, (st != 2).sum())), 4)


# ------------------------------------------------------------------------------------------------
# timing
# ------------------------------------------------------------------------------------------------
def time_steps(torch, fn, steps, warmup):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        fn()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def time_ab(torch, arms, steps, warmup, rounds=5):
    """Balanced interleaved A/B timing: `rounds` rounds, each timing every arm for `steps` calls in
    turn (after `warmup` calls of each arm); returns each arm's median per-call ms over the rounds."""
    for fn in arms.values():
        for _ in range(warmup):
            fn()
    res = {name: [] for name in arms}
    for r in range(rounds):
        order = list(arms) if r % 2 == 0 else list(reversed(list(arms)))
        for name in order:
            res[name].append(time_steps(torch, arms[name], steps, 1))
    return {name: float(np.median(v)) for name, v in res.items()}


# ------------------------------------------------------------------------------------------------
# roofline: achieved rate against the published peak, HBM bytes from the committed profiles
# ------------------------------------------------------------------------------------------------
def source_digest(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


_C = "sparse_attention_flash_amd/csrc/"
_COMMON = [_C + "policies.h", _C + "tile_core.h", _C + "mainloop.h", _C + "kernels.h"]
KERNEL_SOURCES = {
    "skip": [_C + "skip_softmax.hip"] + _COMMON,
    "nm": [_C + "nm_softmax.hip"] + _COMMON,
    "skip_nm": [_C + "skip_nm_softmax.hip"] + _COMMON,
    "proxy": [_C + "proxy.hip", _C + "tile_core.h", _C + "mainloop.h", _C + "kernels.h"],
    "decode": [_C + "decode.hip", _C + "tile_core.h", _C + "mainloop.h", _C + "kernels.h"],
}
SKIP_SOURCES = KERNEL_SOURCES["skip"]
DECODE_PROFILE_LAMBDA = 0.1146   # decode workload: target 0.5 lowered through its own fit


def _summary_fields(summary_name):
    path = os.path.join(PROFILES, summary_name)
    if not os.path.exists(path):
        return {}
    fields = {}
    with open(path) as f:
        for line in f:
            key, sep, val = line.partition(":")
            if sep and key.strip() in ("hbm_bytes_per_launch", "source_digest",
                                       "kernel_avg_us"):
                fields[key.strip()] = val.strip()
    return fields


def measured_traffic(summary_name, kind="skip"):
    """HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, each scaled by the plain-copy factor) from
    the committed rocprofv3 summary, if it was taken on the current kernel source, else None."""
    fields = _summary_fields(summary_name)
    if fields.get("source_digest") != source_digest(KERNEL_SOURCES[kind]):
        return None
    return float(fields["hbm_bytes_per_launch"]) if "hbm_bytes_per_launch" in fields else None


def roofline(bound, achieved, summary=None, kind=None):
    """Roofline block of one kernel: achieved TFLOP/s (mfma) or GB/s (hbm) of algorithmic work,
    the published peak, and the profiled HBM bytes per launch when the profile is current."""
    peak = PEAK_BF16_TFLOPS if bound == "mfma" else PEAK_HBM_GBPS
    rec = {"bound": bound, "achieved": round(achieved, 2), "peak": peak,
           "unit": "TFLOP/s" if bound == "mfma" else "GB/s", "frac": round(achieved / peak, 4),
           "traffic": measured_traffic(summary, kind) if summary else None}
    if summary:
        rec["profile"] = "profiles/" + summary
    return rec


# ------------------------------------------------------------------------------------------------
# CPU baseline: the oracle on a bounded sample of the headline workload
# ------------------------------------------------------------------------------------------------
def cpu_baseline(q, k, v, wl, lam, P, target_s):
    import oracle
    B, S, H, D = q.shape
    nQT = P.shape[0]
    rng = np.random.default_rng(0)
    units = rng.permutation(B * H * nQT)
    threads = oracle.num_threads()
    done, flops, t0 = 0, 0, time.perf_counter()
    batch = max(1, threads)
    while done < units.size:
        sel = units[done:done + batch]
        _, _, st, _ = oracle.skip_softmax(q, k, v, causal=wl.causal, block_q=wl.block_q,
                                          block_k=wl.block_k, scale=wl.scale, lam=lam, units=sel)
        qt = sel % nQT
        Pu = P[qt]
        flops += int(2 * D * (Pu * (st != 2)).sum() + 2 * D * (Pu * (st == 0)).sum())
        done += sel.size
        if time.perf_counter() - t0 >= target_s:
            break
    el = time.perf_counter() - t0
    return {"value": round(flops / el / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{done} of {units.size} query tiles (seeded random order) of the "
                      f"{wl.name} workload at the same lambda, float64 oracle, {el:.1f} s"}


def cpu_full_runs():
    """The oracle as written, over every unit of the small, causal-GQA, N:M (2:4) and proxy
    (use_proxy = 1) workloads, on all host cores; wall seconds of each (the CPU baseline's full
    runs, beside the sampled rate of the headline workload)."""
    import oracle
    import workloads as W
    out = {"cores": oracle.num_threads()}
    for name in ("iid_s256_d64", "llm_prefill_gqa_s8192", "llm_prefill_nm_s4096",
                 "proxy_bitmask_s16257"):
        wl = W.WORKLOADS[name]
        q, k, v = wl.generate()
        S = k.shape[1]
        t0 = time.perf_counter()
        if wl.path == "skip":
            lam = wl.param("lambda") if wl.param("lambda") is not None else \
                oracle.threshold(W.CALIB_A, W.CALIB_B, wl.param("target_sparsity"), S)[1]
            _, _, st, _ = oracle.skip_softmax(q, k, v, causal=wl.causal, block_q=wl.block_q,
                                              block_k=wl.block_k, scale=wl.scale, lam=lam)
            extra = {"lambda": lam, "tile_sparsity": sparsity(st)}
        elif wl.path == "nm":
            oracle.nm_softmax(q, k, v, causal=True, scale=wl.scale, n=2, m=4,
                              sink=wl.param("sink"), recent=wl.param("recent"),
                              block_q=wl.block_q)
            extra = {"n:m": "2:4"}
        else:
            nQB, nKB = -(-S // wl.block_q), -(-S // wl.block_k)
            bm = W.gen_bitmask(wl.seed, q.shape[0], q.shape[2], nQB, nKB,
                               int(round(wl.param("density") * nKB)))
            km, vs = W.block_summaries(k, v, wl.block_k)
            oracle.proxy_fwd(q, k, v, km, vs, bm, block_q=wl.block_q, block_k=wl.block_k,
                             scale=wl.scale, use_proxy=1)
            extra = {"use_proxy": 1}
        out[name] = {"seconds": round(time.perf_counter() - t0, 2), **extra}
        print(json.dumps({name: out[name]}), file=sys.stderr, flush=True)
    return out


# ------------------------------------------------------------------------------------------------
# legs
# ------------------------------------------------------------------------------------------------
class Ctx:
    def __init__(self, torch, sa, W, steps, warmup, only):
        self.torch, self.sa, self.W = torch, sa, W
        self.steps, self.warmup, self.only = steps, warmup, only
        self.dev = torch.device("cuda:0")

    def to_dev(self, bits):
        return self.torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(
            self.torch.bfloat16).to(self.dev)


def skip_gqa_leg(c):
    """Causal GQA LLM prefill: skip-softmax at the calibrated lambda and at lambda = 0, the
    threshold giving 50 % tile sparsity by bisection on the counters, and the speedup-vs-sparsity
    curve (X(sigma)) of this workload."""
    torch, sa, W = c.torch, c.sa, c.W
    wl = W.WORKLOADS["llm_prefill_gqa_s8192"]
    q, k, v = wl.generate()
    B, S, Hq, D = q.shape
    qd, kd, vd = c.to_dev(q), c.to_dev(k), c.to_dev(v)
    o = torch.empty_like(qd)
    nQT, nKT = -(-S // wl.block_q), -(-S // wl.block_k)
    st = torch.empty((B, Hq, nQT, nKT), dtype=torch.uint8, device=c.dev)
    cnt = torch.zeros((B, Hq, 2), dtype=torch.int32, device=c.dev)
    _, lam, _ = sa.sa_threshold_from_calib(W.CALIB_A, W.CALIB_B, wl.param("target_sparsity"), S)
    P = tile_pairs(S, S, wl.block_q, wl.block_k, True)

    def run(lm):
        return lambda: sa.sa_skip_softmax_fwd(qd, kd, vd, o, lm, causal=True,
                                              block_q=wl.block_q, block_k=wl.block_k,
                                              tile_state=st)

    def measure(name, ms, lm):
        run(lm)()
        ts = st.cpu().numpy()
        comp, dense = skip_flops(ts, P, D)
        return {"lambda": lm, "ms": round(ms, 4), "computed_tflops": round(comp / ms / 1e9, 2),
                "dense_equiv_tflops": round(dense / ms / 1e9, 2), "tile_sparsity": sparsity(ts)}

    if c.only:
        ms = time_steps(torch, run(lam), c.steps, c.warmup)
        rec = {"calibrated": measure("calibrated", ms, lam)}
        rec["roofline"] = roofline("mfma", rec["calibrated"]["computed_tflops"],
                                   "skip_softmax_llm_prefill_gqa_s8192.txt", "skip")
        return rec

    def sparsity_at(lm):
        cnt.zero_()
        sa.sa_skip_softmax_fwd(qd, kd, vd, o, lm, causal=True, block_q=wl.block_q,
                               block_k=wl.block_k, head_counters=cnt)
        cc = cnt.cpu().numpy().astype(np.int64)
        return float(cc[..., 1].sum() / max(1, cc[..., 0].sum()))

    # lambda giving 50 % tile sparsity: bisection on log(lambda) over the GPU counters
    lo, hi = 0.25, 4.0
    s_lo, s_hi = sparsity_at(lo), sparsity_at(hi)
    for _ in range(24):
        mid = math.sqrt(lo * hi)
        s_mid = sparsity_at(mid)
        if s_mid < 0.5:
            lo, s_lo = mid, s_mid
        else:
            hi, s_hi = mid, s_mid
    lam50 = hi
    curve_l = [0.0, 0.5, 0.8, 1.0, lam50, lam, 2.0, 3.0, 6.0]
    arms = {f"{lm:.6g}": run(lm) for lm in curve_l}
    times = time_ab(torch, arms, c.steps, c.warmup)
    ms0 = times["0"]
    curve = []
    for lm in curve_l:
        r = measure(f"{lm:.6g}", times[f"{lm:.6g}"], lm)
        r["speedup_vs_lambda0"] = round(ms0 / r["ms"], 3)
        curve.append(r)
    by = {r["lambda"]: r for r in curve}
    rec = {"lambda": lam, "calibrated": by[lam], "lambda0": by[0.0],
           "speedup_vs_lambda0": by[lam]["speedup_vs_lambda0"],
           "lambda50": {**by[lam50], "bisection": f"log-lambda bisection over the head "
                                                  f"counters, bracket [{lo:.6g}, {hi:.6g}]"},
           "speedup_curve": curve,
           "timing": "median of 5 balanced interleaved rounds per arm"}
    rec["roofline"] = roofline("mfma", by[lam]["computed_tflops"],
                               "skip_softmax_llm_prefill_gqa_s8192.txt", "skip")
    return rec


NM_ARMS = ((2, 4), (4, 4), (1, 4), (3, 4), (1, 8), (4, 8), (7, 8))
NM_PROFILES = {(2, 4): "nm_softmax_llm_prefill_nm_s4096_2of4.txt",
               (4, 8): "nm_softmax_llm_prefill_nm_s4096_4of8.txt"}


def nm_leg(c, arm=None):
    """Causal N:M sparse softmax (no flop saving by design: computed = dense-equivalent)."""
    torch, sa, W = c.torch, c.sa, c.W
    wl = W.WORKLOADS["llm_prefill_nm_s4096"]
    q, k, v = wl.generate()
    B, S, H, D = q.shape
    qd, kd, vd = c.to_dev(q), c.to_dev(k), c.to_dev(v)
    o = torch.empty_like(qd)
    dense = 4 * D * tile_pairs(S, S, wl.block_q, wl.block_k, True).sum() * B * H
    arms_nm = (arm,) if arm else NM_ARMS
    arms = {f"{n}:{m}": (lambda n=n, m=m: sa.sa_nm_softmax_fwd(
        qd, kd, vd, o, n, m, wl.param("sink"), wl.param("recent"), causal=True,
        block_q=wl.block_q, block_k=wl.block_k)) for n, m in arms_nm}
    if arm:
        times = {f"{arm[0]}:{arm[1]}": time_steps(torch, next(iter(arms.values())), c.steps,
                                                  c.warmup)}
    else:
        times = time_ab(torch, arms, c.steps, c.warmup)
    rec = {}
    for (n, m) in arms_nm:
        ms = times[f"{n}:{m}"]
        tf = dense / ms / 1e9
        rec[f"{n}:{m}"] = {"ms": round(ms, 4), "dense_equiv_tflops": round(tf, 2),
                           "roofline": roofline("mfma", tf, NM_PROFILES.get((n, m)), "nm")}
    if not arm:
        rec["overhead_2:4_vs_4:4"] = round(rec["2:4"]["ms"] / rec["4:4"]["ms"] - 1, 4)
        rec["timing"] = "median of 5 balanced interleaved rounds per arm"
    rec["note"] = "every visited tile runs QK^T and P.V, so computed flops = dense-equivalent"
    return rec


def skip_nm_leg(c):
    """Skip-softmax with 2:4 inside kept tiles, lambda lowered from target 0.5, and lambda = 0."""
    torch, sa, W = c.torch, c.sa, c.W
    wl = W.WORKLOADS["llm_prefill_nm_s4096"]
    q, k, v = wl.generate()
    B, S, H, D = q.shape
    qd, kd, vd = c.to_dev(q), c.to_dev(k), c.to_dev(v)
    o = torch.empty_like(qd)
    nQT, nKT = -(-S // wl.block_q), -(-S // wl.block_k)
    st = torch.empty((B, H, nQT, nKT), dtype=torch.uint8, device=c.dev)
    _, lam, _ = sa.sa_threshold_from_calib(W.CALIB_A, W.CALIB_B, 0.5, S)
    P = tile_pairs(S, S, wl.block_q, wl.block_k, True)
    rec = {"n:m": "2:4", "lambda": lam}
    lams = (("calibrated", lam),) if c.only else (("calibrated", lam), ("lambda0", 0.0))
    arms = {name: (lambda lm=lm: sa.sa_skip_nm_softmax_fwd(
        qd, kd, vd, o, lm, 2, 4, wl.param("sink"), wl.param("recent"), causal=True,
        block_q=wl.block_q, block_k=wl.block_k, tile_state=st)) for name, lm in lams}
    if c.only:
        times = {"calibrated": time_steps(torch, arms["calibrated"], c.steps, c.warmup)}
    else:
        times = time_ab(torch, arms, c.steps, c.warmup)
    for name, _ in lams:
        ms = times[name]
        arms[name]()
        ts = st.cpu().numpy()
        comp, dense_eq = skip_flops(ts, P, D)
        rec[name] = {"ms": round(ms, 4), "computed_tflops": round(comp / ms / 1e9, 2),
                     "dense_equiv_tflops": round(dense_eq / ms / 1e9, 2),
                     "tile_sparsity": sparsity(ts)}
    if not c.only:
        rec["speedup_vs_lambda0"] = round(rec["lambda0"]["ms"] / rec["calibrated"]["ms"], 3)
        rec["timing"] = "median of 5 balanced interleaved rounds per arm"
    rec["roofline"] = roofline("mfma", rec["calibrated"]["computed_tflops"],
                               "skip_nm_softmax_llm_prefill_nm_s4096.txt", "skip_nm")
    return rec


def proxy_leg(c, name):
    """Route prep and proxy forward (proxy off / on) on one workload; "wrapper" = prep + forward,
    as the pages time their run call."""
    torch, sa, W = c.torch, c.sa, c.W
    wl = W.WORKLOADS[name]
    q, k, v = wl.generate()
    B, S, H, D = q.shape
    Bq, Bk = wl.block_q, wl.block_k
    nQB, nKB = -(-S // Bq), -(-S // Bk)
    n_set = int(round(wl.param("density") * nKB))
    bm = W.gen_bitmask(wl.seed, B, H, nQB, nKB, n_set)
    km, vs = W.block_summaries(k, v, Bk)
    qd, kd, vd, kmd, vsd = c.to_dev(q), c.to_dev(k), c.to_dev(v), c.to_dev(km), c.to_dev(vs)
    o = torch.empty_like(qd)
    bmd = torch.from_numpy(bm.view(np.int32)).to(c.dev)
    n_exact = torch.empty((B, H, nQB), dtype=torch.int32, device=c.dev)
    idx = torch.empty((B, H, nQB, nKB), dtype=torch.int32, device=c.dev)
    keep = torch.empty_like(bmd)
    rec = {"shape": [B, S, H, D], "block_q": Bq, "block_k": Bk, "exact_blocks_per_row": n_set,
           "n_kv_blocks": nKB}
    summary = ("proxy_bitmask_s16257.txt" if name == "proxy_bitmask_s16257"
               else "proxy_pc_page_s32760.txt")

    def prep():
        sa.sa_bitmask_route_prep(bmd, n_exact, idx, keep, batch=B, heads_kv=H, seqlen_q=S,
                                 seqlen_k=S, block_q=Bq, block_k=Bk)

    prep()
    torch.cuda.synchronize()
    ne = n_exact.cpu().numpy().astype(np.int64)
    # exact work: every query row against the tokens of its exact blocks
    lens = np.minimum(Bk, S - np.arange(nKB) * Bk)
    rows = np.minimum(Bq, S - np.arange(nQB) * Bq)
    ix = idx.cpu().numpy()
    exact_tokens = np.where(ix >= 0, lens[np.clip(ix, 0, None)], 0).sum(-1)   # [B,H,nQB]
    exact_flops = int(4 * D * (exact_tokens * rows[None, None]).sum())
    proxy_flops = int(4 * D * ((nKB - ne) * rows[None, None]).sum())

    def fwd(use):
        sa.sa_proxy_block_sparse_fwd(qd, kd, vd, kmd, vsd, n_exact, idx, keep, use, o,
                                     block_q=Bq, block_k=Bk)

    if c.only:
        ms = time_steps(torch, lambda: fwd(1), c.steps, c.warmup)
        fl = exact_flops + proxy_flops
        rec["proxy_on"] = {"ms": round(ms, 4), "computed_tflops": round(fl / ms / 1e9, 2)}
        rec["roofline"] = roofline("mfma", fl / ms / 1e9, summary, "proxy")
        return rec

    rec["route_prep_ms"] = round(time_steps(torch, prep, c.steps, c.warmup), 5)

    def wrapper(use):
        prep()
        fwd(use)

    # the pages' method: balanced, interleaved rounds per arm
    t = time_ab(torch, {"off": lambda: fwd(0), "on": lambda: fwd(1),
                        "w_off": lambda: wrapper(0), "w_on": lambda: wrapper(1)},
                c.steps, c.warmup)
    for arm, use in (("proxy_off", 0), ("proxy_on", 1)):
        ms, ms_w = t["on" if use else "off"], t["w_on" if use else "w_off"]
        fl = exact_flops + (proxy_flops if use else 0)
        rec[arm] = {"ms": round(ms, 4), "wrapper_ms": round(ms_w, 4),
                    "computed_tflops": round(fl / ms / 1e9, 2)}
    rec["proxy_overhead"] = round(rec["proxy_on"]["ms"] / rec["proxy_off"]["ms"] - 1, 4)
    rec["timing"] = "median of 5 balanced interleaved rounds per arm"
    rec["roofline"] = roofline("mfma", rec["proxy_on"]["computed_tflops"], summary, "proxy")
    return rec


def decode_leg(c):
    """Decode skip-softmax at the pages' decode threshold, at a threshold calibrated for 50 %
    tile sparsity, and at lambda = 0, with its HBM roofline (algorithmic bytes: K of every visited
    key, V of every key in a tile kept by some head of its KV group, q and o)."""
    torch, sa, W = c.torch, c.sa, c.W
    wl = W.WORKLOADS["llm_decode_gqa_kv8192"]
    q, k, v, lens = wl.generate()
    B, _, Hq, D = q.shape
    S, Hkv = k.shape[1], k.shape[2]
    G, BC = Hq // Hkv, wl.block_k
    nKT = -(-S // BC)
    qd, kd, vd = c.to_dev(q), c.to_dev(k), c.to_dev(v)
    o = torch.empty_like(qd)
    ln = torch.from_numpy(lens).to(c.dev)
    st = torch.empty((B, Hq, nKT), dtype=torch.uint8, device=c.dev)
    cnt = torch.zeros((B, Hq, 2), dtype=torch.int32, device=c.dev)
    nbytes, _ = sa.sa_skip_softmax_decode_workspace(qd, kd, 1.0, block_k=BC)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=c.dev)
    kw = dict(block_k=BC, seqlens_k=ln, workspace=ws)

    def sparsity_at(lam):
        cnt.zero_()
        sa.sa_skip_softmax_decode_fwd(qd, kd, vd, o, lam, head_counters=cnt, **kw)
        cc = cnt.cpu().numpy().astype(np.int64)
        return float(cc[..., 1].sum() / max(1, cc[..., 0].sum()))

    rec = {"batch": B, "heads_q": Hq, "heads_kv": Hkv, "cache": S, "keys": int(lens.sum()),
           "tile": BC}
    if c.only:
        # the threshold a calibration sweep of this workload lowers target 0.5 to (recorded in
        # the full bench line); no sweep, so that the profile holds only the timed steps
        legs = (("calibrated", DECODE_PROFILE_LAMBDA),)
    else:
        trials = [t for t in W.THRESHOLD_TRIALS if t <= 1.0]
        sp = [sparsity_at(t) for t in trials]
        rec["calibration"] = {"trials": trials, "sparsity": [round(x, 4) for x in sp]}
        try:
            a, b, lo, hi = sa.sa_fit_threshold_calib(trials, sp, S)
            lam_cal = min(1.0, sa.sa_threshold_from_calib(a, b, wl.param("target_sparsity"), S)[1])
            rec["calibration"].update({"fit_a": a, "fit_b": b, "fit_range": [lo, hi]})
        except sa.SaError:
            lam_cal = 1.0   # no usable trials: the largest threshold that keeps the split exact
        legs = (("lambda_page", wl.param("lambda")), ("calibrated", lam_cal), ("lambda0", 0.0))
    keys_b = lens.astype(np.int64)
    qo_bytes = 2 * B * Hq * D * 2
    for name, lam in legs:
        ms = time_steps(torch, lambda: sa.sa_skip_softmax_decode_fwd(
            qd, kd, vd, o, lam, tile_state=st, **kw), c.steps, c.warmup)
        ts = st.cpu().numpy().reshape(B, Hkv, G, nKT)
        kept_any = (ts == 0).any(axis=2)                                   # [B, Hkv, nKT]
        tile_keys = np.clip(keys_b[:, None] - np.arange(nKT)[None, :] * BC, 0, BC)   # [B, nKT]
        k_bytes = int(keys_b.sum()) * Hkv * D * 2
        v_bytes = int((kept_any * tile_keys[:, None, :]).sum()) * D * 2
        alg = k_bytes + v_bytes + qo_bytes
        rec[name] = {"lambda": lam, "ms": round(ms, 4), "tile_sparsity": sparsity(ts),
                     "alg_bytes": alg, "gbps": round(alg / ms / 1e6, 1),
                     "hbm_frac": round(alg / ms / 1e6 / PEAK_HBM_GBPS, 4)}
    if not c.only:
        rec["speedup_calibrated_vs_lambda0"] = round(
            rec["lambda0"]["ms"] / rec["calibrated"]["ms"], 3)
    rec["roofline"] = roofline("hbm", rec["calibrated"]["gbps"],
                               "skip_softmax_decode_llm_gqa_kv8192.txt", "decode")
    rec["note"] = ("roofline.achieved counts the algorithmic bytes of one step (three kernels) "
                   "over the step's time")
    return rec


def video_variant_leg(c, head, kind):
    """The headline workload at the pages' 128x128 decision tiles (kind "bk128") or with every
    32-row wavefront deciding alone (kind "wave"), at the same calibrated lambda and at lambda =
    0 (decision granularity and tile change the tile sparsity the threshold reaches)."""
    torch, sa = c.torch, c.sa
    qd, kd, vd, o, wl, lam, ms_tile = head
    B, S, H, D = qd.shape
    Br = wl.block_q
    Bc = 128 if kind == "bk128" else wl.block_k
    R = 32 if kind == "wave" else Br
    nR, nKT = -(-S // R), -(-S // Bc)
    st = torch.empty((B, H, nR, nKT), dtype=torch.uint8, device=c.dev)

    def run(lm):
        if kind == "wave":
            return lambda: sa.sa_skip_softmax_fwd_ex(qd, kd, vd, o, lm, "wave", causal=wl.causal,
                                                     block_q=Br, block_k=Bc, tile_state=st)
        return lambda: sa.sa_skip_softmax_fwd(qd, kd, vd, o, lm, causal=wl.causal, block_q=Br,
                                              block_k=Bc, tile_state=st)

    lams = (("calibrated", lam),) if c.only else (("calibrated", lam), ("lambda0", 0.0))
    rec = {"lambda": lam, "tile": f"{Br}x{Bc}",
           "granularity": "32-row wavefront" if kind == "wave" else "tile"}
    P_tile = tile_pairs(S, S, Br, Bc, wl.causal)
    P_dec = tile_pairs(S, S, R, Bc, wl.causal)
    for name, lm in lams:
        ms = time_steps(torch, run(lm), c.steps, c.warmup)
        ts = st.cpu().numpy()
        if kind == "wave":
            comp = wave_skip_flops(ts, P_tile, P_dec, D)
            dense = 4 * D * int(P_tile.sum()) * B * H
        else:
            comp, dense = skip_flops(ts, P_dec, D)
        rec[name] = {"ms": round(ms, 4), "tile_sparsity": sparsity(ts),
                     "computed_tflops": round(comp / ms / 1e9, 2),
                     "dense_equiv_tflops": round(dense / ms / 1e9, 2)}
    if not c.only:
        rec["speedup_vs_lambda0"] = round(rec["lambda0"]["ms"] / rec["calibrated"]["ms"], 3)
        rec["speedup_vs_headline_tile_64"] = round(ms_tile / rec["calibrated"]["ms"], 3)
    rec["roofline"] = roofline("mfma", rec["calibrated"]["computed_tflops"],
                               f"skip_softmax_video_dit_s32760_{kind}.txt", "skip")
    return rec


# ------------------------------------------------------------------------------------------------
def speedup_curve(torch, sa, W, qd, kd, vd, o, st, wl, P, D, ms0, steps, warmup):
    """The headline kernel over a range of thresholds: tile sparsity, time, computed TFLOP/s and
    speedup against the same kernel at lambda = 0 (untimed by the headline value)."""
    S = qd.shape[1]
    lams = [0.1, 0.2, 0.3, 0.5, 0.7, 1.5, 3.0]
    for target in (0.5, 0.7):
        lams.append(sa.sa_threshold_from_calib(W.CALIB_A, W.CALIB_B, target, S)[1])
    rows = []
    for lam in sorted(lams):
        ms = time_steps(torch, lambda: sa.sa_skip_softmax_fwd(
            qd, kd, vd, o, lam, causal=wl.causal, block_q=wl.block_q, block_k=wl.block_k,
            tile_state=st), steps, warmup)
        ts = st.cpu().numpy()
        computed, _ = skip_flops(ts, P, D)
        rows.append({"lambda": round(lam, 6), "tile_sparsity": sparsity(ts),
                     "ms": round(ms, 4), "computed_tflops": round(computed / ms / 1e9, 2),
                     "speedup_vs_lambda0": round(ms0 / ms, 3)})
    return rows


def calibration(sa, W, qd, kd, vd, o, cnt, wl, S):
    """Calibration sweep over the pages' trial thresholds on the headline workload, the log-space
    fit of the measured sparsities, and the sparsity reached when targets are lowered through the
    fitted model (untimed)."""
    trials = W.THRESHOLD_TRIALS
    kw = dict(causal=wl.causal, block_q=wl.block_q, block_k=wl.block_k)
    t0 = time.perf_counter()
    sp = sa.sa_skip_softmax_calibrate(qd, kd, vd, o, trials, cnt, **kw)
    a, b, lo, hi = sa.sa_fit_threshold_calib(trials, sp, S)
    reached = {}
    for target in (0.5, 0.7):
        _, lam, _ = sa.sa_threshold_from_calib(a, b, target, S)
        reached[str(target)] = {"lambda": lam, "sparsity": round(
            sa.sa_skip_softmax_calibrate(qd, kd, vd, o, [lam], cnt, **kw)[0], 4)}
    cnt.zero_()
    return {"trials": trials, "sparsity": [round(x, 4) for x in sp], "fit_a": a, "fit_b": b,
            "fit_range": [lo, hi], "targets": reached,
            "sweep_and_fit_s": round(time.perf_counter() - t0, 3)}


def run_one(c, leg):
    """One leg alone (its main arm only), for profiler runs."""
    if leg == "skip_gqa":
        return skip_gqa_leg(c)
    if leg.startswith("nm"):
        parts = leg.split(":")
        arm = (int(parts[1]), int(parts[2])) if len(parts) == 3 else (2, 4)
        return nm_leg(c, arm)
    if leg == "skip_nm":
        return skip_nm_leg(c)
    if leg == "decode":
        return decode_leg(c)
    if leg.startswith("proxy_"):
        return proxy_leg(c, leg)
    raise SystemExit(f"unknown leg {leg!r}: one of {', '.join(LEGS)}")


def main(argv=None):
    args = parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the kernels are "
              "single-GPU and no multi-GPU path is part of this library", file=sys.stderr)
        sys.exit(2)
    if args.cpu_full_runs:
        print(json.dumps(cpu_full_runs()))
        return
    if args.peak_probes:
        print(json.dumps(peak_probes()))
        return
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    if args.profile:
        args.only = "headline"
    only = args.only
    if only and only.split(":")[0] not in LEGS:
        raise SystemExit(f"unknown leg {only!r}: one of {', '.join(LEGS)}")

    import torch
    import sparse_attention_flash_amd as sa
    import workloads as W

    c = Ctx(torch, sa, W, args.steps, args.warmup, bool(only))
    if only and only not in ("headline", "video_bk128", "video_wave"):
        print(json.dumps(run_one(c, only)))
        return
    dev = c.dev
    to_dev = c.to_dev

    wl = W.WORKLOADS[HEADLINE]
    t_gen = time.perf_counter()
    q, k, v = wl.generate()
    t_gen = time.perf_counter() - t_gen
    B, S, H, D = q.shape
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    o = torch.empty_like(qd)
    Br, Bc = wl.block_q, wl.block_k
    nQT, nKT = -(-S // Br), -(-S // Bc)
    st = torch.empty((B, H, nQT, nKT), dtype=torch.uint8, device=dev)
    cnt = torch.zeros((B, H, 2), dtype=torch.int32, device=dev)
    target = wl.param("target_sparsity")
    _, lam, log2_lam = sa.sa_threshold_from_calib(W.CALIB_A, W.CALIB_B, target, S)
    if only in ("video_bk128", "video_wave"):
        rec = video_variant_leg(c, (qd, kd, vd, o, wl, lam, float("nan")), only.split("_")[1])
        print(json.dumps(rec))
        return
    calls = [0]

    def step():
        _, lam_k, _ = sa.sa_threshold_from_calib(W.CALIB_A, W.CALIB_B, target, S)
        sa.sa_skip_softmax_fwd(qd, kd, vd, o, lam_k, causal=wl.causal, block_q=Br, block_k=Bc,
                               tile_state=st, head_counters=cnt)
        calls[0] += 1

    ms = time_steps(torch, step, args.steps, args.warmup)
    P = tile_pairs(S, S, Br, Bc, wl.causal)
    tile_state = st.cpu().numpy()
    computed, dense = skip_flops(tile_state, P, D)
    counters = cnt.cpu().numpy().astype(np.int64)
    visited, skipped = counters[..., 0].sum() // calls[0], counters[..., 1].sum() // calls[0]
    tile_sp = skipped / max(1, visited)
    tflops = computed / (ms * 1e-3) / 1e12

    # the same kernel and build at lambda = 0 (dense baseline)
    def step0():
        sa.sa_skip_softmax_fwd(qd, kd, vd, o, 0.0, causal=wl.causal, block_q=Br, block_k=Bc,
                               tile_state=st, head_counters=cnt)

    ms0 = float("nan") if only else time_steps(torch, step0, args.steps, args.warmup)
    computed0, _ = skip_flops(np.zeros_like(tile_state), P, D)

    result = {
        "metric": "attention TFLOP/s (computed + dense-equiv) & % bf16 MFMA peak at 50% sparsity",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded video-DiT-like Q/K/V with 3-D Gaussian locality bias; "
                "no dataset or weights)",
        "config": {"workload": HEADLINE, "batch": B, "heads": H, "seq_len": S, "head_dim": D,
                   "causal": wl.causal, "tile": f"{Br}x{Bc}", "target_sparsity": target,
                   "lambda": lam, "log2_lambda": log2_lam},
        "roofline": roofline("mfma", tflops, "skip_softmax_video_dit_s32760.txt", "skip"),
        "dense_equiv_tflops": round(dense / (ms * 1e-3) / 1e12, 2),
        "pct_bf16_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "tile_sparsity": round(float(tile_sp), 4),
        "lambda0_ms": None if only else round(ms0, 4),
        "lambda0_tflops": None if only else round(computed0 / (ms0 * 1e-3) / 1e12, 2),
        "speedup_vs_lambda0": None if only else round(ms0 / ms, 3),
        "computed_flops_per_step": computed,
        "dense_flops_per_step": dense,
        "input_generation_s": round(t_gen, 1),
        "timing": "hipEvent over the timed steps on the launch stream; L2/MALL not flushed "
                  "between steps",
    }
    prof = _summary_fields("skip_softmax_video_dit_s32760.txt")
    if "kernel_avg_us" in prof:
        result["roofline"]["profile_kernel_avg_us"] = float(prof["kernel_avg_us"])
        result["roofline"]["profile_note"] = (
            "the profiled average comes from another run (another lease of the part); runs of "
            "this step spread about +-4 % from box to box, so achieved and the profiled duration "
            "agree to that spread")
    if not args.no_paths and not only:
        result["speedup_curve"] = speedup_curve(torch, sa, W, qd, kd, vd, o, st, wl, P, D, ms0,
                                                args.steps, args.warmup)
        result["calibration"] = calibration(sa, W, qd, kd, vd, o, cnt, wl, S)
        head = (qd, kd, vd, o, wl, lam, ms)
        paths = {"video_dit_s32760_bk128": video_variant_leg(c, head, "bk128"),
                 "video_dit_s32760_wave": video_variant_leg(c, head, "wave")}
        del qd, kd, vd, o, head
        torch.cuda.empty_cache()
        paths["llm_prefill_gqa_s8192"] = skip_gqa_leg(c)
        paths["llm_prefill_nm_s4096"] = nm_leg(c)
        paths["llm_prefill_skip_nm_s4096"] = skip_nm_leg(c)
        paths["llm_prefill_skip_nm_s4096"]["speedup_vs_nm_2:4"] = round(
            paths["llm_prefill_nm_s4096"]["2:4"]["ms"] /
            paths["llm_prefill_skip_nm_s4096"]["calibrated"]["ms"], 3)
        paths["llm_decode_gqa_kv8192"] = decode_leg(c)
        for name in ("proxy_bitmask_s16257", "proxy_page_s32760"):
            paths[name] = proxy_leg(c, name)
        paths["proxy_page_s32760"]["context_b200_pages"] = {
            "note": "NVIDIA B200, FlashInfer block-sparse wrapper; other hardware, context only",
            "wrapper_ms_off_on": [1.3172, 1.4298], "attention_ms_off_on": [1.1261, 1.2121],
            "prep_ms_off_on": [0.0145, 0.0176]}
        result["paths"] = paths
        # the part's library bf16 GEMM and its matrix-core rate on random operands in the same
        # run (same lease, clocks and thermals), as reference points for the headline's rate; not
        # part of the roofline, which uses the published peak
        gemm = gemm_probe(torch)
        mfma = mfma_probe(torch, probe_lib(), True)
        result["same_run_reference"] = {"hipblaslt_bf16_gemm_8192_tflops": gemm,
                                        "headline_over_gemm": round(tflops / gemm, 3),
                                        "mfma_bf16_random_operands_tflops": mfma,
                                        "headline_over_mfma": round(tflops / mfma, 3)}
    if not args.no_cpu_baseline and not only:
        result["cpu_baseline"] = cpu_baseline(q, k, v, wl, lam, P, args.cpu_seconds)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
