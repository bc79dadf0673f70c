"""Seeded synthetic inputs for the sparse flash-attention paths.

This module is shared by the tests, the benchmark and the smoke check.  It holds only input
generation -- no step of any attention method -- and neither the HIP package nor the oracle is
imported here.  Every generator is a function of (seed, shape) alone and returns bf16 bit patterns
(numpy ``uint16``) in ``[B, S, H, D]`` layout, so the GPU path and the oracle read identical bits.

Generators (each a stand-in for a workload the pages describe but do not ship):

* ``gen_iid``   -- Q, K, V iid N(0, 1) (``gen_iid_f32``: the same values before bf16 rounding).
* ``gen_llm``   -- LLM-prefill-like: per (batch, KV head) an AR(1) latent (rho 0.9, stationary
  N(0, I)) shared by Q and K, so nearby tokens attend to each other; a per-KV-head unit direction u
  with amplitude alpha = sqrt(sink_nats * sqrt(D)) added to every query and to the first
  ``n_sink`` keys, so each query's scaled logit on those keys is raised by ``sink_nats`` on
  average (attention sinks).  V iid N(0, 1).
* ``gen_llm_decode`` -- one decode step on the LLM generator: K/V built as ``gen_llm`` builds
  them, one query per head made like ``gen_llm``'s query at the sequence's last position, and
  (optionally) ragged sequence lengths drawn uniformly from [S/2, S].
* ``gen_video`` -- video-DiT-like: a 3-D (frame, row, col) token grid; Q = (E_q + Pos)/sqrt(2),
  K = (E_k + Pos)/sqrt(2) with Pos = sqrt(D) * W phi(t), phi a rank-64 random-Fourier embedding
  whose kernel is a separable Gaussian with the given sigmas (frames, rows, cols), W a D x 64
  orthonormal map.  The scaled logit between two tokens is then biased by about
  sqrt(D)/2 * exp(-|dpos / sigma|^2 / 2).  V iid N(0, 1).
* ``gen_bitmask`` -- exact-block bitmaps per (batch, KV head, query block): a fixed number of set
  bits, always including block 0 and the diagonal block, the rest uniform without replacement;
  packed LSB first into uint32 words.  Optional garbage in the padding bits.
* ``block_summaries`` -- the caller-provided proxy summaries: per KV block, the arithmetic mean of
  K over the block's true tokens and the sum of V over them, in double from the bf16 values, then
  rounded to bf16.  (The pages leave summary construction to the caller.)

Random streams come from ``numpy.random.Generator(PCG64(SeedSequence([seed, tag, ...])))``.
"""
from __future__ import annotations

import dataclasses
import math
import os

import numpy as np

try:  # scipy only speeds up the AR(1) recursion; a plain loop gives the same numbers
    from scipy.signal import lfilter as _lfilter
except Exception:  # pragma: no cover
    _lfilter = None


def to_bf16_bits(x) -> np.ndarray:
    """Round float values to bf16 (round to nearest even) and return the bit patterns as uint16."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits) -> np.ndarray:
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return (b.astype(np.uint32) << 16).view(np.float32)


def _rng(seed, *tags):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), *map(int, tags)])))


def _normal(rng, shape):
    return rng.standard_normal(shape, dtype=np.float32)


def gen_iid(seed, B, Sq, Sk, Hq, Hkv, D):
    """Q [B,Sq,Hq,D], K/V [B,Sk,Hkv,D], iid N(0,1), rounded to bf16."""
    q = np.empty((B, Sq, Hq, D), np.uint16)
    k = np.empty((B, Sk, Hkv, D), np.uint16)
    v = np.empty((B, Sk, Hkv, D), np.uint16)
    for b in range(B):
        for h in range(Hq):
            q[b, :, h] = to_bf16_bits(_normal(_rng(seed, 1, b, h), (Sq, D)))
        for h in range(Hkv):
            k[b, :, h] = to_bf16_bits(_normal(_rng(seed, 2, b, h), (Sk, D)))
            v[b, :, h] = to_bf16_bits(_normal(_rng(seed, 3, b, h), (Sk, D)))
    return q, k, v


def gen_iid_f32(seed, B, Sq, Sk, Hq, Hkv, D):
    """The float32 values gen_iid draws, before their rounding to bf16 (same streams)."""
    q = np.empty((B, Sq, Hq, D), np.float32)
    k = np.empty((B, Sk, Hkv, D), np.float32)
    v = np.empty((B, Sk, Hkv, D), np.float32)
    for b in range(B):
        for h in range(Hq):
            q[b, :, h] = _normal(_rng(seed, 1, b, h), (Sq, D))
        for h in range(Hkv):
            k[b, :, h] = _normal(_rng(seed, 2, b, h), (Sk, D))
            v[b, :, h] = _normal(_rng(seed, 3, b, h), (Sk, D))
    return q, k, v


def _ar1(eps: np.ndarray, rho: float) -> np.ndarray:
    """Stationary AR(1) along axis 0: x0 = e0, x_t = rho x_{t-1} + sqrt(1-rho^2) e_t."""
    drive = eps * math.sqrt(1.0 - rho * rho)
    drive[0] = eps[0]
    if _lfilter is not None:
        return _lfilter([1.0], [1.0, -rho], drive, axis=0)
    out = np.empty_like(drive)
    out[0] = drive[0]
    for t in range(1, drive.shape[0]):
        out[t] = rho * out[t - 1] + drive[t]
    return out


def gen_llm(seed, B, S, Hq, Hkv, D, rho=0.9, n_sink=4, sink_nats=3.0):
    """LLM-prefill-like Q/K/V (see module docstring); Sq == Sk == S."""
    q = np.empty((B, S, Hq, D), np.uint16)
    k = np.empty((B, S, Hkv, D), np.uint16)
    v = np.empty((B, S, Hkv, D), np.uint16)
    G = Hq // Hkv
    alpha = math.sqrt(sink_nats * math.sqrt(D))
    for b in range(B):
        for hk in range(Hkv):
            rng = _rng(seed, 10, b, hk)
            x = _ar1(rng.standard_normal((S, D)), rho)
            u = rng.standard_normal(D)
            u /= np.linalg.norm(u)
            ek = rng.standard_normal((S, D))
            kk = (x + ek) / math.sqrt(2.0)
            kk[:n_sink] += alpha * u
            k[b, :, hk] = to_bf16_bits(kk)
            v[b, :, hk] = to_bf16_bits(_normal(_rng(seed, 11, b, hk), (S, D)))
            for g in range(G):
                hq = hk * G + g
                eq = _rng(seed, 12, b, hq).standard_normal((S, D))
                q[b, :, hq] = to_bf16_bits((x + eq) / math.sqrt(2.0) + alpha * u)
    return q, k, v


def gen_llm_decode(seed, B, S, Hq, Hkv, D, rho=0.9, n_sink=4, sink_nats=3.0, ragged=True):
    """Decode-step inputs on the LLM generator: K/V [B,S,Hkv,D] as gen_llm builds them (latent
    AR(1) keys with sink tokens) and one query per head, q [B,1,Hq,D], made like gen_llm's query at
    the sequence's last position.  With ragged=True sequence b holds lens[b] keys, drawn uniformly
    from [S/2, S] (the last sequence always holds S); otherwise every sequence holds S.  Returns
    (q, k, v, lens int32 [B])."""
    q = np.empty((B, 1, Hq, D), np.uint16)
    k = np.empty((B, S, Hkv, D), np.uint16)
    v = np.empty((B, S, Hkv, D), np.uint16)
    G = Hq // Hkv
    alpha = math.sqrt(sink_nats * math.sqrt(D))
    lens = np.full(B, S, np.int32)
    if ragged and B > 1:
        lens[:-1] = _rng(seed, 14).integers(S // 2, S + 1, size=B - 1)

    def one(bh):
        b, hk = bh
        last = int(lens[b]) - 1
        rng = _rng(seed, 10, b, hk)
        x = _ar1(rng.standard_normal((S, D)), rho)
        u = rng.standard_normal(D)
        u /= np.linalg.norm(u)
        ek = rng.standard_normal((S, D))
        kk = (x + ek) / math.sqrt(2.0)
        kk[:n_sink] += alpha * u
        k[b, :, hk] = to_bf16_bits(kk)
        v[b, :, hk] = to_bf16_bits(_normal(_rng(seed, 11, b, hk), (S, D)))
        for g in range(G):
            hq = hk * G + g
            eq = _rng(seed, 13, b, hq).standard_normal(D)
            q[b, 0, hq] = to_bf16_bits((x[max(last, 0)] + eq) / math.sqrt(2.0) + alpha * u)

    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(min(16, os.cpu_count() or 1)) as ex:
        list(ex.map(one, [(b, hk) for b in range(B) for hk in range(Hkv)]))
    return q, k, v, lens


def video_positions(frames, rows, cols):
    f, r, c = np.meshgrid(np.arange(frames), np.arange(rows), np.arange(cols), indexing="ij")
    return np.stack([f.ravel(), r.ravel(), c.ravel()], axis=1).astype(np.float64)


def _video_head(seed, b, h, D, pos, sigma, rank):
    S = pos.shape[0]
    rng = _rng(seed, 20, b, h)
    omega = rng.standard_normal((rank, 3)) / np.asarray(sigma)[None, :]
    beta = rng.uniform(0.0, 2.0 * math.pi, rank)
    phi = math.sqrt(2.0 / rank) * np.cos(pos @ omega.T + beta[None, :])
    w, _ = np.linalg.qr(rng.standard_normal((D, rank)))
    p = (math.sqrt(D) * (phi @ w.T)).astype(np.float32)
    eq = _normal(_rng(seed, 21, b, h), (S, D))
    ek = _normal(_rng(seed, 22, b, h), (S, D))
    inv = np.float32(1.0 / math.sqrt(2.0))
    return (to_bf16_bits((eq + p) * inv), to_bf16_bits((ek + p) * inv),
            to_bf16_bits(_normal(_rng(seed, 23, b, h), (S, D))))


def gen_video(seed, B, H, D, grid=(21, 30, 52), sigma=(2.0, 4.0, 4.0), rank=64, workers=None):
    """Video-DiT-like Q/K/V on a (frames, rows, cols) token grid; S = prod(grid).

    Heads are independent random streams, generated in parallel threads."""
    from concurrent.futures import ThreadPoolExecutor
    S = int(np.prod(grid))
    pos = video_positions(*grid)
    out = np.empty((3, B, H, S, D), np.uint16)

    def one(bh):
        b, h = bh
        out[0, b, h], out[1, b, h], out[2, b, h] = _video_head(seed, b, h, D, pos, sigma, rank)

    workers = workers or min(16, os.cpu_count() or 1)
    with ThreadPoolExecutor(workers) as ex:
        list(ex.map(one, [(b, h) for b in range(B) for h in range(H)]))
    qkv = np.ascontiguousarray(out.transpose(0, 1, 3, 2, 4))
    return qkv[0], qkv[1], qkv[2]


def gen_bitmask(seed, B, Hkv, n_q_blocks, n_kv_blocks, n_set, garbage_padding=False):
    """Packed uint32 exact-block bitmaps [B, Hkv, nQB, ceil(nKB/32)], LSB first.

    Each row has exactly ``min(n_set, nKB)`` set bits among the valid blocks, always including
    block 0 and the diagonal block (qb, when qb < nKB)."""
    W = -(-n_kv_blocks // 32)
    out = np.zeros((B, Hkv, n_q_blocks, W), np.uint32)
    rng = _rng(seed, 30)
    pad_bits = W * 32 - n_kv_blocks
    for b in range(B):
        for h in range(Hkv):
            for qb in range(n_q_blocks):
                forced = sorted({0, qb} & set(range(n_kv_blocks)))
                rest = np.setdiff1d(np.arange(n_kv_blocks), forced)
                extra = max(0, min(n_set, n_kv_blocks) - len(forced))
                chosen = list(forced) + list(rng.choice(rest, size=extra, replace=False))
                for j in chosen:
                    out[b, h, qb, j >> 5] |= np.uint32(1 << (j & 31))
                if garbage_padding and pad_bits:
                    junk = int(rng.integers(0, 1 << 32, dtype=np.uint64))
                    mask = ((1 << pad_bits) - 1) << (32 - pad_bits)
                    out[b, h, qb, W - 1] |= np.uint32(junk & mask)
    return out


def bitmask_to_bsr(bitmask, n_kv_blocks):
    """Canonical BSR of a packed bitmap: (indptr [rows+1] int32, indices [nnz] int32), rows in the
    bitmap's (b, kv head, q block) order, each row's valid set blocks in ascending order."""
    bm = np.ascontiguousarray(bitmask, dtype=np.uint32)
    by = bm.view(np.uint8).reshape(-1, bm.shape[-1] * 4)
    bits = np.unpackbits(by, axis=-1, bitorder="little")[:, :n_kv_blocks].astype(bool)
    counts = bits.sum(-1)
    indptr = np.zeros(bits.shape[0] + 1, np.int32)
    indptr[1:] = np.cumsum(counts)
    indices = np.nonzero(bits)[1].astype(np.int32)   # row-major: rows in order, columns ascending
    return indptr, indices


def scramble_bsr(seed, indptr, indices, n_kv_blocks, frac=0.5):
    """Non-canonical copy of a BSR: in about ``frac`` of the rows the entries are shuffled and
    receive a duplicate and an out-of-range entry.  Returns (indptr, indices, scrambled_rows)."""
    rng = _rng(seed, 31)
    rows = indptr.size - 1
    new_ptr = [0]
    new_idx = []
    scrambled = np.zeros(rows, bool)
    for r in range(rows):
        ent = list(indices[indptr[r]:indptr[r + 1]])
        if ent and rng.random() < frac:
            ent.append(ent[int(rng.integers(len(ent)))])
            ent.append(int(rng.choice([-1, n_kv_blocks, n_kv_blocks + 7])))
            ent = list(rng.permutation(ent))
            scrambled[r] = True
        new_idx += ent
        new_ptr.append(len(new_idx))
    return np.array(new_ptr, np.int32), np.array(new_idx, np.int32), scrambled


def block_summaries(k_bits, v_bits, block_k):
    """Per-KV-block mean of K and sum of V over the block's true tokens: bf16 [B,Hkv,nKB,D]."""
    kf = bf16_bits_to_f32(k_bits).astype(np.float64)
    vf = bf16_bits_to_f32(v_bits).astype(np.float64)
    B, Sk, Hkv, D = kf.shape
    nKB = -(-Sk // block_k)
    km = np.empty((B, Hkv, nKB, D))
    vs = np.empty((B, Hkv, nKB, D))
    for j in range(nKB):
        t0, t1 = j * block_k, min(Sk, (j + 1) * block_k)
        km[:, :, j] = kf[:, t0:t1].mean(axis=1)
        vs[:, :, j] = vf[:, t0:t1].sum(axis=1)
    return to_bf16_bits(km), to_bf16_bits(vs)


# ---------------------------------------------------------------------------------------------
# Workload descriptions (shapes, tiles, parameters and the generator each one uses)
# ---------------------------------------------------------------------------------------------
CALIB_A = 1443.49   # prefill coefficients of the calibrated threshold model (Wan 2.2 example)
CALIB_B = 4.30
# calibration.threshold_trials of the HuggingFace attention-sparsity page's custom configuration
THRESHOLD_TRIALS = [1e-4, 5e-4, 1e-3, 5e-3, 1e-2, 2e-2, 5e-2, 1e-1, 2e-1, 3e-1, 5e-1, 7e-1]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    path: str            # "skip", "nm", "proxy" or "decode"
    B: int
    Hq: int
    Hkv: int
    S: int
    D: int
    causal: bool
    block_q: int
    block_k: int
    gen: str             # "iid", "llm", "video"
    seed: int
    params: tuple = ()   # path-specific: see the definitions below

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    def param(self, key, default=None):
        return dict(self.params).get(key, default)

    def generate(self, S=None, Hq=None, Hkv=None, B=None):
        """Inputs for this workload, optionally at a reduced size (same generator and seed)."""
        S = S or self.S
        B = B or self.B
        Hq = Hq or self.Hq
        Hkv = Hkv or self.Hkv
        if self.gen == "iid":
            return gen_iid(self.seed, B, S, S, Hq, Hkv, self.D)
        if self.gen == "llm":
            return gen_llm(self.seed, B, S, Hq, Hkv, self.D)
        if self.gen == "llm_decode":
            return gen_llm_decode(self.seed, B, S, Hq, Hkv, self.D,
                                  ragged=self.param("ragged", True))
        if self.gen == "video":
            grid = self.param("grid")
            if S != self.S:
                raise ValueError("the video generator is defined on its full token grid")
            return gen_video(self.seed, B, Hq, self.D, grid=grid)
        raise ValueError(self.gen)


WORKLOADS = {
    "iid_s256_d64": Workload("iid_s256_d64", "skip", 1, 2, 2, 256, 64, False, 64, 64, "iid", 1,
                             (("lambda", 1e-3),)),
    "llm_prefill_gqa_s8192": Workload("llm_prefill_gqa_s8192", "skip", 1, 32, 8, 8192, 128, True,
                                      128, 64, "llm", 2, (("target_sparsity", 0.5),)),
    "llm_prefill_nm_s4096": Workload("llm_prefill_nm_s4096", "nm", 2, 32, 32, 4096, 128, True,
                                     128, 64, "llm", 3,
                                     (("n", 2), ("m", 4), ("sink", 4), ("recent", 128))),
    "video_dit_s32760": Workload("video_dit_s32760", "skip", 1, 40, 40, 32760, 128, False, 128, 64,
                                 "video", 4, (("target_sparsity", 0.5), ("grid", (21, 30, 52)))),
    "llm_decode_gqa_kv8192": Workload("llm_decode_gqa_kv8192", "decode", 16, 32, 8, 8192, 128,
                                      False, 1, 64, "llm_decode", 6,
                                      (("lambda", 1e-4), ("target_sparsity", 0.5),
                                       ("ragged", True))),
    "proxy_bitmask_s16257": Workload("proxy_bitmask_s16257", "proxy", 1, 24, 24, 16257, 128, False,
                                     128, 128, "iid", 5, (("density", 0.25),)),
    # the shape of the pages' proxy A/B: [1, 32760, 12, 128], 64-token blocks, 84 of 512 exact
    "proxy_page_s32760": Workload("proxy_page_s32760", "proxy", 1, 12, 12, 32760, 128, False,
                                  64, 64, "iid", 5, (("density", 84 / 512),)),
}
