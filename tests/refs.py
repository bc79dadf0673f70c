"""Independent textbook references used to pin the oracle (CPU, float64).

These call library routines (torch's scaled-dot-product attention on the CPU in float64, numpy
sorting and bit unpacking) that share nothing with the oracle's C code.
"""
from __future__ import annotations

import numpy as np
import torch

from workloads import bf16_bits_to_f32


def f64(bits):
    return bf16_bits_to_f32(bits).astype(np.float64)


def scores(q_bits, k_bits):
    """Raw scores q.k for every (b, hq, r, key), float64 [B, Hq, Sq, Sk] (GQA expanded)."""
    q, k = f64(q_bits), f64(k_bits)
    G = q.shape[2] // k.shape[2]
    k = np.repeat(k, G, axis=2)
    return np.einsum("bqhd,bkhd->bhqk", q, k)


def sdpa(q_bits, k_bits, v_bits, scale, mask=None, causal=False):
    """softmax(scale * q.k + mask) v in float64 with torch SDPA; mask is boolean [B,Hq,Sq,Sk].

    Returns o [B,Sq,Hq,D]."""
    q = torch.from_numpy(f64(q_bits)).permute(0, 2, 1, 3)
    k = torch.from_numpy(f64(k_bits)).permute(0, 2, 1, 3)
    v = torch.from_numpy(f64(v_bits)).permute(0, 2, 1, 3)
    G = q.shape[1] // k.shape[1]
    k = k.repeat_interleave(G, dim=1)
    v = v.repeat_interleave(G, dim=1)
    m = None
    if mask is not None:
        m = torch.from_numpy(np.ascontiguousarray(mask))
    if causal:
        Sq, Sk = q.shape[2], k.shape[2]
        cm = torch.ones(Sq, Sk, dtype=torch.bool).tril()
        m = cm if m is None else (m & cm)
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=m, scale=scale)
    return o.permute(0, 2, 1, 3).numpy()


def lse(q_bits, k_bits, scale, mask):
    s = scale * scores(q_bits, k_bits)
    s = np.where(mask, s, -np.inf)
    mx = s.max(axis=-1, keepdims=True)
    return (mx[..., 0] + np.log(np.exp(s - mx).sum(axis=-1)))


def tile_key_mask(tile_state, Sq, Sk, Br, Bc, causal):
    """Boolean [B,Hq,Sq,Sk]: key allowed for the row and its tile kept (state 0)."""
    B, Hq, nQT, nKT = tile_state.shape
    kept = (tile_state == 0)
    rows = np.arange(Sq) // Br
    cols = np.arange(Sk) // Bc
    m = kept[:, :, rows][:, :, :, cols]
    if causal:
        m = m & np.tril(np.ones((Sq, Sk), bool))[None, None]
    return m
