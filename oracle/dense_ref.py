"""Textbook dense RoPE softmax attention in NumPy fp64 (test infrastructure).

This is ordinary rotary attention with no windows at all: rotate q and k with
the half-split ("rotate_half") rotary embedding, form Q'K'^T / sqrt(d), mask
the keys after the query (causal), softmax, multiply by V.  It shares nothing
with the C oracle and is used only to pin the oracle's special cases: with the
windows switched off (alpha = inf), or made irrelevant (short sequences, or
inputs living only on the never-cut slowest pair), the windowed method must
reduce to exactly this.  The online softmax is unchanged by the method (source
page "ATFlash: RoPE-Frequenzen kuerzen Attention-Arbeit um bis zu 57 Prozent",
section "Die Zahlen - und ihre Grenze"), so a plain softmax is the right
textbook counterpart.
"""
from __future__ import annotations

import numpy as np


def rope_half_split(x: np.ndarray, positions: np.ndarray, base: float) -> np.ndarray:
    """Rotate [..., S, d] rows by angle position * base^(-2p/d) per pair (p, p+d/2)."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    half = d // 2
    inv_freq = base ** (-np.arange(half, dtype=np.float64) * 2.0 / d)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * inv_freq[None, :]
    cos = np.concatenate([np.cos(ang), np.cos(ang)], axis=-1)
    sin = np.concatenate([np.sin(ang), np.sin(ang)], axis=-1)
    rot_half = np.concatenate([-x[..., half:], x[..., :half]], axis=-1)
    return x * cos + rot_half * sin


def rope_interleaved(x: np.ndarray, positions: np.ndarray, base: float) -> np.ndarray:
    """GPT-J rotary: dims (2p, 2p+1) read as the complex number x_2p + i x_2p+1,
    multiplied by exp(i * position * base^(-2p/d)), written back interleaved."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    z = x[..., 0::2] + 1j * x[..., 1::2]
    inv_freq = base ** (-np.arange(d // 2, dtype=np.float64) * 2.0 / d)
    z = z * np.exp(1j * np.asarray(positions, dtype=np.float64)[:, None] * inv_freq[None, :])
    out = np.empty_like(x)
    out[..., 0::2] = z.real
    out[..., 1::2] = z.imag
    return out


def dense_rope_attention(q, k, v, *, base: float, causal: bool = True,
                         q_pos0: int = 0, k_pos0: int = 0, layout: str = "neox") -> np.ndarray:
    """q [B,Hq,Sq,d], k/v [B,Hkv,Sk,d] -> out [B,Hq,Sq,d] in fp64.
    layout "neox": rotate_half rotary; "gptj": interleaved (complex) rotary."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, Sq, d = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    group = Hq // Hkv
    qpos = q_pos0 + np.arange(Sq)
    kpos = k_pos0 + np.arange(Sk)
    rope = rope_interleaved if layout == "gptj" else rope_half_split
    qr = rope(q, qpos, base)
    kr = rope(k, kpos, base)
    kr = np.repeat(kr, group, axis=1)
    vv = np.repeat(v, group, axis=1)
    logits = qr @ np.swapaxes(kr, -1, -2) / np.sqrt(d)
    if causal:
        allowed = (qpos[:, None] - kpos[None, :]) >= 0
        logits = np.where(allowed, logits, -np.inf)
    logits = logits - logits.max(axis=-1, keepdims=True)
    w = np.exp(logits)
    w = w / w.sum(axis=-1, keepdims=True)
    return w @ vv
