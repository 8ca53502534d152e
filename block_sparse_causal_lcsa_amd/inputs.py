"""Seeded synthetic Q/K/V for LCSA workloads (inputs only; none of the method's arithmetic).

The pages measure on real video through a trained DiT (REDS, 101-frame 768x1408 clips, 15 clips
at 1536x2688); none of that is available, so these fields stand in for it at the same shapes.
Q and K are spatially and temporally smooth sinusoids with seeded per-channel frequencies and
phases, shared by Q and K so that nearby blocks correlate (the locality that LCSA's selection
exploits), plus 0.5*N(0,1) noise; V is N(0,1).

    rng([seed, 0]):  w_t, w_h, w_w ~ U(0, pi/8)  per (head, channel);  phi ~ U(0, 2 pi)
    field(t, h, w)   = sin(w_t t + w_h h + w_w w + phi),   t = absolute latent frame index
    Q = field(query frames) + 0.5 N(0,1)  (rng([seed, 1]))
    K = field(kv frames)    + 0.5 N(0,1)  (rng([seed, 2]))
    V = N(0,1)                            (rng([seed, 3]))

bf16 workloads round the fp32 values to bf16 (round to nearest even) and hand out the raw
16-bit patterns; `to_f64` widens either form exactly. Layout is [B, heads, tokens, head_dim],
tokens in raster order (t, h, w).
"""
from __future__ import annotations

import numpy as np


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest, ties to even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> 16) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> 16).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def to_f64(x: np.ndarray) -> np.ndarray:
    """Exact fp64 copy of an input array (bf16 bit patterns or fp32/fp64 values)."""
    if x.dtype == np.uint16:
        return bf16_to_f32(x).astype(np.float64)
    return x.astype(np.float64)


def _field(w, frames0: int, nframes: int, rng_param_draws, b_noise: np.ndarray) -> np.ndarray:
    wt, wh, ww, phi = rng_param_draws
    H, W = w.grid_h, w.grid_w
    t = np.arange(frames0, frames0 + nframes, dtype=np.float32)
    hh = np.arange(H, dtype=np.float32)
    xx = np.arange(W, dtype=np.float32)
    tt, yy, xw = np.meshgrid(t, hh, xx, indexing="ij")
    tt, yy, xw = tt.reshape(-1, 1), yy.reshape(-1, 1), xw.reshape(-1, 1)
    out = b_noise  # [B, heads, N, d] fp32, noise already scaled; field added in place per head
    for h in range(w.heads):
        arg = tt * wt[h][None, :] + yy * wh[h][None, :] + xw * ww[h][None, :] + phi[h][None, :]
        f = np.sin(arg, dtype=np.float32)
        out[:, h] += f[None]
    return out


def make_inputs(w, seed: int = 0, want=("q", "k", "v")) -> dict:
    """Q/K/V for workload `w` (any object with the Workload attributes).

    Returns {"q","k","v"}: np.uint16 bf16 bit patterns for dtype "bf16", np.float32 for "f32".
    """
    d, Hh, B = w.head_dim, w.heads, w.batch
    p = np.random.default_rng([seed, 0])
    wt = p.uniform(0.0, np.pi / 8, size=(Hh, d)).astype(np.float32)
    wh = p.uniform(0.0, np.pi / 8, size=(Hh, d)).astype(np.float32)
    ww = p.uniform(0.0, np.pi / 8, size=(Hh, d)).astype(np.float32)
    phi = p.uniform(0.0, 2 * np.pi, size=(Hh, d)).astype(np.float32)
    params = (wt, wh, ww, phi)
    hw = w.grid_h * w.grid_w
    out = {}
    if "q" in want:
        n = np.random.default_rng([seed, 1]).standard_normal((B, Hh, w.q_frames * hw, d), dtype=np.float32)
        n *= np.float32(0.5)
        out["q"] = _field(w, w.q_frame0, w.q_frames, params, n)
    if "k" in want:
        n = np.random.default_rng([seed, 2]).standard_normal((B, Hh, w.kv_frames * hw, d), dtype=np.float32)
        n *= np.float32(0.5)
        out["k"] = _field(w, 0, w.kv_frames, params, n)
    if "v" in want:
        out["v"] = np.random.default_rng([seed, 3]).standard_normal((B, Hh, w.kv_frames * hw, d),
                                                                    dtype=np.float32)
    if w.dtype == "bf16":
        out = {k: bf16_bits(v) for k, v in out.items()}
    return out


def make_grad(w, seed: int = 0) -> np.ndarray:
    """Upstream gradient dL/dO for the backward: N(0,1) from rng([seed, 4]), [B, heads, Nq, d], as bf16
    bit patterns (the workload's dtype is bf16 for every backward case)."""
    g = np.random.default_rng([seed, 4]).standard_normal(
        (w.batch, w.heads, w.q_frames * w.grid_h * w.grid_w, w.head_dim), dtype=np.float32)
    return bf16_bits(g)
