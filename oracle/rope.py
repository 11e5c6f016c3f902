"""Rotary position embedding (RoPE): the oracle for the fused append with RoPE.

TEST INFRASTRUCTURE ONLY (see the package docstring): not for the product path.

The pages enable one position-encoding mode in the FlashInfer build
(BlitzScale documentation, "Build": the generated kernels are compiled with
POS_ENCODING_MODES=1) without saying what it is, and configure Llama-family
and other decoder models (BlitzScale documentation, the router's model
configuration).  The reading taken here is the rotary position embedding of
Su et al. (RoFormer, 2021): the head dims form d/2 pairs, pair j is rotated
in its plane by the angle pos * theta_j with theta_j = base^(-2j/d):

    (a, b) of pair j  ->  (a cos phi - b sin phi,  a sin phi + b cos phi),
    phi = pos * theta_j

with two pairings: "half" takes dims (j, j + d/2) (the layout of the
Hugging Face checkpoints the configuration names), "interleaved" takes dims
(2j, 2j + 1) (the paper's).  Everything is evaluated in fp64 on the exact
input values.
"""
from __future__ import annotations

import numpy as np

HALF = 0
INTERLEAVED = 1


def pair_dims(d: int, style: int):
    """Dims (a_j, b_j) of the d/2 rotation pairs."""
    j = np.arange(d // 2)
    if style == HALF:
        return j, j + d // 2
    if style == INTERLEAVED:
        return 2 * j, 2 * j + 1
    raise ValueError("style must be HALF or INTERLEAVED")


def frequencies(d: int, base: float) -> np.ndarray:
    """theta_j = base^(-2j/d), j = 0 .. d/2 - 1, fp64."""
    j = np.arange(d // 2, dtype=np.float64)
    return np.float64(base) ** (-2.0 * j / d)


def rope(x: np.ndarray, positions: np.ndarray, base: float, style: int) -> np.ndarray:
    """Rotate ``x [T][H][d]``; row t by ``positions[t]``.  Returns fp64."""
    x = np.asarray(x, np.float64)
    d = x.shape[-1]
    a, b = pair_dims(d, style)
    phi = np.asarray(positions, np.float64)[:, None] * frequencies(d, base)[None, :]  # [T][d/2]
    c = np.cos(phi)[:, None, :]
    s = np.sin(phi)[:, None, :]
    y = np.empty_like(x)
    y[..., a] = x[..., a] * c - x[..., b] * s
    y[..., b] = x[..., a] * s + x[..., b] * c
    return y
