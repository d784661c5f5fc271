"""Rotary position embedding (oracle; test infrastructure).

The pages use RoPE (Su et al.) on the decoupled query q^R and the shared key
k^R ("DeepSeek-V2: Strong, Economical, Efficient", section 2.1.3) but do not
define it.  This oracle takes the RoFormer form with interleaved pairs:
for k = 0 .. d/2-1, theta_k = base^(-2k/d), and the pair (x_{2k}, x_{2k+1}) at
integer position p is rotated by the angle p * theta_k:
    y_{2k}   = x_{2k} cos(p theta_k) - x_{2k+1} sin(p theta_k)
    y_{2k+1} = x_{2k} sin(p theta_k) + x_{2k+1} cos(p theta_k)
The pairing (interleaved rather than half-split) is a convention: parity
unpinned.  Its properties (R_0 = I, <R_m x, R_n y> depends only on m - n) are
pinned in the tests.
"""
from __future__ import annotations

import numpy as np


def rope(x: np.ndarray, pos: np.ndarray, base: float = 10000.0) -> np.ndarray:
    """Rotate the last axis of ``x`` (float64 [..., d]) at positions ``pos``.

    ``pos`` broadcasts against x's leading axes (one position per vector).
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    if d % 2:
        raise ValueError("RoPE needs an even dimension")
    k = np.arange(d // 2, dtype=np.float64)
    theta = base ** (-2.0 * k / d)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * theta
    c, s = np.cos(ang), np.sin(ang)
    xe, xo = x[..., 0::2], x[..., 1::2]
    y = np.empty_like(x)
    y[..., 0::2] = xe * c - xo * s
    y[..., 1::2] = xe * s + xo * c
    return y
