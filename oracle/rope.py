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

Context extension (YaRN, Peng et al. 2023), which DeepSeek-V2 applies to the
decoupled key and query parts only ("DeepSeek-V2", section 3, long context
extension: scale s = 40, alpha = 1, beta = 32, a 160K target from a 4K
training context; the long context extension part of the "DeepSeek-V3
Technical Report" notes repeats the settings).  The pages name the method and its parameters but not its
formulas; the oracle takes YaRN's published "NTK-by-parts" rule: pair k
with wavelength lambda_k = 2 pi / theta_k completes r_k = L / lambda_k turns
over the original context L, and
    gamma_k  = clamp((r_k - alpha) / (beta - alpha), 0, 1)
    theta'_k = (1 - gamma_k) theta_k / s + gamma_k theta_k,
so pairs that turn more than beta times keep their frequency and pairs that
turn less than alpha times are interpolated by s.  The attention temperature
is given on the pages as sqrt(t) = c ln s + 1 with c = 0.0707 (DeepSeek-V2)
or c = 0.1 (the DeepSeek-V3 notes); the oracle reads it as a factor t =
(c ln s + 1)^2 on every attention logit.
"""
from __future__ import annotations

import numpy as np


def rope_theta(d: int, base: float = 10000.0) -> np.ndarray:
    """theta_k = base^(-2k/d), k = 0 .. d/2-1 (float64)."""
    if d % 2:
        raise ValueError("RoPE needs an even dimension")
    k = np.arange(d // 2, dtype=np.float64)
    return base ** (-2.0 * k / d)


def yarn_theta(d: int, base: float, factor: float, alpha: float, beta: float,
               orig_len: float) -> np.ndarray:
    """Per-pair frequencies after YaRN's NTK-by-parts rule (see the module
    docstring); factor <= 1 leaves them unchanged."""
    theta = rope_theta(d, base)
    if factor <= 1.0:
        return theta
    if not (0.0 < alpha < beta):
        raise ValueError("YaRN needs 0 < alpha < beta")
    turns = orig_len * theta / (2.0 * np.pi)          # r_k = L / lambda_k
    gamma = np.clip((turns - alpha) / (beta - alpha), 0.0, 1.0)
    return (1.0 - gamma) * theta / factor + gamma * theta


def yarn_logit_factor(factor: float, coef: float) -> float:
    """t = (coef ln s + 1)^2, the factor on every attention logit (1 for s <= 1)."""
    if factor <= 1.0:
        return 1.0
    m = coef * np.log(factor) + 1.0
    return float(m * m)


def rope(x: np.ndarray, pos: np.ndarray, base: float = 10000.0,
         theta: np.ndarray = None) -> np.ndarray:
    """Rotate the last axis of ``x`` (float64 [..., d]) at positions ``pos``
    by the frequencies ``theta`` (default: rope_theta(d, base)).

    ``pos`` broadcasts against x's leading axes (one position per vector).
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    if theta is None:
        theta = rope_theta(d, base)
    theta = np.asarray(theta, dtype=np.float64)
    if theta.shape != (d // 2,):
        raise ValueError("one frequency per pair")
    ang = np.asarray(pos, dtype=np.float64)[..., None] * theta
    c, s = np.cos(ang), np.sin(ang)
    xe, xo = x[..., 0::2], x[..., 1::2]
    y = np.empty_like(x)
    y[..., 0::2] = xe * c - xo * s
    y[..., 1::2] = xe * s + xo * c
    return y
