"""Helpers of the GPU parity tests: run the HIP path through the C ABI and
compare with the oracle.  Tolerances are the ones the workloads state:
bf16 inputs with fp32 accumulation: rel-L2 <= 5e-3 and max-abs <= 2e-2;
fp8 latent cache: rel-L2 <= 3e-2 (against the oracle on the dequantised
cache).  The fp32 tiny workload (no tolerance stated) is gated on the same
bf16 bounds and, as an internal target, on rel-L2 <= 1e-5."""
from __future__ import annotations

import sys

import numpy as np

REL_L2_BF16 = 5e-3
MAX_ABS_BF16 = 2e-2
REL_L2_FP8 = 3e-2
REL_L2_FP32_TARGET = 1e-5
LSE_ABS = 2e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_np(t) -> np.ndarray:
    import torch
    t = t.detach()
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.cpu().numpy().astype(np.float64)


def rel_l2(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))


def check(name, got, ref, rel, max_abs=None, mask=None):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if mask is not None:
        got, ref = got[mask], ref[mask]
    assert got.shape == ref.shape
    assert np.all(np.isfinite(got)), f"{name}: non-finite GPU output"
    r = rel_l2(got, ref)
    m = float(np.max(np.abs(got - ref))) if got.size else 0.0
    say(f"  {name}: rel-L2 {r:.3e} (gate {rel:.0e}), max-abs {m:.3e}"
        + (f" (gate {max_abs:.0e})" if max_abs is not None else ""))
    assert r <= rel, f"{name}: rel-L2 {r} > {rel}"
    if max_abs is not None:
        assert m <= max_abs, f"{name}: max-abs {m} > {max_abs}"
    return r, m


def sample_mask(shape_tok_head, seqs, heads, T):
    """Boolean [B*T, n_h] mask of the sampled (sequence, head) rows."""
    mask = np.zeros(shape_tok_head, dtype=bool)
    for b in seqs:
        for tau in range(T):
            mask[b * T + tau, list(heads)] = True
    return mask
