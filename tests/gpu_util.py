"""Helpers for the GPU parity tests: device setup, error metrics, and the
conversions between torch device tensors and the oracle's numpy arrays."""

from __future__ import annotations

import sys

import numpy as np
import torch

# Tolerances for bf16 inputs with fp32 state and accumulation.
REL_L2_TOL = 2e-3
MAX_ABS_TOL = 1e-2


def device():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU test run without a visible GPU")
    return torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel_l2(x, ref) -> float:
    x = np.asarray(x, np.float64).ravel()
    ref = np.asarray(ref, np.float64).ravel()
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / (den if den > 0 else 1.0))


def max_abs(x, ref) -> float:
    x = np.asarray(x, np.float64).ravel()
    ref = np.asarray(ref, np.float64).ravel()
    return float(np.max(np.abs(x - ref))) if x.size else 0.0


def to_np(t) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def assert_close(name, got, ref, rel=REL_L2_TOL, mx=MAX_ABS_TOL):
    r = rel_l2(got, ref)
    m = max_abs(got, ref)
    say(f"  {name}: rel_l2={r:.3e} max_abs={m:.3e}")
    assert np.all(np.isfinite(np.asarray(got, np.float64))), f"{name}: non-finite values"
    assert r <= rel, f"{name}: rel_l2 {r:.3e} > {rel:.1e}"
    assert m <= mx, f"{name}: max_abs {m:.3e} > {mx:.1e}"
    return r, m


def within_bf16_of(got_bf16_as_f64, exact, extra_rel=2e-6, extra_abs=1e-6):
    """Each value equals the exact result up to one bf16 rounding (half a
    unit in the last place is at most 2^-8 |x|), plus a little for the fp32
    accumulation that precedes the rounding."""
    got = np.asarray(got_bf16_as_f64, np.float64)
    x = np.asarray(exact, np.float64)
    bound = np.abs(x) * (2.0 ** -8 + extra_rel) + extra_abs
    return bool(np.all(np.abs(got - x) <= bound))
