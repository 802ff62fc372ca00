"""Every planted mistake in the oracle is caught by at least one pin.

The oracle source carries six deliberate mistakes behind a compile-time
switch (decay dropped, decay on the value axis, transposed prediction,
wrong sign of the correction, taps reversed, output read before the update).
Each variant is built here, on the CPU, and run through the pins."""

import pytest

import oracle
import oracle_pins as P

MUTANTS = {1: "decay dropped", 2: "decay on value axis", 3: "S k instead of S^T k",
           4: "sign of correction", 5: "conv taps reversed", 6: "output before update"}


@pytest.mark.parametrize("m", sorted(MUTANTS), ids=lambda m: MUTANTS[m])
def test_mutant_is_caught(m, tmp_path):
    orc = oracle.load_mutant(m, tmp_path)
    assert orc.mutant == m
    failed = []
    for pin in P.ALL_PINS:
        try:
            pin(orc)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"planted mistake {m} ({MUTANTS[m]}) passed every pin"


def _planted_gate_norms():
    """Plausible mistakes in the output gate's norm (each a function with the
    signature of oracle.gated_rmsnorm)."""
    import numpy as np

    def sig(z):
        return 1.0 / (1.0 + np.exp(-np.asarray(z, np.float64)))

    def sum_not_mean(o, z, w, eps=1e-6):
        o = np.asarray(o, np.float64)
        return o / np.sqrt(np.sum(o * o, -1, keepdims=True) + eps) * np.asarray(w, np.float64) * sig(z)

    def all_heads(o, z, w, eps=1e-6):
        o = np.asarray(o, np.float64)
        ms = np.mean(o * o, axis=(-2, -1), keepdims=True)
        return o / np.sqrt(ms + eps) * np.asarray(w, np.float64) * sig(z)

    def no_root(o, z, w, eps=1e-6):
        o = np.asarray(o, np.float64)
        return o / (np.mean(o * o, -1, keepdims=True) + eps) * np.asarray(w, np.float64) * sig(z)

    def silu_gate(o, z, w, eps=1e-6):
        o = np.asarray(o, np.float64)
        z = np.asarray(z, np.float64)
        return o / np.sqrt(np.mean(o * o, -1, keepdims=True) + eps) * np.asarray(w, np.float64) * z * sig(z)

    return [sum_not_mean, all_heads, no_root, silu_gate]


@pytest.mark.parametrize("planted", _planted_gate_norms(), ids=lambda f: f.__name__)
def test_output_gate_pin_catches_planted_mistake(planted, oracle64, monkeypatch):
    """Each planted mistake in the output gate's norm fails pin_output_gate."""
    import oracle
    import oracle_pins as P
    monkeypatch.setattr(oracle, "gated_rmsnorm", planted)
    with pytest.raises(AssertionError):
        P.pin_output_gate(oracle64)


def _planted_conv_operands():
    """Plausible mistakes in forming the prefill's q, k, v from the conv
    output (each a function with the signature of oracle.conv_operands)."""
    import numpy as np

    real = oracle.conv_operands

    def swap_qk(y, H, d, qk_l2norm, norm_eps, operand_dtype):
        q, k, v = real(y, H, d, qk_l2norm, norm_eps, operand_dtype)
        return k, q, v

    def blocks_reversed(y, H, d, qk_l2norm, norm_eps, operand_dtype):
        T = y.shape[0]
        yr = np.asarray(y).reshape(T, 3, H * d)[:, ::-1].reshape(T, -1)
        return real(yr, H, d, qk_l2norm, norm_eps, operand_dtype)

    def v_normalised(y, H, d, qk_l2norm, norm_eps, operand_dtype):
        q, k, v = real(y, H, d, qk_l2norm, norm_eps, operand_dtype)
        if qk_l2norm:
            v = (v / np.sqrt((v.astype(np.float64) ** 2).sum(-1, keepdims=True) + norm_eps)).astype(np.float32)
        return q, k, v

    def norm_over_heads(y, H, d, qk_l2norm, norm_eps, operand_dtype):
        q, k, v = real(y, H, d, 0, norm_eps, operand_dtype)
        if qk_l2norm:
            T = q.shape[0]
            q = (q / np.sqrt((q.astype(np.float64) ** 2).reshape(T, -1).sum(-1)[:, None, None] + norm_eps))
            k = (k / np.sqrt((k.astype(np.float64) ** 2).reshape(T, -1).sum(-1)[:, None, None] + norm_eps))
        return q.astype(np.float32), k.astype(np.float32), v

    def no_rounding(y, H, d, qk_l2norm, norm_eps, operand_dtype):
        return real(y, H, d, qk_l2norm, norm_eps, "f32")

    return [swap_qk, blocks_reversed, v_normalised, norm_over_heads, no_rounding]


@pytest.mark.parametrize("planted", _planted_conv_operands(), ids=lambda f: f.__name__)
def test_prefill_conv_pin_catches_planted_mistake(planted, oracle64, monkeypatch):
    """Each planted mistake in the prefill's operand forming fails
    pin_prefill_conv."""
    monkeypatch.setattr(oracle, "conv_operands", planted)
    with pytest.raises(AssertionError):
        P.pin_prefill_conv(oracle64)
