"""The CPU oracle against closed forms, invariants, special cases and brute
force (see ``oracle_pins.py``), in both of its precisions."""

import numpy as np
import pytest

import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin_f64(pin, oracle64):
    pin(oracle64)


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin_f32(pin, oracle32):
    pin(oracle32)


def test_f32_matches_f64_on_tiny_workload(oracle64, oracle32):
    from hybrid_recurrent_serving_amd.inputs import make_workload
    wl = make_workload(0)
    a = oracle64.kda_varlen(wl.q, wl.k, wl.v, wl.g, wl.beta, wl.cu_seqlens)
    b = oracle32.kda_varlen(wl.q, wl.k, wl.v, wl.g, wl.beta, wl.cu_seqlens)
    rel = np.linalg.norm(a["o"] - b["o"]) / np.linalg.norm(a["o"])
    assert rel < 1e-5


def test_threads_do_not_change_results(oracle64):
    from hybrid_recurrent_serving_amd.inputs import make_workload
    wl = make_workload(2, lengths=[70, 33, 129], H=3, d=8)
    init = wl.init_states
    has = [1 if i >= 0 else 0 for i in wl.init_index]
    full_init = np.zeros((3, 3, 8, 8))
    for s, i in enumerate(wl.init_index):
        if i >= 0:
            full_init[s] = init[i].numpy()
    oracle64.set_threads(1)
    a = oracle64.kda_varlen(wl.q, wl.k, wl.v, wl.g, wl.beta, wl.cu_seqlens, init=full_init,
                            has_init=has)
    oracle64.set_threads(8)
    b = oracle64.kda_varlen(wl.q, wl.k, wl.v, wl.g, wl.beta, wl.cu_seqlens, init=full_init,
                            has_init=has)
    assert np.array_equal(a["o"], b["o"]) and np.array_equal(a["final"], b["final"])
