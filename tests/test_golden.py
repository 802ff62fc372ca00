"""The oracle still reproduces its stored outputs on the tiny workload."""

import json
from pathlib import Path

import numpy as np

from hybrid_recurrent_serving_amd.inputs import make_workload

GOLD = Path(__file__).resolve().parent / "golden" / "tiny_kda_oracle.json"


def test_oracle_matches_stored_tiny_outputs(oracle64):
    ref = json.loads(GOLD.read_text())
    wl = make_workload(0, with_conv=True)
    res = oracle64.kda_varlen(wl.q, wl.k, wl.v, wl.g, wl.beta, wl.cu_seqlens,
                              ckpt_interval=ref["ckpt_interval"])
    np.testing.assert_allclose(res["o"].ravel(), ref["o"], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(res["final"].ravel(), ref["final"], rtol=1e-12, atol=1e-13)
    assert list(res["ckpt_pos"]) == ref["ckpt_pos"]
    # checkpoint contents equal the final states of shorter runs (pinned elsewhere)
    y, ns = oracle64.conv_short(wl.conv_x, wl.conv_w, wl.cu_seqlens)
    np.testing.assert_allclose(y[:4].ravel(), ref["conv_y_first_rows"], rtol=1e-12, atol=1e-13)
    np.testing.assert_array_equal(ns.ravel(), ref["conv_new_state"])
