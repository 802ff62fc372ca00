"""Write the stored expected values under tests/golden/.

The pages print no worked example of the KDA recurrence, so no fixture here
comes from them.  This script calls only the CPU oracle (``oracle/``) on the
tiny seeded workload (T=64, H=2, d=16, fp32, zero initial state, seed 0) and
stores its outputs as a regression anchor: a later change to the oracle's
arithmetic shows up as a mismatch against this file.

Run from the repository root:  python tests/golden/make_golden.py
"""

import json
import sys
from pathlib import Path

ROOT = Path(__file__).resolve().parents[2]
sys.path.insert(0, str(ROOT))

import oracle  # noqa: E402
from hybrid_recurrent_serving_amd.inputs import make_workload  # noqa: E402


def main():
    orc = oracle.load("f64")
    wl = make_workload(0, with_conv=True)
    res = orc.kda_varlen(wl.q, wl.k, wl.v, wl.g, wl.beta, wl.cu_seqlens, ckpt_interval=16)
    y, ns = orc.conv_short(wl.conv_x, wl.conv_w, wl.cu_seqlens)
    out = {
        "workload": "tiny: B=1, T=64, H=2, d=16, fp32, zero initial state, seed 0",
        "producer": "tests/golden/make_golden.py (oracle/kda_oracle.c, fp64)",
        "o": [float(x) for x in res["o"].ravel()],
        "o_shape": list(res["o"].shape),
        "final": [float(x) for x in res["final"].ravel()],
        "final_shape": list(res["final"].shape),
        "ckpt_interval": 16,
        "ckpt_pos": [int(p) for p in res["ckpt_pos"]],
        "conv_y_first_rows": [float(x) for x in y[:4].ravel()],
        "conv_new_state": [float(x) for x in ns.ravel()],
    }
    path = Path(__file__).resolve().parent / "tiny_kda_oracle.json"
    path.write_text(json.dumps(out, separators=(",", ":")))
    print("wrote", path)


if __name__ == "__main__":
    main()
