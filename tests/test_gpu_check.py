"""The KDA_CHECK=1 validation path of libkda: device index arrays and the
prefill's decay range are copied to the host and checked before launch.

The library reads KDA_CHECK once per process, so the checks run in a child
process with the variable set; each case prints one line, and the child
ends with a marker the test looks for."""

from __future__ import annotations

import os
import subprocess
import sys
from pathlib import Path

import numpy as np
import pytest
import torch

import gpu_util as U
from hybrid_recurrent_serving_amd import kda as K
from hybrid_recurrent_serving_amd.inputs import make_workload

pytestmark = pytest.mark.gpu

ROOT = Path(__file__).resolve().parents[1]

CHILD = r'''
import sys
sys.path.insert(0, sys.argv[1])
import torch
from hybrid_recurrent_serving_amd import kda as K
from hybrid_recurrent_serving_amd.inputs import make_workload

dev = torch.device("cuda:0")
K.load_library()


def expect(name, fn, status):
    try:
        fn()
    except K.KDAError as e:
        got = e.status
        assert got == status, (name, got, str(e))
        print(f"{name}: rejected ({e})", flush=True)
        return
    assert status == 0, (name, "accepted")
    print(f"{name}: accepted", flush=True)


# decode: slots
wl = make_workload(1, n_seq=4, H=2, d=32)
q, k, v, g, b = (t.to(dev) for t in (wl.q, wl.k, wl.v, wl.g, wl.beta))
pool = torch.zeros(8, 2, 32, 32, device=dev)
o = torch.empty(4, 2, 32, device=dev)
i32 = lambda x: torch.tensor(x, dtype=torch.int32, device=dev)
expect("decode valid", lambda: K.kda_decode(q, k, v, g, b, o, pool, i32([0, 1, 2, 3]), i32([4, 5, 6, 7])), 0)
expect("decode src of one = dst of another",
       lambda: K.kda_decode(q, k, v, g, b, o, pool, i32([0, 1, 2, 3]), i32([1, 5, 6, 7])), 8)
expect("decode slot out of range",
       lambda: K.kda_decode(q, k, v, g, b, o, pool, i32([0, 1, 2, 30]), i32([4, 5, 6, 7])), 8)

# prefill: cu_seqlens, checkpoint slots, decay range
wl = make_workload(2, lengths=[100, 60, 90], H=2, d=64)
q, k, v, g, b = (t.to(dev) for t in (wl.q, wl.k, wl.v, wl.g, wl.beta))
T = q.shape[0]
pool = torch.zeros(10, 2, 64, 64, device=dev)
o = torch.empty(T, 2, 64, dtype=torch.bfloat16, device=dev)
src, dst = i32([0, 1, 2]), i32([3, 4, 5])
cu = wl.cu_seqlens.to(dev)
expect("prefill valid", lambda: K.kda_prefill_varlen(q, k, v, g, b, o, cu, pool, src, dst, chunk=32), 0)
expect("prefill cu_seqlens decreasing",
       lambda: K.kda_prefill_varlen(q, k, v, g, b, o, i32([0, 100, 90, T]), pool, src, dst, chunk=32), 8)
expect("prefill cu_seqlens past T_tot",
       lambda: K.kda_prefill_varlen(q, k, v, g, b, o, i32([0, 100, 160, T + 1]), pool, src, dst, chunk=32), 8)
ck_cu = i32([0, 1, 1, 2])   # checkpoints at 64 in sequences 0 and 2
expect("prefill checkpoint slot = a source slot",
       lambda: K.kda_prefill_varlen(q, k, v, g, b, o, cu, pool, src, dst, chunk=32, ckpt_interval=64,
                                    ckpt_cu=ck_cu, ckpt_slot=i32([6, 1])), 8)
expect("prefill checkpoint slot free",
       lambda: K.kda_prefill_varlen(q, k, v, g, b, o, cu, pool, src, dst, chunk=32, ckpt_interval=64,
                                    ckpt_cu=ck_cu, ckpt_slot=i32([6, 7])), 0)
# decay range: -4.5 per token over 16 tokens (72 nats) is accepted, -6 (96 nats) rejected
g_ok = torch.full_like(g, -4.5)
expect("prefill g = -4.5 sustained", lambda: K.kda_prefill_varlen(q, k, v, g_ok, b, o, cu, pool, src, dst, chunk=32), 0)
g_bad = g.clone()
g_bad[100:160, 1, 7] = -6.0
expect("prefill g = -6 sustained over a sequence",
       lambda: K.kda_prefill_varlen(q, k, v, g_bad, b, o, cu, pool, src, dst, chunk=32), 8)
torch.cuda.synchronize()
print("__KDA_CHECK_OK__", flush=True)
'''


def test_kda_check_validation():
    """Under KDA_CHECK=1: aliasing and out-of-range slots, malformed
    cu_seqlens, checkpoint slots that alias a source, and a decay beyond the
    documented range are rejected with KDA_ERR_ARG; valid calls pass."""
    U.say("KDA_CHECK=1 validation (child process)")
    env = dict(os.environ)
    env["KDA_CHECK"] = "1"
    res = subprocess.run([sys.executable, "-c", CHILD, str(ROOT)], env=env, capture_output=True,
                         text=True, timeout=300)
    U.say(res.stdout)
    assert res.returncode == 0, res.stderr[-3000:]
    assert "__KDA_CHECK_OK__" in res.stdout


def test_prefill_decay_at_documented_limit(oracle64):
    """g = -4.5 on every token and channel (72 nats over 16 tokens, inside the
    documented range): the chunked prefill stays within tolerance of the
    oracle, states included."""
    U.say("prefill at the decay limit (g = -4.5 sustained)")
    dev = U.device()
    K.load_library()
    wl = make_workload(2, lengths=[300, 77], H=2, d=128)
    wl.g = torch.full_like(wl.g, -4.5)
    init = np.zeros((2, 2, 128, 128))
    init[0] = wl.init_states[0].double().numpy()
    has = np.array([1, 0], np.int32)
    ref = oracle64.kda_varlen(wl.q, wl.k, wl.v, wl.g, wl.beta, wl.cu_seqlens, init=init, has_init=has)
    q, k, v, g, b = (t.to(dev) for t in (wl.q, wl.k, wl.v, wl.g, wl.beta))
    pool = torch.zeros(4, 2, 128, 128, device=dev)
    pool[0] = wl.init_states[0].to(dev)
    o = torch.empty(q.shape[0], 2, 128, dtype=torch.bfloat16, device=dev)
    K.kda_prefill_varlen(q, k, v, g, b, o, wl.cu_seqlens.to(dev), pool,
                         torch.tensor([0, -1], dtype=torch.int32, device=dev),
                         torch.tensor([2, 3], dtype=torch.int32, device=dev), chunk=64)
    torch.cuda.synchronize()
    U.assert_close("o", U.to_np(o), ref["o"])
    U.assert_close("state", U.to_np(pool[2:]), ref["final"])
