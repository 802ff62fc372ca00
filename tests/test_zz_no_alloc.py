"""kda_prefill_varlen_noalloc (the prefill entry point that allocates
nothing: its segment-scan scratch is a static array of the library) against
kda_prefill_varlen with a caller workspace, through the C ABI.

Two calls in a row, the second on a smaller input, each compared bit for bit
with the workspace call on the same inputs (the same kernels run on the same
data in the same order); then a call whose split would need more scratch
than the library holds is refused without launching anything."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import gpu_util as U
from hybrid_recurrent_serving_amd import kda as K
from hybrid_recurrent_serving_amd.inputs import make_workload

pytestmark = pytest.mark.gpu


def _run(dev, wl, entry, *, segment_len, starts, ckpt_interval, in_place):
    N, H, d = wl.n_seq, wl.H, wl.dk
    ck_cu, _ = K.kda_ckpt_plan(wl.cu_seqlens.numpy(), ckpt_interval, 64, start_pos=starts)
    n_ck = int(ck_cu[-1])
    pool = torch.full((2 * N + n_ck, H, d, d), 7.0, device=dev)   # slots no call writes keep 7.0
    for s, i in enumerate(wl.init_index):
        pool[s] = wl.init_states[i].to(dev) if i >= 0 else 0.0
    i32 = lambda x: torch.tensor(x, dtype=torch.int32, device=dev)
    src = i32(list(range(N)))
    dst = src if in_place else i32(list(range(N, 2 * N)))
    o = torch.full((wl.q.shape[0], H, d), float("nan"), dtype=torch.bfloat16, device=dev)
    pos = torch.full((max(n_ck, 1),), -1, dtype=torch.int32, device=dev)
    entry(*(t.to(dev) for t in (wl.q, wl.k, wl.v, wl.g, wl.beta)), o, wl.cu_seqlens.to(dev), pool, src, dst,
          chunk=64, start_pos=i32(starts), ckpt_interval=ckpt_interval, ckpt_cu=i32(list(ck_cu)),
          ckpt_slot=i32(list(range(2 * N, 2 * N + n_ck))), ckpt_pos_out=pos, segment_len=segment_len)
    torch.cuda.synchronize()
    return o, pool, pos


@pytest.fixture(scope="module")
def dev():
    d = U.device()
    K.load_library()
    return d


def test_noalloc_matches_workspace_call_twice(dev, oracle64):
    """Call 1: 6 sequences (3,700 tokens), H=4, d=128, 256-token segments,
    checkpoints every 512, unaligned starts, in place.  Call 2: a smaller
    batch (3 sequences, 1,100 tokens) right after, copy-on-write.  Each
    equals the workspace call bit for bit; call 1 is also checked against the
    oracle."""
    U.say("prefill noalloc: two calls vs the workspace entry point")
    cases = [
        dict(lengths=[900, 333, 1200, 64, 700, 503], starts=[0, 40, 96, 7, 512, 300], in_place=True, seed=21),
        dict(lengths=[500, 260, 340], starts=[64, 0, 13], in_place=False, seed=22),
    ]
    for n, c in enumerate(cases):
        wl = make_workload(2, lengths=c["lengths"], H=4, d=128, seed=c["seed"])
        kw = dict(segment_len=256, starts=c["starts"], ckpt_interval=512, in_place=c["in_place"])
        need = K.kda_prefill_workspace_bytes(
            *(t.to(dev) for t in (wl.q, wl.k, wl.v, wl.g, wl.beta)),
            torch.empty(wl.q.shape[0], 4, 128, dtype=torch.bfloat16, device=dev), wl.cu_seqlens.to(dev),
            torch.empty(1, 4, 128, 128, device=dev), torch.zeros(wl.n_seq, dtype=torch.int32, device=dev),
            torch.zeros(wl.n_seq, dtype=torch.int32, device=dev), chunk=64, segment_len=256)
        assert 0 < need <= K.kda_prefill_noalloc_max_bytes(), need
        U.say(f"  call {n + 1}: {wl.q.shape[0]} tokens, scratch {need} bytes")
        o_a, pool_a, pos_a = _run(dev, wl, K.kda_prefill_varlen_noalloc, **kw)
        o_b, pool_b, pos_b = _run(dev, wl, K.kda_prefill_varlen, **kw)
        assert torch.equal(pos_a, pos_b)
        assert torch.equal(o_a, o_b), f"call {n + 1}: outputs differ"
        assert torch.equal(pool_a, pool_b), f"call {n + 1}: states differ"
        if n == 0:
            N = wl.n_seq
            init = np.stack([wl.init_states[i].double().numpy() if i >= 0 else np.zeros((4, 128, 128))
                             for i in wl.init_index])
            ref = oracle64.kda_varlen(wl.q, wl.k, wl.v, wl.g, wl.beta, wl.cu_seqlens, init=init,
                                      has_init=np.ones(N, np.int32), start_pos=np.array(c["starts"], np.int32),
                                      ckpt_interval=512)
            U.assert_close("o", U.to_np(o_a), ref["o"])
            U.assert_close("final+ckpt", np.concatenate([U.to_np(pool_a[:N]), U.to_np(pool_a[2 * N:])]),
                           np.concatenate([ref["final"], ref["ckpt"]]))


def test_noalloc_refuses_oversized_split(dev):
    """A split needing more scratch than the library holds returns
    KDA_ERR_WORKSPACE and leaves the outputs untouched."""
    U.say("prefill noalloc: oversized split refused")
    T, H, d = 40000, 16, 128
    q = torch.zeros(T, H, d, dtype=torch.bfloat16, device=dev)
    b = torch.zeros(T, H, dtype=torch.bfloat16, device=dev)
    o = torch.full((T, H, d), 3.0, dtype=torch.bfloat16, device=dev)
    pool = torch.zeros(2, H, d, d, device=dev)
    slots = torch.zeros(1, dtype=torch.int32, device=dev)
    cu = torch.tensor([0, T], dtype=torch.int32, device=dev)
    with pytest.raises(K.KDAError) as e:
        K.kda_prefill_varlen_noalloc(q, q, q, q, b, o, cu, pool, slots, slots, chunk=64, segment_len=1024)
    assert e.value.status == 5, e.value
    torch.cuda.synchronize()
    assert torch.all(o == 3.0)
