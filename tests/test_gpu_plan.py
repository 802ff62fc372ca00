"""GPU tests of kda_ckpt_plan_device (the checkpoint plan built on the device)
against the oracle's checkpoint enumeration, and of a HIP graph that records
the plan, the prefill and the fused decode step: every replay must equal the
same calls run eagerly on the same inputs."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import gpu_util as U
from hybrid_recurrent_serving_amd import kda as K
from hybrid_recurrent_serving_amd.inputs import draw_conv, make_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    d = U.device()
    K.load_library()
    return d


def _batch(rng, n, max_len, p_empty=0.1):
    lens = rng.integers(0, max_len + 1, n)
    lens[rng.random(n) < p_empty] = 0
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    starts = rng.integers(0, 3 * max_len + 1, n).astype(np.int32)
    return cu, starts


def _device_plan(dev, cu, starts, interval, chunk, cap, free=None):
    cu_d = torch.tensor(cu, dtype=torch.int32, device=dev)
    sp_d = None if starts is None else torch.tensor(starts, dtype=torch.int32, device=dev)
    fr_d = None if free is None else torch.tensor(free, dtype=torch.int32, device=dev)
    n_seq = len(cu) - 1
    # sentinels: entries the plan must not touch keep them
    ck_cu = torch.full((n_seq + 1,), -7, dtype=torch.int32, device=dev)
    pos = torch.full((max(cap, 1),), -7, dtype=torch.int32, device=dev)
    slot = torch.full((max(cap, 1),), -7, dtype=torch.int32, device=dev)
    tot = torch.full((1,), -7, dtype=torch.int32, device=dev)
    K.kda_ckpt_plan_device(cu_d, interval, chunk, int(cu[-1]), cap=cap, start_pos=sp_d, free_slots=fr_d,
                           ckpt_cu=ck_cu, ckpt_pos=pos, ckpt_slot=slot, n_total=tot)
    torch.cuda.synchronize()
    return ck_cu.cpu().numpy(), pos.cpu().numpy(), slot.cpu().numpy(), int(tot.item())


@pytest.mark.parametrize("n_seq", [1, 7, 100, 1024, 1500, 4099])
def test_device_plan_matches_oracle(dev, oracle64, n_seq):
    rng = np.random.default_rng(n_seq)
    for trial in range(3):
        cu, starts = _batch(rng, n_seq, 3000 if n_seq < 1000 else 400)
        chunk = int(rng.choice([16, 32, 64]))
        interval = chunk * int(rng.integers(1, 20))
        use_start = trial != 0
        o_cu, o_pos = oracle64.ckpt_enumerate(cu, interval, starts if use_start else None)
        total = int(o_cu[-1])
        # full capacity, free list shorter than the total
        n_free = total // 2
        free = rng.permutation(10 * (total + 1))[:n_free].astype(np.int32)
        U.say(f"plan n_seq={n_seq} trial={trial} interval={interval} total={total}")
        ck_cu, pos, slot, tot = _device_plan(dev, cu, starts if use_start else None, interval, chunk,
                                             total, free if n_free else None)
        assert tot == total
        assert np.array_equal(ck_cu, np.asarray(o_cu))
        assert np.array_equal(pos[:total], np.asarray(o_pos))
        want_slot = np.full(total, -1, np.int32)
        want_slot[:n_free] = free
        assert np.array_equal(slot[:total], want_slot)


def test_device_plan_capacity_and_edges(dev, oracle64):
    rng = np.random.default_rng(11)
    cu, starts = _batch(rng, 50, 5000)
    o_cu, o_pos = oracle64.ckpt_enumerate(cu, 256, starts)
    total = int(o_cu[-1])
    assert total > 40
    cap = total // 3
    ck_cu, pos, slot, tot = _device_plan(dev, cu, starts, 256, 64, cap, np.arange(cap + 5, dtype=np.int32))
    assert tot == total and np.array_equal(ck_cu, np.asarray(o_cu))
    assert np.array_equal(pos[:cap], np.asarray(o_pos)[:cap])
    assert np.array_equal(slot[:cap], np.arange(cap))
    # entries past cap are left alone (the arrays here hold exactly cap entries)
    # n_seq = 0: ckpt_cu[0] and the total are still written
    ck_cu, pos, slot, tot = _device_plan(dev, np.zeros(1, np.int32), None, 64, 64, 4)
    assert tot == 0 and ck_cu.tolist() == [0] and pos.tolist() == [-7] * 4
    # cap = 0: counts only
    ck_cu, _, _, tot = _device_plan(dev, cu, starts, 256, 64, 0)
    assert tot == total and np.array_equal(ck_cu, np.asarray(o_cu))
    # all sequences empty
    ck_cu, _, _, tot = _device_plan(dev, np.zeros(9, np.int32), np.arange(8, dtype=np.int32) * 999, 64, 64, 4)
    assert tot == 0 and ck_cu.tolist() == [0] * 9
    # a sequence ending exactly on a multiple: the final state is no checkpoint
    ck_cu, pos, _, tot = _device_plan(dev, np.array([0, 1024], np.int32), None, 256, 64, 8)
    assert tot == 3 and pos[:3].tolist() == [256, 512, 768]


def _prefill_inputs(dev, d=64, H=2):
    wl = make_workload(2, lengths=[700, 0, 1500, 64, 2100, 333], H=H, d=d, seed=5)
    N = wl.n_seq
    pool = torch.zeros(64, H, d, d, device=dev)
    for s, i in enumerate(wl.init_index):
        if i >= 0:
            pool[s] = wl.init_states[i].to(dev)
    src = torch.tensor([s if i >= 0 else -1 for s, i in enumerate(wl.init_index)], dtype=torch.int32,
                       device=dev)
    dst = torch.arange(N, 2 * N, dtype=torch.int32, device=dev)
    return wl, pool, src, dst


def test_device_plan_drives_prefill(dev):
    """The prefill with the device plan (positions, free-list slots) equals the
    prefill with the host plan, bit for bit."""
    wl, pool0, src, dst = _prefill_inputs(dev)
    N, interval, chunk = wl.n_seq, 256, 64
    q, k, v, g, b = (t.to(dev) for t in (wl.q, wl.k, wl.v, wl.g, wl.beta))
    cu_d = wl.cu_seqlens.to(dev)
    starts = torch.tensor([0, 5, 100, 250, 7, 1000], dtype=torch.int32, device=dev)
    host_cu, host_pos = K.kda_ckpt_plan(wl.cu_seqlens.numpy(), interval, chunk,
                                        start_pos=starts.cpu().numpy())
    n_ck = host_cu[-1]
    cap = n_ck + 3
    free = torch.arange(2 * N, 2 * N + cap, dtype=torch.int32, device=dev)
    runs = []
    for mode in ("host", "device"):
        pool = pool0.clone()
        o = torch.empty(q.shape[0], wl.H, wl.dv, dtype=torch.bfloat16, device=dev)
        pos_out = torch.full((cap,), -1, dtype=torch.int32, device=dev)
        if mode == "host":
            ck_cu = torch.tensor(host_cu, dtype=torch.int32, device=dev)
            ck_slot = free[:n_ck].clone()
            n_ckpt = n_ck
        else:
            ck_cu, ck_pos, ck_slot, tot = K.kda_ckpt_plan_device(cu_d, interval, chunk, q.shape[0], cap=cap,
                                                                 start_pos=starts, free_slots=free)
            n_ckpt = cap
        K.kda_prefill_varlen(q, k, v, g, b, o, cu_d, pool, src, dst, chunk=chunk, start_pos=starts,
                             ckpt_interval=interval, ckpt_cu=ck_cu, ckpt_slot=ck_slot, ckpt_pos_out=pos_out)
        torch.cuda.synchronize()
        runs.append((o.cpu(), pool.cpu(), pos_out[:n_ck].cpu().tolist()))
        if mode == "device":
            assert int(tot.item()) == n_ck
            assert ck_pos[:n_ck].cpu().tolist() == host_pos
    assert torch.equal(runs[0][0], runs[1][0])
    assert torch.equal(runs[0][1], runs[1][1])
    assert runs[0][2] == runs[1][2] == host_pos


def test_graph_replays_plan_prefill_decode(dev):
    """Plan, prefill and fused decode recorded in one HIP graph; each replay
    (inputs changed in place, eager work and synchronisation between replays)
    equals the eager calls on the same inputs, bit for bit."""
    wl, pool0, src, dst = _prefill_inputs(dev)
    N, H, d, interval, chunk = wl.n_seq, wl.H, wl.dv, 512, 64
    T = wl.q.shape[0]
    # prefill inputs (captured buffers)
    q, k, v, g, b = (t.to(dev).clone() for t in (wl.q, wl.k, wl.v, wl.g, wl.beta))
    cu_d = wl.cu_seqlens.to(dev)
    cap = 16
    free = torch.arange(2 * N, 2 * N + cap, dtype=torch.int32, device=dev)
    ck_cu = torch.empty(N + 1, dtype=torch.int32, device=dev)
    ck_pos = torch.empty(cap, dtype=torch.int32, device=dev)
    ck_slot = torch.empty(cap, dtype=torch.int32, device=dev)
    tot = torch.empty(1, dtype=torch.int32, device=dev)
    pos_out = torch.empty(cap, dtype=torch.int32, device=dev)
    # decode inputs: one token for each of 8 sequences, from slots [0, 8) to [8, 16)
    Nd = 8
    gen = torch.Generator().manual_seed(77)
    C = 3 * H * d
    w, hist, x = draw_conv(gen, Nd, C, 4, Nd, torch.bfloat16, torch.device("cpu"))
    wd = make_workload(1, n_seq=Nd, H=H, d=d, seed=9)
    xd, wconv = x.to(dev), w.to(dev)
    gd, bd = wd.g.to(dev).clone(), wd.beta.to(dev).clone()
    dsrc = torch.arange(Nd, dtype=torch.int32, device=dev)
    ddst = dsrc + Nd

    def fresh_pools():
        pool = pool0.clone()
        dpool = torch.zeros(2 * Nd, H, d, d, device=dev)
        dpool[:Nd] = wd.init_states.to(dev)
        cpool = torch.zeros(2 * Nd, C, 3, dtype=torch.bfloat16, device=dev)
        cpool[:Nd] = hist.to(dev)
        return pool, dpool, cpool

    pool, dpool, cpool = fresh_pools()
    o = torch.empty(T, H, d, dtype=torch.bfloat16, device=dev)
    od = torch.empty(Nd, H, d, dtype=torch.bfloat16, device=dev)

    def calls(pool, dpool, cpool, o, od):
        K.kda_ckpt_plan_device(cu_d, interval, chunk, T, cap=cap, free_slots=free, ckpt_cu=ck_cu,
                               ckpt_pos=ck_pos, ckpt_slot=ck_slot, n_total=tot)
        K.kda_prefill_varlen(q, k, v, g, b, o, cu_d, pool, src, dst, chunk=chunk, ckpt_interval=interval,
                             ckpt_cu=ck_cu, ckpt_slot=ck_slot, ckpt_pos_out=pos_out)
        K.kda_decode_conv(xd, wconv, cpool, dsrc, ddst, gd, bd, od, dpool, dsrc, ddst, act=1, qk_l2norm=True)

    def snapshot(pool, dpool, cpool, o, od):
        n_ck = int(tot.item())
        return [o.clone(), pool[N:2 * N + n_ck].clone(), od.clone(), dpool[Nd:].clone(), cpool[Nd:].clone(),
                ck_cu.clone(), ck_pos[:n_ck].clone(), pos_out[:n_ck].clone()]

    # warm-up, then capture on a side stream
    calls(pool, dpool, cpool, o, od)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls(pool, dpool, cpool, o, od)
    torch.cuda.synchronize()
    gen2 = torch.Generator().manual_seed(123)
    for rep in range(3):
        U.say(f"graph replay {rep}")
        # new inputs in place, and the output buffers cleared (eager work)
        for t in (q, k, v):
            t.copy_((torch.randn(t.shape, generator=gen2) * 0.1).to(t.dtype))
        xd.copy_(torch.randn(xd.shape, generator=gen2).to(xd.dtype))
        o.fill_(float("nan"))
        od.fill_(float("nan"))
        p2, d2, c2 = fresh_pools()
        pool.copy_(p2)
        dpool.copy_(d2)
        cpool.copy_(c2)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = snapshot(pool, dpool, cpool, o, od)
        # eager on the same inputs
        pe, de, ce = fresh_pools()
        oe = torch.empty_like(o)
        ode = torch.empty_like(od)
        calls(pe, de, ce, oe, ode)
        torch.cuda.synchronize()
        want = snapshot(pe, de, ce, oe, ode)
        assert int(tot.item()) == 7   # 700, 1500, 2100 tokens: 1 + 2 + 4 interior multiples of 512
        for i, (a, e) in enumerate(zip(got, want)):
            assert torch.equal(a, e), (rep, i)
        assert not torch.isnan(o.float()).any() and not torch.isnan(od.float()).any()
