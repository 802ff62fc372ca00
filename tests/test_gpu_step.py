"""GPU parity of kda_decode and kda_verify against the CPU oracle, through
the C ABI, on the seeded workloads and their edge cases."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import gpu_util as U
from hybrid_recurrent_serving_amd import kda as K
from hybrid_recurrent_serving_amd.inputs import make_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    d = U.device()
    K.load_library()
    return d


def _oracle_states(wl):
    init = np.zeros((wl.n_seq, wl.H, wl.dk, wl.dv))
    has = np.zeros(wl.n_seq, np.int32)
    for s, i in enumerate(wl.init_index):
        if i >= 0:
            init[s] = wl.init_states[i].double().numpy()
            has[s] = 1
    return init, has


def test_decode_tiny_stepped_64(dev, oracle64):
    """Tiny workload (T=64, H=2, d=16, fp32): 64 decode steps in place equal
    the oracle's token loop at every position and in the final state."""
    U.say("decode tiny stepped 64x")
    wl = make_workload(0)
    ref = oracle64.kda_varlen(wl.q, wl.k, wl.v, wl.g, wl.beta, wl.cu_seqlens)
    q, k, v, g, b = (t.to(dev) for t in (wl.q, wl.k, wl.v, wl.g, wl.beta))
    pool = torch.zeros(1, wl.H, wl.dk, wl.dv, device=dev)
    slot = torch.zeros(1, dtype=torch.int32, device=dev)
    o = torch.empty(64, wl.H, wl.dv, device=dev)
    for t in range(64):
        K.kda_decode(q[t:t + 1], k[t:t + 1], v[t:t + 1], g[t:t + 1], b[t:t + 1], o[t:t + 1],
                     pool, slot, slot)
    torch.cuda.synchronize()
    U.assert_close("o", U.to_np(o), ref["o"], rel=1e-5, mx=1e-5)
    U.assert_close("state", U.to_np(pool[0]), ref["final"][0], rel=1e-5, mx=1e-5)


def test_verify_tiny_windows_of_8(dev, oracle64):
    """Tiny workload (T=64, H=2, d=16, fp32) verified as 8 consecutive
    8-token windows, each starting from the state the window before
    committed (all 8 accepted): every output and the final state equal the
    oracle's token loop over the 64 tokens.  Then one window with L = 5 from
    the state after 16 tokens commits the oracle's state after 21."""
    U.say("verify tiny, 8-token windows")
    wl = make_workload(0)
    H, d = wl.H, wl.dk
    ref = oracle64.kda_varlen(wl.q, wl.k, wl.v, wl.g, wl.beta, wl.cu_seqlens)
    q, k, v, g, b = (t.to(dev) for t in (wl.q, wl.k, wl.v, wl.g, wl.beta))
    pool = torch.zeros(2, H, d, d, device=dev)
    i32 = lambda x: torch.tensor(x, dtype=torch.int32, device=dev)
    o = torch.empty(8, 8, H, d, device=dev)
    clen = torch.full((8,), -7, dtype=torch.int32, device=dev)
    win = lambda t, j: t[8 * j:8 * j + 8].unsqueeze(0).contiguous()
    for j in range(8):
        K.kda_verify(win(q, j), win(k, j), win(v, j), win(g, j), win(b, j), pool, i32([j % 2]),
                     i32([(j + 1) % 2]), o=o[j:j + 1], accepted_len=i32([8]), committed_len_out=clen[j:j + 1])
    torch.cuda.synchronize()
    assert clen.cpu().tolist() == [8] * 8
    U.assert_close("o", U.to_np(o.reshape(64, H, d)), ref["o"], rel=1e-5, mx=1e-5)
    U.assert_close("state", U.to_np(pool[0]), ref["final"][0], rel=1e-5, mx=1e-5)
    # the state after 16 tokens, then a window of 8 with 5 accepted
    cu16 = torch.tensor([0, 16], dtype=torch.int32)
    s16 = oracle64.kda_varlen(wl.q[:16], wl.k[:16], wl.v[:16], wl.g[:16], wl.beta[:16], cu16)["final"]
    cu21 = torch.tensor([0, 21], dtype=torch.int32)
    s21 = oracle64.kda_varlen(wl.q[:21], wl.k[:21], wl.v[:21], wl.g[:21], wl.beta[:21], cu21)["final"]
    pool2 = torch.zeros(2, H, d, d, device=dev)
    pool2[0] = torch.tensor(s16[0], dtype=torch.float32, device=dev)
    K.kda_verify(win(q, 2), win(k, 2), win(v, 2), win(g, 2), win(b, 2), pool2, i32([0]), i32([1]),
                 accepted_len=i32([5]))
    torch.cuda.synchronize()
    U.assert_close("state after 21", U.to_np(pool2[1]), s21[0], rel=1e-5, mx=1e-5)


def test_decode_batched_128(dev, oracle64):
    """Batched decode: 128 sequences x 1 token, H=16, d=128, bf16 inputs,
    random fp32 states updated in place."""
    U.say("decode batched 128 x H16 x d128")
    wl = make_workload(1)
    init, has = _oracle_states(wl)
    ref = oracle64.kda_varlen(wl.q, wl.k, wl.v, wl.g, wl.beta, wl.cu_seqlens, init=init,
                              has_init=has)
    q, k, v, g, b = (t.to(dev) for t in (wl.q, wl.k, wl.v, wl.g, wl.beta))
    pool = wl.init_states.to(dev).clone()
    slots = torch.arange(128, dtype=torch.int32, device=dev)
    o = torch.empty(128, 16, 128, dtype=torch.bfloat16, device=dev)
    K.kda_decode(q, k, v, g, b, o, pool, slots, slots)
    o32 = torch.empty(128, 16, 128, dtype=torch.float32, device=dev)
    pool2 = wl.init_states.to(dev).clone()
    K.kda_decode(q, k, v, g, b, o32, pool2, slots, slots)
    torch.cuda.synchronize()
    U.assert_close("o(bf16)", U.to_np(o), ref["o"])
    U.assert_close("o(fp32)", U.to_np(o32), ref["o"], rel=1e-5, mx=1e-4)
    U.assert_close("state", U.to_np(pool), ref["final"], rel=1e-5, mx=1e-4)
    # bf16 output = the fp32 output rounded once
    assert torch.equal(o, o32.to(torch.bfloat16))
    assert torch.equal(pool, pool2)


def test_decode_slots_cow_and_edges(dev):
    """src != dst leaves src untouched (copy-on-write); src = -1 starts from
    zero; dst = -1 writes nothing; out-of-range slots are never touched."""
    U.say("decode slots / CoW / edges")
    wl = make_workload(1, n_seq=6)
    q, k, v, g, b = (t.to(dev) for t in (wl.q, wl.k, wl.v, wl.g, wl.beta))
    pool = torch.randn(12, 16, 128, 128, device=dev) * 0.1
    before = pool.clone()
    src = torch.tensor([0, 1, -1, 3, 4, 99], dtype=torch.int32, device=dev)
    dst = torch.tensor([6, 7, 8, -1, 4, 9], dtype=torch.int32, device=dev)
    o = torch.empty(6, 16, 128, device=dev)
    K.kda_decode(q, k, v, g, b, o, pool, src, dst)
    torch.cuda.synchronize()
    for s in (0, 1, 3):
        assert torch.equal(pool[s], before[s]), "source slot modified"
    assert torch.equal(pool[5], before[5]) and torch.equal(pool[10], before[10])
    assert torch.equal(pool[11], before[11])
    # a zero source equals an explicit zero state
    zp = torch.zeros(1, 16, 128, 128, device=dev)
    z = torch.zeros(1, dtype=torch.int32, device=dev)
    o2 = torch.empty(1, 16, 128, device=dev)
    K.kda_decode(q[2:3], k[2:3], v[2:3], g[2:3], b[2:3], o2, zp, z, z)
    torch.cuda.synchronize()
    assert torch.equal(pool[8], zp[0]) and torch.equal(o[2], o2[0])
    # out-of-range source (99) behaves as zero state
    K.kda_decode(q[5:6], k[5:6], v[5:6], g[5:6], b[5:6], o2, zp.zero_(), z, z)
    torch.cuda.synchronize()
    assert torch.equal(pool[9], zp[0])
    # copy-on-write result equals the in-place result
    pool_ip = before.clone()
    slots = torch.tensor([0, 1], dtype=torch.int32, device=dev)
    o3 = torch.empty(2, 16, 128, device=dev)
    K.kda_decode(q[:2], k[:2], v[:2], g[:2], b[:2], o3, pool_ip, slots, slots)
    torch.cuda.synchronize()
    assert torch.equal(pool_ip[0], pool[6]) and torch.equal(pool_ip[1], pool[7])
    assert torch.equal(o3, o[:2])


@pytest.mark.parametrize("d", [16, 32, 64])
def test_decode_small_heads(dev, oracle64, d):
    U.say(f"decode d={d}")
    wl = make_workload(1, n_seq=5, H=3, d=d)
    init, has = _oracle_states(wl)
    ref = oracle64.kda_varlen(wl.q, wl.k, wl.v, wl.g, wl.beta, wl.cu_seqlens, init=init,
                              has_init=has, scale=0.5)
    q, k, v, g, b = (t.to(dev) for t in (wl.q, wl.k, wl.v, wl.g, wl.beta))
    pool = wl.init_states.to(dev).clone()
    slots = torch.arange(5, dtype=torch.int32, device=dev)
    o = torch.empty(5, 3, d, device=dev)
    K.kda_decode(q, k, v, g, b, o, pool, slots, slots, scale=0.5)
    torch.cuda.synchronize()
    U.assert_close("o", U.to_np(o), ref["o"], rel=1e-5, mx=1e-4)
    U.assert_close("state", U.to_np(pool), ref["final"], rel=1e-5, mx=1e-4)


def test_decode_strided_inputs(dev, oracle64):
    """q, k, v as views into one fused projection buffer (token stride 3*H*d)."""
    U.say("decode strided")
    wl = make_workload(1, n_seq=7, H=4, d=64)
    init, has = _oracle_states(wl)
    ref = oracle64.kda_varlen(wl.q, wl.k, wl.v, wl.g, wl.beta, wl.cu_seqlens, init=init,
                              has_init=has)
    fused = torch.cat([wl.q, wl.k, wl.v], dim=1).to(dev)  # [N, 3H, d]
    q, k, v = fused[:, 0:4], fused[:, 4:8], fused[:, 8:12]
    g, b = wl.g.to(dev), wl.beta.to(dev)
    pool = wl.init_states.to(dev).clone()
    slots = torch.arange(7, dtype=torch.int32, device=dev)
    o = torch.empty(7, 4, 64, dtype=torch.bfloat16, device=dev)
    K.kda_decode(q, k, v, g, b, o, pool, slots, slots)
    torch.cuda.synchronize()
    U.assert_close("o", U.to_np(o), ref["o"])
    U.assert_close("state", U.to_np(pool), ref["final"], rel=1e-5, mx=1e-4)


def test_decode_d128_strided_inputs(dev, oracle64):
    """d = 128: q, k, v as views into one fused projection buffer (token
    stride 3 H d), the per-row values staged from strided rows."""
    U.say("decode d128 strided")
    wl = make_workload(1, n_seq=9, H=4, d=128)
    init, has = _oracle_states(wl)
    ref = oracle64.kda_varlen(wl.q, wl.k, wl.v, wl.g, wl.beta, wl.cu_seqlens, init=init,
                              has_init=has)
    fused = torch.cat([wl.q, wl.k, wl.v], dim=1).to(dev)  # [N, 3H, d]
    q, k, v = fused[:, 0:4], fused[:, 4:8], fused[:, 8:12]
    g, b = wl.g.to(dev), wl.beta.to(dev)
    pool = wl.init_states.to(dev).clone()
    slots = torch.arange(9, dtype=torch.int32, device=dev)
    o = torch.empty(9, 4, 128, dtype=torch.bfloat16, device=dev)
    K.kda_decode(q, k, v, g, b, o, pool, slots, slots)
    torch.cuda.synchronize()
    U.assert_close("o", U.to_np(o), ref["o"])
    U.assert_close("state", U.to_np(pool), ref["final"], rel=1e-5, mx=1e-4)


# ------------------------------------------------------------------ verify
def test_verify_fused_128x8(dev, oracle64):
    """Speculative verify: 128 sequences x 8 tokens, outputs at all positions,
    state committed after exactly L ~ U{1..8} tokens; commit index exact."""
    U.say("verify fused 128 x 8")
    wl = make_workload(4)
    L = wl.accepted_len
    ref = oracle64.kda_verify(wl.q, wl.k, wl.v, wl.g, wl.beta, wl.init_states, L)
    q, k, v, g, b = (t.to(dev) for t in (wl.q, wl.k, wl.v, wl.g, wl.beta))
    pool = torch.cat([wl.init_states, torch.zeros_like(wl.init_states)]).to(dev)
    src = torch.arange(128, dtype=torch.int32, device=dev)
    dst = src + 128
    o = torch.empty(128, 8, 16, 128, dtype=torch.bfloat16, device=dev)
    clen = torch.full((128,), -7, dtype=torch.int32, device=dev)
    K.kda_verify(q, k, v, g, b, pool, src, dst, o=o, accepted_len=L.to(dev), committed_len_out=clen)
    torch.cuda.synchronize()
    assert torch.equal(clen.cpu(), L), "committed length differs"
    assert np.array_equal(ref["committed_len"], L.numpy())
    U.assert_close("o", U.to_np(o), ref["o"])
    U.assert_close("committed", U.to_np(pool[128:]), ref["committed"], rel=1e-5, mx=1e-4)
    assert torch.equal(pool[:128].cpu(), wl.init_states), "source states modified"


def test_verify_two_phase_equals_fused(dev):
    """Outputs-only then commit-only gives bit-identical outputs and states to
    the fused pass (same arithmetic in the same order)."""
    U.say("verify two-phase == fused")
    wl = make_workload(4, n_seq=32)
    q, k, v, g, b = (t.to(dev) for t in (wl.q, wl.k, wl.v, wl.g, wl.beta))
    L = wl.accepted_len.to(dev)
    pool_f = wl.init_states.to(dev).clone()
    pool_t = wl.init_states.to(dev).clone()
    slots = torch.arange(32, dtype=torch.int32, device=dev)
    o_f = torch.empty(32, 8, 16, 128, device=dev)
    o_t = torch.empty(32, 8, 16, 128, device=dev)
    K.kda_verify(q, k, v, g, b, pool_f, slots, slots, o=o_f, accepted_len=L)
    K.kda_verify(q, k, v, g, b, pool_t, slots, slots, o=o_t)       # outputs only
    torch.cuda.synchronize()
    assert torch.equal(pool_t, wl.init_states.to(dev)), "outputs-only pass wrote the pool"
    K.kda_verify(q, k, v, g, b, pool_t, slots, slots, accepted_len=L)  # commit only
    torch.cuda.synchronize()
    assert torch.equal(o_f, o_t)
    assert torch.equal(pool_f, pool_t)


def test_verify_edge_lengths(dev, oracle64):
    """L = 0 commits the source state; L outside [0, T_spec] is rejected
    (committed length -1, destination untouched); L = T_spec equals T_spec
    decode steps."""
    U.say("verify edge lengths")
    wl = make_workload(4, n_seq=6, H=2, d=32)
    L = torch.tensor([0, 8, -1, 9, 3, 1], dtype=torch.int32)
    ref = oracle64.kda_verify(wl.q, wl.k, wl.v, wl.g, wl.beta, wl.init_states, L)
    q, k, v, g, b = (t.to(dev) for t in (wl.q, wl.k, wl.v, wl.g, wl.beta))
    pool = torch.cat([wl.init_states, torch.full_like(wl.init_states, 7.0)]).to(dev)
    src = torch.arange(6, dtype=torch.int32, device=dev)
    dst = src + 6
    clen = torch.zeros(6, dtype=torch.int32, device=dev)
    o = torch.empty(6, 8, 2, 32, device=dev)
    K.kda_verify(q, k, v, g, b, pool, src, dst, o=o, accepted_len=L.to(dev), committed_len_out=clen)
    torch.cuda.synchronize()
    assert clen.cpu().tolist() == [0, 8, -1, -1, 3, 1]
    assert torch.equal(pool[6].cpu(), wl.init_states[0])
    assert torch.all(pool[8] == 7.0) and torch.all(pool[9] == 7.0)
    for s in (1, 4, 5):
        U.assert_close(f"committed[{s}]", U.to_np(pool[6 + s]), ref["committed"][s], rel=1e-5, mx=1e-4)
    U.assert_close("o", U.to_np(o), ref["o"], rel=1e-5, mx=1e-4)
    # L = T_spec commit equals 8 in-place decode steps
    pool_d = wl.init_states[1:2].to(dev).clone()
    z = torch.zeros(1, dtype=torch.int32, device=dev)
    od = torch.empty(1, 2, 32, device=dev)
    for t in range(8):
        K.kda_decode(q[1:2, t], k[1:2, t], v[1:2, t], g[1:2, t], b[1:2, t], od, pool_d, z, z)
        torch.cuda.synchronize()
        assert torch.equal(od[0], o[1, t])
    assert torch.equal(pool_d[0], pool[7])


def test_verify_commit_index_probe(dev):
    """alpha = 1, beta = 1, exactly orthonormal keys, queries = keys: the
    committed state reads back v_j for j < L and the source state's value for
    j >= L, so the commit index is recovered exactly from the state."""
    U.say("verify commit-index probe")
    import oracle_pins as P
    r = np.random.default_rng(5)
    N, Ts, H, d = 16, 8, 1, 16
    keys = P.exact_orthonormal_rows(r, d)[:Ts]
    k = torch.tensor(np.broadcast_to(keys[None, :, None, :], (N, Ts, H, d)).copy(), dtype=torch.float32)
    v = torch.tensor(r.standard_normal((N, Ts, H, d)), dtype=torch.float32)
    g = torch.zeros(N, Ts, H, d)
    b = torch.ones(N, Ts, H)
    S0 = torch.tensor(r.standard_normal((N, H, d, d)), dtype=torch.float32)
    L = torch.tensor(r.integers(0, Ts + 1, N), dtype=torch.int32)
    pool = torch.cat([S0, torch.zeros_like(S0)]).to(dev)
    src = torch.arange(N, dtype=torch.int32, device=dev)
    K.kda_verify(k.to(dev), k.to(dev), v.to(dev), g.to(dev), b.to(dev), pool, src, src + N,
                 accepted_len=L.to(dev))
    torch.cuda.synchronize()
    S = pool[N:].double().cpu().numpy()
    kk = keys.astype(np.float64)
    for s in range(N):
        readout = S[s, 0].T @ kk.T  # [d_v, Ts]: column j = S^T k_j
        written = [np.allclose(readout[:, j], v[s, j, 0].numpy(), atol=1e-5) for j in range(Ts)]
        recovered = 0
        while recovered < Ts and written[recovered]:
            recovered += 1
        assert recovered == int(L[s]), (s, recovered, int(L[s]))
        for j in range(int(L[s]), Ts):
            np.testing.assert_allclose(readout[:, j], S0[s, 0].double().numpy().T @ kk[j], atol=1e-5)


@pytest.mark.parametrize("T_spec,d,dtype", [(16, 128, torch.bfloat16), (3, 64, torch.bfloat16),
                                            (16, 32, torch.float32), (2, 16, torch.float32)])
def test_verify_token_counts_and_sizes(dev, oracle64, T_spec, d, dtype):
    """Verify over the supported range of draft counts (up to 16 tokens, the
    most one call stages) and head sizes, bf16 and fp32 inputs, with accepted
    lengths spanning 0..T_spec."""
    U.say(f"verify T_spec={T_spec} d={d} {dtype}")
    N, H = 24, 3
    wl = make_workload(4, n_seq=N, H=H, d=d, T=T_spec)
    q, k, v, g, b = (t.to(dtype) for t in (wl.q, wl.k, wl.v, wl.g, wl.beta))
    L = torch.arange(N, dtype=torch.int32) % (T_spec + 1)
    ref = oracle64.kda_verify(q, k, v, g, b, wl.init_states, L)
    pool = torch.cat([wl.init_states, torch.zeros_like(wl.init_states)]).to(dev)
    src = torch.arange(N, dtype=torch.int32, device=dev)
    dst = src + N
    o = torch.empty(N, T_spec, H, d, dtype=dtype, device=dev)
    clen = torch.full((N,), -7, dtype=torch.int32, device=dev)
    K.kda_verify(q.to(dev), k.to(dev), v.to(dev), g.to(dev), b.to(dev), pool, src, dst, o=o,
                 accepted_len=L.to(dev), committed_len_out=clen)
    torch.cuda.synchronize()
    assert torch.equal(clen.cpu(), L)
    tol = {} if dtype == torch.bfloat16 else {"rel": 1e-5, "mx": 1e-4}
    U.assert_close("o", U.to_np(o), ref["o"], **tol)
    U.assert_close("committed", U.to_np(pool[N:]), ref["committed"], rel=1e-5, mx=1e-4)


@pytest.mark.parametrize("T_spec,dtype,mu_g", [(8, torch.float32, 0.0), (5, torch.bfloat16, 0.0),
                                               (2, torch.float32, 0.0), (8, torch.float32, 4.0),
                                               (7, torch.bfloat16, 4.0)])
def test_verify_d128_window_form(dev, oracle64, T_spec, dtype, mu_g):
    """d = 128 with 2..8 tokens: outputs and committed states against the
    oracle for accepted lengths 0..T_spec, fast (E[alpha] = 0.5) and slow
    (alpha ~ 0.98) decay, a zero source and a rejected length."""
    U.say(f"verify d128 window T_spec={T_spec} {dtype} mu_g={mu_g}")
    N, H, d = 20, 2, 128
    wl = make_workload(4, n_seq=N, H=H, d=d, T=T_spec, mu_g=mu_g)
    q, k, v, g, b = (t.to(dtype) for t in (wl.q, wl.k, wl.v, wl.g, wl.beta))
    L = torch.arange(N, dtype=torch.int32) % (T_spec + 1)
    L[N - 1] = T_spec + 3   # rejected
    init = wl.init_states.clone()
    init[3] = 0.0           # the oracle's zero state for the sequence given src = -1
    ref = oracle64.kda_verify(q, k, v, g, b, init, L)
    pool = torch.cat([wl.init_states, torch.full_like(wl.init_states, 5.0)]).to(dev)
    src = torch.arange(N, dtype=torch.int32, device=dev)
    src[3] = -1
    dst = torch.arange(N, dtype=torch.int32, device=dev) + N
    o = torch.empty(N, T_spec, H, d, dtype=dtype, device=dev)
    clen = torch.full((N,), -7, dtype=torch.int32, device=dev)
    K.kda_verify(q.to(dev), k.to(dev), v.to(dev), g.to(dev), b.to(dev), pool, src, dst, o=o,
                 accepted_len=L.to(dev), committed_len_out=clen)
    torch.cuda.synchronize()
    expect = L.clone()
    expect[N - 1] = -1
    assert torch.equal(clen.cpu(), expect)
    tol = {} if dtype == torch.bfloat16 else {"rel": 1e-5, "mx": 1e-4}
    U.assert_close("o", U.to_np(o), ref["o"], **tol)
    U.assert_close("committed", U.to_np(pool[N:2 * N - 1]), ref["committed"][:N - 1], rel=1e-5, mx=1e-4)
    assert torch.all(pool[2 * N - 1] == 5.0), "rejected sequence wrote its destination"
    assert torch.equal(pool[:N].cpu(), wl.init_states), "source states modified"


def test_verify_d128_decay_spikes(dev, oracle64):
    """Per-token log-decay spikes of -20 on random channels (states decayed
    towards zero on those channels within one token): outputs and committed
    states stay finite and match the oracle."""
    U.say("verify d128 decay spikes")
    N, H, d, T_spec = 8, 2, 128, 8
    wl = make_workload(4, n_seq=N, H=H, d=d, T=T_spec)
    g = wl.g.clone()
    r = torch.Generator().manual_seed(11)
    spike = torch.rand(g.shape, generator=r) < 0.05
    g[spike] = -20.0
    L = torch.full((N,), T_spec, dtype=torch.int32)
    ref = oracle64.kda_verify(wl.q, wl.k, wl.v, g, wl.beta, wl.init_states, L)
    pool = torch.cat([wl.init_states, torch.zeros_like(wl.init_states)]).to(dev)
    src = torch.arange(N, dtype=torch.int32, device=dev)
    o = torch.empty(N, T_spec, H, d, device=dev)
    K.kda_verify(wl.q.to(dev), wl.k.to(dev), wl.v.to(dev), g.to(dev), wl.beta.to(dev), pool, src, src + N,
                 o=o, accepted_len=L.to(dev))
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(pool).all()
    U.assert_close("o", U.to_np(o), ref["o"], rel=1e-5, mx=1e-4)
    U.assert_close("committed", U.to_np(pool[N:]), ref["committed"], rel=1e-5, mx=1e-4)


@pytest.mark.parametrize("T_spec", [2, 9, 16])
def test_verify_d128_matrix_core_fp32_outputs(dev, oracle64, T_spec):
    """d = 128, bf16 inputs (the matrix-core verify, one chunk of T_spec rows
    with reference row (T_spec - 1) / 2), fp32 outputs: outputs and committed
    states against the oracle at fp32-grade tolerance for every accepted
    length 0..T_spec and a rejected one, and a commit-only call that commits
    the same states bit for bit."""
    U.say(f"verify d128 bf16 in / fp32 out T_spec={T_spec}")
    N, H, d = T_spec + 2, 2, 128
    wl = make_workload(4, n_seq=N, H=H, d=d, T=T_spec, seed=70 + T_spec)
    L = torch.arange(N, dtype=torch.int32) % (T_spec + 1)
    L[N - 1] = -2   # rejected
    ref = oracle64.kda_verify(wl.q, wl.k, wl.v, wl.g, wl.beta, wl.init_states, L)
    q, k, v, g, b = (t.to(dev) for t in (wl.q, wl.k, wl.v, wl.g, wl.beta))
    pool = torch.cat([wl.init_states, torch.full_like(wl.init_states, 3.0)]).to(dev)
    src = torch.arange(N, dtype=torch.int32, device=dev)
    dst = src + N
    o = torch.empty(N, T_spec, H, d, device=dev)
    clen = torch.full((N,), -7, dtype=torch.int32, device=dev)
    K.kda_verify(q, k, v, g, b, pool, src, dst, o=o, accepted_len=L.to(dev), committed_len_out=clen)
    torch.cuda.synchronize()
    expect = L.clone()
    expect[N - 1] = -1
    assert torch.equal(clen.cpu(), expect)
    U.assert_close("o", U.to_np(o), ref["o"], rel=2e-5, mx=1e-4)
    U.assert_close("committed", U.to_np(pool[N:2 * N - 1]), ref["committed"][:N - 1], rel=1e-5, mx=1e-4)
    assert torch.all(pool[2 * N - 1] == 3.0), "rejected sequence wrote its destination"
    pool2 = torch.cat([wl.init_states, torch.full_like(wl.init_states, 3.0)]).to(dev)
    K.kda_verify(q, k, v, g, b, pool2, src, dst, accepted_len=L.to(dev))   # commit only
    torch.cuda.synchronize()
    assert torch.equal(pool2, pool)


def test_decode_d128_item_count_not_multiple_of_8(dev, oracle64):
    """d = 128 decode with 5 sequences x 3 heads = 15 (sequence, head) items,
    a grid that is no multiple of the 8 XCDs; fp32 in and out against the
    oracle, in place and copy-on-write."""
    U.say("decode d128, 15 items")
    wl = make_workload(1, n_seq=5, H=3, d=128)
    init, has = _oracle_states(wl)
    q, k, v, g, b = (t.float() for t in (wl.q, wl.k, wl.v, wl.g, wl.beta))
    ref = oracle64.kda_varlen(q, k, v, g, b, wl.cu_seqlens, init=init, has_init=has, scale=0.7)
    pool = torch.cat([wl.init_states, torch.zeros_like(wl.init_states)]).to(dev)
    src = torch.arange(5, dtype=torch.int32, device=dev)
    o = torch.empty(5, 3, 128, device=dev)
    K.kda_decode(q.to(dev), k.to(dev), v.to(dev), g.to(dev), b.to(dev), o, pool, src, src + 5, scale=0.7)
    torch.cuda.synchronize()
    U.assert_close("o", U.to_np(o), ref["o"], rel=1e-5, mx=1e-5)
    U.assert_close("state", U.to_np(pool[5:]), ref["final"], rel=1e-5, mx=1e-5)
    assert torch.equal(pool[:5].cpu(), wl.init_states), "source states modified"
    pool2 = wl.init_states.to(dev).clone()
    o2 = torch.empty(5, 3, 128, device=dev)
    K.kda_decode(q.to(dev), k.to(dev), v.to(dev), g.to(dev), b.to(dev), o2, pool2, src, src, scale=0.7)
    torch.cuda.synchronize()
    assert torch.equal(o2, o) and torch.equal(pool2, pool[5:])


@pytest.mark.parametrize("with_o", [True, False])
def test_verify_one_token_d128(dev, oracle64, with_o):
    """A one-token verify at d = 128 keeps the verify semantics: L = 1 commits
    the state after the token, L = 0 commits the source state, L = -1 / 2 are
    rejected (committed length -1, destination untouched), and a commit-only
    call (o = NULL) writes no outputs."""
    U.say(f"verify T_spec=1 d=128 with_o={with_o}")
    wl = make_workload(4, n_seq=8, H=4)
    q, k, v, g, b = (t[:, :1].contiguous() for t in (wl.q, wl.k, wl.v, wl.g, wl.beta))
    L = torch.tensor([1, 0, -1, 2, 1, 0, 1, -1], dtype=torch.int32)
    ref = oracle64.kda_verify(q, k, v, g, b, wl.init_states, L)
    pool = torch.cat([wl.init_states, torch.full_like(wl.init_states, 7.0)]).to(dev)
    src = torch.arange(8, dtype=torch.int32, device=dev)
    clen = torch.full((8,), -7, dtype=torch.int32, device=dev)
    o = torch.full((8, 1, 4, 128), float("nan"), device=dev) if with_o else None
    K.kda_verify(*(t.to(dev) for t in (q, k, v, g, b)), pool, src, src + 8, o=o,
                 accepted_len=L.to(dev), committed_len_out=clen)
    torch.cuda.synchronize()
    assert clen.cpu().tolist() == [1, 0, -1, -1, 1, 0, 1, -1]
    assert torch.equal(pool[:8].cpu(), wl.init_states), "source states modified"
    for s in range(8):
        if L[s] in (-1, 2):
            assert torch.all(pool[8 + s] == 7.0), f"rejected sequence {s} wrote its destination"
        elif L[s] == 0:
            assert torch.equal(pool[8 + s].cpu(), wl.init_states[s])
        else:
            U.assert_close(f"committed[{s}]", U.to_np(pool[8 + s]), ref["committed"][s], rel=1e-5, mx=1e-4)
    if with_o:
        U.assert_close("o", U.to_np(o), ref["o"], rel=1e-5, mx=1e-4)
