"""Pins of the CPU oracle against facts other than itself.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises AssertionError
when the oracle disagrees with a closed form, an invariant, a special case or
a brute-force evaluation.  ``test_oracle_pins.py`` runs them on the oracle;
``test_oracle_mutants.py`` runs them on builds with a planted mistake and
requires that every mistake is caught by at least one pin.
"""

from __future__ import annotations

import numpy as np

from oracle import bruteforce


def _rng(seed):
    return np.random.default_rng(seed)


def _unit_rows(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def tiny_case(seed, T=6, H=2, dk=5, dv=4, g_scale=1.0):
    r = _rng(seed)
    q = _unit_rows(r.standard_normal((T, H, dk))).astype(np.float32)
    k = _unit_rows(r.standard_normal((T, H, dk))).astype(np.float32)
    v = r.standard_normal((T, H, dv)).astype(np.float32)
    g = (-np.log1p(np.exp(-r.standard_normal((T, H, dk)))) * g_scale).astype(np.float32)
    beta = (1 / (1 + np.exp(-r.standard_normal((T, H))))).astype(np.float32)
    S0 = r.standard_normal((1, H, dk, dv)) * 0.5
    return q, k, v, g, beta, S0


def _run(orc, q, k, v, g, beta, S0=None, scale=1.0, cu=None):
    T = q.shape[0]
    cu = np.array([0, T], np.int32) if cu is None else np.asarray(cu, np.int32)
    return orc.kda_varlen(q, k, v, g, beta, cu, init=S0, scale=scale)


def exact_orthonormal_rows(r, d=16):
    """Rows of a d x d orthonormal matrix whose entries (+-1/4 for d = 16) are
    exact in float32: a Sylvester-Hadamard matrix / sqrt(d), with its rows
    and columns permuted and signs flipped at random."""
    Hm = np.array([[1.0]])
    while Hm.shape[0] < d:
        Hm = np.block([[Hm, Hm], [Hm, -Hm]])
    Hm = Hm / np.sqrt(d)
    Hm = Hm[r.permutation(d)][:, r.permutation(d)] * r.choice([-1.0, 1.0], d)[None, :]
    return Hm


def _tol(orc):
    return 1e-12 if orc.real == np.float64 else 2e-5


def pin_bruteforce(orc):
    """Token loop == explicit transition matrices == unrolled closed sum (tiny, dk != dv)."""
    for seed in range(3):
        q, k, v, g, beta, S0 = tiny_case(seed)
        res = _run(orc, q, k, v, g, beta, S0, scale=0.75)
        for h in range(q.shape[1]):
            args = (q[:, h], k[:, h], v[:, h], g[:, h], beta[:, h], S0[0, h])
            o_m, S_m = bruteforce.matrix_form(*args, scale=0.75)
            o_u, S_u = bruteforce.unrolled_form(*args, scale=0.75)
            np.testing.assert_allclose(o_m, o_u, rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(res["o"][:, h], o_m, rtol=_tol(orc), atol=_tol(orc))
            np.testing.assert_allclose(res["final"][0, h], S_m, rtol=_tol(orc), atol=_tol(orc))


def pin_readback(orc):
    """alpha = 1, beta = 1, orthonormal keys: the state returns v_i for key k_i,
    whatever the initial state, and a later write to the same key overwrites."""
    d = 16
    r = _rng(11)
    keys = exact_orthonormal_rows(r, d)
    n = 6
    T = 2 * n
    k = np.zeros((T, 1, d), np.float32)
    q = np.zeros((T, 1, d), np.float32)
    v = r.standard_normal((T, 1, d)).astype(np.float32)
    k[:n, 0] = keys[:n]
    q[:n, 0] = keys[:n]
    # second half: re-write keys 0..n-1 with new values, query the previous key
    k[n:, 0] = keys[:n]
    q[n:, 0] = keys[np.arange(n) - 1]
    kk = k.astype(np.float64)[:, 0]
    g = np.zeros((T, 1, d), np.float32)
    beta = np.ones((T, 1), np.float32)
    S0 = r.standard_normal((1, 1, d, d))
    res = _run(orc, q, k, v, g, beta, S0)
    o = res["o"][:, 0]
    tol = 1e-10 if orc.real == np.float64 else 5e-5
    # first pass: o_t = v_t (query = the key just written)
    np.testing.assert_allclose(o[:n], v[:n, 0], atol=tol)
    # second pass, step t = n + j writes key j again and queries key j - 1:
    # for j >= 1 that key was re-written one step earlier (value v_{t-1});
    # for j = 0 the query is key d-1, never written, which still reads the
    # initial state's value for that direction.
    for t in range(n, T):
        j = t - n
        expect = v[t - 1, 0] if j >= 1 else S0[0, 0].T @ keys[d - 1]
        np.testing.assert_allclose(o[t], expect, atol=tol)
    # final read-back: S^T k_i = latest value written for key i
    S = res["final"][0, 0]
    for i in range(n):
        np.testing.assert_allclose(S.T @ kk[i], v[n + i, 0], atol=tol)
    # untouched directions keep the initial state's read-out
    for i in range(n, d):
        np.testing.assert_allclose(S.T @ keys[i], S0[0, 0].T @ keys[i], atol=tol)


def pin_pure_decay(orc):
    """beta = 0: S_t = Diag(exp(sum_{s<=t} g_s)) S_0, o_t = S_t^T q_t; S_0 = 0 gives o == 0 exactly."""
    q, k, v, g, beta, S0 = tiny_case(5, T=7, dk=6, dv=3)
    beta = np.zeros_like(beta)
    res = _run(orc, q, k, v, g, beta, S0, scale=1.3)
    G = np.cumsum(g.astype(np.float64), axis=0)  # [T, H, dk]
    for h in range(q.shape[1]):
        for t in range(q.shape[0]):
            St = np.exp(G[t, h])[:, None] * S0[0, h]
            np.testing.assert_allclose(res["o"][t, h], 1.3 * St.T @ q[t, h].astype(np.float64),
                                       rtol=_tol(orc) * 10, atol=_tol(orc))
        np.testing.assert_allclose(res["final"][0, h], np.exp(G[-1, h])[:, None] * S0[0, h],
                                   rtol=_tol(orc) * 10, atol=_tol(orc))
    res0 = _run(orc, q, k, v, g, beta, None)
    assert np.all(res0["o"] == 0) and np.all(res0["final"] == 0)


def pin_linearity(orc):
    """For fixed q, k, g, beta the map (S_0, V) -> (O, S_T) is linear."""
    q, k, v, g, beta, S0 = tiny_case(7, T=9)
    a = _run(orc, q, k, v, g, beta, S0)
    b = _run(orc, q, k, v, g, beta, S0 * 0)
    c = _run(orc, q, k, np.zeros_like(v), g, beta, S0)
    tol = _tol(orc) * 10
    np.testing.assert_allclose(a["o"], b["o"] + c["o"], atol=tol)
    np.testing.assert_allclose(a["final"], b["final"] + c["final"], atol=tol)
    # scaling V by 2 and S_0 by 2 doubles everything
    d = _run(orc, q, k, v * 2, g, beta, S0 * 2)
    np.testing.assert_allclose(d["o"], 2 * a["o"], atol=tol)


def pin_resume(orc):
    """Stopping anywhere and resuming from the returned state equals the
    continuous run, bit for bit (same arithmetic, same order); interval
    checkpoints equal the final states of the shorter runs."""
    q, k, v, g, beta, S0 = tiny_case(9, T=20, dk=4, dv=6)
    full = _run(orc, q, k, v, g, beta, S0)
    for cut in (1, 5, 16):
        a = _run(orc, q[:cut], k[:cut], v[:cut], g[:cut], beta[:cut], S0)
        b = _run(orc, q[cut:], k[cut:], v[cut:], g[cut:], beta[cut:], a["final"])
        assert np.array_equal(np.concatenate([a["o"], b["o"]]), full["o"])
        assert np.array_equal(b["final"], full["final"])
    res = orc.kda_varlen(q, k, v, g, beta, np.array([0, 20], np.int32), init=S0,
                         ckpt_interval=4)
    assert list(res["ckpt_pos"]) == [4, 8, 12, 16]
    for j, p in enumerate(res["ckpt_pos"]):
        a = _run(orc, q[:p], k[:p], v[:p], g[:p], beta[:p], S0)
        assert np.array_equal(res["ckpt"][j], a["final"][0])


def pin_varlen_independent(orc):
    """Packed sequences do not interact: packing equals separate runs."""
    q, k, v, g, beta, S0 = tiny_case(13, T=15)
    cu = np.array([0, 4, 4, 11, 15], np.int32)
    init = np.stack([S0[0], S0[0] * 2, S0[0] * -1, S0[0] * 0.5])
    has = np.array([1, 1, 0, 1], np.int32)
    res = orc.kda_varlen(q, k, v, g, beta, cu, init=init, has_init=has)
    for s in range(4):
        a, b = cu[s], cu[s + 1]
        ini = init[s:s + 1] if has[s] else None
        one = _run(orc, q[a:b], k[a:b], v[a:b], g[a:b], beta[a:b], ini)
        assert np.array_equal(res["o"][a:b], one["o"])
        assert np.array_equal(res["final"][s], one["final"][0])


def pin_verify(orc):
    """Verify: outputs of all positions equal a plain run; the committed state
    is the state after exactly L tokens; orthonormal-key probe recovers L."""
    d = 16
    r = _rng(21)
    N, Ts, H = 5, 6, 1
    keys = exact_orthonormal_rows(r, d)
    k = np.broadcast_to(keys[:Ts][None, :, None, :], (N, Ts, H, d)).astype(np.float32)
    q = k.copy()
    v = r.standard_normal((N, Ts, H, d)).astype(np.float32)
    g = np.zeros((N, Ts, H, d), np.float32)
    beta = np.ones((N, Ts, H), np.float32)
    S0 = r.standard_normal((N, H, d, d))
    L = np.array([0, 1, 3, 6, 9], np.int32)  # 9 is out of range -> rejected
    res = orc.kda_verify(q, k, v, g, beta, S0, L)
    assert list(res["committed_len"]) == [0, 1, 3, 6, -1]
    tol = 1e-10 if orc.real == np.float64 else 5e-5
    for s in range(N):
        if res["committed_len"][s] < 0:
            assert np.all(np.isnan(res["committed"][s]))
            continue
        S = res["committed"][s, 0]
        for j in range(Ts):
            expect = v[s, j, 0] if j < L[s] else S0[s, 0].T @ keys[j]
            np.testing.assert_allclose(S.T @ keys[j], expect, atol=tol)
    # outputs and commit agree with the varlen recurrence
    q2, k2, v2, g2, b2, _ = tiny_case(23, T=Ts, H=2)
    Q = np.stack([q2] * 3)
    K = np.stack([k2] * 3)
    V = np.stack([v2 * (i + 1) for i in range(3)])
    G = np.stack([g2] * 3)
    B = np.stack([b2] * 3)
    init = r.standard_normal((3, 2, 5, 4))
    Lr = np.array([2, Ts, 4], np.int32)
    vr = orc.kda_verify(Q, K, V, G, B, init, Lr)
    for s in range(3):
        full = _run(orc, Q[s], K[s], V[s], G[s], B[s], init[s:s + 1])
        assert np.array_equal(vr["o"][s], full["o"])
        part = _run(orc, Q[s, :Lr[s]], K[s, :Lr[s]], V[s, :Lr[s]], G[s, :Lr[s]], B[s, :Lr[s]],
                    init[s:s + 1])
        assert np.array_equal(vr["committed"][s], part["final"][0])


def ckpt_closed_form(start, length, interval):
    """Number of multiples of interval strictly inside (start, start+length)."""
    if interval <= 0 or length <= 0:
        return 0
    return (start + length - 1) // interval - start // interval


def pin_ckpt_positions(orc):
    """Checkpoint enumeration: closed-form count, positions are the multiples
    of the interval strictly inside each sequence, in order."""
    r = _rng(31)
    for trial in range(20):
        n = int(r.integers(1, 6))
        lens = r.integers(0, 300, n)
        starts = r.integers(0, 5, n) * 16 + r.integers(0, 2, n) * 7
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        interval = int(r.choice([16, 32, 64, 48]))
        ck_cu, pos = orc.ckpt_enumerate(cu, interval, starts.astype(np.int32))
        for s in range(n):
            cnt = ckpt_closed_form(int(starts[s]), int(lens[s]), interval)
            assert ck_cu[s + 1] - ck_cu[s] == cnt
            expect = [p for p in range(int(starts[s]) + 1, int(starts[s] + lens[s]))
                      if p % interval == 0]
            assert list(pos[ck_cu[s]:ck_cu[s + 1]]) == expect
    # the long workload: 1,048,576 tokens, interval 32,768 -> 31 interior positions
    ck_cu, pos = orc.ckpt_enumerate(np.array([0, 1 << 20], np.int32), 32768)
    assert ck_cu[-1] == 31 and pos[0] == 32768 and pos[-1] == 31 * 32768


def pin_conv(orc):
    """Short convolution: one-hot taps are exact shifts, random weights match
    numpy.convolve, the carried state splits and resumes exactly."""
    r = _rng(41)
    T, C, W = 11, 6, 4
    x = r.standard_normal((T, C)).astype(np.float32)
    st = r.standard_normal((1, C, W - 1)).astype(np.float32)
    cu = np.array([0, T], np.int32)
    for tap in range(W):
        w = np.zeros((C, W), np.float32)
        w[:, tap] = 1
        y, ns = orc.conv_short(x, w, cu, state=st)
        xb = np.concatenate([st[0].T, x], axis=0)  # [W-1+T, C]
        # tap W-1 is the current token; tap j looks back W-1-j tokens
        assert np.array_equal(y, xb[tap:tap + T].astype(y.dtype))
        assert np.array_equal(ns[0], xb[-(W - 1):].T)
    w = r.uniform(-0.5, 0.5, (C, W)).astype(np.float32)
    bias = r.standard_normal(C).astype(np.float32)
    for act in (0, 1):
        y, ns = orc.conv_short(x, w, cu, state=st, bias=bias, act=act)
        yb, nb = bruteforce.conv_form(x, w, st[0], bias=bias, act=act)
        np.testing.assert_allclose(y, yb, rtol=_tol(orc) * 10, atol=_tol(orc) * 10)
        assert np.array_equal(ns[0], nb)
    # split and resume
    y_full, ns_full = orc.conv_short(x, w, cu, state=st)
    cut = 5
    y1, s1 = orc.conv_short(x[:cut], w, np.array([0, cut], np.int32), state=st)
    y2, s2 = orc.conv_short(x[cut:], w, np.array([0, T - cut], np.int32),
                            state=s1.astype(np.float32))
    assert np.array_equal(np.concatenate([y1, y2]), y_full)
    assert np.array_equal(s2, ns_full)
    # advance_len: state after only the first a tokens
    for a in (0, 1, 2, 7):
        _, sa = orc.conv_short(x, w, cu, state=st, advance_len=np.array([a], np.int32))
        _, sb = orc.conv_short(x[:a], w, np.array([0, a], np.int32), state=st)
        assert np.array_equal(sa, sb)


def decode_conv_case(seed, N=3, H=2, d=5, W=4):
    r = _rng(seed)
    C = 3 * H * d
    x = r.standard_normal((N, C)).astype(np.float32)
    w = r.uniform(-0.5, 0.5, (C, W)).astype(np.float32)
    bias = (0.1 * r.standard_normal(C)).astype(np.float32)
    cst = r.standard_normal((N, C, W - 1)).astype(np.float32)
    g = (-np.log1p(np.exp(-r.standard_normal((N, H, d))))).astype(np.float32)
    beta = (1 / (1 + np.exp(-r.standard_normal((N, H))))).astype(np.float32)
    S0 = r.standard_normal((N, H, d, d)) * 0.5
    return x, w, bias, cst, g, beta, S0


def pin_decode_conv(orc):
    """Fused decode step: brute force with every sum written out; with the
    current-token tap alone and no activation / normalisation it is the plain
    decode step on the raw projections; with normalisation, positive scalings
    of the q and k projections change nothing; the conv state advances by the
    token.  The composed oracle hands q, k, v to the recurrence as float32
    (rounding ~6e-8 relative), hence the 1e-6 floor on the tolerance."""
    tol = max(_tol(orc) * 10, 1e-6)
    H, d, W = 2, 5, 4
    for seed, act, norm in ((51, 1, 1), (52, 0, 1), (53, 1, 0)):
        x, w, bias, cst, g, beta, S0 = decode_conv_case(seed, H=H, d=d, W=W)
        res = orc.kda_decode_conv(x, w, g, beta, S0, cst, H=H, d=d, bias=bias, act=act,
                                  qk_l2norm=norm, scale=0.7)
        for s in range(x.shape[0]):
            ob, Sb = bruteforce.decode_conv_form(x[s], w, g[s], beta[s], S0[s], cst[s], H, d,
                                                 bias=bias, act=act, qk_l2norm=norm, scale=0.7)
            np.testing.assert_allclose(res["o"][s], ob, rtol=tol, atol=tol)
            np.testing.assert_allclose(res["state"][s], Sb, rtol=tol, atol=tol)
            # the conv state is the history shifted by one token
            assert np.array_equal(res["conv_state"][s][:, :-1], cst[s][:, 1:])
            assert np.array_equal(res["conv_state"][s][:, -1], x[s])
    # current-token tap only: q, k, v are the raw projections
    x, w, bias, cst, g, beta, S0 = decode_conv_case(54, H=H, d=d, W=W)
    w1 = np.zeros_like(w)
    w1[:, W - 1] = 1
    res = orc.kda_decode_conv(x, w1, g, beta, S0, cst, H=H, d=d, act=0, qk_l2norm=0)
    N = x.shape[0]
    xr = x.reshape(N, 3, H, d)
    ref = orc.kda_verify(xr[:, 0][:, None], xr[:, 1][:, None], xr[:, 2][:, None], g[:, None],
                         beta[:, None], S0)
    np.testing.assert_allclose(res["o"], ref["o"][:, 0], rtol=tol, atol=tol)
    np.testing.assert_allclose(res["state"], ref["committed"], rtol=tol, atol=tol)
    # normalisation: the q and k blocks of x scaled by positive constants
    # (linear conv, no activation, no bias, eps = 0) leave everything unchanged
    a = orc.kda_decode_conv(x, w, g, beta, S0, cst, H=H, d=d, act=0, qk_l2norm=1, norm_eps=0.0)
    xs = x.copy().reshape(N, 3, H * d)
    cs = cst.copy().reshape(N, 3, H * d, W - 1)
    xs[:, 0] *= 4.0
    cs[:, 0] *= 4.0
    xs[:, 1] *= 0.25
    cs[:, 1] *= 0.25
    b = orc.kda_decode_conv(xs.reshape(N, -1), w, g, beta, S0, cs.reshape(N, -1, W - 1), H=H, d=d,
                            act=0, qk_l2norm=1, norm_eps=0.0)
    np.testing.assert_allclose(a["o"], b["o"], rtol=tol, atol=tol)
    np.testing.assert_allclose(a["state"], b["state"], rtol=tol, atol=tol)


def pin_verify_conv(orc):
    """Fused verify: with Ts = 1 it is the fused decode step; stepping the
    fused decode step token by token gives every output and, after L steps,
    the committed state and conv history; a rejected length commits
    nothing."""
    tol = max(_tol(orc) * 10, 1e-6)
    r = _rng(61)
    N, Ts, H, d, W = 3, 4, 2, 5, 4
    C = 3 * H * d
    x = r.standard_normal((N, Ts, C)).astype(np.float32)
    w = r.uniform(-0.5, 0.5, (C, W)).astype(np.float32)
    bias = (0.1 * r.standard_normal(C)).astype(np.float32)
    cst = r.standard_normal((N, C, W - 1)).astype(np.float32)
    g = (-np.log1p(np.exp(-r.standard_normal((N, Ts, H, d))))).astype(np.float32)
    beta = (1 / (1 + np.exp(-r.standard_normal((N, Ts, H))))).astype(np.float32)
    S0 = r.standard_normal((N, H, d, d)) * 0.5
    L = np.array([2, 4, 7], np.int32)   # the third is rejected
    res = orc.kda_verify_conv(x, w, g, beta, S0, cst, L, H=H, d=d, bias=bias, act=1, qk_l2norm=1,
                              scale=0.8)
    one = orc.kda_verify_conv(x[:, :1], w, g[:, :1], beta[:, :1], S0, cst, None, H=H, d=d, bias=bias,
                              act=1, qk_l2norm=1, scale=0.8)
    dec = orc.kda_decode_conv(x[:, 0], w, g[:, 0], beta[:, 0], S0, cst, H=H, d=d, bias=bias, act=1,
                              qk_l2norm=1, scale=0.8)
    np.testing.assert_allclose(one["o"][:, 0], dec["o"], rtol=tol, atol=tol)
    np.testing.assert_allclose(one["committed"], dec["state"], rtol=tol, atol=tol)
    assert np.array_equal(one["conv_state"], dec["conv_state"].astype(np.float64))
    # token by token through the fused decode step
    S = S0.copy()
    hist = cst.copy()
    for t in range(Ts):
        step = orc.kda_decode_conv(x[:, t], w, g[:, t], beta[:, t], S, hist, H=H, d=d, bias=bias, act=1,
                                   qk_l2norm=1, scale=0.8)
        np.testing.assert_allclose(res["o"][:, t], step["o"], rtol=tol, atol=tol)
        S = step["state"]
        hist = step["conv_state"].astype(np.float32)
        for s in range(N):
            if L[s] == t + 1:
                np.testing.assert_allclose(res["committed"][s], S[s], rtol=tol, atol=tol)
                assert np.array_equal(res["conv_state"][s], hist[s].astype(np.float64))
    assert res["committed_len"][2] == -1
    assert np.all(np.isnan(res["committed"][2])) and np.all(np.isnan(res["conv_state"][2]))


def pin_output_gate(orc):
    """Gated RMS norm of the fused step's output, by its properties rather
    than its formula: with unit weight and an open gate (sigmoid = 1) the
    output of every (token, head) has root mean square 1 over its channels
    (a sum instead of a mean, or a missing root, fails); positive scalings of
    one head's output change no output (the norm axis is per head: a norm
    over all heads fails); a gate of zero halves the output (sigmoid(0) =
    1/2); a one-hot weight keeps one channel; a zero output stays zero with
    eps > 0.  Then, wired into the fused decode step: its gated output times
    the root mean square of its ungated output is the ungated output (the
    gate acts on o, not on q, k or v)."""
    import oracle as O
    r = _rng(71)
    N, H, d = 4, 3, 8
    o = r.standard_normal((N, H, d)) * r.uniform(0.1, 5.0, (N, H, 1))
    w1 = np.ones(d, np.float32)
    zo = np.full((N, H, d), 40.0, np.float32)        # sigmoid(40) = 1 - 4e-18
    y = O.gated_rmsnorm(o, zo, w1, eps=0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, rtol=1e-12)
    np.testing.assert_allclose(y * np.sqrt(np.mean(o * o, axis=-1, keepdims=True)), o, rtol=1e-12)
    z = r.standard_normal((N, H, d)).astype(np.float32)
    wr = r.uniform(0.5, 1.5, d).astype(np.float32)
    a = O.gated_rmsnorm(o, z, wr, eps=0.0)
    o2 = o.copy()
    o2[1, 2] *= 7.5
    o2[3, 0] *= 0.01
    np.testing.assert_allclose(O.gated_rmsnorm(o2, z, wr, eps=0.0), a, rtol=1e-12, atol=1e-14)
    half = O.gated_rmsnorm(o, np.zeros((N, H, d), np.float32), w1, eps=0.0)
    np.testing.assert_allclose(2.0 * half, O.gated_rmsnorm(o, zo, w1, eps=0.0), rtol=1e-12)
    e3 = np.zeros(d, np.float32)
    e3[3] = 1.0
    y3 = O.gated_rmsnorm(o, z, e3, eps=0.0)
    assert np.all(y3[..., np.arange(d) != 3] == 0.0) and np.all(y3[..., 3] != 0.0)
    assert np.all(O.gated_rmsnorm(np.zeros((N, H, d)), z, wr, eps=1e-6) == 0.0)
    # in the fused decode step
    tol = max(_tol(orc) * 10, 1e-6)
    x, w, bias, cst, g, beta, S0 = decode_conv_case(72, N=3, H=2, d=5)
    plain = orc.kda_decode_conv(x, w, g, beta, S0, cst, H=2, d=5, bias=bias, act=1, qk_l2norm=1)
    gated = orc.kda_decode_conv(x, w, g, beta, S0, cst, H=2, d=5, bias=bias, act=1, qk_l2norm=1,
                                out_gate=np.full((3, 2, 5), 40.0, np.float32),
                                norm_weight=np.ones(5, np.float32), out_norm_eps=0.0)
    rms = np.sqrt(np.mean(plain["o"] ** 2, axis=-1, keepdims=True))
    np.testing.assert_allclose(gated["o"] * rms, plain["o"], rtol=tol, atol=tol)
    assert np.array_equal(gated["state"], plain["state"])


def prefill_conv_case(seed, lengths=(6, 1, 9), H=2, d=5, W=4):
    """A packed batch of raw projections: sequence 0 with conv history and
    an initial state, sequence 1 (one token) with history only, sequence 2
    with neither."""
    r = _rng(seed)
    C = 3 * H * d
    T = sum(lengths)
    N = len(lengths)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    x = r.standard_normal((T, C)).astype(np.float32)
    w = r.uniform(-0.5, 0.5, (C, W)).astype(np.float32)
    bias = (0.1 * r.standard_normal(C)).astype(np.float32)
    cst = r.standard_normal((N, C, W - 1)).astype(np.float32)
    has_c = np.array([1, 1, 0][:N], np.int32)
    g = (-np.log1p(np.exp(-r.standard_normal((T, H, d))))).astype(np.float32)
    beta = (1 / (1 + np.exp(-r.standard_normal((T, H))))).astype(np.float32)
    S0 = r.standard_normal((N, H, d, d)) * 0.5
    has_s = np.array([1, 0, 0][:N], np.int32)
    return x, w, bias, cst, has_c, g, beta, S0, has_s, cu


def pin_prefill_conv(orc):
    """Prefill from raw projections: with the current-token tap alone and no
    activation or normalisation it is the plain prefill of the projections'
    blocks, bit for bit; stepped token by token through the fused decode step
    (a separately written composition) it gives every output, the final state
    and the conv history; split at a token and resumed from the carried conv
    history and state it equals the continuous run bit for bit; positive
    scalings of the q and k projections change nothing under normalisation;
    bf16 operands are bf16 values within half a bf16 unit of the unrounded
    ones."""
    tol = max(_tol(orc) * 10, 1e-6)
    H, d, W = 2, 5, 4
    x, w, bias, cst, has_c, g, beta, S0, has_s, cu = prefill_conv_case(81, H=H, d=d, W=W)
    T, C = x.shape
    N = cu.size - 1
    # current-token tap only: the blocks of x are q, k, v
    w1 = np.zeros_like(w)
    w1[:, W - 1] = 1
    a = orc.kda_prefill_conv(x, w1, g, beta, cu, H=H, d=d, act=0, conv_state=cst, has_conv_state=has_c,
                             qk_l2norm=0, operand_dtype="f32", init=S0, has_init=has_s, scale=0.6)
    xb = x.reshape(T, 3, H, d)
    ref = orc.kda_varlen(xb[:, 0], xb[:, 1], xb[:, 2], g, beta, cu, init=S0, has_init=has_s, scale=0.6)
    assert np.array_equal(a["o"], ref["o"]) and np.array_equal(a["final"], ref["final"])
    # the new history: the last W-1 raw inputs of history ++ tokens
    for s in range(N):
        hist = cst[s] if has_c[s] else np.zeros_like(cst[s])
        full = np.concatenate([hist, x[cu[s]:cu[s + 1]].T], axis=1)
        assert np.array_equal(a["conv_state"][s], full[:, -(W - 1):])
    # token by token through the fused decode step
    res = orc.kda_prefill_conv(x, w, g, beta, cu, H=H, d=d, bias=bias, act=1, conv_state=cst,
                               has_conv_state=has_c, qk_l2norm=1, operand_dtype="f32", init=S0,
                               has_init=has_s, scale=0.6)
    for s in range(N):
        S = S0[s:s + 1] if has_s[s] else np.zeros_like(S0[s:s + 1])
        hist = (cst[s:s + 1] if has_c[s] else np.zeros_like(cst[s:s + 1])).astype(np.float32)
        for t in range(cu[s], cu[s + 1]):
            step = orc.kda_decode_conv(x[t:t + 1], w, g[t:t + 1], beta[t:t + 1], S, hist, H=H, d=d,
                                       bias=bias, act=1, qk_l2norm=1, scale=0.6)
            np.testing.assert_allclose(res["o"][t], step["o"][0], rtol=tol, atol=tol)
            S = step["state"]
            hist = step["conv_state"].astype(np.float32)
        np.testing.assert_allclose(res["final"][s], S[0], rtol=tol, atol=tol)
        assert np.array_equal(res["conv_state"][s], hist[0].astype(np.float64))
    # split sequence 2 after 4 tokens and resume
    p = int(cu[2]) + 4
    one = orc.kda_prefill_conv(x[cu[2]:p], w, g[cu[2]:p], beta[cu[2]:p], np.array([0, 4], np.int32), H=H,
                               d=d, bias=bias, act=1, qk_l2norm=1)
    two = orc.kda_prefill_conv(x[p:cu[3]], w, g[p:cu[3]], beta[p:cu[3]],
                               np.array([0, cu[3] - p], np.int32), H=H, d=d, bias=bias, act=1,
                               conv_state=one["conv_state"].astype(np.float32), qk_l2norm=1,
                               init=one["final"], start_pos=np.array([4], np.int32))
    full = orc.kda_prefill_conv(x[cu[2]:cu[3]], w, g[cu[2]:cu[3]], beta[cu[2]:cu[3]],
                                np.array([0, cu[3] - cu[2]], np.int32), H=H, d=d, bias=bias, act=1,
                                qk_l2norm=1)
    assert np.array_equal(np.concatenate([one["o"], two["o"]]), full["o"])
    assert np.array_equal(two["final"], full["final"])
    assert np.array_equal(two["conv_state"], full["conv_state"])
    # the same split through an interval checkpoint of the continuous run:
    # its recurrent state and conv history resume the tail bit for bit
    ck = orc.kda_prefill_conv(x[cu[2]:cu[3]], w, g[cu[2]:cu[3]], beta[cu[2]:cu[3]],
                              np.array([0, cu[3] - cu[2]], np.int32), H=H, d=d, bias=bias, act=1, qk_l2norm=1,
                              ckpt_interval=4)
    assert list(ck["ckpt_pos"]) == [4, 8]
    assert np.array_equal(ck["o"], full["o"]) and np.array_equal(ck["ckpt"][0], one["final"][0])
    assert np.array_equal(ck["conv_ckpt"][0], one["conv_state"][0])
    tail = orc.kda_prefill_conv(x[p:cu[3]], w, g[p:cu[3]], beta[p:cu[3]], np.array([0, cu[3] - p], np.int32),
                                H=H, d=d, bias=bias, act=1, conv_state=ck["conv_ckpt"][0].astype(np.float32)[None],
                                qk_l2norm=1, init=ck["ckpt"][0][None], start_pos=np.array([4], np.int32))
    assert np.array_equal(tail["o"], full["o"][4:]) and np.array_equal(tail["final"], full["final"])
    # a checkpoint inside the first W-1 tokens takes part of its history from
    # the carried one: the raw inputs before position 2 of sequence 0
    c2 = orc.kda_prefill_conv(x[:cu[1]], w, g[:cu[1]], beta[:cu[1]], np.array([0, cu[1]], np.int32), H=H, d=d,
                              act=1, conv_state=cst[:1], qk_l2norm=1, ckpt_interval=2)
    want = np.concatenate([cst[0], x[:2].T], axis=1)[:, -(W - 1):]
    assert list(c2["ckpt_pos"])[:1] == [2] and np.array_equal(c2["conv_ckpt"][0], want)
    # normalisation: positive scalings of the q and k projections (linear
    # conv, no activation, no bias, eps = 0) leave everything unchanged
    b0 = orc.kda_prefill_conv(x, w, g, beta, cu, H=H, d=d, conv_state=cst, has_conv_state=has_c,
                              qk_l2norm=1, norm_eps=0.0, operand_dtype="f32")
    xs = x.copy().reshape(T, 3, H * d)
    cs = cst.copy().reshape(N, 3, H * d, W - 1)
    xs[:, 0] *= 3.0
    cs[:, 0] *= 3.0
    xs[:, 1] *= 0.2
    cs[:, 1] *= 0.2
    b1 = orc.kda_prefill_conv(xs.reshape(T, C), w, g, beta, cu, H=H, d=d, conv_state=cs.reshape(N, C, W - 1),
                              has_conv_state=has_c, qk_l2norm=1, norm_eps=0.0, operand_dtype="f32")
    np.testing.assert_allclose(b1["o"], b0["o"], rtol=tol, atol=tol)
    np.testing.assert_allclose(b1["final"], b0["final"], rtol=tol, atol=tol)
    # bf16 operands
    r16 = orc.kda_prefill_conv(x, w, g, beta, cu, H=H, d=d, bias=bias, act=1, conv_state=cst,
                               has_conv_state=has_c, qk_l2norm=1, operand_dtype="bf16")
    for name in ("q", "k", "v"):
        o16, o32 = r16[name].astype(np.float64), res[name].astype(np.float64)
        hi = (r16[name].view(np.uint32) & 0xFFFF0000).view(np.float32)
        assert np.array_equal(r16[name], hi), f"{name}: not bf16 values"
        # nearest: within half a unit in the last place of bf16 (8
        # significant bits) at the operand's binade
        half_ulp = np.ldexp(1.0, np.floor(np.log2(np.abs(o32) + 1e-300)).astype(int) - 8)
        assert np.all(np.abs(o16 - o32) <= half_ulp), name


ALL_PINS = [pin_bruteforce, pin_readback, pin_pure_decay, pin_linearity, pin_resume,
            pin_varlen_independent, pin_verify, pin_ckpt_positions, pin_conv, pin_decode_conv,
            pin_verify_conv, pin_output_gate, pin_prefill_conv]
