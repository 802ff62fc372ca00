"""GPU parity of kda_decode_conv (the decode step with the short
convolution, optional SiLU and q/k L2 normalisation fused in) against the
oracle's composed step, through the C ABI."""

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


def _case(N, H, d, W, dtype, seed):
    """Inputs in the distribution of the batched decode workload: conv
    weights U(-1/sqrt(W), 1/sqrt(W)), history and token N(0, 1), gates
    logsigmoid(N(0, 1)), beta sigmoid(N(0, 1)), states N(0, 0.1)."""
    wl = make_workload(1, n_seq=N, H=H, d=d, seed=seed)
    gen = torch.Generator().manual_seed(1000 + seed)
    C = 3 * H * d
    w, st, x = draw_conv(gen, N, C, W, N, dtype, torch.device("cpu"))
    bias = (0.1 * torch.randn(C, generator=gen)).to(dtype)
    g, b = wl.g.to(dtype), wl.beta.to(dtype)
    return x, w, bias, st, g, b, wl.init_states


def _run(dev, x, w, bias, cst, g, b, init, *, act, norm, out_dtype, conv_src, in_place=False,
         scale=1.0, gate=None, gw=None):
    N, C = x.shape
    H, d = g.shape[1], g.shape[2]
    W = w.shape[1]
    # pools: history / state of sequence s in slot s; results to slot N + s
    # (or back to slot s in place)
    cpool = torch.zeros(2 * N, C, W - 1, dtype=x.dtype, device=dev)
    cpool[:N] = cst.to(dev)
    pool = torch.zeros(2 * N, H, d, d, device=dev)
    pool[:N] = init.to(dev)
    src = torch.arange(N, dtype=torch.int32, device=dev)
    dst = src if in_place else src + N
    csrc = torch.tensor(conv_src, dtype=torch.int32, device=dev)
    cdst = src if in_place else src + N
    o = torch.empty(N, H, d, dtype=out_dtype, device=dev)
    K.kda_decode_conv(x.to(dev), w.to(dev), cpool, csrc, cdst, g.to(dev), b.to(dev), o, pool, src, dst,
                      conv_bias=None if bias is None else bias.to(dev), act=act, qk_l2norm=norm,
                      scale=scale, out_gate=gate, out_norm_weight=gw)
    torch.cuda.synchronize()
    return o, pool[dst.long()], cpool[cdst.long()]


def _gate(gen, shape, dtype, d):
    """Output gate logits N(0, 1) and norm weights 1 + 0.1 N(0, 1)."""
    z = torch.randn(*shape, generator=gen).to(dtype)
    wt = (1.0 + 0.1 * torch.randn(d, generator=gen)).to(dtype)
    return z, wt


def _gated_bf16_max_abs(ref):
    """Normalised outputs reach |o| ~ 4, where one bf16 rounding alone is up
    to 2^-9 |o|: the element bound scales with the largest output (2^-7 of
    it, one rounding plus the error carried in from the unnormalised o)."""
    return max(U.MAX_ABS_TOL, 2.0 ** -7 * float(np.abs(ref).max()))


def _reference(orc, x, w, bias, cst, g, b, init, conv_src, *, act, norm, scale=1.0, gate=None, gw=None):
    N = x.shape[0]
    H, d = g.shape[1], g.shape[2]
    hist = cst.float().numpy().copy()
    for s in range(N):
        if conv_src[s] < 0:
            hist[s] = 0.0
    return orc.kda_decode_conv(x, w, g, b, init.double().numpy(), hist, H=H, d=d, bias=bias,
                               act=act, qk_l2norm=norm, scale=scale, out_gate=gate, norm_weight=gw), hist


def _check_conv_state(got, x, hist):
    """The advanced history is a copy of input values: bit-exact."""
    got = got.to("cpu", torch.float32).numpy()
    want = np.concatenate([hist[:, :, 1:], x.float().numpy()[:, :, None]], axis=2)
    assert np.array_equal(got, want.astype(np.float32))


@pytest.mark.parametrize("act,norm", [(1, 1), (0, 1), (1, 0)])
def test_decode_conv_batched_128(dev, oracle64, act, norm):
    """128 sequences x 1 token, H=16, d=128, W=4, bf16; odd sequences start
    from an empty conv history; results copied on write to fresh slots."""
    U.say(f"decode_conv batched 128 x H16 x d128 act={act} norm={norm}")
    N, H, d, W = 128, 16, 128, 4
    x, w, bias, cst, g, b, init = _case(N, H, d, W, torch.bfloat16, seed=11)
    if not norm:
        # without normalisation |k| ~ 6.5 at this scale, so beta |k|^2 >> 1 and
        # the step amplifies the state; shrink the projections to |k| ~ 1
        x = (x.float() * 0.15).to(torch.bfloat16)
        cst = (cst.float() * 0.15).to(torch.bfloat16)
        bias = (bias.float() * 0.15).to(torch.bfloat16)
    conv_src = [s if s % 2 == 0 else -1 for s in range(N)]
    o, st, cs = _run(dev, x, w, bias, cst, g, b, init, act=act, norm=norm,
                     out_dtype=torch.bfloat16, conv_src=conv_src)
    ref, hist = _reference(oracle64, x, w, bias, cst, g, b, init, conv_src, act=act, norm=norm)
    U.assert_close("o", U.to_np(o), ref["o"])
    U.assert_close("state", U.to_np(st), ref["state"])
    _check_conv_state(cs, x, hist)


@pytest.mark.parametrize("W", [2, 3])
def test_decode_conv_widths_in_place(dev, oracle64, W):
    """Conv widths 2 and 3, slots updated in place, d=64, fp32 outputs."""
    U.say(f"decode_conv W={W} in place d64")
    N, H, d = 24, 4, 64
    x, w, bias, cst, g, b, init = _case(N, H, d, W, torch.bfloat16, seed=20 + W)
    conv_src = list(range(N))
    o, st, cs = _run(dev, x, w, bias, cst, g, b, init, act=1, norm=1, out_dtype=torch.float32,
                     conv_src=conv_src, in_place=True, scale=0.5)
    ref, hist = _reference(oracle64, x, w, bias, cst, g, b, init, conv_src, act=1, norm=1, scale=0.5)
    U.assert_close("o", U.to_np(o), ref["o"])
    U.assert_close("state", U.to_np(st), ref["state"])
    _check_conv_state(cs, x, hist)


@pytest.mark.parametrize("d", [16, 32, 128])
def test_decode_conv_fp32_small(dev, oracle64, d):
    """fp32 inputs and outputs (small head sizes, and d = 128 with one
    4-wave workgroup per head and 16-byte conv units): the only roundings
    left are the fp32 accumulation orders."""
    U.say(f"decode_conv fp32 d={d}")
    N, H, W = 9, 3, 4
    x, w, bias, cst, g, b, init = _case(N, H, d, W, torch.float32, seed=30 + d)
    conv_src = [s if s % 3 else -1 for s in range(N)]
    o, st, cs = _run(dev, x, w, bias, cst, g, b, init, act=1, norm=1, out_dtype=torch.float32,
                     conv_src=conv_src)
    ref, hist = _reference(oracle64, x, w, bias, cst, g, b, init, conv_src, act=1, norm=1)
    U.assert_close("o", U.to_np(o), ref["o"], rel=1e-5, mx=1e-5)
    U.assert_close("state", U.to_np(st), ref["state"], rel=1e-5, mx=1e-5)
    _check_conv_state(cs, x, hist)


@pytest.mark.parametrize("W", [2, 3])
def test_decode_conv_d128_widths_absent_slots(dev, oracle64, W):
    """d = 128, bf16 inputs, fp32 outputs, conv widths 2 and 3 with a bias
    (W = 3 also with the gated output norm): absent state sources start from
    zero, absent state destinations store nothing (the slot keeps its
    sentinel), absent conv histories read zeros, results copied on write."""
    U.say(f"decode_conv d128 W={W} absent slots")
    N, H, d = 12, 4, 128
    x, w, bias, cst, g, b, init = _case(N, H, d, W, torch.bfloat16, seed=70 + W)
    C = 3 * H * d
    ssrc = [s if s % 3 != 1 else -1 for s in range(N)]
    sdst = [N + s if s % 4 != 2 else -1 for s in range(N)]
    csrc = [s if s % 2 == 0 else -1 for s in range(N)]
    gate = gw = None
    if W == 3:
        gate, gw = _gate(torch.Generator().manual_seed(470), (N, H, d), torch.bfloat16, d)
    cpool = torch.zeros(2 * N, C, W - 1, dtype=torch.bfloat16, device=dev)
    cpool[:N] = cst.to(dev)
    pool = torch.zeros(2 * N, H, d, d, device=dev)
    pool[:N] = init.to(dev)
    pool[N:] = 7.0
    before = pool.clone()

    def i32(v):
        return torch.tensor(v, dtype=torch.int32, device=dev)

    o = torch.empty(N, H, d, device=dev)
    K.kda_decode_conv(x.to(dev), w.to(dev), cpool, i32(csrc), i32([N + s for s in range(N)]), g.to(dev),
                      b.to(dev), o, pool, i32(ssrc), i32(sdst), conv_bias=bias.to(dev), act=1, qk_l2norm=1,
                      out_gate=None if gate is None else gate.to(dev),
                      out_norm_weight=None if gw is None else gw.to(dev))
    torch.cuda.synchronize()
    init0 = init.clone()
    for s in range(N):
        if ssrc[s] < 0:
            init0[s] = 0.0
    ref, hist = _reference(oracle64, x, w, bias, cst, g, b, init0, csrc, act=1, norm=1, gate=gate, gw=gw)
    U.assert_close("o", U.to_np(o), ref["o"], rel=1e-5, mx=1e-4)
    stored = [s for s in range(N) if sdst[s] >= 0]
    U.assert_close("state", U.to_np(pool[[N + s for s in stored]]), ref["state"][stored], rel=1e-5, mx=1e-4)
    for s in range(N):
        if sdst[s] < 0:
            assert torch.equal(pool[N + s], before[N + s]), "absent destination written"
    assert torch.equal(pool[:N], before[:N]), "source states modified"
    _check_conv_state(cpool[N:], x, hist)


def test_decode_conv_gated_norm_128(dev, oracle64):
    """The output passes the gated RMS norm: 128 sequences x 1 token, H=16,
    d=128, W=4, bf16 gate and weight, bf16 outputs."""
    U.say("decode_conv gated norm 128 x H16 x d128")
    N, H, d, W = 128, 16, 128, 4
    x, w, bias, cst, g, b, init = _case(N, H, d, W, torch.bfloat16, seed=12)
    z, wt = _gate(torch.Generator().manual_seed(312), (N, H, d), torch.bfloat16, d)
    conv_src = list(range(N))
    o, st, cs = _run(dev, x, w, bias, cst, g, b, init, act=1, norm=1, out_dtype=torch.bfloat16,
                     conv_src=conv_src, gate=z.to(dev), gw=wt.to(dev))
    ref, hist = _reference(oracle64, x, w, bias, cst, g, b, init, conv_src, act=1, norm=1, gate=z, gw=wt)
    U.assert_close("o", U.to_np(o), ref["o"], mx=_gated_bf16_max_abs(ref["o"]))
    U.assert_close("state", U.to_np(st), ref["state"])
    _check_conv_state(cs, x, hist)


@pytest.mark.parametrize("d", [16, 32, 64, 128])
def test_decode_conv_gated_norm_fp32(dev, oracle64, d):
    """Gated RMS norm with fp32 inputs and outputs, every head size, the gate
    read with a padded token stride (a view into a wider buffer)."""
    U.say(f"decode_conv gated norm fp32 d={d}")
    N, H, W = 7, 3, 3
    x, w, bias, cst, g, b, init = _case(N, H, d, W, torch.float32, seed=60 + d)
    z, wt = _gate(torch.Generator().manual_seed(360 + d), (N, H, d), torch.float32, d)
    wide = torch.zeros(N, H * d + 8, device=dev)
    wide[:, :H * d] = z.reshape(N, H * d).to(dev)
    zv = wide[:, :H * d].view(N, H, d)
    conv_src = [s if s % 3 else -1 for s in range(N)]
    o, st, cs = _run(dev, x, w, bias, cst, g, b, init, act=1, norm=1, out_dtype=torch.float32,
                     conv_src=conv_src, gate=zv, gw=wt.to(dev), scale=d ** -0.5)
    ref, hist = _reference(oracle64, x, w, bias, cst, g, b, init, conv_src, act=1, norm=1, gate=z, gw=wt,
                           scale=d ** -0.5)
    U.assert_close("o", U.to_np(o), ref["o"], rel=1e-5, mx=1e-5)
    U.assert_close("state", U.to_np(st), ref["state"], rel=1e-5, mx=1e-5)


def _verify_case(N, Ts, H, d, W, dtype, seed):
    wl = make_workload(4, n_seq=N, H=H, d=d, T=max(Ts, 8), seed=seed)
    gen = torch.Generator().manual_seed(2000 + seed)
    C = 3 * H * d
    w, st, x = draw_conv(gen, N * Ts, C, W, N, dtype, torch.device("cpu"))
    x = x.reshape(N, Ts, C)
    return x, w, st, wl.g[:, :Ts].to(dtype).contiguous(), wl.beta[:, :Ts].to(dtype).contiguous(), wl.init_states


def _run_verify(dev, x, w, cst, g, b, init, L, *, out_dtype, with_o=True, commit=True, conv_src=None,
                act=1, norm=1, bias=None, state_src=None, gate=None, gw=None):
    N, Ts, C = x.shape
    H, d = g.shape[2], g.shape[3]
    W = w.shape[1]
    cpool = torch.zeros(2 * N, C, W - 1, dtype=x.dtype, device=dev)
    cpool[:N] = cst.to(dev)
    pool = torch.zeros(2 * N, H, d, d, device=dev)
    pool[:N] = init.to(dev)
    pool[N:] = float("nan")           # destinations hold NaN until written
    cpool[N:] = float("nan")
    src = torch.tensor(state_src if state_src is not None else list(range(N)), dtype=torch.int32, device=dev)
    dst = torch.arange(N, dtype=torch.int32, device=dev) + N
    csrc = torch.tensor(conv_src if conv_src is not None else list(range(N)), dtype=torch.int32, device=dev)
    o = torch.empty(N, Ts, H, d, dtype=out_dtype, device=dev) if with_o else None
    acc = torch.tensor(L, dtype=torch.int32, device=dev) if commit else None
    clen = torch.full((N,), -7, dtype=torch.int32, device=dev)
    K.kda_verify_conv(x.to(dev), w.to(dev), cpool, csrc, dst, g.to(dev), b.to(dev), pool, src, dst, o=o,
                      accepted_len=acc, committed_len_out=clen if commit else None, act=act, qk_l2norm=norm,
                      conv_bias=None if bias is None else bias.to(dev), out_gate=gate, out_norm_weight=gw)
    torch.cuda.synchronize()
    return o, pool[N:], cpool[N:], clen, pool[:N], cpool[:N]


def _verify_reference(orc, x, w, cst, g, b, init, L, conv_src, act=1, norm=1, bias=None, state_src=None,
                      gate=None, gw=None):
    N = x.shape[0]
    H, d = g.shape[2], g.shape[3]
    hist = cst.float().numpy().copy()
    for s in range(N):
        if conv_src[s] < 0:
            hist[s] = 0.0
    S0 = init.double().numpy().copy()
    if state_src is not None:
        for s in range(N):
            if state_src[s] < 0:
                S0[s] = 0.0
    return orc.kda_verify_conv(x, w, g, b, S0, hist, L, H=H, d=d, act=act, qk_l2norm=norm,
                               bias=None if bias is None else bias.float().numpy(), out_gate=gate,
                               norm_weight=gw), hist


def test_verify_conv_batched_128x8(dev, oracle64):
    """128 sequences x 8 tokens, H=16, d=128, W=4, bf16: outputs for all
    positions, state and conv history committed at L ~ U{1..8} (one rejected
    length, one L = 0), odd sequences without conv history."""
    U.say("verify_conv batched 128 x 8 x H16 x d128")
    N, Ts, H, d, W = 128, 8, 16, 128, 4
    x, w, cst, g, b, init = _verify_case(N, Ts, H, d, W, torch.bfloat16, seed=41)
    gen = torch.Generator().manual_seed(7)
    L = torch.randint(1, Ts + 1, (N,), generator=gen).tolist()
    L[3], L[10] = 9, 0
    conv_src = [s if s % 2 == 0 else -1 for s in range(N)]
    o, st, cs, clen, st_src, cs_src = _run_verify(dev, x, w, cst, g, b, init, L, out_dtype=torch.bfloat16,
                                                  conv_src=conv_src)
    ref, hist = _verify_reference(oracle64, x, w, cst, g, b, init, L, conv_src)
    U.assert_close("o", U.to_np(o), ref["o"])
    ok = np.array([0 <= v <= Ts for v in L])
    assert clen.cpu().tolist() == [v if 0 <= v <= Ts else -1 for v in L]
    U.assert_close("committed", U.to_np(st)[ok], ref["committed"][ok])
    assert torch.isnan(st[3]).all() and torch.isnan(cs[3]).all()   # rejected: not written
    got = cs.to("cpu", torch.float32).numpy()[ok]
    assert np.array_equal(got, ref["conv_state"][ok].astype(np.float32))
    # sources are never written
    assert torch.equal(st_src.cpu(), init)
    assert torch.equal(cs_src.cpu(), cst)


def test_verify_conv_modes(dev, oracle64):
    """Outputs-only writes no state; commit-only equals the fused call's
    commit."""
    U.say("verify_conv modes")
    N, Ts, H, d, W = 16, 5, 4, 64, 3
    x, w, cst, g, b, init = _verify_case(N, Ts, H, d, W, torch.bfloat16, seed=43)
    L = [(i % (Ts + 1)) for i in range(N)]
    ref, _ = _verify_reference(oracle64, x, w, cst, g, b, init, L, list(range(N)))
    o, st, cs, _, _, _ = _run_verify(dev, x, w, cst, g, b, init, L, out_dtype=torch.float32, commit=False)
    U.assert_close("o (outputs only)", U.to_np(o), ref["o"])
    assert torch.isnan(st).all() and torch.isnan(cs).all()
    _, st2, cs2, clen, _, _ = _run_verify(dev, x, w, cst, g, b, init, L, out_dtype=torch.float32, with_o=False)
    U.assert_close("committed (commit only)", U.to_np(st2), ref["committed"])
    assert np.array_equal(cs2.to("cpu", torch.float32).numpy(), ref["conv_state"].astype(np.float32))
    assert clen.cpu().tolist() == L


@pytest.mark.parametrize("d,W", [(16, 2), (32, 4)])
def test_verify_conv_fp32_small(dev, oracle64, d, W):
    """fp32 inputs and outputs, small heads, T_spec = 3."""
    U.say(f"verify_conv fp32 d={d} W={W}")
    N, Ts, H = 6, 3, 2
    x, w, cst, g, b, init = _verify_case(N, Ts, H, d, W, torch.float32, seed=50 + d)
    L = [3, 1, 2, 0, 3, 2]
    o, st, cs, clen, _, _ = _run_verify(dev, x, w, cst, g, b, init, L, out_dtype=torch.float32)
    ref, _ = _verify_reference(oracle64, x, w, cst, g, b, init, L, list(range(N)))
    U.assert_close("o", U.to_np(o), ref["o"], rel=1e-5, mx=1e-5)
    U.assert_close("committed", U.to_np(st), ref["committed"], rel=1e-5, mx=1e-5)
    assert np.array_equal(cs.cpu().numpy(), ref["conv_state"].astype(np.float32))


def test_verify_conv_16_tokens_bias_absent_sources(dev, oracle64):
    """The longest window (16 tokens), H=4, d=128, W=4, bf16, with a conv
    bias: every conv input unit of a workgroup is staged (the most units per
    thread); sequences without a state source start from zero, sequences
    without conv history from a zero history; L over {0..16} plus one
    rejected length."""
    U.say("verify_conv 32 x 16 x H4 x d128, bias, absent sources")
    N, Ts, H, d, W = 32, 16, 4, 128, 4
    x, w, cst, g, b, init = _verify_case(N, Ts, H, d, W, torch.bfloat16, seed=61)
    bias = (torch.rand(3 * H * d, generator=torch.Generator().manual_seed(62)) - 0.5).to(torch.bfloat16)
    gen = torch.Generator().manual_seed(63)
    L = torch.randint(0, Ts + 1, (N,), generator=gen).tolist()
    L[5] = Ts + 1
    conv_src = [s if s % 3 else -1 for s in range(N)]
    state_src = [s if s % 4 != 1 else -1 for s in range(N)]
    o, st, cs, clen, st_src, cs_src = _run_verify(dev, x, w, cst, g, b, init, L, out_dtype=torch.bfloat16,
                                                  conv_src=conv_src, bias=bias, state_src=state_src)
    ref, _ = _verify_reference(oracle64, x, w, cst, g, b, init, L, conv_src, bias=bias, state_src=state_src)
    U.assert_close("o", U.to_np(o), ref["o"])
    ok = np.array([0 <= v <= Ts for v in L])
    assert clen.cpu().tolist() == [v if 0 <= v <= Ts else -1 for v in L]
    U.assert_close("committed", U.to_np(st)[ok], ref["committed"][ok])
    assert torch.isnan(st[5]).all() and torch.isnan(cs[5]).all()
    assert np.array_equal(cs.to("cpu", torch.float32).numpy()[ok], ref["conv_state"][ok].astype(np.float32))
    assert torch.equal(st_src.cpu(), init) and torch.equal(cs_src.cpu(), cst)


@pytest.mark.parametrize("W,Ts", [(2, 5), (3, 12)])
def test_verify_conv_matrix_core_widths_fp32_outputs(dev, oracle64, W, Ts):
    """The matrix-core fused verify (d = 128, bf16 inputs) at conv widths 2
    and 3, both window buckets (5 and 12 tokens), with a conv bias, without
    SiLU and without the q/k norm, fp32 outputs: outputs and committed states
    at fp32-grade tolerance, the conv history bit for bit."""
    U.say(f"verify_conv bf16 d128 W={W} T={Ts} fp32 out")
    N, H, d = 6, 2, 128
    x, w, cst, g, b, init = _verify_case(N, Ts, H, d, W, torch.bfloat16, seed=80 + W)
    bias = (torch.rand(3 * H * d, generator=torch.Generator().manual_seed(81 + W)) - 0.5).to(torch.bfloat16)
    L = [Ts, 0, 1, Ts // 2, Ts + 1, 3]
    conv_src = [0, -1, 2, 3, 4, 5]
    o, st, cs, clen, _, _ = _run_verify(dev, x, w, cst, g, b, init, L, out_dtype=torch.float32,
                                        conv_src=conv_src, act=0, norm=0, bias=bias)
    ref, _ = _verify_reference(oracle64, x, w, cst, g, b, init, L, conv_src, act=0, norm=0, bias=bias)
    ok = np.array([0 <= v <= Ts for v in L])
    assert clen.cpu().tolist() == [v if 0 <= v <= Ts else -1 for v in L]
    # without the q / k norm the outputs and states are far from unit scale
    # (|k|^2 ~ 40, so beta k k^T amplifies what it multiplies): the pair
    # products are good to ~1e-5 of their operands, so the relative bounds
    # are 2e-5 and the max-abs bounds scale with the reference's largest
    # magnitude
    o_pk = float(np.abs(ref["o"]).max())
    s_pk = float(np.abs(ref["committed"][ok]).max())
    U.say(f"  largest |o| {o_pk:.3e}, largest |committed| {s_pk:.3e}")
    U.assert_close("o", U.to_np(o), ref["o"], rel=2e-5, mx=5e-5 * max(1.0, o_pk))
    U.assert_close("committed", U.to_np(st)[ok], ref["committed"][ok], rel=2e-5, mx=5e-5 * max(1.0, s_pk))
    assert torch.isnan(st[4]).all() and torch.isnan(cs[4]).all()
    assert np.array_equal(cs.to("cpu", torch.float32).numpy()[ok], ref["conv_state"][ok].astype(np.float32))


def test_verify_conv_fp32_d128_16_tokens(dev, oracle64):
    """fp32 inputs and outputs at d = 128 with 16 tokens: the largest LDS
    footprint of the fused verify (staged units and token arrays)."""
    U.say("verify_conv fp32 d=128 T=16")
    N, Ts, H, d, W = 4, 16, 2, 128, 4
    x, w, cst, g, b, init = _verify_case(N, Ts, H, d, W, torch.float32, seed=64)
    L = [16, 0, 7, 12]
    o, st, cs, clen, _, _ = _run_verify(dev, x, w, cst, g, b, init, L, out_dtype=torch.float32)
    ref, _ = _verify_reference(oracle64, x, w, cst, g, b, init, L, list(range(N)))
    U.assert_close("o", U.to_np(o), ref["o"], rel=1e-5, mx=1e-5)
    U.assert_close("committed", U.to_np(st), ref["committed"], rel=1e-5, mx=1e-5)
    assert np.array_equal(cs.cpu().numpy(), ref["conv_state"].astype(np.float32))
    assert clen.cpu().tolist() == L


def test_verify_conv_gated_norm_128x8(dev, oracle64):
    """Every verified output passes the gated RMS norm: 128 sequences x 8
    tokens, H=16, d=128, bf16; the commit is unaffected by the gate."""
    U.say("verify_conv gated norm 128 x 8 x H16 x d128")
    N, Ts, H, d, W = 128, 8, 16, 128, 4
    x, w, cst, g, b, init = _verify_case(N, Ts, H, d, W, torch.bfloat16, seed=44)
    z, wt = _gate(torch.Generator().manual_seed(344), (N, Ts, H, d), torch.bfloat16, d)
    L = torch.randint(0, Ts + 1, (N,), generator=torch.Generator().manual_seed(8)).tolist()
    o, st, cs, clen, _, _ = _run_verify(dev, x, w, cst, g, b, init, L, out_dtype=torch.bfloat16,
                                        gate=z.to(dev), gw=wt.to(dev))
    ref, _ = _verify_reference(oracle64, x, w, cst, g, b, init, L, list(range(N)), gate=z, gw=wt)
    U.assert_close("o", U.to_np(o), ref["o"], mx=_gated_bf16_max_abs(ref["o"]))
    U.assert_close("committed", U.to_np(st), ref["committed"])
    assert np.array_equal(cs.to("cpu", torch.float32).numpy(), ref["conv_state"].astype(np.float32))
    assert clen.cpu().tolist() == L


@pytest.mark.parametrize("d,Ts", [(16, 3), (64, 5), (128, 16)])
def test_verify_conv_gated_norm_fp32(dev, oracle64, d, Ts):
    """Gated RMS norm on the verify outputs with fp32 inputs and outputs,
    small and large heads, up to the longest window."""
    U.say(f"verify_conv gated norm fp32 d={d} T={Ts}")
    N, H, W = 5, 2, 4
    x, w, cst, g, b, init = _verify_case(N, Ts, H, d, W, torch.float32, seed=70 + d)
    z, wt = _gate(torch.Generator().manual_seed(370 + d), (N, Ts, H, d), torch.float32, d)
    L = [Ts, 1, 0, Ts - 1, 2]
    o, st, _, _, _, _ = _run_verify(dev, x, w, cst, g, b, init, L, out_dtype=torch.float32,
                                    gate=z.to(dev), gw=wt.to(dev))
    ref, _ = _verify_reference(oracle64, x, w, cst, g, b, init, L, list(range(N)), gate=z, gw=wt)
    U.assert_close("o", U.to_np(o), ref["o"], rel=1e-5, mx=1e-5)
    U.assert_close("committed", U.to_np(st), ref["committed"], rel=1e-5, mx=1e-5)
