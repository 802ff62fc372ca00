"""GPU parity of kda_conv_short against the CPU oracle."""

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


def _check_y(name, y_gpu, y_ref, dtype):
    got = U.to_np(y_gpu)
    if dtype == torch.bfloat16:
        # One rounding of the fp32 sum: every element within half a bf16 unit
        # of the exact value (this bounds the absolute error by 2^-8 |y|, so
        # no fixed max-abs bar applies: |y| reaches ~5 with the bias).
        assert U.within_bf16_of(got, y_ref), f"{name}: beyond one bf16 rounding"
        U.assert_close(name, got, y_ref, mx=2.0 ** -8 * float(np.abs(y_ref).max()) + 1e-6)
    else:
        U.assert_close(name, got, y_ref, rel=1e-6, mx=1e-5)


def test_conv_decode_batched(dev, oracle64):
    """Decode-shaped conv: 128 sequences x 1 token, C = 3*16*128 = 6144,
    W = 4, bf16, carried state updated in place."""
    U.say("conv decode 128 x 6144")
    wl = make_workload(1, with_conv=True)
    N = 128
    y_ref, st_ref = oracle64.conv_short(wl.conv_x, wl.conv_w, wl.cu_seqlens, state=wl.conv_state)
    x = wl.conv_x.to(dev)
    w = wl.conv_w.to(dev)
    pool = wl.conv_state.to(dev).clone()
    slots = torch.arange(N, dtype=torch.int32, device=dev)
    cu = wl.cu_seqlens.to(dev)
    y = K.kda_conv_short(x, w, cu, pool, slots, slots)
    torch.cuda.synchronize()
    _check_y("y", y, y_ref, torch.bfloat16)
    assert np.array_equal(U.to_np(pool), st_ref), "new conv state differs"


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("W", [2, 4, 6])
def test_conv_varlen_ragged(dev, oracle64, dtype, W):
    """Packed sequences of lengths 0, 1, 2, 3, 5, 64, 65, 200 (several body
    tiles and ragged tails), some from zero history, with bias and SiLU,
    states written to separate destination slots."""
    U.say(f"conv varlen W={W} {dtype}")
    lens = [0, 1, 2, 3, 5, 64, 65, 200]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T, C, N = int(cu[-1]), 96, len(lens)
    gen = torch.Generator().manual_seed(17)
    x = torch.randn(T, C, generator=gen).to(dtype)
    w = ((torch.rand(C, W, generator=gen) * 2 - 1) / W ** 0.5).to(dtype)
    bias = torch.randn(C, generator=gen).to(dtype)
    st = torch.randn(N, C, W - 1, generator=gen).to(dtype)
    has = np.array([1, 0, 1, 1, 0, 1, 0, 1], np.int32)
    for act in (0, 1):
        y_ref, st_ref = oracle64.conv_short(x, w, cu, state=st, has_state=has, bias=bias, act=act)
        pool = torch.cat([st, torch.zeros_like(st)]).to(dev)
        src = torch.tensor([i if has[i] else -1 for i in range(N)], dtype=torch.int32, device=dev)
        dst = torch.arange(N, 2 * N, dtype=torch.int32, device=dev)
        y = K.kda_conv_short(x.to(dev), w.to(dev), torch.tensor(cu, device=dev), pool, src, dst,
                             bias=bias.to(dev), act=act)
        torch.cuda.synchronize()
        _check_y(f"y act={act}", y, y_ref, dtype)
        assert np.array_equal(U.to_np(pool[N:]), st_ref), "new conv state differs"
        assert torch.equal(pool[:N].cpu(), st), "source conv state modified"


def test_conv_advance_len_and_inplace(dev, oracle64):
    """Verify-commit shape: 8 tokens per sequence, state advanced by only the
    accepted L in {0..8} tokens, in place."""
    U.say("conv advance_len in place")
    N, Ts, C, W = 16, 8, 256, 4
    gen = torch.Generator().manual_seed(3)
    x = torch.randn(N * Ts, C, generator=gen).to(torch.bfloat16)
    w = ((torch.rand(C, W, generator=gen) * 2 - 1) * 0.5).to(torch.bfloat16)
    st = torch.randn(N, C, W - 1, generator=gen).to(torch.bfloat16)
    L = torch.randint(0, Ts + 1, (N,), generator=gen, dtype=torch.int32)
    cu = torch.arange(0, N * Ts + 1, Ts, dtype=torch.int32)
    y_ref, st_ref = oracle64.conv_short(x, w, cu, state=st, advance_len=L)
    pool = st.to(dev).clone()
    slots = torch.arange(N, dtype=torch.int32, device=dev)
    y = K.kda_conv_short(x.to(dev), w.to(dev), cu.to(dev), pool, slots, slots, advance_len=L.to(dev))
    torch.cuda.synchronize()
    _check_y("y", y, y_ref, torch.bfloat16)
    assert np.array_equal(U.to_np(pool), st_ref)


def test_conv_tiny_fp32(dev, oracle64):
    """Tiny workload's conv: T = 64, C = 3*2*16, fp32, zero history."""
    U.say("conv tiny fp32")
    wl = make_workload(0, with_conv=True)
    y_ref, st_ref = oracle64.conv_short(wl.conv_x, wl.conv_w, wl.cu_seqlens)
    pool = torch.zeros(1, 96, 3, device=dev)
    src = torch.full((1,), -1, dtype=torch.int32, device=dev)
    dst = torch.zeros(1, dtype=torch.int32, device=dev)
    y = K.kda_conv_short(wl.conv_x.to(dev), wl.conv_w.to(dev), wl.cu_seqlens.to(dev), pool, src, dst)
    torch.cuda.synchronize()
    _check_y("y", y, y_ref, torch.float32)
    assert np.array_equal(U.to_np(pool), st_ref)


@pytest.mark.parametrize("dtype,hd", [(torch.bfloat16, 128), (torch.bfloat16, 16), (torch.float32, 128),
                                      (torch.float32, 32)])
def test_conv_head_norm(dev, oracle64, dtype, hd):
    """The optional per-head normalisation: C = 3 H d channels, the first
    2 H d (q and k blocks) normalised per token in groups of d after the
    SiLU, the v block as convolved; packed sequences with ragged lengths
    (0, 1, 2, 3, 40, 130), some without history.  Against the oracle's
    operand forming (one rounding to dtype of the normalised fp64 value)."""
    import oracle as O
    U.say(f"conv head norm d={hd} {dtype}")
    H = 2
    C = 3 * H * hd
    lens = [0, 1, 2, 3, 40, 130]
    N = len(lens)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32)
    T = int(cu[-1])
    gen = torch.Generator().manual_seed(700 + hd)
    x = torch.randn(T, C, generator=gen).to(dtype)
    w = (torch.rand(C, 4, generator=gen) - 0.5).to(dtype)
    st = torch.randn(N, C, 3, generator=gen).to(dtype)
    has = np.array([1, 0, 1, 1, 0, 1], np.int32)
    y_ref, st_ref = oracle64.conv_short(x, w, cu, act=1, state=st, has_state=has)
    q, k, v = O.conv_operands(y_ref, H, hd, 1, 1e-6, "bf16" if dtype == torch.bfloat16 else "f32")
    want = np.concatenate([q.reshape(T, -1), k.reshape(T, -1), v.reshape(T, -1)], axis=1)
    pool = torch.cat([st, torch.zeros_like(st)]).to(dev)
    src = torch.tensor([s if has[s] else -1 for s in range(N)], dtype=torch.int32, device=dev)
    dst = torch.arange(N, 2 * N, dtype=torch.int32, device=dev)
    y = K.kda_conv_short(x.to(dev), w.to(dev), cu.to(dev), pool, src, dst, act=1, norm_d=hd,
                         norm_channels=2 * H * hd)
    torch.cuda.synchronize()
    got = y.to("cpu", torch.float32).numpy().astype(np.float64)
    if dtype == torch.bfloat16:
        diff = np.abs(got - want)
        ulp = np.ldexp(1.0, np.floor(np.log2(np.abs(want) + 1e-30)).astype(int) - 7)
        floor = 2.0 ** -16 * np.abs(want).max()
        assert np.all(diff <= ulp + floor), float((diff / (ulp + floor)).max())
        assert float(np.mean(diff > 0)) < 0.02
    else:
        U.assert_close("y", got, want, rel=1e-5, mx=1e-5)
    # the q and k groups have unit norm (up to eps and the rounding)
    norms = np.sqrt((got[:, :2 * H * hd].reshape(T, 2 * H, hd) ** 2).sum(-1))
    if T:
        assert np.all(np.abs(norms - 1.0) < 1e-2)
    assert np.array_equal(pool[N:].to("cpu", torch.float32).numpy(), st_ref.astype(np.float32))
