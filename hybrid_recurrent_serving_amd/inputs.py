"""Seeded synthetic inputs for the KDA layer path.

This module only draws random numbers and lays them out; it holds none of the
recurrence's arithmetic.  Both the CPU oracle (under ``oracle/``) and the HIP
library consume the tensors it returns, so the two sides always see the same
materialised values.

Distributions (the pages give no data; these follow the workloads the library
is measured on):

* q, k ~ N(0, 1), then divided by their L2 norm per (token, head), in fp32,
  then cast to the input dtype.  The library itself never normalises.
* v ~ N(0, 1).
* g = logsigmoid(N(mu_g, 1)) per key channel (the log of the decay alpha);
  mu_g = 0 by default (E[alpha] ~ 0.5), mu_g = 4 for the slow-decay stress
  (alpha ~ 0.98).
* beta = sigmoid(N(0, 1)), one scalar per (token, head).
* initial recurrent states ~ N(0, 0.1) (standard deviation 0.1), fp32.
* short-convolution weights ~ U(-1/sqrt(W), 1/sqrt(W)); conv input x ~ N(0, 1);
  conv state ~ N(0, 1).

Fixed draw order per workload: lengths / accepted lengths -> q -> k -> v -> g
-> beta -> initial states -> conv weights -> conv state -> conv input.
The workload index is the seed.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import torch

# Workload table: index -> human-readable description.  Sizes are fixed here;
# tests may shrink token counts through the ``T`` / ``lengths`` overrides.
WORKLOADS = {
    0: "tiny: B=1, T=64, H=2, d=16, fp32, chunk=16, conv width 4",
    1: "batched decode: 128 sequences x 1 token, H=16, d=128, bf16",
    2: "varlen prefill: 16 packed sequences, lengths U{512..16384}, H=16, d=128, chunk=64, bf16",
    3: "long prefill: B=1, T=1048576, H=16, d=128, chunk=64, checkpoint every 32768, bf16",
    4: "speculative verify: 128 sequences x 8 tokens, H=16, d=128, bf16",
}


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _unit(x: torch.Tensor) -> torch.Tensor:
    # Divide by the L2 norm over the last axis (one vector per token and head).
    return x / x.norm(dim=-1, keepdim=True)


def draw_qkvgb(gen, shape_tok, H, dk, dv, dtype, device, mu_g=0.0):
    """Draw q, k, v, g, beta for a token grid ``shape_tok`` (a tuple)."""
    f32 = torch.float32
    q = _unit(torch.randn(*shape_tok, H, dk, generator=gen, dtype=f32, device=device)).to(dtype)
    k = _unit(torch.randn(*shape_tok, H, dk, generator=gen, dtype=f32, device=device)).to(dtype)
    v = torch.randn(*shape_tok, H, dv, generator=gen, dtype=f32, device=device).to(dtype)
    g = torch.nn.functional.logsigmoid(
        torch.randn(*shape_tok, H, dk, generator=gen, dtype=f32, device=device) + mu_g).to(dtype)
    beta = torch.sigmoid(torch.randn(*shape_tok, H, generator=gen, dtype=f32, device=device)).to(dtype)
    return q, k, v, g, beta


def draw_states(gen, n, H, dk, dv, device, std=0.1):
    return torch.randn(n, H, dk, dv, generator=gen, dtype=torch.float32, device=device) * std


def draw_conv(gen, T, C, W, n_seq, dtype, device, with_state=True):
    bound = 1.0 / math.sqrt(W)
    w = (torch.rand(C, W, generator=gen, dtype=torch.float32, device=device) * 2 - 1) * bound
    st = None
    if with_state:
        st = torch.randn(n_seq, C, W - 1, generator=gen, dtype=torch.float32, device=device).to(dtype)
    x = torch.randn(T, C, generator=gen, dtype=torch.float32, device=device).to(dtype)
    return w.to(dtype), st, x


@dataclass
class Workload:
    """Materialised inputs of one workload (all tensors on ``device``)."""
    index: int
    H: int
    dk: int
    dv: int
    chunk: int
    dtype: torch.dtype
    q: torch.Tensor = None          # [T_tot, H, dk]  (or [N, T_spec, H, dk] for verify)
    k: torch.Tensor = None
    v: torch.Tensor = None
    g: torch.Tensor = None          # log decay, same shape as k
    beta: torch.Tensor = None       # [T_tot, H]
    cu_seqlens: Optional[torch.Tensor] = None   # int32 [N+1]
    init_states: Optional[torch.Tensor] = None  # fp32 [n_init, H, dk, dv]
    init_index: Optional[list] = None           # sequence i -> row of init_states or -1
    accepted_len: Optional[torch.Tensor] = None  # int32 [N] (verify)
    ckpt_interval: int = 0
    conv_w: Optional[torch.Tensor] = None       # [C, W]
    conv_state: Optional[torch.Tensor] = None   # [N, C, W-1]
    conv_x: Optional[torch.Tensor] = None       # [T_tot, C]
    conv_W: int = 4
    extra: dict = field(default_factory=dict)

    @property
    def n_seq(self) -> int:
        if self.cu_seqlens is not None:
            return self.cu_seqlens.numel() - 1
        return self.q.shape[0]


def make_workload(index: int, device="cpu", *, T: Optional[int] = None,
                  lengths: Optional[list] = None, n_seq: Optional[int] = None,
                  H: Optional[int] = None, d: Optional[int] = None, mu_g: float = 0.0,
                  with_conv: bool = False, seed: Optional[int] = None) -> Workload:
    """Build workload ``index`` (0..4).  Overrides shrink it for tests.

    ``seed`` defaults to ``index``.  ``with_conv`` adds the short-convolution
    inputs (weights, state, input) drawn after everything else.
    """
    seed = index if seed is None else seed
    gen = _gen(seed, device)
    if index == 0:
        H_ = H or 2
        d_ = d or 16
        T_ = T or 64
        dtype = torch.float32
        q, k, v, g, b = draw_qkvgb(gen, (T_,), H_, d_, d_, dtype, device, mu_g)
        wl = Workload(0, H_, d_, d_, 16, dtype, q, k, v, g, b,
                      cu_seqlens=torch.tensor([0, T_], dtype=torch.int32, device=device),
                      init_index=[-1])
        if with_conv:
            C = 3 * H_ * d_
            wl.conv_w, wl.conv_state, wl.conv_x = draw_conv(gen, T_, C, 4, 1, dtype, device,
                                                            with_state=False)
        return wl
    if index == 1:
        N = n_seq or 128
        H_ = H or 16
        d_ = d or 128
        dtype = torch.bfloat16
        q, k, v, g, b = draw_qkvgb(gen, (N,), H_, d_, d_, dtype, device, mu_g)
        st = draw_states(gen, N, H_, d_, d_, device)
        wl = Workload(1, H_, d_, d_, 64, dtype, q, k, v, g, b,
                      cu_seqlens=torch.arange(N + 1, dtype=torch.int32, device=device),
                      init_states=st, init_index=list(range(N)))
        if with_conv:
            C = 3 * H_ * d_
            wl.conv_w, wl.conv_state, wl.conv_x = draw_conv(gen, N, C, 4, N, dtype, device)
        return wl
    if index == 2:
        N = n_seq or 16
        H_ = H or 16
        d_ = d or 128
        dtype = torch.bfloat16
        if lengths is None:
            lens = torch.randint(512, 16385, (N,), generator=gen, device=device).tolist()
        else:
            lens = list(lengths)
            N = len(lens)
        cu = [0]
        for L in lens:
            cu.append(cu[-1] + int(L))
        T_tot = cu[-1]
        q, k, v, g, b = draw_qkvgb(gen, (T_tot,), H_, d_, d_, dtype, device, mu_g)
        n_init = (N + 1) // 2
        st = draw_states(gen, n_init, H_, d_, d_, device)
        init_index = [i // 2 if i % 2 == 0 else -1 for i in range(N)]
        wl = Workload(2, H_, d_, d_, 64, dtype, q, k, v, g, b,
                      cu_seqlens=torch.tensor(cu, dtype=torch.int32, device=device),
                      init_states=st, init_index=init_index)
        if with_conv:
            C = 3 * H_ * d_
            wl.conv_w, wl.conv_state, wl.conv_x = draw_conv(gen, T_tot, C, 4, N, dtype, device)
        return wl
    if index == 3:
        T_ = T or 1048576
        H_ = H or 16
        d_ = d or 128
        dtype = torch.bfloat16
        q, k, v, g, b = _draw_long(gen, T_, H_, d_, dtype, device, mu_g)
        return Workload(3, H_, d_, d_, 64, dtype, q, k, v, g, b,
                        cu_seqlens=torch.tensor([0, T_], dtype=torch.int32, device=device),
                        init_index=[-1], ckpt_interval=32768)
    if index == 4:
        N = n_seq or 128
        H_ = H or 16
        d_ = d or 128
        Ts = T or 8
        dtype = torch.bfloat16
        L = torch.randint(1, Ts + 1, (N,), generator=gen, device=device).to(torch.int32)
        q, k, v, g, b = draw_qkvgb(gen, (N, Ts), H_, d_, d_, dtype, device, mu_g)
        st = draw_states(gen, N, H_, d_, d_, device)
        return Workload(4, H_, d_, d_, 64, dtype, q, k, v, g, b, init_states=st,
                        init_index=list(range(N)), accepted_len=L)
    raise ValueError(f"unknown workload {index}")


def _draw_long(gen, T, H, d, dtype, device, mu_g, slab=65536):
    """Draw q, k, v, g, beta for one long sequence in token slabs.

    Same law as :func:`draw_qkvgb`; the slabbing only bounds the fp32
    temporaries.  Order: all of q, then all of k, v, g, beta.
    """
    f32 = torch.float32
    out = [torch.empty(T, H, d, dtype=dtype, device=device) for _ in range(4)]
    beta = torch.empty(T, H, dtype=dtype, device=device)
    for which in range(4):
        for s in range(0, T, slab):
            e = min(T, s + slab)
            x = torch.randn(e - s, H, d, generator=gen, dtype=f32, device=device)
            if which < 2:
                x = _unit(x)
            elif which == 3:
                x = torch.nn.functional.logsigmoid(x + mu_g)
            out[which][s:e] = x.to(dtype)
    for s in range(0, T, slab):
        e = min(T, s + slab)
        beta[s:e] = torch.sigmoid(torch.randn(e - s, H, generator=gen, dtype=f32,
                                              device=device)).to(dtype)
    return out[0], out[1], out[2], out[3], beta
