"""CPU model of the chunked (WY / UT-transform) prefill, with the GPU path's
rounding of matrix-core operands made explicit.

This is NOT the oracle: it is an independent re-derivation of the same
recurrence in chunked form, used (1) with every rounding switched off, in
fp64, as a pin of the oracle (the chunked identity must reproduce the token
loop to ~1e-12 for every chunk size), and (2) with bf16 rounding switched on
per product, to decide which matrix-core operands the HIP kernel must carry
as a hi + lo bf16 pair to meet the error budget.

Chunked form (chunk positions r = 1..C, S_0 = state entering the chunk,
G_r = sum_{j<=r} g_j per key channel, gamma_r = exp(G_r)):

    A[r,s] = beta_r * sum_c k[r,c] k[s,c] exp(G[r,c] - G[s,c])      (s < r)
    T      = (I + A)^{-1} diag(beta)
    W      = T Ktil,  U = T V,        Ktil[r] = gamma_r * k_r
    u      = U - W S_0
    O      = scale * (Qtil S_0 + P u),  Qtil[r] = gamma_r * q_r,
             P[r,s] = sum_c q[r,c] k[s,c] exp(G[r,c] - G[s,c])       (s <= r)
    S_C    = Diag(gamma_C) S_0 + Kend^T u,   Kend[s] = k_s * gamma_C / gamma_s

exp(G_r - G_s) is evaluated as exp(G_r - G_b) * exp(G_b - G_s) with b the
first position of r's 16-row block, so every factor is <= 1 except the
within-block factor exp(G_b - G_s) <= exp(|one block's decay|).

Each product X @ Y is evaluated under a mode:
    "f"  : fp32 operands (no rounding)
    "1"  : both operands rounded to bf16
    "2"  : the first operand as hi + lo bf16 pair, the second rounded once
    "2b" : the second operand as a pair, the first rounded once
    "3"  : both as pairs, hi*hi + hi*lo + lo*hi
with fp32 accumulation ("exact" = fp64 everything, no rounding).
"""

from __future__ import annotations

import torch

PRODUCTS = ("A", "P", "W", "U", "WS", "QS", "Pu", "KS")


def bf16(x):
    return x.to(torch.bfloat16).to(x.dtype)


def split(x):
    hi = bf16(x)
    lo = bf16(x - hi)
    return hi, lo


def mm(x, y, mode, acc=torch.float32):
    """x @ y under a rounding mode, accumulated in `acc`."""
    if mode == "exact":
        return x.double() @ y.double()
    x = x.to(acc)
    y = y.to(acc)
    if mode == "f":
        return x @ y
    if mode == "1":
        return bf16(x) @ bf16(y)
    if mode == "2":
        xh, xl = split(x)
        yb = bf16(y)
        return xh @ yb + xl @ yb
    if mode == "2b":
        yh, yl = split(y)
        xb = bf16(x)
        return xb @ yh + xb @ yl
    if mode == "3":
        xh, xl = split(x)
        yh, yl = split(y)
        return xh @ yh + xh @ yl + xl @ yh
    raise ValueError(mode)


def decayed_pairs(left, right, G, mode, block=16, strict=False):
    """M[r,s] = sum_c left[r,c] right[s,c] exp(G[r,c] - G[s,c]) for s <= r
    (s < r when strict), via per-row-block references."""
    C = left.shape[0]
    dt = torch.float64 if mode == "exact" else torch.float32
    M = torch.zeros(C, C, dtype=dt)
    for b0 in range(0, C, block):
        b1 = min(C, b0 + block)
        Gb = G[b0]
        L = left[b0:b1] * torch.exp(G[b0:b1] - Gb)          # <= 1
        R = right[:b1] * torch.exp(Gb - G[:b1])              # <= 1 before b0, bounded within
        M[b0:b1, :b1] = mm(L, R.T, mode).to(dt)
    mask = torch.tril(torch.ones(C, C, dtype=torch.bool), diagonal=-1 if strict else 0)
    return M * mask


def forward_solve(A, beta):
    """T = (I + A)^{-1} diag(beta), A strictly lower triangular (fp of A)."""
    C = A.shape[0]
    X = torch.zeros_like(A)
    I = torch.eye(C, dtype=A.dtype)
    for r in range(C):
        X[r] = I[r] - A[r, :r] @ X[:r]
    return X * beta[None, :]


def chunked_kda(q, k, v, g, beta, S0, C=64, plan=None, scale=1.0, out_bf16=False):
    """One (sequence, head).  q, k, g [T, dk]; v [T, dv]; beta [T]; S0 [dk, dv].
    plan: dict product -> mode (missing -> "f"); None -> all "exact".
    Returns (O [T, dv], S_T [dk, dv]) in fp64."""
    exact = plan is None
    dt = torch.float64 if exact else torch.float32
    md = (lambda name: "exact") if exact else (lambda name: plan.get(name, "f"))
    q, k, v, g, beta = (torch.as_tensor(t).to(dt) for t in (q, k, v, g, beta))
    S = torch.as_tensor(S0).to(dt).clone()
    T = q.shape[0]
    O = torch.zeros(T, v.shape[1], dtype=torch.float64)
    for c0 in range(0, T, C):
        c1 = min(T, c0 + C)
        qc, kc, vc, gc, bc = q[c0:c1], k[c0:c1], v[c0:c1], g[c0:c1], beta[c0:c1]
        G = torch.cumsum(gc, 0)
        gam = torch.exp(G)
        Ktil = kc * gam
        Qtil = qc * gam
        Kend = kc * torch.exp(G[-1][None, :] - G)
        A = decayed_pairs(kc, kc, G, md("A"), strict=True).to(dt) * bc[:, None]
        Tm = forward_solve(A, bc)
        W = mm(Tm, Ktil, md("W")).to(dt)
        U = mm(Tm, vc, md("U")).to(dt)
        u = U - mm(W, S, md("WS")).to(dt)
        P = decayed_pairs(qc, kc, G, md("P")).to(dt)
        o = mm(Qtil, S, md("QS")).to(dt) + mm(P, u, md("Pu")).to(dt)
        o = o * scale
        if out_bf16:
            o = o.float().to(torch.bfloat16).double()
        O[c0:c1] = o.double()
        S = gam[-1][:, None] * S + mm(Kend.T, u, md("KS")).to(dt)
    return O, S.double()
