"""Brute-force fp64 forms of the KDA definitions, for tiny sizes only.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

These evaluate the recurrence as explicit matrix products rather than the
rank-1 token update of ``kda_oracle.c``, so that the two can be checked
against each other:

* ``matrix_form``: S_t = A_t S_{t-1} + beta_t k_t v_t^T with the transition
  A_t = (I - beta_t k_t k_t^T) Diag(exp g_t) built as a full d_k x d_k matrix.
* ``unrolled_form``: the closed sum
      S_t = Phi(t, 0) S_0 + sum_{s<=t} Phi(t, s) beta_s k_s v_s^T,
      Phi(t, s) = A_t A_{t-1} ... A_{s+1}   (identity when s = t),
  and o_t = scale * S_t^T q_t, with every product formed from scratch.
* ``conv_form``: the causal depthwise convolution via numpy.convolve.
* ``decode_conv_form``: one fused decode step (convolution, optional SiLU,
  per-head L2 normalisation of q and k, one recurrence step) with every sum
  written out.
"""

from __future__ import annotations

import numpy as np


def _transition(k, g, beta):
    dk = k.shape[0]
    return (np.eye(dk) - beta * np.outer(k, k)) @ np.diag(np.exp(g))


def matrix_form(q, k, v, g, beta, S0, scale=1.0):
    """One sequence, one head.  q, k, g [T, dk]; v [T, dv]; beta [T]; S0 [dk, dv]."""
    q, k, v, g, beta, S = (np.asarray(a, np.float64) for a in (q, k, v, g, beta, S0))
    S = S.copy()
    T = q.shape[0]
    o = np.zeros((T, v.shape[1]))
    for t in range(T):
        S = _transition(k[t], g[t], beta[t]) @ S + beta[t] * np.outer(k[t], v[t])
        o[t] = scale * S.T @ q[t]
    return o, S


def unrolled_form(q, k, v, g, beta, S0, scale=1.0):
    """Same result as :func:`matrix_form` through the unrolled sum."""
    q, k, v, g, beta, S0 = (np.asarray(a, np.float64) for a in (q, k, v, g, beta, S0))
    T, dk = q.shape
    A = [_transition(k[t], g[t], beta[t]) for t in range(T)]

    def phi(t, s):
        P = np.eye(dk)
        for j in range(s + 1, t + 1):
            P = A[j] @ P
        return P

    o = np.zeros((T, v.shape[1]))
    S_t = None
    for t in range(T):
        S_t = phi(t, -1) @ S0
        for s in range(t + 1):
            S_t = S_t + phi(t, s) @ (beta[s] * np.outer(k[s], v[s]))
        o[t] = scale * S_t.T @ q[t]
    return o, S_t


def conv_form(x, w, state=None, bias=None, act=0):
    """One sequence.  x [T, C]; w [C, W]; state [C, W-1] (oldest first) or None.
    Returns y [T, C] and the new state [C, W-1]."""
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    T, C = x.shape
    W = w.shape[1]
    hist = np.zeros((C, W - 1)) if state is None else np.asarray(state, np.float64)
    y = np.zeros((T, C))
    new = np.zeros((C, W - 1))
    for c in range(C):
        xb = np.concatenate([hist[c], x[:, c]])
        # np.convolve flips its second argument: taps reversed gives
        # y[t] = sum_j w[j] * xb[t + j] over the 'valid' range.
        full = np.convolve(xb, w[c][::-1], mode="valid")
        y[:, c] = full[:T]
        if W > 1:
            new[c] = xb[-(W - 1):]
    if bias is not None:
        y = y + np.asarray(bias, np.float64)[None, :]
    if act == 1:
        y = y / (1 + np.exp(-y))
    return y, new


def decode_conv_form(x, w, g, beta, S0, conv_state, H, d, bias=None, act=0, qk_l2norm=1,
                     norm_eps=1e-6, scale=1.0):
    """One sequence, one token.  x [3 H d]; w [3 H d, W]; conv_state
    [3 H d, W-1]; g [H, d]; beta [H]; S0 [H, d, d].  Returns o [H, d] and the
    new state [H, d, d]."""
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    hist = np.asarray(conv_state, np.float64)
    C, W = w.shape
    y = np.zeros(C)
    for c in range(C):
        acc = 0.0 if bias is None else float(bias[c])
        for j in range(W):
            # tap W-1 multiplies the current token, tap j the token W-1-j back
            xv = x[c] if j == W - 1 else hist[c, j]
            acc += w[c, j] * xv
        if act == 1:
            acc = acc / (1.0 + np.exp(-acc))
        y[c] = acc
    o = np.zeros((H, d))
    S = np.zeros((H, d, d))
    for h in range(H):
        q = y[h * d:(h + 1) * d]
        k = y[H * d + h * d:H * d + (h + 1) * d]
        v = y[2 * H * d + h * d:2 * H * d + (h + 1) * d]
        if qk_l2norm:
            q = q / np.sqrt(sum(t * t for t in q) + norm_eps)
            k = k / np.sqrt(sum(t * t for t in k) + norm_eps)
        o_h, S_h = matrix_form(q[None], k[None], v[None], np.asarray(g, np.float64)[h][None],
                               np.array([beta[h]], np.float64), S0[h], scale)
        o[h] = o_h[0]
        S[h] = S_h
    return o, S
