"""CPU oracle for the KDA layer path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, the smoke check in ``__graft_entry__`` and the CPU-baseline
leg of ``bench.py`` may import this package.  The HIP library never calls it
and there is no CPU fallback through it.

Two pieces:

* ``kda_oracle.c`` (built here with gcc): the token-by-token recurrence, the
  short causal convolution and the checkpoint enumeration, in fp64 (default)
  or fp32 (``real="f32"``).
* ``bruteforce.py``: numpy fp64 evaluations of the same definitions written
  as explicit matrix products, for tiny sizes only.

Every function takes torch tensors or numpy arrays; values are upcast to
float32 exactly (bf16 -> fp32 is exact) before the C code sees them.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
import sys
from pathlib import Path

import numpy as np

HERE = Path(__file__).resolve().parent
SRC = HERE / "kda_oracle.c"

_LIB_NAMES = {"f64": "liboracle_f64.so", "f32": "liboracle_f32.so"}


def build(real: str = "f64", mutant: int = 0, out: Path | None = None, quiet=True) -> Path:
    """Compile ``kda_oracle.c`` with gcc -O2 -fopenmp.  Returns the .so path."""
    if out is None:
        out = HERE / (_LIB_NAMES[real] if mutant == 0 else f"liboracle_{real}_m{mutant}.so")
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-Wall", "-Wextra",
           "-Wno-unused-parameter", f"-DORACLE_MUTANT={int(mutant)}"]
    if real == "f32":
        cmd.append("-DORACLE_REAL_FLOAT")
    cmd += [str(SRC), "-o", str(out), "-lm"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("oracle build failed:\n" + res.stderr)
    if not quiet and res.stderr:
        print(res.stderr, file=sys.stderr)
    return out


def _as_f32(x):
    if x is None:
        return None
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return np.ascontiguousarray(x.detach().to("cpu", torch.float32).numpy())
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32))


def _as_i32(x):
    if x is None:
        return None
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return np.ascontiguousarray(x.detach().to("cpu", torch.int32).numpy())
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


class Oracle:
    """ctypes front of one build of ``kda_oracle.c``."""

    def __init__(self, path: Path):
        self.path = Path(path)
        self.lib = ctypes.CDLL(str(self.path))
        L = self.lib
        vp, i32, i64, dbl = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        L.oracle_real_bytes.restype = ctypes.c_int
        L.oracle_mutant.restype = ctypes.c_int
        L.oracle_get_threads.restype = ctypes.c_int
        L.oracle_set_threads.argtypes = [ctypes.c_int]
        L.oracle_ckpt_enumerate.restype = i64
        L.oracle_ckpt_enumerate.argtypes = [vp, vp, i32, i32, vp, vp, i64]
        L.oracle_kda_varlen.restype = ctypes.c_int
        L.oracle_kda_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, dbl,
                                        vp, vp, vp, vp, i32, vp, i64, vp, i64, i32]
        L.oracle_kda_verify.restype = ctypes.c_int
        L.oracle_kda_verify.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, dbl,
                                        vp, vp, vp, vp, vp]
        L.oracle_conv_short.restype = ctypes.c_int
        L.oracle_conv_short.argtypes = [vp, i64, vp, vp, i32, vp, i32, i32, i32, vp, vp, vp,
                                        vp, vp]
        self.real = np.float64 if L.oracle_real_bytes() == 8 else np.float32
        self.mutant = L.oracle_mutant()

    # -- threads -----------------------------------------------------------
    def set_threads(self, n: int):
        self.lib.oracle_set_threads(int(n))

    def threads(self) -> int:
        return self.lib.oracle_get_threads()

    # -- checkpoint positions ---------------------------------------------
    def ckpt_enumerate(self, cu_seqlens, interval, start_pos=None):
        cu = _as_i32(cu_seqlens)
        sp = _as_i32(start_pos)
        n = cu.size - 1
        ck_cu = np.zeros(n + 1, np.int32)
        total = self.lib.oracle_ckpt_enumerate(_p(cu), _p(sp), n, int(interval), _p(ck_cu), None, 0)
        pos = np.zeros(max(total, 1), np.int32)
        self.lib.oracle_ckpt_enumerate(_p(cu), _p(sp), n, int(interval), _p(ck_cu), _p(pos), total)
        return ck_cu, pos[:total]

    # -- recurrence ---------------------------------------------------------
    def kda_varlen(self, q, k, v, g, beta, cu_seqlens, *, init=None, has_init=None,
                   start_pos=None, scale=1.0, ckpt_interval=0, pairs=None, want_o=True,
                   want_final=True):
        """Token-by-token recurrence over a packed batch.

        q, k, g [T, H, dk]; v [T, H, dv]; beta [T, H]; cu_seqlens [N+1];
        init [N, H, dk, dv] or None; has_init [N] (0/1) or None.
        Returns dict with o [T, H, dv] (zeros for pairs not computed), final
        [N, H, dk, dv], ckpt [n_ckpt, H, dk, dv], ckpt_cu, ckpt_pos.
        """
        q, k, v, g, beta = (_as_f32(t) for t in (q, k, v, g, beta))
        cu = _as_i32(cu_seqlens)
        sp = _as_i32(start_pos)
        T, H, dk = q.shape
        dv = v.shape[-1]
        N = cu.size - 1
        init_a = None if init is None else np.ascontiguousarray(np.asarray(
            init.detach().cpu().numpy() if hasattr(init, "detach") else init, dtype=self.real))
        hi = _as_i32(has_init)
        pr = None if pairs is None else np.ascontiguousarray(np.asarray(pairs, np.int32).reshape(-1, 2))
        o = np.zeros((T, H, dv), self.real) if want_o else None
        final = np.zeros((N, H, dk, dv), self.real) if want_final else None
        ck_cu, ck_pos = self.ckpt_enumerate(cu, ckpt_interval, sp)
        n_ck = int(ck_cu[-1])
        ck = np.zeros((n_ck, H, dk, dv), self.real) if n_ck else None
        rc = self.lib.oracle_kda_varlen(
            _p(q), _p(k), _p(v), _p(g), _p(beta), _p(cu), _p(sp), N, H, dk, dv, float(scale),
            _p(init_a), _p(hi), _p(o if want_o else np.zeros(1, self.real)), _p(final),
            int(ckpt_interval), _p(ck), n_ck, _p(pr), 0 if pr is None else pr.shape[0],
            0 if want_o else 1)
        if rc != 0:
            raise RuntimeError(f"oracle_kda_varlen failed ({rc})")
        return {"o": o, "final": final, "ckpt": ck, "ckpt_cu": ck_cu, "ckpt_pos": ck_pos}

    def kda_verify(self, q, k, v, g, beta, init, accepted_len=None, *, scale=1.0):
        """Speculative verify.  q, k, g [N, Ts, H, dk]; v [N, Ts, H, dv];
        beta [N, Ts, H]; init [N, H, dk, dv]; accepted_len [N] or None (= Ts).
        Returns dict o [N, Ts, H, dv], committed [N, H, dk, dv] (NaN where
        rejected), committed_len [N]."""
        q, k, v, g, beta = (_as_f32(t) for t in (q, k, v, g, beta))
        N, Ts, H, dk = q.shape
        dv = v.shape[-1]
        init_a = np.ascontiguousarray(np.asarray(
            init.detach().cpu().numpy() if hasattr(init, "detach") else init, dtype=self.real))
        acc = _as_i32(accepted_len)
        o = np.zeros((N, Ts, H, dv), self.real)
        com = np.full((N, H, dk, dv), np.nan, self.real)
        clen = np.zeros(N, np.int32)
        rc = self.lib.oracle_kda_verify(_p(q), _p(k), _p(v), _p(g), _p(beta), N, Ts, H, dk, dv,
                                        float(scale), _p(init_a), _p(acc), _p(o), _p(com),
                                        _p(clen))
        if rc != 0:
            raise RuntimeError(f"oracle_kda_verify failed ({rc})")
        return {"o": o, "committed": com, "committed_len": clen}

    # -- convolution --------------------------------------------------------
    def conv_short(self, x, w, cu_seqlens, *, bias=None, act=0, state=None, has_state=None,
                   advance_len=None):
        """Short causal depthwise convolution.  x [T, C]; w [C, W];
        state [N, C, W-1] or None.  Returns (y [T, C], new_state [N, C, W-1])."""
        x = _as_f32(x)
        w = _as_f32(w)
        b = _as_f32(bias)
        st = _as_f32(state)
        hs = _as_i32(has_state)
        adv = _as_i32(advance_len)
        cu = _as_i32(cu_seqlens)
        T, C = x.shape
        W = w.shape[1]
        N = cu.size - 1
        y = np.zeros((T, C), self.real)
        ns = np.zeros((N, C, W - 1), self.real)
        rc = self.lib.oracle_conv_short(_p(x), C, _p(w), _p(b), int(act), _p(cu), N, C, W,
                                        _p(st), _p(hs), _p(adv), _p(y), _p(ns))
        if rc != 0:
            raise RuntimeError(f"oracle_conv_short failed ({rc})")
        return y, ns


    # -- prefill with the short convolution in front --------------------------
    def kda_prefill_conv(self, x, w, g, beta, cu_seqlens, *, H, d, bias=None, act=0, conv_state=None,
                         has_conv_state=None, qk_l2norm=1, norm_eps=1e-6, operand_dtype="bf16",
                         init=None, has_init=None, start_pos=None, scale=1.0, ckpt_interval=0):
        """The prefill of a packed batch from the tokens' raw projections.

        x [T, 3 H d] (channels ordered q block, k block, v block, each
        [H, d]); w [3 H d, W]; bias [3 H d] or None; conv_state [N, 3 H d,
        W-1] and has_conv_state [N] (0 = no history) or None; g [T, H, d];
        beta [T, H]; init / has_init / start_pos / ckpt_interval as
        :meth:`kda_varlen`.

        Per sequence: y = conv(history ++ tokens) (+ SiLU when act == 1) as
        :meth:`conv_short`, unrounded; q, k, v from y by :func:`conv_operands`
        (per-head normalisation of q and k, then one rounding to the
        recurrence's input type); then :meth:`kda_varlen`.  The new conv
        history of each sequence is the last W-1 raw inputs of history ++
        tokens.

        With ckpt_interval > 0, every checkpoint of the recurrence (the
        positions of :meth:`ckpt_enumerate`) also gets the conv history a
        resumed run needs: the last W-1 raw inputs of history ++ tokens before
        the checkpoint's position, the new-state rule of :meth:`conv_short`
        after that many tokens.

        Returns the dict of :meth:`kda_varlen` plus conv_state [N, 3 H d, W-1],
        conv_ckpt [n_ckpt, 3 H d, W-1] and the operands q, k, v [T, H, d]
        (float32)."""
        xa = np.asarray(_as_f32(x), np.float32)
        T, C = xa.shape
        if C != 3 * H * d:
            raise ValueError("x must have 3 * H * d channels")
        y, ns = self.conv_short(xa, w, cu_seqlens, bias=bias, act=act, state=conv_state,
                                has_state=has_conv_state)
        q, k, v = conv_operands(y, H, d, qk_l2norm, norm_eps, operand_dtype)
        res = self.kda_varlen(q, k, v, g, beta, cu_seqlens, init=init, has_init=has_init,
                              start_pos=start_pos, scale=scale, ckpt_interval=ckpt_interval)
        cu = _as_i32(cu_seqlens)
        W = np.asarray(_as_f32(w)).shape[1]
        sp = np.zeros(cu.size - 1, np.int64) if start_pos is None else np.asarray(_as_i32(start_pos), np.int64)
        ck_cu, ck_pos = res["ckpt_cu"], res["ckpt_pos"]
        cst = None if conv_state is None else np.asarray(_as_f32(conv_state), np.float32)
        hs = None if has_conv_state is None else np.asarray(_as_i32(has_conv_state))
        conv_ckpt = np.zeros((int(ck_cu[-1]), C, W - 1), self.real)
        for s in range(cu.size - 1):
            for j in range(int(ck_cu[s]), int(ck_cu[s + 1])):
                rel = int(ck_pos[j] - sp[s])   # tokens of the sequence before the checkpoint
                one_hist = None
                if cst is not None and (hs is None or hs[s]):
                    one_hist = cst[s:s + 1]
                _, st = self.conv_short(xa[cu[s]:cu[s + 1]], w, np.array([0, cu[s + 1] - cu[s]], np.int32),
                                        bias=bias, act=act, state=one_hist,
                                        advance_len=np.array([rel], np.int32))
                conv_ckpt[j] = st[0]
        res["conv_state"] = ns
        res["conv_ckpt"] = conv_ckpt
        res["q"], res["k"], res["v"] = q, k, v
        return res

    # -- fused decode step -------------------------------------------------
    def kda_decode_conv(self, x, w, g, beta, init, conv_state, *, H, d, bias=None, act=0,
                        qk_l2norm=1, norm_eps=1e-6, scale=1.0, out_gate=None, norm_weight=None,
                        out_norm_eps=1e-6):
        """The decode step with the short convolution in front of the
        recurrence, one token per sequence.

        x [N, 3 H d]: the token's raw projections, channels ordered q block,
        k block, v block, each [H, d]; w [3 H d, W]; bias [3 H d] or None;
        conv_state [N, 3 H d, W-1] (oldest first; zeros = no history);
        g [N, H, d]; beta [N, H]; init [N, H, d, d].

        Per sequence: y = conv(conv_state ++ x) (+ SiLU when act == 1), the
        same definition as :meth:`conv_short`, kept unrounded; q, k, v are the
        three blocks of y, per head; when qk_l2norm, q <- q / sqrt(|q|^2 + eps)
        and k likewise (per token and head); then one recurrence step from
        init as :meth:`kda_verify` with T_spec = 1.  With out_gate [N, H, d]
        and norm_weight [d], the output then passes through
        :func:`gated_rmsnorm`.

        Returns dict o [N, H, d], state [N, H, d, d], conv_state [N, 3 H d, W-1].
        """
        x = np.asarray(_as_f32(x), np.float64)
        N, C = x.shape
        if C != 3 * H * d:
            raise ValueError("x must have 3 * H * d channels")
        cu = np.arange(N + 1, dtype=np.int32)
        st = _as_f32(conv_state)
        y, ns = self.conv_short(x.astype(np.float32), w, cu, bias=bias, act=act, state=st)
        y = np.asarray(y, np.float64).reshape(N, 3, H, d)
        q, k, v = y[:, 0], y[:, 1], y[:, 2]
        if qk_l2norm:
            q = q / np.sqrt((q * q).sum(-1, keepdims=True) + norm_eps)
            k = k / np.sqrt((k * k).sum(-1, keepdims=True) + norm_eps)
        # the recurrence consumes float32 operands (the rounding of an fp64
        # conv output to float32 is far below every comparison tolerance)
        res = self.kda_verify(q[:, None].astype(np.float32), k[:, None].astype(np.float32),
                              v[:, None].astype(np.float32), _as_f32(g)[:, None],
                              _as_f32(beta)[:, None], init, scale=scale)
        o = res["o"][:, 0]
        if out_gate is not None:
            o = gated_rmsnorm(o, out_gate, norm_weight, out_norm_eps)
        return {"o": o, "state": res["committed"], "conv_state": ns}

    def kda_verify_conv(self, x, w, g, beta, init, conv_state, accepted_len=None, *, H, d, bias=None,
                        act=0, qk_l2norm=1, norm_eps=1e-6, scale=1.0, out_gate=None, norm_weight=None,
                        out_norm_eps=1e-6):
        """Speculative verify with the short convolution in front.

        x [N, Ts, 3 H d] (the Ts tokens' raw q | k | v projections);
        conv_state [N, 3 H d, W-1]; g [N, Ts, H, d]; beta [N, Ts, H];
        init [N, H, d, d]; accepted_len [N] or None (= Ts).

        Per sequence: y = conv(conv_state ++ x) over the Ts tokens (+ SiLU),
        q, k, v its blocks, q / k normalised per token and head when
        qk_l2norm, then :meth:`kda_verify`.  The conv history is advanced by
        the accepted length (the W-1 raw inputs ending at token L-1).  With
        out_gate [N, Ts, H, d] and norm_weight [d], every output passes
        through :func:`gated_rmsnorm`.

        Returns dict o [N, Ts, H, d], committed [N, H, d, d] (NaN where
        rejected), committed_len [N], conv_state [N, 3 H d, W-1] (NaN where
        rejected)."""
        x = np.asarray(_as_f32(x), np.float64)
        N, Ts, C = x.shape
        if C != 3 * H * d:
            raise ValueError("x must have 3 * H * d channels")
        st = np.asarray(_as_f32(conv_state), np.float32)
        W = st.shape[-1] + 1
        cu = (np.arange(N + 1) * Ts).astype(np.int32)
        y, _ = self.conv_short(x.reshape(N * Ts, C).astype(np.float32), w, cu, bias=bias, act=act,
                               state=st)
        y = np.asarray(y, np.float64).reshape(N, Ts, 3, H, d)
        q, k, v = y[:, :, 0], y[:, :, 1], y[:, :, 2]
        if qk_l2norm:
            q = q / np.sqrt((q * q).sum(-1, keepdims=True) + norm_eps)
            k = k / np.sqrt((k * k).sum(-1, keepdims=True) + norm_eps)
        res = self.kda_verify(q.astype(np.float32), k.astype(np.float32), v.astype(np.float32), g, beta,
                              init, accepted_len, scale=scale)
        # conv history after L tokens: the last W-1 entries of history ++ x[:L]
        L = np.full(N, Ts, np.int64) if accepted_len is None else np.asarray(_as_i32(accepted_len), np.int64)
        ns = np.full((N, C, W - 1), np.nan)
        for s in range(N):
            if 0 <= L[s] <= Ts:
                xb = np.concatenate([st[s].astype(np.float64), x[s, :L[s]].T], axis=1)  # [C, W-1+L]
                ns[s] = xb[:, -(W - 1):]
        out = dict(res)
        if out_gate is not None:
            out["o"] = gated_rmsnorm(res["o"], out_gate, norm_weight, out_norm_eps)
        out["conv_state"] = ns
        return out


def conv_operands(y, H, d, qk_l2norm, norm_eps, operand_dtype):
    """q, k, v of the chunked prefill from the conv output y [T, 3 H d]
    (fp64): the three channel blocks, per head; q and k divided by
    sqrt(|.|^2 + eps) per token and head when qk_l2norm; then each rounded
    to the recurrence's input type ("bf16": round to nearest even by torch's
    conversion, "f32": to float32).  Returns three [T, H, d] float32 arrays."""
    import torch
    T = y.shape[0]
    y = np.asarray(y, np.float64).reshape(T, 3, H, d)
    q, k, v = y[:, 0], y[:, 1], y[:, 2]
    if qk_l2norm:
        q = q / np.sqrt((q * q).sum(-1, keepdims=True) + norm_eps)
        k = k / np.sqrt((k * k).sum(-1, keepdims=True) + norm_eps)
    out = []
    for t in (q, k, v):
        t32 = np.ascontiguousarray(t, np.float32)
        if operand_dtype == "bf16":
            # fp64 -> fp32 -> bf16: the second rounding decides unless the
            # fp64 value lies within 2^-24 relative of a bf16 midpoint
            t32 = torch.from_numpy(t32).to(torch.bfloat16).float().numpy()
        elif operand_dtype != "f32":
            raise ValueError("operand_dtype must be 'bf16' or 'f32'")
        out.append(t32)
    return out


def gated_rmsnorm(o, z, weight, eps=1e-6):
    """Output gate of the fused decode step (one reading of the output norm
    and gate the Day-0 Integration page's fused decode kernel folds in,
    section "Separate Prefill/Decode Code Paths"): per token and head, the
    output o is divided by its root mean square over the d_v channels (eps
    added under the root), scaled channel-wise by the norm weight (shared by
    the heads), and multiplied by the logistic sigmoid of the gate input z.

    o [..., d] (any float), z [..., d], weight [d].  Returns float64."""
    o = np.asarray(o, np.float64)
    z = np.asarray(_as_f32(z), np.float64)
    wv = np.asarray(_as_f32(weight), np.float64)
    ms = np.mean(o * o, axis=-1, keepdims=True)
    return o / np.sqrt(ms + eps) * wv * (1.0 / (1.0 + np.exp(-z)))


_cache: dict = {}


def load(real: str = "f64", rebuild: bool = False) -> Oracle:
    """Load (building first if needed) the oracle of precision ``real``."""
    key = real
    if key in _cache and not rebuild:
        return _cache[key]
    path = HERE / _LIB_NAMES[real]
    if rebuild or not path.exists() or path.stat().st_mtime < SRC.stat().st_mtime:
        build(real)
    o = Oracle(path)
    _cache[key] = o
    return o


def load_mutant(mutant: int, outdir: Path, real: str = "f64") -> Oracle:
    """Build and load a planted-mistake variant (for pin tests)."""
    path = Path(outdir) / f"liboracle_{real}_m{mutant}.so"
    build(real, mutant=mutant, out=path)
    return Oracle(path)


__all__ = ["Oracle", "load", "load_mutant", "build", "gated_rmsnorm"]
