"""Thin ctypes binding of libkda (``include/kda.h``).

Argument marshalling only: each function fills the C argument struct from
torch tensors (device memory owned by torch) and calls the library on the
current HIP stream.  Every step of the computation runs in libkda's HIP
kernels; there is no fallback.  A non-OK status raises :class:`KDAError`.
"""

from __future__ import annotations

import ctypes
from pathlib import Path
from typing import Optional

PKG = Path(__file__).resolve().parent
LIB_PATH = PKG / "libkda.so"

KDA_BF16, KDA_F32 = 0, 1
KDA_OK = 0

c_vp = ctypes.c_void_p
c_i32 = ctypes.c_int32
c_i64 = ctypes.c_int64
c_f32 = ctypes.c_float
c_size = ctypes.c_size_t


class KDAError(RuntimeError):
    def __init__(self, status: int, name: str, detail: str):
        super().__init__(f"{name}: {detail}")
        self.status = status
        self.name = name


class ConvArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", c_size),
        ("x", c_vp), ("y", c_vp), ("weight", c_vp), ("bias", c_vp), ("cu_seqlens", c_vp),
        ("conv_pool", c_vp), ("src_slot", c_vp), ("dst_slot", c_vp), ("advance_len", c_vp),
        ("x_stride", c_i64), ("y_stride", c_i64), ("T_tot", c_i64), ("n_slots", c_i64),
        ("n_seq", c_i32), ("C", c_i32), ("W", c_i32), ("dtype", c_i32), ("act", c_i32),
        ("norm_d", c_i32), ("norm_channels", c_i64), ("norm_eps", c_f32), ("reserved", c_i32),
    ]


class PlanArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", c_size),
        ("cu_seqlens", c_vp), ("start_pos", c_vp), ("free_slots", c_vp), ("ckpt_cu", c_vp),
        ("ckpt_pos", c_vp), ("ckpt_slot", c_vp), ("n_total", c_vp),
        ("T_tot", c_i64),
        ("n_seq", c_i32), ("interval", c_i32), ("chunk", c_i32), ("cap", c_i32), ("n_free", c_i32),
        ("reserved", c_i32),
    ]


class PrefillArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", c_size),
        ("q", c_vp), ("k", c_vp), ("v", c_vp), ("g", c_vp), ("beta", c_vp), ("o", c_vp),
        ("cu_seqlens", c_vp), ("state_pool", c_vp), ("src_slot", c_vp), ("dst_slot", c_vp),
        ("start_pos", c_vp), ("ckpt_cu", c_vp), ("ckpt_slot", c_vp), ("ckpt_pos_out", c_vp),
        ("workspace", c_vp),
        ("q_stride", c_i64), ("k_stride", c_i64), ("v_stride", c_i64), ("g_stride", c_i64),
        ("beta_stride", c_i64), ("o_stride", c_i64),
        ("T_tot", c_i64), ("n_slots", c_i64), ("workspace_bytes", c_i64), ("n_ckpt", c_i64),
        ("n_seq", c_i32), ("H", c_i32), ("d_k", c_i32), ("d_v", c_i32), ("chunk", c_i32),
        ("in_dtype", c_i32), ("out_dtype", c_i32), ("ckpt_interval", c_i32), ("scale", c_f32),
        ("segment_len", c_i32),
    ]


class PrefillConvArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", c_size),
        ("prefill", PrefillArgs),
        ("x", c_vp), ("conv_weight", c_vp), ("conv_bias", c_vp), ("conv_pool", c_vp),
        ("conv_src_slot", c_vp), ("conv_dst_slot", c_vp), ("conv_ckpt_slot", c_vp), ("qkv", c_vp),
        ("x_stride", c_i64), ("n_conv_slots", c_i64), ("qkv_bytes", c_i64),
        ("W", c_i32), ("act", c_i32), ("qk_l2norm", c_i32), ("norm_eps", c_f32),
    ]


class DecodeArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", c_size),
        ("q", c_vp), ("k", c_vp), ("v", c_vp), ("g", c_vp), ("beta", c_vp), ("o", c_vp),
        ("state_pool", c_vp), ("src_slot", c_vp), ("dst_slot", c_vp),
        ("q_stride", c_i64), ("k_stride", c_i64), ("v_stride", c_i64), ("g_stride", c_i64),
        ("beta_stride", c_i64), ("o_stride", c_i64), ("n_slots", c_i64),
        ("n_seq", c_i32), ("H", c_i32), ("d_k", c_i32), ("d_v", c_i32),
        ("in_dtype", c_i32), ("out_dtype", c_i32), ("scale", c_f32), ("reserved", c_i32),
    ]


class DecodeConvArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", c_size),
        ("x", c_vp), ("conv_weight", c_vp), ("conv_bias", c_vp), ("conv_pool", c_vp),
        ("conv_src_slot", c_vp), ("conv_dst_slot", c_vp),
        ("g", c_vp), ("beta", c_vp), ("o", c_vp),
        ("state_pool", c_vp), ("src_slot", c_vp), ("dst_slot", c_vp),
        ("x_stride", c_i64), ("g_stride", c_i64), ("beta_stride", c_i64), ("o_stride", c_i64),
        ("n_slots", c_i64), ("n_conv_slots", c_i64),
        ("n_seq", c_i32), ("H", c_i32), ("d", c_i32), ("W", c_i32), ("act", c_i32),
        ("qk_l2norm", c_i32), ("norm_eps", c_f32), ("in_dtype", c_i32), ("out_dtype", c_i32),
        ("scale", c_f32),
        ("out_gate", c_vp), ("out_norm_weight", c_vp), ("out_gate_stride", c_i64),
        ("out_norm_eps", c_f32), ("reserved", c_i32),
    ]


class VerifyConvArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", c_size),
        ("x", c_vp), ("conv_weight", c_vp), ("conv_bias", c_vp), ("conv_pool", c_vp),
        ("conv_src_slot", c_vp), ("conv_dst_slot", c_vp),
        ("g", c_vp), ("beta", c_vp), ("o", c_vp),
        ("state_pool", c_vp), ("src_slot", c_vp), ("dst_slot", c_vp),
        ("accepted_len", c_vp), ("committed_len_out", c_vp),
        ("x_stride", c_i64), ("g_stride", c_i64), ("beta_stride", c_i64), ("o_stride", c_i64),
        ("n_slots", c_i64), ("n_conv_slots", c_i64),
        ("n_seq", c_i32), ("T_spec", c_i32), ("H", c_i32), ("d", c_i32), ("W", c_i32), ("act", c_i32),
        ("qk_l2norm", c_i32), ("norm_eps", c_f32), ("in_dtype", c_i32), ("out_dtype", c_i32),
        ("scale", c_f32), ("reserved", c_i32),
        ("out_gate", c_vp), ("out_norm_weight", c_vp), ("out_gate_stride", c_i64),
        ("out_norm_eps", c_f32), ("reserved2", c_i32),
    ]


class VerifyArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", c_size),
        ("q", c_vp), ("k", c_vp), ("v", c_vp), ("g", c_vp), ("beta", c_vp), ("o", c_vp),
        ("state_pool", c_vp), ("src_slot", c_vp), ("dst_slot", c_vp), ("accepted_len", c_vp),
        ("committed_len_out", c_vp),
        ("q_stride", c_i64), ("k_stride", c_i64), ("v_stride", c_i64), ("g_stride", c_i64),
        ("beta_stride", c_i64), ("o_stride", c_i64), ("n_slots", c_i64),
        ("n_seq", c_i32), ("T_spec", c_i32), ("H", c_i32), ("d_k", c_i32), ("d_v", c_i32),
        ("in_dtype", c_i32), ("out_dtype", c_i32), ("scale", c_f32),
    ]


EXPORTS = ["kda_status_str", "kda_abi_version", "kda_last_error", "kda_args_sizeof",
           "kda_conv_short", "kda_ckpt_plan", "kda_ckpt_plan_device", "kda_prefill_workspace_bytes",
           "kda_prefill_varlen", "kda_decode", "kda_verify", "kda_decode_conv", "kda_verify_conv",
           "kda_prefill_varlen_noalloc", "kda_prefill_noalloc_max_bytes", "kda_prefill_varlen_conv"]

_lib = None


def load_library(path: Optional[Path] = None):
    """Load libkda.so (built by ``hybrid_recurrent_serving_amd.build``).

    Raises FileNotFoundError when it is missing: the library is the only
    implementation, there is nothing to fall back to.
    """
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = Path(path) if path else LIB_PATH
    if not p.exists():
        raise FileNotFoundError(f"{p} is missing; build it with "
                                "`python -m hybrid_recurrent_serving_amd.build`")
    lib = ctypes.CDLL(str(p))
    lib.kda_status_str.restype = ctypes.c_char_p
    lib.kda_status_str.argtypes = [ctypes.c_int]
    lib.kda_abi_version.restype = ctypes.c_int
    lib.kda_last_error.restype = ctypes.c_char_p
    lib.kda_args_sizeof.restype = c_size
    lib.kda_args_sizeof.argtypes = [ctypes.c_int]
    lib.kda_conv_short.argtypes = [ctypes.POINTER(ConvArgs), c_vp]
    lib.kda_ckpt_plan.argtypes = [c_vp, c_vp, c_i32, c_i32, c_i32, c_vp, c_vp, c_i32, c_vp]
    lib.kda_ckpt_plan_device.argtypes = [ctypes.POINTER(PlanArgs), c_vp]
    lib.kda_prefill_workspace_bytes.restype = c_i64
    lib.kda_prefill_workspace_bytes.argtypes = [ctypes.POINTER(PrefillArgs)]
    lib.kda_prefill_varlen.argtypes = [ctypes.POINTER(PrefillArgs), c_vp]
    lib.kda_prefill_varlen_noalloc.argtypes = [ctypes.POINTER(PrefillArgs), c_vp]
    lib.kda_prefill_noalloc_max_bytes.restype = c_i64
    lib.kda_prefill_noalloc_max_bytes.argtypes = []
    lib.kda_decode.argtypes = [ctypes.POINTER(DecodeArgs), c_vp]
    lib.kda_verify.argtypes = [ctypes.POINTER(VerifyArgs), c_vp]
    lib.kda_decode_conv.argtypes = [ctypes.POINTER(DecodeConvArgs), c_vp]
    lib.kda_verify_conv.argtypes = [ctypes.POINTER(VerifyConvArgs), c_vp]
    lib.kda_prefill_varlen_conv.argtypes = [ctypes.POINTER(PrefillConvArgs), c_vp]
    for name in ("kda_conv_short", "kda_ckpt_plan", "kda_ckpt_plan_device", "kda_prefill_varlen", "kda_decode", "kda_verify",
                 "kda_decode_conv", "kda_verify_conv", "kda_prefill_varlen_noalloc", "kda_prefill_varlen_conv"):
        getattr(lib, name).restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def _check(status: int, lib=None):
    if status != KDA_OK:
        lib = lib or load_library()
        raise KDAError(status, lib.kda_status_str(status).decode(), lib.kda_last_error().decode())


# --------------------------------------------------------------------- helpers
def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return KDA_BF16
    if t.dtype == torch.float32:
        return KDA_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _tok_stride(t, inner_dims: int) -> int:
    """Element distance between consecutive tokens; the inner dims must be
    packed."""
    if t is None:
        return 0
    st = t.stride()
    exp = 1
    for d in range(t.dim() - 1, t.dim() - 1 - inner_dims, -1):
        if st[d] != exp:
            raise ValueError("inner [H, d] block must be contiguous")
        exp *= t.shape[d]
    return st[t.dim() - 1 - inner_dims]


def _expect(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


def _same_lead(named, lead, what):
    for name, t in named:
        if t is not None:
            _expect(tuple(t.shape[:len(lead)]) == tuple(lead),
                    f"{name}: leading shape {tuple(t.shape[:len(lead)])} != {tuple(lead)} ({what})")


def _device_tensors(**named):
    """Every pointer handed to the library must be device memory of the right
    integer type: a host pointer would be dereferenced by the GPU."""
    import torch
    for name, t in named.items():
        if t is None:
            continue
        _expect(isinstance(t, torch.Tensor) and t.is_cuda, f"{name} must be a GPU tensor")
        if name in ("cu_seqlens", "src_slot", "dst_slot", "advance_len", "start_pos", "ckpt_cu",
                    "ckpt_slot", "ckpt_pos_out", "accepted_len", "committed_len_out",
                    "free_slots", "ckpt_pos", "n_total"):
            _expect(t.dtype == torch.int32 and t.is_contiguous(), f"{name} must be contiguous int32")


def _same_dtype(ref, **named):
    for name, t in named.items():
        if t is not None:
            _expect(t.dtype == ref.dtype, f"{name}: dtype {t.dtype} != {ref.dtype}")


def _stream(stream) -> int:
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


# --------------------------------------------------------------------- API
def kda_status_str(status: int) -> str:
    return load_library().kda_status_str(status).decode()


def kda_abi_version() -> int:
    return load_library().kda_abi_version()


def kda_last_error() -> str:
    return load_library().kda_last_error().decode()


def kda_args_sizeof(which: int) -> int:
    return load_library().kda_args_sizeof(which)


def _conv_args(x, weight, cu_seqlens, conv_pool, src_slot, dst_slot, y, bias, act, advance_len, norm_d=0,
               norm_channels=0, norm_eps=1e-6):
    _expect(x.dim() == 2 and y.shape == x.shape, "x and y must be [T, C]")
    T, C = x.shape
    _expect(weight.dim() == 2 and weight.shape[0] == C, "weight must be [C, W]")
    W = weight.shape[1]
    _expect(conv_pool.dim() == 3 and conv_pool.shape[1] == C and conv_pool.shape[2] == W - 1,
            "conv_pool must be [n_slots, C, W-1]")
    n = cu_seqlens.numel() - 1
    _expect(src_slot.numel() >= n and dst_slot.numel() >= n, "slot arrays shorter than n_seq")
    _expect(bias is None or bias.numel() == C, "bias must be [C]")
    _expect(advance_len is None or advance_len.numel() >= n, "advance_len shorter than n_seq")
    _device_tensors(x=x, y=y, weight=weight, bias=bias, cu_seqlens=cu_seqlens, conv_pool=conv_pool,
                    src_slot=src_slot, dst_slot=dst_slot, advance_len=advance_len)
    _expect(weight.is_contiguous() and conv_pool.is_contiguous(), "weight / conv_pool must be contiguous")
    _same_dtype(x, y=y, weight=weight, bias=bias, conv_pool=conv_pool)
    a = ConvArgs()
    a.struct_size = ctypes.sizeof(ConvArgs)
    a.x, a.y, a.weight, a.bias = _ptr(x), _ptr(y), _ptr(weight), _ptr(bias)
    a.cu_seqlens, a.conv_pool = _ptr(cu_seqlens), _ptr(conv_pool)
    a.src_slot, a.dst_slot, a.advance_len = _ptr(src_slot), _ptr(dst_slot), _ptr(advance_len)
    a.x_stride, a.y_stride = x.stride(0), y.stride(0)
    a.T_tot, a.n_slots = x.shape[0], conv_pool.shape[0]
    a.n_seq, a.C, a.W = cu_seqlens.numel() - 1, x.shape[1], weight.shape[1]
    a.dtype, a.act = _dtype_code(x), act
    a.norm_d, a.norm_channels, a.norm_eps = int(norm_d), int(norm_channels), float(norm_eps)
    return a


def kda_conv_short(x, weight, cu_seqlens, conv_pool, src_slot, dst_slot, *, y=None, bias=None,
                   act: int = 0, advance_len=None, norm_d: int = 0, norm_channels: int = 0,
                   norm_eps: float = 1e-6, stream=None):
    """Short causal conv.  x [T, C]; weight [C, W]; conv_pool [S, C, W-1].
    With norm_d > 0, channels [0, norm_channels) are L2-normalised per token
    in groups of norm_d.  Returns y (allocated by torch when not given)."""
    import torch
    if y is None:
        y = torch.empty_like(x)
    a = _conv_args(x, weight, cu_seqlens, conv_pool, src_slot, dst_slot, y, bias, act, advance_len, norm_d,
                   norm_channels, norm_eps)
    _check(load_library().kda_conv_short(ctypes.byref(a), _stream(stream)))
    return y


class Prepared:
    """An argument struct checked once and bound to its entry point, for
    loops that launch the same call on the same buffers: calling it enqueues
    the call again (only the status is checked).  It holds references to the
    tensors whose addresses it carries."""

    __slots__ = ("_fn", "_args", "_keep")

    def __init__(self, fn, args, keep):
        self._fn, self._args, self._keep = fn, args, keep

    def __call__(self, stream=None):
        _check(self._fn(ctypes.byref(self._args), _stream(stream)))


def prepare_decode(q, k, v, g, beta, o, state_pool, src_slot, dst_slot, *, scale=1.0) -> Prepared:
    """kda_decode with fixed buffers, as a Prepared call."""
    a = _decode_args(q, k, v, g, beta, o, state_pool, src_slot, dst_slot, scale)
    return Prepared(load_library().kda_decode, a, (q, k, v, g, beta, o, state_pool, src_slot, dst_slot))


def prepare_conv_short(x, weight, cu_seqlens, conv_pool, src_slot, dst_slot, *, y, bias=None, act: int = 0,
                       advance_len=None, norm_d: int = 0, norm_channels: int = 0,
                       norm_eps: float = 1e-6) -> Prepared:
    """kda_conv_short with fixed buffers, as a Prepared call."""
    a = _conv_args(x, weight, cu_seqlens, conv_pool, src_slot, dst_slot, y, bias, act, advance_len, norm_d,
                   norm_channels, norm_eps)
    return Prepared(load_library().kda_conv_short, a,
                    (x, weight, cu_seqlens, conv_pool, src_slot, dst_slot, y, bias, advance_len))


def kda_ckpt_plan(cu_seqlens, interval: int, chunk: int, start_pos=None):
    """Host checkpoint plan.  cu_seqlens / start_pos: host int sequences.
    Returns (ckpt_cu list, ckpt_pos list)."""
    import numpy as np
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, np.int32))
    sp = None if start_pos is None else np.ascontiguousarray(np.asarray(start_pos, np.int32))
    n = cu.size - 1
    ck_cu = np.zeros(n + 1, np.int32)
    total = ctypes.c_int32(0)
    lib = load_library()
    vp = lambda a: None if a is None else a.ctypes.data_as(c_vp)  # noqa: E731
    st = lib.kda_ckpt_plan(vp(cu), vp(sp), n, int(interval), int(chunk), vp(ck_cu), None, 0,
                           ctypes.byref(total))
    if st not in (KDA_OK, 9):
        _check(st, lib)
    pos = np.zeros(max(total.value, 1), np.int32)
    _check(lib.kda_ckpt_plan(vp(cu), vp(sp), n, int(interval), int(chunk), vp(ck_cu), vp(pos),
                             total.value, ctypes.byref(total)), lib)
    return ck_cu.tolist(), pos[:total.value].tolist()


def kda_ckpt_plan_device(cu_seqlens, interval: int, chunk: int, T_tot: int, *, cap: int,
                         start_pos=None, free_slots=None, ckpt_cu=None, ckpt_pos=None,
                         ckpt_slot=None, n_total=None, stream=None):
    """Device checkpoint plan; see include/kda.h for the contract.

    cu_seqlens / start_pos / free_slots: device int32.  Outputs that are None
    are allocated here (int32, on cu_seqlens' device); pass them all to keep
    the call allocation-free, e.g. inside graph capture.  ``ckpt_pos`` and
    ``ckpt_slot`` hold ``cap`` entries.  Returns (ckpt_cu, ckpt_pos,
    ckpt_slot, n_total)."""
    import torch
    n_seq = cu_seqlens.numel() - 1
    _expect(n_seq >= 0 and cap >= 0, "cu_seqlens needs n_seq + 1 entries; cap >= 0")
    dev = cu_seqlens.device

    def out(t, n):
        return torch.empty(n, dtype=torch.int32, device=dev) if t is None else t

    ckpt_cu, ckpt_pos = out(ckpt_cu, n_seq + 1), out(ckpt_pos, max(cap, 1))
    ckpt_slot, n_total = out(ckpt_slot, max(cap, 1)), out(n_total, 1)
    _device_tensors(cu_seqlens=cu_seqlens, start_pos=start_pos, free_slots=free_slots, ckpt_cu=ckpt_cu,
                    ckpt_pos=ckpt_pos, ckpt_slot=ckpt_slot, n_total=n_total)
    _expect(ckpt_cu.numel() >= n_seq + 1 and n_total.numel() >= 1, "ckpt_cu / n_total too small")
    _expect(ckpt_pos.numel() >= cap and ckpt_slot.numel() >= cap, "ckpt_pos / ckpt_slot hold fewer than cap")
    _expect(start_pos is None or start_pos.numel() >= n_seq, "start_pos holds fewer than n_seq")
    a = PlanArgs()
    a.struct_size = ctypes.sizeof(PlanArgs)
    a.cu_seqlens, a.start_pos, a.free_slots = _ptr(cu_seqlens), _ptr(start_pos), _ptr(free_slots)
    a.ckpt_cu, a.ckpt_pos, a.ckpt_slot, a.n_total = _ptr(ckpt_cu), _ptr(ckpt_pos), _ptr(ckpt_slot), _ptr(n_total)
    a.T_tot, a.n_seq, a.interval, a.chunk, a.cap = int(T_tot), n_seq, int(interval), int(chunk), int(cap)
    a.n_free = 0 if free_slots is None else free_slots.numel()
    _check(load_library().kda_ckpt_plan_device(ctypes.byref(a), _stream(stream)))
    return ckpt_cu, ckpt_pos, ckpt_slot, n_total


def _prefill_args(q, k, v, g, beta, o, cu_seqlens, state_pool, src_slot, dst_slot, chunk,
                  start_pos, ckpt_interval, ckpt_cu, ckpt_slot, ckpt_pos_out, workspace, scale,
                  segment_len=0):
    import torch
    _expect(q.dim() == 3 and v.dim() == 3 and beta.dim() == 2, "q/k/v/g [T, H, d], beta [T, H]")
    T, H, dk = q.shape
    _same_lead([("k", k), ("g", g)], (T, H, dk), "q")
    _same_lead([("v", v), ("o", o)], (T, H, v.shape[2]), "v")
    _same_lead([("beta", beta)], (T, H), "q")
    _expect(state_pool.dim() == 4 and tuple(state_pool.shape[1:]) == (H, dk, v.shape[2]),
            "state_pool must be [n_slots, H, d_k, d_v]")
    n = cu_seqlens.numel() - 1
    _expect(src_slot.numel() >= n and dst_slot.numel() >= n, "slot arrays shorter than n_seq")
    _expect(start_pos is None or start_pos.numel() >= n, "start_pos shorter than n_seq")
    _expect(ckpt_cu is None or ckpt_cu.numel() >= n + 1, "ckpt_cu shorter than n_seq + 1")
    _expect(ckpt_pos_out is None or ckpt_slot is None or ckpt_pos_out.numel() >= ckpt_slot.numel(),
            "ckpt_pos_out shorter than ckpt_slot")
    _device_tensors(q=q, k=k, v=v, g=g, beta=beta, o=o, cu_seqlens=cu_seqlens, state_pool=state_pool,
                    src_slot=src_slot, dst_slot=dst_slot, start_pos=start_pos, ckpt_cu=ckpt_cu,
                    ckpt_slot=ckpt_slot, ckpt_pos_out=ckpt_pos_out, workspace=workspace)
    _same_dtype(q, k=k, v=v, g=g, beta=beta)
    _expect(state_pool.dtype == torch.float32 and state_pool.is_contiguous(),
            "state_pool must be contiguous float32")
    a = PrefillArgs()
    a.struct_size = ctypes.sizeof(PrefillArgs)
    a.q, a.k, a.v, a.g, a.beta, a.o = map(_ptr, (q, k, v, g, beta, o))
    a.cu_seqlens, a.state_pool = _ptr(cu_seqlens), _ptr(state_pool)
    a.src_slot, a.dst_slot, a.start_pos = _ptr(src_slot), _ptr(dst_slot), _ptr(start_pos)
    a.ckpt_cu, a.ckpt_slot, a.ckpt_pos_out = _ptr(ckpt_cu), _ptr(ckpt_slot), _ptr(ckpt_pos_out)
    a.workspace = _ptr(workspace)
    a.workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    a.q_stride, a.k_stride, a.v_stride = _tok_stride(q, 2), _tok_stride(k, 2), _tok_stride(v, 2)
    a.g_stride, a.beta_stride, a.o_stride = _tok_stride(g, 2), _tok_stride(beta, 1), _tok_stride(o, 2)
    a.T_tot, a.n_slots = q.shape[0], state_pool.shape[0]
    a.n_ckpt = 0 if ckpt_slot is None else ckpt_slot.numel()
    a.n_seq, a.H, a.d_k, a.d_v = cu_seqlens.numel() - 1, q.shape[1], q.shape[2], v.shape[2]
    a.chunk = chunk
    a.in_dtype, a.out_dtype = _dtype_code(q), _dtype_code(o)
    a.ckpt_interval, a.scale = ckpt_interval, scale
    a.segment_len = int(segment_len)
    return a


def kda_prefill_workspace_bytes(q, k, v, g, beta, o, cu_seqlens, state_pool, src_slot, dst_slot,
                                *, chunk=64, start_pos=None, ckpt_interval=0, ckpt_cu=None,
                                ckpt_slot=None, scale=1.0, segment_len=0) -> int:
    a = _prefill_args(q, k, v, g, beta, o, cu_seqlens, state_pool, src_slot, dst_slot, chunk,
                      start_pos, ckpt_interval, ckpt_cu, ckpt_slot, None, None, scale, segment_len)
    n = load_library().kda_prefill_workspace_bytes(ctypes.byref(a))
    if n < 0:
        raise KDAError(8, "KDA_ERR_ARG", kda_last_error())
    return n


def kda_prefill_varlen(q, k, v, g, beta, o, cu_seqlens, state_pool, src_slot, dst_slot, *,
                       chunk=64, start_pos=None, ckpt_interval=0, ckpt_cu=None, ckpt_slot=None,
                       ckpt_pos_out=None, workspace=None, scale=1.0, segment_len=0, stream=None):
    """Chunked varlen prefill; see include/kda.h for the argument contract.

    ``workspace``: a device tensor of at least kda_prefill_workspace_bytes()
    bytes, needed when a sequence may be split (``segment_len``).  When it is
    None and the call needs one, a byte tensor is allocated on q's device."""
    a = _prefill_args(q, k, v, g, beta, o, cu_seqlens, state_pool, src_slot, dst_slot, chunk,
                      start_pos, ckpt_interval, ckpt_cu, ckpt_slot, ckpt_pos_out, workspace, scale,
                      segment_len)
    lib = load_library()
    if workspace is None:
        need = lib.kda_prefill_workspace_bytes(ctypes.byref(a))
        if need > 0:
            import torch
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
            a.workspace, a.workspace_bytes = _ptr(workspace), need
    _check(lib.kda_prefill_varlen(ctypes.byref(a), _stream(stream)))
    return o


def kda_prefill_varlen_noalloc(q, k, v, g, beta, o, cu_seqlens, state_pool, src_slot, dst_slot, *,
                               chunk=64, start_pos=None, ckpt_interval=0, ckpt_cu=None, ckpt_slot=None,
                               ckpt_pos_out=None, scale=1.0, segment_len=0, stream=None):
    """kda_prefill_varlen without a workspace: the library's own scratch array
    serves the segment scan, and nothing is allocated (see include/kda.h)."""
    a = _prefill_args(q, k, v, g, beta, o, cu_seqlens, state_pool, src_slot, dst_slot, chunk,
                      start_pos, ckpt_interval, ckpt_cu, ckpt_slot, ckpt_pos_out, None, scale,
                      segment_len)
    _check(load_library().kda_prefill_varlen_noalloc(ctypes.byref(a), _stream(stream)))
    return o


def kda_prefill_varlen_conv(x, conv_weight, conv_pool, conv_src_slot, conv_dst_slot, g, beta, o, cu_seqlens,
                            state_pool, src_slot, dst_slot, *, qkv=None, conv_bias=None, act: int = 0,
                            qk_l2norm: bool = True, norm_eps: float = 1e-6, chunk=64, start_pos=None,
                            ckpt_interval=0, ckpt_cu=None, ckpt_slot=None, ckpt_pos_out=None, workspace=None,
                            scale=1.0, segment_len=0, conv_ckpt_slot=None, stream=None):
    """Prefill from the tokens' raw projections: the short conv (+ SiLU),
    per-head q / k normalisation and the chunked prefill (include/kda.h).
    ``conv_ckpt_slot`` [n_ckpt]: conv pool slots that receive the conv
    history at each interval checkpoint.

    x [T, 3 H d] (q | k | v projections, packed rows); conv_weight
    [3 H d, W]; conv_pool [n_conv_slots, 3 H d, W-1]; g [T, H, d]; beta
    [T, H]; o [T, H, d].  ``qkv`` [T, 3 H d] (x's dtype, packed) receives the
    formed q | k | v; allocated when None.  ``workspace`` as
    kda_prefill_varlen.  Returns (o, qkv)."""
    import torch
    _expect(x.dim() == 2 and g.dim() == 3, "x [T, 3 H d], g [T, H, d]")
    T, C = x.shape
    H, d = g.shape[1], g.shape[2]
    _expect(C == 3 * H * d, "x must have 3 H d channels")
    _expect(x.stride(1) == 1, "x rows must be contiguous")
    W = conv_weight.shape[1]
    _expect(tuple(conv_weight.shape) == (C, W) and conv_weight.is_contiguous(), "conv_weight must be [3 H d, W]")
    _expect(conv_pool.dim() == 3 and tuple(conv_pool.shape[1:]) == (C, W - 1) and conv_pool.is_contiguous(),
            "conv_pool must be [n_conv_slots, 3 H d, W-1]")
    if qkv is None:
        qkv = torch.empty(T, C, dtype=x.dtype, device=x.device)
    _expect(tuple(qkv.shape) == (T, C) and qkv.is_contiguous() and qkv.dtype == x.dtype,
            "qkv must be a packed [T, 3 H d] tensor of x's dtype")
    _device_tensors(x=x, conv_weight=conv_weight, conv_pool=conv_pool, conv_src_slot=conv_src_slot,
                    conv_dst_slot=conv_dst_slot, conv_bias=conv_bias, qkv=qkv, conv_ckpt_slot=conv_ckpt_slot)
    _expect(conv_ckpt_slot is None or ckpt_slot is None or conv_ckpt_slot.numel() >= ckpt_slot.numel(),
            "conv_ckpt_slot shorter than ckpt_slot")
    _same_dtype(x, conv_weight=conv_weight, conv_pool=conv_pool, g=g)
    if conv_bias is not None:
        _same_dtype(x, conv_bias=conv_bias)
    HD = H * d
    views = [qkv[:, i * HD:(i + 1) * HD].view(T, H, d) if T else qkv.new_empty(0, H, d) for i in range(3)]
    pa = _prefill_args(views[0], views[1], views[2], g, beta, o, cu_seqlens, state_pool, src_slot, dst_slot,
                       chunk, start_pos, ckpt_interval, ckpt_cu, ckpt_slot, ckpt_pos_out, workspace, scale,
                       segment_len)
    lib = load_library()
    if workspace is None:
        need = lib.kda_prefill_workspace_bytes(ctypes.byref(pa))
        if need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
            pa.workspace, pa.workspace_bytes = _ptr(workspace), need
    # q / k / v are formed by the library inside qkv
    pa.q = pa.k = pa.v = None
    pa.q_stride = pa.k_stride = pa.v_stride = 0
    a = PrefillConvArgs()
    a.struct_size = ctypes.sizeof(PrefillConvArgs)
    a.prefill = pa
    a.x, a.conv_weight, a.conv_bias, a.conv_pool = _ptr(x), _ptr(conv_weight), _ptr(conv_bias), _ptr(conv_pool)
    a.conv_src_slot, a.conv_dst_slot, a.qkv = _ptr(conv_src_slot), _ptr(conv_dst_slot), _ptr(qkv)
    a.conv_ckpt_slot = _ptr(conv_ckpt_slot)
    a.x_stride = x.stride(0) if T else 0
    a.n_conv_slots = conv_pool.shape[0]
    a.qkv_bytes = qkv.numel() * qkv.element_size()
    a.W, a.act, a.qk_l2norm, a.norm_eps = W, int(act), int(qk_l2norm), float(norm_eps)
    _check(lib.kda_prefill_varlen_conv(ctypes.byref(a), _stream(stream)))
    return o, qkv


def kda_prefill_noalloc_max_bytes() -> int:
    return int(load_library().kda_prefill_noalloc_max_bytes())


def _decode_args(q, k, v, g, beta, o, state_pool, src_slot, dst_slot, scale):
    import torch
    _expect(q.dim() == 3 and v.dim() == 3 and beta.dim() == 2, "q/k/v/g [N, H, d], beta [N, H]")
    N, H, dk = q.shape
    _same_lead([("k", k), ("g", g)], (N, H, dk), "q")
    _same_lead([("v", v), ("o", o)], (N, H, v.shape[2]), "v")
    _same_lead([("beta", beta)], (N, H), "q")
    _expect(state_pool.dim() == 4 and tuple(state_pool.shape[1:]) == (H, dk, v.shape[2]),
            "state_pool must be [n_slots, H, d_k, d_v]")
    _expect(src_slot.numel() >= N and dst_slot.numel() >= N, "slot arrays shorter than n_seq")
    _device_tensors(q=q, k=k, v=v, g=g, beta=beta, o=o, state_pool=state_pool, src_slot=src_slot,
                    dst_slot=dst_slot)
    _same_dtype(q, k=k, v=v, g=g, beta=beta)
    _expect(state_pool.dtype == torch.float32 and state_pool.is_contiguous(),
            "state_pool must be contiguous float32")
    a = DecodeArgs()
    a.struct_size = ctypes.sizeof(DecodeArgs)
    a.q, a.k, a.v, a.g, a.beta, a.o = map(_ptr, (q, k, v, g, beta, o))
    a.state_pool, a.src_slot, a.dst_slot = _ptr(state_pool), _ptr(src_slot), _ptr(dst_slot)
    a.q_stride, a.k_stride, a.v_stride = _tok_stride(q, 2), _tok_stride(k, 2), _tok_stride(v, 2)
    a.g_stride, a.beta_stride, a.o_stride = _tok_stride(g, 2), _tok_stride(beta, 1), _tok_stride(o, 2)
    a.n_slots = state_pool.shape[0]
    a.n_seq, a.H, a.d_k, a.d_v = q.shape[0], q.shape[1], q.shape[2], v.shape[2]
    a.in_dtype, a.out_dtype, a.scale = _dtype_code(q), _dtype_code(o), scale
    return a


def kda_decode(q, k, v, g, beta, o, state_pool, src_slot, dst_slot, *, scale=1.0, stream=None):
    """One token per sequence.  q, k, v, g [N, H, d]; beta [N, H]; o [N, H, d]."""
    a = _decode_args(q, k, v, g, beta, o, state_pool, src_slot, dst_slot, scale)
    _check(load_library().kda_decode(ctypes.byref(a), _stream(stream)))
    return o


def _out_gate_fields(a, out_gate, out_norm_weight, out_norm_eps, lead, H, d, ref):
    """The optional gated RMS norm of the fused steps' output: out_gate
    [*lead, H, d] (packed inner dims), out_norm_weight [d], same dtype as the
    inputs."""
    if out_gate is None:
        _expect(out_norm_weight is None, "out_norm_weight given without out_gate")
        return
    _expect(out_norm_weight is not None, "out_gate needs out_norm_weight")
    _expect(tuple(out_gate.shape) == tuple(lead) + (H, d), f"out_gate must be {tuple(lead) + (H, d)}")
    _expect(out_norm_weight.numel() == d and out_norm_weight.is_contiguous(), "out_norm_weight must be [d]")
    _device_tensors(out_gate=out_gate, out_norm_weight=out_norm_weight)
    _same_dtype(ref, out_gate=out_gate, out_norm_weight=out_norm_weight)
    a.out_gate, a.out_norm_weight = _ptr(out_gate), _ptr(out_norm_weight)
    a.out_gate_stride = _tok_stride(out_gate, 2)
    a.out_norm_eps = float(out_norm_eps)


def _decode_conv_args(x, conv_weight, conv_pool, conv_src_slot, conv_dst_slot, g, beta, o, state_pool,
                      src_slot, dst_slot, conv_bias, act, qk_l2norm, norm_eps, scale, out_gate=None,
                      out_norm_weight=None, out_norm_eps=1e-6):
    import torch
    _expect(x.dim() == 2 and g.dim() == 3 and beta.dim() == 2 and o.dim() == 3,
            "x [N, 3 H d], g [N, H, d], beta [N, H], o [N, H, d]")
    N, H, d = g.shape
    _expect(x.shape[0] == N and x.shape[1] == 3 * H * d, "x must be [N, 3 H d]")
    _same_lead([("o", o)], (N, H, d), "g")
    _same_lead([("beta", beta)], (N, H), "g")
    _expect(conv_weight.dim() == 2 and conv_weight.shape[0] == 3 * H * d and conv_weight.is_contiguous(),
            "conv_weight must be contiguous [3 H d, W]")
    W = conv_weight.shape[1]
    _expect(conv_pool.dim() == 3 and tuple(conv_pool.shape[1:]) == (3 * H * d, W - 1)
            and conv_pool.is_contiguous(), "conv_pool must be contiguous [n_slots, 3 H d, W-1]")
    _expect(conv_bias is None or (conv_bias.numel() == 3 * H * d and conv_bias.is_contiguous()),
            "conv_bias must be contiguous [3 H d]")
    _expect(state_pool.dim() == 4 and tuple(state_pool.shape[1:]) == (H, d, d)
            and state_pool.dtype == torch.float32 and state_pool.is_contiguous(),
            "state_pool must be contiguous float32 [n_slots, H, d, d]")
    for nm, t in (("src_slot", src_slot), ("dst_slot", dst_slot), ("conv_src_slot", conv_src_slot),
                  ("conv_dst_slot", conv_dst_slot)):
        _expect(t.numel() >= N, f"{nm} shorter than n_seq")
    _device_tensors(x=x, conv_weight=conv_weight, conv_pool=conv_pool, conv_src_slot=conv_src_slot,
                    conv_dst_slot=conv_dst_slot, g=g, beta=beta, o=o, state_pool=state_pool,
                    src_slot=src_slot, dst_slot=dst_slot)
    _same_dtype(x, conv_weight=conv_weight, conv_pool=conv_pool, g=g, beta=beta)
    _expect(x.stride(1) == 1, "x rows must be contiguous")
    a = DecodeConvArgs()
    a.struct_size = ctypes.sizeof(DecodeConvArgs)
    a.x, a.conv_weight, a.conv_bias, a.conv_pool = map(_ptr, (x, conv_weight, conv_bias, conv_pool))
    a.conv_src_slot, a.conv_dst_slot = _ptr(conv_src_slot), _ptr(conv_dst_slot)
    a.g, a.beta, a.o = _ptr(g), _ptr(beta), _ptr(o)
    a.state_pool, a.src_slot, a.dst_slot = _ptr(state_pool), _ptr(src_slot), _ptr(dst_slot)
    a.x_stride = x.stride(0)
    a.g_stride, a.beta_stride, a.o_stride = _tok_stride(g, 2), _tok_stride(beta, 1), _tok_stride(o, 2)
    a.n_slots, a.n_conv_slots = state_pool.shape[0], conv_pool.shape[0]
    a.n_seq, a.H, a.d, a.W = N, H, d, W
    a.act, a.qk_l2norm, a.norm_eps = int(act), int(qk_l2norm), float(norm_eps)
    a.in_dtype, a.out_dtype, a.scale = _dtype_code(x), _dtype_code(o), scale
    _out_gate_fields(a, out_gate, out_norm_weight, out_norm_eps, (N,), H, d, x)
    return a


def kda_decode_conv(x, conv_weight, conv_pool, conv_src_slot, conv_dst_slot, g, beta, o, state_pool,
                    src_slot, dst_slot, *, conv_bias=None, act: int = 0, qk_l2norm: bool = True,
                    norm_eps: float = 1e-6, scale=1.0, out_gate=None, out_norm_weight=None,
                    out_norm_eps: float = 1e-6, stream=None):
    """Decode step with the short convolution fused in.  x [N, 3 H d] (q | k | v
    projections of the token); conv_weight [3 H d, W]; conv_pool
    [n_conv_slots, 3 H d, W-1]; g [N, H, d]; beta [N, H]; o [N, H, d];
    out_gate [N, H, d] and out_norm_weight [d] (optional gated RMS norm of o)."""
    a = _decode_conv_args(x, conv_weight, conv_pool, conv_src_slot, conv_dst_slot, g, beta, o, state_pool,
                          src_slot, dst_slot, conv_bias, act, qk_l2norm, norm_eps, scale, out_gate,
                          out_norm_weight, out_norm_eps)
    _check(load_library().kda_decode_conv(ctypes.byref(a), _stream(stream)))
    return o


def prepare_decode_conv(x, conv_weight, conv_pool, conv_src_slot, conv_dst_slot, g, beta, o, state_pool,
                        src_slot, dst_slot, *, conv_bias=None, act: int = 0, qk_l2norm: bool = True,
                        norm_eps: float = 1e-6, scale=1.0, out_gate=None, out_norm_weight=None,
                        out_norm_eps: float = 1e-6) -> Prepared:
    """kda_decode_conv with fixed buffers, as a Prepared call."""
    a = _decode_conv_args(x, conv_weight, conv_pool, conv_src_slot, conv_dst_slot, g, beta, o, state_pool,
                          src_slot, dst_slot, conv_bias, act, qk_l2norm, norm_eps, scale, out_gate,
                          out_norm_weight, out_norm_eps)
    return Prepared(load_library().kda_decode_conv, a,
                    (x, conv_weight, conv_pool, conv_src_slot, conv_dst_slot, g, beta, o, state_pool,
                     src_slot, dst_slot, conv_bias, out_gate, out_norm_weight))


def _verify_conv_args(x, conv_weight, conv_pool, conv_src_slot, conv_dst_slot, g, beta, state_pool, src_slot,
                      dst_slot, o, accepted_len, committed_len_out, conv_bias, act, qk_l2norm, norm_eps, scale,
                      out_gate, out_norm_weight, out_norm_eps):
    import torch
    _expect(x.dim() == 3 and g.dim() == 4 and beta.dim() == 3,
            "x [N, T_spec, 3 H d], g [N, T_spec, H, d], beta [N, T_spec, H]")
    N, Ts, H, d = g.shape
    _expect(tuple(x.shape) == (N, Ts, 3 * H * d), "x must be [N, T_spec, 3 H d]")
    _same_lead([("beta", beta)], (N, Ts, H), "g")
    _same_lead([("o", o)], (N, Ts, H, d), "g")
    _expect(conv_weight.dim() == 2 and conv_weight.shape[0] == 3 * H * d and conv_weight.is_contiguous(),
            "conv_weight must be contiguous [3 H d, W]")
    W = conv_weight.shape[1]
    _expect(conv_pool.dim() == 3 and tuple(conv_pool.shape[1:]) == (3 * H * d, W - 1)
            and conv_pool.is_contiguous(), "conv_pool must be contiguous [n_slots, 3 H d, W-1]")
    _expect(conv_bias is None or (conv_bias.numel() == 3 * H * d and conv_bias.is_contiguous()),
            "conv_bias must be contiguous [3 H d]")
    _expect(state_pool.dim() == 4 and tuple(state_pool.shape[1:]) == (H, d, d)
            and state_pool.dtype == torch.float32 and state_pool.is_contiguous(),
            "state_pool must be contiguous float32 [n_slots, H, d, d]")
    for nm, t in (("src_slot", src_slot), ("dst_slot", dst_slot), ("conv_src_slot", conv_src_slot),
                  ("conv_dst_slot", conv_dst_slot)):
        _expect(t.numel() >= N, f"{nm} shorter than n_seq")
    _expect(accepted_len is None or accepted_len.numel() >= N, "accepted_len shorter than n_seq")
    _expect(committed_len_out is None or committed_len_out.numel() >= N, "committed_len_out shorter than n_seq")
    _expect(x.stride(2) == 1 and x.stride(0) == Ts * x.stride(1), "x must be [N, T_spec, C] with token rows")
    _device_tensors(x=x, conv_weight=conv_weight, conv_pool=conv_pool, conv_src_slot=conv_src_slot,
                    conv_dst_slot=conv_dst_slot, g=g, beta=beta, o=o, state_pool=state_pool,
                    src_slot=src_slot, dst_slot=dst_slot, accepted_len=accepted_len,
                    committed_len_out=committed_len_out)
    _same_dtype(x, conv_weight=conv_weight, conv_pool=conv_pool, g=g, beta=beta)
    a = VerifyConvArgs()
    a.struct_size = ctypes.sizeof(VerifyConvArgs)
    a.x, a.conv_weight, a.conv_bias, a.conv_pool = map(_ptr, (x, conv_weight, conv_bias, conv_pool))
    a.conv_src_slot, a.conv_dst_slot = _ptr(conv_src_slot), _ptr(conv_dst_slot)
    a.g, a.beta, a.o = _ptr(g), _ptr(beta), _ptr(o)
    a.state_pool, a.src_slot, a.dst_slot = _ptr(state_pool), _ptr(src_slot), _ptr(dst_slot)
    a.accepted_len, a.committed_len_out = _ptr(accepted_len), _ptr(committed_len_out)
    a.x_stride = x.stride(1)
    for nm, t in (("g", g), ("beta", beta), ("o", o)):
        _expect(t is None or t.stride(0) == Ts * t.stride(1), f"{nm}: sequence stride must be T_spec tokens")
    a.g_stride, a.beta_stride = _tok_stride(g, 2), _tok_stride(beta, 1)
    a.o_stride = _tok_stride(o, 2) if o is not None else 0
    a.n_slots, a.n_conv_slots = state_pool.shape[0], conv_pool.shape[0]
    a.n_seq, a.T_spec, a.H, a.d, a.W = N, Ts, H, d, W
    a.act, a.qk_l2norm, a.norm_eps = int(act), int(qk_l2norm), float(norm_eps)
    a.in_dtype = _dtype_code(x)
    a.out_dtype = _dtype_code(o) if o is not None else KDA_BF16
    a.scale = scale
    if out_gate is not None:
        _expect(out_gate.stride(0) == Ts * out_gate.stride(1), "out_gate: sequence stride must be T_spec tokens")
    _out_gate_fields(a, out_gate, out_norm_weight, out_norm_eps, (N, Ts), H, d, x)
    return a


def kda_verify_conv(x, conv_weight, conv_pool, conv_src_slot, conv_dst_slot, g, beta, state_pool, src_slot,
                    dst_slot, *, o=None, accepted_len=None, committed_len_out=None, conv_bias=None,
                    act: int = 0, qk_l2norm: bool = True, norm_eps: float = 1e-6, scale=1.0, out_gate=None,
                    out_norm_weight=None, out_norm_eps: float = 1e-6, stream=None):
    """Speculative verify with the short convolution fused in.  x [N, T_spec,
    3 H d] (q | k | v projections of the tokens); g [N, T_spec, H, d]; beta
    [N, T_spec, H]; o [N, T_spec, H, d] or None; conv and state pools as
    kda_decode_conv; out_gate [N, T_spec, H, d] and out_norm_weight [d]
    (optional gated RMS norm of every output)."""
    a = _verify_conv_args(x, conv_weight, conv_pool, conv_src_slot, conv_dst_slot, g, beta, state_pool, src_slot,
                          dst_slot, o, accepted_len, committed_len_out, conv_bias, act, qk_l2norm, norm_eps, scale,
                          out_gate, out_norm_weight, out_norm_eps)
    _check(load_library().kda_verify_conv(ctypes.byref(a), _stream(stream)))
    return o


def prepare_verify_conv(x, conv_weight, conv_pool, conv_src_slot, conv_dst_slot, g, beta, state_pool, src_slot,
                        dst_slot, *, o=None, accepted_len=None, committed_len_out=None, conv_bias=None,
                        act: int = 0, qk_l2norm: bool = True, norm_eps: float = 1e-6, scale=1.0, out_gate=None,
                        out_norm_weight=None, out_norm_eps: float = 1e-6) -> Prepared:
    """kda_verify_conv with fixed buffers, as a Prepared call."""
    a = _verify_conv_args(x, conv_weight, conv_pool, conv_src_slot, conv_dst_slot, g, beta, state_pool, src_slot,
                          dst_slot, o, accepted_len, committed_len_out, conv_bias, act, qk_l2norm, norm_eps, scale,
                          out_gate, out_norm_weight, out_norm_eps)
    return Prepared(load_library().kda_verify_conv, a,
                    (x, conv_weight, conv_pool, conv_src_slot, conv_dst_slot, g, beta, state_pool, src_slot,
                     dst_slot, o, accepted_len, committed_len_out, conv_bias, out_gate, out_norm_weight))


def _verify_args(q, k, v, g, beta, state_pool, src_slot, dst_slot, o, accepted_len, committed_len_out, scale):
    import torch
    _expect(q.dim() == 4 and v.dim() == 4 and beta.dim() == 3,
            "q/k/v/g [N, T_spec, H, d], beta [N, T_spec, H]")
    N, Ts, H, dk = q.shape
    _same_lead([("k", k), ("g", g)], (N, Ts, H, dk), "q")
    _same_lead([("v", v), ("o", o)], (N, Ts, H, v.shape[3]), "v")
    _same_lead([("beta", beta)], (N, Ts, H), "q")
    _expect(state_pool.dim() == 4 and tuple(state_pool.shape[1:]) == (H, dk, v.shape[3]),
            "state_pool must be [n_slots, H, d_k, d_v]")
    _expect(src_slot.numel() >= N and dst_slot.numel() >= N, "slot arrays shorter than n_seq")
    _expect(accepted_len is None or accepted_len.numel() >= N, "accepted_len shorter than n_seq")
    _expect(committed_len_out is None or committed_len_out.numel() >= N,
            "committed_len_out shorter than n_seq")
    _device_tensors(q=q, k=k, v=v, g=g, beta=beta, o=o, state_pool=state_pool, src_slot=src_slot,
                    dst_slot=dst_slot, accepted_len=accepted_len, committed_len_out=committed_len_out)
    _same_dtype(q, k=k, v=v, g=g, beta=beta)
    _expect(state_pool.dtype == torch.float32 and state_pool.is_contiguous(),
            "state_pool must be contiguous float32")
    a = VerifyArgs()
    a.struct_size = ctypes.sizeof(VerifyArgs)
    a.q, a.k, a.v, a.g, a.beta, a.o = map(_ptr, (q, k, v, g, beta, o))
    a.state_pool, a.src_slot, a.dst_slot = _ptr(state_pool), _ptr(src_slot), _ptr(dst_slot)
    a.accepted_len, a.committed_len_out = _ptr(accepted_len), _ptr(committed_len_out)
    for name, t, inner in (("q", q, 2), ("k", k, 2), ("v", v, 2), ("g", g, 2), ("beta", beta, 1),
                           ("o", o, 2)):
        if t is not None and t.stride(0) != t.shape[1] * t.stride(1):
            raise ValueError(f"{name}: sequences must be T_spec tokens apart")
        setattr(a, f"{name}_stride", 0 if t is None else _tok_stride(t, inner))
    a.n_slots = state_pool.shape[0]
    a.n_seq, a.T_spec, a.H = q.shape[0], q.shape[1], q.shape[2]
    a.d_k, a.d_v = q.shape[3], v.shape[3]
    a.in_dtype = _dtype_code(q)
    a.out_dtype = _dtype_code(o) if o is not None else KDA_F32
    a.scale = scale
    return a


def kda_verify(q, k, v, g, beta, state_pool, src_slot, dst_slot, *, o=None, accepted_len=None,
               committed_len_out=None, scale=1.0, stream=None):
    """Speculative verify.  q, k, v, g [N, T_spec, H, d]; beta [N, T_spec, H]."""
    a = _verify_args(q, k, v, g, beta, state_pool, src_slot, dst_slot, o, accepted_len, committed_len_out, scale)
    _check(load_library().kda_verify(ctypes.byref(a), _stream(stream)))
    return o


def prepare_verify(q, k, v, g, beta, state_pool, src_slot, dst_slot, *, o=None, accepted_len=None,
                   committed_len_out=None, scale=1.0) -> Prepared:
    """kda_verify with fixed buffers, as a Prepared call."""
    a = _verify_args(q, k, v, g, beta, state_pool, src_slot, dst_slot, o, accepted_len, committed_len_out, scale)
    return Prepared(load_library().kda_verify, a,
                    (q, k, v, g, beta, state_pool, src_slot, dst_slot, o, accepted_len, committed_len_out))
