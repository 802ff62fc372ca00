"""The C ABI on the CPU: the library loads, exports every declared entry
point, its structs match the binding, and host-side validation returns the
documented status codes without touching a GPU."""

import ctypes
import re
from pathlib import Path

import numpy as np
import pytest

from hybrid_recurrent_serving_amd import kda as K

ROOT = Path(__file__).resolve().parents[1]


@pytest.fixture(scope="module")
def lib():
    return K.load_library()


def declared_functions():
    text = (ROOT / "include" / "kda.h").read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(K.EXPORTS)


def test_abi_version_and_struct_sizes(lib):
    assert lib.kda_abi_version() == 2
    for which, cls in enumerate([K.ConvArgs, K.PrefillArgs, K.DecodeArgs, K.VerifyArgs, K.DecodeConvArgs,
                                 K.VerifyConvArgs, K.PlanArgs, K.PrefillConvArgs]):
        assert lib.kda_args_sizeof(which) == ctypes.sizeof(cls), cls.__name__
    assert lib.kda_args_sizeof(8) == 0


def test_status_strings(lib):
    assert lib.kda_status_str(0) == b"KDA_OK"
    assert lib.kda_status_str(4) == b"KDA_ERR_ALIGN"
    assert lib.kda_status_str(99) == b"KDA_ERR_UNKNOWN"


def _call(lib, fn, args):
    return getattr(lib, fn)(ctypes.byref(args), None)


def _decode_args(**kw):
    a = K.DecodeArgs()
    a.struct_size = ctypes.sizeof(K.DecodeArgs)
    fake = 1 << 20  # a 16-byte aligned fake device address: never dereferenced on these paths
    for f in ("q", "k", "v", "g", "beta", "o", "state_pool", "src_slot", "dst_slot"):
        setattr(a, f, fake)
    a.n_seq, a.H, a.d_k, a.d_v, a.n_slots = 4, 2, 128, 128, 4
    a.in_dtype, a.out_dtype, a.scale = 0, 0, 1.0
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def _decode_conv_args(**kw):
    a = K.DecodeConvArgs()
    a.struct_size = ctypes.sizeof(K.DecodeConvArgs)
    fake = 1 << 20  # a 16-byte aligned fake device address: never dereferenced on these paths
    for f in ("x", "conv_weight", "conv_pool", "conv_src_slot", "conv_dst_slot", "g", "beta", "o",
              "state_pool", "src_slot", "dst_slot"):
        setattr(a, f, fake)
    a.n_seq, a.H, a.d, a.W, a.n_slots, a.n_conv_slots = 4, 2, 128, 4, 4, 4
    a.in_dtype, a.out_dtype, a.scale, a.norm_eps, a.qk_l2norm = 0, 0, 1.0, 1e-6, 1
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def test_decode_conv_validation(lib):
    f = "kda_decode_conv"
    assert lib.kda_decode_conv(None, None) == 1
    assert _call(lib, f, _decode_conv_args(struct_size=8)) == 8
    assert _call(lib, f, _decode_conv_args(n_seq=0)) == 0          # no-op
    assert _call(lib, f, _decode_conv_args(x=None)) == 1
    assert _call(lib, f, _decode_conv_args(conv_pool=None)) == 1
    assert _call(lib, f, _decode_conv_args(d=96)) == 6
    assert _call(lib, f, _decode_conv_args(W=5)) == 6
    assert _call(lib, f, _decode_conv_args(W=1)) == 6
    assert _call(lib, f, _decode_conv_args(act=2)) == 8
    assert _call(lib, f, _decode_conv_args(qk_l2norm=3)) == 8
    assert _call(lib, f, _decode_conv_args(norm_eps=-1.0)) == 8
    assert _call(lib, f, _decode_conv_args(in_dtype=5)) == 3
    assert _call(lib, f, _decode_conv_args(H=0)) == 2
    assert _call(lib, f, _decode_conv_args(x=(1 << 20) + 2)) == 4
    assert _call(lib, f, _decode_conv_args(x_stride=100)) == 2       # < 3 H d
    assert _call(lib, f, _decode_conv_args(x_stride=769)) == 4       # rows not 16-byte aligned
    assert b"aligned" in lib.kda_last_error()
    fake = 1 << 20
    assert _call(lib, f, _decode_conv_args(conv_bias=fake + 8)) == 4  # bias read in 8- / 16-byte units
    assert b"conv_bias" in lib.kda_last_error()
    assert _call(lib, f, _decode_conv_args(out_gate=fake)) == 1      # gate without norm weight
    assert _call(lib, f, _decode_conv_args(out_gate=fake, out_norm_weight=fake, out_norm_eps=-1.0)) == 8
    assert _call(lib, f, _decode_conv_args(out_gate=fake + 8, out_norm_weight=fake)) == 4
    assert _call(lib, f, _decode_conv_args(out_gate=fake, out_norm_weight=fake, out_gate_stride=100)) == 2


def test_verify_conv_validation(lib):
    f = "kda_verify_conv"
    fake = 1 << 20

    def args(**kw):
        a = K.VerifyConvArgs()
        a.struct_size = ctypes.sizeof(K.VerifyConvArgs)
        for fld in ("x", "conv_weight", "conv_pool", "conv_src_slot", "conv_dst_slot", "g", "beta", "o",
                    "state_pool", "src_slot", "dst_slot"):
            setattr(a, fld, fake)
        a.n_seq, a.T_spec, a.H, a.d, a.W, a.n_slots, a.n_conv_slots = 4, 8, 2, 128, 4, 4, 4
        a.in_dtype, a.out_dtype, a.scale, a.norm_eps, a.qk_l2norm = 0, 0, 1.0, 1e-6, 1
        for k, v in kw.items():
            setattr(a, k, v)
        return a

    assert lib.kda_verify_conv(None, None) == 1
    assert _call(lib, f, args(struct_size=8)) == 8
    assert _call(lib, f, args(n_seq=0)) == 0
    assert _call(lib, f, args(T_spec=0)) == 2
    assert _call(lib, f, args(T_spec=17)) == 2
    assert _call(lib, f, args(o=None)) == 1                 # neither o nor accepted_len
    assert _call(lib, f, args(x=None)) == 1
    assert _call(lib, f, args(d=96)) == 6
    assert _call(lib, f, args(W=5)) == 6
    assert _call(lib, f, args(act=3)) == 8
    assert _call(lib, f, args(x_stride=769)) == 4
    assert _call(lib, f, args(conv_bias=fake + 2)) == 4
    assert _call(lib, f, args(out_gate=fake)) == 1
    assert _call(lib, f, args(out_gate=fake, out_norm_weight=fake + 4)) == 4


def test_decode_validation(lib):
    assert lib.kda_decode(None, None) == 1
    assert _call(lib, "kda_decode", _decode_args(struct_size=8)) == 8
    assert _call(lib, "kda_decode", _decode_args(n_seq=0)) == 0         # no-op
    assert _call(lib, "kda_decode", _decode_args(q=None)) == 1
    assert _call(lib, "kda_decode", _decode_args(d_k=96, d_v=96)) == 6
    assert _call(lib, "kda_decode", _decode_args(d_k=64, d_v=128)) == 6
    assert _call(lib, "kda_decode", _decode_args(in_dtype=5)) == 3
    assert _call(lib, "kda_decode", _decode_args(H=0)) == 2
    assert _call(lib, "kda_decode", _decode_args(q=(1 << 20) + 2)) == 4
    assert _call(lib, "kda_decode", _decode_args(q_stride=100)) == 2     # < H*d
    assert _call(lib, "kda_decode", _decode_args(q_stride=257)) == 4     # not 16-byte aligned
    assert b"aligned" in lib.kda_last_error()


def _verify_args(**kw):
    a = K.VerifyArgs()
    a.struct_size = ctypes.sizeof(K.VerifyArgs)
    fake = 1 << 20
    for f in ("q", "k", "v", "g", "beta", "o", "state_pool", "src_slot", "dst_slot",
              "accepted_len"):
        setattr(a, f, fake)
    a.n_seq, a.T_spec, a.H, a.d_k, a.d_v, a.n_slots = 4, 8, 2, 64, 64, 4
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def test_verify_validation(lib):
    assert _call(lib, "kda_verify", _verify_args(T_spec=0)) == 2
    assert _call(lib, "kda_verify", _verify_args(T_spec=17)) == 2
    assert _call(lib, "kda_verify", _verify_args(o=None, accepted_len=None)) == 1
    assert _call(lib, "kda_verify", _verify_args(n_seq=0)) == 0


def _conv_args(**kw):
    a = K.ConvArgs()
    a.struct_size = ctypes.sizeof(K.ConvArgs)
    fake = 1 << 20
    for f in ("x", "y", "weight", "cu_seqlens", "conv_pool", "src_slot", "dst_slot"):
        setattr(a, f, fake)
    a.n_seq, a.C, a.W, a.T_tot, a.n_slots, a.dtype = 2, 64, 4, 10, 2, 0
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def test_conv_validation(lib):
    assert _call(lib, "kda_conv_short", _conv_args(W=1)) == 6
    assert _call(lib, "kda_conv_short", _conv_args(W=9)) == 6
    assert _call(lib, "kda_conv_short", _conv_args(C=12)) == 2     # not a multiple of 8 (bf16)
    assert _call(lib, "kda_conv_short", _conv_args(dtype=3)) == 3
    assert _call(lib, "kda_conv_short", _conv_args(x_stride=65)) == 4
    assert _call(lib, "kda_conv_short", _conv_args(act=2)) == 8
    assert _call(lib, "kda_conv_short", _conv_args(n_seq=0)) == 0
    # the optional per-head normalisation
    assert _call(lib, "kda_conv_short", _conv_args(norm_d=48, norm_channels=48)) == 6
    assert _call(lib, "kda_conv_short", _conv_args(norm_d=16, norm_channels=32, W=5)) == 6
    assert _call(lib, "kda_conv_short", _conv_args(norm_d=16, norm_channels=24)) == 8
    assert _call(lib, "kda_conv_short", _conv_args(norm_d=16, norm_channels=80)) == 8   # > C
    assert _call(lib, "kda_conv_short", _conv_args(norm_d=128, norm_channels=0)) == 8   # C not a multiple
    assert _call(lib, "kda_conv_short", _conv_args(norm_d=16, norm_channels=32, norm_eps=-1.0)) == 8


def _prefill_args(**kw):
    a = K.PrefillArgs()
    a.struct_size = ctypes.sizeof(K.PrefillArgs)
    fake = 1 << 20
    for f in ("q", "k", "v", "g", "beta", "o", "cu_seqlens", "state_pool", "src_slot", "dst_slot"):
        setattr(a, f, fake)
    a.n_seq, a.H, a.d_k, a.d_v, a.chunk, a.T_tot, a.n_slots = 2, 2, 64, 64, 64, 100, 4
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def test_prefill_validation(lib):
    assert _call(lib, "kda_prefill_varlen", _prefill_args(chunk=48)) == 6
    assert _call(lib, "kda_prefill_varlen", _prefill_args(ckpt_interval=100)) == 4
    assert _call(lib, "kda_prefill_varlen", _prefill_args(ckpt_interval=128)) == 1  # no ckpt arrays
    assert _call(lib, "kda_prefill_varlen", _prefill_args(cu_seqlens=None)) == 1
    assert _call(lib, "kda_prefill_varlen", _prefill_args(n_seq=0)) == 0
    assert lib.kda_prefill_workspace_bytes(ctypes.byref(_prefill_args(chunk=48))) == -1
    assert _call(lib, "kda_prefill_varlen", _prefill_args(segment_len=100)) == 4
    # a batch long enough to be split needs the workspace
    assert _call(lib, "kda_prefill_varlen", _prefill_args(T_tot=65536)) == 5


def test_prefill_workspace_bytes(lib):
    """Segment-scan workspace: seg_cu and blk_cu (int32 [n_seq + 1], 256-byte
    rounded) plus three H x d x d fp32 blocks per block index, one int32 per
    block index and head, and the item order table (int32 per work item,
    min(n_seq + 3 T_tot / seg, T_tot / seg + 2 n_seq) + 1 items), each
    256-byte rounded, with
    3 T_tot / seg + 1 block indices; nothing when T_tot <= seg (no sequence
    can be split)."""
    ws = lambda **kw: lib.kda_prefill_workspace_bytes(ctypes.byref(_prefill_args(**kw)))
    H, d = 2, 64
    blk = 3 * H * d * d * 4
    r256 = lambda x: (x + 255) // 256 * 256
    n_seq = _prefill_args().n_seq

    def want(T, seg):
        nb = 3 * T // seg + 1
        items = min(n_seq + 3 * T // seg, T // seg + 2 * n_seq) + 1
        return 2 * r256(4 * (n_seq + 1)) + nb * blk + r256(nb * H * 4) + r256(items * 4)

    assert ws(T_tot=100) == 0
    assert ws(T_tot=32768) == 0                         # <= 32768: nothing can split
    assert ws(T_tot=32769) == want(32769, 32768)
    assert ws(T_tot=65536) == want(65536, 32768)
    assert ws(T_tot=65536, segment_len=-1) == 0
    assert ws(T_tot=4096, segment_len=1024) == want(4096, 1024)
    assert ws(T_tot=1024, segment_len=1024) == 0


def test_ckpt_plan_matches_oracle_enumeration(oracle64):
    rng = np.random.default_rng(3)
    for trial in range(30):
        n = int(rng.integers(1, 7))
        lens = rng.integers(0, 5000, n)
        starts = rng.integers(0, 3000, n)
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        chunk = int(rng.choice([16, 32, 64]))
        interval = chunk * int(rng.integers(1, 40))
        ck_cu, pos = K.kda_ckpt_plan(cu, interval, chunk, start_pos=starts)
        o_cu, o_pos = oracle64.ckpt_enumerate(cu, interval, starts.astype(np.int32))
        assert ck_cu == list(o_cu)
        assert pos == list(o_pos)
    # the long workload: 31 interior checkpoints
    ck_cu, pos = K.kda_ckpt_plan([0, 1 << 20], 32768, 64)
    assert ck_cu == [0, 31] and pos == [32768 * m for m in range(1, 32)]


def test_ckpt_plan_errors(lib):
    with pytest.raises(K.KDAError) as e:
        K.kda_ckpt_plan([0, 100], 100, 64)
    assert e.value.name == "KDA_ERR_ALIGN"
    with pytest.raises(K.KDAError):
        K.kda_ckpt_plan([0, 100], 64, 48)
    cu = np.array([0, 1000], np.int32)
    ck_cu = np.zeros(2, np.int32)
    pos = np.zeros(2, np.int32)
    total = ctypes.c_int32(0)
    vp = lambda a: a.ctypes.data_as(ctypes.c_void_p)  # noqa: E731
    st = lib.kda_ckpt_plan(vp(cu), None, 1, 64, 64, vp(ck_cu), vp(pos), 2, ctypes.byref(total))
    assert st == 9 and total.value == 15 and ck_cu[1] == 15


def _plan_args(**kw):
    a = K.PlanArgs()
    a.struct_size = ctypes.sizeof(K.PlanArgs)
    fake = 1 << 20  # never dereferenced on these paths
    a.cu_seqlens = a.ckpt_cu = a.ckpt_pos = a.ckpt_slot = a.n_total = fake
    a.T_tot, a.n_seq, a.interval, a.chunk, a.cap, a.n_free = 1000, 3, 128, 64, 16, 0
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("kw,status", [
    (dict(struct_size=8), "KDA_ERR_ARG"),
    (dict(n_seq=-1), "KDA_ERR_SHAPE"),
    (dict(cap=-1), "KDA_ERR_SHAPE"),
    (dict(n_free=-2), "KDA_ERR_SHAPE"),
    (dict(T_tot=-1), "KDA_ERR_SHAPE"),
    (dict(chunk=48), "KDA_ERR_UNSUPPORTED"),
    (dict(interval=100), "KDA_ERR_ALIGN"),
    (dict(interval=0), "KDA_ERR_ALIGN"),
    (dict(cu_seqlens=None), "KDA_ERR_NULL"),
    (dict(ckpt_cu=None), "KDA_ERR_NULL"),
    (dict(n_free=4, free_slots=None), "KDA_ERR_NULL"),
])
def test_ckpt_plan_device_validation(lib, kw, status):
    st = lib.kda_ckpt_plan_device(ctypes.byref(_plan_args(**kw)), None)
    assert lib.kda_status_str(st).decode() == status, lib.kda_last_error()


def test_prefill_conv_validation(lib):
    """kda_prefill_varlen_conv rejects bad arguments before launching
    anything (every case here fails on the host)."""
    f = "kda_prefill_varlen_conv"
    fake = 1 << 20

    def args(**kw):
        a = K.PrefillConvArgs()
        a.struct_size = ctypes.sizeof(K.PrefillConvArgs)
        p = a.prefill
        p.struct_size = ctypes.sizeof(K.PrefillArgs)
        for fld in ("g", "beta", "o", "cu_seqlens", "state_pool", "src_slot", "dst_slot"):
            setattr(p, fld, fake)
        p.T_tot, p.n_slots, p.n_seq, p.H, p.d_k, p.d_v, p.chunk = 64, 4, 2, 2, 64, 64, 64
        p.in_dtype, p.out_dtype, p.scale = 0, 0, 1.0
        for fld in ("x", "conv_weight", "conv_pool", "conv_src_slot", "conv_dst_slot", "qkv"):
            setattr(a, fld, fake)
        a.n_conv_slots, a.qkv_bytes, a.W, a.act, a.qk_l2norm, a.norm_eps = 4, 64 * 384 * 2, 4, 1, 1, 1e-6
        for k, v in kw.items():
            if k.startswith("p_"):
                setattr(p, k[2:], v)
            else:
                setattr(a, k, v)
        return a

    assert lib.kda_prefill_varlen_conv(None, None) == 1
    assert _call(lib, f, args(struct_size=8)) == 8
    assert _call(lib, f, args(p_q=fake)) == 8                    # q is formed by the library
    assert _call(lib, f, args(p_k_stride=384)) == 8
    assert _call(lib, f, args(p_d_v=32)) == 8
    assert _call(lib, f, args(p_in_dtype=7)) == 3
    assert _call(lib, f, args(p_d_k=48, p_d_v=48)) == 6
    assert _call(lib, f, args(W=5)) == 6
    assert _call(lib, f, args(W=1)) == 6
    assert _call(lib, f, args(act=2)) == 8
    assert _call(lib, f, args(qk_l2norm=2)) == 8
    assert _call(lib, f, args(norm_eps=-1.0)) == 8
    assert _call(lib, f, args(qkv=None)) == 1
    assert _call(lib, f, args(x=None)) == 1
    assert _call(lib, f, args(conv_pool=None)) == 1
    assert _call(lib, f, args(p_chunk=48)) == 6                  # prefill's own checks
    assert _call(lib, f, args(p_o=None)) == 1
    assert _call(lib, f, args(qkv_bytes=64 * 384 * 2 - 2)) == 5  # qkv too small
    assert _call(lib, f, args(x=fake + 4)) == 4
    assert _call(lib, f, args(x_stride=100)) == 2                # < 3 H d
    assert _call(lib, f, args(x_stride=388)) == 4                # rows not 16-byte aligned
    assert _call(lib, f, args(p_n_seq=0)) == 0                   # no-op
    assert _call(lib, f, args(conv_ckpt_slot=fake)) == 8         # conv checkpoints without checkpoints

