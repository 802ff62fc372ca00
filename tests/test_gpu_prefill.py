"""GPU parity of kda_prefill_varlen against the CPU oracle, through the C ABI."""

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


def _init_arrays(wl):
    N = wl.n_seq
    init = np.zeros((N, wl.H, wl.dk, wl.dv))
    has = np.zeros(N, np.int32)
    for s, i in enumerate(wl.init_index):
        if i >= 0:
            init[s] = wl.init_states[i].double().numpy()
            has[s] = 1
    return init, has


def run_prefill(dev, wl, *, chunk, out_dtype=torch.bfloat16, start_pos=None, ckpt_interval=0,
                scale=1.0, segment_len=0):
    """Run the GPU prefill with source slots [0, N) (zero where the workload
    has no initial state) and destination slots [N, 2N); checkpoints (if any)
    go to slots from 2N on.  Returns dict of host tensors."""
    N, H, d = wl.n_seq, wl.H, wl.dk
    cu_h = wl.cu_seqlens.cpu()
    n_ck = 0
    ck_cu = ck_pos_plan = None
    if ckpt_interval:
        ck_cu, ck_pos_plan = K.kda_ckpt_plan(cu_h.numpy(), ckpt_interval, chunk,
                                            start_pos=None if start_pos is None else start_pos)
        n_ck = ck_cu[-1]
    pool = torch.full((2 * N + max(n_ck, 1), H, d, d), float("nan"), device=dev)
    init, has = _init_arrays(wl)
    pool[:N] = torch.tensor(init, dtype=torch.float32, device=dev)
    src = torch.tensor([s if has[s] else -1 for s in range(N)], dtype=torch.int32, device=dev)
    dst = torch.arange(N, 2 * N, dtype=torch.int32, device=dev)
    q, k, v, g, b = (t.to(dev) for t in (wl.q, wl.k, wl.v, wl.g, wl.beta))
    o = torch.full((q.shape[0], H, d), float("nan"), dtype=out_dtype, device=dev)
    kw = {}
    if start_pos is not None:
        kw["start_pos"] = torch.tensor(start_pos, dtype=torch.int32, device=dev)
    if ckpt_interval:
        kw["ckpt_interval"] = ckpt_interval
        kw["ckpt_cu"] = torch.tensor(ck_cu, dtype=torch.int32, device=dev)
        kw["ckpt_slot"] = torch.arange(2 * N, 2 * N + n_ck, dtype=torch.int32, device=dev)
        kw["ckpt_pos_out"] = torch.full((max(n_ck, 1),), -1, dtype=torch.int32, device=dev)
    before = pool[:N].clone()
    K.kda_prefill_varlen(q, k, v, g, b, o, wl.cu_seqlens.to(dev), pool, src, dst, chunk=chunk,
                         scale=scale, segment_len=segment_len, **kw)
    torch.cuda.synchronize()
    assert torch.equal(pool[:N], before), "source slots were modified"
    res = {"o": o.float().cpu(), "final": pool[N:2 * N].cpu(), "init": init, "has": has}
    if ckpt_interval:
        res["ckpt"] = pool[2 * N:2 * N + n_ck].cpu()
        res["ckpt_pos"] = kw["ckpt_pos_out"][:n_ck].cpu().tolist()
        res["ckpt_plan"] = ck_pos_plan
        res["ckpt_cu"] = ck_cu
    return res


def oracle_run(oracle64, wl, init, has, start_pos=None, ckpt_interval=0, pairs=None, scale=1.0):
    return oracle64.kda_varlen(wl.q, wl.k, wl.v, wl.g, wl.beta, wl.cu_seqlens, init=init,
                               has_init=has, start_pos=start_pos, ckpt_interval=ckpt_interval,
                               pairs=pairs, scale=scale)


# ------------------------------------------------------------------ tiny
@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_prefill_tiny_fp32(dev, oracle64, chunk):
    """Tiny workload: B=1, T=64, H=2, d=16, fp32 in/out, zero initial state."""
    U.say(f"prefill tiny fp32 chunk={chunk}")
    wl = make_workload(0)
    r = run_prefill(dev, wl, chunk=chunk, out_dtype=torch.float32)
    ref = oracle_run(oracle64, wl, r["init"], r["has"])
    U.assert_close("o", r["o"].numpy(), ref["o"], rel=2e-4, mx=1e-3)
    U.assert_close("state", r["final"].numpy(), ref["final"], rel=2e-4, mx=1e-3)


# ------------------------------------------------------------------ ragged varlen
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("chunk", [16, 64])
def test_prefill_ragged(dev, oracle64, d, chunk):
    """Ragged packed lengths (empty, single token, partial chunks, several
    chunks), half of the sequences from random initial states."""
    U.say(f"prefill ragged d={d} chunk={chunk}")
    lens = [0, 1, 5, 31, 32, 33, 100, 257]
    wl = make_workload(2, lengths=lens, H=3, d=d)
    r = run_prefill(dev, wl, chunk=chunk)
    ref = oracle_run(oracle64, wl, r["init"], r["has"])
    U.assert_close("o", r["o"].numpy(), ref["o"])
    fin = r["final"].numpy()
    # the empty sequence's final state is its (zero) initial state
    U.assert_close("state", fin, ref["final"])


def test_prefill_fp32_out_and_scale(dev, oracle64):
    U.say("prefill fp32 out, scale")
    wl = make_workload(2, lengths=[200, 77, 64], H=2, d=128)
    r = run_prefill(dev, wl, chunk=64, out_dtype=torch.float32, scale=0.125)
    ref = oracle_run(oracle64, wl, r["init"], r["has"], scale=0.125)
    U.assert_close("o", r["o"].numpy(), ref["o"], rel=5e-4, mx=1e-3)
    U.assert_close("state", r["final"].numpy(), ref["final"], rel=5e-4, mx=1e-3)


def test_prefill_checkpoints_unaligned_starts(dev, oracle64):
    """Absolute start positions not on chunk boundaries; interval checkpoints
    land where the plan says (bit-exact positions) with the oracle's states."""
    U.say("prefill checkpoints, unaligned starts")
    lens = [300, 129, 64, 1, 500]
    starts = [0, 7, 96, 63, 1000]
    wl = make_workload(2, lengths=lens, H=2, d=64)
    r = run_prefill(dev, wl, chunk=32, start_pos=starts, ckpt_interval=64)
    ref = oracle_run(oracle64, wl, r["init"], r["has"], start_pos=np.array(starts, np.int32),
                     ckpt_interval=64)
    assert r["ckpt_pos"] == list(ref["ckpt_pos"]) == r["ckpt_plan"]
    assert list(ref["ckpt_cu"]) == r["ckpt_cu"]
    U.assert_close("o", r["o"].numpy(), ref["o"])
    U.assert_close("state", r["final"].numpy(), ref["final"])
    U.assert_close("ckpt", r["ckpt"].numpy(), ref["ckpt"])


def test_prefill_resume_from_checkpoint(dev):
    """Prefill to a checkpoint, resume from the checkpoint slot: outputs and
    final state agree with the continuous run within tolerance."""
    U.say("prefill resume from own checkpoint")
    wl = make_workload(2, lengths=[640], H=4, d=128)
    full = run_prefill(dev, wl, chunk=64, ckpt_interval=256)
    assert full["ckpt_pos"] == [256, 512]
    cut = 512
    wl2 = make_workload(2, lengths=[640], H=4, d=128)
    # second half only, starting from the checkpoint state at absolute position 512
    wl2.q, wl2.k, wl2.v, wl2.g, wl2.beta = (t[cut:] for t in (wl.q, wl.k, wl.v, wl.g, wl.beta))
    wl2.cu_seqlens = torch.tensor([0, 640 - cut], dtype=torch.int32)
    wl2.init_states = full["ckpt"][1:2].clone()
    wl2.init_index = [0]
    part = run_prefill(dev, wl2, chunk=64, start_pos=[cut])
    U.assert_close("o", part["o"].numpy(), full["o"][cut:].numpy())
    U.assert_close("state", part["final"].numpy(), full["final"].numpy())


def test_prefill_decode_identity(dev):
    """A 1-token prefill equals a decode step (within tolerance)."""
    U.say("prefill == decode for one token")
    wl = make_workload(1, n_seq=12, H=4)
    q, k, v, g, b = (t.to(dev) for t in (wl.q, wl.k, wl.v, wl.g, wl.beta))
    pool_p = wl.init_states.to(dev).clone()
    pool_d = wl.init_states.to(dev).clone()
    slots = torch.arange(12, dtype=torch.int32, device=dev)
    o_p = torch.empty(12, 4, 128, device=dev)
    o_d = torch.empty(12, 4, 128, device=dev)
    K.kda_prefill_varlen(q, k, v, g, b, o_p, wl.cu_seqlens.to(dev), pool_p, slots, slots, chunk=64)
    K.kda_decode(q, k, v, g, b, o_d, pool_d, slots, slots)
    torch.cuda.synchronize()
    U.assert_close("o", U.to_np(o_p), U.to_np(o_d), rel=5e-4, mx=1e-3)
    U.assert_close("state", U.to_np(pool_p), U.to_np(pool_d), rel=5e-4, mx=1e-3)


def test_prefill_slow_decay_stress(dev, oracle64):
    """alpha ~ 0.98 (g = logsigmoid(N(4, 1))): long memory through many chunks."""
    U.say("prefill slow decay")
    wl = make_workload(2, lengths=[2048, 1000], H=2, d=128, mu_g=4.0)
    r = run_prefill(dev, wl, chunk=64)
    ref = oracle_run(oracle64, wl, r["init"], r["has"])
    U.assert_close("o", r["o"].numpy(), ref["o"])
    U.assert_close("state", r["final"].numpy(), ref["final"])


def test_prefill_decay_spikes(dev, oracle64):
    """Single very strong decays (g = -20) at scattered tokens."""
    U.say("prefill decay spikes")
    wl = make_workload(2, lengths=[256], H=2, d=64)
    g = wl.g.clone()
    g[5] = -20.0
    g[40, 0, :10] = -20.0
    g[131, 1] = -20.0
    wl.g = g
    r = run_prefill(dev, wl, chunk=64)
    ref = oracle_run(oracle64, wl, r["init"], r["has"])
    U.assert_close("o", r["o"].numpy(), ref["o"])
    U.assert_close("state", r["final"].numpy(), ref["final"])


def test_prefill_deterministic(dev):
    U.say("prefill determinism")
    wl = make_workload(2, lengths=[300, 1000], H=2, d=128)
    a = run_prefill(dev, wl, chunk=64)
    b = run_prefill(dev, wl, chunk=64)
    assert torch.equal(a["o"], b["o"]) and torch.equal(a["final"], b["final"])


# ------------------------------------------------------------------ full-size workloads
@pytest.fixture(scope="module")
def varlen16(oracle64):
    """The 16-sequence varlen workload and the oracle's result on all of it
    (every sequence and head, every output and final state)."""
    wl = make_workload(2)
    init, has = _init_arrays(wl)
    U.say("  oracle: 16-sequence varlen workload, all 256 (sequence, head) pairs")
    ref = oracle_run(oracle64, wl, init, has)
    return wl, ref


@pytest.mark.timeout(600)
@pytest.mark.parametrize("segment_len", [0, 3072, 4096])
def test_prefill_varlen_16_sequences_full(dev, varlen16, segment_len):
    """16 packed sequences, lengths U{512..16384}, H=16, d=128, chunk 64, bf16;
    even sequences from random initial states.  Every output of every
    (sequence, head) and all 16 final states against the oracle.  Unsplit
    (the default segment length exceeds every sequence), with the
    3,072-token segments the benchmark runs, and with 4,096-token ones."""
    U.say(f"prefill 16-sequence varlen (full oracle), segment_len={segment_len}")
    wl, ref = varlen16
    r = run_prefill(dev, wl, chunk=64, segment_len=segment_len)
    U.assert_close("o", r["o"].numpy(), ref["o"])
    U.assert_close("final", r["final"].numpy(), ref["final"])


def test_prefill_long_65536_full(dev, oracle64):
    """B=1, T=65,536, H=16, d=128, chunk 64, checkpoints every 32,768: every
    output, the checkpoint and the final state against the oracle."""
    U.say("prefill long T=65536 (full oracle)")
    wl = make_workload(3, T=65536)
    r = run_prefill(dev, wl, chunk=64, ckpt_interval=32768)
    assert r["ckpt_pos"] == [32768]
    ref = oracle_run(oracle64, wl, r["init"], r["has"], ckpt_interval=32768)
    U.assert_close("o", r["o"].numpy(), ref["o"])
    U.assert_close("ckpt+final", np.concatenate([r["ckpt"].numpy(), r["final"].numpy()]),
                   np.concatenate([ref["ckpt"], ref["final"]]))


# ------------------------------------------------------------------ segment scan
@pytest.mark.parametrize("d", [64, 128])
def test_prefill_segment_scan_slow_decay(dev, oracle64, d):
    """Sequences longer than the segment length run as parallel segments joined by
    the transition combine.  Slow decay (alpha ~ 0.98) keeps the transitions
    far from zero; unaligned starts, initial states, checkpoints that fall on
    and between segment boundaries.  Against the oracle, and against the same
    call without splitting."""
    U.say(f"prefill segment scan, slow decay, d={d}")
    lens = [1000, 300, 2100, 530]
    starts = [0, 40, 96, 7]
    wl = make_workload(2, lengths=lens, H=2, d=d, mu_g=4.0)
    r = run_prefill(dev, wl, chunk=64, start_pos=starts, ckpt_interval=128, segment_len=256)
    ref = oracle_run(oracle64, wl, r["init"], r["has"], start_pos=np.array(starts, np.int32),
                     ckpt_interval=128)
    assert r["ckpt_pos"] == list(ref["ckpt_pos"]) == r["ckpt_plan"]
    U.assert_close("o", r["o"].numpy(), ref["o"])
    U.assert_close("state", r["final"].numpy(), ref["final"])
    U.assert_close("ckpt", r["ckpt"].numpy(), ref["ckpt"])
    whole = run_prefill(dev, wl, chunk=64, start_pos=starts, ckpt_interval=128, segment_len=-1)
    U.assert_close("o(split vs whole)", r["o"].numpy(), whole["o"].numpy())
    U.assert_close("state(split vs whole)", r["final"].numpy(), whole["final"].numpy())


def test_prefill_segment_scan_fast_decay(dev, oracle64):
    """Segments of 2,048 tokens with the usual decay (E[alpha] = 0.5): the
    transition of a segment underflows to exact zeros within a few hundred
    tokens and its chain stops at the next check, which must leave every
    output, checkpoint and final state as the oracle has them, and as the
    same call without splitting."""
    U.say("prefill segment scan, fast decay (transition stops at exact zero)")
    lens = [5000, 7000, 4100]
    starts = [0, 64, 32]
    wl = make_workload(2, lengths=lens, H=2, d=128)
    r = run_prefill(dev, wl, chunk=64, start_pos=starts, ckpt_interval=1024, segment_len=2048)
    ref = oracle_run(oracle64, wl, r["init"], r["has"], start_pos=np.array(starts, np.int32),
                     ckpt_interval=1024)
    assert r["ckpt_pos"] == list(ref["ckpt_pos"]) == r["ckpt_plan"]
    U.assert_close("o", r["o"].numpy(), ref["o"])
    U.assert_close("state", r["final"].numpy(), ref["final"])
    U.assert_close("ckpt", r["ckpt"].numpy(), ref["ckpt"])
    whole = run_prefill(dev, wl, chunk=64, start_pos=starts, ckpt_interval=1024, segment_len=-1)
    U.assert_close("o(split vs whole)", r["o"].numpy(), whole["o"].numpy())
    U.assert_close("state(split vs whole)", r["final"].numpy(), whole["final"].numpy())


def test_prefill_segment_scan_tiny_fp32(dev, oracle64):
    """The tiny fp32 workload (chunk 16) split into 16-token segments."""
    U.say("prefill segment scan, tiny fp32")
    wl = make_workload(0, mu_g=3.0)
    r = run_prefill(dev, wl, chunk=16, out_dtype=torch.float32, segment_len=16)
    ref = oracle_run(oracle64, wl, r["init"], r["has"])
    U.assert_close("o", r["o"].numpy(), ref["o"], rel=2e-4, mx=1e-3)
    U.assert_close("state", r["final"].numpy(), ref["final"], rel=2e-4, mx=1e-3)


@pytest.mark.timeout(900)
def test_prefill_long_1m_segments(dev, oracle64):
    """B=1, T=1,048,576, H=16, d=128, chunk 64, checkpoints every 32,768 (31
    interior + final), run as 32 parallel segments.  The oracle resumes from
    the GPU's own checkpoints on every segment (the first from the zero
    state) and reproduces that segment's outputs and its end state (the next
    checkpoint, or the final state): every output and every returned state
    of the run is compared, and the checkpoint positions are exact."""
    U.say("prefill long T=1,048,576 (every segment resumed by the oracle)")
    T, I = 1048576, 32768
    wl = make_workload(3, device=dev)
    r = run_prefill(dev, wl, chunk=64, ckpt_interval=I)
    assert r["ckpt_pos"] == [I * j for j in range(1, 32)] == r["ckpt_plan"]
    ends = np.concatenate([r["ckpt"].numpy(), r["final"].numpy()])      # [32, H, d, d]
    starts = np.concatenate([np.zeros((1,) + ends.shape[1:]), ends[:-1].astype(np.float64)])
    acc = {"o": [0.0, 0.0, 0.0], "states": [0.0, 0.0, 0.0]}   # sum d^2, sum ref^2, max |d|

    def add(key, got, ref):
        dlt = np.asarray(got, np.float64) - ref
        acc[key][0] += float(np.sum(dlt * dlt))
        acc[key][1] += float(np.sum(ref * ref))
        acc[key][2] = max(acc[key][2], float(np.max(np.abs(dlt))))
        assert np.all(np.isfinite(got)), f"{key}: non-finite values"

    G = 4   # segments per oracle call (one packed batch, resumed states)
    for j0 in range(0, 32, G):
        lo, hi = I * j0, I * (j0 + G)
        q, k, v, g, b = (t[lo:hi].cpu() for t in (wl.q, wl.k, wl.v, wl.g, wl.beta))
        cu = torch.arange(0, G * I + 1, I, dtype=torch.int32)
        ref = oracle64.kda_varlen(q, k, v, g, b, cu, init=starts[j0:j0 + G],
                                  has_init=np.ones(G, np.int32),
                                  start_pos=np.arange(lo, hi, I, dtype=np.int32))
        add("o", r["o"][lo:hi].numpy(), ref["o"])
        add("states", ends[j0:j0 + G], ref["final"])
        U.say(f"  segments {j0}..{j0 + G - 1} compared")
        del ref, q, k, v, g, b
    for key in ("o", "states"):
        rel = (acc[key][0] / acc[key][1]) ** 0.5
        U.say(f"  {key} (all 32 segments): rel_l2={rel:.3e} max_abs={acc[key][2]:.3e}")
        assert rel <= U.REL_L2_TOL and acc[key][2] <= U.MAX_ABS_TOL, key


@pytest.mark.parametrize("mu_g,segment_len", [(4.0, 128), (0.0, 512)])
def test_prefill_segment_scan_in_place(dev, oracle64, mu_g, segment_len):
    """Source slot == destination slot for sequences that are split into
    segments, with unaligned starts and more work items than one wave of
    workgroups holds: the first segment must read the true source state even
    though the final state lands in the same slot.  Slow decay reruns every
    later segment whole; the usual decay stops the last segment's fix-up
    early, so its final state comes from its local chain."""
    U.say(f"prefill segment scan, in place (src == dst), mu_g={mu_g}, segment_len={segment_len}")
    rng = np.random.default_rng(11)
    N = 24
    lens = [int(x) for x in rng.integers(700, 1500, N)]
    starts = [int(x) for x in rng.integers(0, 300, N)]
    wl = make_workload(2, lengths=lens, H=16, d=128, mu_g=mu_g)
    init, has = _init_arrays(wl)
    pool = torch.tensor(init, dtype=torch.float32, device=dev)
    slots = torch.arange(N, dtype=torch.int32, device=dev)
    q, k, v, g, b = (t.to(dev) for t in (wl.q, wl.k, wl.v, wl.g, wl.beta))
    o = torch.full((q.shape[0], 16, 128), float("nan"), dtype=torch.bfloat16, device=dev)
    K.kda_prefill_varlen(q, k, v, g, b, o, wl.cu_seqlens.to(dev), pool, slots, slots, chunk=64,
                         start_pos=torch.tensor(starts, dtype=torch.int32, device=dev), segment_len=segment_len)
    torch.cuda.synchronize()
    ref = oracle_run(oracle64, wl, init, np.ones(N, np.int32), start_pos=np.array(starts, np.int32))
    U.assert_close("o", o.float().cpu().numpy(), ref["o"])
    U.assert_close("state", pool.cpu().numpy(), ref["final"])
