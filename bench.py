#!/usr/bin/env python3
"""Throughput of the KDA layer path on one MI355X.

Default workload: batched decode (128 sequences x 1 token, H=16,
d_k=d_v=128, bf16 inputs, fp32 recurrent state, short conv W=4 over the
3*H*d q/k/v channels).  One step = one kda_decode_conv launch: the conv
(+ SiLU) of the token's q/k/v projections with the carried conv history,
per-head q/k L2 normalisation, the recurrence and the sigmoid-gated RMS
norm of the output, both states advanced in place.  The recurrent state
rotates over 4 pools of 128 MiB so it cannot be served from the 256 MB
Infinity Cache.

Prints ONE JSON line.  ``value`` = recurrent-state bytes read + written per
step / step time (GB/s).  ``roofline`` = the fused kernel's algorithmic
bytes per launch / its average launch time (HIP events on the launch stream
over the timed region) against 8 TB/s.  ``cpu_baseline`` = the CPU oracle on
the same workload (a bounded number of whole steps), timed on the host cores.

``secondary`` carries the other rows of the metric, each with its own
``roofline`` and ``cpu_baseline``: speculative verify (128 x 8 tokens), the
16-sequence varlen prefill, the 1M-token prefill (oracle resumed from the
GPU's checkpoints on a sample of segments, plus a continuous 65,536-token
run), the short conv at prefill scale, the varlen prefill from raw q/k/v
projections (conv + SiLU + q/k norm + prefill in one call), and the device
checkpoint planner.

``--workload prefill|long`` makes a prefill workload the main line.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
METRIC = "KDA prefill tokens/s (H=16,d=128) + decode/verify state GB/s vs HBM peak"
TRAFFIC_FILE = ROOT / "profiles" / "traffic.json"
MFMA_FILE = ROOT / "profiles" / "mfma.json"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=400)
    ap.add_argument("--workload", default="decode", choices=["decode", "prefill", "long"])
    ap.add_argument("--pools", type=int, default=4, help="rotating state pools (MALL defeat)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="CPU oracle time budget")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg")
    ap.add_argument("--long-cpu-segments", type=int, default=32,
                    help="segments of the 1M-token workload the oracle resumes (of 32)")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--pmc-pass", action="store_true",
                    help="run only the launches a rocprofv3 --pmc pass measures: a 256 MiB copy "
                         "(calibration), 8 decode steps, 2 varlen prefills")
    ap.add_argument("--ingest-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn the counter CSVs of two --pmc-pass runs into profiles/traffic.json")
    ap.add_argument("--pmc-long", action="store_true",
                    help="with --pmc-pass: also 2 calls of the 1M-token prefill (inputs drawn on the GPU)")
    ap.add_argument("--ingest-mfma", nargs="+", metavar="CSV",
                    help="turn the MFMA / VALU counter CSVs of --pmc-pass runs (MfmaUtil, VALUBusy, "
                         "SQ_INSTS_VALU_MFMA_MOPS_BF16, GRBM_GUI_ACTIVE) into profiles/mfma.json")
    return ap.parse_args()


def kernel_source_hash(name: str) -> str:
    """The kernel's source file together with the device headers it includes."""
    csrc = ROOT / "hybrid_recurrent_serving_amd" / "csrc"
    h = hashlib.sha256()
    for f in (name, "kda_device.h", "kda_internal.h", "kda_mfma.h"):
        h.update((csrc / f).read_bytes())
    return h.hexdigest()[:16]


def traffic_for(kernel_key: str, src_name: str, per_launch_units: float):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when it is missing or the kernel source has changed since."""
    if not TRAFFIC_FILE.exists():
        return None
    try:
        data = json.loads(TRAFFIC_FILE.read_text())
        ent = data[kernel_key]
    except (KeyError, ValueError):
        return None
    if ent.get("source_sha256_16") != kernel_source_hash(src_name):
        return None
    if ent.get("units_per_launch") != per_launch_units:
        return None
    return float(ent["hbm_bytes_per_launch"])


COPY_BYTES = 256 * 2 ** 20


PMC_PREFILL_CALLS = 3   # varlen prefill calls in a counter pass (2 warm-up + 1)
PMC_LONG_CALLS = 2      # 1M-token prefill calls in a counter pass with --pmc-long (1 warm-up + 1)


GEMM_N = 8192   # the MFMA calibration: a library bf16 GEMM of 2 GEMM_N^3 flops


def pmc_pass(torch, K, make_workload, long=False):
    """The launches the counter passes read: a plain device copy of a known
    size and a library bf16 GEMM of known flops (the calibrations), decode
    and fused decode steps over rotating pools, verify and fused verify
    calls, varlen prefills (and, with long, 1M-token prefills)."""
    dev = torch.device("cuda:0")
    a = torch.ones(COPY_BYTES // 4, device=dev)
    b = torch.empty_like(a)
    for _ in range(4):
        b.copy_(a)
    del a, b
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)
    ga = torch.randn(GEMM_N, GEMM_N, device=dev, generator=gen).to(torch.bfloat16).contiguous()
    gb = torch.randn(GEMM_N, GEMM_N, device=dev, generator=gen).to(torch.bfloat16).contiguous()
    for _ in range(2):
        gc = torch.mm(ga, gb)
    torch.cuda.synchronize()
    del ga, gb, gc
    wl = make_workload(1)
    N, H, D, P = 128, 16, 128, 4
    q, k, v, g, bt = (t.to(dev) for t in (wl.q, wl.k, wl.v, wl.g, wl.beta))
    pool = torch.empty(P * N, H, D, D, device=dev)
    for i in range(P):
        pool[i * N:(i + 1) * N] = wl.init_states.to(dev)
    o = torch.empty(N, H, D, dtype=torch.bfloat16, device=dev)
    for i in range(8):
        s_ = torch.arange((i % P) * N, (i % P + 1) * N, dtype=torch.int32, device=dev)
        K.kda_decode(q, k, v, g, bt, o, pool, s_, s_)
    wlc = make_workload(1, with_conv=True)
    x, cw = wlc.conv_x.to(dev), wlc.conv_w.to(dev)
    cpool = wlc.conv_state.to(dev).clone()
    cs = torch.arange(N, dtype=torch.int32, device=dev)
    z, gw = (t.to(dev) for t in out_gate_inputs(torch, (N, H, D), D, 401))
    for i in range(8):
        s_ = torch.arange((i % P) * N, (i % P + 1) * N, dtype=torch.int32, device=dev)
        K.kda_decode_conv(x, cw, cpool, cs, cs, g, bt, o, pool, s_, s_, act=1, qk_l2norm=True, out_gate=z,
                          out_norm_weight=gw)
    del pool
    bench_verify_secondary(torch, K, make_workload, dev, n=2, warm=2)   # 4 verify + 4 fused verify calls
    torch.cuda.empty_cache()
    bench_prefill_varlen(torch, K, make_workload, dev, iters=1, warm=PMC_PREFILL_CALLS - 1)
    torch.cuda.synchronize()
    if long:
        torch.cuda.empty_cache()
        bench_prefill_long(torch, K, make_workload, dev, iters=1, warm=PMC_LONG_CALLS - 1)
        torch.cuda.synchronize()
    # the conv at prefill scale (3 + 1 launches) and the prefill from raw
    # projections (3 calls, 3 prefills alone, 3 conv + norm launches alone),
    # after every prefill call the ingest counts by position
    torch.cuda.empty_cache()
    wl2 = make_workload(2)
    bench_conv_prefill(torch, K, wl2, dev, iters=1, warm=3)
    torch.cuda.empty_cache()
    bench_prefill_conv(torch, K, wl2, dev, iters=1, warm=2)
    torch.cuda.synchronize()


def varlen_tokens():
    from hybrid_recurrent_serving_amd.inputs import make_workload
    return int(make_workload(2).cu_seqlens[-1])


def check_prefill_calls(first_grids):
    """The counter pass's varlen prefill calls and its 1M-token calls launch
    pass A on different grids: first_grids holds the grid of each call's
    first prefill-kernel dispatch, in call order (None where the CSV has no
    grid column).  Calls whose grids do not fall into the expected groups
    mean the pass's call counts are out of step with PMC_PREFILL_CALLS and
    PMC_LONG_CALLS: the ingestion stops rather than mix the workloads."""
    v = first_grids[:PMC_PREFILL_CALLS]
    lg = first_grids[PMC_PREFILL_CALLS:PMC_PREFILL_CALLS + PMC_LONG_CALLS]
    if None in v + lg:
        return
    if len(set(v)) > 1 or (lg and (len(set(lg)) > 1 or lg[0] == v[0])):
        raise SystemExit(f"prefill calls out of step with the counter pass: pass-A grids {first_grids[:8]}")


def ingest_pmc(fetch_csv, write_csv):
    """Per-launch HBM bytes of the decode and prefill kernels from FETCH_SIZE
    and WRITE_SIZE (KiB per dispatch), each scaled by the factor that makes
    the calibration copy read and write exactly COPY_BYTES."""
    import csv
    out = {}
    rows = {}
    for name, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows[name] = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == name]

    def sel(name, pred):
        return [float(r["Counter_Value"]) * 1024 for r in rows[name] if pred(r)]

    def is_copy(r):
        return r["Kernel_Name"].startswith("__amd_rocclr_copyBuffer")

    cw = [x for x in sel("WRITE_SIZE", is_copy) if abs(x - COPY_BYTES) < 0.25 * COPY_BYTES]
    cf = sel("FETCH_SIZE", is_copy)
    cf = sorted(cf)[-len(cw):] if cw else []
    if not cw or not cf:
        raise SystemExit("calibration copy not found in the counter files")
    f_scale = COPY_BYTES / (sum(cf) / len(cf))
    w_scale = COPY_BYTES / (sum(cw) / len(cw))
    def named(part):
        return lambda r: part in r["Kernel_Name"].replace(" ", "")

    for key, pred, src, units in (
            ("decode_step_kernel_d128_bf16", lambda r: is_decode128(r["Kernel_Name"], 0), "kda_step.hip",
             128 * 16),
            ("decode_conv_kernel_d128_bf16", lambda r: is_decode128(r["Kernel_Name"], 4),
             "kda_step.hip", 128 * 16),
            ("verify_kernel_d128_bf16", named("vf::verify_kernel<unsignedshort>"),
             "kda_verify.hip", 128 * 16),
            ("verify_conv_kernel_d128_bf16", named("vf::verify_conv_kernel<unsignedshort,4,8>"),
             "kda_verify.hip", 128 * 16),
            ("conv_kernel_prefill_bf16", named("conv_kernel<unsignedshort,4,0>"), "kda_conv.hip", varlen_tokens()),
            ("conv_norm_kernel_prefill_bf16", named("conv_kernel<unsignedshort,4,16>"), "kda_conv.hip",
             varlen_tokens())):
        f = sel("FETCH_SIZE", pred)
        w = sel("WRITE_SIZE", pred)
        if not f or not w:
            continue
        fb = sum(f) / len(f) * f_scale
        wb = sum(w) / len(w) * w_scale
        out[key] = {"hbm_bytes_per_launch": round(fb + wb), "fetch_bytes": round(fb), "write_bytes": round(wb),
                    "source_sha256_16": kernel_source_hash(src), "units_per_launch": units,
                    "dispatches": len(f)}
    # prefill calls: each starts with its segment plan launch; the pass's
    # varlen calls come first, then (with --pmc-long) the 1M-token ones.  Per
    # call: every prefill-kernel dispatch of the call, averaged over calls.
    per_call = {}
    for name in ("FETCH_SIZE", "WRITE_SIZE"):
        calls, grids = [], []
        for r in sorted(rows[name], key=lambda r: int(r["Dispatch_Id"])):
            if "segment_plan_kernel" in r["Kernel_Name"]:
                calls.append(0.0)
                grids.append(False)
            elif calls and "prefill_kernel<128" in r["Kernel_Name"]:
                calls[-1] += float(r["Counter_Value"]) * 1024
                if grids[-1] is False:
                    grids[-1] = r.get("Grid_Size")
        check_prefill_calls(grids)
        per_call[name] = calls
    for key, c0, nc, units in (("prefill_kernel_d128_bf16", 0, PMC_PREFILL_CALLS, varlen_tokens()),
                               ("prefill_long_kernel_d128_bf16", PMC_PREFILL_CALLS, PMC_LONG_CALLS, 1 << 20)):
        f = per_call["FETCH_SIZE"][c0:c0 + nc]
        w = per_call["WRITE_SIZE"][c0:c0 + nc]
        if len(f) != nc or len(w) != nc:
            continue
        fb = sum(f) / nc * f_scale
        wb = sum(w) / nc * w_scale
        out[key] = {"hbm_bytes_per_launch": round(fb + wb), "fetch_bytes": round(fb), "write_bytes": round(wb),
                    "source_sha256_16": kernel_source_hash("kda_prefill.hip"), "units_per_launch": units,
                    "calls": nc}
    out["calibration"] = {"copy_bytes": COPY_BYTES, "fetch_scale": round(f_scale, 4),
                          "write_scale": round(w_scale, 4),
                          "note": "FETCH_SIZE / WRITE_SIZE of a plain device copy of copy_bytes, "
                                  "scaled to read and write exactly copy_bytes"}
    return out


def ingest_mfma(paths):
    """Per-call MFMA and VALU figures of the prefill kernels from the counter
    CSVs of --pmc-pass runs: executed bf16 MFMA flops (SQ_INSTS_VALU_MFMA_MOPS_BF16
    x 512), and MfmaUtil / VALUBusy averaged over the call's dispatches with
    GRBM_GUI_ACTIVE (active cycles) as the weight; the same busy figures for
    the decode and verify kernels.  The calibration is the
    pass's library GEMM of 2 GEMM_N^3 flops: its executed flops check the x 512
    scale, its MfmaUtil shows what a dense library kernel reaches."""
    import csv
    out = {}
    want = GEMM_N ** 3 * 2
    for path in paths:
        disp = {}
        for r in csv.DictReader(open(path)):
            d = disp.setdefault(int(r["Dispatch_Id"]), {"name": r["Kernel_Name"], "grid": r.get("Grid_Size")})
            d[r["Counter_Name"]] = float(r["Counter_Value"])
        order = [disp[i] for i in sorted(disp)]
        need = ("MfmaUtil", "VALUBusy", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "GRBM_GUI_ACTIVE")
        order = [d for d in order if all(c in d for c in need)]
        gemm = [d for d in order if abs(d["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512 - want) < 0.1 * want]
        if gemm and "calibration_gemm" not in out:
            g = gemm[-1]
            out["calibration_gemm"] = {
                "flops": want, "executed_flops": g["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512,
                "mfma_util": round(g["MfmaUtil"] / 100, 4), "valu_busy": round(g["VALUBusy"] / 100, 4),
                "kernel": g["name"][:120],
                "note": f"torch.mm of two {GEMM_N} x {GEMM_N} bf16 matrices (library GEMM)"}
        # the decode and verify kernels: MfmaUtil / VALUBusy averaged over
        # their dispatches, weighted by active cycles
        for key, pred, src in (
                ("decode_conv_kernel_d128_bf16", lambda n: is_decode128(n, 4), "kda_step.hip"),
                ("decode_step_kernel_d128_bf16", lambda n: is_decode128(n, 0), "kda_step.hip"),
                ("verify_kernel_d128_bf16", lambda n: n.startswith("void kda::vf::verify_kernel<unsigned short>"),
                 "kda_verify.hip"),
                ("verify_conv_kernel_d128_bf16",
                 lambda n: n.startswith("void kda::vf::verify_conv_kernel<unsigned short, 4, 8>"),
                 "kda_verify.hip")):
            ds = [d for d in order if pred(d["name"])]
            if not ds or key in out:
                continue
            w = sum(d["GRBM_GUI_ACTIVE"] for d in ds)
            out[key] = {"dispatches": len(ds),
                        "mfma_util": round(sum(d["MfmaUtil"] * d["GRBM_GUI_ACTIVE"] for d in ds) / w / 100, 4),
                        "valu_busy": round(sum(d["VALUBusy"] * d["GRBM_GUI_ACTIVE"] for d in ds) / w / 100, 4),
                        "source_sha256_16": kernel_source_hash(src)}
        # calls: each prefill call starts with its segment plan launch
        calls, cur = [], None
        for d in order:
            if "segment_plan_kernel" in d["name"]:
                cur = []
                calls.append(cur)
            elif cur is not None and ("prefill_kernel<" in d["name"] or "segment_combine_kernel" in d["name"]):
                cur.append(d)
        check_prefill_calls([next((d.get("grid") for d in c if "prefill_kernel<" in d["name"]), None)
                             for c in calls])
        groups = [("prefill_varlen", calls[:PMC_PREFILL_CALLS], varlen_tokens())]
        if len(calls) >= PMC_PREFILL_CALLS + PMC_LONG_CALLS:
            groups.append(("prefill_long_1m", calls[PMC_PREFILL_CALLS:PMC_PREFILL_CALLS + PMC_LONG_CALLS],
                           1 << 20))
        for key, grp, tokens in groups:
            if not grp or key in out:
                continue
            last = grp[-1]   # the measured call (the ones before it warm up)
            w = sum(d["GRBM_GUI_ACTIVE"] for d in last)
            ex = sum(d["SQ_INSTS_VALU_MFMA_MOPS_BF16"] for d in last) * 512
            alg = tokens * PREFILL_FLOPS_PER_TOKEN
            out[key] = {
                "tokens": tokens, "dispatches": len(last), "alg_flops": alg, "executed_bf16_flops": ex,
                "executed_over_alg": round(ex / alg, 4),
                "mfma_util": round(sum(d["MfmaUtil"] * d["GRBM_GUI_ACTIVE"] for d in last) / w / 100, 4),
                "valu_busy": round(sum(d["VALUBusy"] * d["GRBM_GUI_ACTIVE"] for d in last) / w / 100, 4),
                "per_dispatch": [{"kernel": d["name"].split("(")[0][-60:],
                                  "role": ("combine" if "combine" in d["name"] else
                                           "pass A" if i == 0 else "fix-up"),
                                  "mfma_util": round(d["MfmaUtil"] / 100, 4),
                                  "valu_busy": round(d["VALUBusy"] / 100, 4),
                                  "executed_bf16_flops": d["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512}
                                 for i, d in enumerate(last)],
                "source_sha256_16": kernel_source_hash("kda_prefill.hip")}
    return out


def mfma_counters(key: str, tokens: int, ms: float):
    """The committed counter figures of a prefill workload (None when missing
    or when the kernel source has changed since), with the executed MFMA rate
    at this run's call time."""
    if not MFMA_FILE.exists():
        return None
    try:
        ent = json.loads(MFMA_FILE.read_text())[key]
    except (KeyError, ValueError):
        return None
    if ent.get("source_sha256_16") != kernel_source_hash("kda_prefill.hip") or ent.get("tokens") != tokens:
        return None
    rate = ent["executed_bf16_flops"] / (ms * 1e-3) / 1e12
    return {"executed_bf16_flops_per_call": ent["executed_bf16_flops"],
            "executed_over_alg": ent["executed_over_alg"],
            "executed_tflops": round(rate, 1), "executed_frac": round(rate / MFMA_BF16_PEAK_TFLOPS, 4),
            "mfma_util": ent["mfma_util"], "valu_busy": ent["valu_busy"],
            "source": "rocprofv3 --pmc MfmaUtil VALUBusy SQ_INSTS_VALU_MFMA_MOPS_BF16 GRBM_GUI_ACTIVE"}


def is_decode128(kernel_name: str, W: int) -> bool:
    """The d = 128 decode kernel with bf16 inputs and outputs (one workgroup
    of four waves per head): plain (W = 0) or with the W-tap conv fused in."""
    return kernel_name.replace(" ", "").endswith(
        f"decode128_kernel<unsignedshort,unsignedshort,{W}>(kda::Dec128Args)")


def cpu_info():
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return model


# ---------------------------------------------------------------- decode
def out_gate_inputs(torch, shape, D, seed):
    """Output gate logits N(0, 1) and the shared norm weight 1 + 0.1 N(0, 1)
    (bf16, on the host)."""
    gen = torch.Generator().manual_seed(seed)
    z = torch.randn(*shape, generator=gen).to(torch.bfloat16)
    w = (1.0 + 0.1 * torch.randn(D, generator=gen)).to(torch.bfloat16)
    return z, w


def bench_decode(args, torch, K, make_workload):
    dev = torch.device("cuda:0")
    N, H, D, W = 128, 16, 128, 4
    C = 3 * H * D
    wl = make_workload(1, with_conv=True)
    q, k, v, g, b = (t.to(dev) for t in (wl.q, wl.k, wl.v, wl.g, wl.beta))
    P = args.pools
    pool = torch.empty(P * N, H, D, D, device=dev)
    for i in range(P):
        pool[i * N:(i + 1) * N] = wl.init_states.to(dev)
    slot_sets = [torch.arange(i * N, (i + 1) * N, dtype=torch.int32, device=dev) for i in range(P)]
    o = torch.empty(N, H, D, dtype=torch.bfloat16, device=dev)
    x = wl.conv_x.to(dev)
    cw = wl.conv_w.to(dev)
    cpool = wl.conv_state.to(dev).clone()
    cslots = torch.arange(N, dtype=torch.int32, device=dev)
    cu = wl.cu_seqlens.to(dev)
    y = torch.empty_like(x)

    # argument structs checked once; the timed loops only enqueue
    conv_call = K.prepare_conv_short(x, cw, cu, cpool, cslots, cslots, y=y)
    dec_calls = [K.prepare_decode(q, k, v, g, b, o, pool, s_, s_) for s_ in slot_sets]
    # the fused step: conv (+ SiLU) of the token's q / k / v projections,
    # per-head q / k L2 normalisation, the recurrence and the gated RMS norm
    # of the output in one launch; the conv history advances in place like
    # the state
    z_h, gw_h = out_gate_inputs(torch, (N, H, D), D, 401)
    z, gw = z_h.to(dev), gw_h.to(dev)
    fused_calls = [K.prepare_decode_conv(x, cw, cpool, cslots, cslots, g, b, o, pool, s_, s_, act=1,
                                         qk_l2norm=True, out_gate=z, out_norm_weight=gw) for s_ in slot_sets]

    def timed(step_fn, nsteps, nwarm):
        """Per-step time over nsteps back-to-back steps, then (in a second
        pass, so that the event records do not stretch the steps) the average
        duration of the recurrent kernel's launch from HIP events around it
        on its stream."""
        for i in range(nwarm):
            step_fn(i, None)
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        w0 = time.perf_counter()
        t0.record()
        for i in range(nsteps):
            step_fn(i, None)
        t1.record()
        torch.cuda.synchronize()
        wall_ = time.perf_counter() - w0
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(nsteps)]
        for i in range(nsteps):
            step_fn(i, evs[i])
        torch.cuda.synchronize()
        return (t0.elapsed_time(t1) / nsteps, sum(a_.elapsed_time(b_) for a_, b_ in evs) / nsteps, wall_)

    def fused_step(i, ev):
        if ev is not None:
            ev[0].record()
        fused_calls[i % P]()
        if ev is not None:
            ev[1].record()

    def two_call_step(i, ev):
        conv_call()
        if ev is not None:
            ev[0].record()
        dec_calls[i % P]()
        if ev is not None:
            ev[1].record()

    ms_step, _, wall = timed(fused_step, args.steps, args.warmup)
    # one launch per step: the launch's average duration is the timed
    # region (HIP events on the launch stream) over the launch count
    k_ms = ms_step

    state_bytes = N * H * D * D * 4 * 2                   # read + write
    # fused step per launch: state r+w, the token's q/k/v projections, the
    # conv history r+w, g, beta and the output gate in, o out (bf16), the
    # conv taps and the norm weight once
    conv_hist_bytes = N * C * (W - 1) * 2 * 2
    io_bytes = N * C * 2 + N * H * (D * 2 + 2 + D * 2 + D * 2) + C * W * 2 + D * 2
    alg_bytes = state_bytes + conv_hist_bytes + io_bytes
    value = state_bytes / (ms_step * 1e-3) / 1e9
    achieved = alg_bytes / (k_ms * 1e-3) / 1e9
    traffic = traffic_for("decode_conv_kernel_d128_bf16", "kda_step.hip", N * H)
    roof = {"kernel": "decode128_kernel<bf16,bf16,W=4> (kda_decode_conv)", "bound": "hbm",
            "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
            "alg_bytes_per_launch": alg_bytes, "avg_launch_us": round(k_ms * 1e3, 3)}

    secondary = {}
    if not args.no_secondary:
        # the same step as two launches: kda_conv_short, then kda_decode on
        # separately drawn (normalised) q / k / v
        ms2, k2, _ = timed(two_call_step, min(args.steps, 200), 10)
        dec_alg = state_bytes + N * H * (4 * D * 2 + 2 + D * 2)
        secondary["two_call_step"] = {
            "step": "kda_conv_short + kda_decode", "us_per_step": round(ms2 * 1e3, 2),
            "state_GB_s": round(state_bytes / (ms2 * 1e-3) / 1e9, 1),
            "decode_kernel": {"avg_launch_us": round(k2 * 1e3, 3), "alg_bytes_per_launch": dec_alg,
                              "GB_s": round(dec_alg / (k2 * 1e-3) / 1e9, 1),
                              "traffic": traffic_for("decode_step_kernel_d128_bf16", "kda_step.hip", N * H)}}
        # hot: one pool only (state may sit in the Infinity Cache) -- labelled, not the value
        s0 = slot_sets[0]
        for _ in range(20):
            K.kda_decode(q, k, v, g, b, o, pool, s0, s0)
        a_, b2 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a_.record()
        for _ in range(200):
            K.kda_decode(q, k, v, g, b, o, pool, s0, s0)
        b2.record()
        torch.cuda.synchronize()
        hot_us = a_.elapsed_time(b2) / 200 * 1e3
        secondary["decode_hot_single_pool"] = {"us": round(hot_us, 2),
                                               "GB_s": round(dec_alg / hot_us / 1e3, 1)}
        # plain device copy of the same bytes (torch copy kernel) as a practical ceiling
        src_t = torch.empty(state_bytes // 8, dtype=torch.float32, device=dev)
        dst_t = torch.empty_like(src_t)
        srcs = [torch.empty_like(src_t) for _ in range(3)] + [src_t]
        dsts = [torch.empty_like(dst_t) for _ in range(3)] + [dst_t]
        for i in range(8):
            dsts[i % 4].copy_(srcs[i % 4])
        torch.cuda.synchronize()
        a_.record()
        for i in range(100):
            dsts[i % 4].copy_(srcs[i % 4])
        b2.record()
        torch.cuda.synchronize()
        cp_us = a_.elapsed_time(b2) / 100 * 1e3
        secondary["copy_same_bytes"] = {"us": round(cp_us, 2),
                                        "GB_s": round(state_bytes / cp_us / 1e3, 1)}
        del srcs, dsts, src_t, dst_t
        cs = 0.0 if args.no_cpu else args.cpu_seconds
        secondary["verify"] = bench_verify_secondary(torch, K, make_workload, dev, cpu_seconds=min(cs, 4.0))
        secondary["ckpt_plan_device"] = bench_planner_secondary(torch, K, dev)
        wl2 = make_workload(2)
        secondary["prefill_varlen"] = bench_prefill_varlen(torch, K, make_workload, dev, iters=10, wl=wl2,
                                                           cpu_seconds=cs)
        secondary["conv_prefill_scale"] = bench_conv_prefill(torch, K, wl2, dev)
        torch.cuda.empty_cache()
        secondary["prefill_conv"] = bench_prefill_conv(torch, K, wl2, dev, cpu_seconds=cs)
        del wl2
        torch.cuda.empty_cache()
        secondary["prefill_long_1m"] = bench_prefill_long(
            torch, K, make_workload, dev, cpu_segments=0 if args.no_cpu else args.long_cpu_segments)

    cpu = None
    if not args.no_cpu:
        cpu = cpu_decode(args, wl, state_bytes, z_h, gw_h)
    cfg = {"workload": "batched decode: 128 seqs x 1 token, H=16, d_k=d_v=128, conv W=4 "
                       "over 6144 q/k/v channels, bf16 inputs, fp32 state",
           "n_seq": N, "H": H, "d": D, "conv_W": W, "state_pools_rotated": P,
           "step": "kda_decode_conv (conv + SiLU of the q/k/v projections, q/k L2 norm, recurrence, "
                   "sigmoid-gated RMS norm of the output; one launch)",
           "value_counts": "recurrent state read+write"}
    return {"metric": METRIC, "value": round(value, 1), "unit": "GB/s", "ms_per_step": ms_step,
            "dtype": "f32", "config": cfg, "roofline": roof, "cpu_baseline": cpu,
            "secondary": secondary, "wall_s": round(wall, 3)}


def bench_planner_secondary(torch, K, dev, iters=200):
    """Latency of the device checkpoint plan (kda_ckpt_plan_device): device
    time per call from a HIP graph that holds `iters` back-to-back calls
    (replay time over the call count, so host enqueue cost is excluded), and
    the host time to enqueue one call eagerly through the binding (argument
    marshalling, validation, two launches).  Checkpoint interval 4096,
    chunk 64."""
    gen = torch.Generator().manual_seed(4242)
    cases = {"batch1_32k": [32768],
             "varlen16": (16, 512, 16384),
             "batch1024": (1024, 1, 16384)}
    out = {}
    for name, spec in cases.items():
        if isinstance(spec, list):
            lens = torch.tensor(spec)
        else:
            n, lo, hi = spec
            lens = torch.randint(lo, hi + 1, (n,), generator=gen)
        cu = torch.zeros(lens.numel() + 1, dtype=torch.int32)
        cu[1:] = torch.cumsum(lens, 0)
        n_seq, T = lens.numel(), int(cu[-1])
        cap = int(sum((int(L) - 1) // 4096 for L in lens.tolist())) + 1
        cu_d = cu.to(dev)
        free = torch.arange(cap, dtype=torch.int32, device=dev)
        outs = dict(ckpt_cu=torch.empty(n_seq + 1, dtype=torch.int32, device=dev),
                    ckpt_pos=torch.empty(cap, dtype=torch.int32, device=dev),
                    ckpt_slot=torch.empty(cap, dtype=torch.int32, device=dev),
                    n_total=torch.empty(1, dtype=torch.int32, device=dev))
        call = lambda: K.kda_ckpt_plan_device(cu_d, 4096, 64, T, cap=cap, free_slots=free, **outs)  # noqa: E731
        for _ in range(10):
            call()
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        for _ in range(iters):
            call()
        host_us = (time.perf_counter() - w0) / iters * 1e6
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(iters):
                call()
        graph.replay()
        torch.cuda.synchronize()
        a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a_.record()
        graph.replay()
        b_.record()
        torch.cuda.synchronize()
        out[name] = {"n_seq": n_seq, "checkpoints": int(outs["n_total"].item()),
                     "graph_us_per_call": round(a_.elapsed_time(b_) / iters * 1e3, 2),
                     "host_enqueue_us_per_call": round(host_us, 2)}
        del graph
    return out


# Untimed calls before the verify timings: after the pools are filled from
# the host (or any idle gap) the first ~200 calls run slower while the
# clocks ramp up (65 us, then 56.5 us per block of 100 calls, then 54.0-54.6
# us steady); 400 calls (~22 ms) start the timed region at the steady rate.
VERIFY_WARMUP = 400


def bench_verify_secondary(torch, K, make_workload, dev, n=200, warm=VERIFY_WARMUP, cpu_seconds=0.0):
    """Speculative verify (128 x 8 tokens, fused commit) -- reported beside the
    decode line.  n timed calls of each form after warm untimed ones, each a
    prepared call (argument struct built once per state pool, as for the
    decode step), so the host does not pace the launches."""
    wl = make_workload(4)
    N, Ts, H, D = 128, 8, 16, 128
    q, k, v, g, b = (t.to(dev) for t in (wl.q, wl.k, wl.v, wl.g, wl.beta))
    P = 4
    pool = torch.empty(P * N, H, D, D, device=dev)
    for i in range(P):
        pool[i * N:(i + 1) * N] = wl.init_states.to(dev)
    slot_sets = [torch.arange(i * N, (i + 1) * N, dtype=torch.int32, device=dev) for i in range(P)]
    L = wl.accepted_len.to(dev)
    o = torch.empty(N, Ts, H, D, dtype=torch.bfloat16, device=dev)
    calls = [K.prepare_verify(q, k, v, g, b, pool, s, s, o=o, accepted_len=L) for s in slot_sets]
    for i in range(warm):
        calls[i % P]()
    a_, b2 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a_.record()
    for i in range(n):
        calls[i % P]()
    b2.record()
    torch.cuda.synchronize()
    us = a_.elapsed_time(b2) / n * 1e3
    state_bytes = N * H * D * D * 4 * 2
    io = N * Ts * H * (4 * D * 2 + 2 + D * 2)
    alg = state_bytes + io
    res = {"workload": "verify 128 x 8 tokens, fused commit at L~U{1..8}", "us": round(us, 2),
           "state_GB_s": round(state_bytes / us / 1e3, 1),
           "alg_GB_s": round(alg / us / 1e3, 1),
           "hbm_frac": round(alg / us / 1e3 / HBM_PEAK_GBS, 4),
           "roofline": {"kernel": "verify_kernel<bf16> (kda_verify on bf16 matrix cores, one launch per call)",
                        "bound": "hbm", "achieved": round(alg / us / 1e3, 1), "peak": HBM_PEAK_GBS,
                        "unit": "GB/s", "frac": round(alg / us / 1e3 / HBM_PEAK_GBS, 4),
                        "traffic": traffic_for("verify_kernel_d128_bf16", "kda_verify.hip", N * H),
                        "alg_bytes_per_launch": alg, "avg_launch_us": round(us, 3)}}
    if cpu_seconds > 0:
        res["cpu_baseline"] = cpu_verify(wl, state_bytes, cpu_seconds)
    # the same verify from the tokens' raw q/k/v projections with the conv
    # (+ SiLU), q/k normalisation and both commits fused (kda_verify_conv)
    from hybrid_recurrent_serving_amd.inputs import draw_conv
    C, W = 3 * H * D, 4
    gen = torch.Generator().manual_seed(4)
    cw, cst, x = draw_conv(gen, N * Ts, C, W, N, torch.bfloat16, torch.device("cpu"))
    x = x.reshape(N, Ts, C).to(dev)
    cw = cw.to(dev)
    cpool = cst.to(dev)
    cs = torch.arange(N, dtype=torch.int32, device=dev)
    z, gw = (t.to(dev) for t in out_gate_inputs(torch, (N, Ts, H, D), D, 404))
    ccalls = [K.prepare_verify_conv(x, cw, cpool, cs, cs, g, b, pool, s, s, o=o, accepted_len=L, act=1,
                                    out_gate=z, out_norm_weight=gw) for s in slot_sets]
    for i in range(warm):
        ccalls[i % P]()
    torch.cuda.synchronize()
    a_.record()
    for i in range(n):
        ccalls[i % P]()
    b2.record()
    torch.cuda.synchronize()
    us2 = a_.elapsed_time(b2) / n * 1e3
    io2 = N * Ts * (C * 2 + H * (D * 2 + 2 + D * 2 + D * 2)) + N * C * (W - 1) * 2 * 2 + C * W * 2 + D * 2
    alg2 = state_bytes + io2
    res["fused_conv"] = {"call": "kda_verify_conv (conv + SiLU + q/k norm + verify + gated output norm, "
                                 "state and conv history committed at L)", "us": round(us2, 2),
                         "state_GB_s": round(state_bytes / us2 / 1e3, 1),
                         "alg_GB_s": round(alg2 / us2 / 1e3, 1),
                         "hbm_frac": round(alg2 / us2 / 1e3 / HBM_PEAK_GBS, 4),
                         "roofline": {"kernel": "verify_conv_kernel<bf16,W=4,window 8> (kda_verify_conv on bf16 "
                                                "matrix cores, one launch per call)", "bound": "hbm",
                                      "achieved": round(alg2 / us2 / 1e3, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                      "frac": round(alg2 / us2 / 1e3 / HBM_PEAK_GBS, 4),
                                      "traffic": traffic_for("verify_conv_kernel_d128_bf16", "kda_verify.hip", N * H),
                                      "alg_bytes_per_launch": alg2, "avg_launch_us": round(us2, 3)}}
    return res


PREFILL_BYTES_PER_TOKEN = 16 * (4 * 128 * 2 + 2 + 128 * 2)      # q,k,v,g + beta + o (bf16), H=16
PREFILL_FLOPS_PER_TOKEN = 16 * (10 * 64 * 128 + 6 * 128 * 128)    # dense chunked count at C=64


# Untimed calls before a prefill-sized timing: the first calls on freshly
# allocated buffers run up to ~8% slower than the steady state measured after
# them (inputs resident in HBM).
PREFILL_WARMUP = 10

# Segment length of the varlen prefill: sequences of >= 2 segments run as
# parallel segments (a caller-chosen launch parameter; same function of the
# inputs up to rounding), which shortens the longest sequence's chain.  On
# this workload (same-process sweep, 4 x 20 calls): 2,048 -> 1.57 ms, 2,560
# -> 1.58, 3,072 -> 1.455, 3,584 -> 1.64, 4,096 -> 1.50, 5,120 -> 1.52,
# 6,144 -> 1.71, 8,192 -> 1.59; the segments' packing onto the CUs decides.
VARLEN_SEGMENT = 3072


def bench_prefill_varlen(torch, K, make_workload, dev, iters=20, wl=None, cpu_seconds=0.0, warm=PREFILL_WARMUP):
    """16 packed sequences, lengths U{512..16384}, H=16, d=128, chunk 64,
    even sequences from random initial states, final states to fresh slots."""
    if wl is None:
        wl = make_workload(2)
    N, H, D = wl.n_seq, 16, 128
    q, k, v, g, b = (t.to(dev) for t in (wl.q, wl.k, wl.v, wl.g, wl.beta))
    T = q.shape[0]
    pool = torch.zeros(2 * N, H, D, D, device=dev)
    for s_, i in enumerate(wl.init_index):
        if i >= 0:
            pool[s_] = wl.init_states[i].to(dev)
    src = torch.tensor([s_ if i >= 0 else -1 for s_, i in enumerate(wl.init_index)], dtype=torch.int32,
                       device=dev)
    dst = torch.arange(N, 2 * N, dtype=torch.int32, device=dev)
    cu = wl.cu_seqlens.to(dev)
    o = torch.empty(T, H, D, dtype=torch.bfloat16, device=dev)
    nws = K.kda_prefill_workspace_bytes(q, k, v, g, b, o, cu, pool, src, dst, chunk=64,
                                        segment_len=VARLEN_SEGMENT)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)

    def run():
        K.kda_prefill_varlen(q, k, v, g, b, o, cu, pool, src, dst, chunk=64, workspace=ws,
                             segment_len=VARLEN_SEGMENT)

    for _ in range(warm):
        run()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
    torch.cuda.synchronize()
    for e0, e1 in evs:
        e0.record()
        run()
        e1.record()
    torch.cuda.synchronize()
    ms = sum(a.elapsed_time(b_) for a, b_ in evs) / iters
    tps = T / (ms * 1e-3)
    res = {"workload": "varlen prefill: 16 seqs, lengths U{512..16384}, H=16, d=128, chunk 64, bf16",
           "tokens": T, "ms": round(ms, 4), "tokens_per_s": round(tps, 1),
           "alg_mfma_frac": round(tps * PREFILL_FLOPS_PER_TOKEN / (MFMA_BF16_PEAK_TFLOPS * 1e12), 4),
           "alg_hbm_frac": round(tps * PREFILL_BYTES_PER_TOKEN / (HBM_PEAK_GBS * 1e9), 4),
           "roofline": prefill_roofline("prefill_kernel<128,bf16,bf16> (kda_prefill_varlen call: segment plan, "
                                        "pass A, combine, fix-up)", T, ms, "prefill_varlen",
                                        "prefill_kernel_d128_bf16")}
    if cpu_seconds > 0:
        res["cpu_baseline"] = cpu_prefill(cpu_seconds, wl)
    return res


def prefill_roofline(kernel, T, ms, counters_key, traffic_key):
    """Both rooflines of a prefill call: algorithmic bytes against 8 TB/s
    (the tighter bound at these shapes) and algorithmic MFMA flops against
    the bf16 dense peak; the call's whole time (all its launches)."""
    achieved = T * PREFILL_BYTES_PER_TOKEN / (ms * 1e-3) / 1e9
    tflops = T * PREFILL_FLOPS_PER_TOKEN / (ms * 1e-3) / 1e12
    return {"kernel": kernel, "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic_for(traffic_key, "kda_prefill.hip", T),
            "alg_bytes_per_launch": T * PREFILL_BYTES_PER_TOKEN, "avg_launch_us": round(ms * 1e3, 2),
            "mfma": {"alg_flops_per_launch": T * PREFILL_FLOPS_PER_TOKEN, "achieved_tflops": round(tflops, 1),
                     "peak_tflops": MFMA_BF16_PEAK_TFLOPS, "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                     "counters": mfma_counters(counters_key, T, ms)}}


def bench_conv_prefill(torch, K, wl, dev, iters=20, warm=PREFILL_WARMUP):
    """kda_conv_short at prefill scale: the varlen workload's 16 sequences
    (140,625 tokens) over the 3 H d = 6,144 q/k/v channels, W = 4 with SiLU,
    bf16, carried conv history read from and written to per-sequence slots.
    Algorithmic bytes: x in and y out (2 B each per element), the history
    read and written, the taps."""
    from hybrid_recurrent_serving_amd.inputs import draw_conv
    N, C, W = wl.n_seq, 3 * 16 * 128, 4
    T = int(wl.cu_seqlens[-1])
    gen = torch.Generator().manual_seed(2)
    cw, cst, x = draw_conv(gen, T, C, W, N, torch.bfloat16, torch.device("cpu"))
    x, cw = x.to(dev), cw.to(dev)
    cpool = torch.cat([cst, torch.zeros_like(cst)]).to(dev)
    src = torch.arange(N, dtype=torch.int32, device=dev)
    dst = src + N
    cu = wl.cu_seqlens.to(dev)
    y = torch.empty_like(x)
    call = K.prepare_conv_short(x, cw, cu, cpool, src, dst, y=y, act=1)
    for _ in range(warm):
        call()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(iters):
        call()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / iters * 1e3
    alg = 2 * T * C * 2 + 2 * N * C * (W - 1) * 2 + C * W * 2
    gbs = alg / us / 1e3
    return {"workload": f"short conv + SiLU, {T} tokens (16 packed sequences) x {C} channels, W=4, bf16, "
                        "carried history in slots", "us": round(us, 2),
            "roofline": {"kernel": "conv_kernel<bf16,4> (kda_conv_short)", "bound": "hbm",
                         "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "traffic": traffic_for("conv_kernel_prefill_bf16", "kda_conv.hip", T),
                         "alg_bytes_per_launch": alg, "avg_launch_us": round(us, 3)}}


def bench_prefill_conv(torch, K, wl, dev, iters=10, cpu_seconds=0.0, warm=PREFILL_WARMUP):
    """kda_prefill_varlen_conv on the varlen workload: the 16 sequences'
    raw q / k / v projections (6,144 channels, bf16) through the conv
    (W = 4, carried history, SiLU), the per-head q / k normalisation and the
    chunked prefill (chunk 64, 3,072-token segments), gates, beta and initial
    states as the varlen row.  Two launches per call (conv + norm, then the
    prefill); each is also timed alone on the same data (the conv through
    kda_conv_short with the same normalisation, the prefill through
    kda_prefill_varlen on the formed operands).  Run back to back inside the
    call, the prefill reads what the conv has just written and measures
    somewhat slower than alone."""
    from hybrid_recurrent_serving_amd.inputs import draw_conv
    N, H, D, W = wl.n_seq, 16, 128, 4
    C = 3 * H * D
    T = int(wl.cu_seqlens[-1])
    gen = torch.Generator().manual_seed(2)
    cw, cst, x = draw_conv(gen, T, C, W, N, torch.bfloat16, torch.device("cpu"))
    x_d, cw_d = x.to(dev), cw.to(dev)
    cpool = torch.cat([cst, torch.zeros_like(cst)]).to(dev)
    csrc = torch.arange(N, dtype=torch.int32, device=dev)
    cdst = csrc + N
    g, b = wl.g.to(dev), wl.beta.to(dev)
    pool = torch.zeros(2 * N, H, D, D, device=dev)
    for s_, i in enumerate(wl.init_index):
        if i >= 0:
            pool[s_] = wl.init_states[i].to(dev)
    src = torch.tensor([s_ if i >= 0 else -1 for s_, i in enumerate(wl.init_index)], dtype=torch.int32,
                       device=dev)
    dst = torch.arange(N, 2 * N, dtype=torch.int32, device=dev)
    cu = wl.cu_seqlens.to(dev)
    o = torch.empty(T, H, D, dtype=torch.bfloat16, device=dev)
    qkv = torch.empty(T, C, dtype=torch.bfloat16, device=dev)
    qv, kv, vv = (qkv[:, i * H * D:(i + 1) * H * D].view(T, H, D) for i in range(3))
    nws = K.kda_prefill_workspace_bytes(qv, kv, vv, g, b, o, cu, pool, src, dst, chunk=64,
                                        segment_len=VARLEN_SEGMENT)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)

    def whole():
        K.kda_prefill_varlen_conv(x_d, cw_d, cpool, csrc, cdst, g, b, o, cu, pool, src, dst, qkv=qkv, act=1,
                                  qk_l2norm=True, chunk=64, workspace=ws, segment_len=VARLEN_SEGMENT)

    def prefill_only():
        K.kda_prefill_varlen(qv, kv, vv, g, b, o, cu, pool, src, dst, chunk=64, workspace=ws,
                             segment_len=VARLEN_SEGMENT)

    # the call's first launch alone: the same conv kernel through kda_conv_short
    # with the same normalisation, writing the same operands
    conv_only = K.prepare_conv_short(x_d, cw_d, cu, cpool, csrc, cdst, y=qkv, act=1, norm_d=D,
                                     norm_channels=2 * H * D)

    def timed(fn):
        for _ in range(warm):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(iters):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / iters

    ms = timed(whole)
    ms_pf = timed(prefill_only)
    conv_us = timed(conv_only) * 1e3
    alg_conv = 2 * T * C * 2 + 2 * N * C * (W - 1) * 2 + C * W * 2
    conv_gbs = alg_conv / conv_us / 1e3
    tps = T / (ms * 1e-3)
    res = {"workload": f"prefill from raw projections: the varlen workload's {T} tokens x {C} q/k/v channels, "
                       "conv W=4 + SiLU + q/k L2 norm + chunked prefill (chunk 64), bf16",
           "tokens": T, "ms": round(ms, 4), "tokens_per_s": round(tps, 1),
           "prefill_launch_ms": round(ms_pf, 4), "conv_launch_us": round(conv_us, 1),
           "roofline": prefill_roofline("prefill_kernel<128,bf16,bf16> on the formed operands (the call's "
                                        "dominant launch)", T, ms_pf, "prefill_varlen", "prefill_kernel_d128_bf16"),
           "conv_roofline": {"kernel": "conv_kernel<bf16,4,norm> (the call's conv + q/k norm launch)",
                             "bound": "hbm", "achieved": round(conv_gbs, 1), "peak": HBM_PEAK_GBS,
                             "unit": "GB/s", "frac": round(conv_gbs / HBM_PEAK_GBS, 4),
                             "traffic": traffic_for("conv_norm_kernel_prefill_bf16", "kda_conv.hip", T),
                             "alg_bytes_per_launch": alg_conv, "avg_launch_us": round(conv_us, 3)}}
    if cpu_seconds > 0:
        res["cpu_baseline"] = cpu_prefill_conv(cpu_seconds, wl, x, cw, cst)
    return res


def bench_prefill_long(torch, K, make_workload, dev, iters=3, cpu_segments=0, warm=3):
    """B=1, T=1,048,576, H=16, d=128, chunk 64, checkpoints every 32,768 (31
    interior + final), run as 32 segments by the segment scan.  Inputs are
    drawn on the GPU (17 GB bf16).  With cpu_segments > 0 the oracle is timed
    resuming from the GPU's checkpoints on that many segments spread over the
    sequence (plus a continuous run over the first 65,536 tokens)."""
    wl = make_workload(3, device=dev)
    T, H, D, I = wl.q.shape[0], 16, 128, wl.ckpt_interval
    cu = wl.cu_seqlens.to(dev)
    ck_cu, _ = K.kda_ckpt_plan(wl.cu_seqlens.cpu().numpy(), I, 64)
    n_ck = ck_cu[-1]
    pool = torch.zeros(1 + n_ck, H, D, D, device=dev)
    src = torch.tensor([-1], dtype=torch.int32, device=dev)
    dst = torch.tensor([0], dtype=torch.int32, device=dev)
    ck_cu_d = torch.tensor(ck_cu, dtype=torch.int32, device=dev)
    ck_slot = torch.arange(1, 1 + n_ck, dtype=torch.int32, device=dev)
    o = torch.empty(T, H, D, dtype=torch.bfloat16, device=dev)
    kw = dict(chunk=64, ckpt_interval=I, ckpt_cu=ck_cu_d, ckpt_slot=ck_slot)
    nws = K.kda_prefill_workspace_bytes(wl.q, wl.k, wl.v, wl.g, wl.beta, o, cu, pool, src, dst, **kw)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)

    def run():
        K.kda_prefill_varlen(wl.q, wl.k, wl.v, wl.g, wl.beta, o, cu, pool, src, dst, workspace=ws, **kw)

    for _ in range(warm):
        run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / iters
    tps = T / (ms * 1e-3)
    res = {"workload": "long prefill: B=1, T=1048576, H=16, d=128, chunk 64, ckpt every 32768, "
                       "32 segments", "tokens": T, "ms": round(ms, 3), "tokens_per_s": round(tps, 1),
           "alg_mfma_frac": round(tps * PREFILL_FLOPS_PER_TOKEN / (MFMA_BF16_PEAK_TFLOPS * 1e12), 4),
           "alg_hbm_frac": round(tps * PREFILL_BYTES_PER_TOKEN / (HBM_PEAK_GBS * 1e9), 4),
           "workspace_bytes": nws,
           "roofline": prefill_roofline("prefill_kernel<128,bf16,bf16> (kda_prefill_varlen call, segment scan: "
                                        "zero-started segments + transitions, combine, fix-up)", T, ms,
                                        "prefill_long_1m", "prefill_long_kernel_d128_bf16")}
    if cpu_segments > 0:
        states = torch.cat([torch.zeros(1, H, D, D, device=dev), pool[1:]]).cpu()   # state entering segment j
        res["cpu_baseline"] = cpu_long(wl, states, I, cpu_segments)
    del wl, o, ws, pool
    torch.cuda.empty_cache()
    return res


def bench_prefill(args, torch, K, make_workload):
    dev = torch.device("cuda:0")
    wl = make_workload(2)
    pf = bench_prefill_varlen(torch, K, make_workload, dev, iters=args.steps, wl=wl,
                              cpu_seconds=0 if args.no_cpu else args.cpu_seconds)
    cfg = {"workload": pf["workload"], "tokens": pf["tokens"], "H": 16, "d": 128, "chunk": 64,
           "initial_states": "even-indexed sequences", "segment_len": VARLEN_SEGMENT}
    secondary = {}
    if not args.no_secondary:
        secondary["prefill_long_1m"] = bench_prefill_long(torch, K, make_workload, torch.device("cuda:0"))
    return {"metric": METRIC, "value": pf["tokens_per_s"], "unit": "tokens/s", "ms_per_step": pf["ms"],
            "dtype": "bf16-mfma/f32-acc", "config": cfg, "roofline": pf["roofline"],
            "cpu_baseline": pf.get("cpu_baseline"), "secondary": secondary}


def bench_long(args, torch, K, make_workload):
    dev = torch.device("cuda:0")
    pf = bench_prefill_long(torch, K, make_workload, dev, iters=max(1, min(args.steps, 10)),
                            cpu_segments=0 if args.no_cpu else args.long_cpu_segments)
    cfg = {"workload": pf["workload"], "tokens": pf["tokens"], "H": 16, "d": 128, "chunk": 64,
           "ckpt_interval": 32768, "segments": 32}
    return {"metric": METRIC, "value": pf["tokens_per_s"], "unit": "tokens/s", "ms_per_step": pf["ms"],
            "dtype": "bf16-mfma/f32-acc", "config": cfg, "roofline": pf["roofline"],
            "cpu_baseline": pf.get("cpu_baseline"), "secondary": {}}


def cpu_long(wl, states, I, n_seg):
    """The oracle on the 1M-token workload, resumed from the GPU's checkpoints:
    n_seg of the 32 segments (32,768 tokens, all 16 heads each), spread over
    the sequence, in one packed call; then, separately, one continuous run
    over the first 65,536 tokens.  tokens/s of the resumed segments."""
    import numpy as np
    import torch
    import oracle
    orc = oracle.load("f64")
    threads = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    orc.set_threads(threads)
    nseg_all = wl.q.shape[0] // I
    pick = sorted({int(round(j * (nseg_all - 1) / max(n_seg - 1, 1))) for j in range(n_seg)})
    dt = 0.0
    G = 4   # segments per oracle call (one packed batch), which bounds the host memory
    for i0 in range(0, len(pick), G):
        grp = pick[i0:i0 + G]
        parts = [[t[j * I:(j + 1) * I].float().cpu() for j in grp] for t in (wl.q, wl.k, wl.v, wl.g, wl.beta)]
        q, k, v, g, b = (torch.cat(x).numpy() for x in parts)
        init = states[grp].double().numpy()
        cu = torch.arange(0, len(grp) * I + 1, I, dtype=torch.int32)
        t0 = time.perf_counter()
        orc.kda_varlen(q, k, v, g, b, cu, init=init, has_init=np.ones(len(grp), np.int32),
                       start_pos=np.array([j * I for j in grp], np.int32))
        dt += time.perf_counter() - t0
        del q, k, v, g, b, parts
    T2 = 2 * I
    q, k, v, g, b = (t[:T2].float().cpu().numpy() for t in (wl.q, wl.k, wl.v, wl.g, wl.beta))
    t1 = time.perf_counter()
    orc.kda_varlen(q, k, v, g, b, torch.tensor([0, T2], dtype=torch.int32))
    dt2 = time.perf_counter() - t1
    return {"value": round(len(pick) * I / dt, 1), "unit": "tokens/s", "cores": orc.threads(),
            "kind": "oracle", "cpu": cpu_info(),
            "sample": (f"all {nseg_all} segments" if len(pick) == nseg_all else
                       f"{len(pick)} of {nseg_all} segments ({pick})") +
                      f", 32768 tokens x 16 heads each, resumed from the GPU's checkpoints (4 segments per "
                      f"oracle call), fp64 oracle, {dt:.1f} s",
            "continuous_65536": {"value": round(T2 / dt2, 1), "unit": "tokens/s",
                                 "sample": f"tokens 0..65535 from the zero state, 16 heads, {dt2:.1f} s"}}


def cpu_prefill(cpu_seconds, wl):
    """Oracle on whole (sequence, head) pairs of the same workload until the
    time budget is spent; tokens/s scaled to all 16 heads."""
    import numpy as np
    import oracle
    orc = oracle.load("f64")
    threads = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    orc.set_threads(threads)
    N = wl.n_seq
    init = np.zeros((N, 16, 128, 128))
    has = np.zeros(N, np.int32)
    for s_, i in enumerate(wl.init_index):
        if i >= 0:
            init[s_] = wl.init_states[i].double().numpy()
            has[s_] = 1
    q, k, v, g, b = (t.float().numpy() for t in (wl.q, wl.k, wl.v, wl.g, wl.beta))
    lens = (wl.cu_seqlens[1:] - wl.cu_seqlens[:-1]).tolist()
    order = sorted(range(N), key=lambda s_: lens[s_])   # shortest sequences first
    tok_heads = 0
    t0 = time.perf_counter()
    done = []
    for s_ in order:
        pairs = [(s_, h) for h in range(16)]
        orc.kda_varlen(q, k, v, g, b, wl.cu_seqlens, init=init, has_init=has, pairs=pairs)
        tok_heads += lens[s_] * 16
        done.append(s_)
        if time.perf_counter() - t0 > cpu_seconds:
            break
    dt = time.perf_counter() - t0
    return {"value": round(tok_heads / 16 / dt, 1), "unit": "tokens/s", "cores": orc.threads(),
            "kind": "oracle", "cpu": cpu_info(),
            "sample": f"{len(done)} of 16 sequences (all 16 heads each, {tok_heads // 16} tokens), "
                      f"fp64 oracle, {dt:.1f} s"}


def cpu_prefill_conv(cpu_seconds, wl, x, cw, cst):
    """The oracle's prefill from raw projections on whole sequences (all 16
    heads), shortest first, until the time budget is spent."""
    import numpy as np
    import oracle
    orc = oracle.load("f64")
    threads = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    orc.set_threads(threads)
    N = wl.n_seq
    cu = wl.cu_seqlens.numpy()
    lens = np.diff(cu)
    done, toks = 0, 0
    t0 = time.perf_counter()
    for s_ in sorted(range(N), key=lambda i: lens[i]):
        i = wl.init_index[s_]
        init = wl.init_states[i].double().numpy()[None] if i >= 0 else None
        rows = slice(int(cu[s_]), int(cu[s_ + 1]))
        orc.kda_prefill_conv(x[rows], cw, wl.g[rows], wl.beta[rows], np.array([0, lens[s_]], np.int32), H=16,
                             d=128, act=1, conv_state=cst[s_:s_ + 1], qk_l2norm=1, init=init)
        done += 1
        toks += int(lens[s_])
        if time.perf_counter() - t0 > cpu_seconds:
            break
    dt = time.perf_counter() - t0
    return {"value": round(toks / dt, 1), "unit": "tokens/s", "cores": orc.threads(), "kind": "oracle",
            "cpu": cpu_info(),
            "sample": f"{done} of 16 sequences ({toks} tokens, all 16 heads: conv + norm + recurrence), "
                      f"fp64 oracle, {dt:.1f} s"}


def cpu_verify(wl, state_bytes, cpu_seconds):
    """The oracle on the whole verify workload (128 sequences x 8 tokens x 16
    heads, fused commit), repeated until the time budget is spent; state GB/s
    with the GPU's byte count."""
    import oracle
    orc = oracle.load("f64")
    threads = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    orc.set_threads(threads)
    q, k, v, g, b = (t.float().numpy() for t in (wl.q, wl.k, wl.v, wl.g, wl.beta))
    init = wl.init_states.double().numpy()
    L = wl.accepted_len.numpy()
    reps = 0
    t0 = time.perf_counter()
    while True:
        orc.kda_verify(q, k, v, g, b, init, L)
        reps += 1
        if time.perf_counter() - t0 > cpu_seconds:
            break
    dt = time.perf_counter() - t0
    return {"value": round(state_bytes * reps / dt / 1e9, 3), "unit": "GB/s", "cores": orc.threads(),
            "kind": "oracle", "cpu": cpu_info(),
            "sample": f"{reps} whole verify calls (128 seqs x 8 tokens x 16 heads, commit at L), fp64 oracle, "
                      f"{dt:.1f} s"}


def cpu_decode(args, wl, state_bytes, z, gw):
    import numpy as np
    import oracle
    orc = oracle.load("f64")
    threads = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    orc.set_threads(threads)
    init = wl.init_states.double().numpy()
    has = np.ones(wl.n_seq, np.int32)
    g, b = (t.float().numpy() for t in (wl.g, wl.beta))
    cx, cw, cs = wl.conv_x.float().numpy(), wl.conv_w.float().numpy(), wl.conv_state.float().numpy()
    del has
    reps = 0
    t0 = time.perf_counter()
    while True:
        orc.kda_decode_conv(cx, cw, g, b, init, cs, H=wl.H, d=wl.dk, act=1, qk_l2norm=1, out_gate=z,
                            norm_weight=gw)
        reps += 1
        if time.perf_counter() - t0 > args.cpu_seconds:
            break
    dt = time.perf_counter() - t0
    return {"value": round(state_bytes * reps / dt / 1e9, 3), "unit": "GB/s", "cores": orc.threads(),
            "kind": "oracle", "cpu": cpu_info(),
            "sample": f"{reps} whole fused decode steps (conv + SiLU + q/k norm + 128 seqs x 16 heads "
                      f"x 1 token + gated output norm, fp64 oracle), "
                      f"{dt:.1f} s"}


def main():
    args = parse()
    if args.ingest_pmc:
        data = ingest_pmc(*args.ingest_pmc)
        TRAFFIC_FILE.write_text(json.dumps(data, indent=1) + "\n")
        print(json.dumps(data))
        return
    if args.ingest_mfma:
        data = ingest_mfma(args.ingest_mfma)
        MFMA_FILE.write_text(json.dumps(data, indent=1) + "\n")
        print(json.dumps(data))
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    from hybrid_recurrent_serving_amd import kda as K
    from hybrid_recurrent_serving_amd.inputs import make_workload
    K.load_library()
    if args.pmc_pass:
        pmc_pass(torch, K, make_workload, long=args.pmc_long)
        print(json.dumps({"pmc_pass": "done"}))
        return
    if args.workload == "decode":
        res = bench_decode(args, torch, K, make_workload)
    elif args.workload == "long":
        res = bench_long(args, torch, K, make_workload)
    else:
        res = bench_prefill(args, torch, K, make_workload)
    line = {"metric": res["metric"], "value": res["value"], "unit": res["unit"], "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(res["ms_per_step"], 6),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": res["dtype"], "data": "synthetic (seeded; no datasets or weights)",
            "config": res["config"], "roofline": res["roofline"],
            "cpu_baseline": res["cpu_baseline"], "secondary": res["secondary"]}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
