"""Host logic of the benchmark's counter ingestion (no GPU): per-call grouping
of prefill dispatches by their segment-plan launch, the active-cycle
weighting of MfmaUtil / VALUBusy, the GEMM calibration and the copy
calibration of FETCH_SIZE / WRITE_SIZE, on synthetic rocprofv3 CSV rows."""
import csv

import pytest

import bench

PLAN = "kda::pf::segment_plan_kernel(kda::PrefillParams, int*, int*)"
PF = "void kda::pf::prefill_kernel<128, unsigned short, unsigned short>(kda::PrefillParams, int, int)"
COMB = "kda::pf::segment_combine_kernel(kda::PrefillParams, int)"
VER = "void kda::vf::verify_kernel<unsigned short>(kda::StepParams)"
COPY = "__amd_rocclr_copyBuffer"


@pytest.fixture
def tokens(monkeypatch):
    monkeypatch.setattr(bench, "varlen_tokens", lambda: 1000)
    return 1000


def _write(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name",
                                          "Counter_Value"])
        w.writeheader()
        w.writerows(rows)


def _grid(call):
    """pass-A grid of a prefill call of the counter pass: the varlen calls
    first, then the 1M-token calls (another grid)"""
    return 1000 if call < bench.PMC_PREFILL_CALLS else 500


def test_ingest_mfma_groups_and_weights(tmp_path, tokens):
    rows, did = [], [0]

    def add(name, util, valu, mops, grbm, grid=64):
        did[0] += 1
        for c, v in (("MfmaUtil", util), ("VALUBusy", valu), ("SQ_INSTS_VALU_MFMA_MOPS_BF16", mops),
                     ("GRBM_GUI_ACTIVE", grbm)):
            rows.append({"Dispatch_Id": did[0], "Kernel_Name": name, "Grid_Size": grid, "Counter_Name": c,
                         "Counter_Value": v})

    add(COPY, 0, 1, 0, 100)
    add("Cijk_gemm", 70, 20, 2 * bench.GEMM_N ** 3 / 512, 1000)
    add(VER, 0, 60, 0, 300)
    add(VER, 0, 40, 0, 100)
    for call in range(bench.PMC_PREFILL_CALLS + bench.PMC_LONG_CALLS):
        add(PLAN, 0, 5, 0, 10)
        add(PF, 20, 40, 1000 * (call + 1), 300, _grid(call))   # pass A
        add(COMB, 0, 2, 0, 10)
        add(PF, 10, 30, 100, 100, _grid(call) // 2)            # fix-up
    path = tmp_path / "mfma.csv"
    _write(path, rows)
    out = bench.ingest_mfma([str(path)])
    assert out["calibration_gemm"]["executed_flops"] == 2 * bench.GEMM_N ** 3
    v = out["verify_kernel_d128_bf16"]
    assert v["dispatches"] == 2 and v["valu_busy"] == pytest.approx((60 * 300 + 40 * 100) / 400 / 100)
    pv = out["prefill_varlen"]
    last = bench.PMC_PREFILL_CALLS   # the measured varlen call is the last of its group
    assert pv["tokens"] == tokens and pv["dispatches"] == 3
    assert pv["executed_bf16_flops"] == (1000 * last + 100) * 512
    assert pv["mfma_util"] == pytest.approx((20 * 300 + 0 * 10 + 10 * 100) / 410 / 100, abs=1e-4)
    assert [d["role"] for d in pv["per_dispatch"]] == ["pass A", "combine", "fix-up"]
    pl = out["prefill_long_1m"]
    assert pl["executed_bf16_flops"] == (1000 * (last + bench.PMC_LONG_CALLS) + 100) * 512


def test_ingest_pmc_calibrates_and_splits_calls(tmp_path, tokens):
    def rows_for(counter, copy_val, pf_val):
        rows, did = [], 0
        for name, val, grid in [(COPY, copy_val, 1)] + [
                (x, y, z) for c in range(bench.PMC_PREFILL_CALLS + bench.PMC_LONG_CALLS)
                for x, y, z in ((PLAN, 1.0, 1), (PF, pf_val, _grid(c)), (COMB, 1.0, 1), (PF, pf_val, _grid(c)))]:
            did += 1
            rows.append({"Dispatch_Id": did, "Kernel_Name": name, "Grid_Size": grid, "Counter_Name": counter,
                         "Counter_Value": val})
        return rows

    kib = bench.COPY_BYTES / 1024
    fp, wp = tmp_path / "f.csv", tmp_path / "w.csv"
    _write(fp, rows_for("FETCH_SIZE", kib / 2, 10.0))   # fetch reads half the copy: scale 2
    _write(wp, rows_for("WRITE_SIZE", kib, 4.0))
    out = bench.ingest_pmc(str(fp), str(wp))
    assert out["calibration"]["fetch_scale"] == pytest.approx(2.0)
    assert out["calibration"]["write_scale"] == pytest.approx(1.0)
    for key, units in (("prefill_kernel_d128_bf16", tokens), ("prefill_long_kernel_d128_bf16", 1 << 20)):
        e = out[key]
        assert e["units_per_launch"] == units
        assert e["fetch_bytes"] == round(2 * 10.0 * 1024 * 2)   # two dispatches per call, scaled x 2
        assert e["write_bytes"] == round(2 * 4.0 * 1024)


def test_ingest_pmc_single_kernels(tmp_path, tokens):
    """The verify, fused verify and prefill-scale conv kernels: their
    dispatches averaged, each counter scaled by the calibration copy."""
    names = {"verify_kernel_d128_bf16": "void kda::vf::verify_kernel<unsigned short>(kda::StepParams)",
             "verify_conv_kernel_d128_bf16": "void kda::vf::verify_conv_kernel<unsigned short, 4, 8>(kda::DecodeConvParams)",
             "conv_kernel_prefill_bf16": "void kda::conv_kernel<unsigned short, 4, 0>(kda::ConvParams)",
             "conv_norm_kernel_prefill_bf16": "void kda::conv_kernel<unsigned short, 4, 16>(kda::ConvParams)"}

    def rows_for(counter, copy_val):
        rows, did = [], 0
        for name, val in [(COPY, copy_val)] + [(n, 8.0 + i) for i, n in enumerate(names.values()) for _ in range(2)]:
            did += 1
            rows.append({"Dispatch_Id": did, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": val})
        return rows

    kib = bench.COPY_BYTES / 1024
    fp, wp = tmp_path / "f.csv", tmp_path / "w.csv"
    _write(fp, rows_for("FETCH_SIZE", kib / 2))
    _write(wp, rows_for("WRITE_SIZE", kib))
    out = bench.ingest_pmc(str(fp), str(wp))
    for i, key in enumerate(names):
        e = out[key]
        assert e["dispatches"] == 2
        assert e["fetch_bytes"] == round((8.0 + i) * 1024 * 2)
        assert e["write_bytes"] == round((8.0 + i) * 1024)
    assert out["verify_kernel_d128_bf16"]["units_per_launch"] == 128 * 16
    assert out["conv_norm_kernel_prefill_bf16"]["units_per_launch"] == tokens


def test_decode_kernel_names():
    """The decode rows of the counter ingestion pick the bf16 d = 128 decode
    kernel by its template arguments: the plain step (W = 0) and the fused
    conv step (W = 4), not the fp32 instances or the other widths."""
    plain = "void kda::decode128_kernel<unsigned short, unsigned short, 0>(kda::Dec128Args)"
    fused = "void kda::decode128_kernel<unsigned short, unsigned short, 4>(kda::Dec128Args)"
    assert bench.is_decode128(plain, 0) and not bench.is_decode128(plain, 4)
    assert bench.is_decode128(fused, 4) and not bench.is_decode128(fused, 0)
    assert not bench.is_decode128("void kda::decode128_kernel<unsigned short, float, 4>(kda::Dec128Args)", 4)
    assert not bench.is_decode128("void kda::decode128_kernel<unsigned short, unsigned short, 3>(kda::Dec128Args)", 4)


def test_prefill_call_layout_checked():
    """A counter pass whose call counts drift from the ingestion's (more
    warm-up calls than PMC_PREFILL_CALLS / PMC_LONG_CALLS allow for) would put
    varlen calls where the 1M-token calls are expected: the pass-A grids
    expose it and the ingestion stops."""
    n, m = bench.PMC_PREFILL_CALLS, bench.PMC_LONG_CALLS
    bench.check_prefill_calls([1000] * n + [500] * m + [1000] * 3)   # as expected
    bench.check_prefill_calls([None] * (n + m))                       # no grid column: nothing to check
    with pytest.raises(SystemExit):
        bench.check_prefill_calls([1000] * (n + m + 4))               # long calls late
    with pytest.raises(SystemExit):
        bench.check_prefill_calls([1000] * (n - 1) + [500] * (m + 1))  # long calls early
