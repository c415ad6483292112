"""Host-side logic of bench.py (no GPU): the single-GPU guard and the HBM-traffic
arithmetic that turns rocprofv3 counter CSVs into bytes per launch."""
import csv
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "--gpus 1" in r.stderr


def _write_pmc(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                           "Counter_Value"])
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                 "Counter_Value"], r)))


NEG = "void at::native::elementwise_kernel<128, 4, neg>(int, F)"
DKDV = "void psa::(anonymous namespace)::dkdv_kernel<psa::bf16_t, float, 128, 0, 0, false>(BwdParams)"
FWD = "void psa::(anonymous namespace)::fwd_kernel<psa::bf16_t, 128, false>(FwdParams)"
FWD32 = "void psa::(anonymous namespace)::fwd_kernel<float, 64, false>(FwdParams)"
FWD8 = "void psa::(anonymous namespace)::fwd_kernel<psa::fp8_t, 128, false>(FwdParams)"


def test_traffic_scaling_by_the_reference_copy(tmp_path):
    """FETCH_SIZE reads half of the negation's 64 MiB (factor 2), WRITE_SIZE all of it
    (factor 1); per-channel rows of one dispatch add up, dispatches of one kernel
    average, fp32 variants are not attention traffic of the bf16 path."""
    mib = 64
    kib = mib * 1024.0
    _write_pmc(str(tmp_path / "FETCH_SIZE" / "a" / "run_counter_collection.csv"), [
        (1, NEG, "FETCH_SIZE", kib / 4), (1, NEG, "FETCH_SIZE", kib / 4),  # two channels
        (2, DKDV, "FETCH_SIZE", 1000.0), (3, DKDV, "FETCH_SIZE", 3000.0),
        (4, FWD, "FETCH_SIZE", 500.0), (5, FWD32, "FETCH_SIZE", 9.0),
    ])
    _write_pmc(str(tmp_path / "WRITE_SIZE" / "a" / "run_counter_collection.csv"), [
        (1, NEG, "WRITE_SIZE", kib),
        (2, DKDV, "WRITE_SIZE", 100.0), (3, DKDV, "WRITE_SIZE", 300.0),
        (4, FWD, "WRITE_SIZE", 50.0),
    ])
    out = bench.traffic_from_pmc(str(tmp_path), mib)
    assert set(out) == {"bwd_dkdv", "fwd"}
    d = out["bwd_dkdv"]
    assert d["kernel"] == "dkdv_kernel<bf16_t, float, 128, 0, 0, false>"
    assert d["FETCH_SIZE_scale"] == pytest.approx(2.0)
    assert d["WRITE_SIZE_scale"] == pytest.approx(1.0)
    assert d["FETCH_SIZE_KiB"] == pytest.approx(2000.0)
    assert d["bytes_per_launch"] == int((2000.0 * 2 + 200.0) * 1024)
    assert out["fwd"]["bytes_per_launch"] == int((500.0 * 2 + 50.0) * 1024)


def test_traffic_of_the_e4m3_forward(tmp_path):
    """With dtype_tag fp8 only the e4m3 kernels count."""
    kib = 64 * 1024.0
    _write_pmc(str(tmp_path / "F" / "run_counter_collection.csv"), [
        (1, NEG, "FETCH_SIZE", kib / 2), (2, FWD8, "FETCH_SIZE", 300.0),
        (3, FWD, "FETCH_SIZE", 500.0), (1, NEG, "WRITE_SIZE", kib),
        (2, FWD8, "WRITE_SIZE", 40.0), (3, FWD, "WRITE_SIZE", 50.0)])
    out = bench.traffic_from_pmc(str(tmp_path), 64, "fp8")
    assert set(out) == {"fwd"}
    assert out["fwd"]["kernel"] == "fwd_kernel<fp8_t, 128, false>"
    assert out["fwd"]["bytes_per_launch"] == int((300.0 * 2 + 40.0) * 1024)


def test_traffic_needs_the_reference_copy(tmp_path):
    _write_pmc(str(tmp_path / "x" / "run_counter_collection.csv"),
               [(1, DKDV, "FETCH_SIZE", 1.0), (1, DKDV, "WRITE_SIZE", 1.0)])
    with pytest.raises(SystemExit, match="reference negation"):
        bench.traffic_from_pmc(str(tmp_path), 64)


DKDV1 = "void psa::(anonymous namespace)::dkdv_kernel<psa::bf16_t, float, 256, 0, 1, false, 1>(BwdParams)"
DKDV2 = "void psa::(anonymous namespace)::dkdv_kernel<psa::bf16_t, float, 256, 0, 2, false, 1>(BwdParams)"


def test_traffic_sums_the_launches_of_a_stage(tmp_path):
    """At d = 256 dK/dV is two launches (dV pass, dK pass): the stage's bytes are the sum."""
    kib = 64 * 1024.0
    _write_pmc(str(tmp_path / "F" / "run_counter_collection.csv"), [
        (1, NEG, "FETCH_SIZE", kib / 2), (2, DKDV1, "FETCH_SIZE", 100.0),
        (3, DKDV2, "FETCH_SIZE", 300.0), (1, NEG, "WRITE_SIZE", kib),
        (2, DKDV1, "WRITE_SIZE", 10.0), (3, DKDV2, "WRITE_SIZE", 30.0)])
    out = bench.traffic_from_pmc(str(tmp_path), 64)
    assert out["bwd_dkdv"]["bytes_per_launch"] == int((400.0 * 2 + 40.0) * 1024)
    assert out["bwd_dkdv"]["kernel"].count("dkdv_kernel") == 2


def test_mfma_busy_arithmetic(tmp_path):
    """MFMA busy = MFMA busy cycles over (GRBM_GUI_ACTIVE / 8 XCDs) x 256 CUs x 4 SIMDs,
    cycles summed over a stage's kernels and averaged over dispatches."""
    act = 8 * 1000.0  # 1000 busy clocks per XCD
    _write_pmc(str(tmp_path / "B" / "run_counter_collection.csv"), [
        (1, DKDV, "GRBM_GUI_ACTIVE", act), (1, DKDV, "SQ_VALU_MFMA_BUSY_CYCLES", 0.25 * 1000 * 1024),
        (1, DKDV, "SQ_BUSY_CU_CYCLES", 0.5 * 1000 * 256), (1, DKDV, "GRBM_COUNT", 8 * 2000.0),
        (2, DKDV, "GRBM_GUI_ACTIVE", act), (2, DKDV, "SQ_VALU_MFMA_BUSY_CYCLES", 0.75 * 1000 * 1024),
        (2, DKDV, "SQ_BUSY_CU_CYCLES", 0.5 * 1000 * 256), (2, DKDV, "GRBM_COUNT", 8 * 2000.0),
        (3, FWD32, "GRBM_GUI_ACTIVE", act)])
    out = bench.busy_from_pmc(str(tmp_path))
    assert set(out) == {"bwd_dkdv"}
    assert out["bwd_dkdv"]["mfma_busy"] == pytest.approx(0.5)
    assert out["bwd_dkdv"]["cu_busy"] == pytest.approx(0.5)


def test_oracle_dense_work_and_bounded_sample():
    """The oracle's dense work is per group: sum of |group|^2 x hq x (4 or 12) d; the
    sample shrinks heads, then completions, to fit the budget, and its times scale to
    the workload by that work."""
    from shared_prefix_block_amd import workloads as wl
    cfg = wl.WORKLOADS[2]
    lay = wl.layout_for(cfg)
    assert bench.oracle_dense_flops(lay, 32, 128, False) == 8 * 2560 ** 2 * 32 * 4 * 128
    assert bench.oracle_dense_flops(lay, 32, 128, True) == 8 * 2560 ** 2 * 32 * 12 * 128
    c = bench.cpu_baseline(cfg, lay, budget_flop=1e9)
    assert "4 of 32 q heads (1 kv heads)" in c["sample"]
    assert "with 1 of its 8 completions" in c["sample"]
    scale = bench.oracle_dense_flops(lay, 32, 128, True) / (768 ** 2 * 4 * 12 * 128)
    assert c["est_fwd_bwd_s"] == pytest.approx(c["sample_fwd_bwd_s"] * scale, rel=1e-2, abs=0.02)
    assert c["tokens_per_s"] > 0 and c["blas_threads"] >= 1
