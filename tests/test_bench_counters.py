"""bench.py's counter arithmetic on synthetic rocprofv3 counter files (host logic, no GPU).

A counter file has one row per (dispatch, counter, hardware instance); the parser sums a
dispatch's rows.  Traffic per launch is FETCH_SIZE and WRITE_SIZE (KiB per dispatch, mean over a
kernel's dispatches) times bytes / counter of the run's largest device copy, summed over a leg's
kernels; busy fractions divide by 1024 SIMDs and the kernel's cycles (GRBM_GUI_ACTIVE summed
over 8 XCDs).
"""
import csv
import importlib.util
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


PRE = "void hifa4::(anonymous namespace)::attn_prefill_kernel<128, true, 0, false, 0, 8>(hifa4::AttnArgs)"
D256 = "void hifa4::(anonymous namespace)::attn_prefill_kernel<256, true, 0, false, 0, 8>(hifa4::AttnArgs)"
DP = "void hifa4::(anonymous namespace)::attn_prefill_kernel<128, true, 0, false, 2, 8>(hifa4::AttnArgs)"
SPLIT = "void hifa4::(anonymous namespace)::attn_decode_split_kernel<128, 0, 0, 2>(hifa4::AttnArgs)"
MERGE = "void hifa4::(anonymous namespace)::attn_decode_merge_kernel<128>(hifa4::AttnArgs)"
COPY = "__amd_rocclr_copyBuffer"


def write_csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for disp, name, counter, values in rows:
            for v in values:  # one row per hardware instance
                w.writerow({"Dispatch_Id": disp, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": v})


def test_parser_sums_instances_per_dispatch_in_order(bench, tmp_path):
    p = tmp_path / "c_counter_collection.csv"
    write_csv(p, [(2, PRE, "FETCH_SIZE", [10.0, 20.0]), (1, PRE, "FETCH_SIZE", [1.0, 2.0, 3.0]),
                  (3, COPY, "FETCH_SIZE", [5.0])])
    r = bench.parse_counter_csv(str(p))
    assert r[PRE]["FETCH_SIZE"] == [6.0, 30.0]  # dispatch 1, then 2
    assert r[COPY]["FETCH_SIZE"] == [5.0]


def test_derived_traffic_and_busy_fractions(bench, tmp_path):
    mib512_kib = 512 * 1024
    fetch = {PRE: {"FETCH_SIZE": [100.0, 300.0]}, D256: {"FETCH_SIZE": [50.0]}, DP: {"FETCH_SIZE": [70.0]},
             SPLIT: {"FETCH_SIZE": [1000.0]}, MERGE: {"FETCH_SIZE": [10.0]},
             COPY: {"FETCH_SIZE": [3.0, mib512_kib / 2.0]}}  # the counter reads half of the copied bytes
    write = {PRE: {"WRITE_SIZE": [400.0]}, D256: {"WRITE_SIZE": [40.0]}, DP: {"WRITE_SIZE": [400.0]},
             SPLIT: {"WRITE_SIZE": [20.0]}, MERGE: {"WRITE_SIZE": [4.0]}, COPY: {"WRITE_SIZE": [float(mib512_kib)]}}
    cyc = 1000.0
    busy = {PRE: {"GRBM_GUI_ACTIVE": [8 * cyc], "SQ_VALU_MFMA_BUSY_CYCLES": [0.25 * 1024 * cyc],
                  "SQ_ACTIVE_INST_VALU": [0.9 * 1024 * cyc / 4]}}
    out = bench.derive_counters([fetch, write, busy])
    assert out["_scale"]["fetch_factor"] == 2.0 and out["_scale"]["write_factor"] == 1.0
    assert out["prefill"]["fetch_bytes"] == 200 * 1024 * 2  # mean of 100 and 300 KiB, doubled
    assert out["prefill"]["traffic"] == 200 * 1024 * 2 + 400 * 1024
    assert out["decode"]["traffic"] == (1000 + 10) * 1024 * 2 + (20 + 4) * 1024  # split + merge
    assert out["prefill"]["mfma_busy"] == 0.25 and out["prefill"]["valu_busy"] == 0.9
    assert "mfma_busy" not in out["decode"]  # no busy counters for it in this run


def test_no_copy_probe_means_no_figures(bench):
    runs = [{PRE: {"FETCH_SIZE": [1.0]}}, {PRE: {"WRITE_SIZE": [1.0]}}, {}]
    assert bench.derive_counters(runs) is None


def test_add_counters_without_any_source_leaves_traffic_null(bench):
    line = {"roofline": {"traffic": None}, "decode": {"roofline": {"traffic": None}}}
    bench.add_counters(line, "none")
    assert line["roofline"]["traffic"] is None and line["counters"]["source"] is None
