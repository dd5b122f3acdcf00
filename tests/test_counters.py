"""The rocprofv3 counter summary the benchmark reads (no GPU needed): kernel names
are reduced to name<template args>, counters averaged per dispatch, INT8 ops taken
from the 512-op units of SQ_INSTS_VALU_MFMA_MOPS_I8, the clock from GRBM_GUI_ACTIVE
over the XCDs, utilisation from the MFMA busy cycles over all SIMDs."""
import csv
import os

from block_scaled_bit_amd import counters


def test_short_names():
    assert counters.short_name("void bsb::(anonymous namespace)::gemm_big_kernel<0, false>"
                               "(signed char const*, int)") == "gemm_big_kernel<0, false>"
    assert counters.short_name("void bsb::(anonymous namespace)::gemm_packed_kernel<2, 7, 0, true, "
                               "false>(signed char const*)") == "gemm_packed_kernel<2, 7, 0, true, false>"
    assert counters.short_name("__amd_rocclr_copyBuffer") == "__amd_rocclr_copyBuffer"


def test_summary_arithmetic(tmp_path):
    d = tmp_path / "run"
    d.mkdir()
    name = "void bsb::(anonymous namespace)::gemm_big_kernel<0, false>(signed char const*)"
    rows = []
    # two dispatches of 1 ms; 8 XCDs x 2e6 cycles = 2 GHz; MFMA busy half of 1024 SIMDs' cycles
    for disp in (1, 2):
        for cname, val in (("SQ_INSTS_VALU_MFMA_MOPS_I8", 2 ** 30), ("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0),
                           ("GRBM_GUI_ACTIVE", 8 * 2e6), ("SQ_VALU_MFMA_BUSY_CYCLES", 1024 * 1e6)):
            rows.append({"Dispatch_Id": disp, "Kernel_Name": name, "Grid_Size": 262144,
                         "Counter_Name": cname,
                         "Counter_Value": val, "Start_Timestamp": 0, "End_Timestamp": 1_000_000})
    with open(d / "run_counter_collection.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=list(rows[0]))
        w.writeheader()
        w.writerows(rows)
    s = counters.summarise([str(d)])["gemm_big_kernel<0, false> [grid 262144]"]
    assert s["dispatches"] == 2
    assert s["mfma_ops_i8"] == 2 ** 39 and s["mfma_ops_bf16"] == 0
    assert s["sclk_mhz"] == 2000
    assert s["mfma_util"] == 0.5
