"""Summarise rocprofv3 counter runs of the benchmark for bench.py.

    rocprofv3 --pmc <counters> --output-format csv -d <dir> -o run -- python3 bench.py ...
    python -m block_scaled_bit_amd.counters mfma <dir> [<dir> ...] --out profiles/mfma_counters.json
    python -m block_scaled_bit_amd.counters traffic --fetch <dir> --write <dir> --out profiles/traffic.json

For every kernel and launch grid seen in the runs (key "name<args> [grid N]") it
records the mean of each counter per dispatch and, where the counters are present:
  * mfma_ops_i8: INT8 matrix ops, SQ_INSTS_VALU_MFMA_MOPS_I8 x 512 (the counter
    counts in units of 512 ops); mfma_ops_f16 / _bf16 / _f8 likewise: zero for a
    kernel that really runs INT8 (the check of [P3] sec. 4.1 / sec. 6 that INT8 was
    not replaced by a 16-bit path);
  * sclk_mhz: GRBM_GUI_ACTIVE (summed over the XCDs) / XCDs / kernel duration
    (kernels of at least 100 us only: the counter window is wider than the kernel);
  * mfma_util: SQ_VALU_MFMA_BUSY_CYCLES (summed over SIMDs) / (SIMDs x the kernel's
    cycles at that clock): the share of the kernel's time the matrix cores were busy.
The traffic mode turns a FETCH_SIZE run and a WRITE_SIZE run into HBM bytes per
launch of the benchmark's main kernels, each counter scaled by what it reads for the
benchmark's own 512 MiB device-to-device copy (the largest copy in the run).
Each file carries the digest of the kernel sources it was taken on; bench.py uses it
only while the digest matches.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys

XCDS = 8
SIMDS = 256 * 4
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_scaled_bit_amd", "csrc")


def sources_digest() -> str:
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def short_name(kernel: str) -> str:
    """'void bsb::(anonymous namespace)::gemm_big_kernel<0, false, false>(signed char...)' ->
    'gemm_big_kernel<0, false, false>'."""
    k = kernel.strip()
    if k.startswith("void "):
        k = k[5:]
    depth, cut = 0, len(k)
    for i, ch in enumerate(k):          # the argument list starts at the first '(' outside <>
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0 and not k[i:].startswith("(anonymous"):
            cut = i
            break
    k = k[:cut]
    return re.sub(r"^.*::", "", k.replace("(anonymous namespace)::", ""))


def summarise(dirs):
    per = {}
    for d in dirs:
        for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(path) as f:
                for r in csv.DictReader(f):
                    k = f"{short_name(r['Kernel_Name'])} [grid {r['Grid_Size']}]"
                    e = per.setdefault(k, {"counters": {}, "dur": {}})
                    e["counters"].setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
                    key = (path, r["Dispatch_Id"])
                    e["dur"][key] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    out = {}
    for k, e in per.items():
        c = {n: sum(v) / len(v) for n, v in e["counters"].items()}
        dur = sum(e["dur"].values()) / len(e["dur"])
        ent = {"dispatches": len(e["dur"]), "duration_ns": round(dur, 1),
               "counters": {n: round(v, 1) for n, v in sorted(c.items())}}
        for name, key in (("mfma_ops_i8", "SQ_INSTS_VALU_MFMA_MOPS_I8"),
                          ("mfma_ops_f16", "SQ_INSTS_VALU_MFMA_MOPS_F16"),
                          ("mfma_ops_bf16", "SQ_INSTS_VALU_MFMA_MOPS_BF16"),
                          ("mfma_ops_f8", "SQ_INSTS_VALU_MFMA_MOPS_F8")):
            if key in c:
                ent[name] = int(round(c[key] * 512))
        # the counter window of a dispatch is wider than the kernel: the clock and
        # utilisation derived from it are stated only for kernels of >= 100 us
        if "GRBM_GUI_ACTIVE" in c and dur >= 100e3:
            cycles = c["GRBM_GUI_ACTIVE"] / XCDS
            ent["sclk_mhz"] = round(cycles / (dur * 1e-9) / 1e6)
            if "SQ_VALU_MFMA_BUSY_CYCLES" in c:
                ent["mfma_util"] = round(c["SQ_VALU_MFMA_BUSY_CYCLES"] / (SIMDS * cycles), 4)
        out[k] = ent
    return out


# bench.py's keys: (kernel, launch grid in threads, algorithmic bytes per launch)
TRAFFIC_KEYS = {
    "gemm_decode_packed": ("gemm_packed_kernel<2, 7, 0, true, false>", 114688, 244318336),
    "gemm_decode": ("gemm_smallm_kernel<2, 7, 0, 2, 4, false, true, 0>", 114688, 244318336),
    "quant_decode": ("quantize_act_kernel<4>", 8192, 786560),
    "gemm_prefill": ("gemm_big_kernel<0, false, false>", 262144, 169885696),
    "moe_grouped": ("gemm_big_kernel<0, true, false>", 786432, 787611908),
    # the same GEMM gathering its rows: the 4096 tokens and the row index instead of the rows
    "moe_grouped_gather": ("gemm_big_kernel<0, true, true>", 786432, 670187780),
    "kv_attention": ("attn_split_kernel<0, 8, 1>", 131072, 277872640),
    "kv_attention_bf16": ("attn_split_kernel<1, 8, 1>", 131072, 537919488),
    "gemm_mid_m1024": ("gemm_mid_kernel<0, false, false>", 131072, 46010368),
    "w8a16_prefill": ("gemm_a16_kernel<0, 1>", 1048576, 203423744),
    "bf16_prefill": ("gemm_a16_kernel<0, 2>", 1048576, 268435456),
    "decode_fp8": ("decode_fp8_block_kernel<false>", 917504, 59639552),
    "decode_fp8_layer": ("decode_fp8_block_kernel<false>", 3670016, 238558208),
    "decode_mxfp4": ("decode_mxfp4_kernel<false>", 1048576, 104857600),
}
CAL_BYTES = 512 << 20


def _per_dispatch(d, counter):
    """{(kernel, grid): [values]} of one counter over a run."""
    out = {}
    for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == counter:
                    key = (short_name(r["Kernel_Name"]), int(r["Grid_Size"]))
                    out.setdefault(key, []).append(float(r["Counter_Value"]))
    return out


def traffic(fetch_dir, write_dir):
    fe, wr = _per_dispatch(fetch_dir, "FETCH_SIZE"), _per_dispatch(write_dir, "WRITE_SIZE")
    copy_f = max(v for (k, _), vs in fe.items() if k == "__amd_rocclr_copyBuffer" for v in vs)
    copy_w = max(v for (k, _), vs in wr.items() if k == "__amd_rocclr_copyBuffer" for v in vs)
    ff, wf = CAL_BYTES / (copy_f * 1024), CAL_BYTES / (copy_w * 1024)
    res = {"sources": sources_digest(),
           "calibration": {"copy_bytes": CAL_BYTES, "fetch_kib": copy_f, "write_kib": copy_w,
                           "fetch_factor": round(ff, 4), "write_factor": round(wf, 4)},
           "kernels": {}}
    for key, (name, grid, alg) in TRAFFIC_KEYS.items():
        f, w = fe.get((name, grid)), wr.get((name, grid))
        if not f or not w:
            continue
        fk, wk = sum(f) / len(f), sum(w) / len(w)
        res["kernels"][key] = {"kernel": name, "grid": grid, "algorithmic_bytes": alg,
                               "fetch_kib": round(fk, 1), "write_kib": round(wk, 1),
                               "bytes_per_launch": int(round(fk * 1024 * ff + wk * 1024 * wf)),
                               "dispatches": min(len(f), len(w))}
    return res


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    sub = ap.add_subparsers(dest="mode", required=True)
    m = sub.add_parser("mfma", help="per-kernel counter means, INT8 ops, clock, MFMA utilisation")
    m.add_argument("dirs", nargs="+", help="rocprofv3 output directories (csv)")
    m.add_argument("--out", required=True)
    m.add_argument("--command", default="", help="the command that produced the runs")
    t = sub.add_parser("traffic", help="HBM bytes per launch from FETCH_SIZE / WRITE_SIZE runs")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--out", required=True)
    a = ap.parse_args(argv)
    if a.mode == "traffic":
        res = traffic(a.fetch, a.write)
    else:
        res = {"sources": sources_digest(), "command": a.command, "kernels": summarise(a.dirs)}
    with open(a.out, "w") as f:
        json.dump(res, f, indent=1, sort_keys=True)
        f.write("\n")
    print(f"wrote {a.out}: {len(res['kernels'])} kernels", file=sys.stderr)


if __name__ == "__main__":
    main()
