"""Benchmark of the block-scaled INT8 linear layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step = one pass of the hot path over one batch: dynamic per-token INT8
quantisation of the BF16 activations (bsb_quantize_act) followed by the W8A8
per-group-128 GEMM with BF16 output (bsb_gemm_w8a8_g128), on the
decode-shaped linear M=32 tokens, K=8192, N=28672 (seeded synthetic inputs:
activations N(0,1) with 0.5 % outliers x30, INT8 weights uniform in
[-127,127], lognormal group scales). All inputs are resident in HBM before
timing starts; the weights are rotated over several copies (> 1 GB of
traffic between reuses) so that the 256 MB last-level cache cannot serve them.

Reported (one JSON line on stdout):
  value          algorithmic HBM bytes of the step / step time, GB/s
  roofline       the GEMM kernel's algorithmic bytes per launch / its mean
                 duration (a timed region of back-to-back GEMM launches
                 between HIP events on the launch stream), against 8 TB/s;
                 `traffic`
                 = measured HBM bytes per launch from rocprofv3 counters
                 (profiles/traffic.json), null when the kernel sources have
                 changed since they were taken
  cpu_baseline   the CPU oracle on the same workload, timed on this host
  prefill        the prefill-shaped GEMM M=4096, K=8192, N=8192 timed the same
                 way, against the 5.0 POPS dense INT8 MFMA peak
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "W8A8-g128 GEMM TOPS & HBM GB/s (M=32 decode, M=4096 prefill), % roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
INT8_PEAK_TOPS = 5000.0        # MI355X dense INT8 MFMA, published
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
CSRC = os.path.join(ROOT, "block_scaled_bit_amd", "csrc")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def gemm_bytes(M, N, K):
    """Algorithmic bytes of one GEMM launch: q, sa, qw, sw read once, y (BF16) written once."""
    G = K // 128
    return M * K + 4 * M + N * K + 4 * N * G + 2 * M * N


def quant_bytes(M, K):
    """Algorithmic bytes of one quantize_act launch: x (BF16) read, q and sa written."""
    return 2 * M * K + M * K + 4 * M


def sources_digest():
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel_key):
    """HBM bytes per launch from the committed counter runs, if they match these sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("sources") != sources_digest():
        return None
    ent = t.get("kernels", {}).get(kernel_key)
    return None if ent is None else ent.get("bytes_per_launch")


class Linear:
    """Device-resident inputs/outputs of one linear layer, `copies` rotating copies."""

    def __init__(self, torch, M, K, N, p, f, copies, device, seed=0):
        from block_scaled_bit_amd import synth
        d = synth.linear_inputs(M, K, N, outlier_p=p, outlier_f=f, seed=seed)
        self.M, self.K, self.N = M, K, N
        x = torch.from_numpy(d["x"].view("int16")).to(device)
        qw = torch.from_numpy(d["qw"]).to(device)
        sw = torch.from_numpy(d["sw"]).to(device)
        self.bufs = []
        for _ in range(copies):
            b = dict(x=x.clone(), qw=qw.clone(), sw=sw.clone(),
                     q=torch.empty((M, K), dtype=torch.int8, device=device),
                     sa=torch.empty((M,), dtype=torch.float32, device=device),
                     y=torch.empty((M, N), dtype=torch.int16, device=device))
            b["ptr"] = {k: v.data_ptr() for k, v in b.items()}
            self.bufs.append(b)
        del x, qw, sw


def enqueue(L, lin, stream, n, what=("quant", "gemm")):
    """Enqueue n passes over the rotating copies: the quantisation and/or the GEMM."""
    M, K, N = lin.M, lin.K, lin.N
    for i in range(n):
        p = lin.bufs[i % len(lin.bufs)]["ptr"]
        if "quant" in what:
            s = L.bsb_quantize_act(p["x"], M, K, p["q"], p["sa"], stream)
            if s:
                raise RuntimeError(L.bsb_status_string(s).decode())
        if "gemm" in what:
            s = L.bsb_gemm_w8a8_g128(p["q"], p["sa"], p["qw"], p["sw"], M, N, K, p["y"], 0,
                                     stream)
            if s:
                raise RuntimeError(L.bsb_status_string(s).decode())


def timed(torch, L, lin, stream, steps, warmup, what=("quant", "gemm")):
    """Warm up, then time `steps` back-to-back passes between two HIP events
    recorded on the launch stream (torch's current stream). Returns
    (ms per pass from the events, wall-clock s per pass)."""
    enqueue(L, lin, stream, warmup, what)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    enqueue(L, lin, stream, steps, what)
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return start.elapsed_time(end) / steps, wall / steps


def cpu_baseline(budget_s=10.0):
    """The oracle as it stands, on the decode workload, on this host's cores."""
    import numpy as np
    from block_scaled_bit_amd import synth
    import oracle
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        threads = max([i.get("num_threads", 1) for i in info if i.get("user_api") == "blas"] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    M, K, N = 32, 8192, 28672
    Ns = 7168                                # a quarter of the output columns
    d = synth.linear_inputs(M, K, Ns, outlier_p=0.005, outlier_f=30.0, seed=0)
    runs, t_tot = 0, 0.0
    while t_tot < budget_s and runs < 20:
        t0 = time.perf_counter()
        q, sa = oracle.quantize_act_ref(d["x"])
        oracle.gemm_fp32_ordered_ref(q, sa, d["qw"], d["sw"])
        t_tot += time.perf_counter() - t0
        runs += 1
    t = t_tot / runs
    byts = quant_bytes(M, K) + gemm_bytes(M, Ns, K)
    return {"value": round(byts / t / 1e9, 4), "unit": "GB/s", "cores": int(threads),
            "kind": "oracle",
            "sample": (f"oracle quantize_act_ref + gemm_fp32_ordered_ref on M={M}, K={K} and "
                       f"{Ns} of the {N} output columns (same per-column work as the full "
                       f"layer), mean of {runs} runs = {t:.3f} s; GB/s = that sample's "
                       f"algorithmic bytes / time")}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--copies", type=int, default=5, help="rotating weight copies (decode)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    from block_scaled_bit_amd import _lib
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    L = _lib.lib()
    stream = torch.cuda.current_stream(dev).cuda_stream
    props = torch.cuda.get_device_properties(dev)
    log(f"device: {props.name} {getattr(props, 'gcnArchName', '')} CUs={props.multi_processor_count}")

    # counter calibration: a plain copy of known size (read 512 MiB, write 512 MiB)
    cal = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    cal_dst = torch.empty_like(cal)
    cal_dst.copy_(cal)
    torch.cuda.synchronize()
    del cal, cal_dst

    # ---- decode-shaped linear: the step ----
    M, K, N = 32, 8192, 28672
    lin = Linear(torch, M, K, N, 0.005, 30.0, args.copies, dev)
    ms_step, wall = timed(torch, L, lin, stream, args.steps, args.warmup)
    # per-kernel mean durations: each kernel alone, back to back, same buffers
    g_avg, _ = timed(torch, L, lin, stream, args.steps, args.warmup, ("gemm",))
    q_avg, _ = timed(torch, L, lin, stream, args.steps, args.warmup, ("quant",))
    step_bytes = quant_bytes(M, K) + gemm_bytes(M, N, K)
    g_bytes = gemm_bytes(M, N, K)
    achieved = g_bytes / (g_avg * 1e-3) / 1e9
    log(f"decode step {ms_step * 1e3:.1f} us (wall {wall * 1e6:.1f} us/step); "
        f"gemm {g_avg * 1e3:.1f} us = {achieved:.0f} GB/s; quant {q_avg * 1e3:.1f} us")
    del lin
    torch.cuda.empty_cache()

    out = {
        "metric": METRIC,
        "value": round(step_bytes / (ms_step * 1e-3) / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": "decode-shaped W8A8-g128 linear: quantize_act + gemm_w8a8_g128 "
                               "(BF16 out)", "M": M, "K": K, "N": N, "group": 128,
                   "weight_copies": args.copies,
                   "tops": round(2.0 * M * N * K / (ms_step * 1e-3) / 1e12, 2)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic("gemm_decode"),
                     "kernel": "gemm_smallm_kernel (M<=32)",
                     "timing": "mean of back-to-back launches between HIP events on the launch stream",
                     "bytes_per_launch": g_bytes, "avg_us": round(g_avg * 1e3, 2),
                     "quant_avg_us": round(q_avg * 1e3, 2)},
    }

    # ---- prefill-shaped GEMM ----
    if not args.no_prefill:
        Mp, Kp, Np = 4096, 8192, 8192
        pre = Linear(torch, Mp, Kp, Np, 0.005, 30.0, 3, dev)
        # quantise once per copy, then time the GEMM alone
        for b in pre.bufs:
            L.bsb_quantize_act(b["ptr"]["x"], Mp, Kp, b["ptr"]["q"], b["ptr"]["sa"], stream)
        psteps = max(5, min(50, args.steps // 4))
        pg, _ = timed(torch, L, pre, stream, psteps, max(2, args.warmup // 4), ("gemm",))
        tops = 2.0 * Mp * Np * Kp / (pg * 1e-3) / 1e12
        log(f"prefill gemm {pg * 1e3:.1f} us = {tops:.0f} TOPS")
        out["prefill"] = {"M": Mp, "K": Kp, "N": Np, "avg_us": round(pg * 1e3, 2),
                          "tops": round(tops, 1), "peak_tops": INT8_PEAK_TOPS,
                          "frac": round(tops / INT8_PEAK_TOPS, 4), "bound": "mfma",
                          "kernel": "gemm_tile_kernel 128x128",
                          "traffic": measured_traffic("gemm_prefill")}
        del pre
        torch.cuda.empty_cache()

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
