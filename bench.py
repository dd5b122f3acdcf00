"""Benchmark of the block-scaled INT8 linear layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step = one pass of the hot path over one batch: dynamic per-token INT8
quantisation of the BF16 activations (bsb_quantize_act) followed by the W8A8
per-group-128 GEMM with BF16 output on the decode-shaped linear M=32 tokens,
K=8192, N=28672 (seeded synthetic inputs: activations N(0,1) with 0.5 %
outliers x30, INT8 weights uniform in [-127,127], lognormal group scales). The
GEMM reads the weights in the matrix cores' operand order
(bsb_gemm_w8a8_g128_packed, bit-identical to bsb_gemm_w8a8_g128 on the
row-major weights); they are repacked once per weight copy while the inputs
are set up, as a serving stack does at load time, outside the timed region.
All inputs are resident in HBM before timing starts; the weights are rotated
over several copies (> 1 GB of traffic between reuses) so that the 256 MB
last-level cache cannot serve them.

Reported (one JSON line on stdout):
  value          algorithmic HBM bytes of the step / step time, GB/s
  row_major      the same GEMM on the row-major weights (bsb_gemm_w8a8_g128)
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
  rows           every other workload, each kernel timed alone the same way
                 with its own rotating input sets: the tiny linear (16x1024x1024),
                 the prefill quantisation, the routed MoE layer (4096 tokens,
                 top-8 of 64 Zipf-routed experts, K=4096, N=2048: quantisation,
                 gather into expert order, grouped GEMM, top-k combine), the block-format decoders (FP8 [128,128]
                 4096x7168 in both dialects, MXFP4 8x2048x4096) and the dense and
                 grouped GEMMs on the decoded weights at 32 and 1024 tokens
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
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense BF16 MFMA, published
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
COUNTER_FILE = os.path.join(ROOT, "profiles", "mfma_counters.json")
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

    def __init__(self, torch, M, K, N, p, f, copies, device, seed=0, L=None, stream=None):
        """With L and stream given, each copy also holds its weights repacked into the
        matrix cores' operand order, and the GEMM passes read those."""
        from block_scaled_bit_amd import synth
        d = synth.linear_inputs(M, K, N, outlier_p=p, outlier_f=f, seed=seed)
        self.M, self.K, self.N = M, K, N
        self.packed = L is not None
        x = torch.from_numpy(d["x"].view("int16")).to(device)
        qw = torch.from_numpy(d["qw"]).to(device)
        sw = torch.from_numpy(d["sw"]).to(device)
        self.bufs = []
        for _ in range(copies):
            b = dict(x=x.clone(), qw=qw.clone(), sw=sw.clone(),
                     q=torch.empty((M, K), dtype=torch.int8, device=device),
                     sa=torch.empty((M,), dtype=torch.float32, device=device),
                     y=torch.empty((M, N), dtype=torch.int16, device=device))
            if self.packed:
                b["qwp"] = torch.empty((N * K,), dtype=torch.int8, device=device)
                s = L.bsb_repack_weights_mfma(b["qw"].data_ptr(), N, K, b["qwp"].data_ptr(),
                                              stream)
                if s:
                    raise RuntimeError(L.bsb_status_string(s).decode())
            b["ptr"] = {k: v.data_ptr() for k, v in b.items()}
            self.bufs.append(b)
        del x, qw, sw


def enqueue(L, lin, stream, n, what=("quant", "gemm")):
    """Enqueue n passes over the rotating copies: the quantisation and/or the GEMM
    ("gemm": on the packed weights where the copies hold them; "gemm_rm": always on
    the row-major weights)."""
    M, K, N = lin.M, lin.K, lin.N
    for i in range(n):
        p = lin.bufs[i % len(lin.bufs)]["ptr"]
        if "quant" in what:
            s = L.bsb_quantize_act(p["x"], M, K, p["q"], p["sa"], stream)
            if s:
                raise RuntimeError(L.bsb_status_string(s).decode())
        if "gemm" in what and lin.packed:
            s = L.bsb_gemm_w8a8_g128_packed(p["q"], p["sa"], p["qwp"], p["sw"], M, N, K, p["y"],
                                            0, stream)
            if s:
                raise RuntimeError(L.bsb_status_string(s).decode())
        elif "gemm" in what or "gemm_rm" in what:
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


WARM_MS = 25.0   # untimed work before each timed row: the clock settles under load


def warm_up(torch, call, calls, ms=WARM_MS):
    """At least `calls` untimed calls, and more until `ms` of GPU time have passed
    (the first milliseconds of a workload run at a lower, rising clock)."""
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    done = 0
    while True:
        for _ in range(max(1, calls - done)):
            call()
            done += 1
        b.record()
        torch.cuda.synchronize()
        if a.elapsed_time(b) >= ms or done >= 10000:
            return


def percall(torch, call, n, warmup):
    """Per-call durations: a HIP event pair around each of n calls on the launch
    stream (torch's current stream), after `warmup` untimed calls (and at least
    WARM_MS of untimed work). Returns a dict of median / p10 / p90 / mean in
    microseconds."""
    warm_up(torch, call, warmup)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n)]
    torch.cuda.synchronize()
    for a, b in ev:
        a.record()
        call()
        b.record()
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) * 1e3 for a, b in ev)

    def q(f):
        return round(t[min(n - 1, int(f * (n - 1) + 0.5))], 2)
    return {"median_us": q(0.5), "p10_us": q(0.1), "p90_us": q(0.9),
            "mean_us": round(sum(t) / n, 2), "calls": n}


def read_sclk_mhz():
    """The GPU's current shader clock from sysfs (None where it is not readable)."""
    import glob
    for f in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            with open(f) as h:
                for line in h:
                    if line.startswith("S:") or line.rstrip().endswith("*"):
                        return int(line.split(":")[1].strip().lower().split("mhz")[0])
        except (OSError, ValueError, IndexError):
            continue
    return None


def sampled_sclk(torch, call, seconds=0.4):
    """Shader clocks sampled from sysfs while `call` runs back to back for about
    `seconds`: (median, min, max) in MHz, or None."""
    import threading
    samples, stop = [], threading.Event()

    def sampler():
        while not stop.is_set():
            v = read_sclk_mhz()
            if v is not None:
                samples.append(v)
            stop.wait(0.01)
    call()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    call()
    b.record()
    torch.cuda.synchronize()
    n = max(1, int(seconds / max(1e-6, a.elapsed_time(b) * 1e-3)))
    th = threading.Thread(target=sampler, daemon=True)
    th.start()
    for _ in range(n):
        call()
    torch.cuda.synchronize()
    stop.set()
    th.join()
    busy = [v for v in samples if v > 600] or samples   # drop idle readings at the edges
    if not busy:
        return None
    busy.sort()
    return {"median_mhz": busy[len(busy) // 2], "min_mhz": busy[0], "max_mhz": busy[-1],
            "samples": len(busy), "source": "sysfs pp_dpm_sclk"}


def measured_peaks(torch, L, stream, dev, a_bytes=None, b_bytes=None):
    """What this part sustains, measured with the library's probes: a streaming
    HBM read of 2 GiB (8x the last-level cache) and INT8 MFMA-only loops on
    uniform random codes and (when given) on the prefill workload's own
    activation and weight bytes (the matrix cores' rate depends on the operand bits)."""
    out = torch.empty((131072,), dtype=torch.int32, device=dev)
    nbytes = 2 << 30
    src = torch.empty((nbytes,), dtype=torch.uint8, device=dev)
    src.fill_(0x5A)

    def hbm():
        _ok(L, L.bsb_probe_hbm_read(src.data_ptr(), nbytes, out.data_ptr(), stream))
    h = percall(torch, hbm, 10, 2)
    # the same read at the decode GEMM's size (its weights: 232 MiB), windows of the
    # 2 GiB buffer in turn so that no call finds its bytes in a cache
    small = 232 << 20
    win = [0]

    def hbm_small():
        off = (win[0] % (nbytes // small)) * small
        win[0] += 1
        _ok(L, L.bsb_probe_hbm_read(src.data_ptr() + off, small, out.data_ptr(), stream))
    hs = percall(torch, hbm_small, 10, 2)
    # a read + write stream, as the decoders run: 512 MiB copied by the copy probe
    cb = 512 << 20
    dst = torch.empty((cb,), dtype=torch.uint8, device=dev)
    cwin = [0]

    def copy():
        off = (cwin[0] % (nbytes // cb)) * cb
        cwin[0] += 1
        _ok(L, L.bsb_probe_hbm_copy(src.data_ptr() + off, dst.data_ptr(), cb, stream))
    cs = percall(torch, copy, 10, 2)
    del src, dst
    torch.cuda.empty_cache()
    res = {"hbm_read_gbs": round(nbytes / (h["median_us"] * 1e-6) / 1e9, 1),
           "hbm_read_probe": "2 GiB streamed once per call, median of 10 calls",
           "hbm_read_gbs_232mib": round(small / (hs["median_us"] * 1e-6) / 1e9, 1),
           "copy_gbs": round(2 * cb / (cs["median_us"] * 1e-6) / 1e9, 1),
           "copy_probe": ("bsb_probe_hbm_copy of 512 MiB windows of the 2 GiB buffer (read + "
                          "write bytes, non-temporal), median of 10")}
    rounds = 512   # about a millisecond of matrix-core work per call
    ops = 2048 * rounds * 64 * 65536   # 131072 threads = 2048 waves of 64 MFMAs per round

    def mfma_rate(a, b, probe=None):
        probe = probe or L.bsb_probe_mfma_i8
        def call():
            _ok(L, probe(a.data_ptr(), b.data_ptr(), a.numel(), rounds, out.data_ptr(), stream))
        m = percall(torch, call, 10, 3)
        return round(ops / (m["median_us"] * 1e-6) / 1e12, 1)
    g = torch.Generator(device="cpu").manual_seed(0)
    u8 = 8 << 20
    ua = torch.randint(-127, 128, (u8,), dtype=torch.int8, generator=g).to(dev)
    ub = torch.randint(-127, 128, (u8,), dtype=torch.int8, generator=g).to(dev)
    res["mfma_i8_tops_uniform"] = mfma_rate(ua, ub)
    if a_bytes is not None and b_bytes is not None:
        n = min(u8, a_bytes.numel(), b_bytes.numel()) // 16 * 16
        wa, wb = a_bytes.reshape(-1)[:n], b_bytes.reshape(-1)[:n]
        res["mfma_i8_tops_workload"] = mfma_rate(wa, wb)
        # the same stream with the per-group epilogue beside it (4 conversions and
        # 4 fused multiply-adds after every MFMA, as the W8A8-g128 kernels run)
        res["mfma_i8_epilogue_tops_workload"] = mfma_rate(wa, wb, L.bsb_probe_mfma_i8_epilogue)
    res["mfma_probe"] = ("only v_mfma_i32_32x32x32_i8, 2 waves per SIMD on every CU, operands "
                         "cycled over 8 register sets; median of 10 calls; the epilogue probe "
                         "adds the per-group conversion and fused multiply-add work, no memory")
    return res


def counter_summary(kernel_key):
    """INT8 MFMA counters of one kernel from the committed rocprofv3 runs, if they
    match these sources: ops counted by SQ_INSTS_VALU_MFMA_MOPS_I8 against 2MNK, the
    F16/BF16/F8 MFMA op counts, and utilisation = MFMA busy cycles per SIMD / the
    kernel's cycles at the clock GRBM_GUI_ACTIVE gives."""
    try:
        with open(COUNTER_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("sources") != sources_digest():
        return None
    return t.get("kernels", {}).get(kernel_key)


def cpu_baseline(budget_s=12.0):
    """The oracle as it stands, on the decode workload, on this host's cores,
    stage by stage: quantisation, the exact INT32 group partials (float64 BLAS),
    the float64 definition with its magnitude, and the float32 replay in the
    stated order (what the strict parity checks compare against)."""
    import numpy as np
    from block_scaled_bit_amd import synth
    import oracle
    cores = len(os.sched_getaffinity(0))
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        blas = max([i.get("num_threads", 1) for i in info if i.get("user_api") == "blas"] or [1])
    except Exception:
        blas = None
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    M, K, N = 32, 8192, 28672
    Ns = 7168                                # a quarter of the output columns
    d = synth.linear_inputs(M, K, Ns, outlier_p=0.005, outlier_f=30.0, seed=0)
    stages = {"quantize_act_ref": 0.0, "group_partials_ref": 0.0, "gemm_ref": 0.0,
              "gemm_fp32_ordered_ref": 0.0}
    runs, t_tot = 0, 0.0
    while t_tot < budget_s and runs < 1000:
        t0 = time.perf_counter()
        q, sa = oracle.quantize_act_ref(d["x"])
        t1 = time.perf_counter()
        oracle.gemm_fp32_ordered_ref(q, sa, d["qw"], d["sw"])
        t2 = time.perf_counter()
        stages["quantize_act_ref"] += t1 - t0
        stages["gemm_fp32_ordered_ref"] += t2 - t1
        t_tot += t2 - t0
        runs += 1
    # the other two stages once each, outside the throughput figure
    t0 = time.perf_counter()
    oracle.group_partials_ref(q, d["qw"])
    t1 = time.perf_counter()
    oracle.gemm_ref(q, sa, d["qw"], d["sw"])
    t2 = time.perf_counter()
    t = t_tot / runs
    byts = quant_bytes(M, K) + gemm_bytes(M, Ns, K)
    return {"value": round(byts / t / 1e9, 4), "unit": "GB/s", "cores": cores,
            "kind": "oracle",
            "sample": (f"oracle quantize_act_ref + gemm_fp32_ordered_ref on M={M}, K={K} and "
                       f"{Ns} of the {N} output columns (same per-column work as the full "
                       f"layer), mean of {runs} runs = {t:.3f} s; GB/s = that sample's "
                       f"algorithmic bytes / time"),
            "cores_affinity": cores, "blas_threads": blas, "cpu_model": model,
            "stage_s": {"quantize_act_ref": round(stages["quantize_act_ref"] / runs, 4),
                        "gemm_fp32_ordered_ref": round(stages["gemm_fp32_ordered_ref"] / runs, 4),
                        "group_partials_ref": round(t1 - t0, 4),
                        "gemm_ref": round(t2 - t1, 4)}}


def _decoders_at_load_size(torch, L, stream, steps, dev, rows, log):
    """The two decoders over a whole layer's weights at once (a 16384 x 7168 FP8
    linear; 32 MXFP4 experts of 2048 x 4096), where the fixed cost of a launch
    (a few microseconds) is small against the stream; random bytes with finite
    UE8M0 exponents (the decoders' time does not depend on the values)."""
    g = torch.Generator(device=dev)
    g.manual_seed(5)
    N, K = 16384, 7168
    byts = N * K + (N // 128) * (K // 128) + N * K + 4 * N * (K // 128)
    sets = []
    for _ in range(_copies(byts)):
        o = dict(w=torch.randint(0, 256, (N, K), dtype=torch.uint8, device=dev, generator=g),
                 bs=torch.randint(100, 140, (N // 128, K // 128), dtype=torch.uint8, device=dev,
                                  generator=g),
                 qw=torch.empty((N, K), dtype=torch.int8, device=dev),
                 sw=torch.empty((N, K // 128), dtype=torch.float32, device=dev))
        o["w"][(o["w"] & 0x7F) == 0x7F] = 0   # OCP NaN bytes are outside the domain
        sets.append({k: v.data_ptr() for k, v in o.items()} | {"_keep": o})
    tf = Row("decode fp8 (layer)", sets, lambda p, st: _ok(
        L, L.bsb_decode_fp8_block(p["w"], p["bs"], N, K, 0, p["qw"], p["sw"], st))).time(
        torch, stream, steps, 3)
    rows[f"blockfmt_decode_fp8_ocp_{N}x{K}"] = _rate(tf * 1e3, byts=byts)
    log(f"decode fp8 {N}x{K} {tf * 1e3:.1f} us")
    del sets
    torch.cuda.empty_cache()
    E, N, K = 32, 2048, 4096
    byts = E * N * K // 2 + E * N * K // 32 + E * N * K + 4 * E * N * (K // 128)
    sets = []
    for _ in range(_copies(byts)):
        o = dict(pk=torch.randint(0, 256, (E, N, K // 2), dtype=torch.uint8, device=dev,
                                  generator=g),
                 sc=torch.randint(100, 140, (E, N, K // 32), dtype=torch.uint8, device=dev,
                                  generator=g),
                 qw=torch.empty((E * N * K,), dtype=torch.int8, device=dev),
                 sw=torch.empty((E, N, K // 128), dtype=torch.float32, device=dev))
        sets.append({k: v.data_ptr() for k, v in o.items()} | {"_keep": o})
    for packed in (False, True):
        fn = L.bsb_decode_mxfp4_packed if packed else L.bsb_decode_mxfp4
        tx = Row("decode mxfp4 (layer)", sets, lambda p, st, fn=fn: _ok(
            L, fn(p["pk"], p["sc"], E, N, K, p["qw"], p["sw"], st))).time(torch, stream, steps, 3)
        key = f"blockfmt_decode_mxfp4_{E}x{N}x{K}" + ("_packed" if packed else "")
        rows[key] = _rate(tx * 1e3, byts=byts)
        log(f"decode mxfp4 {E}x{N}x{K}{' packed' if packed else ''} {tx * 1e3:.1f} us")
    del sets
    torch.cuda.empty_cache()


class Row:
    """One measured workload: device-resident inputs in `copies` rotating sets
    and a raw C-ABI call that enqueues one pass over set i."""

    def __init__(self, name, sets, call):
        self.name, self.sets, self.call = name, sets, call

    def time(self, torch, stream, steps, warmup):
        """Mean ms per pass over `steps` back-to-back passes between HIP events
        recorded on the launch stream."""
        n = len(self.sets)
        k = [0]

        def one():
            self.call(self.sets[k[0] % n], stream)
            k[0] += 1
        warm_up(torch, one, warmup)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for i in range(steps):
            self.call(self.sets[i % n], stream)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps


def _ok(L, status):
    if status:
        raise RuntimeError(L.bsb_status_string(status).decode())


def _copies(bytes_per_set, floor=1 << 30, cap=64):
    """Rotating sets so that a set is reused only after >= 1 GiB of other traffic."""
    return max(1, min(cap, -(-floor // max(1, bytes_per_set)) + 1))


def _rate(us, ops=None, byts=None, bound="hbm", peak_tops=None):
    """avg_us plus achieved TOPS / GB/s against the published peaks (the matrix
    peak of the path's own type: INT8 unless peak_tops says otherwise)."""
    peak_tops = INT8_PEAK_TOPS if peak_tops is None else peak_tops
    r = {"avg_us": round(us, 2), "bound": bound}
    t = us * 1e-6
    if byts is not None:
        r["bytes"] = int(byts)
        r["gbs"] = round(byts / t / 1e9, 1)
        r["hbm_frac"] = round(byts / t / 1e9 / HBM_PEAK_GBS, 4)
    if ops is not None:
        r["ops"] = int(ops)
        r["tops"] = round(ops / t / 1e12, 1)
        r["mfma_frac"] = round(ops / t / 1e12 / peak_tops, 4)
        if peak_tops != INT8_PEAK_TOPS:
            r["peak_tops"] = peak_tops
    if ops is not None and byts is not None:
        # a kernel bound by both: the slower roofline over the measured time
        r["frac"] = round(max(ops / (peak_tops * 1e12), byts / (HBM_PEAK_GBS * 1e9)) / t, 4)
    else:
        r["frac"] = r.get("mfma_frac" if bound == "mfma" else "hbm_frac")
    return r


def extra_rows(torch, L, stream, dev, steps):
    """Every other workload of the path, each kernel timed on its own:
    the tiny linear, the prefill quantisation, the per-channel and per-tensor
    GEMMs at the decode and prefill shapes, the routed MoE layer, the
    block-format weights (decoders, then the dense and grouped GEMMs on the
    decoded weights) and the INT8 KV cache (write, decode attention)."""
    import numpy as np
    from block_scaled_bit_amd import synth
    rows = {}

    def t(x):
        return torch.from_numpy(np.ascontiguousarray(x)).to(dev)

    def linear_rows(tag, M, K, N, p, f, packed=False):
        """Mean us of quantize_act and of the GEMM; with packed=True also of the GEMM on
        weights repacked into the matrix cores' operand order (a third value)."""
        d = synth.linear_inputs(M, K, N, outlier_p=p, outlier_f=f, seed=0)
        gb = gemm_bytes(M, N, K)
        n = _copies(gb)
        x, qw, sw = t(d["x"].view(np.int16)), t(d["qw"]), t(d["sw"])
        sets = []
        for _ in range(n):
            b = dict(x=x.clone(), qw=qw.clone(), sw=sw.clone(),
                     q=torch.empty((M, K), dtype=torch.int8, device=dev),
                     sa=torch.empty((M,), dtype=torch.float32, device=dev),
                     y=torch.empty((M, N), dtype=torch.int16, device=dev))
            if packed:
                b["qwp"] = torch.empty((N * K,), dtype=torch.int8, device=dev)
                _ok(L, L.bsb_repack_weights_mfma(b["qw"].data_ptr(), N, K, b["qwp"].data_ptr(),
                                                 stream))
            sets.append({k: v.data_ptr() for k, v in b.items()} | {"_keep": b})
        quant = Row(f"{tag} quantize_act", sets, lambda p, st: _ok(
            L, L.bsb_quantize_act(p["x"], M, K, p["q"], p["sa"], st)))
        gemm = Row(f"{tag} gemm", sets, lambda p, st: _ok(
            L, L.bsb_gemm_w8a8_g128(p["q"], p["sa"], p["qw"], p["sw"], M, N, K, p["y"], 0, st)))
        tq = quant.time(torch, stream, steps, 3)
        tg = gemm.time(torch, stream, steps, 3)
        if not packed:
            return tq, tg
        for b in sets:   # the quantised activations the packed GEMM reads
            _ok(L, L.bsb_quantize_act(b["x"], M, K, b["q"], b["sa"], stream))
        tp = Row(f"{tag} gemm packed", sets, lambda p, st: _ok(
            L, L.bsb_gemm_w8a8_g128_packed(p["q"], p["sa"], p["qwp"], p["sw"], M, N, K, p["y"], 0,
                                           st))).time(torch, stream, steps, 3)
        return tq, tg, tp

    # tiny linear: latency-bound, reported in microseconds
    tq, tg = linear_rows("tiny", 16, 1024, 1024, 0.01, 20.0)
    rows["tiny_16x1024x1024_quant"] = _rate(tq * 1e3, byts=quant_bytes(16, 1024),
                                            bound="latency")
    rows["tiny_16x1024x1024_gemm"] = _rate(tg * 1e3, ops=2 * 16 * 1024 * 1024,
                                           byts=gemm_bytes(16, 1024, 1024), bound="latency")
    log(f"tiny: quant {tq * 1e3:.1f} us, gemm {tg * 1e3:.1f} us")
    torch.cuda.empty_cache()

    # one GPU's share of the decode linear under 8-way column (tensor) parallelism:
    # N / 8 = 3584 columns, 29 MB of weights (the exchange itself is not run)
    tq, tg, tp = linear_rows("tp8", 32, 8192, 3584, 0.005, 30.0, packed=True)
    rows["tp8_share_decode_32x8192x3584_gemm"] = _rate(tg * 1e3, ops=2 * 32 * 3584 * 8192,
                                                       byts=gemm_bytes(32, 3584, 8192))
    rows["tp8_share_decode_32x8192x3584_gemm_packed"] = _rate(
        tp * 1e3, ops=2 * 32 * 3584 * 8192, byts=gemm_bytes(32, 3584, 8192))
    log(f"tp8 share of the decode linear: gemm {tg * 1e3:.1f} us, on packed weights "
        f"{tp * 1e3:.1f} us")
    torch.cuda.empty_cache()

    # prefill-shaped quantisation (the GEMM is timed separately)
    M, K = 4096, 8192
    d = synth.linear_inputs(M, K, 128, outlier_p=0.005, outlier_f=30.0, seed=0)
    x = t(d["x"].view(np.int16))
    sets = []
    for _ in range(_copies(quant_bytes(M, K))):
        b = dict(x=x.clone(), q=torch.empty((M, K), dtype=torch.int8, device=dev),
                 sa=torch.empty((M,), dtype=torch.float32, device=dev))
        sets.append({k: v.data_ptr() for k, v in b.items()} | {"_keep": b})
    tq = Row("prefill quant", sets, lambda p, st: _ok(
        L, L.bsb_quantize_act(p["x"], M, K, p["q"], p["sa"], st))).time(torch, stream, steps, 3)
    rows["prefill_4096x8192_quant"] = _rate(tq * 1e3, byts=quant_bytes(M, K))
    log(f"prefill quant {tq * 1e3:.1f} us")
    del sets, x
    torch.cuda.empty_cache()

    # the coarser weight-scale granularities on the same shapes: one scale per output
    # row (per-channel) or one for the whole weight (per-tensor), INT32 totals over
    # all of K rescaled once ([P3] sec. 3.1's taxonomy)
    for shape, (M, K, N) in (("decode_32x8192x28672", (32, 8192, 28672)),
                             ("prefill_4096x8192x8192", (4096, 8192, 8192))):
        d = synth.linear_inputs(M, K, N, outlier_p=0.005, outlier_f=30.0, seed=0)
        x, qw = t(d["x"].view(np.int16)), t(d["qw"])
        for form, ns in (("channel", N), ("tensor", 1)):
            sw = t(synth.channel_scales(ns))
            byts = M * K + 4 * M + N * K + 4 * ns + 2 * M * N
            sets = []
            for _ in range(_copies(byts)):
                b = dict(qw=qw.clone(), sw=sw.clone(),
                         q=torch.empty((M, K), dtype=torch.int8, device=dev),
                         sa=torch.empty((M,), dtype=torch.float32, device=dev),
                         y=torch.empty((M, N), dtype=torch.int16, device=dev))
                _ok(L, L.bsb_quantize_act(x.data_ptr(), M, K, b["q"].data_ptr(),
                                          b["sa"].data_ptr(), stream))
                sets.append({k: v.data_ptr() for k, v in b.items()} | {"_keep": b})
            stride = 1 if ns == N else 0
            tg = Row(f"{form} {shape}", sets, lambda p, st: _ok(
                L, L.bsb_gemm_w8a8_channel(p["q"], p["sa"], p["qw"], p["sw"], stride, M, N, K,
                                           p["y"], 0, st))).time(torch, stream, steps, 3)
            rows[f"granularity_{form}_{shape}"] = _rate(
                tg * 1e3, ops=2 * M * N * K, byts=byts, bound="hbm" if M <= 64 else "mfma")
            log(f"per-{form} {shape}: gemm {tg * 1e3:.1f} us")
            del sets
        del x, qw
        torch.cuda.empty_cache()

    # the BF16-activation routes at the decode shape: weight-only INT8 (W8A16, no
    # activation quantisation) and BF16 weights (twice the weight bytes)
    M, K, N = 32, 8192, 28672
    d = synth.linear_inputs(M, K, N, outlier_p=0.005, outlier_f=30.0, seed=0)
    x, qw, sw = t(d["x"].view(np.int16)), t(d["qw"]), t(d["sw"])
    byts = 2 * M * K + N * K + 4 * N * K // 128 + 2 * M * N
    sets = []
    for _ in range(_copies(byts)):
        b = dict(x=x.clone(), qw=qw.clone(), sw=sw.clone(),
                 y=torch.empty((M, N), dtype=torch.int16, device=dev))
        sets.append({k: v.data_ptr() for k, v in b.items()} | {"_keep": b})
    tg = Row("w8a16 decode", sets, lambda p, st: _ok(
        L, L.bsb_gemm_w8a16_g128(p["x"], p["qw"], p["sw"], M, N, K, p["y"], 0, st))).time(
        torch, stream, steps, 3)
    rows["w8a16_decode_32x8192x28672"] = _rate(tg * 1e3, ops=2 * M * N * K, byts=byts,
                                               peak_tops=BF16_PEAK_TFLOPS)
    log(f"w8a16 decode: gemm {tg * 1e3:.1f} us")
    del sets, qw, sw
    torch.cuda.empty_cache()
    wb = t((np.random.default_rng(0).standard_normal((N, K)).astype(np.float32) * 0.02)
           ).to(torch.bfloat16).view(torch.int16)
    byts = 2 * M * K + 2 * N * K + 2 * M * N
    sets = []
    for _ in range(_copies(byts, cap=6)):
        b = dict(x=x.clone(), w=wb.clone(), y=torch.empty((M, N), dtype=torch.int16, device=dev))
        sets.append({k: v.data_ptr() for k, v in b.items()} | {"_keep": b})
    tg = Row("bf16 decode", sets, lambda p, st: _ok(
        L, L.bsb_gemm_bf16(p["x"], p["w"], M, N, K, p["y"], 0, st))).time(torch, stream, steps, 3)
    rows["bf16_decode_32x8192x28672"] = _rate(tg * 1e3, ops=2 * M * N * K, byts=byts,
                                              peak_tops=BF16_PEAK_TFLOPS)
    log(f"bf16 decode: gemm {tg * 1e3:.1f} us")
    del sets, wb, x
    torch.cuda.empty_cache()

    # the same two routes at the prefill shape (BF16 matrix instructions, 128x128 tiles)
    M, K, N = 4096, 8192, 8192
    d = synth.linear_inputs(M, K, N, outlier_p=0.005, outlier_f=30.0, seed=0)
    x, qw, sw = t(d["x"].view(np.int16)), t(d["qw"]), t(d["sw"])
    wb = t((np.random.default_rng(0).standard_normal((N, K), dtype=np.float32) * 0.02)
           ).to(torch.bfloat16).view(torch.int16)
    y = torch.empty((M, N), dtype=torch.int16, device=dev)
    p = {"x": x.data_ptr(), "qw": qw.data_ptr(), "sw": sw.data_ptr(), "w": wb.data_ptr(),
         "y": y.data_ptr()}
    ops = 2 * M * N * K
    tg = Row("w8a16 prefill", [p], lambda p, st: _ok(
        L, L.bsb_gemm_w8a16_g128(p["x"], p["qw"], p["sw"], M, N, K, p["y"], 0, st))).time(
        torch, stream, 10, 3)
    rows["w8a16_prefill_4096x8192x8192"] = _rate(
        tg * 1e3, ops=ops, byts=2 * M * K + N * K + 4 * N * K // 128 + 2 * M * N, bound="mfma",
        peak_tops=BF16_PEAK_TFLOPS)
    tb = Row("bf16 prefill", [p], lambda p, st: _ok(
        L, L.bsb_gemm_bf16(p["x"], p["w"], M, N, K, p["y"], 0, st))).time(torch, stream, 10, 3)
    rows["bf16_prefill_4096x8192x8192"] = _rate(
        tb * 1e3, ops=ops, byts=2 * M * K + 2 * N * K + 2 * M * N, bound="mfma",
        peak_tops=BF16_PEAK_TFLOPS)
    log(f"prefill 4096x8192x8192: w8a16 {tg * 1e3:.1f} us, bf16 {tb * 1e3:.1f} us")
    del x, qw, sw, wb, y, p
    torch.cuda.empty_cache()

    # routed MoE layer: 4096 tokens, top-8 of 64 experts (Zipf, 4 empty), K=4096, N=2048
    m = synth.moe_inputs()
    R, E, K, N = m["R"], m["E"], m["K"], m["N"]
    G = K // 128
    off_h = m["offsets"]
    nonempty = int((np.diff(off_h) > 0).sum())
    xs, qw, sw, off = t(m["x_sorted"].view(np.int16)), t(m["qw"]), t(m["sw"]), t(off_h)
    q = torch.empty((R, K), dtype=torch.int8, device=dev)
    sa = torch.empty((R,), dtype=torch.float32, device=dev)
    y = torch.empty((R, N), dtype=torch.int16, device=dev)
    p = {"x": xs.data_ptr(), "q": q.data_ptr(), "sa": sa.data_ptr(), "qw": qw.data_ptr(),
         "sw": sw.data_ptr(), "off": off.data_ptr(), "y": y.data_ptr()}
    # 768 MB of weights and activations per pass: larger than the last-level cache
    tq = Row("moe quant", [p], lambda p, st: _ok(
        L, L.bsb_quantize_act(p["x"], R, K, p["q"], p["sa"], st))).time(torch, stream, 20, 3)
    tg = Row("moe grouped", [p], lambda p, st: _ok(
        L, L.bsb_grouped_gemm_w8a8_g128(p["q"], p["sa"], p["qw"], p["sw"], p["off"], E, R, N, K,
                                        p["y"], 0, st))).time(torch, stream, 20, 3)
    gbytes = R * K + 4 * R + nonempty * (N * K + 4 * N * G) + 2 * R * N + 4 * (E + 1)
    rows["moe_4096tok_top8_64e_quant"] = _rate(tq * 1e3, byts=quant_bytes(R, K))
    rows["moe_4096tok_top8_64e_grouped"] = _rate(tg * 1e3, ops=2 * R * N * K, byts=gbytes,
                                                 bound="mfma+hbm")
    rows["moe_4096tok_top8_64e_grouped"].update(rows=R, experts_nonempty=nonempty)
    cs = counter_summary("gemm_big_kernel<0, true, false> [grid 786432]")
    if cs:
        rows["moe_4096tok_top8_64e_grouped"].update(counters=cs, mfma_util=cs.get("mfma_util"))
    log(f"moe: quant {tq * 1e3:.1f} us, grouped {tg * 1e3:.1f} us")
    # one GPU's share under 8-way expert parallelism (experts e with e % 8 == r on
    # GPU r): the grouped GEMM over the 8 experts of the GPU with the most rows,
    # with their real skewed row counts (the all-to-all itself is not run)
    per = np.diff(off_h)
    gpu = max(range(8), key=lambda r: int(per[r::8].sum()))
    mine = list(range(gpu, E, 8))
    idx = np.concatenate([np.arange(off_h[e], off_h[e + 1]) for e in mine]).astype(np.int64)
    off8 = np.concatenate([[0], np.cumsum(per[mine])]).astype(np.int32)
    R8 = int(off8[-1])
    ii = torch.from_numpy(idx).to(dev)
    ei = torch.tensor(mine, dtype=torch.int64, device=dev)
    p8 = dict(q=q[ii].contiguous(), sa=sa[ii].contiguous(), qw=qw[ei].contiguous(),
              sw=sw[ei].contiguous(), off=t(off8),
              y=torch.empty((R8, N), dtype=torch.int16, device=dev))
    pp8 = {k: v.data_ptr() for k, v in p8.items()}
    t8 = Row("ep8 share grouped", [pp8], lambda p, st: _ok(
        L, L.bsb_grouped_gemm_w8a8_g128(p["q"], p["sa"], p["qw"], p["sw"], p["off"], 8, R8, N, K,
                                        p["y"], 0, st))).time(torch, stream, 20, 3)
    ne8 = int((per[mine] > 0).sum())
    b8 = R8 * K + 4 * R8 + ne8 * (N * K + 4 * N * G) + 2 * R8 * N + 36
    rows["ep8_share_moe_grouped"] = _rate(t8 * 1e3, ops=2 * R8 * N * K, byts=b8,
                                          bound="mfma+hbm") | {
        "gpu": gpu, "experts": mine, "rows": R8, "rows_per_gpu": [int(per[r::8].sum()) for r in range(8)]}
    log(f"ep8 share (GPU {gpu}, {R8} rows): grouped {t8 * 1e3:.1f} us")
    del p8, pp8, ii, ei
    # the glue either side: quantise the T tokens, gather into expert order,
    # (grouped GEMM), combine the top-k outputs per token
    T, topk = m["T"], m["topk"]
    xt = t(m["x_tokens"].view(np.int16))
    qt = torch.empty((T, K), dtype=torch.int8, device=dev)
    st = torch.empty((T,), dtype=torch.float32, device=dev)
    tor, rp, gate = t(m["token_of_row"]), t(m["row_of_pair"]), t(m["gate"])
    out = torch.empty((T, N), dtype=torch.int16, device=dev)
    p.update(xt=xt.data_ptr(), qt=qt.data_ptr(), st=st.data_ptr(), tor=tor.data_ptr(),
             rp=rp.data_ptr(), gate=gate.data_ptr(), out=out.data_ptr())
    tqt = Row("moe quant tokens", [p], lambda p, st_: _ok(
        L, L.bsb_quantize_act(p["xt"], T, K, p["qt"], p["st"], st_))).time(torch, stream, 20, 3)
    tga = Row("moe gather", [p], lambda p, st_: _ok(
        L, L.bsb_gather_rows(p["qt"], p["st"], p["tor"], R, T, K, p["q"], p["sa"], st_))).time(
        torch, stream, 20, 3)
    tco = Row("moe combine", [p], lambda p, st_: _ok(
        L, L.bsb_moe_combine(p["y"], p["rp"], p["gate"], T, topk, R, N, p["out"], st_))).time(
        torch, stream, 20, 3)
    rows["moe_4096tok_top8_64e_quant_tokens"] = _rate(tqt * 1e3, byts=quant_bytes(T, K))
    # gather: the token rows (which the last-level cache holds) are read once
    # per slot, the sorted rows written once; counted: T*K + R*K + scales + index
    rows["moe_4096tok_top8_64e_gather"] = _rate(tga * 1e3, byts=T * K + R * K + 4 * T + 8 * R)
    rows["moe_4096tok_top8_64e_combine"] = _rate(
        tco * 1e3, byts=2 * R * N + 2 * T * N + 8 * T * topk)
    # the grouped GEMM reading its rows through the token index (no gathered copy)
    tgg = Row("moe grouped gather", [p], lambda p, st_: _ok(
        L, L.bsb_grouped_gemm_w8a8_g128_gather(p["qt"], p["st"], p["tor"], T, p["qw"], p["sw"],
                                               p["off"], E, R, N, K, p["y"], 0, st_))).time(
        torch, stream, 20, 3)
    rows["moe_4096tok_top8_64e_grouped_gather"] = _rate(
        tgg * 1e3, ops=2 * R * N * K, byts=gbytes - R * K - 4 * R + T * K + 4 * T + 4 * R,
        bound="mfma+hbm") | {"vs_gather_then_grouped": round(tgg / (tga + tg), 3)}
    rows["moe_4096tok_top8_64e_layer"] = {
        "avg_us": round((tqt + tgg + tco) * 1e3, 2),
        "parts": "quantize_act(tokens) + grouped GEMM gathering its rows + moe_combine",
        "with_separate_gather_us": round((tqt + tga + tg + tco) * 1e3, 2),
        "quantise_after_gather_us": round((tq + tg) * 1e3, 2),
        "note": "with_separate_gather_us: gather_rows then the grouped GEMM; "
                "quantise_after_gather_us = quantize_act(gathered rows) + grouped GEMM, no combine"}
    log(f"moe glue: quant tokens {tqt * 1e3:.1f} us, gather {tga * 1e3:.1f} us, "
        f"combine {tco * 1e3:.1f} us; grouped GEMM gathering its rows {tgg * 1e3:.1f} us "
        f"(gather + grouped {(tga + tg) * 1e3:.1f} us)")
    del m, xs, qw, sw, off, q, sa, y, p, xt, qt, st, tor, rp, gate, out
    torch.cuda.empty_cache()

    # block formats: FP8 [128,128] dense 4096x7168 and MXFP4 experts 8x2048x4096
    b = synth.blockfmt_inputs(M=32)
    Nd, Kd, Ee, Ne, Ke = b["N_d"], b["K_d"], b["E"], b["N_e"], b["K_e"]
    Gd, Ge = Kd // 128, Ke // 128
    fp8_bytes = Nd * Kd + (Nd // 128) * (Kd // 128) + Nd * Kd + 4 * Nd * Gd
    w, bs = t(b["w_fp8"]), t(b["bs"])
    dsets = []
    for _ in range(_copies(fp8_bytes)):
        o = dict(w=w.clone(), bs=bs.clone(),
                 qw=torch.empty((Nd, Kd), dtype=torch.int8, device=dev),
                 sw=torch.empty((Nd, Gd), dtype=torch.float32, device=dev))
        dsets.append({k: v.data_ptr() for k, v in o.items()} | {"_keep": o})
    for dialect, dname in ((0, "ocp"), (1, "fnuz")):
        td = Row("decode fp8", dsets, lambda p, st, dl=dialect: _ok(
            L, L.bsb_decode_fp8_block(p["w"], p["bs"], Nd, Kd, dl, p["qw"], p["sw"], st))).time(
            torch, stream, steps, 3)
        rows[f"blockfmt_decode_fp8_{dname}_4096x7168"] = _rate(td * 1e3, byts=fp8_bytes)
        if dialect == 0:   # the same decode written in the packed GEMM's operand order
            tdp = Row("decode fp8 packed", dsets, lambda p, st: _ok(
                L, L.bsb_decode_fp8_block_packed(p["w"], p["bs"], Nd, Kd, 0, p["qw"], p["sw"],
                                                 st))).time(torch, stream, steps, 3)
            rows["blockfmt_decode_fp8_ocp_4096x7168_packed"] = _rate(tdp * 1e3, byts=fp8_bytes)
            log(f"fp8 decode into the packed layout {tdp * 1e3:.1f} us")
        log(f"decode fp8 {dname} {td * 1e3:.1f} us")
    # the BF16 route's load-time dequantisation of the same FP8 blocks
    bf_bytes = Nd * Kd + (Nd // 128) * (Kd // 128) + 2 * Nd * Kd
    bsets = []
    for i in range(_copies(bf_bytes)):
        o = dict(w=w.clone(), bs=bs.clone(),
                 wb=torch.empty((Nd, Kd), dtype=torch.int16, device=dev))
        bsets.append({k: v.data_ptr() for k, v in o.items()} | {"_keep": o})
    tb = Row("dequant fp8 bf16", bsets, lambda p, st: _ok(
        L, L.bsb_dequant_fp8_block_bf16(p["w"], p["bs"], Nd, Kd, 0, p["wb"], st))).time(
        torch, stream, steps, 3)
    rows["blockfmt_dequant_fp8_bf16_4096x7168"] = _rate(tb * 1e3, byts=bf_bytes)
    log(f"dequant fp8 -> bf16 {tb * 1e3:.1f} us")
    del bsets
    qwd = torch.empty((Nd, Kd), dtype=torch.int8, device=dev)
    swd = torch.empty((Nd, Gd), dtype=torch.float32, device=dev)
    _ok(L, L.bsb_decode_fp8_block(w.data_ptr(), bs.data_ptr(), Nd, Kd, 0, qwd.data_ptr(),
                                  swd.data_ptr(), stream))
    del dsets, w, bs
    torch.cuda.empty_cache()

    mx_bytes = Ee * Ne * Ke // 2 + Ee * Ne * Ke // 32 + Ee * Ne * Ke + 4 * Ee * Ne * Ge
    pk, sc = t(b["packed"]), t(b["scale"])
    msets = []
    for _ in range(_copies(mx_bytes)):
        o = dict(pk=pk.clone(), sc=sc.clone(),
                 qw=torch.empty((Ee, Ne, Ke), dtype=torch.int8, device=dev),
                 sw=torch.empty((Ee, Ne, Ge), dtype=torch.float32, device=dev))
        msets.append({k: v.data_ptr() for k, v in o.items()} | {"_keep": o})
    tm = Row("decode mxfp4", msets, lambda p, st: _ok(
        L, L.bsb_decode_mxfp4(p["pk"], p["sc"], Ee, Ne, Ke, p["qw"], p["sw"], st))).time(
        torch, stream, steps, 3)
    rows["blockfmt_decode_mxfp4_8x2048x4096"] = _rate(tm * 1e3, byts=mx_bytes)
    log(f"decode mxfp4 {tm * 1e3:.1f} us")
    # the same decode written in the grouped packed GEMM's operand order
    tmp = Row("decode mxfp4 packed", msets, lambda p, st: _ok(
        L, L.bsb_decode_mxfp4_packed(p["pk"], p["sc"], Ee, Ne, Ke, p["qw"], p["sw"], st))).time(
        torch, stream, steps, 3)
    rows["blockfmt_decode_mxfp4_8x2048x4096_packed"] = _rate(tmp * 1e3, byts=mx_bytes)
    log(f"decode mxfp4 into the packed layout {tmp * 1e3:.1f} us")
    qwe = torch.empty((Ee, Ne, Ke), dtype=torch.int8, device=dev)
    swe = torch.empty((Ee, Ne, Ge), dtype=torch.float32, device=dev)
    _ok(L, L.bsb_decode_mxfp4(pk.data_ptr(), sc.data_ptr(), Ee, Ne, Ke, qwe.data_ptr(),
                              swe.data_ptr(), stream))
    del msets, pk, sc
    torch.cuda.empty_cache()
    _decoders_at_load_size(torch, L, stream, steps, dev, rows, log)

    # GEMMs on the decoded weights, M = 32 and 1024 tokens (per expert for the grouped one)
    for Mt in (32, 1024):
        bb = b if Mt == 32 else synth.blockfmt_inputs(M=Mt)
        xd, xe = t(bb["x_d"].view(np.int16)), t(bb["x_e"].view(np.int16))
        offe = t(bb["offsets"])
        Re = Ee * Mt
        db = gemm_bytes(Mt, Nd, Kd)
        eb = Re * Ke + 4 * Re + Ee * (Ne * Ke + 4 * Ne * Ge) + 2 * Re * Ne + 4 * (Ee + 1)
        gs, es = [], []
        for _ in range(_copies(db)):
            o = dict(qw=qwd.clone(), sw=swd.clone(),
                     q=torch.empty((Mt, Kd), dtype=torch.int8, device=dev),
                     sa=torch.empty((Mt,), dtype=torch.float32, device=dev),
                     y=torch.empty((Mt, Nd), dtype=torch.int16, device=dev))
            if Mt == 32:   # the decoded weight repacked at load time for the packed GEMM
                o["qwp"] = torch.empty((Nd * Kd,), dtype=torch.int8, device=dev)
                _ok(L, L.bsb_repack_weights_mfma(o["qw"].data_ptr(), Nd, Kd, o["qwp"].data_ptr(),
                                                 stream))
            _ok(L, L.bsb_quantize_act(xd.data_ptr(), Mt, Kd, o["q"].data_ptr(),
                                      o["sa"].data_ptr(), stream))
            gs.append({k: v.data_ptr() for k, v in o.items()} | {"_keep": o})
        for _ in range(_copies(eb)):
            o = dict(qw=qwe.clone(), sw=swe.clone(), off=offe.clone(),
                     q=torch.empty((Re, Ke), dtype=torch.int8, device=dev),
                     sa=torch.empty((Re,), dtype=torch.float32, device=dev),
                     y=torch.empty((Re, Ne), dtype=torch.int16, device=dev))
            if Mt == 32:   # the stacked experts repacked at load time for the packed form
                o["qwp"] = torch.empty((Ee * Ne * Ke,), dtype=torch.int8, device=dev)
                _ok(L, L.bsb_repack_weights_mfma(o["qw"].data_ptr(), Ee * Ne, Ke,
                                                 o["qwp"].data_ptr(), stream))
            _ok(L, L.bsb_quantize_act(xe.data_ptr(), Re, Ke, o["q"].data_ptr(),
                                      o["sa"].data_ptr(), stream))
            es.append({k: v.data_ptr() for k, v in o.items()} | {"_keep": o})
        tg = Row("blockfmt gemm", gs, lambda p, st: _ok(
            L, L.bsb_gemm_w8a8_g128(p["q"], p["sa"], p["qw"], p["sw"], Mt, Nd, Kd, p["y"], 0,
                                    st))).time(torch, stream, steps, 3)
        te = Row("blockfmt grouped", es, lambda p, st: _ok(
            L, L.bsb_grouped_gemm_w8a8_g128(p["q"], p["sa"], p["qw"], p["sw"], p["off"], Ee, Re,
                                            Ne, Ke, p["y"], 0, st))).time(torch, stream, steps, 3)
        bound = "hbm" if Mt == 32 else "mfma"
        rows[f"blockfmt_gemm_m{Mt}_4096x7168"] = _rate(tg * 1e3, ops=2 * Mt * Nd * Kd,
                                                       byts=db, bound=bound)
        if Mt == 32:
            tp = Row("blockfmt gemm packed", gs, lambda p, st: _ok(
                L, L.bsb_gemm_w8a8_g128_packed(p["q"], p["sa"], p["qwp"], p["sw"], Mt, Nd, Kd,
                                               p["y"], 0, st))).time(torch, stream, steps, 3)
            rows["blockfmt_gemm_m32_4096x7168_packed"] = _rate(tp * 1e3, ops=2 * Mt * Nd * Kd,
                                                               byts=db, bound=bound)
            log(f"blockfmt M=32: gemm on packed weights {tp * 1e3:.1f} us")
            tep = Row("blockfmt grouped packed", es, lambda p, st: _ok(
                L, L.bsb_grouped_gemm_w8a8_g128_packed(p["q"], p["sa"], p["qwp"], p["sw"],
                                                       p["off"], Ee, Re, Ne, Ke, p["y"], 0,
                                                       st))).time(torch, stream, steps, 3)
            rows["blockfmt_grouped_m32_8x2048x4096_packed"] = _rate(
                tep * 1e3, ops=2 * Re * Ne * Ke, byts=eb, bound=bound)
            log(f"blockfmt M=32: grouped on packed weights {tep * 1e3:.1f} us")
        rows[f"blockfmt_grouped_m{Mt}_8x2048x4096"] = _rate(te * 1e3, ops=2 * Re * Ne * Ke,
                                                            byts=eb, bound=bound)
        log(f"blockfmt M={Mt}: gemm {tg * 1e3:.1f} us, grouped {te * 1e3:.1f} us")
        del gs, es, xd, xe, offe
        torch.cuda.empty_cache()
    del qwd, swd, qwe, swe
    torch.cuda.empty_cache()
    rows.update(kv_rows(torch, L, stream, dev, steps))
    return rows


def kv_rows(torch, L, stream, dev, steps):
    """The INT8 KV cache at 32 sequences x 4096 cached tokens, 64 query heads over
    8 KV heads of 128: one decode step's write of the new keys and values, and the
    decode attention over the whole cache (dequantisation fused in). Algorithmic
    bytes of the attention: the INT8 codes and float32 scales of every cached key
    and value, the BF16 queries and the BF16 output."""
    import numpy as np
    from block_scaled_bit_amd import synth
    from block_scaled_bit_amd import _lib as bsb_lib
    rows = {}
    c = synth.KV_CONFIG
    B, Hq, Hkv, T, D = c["B"], c["Hq"], c["Hkv"], c["T"], c["D"]
    inp = synth.kv_inputs(B, Hq, Hkv, T, lens=np.full(B, T), seed=0)

    def t(x):
        return torch.from_numpy(np.ascontiguousarray(x)).to(dev)

    kt = t(inp["k"].view(np.int16)).permute(0, 2, 1, 3).reshape(B * T, Hkv, D).contiguous()
    vt = t(inp["v"].view(np.int16)).permute(0, 2, 1, 3).reshape(B * T, Hkv, D).contiguous()
    seq = torch.arange(B, dtype=torch.int32, device=dev).repeat_interleave(T)
    pos = torch.arange(T, dtype=torch.int32, device=dev).repeat(B)
    kc, ks, vc, vs = bsb_lib.kv_cache_empty(B, Hkv, T, dev)
    _ok(L, L.bsb_kv_cache_write(kt.data_ptr(), vt.data_ptr(), seq.data_ptr(), pos.data_ptr(),
                                B * T, B, Hkv, T, D, kc.data_ptr(), ks.data_ptr(), vc.data_ptr(),
                                vs.data_ptr(), stream))
    # the BF16 cache the INT8 one replaces, written from the same keys and values
    kb, vb = (c.view(torch.int16) for c in bsb_lib.kv_cache_empty_bf16(B, Hkv, T, dev))
    _ok(L, L.bsb_kv_cache_write_bf16(kt.data_ptr(), vt.data_ptr(), seq.data_ptr(), pos.data_ptr(),
                                     B * T, B, Hkv, T, D, kb.data_ptr(), vb.data_ptr(), stream))
    # one decode step: the last slot of every sequence rewritten with its own key / value
    step = dict(k=kt.view(B, T, Hkv, D)[:, T - 1].contiguous(),
                v=vt.view(B, T, Hkv, D)[:, T - 1].contiguous(),
                seq=torch.arange(B, dtype=torch.int32, device=dev),
                pos=torch.full((B,), T - 1, dtype=torch.int32, device=dev))
    del kt, vt, seq, pos
    torch.cuda.empty_cache()
    wsets = [{k: v.data_ptr() for k, v in step.items()} | {"_keep": step}]
    tw = Row("kv write", wsets, lambda p, st: _ok(L, L.bsb_kv_cache_write(
        p["k"], p["v"], p["seq"], p["pos"], B, B, Hkv, T, D, kc.data_ptr(), ks.data_ptr(),
        vc.data_ptr(), vs.data_ptr(), st))).time(torch, stream, steps, 3)
    w_bytes = 2 * (B * Hkv * D * 2 + B * Hkv * D + 4 * B * Hkv) + 8 * B
    rows["kv_int8_write_decode_step_b32"] = _rate(tw * 1e3, byts=w_bytes)
    log(f"kv write (decode step) {tw * 1e3:.1f} us")

    a_bytes = 2 * B * Hkv * T * D + 8 * B * Hkv * T + 2 * B * Hq * D + 2 * B * Hq * D
    lens = t(inp["lens"])
    q = t(inp["q"].view(np.int16))
    wbytes = L.bsb_attention_workspace_bytes(B, Hq, T)
    asets = []
    for i in range(_copies(a_bytes)):
        o = dict(kc=kc if i == 0 else kc.clone(), ks=ks if i == 0 else ks.clone(),
                 vc=vc if i == 0 else vc.clone(), vs=vs if i == 0 else vs.clone(), q=q.clone(),
                 lens=lens, out=torch.empty((B, Hq, D), dtype=torch.int16, device=dev),
                 work=torch.empty((wbytes // 4,), dtype=torch.float32, device=dev))
        asets.append({k: v.data_ptr() for k, v in o.items()} | {"_keep": o})
    ta = Row("kv attention", asets, lambda p, st: _ok(L, L.bsb_attention_decode_int8kv(
        p["q"], p["kc"], p["ks"], p["vc"], p["vs"], p["lens"], B, Hq, Hkv, T, D, T, p["work"],
        wbytes, p["out"], 0, st))).time(torch, stream, steps, 3)
    rows["kv_int8_attention_decode_b32_t4096"] = _rate(ta * 1e3, byts=a_bytes) | {
        "kernel": "attn_split_kernel<0, 8, 1> (INT8 cache, one launch)", "traffic": measured_traffic("kv_attention")}
    log(f"kv attention (decode, 32 x 4096 tokens) {ta * 1e3:.1f} us")

    # two query tokens per sequence (checking a drafted token, a prefill chunk):
    # 2 x G = 16 query columns per KV head, the cache still read once
    Qn = 16 // (Hq // Hkv)
    if Qn > 1:
        c_bytes = 2 * B * Hkv * T * D + 8 * B * Hkv * T + 4 * B * Qn * Hq * D
        cw = L.bsb_attention_workspace_bytes(B, Qn * Hq, T)
        qc = t(synth.to_bf16_bits(np.random.default_rng(5).standard_normal(
            (B, Qn, Hq, D), dtype=np.float32)).view(np.int16))
        csets = []
        for i, a in enumerate(asets):
            o = dict(q=qc.clone(), out=torch.empty((B, Qn, Hq, D), dtype=torch.int16, device=dev),
                     work=torch.empty((cw // 4,), dtype=torch.float32, device=dev))
            csets.append(a | {k: v.data_ptr() for k, v in o.items()} | {"_keep2": o})
        tc = Row("kv attention chunk", csets, lambda p, st: _ok(L, L.bsb_attention_chunk_int8kv(
            p["q"], p["kc"], p["ks"], p["vc"], p["vs"], p["lens"], B, Qn, Hq, Hkv, T, D, T,
            p["work"], cw, p["out"], 0, st))).time(torch, stream, steps, 3)
        rows[f"kv_int8_attention_chunk{Qn}_b32_t4096"] = _rate(tc * 1e3, byts=c_bytes) | {
            "kernel": "attn_split_kernel<0, 8, 1> (INT8 cache, one launch)",
            "query_tokens": Qn, "vs_decode_time": round(tc / ta, 3)}
        log(f"kv attention ({Qn} query tokens per sequence) {tc * 1e3:.1f} us "
            f"({tc / ta:.2f}x the one-token time)")
        del csets
    del asets, kc, ks, vc, vs, step, wsets
    torch.cuda.empty_cache()

    # the same attention over the BF16 cache: the comparison the pages quote for
    # fusing the dequantisation (attention time with and without the INT8 cache)
    b_bytes = 4 * B * Hkv * T * D + 2 * B * Hq * D + 2 * B * Hq * D
    bsets = []
    for i in range(_copies(b_bytes)):
        o = dict(kc=kb if i == 0 else kb.clone(), vc=vb if i == 0 else vb.clone(), q=q.clone(),
                 lens=lens, out=torch.empty((B, Hq, D), dtype=torch.int16, device=dev),
                 work=torch.empty((wbytes // 4,), dtype=torch.float32, device=dev))
        bsets.append({k: v.data_ptr() for k, v in o.items()} | {"_keep": o})
    tbf = Row("kv attention bf16", bsets, lambda p, st: _ok(L, L.bsb_attention_decode_bf16kv(
        p["q"], p["kc"], p["vc"], p["lens"], B, Hq, Hkv, T, D, T, p["work"], wbytes, p["out"], 0,
        st))).time(torch, stream, steps, 3)
    rows["kv_bf16_attention_decode_b32_t4096"] = _rate(tbf * 1e3, byts=b_bytes) | {
        "kernel": "attn_split_kernel<1, 8, 1> (BF16 cache, one launch)",
        "traffic": measured_traffic("kv_attention_bf16"), "int8_kv_speedup": round(tbf / ta, 3)}
    log(f"kv attention over a BF16 cache {tbf * 1e3:.1f} us (INT8 cache {tbf / ta:.2f}x faster)")
    del bsets, kb, vb
    torch.cuda.empty_cache()
    return rows


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--copies", type=int, default=5, help="rotating weight copies (decode)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-rows", action="store_true",
                    help="skip the other workloads (tiny, MoE, block formats)")
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
    lin = Linear(torch, M, K, N, 0.005, 30.0, args.copies, dev, L=L, stream=stream)
    ms_step, wall = timed(torch, L, lin, stream, args.steps, args.warmup)
    # per-kernel mean durations: each kernel alone, back to back, same buffers
    g_avg, _ = timed(torch, L, lin, stream, args.steps, args.warmup, ("gemm",))
    q_avg, _ = timed(torch, L, lin, stream, args.steps, args.warmup, ("quant",))
    rm_avg, _ = timed(torch, L, lin, stream, args.steps, args.warmup, ("gemm_rm",))
    # per-call HIP events around the packed GEMM (copies rotated as in the step)
    it = [0]

    def one_gemm():
        p = lin.bufs[it[0] % len(lin.bufs)]["ptr"]
        it[0] += 1
        _ok(L, L.bsb_gemm_w8a8_g128_packed(p["q"], p["sa"], p["qwp"], p["sw"], M, N, K, p["y"], 0,
                                           stream))
    g_calls = percall(torch, one_gemm, max(20, min(200, args.steps)), 10)
    step_bytes = quant_bytes(M, K) + gemm_bytes(M, N, K)
    g_bytes = gemm_bytes(M, N, K)
    achieved = g_bytes / (g_avg * 1e-3) / 1e9
    rm_rate = g_bytes / (rm_avg * 1e-3) / 1e9
    log(f"decode step {ms_step * 1e3:.1f} us (wall {wall * 1e6:.1f} us/step); "
        f"gemm {g_avg * 1e3:.1f} us = {achieved:.0f} GB/s; quant {q_avg * 1e3:.1f} us; "
        f"row-major gemm {rm_avg * 1e3:.1f} us = {rm_rate:.0f} GB/s")
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
        "config": {"workload": "decode-shaped W8A8-g128 linear: quantize_act + "
                               "gemm_w8a8_g128_packed (weights in MFMA operand order, "
                               "BF16 out)", "M": M, "K": K, "N": N, "group": 128,
                   "weight_copies": args.copies,
                   "tops": round(2.0 * M * N * K / (ms_step * 1e-3) / 1e12, 2)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic("gemm_decode_packed"),
                     "kernel": "gemm_packed_kernel<2, 7, 0, true, false>",
                     "timing": "mean of back-to-back launches between HIP events on the launch stream",
                     "bytes_per_launch": g_bytes, "avg_us": round(g_avg * 1e3, 2),
                     "per_call": g_calls,
                     "quant_avg_us": round(q_avg * 1e3, 2)},
        "row_major": {"kernel": "gemm_smallm_kernel<2, 7, 0, ...>", "avg_us": round(rm_avg * 1e3, 2),
                      "achieved": round(rm_rate, 1), "frac": round(rm_rate / HBM_PEAK_GBS, 4),
                      "traffic": measured_traffic("gemm_decode")},
    }

    # ---- prefill-shaped GEMM ----
    if not args.no_prefill:
        Mp, Kp, Np = 4096, 8192, 8192
        pre = Linear(torch, Mp, Kp, Np, 0.005, 30.0, 3, dev)
        # quantise once per copy, then time the GEMM alone
        for b in pre.bufs:
            L.bsb_quantize_act(b["ptr"]["x"], Mp, Kp, b["ptr"]["q"], b["ptr"]["sa"], stream)
        psteps = max(5, min(50, args.steps // 4))
        pg, _ = timed(torch, L, pre, stream, psteps, 10, ("gemm",))
        pit = [0]

        def one_prefill():
            p = pre.bufs[pit[0] % len(pre.bufs)]["ptr"]
            pit[0] += 1
            _ok(L, L.bsb_gemm_w8a8_g128(p["q"], p["sa"], p["qw"], p["sw"], Mp, Np, Kp, p["y"], 0,
                                        stream))
        pc = percall(torch, one_prefill, max(10, min(40, args.steps // 5)), 5)
        ops = 2.0 * Mp * Np * Kp
        tops = ops / (pc["median_us"] * 1e-6) / 1e12
        log(f"prefill gemm median {pc['median_us']:.1f} us (p10 {pc['p10_us']:.1f}, p90 "
            f"{pc['p90_us']:.1f}; back-to-back mean {pg * 1e3:.1f} us) = {tops:.0f} TOPS")
        peaks = measured_peaks(torch, L, stream, dev, pre.bufs[0]["q"], pre.bufs[0]["qw"])
        clk = sampled_sclk(torch, one_prefill)
        log(f"measured peaks {peaks}; prefill clock {clk}")
        out["prefill"] = {"M": Mp, "K": Kp, "N": Np, "median_us": pc["median_us"],
                          "p10_us": pc["p10_us"], "p90_us": pc["p90_us"],
                          "back_to_back_mean_us": round(pg * 1e3, 2),
                          "tops": round(tops, 1), "peak_tops": INT8_PEAK_TOPS,
                          "frac": round(tops / INT8_PEAK_TOPS, 4), "bound": "mfma",
                          "frac_of_measured_mfma_workload": round(
                              tops / peaks["mfma_i8_tops_workload"], 4),
                          "frac_of_measured_mfma_uniform": round(
                              tops / peaks["mfma_i8_tops_uniform"], 4),
                          "frac_of_measured_mfma_epilogue": round(
                              tops / peaks["mfma_i8_epilogue_tops_workload"], 4),
                          "kernel": "gemm_big_kernel<0, false, false> (256x256)",
                          "sclk": clk,
                          "counters": counter_summary("gemm_big_kernel<0, false, false> [grid 262144]"),
                          "traffic": measured_traffic("gemm_prefill")}
        if out["prefill"]["counters"]:
            out["prefill"]["mfma_util"] = out["prefill"]["counters"].get("mfma_util")
        out["measured_peaks"] = peaks
        # against the read probe at the same size (its weights' 232 MiB), and at 2 GiB
        out["roofline"]["frac_of_measured_hbm"] = round(achieved / peaks["hbm_read_gbs_232mib"], 4)
        out["roofline"]["frac_of_measured_hbm_2gib"] = round(achieved / peaks["hbm_read_gbs"], 4)
        del pre
        torch.cuda.empty_cache()

    if not args.no_rows:
        out["rows"] = extra_rows(torch, L, stream, dev, max(10, min(50, args.steps // 4)))
        # the committed counter runs of these rows' kernels (null once the sources change)
        for key, ck, tk in (
                ("moe_4096tok_top8_64e_grouped", None, "moe_grouped"),
                ("moe_4096tok_top8_64e_grouped_gather", "gemm_big_kernel<0, true, true> [grid 786432]",
                 "moe_grouped_gather"),
                ("w8a16_prefill_4096x8192x8192", "gemm_a16_kernel<0, 1> [grid 1048576]",
                 "w8a16_prefill"),
                ("bf16_prefill_4096x8192x8192", "gemm_a16_kernel<0, 2> [grid 1048576]",
                 "bf16_prefill"),
                ("blockfmt_gemm_m1024_4096x7168", "gemm_mid_kernel<0, false, false> [grid 131072]",
                 "gemm_mid_m1024"),
                ("blockfmt_decode_fp8_ocp_4096x7168", None, "decode_fp8"),
                ("blockfmt_decode_fp8_ocp_16384x7168", None, "decode_fp8_layer"),
                ("blockfmt_decode_mxfp4_8x2048x4096", None, "decode_mxfp4")):
            r = out["rows"].get(key)
            if r is None:
                continue
            if ck:
                cs = counter_summary(ck)
                r["counters"] = cs
                r["mfma_util"] = cs.get("mfma_util") if cs else None
            r["traffic"] = measured_traffic(tk)
        peaks = out.get("measured_peaks")
        if peaks:
            # streams against what this part sustains for the same kind of stream:
            # the decoders read and write (the copy probe), attention reads
            for k, r in out["rows"].items():
                if k.startswith("blockfmt_decode") or k.startswith("blockfmt_dequant"):
                    r["frac_of_measured_copy"] = round(r["gbs"] / peaks["copy_gbs"], 4)
                elif k.startswith("kv_") and "attention" in k:
                    r["frac_of_measured_hbm"] = round(r["gbs"] / peaks["hbm_read_gbs"], 4)

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
