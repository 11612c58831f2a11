#!/usr/bin/env python3
"""Benchmark of the single-GPU MoE layer on MI355X.

A step is one pass of the whole hot path over one batch of synthetic input:
one moe_layer call (route -> index permute -> GEMM 1 gathering the token
rows, ReLU -> GEMM 2 -> weighted combine) on torch's current stream. Inputs
are resident in HBM before the timed region. The same path run stage by
stage through the separate entry points, with HIP events between them, gives
per-kernel durations; the dominant kernel (moe_gmm) is reported against its
roofline. The fp8 workloads time the page-2 step instead: E4M3 grouped GEMM
(per-tensor or MX block scales) + Unpermute, with the shared bf16 expert on
a second stream (fp8dyn: gmmX quantised per row on the device first).

Prints ONE JSON line. Default workload: prefill (T=4096, H=4096, E=8, K=2,
F=14336, bf16). Other workloads: --workload skewed|decode16|decode64|
decode256|fp8gmm|fp8gmm_one|fp8mx|fp8mx_one|fp8dyn|fp4mx|fp4mx_one|prefill_fp8|tiny.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0
PEAK_FP8_TFLOPS = 5000.0
PEAK_FP4_TFLOPS = 10100.0  # dense E2M1 MFMA
PEAK_HBM_GBS = 8000.0
METRIC = "MoE layer tokens/s; moe_gmm TFLOP/s and % of MFMA/HBM peak (1 GPU)"

LAYER_WORKLOADS = {
    # name: (recipe, T)
    "prefill": ("prefill", 4096),
    "skewed": ("skewed", 16384),
    "decode16": ("decode", 16),
    "decode64": ("decode", 64),
    "decode256": ("decode", 256),
    "tiny": ("tiny", 64),
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed warm-up steps (default: as many as fill 0.4 s, so the GPU's "
                         "clocks have left their idle state; the count is reported)")
    ap.add_argument("--workload", default="prefill",
                    choices=sorted(LAYER_WORKLOADS) + ["fp8gmm", "fp8gmm_one", "fp8mx", "fp8mx_one", "fp8dyn",
                                                       "fp4mx", "fp4mx_one", "prefill_fp8"])
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle baseline sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of known size (for counter calibration)")
    return ap.parse_args()


GMM_SRC = [os.path.join(ROOT, "mixture_experts_layer_06_amd", "csrc", f) for f in ("gmm.hip", "common.h")]


def source_digest(paths=GMM_SRC) -> str:
    """Digest of the grouped GEMM's sources (its kernel file and the helpers
    it includes): counter summaries taken on other sources are not used."""
    import hashlib
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per moe_gmm launch from the committed counter summary
    (FETCH_SIZE + WRITE_SIZE, copy-calibrated), or None when the summary is
    missing or was taken on a different gmm.hip."""
    path = os.path.join(ROOT, "profiles", f"moe_gmm_{workload}_counters.md")
    if not os.path.exists(path):
        return None
    for line in open(path):
        if line.startswith("machine: "):
            rec = json.loads(line[len("machine: "):])
            if rec.get("gmm_source") == source_digest():
                return rec.get("traffic_bytes_per_launch")
    return None


def copy_calibration():
    """A plain copy kernel of known size: 1 GiB read + 1 GiB written per launch."""
    import torch
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 3}), flush=True)


def warm_up(fn, count):
    """Run fn `count` times, or (count None) until 0.4 s have passed; return the count."""
    import torch
    if count is not None:
        for _ in range(count):
            fn()
        torch.cuda.synchronize()
        return count
    n, t0 = 0, time.perf_counter()
    while True:
        fn()
        n += 1
        if n % 4 == 0:
            torch.cuda.synchronize()
            if time.perf_counter() - t0 >= 0.4:
                return n


FLUSH_BYTES = 1 << 30  # read before every timed step: evicts the 256 MB MALL and the L2s


class Flush:
    """A 1 GiB device buffer read (a sum over it) before each timed step,
    outside the step's events, so every step starts from cold caches: the
    read evicts the 256 MB MALL and the L2s without leaving dirty lines
    behind, whose write-back a written buffer would charge to the step's
    first kernel."""

    def __init__(self, dev):
        import torch
        self.buf = torch.ones(FLUSH_BYTES // 8, dtype=torch.int64, device=dev)
        self.sink = torch.empty((), dtype=torch.int64, device=dev)

    def __call__(self):
        import torch
        torch.sum(self.buf, dim=0, out=self.sink)


def pp_kernel_names(H, F):
    """The bf16 ping-pong kernels GEMM 1 (K = H) and GEMM 2 (K = F) run on:
    the persistent form for tiles of at most 64 K slices of 32 values."""
    names = []
    for k in (H, F):
        n = "gmm_ppd_kernel" if (k + 31) // 32 <= 64 else "gmm_pp_kernel"
        if n not in names:
            names.append(n)
    return " / ".join(names)


def median_min(values):
    import numpy as np
    v = np.asarray(values, np.float64)
    return float(np.median(v)), float(v.min())


def _time_ms(fn, iters):
    import torch
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / iters


def reported_sclk():
    """The shader clock level the driver marks as current in sysfs right now
    (informational), or None. Read from a file: no child process."""
    import glob
    for path in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            lines = open(path).read().splitlines()
        except OSError:
            continue
        for line in lines:
            if line.rstrip().endswith("*"):
                return line.split(":", 1)[-1].strip(" *")
    return None


def cu_read_rate(dev, mfma=None):
    """What one CU reads per second (moe_fetch_probe: one block of 8 waves per
    CU, 8 KB in flight per wave; timed with HIP events, since the probe's own
    s_memtime ticks do not run at a fixed rate), from a 2 MiB window every CU
    shares (stays in L2) and from a private 1/ncu slice of 1 GiB each (HBM);
    LDS DMA as the GEMM kernels fetch, and plain vector loads. A 256 x 256
    ping-pong GEMM tile reads 32 KB per 4.19 MFLOP (bf16); at the MFMA-only
    rate of one CU (mfma) that is the read rate it needs, and the DMA rate
    from L2 over it is the share of that MFMA rate the reads alone allow."""
    import torch
    import mixture_experts_layer_06_amd as moe
    out = {"unit": "GB/s per CU (mean over the launch)"}
    ncu = torch.cuda.get_device_properties(dev).multi_processor_count
    cycles = torch.zeros((ncu,), dtype=torch.int64, device=dev)
    for name, nbytes, shared, kb in (("l2_2MiB", 2 << 20, True, 4096), ("hbm_1GiB", 1 << 30, False, 2048)):
        buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        for mode, mname in ((0, "lds_dma"), (1, "vector")):
            moe.fetch_probe(buf, mode, shared, 64, cycles=cycles)  # warm
            best = None
            for _ in range(3):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                _, per_cu = moe.fetch_probe(buf, mode, shared, kb, cycles=cycles)
                e1.record()
                torch.cuda.synchronize()
                r = per_cu / (e0.elapsed_time(e1) * 1e-3) / 1e9
                best = r if best is None or r > best else best
            out[f"{name}_{mname}"] = best
        del buf
    if mfma is not None:
        ncu = torch.cuda.get_device_properties(dev).multi_processor_count
        per_cu_flops = mfma["bf16"]["TFLOP/s"] * 1e12 / ncu
        need = 32768.0 / (256 * 256 * 32 * 2) * per_cu_flops / 1e9
        out["bf16_tile_need_at_mfma_only_rate"] = need
        out["mfma_bound_256x256_tile"] = min(1.0, out["l2_2MiB_lds_dma"] / need)
    return out


def mfma_only(dev):
    """MFMA rate without memory traffic (moe_mfma_probe, every CU, 8 waves,
    long enough that the launch gap does not count), by HIP events; and the
    shader clock that rate implies at the MFMA issue peak (bf16 4096, E4M3
    8192 flops per clock per CU)."""
    import torch
    import mixture_experts_layer_06_amd as moe
    out = {}
    ncu = torch.cuda.get_device_properties(dev).multi_processor_count
    cycles = torch.zeros((ncu,), dtype=torch.int64, device=dev)
    sink = torch.empty((ncu * 512,), dtype=torch.float32, device=dev)
    for name, fp8, iters, per_clk in (("bf16", False, 16384, 4096.0), ("fp8_e4m3", True, 8192, 8192.0)):
        moe.mfma_probe(fp8, 64, device=dev, cycles=cycles, sink=sink)  # warm
        best = None
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            _, fl = moe.mfma_probe(fp8, iters, device=dev, cycles=cycles, sink=sink)
            e1.record()
            torch.cuda.synchronize()
            tf = fl * ncu / (e0.elapsed_time(e1) * 1e-3) / 1e12
            best = tf if best is None or tf > best else best
        out[name] = {"TFLOP/s": best, "implied_clock_GHz_at_full_issue": best * 1e12 / ncu / per_clk / 1e9}
    return out


def achievable(dev, even_experts=None):
    """What the GPU sustains on plain work of the same kind, outside the timed
    region, on random data (informational, beside the published peaks): a
    1 GiB device copy (read + write bytes), one dense bf16 GEMM of the prefill
    GEMM 1 shape through the vendor BLAS (hipBLASLt), the read rate of one CU
    (cu_read_rate), the MFMA rate without memory traffic (mfma_only), and
    optionally the vendor's batched GEMM on even expert loads of the given
    shapes."""
    import torch
    res = {"sclk_reported_after_run": reported_sclk()}
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    ms = _time_ms(lambda: dst.copy_(src), 10)
    res["hbm_copy_GBps"] = 2 * n / (ms * 1e-3) / 1e9
    del src, dst
    g = torch.Generator(device=dev)
    g.manual_seed(5)
    a = torch.randn(8192, 4096, device=dev, generator=g).to(torch.bfloat16)
    b = (torch.randn(4096, 14336, device=dev, generator=g) * 4096 ** -0.5).to(torch.bfloat16)
    ms = _time_ms(lambda: torch.matmul(a, b), 10)
    res["vendor_dense_bf16_gemm_8192x4096x14336_TFLOPs"] = 2.0 * 8192 * 4096 * 14336 / (ms * 1e-3) / 1e12
    del a, b
    res["mfma_only"] = mfma_only(dev)
    res["cu_read_rate"] = cu_read_rate(dev, res["mfma_only"])
    if even_experts is not None:
        E, M, shapes = even_experts
        for name, (Hin, N) in shapes.items():
            a = torch.randn(E, M, Hin, device=dev, generator=g).to(torch.bfloat16)
            b = (torch.randn(E, Hin, N, device=dev, generator=g) * Hin ** -0.5).to(torch.bfloat16)
            ms = _time_ms(lambda: torch.bmm(a, b), 10)
            res[f"vendor_bmm_bf16_{name}_{E}x{M}x{Hin}x{N}_TFLOPs"] = 2.0 * E * M * Hin * N / (ms * 1e-3) / 1e12
            del a, b
    return res


def cpu_share():
    """(CPUs this process may run on, CPUs its cgroup quota grants or None)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    quota = None
    try:
        q, period = open("/sys/fs/cgroup/cpu.max").read().split()[:2]
        if q != "max":
            quota = max(1, int(math.ceil(int(q) / int(period))))
    except (OSError, ValueError):
        pass
    return n, quota


def cpu_threads() -> int:
    """Oracle threads: every CPU granted to this process, at most 16 (the
    host CPU share that goes with one GPU on the measurement boxes)."""
    n, quota = cpu_share()
    if quota is not None:
        n = min(n, quota)
    return max(1, min(16, n))


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_info(nth):
    n, quota = cpu_share()
    return {"cores": nth, "cpu_model": cpu_model(), "cpus_visible": n, "cgroup_cpu_quota": quota}


def host_to_dev(a, dev):
    import numpy as np
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(a).to(dev)


def flops_bytes_gmm(counts, Hin, N, elem):
    """Algorithmic work of one grouped-GEMM launch: 2*A*Hin*N flops; bytes =
    weights of experts that received rows + activations in + outputs out."""
    A = int(sum(counts))
    used = sum(1 for c in counts if c > 0)
    fl = 2.0 * A * Hin * N
    by = used * Hin * N * elem + A * Hin * elem + A * N * 2
    return fl, by


def bench_layer(args, dev):
    import numpy as np
    import torch

    import mixture_experts_layer_06_amd as moe
    from synth import configs

    recipe, T = LAYER_WORKLOADS[args.workload]
    d = configs.layer_inputs(recipe, T=T)
    H, E, K, F, dt = d["H"], d["E"], d["K"], d["F"], d["dtype"]
    es = 4 if dt == "f32" else 2
    A = T * K
    x = host_to_dev(d["x"], dev)
    wr = host_to_dev(d["wr"], dev)
    w1 = host_to_dev(d["w1"], dev)
    w2 = host_to_dev(d["w2"], dev)
    bias = host_to_dev(d["bias"], dev) if d["bias"] is not None else None
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    idx = torch.empty((T, K), dtype=torch.int32, device=dev)
    gate = torch.empty((T, K), dtype=torch.float32, device=dev)
    bufs = {"counts": torch.empty((E,), dtype=torch.int32, device=dev),
            "offsets": torch.empty((E + 1,), dtype=torch.int32, device=dev),
            "perm_src": torch.empty((A,), dtype=torch.int32, device=dev),
            "perm_dst": torch.empty((A,), dtype=torch.int32, device=dev)}
    hm = torch.empty((A, F), dtype=tdt, device=dev)
    yp = torch.empty((A, H), dtype=tdt, device=dev)
    y = torch.empty((T, H), dtype=tdt, device=dev)
    pws_n = moe.permute_workspace_size(T, E, K)
    pws = torch.empty((max(pws_n, 16),), dtype=torch.uint8, device=dev)
    rws_n = moe.route_workspace_size(T, H, E, K, moe.dtype_code(x))
    rws = torch.empty((max(rws_n, 16),), dtype=torch.uint8, device=dev)
    gws_n = max(moe.gmm_workspace_size(moe.dtype_code(x), E, A, H, F),
                moe.gmm_workspace_size(moe.dtype_code(x), E, A, F, H))
    gws = torch.empty((max(gws_n, 16),), dtype=torch.uint8, device=dev)  # shared: one stream

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        moe.route(x, wr, K, bias=bias, topk_idx=idx, topk_gate=gate, ws=rws)
        if ev is not None:
            ev[1].record()
        moe.permute(idx, E, ws=pws, out=bufs)  # indices only: GEMM 1 gathers the token rows
        if ev is not None:
            ev[2].record()
        moe.gmm(x, w1, bufs["offsets"], act=moe.ACT_RELU, out=hm, ws=gws, rows=bufs["perm_src"],
                row_div=K)
        if ev is not None:
            ev[3].record()
        moe.gmm(hm, w2, bufs["offsets"], out=yp, ws=gws)
        if ev is not None:
            ev[4].record()
        moe.combine(yp, bufs["perm_dst"], gate, T, K, out=y)
        if ev is not None:
            ev[5].record()

    # The timed step is one moe_layer call (route, index permute, GEMM 1 gathering
    # the token rows, GEMM 2, weighted combine: the whole path on one stream).
    ws_layer = torch.empty((moe.layer_workspace_size(T, H, E, K, F, moe.dtype_code(x)),),
                           dtype=torch.uint8, device=dev)
    y2 = torch.empty_like(y)

    def layer_step():
        moe.layer(x, wr, w1, w2, K, bias=bias, y=y2, ws=ws_layer)

    def warm_step():
        layer_step()
        step()

    flush = Flush(dev)
    warmup = warm_up(warm_step, args.warmup)
    sclk_start = reported_sclk()
    # Timed: every step after a 1 GiB read (outside its events), between two
    # events on the stream; median and min over the steps.
    lev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        flush()
        lev[s][0].record()
        layer_step()
        lev[s][1].record()
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - t0
    ms_step, ms_min = median_min([e[0].elapsed_time(e[1]) for e in lev])
    # The same steps back to back, no flush (informational).
    t0 = time.perf_counter()
    for _ in range(args.steps):
        layer_step()
    torch.cuda.synchronize()
    ms_b2b = (time.perf_counter() - t0) * 1e3 / args.steps

    # The same path stage by stage through the separate entry points, with HIP
    # events on the stream between them, each step after a flush: per-kernel
    # times (the grouped GEMM's launch time feeds the roofline).
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for s in range(args.steps):
        flush()
        step(evs[s])
    torch.cuda.synchronize()
    names = ["route", "permute", "gmm1", "gmm2", "combine"]
    per = {n: median_min([evs[s][i].elapsed_time(evs[s][i + 1]) for s in range(args.steps)])[0]
           for i, n in enumerate(names)}
    ms_stages = sum(per.values())

    counts = bufs["counts"].cpu().numpy().tolist()
    fl1, by1 = flops_bytes_gmm(counts, H, F, es)
    fl2, by2 = flops_bytes_gmm(counts, F, H, es)
    gmm_ms = (per["gmm1"] + per["gmm2"]) / 2.0  # one kernel, two launches of equal work
    fl_launch, by_launch = (fl1 + fl2) / 2.0, (by1 + by2) / 2.0
    hbm_bound = (fl_launch / by_launch) < (PEAK_BF16_TFLOPS / PEAK_HBM_GBS) * 1e3
    if hbm_bound:
        achieved = by_launch / (gmm_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS, "traffic": measured_traffic(args.workload)}
    else:
        achieved = fl_launch / (gmm_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / PEAK_BF16_TFLOPS, "traffic": measured_traffic(args.workload)}
    bytes_stage = {
        "route": T * H * es + H * E * es + T * K * 8,
        "permute": T * K * 4 * 3,
        "combine": A * H * es + T * H * es + T * K * 8,
    }
    kernels = {n: {"ms": per[n]} for n in names}
    for n, b in bytes_stage.items():
        kernels[n]["GB/s"] = b / (per[n] * 1e-3) / 1e9
    for n, fl, by in (("gmm1", fl1, by1), ("gmm2", fl2, by2)):
        kernels[n]["TFLOP/s"] = fl / (per[n] * 1e-3) / 1e12
        kernels[n]["GB/s"] = by / (per[n] * 1e-3) / 1e9
    gmm_tflops = (fl1 + fl2) / ((per["gmm1"] + per["gmm2"]) * 1e-3) / 1e12
    workload = (f"{args.workload}: T={T} H={H} E={E} K={K} F={F} ReLU {dt}"
                + (" router bias -1.2ln(e+1)" if bias is not None else ""))
    res = {
        "metric": METRIC, "value": T / (ms_step * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dt,
        "data": "synthetic (seeded N(0,1/fan_in) weights, N(0,1) tokens)",
        "timing": timing_record(ms_step, ms_min, ms_b2b, wall_s, args.steps, sclk_start),
        "config": {"workload": workload, "T": T, "H": H, "E": E, "K": K, "F": F,
                   "tokens_per_step": T, "parallelism": "single GPU"},
        "roofline": dict(roof, kernel="moe_gmm (" + ("gmm_f32_kernel" if dt == "f32" else "gmm_stream_kernel"
                                                    if hbm_bound else pp_kernel_names(H, F)) + ")",
                         gmm_source=source_digest(),
                         launches_per_step=2, flops_per_launch=fl_launch,
                         bytes_per_launch=by_launch, avg_launch_ms=gmm_ms),
        "moe_gmm_tflops": gmm_tflops,
        "moe_gmm_frac_bf16_peak": gmm_tflops / PEAK_BF16_TFLOPS if dt != "f32" else None,
        "kernels": kernels,
        "ms_per_step_stage_by_stage": ms_stages,
        "expert_counts": {"min": min(counts), "max": max(counts), "empty": counts.count(0)},
    }
    host = {"x": d["x"], "wr": d["wr"], "w1": d["w1"], "w2": d["w2"], "bias": d["bias"], "K": K}
    return res, host


def bench_fp8(args, dev, mode="pt"):
    """Page-2 form: fp8 grouped GEMM + Unpermute, with the bf16 shared-expert
    GEMM on a second stream, joined by events. mode "pt": per-tensor scales,
    the Unpermute fused into the GEMM's stores; "mx": E8M0 block scales, then
    the Unpermute kernel; "dyn": gmmX arrives in bf16 and is quantised per row
    on the device (per-token dynamic), then the per-token-scaled GEMM with the
    fused Unpermute; "one": as "pt", with the routed and the shared GEMM in
    one launch (moe_gmm_routed_shared) instead of two streams; "mx_one" and
    "mx4_one": as "mx" and "mx4", with moe_gmm_mx_routed_shared."""
    import numpy as np
    import torch

    import mixture_experts_layer_06_amd as moe
    import synth
    from synth import configs

    one = mode in ("one", "mx_one", "mx4_one")
    fp4 = mode in ("mx4", "mx4_one")
    use_mx, dyn = mode in ("mx", "mx4", "mx_one", "mx4_one"), mode == "dyn"
    d = (configs.fp4_mx_inputs() if fp4 else configs.fp8_mx_inputs() if use_mx else
         configs.fp8_dyn_inputs() if dyn else configs.fp8_inputs())
    T, e, K, A, H1, N1, H2, N2 = (d[k] for k in ("T", "e", "K", "A", "H1", "N1", "H2", "N2"))
    # dispatch layout of the routed rows: computed once on the device by moe_permute
    idx = host_to_dev(d["topk_idx"], dev)
    perm = moe.permute(idx, e)
    gx = host_to_dev(d["gmm_x"], dev)
    gw = host_to_dev(d["gmm_w"], dev)
    if use_mx:
        sx = host_to_dev(synth.mx_scales_slice_major(d["gmm_x_scale"], 8 if fp4 else 4), dev)
        sw = host_to_dev(synth.mx_weight_scales_interleaved(d["gmm_w_scale"]), dev)
    elif dyn:
        qx = torch.empty((A, H1), dtype=torch.float8_e4m3fn, device=dev)
        sx = torch.empty((A,), dtype=torch.float32, device=dev)
        sw = torch.tensor([float(d["gmm_w_scale"])], dtype=torch.float32, device=dev)
    else:
        sx = torch.tensor([float(d["gmm_x_scale"])], dtype=torch.float32, device=dev)
        sw = torch.tensor([float(d["gmm_w_scale"])], dtype=torch.float32, device=dev)
    mx = host_to_dev(d["mm_x"], dev)
    mw = host_to_dev(d["mm_w"], dev).view(1, H2, N2)
    host = {"d": d, "mode": "mx4" if fp4 else "mx" if use_mx else "dyn" if dyn else "pt"}
    moff = torch.tensor([0, T], dtype=torch.int32, device=dev)
    gy = torch.empty((A, N1), dtype=torch.bfloat16, device=dev)
    un = torch.empty((A, N1), dtype=torch.bfloat16, device=dev)
    my = torch.empty((T, N2), dtype=torch.bfloat16, device=dev)
    side = torch.cuda.Stream(device=dev)
    sws_n = moe.gmm_workspace_size(moe.BF16, 1, T, H2, N2)   # shared expert, on the side stream
    sws = torch.empty((max(sws_n, 16),), dtype=torch.uint8, device=dev)
    gws_n = moe.gmm_workspace_size(moe.FP8_E4M3, e, A, H1, N1)
    gws = torch.empty((max(gws_n, 16),), dtype=torch.uint8, device=dev)

    # events: 0 start, 5 after the quantisation (dyn), 1 after the GEMM, 2 after
    # the Unpermute (mx), 3/4 around the shared expert on the side stream
    def step_one(ev=None):
        if ev is not None:
            ev[0].record()
            ev[5].record()
        if use_mx:
            moe.gmm_mx_routed_shared(gx, sx, gw, sw, perm["offsets"], mx, mw, moff, fp4=fp4, out=gy, ys=my)
        else:
            moe.gmm_routed_shared(gx, gw, perm["offsets"], sx, sw, mx, mw, moff, dst=perm["perm_src"], out=un,
                                  ys=my)
        if ev is not None:
            ev[1].record()
        if use_mx:
            moe.combine(gy, perm["perm_dst"], None, T, K, out=un)
        if ev is not None:
            ev[2].record()
            ev[6].record()

    def step(ev=None):
        main = torch.cuda.current_stream()
        fork = torch.cuda.Event()
        fork.record(main)
        side.wait_event(fork)
        if ev is not None:
            ev[0].record(main)
        with torch.cuda.stream(side):
            if ev is not None:
                ev[3].record(side)
            moe.gmm(mx, mw, moff, out=my, ws=sws, stream=side)
            if ev is not None:
                ev[4].record(side)
        if use_mx:
            if ev is not None:
                ev[5].record(main)
            if fp4:
                moe.gmm_mxfp4(gx, sx, gw, sw, perm["offsets"], out=gy)
            else:
                moe.gmm_mx(gx, sx, gw, sw, perm["offsets"], out=gy)
            if ev is not None:
                ev[1].record(main)
            moe.combine(gy, perm["perm_dst"], None, T, K, out=un)
        else:
            a, asc = gx, sx
            if dyn:
                moe.quant_rows(gx, q=qx, scale=sx)
                a = qx
            if ev is not None:
                ev[5].record(main)
            # Unpermute fused into the GEMM's stores: grouped row r lands in row perm_src[r]
            moe.gmm(a, gw, perm["offsets"], a_scale=asc, w_scale=sw, out=un, ws=gws, dst=perm["perm_src"],
                    per_token=dyn)
            if ev is not None:
                ev[1].record(main)
        if ev is not None:
            ev[2].record(main)
        join = torch.cuda.Event()
        join.record(side)
        main.wait_event(join)
        if ev is not None:
            ev[6].record(main)  # both streams joined: the step's end

    if one:
        step = step_one
    flush = Flush(dev)
    warmup = warm_up(step, args.warmup)
    sclk_start = reported_sclk()
    # Timed: every step after a 1 GiB read (outside its events); the step
    # runs from its first launch on either stream to the join of both.
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        flush()
        step(evs[s])
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - t0
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_b2b = (time.perf_counter() - t0) * 1e3 / args.steps

    # The routed grouped GEMM launched alone (no shared GEMM beside it), each
    # launch after a flush: its own rate, which the in-step time (shared with
    # the side stream's GEMM) understates.
    alone_ms = None
    if not one:
        def routed():
            if use_mx:
                if fp4:
                    moe.gmm_mxfp4(gx, sx, gw, sw, perm["offsets"], out=gy)
                else:
                    moe.gmm_mx(gx, sx, gw, sw, perm["offsets"], out=gy)
            else:
                moe.gmm(qx if dyn else gx, gw, perm["offsets"], a_scale=sx, w_scale=sw, out=un, ws=gws,
                        dst=perm["perm_src"], per_token=dyn)
        lev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        for s in range(args.steps):
            flush()
            lev[s][0].record()
            routed()
            lev[s][1].record()
        torch.cuda.synchronize()
        alone_ms = median_min([e0.elapsed_time(e1) for e0, e1 in lev])[0]

    def span(i, j):
        return median_min([evs[s][i].elapsed_time(evs[s][j]) for s in range(args.steps)])

    ms_step, ms_min = span(0, 6)
    q_ms, gmm_ms, un_ms = span(0, 5)[0], span(5, 1)[0], span(1, 2)[0]
    sh_ms = None if one else span(3, 4)[0]
    counts = perm["counts"].cpu().numpy().tolist()
    fl, by = flops_bytes_gmm(counts, H1, N1, 1)
    if fp4:  # half a byte per activation and weight element
        by -= (A * H1 + sum(1 for c in counts if c > 0) * H1 * N1) // 2
    if use_mx:  # E8M0 scales: one byte per 32 activation and weight elements
        by += A * (H1 // 32) + sum(1 for c in counts if c > 0) * (H1 // 32) * N1
    if dyn:  # one fp32 scale per activation row
        by += A * 4
    peak = PEAK_FP4_TFLOPS if fp4 else PEAK_FP8_TFLOPS
    if one:  # the launch also runs the bf16 shared GEMM: its flops, at the bf16 peak
        fl_s = 2.0 * T * H2 * N2
        by += 2 * (T * H2 + H2 * N2 + T * N2)
        peak = (fl + fl_s) / (fl / (peak * 1e12) + fl_s / (PEAK_BF16_TFLOPS * 1e12)) / 1e12
        fl += fl_s
    achieved = fl / (gmm_ms * 1e-3) / 1e12
    wl = {"pt": "fp8gmm", "one": "fp8gmm_one", "mx": "fp8mx", "mx_one": "fp8mx_one", "dyn": "fp8dyn",
          "mx4": "fp4mx", "mx4_one": "fp4mx_one"}[mode]
    data = {"pt": "synthetic (seeded; E4M3 per-tensor scales amax/448; random top-8 of 32 routing)",
            "one": "synthetic (seeded; E4M3 per-tensor scales amax/448; random top-8 of 32 routing)",
            "mx": "synthetic (seeded; E4M3 with MX E8M0 scales per 32 elements, OCP recipe; "
                  "random top-8 of 32 routing)",
            "dyn": "synthetic (seeded; bf16 gmmX quantised per row on the device, E4M3 weights with a "
                   "per-tensor scale; random top-8 of 32 routing)",
            "mx4": "synthetic (seeded; E2M1 with MX E8M0 scales per 32 elements, OCP recipe; "
                   "random top-8 of 32 routing)"}[mode.replace("_one", "") if mode != "one" else mode]
    kernel = {"pt": "moe_gmm_scatter E4M3 (gmm_pp8w_kernel, Unpermute fused into its stores)",
              "one": "moe_gmm_routed_shared (gmm_pair_kernel: E4M3 routed tiles, Unpermute fused into their "
                     "stores, and bf16 shared-expert tiles in one launch)",
              "mx": "moe_gmm_mx E4M3 + E8M0 (gmm_pp8_kernel<true>)",
              "dyn": "moe_gmm_scatter E4M3, per-token scales (gmm_pp8w_kernel, Unpermute fused)",
              "mx4": "moe_gmm_mxfp4 E2M1 + E8M0 (gmm_pp8_kernel<true, true>)",
              "mx_one": "moe_gmm_mx_routed_shared E4M3 + E8M0 (gmm_pair_kernel<.., true, false>: MX routed "
                        "tiles and bf16 shared-expert tiles in one launch)",
              "mx4_one": "moe_gmm_mx_routed_shared E2M1 + E8M0 (gmm_pair_kernel<.., true, true>: MX routed "
                         "tiles and bf16 shared-expert tiles in one launch)"}[mode]
    kernels = {"gmm_fp8": {"ms": gmm_ms, "TFLOP/s": achieved},
               "unpermute": ({"ms": un_ms, "GB/s": 2 * A * N1 * 2 / (un_ms * 1e-3) / 1e9} if use_mx
                             else "fused into the grouped GEMM's stores"),
               "shared_gemm_bf16": ({"ms": sh_ms, "TFLOP/s": 2.0 * T * H2 * N2 / (sh_ms * 1e-3) / 1e12}
                                    if sh_ms is not None else "in the same launch")}
    if dyn:  # bf16 rows read once, codes and scales written
        kernels["quant_rows"] = {"ms": q_ms, "GB/s": (A * H1 * 3 + A * 4) / (q_ms * 1e-3) / 1e9}
    res = {
        "metric": METRIC, "value": T / (ms_step * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp4_e2m1" if fp4 else "fp8_e4m3", "data": data,
        "timing": timing_record(ms_step, ms_min, ms_b2b, wall_s, args.steps, sclk_start),
        "config": {"workload": f"{wl}: T={T} e={e} K={K} A={A} H1={H1} N1={N1} + shared "
                               f"({T},{H2})x({H2},{N2}) bf16", "tokens_per_step": T},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": peak,
                     "unit": "TFLOP/s", "frac": achieved / peak,
                     "traffic": measured_traffic(wl), "kernel": kernel, "gmm_source": source_digest(),
                     "flops_per_launch": fl, "bytes_per_launch": by, "avg_launch_ms": gmm_ms},
        "kernels": kernels,
    }
    if alone_ms is not None:
        res["roofline"]["launch_alone"] = {"ms": alone_ms, "TFLOP/s": fl / (alone_ms * 1e-3) / 1e12,
                                           "frac": fl / (alone_ms * 1e-3) / 1e12 / peak}
    return res, host


def bench_layer_fp8(args, dev):
    """The E4M3 layer on the prefill shapes: one moe_layer_fp8 call per step
    (route, index permute, per-token quantisation of the tokens, GEMM 1
    gathering the quantised tokens, per-row quantisation of the hidden rows,
    GEMM 2, weighted combine); the same path stage by stage for per-kernel times."""
    import numpy as np
    import torch

    import mixture_experts_layer_06_amd as moe
    from synth import configs

    d = configs.layer_fp8_inputs("prefill")
    T, H, E, K, F = d["T"], d["H"], d["E"], d["K"], d["F"]
    A = T * K
    x, wr = host_to_dev(d["x"], dev), host_to_dev(d["wr"], dev)
    w1, w2 = host_to_dev(d["w1"], dev), host_to_dev(d["w2"], dev)
    s1 = torch.tensor([float(d["w1_scale"])], dtype=torch.float32, device=dev)
    s2 = torch.tensor([float(d["w2_scale"])], dtype=torch.float32, device=dev)
    ws = torch.empty((moe.layer_fp8_workspace_size(T, H, E, K, F),), dtype=torch.uint8, device=dev)
    y = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    idx = torch.empty((T, K), dtype=torch.int32, device=dev)
    gate = torch.empty((T, K), dtype=torch.float32, device=dev)
    bufs = {"counts": torch.empty((E,), dtype=torch.int32, device=dev),
            "offsets": torch.empty((E + 1,), dtype=torch.int32, device=dev),
            "perm_src": torch.empty((A,), dtype=torch.int32, device=dev),
            "perm_dst": torch.empty((A,), dtype=torch.int32, device=dev)}
    xq = torch.empty((T, H), dtype=torch.float8_e4m3fn, device=dev)
    xs = torch.empty((T,), dtype=torch.float32, device=dev)
    hm = torch.empty((A, F), dtype=torch.bfloat16, device=dev)
    hq = torch.empty((A, F), dtype=torch.float8_e4m3fn, device=dev)
    hs = torch.empty((A,), dtype=torch.float32, device=dev)
    yp = torch.empty((A, H), dtype=torch.bfloat16, device=dev)
    y2 = torch.empty_like(y)
    pws = torch.empty((max(moe.permute_workspace_size(T, E, K), 16),), dtype=torch.uint8, device=dev)
    rws = torch.empty((max(moe.route_workspace_size(T, H, E, K, moe.BF16), 16),), dtype=torch.uint8, device=dev)
    gws = torch.empty((max(moe.gmm_workspace_size(moe.FP8_E4M3, E, A, H, F),
                           moe.gmm_workspace_size(moe.FP8_E4M3, E, A, F, H), 16),), dtype=torch.uint8, device=dev)

    def layer_step():
        moe.layer_fp8(x, wr, w1, s1, w2, s2, K, y=y, ws=ws)

    names = ["route", "permute", "quant_x", "gmm1", "quant_h", "gmm2", "combine"]

    def step(ev):
        ev[0].record()
        moe.route(x, wr, K, topk_idx=idx, topk_gate=gate, ws=rws)
        ev[1].record()
        moe.permute(idx, E, ws=pws, out=bufs)
        ev[2].record()
        moe.quant_rows(x, q=xq, scale=xs)
        ev[3].record()
        moe.gmm(xq, w1, bufs["offsets"], act=moe.ACT_RELU, a_scale=xs, per_token=True, w_scale=s1, out=hm,
                ws=gws, rows=bufs["perm_src"], row_div=K)
        ev[4].record()
        moe.quant_rows(hm, q=hq, scale=hs)
        ev[5].record()
        moe.gmm(hq, w2, bufs["offsets"], a_scale=hs, per_token=True, w_scale=s2, out=yp, ws=gws)
        ev[6].record()
        moe.combine(yp, bufs["perm_dst"], gate, T, K, out=y2)
        ev[7].record()

    flush = Flush(dev)
    warmup = warm_up(layer_step, args.warmup)
    sclk_start = reported_sclk()
    lev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        flush()
        lev[s][0].record()
        layer_step()
        lev[s][1].record()
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - t0
    ms_step, ms_min = median_min([e[0].elapsed_time(e[1]) for e in lev])
    t0 = time.perf_counter()
    for _ in range(args.steps):
        layer_step()
    torch.cuda.synchronize()
    ms_b2b = (time.perf_counter() - t0) * 1e3 / args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(8)] for _ in range(args.steps)]
    for s in range(args.steps):
        flush()
        step(evs[s])
    torch.cuda.synchronize()
    per = {n: median_min([evs[s][i].elapsed_time(evs[s][i + 1]) for s in range(args.steps)])[0]
           for i, n in enumerate(names)}
    counts = bufs["counts"].cpu().numpy().tolist()
    fl1, by1 = flops_bytes_gmm(counts, H, F, 1)
    fl2, by2 = flops_bytes_gmm(counts, F, H, 1)
    by1, by2 = by1 + A * 4, by2 + A * 4  # one fp32 scale per activation row
    gmm_ms = (per["gmm1"] + per["gmm2"]) / 2.0
    fl_launch = (fl1 + fl2) / 2.0
    achieved = fl_launch / (gmm_ms * 1e-3) / 1e12
    kernels = {n: {"ms": per[n]} for n in names}
    kernels["gmm1"]["TFLOP/s"] = fl1 / (per["gmm1"] * 1e-3) / 1e12
    kernels["gmm2"]["TFLOP/s"] = fl2 / (per["gmm2"] * 1e-3) / 1e12
    kernels["quant_x"]["GB/s"] = (T * H * 3 + T * 4) / (per["quant_x"] * 1e-3) / 1e9
    kernels["quant_h"]["GB/s"] = (A * F * 3 + A * 4) / (per["quant_h"] * 1e-3) / 1e9
    res = {
        "metric": METRIC, "value": T / (ms_step * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp8_e4m3",
        "timing": timing_record(ms_step, ms_min, ms_b2b, wall_s, args.steps, sclk_start),
        "data": "synthetic (seeded; bf16 N(0,1) tokens and router; N(0,1/fan_in) expert weights quantised "
                "per tensor to E4M3; activations quantised per token on the device)",
        "config": {"workload": f"prefill_fp8: T={T} H={H} E={E} K={K} F={F} ReLU, E4M3 experts, per-token "
                               "dynamic activation quantisation", "T": T, "H": H, "E": E, "K": K, "F": F,
                   "tokens_per_step": T, "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_FP8_TFLOPS, "traffic": measured_traffic("prefill_fp8"),
                     "kernel": "moe_gmm E4M3, per-token scales (gmm_pp8w_kernel)", "gmm_source": source_digest(),
                     "launches_per_step": 2, "flops_per_launch": fl_launch,
                     "bytes_per_launch": (by1 + by2) / 2.0, "avg_launch_ms": gmm_ms},
        "kernels": kernels,
        "ms_per_step_stage_by_stage": sum(per.values()),
    }
    host = {k: d[k] for k in ("x", "wr", "w1", "w1_scale", "w2", "w2_scale", "K")}
    return res, host


def timing_record(ms_med, ms_min, ms_b2b, wall_s, steps, sclk_start):
    return {"ms_per_step_median": ms_med, "ms_per_step_min": ms_min, "ms_per_step_back_to_back": ms_b2b,
            "timed_loop_wall_s": wall_s, "steps": steps, "sclk_reported_at_start": sclk_start,
            "protocol": "each step after a 1 GiB device read (outside its events), timed with HIP events "
                        "on its stream; value from the median step"}


def cpu_baseline_tokens(run, T, target_s, what):
    """Time run(n, threads) -- the oracle on the first n tokens of the
    workload -- with n grown until one run takes about a third of target_s
    (or all T tokens); tokens/s of the last run."""
    nth = cpu_threads()
    n = min(T, 4)
    spent = 0.0
    while True:
        t0 = time.perf_counter()
        run(n, nth)
        dt = time.perf_counter() - t0
        spent += dt
        if dt >= target_s / 3 or n >= T or spent > target_s:
            break
        n = min(T, max(n + 1, int(n * min(8.0, (target_s / 2) / max(dt, 1e-3)))))
    return dict(cpu_info(nth), value=n / dt, unit="tokens/s", kind="oracle",
                sample=f"{what} on the first {n} of {T} tokens, {dt:.1f} s (growing runs {spent:.1f} s in all)")


def cpu_baseline_layer(host, target_s):
    """The oracle (plain fp64 C) on the host cores: the whole layer on the
    first n tokens of the same inputs (full weights)."""
    import oracle
    T = host["x"].shape[0]

    def run(n, nth):
        oracle.layer(host["x"][:n], host["wr"], host["w1"], host["w2"], host["K"], bias=host["bias"],
                     nthreads=nth)

    return cpu_baseline_tokens(run, T, target_s, "whole layer (route, permute, both GEMMs, combine)")


def cpu_baseline_layer_fp8(host, target_s):
    """The oracle's E4M3 layer on the first n tokens (full weights)."""
    import numpy as np

    import oracle
    T = host["x"].shape[0]

    def run(n, nth):
        oracle.layer_fp8(host["x"], host["wr"], host["w1"], host["w1_scale"], host["w2"], host["w2_scale"],
                         host["K"], tokens=np.arange(n), nthreads=nth)

    return cpu_baseline_tokens(run, T, target_s, "whole E4M3 layer (per-token quantisation, both GEMMs)")


def cpu_baseline_page2(host, target_s):
    """The oracle on the page-2 step of the first n tokens: their K routed rows
    through the grouped GEMM in the workload's quantisation (per-tensor, MX,
    MXFP4, or per-token after the oracle's own quantisation), the Unpermute of
    those rows, and their rows of the shared bf16 expert."""
    import numpy as np

    import oracle
    d, mode = host["d"], host["mode"]
    T, e, K = d["T"], d["e"], d["K"]
    _, off, _, pdst = oracle.permute(d["topk_idx"], e)

    def run(n, nth):
        grouped = pdst[: n * K]
        rows = np.sort(grouped)
        ex = np.searchsorted(off, rows, side="right") - 1
        sub_off = np.concatenate([[0], np.cumsum(np.bincount(ex, minlength=e))]).astype(np.int32)
        if mode in ("mx", "mx4"):
            f = oracle.gmm_mx4 if mode == "mx4" else oracle.gmm_mx
            y = f(d["gmm_x"][rows], d["gmm_x_scale"][rows], d["gmm_w"], d["gmm_w_scale"], sub_off, nthreads=nth)
        elif mode == "dyn":
            q, sc = oracle.quant_rows(d["gmm_x"], rows=rows)
            y = oracle.gmm(q, d["gmm_w"], sub_off, a_scale=sc.astype(np.float64), w_scale=float(d["gmm_w_scale"]),
                           nthreads=nth)
        else:
            y = oracle.gmm(d["gmm_x"][rows], d["gmm_w"], sub_off, a_scale=float(d["gmm_x_scale"]),
                           w_scale=float(d["gmm_w_scale"]), nthreads=nth)
        local = np.searchsorted(rows, grouped).astype(np.int32)
        oracle.combine(y, local, None, n, K)  # Unpermute into (token, slot) order
        oracle.gmm(d["mm_x"][:n], d["mm_w"].reshape(1, d["H2"], d["N2"]), np.array([0, n], np.int32),
                   nthreads=nth)

    return cpu_baseline_tokens(run, T, target_s, "routed grouped GEMM + Unpermute + shared expert")


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "the MoE layer here runs on one GPU; --gpus must be 1 (the "
                                   "expert-parallel all-to-all across GPUs is not implemented)"}))
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    import mixture_experts_layer_06_amd as moe
    moe.lib()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.workload == "prefill_fp8":
        res, host = bench_layer_fp8(args, dev)
        res["achievable"] = achievable(dev)
    elif args.workload in ("fp8gmm", "fp8gmm_one", "fp8mx", "fp8mx_one", "fp8dyn", "fp4mx", "fp4mx_one"):
        res, host = bench_fp8(args, dev, mode={"fp8gmm": "pt", "fp8gmm_one": "one", "fp8mx": "mx",
                                               "fp8mx_one": "mx_one", "fp8dyn": "dyn", "fp4mx": "mx4",
                                               "fp4mx_one": "mx4_one"}[args.workload])
        res["achievable"] = achievable(dev)
    else:
        res, host = bench_layer(args, dev)
        c = res["config"]
        even = None
        if args.workload == "prefill":  # the vendor's batched GEMM on even expert loads, for context
            even = (c["E"], c["T"] * c["K"] // c["E"], {"gemm1": (c["H"], c["F"]), "gemm2": (c["F"], c["H"])})
        res["achievable"] = achievable(dev, even)
    if not args.no_cpu:
        if args.workload == "prefill_fp8":
            res["cpu_baseline"] = cpu_baseline_layer_fp8(host, args.cpu_seconds)
        elif "d" in host:
            res["cpu_baseline"] = cpu_baseline_page2(host, args.cpu_seconds)
        else:
            res["cpu_baseline"] = cpu_baseline_layer(host, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
