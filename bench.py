#!/usr/bin/env python3
"""Benchmark of the GLM-5.3-Flash routed MoE MLP on one MI355X.

One step = one decode pass of the whole layer (router logits, top-k,
routed NVFP4 gate/up + clamped SwiGLU, routed NVFP4 down, BF16 shared
expert, combine) for one token of the GLM-Flash-sized workload: T=1,
H=4096, I=1536, E=288 experts resident on the GPU, K=8, shared expert
intermediate 1536.  Inputs are synthetic (seeded), already in HBM.

`value` is decode weight-stream GB/s: the algorithmic bytes of a step
(unique touched experts x 10,616,832 B NVFP4 + 37,748,736 B shared BF16 +
4,718,592 B fp32 router + x and out) over the measured step time of the
K timed steps (issued back to back between two stream events).  Steps
rotate over several copies of the layer's weights (each with its own input
token; 8 copies touch ~1 GB between two visits of one copy, 4x the 256 MB
last-level cache) so every step streams its weights from HBM, as a layer
inside a full model would.  The median and p10/p90 step time come from 64
further event-bracketed runs of 8 back-to-back steps.

Also reported: per-stage kernel times (HIP events attached to the stages'
dispatches, steps issued back to back), the roofline of the dominant
kernel (routed gate/up GEMV) with its rocprofv3 HBM traffic, a measured
device-copy bandwidth beside the 8 TB/s datasheet peak, decode at T=2, 4,
16, 64, the skewed 64-token top-16 workload, the literal-bias workloads,
the prefill grouped-GEMM path at T=4096 (TFLOP/s), the dense FFN, and the
fp64 CPU oracle timed on bounded samples on the host cores.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
import argparse
import ctypes
import dataclasses
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E
CALIB_BYTES = 512 << 20         # the counter-calibration copy
COPY_BYTES = 1 << 30            # the measured device copy
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "routed_gateup_flash_decode_t1_traffic.txt")
GEMV_SOURCES = ["routed_expert_mlp_amd/csrc/decode1.hpp", "routed_expert_mlp_amd/csrc/router.hpp",
                "routed_expert_mlp_amd/csrc/gemv.hpp", "routed_expert_mlp_amd/csrc/common.hpp"]
DOMINANT = "routed_gateup"      # stage of the dominant one-token kernel (k_dec_gateup)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=400)
    p.add_argument("--warmup", type=int, default=40)
    p.add_argument("--copies", type=int, default=8, help="weight copies rotated over (cold HBM reads)")
    p.add_argument("--no-prefill", action="store_true")
    p.add_argument("--no-extra-decode", action="store_true")
    p.add_argument("--no-variants", action="store_true", help="skip the skewed and literal-bias workloads")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="target oracle CPU time per sample")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="end the decode part with 3 device copies of 512 MiB (counter calibration)")
    p.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                   help="write the traffic summary from two rocprofv3 --pmc counter_collection.csv files and exit")
    return p.parse_args()


class HipEvents:
    """Raw hipEvent_t handles from the HIP runtime torch has loaded."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        out = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            out.append(e.value)
        return out

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, evs):
        for e in evs:
            self.hip.hipEventDestroy(e)


def upload_routed(w, device):
    """All weights of a routed workload on the device (synth's bytes)."""
    import numpy as np
    import torch
    import synth
    from routed_expert_mlp_amd import capi
    E, H, I = w.E, w.H, w.I
    wt = capi.Weights(router_w=torch.from_numpy(synth.router_weight(w)).to(device),
                      router_bias=torch.from_numpy(synth.router_bias(w)).to(device))
    if w.fmt == "fp8":
        B = capi.FP8_BLOCK
        wt.w13_f8 = torch.empty((E, 2 * I, H), dtype=torch.uint8, device=device)
        wt.w13_f8_scale = torch.empty((E, 2 * I // B, H // B), dtype=torch.float32, device=device)
        wt.w2_f8 = torch.empty((E, H, I), dtype=torch.uint8, device=device)
        wt.w2_f8_scale = torch.empty((E, H // B, I // B), dtype=torch.float32, device=device)
        dst = (wt.w13_f8, wt.w13_f8_scale, wt.w2_f8, wt.w2_f8_scale)
    else:
        wt.w13_q = torch.empty((E, 2 * I, H // 2), dtype=torch.uint8, device=device)
        wt.w13_s = torch.empty((E, 2 * I, H // 16), dtype=torch.uint8, device=device)
        wt.w13_g = torch.from_numpy(synth.w13_globals(w)).to(device)
        wt.w2_q = torch.empty((E, H, I // 2), dtype=torch.uint8, device=device)
        wt.w2_s = torch.empty((E, H, I // 16), dtype=torch.uint8, device=device)
        wt.w2_g = torch.from_numpy(synth.w2_globals(w)).to(device)
        dst = (wt.w13_q, wt.w13_s, wt.w2_q, wt.w2_s)

    def put(e, q13, s13, q2, s2):
        for d, v in zip(dst, (q13, s13, q2, s2)):
            d[e].copy_(torch.from_numpy(v))

    synth.for_each_expert(w, put)
    if w.Is:
        def bf(bits):
            return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.bfloat16)
        wt.shared_w13 = bf(synth.shared_w13(w))
        wt.shared_w2 = bf(synth.shared_w2(w))
    return wt


def clone_weights(wt):
    import dataclasses
    return dataclasses.replace(wt, **{f.name: (None if getattr(wt, f.name) is None else getattr(wt, f.name).clone())
                                      for f in dataclasses.fields(wt)})


def config_of(w):
    from routed_expert_mlp_amd import capi
    return capi.Config(kind=capi.KIND_ROUTED_FP8 if w.fmt == "fp8" else capi.KIND_ROUTED, hidden=w.H, moe_intermediate=w.I, num_experts=w.E, top_k=w.K,
                       n_shared_experts=1 if w.Is else 0, shared_intermediate=w.Is, dense_intermediate=0,
                       routed_scaling_factor=w.rsf, swiglu_limit=w.swiglu_limit)


def x_dev(w, tokens, device):
    import numpy as np
    import torch
    import synth
    bits = np.stack([synth.x_row(w, int(t)) for t in tokens])
    return torch.from_numpy(bits.view(np.int16)).to(device).view(torch.bfloat16)


def decode_bytes(w, n_unique, T):
    return (n_unique * w.expert_bytes + 2 * 3 * w.Is * w.H + 4 * w.E * w.H + 2 * 2 * T * w.H)


def source_hash(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic():
    """HBM bytes per launch of the routed gate/up GEMV measured with rocprofv3
    counters, if the committed measurement is of the current kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    vals = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                vals[k.strip()] = v.strip()
    if vals.get("source_sha256_16") != source_hash(GEMV_SOURCES):
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def summarize_traffic(fetch_csv, write_csv):
    """HBM bytes per launch of the one-token decode kernels from two rocprofv3 --pmc runs of
    `bench.py --calibrate-copy` (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch).  Each counter is
    scaled by what it reads for the 512 MiB device copies the run ends its decode part with."""
    import csv
    import numpy as np

    def per_kernel(path):
        rows = list(csv.DictReader(open(path)))
        vals = {}
        order = []
        for r in rows:
            v = float(r["Counter_Value"])
            name = r["Kernel_Name"]
            vals.setdefault(name, []).append(v)
            order.append((name, v))
        return vals, order

    out = []
    scale = {}
    per = {}
    for label, path in (("fetch", fetch_csv), ("write", write_csv)):
        vals, order = per_kernel(path)
        # the calibration copies: the first three copies after the last decode dispatch
        last = max(i for i, (n, _) in enumerate(order) if "k_dec_" in n)
        copies = [v for n, v in order[last + 1:] if "copyBuffer" in n][:3]
        if len(copies) < 3:
            raise SystemExit(f"{path}: the calibration copies are missing")
        scale[label] = CALIB_BYTES / (float(np.mean(copies)) * 1024.0)
        for name, v in vals.items():
            if "k_dec_" in name:
                short = name.split("(")[0].replace("void ", "")
                per.setdefault(short, {})[label] = float(np.mean(v)) * 1024.0 * scale[label]
                per[short]["n"] = len(v)
    out.append(f"fetch_scale = {scale['fetch']:.5f}")
    out.append(f"write_scale = {scale['write']:.5f}")
    main_kernel = None
    for short, d in sorted(per.items()):
        out.append(f"# {short}: {d['n']} dispatches, fetch {d.get('fetch', 0):.0f} B, write {d.get('write', 0):.0f} B "
                   f"per launch (scaled)")
        if short.startswith("moe::k_dec_gateup"):
            main_kernel = d
    if main_kernel is None:
        raise SystemExit("no k_dec_gateup dispatches in the counter files")
    out.append(f"source_sha256_16 = {source_hash(GEMV_SOURCES)}")
    out.append(f"hbm_bytes_per_launch = {main_kernel.get('fetch', 0) + main_kernel.get('write', 0):.0f}")
    return out


def loop_seconds(fn, n):
    """Mean seconds per call of n calls issued back to back (one synchronisation at each end)."""
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(n):
        fn(i)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / max(n, 1)


def timed_region_ms(fn, n):
    """Exactly n calls back to back between two stream events, with a device synchronisation on
    both sides: ms from the first event to the second."""
    import torch
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for i in range(n):
        fn(i)
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b)


def chunk_step_ms(fn, n_chunks, per_chunk):
    """n_chunks runs of per_chunk back-to-back calls with a stream event between runs (none inside
    a run): the mean ms per call of each run."""
    import torch
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n_chunks + 1)]
    torch.cuda.synchronize()
    evs[0].record()
    i = 0
    for c in range(n_chunks):
        for _ in range(per_chunk):
            fn(i)
            i += 1
        evs[c + 1].record()
    torch.cuda.synchronize()
    return [evs[c].elapsed_time(evs[c + 1]) / per_chunk for c in range(n_chunks)]


def pctl(vals_ms):
    import numpy as np
    a = np.asarray(vals_ms, dtype=np.float64) * 1e3
    return [round(float(v), 2) for v in np.percentile(a, [10, 50, 90])]


def stage_times(cfg, wts, xs, out, prefill, n, ev, ws):
    """Per-stage milliseconds (mean over n steps) from HIP events attached to each stage's first
    and last kernel dispatch; the n steps are issued back to back and read after one sync."""
    import numpy as np
    import torch
    from routed_expert_mlp_amd import capi
    names = capi.stage_names(cfg, xs[0].shape[0], prefill)
    m = 2 * len(names)
    evs = ev.create(m * n)
    try:
        torch.cuda.synchronize()
        for i in range(n):
            r = i % len(wts)
            capi.moe_mlp_forward_profiled(cfg, wts[r], xs[r], out[r], prefill, evs[m * i:m * (i + 1)], ws=ws)
        torch.cuda.synchronize()
        t = np.zeros((n, len(names)))
        for i in range(n):
            for j in range(len(names)):
                t[i, j] = ev.elapsed_ms(evs[m * i + 2 * j], evs[m * i + 2 * j + 1])
    finally:
        torch.cuda.synchronize()
        ev.destroy(evs)
    skip = min(n // 4, 8)                        # the first steps start on an idle GPU
    return {nm: float(np.mean(t[skip:, j])) for j, nm in enumerate(names)}


def device_copy_gbs(device):
    """Read+write GB/s of a 1 GiB device-to-device copy (best of 5)."""
    import torch
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=device).fill_(1.0)
    dst = torch.empty_like(src)
    best = 1e9
    for i in range(6):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        torch.cuda.synchronize()
        if i:
            best = min(best, a.elapsed_time(b))
    del src, dst
    torch.cuda.empty_cache()
    return 2 * COPY_BYTES / (best * 1e-3) / 1e9


def decode_line(cfg, w, wts, xs, T, dev, steps, ws=None):
    """Decode of T tokens over rotated weight copies: GB/s, us/step (mean of a back-to-back loop),
    tokens/s, unique experts touched."""
    import numpy as np
    import torch
    from routed_expert_mlp_amd import capi
    R = len(wts)
    out_t = [torch.empty((T, w.H), dtype=torch.bfloat16, device=dev) for _ in range(R)]
    ids_t = [torch.empty((T, w.K), dtype=torch.int32, device=dev) for _ in range(R)]
    ws = capi.workspace(cfg, T, False, dev) if ws is None else ws
    calls = [capi.bind_layer(cfg, wts[r], xs[r], out_t[r], ids_t[r], ws=ws) for r in range(R)]
    for i in range(2 * R):
        calls[i % R]()
    s_t = loop_seconds(lambda i: calls[i % R](), steps)
    u = [int(torch.unique(ids_t[r]).numel()) for r in range(R)]
    b = float(np.mean([decode_bytes(w, x, T) for x in u]))
    return {"gbs": round(b / s_t / 1e9, 1), "us_per_step": round(s_t * 1e6, 1),
            "tokens_per_s": round(T / s_t, 1), "unique_experts": float(np.mean(u))}


def cpu_decode_baseline(w, budget_s, blas_threads=None):
    """The fp64 oracle, as it stands, on a bounded sample of single-token decodes."""
    import contextlib
    import psutil
    import threadpoolctl
    import oracle as O
    import synth
    limiter = threadpoolctl.threadpool_limits(blas_threads) if blas_threads else contextlib.nullcontext()
    with limiter:
        blas = threadpoolctl.threadpool_info()
        threads = max([b.get("num_threads", 1) for b in blas] or [1])
        rw, rb = synth.router_weight(w), synth.router_bias(w)
        g13, g2 = synth.w13_globals(w), synth.w2_globals(w)
        s13, s2 = synth.shared_w13(w), synth.shared_w2(w)
        cache = {}

        def expert(e):
            if e not in cache:
                cache[e] = synth.expert_w13(w, e) + synth.expert_w2(w, e)
            return cache[e]

        wts = O.RoutedWeights(rw, rb, g13, g2, expert, s13, s2)
        proc = psutil.Process()
        done, elapsed, cpu = 0, 0.0, 0.0
        t = 0
        while elapsed < budget_s and done < 64:
            x = synth.x_row(w, 1000 + t)[None, :]
            ids, _, _, _ = O.route(O.decode_bf16(x), rw, rb, w.K, w.rsf)
            for e in ids[0]:
                expert(int(e))                    # input generation is not timed
            c0 = proc.cpu_times()
            t0 = time.perf_counter()
            O.moe_layer(x, wts, w.K, w.rsf, w.swiglu_limit)
            elapsed += time.perf_counter() - t0
            c1 = proc.cpu_times()
            cpu += (c1.user - c0.user) + (c1.system - c0.system)
            done += 1
            t += 1
            if len(cache) > 64:
                cache.clear()
    per_tok = elapsed / done
    return {
        "value": round(decode_bytes(w, w.K, 1) / per_tok / 1e9, 4),
        "unit": "GB/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{done} single-token decodes of the T=1 workload (fp64 NumPy oracle, contract mode); "
                  f"{per_tok * 1e3:.1f} ms/token, {1.0 / per_tok:.2f} tokens/s; "
                  f"cpu_util={cpu / elapsed:.2f} cores busy on {os.cpu_count()} host cpus",
    }


def cpu_prefill_baseline(wp, n_tokens):
    """The fp64 oracle on the first n_tokens tokens of the 4096-token prefill workload (one
    moe_layer call; its cost is dominated by building the touched experts' fp64 weights)."""
    import numpy as np
    import threadpoolctl
    import oracle as O
    import synth
    threads = max([b.get("num_threads", 1) for b in threadpoolctl.threadpool_info()] or [1])
    x = synth.x_rows(wp, n_tokens)
    wts = O.RoutedWeights(synth.router_weight(wp), synth.router_bias(wp), synth.w13_globals(wp),
                          synth.w2_globals(wp), lambda e: synth.expert_w13(wp, e) + synth.expert_w2(wp, e),
                          synth.shared_w13(wp), synth.shared_w2(wp))
    t0 = time.perf_counter()
    _, ids, _ = O.moe_layer(x, wts, wp.K, wp.rsf, wp.swiglu_limit)
    el = time.perf_counter() - t0
    fl = 2.0 * n_tokens * (wp.K * 3 * wp.H * wp.I + 3 * wp.H * wp.Is + wp.H * wp.E)
    return {"value": round(fl / el / 1e9, 3), "unit": "GFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"the first {n_tokens} tokens of the 4096-token prefill workload in one oracle call "
                      f"({len(np.unique(ids))} experts touched, expert weights regenerated inside the "
                      f"timed call); {el:.1f} s, {n_tokens / el:.3f} tokens/s"}


def main():
    args = parse()
    if args.summarize_traffic:
        lines = summarize_traffic(*args.summarize_traffic)
        head = ["# HBM traffic of the one-token decode kernels, flash_decode_t1 (T=1, H=4096, I=1536, E=288, K=8,",
                "# Is=1536), from two rocprofv3 counter runs on one MI355X (from the repository root):",
                "#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d <out>/pmc_fetch -o run -- \\",
                "#       python3 bench.py --steps 20 --warmup 5 --no-prefill --no-extra-decode --no-variants \\",
                "#       --no-cpu-baseline --calibrate-copy",
                "#   rocprofv3 --pmc WRITE_SIZE --output-format csv -d <out>/pmc_write -o run -- (same)",
                "#   python3 bench.py --summarize-traffic <fetch counter_collection.csv> <write counter_collection.csv>",
                "# FETCH_SIZE / WRITE_SIZE are KiB per dispatch; each is scaled so that the run's 512 MiB device",
                "# copies read and write 512 MiB.  bench.py reports hbm_bytes_per_launch (k_dec_gateup) as",
                "# roofline.traffic while source_sha256_16 matches the kernel sources."]
        with open(TRAFFIC_FILE, "w") as f:
            f.write("\n".join(head + lines) + "\n")
        print("\n".join(lines))
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only (the layer holds all 288 experts on "
                                   "one MI355X); --gpus N>1 is not supported"}))
        sys.exit(2)
    import numpy as np
    import torch
    import synth
    from routed_expert_mlp_amd import capi

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    dev = "cuda:0"
    capi.lib()
    ev = HipEvents()

    # ---------------- decode T=1 (the headline) ----------------
    w = synth.workload("flash_decode_t1")
    cfg = config_of(w)
    log(f"[bench] generating + uploading {w.name}: E={w.E} experts, {w.E * w.expert_bytes / 1e9:.2f} GB NVFP4")
    base = upload_routed(w, dev)
    R = max(1, args.copies)
    wts = [base] + [clone_weights(base) for _ in range(R - 1)]
    xs = [x_dev(w, [r], dev) for r in range(R)]
    outs = [torch.empty((1, w.H), dtype=torch.bfloat16, device=dev) for _ in range(R)]
    ids = [torch.empty((1, w.K), dtype=torch.int32, device=dev) for _ in range(R)]
    ws = capi.workspace(cfg, 1, False, dev)
    torch.cuda.synchronize()

    calls = [capi.bind_layer(cfg, wts[r], xs[r], outs[r], ids[r], ws=ws) for r in range(R)]

    def step(i):
        calls[i % R]()

    for i in range(args.warmup):
        step(i)
    uniq = [int(torch.unique(ids[r]).numel()) for r in range(R)]
    step_bytes = float(np.mean([decode_bytes(w, u, 1) for u in uniq]))
    log(f"[bench] timing {args.steps} decode steps over {R} weight copies")
    total_ms = timed_region_ms(step, args.steps)
    sec = total_ms * 1e-3 / args.steps
    gbs = step_bytes / sec / 1e9
    n_chunks = 64
    p10, p50, p90 = pctl(chunk_step_ms(step, n_chunks, R))

    st = stage_times(cfg, wts, xs, outs, False, 8 * R, ev, ws)
    # warm: one weight copy, so the 8 experts + shared + router (~128 MB) stay in the 256 MB MALL
    for i in range(20):
        calls[0]()
    sec_warm = min(loop_seconds(lambda i: calls[0](), 400) for _ in range(3))
    # the same steps replayed from HIP graphs of 16 steps each (one graph per starting copy)
    graph_us = None
    try:
        gs = []
        gsm = torch.cuda.Stream()
        gsm.wait_stream(torch.cuda.current_stream())
        for r in range(R):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=gsm):
                for j in range(16):
                    q = (r + j) % R
                    capi.moe_mlp_decode(cfg, wts[q], xs[q], outs[q], ids[q], ws=ws)
            gs.append(g)
        for i in range(2 * R):
            gs[i % R].replay()
        n_rep = max(8, 400 // 16)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(n_rep):
            gs[i % R].replay()
        torch.cuda.synchronize()
        graph_us = (time.perf_counter() - t0) / (n_rep * 16) * 1e6
        del gs
    except RuntimeError as exc:                       # capture unsupported: report, do not fail the run
        log(f"[bench] graph capture failed: {exc}")
    if args.calibrate_copy:
        # a plain device copy of known size, for scaling the FETCH_SIZE / WRITE_SIZE counters
        src = torch.empty(CALIB_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    dom_ms = st[DOMINANT]
    # algorithmic bytes of each one-token stage
    exp13 = 2 * w.I * w.H // 2 + 2 * w.I * w.H // 16          # NVFP4 gate/up of one expert
    exp2 = w.H * w.I // 2 + w.H * w.I // 16                    # NVFP4 down of one expert
    stage_bytes = {
        "logits_shared_gateup": 4 * w.E * w.H + 2 * 2 * w.Is * w.H + 2 * w.H + 4 * w.E + 2 * w.Is,
        "routed_gateup": w.K * exp13 + 2 * w.H + 4 * w.E * 2 + 2 * w.K * w.I + 8 * w.K,
        "shared_routed_down_combine": (w.K * exp2 + 2 * w.H * w.Is + 2 * w.K * w.I + 2 * w.Is + 2 * w.H
                                       + 8 * w.K),
    }
    dom_bytes = stage_bytes[DOMINANT]
    dom_gbs = dom_bytes / (dom_ms * 1e-3) / 1e9
    traffic = read_traffic()
    copy_gbs = None
    if not args.calibrate_copy:
        log("[bench] measuring the device copy bandwidth")
        copy_gbs = device_copy_gbs(dev)
    extra = {"tokens_per_s": round(1.0 / sec, 1), "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
             "bytes_per_step": int(step_bytes),
             "step_us_p10_p50_p90": [p10, p50, p90],
             "step_timing": f"value and ms_per_step: the {args.steps} timed steps issued back to back between two "
                            f"stream events; percentiles: {n_chunks} further runs of {R} back-to-back steps (one per "
                            f"weight copy) with a stream event between runs, mean per step of each run",
             "decode_stage_us": {k: round(v * 1e3, 2) for k, v in st.items()},
             "decode_stage_gbs": {k: round(stage_bytes[k] / (v * 1e-3) / 1e9, 1)
                                  for k, v in st.items() if k in stage_bytes and v > 0},
             "decode_graph_us_per_step": None if graph_us is None else round(graph_us, 2),
             "decode_warm": {"us_per_step": round(sec_warm * 1e6, 2),
                             "gbs": round(decode_bytes(w, uniq[0], 1) / sec_warm / 1e9, 1),
                             "tokens_per_s": round(1.0 / sec_warm, 1),
                             "note": "one weight copy, resident in the 256 MB last-level cache"}}

    # ---------------- decode T=2..64 (same weights, more tokens) ----------------
    if not args.no_extra_decode:
        wts_tiled = None
        for T in (2, 4, 16, 64):
            xs_t = [x_dev(w, range(100 + r * T, 100 + (r + 1) * T), dev) for r in range(R)]
            wts_t = wts
            if T >= 16:
                # decode batches read the tile-layout copies of the routed
                # weights (packed once at load) in their few-token MFMA
                # kernels and the grouped GEMM
                if wts_tiled is None:
                    wts_tiled = [capi.with_tiled_weights(x) for x in wts]
                wts_t = wts_tiled
            extra[f"decode_t{T}"] = decode_line(cfg, w, wts_t, xs_t, T, dev, max(40, args.steps // 4))
            if T in (16, 64):
                outs_t = [torch.empty((T, w.H), dtype=torch.bfloat16, device=dev) for _ in range(R)]
                st_t = stage_times(cfg, wts_t, xs_t, outs_t, False, 4 * R, ev, capi.workspace(cfg, T, False, dev))
                extra[f"decode_t{T}"]["stage_us"] = {k: round(v * 1e3, 1) for k, v in st_t.items()}
                # the routed expert projections alone: the touched experts' bytes over the
                # routed gate/up + routed down kernel time (the decode expert-GEMV figure)
                ue = extra[f"decode_t{T}"]["unique_experts"]
                rt = (st_t["routed_gateup"] + st_t["routed_down"]) * 1e-3
                r_gbs = ue * w.expert_bytes / rt / 1e9
                extra[f"decode_t{T}"]["routed_expert_gbs"] = round(r_gbs, 1)
                extra[f"decode_t{T}"]["routed_expert_frac_hbm_peak"] = round(r_gbs / HBM_PEAK_GBS, 4)
            if T >= 16:
                extra[f"decode_t{T}"]["weights"] = ("routed NVFP4: row-major and tile-layout copies resident "
                                                    "(the few-token MFMA kernels read the tile layout)")
        # one resident copy of the codes: the same copies with the row-major
        # codes left out, so every kernel reads the tile-layout codes
        one = [dataclasses.replace(x, w13_q=None, w2_q=None) for x in wts_tiled]
        codes = w.E * (2 * w.I * w.H // 2 + w.H * w.I // 2)
        scales = w.E * (2 * w.I * w.H // 16 + w.H * w.I // 16)
        oc = {"t1": decode_line(cfg, w, one, xs, 1, dev, args.steps)}
        xs16 = [x_dev(w, range(100 + r * 16, 100 + (r + 1) * 16), dev) for r in range(R)]
        oc["t16"] = decode_line(cfg, w, one, xs16, 16, dev, max(40, args.steps // 4))
        oc["resident_routed_weight_bytes"] = {
            "tile_codes_only": codes + 2 * scales, "row_major_and_tile": 2 * (codes + scales),
            "note": "tile-layout codes once, scales in both layouts (the decode kernels read row-major scales, "
                    "the grouped GEMM tile-layout ones)"}
        extra["decode_tile_codes_only"] = oc
        del wts_tiled, one
    del calls
    del wts[1:]
    torch.cuda.empty_cache()

    # ---------------- skewed top-16 and literal-bias decode workloads ----------------
    if not args.no_variants:
        RV = 4          # weight copies per variant (4 x 3.06 GB)
        for name, T in (("skewed_decode_t64_k16", 64), ("flash_decode_t1_literal_bias", 1),
                        ("flash_decode_t64_literal_bias", 64)):
            wv = synth.workload(name)
            cfgv = config_of(wv)
            log(f"[bench] generating + uploading {name}")
            bv = upload_routed(wv, dev)
            wts_v = [bv] + [clone_weights(bv) for _ in range(RV - 1)]
            if T >= 64:
                wts_v = [capi.with_tiled_weights(x) for x in wts_v]
            xs_v = [x_dev(wv, range(r * T, (r + 1) * T), dev) for r in range(RV)]
            line = decode_line(cfgv, wv, wts_v, xs_v, T, dev, max(40, args.steps // 4))
            line["workload"] = f"T={T}, K={wv.K}, E={wv.E}, bias " + (
                "+1.0 on 8 hot experts, U(-0.1,0.1) elsewhere" if wv.hot_experts else f"U(-{wv.bias_amp}, {wv.bias_amp})")
            if T >= 64:
                line["weights"] = ("routed NVFP4: row-major and tile-layout copies resident "
                                   "(the few-token MFMA kernels read the tile layout)")
            if wv.hot_experts:
                # per-stage kernel times, and the routed projections' bytes over their time
                outs_v = [torch.empty((T, wv.H), dtype=torch.bfloat16, device=dev) for _ in range(RV)]
                st_v = stage_times(cfgv, wts_v, xs_v, outs_v, False, 4 * RV, ev, capi.workspace(cfgv, T, False, dev))
                line["stage_us"] = {k: round(v * 1e3, 1) for k, v in st_v.items()}
                rt = (st_v["routed_gateup"] + st_v["routed_down"]) * 1e-3
                line["routed_expert_gbs"] = round(line["unique_experts"] * wv.expert_bytes / rt / 1e9, 1)
                del outs_v
            extra[name] = line
            del wts_v, bv, xs_v
            torch.cuda.empty_cache()
        # FP8 block-scaled experts (E4M3, fp32 scale per 128 x 128 block): one-token decode
        wv = synth.workload("flash_decode_t1_fp8")
        cfgv = config_of(wv)
        log(f"[bench] generating + uploading {wv.name}: {wv.E * wv.expert_bytes / 1e9:.2f} GB FP8")
        bv = upload_routed(wv, dev)
        wts_v = [bv] + [clone_weights(bv) for _ in range(RV - 1)]
        xs_v = [x_dev(wv, [r], dev) for r in range(RV)]
        line = decode_line(cfgv, wv, wts_v, xs_v, 1, dev, max(40, args.steps // 4))
        line["workload"] = (f"T=1, H={wv.H}, I={wv.I}, E={wv.E}, K={wv.K}, routed experts FP8 E4M3 with fp32 "
                            f"128x128 block scales ({wv.expert_bytes} B per expert), BF16 shared expert")
        extra["flash_decode_t1_fp8"] = line
        del wts_v, bv, xs_v
        torch.cuda.empty_cache()

    # ---------------- prefill T=4096 ----------------
    if not args.no_prefill:
        del wts
        torch.cuda.empty_cache()
        for pname in ("prefill_t4096", "prefill_t4096_literal_bias", "prefill_t4096_fp8"):
            wp = synth.workload(pname)
            cfgp = config_of(wp)
            log(f"[bench] generating + uploading {wp.name}")
            wt_rm = upload_routed(wp, dev)
            # the NVFP4 grouped GEMM reads the routed weights in the tile layout,
            # packed once at load (the row-major arrays stay for the GEMV forms)
            wtp = wt_rm if wp.fmt == "fp8" else capi.with_tiled_weights(wt_rm)
            xp = torch.from_numpy(synth.x_rows(wp).view(np.int16)).to(dev).view(torch.bfloat16)
            outp = torch.empty((wp.T, wp.H), dtype=torch.bfloat16, device=dev)
            wsp = capi.workspace(cfgp, wp.T, True, dev)
            for _ in range(3):
                capi.moe_mlp_prefill(cfgp, wtp, xp, outp, ws=wsp)
            n = 10
            s_rm = loop_seconds(lambda i: capi.moe_mlp_prefill(cfgp, wt_rm, xp, outp, ws=wsp), n)
            s_p = loop_seconds(lambda i: capi.moe_mlp_prefill(cfgp, wtp, xp, outp, ws=wsp), n)
            stp = stage_times(cfgp, [wtp], [xp], [outp], True, 8, ev, wsp)
            T, K, H, I, Is, E = wp.T, wp.K, wp.H, wp.I, wp.Is, wp.E
            fl_routed = 2.0 * T * K * 3 * H * I
            fl_total = fl_routed + 2.0 * T * 3 * H * Is + 2.0 * T * H * E
            gg_ms = stp["routed_gateup"] + stp["routed_down"]
            if wp.fmt == "fp8":
                res = {"weights": "routed FP8 E4M3, fp32 128x128 block scales (row-major)",
                       "resident_routed_weight_bytes": {"row_major": int(wp.E * wp.expert_bytes)}}
            else:
                rm_bytes = sum(t.numel() for t in (wt_rm.w13_q, wt_rm.w13_s, wt_rm.w2_q, wt_rm.w2_s))
                res = {"weights": "routed NVFP4 in the tile layout (packed once at load)",
                       "resident_routed_weight_bytes": {"row_major": int(rm_bytes), "tile_layout": int(rm_bytes),
                                                        "note": "both copies stay resident: the GEMV forms read "
                                                                "the row-major arrays, the grouped GEMM the tile "
                                                                "layout"},
                       "ms_per_step_row_major_weights": round(s_rm * 1e3, 3)}
            extra[pname] = {
                "ms_per_step": round(s_p * 1e3, 3), "layer_tflops": round(fl_total / s_p / 1e12, 1),
                **res,
                "grouped_gemm_tflops": round(fl_routed / (gg_ms * 1e-3) / 1e12, 1),
                "grouped_gemm_frac_bf16_peak": round(fl_routed / (gg_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                "stage_us": {k: round(v * 1e3, 1) for k, v in stp.items()}}
            del wtp, wt_rm, xp, outp, wsp
            torch.cuda.empty_cache()

        # ---------------- dense FFN variant: prefill T=4096 and one-token decode ----------------
        wd = synth.workload("dense_prefill_t4096")
        cfgd = capi.Config(kind=capi.KIND_DENSE, hidden=wd.H, moe_intermediate=0, num_experts=0, top_k=0,
                           n_shared_experts=0, shared_intermediate=0, dense_intermediate=wd.Id,
                           routed_scaling_factor=wd.rsf, swiglu_limit=wd.swiglu_limit)

        def bf(bits):
            return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

        log(f"[bench] generating + uploading {wd.name}")
        wtd = capi.Weights(dense_w13=bf(synth.dense_w13(wd)), dense_w2=bf(synth.dense_w2(wd)))
        xd = bf(synth.x_rows(wd))
        outd = torch.empty((wd.T, wd.H), dtype=torch.bfloat16, device=dev)
        wsd = capi.workspace(cfgd, wd.T, True, dev)
        call_d = capi.bind_layer(cfgd, wtd, xd, outd, ws=wsd, prefill=True)
        for _ in range(3):
            call_d()
        s_d = loop_seconds(lambda i: call_d(), 10)
        std = stage_times(cfgd, [wtd], [xd], [outd], True, 8, ev, wsd)
        fl_d = 2.0 * wd.T * 3 * wd.H * wd.Id
        x1 = xd[:1].contiguous()
        out1 = torch.empty((1, wd.H), dtype=torch.bfloat16, device=dev)
        ws1 = capi.workspace(cfgd, 1, False, dev)
        call_d1 = capi.bind_layer(cfgd, wtd, x1, out1, ws=ws1)
        for _ in range(10):
            call_d1()
        s_d1 = loop_seconds(lambda i: call_d1(), 200)
        dense_bytes = 2 * 3 * wd.H * wd.Id
        extra["dense_prefill_t4096"] = {
            "ms_per_step": round(s_d * 1e3, 3), "tflops": round(fl_d / s_d / 1e12, 1),
            "frac_bf16_peak": round(fl_d / s_d / 1e12 / BF16_PEAK_TFLOPS, 4),
            "stage_us": {k: round(v * 1e3, 1) for k, v in std.items()},
            "decode_t1_us": round(s_d1 * 1e6, 2),
            "decode_t1_gbs_warm": round(dense_bytes / s_d1 / 1e9, 1),
            "note": "dense FFN H=4096, Id=12288, bf16 weights (302 MB: the T=1 decode line reads them "
                    "from the 256 MB last-level cache only in part)"}
        del call_d, call_d1, wtd, xd, outd, wsd

    # ---------------- CPU oracle baselines ----------------
    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle")
        cpu = cpu_decode_baseline(w, args.cpu_seconds)
        extra["cpu_baseline_1_blas_thread"] = cpu_decode_baseline(w, args.cpu_seconds / 2, blas_threads=1)
        extra["cpu_baseline_prefill_t4096"] = cpu_prefill_baseline(synth.workload("prefill_t4096"), 8)

    rec = {
        "metric": "MoE-MLP decode weight GB/s (% HBM peak) + tokens/s; prefill TFLOP/s",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(sec * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "flash_decode_t1: GLM-Flash routed MoE MLP decode, T=1, H=4096, I=1536, "
                               "E=288 NVFP4 experts (all resident), K=8, BF16 shared expert Is=1536",
                   "tokens": 1, "hidden": w.H, "moe_intermediate": w.I, "experts": w.E, "top_k": w.K,
                   "weights": "nvfp4 (e2m1 + e4m3/16) routed, bf16 shared, fp32 router",
                   "weight_copies_rotated": R},
        "roofline": {"bound": "hbm",
                     "kernel": "routed_gateup (k_dec_gateup: router top-k, NVFP4 gate/up + clamped SwiGLU)",
                     "achieved": round(dom_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(dom_gbs / HBM_PEAK_GBS, 4), "avg_launch_us": round(dom_ms * 1e3, 3),
                     "algorithmic_bytes_per_launch": int(dom_bytes),
                     "traffic": None if traffic is None else int(traffic),
                     "measured_copy_gbs": None if copy_gbs is None else round(copy_gbs, 1),
                     "measured_copy_note": "1 GiB device-to-device copy, read + write bytes over its time"},
        "cpu_baseline": cpu,
    }
    rec.update(extra)
    # the headline must be the bytes of a step over its measured time
    chk = rec["bytes_per_step"] / (rec["ms_per_step"] * 1e-3) / 1e9
    if abs(chk - rec["value"]) > 0.01 * chk:
        raise RuntimeError(f"bench: value {rec['value']} is not bytes_per_step / ms_per_step ({chk:.1f})")
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
