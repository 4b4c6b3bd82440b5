"""Benchmark of the fused tiled attention hot path on one MI355X.

One step = one pass over every stage of the path, each on its own synthetic
batch (already resident in HBM when timing starts):
  1. causal forward,            B=4, H=32, N=4096, d=128, bf16
  2. sliding-window forward,    same tensors, window 1024 (causal band)
  3. KV-cache decode,           64 sequences x 32 heads, d=128, lengths U[512, 8192]
  4. causal backward,           B=2, H=16, N=4096, d=128, bf16 (from the forward's O and L)
  5. paged KV-cache decode,     the decode batch of 3 in 64-token pages scattered over a pool
  6. causal forward in fp16,    the shape of 1 with fp16 inputs (same seeds)
  7. windowed decode,           the decode batch of 3 with a 1024-token sliding window
  8. windowed backward,         the backward of 4 with a 1024-token sliding window
  9. decode in fp16,            the decode batch of 3 with fp16 inputs (same seeds)
 10. backward in fp16,          the backward of 4 with fp16 inputs (same seeds)
 11. small forward,             B=1, H=8, N=1024, d=64, bf16, 64 x 64 tiles, full attention
 12. small causal forward,      the same, causal

The headline value is the causal forward's TFLOP/s (4*B*H*N^2*d/2 algorithmic
flops per launch over its median time per step); every stage is timed with HIP
events recorded on the stream the kernels run on, and each stage reports the
median, 10th and 90th percentile over the timed steps.  After the timed steps
the causal forward and the two small forwards are also timed back to back
(many launches between one pair of events, no event between launches).  The
GFX clock is sampled (amdsmi) while the steps run.  The fp64 oracle is timed
on the host on a bounded sample of the causal forward (a few heads) as the CPU
baseline.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
# Stages of one step, in the order they run.
STAGES = ("fwd", "window", "decode", "bwd", "paged", "fwd16", "decw", "bwdw", "dec16", "bwd16", "c2", "c2c")
# The float32 path, timed only when named in --stages: the causal forward and
# backward at the backward's shape (d = 128: the float32 MFMA kernels).
OPT_STAGES = ("fwd32", "bwd32", "bwdr")
PEAK_FP32_MFMA_TFLOPS = 157.3  # MI355X dense float32 MFMA
W_DEC = 1024   # sliding window of the windowed decode stage
W_BWD = 1024   # sliding window of the windowed backward stage


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def window_pairs(N, W):
    i = np.arange(N, dtype=np.int64)
    return int(np.minimum(i + 1, W + 1).sum())


def source_digest(names):
    """sha256 over the kernel sources a counter measurement was taken on."""
    import hashlib
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "tiled_attention_04_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel):
    """HBM bytes per launch from the committed counter runs (FETCH_SIZE +
    WRITE_SIZE, scaled by a plain copy kernel), or None if the kernel's
    sources changed since they were taken."""
    rec = traffic_record(kernel)
    return rec["bytes_per_launch"] if rec else None


def traffic_record(kernel):
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(kernel)
    except (OSError, ValueError):
        return None
    try:
        if not rec or rec.get("sources_sha256") != source_digest(rec["sources"]):
            return None
    except OSError:  # a source was renamed or removed since
        return None
    return rec


def traffic_note(kernel):
    rec = traffic_record(kernel)
    if rec is None:
        return "null: no counter run of the current kernel sources"
    return (f"stored, not measured in this run: rocprofv3 --pmc FETCH_SIZE then WRITE_SIZE per "
            f"dispatch, scaled by a plain copy's counts (profiles/traffic.json, kernel sources sha256 "
            f"{rec['sources_sha256']})")


class ClockSampler:
    """Samples the GPU's GFX clock on a background thread (amdsmi GPU
    metrics: the per-XCD current clocks when reported, else the current or
    average clock), tagging each sample with the phase the run is in."""

    def __init__(self, period_s=0.005):
        import threading
        self.period, self.samples, self.phase, self.source = period_s, [], None, None
        self._stop = threading.Event()
        self._thread = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            self._smi = amdsmi
            self._h = amdsmi.amdsmi_get_processor_handles()[0]
            if self._read() is None:
                self._smi = None
        except Exception as e:  # no amdsmi, no permission, no device: report without clocks
            self._smi = None
            self.error = f"{type(e).__name__}: {e}"
        if self._smi is not None:
            self._thread = threading.Thread(target=self._loop, daemon=True)
            self._thread.start()

    def _read(self):
        try:
            m = self._smi.amdsmi_get_gpu_metrics_info(self._h)
        except Exception as e:
            self.error = f"{type(e).__name__}: {e}"
            return None
        for key in ("current_gfxclks", "current_gfxclk", "average_gfxclk_frequency"):
            v = m.get(key)
            if isinstance(v, (list, tuple)):
                v = [x for x in v if isinstance(x, (int, float)) and 0 < x < 0xFFFF]
                if v:
                    self.source = f"amdsmi gpu_metrics {key} (mean over {len(v)} XCDs)"
                    return float(sum(v)) / len(v)
            elif isinstance(v, (int, float)) and 0 < v < 0xFFFF:
                self.source = f"amdsmi gpu_metrics {key}"
                return float(v)
        return None

    def _loop(self):
        while not self._stop.is_set():
            if self.phase is not None:
                v = self._read()
                if v is not None:
                    self.samples.append((self.phase, v))
            self._stop.wait(self.period)

    def stop(self):
        self._stop.set()
        if self._thread is not None:
            self._thread.join()

    def summary(self, phase):
        v = np.array([x for p, x in self.samples if p == phase])
        if self._smi is None:
            return {"available": False, "why": getattr(self, "error", "amdsmi unavailable")}
        if len(v) == 0:
            return {"available": True, "samples": 0}
        return {"median_mhz": float(np.median(v)), "min_mhz": float(v.min()), "max_mhz": float(v.max()),
                "samples": int(len(v)), "source": self.source}


def cpu_baseline(q, k, v, budget_s=12.0):
    """The oracle, as it stands, on whole heads of the causal forward."""
    import oracle
    from threadpoolctl import threadpool_info

    B, H, N, d = q.shape
    s = 1 / math.sqrt(d)
    flops_head = 4.0 * N * N * d / 2
    heads, t0 = 0, time.perf_counter()
    while True:
        b, h = divmod(heads, H)
        oracle.attention_ref(q[b, h][None], k[b, h][None], v[b, h][None], s, causal=True)
        heads += 1
        if time.perf_counter() - t0 >= budget_s or heads >= B * H:
            break
    dt = time.perf_counter() - t0
    info = [p for p in threadpool_info() if p.get("user_api") == "blas"]
    threads = max([p.get("num_threads", 1) for p in info] or [1])
    blas = ", ".join(f"{p.get('internal_api')} {p.get('version')} ({p.get('threading_layer')}, "
                     f"{p.get('num_threads')} threads)" for p in info) or "none found"
    return {"value": round(heads * flops_head / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle", "blas": blas, "host_cpus": len(os.sched_getaffinity(0)),
            "sample": f"{heads} of {B * H} (batch, head) slices of the causal N={N}, d={d} forward, "
                      f"fp64 NumPy, {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=15)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--stages", default=",".join(STAGES),
                    help="comma-separated stages; the default runs every stage of STAGES, the "
                         "float32 ones (" + ",".join(OPT_STAGES) + ") run only when named")
    ap.add_argument("--page-size", type=int, default=64)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after timing, copy 1 GiB device-to-device three times: the reference "
                         "kernel that scales the FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); every stage of this "
              "path is independent per (batch, head) and is not run across GPUs here.", file=sys.stderr)
        sys.exit(2)

    import torch

    import tiled_attention_04_amd as fa
    from tiled_attention_04_amd.inputs import (WORKLOADS, attention_inputs, decode_inputs, dense_cache,
                                              paged_cache)

    stages = args.stages.split(",")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    fa.lib()

    # ---- inputs -----------------------------------------------------------
    w3 = WORKLOADS["fwd_b4_h32_n4096_d128_bf16"]
    B3, H3, N3, d3 = w3["B"], w3["H"], w3["N"], w3["d"]
    log("generating forward inputs")
    q3c, k3c, v3c = attention_inputs(B3, H3, N3, d3, "bf16", seed=0)
    q3, k3, v3 = (t.to(dev) for t in (q3c, k3c, v3c))
    o3 = torch.empty_like(q3)
    l3 = torch.empty((B3, H3, N3), dtype=torch.float32, device=dev)
    o3w = torch.empty_like(q3)
    l3w = torch.empty_like(l3)
    if "fwd16" in stages:
        q7, k7, v7 = (t.to(dev) for t in attention_inputs(B3, H3, N3, d3, "fp16", seed=0))
        o7 = torch.empty_like(q7)
        l7 = torch.empty_like(l3)

    w4 = WORKLOADS["decode_s64_h32_d128_len512to8192_bf16"]
    if "decode" in stages or "paged" in stages or "decw" in stages:
        log("generating decode inputs (ragged KV cache)")
        inp4 = decode_inputs(w4["S"], w4["H"], w4["d"], w4["len_lo"], w4["len_hi"], seed=0)
        q4 = inp4.q.to(dev)
        sl4 = torch.from_numpy(inp4.seqlens).to(dev)
        o4 = torch.empty_like(q4)
        l4 = torch.empty(q4.shape[:2], dtype=torch.float32, device=dev)
        dec_bytes = inp4.valid_bytes(2) + 2 * q4.numel() * 2
        # with a window the query reads only the last W+1 rows of each cache
        seen = np.minimum(inp4.seqlens.astype(np.int64), W_DEC + 1)
        decw_bytes = int(seen.sum()) * w4["H"] * w4["d"] * 2 * 2 + 2 * q4.numel() * 2
    if "decode" in stages or "decw" in stages:
        kc4, vc4 = dense_cache(inp4, w4["Lmax"], device=dev)
        ws4 = torch.empty(fa.fa_decode_workspace_size(w4["S"], w4["H"], w4["Lmax"], w4["d"]),
                          dtype=torch.uint8, device=dev)
    if "paged" in stages:
        log(f"paging the decode cache ({args.page_size}-token pages)")
        kp6, vp6, tb6 = paged_cache(inp4, args.page_size, device=dev, seed=0)
        o6 = torch.empty_like(q4)
        l6 = torch.empty_like(l4)
        ws6 = torch.empty(fa.fa_decode_workspace_size(w4["S"], w4["H"], tb6.shape[1] * args.page_size,
                                                      w4["d"]), dtype=torch.uint8, device=dev)
    if "decode" in stages or "paged" in stages or "decw" in stages:
        del inp4
    if "dec16" in stages:
        inp8 = decode_inputs(w4["S"], w4["H"], w4["d"], w4["len_lo"], w4["len_hi"], dtype="fp16", seed=0)
        kc8, vc8 = dense_cache(inp8, w4["Lmax"], device=dev)
        q8 = inp8.q.to(dev)
        sl8 = torch.from_numpy(inp8.seqlens).to(dev)
        o8 = torch.empty_like(q8)
        l8 = torch.empty(q8.shape[:2], dtype=torch.float32, device=dev)
        ws8 = torch.empty(fa.fa_decode_workspace_size(w4["S"], w4["H"], w4["Lmax"], w4["d"]),
                          dtype=torch.uint8, device=dev)
        dec16_bytes = inp8.valid_bytes(2) + 2 * q8.numel() * 2
        del inp8

    w5 = WORKLOADS["bwd_b2_h16_n4096_d128_bf16"]
    B5, H5, N5, d5 = w5["B"], w5["H"], w5["N"], w5["d"]
    if "bwd" in stages:
        log("generating backward inputs")
        q5, k5, v5, g5 = (t.to(dev) for t in attention_inputs(B5, H5, N5, d5, "bf16", seed=0, with_grad=True))
        o5, l5 = fa.fa_fwd(q5, k5, v5, causal=True)
        dq5, dk5, dv5 = (torch.empty(q5.shape, dtype=torch.float32, device=dev) for _ in range(3))
    if "bwdw" in stages or "bwdr" in stages:
        if "bwd" not in stages:
            q5, k5, v5, g5 = (t.to(dev) for t in attention_inputs(B5, H5, N5, d5, "bf16", seed=0,
                                                                  with_grad=True))
            o5, l5 = fa.fa_fwd(q5, k5, v5, causal=True)
            dq5, dk5, dv5 = (torch.empty(q5.shape, dtype=torch.float32, device=dev) for _ in range(3))
    if "bwdw" in stages:
        o5w, l5w = fa.fa_fwd(q5, k5, v5, causal=True, window=W_BWD)
    if any(s_ in stages for s_ in ("bwd", "bwdw", "bwd16", "bwdr")):
        # The binding's default: dQ from the stored dS (0.54 GB of dS blocks for the causal
        # backward, which also covers the windowed one); the opt-in stage bwdr times the
        # recompute path with the minimum workspace.
        ws5 = torch.empty(fa.fa_bwd_default_workspace_size(B5, H5, N5, d5, True, -1), dtype=torch.uint8,
                          device=dev)
        ws5r = torch.empty(fa.fa_bwd_workspace_size(B5, H5, N5, d5), dtype=torch.uint8, device=dev)
    if "bwd16" in stages:
        q9, k9, v9, g9 = (t.to(dev) for t in attention_inputs(B5, H5, N5, d5, "fp16", seed=0, with_grad=True))
        o9, l9 = fa.fa_fwd(q9, k9, v9, causal=True)
        dq9, dk9, dv9 = (torch.empty(q9.shape, dtype=torch.float32, device=dev) for _ in range(3))
        ws9 = ws5

    if "fwd32" in stages or "bwd32" in stages:
        log("generating float32 inputs")
        q10, k10, v10, g10 = (t.to(dev) for t in attention_inputs(B5, H5, N5, d5, "fp32", seed=0,
                                                                  with_grad=True))
        o10, l10 = fa.fa_fwd(q10, k10, v10, causal=True)
        dq10, dk10, dv10 = (torch.empty_like(q10) for _ in range(3))
        ws10 = torch.empty(fa.fa_bwd_workspace_size(B5, H5, N5, d5), dtype=torch.uint8, device=dev)

    w2 = WORKLOADS["fwd_b1_h8_n1024_d64_bf16"]
    B2, H2, N2, d2, T2 = w2["B"], w2["H"], w2["N"], w2["d"], w2["block"]
    if "c2" in stages or "c2c" in stages:
        q2, k2, v2 = (t.to(dev) for t in attention_inputs(B2, H2, N2, d2, "bf16", seed=0))
        o2, o2c = torch.empty_like(q2), torch.empty_like(q2)
        l2 = torch.empty((B2, H2, N2), dtype=torch.float32, device=dev)
        l2c = torch.empty_like(l2)

    # ---- one step: every stage once, each bracketed by events -------------------
    flops3 = 4.0 * B3 * H3 * N3 * N3 * d3 / 2
    flops3w = 4.0 * d3 * B3 * H3 * window_pairs(N3, w3["window"])
    flops5 = 10.0 * B5 * H5 * N5 * N5 * d5 / 2
    flops5w = 10.0 * d5 * B5 * H5 * window_pairs(N5, W_BWD)
    flops2 = 4.0 * B2 * H2 * N2 * N2 * d2

    calls = {
        "fwd": lambda: fa.fa_fwd(q3, k3, v3, causal=True, o=o3, lse=l3),
        "window": lambda: fa.fa_fwd(q3, k3, v3, causal=True, window=w3["window"], o=o3w, lse=l3w),
        "decode": lambda: fa.fa_decode(q4, kc4, vc4, sl4, o=o4, lse=l4, workspace=ws4),
        "bwd": lambda: fa.fa_bwd(q5, k5, v5, o5, g5, l5, causal=True, dq=dq5, dk=dk5, dv=dv5,
                                 workspace=ws5),
        "paged": lambda: fa.fa_decode_paged(q4, kp6, vp6, tb6, sl4, o=o6, lse=l6, workspace=ws6),
        "fwd16": lambda: fa.fa_fwd(q7, k7, v7, causal=True, o=o7, lse=l7),
        "decw": lambda: fa.fa_decode(q4, kc4, vc4, sl4, window=W_DEC, o=o4, lse=l4, workspace=ws4),
        "bwdw": lambda: fa.fa_bwd(q5, k5, v5, o5w, g5, l5w, causal=True, window=W_BWD, dq=dq5, dk=dk5,
                                  dv=dv5, workspace=ws5),
        "dec16": lambda: fa.fa_decode(q8, kc8, vc8, sl8, o=o8, lse=l8, workspace=ws8),
        "bwd16": lambda: fa.fa_bwd(q9, k9, v9, o9, g9, l9, causal=True, dq=dq9, dk=dk9, dv=dv9,
                                   workspace=ws9),
        "bwdr": lambda: fa.fa_bwd(q5, k5, v5, o5, g5, l5, causal=True, dq=dq5, dk=dk5, dv=dv5,
                                  workspace=ws5r),
        "c2": lambda: fa.fa_fwd_ex(q2, k2, v2, T2, T2, o=o2, lse=l2),
        "c2c": lambda: fa.fa_fwd_ex(q2, k2, v2, T2, T2, causal=True, o=o2c, lse=l2c),
        "fwd32": lambda: fa.fa_fwd(q10, k10, v10, causal=True, o=o10, lse=l10),
        "bwd32": lambda: fa.fa_bwd(q10, k10, v10, o10, g10, l10, causal=True, dq=dq10, dk=dk10, dv=dv10,
                                   workspace=ws10),
    }
    unknown = [n for n in stages if n not in calls]
    if unknown:
        print(f"unknown stages: {', '.join(unknown)}", file=sys.stderr)
        sys.exit(2)
    run = [n for n in STAGES + OPT_STAGES if n in stages]

    def step(ev=None):
        for i, n in enumerate(run):
            if ev is not None:
                ev[i].record()
            calls[n]()
        if ev is not None:
            ev[len(run)].record()

    clock = ClockSampler()
    log(f"warmup {args.warmup} steps")
    clock.phase = "warmup"
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    log(f"timing {args.steps} steps")
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(run) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    clock.phase = "timed"
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    clock.phase = None
    comp = np.array([[events[i][j].elapsed_time(events[i][j + 1]) for j in range(len(run))]
                     for i in range(args.steps)])  # ms
    stats = {n: {"median": float(np.median(comp[:, j])), "p10": float(np.percentile(comp[:, j], 10)),
                 "p90": float(np.percentile(comp[:, j], 90)), "mean": float(comp[:, j].mean())}
             for j, n in enumerate(run)}
    ms = {n: st["median"] for n, st in stats.items()}
    log("stage ms (median [p10, p90]): " + ", ".join(
        f"{n}={st['median']:.4f} [{st['p10']:.4f}, {st['p90']:.4f}]" for n, st in stats.items()))

    # Back to back: many launches between one pair of events, so that no
    # event sits between two launches; the median over repetitions.
    b2b = {}
    clock.phase = "b2b"
    for n, launches in (("fwd", 20), ("c2", 200), ("c2c", 200)):
        if n not in run:
            continue
        pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(5)]
        for a, b in pairs:
            a.record()
            for _ in range(launches):
                calls[n]()
            b.record()
        torch.cuda.synchronize()
        per = np.array([a.elapsed_time(b) / launches for a, b in pairs])
        b2b[n] = {"ms_per_launch_median": float(np.median(per)), "min": float(per.min()),
                  "max": float(per.max()), "launches": launches, "repetitions": len(pairs)}
    clock.phase = None
    clock.stop()
    if b2b:
        log("back to back ms per launch (median): " + ", ".join(
            f"{n}={r['ms_per_launch_median']:.4f}" for n, r in b2b.items()))

    components = {}

    def stage_stats(key):
        st = stats[key]
        return {"ms": round(st["median"], 5), "ms_p10": round(st["p10"], 5), "ms_p90": round(st["p90"], 5),
                "ms_mean": round(st["mean"], 5)}

    def mfma_stage(name, flops, key, kernel):
        tf = flops / (ms[key] * 1e-3) / 1e12
        components[name] = {
            **stage_stats(key), "TFLOP/s": round(tf, 2), "algorithmic_tflop": round(flops / 1e12, 5),
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                         "traffic": measured_traffic(kernel)}}
        if key in b2b:
            t = b2b[key]["ms_per_launch_median"]
            components[name]["back_to_back"] = {**b2b[key], "TFLOP/s": round(flops / (t * 1e-3) / 1e12, 2)}

    def hbm_stage(name, nbytes, key, kernel):
        gbs = nbytes / (ms[key] * 1e-3) / 1e9
        components[name] = {
            **stage_stats(key), "GB/s": round(gbs, 1), "algorithmic_gb": round(nbytes / 1e9, 4),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": measured_traffic(kernel)}}

    if "fwd" in ms:
        mfma_stage("fwd_causal_b4_h32_n4096_d128", flops3, "fwd", "fwd_bf16_causal")
    if "window" in ms:
        mfma_stage("fwd_window1024_b4_h32_n4096_d128", flops3w, "window", "fwd_bf16_window")
    if "decode" in ms:
        hbm_stage("decode_s64_h32_d128_len512to8192", dec_bytes, "decode", "decode")
    if "bwd" in ms:
        mfma_stage("bwd_causal_b2_h16_n4096_d128", flops5, "bwd", "bwd_bf16")
    if "paged" in ms:
        hbm_stage(f"decode_paged{args.page_size}_s64_h32_d128_len512to8192", dec_bytes, "paged",
                  f"decode_paged{args.page_size}")
    if "fwd16" in ms:
        mfma_stage("fwd_causal_fp16_b4_h32_n4096_d128", flops3, "fwd16", "fwd_fp16_causal")
    if "decw" in ms:
        hbm_stage(f"decode_window{W_DEC}_s64_h32_d128_len512to8192", decw_bytes, "decw", "decode_window")
    if "bwdw" in ms:
        mfma_stage(f"bwd_window{W_BWD}_b2_h16_n4096_d128", flops5w, "bwdw", "bwd_bf16_window")
    if "dec16" in ms:
        hbm_stage("decode_fp16_s64_h32_d128_len512to8192", dec16_bytes, "dec16", "decode_fp16")
    if "bwd16" in ms:
        mfma_stage("bwd_causal_fp16_b2_h16_n4096_d128", flops5, "bwd16", "bwd_fp16")
    if "bwdr" in ms:
        mfma_stage("bwd_causal_recompute_dq_b2_h16_n4096_d128", flops5, "bwdr", None)
    # The small forward is cache-resident and launch-bound: reported as is,
    # not a roofline target.
    if "c2" in ms:
        mfma_stage(f"fwd_b1_h8_n1024_d64_tile{T2}", flops2, "c2", None)
    if "c2c" in ms:
        mfma_stage(f"fwd_causal_b1_h8_n1024_d64_tile{T2}", flops2 / 2, "c2c", None)

    # The float32 path at d = 128 runs on float32 MFMA: priced against its peak.
    for key, name, flops in (("fwd32", "fwd_causal_fp32_b2_h16_n4096_d128", flops5 * 0.4),
                             ("bwd32", "bwd_causal_fp32_b2_h16_n4096_d128", flops5)):
        if key in ms:
            tf = flops / (ms[key] * 1e-3) / 1e12
            components[name] = {
                **stage_stats(key), "TFLOP/s": round(tf, 2), "algorithmic_tflop": round(flops / 1e12, 5),
                "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_FP32_MFMA_TFLOPS,
                             "unit": "TFLOP/s", "frac": round(tf / PEAK_FP32_MFMA_TFLOPS, 4), "traffic": None}}

    if args.copy_calibration:
        log("copy calibration: 3 x 1 GiB device-to-device")
        src = torch.ones(1 << 29, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    value = flops3 / (ms["fwd"] * 1e-3) / 1e12 if "fwd" in ms else None
    (bq3, bk3), tuned3 = fa.fa_fwd_auto_tile(B3, H3, N3, d3, causal=True)
    kernel3 = (f"fwd_pingpong_kernel<bf16, {d3}>" if bq3 == 256 else
               f"fwd_mfma_kernel<bf16, {d3}, {bq3 // 32}, {bk3}>")
    kernel3 += (f" ({bq3} query rows x {bk3} keys per tile, "
                f"{'tuned' if tuned3 else 'heuristic'} choice)")
    result = {
        "metric": "causal fwd TFLOP/s & % bf16 MFMA peak (N=4096,d=128); decode % HBM BW",
        "value": round(value, 3) if value is not None else None,
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded N(0,1), rounded to bf16)",
        "config": {"workload": "causal forward B=4 H=32 N=4096 d=128 bf16 (step also runs: window-1024 "
                               "forward, 64x32 ragged decode d=128 lengths U[512,8192] from a dense and "
                               "from a 64-token paged cache and with a 1024 window, causal backward B=2 H=16 "
                               "N=4096 d=128 without and with a 1024 window, the causal forward, the decode "
                               "and the causal backward in fp16, and the B=1 H=8 N=1024 d=64 forward with "
                               "64x64 tiles, full and causal)",
                   "global_batch": B3, "seq_len": N3, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma", "achieved": round(value, 3) if value is not None else None,
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(value / PEAK_BF16_TFLOPS, 4) if value is not None else None,
                     "traffic": measured_traffic("fwd_bf16_causal"),
                     "kernel": kernel3, "time": "median over the timed steps of the stage's event pair",
                     "traffic_source": traffic_note("fwd_bf16_causal")},
        "gpu_clock": {"timed_steps": clock.summary("timed"), "back_to_back": clock.summary("b2b"),
                      "warmup": clock.summary("warmup")},
        "components": components,
    }
    if not args.no_cpu_baseline and "fwd" in stages:
        log("timing the fp64 oracle on the host (bounded sample)")
        result["cpu_baseline"] = cpu_baseline(q3c, k3c, v3c)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
