"""Sweep of the tuned choices on the measured workloads.

    python -m tiled_attention_04_amd.tune [--reps 20] [--save tuning.json]
    python -m tiled_attention_04_amd.tune --tile-grid [--reps 20]

Three tables (markdown), each setting the measured candidates beside the
built-in heuristic's choice:
  * the forward's tile (fa_fwd_tune: 32, 64 or 128 query rows with 32-, 64-
    or (at d = 64) 128-key tiles, and 256 x 64);
  * the decode's split length (fa_decode_tune: 256 to 4096 tokens);
  * the backward's dQ kernel (fa_bwd_tune: 128 or 256 query rows per
    workgroup).
With --tile-grid only the forward table is printed, over a grid of shapes
(d = 64 and 128, 1 x 8 x 64 to 4 x 32 x 4096, with and without windows):
the measurements the built-in tile choice rests on.
Every tuning call remembers its fastest candidate; with --save the choices
are written to a JSON file that a later process loads with ``load_tuning``
(no re-measuring).  Inputs are the seeded synthetic ones the tests and the
bench use.
"""

from __future__ import annotations

import argparse

import numpy as np
import torch

from . import fa355
from .inputs import attention_inputs, decode_inputs, dense_cache

# name, (B, H, N, d), dtype, causal, window
WORKLOADS = [
    ("causal 4x32x4096x128 bf16", (4, 32, 4096, 128), "bf16", True, -1),
    ("window-1024 4x32x4096x128 bf16", (4, 32, 4096, 128), "bf16", True, 1024),
    ("causal 4x32x4096x128 fp16", (4, 32, 4096, 128), "fp16", True, -1),
    ("causal 2x16x4096x128 bf16", (2, 16, 4096, 128), "bf16", True, -1),
    ("full 1x8x1024x64 bf16", (1, 8, 1024, 64), "bf16", False, -1),
    ("causal 1x8x1024x64 bf16", (1, 8, 1024, 64), "bf16", True, -1),
]

# name, (S, H, d, shortest, longest cache), dtype, window
DECODE_WORKLOADS = [
    ("ragged 64x32 d128 512-8192 bf16", (64, 32, 128, 512, 8192), "bf16", -1),
    ("ragged 64x32 d128 512-8192 window-1024 bf16", (64, 32, 128, 512, 8192), "bf16", 1024),
    ("ragged 8x8 d128 512-8192 bf16", (8, 8, 128, 512, 8192), "bf16", -1),
    ("ragged 64x32 d128 512-8192 fp16", (64, 32, 128, 512, 8192), "fp16", -1),
]

# name, (B, H, N, d), dtype, causal, window
BWD_WORKLOADS = [
    ("causal 2x16x4096x128 bf16", (2, 16, 4096, 128), "bf16", True, -1),
    ("window-1024 2x16x4096x128 bf16", (2, 16, 4096, 128), "bf16", True, 1024),
    ("causal 2x16x4096x128 fp16", (2, 16, 4096, 128), "fp16", True, -1),
    ("causal 1x8x1024x64 bf16", (1, 8, 1024, 64), "bf16", True, -1),
    ("full 1x8x1024x64 bf16", (1, 8, 1024, 64), "bf16", False, -1),
]


# The grid of --tile-grid: (B, H, N) for d = 64 and 128, causal and full,
# and causal with windows on a subset.
TILE_GRID_SHAPES = [(1, 8, 64), (1, 8, 256), (1, 8, 1024), (2, 8, 512), (1, 4, 4096), (1, 16, 2048),
                    (2, 16, 1024), (4, 16, 1024), (1, 32, 2048), (1, 64, 2048), (2, 16, 4096), (4, 32, 4096)]
TILE_GRID_WINDOWS = [((1, 8, 1024), (128, 512)), ((2, 16, 1024), (128, 512)), ((1, 4, 4096), (128, 512)),
                     ((2, 16, 4096), (256, 1024)), ((4, 32, 4096), (1024,))]


def tile_grid_workloads():
    out = []
    for d in (64, 128):
        for B, H, N in TILE_GRID_SHAPES:
            for causal in (False, True):
                out.append((f"{'causal' if causal else 'full'} {B}x{H}x{N}x{d} bf16", (B, H, N, d), "bf16", causal, -1))
        for (B, H, N), windows in TILE_GRID_WINDOWS:
            for w in windows:
                out.append((f"window-{w} {B}x{H}x{N}x{d} bf16", (B, H, N, d), "bf16", True, w))
    return out


def visible_pairs(N: int, causal: bool, window: int) -> int:
    i = np.arange(N, dtype=np.int64)
    hi = i + 1 if causal else np.full(N, N, dtype=np.int64)
    lo = np.maximum(0, i - window) if window >= 0 else np.zeros(N, dtype=np.int64)
    return int((hi - lo).sum())


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--reps", type=int, default=20)
    ap.add_argument("--save", default=None, help="write the tuned choices to this JSON file")
    ap.add_argument("--tile-grid", action="store_true", help="only the forward table, over a grid of shapes")
    args = ap.parse_args()
    dev = torch.device("cuda:0")
    print("| workload | " + " | ".join(f"{bq}x{bk} ms" for bq, bk in fa355.TUNE_CANDIDATES)
          + " | fastest | TFLOP/s | heuristic | heuristic ms | heuristic / fastest |")
    print("|---|" + "---|" * (len(fa355.TUNE_CANDIDATES) + 5))
    tuned = []
    for name, (B, H, N, d), dtype, causal, window in (tile_grid_workloads() if args.tile_grid else WORKLOADS):
        q, k, v = (t.to(dev) for t in attention_inputs(B, H, N, d, dtype, seed=0))
        fa355.fa_tune_reset()
        heur, _ = fa355.fa_fwd_auto_tile(B, H, N, d, causal=causal, window=window, dtype=q.dtype)
        best, times, _, _ = fa355.fa_fwd_tune(q, k, v, causal=causal, window=window, reps=args.reps)
        flops = 4.0 * d * B * H * visible_pairs(N, causal, window)
        tf = flops / (times[best] * 1e-3) / 1e12
        cells = " | ".join(f"{times[t]:.4f}" if times[t] >= 0 else "-" for t in fa355.TUNE_CANDIDATES)
        print(f"| {name} | {cells} | {best[0]}x{best[1]} | {tf:.1f} | {heur[0]}x{heur[1]} | {times[heur]:.4f} | "
              f"{times[heur] / times[best]:.2f} |", flush=True)
        tuned += fa355.fa_tune_export()
        del q, k, v
    if args.tile_grid:
        return

    print()
    print("| decode workload | " + " | ".join(f"{c} tok ms" for c in fa355.DECODE_TUNE_CANDIDATES)
          + " | fastest | TB/s | heuristic | heuristic ms |")
    print("|---|" + "---|" * (len(fa355.DECODE_TUNE_CANDIDATES) + 4))
    for name, (S, H, d, lo, hi), dtype, window in DECODE_WORKLOADS:
        inp = decode_inputs(S, H, d, lo, hi, dtype=dtype, seed=0)
        kc, vc = dense_cache(inp, hi, device=dev, fill=0.0)
        q, sl = inp.q.to(dev), torch.from_numpy(inp.seqlens).to(dev)
        fa355.fa_tune_reset()
        heur, _ = fa355.fa_decode_auto_chunk(S, H, hi, d, window=window, dtype=q.dtype)
        best, times, _, _ = fa355.fa_decode_tune(q, kc, vc, sl, window=window, reps=args.reps)
        if times.get(heur, -1) < 0:  # the heuristic's split is not a candidate: time it too
            ws = torch.empty(fa355.fa_decode_workspace_size(S, H, hi, d, 0), dtype=torch.uint8, device=dev)
            fa355.fa_decode(q, kc, vc, sl, window=window, chunk=heur, workspace=ws)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(args.reps):
                fa355.fa_decode(q, kc, vc, sl, window=window, chunk=heur, workspace=ws)
            e1.record()
            torch.cuda.synchronize()
            times[heur] = e0.elapsed_time(e1) / args.reps
        rows_read = np.minimum(inp.seqlens.astype(np.int64), window + 1 if window >= 0 else 1 << 62)
        nbytes = int(rows_read.sum()) * H * d * q.element_size() * 2
        tbs = nbytes / (times[best] * 1e-3) / 1e12
        cells = " | ".join(f"{times[c]:.4f}" if times[c] >= 0 else "-" for c in fa355.DECODE_TUNE_CANDIDATES)
        print(f"| {name} | {cells} | {best} | {tbs:.2f} | {heur} | {times[heur]:.4f} |", flush=True)
        tuned += fa355.fa_tune_export()
        del kc, vc, q

    print()
    def dq_name(r):
        return "stored dS" if r == fa355.FA_BWD_DQ_STORED else f"dQ {r} rows"

    print("| backward workload | " + " | ".join(f"{dq_name(r)} ms" for r in fa355.BWD_TUNE_CANDIDATES)
          + " | fastest | TFLOP/s | heuristic |")
    print("|---|" + "---|" * (len(fa355.BWD_TUNE_CANDIDATES) + 3))
    for name, (B, H, N, d), dtype, causal, window in BWD_WORKLOADS:
        q, k, v, g = (t.to(dev) for t in attention_inputs(B, H, N, d, dtype, seed=0, with_grad=True))
        o, lse = fa355.fa_fwd(q, k, v, causal=causal, window=window)
        fa355.fa_tune_reset()
        heur, _ = fa355.fa_bwd_auto_dq_rows(B, H, N, d, causal=causal, window=window, dtype=q.dtype)
        best, times, _ = fa355.fa_bwd_tune(q, k, v, o, g, lse, causal=causal, window=window, reps=args.reps)
        flops = 10.0 * d * B * H * visible_pairs(N, causal, window)
        tf = flops / (times[best] * 1e-3) / 1e12
        cells = " | ".join(f"{times[r]:.4f}" if times[r] >= 0 else "-" for r in fa355.BWD_TUNE_CANDIDATES)
        print(f"| {name} | {cells} | {dq_name(best)} | {tf:.1f} | {dq_name(heur)} |", flush=True)
        tuned += fa355.fa_tune_export()
        del q, k, v, g, o, lse

    if args.save:
        fa355.fa_tune_reset()
        fa355.fa_tune_import(tuned)
        fa355.save_tuning(args.save)


if __name__ == "__main__":
    main()
