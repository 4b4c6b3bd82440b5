"""Sweep of the forward's query-tile sizes on the measured workloads.

    python -m tiled_attention_04_amd.tune [--reps 20] [--save tuning.json]

For each workload, fa_fwd_tune times every tile (32, 64, 128 and 256 query
rows; 64-key tiles) on the GPU and remembers the fastest; the table printed
here (markdown) sets those times beside the built-in heuristic's choice.
With --save the choices are written to a JSON file that a later process
loads with ``load_tuning`` (no re-measuring).
Inputs are the seeded synthetic ones the tests and the bench use.
"""

from __future__ import annotations

import argparse

import numpy as np
import torch

from . import fa355
from .inputs import attention_inputs

# name, (B, H, N, d), dtype, causal, window
WORKLOADS = [
    ("causal 4x32x4096x128 bf16", (4, 32, 4096, 128), "bf16", True, -1),
    ("window-1024 4x32x4096x128 bf16", (4, 32, 4096, 128), "bf16", True, 1024),
    ("causal 4x32x4096x128 fp16", (4, 32, 4096, 128), "fp16", True, -1),
    ("causal 2x16x4096x128 bf16", (2, 16, 4096, 128), "bf16", True, -1),
    ("full 1x8x1024x64 bf16", (1, 8, 1024, 64), "bf16", False, -1),
    ("causal 1x8x1024x64 bf16", (1, 8, 1024, 64), "bf16", True, -1),
]


def visible_pairs(N: int, causal: bool, window: int) -> int:
    i = np.arange(N, dtype=np.int64)
    hi = i + 1 if causal else np.full(N, N, dtype=np.int64)
    lo = np.maximum(0, i - window) if window >= 0 else np.zeros(N, dtype=np.int64)
    return int((hi - lo).sum())


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--reps", type=int, default=20)
    ap.add_argument("--save", default=None, help="write the tuned choices to this JSON file")
    args = ap.parse_args()
    dev = torch.device("cuda:0")
    print("| workload | " + " | ".join(f"{b} rows ms" for b in fa355.TUNE_CANDIDATES)
          + " | fastest | TFLOP/s | heuristic | heuristic ms |")
    print("|---|" + "---|" * (len(fa355.TUNE_CANDIDATES) + 4))
    tuned = []
    for name, (B, H, N, d), dtype, causal, window in WORKLOADS:
        q, k, v = (t.to(dev) for t in attention_inputs(B, H, N, d, dtype, seed=0))
        fa355.fa_tune_reset()
        heur, _ = fa355.fa_fwd_auto_block_q(B, H, N, d, causal=causal, window=window, dtype=q.dtype)
        best, times, _, _ = fa355.fa_fwd_tune(q, k, v, causal=causal, window=window, reps=args.reps)
        flops = 4.0 * d * B * H * visible_pairs(N, causal, window)
        tf = flops / (times[best] * 1e-3) / 1e12
        cells = " | ".join(f"{times[b]:.4f}" for b in fa355.TUNE_CANDIDATES)
        print(f"| {name} | {cells} | {best} | {tf:.1f} | {heur} | {times[heur]:.4f} |", flush=True)
        tuned += fa355.fa_tune_export()
        del q, k, v
    if args.save:
        fa355.fa_tune_reset()
        fa355.fa_tune_import(tuned)
        fa355.save_tuning(args.save)


if __name__ == "__main__":
    main()
