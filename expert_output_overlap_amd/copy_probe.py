"""A plain device-to-device copy of known size, for calibrating HBM byte counters.

Run under a counter profiler (FETCH_SIZE / WRITE_SIZE): each of the timed copies reads and writes exactly
``--mib`` MiB, so the counters' per-dispatch readings divided by that size give the factor that turns the same
counters' readings for another kernel into bytes.

    python -m expert_output_overlap_amd.copy_probe --mib 1024 --reps 5
"""
from __future__ import annotations

import argparse


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--mib", type=int, default=1024)
    ap.add_argument("--reps", type=int, default=5)
    args = ap.parse_args()
    import torch

    n = args.mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(args.reps):
        dst.copy_(src)
    ev1.record()
    ev1.synchronize()
    ms = ev0.elapsed_time(ev1) / args.reps
    print("copy %d MiB: %.3f ms, %.1f GB/s (read + write)" % (args.mib, ms, 2 * n / ms / 1e6))


if __name__ == "__main__":
    main()
