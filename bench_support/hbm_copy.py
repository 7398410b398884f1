"""A plain device copy of a known byte count, for calibrating HBM byte counters.

rocprofv3's FETCH_SIZE and WRITE_SIZE report the bytes a kernel moved between
the L2 caches and memory.  Running this script under the same counters gives
the factor between what they read and the true byte count of a kernel that
reads every input byte once and writes every output byte once; the attention
kernels' counter readings are scaled by that factor.

    python3 hbm_copy.py [--mib N] [--reps R]

The copy is an elementwise negation of float32 data (one read and one write
per element, no reuse), launched R times on fresh buffers much larger than the
caches.  Prints one JSON line with the bytes read and written per launch.
"""
import argparse
import json

import torch


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--mib", type=int, default=4096, help="bytes read (and written) per launch")
    ap.add_argument("--reps", type=int, default=3)
    args = ap.parse_args()
    n = args.mib * (1 << 20) // 4
    src = torch.empty(n, dtype=torch.float32, device="cuda").uniform_()
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    times = []
    for _ in range(args.reps):
        a.record()
        torch.neg(src, out=dst)
        b.record()
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    nbytes = 4 * n
    best = min(times)
    print(json.dumps({"kernel": "elementwise neg (copy)", "read_bytes": nbytes,
                      "write_bytes": nbytes, "reps": args.reps, "best_ms": round(best, 4),
                      "GB/s": round(2 * nbytes / (best * 1e-3) / 1e9, 1)}), flush=True)


if __name__ == "__main__":
    main()
