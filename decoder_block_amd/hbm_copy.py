"""Plain device-to-device copy of a known size, for scaling HBM traffic counters.

    python -m decoder_block_amd.hbm_copy [--mib 1024] [--reps 3]

Under ``rocprofv3 --pmc FETCH_SIZE`` (or ``WRITE_SIZE``) each copy dispatch
must read (write) exactly ``mib`` MiB; the ratio of that to the counter's
value is the factor that turns the counter into bytes for other kernels.
"""
from __future__ import annotations

import argparse


def main() -> None:
    import torch

    ap = argparse.ArgumentParser()
    ap.add_argument("--mib", type=int, default=1024)
    ap.add_argument("--reps", type=int, default=3)
    args = ap.parse_args()
    n = args.mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(args.reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"copied {args.mib} MiB x {args.reps}: {args.mib * (1 << 20)} bytes read and written per copy", flush=True)


if __name__ == "__main__":
    main()
