"""Plain device-to-device copy of a known size, for scaling HBM traffic counters.

    python -m decoder_block_amd.hbm_copy [--mib 1024] [--reps 3]
    python -m decoder_block_amd.hbm_copy --time [--mib 64] [--reps 15]

Under ``rocprofv3 --pmc FETCH_SIZE`` (or ``WRITE_SIZE``) each copy dispatch
must read (write) exactly ``mib`` MiB; the ratio of that to the counter's
value is the factor that turns the counter into bytes for other kernels.

``--time``: the rate of a device-to-device copy of ``mib`` MiB (bytes read plus
bytes written over the copy's time, HIP events, median of ``reps``), once right
after a 1 GiB copy that evicts the last-level cache and leaves it dirty, once
back to back (the source may then sit in that cache): the reference rate for
kernels that, like the RMSNorm passes, read a tensor once and write one.
"""
from __future__ import annotations

import argparse


def time_copy(mib: int, reps: int) -> None:
    import statistics

    import torch

    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    big = torch.ones((1 << 30) // 4, dtype=torch.float32, device="cuda")
    big2 = torch.empty_like(big)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for flush in (True, False):
        ts = []
        for _ in range(reps + 1):
            if flush:
                big2.copy_(big)
            e0.record()
            dst.copy_(src)
            e1.record()
            e1.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3)
        us = statistics.median(ts[1:])
        gbs = 2 * mib * (1 << 20) / (us * 1e-6) / 1e9
        what = "after a 1 GiB copy" if flush else "back to back"
        print(f"copy {mib} MiB {what}: {us:.1f} us, {gbs:.0f} GB/s (read + written)", flush=True)


def main() -> None:
    import torch

    ap = argparse.ArgumentParser()
    ap.add_argument("--mib", type=int, default=1024)
    ap.add_argument("--reps", type=int, default=3)
    ap.add_argument("--time", action="store_true")
    args = ap.parse_args()
    if args.time:
        time_copy(args.mib, args.reps)
        return
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
