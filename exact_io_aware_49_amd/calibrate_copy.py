"""Plain device-to-device copy of a known size, for calibrating HBM byte counters.

    rocprofv3 --pmc FETCH_SIZE -- python3 -m exact_io_aware_49_amd.calibrate_copy
    rocprofv3 --pmc WRITE_SIZE -- python3 -m exact_io_aware_49_amd.calibrate_copy

Copies a 512 MiB buffer three times; each copy reads and writes exactly
536,870,912 bytes, so counter value / true bytes gives the scale factor.
"""

import torch

MIB = 1 << 20


def main(mib: int = 512, reps: int = 3):
    a = torch.ones(mib * MIB // 2, dtype=torch.bfloat16, device="cuda")
    b = torch.empty_like(a)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(f"copied {mib} MiB x{reps}", flush=True)


if __name__ == "__main__":
    main()
