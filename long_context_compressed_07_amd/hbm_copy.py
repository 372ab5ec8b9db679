"""HBM traffic calibration for hardware-counter runs.

`python -m long_context_compressed_07_amd.hbm_copy` copies a 1 GiB device buffer into another one
a few times with torch's device-to-device copy (one copy kernel per call, reading and writing
exactly 2^30 bytes). Under `rocprofv3 --pmc FETCH_SIZE` (then `WRITE_SIZE`) the counters those
dispatches report give the factor that turns the same counters of another kernel into HBM bytes.
"""
import sys

import torch

NBYTES = 1 << 30


def main(copies: int = 4) -> None:
    x = torch.ones(NBYTES // 4, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    for _ in range(copies):
        y.copy_(x)
    torch.cuda.synchronize()
    print(f"copied {NBYTES} bytes {copies} times", flush=True)


if __name__ == "__main__":
    main(int(sys.argv[1]) if len(sys.argv) > 1 else 4)
