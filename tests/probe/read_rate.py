"""HBM read-stream rate: a 4 GiB buffer read once per launch by 256-thread
workgroups, each streaming one contiguous span with 16-byte loads (eight per
lane in flight), with and without the non-temporal hint, for several grid
sizes.  Prints TB/s (bytes read / launch time, mean of 10 launches).

Usage (needs a GPU; tests/probe/libmfma_block.so built by the build step):
    python tests/probe/read_rate.py
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))


def main():
    import torch
    L = ctypes.CDLL(os.path.join(HERE, "libmfma_block.so"))
    L.hbm_read_run.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                               ctypes.c_void_p]
    nbytes = 4 << 30
    buf = torch.randint(0, 255, (nbytes,), dtype=torch.uint8, device="cuda:0")
    out = torch.zeros(1 << 16, dtype=torch.int32, device="cuda:0")
    stream = torch.cuda.current_stream()
    for blocks in (1024, 4096, 16384, 65536):
        for nt in (0, 1):
            args = (buf.data_ptr(), nbytes, blocks, nt, out.data_ptr(), stream.cuda_stream)
            assert L.hbm_read_run(*args) == 0
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(10):
                L.hbm_read_run(*args)
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / 10
            print(f"workgroups {blocks:6d}  non-temporal {nt}:  {ms:.3f} ms  {nbytes / ms / 1e9:.2f} TB/s",
                  flush=True)


if __name__ == "__main__":
    main()
