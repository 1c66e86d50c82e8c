"""Dense throughput of v_mfma_scale_f32_32x32x64_f8f6f4 with register-resident
operands on the whole GPU (one 256-thread workgroup per CU, 8 independent
accumulator chains per wave): e4m3 x e2m1 and e4m3 x e4m3, with
one constant byte pattern or with pseudo-random operands that change from
one MFMA to the next.  Prints PFLOP/s (2 * 32 * 32 * 64 per MFMA).

Usage (needs a GPU; tests/probe/libmfma_block.so built by the build step):
    python tests/probe/mfma_rate.py [--iters N]
"""
from __future__ import annotations

import argparse
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--iters", type=int, default=20000)  # a multiple of 4
    ap.add_argument("--repeats", type=int, default=5)
    a = ap.parse_args()
    import torch
    L = ctypes.CDLL(os.path.join(HERE, "libmfma_block.so"))
    L.mfma_rate_run.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    L.mfma_rate_run.restype = ctypes.c_float
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    out = torch.empty(cus * 256, dtype=torch.float32, device="cuda:0")
    flop = 2.0 * 32 * 32 * 64 * 8 * 4 * cus * a.iters  # per launch: 8 chains x 4 waves x CUs
    for fmt_b, name in ((4, "e4m3 x e2m1"), (0, "e4m3 x e4m3")):
        for random in (0, 1):
            L.mfma_rate_run(fmt_b, random, 200, cus, ctypes.c_void_p(out.data_ptr()))  # warm-up
            best = None
            for _ in range(a.repeats):
                ms = L.mfma_rate_run(fmt_b, random, a.iters, cus, ctypes.c_void_p(out.data_ptr()))
                assert ms > 0, ms
                best = ms if best is None else min(best, ms)
            print(f"{name:12s} {'random' if random else 'constant':8s} operands: "
                  f"{flop / (best * 1e-3) / 1e15:.3f} PFLOP/s ({best:.2f} ms for {a.iters} rounds on "
                  f"{cus} CUs)", flush=True)


if __name__ == "__main__":
    main()
