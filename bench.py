#!/usr/bin/env python3
"""Benchmark of the fused MoE layer on one MI355X.

One step = one moe_fused_forward_prepacked call over the whole batch of the
workload: dispatch (routing histogram, prefix sum, stable rank, gather + e4m3
quantisation) -> L1 grouped GEMM with the SwiGLU*w / e4m3 epilogue -> L2
grouped GEMM -> combine.  Inputs are seeded synthetic tensors already resident
in HBM when the timed region starts.  The weights are laid out once before
timing (moe_pack_weights: FP4 codes tile-blocked, scales packed; weights are
constant across calls, and the pages' fused entry also takes pre-transformed
weights); the same number of steps of moe_fused_forward, which takes the
weights as given and re-lays the scales every call, is timed after the main
region and reported as ms_per_step_canonical.  --weights packed-scales times
moe_fused_forward_packed (codes as given, scales packed once), --weights
canonical times moe_fused_forward.

Prints ONE JSON line (rank 0):
  value        whole-layer TFLOP/s = 6*R*H*I / step time (R = routed rows)
  routed_rows_per_s
  roofline     the dominant kernel (the L1 GEMM), its average duration from
               HIP events on its stream (recorded by the library around each
               launch over a second run of the same number of steps; the
               first, timed run has none), against whichever bound its
               algorithmic work meets first: FLOP per launch against the FP8
               dense MFMA peak (the FP8 x FP4 scaled MFMA runs at the FP8
               rate), or algorithmic bytes per launch (experts' W1 and its
               scales once, token codes once, routed rows' A-scale words,
               activations written) against HBM bandwidth
  cpu_baseline the CPU oracle on a bounded sample of the same workload
"""
from __future__ import annotations

import argparse
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused MoE layer TFLOPS (% of FP8/FP4 MFMA peak) + routed rows/s, 1 GPU"
PEAK_TFLOPS = 5000.0      # MI355X dense FP8 MFMA (published)
PEAK_HBM_GBS = 8000.0     # MI355X HBM3E (published)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--warmup-ms", type=float, default=1500.0,
                   help="keep warming up (whole steps) until at least this much GPU time has run, "
                        "so that the timed steps start at steady clocks")
    p.add_argument("--workload", default="prefill",
                   help="tiny | small | prefill | skewed | many")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="target CPU time of the oracle baseline sample (0 = skip)")
    p.add_argument("--weights", choices=("prepacked", "packed-scales", "canonical"), default="prepacked",
                   help="prepacked: codes and scales laid out once before timing (moe_pack_weights, "
                        "default); packed-scales: scales laid out once, codes as given; canonical: "
                        "moe_fused_forward re-lays the scales every step")
    p.add_argument("--graph", action="store_true",
                   help="also capture one moe_fused_forward_packed step into a HIP graph and report the replayed step "
                        "time (ms_per_step_graph) beside the main number")
    p.add_argument("--gemm-tiles", choices=("auto", "persistent", "64", "128", "fused"), default="auto",
                   help="which grouped-GEMM kernels the layer runs (moe_options_t.gemm_tiles); "
                        "auto: the library's choice by shape")
    p.add_argument("--copy-mib", type=int, default=0,
                   help="after the timed region, run one plain device-to-device copy of this "
                        "many MiB (the known-size kernel that scales the HBM byte counters)")
    return p.parse_args()


# Bytes the L1 GEMM moves across its XCDs' L2 boundary per launch (reads
# that leave the L2 for the fabric -- Infinity Cache hits included -- plus
# writes), from two rocprofv3 --pmc passes (FETCH_SIZE, WRITE_SIZE) scaled by
# a plain copy of known size.  This is an upper bound on its HBM bytes, not
# HBM bytes themselves.  One summary per workload; each names the sha256 of
# the GEMM sources it was measured on, and a changed kernel reports null.
def traffic_summary(workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"gemm_l1_{workload}_hbm_traffic.md")



GEMM_SOURCES = ("combine_dispatch_amd/csrc/gemm.hip", "combine_dispatch_amd/csrc/moe_kernels.hpp",
                "combine_dispatch_amd/csrc/moe_device.hpp")


def gemm_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in GEMM_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload: str):
    path = traffic_summary(workload)
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        m = re.match(r"^\s*-?\s*`?([a-z0-9_]+)`?\s*:\s*`?([0-9a-f.]+)`?\s*$", line)
        if m:
            fields[m.group(1)] = m.group(2)
    if fields.get("gemm_source_sha256") != gemm_source_hash():
        return None
    try:
        return int(float(fields["fabric_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {a.gpus} is not supported "
              "(multi-GPU expert parallelism is a design note, not built)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import combine_dispatch_amd as moe
    import moe_inputs

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    moe.lib()  # loud failure if the HIP library is missing

    cfg = moe_inputs.CONFIG_BY_NAME[a.workload]
    t0 = time.time()
    inp = moe_inputs.config_inputs(a.workload)
    gen_s = time.time() - t0
    T, H, I, E, K = (inp[k] for k in ("T", "H", "I", "E", "K"))
    R = int((inp["topk_idx"] >= 0).sum())
    dev = "cuda:0"

    def up(arr):
        if arr.dtype == np.uint16:
            arr = arr.view(np.int16)
        return torch.from_numpy(np.ascontiguousarray(arr)).to(dev)

    d = {k: up(inp[k]) for k in ("x", "topk_idx", "topk_w", "W1q", "S1", "W2q", "S2")}
    ws = torch.empty(moe.moe_workspace_bytes(T, H, I, E, K), dtype=torch.uint8, device=dev)
    y = torch.empty((T, H), dtype=torch.int16, device=dev)
    stream = torch.cuda.current_stream()
    packed = torch.empty(moe.moe_packed_scales_bytes(H, I, E), dtype=torch.uint8, device=dev)
    moe.moe_pack_weight_scales(d["S1"], d["S2"], packed, E=E, H=H, I=I, stream=stream)
    prepacked = torch.empty(moe.moe_packed_weights_bytes(H, I, E), dtype=torch.uint8, device=dev)
    moe.moe_pack_weights(d["W1q"], d["S1"], d["W2q"], d["S2"], prepacked, E=E, H=H, I=I, stream=stream)

    opts = moe.options(gemm_tiles={"auto": moe.MOE_TILES_AUTO, "persistent": moe.MOE_TILES_PERSISTENT,
                                   "64": moe.MOE_TILES_64, "128": moe.MOE_TILES_128,
                                   "fused": moe.MOE_TILES_FUSED}[a.gemm_tiles])

    def call(mode, st):
        if mode == "prepacked":
            moe.moe_fused_forward_prepacked(d["x"], d["topk_idx"], d["topk_w"], prepacked, y, ws, E=E, I=I,
                                            opts=opts, stream=st)
        elif mode == "packed-scales":
            moe.moe_fused_forward_packed(d["x"], d["topk_idx"], d["topk_w"], d["W1q"], d["W2q"],
                                         packed, y, ws, opts=opts, E=E, I=I, stream=st)
        else:
            moe.moe_fused_forward(d["x"], d["topk_idx"], d["topk_w"], d["W1q"], d["S1"], d["W2q"],
                                  d["S2"], y, ws, opts=opts, E=E, I=I, stream=st)

    other_mode = "canonical" if a.weights != "canonical" else "prepacked"
    step = lambda: call(a.weights, stream)
    other = lambda: call(other_mode, stream)

    # warm-up: at least `warmup` steps and at least `warmup_ms` of GPU time
    # (the clocks take a few hundred milliseconds of load to settle)
    warm_steps = 0
    w0 = time.perf_counter()
    while True:
        for _ in range(max(a.warmup, 1)):
            step()
        warm_steps += max(a.warmup, 1)
        torch.cuda.synchronize()
        if warm_steps >= a.warmup and (time.perf_counter() - w0) * 1e3 >= a.warmup_ms:
            break
    warm_s = time.perf_counter() - w0

    # timed region: exactly `steps` whole-layer steps, nothing else on the
    # stream between them
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(a.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = ev0.elapsed_time(ev1) / a.steps

    # per-kernel durations: the same number of steps again, with the library
    # recording a HIP event on the launch stream around each of its launches.
    # An event between two launches delays the second by a few microseconds,
    # so this region's step time is reported separately and not as `value`.
    ep0, ep1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    moe.moe_profile_start(a.steps)
    ep0.record(stream)
    for _ in range(a.steps):
        step()
    ep1.record(stream)
    torch.cuda.synchronize()
    ms_per_step_events = ep0.elapsed_time(ep1) / a.steps
    stage_ms, ncalls = moe.moe_profile_stop()
    per_launch = {k: v / max(ncalls, 1) for k, v in stage_ms.items()}

    # the other scale path, same step count, outside the main region
    eo0, eo1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    other()
    eo0.record(stream)
    for _ in range(a.steps):
        other()
    eo1.record(stream)
    torch.cuda.synchronize()
    other_ms = eo0.elapsed_time(eo1) / a.steps

    # one more step with cold caches: a 512 MiB scrub (twice the 256 MB
    # infinity cache) right before it; reported beside the warm number
    scrub = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    scrub.fill_(3)
    ec0, ec1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ec0.record(stream)
    step()
    ec1.record(stream)
    torch.cuda.synchronize()
    cold_ms = ec0.elapsed_time(ec1)
    del scrub

    graph_ms = None
    if a.graph:
        # one step captured into a HIP graph (the library allocates, sets and
        # synchronises nothing, and takes every size from the device), then
        # the same number of replays timed
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        with torch.cuda.stream(cap):
            call(a.weights, cap)
        stream.wait_stream(cap)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            call(a.weights, torch.cuda.current_stream())
        for _ in range(3):
            graph.replay()
        torch.cuda.synchronize()
        eg0, eg1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        eg0.record(stream)
        for _ in range(a.steps):
            graph.replay()
        eg1.record(stream)
        torch.cuda.synchronize()
        graph_ms = eg0.elapsed_time(eg1) / a.steps
        del graph

    if a.copy_mib > 0:
        n = a.copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    flop = 6.0 * R * H * I
    tflops = flop / (ms_per_step * 1e-3) / 1e12
    rows_s = R / (ms_per_step * 1e-3)
    l1_flop = 4.0 * R * H * I
    l2_flop = 2.0 * R * I * H
    l1_s = per_launch["gemm_l1"] * 1e-3
    l1_tflops = l1_flop / l1_s / 1e12
    # the library's GEMMs with 64-row tiles serve batches with at most 64
    # routed slots per expert on average
    l1_kernel = {"64": "gemm_l1_decode", "128": "gemm_l1_t128", "persistent": "gemm_l1"}.get(
        a.gemm_tiles, "gemm_l1_decode" if T * K <= 64 * E else "gemm_l1")
    if l1_kernel == "gemm_l1_decode" and a.weights == "prepacked":
        l1_kernel = "gemm_l1_decode_nt"  # its variant for tile-blocked weights
    # L1 algorithmic bytes: W1 codes and scales of every expert that holds a
    # routed row, the token rows' codes once, the A-scale words (by token in
    # the 64-row-tile GEMM up to 1024 routed slots, else per routed row), each
    # routed row's weight and token index, the e4m3 activations and their
    # scales
    experts_used = int(np.unique(inp["topk_idx"][inp["topk_idx"] >= 0]).size)
    a_scale_rows = T if (l1_kernel.startswith("gemm_l1_decode") and T * K <= 1024) else R
    l1_bytes = (experts_used * 2 * I * (H // 2 + H // 32) + T * H + a_scale_rows * (H // 32) + R * 8
                + R * (I + I // 32))
    if a.gemm_tiles == "fused":
        # L1 and L2 in one launch (the L2 stage is empty): both GEMMs' FLOP;
        # bytes = both weights of the experts in use, the token codes, the
        # A-scale words, weights and token indices, the bf16 L2 rows written
        l1_kernel = "gemm_fused"
        l1_flop = l1_flop + l2_flop
        l1_bytes = (experts_used * 3 * I * (H // 2 + H // 32) + T * H + R * (H // 32 + 8) + R * H * 2)
        l1_tflops = l1_flop / l1_s / 1e12
    l1_bound = "mfma" if l1_flop / PEAK_TFLOPS >= l1_bytes / PEAK_HBM_GBS * 1e3 else "hbm"
    l1_gbs = l1_bytes / l1_s / 1e9
    l2_tflops = None if a.gemm_tiles == "fused" else l2_flop / (per_launch["gemm_l2"] * 1e-3) / 1e12
    # algorithmic bytes of the bandwidth-bound kernels (see the design notes):
    # dispatch = x read, token-major codes and scale words written, topk_idx
    # read by the histogram in the same launch; pool scales = the pool rows'
    # scale words gathered (read and written) by their token index
    disp_bytes = T * H * 2 + T * (H + H // 32) + 8 * T * K
    pool_s_bytes = 2 * R * (H // 32) + 4 * R
    comb_bytes = R * H * 2 + T * H * 2 + T * K * 4

    traffic = None if a.gemm_tiles == "fused" else measured_traffic(a.workload)
    roofline = {"bound": l1_bound, "kernel": l1_kernel}
    if l1_bound == "mfma":
        roofline.update(achieved=round(l1_tflops, 2), peak=PEAK_TFLOPS, unit="TFLOP/s",
                        frac=round(l1_tflops / PEAK_TFLOPS, 4))
    else:
        roofline.update(achieved=round(l1_gbs, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                        frac=round(l1_gbs / PEAK_HBM_GBS, 4))
    roofline.update(traffic=traffic, algorithmic_flop_per_launch=l1_flop,
                    algorithmic_bytes_per_launch=l1_bytes,
                    traffic_kind="bytes across the XCD L2 boundary per launch (FETCH_SIZE x2 + "
                                 "WRITE_SIZE, Infinity Cache hits included): an upper bound on HBM bytes")

    out = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "warmup_steps_run": warm_steps,
        "warmup_s": round(warm_s, 3),
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3 x fp4_e2m1 (ue8m0/32), fp32 accumulate",
        "data": "synthetic (seeded; see moe_inputs)",
        "config": {"workload": f"{a.workload}: T={T} H={H} I={I} E={E} K={K} routing={cfg['routing']}",
                   "T": T, "H": H, "I": I, "E": E, "K": K, "routed_rows": R,
                   "weights": {"prepacked": "codes tile-blocked and scales packed once before timing "
                                            "(moe_pack_weights)",
                               "packed-scales": "codes as given, scales packed once before timing "
                                                "(moe_pack_weight_scales)",
                               "canonical": "as given, scales re-laid every step"}[a.weights],
                   "parallelism": "single GPU, all experts local", "gemm_tiles": a.gemm_tiles},
        "routed_rows_per_s": round(rows_s, 1),
        "frac_of_fp8_peak": round(tflops / PEAK_TFLOPS, 4),
        "roofline": roofline,
        "kernels_ms_per_launch": {k: round(v, 4) for k, v in per_launch.items()},
        "ms_per_step_with_kernel_events": round(ms_per_step_events, 4),
        "kernels": {
            "gemm_l2_tflops": None if l2_tflops is None else round(l2_tflops, 2),
            "dispatch_gbs": round(disp_bytes / (per_launch["dispatch"] * 1e-3) / 1e9, 1),
            "pool_scales_gbs": round(pool_s_bytes / (per_launch["pool_scales"] * 1e-3) / 1e9, 1),
            "combine_gbs": round(comb_bytes / (per_launch["combine"] * 1e-3) / 1e9, 1),
            "hbm_peak_gbs": PEAK_HBM_GBS,
        },
        f"ms_per_step_{other_mode}": round(other_ms, 4),
        "cold_ms_per_step": round(cold_ms, 4),
        **({"ms_per_step_graph": round(graph_ms, 4)} if graph_ms is not None else {}),
        "wall_s_timed": round(wall, 4),
        "input_gen_s": round(gen_s, 2),
    }

    if a.cpu_seconds > 0:
        out["cpu_baseline"] = cpu_baseline(inp, a.cpu_seconds)
    print(json.dumps(out), flush=True)
    return 0


def cpu_baseline(inp, budget_s: float) -> dict:
    """The CPU oracle, as it stands, on a bounded sample of the same workload:
    whole tokens (all their routes) until the time budget is spent."""
    import numpy as np

    import oracle
    T, H, I, K = inp["T"], inp["H"], inp["I"], inp["K"]
    rng = np.random.default_rng(12345)
    order = rng.permutation(T)
    done_tok, routes = 0, 0
    t0 = time.perf_counter()
    for t in order:
        oracle.forward_tokens(inp, [int(t)])
        done_tok += 1
        routes += int((inp["topk_idx"][t] >= 0).sum())
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    flop = 6.0 * routes * H * I
    return {"value": round(flop / el / 1e12, 6), "unit": "TFLOP/s",
            "routed_rows_per_s": round(routes / el, 3), "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"{done_tok} whole tokens ({routes} routed rows) of the same workload, drawn "
                      f"at random, each through the oracle's per-token path (quantise, L1, "
                      f"SwiGLU*w, requant, L2 per route, fp32 combine; the same arithmetic as its "
                      f"grouped path), {el:.1f} s; rate scaled to the workload by routed rows",
            "threads_kind": "OpenMP threads of the oracle's parallel loops",
            "nproc": len(os.sched_getaffinity(0)), "cpu_model": cpu_model()}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


if __name__ == "__main__":
    sys.exit(main())
