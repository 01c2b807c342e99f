"""Streaming-read probe: per-workgroup and whole-grid read bandwidth of the two load forms the
decode kernel streams weights with (16-byte non-temporal register loads with DEPTH in flight per
lane, and 16-byte LDS DMA copies through an 8-slot ring), for several grid sizes.

python -m persistent_moe_decode_amd.probe.stream_probe [--quick]

Each workgroup (512 threads, one per compute unit) reads a disjoint range once; every byte is
read exactly once, so `bytes` is also the reference for counter calibration (FETCH_SIZE).
Prints one JSON line per configuration.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libprobe.so")
SRC = os.path.join(HERE, "stream_probe.hip")


def build() -> str:
    import subprocess
    cmd = ["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-o", LIB + ".tmp", SRC]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode:
        raise RuntimeError("hipcc failed:\n" + r.stderr)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def run(configs, per_wg: int, reps: int = 3):
    import numpy as np
    import torch
    if not os.path.exists(LIB):
        raise RuntimeError(f"{LIB} is not built")
    L = ctypes.CDLL(LIB)
    for f in (L.probe_reg_stream, L.probe_lds_stream):
        f.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                      ctypes.c_void_p]
        f.restype = ctypes.c_int
    max_wg = max(c[1] for c in configs)
    src = torch.ones(max_wg * per_wg // 4, dtype=torch.int32, device="cuda")
    times = torch.zeros(2 * max_wg, dtype=torch.int64, device="cuda")
    sink = torch.zeros(512, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    out = []
    for kind, nwg, depth in configs:
        assert nwg * per_wg <= src.numel() * 4
        fn = L.probe_reg_stream if kind == "reg" else L.probe_lds_stream
        best = None
        for _ in range(reps):
            rc = fn(src.data_ptr(), per_wg, nwg, depth, times.data_ptr(), sink.data_ptr(), stream)
            if rc:
                raise RuntimeError(f"launch {kind} depth {depth}: {rc}")
            torch.cuda.synchronize()
            t = times[: 2 * nwg].view(nwg, 2).cpu().numpy().astype(np.int64)
            span_us = (t[:, 1].max() - t[:, 0].min()) * 0.01
            per_us = (t[:, 1] - t[:, 0]) * 0.01
            rec = {"kind": kind, "depth": depth, "workgroups": nwg, "bytes": nwg * per_wg,
                   "grid_GBps": round(nwg * per_wg / span_us / 1e3, 1),
                   "per_wg_GBps_median": round(float(np.median(per_wg / per_us / 1e3)), 1),
                   "span_us": round(float(span_us), 1)}
            if best is None or rec["grid_GBps"] > best["grid_GBps"]:
                best = rec
        out.append(best)
        print(json.dumps(best), flush=True)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--quick", action="store_true")
    ap.add_argument("--calib", action="store_true",
                    help="one dispatch of each load form at 170 workgroups (counter calibration runs)")
    ap.add_argument("--per-wg", type=int, default=4 << 20)
    args = ap.parse_args()
    if args.calib:
        run([("reg", 170, 8), ("lds", 170, 2)], args.per_wg, reps=1)
        return
    grids = [1, 8, 86, 170, 256] if not args.quick else [1, 170, 256]
    configs = [("reg", g, d) for d in (8, 16, 32, 48) for g in grids] + [("lds", g, c) for c in (1, 2) for g in grids]
    run(configs, args.per_wg)


if __name__ == "__main__":
    main()
