"""Decode throughput of the persistent megakernel on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu]

Default workload: the 30B-total / 3.3B-active shape (48 layers, hidden 2048,
32 q / 4 kv heads of 128, 128 experts top-8 with intermediate 768, vocab
151936), batch 1, 8192 cached tokens of synthetic KV, random-init BF16
weights from the seeded generator.  A step is one whole decode step: one
launch of the megakernel, whose device argmax feeds the next step's token;
sequence lengths for every step are precomputed on the device, so nothing
but decode launches sits in the timed region.

Prints one JSON line (rank 0): tok/s, the megakernel's achieved HBM
bandwidth (algorithmic bytes per step / average launch time, timed with
events on the launch stream) against MI355X's 8 TB/s, and the CPU oracle's
rate on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
DTYPES = {"bf16": "bf16", "fp8": "fp8-e4m3 weights, bf16 activations", "fp4": "fp4-e2m1 weights, bf16 activations"}
KERNELS = {"bf16": "mk_megakernel", "fp8": "mk_megakernel_fp8", "fp4": "mk_megakernel_fp4"}
METRIC = "decode tok/s at bs=1 8K ctx; achieved HBM GB/s as % of MI355X peak"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("mk_kernel.hip", "mk_kernel_fp8.hip", "mk_kernel_fp4.hip", "mk_kernel_seq.hip", "mk_host.cpp", "mk_types.h"):
        with open(os.path.join(ROOT, "persistent_moe_decode_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per decode step (one step per dispatch in the counter runs) from the committed rocprofv3
    counter record, if it was taken with this kernel source."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return t.get("hbm_bytes_per_step")


def write_traffic(fetch_csv: str, write_csv: str, workload: str, copy_bytes: int) -> dict:
    """profiles/traffic_<workload>.json from two rocprofv3 counter runs (FETCH_SIZE, then WRITE_SIZE, csv),
    each of bench.py with --steps-per-launch 1 (one decode step per mk_megakernel dispatch).

    Each run ends with one plain copy of copy_bytes (read copy_bytes, write
    copy_bytes): the largest __amd_rocclr_copyBuffer dispatch of a run scales
    that counter's KiB to bytes; mk_megakernel dispatches give the per-step values.
    """
    import csv

    import numpy as np

    def read(path, counter):
        kern, copies = [], []
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                v = float(r["Counter_Value"])
                if r["Kernel_Name"].startswith("mk_megakernel"):
                    kern.append(v)
                elif r["Kernel_Name"].startswith("__amd_rocclr_copyBuffer"):
                    copies.append(v)
        if not kern or not copies:
            raise SystemExit(f"{path}: no {counter} values for mk_megakernel and the calibration copy")
        return kern, max(copies)

    fk, fcal = read(fetch_csv, "FETCH_SIZE")
    wk, wcal = read(write_csv, "WRITE_SIZE")
    fscale = copy_bytes / (fcal * 1024.0)
    wscale = copy_bytes / (wcal * 1024.0)
    fb = float(np.median(fk)) * 1024.0 * fscale
    wb = float(np.median(wk)) * 1024.0 * wscale
    rec = {
        "workload": workload, "kernel": "mk_megakernel", "kernel_source_sha256_16": kernel_source_hash(),
        "fetch_kib_per_dispatch": fk, "write_kib_per_dispatch": wk, "calib_copy_bytes": copy_bytes,
        "calib_fetch_kib": fcal, "calib_write_kib": wcal,
        "fetch_scale": round(fscale, 5), "write_scale": round(wscale, 5),
        "steps_per_dispatch": 1,
        "hbm_fetch_bytes_per_step": round(fb), "hbm_write_bytes_per_step": round(wb),
        "hbm_bytes_per_step": round(fb + wb),
    }
    with open(os.path.join(ROOT, "profiles", f"traffic_{workload}.json"), "w") as f:
        json.dump(rec, f, indent=1)
    return rec


def step_bytes_kernel(shape, seq_lens, distinct):
    """Algorithmic HBM bytes one decode step reads: active weights (one embedding row per token) + KV 0..p."""
    H = shape.hidden
    w = shape.active_weight_bytes(distinct) + 2.0 * H * len(seq_lens)
    kv = sum(shape.kv_bytes_per_token() * (int(p) + 1) for p in seq_lens)
    return w + kv


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_steps(w, W, kv, pt, toks, first_step: int, budget_s: float, max_steps: int, src):
    """Decode steps of the oracle until budget_s of wall time; returns (steps, wall_s, regen_s, next tokens)."""
    from oracle import oracle as O

    n, t0 = 0, time.perf_counter()
    regen0 = src.regen_s
    while True:
        lens = [c + first_step + n for c in w.context]
        out = O.decode_step(W, kv, toks, pt, lens)
        toks = [int(t) for t in out.next_token]
        n += 1
        if time.perf_counter() - t0 > budget_s or n >= max_steps:
            break
    return n, time.perf_counter() - t0, src.regen_s - regen0, toks


class _TimedSource:
    """Wraps the oracle's weight source to time regeneration (generator + bf16 -> float64 decode)."""

    def __init__(self, shape):
        import synth
        self.shape, self.synth, self.regen_s = shape, synth, 0.0

    def __call__(self, kind, layer, expert):
        t = time.perf_counter()
        a = self.synth.weight_bits(self.shape, kind, layer, expert)
        self.regen_s += time.perf_counter() - t
        return a


def cpu_baseline(w, budget_s: float = 25.0, budget_1t_s: float = 20.0):
    """The CPU oracle, untuned, on a bounded sample of the same workload.

    One untimed step fills the oracle's weight cache with everything but newly routed experts;
    then decode steps run until budget_s with every host thread, then until budget_1t_s on one
    thread (BLAS and OpenMP pools limited to 1).  Weight regeneration (generator plus bf16
    decode, for experts first routed in a timed step) is timed separately: `value` includes it,
    `value_excl_regen` does not."""
    import threadpoolctl

    import synth
    from oracle import oracle as O

    src = _TimedSource(w.shape)
    W = O.Weights(w.shape, budget_bytes=float(2 ** 36), source=src)
    pt = w.page_table()
    kv = O.PagedKV(w.shape, w.num_pages)
    t_kv = time.perf_counter()
    kv.fill_synthetic(pt, w.context)
    kv_s = time.perf_counter() - t_kv
    toks = [int(w.prompt(b)[w.context[b]]) for b in range(w.batch)]
    out = O.decode_step(W, kv, toks, pt, list(w.context))
    toks = [int(t) for t in out.next_token]
    pools = threadpoolctl.threadpool_info()
    threads = max([p.get("num_threads", 1) for p in pools] or [1])

    n, dt, regen, toks = _oracle_steps(w, W, kv, pt, toks, 1, budget_s, 16, src)
    with threadpoolctl.threadpool_limits(limits=1):
        n1, dt1, regen1, _ = _oracle_steps(w, W, kv, pt, toks, 1 + n, budget_1t_s, 4, src)
    B = w.batch
    return {
        "value": round(B * n / dt, 4), "unit": "tok/s", "cores": int(threads), "kind": "oracle",
        "sample": f"{n} decode step(s) of {w.name} (batch {B}, context "
                  f"{w.context[0] if B == 1 else 'ragged'}) after one warm-up step; float64 numpy; "
                  f"then {n1} step(s) on 1 thread",
        "value_excl_regen": round(B * n / max(dt - regen, 1e-9), 4),
        "regen_s": round(regen, 3), "wall_s": round(dt, 3),
        "value_1thread": round(B * n1 / dt1, 4), "value_1thread_excl_regen": round(B * n1 / max(dt1 - regen1, 1e-9), 4),
        "regen_1thread_s": round(regen1, 3),
        "kv_fill_s": round(kv_s, 2),
        "host_cores": len(os.sched_getaffinity(0)), "cpu_model": _cpu_model(),
        "thread_pools": {p.get("internal_api", "?"): p.get("num_threads") for p in pools},
    }


def mixed_bench(args, w0, total):
    """Mixed steps: sequence A (the workload's single sequence) decodes one token per step while
    sequence B's prompt runs K tokens per step at positions K*i .. K*i + K - 1 (its own page-table
    row).  Timed against plain single-entry decode steps of A at the same contexts."""
    import numpy as np
    import torch

    import synth
    from persistent_moe_decode_amd.runtime import DeviceDecoder

    K = args.mixed
    if w0.batch != 1 or not 1 <= K <= 7:
        sys.exit("--mixed needs a batch-1 workload and 1 <= K <= 7")
    w = synth.Workload(w0.name + f"_mixed{K}", w0.shape, batch=1 + K, steps=K * total + 16,
                       context=[w0.context[0]] + [0] * K)
    # the default split would size attention for 1 + K sequences of the mean context and reserve a
    # lead unit per possible (entry, kv head): here one sequence holds nearly all K/V, so keep the
    # batch-1 split's other attention units (--attn-units overrides)
    ref = synth.workload(w0.name)
    from persistent_moe_decode_amd import mk
    c1 = mk.Context(mk.config_from_shape(ref.shape, 1, ref.max_pages_per_seq, ref.num_pages))
    c1.build_schedule(0, ref.context[0] + ref.steps // 2)
    n_other = c1.info().n_attn - ref.shape.n_kv_heads
    attn = args.attn_units or (1 + K) * w.shape.n_kv_heads + n_other
    log(f"[bench] mixed: {attn} attention units ({n_other} besides the {(1 + K) * w.shape.n_kv_heads} segment leads)")
    dec = DeviceDecoder(w, attn_units=attn)
    dec.fill_synthetic_kv()
    dev, n = dec.dev, 1 + K
    pt_np = dec.page_table_np.copy()
    pt_np[2:] = pt_np[1]
    pt = torch.from_numpy(np.ascontiguousarray(pt_np)).to(dev)
    ctx = w0.context[0]
    b_prompt = synth.uniform_u32(synth.SEED_PROMPT, synth.tid(synth.K_PROMPT, 1), 0, K * total,
                                 w.shape.vocab).astype(np.int32)
    toks = torch.zeros(total, n, dtype=torch.int32, device=dev)
    lens = torch.zeros(total, n, dtype=torch.int32, device=dev)
    for i in range(total):
        toks[i, 0] = int(w0.prompt(0)[ctx])
        toks[i, 1:] = torch.from_numpy(b_prompt[K * i:K * (i + 1)])
        lens[i, 0] = ctx + i
        lens[i, 1:] = torch.arange(K * i, K * (i + 1), dtype=torch.int32)
    nxt = torch.zeros(n, dtype=torch.int32, device=dev)

    def timed(fn):
        for i in range(args.warmup):
            fn(i)
        torch.cuda.synchronize(dev)
        dec.check_error()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(args.warmup, total):
            fn(i)
        e1.record()
        torch.cuda.synchronize(dev)
        dec.check_error()
        return e0.elapsed_time(e1) / args.steps

    ms_mixed = timed(lambda i: dec.ctx.mixed_step(n, toks[i].data_ptr(), pt.data_ptr(), lens[i].data_ptr(),
                                                  dec.logits.data_ptr(), nxt.data_ptr(), dec.stream))
    ms_decode = timed(lambda i: dec.ctx.decode_step(1, toks[i].data_ptr(), pt.data_ptr(), lens[i].data_ptr(),
                                                    dec.logits.data_ptr(), nxt.data_ptr(), dec.stream))
    log(f"[bench] mixed step ({K} prompt tokens + 1 decode): {ms_mixed:.3f} ms; plain decode step "
        f"{ms_decode:.3f} ms")
    dec.close()
    s = w.shape
    print(json.dumps({
        "metric": "mixed step: one decode token plus K chunked-prefill tokens per persistent launch",
        "value": round(n / (ms_mixed / 1e3), 2), "unit": "tok/s (decode + prefill)", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_mixed, 4), "higher_is_better": True,
        "dtype": DTYPES[s.weights], "data": "synthetic",
        "config": {"workload": f"{w0.name}: decode at {ctx}+ plus a prompt in chunks of {K}", "prefill_chunk": K,
                   "decode_tok_s": round(1 / (ms_mixed / 1e3), 2),
                   "prefill_tok_s": round(K / (ms_mixed / 1e3), 2),
                   "plain_decode_ms_per_step": round(ms_decode, 4)},
    }), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=128)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--workload", default="moe30b_8k",
                    help="tiny, mid, moe30b_8k, moe30b_bs8_ragged or moe30b_256k; suffixes _seq (the sequential "
                         "block), _fp8 / _fp4 (quantized weights), e.g. moe30b_8k_fp4, moe30b_bs8_ragged_seq")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-budget", type=float, default=25.0)
    ap.add_argument("--trace", default="", help="write a Perfetto timeline of one extra step to this path")
    ap.add_argument("--steps-per-launch", type=int, default=16,
                    help="decode steps per launch of the persistent kernel (greedy tokens fed on the device)")
    ap.add_argument("--attn-units", type=int, default=0, help="schedule: attention compute units (0 = default)")
    ap.add_argument("--router-units", type=int, default=0, help="schedule: router compute units (0 = default)")
    ap.add_argument("--qkv-units", type=int, default=0, help="schedule: dedicated Wqkv compute units (0 = none)")
    ap.add_argument("--pool-64ths", type=int, default=0, help="schedule: shared gate/up pool share (0 = none)")
    ap.add_argument("--copy-calib", type=int, default=0,
                    help="after the run, one plain device-to-device copy of this many bytes (counter calibration)")
    ap.add_argument("--mixed", type=int, default=0, metavar="K",
                    help="time mixed steps instead (mk_mixed_step): the workload's batch-1 decode plus K "
                         "prompt tokens of a second sequence per step (its prompt advancing K positions a "
                         "step), against plain decode steps of the same context; prints its own JSON line")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic_<workload>.json from two rocprofv3 counter runs made with "
                         "--copy-calib 1073741824, then exit (no GPU needed)")
    args = ap.parse_args()
    if args.write_traffic:
        rec = write_traffic(*args.write_traffic, args.workload, 1 << 30)
        print(json.dumps({k: rec[k] for k in ("fetch_scale", "write_scale", "hbm_bytes_per_step")}))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one MI355X: the decode megakernel runs on a single GPU and has no "
              "multi-GPU path (use --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    from persistent_moe_decode_amd.runtime import DeviceDecoder

    w = synth.workload(args.workload)
    total = args.warmup + args.steps
    if args.mixed:
        return mixed_bench(args, w, total)
    if total > w.steps:
        w.steps = total  # page capacity for every position the run writes
    t0 = time.time()
    dec = DeviceDecoder(w, attn_units=args.attn_units, router_units=args.router_units, qkv_units=args.qkv_units,
                        pool_64ths=args.pool_64ths)
    dec.fill_synthetic_kv()
    log(f"[bench] setup {time.time() - t0:.1f}s, {dec.info.num_cus} CUs, n_attn {dec.info.n_attn}, "
        f"lds {dec.info.lds_bytes} B, workspace {dec.ws_bytes / 2**20:.1f} MiB")
    dev = dec.dev
    B = w.batch
    ctx = torch.tensor(w.context, dtype=torch.int32, device=dev)
    lens_all = torch.stack([ctx + i for i in range(total)]).contiguous()  # [step][B]
    # toks[i] = the token step i feeds; a launch of k steps from step i writes toks[i + 1 .. i + k]
    toks = torch.zeros(total + 1, B, dtype=torch.int32, device=dev)
    toks[0] = torch.tensor([int(w.prompt(b)[w.context[b]]) for b in range(B)], dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    spl = max(1, args.steps_per_launch)

    def run(i, k):
        """Steps i .. i + k - 1 in one launch."""
        dec.ctx.decode_steps(B, k, toks[i].data_ptr(), dec.page_table.data_ptr(), lens_all[i].data_ptr(),
                             dec.logits.data_ptr(), toks[i + 1].data_ptr(), dec.stream)

    def run_range(i0, i1):
        i = i0
        while i < i1:
            k = min(spl, i1 - i)
            run(i, k)
            i += k

    run_range(0, args.warmup)
    torch.cuda.synchronize(dev)
    dec.check_error()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize(dev)
    e0.record(stream)
    run_range(args.warmup, total)
    e1.record(stream)
    torch.cuda.synchronize(dev)
    dec.check_error()
    ms = e0.elapsed_time(e1)
    ms_step = ms / args.steps
    tok_s = B * args.steps / (ms / 1e3)

    # algorithmic bytes over the timed steps: distinct experts per layer from the routing of each step
    sel = dec.sel()[:, :B, :]
    distinct = np.mean([len(set(sel[l].reshape(-1).tolist())) for l in range(w.shape.n_layers)])
    bytes_tot = sum(step_bytes_kernel(w.shape, [c + i for c in w.context], distinct)
                    for i in range(args.warmup, total))
    bytes_step = bytes_tot / args.steps
    gbs = bytes_step / (ms_step / 1e3) / 1e9
    traffic = measured_traffic(args.workload)
    n_launch = -(-args.steps // spl)
    launch_ms = ms / n_launch
    log(f"[bench] {ms_step:.3f} ms/step, {tok_s:.1f} tok/s, {bytes_step / 1e9:.4f} GB/step, {gbs:.0f} GB/s "
        f"({100 * gbs / PEAK_HBM_GBS:.1f}% of peak)")

    if args.trace:
        # one more step, traced, outside the timed region
        from persistent_moe_decode_amd import trace as tr
        ntask = dec.info.n_tasks
        buf = torch.zeros(tr.WORDS * ntask, dtype=torch.int64, device=dev)
        dec.ctx.set_trace(buf.data_ptr(), ntask)
        run(total - 1, 1)
        torch.cuda.synchronize(dev)
        dec.ctx.set_trace(None)
        tasks, qoff = dec.ctx.schedule()
        rec = buf.view(ntask, tr.WORDS).cpu().numpy()
        log("[bench] trace " + json.dumps(tr.summarize(tasks, qoff, rec)))
        tr.dump(args.trace, tasks, qoff, rec)

    if args.copy_calib:
        # a plain copy of known size: its FETCH_SIZE / WRITE_SIZE per dispatch calibrate the counters
        n = args.copy_calib // 2
        src = torch.ones(n, dtype=torch.int16, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize(dev)
        dst.copy_(src)
        torch.cuda.synchronize(dev)
        log(f"[bench] calibration copy of {2 * n} bytes done")
        del src, dst

    # ordered teardown before anything else runs: the device is idle, the context destroyed and its
    # buffers released, then libmk.so is unloaded so its HIP code-object unregistration runs now
    # rather than among the interpreter's exit handlers (after a profiler has finalized)
    dec.close()
    del dec, toks, lens_all, ctx
    from persistent_moe_decode_amd import mk
    mk.unload()

    cpu = None
    if not args.no_cpu:
        t1 = time.time()
        cpu = cpu_baseline(w, args.cpu_budget)
        log(f"[bench] cpu baseline {cpu['value']} tok/s ({time.time() - t1:.0f}s)")

    s = w.shape
    out = {
        "metric": METRIC,
        "value": round(tok_s, 2),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPES[s.weights],
        "data": ("synthetic: seeded random-init weights " +
                 {"fp8": "as E4M3 codes (N(0, 32) rounded) times row scales near 0.02/32, ",
                  "fp4": "as E2M1 codes (N(0, 1.5) rounded) times row scales near 0.02/1.5, "}.get(s.weights, "N(0, 0.02), ") + "synthetic N(0, 1) KV, shuffled pages"),
        "config": {
            "workload": f"{w.name}: {'sequential block, ' if s.sequential else ''}{s.n_layers} layers, hidden {s.hidden}, "
                        f"{s.n_q_heads}q/{s.n_kv_heads}kv x "
                        f"{s.head_dim}, {s.n_experts} experts top-{s.top_k} inter {s.inter}, vocab {s.vocab}; "
                        f"batch {B}, context {w.context if B > 1 else w.context[0]}, page {s.page_size}",
            "batch": B,
            "steps_per_launch": spl,
            "context": w.context[0] if B == 1 else w.context,
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(gbs, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4),
            "traffic": None if traffic is None else round(traffic * spl),
            "algorithmic_bytes_per_launch": round(bytes_step * spl),
            "launch_ms": round(launch_ms, 4),
            "steps_per_launch": spl,
            "kernel": KERNELS[s.weights] + ("_seq" if s.sequential else ""),
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
