"""Throughput of the absorbed-MLA decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config c2]

A step is one full decode call (plan -> split-KV decode -> LSE combine) over
one batch of the workload, with its inputs already resident in HBM. The
latent cache is replicated in several buffer sets that the steps rotate
through, so that the 256 MB last-level cache cannot serve a step from the
previous step's reads. Prints one JSON line.

The metric is latent-cache bytes per second (each cached token read once per
step; 1152 B per token in bf16), with TFLOP/s alongside (2 flops per MAC,
576 lanes for scores plus 512 for the weighted sum, per attended query row and
token). The CPU baseline is the fp64 oracle on the host cores over a bounded
sample of the same workload.
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

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
BF16_MFMA_PEAK_TFS = 2500.0  # dense bf16 matrix peak
RIDGE_BF16 = BF16_MFMA_PEAK_TFS * 1e12 / (HBM_PEAK_GBS * 1e9)   # flop per byte
COUNTERS_FILE = os.path.join(ROOT, "profiles", "decode_counters.json")

WORKLOAD_TEXT = {
    "c2": "bf16 latent cache, batch 32, one query per sequence, context 4096, 128 heads, d_c 512, d_R 64",
    "c3": "bf16 latent cache, batch 4, context 32768, 128 heads, d_c 512, d_R 64",
    "c4": "bf16 paged ragged batch 64, contexts U[512,16384], permuted pages, 128 heads",
    "c5": "fp8 e4m3 latent + bf16 rope key, batch 128, context 8192, 2 queries (causal pair), 128 heads",
}


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "latent_kv_cache_mla_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h")):
            with open(os.path.join(csrc, f), "rb") as fh:
                h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def settle(fn, seconds: float = 0.3):
    """Run `fn` untimed for about `seconds` before the warm-up steps: the GPU
    raises its clocks only under sustained load, and a few warm-up steps are
    not enough for that (the timed steps then mix two clock levels)."""
    import torch
    t0 = time.perf_counter()
    i = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(20):
            fn(i)
            i += 1
        torch.cuda.synchronize()


def workload_sizes(cfg, seq_lens):
    import numpy as np
    bpt = {"bf16": 2 * cfg.lanes, "fp32": 4 * cfg.lanes, "fp8": cfg.d_c + 2 * cfg.d_rope + 4}[cfg.cache_dtype]
    lens = np.asarray(seq_lens, dtype=np.int64)
    cache_bytes = int(lens.sum()) * bpt
    # attended (query, token) pairs: query m sees S - q_len + m + 1 positions
    pairs = sum(max(0, int(s) - cfg.q_len + m + 1) for s in lens for m in range(cfg.q_len))
    flops = 2 * pairs * cfg.n_heads * (cfg.lanes + cfg.d_c)
    return cache_bytes, flops, bpt


def cpu_baseline(inp, budget_s: float = 12.0):
    """The oracle (as it stands) over whole sequences of the workload until
    about budget_s seconds of CPU work; GB/s of latent cache processed."""
    import numpy as np
    import oracle
    from tests import gpu_harness as H
    cfg = inp.cfg
    qa, qr = H.oracle_queries(inp)
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # noqa: BLE001
        cores = len(os.sched_getaffinity(0))
    done_bytes, t_total, n_seq = 0, 0.0, 0
    _, _, bpt = workload_sizes(cfg, inp.seq_lens)
    b = 0
    while t_total < budget_s and n_seq < 1000 * cfg.batch:
        c, kr = H.oracle_inputs(inp, b % cfg.batch)
        t0 = time.perf_counter()
        oracle.latent_attention(qa[b % cfg.batch], qr[b % cfg.batch], c, kr, cfg.softmax_scale)
        t_total += time.perf_counter() - t0
        done_bytes += int(inp.seq_lens[b % cfg.batch]) * bpt
        n_seq += 1
        b += 1
    return {"value": round(done_bytes / t_total / 1e9, 4), "unit": "GB/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"{n_seq} sequences of the workload ({done_bytes / 1e6:.1f} MB of cache), "
                      f"fp64 numpy oracle, {t_total:.1f} s of CPU time"}


def measured_read_gbs(n_bytes: int = 1 << 30, reps: int = 10):
    """Achievable HBM read bandwidth: row sums over n_bytes of fp32 in rows of
    1024 (the fastest plain reduction shape measured here; the output is 1/1024
    of the input), untimed warm-up, then the best of `reps` timed passes."""
    import torch
    x = torch.ones(n_bytes // 4, dtype=torch.float32, device="cuda").view(-1, 1024)
    out = torch.empty(x.shape[0], dtype=torch.float32, device="cuda")
    for _ in range(3):
        torch.sum(x, dim=1, out=out)
    torch.cuda.synchronize()
    best = float("inf")
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        torch.sum(x, dim=1, out=out)
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1) * 1e-3)
    del x
    return round(n_bytes / best / 1e9, 1)


def gpu_clocks():
    """Current shader and memory clocks as rocm-smi reports them (None if it
    cannot be run)."""
    import subprocess
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True, text=True,
                           timeout=20)
        d = json.loads(r.stdout)
        card = d[sorted(d)[0]]
        return {k: v for k, v in card.items() if "sclk" in k.lower() or "mclk" in k.lower()}
    except Exception:   # no rocm-smi, no permission, unexpected output
        return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="c2", choices=sorted(WORKLOAD_TEXT))
    ap.add_argument("--rotate", type=int, default=0, help="buffer sets (0: enough for 600 MB)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--fp8-math", action="store_true",
                    help="fp8 cache: scores on the fp8 matrix cores (MLA_DECODE_FP8_MATH)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="also run a plain device copy of MIB MiB three times (untimed), "
                         "so that hardware byte counters can be scaled against a known size")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import latent_kv_cache_mla_amd as mla
    import workloads as wl
    from tests import gpu_harness as H

    cfg = wl.CONFIGS[args.config]
    inp = wl.make_decode_inputs(cfg)
    cache_bytes, flops, _ = workload_sizes(cfg, inp.seq_lens)
    dev = H.device_inputs(inp)
    rotate = args.rotate or max(2, int(np.ceil(600e6 / cache_bytes)))
    caches = [dev["cache"]] + [dev["cache"].clone() for _ in range(rotate - 1)]
    qas = [dev["q_abs"]] + [dev["q_abs"].clone() for _ in range(rotate - 1)]
    qrs = [dev["q_rope"]] + [dev["q_rope"].clone() for _ in range(rotate - 1)]
    flags = mla.MLA_DECODE_FP8_MATH if args.fp8_math else 0
    if args.fp8_math and cfg.cache_dtype != "fp8":
        print("--fp8-math applies to the fp8 workload (c5) only", file=sys.stderr)
        sys.exit(2)
    desc = mla.decode_desc(cfg.batch, cfg.q_len, cfg.n_heads, cfg.d_c, cfg.d_rope, dev["max_blocks"],
                           cfg.cache_dtype, "bf16", cfg.out_dtype, flags=flags)
    ws = torch.empty(mla.mla_decode_workspace_size(desc), dtype=torch.uint8, device="cuda")
    odt = torch.float32 if cfg.out_dtype == "fp32" else torch.bfloat16
    outs = [torch.empty((cfg.batch, cfg.q_len, cfg.n_heads, cfg.d_c), dtype=odt, device="cuda")
            for _ in range(rotate)]
    scale = cfg.softmax_scale

    def step(i):
        k = i % rotate
        mla.mla_decode(desc, qas[k], qrs[k], caches[k], dev["cache_scale"], dev["block_table"],
                       dev["seq_lens"], scale, outs[k], None, ws)

    settle(step)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(args.steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps

    # per-step distribution (a separate pass: an event pair around every step)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for i, (a, b) in enumerate(evs):
        a.record()
        step(i)
        b.record()
    torch.cuda.synchronize()
    per_step_us = np.array([a.elapsed_time(b) * 1e3 for a, b in evs])

    # the dominant kernel alone: split-KV decode with the plan already built
    pdesc = mla.decode_desc(cfg.batch, cfg.q_len, cfg.n_heads, cfg.d_c, cfg.d_rope, dev["max_blocks"],
                            cfg.cache_dtype, "bf16", cfg.out_dtype, plan_ready=1, flags=flags)
    mla.mla_decode_plan(desc, dev["seq_lens"], ws)

    def part(i):
        k = i % rotate
        mla.mla_decode_partial(pdesc, qas[k], qrs[k], caches[k], dev["cache_scale"],
                               dev["block_table"], dev["seq_lens"], scale, ws)

    settle(part)
    for i in range(args.warmup):
        part(i)
    torch.cuda.synchronize()
    k0, k1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    k0.record()
    for i in range(args.steps):
        part(i)
    k1.record()
    torch.cuda.synchronize()
    kern_ms = k0.elapsed_time(k1) / args.steps

    gbs = cache_bytes / (ms * 1e-3) / 1e9
    tfs = flops / (ms * 1e-3) / 1e12
    k_gbs = cache_bytes / (kern_ms * 1e-3) / 1e9
    traffic = None
    if os.path.exists(COUNTERS_FILE):
        with open(COUNTERS_FILE) as f:
            cnt = json.load(f)
        rec = cnt.get(args.config + ("+fp8math" if args.fp8_math else ""))
        if rec and rec.get("kernel_source_hash") == kernel_source_hash():
            traffic = rec.get("hbm_bytes_per_launch")

    line = {
        "metric": "absorbed-MLA decode latent-cache GB/s + TFLOP/s (% of peak), 128 heads, 1 GPU",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8" if cfg.cache_dtype == "fp8" else "bf16",
        "data": "synthetic",
        "config": {"workload": f"{args.config}: {WORKLOAD_TEXT[args.config]}", "batch": cfg.batch,
                   "seq_len": cfg.seq_len if cfg.seq_len else "ragged", "q_len": cfg.q_len,
                   "n_heads": cfg.n_heads, "d_c": cfg.d_c, "d_rope": cfg.d_rope,
                   "cache_bytes": cache_bytes, "flops": flops, "buffer_sets": rotate,
                   "parallelism": "single GPU", "fp8_math": bool(args.fp8_math)},
        "step_us_p10_p50_p90": [round(float(np.percentile(per_step_us, q)), 2) for q in (10, 50, 90)],
        "tflops": round(tfs, 2),
        "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "pct_bf16_mfma_peak": round(100 * tfs / BF16_MFMA_PEAK_TFS, 2),
        "roofline": {"bound": "hbm", "kernel": "split-KV decode", "achieved": round(k_gbs, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(k_gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "kernel_ms": round(kern_ms, 5),
                     "algorithmic_bytes_per_launch": cache_bytes},
    }
    if flops / cache_bytes > RIDGE_BF16:
        # above the bf16 ridge point (the fp8 workload: two query rows per
        # head and 644 bytes per token) the matrix cores bound the kernel; it
        # is priced at the dense bf16 peak in both fp8 modes (with the fp8
        # flag the score products run at the fp8 rate, whose peak is twice
        # that, and the weighted sum stays bf16)
        k_tfs = flops / (kern_ms * 1e-3) / 1e12
        line["roofline"].update({"bound": "mfma", "achieved": round(k_tfs, 2),
                                 "peak": BF16_MFMA_PEAK_TFS, "unit": "TFLOP/s",
                                 "frac": round(k_tfs / BF16_MFMA_PEAK_TFS, 4),
                                 "algorithmic_flops_per_launch": flops,
                                 "hbm_achieved_gbs": round(k_gbs, 2)})
    # context for the roofline: a measured streaming read (a plain reduction
    # over 1 GiB, far larger than the 256 MB last-level cache) and the clocks
    line["hbm_read_measured_gbs"] = measured_read_gbs()
    line["clocks"] = gpu_clocks()
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        line["copy_calibration_bytes"] = n
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(inp)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
