#!/usr/bin/env python3
"""Throughput of the fused token-selection kernel on one MI355X.

Workload (one step = one tsel_process_select call over the whole batch): 256
rows of 128256 bf16 logits (log-Zipf(1.1) over a random permutation plus
N(0,1) noise), 4096-token histories, repetition penalty 1.05, 100
suppress_tokens, 50 single-token bad words, temperature 1.0, top_p 0.95 and
inverse-CDF sampling from one uniform per row.  Inputs are seeded synthetic
data, resident in HBM before the timed region; R copies at distinct addresses
rotate from step to step so that the 256 MB last-level cache cannot hold a
step's input (R * 70 MB > 512 MB).

Prints one JSON line: whole-job rows/s, the per-launch kernel time from HIP
events on the launch stream, the kernel's achieved algorithmic HBM bandwidth
against the MI355X peak (8 TB/s), and the CPU oracle timed on the host cores
over the same rows.
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

METRIC = "logit rows/sec + achieved HBM GB/s (% peak), B=256 V=128256 full chain"
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_vres_b256_v128256_traffic.txt")
KERNEL_SOURCES = ("logits_processing_token_amd/csrc/k_vres.hip",
                  "logits_processing_token_amd/csrc/k_res_common.hpp",
                  "logits_processing_token_amd/csrc/k_mass.hpp",
                  "logits_processing_token_amd/csrc/k_select_common.hpp",
                  "logits_processing_token_amd/csrc/tsel_device.hpp",
                  "logits_processing_token_amd/csrc/tsel_internal.hpp")


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def algorithmic_bytes(w) -> int:
    """Bytes the method must move per launch: every logit once, every
    history id once, the per-row scalars (3 lengths, the uniform, the token)
    and the two static bitmasks once."""
    B, V = w.logits.shape
    esize = 2 if w.dtype == "bf16" else 4
    per_row = V * esize + 4 * w.history.shape[1] + 4 * 3 + 4 + 4
    masks = sum(4 * ((V + 31) // 32) for n in ("bad_words_ids", "suppress_tokens")
                if w.settings.get(n))
    return B * per_row + masks


def measured_traffic():
    """HBM bytes per launch from the committed rocprofv3 counter runs, or
    None when they are absent or were taken on other kernel sources."""
    t = {}
    try:
        with open(TRAFFIC_FILE) as f:
            for line in f:
                k, sep, v = line.partition("=")
                if sep:
                    t[k.strip()] = v.strip()
    except OSError:
        return None
    if t.get("source_sha256") != kernel_source_sha():
        return None
    try:
        return float(t["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(w, gpu_tokens, threads: int):
    """The CPU oracle as it stands, over every row of the workload, rows
    spread over `threads` host threads."""
    import numpy as np
    import oracle
    t0 = time.perf_counter()
    r = oracle.select(w.logits, w.history, w.lens, w.prompt_lens, w.max_lengths,
                      oracle.Config(**w.settings), uniforms=w.uniforms, threads=threads)
    dt = time.perf_counter() - t0
    low = r["margin"] < 1e-4
    same = gpu_tokens == r["token"]
    adm = [int(g) in a.tolist() or g == o
           for g, o, a in zip(gpu_tokens, r["token"], r["admissible"])]
    parity = {"rows": int(w.batch), "exact": int(same.sum()),
              "high_margin_mismatch": int((~same & ~low).sum()),
              "low_margin_rows": int(low.sum()),
              "low_margin_mismatch": int((~same & low).sum()),
              "admissible": int(np.sum(adm))}
    base = {"value": w.batch / dt, "unit": "rows/s", "cores": threads, "kind": "oracle",
            "sample": f"all {w.batch} rows of the benchmark batch, one pass "
                      f"({dt:.2f} s wall on {threads} threads)"}
    return base, parity


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--rotate", type=int, default=8, help="distinct input copies")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--rows", type=int, default=0,
                    help="time only the first ROWS rows of the batch (a latency sweep; "
                         "the metric's own line is the whole batch)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a plain 256 MiB device copy (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(rows would shard with no exchange); run with --gpus 1", file=sys.stderr)
        return 2

    import numpy as np
    import torch
    from logits_processing_token_amd import synth, tsel

    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import harness

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    tsel.load()
    dev = torch.device("cuda:0")
    print("bench: generating the workload", file=sys.stderr, flush=True)
    w = synth.c3_select()
    sweep = 0 < args.rows < w.batch
    if sweep:
        n = args.rows
        w = synth.SelectWorkload(w.name, w.logits[:n].copy(), w.history[:n].copy(),
                                 w.lens[:n].copy(), w.prompt_lens[:n].copy(),
                                 w.max_lengths[:n].copy(), w.settings, w.uniforms[:n].copy())
    B, V = w.logits.shape

    if args.copy_calibration:
        src = torch.empty(64 << 20, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    d = harness.upload_select(w)
    R = max(1, args.rotate)
    if sweep:  # (enough copies that a few rows still come from HBM, not the caches)
        R = max(R, -(-(768 << 20) // (d["logits"].numel() * d["logits"].element_size())))
    logits = [d["logits"]] + [d["logits"].clone() for _ in range(R - 1)]
    hists = [d["hist"]] + [d["hist"].clone() for _ in range(R - 1)]
    out = torch.empty(B, dtype=torch.int32, device=dev)
    params = d["params"]

    def step(i):
        tsel.process_select(logits[i % R], hists[i % R], d["lens"], params, d["u"], out)

    print("bench: warmup", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    first_tokens = None
    step(0)
    torch.cuda.synchronize()
    first_tokens = out.cpu().numpy().copy()

    K = args.steps
    # One event pair on the launch stream brackets the K launches: the mean
    # launch duration includes the gaps between launches (an event pair per
    # launch would put its own timestamp packets between the kernels).
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    print(f"bench: timing {K} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record()
    for i in range(K):
        step(i)
    ev1.record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    kernel_ms = ev0.elapsed_time(ev1) / K

    alg = algorithmic_bytes(w)
    achieved = alg / (kernel_ms * 1e-3) / 1e9
    # (the counters were taken on the whole batch)
    traffic = None if sweep else measured_traffic()
    result = {
        "metric": METRIC,
        "value": B * K / elapsed,
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": elapsed / K * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "C3 full chain: B=256 V=128256 bf16 logits, log-Zipf(1.1) "
                               "over a random permutation + N(0,1); history 4096; "
                               "repetition_penalty 1.05; 100 suppress_tokens; 50 bad words; "
                               "temperature 1.0; top_p 0.95; inverse-CDF sampling",
                   "batch": B, "vocab": V, "logits_dtype": "bf16", "rotated_copies": R,
                   **({"rows_timed": f"the first {B} rows of the batch"} if sweep else {})},
        "kernel_ms": kernel_ms,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS,
                     "traffic": traffic, "algorithmic_bytes": alg},
    }
    if not args.no_cpu_baseline:
        threads = min(16, os.cpu_count() or 1)
        base, parity = cpu_baseline(w, first_tokens, threads)
        result["cpu_baseline"] = base
        result["parity"] = parity
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
