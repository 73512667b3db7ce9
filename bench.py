#!/usr/bin/env python3
"""Throughput of the token-selection path on one MI355X.

Default workload (C3; one step = one tsel_process_select call over the whole
batch): 256 rows of 128256 bf16 logits (log-Zipf(1.1) over a random
permutation plus N(0,1) noise), 4096-token histories, repetition penalty
1.05, 100 suppress_tokens, 50 single-token bad words, temperature 1.0, top_p
0.95 and inverse-CDF sampling from one uniform per row.  Inputs are seeded
synthetic data, resident in HBM before the timed region; R copies at
distinct addresses rotate from step to step so that the 256 MB last-level
cache cannot hold a step's input (R * bytes > 512 MB).

--config picks another workload (C1, C1v, C2, C4, C5: the other named
configurations; F1: C3 with the token log-probability; F2: one beam-search
step over the C3 batch read as 64 prompts x 4 beams; F3: verification with
sampling at every position on the C4 shape), or "all" for one line each.

Prints one JSON line per workload: whole-job rows/s, the per-step time from
HIP events on the launch stream, the achieved algorithmic HBM bandwidth
against the MI355X peak (8 TB/s), the HBM traffic the committed rocprofv3
counters give, and the CPU oracle timed on the host cores.
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
HOST_THREADS_CAP = 16  # worker threads per GPU on a shared host
CSRC = "logits_processing_token_amd/csrc/"
COMMON = (CSRC + "tsel_api.cpp", CSRC + "tsel_internal.hpp", CSRC + "tsel_device.hpp")
SELECT_COMMON = COMMON + (CSRC + "k_select_common.hpp", CSRC + "k_mass.hpp")


def source_sha(paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(name: str, sources):
    """HBM bytes per step from a committed rocprofv3 counter summary, or
    None when it is absent or was taken on other sources."""
    t = {}
    try:
        with open(os.path.join(ROOT, "profiles", name)) as f:
            for line in f:
                k, sep, v = line.partition("=")
                if sep:
                    t[k.strip()] = v.strip()
    except OSError:
        return None
    if t.get("source_sha256") != source_sha(sources):
        return None
    try:
        return float(t["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def read_ceiling_gbs(dev) -> float:
    """The HBM read rate a plain streaming kernel (libtsel_probe.so: 16-byte
    loads, four in flight, 512 workgroups of 256 lanes, the fastest grid of a
    sweep from 128 to 16384) reaches over 1 GiB, two buffers alternating so
    that neither stays in the 256 MB last-level cache."""
    import torch
    from logits_processing_token_amd import probe
    n = 1 << 30
    bufs = [torch.empty(n, dtype=torch.uint8, device=dev).fill_(1) for _ in range(2)]
    out = torch.zeros(1, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()

    def run(i):
        probe.read(bufs[i % 2], 512, out, stream)
    for i in range(4):
        run(i)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    K = 20
    for i in range(K):
        run(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / K
    del bufs
    torch.cuda.empty_cache()
    return n / (ms * 1e-3) / 1e9


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, HOST_THREADS_CAP))


def select_bytes(w, forced_free: bool = True) -> int:
    """Bytes a selection must move per launch: every logit and history id of
    a row once, its scalars (3 lengths, uniform, token), and the static
    bitmasks once.  A row forced to one id needs only its scalars."""
    import numpy as np
    B, V = w.logits.shape
    esize = 2 if w.dtype == "bf16" else 4
    per_row = V * esize + 4 * w.history.shape[1]
    scalars = 4 * 3 + 4 + 4
    s = w.settings
    forced = np.zeros(B, bool)
    if forced_free:
        if s.get("forced_eos_token_id", -1) >= 0:
            forced |= w.lens == w.max_lengths - 1
        if s.get("forced_bos_token_id", -1) >= 0:
            forced |= w.lens == 1
    masks = sum(4 * ((V + 31) // 32) for n in ("bad_words_ids", "suppress_tokens",
                                              "begin_suppress_tokens") if s.get(n))
    return int((~forced).sum()) * per_row + B * scalars + masks


# Per workload: the launches of one step (the dominant first), the committed
# counter summary, and the sources whose hash that summary must match.
PROFILED = {
    "C1": (("k_greedy",), "k_greedy_c1_traffic.txt", SELECT_COMMON + (CSRC + "k_greedy.hip",)),
    "C1v": (("k_verify_part", "k_verify_merge"), "k_verify_c1_traffic.txt",
            COMMON + (CSRC + "k_verify.hip",)),
    "C2": (("k_topk",), "k_topk_c2_traffic.txt",
           SELECT_COMMON + (CSRC + "k_full.hip", CSRC + "k_vkey.hpp")),
    "C3": (("k_vres",), "k_vres_b256_v128256_traffic.txt",
           SELECT_COMMON + (CSRC + "k_vres.hip", CSRC + "k_res_common.hpp", CSRC + "k_vkey.hpp")),
    "C4": (("k_verify_part", "k_verify_merge"), "k_verify_c4_traffic.txt",
           COMMON + (CSRC + "k_verify.hip",)),
    "C5": (("k_topk",), "k_topk_c5_traffic.txt",
           SELECT_COMMON + (CSRC + "k_full.hip", CSRC + "k_vkey.hpp")),
    "F1": (("k_vres",), "k_vres_logprob_c3_traffic.txt",
           SELECT_COMMON + (CSRC + "k_vres.hip", CSRC + "k_res_common.hpp", CSRC + "k_vkey.hpp")),
    "F2": (("k_beam_rows", "k_beam_merge_wave"), "k_beam_c3_traffic.txt",
           COMMON + (CSRC + "k_beam.hip", CSRC + "k_vkey.hpp")),
    "F3": (("k_full", "k_vsel_expand", "k_vsel_match"), "k_vsel_c4_traffic.txt",
           SELECT_COMMON + (CSRC + "k_full.hip", CSRC + "k_vsel.hip", CSRC + "k_vkey.hpp")),
}


# --------------------------------------------------------------------------
# One case per workload: device inputs, the step, its bytes, the CPU oracle.

class Case:
    name = ""
    workload = ""
    rows = 0          # rows one step processes (the rows/s unit)
    kernels = ()      # launches of one step, the dominant first
    traffic_file = ""
    sources = ()

    def step(self, i):
        raise NotImplementedError

    def result(self):
        raise NotImplementedError


def _rotated(t, R):
    return [t] + [t.clone() for _ in range(R - 1)]


def _copies(nbytes: int) -> int:
    return max(1, -(-(512 << 20) // max(nbytes, 1)) + 1)


class SelectCase(Case):
    def __init__(self, name, w, workload, rotate=None, logprobs=False):
        import torch
        from logits_processing_token_amd import tsel, upload
        self.name, self.w, self.workload = name, w, workload
        self.kernels, self.traffic_file, self.sources = PROFILED[name]
        self.rows = w.batch
        self.alg_bytes = select_bytes(w) + (4 * w.batch if logprobs else 0)
        d = upload.upload_select(w)
        nbytes = d["logits"].numel() * d["logits"].element_size()
        self.R = rotate if rotate is not None else _copies(nbytes)
        self.logits = _rotated(d["logits"], self.R)
        self.hists = _rotated(d["hist"], self.R)
        self.d = d
        self.params = d["params"]
        self.logprobs = logprobs
        dev = d["logits"].device
        self.out = torch.empty(w.batch, dtype=torch.int32, device=dev)
        self.lp = None
        self.ws = None
        if logprobs:
            self.params.output_logprobs = 1
            self.lp = torch.empty(w.batch, dtype=torch.float32, device=dev)
            self.ws = torch.empty(max(tsel.process_select_workspace_size(self.params), 256),
                                  dtype=torch.uint8, device=dev)
        self.tsel = tsel

    def step(self, i):
        self.tsel.process_select(self.logits[i % self.R], self.hists[i % self.R], self.d["lens"],
                                 self.params, self.d["u"], self.out, out_logprobs=self.lp,
                                 workspace=self.ws)

    def result(self):
        r = {"tokens": self.out.cpu().numpy().copy()}
        if self.lp is not None:
            r["logprobs"] = self.lp.cpu().numpy().copy()
        return r

    def oracle(self, threads, rows=None):
        import oracle
        w = self.w
        return oracle.select(w.logits, w.history, w.lens, w.prompt_lens, w.max_lengths,
                             oracle.Config(**w.settings), uniforms=w.uniforms, rows=rows,
                             threads=threads)

    def parity(self, got, ref, n):
        import numpy as np
        same = got["tokens"][:n] == ref["token"]
        p = {"rows": int(n), "exact_tokens": int(same.sum())}
        if "logprobs" in got:
            a = got["logprobs"][:n].view(np.int32).astype(np.int64)
            b = np.asarray(ref["logprob"], np.float32).view(np.int32).astype(np.int64)
            p["logprobs_within_2ulp"] = int((np.abs(a - b) <= 2).sum())
        return p


class VerifyCase(Case):
    def __init__(self, name, w, workload, rotate=None):
        import torch
        from logits_processing_token_amd import tsel, upload
        self.name, self.w, self.workload = name, w, workload
        self.kernels, self.traffic_file, self.sources = PROFILED[name]
        B, K1, V = w.logits.shape
        self.rows = B
        esize = 2 if w.dtype == "bf16" else 4
        self.alg_bytes = B * (K1 * V * esize + 4 * (K1 - 1) + 4 * (K1 - 1 + 4))
        d = upload.upload_verify(w)
        nbytes = d["logits"].numel() * d["logits"].element_size()
        self.R = rotate if rotate is not None else _copies(nbytes)
        self.logits = _rotated(d["logits"], self.R)
        self.d = d
        dev = d["logits"].device
        self.outs = (torch.empty(B, dtype=torch.int32, device=dev),
                     torch.empty((B, K1), dtype=torch.int32, device=dev),
                     torch.empty(B, dtype=torch.int32, device=dev),
                     torch.empty(B, dtype=torch.int32, device=dev))
        self.tsel = tsel

    def step(self, i):
        self.tsel.verify(self.logits[i % self.R], self.d["cand"], self.d["ws"], self.d["dtype"],
                         vocab=self.d["V"], outs=self.outs)

    def result(self):
        keys = ("n_match", "tokens", "next", "k_next")
        return {k: t.cpu().numpy().copy() for k, t in zip(keys, self.outs)}

    def oracle(self, threads, rows=None):
        import oracle
        x, c = self.w.logits, self.w.candidates
        if rows is not None:
            x, c = x[rows], c[rows]
        return oracle.verify(x, c, threads=threads)

    def parity(self, got, ref, n):
        import numpy as np
        same = np.ones(n, bool)
        for k in ("n_match", "tokens", "next", "k_next"):
            g, r = got[k][:n], ref[k]
            same &= (g == r) if g.ndim == 1 else (g == r).all(axis=1)
        return {"rows": int(n), "exact_rows": int(same.sum())}


class VerifySelectCase(Case):
    def __init__(self, name, w, workload, rotate=None):
        import numpy as np
        import torch
        from logits_processing_token_amd import tsel
        self.name, self.w, self.workload = name, w, workload
        self.kernels, self.traffic_file, self.sources = PROFILED[name]
        B, K1, V = w.logits.shape
        k = K1 - 1
        H = w.history.shape[1]
        self.rows = B
        esize = 2 if w.logits.dtype == np.uint16 else 4
        # each position row: its logits once; each batch row: its history,
        # drafts, uniforms, lengths and outputs
        self.alg_bytes = B * (K1 * V * esize + 4 * H + 4 * k + 4 * K1 + 12 + 4 * (K1 + 3))
        epc = 8 if esize == 2 else 4
        stride = ((V + epc - 1) // epc) * epc
        host = np.zeros((B, K1, stride), w.logits.dtype)
        host[:, :, :V] = w.logits
        dev = torch.device("cuda:0")
        logits = torch.from_numpy(host.view(np.int16) if esize == 2 else host).to(dev)
        self.R = rotate if rotate is not None else _copies(logits.numel() * esize)
        self.logits = _rotated(logits, self.R)
        dt = tsel.TSEL_BF16 if esize == 2 else tsel.TSEL_F32
        self.params = tsel.make_params(B, V, stride, dt, H, w.settings, {})
        self.hist = torch.from_numpy(w.history).to(dev)
        self.lens = torch.from_numpy(np.concatenate([w.lens, w.prompt_lens, w.max_lengths])
                                     .astype(np.int32)).to(dev)
        self.cand = torch.from_numpy(w.candidates).to(dev)
        self.u = torch.from_numpy(w.uniforms.reshape(-1).astype(np.float32)).to(dev)
        self.ws = torch.empty(max(int(tsel.load().tsel_verify_select_workspace_size(
            tsel.C.byref(self.params), k)), 256), dtype=torch.uint8, device=dev)
        self.outs = (torch.empty(B, dtype=torch.int32, device=dev),
                     torch.empty((B, K1), dtype=torch.int32, device=dev),
                     torch.empty(B, dtype=torch.int32, device=dev),
                     torch.empty(B, dtype=torch.int32, device=dev))
        self.tsel = tsel

    def step(self, i):
        self.tsel.verify_select(self.logits[i % self.R], self.hist, self.lens, self.params,
                                self.cand, self.u, workspace=self.ws, outs=self.outs)

    def result(self):
        keys = ("n_match", "tokens", "next", "k_next")
        return {k: t.cpu().numpy().copy() for k, t in zip(keys, self.outs)}

    def oracle(self, threads, rows=None):
        import oracle
        w = self.w
        sl = slice(None) if rows is None else rows
        return oracle.verify_select(w.logits[sl], w.candidates[sl], w.history[sl], w.lens[sl],
                                    w.prompt_lens[sl], w.max_lengths[sl],
                                    oracle.Config(**w.settings), uniforms=w.uniforms[sl],
                                    threads=threads)

    parity = VerifyCase.parity


class BeamCase(Case):
    def __init__(self, name, w, workload, rotate=None):
        import numpy as np
        import torch
        from logits_processing_token_amd import tsel, upload, synth
        self.name, self.w, self.workload = name, w, workload
        self.kernels, self.traffic_file, self.sources = PROFILED[name]
        sw = synth.SelectWorkload(w.name, w.logits, w.history, w.lens, w.prompt_lens,
                                  w.max_lengths, w.settings, None)
        rows, V = w.logits.shape
        self.prompts = rows // w.num_beams
        self.K = tsel.beam_width(w.num_beams, len(w.settings.get("eos_token_ids", [])))
        self.rows = rows
        # select_bytes counts the uniform and token of a row; a beam row has
        # its score instead, and each prompt writes K (score, beam, id)
        self.alg_bytes = select_bytes(sw) - 4 * rows + self.prompts * self.K * 12
        d = upload.upload_select(sw)
        nbytes = d["logits"].numel() * d["logits"].element_size()
        self.R = rotate if rotate is not None else _copies(nbytes)
        self.logits = _rotated(d["logits"], self.R)
        self.hists = _rotated(d["hist"], self.R)
        self.d = d
        dev = d["logits"].device
        self.bs = torch.from_numpy(np.ascontiguousarray(w.beam_scores)).to(dev)
        self.ws = torch.empty(max(int(tsel.load().tsel_beam_step_workspace_size(
            tsel.C.byref(d["params"]), w.num_beams)), 256), dtype=torch.uint8, device=dev)
        self.outs = (torch.empty((self.prompts, self.K), dtype=torch.float32, device=dev),
                     torch.empty((self.prompts, self.K), dtype=torch.int32, device=dev),
                     torch.empty((self.prompts, self.K), dtype=torch.int32, device=dev))
        self.tsel = tsel

    def step(self, i):
        self.tsel.beam_step(self.logits[i % self.R], self.hists[i % self.R], self.d["lens"],
                            self.d["params"], self.w.num_beams, self.bs, workspace=self.ws,
                            outs=self.outs)

    def result(self):
        return {k: t.cpu().numpy().copy() for k, t in zip(("scores", "beams", "tokens"),
                                                          self.outs)}

    def oracle(self, threads, rows=None):
        import oracle
        w = self.w
        sl = slice(None)
        if rows is not None:  # whole prompts
            nb = w.num_beams
            sl = slice(rows[0] * nb, (rows[-1] + 1) * nb)
        return oracle.beam_step(w.logits[sl], w.history[sl], w.lens[sl], w.prompt_lens[sl],
                                w.max_lengths[sl], oracle.Config(**w.settings), w.num_beams,
                                w.beam_scores[sl], threads=threads)

    def parity(self, got, ref, n):
        import numpy as np
        same = ((got["beams"][:n] == ref["beams"]).all(axis=1) &
                (got["tokens"][:n] == ref["tokens"]).all(axis=1) &
                (got["scores"][:n].view(np.uint32) == ref["scores"].view(np.uint32)).all(axis=1))
        return {"prompts": int(n), "exact_prompts": int(same.sum())}


def make_case(name: str) -> Case:
    from logits_processing_token_amd import synth
    if name == "C1":
        return SelectCase("C1", synth.c1_select(),
                          "C1 greedy: B=1 V=50272 fp32 logits N(0,3), history 64, "
                          "repetition_penalty 1.2 (warm latency)", rotate=1)
    if name == "C1v":
        return VerifyCase("C1v", synth.c1_verify(),
                          "C1 verify: [1, 6, 50272] fp32 N(0,3), k=5 greedy drafts (warm latency)",
                          rotate=1)
    if name == "C2":
        return SelectCase("C2", synth.c2_select(),
                          "C2: B=64 V=32000 bf16 N(0,2), history 1024 with planted 3-gram "
                          "repeats; rep 1.1, no_repeat_ngram 3, min_new_tokens 300 (eos 2), "
                          "temperature 0.7, top_k 50, top_p 0.9, sampling")
    if name == "C3":
        return SelectCase("C3", synth.c3_select(),
                          "C3 full chain: B=256 V=128256 bf16 logits, log-Zipf(1.1) over a "
                          "random permutation + N(0,1); history 4096; repetition_penalty 1.05; "
                          "100 suppress_tokens; 50 bad words; temperature 1.0; top_p 0.95; "
                          "inverse-CDF sampling", rotate=8)
    if name == "C4":
        return VerifyCase("C4", synth.c4_verify(),
                          "C4 verify: [32, 9, 151936] bf16 N(0,3), k=8 greedy drafts",
                          rotate=6)
    if name == "C5":
        return SelectCase("C5", synth.c5_select(),
                          "C5: B=1024 V=262144 fp32, log-Zipf(1.2) + N(0,0.5); history 8192 "
                          "with planted 4-gram repeats; rep 1.1, no_repeat_ngram 4, forced_eos "
                          "on 102 rows, temperature 0.8, top_k 64, top_p 0.95, sampling",
                          rotate=1)
    if name == "F1":
        return SelectCase("F1", synth.c3_select(),
                          "C3 with the token log-probability (output_logprobs)",
                          rotate=8, logprobs=True)
    if name == "F2":
        return BeamCase("F2", synth.c3_beam(),
                        "one beam-search step over the C3 batch read as 64 prompts x 4 beams "
                        "(V=128256 bf16, history 4096, rep 1.05, 100 suppress, 50 bad words, "
                        "1 eos id: K=8 per prompt)", rotate=8)
    if name == "F3":
        return VerifySelectCase("F3", synth.c4_verify_select(),
                                "verification with sampling at every position: [32, 9, 151936] "
                                "bf16 N(0,3), k=8, history 256, rep 1.1, temperature 0.7, "
                                "top_p 0.9", rotate=6)
    raise ValueError(f"unknown config {name}")


CONFIGS = ("C1", "C1v", "C2", "C3", "C4", "C5", "F1", "F2", "F3")
# single-thread oracle figures (a bounded sample) for the small configs
SINGLE_THREAD_ROWS = {"C1": 1, "C1v": 1, "C2": 8, "C3": 4}
# rows of the multi-thread oracle sample; None = the whole batch
ORACLE_ROWS = {"C5": 64, "F2": 16, "F3": 8}


def run_case(case: Case, args, ceiling=None) -> dict:
    import numpy as np
    import torch
    print(f"bench: {case.name}: warmup", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        case.step(i)
    torch.cuda.synchronize()
    case.step(0)
    torch.cuda.synchronize()
    got = case.result()

    K = args.steps
    # One event pair on the launch stream brackets the K steps: the mean step
    # time includes the gaps between launches (an event pair per launch would
    # put its own timestamp packets between the kernels).
    stream = torch.cuda.current_stream()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    print(f"bench: {case.name}: timing {K} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(K):
        case.step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    step_ms = ev0.elapsed_time(ev1) / K

    achieved = case.alg_bytes / (step_ms * 1e-3) / 1e9
    traffic = measured_traffic(case.traffic_file, case.sources) if case.traffic_file else None
    result = {
        "metric": METRIC,
        "value": case.rows * K / elapsed,
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
        "config": {"workload": case.workload, "name": case.name, "rows": case.rows,
                   "rotated_copies": case.R},
        "kernel_ms": step_ms,
        "kernel_us": step_ms * 1e3,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": traffic,
                     "algorithmic_bytes": case.alg_bytes,
                     "kernel": " + ".join(case.kernels)},
    }
    if ceiling:
        result["roofline"]["measured_read_ceiling"] = ceiling
        result["roofline"]["frac_of_measured_ceiling"] = achieved / ceiling
    if not args.no_cpu_baseline:
        threads = host_threads()
        rows = ORACLE_ROWS.get(case.name)
        sel = None
        n = case.rows if not isinstance(case, BeamCase) else case.prompts
        if rows is not None and rows < n:
            sel = list(range(rows))
            n = rows
        print(f"bench: {case.name}: oracle on {n} rows, {threads} threads", file=sys.stderr,
              flush=True)
        t0 = time.perf_counter()
        ref = case.oracle(threads, sel)
        dt = time.perf_counter() - t0
        unit_rows = n * (case.w.num_beams if isinstance(case, BeamCase) else 1)
        base = {"value": unit_rows / dt, "unit": "rows/s", "cores": threads, "kind": "oracle",
                "sample": f"{'the first ' + str(n) if sel else 'all ' + str(n)} "
                          f"{'prompts' if isinstance(case, BeamCase) else 'rows'} of the "
                          f"workload, one pass ({dt:.2f} s wall on {threads} threads)",
                "cpu_model": cpu_model(), "host_cpus": os.cpu_count()}
        one = SINGLE_THREAD_ROWS.get(case.name)
        if one:
            sel1 = list(range(min(one, case.rows)))
            t1 = time.perf_counter()
            case.oracle(1, sel1)
            d1 = time.perf_counter() - t1
            base["single_thread"] = {"value": len(sel1) / d1, "unit": "rows/s",
                                     "sample": f"the first {len(sel1)} rows ({d1:.2f} s)"}
        result["cpu_baseline"] = base
        result["parity"] = case.parity(got, ref, n)
    return result


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="C3", help="one of %s, or all" % ", ".join(CONFIGS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the measured HBM read ceiling (a plain streaming kernel)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a plain 256 MiB device copy (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(rows would shard with no exchange); run with --gpus 1", file=sys.stderr)
        return 2
    names = CONFIGS if args.config == "all" else tuple(args.config.split(","))
    for n in names:
        if n not in CONFIGS:
            print(f"unknown config {n}; one of {', '.join(CONFIGS)} or all", file=sys.stderr)
            return 2

    import torch
    from logits_processing_token_amd import tsel

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    tsel.load()
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        src = torch.empty(64 << 20, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    ceiling = None
    if not args.no_ceiling:
        print("bench: read ceiling", file=sys.stderr, flush=True)
        ceiling = read_ceiling_gbs(dev)
    for n in names:
        print(f"bench: {n}: generating the workload", file=sys.stderr, flush=True)
        case = make_case(n)
        print(json.dumps(run_case(case, args, ceiling)), flush=True)
        del case
        torch.cuda.empty_cache()
    return 0


if __name__ == "__main__":
    sys.exit(main())
