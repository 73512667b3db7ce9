"""Helpers shared by the GPU parity tests: upload a seeded workload, run the
HIP library through its C ABI, run the CPU oracle on the same host arrays,
and compare the two under the exactness policy:

* token ids, match counts and next counts are compared exactly;
* sampled rows whose decision margin (normalized probability mass) is below
  MARGIN are counted apart; for them the GPU id must be one of the oracle's
  admissible ids (those some perturbation of the cumulative sums by 1e-6 of
  the kept mass selects);
* processed scores are compared bit for bit where both sides keep an id;
  the kept sets must be equal, except in a low-margin sampled row, where the
  GPU's kept set may differ from the oracle's only at the top_p boundary: it
  must be a prefix of the same (score desc, id asc) order whose size lies in
  the oracle's [keep_min, keep_max].
"""
from __future__ import annotations

import numpy as np

import oracle
from logits_processing_token_amd import synth
from logits_processing_token_amd.upload import upload_select, upload_verify  # noqa: F401

MARGIN = 1e-4


def torch_mod():
    import torch
    return torch


def run_gpu_select(w: synth.SelectWorkload, want_processed: bool = False,
                   stride_pad: int = 0, want_logprobs: bool = False) -> dict:
    from logits_processing_token_amd import tsel
    torch = torch_mod()
    d = upload_select(w, stride_pad)
    B, V = w.logits.shape
    out = torch.full((B,), -7, dtype=torch.int32, device="cuda:0")
    proc = None
    if want_processed:
        proc = torch.full((B, V), float("nan"), dtype=torch.float32, device="cuda:0")
    params = d["params"]
    params.output_logprobs = int(want_logprobs)
    r = tsel.process_select(d["logits"], d["hist"], d["lens"], params, d["u"], out, proc)
    torch.cuda.synchronize()
    res = {"token": out.cpu().numpy()}
    if want_logprobs:
        res["logprob"] = r[1].cpu().numpy()
    if want_processed:
        res["processed"] = proc.cpu().numpy()
    return res


def run_oracle_select(w: synth.SelectWorkload, rows=None, want_processed=False,
                      threads: int = 16) -> dict:
    return oracle.select(w.logits, w.history, w.lens, w.prompt_lens, w.max_lengths,
                         oracle.Config(**w.settings), uniforms=w.uniforms, rows=rows,
                         want_processed=want_processed, threads=threads)


def compare_select(w: synth.SelectWorkload, gpu: dict, ora: dict, rows=None,
                   check_processed: bool = False) -> dict:
    """Compare GPU results (full batch) with oracle results (for rows)."""
    rows = list(range(w.batch)) if rows is None else list(rows)
    sampling = bool(w.settings.get("do_sample"))
    rep = dict(rows=len(rows), exact=0, low_margin=0, low_margin_mismatch=0,
               high_margin_mismatch=[], not_admissible=[], processed_mismatch=[],
               logprob_mismatch=[])
    for i, b in enumerate(rows):
        g, o = int(gpu["token"][b]), int(ora["token"][i])
        low = sampling and ora["margin"][i] < MARGIN
        if low:
            rep["low_margin"] += 1
            if g != o:
                rep["low_margin_mismatch"] += 1
                if g not in ora["admissible"][i].tolist():
                    rep["not_admissible"].append((b, g, o, float(ora["margin"][i])))
            else:
                rep["exact"] += 1
        else:
            if g == o:
                rep["exact"] += 1
            else:
                rep["high_margin_mismatch"].append((b, g, o))
        if "logprob" in gpu and g == o and not logprobs_agree(gpu["logprob"][b], ora["logprob"][i]):
            # a low-margin row may keep a different top_p set (see the kept
            # sets below); its log-probability must then be the log-softmax
            # of the GPU's own kept scores at the token
            if check_processed:
                own = low and logprobs_agree(gpu["logprob"][b], logprob_of(gpu["processed"][b], g))
            else:  # (without the GPU's kept set: any count the margin allows)
                own = low and any(logprobs_agree(gpu["logprob"][b], c) for c in logprob_over_prefixes(
                    w, b, g, int(ora["keep_min"][i]), int(ora["keep_max"][i])))
            if not own:
                rep["logprob_mismatch"].append((b, float(gpu["logprob"][b]),
                                                float(ora["logprob"][i])))
        if check_processed and g == o:
            gp, op = gpu["processed"][b], ora["processed"][i]
            if low:
                ok = kept_sets_agree(gp, op, int(ora["keep_min"][i]), int(ora["keep_max"][i]))
            else:
                ok = np.array_equal(gp.view(np.uint32), op.view(np.uint32))
            if not ok:
                rep["processed_mismatch"].append(b)
    return rep


def logprob_of(row: np.ndarray, t: int) -> np.float32:
    """The log-softmax of a row of final scores at t, in binary64."""
    x = row.astype(np.float64)
    fin = np.isfinite(x)
    if not fin.any():
        return np.float32(np.nan)
    m = x[fin].max()
    return np.float32((x[t] - m) - np.log(np.sum(np.exp(x[fin] - m))))


def logprob_over_prefixes(w: synth.SelectWorkload, b: int, t: int, keep_min: int,
                          keep_max: int) -> list:
    """The log-probability of token t of row b over each kept set a top_p
    boundary within the margin allows: the first k final scores in (score
    desc, id asc) order, keep_min <= k <= keep_max, from the oracle's scores
    before the top_p cut, in binary64."""
    cfg = oracle.Config(**dict(w.settings, top_p=1.0))
    r = oracle.select(w.logits, w.history, w.lens, w.prompt_lens, w.max_lengths, cfg,
                      uniforms=w.uniforms, rows=[b], want_processed=True)
    x = r["processed"][0].astype(np.float64)
    fin = np.flatnonzero(np.isfinite(x))
    if fin.size == 0:
        return []
    order = fin[np.lexsort((fin, -x[fin]))]
    m = x[order[0]]
    cs = np.cumsum(np.exp(x[order] - m))
    pos = {int(v): k for k, v in enumerate(order)}
    if t not in pos:
        return []
    return [np.float32((x[t] - m) - np.log(cs[k - 1]))
            for k in range(max(keep_min, pos[t] + 1), min(keep_max, order.size) + 1)]


def logprobs_agree(g: float, o: float) -> bool:
    """Both sides take the log-sum-exp in binary64 and round once: the same
    binary32 value up to a rounding boundary the two sums straddle (2 ulp
    allowed); NaN must meet NaN with the same bits."""
    g, o = np.float32(g), np.float32(o)
    if np.isnan(o) or np.isnan(g):
        return bool(np.isnan(o) and np.isnan(g) and g.view(np.uint32) == o.view(np.uint32))
    if np.isinf(o) or np.isinf(g):
        return bool(g == o)
    return bool(abs(float(g) - float(o)) <= 2 * float(np.spacing(np.abs(o))))


def kept_sets_agree(gp: np.ndarray, op: np.ndarray, keep_min: int, keep_max: int) -> bool:
    """Processed rows of a low-margin sampled row: bit-equal scores where
    both keep an id; the two kept sets prefixes of one (score desc, id asc)
    order over the scores either side keeps; the GPU's count within the
    oracle's allowed range."""
    gk, ok_ = np.isfinite(gp), np.isfinite(op)
    both = gk & ok_
    if not np.array_equal(gp[both].view(np.uint32), op[both].view(np.uint32)):
        return False
    if np.array_equal(gk, ok_):
        return True
    n = int(gk.sum())
    if not keep_min <= n <= keep_max:
        return False
    union = np.flatnonzero(gk | ok_)
    val = np.where(gk[union], gp[union], op[union])
    order = union[np.lexsort((union, -val.astype(np.float64)))]
    rank = np.empty(gp.size, np.int64)
    rank[order] = np.arange(order.size)
    return bool(rank[gk].max() == n - 1 and rank[ok_].max() == int(ok_.sum()) - 1)


def run_gpu_verify(w: synth.VerifyWorkload, d=None) -> dict:
    from logits_processing_token_amd import tsel
    torch = torch_mod()
    d = d or upload_verify(w)
    n, t, nx, kk = tsel.verify(d["logits"], d["cand"], d["ws"], d["dtype"], vocab=d["V"],
                               row_stride=d["stride"])
    torch.cuda.synchronize()
    return {"n_match": n.cpu().numpy(), "tokens": t.cpu().numpy(), "next": nx.cpu().numpy(),
            "k_next": kk.cpu().numpy()}


def compare_verify(gpu: dict, ora: dict) -> list:
    bad = []
    for key in ("n_match", "tokens", "next", "k_next"):
        if not np.array_equal(gpu[key], ora[key]):
            bad.append(key)
    return bad
