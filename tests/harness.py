"""Helpers shared by the GPU parity tests: upload a seeded workload, run the
HIP library through its C ABI, run the CPU oracle on the same host arrays,
and compare the two under the exactness policy:

* token ids, match counts and next counts are compared exactly;
* sampled rows whose decision margin (normalized probability mass) is below
  MARGIN are counted apart; for them the GPU id must be one of the oracle's
  admissible ids (those some perturbation of the cumulative sums by 1e-6 of
  the kept mass selects);
* processed scores are compared bit for bit where both sides keep an id.
"""
from __future__ import annotations

import numpy as np

import oracle
from logits_processing_token_amd import synth

MARGIN = 1e-4


def torch_mod():
    import torch
    return torch


def upload_select(w: synth.SelectWorkload, stride_pad: int = 0):
    """Device tensors of a selection workload.  Rows are padded to a stride
    that keeps every row 16-byte aligned (plus stride_pad elements)."""
    from logits_processing_token_amd import tsel
    torch = torch_mod()
    dev = torch.device("cuda:0")
    B, V = w.logits.shape
    epc = 8 if w.dtype == "bf16" else 4
    stride = ((V + epc - 1) // epc) * epc + stride_pad * epc
    if w.dtype == "bf16":
        host = np.zeros((B, stride), np.uint16)
        host[:, :V] = w.logits
        logits = torch.from_numpy(host.view(np.int16)).to(dev)
        dtype = tsel.TSEL_BF16
    else:
        host = np.zeros((B, stride), np.float32)
        host[:, :V] = w.logits
        logits = torch.from_numpy(host).to(dev)
        dtype = tsel.TSEL_F32
    hist = torch.from_numpy(np.ascontiguousarray(w.history, dtype=np.int32)).to(dev)
    lens = torch.from_numpy(np.concatenate([w.lens, w.prompt_lens, w.max_lengths])
                            .astype(np.int32)).to(dev)
    u = None if w.uniforms is None else torch.from_numpy(w.uniforms.astype(np.float32)).to(dev)
    masks = {}
    for name in ("bad_words_ids", "suppress_tokens", "begin_suppress_tokens"):
        ids = w.settings.get(name)
        if ids:
            t = torch.tensor(list(ids), dtype=torch.int32, device=dev)
            masks[name] = tsel.mask_build(V, t)
    params = tsel.make_params(B, V, stride, dtype, w.history.shape[1], w.settings, masks)
    return dict(logits=logits, hist=hist, lens=lens, u=u, masks=masks, params=params,
                stride=stride)


def run_gpu_select(w: synth.SelectWorkload, want_processed: bool = False,
                   stride_pad: int = 0) -> dict:
    from logits_processing_token_amd import tsel
    torch = torch_mod()
    d = upload_select(w, stride_pad)
    B, V = w.logits.shape
    out = torch.full((B,), -7, dtype=torch.int32, device="cuda:0")
    proc = None
    if want_processed:
        proc = torch.full((B, V), float("nan"), dtype=torch.float32, device="cuda:0")
    tsel.process_select(d["logits"], d["hist"], d["lens"], d["params"], d["u"], out, proc)
    torch.cuda.synchronize()
    res = {"token": out.cpu().numpy()}
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
               high_margin_mismatch=[], not_admissible=[], processed_mismatch=[])
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
        if check_processed and g == o:
            gp, op = gpu["processed"][b], ora["processed"][i]
            if low:
                both = np.isfinite(gp) & np.isfinite(op)
                ok = np.array_equal(gp[both].view(np.uint32), op[both].view(np.uint32))
            else:
                ok = np.array_equal(gp.view(np.uint32), op.view(np.uint32))
            if not ok:
                rep["processed_mismatch"].append(b)
    return rep


def upload_verify(w: synth.VerifyWorkload):
    """Device tensors of a verification workload; rows are padded to a
    16-byte multiple so that every row starts aligned."""
    from logits_processing_token_amd import tsel
    torch = torch_mod()
    dev = torch.device("cuda:0")
    B, K1, V = w.logits.shape
    epc = 8 if w.dtype == "bf16" else 4
    stride = ((V + epc - 1) // epc) * epc
    if w.dtype == "bf16":
        host = np.zeros((B, K1, stride), np.uint16)
        host[:, :, :V] = w.logits
        logits = torch.from_numpy(host.view(np.int16)).to(dev)
        dtype = tsel.TSEL_BF16
    else:
        host = np.zeros((B, K1, stride), np.float32)
        host[:, :, :V] = w.logits
        logits = torch.from_numpy(host).to(dev)
        dtype = tsel.TSEL_F32
    cand = torch.from_numpy(np.ascontiguousarray(w.candidates, dtype=np.int32)).to(dev)
    ws = torch.zeros(max(tsel.verify_workspace_size(B, K1 - 1, V), 16), dtype=torch.uint8,
                     device=dev)
    return dict(logits=logits, cand=cand, ws=ws, dtype=dtype, V=V, stride=stride)


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
