"""Device copies of a seeded workload (``synth``): the logits padded to a
16-byte aligned row stride, the history, the three length arrays, the
uniforms, the static masks (built on the device by ``tsel_mask_build``) and
the params struct.  Plumbing shared by the tests and the benchmark; no
arithmetic of the method happens here.
"""
from __future__ import annotations

import numpy as np

from . import synth


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
    ws = torch.empty(max(tsel.verify_workspace_size(B, K1 - 1, V), 16), dtype=torch.uint8,
                     device=dev)
    return dict(logits=logits, cand=cand, ws=ws, dtype=dtype, V=V, stride=stride)
