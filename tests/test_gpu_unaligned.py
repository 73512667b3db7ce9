"""GPU: logits rows whose byte stride is not a multiple of 16 (a contiguous
batch with an odd vocabulary).  The library copies them to an aligned stride
in the workspace first, so every output must equal, bit for bit, what the
same rows give at an aligned stride -- whose parity with the oracle the
other GPU tests establish -- on the selection (greedy, sampling with
log-probabilities, fp32 and bf16), the beam step and sampled verification.
Greedy ids are also compared with the oracle directly."""
import os
import sys

import numpy as np
import pytest

import oracle
from logits_processing_token_amd import synth

pytestmark = pytest.mark.gpu

sys.path.insert(0, os.path.dirname(__file__))
from test_gpu_parity import _gpu  # noqa: E402,F401


def _say(*a):
    print(*a, flush=True)


def _dev_rows(x, stride):
    """Device copy of rows x [..., V] at `stride` elements per row."""
    import torch
    host = np.zeros(x.shape[:-1] + (stride,), x.dtype)
    host[..., :x.shape[-1]] = x
    t = torch.from_numpy(host.view(np.int16) if host.dtype == np.uint16 else host)
    return t.to(torch.device("cuda:0"))


def _aligned(V, dt_bits):
    epc = 8 if dt_bits == 16 else 4
    return V + (-V) % epc


def _select(w, stride):
    import torch
    from logits_processing_token_amd import tsel
    B, V = w.logits.shape
    dev = torch.device("cuda:0")
    dt = tsel.TSEL_BF16 if w.dtype == "bf16" else tsel.TSEL_F32
    s = dict(w.settings)
    params = tsel.make_params(B, V, stride, dt, w.history.shape[1], s, {})
    lens = torch.from_numpy(np.concatenate([w.lens, w.prompt_lens, w.max_lengths])
                            .astype(np.int32)).to(dev)
    u = None if w.uniforms is None else torch.from_numpy(w.uniforms.astype(np.float32)).to(dev)
    out = tsel.process_select(_dev_rows(w.logits, stride),
                              torch.from_numpy(np.ascontiguousarray(w.history)).to(dev), lens,
                              params, u)
    torch.cuda.synchronize()
    if isinstance(out, tuple):
        return out[0].cpu().numpy(), out[1].cpu().numpy()
    return out.cpu().numpy(), None


@pytest.mark.parametrize("dtype,V,sample", [
    ("bf16", 50273, False), ("bf16", 50273, True), ("f32", 5001, False), ("f32", 5001, True),
    ("bf16", 131071, True),
])
def test_select_unaligned_stride(dtype, V, sample):
    settings = dict(repetition_penalty=1.2, output_logprobs=True)
    if sample:
        settings.update(do_sample=True, temperature=0.8, top_p=0.9)
    w = synth.random_select(4100 + V, batch=6, vocab=V, hist_len=40, dtype=dtype,
                            settings=settings)
    bits = 16 if dtype == "bf16" else 32
    _say(f"  select {dtype} V {V} sample {sample}: stride {V} against {_aligned(V, bits)}")
    tu, lu = _select(w, V)
    ta, la = _select(w, _aligned(V, bits))
    assert np.array_equal(tu, ta), (tu, ta)
    assert np.array_equal(lu.view(np.uint32), la.view(np.uint32)), (lu, la)
    if not sample:
        cfg = {k: v for k, v in w.settings.items() if k != "output_logprobs"}
        r = oracle.select(w.logits, w.history, w.lens, w.prompt_lens, w.max_lengths,
                          oracle.Config(**cfg), threads=16)
        assert np.array_equal(tu, r["token"]), (tu, r["token"])


def test_beam_unaligned_stride():
    import torch
    from logits_processing_token_amd import tsel
    g = np.random.default_rng(77)
    P, nb, V = 3, 4, 50273
    rows = P * nb
    x = synth.bf16_bits((g.standard_normal((rows, V)) * 2.0).astype(np.float32))
    hist = g.integers(0, V, (rows, 24)).astype(np.int32)
    L = np.full(rows, 24, np.int32)
    dev = torch.device("cuda:0")
    lens = torch.from_numpy(np.concatenate([L, L, np.full(rows, 1 << 30, np.int32)])).to(dev)
    bs = torch.from_numpy((-6.0 * g.random(rows)).astype(np.float32)).to(dev)
    s = dict(repetition_penalty=1.3, eos_token_ids=[2])
    got = []
    for stride in (V, _aligned(V, 16)):
        _say(f"  beam step V {V} stride {stride}")
        params = tsel.make_params(rows, V, stride, tsel.TSEL_BF16, 24, s, {})
        sc, bm, tk = tsel.beam_step(_dev_rows(x, stride), torch.from_numpy(hist).to(dev), lens,
                                    params, nb, bs)
        torch.cuda.synchronize()
        got.append((sc.cpu().numpy().view(np.uint32), bm.cpu().numpy(), tk.cpu().numpy()))
    for a, b in zip(*got):
        assert np.array_equal(a, b), (a, b)


def test_verify_select_unaligned_stride():
    import torch
    from logits_processing_token_amd import tsel
    g = np.random.default_rng(78)
    B, k, V = 4, 3, 50273
    x = synth.bf16_bits((g.standard_normal((B, k + 1, V)) * 2.0).astype(np.float32))
    hist = g.integers(0, V, (B, 32)).astype(np.int32)
    cand = g.integers(0, V, (B, k)).astype(np.int32)
    L = np.full(B, 32, np.int32)
    u = synth.uniforms(g, B * (k + 1)).astype(np.float32)
    dev = torch.device("cuda:0")
    lens = torch.from_numpy(np.concatenate([L, L, np.full(B, 1 << 30, np.int32)])).to(dev)
    s = dict(do_sample=True, temperature=0.7, top_p=0.9, repetition_penalty=1.1)
    got = []
    for stride in (V, _aligned(V, 16)):
        _say(f"  verify_select V {V} stride {stride}")
        params = tsel.make_params(B, V, stride, tsel.TSEL_BF16, 32, s, {})
        outs = tsel.verify_select(_dev_rows(x, stride), torch.from_numpy(hist).to(dev), lens,
                                  params, torch.from_numpy(cand).to(dev),
                                  torch.from_numpy(u).to(dev))
        torch.cuda.synchronize()
        got.append([o.cpu().numpy() for o in outs])
    for a, b in zip(*got):
        assert np.array_equal(a, b), (a, b)
