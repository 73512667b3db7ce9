"""GPU: determinism.  The same inputs give the same outputs, bit for bit,
over ten launches, and a row's result does not depend on the batch it sits
in: each path's batch is run whole, then as a subset of its rows in another
order (another grid size, other row positions).  Covered: the value-bin
kernel (bf16, no top_k, T = 1), the resident fp32 kernel, top-k, the
streamed full path (bf16, T != 1, a vocabulary past the registers), greedy,
greedy verification (chunk keys merged per row) and the beam step (row keys
merged per prompt)."""
import os
import sys
from dataclasses import replace

import numpy as np
import pytest

from logits_processing_token_amd import synth

pytestmark = pytest.mark.gpu

sys.path.insert(0, os.path.dirname(__file__))
from harness import run_gpu_select, run_gpu_verify  # noqa: E402
from test_gpu_parity import _gpu  # noqa: E402,F401

REPEATS = 10


def _say(*a):
    print(*a, flush=True)


def _rows(w, idx):
    """The workload restricted to rows idx, in that order."""
    idx = np.asarray(idx)
    return replace(w, logits=w.logits[idx].copy(), history=w.history[idx].copy(),
                   lens=w.lens[idx].copy(), prompt_lens=w.prompt_lens[idx].copy(),
                   max_lengths=w.max_lengths[idx].copy(),
                   uniforms=None if w.uniforms is None else w.uniforms[idx].copy())


def _bits(r):
    out = {"token": r["token"]}
    if "logprob" in r:
        out["logprob"] = r["logprob"].view(np.uint32)
    return out


SELECT_CASES = {
    "value bins": lambda: synth.c3_select(batch=24),
    "resident fp32": lambda: synth.random_select(
        61, batch=24, vocab=30011, hist_len=300, dtype="f32",
        settings=dict(do_sample=True, top_p=0.9, repetition_penalty=1.2, suppress_tokens=[5, 9])),
    "top-k": lambda: synth.c2_select(batch=24),
    "full streamed": lambda: synth.random_select(
        62, batch=24, vocab=151936, hist_len=200, dtype="bf16", sigma=3.0,
        settings=dict(do_sample=True, temperature=0.7, top_p=0.9, repetition_penalty=1.1)),
    "greedy": lambda: synth.random_select(
        63, batch=24, vocab=50272, hist_len=64, dtype="f32",
        settings=dict(repetition_penalty=1.3, no_repeat_ngram_size=2)),
}


@pytest.mark.parametrize("name", list(SELECT_CASES))
def test_select_repeats_and_row_independence(name):
    w = SELECT_CASES[name]()
    _say(f"  {name}: B {w.batch} V {w.vocab} {w.dtype}")
    ref = _bits(run_gpu_select(w, want_logprobs=True))
    for i in range(REPEATS - 1):
        got = _bits(run_gpu_select(w, want_logprobs=True))
        for k in ref:
            assert np.array_equal(got[k], ref[k]), (name, "launch", i + 1, k)
    idx = np.arange(w.batch)[::-1][::2]  # every other row, reversed
    sub = _bits(run_gpu_select(_rows(w, idx), want_logprobs=True))
    for k in ref:
        assert np.array_equal(sub[k], ref[k][idx]), (name, "subset", k)


def test_verify_repeats_and_row_independence():
    w = synth.c4_verify(batch=12)
    _say(f"  verify: {w.logits.shape}")
    ref = run_gpu_verify(w)
    for i in range(REPEATS - 1):
        got = run_gpu_verify(w)
        for k in ref:
            assert np.array_equal(got[k], ref[k]), ("launch", i + 1, k)
    idx = np.array([11, 4, 7, 0])
    sub = run_gpu_verify(replace(w, logits=w.logits[idx].copy(),
                                 candidates=w.candidates[idx].copy()))
    for k in ref:
        assert np.array_equal(sub[k], ref[k][idx]), ("subset", k)


def test_beam_repeats_and_prompt_independence():
    import torch
    from logits_processing_token_amd import tsel
    g = np.random.default_rng(64)
    P, nb, V = 6, 4, 32000
    rows = P * nb
    x = synth.bf16_bits((g.standard_normal((rows, V)) * 2.0).astype(np.float32))
    hist = g.integers(0, V, (rows, 32)).astype(np.int32)
    bs = (-6.0 * g.random(rows)).astype(np.float32)
    dev = torch.device("cuda:0")
    s = dict(repetition_penalty=1.2, eos_token_ids=[2])

    def run(prompts):
        r = np.concatenate([np.arange(p * nb, (p + 1) * nb) for p in prompts])
        n = len(r)
        L = np.full(n, 32, np.int32)
        stride = V + (-V) % 8
        host = np.zeros((n, stride), np.uint16)
        host[:, :V] = x[r]
        params = tsel.make_params(n, V, stride, tsel.TSEL_BF16, 32, s, {})
        lens = torch.from_numpy(np.concatenate([L, L, np.full(n, 1 << 30, np.int32)])).to(dev)
        sc, bm, tk = tsel.beam_step(torch.from_numpy(host.view(np.int16)).to(dev),
                                    torch.from_numpy(hist[r].copy()).to(dev), lens, params, nb,
                                    torch.from_numpy(bs[r].copy()).to(dev))
        torch.cuda.synchronize()
        return sc.cpu().numpy().view(np.uint32), bm.cpu().numpy(), tk.cpu().numpy()

    ref = run(range(P))
    for i in range(REPEATS - 1):
        for a, b in zip(run(range(P)), ref):
            assert np.array_equal(a, b), ("launch", i + 1)
    idx = [5, 2, 3]
    for a, b in zip(run(idx), ref):
        assert np.array_equal(a, b[idx]), "subset"
