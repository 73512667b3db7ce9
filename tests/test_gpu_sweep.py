"""A seeded sweep of the selection over mixed settings: each case draws the
vocabulary (ragged sizes, resident and streamed rows, both dtypes), the
history (repeats, planted n-grams), the processors of "Transmuter.Generation
(transmuter v2.0.0)" in their module-doc order, and the warpers (greedy,
temperature, top_k, top_p), and compares token ids and processed rows with
the oracle as the named parity tests do.  Lengths are mixed too, so that the
forced, begin-suppress and minimum-length rules fire on some rows.  Beam
steps and verification with selection get sweeps of their own, checked by
their parity tests' helpers."""
import os
import sys

import numpy as np
import pytest

from logits_processing_token_amd import synth

pytestmark = pytest.mark.gpu

sys.path.insert(0, os.path.dirname(__file__))
from test_gpu_parity import _assert_select, _gpu  # noqa: E402,F401

VOCABS = [97, 4099, 32000, 50273, 131072, 151936, 200003]


def _case(seed):
    g = np.random.default_rng(9000 + seed)
    V = int(g.choice(VOCABS))
    dtype = "bf16" if g.random() < 0.6 else "f32"
    B = 3
    H = int(g.choice([0, 8, 300, 2500]))
    id_range = int(g.choice([V, max(8, V // 50)]))
    s = {}
    if g.random() < 0.7:
        s["repetition_penalty"] = float(g.choice([1.3, 0.8, 1.05]))
    if g.random() < 0.4:
        s["no_repeat_ngram_size"] = int(g.choice([2, 3]))
    if g.random() < 0.5:
        s["bad_words_ids"] = [int(v) for v in g.choice(V, size=min(V, 20), replace=False)]
    if g.random() < 0.5:
        s["suppress_tokens"] = [int(v) for v in g.choice(V, size=min(V, 10), replace=False)]
    eos = [int(v) for v in g.choice(V, size=2, replace=False)]
    if g.random() < 0.6:
        s["eos_token_ids"] = eos
        if g.random() < 0.5:
            s["min_new_tokens"] = 4
    if g.random() < 0.3:
        s["begin_suppress_tokens"] = [int(v) for v in g.choice(V, size=min(V, 5), replace=False)]
    if g.random() < 0.3:
        s["forced_eos_token_id"] = eos[0]
    if g.random() < 0.7:
        s["do_sample"] = True
        s["temperature"] = float(g.choice([1.0, 0.7, 1.3]))
        s["top_k"] = int(g.choice([0, 0, 1, 5, 64, 1000]))
        s["top_p"] = float(g.choice([1.0, 0.9, 0.5]))
    L = max(H, 1)
    lens = np.array([L, max(L - 2, 1), L], np.int32)
    prompt = np.array([L, max(L - 3, 0), L], np.int32)
    maxl = np.array([1 << 30, 1 << 30, L + 1], np.int32)  # (row 2 one short of max_length)
    w = synth.random_select(seed + 500, B, V, H, dtype=dtype, sigma=float(g.choice([1.0, 3.0])),
                            settings=s, id_range=id_range, lens=lens, prompt_lens=prompt,
                            max_lengths=maxl, plant_n=3 if H >= 8 else 0)
    return w


@pytest.mark.parametrize("seed", list(range(64)))
def test_selection_sweep(seed):
    _assert_select(_case(seed))


def _beam_case(seed):
    from test_gpu_beam import _workload
    g = np.random.default_rng(9500 + seed)
    V = int(g.choice([7, 4099, 32000, 50257, 151936]))
    dtype = "bf16" if g.random() < 0.6 else "f32"
    nb = int(g.choice([1, 2, 4, 8]))
    P = int(g.choice([1, 3]))
    s = {}
    if g.random() < 0.7:
        s["repetition_penalty"] = float(g.choice([1.3, 0.8, 1.05]))
    if g.random() < 0.4 and V > 8:
        s["no_repeat_ngram_size"] = 2
    if g.random() < 0.5:
        s["bad_words_ids"] = [int(v) for v in g.choice(V, size=min(V, 5), replace=False)]
    if g.random() < 0.5:
        s["suppress_tokens"] = [int(v) for v in g.choice(V, size=min(V, 3), replace=False)]
    s["eos_token_ids"] = [int(v) for v in g.choice(V, size=int(g.choice([0, 1, 3])), replace=False)]
    return _workload(seed + 700, P, nb, V, dtype, s, hist_len=int(g.choice([4, 60])),
                     scale=float(g.choice([1.0, 3.0])), hot_hist=bool(g.random() < 0.5) and V > 12)


@pytest.mark.parametrize("seed", list(range(24)))
def test_beam_sweep(seed):
    from test_gpu_beam import _check
    _check(_beam_case(seed), first_step=seed % 5 == 0)


def _verify_select_case(seed):
    from test_gpu_verify_select import _workload
    g = np.random.default_rng(9800 + seed)
    V = int(g.choice([97, 4099, 32000, 151936]))
    dtype = "bf16" if g.random() < 0.6 else "f32"
    k = int(g.choice([1, 3, 8]))
    s = {}
    if g.random() < 0.7:
        s["repetition_penalty"] = float(g.choice([1.3, 0.8, 1.1]))
    if g.random() < 0.4:
        s["no_repeat_ngram_size"] = int(g.choice([2, 3]))
    if g.random() < 0.5:
        s["suppress_tokens"] = [int(v) for v in g.choice(V, size=min(V, 5), replace=False)]
    if g.random() < 0.7:
        s["do_sample"] = True
        s["temperature"] = float(g.choice([1.0, 0.7]))
        s["top_k"] = int(g.choice([0, 0, 5, 64]))
        s["top_p"] = float(g.choice([1.0, 0.9]))
    return _workload(seed + 900, 3, k, V, dtype, s, hist_len=int(g.choice([8, 200])),
                     p_match=float(g.choice([0.5, 0.9])))


@pytest.mark.parametrize("seed", list(range(24)))
def test_verify_select_sweep(seed):
    from test_gpu_verify_select import _check
    _check(_verify_select_case(seed))
