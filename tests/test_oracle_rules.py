"""Pins of the CPU oracle against hand-worked cases of the page rules.

The expectations in tests/golden/rules.json were worked out by hand from the
rules the pages state (each case names its page and section); none of them
was produced by running the oracle or the HIP library.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "rules.json")
DOC = json.load(open(GOLDEN))


def _case_inputs(c):
    if "logits_ln" in c:
        x = np.log(np.asarray(c["logits_ln"], np.float64)).astype(np.float32)
    else:
        x = np.asarray(c["logits"], np.float32)
    V = x.size
    h = np.asarray(c["history"], np.int32).reshape(1, -1)
    if h.shape[1] == 0:
        h = np.zeros((1, 1), np.int32)
    L = len(c["history"])
    P = c.get("prompt_len", L)
    M = c.get("max_length", 1 << 30)
    cfg = oracle.Config(**c["settings"])
    u = np.asarray([c.get("uniform", 0.0)], np.float32)
    return x.reshape(1, V), h, np.array([L], np.int32), np.array([P], np.int32), \
        np.array([M], np.int32), cfg, u


def _expected_array(vals):
    return np.asarray([-np.inf if v == "-inf" else v for v in vals], np.float32)


@pytest.mark.parametrize("case", DOC["select"], ids=[c["id"] for c in DOC["select"]])
def test_golden_select(case):
    x, h, L, P, M, cfg, u = _case_inputs(case)
    r = oracle.select(x, h, L, P, M, cfg, uniforms=u, want_processed=True)
    assert r["token"][0] == case["expect_token"], case["cite"]
    if "expect_processed" in case:
        exp = _expected_array(case["expect_processed"])
        got = r["processed"][0]
        # bit equality, so that -0.0 and +0.0 are told apart
        assert np.array_equal(got.view(np.uint32), exp.view(np.uint32)), (got, exp)
    if "expect_finite" in case:
        fin = np.flatnonzero(np.isfinite(r["processed"][0])).tolist()
        assert fin == case["expect_finite"]


@pytest.mark.parametrize("case", DOC["verify"], ids=[c["id"] for c in DOC["verify"]])
def test_golden_verify(case):
    am = case["argmax"]
    k = len(case["candidates"])
    V = 5
    x = np.zeros((1, k + 1, V), np.float32)
    for j, t in enumerate(am):
        x[0, j, t] = 1.0
    cand = np.asarray(case["candidates"], np.int32).reshape(1, k)
    r = oracle.verify(x, cand)
    e = case["expect"]
    assert r["n_match"][0] == e["n_match"]
    assert r["tokens"][0].tolist() == e["tokens"]
    assert r["next"][0] == e["next"]
    assert r["k_next"][0] == e["k_next"]


# ---------------------------------------------------------------------------
# Invariants that need no printed numbers.

def _rand(seed, V=97, L=40, dtype=np.float32):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((1, V)) * 3).astype(np.float32)
    h = rng.integers(0, V, size=(1, L)).astype(np.int32)
    return x, h


def _sel(x, h, cfg, u=0.5, L=None, P=None, M=1 << 30):
    L = h.shape[1] if L is None else L
    P = L if P is None else P
    return oracle.select(x, h, np.array([L]), np.array([P]), np.array([M]), cfg,
                         uniforms=np.array([u], np.float32), want_processed=True)


@pytest.mark.parametrize("seed", range(5))
def test_identities(seed):
    """penalty 1, temperature 1, top_k >= V and top_p 1 leave every score
    bit-unchanged."""
    x, h = _rand(seed)
    for cfg in (oracle.Config(repetition_penalty=1.0),
                oracle.Config(do_sample=True, temperature=1.0),
                oracle.Config(do_sample=True, top_k=x.shape[1]),
                oracle.Config(do_sample=True, top_k=10 * x.shape[1]),
                oracle.Config(do_sample=True, top_p=1.0)):
        r = _sel(x, h, cfg)
        assert np.array_equal(r["processed"][0].view(np.uint32), x[0].view(np.uint32))


@pytest.mark.parametrize("seed", range(5))
def test_penalty_invariants(seed):
    x, h = _rand(seed)
    p = np.float32(1.3)
    r = _sel(x, h, oracle.Config(repetition_penalty=float(p)))
    y = r["processed"][0]
    seen = np.zeros(x.shape[1], bool)
    seen[h[0]] = True
    # unseen ids are bit-unchanged
    assert np.array_equal(y[~seen].view(np.uint32), x[0][~seen].view(np.uint32))
    # sign is kept; |score| shrinks for positive, grows for negative (p > 1)
    xs, ys = x[0][seen], y[seen]
    assert np.all(np.sign(xs) == np.sign(ys))
    assert np.all(ys[xs > 0] < xs[xs > 0])
    assert np.all(ys[xs < 0] < xs[xs < 0])
    # duplicated history ids act once: [7,7,7] == [7]
    h3 = np.array([[7, 7, 7]], np.int32)
    h1 = np.array([[7]], np.int32)
    y3 = _sel(x, h3, oracle.Config(repetition_penalty=2.0))["processed"][0]
    y1 = _sel(x, h1, oracle.Config(repetition_penalty=2.0))["processed"][0]
    assert np.array_equal(y3.view(np.uint32), y1.view(np.uint32))


def test_penalty_matches_gather_scatter():
    """The gather / where / scatter form over every history position (one
    write per position, repeats included) equals the once-per-id rule."""
    torch = pytest.importorskip("torch")
    for seed in range(8):
        x, h = _rand(seed, V=31, L=60)
        p = 1.7
        t = torch.from_numpy(x.copy())
        ids = torch.from_numpy(h.astype(np.int64))
        g = torch.gather(t, 1, ids)
        g = torch.where(g < 0, g * p, g / p)
        t.scatter_(1, ids, g)
        y = _sel(x, h, oracle.Config(repetition_penalty=p))["processed"][0]
        assert np.array_equal(y.view(np.uint32), t.numpy()[0].view(np.uint32))


@pytest.mark.parametrize("seed", range(10))
def test_greedy_matches_torch_argmax(seed):
    """Greedy = torch.argmax on CPU, whose documented tie rule is the first
    maximal index; quantized logits make many exact ties."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(seed)
    x = np.round(rng.standard_normal((1, 257)) * 2).astype(np.float32)
    h = np.zeros((1, 1), np.int32)
    r = _sel(x, h, oracle.Config())
    assert r["token"][0] == int(torch.argmax(torch.from_numpy(x[0])))


@pytest.mark.parametrize("seed", range(10))
def test_top_k_matches_torch_topk(seed):
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(100 + seed)
    V = 211
    x = np.round(rng.standard_normal((1, V)) * 4).astype(np.float32)  # ties
    k = int(rng.integers(1, 40))
    r = _sel(x, np.zeros((1, 1), np.int32), oracle.Config(do_sample=True, top_k=k))
    t = torch.topk(torch.from_numpy(x[0]), k).values[-1].item()
    assert r["topk_threshold"][0] == np.float32(t)
    kept = np.isfinite(r["processed"][0])
    assert np.array_equal(kept, x[0] >= t)
    assert kept.sum() >= k


@pytest.mark.parametrize("seed", range(6))
def test_greedy_unchanged_by_warpers_and_sampling_u0(seed):
    """top_k / top_p always keep the largest score, so the u=0 sample is the
    greedy token."""
    x, h = _rand(seed, V=300)
    g = _sel(x, h, oracle.Config(repetition_penalty=1.2))["token"][0]
    s = _sel(x, h, oracle.Config(repetition_penalty=1.2, do_sample=True, top_k=7,
                                 top_p=0.3), u=0.0)["token"][0]
    assert g == s


def test_forced_row_selects_forced_token_in_both_modes():
    x, h = _rand(3, V=50, L=1)
    for cfg in (oracle.Config(forced_bos_token_id=17),
                oracle.Config(forced_bos_token_id=17, do_sample=True, temperature=0.5,
                              top_k=3, top_p=0.5)):
        assert _sel(x, h, cfg, u=0.99)["token"][0] == 17


def test_padding_row_batch():
    x = np.ones((3, 4), np.float32)
    h = np.zeros((3, 2), np.int32)
    r = oracle.select(x, h, np.array([2, 0, 1]), np.array([2, 0, 1]),
                      np.array([1 << 30] * 3), oracle.Config())
    assert r["token"].tolist() == [0, -1, 0]


def test_mask_build_bits():
    V = 70
    ids = [0, 31, 32, 69, 5, 5, -3, 70, 1000]
    m = oracle.mask_build(V, ids)
    assert m.shape == (3,)
    want = np.zeros(3, np.uint64)
    for i in ids:
        if 0 <= i < V:
            want[i // 32] |= np.uint64(1) << np.uint64(i % 32)
    assert m.astype(np.uint64).tolist() == want.tolist()


@pytest.mark.parametrize("case", DOC["finish"], ids=[c["id"] for c in DOC["finish"]])
def test_golden_finish(case):
    out, fin = oracle.finish_step([case["token"]], [case["len"]], [case["max_length"]],
                                  case["eos"], [case["finished"]])
    assert out[0] == case["expect"]["token"], case["cite"]
    assert fin[0] == case["expect"]["finished"], case["cite"]


def test_finish_batch_rows_independent():
    """A batch gives each row the result it gets alone (the golden cases
    stacked in one call, the finished flags of the input left untouched)."""
    cs = [c for c in DOC["finish"] if c["eos"] == [2]]
    fin_in = np.array([c["finished"] for c in cs], np.uint8)
    out, fin = oracle.finish_step([c["token"] for c in cs], [c["len"] for c in cs],
                                  [c["max_length"] for c in cs], [2], fin_in)
    assert out.tolist() == [c["expect"]["token"] for c in cs]
    assert fin.tolist() == [c["expect"]["finished"] for c in cs]
    assert fin_in.tolist() == [c["finished"] for c in cs]
