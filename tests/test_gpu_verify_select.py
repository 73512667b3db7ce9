"""GPU parity of verification with the full token selection at each
position (tsel_verify_select) against the oracle ("Assisted Generation: a
new direction toward low-latency text generation", step 3 with the
selection method of the step, and "Sample with assisted generation").

Greedy positions are exact.  A sampled position whose decision margin is
below 1e-4 may select another admissible id (the margin policy of the
selection tests); a row is compared exactly when every position up to the
oracle's first mismatch is above that margin, and otherwise its kept tokens
must be admissible at each position and consistent with the drafts."""
import os
import sys

import numpy as np
import pytest

import oracle
from logits_processing_token_amd import synth

pytestmark = pytest.mark.gpu

sys.path.insert(0, os.path.dirname(__file__))
from test_gpu_parity import _gpu  # noqa: E402,F401

MARGIN = 1e-4


def _say(*a):
    print(*a, flush=True)


def _workload(seed, B, k, V, dtype, settings, hist_len=48, p_match=0.8, lens=None,
              prompt=None, maxl=None, id_range=None):
    g = np.random.default_rng(seed)
    x = (g.standard_normal((B, k + 1, V)) * 2.0).astype(np.float32)
    hist = g.integers(0, id_range or V, size=(B, hist_len)).astype(np.int32)
    # drafts: often the raw argmax (so that rules like the penalty decide)
    am = x.argmax(axis=2)
    cand = np.where(g.random((B, k)) < p_match, am[:, :k], g.integers(0, V, (B, k))).astype(np.int32)
    L = np.full(B, hist_len, np.int32) if lens is None else np.asarray(lens, np.int32)
    P = L.copy() if prompt is None else np.asarray(prompt, np.int32)
    M = np.full(B, 1 << 30, np.int32) if maxl is None else np.asarray(maxl, np.int32)
    u = synth.uniforms(g, B * (k + 1)).reshape(B, k + 1)
    if dtype == "bf16":
        x = synth.bf16_bits(x)
    return dict(x=x, hist=hist, cand=cand, L=L, P=P, M=M, u=u, s=settings)


def _gpu_run(w):
    import torch
    from logits_processing_token_amd import tsel
    B, K1, V = w["x"].shape
    epc = 8 if w["x"].dtype == np.uint16 else 4
    stride = ((V + epc - 1) // epc) * epc
    host = np.zeros((B, K1, stride), w["x"].dtype)
    host[:, :, :V] = w["x"]
    dev = torch.device("cuda:0")
    logits = torch.from_numpy(host.view(np.int16) if host.dtype == np.uint16 else host).to(dev)
    dt = tsel.TSEL_BF16 if host.dtype == np.uint16 else tsel.TSEL_F32
    masks = {}
    for name in ("bad_words_ids", "suppress_tokens", "begin_suppress_tokens"):
        if w["s"].get(name):
            masks[name] = tsel.mask_build(V, torch.tensor(list(w["s"][name]), dtype=torch.int32,
                                                          device=dev))
    params = tsel.make_params(B, V, stride, dt, w["hist"].shape[1], w["s"], masks)
    lens = torch.from_numpy(np.concatenate([w["L"], w["P"], w["M"]]).astype(np.int32)).to(dev)
    u = torch.from_numpy(w["u"].astype(np.float32).reshape(-1)).to(dev) if w["s"].get("do_sample") else None
    n, t, nx, kk = tsel.verify_select(logits, torch.from_numpy(w["hist"]).to(dev), lens, params,
                                      torch.from_numpy(w["cand"]).to(dev), u)
    torch.cuda.synchronize()
    return {"n_match": n.cpu().numpy(), "tokens": t.cpu().numpy(), "next": nx.cpu().numpy(),
            "k_next": kk.cpu().numpy()}


def _position_margins(w):
    """Each position's oracle selection (token, margin, admissible ids) over
    its extended history: the row's ids then the drafts before it."""
    B, K1, V = w["x"].shape
    k = K1 - 1
    H = w["hist"].shape[1] + k
    hx = np.zeros((B * K1, H), np.int32)
    L2 = np.zeros(B * K1, np.int32)
    for b in range(B):
        for j in range(K1):
            r = b * K1 + j
            Lb = int(w["L"][b])
            hx[r, :Lb] = w["hist"][b, :Lb]
            hx[r, Lb:Lb + j] = w["cand"][b, :j]
            L2[r] = Lb + j if Lb > 0 else 0
    rep = lambda a: np.repeat(np.asarray(a), K1)
    return oracle.select(w["x"].reshape(B * K1, V), hx, L2, rep(w["P"]), rep(w["M"]),
                         oracle.Config(**w["s"]), uniforms=w["u"].reshape(-1), threads=16)


def _check(w):
    B, K1, V = w["x"].shape
    k = K1 - 1
    gpu = _gpu_run(w)
    ora = oracle.verify_select(w["x"], w["cand"], w["hist"], w["L"], w["P"], w["M"],
                               oracle.Config(**w["s"]), uniforms=w["u"], threads=16)
    pos = _position_margins(w)
    sampling = bool(w["s"].get("do_sample"))
    exact = low = low_same = 0
    for b in range(B):
        n_o = int(ora["n_match"][b])
        marg = pos["margin"][b * K1: b * K1 + n_o + 1]
        is_low = sampling and bool((marg < MARGIN).any())
        same = all(np.array_equal(gpu[key][b], ora[key][b])
                   for key in ("n_match", "tokens", "next", "k_next"))
        if not is_low:
            assert same, (b, {key: (gpu[key][b], ora[key][b]) for key in gpu})
            exact += 1
            continue
        low += 1
        low_same += same
        n_g = int(gpu["n_match"][b])
        kept = gpu["tokens"][b]
        # consistent: n_g leading drafts accepted, the kept tokens admissible
        assert np.array_equal(kept[:n_g], w["cand"][b, :n_g])
        assert n_g == k or kept[n_g] != w["cand"][b, n_g]
        assert (kept[n_g + 1:] == -1).all()
        for j in range(n_g + 1):
            r = b * K1 + j
            assert kept[j] == pos["token"][r] or kept[j] in pos["admissible"][r].tolist(), (b, j)
        assert gpu["next"][b] == kept[n_g]
        assert gpu["k_next"][b] == (k + 2 if n_g == k else max(1, k - 1))
    _say(f"  rows {B}: exact {exact}, low-margin {low} (of them equal to the oracle: {low_same})")
    assert low_same == low  # (as the selection tests require of their low-margin rows)


RULES = dict(repetition_penalty=1.5, no_repeat_ngram_size=2, min_new_tokens=3,
             eos_token_ids=[3], suppress_tokens=[13], forced_eos_token_id=7)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("k", [0, 1, 5])
def test_verify_select_greedy_rules(dtype, k):
    B, V = 12, 5000
    L = np.array([48, 48, 0, 46, 48, 47, 48, 48, 30, 48, 48, 48], np.int32)
    P = np.array([48, 46, 0, 46, 45, 47, 48, 48, 30, 44, 48, 48], np.int32)
    M = np.full(B, 1 << 30, np.int32)
    M[4] = 50  # forced eos at position 1
    M[9] = 49  # forced eos at position 0
    w = _workload(900 + k, B, k, V, dtype, RULES, lens=L, prompt=P, maxl=M, id_range=60)
    # on half the rows the first draft repeats the last history id, so the
    # penalty and the n-gram ban (which see the drafts) decide later positions
    if k:
        w["cand"][::2, 0] = w["hist"][::2, -1]
    _check(w)


@pytest.mark.parametrize("dtype,V,s", [
    ("bf16", 32000, dict(do_sample=True, top_k=50, top_p=0.9, temperature=0.7)),
    ("f32", 32000, dict(do_sample=True, top_k=4, temperature=0.5)),
    ("bf16", 50272, dict(do_sample=True, top_p=0.95)),
    ("f32", 20000, dict(do_sample=True, top_p=0.8, temperature=1.3)),
    ("bf16", 5000, dict(do_sample=True, top_p=0.9, renormalize_logits=True)),
])
def test_verify_select_sampling(dtype, V, s):
    w = _workload(1000 + V, 16, 4, V, dtype, dict(RULES, **s), p_match=0.9)
    _check(w)


def test_verify_select_assisted_batch_shape():
    """The B=32, k=8, V=151936 bf16 shape of greedy verification, sampled at
    temperature 0.7 with top_p 0.9 and a repetition penalty."""
    w = _workload(1004, 32, 8, 151936, "bf16",
                  dict(repetition_penalty=1.1, do_sample=True, temperature=0.7, top_p=0.9),
                  hist_len=256, p_match=0.8)
    _check(w)
