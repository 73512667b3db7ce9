"""GPU parity: the HIP library (through its C ABI) against the CPU oracle on
the same seeded inputs.  Needs an MI355X."""
import json
import os
import sys

import numpy as np
import pytest

from logits_processing_token_amd import synth

pytestmark = pytest.mark.gpu

sys.path.insert(0, os.path.dirname(__file__))
import harness  # noqa: E402
import oracle  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from logits_processing_token_amd import tsel
    tsel.load()  # a missing library fails here, loudly
    yield


def _say(*a):
    print(*a, flush=True)


def _assert_select(w, rows=None, processed=True, max_low_mismatch_frac=0.0,
                   stride_pad=0, logprobs=False):
    _say(f"case {w.name}: B={w.batch} V={w.vocab} {w.dtype} settings={w.settings}")
    gpu = harness.run_gpu_select(w, want_processed=processed, stride_pad=stride_pad,
                                 want_logprobs=logprobs)
    ora = harness.run_oracle_select(w, rows=rows, want_processed=processed)
    rep = harness.compare_select(w, gpu, ora, rows=rows, check_processed=processed)
    _say("  report:", {k: (v if not isinstance(v, list) else v[:5]) for k, v in rep.items()})
    assert rep["high_margin_mismatch"] == [], rep
    assert rep["not_admissible"] == [], rep
    assert rep["processed_mismatch"] == [], rep
    assert rep["logprob_mismatch"] == [], rep
    if rep["low_margin"]:
        assert rep["low_margin_mismatch"] <= max_low_mismatch_frac * rep["low_margin"], rep
    return rep


# ---------------------------------------------------------------------------
def test_device_exp2_is_monotone():
    """The full sampling path maps histogram bins of exp2 masses back to
    score intervals; that needs the device exp2 to be monotone.  Checked
    exhaustively over every binary32 input in [-160, 130] by the diagnostics
    library."""
    from logits_processing_token_amd import probe
    assert probe.exp2_monotone(-160.0, -0.0) == 0
    assert probe.exp2_monotone(0.0, 130.0) == 0


def test_mask_build():
    import torch
    from logits_processing_token_amd import tsel
    rng = np.random.default_rng(0)
    for V in (1, 31, 32, 33, 1000, 128256):
        ids = rng.integers(-5, V + 5, size=300).astype(np.int32)
        got = tsel.mask_build(V, torch.from_numpy(ids).cuda()).cpu().numpy().view(np.uint32)
        assert np.array_equal(got, oracle.mask_build(V, ids)), V


GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "rules.json")))


@pytest.mark.parametrize("case", GOLDEN["select"], ids=[c["id"] for c in GOLDEN["select"]])
def test_golden_rules_gpu(case):
    if "logits_ln" in case:
        x = np.log(np.asarray(case["logits_ln"], np.float64)).astype(np.float32)
    else:
        x = np.asarray(case["logits"], np.float32)
    hist = list(case["history"]) or [0]
    L = len(case["history"])
    w = synth.SelectWorkload(
        case["id"], x.reshape(1, -1), np.asarray([hist], np.int32), np.array([L], np.int32),
        np.array([case.get("prompt_len", L)], np.int32),
        np.array([case.get("max_length", 1 << 30)], np.int32), dict(case["settings"]),
        np.array([case.get("uniform", 0.0)], np.float32))
    gpu = harness.run_gpu_select(w, want_processed=True)
    assert gpu["token"][0] == case["expect_token"]
    if "expect_processed" in case:
        exp = np.asarray([-np.inf if v == "-inf" else v for v in case["expect_processed"]],
                         np.float32)
        assert np.array_equal(gpu["processed"][0].view(np.uint32), exp.view(np.uint32))


ALL_RULES = dict(repetition_penalty=1.3, no_repeat_ngram_size=2, min_length=10**6,
                 eos_token_ids=[3, 7], bad_words_ids=[5, 11, 400], suppress_tokens=[13, 21],
                 begin_suppress_tokens=[1, 2])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("V", [97, 4096, 50272])
def test_greedy_all_rules(dtype, V):
    B = 12
    L = np.array([40, 0, 1, 40, 39, 40, 2, 300, 40, 40, 17, 40], np.int32)
    P = np.array([40, 0, 1, 38, 39, 1, 1, 200, 40, 30, 17, 40], np.int32)
    M = np.full(B, 1 << 30, np.int32)
    M[3] = 41  # forced eos (L == M - 1)
    s = dict(ALL_RULES, forced_bos_token_id=9, forced_eos_token_id=7)
    w = synth.random_select(11 + V, B, V, 300, dtype=dtype, settings=s, id_range=min(V, 60),
                            lens=L, prompt_lens=P, max_lengths=M, plant_n=2)
    _assert_select(w)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_greedy_ties_and_out_of_range_ids(dtype):
    w = synth.random_select(5, 8, 3001, 64, dtype=dtype, id_range=5000, quantize=0.5,
                            settings=dict(repetition_penalty=0.7))
    _assert_select(w)


def test_greedy_odd_stride():
    w = synth.random_select(6, 4, 1001, 64, settings=dict(repetition_penalty=1.2))
    _assert_select(w, stride_pad=3)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("topk,topp,T", [(50, 0.9, 0.7), (1, 1.0, 1.0), (7, 0.5, 1.3),
                                          (300, 0.95, 1.0), (4, 1.0, 0.25)])
def test_sampling_top_k(dtype, topk, topp, T):
    s = dict(repetition_penalty=1.1, no_repeat_ngram_size=3, do_sample=True,
             temperature=T, top_k=topk, top_p=topp)
    w = synth.random_select(100 + topk, 24, 32000, 512, dtype=dtype, settings=s,
                            plant_n=3)
    _assert_select(w)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("V,topp,T", [(5000, 0.9, 1.0), (50272, 0.95, 0.8), (128256, 0.5, 1.0),
                                      (77, 1.0, 1.0), (128256, 1.0, 1.5)])
def test_sampling_full(dtype, V, topp, T):
    s = dict(repetition_penalty=1.05, do_sample=True, temperature=T, top_p=topp,
             suppress_tokens=list(range(0, 60, 7)))
    w = synth.random_select(200 + V, 16, V, 256, dtype=dtype, settings=s, sigma=3.0)
    _assert_select(w)


def test_sampling_forced_padding_all_removed():
    B, V = 6, 500
    L = np.array([1, 0, 30, 30, 1, 30], np.int32)
    P = np.array([1, 0, 30, 20, 1, 30], np.int32)
    M = np.array([1 << 30, 1 << 30, 31, 1 << 30, 1 << 30, 1 << 30], np.int32)
    s = dict(do_sample=True, top_k=5, top_p=0.8, temperature=0.9, forced_bos_token_id=4,
             forced_eos_token_id=9, suppress_tokens=[4])
    w = synth.random_select(9, B, V, 30, settings=s, lens=L, prompt_lens=P, max_lengths=M)
    _assert_select(w)
    s2 = dict(do_sample=True, top_p=0.8, suppress_tokens=list(range(V)))
    w2 = synth.random_select(10, 3, V, 30, settings=s2)
    r = _assert_select(w2)
    assert r["exact"] == 3


@pytest.mark.parametrize("topk", [3, 2000])
def test_top_k_with_heavy_ties(topk):
    """Quantized logits: the k-th value is shared by many ids, so the
    candidate buffer overflows and the exact radix path takes over."""
    s = dict(do_sample=True, top_k=topk, top_p=0.9)
    w = synth.random_select(31, 8, 20000, 16, settings=s, quantize=1.0, sigma=1.0)
    _assert_select(w)


RESIDENT_RULES = dict(repetition_penalty=1.3, no_repeat_ngram_size=3, min_new_tokens=5,
                      eos_token_ids=[3, 7], bad_words_ids=[5, 11, 400],
                      suppress_tokens=[13, 21], begin_suppress_tokens=[1, 2],
                      forced_bos_token_id=9, forced_eos_token_id=7, do_sample=True,
                      temperature=1.0, top_k=0)


@pytest.mark.parametrize("dtype,V", [("bf16", 50273), ("bf16", 131072), ("f32", 4099),
                                     ("f32", 65536)])
@pytest.mark.parametrize("topp,id_range", [(0.9, 60), (1.0, 60), (0.95, None)])
def test_resident_path_processors(dtype, V, topp, id_range):
    """Sampling without top_k at temperature 1 takes the kernels that hold the
    row in registers (bf16 up to V = 131072, fp32 up to V = 65536).  Every
    processor is active on some row: penalty, n-gram bans (planted repeats
    of the last two ids), bad words, the eos ban of min_new_tokens, forced bos
    (L = 1) and eos (L = max_length - 1), suppress, begin-suppress at the
    first new token and, after a forced bos on a one-token prompt, at the
    second; a padding row.  The ids the processors touch carry the largest
    logits, so a missed rule changes the draw."""
    B = 12
    L = np.array([40, 0, 1, 40, 39, 40, 2, 300, 40, 40, 17, 40], np.int32)
    P = np.array([40, 0, 1, 38, 39, 1, 1, 200, 40, 30, 17, 40], np.int32)
    M = np.full(B, 1 << 30, np.int32)
    M[3] = 41  # forced eos (L == M - 1)
    s = dict(RESIDENT_RULES, top_p=topp)
    w = synth.random_select(500 + V + int(topp * 100), B, V, 300, dtype="f32", settings=s,
                            id_range=id_range, lens=L, prompt_lens=P, max_lengths=M,
                            plant_n=2, sigma=2.0)
    boost = w.history[:, :8].ravel().tolist() + [1, 2, 3, 5, 7, 9, 11, 13, 21, 400]
    w.logits[:, np.unique(np.asarray(boost)) % V] += np.float32(6.0)
    if dtype == "bf16":
        w.logits = synth.bf16_bits(w.logits)
    _assert_select(w)


@pytest.mark.parametrize("V", [77, 4099, 50273, 131072])
@pytest.mark.parametrize("q,topp", [(0.25, 0.9), (1.0, 0.3), (0.0625, 1.0), (0.5, 0.999)])
def test_resident_tie_groups(V, q, topp):
    """Quantized bf16 logits without top_k at temperature 1 (the resident
    path): top_p boundaries and draws fall inside tie groups, whose members
    are named in id order by counting over the registers.  Seen ids with
    logit 0 keep 0 under the penalty and tie with the unseen zeros; odd V
    leaves a partial last chunk."""
    s = dict(repetition_penalty=1.2, do_sample=True, top_p=topp,
             suppress_tokens=[3, 5, 8], bad_words_ids=[1, V - 1])
    w = synth.random_select(300 + V, 16, V, 400, dtype="bf16", settings=s, sigma=2.0, quantize=q,
                            id_range=min(V, 5000))
    _assert_select(w)


def test_resident_rows_of_one_value():
    """Every logit equal: one tie group holds the whole row; the boundary and
    the draw are ranks in id order."""
    for V, topp in ((40000, 0.3), (1001, 0.77), (131072, 1.0)):
        w = synth.random_select(7, 4, V, 64, dtype="bf16",
                                settings=dict(do_sample=True, top_p=topp, repetition_penalty=1.5))
        w.logits[:] = synth.bf16_bits(np.full((1,), 0.75, np.float32))[0]
        _assert_select(w)


@pytest.mark.parametrize("n_zone", [40, 3000])
def test_value_bins_near_zero(n_zone):
    """bf16 scores of magnitude at most 2^-8 share two histogram bins and are
    listed one by one (40 per row); more than the list holds, with several
    values among them, leave the row to the bisection (3000).  They are the
    rows' largest scores, zeros of both signs among them, and some are seen
    ids (penalized near zero)."""
    V = 50000
    s = dict(repetition_penalty=1.3, do_sample=True, top_p=0.999)
    w = synth.random_select(91 + n_zone, 8, V, 300, dtype="bf16", settings=s, sigma=1.0,
                            id_range=3000)
    g = np.random.default_rng(n_zone)
    x = (g.standard_normal((w.batch, V)).astype(np.float32) - np.float32(6.0))
    for b in range(w.batch):
        idx = g.choice(V, size=n_zone, replace=False)
        vals = g.uniform(-2.0 ** -8, 2.0 ** -8, size=n_zone).astype(np.float32)
        vals[::7] = 0.0
        vals[1::7] = -0.0
        x[b, idx] = vals
        w.history[b, :20] = idx[:20]
    w.logits[:] = synth.bf16_bits(x)
    _assert_select(w)


@pytest.mark.parametrize("n_seen", [40, 64, 65, 250])
@pytest.mark.parametrize("topp", [1.0, 0.5])
def test_value_bins_seen_ids_of_one_score(n_seen, topp):
    """n_seen seen ids share one logit that the penalty moves off the bf16
    grid: they are one bin's individuals, all of one score, and hold most of
    the mass, so the draw (and at top_p 0.5 the boundary too) walks them in
    id order; up to 64 of them are ordered by one wave, more by the block."""
    V = 40000
    w = synth.random_select(500 + n_seen, 16, V, n_seen, dtype="bf16", sigma=1.0,
                            settings=dict(repetition_penalty=1.3, do_sample=True, top_p=topp))
    g = np.random.default_rng(n_seen)
    x = g.standard_normal((w.batch, V)).astype(np.float32) - np.float32(6.0)
    for b in range(w.batch):
        ids = g.choice(V, size=n_seen, replace=False)
        x[b, ids] = 4.0
        w.history[b] = ids
    w.logits[:] = synth.bf16_bits(x)
    _assert_select(w)


def test_value_bins_zeros_of_both_signs():
    """Rows of zeros of both signs: too many near-zero scores to list, all of
    one value, form one tie group across the two near-zero bins."""
    V = 40000
    w = synth.random_select(17, 4, V, 64, dtype="bf16",
                            settings=dict(do_sample=True, top_p=0.6, repetition_penalty=1.5))
    z = np.zeros((w.batch, V), np.float32)
    z[:, 1::3] = -0.0
    w.logits[:] = synth.bf16_bits(z)
    _assert_select(w)


def test_value_bins_crowded_list():
    """A history of 3000 distinct ids below 3000: one chunk index of the
    registers holds more seen ids than one gather per lane reaches; the rest
    are read after the row."""
    V, H = 60000, 3000
    w = synth.random_select(23, 4, V, H, dtype="bf16",
                            settings=dict(repetition_penalty=1.4, do_sample=True, top_p=0.9))
    for b in range(w.batch):
        w.history[b] = np.random.default_rng(b).permutation(H)
    _assert_select(w)


def test_value_bins_past_the_last_bin():
    """The first chunks of every lane far below the row's maximum: the value
    bins, placed from those chunks, end below the maximum, and the bisection
    decides."""
    V = 50000
    w = synth.random_select(29, 4, V, 100, dtype="bf16",
                            settings=dict(do_sample=True, top_p=0.95, repetition_penalty=1.2))
    x = np.random.default_rng(29).standard_normal((w.batch, V)).astype(np.float32)
    x[:, :8192] = -1000.0
    x[:, 9000] = 100.0
    x[:, 9001] = 99.5
    w.logits[:] = synth.bf16_bits(x)
    _assert_select(w)


def test_constant_logits_bisection():
    """Every score equal: the top_p boundary and the sample fall inside one
    histogram bin far larger than the collect buffer (bisection path)."""
    B, V = 4, 40000
    w = synth.random_select(3, B, V, 8, settings=dict(do_sample=True, top_p=0.3))
    w.logits[:] = 0.5
    _assert_select(w)


def test_many_distinct_seen_ids():
    """More distinct history ids than the on-chip list holds: the stream
    applies the penalty itself."""
    B, V, H = 3, 60000, 12000
    g = np.random.default_rng(4)
    w = synth.random_select(12, B, V, H, settings=dict(repetition_penalty=1.4))
    for b in range(B):
        w.history[b] = g.permutation(V)[:H]
    _assert_select(w)
    w.settings = dict(repetition_penalty=1.4, do_sample=True, top_p=0.9)
    _assert_select(w)


@pytest.mark.parametrize("rep", [1.4, 0.8])
def test_many_distinct_seen_ids_streamed_bf16(rep):
    """A bf16 row past the registers (V = 151936: the streamed full path,
    which counts each score into a bin per bf16 value) with more distinct
    history ids than the on-chip list holds: the stream penalizes them
    itself, each penalized score first taking its value count back; with
    removed ids, a temperature and top_p."""
    B, V, H = 3, 151936, 12000
    g = np.random.default_rng(5)
    w = synth.random_select(13, B, V, H, dtype="bf16", sigma=3.0,
                            settings=dict(repetition_penalty=rep, do_sample=True, top_p=0.9,
                                          temperature=0.7, bad_words_ids=[5, 77, 150000],
                                          suppress_tokens=[9]))
    for b in range(B):
        w.history[b] = g.permutation(V)[:H]
    _assert_select(w)


@pytest.mark.parametrize("settings", [
    dict(do_sample=True, top_p=0.9, temperature=0.7, repetition_penalty=1.2),
    dict(do_sample=True, top_k=50, top_p=0.95),
])
def test_largest_bf16_vocabulary_sampling(settings):
    """bf16 rows of 524,288 ids, sampled: the full path's on-chip layout has
    no room left for the value bins, so its histogram pass counts by mass."""
    w = synth.random_select(21, 2, 524288, 300, dtype="bf16", sigma=3.0, settings=settings)
    _assert_select(w)


# ---------------------------------------------------------------------------
# The named workloads.

def test_c1_select():
    _assert_select(synth.c1_select())


def test_c2_select():
    _assert_select(synth.c2_select())


def test_c3_select_all_rows():
    """Every row of the benchmark batch, in the launch configuration the
    benchmark times (full path, row resident in registers)."""
    w = synth.c3_select()
    rep = _assert_select(w, processed=False)
    _say("C3 low-margin rows:", rep["low_margin"], "mismatches:", rep["low_margin_mismatch"])


def test_c3_processed_rows():
    """Processed scores after top_p on a slice of the C3 batch."""
    w = synth.c3_select(batch=16)
    _assert_select(w, processed=True)


def test_c5_select_all_rows():
    """Every row of the B=1024, V=262144 fp32 batch (top_k path), the
    forced-eos rows among them."""
    w = synth.c5_select()
    forced = np.flatnonzero(w.max_lengths == w.lens + 1)
    gpu = harness.run_gpu_select(w)
    assert (gpu["token"][forced] == 2).all()
    rep = _assert_select(w, processed=False)
    _say("C5 forced rows:", forced.size, "low-margin rows:", rep["low_margin"])


@pytest.mark.parametrize("maker", [synth.c1_verify, synth.c4_verify])
def test_verify_named(maker):
    w = maker()
    d = harness.upload_verify(w)
    gpu = harness.run_gpu_verify(w, d)
    ora = oracle.verify(w.logits, w.candidates, threads=8)
    assert harness.compare_verify(gpu, ora) == []
    # a second call on a workspace full of stale bytes: no state carries over
    d["ws"].fill_(0xAB)
    gpu2 = harness.run_gpu_verify(w, d)
    assert harness.compare_verify(gpu2, ora) == []


@pytest.mark.parametrize("V", [8192, 70001])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_verify_all_removed_positions(V, dtype):
    """Position rows whose every logit is -inf select id 0, the lowest id of
    the tied maxima, whether or not V fills the last 16-byte chunk."""
    w = synth.random_verify(77, 6, 3, V, dtype=dtype, p_match=0.9)
    ninf = synth.bf16_bits(np.array([-np.inf], np.float32))[0] if dtype == "bf16" else -np.inf
    w.logits[1, 0, :] = ninf
    w.logits[2, 2, :] = ninf
    w.logits[4, 3, :] = ninf
    w.candidates[1, 0] = 0  # a match on the all -inf position
    gpu = harness.run_gpu_verify(w)
    ora = oracle.verify(w.logits, w.candidates)
    assert ora["tokens"][1, 0] == 0
    assert harness.compare_verify(gpu, ora) == []


@pytest.mark.parametrize("k", [0, 1, 3, 8])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_verify_random(k, dtype):
    w = synth.random_verify(40 + k, 20, k, 70001, dtype=dtype, p_match=0.75, quantize=0.25)
    gpu = harness.run_gpu_verify(w)
    ora = oracle.verify(w.logits, w.candidates)
    assert harness.compare_verify(gpu, ora) == []


# ---------------------------------------------------------------------------
@pytest.mark.parametrize("B,n_eos", [(1, 1), (255, 0), (256, 8), (257, 3), (5000, 256)])
def test_finish_step(B, n_eos):
    """The end of a decode step against the oracle, bit for bit: tokens with
    -1s and stop ids among them, rows already finished, lengths around the
    maximum; several workgroups and a ragged last one; the largest stop set."""
    import torch
    from logits_processing_token_amd import tsel
    _say(f"case finish_step: B={B} n_eos={n_eos}")
    g = np.random.default_rng(B * 7 + n_eos)
    V = 1000
    eos = g.choice(V, size=n_eos, replace=n_eos > V).astype(np.int32)
    tok = g.integers(0, V, size=B).astype(np.int32)
    if n_eos:
        pick = g.random(B) < 0.2
        tok[pick] = eos[g.integers(0, n_eos, size=int(pick.sum()))]
    tok[g.random(B) < 0.1] = -1
    M = g.integers(1, 60, size=B).astype(np.int32)
    L = (M + g.integers(-3, 2, size=B)).astype(np.int32)
    fin = (g.random(B) < 0.3).astype(np.uint8)
    want_t, want_f = oracle.finish_step(tok, L, M, eos, fin)
    dev = torch.device("cuda:0")
    d_tok = torch.from_numpy(tok).to(dev)
    d_fin = torch.from_numpy(fin).to(dev)
    out = tsel.finish_step(d_tok, torch.from_numpy(L).to(dev), torch.from_numpy(M).to(dev),
                           torch.from_numpy(eos).to(dev), d_fin)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), want_t)
    assert np.array_equal(d_fin.cpu().numpy(), want_f)
    # in place: the tokens buffer takes the emitted tokens; a second step
    # from the flags just written
    d_fin2 = d_fin.clone()
    tsel.finish_step(d_tok, torch.from_numpy(L + 1).to(dev), torch.from_numpy(M).to(dev),
                     torch.from_numpy(eos).to(dev), d_fin2, out_tokens=d_tok)
    torch.cuda.synchronize()
    want_t2, want_f2 = oracle.finish_step(tok, L + 1, M, eos, want_f)
    assert np.array_equal(d_tok.cpu().numpy(), want_t2)
    assert np.array_equal(d_fin2.cpu().numpy(), want_f2)
