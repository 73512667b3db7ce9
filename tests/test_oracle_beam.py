"""Pins of the oracle's beam-search step, worked out by hand from
"Transmuter.Generation (transmuter v2.0.0)", the beam paragraph under
"Log-probabilities": each step takes the log-softmax of the logits, applies
the processors to it and adds the score of the beam; of the num_beams * V
candidates of a prompt it keeps the best max(2, 1 + eos tokens) * num_beams;
removed tokens have the smallest finite value in place of an infinite one,
and a score never goes below it; at the start only the first beam counts.

Scores x = ln w with integer w make the log-softmax ln(w / sum(w)) up to a
few binary32 roundings (5e-7 here).  (Because a candidate's score never goes
below the smallest finite value, removing an id with that value or with
-inf gives the same candidate scores; the pins see the clamp.)  Equal
scores go by flattened index (beam * V + id), the plainest reading of the
paragraph, which names no order among equal scores.  Each pin is shown to
fail on a copy of the oracle with a planted mistake.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle

ORACLE_SRC = os.path.join(os.path.dirname(oracle.__file__), "tsel_oracle.c")
FMAX = np.finfo(np.float32).max
LN1234 = np.log(np.array([1.0, 2.0, 3.0, 4.0])).astype(np.float32)


def _step(rows, beam_scores, cfg, first=False, L=None, P=None, M=None, hist=None, nb=None,
          lib=None):
    x = np.asarray(rows, np.float32)
    n = x.shape[0]
    nb = n if nb is None else nb
    L = np.full(n, 5, np.int32) if L is None else np.asarray(L, np.int32)
    P = L.copy() if P is None else np.asarray(P, np.int32)
    M = np.full(n, 1 << 30, np.int32) if M is None else np.asarray(M, np.int32)
    h = np.zeros((n, 5), np.int32) + 99 if hist is None else np.asarray(hist, np.int32)
    saved = oracle._lib
    if lib is not None:
        oracle._lib = lib
    try:
        return oracle.beam_step(x, h, L, P, M, cfg, nb, np.asarray(beam_scores, np.float32),
                                first_step=first)
    finally:
        oracle._lib = saved


def _close(got, want, tol=5e-7):
    return np.all(np.abs(np.asarray(got, np.float64) - np.asarray(want)) <= tol)


def check_beam_basic(lib=None):
    lw = np.log(np.array([1.0, 2.0, 3.0, 4.0]) / 10.0)
    # two beams, masses 1:2:3:4 and 4:3:2:1, beam scores -1 and -0.5:
    # K = max(2, 1) * 2 = 4; the best are (b1,0), (b1,1), (b0,3), (b1,2)
    r = _step([LN1234, LN1234[::-1]], [-1.0, -0.5], oracle.Config(), lib=lib)
    assert r["beams"][0].tolist() == [1, 1, 0, 1] and r["tokens"][0].tolist() == [0, 1, 3, 2]
    assert _close(r["scores"][0], [lw[3] - 0.5, lw[2] - 0.5, lw[3] - 1.0, lw[1] - 0.5])
    # the first step: only beam 0 counts
    r = _step([LN1234, LN1234[::-1]], [-1.0, -0.5], oracle.Config(), first=True, lib=lib)
    assert r["beams"][0].tolist() == [0, 0, 0, 0] and r["tokens"][0].tolist() == [3, 2, 1, 0]
    # equal candidates go by flattened index: beam 0 before beam 1
    r = _step([LN1234, LN1234], [0.0, 0.0], oracle.Config(), lib=lib)
    assert r["beams"][0].tolist() == [0, 1, 0, 1] and r["tokens"][0].tolist() == [3, 3, 2, 2]


def check_beam_removed(lib=None):
    # a suppressed id takes the smallest finite value, and adding the beam
    # score does not take it below
    r = _step([LN1234, LN1234], [-1.0, -0.5], oracle.Config(suppress_tokens=[3]), first=True,
              lib=lib)
    assert r["tokens"][0].tolist() == [2, 1, 0, 3]
    assert r["scores"][0][3] == -FMAX
    # a dead beam (score -inf) gives candidates at the smallest finite value
    r = _step([LN1234, LN1234[::-1]], [0.0, -np.inf], oracle.Config(), lib=lib)
    assert r["beams"][0].tolist() == [0, 0, 0, 0]
    r2 = _step([LN1234[::-1], LN1234], [-np.inf, 0.0], oracle.Config(), lib=lib)
    assert r2["beams"][0].tolist() == [1, 1, 1, 1]
    # the dead beam's candidates sit at the smallest finite value, level
    # with a live beam's removed id, so they go by flattened index: two ids,
    # beam 0 dead, id 1 suppressed on beam 1
    r3 = _step([LN1234[:2], LN1234[:2]], [-np.inf, 0.0], oracle.Config(suppress_tokens=[1]),
               lib=lib)
    assert r3["beams"][0].tolist() == [1, 0, 0, 1] and r3["tokens"][0].tolist() == [0, 0, 1, 1]
    assert (r3["scores"][0][1:] == -FMAX).all()
    # a forced eos (L = max_length - 1): its log-probability row is -max
    # everywhere but the forced id, 0
    r = _step([LN1234, LN1234], [-2.0, -3.0], oracle.Config(forced_eos_token_id=1),
              L=[5, 5], M=[6, 1 << 30], lib=lib)
    assert r["beams"][0][0] == 0 and r["tokens"][0][0] == 1 and r["scores"][0][0] == -2.0


def check_beam_width_and_penalty(lib=None):
    # two eos ids: K = max(2, 1 + 2) * 2 = 6
    r = _step([LN1234, LN1234], [0.0, -10.0], oracle.Config(eos_token_ids=[1, 2]), lib=lib)
    assert r["tokens"].shape == (1, 6)
    # the penalty acts on the log-probabilities: seen id 3 of beam 0 has
    # ln(0.4) < 0, multiplied by 2
    # (one beam, two eos ids outside the vocabulary: K = 3)
    r = _step([LN1234], [0.0], oracle.Config(repetition_penalty=2.0, eos_token_ids=[8, 9]),
              hist=[[3, 3, 3, 3, 3]], lib=lib)
    lw = np.log(np.array([1.0, 2.0, 3.0, 4.0]) / 10.0)
    assert r["tokens"][0].tolist() == [2, 1, 3]
    assert _close(r["scores"][0], [lw[2], lw[1], 2 * lw[3]])
    # a padding beam row gives no candidates; slots past them are empty
    r = _step([LN1234, LN1234], [0.0, 0.0], oracle.Config(), L=[5, 0], lib=lib)
    assert r["beams"][0].tolist() == [0, 0, 0, 0]
    r = _step([LN1234[:2], LN1234[:2]], [0.0, 0.0], oracle.Config(), first=True, lib=lib)
    assert r["tokens"][0].tolist() == [1, 0, -1, -1] and r["beams"][0][2] == -1


def test_beam_basic():
    check_beam_basic()


def test_beam_removed():
    check_beam_removed()


def test_beam_width_and_penalty():
    check_beam_width_and_penalty()


def test_beam_prompts_are_independent():
    g = np.random.default_rng(3)
    nb, V = 3, 50
    x = (g.standard_normal((4 * nb, V)) * 2).astype(np.float32)
    h = g.integers(0, V, (4 * nb, 6)).astype(np.int32)
    L = np.full(4 * nb, 6, np.int32)
    bs = (-g.random(4 * nb)).astype(np.float32)
    cfg = oracle.Config(repetition_penalty=1.3, suppress_tokens=[4])
    whole = oracle.beam_step(x, h, L, L, np.full(4 * nb, 1 << 30, np.int32), cfg, nb, bs)
    for i in range(4):
        s = slice(i * nb, (i + 1) * nb)
        one = oracle.beam_step(x[s], h[s], L[s], L[s], np.full(nb, 1 << 30, np.int32), cfg, nb, bs[s])
        for key in ("scores", "beams", "tokens"):
            assert np.array_equal(whole[key][i], one[key][0]), key


def _mutant(tmp_path, old, new):
    src = open(ORACLE_SRC).read()
    assert src.count(old) == 1, f"mutation site not unique: {old!r}"
    path = tmp_path / "mut.c"
    path.write_text(src.replace(old, new))
    so = tmp_path / "libmut.so"
    subprocess.check_call(["gcc", *oracle.CFLAGS, "-o", str(so), str(path), "-lm"])
    return oracle.bind(str(so))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
@pytest.mark.parametrize("check,old,new", [
    (check_beam_basic, "    renormalize(x, V);  /* the log-softmax of the logits */\n", ""),
    (check_beam_basic, "    if ((first_step && j > 0) || L[j] == 0) continue;",
     "    if (L[j] == 0) continue;"),
    (check_beam_basic, "  return (x->flat > y->flat) - (x->flat < y->flat);",
     "  return (x->flat < y->flat) - (x->flat > y->flat);"),
    (check_beam_removed, "      if (!(sc >= -FLT_MAX)) sc = -FLT_MAX;  /* never below the smallest finite value */\n", ""),
])
def test_beam_pins_catch_planted_mistakes(tmp_path, check, old, new):
    lib = _mutant(tmp_path, old, new)
    with pytest.raises(AssertionError):
        check(lib)
