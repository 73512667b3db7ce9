"""Pins of the oracle's token log-probability and renormalize_logits, worked
out by hand from "Transmuter.Generation (transmuter v2.0.0)":

* "Log-probabilities" and the function doc of generate/5: the log-softmax of
  the scores the step selects from, at the token -- the scores after the
  processors and, when sampling, after temperature, top-k and top-p; NaN
  (the quiet NaN with sign bit 0) for a row without a token.
* Module doc, processor order: renormalize_logits comes after the
  processors of the task and before temperature; it is the log-softmax of
  the row.

Scores x = ln w with integer w make the softmax masses w / sum(w) up to the
binary32 rounding of ln w (at most 6e-8 relative per score), so the
expected log-probabilities hold to 5e-7.  Each pin is then shown to fail on
a copy of the oracle with a mistake planted in the part it pins.
"""
import math
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle

ORACLE_SRC = os.path.join(os.path.dirname(oracle.__file__), "tsel_oracle.c")
LN1234 = np.log(np.array([1.0, 2.0, 3.0, 4.0])).astype(np.float32)
LN4321 = LN1234[::-1].copy()
QNAN_BITS = 0x7FC00000


def _one(x, cfg, u=0.0, L=None, P=None, M=1 << 30, hist=(0,), lib=None):
    x = np.asarray(x, np.float32).reshape(1, -1)
    h = np.asarray(list(hist), np.int32).reshape(1, -1)
    L = len(hist) if L is None else L
    P = L if P is None else P
    saved = oracle._lib
    if lib is not None:
        oracle._lib = lib
    try:
        return oracle.select(x, h, np.array([L], np.int32), np.array([P], np.int32),
                             np.array([M], np.int32), cfg,
                             uniforms=np.array([u], np.float32), want_processed=True)
    finally:
        oracle._lib = saved


LOGPROB_CASES = [
    # greedy over masses 1:2:3:4: token 3, log(4 / 10)
    dict(cfg=dict(), x=LN1234, u=0.0, token=3, lp=math.log(0.4)),
    # masses 4:3:2:1, top_p 0.75 keeps ids 0..2 (mass 9); u W' = 4.5 draws
    # id 1; its log-probability is over the kept scores: log(3 / 9)
    dict(cfg=dict(do_sample=True, top_p=0.75), x=LN4321, u=0.5, token=1, lp=math.log(3 / 9)),
    # top_k 2 keeps ids 3 and 2 (masses 4, 3); u W' = 6.3 in [4, 7): id 2,
    # log(3 / 7)
    dict(cfg=dict(do_sample=True, top_k=2), x=LN1234, u=0.9, token=2, lp=math.log(3 / 7)),
    # temperature 2: the scores become ln(w) / 2, masses sqrt(w); u = 0
    # draws the first id of the order, id 3: log(2 / (1 + sqrt2 + sqrt3 + 2))
    dict(cfg=dict(do_sample=True, temperature=2.0), x=LN1234, u=0.0, token=3,
         lp=math.log(2.0 / (1.0 + math.sqrt(2.0) + math.sqrt(3.0) + 2.0))),
    # top_k 1 over two equal maxima: both kept, each log(1 / 2)
    dict(cfg=dict(do_sample=True, top_k=1), x=np.array([0.5, 2.0, 2.0, -1.0], np.float32),
         u=0.75, token=2, lp=math.log(0.5)),
]


def check_logprob(lib=None):
    for c in LOGPROB_CASES:
        r = _one(c["x"], oracle.Config(**c["cfg"]), u=c["u"], lib=lib)
        assert r["token"][0] == c["token"], c
        assert abs(float(r["logprob"][0]) - c["lp"]) <= 5e-7, (c, r["logprob"][0])


def check_logprob_special_rows(lib=None):
    # a padding row: no token, the quiet NaN with sign bit 0
    r = _one(LN1234, oracle.Config(), L=0, hist=(0,), lib=lib)
    assert r["token"][0] == -1
    assert r["logprob"].view(np.uint32)[0] == QNAN_BITS
    # a forced token: its score 0 is the only finite one, log-probability 0
    r = _one(LN1234, oracle.Config(forced_bos_token_id=1), L=1, hist=(0,), lib=lib)
    assert r["token"][0] == 1 and r["logprob"][0] == 0.0
    # every id removed: id 0 over scores all -inf, whose log-softmax is NaN
    r = _one(LN1234, oracle.Config(suppress_tokens=[0, 1, 2, 3]), lib=lib)
    assert r["token"][0] == 0 and np.isnan(r["logprob"][0])


def test_logprob_hand_worked():
    check_logprob()


def test_logprob_special_rows():
    check_logprob_special_rows()


def _bits(v):
    return np.asarray(v, np.float32).view(np.uint32)


def check_renormalize(lib=None):
    # x = [1, 1, 1, 1]: m = 1, ls = binary32(ln 4); every score is
    # (1 - 1) - ln4 = -ln 4 exactly (one rounding, of ln 4)
    r = _one(np.ones(4, np.float32), oracle.Config(renormalize_logits=True), lib=lib)
    assert np.array_equal(_bits(r["processed"][0]), _bits(np.full(4, -np.float32(math.log(4.0)))))
    # masses 1:2:3:4: the scores become ln(w / 10) (to two binary32 ulps)
    r = _one(LN1234, oracle.Config(renormalize_logits=True), lib=lib)
    want = np.log(np.array([0.1, 0.2, 0.3, 0.4]))
    assert np.all(np.abs(r["processed"][0] - want) <= 2 * np.spacing(np.abs(want).astype(np.float32)))
    assert r["token"][0] == 3
    # renormalize comes before temperature: ln(w / 10) / 2, not
    # ln(sqrt(w) / sum(sqrt(w))) (the other order)
    r = _one(LN1234, oracle.Config(renormalize_logits=True, do_sample=True, temperature=2.0),
             u=0.0, lib=lib)
    assert np.all(np.abs(r["processed"][0] - want / 2) <= 2e-7), r["processed"][0]
    # a removed id stays -inf and the others normalize among themselves:
    # masses 2:3:4 over ids 1..3
    r = _one(LN1234, oracle.Config(renormalize_logits=True, suppress_tokens=[0]), lib=lib)
    p = r["processed"][0]
    assert p[0] == -np.inf
    assert np.all(np.abs(p[1:] - np.log(np.array([2.0, 3.0, 4.0]) / 9.0)) <= 3e-7), p


def test_renormalize_hand_worked():
    check_renormalize()


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
    # the log-probability over the scores before top_p
    (check_logprob, "  res->logprob = token_logprob(x, V, t);\n  if (x_out)",
     "  res->logprob = token_logprob(pre, V, t);\n  if (x_out)"),
    # a dropped shift by the maximum
    (check_logprob, "  return (float)(((double)x[t] - m) - ls);", "  return (float)((double)x[t] - ls);"),
    (check_logprob_special_rows, "    res->logprob = NAN;\n", "    res->logprob = 0.0f;\n"),
    # renormalize after temperature
    (check_renormalize, "  if (cfg->renormalize_logits) renormalize(x, V);\n", ""),
    (check_renormalize, "    if (x[v] > -INFINITY) x[v] = (x[v] - mf) - lsf;",
     "    if (x[v] > -INFINITY) x[v] = x[v] - lsf;"),
])
def test_logprob_pins_catch_planted_mistakes(tmp_path, check, old, new):
    lib = _mutant(tmp_path, old, new)
    with pytest.raises(AssertionError):
        check(lib)
