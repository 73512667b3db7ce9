"""Pins of three oracle parts that the rule cases alone leave loose: the
exact widening of bf16 logits, the decision margin of a sampled row, and its
admissible-id set.

* Widening: "Transmuter.Generation (transmuter v2.0.0)", module doc (the
  selection works on f32 scores; beam paragraph under "Log-probabilities":
  the scores are f32).  A bf16 value is the high half of a binary32, so its
  widening is exact.  The pin feeds bf16 bit patterns (signed zeros,
  subnormals, infinities, the largest finite values, ordinary values) and
  checks the oracle against torch's own bf16 -> float32 conversion: the
  processed row must be those values bit for bit, and the same row given as
  float32 must select the same tokens with bit-identical processed rows
  under the penalty and the temperature.
* Margin: hand-worked from the top_p rule of the same module doc (keep the
  id at position j while the mass before it is below p) and the inverse-CDF
  draw.  Scores x = ln w with integer w make the masses w / sum(w) up to the
  binary32 rounding of ln w (at most 6e-8 relative per score), so the
  expected margins hold to well within 5e-7.
* Admissible set: the ids some perturbation of the cumulative sums by at
  most 1e-6 of the kept mass can select (1e-6 in normalized mass for the
  top_p decisions).  Four equal masses put the draw's target exactly on, or
  a chosen distance from, a bracket edge.

Each pin is then checked to fail on a copy of the oracle with a mistake
planted in the part it pins (built here, on the CPU, from the oracle source
with one textual change).
"""
import os
import shutil
import subprocess

import numpy as np
import pytest
import torch

import oracle

ORACLE_SRC = os.path.join(os.path.dirname(oracle.__file__), "tsel_oracle.c")

# bf16 bit patterns: +0, -0, smallest subnormals, largest subnormals,
# smallest normals, +-1, +-2, ordinary values, largest finite, +-inf.
BF16_PATTERNS = [0x0000, 0x8000, 0x0001, 0x8001, 0x007F, 0x807F, 0x0080, 0x8080,
                 0x3F80, 0xBF80, 0x4000, 0xC000, 0x3FC0, 0xC0A0, 0x4120, 0xBDCD,
                 0x7F7F, 0xFF7F, 0x7F80, 0xFF80]
# finite patterns only (sampling needs finite masses)
BF16_FINITE = [p for p in BF16_PATTERNS if (p & 0x7F80) != 0x7F80]


def _torch_widen(bits):
    t = torch.tensor(np.asarray(bits, np.uint16).view(np.int16)).view(torch.bfloat16)
    return t.float().numpy()


def _one_row(x, cfg, u=0.0, hist=(), L=None, P=None, M=1 << 30, lib=None):
    x = np.asarray(x).reshape(1, -1)
    h = np.asarray(list(hist) or [0], np.int32).reshape(1, -1)
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


# ---------------------------------------------------------------- widening

def check_widening(lib=None):
    bits = np.asarray(BF16_PATTERNS, np.uint16)
    want = _torch_widen(bits)
    # identity processing, greedy: the processed row is the widened row
    r = _one_row(bits, oracle.Config(), hist=[1], lib=lib)
    assert np.array_equal(r["processed"][0].view(np.uint32), want.view(np.uint32)), \
        (r["processed"][0], want)
    # the same row given as bf16 and as float32 under the penalty (greedy),
    # then with temperature and sampling over the finite patterns
    hist = [0, 1, 2, 3, 8, 9, 13, 15, 17]
    for cfg, pats, us in (
            (oracle.Config(repetition_penalty=1.3), BF16_PATTERNS, [0.0]),
            (oracle.Config(repetition_penalty=1.3, do_sample=True, temperature=0.7),
             BF16_FINITE, [0.0, 0.3, 0.71, 0.999]),
            (oracle.Config(repetition_penalty=0.8, do_sample=True, temperature=1.9,
                           top_p=0.9), BF16_FINITE, [0.05, 0.5, 0.95])):
        b = np.asarray(pats, np.uint16)
        f = _torch_widen(b)
        hh = [i for i in hist if i < b.size]
        for u in us:
            rb = _one_row(b, cfg, u=u, hist=hh, lib=lib)
            rf = _one_row(f, cfg, u=u, hist=hh, lib=lib)
            assert rb["token"][0] == rf["token"][0], (cfg, u)
            assert np.array_equal(rb["processed"][0].view(np.uint32),
                                  rf["processed"][0].view(np.uint32)), (cfg, u)


def test_bf16_widening_is_exact():
    check_widening()


# ---------------------------------------------------------------- margin

LN4321 = np.log(np.array([4.0, 3.0, 2.0, 1.0])).astype(np.float32)
MARGIN_CASES = [
    # masses 4:3:2:1, p = 0.75: A = [0, .4, .7, .9], ids 0..2 kept, so
    # m_p = min(.75 - .7, .9 - .75) = .05; W' = 9, u W' = 4.5 in [4, 7):
    # id 1, m_u = .5 / 9; the margin is .05
    dict(p=0.75, u=0.5, token=1, margin=0.05),
    # no top_p: W' = 10, u W' = 3.8 in [0, 4): id 0, m_u = .2 / 10
    dict(p=1.0, u=0.38, token=0, margin=0.02),
    # no top_p: u W' = 9.3 in [9, 10): id 3, m_u = .3 / 10
    dict(p=1.0, u=0.93, token=3, margin=0.03),
    # p = 0.95: A = [0, .4, .7, .9] all below p, all kept, m_p = .95 - .9;
    # u W' = 6.9 in [4, 7): id 1, m_u = .1 / 10; the margin is .01
    dict(p=0.95, u=0.69, token=1, margin=0.01),
]


def check_margin(lib=None):
    for c in MARGIN_CASES:
        r = _one_row(LN4321, oracle.Config(do_sample=True, top_p=c["p"]), u=c["u"],
                     hist=[0], lib=lib)
        assert r["token"][0] == c["token"], c
        assert abs(r["margin"][0] - c["margin"]) <= 5e-7, (c, r["margin"][0])


def test_decision_margin_hand_worked():
    check_margin()


# ---------------------------------------------------------------- admissible

ADMISSIBLE_CASES = [
    # four equal masses, no top_p: u W' = 1.0 sits on the edge of ids 0 and 1
    dict(p=1.0, u=0.25, token=1, ids=[0, 1]),
    # u W' = 1.5: inside id 1's bracket, far from both edges
    dict(p=1.0, u=0.375, token=1, ids=[1]),
    # u W' = 1 + 9.5e-7, within 1e-6 W' = 4e-6 of the edge: both
    dict(p=1.0, u=float(np.float32(0.25) + np.float32(2.0 ** -22)), token=1, ids=[0, 1]),
    # u W' = 1 + 8e-6, twice 1e-6 W' past the edge: id 1 alone
    dict(p=1.0, u=float(np.float32(0.250002)), token=1, ids=[1]),
    # p = 0.5: A_2 = 0.5 = p, so keeping 2 or 3 ids are both admissible:
    # u = 0.7 draws id 1 of 2 (target 1.4) and id 2 of 3 (target 2.1)
    dict(p=0.5, u=0.7, token=1, ids=[1, 2]),
    # p = 0.6: A_2 = 0.5 < 0.6 - 1e-6 and A_3 = 0.75 > p: 3 ids kept for
    # sure; u W' = 2.1 inside id 2's bracket
    dict(p=0.6, u=0.7, token=2, ids=[2]),
]


def check_admissible(lib=None):
    for c in ADMISSIBLE_CASES:
        r = _one_row(np.zeros(4, np.float32), oracle.Config(do_sample=True, top_p=c["p"]),
                     u=c["u"], hist=[0], lib=lib)
        assert r["token"][0] == c["token"], (c, r["token"][0])
        assert sorted(r["admissible"][0].tolist()) == c["ids"], (c, r["admissible"][0])


def test_admissible_set_hand_worked():
    check_admissible()


# ---------------------------------------------------------------- planted mistakes

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
    (check_widening, "<< 16;", "<< 15;"),
    (check_widening, "((const uint16_t *)row)[v]", "((const uint16_t *)row)[v] & 0x7FFF"),
    (check_margin, "*margin_u = mu / Wp;", "*margin_u = mu;"),
    (check_margin, "double a = (double)cfg->top_p - info.a_last;",
     "double a = info.a_next - info.a_last;"),
    (check_margin, "double mu = target - lo < hi - target ? target - lo : hi - target;",
     "double mu = target - lo;"),
    (check_admissible, "const double eps = 1e-6;", "const double eps = 1e-5;"),
    (check_admissible, "const double eps = 1e-6;", "const double eps = 1e-7;"),
    (check_admissible, "if (A - eps < (double)cfg->top_p) may = j + 1;",
     "if (A < (double)cfg->top_p) may = j + 1;"),
    (check_admissible, "int hit = (C > target - tol) && (lo <= target + tol);",
     "int hit = (C > target + tol) && (lo <= target + tol);"),
])
def test_pins_catch_planted_mistakes(tmp_path, check, old, new):
    lib = _mutant(tmp_path, old, new)
    with pytest.raises(AssertionError):
        check(lib)

