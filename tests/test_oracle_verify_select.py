"""Pins of the oracle's verification with the full token selection at each
position ("Assisted Generation: a new direction toward low-latency text
generation", "Greedy decoding with assisted generation" step 3 with the
selection method of the step, and "Sample with assisted generation").

Position j of a row was computed after the history and drafts 0..j-1, so its
selection sees that extended history and the length L + j; each position
draws with its own uniform.  The cases are worked out by hand; the greedy
case without processors is also checked against the plain verification.
"""
import numpy as np
import pytest

import oracle


def _run(pos_logits, cand, hist, cfg, P=None, M=1 << 30, u=None):
    x = np.asarray(pos_logits, np.float32)[None]  # [1, k+1, V]
    k = x.shape[1] - 1
    h = np.asarray([hist], np.int32)
    L = len(hist)
    P = L if P is None else P
    uu = None if u is None else np.asarray([u], np.float32)
    return oracle.verify_select(x, np.asarray([cand], np.int32).reshape(1, k), h,
                                np.array([L], np.int32), np.array([P], np.int32),
                                np.array([M], np.int32), cfg, uniforms=uu)


def _expect(r, n, tokens, nxt, kn):
    assert r["n_match"][0] == n
    assert r["tokens"][0].tolist() == tokens
    assert r["next"][0] == nxt
    assert r["k_next"][0] == kn


def test_penalty_sees_the_drafts():
    # position 0 picks 1, the draft; at position 1 the history holds that
    # draft, so its score 5 becomes 5 / 2 = 2.5 and id 2 (4.9) wins: the
    # second draft (1) is rejected: 1 match, kept [1, 2], next 2, k' = 1
    pos = [[0.0, 5.0, 1.0, 1.0], [0.0, 5.0, 4.9, 1.0], [0.0, 0.0, 0.0, 9.0]]
    r = _run(pos, [1, 1], [0], oracle.Config(repetition_penalty=2.0))
    _expect(r, 1, [1, 2, -1], 2, 1)
    # without the penalty both drafts match and the bonus token follows
    r = _run(pos, [1, 1], [0], oracle.Config())
    _expect(r, 2, [1, 1, 3], 3, 4)


def test_min_new_tokens_counts_the_drafts():
    # prompt of 3 ids, no new ones yet, min_new_tokens 2, eos 3: eos is
    # banned at positions 0 and 1 (0 and 1 new tokens) and allowed at 2
    pos = [[0.0, 1.0, 0.0, 9.0]] * 3
    r = _run(pos, [1, 1], [5, 5, 5], oracle.Config(min_new_tokens=2, eos_token_ids=[3]))
    _expect(r, 2, [1, 1, 3], 3, 4)


def test_ngram_ban_uses_the_drafts():
    # history [5, 6], n = 2, draft 0 is 5: at position 1 the history is
    # [5, 6, 5], whose bigram (5, 6) already occurred, so 6 is banned there
    V = 8
    pos = np.zeros((2, V), np.float32)
    pos[0, 5] = 3.0
    pos[1, 6] = 3.0
    pos[1, 2] = 2.0
    r = _run(pos, [5], [5, 6], oracle.Config(no_repeat_ngram_size=2))
    _expect(r, 1, [5, 2], 2, 3)


def test_forced_eos_moves_with_the_position():
    # max_length 5, history of 3: position 1 has length 4 = max_length - 1,
    # where forced_eos (7) is the only choice
    V = 8
    pos = np.zeros((3, V), np.float32)
    pos[:, 1] = 2.0
    r = _run(pos, [1, 1], [0, 0, 0], oracle.Config(forced_eos_token_id=7), M=5)
    _expect(r, 1, [1, 7, -1], 7, 1)


def test_each_position_draws_with_its_uniform():
    # four equal masses and no top_p: u = 0.1 draws id 0, u = 0.6 id 2,
    # u = 0.9 id 3
    pos = np.zeros((3, 4), np.float32)
    r = _run(pos, [0, 2], [0], oracle.Config(do_sample=True), u=[0.1, 0.6, 0.9])
    _expect(r, 2, [0, 2, 3], 3, 4)
    r = _run(pos, [0, 1], [0], oracle.Config(do_sample=True), u=[0.1, 0.6, 0.9])
    _expect(r, 1, [0, 2, -1], 2, 1)


def test_padding_row_stays_padding():
    pos = np.zeros((2, 4), np.float32)
    x = pos[None]
    r = oracle.verify_select(x, np.array([[1]], np.int32), np.zeros((1, 1), np.int32),
                             np.array([0], np.int32), np.array([0], np.int32),
                             np.array([1 << 30], np.int32), oracle.Config())
    _expect(r, 0, [-1, -1], -1, 1)


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_greedy_without_processors_is_plain_verification(seed):
    g = np.random.default_rng(seed)
    B, k, V = 6, 4, 300
    x = np.round(g.standard_normal((B, k + 1, V)) * 2).astype(np.float32)  # ties too
    am = x.argmax(axis=2)
    cand = np.where(g.random((B, k)) < 0.7, am[:, :k], g.integers(0, V, (B, k))).astype(np.int32)
    h = g.integers(0, V, (B, 10)).astype(np.int32)
    L = np.full(B, 10, np.int32)
    r = oracle.verify_select(x, cand, h, L, L, np.full(B, 1 << 30, np.int32), oracle.Config())
    want = oracle.verify(x, cand)
    for key in ("n_match", "tokens", "next", "k_next"):
        assert np.array_equal(r[key], want[key]), key
