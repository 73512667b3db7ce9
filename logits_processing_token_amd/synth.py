"""Seeded synthetic inputs for token selection and draft verification.

This module is shared by the oracle side (tests) and the HIP side (tests,
benchmark, smoke check).  It draws random numbers and lays them out; it holds
none of the selection arithmetic.  Every tensor gets its own numpy PCG64
sub-stream spawned from one seed, so a workload is reproducible bit for bit.

The five named workloads follow the shapes and value distributions the
project's benchmark configurations state (vocabulary sizes of common decoder
models; log-Zipf logits stand in for a language model's peaked next-token
distribution).  No dataset item is used.

Conventions:
* "N(0, s)" draws a normal with standard deviation s.
* bf16 logits are binary32 values rounded to nearest even and stored as their
  uint16 bit patterns (the high half of the binary32).
* A uniform is (r >> 40) * 2**-24 for a 64-bit random r: an exact binary32
  value in [0, 1).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np

LARGE_MAX_LENGTH = 1 << 30  # "max_length far away": no forced eos


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round binary32 values to bf16 (nearest even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def uniforms(rng: np.random.Generator, n: int) -> np.ndarray:
    r = rng.integers(0, 2**64, size=n, dtype=np.uint64)
    return ((r >> np.uint64(40)).astype(np.float64) * 2.0**-24).astype(np.float32)


def _streams(seed: int, n: int) -> List[np.random.Generator]:
    return [np.random.Generator(np.random.PCG64(s))
            for s in np.random.SeedSequence(seed).spawn(n)]


@dataclass
class SelectWorkload:
    """One decode step's token-selection inputs for a batch."""
    name: str
    logits: np.ndarray            # [B, V] float32, or uint16 bf16 bits
    history: np.ndarray           # [B, H] int32, chronological
    lens: np.ndarray              # [B] int32: prompt + new tokens
    prompt_lens: np.ndarray       # [B] int32
    max_lengths: np.ndarray       # [B] int32: prompt_len + max_new_tokens
    settings: Dict                # generation_config names
    uniforms: Optional[np.ndarray]  # [B] float32, sampling only

    @property
    def dtype(self) -> str:
        return "bf16" if self.logits.dtype == np.uint16 else "f32"

    @property
    def batch(self) -> int:
        return self.logits.shape[0]

    @property
    def vocab(self) -> int:
        return self.logits.shape[1]


@dataclass
class VerifyWorkload:
    """Greedy verification inputs: logits of k+1 positions and k drafts."""
    name: str
    logits: np.ndarray            # [B, k+1, V] float32 or uint16 bf16 bits
    candidates: np.ndarray        # [B, k] int32
    settings: Dict = field(default_factory=dict)

    @property
    def dtype(self) -> str:
        return "bf16" if self.logits.dtype == np.uint16 else "f32"


def _plant_repeats(rng: np.random.Generator, hist: np.ndarray, L: int, n: int,
                   V: int, max_copies: int = 8) -> None:
    """Copy the last n-1 ids of each row to a few random earlier places, each
    followed by a random id, so that a no-repeat n-gram rule has n-grams to
    find (uniform ids over a large vocabulary almost never repeat)."""
    m = n - 1
    if m <= 0 or L < 3 * n:
        return
    for b in range(hist.shape[0]):
        tail = hist[b, L - m:L].copy()
        copies = int(rng.integers(0, max_copies + 1))
        for _ in range(copies):
            s = int(rng.integers(0, L - 2 * n))
            hist[b, s:s + m] = tail
            hist[b, s + m] = int(rng.integers(0, V))


def _planted_candidates(rng_pick: np.random.Generator, rng_id: np.random.Generator,
                        x: np.ndarray, k: int, p_match: float, V: int) -> np.ndarray:
    """Drafts for [B, k+1, V] float32 logits x (modified in place): with
    probability p_match position j's draft is planted as the row's unique
    largest logit (its value is raised to the row's largest value + 1);
    otherwise it is a uniform random id."""
    B = x.shape[0]
    cand = rng_id.integers(0, V, size=(B, k)).astype(np.int32)
    hit = rng_pick.random(size=(B, k)) < p_match
    for b in range(B):
        for j in range(k):
            if hit[b, j]:
                x[b, j, cand[b, j]] = x[b, j].max() + 1.0
    return cand


# --------------------------------------------------------------------------
# The five named workloads.

def c1_select(seed: int = 1001) -> SelectWorkload:
    """B=1, V=50272 fp32 logits ~N(0,3); 64 uniform history ids (all prompt);
    repetition_penalty 1.2; greedy."""
    g_x, g_h = _streams(seed, 2)
    B, V, L = 1, 50272, 64
    x = (g_x.standard_normal((B, V), dtype=np.float32) * np.float32(3.0))
    h = g_h.integers(0, V, size=(B, L)).astype(np.int32)
    return SelectWorkload(
        "C1", x, h, np.full(B, L, np.int32), np.full(B, L, np.int32),
        np.full(B, L + 1000, np.int32), dict(repetition_penalty=1.2), None)


def c1_verify(seed: int = 1001) -> VerifyWorkload:
    """[1, 6, 50272] fp32 ~N(0,3), k=5; each draft is the position's argmax
    with probability 0.7."""
    g_x, g_p, g_c = _streams(seed + 100, 3)
    B, k, V = 1, 5, 50272
    x = g_x.standard_normal((B, k + 1, V), dtype=np.float32) * np.float32(3.0)
    cand = _planted_candidates(g_p, g_c, x, k, 0.7, V)
    return VerifyWorkload("C1-verify", x, cand)


def c2_select(seed: int = 1002, batch: int = 64) -> SelectWorkload:
    """B=64, V=32000 bf16 ~N(0,2); history 1024 (prompt 768 + 256 new) with
    planted 3-gram repeats; rep 1.1, no_repeat_ngram 3, min_new_tokens 300
    (eos 2), temperature 0.7, top_k 50, top_p 0.9, sampling."""
    g_x, g_h, g_r, g_u = _streams(seed, 4)
    B, V, L, P = batch, 32000, 1024, 768
    x = bf16_bits(g_x.standard_normal((B, V), dtype=np.float32) * np.float32(2.0))
    h = g_h.integers(0, V, size=(B, L)).astype(np.int32)
    _plant_repeats(g_r, h, L, 3, V)
    settings = dict(repetition_penalty=1.1, no_repeat_ngram_size=3,
                    min_new_tokens=300, eos_token_ids=[2], do_sample=True,
                    temperature=0.7, top_k=50, top_p=0.9)
    return SelectWorkload("C2", x, h, np.full(B, L, np.int32),
                          np.full(B, P, np.int32), np.full(B, P + 1024, np.int32),
                          settings, uniforms(g_u, B))


def c3_select(seed: int = 1003, batch: int = 256) -> SelectWorkload:
    """B=256, V=128256 bf16: logit of the rank-r id (through a random
    permutation per row) = -1.1 ln(r+1) + N(0,1); history 4096 uniform ids;
    100 suppress_tokens, 50 single-token bad words (disjoint); rep 1.05,
    temperature 1.0, top_p 0.95, no top_k, sampling."""
    g_x, g_perm, g_h, g_s, g_u = _streams(seed, 5)
    B, V, L, P = batch, 128256, 4096, 3072
    base = (-1.1 * np.log(np.arange(1, V + 1, dtype=np.float64))).astype(np.float32)
    x = np.empty((B, V), np.float32)
    for b in range(B):
        perm = g_perm.permutation(V)
        row = base + g_x.standard_normal(V, dtype=np.float32)
        x[b, perm] = row
    x = bf16_bits(x)
    h = g_h.integers(0, V, size=(B, L)).astype(np.int32)
    special = g_s.choice(V, size=150, replace=False).astype(np.int32)
    settings = dict(repetition_penalty=1.05, suppress_tokens=special[:100].tolist(),
                    bad_words_ids=special[100:].tolist(), do_sample=True,
                    temperature=1.0, top_p=0.95)
    return SelectWorkload("C3", x, h, np.full(B, L, np.int32),
                          np.full(B, P, np.int32),
                          np.full(B, LARGE_MAX_LENGTH, np.int32),
                          settings, uniforms(g_u, B))


def c4_verify(seed: int = 1004, batch: int = 32) -> VerifyWorkload:
    """Greedy verification, B=32, k=8, V=151936, bf16 logits [32, 9, V]
    ~N(0,3); each draft is the position's argmax with probability 0.8,
    otherwise a uniform id."""
    g_x, g_p, g_c = _streams(seed, 3)
    B, k, V = batch, 8, 151936
    x = g_x.standard_normal((B, k + 1, V), dtype=np.float32) * np.float32(3.0)
    # Round first so that the planted maximum is compared in bf16.
    x = bf16_bits(x).astype(np.uint32) << 16
    x = x.view(np.float32)
    cand = _planted_candidates(g_p, g_c, x, k, 0.8, V)
    return VerifyWorkload("C4", bf16_bits(x), cand)


def c5_select(seed: int = 1005, batch: int = 1024) -> SelectWorkload:
    """B=1024, V=262144 fp32: logit of id r = -1.2 ln(r+1) + N(0, 0.5);
    history 8192 uniform ids with planted 4-gram repeats; forced_eos (id 2)
    active on ~10% of rows (max_length = len + 1); rep 1.1,
    no_repeat_ngram 4, temperature 0.8, top_k 64, top_p 0.95, sampling."""
    g_x, g_h, g_r, g_f, g_u = _streams(seed, 5)
    B, V, L = batch, 262144, 8192
    base = (-1.2 * np.log(np.arange(1, V + 1, dtype=np.float64))).astype(np.float32)
    x = g_x.standard_normal((B, V), dtype=np.float32)
    x *= np.float32(0.5)
    x += base
    h = g_h.integers(0, V, size=(B, L)).astype(np.int32)
    _plant_repeats(g_r, h, L, 4, V)
    max_len = np.full(B, LARGE_MAX_LENGTH, np.int32)
    forced = g_f.choice(B, size=B // 10, replace=False)
    max_len[forced] = L + 1
    settings = dict(repetition_penalty=1.1, no_repeat_ngram_size=4,
                    forced_eos_token_id=2, eos_token_ids=[2], do_sample=True,
                    temperature=0.8, top_k=64, top_p=0.95)
    return SelectWorkload("C5", x, h, np.full(B, L, np.int32),
                          np.full(B, L - 256, np.int32), max_len, settings,
                          uniforms(g_u, B))


@dataclass
class BeamWorkload:
    """One beam-search step: num_beams rows per prompt, prompt p owning rows
    p * num_beams .. (p + 1) * num_beams - 1."""
    name: str
    logits: np.ndarray            # [P * num_beams, V] float32, or uint16 bf16 bits
    history: np.ndarray           # [P * num_beams, H] int32
    lens: np.ndarray
    prompt_lens: np.ndarray
    max_lengths: np.ndarray
    settings: Dict
    num_beams: int
    beam_scores: np.ndarray       # [P * num_beams] float32


def c3_beam(seed: int = 1006, num_beams: int = 4) -> BeamWorkload:
    """The C3 batch read as 64 prompts x 4 beams: the same logits, histories
    and static masks, one eos id (so K = 8 candidates per prompt), and beam
    scores uniform in [-8, 0)."""
    w = c3_select(seed)
    (g_b,) = _streams(seed + 100, 1)
    settings = {k: v for k, v in w.settings.items()
                if k in ("repetition_penalty", "suppress_tokens", "bad_words_ids")}
    settings["eos_token_ids"] = [2]
    bs = (-8.0 * g_b.random(w.batch)).astype(np.float32)
    return BeamWorkload("C3-beam", w.logits, w.history, w.lens, w.prompt_lens, w.max_lengths,
                        settings, num_beams, bs)


@dataclass
class VerifySelectWorkload:
    """Verification with the selection of the step at every position."""
    name: str
    logits: np.ndarray            # [B, k+1, V] float32 or uint16 bf16 bits
    candidates: np.ndarray        # [B, k] int32
    history: np.ndarray           # [B, H] int32
    lens: np.ndarray
    prompt_lens: np.ndarray
    max_lengths: np.ndarray
    settings: Dict
    uniforms: Optional[np.ndarray]  # [B, k+1] float32, sampling only


def c4_verify_select(seed: int = 1007) -> VerifySelectWorkload:
    """The C4 shape ([32, 9, 151936] bf16 ~N(0,3), drafts planted as the
    position's argmax with probability 0.8) sampled at temperature 0.7 with
    top_p 0.9 and repetition penalty 1.1 over 256 uniform history ids."""
    v = c4_verify(seed)
    g_h, g_u = _streams(seed + 100, 2)
    B, K1, V = v.logits.shape
    L = 256
    h = g_h.integers(0, V, size=(B, L)).astype(np.int32)
    settings = dict(repetition_penalty=1.1, do_sample=True, temperature=0.7, top_p=0.9)
    return VerifySelectWorkload("C4-sampled", v.logits, v.candidates, h,
                                np.full(B, L, np.int32), np.full(B, L, np.int32),
                                np.full(B, LARGE_MAX_LENGTH, np.int32), settings,
                                uniforms(g_u, B * K1).reshape(B, K1))


# --------------------------------------------------------------------------
# Small random cases for rule and edge coverage.

def random_select(seed: int, batch: int, vocab: int, hist_len: int,
                  dtype: str = "f32", sigma: float = 2.0,
                  settings: Optional[Dict] = None, id_range: Optional[int] = None,
                  lens: Optional[np.ndarray] = None,
                  prompt_lens: Optional[np.ndarray] = None,
                  max_lengths: Optional[np.ndarray] = None,
                  plant_n: int = 0, quantize: Optional[float] = None) -> SelectWorkload:
    """A small batch with N(0, sigma) logits and uniform history ids drawn
    from [0, id_range) (default: the vocabulary; a smaller range makes
    repeats; a larger one makes out-of-range ids).  quantize rounds the logits
    to multiples of the given step, which makes exact ties."""
    g_x, g_h, g_r, g_u = _streams(seed, 4)
    x = g_x.standard_normal((batch, vocab), dtype=np.float32) * np.float32(sigma)
    if quantize:
        x = (np.round(x / quantize) * quantize).astype(np.float32)
    x = bf16_bits(x) if dtype == "bf16" else x
    rng_ids = vocab if id_range is None else id_range
    H = max(hist_len, 1)
    h = g_h.integers(0, rng_ids, size=(batch, H)).astype(np.int32)
    if plant_n:
        _plant_repeats(g_r, h, hist_len, plant_n, min(rng_ids, vocab))
    L = np.full(batch, hist_len, np.int32) if lens is None else np.asarray(lens, np.int32)
    P = L.copy() if prompt_lens is None else np.asarray(prompt_lens, np.int32)
    M = (np.full(batch, LARGE_MAX_LENGTH, np.int32) if max_lengths is None
         else np.asarray(max_lengths, np.int32))
    s = dict(settings or {})
    u = uniforms(g_u, batch)
    return SelectWorkload("random", x, h, L, P, M, s, u)


def random_verify(seed: int, batch: int, k: int, vocab: int, dtype: str = "f32",
                  p_match: float = 0.8, quantize: Optional[float] = None) -> VerifyWorkload:
    g_x, g_p, g_c = _streams(seed, 3)
    x = g_x.standard_normal((batch, k + 1, vocab), dtype=np.float32) * np.float32(3.0)
    if quantize:
        x = (np.round(x / quantize) * quantize).astype(np.float32)
    if dtype == "bf16":
        x = (bf16_bits(x).astype(np.uint32) << 16).view(np.float32)
    cand = _planted_candidates(g_p, g_c, x, k, p_match, vocab) if k > 0 else \
        np.zeros((batch, 0), np.int32)
    return VerifyWorkload("random-verify", bf16_bits(x) if dtype == "bf16" else x, cand)


WORKLOADS = {"C1": c1_select, "C2": c2_select, "C3": c3_select, "C5": c5_select}
VERIFY_WORKLOADS = {"C1": c1_verify, "C4": c4_verify}
