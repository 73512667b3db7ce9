"""Python front of the CPU oracle (``tsel_oracle.c``).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the CPU
baseline leg of the benchmark import this package; the product path (the HIP
library and its binding) never does.  The oracle shares no code with the HIP
path; the only thing the two sides share is the seeded input generator, which
holds none of the method's arithmetic.

Every function here is marshalling: numpy arrays in, ctypes calls into the C
oracle, numpy arrays out.  The arithmetic lives in ``tsel_oracle.c`` and
follows, step by step, the pages it cites there.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "tsel_oracle.c")
_LIB = os.path.join(_HERE, "libtsel_oracle.so")
MAX_ADMISSIBLE = 64

# Compile flags: one IEEE binary32 rounding per elementwise operation, so no
# contraction into FMA and no fast-math.
CFLAGS = ["-std=c11", "-O2", "-Wall", "-ffp-contract=off", "-fno-fast-math",
          "-fPIC", "-shared"]


def build(force: bool = True) -> str:
    """Compile the oracle into ``libtsel_oracle.so`` with gcc."""
    if force or not os.path.exists(_LIB) or (
            os.path.getmtime(_LIB) < os.path.getmtime(_SRC)):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class _Cfg(C.Structure):
    _fields_ = [
        ("vocab", C.c_int32), ("dtype", C.c_int32),
        ("repetition_penalty", C.c_float), ("no_repeat_ngram_size", C.c_int32),
        ("bad_ids", C.POINTER(C.c_int32)), ("n_bad", C.c_int32),
        ("min_length", C.c_int32), ("min_new_tokens", C.c_int32),
        ("eos_ids", C.POINTER(C.c_int32)), ("n_eos", C.c_int32),
        ("forced_bos", C.c_int32), ("forced_eos", C.c_int32),
        ("suppress_ids", C.POINTER(C.c_int32)), ("n_suppress", C.c_int32),
        ("begin_ids", C.POINTER(C.c_int32)), ("n_begin", C.c_int32),
        ("do_sample", C.c_int32), ("temperature", C.c_float),
        ("top_k", C.c_int32), ("top_p", C.c_float),
        ("renormalize_logits", C.c_int32),
    ]


class _Res(C.Structure):
    _fields_ = [
        ("token", C.c_int32), ("n_finite", C.c_int32),
        ("topk_threshold", C.c_float), ("margin", C.c_double),
        ("greedy_margin", C.c_double), ("n_admissible", C.c_int32),
        ("admissible", C.c_int32 * MAX_ADMISSIBLE),
        ("keep_min", C.c_int32), ("keep_max", C.c_int32),
        ("logprob", C.c_float),
    ]


_lib = None


def bind(path: str):
    """The oracle library at ``path`` with its call signatures declared (the
    pin tests also bind copies of the oracle built with a planted mistake)."""
    lib = C.CDLL(path)
    lib.oracle_select_row.restype = C.c_int
    lib.oracle_select_row.argtypes = [
        C.c_void_p, C.c_void_p, C.c_int32, C.c_int32, C.c_int32,
        C.POINTER(_Cfg), C.c_float, C.c_void_p, C.POINTER(_Res)]
    lib.oracle_verify_row.restype = None
    lib.oracle_verify_row.argtypes = [
        C.c_void_p, C.c_int32, C.c_int32, C.c_int32, C.c_int64, C.c_void_p,
        C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p]
    lib.oracle_verify_select_row.restype = C.c_int
    lib.oracle_verify_select_row.argtypes = [
        C.c_void_p, C.c_int32, C.c_int64, C.c_void_p, C.c_int32, C.c_int32, C.c_int32,
        C.POINTER(_Cfg), C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
        C.c_void_p]
    lib.oracle_beam_step.restype = C.c_int
    lib.oracle_beam_step.argtypes = [
        C.c_void_p, C.c_int64, C.c_int32, C.c_void_p, C.c_int64, C.c_void_p, C.c_void_p,
        C.c_void_p, C.POINTER(_Cfg), C.c_void_p, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p,
        C.c_void_p]
    lib.oracle_finish_row.restype = C.c_int32
    lib.oracle_finish_row.argtypes = [C.c_int32, C.c_int32, C.c_int32, C.c_void_p,
                                      C.c_int32, C.c_void_p]
    lib.oracle_mask_build.restype = None
    lib.oracle_mask_build.argtypes = [C.c_int32, C.c_void_p, C.c_int32,
                                      C.c_void_p]
    return lib


def _load():
    global _lib
    if _lib is None:
        build(force=False)
        _lib = bind(_LIB)
    return _lib


@dataclass
class Config:
    """Generation settings, named as in generation_config.json."""
    repetition_penalty: float = 1.0
    no_repeat_ngram_size: int = 0
    bad_words_ids: Sequence[int] = field(default_factory=list)  # single-token
    min_length: int = 0
    min_new_tokens: int = 0
    eos_token_ids: Sequence[int] = field(default_factory=list)
    forced_bos_token_id: int = -1
    forced_eos_token_id: int = -1
    suppress_tokens: Sequence[int] = field(default_factory=list)
    begin_suppress_tokens: Sequence[int] = field(default_factory=list)
    do_sample: bool = False
    temperature: float = 1.0
    top_k: int = 0
    top_p: float = 1.0
    renormalize_logits: bool = False


def _ids(seq) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(list(seq), dtype=np.int32).reshape(-1))


def _ptr(a: np.ndarray):
    return C.cast(a.ctypes.data, C.POINTER(C.c_int32))


def _dtype_code(logits: np.ndarray) -> int:
    if logits.dtype == np.float32:
        return 0
    if logits.dtype == np.uint16:  # bf16 bit patterns
        return 1
    raise TypeError("logits must be float32 or uint16 (bf16 bits)")


def _c_cfg(cfg: Config, V: int, dcode: int):
    """The C struct of cfg (and the id arrays it points into, which must
    outlive it)."""
    keep = {k: _ids(getattr(cfg, k)) for k in (
        "bad_words_ids", "eos_token_ids", "suppress_tokens", "begin_suppress_tokens")}
    ccfg = _Cfg(
        vocab=V, dtype=dcode, repetition_penalty=cfg.repetition_penalty,
        no_repeat_ngram_size=cfg.no_repeat_ngram_size,
        bad_ids=_ptr(keep["bad_words_ids"]), n_bad=keep["bad_words_ids"].size,
        min_length=cfg.min_length, min_new_tokens=cfg.min_new_tokens,
        eos_ids=_ptr(keep["eos_token_ids"]), n_eos=keep["eos_token_ids"].size,
        forced_bos=cfg.forced_bos_token_id, forced_eos=cfg.forced_eos_token_id,
        suppress_ids=_ptr(keep["suppress_tokens"]),
        n_suppress=keep["suppress_tokens"].size,
        begin_ids=_ptr(keep["begin_suppress_tokens"]),
        n_begin=keep["begin_suppress_tokens"].size,
        do_sample=int(bool(cfg.do_sample)), temperature=cfg.temperature,
        top_k=cfg.top_k, top_p=cfg.top_p,
        renormalize_logits=int(bool(cfg.renormalize_logits)))
    return ccfg, keep


def select(logits: np.ndarray, history: np.ndarray, lens: np.ndarray,
           prompt_lens: np.ndarray, max_lengths: np.ndarray, cfg: Config,
           uniforms: Optional[np.ndarray] = None, rows: Optional[Sequence[int]] = None,
           want_processed: bool = False, threads: int = 1) -> dict:
    """Token selection for the rows ``rows`` (default: all) of a batch.

    logits: [B, V] float32, or uint16 holding bf16 bit patterns.
    history: [B, H] int32, chronological ids; row b uses its first lens[b].
    Returns a dict of numpy arrays indexed like ``rows``: token, n_finite,
    topk_threshold, margin, greedy_margin, admissible (list of arrays),
    keep_min and keep_max (the kept counts top_p allows under the margin
    policy's perturbation), logprob (the token's log-probability, NaN for a
    padding row) and, when asked, processed [len(rows), V] float32.
    """
    lib = _load()
    logits = np.ascontiguousarray(logits)
    history = np.ascontiguousarray(history, dtype=np.int32)
    B, V = logits.shape
    rows = list(range(B)) if rows is None else [int(r) for r in rows]
    dcode = _dtype_code(logits)
    ccfg, keep = _c_cfg(cfg, V, dcode)
    if cfg.do_sample and uniforms is None:
        raise ValueError("sampling needs one uniform per row")
    u = (np.zeros(B, np.float32) if uniforms is None
         else np.ascontiguousarray(uniforms, dtype=np.float32))
    n = len(rows)
    out = {
        "token": np.empty(n, np.int32), "n_finite": np.empty(n, np.int32),
        "topk_threshold": np.empty(n, np.float32), "margin": np.empty(n, np.float64),
        "greedy_margin": np.empty(n, np.float64), "admissible": [None] * n,
        "keep_min": np.empty(n, np.int32), "keep_max": np.empty(n, np.int32),
        "logprob": np.empty(n, np.float32),
    }
    processed = np.empty((n, V), np.float32) if want_processed else None
    esize = logits.itemsize
    base = logits.ctypes.data
    hbase = history.ctypes.data
    hstride = history.shape[1] * 4

    def one(i):
        b = rows[i]
        res = _Res()
        xo = processed[i].ctypes.data if want_processed else None
        rc = lib.oracle_select_row(
            base + b * V * esize, hbase + b * hstride, int(lens[b]),
            int(prompt_lens[b]), int(max_lengths[b]), C.byref(ccfg),
            float(u[b]), xo, C.byref(res))
        if rc != 0:
            raise MemoryError("oracle allocation failed")
        out["token"][i] = res.token
        out["n_finite"][i] = res.n_finite
        out["topk_threshold"][i] = res.topk_threshold
        out["margin"][i] = res.margin
        out["greedy_margin"][i] = res.greedy_margin
        out["admissible"][i] = np.array(res.admissible[:res.n_admissible], np.int32)
        out["keep_min"][i] = res.keep_min
        out["keep_max"][i] = res.keep_max
        out["logprob"][i] = res.logprob

    if threads > 1 and n > 1:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(one, range(n)))
    else:
        for i in range(n):
            one(i)
    if want_processed:
        out["processed"] = processed
    return out


def verify(logits: np.ndarray, candidates: np.ndarray, threads: int = 1) -> dict:
    """Greedy verification of k drafts per row.

    logits: [B, k+1, V] float32 or uint16 (bf16 bits); candidates: [B, k].
    Returns n_match [B], tokens [B, k+1] (-1 after the kept ones), next [B],
    k_next [B].
    """
    lib = _load()
    logits = np.ascontiguousarray(logits)
    candidates = np.ascontiguousarray(candidates, dtype=np.int32)
    B, K1, V = logits.shape
    k = K1 - 1
    dcode = _dtype_code(logits)
    n_match = np.empty(B, np.int32)
    tokens = np.empty((B, K1), np.int32)
    nxt = np.empty(B, np.int32)
    k_next = np.empty(B, np.int32)
    esize = logits.itemsize
    cand2 = candidates.reshape(B, max(k, 0)) if k > 0 else np.zeros((B, 1), np.int32)

    def one(b):
        lib.oracle_verify_row(
            logits.ctypes.data + b * K1 * V * esize, dcode, k, V, V,
            cand2[b].ctypes.data, n_match[b:].ctypes.data, tokens[b].ctypes.data,
            nxt[b:].ctypes.data, k_next[b:].ctypes.data)

    if threads > 1 and B > 1:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(one, range(B)))
    else:
        for b in range(B):
            one(b)
    if (n_match < 0).any():
        raise MemoryError("oracle allocation failed")
    return {"n_match": n_match, "tokens": tokens, "next": nxt, "k_next": k_next}


def mask_build(vocab: int, ids: Sequence[int]) -> np.ndarray:
    """uint32 bitmask of ``ids`` over a vocabulary of ``vocab`` ids."""
    lib = _load()
    a = _ids(ids)
    mask = np.empty((vocab + 31) // 32, np.uint32)
    lib.oracle_mask_build(vocab, a.ctypes.data, a.size, mask.ctypes.data)
    return mask


def finish_step(tokens, lens, max_lengths, eos_ids, finished):
    """The end of one decode step, row by row: (emitted tokens [B] int32,
    finished flags [B] uint8).  tokens: the step's selected tokens (-1 for
    none); lens: the rows' lengths before them; finished: the flags before
    the step (not modified)."""
    lib = _load()
    t = np.ascontiguousarray(tokens, dtype=np.int32)
    L = np.ascontiguousarray(lens, dtype=np.int32)
    M = np.ascontiguousarray(max_lengths, dtype=np.int32)
    e = _ids(eos_ids)
    fin = np.array(finished, dtype=np.uint8, copy=True).reshape(-1)
    out = np.empty(t.shape[0], np.int32)
    for b in range(t.shape[0]):
        out[b] = lib.oracle_finish_row(int(t[b]), int(L[b]), int(M[b]), e.ctypes.data, e.size,
                                       fin[b:].ctypes.data)
    return out, fin


def verify_select(logits: np.ndarray, candidates: np.ndarray, history: np.ndarray,
                  lens: np.ndarray, prompt_lens: np.ndarray, max_lengths: np.ndarray,
                  cfg: Config, uniforms: Optional[np.ndarray] = None, threads: int = 1) -> dict:
    """Verification of k drafts per row with the full selection at each
    position (the processors over the history extended by the drafts before
    it, and for sampling the warpers and a draw from uniforms[b, j]).

    logits: [B, k+1, V] float32 or uint16 (bf16 bits); candidates: [B, k];
    history: [B, H] (row b uses its first lens[b] ids); uniforms: [B, k+1]
    when sampling.  Returns n_match [B], tokens [B, k+1], next [B], k_next [B].
    """
    lib = _load()
    logits = np.ascontiguousarray(logits)
    candidates = np.ascontiguousarray(candidates, dtype=np.int32)
    history = np.ascontiguousarray(history, dtype=np.int32)
    B, K1, V = logits.shape
    k = K1 - 1
    dcode = _dtype_code(logits)
    ccfg, keep = _c_cfg(cfg, V, dcode)
    if cfg.do_sample and uniforms is None:
        raise ValueError("sampling needs one uniform per position")
    u = None if uniforms is None else np.ascontiguousarray(uniforms, dtype=np.float32).reshape(B, K1)
    cand2 = candidates.reshape(B, max(k, 0)) if k > 0 else np.zeros((B, 1), np.int32)
    n_match = np.empty(B, np.int32)
    tokens = np.empty((B, K1), np.int32)
    nxt = np.empty(B, np.int32)
    k_next = np.empty(B, np.int32)
    esize = logits.itemsize

    def one(b):
        rc = lib.oracle_verify_select_row(
            logits.ctypes.data + b * K1 * V * esize, k, V, history[b].ctypes.data,
            int(lens[b]), int(prompt_lens[b]), int(max_lengths[b]), C.byref(ccfg),
            None if u is None else u[b].ctypes.data, cand2[b].ctypes.data,
            n_match[b:].ctypes.data, tokens[b].ctypes.data, nxt[b:].ctypes.data,
            k_next[b:].ctypes.data)
        if rc != 0:
            raise MemoryError("oracle allocation failed")

    if threads > 1 and B > 1:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(one, range(B)))
    else:
        for b in range(B):
            one(b)
    _ = keep
    return {"n_match": n_match, "tokens": tokens, "next": nxt, "k_next": k_next}


def beam_width(num_beams: int, n_eos: int) -> int:
    """Candidates kept per prompt and step: max(2, 1 + eos ids) * num_beams."""
    return max(2, 1 + n_eos) * num_beams


def beam_step(logits: np.ndarray, history: np.ndarray, lens: np.ndarray,
              prompt_lens: np.ndarray, max_lengths: np.ndarray, cfg: Config, num_beams: int,
              beam_scores: np.ndarray, first_step: bool = False, threads: int = 1,
              width: Optional[int] = None) -> dict:
    """One beam-search step for B = rows / num_beams prompts (prompt i owns
    rows i * num_beams .. i * num_beams + num_beams - 1).

    logits: [rows, V] float32 or uint16 (bf16 bits); history: [rows, H];
    lens, prompt_lens, max_lengths, beam_scores: [rows].  Returns scores
    [B, K] float32, beams [B, K] int32 (the beam within its prompt) and
    tokens [B, K] int32, K = max(2, 1 + eos ids) * num_beams (or `width`,
    to see the candidates just past the kept ones)."""
    lib = _load()
    logits = np.ascontiguousarray(logits)
    history = np.ascontiguousarray(history, dtype=np.int32)
    rows, V = logits.shape
    nb = int(num_beams)
    B = rows // nb
    K = beam_width(nb, len(list(cfg.eos_token_ids))) if width is None else int(width)
    ccfg, keep = _c_cfg(cfg, V, _dtype_code(logits))
    L = np.ascontiguousarray(lens, dtype=np.int32)
    P = np.ascontiguousarray(prompt_lens, dtype=np.int32)
    M = np.ascontiguousarray(max_lengths, dtype=np.int32)
    bs = np.ascontiguousarray(beam_scores, dtype=np.float32)
    scores = np.empty((B, K), np.float32)
    beams = np.empty((B, K), np.int32)
    tokens = np.empty((B, K), np.int32)
    esize = logits.itemsize
    H = history.shape[1]

    def one(i):
        r0 = i * nb
        rc = lib.oracle_beam_step(
            logits.ctypes.data + r0 * V * esize, V, nb, history.ctypes.data + r0 * H * 4, H,
            L[r0:].ctypes.data, P[r0:].ctypes.data, M[r0:].ctypes.data, C.byref(ccfg),
            bs[r0:].ctypes.data, int(bool(first_step)), K, scores[i].ctypes.data,
            beams[i].ctypes.data, tokens[i].ctypes.data)
        if rc != 0:
            raise MemoryError("oracle allocation failed")

    if threads > 1 and B > 1:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(one, range(B)))
    else:
        for i in range(B):
            one(i)
    _ = keep
    return {"scores": scores, "beams": beams, "tokens": tokens}
