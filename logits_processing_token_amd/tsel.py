"""ctypes binding of libtsel.so (include/tsel.h).

Argument marshalling only: every step of selection and verification runs in
the library's HIP kernels.  Tensors are torch tensors on the GPU; the binding
passes their device pointers and torch's current HIP stream.  A missing or
unloadable library raises immediately: there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Dict, Optional, Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libtsel.so")

TSEL_OK = 0
TSEL_ERR_INVALID_ARG = -1
TSEL_ERR_UNSUPPORTED = -2
TSEL_ERR_LAUNCH = -3
TSEL_ERR_WORKSPACE = -4
TSEL_F32 = 0
TSEL_BF16 = 1
TSEL_INITIAL_K = 5
TSEL_MAX_EOS = 8

# Every entry point include/tsel.h declares.
EXPORTS = (
    "tsel_process_select", "tsel_process_select_workspace_size", "tsel_validate_params",
    "tsel_mask_build", "tsel_verify", "tsel_verify_workspace_size", "tsel_status_string",
    "tsel_finish_step", "tsel_verify_noalloc",
    "tsel_verify_select", "tsel_verify_select_workspace_size", "tsel_beam_step",
    "tsel_beam_width", "tsel_beam_step_workspace_size",
)
TSEL_NOALLOC_SCRATCH_BYTES = 1 << 20


class TselError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)} ({status})")
        self.status = status


class Params(C.Structure):
    """Mirror of struct tsel_params."""
    _fields_ = [
        ("batch", C.c_int32), ("vocab", C.c_int32), ("logits_row_stride", C.c_int64),
        ("dtype", C.c_int32), ("hist_stride", C.c_int32),
        ("repetition_penalty", C.c_float), ("no_repeat_ngram_size", C.c_int32),
        ("bad_words_mask", C.c_void_p), ("suppress_mask", C.c_void_p),
        ("begin_suppress_mask", C.c_void_p),
        ("min_length", C.c_int32), ("min_new_tokens", C.c_int32),
        ("n_eos", C.c_int32), ("eos_ids", C.c_int32 * TSEL_MAX_EOS),
        ("forced_bos_token_id", C.c_int32), ("forced_eos_token_id", C.c_int32),
        ("do_sample", C.c_int32), ("temperature", C.c_float), ("top_k", C.c_int32),
        ("top_p", C.c_float),
        ("renormalize_logits", C.c_int32), ("output_logprobs", C.c_int32),
    ]


_lib = None


def load() -> C.CDLL:
    """Load libtsel.so from the package directory (raises if it is absent)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() or "
                          "python -m logits_processing_token_amd.build")
    lib = C.CDLL(LIB_PATH)
    vp, i32, i64, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
    lib.tsel_process_select.restype = i32
    lib.tsel_process_select.argtypes = [vp, vp, vp, C.POINTER(Params), vp, vp, vp, vp, vp, sz,
                                        vp]
    lib.tsel_process_select_workspace_size.restype = sz
    lib.tsel_process_select_workspace_size.argtypes = [C.POINTER(Params)]
    lib.tsel_validate_params.restype = i32
    lib.tsel_validate_params.argtypes = [C.POINTER(Params), i32]
    lib.tsel_mask_build.restype = i32
    lib.tsel_mask_build.argtypes = [i32, vp, i32, vp, vp]
    lib.tsel_verify.restype = i32
    lib.tsel_verify.argtypes = [vp, i32, i32, i32, i32, i64, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.tsel_verify_noalloc.restype = i32
    lib.tsel_verify_noalloc.argtypes = [vp, i32, i32, i32, i32, i64, vp, vp, vp, vp, vp, vp]
    lib.tsel_verify_select.restype = i32
    lib.tsel_verify_select.argtypes = [vp, vp, vp, C.POINTER(Params), i32, vp, vp, vp, vp, vp,
                                       vp, vp, sz, vp]
    lib.tsel_verify_select_workspace_size.restype = sz
    lib.tsel_verify_select_workspace_size.argtypes = [C.POINTER(Params), i32]
    lib.tsel_beam_step.restype = i32
    lib.tsel_beam_step.argtypes = [vp, vp, vp, C.POINTER(Params), i32, vp, i32, vp, vp, vp, vp,
                                   sz, vp]
    lib.tsel_beam_width.restype = i32
    lib.tsel_beam_width.argtypes = [i32, i32]
    lib.tsel_beam_step_workspace_size.restype = sz
    lib.tsel_beam_step_workspace_size.argtypes = [C.POINTER(Params), i32]
    lib.tsel_verify_workspace_size.restype = sz
    lib.tsel_verify_workspace_size.argtypes = [i32, i32, i32]
    lib.tsel_status_string.restype = C.c_char_p
    lib.tsel_status_string.argtypes = [i32]
    lib.tsel_finish_step.restype = i32
    lib.tsel_finish_step.argtypes = [i32, vp, vp, vp, vp, i32, vp, vp, vp]
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().tsel_status_string(int(status)).decode()


def _check(status: int, what: str):
    if status != TSEL_OK:
        raise TselError(status, what)


def _ptr(t) -> Optional[int]:
    return None if t is None else int(t.data_ptr())


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return int(stream)
    import torch
    return int(torch.cuda.current_stream().cuda_stream)


def make_params(batch: int, vocab: int, row_stride: int, dtype: int, hist_stride: int,
                settings: Dict, masks: Optional[Dict] = None) -> Params:
    """Fill a Params from generation settings named as in
    generation_config.json; masks maps "bad_words_ids" / "suppress_tokens" /
    "begin_suppress_tokens" to device bitmask tensors."""
    masks = masks or {}
    eos = list(settings.get("eos_token_ids", []))
    if len(eos) > TSEL_MAX_EOS:
        raise ValueError("at most %d eos ids" % TSEL_MAX_EOS)
    p = Params()
    p.batch, p.vocab, p.logits_row_stride = batch, vocab, row_stride
    p.dtype, p.hist_stride = dtype, hist_stride
    p.repetition_penalty = settings.get("repetition_penalty", 1.0)
    p.no_repeat_ngram_size = settings.get("no_repeat_ngram_size", 0)
    p.bad_words_mask = _ptr(masks.get("bad_words_ids"))
    p.suppress_mask = _ptr(masks.get("suppress_tokens"))
    p.begin_suppress_mask = _ptr(masks.get("begin_suppress_tokens"))
    p.min_length = settings.get("min_length", 0)
    p.min_new_tokens = settings.get("min_new_tokens", 0)
    p.n_eos = len(eos)
    for i, e in enumerate(eos):
        p.eos_ids[i] = e
    p.forced_bos_token_id = settings.get("forced_bos_token_id", -1)
    p.forced_eos_token_id = settings.get("forced_eos_token_id", -1)
    p.do_sample = int(bool(settings.get("do_sample", False)))
    p.temperature = settings.get("temperature", 1.0)
    p.top_k = settings.get("top_k", 0)
    p.top_p = settings.get("top_p", 1.0)
    p.renormalize_logits = int(bool(settings.get("renormalize_logits", False)))
    p.output_logprobs = int(bool(settings.get("output_logprobs", False)))
    return p


def validate(params: Params, uniforms_given: bool = True) -> int:
    return int(load().tsel_validate_params(C.byref(params), int(uniforms_given)))


def process_select_workspace_size(params: Params) -> int:
    return int(load().tsel_process_select_workspace_size(C.byref(params)))


def process_select(logits, history, lens, params: Params, uniforms=None, out_tokens=None,
                   out_processed=None, out_logprobs=None, workspace=None, stream=None):
    """Run tsel_process_select; returns out_tokens (allocated if None).  When
    params.output_logprobs is set, out_logprobs (float32 [B]) is allocated if
    None and returned as well: (out_tokens, out_logprobs).  The workspace
    (a uint8 device tensor) is allocated when None and the call needs one."""
    import torch
    lib = load()
    if out_tokens is None:
        out_tokens = torch.empty(params.batch, dtype=torch.int32, device=logits.device)
    if params.output_logprobs and out_logprobs is None:
        out_logprobs = torch.empty(params.batch, dtype=torch.float32, device=logits.device)
    need = process_select_workspace_size(params)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=logits.device)
    ws_bytes = 0 if workspace is None else int(workspace.numel() * workspace.element_size())
    st = lib.tsel_process_select(_ptr(logits), _ptr(history), _ptr(lens), C.byref(params),
                                 _ptr(uniforms), _ptr(out_tokens), _ptr(out_processed),
                                 _ptr(out_logprobs), _ptr(workspace), ws_bytes, _stream(stream))
    _check(st, "tsel_process_select")
    if params.output_logprobs:
        return out_tokens, out_logprobs
    return out_tokens


def mask_build(vocab: int, ids, out_mask=None, stream=None):
    """Bitmask of the int32 device tensor ids; returns out_mask."""
    import torch
    lib = load()
    if out_mask is None:
        out_mask = torch.empty((vocab + 31) // 32, dtype=torch.int32, device=ids.device)
    st = lib.tsel_mask_build(vocab, _ptr(ids), int(ids.numel()), _ptr(out_mask), _stream(stream))
    _check(st, "tsel_mask_build")
    return out_mask


def finish_step(tokens, lens, max_lengths, eos_ids, finished, out_tokens=None, stream=None):
    """The end of one decode step on the device: out_tokens (int32 [B]: the
    emitted token or -1) and finished (uint8 [B], updated in place).  eos_ids
    is an int32 device tensor (possibly empty); tokens, lens and max_lengths
    are contiguous int32 device tensors of B rows.  Returns out_tokens."""
    import torch
    B = int(tokens.numel())
    for name, t, dt in (("tokens", tokens, torch.int32), ("lens", lens, torch.int32),
                        ("max_lengths", max_lengths, torch.int32),
                        ("finished", finished, torch.uint8)):
        if t.dtype != dt or t.numel() != B or not t.is_contiguous():
            raise ValueError(f"finish_step: {name} must be a contiguous {dt} tensor of {B} rows")
    if eos_ids.dtype != torch.int32 or not eos_ids.is_contiguous():
        raise ValueError("finish_step: eos_ids must be a contiguous int32 tensor")
    if out_tokens is None:
        out_tokens = torch.empty_like(tokens)
    n_eos = int(eos_ids.numel())
    st = load().tsel_finish_step(B, _ptr(tokens), _ptr(lens), _ptr(max_lengths),
                                 _ptr(eos_ids) if n_eos else None, n_eos, _ptr(finished),
                                 _ptr(out_tokens), _stream(stream))
    _check(st, "tsel_finish_step")
    return out_tokens


def verify_workspace_size(batch: int, k: int, vocab: int) -> int:
    return int(load().tsel_verify_workspace_size(batch, k, vocab))


def verify(logits, candidates, workspace, dtype: int, vocab: Optional[int] = None,
           row_stride: Optional[int] = None, outs: Optional[Sequence] = None, stream=None):
    """Run tsel_verify on logits [B, k+1, stride] holding V = vocab ids per
    position row; returns (n_match, tokens, next, k_next)."""
    import torch
    lib = load()
    B, K1, W = logits.shape
    V = W if vocab is None else vocab
    k = K1 - 1
    dev = logits.device
    if outs is None:
        outs = (torch.empty(B, dtype=torch.int32, device=dev),
                torch.empty((B, K1), dtype=torch.int32, device=dev),
                torch.empty(B, dtype=torch.int32, device=dev),
                torch.empty(B, dtype=torch.int32, device=dev))
    n_match, tokens, nxt, k_next = outs
    stride = W if row_stride is None else row_stride
    st = lib.tsel_verify(_ptr(logits), dtype, B, k, V, stride,
                         _ptr(candidates) if k > 0 else None, _ptr(n_match), _ptr(tokens),
                         _ptr(nxt), _ptr(k_next), _ptr(workspace),
                         int(workspace.numel() * workspace.element_size()), _stream(stream))
    _check(st, "tsel_verify")
    return n_match, tokens, nxt, k_next


def verify_noalloc(logits, candidates, dtype: int, vocab: Optional[int] = None,
                   row_stride: Optional[int] = None, outs: Optional[Sequence] = None,
                   stream=None):
    """Run tsel_verify_noalloc (no workspace: the library's per-device
    scratch array); returns (n_match, tokens, next, k_next)."""
    import torch
    lib = load()
    B, K1, W = logits.shape
    V = W if vocab is None else vocab
    k = K1 - 1
    dev = logits.device
    if outs is None:
        outs = (torch.empty(B, dtype=torch.int32, device=dev),
                torch.empty((B, K1), dtype=torch.int32, device=dev),
                torch.empty(B, dtype=torch.int32, device=dev),
                torch.empty(B, dtype=torch.int32, device=dev))
    n_match, tokens, nxt, k_next = outs
    stride = W if row_stride is None else row_stride
    st = lib.tsel_verify_noalloc(_ptr(logits), dtype, B, k, V, stride,
                                 _ptr(candidates) if k > 0 else None, _ptr(n_match),
                                 _ptr(tokens), _ptr(nxt), _ptr(k_next), _stream(stream))
    _check(st, "tsel_verify_noalloc")
    return n_match, tokens, nxt, k_next


def verify_select(logits, history, lens, params: Params, candidates, uniforms=None,
                  workspace=None, outs: Optional[Sequence] = None, stream=None):
    """Run tsel_verify_select on logits [B, k+1, stride] (params.batch = B,
    params.logits_row_stride = stride); returns (n_match, tokens, next,
    k_next)."""
    import torch
    lib = load()
    B, K1 = logits.shape[0], logits.shape[1]
    k = K1 - 1
    dev = logits.device
    if outs is None:
        outs = (torch.empty(B, dtype=torch.int32, device=dev),
                torch.empty((B, K1), dtype=torch.int32, device=dev),
                torch.empty(B, dtype=torch.int32, device=dev),
                torch.empty(B, dtype=torch.int32, device=dev))
    n_match, tokens, nxt, k_next = outs
    need = int(lib.tsel_verify_select_workspace_size(C.byref(params), k))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    st = lib.tsel_verify_select(_ptr(logits), _ptr(history), _ptr(lens), C.byref(params), k,
                                _ptr(candidates) if k > 0 else None, _ptr(uniforms),
                                _ptr(n_match), _ptr(tokens), _ptr(nxt), _ptr(k_next),
                                _ptr(workspace), int(workspace.numel() * workspace.element_size()),
                                _stream(stream))
    _check(st, "tsel_verify_select")
    return n_match, tokens, nxt, k_next


def beam_width(num_beams: int, n_eos: int) -> int:
    """tsel_beam_width: the candidates a prompt keeps per beam step."""
    return int(load().tsel_beam_width(int(num_beams), int(n_eos)))


def beam_step(logits, history, lens, params: Params, num_beams: int, beam_scores,
              first_step: bool = False, workspace=None, outs: Optional[Sequence] = None,
              stream=None):
    """Run tsel_beam_step over params.batch = prompts * num_beams beam rows;
    returns (scores [P, K] fp32, beams [P, K] int32, tokens [P, K] int32)."""
    import torch
    lib = load()
    dev = logits.device
    P = params.batch // max(int(num_beams), 1)
    K = beam_width(num_beams, params.n_eos)
    if outs is None:
        outs = (torch.empty((P, K), dtype=torch.float32, device=dev),
                torch.empty((P, K), dtype=torch.int32, device=dev),
                torch.empty((P, K), dtype=torch.int32, device=dev))
    scores, beams, tokens = outs
    need = int(lib.tsel_beam_step_workspace_size(C.byref(params), int(num_beams)))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    st = lib.tsel_beam_step(_ptr(logits), _ptr(history), _ptr(lens), C.byref(params),
                            int(num_beams), _ptr(beam_scores), 1 if first_step else 0,
                            _ptr(scores), _ptr(beams), _ptr(tokens), _ptr(workspace),
                            int(workspace.numel() * workspace.element_size()), _stream(stream))
    _check(st, "tsel_beam_step")
    return scores, beams, tokens
