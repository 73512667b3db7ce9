"""Binding of libtsel_probe.so (include/tsel_probe.h): diagnostics beside the
product library, not part of the decode step.  Argument marshalling only."""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libtsel_probe.so")
EXPORTS = ["tsel_probe_exp2_monotone", "tsel_probe_read"]

_lib = None


def load():
    """The probe library; raises if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run logits_processing_token_amd.build")
        lib = C.CDLL(LIB_PATH)
        vp = C.c_void_p
        lib.tsel_probe_read.restype = C.c_int
        lib.tsel_probe_read.argtypes = [vp, C.c_size_t, C.c_int, vp, vp]
        lib.tsel_probe_exp2_monotone.restype = C.c_int
        lib.tsel_probe_exp2_monotone.argtypes = [C.c_float, C.c_float, vp, vp]
        _lib = lib
    return _lib


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return C.c_void_p(s.cuda_stream)


def read(buf, blocks: int, out, stream=None) -> None:
    """One streaming read of the whole of ``buf`` (a device tensor whose size
    in bytes is a multiple of 16); ``out`` is a device int32 tensor."""
    rc = load().tsel_probe_read(buf.data_ptr(), buf.numel() * buf.element_size(), blocks,
                                out.data_ptr(), _stream(stream))
    if rc != 0:
        raise RuntimeError(f"tsel_probe_read failed: HIP error {rc}")


def exp2_monotone(lo: float, hi: float, stream=None) -> int:
    """Number of binary32 x in [lo, hi] where the device exp2 decreases from x
    to the next float up (synchronises)."""
    import torch
    out = torch.zeros(1, dtype=torch.int64, device="cuda")
    rc = load().tsel_probe_exp2_monotone(lo, hi, out.data_ptr(), _stream(stream))
    if rc != 0:
        raise RuntimeError(f"tsel_probe_exp2_monotone failed: HIP error {rc}")
    return int(out.item())
