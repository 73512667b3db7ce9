"""tsel: MI355X-native batched token selection and greedy draft verification.

The compute lives in ``libtsel.so`` (hand-written HIP for gfx950 behind a
C ABI, declared in ``include/tsel.h``).  ``logits_processing_token_amd.tsel``
is the thin ctypes binding; ``logits_processing_token_amd.synth`` draws the
seeded synthetic inputs.
"""
