"""Engram conditional-memory forward pass for AMD Instinct MI355X (gfx950).

The compute lives in ``libengram.so`` (hand-written HIP kernels behind the C
ABI of ``include/engram.h``); ``binding`` only marshals torch tensors and the
current HIP stream into those calls.
"""

from .binding import (  # noqa: F401
    BF16,
    CONV_LINEAR,
    CONV_SILU_SKIP,
    F32,
    OUT_DELTA,
    EngramError,
    Plan,
    Weights,
    engram_synth_fill_table,
    lib,
)
