"""Seeded synthetic inputs for the Sparse Gated Attention (SGA) hot path.

This package only draws numbers. It holds none of SGA's arithmetic: no
scoring, selection, softmax or gating happens here. Both the CPU oracle
(through the tests) and the HIP library (through the tests and the bench)
are fed from the same tensors made here.

Every value is a pure function of (seed, tensor name, element index): a
counter-based generator built on the 32-bit MurmurHash3 finaliser, written
with torch integer ops so that the CPU and the GPU produce bit-identical
tensors. That lets the bench build multi-GB caches on the device in
milliseconds while the tests rebuild the very same bytes on the host.
"""

from .gen import (  # noqa: F401
    CONFIG_NAMES,
    EXTRA_NAMES,
    SgaCase,
    block_scaled_rows,
    config_dims,
    make_case,
    make_custom,
    paged_copy,
)
