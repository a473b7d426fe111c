"""Seeded synthetic inputs for paged KV-cache attention.

This package is the only code that both the oracle side and the library side
of the tests (and ``bench.py``) use.  It holds random draws and shapes only:
no slot arithmetic, no gathering, no attention.  Every value is drawn from
``numpy.random.default_rng(seed)`` in a fixed order, so a seed names one input
exactly.
"""

from .synth import (  # noqa: F401
    DecodeCase,
    ExtendCase,
    SharedPrefixCase,
    bf16_words,
    decode_case,
    extend_case,
    gqa4_decode,
    long_context_decode,
    multiturn_extend,
    normal_words,
    shared_prefix_case,
    shared_prefix_decode,
    tiny_fp32_decode,
)
