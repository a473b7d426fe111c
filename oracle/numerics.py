"""Exact widening of stored K/V/Q words to float64 (oracle, test infrastructure).

Storage types:
  * ``"fp32"`` -- IEEE binary32, held by the oracle as ``uint32`` words.
  * ``"bf16"`` -- bfloat16, held as ``uint16`` words (the top half of a
    binary32).

Working on raw words keeps every copy bit-exact, NaN payloads included, so
pool comparisons can be made on the integers themselves.
"""

import numpy as np

STORAGE_WORD = {"fp32": np.uint32, "bf16": np.uint16}
ELEM_BYTES = {"fp32": 4, "bf16": 2}


def nan_word(dtype: str) -> int:
    """A quiet-NaN bit pattern of the storage type (used to poison memory)."""
    return 0x7FC00000 if dtype == "fp32" else 0x7FC0


def to_f64(words: np.ndarray, dtype: str) -> np.ndarray:
    """Widen raw storage words to float64 without rounding.

    bf16 word w is the binary32 whose bits are ``w << 16``; every binary32 is
    exactly representable in binary64.
    """
    if dtype == "fp32":
        return np.ascontiguousarray(words, dtype=np.uint32).view(np.float32).astype(np.float64)
    if dtype == "bf16":
        wide = np.asarray(words, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return wide.view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")
