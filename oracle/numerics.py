"""Exact decoding of stored element bits to fp64 (oracle; test infrastructure only).

Every fp32, fp16 and bf16 value is exactly representable in fp64, so this step
loses nothing.  bf16 is the upper half of an IEEE-754 binary32; it is decoded
by moving the 16 stored bits into the high half of a 32-bit word.
"""

import numpy as np


def to_f64(bits: np.ndarray, dtype: str) -> np.ndarray:
    bits = np.asarray(bits)
    if dtype == "f32":
        return bits.astype(np.uint32).view(np.float32).astype(np.float64)
    if dtype == "f16":
        return bits.astype(np.uint16).view(np.float16).astype(np.float64)
    if dtype == "bf16":
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def elem_bytes(dtype: str) -> int:
    return {"f32": 4, "f16": 2, "bf16": 2}[dtype]
