"""Exact decoding of stored element bytes to float64 (oracle, test-only).

Storage codes: 0 = IEEE fp32, 1 = bfloat16 (upper half of an fp32),
2 = OCP fp8 e4m3fn.  The verify page only says that K/V may be fp8 with
per-tensor scaling; the variant read here is the one gfx950 implements
natively: sign bit, 4 exponent bits with bias 7, 3 mantissa bits, no
infinities, codes 0x7F / 0xFF are NaN, largest finite value 448, subnormals
m/8 * 2^-6.

Pinned by tests/test_oracle_decode.py against PyTorch's own dtype casts.
"""
import math

import numpy as np


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float64 (exact: shift into an fp32 word)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def _fp8_value(code: int) -> float:
    s = -1.0 if (code >> 7) & 1 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return s * (m / 8.0) * 2.0 ** (-6)
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def fp8_e4m3_table() -> np.ndarray:
    """256-entry code -> float64 table built from the format's definition."""
    return np.array([_fp8_value(c) for c in range(256)], dtype=np.float64)


_FP8_TABLE = fp8_e4m3_table()


def decode_fp8_e4m3(codes: np.ndarray) -> np.ndarray:
    return _FP8_TABLE[np.ascontiguousarray(codes, dtype=np.uint8)]


def decode(arr: np.ndarray, dtype: int) -> np.ndarray:
    if dtype == 0:
        return np.asarray(arr, dtype=np.float32).astype(np.float64)
    if dtype == 1:
        return decode_bf16(arr)
    if dtype == 2:
        return decode_fp8_e4m3(arr)
    raise ValueError(f"unknown storage dtype {dtype}")
