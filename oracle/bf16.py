"""bfloat16 storage codec of the oracle (test infrastructure, CPU only).

bfloat16 keeps the top 16 bits of an IEEE-754 binary32 pattern: sign, the
8-bit exponent and 7 fraction bits.  Encoding an f32 value rounds to nearest,
ties to even, on the 16 dropped bits (the IEEE default rounding direction;
the Karume pages say nothing of the cache's storage rounding).  A NaN stays a
NaN: its top half is kept and the quiet bit (0x0040) is set, so no NaN can
round into an infinity.  Decoding is exact: the 16 bits are shifted back into
the high half of a binary32 word.

Only ``tests/``, the smoke check and the benchmark's CPU baseline use this
module; the GPU library never imports it and it never imports the library.
"""
from __future__ import annotations

import numpy as np

__all__ = ["encode_rne", "decode", "round_trip"]


def encode_rne(x) -> np.ndarray:
    """f32 values -> uint16 bfloat16 bit patterns, round to nearest even."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    is_nan = (u & 0x7FFFFFFF) > 0x7F800000
    # Round half to even on the 16 dropped bits: add 0x7FFF plus the bit that
    # becomes the new least significant bit, then truncate.
    keep_lsb = (u >> 16) & 1
    rounded = (u + 0x7FFF + keep_lsb) >> 16
    quiet_nan = (u >> 16) | 0x0040
    out = np.where(is_nan, quiet_nan, rounded) & 0xFFFF
    return out.astype(np.uint16).reshape(f.shape)


def decode(bits) -> np.ndarray:
    """uint16 bfloat16 bit patterns -> exact f32 values."""
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return (b.astype(np.uint32) << 16).view(np.float32).reshape(b.shape)


def round_trip(x) -> np.ndarray:
    """The f32 value a bfloat16 cache slot holds after storing x."""
    return decode(encode_rne(x))
