"""numpy readers of the cache layouts documented in include/ka_attn.h.

Test code only: turns the raw bytes of a K or V cache buffer into logical
[B][Hkv][C][D] arrays (f32 values, or uint16 bfloat16 bit patterns), written
from the header's index formulas.  Shares nothing with the HIP sources.
"""
import numpy as np


def _elems(raw: np.ndarray, kv_dtype: str) -> np.ndarray:
    raw = np.ascontiguousarray(raw).view(np.uint8)
    return raw.view(np.uint16) if kv_dtype == "bf16" else raw.view(np.float32)


def unpack_k(raw, B, Hkv, C, D, kv_dtype):
    E = 8 if kv_dtype == "bf16" else 4
    a = _elems(raw, kv_dtype)[: B * Hkv * C * D].reshape(B, Hkv, C // 64, D // E, 64, E)
    return a.transpose(0, 1, 2, 4, 3, 5).reshape(B, Hkv, C, D)


def unpack_v(raw, B, Hkv, C, D, kv_dtype):
    a = _elems(raw, kv_dtype)[: B * Hkv * C * D]
    if kv_dtype == "f32":
        a = a.reshape(B, Hkv, C // 4, D, 4)
        return a.transpose(0, 1, 2, 4, 3).reshape(B, Hkv, C, D)
    a = a.reshape(B, Hkv, C // 32, 4, D, 8)
    out = np.empty((B, Hkv, C // 32, 32, D), dtype=a.dtype)
    for r in range(32):
        s = 2 * (r // 16) + (r % 8) // 4
        t = r % 4 + 4 * ((r % 16) // 8)
        out[:, :, :, r, :] = a[:, :, :, s, :, t]
    return out.reshape(B, Hkv, C, D)


def bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def logical_values(raw, B, Hkv, C, D, kv_dtype, which):
    """Cache contents as f32 values in [B][C][Hkv][D] order (position-major)."""
    un = (unpack_k if which == "k" else unpack_v)(raw, B, Hkv, C, D, kv_dtype)
    vals = bits_to_f32(un) if kv_dtype == "bf16" else un
    return np.ascontiguousarray(vals.transpose(0, 2, 1, 3))


def unpack_k_i8(raw, B, Hkv, C, D):
    """int8-K caches: codes [B][Hkv][C][D] (int8) and row scales [B][Hkv][C]
    (f32) from the raw K buffer, by the header's byte index formulas."""
    a = np.ascontiguousarray(raw).view(np.uint8)
    n = B * Hkv * C * D
    codes = a[:n].view(np.int8).reshape(B, Hkv, C // 64, D // 16, 64, 16)
    codes = codes.transpose(0, 1, 2, 4, 3, 5).reshape(B, Hkv, C, D)
    scales = a[n:n + B * Hkv * C * 4].view(np.float32).reshape(B, Hkv, C)
    return codes, scales
