"""Rotary position embedding of rows, as the oracle computes it (test
infrastructure, CPU only: only ``tests/``, the smoke check and the benchmark's
CPU baseline use it; it shares no code with the GPU library).

The Karume pages fix only where the rotary tables come from: the host builds
the cos / sin rows of every chunk from the model's declared rope parameters
and feeds them to the graph (Karume v0.8.0 release notes, "Features", the
conversation-window bullet; karume-gemma4-e2b model card, the context and the
changes-made bullets).  The rotation itself is not on the pages.  Reading
taken: the rotate-half pairing of the transformers Gemma code the model was
exported from.  With h = D / 2 and the row's cos / sin values c[0..h),
s[0..h), dims d and d + h form one pair:

    y[d]     = x[d] c[d] - x[d + h] s[d]
    y[d + h] = x[d + h] c[d] + x[d] s[d]

i.e. the complex number x[d] + i x[d + h] multiplied by c[d] + i s[d].

``rotate_half_f32`` evaluates this in binary32 as two rounded products and
one rounded sum or difference, in that order and without fused multiply-add:
that is the arithmetic the kernels are specified to perform, so the stored
results can be compared bit for bit.  ``rotate_half_f64`` is the same map in
float64 complex arithmetic, an independent statement used to pin the f32 one.
"""
from __future__ import annotations

import numpy as np

__all__ = ["rotate_half_f32", "rotate_half_f64", "angles_table"]


def rotate_half_f32(x, cos, sin) -> np.ndarray:
    """x [..., R, H, D] f32; cos, sin [R][D/2] f32 -> rotated rows, f32."""
    x = np.asarray(x, dtype=np.float32)
    c = np.asarray(cos, dtype=np.float32)[:, None, :]   # [R][1][h]
    s = np.asarray(sin, dtype=np.float32)[:, None, :]
    h = x.shape[-1] // 2
    a, b = x[..., :h], x[..., h:]
    with np.errstate(invalid="ignore", over="ignore"):
        lo = np.float32(a * c) - np.float32(b * s)
        hi = np.float32(b * c) + np.float32(a * s)
    return np.concatenate([lo, hi], axis=-1).astype(np.float32)


def rotate_half_f64(x, cos, sin) -> np.ndarray:
    """The same rotation as complex multiplication in float64."""
    x = np.asarray(x, dtype=np.float64)
    h = x.shape[-1] // 2
    z = (x[..., :h] + 1j * x[..., h:]) * (np.asarray(cos, np.float64) +
                                          1j * np.asarray(sin, np.float64))[:, None, :]
    return np.concatenate([z.real, z.imag], axis=-1)


def angles_table(positions, head_dim: int, base: float = 10000.0):
    """cos / sin rows for the given positions with the usual geometric
    frequencies base^(-2i/D), i < D/2 (a test input; the pages leave the rope
    parameters to the model's configuration)."""
    p = np.asarray(positions, dtype=np.float64)[:, None]
    inv = base ** (-np.arange(head_dim // 2, dtype=np.float64) * 2.0 / head_dim)
    ang = p * inv[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)
