"""Int8 scores: per-row quantisation of Q and K and attention on the integer
dot product.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this module.  It shares no code
with the GPU library.

What the pages fix (Karume v0.8.0 release notes): the attention's scores
may come from an int8 dot product with 32-bit integer accumulation and a
shared f32 epilogue ("Fixes", the dp4a bullet), and the scale of a
per-token int8 quantisation is amax times the f32 value of 1/127, computed
in f32 ("Fixes", the activation-quantisation scale bullet).  Readings where
they stop:

* symmetric quantisation of each row (one query head's row, one key row of
  a KV head) over its D values: s = f32(amax * f32(1/127)) with amax = max|x|
  (NaN if any value is NaN), code = round-half-even(f32(x / s)) limited to
  -127 .. 127;
* a row whose s is 0 (all zeros) or not finite (a NaN or an infinity in the
  row) gets codes 0 and keeps its s, so every score it takes part in is
  0 * s: 0 for the zero row, NaN for the non-finite one (the softmax NaN
  rule then applies);
* score = scale * s_q * s_k * sum_d code_q[d] * code_k[d]; the softmax, the
  weights and the values are as in ``oracle.attention`` (V is not
  quantised).

Every decision that yields an integer (amax, s, each code) is taken in f32,
as the GPU takes it; the integer dot is exact; the rest is float64.
"""
from __future__ import annotations

from typing import Sequence

import numpy as np

__all__ = ["INV127", "quantize_rows", "dequantize", "attend_rows_i8", "prefill_chunk_i8",
           "decode_i8"]

INV127 = np.float32(1.0) / np.float32(127.0)   # the f32 value of 1/127


def quantize_rows(x):
    """x [..., D] f32 -> (codes int8 [..., D], scale f32 [...])."""
    x = np.asarray(x, dtype=np.float32)
    with np.errstate(invalid="ignore", over="ignore", divide="ignore"):
        ax = np.abs(x)
        amax = ax.max(axis=-1)                                  # exact in f32
        amax = np.where(np.isnan(x).any(axis=-1), np.float32(np.nan), amax).astype(np.float32)
        s = (amax * INV127).astype(np.float32)                  # one f32 rounding
        ok = np.isfinite(s) & (s > 0)
        safe = np.where(ok, s, np.float32(1)).astype(np.float32)
        r = (x / safe[..., None]).astype(np.float32)            # one f32 rounding
        c = np.clip(np.rint(r), -127, 127)                      # rint: half to even
        c = np.where(ok[..., None], c, 0)
    return c.astype(np.int8), s


def dequantize(codes, s):
    """codes * s in float64 (the value a code row stands for)."""
    return np.asarray(codes, dtype=np.float64) * np.asarray(s, dtype=np.float64)[..., None]


def attend_rows_i8(qc, qs, kc, ks, v, q_pos: Sequence[int], scale: float,
                   row_block: int = 256) -> np.ndarray:
    """One session: qc [n][Hq][D] int8 and qs [n][Hq] f32 (query codes and
    scales), kc [P][Hkv][D] int8 and ks [P][Hkv] f32, v [P][Hkv][D] stored
    values; row i at absolute position q_pos[i] sees keys 0 .. q_pos[i].
    Returns float64 [n][Hq][D].

    The integer dot is formed by a float64 matrix product, which is exact
    here: every product and partial sum is an integer of magnitude at most
    D * 127^2 < 2^53."""
    qc = np.asarray(qc)
    kc = np.asarray(kc)
    qs = np.asarray(qs, dtype=np.float64)
    ks = np.asarray(ks, dtype=np.float64)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    n, Hq, D = qc.shape
    Hkv = kc.shape[1]
    G = Hq // Hkv
    sc = float(np.float32(scale))
    out = np.zeros((n, Hq, D))
    with np.errstate(invalid="ignore", over="ignore"):
        for r0 in range(0, n, row_block):
            r1 = min(n, r0 + row_block)
            pos = q_pos[r0:r1]
            nk = int(pos.max()) + 1
            visible = np.arange(nk)[None, :] <= pos[:, None]             # [r][nk]
            for g in range(Hkv):
                qb = qc[r0:r1, g * G:(g + 1) * G].reshape(-1, D).astype(np.float64)
                kb = kc[:nk, g].astype(np.float64)
                dot = (qb @ kb.T).reshape(r1 - r0, G, nk)                # exact integers
                s = sc * dot * qs[r0:r1, g * G:(g + 1) * G, None] * ks[None, None, :nk, g]
                s = np.where(visible[:, None, :], s, -np.inf)
                m = np.max(s, axis=2, keepdims=True)                      # NaN propagates
                w = np.where(visible[:, None, :], np.exp(s - m), 0.0)
                Z = w.sum(axis=2, keepdims=True)
                vb = np.asarray(v[:nk, g], dtype=np.float64)
                if np.isfinite(vb).all():
                    o = (w.reshape(-1, nk) @ vb).reshape(r1 - r0, G, D)
                else:
                    # A non-finite V row reaches only the rows that see it:
                    # each row sums over its own visible keys, since a zero
                    # weight times NaN or infinity is NaN.
                    o = np.empty((r1 - r0, G, D))
                    for i in range(r1 - r0):
                        nv = int(pos[i]) + 1
                        o[i] = w[i, :, :nv] @ vb[:nv]
                out[r0:r1, g * G:(g + 1) * G] = o / Z
    return out


def prefill_chunk_i8(q, k, v_store, start: int, scale: float) -> np.ndarray:
    """A chunk with int8 scores: q [B][R][Hq][D] f32 and k [B][P][Hkv][D] f32
    are quantised here (per row), v_store [B][P][Hkv][D] are the stored V
    values.  Rows at start .. start+R-1.  Returns float64 [B][R][Hq][D]."""
    qc, qs = quantize_rows(q)
    kc, ks = quantize_rows(k)
    R = np.asarray(q).shape[1]
    pos = np.arange(start, start + R)
    return np.stack([attend_rows_i8(qc[b], qs[b], kc[b], ks[b], v_store[b], pos, scale)
                     for b in range(qc.shape[0])])


def decode_i8(q, k, v_store, ctx_len: Sequence[int], scale: float) -> np.ndarray:
    """One decode row per session with int8 scores: q [B][Hq][D] at position
    ctx - 1, k [B][P][Hkv][D] f32 (quantised here), v_store stored values."""
    qc, qs = quantize_rows(q)
    kc, ks = quantize_rows(k)
    return np.stack([attend_rows_i8(qc[b][None], qs[b][None], kc[b], ks[b], v_store[b],
                                    [int(ctx_len[b]) - 1], scale)[0]
                     for b in range(qc.shape[0])])
