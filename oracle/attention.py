"""CPU reference of grouped-query causal attention against a KV cache.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this module.  It shares no code
with the GPU library and the library never calls it.

What is computed (the "states-form" attention of Karume's generation-context
path, Karume v0.12.0 release notes, "Performance", the tiled-prefill bullet:
rows of a chunk attend to the K / V rows held in the session state; v0.8.0
release notes, "Features", the conversation-window bullet: chunked prefill and
a cache of up to 131072 positions).  For a query row at absolute position p,
query head h and its KV head g(h):

    s_j  = scale * sum_d q[d] * k_g[j, d]          for keys j = 0 .. p
    m    = max_j s_j
    w_j  = exp(s_j - m),  Z = sum_j w_j
    o[d] = sum_j w_j * v_g[j, d] / Z

which is the textbook two-pass softmax over the whole visible row.  Readings
this oracle takes where the pages leave a step open:

* causal alignment: row i of a chunk starting at ``start`` sits at absolute
  position start + i and sees keys 0 .. start + i, itself included;
* decode with context length ``ctx`` is the row at position ctx - 1;
* GQA map: consecutive query heads share a KV head, g(h) = h // (Hq / Hkv);
* no soft-capping, window, bias or sink: plain causal softmax;
* NaN rule (v0.8.0 release notes, "Breaking Changes", the softmax NaN
  bullet): a NaN among the visible scores or values makes the output row NaN
  (the row max propagates NaN), while a row with no visible key gives exactly
  0;
* K / V enter as the values the cache stores (f32 copies, or bfloat16 after
  round-to-nearest-even, see ``oracle.bf16``); q and the scale are f32 values;
  every product, sum and exponential here is float64.

Two implementations are given: a scalar pure-Python one (``math.fsum``,
``math.exp``) for tiny inputs, and a numpy float64 one, vectorised over rows
and heads in blocks of rows so that a 16K x 16K score matrix never exists at
once.  Neither uses an online softmax or a split of the keys.
"""
from __future__ import annotations

import math
from typing import Iterable, Sequence

import numpy as np

from . import bf16 as _bf16

__all__ = ["kv_group", "stored_values", "attend_rows_scalar", "attend_rows",
           "prefill_chunk", "prefill_ragged", "decode", "rel_error"]


def kv_group(h: int, num_q_heads: int, num_kv_heads: int) -> int:
    """KV head serving query head h: consecutive query heads share one."""
    return h // (num_q_heads // num_kv_heads)


def stored_values(x, kv_dtype: str) -> np.ndarray:
    """Values a cache of dtype ``kv_dtype`` holds after appending f32 rows x."""
    x = np.asarray(x, dtype=np.float32)
    if kv_dtype == "f32":
        return x.copy()
    if kv_dtype == "bf16":
        return _bf16.round_trip(x)
    raise ValueError(f"unknown kv dtype {kv_dtype!r}")


def attend_rows_scalar(q, k, v, q_pos: Sequence[int], scale: float):
    """Scalar brute force for one session.

    q: [n][Hq][D], k / v: [P][Hkv][D] (stored values), q_pos: absolute
    positions of the n rows.  Returns a nested list [n][Hq][D] of floats.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, Hq, D = q.shape
    Hkv = k.shape[1]
    sc = float(np.float32(scale))
    out = []
    for i in range(n):
        p = int(q_pos[i])
        row = []
        for h in range(Hq):
            g = kv_group(h, Hq, Hkv)
            qv = [float(t) for t in q[i, h]]
            s = []
            for j in range(p + 1):
                kj = k[j, g]
                s.append(sc * math.fsum(qv[d] * float(kj[d]) for d in range(D)))
            if not s:
                row.append([0.0] * D)
                continue
            if any(math.isnan(t) for t in s):
                row.append([math.nan] * D)
                continue
            m = max(s)
            w = [math.exp(t - m) for t in s]
            Z = math.fsum(w)
            o = []
            for d in range(D):
                o.append(math.fsum(w[j] * float(v[j, g, d]) for j in range(p + 1)) / Z)
            row.append(o)
        out.append(row)
    return out


def attend_rows(q, k, v, q_pos: Sequence[int], scale: float,
                row_block: int = 256) -> np.ndarray:
    """numpy float64 reference for one session.

    q: [n][Hq][D] f32, k / v: [P][Hkv][D] stored values, q_pos: [n] absolute
    positions.  Returns float64 [n][Hq][D].
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    n, Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    sc = float(np.float32(scale))
    out = np.zeros((n, Hq, D), dtype=np.float64)
    if n == 0:
        return out
    with np.errstate(invalid="ignore", divide="ignore"):
        for r0 in range(0, n, row_block):
            _attend_block(q, k, v, q_pos, sc, r0, min(n, r0 + row_block), G, out)
    return out


def _attend_block(q, k, v, q_pos, sc, r0, r1, G, out):
    """Rows r0 .. r1-1 of one session, every KV head; writes into out."""
    D = q.shape[2]
    Hkv = k.shape[1]
    pos = q_pos[r0:r1]
    nk = int(pos.max()) + 1
    if nk <= 0:
        return                      # no row sees a key: out keeps its zeros
    # visible[i, j] is True where key j is at or before row i's position
    visible = np.arange(nk)[None, :] <= pos[:, None]
    for g in range(Hkv):
        qb = q[r0:r1, g * G:(g + 1) * G, :].astype(np.float64)      # [r][G][D]
        kb = k[:nk, g, :].astype(np.float64)                         # [nk][D]
        vb = v[:nk, g, :].astype(np.float64)                         # [nk][D]
        s = sc * (qb.reshape(-1, D) @ kb.T).reshape(r1 - r0, G, nk)  # [r][G][nk]
        s = np.where(visible[:, None, :], s, -np.inf)
        m = np.max(s, axis=2, keepdims=True)                         # NaN propagates
        w = np.exp(s - m)
        w = np.where(visible[:, None, :], w, 0.0)
        Z = w.sum(axis=2, keepdims=True)
        if np.isfinite(vb).all():
            o = (w.reshape(-1, nk) @ vb).reshape(r1 - r0, G, D) / Z
        else:
            # A non-finite V row must reach only the rows that see it, so
            # each row sums over its own visible keys (0 * NaN is NaN).
            o = np.empty((r1 - r0, G, D))
            for i in range(r1 - r0):
                nv = int(pos[i]) + 1
                o[i] = (w[i, :, :nv] @ vb[:nv]) / Z[i]
        # a row with no visible key gives exactly 0
        empty = ~visible.any(axis=1)
        if empty.any():
            o[empty] = 0.0
        out[r0:r1, g * G:(g + 1) * G, :] = o


def prefill_chunk(q, k_store, v_store, start: int, scale: float,
                  row_block: int = 256) -> np.ndarray:
    """Attention of a chunk of rows at positions start .. start+R-1.

    q: [B][R][Hq][D] f32; k_store / v_store: [B][P][Hkv][D] stored values
    with P >= start + R.  Returns float64 [B][R][Hq][D].
    """
    q = np.asarray(q)
    B, R = q.shape[:2]
    pos = np.arange(start, start + R)
    return np.stack([attend_rows(q[b], k_store[b], v_store[b], pos, scale, row_block)
                     for b in range(B)]) if B else np.zeros(q.shape)


def prefill_ragged(q, k_store, v_store, starts: Sequence[int], rows: Sequence[int],
                   scale: float) -> np.ndarray:
    """Sessions at different positions in one call (several conversations,
    each continuing its own cache; Karume v0.8.0 release notes, "Features":
    the multi-turn chat session).  Session b's rows[b] rows sit at positions
    starts[b] .. starts[b] + rows[b] - 1 and attend to its own keys, exactly as
    a chunk of that session alone.

    q: [sum rows][Hq][D] f32, rows packed session by session; k_store /
    v_store: [B][P][Hkv][D] stored values.  Returns float64 [sum rows][Hq][D].
    """
    q = np.asarray(q)
    parts, r0 = [], 0
    for b, (s0, n) in enumerate(zip(starts, rows)):
        n = int(n)
        if n == 0:
            continue
        parts.append(attend_rows(q[r0:r0 + n], k_store[b], v_store[b],
                                 np.arange(int(s0), int(s0) + n), scale))
        r0 += n
    if not parts:
        return np.zeros((0,) + q.shape[1:])
    return np.concatenate(parts, axis=0)


def decode(q, k_store, v_store, ctx_len: Iterable[int], scale: float) -> np.ndarray:
    """One decode step per session: q [B][Hq][D] attends to keys 0 .. ctx-1."""
    q = np.asarray(q)
    ctx = [int(c) for c in ctx_len]
    return np.stack([attend_rows(q[b][None], k_store[b], v_store[b], [ctx[b] - 1], scale)[0]
                     for b in range(q.shape[0])])


def rel_error(got, ref, v_store) -> float:
    """max |got - ref| / max |V|, the error measure the tolerances are set in.

    max |V| is taken over every stored V value of the test case's cache.
    """
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    vmax = float(np.max(np.abs(np.asarray(v_store, dtype=np.float64))))
    if got.size == 0:
        return 0.0
    return float(np.max(np.abs(got - ref))) / vmax
