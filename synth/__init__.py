"""Seeded synthetic inputs for the five attention workloads.

This module is shared by the CPU oracle, the GPU tests and the benchmark.  It
holds no attention arithmetic and no storage rounding: it only draws f32
values from seeded numpy generators and returns them in the logical layouts

    K, V : float32 [B][P][Hkv][D]   rows for cache positions 0..P-1
    Q    : float32 [B][P_q][Hq][D]  rows for the query positions listed

where B = sessions, P = positions drawn, Hq / Hkv = query / KV heads, D =
head_dim.  Every draw is ``Generator(PCG64(seed)).standard_normal(dtype=f32)``
in a fixed order per session: all K rows, then all V rows, then the Q rows,
then (max-context workload only) the outlier row indices.  Session b > 0 uses
seed ``1000 * workload_id + b``; session 0 uses ``workload_id``.

The workloads follow the problem statement of Karume's states-form attention
for Gemma 4 E2B (chunked prefill of up to 768 rows, decode, contexts up to
131072 positions; Karume v0.8.0 release notes, "Features", the bullet on the
conversation window; v0.12.0 release notes, "Performance", the bullets on
tiled prefill and parallel decode).  The pages never give Gemma's attention
shape; the shapes below (8 query heads sharing 1 KV head, head_dim 256) are
the ones this project benchmarks.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence

import numpy as np

__all__ = ["Workload", "WORKLOADS", "workload", "draw_session", "draw_batch",
           "SessionInputs"]


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: shapes, schedule and value distribution."""
    wid: int                  # 1..5, also the base seed
    name: str
    batch: int                # independent sessions
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    capacity: int             # cache rows per session per KV head (multiple of 64)
    kv_dtype: str             # "f32" or "bf16" storage
    chunks: tuple             # ((start, rows), ...) prefill chunks, in order
    decode_positions: tuple   # positions of the decode steps, in order
    fill_rows: int            # rows appended before the chunks / steps (untimed fill)
    k_scale: float = 1.0      # K drawn as k_scale * N(0,1), multiplied in f32
    outlier_rows: int = 0     # K rows per session multiplied by outlier_scale
    outlier_scale: float = 1.0

    @property
    def scale(self) -> float:
        """Softmax scale 1/sqrt(head_dim) rounded to f32."""
        return float(np.float32(1.0 / math.sqrt(self.head_dim)))

    @property
    def positions(self) -> int:
        """Number of cache positions whose K/V rows are drawn."""
        last = self.fill_rows
        for s, r in self.chunks:
            last = max(last, s + r)
        for p in self.decode_positions:
            last = max(last, p + 1)
        return last

    @property
    def query_positions(self) -> List[int]:
        """Positions that get a Q row: every chunk row, then every decode step."""
        qp: List[int] = []
        for s, r in self.chunks:
            qp.extend(range(s, s + r))
        qp.extend(self.decode_positions)
        return qp


def _mk() -> dict:
    w = {}
    w[1] = Workload(1, "tiny-prefill-f32", 1, 2, 1, 64, 128, "f32",
                    chunks=((0, 128),), decode_positions=(), fill_rows=0)
    # decode at position 4096 against 4096 cached rows: the step appends row
    # 4096 and attends to 4097 keys (its own included).
    w[2] = Workload(2, "decode-4k-f32", 1, 8, 1, 256, 4160, "f32",
                    chunks=(), decode_positions=(4096,), fill_rows=4096)
    w[3] = Workload(3, "chunked-prefill-3k+768-f32", 1, 8, 1, 256, 3840, "f32",
                    chunks=((3072, 768),), decode_positions=(), fill_rows=3072)
    ch = tuple((768 * i, 768) for i in range(21)) + ((16128, 256),)
    w[4] = Workload(4, "session-16k-bf16", 1, 8, 1, 256, 16448, "bf16",
                    chunks=ch, decode_positions=tuple(range(16384, 16448)),
                    fill_rows=0, k_scale=3.0)
    w[5] = Workload(5, "decode-128k-x4-bf16", 4, 8, 1, 256, 131072, "bf16",
                    chunks=(), decode_positions=tuple(range(131040, 131072)),
                    fill_rows=131040, outlier_rows=1311, outlier_scale=8.0)
    return w


WORKLOADS = _mk()


def workload(wid: int) -> Workload:
    return WORKLOADS[wid]


@dataclasses.dataclass
class SessionInputs:
    k: np.ndarray            # float32 [P][Hkv][D]
    v: np.ndarray            # float32 [P][Hkv][D]
    q: np.ndarray            # float32 [len(q_positions)][Hq][D]
    q_positions: np.ndarray  # int64 positions of the q rows
    outlier_idx: Optional[np.ndarray]


def session_seed(wid: int, b: int) -> int:
    return wid if b == 0 else 1000 * wid + b


def draw_session(w: Workload, b: int, positions: Optional[int] = None,
                 q_positions: Optional[Sequence[int]] = None) -> SessionInputs:
    """Draw session b of workload w.

    ``positions`` may shrink the number of K/V rows (for sampled checks of the
    largest workloads the full draw is still used, so this is only for tests
    that want a smaller cache with the same recipe).
    """
    P = w.positions if positions is None else int(positions)
    qp = np.asarray(w.query_positions if q_positions is None else list(q_positions),
                    dtype=np.int64)
    g = np.random.Generator(np.random.PCG64(session_seed(w.wid, b)))
    Hkv, Hq, D = w.num_kv_heads, w.num_q_heads, w.head_dim
    k = g.standard_normal((P, Hkv, D), dtype=np.float32)
    v = g.standard_normal((P, Hkv, D), dtype=np.float32)
    q = g.standard_normal((len(qp), Hq, D), dtype=np.float32)
    if w.k_scale != 1.0:
        k *= np.float32(w.k_scale)
    idx = None
    if w.outlier_rows:
        n = min(w.outlier_rows, P)
        idx = np.sort(g.choice(P, size=n, replace=False))
        k[idx] *= np.float32(w.outlier_scale)
    return SessionInputs(k=k, v=v, q=q, q_positions=qp, outlier_idx=idx)


def draw_batch(w: Workload, positions: Optional[int] = None,
               q_positions: Optional[Sequence[int]] = None) -> SessionInputs:
    """All sessions of w stacked on a leading batch axis."""
    ss = [draw_session(w, b, positions, q_positions) for b in range(w.batch)]
    return SessionInputs(
        k=np.stack([s.k for s in ss]), v=np.stack([s.v for s in ss]),
        q=np.stack([s.q for s in ss]), q_positions=ss[0].q_positions,
        outlier_idx=None if ss[0].outlier_idx is None
        else np.stack([s.outlier_idx for s in ss]))


def random_case(seed: int, batch: int, num_q_heads: int, num_kv_heads: int,
                head_dim: int, positions: int, n_q: int) -> SessionInputs:
    """Small random case for property tests: N(0,1) K, V, Q in the same order."""
    g = np.random.Generator(np.random.PCG64(seed))
    k = g.standard_normal((batch, positions, num_kv_heads, head_dim), dtype=np.float32)
    v = g.standard_normal((batch, positions, num_kv_heads, head_dim), dtype=np.float32)
    q = g.standard_normal((batch, n_q, num_q_heads, head_dim), dtype=np.float32)
    return SessionInputs(k=k, v=v, q=q, q_positions=np.arange(n_q), outlier_idx=None)
