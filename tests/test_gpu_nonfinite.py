"""Causality with non-finite values in V, on every path that attends a chunk.

The softmax NaN rule of the Karume v0.8.0 release notes ("Breaking Changes")
and causality together fix the result: a NaN or an infinity in V at position
j reaches exactly the rows that see position j, in exactly that value's
dimension, as the oracle's row-by-row sum gives it (NaN for a NaN, for +inf
and -inf together, and +-inf otherwise); every other output stays finite and
within the usual tolerance.  Rows before j must not change at all with what
V holds at j: the kernels share one value product between the rows of a
tile, and a zero weight times NaN would leak it.

Cases cover the bf16 M-tile kernel (several tiles crossing a limit, and an
M-tile of 128 rows whose crossing range spans three key tiles), the int8-K
M-tile, the f32 chunk kernels (pipelined at head_dim 64 and 128, sequential
at 256), the few-row streaming kernel (bf16 and int8-K), ragged batches and
split key ranges.
"""
import numpy as np
import pytest
import torch

import kv_cache_attention_amd as ka
import oracle
from oracle import int8 as oi8
from synth import random_case
from tests.gpu_session import DevCaches, dev

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

TOL = {"f32": 1e-5, "bf16": 1e-2, "i8k": 1e-2}


def _plant(v, start, R, g, D):
    """Non-finite values in KV head g of session 0 (positions relative to
    the chunk start): NaN at chunk row max(1, R // 4) dim 9; +inf at row
    R // 2 and -inf at row R // 2 + 2 in dim 21 (NaN from there on); -inf at
    row R - 1 dim D - 1; NaN 5 positions before the chunk in dim 33 (every
    row sees it).  Returns the list of (position, dim) planted."""
    marks = [(start + max(1, R // 4), 9, np.nan), (start + R // 2, 21, np.inf),
             (start + R // 2 + 2, 21, -np.inf), (start + R - 1, D - 1, -np.inf),
             (start - 5, 33, np.nan)]
    out = []
    for p, d, x in marks:
        if 0 <= p < start + R:
            v[0, p, g, d] = x
            out.append((p, d))
    return out


def _compare(got, ref, vs, dt, what):
    """Same non-finite pattern (NaN where the oracle has NaN, the same
    infinity where it has one), finite values within tolerance."""
    print(what, flush=True)
    ref_nan, ref_inf = np.isnan(ref), np.isinf(ref)
    assert np.array_equal(np.isnan(got), ref_nan), f"{what}: NaN pattern differs"
    assert np.array_equal(np.isinf(got), ref_inf), f"{what}: infinity pattern differs"
    assert np.array_equal(got[ref_inf], ref[ref_inf]), f"{what}: infinity signs differ"
    fin = np.isfinite(ref)
    vmax = float(np.max(np.abs(vs[np.isfinite(vs)])))
    err = float(np.max(np.abs(got[fin] - ref[fin]))) / vmax
    print(f"  finite outputs rel err {err:.3e} (tol {TOL[dt]:g}); "
          f"{int((~fin).sum())} non-finite outputs", flush=True)
    assert err <= TOL[dt], f"{what}: {err}"
    assert (~fin).any()


CASES = [
    # dt, B, Hq, Hkv, D, C, start, R
    ("bf16", 1, 8, 1, 256, 4096, 3000, 40),     # M-tile, 8 query heads
    ("bf16", 1, 8, 1, 256, 4096, 3000, 200),    # several M-tiles
    ("bf16", 1, 1, 1, 64, 4096, 3000, 300),     # 128-row M-tiles: three crossing key tiles
    ("bf16", 2, 4, 2, 128, 2048, 1500, 70),     # two sessions, two KV heads
    ("bf16", 1, 8, 1, 256, 4096, 3072, 768),    # a full 768-row chunk (split key range)
    ("i8k", 1, 8, 1, 256, 4096, 3000, 40),
    ("i8k", 1, 8, 1, 256, 4096, 3000, 2),       # few rows (streaming kernel)
    ("bf16", 1, 8, 1, 256, 4096, 3000, 2),      # few rows: 16 columns
    ("bf16", 1, 2, 1, 256, 4096, 3000, 6),      # few rows: 12 columns
    ("bf16", 1, 8, 1, 256, 131072, 131072 - 15, 15),  # few rows at full capacity
    ("f32", 1, 8, 1, 256, 4096, 3000, 40),      # f32 sequential kernel
    ("f32", 1, 4, 2, 128, 2048, 1000, 70),      # f32 pipelined kernel
    ("f32", 1, 2, 1, 64, 2048, 1000, 30),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_nonfinite_value_reaches_only_rows_that_see_it(case):
    dt, B, Hq, Hkv, D, C, start, R = case
    P = start + R
    c = random_case(31 + R + D, B, Hq, Hkv, D, P, R)
    g = Hkv - 1
    _plant(c.v, start, R, g, D)
    caches = DevCaches(B, Hq, Hkv, D, C, dt)
    caches.append(c.k[:, :start], c.v[:, :start], 0)
    caches.append(c.k[:, start:], c.v[:, start:], start)
    scale = 1.0 / np.sqrt(D)
    print(f"case {case}: plan {ka.prefill_workspace_bytes(caches.shape, R)} B workspace", flush=True)
    got = caches.prefill(c.q, start, scale)
    vs = oracle.stored_values(c.v, "f32" if dt == "f32" else "bf16")
    if dt == "i8k":
        ref = oi8.prefill_chunk_i8(c.q, c.k, vs, start, scale)
    else:
        ref = oracle.prefill_chunk(c.q, oracle.stored_values(c.k, dt), vs, start, scale)
    _compare(got, ref, vs, dt, f"chunk {case}")
    # rows before the first planted position inside the chunk hold no
    # non-finite value except the dim every row sees
    first = min(max(1, R // 4), R // 2)
    before = got[0, :first].copy()
    before[..., 33] = 0.0
    assert np.isfinite(before).all()


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_nonfinite_values_in_a_ragged_batch(dt):
    """Three sessions in one ragged call, each with values planted in its own
    chunk: every session's rows against its own oracle."""
    B, Hq, Hkv, D, C = 3, 8, 1, 128, 2048
    starts, rows = [1000, 40, 1500], [37, 300, 5]
    c = random_case(41, B, Hq, Hkv, D, max(s + r for s, r in zip(starts, rows)), max(rows))
    for b, (s0, n) in enumerate(zip(starts, rows)):
        c.v[b, s0 + 1, 0, 9] = np.nan
        c.v[b, s0 + n // 2, 0, 21] = np.inf
        c.v[b, s0 + n - 1, 0, 50] = -np.inf
    caches = DevCaches(B, Hq, Hkv, D, C, dt)
    caches.append(c.k, c.v, 0)
    q = np.concatenate([c.q[b, :n] for b, n in enumerate(rows)])
    qt = dev(q)
    out = torch.full_like(qt, float("nan"))
    need = ka.prefill_ragged_workspace_need(caches.shape, starts, rows)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    ka.prefill_ragged(caches.shape, qt, caches.k, caches.v, out, starts, rows, 1 / np.sqrt(D), ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    ks, vs = oracle.stored_values(c.k, dt), oracle.stored_values(c.v, dt)
    ref = oracle.prefill_ragged(q, ks, vs, starts, rows, 1 / np.sqrt(D))
    _compare(got, ref, vs, dt, f"ragged {dt} starts {starts} rows {rows}")


@pytest.mark.parametrize("dt", ["bf16", "i8k", "f32"])
def test_a_whole_key_range_of_nan_rows(dt):
    """256 consecutive NaN key rows (more than a split's share of keys): every
    row that sees them is NaN in full, on the decode path and on the chunk
    path, even where a whole split sees nothing but NaN scores; rows that
    cannot see them match the oracle."""
    B, Hq, Hkv, D, C = 1, 8, 1, 256, 8192
    c = random_case(47, B, Hq, Hkv, D, 8192, 4)
    c.k[0, 4096:4352] = np.nan
    caches = DevCaches(B, Hq, Hkv, D, C, dt)
    caches.append(c.k, c.v, 0)
    got = caches.decode(c.q[:, 0], [8192], 1 / 16)
    assert np.isnan(got).all()
    got = caches.decode(c.q[:, 0], [4000], 1 / 16)
    vs = oracle.stored_values(c.v, "f32" if dt == "f32" else "bf16")
    ks = oracle.stored_values(c.k, "f32" if dt == "f32" else "bf16")
    if dt == "i8k":
        ref = oi8.decode_i8(c.q[:, 0], c.k, vs, [4000], 1 / 16)
    else:
        ref = oracle.decode(c.q[:, 0], ks, vs, [4000], 1 / 16)
    assert oracle.rel_error(got, ref, vs[:, :4000]) <= TOL[dt]
    # a chunk straddling the NaN range: rows before 4096 finite, rows after NaN
    q = c.q[:, :4].repeat(10, axis=1)[:, :40]
    got = caches.prefill(q, 4076, 1 / 16)
    assert np.isfinite(got[:, :20]).all() and np.isnan(got[:, 20:]).all()
