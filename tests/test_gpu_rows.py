"""GPU parity of chunks of a few rows (1 to 15) against the CPU float64 oracle.

On bf16 caches a chunk whose (row, head) pairs fit 16 MFMA columns is served
by the streaming decode kernel, each column with its own causal limit; longer
chunks take the MFMA prefill tile.  Either way the results must match the
oracle, so these cases do not depend on where the dispatch line sits.  Same
tolerances as the other parity tests (error relative to max |V stored|).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from synth import random_case
from tests.gpu_session import DevCaches

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

TOL = {"f32": 1e-5, "bf16": 1e-2}


def _check(got, ref, v_store, dt, what):
    err = oracle.rel_error(got, ref, v_store)
    print(f"{what}: rel err {err:.3e} (tol {TOL[dt]:g})", flush=True)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    assert err <= TOL[dt], f"{what}: {err} > {TOL[dt]}"


def _case(dt, B, Hq, Hkv, D, C, start, R, seed):
    P = start + R
    c = random_case(seed, B, Hq, Hkv, D, P, R)
    caches = DevCaches(B, Hq, Hkv, D, C, dt)
    if start:
        caches.append(c.k[:, :start], c.v[:, :start], 0)
    caches.append(c.k[:, start:P], c.v[:, start:P], start)
    scale = 1.0 / math.sqrt(D)
    got = caches.prefill(c.q, start, scale)
    ks, vs = oracle.stored_values(c.k, dt), oracle.stored_values(c.v, dt)
    ref = oracle.prefill_chunk(c.q, ks, vs, start, scale)
    return got, ref, vs


ROW_CASES = [
    # dt, B, Hq, Hkv, D, C, start, R
    ("bf16", 1, 8, 1, 256, 64, 0, 2),        # row 0 sees one key
    ("bf16", 1, 8, 1, 256, 1024, 1000, 2),
    ("bf16", 1, 8, 1, 256, 1024, 30, 2),     # the chunk crosses a 32-position tile
    ("bf16", 1, 8, 1, 256, 1088, 1001, 3),
    ("bf16", 1, 8, 1, 256, 1088, 1017, 15),
    ("bf16", 1, 4, 4, 64, 512, 477, 15),     # one head per group: 15 columns
    ("bf16", 2, 4, 2, 128, 640, 600, 8),     # 2 heads x 8 rows = 16 columns
    ("bf16", 1, 6, 2, 64, 256, 200, 5),      # 3 heads x 5 rows = 15 columns
    ("bf16", 1, 16, 1, 128, 256, 100, 1),    # 16 heads, one row
    ("bf16", 1, 16, 1, 128, 256, 100, 2),    # 32 pairs
    ("bf16", 3, 2, 1, 256, 5120, 4999, 7),   # split context, several sessions
    ("bf16", 1, 1, 1, 64, 128, 0, 15),
    ("bf16", 1, 8, 1, 256, 16384, 16368, 16),  # past the band: one M-tile, many splits
    ("f32", 1, 8, 1, 256, 1024, 1000, 2),
    ("f32", 2, 4, 2, 64, 320, 290, 9),
]


@pytest.mark.parametrize("case", ROW_CASES, ids=lambda c: "-".join(map(str, c)))
def test_few_row_chunks(case):
    dt, B, Hq, Hkv, D, C, start, R = case
    got, ref, vs = _case(dt, B, Hq, Hkv, D, C, start, R, seed=sum(case[1:]) + 5)
    _check(got, ref, vs, dt, f"rows {case}")
    if start == 0:
        # row 0 attends to key 0 alone: its output is that value row exactly
        for h in range(Hq):
            assert np.array_equal(got[:, 0, h], vs[:, 0, h // (Hq // Hkv)].astype(np.float32))


@pytest.mark.parametrize("R", list(range(1, 16)))
def test_every_row_count_at_16k(R):
    """R = 1 .. 15 rows ending at position 16384 (8 query heads on one KV
    head, head_dim 256): the few-row band of the long-session shape."""
    got, ref, vs = _case("bf16", 1, 8, 1, 256, 16384, 16384 - R, R, seed=100 + R)
    _check(got, ref, vs, "bf16", f"{R} rows at 16K")


def test_rows_at_full_capacity():
    """15 rows ending at position 131072, the largest context."""
    C = 131072
    got, ref, vs = _case("bf16", 1, 8, 1, 256, C, C - 15, 15, seed=77)
    _check(got, ref, vs, "bf16", "15 rows at 131072")
    got, ref, vs = _case("bf16", 1, 8, 1, 256, C, C - 2, 2, seed=78)
    _check(got, ref, vs, "bf16", "2 rows at 131072")


def test_incremental_suffix_chunks():
    """A session extended by short chunks (append, then attend), each checked
    against the oracle on the whole prefix."""
    dt, B, Hq, Hkv, D, C = "bf16", 1, 8, 1, 256, 2048
    sizes = [3, 7, 1, 15, 2, 2, 11, 1]
    total = 700 + sum(sizes)
    c = random_case(55, B, Hq, Hkv, D, total, total)
    caches = DevCaches(B, Hq, Hkv, D, C, dt)
    caches.append(c.k[:, :700], c.v[:, :700], 0)
    ks, vs = oracle.stored_values(c.k, dt), oracle.stored_values(c.v, dt)
    pos = 700
    for r in sizes:
        caches.append(c.k[:, pos:pos + r], c.v[:, pos:pos + r], pos)
        got = caches.prefill(c.q[:, pos:pos + r], pos, 1 / 16)
        ref = oracle.prefill_chunk(c.q[:, pos:pos + r], ks[:, :pos + r], vs[:, :pos + r], pos, 1 / 16)
        _check(got, ref, vs[:, :pos + r], dt, f"suffix chunk {pos}+{r}")
        pos += r


def test_few_rows_deterministic_and_key_nan_reaches_later_rows_only():
    """Same call twice: identical bits.  A NaN in the key at the chunk's third
    position (2 query heads on one KV head, 6 rows: 12 columns): rows 0 and 1,
    which cannot see it, match the oracle; every later row is NaN in full (a
    NaN score poisons its row)."""
    dt, B, Hkv, D, C, start = "bf16", 1, 1, 256, 4096, 3000
    c = random_case(9, B, 8, Hkv, D, start + 2, 2)
    caches = DevCaches(B, 8, Hkv, D, C, dt)
    caches.append(c.k, c.v, 0)
    a = caches.prefill(c.q, start, 1 / 16)
    b = caches.prefill(c.q, start, 1 / 16)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))

    Hq, R = 2, 6
    c = random_case(19, B, Hq, Hkv, D, start + R, R)
    c.k[0, start + 2, 0, 5] = np.nan
    caches = DevCaches(B, Hq, Hkv, D, C, dt)
    caches.append(c.k, c.v, 0)
    got = caches.prefill(c.q, start, 1 / 16)
    ks, vs = oracle.stored_values(c.k, dt), oracle.stored_values(c.v, dt)
    ref = oracle.prefill_chunk(c.q[:, :2], ks, vs, start, 1 / 16)
    assert np.isfinite(got[:, :2]).all()
    assert oracle.rel_error(got[:, :2], ref, vs) <= TOL[dt]
    assert np.isnan(got[:, 2:]).all()


@pytest.mark.parametrize("Hq,R,start", [(8, 2, 3000), (2, 6, 3000), (8, 40, 3000)])
def test_value_nan_inside_chunk_stays_in_its_dimension(Hq, R, start):
    """A NaN value at (chunk position 1, dim 9): rows from position 1 on are
    NaN in dim 9 and nowhere else; row 0, which cannot see it, is finite and
    matches the oracle, as does every other dim of every row.  Covers the
    streaming kernel (16 and 12 columns) and the M-tile kernel (40 rows)."""
    dt, B, Hkv, D, C = "bf16", 1, 1, 256, 4096
    c = random_case(23 + R, B, Hq, Hkv, D, start + R, R)
    c.v[0, start + 1, 0, 9] = np.nan
    caches = DevCaches(B, Hq, Hkv, D, C, dt)
    caches.append(c.k, c.v, 0)
    got = caches.prefill(c.q, start, 1 / 16)
    ks, vs = oracle.stored_values(c.k, dt), oracle.stored_values(c.v, dt)
    ref = oracle.prefill_chunk(c.q, ks, vs, start, 1 / 16)
    finite_v = np.nan_to_num(vs)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.isnan(got[:, 1:, :, 9]).all()
    assert np.isfinite(got[:, 0]).all()
    fin = np.isfinite(ref)
    assert float(np.max(np.abs(got[fin] - ref[fin]))) / np.abs(finite_v).max() <= TOL[dt]
