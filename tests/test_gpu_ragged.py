"""GPU parity of ragged batches (sessions at different positions in one
call), of the session memory estimate and of the cache resize, against the
CPU float64 oracle and the test-side layout readers.

Appends are compared bit for bit; attention within the usual tolerances
(error relative to max |V stored|): 1e-5 for f32 caches, 1e-2 for bf16.
"""
import math

import numpy as np
import pytest
import torch

import kv_cache_attention_amd as ka
import oracle
from oracle import bf16 as obf16
from oracle import rope as orope
from synth import random_case
from tests.gpu_session import DevCaches, dev

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

TOL = {"f32": 1e-5, "bf16": 1e-2}


def _say(*a):
    print(*a, flush=True)


def _bits(x, dt):
    """Bit patterns a cache of dtype dt holds for f32 values x."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return obf16.encode_rne(x) if dt == "bf16" else x.view(np.uint32)


def _cache_bits(caches, dt):
    """K and V element bit patterns [B][Hkv][C][D] (uint16 or uint32)."""
    kb, vb = caches.bits()
    if dt == "f32":
        kb, vb = np.ascontiguousarray(kb).view(np.uint32), np.ascontiguousarray(vb).view(np.uint32)
    return kb, vb


def _poison_bits(dt):
    return np.uint16(0xFFFF) if dt == "bf16" else np.uint32(0xFFFFFFFF)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_ragged_append_is_exact_and_touches_only_its_rows(dt):
    B, Hq, Hkv, D, C = 4, 8, 2, 128, 1088
    starts, rows = [0, 100, 37, 1000], [5, 0, 64, 88]
    _say(f"ragged append {dt} starts {starts} rows {rows}")
    g = np.random.default_rng(7)
    k_rows = [g.standard_normal((r, Hkv, D)).astype(np.float32) for r in rows]
    v_rows = [g.standard_normal((r, Hkv, D)).astype(np.float32) for r in rows]
    caches = DevCaches(B, Hq, Hkv, D, C, dt)
    ka.append_kv_ragged(caches.shape, caches.k, caches.v, dev(np.concatenate(k_rows)),
                        dev(np.concatenate(v_rows)), starts, rows)
    kb, vb = _cache_bits(caches, dt)   # [B][Hkv][C][D]
    for b in range(B):
        written = np.zeros(C, bool)
        written[starts[b]:starts[b] + rows[b]] = True
        for got, src in ((kb, k_rows[b]), (vb, v_rows[b])):
            want = _bits(src, dt).transpose(1, 0, 2)           # [Hkv][r][D]
            assert np.array_equal(got[b][:, written], want)
            assert (got[b][:, ~written] == _poison_bits(dt)).all()


def test_ragged_append_rope_rotates_each_row_at_its_own_position():
    B, Hq, Hkv, D, C = 3, 8, 1, 256, 640
    starts, rows = [10, 0, 500], [7, 0, 33]
    g = np.random.default_rng(8)
    T = sum(rows)
    k = g.standard_normal((T, Hkv, D)).astype(np.float32)
    v = g.standard_normal((T, Hkv, D)).astype(np.float32)
    pos = np.concatenate([np.arange(s, s + r) for s, r in zip(starts, rows)])
    cos, sin = orope.angles_table(pos, D)
    caches = DevCaches(B, Hq, Hkv, D, C, "bf16")
    ka.append_kv_ragged(caches.shape, caches.k, caches.v, dev(k), dev(v), starts, rows,
                        rope_cos=dev(cos), rope_sin=dev(sin))
    kb, vb = _cache_bits(caches, "bf16")
    r0 = 0
    for b in range(B):
        if rows[b] == 0:
            assert (kb[b] == _poison_bits("bf16")).all()
            continue
        kr = orope.rotate_half_f32(k[r0:r0 + rows[b]], cos[r0:r0 + rows[b]], sin[r0:r0 + rows[b]])
        sl = slice(starts[b], starts[b] + rows[b])
        assert np.array_equal(kb[b][:, sl], _bits(kr, "bf16").transpose(1, 0, 2))
        assert np.array_equal(vb[b][:, sl], _bits(v[r0:r0 + rows[b]], "bf16").transpose(1, 0, 2))
        r0 += rows[b]


def _ragged_case(dt, B, Hq, Hkv, D, C, starts, rows, seed):
    c = random_case(seed, B, Hq, Hkv, D, C, 1)
    caches = DevCaches(B, Hq, Hkv, D, C, dt)
    caches.append(c.k, c.v, 0)
    g = np.random.default_rng(seed + 1)
    T = sum(rows)
    q = g.standard_normal((T, Hq, D)).astype(np.float32)
    qt = dev(q)
    out = torch.full_like(qt, float("nan"))
    ws = caches.workspace(ka.prefill_ragged_workspace_bytes(caches.shape, T))
    scale = 1.0 / math.sqrt(D)
    ka.prefill_ragged(caches.shape, qt, caches.k, caches.v, out, starts, rows, scale, ws)
    torch.cuda.synchronize()
    ks, vs = oracle.stored_values(c.k, dt), oracle.stored_values(c.v, dt)
    ref = oracle.prefill_ragged(q, ks, vs, starts, rows, scale)
    return out.cpu().numpy(), ref, vs, caches, q


RAGGED_CASES = [
    # dt, B, Hq, Hkv, D, C, starts, rows
    ("bf16", 5, 8, 1, 256, 4096, [0, 100, 2048, 3000, 17], [1, 0, 37, 768, 300]),
    ("f32", 3, 8, 1, 256, 2048, [1000, 0, 5], [200, 64, 2]),
    ("bf16", 2, 16, 2, 128, 1024, [500, 3], [100, 500]),
    ("f32", 2, 6, 2, 64, 320, [250, 0], [70, 1]),
]


@pytest.mark.parametrize("case", RAGGED_CASES, ids=lambda c: f"{c[0]}-B{c[1]}-D{c[4]}")
def test_ragged_prefill_matches_oracle(case):
    dt, B, Hq, Hkv, D, C, starts, rows = case
    _say(f"ragged prefill {case}")
    got, ref, vs, _, _ = _ragged_case(dt, B, Hq, Hkv, D, C, starts, rows, seed=B + D)
    err = oracle.rel_error(got, ref, vs)
    _say(f"  rel err {err:.3e}")
    assert np.isfinite(got).all()
    assert err <= TOL[dt]


def test_ragged_prefill_many_sessions():
    """40 sessions (more than one launch table), random positions and row
    counts, some empty."""
    B, Hq, Hkv, D, C = 40, 8, 1, 64, 256
    g = np.random.default_rng(40)
    rows = [int(x) for x in g.integers(0, 41, size=B)]
    rows[3] = rows[17] = 0
    starts = [int(g.integers(0, C - r + 1)) for r in rows]
    _say(f"ragged prefill 40 sessions, {sum(rows)} rows")
    got, ref, vs, _, _ = _ragged_case("bf16", B, Hq, Hkv, D, C, starts, rows, seed=41)
    err = oracle.rel_error(got, ref, vs)
    _say(f"  rel err {err:.3e}")
    assert np.isfinite(got).all() and err <= TOL["bf16"]


def test_ragged_with_equal_sessions_is_bitwise_the_uniform_chunk():
    B, Hq, Hkv, D, C, start, R = 3, 8, 1, 256, 2048, 1000, 100
    c = random_case(77, B, Hq, Hkv, D, C, R)
    caches = DevCaches(B, Hq, Hkv, D, C, "bf16")
    caches.append(c.k, c.v, 0)
    uni = caches.prefill(c.q, start, 1 / 16)
    qt = dev(c.q.reshape(B * R, Hq, D))
    out = torch.full_like(qt, float("nan"))
    ws = caches.workspace(ka.prefill_ragged_workspace_bytes(caches.shape, B * R))
    ka.prefill_ragged(caches.shape, qt, caches.k, caches.v, out, [start] * B, [R] * B, 1 / 16, ws)
    torch.cuda.synchronize()
    rag = out.cpu().numpy().reshape(B, R, Hq, D)
    assert np.array_equal(rag.view(np.uint32), uni.view(np.uint32))


def test_session_memory_workspace_serves_prefill_and_decode():
    """The estimate's workspace (the larger of the two) serves a 768-row
    chunk at the end of the window and a decode at full capacity."""
    B, Hq, Hkv, D, C = 2, 8, 1, 256, 8192
    caches = DevCaches(B, Hq, Hkv, D, C, "bf16")
    m = ka.session_memory(caches.shape, 768)
    ws = torch.empty(max(m.prefill_workspace_bytes, m.decode_workspace_bytes), dtype=torch.uint8,
                     device="cuda")
    c = random_case(5, B, Hq, Hkv, D, C, 768)
    caches.append(c.k, c.v, 0)
    ks, vs = oracle.stored_values(c.k, "bf16"), oracle.stored_values(c.v, "bf16")
    qt = dev(c.q)
    out = torch.full_like(qt, float("nan"))
    ka.prefill_chunk(caches.shape, qt, caches.k, caches.v, out, C - 768, 768, 1 / 16, ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    rows = [0, 383, 767]
    ref = np.stack([oracle.attend_rows(c.q[b, rows], ks[b], vs[b], [C - 768 + r for r in rows], 1 / 16)
                    for b in range(B)])
    assert oracle.rel_error(got[:, rows], ref, vs) <= TOL["bf16"]
    qd = dev(c.q[:, 0])
    od = torch.full_like(qd, float("nan"))
    ka.decode(caches.shape, qd, caches.k, caches.v, od, [C] * B, 1 / 16, ws)
    torch.cuda.synchronize()
    refd = oracle.decode(c.q[:, 0], ks, vs, [C] * B, 1 / 16)
    assert oracle.rel_error(od.cpu().numpy(), refd, vs) <= TOL["bf16"]


@pytest.mark.parametrize("dt,C2", [("bf16", 2048), ("bf16", 704), ("f32", 1472)])
def test_cache_resize_keeps_every_row(dt, C2):
    B, Hq, Hkv, D, C, n = 2, 4, 2, 64, 1024, 700
    _say(f"resize {dt} {C} -> {C2}, {n} rows")
    c = random_case(9, B, Hq, Hkv, D, n, 16)
    a = DevCaches(B, Hq, Hkv, D, C, dt)
    a.append(c.k, c.v, 0)
    b = DevCaches(B, Hq, Hkv, D, C2, dt)
    ka.cache_resize(a.shape, a.k, a.v, b.shape, b.k, b.v, n)
    ka_, va_ = _cache_bits(a, dt)
    kb_, vb_ = _cache_bits(b, dt)
    assert np.array_equal(ka_[:, :, :n], kb_[:, :, :n])
    assert np.array_equal(va_[:, :, :n], vb_[:, :, :n])
    # the resized cache serves attention like the original
    got = b.prefill(c.q, n - 16, 0.125)
    ks, vs = oracle.stored_values(c.k, dt), oracle.stored_values(c.v, dt)
    ref = oracle.prefill_chunk(c.q, ks, vs, n - 16, 0.125)
    assert oracle.rel_error(got, ref, vs) <= TOL[dt]
