"""GPU parity of the rotary-embedding entry points against the oracle.

The rotation is specified in f32 as two rounded products and one rounded sum
or difference (no fused multiply-add), and the oracle evaluates it the same
way, so rotated K rows are compared bit for bit in the cache (after the
cache's own RNE rounding for bf16) and rotated query rows bit for bit in f32.
Rows holding a NaN are compared as NaN only: NaN payloads are not specified.
"""
import math

import numpy as np
import pytest
import torch

import kv_cache_attention_amd as ka
import oracle
from oracle import bf16 as obf16
from synth import random_case
from tests.gpu_session import DevCaches, dev

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

TOL = {"f32": 1e-5, "bf16": 1e-2}


@pytest.mark.parametrize("dt,B,Hkv,D,start,R", [
    ("bf16", 1, 1, 256, 0, 768),
    ("bf16", 2, 2, 128, 100, 77),
    ("f32", 2, 1, 64, 37, 300),
    ("f32", 1, 2, 256, 4000, 96),
])
def test_append_rope_stores_rotated_k_bit_exactly(dt, B, Hkv, D, start, R):
    C = ((start + R + 63) // 64) * 64
    c = random_case(60 + D + R, B, Hkv, Hkv, D, start + R, 1)
    k_new = (c.k[:, start:] * 4).astype(np.float32)
    v_new = c.v[:, start:]
    cos, sin = oracle.rope.angles_table(np.arange(start, start + R), D)
    caches = DevCaches(B, Hkv, Hkv, D, C, dt)
    caches.append_rope(k_new, v_new, cos, sin, start)
    kb, vb = caches.bits()                                   # [B][Hkv][C][D]
    want_k = oracle.rope.rotate_half_f32(k_new, cos, sin)    # [B][R][Hkv][D]
    want_k = want_k.transpose(0, 2, 1, 3)
    want_v = v_new.transpose(0, 2, 1, 3)
    if dt == "bf16":
        got_k, exp_k = kb[:, :, start:start + R], obf16.encode_rne(want_k)
        bad = np.argwhere(got_k != exp_k)
        assert len(bad) == 0, (len(bad), [(tuple(i), int(got_k[tuple(i)]), int(exp_k[tuple(i)]),
                                           float(want_k[tuple(i)])) for i in bad[:6]])
        assert np.array_equal(vb[:, :, start:start + R], obf16.encode_rne(want_v))
        assert np.all(kb[:, :, :start] == 0xFFFF) and np.all(kb[:, :, start + R:] == 0xFFFF)
    else:
        assert np.array_equal(kb[:, :, start:start + R].view(np.uint32),
                              np.ascontiguousarray(want_k).view(np.uint32))
        assert np.array_equal(vb[:, :, start:start + R].view(np.uint32),
                              np.ascontiguousarray(want_v).view(np.uint32))


def test_append_rope_nan_reaches_both_dims_of_its_pair_only():
    B, Hkv, D, R = 1, 1, 64, 4
    c = random_case(70, B, Hkv, Hkv, D, R, 1)
    k_new = c.k.copy()
    k_new[0, 2, 0, 5] = np.nan                   # pair (5, 37) of row 2
    cos, sin = oracle.rope.angles_table(np.arange(R), D)
    caches = DevCaches(B, Hkv, Hkv, D, 64, "f32")
    caches.append_rope(k_new, c.v, cos, sin, 0)
    kl, _ = caches.logical()                      # [B][C][Hkv][D]
    nan = np.isnan(kl[0, :R, 0])
    assert nan[2, 5] and nan[2, 37] and nan.sum() == 2


@pytest.mark.parametrize("inplace", [False, True])
def test_rope_rows_bit_exact(inplace):
    B, Hq, D, R = 2, 8, 256, 33
    rng = np.random.default_rng(80)
    x = (rng.standard_normal((B, R, Hq, D)) * 3).astype(np.float32)
    cos, sin = oracle.rope.angles_table(np.arange(500, 500 + R), D)
    shape = ka.Shape(B, Hq, 1, D, 1024, ka.BF16)
    xt = dev(x)
    yt = xt if inplace else torch.empty_like(xt)
    ka.rope_rows(shape, xt, yt, dev(cos), dev(sin), R)
    torch.cuda.synchronize()
    want = oracle.rope.rotate_half_f32(x, cos, sin)
    assert np.array_equal(yt.cpu().numpy().view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_prefill_and_decode_on_rotated_rows(dt):
    """Q rotated by rope_rows, K by append_kv_rope, then a chunk prefill and
    a decode step: the oracle attends over the same rotated values."""
    B, Hq, Hkv, D, start, R = 1, 8, 1, 128, 600, 200
    C = 832
    c = random_case(90, B, Hq, Hkv, D, start + R + 1, R + 1)
    pos = np.arange(start + R + 1)
    cos, sin = oracle.rope.angles_table(pos, D)
    caches = DevCaches(B, Hq, Hkv, D, C, dt)
    caches.append_rope(c.k[:, :start], c.v[:, :start], cos[:start], sin[:start], 0)
    caches.append_rope(c.k[:, start:start + R], c.v[:, start:start + R], cos[start:start + R],
                       sin[start:start + R], start)
    shape = caches.shape
    q = c.q[:, :R]
    qt = dev(q)
    ka.rope_rows(shape, qt, qt, dev(cos[start:start + R]), dev(sin[start:start + R]), R)
    out = torch.full_like(qt, float("nan"))
    ws = caches.workspace(ka.prefill_workspace_bytes(shape, R))
    scale = 1 / math.sqrt(D)
    ka.prefill_chunk(shape, qt, caches.k, caches.v, out, start, R, scale, ws)
    torch.cuda.synchronize()
    k_rot = oracle.rope.rotate_half_f32(c.k[:, :start + R], cos[:start + R], sin[:start + R])
    q_rot = oracle.rope.rotate_half_f32(q, cos[start:start + R], sin[start:start + R])
    ks, vs = oracle.stored_values(k_rot, dt), oracle.stored_values(c.v[:, :start + R], dt)
    ref = oracle.prefill_chunk(q_rot, ks, vs, start, scale)
    err = oracle.rel_error(out.cpu().numpy(), ref, vs)
    assert err <= TOL[dt], err
    # one decode step at position start + R: append the rotated row, rotate q, decode
    p = start + R
    caches.append_rope(c.k[:, p:p + 1], c.v[:, p:p + 1], cos[p:p + 1], sin[p:p + 1], p)
    qd = c.q[:, R:R + 1]                                    # [B][1][Hq][D]
    qdt = dev(qd)
    ka.rope_rows(shape, qdt, qdt, dev(cos[p:p + 1]), dev(sin[p:p + 1]), 1)
    got = caches.decode(qdt.cpu().numpy()[:, 0], [p + 1], scale)
    k_rot = oracle.rope.rotate_half_f32(c.k[:, :p + 1], cos[:p + 1], sin[:p + 1])
    ks, vs = oracle.stored_values(k_rot, dt), oracle.stored_values(c.v[:, :p + 1], dt)
    qd_rot = oracle.rope.rotate_half_f32(qd, cos[p:p + 1], sin[p:p + 1])[:, 0]
    ref = oracle.decode(qd_rot, ks, vs, [p + 1], scale)
    err = oracle.rel_error(got, ref, vs)
    assert err <= TOL[dt], err
