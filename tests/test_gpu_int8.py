"""GPU parity of int8-K caches (int8 K codes with per-row scales, bf16 V,
integer scores) against the CPU oracle ``oracle.int8``.

Codes and scales are integer / f32 decisions both sides take in f32: they
are compared bit for bit.  Attention outputs are compared within the bf16
tolerance (1e-2 of max |V stored|): the GPU's remaining differences are its
f32 epilogue, its bf16 weights and its summation order, as on bf16 caches.
"""
import math

import numpy as np
import pytest
import torch

import kv_cache_attention_amd as ka
import oracle
from oracle import bf16 as obf16
from oracle import int8 as oi8
from oracle import rope as orope
from synth import random_case
from tests.gpu_session import DevCaches, dev

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

TOL = 1e-2


def _say(*a):
    print(*a, flush=True)


def _check(got, ref, vs, what):
    err = oracle.rel_error(got, ref, vs)
    _say(f"{what}: rel err {err:.3e} (tol {TOL:g})")
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    assert err <= TOL, f"{what}: {err} > {TOL}"


def test_int8_self_test_passes():
    ka.int8_self_test()
    ka.int8_self_test()   # cached


def _codes_match(caches, k, upto):
    """Codes and scales of positions 0 .. upto-1 equal the oracle's (k [B][P][Hkv][D])."""
    codes, scales = caches.k_i8()
    wc, ws = oi8.quantize_rows(k[:, :upto])                  # [B][P][Hkv][D], [B][P][Hkv]
    assert np.array_equal(codes[:, :, :upto], wc.transpose(0, 2, 1, 3))
    got_s = scales[:, :, :upto].view(np.uint32)
    want_s = np.ascontiguousarray(ws.transpose(0, 2, 1)).view(np.uint32)
    nan = np.isnan(ws.transpose(0, 2, 1))
    assert np.array_equal(got_s[~nan], want_s[~nan])
    assert np.isnan(scales[:, :, :upto][nan]).all()


def test_append_quantises_rows_exactly():
    """Chunked appends, with a zero row, a NaN row, an infinite row and rows
    of very large and very small magnitude; V is stored as bf16."""
    B, Hq, Hkv, D, C = 2, 4, 2, 128, 256
    c = random_case(3, B, Hq, Hkv, D, 200, 1)
    c.k[0, 5] = 0.0
    c.k[1, 9, 0, 17] = np.nan
    c.k[0, 33, 1, 4] = np.inf
    c.k[1, 70] *= np.float32(1e30)
    c.k[0, 71] *= np.float32(1e-30)
    caches = DevCaches(B, Hq, Hkv, D, C, "i8k")
    for s0, s1 in [(0, 37), (37, 38), (38, 130), (130, 200)]:
        caches.append(c.k[:, s0:s1], c.v[:, s0:s1], s0)
    _codes_match(caches, c.k, 200)
    vb = caches.v_bits()
    assert np.array_equal(vb[:, :, :200], obf16.encode_rne(np.ascontiguousarray(c.v.transpose(0, 2, 1, 3))))


def test_append_codes_at_rounding_boundaries():
    """Values whose quotient x / s lies at, or one f32 step beside, a
    half-integer k + 1/2: the codes there depend on the exact rounding of the
    division, which the kernels' product form hands to the division.  Row
    magnitudes span the f32 range, including scales outside [2^-125, 2^125]."""
    B, Hq, Hkv, D, C = 1, 4, 2, 128, 128
    g = np.random.default_rng(12)
    rows = 100
    k = np.zeros((B, rows, Hkv, D), np.float32)
    for r in range(rows):
        for h in range(Hkv):
            mag = np.float32(10.0) ** np.float32(g.uniform(-40, 36))
            amax = np.float32(127) * mag
            s = np.float32(amax * oi8.INV127)
            half = ((g.integers(-127, 127, size=D).astype(np.float32) + np.float32(0.5)) * s).astype(np.float32)
            step = g.integers(-1, 2, size=D)
            x = np.where(step > 0, np.nextafter(half, np.float32(np.inf)),
                         np.where(step < 0, np.nextafter(half, np.float32(-np.inf)), half)).astype(np.float32)
            x = np.clip(x, -amax, amax)
            x[0] = amax  # fixes the row's amax, so its scale is s
            k[0, r, h] = x
    v = g.standard_normal((B, rows, Hkv, D)).astype(np.float32)
    caches = DevCaches(B, Hq, Hkv, D, C, "i8k")
    caches.append(k, v, 0)
    _codes_match(caches, k, rows)


def test_append_rope_then_quantise():
    B, Hq, Hkv, D, C, start, R = 1, 8, 1, 256, 640, 300, 77
    c = random_case(4, B, Hq, Hkv, D, start + R, 1)
    cos, sin = orope.angles_table(np.arange(start, start + R), D)
    caches = DevCaches(B, Hq, Hkv, D, C, "i8k")
    ka.append_kv_rope(caches.shape, caches.k, caches.v, dev(c.k[:, start:]), dev(c.v[:, start:]),
                      dev(cos), dev(sin), start, R)
    rot = orope.rotate_half_f32(c.k[0, start:], cos, sin)[None]
    codes, scales = caches.k_i8()
    wc, ws = oi8.quantize_rows(rot)
    assert np.array_equal(codes[:, :, start:start + R], wc.transpose(0, 2, 1, 3))
    assert np.array_equal(scales[:, :, start:start + R], ws.transpose(0, 2, 1))


DECODE_CASES = [
    # B, Hq, Hkv, D, C, ctxs
    (1, 8, 1, 256, 64, [1]),
    (3, 8, 1, 256, 1088, [17, 1000, 1025]),
    (2, 16, 2, 128, 5120, [5000, 4097]),
    (1, 6, 3, 64, 256, [200]),
    (2, 32, 4, 128, 128, [100, 128]),
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=lambda c: "-".join(map(str, c[:5])))
def test_decode(case):
    B, Hq, Hkv, D, C, ctxs = case
    c = random_case(20 + D + B, B, Hq, Hkv, D, max(ctxs), 1)
    caches = DevCaches(B, Hq, Hkv, D, C, "i8k")
    caches.append(c.k, c.v, 0)
    scale = 1 / math.sqrt(D)
    got = caches.decode(c.q[:, 0], ctxs, scale)
    vs = oracle.stored_values(c.v, "bf16")
    ref = oi8.decode_i8(c.q[:, 0], c.k, vs, ctxs, scale)
    _check(got, ref, vs, f"int8 decode {case}")


def test_decode_at_128k():
    """Four sessions at 131072 positions, the long-context shape."""
    B, Hq, Hkv, D, C = 4, 8, 1, 256, 131072
    c = random_case(31, B, Hq, Hkv, D, C, 1)
    caches = DevCaches(B, Hq, Hkv, D, C, "i8k")
    caches.append(c.k, c.v, 0)
    got = caches.decode(c.q[:, 0], [C] * B, 1 / 16)
    vs = oracle.stored_values(c.v, "bf16")
    ref = oi8.decode_i8(c.q[:, 0], c.k, vs, [C] * B, 1 / 16)
    _check(got, ref, vs, "int8 decode 4 x 131072")


def test_decode_step_appends_then_decodes():
    """Session b holds rows 0 .. pos[b] - 1; its step appends row pos[b]
    (quantised by the append kernel) and decodes there."""
    B, Hq, Hkv, D, C = 2, 8, 1, 256, 2048
    pos = [1000, 1499]
    c = random_case(32, B, Hq, Hkv, D, 1500, 1)
    caches = DevCaches(B, Hq, Hkv, D, C, "i8k")
    ka.append_kv_ragged(caches.shape, caches.k, caches.v,
                        dev(np.concatenate([c.k[b, :pos[b]] for b in range(B)])),
                        dev(np.concatenate([c.v[b, :pos[b]] for b in range(B)])), [0, 0], pos)
    kn = np.stack([c.k[b, pos[b]] for b in range(B)])   # [B][Hkv][D]
    vn = np.stack([c.v[b, pos[b]] for b in range(B)])
    got = caches.decode_step(c.q[:, 0], kn, vn, pos, 1 / 16)
    vs = oracle.stored_values(c.v, "bf16")
    ref = oi8.decode_i8(c.q[:, 0], c.k, vs, [p + 1 for p in pos], 1 / 16)
    _check(got, ref, vs, "int8 decode step")
    codes, scales = caches.k_i8()
    wc, ws = oi8.quantize_rows(kn)
    for b in range(B):
        assert np.array_equal(codes[b, :, pos[b]], wc[b])
        assert np.array_equal(scales[b, :, pos[b]], ws[b])


PREFILL_CASES = [
    # B, Hq, Hkv, D, C, start, R
    (1, 8, 1, 256, 448, 100, 77),
    (1, 8, 1, 256, 2048, 1500, 548),
    (2, 8, 2, 128, 384, 37, 300),
    (1, 4, 4, 64, 192, 64, 64),
    (3, 2, 1, 64, 512, 300, 150),
    (1, 8, 1, 256, 4096, 3000, 768),
    (1, 8, 1, 256, 1024, 1000, 2),       # few rows: the streaming kernel
    (1, 8, 1, 256, 16384, 16369, 15),
    (2, 4, 2, 128, 640, 600, 8),
]


@pytest.mark.parametrize("case", PREFILL_CASES, ids=lambda c: "-".join(map(str, c)))
def test_prefill(case):
    B, Hq, Hkv, D, C, start, R = case
    c = random_case(40 + R + D, B, Hq, Hkv, D, start + R, R)
    caches = DevCaches(B, Hq, Hkv, D, C, "i8k")
    caches.append(c.k, c.v, 0)
    scale = 1 / math.sqrt(D)
    got = caches.prefill(c.q, start, scale)
    vs = oracle.stored_values(c.v, "bf16")
    ref = oi8.prefill_chunk_i8(c.q, c.k, vs, start, scale)
    _check(got, ref, vs, f"int8 prefill {case}")


def test_prefill_split_partials_per_dim_range():
    """Value dims scaled by 2^-6 .. 2^6 (a different power per dim), a chunk
    long enough to be split: every dim keeps its own relative accuracy through
    the binary16 split partials (per-lane scales), as on bf16 caches."""
    B, Hq, Hkv, D, start, R = 1, 8, 1, 256, 2048, 256
    C = start + R
    c = random_case(42, B, Hq, Hkv, D, C, R)
    rng = np.random.default_rng(42)
    c.v[:] = c.v * np.ldexp(np.float32(1), rng.integers(-6, 7, size=D)).astype(np.float32)
    caches = DevCaches(B, Hq, Hkv, D, C, "i8k")
    caches.append(c.k, c.v, 0)
    got = caches.prefill(c.q, start, 1 / 16)
    vs = oracle.stored_values(c.v, "bf16")
    ref = oi8.prefill_chunk_i8(c.q, c.k, vs, start, 1 / 16)
    _check(got, ref, vs, "int8 prefill per-dim range")
    per_dim = np.abs(got - ref).max(axis=(0, 1, 2)) / np.abs(vs).max(axis=(0, 1, 2))
    assert per_dim.max() <= TOL, f"worst per-dim rel err {per_dim.max():.3e}"


def test_ragged_prefill():
    B, Hq, Hkv, D, C = 4, 8, 1, 256, 2048
    starts, rows = [0, 100, 1500, 7], [1, 0, 500, 64]
    c = random_case(50, B, Hq, Hkv, D, C, 1)
    caches = DevCaches(B, Hq, Hkv, D, C, "i8k")
    caches.append(c.k, c.v, 0)
    g = np.random.default_rng(51)
    q = g.standard_normal((sum(rows), Hq, D)).astype(np.float32)
    qt = dev(q)
    out = torch.full_like(qt, float("nan"))
    ws = caches.workspace(ka.prefill_ragged_workspace_bytes(caches.shape, sum(rows)))
    ka.prefill_ragged(caches.shape, qt, caches.k, caches.v, out, starts, rows, 1 / 16, ws)
    torch.cuda.synchronize()
    vs = oracle.stored_values(c.v, "bf16")
    qc, qs = oi8.quantize_rows(q)
    kc, ks = oi8.quantize_rows(c.k)
    ref, r0 = [], 0
    for b in range(B):
        if rows[b]:
            ref.append(oi8.attend_rows_i8(qc[r0:r0 + rows[b]], qs[r0:r0 + rows[b]], kc[b], ks[b], vs[b],
                                          np.arange(starts[b], starts[b] + rows[b]), 1 / 16))
            r0 += rows[b]
    _check(out.cpu().numpy(), np.concatenate(ref), vs, "int8 ragged prefill")


def test_nan_key_row_reaches_later_rows_only():
    """A NaN in K row start + 3: its scale is NaN, so every score against it
    is NaN: rows from position start + 3 on are NaN, earlier rows are not."""
    B, Hq, Hkv, D, C, start, R = 1, 8, 1, 256, 1024, 500, 64
    c = random_case(60, B, Hq, Hkv, D, start + R, R)
    c.k[0, start + 3, 0, 11] = np.nan
    caches = DevCaches(B, Hq, Hkv, D, C, "i8k")
    caches.append(c.k, c.v, 0)
    got = caches.prefill(c.q, start, 1 / 16)
    vs = oracle.stored_values(c.v, "bf16")
    ref = oi8.prefill_chunk_i8(c.q[:, :3], c.k, vs, start, 1 / 16)
    assert np.isfinite(got[:, :3]).all()
    assert oracle.rel_error(got[:, :3], ref, vs) <= TOL
    assert np.isnan(got[:, 3:]).all()


def test_resize_keeps_codes_and_scales():
    B, Hq, Hkv, D, C, n = 2, 4, 2, 64, 1024, 700
    c = random_case(70, B, Hq, Hkv, D, n, 16)
    a = DevCaches(B, Hq, Hkv, D, C, "i8k")
    a.append(c.k, c.v, 0)
    b = DevCaches(B, Hq, Hkv, D, 1472, "i8k")
    ka.cache_resize(a.shape, a.k, a.v, b.shape, b.k, b.v, n)
    ca_, sa_ = a.k_i8()
    cb_, sb_ = b.k_i8()
    assert np.array_equal(ca_[:, :, :n], cb_[:, :, :n])
    assert np.array_equal(sa_[:, :, :n], sb_[:, :, :n])
    assert np.array_equal(a.v_bits()[:, :, :n], b.v_bits()[:, :, :n])
    got = b.prefill(c.q, n - 16, 0.125)
    vs = oracle.stored_values(c.v, "bf16")
    ref = oi8.prefill_chunk_i8(c.q, c.k, vs, n - 16, 0.125)
    _check(got, ref, vs, "int8 prefill on a resized cache")
