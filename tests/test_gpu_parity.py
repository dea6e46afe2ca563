"""GPU parity of the three kernels against the CPU float64 oracle.

Every case: seeded synthetic inputs, caches pre-filled with NaN bytes (so a
read of a position that was never appended would poison the result), the
HIP path through the C ABI, and the oracle on the same inputs.

Tolerances (error = max |out - ref| / max |V stored|, over the whole case):
  f32 caches  1e-5   (f32 arithmetic throughout; the pages report 4.2e-7 for
                      their f32 parallel reduction against an f64 reference)
  bf16 caches 1e-2   (the oracle consumes the stored bf16 values; the GPU
                      additionally rounds q and the softmax weights to bf16
                      for its MFMA / dot2 operands)
bf16 storage itself is compared bit for bit.
"""
import math

import numpy as np
import pytest
import torch

import kv_cache_attention_amd as ka
import oracle
from oracle import bf16 as obf16
from synth import WORKLOADS, draw_batch, random_case
from tests.gpu_session import DevCaches

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

TOL = {"f32": 1e-5, "bf16": 1e-2}


def _print(*a):
    print(*a, flush=True)


def _stored(x, dt):
    return oracle.stored_values(x, dt)


def _check(got, ref, v_store, dt, what):
    err = oracle.rel_error(got, ref, v_store)
    _print(f"{what}: rel err {err:.3e} (tol {TOL[dt]:g})")
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    assert err <= TOL[dt], f"{what}: {err} > {TOL[dt]}"
    return err


# ------------------------------------------------------------------ append

@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_append_is_exact_and_touches_only_its_rows(dt):
    B, Hq, Hkv, D, C = 2, 4, 2, 64, 128
    c = random_case(7, B, Hq, Hkv, D, C, 1)
    c.k[0, 3, 1, 5] = np.nan
    c.v[1, 40, 0, 2] = -np.inf
    caches = DevCaches(B, Hq, Hkv, D, C, dt)
    done = np.zeros(C, bool)
    for s, e in [(0, 37), (37, 38), (38, 100), (100, 101), (120, 128)]:
        caches.append(c.k[:, s:e], c.v[:, s:e], s)
        done[s:e] = True
        kb, vb = caches.bits()                         # [B][Hkv][C][D]
        for name, got, src in (("k", kb, c.k), ("v", vb, c.v)):
            src_l = src.transpose(0, 2, 1, 3)          # [B][Hkv][P][D]
            if dt == "bf16":
                want = obf16.encode_rne(src_l[:, :, done])
                assert np.array_equal(got[:, :, done], want), name
                assert np.all(got[:, :, ~done] == 0xFFFF), name
                finite = np.isfinite(src_l[:, :, done])
                tb = torch.from_numpy(np.ascontiguousarray(src_l[:, :, done])).to(torch.bfloat16)
                tbits = tb.view(torch.int16).numpy().view(np.uint16)
                assert np.array_equal(got[:, :, done][finite], tbits[finite]), name
            else:
                g = got[:, :, done].view(np.uint32)
                w = np.ascontiguousarray(src_l[:, :, done]).view(np.uint32)
                assert np.array_equal(g, w), name
                assert np.all(got[:, :, ~done].view(np.uint32) == 0xFFFFFFFF), name


def test_append_full_chunk_long_session_shape():
    w = WORKLOADS[4]
    c = draw_batch(w, positions=1536, q_positions=[0])
    caches = DevCaches(1, 8, 1, 256, w.capacity, "bf16")
    caches.append(c.k[:, 768:1536], c.v[:, 768:1536], 768)
    kb, vb = caches.bits()
    assert np.array_equal(kb[0, 0, 768:1536], obf16.encode_rne(c.k[0, 768:1536, 0]))
    assert np.array_equal(vb[0, 0, 768:1536], obf16.encode_rne(c.v[0, 768:1536, 0]))
    assert np.all(kb[0, 0, :768] == 0xFFFF) and np.all(vb[0, 0, 1536:] == 0xFFFF)


# ----------------------------------------------------------------- prefill

def _prefill_case(dt, B, Hq, Hkv, D, C, start, R, seed, scale=None):
    P = start + R
    c = random_case(seed, B, Hq, Hkv, D, P, R)
    scale = scale if scale is not None else 1.0 / math.sqrt(D)
    caches = DevCaches(B, Hq, Hkv, D, C, dt)
    if start:
        caches.append(c.k[:, :start], c.v[:, :start], 0)
    caches.append(c.k[:, start:P], c.v[:, start:P], start)
    got = caches.prefill(c.q, start, scale)
    ks, vs = _stored(c.k, dt), _stored(c.v, dt)
    ref = oracle.prefill_chunk(c.q, ks, vs, start, scale)
    return got, ref, vs, c, caches


def test_prefill_tiny_workload():
    """128-row chunk at position 0, 2 query heads on 1 KV head, head_dim 64, f32."""
    w = WORKLOADS[1]
    c = draw_batch(w)
    caches = DevCaches(1, 2, 1, 64, w.capacity, "f32")
    caches.append(c.k, c.v, 0)
    got = caches.prefill(c.q, 0, w.scale)
    ref = oracle.prefill_chunk(c.q, c.k, c.v, 0, w.scale)
    _check(got, ref, c.v, "f32", "tiny prefill")
    # row 0 sees only key 0: its output is V[0] exactly
    assert np.array_equal(got[0, 0, 0], c.v[0, 0, 0]) and np.array_equal(got[0, 0, 1], c.v[0, 0, 0])


def test_prefill_chunked_workload_f32():
    """768-row chunk at positions 3072..3839 over 3072 cached rows, f32, all outputs."""
    w = WORKLOADS[3]
    c = draw_batch(w)
    caches = DevCaches(1, 8, 1, 256, w.capacity, "f32")
    caches.append(c.k[:, :3072], c.v[:, :3072], 0)
    caches.append(c.k[:, 3072:3840], c.v[:, 3072:3840], 3072)
    got = caches.prefill(c.q, 3072, w.scale)
    ref = oracle.prefill_chunk(c.q, c.k, c.v, 3072, w.scale)
    _check(got, ref, c.v, "f32", "chunked prefill 3072+768")


PREFILL_CASES = [
    # dt, B, Hq, Hkv, D, C, start, R
    ("f32", 1, 8, 1, 256, 256, 0, 1),
    ("bf16", 1, 8, 1, 256, 256, 0, 1),
    ("f32", 1, 8, 1, 256, 448, 100, 77),
    ("bf16", 1, 8, 1, 256, 448, 100, 77),
    ("bf16", 2, 8, 2, 128, 384, 37, 300),
    ("f32", 2, 6, 2, 64, 320, 5, 250),
    ("bf16", 1, 4, 4, 64, 192, 64, 64),
    ("bf16", 3, 2, 1, 64, 512, 300, 150),
    ("f32", 1, 16, 2, 128, 1024, 700, 129),
    ("bf16", 1, 8, 1, 256, 2048, 1500, 548),
]


@pytest.mark.parametrize("case", PREFILL_CASES, ids=lambda c: "-".join(map(str, c)))
def test_prefill_shapes(case):
    dt, B, Hq, Hkv, D, C, start, R = case
    got, ref, vs, _, _ = _prefill_case(dt, B, Hq, Hkv, D, C, start, R, seed=sum(case[1:]))
    _check(got, ref, vs, dt, f"prefill {case}")


def test_prefill_is_deterministic():
    got, ref, vs, c, caches = _prefill_case("bf16", 1, 8, 1, 256, 1024, 512, 400, seed=3)
    again = caches.prefill(c.q, 512, 1 / 16)
    assert np.array_equal(got.view(np.uint32), again.view(np.uint32))


def test_prefill_chunked_equals_single_shot():
    dt, B, Hq, Hkv, D, C = "bf16", 1, 8, 1, 128, 512
    c = random_case(9, B, Hq, Hkv, D, 448, 448)
    caches = DevCaches(B, Hq, Hkv, D, C, dt)
    caches.append(c.k, c.v, 0)
    one = caches.prefill(c.q, 0, 0.1)
    parts = [caches.prefill(c.q[:, s:s + r], s, 0.1) for s, r in [(0, 100), (100, 200), (300, 148)]]
    vs = _stored(c.v, dt)
    err = oracle.rel_error(np.concatenate(parts, axis=1), one, vs)
    assert err <= TOL[dt]


def test_prefill_nan_in_visible_key_poisons_later_rows_only():
    dt, B, Hq, Hkv, D, C = "f32", 1, 8, 1, 64, 192
    c = random_case(10, B, Hq, Hkv, D, 150, 150)
    c.k[0, 70, 0, 3] = np.nan
    caches = DevCaches(B, Hq, Hkv, D, C, dt)
    caches.append(c.k, c.v, 0)
    got = caches.prefill(c.q, 0, 0.125)
    ref = oracle.prefill_chunk(c.q, c.k, c.v, 0, 0.125)
    assert np.isnan(got[0, 70:]).all()
    assert np.isfinite(got[0, :70]).all()
    assert oracle.rel_error(got[0, :70], ref[0, :70], c.v) <= TOL[dt]


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_prefill_scores_far_above_the_first_tile(dt):
    """Queries share one direction u and the keys at odd 64-position tiles are
    3u, so those keys score about 40 (natural units) above every other key: a
    split that starts on an even tile meets scores far above its first tile's
    maximum (the bf16 kernel then redoes the split in a wider frame, the f32
    kernel rescales).  Every row that sees such keys averages their values."""
    B, Hq, Hkv, D, start, R = 1, 8, 1, 256, 1024, 128
    C = start + R + 64
    rng = np.random.default_rng(31)
    c = random_case(31, B, Hq, Hkv, D, start + R, R)
    u = rng.standard_normal(D).astype(np.float32)
    c.q[:] = u + np.float32(0.1) * c.q
    for t0 in range(64, start + R, 128):
        c.k[0, t0 + 17, 0] = 3 * u
    caches = DevCaches(B, Hq, Hkv, D, C, dt)
    caches.append(c.k[:, :start], c.v[:, :start], 0)
    caches.append(c.k[:, start:], c.v[:, start:], start)
    got = caches.prefill(c.q, start, 1 / 16)
    ks, vs = _stored(c.k, dt), _stored(c.v, dt)
    ref = oracle.prefill_chunk(c.q, ks, vs, start, 1 / 16)
    _check(got, ref, vs, dt, f"prefill far-above-first-tile {dt}")


def test_prefill_split_partials_per_dim_range():
    """Value dims scaled by 2^-6 .. 2^6 (a different power per dim), a chunk
    long enough to be split: every dim must keep its own relative accuracy
    through the split partials, not only accuracy relative to the largest
    dim (the bf16 kernel stores partials as binary16 with per-lane scales)."""
    B, Hq, Hkv, D, start, R = 1, 8, 1, 256, 2048, 256
    C = start + R
    c = random_case(41, B, Hq, Hkv, D, start + R, R)
    rng = np.random.default_rng(41)
    dim_scale = np.ldexp(np.float32(1), rng.integers(-6, 7, size=D)).astype(np.float32)
    c.v[:] = c.v * dim_scale
    caches = DevCaches(B, Hq, Hkv, D, C, "bf16")
    caches.append(c.k, c.v, 0)
    got = caches.prefill(c.q, start, 1 / 16)
    ks, vs = _stored(c.k, "bf16"), _stored(c.v, "bf16")
    ref = oracle.prefill_chunk(c.q, ks, vs, start, 1 / 16)
    _check(got, ref, vs, "bf16", "prefill per-dim range")
    per_dim_max = np.abs(vs).max(axis=(0, 1, 2))  # [D]
    per_dim_err = np.abs(got - ref).max(axis=(0, 1, 2)) / per_dim_max
    assert per_dim_err.max() <= TOL["bf16"], f"worst per-dim rel err {per_dim_err.max():.3e}"


# ------------------------------------------------------------------ decode

def _decode_case(dt, B, Hq, Hkv, D, C, ctxs, seed):
    P = max(ctxs)
    c = random_case(seed, B, Hq, Hkv, D, P, 1)
    caches = DevCaches(B, Hq, Hkv, D, C, dt)
    caches.append(c.k, c.v, 0)
    q = c.q[:, 0]
    got = caches.decode(q, ctxs, 1 / math.sqrt(D))
    ks, vs = _stored(c.k, dt), _stored(c.v, dt)
    ref = oracle.decode(q, ks, vs, ctxs, 1 / math.sqrt(D))
    return got, ref, vs, q, caches


DECODE_CASES = [
    ("f32", 1, 8, 1, 256, 64, [1]),
    ("bf16", 1, 8, 1, 256, 64, [1]),
    ("bf16", 1, 8, 1, 256, 64, [8]),
    ("bf16", 3, 8, 1, 256, 1088, [17, 1000, 1025]),
    ("f32", 3, 8, 1, 256, 1088, [15, 33, 1088]),
    ("bf16", 2, 16, 2, 128, 5120, [5000, 4097]),
    ("f32", 2, 4, 2, 64, 640, [31, 600]),
    ("bf16", 1, 6, 3, 64, 256, [200]),
    ("f32", 1, 1, 1, 128, 2048, [2047]),
    ("bf16", 2, 32, 4, 128, 128, [100, 128]),
    ("bf16", 1, 16, 1, 64, 256, [250]),
    ("f32", 1, 3, 1, 64, 128, [77]),
    # f32 plans by the step's size (8 heads: 2, 4 or 8 heads per workgroup)
    ("f32", 2, 8, 1, 128, 16448, [16385, 9000]),
    ("f32", 1, 8, 1, 64, 16448, [16385]),
    ("f32", 1, 1, 1, 64, 19264, [19200]),          # 300 splits: the merge's later batches
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=lambda c: "-".join(map(str, c[:6])) + "-" + "_".join(map(str, c[6])))
def test_decode_shapes(case):
    dt, B, Hq, Hkv, D, C, ctxs = case
    got, ref, vs, _, _ = _decode_case(dt, B, Hq, Hkv, D, C, ctxs, seed=11 + B + D)
    _check(got, ref, vs, dt, f"decode {case}")


def test_decode_workload_f32():
    """One query row at position 4096 over the 4096 cached rows, f32."""
    w = WORKLOADS[2]
    c = draw_batch(w)
    caches = DevCaches(1, 8, 1, 256, w.capacity, "f32")
    caches.append(c.k[:, :4096], c.v[:, :4096], 0)
    caches.append(c.k[:, 4096:4097], c.v[:, 4096:4097], 4096)
    got = caches.decode(c.q[:, 0], [4097], w.scale)
    ref = oracle.decode(c.q[:, 0], c.k, c.v, [4097], w.scale)
    _check(got, ref, c.v, "f32", "decode 4097 f32")


def test_decode_equals_prefill_row():
    dt, B, Hq, Hkv, D, C = "f32", 1, 8, 1, 256, 640
    c = random_case(12, B, Hq, Hkv, D, 600, 600)
    caches = DevCaches(B, Hq, Hkv, D, C, dt)
    caches.append(c.k, c.v, 0)
    full = caches.prefill(c.q, 0, 1 / 16)
    for t in [0, 63, 64, 599]:
        d = caches.decode(c.q[:, t], [t + 1], 1 / 16)
        assert oracle.rel_error(d, full[:, t], c.v) <= TOL[dt]


def test_decode_is_deterministic_and_nan_safe():
    got, ref, vs, q, caches = _decode_case("bf16", 2, 8, 1, 256, 4096, [4000, 2500], seed=13)
    again = caches.decode(q, [4000, 2500], 1 / 16)
    assert np.array_equal(got.view(np.uint32), again.view(np.uint32))


def test_decode_nan_value_reaches_only_its_dimension():
    """A NaN value at (position 200, dim 7): every head's dim 7 turns NaN once
    position 200 is visible; the other dims, and every dim before, match."""
    dt, B, Hq, Hkv, D, C = "bf16", 1, 8, 1, 128, 512
    c = random_case(14, B, Hq, Hkv, D, 500, 1)
    c.v[0, 200, 0, 7] = np.nan
    caches = DevCaches(B, Hq, Hkv, D, C, dt)
    caches.append(c.k, c.v, 0)
    q = c.q[:, 0]
    ks, vs = _stored(c.k, dt), _stored(c.v, dt)
    for ctx in (200, 201, 500):
        out = caches.decode(q, [ctx], 0.1)
        ref = oracle.decode(q, ks, vs, [ctx], 0.1)
        assert np.array_equal(np.isnan(out), np.isnan(ref))
        assert np.isnan(out[..., 7]).all() == (ctx > 200)
        fin = ~np.isnan(ref)
        assert oracle.rel_error(out[fin], ref[fin], vs[:, :200]) <= TOL[dt]


DECODE_STEP_CASES = [
    # dt, B, Hq, Hkv, D, C, per-session positions of the new row
    ("bf16", 1, 8, 1, 256, 4160, [4096]),
    ("bf16", 3, 16, 1, 128, 640, [0, 31, 600]),
    ("bf16", 2, 3, 1, 64, 192, [32, 63]),
    ("bf16", 2, 8, 2, 256, 1024, [64, 1000]),
    ("f32", 2, 8, 1, 128, 512, [5, 300]),
    ("f32", 1, 4, 2, 64, 128, [0]),
    ("f32", 3, 16, 1, 256, 1088, [0, 517, 1087]),  # two head groups per KV head
    ("f32", 2, 8, 2, 256, 4160, [4096, 33]),
    ("f32", 1, 8, 1, 64, 40000, [39000]),          # all heads per workgroup, 512 splits
    ("f32", 2, 8, 1, 64, 512, [7, 298]),           # new row in slots 3 and 2 of its V group
    ("f32", 1, 8, 1, 256, 4160, [4096]),           # two heads per workgroup
]


@pytest.mark.parametrize("case", DECODE_STEP_CASES,
                         ids=lambda c: "-".join(map(str, c[:6])) + "-" + "_".join(map(str, c[6])))
def test_decode_step_appends_then_decodes(case):
    """ka_attn_decode_step: the new rows land in the cache bit for bit as
    appended rows would, the output matches the oracle, and it is bitwise the
    output of a plain decode of the cache it leaves behind."""
    dt, B, Hq, Hkv, D, C, pos = case
    P = max(pos) + 1
    c = random_case(sum(pos) + D, B, Hq, Hkv, D, P, 1)
    rng = np.random.default_rng(7 + B)
    k_new = rng.standard_normal((B, Hkv, D), dtype=np.float32)
    v_new = rng.standard_normal((B, Hkv, D), dtype=np.float32)
    q = c.q[:, 0]                                      # [B][Hq][D]
    caches = DevCaches(B, Hq, Hkv, D, C, dt)
    caches.append(c.k, c.v, 0)                         # rows 0 .. P-1 (new rows overwrite)
    got = caches.decode_step(q, k_new, v_new, pos, 0.0625)
    # the cache as an append of the new rows would leave it
    k_all, v_all = c.k.copy(), c.v.copy()
    for b, p in enumerate(pos):
        k_all[b, p], v_all[b, p] = k_new[b], v_new[b]
    kb, vb = caches.bits()                             # [B][Hkv][C][D]
    for b, p in enumerate(pos):
        for name, got_bits, src in (("k", kb, k_all), ("v", vb, v_all)):
            row = src[b, p]                            # [Hkv][D]
            if dt == "bf16":
                assert np.array_equal(got_bits[b, :, p], obf16.encode_rne(row)), (name, b)
            else:
                assert np.array_equal(got_bits[b, :, p].view(np.uint32), row.view(np.uint32)), (name, b)
    # oracle: each session's row at its position, over its own context
    ks, vs = _stored(k_all, dt), _stored(v_all, dt)
    for b, p in enumerate(pos):
        ref = oracle.decode(q[b:b + 1], ks[b:b + 1, :p + 1], vs[b:b + 1, :p + 1], [p + 1], 0.0625)
        _check(got[b:b + 1], ref, vs[b:b + 1, :p + 1], dt, f"decode step {case} session {b}")
    again = caches.decode(q, [p + 1 for p in pos], 0.0625)
    assert np.array_equal(got.view(np.uint32), again.view(np.uint32))


def test_rejected_call_leaves_output_untouched():
    caches = DevCaches(1, 8, 1, 256, 4096, ka.BF16)
    q = torch.zeros(8 * 256, device="cuda")
    out = torch.full((8 * 256,), 3.0, device="cuda")
    with pytest.raises(ka.KaAttnError) as e:
        ka.decode(caches.shape, q, caches.k, caches.v, out, [4096], 0.1, None)
    assert e.value.status == 4
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)
