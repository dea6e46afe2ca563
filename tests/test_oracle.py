"""Pins of the CPU oracle against facts fixed outside the oracle itself.

Each test checks the oracle against something it does not compute itself:
closed forms, limits, a second independent implementation (scalar brute
force, torch's float64 scaled-dot-product attention), invariants of causal
attention, and hand-derived bfloat16 rounding cases.  Each is chosen so that a
plausible slip in the oracle (a dropped scale, an off-by-one in the causal
limit, the wrong KV head, a transposed operand, a max that drops NaN) fails.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import bf16
from synth import WORKLOADS, draw_batch, random_case

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(seed, n, Hq, Hkv, D, P=None):
    c = random_case(seed, 1, Hq, Hkv, D, P if P is not None else n, n)
    return c.q[0], c.k[0], c.v[0]


# ---------------------------------------------------------------- closed forms

def test_first_row_is_first_value_row_exactly():
    """Row 0 of a chunk at position 0 sees only key 0: softmax weight 1."""
    q, k, v = _rand(11, 7, 4, 2, 16)
    o = oracle.attend_rows(q, k, v, np.arange(7), 0.25)
    for h in range(4):
        g = oracle.kv_group(h, 4, 2)
        assert np.array_equal(o[0, h], v[0, g].astype(np.float64))


def test_equal_scores_give_mean_of_visible_values():
    """q = 0 makes every visible score 0, so o is the plain mean of V rows."""
    _, k, v = _rand(12, 40, 2, 1, 32)
    q = np.zeros((40, 2, 32), np.float32)
    o = oracle.attend_rows(q, k, v, np.arange(40), 0.125)
    for i in [0, 1, 5, 39]:
        mean = np.array([math.fsum(v[:i + 1, 0, d].astype(np.float64)) / (i + 1)
                         for d in range(32)])
        np.testing.assert_allclose(o[i, 0], mean, rtol=0, atol=1e-14)
        np.testing.assert_allclose(o[i, 1], mean, rtol=0, atol=1e-14)


def test_identical_key_rows_give_mean_of_values():
    """Every visible K row identical: equal scores whatever q is."""
    q, k, v = _rand(13, 20, 2, 1, 8)
    k[:] = k[3]
    o = oracle.attend_rows(q, k, v, np.arange(20), 0.5)
    np.testing.assert_allclose(o[19, 1], v[:, 0].astype(np.float64).mean(axis=0),
                               rtol=0, atol=1e-14)


def test_two_keys_logistic_weight():
    """Two visible keys: o = sigma(s0 - s1) v0 + (1 - sigma) v1.

    q and k are axis-aligned so the scores are scale * a * b_j with no
    rounding: with a = 2, scale = 0.5, b0 = ln 3 (as f32), b1 = 0 the weight
    of key 0 is 3/4 up to the f32 rounding of ln 3.
    """
    D = 8
    q = np.zeros((2, 1, D), np.float32)
    k = np.zeros((2, 1, D), np.float32)
    q[1, 0, 0] = 2.0
    k[0, 0, 0] = np.float32(math.log(3.0))
    v = np.zeros((2, 1, D), np.float32)
    v[0, 0] = np.arange(D, dtype=np.float32)
    v[1, 0] = -1.0
    o = oracle.attend_rows(q, k, v, [0, 1], 0.5)
    gap = 0.5 * 2.0 * float(k[0, 0, 0])
    w0 = 1.0 / (1.0 + math.exp(-gap))
    expect = w0 * v[0, 0].astype(np.float64) + (1 - w0) * v[1, 0].astype(np.float64)
    np.testing.assert_allclose(o[1, 0], expect, rtol=0, atol=1e-15)
    assert abs(w0 - 0.75) < 1e-7


def test_dominant_key_limit():
    """A key whose score leads every other by >= 50 takes weight 1 - O(e^-50)."""
    q, k, v = _rand(14, 30, 1, 1, 16)
    q[29, 0] = 0.0
    q[29, 0, 0] = 1.0
    k[:, 0, 0] = 0.0
    k[17, 0, 0] = 400.0               # scale 0.125 -> score 50 vs 0
    o = oracle.attend_rows(q, k, v, np.arange(30), 0.125)
    err = np.abs(o[29, 0] - v[17, 0]).max()
    assert err <= 30 * math.exp(-50.0) * np.abs(v).max()


def test_scale_is_applied_to_scores():
    """Doubling the scale equals doubling q (a dropped scale fails this)."""
    q, k, v = _rand(15, 12, 2, 1, 16)
    a = oracle.attend_rows(q, k, v, np.arange(12), 0.5)
    b = oracle.attend_rows(q * 2, k, v, np.arange(12), 0.25)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-14)
    c = oracle.attend_rows(q, k, v, np.arange(12), 0.25)
    assert np.abs(a - c).max() > 1e-3


# ------------------------------------------------------- independent routines

def test_scalar_brute_force_matches_numpy_on_tiny_workload():
    """The 128-row tiny prefill (2 heads, head_dim 64): two implementations."""
    w = WORKLOADS[1]
    c = draw_batch(w)
    ks = oracle.stored_values(c.k[0], "f32")
    vs = oracle.stored_values(c.v[0], "f32")
    rows = list(range(0, 8)) + [63, 64, 127]
    ref = oracle.attend_rows(c.q[0], ks, vs, np.arange(128), w.scale)
    sc = oracle.attend_rows_scalar(c.q[0][rows], ks, vs, rows, w.scale)
    np.testing.assert_allclose(np.array(sc), ref[rows], rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("seed", range(6))
def test_scalar_matches_numpy_random_shapes(seed):
    g = np.random.default_rng(seed)
    Hkv = int(g.integers(1, 3))
    G = int(g.integers(1, 4))
    D = int(g.choice([1, 3, 8, 16]))
    n = int(g.integers(1, 9))
    start = int(g.integers(0, 6))
    q, k, v = _rand(100 + seed, n, Hkv * G, Hkv, D, P=start + n)
    pos = np.arange(start, start + n)
    ref = oracle.attend_rows(q, k, v, pos, 0.3, row_block=3)
    sc = np.array(oracle.attend_rows_scalar(q, k, v, pos, 0.3))
    np.testing.assert_allclose(sc, ref, rtol=1e-12, atol=1e-13)


def _torch_sdpa_f64(q, k, v, pos, scale, G):
    """torch's float64 SDPA with an explicit boolean mask (row i sees j <= pos[i])."""
    qt = torch.from_numpy(q.astype(np.float64)).permute(1, 0, 2)          # [Hq][n][D]
    kt = torch.from_numpy(k.astype(np.float64)).permute(1, 0, 2)          # [Hkv][P][D]
    vt = torch.from_numpy(v.astype(np.float64)).permute(1, 0, 2)
    kt = kt.repeat_interleave(G, dim=0).contiguous()
    vt = vt.repeat_interleave(G, dim=0).contiguous()
    P = k.shape[0]
    mask = torch.arange(P)[None, :] <= torch.from_numpy(np.asarray(pos))[:, None]
    o = torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, attn_mask=mask, scale=float(np.float32(scale)))
    return o.permute(1, 0, 2).numpy()


def test_matches_torch_sdpa_tiny_workload():
    w = WORKLOADS[1]
    c = draw_batch(w)
    ref = oracle.attend_rows(c.q[0], c.k[0], c.v[0], np.arange(128), w.scale)
    t = _torch_sdpa_f64(c.q[0], c.k[0], c.v[0], np.arange(128), w.scale, 2)
    np.testing.assert_allclose(ref, t, rtol=0, atol=1e-12)


def test_matches_torch_sdpa_gqa_chunk_with_history():
    """A 96-row chunk at start 160 over 2 KV heads x 3 query heads each."""
    q, k, v = _rand(21, 96, 6, 2, 32, P=256)
    pos = np.arange(160, 256)
    ref = oracle.attend_rows(q, k, v, pos, 0.2, row_block=40)
    t = _torch_sdpa_f64(q, k, v, pos, 0.2, 3)
    np.testing.assert_allclose(ref, t, rtol=0, atol=1e-12)


@pytest.mark.slow
def test_matches_torch_sdpa_chunked_prefill_workload():
    """The 768-row chunk at position 3072 (8 heads, head_dim 256), sampled rows."""
    w = WORKLOADS[3]
    c = draw_batch(w)
    rows = np.r_[0:64, 700:768]
    pos = 3072 + rows
    ref = oracle.attend_rows(c.q[0][rows], c.k[0], c.v[0], pos, w.scale)
    t = _torch_sdpa_f64(c.q[0][rows], c.k[0][:3840], c.v[0][:3840], pos, w.scale, 8)
    np.testing.assert_allclose(ref, t, rtol=0, atol=1e-12)


# ----------------------------------------------------------------- invariants

def test_causality_later_rows_do_not_leak():
    q, k, v = _rand(31, 24, 4, 1, 16)
    base = oracle.attend_rows(q, k, v, np.arange(24), 0.3)
    k2, v2 = k.copy(), v.copy()
    k2[11:] = 1e3 * np.random.default_rng(0).standard_normal(k2[11:].shape)
    v2[11:] = np.nan
    o = oracle.attend_rows(q, k2, v2, np.arange(24), 0.3)
    assert np.array_equal(o[:11], base[:11])
    assert np.isnan(o[11:]).all()


def test_gqa_head_to_group_map():
    """With 2 KV heads x 3 query heads each, heads 3..5 read KV head 1 only."""
    q, k, v = _rand(32, 10, 6, 2, 8)
    v[:, 1, :] = 0.5
    o = oracle.attend_rows(q, k, v, np.arange(10), 0.4)
    # weights sum to 1: a constant V row set gives that constant (to rounding)
    np.testing.assert_allclose(o[:, 3:6, :], 0.5, rtol=0, atol=1e-15)
    assert not np.any(np.isclose(o[1:, 0:3, :], 0.5))
    # a wrong map (h % Hkv, say) would send head 1 to KV head 1
    v2 = v.copy()
    v2[:, 0, :] = 7.0
    o2 = oracle.attend_rows(q, k, v2, np.arange(10), 0.4)
    np.testing.assert_allclose(o2[:, 0:3, :], 7.0, rtol=0, atol=1e-14)
    np.testing.assert_allclose(o2[:, 3:6, :], 0.5, rtol=0, atol=1e-15)


def test_chunked_equals_single_shot():
    q, k, v = _rand(33, 200, 4, 1, 16)
    one = oracle.attend_rows(q, k, v, np.arange(200), 0.25)
    parts = []
    for s, r in [(0, 64), (64, 64), (128, 50), (178, 22)]:
        parts.append(oracle.prefill_chunk(q[None, s:s + r], k[None], v[None], s, 0.25)[0])
    np.testing.assert_allclose(np.concatenate(parts), one, rtol=0, atol=1e-14)


def test_decode_equals_prefill_row():
    q, k, v = _rand(34, 70, 4, 2, 16)
    full = oracle.attend_rows(q, k, v, np.arange(70), 0.25)
    for t in [0, 1, 33, 69]:
        d = oracle.decode(q[None, t], k[None], v[None], [t + 1], 0.25)[0]
        np.testing.assert_allclose(d, full[t], rtol=0, atol=1e-14)


def test_joint_permutation_of_visible_keys():
    q, k, v = _rand(35, 16, 2, 1, 8)
    perm = np.random.default_rng(3).permutation(16)
    a = oracle.attend_rows(q[15:16], k, v, [15], 0.5)
    b = oracle.attend_rows(q[15:16], k[perm], v[perm], [15], 0.5)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-14)


# ------------------------------------------------------------- NaN and masking

def test_nan_in_visible_key_makes_row_nan_only_from_there_on():
    q, k, v = _rand(41, 12, 2, 1, 8)
    k[5, 0, 3] = np.nan
    o = oracle.attend_rows(q, k, v, np.arange(12), 0.5)
    assert np.isfinite(o[:5]).all()
    assert np.isnan(o[5:]).all()


def test_nan_query_row_gives_nan_row():
    q, k, v = _rand(42, 6, 2, 1, 8)
    q[4, 1, 0] = np.nan
    o = oracle.attend_rows(q, k, v, np.arange(6), 0.5)
    assert np.isnan(o[4, 1]).all() and np.isfinite(o[4, 0]).all()


def test_all_nan_scores_give_nan_not_zero():
    q, k, v = _rand(43, 4, 1, 1, 8)
    k[:] = np.nan
    o = oracle.attend_rows(q, k, v, np.arange(4), 0.5)
    assert np.isnan(o).all()


def test_row_without_visible_key_is_exactly_zero():
    q, k, v = _rand(44, 3, 1, 1, 8)
    o = oracle.attend_rows(q[:1], k, v, [-1], 0.5)
    assert np.array_equal(o, np.zeros_like(o))


def test_rel_error_measure():
    v = np.array([[1.0, -4.0]])
    assert oracle.rel_error([0.5, 1.0], [0.5, 0.0], v) == 0.25


# ------------------------------------------------------------------- bfloat16

def _golden_rne():
    rows = []
    with open(os.path.join(GOLDEN, "bf16_rne.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            a, b = line.split()[:2]
            rows.append((int(a, 16), int(b, 16)))
    return rows


def test_bf16_rne_golden_cases():
    rows = _golden_rne()
    assert len(rows) >= 20
    src = np.array([a for a, _ in rows], dtype=np.uint32).view(np.float32)
    got = bf16.encode_rne(src)
    assert [int(x) for x in got] == [b for _, b in rows]


def test_bf16_rne_matches_torch_cpu_conversion():
    g = np.random.default_rng(5)
    x = np.concatenate([
        g.standard_normal(200000).astype(np.float32) * 3,
        (g.integers(0, 2**32, 200000, dtype=np.uint64).astype(np.uint32)).view(np.float32),
        np.array([0.0, -0.0, np.inf, -np.inf, 3.4028235e38, 1e-45, 1.17549435e-38], np.float32),
    ])
    finite_or_inf = ~np.isnan(x)
    ours = bf16.encode_rne(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours[finite_or_inf], theirs[finite_or_inf])
    # NaN stays NaN in both
    dec = bf16.decode(ours)
    assert np.isnan(dec[~finite_or_inf]).all()


def test_bf16_round_trip_is_exact_on_representable_values():
    bits = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    vals = bf16.decode(bits)
    back = bf16.encode_rne(vals)
    finite = ~np.isnan(vals)
    assert np.array_equal(back[finite], bits[finite])


def test_stored_values_bf16_error_bound():
    """RNE error is at most half a unit in the last place: 8 significant
    bits, so |x - bf16(x)| <= 2^(e-8) where 2^e <= |x| < 2^(e+1)."""
    x = np.random.default_rng(6).standard_normal(10000).astype(np.float32)
    s = oracle.stored_values(x, "bf16").astype(np.float64)
    e = np.floor(np.log2(np.abs(x.astype(np.float64))))
    assert np.all(np.abs(s - x) <= 2.0 ** (e - 8))
    # and truncation would break it somewhere: the bound is tight enough to see
    trunc = (x.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32).astype(np.float64)
    assert np.any(np.abs(trunc - x) > 2.0 ** (e - 8))


# ------------------------------------------------------------------- workloads

def test_workload_recipes():
    w4, w5 = WORKLOADS[4], WORKLOADS[5]
    assert sum(r for _, r in w4.chunks) == 16384 and len(w4.chunks) == 22
    assert w4.decode_positions[0] == 16384 and len(w4.decode_positions) == 64
    assert w4.capacity >= w4.positions and w4.capacity % 64 == 0
    assert w5.decode_positions[-1] + 1 == 131072 == w5.capacity
    assert WORKLOADS[2].decode_positions == (4096,)
    for w in WORKLOADS.values():
        assert w.capacity % 64 == 0 and w.positions <= w.capacity


def test_outlier_rows_are_drawn_without_replacement():
    w = WORKLOADS[5]
    from synth import draw_session
    c = draw_session(w, 1, positions=4096)
    assert len(np.unique(c.outlier_idx)) == c.outlier_idx.size


# ------------------------------------------------------------------- rotary

def test_rope_identity_and_quarter_turn_exact():
    """cos 1 / sin 0 leaves rows unchanged; cos 0 / sin 1 turns each pair
    (x[d], x[d + D/2]) by a quarter: (-x[d + D/2], x[d]).  Worked by hand for
    D = 4, pairs (0, 2) and (1, 3): [1, 2, 3, 4] with the first pair turned
    and the second left alone gives [-3, 2, 1, 4]."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, 2, 8)).astype(np.float32)
    one, zero = np.ones((5, 4), np.float32), np.zeros((5, 4), np.float32)
    assert np.array_equal(oracle.rope.rotate_half_f32(x, one, zero), x)
    turned = oracle.rope.rotate_half_f32(x, zero, one)
    assert np.array_equal(turned[..., :4], -x[..., 4:]) and np.array_equal(turned[..., 4:], x[..., :4])
    y = oracle.rope.rotate_half_f32(np.array([[[1, 2, 3, 4]]], np.float32),
                                    np.array([[0, 1]], np.float32), np.array([[1, 0]], np.float32))
    assert y.tolist() == [[[-3.0, 2.0, 1.0, 4.0]]]


def test_rope_f32_within_rounding_of_complex_f64():
    """The f32 evaluation (two rounded products, one rounded sum) stays within
    1.5 units in the last place of the larger product of the complex-number
    statement in float64."""
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((64, 3, 256)) * 10).astype(np.float32)
    cos, sin = oracle.rope.angles_table(np.arange(1000, 1064), 256)
    got = oracle.rope.rotate_half_f32(x, cos, sin).astype(np.float64)
    ref = oracle.rope.rotate_half_f64(x, cos, sin)
    h = 128
    a, b = x[..., :h].astype(np.float64), x[..., h:].astype(np.float64)
    c, s = cos[:, None, :].astype(np.float64), sin[:, None, :].astype(np.float64)
    mag = np.concatenate([np.maximum(abs(a * c), abs(b * s)), np.maximum(abs(b * c), abs(a * s))], -1)
    assert np.all(np.abs(got - ref) <= 1.5 * 2.0 ** -23 * 2 * mag + 1e-30)


def test_rope_dot_products_depend_only_on_position_difference():
    """With angles p * w (the usual table), <rope(q, m), rope(k, n)> depends
    on m - n only: shifting both positions by t leaves it unchanged, and a
    lag of zero gives the plain dot product (float64)."""
    rng = np.random.default_rng(5)
    q = rng.standard_normal((1, 1, 64))
    k = rng.standard_normal((1, 1, 64))
    def dot(m, n):
        # float64 tables of the angles p * w
        pm = np.asarray([m], float)[:, None] * 10000.0 ** (-np.arange(32) * 2.0 / 64)
        pn = np.asarray([n], float)[:, None] * 10000.0 ** (-np.arange(32) * 2.0 / 64)
        a = oracle.rope.rotate_half_f64(q, np.cos(pm), np.sin(pm))
        b = oracle.rope.rotate_half_f64(k, np.cos(pn), np.sin(pn))
        return float(np.sum(a * b))
    base = dot(37, 5)
    for t in (1, 100, 4096):
        assert abs(dot(37 + t, 5 + t) - base) <= 1e-9 * (1 + abs(base))
    assert abs(dot(9, 9) - float(np.sum(q * k))) <= 1e-12 * (1 + abs(base))
    # and rotation keeps the norm of every pair
    p = 123.0 * 10000.0 ** (-np.arange(32) * 2.0 / 64)
    r = oracle.rope.rotate_half_f64(q, np.cos(p)[None], np.sin(p)[None])
    assert np.allclose(r[..., :32] ** 2 + r[..., 32:] ** 2, q[..., :32] ** 2 + q[..., 32:] ** 2, rtol=1e-12)


# ---------------------------------------------------------------- ragged batches

def test_ragged_matches_scalar_brute_force_per_session():
    """Three sessions at different positions, one of them empty, packed rows:
    each session's rows equal the scalar brute force on that session's own
    cache (a slip in the row packing or the session-to-cache map fails)."""
    B, Hq, Hkv, D, P = 3, 4, 2, 8, 12
    g = np.random.default_rng(5)
    k = g.standard_normal((B, P, Hkv, D)).astype(np.float32)
    v = g.standard_normal((B, P, Hkv, D)).astype(np.float32)
    starts, rows = [4, 0, 7], [3, 0, 5]
    q = g.standard_normal((sum(rows), Hq, D)).astype(np.float32)
    got = oracle.prefill_ragged(q, k, v, starts, rows, 0.4)
    assert got.shape == (8, Hq, D)
    want0 = oracle.attend_rows_scalar(q[:3], k[0], v[0], [4, 5, 6], 0.4)
    want2 = oracle.attend_rows_scalar(q[3:], k[2], v[2], [7, 8, 9, 10, 11], 0.4)
    np.testing.assert_allclose(got[:3], np.array(want0), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(got[3:], np.array(want2), rtol=1e-12, atol=1e-13)


def test_ragged_with_equal_sessions_is_the_uniform_chunk():
    B, Hq, Hkv, D, start, R = 2, 4, 1, 16, 6, 5
    c = random_case(21, B, Hq, Hkv, D, start + R, R)
    uni = oracle.prefill_chunk(c.q, c.k, c.v, start, 0.25)
    rag = oracle.prefill_ragged(c.q.reshape(B * R, Hq, D), c.k, c.v, [start] * B, [R] * B, 0.25)
    np.testing.assert_array_equal(rag, uni.reshape(B * R, Hq, D))
    assert oracle.prefill_ragged(c.q[0, :0], c.k, c.v, [0, 0], [0, 0], 0.25).shape == (0, Hq, D)


# ---------------------------------------------------------------- int8 scores

from oracle import int8 as oi8  # noqa: E402


def test_int8_quantisation_hand_cases():
    """Worked by hand: amax 1 gives s = f32(1/127) (bits 0x3C010204); 0.5 / s
    is 63.50000024 exactly, which is 63.5 in f32, a tie that goes to the even
    code 64; 0.25 / s is 31.75 -> 32; amax maps to 127.  A zero row keeps s = 0
    and codes 0; a row with NaN gets s = NaN, one with an infinity s = inf,
    both with codes 0 (their scores then come out NaN)."""
    x = np.array([[1.0, -0.5, 0.25, 0.0], [0, 0, 0, 0], [1, np.nan, 2, 3], [1, np.inf, 0, 0]],
                 np.float32)
    c, s = oi8.quantize_rows(x)
    assert c.dtype == np.int8
    assert c[0].tolist() == [127, -64, 32, 0]
    assert s[0].view(np.uint32) == 0x3C010204
    assert c[1].tolist() == [0, 0, 0, 0] and s[1] == 0
    assert c[2].tolist() == [0, 0, 0, 0] and np.isnan(s[2])
    assert c[3].tolist() == [0, 0, 0, 0] and np.isinf(s[3])


def test_int8_quantisation_bounds():
    """Random rows: codes in -127 .. 127, the largest |x| maps to +-127 with
    its sign, and every value is within half a step of code * s (plus the
    f32 rounding of x / s)."""
    g = np.random.default_rng(11)
    x = (g.standard_normal((64, 256)) * np.exp(g.uniform(-8, 8, size=(64, 1)))).astype(np.float32)
    c, s = oi8.quantize_rows(x)
    assert np.abs(c.astype(int)).max() <= 127
    i = np.abs(x).argmax(axis=1)
    assert (c[np.arange(64), i].astype(int) == 127 * np.sign(x[np.arange(64), i])).all()
    err = np.abs(x.astype(np.float64) - oi8.dequantize(c, s))
    assert (err <= s[:, None].astype(np.float64) * (0.5 + 2 ** -16)).all()


def test_int8_attention_is_exact_attention_when_quantisation_is_lossless():
    """Rows that are integer codes (largest |code| 127) times a power of two
    quantise back to exactly those codes with s = that power of two (127 *
    f32(1/127) rounds to 1 in f32), so the int8 scores are the exact scores
    and the int8 attention equals the float64 attention: a dropped or doubled
    scale factor, or a transposed code matrix, fails here."""
    g = np.random.default_rng(12)
    Hq, Hkv, D, P, n = 4, 2, 64, 40, 6

    def rows(shape, e):
        c = g.integers(-127, 128, size=shape + (D,)).astype(np.float32)
        c[..., 0] = 127 * np.where(g.random(shape) < 0.5, -1, 1)
        return (c * np.float32(2.0 ** e)).astype(np.float32)

    q = rows((n, Hq), -9)
    k = rows((P, Hkv), -7)
    v = g.standard_normal((P, Hkv, D)).astype(np.float32)
    qc, qs = oi8.quantize_rows(q)
    kc, ks = oi8.quantize_rows(k)
    assert (qs == np.float32(2.0 ** -9)).all() and (ks == np.float32(2.0 ** -7)).all()
    np.testing.assert_array_equal(oi8.dequantize(qc, qs), q.astype(np.float64))
    pos = np.arange(P - n, P)
    want = oracle.attend_rows(q, k, v, pos, 0.5)
    got = oi8.attend_rows_i8(qc, qs, kc, ks, v, pos, 0.5)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_int8_scores_match_integer_brute_force():
    """One row, tiny sizes: the scores from Python integers and the scales
    (the scale enters as its f32 value, as everywhere in the oracle)."""
    g = np.random.default_rng(13)
    q = g.standard_normal((1, 2, 8)).astype(np.float32)
    k = g.standard_normal((5, 1, 8)).astype(np.float32)
    v = np.eye(5, 8, dtype=np.float32)[:, None, :]            # value row j = e_j
    qc, qs = oi8.quantize_rows(q)
    kc, ks = oi8.quantize_rows(k)
    out = oi8.attend_rows_i8(qc, qs, kc, ks, v, [4], 0.3)
    for h in range(2):
        s = [float(np.float32(0.3)) * sum(int(a) * int(b) for a, b in zip(qc[0, h], kc[j, 0])) *
             float(qs[0, h]) *
             float(ks[j, 0]) for j in range(5)]
        m = max(s)
        w = [math.exp(t - m) for t in s]
        np.testing.assert_allclose(out[0, h, :5], np.array(w) / sum(w), rtol=1e-12)


def _lossless_rows(g, shape, D, e):
    """Rows of integer codes (largest |code| exactly 127) times 2**e: they
    quantise back to themselves with s = 2**e."""
    c = g.integers(-127, 128, size=shape + (D,)).astype(np.float32)
    c[..., 0] = 127 * np.where(g.random(shape) < 0.5, -1, 1)
    return (c * np.float32(2.0 ** e)).astype(np.float32)


@pytest.mark.parametrize("bad", [np.nan, np.inf, -np.inf])
def test_int8_nonfinite_value_reaches_only_rows_that_see_it(bad):
    """Causality (an output row does not change with keys after its
    position) with a non-finite V value inside a row block: the rows before
    the bad position equal those computed without it, and
    blocking the rows one at a time gives the default block's result (to
    rounding: the products may sum in another order).  A block product with
    zero weights (0 * NaN = NaN) fails here."""
    g = np.random.default_rng(14)
    Hq, Hkv, D, n = 4, 2, 32, 24
    q = g.standard_normal((n, Hq, D)).astype(np.float32)
    k = g.standard_normal((n, Hkv, D)).astype(np.float32)
    v = g.standard_normal((n, Hkv, D)).astype(np.float32)
    qc, qs = oi8.quantize_rows(q)
    kc, ks = oi8.quantize_rows(k)
    j = 15
    vb = v.copy()
    vb[j, 1, 9] = bad
    pos = np.arange(n)
    clean = oi8.attend_rows_i8(qc, qs, kc, ks, v, pos, 0.2)
    got = oi8.attend_rows_i8(qc, qs, kc, ks, vb, pos, 0.2)
    one = oi8.attend_rows_i8(qc, qs, kc, ks, vb, pos, 0.2, row_block=1)
    # (the matrix products may sum in another order: equal to rounding)
    np.testing.assert_allclose(got, one, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(got[:j], clean[:j], rtol=1e-13, atol=1e-13)
    assert np.isfinite(got[:j]).all()
    # rows at j and after see the bad value in exactly that dim of the heads of KV head 1
    assert (~np.isfinite(got[j:, 2:, 9])).all()
    other = np.ones(got.shape, bool)
    other[j:, 2:, 9] = False
    assert np.isfinite(got[other]).all()


def test_int8_chunk_and_decode_wrappers_on_lossless_inputs():
    """prefill_chunk_i8 and decode_i8 quantise their own inputs and place the
    rows.  On losslessly quantisable inputs their results are plain
    attention's, which is pinned above against torch's float64 attention:
    an error in the chunk's start offset, or in decode's ctx - 1 position,
    fails here."""
    g = np.random.default_rng(15)
    B, Hq, Hkv, D, start, R = 2, 4, 2, 64, 37, 9
    P = start + R
    q = np.stack([_lossless_rows(g, (R, Hq), D, -8) for _ in range(B)])
    k = np.stack([_lossless_rows(g, (P, Hkv), D, -6) for _ in range(B)])
    v = g.standard_normal((B, P, Hkv, D)).astype(np.float32)
    want = oracle.prefill_chunk(q, k, v, start, 0.5)
    got = oi8.prefill_chunk_i8(q, k, v, start, 0.5)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)
    ctx = [P, 11]
    qd = q[:, 3]
    np.testing.assert_allclose(oi8.decode_i8(qd, k, v, ctx, 0.5),
                               oracle.decode(qd, k, v, ctx, 0.5), rtol=1e-12, atol=1e-12)


def test_int8_chunk_rows_are_decode_rows():
    """Row t of a chunk at start s is the decode of that row with context
    s + t + 1, and the chunk's rows are attend_rows_i8 at s .. s + R - 1."""
    g = np.random.default_rng(16)
    Hq, Hkv, D, start, R = 4, 1, 32, 20, 6
    P = start + R
    q = g.standard_normal((1, R, Hq, D)).astype(np.float32)
    k = g.standard_normal((1, P, Hkv, D)).astype(np.float32)
    v = g.standard_normal((1, P, Hkv, D)).astype(np.float32)
    chunk = oi8.prefill_chunk_i8(q, k, v, start, 0.3)
    qc, qs = oi8.quantize_rows(q[0])
    kc, ks = oi8.quantize_rows(k[0])
    np.testing.assert_array_equal(
        chunk[0], oi8.attend_rows_i8(qc, qs, kc, ks, v[0], np.arange(start, P), 0.3))
    for t in range(R):
        d = oi8.decode_i8(q[:, t], k, v, [start + t + 1], 0.3)
        np.testing.assert_allclose(d[0], chunk[0, t], rtol=1e-13, atol=1e-13)
