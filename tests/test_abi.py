"""The C ABI: the library loads, exports what the header declares, and
rejects bad arguments on the host before touching the GPU (no GPU needed:
every call here fails validation, which runs before any HIP call)."""
import ctypes
import os
import re

import numpy as np
import pytest

import kv_cache_attention_amd as ka
from tests.cache_layout import unpack_k, unpack_k_i8, unpack_v

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ka_attn.h")


def _lib_or_skip():
    try:
        return ka.lib()
    except ka.KaAttnUnavailable as e:
        pytest.fail(f"library not built: {e}")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ka_attn_\w+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = header_functions()
    for n in ["ka_attn_append_kv", "ka_attn_append_kv_rope", "ka_attn_rope_rows",
              "ka_attn_prefill_chunk", "ka_attn_decode", "ka_attn_decode_step",
              "ka_attn_decode_workspace_bytes", "ka_attn_prefill_workspace_bytes",
              "ka_attn_cache_bytes", "ka_attn_status_string", "ka_attn_last_error",
              "ka_attn_abi_version", "ka_attn_append_kv_ragged", "ka_attn_prefill_ragged",
              "ka_attn_prefill_ragged_workspace_bytes", "ka_attn_prefill_ragged_workspace_need",
              "ka_attn_session_memory",
              "ka_attn_cache_resize"]:
        assert n in names
    assert set(names) == set(ka.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol():
    L = _lib_or_skip()
    for n in header_functions():
        assert hasattr(L, n), n
    assert ka.abi_version() == 1


def test_status_strings():
    _lib_or_skip()
    assert ka.status_string(0) == "KA_OK"
    assert ka.status_string(4) == "KA_ERR_WORKSPACE"
    assert ka.status_string(99) == "KA_ERR_UNKNOWN"


def S(**kw):
    d = dict(batch=1, num_q_heads=8, num_kv_heads=1, head_dim=256, capacity=4096, kv_dtype=ka.BF16)
    d.update(kw)
    return ka.Shape(**d)


def test_cache_bytes():
    _lib_or_skip()
    assert ka.cache_bytes(S()) == 4096 * 256 * 2
    # int8 K: both buffers the bf16 V size, which holds the codes and the row scales
    assert ka.cache_bytes(S(kv_dtype=ka.I8K, batch=2)) == 2 * 4096 * 256 * 2
    assert ka.cache_bytes(S(kv_dtype=ka.I8K, head_dim=64)) >= 4096 * (64 + 4)
    assert ka.cache_bytes(S(kv_dtype=ka.F32, batch=3, num_kv_heads=2)) == 3 * 2 * 4096 * 256 * 4
    assert ka.cache_bytes(S(head_dim=96)) == 0
    assert ka.cache_bytes(S(capacity=100)) == 0
    # the largest shape the ABI takes: sizes stay exact
    big = S(batch=65536, num_q_heads=1024, num_kv_heads=1024, capacity=131072, kv_dtype=ka.F32)
    assert ka.cache_bytes(big) == 65536 * 1024 * 131072 * 256 * 4
    assert ka.cache_bytes(S(batch=65537)) == 0 and ka.cache_bytes(S(num_q_heads=1032)) == 0


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first


def _append(shape, start, rows, ptr=FAKE):
    return ka.lib().ka_attn_append_kv(ctypes.byref(shape), ptr, ptr, ptr, ptr, start, rows, None)


def _prefill(shape, start, rows, scale=0.0625, ws=None, ws_bytes=0, q=FAKE, out=ctypes.c_void_p(0x2000)):
    return ka.lib().ka_attn_prefill_chunk(ctypes.byref(shape), q, FAKE, FAKE, out, start, rows,
                                          scale, ws, ws_bytes, None)


def _decode(shape, ctx, scale=0.0625, ws=None, ws_bytes=0, q=FAKE, out=ctypes.c_void_p(0x2000)):
    arr = (ctypes.c_int32 * len(ctx))(*ctx)
    return ka.lib().ka_attn_decode(ctypes.byref(shape), q, FAKE, FAKE, out, arr, scale, ws,
                                   ws_bytes, None)


@pytest.mark.parametrize("shape,status", [
    (S(batch=0), 1), (S(num_q_heads=0), 1), (S(num_kv_heads=3), 1), (S(head_dim=80), 3),
    (S(kv_dtype=7), 3), (S(capacity=131072 + 64), 2), (S(capacity=1000), 1), (S(capacity=0), 1),
    (S(num_q_heads=1025, num_kv_heads=1025), 2), (S(num_q_heads=2048, num_kv_heads=2), 2),
    (S(batch=65537), 2),
])
def test_bad_shapes_rejected_everywhere(shape, status):
    _lib_or_skip()
    assert _append(shape, 0, 1) == status
    assert _prefill(shape, 0, 1) == status
    assert _decode(shape, [1] * max(shape.batch, 1)) == status
    assert ka.last_error() != ""


def test_append_argument_errors():
    _lib_or_skip()
    s = S()
    assert _append(s, -1, 1) == 1
    assert _append(s, 0, -1) == 1
    assert _append(s, 4000, 97) == 2
    assert _append(s, 0, 1, ptr=None) == 1
    assert _append(s, 4096, 0) == 0          # an empty append is a no-op
    assert ka.last_error() == ""


def test_rope_argument_errors():
    _lib_or_skip()
    L = ka.lib()
    s = S()
    def app(start, rows, cos=FAKE, sin=FAKE, ptr=FAKE):
        return L.ka_attn_append_kv_rope(ctypes.byref(s), ptr, ptr, ptr, ptr, cos, sin, start, rows, None)
    assert app(-1, 1) == 1
    assert app(0, -1) == 1
    assert app(4000, 97) == 2
    assert app(0, 1, cos=None) == 1
    assert app(0, 1, sin=None) == 1
    assert app(0, 1, ptr=None) == 1
    assert app(0, 0, cos=None, sin=None) == 0     # an empty append is a no-op
    assert L.ka_attn_rope_rows(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, -1, None) == 1
    assert L.ka_attn_rope_rows(ctypes.byref(s), None, FAKE, FAKE, FAKE, 3, None) == 1
    assert L.ka_attn_rope_rows(ctypes.byref(s), FAKE, FAKE, FAKE, None, 3, None) == 1
    assert L.ka_attn_rope_rows(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, 0, None) == 0
    bad = S(head_dim=96)
    assert L.ka_attn_rope_rows(ctypes.byref(bad), FAKE, FAKE, FAKE, FAKE, 3, None) == 3


def test_prefill_argument_errors():
    _lib_or_skip()
    s = S()
    assert _prefill(s, 0, 1, scale=float("nan")) == 1
    assert _prefill(s, 0, 1, scale=float("inf")) == 1
    assert _prefill(s, 0, 1, scale=0.0) == 1
    assert _prefill(s, 0, 1, scale=-1.0) == 1
    assert _prefill(s, 4090, 7) == 2
    assert _prefill(s, 0, 1, q=None) == 1
    assert _prefill(s, 0, 1, out=FAKE) == 1      # out aliases q
    assert _prefill(s, 0, 0) == 0                # empty chunk is a no-op
    # a long chunk needs a workspace; a missing or short one is rejected.  The
    # exact need of this call gates the fake-pointer calls: with none needed
    # they would pass validation and enqueue kernels on fake addresses.
    need = ka.prefill_workspace_need(s, 3000, 768)
    assert 0 < need <= ka.prefill_workspace_bytes(s, 768)
    assert _prefill(s, 3000, 768) == 4
    assert _prefill(s, 3000, 768, ws=FAKE, ws_bytes=need - 1) == 4
    assert ka.prefill_workspace_need(s, 3000, 0) == 0
    assert ka.prefill_workspace_need(s, 4000, 97) == 0       # past the capacity


def _fused(shape, start, rows, scale=0.0625, ws=None, ws_bytes=0, q=FAKE, kn=FAKE,
           out=ctypes.c_void_p(0x2000)):
    return ka.lib().ka_attn_append_prefill_chunk(ctypes.byref(shape), q, kn, FAKE, FAKE, FAKE,
                                                 out, start, rows, scale, ws, ws_bytes, None)


def test_fused_append_prefill_argument_errors():
    _lib_or_skip()
    s = S()
    assert _fused(s, 0, 1, scale=float("nan")) == 1
    assert _fused(s, 0, 1, scale=0.0) == 1
    assert _fused(s, 4090, 7) == 2
    assert _fused(s, -1, 7) == 1
    assert _fused(s, 0, -1) == 1
    assert _fused(s, 0, 1, q=None) == 1
    assert _fused(s, 0, 1, kn=None) == 1
    assert _fused(s, 0, 1, out=FAKE) == 1       # out aliases q
    assert _fused(s, 0, 0) == 0                 # empty chunk is a no-op
    assert _fused(S(head_dim=80), 0, 1) == 3
    assert ka.last_error() != ""
    # the exact need gates the fake-pointer calls (see the prefill test)
    for kv in (ka.BF16, ka.I8K, ka.F32):
        sk = S(kv_dtype=kv)
        need = ka.append_prefill_workspace_need(sk, 3000, 768)
        assert 0 < need <= ka.append_prefill_workspace_bytes(sk, 768)
        assert _fused(sk, 3000, 768) == 4
        assert _fused(sk, 3000, 768, ws=FAKE, ws_bytes=need - 1) == 4
        part = ka.prefill_workspace_need(sk, 3000, 768)
        if kv == ka.BF16:   # the bf16 Q copy behind the partials
            assert need == ((part + 255) // 256) * 256 + 768 * 8 * 256 * 2
        else:
            assert need == part
    assert ka.append_prefill_workspace_need(s, 4000, 97) == 0
    assert ka.append_prefill_workspace_bytes(s, 0) == 0


def test_fused_workspace_bound_covers_every_chunk():
    _lib_or_skip()
    rng = np.random.default_rng(7)
    for kv in (ka.BF16, ka.I8K, ka.F32):
        for B, hq, hkv, D in ((1, 8, 1, 256), (3, 8, 2, 128), (2, 2, 1, 64)):
            s = S(batch=B, num_q_heads=hq, num_kv_heads=hkv, head_dim=D, kv_dtype=kv)
            for R in (1, 15, 16, 100, 768, 4096):
                bound = ka.append_prefill_workspace_bytes(s, R)
                for start in rng.integers(0, 4096 - R + 1, size=6):
                    for r in (R, max(1, R // 2)):
                        assert ka.append_prefill_workspace_need(s, int(start), r) <= bound


def test_decode_argument_errors():
    _lib_or_skip()
    s = S(batch=2)
    assert _decode(s, [1, 0]) == 2
    assert _decode(s, [4097, 3]) == 2
    assert _decode(s, [5, 5], scale=float("nan")) == 1
    arr = None
    assert ka.lib().ka_attn_decode(ctypes.byref(s), FAKE, FAKE, FAKE, ctypes.c_void_p(0x2000), arr,
                                   0.1, None, 0, None) == 1
    # the bound at this call's longest context is the call's own need (the
    # plan depends on the shape and that context only), 0 for a one-split
    # plan: need > 0 gates the fake-pointer calls
    need = ka.decode_workspace_bytes(s, 4096)
    assert need > 0
    assert _decode(s, [4096, 10]) == 4
    assert _decode(s, [4096, 10], ws=FAKE, ws_bytes=need - 1) == 4


def _step(shape, pos, scale=0.0625, ws=None, ws_bytes=0, q=FAKE, out=ctypes.c_void_p(0x2000)):
    arr = (ctypes.c_int32 * len(pos))(*pos)
    return ka.lib().ka_attn_decode_step(ctypes.byref(shape), q, FAKE, FAKE, FAKE, FAKE, out, arr,
                                        scale, ws, ws_bytes, None)


def test_decode_step_argument_errors():
    _lib_or_skip()
    s = S(batch=2)
    assert _step(s, [0, 4096]) == 2          # pos is a position: 0 .. C - 1
    assert _step(s, [-1, 3]) == 2
    assert _step(s, [5, 5], scale=float("nan")) == 1
    assert _step(s, [5, 5], q=None) == 1
    assert _step(s, [5, 5], out=FAKE) == 1   # out aliases q
    assert ka.lib().ka_attn_decode_step(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE,
                                        ctypes.c_void_p(0x2000), None, 0.1, None, 0, None) == 1
    need = ka.decode_workspace_bytes(s, 4096)   # the call's own need (ctx 4096), as above
    assert need > 0
    assert _step(s, [4095, 10]) == 4
    assert _step(s, [4095, 10], ws=FAKE, ws_bytes=need - 1) == 4
    assert "workspace" in ka.last_error()


def test_workspace_sizes_cover_smaller_requests():
    _lib_or_skip()
    s = S(batch=4, capacity=131072)
    big = ka.decode_workspace_bytes(s, 131072)
    for c in [1, 64, 1000, 16384, 65536]:
        assert ka.decode_workspace_bytes(s, c) <= big
    p = ka.prefill_workspace_bytes(s, 768)
    for r in [1, 16, 100, 767]:
        assert ka.prefill_workspace_bytes(s, r) <= p


@pytest.mark.parametrize("kv", ["f32", "bf16", "i8k"])
@pytest.mark.parametrize("batch,hq,hkv", [(1, 8, 1), (2, 8, 1), (4, 8, 2), (1, 1, 1), (3, 2, 1),
                                          (16, 16, 1), (1, 12, 3)])
def test_decode_workspace_never_shrinks_with_the_context(kv, batch, hq, hkv):
    """A workspace sized for the longest context serves every shorter one:
    the f32 plan changes its heads per workgroup with the step's size, and
    its reported bound must still grow with the context."""
    _lib_or_skip()
    s = ka.Shape(batch, hq, hkv, 128, 70016, kv)
    cs = sorted(set(list(range(1, 70016, 97)) + [16 * u + d for u in (512, 1024, 2048, 4096)
                                                 for k in (1, 2, 3, 4, 8, 16)
                                                 for u in [u // k] for d in (-1, 0, 1)
                                                 if 1 <= 16 * u + d <= 70016]))
    prev = 0
    for c in cs:
        b = ka.decode_workspace_bytes(s, c)
        assert b >= prev, (c, b, prev)
        prev = b


def _i32(xs):
    return (ctypes.c_int32 * len(xs))(*xs)


def test_ragged_argument_errors():
    _lib_or_skip()
    L = ka.lib()
    s = S(batch=3)
    def pre(starts, rows, scale=0.0625, ws=None, ws_bytes=0, q=FAKE, out=ctypes.c_void_p(0x2000)):
        return L.ka_attn_prefill_ragged(ctypes.byref(s), q, FAKE, FAKE, out, _i32(starts),
                                        _i32(rows), scale, ws, ws_bytes, None)
    def app(starts, rows, cos=None, sin=None):
        return L.ka_attn_append_kv_ragged(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, cos, sin,
                                          _i32(starts), _i32(rows), None)
    assert pre([0, 0, 0], [1, -1, 1]) == 1
    assert pre([0, -2, 0], [1, 1, 1]) == 1
    assert pre([0, 4000, 0], [1, 97, 1]) == 2
    assert "start_pos[1]" in ka.last_error()
    assert pre([0, 0, 0], [0, 0, 0]) == 0             # nothing to do
    assert pre([0, 0, 0], [1, 1, 1], scale=float("nan")) == 1
    assert pre([0, 0, 0], [1, 1, 1], out=FAKE) == 1   # out aliases q
    assert L.ka_attn_prefill_ragged(ctypes.byref(s), FAKE, FAKE, FAKE, ctypes.c_void_p(0x2000),
                                    None, _i32([1, 1, 1]), 0.1, None, 0, None) == 1
    # long chunks need a workspace: the exact need of this call (which the
    # bound for their total covers) gates the fake-pointer calls
    starts, rows = [3000, 0, 1000], [768, 0, 500]
    need = ka.prefill_ragged_workspace_need(s, starts, rows)
    assert 0 < need <= ka.prefill_ragged_workspace_bytes(s, sum(rows))
    assert pre(starts, rows) == 4
    assert pre(starts, rows, ws=FAKE, ws_bytes=need - 1) == 4
    assert app([0, 0, 0], [1, 0, -1]) == 1
    assert app([0, 4090, 0], [1, 7, 1]) == 2
    assert app([0, 0, 0], [1, 1, 1], cos=FAKE) == 1   # only one rotary table
    assert app([5, 5, 5], [0, 0, 0]) == 0


def test_ragged_workspace_bound_covers_every_split_of_the_rows():
    """The bound for T rows covers the exact need of any split of T rows over
    the sessions at any starts (host-side queries only)."""
    _lib_or_skip()
    s = S(batch=4, capacity=16384)
    g = np.random.default_rng(3)
    needed = 0
    for _ in range(200):
        total = int(g.integers(1, 4000))
        cuts = np.sort(g.integers(0, total + 1, size=3))
        rows = np.diff(np.concatenate([[0], cuts, [total]])).astype(int).tolist()
        if max(rows) > 16384:
            continue
        starts = [int(g.integers(0, 16384 - r + 1)) for r in rows]
        need = ka.prefill_ragged_workspace_need(s, starts, rows)
        assert need <= ka.prefill_ragged_workspace_bytes(s, total), (rows, starts)
        needed += need > 0
    assert needed > 50
    assert ka.prefill_ragged_workspace_need(s, [0] * 4, [0] * 4) == 0
    assert ka.prefill_ragged_workspace_need(s, [0, 0, 0, 16384], [1, 1, 1, 1]) == 0  # invalid


def test_session_memory_closed_forms():
    _lib_or_skip()
    for sh, rows in [(S(batch=1, num_q_heads=8, num_kv_heads=1, head_dim=256, capacity=16384), 768),
                     (S(batch=4, num_q_heads=8, num_kv_heads=1, head_dim=256, capacity=131072), 768),
                     (S(batch=2, num_q_heads=16, num_kv_heads=2, head_dim=128, capacity=4096,
                        kv_dtype=ka.F32), 100)]:
        m = ka.session_memory(sh, rows)
        es = 2 if sh.kv_dtype == ka.BF16 else 4
        assert m.cache_bytes == 2 * sh.batch * sh.num_kv_heads * sh.capacity * sh.head_dim * es
        assert m.cache_bytes == 2 * ka.cache_bytes(sh)
        assert m.prefill_workspace_bytes == ka.prefill_workspace_bytes(sh, rows)
        assert m.decode_workspace_bytes == ka.decode_workspace_bytes(sh, sh.capacity)
        assert m.chunk_io_bytes == sh.batch * rows * (2 * sh.num_q_heads + 2 * sh.num_kv_heads) * sh.head_dim * 4
        assert m.total_bytes == (m.cache_bytes + max(m.prefill_workspace_bytes, m.decode_workspace_bytes)
                                 + m.chunk_io_bytes)
    # 4 sessions x 131072 positions of bf16 K and V, head_dim 256: exactly 512 MiB
    assert ka.session_memory(S(batch=4, capacity=131072), 768).cache_bytes == 512 * 2**20
    with pytest.raises(ka.KaAttnError):
        ka.session_memory(S(), 0)
    with pytest.raises(ka.KaAttnError):
        ka.session_memory(S(), 4097)


def test_cache_resize_argument_errors():
    _lib_or_skip()
    L = ka.lib()
    a, b = S(capacity=1024), S(capacity=2048)
    A, Bp = ctypes.c_void_p(0x100000), ctypes.c_void_p(0x200000)
    Av, Bv = ctypes.c_void_p(0x300000), ctypes.c_void_p(0x400000)
    def rs(src, dst, rows, sk=A, sv=Av, dk=Bp, dv=Bv):
        return L.ka_attn_cache_resize(ctypes.byref(src), sk, sv, ctypes.byref(dst), dk, dv, rows, None)
    assert rs(a, S(capacity=2048, head_dim=128), 10) == 1     # more than capacity differs
    assert rs(a, S(capacity=2048, kv_dtype=ka.F32), 10) == 1
    assert rs(a, b, -1) == 1
    assert rs(a, b, 1025) == 2
    assert rs(b, a, 1500) == 2
    assert rs(a, b, 0) == 0
    assert rs(a, b, 10, dk=None) == 1
    # overlapping caches: K of the destination inside K of the source
    assert rs(a, b, 10, dk=ctypes.c_void_p(0x100000 + 64)) == 1
    assert "overlap" in ka.last_error()


# ------------------------------------------- the test-side layout readers

def test_layout_reader_round_trip_k_and_v():
    """The readers invert the header's index formulas (checked on a marked
    cache: each element stores its own logical coordinates)."""
    B, Hkv, C, D = 2, 2, 64, 16
    for dt, E in (("f32", 4), ("bf16", 8)):
        nel = B * Hkv * C * D
        # element index formulas from the header
        raw_k = np.zeros(nel, np.uint16 if dt == "bf16" else np.float32)
        raw_v = np.zeros_like(raw_k)
        want = np.zeros((B, Hkv, C, D))
        for b in range(B):
            for g in range(Hkv):
                for j in range(C):
                    for d in range(D):
                        val = ((b * Hkv + g) * C + j) * D + d
                        want[b, g, j, d] = val
                        ki = ((((b * Hkv + g) * (C // 64) + j // 64) * (D // E) + d // E) * 64 + j % 64) * E + d % E
                        if dt == "f32":
                            vi = (((b * Hkv + g) * (C // 4) + j // 4) * D + d) * 4 + j % 4
                        else:
                            r = j % 32
                            s_, t = 2 * (r // 16) + (r % 8) // 4, r % 4 + 4 * ((r % 16) // 8)
                            vi = ((((b * Hkv + g) * (C // 32) + j // 32) * 4 + s_) * D + d) * 8 + t
                        raw_k[ki] = val
                        raw_v[vi] = val
        assert np.array_equal(unpack_k(raw_k, B, Hkv, C, D, dt).astype(np.float64), want)
        assert np.array_equal(unpack_v(raw_v, B, Hkv, C, D, dt).astype(np.float64), want)


def test_int8_k_layout_reader():
    """The int8-K reader inverts the header's byte formulas (a marked buffer:
    every code byte holds its (j + d) mod 251 - 125, every scale its row)."""
    B, Hkv, C, D = 2, 2, 128, 32
    raw = np.zeros(B * Hkv * C * D + B * Hkv * C * 4, np.uint8)
    want_c = np.zeros((B, Hkv, C, D), np.int8)
    for b in range(B):
        for g in range(Hkv):
            for j in range(C):
                for d in range(D):
                    v = (j + d + 7 * b + 3 * g) % 251 - 125
                    want_c[b, g, j, d] = v
                    i = (((b * Hkv + g) * (C // 64) + j // 64) * (D // 16) + d // 16) * 64 * 16 + (j % 64) * 16 + d % 16
                    raw[i] = np.uint8(v & 0xFF)
    sc = np.arange(B * Hkv * C, dtype=np.float32) * 0.5
    raw[B * Hkv * C * D:] = sc.view(np.uint8)
    codes, scales = unpack_k_i8(raw, B, Hkv, C, D)
    assert np.array_equal(codes, want_c)
    assert np.array_equal(scales.reshape(-1), sc)


def test_noalloc_decode_step_validation():
    """The allocation-free decode step validates as the decode step does, and
    rejects partials beyond its scratch (f32 caches with 511 slabs split
    into 1022 partials of 8 heads), all before anything is enqueued."""
    _lib_or_skip()
    L = ka.lib()
    out = ctypes.c_void_p(0x2000)

    def call(s, pos, scale=0.1, q=FAKE, o=out):
        arr = (ctypes.c_int32 * len(pos))(*pos)
        return L.ka_attn_decode_step_noalloc(ctypes.byref(s), q, FAKE, FAKE, FAKE, FAKE, o, arr,
                                             ctypes.c_float(scale), None)
    s = S(batch=2)
    assert call(s, [0, 4096]) == 2
    assert call(s, [5, 5], scale=float("nan")) == 1
    assert call(s, [5, 5], q=None) == 1
    assert call(s, [5, 5], o=FAKE) == 1            # out aliases q
    assert call(S(head_dim=96), [5]) == 3
    big = S(batch=511, kv_dtype=ka.F32)
    assert ka.decode_workspace_bytes(big, 4096) > ka.decode_step_noalloc_max_bytes()
    assert call(big, [4095] * 511) == 4 and "scratch" in ka.last_error()
    assert ka.decode_step_noalloc_max_bytes() == 8 << 20
