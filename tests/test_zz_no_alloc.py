"""The allocation-free decode step (ka_attn_decode_step_noalloc) against the
decode step with a caller's workspace (ka_attn_decode_step), through the C
ABI: the same kernels on the same inputs, so the outputs must agree bit for
bit (and with the oracle within the usual tolerance).  Each case makes two
calls in a row on the library's scratch array, the second with a smaller
input, so nothing of the first call's partials may reach the second."""
import ctypes

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

PAIRS = [
    # dt, (B, Hq, Hkv, D, C, pos) of the first call, then of the second
    ("bf16", (4, 8, 1, 256, 16448, [16384, 9000, 16447, 1]), (1, 8, 1, 256, 4160, [1000])),
    ("i8k", (2, 8, 1, 256, 16448, [16384, 4097]), (1, 16, 2, 128, 1024, [300])),
    ("f32", (2, 8, 1, 256, 8192, [8000, 5000]), (1, 4, 2, 64, 512, [200])),
]


def _call(dt, B, Hq, Hkv, D, C, pos, seed):
    P = max(pos) + 1
    c = random_case(seed, B, Hq, Hkv, D, P, 1)
    g = np.random.default_rng(seed + 1)
    k_new = g.standard_normal((B, Hkv, D), dtype=np.float32)
    v_new = g.standard_normal((B, Hkv, D), dtype=np.float32)
    caches = DevCaches(B, Hq, Hkv, D, C, dt)
    caches.append(c.k, c.v, 0)
    q = dev(c.q[:, 0])
    kn, vn = dev(k_new), dev(v_new)
    scale = 1.0 / np.sqrt(D)
    # the decode step with a workspace
    ws_n = ka.decode_workspace_bytes(caches.shape, P)
    ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device="cuda")
    want = torch.full_like(q, float("nan"))
    ka.decode_step(caches.shape, q, kn, vn, caches.k, caches.v, want, pos, scale, ws)
    # the allocation-free step on the same cache (it stores the same rows again)
    got = torch.full_like(q, float("nan"))
    arr = (ctypes.c_int32 * B)(*pos)
    st = ka.lib().ka_attn_decode_step_noalloc(
        ctypes.byref(caches.shape), ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(kn.data_ptr()),
        ctypes.c_void_p(vn.data_ptr()), ctypes.c_void_p(caches.k.data_ptr()),
        ctypes.c_void_p(caches.v.data_ptr()), ctypes.c_void_p(got.data_ptr()), arr,
        ctypes.c_float(scale), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, ka.last_error()
    torch.cuda.synchronize()
    got, want = got.cpu().numpy(), want.cpu().numpy()
    print(f"{dt} B={B} D={D} pos={pos}: workspace variant needs {ws_n} bytes", flush=True)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    # and the oracle
    k_all, v_all = c.k.copy(), c.v.copy()
    for b, p in enumerate(pos):
        k_all[b, p], v_all[b, p] = k_new[b], v_new[b]
    store = "f32" if dt == "f32" else "bf16"
    vs = oracle.stored_values(v_all, store)
    for b, p in enumerate(pos):
        if dt == "i8k":
            ref = oi8.decode_i8(c.q[b:b + 1, 0], k_all[b:b + 1, :p + 1], vs[b:b + 1, :p + 1],
                                [p + 1], scale)
        else:
            ref = oracle.decode(c.q[b:b + 1, 0], oracle.stored_values(k_all, store)[b:b + 1, :p + 1],
                                vs[b:b + 1, :p + 1], [p + 1], scale)
        assert oracle.rel_error(got[b:b + 1], ref, vs[b:b + 1, :p + 1]) <= TOL[dt]


@pytest.mark.parametrize("pair", PAIRS, ids=lambda p: p[0])
def test_noalloc_decode_step_matches_the_workspace_variant(pair):
    dt, first, second = pair
    _call(dt, *first, seed=61)
    _call(dt, *second, seed=62)
