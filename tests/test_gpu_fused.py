"""ka_attn_append_prefill_chunk: the chunk's append and prefill in one call.

It must give, bit for bit, the caches and the output of ka_attn_append_kv
followed by ka_attn_prefill_chunk (which the parity tests check against the
oracle): on bf16 caches its prefill reads Q that the append kernel scaled and
rounded exactly as the prefill kernel does itself, on the other caches it is
the two kernels back to back.  Shapes cover the M-tile plans with and without
splits, ragged M-tiles, the few-row plans, several sessions and KV heads, and
every head dim; one case is also checked against the oracle directly."""
import math

import numpy as np
import pytest
import torch

import kv_cache_attention_amd as ka
import oracle
from tests.gpu_session import DevCaches, dev

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

# (kv dtype, B, Hq, Hkv, D, C, [(start, R), ...]): each chunk follows a prefix
# appended up to its start
CASES = [
    ("bf16", 1, 8, 1, 256, 16448, [(0, 768), (768, 768), (15360, 768), (16128, 256)]),
    ("bf16", 2, 8, 2, 128, 4160, [(0, 300), (300, 17), (317, 5), (322, 1000)]),
    ("bf16", 1, 2, 1, 64, 1024, [(0, 128), (128, 16), (144, 3), (147, 500)]),
    ("bf16", 3, 4, 1, 256, 2048, [(0, 40), (40, 129), (169, 777)]),
    ("i8k", 1, 8, 1, 256, 4160, [(0, 768), (768, 300), (1068, 7)]),
    ("f32", 1, 8, 1, 256, 4160, [(0, 768), (768, 129)]),
    ("f32", 2, 2, 1, 64, 1024, [(0, 100), (100, 33)]),
]


def _same_bits(a: torch.Tensor, b: torch.Tensor) -> bool:
    ai, bi = a.view(torch.int32), b.view(torch.int32)
    return bool(torch.equal(ai, bi))


@pytest.mark.parametrize("dt,B,Hq,Hkv,D,C,chunks", CASES)
def test_fused_call_equals_append_then_prefill_bitwise(dt, B, Hq, Hkv, D, C, chunks):
    rng = np.random.default_rng(71 + D + B)
    sep = DevCaches(B, Hq, Hkv, D, C, dt)
    fus = DevCaches(B, Hq, Hkv, D, C, dt)
    sh = sep.shape
    scale = 1 / math.sqrt(D)
    R_max = max(R for _, R in chunks)
    ws_sep = torch.empty(max(ka.prefill_workspace_bytes(sh, R_max), 1), dtype=torch.uint8,
                         device="cuda")
    ws_fus = torch.empty(max(ka.append_prefill_workspace_bytes(sh, R_max), 1), dtype=torch.uint8,
                         device="cuda")
    filled = 0
    for start, R in chunks:
        if start > filled:  # the prefix up to the chunk, the same in both caches
            kp = rng.standard_normal((B, start - filled, Hkv, D), dtype=np.float32)
            vp = rng.standard_normal((B, start - filled, Hkv, D), dtype=np.float32)
            sep.append(kp, vp, filled)
            fus.append(kp, vp, filled)
        filled = start + R
        k = dev(rng.standard_normal((B, R, Hkv, D), dtype=np.float32))
        v = dev(rng.standard_normal((B, R, Hkv, D), dtype=np.float32))
        q = dev(rng.standard_normal((B, R, Hq, D), dtype=np.float32) * 2)
        need = ka.append_prefill_workspace_need(sh, start, R)
        assert need <= ka.append_prefill_workspace_bytes(sh, R)
        part = ka.prefill_workspace_need(sh, start, R)
        with_qb = ((part + 255) // 256) * 256 + B * R * Hq * D * 2
        if dt != "bf16":
            assert need == part
        elif R >= 16:          # always the M-tile kernel, which reads the bf16 Q copy
            assert need == with_qb
        else:                  # the few-row plan may serve it, without the copy
            assert need in (part, with_qb)
        out_sep = torch.full_like(q, float("nan"))
        out_fus = torch.full_like(q, float("nan"))
        ka.append_kv(sh, sep.k, sep.v, k, v, start, R)
        ka.prefill_chunk(sh, q, sep.k, sep.v, out_sep, start, R, scale, ws_sep)
        ka.append_prefill_chunk(sh, q, k, v, fus.k, fus.v, out_fus, start, R, scale, ws_fus)
        torch.cuda.synchronize()
        assert torch.isfinite(out_fus).all(), (start, R)
        assert _same_bits(out_fus, out_sep), (start, R)
        assert torch.equal(fus.k, sep.k) and torch.equal(fus.v, sep.v), (start, R)


def test_fused_call_against_the_oracle():
    """The 16K session's last 768-row chunk through the fused call, every row
    against the oracle (bf16 caches)."""
    B, Hq, Hkv, D, C = 1, 8, 1, 256, 16448
    start, R = 15360, 768
    rng = np.random.default_rng(83)
    caches = DevCaches(B, Hq, Hkv, D, C, "bf16")
    sh = caches.shape
    k_all = rng.standard_normal((B, start + R, Hkv, D), dtype=np.float32)
    v_all = rng.standard_normal((B, start + R, Hkv, D), dtype=np.float32)
    q = rng.standard_normal((B, R, Hq, D), dtype=np.float32)
    caches.append(k_all[:, :start], v_all[:, :start], 0)
    out = torch.full((B, R, Hq, D), float("nan"), device="cuda")
    ws = torch.empty(ka.append_prefill_workspace_bytes(sh, R), dtype=torch.uint8, device="cuda")
    ka.append_prefill_chunk(sh, dev(q), dev(k_all[:, start:]), dev(v_all[:, start:]), caches.k,
                            caches.v, out, start, R, 1 / 16, ws)
    torch.cuda.synchronize()
    ks, vs = oracle.stored_values(k_all, "bf16"), oracle.stored_values(v_all, "bf16")
    ref = oracle.prefill_chunk(q, ks, vs, start, 1 / 16)
    err = oracle.rel_error(out.cpu().numpy(), ref, vs)
    assert err <= 1e-2, err


def test_fused_call_nonfinite_value_reaches_only_later_rows():
    """A NaN in one appended V row: rows before it stay finite and equal to
    the separate calls; rows from it on are NaN in that dim only."""
    B, Hq, Hkv, D, C = 1, 8, 1, 128, 1024
    start, R, j, d = 64, 200, 150, 17
    rng = np.random.default_rng(89)
    sep = DevCaches(B, Hq, Hkv, D, C, "bf16")
    fus = DevCaches(B, Hq, Hkv, D, C, "bf16")
    k0 = rng.standard_normal((B, start, Hkv, D), dtype=np.float32)
    v0 = rng.standard_normal((B, start, Hkv, D), dtype=np.float32)
    sep.append(k0, v0, 0)
    fus.append(k0, v0, 0)
    k = rng.standard_normal((B, R, Hkv, D), dtype=np.float32)
    v = rng.standard_normal((B, R, Hkv, D), dtype=np.float32)
    v[0, j - start, 0, d] = np.nan
    q = dev(rng.standard_normal((B, R, Hq, D), dtype=np.float32))
    sh = sep.shape
    ws = torch.empty(ka.append_prefill_workspace_bytes(sh, R), dtype=torch.uint8, device="cuda")
    o_sep = torch.full_like(q, float("nan"))
    o_fus = torch.full_like(q, float("nan"))
    ka.append_kv(sh, sep.k, sep.v, dev(k), dev(v), start, R)
    ka.prefill_chunk(sh, q, sep.k, sep.v, o_sep, start, R, 1 / 16, ws)
    ka.append_prefill_chunk(sh, q, dev(k), dev(v), fus.k, fus.v, o_fus, start, R, 1 / 16, ws)
    torch.cuda.synchronize()
    o = o_fus.cpu().numpy()[0]
    assert np.isfinite(o[:j - start]).all()
    assert np.isnan(o[j - start:, :, d]).all()
    others = np.delete(o[j - start:], d, axis=2)
    assert np.isfinite(others).all()
    assert _same_bits(o_fus, o_sep)
