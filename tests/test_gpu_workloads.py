"""GPU parity at the benchmark's full sizes, through the calls the benchmark
times, with the same shapes and schedule:

  * 16K session, bf16 cache: 21 chunks of 768 rows + one of 256, each one
    ka_attn_append_prefill_chunk call (the chunk's append and prefill);
    the last 768-row chunk and the 256-row chunk are compared in full, the
    others on sampled rows.  Then 64 decode steps, each one
    ka_attn_decode_step call (append of the step's row + decode), every step
    compared with the oracle.  The same session on an int8-K cache.
  * 128K decode, 4 sessions, bf16 and int8-K caches: fill 131040 positions,
    then 32 batched ka_attn_decode_step calls up to context 131072; steps 0,
    1, 16 and 31 compared with the oracle.
  * The f32 decode step at context 4097 (8 query heads, head_dim 256) and
    the f32 chunk of 768 rows at 3072, both compared in full.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import int8 as oi8
from synth import WORKLOADS, draw_batch
from tests.gpu_session import DevCaches

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

TOL = {"bf16": 1e-2, "i8k": 1e-2, "f32": 1e-5}


def _say(*a):
    print(*a, flush=True)


def _ref_rows(dt, q_rows, k, vs, ks, positions, scale):
    """Oracle rows of session 0 at the given absolute positions."""
    if dt == "i8k":
        qc, qs = oi8.quantize_rows(q_rows)
        kc, ksc = oi8.quantize_rows(k[0])
        return oi8.attend_rows_i8(qc, qs, kc, ksc, vs[0], positions, scale)
    return oracle.attend_rows(q_rows, ks[0], vs[0], positions, scale)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("dt", ["bf16", "i8k"])
def test_long_session_16k(dt):
    w = WORKLOADS[4]
    c = draw_batch(w)
    ks = oracle.stored_values(c.k, "bf16")
    vs = oracle.stored_values(c.v, "bf16")
    caches = DevCaches(1, 8, 1, 256, w.capacity, dt)
    rng = np.random.default_rng(44)
    worst = 0.0
    qrow = 0
    last = len(w.chunks) - 1
    for ci, (start, R) in enumerate(w.chunks):
        got = caches.append_prefill(c.q[:, qrow:qrow + R], c.k[:, start:start + R],
                                    c.v[:, start:start + R], start, w.scale)
        assert np.isfinite(got).all(), f"chunk {ci}: non-finite output"
        if ci >= last - 1:
            rows = list(range(R))          # the last 768-row chunk and the 256-row chunk
        else:
            rows = sorted(set([0, 1, R // 2, R - 1] + list(rng.integers(0, R, 4))))
        ref = _ref_rows(dt, c.q[0, qrow + np.array(rows)], c.k, vs, ks, start + np.array(rows),
                        w.scale)
        err = oracle.rel_error(got[0, rows], ref, vs)
        worst = max(worst, err)
        if len(rows) == R:
            _say(f"{dt} chunk {ci} at {start}: all {R} rows, rel err {err:.3e}")
        assert err <= TOL[dt], f"chunk {ci} at {start}: {err}"
        qrow += R
    _say(f"{dt} 16K prefill: worst rel err {worst:.3e} over {len(w.chunks)} chunks")
    worst = 0.0
    for t, p in enumerate(w.decode_positions):
        q = c.q[:, qrow + t]
        got = caches.decode_step(q, c.k[:, p], c.v[:, p], [p], w.scale)
        ref = _ref_rows(dt, q, c.k[:, :p + 1], vs[:, :p + 1], ks[:, :p + 1], [p], w.scale)
        err = oracle.rel_error(got, ref, vs)
        worst = max(worst, err)
        assert err <= TOL[dt], f"decode step {t} at {p}: {err}"
    _say(f"{dt} 16K decode steps: worst rel err {worst:.3e} over {len(w.decode_positions)} steps")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("dt", ["bf16", "i8k"])
def test_max_context_decode_4x128k(dt):
    w = WORKLOADS[5]
    c = draw_batch(w)
    _say(f"{dt}: drawn 4 x 131072 positions")
    caches = DevCaches(w.batch, 8, 1, 256, w.capacity, dt)
    step = 16384
    for s in range(0, w.fill_rows, step):
        e = min(w.fill_rows, s + step)
        caches.append(c.k[:, s:e], c.v[:, s:e], s)
    torch.cuda.synchronize()
    _say("filled 131040 positions")
    ks = oracle.stored_values(c.k, "bf16")
    vs = oracle.stored_values(c.v, "bf16")
    worst = 0.0
    outs = []
    for t, p in enumerate(w.decode_positions):
        q = c.q[:, t]
        got = caches.decode_step(q, c.k[:, p], c.v[:, p], [p] * w.batch, w.scale)
        assert np.isfinite(got).all()
        outs.append(got)
        if t in (0, 1, 16, 31):
            ctx = [p + 1] * w.batch
            if dt == "i8k":
                ref = oi8.decode_i8(q, c.k, vs, ctx, w.scale)
            else:
                ref = oracle.decode(q, ks, vs, ctx, w.scale)
            err = oracle.rel_error(got, ref, vs)
            worst = max(worst, err)
            _say(f"{dt} step {t} ctx {p + 1}: rel err {err:.3e}")
            assert err <= TOL[dt], f"step {t}: {err}"
    # run-to-run: a plain decode of the cache the steps left gives the last step's bits
    again = caches.decode(c.q[:, 31], [131072] * w.batch, w.scale)
    assert np.array_equal(again.view(np.uint32), outs[-1].view(np.uint32))
    _say(f"{dt} 128K x4 decode steps: worst sampled rel err {worst:.3e}")


def test_f32_decode_step_at_4097():
    """8 query heads on one KV head, head_dim 256, 4096 cached rows: the step
    appends row 4096 and attends to 4097 keys."""
    w = WORKLOADS[2]
    c = draw_batch(w)
    caches = DevCaches(1, 8, 1, 256, w.capacity, "f32")
    caches.append(c.k[:, :w.fill_rows], c.v[:, :w.fill_rows], 0)
    p = w.decode_positions[0]
    q = c.q[:, 0]
    got = caches.decode_step(q, c.k[:, p], c.v[:, p], [p], w.scale)
    ref = oracle.decode(q, c.k, c.v, [p + 1], w.scale)
    err = oracle.rel_error(got, ref, c.v)
    _say(f"f32 decode step at {p}: rel err {err:.3e}")
    assert err <= TOL["f32"]


def test_f32_chunk_768_at_3072():
    w = WORKLOADS[3]
    c = draw_batch(w)
    caches = DevCaches(1, 8, 1, 256, w.capacity, "f32")
    (start, R), = w.chunks
    caches.append(c.k[:, :start + R], c.v[:, :start + R], 0)
    got = caches.prefill(c.q, start, w.scale)
    ref = oracle.prefill_chunk(c.q, c.k, c.v, start, w.scale)
    err = oracle.rel_error(got, ref, c.v)
    _say(f"f32 chunk {R} at {start}: rel err {err:.3e}")
    assert err <= TOL["f32"]
