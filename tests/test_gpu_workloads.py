"""GPU parity at the benchmark's full sizes, in the launch configuration the
benchmark times (same entry points, shapes and chunk schedule), checked on
sampled outputs that the oracle computes row by row.

  * 16K session, bf16 cache: 21 chunks of 768 rows + one of 256 (append then
    prefill each), then 64 decode steps (append the step's row, decode).
  * 128K decode, bf16 cache, 4 sessions: fill 131040 positions, then 32
    batched decode steps up to context 131072.
"""
import numpy as np
import pytest
import torch

import oracle
from synth import WORKLOADS, draw_batch
from tests.gpu_session import DevCaches, dev

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

TOL_BF16 = 1e-2


def _say(*a):
    print(*a, flush=True)


def test_long_session_16k_bf16():
    w = WORKLOADS[4]
    c = draw_batch(w)
    ks = oracle.stored_values(c.k, "bf16")
    vs = oracle.stored_values(c.v, "bf16")
    caches = DevCaches(1, 8, 1, 256, w.capacity, "bf16")
    rng = np.random.default_rng(44)
    worst = 0.0
    qrow = 0
    for ci, (start, R) in enumerate(w.chunks):
        caches.append(c.k[:, start:start + R], c.v[:, start:start + R], start)
        got = caches.prefill(c.q[:, qrow:qrow + R], start, w.scale)
        rows = sorted(set([0, 1, R // 2, R - 1] + list(rng.integers(0, R, 4))))
        ref = oracle.attend_rows(c.q[0, qrow + np.array(rows)], ks[0], vs[0],
                                 start + np.array(rows), w.scale)
        err = oracle.rel_error(got[0, rows], ref, vs)
        assert np.isfinite(got).all(), f"chunk {ci}: non-finite output"
        worst = max(worst, err)
        assert err <= TOL_BF16, f"chunk {ci} at {start}: {err}"
        qrow += R
    _say(f"16K prefill: worst sampled rel err {worst:.3e} over {len(w.chunks)} chunks")
    worst = 0.0
    for t, p in enumerate(w.decode_positions):
        caches.append(c.k[:, p:p + 1], c.v[:, p:p + 1], p)
        q = c.q[:, qrow + t]
        got = caches.decode(q, [p + 1], w.scale)
        ref = oracle.decode(q, ks, vs, [p + 1], w.scale)
        err = oracle.rel_error(got, ref, vs)
        worst = max(worst, err)
        assert err <= TOL_BF16, f"decode step {t}: {err}"
    _say(f"16K decode: worst rel err {worst:.3e} over {len(w.decode_positions)} steps")


def test_max_context_decode_4x128k_bf16():
    w = WORKLOADS[5]
    c = draw_batch(w)
    _say("drawn 4 x 131072 positions")
    caches = DevCaches(w.batch, 8, 1, 256, w.capacity, "bf16")
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
        caches.append(c.k[:, p:p + 1], c.v[:, p:p + 1], p)
        q = c.q[:, t]
        got = caches.decode(q, [p + 1] * w.batch, w.scale)
        assert np.isfinite(got).all()
        outs.append(got)
        if t in (0, 1, 16, 31):
            ref = oracle.decode(q, ks, vs, [p + 1] * w.batch, w.scale)
            err = oracle.rel_error(got, ref, vs)
            worst = max(worst, err)
            _say(f"step {t} ctx {p + 1}: rel err {err:.3e}")
            assert err <= TOL_BF16, f"step {t}: {err}"
    # run-to-run: the last step again gives the same bits
    again = caches.decode(c.q[:, 31], [131072] * w.batch, w.scale)
    assert np.array_equal(again.view(np.uint32), outs[-1].view(np.uint32))
    _say(f"128K x4 decode: worst sampled rel err {worst:.3e}")
