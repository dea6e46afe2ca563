"""The C-ABI calls under HIP graph capture.

The library never allocates, synchronises or clears memory on its launch
paths (workspaces are the caller's), so a chunk's append, its prefill, the
fused append-and-prefill call and a decode step can be captured into one
graph and replayed.  Each replay, with
the program's own eager work and synchronisations between replays, must give
bitwise the output of the same calls made eagerly, also after the captured
inputs have been rewritten in place."""
import numpy as np
import pytest
import torch

import kv_cache_attention_amd as ka
from tests.gpu_session import DevCaches, dev

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


@pytest.mark.parametrize("dt", ["bf16", "i8k", "f32"])
def test_chunk_and_decode_step_replay_bitwise(dt):
    B, Hq, Hkv, D, C = 1, 8, 1, 256, 4160
    start, R = 3072, 768
    pos = start + R                                    # the decode step's row
    rng = np.random.default_rng(61)
    caches = DevCaches(B, Hq, Hkv, D, C, dt)
    caches.append(rng.standard_normal((B, start, Hkv, D), dtype=np.float32),
                  rng.standard_normal((B, start, Hkv, D), dtype=np.float32), 0)
    k_rows = dev(rng.standard_normal((B, R, Hkv, D), dtype=np.float32))
    v_rows = dev(rng.standard_normal((B, R, Hkv, D), dtype=np.float32))
    q_chunk = dev(rng.standard_normal((B, R, Hq, D), dtype=np.float32))
    q_step = dev(rng.standard_normal((B, Hq, D), dtype=np.float32))
    k_new = dev(rng.standard_normal((B, Hkv, D), dtype=np.float32))
    v_new = dev(rng.standard_normal((B, Hkv, D), dtype=np.float32))
    out_chunk = torch.empty_like(q_chunk)
    out_fused = torch.empty_like(q_chunk)
    out_step = torch.empty_like(q_step)
    sh = caches.shape
    ws = torch.empty(max(ka.prefill_workspace_bytes(sh, R), ka.decode_workspace_bytes(sh, pos + 1), 1),
                     dtype=torch.uint8, device="cuda")
    ws_fused = torch.empty(max(ka.append_prefill_workspace_bytes(sh, R), 1), dtype=torch.uint8,
                           device="cuda")

    def calls():
        # every call writes the same cache rows from the same inputs, so
        # repeating the sequence leaves the caches as one pass does
        ka.append_kv(sh, caches.k, caches.v, k_rows, v_rows, start, R)
        ka.prefill_chunk(sh, q_chunk, caches.k, caches.v, out_chunk, start, R, 1 / 16, ws)
        ka.append_prefill_chunk(sh, q_chunk, k_rows, v_rows, caches.k, caches.v, out_fused, start, R,
                                1 / 16, ws_fused)
        ka.decode_step(sh, q_step, k_new, v_new, caches.k, caches.v, out_step, [pos], 1 / 16, ws)

    def eager():
        calls()
        torch.cuda.synchronize()
        # the fused call gives the two calls' result bit for bit
        assert torch.equal(out_fused.view(torch.int32), out_chunk.view(torch.int32))
        return out_chunk.clone(), out_step.clone()

    want_chunk, want_step = eager()         # also runs the int8 self-test before capture
    assert torch.isfinite(want_chunk).all() and torch.isfinite(want_step).all()

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g):
            calls()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    def check_replays(want_c, want_s, n=3):
        for i in range(n):
            out_chunk.fill_(float("nan"))
            out_fused.fill_(float("nan"))
            out_step.fill_(float("nan"))
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out_chunk.view(torch.int32), want_c.view(torch.int32)), f"replay {i}"
            assert torch.equal(out_fused.view(torch.int32), want_c.view(torch.int32)), f"replay {i}"
            assert torch.equal(out_step.view(torch.int32), want_s.view(torch.int32)), f"replay {i}"
            # the program's own eager work between replays
            x = torch.randn(512, 512, device="cuda")
            (x @ x).sum().item()

    check_replays(want_chunk, want_step)

    # new query rows in the captured input tensors: the graph reads them live
    q_chunk.copy_(dev(rng.standard_normal((B, R, Hq, D), dtype=np.float32)))
    q_step.copy_(dev(rng.standard_normal((B, Hq, D), dtype=np.float32)))
    want_chunk2, want_step2 = eager()
    assert not torch.equal(want_chunk2, want_chunk)
    check_replays(want_chunk2, want_step2)
