"""Device-side helpers for the GPU tests: a set of caches plus thin wrappers
that move numpy inputs to the GPU, call the library and bring results back."""
import numpy as np
import torch

import kv_cache_attention_amd as ka
from tests.cache_layout import logical_values, unpack_k, unpack_k_i8, unpack_v

POISON = 0xFF   # every byte 0xFF: a NaN in both f32 and bf16


def dev(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda")


class DevCaches:
    def __init__(self, B, Hq, Hkv, D, C, kv_dtype, poison=True):
        if isinstance(kv_dtype, str):
            kv_dtype = {"f32": ka.F32, "bf16": ka.BF16, "i8k": ka.I8K}[kv_dtype]
        self.B, self.Hq, self.Hkv, self.D, self.C, self.dt = B, Hq, Hkv, D, C, kv_dtype
        self.shape = ka.Shape(B, Hq, Hkv, D, C, kv_dtype)
        fill = POISON if poison else 0
        self.k = ka.alloc_cache(self.shape, fill_byte=fill)
        self.v = ka.alloc_cache(self.shape, fill_byte=fill)
        self._ws = None

    def workspace(self, nbytes):
        if nbytes == 0:
            return None
        if self._ws is None or self._ws.numel() < nbytes:
            self._ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        return self._ws

    def append(self, k_rows, v_rows, start):
        """k_rows / v_rows: [B][R][Hkv][D] float32."""
        R = k_rows.shape[1]
        ka.append_kv(self.shape, self.k, self.v, dev(k_rows), dev(v_rows), start, R)

    def append_rope(self, k_rows, v_rows, cos, sin, start):
        """As append, with K rows rotated by cos / sin ([R][D/2] float32)."""
        R = k_rows.shape[1]
        ka.append_kv_rope(self.shape, self.k, self.v, dev(k_rows), dev(v_rows), dev(cos), dev(sin),
                          start, R)

    def append_dev(self, k_rows_t, v_rows_t, start, R):
        ka.append_kv(self.shape, self.k, self.v, k_rows_t, v_rows_t, start, R)

    def prefill(self, q, start, scale, sync=True):
        """q: [B][R][Hq][D] float32 -> out numpy [B][R][Hq][D]."""
        R = q.shape[1]
        qt = dev(q)
        out = torch.full_like(qt, float("nan"))
        ws = self.workspace(ka.prefill_workspace_bytes(self.shape, R))
        ka.prefill_chunk(self.shape, qt, self.k, self.v, out, start, R, scale, ws)
        if sync:
            torch.cuda.synchronize()
        return out.cpu().numpy()

    def append_prefill(self, q, k_rows, v_rows, start, scale):
        """ka_attn_append_prefill_chunk: the chunk's K / V rows appended and its
        q rows ([B][R][Hq][D] float32) attended, in one call -> out numpy."""
        R = q.shape[1]
        qt = dev(q)
        out = torch.full_like(qt, float("nan"))
        ws = self.workspace(ka.append_prefill_workspace_bytes(self.shape, R))
        ka.append_prefill_chunk(self.shape, qt, dev(k_rows), dev(v_rows), self.k, self.v, out,
                                start, R, scale, ws)
        torch.cuda.synchronize()
        return out.cpu().numpy()

    def decode(self, q, ctx, scale):
        """q: [B][Hq][D] float32, ctx: list of B ints -> out numpy [B][Hq][D]."""
        qt = dev(q)
        out = torch.full_like(qt, float("nan"))
        ws = self.workspace(ka.decode_workspace_bytes(self.shape, max(ctx)))
        ka.decode(self.shape, qt, self.k, self.v, out, list(ctx), scale, ws)
        torch.cuda.synchronize()
        return out.cpu().numpy()

    def decode_step(self, q, k_new, v_new, pos, scale):
        """q: [B][Hq][D], k_new / v_new: [B][Hkv][D] float32 -> out [B][Hq][D]."""
        qt = dev(q)
        out = torch.full_like(qt, float("nan"))
        ws = self.workspace(ka.decode_workspace_bytes(self.shape, max(pos) + 1))
        ka.decode_step(self.shape, qt, dev(k_new), dev(v_new), self.k, self.v, out, list(pos),
                       scale, ws)
        torch.cuda.synchronize()
        return out.cpu().numpy()

    def raw(self):
        torch.cuda.synchronize()
        return self.k.cpu().numpy(), self.v.cpu().numpy()

    def logical(self):
        """Cache contents as f32 values [B][C][Hkv][D] (K, V)."""
        rk, rv = self.raw()
        a = (self.B, self.Hkv, self.C, self.D, self.dt_name)
        return (logical_values(rk, *a, "k"), logical_values(rv, *a, "v"))

    def bits(self):
        """Cache contents as raw element bit patterns [B][Hkv][C][D]."""
        rk, rv = self.raw()
        a = (self.B, self.Hkv, self.C, self.D, self.dt_name)
        return unpack_k(rk, *a), unpack_v(rv, *a)

    def k_i8(self):
        """int8-K caches: K codes [B][Hkv][C][D] and row scales [B][Hkv][C]."""
        rk, _ = self.raw()
        return unpack_k_i8(rk, self.B, self.Hkv, self.C, self.D)

    def v_bits(self):
        """V element bit patterns [B][Hkv][C][D] (bf16 layout for int8-K caches)."""
        _, rv = self.raw()
        return unpack_v(rv, self.B, self.Hkv, self.C, self.D, "f32" if self.dt == ka.F32 else "bf16")

    @property
    def dt_name(self):
        return {ka.BF16: "bf16", ka.F32: "f32", ka.I8K: "i8k"}[self.dt]
