"""Python binding of libka_attn: grouped-query causal KV-cache attention on
MI355X (gfx950).

Thin ctypes marshalling over the C ABI in ``include/ka_attn.h``: each
function takes torch tensors that live on the GPU, checks dtype / size /
contiguity, and passes raw device pointers and the current HIP stream to the
library.  Every step of the computation runs in the library's HIP kernels;
there is no fallback.  If the shared library is missing the import of this
module still works but every call raises ``KaAttnUnavailable``.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

__all__ = ["Shape", "KaAttnError", "KaAttnUnavailable", "lib", "lib_path", "F32", "BF16",
           "cache_bytes", "alloc_cache", "append_kv", "prefill_workspace_bytes",
           "prefill_workspace_need", "prefill_chunk", "decode_workspace_bytes", "decode", "status_string",
           "last_error", "abi_version", "EXPORTED_SYMBOLS", "decode_step", "append_kv_rope",
           "rope_rows", "append_kv_ragged", "prefill_ragged_workspace_bytes",
           "prefill_ragged_workspace_need", "prefill_ragged",
           "Memory", "session_memory", "cache_resize", "I8K", "int8_self_test",
           "decode_step_noalloc", "decode_step_noalloc_max_bytes", "append_prefill_chunk",
           "append_prefill_workspace_bytes", "append_prefill_workspace_need"]

F32 = 0
BF16 = 1
I8K = 2

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libka_attn.so"

EXPORTED_SYMBOLS = (
    "ka_attn_abi_version", "ka_attn_cache_bytes", "ka_attn_append_kv", "ka_attn_append_kv_rope",
    "ka_attn_rope_rows",
    "ka_attn_prefill_workspace_bytes", "ka_attn_prefill_workspace_need", "ka_attn_prefill_chunk",
    "ka_attn_append_prefill_chunk", "ka_attn_append_prefill_workspace_bytes",
    "ka_attn_append_prefill_workspace_need",
    "ka_attn_decode_workspace_bytes", "ka_attn_decode", "ka_attn_decode_step",
    "ka_attn_decode_step_noalloc", "ka_attn_decode_step_noalloc_max_bytes",
    "ka_attn_append_kv_ragged", "ka_attn_prefill_ragged_workspace_bytes",
    "ka_attn_prefill_ragged_workspace_need", "ka_attn_prefill_ragged",
    "ka_attn_session_memory", "ka_attn_cache_resize", "ka_attn_int8_self_test",
    "ka_attn_status_string",
    "ka_attn_last_error",
)

STATUS = {0: "KA_OK", 1: "KA_ERR_INVALID_ARGUMENT", 2: "KA_ERR_OUT_OF_RANGE",
          3: "KA_ERR_UNSUPPORTED", 4: "KA_ERR_WORKSPACE", 5: "KA_ERR_HIP"}


class KaAttnUnavailable(RuntimeError):
    """The compiled library is not present (build it first)."""


class KaAttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status
        self.message = message


class Shape(ctypes.Structure):
    """Mirror of ka_attn_shape."""
    _fields_ = [("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("capacity", ctypes.c_int32), ("kv_dtype", ctypes.c_int32)]

    def __init__(self, batch, num_q_heads, num_kv_heads, head_dim, capacity, kv_dtype):
        if isinstance(kv_dtype, str):
            kv_dtype = {"f32": F32, "bf16": BF16, "i8k": I8K}[kv_dtype]
        super().__init__(int(batch), int(num_q_heads), int(num_kv_heads), int(head_dim),
                         int(capacity), int(kv_dtype))

    def __repr__(self):
        return (f"Shape(batch={self.batch}, Hq={self.num_q_heads}, Hkv={self.num_kv_heads}, "
                f"D={self.head_dim}, C={self.capacity}, "
                f"kv={ {F32: 'f32', BF16: 'bf16', I8K: 'i8k'}.get(self.kv_dtype, self.kv_dtype)})")


_lib = None


def lib_path() -> str:
    return os.environ.get("KA_ATTN_LIB", os.path.join(_HERE, _LIB_NAME))


def lib() -> ctypes.CDLL:
    """Loads (once) and returns the shared library."""
    global _lib
    if _lib is not None:
        return _lib
    path = lib_path()
    if not os.path.exists(path):
        raise KaAttnUnavailable(
            f"{path} not found; build it with `python -m kv_cache_attention_amd.build`")
    L = ctypes.CDLL(path)
    c_void_p, c_int32, c_size_t, c_float = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float
    P = ctypes.POINTER(Shape)
    L.ka_attn_abi_version.restype = c_int32
    L.ka_attn_abi_version.argtypes = []
    L.ka_attn_cache_bytes.restype = c_size_t
    L.ka_attn_cache_bytes.argtypes = [P]
    L.ka_attn_append_kv.restype = c_int32
    L.ka_attn_append_kv.argtypes = [P, c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_void_p]
    L.ka_attn_prefill_workspace_bytes.restype = c_size_t
    L.ka_attn_append_kv_rope.argtypes = [P, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                         c_void_p, c_int32, c_int32, c_void_p]
    L.ka_attn_append_kv_rope.restype = c_int32
    L.ka_attn_rope_rows.argtypes = [P, c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_void_p]
    L.ka_attn_rope_rows.restype = c_int32
    L.ka_attn_prefill_workspace_bytes.argtypes = [P, c_int32]
    L.ka_attn_prefill_workspace_need.restype = c_size_t
    L.ka_attn_prefill_workspace_need.argtypes = [P, c_int32, c_int32]
    L.ka_attn_prefill_chunk.restype = c_int32
    L.ka_attn_prefill_chunk.argtypes = [P, c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_int32,
                                        c_float, c_void_p, c_size_t, c_void_p]
    L.ka_attn_append_prefill_chunk.restype = c_int32
    L.ka_attn_append_prefill_chunk.argtypes = [P, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                               c_void_p, c_int32, c_int32, ctypes.c_float,
                                               c_void_p, c_size_t, c_void_p]
    L.ka_attn_append_prefill_workspace_bytes.restype = c_size_t
    L.ka_attn_append_prefill_workspace_bytes.argtypes = [P, c_int32]
    L.ka_attn_append_prefill_workspace_need.restype = c_size_t
    L.ka_attn_append_prefill_workspace_need.argtypes = [P, c_int32, c_int32]
    L.ka_attn_decode_workspace_bytes.restype = c_size_t
    L.ka_attn_decode_workspace_bytes.argtypes = [P, c_int32]
    L.ka_attn_decode.restype = c_int32
    L.ka_attn_decode.argtypes = [P, c_void_p, c_void_p, c_void_p, c_void_p,
                                 ctypes.POINTER(c_int32), c_float, c_void_p, c_size_t, c_void_p]
    L.ka_attn_decode_step.restype = c_int32
    L.ka_attn_decode_step.argtypes = [P, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                      c_void_p, ctypes.POINTER(c_int32), ctypes.c_float,
                                      c_void_p, c_size_t, c_void_p]
    L.ka_attn_decode_step_noalloc.restype = c_int32
    L.ka_attn_decode_step_noalloc.argtypes = [P, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                              c_void_p, ctypes.POINTER(c_int32), ctypes.c_float,
                                              c_void_p]
    L.ka_attn_decode_step_noalloc_max_bytes.restype = c_size_t
    L.ka_attn_decode_step_noalloc_max_bytes.argtypes = []
    I32P = ctypes.POINTER(c_int32)
    L.ka_attn_append_kv_ragged.restype = c_int32
    L.ka_attn_append_kv_ragged.argtypes = [P, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                           c_void_p, I32P, I32P, c_void_p]
    L.ka_attn_prefill_ragged_workspace_bytes.restype = c_size_t
    L.ka_attn_prefill_ragged_workspace_bytes.argtypes = [P, ctypes.c_int64]
    L.ka_attn_prefill_ragged_workspace_need.restype = c_size_t
    L.ka_attn_prefill_ragged_workspace_need.argtypes = [P, I32P, I32P]
    L.ka_attn_prefill_ragged.restype = c_int32
    L.ka_attn_prefill_ragged.argtypes = [P, c_void_p, c_void_p, c_void_p, c_void_p, I32P, I32P,
                                         ctypes.c_float, c_void_p, c_size_t, c_void_p]
    L.ka_attn_session_memory.restype = c_int32
    L.ka_attn_session_memory.argtypes = [P, c_int32, ctypes.POINTER(Memory)]
    L.ka_attn_cache_resize.restype = c_int32
    L.ka_attn_cache_resize.argtypes = [P, c_void_p, c_void_p, P, c_void_p, c_void_p, c_int32,
                                       c_void_p]
    L.ka_attn_int8_self_test.restype = c_int32
    L.ka_attn_int8_self_test.argtypes = []
    L.ka_attn_status_string.restype = ctypes.c_char_p
    L.ka_attn_status_string.argtypes = [c_int32]
    L.ka_attn_last_error.restype = ctypes.c_char_p
    L.ka_attn_last_error.argtypes = []
    _lib = L
    return L


class Memory(ctypes.Structure):
    """ka_attn_memory: what a session window costs (bytes)."""
    _fields_ = [("cache_bytes", ctypes.c_size_t), ("prefill_workspace_bytes", ctypes.c_size_t),
                ("decode_workspace_bytes", ctypes.c_size_t), ("chunk_io_bytes", ctypes.c_size_t),
                ("total_bytes", ctypes.c_size_t)]


def abi_version() -> int:
    return int(lib().ka_attn_abi_version())


def status_string(status: int) -> str:
    return lib().ka_attn_status_string(int(status)).decode()


def last_error() -> str:
    return lib().ka_attn_last_error().decode()


def _check(status: int):
    if status != 0:
        raise KaAttnError(status, last_error())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    return ctypes.c_void_p(handle)


def _need(t: torch.Tensor, name: str, dtype, numel: Optional[int] = None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must live on the GPU (got {t.device})")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")


def cache_bytes(shape: Shape) -> int:
    return int(lib().ka_attn_cache_bytes(ctypes.byref(shape)))


def alloc_cache(shape: Shape, device="cuda", fill_byte: Optional[int] = None) -> torch.Tensor:
    """A byte tensor sized for one cache buffer (K or V) of ``shape``."""
    n = cache_bytes(shape)
    if n == 0:
        raise KaAttnError(1, last_error())
    t = torch.empty(n, dtype=torch.uint8, device=device)
    if fill_byte is not None:
        t.fill_(int(fill_byte))
    return t


def append_kv(shape: Shape, k_cache: torch.Tensor, v_cache: torch.Tensor,
              k_new: torch.Tensor, v_new: torch.Tensor, start_pos: int, row_count: int,
              stream=None) -> None:
    n = shape.batch * row_count * shape.num_kv_heads * shape.head_dim
    for t, nm in ((k_new, "k_new"), (v_new, "v_new")):
        _need(t, nm, torch.float32, n)
    cb = cache_bytes(shape)
    for t, nm in ((k_cache, "k_cache"), (v_cache, "v_cache")):
        _need(t, nm, None)
        if t.numel() * t.element_size() < cb:
            raise ValueError(f"{nm} is smaller than {cb} bytes")
    _check(lib().ka_attn_append_kv(ctypes.byref(shape), _ptr(k_cache), _ptr(v_cache),
                                   _ptr(k_new), _ptr(v_new), int(start_pos), int(row_count),
                                   _stream(stream)))


def append_kv_rope(shape: Shape, k_cache: torch.Tensor, v_cache: torch.Tensor,
                   k_new: torch.Tensor, v_new: torch.Tensor, rope_cos: torch.Tensor,
                   rope_sin: torch.Tensor, start_pos: int, row_count: int, stream=None) -> None:
    """ka_attn_append_kv_rope: rope_cos / rope_sin f32 [row_count][head_dim / 2]."""
    n = shape.batch * row_count * shape.num_kv_heads * shape.head_dim
    for t, nm in ((k_new, "k_new"), (v_new, "v_new")):
        _need(t, nm, torch.float32, n)
    for t, nm in ((rope_cos, "rope_cos"), (rope_sin, "rope_sin")):
        _need(t, nm, torch.float32, row_count * (shape.head_dim // 2))
    cb = cache_bytes(shape)
    for t, nm in ((k_cache, "k_cache"), (v_cache, "v_cache")):
        _need(t, nm, None)
        if t.numel() * t.element_size() < cb:
            raise ValueError(f"{nm} is smaller than {cb} bytes")
    _check(lib().ka_attn_append_kv_rope(ctypes.byref(shape), _ptr(k_cache), _ptr(v_cache),
                                        _ptr(k_new), _ptr(v_new), _ptr(rope_cos), _ptr(rope_sin),
                                        int(start_pos), int(row_count), _stream(stream)))


def rope_rows(shape: Shape, x: torch.Tensor, y: torch.Tensor, rope_cos: torch.Tensor,
              rope_sin: torch.Tensor, row_count: int, stream=None) -> None:
    """ka_attn_rope_rows: x, y f32 [batch][row_count][num_q_heads][head_dim] (y may be x)."""
    n = shape.batch * row_count * shape.num_q_heads * shape.head_dim
    _need(x, "x", torch.float32, n)
    _need(y, "y", torch.float32, n)
    for t, nm in ((rope_cos, "rope_cos"), (rope_sin, "rope_sin")):
        _need(t, nm, torch.float32, row_count * (shape.head_dim // 2))
    _check(lib().ka_attn_rope_rows(ctypes.byref(shape), _ptr(x), _ptr(y), _ptr(rope_cos),
                                   _ptr(rope_sin), int(row_count), _stream(stream)))


def prefill_workspace_bytes(shape: Shape, max_rows: int) -> int:
    return int(lib().ka_attn_prefill_workspace_bytes(ctypes.byref(shape), int(max_rows)))


def prefill_workspace_need(shape: Shape, start_pos: int, row_count: int) -> int:
    return int(lib().ka_attn_prefill_workspace_need(ctypes.byref(shape), int(start_pos),
                                                    int(row_count)))


def prefill_chunk(shape: Shape, q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                  out: torch.Tensor, start_pos: int, row_count: int, scale: float,
                  workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    n = shape.batch * row_count * shape.num_q_heads * shape.head_dim
    _need(q, "q", torch.float32, n)
    _need(out, "out", torch.float32, n)
    ws_bytes = 0
    if workspace is not None:
        _need(workspace, "workspace", None)
        ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().ka_attn_prefill_chunk(ctypes.byref(shape), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                       _ptr(out), int(start_pos), int(row_count), float(scale),
                                       _ptr(workspace), ws_bytes, _stream(stream)))


def append_prefill_workspace_bytes(shape: Shape, max_rows: int) -> int:
    return int(lib().ka_attn_append_prefill_workspace_bytes(ctypes.byref(shape), int(max_rows)))


def append_prefill_workspace_need(shape: Shape, start_pos: int, row_count: int) -> int:
    return int(lib().ka_attn_append_prefill_workspace_need(ctypes.byref(shape), int(start_pos),
                                                           int(row_count)))


def append_prefill_chunk(shape: Shape, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                         k_cache: torch.Tensor, v_cache: torch.Tensor, out: torch.Tensor,
                         start_pos: int, row_count: int, scale: float,
                         workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """ka_attn_append_prefill_chunk: append_kv then prefill_chunk in one call."""
    n = shape.batch * row_count * shape.num_q_heads * shape.head_dim
    _need(q, "q", torch.float32, n)
    _need(out, "out", torch.float32, n)
    nk = shape.batch * row_count * shape.num_kv_heads * shape.head_dim
    for t, nm in ((k_new, "k_new"), (v_new, "v_new")):
        _need(t, nm, torch.float32, nk)
    cb = cache_bytes(shape)
    for t, nm in ((k_cache, "k_cache"), (v_cache, "v_cache")):
        _need(t, nm, None)
        if t.numel() * t.element_size() < cb:
            raise ValueError(f"{nm} is smaller than {cb} bytes")
    ws_bytes = 0
    if workspace is not None:
        _need(workspace, "workspace", None)
        ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().ka_attn_append_prefill_chunk(ctypes.byref(shape), _ptr(q), _ptr(k_new),
                                              _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(out),
                                              int(start_pos), int(row_count), float(scale),
                                              _ptr(workspace), ws_bytes, _stream(stream)))


def decode_workspace_bytes(shape: Shape, max_ctx_len: int) -> int:
    return int(lib().ka_attn_decode_workspace_bytes(ctypes.byref(shape), int(max_ctx_len)))


def decode(shape: Shape, q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
           out: torch.Tensor, ctx_len: Sequence[int], scale: float,
           workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    n = shape.batch * shape.num_q_heads * shape.head_dim
    _need(q, "q", torch.float32, n)
    _need(out, "out", torch.float32, n)
    if len(ctx_len) != shape.batch:
        raise ValueError(f"ctx_len has {len(ctx_len)} entries, expected {shape.batch}")
    arr = (ctypes.c_int32 * shape.batch)(*[int(c) for c in ctx_len])
    ws_bytes = 0
    if workspace is not None:
        _need(workspace, "workspace", None)
        ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().ka_attn_decode(ctypes.byref(shape), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                _ptr(out), arr, float(scale), _ptr(workspace), ws_bytes,
                                _stream(stream)))


def decode_step(shape: Shape, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                k_cache: torch.Tensor, v_cache: torch.Tensor, out: torch.Tensor,
                pos: Sequence[int], scale: float, workspace: Optional[torch.Tensor] = None,
                stream=None) -> None:
    """Append one K/V row per session at pos[b] and decode the query there
    (ka_attn_decode_step).  k_new, v_new: f32 [B][Hkv][D]; q, out: [B][Hq][D]."""
    n = shape.batch * shape.num_q_heads * shape.head_dim
    nk = shape.batch * shape.num_kv_heads * shape.head_dim
    _need(q, "q", torch.float32, n)
    _need(out, "out", torch.float32, n)
    _need(k_new, "k_new", torch.float32, nk)
    _need(v_new, "v_new", torch.float32, nk)
    if len(pos) != shape.batch:
        raise ValueError(f"pos has {len(pos)} entries, expected {shape.batch}")
    arr = (ctypes.c_int32 * shape.batch)(*[int(p) for p in pos])
    ws_bytes = 0
    if workspace is not None:
        _need(workspace, "workspace", None)
        ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().ka_attn_decode_step(ctypes.byref(shape), _ptr(q), _ptr(k_new), _ptr(v_new),
                                     _ptr(k_cache), _ptr(v_cache), _ptr(out), arr, float(scale),
                                     _ptr(workspace), ws_bytes, _stream(stream)))


def decode_step_noalloc_max_bytes() -> int:
    return int(lib().ka_attn_decode_step_noalloc_max_bytes())


def decode_step_noalloc(shape: Shape, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                        k_cache: torch.Tensor, v_cache: torch.Tensor, out: torch.Tensor,
                        pos: Sequence[int], scale: float, stream=None) -> None:
    """decode_step without a workspace (ka_attn_decode_step_noalloc): the
    partials go to the library's own per-device scratch array."""
    n = shape.batch * shape.num_q_heads * shape.head_dim
    nk = shape.batch * shape.num_kv_heads * shape.head_dim
    _need(q, "q", torch.float32, n)
    _need(out, "out", torch.float32, n)
    _need(k_new, "k_new", torch.float32, nk)
    _need(v_new, "v_new", torch.float32, nk)
    if len(pos) != shape.batch:
        raise ValueError(f"pos has {len(pos)} entries, expected {shape.batch}")
    arr = (ctypes.c_int32 * shape.batch)(*[int(p) for p in pos])
    _check(lib().ka_attn_decode_step_noalloc(ctypes.byref(shape), _ptr(q), _ptr(k_new),
                                             _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(out),
                                             arr, float(scale), _stream(stream)))


def _int32_array(xs: Sequence[int], n: int, name: str):
    if len(xs) != n:
        raise ValueError(f"{name} has {len(xs)} entries, expected {n}")
    return (ctypes.c_int32 * n)(*[int(x) for x in xs])


def append_kv_ragged(shape: Shape, k_cache: torch.Tensor, v_cache: torch.Tensor,
                     k_new: torch.Tensor, v_new: torch.Tensor, start_pos: Sequence[int],
                     row_count: Sequence[int], rope_cos: Optional[torch.Tensor] = None,
                     rope_sin: Optional[torch.Tensor] = None, stream=None) -> None:
    """ka_attn_append_kv_ragged: k_new / v_new f32 [sum row_count][Hkv][D], rows
    packed session by session; rope_cos / rope_sin None or [sum row_count][D/2]."""
    st = _int32_array(start_pos, shape.batch, "start_pos")
    rc = _int32_array(row_count, shape.batch, "row_count")
    total = sum(int(r) for r in row_count)
    n = total * shape.num_kv_heads * shape.head_dim
    for t, nm in ((k_new, "k_new"), (v_new, "v_new")):
        _need(t, nm, torch.float32, n)
    if rope_cos is not None or rope_sin is not None:
        for t, nm in ((rope_cos, "rope_cos"), (rope_sin, "rope_sin")):
            _need(t, nm, torch.float32, total * (shape.head_dim // 2))
    cb = cache_bytes(shape)
    for t, nm in ((k_cache, "k_cache"), (v_cache, "v_cache")):
        _need(t, nm, None)
        if t.numel() * t.element_size() < cb:
            raise ValueError(f"{nm} is smaller than {cb} bytes")
    _check(lib().ka_attn_append_kv_ragged(ctypes.byref(shape), _ptr(k_cache), _ptr(v_cache),
                                          _ptr(k_new), _ptr(v_new), _ptr(rope_cos), _ptr(rope_sin),
                                          st, rc, _stream(stream)))


def prefill_ragged_workspace_bytes(shape: Shape, max_total_rows: int) -> int:
    return int(lib().ka_attn_prefill_ragged_workspace_bytes(ctypes.byref(shape), int(max_total_rows)))


def prefill_ragged_workspace_need(shape: Shape, start_pos: Sequence[int],
                                  row_count: Sequence[int]) -> int:
    return int(lib().ka_attn_prefill_ragged_workspace_need(
        ctypes.byref(shape), _int32_array(start_pos, shape.batch, "start_pos"),
        _int32_array(row_count, shape.batch, "row_count")))


def prefill_ragged(shape: Shape, q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                   out: torch.Tensor, start_pos: Sequence[int], row_count: Sequence[int],
                   scale: float, workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """ka_attn_prefill_ragged: q / out f32 [sum row_count][Hq][D], rows packed
    session by session."""
    st = _int32_array(start_pos, shape.batch, "start_pos")
    rc = _int32_array(row_count, shape.batch, "row_count")
    n = sum(int(r) for r in row_count) * shape.num_q_heads * shape.head_dim
    _need(q, "q", torch.float32, n)
    _need(out, "out", torch.float32, n)
    ws_bytes = 0
    if workspace is not None:
        _need(workspace, "workspace", None)
        ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().ka_attn_prefill_ragged(ctypes.byref(shape), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                        _ptr(out), st, rc, float(scale), _ptr(workspace), ws_bytes,
                                        _stream(stream)))


def session_memory(shape: Shape, max_chunk_rows: int) -> Memory:
    """ka_attn_session_memory: the bytes a window of shape.capacity costs."""
    m = Memory()
    _check(lib().ka_attn_session_memory(ctypes.byref(shape), int(max_chunk_rows), ctypes.byref(m)))
    return m


def cache_resize(src: Shape, src_k: torch.Tensor, src_v: torch.Tensor, dst: Shape,
                 dst_k: torch.Tensor, dst_v: torch.Tensor, rows: int, stream=None) -> None:
    """ka_attn_cache_resize: copy positions 0 .. rows - 1 into caches of another capacity."""
    for t, nm, sh in ((src_k, "src_k", src), (src_v, "src_v", src), (dst_k, "dst_k", dst),
                      (dst_v, "dst_v", dst)):
        _need(t, nm, None)
        if t.numel() * t.element_size() < cache_bytes(sh):
            raise ValueError(f"{nm} is smaller than {cache_bytes(sh)} bytes")
    _check(lib().ka_attn_cache_resize(ctypes.byref(src), _ptr(src_k), _ptr(src_v), ctypes.byref(dst),
                                      _ptr(dst_k), _ptr(dst_v), int(rows), _stream(stream)))


def int8_self_test() -> None:
    """ka_attn_int8_self_test: raises KaAttnError if the device's int8 scores
    are not sane."""
    _check(lib().ka_attn_int8_self_test())
