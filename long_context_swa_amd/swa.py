"""Python binding of libswa (include/swa.h): argument marshalling only.

Every function here has the name of the C entry point it calls and does nothing but convert
arguments (torch tensors -> device pointers, streams -> hipStream_t, Python ints -> C ints) and
raise ``SwaError`` on a negative return code.  All attention, pool and planning work runs in the
native library; there is no fallback: importing this package fails loudly when the library has not
been built (``python -m long_context_swa_amd.build``).

torch is used only for device memory (the caller's tensors, the pool arena, the workspace) and
for streams.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libswa.so")
if not os.path.exists(_LIB_PATH):
    raise ImportError(
        f"libswa.so not found at {_LIB_PATH}; build it with `python -m long_context_swa_amd.build`")
_lib = ctypes.CDLL(_LIB_PATH)

SWA_F32, SWA_BF16, SWA_FP8_E4M3 = 0, 1, 2
SWA_ROPE_PAIRS, SWA_ROPE_HALVES = 0, 1
SWA_PLAN_UNIFORM, SWA_PLAN_BUCKETED = 0, 1
SWA_OK, SWA_EINVAL, SWA_ENOSEQ, SWA_ENOMEM, SWA_EHIP = 0, -1, -2, -3, -4
_CODE_NAMES = {SWA_EINVAL: "SWA_EINVAL", SWA_ENOSEQ: "SWA_ENOSEQ", SWA_ENOMEM: "SWA_ENOMEM",
               SWA_EHIP: "SWA_EHIP"}

EXPORTS = [
    "kvpool_arena_bytes", "kvpool_create", "kvpool_destroy", "kvpool_seq_open", "kvpool_seq_close",
    "kvpool_window_safe_len", "kvpool_seq_fork", "kvpool_snapshot", "kvpool_seq_fork_snapshot",
    "kvpool_snapshot_len", "kvpool_snapshot_release", "kvpool_append", "kvpool_append_batch", "kvpool_rope",
    "kvpool_seq_len",
    "kvpool_bytes",
    "kvpool_layer_is_full", "kvpool_free_pages", "kvpool_locate", "kvpool_slot_tags",
    "swa_attn_prefill", "swa_attn_decode", "full_attn", "full_attn_noalloc", "swa_attn_workspace_bytes",
    "swa_last_error",
    "swa_clock_probe",
]


class SwaError(RuntimeError):
    def __init__(self, code: int, fn: str):
        self.code = code
        msg = _lib.swa_last_error().decode(errors="replace")
        super().__init__(f"{fn}: {_CODE_NAMES.get(code, code)}: {msg}")


class swa_pool_desc(ctypes.Structure):
    _fields_ = [
        ("n_layers", ctypes.c_int32),
        ("layer_is_full", ctypes.POINTER(ctypes.c_uint8)),
        ("window", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("page_tokens", ctypes.c_int32),
        ("pages_per_full_layer", ctypes.c_int64),
        ("max_seqs", ctypes.c_int32),
        ("max_seq_len", ctypes.c_int64),
        ("max_snapshots", ctypes.c_int32),
        ("k_scale", ctypes.c_float),
        ("v_scale", ctypes.c_float),
        ("rope_base", ctypes.c_float),
        ("rope_style", ctypes.c_int32),
        ("decode_plan", ctypes.c_int32),
        ("rope_fused", ctypes.c_int32),
        ("max_chunk", ctypes.c_int32),
    ]


_P = ctypes.c_void_p
_i32, _i64 = ctypes.c_int32, ctypes.c_int64
_pi32, _pi64 = ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64)
_SIGS = {
    "kvpool_arena_bytes": (_i64, [ctypes.POINTER(swa_pool_desc)]),
    "kvpool_create": (ctypes.c_int, [ctypes.POINTER(swa_pool_desc), _P, _i64, ctypes.POINTER(_P)]),
    "kvpool_destroy": (ctypes.c_int, [_P]),
    "kvpool_seq_open": (ctypes.c_int, [_P, _pi32]),
    "kvpool_seq_close": (ctypes.c_int, [_P, _i32]),
    "kvpool_window_safe_len": (ctypes.c_int, [_P, _i32, _i64, _pi64]),
    "kvpool_seq_fork": (ctypes.c_int, [_P, _i32, _i64, _pi32, _P]),
    "kvpool_snapshot": (ctypes.c_int, [_P, _i32, _pi32, _P]),
    "kvpool_seq_fork_snapshot": (ctypes.c_int, [_P, _i32, _pi32, _P]),
    "kvpool_snapshot_len": (ctypes.c_int, [_P, _i32, _pi64]),
    "kvpool_snapshot_release": (ctypes.c_int, [_P, _i32]),
    "kvpool_append": (ctypes.c_int, [_P, _i32, _i32, _P, _P, _i32, _P]),
    "kvpool_append_batch": (ctypes.c_int, [_P, _i32, _P, _i32, _P, _P, _i32, _P]),
    "kvpool_rope": (ctypes.c_int, [_P, _i32, _P, _i32, _P, _i32, _P, _i32, ctypes.c_int, _P]),
    "kvpool_seq_len": (ctypes.c_int, [_P, _i32, _i32, _pi64]),
    "kvpool_bytes": (ctypes.c_int, [_P, _pi64, _pi64]),
    "kvpool_layer_is_full": (ctypes.c_int, [_P, _i32]),
    "kvpool_free_pages": (ctypes.c_int, [_P, _i32, _pi64]),
    "kvpool_locate": (ctypes.c_int, [_P, _i32, _i32, _i64, _i32, _pi64, _pi64, _pi64]),
    "kvpool_slot_tags": (ctypes.c_int, [_P, _i32, _i32, _pi64]),
    "swa_attn_prefill": (ctypes.c_int, [_P, _i32, _i32, _P, _P, _P, _i32, _i32, ctypes.c_int, _P, _P]),
    "swa_attn_decode": (ctypes.c_int, [_P, _i32, _P, _i32, _P, _P, _P, _i32, _i32, ctypes.c_int, _P,
                                       _P, _i64, _P]),
    "full_attn": (ctypes.c_int, [_P, _i32, _P, _i32, _P, _P, _P, _i32, _i32, ctypes.c_int, _P, _P,
                                 _i64, _P]),
    "full_attn_noalloc": (ctypes.c_int, [_P, _i32, _P, _i32, _P, _P, _P, _i32, _i32, ctypes.c_int, _P, _P]),
    "swa_attn_workspace_bytes": (_i64, [_P, _i32, _P, _i32, _i32, _i32]),
    "swa_last_error": (ctypes.c_char_p, []),
    "swa_clock_probe": (ctypes.c_int, [_P, _i64, _P]),
}
for _name, (_res, _args) in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.restype, _f.argtypes = _res, _args


def _check(rc: int, fn: str) -> int:
    if rc < 0:
        raise SwaError(rc, fn)
    return rc


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)  # device index -> hipStream_t


def _stream(stream) -> int | None:
    if stream is None:
        # the current stream's handle; torch's raw accessor skips building a Stream object
        # (about 3 us per call), which matters for per-layer calls on small batches
        if _raw_stream is not None and torch.cuda.is_initialized():
            return _raw_stream(torch.cuda.current_device())
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _dt(dtype) -> int:
    if isinstance(dtype, int) and dtype in (SWA_F32, SWA_BF16, SWA_FP8_E4M3):
        return dtype
    if dtype == torch.float32:
        return SWA_F32
    if dtype == torch.bfloat16:
        return SWA_BF16
    if dtype == torch.float8_e4m3fn or dtype == "fp8_e4m3":
        return SWA_FP8_E4M3
    raise ValueError(f"unsupported dtype {dtype}")


class _I32:
    """Sequence-id list as an int32 buffer for the C ABI: a contiguous numpy int32 array is passed
    by pointer without a copy (building a ctypes array from a Python list costs tens of
    microseconds per call for a few hundred ids); anything else is converted once."""

    def __init__(self, xs):
        self.a = np.ascontiguousarray(xs, dtype=np.int32)
        self.ptr = self.a.__array_interface__["data"][0]  # passed as void*: data_as() costs ~5 us

    def __len__(self):
        return self.a.shape[0]


def _i32_array(xs):
    return _I32(xs)


def make_desc(n_layers, window, n_kv_heads, head_dim, kv_dtype, pages_per_full_layer, max_seqs,
              max_seq_len, layer_is_full=None, page_tokens=16, k_scale=1.0, v_scale=1.0, max_snapshots=0,
              rope_base=0.0, rope_style=SWA_ROPE_PAIRS, decode_plan=SWA_PLAN_UNIFORM, rope_fused=False,
              max_chunk=0):
    """Build a swa_pool_desc; ``layer_is_full`` None = the library's default hybrid map;
    ``kv_dtype`` torch.float32, torch.bfloat16 or torch.float8_e4m3fn (the scales apply to FP8
    pools); ``rope_base`` 0 = no RoPE tables, ``rope_style`` "pairs"/"halves" or SWA_ROPE_*;
    ``decode_plan`` "uniform"/"bucketed" or SWA_PLAN_*; ``rope_fused`` True = attention and commit
    calls take unrotated q/k and rotate them inside (needs ``max_chunk``, the longest prefill chunk).
    The returned object keeps the flag array alive."""
    d = swa_pool_desc()
    d.rope_base = rope_base
    d.rope_style = {"pairs": SWA_ROPE_PAIRS, "halves": SWA_ROPE_HALVES}.get(rope_style, rope_style)
    d.decode_plan = {"uniform": SWA_PLAN_UNIFORM, "bucketed": SWA_PLAN_BUCKETED}.get(decode_plan, decode_plan)
    d.k_scale, d.v_scale = k_scale, v_scale
    d.max_snapshots = max_snapshots
    d.rope_fused, d.max_chunk = int(bool(rope_fused)), max_chunk
    d.n_layers, d.window, d.n_kv_heads, d.head_dim = n_layers, window, n_kv_heads, head_dim
    d.kv_dtype, d.page_tokens = _dt(kv_dtype), page_tokens
    d.pages_per_full_layer, d.max_seqs, d.max_seq_len = pages_per_full_layer, max_seqs, max_seq_len
    if layer_is_full is not None:
        flags = (ctypes.c_uint8 * n_layers)(*[1 if f else 0 for f in layer_is_full])
        d._flags = flags
        d.layer_is_full = ctypes.cast(flags, ctypes.POINTER(ctypes.c_uint8))
    return d


def kvpool_arena_bytes(desc) -> int:
    return _check(_lib.kvpool_arena_bytes(ctypes.byref(desc)), "kvpool_arena_bytes")


def kvpool_create(desc, arena=None, arena_bytes: int | None = None) -> int:
    """Returns the pool handle.  ``arena`` None creates a planning pool (host metadata only)."""
    h = ctypes.c_void_p()
    nbytes = arena_bytes if arena_bytes is not None else (
        arena.numel() * arena.element_size() if arena is not None else 0)
    _check(_lib.kvpool_create(ctypes.byref(desc), _ptr(arena), nbytes, ctypes.byref(h)), "kvpool_create")
    return h.value


def kvpool_destroy(pool) -> None:
    _check(_lib.kvpool_destroy(pool), "kvpool_destroy")


def kvpool_seq_open(pool) -> int:
    s = ctypes.c_int32()
    _check(_lib.kvpool_seq_open(pool, ctypes.byref(s)), "kvpool_seq_open")
    return s.value


def kvpool_seq_close(pool, seq) -> None:
    _check(_lib.kvpool_seq_close(pool, seq), "kvpool_seq_close")


def kvpool_window_safe_len(pool, donor, match_len) -> int:
    out = ctypes.c_int64()
    _check(_lib.kvpool_window_safe_len(pool, donor, match_len, ctypes.byref(out)), "kvpool_window_safe_len")
    return out.value


def kvpool_seq_fork(pool, donor, reuse_len, stream=None) -> int:
    s = ctypes.c_int32()
    _check(_lib.kvpool_seq_fork(pool, donor, reuse_len, ctypes.byref(s), _stream(stream)), "kvpool_seq_fork")
    return s.value


def kvpool_snapshot(pool, seq, stream=None) -> int:
    out = ctypes.c_int32()
    _check(_lib.kvpool_snapshot(pool, seq, ctypes.byref(out), _stream(stream)), "kvpool_snapshot")
    return out.value


def kvpool_seq_fork_snapshot(pool, snap, stream=None) -> int:
    out = ctypes.c_int32()
    _check(_lib.kvpool_seq_fork_snapshot(pool, snap, ctypes.byref(out), _stream(stream)),
           "kvpool_seq_fork_snapshot")
    return out.value


def kvpool_snapshot_len(pool, snap) -> int:
    out = ctypes.c_int64()
    _check(_lib.kvpool_snapshot_len(pool, snap, ctypes.byref(out)), "kvpool_snapshot_len")
    return out.value


def kvpool_snapshot_release(pool, snap) -> None:
    _check(_lib.kvpool_snapshot_release(pool, snap), "kvpool_snapshot_release")


def kvpool_append(pool, seq, layer, k, v, n=None, stream=None) -> None:
    if n is None:
        n = k.shape[0]
    _check(_lib.kvpool_append(pool, seq, layer, _ptr(k), _ptr(v), n, _stream(stream)), "kvpool_append")


def kvpool_append_batch(pool, seqs, layer, k, v, n, stream=None) -> None:
    arr = _i32_array(seqs)
    _check(_lib.kvpool_append_batch(pool, len(arr), arr.ptr, layer, _ptr(k), _ptr(v), n, _stream(stream)),
           "kvpool_append_batch")


def kvpool_rope(pool, seqs, layer, q, n_q_heads, k, n, dtype=None, stream=None) -> None:
    """Rotate q [n_seqs, n, Hq, d] and/or k [n_seqs, n, Hkv, d] in place (either may be None)."""
    arr = _i32_array(seqs)
    t = q if q is not None else k
    _check(_lib.kvpool_rope(pool, len(arr), arr.ptr, layer, _ptr(q), n_q_heads, _ptr(k), n,
                            _dt(dtype if dtype is not None else t.dtype), _stream(stream)), "kvpool_rope")


def kvpool_seq_len(pool, seq, layer) -> int:
    out = ctypes.c_int64()
    _check(_lib.kvpool_seq_len(pool, seq, layer, ctypes.byref(out)), "kvpool_seq_len")
    return out.value


def kvpool_bytes(pool) -> tuple[int, int]:
    a, r = ctypes.c_int64(), ctypes.c_int64()
    _check(_lib.kvpool_bytes(pool, ctypes.byref(a), ctypes.byref(r)), "kvpool_bytes")
    return a.value, r.value


def kvpool_layer_is_full(pool, layer) -> bool:
    return bool(_check(_lib.kvpool_layer_is_full(pool, layer), "kvpool_layer_is_full"))


def kvpool_free_pages(pool, layer) -> int:
    out = ctypes.c_int64()
    _check(_lib.kvpool_free_pages(pool, layer, ctypes.byref(out)), "kvpool_free_pages")
    return out.value


def kvpool_locate(pool, seq, layer, pos, head) -> tuple[int, int, int]:
    k, v, s = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    _check(_lib.kvpool_locate(pool, seq, layer, pos, head, ctypes.byref(k), ctypes.byref(v), ctypes.byref(s)),
           "kvpool_locate")
    return k.value, v.value, s.value


def kvpool_slot_tags(pool, seq, layer, window) -> list[int]:
    arr = (ctypes.c_int64 * window)()
    _check(_lib.kvpool_slot_tags(pool, seq, layer, arr), "kvpool_slot_tags")
    return list(arr)


def swa_attn_prefill(pool, seq, layer, q, k, v, n_q_heads, out, n=None, stream=None) -> None:
    if n is None:
        n = q.shape[0]
    _check(_lib.swa_attn_prefill(pool, seq, layer, _ptr(q), _ptr(k), _ptr(v), n, n_q_heads, _dt(q.dtype),
                                 _ptr(out), _stream(stream)), "swa_attn_prefill")


def swa_attn_workspace_bytes(pool, seqs, layer, q_len_or_chunk, n_q_heads) -> int:
    arr = _i32_array(seqs)
    return _check(_lib.swa_attn_workspace_bytes(pool, len(arr), arr.ptr, layer, q_len_or_chunk, n_q_heads),
                  "swa_attn_workspace_bytes")


def swa_attn_decode(pool, seqs, layer, q, k_new, v_new, q_len, n_q_heads, out, workspace,
                    stream=None) -> None:
    arr = _i32_array(seqs)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(_lib.swa_attn_decode(pool, len(arr), arr.ptr, layer, _ptr(q), _ptr(k_new), _ptr(v_new), q_len,
                                n_q_heads, _dt(q.dtype), _ptr(out), _ptr(workspace), ws_bytes,
                                _stream(stream)), "swa_attn_decode")


def full_attn(pool, seqs, layer, q, k_new, v_new, q_len_or_chunk, n_q_heads, out, workspace=None,
              stream=None) -> None:
    arr = _i32_array(seqs)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(_lib.full_attn(pool, len(arr), arr.ptr, layer, _ptr(q), _ptr(k_new), _ptr(v_new), q_len_or_chunk,
                          n_q_heads, _dt(q.dtype), _ptr(out), _ptr(workspace), ws_bytes, _stream(stream)),
           "full_attn")


def full_attn_noalloc(pool, seqs, layer, q, k_new, v_new, q_len_or_chunk, n_q_heads, out, stream=None) -> None:
    arr = _i32_array(seqs)
    _check(_lib.full_attn_noalloc(pool, len(arr), arr.ptr, layer, _ptr(q), _ptr(k_new), _ptr(v_new), q_len_or_chunk,
                                  n_q_heads, _dt(q.dtype), _ptr(out), _stream(stream)),
           "full_attn_noalloc")


def swa_last_error() -> str:
    return _lib.swa_last_error().decode(errors="replace")


def swa_clock_probe(out, spin_us: int, stream=None) -> None:
    """Measurement aid: `out` is a device int64 tensor of 5 (see the C header); after the stream
    has passed the call, clock_mhz(out) is the shader clock over the spin."""
    _check(_lib.swa_clock_probe(_ptr(out), spin_us, _stream(stream)), "swa_clock_probe")


def clock_mhz(vals) -> float:
    """Shader clock (MHz) from the 5 values swa_clock_probe wrote: shader ticks over wall ticks
    times the wall clock's rate."""
    t0, t1, r0, r1, khz = (int(x) for x in vals)
    return (t1 - t0) / (r1 - r0) * khz / 1e3 if r1 > r0 else float("nan")


def library_path() -> str:
    return _LIB_PATH
