"""Paged attention over one packed continuous-batching tick, for MI355X (gfx950).

Thin Python binding over ``libpa.so`` (C ABI in ``include/pa.h``). Each
function here has the name of the C entry point it calls and only marshals
arguments: torch tensors supply device pointers and shapes, and the current
torch stream supplies the HIP stream. Every step of the computation runs in the
library's HIP kernels. There is no fallback: if ``libpa.so`` is not built, or a
tensor is not on a GPU, the call raises.

``paged_kv_cache_page_amd.workloads`` (seeded synthetic inputs) imports
without the library.
"""

import ctypes
import math
import os

__all__ = [
    "PA_F32", "PA_BF16", "lib", "lib_path", "PaError",
    "pa_abi_version", "pa_status_string", "pa_rope_cos_sin_table", "pa_compute_slot_mapping",
    "pa_rope_and_cache_write", "pa_paged_attention_workspace_size", "pa_paged_attention_varlen",
    "pa_tick_forward", "pa_profile_start", "pa_profile_stop", "pa_profile_reset",
    "BlockManager", "PA_ERR_NO_PAGES", "pa_sample_tokens", "pa_set_validation",
    "pa_validation_message", "pa_probe_stream_read", "pa_tick_forward_noalloc",
]

PA_F32 = 0
PA_BF16 = 1
PA_ERR_NO_PAGES = 5
_HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_HERE, "libpa.so")
_lib = None

_vp, _i32, _f32, _f64, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_double, ctypes.c_size_t

# name -> (restype, argtypes)
SIGNATURES = {
    "pa_abi_version": (_i32, []),
    "pa_status_string": (ctypes.c_char_p, [_i32]),
    "pa_rope_cos_sin_table": (_i32, [_vp, _i32, _i32, _f64, _vp]),
    "pa_compute_slot_mapping": (_i32, [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _vp]),
    "pa_rope_and_cache_write": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32,
                                       _i32, _i32, _i32, _i32, _i32, _vp]),
    "pa_paged_attention_workspace_size": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                                _i32]),
    "pa_paged_attention_varlen": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32,
                                         _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _i32,
                                         _i32, _vp, _sz, _vp]),
    "pa_tick_forward": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                               _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                               _i32, _f32, _i32, _i32, _vp, _sz, _vp]),
    "pa_tick_forward_noalloc": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                       _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                       _i32, _i32, _i32, _f32, _i32, _i32, _vp]),
    "pa_bm_create": (_i32, [_i32, _i32, ctypes.POINTER(_vp)]),
    "pa_bm_destroy": (None, [_vp]),
    "pa_bm_admit": (_i32, [_vp, ctypes.c_int64, _vp, _i32, _i32, ctypes.POINTER(_i32)]),
    "pa_bm_append": (_i32, [_vp, ctypes.c_int64, _i32]),
    "pa_bm_finish": (_i32, [_vp, ctypes.c_int64, _i32]),
    "pa_bm_evict": (_i32, [_vp, _i32, ctypes.POINTER(_i32)]),
    "pa_bm_block_table": (_i32, [_vp, ctypes.c_int64, _vp, _i32, ctypes.POINTER(_i32)]),
    "pa_bm_stats": (_i32, [_vp, ctypes.POINTER(_i32), ctypes.POINTER(_i32), ctypes.POINTER(_i32)]),
    "pa_bm_refcount": (_i32, [_vp, _i32, ctypes.POINTER(_i32)]),
    "pa_sample_workspace_size": (ctypes.c_size_t, [_i32, _i32]),
    "pa_sample_tokens": (_i32, [_vp, ctypes.c_int64, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp,
                                ctypes.c_size_t, _vp]),
    "pa_profile_start": (_i32, [_i32]),
    "pa_profile_stop": (_i32, [ctypes.POINTER(_i32)]),
    "pa_profile_get": (_i32, [_i32, ctypes.c_char_p, _i32, ctypes.POINTER(_f32)]),
    "pa_profile_reset": (_i32, []),
    "pa_set_validation": (None, [_i32]),
    "pa_probe_sink_words": (_sz, []),
    "pa_probe_stream_read": (_i32, [_vp, _sz, _vp, _vp]),
    "pa_validation_message": (ctypes.c_char_p, []),
}


class PaError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        detail = pa_validation_message() if status in (1, 3) else ""
        super().__init__(f"{where}: {pa_status_string(status)} (status {status})"
                         + (f": {detail}" if detail else ""))


def lib():
    """The loaded ``libpa.so`` (ctypes), with signatures set. Raises if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(lib_path):
            raise RuntimeError(f"{lib_path} is not built; run `python -m paged_kv_cache_page_amd.build`"
                               " (or __graft_entry__.build())")
        handle = ctypes.CDLL(lib_path)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def pa_abi_version():
    return int(lib().pa_abi_version())


def pa_status_string(status):
    return lib().pa_status_string(int(status)).decode()


def _check(status, where):
    if status != 0:
        raise PaError(status, where)


# ---------------------------------------------------------------- marshalling
def _torch():
    import torch
    return torch


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.float32:
        return PA_F32
    if t.dtype == torch.bfloat16:
        return PA_BF16
    raise ValueError(f"unsupported tensor dtype {t.dtype} (float32 or bfloat16)")


def _dev(t, name, dtype=None, ndim=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (the library has no CPU path)")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {t.dim()}")
    return t


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _empty(shape, dtype, device, stream):
    """A new tensor owned by the stream the kernels run on: the caching
    allocator then hands its bytes to no other stream until that stream's work
    on them is done (allocated on another stream, the bytes could be reused
    while the library's kernels still read or write them)."""
    torch = _torch()
    if stream is None:
        return torch.empty(shape, dtype=dtype, device=device)
    with torch.cuda.stream(stream):
        return torch.empty(shape, dtype=dtype, device=device)


# ---------------------------------------------------------------- entry points
def pa_rope_cos_sin_table(max_pos, head_dim, theta, device="cuda", out=None, stream=None):
    """float32 ``[max_pos, head_dim]`` cos/sin table built on the GPU."""
    torch = _torch()
    if out is None:
        out = _empty((max_pos, head_dim), torch.float32, device, stream)
    _dev(out, "out", torch.float32, 2)
    _check(lib().pa_rope_cos_sin_table(_ptr(out), int(max_pos), int(head_dim), float(theta),
                                       _stream(stream)), "pa_rope_cos_sin_table")
    return out


def pa_compute_slot_mapping(block_tables, query_start_loc, positions, page_size, num_pages,
                            out=None, stream=None):
    """int32 ``[T]`` slot of every new token (-1 when out of range)."""
    torch = _torch()
    _dev(block_tables, "block_tables", torch.int32, 2)
    _dev(query_start_loc, "query_start_loc", torch.int32, 1)
    _dev(positions, "positions", torch.int32, 1)
    S, max_blocks = block_tables.shape
    T = positions.shape[0]
    if query_start_loc.shape[0] != S + 1:
        raise ValueError("query_start_loc must have S + 1 entries")
    if out is None:
        out = _empty(T, torch.int32, positions.device, stream)
    _dev(out, "out", torch.int32, 1)
    _check(lib().pa_compute_slot_mapping(_ptr(block_tables), _ptr(query_start_loc),
                                         _ptr(positions), _ptr(out), S, T, max_blocks,
                                         int(page_size), int(num_pages), _stream(stream)),
           "pa_compute_slot_mapping")
    return out


def pa_rope_and_cache_write(q, k, v, positions, slot_mapping, cos_sin, k_pool, v_pool,
                            stream=None):
    """RoPE on q (may be None) and k in place, then k/v into their pool slots."""
    torch = _torch()
    _dev(k, "k", ndim=3)
    dt = _dtype_code(k)
    _dev(v, "v", k.dtype, 3)
    if q is not None:
        _dev(q, "q", k.dtype, 3)
    _dev(positions, "positions", torch.int32, 1)
    _dev(slot_mapping, "slot_mapping", torch.int32, 1)
    _dev(k_pool, "k_pool", k.dtype, 4)
    _dev(v_pool, "v_pool", k.dtype, 4)
    if cos_sin is not None:
        _dev(cos_sin, "cos_sin", torch.float32, 2)
    T, Hkv, D = k.shape
    Hq = q.shape[1] if q is not None else 0
    num_pages, P = k_pool.shape[0], k_pool.shape[1]
    if tuple(v.shape) != (T, Hkv, D) or (q is not None and (q.shape[0] != T or q.shape[2] != D)):
        raise ValueError("q/k/v shapes disagree")
    if tuple(k_pool.shape) != (num_pages, P, Hkv, D) or tuple(v_pool.shape) != tuple(k_pool.shape):
        raise ValueError("pool shape must be [num_pages, P, Hkv, D]")
    if positions.shape[0] != T or slot_mapping.shape[0] != T:
        raise ValueError("positions and slot_mapping need one entry per token")
    max_pos = cos_sin.shape[0] if cos_sin is not None else 0
    if cos_sin is not None and cos_sin.shape[1] != D:
        raise ValueError("cos_sin must be [max_pos, head_dim]")
    _check(lib().pa_rope_and_cache_write(_ptr(q), _ptr(k), _ptr(v), _ptr(positions),
                                         _ptr(slot_mapping), _ptr(cos_sin), _ptr(k_pool),
                                         _ptr(v_pool), T, Hq, Hkv, D, P, num_pages, max_pos, dt,
                                         _stream(stream)), "pa_rope_and_cache_write")


def pa_paged_attention_workspace_size(S, T, Hq, head_dim, max_query_len, max_seq_len, page_size,
                                      kv_split_tokens, dtype):
    return int(lib().pa_paged_attention_workspace_size(S, T, Hq, head_dim, max_query_len,
                                                       max_seq_len, page_size, kv_split_tokens,
                                                       int(dtype)))


def pa_paged_attention_varlen(q, k_pool, v_pool, block_tables, seq_lens, query_start_loc,
                              max_query_len, max_seq_len, scale=None, kv_split_tokens=0,
                              out=None, workspace=None, stream=None):
    """Attention of a packed tick; returns ``out`` ``[T, Hq, D]`` (allocated if None).

    ``max_query_len`` / ``max_seq_len`` are host-side upper bounds of the query
    and key counts per sequence (the library never reads device metadata from
    the host). ``workspace`` is a uint8 GPU tensor, allocated here if None.
    """
    torch = _torch()
    _dev(q, "q", ndim=3)
    dt = _dtype_code(q)
    _dev(k_pool, "k_pool", q.dtype, 4)
    _dev(v_pool, "v_pool", q.dtype, 4)
    _dev(block_tables, "block_tables", torch.int32, 2)
    _dev(seq_lens, "seq_lens", torch.int32, 1)
    _dev(query_start_loc, "query_start_loc", torch.int32, 1)
    T, Hq, D = q.shape
    num_pages, P, Hkv, Dp = k_pool.shape
    S, max_blocks = block_tables.shape
    if Dp != D or tuple(v_pool.shape) != tuple(k_pool.shape):
        raise ValueError("pool shape must be [num_pages, P, Hkv, D] with q's head_dim")
    if seq_lens.shape[0] != S or query_start_loc.shape[0] != S + 1:
        raise ValueError("seq_lens needs S entries and query_start_loc S + 1")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = _empty(tuple(q.shape), q.dtype, q.device, stream)
    _dev(out, "out", q.dtype, 3)
    need = pa_paged_attention_workspace_size(S, T, Hq, D, int(max_query_len), int(max_seq_len),
                                             P, int(kv_split_tokens), dt)
    if workspace is None and need > 0:
        workspace = _empty(need, torch.uint8, q.device, stream)
    ws_bytes = 0
    if workspace is not None:
        _dev(workspace, "workspace")
        ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().pa_paged_attention_varlen(
        _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_tables), _ptr(seq_lens),
        _ptr(query_start_loc), _ptr(out), S, T, Hq, Hkv, D, P, num_pages, max_blocks,
        int(max_query_len), int(max_seq_len), float(scale), int(kv_split_tokens), dt,
        _ptr(workspace), ws_bytes, _stream(stream)), "pa_paged_attention_varlen")
    return out


def pa_tick_forward(q, k, v, positions, block_tables, seq_lens, query_start_loc, cos_sin,
                    k_pool, v_pool, max_query_len, max_seq_len, scale=None, kv_split_tokens=0,
                    out=None, slot_mapping=None, workspace=None, stream=None):
    """One layer's tick in one call: slot mapping, RoPE + page write, attention.

    ``out``, the slots and the pools are those of ``pa_compute_slot_mapping`` +
    ``pa_rope_and_cache_write`` + ``pa_paged_attention_varlen`` with these
    arguments, bit for bit. bf16 ticks leave ``q`` and ``k`` unchanged (the
    attention rotates what it reads); float32 ticks rotate them in place as
    the page write does. Returns ``out``; ``slot_mapping`` ``[T]`` int32 is
    written (allocated if None).
    """
    torch = _torch()
    _dev(q, "q", ndim=3)
    dt = _dtype_code(q)
    _dev(k, "k", q.dtype, 3)
    _dev(v, "v", q.dtype, 3)
    _dev(positions, "positions", torch.int32, 1)
    _dev(k_pool, "k_pool", q.dtype, 4)
    _dev(v_pool, "v_pool", q.dtype, 4)
    _dev(block_tables, "block_tables", torch.int32, 2)
    _dev(seq_lens, "seq_lens", torch.int32, 1)
    _dev(query_start_loc, "query_start_loc", torch.int32, 1)
    if cos_sin is not None:
        _dev(cos_sin, "cos_sin", torch.float32, 2)
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    num_pages, P = k_pool.shape[0], k_pool.shape[1]
    S, max_blocks = block_tables.shape
    if tuple(k.shape) != (T, Hkv, D) or tuple(v.shape) != (T, Hkv, D):
        raise ValueError("q/k/v shapes disagree")
    if tuple(k_pool.shape) != (num_pages, P, Hkv, D) or tuple(v_pool.shape) != tuple(k_pool.shape):
        raise ValueError("pool shape must be [num_pages, P, Hkv, D]")
    if positions.shape[0] != T:
        raise ValueError("positions needs one entry per token")
    if seq_lens.shape[0] != S or query_start_loc.shape[0] != S + 1:
        raise ValueError("seq_lens needs S entries and query_start_loc S + 1")
    max_pos = cos_sin.shape[0] if cos_sin is not None else 0
    if cos_sin is not None and cos_sin.shape[1] != D:
        raise ValueError("cos_sin must be [max_pos, head_dim]")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = _empty(tuple(q.shape), q.dtype, q.device, stream)
    _dev(out, "out", q.dtype, 3)
    if slot_mapping is None:
        slot_mapping = _empty(T, torch.int32, q.device, stream)
    _dev(slot_mapping, "slot_mapping", torch.int32, 1)
    if slot_mapping.shape[0] != T:
        raise ValueError("slot_mapping needs one entry per token")
    need = pa_paged_attention_workspace_size(S, T, Hq, D, int(max_query_len), int(max_seq_len),
                                             P, int(kv_split_tokens), dt)
    if workspace is None and need > 0:
        workspace = _empty(need, torch.uint8, q.device, stream)
    ws_bytes = 0
    if workspace is not None:
        _dev(workspace, "workspace")
        ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().pa_tick_forward(
        _ptr(q), _ptr(k), _ptr(v), _ptr(positions), _ptr(block_tables), _ptr(seq_lens),
        _ptr(query_start_loc), _ptr(cos_sin), _ptr(k_pool), _ptr(v_pool), _ptr(out),
        _ptr(slot_mapping), S, T, Hq, Hkv, D, P, num_pages, max_blocks, int(max_query_len),
        int(max_seq_len), max_pos, float(scale), int(kv_split_tokens), dt, _ptr(workspace),
        ws_bytes, _stream(stream)), "pa_tick_forward")
    return out


def pa_set_validation(on):
    """Turn the library's opt-in metadata validation on or off (process-wide).
    While on, the attention and tick calls copy their device metadata to the
    host (synchronising the stream) and reject inconsistent metadata with
    PA_ERR_INVALID_ARG before anything is enqueued; the raised PaError then
    names the offending sequence or token."""
    lib().pa_set_validation(1 if on else 0)


def pa_validation_message():
    """Why the last call on this thread failed validation ('' if it did not)."""
    return lib().pa_validation_message().decode()


def pa_probe_stream_read(buf, sink=None, stream=None):
    """Read the GPU tensor ``buf`` once as a plain 16-byte-load stream (a
    measurement of the practical read bandwidth). Returns the sink tensor."""
    torch = _torch()
    _dev(buf, "buf")
    if sink is None:
        sink = _empty(int(lib().pa_probe_sink_words()), torch.int32, buf.device, stream)
    _check(lib().pa_probe_stream_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink),
                                      _stream(stream)), "pa_probe_stream_read")
    return sink


def pa_tick_forward_noalloc(q, k, v, positions, block_tables, seq_lens, query_start_loc,
                            cos_sin, k_pool, v_pool, max_query_len, max_seq_len, out, slot_mapping,
                            scale=None, kv_split_tokens=0, stream=None):
    """``pa_tick_forward`` on the library's fixed scratch: no workspace, and
    the caller passes ``out`` and ``slot_mapping`` (nothing is allocated here
    or in the library). Raises PaError (PA_ERR_WORKSPACE_TOO_SMALL) when the
    tick needs more scratch than the library holds."""
    torch = _torch()
    _dev(q, "q", ndim=3)
    dt = _dtype_code(q)
    for t, name in ((k, "k"), (v, "v"), (out, "out")):
        _dev(t, name, q.dtype, 3)
    _dev(k_pool, "k_pool", q.dtype, 4)
    _dev(v_pool, "v_pool", q.dtype, 4)
    for t, name in ((positions, "positions"), (seq_lens, "seq_lens"),
                    (query_start_loc, "query_start_loc"), (slot_mapping, "slot_mapping")):
        _dev(t, name, torch.int32, 1)
    _dev(block_tables, "block_tables", torch.int32, 2)
    if cos_sin is not None:
        _dev(cos_sin, "cos_sin", torch.float32, 2)
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    num_pages, P = k_pool.shape[0], k_pool.shape[1]
    S, max_blocks = block_tables.shape
    if (tuple(k.shape) != (T, Hkv, D) or tuple(v.shape) != (T, Hkv, D)
            or tuple(out.shape) != (T, Hq, D)):
        raise ValueError("q/k/v/out shapes disagree")
    if tuple(k_pool.shape) != (num_pages, P, Hkv, D) or tuple(v_pool.shape) != tuple(k_pool.shape):
        raise ValueError("pool shape must be [num_pages, P, Hkv, D]")
    if positions.shape[0] != T or slot_mapping.shape[0] != T:
        raise ValueError("positions and slot_mapping need one entry per token")
    if seq_lens.shape[0] != S or query_start_loc.shape[0] != S + 1:
        raise ValueError("seq_lens needs S entries and query_start_loc S + 1")
    max_pos = cos_sin.shape[0] if cos_sin is not None else 0
    if cos_sin is not None and cos_sin.shape[1] != D:
        raise ValueError("cos_sin must be [max_pos, head_dim]")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    _check(lib().pa_tick_forward_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(positions), _ptr(block_tables), _ptr(seq_lens),
        _ptr(query_start_loc), _ptr(cos_sin), _ptr(k_pool), _ptr(v_pool), _ptr(out),
        _ptr(slot_mapping), S, T, Hq, Hkv, D, P, num_pages, max_blocks, int(max_query_len),
        int(max_seq_len), max_pos, float(scale), int(kv_split_tokens), dt, _stream(stream)),
        "pa_tick_forward_noalloc")
    return out


def pa_profile_start(capacity=4096):
    _check(lib().pa_profile_start(int(capacity)), "pa_profile_start")


def pa_profile_stop():
    """Stop timing; return [(kernel_name, milliseconds), ...] in launch order."""
    n = ctypes.c_int32(0)
    _check(lib().pa_profile_stop(ctypes.byref(n)), "pa_profile_stop")
    out = []
    buf = ctypes.create_string_buffer(64)
    for i in range(n.value):
        ms = ctypes.c_float(0.0)
        _check(lib().pa_profile_get(i, buf, 64, ctypes.byref(ms)), "pa_profile_get")
        out.append((buf.value.decode(), ms.value))
    return out


def pa_profile_reset():
    _check(lib().pa_profile_reset(), "pa_profile_reset")


# ---------------------------------------------------------------- block manager
def pa_sample_tokens(logits, temperature, top_k, top_p, uniforms, out=None, workspace=None,
                     stream=None):
    """Sample one token per row of ``logits`` [rows, vocab] float32 (row stride
    ``logits.stride(0)``), each row with its own ``temperature``, ``top_k``,
    ``top_p`` and caller-drawn ``uniforms`` in [0, 1) (float32, int32, float32,
    float32 [rows]). Greedy when temperature <= 0 or top_k == 1. Returns
    ``out`` int32 [rows] (allocated if None)."""
    torch = _torch()
    _dev(logits, "logits", torch.float32, 2)
    R, V = logits.shape
    for t, name, dt in ((temperature, "temperature", torch.float32), (top_k, "top_k", torch.int32),
                        (top_p, "top_p", torch.float32), (uniforms, "uniforms", torch.float32)):
        _dev(t, name, dt, 1)
        if t.shape[0] != R or not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous [{R}]")
    if out is None:
        out = _empty(R, torch.int32, logits.device, stream)
    _dev(out, "out", torch.int32, 1)
    if out.shape[0] != R:
        raise ValueError("out must be [rows]")
    need = int(lib().pa_sample_workspace_size(R, V))
    if workspace is None:
        workspace = _empty(max(need, 1), torch.uint8, logits.device, stream)
    _dev(workspace, "workspace", torch.uint8, 1)
    _check(lib().pa_sample_tokens(_ptr(logits), logits.stride(0), R, V, _ptr(temperature),
                                  _ptr(top_k), _ptr(top_p), _ptr(uniforms), _ptr(out),
                                  _ptr(workspace), workspace.numel(), _stream(stream)),
           "pa_sample_tokens")
    return out


class BlockManager:
    """Host-side paged block manager (``include/pa_blocks.h``): the pool's
    pages, each request's page table and reservation, and the prefix cache of
    complete blocks. The block tables it returns feed the attention calls."""

    def __init__(self, num_pages, page_size):
        h = _vp()
        _check(lib().pa_bm_create(int(num_pages), int(page_size), ctypes.byref(h)), "pa_bm_create")
        self._h = h
        self.num_pages, self.page_size = int(num_pages), int(page_size)

    def close(self):
        if self._h:
            lib().pa_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def admit(self, req, prompt, max_new_tokens):
        """Admit request ``req``; returns the prompt tokens already cached."""
        import numpy as np
        arr = np.ascontiguousarray(prompt, dtype=np.int32)
        out = _i32(0)
        _check(lib().pa_bm_admit(self._h, int(req), arr.ctypes.data_as(_vp), int(arr.size),
                                 int(max_new_tokens), ctypes.byref(out)), "pa_bm_admit")
        return out.value

    def append(self, req, n_tokens):
        _check(lib().pa_bm_append(self._h, int(req), int(n_tokens)), "pa_bm_append")

    def finish(self, req, publish=True):
        _check(lib().pa_bm_finish(self._h, int(req), 1 if publish else 0), "pa_bm_finish")

    def evict(self, pages):
        out = _i32(0)
        _check(lib().pa_bm_evict(self._h, int(pages), ctypes.byref(out)), "pa_bm_evict")
        return out.value

    def block_table(self, req):
        """int32 numpy array: the request's pages in order."""
        import numpy as np
        out = np.zeros(self.num_pages, dtype=np.int32)
        n = _i32(0)
        _check(lib().pa_bm_block_table(self._h, int(req), out.ctypes.data_as(_vp), out.size,
                                       ctypes.byref(n)), "pa_bm_block_table")
        return out[:n.value].copy()

    def stats(self):
        """(free pages, reserved pages, cached blocks)."""
        f, r, c = _i32(0), _i32(0), _i32(0)
        _check(lib().pa_bm_stats(self._h, ctypes.byref(f), ctypes.byref(r), ctypes.byref(c)),
               "pa_bm_stats")
        return f.value, r.value, c.value

    def refcount(self, page):
        out = _i32(0)
        _check(lib().pa_bm_refcount(self._h, int(page), ctypes.byref(out)), "pa_bm_refcount")
        return out.value
