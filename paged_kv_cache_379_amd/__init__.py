"""Paged-attention decode for AMD MI355X (gfx950): Python binding of libpkv.so.

The binding only marshals arguments: torch tensors supply device memory and
the current HIP stream, every step of the computation runs in the library's
HIP kernels, and there is no CPU fallback.  If libpkv.so is missing the first
call raises; build it with ``python -m paged_kv_cache_379_amd.build``.

The host-side block allocator (:class:`BlockAllocator`) runs in the same
library and needs no GPU.
"""
import contextlib
import ctypes
import os

import numpy as np

__all__ = [
    "load", "LIB_PATH", "PkvError", "OutOfBlocks", "DoubleFree",
    "paged_attention_decode", "decode_workspace_size", "decode_partition_size", "decode_plan",
    "paged_attention_decode_noalloc", "NOALLOC_SCRATCH_BYTES",
    "paged_attention_decode_prefix", "decode_prefix_workspace_size", "find_shared_prefixes",
    "reshape_and_cache", "copy_blocks", "swap_blocks", "stream_copy", "stream_read",
    "validate_tables",
    "BlockAllocator", "F32", "F16", "BF16", "I8", "FP8", "SWAP_OUT", "SWAP_IN",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpkv.so")

# Status codes and formats (include/pkv.h).
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_OOM, ERR_DOUBLE_FREE, ERR_INDEX, ERR_HIP, ERR_WORKSPACE = range(8)
F32, F16, BF16, I8, FP8 = 0, 1, 2, 3, 4
SWAP_OUT, SWAP_IN = 0, 1


class PkvError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"pkv error {code}: {msg}")
        self.code = code


class OutOfBlocks(PkvError):
    """Not enough free blocks (the allocator state is unchanged)."""


class DoubleFree(PkvError):
    """A block reference was dropped more often than it was taken."""


_lib = None

_c_int, _c_size, _vp = ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p
_i32p = ctypes.POINTER(ctypes.c_int32)
_SIGS = {
    "pkv_last_error": (ctypes.c_char_p, []),
    "pkv_abi_version": (_c_int, []),
    "pkv_decode_partition_size": (_c_int, [_c_int] * 8),
    "pkv_decode_workspace_size": (_c_size, [_c_int] * 8),
    "pkv_decode_plan": (_c_int, [_c_int] * 9 + [_i32p]),
    "pkv_paged_attention_decode": (_c_int, [_vp] * 8 + [_c_int] * 7 + [ctypes.c_float] + [_c_int] * 4
                                   + [_vp, _c_size, _vp]),
    "pkv_paged_attention_decode_noalloc": (_c_int, [_vp] * 8 + [_c_int] * 7 + [ctypes.c_float]
                                           + [_c_int] * 4 + [_vp]),
    "pkv_paged_attention_decode_prefix": (_c_int, [_vp] * 9 + [_c_int] * 7 + [ctypes.c_float]
                                          + [_c_int] * 2 + [_i32p, _c_int, _vp, _c_size, _vp]),
    "pkv_decode_prefix_workspace_size": (_c_size, [_c_int] * 6 + [_i32p, _c_int]),
    "pkv_reshape_and_cache": (_c_int, [_vp] * 7 + [_c_int] * 7 + [_vp]),
    "pkv_copy_blocks": (_c_int, [_vp] * 4 + [_i32p, _c_int, _c_size, _c_int, _c_int, _vp]),
    "pkv_swap_blocks": (_c_int, [_vp] * 8 + [_i32p, _c_int, _c_size] + [_c_int] * 4 + [_vp]),
    "pkv_stream_copy": (_c_int, [_vp, _vp, _c_size, _vp]),
    "pkv_stream_read": (_c_int, [_vp, _c_size, _vp, ctypes.c_uint32, _vp]),
    "pkv_allocator_create": (_c_int, [_c_int, _c_int, ctypes.POINTER(_vp)]),
    "pkv_allocator_destroy": (_c_int, [_vp]),
    "pkv_allocator_set_free_order": (_c_int, [_vp, _i32p, _c_int]),
    "pkv_allocate": (_c_int, [_vp, _c_int, _i32p]),
    "pkv_free": (_c_int, [_vp, _i32p, _c_int]),
    "pkv_incref": (_c_int, [_vp, _i32p, _c_int]),
    "pkv_copy_on_write": (_c_int, [_vp, ctypes.c_int32, _i32p, ctypes.POINTER(_c_int)]),
    "pkv_ref_count": (_c_int, [_vp, ctypes.c_int32, ctypes.POINTER(_c_int)]),
    "pkv_num_free": (_c_int, [_vp, ctypes.POINTER(_c_int)]),
    "pkv_usage_ratio": (_c_int, [_vp, ctypes.POINTER(ctypes.c_double)]),
    "pkv_free_list": (_c_int, [_vp, _i32p, _c_int, ctypes.POINTER(_c_int)]),
    "pkv_cow_count": (_c_int, [_vp, ctypes.POINTER(ctypes.c_int64)]),
    "pkv_seq_create": (_c_int, [_vp, _i32p]),
    "pkv_seq_fork": (_c_int, [_vp, ctypes.c_int32, _i32p]),
    "pkv_seq_append_tokens": (_c_int, [_vp, ctypes.c_int32, _c_int, _i32p, _i32p, _c_int,
                                       ctypes.POINTER(_c_int)]),
    "pkv_seq_trim_window": (_c_int, [_vp, ctypes.c_int32, _c_int, _i32p, _c_int, ctypes.POINTER(_c_int)]),
    "pkv_allocator_set_host_pool": (_c_int, [_vp, _c_int]),
    "pkv_host_num_free": (_c_int, [_vp, ctypes.POINTER(_c_int)]),
    "pkv_seq_swap_out": (_c_int, [_vp, ctypes.c_int32, _i32p, _c_int, ctypes.POINTER(_c_int)]),
    "pkv_seq_swap_in": (_c_int, [_vp, ctypes.c_int32, _i32p, _c_int, ctypes.POINTER(_c_int)]),
    "pkv_seq_is_swapped": (_c_int, [_vp, ctypes.c_int32, ctypes.POINTER(_c_int)]),
    "pkv_seq_free": (_c_int, [_vp, ctypes.c_int32]),
    "pkv_seq_num_tokens": (_c_int, [_vp, ctypes.c_int32, ctypes.POINTER(_c_int)]),
    "pkv_seq_block_ids": (_c_int, [_vp, ctypes.c_int32, _i32p, _c_int, ctypes.POINTER(_c_int)]),
    "pkv_seq_physical_block": (_c_int, [_vp, ctypes.c_int32, _c_int, _i32p]),
    "pkv_export_block_tables": (_c_int, [_vp, _i32p, _c_int, _c_int, ctypes.c_int32, _i32p, _i32p]),
    "pkv_validate_tables": (_c_int, [_i32p, _i32p, _c_int, _c_int, _c_int, _c_int, _c_int,
                                     ctypes.POINTER(_c_int), ctypes.POINTER(_c_int)]),
    "pkv_find_shared_prefixes": (_c_int, [_i32p, _i32p] + [_c_int] * 5 + [_i32p, _c_int,
                                                                         ctypes.POINTER(_c_int)]),
}
EXPORTED = tuple(_SIGS)
SIGNATURES = _SIGS


def load(path=None):
    """Load libpkv.so (once) and return the ctypes handle; raises if missing."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"libpkv.so not found at {path}: run "
                           "`python -m paged_kv_cache_379_amd.build` first")
    # torch carries its own HIP runtime.  The library must resolve to that
    # same runtime (streams and pinned allocations come from torch), so torch
    # is loaded first; loaded the other way round, the process ends up with
    # two runtimes and torch's pinned memory is unknown to the library's.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(rc):
    if rc == OK:
        return
    msg = _lib.pkv_last_error().decode(errors="replace")
    if rc == ERR_OOM:
        raise OutOfBlocks(rc, msg)
    if rc == ERR_DOUBLE_FREE:
        raise DoubleFree(rc, msg)
    if rc == ERR_INDEX:
        raise IndexError(msg)
    if rc == ERR_INVALID_ARG:
        raise ValueError(msg)
    raise PkvError(rc, msg)


# ---------------------------------------------------------------------------
# Device entry points (torch tensors in, nothing computed here).

def _torch():
    import torch
    return torch


def _fmt(t):
    torch = _torch()
    fmt = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16, torch.int8: I8,
           torch.float8_e4m3fn: FP8}.get(t.dtype)
    if fmt is None:
        raise ValueError(f"unsupported dtype {t.dtype} (float32, float16, bfloat16, int8, "
                         "float8_e4m3fn)")
    return fmt


def _dev_ptr(t, name, dtype=None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _temporaries_on(stream):
    """Context for allocating a call's temporary device buffers: on the stream
    its kernels run on, so that torch's caching allocator hands their memory
    to later allocations only in that stream's order (a buffer allocated on
    another stream could be reused there while the kernels still use it)."""
    if stream is None:
        return contextlib.nullcontext()
    return _torch().cuda.stream(stream)


def decode_partition_size(num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                          max_blocks_per_seq, partition_size=0, window=0):
    return load().pkv_decode_partition_size(num_seqs, num_heads, num_kv_heads, head_dim,
                                            block_size, max_blocks_per_seq, partition_size,
                                            window)


def decode_workspace_size(num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                          max_blocks_per_seq, partition_size=0, window=0):
    return load().pkv_decode_workspace_size(num_seqs, num_heads, num_kv_heads, head_dim,
                                            block_size, max_blocks_per_seq, partition_size,
                                            window)


def decode_plan(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                kv_dtype, partition_size=0, window=0):
    """How the decode runs for these shapes: a dict with partition_tokens (0 =
    not split), partitions, kv_heads_per_workgroup, kernel ("multi_head" or
    "grouped_query") and workgroups."""
    out = np.zeros(5, dtype=np.int32)
    _check(load().pkv_decode_plan(num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                                  max_blocks_per_seq, partition_size, window, kv_dtype,
                                  out.ctypes.data_as(_i32p)))
    return {"partition_tokens": int(out[0]), "partitions": int(out[1]),
            "kv_heads_per_workgroup": int(out[2]),
            "kernel": ("multi_head", "grouped_query")[int(out[3])], "workgroups": int(out[4])}


def paged_attention_decode(out, q, key_cache, value_cache, block_tables, context_lens,
                           block_size, scale, k_scales=None, v_scales=None,
                           partition_size=0, workspace=None, stream=None, window=0):
    """Decode attention over a paged KV cache (see include/pkv.h).

    out, q [B, H, D]; key_cache, value_cache [NB, block_size, Hkv, D];
    block_tables int32 [B, MB]; context_lens int32 [B]; k/v_scales fp32
    [NB, Hkv] for int8 and fp8 (torch.float8_e4m3fn) caches; window: 0 or a
    sliding window in tokens.  A
    workspace of the needed size is allocated from torch when none is given.
    """
    torch = _torch()
    lib = load()
    B, H, D = q.shape
    NB, bs, Hkv, D2 = key_cache.shape
    if D2 != D or bs != block_size or tuple(out.shape) != (B, H, D) or out.dtype != q.dtype:
        raise ValueError("shape or dtype mismatch between q, out and the caches")
    if tuple(value_cache.shape) != tuple(key_cache.shape) or value_cache.dtype != key_cache.dtype:
        raise ValueError("value_cache must match key_cache")
    if block_tables.dim() != 2 or block_tables.shape[0] != B or context_lens.shape != (B,):
        raise ValueError("block_tables must be [B, MB] and context_lens [B]")
    MB = block_tables.shape[1]
    need = lib.pkv_decode_workspace_size(B, H, Hkv, D, bs, MB, partition_size, window)
    if need and workspace is None:
        with _temporaries_on(stream):
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = lib.pkv_paged_attention_decode(
        _dev_ptr(out, "out"), _dev_ptr(q, "q"), _dev_ptr(key_cache, "key_cache"),
        _dev_ptr(value_cache, "value_cache"), _dev_ptr(k_scales, "k_scales", torch.float32),
        _dev_ptr(v_scales, "v_scales", torch.float32),
        _dev_ptr(block_tables, "block_tables", torch.int32),
        _dev_ptr(context_lens, "context_lens", torch.int32),
        B, H, Hkv, D, bs, MB, NB, float(scale), _fmt(q), _fmt(key_cache), int(partition_size),
        int(window), _dev_ptr(workspace, "workspace"), ws_bytes, _stream(stream))
    _check(rc)
    return out


NOALLOC_SCRATCH_BYTES = 32 << 20   # PKV_NOALLOC_SCRATCH_BYTES (include/pkv.h)


def paged_attention_decode_noalloc(out, q, key_cache, value_cache, block_tables, context_lens,
                                   block_size, scale, k_scales=None, v_scales=None,
                                   partition_size=0, stream=None, window=0):
    """:func:`paged_attention_decode` with the split-context partials in the
    library's static per-GPU scratch (NOALLOC_SCRATCH_BYTES) instead of a
    workspace: neither the library nor this binding allocates device memory.
    Calls that may overlap on one GPU share that scratch and must be ordered."""
    lib = load()
    B, H, D = q.shape
    NB, bs, Hkv, D2 = key_cache.shape
    if D2 != D or bs != block_size or tuple(out.shape) != (B, H, D) or out.dtype != q.dtype:
        raise ValueError("shape or dtype mismatch between q, out and the caches")
    if tuple(value_cache.shape) != tuple(key_cache.shape) or value_cache.dtype != key_cache.dtype:
        raise ValueError("value_cache must match key_cache")
    if block_tables.dim() != 2 or block_tables.shape[0] != B or context_lens.shape != (B,):
        raise ValueError("block_tables must be [B, MB] and context_lens [B]")
    torch = _torch()
    rc = lib.pkv_paged_attention_decode_noalloc(
        _dev_ptr(out, "out"), _dev_ptr(q, "q"), _dev_ptr(key_cache, "key_cache"),
        _dev_ptr(value_cache, "value_cache"), _dev_ptr(k_scales, "k_scales", torch.float32),
        _dev_ptr(v_scales, "v_scales", torch.float32),
        _dev_ptr(block_tables, "block_tables", torch.int32),
        _dev_ptr(context_lens, "context_lens", torch.int32),
        B, H, Hkv, D, bs, block_tables.shape[1], NB, float(scale), _fmt(q), _fmt(key_cache),
        int(partition_size), int(window), _stream(stream))
    _check(rc)
    return out


def _group_array(groups):
    """[(first_seq, num_seqs, prefix_tokens), ...] -> host int32 [3 * G]."""
    arr = np.ascontiguousarray(np.asarray(groups, dtype=np.int32).reshape(-1, 3))
    if len(arr) == 0:
        raise ValueError("at least one prefix group is needed")
    return arr


def decode_prefix_workspace_size(num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                                 max_blocks_per_seq, groups):
    """Workspace bytes of :func:`paged_attention_decode_prefix`."""
    arr = _group_array(groups)
    return load().pkv_decode_prefix_workspace_size(
        num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
        arr.ctypes.data_as(_i32p), len(arr))


def paged_attention_decode_prefix(out, q, key_cache, value_cache, block_tables, context_lens,
                                  block_size, scale, groups, k_scales=None, v_scales=None,
                                  workspace=None, stream=None, prefix_lens=None):
    """Decode with shared prefixes computed once per group (see include/pkv.h).

    ``groups``: list of (first_seq, num_seqs, prefix_tokens): non-overlapping
    ranges of the batch whose sequences share the blocks of their first
    ``prefix_tokens`` tokens.  The result equals :func:`paged_attention_decode`.
    ``prefix_lens`` (device int32 [B], each sequence's shared tokens) is built
    from ``groups`` when not given.
    """
    torch = _torch()
    lib = load()
    B, H, D = q.shape
    NB, bs, Hkv, D2 = key_cache.shape
    if D2 != D or bs != block_size or tuple(out.shape) != (B, H, D) or out.dtype != q.dtype:
        raise ValueError("shape or dtype mismatch between q, out and the caches")
    if tuple(value_cache.shape) != tuple(key_cache.shape) or value_cache.dtype != key_cache.dtype:
        raise ValueError("value_cache must match key_cache")
    if block_tables.dim() != 2 or block_tables.shape[0] != B or context_lens.shape != (B,):
        raise ValueError("block_tables must be [B, MB] and context_lens [B]")
    MB = block_tables.shape[1]
    arr = _group_array(groups)
    if prefix_lens is None:
        lens = np.zeros(B, dtype=np.int32)
        for first, n, p in arr.tolist():
            lens[max(first, 0):max(first + n, 0)] = p
        with _temporaries_on(stream):
            prefix_lens = torch.from_numpy(lens).to(q.device)
    elif prefix_lens.shape != (B,):
        raise ValueError("prefix_lens must be [B]")
    need = lib.pkv_decode_prefix_workspace_size(B, H, Hkv, D, bs, MB, arr.ctypes.data_as(_i32p),
                                                len(arr))
    if workspace is None:
        with _temporaries_on(stream):
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    rc = lib.pkv_paged_attention_decode_prefix(
        _dev_ptr(out, "out"), _dev_ptr(q, "q"), _dev_ptr(key_cache, "key_cache"),
        _dev_ptr(value_cache, "value_cache"), _dev_ptr(k_scales, "k_scales", torch.float32),
        _dev_ptr(v_scales, "v_scales", torch.float32),
        _dev_ptr(block_tables, "block_tables", torch.int32),
        _dev_ptr(context_lens, "context_lens", torch.int32),
        _dev_ptr(prefix_lens, "prefix_lens", torch.int32),
        B, H, Hkv, D, bs, MB, NB, float(scale), _fmt(q), _fmt(key_cache),
        arr.ctypes.data_as(_i32p), len(arr), _dev_ptr(workspace, "workspace"), ws_bytes,
        _stream(stream))
    _check(rc)
    return out


def reshape_and_cache(k, v, key_cache, value_cache, slot_mapping, k_scales=None,
                      v_scales=None, stream=None):
    """Write new tokens' K/V rows [T, Hkv, D] into their slots (see include/pkv.h)."""
    torch = _torch()
    lib = load()
    T, Hkv, D = k.shape
    NB, bs, Hkv2, D2 = key_cache.shape
    if (Hkv2, D2) != (Hkv, D) or tuple(v.shape) != tuple(k.shape) or slot_mapping.shape != (T,):
        raise ValueError("shape mismatch")
    rc = lib.pkv_reshape_and_cache(
        _dev_ptr(k, "k"), _dev_ptr(v, "v"), _dev_ptr(key_cache, "key_cache"),
        _dev_ptr(value_cache, "value_cache"), _dev_ptr(k_scales, "k_scales", torch.float32),
        _dev_ptr(v_scales, "v_scales", torch.float32),
        _dev_ptr(slot_mapping, "slot_mapping", torch.int32),
        T, Hkv, D, bs, NB, _fmt(k), _fmt(key_cache), _stream(stream))
    _check(rc)


def copy_blocks(key_cache, value_cache, pairs, k_scales=None, v_scales=None, stream=None):
    """Copy whole blocks src -> dst for each (src, dst) in ``pairs`` (host ints)."""
    lib = load()
    arr = np.ascontiguousarray(np.asarray(pairs, dtype=np.int32).reshape(-1, 2))
    NB = key_cache.shape[0]
    block_bytes = key_cache[0].numel() * key_cache.element_size()
    rc = lib.pkv_copy_blocks(
        _dev_ptr(key_cache, "key_cache"), _dev_ptr(value_cache, "value_cache"),
        _dev_ptr(k_scales, "k_scales"), _dev_ptr(v_scales, "v_scales"),
        arr.ctypes.data_as(_i32p), len(arr), block_bytes, NB,
        key_cache.shape[2], _stream(stream))
    _check(rc)


def _pinned_ptr(t, name, like, dtype=None):
    """Pointer of a pinned host tensor whose rows have the shape of ``like``'s rows."""
    if t is None:
        return None
    if t.is_cuda or not t.is_pinned():
        raise ValueError(f"{name} must be a pinned host tensor (pin_memory=True)")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dtype != (dtype or like.dtype) or tuple(t.shape[1:]) != tuple(like.shape[1:]):
        raise ValueError(f"{name} must have rows like {tuple(like.shape[1:])} {like.dtype}, "
                         f"got {tuple(t.shape)} {t.dtype}")
    return t.data_ptr()


def swap_blocks(key_cache, value_cache, host_key, host_value, pairs, direction,
                k_scales=None, v_scales=None, host_k_scales=None, host_v_scales=None,
                stream=None):
    """Copy whole blocks between the device pool and a pinned host pool.

    ``pairs`` (host ints) are (device, host) for ``SWAP_OUT`` and (host,
    device) for ``SWAP_IN``, as :meth:`BlockAllocator.seq_swap_out` and
    :meth:`BlockAllocator.seq_swap_in` return them.  ``host_key`` and
    ``host_value`` are pinned tensors [num_host_blocks, bs, Hkv, D] of the
    cache's dtype; int8 caches also pass their scales and pinned host scales
    [num_host_blocks, Hkv].
    """
    torch = _torch()
    lib = load()
    arr = np.ascontiguousarray(np.asarray(pairs, dtype=np.int32).reshape(-1, 2))
    NB = key_cache.shape[0]
    NHB = host_key.shape[0]
    if host_value.shape != host_key.shape:
        raise ValueError("host_key and host_value differ in shape")
    if tuple(value_cache.shape) != tuple(key_cache.shape) or value_cache.dtype != key_cache.dtype:
        raise ValueError("key_cache and value_cache differ")
    for t, n, name in ((k_scales, NB, "k_scales"), (v_scales, NB, "v_scales"),
                       (host_k_scales, NHB, "host_k_scales"), (host_v_scales, NHB, "host_v_scales")):
        if t is not None and (t.dim() != 2 or t.shape[0] != n or t.shape[1] != key_cache.shape[2]):
            raise ValueError(f"{name} must be [{n}, {key_cache.shape[2]}]")
    block_bytes = key_cache[0].numel() * key_cache.element_size()
    rc = lib.pkv_swap_blocks(
        _dev_ptr(key_cache, "key_cache"), _dev_ptr(value_cache, "value_cache"),
        _dev_ptr(k_scales, "k_scales", torch.float32), _dev_ptr(v_scales, "v_scales", torch.float32),
        _pinned_ptr(host_key, "host_key", key_cache), _pinned_ptr(host_value, "host_value", value_cache),
        _pinned_ptr(host_k_scales, "host_k_scales", k_scales, torch.float32) if k_scales is not None else None,
        _pinned_ptr(host_v_scales, "host_v_scales", v_scales, torch.float32) if v_scales is not None else None,
        arr.ctypes.data_as(_i32p), len(arr), block_bytes, NB, NHB, key_cache.shape[2], direction,
        _stream(stream))
    _check(rc)


def stream_copy(dst, src, nbytes=None, stream=None):
    """The library's streaming copy kernel (bandwidth reference)."""
    lib = load()
    nbytes = nbytes if nbytes is not None else src.numel() * src.element_size()
    _check(lib.pkv_stream_copy(_dev_ptr(dst, "dst"), _dev_ptr(src, "src"), nbytes, _stream(stream)))


def stream_read(src, sink, nbytes=None, sentinel=0x9E3779B9, stream=None):
    """The library's read-only streaming probe (read bandwidth reference);
    sink: a device int32 tensor, written only if a thread's XOR fold of the
    words it read equals the sentinel."""
    lib = load()
    nbytes = nbytes if nbytes is not None else src.numel() * src.element_size()
    _check(lib.pkv_stream_read(_dev_ptr(src, "src"), nbytes, _dev_ptr(sink, "sink"),
                               int(sentinel) & 0xFFFFFFFF, _stream(stream)))


def validate_tables(tables, lens, block_size, num_blocks, window=0):
    """Host check of decode tables; returns None or (bad_seq, bad_block)."""
    lib = load()
    t = np.ascontiguousarray(tables, dtype=np.int32)
    l = np.ascontiguousarray(lens, dtype=np.int32)
    bs_, bb = ctypes.c_int(), ctypes.c_int()
    rc = lib.pkv_validate_tables(t.ctypes.data_as(_i32p), l.ctypes.data_as(_i32p), t.shape[0],
                                 t.shape[1], block_size, num_blocks, window, ctypes.byref(bs_),
                                 ctypes.byref(bb))
    if rc == OK:
        return None
    if rc == ERR_INVALID_ARG and bs_.value >= 0:
        return (bs_.value, bb.value)
    _check(rc)


def find_shared_prefixes(tables, lens, block_size, min_tokens=256, min_group=2):
    """Groups (first_seq, num_seqs, shared_tokens) of consecutive sequences
    whose host tables share leading blocks (see include/pkv.h), ready for
    :func:`paged_attention_decode_prefix`."""
    lib = load()
    t = np.ascontiguousarray(tables, dtype=np.int32)
    l = np.ascontiguousarray(lens, dtype=np.int32)
    out = np.empty(3 * 32, dtype=np.int32)
    n = ctypes.c_int()
    _check(lib.pkv_find_shared_prefixes(t.ctypes.data_as(_i32p), l.ctypes.data_as(_i32p),
                                        t.shape[0], t.shape[1], block_size, min_tokens, min_group,
                                        out.ctypes.data_as(_i32p), 32, ctypes.byref(n)))
    return [tuple(int(x) for x in out[3 * i:3 * i + 3]) for i in range(n.value)]


# ---------------------------------------------------------------------------
# Host block allocator.

def _i32(a):
    arr = np.ascontiguousarray(np.asarray(a, dtype=np.int32).reshape(-1))
    return arr, arr.ctypes.data_as(_i32p)


class BlockAllocator:
    """Ref-counted free-list allocator with copy-on-write (host only)."""

    def __init__(self, num_blocks, block_size):
        self._lib = load()
        h = _vp()
        _check(self._lib.pkv_allocator_create(num_blocks, block_size, ctypes.byref(h)))
        self._h = h
        self.num_blocks = num_blocks
        self.block_size = block_size

    def close(self):
        if getattr(self, "_h", None):
            self._lib.pkv_allocator_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    def set_free_order(self, order):
        arr, p = _i32(order)
        _check(self._lib.pkv_allocator_set_free_order(self._h, p, len(arr)))

    def allocate(self, n=1):
        out = np.empty(n, dtype=np.int32)
        _check(self._lib.pkv_allocate(self._h, n, out.ctypes.data_as(_i32p)))
        return out.tolist()

    def free(self, ids):
        arr, p = _i32(ids)
        _check(self._lib.pkv_free(self._h, p, len(arr)))

    def incref(self, ids):
        arr, p = _i32(ids)
        _check(self._lib.pkv_incref(self._h, p, len(arr)))

    def copy_on_write(self, block_id):
        new, copied = ctypes.c_int32(), ctypes.c_int()
        _check(self._lib.pkv_copy_on_write(self._h, block_id, ctypes.byref(new), ctypes.byref(copied)))
        return new.value, bool(copied.value)

    def ref_count(self, block_id):
        out = ctypes.c_int()
        _check(self._lib.pkv_ref_count(self._h, block_id, ctypes.byref(out)))
        return out.value

    def num_free(self):
        out = ctypes.c_int()
        _check(self._lib.pkv_num_free(self._h, ctypes.byref(out)))
        return out.value

    def usage_ratio(self):
        out = ctypes.c_double()
        _check(self._lib.pkv_usage_ratio(self._h, ctypes.byref(out)))
        return out.value

    def free_list(self):
        out = np.empty(self.num_blocks, dtype=np.int32)
        n = ctypes.c_int()
        _check(self._lib.pkv_free_list(self._h, out.ctypes.data_as(_i32p), self.num_blocks,
                                       ctypes.byref(n)))
        return out[:n.value].tolist()

    def cow_count(self):
        out = ctypes.c_int64()
        _check(self._lib.pkv_cow_count(self._h, ctypes.byref(out)))
        return out.value

    def seq_create(self):
        out = ctypes.c_int32()
        _check(self._lib.pkv_seq_create(self._h, ctypes.byref(out)))
        return out.value

    def seq_fork(self, seq):
        out = ctypes.c_int32()
        _check(self._lib.pkv_seq_fork(self._h, seq, ctypes.byref(out)))
        return out.value

    def seq_append_tokens(self, seq, n):
        """Returns (slots, cow_pairs) like the allocator model."""
        slots = np.empty(max(n, 1), dtype=np.int32)
        cow = np.empty(2, dtype=np.int32)
        ncow = ctypes.c_int()
        _check(self._lib.pkv_seq_append_tokens(self._h, seq, n, slots.ctypes.data_as(_i32p),
                                               cow.ctypes.data_as(_i32p), 1, ctypes.byref(ncow)))
        pairs = [(int(cow[0]), int(cow[1]))] if ncow.value else []
        return slots[:n].tolist(), pairs

    def seq_trim_window(self, seq, window):
        """Release the blocks behind the last ``window`` tokens; returns their ids."""
        cap = len(self.seq_block_ids(seq))
        out = np.empty(max(cap, 1), dtype=np.int32)
        n = ctypes.c_int()
        _check(self._lib.pkv_seq_trim_window(self._h, seq, window, out.ctypes.data_as(_i32p),
                                             cap, ctypes.byref(n)))
        return out[:n.value].tolist()

    def set_host_pool(self, num_host_blocks):
        _check(self._lib.pkv_allocator_set_host_pool(self._h, num_host_blocks))

    def host_num_free(self):
        out = ctypes.c_int()
        _check(self._lib.pkv_host_num_free(self._h, ctypes.byref(out)))
        return out.value

    def _swap(self, fn, seq):
        cap = len(self.seq_block_ids(seq))
        out = np.empty((max(cap, 1), 2), dtype=np.int32)
        n = ctypes.c_int()
        _check(fn(self._h, seq, out.ctypes.data_as(_i32p), cap, ctypes.byref(n)))
        return [tuple(int(x) for x in r) for r in out[:n.value]]

    def seq_swap_out(self, seq):
        """Preempt ``seq``; returns the (device, host) block pairs to copy out."""
        return self._swap(self._lib.pkv_seq_swap_out, seq)

    def seq_swap_in(self, seq):
        """Resume ``seq``; returns the (host, device) block pairs to copy in."""
        return self._swap(self._lib.pkv_seq_swap_in, seq)

    def seq_is_swapped(self, seq):
        out = ctypes.c_int()
        _check(self._lib.pkv_seq_is_swapped(self._h, seq, ctypes.byref(out)))
        return bool(out.value)

    def seq_free(self, seq):
        _check(self._lib.pkv_seq_free(self._h, seq))

    def seq_num_tokens(self, seq):
        out = ctypes.c_int()
        _check(self._lib.pkv_seq_num_tokens(self._h, seq, ctypes.byref(out)))
        return out.value

    def seq_block_ids(self, seq):
        n = ctypes.c_int()
        rc = self._lib.pkv_seq_block_ids(self._h, seq, None, 0, ctypes.byref(n))
        if rc not in (OK, ERR_INVALID_ARG):
            _check(rc)
        out = np.empty(max(n.value, 1), dtype=np.int32)
        _check(self._lib.pkv_seq_block_ids(self._h, seq, out.ctypes.data_as(_i32p), n.value,
                                           ctypes.byref(n)))
        return out[:n.value].tolist()

    def seq_physical_block(self, seq, token):
        out = ctypes.c_int32()
        _check(self._lib.pkv_seq_physical_block(self._h, seq, token, ctypes.byref(out)))
        return out.value

    def export_block_tables(self, seqs, max_blocks, pad=-1):
        arr, p = _i32(seqs)
        tables = np.empty((len(arr), max_blocks), dtype=np.int32)
        lens = np.empty(len(arr), dtype=np.int32)
        _check(self._lib.pkv_export_block_tables(self._h, p, len(arr), max_blocks, pad,
                                                 tables.ctypes.data_as(_i32p),
                                                 lens.ctypes.data_as(_i32p)))
        return tables, lens
