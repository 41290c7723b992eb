"""Paged-attention decode and the cache write, written out plainly in fp64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): the product path never
imports this module.

What is computed, and where the pages define it:

* [P1] "PagedAttention分页内存管理原理": the cache is a pool of fixed-size
  physical blocks of ``block_size`` tokens; each sequence owns a logical block
  table mapping its logical block numbers to physical block numbers.
* [P1] "PagedAttention注意力计算流程" (kernel sketch) and [P3] section 二:
  logical token ``i`` lives in logical block ``i // block_size`` at offset
  ``i % block_size``; the physical row is ``phys * block_size + offset``, and
  inside that row the cache is laid out head-major then head_dim, so element
  ``(phys, off, kvh, d)`` sits at ``((phys*bs + off)*Hkv + kvh)*D + d``.
* [P1] kernel sketch: score = dot(q, k) * scale, then softmax over the
  context and the softmax-weighted sum of V (the sketch elides those two steps;
  they are the textbook definition of attention, written out below).
* [P2] "量化压缩KV Cache的INT8与FP8方案": an INT8 cache halves the bytes of
  an FP16 one.  The pages give no scale granularity; the reading taken here is
  symmetric INT8 with one fp32 scale per (physical block, kv head), value =
  code * scale.

Readings of points the pages leave open (each also listed in the design doc):

* one query per sequence (decode); per-sequence ``context_lens`` rather than
  the sketch's single ``context_len``; the table row stride is the table's
  second dimension (the sketch's undefined ``max_blocks``);
* grouped-query attention maps query head ``h`` to kv head ``h // (H // Hkv)``;
* a sequence with context length 0 yields an all-zero output;
* table entries past ``ceil(ctx / bs)`` and cache slots past ``ctx`` are never
  read, whatever their contents;
* the int8 cache write rounds ``x / scale`` in fp32, half to even, and
  saturates to [-127, 127];
* the page's FP8 option is read as OCP E4M3 codes with the same per-(block,
  kv head) scale, value = decode(code) * scale (``fp8_e4m3``);
* a sliding window W keeps the last W tokens, the decoded token included:
  positions max(0, n - W) .. n - 1 ([P2] sliding window section).

Pins (tests/oracle_pins.py, run by tests/test_oracle_decode.py): identity
tables against torch's CPU ``scaled_dot_product_attention`` in fp64; pure-Python
brute force on tiny shuffled tables; closed forms (ctx = 1, constant V, equal
keys, scale 0); a one-hot score probe; permutation of physical block ids;
shared-versus-duplicated blocks; GQA against MHA with repeated kv heads; NaN in
never-read slots; int8 against the float path on the dequantised values; the
cache write against per-element scalar assignment and a write-then-gather round
trip.  tests/test_oracle_mutations.py plants plausible mistakes in a copy of
this file and checks that the pins catch each one.
"""
import numpy as np

from . import fp8_e4m3

FORMATS = ("f32", "f16", "bf16", "i8", "fp8")
SCALED_FORMATS = ("i8", "fp8")


def to_f64(x, fmt):
    """Upcast stored values to float64 exactly.

    ``bf16`` arrays are carried as their raw uint16 bit patterns (numpy has no
    bfloat16); a bfloat16 is the upper half of an fp32, so shifting the bits
    left by 16 gives the fp32 of the same value.
    """
    if fmt == "bf16":
        bits = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    if fmt == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if fmt == "f16":
        return np.asarray(x, dtype=np.float16).astype(np.float64)
    if fmt == "i8":
        return np.asarray(x, dtype=np.int8).astype(np.float64)
    if fmt == "fp8":
        return fp8_e4m3.decode(x)
    raise ValueError(f"unknown format {fmt!r}")


def gather_context(key_cache, value_cache, table_row, n, block_size, kv_fmt,
                   k_scales=None, v_scales=None, start=0):
    """K and V of a sequence's logical tokens start .. n - 1, as float64
    [n - start, Hkv, D].

    Address translation of [P1] (kernel sketch) and [P3] section 二: token i is
    in logical block i // block_size at offset i % block_size, and the table row
    gives the physical block of each logical block.  Table entries of blocks
    that hold no token of the range are not looked at.
    """
    num_blocks = key_cache.shape[0]
    tokens = np.arange(start, n)
    logical_block = tokens // block_size
    offset = tokens % block_size
    if n and logical_block[-1] >= len(table_row):
        raise IndexError("context longer than the block table row")
    phys = np.asarray(table_row)[logical_block].astype(np.int64)
    if np.any(phys < 0) or np.any(phys >= num_blocks):
        raise IndexError("block table entry outside the physical pool")
    k = to_f64(key_cache[phys, offset], kv_fmt)
    v = to_f64(value_cache[phys, offset], kv_fmt)
    if kv_fmt in SCALED_FORMATS:
        # One scale per (physical block, kv head), applied to every element of
        # that block's rows for that head.
        k = k * np.asarray(k_scales, dtype=np.float64)[phys][:, :, None]
        v = v * np.asarray(v_scales, dtype=np.float64)[phys][:, :, None]
    return k, v


def paged_decode(q, q_fmt, key_cache, value_cache, kv_fmt, block_tables,
                 context_lens, block_size, scale, k_scales=None, v_scales=None,
                 window=0):
    """Decode attention over a paged KV cache; returns float64 [B, H, D].

    q            [B, H, D] in ``q_fmt``
    key_cache    [NB, block_size, Hkv, D] in ``kv_fmt``; value_cache likewise
    block_tables [B, MB] int, context_lens [B] int
    k_scales, v_scales [NB, Hkv] fp32 (``kv_fmt`` "i8" or "fp8" only)
    window       0, or the sliding window W of [P2] "Sliding Window
                 Attention控制长序列显存": positions max(0, n - W) .. n - 1 of a
                 context of n tokens are attended to

    For each sequence s and query head h: gather the attended keys and values
    through the table (the first ctx[s] tokens, or the last W of them), score
    each key as scale * dot(q, k), take the softmax of the scores (shifted by
    their maximum, which leaves the softmax unchanged and keeps exp in range)
    and return the weighted sum of values.
    """
    q = np.asarray(q)
    num_seqs, num_heads, head_dim = q.shape
    num_kv_heads = key_cache.shape[2]
    if num_heads % num_kv_heads:
        raise ValueError("num_heads must be a multiple of num_kv_heads")
    group = num_heads // num_kv_heads
    block_tables = np.asarray(block_tables)
    out = np.zeros((num_seqs, num_heads, head_dim), dtype=np.float64)
    for s in range(num_seqs):
        n = int(context_lens[s])
        if n == 0:
            continue
        start = max(0, n - int(window)) if window else 0
        k, v = gather_context(key_cache, value_cache, block_tables[s], n,
                              block_size, kv_fmt, k_scales, v_scales, start)
        qs = to_f64(q[s], q_fmt)
        for h in range(num_heads):
            kvh = h // group
            scores = scale * (k[:, kvh, :] @ qs[h])
            m = scores.max()
            w = np.exp(scores - m)
            out[s, h] = (w @ v[:, kvh, :]) / w.sum()
    return out


def reshape_and_cache(k, v, src_fmt, key_cache, value_cache, kv_fmt,
                      slot_mapping, block_size, k_scales=None, v_scales=None,
                      in_place=False):
    """Scatter new tokens' K/V rows into their cache slots.

    k, v [T, Hkv, D] in ``src_fmt``; slot_mapping [T] int.  Token t goes to
    physical block slot // block_size, offset slot % block_size (the inverse of
    the sketch's physical offset phys * block_size + offset); a negative slot
    means "no slot" and the token is skipped.  Float caches take the rows
    unchanged (``src_fmt`` must equal ``kv_fmt``).  An int8 cache stores
    clip(rint(x / scale), -127, 127) with the existing scale of that
    (block, kv head); the division and the rounding are done in fp32, half to
    even.  An fp8 cache stores the E4M3 code of x / scale (division in fp32,
    nearest value, ties to even, saturating at 448; see ``fp8_e4m3``).
    Returns the (possibly copied) caches.
    """
    if not in_place:
        key_cache = key_cache.copy()
        value_cache = value_cache.copy()
    for t, slot in enumerate(np.asarray(slot_mapping).tolist()):
        if slot < 0:
            continue
        blk, off = slot // block_size, slot % block_size
        if blk >= key_cache.shape[0]:
            raise IndexError("slot outside the physical pool")
        if kv_fmt == "i8":
            for src, cache, scales in ((k, key_cache, k_scales),
                                       (v, value_cache, v_scales)):
                x = to_f64(src[t], src_fmt).astype(np.float32)  # exact
                sc = np.asarray(scales, dtype=np.float32)[blk][:, None]
                code = np.clip(np.rint(x / sc), -127, 127)
                cache[blk, off] = code.astype(np.int8)
        elif kv_fmt == "fp8":
            for src, cache, scales in ((k, key_cache, k_scales),
                                       (v, value_cache, v_scales)):
                x = to_f64(src[t], src_fmt).astype(np.float32)  # exact
                sc = np.asarray(scales, dtype=np.float32)[blk][:, None]
                cache[blk, off] = fp8_e4m3.encode(x / sc)
        else:
            if src_fmt != kv_fmt:
                raise ValueError("float caches take rows of their own format")
            key_cache[blk, off] = k[t]
            value_cache[blk, off] = v[t]
    return key_cache, value_cache
