"""Seeded synthetic decode workloads, shared by the tests and the benchmark.

This module draws inputs only.  It holds none of the method's arithmetic:
no attention, no cache write, no address translation beyond naming which
cache slot the newest token of each sequence occupies, and it imports neither
the HIP binding nor the CPU oracle.  Both sides receive the same arrays.

The pages measure Llama-2 class models serving real requests; those weights
and request traces are not available, so these layers stand in for their
shapes: 64 heads of dimension 128 in FP16 at 2048 tokens and batch 32 (the
70B memory example of [P1] "大模型推理KV Cache内存消耗模型"), block size 16
([P1] "PagedAttention分页内存管理原理"), a 2000-token shared system prompt
([P2] "Prefix Cache复用共享前缀的KV Cache") and an INT8 cache ([P2]
"量化压缩KV Cache的INT8与FP8方案").

A sliding-window workload keeps, per sequence, only the blocks that hold one
of its last W tokens (the others are released, their table entries -1), as
[P2] "Sliding Window Attention控制长序列显存" describes for Mistral-7B with
W = 4096.

Recipe (``np.random.default_rng(seed)``; draw order ctx -> pool permutation
-> Q -> K -> V -> new K -> new V):

* block tables come from a seeded permutation of the physical pool handed
  out the way a LIFO free list does: the permutation is the free list, blocks
  are popped from its end, sequence by sequence;
* a shared prefix is allocated once and every sequence's table starts with
  the same physical blocks (reference count = number of sequences);
* Q, K, V are N(0, 1) drawn in fp32 and rounded to the storage format
  (round to nearest even); bfloat16 arrays are carried as uint16 bits;
* an int8 cache is quantised per (physical block, kv head) with
  scale = max|x| / 127 over that block's rows (scale 1 if all are zero) and
  code = rint(x / scale) clipped to [-127, 127];
* an fp8 (E4M3) cache likewise with scale = max|x| / 448 and the codes of
  x / scale from torch's float8_e4m3fn conversion (a library routine: this
  module still holds none of the method's arithmetic); fp8 codes are carried
  as uint8;
* the newest token of sequence s is its last context position ctx[s] - 1,
  and ``slot_mapping[s]`` names that token's cache slot.
"""
from dataclasses import dataclass, field
import math

import numpy as np

BLOCK_SIZE = 16

# (index, name, description) of the five standard configurations.
CONFIG_NAMES = {
    1: "tiny_fp32_mha",
    2: "llama2_7b_fp16_mha",
    3: "llama2_70b_fp16_mha",
    4: "shared_prefix_gqa_bf16",
    5: "high_concurrency_int8_gqa",
    6: "sliding_window_gqa_bf16",
    7: "llama2_70b_fp8_mha",
    8: "high_concurrency_fp8_gqa",
}
SCALED_FORMATS = ("i8", "fp8")


@dataclass
class Workload:
    name: str
    seed: int
    q: np.ndarray                 # [B, H, D], q_fmt
    q_fmt: str
    key_cache: np.ndarray         # [NB, bs, Hkv, D], kv_fmt
    value_cache: np.ndarray
    kv_fmt: str
    block_tables: np.ndarray      # [B, MB] int32, -1 padded
    context_lens: np.ndarray      # [B] int32
    block_size: int
    scale: float
    k_new: np.ndarray             # [B, Hkv, D], new_fmt
    v_new: np.ndarray
    new_fmt: str
    slot_mapping: np.ndarray      # [B] int32
    k_scales: np.ndarray = None   # [NB, Hkv] fp32 (int8 and fp8 only)
    v_scales: np.ndarray = None
    shared_prefix_blocks: int = 0
    window: int = 0               # sliding window in tokens (0 = whole context)
    extra: dict = field(default_factory=dict)

    @property
    def num_seqs(self):
        return self.q.shape[0]

    @property
    def num_heads(self):
        return self.q.shape[1]

    @property
    def head_dim(self):
        return self.q.shape[2]

    @property
    def num_kv_heads(self):
        return self.key_cache.shape[2]

    @property
    def num_blocks(self):
        return self.key_cache.shape[0]

    @property
    def max_blocks_per_seq(self):
        return self.block_tables.shape[1]

    def referenced_blocks(self):
        """Sorted unique physical block ids any sequence reads."""
        ids = []
        for s in range(self.num_seqs):
            n = int(self.context_lens[s])
            nb = (n + self.block_size - 1) // self.block_size
            fb = max(0, n - self.window) // self.block_size if self.window else 0
            ids.append(self.block_tables[s, fb:nb])
        return np.unique(np.concatenate(ids)) if ids else np.zeros(0, np.int32)


def _round_to(x32, fmt):
    """Round fp32 draws to the storage format (nearest even)."""
    if fmt == "f32":
        return x32.astype(np.float32)
    if fmt == "f16":
        return x32.astype(np.float16)
    if fmt == "bf16":
        u = x32.astype(np.float32).view(np.uint32)
        rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
        return rounded.astype(np.uint16)
    raise ValueError(fmt)


def _normal(rng, shape, fmt):
    return _round_to(rng.standard_normal(shape, dtype=np.float32), fmt)


def _quantise_blocks(x32):
    """int8 codes and per-(block, kv head) scales for x32 [NB, bs, Hkv, D]."""
    amax = np.abs(x32).max(axis=(1, 3))                    # [NB, Hkv]
    scales = np.where(amax > 0, amax / np.float32(127.0), np.float32(1.0)).astype(np.float32)
    codes = np.clip(np.rint(x32 / scales[:, None, :, None]), -127, 127).astype(np.int8)
    return codes, scales


def _quantise_blocks_fp8(x32):
    """fp8 E4M3 codes (uint8) and per-(block, kv head) scales for x32."""
    import torch
    amax = np.abs(x32).max(axis=(1, 3))
    scales = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    y = np.clip(x32 / scales[:, None, :, None], -448, 448).astype(np.float32)
    codes = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, scales


def _draw_lengths(cfg, rng, num_seqs):
    kind = cfg["ctx"][0]
    if kind == "fixed":
        lens = np.asarray(cfg["ctx"][1], dtype=np.int64)
        if lens.size == 1:
            lens = np.full(num_seqs, int(lens.reshape(-1)[0]), dtype=np.int64)
    elif kind == "uniform":
        lo, hi = cfg["ctx"][1], cfg["ctx"][2]
        lens = rng.integers(lo, hi + 1, size=num_seqs)
    elif kind == "prefix_plus_uniform":
        prefix, lo, hi = cfg["ctx"][1], cfg["ctx"][2], cfg["ctx"][3]
        lens = prefix + rng.integers(lo, hi + 1, size=num_seqs)
    elif kind == "lognormal":
        median, sigma, cap = cfg["ctx"][1], cfg["ctx"][2], cfg["ctx"][3]
        raw = np.exp(rng.normal(math.log(median), sigma, size=num_seqs))
        lens = np.clip(np.rint(raw), 1, cap).astype(np.int64)
    else:
        raise ValueError(kind)
    return lens.astype(np.int32)


def _spec(index):
    """The five configurations (full size)."""
    if index == 1:
        return dict(num_seqs=2, num_heads=4, num_kv_heads=4, head_dim=64,
                    kv_fmt="f32", q_fmt="f32", ctx=("fixed", [37, 100]),
                    pool=("fixed", 32), max_blocks=7, prefix=0)
    if index == 2:
        return dict(num_seqs=32, num_heads=32, num_kv_heads=32, head_dim=128,
                    kv_fmt="f16", q_fmt="f16", ctx=("uniform", 128, 2048),
                    pool=("factor", 1.25), max_blocks=128, prefix=0)
    if index == 3:
        return dict(num_seqs=32, num_heads=64, num_kv_heads=64, head_dim=128,
                    kv_fmt="f16", q_fmt="f16", ctx=("fixed", [2048]),
                    pool=("factor", 1.0), max_blocks=128, prefix=0)
    if index == 4:
        return dict(num_seqs=64, num_heads=64, num_kv_heads=8, head_dim=128,
                    kv_fmt="bf16", q_fmt="bf16",
                    ctx=("prefix_plus_uniform", 2000, 1, 512),
                    pool=("factor", 1.25), max_blocks=157, prefix=2000)
    if index == 5:
        return dict(num_seqs=256, num_heads=32, num_kv_heads=8, head_dim=128,
                    kv_fmt="i8", q_fmt="f16", ctx=("lognormal", 512, 0.8, 4096),
                    pool=("factor", 1.25), max_blocks=256, prefix=0)
    if index == 6:
        return dict(num_seqs=32, num_heads=32, num_kv_heads=8, head_dim=128,
                    kv_fmt="bf16", q_fmt="bf16", ctx=("uniform", 4096, 16384),
                    pool=("factor", 1.25), max_blocks=1024, prefix=0, window=4096)
    if index == 7:   # the 70B-shaped layer of configuration 3 with an FP8 cache
        return dict(_spec(3), kv_fmt="fp8")
    if index == 8:   # the high-concurrency GQA batch of configuration 5 with an FP8 cache
        return dict(_spec(5), kv_fmt="fp8")
    raise ValueError(f"no configuration {index}")


def _config(index, overrides):
    cfg = dict(_spec(index))
    for key, val in overrides.items():
        if val is not None:
            cfg[key] = val
    return cfg


def _draw_structure(cfg, rng, bs):
    """Context lengths and block tables (the first two draws of the recipe)."""
    B, H, Hkv = cfg["num_seqs"], cfg["num_heads"], cfg["num_kv_heads"]
    if H % Hkv:
        raise ValueError("num_heads must be a multiple of num_kv_heads")
    lens = _draw_lengths(cfg, rng, B)
    prefix_tokens = int(cfg["prefix"])
    prefix_blocks = prefix_tokens // bs if prefix_tokens else 0
    blocks_per_seq = (lens.astype(np.int64) + bs - 1) // bs
    # With a sliding window only the blocks that hold one of the last `window`
    # tokens are kept; the table entries before them are -1 (released).
    window = int(cfg.get("window", 0))
    if window and prefix_tokens:
        raise ValueError("a shared prefix and a sliding window are not combined")
    first_block = (np.maximum(lens.astype(np.int64) - window, 0) // bs if window
                   else np.zeros(B, dtype=np.int64))
    if prefix_tokens and lens.min() <= prefix_tokens:
        raise ValueError("every sequence must extend past the shared prefix")
    own_blocks = blocks_per_seq - prefix_blocks - first_block
    needed = int(prefix_blocks + own_blocks.sum())
    if cfg["pool"][0] == "fixed":
        nb = int(cfg["pool"][1])
    else:
        nb = int(math.ceil(cfg["pool"][1] * needed))
    if nb < needed:
        raise ValueError("pool smaller than the blocks the sequences need")
    mb = int(cfg["max_blocks"])
    if blocks_per_seq.max() > mb:
        raise ValueError("max_blocks smaller than the longest sequence")

    # Free list = a seeded permutation; blocks leave from its end.
    free_list = rng.permutation(nb).astype(np.int32)
    handout = free_list[::-1]
    tables = np.full((B, mb), -1, dtype=np.int32)
    pos = 0
    shared = handout[pos:pos + prefix_blocks]
    pos += prefix_blocks
    for s in range(B):
        tables[s, :prefix_blocks] = shared
        n_own = int(own_blocks[s])
        lo = prefix_blocks + int(first_block[s])
        tables[s, lo:lo + n_own] = handout[pos:pos + n_own]
        pos += n_own
    return dict(lens=lens, tables=tables, num_blocks=nb, prefix_blocks=prefix_blocks,
                free_list=free_list, blocks_needed=needed)


def make_structure(index, seed=None, block_size=BLOCK_SIZE, **overrides):
    """Only the context lengths and block tables of a configuration (cheap)."""
    cfg = _config(index, overrides)
    rng = np.random.default_rng(index - 1 if seed is None else seed)
    return _draw_structure(cfg, rng, block_size)


def make_workload(index, seed=None, *, num_seqs=None, num_heads=None,
                  num_kv_heads=None, head_dim=None, ctx=None, prefix=None,
                  max_blocks=None, kv_fmt=None, q_fmt=None, block_size=BLOCK_SIZE,
                  poison_unused=False, pool=None, window=None):
    """Draw configuration ``index`` (1..8) with optional overrides.

    Overrides shrink or reshape a configuration for parity tests while keeping
    its structure (length mix, sharing, formats).  ``poison_unused`` fills every
    cache slot no sequence reads with NaN (float caches) or with +/-127 codes
    (int8), and leaves -1 in the table padding, so that a reader that touches
    them shows it.
    """
    cfg = _config(index, dict(num_seqs=num_seqs, num_heads=num_heads,
                              num_kv_heads=num_kv_heads, head_dim=head_dim,
                              kv_fmt=kv_fmt, q_fmt=q_fmt, ctx=ctx, prefix=prefix,
                              max_blocks=max_blocks, pool=pool, window=window))
    if seed is None:
        seed = index - 1
    rng = np.random.default_rng(seed)
    B, H, Hkv, D = cfg["num_seqs"], cfg["num_heads"], cfg["num_kv_heads"], cfg["head_dim"]
    bs = block_size
    st = _draw_structure(cfg, rng, bs)
    lens, tables, nb = st["lens"], st["tables"], st["num_blocks"]

    kv_fmt_, q_fmt_ = cfg["kv_fmt"], cfg["q_fmt"]
    q = _normal(rng, (B, H, D), q_fmt_)
    pool_shape = (nb, bs, Hkv, D)
    k_scales = v_scales = None
    if kv_fmt_ in SCALED_FORMATS:
        quant = _quantise_blocks if kv_fmt_ == "i8" else _quantise_blocks_fp8
        key_cache, k_scales = quant(rng.standard_normal(pool_shape, dtype=np.float32))
        value_cache, v_scales = quant(rng.standard_normal(pool_shape, dtype=np.float32))
        new_fmt = q_fmt_
    else:
        key_cache = _normal(rng, pool_shape, kv_fmt_)
        value_cache = _normal(rng, pool_shape, kv_fmt_)
        new_fmt = kv_fmt_
    k_new = _normal(rng, (B, Hkv, D), new_fmt)
    v_new = _normal(rng, (B, Hkv, D), new_fmt)

    last = np.maximum(lens - 1, 0)
    last_block = tables[np.arange(B), last // bs]
    slots = np.where(lens > 0, last_block * bs + last % bs, -1).astype(np.int32)

    wl = Workload(
        name=CONFIG_NAMES.get(index, f"config{index}"), seed=seed,
        q=q, q_fmt=q_fmt_, key_cache=key_cache, value_cache=value_cache,
        kv_fmt=kv_fmt_, block_tables=tables, context_lens=lens, block_size=bs,
        scale=1.0 / math.sqrt(D), k_new=k_new, v_new=v_new, new_fmt=new_fmt,
        slot_mapping=slots, k_scales=k_scales, v_scales=v_scales,
        shared_prefix_blocks=st["prefix_blocks"], window=int(cfg.get("window", 0)),
        extra={"free_list": st["free_list"], "blocks_needed": st["blocks_needed"]},
    )
    if poison_unused:
        poison(wl)
    return wl


def used_slot_mask(wl):
    """Boolean [NB, bs]: True where some sequence's context (its window, if the
    workload has one) reads the slot."""
    used = np.zeros((wl.num_blocks, wl.block_size), dtype=bool)
    for s in range(wl.num_seqs):
        n = int(wl.context_lens[s])
        first = max(0, n - wl.window) if wl.window else 0
        for i in range(first, n):
            used[wl.block_tables[s, i // wl.block_size], i % wl.block_size] = True
    return used


def poison(wl):
    """Fill unread cache slots with NaN (float; the NaN code 0x7F for fp8) or
    alternating +/-127 (int8)."""
    unused = ~used_slot_mask(wl)
    for cache in (wl.key_cache, wl.value_cache):
        if wl.kv_fmt == "fp8":
            cache[unused] = np.uint8(0x7F)
        elif wl.kv_fmt == "i8":
            cache[unused] = np.int8(127)
            cache[unused, ..., 1::2] = np.int8(-127)
        elif wl.kv_fmt == "bf16":
            cache[unused] = np.uint16(0x7FC0)
        else:
            cache[unused] = np.nan
    return wl
