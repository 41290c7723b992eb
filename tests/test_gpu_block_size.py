"""Decode with 8- and 32-token blocks ([P1] "vLLM部署配置与PagedAttention参数调优":
the block size trades table overhead against internal fragmentation) against
the oracle, which takes any block size."""
import numpy as np
import pytest
import torch

import paged_kv_cache_379_amd as pkv_mod
from gpu_util import assert_parity, gpu_decode, oracle_decode, out_f64
from paged_kv_cache_379_amd import workloads as W

pytestmark = pytest.mark.gpu

LENS = [1, 7, 8, 9, 17, 300, 513, 700]


@pytest.mark.parametrize("bs", [8, 32])
@pytest.mark.parametrize("kv_fmt,q_fmt", [("f32", "f32"), ("f16", "f16"), ("bf16", "bf16"),
                                          ("i8", "f16"), ("fp8", "bf16")])
@pytest.mark.parametrize("head_dim", [64, 128])
@pytest.mark.parametrize("group", [1, 2, 4, 8, 16])
def test_block_size_parity(gpu_lib, bs, kv_fmt, q_fmt, head_dim, group):
    """Every kernel at block sizes 8 and 32: ragged lengths around the block
    and tile boundaries, whole contexts and 32-token partitions, poisoned
    unread slots and table padding.  One-byte multi-head rows of head_dim 64
    at 8-token blocks fill 16 rows per load instruction, two blocks' worth:
    the rows past the block are re-read and masked."""
    wl = W.make_workload(2, seed=11 + group + bs, num_seqs=len(LENS), num_heads=2 * group,
                         num_kv_heads=2, head_dim=head_dim, kv_fmt=kv_fmt, q_fmt=q_fmt,
                         ctx=("fixed", LENS), max_blocks=-(-700 // bs) + 3, block_size=bs,
                         poison_unused=True)
    ref = oracle_decode(wl)
    for part in (0, 32, 64):
        got = out_f64(gpu_decode(gpu_lib, wl, partition_size=part))
        assert_parity(got, ref, kv_fmt, q_fmt, with_output_rounding=True,
                      label=f"bs={bs} {kv_fmt}/{q_fmt} D={head_dim} G={group} part={part}")


@pytest.mark.parametrize("bs", [8, 16, 32])
@pytest.mark.parametrize("kv_fmt,q_fmt", [("i8", "f16"), ("fp8", "bf16")])
def test_one_byte_head_dim_64(gpu_lib, kv_fmt, q_fmt, bs):
    """One-byte multi-head rows of head_dim 64: every length from 1 to 44 (each
    offset of the last block), whole and split contexts.  With 16-token (or
    block-sized) partitions 8 and 16 kv heads put two and four kv heads in a
    workgroup, whose load rows then cover two heads each; one kv head reads
    half-line rows (and at 8-token blocks re-reads the block's rows)."""
    for hkv in (1, 8, 16):
        wl = W.make_workload(2, seed=40 + hkv + bs, num_seqs=44, num_heads=hkv, num_kv_heads=hkv,
                             head_dim=64, kv_fmt=kv_fmt, q_fmt=q_fmt,
                             ctx=("fixed", list(range(1, 45))), max_blocks=-(-48 // bs),
                             block_size=bs, poison_unused=True)
        ref = oracle_decode(wl)
        for part in (0, max(bs, 16)):
            got = out_f64(gpu_decode(gpu_lib, wl, partition_size=part))
            assert_parity(got, ref, kv_fmt, q_fmt, with_output_rounding=True,
                          label=f"{kv_fmt} bs={bs} Hkv={hkv} part={part}")


@pytest.mark.parametrize("kv_fmt,q_fmt", [("fp8", "f16"), ("i8", "bf16")])
def test_one_byte_head_dim_64_head_pairs_70b_shape(gpu_lib, kv_fmt, q_fmt):
    """The 70B-shaped layer's heads at head_dim 64 with a one-byte cache: 32
    sequences x 64 kv heads give four kv heads per workgroup, read two per
    load row; ragged lengths, table padding and unread slots poisoned."""
    rng = np.random.default_rng(64)
    lens = [int(x) for x in rng.integers(1, 400, 32)]
    wl = W.make_workload(3, seed=64, num_seqs=32, head_dim=64, kv_fmt=kv_fmt, q_fmt=q_fmt,
                         ctx=("fixed", lens), max_blocks=26, poison_unused=True)
    assert pkv_mod.decode_partition_size(32, 64, 64, 64, 16, 26) == 0
    got = out_f64(gpu_decode(gpu_lib, wl))
    ref = oracle_decode(wl)
    assert_parity(got, ref, kv_fmt, q_fmt, with_output_rounding=True, label=f"{kv_fmt} D=64 pairs")


@pytest.mark.parametrize("bs", [8, 32])
@pytest.mark.parametrize("kv_fmt,q_fmt,group", [("f16", "f16", 1), ("bf16", "bf16", 8),
                                                ("i8", "f16", 4), ("fp8", "f16", 2)])
def test_block_size_sliding_window(gpu_lib, bs, kv_fmt, q_fmt, group):
    """Windows that start inside a block and inside a tile; the blocks wholly
    behind the window are released (-1) and their slots poisoned."""
    from test_gpu_decode import _behind_window
    hkv = 2
    wl = W.make_workload(2, seed=5 + bs, num_seqs=5, num_heads=group * hkv, num_kv_heads=hkv,
                         head_dim=128, kv_fmt=kv_fmt, q_fmt=q_fmt,
                         ctx=("fixed", [1, 17, 300, 700, 1000]), max_blocks=-(-1000 // bs) + 2,
                         block_size=bs, poison_unused=True)
    for window in (1, 7, 8, 9, 24, 333, 5000):
        w2 = _behind_window(wl, window)
        ref = oracle_decode(w2, window=window)
        for part in (0, 64):
            got = out_f64(gpu_decode(gpu_lib, w2, partition_size=part, window=window))
            assert_parity(got, ref, kv_fmt, q_fmt, with_output_rounding=True,
                          label=f"bs={bs} {kv_fmt} G={group} W={window} part={part}")


@pytest.mark.parametrize("bs", [8, 32])
@pytest.mark.parametrize("group", [1, 8])
def test_block_size_one_hot_gather(gpu_lib, bs, group):
    """Each position t* of a context scores far above the others, so the output
    is V[t*] bit for bit: the address translation at every offset of 8- and
    32-token blocks (and of the two-blocks-per-tile case)."""
    hkv, n = 2, 70
    wl = W.make_workload(2, seed=3, num_seqs=1, num_heads=group * hkv, num_kv_heads=hkv,
                         head_dim=128, kv_fmt="f16", q_fmt="f16", ctx=("fixed", [n]),
                         max_blocks=-(-n // bs) + 1, block_size=bs)
    q = np.zeros(wl.q.shape, np.float32)
    q[..., 0] = 1.0
    wl.q = q.astype(np.float16)
    table = wl.block_tables[0]
    for t_star in range(n):
        kc = wl.key_cache.copy()
        for i in range(n):
            kc[table[i // bs], i % bs, :, 0] = 0.0
        kc[table[t_star // bs], t_star % bs, :, 0] = 2000.0
        saved = wl.key_cache
        wl.key_cache = kc
        out = gpu_decode(gpu_lib, wl).cpu().numpy()
        wl.key_cache = saved
        want = np.repeat(wl.value_cache[table[t_star // bs], t_star % bs], group, axis=0)
        assert np.array_equal(out[0], want), (bs, group, t_star)


@pytest.mark.parametrize("bs", [8, 32])
def test_block_size_full_size(gpu_lib, bs):
    """The 70B-shaped layer (32 x 2048 tokens, 64 heads) at block size bs in the
    benchmark's launch configuration; every sequence against the oracle."""
    wl = W.make_workload(3, block_size=bs, max_blocks=2048 // bs)
    got = out_f64(gpu_decode(gpu_lib, wl))
    err = assert_parity(got, oracle_decode(wl), "f16", label=f"70B layer bs={bs}")
    print(f"70B layer bs={bs}: all {wl.num_seqs} sequences, max abs err {err:.3g}")
