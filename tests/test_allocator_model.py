"""The allocator model (oracle) against the pages' printed tables and semantics (CPU)."""
import json
import os

import numpy as np
import pytest

from oracle.allocator_model import AllocatorModel, DoubleFree, OutOfBlocks

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _flowchart():
    with open(os.path.join(GOLDEN, "p3_flowchart_block_tables.json"), encoding="utf-8") as f:
        return json.load(f)


def test_flowchart_tables_and_translations():
    fx = _flowchart()
    bs = fx["block_size"]
    n = sum(len(t) for t in fx["tables"].values())
    a = AllocatorModel(n, bs)
    # Free list ordered so that pops from its end hand out 0, 1, 2, ...
    a.set_free_order(list(range(n - 1, -1, -1)))
    sids = {name: a.seq_create() for name in fx["tables"]}
    for name in fx["allocation_order"]:
        sid = sids[name]
        # append one block's worth of tokens: the first token opens a new block
        a.seq_append_tokens(sid, bs)
    for name, table in fx["tables"].items():
        got, _ = a.export_block_tables([sids[name]], len(table))
        assert got[0] == table
    for tr in fx["translations"]:
        sid = sids[tr["seq"]]
        assert a.seq_physical_block(sid, tr["token"]) == tr["physical_block"]
        assert tr["physical_block"] * bs + tr["token"] % bs == tr["slot"]
    for lk in fx["unallocated_lookups"]:
        with pytest.raises(IndexError):
            a.seq_physical_block(sids[lk["seq"]], lk["token"])


def test_lifo_pop_from_end():
    a = AllocatorModel(8, 16)
    assert a.allocate(3) == [7, 6, 5]      # pop() from the end of range(8)
    a.free([6])
    assert a.allocate(1) == [6]            # a freed block is reused first
    assert a.usage_ratio() == pytest.approx(3 / 8)


def test_oom_all_or_nothing():
    a = AllocatorModel(4, 16)
    a.allocate(3)
    before = (list(a.free_blocks), list(a.ref_count))
    with pytest.raises(OutOfBlocks):
        a.allocate(2)
    assert (a.free_blocks, a.ref_count) == before


def test_double_free_leaves_state():
    a = AllocatorModel(4, 16)
    b = a.allocate(2)
    before = (list(a.free_blocks), list(a.ref_count))
    with pytest.raises(DoubleFree):
        a.free([b[0], b[0]])
    assert (a.free_blocks, a.ref_count) == before
    a.free([b[0]])
    with pytest.raises(DoubleFree):
        a.free([b[0]])


def test_copy_on_write_semantics():
    a = AllocatorModel(6, 16)
    (b,) = a.allocate(1)
    assert a.copy_on_write(b) == (b, False)        # sole owner writes in place
    a.incref([b])
    new, copied = a.copy_on_write(b)
    assert copied and new != b
    assert a.ref_count[b] == 1 and a.ref_count[new] == 1
    with pytest.raises(ValueError):
        a.copy_on_write(a.free_blocks[0])          # unowned block


def test_fork_and_partial_block_cow():
    bs = 16
    a = AllocatorModel(32, bs)
    parent = a.seq_create()
    a.seq_append_tokens(parent, 37)                # 2 full blocks + 5 tokens
    kids = [a.seq_fork(parent) for _ in range(3)]
    shared = a.seqs[parent]["blocks"]
    assert all(a.ref_count[b] == 4 for b in shared)
    copies = []
    for sid in kids + [parent]:
        slots, cow = a.seq_append_tokens(sid, 1)
        copies.append(cow)
        assert slots[0] % bs == 37 % bs
    # the first three writers copy the shared partial block; the last owner
    # writes in place
    assert [len(c) for c in copies] == [1, 1, 1, 0]
    assert all(c[0][0] == shared[2] for c in copies[:3])
    assert a.ref_count[shared[2]] == 1
    assert all(a.ref_count[b] == 4 for b in shared[:2])
    for sid in kids + [parent]:
        a.seq_free(sid)
    assert not any(a.ref_count)
    assert sorted(a.free_blocks) == list(range(32))


def test_append_all_or_nothing():
    a = AllocatorModel(3, 16)
    s = a.seq_create()
    a.seq_append_tokens(s, 40)                     # 3 blocks
    before = (list(a.free_blocks), list(a.ref_count), dict(a.seqs[s]))
    with pytest.raises(OutOfBlocks):
        a.seq_append_tokens(s, 9)                  # needs a 4th block
    assert (a.free_blocks, a.ref_count, a.seqs[s]) == (before[0], before[1], before[2])


def test_random_ops_invariants():
    rng = np.random.default_rng(5)
    a = AllocatorModel(64, 16)
    a.set_free_order(rng.permutation(64).tolist())
    live = []
    for _ in range(2000):
        op = rng.integers(0, 4)
        try:
            if op == 0 or not live:
                live.append(a.seq_create())
            elif op == 1:
                a.seq_append_tokens(live[rng.integers(len(live))], int(rng.integers(1, 40)))
            elif op == 2:
                live.append(a.seq_fork(live[rng.integers(len(live))]))
            else:
                a.seq_free(live.pop(rng.integers(len(live))))
        except OutOfBlocks:
            pass
        refs = np.zeros(64, int)
        for sid in live:
            for b in a.seqs[sid]["blocks"]:
                refs[b] += 1
        assert refs.tolist() == a.ref_count
        assert sorted(a.free_blocks + [b for b in range(64) if refs[b]]) == list(range(64))
    for sid in live:
        a.seq_free(sid)
    assert not any(a.ref_count)
    assert sorted(a.free_blocks) == list(range(64))
