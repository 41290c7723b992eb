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
    before = (a.free_order(), a.ref_counts())
    with pytest.raises(OutOfBlocks):
        a.allocate(2)
    assert (a.free_order(), a.ref_counts()) == before


def test_double_free_leaves_state():
    a = AllocatorModel(4, 16)
    b = a.allocate(2)
    before = (a.free_order(), a.ref_counts())
    with pytest.raises(DoubleFree):
        a.free([b[0], b[0]])
    assert (a.free_order(), a.ref_counts()) == before
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
    assert a.refs(b) == 1 and a.refs(new) == 1
    with pytest.raises(ValueError):
        a.copy_on_write(a.free_order()[0])          # unowned block


def test_fork_and_partial_block_cow():
    bs = 16
    a = AllocatorModel(32, bs)
    parent = a.seq_create()
    a.seq_append_tokens(parent, 37)                # 2 full blocks + 5 tokens
    kids = [a.seq_fork(parent) for _ in range(3)]
    shared = a.table(parent)
    assert all(a.refs(b) == 4 for b in shared)
    copies = []
    for sid in kids + [parent]:
        slots, cow = a.seq_append_tokens(sid, 1)
        copies.append(cow)
        assert slots[0] % bs == 37 % bs
    # the first three writers copy the shared partial block; the last owner
    # writes in place
    assert [len(c) for c in copies] == [1, 1, 1, 0]
    assert all(c[0][0] == shared[2] for c in copies[:3])
    assert a.refs(shared[2]) == 1
    assert all(a.refs(b) == 4 for b in shared[:2])
    for sid in kids + [parent]:
        a.seq_free(sid)
    assert not any(a.ref_counts())
    assert sorted(a.free_order()) == list(range(32))


def test_append_all_or_nothing():
    a = AllocatorModel(3, 16)
    s = a.seq_create()
    a.seq_append_tokens(s, 40)                     # 3 blocks
    before = (a.free_order(), a.ref_counts(), a.table(s), a.length(s))
    with pytest.raises(OutOfBlocks):
        a.seq_append_tokens(s, 9)                  # needs a 4th block
    assert (a.free_order(), a.ref_counts(), a.table(s), a.length(s)) == before


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
            for b in a.table(sid):
                refs[b] += 1
        assert refs.tolist() == a.ref_counts()
        assert sorted(a.free_order() + [b for b in range(64) if refs[b]]) == list(range(64))
    for sid in live:
        a.seq_free(sid)
    assert not any(a.ref_counts())
    assert sorted(a.free_order()) == list(range(64))


# ---------------------------------------------------------------------------
# Swap pool ([P1] scheduler section, item 3: a preempted request's KV goes to
# CPU memory, its device blocks are freed, and it is copied back later).  The
# pins below simulate the memory contents the pair lists move, so they check
# the model against what a swap must achieve, not against its own code.

def _write_tokens(mem, slots, bs, values):
    for slot, v in zip(slots, values):
        mem.setdefault(slot // bs, {})[slot % bs] = v


def _gather(model, sid, mem):
    table = model.table(sid)
    bs = model.block_size
    return [mem[table[t // bs]][t % bs] for t in range(model.length(sid))]


def pin_swap_round_trip_preserves_contents(cls):
    """Contents survive swap-out, reuse of the freed device blocks by another
    request, and swap-in to different blocks; the running sequence that
    shares the preempted one's prompt blocks is never disturbed."""
    bs = 4
    m = cls(16, bs)
    m.set_host_pool(8)
    dev, host = {}, {}
    p = m.seq_create()
    slots, _ = m.seq_append_tokens(p, 10)
    _write_tokens(dev, slots, bs, [("p", i) for i in range(10)])
    c = m.seq_fork(p)
    slots, cow = m.seq_append_tokens(c, 7)
    for s_, d_ in cow:
        dev[d_] = dict(dev[s_])
    _write_tokens(dev, slots, bs, [("c", i) for i in range(7)])
    want_c, want_p = _gather(m, c, dev), _gather(m, p, dev)
    for d_, h_ in m.seq_swap_out(c):
        host[h_] = dict(dev[d_])
    assert m.seq_is_swapped(c)
    n = m.seq_create()                      # another request takes the freed blocks
    slots, _ = m.seq_append_tokens(n, len(m.free_order()) * bs)
    _write_tokens(dev, slots, bs, ["junk"] * len(slots))
    assert _gather(m, p, dev) == want_p
    m.seq_free(n)
    for h_, d_ in m.seq_swap_in(c):
        dev[d_] = dict(host[h_])
    assert not m.seq_is_swapped(c)
    assert _gather(m, c, dev) == want_c and _gather(m, p, dev) == want_p
    # it resumes: the next token lands after the restored ones
    slots, cow = m.seq_append_tokens(c, 1)
    assert not cow and slots[0] // bs == m.table(c)[-1]


def pin_swap_conservation(cls):
    """Random operations with swaps: every device block is either free or
    held by resident sequences exactly as often as its count says; every host
    block is either free or held by exactly one swapped-out sequence; swapping
    every sequence out frees the whole device pool."""
    rng = np.random.default_rng(9)
    nb, nhb, bs = 24, 20, 4
    m = cls(nb, bs)
    m.set_host_pool(nhb)
    live = []
    for _ in range(1500):
        op = int(rng.integers(0, 6))
        try:
            if op == 0 or not live:
                live.append(m.seq_create())
            elif op == 1:
                m.seq_append_tokens(live[rng.integers(len(live))], int(rng.integers(1, 9)))
            elif op == 2:
                live.append(m.seq_fork(live[rng.integers(len(live))]))
            elif op == 3:
                m.seq_free(live.pop(rng.integers(len(live))))
            elif op == 4:
                m.seq_swap_out(live[rng.integers(len(live))])
            else:
                m.seq_swap_in(live[rng.integers(len(live))])
        except (OutOfBlocks, ValueError):
            pass
        refs = np.zeros(nb, int)
        held_host = []
        for sid in live:
            ids = [b for b in m.table(sid) if b >= 0]
            if m.seq_is_swapped(sid):
                held_host += ids
            else:
                np.add.at(refs, ids, 1)
        assert refs.tolist() == m.ref_counts()
        assert sorted(m.free_order() + [b for b in range(nb) if refs[b]]) == list(range(nb))
        assert sorted(m.host_free_order() + held_host) == list(range(nhb))
    for sid in [s for s in live if m.seq_is_swapped(s)]:
        m.seq_free(sid)
        live.remove(sid)
    assert sorted(m.host_free_order()) == list(range(nhb))
    m.set_host_pool(nb * 2)
    for sid in live:
        m.seq_swap_out(sid)
    assert not any(m.ref_counts()) and sorted(m.free_order()) == list(range(nb))


def pin_swap_all_or_nothing(cls):
    m = cls(6, 4)
    m.set_host_pool(2)
    s = m.seq_create()
    m.seq_append_tokens(s, 12)
    before = (m.table(s), m.free_order(), m.host_free_order())
    with pytest.raises(OutOfBlocks):
        m.seq_swap_out(s)
    assert (m.table(s), m.free_order(), m.host_free_order()) == before
    with pytest.raises(ValueError):
        m.seq_swap_in(s)


SWAP_PINS = [pin_swap_round_trip_preserves_contents, pin_swap_conservation, pin_swap_all_or_nothing]


@pytest.mark.parametrize("pin", SWAP_PINS, ids=lambda f: f.__name__)
def test_swap_pins(pin):
    pin(AllocatorModel)


SWAP_MUTATIONS = {
    "pairs_reversed": ("out.append((dev, host))", "out.append((host, dev))"),
    "out_keeps_reference": ("            self.free([dev])\n", ""),
    "in_keeps_host_block": ("            self._host_stack.give_back(host)\n", ""),
    "in_pairs_reversed": ("pairs.append((host, dev))", "pairs.append((dev, host))"),
    "out_not_all_or_nothing": ("        if len(moving) > len(self._host_stack):\n"
                               "            raise OutOfBlocks(f\"need {len(moving)} host blocks, "
                               "{len(self._host_stack)} free\")\n", ""),
    "in_table_not_updated": ("            seq.table[j] = dev\n", ""),
}


@pytest.mark.parametrize("name", sorted(SWAP_MUTATIONS))
def test_swap_pins_catch_mutation(name):
    import types
    import oracle.allocator_model as am
    old, new = SWAP_MUTATIONS[name]
    src = open(am.__file__, encoding="utf-8").read()
    assert src.count(old) == 1, name
    mod = types.ModuleType(f"allocator_mutant_{name}")
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    caught = []
    for pin in SWAP_PINS:
        try:
            pin(mod.AllocatorModel)
        except (Exception, pytest.fail.Exception):
            caught.append(pin.__name__)
    assert caught, f"no pin caught {name}"
