"""Reference model of the ref-counted free-list block allocator.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  The C++ allocator in the
library is checked against this model op by op on random op sequences.

What the model follows: [P3] section 二 (a block manager that hands out
fixed-size blocks from a free list, counts the owners of each block, gives a
writer of a shared block its own copy, and reports the share of the pool in
use; per-sequence tables from logical to physical blocks), [P1]
"PagedAttention分页内存管理原理" (equal-size blocks, so one free list is enough)
and [P1] "vLLM调度器与PagedAttention协同工作" (a block is taken when a token
crosses into a new logical block; shared prompts are counted, not copied;
preemption moves a request's KV to CPU memory and back).  The page's own
listing lost most of its comparison operators in extraction; the model is
written from the behaviour stated here, and from these readings:

* order: the pool starts with blocks 0 .. N-1 stacked so that N-1 is handed
  out first; a released block goes on top of the stack, so it is the next
  one handed out (last in, first out);
* a request for n blocks with fewer than n free fails (OutOfBlocks) and
  changes nothing; a handed-out block has one owner;
* releasing drops one owner per listed id; a block left with no owner goes
  back on the stack; a release that would take a block below zero owners is a
  double free, found before anything changes;
* a write into a block with one owner happens in place; into a shared block,
  the writer gets a fresh block (the caller copies the data) and the old block
  loses that owner; a block without owners cannot be written;
* adding an owner is only possible for a block that already has one (the
  pages describe shared prompt blocks but show no such method: ``incref`` and
  ``seq_fork``, a child sharing every block of its parent, are that step);
* usage ratio = share of the pool not on the stack;
* a token whose logical block the sequence does not hold (never allocated, or
  released behind a sliding window) has no physical block: IndexError;
* a sliding window of W tokens ([P2] sliding window section) lets a sequence
  release every block that holds none of its last W tokens; those table
  entries read -1;
* preemption: a host pool of whole blocks with its own stack.  Swapping a
  sequence out gives each of its blocks a host block (in logical order) and
  drops the sequence's device ownership (a block other sequences share stays
  theirs); swapping it in gives each host block a fresh device block with one
  owner (sharing is not restored) and returns the host block.  Both are all
  or nothing.  A swapped-out sequence cannot grow, fork, trim, be looked up or
  be exported.
"""
from collections import Counter, deque
from dataclasses import dataclass, field


class OutOfBlocks(RuntimeError):
    """Fewer free blocks than requested."""


class DoubleFree(RuntimeError):
    """A reference was dropped from a block that holds none."""


class _Stack:
    """Ids stacked for hand-out; ``top`` is handed out next."""

    def __init__(self, bottom_to_top):
        self._ids = deque(reversed(list(bottom_to_top)))   # index 0 = top

    def __len__(self):
        return len(self._ids)

    def take(self):
        return self._ids.popleft()

    def give_back(self, block):
        self._ids.appendleft(block)

    def bottom_to_top(self):
        return list(reversed(self._ids))


@dataclass
class _Sequence:
    table: list = field(default_factory=list)   # logical block -> id (-1 released)
    length: int = 0                             # tokens held
    on_host: bool = False                       # swapped out: ``table`` holds host ids


class AllocatorModel:
    def __init__(self, num_blocks, block_size):
        if num_blocks <= 0 or block_size <= 0:
            raise ValueError("num_blocks and block_size must be positive")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self._stack = _Stack(range(num_blocks))
        self._owners = Counter()              # block -> owners (absent = free)
        self._sequences = {}
        self._ids_issued = 0
        self._copies = 0
        self._host_stack = _Stack([])

    # ---- read-only views (what the tests compare) ---------------------------
    def free_order(self):
        """Free blocks from the bottom of the stack to its top (handed out next)."""
        return self._stack.bottom_to_top()

    def refs(self, block):
        return self._owners[block]

    def ref_counts(self):
        return [self._owners[b] for b in range(self.num_blocks)]

    def host_free_order(self):
        return self._host_stack.bottom_to_top()

    def table(self, sid):
        return list(self._sequences[sid].table)

    def length(self, sid):
        return self._sequences[sid].length

    def cow_count(self):
        return self._copies

    # ---- blocks -------------------------------------------------------------
    def set_free_order(self, order):
        """Restack the free blocks so that order[-1] is handed out first; only
        while no block has an owner, and ``order`` must be a permutation."""
        order = [int(x) for x in order]
        if +self._owners:
            raise ValueError("set_free_order needs every block free")
        if sorted(order) != list(range(self.num_blocks)):
            raise ValueError("order must be a permutation of range(num_blocks)")
        self._stack = _Stack(order)

    def _in_pool(self, ids):
        bad = [b for b in ids if not 0 <= b < self.num_blocks]
        if bad:
            raise ValueError(f"block id {bad[0]} out of range")

    def allocate(self, n=1):
        if n < 0:
            raise ValueError("negative count")
        if n > len(self._stack):
            raise OutOfBlocks(f"need {n} blocks, {len(self._stack)} free")
        taken = [self._stack.take() for _ in range(n)]
        self._owners.update(taken)
        return taken

    def free(self, ids):
        ids = [int(b) for b in ids]
        self._in_pool(ids)
        tally = Counter(ids)
        over = [b for b, k in tally.items() if k > self._owners[b]]
        if over:
            raise DoubleFree(f"block {over[0]} freed more often than referenced")
        for b in ids:
            self._owners[b] -= 1
            if self._owners[b] == 0:
                del self._owners[b]
                self._stack.give_back(b)

    def incref(self, ids):
        ids = [int(b) for b in ids]
        self._in_pool(ids)
        loose = [b for b in ids if self._owners[b] == 0]
        if loose:
            raise ValueError(f"block {loose[0]} is not allocated")
        self._owners.update(ids)

    def copy_on_write(self, block_id):
        """Returns (id_to_write, copied)."""
        self._in_pool([block_id])
        owners = self._owners[block_id]
        if owners == 0:
            raise ValueError(f"block {block_id} is not allocated")
        if owners == 1:
            return block_id, False
        (fresh,) = self.allocate(1)
        self._owners[block_id] -= 1
        self._copies += 1
        return fresh, True

    def usage_ratio(self):
        return (self.num_blocks - len(self._stack)) / self.num_blocks

    # ---- sequences ----------------------------------------------------------
    def _on_device(self, sid):
        seq = self._sequences[sid]
        if seq.on_host:
            raise ValueError(f"sequence {sid} is swapped out")
        return seq

    def _new_id(self):
        sid = self._ids_issued
        self._ids_issued += 1
        return sid

    def seq_create(self):
        sid = self._new_id()
        self._sequences[sid] = _Sequence()
        return sid

    def seq_fork(self, sid):
        parent = self._on_device(sid)
        self.incref([b for b in parent.table if b >= 0])
        child = self._new_id()
        self._sequences[child] = _Sequence(table=list(parent.table), length=parent.length)
        return child

    def seq_append_tokens(self, sid, n):
        """Append ``n`` tokens; returns (slots, cow_pairs).

        A token that opens a logical block takes a fresh block; the first token
        written into a partly filled last block that other sequences share
        makes the sequence's own copy of it (the (src, dst) pair is returned
        for the caller to copy the data).  All or nothing: when the stack
        cannot cover every block the call needs, nothing changes.
        """
        seq = self._on_device(sid)
        if n < 0:
            raise ValueError("negative token count")
        bs = self.block_size
        opens = -(-(seq.length + n) // bs) - (-(-seq.length // bs))
        copies = 1 if n and seq.length % bs and self._owners[seq.table[-1]] > 1 else 0
        if opens + copies > len(self._stack):
            raise OutOfBlocks(f"need {opens + copies} blocks, {len(self._stack)} free")
        slots, pairs = [], []
        for pos in range(seq.length, seq.length + n):
            if pos % bs == 0:
                seq.table.extend(self.allocate(1))
            else:
                target, copied = self.copy_on_write(seq.table[-1])
                if copied:
                    pairs.append((seq.table[-1], target))
                    seq.table[-1] = target
            slots.append(seq.table[-1] * bs + pos % bs)
        seq.length += n
        return slots, pairs

    def seq_trim_window(self, sid, window):
        """Release every block holding none of the last ``window`` tokens ([P2]
        sliding window: older tokens are dropped, so a sequence holds at most
        ceil(window / block_size) + 1 blocks); their entries become -1.
        Returns the released ids in logical order."""
        if window <= 0:
            raise ValueError("window must be positive")
        seq = self._on_device(sid)
        keep_from = max(0, seq.length - window) // self.block_size
        gone = [b for b in seq.table[:keep_from] if b >= 0]
        seq.table[:keep_from] = [-1] * keep_from
        self.free(gone)
        return gone

    def set_host_pool(self, num_host_blocks):
        if num_host_blocks < 0:
            raise ValueError("negative host pool")
        if any(s.on_host for s in self._sequences.values()):
            raise ValueError("a sequence is swapped out")
        self._host_stack = _Stack(range(num_host_blocks))

    def seq_swap_out(self, sid):
        """Returns the (device block, host block) pairs to copy, in logical order."""
        seq = self._on_device(sid)
        moving = [j for j, b in enumerate(seq.table) if b >= 0]
        if len(moving) > len(self._host_stack):
            raise OutOfBlocks(f"need {len(moving)} host blocks, {len(self._host_stack)} free")
        out = []
        for j in moving:
            dev, host = seq.table[j], self._host_stack.take()
            self.free([dev])
            seq.table[j] = host
            out.append((dev, host))
        seq.on_host = True
        return out

    def seq_swap_in(self, sid):
        """Returns the (host block, device block) pairs to copy, in logical order."""
        seq = self._sequences[sid]
        if not seq.on_host:
            raise ValueError(f"sequence {sid} is not swapped out")
        moving = [j for j, h in enumerate(seq.table) if h >= 0]
        if len(moving) > len(self._stack):
            raise OutOfBlocks(f"need {len(moving)} blocks, {len(self._stack)} free")
        pairs = []
        for j in moving:
            host = seq.table[j]
            (dev,) = self.allocate(1)
            self._host_stack.give_back(host)
            seq.table[j] = dev
            pairs.append((host, dev))
        seq.on_host = False
        return pairs

    def seq_is_swapped(self, sid):
        return self._sequences[sid].on_host

    def seq_free(self, sid):
        seq = self._sequences.pop(sid)
        held = [b for b in seq.table if b >= 0]
        if seq.on_host:
            for h in held:
                self._host_stack.give_back(h)
        else:
            self.free(held)

    def seq_physical_block(self, sid, token):
        seq = self._on_device(sid)
        j = token // self.block_size
        if token < 0 or j >= len(seq.table) or seq.table[j] < 0:
            raise IndexError(f"token {token}: block {j} not allocated")
        return seq.table[j]

    def export_block_tables(self, sids, max_blocks, pad=-1):
        tables, lens = [], []
        for sid in sids:
            seq = self._on_device(sid)
            if len(seq.table) > max_blocks:
                raise ValueError("max_blocks smaller than a sequence's table")
            row = [b if b >= 0 else pad for b in seq.table]
            tables.append(row + [pad] * (max_blocks - len(row)))
            lens.append(seq.length)
        return tables, lens
