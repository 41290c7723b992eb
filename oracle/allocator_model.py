"""Reference model of the ref-counted free-list block allocator.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  The C++ allocator in the
library is checked against this model op by op on random op sequences.

Semantics follow [P3] section 二 (BlockManager, BlockTable, copy-on-write) and
[P1] "PagedAttention分页内存管理原理" / "vLLM调度器与PagedAttention协同工作"
(all blocks are the same size, so a plain free list suffices; blocks are
allocated on demand when a token crosses a block boundary; shared prefixes are
tracked with reference counts).  The page's listing lost most of its operators
in extraction; the readings taken here:

* the free list starts as ``[0, 1, ..., N-1]`` and ``allocate`` pops from its
  END, so the first id handed out is N-1; freed blocks are appended and are
  therefore reused first;
* ``allocate(n)`` with fewer than ``n`` free blocks raises and changes nothing
  (all or nothing); each allocated block gets reference count 1;
* ``free(ids)`` drops one reference per listed id; a block whose count
  reaches 0 goes back on the free list; dropping a reference that does not
  exist (count would go below 0) is a double free, detected BEFORE any count
  changes, so a failing call leaves the state untouched;
* ``copy_on_write(id)``: a block with exactly one owner is written in place
  (same id back); a shared block gives the writer a fresh block (the caller
  copies the data) and loses one reference; a block with no owner is an error;
* sharing: the page describes shared prompt blocks but shows no method that
  adds a reference; ``incref`` and ``fork`` (a child sequence that shares all
  of its parent's blocks) are that missing step;
* ``usage_ratio = 1 - free / num_blocks``;
* looking up a token whose logical block has not been allocated (or has
  been released behind a sliding window) raises IndexError;
* ``seq_trim_window`` releases the blocks entirely before the last W tokens
  ([P2] sliding window section); their table entries read -1;
* preemption ([P1] scheduler section, item 3: under memory pressure a
  low-priority request's KV goes to CPU memory, its device blocks are freed,
  and it comes back when blocks are free again; [P1] deployment section,
  swap_space): a host pool of ``num_host_blocks`` blocks with its own LIFO free
  list.  ``seq_swap_out`` gives each of the sequence's blocks a host block, in
  logical order, and drops the sequence's device reference (a block other
  sequences share stays theirs); ``seq_swap_in`` gives each host block a fresh
  device block (count 1: sharing is not restored) and returns the host block.
  Both are all or nothing.  A swapped-out sequence cannot be appended to,
  forked, trimmed, looked up or exported.
"""


class OutOfBlocks(RuntimeError):
    """Fewer free blocks than requested."""


class DoubleFree(RuntimeError):
    """A reference was dropped from a block that holds none."""


class AllocatorModel:
    def __init__(self, num_blocks, block_size):
        if num_blocks <= 0 or block_size <= 0:
            raise ValueError("num_blocks and block_size must be positive")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.free_blocks = list(range(num_blocks))
        self.ref_count = [0] * num_blocks
        self.seqs = {}          # seq id -> {"blocks": [...], "tokens": int}
        self.next_seq = 0
        self.cow_copies = 0
        self.num_host_blocks = 0
        self.host_free = []

    # ---- block level -------------------------------------------------------
    def set_free_order(self, order):
        """Replace the free list by ``order`` (pop from its end); only legal
        while every block is free, and ``order`` must be a permutation."""
        order = [int(x) for x in order]
        if any(self.ref_count):
            raise ValueError("set_free_order needs every block free")
        if sorted(order) != list(range(self.num_blocks)):
            raise ValueError("order must be a permutation of range(num_blocks)")
        self.free_blocks = order

    def allocate(self, n=1):
        if n < 0:
            raise ValueError("negative count")
        if len(self.free_blocks) < n:
            raise OutOfBlocks(f"need {n} blocks, {len(self.free_blocks)} free")
        out = []
        for _ in range(n):
            b = self.free_blocks.pop()
            self.ref_count[b] = 1
            out.append(b)
        return out

    def _check_ids(self, ids):
        for b in ids:
            if not 0 <= b < self.num_blocks:
                raise ValueError(f"block id {b} out of range")

    def free(self, ids):
        ids = [int(b) for b in ids]
        self._check_ids(ids)
        drop = {}
        for b in ids:
            drop[b] = drop.get(b, 0) + 1
        for b, c in drop.items():
            if self.ref_count[b] - c < 0:
                raise DoubleFree(f"block {b} freed more often than referenced")
        for b in ids:
            self.ref_count[b] -= 1
            if self.ref_count[b] == 0:
                self.free_blocks.append(b)

    def incref(self, ids):
        ids = [int(b) for b in ids]
        self._check_ids(ids)
        for b in ids:
            if self.ref_count[b] == 0:
                raise ValueError(f"block {b} is not allocated")
        for b in ids:
            self.ref_count[b] += 1

    def copy_on_write(self, block_id):
        """Returns (id_to_write, copied)."""
        self._check_ids([block_id])
        rc = self.ref_count[block_id]
        if rc == 0:
            raise ValueError(f"block {block_id} is not allocated")
        if rc == 1:
            return block_id, False
        new_id = self.allocate(1)[0]
        self.ref_count[block_id] -= 1
        self.cow_copies += 1
        return new_id, True

    def usage_ratio(self):
        return 1.0 - len(self.free_blocks) / self.num_blocks

    # ---- sequence level ----------------------------------------------------
    def seq_create(self):
        sid = self.next_seq
        self.next_seq += 1
        self.seqs[sid] = {"blocks": [], "tokens": 0, "swapped": False}
        return sid

    def _resident(self, sid):
        seq = self.seqs[sid]
        if seq["swapped"]:
            raise ValueError(f"sequence {sid} is swapped out")
        return seq

    def seq_fork(self, sid):
        parent = self._resident(sid)
        self.incref([b for b in parent["blocks"] if b >= 0])
        cid = self.next_seq
        self.next_seq += 1
        self.seqs[cid] = {"blocks": list(parent["blocks"]),
                          "tokens": parent["tokens"], "swapped": False}
        return cid

    def seq_append_tokens(self, sid, n):
        """Append ``n`` tokens; returns (slots, cow_pairs).

        A token that starts a new logical block takes a freshly allocated
        block; a token that lands in a partly filled last block that other
        sequences share first gets its own copy of that block (copy-on-write;
        the (src, dst) pair is returned for the caller to copy the data).
        All or nothing: if the free list cannot cover every block the call
        needs, nothing changes.
        """
        seq = self._resident(sid)
        bs = self.block_size
        tokens = seq["tokens"]
        need = 0
        if n > 0 and tokens % bs != 0 and self.ref_count[seq["blocks"][-1]] > 1:
            need += 1
        need += (tokens + n + bs - 1) // bs - (tokens + bs - 1) // bs
        if need > len(self.free_blocks):
            raise OutOfBlocks(f"need {need} blocks, {len(self.free_blocks)} free")
        slots, cow = [], []
        for _ in range(n):
            off = tokens % bs
            if off == 0:
                seq["blocks"].append(self.allocate(1)[0])
            else:
                last = seq["blocks"][-1]
                new, copied = self.copy_on_write(last)
                if copied:
                    seq["blocks"][-1] = new
                    cow.append((last, new))
            slots.append(seq["blocks"][-1] * bs + off)
            tokens += 1
        seq["tokens"] = tokens
        return slots, cow

    def seq_trim_window(self, sid, window):
        """Release the blocks that hold no token of the last ``window`` tokens
        ([P2] sliding window: tokens older than the window are dropped, so the
        cache of a sequence stays within ceil(window / block_size) + 1 blocks).
        Their table entries become -1; returns the released ids in order."""
        if window <= 0:
            raise ValueError("window must be positive")
        seq = self._resident(sid)
        first_kept = max(0, seq["tokens"] - window) // self.block_size
        released = []
        for j in range(first_kept):
            b = seq["blocks"][j]
            if b >= 0:
                released.append(b)
                seq["blocks"][j] = -1
        self.free(released)
        return released

    def set_host_pool(self, num_host_blocks):
        if num_host_blocks < 0:
            raise ValueError("negative host pool")
        if any(s["swapped"] for s in self.seqs.values()):
            raise ValueError("a sequence is swapped out")
        self.num_host_blocks = num_host_blocks
        self.host_free = list(range(num_host_blocks))

    def seq_swap_out(self, sid):
        """Returns the (device block, host block) pairs to copy, in logical order."""
        seq = self._resident(sid)
        held = [b for b in seq["blocks"] if b >= 0]
        if len(held) > len(self.host_free):
            raise OutOfBlocks(f"need {len(held)} host blocks, {len(self.host_free)} free")
        pairs = []
        for j, b in enumerate(seq["blocks"]):
            if b < 0:
                continue
            h = self.host_free.pop()
            pairs.append((b, h))
            self.free([b])
            seq["blocks"][j] = h
        seq["swapped"] = True
        return pairs

    def seq_swap_in(self, sid):
        """Returns the (host block, device block) pairs to copy, in logical order."""
        seq = self.seqs[sid]
        if not seq["swapped"]:
            raise ValueError(f"sequence {sid} is not swapped out")
        held = [h for h in seq["blocks"] if h >= 0]
        if len(held) > len(self.free_blocks):
            raise OutOfBlocks(f"need {len(held)} blocks, {len(self.free_blocks)} free")
        pairs = []
        for j, h in enumerate(seq["blocks"]):
            if h < 0:
                continue
            d = self.allocate(1)[0]
            pairs.append((h, d))
            self.host_free.append(h)
            seq["blocks"][j] = d
        seq["swapped"] = False
        return pairs

    def seq_is_swapped(self, sid):
        return self.seqs[sid]["swapped"]

    def seq_free(self, sid):
        seq = self.seqs.pop(sid)
        if seq["swapped"]:
            self.host_free.extend(h for h in seq["blocks"] if h >= 0)
        else:
            self.free([b for b in seq["blocks"] if b >= 0])

    def seq_physical_block(self, sid, token):
        seq = self._resident(sid)
        idx = token // self.block_size
        if token < 0 or idx >= len(seq["blocks"]) or seq["blocks"][idx] < 0:
            raise IndexError(f"token {token}: block {idx} not allocated")
        return seq["blocks"][idx]

    def export_block_tables(self, sids, max_blocks, pad=-1):
        tables, lens = [], []
        for sid in sids:
            seq = self._resident(sid)
            if len(seq["blocks"]) > max_blocks:
                raise ValueError("max_blocks smaller than a sequence's table")
            row = [b if b >= 0 else pad for b in seq["blocks"]]
            tables.append(row + [pad] * (max_blocks - len(row)))
            lens.append(seq["tokens"])
        return tables, lens
