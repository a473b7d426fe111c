"""A plain, token-at-a-time model of the reference-counted block manager
(oracle for the host-side allocator).

TEST INFRASTRUCTURE ONLY -- see the package docstring.

Behaviour, as the pages describe it:

* Blocks of B tokens come from one pool of interchangeable physical blocks;
  a sequence takes a block only when it needs one, so it never holds more
  than one partly filled block (Triptych page "Paged Attention for Efficient
  Memory Management", technical summary and "The story"; "PagedAttention 与
  RadixAttention", section "PagedAttention": the last block's filled state
  decides whether a decode step must allocate).
* Sequences that share a prefix (a common prompt, parallel samples, beams)
  point at the same physical blocks; each block counts its references and
  returns to the pool when the count reaches zero (Triptych page, technical
  summary and "Look closer / Sharing is a pointer change").
* A write into a block that is still shared first copies that block
  (copy-on-write), so every other reference keeps its contents (same places).

Where the pages leave a choice open, this model fixes it (and the library's
allocator follows the same rules):

* The free list is first-in first-out: ``allocate`` takes the oldest free
  block; a block whose count drops to zero goes to the back.  The initial
  order is given by the caller (a seeded permutation in the workloads).
* ``append`` handles one token at a time, in the order given.  When a
  sequence writes into a shared partly filled block it receives a fresh
  block, records the pair (shared block, fresh block) for the device copy and
  drops its reference to the shared block; the last remaining owner writes
  in place.
* Freeing a sequence releases its blocks in logical order.
"""

from collections import deque


class OutOfBlocks(RuntimeError):
    """The pool has no free block left."""


class RefBlockManager:
    def __init__(self, num_blocks: int, block_size: int, free_order=None):
        self.block_size = block_size
        order = range(num_blocks) if free_order is None else free_order
        self.free = deque(int(b) for b in order)
        self.ref = {}            # physical block -> reference count (> 0)
        self.tables = {}         # seq id -> list of physical blocks
        self.lens = {}           # seq id -> tokens written
        self._next = 0

    # -- blocks ---------------------------------------------------------
    def _take(self) -> int:
        if not self.free:
            raise OutOfBlocks("no free block")
        b = self.free.popleft()
        self.ref[b] = 1
        return b

    def _drop(self, b: int) -> None:
        self.ref[b] -= 1
        if self.ref[b] == 0:
            del self.ref[b]
            self.free.append(b)

    # -- sequences ------------------------------------------------------
    def new_seq(self) -> int:
        sid = self._next
        self._next += 1
        self.tables[sid] = []
        self.lens[sid] = 0
        return sid

    def append(self, sid: int, n: int):
        """Append n tokens; returns (slots, copy_pairs)."""
        B = self.block_size
        table = self.tables[sid]
        slots, pairs = [], []
        for _ in range(n):
            pos = self.lens[sid]
            if pos % B == 0:                      # last block full (or none)
                table.append(self._take())
            elif self.ref[table[-1]] > 1:         # partly filled and shared
                src = table[-1]
                dst = self._take()
                pairs.append((src, dst))
                self._drop(src)
                table[-1] = dst
            slots.append(table[pos // B] * B + pos % B)
            self.lens[sid] = pos + 1
        return slots, pairs

    def fork(self, sid: int) -> int:
        """New sequence sharing every block of ``sid`` by reference."""
        child = self.new_seq()
        self.tables[child] = list(self.tables[sid])
        self.lens[child] = self.lens[sid]
        for b in self.tables[child]:
            self.ref[b] += 1
        return child

    def free_seq(self, sid: int) -> None:
        for b in self.tables.pop(sid):
            self._drop(b)
        del self.lens[sid]

    def table(self, sid: int):
        return list(self.tables[sid])


class SwapBlockManager(RefBlockManager):
    """The block manager plus a host tier: a group of sequences can be moved
    out of the device pool into host blocks and back ("PagedAttention and
    RadixAttention: Let's Talk About KV Cache", "Beyond the Two Techniques":
    hot blocks in GPU memory, recently used ones in host RAM).

    Rules fixed here (the library follows them):

    * A move takes a set of sequences; every block they reference, in the
      order first met (sequences in the order given, then logical order), gets
      one block of the other tier, taken first-in first-out from that tier's
      free list, with the same reference count.  Their tables are rewritten;
      the old blocks return to their free list in that same order.
    * A block also referenced by a sequence outside the set cannot move
      (ValueError); too few free blocks in the other tier raise OutOfBlocks.
      Either leaves the state unchanged.
    * A sequence on the host tier takes no appends or forks until it is moved
      back.
    """

    def __init__(self, num_blocks: int, block_size: int, free_order=None, num_host_blocks=0):
        super().__init__(num_blocks, block_size, free_order)
        self.host_free = deque(range(num_host_blocks))
        self.host_ref = {}
        self.on_host = set()

    def _move(self, sids, to_host: bool):
        src_ref = self.ref if to_host else self.host_ref
        dst_ref = self.host_ref if to_host else self.ref
        src_free = self.free if to_host else self.host_free
        dst_free = self.host_free if to_host else self.free
        blocks = []
        for s in sids:
            if (s in self.on_host) == to_host:
                raise ValueError("sequence already on that tier")
            for b in self.tables[s]:
                if b not in blocks:
                    blocks.append(b)
        for b in blocks:
            inside = sum(self.tables[s].count(b) for s in sids)
            if inside != src_ref[b]:
                raise ValueError("a block is shared with a sequence outside the set")
        if len(blocks) > len(dst_free):
            raise OutOfBlocks("the other tier has too few free blocks")
        new = {}
        for b in blocks:
            new[b] = dst_free.popleft()
            dst_ref[new[b]] = src_ref[b]
        for s in sids:
            self.tables[s] = [new[b] for b in self.tables[s]]
            if to_host:
                self.on_host.add(s)
            else:
                self.on_host.discard(s)
        for b in blocks:
            del src_ref[b]
            src_free.append(b)
        return [(b, new[b]) for b in blocks]

    def swap_out(self, sids):
        """Move the sequences to the host tier; returns (device, host) pairs."""
        return self._move(list(sids), True)

    def swap_in(self, sids):
        """Move them back; returns (host, device) pairs."""
        return self._move(list(sids), False)

    def append(self, sid, n):
        if sid in self.on_host:
            raise ValueError("sequence is on the host tier")
        return super().append(sid, n)

    def fork(self, sid):
        if sid in self.on_host:
            raise ValueError("sequence is on the host tier")
        return super().fork(sid)

    def free_seq(self, sid):
        if sid not in self.on_host:
            return super().free_seq(sid)
        for b in self.tables.pop(sid):
            self.host_ref[b] -= 1
            if self.host_ref[b] == 0:
                del self.host_ref[b]
                self.host_free.append(b)
        del self.lens[sid]
        self.on_host.discard(sid)
