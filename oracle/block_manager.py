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
