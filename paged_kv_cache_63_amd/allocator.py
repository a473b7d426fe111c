"""Host-side block manager for the paged KV cache.

The pages put this layer on the host: a per-sequence block table, a pool of
interchangeable physical blocks, allocation one block at a time when the last
block is full, sharing by reference count, and copy-on-write when a shared
block is about to change ("Paged Attention for Efficient Memory Management",
The Daily Triptych, technical summary and "Look closer"; "PagedAttention 与
RadixAttention", section "PagedAttention"; "PagedAttention and
RadixAttention: Let's Talk About KV Cache", section "PagedAttention: Memory
Like an Operating System").

State lives in flat numpy arrays, which the library's native decode step
(``block_manager_append_step``) updates in place for a whole batch:

* ``tables``  int32 ``[max_seqs][max_blocks_per_seq]``; row = sequence id;
  entries past the sequence's block count are ``-1``.  A slice of rows is
  exactly the ``block_tables`` argument the device calls take.
* ``lens``    int32 ``[max_seqs]`` tokens written per sequence.
* ``ref``     int32 ``[num_blocks]`` references per physical block.
* the free list, a FIFO ring of block ids (int32 ``[num_blocks]``) with its
  head and count in an int64 pair.

Rules where the pages leave a choice (the oracle's block-manager model fixes
the same ones, and the tests compare the two token for token):

* The free list is FIFO: the oldest free block is handed out first; a block
  whose count reaches zero goes to the back.  The initial order is the
  caller's (``free_order``).
* A sequence that writes into a partly filled block still shared with others
  gets a fresh block and a ``(src, dst)`` pair for :func:`copy_blocks`; the
  last owner writes in place.  Within one call the copy destination is taken
  before any new block.
* A sequence holds ``ceil(len / B)`` blocks, so at most ``B - 1`` slots of
  one partly filled block are idle (the waste bound of the pages).
"""

from collections import deque

import numpy as np


class OutOfBlocks(RuntimeError):
    """Raised when an operation needs more free blocks than the pool has.
    The allocator state is left unchanged."""


# Positive returns of block_manager_append_step: nothing was changed.
_STEP_SEALED = 1    # a sequence would write into a sealed block
_STEP_SHORT = 2     # the free list holds fewer blocks than the step needs
_NATIVE = None


def _native_step():
    global _NATIVE
    if _NATIVE is None:
        from . import _lib      # imports torch first, then loads the library
        _NATIVE = _lib.load().block_manager_append_step
    return _NATIVE


def _native_error() -> str:
    from . import _lib
    return _lib.load().paged_kv_last_error().decode()


class _BlockFifo:
    """FIFO of free block ids: a ring (``ring`` int32) whose head index and
    count sit in ``state`` (int64 ``[2]``), where native code can update
    them.  Capacity: every block of the pool once."""

    def __init__(self, capacity: int, items=()):
        self.ring = np.zeros(max(int(capacity), 1), dtype=np.int32)
        self.state = np.zeros(2, dtype=np.int64)
        self.extend(items)

    def __len__(self) -> int:
        return int(self.state[1])

    def _index(self, start: int, n: int) -> np.ndarray:
        return (start + np.arange(n)) % len(self.ring)

    def popleft_n(self, n: int) -> np.ndarray:
        head, count = int(self.state[0]), int(self.state[1])
        if n > count:
            raise IndexError("pop from a short free list")
        out = self.ring[self._index(head, n)]
        self.state[0] = (head + n) % len(self.ring)
        self.state[1] = count - n
        return out

    def popleft(self) -> int:
        return int(self.popleft_n(1)[0])

    def extend(self, blocks) -> None:
        arr = np.asarray(blocks if isinstance(blocks, np.ndarray) else list(blocks),
                         dtype=np.int32).reshape(-1)
        head, count = int(self.state[0]), int(self.state[1])
        if count + len(arr) > len(self.ring):
            raise ValueError("free list over capacity (a block freed twice)")
        self.ring[self._index(head + count, len(arr))] = arr
        self.state[1] = count + len(arr)

    def append(self, block: int) -> None:
        self.extend([block])

    def __iter__(self):
        return iter(self.ring[self._index(int(self.state[0]), len(self))].tolist())

    def copy(self) -> "_BlockFifo":
        c = _BlockFifo.__new__(_BlockFifo)
        c.ring = self.ring.copy()
        c.state = self.state.copy()
        return c


def kv_bytes_per_token(num_layers: int, num_kv_heads: int, head_dim: int,
                       elem_bytes: int) -> int:
    """Bytes of KV cache one token occupies across a model: a key and a value
    vector per KV head per layer.  ("PagedAttention and RadixAttention: Let's
    Talk About KV Cache", opening section, gives about 0.31 MB per token for
    Llama-3.1-70B in BF16.)"""
    return 2 * num_layers * num_kv_heads * head_dim * elem_bytes


class BlockAllocator:
    def __init__(self, num_blocks: int, block_size: int = 16, max_seqs: int = 256,
                 max_blocks_per_seq: int = None, free_order=None, num_host_blocks: int = 0):
        if num_blocks <= 0 or block_size <= 0 or max_seqs <= 0:
            raise ValueError("num_blocks, block_size and max_seqs must be positive")
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        self.max_seqs = int(max_seqs)
        self.max_blocks_per_seq = int(max_blocks_per_seq or num_blocks)
        self.tables = np.full((self.max_seqs, self.max_blocks_per_seq), -1, dtype=np.int32)
        self.lens = np.zeros(self.max_seqs, dtype=np.int32)
        self.nblk = np.zeros(self.max_seqs, dtype=np.int32)
        self.ref = np.zeros(self.num_blocks, dtype=np.int32)
        self.live = np.zeros(self.max_seqs, dtype=bool)
        # A sealed block's contents are frozen (a prefix cache indexes them):
        # a write into it copies it first, even by its only owner.
        self.sealed = np.zeros(self.num_blocks, dtype=bool)
        order = np.arange(self.num_blocks) if free_order is None else np.asarray(free_order)
        if sorted(int(b) for b in order) != list(range(self.num_blocks)):
            raise ValueError("free_order must be a permutation of range(num_blocks)")
        self._free = _BlockFifo(self.num_blocks, order)
        self._rows = deque(range(self.max_seqs))
        # host tier: blocks of sequences moved out of the device pool
        self.num_host_blocks = int(num_host_blocks)
        self.host_ref = np.zeros(self.num_host_blocks, dtype=np.int32)
        self._host_free = deque(range(self.num_host_blocks))
        self.on_host = np.zeros(self.max_seqs, dtype=bool)
        self._native_args = None                    # (state arrays, their pointers) for the native step
        self._npairs = np.zeros(1, dtype=np.int32)

    # ---------------------------------------------------------------- blocks
    def _take(self, n: int) -> np.ndarray:
        """Hand out ``n`` blocks (the caller has checked ``_available``)."""
        out = self._free.popleft_n(n)
        self.ref[out] = 1
        return out

    def _available(self) -> int:
        """Blocks a request may still take."""
        return len(self._free)

    def _release(self, blocks) -> None:
        """Blocks whose count just reached zero, in logical order."""
        self._free.extend(blocks)

    def _idle(self):
        """Unreferenced blocks kept out of the free list (none here)."""
        return ()

    def num_free(self) -> int:
        return self._available()

    def incref(self, blocks) -> None:
        """One more reference on each block (a cache holding it, a new owner).
        Every block must already be referenced."""
        blocks = np.asarray(blocks, dtype=np.int64)
        if len(blocks) and (self.ref[blocks] <= 0).any():
            raise ValueError("incref on an unreferenced block")
        np.add.at(self.ref, blocks, 1)

    def decref(self, blocks) -> int:
        """Drop one reference from each block; blocks that reach zero are
        released in the order given.  Returns how many were released."""
        blocks = np.asarray(blocks, dtype=np.int64)
        if len(blocks) and (self.ref[blocks] <= 0).any():
            raise ValueError("decref on an unreferenced block")
        zero = []
        for b in blocks:
            self.ref[b] -= 1
            if self.ref[b] == 0:
                zero.append(int(b))
        self._release(zero)
        return len(zero)

    def adopt(self, blocks, num_tokens: int) -> int:
        """New sequence whose first blocks are ``blocks`` (already referenced
        elsewhere, e.g. by a prefix cache), holding ``num_tokens`` tokens.
        Each block gains a reference."""
        blocks = np.asarray(blocks, dtype=np.int64)
        if num_tokens != len(blocks) * self.block_size:
            raise ValueError("adopted blocks must be full")
        if len(blocks) > self.max_blocks_per_seq:
            raise ValueError("sequence would exceed max_blocks_per_seq")
        if len(np.unique(blocks)) != len(blocks):
            raise ValueError("a block may appear once per sequence")
        if len(blocks) and (self.ref[blocks] <= 0).any():
            raise ValueError("adopted blocks must be referenced")
        sid = self.new_seq()
        self.ref[blocks] += 1
        self.tables[sid, :len(blocks)] = blocks
        self.nblk[sid] = len(blocks)
        self.lens[sid] = num_tokens
        return sid

    def refcount(self, block: int) -> int:
        return int(self.ref[block])

    # ------------------------------------------------------------- sequences
    def new_seq(self) -> int:
        if not self._rows:
            raise RuntimeError("no free sequence row (max_seqs reached)")
        sid = self._rows.popleft()
        self.live[sid] = True
        self.lens[sid] = 0
        self.nblk[sid] = 0
        return sid

    def _check(self, sid: int) -> None:
        if not (0 <= sid < self.max_seqs) or not self.live[sid]:
            raise KeyError(f"sequence {sid} is not live")

    def _check_dev(self, sid: int) -> None:
        self._check(sid)
        if self.on_host[sid]:
            raise ValueError(f"sequence {sid} is on the host tier (swap it in first)")

    def append_tokens(self, sid: int, n: int):
        """Reserve slots for ``n`` more tokens of one sequence.

        Returns ``(slots int32[n], pairs int32[k][2])``: the pool slot of each
        new token, in order, and the copy-on-write pairs that must be copied
        on the device before the tokens are written.
        """
        self._check_dev(sid)
        B = self.block_size
        pos0 = int(self.lens[sid])
        nb = int(self.nblk[sid])
        pairs = np.zeros((0, 2), dtype=np.int32)
        if n <= 0:
            return np.zeros(0, dtype=np.int32), pairs
        last = int(self.tables[sid, nb - 1]) if nb else -1
        cow = pos0 % B != 0 and (self.ref[last] > 1 or bool(self.sealed[last]))
        new = -(-(pos0 + n) // B) - nb
        # a copied block that nobody else holds becomes available right after
        # its copy is taken, before the new blocks are
        gain = int(cow and self.ref[last] == 1)
        avail = self._available()
        if int(cow) + new > avail + gain or (cow and avail == 0):
            raise OutOfBlocks(f"need {int(cow) + new} blocks, {avail} free")
        if nb + new > self.max_blocks_per_seq:
            raise ValueError("sequence would exceed max_blocks_per_seq")
        if cow:
            dst = int(self._take(1)[0])
            self.ref[last] -= 1
            if self.ref[last] == 0:
                self._release([last])
            self.tables[sid, nb - 1] = dst
            pairs = np.array([[last, dst]], dtype=np.int32)
        if new:
            self.tables[sid, nb:nb + new] = self._take(new)
            self.nblk[sid] = nb + new
        pos = np.arange(pos0, pos0 + n)
        slots = self.tables[sid, pos // B].astype(np.int64) * B + pos % B
        self.lens[sid] = pos0 + n
        return slots.astype(np.int32), pairs

    def append_step(self, sids):
        """One new token for each sequence in ``sids`` (a decode step), handled
        in the order given.  Same result as ``append_tokens(s, 1)`` for each
        ``s`` in turn; the common case runs in the library's native step
        (``block_manager_append_step``) on this object's arrays.

        Returns ``(slots int32[len(sids)], pairs int32[k][2])``.
        """
        sids = np.ascontiguousarray(sids, dtype=np.int64)
        n = len(sids)
        slots = np.empty(n, dtype=np.int32)
        pairs = np.empty((n, 2), dtype=np.int32)
        arrays = (self.tables, self.lens, self.nblk, self.live, self.on_host, self.ref,
                  self.sealed, self._free)
        cached = self._native_args
        if cached is None or any(x is not y for x, y in zip(cached[0], arrays)):
            self._native_args = cached = (arrays, self._native_pointers())
        rc = _native_step()(*cached[1], sids.ctypes.data, n,
                            self._free.ring.ctypes.data, self._free.state.ctypes.data,
                            slots.ctypes.data, pairs.ctypes.data, self._npairs.ctypes.data)
        if rc == 0:
            return slots, pairs[:int(self._npairs[0])]
        if rc in (_STEP_SEALED, _STEP_SHORT):
            # a write into a sealed block (its copy may free it part-way), or
            # more blocks than the free list holds (a subclass may evict)
            return self._append_step_in_turn(sids)
        msg = _native_error()
        raise (KeyError if "not live" in msg else ValueError)(msg)

    def _native_pointers(self):
        return (self.tables.ctypes.data, self.lens.ctypes.data, self.nblk.ctypes.data,
                self.live.ctypes.data, self.on_host.ctypes.data, self.max_seqs,
                self.max_blocks_per_seq, self.ref.ctypes.data, self.sealed.ctypes.data,
                self.num_blocks, self.block_size)

    def _append_step_in_turn(self, sids):
        """``append_tokens(s, 1)`` for each sequence in turn; used when a step
        writes into a sealed block, whose copy may free it part-way through
        the step.  All-or-nothing like the batched path."""
        saved = self._snapshot()
        slots, pairs = [], []
        try:
            for s in sids:
                sl, pr = self.append_tokens(int(s), 1)
                slots.append(sl)
                pairs.append(pr)
        except (OutOfBlocks, ValueError):
            self._restore(saved)
            raise
        return (np.concatenate(slots).astype(np.int32),
                np.concatenate(pairs).astype(np.int32).reshape(-1, 2))

    def _snapshot(self):
        return (self.tables.copy(), self.lens.copy(), self.nblk.copy(), self.ref.copy(),
                self.sealed.copy(), self._free.copy())

    def _restore(self, saved):
        self.tables, self.lens, self.nblk, self.ref, self.sealed, self._free = saved
        self._native_args = None

    def fork(self, sid: int, n: int = 1):
        """``n`` new sequences sharing every block of ``sid`` by reference."""
        self._check_dev(sid)
        if n > len(self._rows):
            raise RuntimeError("no free sequence row (max_seqs reached)")
        nb = int(self.nblk[sid])
        out = []
        for _ in range(n):
            c = self.new_seq()
            self.tables[c] = self.tables[sid]
            self.lens[c] = self.lens[sid]
            self.nblk[c] = nb
            self.ref[self.tables[sid, :nb]] += 1
            out.append(c)
        return out

    def truncate(self, sid: int, new_len: int) -> None:
        """Drop the sequence's tokens from ``new_len`` on (a rejected draft, a
        re-run chunk).  Blocks no longer needed lose this sequence's reference
        and, at zero, return to the back of the free list in logical order."""
        self._check_dev(sid)
        if not 0 <= new_len <= int(self.lens[sid]):
            raise ValueError("new_len must be within the current length")
        nb = int(self.nblk[sid])
        keep = -(-new_len // self.block_size)
        blocks = self.tables[sid, keep:nb].copy()
        self.ref[blocks] -= 1
        self._release(blocks[self.ref[blocks] == 0])
        self.tables[sid, keep:nb] = -1
        self.nblk[sid] = keep
        self.lens[sid] = new_len

    def free(self, sid: int) -> None:
        """Drop the sequence; blocks whose count reaches zero return to the
        back of the free list in logical order."""
        self._check(sid)
        nb = int(self.nblk[sid])
        blocks = self.tables[sid, :nb].copy()
        if self.on_host[sid]:
            for b in blocks:
                self.host_ref[b] -= 1
                if self.host_ref[b] == 0:
                    self._host_free.append(int(b))
            self.on_host[sid] = False
        else:
            self.ref[blocks] -= 1
            self._release(blocks[self.ref[blocks] == 0])
        self.tables[sid] = -1
        self.lens[sid] = 0
        self.nblk[sid] = 0
        self.live[sid] = False
        self._rows.append(sid)

    # ------------------------------------------------------------ host tier
    def _move(self, sids, to_host: bool) -> np.ndarray:
        sids = [int(x) for x in sids]
        for x in sids:
            self._check(x)
            if bool(self.on_host[x]) == to_host:
                raise ValueError(f"sequence {x} is already on that tier")
        if len(set(sids)) != len(sids):
            raise ValueError("a sequence may appear once")
        rows = [self.tables[x, :self.nblk[x]] for x in sids]
        cat = np.concatenate(rows) if rows else np.zeros(0, np.int32)
        blocks, first = np.unique(cat, return_index=True)
        blocks = blocks[np.argsort(first)]               # in the order first met
        inside = np.zeros(len(blocks), dtype=np.int64)
        pos = {int(b): i for i, b in enumerate(blocks)}
        for b in cat:
            inside[pos[int(b)]] += 1
        src_ref = self.ref if to_host else self.host_ref
        if len(blocks) and (src_ref[blocks] != inside).any():
            raise ValueError("a block is shared with a sequence outside the set")
        avail = len(self._host_free) if to_host else self._available()
        if len(blocks) > avail:
            raise OutOfBlocks(f"need {len(blocks)} blocks on the other tier, {avail} free")
        if to_host:
            new = np.fromiter((self._host_free.popleft() for _ in range(len(blocks))),
                              dtype=np.int32, count=len(blocks))
            self.host_ref[new] = src_ref[blocks]
        else:
            new = self._take(len(blocks))
            self.ref[new] = src_ref[blocks]
        remap = dict(zip(blocks.tolist(), new.tolist()))
        for x in sids:
            nb = int(self.nblk[x])
            self.tables[x, :nb] = [remap[int(b)] for b in self.tables[x, :nb]]
            self.on_host[x] = to_host
        src_ref[blocks] = 0
        if to_host:
            self._release(blocks)
        else:
            self._host_free.extend(int(b) for b in blocks)
        return np.stack([blocks, new], axis=1).astype(np.int32) if len(blocks) else \
            np.zeros((0, 2), dtype=np.int32)

    def swap_out(self, sids) -> np.ndarray:
        """Move the sequences' blocks to the host tier.  Every block they
        reference, in the order first met, gets a host block (first-in
        first-out) with the same reference count; their tables now name host
        blocks and the device blocks return to the free list in that order.
        Returns ``(device block, host block)`` pairs for :func:`swap_blocks`.
        A block shared with a sequence outside the set raises ValueError; too
        few host blocks raise OutOfBlocks; either leaves the state unchanged."""
        return self._move(sids, True)

    def swap_in(self, sids) -> np.ndarray:
        """The inverse move; returns ``(host block, device block)`` pairs."""
        return self._move(sids, False)

    def num_free_host(self) -> int:
        return len(self._host_free)

    # --------------------------------------------------------------- queries
    def context_len(self, sid: int) -> int:
        return int(self.lens[sid])

    def block_table(self, sid: int) -> np.ndarray:
        return self.tables[sid, :self.nblk[sid]].copy()

    def waste(self, sid: int) -> int:
        """Idle slots of the sequence (all in its last block)."""
        return int(self.nblk[sid]) * self.block_size - int(self.lens[sid])

    def validate(self, held=None) -> None:
        """Check every invariant; raises AssertionError on the first breach.
        ``held``: references per block held outside sequence tables (a prefix
        tree's), if any."""
        count = np.zeros(self.num_blocks, dtype=np.int64)
        hcount = np.zeros(self.num_host_blocks, dtype=np.int64)
        if held is not None:
            count += held
        for sid in np.flatnonzero(self.live):
            nb = int(self.nblk[sid])
            row = self.tables[sid, :nb]
            assert nb == -(-int(self.lens[sid]) // self.block_size), "block count"
            assert (self.tables[sid, nb:] == -1).all(), "table padding"
            assert len(np.unique(row)) == nb, "block repeated within a sequence"
            assert 0 <= self.waste(sid) < self.block_size or nb == 0, "waste bound"
            if self.on_host[sid]:
                hcount[row] += 1
            else:
                count[row] += 1
        assert (count + self._holders() == self.ref).all(), "refcount != number of references"
        assert (hcount == self.host_ref).all(), "host refcount != number of references"
        hfree = np.array(list(self._host_free), dtype=np.int64)
        assert len(np.unique(hfree)) == len(hfree) and (self.host_ref[hfree] == 0).all(), \
            "host free list"
        assert len(hfree) + int((self.host_ref > 0).sum()) == self.num_host_blocks, \
            "host block leaked"
        free = np.array(list(self._free) + list(self._idle()), dtype=np.int64)
        assert len(np.unique(free)) == len(free), "block twice on the free list"
        assert (self.ref[free] == 0).all(), "referenced block on the free list"
        assert not self.sealed[np.asarray(list(self._free), dtype=np.int64)].any(), \
            "sealed block on the free list"
        assert len(free) + int((self.ref > 0).sum()) == self.num_blocks, "block leaked"

    def _holders(self) -> np.ndarray:
        """References held outside sequence tables, per block (a cache's)."""
        return np.zeros(self.num_blocks, dtype=np.int64)


def shared_prefix_groups(tables, lens, block_size: int = 16, min_blocks: int = 1):
    """Groups of sequences that share the leading physical blocks of their
    tables, for the shared-prefix decode: sharing a prefix is a pointer
    change, every sharer's table naming the same physical blocks ("Paged
    Attention for Efficient Memory Management", The Daily Triptych, "Look
    closer / Sharing is a pointer change").

    ``tables``: ``[S][max_blocks]`` block tables; ``lens``: ``[S]`` context
    lengths.  Sequences whose first table entry is the same physical block
    form a group; its prefix is the longest run of leading entries all of
    them hold, cut so that every member keeps the block with its last token
    to itself.  Groups of one member, or with a prefix shorter than
    ``min_blocks``, are left out.  Returns ``(group_offsets, group_seqs,
    group_prefix_blocks, max_group_size, max_prefix_blocks)``: three int32
    arrays (members of group i are ``group_seqs[group_offsets[i] :
    group_offsets[i + 1]]``) and two ints."""
    tables = np.asarray(tables)
    lens = np.asarray(lens).astype(np.int64)
    nb = (lens + block_size - 1) // block_size
    usable = np.where(lens > 0, (lens - 1) // block_size, 0)   # blocks before the last one
    first = np.where(nb > 0, tables[:, 0], -1)
    order = np.argsort(first, kind="stable")
    offs, seqs, pblk = [0], [], []
    i = 0
    while i < len(order):
        j = i
        while j < len(order) and first[order[j]] == first[order[i]]:
            j += 1
        members = order[i:j]
        if first[order[i]] >= 0 and len(members) > 1:
            limit = int(usable[members].min())
            rows = tables[members, :limit]
            same = (rows == rows[0]).all(axis=0)
            k = limit if same.all() else int(np.argmin(same))
            if k >= min_blocks:
                seqs += members.tolist()
                pblk.append(k)
                offs.append(len(seqs))
        i = j
    sizes = [offs[g + 1] - offs[g] for g in range(len(pblk))]
    return (np.asarray(offs, np.int32), np.asarray(seqs, np.int32), np.asarray(pblk, np.int32),
            max(sizes, default=0), max(pblk, default=0))
