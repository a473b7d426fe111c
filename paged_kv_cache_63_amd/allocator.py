"""Host-side block manager for the paged KV cache.

The pages put this layer on the host: a per-sequence block table, a pool of
interchangeable physical blocks, allocation one block at a time when the last
block is full, sharing by reference count, and copy-on-write when a shared
block is about to change ("Paged Attention for Efficient Memory Management",
The Daily Triptych, technical summary and "Look closer"; "PagedAttention 与
RadixAttention", section "PagedAttention"; "PagedAttention and
RadixAttention: Let's Talk About KV Cache", section "PagedAttention: Memory
Like an Operating System").

State lives in flat numpy arrays so a decode step over a whole batch is a few
vector operations:

* ``tables``  int32 ``[max_seqs][max_blocks_per_seq]``; row = sequence id;
  entries past the sequence's block count are ``-1``.  A slice of rows is
  exactly the ``block_tables`` argument the device calls take.
* ``lens``    int32 ``[max_seqs]`` tokens written per sequence.
* ``ref``     int32 ``[num_blocks]`` references per physical block.

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
        self._free = deque(int(b) for b in order)
        self._rows = deque(range(self.max_seqs))
        # host tier: blocks of sequences moved out of the device pool
        self.num_host_blocks = int(num_host_blocks)
        self.host_ref = np.zeros(self.num_host_blocks, dtype=np.int32)
        self._host_free = deque(range(self.num_host_blocks))
        self.on_host = np.zeros(self.max_seqs, dtype=bool)

    # ---------------------------------------------------------------- blocks
    def _take(self, n: int) -> np.ndarray:
        """Hand out ``n`` blocks (the caller has checked ``_available``)."""
        out = np.fromiter((self._free.popleft() for _ in range(n)), dtype=np.int32, count=n)
        self.ref[out] = 1
        return out

    def _available(self) -> int:
        """Blocks a request may still take."""
        return len(self._free)

    def _release(self, blocks) -> None:
        """Blocks whose count just reached zero, in logical order."""
        self._free.extend(int(b) for b in blocks)

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
        ``s`` in turn, done with whole-batch array operations.

        Returns ``(slots int32[len(sids)], pairs int32[k][2])``.
        """
        sids = np.asarray(sids, dtype=np.int64)
        if len(np.unique(sids)) != len(sids):
            raise ValueError("a sequence may appear once per step")
        if not self.live[sids].all():
            raise KeyError("append_step on a sequence that is not live")
        if self.on_host[sids].any():
            raise ValueError("append_step on a sequence on the host tier")
        B = self.block_size
        pos = self.lens[sids].astype(np.int64)
        nb = self.nblk[sids].astype(np.int64)
        need_new = pos % B == 0
        last = np.where(need_new, 0, self.tables[sids, np.maximum(nb - 1, 0)]).astype(np.int64)
        if self.sealed[last[~need_new]].any():
            return self._append_step_in_turn(sids)
        shared = (~need_new) & (self.ref[last] > 1)
        cow = np.zeros(len(sids), dtype=bool)
        ref_after = {}
        for i in np.flatnonzero(shared):          # rare: seqs on a shared partial block
            b = int(last[i])
            c = ref_after.get(b, int(self.ref[b]))
            if c > 1:
                cow[i] = True
                ref_after[b] = c - 1
        takers = need_new | cow
        k = int(takers.sum())
        if k > self._available():
            raise OutOfBlocks(f"need {k} blocks, {self._available()} free")
        if (nb[need_new] + 1 > self.max_blocks_per_seq).any():
            raise ValueError("sequence would exceed max_blocks_per_seq")
        fresh = self._take(k)
        idx = np.flatnonzero(takers)
        got = np.empty(len(sids), dtype=np.int64)
        got[idx] = fresh
        for b, c in ref_after.items():
            self.ref[b] = c
        nn = np.flatnonzero(need_new)
        self.tables[sids[nn], nb[nn]] = got[nn]
        self.nblk[sids[nn]] += 1
        cw = np.flatnonzero(cow)
        self.tables[sids[cw], nb[cw] - 1] = got[cw]
        pairs = np.stack([last[cw], got[cw]], axis=1).astype(np.int32)
        slots = self.tables[sids, pos // B].astype(np.int64) * B + pos % B
        self.lens[sids] += 1
        return slots.astype(np.int32), pairs

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
                self.sealed.copy(), deque(self._free))

    def _restore(self, saved):
        self.tables, self.lens, self.nblk, self.ref, self.sealed, self._free = saved

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
