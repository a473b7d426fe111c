"""Automatic prefix caching by chained block hashes.

Each full block of a sequence is named by a digest of three things: its
parent block's digest, the token ids the block holds, and extra metadata.
Because every digest folds in its parent's, one digest stands for the whole
token prefix up to the end of its block, so two requests with the same
leading tokens produce the same chain and the second one finds the first
one's physical blocks instead of recomputing them ("PagedAttention and
RadixAttention: Let's Talk About KV Cache", section "Two Layers, Not Two
Rivals"; "PagedAttention 与 RadixAttention", section "PagedAttention", on
hashing a block's tokens so that equal blocks are shared through the block
table).  A tenant salt enters the first block's digest, so identical prompts
of different tenants never share blocks (same article, section "Beyond the
Two Techniques", on cache salting).

Rules this module fixes where the pages leave a choice:

* Digest: SHA-256 over the length-prefixed parent digest (empty for the first
  block), the block's token ids as little-endian int64, and the extra bytes
  (the tenant salt for the first block, empty for the others).
* Only full blocks are named.  A lookup uses at most ``(len(tokens) - 1) // B``
  blocks, so at least one prompt token is always left to compute (the one
  whose logits start generation).
* A block is indexed (sealed) by :meth:`PrefixCachingAllocator.commit` once
  the caller has written its keys and values.  If the digest already names
  another block (two requests prefilled the same prefix at once), the first
  one stays indexed and the later block is not.  Sealed blocks are never
  written again: a sequence that would write into one copies it first.
* A sealed block whose last reference goes away stays indexed but idle.
  Allocation takes plain free blocks first, then evicts idle blocks least
  recently released first; one sequence releases its sealed blocks from the
  deepest back, so a chain loses its tail before its head.  A hit on an idle
  block takes it back.
"""

import hashlib
from collections import OrderedDict

import numpy as np

from .allocator import BlockAllocator


def _digest(parent: bytes, tok: bytes, extra: bytes) -> bytes:
    return hashlib.sha256(b"".join((len(parent).to_bytes(8, "little"), parent,
                                    len(tok).to_bytes(8, "little"), tok,
                                    len(extra).to_bytes(8, "little"), extra))).digest()


def block_hash(parent: bytes, tokens, extra: bytes = b"") -> bytes:
    """Digest naming one full block: SHA-256 of the length-prefixed parent
    digest, token ids (int64 little-endian) and extra bytes."""
    return _digest(parent, np.ascontiguousarray(tokens, dtype="<i8").tobytes(), extra)


class PrefixCachingAllocator(BlockAllocator):
    """:class:`BlockAllocator` whose full blocks can be found again by the
    token prefix they hold.

    Typical use for one request::

        sid, cached = pc.start(prompt, salt)      # reuse what is cached
        slots, pairs = pc.append_tokens(sid, len(prompt) - cached)
        ...write K/V of prompt[cached:] into ``slots``...
        pc.commit(sid, prompt)                    # index the full blocks
        ...decode steps (append_step), commit again to index new blocks...
        pc.free(sid)                              # sealed blocks stay cached
    """

    def __init__(self, *args, **kw):
        super().__init__(*args, **kw)
        self._block_of = {}            # digest -> sealed block
        self._digest = {}              # sealed block -> digest
        self._idle_lru = OrderedDict() # unreferenced sealed blocks, oldest first
        self._chain = {}               # sequence -> digests of its leading full blocks
        self._salt = {}                # sequence -> tenant salt
        self.hits = 0                  # blocks found by start()
        self.lookups = 0               # blocks looked up by start()

    # ------------------------------------------------------ allocator hooks
    def _available(self) -> int:
        return len(self._free) + len(self._idle_lru)

    def _take(self, n: int) -> np.ndarray:
        k = min(n, len(self._free))
        out = np.empty(n, dtype=np.int32)
        out[:k] = self._free.popleft_n(k)
        for i in range(k, n):                   # evict the least recently released
            b, _ = self._idle_lru.popitem(last=False)
            del self._block_of[self._digest.pop(b)]
            self.sealed[b] = False
            out[i] = b
        self.ref[out] = 1
        return out

    def _release(self, blocks) -> None:
        blocks = [int(b) for b in blocks]
        self._free.extend([b for b in blocks if not self.sealed[b]])
        for b in reversed(blocks):
            if self.sealed[b]:
                self._idle_lru[b] = None

    def _idle(self):
        return self._idle_lru.keys()

    def _snapshot(self):
        return (super()._snapshot(), dict(self._block_of), dict(self._digest),
                OrderedDict(self._idle_lru))

    def _restore(self, saved):
        base, self._block_of, self._digest, self._idle_lru = saved
        super()._restore(base)

    # ----------------------------------------------------------- sequences
    def _digests(self, tokens, salt: bytes, count: int, parent: bytes = b"", start: int = 0):
        step = self.block_size * 8
        raw = np.ascontiguousarray(tokens[start * self.block_size:count * self.block_size],
                                   dtype="<i8").tobytes()
        out = []
        for i, k in enumerate(range(start, count)):
            parent = _digest(parent, raw[i * step:(i + 1) * step], salt if k == 0 else b"")
            out.append(parent)
        return out

    def start(self, tokens, salt: bytes = b""):
        """New sequence for a prompt: its leading full blocks that are cached
        (same tokens, same salt) are mapped into its table by reference.

        Returns ``(sid, cached_tokens)``; the caller appends and computes only
        ``tokens[cached_tokens:]``.
        """
        tokens = np.asarray(tokens, dtype=np.int64)
        B = self.block_size
        want = min(max(0, (len(tokens) - 1) // B), self.max_blocks_per_seq)
        chain, hits = [], []
        step = B * 8
        raw = np.ascontiguousarray(tokens[:want * B], dtype="<i8").tobytes()
        parent = b""
        for k in range(want):
            parent = _digest(parent, raw[k * step:(k + 1) * step], salt if k == 0 else b"")
            b = self._block_of.get(parent)
            if b is None:
                break
            chain.append(parent)
            hits.append(b)
        self.lookups += want
        self.hits += len(hits)
        sid = self.new_seq()
        for b in hits:
            self._idle_lru.pop(b, None)
        hits = np.asarray(hits, dtype=np.int64)
        self.ref[hits] += 1
        self.tables[sid, :len(hits)] = hits
        self.nblk[sid] = len(hits)
        self.lens[sid] = len(hits) * B
        self._chain[sid] = chain
        self._salt[sid] = bytes(salt)
        return sid, len(hits) * B

    def commit(self, sid: int, tokens) -> int:
        """Index the sequence's full blocks.  ``tokens`` are the sequence's
        token ids from position 0 (at least ``context_len(sid)`` of them, the
        same ones on every call).  A block is indexed unless it already is or
        its digest already names another block.  Returns how many blocks were
        newly indexed."""
        self._check(sid)
        tokens = np.asarray(tokens, dtype=np.int64)
        L = int(self.lens[sid])
        if len(tokens) < L:
            raise ValueError("commit needs the token ids of every cached position")
        full = L // self.block_size
        chain = self._chain.setdefault(sid, [])
        if len(chain) < full:
            salt = self._salt.get(sid, b"")
            chain += self._digests(tokens, salt, full, chain[-1] if chain else b"", len(chain))
        added = 0
        row = self.tables[sid, :full]
        for k in np.flatnonzero(~self.sealed[row]).tolist():   # sealed blocks stay as they are
            b = int(row[k])
            h = chain[k]
            if not self.sealed[b] and h not in self._block_of:
                self._block_of[h] = b
                self._digest[b] = h
                self.sealed[b] = True
                added += 1
        return added

    def new_seq(self) -> int:
        sid = super().new_seq()
        self._chain[sid] = []
        self._salt[sid] = b""
        return sid

    def fork(self, sid: int, n: int = 1):
        kids = super().fork(sid, n)
        for c in kids:
            self._chain[c] = list(self._chain[sid])
            self._salt[c] = self._salt[sid]
        return kids

    def truncate(self, sid: int, new_len: int) -> None:
        super().truncate(sid, new_len)
        del self._chain[sid][new_len // self.block_size:]

    def free(self, sid: int) -> None:
        super().free(sid)
        self._chain.pop(sid, None)
        self._salt.pop(sid, None)

    # -------------------------------------------------------------- queries
    def cached_blocks(self) -> int:
        """Blocks currently indexed (in use or idle)."""
        return len(self._digest)

    def idle_blocks(self) -> int:
        return len(self._idle_lru)

    def is_cached(self, block: int) -> bool:
        return bool(self.sealed[block])

    def validate(self) -> None:
        super().validate()
        assert len(self._block_of) == len(self._digest) == int(self.sealed.sum()), "index size"
        for h, b in self._block_of.items():
            assert self._digest[b] == h and self.sealed[b], "index out of step"
        for b in self._idle_lru:
            assert self.sealed[b] and self.ref[b] == 0, "idle block not sealed or in use"
        assert int(((self.ref == 0) & self.sealed).sum()) == len(self._idle_lru), "idle count"
