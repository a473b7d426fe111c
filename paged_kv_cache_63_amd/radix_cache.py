"""Radix-tree prefix cache over the paged block allocator.

The tree remembers the key/value blocks of finished (and running) requests
by their token prefix, so a later request that starts with the same tokens
maps those physical blocks into its table instead of recomputing them.  Edges
hold runs of tokens together with the blocks that store them; each unique
prefix is stored once, and requests that share it walk the same branch
("PagedAttention and RadixAttention: Let's Talk About KV Cache", section
"RadixAttention: A Tree That Does Not Forget"; "RadixAttention: Tree-Based KV
Cache Reuse in SGLang Guide", "Architecture", parts 1 and 3).  The tree only
points at blocks the allocator manages; it is a layer on top of paging, not a
second allocator (first article, "Two Layers, Not Two Rivals").

* Lookup walks from the root matching whole blocks of the prompt against edge
  labels until the first mismatch; the blocks on the matched path are reused
  and only the rest of the prompt is computed.  If the match ends inside an
  edge, the edge is split there so the shared part becomes its own node
  (guide, part 3, node splitting).
* A running request holds a reference on every node of its path; only
  unreferenced leaves are evictable, oldest use first, so shared inner nodes
  (system prompts) outlive the branches below them (guide, part 4; the
  five-step figure of "PagedAttention 与 RadixAttention", section
  "RadixAttention", where eviction starts at the leaves).
* Eviction runs when the allocator's free blocks fall below a watermark
  (guide, part 4: a free-space threshold).

Rules fixed here where the pages leave a choice (the oracle's tree model
fixes the same ones):

* Granularity is the block: only whole blocks are cached, matches are
  rounded down to whole blocks and edges split only between blocks.  A
  prompt of n tokens reuses at most ``(n - 1) // B`` blocks, so one prompt
  token is always computed.
* The tree holds one allocator reference on each block of its edges, so a
  cached block outlives the request that wrote it, and a write into it by a
  sequence copies it first (its count is above one).
* Time is a counter advanced once per lookup or insertion; all nodes on the
  touched path take the new value.  Eviction removes the unreferenced leaf
  with the oldest time (ties: the node created first) and drops the tree's
  references on its blocks, until the requested number of blocks have come
  back to the free list or no leaf is evictable.  A split creates a new node
  for the upper part; the lower part keeps its identity, time and hold count.
"""

import heapq

import numpy as np

from .allocator import BlockAllocator
from .prefix_cache import PrefixCachingAllocator


class _Node:
    __slots__ = ("id", "parent", "children", "tokens", "blocks", "lock", "time")

    def __init__(self, nid, parent, tokens, blocks, lock=0, time=0):
        self.id = nid
        self.parent = parent
        self.children = {}          # first block's token bytes -> child
        self.tokens = tokens        # int64 array, a whole number of blocks
        self.blocks = blocks        # list of physical blocks, one per B tokens
        self.lock = lock            # requests holding this node or one below it
        self.time = time


class RadixCache:
    def __init__(self, alloc: BlockAllocator, watermark: int = 0):
        if isinstance(alloc, PrefixCachingAllocator):
            raise TypeError("the radix cache sits on a plain BlockAllocator")
        self.alloc = alloc
        self.B = alloc.block_size
        self.watermark = int(watermark)
        self.root = _Node(0, None, np.zeros(0, dtype=np.int64), [], lock=1)
        self._next_id = 1
        self._clock = 0
        self._held = {}             # sequence -> node holding its reference
        self._cached = 0            # blocks on edges
        self.hit_tokens = 0
        self.query_tokens = 0
        self.evicted_blocks = 0

    # -------------------------------------------------------------- helpers
    def _key(self, tokens, at):
        return tokens[at:at + self.B].tobytes()

    def _split(self, node, nblk):
        """Cut ``node``'s edge after ``nblk`` blocks; returns the new upper node."""
        B = self.B
        up = _Node(self._next_id, node.parent, node.tokens[:nblk * B], node.blocks[:nblk],
                   node.lock, node.time)
        self._next_id += 1
        node.parent.children[self._key(node.tokens, 0)] = up
        node.tokens = node.tokens[nblk * B:]
        node.blocks = node.blocks[nblk:]
        node.parent = up
        up.children[self._key(node.tokens, 0)] = node
        return up

    def _walk(self, tokens):
        """Deepest node whose path is a whole-block prefix of ``tokens``
        (splitting an edge matched part-way) and the blocks on that path."""
        B = self.B
        node, pos, blocks = self.root, 0, []
        while pos + B <= len(tokens):
            child = node.children.get(self._key(tokens, pos))
            if child is None:
                break
            nb = len(child.blocks)
            run = min(nb, (len(tokens) - pos) // B)
            edge = child.tokens[:run * B].reshape(run, B)
            mine = tokens[pos:pos + run * B].reshape(run, B)
            same = (edge == mine).all(axis=1)
            k = run if same.all() else int(np.argmin(same))
            if k < nb:
                child = self._split(child, k)
            blocks += child.blocks
            pos += k * B
            node = child
            if k < nb:
                break
        return node, blocks, pos

    def _touch(self, node):
        self._clock += 1
        while node is not None:
            node.time = self._clock
            node = node.parent

    def _hold(self, node, d):
        while node is not None:
            node.lock += d
            node = node.parent

    # ---------------------------------------------------------------- lookup
    def match(self, tokens):
        """Longest cached whole-block prefix of ``tokens``: returns
        ``(blocks, cached_tokens)``.  Marks the path as used."""
        tokens = np.asarray(tokens, dtype=np.int64)
        node, blocks, got = self._walk(tokens)
        self._touch(node)
        return blocks, got

    def insert(self, tokens, blocks):
        """Cache ``tokens`` (its whole blocks) stored in ``blocks``.  The part
        already cached is kept as it is; the tree takes a reference on the
        blocks of the new part.  Returns the node that ends the path."""
        tokens = np.asarray(tokens, dtype=np.int64)
        B = self.B
        nblk = len(tokens) // B
        tokens = tokens[:nblk * B]
        node, _, got = self._walk(tokens)
        k = got // B
        if k < nblk:
            new = [int(b) for b in blocks[k:nblk]]
            self.alloc.incref(new)
            leaf = _Node(self._next_id, node, tokens[k * B:].copy(), new)
            self._next_id += 1
            node.children[self._key(leaf.tokens, 0)] = leaf
            self._cached += len(new)
            node = leaf
        self._touch(node)
        return node

    # -------------------------------------------------------------- requests
    def admit(self, tokens):
        """New sequence for a prompt whose cached prefix is mapped into its
        table by reference.  Returns ``(sid, cached_tokens)``; the caller
        appends and computes ``tokens[cached_tokens:]``."""
        tokens = np.asarray(tokens, dtype=np.int64)
        limit = max(0, (len(tokens) - 1) // self.B)
        limit = min(limit, self.alloc.max_blocks_per_seq)
        node, blocks, got = self._walk(tokens[:limit * self.B])
        self._touch(node)
        sid = self.alloc.adopt(blocks, got)
        self._hold(node, +1)
        self._held[sid] = node
        self.query_tokens += len(tokens)
        self.hit_tokens += got
        return sid, got

    def cache_seq(self, sid: int, tokens) -> None:
        """Insert the sequence's full blocks (``tokens`` are its token ids
        from position 0) and move its hold to the end of that path, so other
        requests can share what it has computed so far."""
        full = self.alloc.context_len(sid) // self.B
        node = self.insert(np.asarray(tokens, dtype=np.int64)[:full * self.B],
                           self.alloc.block_table(sid)[:full])
        self._hold(node, +1)
        self._hold(self._held[sid], -1)
        self._held[sid] = node

    def finish(self, sid: int, tokens=None) -> None:
        """End a request: optionally cache its full blocks, release its hold
        and free the sequence (blocks the tree holds stay allocated)."""
        if tokens is not None:
            self.cache_seq(sid, tokens)
        self._hold(self._held.pop(sid), -1)
        self.alloc.free(sid)

    # -------------------------------------------------------------- eviction
    def evict(self, want: int) -> int:
        """Evict least recently used unreferenced leaves until ``want``
        blocks have returned to the free list (or nothing is evictable).
        Returns the number returned."""
        heap = []
        stack = [self.root]
        while stack:
            n = stack.pop()
            stack.extend(n.children.values())
            if n is not self.root and not n.children and n.lock == 0:
                heap.append((n.time, n.id, n))
        heapq.heapify(heap)
        freed = 0
        while freed < want and heap:
            _, _, n = heapq.heappop(heap)
            p = n.parent
            del p.children[self._key(n.tokens, 0)]
            self._cached -= len(n.blocks)
            self.evicted_blocks += len(n.blocks)
            freed += self.alloc.decref(n.blocks)
            if p is not self.root and not p.children and p.lock == 0:
                heapq.heappush(heap, (p.time, p.id, p))
        return freed

    def ensure_free(self) -> int:
        """Evict until the allocator has ``watermark`` free blocks (if it can)."""
        short = self.watermark - self.alloc.num_free()
        return self.evict(short) if short > 0 else 0

    # --------------------------------------------------------------- queries
    def cached_blocks(self) -> int:
        return self._cached

    def nodes(self):
        """(id, path length in tokens, blocks, hold count, time) of every
        node but the root, in depth-first order."""
        out = []
        stack = [(self.root, 0)]
        while stack:
            n, depth = stack.pop()
            if n is not self.root:
                out.append((n.id, depth, list(n.blocks), n.lock, n.time))
            for c in n.children.values():
                stack.append((c, depth + len(c.tokens)))
        return out

    def validate(self) -> None:
        holders = np.zeros(self.alloc.num_blocks, dtype=np.int64)
        total = 0
        stack = [self.root]
        while stack:
            n = stack.pop()
            want = sum(c.lock for c in n.children.values())
            assert n.lock >= want, "hold count below its children's"
            for key, c in n.children.items():
                assert c.parent is n and key == self._key(c.tokens, 0), "child link"
                assert len(c.tokens) == len(c.blocks) * self.B and c.blocks, "edge size"
                holders[c.blocks] += 1
                total += len(c.blocks)
                stack.append(c)
        assert total == self._cached, "cached block count"
        self.alloc.validate(held=holders)
