"""Plain models of the two automatic prefix caches (oracle for the host-side
caches).

TEST INFRASTRUCTURE ONLY -- see the package docstring.

1. ``PrefixKeyedCache`` -- the chained-hash cache, written from what the
   chain stands for rather than from hashes.  A full block's chain digest
   depends on its parent's digest, its own tokens and extra metadata, so the
   chain names the whole token prefix up to that block ("PagedAttention and
   RadixAttention: Let's Talk About KV Cache", section "Two Layers, Not Two
   Rivals"); with a tenant salt in the key, equal prompts of different tenants
   never meet (same article, "Beyond the Two Techniques", cache salting).
   This model therefore keys each cached block by the tuple
   ``(salt, all tokens from position 0 to the end of the block)`` -- no hash
   at all, so a collision cannot occur in it.

2. ``FlatRadixTree`` -- the radix tree, kept as a flat list of nodes, each
   holding its full token path from the root; parents, children and matches
   are found by scanning the whole list.  Edges carry runs of tokens and the
   physical blocks that hold them; a lookup walks the longest cached prefix;
   an edge matched part-way is split at the point of divergence; a request
   holds a reference on every node of its path; under memory pressure the
   least recently used unreferenced leaves go first and shared inner nodes
   stay ("RadixAttention: Tree-Based KV Cache Reuse in SGLang Guide",
   "Architecture" parts 1, 3 and 4; "PagedAttention and RadixAttention",
   section "RadixAttention: A Tree That Does Not Forget"; "PagedAttention 与
   RadixAttention", section "RadixAttention", on the five-step figure where
   eviction starts at the leaves).

Both sit on the block-manager model of ``block_manager`` (FIFO free list,
copy-on-write of a shared partly filled block) and fix the same open points
as the library:

* Granularity is the block of B tokens: only whole blocks are cached, a
  match is rounded down to whole blocks, and a tree edge is split only
  between blocks.  A lookup for a prompt of n tokens uses at most
  ``(n - 1) // B`` blocks, so one prompt token is always left to compute.
* Hash model: a block is indexed when the caller commits it (after its K/V
  are written), unless its prefix already names another block or it is
  already indexed.  Indexed blocks are never written again (a write copies
  them first).  An indexed block with no reference is idle: allocation takes
  the FIFO free list first, then the idle block released longest ago; one
  sequence releases its idle-bound blocks deepest first, and plain blocks in
  logical order to the free list.
* Tree model: the tree holds one block reference for every block on its
  edges.  Time is a counter advanced once per lookup or insertion; every node
  on the path touched gets the new time.  Eviction removes, one at a time,
  the unreferenced leaf with the oldest time (ties: the node created
  first), dropping the tree's references on its blocks; it stops once the
  requested number of blocks have returned to the free list, or nothing is
  left to evict.  A split makes a new node for the upper (shared) part; the
  lower part keeps its identity, time and references.
"""

from .block_manager import OutOfBlocks, RefBlockManager


# ============================================================== hash model
class PrefixKeyedCache(RefBlockManager):
    def __init__(self, num_blocks: int, block_size: int, free_order=None):
        super().__init__(num_blocks, block_size, free_order)
        self.key_of = {}     # indexed block -> (salt, prefix tokens)
        self.block_of = {}   # (salt, prefix tokens) -> indexed block
        self.idle = []       # indexed blocks with no reference, released longest ago first
        self.salt = {}

    def _key(self, salt, tokens, k):
        B = self.block_size
        return (bytes(salt), tuple(int(t) for t in tokens[:(k + 1) * B]))

    def _take(self) -> int:
        if self.free:
            b = self.free.popleft()
        elif self.idle:
            b = self.idle.pop(0)
            del self.block_of[self.key_of.pop(b)]
        else:
            raise OutOfBlocks("no free block")
        self.ref[b] = 1
        return b

    def _drop_all(self, blocks) -> None:
        """Drop one reference from each block of a logical run."""
        zero = []
        for b in blocks:
            self.ref[b] -= 1
            if self.ref[b] == 0:
                del self.ref[b]
                zero.append(b)
        self.free.extend(b for b in zero if b not in self.key_of)
        self.idle.extend(b for b in reversed(zero) if b in self.key_of)

    def _drop(self, b: int) -> None:
        self._drop_all([b])

    def new_seq(self, salt=b"") -> int:
        sid = super().new_seq()
        self.salt[sid] = bytes(salt)
        return sid

    def start(self, tokens, salt=b""):
        """(sid, cached tokens): longest run of leading full blocks whose
        prefix is indexed, at most (len - 1) // B of them."""
        B = self.block_size
        sid = self.new_seq(salt)
        limit = max(0, (len(tokens) - 1) // B)
        for k in range(limit):
            key = self._key(salt, tokens, k)
            if key not in self.block_of:
                break
            b = self.block_of[key]
            if b in self.idle:
                self.idle.remove(b)
            self.ref[b] = self.ref.get(b, 0) + 1
            self.tables[sid].append(b)
        self.lens[sid] = len(self.tables[sid]) * B
        return sid, self.lens[sid]

    def append(self, sid: int, n: int):
        """Token-at-a-time append; a write into a shared or indexed partly
        filled block copies it first."""
        B = self.block_size
        table = self.tables[sid]
        slots, pairs = [], []
        for _ in range(n):
            pos = self.lens[sid]
            if pos % B == 0:
                table.append(self._take())
            elif self.ref[table[-1]] > 1 or table[-1] in self.key_of:
                src = table[-1]
                dst = self._take()
                pairs.append((src, dst))
                self._drop(src)
                table[-1] = dst
            slots.append(table[pos // B] * B + pos % B)
            self.lens[sid] = pos + 1
        return slots, pairs

    def commit(self, sid: int, tokens) -> int:
        added = 0
        for k in range(self.lens[sid] // self.block_size):
            b = self.tables[sid][k]
            key = self._key(self.salt[sid], tokens, k)
            if b not in self.key_of and key not in self.block_of:
                self.key_of[b] = key
                self.block_of[key] = b
                added += 1
        return added

    def fork(self, sid: int) -> int:
        child = super().fork(sid)
        self.salt[child] = self.salt[sid]
        return child

    def truncate(self, sid: int, new_len: int) -> None:
        keep = -(-new_len // self.block_size)
        gone = self.tables[sid][keep:]
        del self.tables[sid][keep:]
        self.lens[sid] = new_len
        self._drop_all(gone)

    def free_seq(self, sid: int) -> None:
        self._drop_all(self.tables.pop(sid))
        del self.lens[sid]
        del self.salt[sid]


# ============================================================== tree model
class FlatRadixTree:
    """Radix-tree prefix cache as a flat list of nodes over a
    ``RefBlockManager`` (whose ``ref`` the tree's own references add to)."""

    def __init__(self, bm: RefBlockManager):
        self.bm = bm
        self.B = bm.block_size
        # node: {"id", "path" (tokens root..end), "blocks" (this edge's), "lock", "time"}
        self.nodes = [{"id": 0, "path": (), "blocks": [], "lock": 1, "time": 0}]
        self.next_id = 1
        self.clock = 0
        self.seq_node = {}       # sequence -> node id its lock sits on

    # -- structure, by scanning ------------------------------------------
    def node(self, nid):
        return next(n for n in self.nodes if n["id"] == nid)

    def parent(self, n):
        """The node whose path is the longest proper prefix of n's path."""
        best = None
        for m in self.nodes:
            if len(m["path"]) < len(n["path"]) and n["path"][:len(m["path"])] == m["path"]:
                if best is None or len(m["path"]) > len(best["path"]):
                    best = m
        return best

    def children(self, n):
        return [m for m in self.nodes if m is not n and self.parent(m) is n]

    def ancestors(self, n):
        """n and every node above it, up to the root."""
        out = [n]
        while out[-1]["id"] != 0:
            out.append(self.parent(out[-1]))
        return out

    # -- lookup --------------------------------------------------------------
    def _matched_blocks(self, tokens):
        """Whole blocks of ``tokens`` found along some node path."""
        B = self.B
        best = 0
        for n in self.nodes:
            p = n["path"]
            k = 0
            while (k + 1) * B <= min(len(p), len(tokens)) and \
                    p[k * B:(k + 1) * B] == tuple(tokens[k * B:(k + 1) * B]):
                k += 1
            best = max(best, k)
        return best

    def _node_ending_at(self, tokens, nblk):
        """The node whose edge holds block nblk - 1 of tokens' path, split so
        that it ends exactly there."""
        B = self.B
        end = nblk * B
        want = tuple(int(t) for t in tokens[:end])
        for n in self.nodes:
            start = len(self.parent(n)["path"]) if n["id"] else 0
            if start < end <= len(n["path"]) and n["path"][:end] == want:
                if end == len(n["path"]):
                    return n
                upper = {"id": self.next_id, "path": want,
                         "blocks": n["blocks"][:(end - start) // B],
                         "lock": n["lock"], "time": n["time"]}
                self.next_id += 1
                n["blocks"] = n["blocks"][(end - start) // B:]
                self.nodes.append(upper)
                return upper
        return self.nodes[0] if nblk == 0 else None

    def _touch(self, n):
        self.clock += 1
        for m in self.ancestors(n):
            m["time"] = self.clock

    def match(self, tokens):
        """(node, blocks, cached tokens) for the longest cached prefix."""
        k = self._matched_blocks(tokens)
        n = self._node_ending_at(tokens, k)
        self._touch(n)
        blocks = []
        for m in reversed(self.ancestors(n)):
            blocks += m["blocks"]
        return n, blocks, k * self.B

    def insert(self, tokens, blocks):
        """Cache ``tokens`` (whole blocks) held in ``blocks``; blocks whose
        prefix is already cached are not taken.  Returns the node at the end."""
        B = self.B
        nblk = len(tokens) // B
        k = self._matched_blocks(tokens[:nblk * B])
        n = self._node_ending_at(tokens, k)
        if k < nblk:
            new = {"id": self.next_id, "path": tuple(int(t) for t in tokens[:nblk * B]),
                   "blocks": [int(b) for b in blocks[k:nblk]], "lock": 0, "time": 0}
            self.next_id += 1
            for b in new["blocks"]:
                self.bm.ref[b] += 1
            self.nodes.append(new)
            n = new
        self._touch(n)
        return n

    def lock(self, n, d):
        for m in self.ancestors(n):
            m["lock"] += d

    # -- requests ------------------------------------------------------------
    def admit(self, tokens):
        """New sequence for a prompt: map the cached prefix (at most
        (len - 1) // B blocks) by reference and hold its path."""
        B = self.B
        limit = max(0, (len(tokens) - 1) // B)
        n, blocks, got = self.match(list(tokens[:limit * B]))
        sid = self.bm.new_seq()
        self.bm.tables[sid] = list(blocks)
        self.bm.lens[sid] = got
        for b in blocks:
            self.bm.ref[b] += 1
        self.lock(n, +1)
        self.seq_node[sid] = n["id"]
        return sid, got

    def cache_seq(self, sid, tokens):
        """Insert the sequence's full blocks and move its hold to their end."""
        full = self.bm.lens[sid] // self.B
        n = self.insert(list(tokens[:full * self.B]), self.bm.tables[sid][:full])
        self.lock(n, +1)
        self.lock(self.node(self.seq_node[sid]), -1)
        self.seq_node[sid] = n["id"]

    def finish(self, sid, tokens=None):
        if tokens is not None:
            self.cache_seq(sid, tokens)
        self.lock(self.node(self.seq_node.pop(sid)), -1)
        self.bm.free_seq(sid)

    # -- eviction --------------------------------------------------------------
    def evict(self, want: int) -> int:
        freed = 0
        while freed < want:
            leaves = [n for n in self.nodes
                      if n["id"] != 0 and n["lock"] == 0 and not self.children(n)]
            if not leaves:
                break
            n = min(leaves, key=lambda m: (m["time"], m["id"]))
            self.nodes.remove(n)
            before = len(self.bm.free)
            for b in n["blocks"]:
                self.bm._drop(b)
            freed += len(self.bm.free) - before
        return freed

    def cached_blocks(self):
        return sum(len(n["blocks"]) for n in self.nodes)
