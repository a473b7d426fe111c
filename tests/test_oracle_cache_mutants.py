"""Plant plausible mistakes in copies of the oracle's prefix-cache models and
check that at least one pin catches each (CPU)."""

import pytest

import cache_pins as P
from oracle.prefix_cache import FlatRadixTree, PrefixKeyedCache


def _caught(pin, *a):
    try:
        pin(*a)
    except Exception:           # an assertion or a crash
        return True
    return False


# ------------------------------------------------------------ hash mutants
class SaltIgnored(PrefixKeyedCache):
    def _key(self, salt, tokens, k):
        return super()._key(b"", tokens, k)              # planted: salt dropped


class OwnBlockOnly(PrefixKeyedCache):
    def _key(self, salt, tokens, k):
        B = self.block_size                              # planted: no chaining
        return (bytes(salt), tuple(tokens[k * B:(k + 1) * B]))


class EvictNewest(PrefixKeyedCache):
    def _take(self):
        if not self.free and self.idle:
            self.idle.insert(0, self.idle.pop())         # planted: most recent first
        return super()._take()


class ShallowFirst(PrefixKeyedCache):
    def _drop_all(self, blocks):
        zero = []
        for b in blocks:
            self.ref[b] -= 1
            if self.ref[b] == 0:
                del self.ref[b]
                zero.append(b)
        self.free.extend(b for b in zero if b not in self.key_of)
        self.idle.extend(b for b in zero if b in self.key_of)   # planted: head first


class NoCap(PrefixKeyedCache):
    def start(self, tokens, salt=b""):
        B = self.block_size
        sid = self.new_seq(salt)
        for k in range(len(tokens) // B):                # planted: may reuse every token
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


class WritesCachedBlock(PrefixKeyedCache):
    def append(self, sid, n):
        saved = self.key_of
        self.key_of = {}                                 # planted: no copy of cached blocks
        try:
            return super().append(sid, n)
        finally:
            self.key_of = saved


HASH_PINS = [
    lambda m: P.pin_ttft(P.hash_driver(m)),
    lambda m: P.pin_three_users(P.hash_driver(m)),
    lambda m: P.pin_multi_turn(P.hash_driver(m)),
    lambda m: P.pin_five_step(P.hash_driver(m)),
    lambda m: P.pin_brute_force_lcp(P.hash_driver(m), 0, salts=True),
    lambda m: P.pin_salt(P.hash_driver(m)),
    lambda m: P.pin_lru_order(P.hash_driver(m), (4, 8)),
    lambda m: P.pin_cached_block_copied(m),
]


def test_hash_pins_hold():
    assert not any(_caught(p, PrefixKeyedCache) for p in HASH_PINS)


@pytest.mark.parametrize("mutant", [SaltIgnored, OwnBlockOnly, EvictNewest, ShallowFirst,
                                    NoCap, WritesCachedBlock])
def test_hash_mutants_caught(mutant):
    assert any(_caught(p, mutant) for p in HASH_PINS)


# ------------------------------------------------------------ tree mutants
class TreeEvictNewest(FlatRadixTree):
    def evict(self, want):
        freed = 0
        while freed < want:
            leaves = [n for n in self.nodes
                      if n["id"] != 0 and n["lock"] == 0 and not self.children(n)]
            if not leaves:
                break
            n = max(leaves, key=lambda m: (m["time"], m["id"]))   # planted
            self.nodes.remove(n)
            before = len(self.bm.free)
            for b in n["blocks"]:
                self.bm._drop(b)
            freed += len(self.bm.free) - before
        return freed


class TreeIgnoresHolds(FlatRadixTree):
    def lock(self, n, d):
        pass                                             # planted: holds never counted


class TreeEvictsInner(FlatRadixTree):
    def children(self, n):
        return []                                        # planted: every node looks like a leaf


class TreeNoSplit(FlatRadixTree):
    def _matched_blocks(self, tokens):
        # planted: a match stops at the last node boundary it fully covers
        k = super()._matched_blocks(tokens)
        ends = [len(n["path"]) // self.B for n in self.nodes if len(n["path"]) // self.B <= k
                and tuple(n["path"]) == tuple(tokens[:len(n["path"])])]
        return max(ends)


TREE_PINS = [
    lambda m: P.pin_ttft(P.tree_driver(m)),
    lambda m: P.pin_three_users(P.tree_driver(m), tree=True),
    lambda m: P.pin_multi_turn(P.tree_driver(m)),
    lambda m: P.pin_five_step(P.tree_driver(m), tree=True),
    lambda m: P.pin_brute_force_lcp(P.tree_driver(m), 0),
    lambda m: P.pin_lru_order(P.tree_driver(m), (0, 8)),
    lambda m: P.pin_tree_holds(P.tree_driver(m)),
]


def test_tree_pins_hold():
    assert not any(_caught(p, FlatRadixTree) for p in TREE_PINS)


@pytest.mark.parametrize("mutant", [TreeEvictNewest, TreeIgnoresHolds, TreeEvictsInner,
                                    TreeNoSplit])
def test_tree_mutants_caught(mutant):
    assert any(_caught(p, mutant) for p in TREE_PINS)
