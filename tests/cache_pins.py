"""Pins for the oracle's prefix-cache models: the pages' worked examples
(``golden/prefix_reuse.json``), brute-force longest-common-prefix reuse and
the eviction rules.  Each ``pin_*`` raises AssertionError when the model it
is given disagrees; the mutant tests hand them models with planted mistakes.

The hash model is driven through ``start/append/commit/free_seq``, the tree
model through ``admit/append/finish`` over a ``RefBlockManager``.
"""

import json
import os

import numpy as np

from oracle.block_manager import RefBlockManager
from oracle.prefix_cache import FlatRadixTree, PrefixKeyedCache

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "prefix_reuse.json")))


def part(tag: int, n: int):
    """n token ids unique to part ``tag``: parts that differ differ at once."""
    return list(range(tag * 1_000_000, tag * 1_000_000 + n))


# ------------------------------------------------------------ two drivers
class HashDriver:
    """One interface over the hash model for the scenario pins.  Idle cached
    blocks are evicted on demand by the model itself."""

    def __init__(self, cls, num_blocks, B):
        self.m = cls(num_blocks, B, None)
        self.B = B

    def open(self, tokens, salt=b""):
        """Admit a prompt, compute (append) the rest, cache it; the request
        stays open.  Returns (sid, cached tokens at admission)."""
        sid, got = self.m.start(tokens, salt)
        self.m.append(sid, len(tokens) - got)
        self.m.commit(sid, tokens)
        return sid, got

    def extend(self, sid, n):
        self.m.append(sid, n)

    def close(self, sid, tokens):
        if tokens is not None:
            self.m.commit(sid, tokens)
        self.m.free_seq(sid)

    def run(self, tokens, keep_tokens=None, salt=b""):
        """open + close; only the first ``keep_tokens`` stay cached."""
        sid, got = self.m.start(tokens, salt)
        self.m.append(sid, len(tokens) - got)
        if keep_tokens is not None:
            self.m.truncate(sid, keep_tokens)
            tokens = tokens[:keep_tokens]
        self.m.commit(sid, tokens)
        self.m.free_seq(sid)
        return got

    def probe(self, tokens, salt=b""):
        """Cached tokens a prompt would reuse (admits and frees at once)."""
        sid, got = self.m.start(tokens, salt)
        self.m.free_seq(sid)
        return got

    def refs(self, sid):
        return [self.m.ref[b] for b in self.m.tables[sid]]


class TreeDriver:
    """The same interface over the tree model; before appending it evicts
    just enough to have the blocks the append needs."""

    def __init__(self, cls, num_blocks, B, bm_cls=RefBlockManager):
        self.bm = bm_cls(num_blocks, B, None)
        self.t = cls(self.bm)
        self.B = B

    def make_room(self, n):
        short = n - len(self.bm.free)
        if short > 0:
            self.t.evict(short)

    def extend(self, sid, n):
        B = self.B
        L = self.bm.lens[sid]
        self.make_room(-(-(L + n) // B) - len(self.bm.tables[sid]))
        self.bm.append(sid, n)

    def open(self, tokens, salt=b""):
        sid, got = self.t.admit(tokens)
        self.extend(sid, len(tokens) - got)
        self.t.cache_seq(sid, tokens)
        return sid, got

    def close(self, sid, tokens):
        self.t.finish(sid, tokens)

    def run(self, tokens, keep_tokens=None, salt=b""):
        sid, got = self.t.admit(tokens)
        self.extend(sid, len(tokens) - got)
        self.t.finish(sid, tokens[:keep_tokens] if keep_tokens is not None else tokens)
        return got

    def probe(self, tokens, salt=b""):
        sid, got = self.t.admit(tokens)
        self.t.finish(sid)
        return got

    def refs(self, sid):
        return [self.bm.ref[b] for b in self.bm.tables[sid]]


# ------------------------------------------------------------------ pins
def pin_ttft(make):
    g = GOLDEN["ttft_example"]
    for B, want in g["expected"].items():
        B = int(B)
        d = make(4096, B)
        shared = part(1, g["cached_prefix_tokens"])
        rest = g["prompt_tokens"] - g["cached_prefix_tokens"]
        d.run(shared + part(2, rest))
        got = d.run(shared + part(3, rest))
        assert got == want["cached"], (B, got)
        assert g["prompt_tokens"] - got == want["computed"]


def pin_three_users(make, tree=False):
    g = GOLDEN["three_users"]
    d = make(1024, g["block_size"])
    sys = part(1, g["system_tokens"])
    sids, got = [], []
    for i, q in enumerate(g["question_tokens"]):
        s, c = d.open(sys + part(10 + i, q))
        sids.append(s)
        got.append(c)
    assert got == g["expected_cached_tokens"], got
    nsys = g["system_tokens"] // g["block_size"]
    holds = g["expected_shared_node_holds"]
    if tree:
        shared = [n for n in d.t.nodes if len(n["path"]) == g["system_tokens"]]
        assert len(shared) == 1 and shared[0]["lock"] == holds, shared
        assert len(d.t.nodes) - 1 == g["expected_nodes"]
        holds += 1                      # the tree's own reference on each block
    assert all(r == holds for r in d.refs(sids[2])[:nsys])
    for s in sids:
        d.close(s, None)


def pin_multi_turn(make):
    g = GOLDEN["multi_turn_agent"]
    for B, want in g["expected_cached_prompt_only"].items():
        B = int(B)
        d = make(8192, B)
        prompt, got = [], []
        for i, n in enumerate(g["prompt_tokens"]):
            prompt = prompt + part(20 + i, n - len(prompt))
            answer = part(40 + i, 300)
            # generation appends an answer, but only the prompt is kept in the cache
            got.append(d.run(prompt + answer, keep_tokens=len(prompt)))
        assert got == want, (B, got)
        assert [min(g, p) for g, p in zip(got, g["printed_repeated_tokens"])] == got


def pin_five_step(make, tree=False):
    g = GOLDEN["five_step_figure"]
    L = g["lengths"]
    B = g["block_size"]
    d = make(g["pool_blocks"], B)
    sys = part(1, L["system"])
    s1t1, s1t2 = part(2, L["s1_turn1"]), part(3, L["s1_turn2"])
    s2t1 = part(4, L["s2_turn1"])

    def shape():
        return sorted([len(n["path"]), len(n["blocks"])] for n in d.t.nodes if n["id"])

    d.run(sys + s1t1)                                           # step 2
    if tree:
        assert shape() == g["expected_nodes_after"]["2"], shape()
    got = d.run(sys + s1t1 + s1t2)                              # step 3
    assert got == L["system"] + L["s1_turn1"]
    if tree:
        assert shape() == g["expected_nodes_after"]["3"], shape()
    got = d.run(sys + s2t1)                                     # step 4
    assert got == L["system"]
    if tree:
        assert shape() == g["expected_nodes_after"]["4"], shape()
    # step 5: the new session continues; its two new blocks force eviction
    q, a = part(5, L["s2_turn2_question"]), part(6, L["s2_turn2_answer"])
    prompt = sys + s2t1 + q
    sid, got = d.open(prompt + a[:1])
    assert got == L["system"] + L["s2_turn1"], got
    d.extend(sid, len(a) - 1)
    d.close(sid, prompt + a)
    want = g["expected_cached_after_step5"]
    # session 1's second turn is gone; its first turn and the system prompt stay
    assert d.probe(sys + s1t1 + s1t2 + [7]) == want["session1_full"]
    assert d.probe(sys + s2t1 + [7]) == want["session2_prompt"]
    if tree:
        d2 = make(g["pool_blocks"], B)
        d2.run(sys + s1t1)
        d2.run(sys + s1t1 + s1t2)
        d2.run(sys + s2t1)
        ids = {n["id"]: len(n["path"]) for n in d2.t.nodes}
        freed = d2.t.evict(5)
        left = {n["id"] for n in d2.t.nodes}
        gone = sorted(ids[i] for i in ids if i not in left)
        assert freed == 5 and gone == [112, 144], gone      # s1_turn2, then s1_turn1


def blocks_lcp(a, b, B):
    k = 0
    while (k + 1) * B <= min(len(a), len(b)) and a[k * B:(k + 1) * B] == b[k * B:(k + 1) * B]:
        k += 1
    return k


def pin_brute_force_lcp(make, seed=0, salts=False):
    """Without eviction, a prompt reuses exactly the longest whole-block
    common prefix it has with anything cached before (same salt), at most
    (n - 1) // B blocks."""
    rng = np.random.default_rng(seed)
    for B in (1, 2, 4):
        d = make(4096, B)
        seen = []
        for _ in range(40):
            if seen and rng.random() < 0.7:
                base_salt, base = seen[rng.integers(len(seen))]
                cut = int(rng.integers(0, len(base) + 1))
                toks = base[:cut] + [int(t) for t in rng.integers(0, 3, int(rng.integers(0, 12)))]
            else:
                toks = [int(t) for t in rng.integers(0, 3, int(rng.integers(0, 20)))]
            salt = bytes([int(rng.integers(0, 2))]) if salts else b""
            cap = max(0, (len(toks) - 1) // B)
            want = max([blocks_lcp(toks[:cap * B], t, B) for s, t in seen if s == salt] + [0])
            got = d.run(toks, salt=salt)
            assert got == want * B, (B, toks, got, want)
            seen.append((salt, toks[:len(toks) // B * B]))


def pin_salt(make):
    d = make(256, 4)
    toks = part(1, 40)
    d.run(toks, salt=b"tenant-a")
    assert d.run(toks, salt=b"tenant-b") == 0
    assert d.run(toks, salt=b"tenant-a") == 36


def pin_lru_order(make, want):
    """Pool of 6 blocks of 4 tokens: prompts a and b are cached in turn,
    then c's three blocks need room.  The hash model evicts one idle block:
    a's deepest (a released first, deepest first); the tree evicts a's whole
    leaf (the least recently used).  b survives in both."""
    d = make(6, 4)
    a, b, c = part(1, 8), part(2, 8), part(3, 8)
    d.run(a + [0])
    d.run(b + [0])
    sid, _ = d.open(c + [0])
    got = (d.probe(a + [9]), d.probe(b + [9]))
    assert got == want, got
    d.close(sid, None)


def pin_tree_holds(make):
    """A held path (a running request's) and inner nodes are never evicted."""
    d = make(64, 4)
    sys = part(1, 16)
    held, _ = d.open(sys + part(2, 9))
    d.run(sys + part(3, 9))
    d.run(sys + part(4, 9))
    freed = d.t.evict(10**6)
    # only the two unheld leaves go; the held path (system prompt and its leaf) stays
    assert freed == 4, freed
    assert sorted(len(n["path"]) for n in d.t.nodes if n["id"]) == [16, 24]
    d.close(held, None)
    assert d.t.evict(10**6) == 6 and len(d.t.nodes) == 1


def pin_cached_block_copied(cls=PrefixKeyedCache):
    """A write into a cached block copies it first, so the cache still holds
    the prefix afterwards."""
    m = cls(16, 4)
    toks = part(1, 12)
    sid, _ = m.start(toks)
    m.append(sid, 12)
    m.commit(sid, toks)
    m.truncate(sid, 6)                    # the next write lands in cached block 1
    _, pairs = m.append(sid, 1)
    assert pairs == [(1, 3)], pairs       # copied into free block 3
    m.free_seq(sid)
    _, got = m.start(toks + [5])
    assert got == 12


def hash_driver(cls=PrefixKeyedCache):
    return lambda nb, B: HashDriver(cls, nb, B)


def tree_driver(cls=FlatRadixTree, bm_cls=RefBlockManager):
    return lambda nb, B: TreeDriver(cls, nb, B, bm_cls)
