"""Seeded input generators (random draws and shapes only).

Values: keys, values and queries are standard normal draws in float32,
made by the Box-Muller transform of float32 uniforms; a tensor is filled in
fixed chunks of 2^22 values, chunk i from the i-th child generator spawned
from the seed's generator (so the bits do not depend on how many threads fill
it).  bf16 inputs are those draws rounded to nearest-even bfloat16.  Integer lengths are inclusive uniform draws
(``rng.integers(lo, hi, endpoint=True)``), deliberately not multiples of the
block size, so partly filled last blocks occur.  The order in which physical
blocks leave the free list is a seeded permutation of the pool, so the blocks
of one sequence land scattered through the pool.

The five named workloads follow the shapes the pages discuss: grouped-query
decode, long contexts of ~10^5 tokens (the 128K-token context of "PagedAttention
and RadixAttention: Let's Talk About KV Cache", opening section), a shared
system prompt with parallel samples that fork from it ("Paged Attention for
Efficient Memory Management", technical summary; "RadixAttention: Tree-Based
KV Cache Reuse in SGLang Guide", "Multi-Candidate Tree Search"), and multi-turn
prefill over a cached history (same guide, "The Problem").
"""

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

DTYPES = ("fp32", "bf16")


def bf16_words(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return the
    16-bit words.  Inputs are finite."""
    bits = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (bits >> np.uint32(16)) & np.uint32(1)
    return ((bits + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


_CHUNK = 1 << 22
_THREADS = max(1, min(16, os.cpu_count() or 1))


def _box_muller(rng, n: int) -> np.ndarray:
    """n standard normal float32 values from 2*ceil(n/2) uniforms."""
    h = (n + 1) // 2
    u1 = np.float32(1) - rng.random(h, dtype=np.float32)      # (0, 1]
    u2 = rng.random(h, dtype=np.float32)
    r = np.sqrt(np.float32(-2) * np.log(u1))
    th = np.float32(2 * np.pi) * u2
    out = np.empty(2 * h, dtype=np.float32)
    out[:h] = r * np.cos(th)
    out[h:] = r * np.sin(th)
    return out[:n]


def normal_words(rng, shape, dtype: str) -> np.ndarray:
    """Standard normal draws stored as raw words of ``dtype``."""
    if dtype not in DTYPES:
        raise ValueError(dtype)
    n = int(np.prod(shape))
    word = np.uint32 if dtype == "fp32" else np.uint16
    out = np.empty(n, dtype=word)
    kids = rng.spawn(max(1, -(-n // _CHUNK)))

    def fill(i):
        a, b = i * _CHUNK, min(n, (i + 1) * _CHUNK)
        x = _box_muller(kids[i], b - a)
        out[a:b] = x.view(np.uint32) if dtype == "fp32" else bf16_words(x)

    if n:
        with ThreadPoolExecutor(_THREADS) as ex:
            list(ex.map(fill, range(len(kids))))
    return out.reshape(shape)


def _scale(head_dim: int) -> float:
    """1/sqrt(head_dim), rounded to float32 (the value both sides receive)."""
    return float(np.float32(1.0 / np.sqrt(head_dim)))


def _blocks_for(n: int, block_size: int) -> int:
    return -(-int(n) // block_size)


# --------------------------------------------------------------------------
# decode: one query token per sequence over a pre-populated context
# --------------------------------------------------------------------------
@dataclass
class DecodeCase:
    name: str
    dtype: str
    block_size: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    scale: float
    context_lens: np.ndarray      # int64 [S]; includes the token being decoded
    q: np.ndarray                 # words [S][Hq][D]
    k: np.ndarray                 # words [T][Hkv][D], sequences back to back
    v: np.ndarray                 # words [T][Hkv][D]
    cu_tokens: np.ndarray         # int64 [S+1]; sequence s owns k[cu[s]:cu[s+1]]
    num_blocks: int
    free_order: np.ndarray        # int64 permutation of range(num_blocks)
    extra: dict = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return len(self.context_lens)


def decode_case(seed: int, num_seqs: int, len_lo: int, len_hi: int, num_q_heads: int,
                num_kv_heads: int, head_dim: int, dtype: str, block_size: int = 16,
                lens=None, num_blocks=None, spare_blocks: int = 0,
                name: str = "decode") -> DecodeCase:
    """Draw order: lengths (unless given), q, k, v, free-list permutation."""
    rng = np.random.default_rng(seed)
    if lens is None:
        lens = rng.integers(len_lo, len_hi, size=num_seqs, endpoint=True)
    lens = np.asarray(lens, dtype=np.int64)
    cu = np.zeros(len(lens) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(lens)
    T = int(cu[-1])
    q = normal_words(rng, (len(lens), num_q_heads, head_dim), dtype)
    k = normal_words(rng, (T, num_kv_heads, head_dim), dtype)
    v = normal_words(rng, (T, num_kv_heads, head_dim), dtype)
    if num_blocks is None:
        num_blocks = sum(_blocks_for(L, block_size) for L in lens) + spare_blocks
    free_order = rng.permutation(num_blocks).astype(np.int64)
    return DecodeCase(name, dtype, block_size, num_q_heads, num_kv_heads, head_dim,
                      _scale(head_dim), lens, q, k, v, cu, int(num_blocks), free_order)


def tiny_fp32_decode(seed: int = 1) -> DecodeCase:
    """4 sequences of 5, 17, 33 and 64 tokens; 4 query heads = 4 KV heads;
    head_dim 64; fp32; a pool of 32 blocks of which the 10 needed ones are
    the first 10 entries of the seeded permutation."""
    return decode_case(seed, 4, 0, 0, 4, 4, 64, "fp32", lens=[5, 17, 33, 64],
                       num_blocks=32, name="tiny-fp32-decode")


def gqa4_decode(seed: int = 2, spare_blocks: int = 0) -> DecodeCase:
    """Llama-3-8B attention shape: 32 query heads over 8 KV heads, head_dim
    128, bf16; 64 sequences with contexts uniform in [512, 4096]; a pool sized
    to fit exactly (plus ``spare_blocks`` for decode steps that grow it)."""
    return decode_case(seed, 64, 512, 4096, 32, 8, 128, "bf16",
                       spare_blocks=spare_blocks, name="gqa4-decode-64x512-4096")


def long_context_decode(seed: int = 3) -> DecodeCase:
    """Llama-3.1-70B attention shape: 64 query heads over 8 KV heads,
    head_dim 128, bf16; 8 sequences with contexts uniform in [32768, 131072]."""
    return decode_case(seed, 8, 32768, 131072, 64, 8, 128, "bf16",
                       name="long-context-decode-8x32K-128K")


# --------------------------------------------------------------------------
# shared system prompt, forked parallel samples, one decode step
# --------------------------------------------------------------------------
@dataclass
class SharedPrefixCase:
    name: str
    dtype: str
    block_size: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    scale: float
    prefix_len: int
    suffix_lens: np.ndarray       # int64 [S0]
    parents: np.ndarray           # int64 [F]: original sequences that fork
    samples_per_parent: int       # each parent plus (samples-1) children
    prefix_k: np.ndarray          # words [prefix_len][Hkv][D]
    prefix_v: np.ndarray
    suffix_k: np.ndarray          # words [sum suffix][Hkv][D]
    suffix_v: np.ndarray
    cu_suffix: np.ndarray         # int64 [S0+1]
    new_k: np.ndarray             # words [S][Hkv][D]: one new token per decoding seq
    new_v: np.ndarray
    q: np.ndarray                 # words [S][Hq][D]
    num_blocks: int
    free_order: np.ndarray

    @property
    def num_decoding(self) -> int:
        """Decoding sequences: the originals, then for each parent in order
        its (samples_per_parent - 1) children."""
        return len(self.suffix_lens) + len(self.parents) * (self.samples_per_parent - 1)


def shared_prefix_case(seed: int, num_seqs: int, prefix_len: int, suffix_lo: int,
                       suffix_hi: int, num_parents: int, samples_per_parent: int,
                       num_q_heads: int, num_kv_heads: int, head_dim: int, dtype: str,
                       block_size: int = 16, name: str = "shared-prefix") -> SharedPrefixCase:
    """Draw order: suffix lengths; parents (without replacement); for each
    parent, suffix length redrawn until the parent's length is not a multiple
    of the block size (so its last block is partly filled and shared after the
    fork); prefix k, v; suffix k, v; new k, v; q; free-list permutation."""
    rng = np.random.default_rng(seed)
    suffix = rng.integers(suffix_lo, suffix_hi, size=num_seqs, endpoint=True).astype(np.int64)
    parents = np.sort(rng.choice(num_seqs, size=num_parents, replace=False)).astype(np.int64)
    for p in parents:
        while (prefix_len + suffix[p]) % block_size == 0:
            suffix[p] = rng.integers(suffix_lo, suffix_hi, endpoint=True)
    cu = np.zeros(num_seqs + 1, dtype=np.int64)
    cu[1:] = np.cumsum(suffix)
    S = num_seqs + num_parents * (samples_per_parent - 1)
    pk = normal_words(rng, (prefix_len, num_kv_heads, head_dim), dtype)
    pv = normal_words(rng, (prefix_len, num_kv_heads, head_dim), dtype)
    sk = normal_words(rng, (int(cu[-1]), num_kv_heads, head_dim), dtype)
    sv = normal_words(rng, (int(cu[-1]), num_kv_heads, head_dim), dtype)
    nk = normal_words(rng, (S, num_kv_heads, head_dim), dtype)
    nv = normal_words(rng, (S, num_kv_heads, head_dim), dtype)
    q = normal_words(rng, (S, num_q_heads, head_dim), dtype)
    # every block the case can ever hold: prefix, suffixes, one fresh block per
    # decoding sequence (overflow or copy-on-write), nothing more
    num_blocks = (_blocks_for(prefix_len, block_size)
                  + sum(_blocks_for(s, block_size) for s in suffix) + S)
    free_order = rng.permutation(num_blocks).astype(np.int64)
    return SharedPrefixCase(name, dtype, block_size, num_q_heads, num_kv_heads, head_dim,
                            _scale(head_dim), prefix_len, suffix, parents,
                            samples_per_parent, pk, pv, sk, sv, cu, nk, nv, q,
                            int(num_blocks), free_order)


def shared_prefix_decode(seed: int = 4) -> SharedPrefixCase:
    """256 sequences behind one 4096-token system prompt (256 shared blocks),
    each with its own 64..1024-token suffix; 4 of them fork into 4 parallel
    samples each (268 decoding sequences); Llama-3-8B attention shape, bf16."""
    return shared_prefix_case(seed, 256, 4096, 64, 1024, 4, 4, 32, 8, 128, "bf16",
                              name="shared-prefix-decode-256+4x4")


# --------------------------------------------------------------------------
# extend: new tokens over a cached prefix
# --------------------------------------------------------------------------
@dataclass
class ExtendCase:
    name: str
    dtype: str
    block_size: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    scale: float
    prefix_lens: np.ndarray       # int64 [R]
    new_lens: np.ndarray          # int64 [R]
    prefix_k: np.ndarray          # words [sum prefix][Hkv][D]
    prefix_v: np.ndarray
    cu_prefix: np.ndarray         # int64 [R+1]
    new_k: np.ndarray             # words [sum new][Hkv][D]
    new_v: np.ndarray
    q: np.ndarray                 # words [sum new][Hq][D]
    cu_new: np.ndarray            # int64 [R+1]
    num_blocks: int
    free_order: np.ndarray

    @property
    def seq_lens(self) -> np.ndarray:
        return self.prefix_lens + self.new_lens


def extend_case(seed: int, num_reqs: int, prefix_lo: int, prefix_hi: int, new_lo: int,
                new_hi: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                dtype: str, block_size: int = 16, prefix_lens=None, new_lens=None,
                name: str = "extend") -> ExtendCase:
    """Draw order: prefix lengths, new lengths (unless given), prefix k, v,
    new k, v, q, free-list permutation.  The pool fits exactly."""
    rng = np.random.default_rng(seed)
    if prefix_lens is None:
        prefix_lens = rng.integers(prefix_lo, prefix_hi, size=num_reqs, endpoint=True)
    if new_lens is None:
        new_lens = rng.integers(new_lo, new_hi, size=num_reqs, endpoint=True)
    P = np.asarray(prefix_lens, dtype=np.int64)
    N = np.asarray(new_lens, dtype=np.int64)
    cup = np.zeros(len(P) + 1, dtype=np.int64)
    cup[1:] = np.cumsum(P)
    cun = np.zeros(len(N) + 1, dtype=np.int64)
    cun[1:] = np.cumsum(N)
    pk = normal_words(rng, (int(cup[-1]), num_kv_heads, head_dim), dtype)
    pv = normal_words(rng, (int(cup[-1]), num_kv_heads, head_dim), dtype)
    nk = normal_words(rng, (int(cun[-1]), num_kv_heads, head_dim), dtype)
    nv = normal_words(rng, (int(cun[-1]), num_kv_heads, head_dim), dtype)
    q = normal_words(rng, (int(cun[-1]), num_q_heads, head_dim), dtype)
    num_blocks = sum(_blocks_for(p + n, block_size) for p, n in zip(P, N))
    free_order = rng.permutation(num_blocks).astype(np.int64)
    return ExtendCase(name, dtype, block_size, num_q_heads, num_kv_heads, head_dim,
                      _scale(head_dim), P, N, pk, pv, cup, nk, nv, q, cun,
                      int(num_blocks), free_order)


def multiturn_extend(seed: int = 5) -> ExtendCase:
    """16 requests, each a cached history of 2048..8192 tokens plus 512 new
    tokens; 32 query heads over 8 KV heads, head_dim 128, bf16."""
    return extend_case(seed, 16, 2048, 8192, 512, 512, 32, 8, 128, "bf16",
                       name="multiturn-extend-16x(2K-8K+512)")
