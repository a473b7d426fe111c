"""Pool layout, slot arithmetic, append, copy-on-write copy and gather (oracle).

TEST INFRASTRUCTURE ONLY -- see the package docstring.

The method (The Daily Triptych, "Paged Attention for Efficient Memory
Management", technical summary and "Look closer / Logical blocks, physical
frames"): the KV cache of every sequence is cut into blocks of B tokens; a
per-sequence block table maps logical block i to a physical block id in one
global pool; logical neighbours need not be physical neighbours.

Pool layout (the pages fix none; this is the layout the library uses and the
oracle reproduces, element for element):

  * K pool: ``[num_blocks][num_kv_heads][B][head_dim]`` -- one token's key is a
    contiguous row of ``head_dim`` words.
  * V pool: ``[num_blocks][num_kv_heads]`` slabs of ``head_dim * B`` words.
    A slab holds the block's value vectors transposed, in ``B / 16`` halves
    of 16 tokens: half ``off // 16`` is ``[head_dim][16]``, one row of 16
    tokens per channel, and inside a row the token at offset ``off % 16``
    sits at position ``v_pos(off % 16)``: bits 2 and 3 of the offset
    exchanged (tokens 0-3, 8-11, 4-7, 12-15; the map is its own inverse).
    For B = 16 this is ``[head_dim][16]``; the array's shape is
    ``[num_blocks][num_kv_heads][head_dim][B]`` for every B, a container
    of the slab's words (:func:`v_halves` gives the view by halves).

A *slot* names one token position in the pool: ``slot = phys_block * B + off``
with ``off`` in ``[0, B)``.  Logical position ``pos`` of a sequence lives in
slot ``table[pos // B] * B + pos % B``.
"""

import numpy as np

from .numerics import STORAGE_WORD, nan_word


def v_pos(off):
    """Position of a block's token ``off`` inside a V channel row (bits 2
    and 3 exchanged).  Works on ints and integer arrays."""
    return (off & ~12) | ((off & 4) << 1) | ((off & 8) >> 1)


def v_halves(v_pool):
    """The V pool viewed by 16-token halves: ``[num_blocks][num_kv_heads]
    [B / 16][head_dim][16]``, the same words (token ``off`` of a block, channel
    ``c``: ``[blk, h, off // 16, c, v_pos(off % 16)]``).  A block of fewer
    than 16 tokens (the model's small test blocks) is one ``[head_dim][B]``
    part."""
    nb, hkv, d, bs = v_pool.shape
    return v_pool.reshape(nb, hkv, max(bs // 16, 1), d, min(bs, 16))


def slot_of(table_row, pos: int, block_size: int) -> int:
    """Slot of logical position ``pos`` through one sequence's block table."""
    return int(table_row[pos // block_size]) * block_size + pos % block_size


def new_pools(num_blocks: int, num_kv_heads: int, head_dim: int, block_size: int,
              dtype: str):
    """Allocate K and V pools of raw words, every word a NaN (poison).

    Anything the method never writes keeps the NaN, so a read of an unused
    block or of the tail of a partly filled block shows up in every result
    that depends on it.
    """
    word = STORAGE_WORD[dtype]
    k = np.full((num_blocks, num_kv_heads, block_size, head_dim), nan_word(dtype), dtype=word)
    v = np.full((num_blocks, num_kv_heads, head_dim, block_size), nan_word(dtype), dtype=word)
    return k, v


def append(k_pool, v_pool, k_new, v_new, slot_mapping, block_size: int) -> None:
    """Write new tokens' keys and values into their pool slots, in place.

    Triptych page, "The story": a newly generated token's keys and values go
    into the next slot of the sequence's current block (a fresh block having
    been taken from the free pool when the current one was full).

    ``k_new``/``v_new``: ``[T][num_kv_heads][head_dim]`` raw words.
    ``slot_mapping``: ``[T]`` slots; a negative slot means "skip this token".
    Every head of token t is written.  Slots of one call are distinct (the
    caller guarantees it), so the order of the writes does not matter.
    """
    slots = np.asarray(slot_mapping, dtype=np.int64)
    vh = v_halves(v_pool)
    for t in range(slots.shape[0]):
        s = int(slots[t])
        if s < 0:
            continue
        blk, off = s // block_size, s % block_size
        k_pool[blk, :, off, :] = k_new[t]
        vh[blk, :, off // 16, :, v_pos(off % 16)] = v_new[t]


def copy_blocks(k_pool, v_pool, block_mapping) -> None:
    """Copy-on-write: make each ``dst`` block an exact copy of its ``src``.

    Triptych page, technical summary and "The story": after a fork, the
    first write into a block that is still shared copies that block, so the
    other references keep seeing the old contents.  The whole block (all KV
    heads, all B slots) is copied, for K and for V.  Sources are read from the
    pool as it was before the call.
    """
    pairs = np.asarray(block_mapping, dtype=np.int64).reshape(-1, 2)
    k_before = k_pool.copy()
    v_before = v_pool.copy()
    for src, dst in pairs:
        k_pool[dst] = k_before[src]
        v_pool[dst] = v_before[src]


def swap_blocks(dst_k, dst_v, src_k, src_v, block_mapping) -> None:
    """Move whole blocks between two pools (device and host tiers): each
    ``dst`` block of the destination pools becomes an exact copy of its
    ``src`` block of the source pools, K and V, all heads and slots.

    "PagedAttention and RadixAttention: Let's Talk About KV Cache", section
    "Beyond the Two Techniques": blocks move between GPU memory and host RAM
    and come back when needed; a block's contents travel unchanged.
    """
    for src, dst in np.asarray(block_mapping, dtype=np.int64).reshape(-1, 2):
        dst_k[dst] = src_k[src]
        dst_v[dst] = src_v[src]


def gather(k_pool, v_pool, table_row, context_len: int, block_size: int):
    """Follow one sequence's block table and return its keys and values in
    logical order, as ``[context_len][num_kv_heads][head_dim]`` raw words.

    Triptych page, "The story": the kernel walks the block table and collects
    the physical blocks; the history it sees is still in order.
    """
    _, hkv, _, d = k_pool.shape
    k_out = np.empty((context_len, hkv, d), dtype=k_pool.dtype)
    v_out = np.empty((context_len, hkv, d), dtype=v_pool.dtype)
    vh = v_halves(v_pool)
    for pos in range(context_len):
        blk = int(table_row[pos // block_size])
        off = pos % block_size
        k_out[pos] = k_pool[blk, :, off, :]
        v_out[pos] = vh[blk, :, off // 16, :, v_pos(off % 16)]
    return k_out, v_out


def gather_fast(k_pool, v_pool, table_row, context_len: int, block_size: int):
    """Same result as :func:`gather`, by whole blocks (for long contexts).

    Used where the per-token loop would take minutes (contexts of 10^5
    tokens).  A test checks it against :func:`gather` word for word.
    """
    nblk = -(-context_len // block_size)
    ids = np.asarray(table_row[:nblk], dtype=np.int64)
    kb = k_pool[ids]                               # [nblk][Hkv][B][D]
    vb = v_halves(v_pool)[ids][..., v_pos(np.arange(16))]   # [nblk][Hkv][B/16][D][16], token order
    _, hkv, _, d = k_pool.shape
    k_out = kb.transpose(0, 2, 1, 3).reshape(nblk * block_size, hkv, d)[:context_len]
    v_out = vb.transpose(0, 2, 4, 1, 3).reshape(nblk * block_size, hkv, d)[:context_len]
    return np.ascontiguousarray(k_out), np.ascontiguousarray(v_out)


def words(dtype: str):
    """numpy word type of a storage dtype."""
    return STORAGE_WORD[dtype]
