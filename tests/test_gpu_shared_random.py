"""Seeded random families for the shared-prefix decode, every output against
the oracle's plain decode.  Each case draws its own batch: one to four
parents with prompts of various lengths, each forked into up to six children
(some early, before the parent grows on), children with empty to long
suffixes, lone sequences, a GQA ratio from 1 to 16, head dim 64 or 128 and a
partition size.  The block manager runs the same operations on both sides
(forks share blocks, a write into a shared partial block copies it first),
the groups come from the host helper, and the result must equal attention
over each sequence's own tokens (Triptych page, technical summary: sharing
is a pointer change and does not alter the attention scores)."""

import numpy as np
import pytest
import torch

from gpu_helpers import f64_of, i32, poisoned_pools, to_dev
from oracle import attention, block_manager, paging
from paged_kv_cache_63_amd import BlockAllocator, _lib, shared_prefix_groups
from workloads import normal_words

pytestmark = pytest.mark.gpu

HEADS = [(8, 2), (32, 8), (16, 1), (4, 4), (64, 8), (12, 4)]
NB = 4096


def _script(rng):
    ops, n = [], 0
    for p in range(int(rng.integers(1, 5))):
        par = f"P{p}"
        ops += [("new", par), ("add", par, int(rng.choice([16, 40, 100, 257, 600])))]
        if rng.random() < 0.4:   # a child forked before the parent grows on
            ops += [("fork", par, f"{par}e"), ("add", f"{par}e", int(rng.integers(0, 60)))]
            ops += [("add", par, int(rng.integers(1, 70)))]
        for c in range(int(rng.integers(0, 7))):
            ch = f"{par}c{c}"
            ops += [("fork", par, ch), ("add", ch, int(rng.choice([0, 1, 5, 30, 200, 500])))]
        ops += [("add", par, int(rng.integers(0, 50)))]
    for i in range(int(rng.integers(0, 4))):
        ops += [("new", f"L{i}"), ("add", f"L{i}", int(rng.integers(1, 400)))]
    return ops


def _run(side, ops, order, seed, hq, hkv, d):
    """Run ``ops`` on one side ('lib' or 'oracle'), K/V of every appended
    token drawn in op order from one seeded generator, then one decode step
    for every sequence."""
    rng = np.random.default_rng(seed)
    if side == "lib":
        bm = BlockAllocator(NB, 16, max_seqs=64, max_blocks_per_seq=128, free_order=order)
        k, v = poisoned_pools(NB, hkv, d, "bf16")
    else:
        bm = block_manager.RefBlockManager(NB, 16, order)
        k, v = paging.new_pools(NB, hkv, d, 16, "bf16")
    ids = {}

    def write(slots, pairs, kw, vw):
        if side == "lib":
            if len(pairs):
                _lib.copy_blocks(k, v, i32(np.asarray(pairs).reshape(-1, 2)))
            _lib.paged_kv_append(to_dev(kw, "bf16"), to_dev(vw, "bf16"), i32(slots), k, v)
        else:
            paging.copy_blocks(k, v, np.asarray(pairs, dtype=np.int64).reshape(-1, 2))
            paging.append(k, v, kw, vw, np.asarray(slots), 16)

    for op in ops:
        if op[0] == "new":
            ids[op[1]] = bm.new_seq()
        elif op[0] == "fork":
            ids[op[2]] = bm.fork(ids[op[1]])[0] if side == "lib" else bm.fork(ids[op[1]])
        elif op[0] == "add" and op[2] > 0:
            kw = normal_words(rng, (op[2], hkv, d), "bf16")
            vw = normal_words(rng, (op[2], hkv, d), "bf16")
            if side == "lib":
                s, p = bm.append_tokens(ids[op[1]], op[2])
                write(s, p.tolist(), kw, vw)
            else:
                s, p = bm.append(ids[op[1]], op[2])
                write(s, p, kw, vw)
    names = sorted(ids)
    kw = normal_words(rng, (len(names), hkv, d), "bf16")
    vw = normal_words(rng, (len(names), hkv, d), "bf16")
    if side == "lib":
        s, p = bm.append_step([ids[n] for n in names])
        write(s, p.tolist(), kw, vw)
        tables = bm.tables[[ids[n] for n in names]]
        lens = bm.lens[[ids[n] for n in names]]
    else:
        slots, pairs = [], []
        for n in names:
            a, b = bm.append(ids[n], 1)
            slots += a
            pairs += b
        write(slots, pairs, kw, vw)
        w = max(len(bm.table(ids[n])) for n in names)
        tables = np.full((len(names), w), -1, dtype=np.int64)
        for i, n in enumerate(names):
            t = bm.table(ids[n])
            tables[i, :len(t)] = t
        lens = np.array([bm.lens[ids[n]] for n in names])
    q = normal_words(rng, (len(names), hq, d), "bf16")
    return dict(k=k, v=v, tables=tables, lens=lens, q=q)


@pytest.mark.parametrize("seed", range(16))
def test_shared_decode_random_family(gpu, seed):
    rng = np.random.default_rng(9300 + seed)
    hq, hkv = HEADS[int(rng.integers(len(HEADS)))]
    d = int(rng.choice([64, 128]))
    ptok = int(rng.choice([0, 16, 64, 256]))
    ops = _script(rng)
    order = rng.permutation(NB)
    lib = _run("lib", ops, order, 9300 + seed, hq, hkv, d)
    ref = _run("oracle", ops, order, 9300 + seed, hq, hkv, d)
    w = ref["tables"].shape[1]
    assert np.array_equal(lib["tables"][:, :w], ref["tables"])
    assert np.array_equal(lib["lens"], ref["lens"])
    groups = shared_prefix_groups(lib["tables"], lib["lens"])
    scale = float(np.float32(1.0 / np.sqrt(d)))
    q = to_dev(lib["q"], "bf16")
    out = torch.full_like(q, float("nan"))
    _lib.paged_attention_decode_shared(out, q, lib["k"], lib["v"], i32(lib["tables"]),
                                       i32(lib["lens"]), int(lib["lens"].max()), scale,
                                       _lib.groups_to_device(groups), ptok)
    want = attention.decode(ref["q"], ref["k"], ref["v"], ref["tables"], ref["lens"],
                            np.float32(scale), 16, "bf16")
    got = f64_of(out)
    err = np.abs(got - want).max()
    print(f"seqs={len(ref['lens'])} groups={len(groups[2])} max_group={groups[3]} "
          f"max_prefix_blocks={groups[4]} max_len={int(ref['lens'].max())} hq={hq} hkv={hkv} "
          f"d={d} ptok={ptok}: max |err| {err:.3e}")
    assert np.isfinite(got).all() and err <= 2e-2, err
