"""Bit-exact parity of the pool-moving calls (append, copy_blocks, gather)
and of the allocator's slots/tables against the oracle."""

import numpy as np
import pytest
import torch

import oracle_pins as P
from gpu_helpers import LibDecodeState, i32, poisoned_pools, to_dev, words_of
from oracle import block_manager, paging
from paged_kv_cache_63_amd import BlockAllocator, _lib
from workloads import decode_case, gqa4_decode, normal_words, tiny_fp32_decode

pytestmark = pytest.mark.gpu


def _oracle_slots_tables(case):
    bm = block_manager.RefBlockManager(case.num_blocks, 16, case.free_order)
    slots, tables = [], []
    for L in case.context_lens:
        sid = bm.new_seq()
        s, _ = bm.append(sid, int(L))
        slots += s
        tables.append(bm.table(sid))
    return np.asarray(slots), tables


@pytest.mark.parametrize("case_fn", [
    lambda: tiny_fp32_decode(),
    lambda: decode_case(101, 7, 1, 300, 8, 2, 128, "bf16", spare_blocks=5),
    lambda: decode_case(102, 5, 1, 200, 4, 4, 64, "bf16"),
    lambda: decode_case(103, 5, 1, 200, 6, 3, 128, "fp32"),
], ids=["tiny-fp32", "bf16-d128", "bf16-d64", "fp32-d128"])
def test_append_pool_bit_exact(gpu, case_fn):
    case = case_fn()
    st = LibDecodeState(case)
    slots, tables = _oracle_slots_tables(case)
    assert np.array_equal(st.slots, slots)                      # a1: slots
    for s, t in enumerate(tables):                              # a1: tables
        row = st.alloc.tables[s]
        assert row[:len(t)].tolist() == t and (row[len(t):] == -1).all()
    kp, vp = paging.new_pools(case.num_blocks, case.num_kv_heads, case.head_dim, 16, case.dtype)
    paging.append(kp, vp, case.k, case.v, slots, 16)
    torch.cuda.synchronize()
    assert np.array_equal(words_of(st.k_pool), kp)              # a2: whole pool, NaN included
    assert np.array_equal(words_of(st.v_pool), vp)


def test_append_full_size_gqa4(gpu):
    """Llama-3-8B-shaped pool (64 sequences, ~147K tokens, 0.6 GB): every word."""
    case = gqa4_decode()
    st = LibDecodeState(case)
    kp, vp, _ = P.oracle_pools_for_decode(case)
    torch.cuda.synchronize()
    assert np.array_equal(words_of(st.k_pool), kp)
    assert np.array_equal(words_of(st.v_pool), vp)


def test_append_skips_negative_slots(gpu):
    k, v = poisoned_pools(4, 2, 64, "bf16")
    before = words_of(k).copy()
    kn = torch.ones((3, 2, 64), dtype=torch.bfloat16, device="cuda")
    _lib.paged_kv_append(kn, kn, i32([-1, 21, -7]), k, v)     # slot 21 = block 1, offset 5
    after = words_of(k)
    assert (after[1, :, 5, :] == 0x3F80).all()                  # bf16 1.0
    after[1, :, 5, :] = before[1, :, 5, :]
    assert np.array_equal(after, before)                        # nothing else written


def _mixed_run_slots(copies):
    """Slots for one append that mixes full-block runs with everything that
    must not be taken for one; ``copies`` repeats the pattern over disjoint
    blocks (16 per copy), and one more full run ends the input."""
    s = []
    for k in range(copies):
        b = 16 * k
        s += [(b + 3) * 16 + o for o in range(16)]            # full run, window-aligned
        s += [(b + 7) * 16 + o for o in range(11, 16)]        # partial tail of a block
        s += [(b + 2) * 16 + o for o in range(16)]            # full run starting mid-window
        s += [(b + 5) * 16 + o for o in range(15)]            # 15 consecutive: not a full block
        s += [-1]                                             # skipped token
        s += [(b + 9) * 16 + o for o in range(8)]             # two half blocks: broken run
        s += [(b + 10) * 16 + o for o in range(8, 16)]
        s += [(b + 11) * 16 + o for o in range(16)]           # full run across two windows
        s += [(b + 0) * 16 + o for o in range(16)]            # full run
        s += [(b + 12) * 16 + o for o in (0, 2, 1, 3)]        # right block, wrong order
        s += [-5, (b + 13) * 16 + 15, (b + 13) * 16]          # scattered single tokens
    s += [(16 * copies + 1) * 16 + o for o in range(16)]      # full run ending the input
    return np.asarray(s), 16 * copies + 2


@pytest.mark.parametrize("copies", [1, 5], ids=["per-token-path", "bulk-path"])
@pytest.mark.parametrize("dtype,d,hkv", [("bf16", 128, 8), ("bf16", 64, 3), ("fp32", 128, 2)])
def test_append_mixed_runs_bit_exact(gpu, dtype, d, hkv, copies):
    """One call with full-block runs and partial, broken and skipped tokens.
    Below 512 tokens every token is written on its own; from 512 on, full
    runs go through the transposed-V path and the rest token by token."""
    slots, nb = _mixed_run_slots(copies)
    assert (len(slots) >= 512) == (copies > 1)
    live = slots[slots >= 0]
    assert len(np.unique(live)) == len(live)
    rng = np.random.default_rng(7 + copies)
    kw = normal_words(rng, (len(slots), hkv, d), dtype)
    vw = normal_words(rng, (len(slots), hkv, d), dtype)
    k, v = poisoned_pools(nb, hkv, d, dtype)
    kp, vp = words_of(k).copy(), words_of(v).copy()
    _lib.paged_kv_append(to_dev(kw, dtype), to_dev(vw, dtype), i32(slots), k, v)
    paging.append(kp, vp, kw, vw, slots, 16)
    torch.cuda.synchronize()
    assert np.array_equal(words_of(k), kp)
    assert np.array_equal(words_of(v), vp)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("fp32", 64)])
def test_copy_blocks_bit_exact(gpu, dtype, d):
    rng = np.random.default_rng(7)
    nb, hkv = 40, 8
    kw = normal_words(rng, (nb, hkv, 16, d), dtype)
    vw = normal_words(rng, (nb, hkv, d, 16), dtype)
    pairs = np.array([[3, 30], [17, 2], [5, 39], [0, 12]])
    k, v = to_dev(kw, dtype), to_dev(vw, dtype)
    _lib.copy_blocks(k, v, i32(pairs))
    kr, vr = kw.copy(), vw.copy()
    paging.copy_blocks(kr, vr, pairs)
    torch.cuda.synchronize()
    assert np.array_equal(words_of(k), kr) and np.array_equal(words_of(v), vr)


@pytest.mark.parametrize("case_fn", [
    lambda: decode_case(111, 3, 1, 500, 8, 2, 128, "bf16"),
    lambda: decode_case(112, 3, 1, 100, 4, 4, 64, "fp32"),
], ids=["bf16", "fp32"])
def test_gather_bit_exact(gpu, case_fn):
    case = case_fn()
    st = LibDecodeState(case)
    kp, vp, tab = P.oracle_pools_for_decode(case)
    for s in range(case.num_seqs):
        L = int(case.context_lens[s])
        ko = torch.empty((L, case.num_kv_heads, case.head_dim), dtype=st.q.dtype, device="cuda")
        vo = torch.empty_like(ko)
        _lib.paged_kv_gather(ko, vo, st.k_pool, st.v_pool, st.tables[s].contiguous(), L)
        kr, vr = paging.gather(kp, vp, tab[s], L, 16)
        assert np.array_equal(words_of(ko), kr) and np.array_equal(words_of(vo), vr)
        c0, c1 = case.cu_tokens[s], case.cu_tokens[s + 1]
        assert np.array_equal(kr, case.k[c0:c1])


def test_decode_step_allocator_and_append(gpu):
    """Steps of one-token appends (allocate on overflow) through the batched
    allocator path, compared with the oracle model and oracle append."""
    rng = np.random.default_rng(5)
    S, hkv, d, nb = 12, 2, 64, 400
    order = rng.permutation(nb)
    lib = BlockAllocator(nb, 16, max_seqs=S, max_blocks_per_seq=40, free_order=order)
    ref = block_manager.RefBlockManager(nb, 16, order)
    sids = [lib.new_seq() for _ in range(S)]
    rids = [ref.new_seq() for _ in range(S)]
    k, v = poisoned_pools(nb, hkv, d, "bf16")
    kr, vr = paging.new_pools(nb, hkv, d, 16, "bf16")
    for step in range(40):
        kw = normal_words(rng, (S, hkv, d), "bf16")
        vw = normal_words(rng, (S, hkv, d), "bf16")
        slots, pairs = lib.append_step(sids)
        want = [ref.append(r, 1)[0][0] for r in rids]
        assert slots.tolist() == want and len(pairs) == 0
        _lib.paged_kv_append(to_dev(kw, "bf16"), to_dev(vw, "bf16"), i32(slots), k, v)
        paging.append(kr, vr, kw, vw, np.asarray(want), 16)
    torch.cuda.synchronize()
    assert np.array_equal(words_of(k), kr) and np.array_equal(words_of(v), vr)


@pytest.mark.parametrize("nbytes", [1, 15, 16, 17, 4099, 67840])
@pytest.mark.parametrize("dst_off,src_off", [(0, 0), (4, 0), (0, 1), (3, 5)])
def test_pinned_upload_bytes(gpu, nbytes, dst_off, src_off):
    """Bytes from pinned host memory (and from device memory) land exactly;
    the bytes around the destination range stay as they were."""
    rng = np.random.default_rng(nbytes * 31 + dst_off * 7 + src_off)
    payload = rng.integers(0, 256, nbytes + src_off, dtype=np.uint8)
    src = torch.from_numpy(payload).pin_memory()[src_off:]
    dst = torch.full((nbytes + dst_off + 8,), 0xA5, dtype=torch.uint8, device="cuda")
    _lib.pinned_upload(dst[dst_off:dst_off + nbytes], src)
    dev_src = torch.from_numpy(payload[src_off:].copy()).cuda()
    dst2 = torch.full_like(dst, 0x5A)
    _lib.pinned_upload(dst2[dst_off:dst_off + nbytes], dev_src)
    torch.cuda.synchronize()
    for d, fill in ((dst, 0xA5), (dst2, 0x5A)):
        got = d.cpu().numpy()
        assert np.array_equal(got[dst_off:dst_off + nbytes], payload[src_off:])
        assert (got[:dst_off] == fill).all() and (got[dst_off + nbytes:] == fill).all()


def test_pinned_upload_rejects_pageable_host_memory(gpu):
    dst = torch.empty(64, dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError):
        _lib.pinned_upload(dst, torch.zeros(64, dtype=torch.uint8))


@pytest.mark.parametrize("n", [0, 64, 300, 600])
@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("fp32", 64)])
def test_upload_and_append_matches_separate_calls(gpu, n, dtype, d):
    """One call = pinned_upload of the staging buffer + paged_kv_append with
    the slot mapping found inside it (at an offset), bit for bit: below 512
    tokens in one launch, from 512 on as upload + bulk append."""
    hkv, nb = 4, 96
    rng = np.random.default_rng(n * 3 + d)
    slots = rng.permutation(nb * 16)[:n].astype(np.int32)
    if n:
        slots[rng.integers(0, n, max(1, n // 20))] = -1          # skipped tokens
    head = rng.integers(0, 1000, 37).astype(np.int32)              # other index arrays
    tail = rng.integers(-5, 1000, 101).astype(np.int32)
    staging = torch.from_numpy(np.concatenate([head, slots, tail])).pin_memory()
    kw = normal_words(rng, (n, hkv, d), dtype)
    vw = normal_words(rng, (n, hkv, d), dtype)
    kn, vn = to_dev(kw, dtype), to_dev(vw, dtype)
    k1, v1 = poisoned_pools(nb, hkv, d, dtype)
    k2, v2 = poisoned_pools(nb, hkv, d, dtype)
    dst1 = torch.full((staging.numel() + 3,), -7, dtype=torch.int32, device="cuda")
    dst2 = torch.full_like(dst1, -7)
    _lib.upload_and_append(dst1[:staging.numel()], staging, kn, vn, k1, v1, slots_at=len(head))
    _lib.pinned_upload(dst2[:staging.numel()], staging)
    if n:
        _lib.paged_kv_append(kn, vn, dst2[len(head):len(head) + n], k2, v2)
    torch.cuda.synchronize()
    assert np.array_equal(dst1.cpu().numpy(), dst2.cpu().numpy())
    assert (dst1.cpu().numpy()[staging.numel():] == -7).all()
    assert np.array_equal(words_of(k1), words_of(k2))
    assert np.array_equal(words_of(v1), words_of(v2))
    k0, v0 = poisoned_pools(nb, hkv, d, dtype)                     # and against the oracle
    kp, vp = words_of(k0).copy(), words_of(v0).copy()
    paging.append(kp, vp, kw, vw, slots, 16)
    assert np.array_equal(words_of(k1), kp) and np.array_equal(words_of(v1), vp)


@pytest.mark.parametrize("n", [0, 64, 600])
@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("fp32", 64)])
def test_upload_and_append_tables(gpu, n, dtype, d):
    """upload_and_append_tables: the same upload and append as
    upload_and_append, plus (index, value) pairs stored after the staged words
    written into a device-resident table in the same launch (from 512 tokens
    in the upload launch before the bulk append), bit for bit; indexes
    outside the table are skipped, and the table's other words keep their
    contents."""
    hkv, nb = 4, 96
    rng = np.random.default_rng(910 + n + d)
    slots = rng.permutation(nb * 16)[:n].astype(np.int32)
    head = rng.integers(0, 1000, 12).astype(np.int32)
    S, maxb = 37, 23
    table0 = rng.integers(-1, nb, (S, maxb)).astype(np.int32)
    idx = np.concatenate([rng.choice(S * maxb, 50, replace=False),
                          [-1, S * maxb, S * maxb + 7]]).astype(np.int32)   # the last 3 are outside
    val = rng.integers(0, nb, len(idx)).astype(np.int32)
    pairs = np.stack([idx, val], 1).reshape(-1)
    staging = torch.from_numpy(np.concatenate([head, slots, pairs])).pin_memory()
    kw = normal_words(rng, (n, hkv, d), dtype)
    vw = normal_words(rng, (n, hkv, d), dtype)
    kn, vn = to_dev(kw, dtype), to_dev(vw, dtype)
    k1, v1 = poisoned_pools(nb, hkv, d, dtype)
    staged = len(head) + n
    dst = torch.full((staged + 3,), -7, dtype=torch.int32, device="cuda")
    tables = torch.from_numpy(table0).to("cuda")
    _lib.upload_and_append(dst[:staged], staging, kn, vn, k1, v1, slots_at=len(head),
                           tables=tables, num_updates=len(idx))
    torch.cuda.synchronize()
    want = table0.reshape(-1).copy()
    inside = (idx >= 0) & (idx < S * maxb)
    want[idx[inside]] = val[inside]
    assert np.array_equal(tables.cpu().numpy().reshape(-1), want)
    got = dst.cpu().numpy()
    assert np.array_equal(got[:staged], np.concatenate([head, slots]))
    assert (got[staged:] == -7).all()
    k0, v0 = poisoned_pools(nb, hkv, d, dtype)
    kp, vp = words_of(k0).copy(), words_of(v0).copy()
    paging.append(kp, vp, kw, vw, slots, 16)
    assert np.array_equal(words_of(k1), kp) and np.array_equal(words_of(v1), vp)
