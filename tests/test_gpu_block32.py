"""Block size 32, the pages' alternative to 16 ("PagedAttention and
RadixAttention: Let's Talk About KV Cache", section "PagedAttention: Memory
Like an Operating System"; "RadixAttention: Tree-Based KV Cache Reuse in
SGLang Guide", section 2): append, copy-on-write copy and gather bit for bit
against the oracle's 32-token pools, decode and extend within tolerance, the
output bits independent of block placement, and the same attention as with
16-token blocks over the same tokens."""

import numpy as np
import pytest
import torch

import oracle_pins as P
from gpu_helpers import f64_of, i32, poisoned_pools, to_dev, words_of
from oracle import attention, paging
from paged_kv_cache_63_amd import BlockAllocator, _lib
from workloads import decode_case, extend_case

pytestmark = pytest.mark.gpu

TOL = {"fp32": 1e-5, "bf16": 2e-2}


class Decode32:
    """A decode case laid into a pool of `bs`-token blocks by the library."""

    def __init__(self, case, bs, free_order=None):
        self.case, self.bs = case, bs
        S = case.num_seqs
        order = case.free_order if free_order is None else free_order
        mb = max(1, int(max(-(-int(L) // bs) for L in case.context_lens)))
        self.alloc = BlockAllocator(case.num_blocks, bs, max_seqs=S, max_blocks_per_seq=mb,
                                    free_order=order)
        self.slots = np.concatenate([self.alloc.append_tokens(self.alloc.new_seq(), int(L))[0]
                                     for L in case.context_lens])
        self.k, self.v = poisoned_pools(case.num_blocks, case.num_kv_heads, case.head_dim,
                                        case.dtype, bs=bs)
        _lib.paged_kv_append(to_dev(case.k, case.dtype), to_dev(case.v, case.dtype),
                             i32(self.slots), self.k, self.v)
        self.tables = i32(self.alloc.tables[:S])
        self.lens = i32(case.context_lens)
        self.q = to_dev(case.q, case.dtype)

    def decode(self, partition_size=0):
        out = torch.empty_like(self.q)
        _lib.paged_attention_decode(out, self.q, self.k, self.v, self.tables, self.lens,
                                    int(max(self.case.context_lens)), self.case.scale,
                                    partition_size)
        return out


@pytest.mark.parametrize("dtype,hq,hkv,d,ptok", [
    ("bf16", 32, 8, 128, 0), ("bf16", 32, 8, 128, 64), ("bf16", 16, 2, 64, 32),
    ("fp32", 8, 2, 128, 64), ("fp32", 4, 4, 64, 0),
])
def test_decode_and_pool_at_block_size_32(gpu, dtype, hq, hkv, d, ptok):
    case = decode_case(3200 + hq + d + ptok, 9, 1, 900, hq, hkv, d, dtype, block_size=32)
    st = Decode32(case, 32)
    kp, vp, tab = P.oracle_pools_for_decode(case)
    # slots and the whole pool (NaN poison included) bit for bit
    assert np.array_equal(st.alloc.tables[:case.num_seqs, :tab.shape[1]], tab)
    torch.cuda.synchronize()
    assert np.array_equal(words_of(st.k), kp) and np.array_equal(words_of(st.v), vp)
    # the device walk of a table returns the tokens in logical order
    s = int(np.argmax(case.context_lens))
    L = int(case.context_lens[s])
    ko = torch.empty((L, hkv, d), dtype=st.q.dtype, device="cuda")
    vo = torch.empty_like(ko)
    _lib.paged_kv_gather(ko, vo, st.k, st.v, st.tables[s], L)
    kw, vw = paging.gather(kp, vp, tab[s], L, 32)
    torch.cuda.synchronize()
    assert np.array_equal(words_of(ko), kw) and np.array_equal(words_of(vo), vw)
    want = attention.decode(case.q, kp, vp, tab, case.context_lens, case.scale, 32, dtype)
    err = np.abs(f64_of(st.decode(ptok)) - want).max()
    assert err <= TOL[dtype], err


def test_copy_blocks_at_block_size_32(gpu):
    case = decode_case(3301, 5, 40, 200, 8, 2, 128, "bf16", block_size=32, spare_blocks=6)
    st = Decode32(case, 32)
    kp, vp, _ = P.oracle_pools_for_decode(case)
    used = sorted(set(int(b) for b in st.alloc.tables[:case.num_seqs].ravel() if b >= 0))
    free = [b for b in range(case.num_blocks) if b not in used]
    pairs = np.array([[used[0], free[0]], [used[3], free[1]], [used[-1], free[2]]], np.int32)
    _lib.copy_blocks(st.k, st.v, i32(pairs))
    paging.copy_blocks(kp, vp, pairs)
    torch.cuda.synchronize()
    assert np.array_equal(words_of(st.k), kp) and np.array_equal(words_of(st.v), vp)


def test_decode_block_size_32_permutation_and_16_equivalence(gpu):
    """A second placement gives the same bits; 16-token blocks holding the
    same tokens give the same attention within tolerance."""
    case = decode_case(3401, 12, 1, 2500, 32, 8, 128, "bf16", block_size=32, spare_blocks=20)
    a = Decode32(case, 32)
    b = Decode32(case, 32, free_order=np.random.default_rng(3402).permutation(case.num_blocks))
    assert not torch.equal(a.tables, b.tables)
    oa, ob = a.decode(), b.decode()
    assert np.array_equal(words_of(oa), words_of(ob))
    c16 = decode_case(3401, 12, 1, 2500, 32, 8, 128, "bf16", block_size=16)
    o16 = Decode32(c16, 16).decode()
    assert np.array_equal(c16.k, case.k) and np.array_equal(c16.q, case.q)
    assert np.abs(f64_of(oa) - f64_of(o16)).max() <= 2e-2


@pytest.mark.parametrize("dtype,R,plo,phi,nlo,nhi,hq,hkv,d", [
    ("bf16", 3, 0, 900, 1, 300, 32, 8, 128),
    ("bf16", 2, 33, 700, 60, 200, 16, 2, 64),
    ("bf16", 2, 2000, 3000, 500, 512, 32, 8, 128),
    ("fp32", 2, 10, 200, 20, 70, 8, 2, 128),
])
def test_extend_at_block_size_32(gpu, dtype, R, plo, phi, nlo, nhi, hq, hkv, d):
    e = extend_case(3500 + R + plo + hq + d, R, plo, phi, nlo, nhi, hq, hkv, d, dtype,
                    block_size=32)
    mb = int(max(-(-int(x) // 32) for x in e.seq_lens))
    alloc = BlockAllocator(e.num_blocks, 32, max_seqs=R, max_blocks_per_seq=mb,
                           free_order=e.free_order)
    k, v = poisoned_pools(e.num_blocks, hkv, d, dtype, bs=32)
    sids = [alloc.new_seq() for _ in range(R)]
    ps = np.concatenate([alloc.append_tokens(s, int(p))[0] for s, p in zip(sids, e.prefix_lens)])
    if len(ps):
        _lib.paged_kv_append(to_dev(e.prefix_k, dtype), to_dev(e.prefix_v, dtype), i32(ps), k, v)
    ns = np.concatenate([alloc.append_tokens(s, int(n))[0] for s, n in zip(sids, e.new_lens)])
    _lib.paged_kv_append(to_dev(e.new_k, dtype), to_dev(e.new_v, dtype), i32(ns), k, v)
    q = to_dev(e.q, dtype)
    out = torch.empty_like(q)
    _lib.paged_attention_extend(out, q, i32(e.cu_new), i32(e.seq_lens), k, v,
                                i32(alloc.tables[:R]), int(max(e.new_lens)), int(max(e.seq_lens)),
                                e.scale)
    kp, vp, tab, _, nslots = P.extend_state(e)
    assert np.array_equal(ns, nslots)
    torch.cuda.synchronize()
    assert np.array_equal(words_of(k), kp) and np.array_equal(words_of(v), vp)
    want = attention.extend(e.q, e.cu_new, e.seq_lens, kp, vp, tab, e.scale, 32, dtype)
    err = np.abs(f64_of(out) - want).max()
    print(f"extend block 32 {dtype} R={R} d={d}: max |err| {err:.3e}")
    assert err <= TOL[dtype], err


def test_shared_entry_at_block_size_32_without_groups_is_the_plain_decode(gpu):
    """With no groups the shared-prefix entry at 32-token blocks runs the
    plain decode and returns its bits (the forked families at 32-token
    blocks, with a prefix pass, are in the shared-prefix tests)."""
    case = decode_case(3601, 6, 100, 600, 32, 8, 128, "bf16", block_size=32)
    st = Decode32(case, 32)
    groups = _lib.groups_to_device((np.array([0], np.int32), np.zeros(0, np.int32),
                                    np.zeros(0, np.int32), 0, 0))
    out = torch.empty_like(st.q)
    _lib.paged_attention_decode_shared(out, st.q, st.k, st.v, st.tables, st.lens,
                                       int(max(case.context_lens)), case.scale, groups)
    assert np.array_equal(words_of(out), words_of(st.decode()))
