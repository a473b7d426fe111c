"""Seeded random shapes for decode and extend, every output against the
oracle.  Each case draws its own combination (sequence or request count,
context and chunk lengths with empty and one-token ones among them, GQA
ratio from 1 to 16, head dim 64 or 128, block size 16 or 32, bf16 or fp32,
partition size), so that the kernels meet combinations that no hand-written
case names.  The pages fix the result as ordinary attention over the
sequence's tokens (Triptych page, technical summary: paging does not change
the attention scores; "RadixAttention: Tree-Based KV Cache Reuse in SGLang
Guide", "RadixAttention Architecture": only the unmatched suffix is
prefilled over the reused pages)."""

import numpy as np
import pytest
import torch

import oracle_pins as P
from gpu_helpers import f64_of, i32, poisoned_pools, to_dev, words_of
from oracle import attention
from paged_kv_cache_63_amd import BlockAllocator, _lib
from test_gpu_extend import LibExtendState
from workloads import decode_case, extend_case

pytestmark = pytest.mark.gpu

TOL = {"fp32": 1e-5, "bf16": 2e-2}
HEADS = [(4, 4), (8, 2), (16, 1), (32, 8), (64, 8), (8, 8), (24, 8), (12, 4)]


def _common(rng):
    hq, hkv = HEADS[int(rng.integers(len(HEADS)))]
    return (hq, hkv, int(rng.choice([64, 128])), int(rng.choice([16, 32])),
            "fp32" if rng.random() < 0.25 else "bf16")


@pytest.mark.parametrize("seed", range(24))
def test_decode_random_shape(gpu, seed):
    rng = np.random.default_rng(9100 + seed)
    hq, hkv, d, bs, dtype = _common(rng)
    S = int(rng.integers(1, 41))
    hi = int(rng.choice([40, 300, 2000]))
    lens = rng.integers(0, hi + 1, size=S)
    lens[rng.random(S) < 0.1] = 0
    lens[rng.random(S) < 0.1] = 1
    if lens.max() == 0:
        lens[0] = 1
    ptok = int(rng.choice([0, 32, 64, 256, 512]))
    case = decode_case(9100 + seed, S, 0, 0, hq, hkv, d, dtype, block_size=bs, lens=lens)
    mb = max(1, int(max(-(-int(L) // bs) for L in lens)))
    alloc = BlockAllocator(case.num_blocks, bs, max_seqs=S, max_blocks_per_seq=mb,
                           free_order=case.free_order)
    slots = [alloc.append_tokens(alloc.new_seq(), int(L))[0] for L in lens]
    k, v = poisoned_pools(case.num_blocks, hkv, d, dtype, bs=bs)
    slots = np.concatenate(slots)
    if len(slots):
        _lib.paged_kv_append(to_dev(case.k, dtype), to_dev(case.v, dtype), i32(slots), k, v)
    q = to_dev(case.q, dtype)
    out = torch.empty_like(q)
    _lib.paged_attention_decode(out, q, k, v, i32(alloc.tables[:S]), i32(lens),
                                int(lens.max()), case.scale, ptok)
    kp, vp, tab = P.oracle_pools_for_decode(case, block_size=bs)
    torch.cuda.synchronize()
    assert np.array_equal(words_of(k), kp) and np.array_equal(words_of(v), vp)
    want = attention.decode(case.q, kp, vp, tab, lens, case.scale, bs, dtype)
    err = np.abs(f64_of(out) - want).max()
    print(f"decode S={S} max_len={int(lens.max())} hq={hq} hkv={hkv} d={d} bs={bs} {dtype} "
          f"ptok={ptok}: max |err| {err:.3e}")
    assert err <= TOL[dtype], err


@pytest.mark.parametrize("seed", range(24))
def test_extend_random_shape(gpu, seed):
    rng = np.random.default_rng(9200 + seed)
    hq, hkv, d, bs, dtype = _common(rng)
    R = int(rng.integers(1, 9))
    new = rng.integers(0, int(rng.choice([8, 64, 160])) + 1, size=R)
    new[rng.random(R) < 0.15] = 0
    new[rng.random(R) < 0.15] = 1
    if new.max() == 0:
        new[0] = 1
    prefix = rng.integers(0, int(rng.choice([0, 100, 1000])) + 1, size=R)
    e = extend_case(9200 + seed, R, 0, 0, 0, 0, hq, hkv, d, dtype, block_size=bs,
                    prefix_lens=prefix, new_lens=new)
    st = LibExtendState(e)
    out = st.extend()
    kp, vp, tab, _, nslots = P.extend_state(e)
    assert np.array_equal(st.new_slots, nslots)
    torch.cuda.synchronize()
    assert np.array_equal(words_of(st.k_pool), kp) and np.array_equal(words_of(st.v_pool), vp)
    want = attention.extend(e.q, e.cu_new, e.seq_lens, kp, vp, tab, e.scale, bs, dtype)
    err = np.abs(f64_of(out) - want).max() if len(want) else 0.0
    print(f"extend R={R} max_new={int(new.max())} max_prefix={int(prefix.max())} hq={hq} "
          f"hkv={hkv} d={d} bs={bs} {dtype}: max |err| {err:.3e}")
    assert err <= TOL[dtype], err
