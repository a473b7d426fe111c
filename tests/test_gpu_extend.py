"""Extend (new tokens over a cached prefix, causal) against the oracle, plus
the cross-check extend row i == decode at context P+i+1 on the GPU."""

import numpy as np
import pytest
import torch

import oracle_pins as P
from gpu_helpers import f64_of, i32, poisoned_pools, to_dev, words_of
from oracle import attention
from paged_kv_cache_63_amd import BlockAllocator, _lib
from workloads import extend_case, multiturn_extend

pytestmark = pytest.mark.gpu

TOL = {"fp32": 1e-5, "bf16": 2e-2}


class LibExtendState:
    """Prefixes placed first, then every request's new chunk appended (the
    allocator continues each request's partly filled last block)."""

    def __init__(self, e, free_order=None):
        R = len(e.prefix_lens)
        bs = e.block_size
        mb = int(max(-(-int(x) // bs) for x in e.seq_lens))
        self.alloc = BlockAllocator(e.num_blocks, bs, max_seqs=R, max_blocks_per_seq=mb,
                                    free_order=e.free_order if free_order is None else free_order)
        self.k_pool, self.v_pool = poisoned_pools(e.num_blocks, e.num_kv_heads, e.head_dim, e.dtype,
                                                  bs=bs)
        sids = [self.alloc.new_seq() for _ in range(R)]
        pslots = np.concatenate([self.alloc.append_tokens(s, int(p))[0]
                                 for s, p in zip(sids, e.prefix_lens)])
        if len(pslots):
            _lib.paged_kv_append(to_dev(e.prefix_k, e.dtype), to_dev(e.prefix_v, e.dtype),
                                 i32(pslots), self.k_pool, self.v_pool)
        self.new_slots = np.concatenate([self.alloc.append_tokens(s, int(n))[0]
                                         for s, n in zip(sids, e.new_lens)])
        _lib.paged_kv_append(to_dev(e.new_k, e.dtype), to_dev(e.new_v, e.dtype),
                             i32(self.new_slots), self.k_pool, self.v_pool)
        self.tables = i32(self.alloc.tables[:R])
        self.q = to_dev(e.q, e.dtype)
        self.cu = i32(e.cu_new)
        self.seq_lens = i32(e.seq_lens)
        self.e = e

    def extend(self):
        e = self.e
        out = torch.empty_like(self.q)
        _lib.paged_attention_extend(out, self.q, self.cu, self.seq_lens, self.k_pool, self.v_pool,
                                    self.tables, int(max(e.new_lens)), int(max(e.seq_lens)),
                                    e.scale)
        return out


@pytest.mark.parametrize("dtype,R,plo,phi,nlo,nhi,hq,hkv,d", [
    ("fp32", 3, 0, 70, 1, 40, 4, 2, 64),
    ("fp32", 2, 100, 200, 30, 80, 8, 8, 128),
    ("bf16", 3, 0, 300, 1, 300, 32, 8, 128),
    ("bf16", 4, 17, 500, 60, 200, 8, 8, 128),
    ("bf16", 2, 1, 100, 5, 90, 16, 1, 64),
    ("bf16", 3, 1000, 2000, 250, 260, 64, 8, 128),
])
def test_small_cases(gpu, dtype, R, plo, phi, nlo, nhi, hq, hkv, d):
    e = extend_case(600 + R + plo + hq + d, R, plo, phi, nlo, nhi, hq, hkv, d, dtype)
    st = LibExtendState(e)
    out = st.extend()
    kp, vp, tab, pslots, nslots = P.extend_state(e)
    assert np.array_equal(st.new_slots, nslots)
    torch.cuda.synchronize()
    assert np.array_equal(words_of(st.k_pool), kp) and np.array_equal(words_of(st.v_pool), vp)
    want = attention.extend(e.q, e.cu_new, e.seq_lens, kp, vp, tab, e.scale, 16, dtype)
    err = np.abs(f64_of(out) - want).max()
    print(f"extend {dtype} R={R} hq={hq} hkv={hkv} d={d}: max |err| {err:.3e}")
    assert err <= TOL[dtype], err


@pytest.mark.timeout(600)
def test_multiturn_full_size(gpu):
    """16 requests, 2K..8K-token cached histories + 512 new tokens each,
    32 query heads over 8 KV heads: pool after the append bit for bit, and
    every output (8,192 new tokens x 32 query heads) against the oracle,
    one request per host thread."""
    from concurrent.futures import ThreadPoolExecutor
    e = multiturn_extend()
    st = LibExtendState(e)
    out = st.extend()
    kp, vp, tab, _, nslots = P.extend_state(e)
    assert np.array_equal(st.new_slots, nslots)
    torch.cuda.synchronize()
    assert np.array_equal(words_of(st.k_pool), kp) and np.array_equal(words_of(st.v_pool), vp)
    got = f64_of(out)
    assert np.isfinite(got).all()

    def one_req(r):
        want = attention.extend(e.q, e.cu_new, e.seq_lens, kp, vp, tab, e.scale, 16, "bf16",
                                reqs=[r])
        a, b = int(e.cu_new[r]), int(e.cu_new[r + 1])
        return float(np.abs(got[a:b] - want[a:b]).max())

    with ThreadPoolExecutor(max_workers=4) as ex:
        errs = list(ex.map(one_req, range(len(e.prefix_lens))))
    print("multiturn extend max |err| per request:", ["%.2e" % x for x in errs])
    assert max(errs) <= 2e-2, errs


@pytest.mark.parametrize("bs", [16, 32])
def test_permutation_bit_identical(gpu, bs):
    """The same prefixes and chunks placed by a second permutation of the
    pool (other physical blocks, other tables): the output bits do not
    change (Triptych page, "Look closer / Logical blocks, physical frames":
    logical neighbours need not be physical neighbours); at 16- and 32-token
    blocks."""
    e = extend_case(731, 5, 100, 3000, 1, 600, 32, 8, 128, "bf16", block_size=bs)
    a = LibExtendState(e)
    other = np.random.default_rng(931).permutation(e.num_blocks)
    b = LibExtendState(e, free_order=other)
    assert not torch.equal(a.tables, b.tables)
    oa, ob = a.extend(), b.extend()
    assert np.array_equal(words_of(oa), words_of(ob))
    kp, vp, tab, _, _ = P.extend_state(e)
    want = attention.extend(e.q, e.cu_new, e.seq_lens, kp, vp, tab, e.scale, bs, "bf16")
    assert np.abs(f64_of(oa) - want).max() <= 2e-2


def test_extend_equals_decode_per_token_on_gpu(gpu):
    """Row i of extend == the decode kernel over the context cut at P+i+1."""
    e = extend_case(701, 2, 30, 90, 20, 40, 16, 4, 128, "bf16")
    st = LibExtendState(e)
    ext = f64_of(st.extend())
    rows, tabs, lens = [], [], []
    for r in range(2):
        P_r = int(e.prefix_lens[r])
        for i in range(int(e.new_lens[r])):
            rows.append(int(e.cu_new[r]) + i)
            tabs.append(r)
            lens.append(P_r + i + 1)
    q = st.q[rows].contiguous()
    out = torch.empty_like(q)
    tables = st.tables[tabs].contiguous()
    _lib.paged_attention_decode(out, q, st.k_pool, st.v_pool, tables, i32(lens), max(lens),
                                e.scale, 64)
    assert np.abs(f64_of(out) - ext[rows]).max() <= 2e-2


def test_zero_prefix_is_causal_self_attention(gpu):
    e = extend_case(711, 2, 0, 0, 40, 130, 8, 2, 128, "bf16", prefix_lens=[0, 0])
    st = LibExtendState(e)
    out = f64_of(st.extend())
    kp, vp, tab, _, _ = P.extend_state(e)
    want = attention.extend(e.q, e.cu_new, e.seq_lens, kp, vp, tab, e.scale, 16, "bf16")
    assert np.abs(out - want).max() <= 2e-2


@pytest.mark.parametrize("factor", [40.0, -25.0])
def test_large_logits(gpu, factor):
    """Queries scaled so that row maxima reach hundreds of base-2 exponent
    units (and, with a negative factor, whole rows sit far below zero): the
    running reference of the online softmax must follow them without
    overflow or underflow."""
    from workloads.synth import bf16_words
    e = extend_case(721, 3, 100, 700, 30, 150, 16, 4, 128, "bf16")
    qf = (e.q.astype(np.uint32) << np.uint32(16)).view(np.float32) * np.float32(factor)
    e.q[...] = bf16_words(qf)
    st = LibExtendState(e)
    out = f64_of(st.extend())
    kp, vp, tab, _, _ = P.extend_state(e)
    want = attention.extend(e.q, e.cu_new, e.seq_lens, kp, vp, tab, e.scale, 16, "bf16")
    assert np.isfinite(out).all()
    err = np.abs(out - want).max()
    print(f"large logits x{factor}: max |err| {err:.3e}")
    assert err <= 2e-2, err


# Many workgroups.  The bf16 kernel runs one workgroup per (request, KV
# head, 256-row tile); the (request, KV head) units x, x + 8, ... share XCD
# x.  The cases below give every XCD several times more workgroups than it
# has compute units, of very different lengths, including empty ones.


def _extend_checked(e, reqs=None):
    """Pool bits, then the extend output against the oracle (all requests,
    or the listed ones); returns the max error."""
    st = LibExtendState(e)
    out = st.extend()
    kp, vp, tab, _, nslots = P.extend_state(e)
    assert np.array_equal(st.new_slots, nslots)
    torch.cuda.synchronize()
    assert np.array_equal(words_of(st.k_pool), kp) and np.array_equal(words_of(st.v_pool), vp)
    assert bool(torch.isfinite(out.float()).all())
    want = attention.extend(e.q, e.cu_new, e.seq_lens, kp, vp, tab, e.scale, e.block_size,
                            "bf16", reqs=reqs)
    rows = np.concatenate([np.arange(int(e.cu_new[r]), int(e.cu_new[r + 1]))
                           for r in (range(len(e.new_lens)) if reqs is None else reqs)])
    if not len(rows):
        return 0.0
    got = f64_of(out[torch.from_numpy(rows).to(out.device)])
    return float(np.abs(got - want[rows]).max())


@pytest.mark.parametrize("bs,hq,hkv,d", [(16, 32, 8, 128), (16, 32, 8, 64), (32, 32, 8, 128),
                                         (16, 8, 2, 128)])
def test_many_ragged_requests(gpu, bs, hq, hkv, d):
    """Ragged requests (some with no new token, some with one, chunks that
    end inside a row tile and inside a key block, cached prefixes from none
    to ~900 tokens), 120 workgroups per XCD: every output against the
    oracle."""
    R = 24 if hkv == 8 else 96
    rng = np.random.default_rng(4100 + bs + d + hkv)
    new = rng.integers(1, 300, size=R, endpoint=True)
    new[[0, 5, 11]] = 0
    new[[1, 7]] = 1
    new[2] = 300
    e = extend_case(4100 + bs + d + hkv, R, 0, 900, 0, 0, hq, hkv, d, "bf16", block_size=bs,
                    new_lens=new)
    g = hq // hkv
    items = -(-R * hkv // 8) * -(-300 * g // 256)
    assert 32 < items <= 1024
    err = _extend_checked(e)
    print(f"ragged bs={bs} d={d} hq={hq} hkv={hkv} workgroups/XCD={items}: max |err| {err:.3e}")
    assert err <= 2e-2, err


@pytest.mark.timeout(600)
@pytest.mark.parametrize("R", [128, 129])
def test_large_batches(gpu, R):
    """128 and 129 requests x 8 KV heads x 8 row tiles (1024 and 1032
    workgroups per XCD, the first request 512 new tokens long, the others
    1..512): every output finite, the pool bit for bit, and nine requests
    spread over the batch against the oracle."""
    rng = np.random.default_rng(4200 + R)
    new = rng.integers(1, 512, size=R, endpoint=True)
    new[0] = 512
    e = extend_case(4200 + R, R, 0, 96, 0, 0, 32, 8, 128, "bf16", new_lens=new)
    items = -(-R * 8 // 8) * 8
    assert items == (1024 if R == 128 else 1032)
    reqs = sorted({0, 1, R // 4, R // 2, R // 2 + 1, 3 * R // 4, R - 3, R - 2, R - 1})
    err = _extend_checked(e, reqs=reqs)
    print(f"R={R} ({items} workgroups/XCD): max |err| over {len(reqs)} requests {err:.3e}")
    assert err <= 2e-2, err
