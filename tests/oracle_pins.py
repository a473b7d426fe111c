"""Pin checks for the oracle, written so that a test can run each check on the
real oracle (it must pass) and on a copy with a planted mistake (it must
fail).  Each check pins the oracle to something other than itself: a closed
form, brute force with Python floats, a library routine on contiguous data,
or an invariant the pages state.
"""

import math

import numpy as np
import torch

from oracle import attention, block_manager, numerics, paging


# ----------------------------------------------------------------- builders
def oracle_pools_for_decode(case, block_size=None, bm_cls=block_manager.RefBlockManager,
                            append_fn=paging.append, free_order=None):
    """Place every context token of a decode case into a fresh poisoned pool
    with the oracle's block manager and append; return (k_pool, v_pool, tables)."""
    B = block_size or case.block_size
    if free_order is not None:
        order = np.asarray(free_order)
    elif B == case.block_size:
        order = case.free_order
    else:   # another block size: a pool that fits, in a seeded order
        order = np.random.default_rng(0).permutation(sum(-(-int(L) // B) for L in case.context_lens))
    nb = len(order)
    bm = bm_cls(nb, B, order)
    slots = []
    tables = []
    for L in case.context_lens:
        sid = bm.new_seq()
        s, _ = bm.append(sid, int(L))
        slots += s
        tables.append(bm.table(sid))
    kp, vp = paging.new_pools(nb, case.num_kv_heads, case.head_dim, B, case.dtype)
    append_fn(kp, vp, case.k, case.v, np.asarray(slots), B)
    width = max(len(t) for t in tables)
    tab = np.full((len(tables), width), -1, dtype=np.int64)
    for i, t in enumerate(tables):
        tab[i, :len(t)] = t
    return kp, vp, tab


def torch_widen(words, dtype):
    """Independent widening through torch's own bf16/fp32 conversion."""
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(words).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(words).view(np.float32))
    return t.to(torch.float64)


def dense_sdpa(case, s):
    """torch's scaled_dot_product_attention (float64, CPU, grouped-query
    mode) on sequence s's contiguous keys and values, straight from the
    generator (never through a pool)."""
    c0, c1 = int(case.cu_tokens[s]), int(case.cu_tokens[s + 1])
    q = torch_widen(case.q[s], case.dtype)[None, :, None, :]          # [1][Hq][1][D]
    k = torch_widen(case.k[c0:c1], case.dtype).permute(1, 0, 2)[None]  # [1][Hkv][L][D]
    v = torch_widen(case.v[c0:c1], case.dtype).permute(1, 0, 2)[None]
    o = torch.nn.functional.scaled_dot_product_attention(
        q, k.contiguous(), v.contiguous(), scale=case.scale, enable_gqa=True)
    return o[0, :, 0, :].numpy()


def brute_force(case, s):
    """Python floats, math.exp and math.fsum, over contiguous keys/values."""
    c0, c1 = int(case.cu_tokens[s]), int(case.cu_tokens[s + 1])
    q = numerics.to_f64(case.q[s], case.dtype).tolist()
    k = numerics.to_f64(case.k[c0:c1], case.dtype).tolist()
    v = numerics.to_f64(case.v[c0:c1], case.dtype).tolist()
    hq, hkv, D = case.num_q_heads, case.num_kv_heads, case.head_dim
    out = []
    for j in range(hq):
        h = j * hkv // hq
        z = [case.scale * math.fsum(q[j][d] * k[t][h][d] for d in range(D)) for t in range(c1 - c0)]
        m = max(z)
        w = [math.exp(x - m) for x in z]
        den = math.fsum(w)
        out.append([math.fsum(w[t] * v[t][h][d] for t in range(len(w))) / den for d in range(D)])
    return np.array(out)


# ------------------------------------------------------------------- checks
def err_contiguous(case, decode_fn=attention.decode, **pool_kw):
    kp, vp, tab = oracle_pools_for_decode(case, **pool_kw)
    got = decode_fn(case.q, kp, vp, tab, case.context_lens, case.scale, case.block_size, case.dtype)
    return max(np.abs(got[s] - dense_sdpa(case, s)).max() for s in range(case.num_seqs))


def err_brute(case, decode_fn=attention.decode):
    kp, vp, tab = oracle_pools_for_decode(case)
    got = decode_fn(case.q, kp, vp, tab, case.context_lens, case.scale, case.block_size, case.dtype)
    return max(np.abs(got[s] - brute_force(case, s)).max() for s in range(case.num_seqs))


def err_scale_closed_form(attend_fn=attention.attend):
    """Two keys, one channel: q=1, k0=0, k1=ln(3)/scale gives weights 1/4 and
    3/4, so out = v0/4 + 3 v1/4 exactly in real arithmetic."""
    scale = 0.125
    q = np.array([[1.0]])
    k = np.array([[[0.0]], [[math.log(3.0) / scale]]])
    v = np.array([[[2.0]], [[-6.0]]])
    return abs(attend_fn(q, k, v, scale)[0, 0] - (2.0 / 4 + 3 * -6.0 / 4))


def err_gqa_mapping(attend_fn=attention.attend, hq=8, hkv=2):
    """KV head h holds the constant value vector h+1, keys random: query head
    j must return exactly the value of its KV head, j // (hq // hkv), plus 1."""
    rng = np.random.default_rng(7)
    L, D = 9, 4
    k = rng.standard_normal((L, hkv, D))
    v = np.broadcast_to((np.arange(hkv) + 1.0)[None, :, None], (L, hkv, D)).copy()
    q = rng.standard_normal((hq, D))
    out = attend_fn(q, k, v, 0.5)
    want = (np.arange(hq) // (hq // hkv) + 1.0)[:, None]
    return np.abs(out - want).max()


def err_all_keys_equal(attend_fn=attention.attend):
    """All keys identical: every score is equal, so out = mean of V (fsum)."""
    rng = np.random.default_rng(11)
    L, hkv, hq, D = 37, 2, 4, 8
    k = np.broadcast_to(rng.standard_normal((1, hkv, D)), (L, hkv, D)).copy()
    v = rng.standard_normal((L, hkv, D))
    q = rng.standard_normal((hq, D)) * 5
    out = attend_fn(q, k, v, 0.3)
    want = np.array([[math.fsum(v[:, j // 2, d]) / L for d in range(D)] for j in range(hq)])
    return np.abs(out - want).max()


def err_single_token(attend_fn=attention.attend):
    """A context of one token returns that token's value vector exactly."""
    rng = np.random.default_rng(13)
    k = rng.standard_normal((1, 2, 8))
    v = rng.standard_normal((1, 2, 8))
    q = rng.standard_normal((4, 8)) * 100
    out = attend_fn(q, k, v, 1.0)
    return np.abs(out - v[0][np.arange(4) // 2]).max()


def err_partition_identity(case, s, partition_tokens, partials_fn=attention.partition_partials,
                           merge_fn=attention.lse_merge):
    c0, c1 = int(case.cu_tokens[s]), int(case.cu_tokens[s + 1])
    q = numerics.to_f64(case.q[s], case.dtype)
    k = numerics.to_f64(case.k[c0:c1], case.dtype)
    v = numerics.to_f64(case.v[c0:c1], case.dtype)
    o, m, l = partials_fn(q, k, v, case.scale, partition_tokens)
    return np.abs(merge_fn(o, m, l) - dense_sdpa(case, s)).max()


def extend_state(ecase, bm_cls=block_manager.RefBlockManager, append_fn=paging.append):
    """Pools after the prefixes and then the new tokens are placed, in the
    order a server would (all prefixes, then all new chunks)."""
    B = ecase.block_size
    bm = bm_cls(ecase.num_blocks, B, ecase.free_order)
    sids = []
    pslots = []
    for r, P in enumerate(ecase.prefix_lens):
        sid = bm.new_seq()
        sids.append(sid)
        s, _ = bm.append(sid, int(P))
        pslots += s
    nslots = []
    for r, n in enumerate(ecase.new_lens):
        s, _ = bm.append(sids[r], int(n))
        nslots += s
    kp, vp = paging.new_pools(ecase.num_blocks, ecase.num_kv_heads, ecase.head_dim, B, ecase.dtype)
    append_fn(kp, vp, ecase.prefix_k, ecase.prefix_v, np.asarray(pslots), B)
    append_fn(kp, vp, ecase.new_k, ecase.new_v, np.asarray(nslots), B)
    tables = [bm.table(s) for s in sids]
    tab = np.full((len(tables), max(map(len, tables))), -1, dtype=np.int64)
    for i, t in enumerate(tables):
        tab[i, :len(t)] = t
    return kp, vp, tab, np.asarray(pslots), np.asarray(nslots)


def err_extend_causal_closed_form(extend_fn=attention.extend):
    """All keys of a request equal: new token i (position P+i) must return
    the mean of the values at positions 0..P+i, an fsum closed form.  An
    off-by-one in the causal rule changes the set being averaged."""
    from workloads import extend_case
    e = extend_case(17, 2, 5, 20, 3, 9, 4, 2, 8, "fp32")
    # make every key of the pool identical before placing it
    one_k = e.prefix_k[:1].copy()
    e.prefix_k[:] = one_k
    e.new_k[:] = one_k
    kp, vp, tab, _, _ = extend_state(e)
    got = extend_fn(e.q, e.cu_new, e.seq_lens, kp, vp, tab, e.scale, e.block_size, e.dtype)
    err = 0.0
    for r in range(len(e.prefix_lens)):
        P = int(e.prefix_lens[r])
        vals = np.concatenate([numerics.to_f64(e.prefix_v[e.cu_prefix[r]:e.cu_prefix[r + 1]], "fp32"),
                               numerics.to_f64(e.new_v[e.cu_new[r]:e.cu_new[r + 1]], "fp32")])
        for i in range(int(e.new_lens[r])):
            for j in range(e.num_q_heads):
                h = j // (e.num_q_heads // e.num_kv_heads)
                want = [math.fsum(vals[:P + i + 1, h, d]) / (P + i + 1) for d in range(e.head_dim)]
                err = max(err, np.abs(got[e.cu_new[r] + i, j] - want).max())
    return err


def err_extend_vs_decode(ecase, extend_fn=attention.extend, decode_fn=attention.decode):
    """Extend row i equals decode with the context cut at P+i+1 (same pool)."""
    kp, vp, tab, _, _ = extend_state(ecase)
    ext = extend_fn(ecase.q, ecase.cu_new, ecase.seq_lens, kp, vp, tab, ecase.scale,
                    ecase.block_size, ecase.dtype)
    err = 0.0
    for r in range(len(ecase.prefix_lens)):
        P = int(ecase.prefix_lens[r])
        for i in range(int(ecase.new_lens[r])):
            row = int(ecase.cu_new[r]) + i
            dec = decode_fn(ecase.q[row:row + 1], kp, vp, tab[r:r + 1], np.array([P + i + 1]),
                            ecase.scale, ecase.block_size, ecase.dtype)
            err = max(err, np.abs(ext[row] - dec[0]).max())
    return err
