"""Exact softmax attention over paged K/V, in float64 (oracle).

TEST INFRASTRUCTURE ONLY -- see the package docstring.

Paging changes where keys and values live, never what attention computes
("PagedAttention and RadixAttention: Let's Talk About KV Cache", end of section
"PagedAttention: Memory Like an Operating System"; The Daily Triptych, "Paged
Attention for Efficient Memory Management", technical summary).  So the oracle
is the plain definition: gather the sequence's keys and values through its
block table, then

    z_t   = scale * <q_j, k_t[h(j)]>
    w_t   = exp(z_t - max_t z_t)
    out_j = sum_t w_t v_t[h(j)] / sum_t w_t

Grouped-query attention (named, without a head mapping, in "RadixAttention:
Tree-Based KV Cache Reuse in SGLang Guide", section "3. Integrating FlashInfer
..."): query heads are split into ``num_kv_heads`` runs of
``g = num_q_heads // num_kv_heads`` consecutive heads and run ``h`` reads KV
head ``h``, i.e. ``h(j) = j // g``.

A context of length 0 yields an all-zero output row.
"""

import numpy as np

from .numerics import to_f64
from .paging import gather, gather_fast


def attend(q, k, v, scale: float):
    """Attention of one query token.

    q: ``[Hq][D]`` float64; k, v: ``[L][Hkv][D]`` float64.  Returns ``[Hq][D]``.
    """
    hq, d = q.shape
    L, hkv, _ = k.shape
    out = np.zeros((hq, d), dtype=np.float64)
    if L == 0:
        return out
    g = hq // hkv
    for j in range(hq):
        h = j // g
        z = scale * (k[:, h, :] @ q[j])
        w = np.exp(z - z.max())
        out[j] = (w @ v[:, h, :]) / w.sum()
    return out


def _gathered(k_pool, v_pool, table_row, L, block_size, dtype):
    gfun = gather_fast if L > 4096 else gather
    kw, vw = gfun(k_pool, v_pool, table_row, L, block_size)
    return to_f64(kw, dtype), to_f64(vw, dtype)


def decode(q_words, k_pool, v_pool, block_tables, context_lens, scale: float,
           block_size: int, dtype: str, seqs=None):
    """Decode attention: one query token per sequence over its whole context.

    q_words: ``[S][Hq][D]`` raw words.  Returns ``[S][Hq][D]`` float64 (rows of
    sequences not listed in ``seqs`` are left as NaN).
    The context includes the token being decoded: its key and value were
    appended into the pool before attention runs (Triptych page, "The story").
    """
    q = to_f64(q_words, dtype)
    S = q.shape[0]
    out = np.full(q.shape, np.nan, dtype=np.float64)
    for s in (range(S) if seqs is None else seqs):
        L = int(context_lens[s])
        k, v = _gathered(k_pool, v_pool, block_tables[s], L, block_size, dtype)
        out[s] = attend(q[s], k, v, scale)
    return out


def partition_partials(q_row, k, v, scale: float, partition_tokens: int):
    """Split-KV pieces of one sequence: for every partition p of
    ``partition_tokens`` consecutive context tokens, the attention of the
    query over that partition alone plus its softmax statistics.

    Split-KV decode ("RadixAttention: Tree-Based KV Cache Reuse in SGLang
    Guide", section "3. Integrating FlashInfer ...") divides the work along the
    sequence; this is what each piece holds:

        m_p = max_{t in p} z_t
        l_p = sum_{t in p} exp(z_t - m_p)
        o_p = sum_{t in p} exp(z_t - m_p) v_t / l_p

    Returns ``(o [P][Hq][D], m [P][Hq], l [P][Hq])``, float64.
    """
    hq, d = q_row.shape
    L, hkv, _ = k.shape
    g = hq // hkv
    P = -(-L // partition_tokens)
    o = np.zeros((P, hq, d))
    m = np.zeros((P, hq))
    l = np.zeros((P, hq))
    for p in range(P):
        lo, hi = p * partition_tokens, min(L, (p + 1) * partition_tokens)
        for j in range(hq):
            h = j // g
            z = scale * (k[lo:hi, h, :] @ q_row[j])
            m[p, j] = z.max()
            w = np.exp(z - m[p, j])
            l[p, j] = w.sum()
            o[p, j] = (w @ v[lo:hi, h, :]) / l[p, j]
    return o, m, l


def lse_merge(o, m, l):
    """Recombine split-KV pieces (standard log-sum-exp identity):

        M   = max_p m_p
        out = sum_p o_p l_p exp(m_p - M) / sum_p l_p exp(m_p - M)

    o: ``[P][Hq][D]``; m, l: ``[P][Hq]``.  Returns ``[Hq][D]``.
    """
    M = m.max(axis=0)
    wgt = l * np.exp(m - M[None, :])
    return (o * wgt[:, :, None]).sum(axis=0) / wgt.sum(axis=0)[:, None]


def extend(q_words, cu_seqlens_q, seq_lens, k_pool, v_pool, block_tables,
           scale: float, block_size: int, dtype: str, reqs=None, heads=None):
    """Extend (chunked prefill over a cached prefix).

    Request r has ``n_r = cu[r+1] - cu[r]`` new tokens whose keys and values
    are already in the pool, after a prefix of ``P_r = seq_lens[r] - n_r``
    cached tokens.  New token i sits at position ``P_r + i`` and attends to
    positions ``0 .. P_r + i`` inclusive: the reused prefix plus the new
    tokens up to itself ("RadixAttention: Tree-Based KV Cache Reuse in SGLang
    Guide", "RadixAttention Architecture", steps of the longest-prefix search:
    only the unmatched suffix is prefilled over the reused pages).

    A request with no new token owns no row of the output, whatever its
    prefix, so it is passed over.

    q_words: ``[Tq][Hq][D]`` raw words.  Returns ``[Tq][Hq][D]`` float64
    (rows outside ``reqs``/``heads`` are NaN).
    """
    q = to_f64(q_words, dtype)
    hq = q.shape[1]
    R = len(seq_lens)
    out = np.full(q.shape, np.nan, dtype=np.float64)
    for r in (range(R) if reqs is None else reqs):
        q0, q1 = int(cu_seqlens_q[r]), int(cu_seqlens_q[r + 1])
        n = q1 - q0
        if n == 0:
            continue                                        # no new token, no output row
        L = int(seq_lens[r])
        prefix = L - n
        k, v = _gathered(k_pool, v_pool, block_tables[r], L, block_size, dtype)
        hkv = k.shape[1]
        g = hq // hkv
        pos_q = prefix + np.arange(n)                       # absolute positions
        visible = np.arange(L)[None, :] <= pos_q[:, None]   # [n][L] causal rule
        for j in (range(hq) if heads is None else heads):
            h = j // g
            z = scale * (q[q0:q1, j, :] @ k[:, h, :].T)     # [n][L]
            z = np.where(visible, z, -np.inf)
            w = np.exp(z - z.max(axis=1, keepdims=True))
            out[q0:q1, j, :] = (w @ v[:, h, :]) / w.sum(axis=1, keepdims=True)
    return out
