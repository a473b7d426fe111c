"""Decode attention (pass 1 + pass 2) against the oracle.

Tolerances (max-abs over every output element): 1e-5 for fp32 inputs,
2e-2 for bf16 inputs with fp32 accumulation."""

import numpy as np
import pytest
import torch

import oracle_pins as P
from gpu_helpers import LibDecodeState, f64_of, i32, words_of
from oracle import attention, numerics, paging
from workloads import decode_case, gqa4_decode, long_context_decode, tiny_fp32_decode

pytestmark = pytest.mark.gpu

TOL = {"fp32": 1e-5, "bf16": 2e-2}


def _oracle_out(case, seqs=None):
    kp, vp, tab = P.oracle_pools_for_decode(case)
    return attention.decode(case.q, kp, vp, tab, case.context_lens, case.scale, 16, case.dtype,
                            seqs=seqs)


def test_tiny_fp32(gpu):
    """4 sequences (5/17/33/64 tokens), 4 heads, head_dim 64, fp32, NaN in
    every unused block and tail slot."""
    case = tiny_fp32_decode()
    st = LibDecodeState(case)
    out, _ = st.decode()
    err = np.abs(f64_of(out) - _oracle_out(case)).max()
    assert err <= 1e-5, err


@pytest.mark.parametrize("dtype,hq,hkv,d,ptok", [
    ("bf16", 32, 8, 128, 0), ("bf16", 32, 8, 128, 64), ("bf16", 32, 8, 128, 16),
    ("bf16", 8, 8, 128, 128), ("bf16", 64, 8, 128, 256), ("bf16", 16, 1, 64, 32),
    ("bf16", 4, 2, 64, 0), ("fp32", 8, 2, 128, 64), ("fp32", 16, 1, 64, 0),
    ("fp32", 4, 4, 64, 16),
])
def test_small_cases(gpu, dtype, hq, hkv, d, ptok):
    """Ragged contexts 1..700 spanning one to many partitions and blocks."""
    case = decode_case(200 + hq + d + ptok, 9, 1, 700, hq, hkv, d, dtype)
    st = LibDecodeState(case)
    out, _ = st.decode(partition_size=ptok)
    err = np.abs(f64_of(out) - _oracle_out(case)).max()
    assert err <= TOL[dtype], err


def test_gqa4_full_size(gpu):
    """Llama-3-8B shape, 64 sequences of 512..4096 tokens, every output."""
    case = gqa4_decode()
    st = LibDecodeState(case)
    out, _ = st.decode()
    err = np.abs(f64_of(out) - _oracle_out(case)).max()
    assert err <= 2e-2, err


def test_long_context_full_size_sampled(gpu):
    """Llama-3.1-70B shape, 8 sequences of 32K..128K tokens, 512-token
    partitions; the oracle checks two sequences x two KV heads (all their
    query heads) and, for every sequence, the all-heads output is finite."""
    case = long_context_decode()
    st = LibDecodeState(case)
    out, _ = st.decode(partition_size=512)
    got = f64_of(out)
    assert np.isfinite(got).all()
    kp, vp, tab = P.oracle_pools_for_decode(case)
    g = case.num_q_heads // case.num_kv_heads
    q = numerics.to_f64(case.q, "bf16")
    for s in (int(np.argmax(case.context_lens)), int(np.argmin(case.context_lens))):
        L = int(case.context_lens[s])
        kw, vw = paging.gather_fast(kp, vp, tab[s], L, 16)
        for h in (0, case.num_kv_heads - 1):
            k = numerics.to_f64(kw[:, h:h + 1], "bf16")
            v = numerics.to_f64(vw[:, h:h + 1], "bf16")
            want = attention.attend(q[s, h * g:(h + 1) * g], k, v, case.scale)
            err = np.abs(got[s, h * g:(h + 1) * g] - want).max()
            assert err <= 2e-2, (s, h, err)


def test_partials_match_oracle_partitions(gpu):
    """Pass-1 workspace: each partition's (o_p, m_p, l_p) against the
    oracle's split-KV pieces."""
    case = decode_case(301, 3, 700, 1500, 16, 4, 128, "bf16")
    st = LibDecodeState(case)
    ptok = 256
    out, ws = st.decode(partition_size=ptok)
    torch.cuda.synchronize()
    S, hq, d = case.num_seqs, case.num_q_heads, case.head_dim
    Pm = -(-int(max(case.context_lens)) // ptok)
    w = ws.view(torch.float32).cpu().numpy().astype(np.float64)
    rows = S * hq * Pm
    o = w[:rows * d].reshape(S, hq, Pm, d)
    m = w[rows * d:rows * (d + 1)].reshape(S, hq, Pm)
    l = w[rows * (d + 1):rows * (d + 2)].reshape(S, hq, Pm)
    for s in range(S):
        c0, c1 = case.cu_tokens[s], case.cu_tokens[s + 1]
        oo, mm, ll = attention.partition_partials(numerics.to_f64(case.q[s], "bf16"),
                                                  numerics.to_f64(case.k[c0:c1], "bf16"),
                                                  numerics.to_f64(case.v[c0:c1], "bf16"),
                                                  case.scale, ptok)
        n = oo.shape[0]
        assert np.abs(o[s, :, :n].transpose(1, 0, 2) - oo).max() <= 2e-2
        assert np.abs(m[s, :, :n].T - mm).max() <= 2e-2
        assert (np.abs(l[s, :, :n].T - ll) / ll).max() <= 2e-2


def test_permutation_bit_identical(gpu):
    """Same logical contents placed by a second permutation of the pool:
    the GPU output bits do not change."""
    case = decode_case(401, 16, 1, 3000, 32, 8, 128, "bf16", spare_blocks=50)
    a = LibDecodeState(case)
    other = np.random.default_rng(501).permutation(case.num_blocks)
    b = LibDecodeState(case, free_order=other)
    assert not torch.equal(a.tables, b.tables)
    for ptok in (0, 64):
        oa, _ = a.decode(partition_size=ptok)
        ob, _ = b.decode(partition_size=ptok)
        assert np.array_equal(words_of(oa), words_of(ob))


def test_all_keys_equal_is_mean_of_values(gpu):
    """All keys identical -> every head returns the mean of its values."""
    case = decode_case(411, 5, 10, 900, 8, 2, 128, "bf16")
    case.k[:] = case.k[:1]
    st = LibDecodeState(case)
    out, _ = st.decode(partition_size=128)
    got = f64_of(out)
    for s in range(case.num_seqs):
        c0, c1 = case.cu_tokens[s], case.cu_tokens[s + 1]
        mean = numerics.to_f64(case.v[c0:c1], "bf16").mean(axis=0)   # [Hkv][D]
        want = np.repeat(mean, 4, axis=0)
        assert np.abs(got[s] - want).max() <= 2e-2


def test_empty_and_single_token_contexts(gpu):
    case = decode_case(421, 4, 0, 0, 8, 2, 128, "bf16", lens=[1, 0, 16, 17], num_blocks=8)
    st = LibDecodeState(case)
    out, _ = st.decode(partition_size=16, max_context_len=64)
    got = f64_of(out)
    assert np.array_equal(got[1], np.zeros_like(got[1]))
    v0 = numerics.to_f64(case.v[0], "bf16")                            # [Hkv][D]
    assert np.abs(got[0] - np.repeat(v0, 4, axis=0)).max() <= 4e-3
    err = np.abs(got[[0, 2, 3]] - _oracle_out(case)[[0, 2, 3]]).max()
    assert err <= 2e-2


def test_context_longer_than_declared_max_is_cut_not_overrun(gpu):
    """A context above max_context_len is cut to it (memory-safe); the
    result equals the decode of the cut context."""
    case = decode_case(431, 2, 300, 300, 4, 1, 64, "bf16")
    st = LibDecodeState(case)
    out, _ = st.decode(partition_size=64, max_context_len=128)
    cut = decode_case(431, 2, 300, 300, 4, 1, 64, "bf16")
    kp, vp, tab = P.oracle_pools_for_decode(cut)
    want = attention.decode(cut.q, kp, vp, tab, np.array([128, 128]), cut.scale, 16, "bf16")
    assert np.abs(f64_of(out) - want).max() <= 2e-2
