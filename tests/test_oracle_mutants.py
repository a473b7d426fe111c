"""Plant plausible mistakes in (copies of) the oracle and check that at least
one pin catches each of them.  Everything here runs on the CPU."""

import numpy as np
import pytest

import oracle_pins as P
from oracle import attention, block_manager, paging
from workloads import decode_case, extend_case, shared_prefix_case, tiny_fp32_decode


def _caught(fn, *a, tol=1e-9, **kw):
    try:
        return not (fn(*a, **kw) <= tol)    # NaN counts as caught
    except Exception:           # a crash is a caught mistake too
        return True


# ------------------------------------------------------------ attend mutants
def attend_gqa_modulo(q, k, v, scale):
    hq, d = q.shape
    hkv = k.shape[1]
    out = np.zeros((hq, d))
    for j in range(hq):
        h = j % hkv                                  # planted: wrong head mapping
        z = scale * (k[:, h, :] @ q[j])
        w = np.exp(z - z.max())
        out[j] = (w @ v[:, h, :]) / w.sum()
    return out


def attend_no_scale(q, k, v, scale):
    return attention.attend(q, k, v, 1.0)            # planted: scale dropped


def attend_neg_sign(q, k, v, scale):
    return attention.attend(q, k, v, -scale)         # planted: sign flip


def attend_no_normalise(q, k, v, scale):
    hq, d = q.shape
    g = hq // k.shape[1]
    out = np.zeros((hq, d))
    for j in range(hq):
        z = scale * (k[:, j // g, :] @ q[j])
        out[j] = np.exp(z - z.max()) @ v[:, j // g, :]   # planted: no division
    return out


def attend_uses_k_for_v(q, k, v, scale):
    return attention.attend(q, k, k, scale)          # planted: transposed operand


@pytest.mark.parametrize("mutant", [attend_gqa_modulo, attend_no_scale, attend_neg_sign,
                                    attend_no_normalise, attend_uses_k_for_v])
def test_attend_mutants_caught(mutant):
    checks = [P.err_gqa_mapping, P.err_scale_closed_form, P.err_all_keys_equal, P.err_single_token]
    assert any(_caught(c, attend_fn=mutant) for c in checks)

    def dec(*a, **kw):
        orig = attention.attend
        attention.attend = mutant
        try:
            return attention.decode(*a, **kw)
        finally:
            attention.attend = orig
    assert _caught(P.err_contiguous, decode_case(31, 4, 1, 90, 8, 2, 16, "bf16"), decode_fn=dec)


# --------------------------------------------------- gather / append mutants
def gather_off_by_one(k_pool, v_pool, table_row, L, B):
    k, v = paging.gather(k_pool, v_pool, table_row, L, B)
    k[1:] = k[:-1].copy()                             # planted: shifted positions
    return k, v


def gather_wrong_block(k_pool, v_pool, table_row, L, B):
    row = np.asarray(table_row).copy()
    row[:-1] = row[1:].copy()                         # planted: block i+1 for block i
    return paging.gather(k_pool, v_pool, row, L, B)


def append_swapped(k_pool, v_pool, k_new, v_new, slots, B):
    nb = k_pool.shape[0]
    sl = np.asarray(slots)
    # planted: block/offset decoded with the wrong divisor
    alt = (sl % B) * B + (sl // B) % B
    alt = np.where(alt // B < nb, alt, sl)
    paging.append(k_pool, v_pool, k_new, v_new, alt, B)


@pytest.mark.parametrize("mutant", [gather_off_by_one, gather_wrong_block])
def test_gather_mutants_caught(mutant, monkeypatch):
    monkeypatch.setattr(attention, "gather", mutant)
    monkeypatch.setattr(attention, "gather_fast", mutant)
    assert _caught(P.err_contiguous, decode_case(32, 4, 20, 90, 4, 2, 16, "fp32"))


def test_append_mutant_caught():
    assert _caught(P.err_contiguous, decode_case(33, 4, 20, 90, 4, 2, 16, "fp32"),
                   append_fn=append_swapped)


# ------------------------------------------------------------ extend mutants
def extend_strict_causal(q_words, cu, seq_lens, kp, vp, tabs, scale, B, dtype, **kw):
    # planted: a token does not see itself (uses seq_lens - 1 context)
    from oracle.numerics import to_f64
    q = to_f64(q_words, dtype)
    out = np.full(q.shape, np.nan)
    hq = q.shape[1]
    for r in range(len(seq_lens)):
        q0, q1 = int(cu[r]), int(cu[r + 1])
        n, L = q1 - q0, int(seq_lens[r])
        k, v = attention._gathered(kp, vp, tabs[r], L, B, dtype)
        g = hq // k.shape[1]
        vis = np.arange(L)[None, :] < (L - n + np.arange(n))[:, None]
        vis[:, 0] = True
        for j in range(hq):
            z = np.where(vis, scale * (q[q0:q1, j] @ k[:, j // g].T), -np.inf)
            w = np.exp(z - z.max(axis=1, keepdims=True))
            out[q0:q1, j] = (w @ v[:, j // g]) / w.sum(axis=1, keepdims=True)
    return out


def extend_no_mask(q_words, cu, seq_lens, kp, vp, tabs, scale, B, dtype, **kw):
    # planted: every new token sees the whole chunk
    from oracle.numerics import to_f64
    q = to_f64(q_words, dtype)
    out = np.full(q.shape, np.nan)
    for r in range(len(seq_lens)):
        q0, q1 = int(cu[r]), int(cu[r + 1])
        k, v = attention._gathered(kp, vp, tabs[r], int(seq_lens[r]), B, dtype)
        for i in range(q1 - q0):
            out[q0 + i] = attention.attend(q[q0 + i], k, v, scale)
    return out


@pytest.mark.parametrize("mutant", [extend_strict_causal, extend_no_mask])
def test_extend_mutants_caught(mutant):
    assert _caught(P.err_extend_causal_closed_form, extend_fn=mutant)
    e = extend_case(71, 3, 1, 60, 2, 40, 4, 2, 16, "fp32")
    assert _caught(P.err_extend_vs_decode, e, extend_fn=mutant)


# ------------------------------------------------------- split-KV mutants
def merge_without_l(o, m, l):
    M = m.max(axis=0)
    w = np.exp(m - M[None, :])                       # planted: l_p weight dropped
    return (o * w[:, :, None]).sum(axis=0) / w.sum(axis=0)[:, None]


def merge_wrong_sign(o, m, l):
    M = m.max(axis=0)
    w = l * np.exp(M[None, :] - m)                   # planted: exponent reversed
    return (o * w[:, :, None]).sum(axis=0) / w.sum(axis=0)[:, None]


@pytest.mark.parametrize("mutant", [merge_without_l, merge_wrong_sign])
def test_merge_mutants_caught(mutant):
    case = decode_case(61, 2, 900, 3000, 4, 2, 16, "bf16")
    assert _caught(P.err_partition_identity, case, 0, 512, merge_fn=mutant)


# ------------------------------------------------------ block-manager mutants
class NoCowManager(block_manager.RefBlockManager):
    """planted: writes into a shared partial block in place (no copy)."""

    def append(self, sid, n):
        B = self.block_size
        table = self.tables[sid]
        slots = []
        for _ in range(n):
            pos = self.lens[sid]
            if pos % B == 0:
                table.append(self._take())
            slots.append(table[pos // B] * B + pos % B)
            self.lens[sid] = pos + 1
        return slots, []


class LeakyFreeManager(block_manager.RefBlockManager):
    """planted: frees every block of a sequence regardless of its count."""

    def free_seq(self, sid):
        for b in self.tables.pop(sid):
            self.ref.pop(b, None)
            self.free.append(b)
        del self.lens[sid]


def _cow_scenario(bm_cls):
    bm = bm_cls(10, 4, list(range(10)))
    a = bm.new_seq()
    bm.append(a, 6)
    b = bm.fork(a)
    _, pairs = bm.append(b, 1)
    return pairs == [(1, 2)] and bm.table(b) == [0, 2] and bm.table(a) == [0, 1]


def _free_scenario(bm_cls):
    bm = bm_cls(10, 4, list(range(10)))
    a = bm.new_seq()
    bm.append(a, 6)
    b = bm.fork(a)
    bm.free_seq(a)
    return 0 not in bm.free and 1 not in bm.free and bm.table(b) == [0, 1]


def test_block_manager_scenarios_hold():
    assert _cow_scenario(block_manager.RefBlockManager)
    assert _free_scenario(block_manager.RefBlockManager)


def test_block_manager_mutants_caught():
    assert not _cow_scenario(NoCowManager)
    assert not _free_scenario(LeakyFreeManager)


def test_brute_force_catches_scale_mutant():
    case = tiny_fp32_decode()

    def dec(*a, **kw):
        orig = attention.attend
        attention.attend = attend_no_scale
        try:
            return attention.decode(*a, **kw)
        finally:
            attention.attend = orig
    assert _caught(P.err_brute, case, decode_fn=dec)


def _fork_and_write_both(bm_cls):
    """Parent with a partly filled last block forks; the child and then the
    parent each write one new token.  Returns True when both see their own
    token (the pages: other references stay valid after a write)."""
    case = shared_prefix_case(82, 3, 32, 3, 40, 1, 2, 4, 2, 16, "fp32")
    bm = bm_cls(case.num_blocks, 16, case.free_order)
    kp, vp = paging.new_pools(case.num_blocks, 2, 16, 16, "fp32")
    root = bm.new_seq()
    n0 = 32 + int(case.suffix_lens[0])
    assert n0 % 16 != 0
    s, _ = bm.append(root, n0)
    k = np.concatenate([case.prefix_k, case.suffix_k[:case.suffix_lens[0]]])
    v = np.concatenate([case.prefix_v, case.suffix_v[:case.suffix_lens[0]]])
    paging.append(kp, vp, k, v, np.asarray(s), 16)
    child = bm.fork(root)
    for i, sid in enumerate((child, root)):
        sl, pairs = bm.append(sid, 1)
        paging.copy_blocks(kp, vp, np.asarray(pairs).reshape(-1, 2))
        paging.append(kp, vp, case.new_k[i:i + 1], case.new_v[i:i + 1], np.asarray(sl), 16)
    kc, _ = paging.gather(kp, vp, bm.table(child), bm.lens[child], 16)
    kr, _ = paging.gather(kp, vp, bm.table(root), bm.lens[root], 16)
    return (np.array_equal(kc[-1], case.new_k[0]) and np.array_equal(kr[-1], case.new_k[1])
            and np.array_equal(kc[:-1], k) and np.array_equal(kr[:-1], k))


def test_fork_write_both_scenario():
    assert _fork_and_write_both(block_manager.RefBlockManager)
    assert not _fork_and_write_both(NoCowManager)
