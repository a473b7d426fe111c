"""paged_attention_decode_noalloc (the decode entry whose workspace is the
library's fixed per-GPU array) against paged_attention_decode with a
caller's workspace, through the C ABI: two calls in a row, the second with a
smaller input, then a call whose partials exceed the fixed array, which is
refused before any device work."""

import ctypes

import numpy as np
import pytest
import torch

import oracle_pins as P
from gpu_helpers import LibDecodeState, f64_of, words_of
from oracle import attention
from paged_kv_cache_63_amd import _lib
from workloads import decode_case

pytestmark = pytest.mark.gpu


def _both(case, ptok):
    st = LibDecodeState(case)
    want_ws, _ = st.decode(partition_size=ptok)
    out = torch.full_like(st.q, float("nan"))
    _lib.paged_attention_decode_noalloc(out, st.q, st.k_pool, st.v_pool, st.tables, st.lens,
                                        int(max(case.context_lens)), case.scale, ptok)
    torch.cuda.synchronize()
    kp, vp, tab = P.oracle_pools_for_decode(case)
    want = attention.decode(case.q, kp, vp, tab, case.context_lens, case.scale, case.block_size,
                            case.dtype)
    return out, want_ws, want


def test_noalloc_matches_workspace_entry_twice(gpu):
    tol = {"bf16": 2e-2, "fp32": 1e-5}
    # a larger call, then smaller ones: each reuses the array the one before
    # left behind (other offsets, stale pieces and piece-count words); the
    # last at 32-token blocks
    for case, ptok in [(decode_case(951, 24, 1, 3000, 32, 8, 128, "bf16"), 0),
                       (decode_case(952, 5, 1, 700, 32, 8, 128, "bf16"), 64),
                       (decode_case(953, 3, 1, 300, 8, 2, 64, "fp32"), 32),
                       (decode_case(955, 4, 1, 900, 16, 2, 128, "bf16", block_size=32), 64)]:
        out, ref, want = _both(case, ptok)
        assert np.array_equal(words_of(out), words_of(ref))
        err = np.abs(f64_of(out) - want).max()
        assert err <= tol[case.dtype], err


def test_noalloc_refuses_calls_beyond_its_array(gpu):
    case = decode_case(954, 8, 1, 40, 8, 8, 128, "bf16")
    st = LibDecodeState(case)
    out = torch.full_like(st.q, float("nan"))
    lib = _lib.load()
    # a 32768-token bound over 16-token pieces: 2,049 pieces per context, so
    # 8 x 8 x 2049 x 130 x 4 bytes of partials, over the 64 MiB array
    rc = lib.paged_attention_decode_noalloc(
        _lib._ptr(out), _lib._ptr(st.q), _lib._ptr(st.k_pool), _lib._ptr(st.v_pool),
        case.num_blocks, _lib._ptr(st.tables), st.tables.shape[1], _lib._ptr(st.lens),
        case.num_seqs, 32768, 8, 8, 128, 16, ctypes.c_float(case.scale), 16, 1,
        _lib._stream())
    assert rc == -3
    assert b"fixed workspace" in lib.paged_kv_last_error()
    torch.cuda.synchronize()
    assert torch.isnan(out.float()).all()
