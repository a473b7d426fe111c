"""The loops that bench.py times compute what the oracle computes.

After a few timed steps of the GQA-4 workload at full size (64 sequences,
~150K context tokens), through the same function the benchmark times (host
allocator step, upload of the index arrays and the changed table entries
fused with the append, decode): the device-resident tables equal the host
block manager's;
the last step's output rows for sampled sequences match the oracle's decode
over the pool the loop left behind, and the last step's new keys and values
sit in their slots bit for bit.  Tolerance as for every bf16 decode: 2e-2
max-abs."""

import argparse

import numpy as np
import pytest
import torch

import bench
from gpu_helpers import f64_of, words_of
from oracle import attention, paging
from paged_kv_cache_63_amd import BlockAllocator, _lib

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("bs", [16, 32])
def test_decode_loop_output_and_appends(gpu, bs):
    args = argparse.Namespace(warmup=2, steps=3, partition_size=0, event_every=1, flush_iters=2,
                              keep_state=True, block_size=bs)
    case = bench.make_case("gqa4-decode", args.warmup + args.steps)
    r = bench.run_decode(args, case, torch, _lib, BlockAllocator)
    st = r["state"]
    torch.cuda.synchronize()
    assert len(r["durs"]) == args.steps and all(d > 0 for d in r["durs"])
    assert len(r["flush_durs"]) == 2 and min(r["flush_durs"]) > 0
    # the device-resident tables, kept current by per-step last-entry
    # updates, equal the host block manager's, bit for bit
    assert np.array_equal(st["tables_dev"], st["tables"])
    kp, vp = words_of(st["k_pool"]), words_of(st["v_pool"])
    lens = st["lens"]
    tables = [row[:-(-int(L) // bs)].tolist() for row, L in zip(st["tables"], lens)]
    seqs = [0, 17, 40, 63]
    want = attention.decode(words_of(st["q"]), kp, vp, tables, lens, case.scale, bs, "bf16",
                            seqs=seqs)
    got = f64_of(st["out"])
    assert np.abs(got[seqs] - want[seqs]).max() <= 2e-2
    kn, vn = words_of(st["k_new"]), words_of(st["v_new"])
    for s in range(case.num_seqs):
        p = int(lens[s]) - 1                      # the last step's token
        blk, off = tables[s][p // bs], p % bs
        assert np.array_equal(kp[blk, :, off, :], kn[s])
        assert np.array_equal(paging.v_halves(vp)[blk, :, off // 16, :, paging.v_pos(off % 16)],
                              vn[s])


def test_extend_loop_output(gpu):
    """The multi-turn extend loop (16 requests, 2K-8K cached tokens + 512 new
    each): the last step's output for 2 requests x 2 query heads against the
    oracle over the pool and tables that step used."""
    args = argparse.Namespace(warmup=1, steps=2, keep_state=True, flush_iters=2)
    e = bench.make_case("multiturn-extend", args.warmup + args.steps)
    r = bench.run_extend(args, e, torch, _lib, BlockAllocator)
    st = r["state"]
    torch.cuda.synchronize()
    kp, vp = words_of(st["k_pool"]), words_of(st["v_pool"])
    tables = [row[:-(-int(L) // 16)].tolist() for row, L in zip(st["tables"], e.seq_lens)]
    reqs, heads = [int(np.argmax(e.prefix_lens)), 3], [0, 29]
    want = attention.extend(e.q, e.cu_new, e.seq_lens, kp, vp, tables, e.scale, 16, "bf16",
                            reqs=reqs, heads=heads)
    got = f64_of(st["out"])
    for q in reqs:
        a, b = int(e.cu_new[q]), int(e.cu_new[q + 1])
        assert np.abs(got[a:b][:, heads] - want[a:b][:, heads]).max() <= 2e-2, q
