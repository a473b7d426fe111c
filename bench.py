#!/usr/bin/env python3
"""Throughput of the paged KV-cache hot path on one MI355X.

Default workload (the headline): decode steps at the Llama-3-8B attention
shape -- 64 sequences, contexts drawn uniformly from [512, 4096] tokens,
32 query heads over 8 KV heads, head_dim 128, bf16, 16-token blocks scattered
through one pool.  One step is the whole path for one new token per
sequence:

  host   block manager appends a token to every sequence (slots, new blocks,
         copy-on-write pairs, block tables)
  device copy_blocks (when the step produced copy-on-write pairs)
         upload_and_append_tables: the step's slots, lengths and each
           sequence's last table entry (the only one a decode step can
           change) read from pinned host memory into the device-resident
           tables, and the new token's K/V written into its slot, one launch
         paged_attention_decode (pass 1 + the log-sum-exp merge)

Contexts grow by one token per step, as in a real decode loop.  All inputs
(queries and new K/V of every step, the populated pool) are in device memory
before the timed region.  Prints one JSON line.

Other workloads (``--workload``) exist for measurement, not as the headline:
long-context-decode (8 x 32K..128K tokens, 64/8 heads), shared-prefix-decode
(256 + 12 forked sequences behind a 4096-token prompt) and multiturn-extend
(16 requests x (2K..8K cached + 512 new), bf16 matrix cores).
"""

import argparse
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 matrix-core peak
METRIC = "paged decode HBM GB/s (% of peak) and tokens/s at Llama-3-8B GQA shape"

WORKLOADS = ("gqa4-decode", "long-context-decode", "shared-prefix-decode", "multiturn-extend",
             "swap-host", "prefix-cache-host")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", choices=WORKLOADS, default="gqa4-decode")
    ap.add_argument("--event-every", type=int, default=5,
                    help="decode workloads: time the decode call with HIP events on every n-th "
                         "timed step (1 = every step)")
    ap.add_argument("--partition-size", type=int, default=0)
    ap.add_argument("--block-size", type=int, choices=(16, 32), default=16,
                    help="tokens per block of the plain decode workloads (gqa4-decode, "
                         "long-context-decode); the others use 16")
    ap.add_argument("--plain-decode", action="store_true",
                    help="shared-prefix workload: decode every sequence on its own "
                         "(paged_attention_decode) instead of the shared-prefix decode")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-probe", action="store_true",
                    help="run one 1 GiB device copy first (counter calibration)")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the device-copy bandwidth ceiling measurement")
    ap.add_argument("--flush-iters", type=int, default=50,
                    help="separate timing pass: this many calls of the dominant kernel on the "
                         "last step's inputs, each after a 1 GiB scratch write that evicts the "
                         "L2 and MALL caches, each bracketed by HIP events (0 = skip)")
    return ap.parse_args()


# ---------------------------------------------------------------- workloads
def make_case(name, total_steps):
    import workloads as W
    if name in ("gqa4-decode", "swap-host"):
        return W.gqa4_decode(spare_blocks=64 * (total_steps // 16 + 2))
    if name == "long-context-decode":
        # the long-context workload's draws (seed 3), with room for the decode steps
        return W.decode_case(3, 8, 32768, 131072, 64, 8, 128, "bf16",
                             spare_blocks=8 * (total_steps // 16 + 2),
                             name="long-context-decode-8x32K-128K")
    if name == "shared-prefix-decode":
        return W.shared_prefix_decode()
    return W.multiturn_extend()


# ------------------------------------------------------------- cpu baseline
_CPU = {}


def _cpu_worker(seqs):
    from threadpoolctl import threadpool_limits
    from oracle import attention
    c = _CPU
    with threadpool_limits(1):
        o = attention.decode(c["q"], c["kp"], c["vp"], c["tab"], c["lens"], c["scale"], 16, "bf16",
                             seqs=seqs)
    return seqs, o[seqs]


def cpu_baseline(case, seconds):
    """The oracle (numpy float64) on the same decode workload, one process per
    host core, one BLAS thread each, each taking whole sequences.  Runs before
    the GPU is touched (the pool of workers is forked).  Returns the JSON
    fields and the oracle's output rows of the workload's initial state (the
    first pass), against which the GPU's decode of that state is checked."""
    import multiprocessing as mp

    from oracle import block_manager, paging
    bm = block_manager.RefBlockManager(case.num_blocks, 16, case.free_order)
    kp, vp = paging.new_pools(case.num_blocks, case.num_kv_heads, case.head_dim, 16, case.dtype)
    tabs = []
    for s, L in enumerate(case.context_lens):
        sid = bm.new_seq()
        sl, _ = bm.append(sid, int(L))
        a, b = case.cu_tokens[s], case.cu_tokens[s + 1]
        paging.append(kp, vp, case.k[a:b], case.v[a:b], np.asarray(sl), 16)
        tabs.append(bm.table(sid))
    tab = np.full((len(tabs), max(map(len, tabs))), -1, dtype=np.int64)
    for i, t in enumerate(tabs):
        tab[i, :len(t)] = t
    _CPU.update(q=case.q, kp=kp, vp=vp, tab=tab, lens=case.context_lens, scale=case.scale)
    # one worker per core this process may run on, at most 16: the host share
    # a single GPU's job gets on the measurement machines, whatever the
    # affinity mask shows
    affinity = len(os.sched_getaffinity(0))
    cores = max(1, min(16, affinity))
    S = case.num_seqs
    chunks = [list(range(i, S, cores)) for i in range(cores)]
    ctx = mp.get_context("fork")
    ref = np.full((S, case.num_q_heads, case.head_dim), np.nan)
    with ctx.Pool(cores) as pool:
        t0 = time.perf_counter()
        steps = 0
        while True:
            rows = pool.map(_cpu_worker, chunks)
            if steps == 0:
                for seqs, o in rows:
                    ref[seqs] = o
            steps += 1
            el = time.perf_counter() - t0
            if el >= seconds or el / steps * (steps + 1) > 2.5 * seconds:
                break
    _CPU.clear()
    tok_s = steps * S / el
    kv_bytes = float(np.sum(case.context_lens)) * 2 * case.num_kv_heads * case.head_dim * 2
    return {"value": round(tok_s, 3), "unit": "tokens/s", "cores": cores,
            "affinity_cores": affinity, "kind": "oracle",
            "sample": f"{steps} full decode step(s) of the same workload ({S} sequences x "
                      f"{case.num_q_heads} heads, {int(np.sum(case.context_lens))} context "
                      f"tokens), {el:.1f} s on {cores} processes x 1 BLAS thread",
            "gbps": round(steps * kv_bytes / el / 1e9, 4)}, ref


# ------------------------------------------------------------------ traffic
def kernel_hash(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "paged_kv_cache_63_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(workload, files):
    """HBM bytes per launch measured by rocprofv3 counters (profiles/*.json),
    or None when no measurement exists for the current kernel source."""
    hsh = kernel_hash(files)
    for p in sorted(glob.glob(os.path.join(ROOT, "profiles", "*traffic*.json"))):
        try:
            with open(p) as f:
                d = json.load(f)
        except (OSError, ValueError):
            continue
        if d.get("workload") == workload and d.get("kernel_source_hash") == hsh:
            return d.get("hbm_bytes_per_launch"), d
    return None, None


# ---------------------------------------------------------------- GPU steps
def flushed_times(torch, call, iters):
    """Durations in seconds of ``call()`` (kernels on torch's current stream,
    the stream the library launches on), each call preceded by a 1 GiB
    scratch write that evicts the L2 caches and the MALL, and bracketed by
    HIP events on that stream (the write is outside the events)."""
    if iters <= 0:
        return []
    scratch = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    pairs = []
    for i in range(iters):
        scratch.fill_(i & 0xff)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        call()
        e1.record()
        pairs.append((e0, e1))
    torch.cuda.synchronize()
    del scratch
    return [a.elapsed_time(b) * 1e-3 for a, b in pairs]


def bandwidth_ceilings(torch, lib, iters=10):
    """Measured HBM ceilings, GB/s, each the median of ``iters`` calls with
    the caches flushed before each: the library's read probe over a 2 GiB
    buffer in a random order of 4 KB chunks (the scatter a paged pool's
    (block, KV head) slabs have) and in address order, and a 2 GiB
    device-to-device copy (torch copy_; read + written bytes)."""
    n = 2 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    order = torch.from_numpy(np.random.default_rng(0).permutation(n // 4096).astype(np.int32)).cuda()
    sink = torch.zeros(8 * torch.cuda.get_device_properties(0).multi_processor_count,
                       dtype=torch.int32, device="cuda")
    rnd = flushed_times(torch, lambda: lib.hbm_read_probe(a, 4096, order, sink), iters)
    seq = flushed_times(torch, lambda: lib.hbm_read_probe(a, 4096, None, sink), iters)
    b = torch.empty_like(a)
    cpy = flushed_times(torch, lambda: b.copy_(a), iters)
    del a, b
    return {"read_random_4k_gbps": round(n / float(np.median(rnd)) / 1e9, 1),
            "read_sequential_gbps": round(n / float(np.median(seq)) / 1e9, 1),
            "copy_gbps": round(2 * n / float(np.median(cpy)) / 1e9, 1)}


def run_decode(args, case, torch, lib, alloc_cls, ref=None):
    """Decode loop over a plain (unshared) decode case.  With ``ref`` (the
    oracle's output rows for the initial state), the GPU's decode of that
    state is compared with it first (max-abs error, every output)."""
    dev = torch.device("cuda:0")
    S, hq, hkv, d = case.num_seqs, case.num_q_heads, case.num_kv_heads, case.head_dim
    T = args.warmup + args.steps
    B = args.block_size
    # (the case's pool is sized for 16-token blocks: as many 32-token blocks
    # hold at least the same tokens)
    maxb = -(-(int(case.context_lens.max()) + T + 1) // B)
    alloc = alloc_cls(case.num_blocks, B, max_seqs=S, max_blocks_per_seq=maxb,
                      free_order=case.free_order)
    sids = [alloc.new_seq() for _ in range(S)]
    slots = np.concatenate([alloc.append_tokens(s, int(L))[0] for s, L in zip(sids, case.context_lens)])

    def dev_words(w):
        return torch.from_numpy(np.ascontiguousarray(w).view(np.int16)).view(torch.bfloat16).to(dev)

    k_pool, v_pool = lib.new_pools(case.num_blocks, hkv, d, B, torch.bfloat16, dev)
    lib.paged_kv_append(dev_words(case.k), dev_words(case.v),
                        torch.from_numpy(slots).to(dev), k_pool, v_pool)
    import workloads as W
    rng = np.random.default_rng(1000 + S)
    q_steps = dev_words(W.normal_words(rng, (T, S, hq, d), "bf16"))
    k_steps = dev_words(W.normal_words(rng, (T, S, hkv, d), "bf16"))
    v_steps = dev_words(W.normal_words(rng, (T, S, hkv, d), "bf16"))
    out = torch.empty((S, hq, d), dtype=torch.bfloat16, device=dev)
    ws_bytes = lib.paged_attention_decode_workspace_size(S, hq, hkv, d, maxb * B,
                                                         args.partition_size)
    ws = torch.zeros(max(ws_bytes, 1), dtype=torch.uint8, device=dev)    # zeroed once

    # The block tables stay resident on the device; a decode step changes at
    # most each sequence's last entry (a fresh block, or a copy-on-write
    # replacement), so one pinned staging buffer per in-flight step carries
    # [slots | lens | (index, value) of every sequence's last entry].
    n_i32 = 4 * S
    ring = [torch.empty(n_i32, dtype=torch.int32, pin_memory=True) for _ in range(3)]
    ring_np = [r.numpy() for r in ring]
    ring_ev = [torch.cuda.Event() for _ in range(3)]
    for e in ring_ev:
        e.record()
    stage = torch.empty(2 * S, dtype=torch.int32, device=dev)
    lens_d = stage[S:2 * S]
    tables_d = torch.from_numpy(alloc.tables[:S]).to(dev)
    rows_s = np.arange(S)
    torch.cuda.synchronize()

    parity = {}
    if ref is not None:
        lens0 = torch.from_numpy(np.asarray(case.context_lens, dtype=np.int32)).to(dev)
        lib.paged_attention_decode(out, dev_words(case.q), k_pool, v_pool, tables_d, lens0,
                                   int(case.context_lens.max()), case.scale, args.partition_size,
                                   ws)
        got = out.float().cpu().numpy().astype(np.float64)
        parity = dict(max_abs_err=float(np.abs(got - ref).max()), parity_rows=int(S * hq))

    kv_per_tok = 2 * hkv * d * 2
    ev_pairs = []
    lens_seen = []

    def step(i, timed):
        sl, pairs = alloc.append_step(sids)                                  # a1
        r = i % 3
        ring_ev[r].synchronize()
        buf = ring_np[r]
        buf[:S] = sl
        lens = alloc.lens[:S]
        buf[S:2 * S] = lens
        last = (lens - 1) // B
        buf[2 * S::2] = rows_s * maxb + last
        buf[2 * S + 1::2] = alloc.tables[rows_s, last]
        if len(pairs):                                                       # a3
            lib.copy_blocks(k_pool, v_pool, torch.from_numpy(pairs).to(dev))
        # a2, with the step's index arrays and table entries going up in the
        # same launch
        lib.upload_and_append(stage, ring[r], k_steps[i], v_steps[i], k_pool, v_pool,
                              tables=tables_d, num_updates=S)
        ring_ev[r].record()
        mcl = int(alloc.lens[:S].max())
        # the decode call is bracketed by timing events on every event_every-th
        # timed step (each event is a marker the GPU processes between kernels)
        sample = timed and (i - args.warmup) % args.event_every == 0
        if sample:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
        lib.paged_attention_decode(out, q_steps[i], k_pool, v_pool, tables_d, lens_d, mcl,
                                   case.scale, args.partition_size, ws)       # a4 + a5
        if sample:
            e1.record()
            ev_pairs.append((e0, e1))
            lens_sampled.append(alloc.lens[:S].copy())
        if timed:
            lens_seen.append(alloc.lens[:S].copy())     # bytes are counted after timing
        return mcl

    lens_sampled = []
    for i in range(args.warmup):
        step(i, False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.warmup, T):
        mcl = step(i, True)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    durs = [a.elapsed_time(b) * 1e-3 for a, b in ev_pairs]

    def call_bytes(ln):
        return (int(ln.sum()) * kv_per_tok + 2 * S * hq * d * 2 + int((-(-ln // B)).sum()) * 4
                + S * 4)

    # the last step's decode call again, caches flushed before each
    flush = flushed_times(torch, lambda: lib.paged_attention_decode(
        out, q_steps[T - 1], k_pool, v_pool, tables_d, lens_d, mcl, case.scale,
        args.partition_size, ws), args.flush_iters)
    alloc.validate()
    res = dict(elapsed=el, tokens=S * args.steps, durs=durs,
               bytes=[call_bytes(ln) for ln in lens_sampled],
               step_bytes=[call_bytes(ln) for ln in lens_seen],
               flush_durs=flush, flush_bytes=call_bytes(lens_seen[-1]),
               ctx_mean=float(alloc.lens[:S].mean()), **parity)
    if getattr(args, "keep_state", False):     # for tests of this loop: what the last step saw
        res["state"] = dict(out=out, q=q_steps[T - 1], k_new=k_steps[T - 1], v_new=v_steps[T - 1],
                            k_pool=k_pool, v_pool=v_pool, tables=alloc.tables[:S].copy(),
                            lens=alloc.lens[:S].copy(), tables_dev=tables_d.cpu().numpy())
    return res


def run_extend(args, case, torch, lib, alloc_cls):
    """Repeated extend steps: allocate the new chunk (a1), append it (a2),
    extend (a6), then hand the chunk's blocks back (truncate)."""
    dev = torch.device("cuda:0")
    R = len(case.prefix_lens)
    hq, hkv, d = case.num_q_heads, case.num_kv_heads, case.head_dim
    maxb = -(-int(case.seq_lens.max()) // 16) + 1
    alloc = alloc_cls(case.num_blocks + R, 16, max_seqs=R, max_blocks_per_seq=maxb,
                      free_order=np.concatenate([case.free_order,
                                                 np.arange(case.num_blocks, case.num_blocks + R)]))
    sids = [alloc.new_seq() for _ in range(R)]

    def dev_words(w):
        return torch.from_numpy(np.ascontiguousarray(w).view(np.int16)).view(torch.bfloat16).to(dev)

    ps = np.concatenate([alloc.append_tokens(s, int(p))[0] for s, p in zip(sids, case.prefix_lens)])
    k_pool, v_pool = lib.new_pools(case.num_blocks + R, hkv, d, 16, torch.bfloat16, dev)
    lib.paged_kv_append(dev_words(case.prefix_k), dev_words(case.prefix_v),
                        torch.from_numpy(ps).to(dev), k_pool, v_pool)
    k_new, v_new, q = dev_words(case.new_k), dev_words(case.new_v), dev_words(case.q)
    out = torch.empty_like(q)
    cu = torch.from_numpy(case.cu_new.astype(np.int32)).to(dev)
    seq_lens = torch.from_numpy(case.seq_lens.astype(np.int32)).to(dev)
    n_new = int(case.new_lens.sum())
    ring = [torch.empty(n_new + R * maxb, dtype=torch.int32, pin_memory=True) for _ in range(3)]
    ring_ev = [torch.cuda.Event() for _ in range(3)]
    for e in ring_ev:
        e.record()
    stage = torch.empty(n_new + R * maxb, dtype=torch.int32, device=dev)
    tables_d = stage[n_new:].view(R, maxb)
    T = args.warmup + args.steps
    flops = 4.0 * d * hq * float(sum(int(n) * int(p) + int(n) * (int(n) + 1) / 2
                                     for p, n in zip(case.prefix_lens, case.new_lens)))
    ev_pairs = []
    torch.cuda.synchronize()

    def step(i, timed):
        sl = np.concatenate([alloc.append_tokens(s, int(n))[0] for s, n in zip(sids, case.new_lens)])
        r = i % 3
        ring_ev[r].synchronize()
        buf = ring[r].numpy()
        buf[:n_new] = sl
        buf[n_new:] = alloc.tables[:R].reshape(-1)
        lib.upload_and_append(stage, ring[r], k_new, v_new, k_pool, v_pool)   # index arrays + a2
        ring_ev[r].record()
        if timed:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
        lib.paged_attention_extend(out, q, cu, seq_lens, k_pool, v_pool, tables_d,
                                   int(case.new_lens.max()), int(case.seq_lens.max()), case.scale)
        if timed:
            e1.record()
            ev_pairs.append((e0, e1))
        for s, p in zip(sids, case.prefix_lens):
            alloc.truncate(s, int(p))

    for i in range(args.warmup):
        step(i, False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.warmup, T):
        step(i, True)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    durs = [a.elapsed_time(b) * 1e-3 for a, b in ev_pairs]
    # one more chunk in place, then the extend call again with caches flushed
    # before each call
    sl = np.concatenate([alloc.append_tokens(s, int(n))[0] for s, n in zip(sids, case.new_lens)])
    buf = ring[0].numpy()
    ring_ev[0].synchronize()
    buf[:n_new] = sl
    buf[n_new:] = alloc.tables[:R].reshape(-1)
    lib.upload_and_append(stage, ring[0], k_new, v_new, k_pool, v_pool)
    torch.cuda.synchronize()
    flush = flushed_times(torch, lambda: lib.paged_attention_extend(
        out, q, cu, seq_lens, k_pool, v_pool, tables_d, int(case.new_lens.max()),
        int(case.seq_lens.max()), case.scale), args.flush_iters)
    res = dict(elapsed=el, tokens=n_new * args.steps, durs=durs, flops=flops, flush_durs=flush)
    if getattr(args, "keep_state", False):     # for tests of this loop: what the last step saw
        res["state"] = dict(out=out, k_pool=k_pool, v_pool=v_pool,
                            tables=tables_d.cpu().numpy().copy())
    return res


def run_shared(args, case, torch, lib, alloc_cls):
    """Fork + copy-on-write + decode steps over the shared-prefix case: the
    fork and its copy-on-write step happen in warm-up; timed steps decode all
    268 sequences (the 4096-token prompt's 256 blocks shared by all)."""
    dev = torch.device("cuda:0")
    hq, hkv, d = case.num_q_heads, case.num_kv_heads, case.head_dim
    T = args.warmup + args.steps
    S = case.num_decoding
    extra = S * (T // 16 + 2)
    nb = case.num_blocks + extra
    order = np.concatenate([case.free_order, np.arange(case.num_blocks, nb)])
    maxb = -(-(case.prefix_len + int(case.suffix_lens.max()) + T + 1) // 16)
    alloc = alloc_cls(nb, 16, max_seqs=S + 1, max_blocks_per_seq=maxb, free_order=order)

    def dev_words(w):
        return torch.from_numpy(np.ascontiguousarray(w).view(np.int16)).view(torch.bfloat16).to(dev)

    k_pool, v_pool = lib.new_pools(nb, hkv, d, 16, torch.bfloat16, dev)
    root = alloc.new_seq()
    s, _ = alloc.append_tokens(root, case.prefix_len)
    lib.paged_kv_append(dev_words(case.prefix_k), dev_words(case.prefix_v),
                        torch.from_numpy(s).to(dev), k_pool, v_pool)
    sids, sl = [], []
    for i in range(len(case.suffix_lens)):
        sid = alloc.fork(root)[0]
        sl.append(alloc.append_tokens(sid, int(case.suffix_lens[i]))[0])
        sids.append(sid)
    lib.paged_kv_append(dev_words(case.suffix_k), dev_words(case.suffix_v),
                        torch.from_numpy(np.concatenate(sl)).to(dev), k_pool, v_pool)
    alloc.free(root)
    order_s = list(sids)
    for p in case.parents:
        order_s += alloc.fork(sids[int(p)], case.samples_per_parent - 1)
    rows = np.asarray(order_s)
    import workloads as W
    rng = np.random.default_rng(4000)
    q_steps = dev_words(W.normal_words(rng, (T, S, hq, d), "bf16"))
    k_steps = dev_words(W.normal_words(rng, (T, S, hkv, d), "bf16"))
    v_steps = dev_words(W.normal_words(rng, (T, S, hkv, d), "bf16"))
    out = torch.empty((S, hq, d), dtype=torch.bfloat16, device=dev)
    ws = torch.zeros(max(1, lib.paged_attention_decode_workspace_size(S, hq, hkv, d, maxb * 16, 0)),
                     dtype=torch.uint8, device=dev)
    ev_pairs, snaps = [], []
    kv_per_tok = 2 * hkv * d * 2
    n_pairs = 0
    # device-resident tables; pinned staging per in-flight step: [slots | lens
    # | (index, value) of every sequence's last table entry], uploaded by a kernel
    n_i32 = 4 * S
    ring = [torch.empty(n_i32, dtype=torch.int32, pin_memory=True) for _ in range(3)]
    ring_np = [r.numpy() for r in ring]
    ring_ev = [torch.cuda.Event() for _ in range(3)]
    for e in ring_ev:
        e.record()
    stage = torch.empty(2 * S, dtype=torch.int32, device=dev)
    lens_d = stage[S:2 * S]
    tables_d = torch.from_numpy(alloc.tables[rows]).to(dev)
    rows_s = np.arange(S)
    groups = None
    if not args.plain_decode:
        from paged_kv_cache_63_amd import shared_prefix_groups
        # the shared prompt's blocks lead every table for the whole run: the
        # groups are found once, from the tables the allocator holds
        groups = lib.groups_to_device(shared_prefix_groups(alloc.tables[rows], alloc.lens[rows] + 1))
        ws = torch.zeros(lib.paged_attention_decode_shared_workspace_size(
            S, hq, hkv, d, maxb * 16, 0, len(groups[2]), groups[3], groups[4]),
            dtype=torch.uint8, device=dev)
    for i in range(T):
        timed = i >= args.warmup
        if i == args.warmup:
            torch.cuda.synchronize()
            t0 = time.perf_counter()
        slots, pairs = alloc.append_step(order_s)
        n_pairs += len(pairs)
        if len(pairs):
            lib.copy_blocks(k_pool, v_pool, torch.from_numpy(pairs).to(dev))
        lens = alloc.lens[rows]
        r = i % 3
        ring_ev[r].synchronize()
        buf = ring_np[r]
        buf[:S] = slots
        buf[S:2 * S] = lens
        last = (lens - 1) // 16
        buf[2 * S::2] = rows_s * maxb + last
        buf[2 * S + 1::2] = alloc.tables[rows, last]
        lib.upload_and_append(stage, ring[r], k_steps[i], v_steps[i], k_pool, v_pool,
                              tables=tables_d, num_updates=S)
        ring_ev[r].record()
        if timed:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
        if groups is None:
            lib.paged_attention_decode(out, q_steps[i], k_pool, v_pool, tables_d, lens_d,
                                       int(lens.max()), case.scale, 0, ws)
        else:
            lib.paged_attention_decode_shared(out, q_steps[i], k_pool, v_pool, tables_d, lens_d,
                                              maxb * 16, case.scale, groups, 0, ws)
        if timed:
            e1.record()
            ev_pairs.append((e0, e1))
            snaps.append((alloc.tables[rows].copy(), lens.copy()))
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    # the last step's decode call again, caches flushed before each call
    if groups is None:
        again = lambda: lib.paged_attention_decode(out, q_steps[T - 1], k_pool, v_pool, tables_d,
                                                   lens_d, int(lens.max()), case.scale, 0, ws)
    else:
        again = lambda: lib.paged_attention_decode_shared(out, q_steps[T - 1], k_pool, v_pool,
                                                          tables_d, lens_d, maxb * 16, case.scale,
                                                          groups, 0, ws)
    flush = flushed_times(torch, again, args.flush_iters)
    uniq, logical = [], []
    for tabs, lens in snaps:        # distinct (block, used slot) pairs, counted once
        used = {}
        for row, L in zip(tabs, lens):
            nb = -(-int(L) // 16)
            for j in range(nb):
                b = int(row[j])
                used[b] = max(used.get(b, 0), min(16, int(L) - 16 * j))
        uniq.append(sum(used.values()) * kv_per_tok)
        logical.append(int(lens.sum()) * kv_per_tok)
    durs = [a.elapsed_time(b) * 1e-3 for a, b in ev_pairs]
    return dict(elapsed=el, tokens=S * args.steps, durs=durs, bytes=uniq, step_bytes=uniq,
                logical=logical, cow_pairs=n_pairs, shared=groups is not None,
                flush_durs=flush, flush_bytes=uniq[-1], flush_logical=logical[-1])


def run_swap(args, case, torch, lib, alloc_cls):
    """The gqa4 decode case's whole KV cache moved to pinned host memory and
    back: one step = swap_out of all 64 sequences + swap_blocks (device ->
    host), then swap_in + swap_blocks (host -> device).  A pinned DMA copy
    of the same byte count (torch copy_) is timed beside it as the link's
    practical rate."""
    dev = torch.device("cuda:0")
    S, hkv, d = case.num_seqs, case.num_kv_heads, case.head_dim
    nb = case.num_blocks
    alloc = alloc_cls(nb, 16, max_seqs=S, free_order=case.free_order, num_host_blocks=nb)
    sids = [alloc.new_seq() for _ in range(S)]
    slots = np.concatenate([alloc.append_tokens(s, int(L))[0] for s, L in zip(sids, case.context_lens)])
    k_pool, v_pool = lib.new_pools(nb, hkv, d, 16, torch.bfloat16, dev)
    lib.paged_kv_append(torch.from_numpy(case.k.view(np.int16)).view(torch.bfloat16).to(dev),
                        torch.from_numpy(case.v.view(np.int16)).view(torch.bfloat16).to(dev),
                        torch.from_numpy(slots).to(dev), k_pool, v_pool)
    hk, hv = lib.new_host_pools(nb, hkv, d, 16, torch.bfloat16)
    blk_bytes = 2 * hkv * 16 * d * 2
    outs, ins, moved = [], [], []
    T = args.warmup + args.steps
    torch.cuda.synchronize()
    t0 = None
    for i in range(T):
        if i == args.warmup:
            torch.cuda.synchronize()
            t0 = time.perf_counter()
        e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        pairs = torch.from_numpy(alloc.swap_out(sids)).to(dev)
        e[0].record()
        lib.swap_blocks(hk, hv, k_pool, v_pool, pairs)
        e[1].record()
        pairs = torch.from_numpy(alloc.swap_in(sids)).to(dev)
        e[2].record()
        lib.swap_blocks(k_pool, v_pool, hk, hv, pairs)
        e[3].record()
        if i >= args.warmup:
            outs.append((e[0], e[1]))
            ins.append((e[2], e[3]))
            moved.append(len(pairs) * blk_bytes)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    alloc.validate()
    # reference: one pinned DMA copy each way of the same bytes
    n = moved[0]
    h = torch.empty(n, dtype=torch.uint8, pin_memory=True)
    g = torch.empty(n, dtype=torch.uint8, device=dev)
    ref = {}
    for name, (dst, src) in (("d2h", (h, g)), ("h2d", (g, h))):
        ts = []
        for _ in range(4):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            dst.copy_(src, non_blocking=True)
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) * 1e-3)
        ref[name] = n / float(np.median(ts[1:])) / 1e9
    d_out = [a.elapsed_time(b) * 1e-3 for a, b in outs]
    d_in = [a.elapsed_time(b) * 1e-3 for a, b in ins]
    return dict(elapsed=el, moved=moved, d_out=d_out, d_in=d_in, ref=ref)


def agent_trace(sessions=64, turns=4, seed=7):
    """Synthetic multi-turn agent requests shaped like the SGLang guide's
    prefill diagram: every session starts with the same 2,048-token system
    prompt and 1,024 tokens of tool definitions, then alternates 500-token
    user turns and 300-token answers; turn k's prompt is turn k-1's prompt
    plus its answer plus the new question.  Requests are interleaved across
    sessions turn by turn.  Returns [(session, prompt tokens, answer tokens)]."""
    rng = np.random.default_rng(seed)
    head = rng.integers(0, 32000, 3072).tolist()
    hist = [list(head) for _ in range(sessions)]
    out = []
    for _ in range(turns):
        for s in range(sessions):
            hist[s] = hist[s] + rng.integers(0, 32000, 500).tolist()
            ans = rng.integers(0, 32000, 300).tolist()
            out.append((s, list(hist[s]), ans))
            hist[s] = hist[s] + ans
    return out


def replay(trace, kind, num_blocks, limit=None, model=False):
    """Run requests through a prefix cache: admit, append what is not cached,
    append the answer, index the sequence, finish.  kind: 'hash' or 'radix';
    model=True runs the oracle's plain model instead of the library."""
    B = 16
    hit = total = 0
    if model:
        from oracle.block_manager import RefBlockManager
        from oracle.prefix_cache import FlatRadixTree, PrefixKeyedCache
        if kind == "hash":
            c = PrefixKeyedCache(num_blocks, B)
        else:
            bm = RefBlockManager(num_blocks, B)
            c = FlatRadixTree(bm)
    else:
        from paged_kv_cache_63_amd import BlockAllocator, PrefixCachingAllocator, RadixCache
        if kind == "hash":
            c = PrefixCachingAllocator(num_blocks, B, max_seqs=8, max_blocks_per_seq=num_blocks)
        else:
            c = RadixCache(BlockAllocator(num_blocks, B, max_seqs=8, max_blocks_per_seq=num_blocks))
    t0 = time.perf_counter()
    for n, (_, prompt, ans) in enumerate(trace[:limit]):
        full = prompt + ans
        if kind == "hash":
            sid, got = c.start(prompt)
            if model:
                c.append(sid, len(full) - got)
                c.commit(sid, full)
                c.free_seq(sid)
            else:
                c.append_tokens(sid, len(prompt) - got)
                c.append_tokens(sid, len(ans))
                c.commit(sid, full)
                c.free(sid)
        else:
            sid, got = c.admit(prompt)
            need = -(-len(full) // B) - got // B
            if model:
                short = need - len(c.bm.free)
                if short > 0:
                    c.evict(short)
                c.bm.append(sid, len(full) - got)
            else:
                short = need - c.alloc.num_free()
                if short > 0:
                    c.evict(short)
                c.alloc.append_tokens(sid, len(full) - got)
            c.finish(sid, full)
        hit += got
        total += len(prompt)
    return time.perf_counter() - t0, hit, total


def run_prefix_host(args):
    trace = agent_trace()
    nb = 6000    # 96K tokens: about a third of the trace's distinct tokens
    res = {}
    for kind in ("hash", "radix"):
        best = None
        for _ in range(max(1, args.steps)):
            el, hit, total = replay(trace, kind, nb)
            best = el if best is None else min(best, el)
        res[kind] = (best, hit, total)
    cpu = None
    if not args.no_cpu_baseline:
        n = 48
        el, _, _ = replay(trace, "radix", nb, limit=n, model=True)
        eh, _, _ = replay(trace, "hash", nb, limit=n, model=True)
        cpu = {"value": round(2 * n / (el + eh), 2), "unit": "requests/s", "cores": 1,
               "kind": "oracle",
               "sample": f"the first {n} requests of the same trace through each oracle model "
                         "(the prefix-keyed hash model and the flat-list radix tree), "
                         "one thread; value = requests/s over both"}
    nreq = len(trace)
    hb, hh, ht = res["hash"]
    rb, rh, rt = res["radix"]
    line = {"metric": "host prefix-cache requests/s (admit, append, index, finish) on a "
                      "multi-turn agent trace",
            "value": round(nreq / hb, 2), "unit": "requests/s", "n_gpus": 1,
            "steps": args.steps, "warmup": 0, "ms_per_step": round(hb * 1e3, 3),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int64",
            "data": "synthetic token ids (64 sessions x 4 turns, 3,072-token shared head)",
            "config": {"workload": "prefix-cache-host", "requests": nreq, "block_size": 16,
                       "pool_blocks": nb},
            "hash_cache": {"requests_per_s": round(nreq / hb, 2),
                           "hit_fraction": round(hh / ht, 4)},
            "radix_cache": {"requests_per_s": round(nreq / rb, 2),
                            "hit_fraction": round(rh / rt, 4)},
            "roofline": None, "cpu_baseline": cpu}
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}, WORLD_SIZE={world}); "
              "the paged-attention path here runs on a single GPU", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        sys.exit("--steps must be >= 1 and --warmup >= 0")

    if args.event_every < 1:
        sys.exit("--event-every must be at least 1")
    if args.workload == "prefix-cache-host":     # host-side only: no GPU involved
        run_prefix_host(args)
        return
    T = args.warmup + args.steps
    if args.block_size != 16 and args.workload not in ("gqa4-decode", "long-context-decode"):
        sys.exit("--block-size 32 applies to gqa4-decode and long-context-decode only")
    if args.workload == "long-context-decode" and args.partition_size == 0:
        args.partition_size = 512          # the long-context workload's stated split
    case = make_case(args.workload, T)
    cpu, ref = None, None
    if not args.no_cpu_baseline and args.workload in ("gqa4-decode",):
        cpu, ref = cpu_baseline(case, args.cpu_seconds)

    import torch
    from paged_kv_cache_63_amd import BlockAllocator
    from paged_kv_cache_63_amd import _lib as lib
    lib.load()
    if not torch.cuda.is_available():
        sys.exit("no GPU visible")

    if args.copy_probe:   # a plain copy of known size, for counter calibration
        a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    if args.workload == "swap-host":
        r = run_swap(args, case, torch, lib, BlockAllocator)
        per = float(np.mean(r["moved"]))
        go, gi = per / np.mean(r["d_out"]) / 1e9, per / np.mean(r["d_in"]) / 1e9
        line = {"metric": "KV block swap GB/s, device pool <-> pinned host pool (whole cache "
                          "of the gqa4 decode workload, both directions)",
                "value": round(2 * per * args.steps / r["elapsed"] / 1e9, 2), "unit": "GB/s",
                "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
                "ms_per_step": round(r["elapsed"] / args.steps * 1e3, 3),
                "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
                "dtype": "bf16", "data": "synthetic (the gqa4 decode workload's pool)",
                "config": {"workload": "swap-host", "blocks_per_direction": int(per // (2 * 8 * 16 * 128 * 2)),
                           "bytes_per_direction": int(per)},
                "roofline": {"bound": "host-link", "achieved": round(min(go, gi), 1),
                             "peak": round(min(r["ref"]["d2h"], r["ref"]["h2d"]), 1),
                             "unit": "GB/s", "frac": round(min(go / r["ref"]["d2h"], gi / r["ref"]["h2d"]), 4),
                             "traffic": None, "kernel": "swap_blocks (swap_blocks_kernel)",
                             "d2h_gbps": round(go, 1), "h2d_gbps": round(gi, 1),
                             "peak_is": "pinned DMA copy of the same bytes (torch copy_), measured",
                             "dma_d2h_gbps": round(r["ref"]["d2h"], 1),
                             "dma_h2d_gbps": round(r["ref"]["h2d"], 1)},
                "cpu_baseline": None}
        print(json.dumps(line), flush=True)
        return
    if args.workload == "multiturn-extend":
        r = run_extend(args, case, torch, lib, BlockAllocator)
        kern = ["extend.hip"]
    elif args.workload == "shared-prefix-decode":
        r = run_shared(args, case, torch, lib, BlockAllocator)
        kern = ["decode.hip"] if args.plain_decode else ["decode.hip", "extend.hip"]
    else:
        r = run_decode(args, case, torch, lib, BlockAllocator, ref=ref)
        kern = ["decode.hip"]
        if cpu is not None and "max_abs_err" in r:
            cpu["parity"] = {"max_abs_err": r["max_abs_err"], "tolerance": 2e-2,
                             "rows": r["parity_rows"],
                             "what": "GPU decode of the workload's initial state against these "
                                     "oracle rows, every output"}

    el = r["elapsed"]
    ms_step = el / args.steps * 1e3
    # (the counter profiles are of 16-token blocks)
    traffic, _ = load_traffic(args.workload, kern) if args.block_size == 16 else (None, None)
    # Launch time of the dominant call: the median of the flushed timing pass
    # (caches evicted before every call); without that pass, the mean of the
    # step loop's sampled events.
    flush = r.get("flush_durs") or []
    warm = float(np.mean(r["durs"]))
    t_call = float(np.median(flush)) if flush else warm
    timing = {"launch_us": round(t_call * 1e6, 2),
              "launch_us_is": ("median of %d calls, L2/MALL flushed by a 1 GiB write before each"
                               % len(flush)) if flush else
                              "mean of the step loop's sampled calls (no flush)",
              "launch_us_min": round(float(np.min(flush)) * 1e6, 2) if flush else None,
              "launch_us_mean_flushed": round(float(np.mean(flush)) * 1e6, 2) if flush else None,
              "launch_us_mean_in_step_loop": round(warm * 1e6, 2)}
    if args.workload == "multiturn-extend":
        achieved = r["flops"] / t_call / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4),
                "traffic": traffic, "kernel": "paged_attention_extend (extend_bf16_kernel)",
                **timing, "flops_per_launch": r["flops"]}
        value = r["tokens"] / el
        unit = "tokens/s"
        metric = "paged extend bf16 matrix-core TFLOP/s and new tokens/s (multi-turn prefill)"
    else:
        per_launch = float(r["flush_bytes"]) if flush else float(np.mean(r["bytes"]))
        achieved = per_launch / t_call / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                "kernel": ("paged_attention_decode_shared (prefix pass extend_bf16_kernel<PREFIX> "
                           "+ decode_bf16_kernel<SHARED> + decode_fold_kernel)" if r.get("shared")
                           else "paged_attention_decode (decode_bf16_kernel + decode_fold_kernel)"),
                **timing, "bytes_per_launch": int(per_launch)}
        if not args.no_ceiling:
            ceil = bandwidth_ceilings(torch, lib)
            ceil["frac_of_read_random_4k"] = round(achieved / ceil["read_random_4k_gbps"], 4)
            ceil["note"] = ("medians of 10 flushed calls: hbm_read_probe over a 2 GiB buffer in a "
                            "random order of 4 KB chunks and in address order; torch copy_ of "
                            "2 GiB counts read + written bytes")
            roof["ceiling"] = ceil
        value = r["tokens"] / el
        unit = "tokens/s"
        metric = METRIC
    cfg = {"gqa4-decode": {"workload": "gqa4-decode", "seqs": 64, "context": "U[512,4096] + steps",
                           "q_heads": 32, "kv_heads": 8, "head_dim": 128, "block_size": 16,
                           "layers": 1},
           "long-context-decode": {"workload": "long-context-decode", "seqs": 8,
                                   "context": "U[32768,131072] + steps", "q_heads": 64,
                                   "kv_heads": 8, "head_dim": 128, "block_size": 16,
                                   "partition_tokens": 512, "layers": 1},
           "shared-prefix-decode": {"workload": "shared-prefix-decode", "seqs": 268,
                                    "shared_prefix_tokens": 4096, "suffix": "U[64,1024] + steps",
                                    "forks": "4 x 4 samples", "q_heads": 32, "kv_heads": 8,
                                    "head_dim": 128, "block_size": 16, "layers": 1},
           "multiturn-extend": {"workload": "multiturn-extend", "requests": 16,
                                "cached_prefix": "U[2048,8192]", "new_tokens": 512,
                                "q_heads": 32, "kv_heads": 8, "head_dim": 128, "block_size": 16,
                                "layers": 1}}[args.workload]
    cfg["block_size"] = args.block_size
    if "ctx_mean" in r:
        cfg["mean_context_in_timed_steps"] = round(r["ctx_mean"] - args.steps / 2, 1)
    line = {"metric": metric, "value": round(value, 2), "unit": unit, "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic (seeded N(0,1) bf16 K/V/Q, shuffled block placement)",
            "config": cfg, "roofline": roof, "cpu_baseline": cpu}
    if args.workload != "multiturn-extend":
        # algorithmic bytes of every timed step's decode call over the wall
        # time of all timed steps (the whole step, not just the decode call)
        line["step_hbm_gbps"] = round(float(np.sum(r["step_bytes"])) / el / 1e9, 1)
    if "logical" in r:
        lg = float(r["flush_logical"]) if flush else float(np.mean(r["logical"]))
        roof["logical_gbps_effective"] = round(lg / t_call / 1e9, 1)
        line["cow_pairs_in_run"] = r["cow_pairs"]
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
