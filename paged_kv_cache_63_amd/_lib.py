"""ctypes binding of libpagedkv.so.

Argument marshalling only: shapes and dtypes are checked on the host, raw
device pointers and torch's current HIP stream are handed to the C ABI, and a
non-zero status becomes a :class:`PagedKVError`.  Every step runs in the
library's kernels; there is no other implementation in this module.

Function names and argument meanings follow ``include/pagedkv.h``.
"""

import ctypes
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpagedkv.so")

_LIB = None

PKV_DTYPE = {torch.float32: 0, torch.bfloat16: 1}
SYMBOLS = ("paged_kv_append", "copy_blocks", "swap_blocks", "paged_attention_decode_workspace_size",
           "paged_attention_decode", "paged_attention_decode_shared_workspace_size",
           "paged_attention_decode_shared", "paged_attention_extend", "paged_kv_gather",
           "paged_kv_last_error", "block_manager_append_step", "pinned_upload",
           "upload_and_append", "upload_and_append_tables", "hbm_read_probe",
           "paged_attention_decode_noalloc")


class PagedKVError(RuntimeError):
    """A library call returned a non-zero status."""


def load():
    """Load the library once (after torch, so the HIP runtime torch already
    loaded is the one the library binds to).  Raises if it is not built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise PagedKVError(f"{LIB_PATH} is not built; run `python -m paged_kv_cache_63_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    i32, p, f32, sz = ctypes.c_int32, ctypes.c_void_p, ctypes.c_float, ctypes.c_size_t
    lib.paged_kv_last_error.restype = ctypes.c_char_p
    lib.paged_kv_last_error.argtypes = []
    lib.paged_kv_append.restype = ctypes.c_int
    lib.paged_kv_append.argtypes = [p, p, p, i32, p, p, i32, i32, i32, i32, i32, p]
    lib.copy_blocks.restype = ctypes.c_int
    lib.copy_blocks.argtypes = [p, p, i32, p, i32, i32, i32, i32, i32, p]
    lib.swap_blocks.restype = ctypes.c_int
    lib.swap_blocks.argtypes = [p, p, i32, p, p, i32, p, i32, i32, i32, i32, i32, p]
    lib.paged_attention_decode_workspace_size.restype = sz
    lib.paged_attention_decode_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.paged_attention_decode.restype = ctypes.c_int
    lib.paged_attention_decode.argtypes = [p, p, p, p, i32, p, i32, p, i32, i32, i32, i32, i32,
                                           i32, f32, i32, p, sz, i32, p]
    lib.paged_attention_decode_noalloc.restype = ctypes.c_int
    lib.paged_attention_decode_noalloc.argtypes = [p, p, p, p, i32, p, i32, p, i32, i32, i32, i32,
                                                   i32, i32, f32, i32, i32, p]
    lib.paged_attention_decode_shared_workspace_size.restype = sz
    lib.paged_attention_decode_shared_workspace_size.argtypes = [i32] * 9
    lib.paged_attention_decode_shared.restype = ctypes.c_int
    lib.paged_attention_decode_shared.argtypes = [p, p, p, p, i32, p, i32, p, i32, i32, i32, i32,
                                                  i32, i32, ctypes.c_float, p, p, p, i32, i32,
                                                  i32, i32, p, sz, i32, p]
    lib.paged_attention_extend.restype = ctypes.c_int
    lib.paged_attention_extend.argtypes = [p, p, p, p, i32, i32, i32, i32, p, p, i32, p, i32,
                                           i32, i32, i32, i32, f32, i32, p]
    lib.paged_kv_gather.restype = ctypes.c_int
    lib.paged_kv_gather.argtypes = [p, p, p, p, i32, p, i32, i32, i32, i32, i32, p]
    lib.pinned_upload.restype = ctypes.c_int
    lib.pinned_upload.argtypes = [p, p, ctypes.c_int64, p]
    lib.upload_and_append.restype = ctypes.c_int
    lib.upload_and_append.argtypes = [p, p, ctypes.c_int64, ctypes.c_int64, p, p, i32, p, p, i32,
                                      i32, i32, i32, i32, p]
    lib.upload_and_append_tables.restype = ctypes.c_int
    lib.upload_and_append_tables.argtypes = [p, p, ctypes.c_int64, ctypes.c_int64, p,
                                             ctypes.c_int64, i32, p, p, i32, p, p, i32, i32, i32,
                                             i32, i32, p]
    lib.hbm_read_probe.restype = ctypes.c_int
    lib.hbm_read_probe.argtypes = [p, ctypes.c_int64, i32, p, p, i32, p]
    lib.block_manager_append_step.restype = ctypes.c_int
    lib.block_manager_append_step.argtypes = [p, p, p, p, p, i32, i32, p, p, i32, i32, p, i32,
                                              p, p, p, p, p]
    _LIB = lib
    return lib


def _check(rc: int) -> None:
    if rc != 0:
        raise PagedKVError(f"status {rc}: {load().paged_kv_last_error().decode()}")


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _dev(*ts):
    for t in ts:
        if not t.is_cuda:
            raise ValueError("all tensors must be on the GPU")
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")


def _int32(*ts):
    for t in ts:
        if t.dtype != torch.int32:
            raise ValueError("index tensors must be int32")


def _pools(k_pool, v_pool, host_ok=False):
    for t in (k_pool, v_pool):
        if not t.is_contiguous():
            raise ValueError("pools must be contiguous")
        if not t.is_cuda and not (host_ok and t.is_pinned()):
            raise ValueError("pools must be on the GPU" + (" or in pinned host memory"
                                                            if host_ok else ""))
    if k_pool.dim() != 4 or v_pool.dim() != 4:
        raise ValueError("pools must be 4-D")
    nb, hkv, bs, d = k_pool.shape
    if tuple(v_pool.shape) != (nb, hkv, d, bs):
        raise ValueError(f"v_pool must be [num_blocks][Hkv][D][B] (one D x B slab per block "
                         f"and head, stored in 16-token halves) = {(nb, hkv, d, bs)}, "
                         f"got {tuple(v_pool.shape)}")
    if k_pool.dtype != v_pool.dtype or k_pool.dtype not in PKV_DTYPE:
        raise ValueError("pools must share a dtype in (float32, bfloat16)")
    return nb, hkv, bs, d, PKV_DTYPE[k_pool.dtype]


def new_pools(num_blocks, num_kv_heads, head_dim, block_size=16, dtype=torch.bfloat16,
              device="cuda"):
    """Empty K and V pools in the library's layout (contents undefined)."""
    k = torch.empty((num_blocks, num_kv_heads, block_size, head_dim), dtype=dtype, device=device)
    v = torch.empty((num_blocks, num_kv_heads, head_dim, block_size), dtype=dtype, device=device)
    return k, v


def paged_kv_append(k_new, v_new, slot_mapping, k_pool, v_pool):
    nb, hkv, bs, d, dt = _pools(k_pool, v_pool)
    _dev(k_new, v_new, slot_mapping, k_pool, v_pool)
    _int32(slot_mapping)
    T = slot_mapping.shape[0]
    if tuple(k_new.shape) != (T, hkv, d) or tuple(v_new.shape) != (T, hkv, d):
        raise ValueError("k_new/v_new must be [T][Hkv][D]")
    if k_new.dtype != k_pool.dtype or v_new.dtype != k_pool.dtype:
        raise ValueError("k_new/v_new dtype must match the pools")
    _check(load().paged_kv_append(_ptr(k_new), _ptr(v_new), _ptr(slot_mapping), T, _ptr(k_pool),
                                  _ptr(v_pool), nb, hkv, d, bs, dt, _stream()))


def copy_blocks(k_pool, v_pool, block_mapping):
    nb, hkv, bs, d, dt = _pools(k_pool, v_pool)
    _dev(k_pool, v_pool, block_mapping)
    _int32(block_mapping)
    if block_mapping.dim() != 2 or block_mapping.shape[1] != 2:
        raise ValueError("block_mapping must be [N][2]")
    _check(load().copy_blocks(_ptr(k_pool), _ptr(v_pool), nb, _ptr(block_mapping),
                              block_mapping.shape[0], hkv, d, bs, dt, _stream()))


def pinned_upload(dst, src, nbytes=None):
    """Copy ``src`` (a pinned host tensor, or a device tensor) into the device
    tensor ``dst`` with a kernel on the current stream; ``nbytes`` defaults to
    ``src``'s size.  ``src`` must stay unchanged until the stream has passed
    the copy (record an event after it)."""
    if not dst.is_cuda:
        raise ValueError("dst must be a device tensor")
    if not (src.is_cuda or src.is_pinned()):
        raise ValueError("src must be pinned host memory or a device tensor")
    if not (dst.is_contiguous() and src.is_contiguous()):
        raise ValueError("dst and src must be contiguous")
    n = src.numel() * src.element_size() if nbytes is None else int(nbytes)
    if n > dst.numel() * dst.element_size() or n > src.numel() * src.element_size():
        raise ValueError("nbytes exceeds a buffer")
    _check(load().pinned_upload(_ptr(dst), _ptr(src), n, _stream()))


def upload_and_append(dst, staging, k_new, v_new, k_pool, v_pool, slots_at=0, tables=None,
                      num_updates=0):
    """:func:`pinned_upload` of the int32 ``staging`` buffer into ``dst`` and
    :func:`paged_kv_append` of ``k_new``/``v_new`` whose slot mapping is
    ``staging[slots_at : slots_at + len(k_new)]``, in one call.

    With ``tables`` (a device int32 tensor) and ``num_updates`` > 0, the last
    ``2 * num_updates`` words of ``staging`` are (index, value) pairs written
    into ``tables.view(-1)`` in the same launch, and only the words before
    them are copied to ``dst``."""
    nb, hkv, bs, d, dt = _pools(k_pool, v_pool)
    _dev(k_new, v_new, k_pool, v_pool)
    if not dst.is_cuda or not (staging.is_cuda or staging.is_pinned()):
        raise ValueError("dst must be a device tensor and staging pinned (or on the device)")
    if staging.dtype != torch.int32 or not (dst.is_contiguous() and staging.is_contiguous()):
        raise ValueError("staging must be a contiguous int32 tensor, dst contiguous")
    T = k_new.shape[0]
    if tuple(k_new.shape) != (T, hkv, d) or tuple(v_new.shape) != (T, hkv, d):
        raise ValueError("k_new/v_new must be [T][Hkv][D]")
    if k_new.dtype != k_pool.dtype or v_new.dtype != k_pool.dtype:
        raise ValueError("k_new/v_new dtype must match the pools")
    nu = int(num_updates)
    if nu < 0 or 2 * nu > staging.numel():
        raise ValueError("num_updates must be in [0, staging.numel() / 2]")
    if nu and (tables is None or not tables.is_cuda or tables.dtype != torch.int32
               or not tables.is_contiguous()):
        raise ValueError("table updates need a contiguous int32 device tensor of tables")
    n = (staging.numel() - 2 * nu) * 4
    if n > dst.numel() * dst.element_size():
        raise ValueError("dst is smaller than the staged words")
    if nu == 0:
        _check(load().upload_and_append(_ptr(dst), _ptr(staging), n, 4 * int(slots_at),
                                        _ptr(k_new), _ptr(v_new), T, _ptr(k_pool), _ptr(v_pool),
                                        nb, hkv, d, bs, dt, _stream()))
        return
    _check(load().upload_and_append_tables(_ptr(dst), _ptr(staging), n, 4 * int(slots_at),
                                           _ptr(tables), tables.numel(), nu, _ptr(k_new),
                                           _ptr(v_new), T, _ptr(k_pool), _ptr(v_pool), nb, hkv,
                                           d, bs, dt, _stream()))


def new_host_pools(num_blocks, num_kv_heads, head_dim, block_size=16, dtype=torch.bfloat16):
    """Pinned host pools with the device pools' layout (the host tier for
    :func:`swap_blocks`)."""
    return (torch.empty((num_blocks, num_kv_heads, block_size, head_dim), dtype=dtype,
                        pin_memory=True),
            torch.empty((num_blocks, num_kv_heads, head_dim, block_size), dtype=dtype,
                        pin_memory=True))


def swap_blocks(dst_k, dst_v, src_k, src_v, block_mapping):
    """Copy blocks ``block_mapping[i] = (src, dst)`` from the (src_k, src_v)
    pools into the (dst_k, dst_v) pools; either pair may be pinned host
    pools.  Runs on torch's current stream."""
    dnb, hkv, bs, d, dt = _pools(dst_k, dst_v, host_ok=True)
    snb, hkv2, bs2, d2, dt2 = _pools(src_k, src_v, host_ok=True)
    if (hkv, bs, d, dt) != (hkv2, bs2, d2, dt2):
        raise ValueError("source and destination pools differ in shape or dtype")
    _dev(block_mapping)
    _int32(block_mapping)
    if block_mapping.dim() != 2 or block_mapping.shape[1] != 2:
        raise ValueError("block_mapping must be [n][2]")
    _check(load().swap_blocks(_ptr(dst_k), _ptr(dst_v), dnb, _ptr(src_k), _ptr(src_v), snb,
                              _ptr(block_mapping), block_mapping.shape[0], hkv, d, bs, dt,
                              _stream()))


def paged_attention_decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                          max_context_len, partition_size=0):
    return int(load().paged_attention_decode_workspace_size(num_seqs, num_q_heads, num_kv_heads,
                                                             head_dim, max_context_len,
                                                             partition_size))


def paged_attention_decode(out, q, k_pool, v_pool, block_tables, context_lens, max_context_len,
                           scale, partition_size=0, workspace=None):
    nb, hkv, bs, d, dt = _pools(k_pool, v_pool)
    _dev(out, q, k_pool, v_pool, block_tables, context_lens)
    _int32(block_tables, context_lens)
    S, hq, dq = q.shape
    if dq != d or tuple(out.shape) != (S, hq, d) or out.dtype != q.dtype or q.dtype != k_pool.dtype:
        raise ValueError("q/out must be [S][Hq][D] in the pool dtype")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.shape[0] != S:
        raise ValueError("block_tables [S][max_blocks], context_lens [S]")
    need = paged_attention_decode_workspace_size(S, hq, hkv, d, max_context_len, partition_size)
    if need and workspace is None:
        # zero-filled once: no piece-count word can then hold a call's tag by chance
        workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)
    if workspace is not None:
        _dev(workspace)
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load().paged_attention_decode(_ptr(out), _ptr(q), _ptr(k_pool), _ptr(v_pool), nb,
                                         _ptr(block_tables), block_tables.shape[1],
                                         _ptr(context_lens), S, int(max_context_len), hq, hkv, d,
                                         bs, float(scale), int(partition_size), _ptr(workspace),
                                         wbytes, dt, _stream()))
    return workspace


def paged_attention_decode_noalloc(out, q, k_pool, v_pool, block_tables, context_lens,
                                   max_context_len, scale, partition_size=0):
    """paged_attention_decode with the library's fixed per-GPU workspace
    (nothing is allocated, here or in the library)."""
    nb, hkv, bs, d, dt = _pools(k_pool, v_pool)
    _dev(out, q, k_pool, v_pool, block_tables, context_lens)
    _int32(block_tables, context_lens)
    S, hq, dq = q.shape
    if dq != d or tuple(out.shape) != (S, hq, d) or out.dtype != q.dtype or q.dtype != k_pool.dtype:
        raise ValueError("q/out must be [S][Hq][D] in the pool dtype")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.shape[0] != S:
        raise ValueError("block_tables [S][max_blocks], context_lens [S]")
    _check(load().paged_attention_decode_noalloc(
        _ptr(out), _ptr(q), _ptr(k_pool), _ptr(v_pool), nb, _ptr(block_tables),
        block_tables.shape[1], _ptr(context_lens), S, int(max_context_len), hq, hkv, d, bs,
        float(scale), int(partition_size), dt, _stream()))


def paged_attention_decode_shared_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                                 max_context_len, partition_size, num_groups,
                                                 max_group_size, max_prefix_blocks):
    return int(load().paged_attention_decode_shared_workspace_size(
        num_seqs, num_q_heads, num_kv_heads, head_dim, int(max_context_len), int(partition_size),
        int(num_groups), int(max_group_size), int(max_prefix_blocks)))


def paged_attention_decode_shared(out, q, k_pool, v_pool, block_tables, context_lens,
                                  max_context_len, scale, groups, partition_size=0,
                                  workspace=None):
    """``groups``: ``(group_offsets, group_seqs, group_prefix_blocks, max_group_size,
    max_prefix_blocks)`` -- three int32 device tensors and two host ints, as
    :func:`groups_to_device` makes them from the host grouping
    (``allocator.shared_prefix_groups``)."""
    nb, hkv, bs, d, dt = _pools(k_pool, v_pool)
    offs, seqs, pblk, max_size, max_pb = groups
    _dev(out, q, k_pool, v_pool, block_tables, context_lens, offs, seqs, pblk)
    _int32(block_tables, context_lens, offs, seqs, pblk)
    S, hq, dq = q.shape
    if dq != d or tuple(out.shape) != (S, hq, d) or out.dtype != q.dtype or q.dtype != k_pool.dtype:
        raise ValueError("q/out must be [S][Hq][D] in the pool dtype")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.shape[0] != S:
        raise ValueError("block_tables [S][max_blocks], context_lens [S]")
    G = offs.shape[0] - 1
    if G < 0 or pblk.shape[0] != G:
        raise ValueError("group_offsets [G+1], group_prefix_blocks [G]")
    need = paged_attention_decode_shared_workspace_size(S, hq, hkv, d, max_context_len,
                                                        partition_size, G, max_size, max_pb)
    if need and workspace is None:
        # zero-filled: no piece-count word or per-sequence word then holds a tag
        workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)
    if workspace is not None:
        _dev(workspace)
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load().paged_attention_decode_shared(
        _ptr(out), _ptr(q), _ptr(k_pool), _ptr(v_pool), nb, _ptr(block_tables),
        block_tables.shape[1], _ptr(context_lens), S, int(max_context_len), hq, hkv, d, bs,
        float(scale), _ptr(offs), _ptr(seqs), _ptr(pblk), G, int(max_size), int(max_pb),
        int(partition_size), _ptr(workspace), wbytes, dt, _stream()))
    return workspace


def groups_to_device(groups, device=None):
    """The ``groups`` tuple of :func:`allocator.shared_prefix_groups` (three
    int32 numpy arrays and two ints) with its arrays as int32 tensors on the
    GPU, as :func:`paged_attention_decode_shared` takes it."""
    offs, seqs, pblk, max_size, max_pb = groups
    dev = device if device is not None else "cuda"
    t = lambda x: torch.as_tensor(np.asarray(x, dtype=np.int32)).to(dev)
    return (t(offs), t(seqs), t(pblk), int(max_size), int(max_pb))


def paged_attention_extend(out, q, cu_seqlens_q, seq_lens, k_pool, v_pool, block_tables,
                           max_q_len, max_seq_len, scale):
    nb, hkv, bs, d, dt = _pools(k_pool, v_pool)
    _dev(out, q, cu_seqlens_q, seq_lens, k_pool, v_pool, block_tables)
    _int32(cu_seqlens_q, seq_lens, block_tables)
    Tq, hq, dq = q.shape
    R = seq_lens.shape[0]
    if dq != d or tuple(out.shape) != (Tq, hq, d) or out.dtype != q.dtype or q.dtype != k_pool.dtype:
        raise ValueError("q/out must be [Tq][Hq][D] in the pool dtype")
    if cu_seqlens_q.shape[0] != R + 1 or block_tables.dim() != 2 or block_tables.shape[0] != R:
        raise ValueError("cu_seqlens_q [R+1], seq_lens [R], block_tables [R][max_blocks]")
    _check(load().paged_attention_extend(_ptr(out), _ptr(q), _ptr(cu_seqlens_q), _ptr(seq_lens),
                                         R, Tq, int(max_q_len), int(max_seq_len), _ptr(k_pool),
                                         _ptr(v_pool), nb, _ptr(block_tables),
                                         block_tables.shape[1], hq, hkv, d, bs, float(scale), dt,
                                         _stream()))


def hbm_read_probe(buf, chunk_bytes, chunk_order=None, sink=None, num_workgroups=None):
    """Read the device buffer ``buf`` once in chunks of ``chunk_bytes`` bytes
    (in the order of the int32 device tensor ``chunk_order``, or in address
    order) -- the measured ceiling for scattered block reads.  Returns the
    sink tensor the reads are folded into."""
    _dev(buf)
    nbytes = buf.numel() * buf.element_size()
    if nbytes % chunk_bytes:
        raise ValueError("the buffer must hold a whole number of chunks")
    n = nbytes // chunk_bytes
    if chunk_order is not None:
        _dev(chunk_order)
        _int32(chunk_order)
        if chunk_order.numel() != n:
            raise ValueError("chunk_order must list every chunk once")
    if num_workgroups is None:
        num_workgroups = 8 * torch.cuda.get_device_properties(buf.device).multi_processor_count
    if sink is None:
        sink = torch.zeros(num_workgroups, dtype=torch.int32, device=buf.device)
    _check(load().hbm_read_probe(_ptr(buf), n, int(chunk_bytes), _ptr(chunk_order), _ptr(sink),
                                 int(num_workgroups), _stream()))
    return sink


def paged_kv_gather(k_out, v_out, k_pool, v_pool, block_table_row, context_len):
    nb, hkv, bs, d, dt = _pools(k_pool, v_pool)
    _dev(k_out, v_out, k_pool, v_pool, block_table_row)
    _int32(block_table_row)
    if tuple(k_out.shape) != (context_len, hkv, d) or tuple(v_out.shape) != (context_len, hkv, d):
        raise ValueError("k_out/v_out must be [context_len][Hkv][D]")
    _check(load().paged_kv_gather(_ptr(k_out), _ptr(v_out), _ptr(k_pool), _ptr(v_pool), nb,
                                  _ptr(block_table_row), int(context_len), hkv, d, bs, dt,
                                  _stream()))
