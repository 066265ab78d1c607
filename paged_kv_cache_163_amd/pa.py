"""Thin ctypes binding over libpa.so (include/pa.h).

Argument marshalling only: every step of the decode path runs in the HIP
kernels of libpa.so.  Tensors are torch device tensors (torch provides device
memory and streams); calls are issued on torch's current stream.  Importing
this module raises ImportError when libpa.so has not been built -- there is no
fallback implementation.

Tensor layouts (C-contiguous):
    q, out              [num_seqs, num_heads, head_dim]          float32 | bfloat16
    k_cache, v_cache    [num_blocks, kv_heads, block_size, head_dim]
    block_tables        int32 [num_seqs, max_blocks_per_seq]
    seq_lens            int32 [num_seqs]
    k_new, v_new        [num_tokens, kv_heads, head_dim]
    slot_mapping        int64 [num_tokens]
    block_mapping       int64 [num_pairs, 2]   (src, dst)
    kv_pool (layered)   [num_blocks, 2, num_layers, kv_heads, block_size, head_dim]
    layered q, out      [layers, num_seqs, num_heads, head_dim]
    prefill q, out      [num_queries, num_heads, head_dim]       float32 | bfloat16
    query_start         int32 [num_seqs + 1]   chunk offsets into the prefill q
"""

from __future__ import annotations

import ctypes
import os
from typing import NamedTuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpa.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with "
                      "`python -m paged_kv_cache_163_amd.build`")

_lib = ctypes.CDLL(LIB_PATH)

PA_OK, PA_ERR_INVALID_ARG, PA_ERR_UNSUPPORTED, PA_ERR_HIP, PA_ERR_NO_SPACE = 0, 1, 2, 3, 4
PA_ERR_SCRATCH = 5
NOALLOC_SCRATCH_BYTES = 16 * 1024 * 1024
PA_F32, PA_BF16 = 0, 1
KERNELS = {"auto": 0, "valu": 1, "mfma": 2}
KERNEL_NAMES = {v: k for k, v in KERNELS.items()}

_i32, _i64, _f32, _vp, _sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t


def _sig(name, restype, *argtypes):
    fn = getattr(_lib, name)
    fn.restype = restype
    fn.argtypes = list(argtypes)
    return fn


_abi_version = _sig("pa_abi_version", _i32)
_status_string = _sig("pa_status_string", ctypes.c_char_p, _i32)
_block_layout = _sig("pa_block_layout", _i32, _i64, _i32, ctypes.POINTER(_i64), ctypes.POINTER(_i64))
_kv_append = _sig("pa_kv_append", _i32, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _vp)
_decode_plan = _sig("pa_decode_plan", _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                    ctypes.POINTER(_i32), ctypes.POINTER(_i32), ctypes.POINTER(_i32),
                    ctypes.POINTER(_sz))
_workspace_bytes = _sig("pa_decode_workspace_bytes", _sz, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32)
_decode = _sig("pa_decode", _i32, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _i32, _i32, _i32,
               _i32, _i32, _f32, _i32, _vp, _sz, _i32, _vp)
_decode_ex = _sig("pa_decode_ex", _i32, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _i32, _i32,
                  _i32, _i32, _i32, _f32, _i32, _vp, _sz, _i32, _i32, _vp)
_decode_ordered = _sig("pa_decode_ordered", _i32, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _vp, _i32,
                       _i32, _i32, _i32, _i32, _i32, _f32, _i32, _vp, _sz, _i32, _i32, _vp)
_decode_append = _sig("pa_decode_append", _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp,
                      _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _i32, _vp, _sz, _i32, _i32,
                      _vp)
_decode_append_ordered = _sig("pa_decode_append_ordered", _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                              _vp, _i32, _vp, _i32, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _f32,
                              _i32, _vp, _sz, _i32, _i32, _vp)
_decode_shared_prefix = _sig("pa_decode_shared_prefix", _i32, _vp, _vp, _vp, _vp, _vp, _i32, _vp,
                            _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _vp, _vp, _i32, _i32,
                            _i32, _vp, _sz, _i32, _vp)
_decode_shared_prefix_ordered = _sig("pa_decode_shared_prefix_ordered", _i32, _vp, _vp, _vp, _vp,
                                    _vp, _i32, _vp, _i32, _vp, _i32, _i32, _i32, _i32, _i32,
                                    _i32, _f32, _vp, _vp, _i32, _i32, _i32, _vp, _sz, _i32, _vp)
_shared_prefix_ws = _sig("pa_decode_shared_prefix_workspace_bytes", _sz, _i32, _i32, _i32, _i32,
                         _i32, _i32, _i32, _vp, _vp, _i32, _i32, _i32, _i32)
_copy_blocks = _sig("pa_copy_blocks", _i32, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _vp)
_P = ctypes.POINTER
_bm_create = _sig("pa_bm_create", _i32, _i64, _i32, _i64, _i64, _P(_vp))
_bm_destroy = _sig("pa_bm_destroy", _i32, _vp)
_bm_can_admit = _sig("pa_bm_can_admit", _i32, _vp, _i64, _P(_i32))
_bm_admit = _sig("pa_bm_admit", _i32, _vp, _i64, _i64)
_bm_fork = _sig("pa_bm_fork", _i32, _vp, _i64, _i64)
_bm_append_slots = _sig("pa_bm_append_slots", _i32, _vp, _P(_i64), _i32, _P(_i64), _P(_i64), _P(_i32))
_bm_release = _sig("pa_bm_release", _i32, _vp, _i64)
_bm_swap_out = _sig("pa_bm_swap_out", _i32, _vp, _i64, _P(_i64), _i64, _P(_i64))
_bm_swap_in = _sig("pa_bm_swap_in", _i32, _vp, _i64, _P(_i64), _i64, _P(_i64))
_bm_decode_inputs = _sig("pa_bm_decode_inputs", _i32, _vp, _P(_i64), _i32, _i32, _i32, _P(_i32),
                         _P(_i32))
_bm_sequence = _sig("pa_bm_sequence", _i32, _vp, _i64, _P(_i64), _P(_i64), _P(_i32))
_bm_stats = _sig("pa_bm_stats", _i32, _vp, _P(_i64), _P(_i64), _P(_i64))
_bm_refcount = _sig("pa_bm_refcount", _i32, _vp, _i64, _i32, _P(_i32))
_kv_append_layered = _sig("pa_kv_append_layered", _i32, _vp, _vp, _vp, _i32, _i32, _vp, _i32, _i32,
                          _i32, _i32, _i32, _i32, _vp)
_decode_layered = _sig("pa_decode_layered", _i32, _vp, _vp, _vp, _i32, _i32, _i32, _vp, _i32, _vp,
                       _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _i32, _vp, _sz, _i32, _vp)
_copy_blocks_layered = _sig("pa_copy_blocks_layered", _i32, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                            _i32, _i32, _vp)
_swap_blocks_layered = _sig("pa_swap_blocks_layered", _i32, _vp, _i64, _vp, _i64, _vp, _i32, _i32,
                            _i32, _i32, _i32, _i32, _vp)
_swap_blocks = _sig("pa_swap_blocks", _i32, _vp, _vp, _i64, _vp, _vp, _i64, _vp, _i32, _i32, _i32,
                    _i32, _i32, _vp)
_decode_noalloc = _sig("pa_decode_noalloc", _i32, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32,
                       _i32, _i32, _i32, _i32, _i32, _f32, _i32, _i32, _i32, _vp)
_prefill = _sig("pa_prefill", _i32, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _i32, _i32, _i32, _i32,
                _i32, _i32, _i32, _i32, _f32, _i32, _vp)

EXPORTED = ["pa_abi_version", "pa_status_string", "pa_block_layout", "pa_kv_append",
            "pa_decode_plan", "pa_decode_workspace_bytes", "pa_decode", "pa_decode_ex",
            "pa_decode_append", "pa_copy_blocks", "pa_prefill", "pa_swap_blocks",
            "pa_bm_create", "pa_bm_destroy", "pa_bm_can_admit", "pa_bm_admit", "pa_bm_fork",
            "pa_bm_append_slots", "pa_bm_release", "pa_bm_swap_out", "pa_bm_swap_in",
            "pa_bm_decode_inputs", "pa_bm_sequence", "pa_bm_stats", "pa_bm_refcount",
            "pa_kv_append_layered", "pa_decode_layered", "pa_copy_blocks_layered",
            "pa_swap_blocks_layered", "pa_decode_ordered", "pa_decode_shared_prefix",
            "pa_decode_shared_prefix_workspace_bytes", "pa_decode_noalloc",
            "pa_decode_shared_prefix_ordered", "pa_decode_append_ordered"]
MAX_PREFIX_GROUPS = 32


def abi_version() -> int:
    return int(_abi_version())


def _check(status: int, what: str) -> None:
    if status == PA_OK:
        return
    msg = f"{what}: {_status_string(status).decode()}"
    if status == PA_ERR_INVALID_ARG:
        raise ValueError(msg)
    if status == PA_ERR_UNSUPPORTED:
        raise NotImplementedError(msg)
    if status == PA_ERR_NO_SPACE:
        raise NoSpace(msg)
    if status == PA_ERR_SCRATCH:
        raise ScratchTooSmall(msg)
    raise RuntimeError(msg)


class NoSpace(MemoryError):
    """The block pool cannot cover the request (PA_ERR_NO_SPACE): wait or preempt."""


class ScratchTooSmall(ValueError):
    """pa_decode_noalloc: the call needs more workspace than the library's
    static scratch (PA_ERR_SCRATCH); use decode() with a workspace."""


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return PA_F32
    if t.dtype == torch.bfloat16:
        return PA_BF16
    raise ValueError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _dev(t: torch.Tensor, name: str, dtype=None, ndim=None) -> int:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    return t.data_ptr()


def _stream(stream=None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


# --------------------------------------------------------------------------


def block_layout(tokens: int, block_size: int) -> tuple[int, int]:
    """(blocks, unused tail slots) for one unshared sequence; ValueError on bad sizes."""
    b, u = _i64(), _i64()
    _check(_block_layout(int(tokens), int(block_size), ctypes.byref(b), ctypes.byref(u)),
           "block_layout")
    return int(b.value), int(u.value)


def kv_append(k_new, v_new, k_cache, v_cache, slot_mapping, stream=None) -> None:
    """Write new tokens' K/V into the cache slots of ``slot_mapping`` (in place)."""
    dt = _dtype_code(k_cache)
    for name, t in (("v_cache", v_cache), ("k_new", k_new), ("v_new", v_new)):
        if t.dtype != k_cache.dtype:
            raise ValueError(f"{name} dtype {t.dtype} != cache dtype {k_cache.dtype}")
    nb, hkv, bs, d = k_cache.shape
    if tuple(v_cache.shape) != (nb, hkv, bs, d):
        raise ValueError("k_cache and v_cache shapes differ")
    if k_new.dim() != 3 or tuple(k_new.shape[1:]) != (hkv, d) or k_new.shape != v_new.shape:
        raise ValueError("k_new/v_new must be [num_tokens, kv_heads, head_dim]")
    if slot_mapping.dim() != 1 or slot_mapping.shape[0] != k_new.shape[0]:
        raise ValueError("slot_mapping must be [num_tokens]")
    st = _kv_append(_dev(k_new, "k_new"), _dev(v_new, "v_new"), _dev(k_cache, "k_cache", ndim=4),
                    _dev(v_cache, "v_cache", ndim=4), _dev(slot_mapping, "slot_mapping", torch.int64),
                    k_new.shape[0], nb, hkv, bs, d, dt, _stream(stream))
    _check(st, "kv_append")


def copy_blocks(k_cache, v_cache, block_mapping, stream=None) -> None:
    """Copy-on-write: block dst <- block src for each (src, dst) row, both caches."""
    dt = _dtype_code(k_cache)
    nb, hkv, bs, d = k_cache.shape
    if v_cache.shape != k_cache.shape or v_cache.dtype != k_cache.dtype:
        raise ValueError("k_cache and v_cache must match")
    if block_mapping.dim() != 2 or block_mapping.shape[1] != 2:
        raise ValueError("block_mapping must be [num_pairs, 2]")
    st = _copy_blocks(_dev(k_cache, "k_cache", ndim=4), _dev(v_cache, "v_cache", ndim=4),
                      _dev(block_mapping, "block_mapping", torch.int64), block_mapping.shape[0],
                      nb, hkv, bs, d, dt, _stream(stream))
    _check(st, "copy_blocks")


class Plan(NamedTuple):
    kernel: str            # "valu" or "mfma" (split partitions)
    partition_size: int    # tokens per partition
    num_partitions: int    # partitions per sequence (grid extent)
    workspace_bytes: int


def decode_plan(num_seqs, num_heads, kv_heads, head_dim, block_size, max_seq_len,
                partition_size=0, dtype=torch.bfloat16, kernel="auto") -> Plan:
    """The kernel, partition size, grid and workspace the library will use."""
    k, p, n, w = _i32(), _i32(), _i32(), _sz()
    code = PA_BF16 if dtype == torch.bfloat16 else PA_F32
    _check(_decode_plan(num_seqs, num_heads, kv_heads, head_dim, block_size, max_seq_len,
                        partition_size, code, KERNELS[kernel], ctypes.byref(k), ctypes.byref(p),
                        ctypes.byref(n), ctypes.byref(w)), "decode_plan")
    return Plan(KERNEL_NAMES[int(k.value)], int(p.value), int(n.value), int(w.value))


def _decode_common(q, k_cache, v_cache, block_tables, seq_lens, max_seq_len, partition_size,
                   out, workspace, kernel):
    dt = _dtype_code(q)
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise ValueError("q, k_cache and v_cache must share a dtype")
    B, hq, d = q.shape
    nb, hkv, bs, d2 = k_cache.shape
    if d2 != d or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("cache shape does not match q")
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be [num_seqs, max_blocks_per_seq]")
    if seq_lens.dim() != 1 or seq_lens.shape[0] != B:
        raise ValueError("seq_lens must be [num_seqs]")
    if max_seq_len is None:
        max_seq_len = int(seq_lens.max().item()) if B > 0 else 0
    ws_bytes = decode_plan(B, hq, hkv, d, bs, max_seq_len, partition_size, q.dtype,
                           kernel).workspace_bytes
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q")
    if ws_bytes > 0 and workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    ws_ptr = _dev(workspace, "workspace") if workspace is not None else None
    ws_len = workspace.numel() * workspace.element_size() if workspace is not None else 0
    common = (_dev(block_tables, "block_tables", torch.int32), block_tables.shape[1],
              _dev(seq_lens, "seq_lens", torch.int32), int(max_seq_len), B, hq, hkv, d, bs, nb)
    return out, dt, common, ws_ptr, ws_len


def decode(q, k_cache, v_cache, block_tables, seq_lens, scale, max_seq_len=None,
           partition_size=0, out=None, workspace=None, kernel="auto", stream=None):
    """Paged decode attention; returns ``out`` ([num_seqs, num_heads, head_dim], q's dtype).

    ``max_seq_len`` is a host upper bound of ``seq_lens``; when None it is read
    from the device (one synchronising copy).  ``workspace`` (uint8 device
    tensor) is allocated when needed and not given.
    """
    out, dt, common, ws_ptr, ws_len = _decode_common(
        q, k_cache, v_cache, block_tables, seq_lens, max_seq_len, partition_size, out,
        workspace, kernel)
    st = _decode_ex(_dev(out, "out", ndim=3), _dev(q, "q", ndim=3), _dev(k_cache, "k_cache", ndim=4),
                    _dev(v_cache, "v_cache", ndim=4), *common, float(scale), int(partition_size),
                    ws_ptr, ws_len, dt, KERNELS[kernel], _stream(stream))
    _check(st, "decode")
    return out


def decode_noalloc(q, k_cache, v_cache, block_tables, seq_lens, scale, max_seq_len=None,
                   partition_size=0, out=None, kernel="auto", stream=None):
    """decode() through pa_decode_noalloc: no workspace; the library's static
    device scratch holds the partials.  ScratchTooSmall when the plan needs
    more than NOALLOC_SCRATCH_BYTES.  Calls that can overlap on one device
    race (they share the scratch)."""
    B, hq, d = q.shape
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise ValueError("q, k_cache and v_cache must share a dtype")
    nb, hkv, bs, d2 = k_cache.shape
    if d2 != d or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("cache shape does not match q")
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be [num_seqs, max_blocks_per_seq]")
    if seq_lens.dim() != 1 or seq_lens.shape[0] != B:
        raise ValueError("seq_lens must be [num_seqs]")
    if max_seq_len is None:
        max_seq_len = int(seq_lens.max().item()) if B > 0 else 0
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q")
    st = _decode_noalloc(_dev(out, "out", ndim=3), _dev(q, "q", ndim=3),
                         _dev(k_cache, "k_cache", ndim=4), _dev(v_cache, "v_cache", ndim=4),
                         _dev(block_tables, "block_tables", torch.int32), block_tables.shape[1],
                         _dev(seq_lens, "seq_lens", torch.int32), int(max_seq_len), B, hq, hkv, d,
                         bs, nb, float(scale), int(partition_size), _dtype_code(q),
                         KERNELS[kernel], _stream(stream))
    _check(st, "decode_noalloc")
    return out


def longest_first(seq_lens) -> torch.Tensor:
    """A longest-first processing order for pa_decode_ordered (host helper:
    stable sort of the lengths, descending), as an int32 tensor on the lengths'
    device."""
    return torch.sort(seq_lens.to(torch.int64), descending=True, stable=True).indices.to(
        torch.int32)


def longest_tail_first(seq_lens, group_start, group_prefix_blocks, block_size) -> torch.Tensor:
    """A processing order for decode_shared_prefix(order=...): the sequences by
    the length of their tail (positions after their group's shared prefix;
    the whole length outside every group), longest first, stable.  Host
    helper, int32 on the lengths' device."""
    gs, gb, n = _host_groups(group_start, group_prefix_blocks)
    pfx = torch.zeros(seq_lens.shape[0], dtype=torch.int64, device=seq_lens.device)
    for g in range(n):
        pfx[int(gs[g]):int(gs[g + 1])] = int(gb[g]) * int(block_size)
    tails = seq_lens.to(torch.int64) - pfx
    return torch.sort(tails, descending=True, stable=True).indices.to(torch.int32)


def decode_ordered(q, k_cache, v_cache, block_tables, seq_lens, order, scale, max_seq_len=None,
                   partition_size=0, out=None, workspace=None, kernel="auto", stream=None):
    """decode() with a caller-kept processing order (see pa_decode_ordered)."""
    if order.dim() != 1 or order.shape[0] != q.shape[0]:
        raise ValueError("order must be [num_seqs]")
    out, dt, common, ws_ptr, ws_len = _decode_common(
        q, k_cache, v_cache, block_tables, seq_lens, max_seq_len, partition_size, out,
        workspace, kernel)
    bt_ptr, maxblk, sl_ptr, mx, *rest = common
    st = _decode_ordered(_dev(out, "out", ndim=3), _dev(q, "q", ndim=3),
                         _dev(k_cache, "k_cache", ndim=4), _dev(v_cache, "v_cache", ndim=4),
                         bt_ptr, maxblk, sl_ptr, mx, _dev(order, "order", torch.int32), *rest,
                         float(scale), int(partition_size), ws_ptr, ws_len, dt, KERNELS[kernel],
                         _stream(stream))
    _check(st, "decode_ordered")
    return out


def _host_groups(group_start, group_prefix_blocks):
    starts = [int(x) for x in group_start]
    blocks = [int(x) for x in group_prefix_blocks]
    if len(starts) != len(blocks) + 1:
        raise ValueError("group_start needs one entry more than group_prefix_blocks")
    n = len(blocks)
    return ((_i32 * (n + 1))(*starts), (_i32 * max(n, 1))(*(blocks or [0])), n)


def shared_prefix_workspace_bytes(num_seqs, num_heads, kv_heads, head_dim, block_size,
                                  max_seq_len, max_blocks_per_seq, group_start,
                                  group_prefix_blocks, prefix_partition_size=0,
                                  partition_size=0, dtype=torch.bfloat16) -> int:
    """Workspace bytes of decode_shared_prefix (pa_decode_shared_prefix_workspace_bytes)."""
    gs, gb, n = _host_groups(group_start, group_prefix_blocks)
    code = PA_BF16 if dtype == torch.bfloat16 else PA_F32
    return int(_shared_prefix_ws(num_seqs, num_heads, kv_heads, head_dim, block_size, max_seq_len,
                                 max_blocks_per_seq, gs, gb, n, prefix_partition_size,
                                 partition_size, code))


def decode_shared_prefix(q, k_cache, v_cache, block_tables, seq_lens, scale, group_start,
                         group_prefix_blocks, max_seq_len=None, prefix_partition_size=0,
                         partition_size=0, out=None, workspace=None, stream=None, order=None):
    """decode() for a batch whose groups of adjacent sequences share the leading
    blocks of their tables (see pa_decode_shared_prefix).

    ``group_start`` (host ints, length num_groups + 1) delimits the groups;
    ``group_prefix_blocks`` (host ints) gives each group's shared leading
    table entries.  The result equals decode() up to rounding.  ``order``
    (device int32 [num_seqs], optional): the tails' processing order, a
    permutation of the sequences with the longest tail first
    (pa_decode_shared_prefix_ordered; same outputs, faster).
    """
    gs, gb, n = _host_groups(group_start, group_prefix_blocks)
    dt = _dtype_code(q)
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise ValueError("q, k_cache and v_cache must share a dtype")
    B, hq, d = q.shape
    nb, hkv, bs, d2 = k_cache.shape
    if d2 != d or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("cache shape does not match q")
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be [num_seqs, max_blocks_per_seq]")
    if seq_lens.dim() != 1 or seq_lens.shape[0] != B:
        raise ValueError("seq_lens must be [num_seqs]")
    if out is not None and (out.shape != q.shape or out.dtype != q.dtype):
        raise ValueError("out must match q")
    if max_seq_len is None:
        max_seq_len = int(seq_lens.max().item()) if B > 0 else 0
    maxblk = int(block_tables.shape[1])
    ws_bytes = int(_shared_prefix_ws(B, hq, hkv, d, bs, int(max_seq_len), maxblk, gs, gb, n,
                                     int(prefix_partition_size), int(partition_size), dt))
    if out is None:
        out = torch.empty_like(q)
    if ws_bytes > 0 and workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    ws_ptr = _dev(workspace, "workspace") if workspace is not None else None
    ws_len = workspace.numel() * workspace.element_size() if workspace is not None else 0
    head = (_dev(out, "out", ndim=3), _dev(q, "q", ndim=3), _dev(k_cache, "k_cache", ndim=4),
            _dev(v_cache, "v_cache", ndim=4), _dev(block_tables, "block_tables", torch.int32),
            maxblk, _dev(seq_lens, "seq_lens", torch.int32), int(max_seq_len))
    tail = (B, hq, hkv, d, bs, nb, float(scale), gs, gb, n, int(prefix_partition_size),
            int(partition_size), ws_ptr, ws_len, dt, _stream(stream))
    if order is None:
        st = _decode_shared_prefix(*head, *tail)
        _check(st, "decode_shared_prefix")
    else:
        if order.dim() != 1 or order.shape[0] != B:
            raise ValueError("order must be [num_seqs]")
        st = _decode_shared_prefix_ordered(*head, _dev(order, "order", torch.int32), *tail)
        _check(st, "decode_shared_prefix_ordered")
    return out


def decode_append(q, k_cache, v_cache, k_new, v_new, slot_mapping, block_tables, seq_lens, scale,
                  max_seq_len=None, partition_size=0, out=None, workspace=None, kernel="auto",
                  stream=None, order=None):
    """Fused decode step: append one new token per sequence, then decode.

    ``k_new``/``v_new`` are [num_seqs, kv_heads, head_dim]; ``slot_mapping``
    int64 [num_seqs] (< 0: no new token for that sequence); ``seq_lens`` are
    the lengths after the append.  Same result as ``kv_append`` + ``decode``.
    With ``order`` (see longest_first) the call is pa_decode_append_ordered.
    """
    B = q.shape[0]
    if k_new.shape != (B, k_cache.shape[1], q.shape[2]) or v_new.shape != k_new.shape:
        raise ValueError("k_new/v_new must be [num_seqs, kv_heads, head_dim]")
    if k_new.dtype != q.dtype or v_new.dtype != q.dtype:
        raise ValueError("k_new/v_new must have q's dtype")
    if slot_mapping.dim() != 1 or slot_mapping.shape[0] != B:
        raise ValueError("slot_mapping must be [num_seqs]")
    out, dt, common, ws_ptr, ws_len = _decode_common(
        q, k_cache, v_cache, block_tables, seq_lens, max_seq_len, partition_size, out,
        workspace, kernel)
    head = (_dev(out, "out", ndim=3), _dev(q, "q", ndim=3), _dev(k_cache, "k_cache", ndim=4),
            _dev(v_cache, "v_cache", ndim=4), _dev(k_new, "k_new", ndim=3),
            _dev(v_new, "v_new", ndim=3), _dev(slot_mapping, "slot_mapping", torch.int64))
    tail = (float(scale), int(partition_size), ws_ptr, ws_len, dt, KERNELS[kernel],
            _stream(stream))
    if order is None:
        st = _decode_append(*head, *common, *tail)
        _check(st, "decode_append")
        return out
    if order.dim() != 1 or order.shape[0] != B:
        raise ValueError("order must be [num_seqs]")
    bt_ptr, maxblk, sl_ptr, mx, *rest = common
    st = _decode_append_ordered(*head, bt_ptr, maxblk, sl_ptr, mx,
                                _dev(order, "order", torch.int32), *rest, *tail)
    _check(st, "decode_append_ordered")
    return out


def prefill(q, k_cache, v_cache, block_tables, seq_lens, query_start, scale, max_query_len=None,
            out=None, stream=None):
    """Chunked causal prefill over the paged cache (bf16 or float32).

    Sequence s's chunk is rows query_start[s]..query_start[s+1] of ``q``; its
    queries are the last positions of the seq_lens[s] cached ones (their K/V
    already appended) and each attends every position up to its own.
    ``max_query_len`` bounds every chunk (read from ``query_start`` when not
    given, which synchronises with the device).
    """
    dt = _dtype_code(q)
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise ValueError("q, k_cache and v_cache must share a dtype")
    T, hq, d = q.shape
    nb, hkv, bs, d2 = k_cache.shape
    if d2 != d or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("cache shape does not match q")
    B = seq_lens.shape[0] if seq_lens.dim() == 1 else -1
    if B < 0 or block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be [num_seqs, max_blocks_per_seq], seq_lens [num_seqs]")
    if query_start.dim() != 1 or query_start.shape[0] != B + 1:
        raise ValueError("query_start must be [num_seqs + 1]")
    if max_query_len is None:
        max_query_len = int((query_start[1:] - query_start[:-1]).max().item()) if B > 0 else 0
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q")
    st = _prefill(_dev(out, "out", ndim=3), _dev(q, "q", ndim=3), _dev(k_cache, "k_cache", ndim=4),
                  _dev(v_cache, "v_cache", ndim=4), _dev(block_tables, "block_tables", torch.int32),
                  block_tables.shape[1], _dev(seq_lens, "seq_lens", torch.int32),
                  _dev(query_start, "query_start", torch.int32), int(max_query_len), B, T, hq, hkv,
                  d, bs, nb, float(scale), dt, _stream(stream))
    _check(st, "prefill")
    return out


def _ptr_any(t: torch.Tensor, name: str, dtype=None, ndim=None) -> int:
    """Address of a device tensor or of a pinned host tensor."""
    if not isinstance(t, torch.Tensor) or not (t.is_cuda or t.is_pinned()):
        raise ValueError(f"{name} must be a device tensor or pinned host memory")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    return t.data_ptr()


def swap_blocks(dst_k, dst_v, src_k, src_v, block_mapping, stream=None) -> None:
    """Copy whole blocks between pools: device <-> pinned host, or device <-> device.

    Pools are [num_blocks, kv_heads, block_size, head_dim] of one dtype and
    block shape; ``block_mapping`` is int64 [num_pairs, 2] (src, dst), on the
    device or pinned.
    """
    if dst_k.shape[1:] != src_k.shape[1:] or dst_v.shape != dst_k.shape or src_v.shape != src_k.shape:
        raise ValueError("pools must share the block shape")
    if len({dst_k.dtype, dst_v.dtype, src_k.dtype, src_v.dtype}) != 1:
        raise ValueError("pools must share a dtype")
    if block_mapping.dim() != 2 or block_mapping.shape[1] != 2:
        raise ValueError("block_mapping must be [num_pairs, 2]")
    _, hkv, bs, d = src_k.shape
    st = _swap_blocks(_ptr_any(dst_k, "dst_k", ndim=4), _ptr_any(dst_v, "dst_v", ndim=4),
                      dst_k.shape[0], _ptr_any(src_k, "src_k", ndim=4),
                      _ptr_any(src_v, "src_v", ndim=4), src_k.shape[0],
                      _ptr_any(block_mapping, "block_mapping", torch.int64), block_mapping.shape[0],
                      hkv, bs, d, _dtype_code(src_k), _stream(stream))
    _check(st, "swap_blocks")


class BlockManager:
    """Host block bookkeeping (pa_bm_*): admission, sharing, copy-on-write,
    swap, and the decode inputs.  Raises NoSpace when the pool is short."""

    def __init__(self, num_blocks: int, block_size: int, watermark: int = 0,
                 num_host_blocks: int = 0):
        h = _vp()
        _check(_bm_create(int(num_blocks), int(block_size), int(watermark), int(num_host_blocks),
                          ctypes.byref(h)), "bm_create")
        self._h = h
        self._destroy = _bm_destroy   # kept for interpreter shutdown, when globals are gone
        self.block_size = int(block_size)

    def close(self) -> None:
        if getattr(self, "_h", None):
            self._destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    def can_admit(self, prompt_tokens: int) -> bool:
        ok = _i32()
        _check(_bm_can_admit(self._h, int(prompt_tokens), ctypes.byref(ok)), "bm_can_admit")
        return bool(ok.value)

    def admit(self, seq: int, prompt_tokens: int) -> None:
        _check(_bm_admit(self._h, int(seq), int(prompt_tokens)), "bm_admit")

    def fork(self, parent: int, child: int) -> None:
        _check(_bm_fork(self._h, int(parent), int(child)), "bm_fork")

    def append_slots(self, seqs):
        """Returns (slots, cow_pairs) as lists (slots in batch order)."""
        seqs = [int(x) for x in seqs]
        n = len(seqs)
        arr = (_i64 * max(n, 1))(*seqs)
        slots = (_i64 * max(n, 1))()
        cow = (_i64 * max(2 * n, 2))()
        ncow = _i32()
        _check(_bm_append_slots(self._h, arr, n, slots, cow, ctypes.byref(ncow)), "bm_append_slots")
        return list(slots[:n]), [(cow[2 * i], cow[2 * i + 1]) for i in range(ncow.value)]

    def release(self, seq: int) -> None:
        _check(_bm_release(self._h, int(seq)), "bm_release")

    def _swap(self, fn, seq, what):
        _, nblocks, _ = self.sequence(seq)
        pairs = (_i64 * max(2 * nblocks, 2))()
        n = _i64()
        _check(fn(self._h, int(seq), pairs, nblocks, ctypes.byref(n)), what)
        return [(pairs[2 * i], pairs[2 * i + 1]) for i in range(n.value)]

    def swap_out(self, seq: int):
        """(device, host) block pairs for pa_swap_blocks."""
        return self._swap(_bm_swap_out, seq, "bm_swap_out")

    def swap_in(self, seq: int):
        """(host, device) block pairs for pa_swap_blocks."""
        return self._swap(_bm_swap_in, seq, "bm_swap_in")

    def decode_inputs(self, seqs, max_blocks: int, pad_block: int):
        """(tables [n][max_blocks], seq_lens [n]) as nested lists."""
        seqs = [int(x) for x in seqs]
        n = len(seqs)
        arr = (_i64 * max(n, 1))(*seqs)
        tables = (_i32 * max(n * max_blocks, 1))()
        lens = (_i32 * max(n, 1))()
        _check(_bm_decode_inputs(self._h, arr, n, int(max_blocks), int(pad_block), tables, lens),
               "bm_decode_inputs")
        return ([list(tables[i * max_blocks:(i + 1) * max_blocks]) for i in range(n)],
                list(lens[:n]))

    def sequence(self, seq: int):
        """(cached length, number of blocks, swapped out?)"""
        ln, nb, sw = _i64(), _i64(), _i32()
        _check(_bm_sequence(self._h, int(seq), ctypes.byref(ln), ctypes.byref(nb),
                            ctypes.byref(sw)), "bm_sequence")
        return ln.value, nb.value, bool(sw.value)

    def stats(self):
        """(free device blocks, free host blocks, sequences)"""
        a, b, c = _i64(), _i64(), _i64()
        _check(_bm_stats(self._h, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)), "bm_stats")
        return a.value, b.value, c.value

    def free_blocks(self) -> int:
        return self.stats()[0]

    def free_host_blocks(self) -> int:
        return self.stats()[1]

    def refcount(self, block: int, host: bool = False) -> int:
        r = _i32()
        _check(_bm_refcount(self._h, int(block), int(host), ctypes.byref(r)), "bm_refcount")
        return r.value


# ---- layered pool: [num_blocks, 2, num_layers, kv_heads, block_size, head_dim] ----

def _pool_dims(kv_pool):
    if kv_pool.dim() != 6 or kv_pool.shape[1] != 2:
        raise ValueError("kv_pool must be [num_blocks, 2, num_layers, kv_heads, block_size, head_dim]")
    nb, _, nl, hkv, bs, d = kv_pool.shape
    return nb, nl, hkv, bs, d


def kv_append_layered(k_new, v_new, kv_pool, layer, slot_mapping, stream=None) -> None:
    """Append layer ``layer``'s new rows ([num_tokens, kv_heads, head_dim]) into a layered pool."""
    nb, nl, hkv, bs, d = _pool_dims(kv_pool)
    if k_new.shape != v_new.shape or k_new.dim() != 3 or k_new.shape[1:] != (hkv, d):
        raise ValueError("k_new/v_new must be [num_tokens, kv_heads, head_dim]")
    if k_new.dtype != kv_pool.dtype or v_new.dtype != kv_pool.dtype:
        raise ValueError("dtype mismatch")
    if slot_mapping.dim() != 1 or slot_mapping.shape[0] != k_new.shape[0]:
        raise ValueError("slot_mapping must be [num_tokens]")
    _check(_kv_append_layered(_dev(k_new, "k_new"), _dev(v_new, "v_new"), _dev(kv_pool, "kv_pool"),
                              int(layer), nl, _dev(slot_mapping, "slot_mapping", torch.int64),
                              k_new.shape[0], nb, hkv, bs, d, _dtype_code(kv_pool), _stream(stream)),
           "kv_append_layered")


def decode_layered(q, kv_pool, block_tables, seq_lens, scale, first_layer=0, max_seq_len=None,
                   partition_size=0, out=None, workspace=None, stream=None):
    """Decode q [layers, num_seqs, num_heads, head_dim] over layers
    first_layer .. first_layer + layers - 1 of a layered pool, in one launch."""
    nb, nl, hkv, bs, d = _pool_dims(kv_pool)
    if q.dim() != 4 or q.shape[3] != d:
        raise ValueError("q must be [layers, num_seqs, num_heads, head_dim]")
    L, B, hq, _ = q.shape
    if q.dtype != kv_pool.dtype:
        raise ValueError("q and kv_pool must share a dtype")
    if block_tables.dim() != 2 or block_tables.shape[0] != B or seq_lens.shape != (B,):
        raise ValueError("block_tables [num_seqs, max_blocks], seq_lens [num_seqs]")
    if max_seq_len is None:
        max_seq_len = int(seq_lens.max().item()) if B > 0 else 0
    ws = decode_plan(B, hq, hkv, d, bs, max_seq_len, partition_size, q.dtype,
                     "auto").workspace_bytes * L
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q")
    if ws > 0 and workspace is None:
        workspace = torch.empty(ws, dtype=torch.uint8, device=q.device)
    ws_ptr = _dev(workspace, "workspace") if workspace is not None else None
    ws_len = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(_decode_layered(_dev(out, "out"), _dev(q, "q"), _dev(kv_pool, "kv_pool"),
                           int(first_layer), L, nl, _dev(block_tables, "block_tables", torch.int32),
                           block_tables.shape[1], _dev(seq_lens, "seq_lens", torch.int32),
                           int(max_seq_len), B, hq, hkv, d, bs, nb, float(scale),
                           int(partition_size), ws_ptr, ws_len, _dtype_code(q), _stream(stream)),
           "decode_layered")
    return out


def copy_blocks_layered(kv_pool, block_mapping, stream=None) -> None:
    nb, nl, hkv, bs, d = _pool_dims(kv_pool)
    if block_mapping.dim() != 2 or block_mapping.shape[1] != 2:
        raise ValueError("block_mapping must be [num_pairs, 2]")
    _check(_copy_blocks_layered(_dev(kv_pool, "kv_pool"),
                                _dev(block_mapping, "block_mapping", torch.int64),
                                block_mapping.shape[0], nb, nl, hkv, bs, d, _dtype_code(kv_pool),
                                _stream(stream)), "copy_blocks_layered")


def swap_blocks_layered(dst_pool, src_pool, block_mapping, stream=None) -> None:
    """Whole layered blocks between a device pool and a pinned host pool (either way)."""
    dnb, nl, hkv, bs, d = _pool_dims(dst_pool)
    snb, nl2, hkv2, bs2, d2 = _pool_dims(src_pool)
    if (nl, hkv, bs, d) != (nl2, hkv2, bs2, d2) or dst_pool.dtype != src_pool.dtype:
        raise ValueError("pools must share the block shape and dtype")
    if block_mapping.dim() != 2 or block_mapping.shape[1] != 2:
        raise ValueError("block_mapping must be [num_pairs, 2]")
    _check(_swap_blocks_layered(_ptr_any(dst_pool, "dst_pool"), dnb, _ptr_any(src_pool, "src_pool"),
                                snb, _ptr_any(block_mapping, "block_mapping", torch.int64),
                                block_mapping.shape[0], nl, hkv, bs, d, _dtype_code(src_pool),
                                _stream(stream)), "swap_blocks_layered")
