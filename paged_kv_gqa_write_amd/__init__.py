"""Grouped-query attention over a paged KV cache on AMD Instinct MI355X.

Thin ctypes binding of the C ABI in include/pa.h (libpa.so, built by
paged_kv_gqa_write_amd/build.py).  PyTorch supplies device memory and the
current HIP stream; every step of the computation runs in the library's HIP
kernels.  There is no fallback: if the library is missing, every call
raises.

Pool layout (see include/pa.h):
  k_cache [num_blocks, Hkv, D/32, 16, 32] bf16 (element d of the K row of
  in-block offset o at [b, g, d // 32, o, d % 32]),
  v_cache [num_blocks, Hkv, D, 16] bf16.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "PAError", "load_library", "library_path", "write_kv", "decode", "decode_partials",
    "decode_reduce", "decode_append", "decode_multi", "decode_multi_partials", "decode_multi_reduce", "prefill",
    "copy_blocks", "PrefixIndex", "decode_split_plan", "decode_split_plan_lens",
    "decode_multi_split_plan", "decode_noalloc", "status_string", "EXPORTED_SYMBOLS",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libpa.so")
_lib = None

BLOCK_SIZE = 16
PA_OK, PA_ERR_INVALID_ARG, PA_ERR_UNSUPPORTED, PA_ERR_LAUNCH, PA_ERR_NO_MEMORY = 0, -1, -2, -3, -4
PA_ERR_TOO_LARGE = -5

_vp, _i32, _i64, _f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
_pi32 = ctypes.POINTER(ctypes.c_int32)
_pvp = ctypes.POINTER(ctypes.c_void_p)

# name -> (restype, argtypes); mirrors include/pa.h
_SIGNATURES = {
    "pa_write_kv": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i64, _vp]),
    "pa_decode": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                 _i32, _i64, _i32, _i32, _i32, _f32, _vp]),
    "pa_decode_reduce": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _vp]),
    "pa_decode_noalloc": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                         _i32, _i64, _i32, _i32, _i32, _f32, _vp]),
    "pa_decode_append": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32,
                                        _i32, _i32, _i32, _i32, _i64, _i32, _i32, _i32, _f32,
                                        _vp]),
    "pa_decode_multi": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32,
                                       _i32, _i32, _i32, _i64, _i32, _i32, _i32, _f32, _vp]),
    "pa_decode_multi_reduce": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                              _i32, _vp]),
    "pa_prefill": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                  _i32, _i32, _i32, _i64, _i32, _f32, _vp]),
    "pa_copy_blocks": (ctypes.c_int, [_vp, _vp, _i64, _vp, _vp, _vp, _i64, _vp, _i32, _i32, _i32,
                                      _i32, _vp]),
    "pa_decode_split_plan": (ctypes.c_int, [_i32, _i32, _i32, _i32, _pi32, _pi32]),
    "pa_decode_split_plan_lens": (ctypes.c_int, [_i32, _i32, _vp, _i32, _pi32, _pi32]),
    "pa_decode_multi_split_plan": (ctypes.c_int, [_i32, _i32, _i32, _i32, _i32, _i32, _pi32,
                                                  _pi32]),
    "pa_prefix_index_create": (ctypes.c_int, [_i64, _pvp]),
    "pa_prefix_index_destroy": (None, [_vp]),
    "pa_prefix_index_size": (ctypes.c_int64, [_vp]),
    "pa_prefix_index_match": (ctypes.c_int, [_vp, _vp, _i32, _vp, _pi32]),
    "pa_prefix_index_insert": (ctypes.c_int, [_vp, _vp, _i32, _vp, _i32, _pi32]),
    "pa_prefix_index_remove": (ctypes.c_int, [_vp, _i32, _pi32]),
    "pa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
}
EXPORTED_SYMBOLS = tuple(_SIGNATURES)


class PAError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_string(status)} ({status})")
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def load_library(path: str | None = None):
    """Load libpa.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or _LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(
            f"HIP library not found at {p}; build it with "
            "`python -m paged_kv_gqa_write_amd.build` (there is no fallback path)")
    lib = ctypes.CDLL(p)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().pa_status_string(int(status)).decode()


def _check(status: int, where: str):
    if status != PA_OK:
        raise PAError(status, where)


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _need(t: torch.Tensor, name: str, dtype, ndim: int | None = None):
    """Type, dtype, rank and contiguity of an argument.  Where it lives is
    checked separately (_on_gpu), after every shape check of the call."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _need_shape(t, name: str, dtype, shape):
    """A caller-supplied output or workspace (None: not given) must have
    exactly the shape the kernels write: a larger one would be only partly
    written, a smaller one overrun."""
    if t is None:
        return
    _need(t, name, dtype, len(shape))
    if tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError(f"{name} must have shape {tuple(int(x) for x in shape)}, "
                         f"got {tuple(t.shape)}")


def _on_gpu(*tensors):
    """Every given tensor (None skipped) is GPU memory of one device; returns
    that device."""
    dev = None
    for t in tensors:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("every tensor argument must be a GPU tensor")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"tensors on different devices: {dev} and {t.device}")
    return dev


def _pools(k_cache, v_cache):
    _need(k_cache, "k_cache", torch.bfloat16, 5)
    _need(v_cache, "v_cache", torch.bfloat16, 4)
    nb, hkv, ns, bs, w = k_cache.shape
    d = ns * w
    if bs != BLOCK_SIZE or w != 32 or tuple(v_cache.shape) != (nb, hkv, d, BLOCK_SIZE):
        raise ValueError("pools must be K [NB, Hkv, D/32, 16, 32] and V [NB, Hkv, D, 16]; "
                         f"got {tuple(k_cache.shape)} and {tuple(v_cache.shape)}")
    return nb, hkv, d


def write_kv(k_new, v_new, slot_mapping, k_cache, v_cache):
    """Write each token's K/V into its slot (slot < 0: skipped)."""
    nb, hkv, d = _pools(k_cache, v_cache)
    _need(k_new, "k_new", torch.bfloat16, 3)
    _need(v_new, "v_new", torch.bfloat16, 3)
    _need(slot_mapping, "slot_mapping", torch.int64, 1)
    T = k_new.shape[0]
    if tuple(k_new.shape) != (T, hkv, d) or tuple(v_new.shape) != (T, hkv, d) \
            or slot_mapping.shape[0] != T:
        raise ValueError("k_new/v_new must be [T, Hkv, D] and slot_mapping [T]")
    _on_gpu(k_new, v_new, slot_mapping, k_cache, v_cache)
    st = load_library().pa_write_kv(k_new.data_ptr(), v_new.data_ptr(), slot_mapping.data_ptr(),
                                    k_cache.data_ptr(), v_cache.data_ptr(), T, hkv, d,
                                    BLOCK_SIZE, nb, _stream(k_cache.device))
    _check(st, "pa_write_kv")


def decode_split_plan(num_seqs: int, num_kv_heads: int, max_context_len: int,
                      num_compute_units: int | None = None):
    """(partition_size, num_partitions) from the library's host heuristic."""
    if num_compute_units is None:
        num_compute_units = torch.cuda.get_device_properties(0).multi_processor_count
    ps, npart = ctypes.c_int32(0), ctypes.c_int32(0)
    st = load_library().pa_decode_split_plan(int(num_seqs), int(num_kv_heads),
                                             int(max_context_len), int(num_compute_units),
                                             ctypes.byref(ps), ctypes.byref(npart))
    _check(st, "pa_decode_split_plan")
    return ps.value, npart.value


def decode_split_plan_lens(num_kv_heads: int, context_lens,
                           num_compute_units: int | None = None):
    """(partition_size, num_partitions) from the batch's actual context
    lengths (a host sequence of ints): long sequences of a mixed batch get
    more partitions (pa_decode_split_plan_lens)."""
    import numpy as np
    if isinstance(context_lens, torch.Tensor):
        if context_lens.is_cuda:
            raise ValueError("context_lens for the host plan must be host memory")
        context_lens = context_lens.numpy()
    lens = np.ascontiguousarray(np.asarray(context_lens, dtype=np.int64).astype(np.int32))
    if num_compute_units is None:
        num_compute_units = torch.cuda.get_device_properties(0).multi_processor_count
    ps, npart = ctypes.c_int32(0), ctypes.c_int32(0)
    st = load_library().pa_decode_split_plan_lens(int(lens.size), int(num_kv_heads),
                                                  lens.ctypes.data if lens.size else None,
                                                  int(num_compute_units), ctypes.byref(ps),
                                                  ctypes.byref(npart))
    _check(st, "pa_decode_split_plan_lens")
    return ps.value, npart.value


def decode_multi_split_plan(num_seqs: int, query_len: int, num_q_heads: int, num_kv_heads: int,
                            max_context_len: int, num_compute_units: int | None = None):
    """(partition_size, num_partitions) for decode_multi from the library's host heuristic."""
    if num_compute_units is None:
        num_compute_units = torch.cuda.get_device_properties(0).multi_processor_count
    ps, npart = ctypes.c_int32(0), ctypes.c_int32(0)
    st = load_library().pa_decode_multi_split_plan(
        int(num_seqs), int(query_len), int(num_q_heads), int(num_kv_heads), int(max_context_len),
        int(num_compute_units), ctypes.byref(ps), ctypes.byref(npart))
    _check(st, "pa_decode_multi_split_plan")
    return ps.value, npart.value


def _plan(B, T, hq, hkv, context_lens, max_context_len, partition_size, num_partitions):
    """The split-K plan of a decode call: the library's heuristic unless the
    caller gives a partition size (then enough partitions to cover the
    longest context)."""
    if partition_size is not None and num_partitions is not None:
        return int(partition_size), int(num_partitions)
    if max_context_len is None:
        max_context_len = int(context_lens.max().item()) if B > 0 else 0
    if partition_size is None:
        if T == 1:
            return decode_split_plan(B, hkv, max_context_len)
        return decode_multi_split_plan(B, T, hq, hkv, max_context_len)
    return int(partition_size), max(1, -(-max_context_len // int(partition_size)))


def _decode_checks(q, k_cache, v_cache, block_tables, context_lens, T, out, part_out, part_lse,
                   num_partitions, k_new=None, v_new=None):
    """Shapes of a decode call's inputs and of the buffers it writes; returns
    (B, Hq, Hkv, D, num_blocks).  T = 0: q is [B, Hq, D] (one query token);
    otherwise q is [B, T, Hq, D]."""
    nb, hkv, d = _pools(k_cache, v_cache)
    _need(q, "q", torch.bfloat16, 3 if T == 0 else 4)
    _need(block_tables, "block_tables", torch.int32, 2)
    _need(context_lens, "context_lens", torch.int32, 1)
    if T == 0:
        B, hq, dq = q.shape
        lead = (B,)
    else:
        B, Tq, hq, dq = q.shape
        if Tq != T:
            raise ValueError(f"q must be [B, {T}, Hq, D], got {tuple(q.shape)}")
        lead = (B, T)
    if dq != d or block_tables.shape[0] != B or context_lens.shape[0] != B:
        raise ValueError("q [B, (T,) Hq, D], block_tables [B, max_blocks], context_lens [B] "
                         "mismatch")
    if hq % hkv != 0:
        raise ValueError(f"num_q_heads {hq} is not a multiple of num_kv_heads {hkv}")
    if k_new is not None:
        _need_shape(k_new, "k_new", torch.bfloat16, (B, hkv, d))
        _need_shape(v_new, "v_new", torch.bfloat16, (B, hkv, d))
    P = int(num_partitions)
    if P < 1:
        raise ValueError("num_partitions must be >= 1")
    if P == 1:
        if out is None:
            raise ValueError("out is required with one partition")
        _need_shape(out, "out", torch.bfloat16, (*lead, hq, d))
    else:
        if part_out is None or part_lse is None:
            raise ValueError("part_out and part_lse are required with more than one partition")
        _need_shape(part_out, "part_out", torch.float32, (*lead, hq, P, d))
        _need_shape(part_lse, "part_lse", torch.float32, (*lead, hq, P))
        _need_shape(out, "out", torch.bfloat16, (*lead, hq, d))
    _on_gpu(q, k_cache, v_cache, block_tables, context_lens, k_new, v_new, out, part_out,
            part_lse)
    return B, hq, hkv, d, nb


def _ptr(t):
    return 0 if t is None else t.data_ptr()


def _decode_call(out, part_out, part_lse, q, k_cache, v_cache, block_tables, context_lens,
                 scale, partition_size, num_partitions):
    B, hq, hkv, d, nb = _decode_checks(q, k_cache, v_cache, block_tables, context_lens, 0, out,
                                       part_out, part_lse, num_partitions)
    P = int(num_partitions)
    st = load_library().pa_decode(_ptr(out) if P == 1 else 0, _ptr(part_out), _ptr(part_lse),
                                  q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                  block_tables.data_ptr(), context_lens.data_ptr(), B, hq, hkv, d,
                                  BLOCK_SIZE, nb, block_tables.shape[1], int(partition_size), P,
                                  float(scale), _stream(q.device))
    _check(st, "pa_decode")


def _workspace(q, lead, hq, P, d, part_out, part_lse):
    if part_out is None:
        part_out = torch.empty(*lead, hq, P, d, dtype=torch.float32, device=q.device)
    if part_lse is None:
        part_lse = torch.empty(*lead, hq, P, dtype=torch.float32, device=q.device)
    return part_out, part_lse


def decode_partials(q, k_cache, v_cache, block_tables, context_lens, scale, partition_size,
                    num_partitions, part_out=None, part_lse=None):
    """Split-K pieces only (num_partitions > 1): (part_out [B,Hq,P,D], part_lse [B,Hq,P])."""
    if int(num_partitions) < 2:
        raise ValueError("decode_partials needs num_partitions > 1")
    _need(q, "q", torch.bfloat16, 3)
    B, hq, d = q.shape
    part_out, part_lse = _workspace(q, (B,), hq, int(num_partitions), d, part_out, part_lse)
    _decode_call(None, part_out, part_lse, q, k_cache, v_cache, block_tables, context_lens,
                 scale, partition_size, num_partitions)
    return part_out, part_lse


def _reduce_checks(part_out, part_lse, context_lens, out, T):
    _need(part_out, "part_out", torch.float32, 4 if T == 0 else 5)
    if T == 0:
        B, hq, P, d = part_out.shape
        lead = (B,)
    else:
        B, Tq, hq, P, d = part_out.shape
        lead = (B, Tq)
    if part_lse is None:
        raise ValueError("part_lse is required")
    _need_shape(part_lse, "part_lse", torch.float32, (*lead, hq, P))
    if context_lens is not None:
        _need_shape(context_lens, "context_lens", torch.int32, (B,))
    _need_shape(out, "out", torch.bfloat16, (*lead, hq, d))
    _on_gpu(part_out, part_lse, context_lens, out)
    return lead, hq, P, d


def decode_reduce(part_out, part_lse, context_lens, partition_size, out=None):
    """Log-sum-exp combine of split-K pieces into bf16 [B, Hq, D]."""
    lead, hq, P, d = _reduce_checks(part_out, part_lse, context_lens, out, 0)
    if out is None:
        out = torch.empty(*lead, hq, d, dtype=torch.bfloat16, device=part_out.device)
    st = load_library().pa_decode_reduce(out.data_ptr(), part_out.data_ptr(), part_lse.data_ptr(),
                                         _ptr(context_lens), lead[0], hq, d,
                                         int(partition_size), P, _stream(part_out.device))
    _check(st, "pa_decode_reduce")
    return out


def decode(q, k_cache, v_cache, block_tables, context_lens, scale, *, max_context_len=None,
           partition_size=None, num_partitions=None, out=None, part_out=None, part_lse=None):
    """Decode attention, one query token per sequence -> bf16 [B, Hq, D].

    The split-K plan comes from the library heuristic unless given; with more
    than one partition the pieces are combined by pa_decode_reduce.  Given
    out / part_out / part_lse must have exactly the shapes written."""
    _need(q, "q", torch.bfloat16, 3)
    B, hq, d = q.shape
    ps, P = _plan(B, 1, hq, k_cache.shape[1], context_lens, max_context_len, partition_size,
                  num_partitions)
    _need_shape(out, "out", torch.bfloat16, (B, hq, d))
    if out is None:
        out = torch.empty(B, hq, d, dtype=torch.bfloat16, device=q.device)
    if P == 1:
        _decode_call(out, None, None, q, k_cache, v_cache, block_tables, context_lens, scale,
                     ps, 1)
        return out
    part_out, part_lse = decode_partials(q, k_cache, v_cache, block_tables, context_lens, scale,
                                         ps, P, part_out, part_lse)
    return decode_reduce(part_out, part_lse, context_lens, ps, out=out)


def decode_noalloc(q, k_cache, v_cache, block_tables, context_lens, scale, partition_size,
                   num_partitions, out=None):
    """Decode (+ the reduce when num_partitions > 1) with the split-K pieces in
    the library's static per-GPU scratch instead of a workspace: nothing is
    allocated by the library (pa_decode_noalloc).  Calls that overlap on one
    GPU race on that scratch.  -> bf16 [B, Hq, D]"""
    _need(q, "q", torch.bfloat16, 3)
    B, hq, d = q.shape
    _need_shape(out, "out", torch.bfloat16, (B, hq, d))
    if out is None:
        out = torch.empty(B, hq, d, dtype=torch.bfloat16, device=q.device)
    B, hq, hkv, d, nb = _decode_checks(q, k_cache, v_cache, block_tables, context_lens, 0, out,
                                       None, None, 1)
    st = load_library().pa_decode_noalloc(out.data_ptr(), q.data_ptr(), k_cache.data_ptr(),
                                          v_cache.data_ptr(), block_tables.data_ptr(),
                                          context_lens.data_ptr(), B, hq, hkv, d, BLOCK_SIZE, nb,
                                          block_tables.shape[1], int(partition_size),
                                          int(num_partitions), float(scale), _stream(q.device))
    _check(st, "pa_decode_noalloc")
    return out


def decode_append(q, k_new, v_new, k_cache, v_cache, block_tables, context_lens, scale, *,
                  max_context_len=None, partition_size=None, num_partitions=None, out=None,
                  part_out=None, part_lse=None):
    """Append each sequence's new token (k_new/v_new [B, Hkv, D], position
    ctx-1, slot from the block table) and decode, in one kernel; with more
    than one partition the pieces are combined by pa_decode_reduce."""
    _need(q, "q", torch.bfloat16, 3)
    B, hq, d = q.shape
    ps, P = _plan(B, 1, hq, k_cache.shape[1], context_lens, max_context_len, partition_size,
                  num_partitions)
    _need_shape(out, "out", torch.bfloat16, (B, hq, d))
    if out is None:
        out = torch.empty(B, hq, d, dtype=torch.bfloat16, device=q.device)
    if P > 1:
        part_out, part_lse = _workspace(q, (B,), hq, P, d, part_out, part_lse)
    else:
        part_out = part_lse = None
    B, hq, hkv, d, nb = _decode_checks(q, k_cache, v_cache, block_tables, context_lens, 0, out,
                                       part_out, part_lse, P, k_new, v_new)
    st = load_library().pa_decode_append(
        _ptr(out), _ptr(part_out), _ptr(part_lse), q.data_ptr(), k_new.data_ptr(),
        v_new.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), block_tables.data_ptr(),
        context_lens.data_ptr(), B, hq, hkv, d, BLOCK_SIZE, nb, block_tables.shape[1], ps, P,
        float(scale), _stream(q.device))
    _check(st, "pa_decode_append")
    if P == 1:
        return out
    return decode_reduce(part_out, part_lse, context_lens, ps, out=out)


def prefill(q, k_cache, v_cache, block_tables, cu_seqlens, prefix_lens, scale, max_q_len,
            out=None):
    """Varlen causal prefill with cached prefixes -> bf16 [total_q, Hq, D].

    max_q_len is a host-side upper bound of the per-sequence new-token count."""
    nb, hkv, d = _pools(k_cache, v_cache)
    _need(q, "q", torch.bfloat16, 3)
    _need(block_tables, "block_tables", torch.int32, 2)
    _need(cu_seqlens, "cu_seqlens", torch.int32, 1)
    S = cu_seqlens.shape[0] - 1
    if prefix_lens is not None:
        _need_shape(prefix_lens, "prefix_lens", torch.int32, (S,))
    total_q, hq, dq = q.shape
    if dq != d or block_tables.shape[0] != S:
        raise ValueError("q [total_q, Hq, D] / block_tables [S, max_blocks] mismatch")
    if hq % hkv != 0:
        raise ValueError(f"num_q_heads {hq} is not a multiple of num_kv_heads {hkv}")
    _need_shape(out, "out", torch.bfloat16, (total_q, hq, d))
    _on_gpu(q, k_cache, v_cache, block_tables, cu_seqlens, prefix_lens, out)
    if out is None:
        out = torch.empty_like(q)
    st = load_library().pa_prefill(out.data_ptr(), q.data_ptr(), k_cache.data_ptr(),
                                   v_cache.data_ptr(), block_tables.data_ptr(),
                                   cu_seqlens.data_ptr(), _ptr(prefix_lens),
                                   S, total_q, int(max_q_len), hq, hkv, d, BLOCK_SIZE, nb,
                                   block_tables.shape[1], float(scale), _stream(q.device))
    _check(st, "pa_prefill")
    return out


# ---------------------------------------------------------------------------
# Several query tokens per sequence (verifying a block of drafted tokens)
# ---------------------------------------------------------------------------

def _decode_multi_call(out, part_out, part_lse, q, k_cache, v_cache, block_tables, context_lens,
                       scale, partition_size, num_partitions):
    _need(q, "q", torch.bfloat16, 4)
    T = q.shape[1]
    B, hq, hkv, d, nb = _decode_checks(q, k_cache, v_cache, block_tables, context_lens, T, out,
                                       part_out, part_lse, num_partitions)
    P = int(num_partitions)
    st = load_library().pa_decode_multi(_ptr(out) if P == 1 else 0, _ptr(part_out),
                                        _ptr(part_lse), q.data_ptr(), k_cache.data_ptr(),
                                        v_cache.data_ptr(), block_tables.data_ptr(),
                                        context_lens.data_ptr(), B, T, hq, hkv, d, BLOCK_SIZE, nb,
                                        block_tables.shape[1], int(partition_size), P,
                                        float(scale), _stream(q.device))
    _check(st, "pa_decode_multi")


def decode_multi_partials(q, k_cache, v_cache, block_tables, context_lens, scale,
                          partition_size, num_partitions, part_out=None, part_lse=None):
    """Split-K pieces of a multi-token decode (num_partitions > 1):
    (part_out [B, T, Hq, P, D], part_lse [B, T, Hq, P])."""
    if int(num_partitions) < 2:
        raise ValueError("decode_multi_partials needs num_partitions > 1")
    _need(q, "q", torch.bfloat16, 4)
    B, T, hq, d = q.shape
    part_out, part_lse = _workspace(q, (B, T), hq, int(num_partitions), d, part_out, part_lse)
    _decode_multi_call(None, part_out, part_lse, q, k_cache, v_cache, block_tables,
                       context_lens, scale, partition_size, num_partitions)
    return part_out, part_lse


def decode_multi_reduce(part_out, part_lse, context_lens, partition_size, out=None):
    """Log-sum-exp combine of multi-token split-K pieces into bf16 [B, T, Hq, D]."""
    lead, hq, P, d = _reduce_checks(part_out, part_lse, context_lens, out, 1)
    B, T = lead
    if out is None:
        out = torch.empty(B, T, hq, d, dtype=torch.bfloat16, device=part_out.device)
    st = load_library().pa_decode_multi_reduce(
        out.data_ptr(), part_out.data_ptr(), part_lse.data_ptr(), _ptr(context_lens), B, T, hq,
        d, int(partition_size), P, _stream(part_out.device))
    _check(st, "pa_decode_multi_reduce")
    return out


def decode_multi(q, k_cache, v_cache, block_tables, context_lens, scale, *,
                 max_context_len=None, partition_size=None, num_partitions=None, out=None,
                 part_out=None, part_lse=None):
    """Decode attention with T query tokens per sequence -> bf16 [B, T, Hq, D].

    context_lens counts every cached token including the T query tokens
    (whose K/V are already in the pool); token t sits at position
    ctx - T + t and sees keys 0..ctx - T + t."""
    _need(q, "q", torch.bfloat16, 4)
    B, T, hq, d = q.shape
    ps, P = _plan(B, T, hq, k_cache.shape[1], context_lens, max_context_len, partition_size,
                  num_partitions)
    _need_shape(out, "out", torch.bfloat16, (B, T, hq, d))
    if out is None:
        out = torch.empty(B, T, hq, d, dtype=torch.bfloat16, device=q.device)
    if P == 1:
        _decode_multi_call(out, None, None, q, k_cache, v_cache, block_tables, context_lens,
                           scale, ps, 1)
        return out
    part_out, part_lse = decode_multi_partials(q, k_cache, v_cache, block_tables, context_lens,
                                               scale, ps, P, part_out, part_lse)
    return decode_multi_reduce(part_out, part_lse, context_lens, ps, out=out)


# ---------------------------------------------------------------------------
# Block-granular copy (host-tier restore / save, duplicating a shared block)
# ---------------------------------------------------------------------------

def _reachable(t: torch.Tensor, name: str, dtype, ndim: int):
    """A GPU tensor or a pinned host tensor (the kernel reaches pinned host
    memory through its device mapping); contiguous, of the given dtype."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if not (t.is_cuda or t.is_pinned()):
        raise ValueError(f"{name} must be a GPU tensor or pinned host memory")


def copy_blocks(dst_k, dst_v, src_k, src_v, dst_ids=None, src_ids=None, num_copies=None):
    """Copy whole blocks: dst block dst_ids[i] := src block src_ids[i] for K
    and V (ids None: blocks 0..n-1, a packed run).  Either side may be a GPU
    pool or pinned host memory in the pool layout.  Runs on the current
    stream of the GPU in use."""
    for t, n in ((dst_k, "dst_k"), (src_k, "src_k")):
        _reachable(t, n, torch.bfloat16, 5)
    for t, n in ((dst_v, "dst_v"), (src_v, "src_v")):
        _reachable(t, n, torch.bfloat16, 4)
    dnb, hkv, ns, bs, w = dst_k.shape
    d = ns * w
    snb = src_k.shape[0]
    if bs != BLOCK_SIZE or w != 32 or tuple(src_k.shape[1:]) != (hkv, ns, bs, w) \
            or tuple(dst_v.shape) != (dnb, hkv, d, bs) or tuple(src_v.shape) != (snb, hkv, d, bs):
        raise ValueError("pools must be K [NB, Hkv, D/32, 16, 32] and V [NB, Hkv, D, 16] "
                         "on both sides")
    for t, n in ((dst_ids, "dst_ids"), (src_ids, "src_ids")):
        if t is not None:
            _reachable(t, n, torch.int32, 1)
    if num_copies is None:
        given = [t.shape[0] for t in (dst_ids, src_ids) if t is not None]
        num_copies = given[0] if given else min(dnb, snb)
    for t, n in ((dst_ids, "dst_ids"), (src_ids, "src_ids")):
        if t is not None and t.shape[0] < num_copies:
            raise ValueError(f"{n} holds fewer than num_copies ids")
    dev = next((t.device for t in (dst_k, src_k) if t.is_cuda), torch.device("cuda"))
    ptr = lambda t: 0 if t is None else t.data_ptr()  # noqa: E731
    st = load_library().pa_copy_blocks(dst_k.data_ptr(), dst_v.data_ptr(), dnb, ptr(dst_ids),
                                       src_k.data_ptr(), src_v.data_ptr(), snb, ptr(src_ids),
                                       int(num_copies), hkv, d, BLOCK_SIZE, _stream(dev))
    _check(st, "pa_copy_blocks")


# ---------------------------------------------------------------------------
# Prefix-block index (host side of the prefix cache; CPU only)
# ---------------------------------------------------------------------------

class PrefixIndex:
    """The library's host-side prefix-block index (pa_prefix_index_*).

    match(tokens) -> physical block ids of the longest cached run of leading
    full blocks; insert(tokens, block_ids) registers a sequence's sealed
    blocks (returns how many were added); remove(block_id) drops a block and
    every entry extending it.  Token and block ids are int32."""

    def __init__(self, capacity: int):
        import numpy as np
        self._np = np
        self._lib = load_library()
        h = ctypes.c_void_p()
        _check(self._lib.pa_prefix_index_create(int(capacity), ctypes.byref(h)),
               "pa_prefix_index_create")
        self._h = h

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            self._lib.pa_prefix_index_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    def _tokens(self, tokens):
        return self._np.ascontiguousarray(tokens, dtype=self._np.int32)

    def match(self, tokens) -> list:
        t = self._tokens(tokens)
        out = self._np.empty(max(t.size // 16, 1), dtype=self._np.int32)
        n = ctypes.c_int32(0)
        _check(self._lib.pa_prefix_index_match(self._h, t.ctypes.data, t.size, out.ctypes.data,
                                               ctypes.byref(n)), "pa_prefix_index_match")
        return out[:n.value].tolist()

    def insert(self, tokens, block_ids) -> int:
        t = self._tokens(tokens)
        b = self._np.ascontiguousarray(block_ids, dtype=self._np.int32)
        n = ctypes.c_int32(0)
        _check(self._lib.pa_prefix_index_insert(self._h, t.ctypes.data, t.size, b.ctypes.data,
                                                b.size, ctypes.byref(n)),
               "pa_prefix_index_insert")
        return n.value

    def remove(self, block_id: int) -> int:
        n = ctypes.c_int32(0)
        _check(self._lib.pa_prefix_index_remove(self._h, int(block_id), ctypes.byref(n)),
               "pa_prefix_index_remove")
        return n.value

    def __len__(self) -> int:
        return int(self._lib.pa_prefix_index_size(self._h))
