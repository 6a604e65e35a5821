"""Python binding of libpkv (paged-KV decode attention for MI355X / gfx950).

Argument marshalling only: every operation runs in the HIP library through its
C ABI (``include/pkv.h``).  torch supplies device memory and the current
stream.  Importing this package fails if the library has not been built
(``python paged_kv_cache_466_amd/build.py``); there is no fallback.
"""

import ctypes
import os

import torch

__all__ = [
    "PkvError", "lib", "version", "last_error",
    "paged_attn_decode", "paged_attn_partition", "paged_attn_merge",
    "paged_attn_workspace_bytes", "paged_attn_num_partitions", "paged_attn_partition_size",
    "paged_attn_decode_multi", "paged_attn_decode_selected", "quest_summarize", "quest_summary_like", "quest_select",
    "paged_attn_decode_append", "paged_attn_decode_shared_prefix", "paged_attn_shared_prefix_workspace_bytes",
    "validate_shared_prefix", "paged_attn_decode_grouped", "quantize_kv_grouped", "append_kv_quantized_grouped", "GROUP_CHANNEL",
    "GROUP_TOKEN",
    "slot_mapping", "reshape_and_cache", "append_kv", "append_kv_quantized", "copy_blocks", "quantize_kv",
    "stream_read", "validate_tables", "BlockPool", "PrefixCache", "h2o_retain", "DTYPES",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "_lib", "libpkv.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"libpkv.so not found at {LIB_PATH}: build it with `python paged_kv_cache_466_amd/build.py`")
lib = ctypes.CDLL(LIB_PATH)

# pkv_dtype
F32, BF16, F16, I8, FP8E4M3, I4, FP8E5M2 = 0, 1, 2, 3, 4, 5, 6
# decode flags
DECODE_STREAM_KV = 1
# scale groups of the grouped quantiser / decode
GROUP_CHANNEL, GROUP_TOKEN = 0, 1
DTYPES = {"f32": F32, "bf16": BF16, "f16": F16, "i8": I8, "fp8e4m3": FP8E4M3, "i4": I4, "fp8e5m2": FP8E5M2}
_TORCH_TO_PKV = {torch.float32: F32, torch.bfloat16: BF16, torch.float16: F16, torch.int8: I8,
                 torch.float8_e4m3fn: FP8E4M3, torch.float8_e5m2: FP8E5M2}
_STATUS = {0: "PKV_OK", 1: "PKV_EINVAL", 2: "PKV_EUNSUPPORTED", 3: "PKV_EWORKSPACE", 4: "PKV_EHIP",
           5: "PKV_ENOMEM"}

_p, _i, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
_i32p = ctypes.POINTER(ctypes.c_int32)

_ATTN = [_p, _p, _i, _p, _p, _i, _p, _p, _p, _i, _p, _i, _i, _i, _i, _i, _i, _f, _i, _i, _i, ctypes.c_uint, _p, _sz,
         _p]
_SIGS = {
    "pkv_last_error": ([], ctypes.c_char_p),
    "pkv_version": ([], ctypes.c_char_p),
    "pkv_paged_attn_num_partitions": ([_i, _i, _i, _i], _i),
    "pkv_paged_attn_partition_size": ([_i, _i, _i], _i),
    "pkv_paged_attn_workspace_bytes": ([_i, _i, _i, _i, _i, _i, _i], _sz),
    "pkv_paged_attn_decode": (_ATTN, _i),
    "pkv_paged_attn_partition": (_ATTN, _i),
    "pkv_paged_attn_noalloc_scratch_bytes": ([], _sz),
    "pkv_paged_attn_decode_noalloc": (_ATTN[:-3] + [_p], _i),
    "pkv_paged_attn_merge": ([_p, _i, _p, _i, _i, _i, _i, _i, _i, _i, _i, _p, _sz, _p], _i),
    "pkv_paged_attn_decode_multi": ([_p, _p, _i, _p, _p, _i, _p, _p, _p, _i, _p, _i, _i, _i, _i, _i, _i, _i, _f, _i,
                                     ctypes.c_uint, _p, _sz, _p], _i),
    "pkv_paged_attn_decode_selected": ([_p, _p, _i, _p, _p, _i, _p, _p, _p, _i, _p, _i, _i, _i, _i, _i, _i, _f,
                                        ctypes.c_uint, _p, _sz, _p], _i),
    "pkv_paged_attn_decode_append": ([_p, _p, _i, _p, _p, _i, _p, _p, _p, _p, _p, _i, _p, _i, _i, _i, _i, _i, _i, _f,
                                      _i, _i, _i, ctypes.c_uint, _p, _sz, _p], _i),
    "pkv_paged_attn_decode_shared_prefix": ([_p, _p, _i, _p, _p, _i, _p, _p, _p, _p, _p, _i, _p, _i, _i, _i, _i, _i,
                                             _i, _f, _i, _i, ctypes.c_uint, _p, _sz, _p], _i),
    "pkv_paged_attn_shared_prefix_workspace_bytes": ([_i, _i, _i, _i, _i, _i, _i, _i], _sz),
    "pkv_validate_shared_prefix": ([_p, _i, _p, _i, _i, _i], _i),
    "pkv_paged_attn_decode_grouped": ([_p, _p, _i, _p, _p, _i, _p, _p, _p, _p, _i, _p, _i, _i, _i, _i, _i, _i, _f,
                                       _i, ctypes.c_uint, _p, _sz, _p], _i),
    "pkv_append_kv_quantized_grouped": ([_p, _p, _i, _p, _p, _p, _p, _i, _p, _p, _p, _p, _i, _p, _i, _i, _i, _i, _i,
                                         _p], _i),
    "pkv_quantize_kv_grouped": ([_p, _i, _p, _i, _p, _p, _i, _p, _i, _i, _i, _i, _i, _p], _i),
    "pkv_stream_read_sink_words": ([], _i),
    "pkv_stream_read": ([_p, _sz, _p, _p], _i),
    "pkv_quest_summarize": ([_p, _i, _p, _p, _i, _p, _i, _i, _i, _i, _i, _i, _p], _i),
    "pkv_quest_scratch_bytes": ([_i, _i, _i], _sz),
    "pkv_quest_select": ([_p, _i, _p, _p, _i, _p, _i, _i, _i, _i, _i, _i, _i, _p, _p, _sz, _p], _i),
    "pkv_slot_mapping": ([_p, _p, _i, _p, _p, _i, _i, _i, _i, _p], _i),
    "pkv_reshape_and_cache": ([_p, _p, _p, _p, _i, _p, _i, _i, _i, _i, _i, _p], _i),
    "pkv_append_kv": ([_p, _p, _p, _p, _i, _p, _i, _p, _p, _p, _i, _i, _i, _i, _i, _i, _p], _i),
    "pkv_append_kv_quantized": ([_p, _p, _i, _p, _p, _p, _p, _i, _p, _p, _p, _i, _p, _i, _i, _i, _i, _i, _p], _i),
    "pkv_copy_blocks": ([_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _p], _i),
    "pkv_quantize_kv": ([_p, _i, _p, _i, _p, _p, _i, _i, _i, _i, _i, _p], _i),
    "pkv_validate_tables": ([_p, _i, _p, _i, _i, _i, _p, _i], _i),
    "pkv_pool_create": ([_i, _p], _p),
    "pkv_prefix_cache_create": ([_p, _i], _p),
    "pkv_prefix_cache_destroy": ([_p], None),
    "pkv_prefix_cache_match": ([_p, _p, _i, _p, _i, _p], _i),
    "pkv_prefix_cache_insert": ([_p, _p, _i, _p, _i, _p], _i),
    "pkv_prefix_cache_evict": ([_p, _i, _p], _i),
    "pkv_prefix_cache_size": ([_p], _i),
    "pkv_h2o_retain": ([_p, _i, _i, _i, _p, _p], _i),
    "pkv_pool_destroy": ([_p], None),
    "pkv_pool_alloc": ([_p, _i32p], _i),
    "pkv_pool_incref": ([_p, ctypes.c_int32], _i),
    "pkv_pool_decref": ([_p, ctypes.c_int32], _i),
    "pkv_pool_refcount": ([_p, ctypes.c_int32], ctypes.c_int32),
    "pkv_pool_append": ([_p, _p, ctypes.c_int32, _i32p, ctypes.c_int32, _i, _i32p, _i32p, _i32p], _i),
    "pkv_pool_stats": ([_p, _i32p, _i32p, _i32p], _i),
    "pkv_pool_allocate_sequence": ([_p, ctypes.c_int32, _i, _p, ctypes.c_int32, _i32p], _i),
    "pkv_pool_fork": ([_p, _p, ctypes.c_int32], _i),
    "pkv_pool_release": ([_p, _p, ctypes.c_int32], _i),
    "pkv_pool_free_list": ([_p, _p, ctypes.c_int32, _i32p], _i),
}
for _name, (_args, _res) in _SIGS.items():
    _fn = getattr(lib, _name)
    _fn.argtypes = _args
    _fn.restype = _res


class PkvError(RuntimeError):
    """A libpkv call returned a status other than PKV_OK."""

    def __init__(self, status, message):
        self.status = status
        super().__init__(f"{_STATUS.get(status, status)}: {message}")


def last_error():
    return lib.pkv_last_error().decode()


def version():
    return lib.pkv_version().decode()


def _check(status):
    if status != 0:
        raise PkvError(status, last_error())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(*tensors):
    for t in tensors:
        if t is not None and t.is_cuda:
            return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)
    return None


def _dtype(t, override=None):
    if override is not None:
        return DTYPES[override] if isinstance(override, str) else int(override)
    if t.dtype not in _TORCH_TO_PKV:
        raise TypeError(f"unsupported tensor dtype {t.dtype}")
    return _TORCH_TO_PKV[t.dtype]


def _head_dim(cache, kvdt):
    """head_dim of a cache tensor: an INT4 cache holds two elements per byte."""
    return cache.shape[-1] * 2 if kvdt == I4 else cache.shape[-1]


def _contig(*tensors):
    for t in tensors:
        if t is not None and not t.is_contiguous():
            raise ValueError("libpkv takes C-contiguous tensors")


# ---------------------------------------------------------------------------
# decode attention
# ---------------------------------------------------------------------------

def _dtype_code(dt):
    """A pkv dtype code from a name ("bf16", "i8", ...), a torch dtype or a code."""
    if isinstance(dt, str):
        return DTYPES[dt]
    if isinstance(dt, torch.dtype):
        return _TORCH_TO_PKV[dt]
    return int(dt)


def paged_attn_num_partitions(kv_dtype, max_seq_len, partition_size=0, block_size=16):
    return lib.pkv_paged_attn_num_partitions(_dtype_code(kv_dtype), max_seq_len, block_size, partition_size)


def paged_attn_partition_size(kv_dtype, max_seq_len, block_size=16):
    return lib.pkv_paged_attn_partition_size(_dtype_code(kv_dtype), max_seq_len, block_size)


def paged_attn_workspace_bytes(kv_dtype, num_seqs, num_q_heads, num_kv_heads, head_dim, max_seq_len,
                               partition_size=0):
    return lib.pkv_paged_attn_workspace_bytes(_dtype_code(kv_dtype), num_seqs, num_q_heads, num_kv_heads,
                                              head_dim, max_seq_len, partition_size)


def _check_tables(block_tables, seq_lens, S):
    """block_tables [S, max_blocks] and seq_lens [S], both int32."""
    if block_tables.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise TypeError("block_tables and seq_lens must be int32")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or tuple(seq_lens.shape) != (S,):
        raise ValueError("block_tables must be [num_seqs, max_blocks] and seq_lens [num_seqs]")


def _attn_call(fn, out, query, k_cache, v_cache, block_tables, seq_lens, sm_scale, k_scales, v_scales,
               partition_size, sink_tokens, window_tokens, workspace, kv_dtype, stream_kv):
    _contig(out, query, k_cache, v_cache, block_tables, seq_lens, k_scales, v_scales, workspace)
    S, Hq, D = query.shape
    NB, BS, Hkv = k_cache.shape[:3]
    if _head_dim(k_cache, _dtype(k_cache, kv_dtype)) != D or tuple(v_cache.shape) != tuple(k_cache.shape) \
            or tuple(out.shape) != tuple(query.shape):
        raise ValueError("shape mismatch between query, caches and out")
    _check_tables(block_tables, seq_lens, S)
    mbs = block_tables.shape[1]
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(fn(_ptr(out), _ptr(query), _dtype(query), _ptr(k_cache), _ptr(v_cache), _dtype(k_cache, kv_dtype),
              _ptr(k_scales), _ptr(v_scales), _ptr(block_tables), mbs, _ptr(seq_lens), S, Hq, Hkv, D, BS, NB,
              float(sm_scale), int(partition_size), int(sink_tokens), int(window_tokens),
              DECODE_STREAM_KV if stream_kv else 0, _ptr(workspace), ws_bytes, _stream(query)))
    return out


def _workspace_for(query, k_cache, block_tables, partition_size, workspace, kv_dtype):
    if workspace is not None:
        return workspace
    S, Hq, D = query.shape
    nbytes = paged_attn_workspace_bytes(_dtype(k_cache, kv_dtype), S, Hq, k_cache.shape[2], D,
                                        block_tables.shape[1] * k_cache.shape[1], partition_size)
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=query.device)


def paged_attn_decode(out, query, k_cache, v_cache, block_tables, seq_lens, sm_scale, k_scales=None,
                      v_scales=None, partition_size=0, sink_tokens=0, window_tokens=0, workspace=None,
                      kv_dtype=None, stream_kv=False):
    """Decode attention over a paged cache (``pkv_paged_attn_decode``).

    query/out [S, Hq, D]; caches [NB, 16, Hkv, D]; block_tables [S, MBS] int32;
    seq_lens [S] int32.  A workspace is taken from torch when none is given.
    ``kv_dtype`` ("i8" / "fp8e4m3" / "fp8e5m2" / "i4") names the code type when the caches are
    uint8 tensors.  ``stream_kv`` sets PKV_DECODE_STREAM_KV (no block is
    shared between the batch's sequences).
    """
    workspace = _workspace_for(query, k_cache, block_tables, partition_size, workspace, kv_dtype)
    return _attn_call(lib.pkv_paged_attn_decode, out, query, k_cache, v_cache, block_tables, seq_lens,
                      sm_scale, k_scales, v_scales, partition_size, sink_tokens, window_tokens, workspace,
                      kv_dtype, stream_kv)


def paged_attn_decode_noalloc(out, query, k_cache, v_cache, block_tables, seq_lens, sm_scale, k_scales=None,
                              v_scales=None, partition_size=0, sink_tokens=0, window_tokens=0, kv_dtype=None,
                              stream_kv=False):
    """``paged_attn_decode`` without a workspace (``pkv_paged_attn_decode_noalloc``):
    the library's fixed device scratch array stands in for it, so the call
    allocates nothing.  Calls that overlap on one GPU race on that array."""
    _contig(out, query, k_cache, v_cache, block_tables, seq_lens, k_scales, v_scales)
    S, Hq, D = query.shape
    NB, BS, Hkv = k_cache.shape[:3]
    if _head_dim(k_cache, _dtype(k_cache, kv_dtype)) != D or tuple(v_cache.shape) != tuple(k_cache.shape) \
            or tuple(out.shape) != tuple(query.shape):
        raise ValueError("shape mismatch between query, caches and out")
    _check_tables(block_tables, seq_lens, S)
    _check(lib.pkv_paged_attn_decode_noalloc(
        _ptr(out), _ptr(query), _dtype(query), _ptr(k_cache), _ptr(v_cache), _dtype(k_cache, kv_dtype),
        _ptr(k_scales), _ptr(v_scales), _ptr(block_tables), block_tables.shape[1], _ptr(seq_lens), S, Hq, Hkv, D, BS,
        NB, float(sm_scale), int(partition_size), int(sink_tokens), int(window_tokens),
        DECODE_STREAM_KV if stream_kv else 0, _stream(query)))
    return out


def paged_attn_partition(out, query, k_cache, v_cache, block_tables, seq_lens, sm_scale, workspace,
                         k_scales=None, v_scales=None, partition_size=0, sink_tokens=0, window_tokens=0,
                         kv_dtype=None, stream_kv=False):
    """First pass of the decode (``pkv_paged_attn_partition``)."""
    return _attn_call(lib.pkv_paged_attn_partition, out, query, k_cache, v_cache, block_tables, seq_lens,
                      sm_scale, k_scales, v_scales, partition_size, sink_tokens, window_tokens, workspace,
                      kv_dtype, stream_kv)


def paged_attn_decode_multi(out, query, k_cache, v_cache, block_tables, seq_lens, sm_scale, k_scales=None,
                            v_scales=None, partition_size=0, workspace=None, kv_dtype=None, stream_kv=False):
    """Several new tokens per sequence (``pkv_paged_attn_decode_multi``):
    query/out [S, T, Hq, D]; seq_lens count the T new tokens (already in
    the cache); token t sees positions up to L - T + t."""
    _contig(out, query, k_cache, v_cache, block_tables, seq_lens, k_scales, v_scales, workspace)
    S, T, Hq, D = query.shape
    NB, BS, Hkv = k_cache.shape[:3]
    kvdt = _dtype(k_cache, kv_dtype)
    if _head_dim(k_cache, kvdt) != D or tuple(out.shape) != tuple(query.shape) \
            or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("shape mismatch between query, caches and out")
    _check_tables(block_tables, seq_lens, S)
    mbs = block_tables.shape[1]
    if workspace is None:
        nbytes = paged_attn_workspace_bytes(kvdt, S, Hq * T, Hkv, D, mbs * BS, partition_size)
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=query.device) if nbytes else None
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.pkv_paged_attn_decode_multi(
        _ptr(out), _ptr(query), _dtype(query), _ptr(k_cache), _ptr(v_cache), kvdt, _ptr(k_scales), _ptr(v_scales),
        _ptr(block_tables), mbs, _ptr(seq_lens), S, T, Hq, Hkv, D, BS, NB, float(sm_scale), int(partition_size),
        DECODE_STREAM_KV if stream_kv else 0, _ptr(workspace), ws_bytes, _stream(query)))
    return out


def paged_attn_decode_selected(out, query, k_cache, v_cache, selected, seq_lens, sm_scale, k_scales=None,
                               v_scales=None, workspace=None, kv_dtype=None):
    """Decode reading only the selected pages (``pkv_paged_attn_decode_selected``).

    ``selected`` [S, Hkv, budget, 2] int32 (physical, logical block) as
    ``quest_select`` returns it."""
    _contig(out, query, k_cache, v_cache, selected, seq_lens, k_scales, v_scales, workspace)
    S, Hq, D = query.shape
    NB, BS, Hkv = k_cache.shape[:3]
    if _head_dim(k_cache, _dtype(k_cache, kv_dtype)) != D or tuple(v_cache.shape) != tuple(k_cache.shape) \
            or tuple(out.shape) != tuple(query.shape):
        raise ValueError("shape mismatch between query, caches and out")
    if selected.dtype != torch.int32 or selected.dim() != 4 or tuple(selected.shape[:2]) != (S, Hkv) \
            or selected.shape[3] != 2:
        raise ValueError("selected must be int32 [num_seqs, num_kv_heads, budget, 2]")
    budget = selected.shape[2]
    kvdt = _dtype(k_cache, kv_dtype)
    if workspace is None:
        nbytes = paged_attn_workspace_bytes(kvdt, S, Hq, Hkv, D, budget * BS, BS)
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=query.device) if nbytes else None
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.pkv_paged_attn_decode_selected(
        _ptr(out), _ptr(query), _dtype(query), _ptr(k_cache), _ptr(v_cache), kvdt, _ptr(k_scales), _ptr(v_scales),
        _ptr(selected), budget, _ptr(seq_lens), S, Hq, Hkv, D, BS, NB, float(sm_scale), 0, _ptr(workspace),
        ws_bytes, _stream(query)))
    return out


def quest_summary_like(k_cache):
    """An empty page-summary tensor for ``k_cache`` [NB, BS, Hkv, D]:
    [NB, Hkv, 2, D] of the cache's dtype."""
    NB, BS, Hkv, D = k_cache.shape
    return torch.empty((NB, Hkv, 2, D), dtype=k_cache.dtype, device=k_cache.device)


def quest_summarize(k_cache, k_summary, block_tables, seq_lens, last_only=False):
    """Page summaries (``pkv_quest_summarize``): per (block, KV head) the
    minimum and maximum of the written keys."""
    _contig(k_cache, k_summary, block_tables, seq_lens)
    NB, BS, Hkv, D = k_cache.shape
    if tuple(k_summary.shape) != (NB, Hkv, 2, D) or k_summary.dtype != k_cache.dtype:
        raise ValueError("k_summary must be [num_blocks, num_kv_heads, 2, head_dim] of the cache's dtype")
    S, mbs = block_tables.shape
    _check(lib.pkv_quest_summarize(_ptr(k_cache), _dtype(k_cache), _ptr(k_summary), _ptr(block_tables), mbs,
                                   _ptr(seq_lens), S, NB, BS, Hkv, D, 1 if last_only else 0, _stream(k_cache)))
    return k_summary


def quest_select(query, k_summary, block_tables, seq_lens, budget_blocks, selected=None, scratch=None):
    """Top-``budget_blocks`` pages per (sequence, KV head) (``pkv_quest_select``).
    Returns ``selected`` [S, Hkv, budget, 2] int32 (physical, logical block)."""
    _contig(query, k_summary, block_tables, seq_lens, selected, scratch)
    S, Hq, D = query.shape
    NB, Hkv, two, D2 = k_summary.shape
    if two != 2 or D2 != D:
        raise ValueError("k_summary must be [num_blocks, num_kv_heads, 2, head_dim]")
    mbs = block_tables.shape[1]
    if selected is None:
        selected = torch.zeros((S, Hkv, budget_blocks, 2), dtype=torch.int32, device=query.device)
    if scratch is None:
        nbytes = lib.pkv_quest_scratch_bytes(S, Hkv, mbs)
        scratch = torch.empty(max(nbytes, 8), dtype=torch.uint8, device=query.device)
    sb = scratch.numel() * scratch.element_size()
    _check(lib.pkv_quest_select(_ptr(query), _dtype(query), _ptr(k_summary), _ptr(block_tables), mbs,
                                _ptr(seq_lens), S, Hq, Hkv, D, 16, NB, budget_blocks, _ptr(selected),
                                _ptr(scratch), sb, _stream(query)))
    return selected


def paged_attn_merge(out, seq_lens, num_kv_heads, max_seq_len, workspace, partition_size=0, sink_tokens=0,
                     window_tokens=0):
    """Second pass of the decode (``pkv_paged_attn_merge``); partition_size,
    sink_tokens and window_tokens must match the partition call."""
    _contig(out, seq_lens, workspace)
    S, Hq, D = out.shape
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.pkv_paged_attn_merge(_ptr(out), _dtype(out), _ptr(seq_lens), S, Hq, num_kv_heads, D,
                                    max_seq_len, partition_size, int(sink_tokens), int(window_tokens),
                                    _ptr(workspace), ws_bytes, _stream(out)))
    return out


# ---------------------------------------------------------------------------
# cache writes
# ---------------------------------------------------------------------------

def slot_mapping(block_tables, positions, num_blocks, seq_ids=None, block_size=16, out=None):
    """Slots of new tokens (``pkv_slot_mapping``); returns an int32 tensor."""
    _contig(block_tables, positions, seq_ids)
    T = positions.numel()
    if out is None:
        out = torch.empty(T, dtype=torch.int32, device=positions.device)
    _check(lib.pkv_slot_mapping(_ptr(out), _ptr(block_tables), block_tables.shape[1], _ptr(seq_ids),
                                _ptr(positions), T, block_tables.shape[0], block_size, num_blocks,
                                _stream(positions)))
    return out


def reshape_and_cache(key, value, k_cache, v_cache, slot_mapping):
    """Slot write (``pkv_reshape_and_cache``): key/value [T, Hkv, D]."""
    _contig(key, value, k_cache, v_cache, slot_mapping)
    T = key.shape[0]
    NB, BS, Hkv, D = k_cache.shape
    if tuple(key.shape[1:]) != (Hkv, D) or key.shape != value.shape or key.dtype != k_cache.dtype:
        raise ValueError("key/value must be [T, Hkv, D] of the cache's dtype")
    _check(lib.pkv_reshape_and_cache(_ptr(key), _ptr(value), _ptr(k_cache), _ptr(v_cache), _dtype(k_cache),
                                     _ptr(slot_mapping), T, NB, BS, Hkv, D, _stream(key)))


def append_kv(key, value, k_cache, v_cache, block_tables, positions, seq_ids=None, slot_mapping=None):
    """Slot mapping + slot write in one launch (``pkv_append_kv``); key/value
    [T, Hkv, D] of the cache's dtype.  ``slot_mapping`` (int32 [T]) receives
    the slots when given."""
    _contig(key, value, k_cache, v_cache, block_tables, positions, seq_ids, slot_mapping)
    T = key.shape[0]
    NB, BS, Hkv, D = k_cache.shape
    if tuple(key.shape[1:]) != (Hkv, D) or key.shape != value.shape or key.dtype != k_cache.dtype:
        raise ValueError("key/value must be [T, Hkv, D] of the cache's dtype")
    _check(lib.pkv_append_kv(_ptr(key), _ptr(value), _ptr(k_cache), _ptr(v_cache), _dtype(k_cache),
                             _ptr(block_tables), block_tables.shape[1], _ptr(seq_ids), _ptr(positions),
                             _ptr(slot_mapping), T, block_tables.shape[0], NB, BS, Hkv, D, _stream(key)))


def append_kv_quantized(key, value, k_tail, v_tail, k_codes, v_codes, k_scales, v_scales, block_tables,
                        positions, code_dtype):
    """Appends one token per sequence to a quantised cache
    (``pkv_append_kv_quantized``): key/value [S, Hkv, D] and the tails
    [S, 16, Hkv, D] in the source dtype; codes [NB, 16, Hkv, D] int8 /
    uint8 ([NB, 16, Hkv, D / 2] uint8 for "i4"), scales [NB, Hkv] fp32;
    positions int32 [S] (< 0 skips)."""
    _contig(key, value, k_tail, v_tail, k_codes, v_codes, k_scales, v_scales, block_tables, positions)
    S, Hkv, D = key.shape
    NB, BS = k_codes.shape[:2]
    if tuple(k_tail.shape) != (S, BS, Hkv, D) or k_tail.dtype != key.dtype or value.shape != key.shape:
        raise ValueError("tails must be [S, block_size, Hkv, D] of the key dtype")
    if _head_dim(k_codes, DTYPES[code_dtype]) != D or k_codes.shape != v_codes.shape:
        raise ValueError("codes must be [NB, block_size, Hkv, D] (D / 2 bytes for i4)")
    _check(lib.pkv_append_kv_quantized(_ptr(key), _ptr(value), _dtype(key), _ptr(k_tail), _ptr(v_tail),
                                       _ptr(k_codes), _ptr(v_codes), DTYPES[code_dtype], _ptr(k_scales),
                                       _ptr(v_scales), _ptr(block_tables), block_tables.shape[1], _ptr(positions),
                                       S, NB, BS, Hkv, D, _stream(key)))


def append_kv_quantized_grouped(key, value, k_tail, v_tail, k_codes, v_codes, k_tile_scales, k_channel_scales,
                                v_token_scales, block_tables, positions, code_dtype):
    """``append_kv_quantized`` for a grouped-scale cache
    (``pkv_append_kv_quantized_grouped``): keys per channel, values per token."""
    _contig(key, value, k_tail, v_tail, k_codes, v_codes, k_tile_scales, k_channel_scales, v_token_scales,
            block_tables, positions)
    S, Hkv, D = key.shape
    NB, BS = k_codes.shape[:2]
    if tuple(k_tail.shape) != (S, BS, Hkv, D) or k_tail.dtype != key.dtype or value.shape != key.shape:
        raise ValueError("tails must be [S, block_size, Hkv, D] of the key dtype")
    if _head_dim(k_codes, DTYPES[code_dtype]) != D or k_codes.shape != v_codes.shape:
        raise ValueError("codes must be [NB, block_size, Hkv, D] (D / 2 bytes for i4)")
    if tuple(k_channel_scales.shape) != (NB, Hkv, D) or tuple(v_token_scales.shape) != (NB, Hkv, BS) \
            or tuple(k_tile_scales.shape) != (NB, Hkv):
        raise ValueError("scales must be [NB, Hkv] (tile), [NB, Hkv, D] (channel) and [NB, Hkv, 16] (token)")
    _check(lib.pkv_append_kv_quantized_grouped(
        _ptr(key), _ptr(value), _dtype(key), _ptr(k_tail), _ptr(v_tail), _ptr(k_codes), _ptr(v_codes),
        DTYPES[code_dtype], _ptr(k_tile_scales), _ptr(k_channel_scales), _ptr(v_token_scales), _ptr(block_tables),
        block_tables.shape[1], _ptr(positions), S, NB, BS, Hkv, D, _stream(key)))


def copy_blocks(k_cache, v_cache, src_dst, k_scales=None, v_scales=None, dtype=None):
    """Copy-on-write block copies (``pkv_copy_blocks``); src_dst int32 [n, 2]."""
    _contig(k_cache, v_cache, src_dst, k_scales, v_scales)
    NB, BS, Hkv = k_cache.shape[:3]
    dt = _dtype(k_cache, dtype) if k_cache.dtype != torch.uint8 or dtype else FP8E4M3
    D = _head_dim(k_cache, dt)
    _check(lib.pkv_copy_blocks(_ptr(k_cache), _ptr(v_cache), _ptr(k_scales), _ptr(v_scales), _ptr(src_dst),
                               src_dst.shape[0], dt, NB, BS, Hkv, D, _stream(k_cache)))


def quantize_kv(src_cache, dst_codes, dst_scales, code_dtype, block_ids=None, n_blocks=None):
    """Absmax block quantisation (``pkv_quantize_kv``).  code_dtype "i8",
    "fp8e4m3", "fp8e5m2" or "i4"; dst_codes has the cache's shape (int8 / uint8), with
    D / 2 bytes per row for "i4" (element 2i in the low nibble of byte i)."""
    _contig(src_cache, dst_codes, dst_scales, block_ids)
    NB, BS, Hkv, D = src_cache.shape
    if _head_dim(dst_codes, DTYPES[code_dtype]) != D or tuple(dst_codes.shape[:3]) != (NB, BS, Hkv):
        raise ValueError("dst_codes must be [NB, block_size, Hkv, D] (D / 2 bytes for i4)")
    if n_blocks is None:
        n_blocks = block_ids.numel() if block_ids is not None else NB
    _check(lib.pkv_quantize_kv(_ptr(src_cache), _dtype(src_cache), _ptr(dst_codes), DTYPES[code_dtype],
                               _ptr(dst_scales), _ptr(block_ids), n_blocks, NB, BS, Hkv, D,
                               _stream(src_cache)))


def quantize_kv_grouped(src_cache, dst_codes, dst_group_scales, code_dtype, group, dst_tile_scales=None,
                        block_ids=None, n_blocks=None):
    """Absmax quantisation with grouped scales (``pkv_quantize_kv_grouped``):
    ``group`` GROUP_CHANNEL (dst_group_scales [NB, Hkv, D]) or GROUP_TOKEN
    ([NB, Hkv, 16]); dst_tile_scales [NB, Hkv] receives each tile's largest
    group scale when given."""
    _contig(src_cache, dst_codes, dst_group_scales, dst_tile_scales, block_ids)
    NB, BS, Hkv, D = src_cache.shape
    if _head_dim(dst_codes, DTYPES[code_dtype]) != D or tuple(dst_codes.shape[:3]) != (NB, BS, Hkv):
        raise ValueError("dst_codes must be [NB, block_size, Hkv, D] (D / 2 bytes for i4)")
    want = (NB, Hkv, D if group == GROUP_CHANNEL else BS)
    if tuple(dst_group_scales.shape) != want or dst_group_scales.dtype != torch.float32:
        raise ValueError(f"dst_group_scales must be float32 {want}")
    if n_blocks is None:
        n_blocks = block_ids.numel() if block_ids is not None else NB
    _check(lib.pkv_quantize_kv_grouped(_ptr(src_cache), _dtype(src_cache), _ptr(dst_codes), DTYPES[code_dtype],
                                       _ptr(dst_tile_scales), _ptr(dst_group_scales), int(group), _ptr(block_ids),
                                       n_blocks, NB, BS, Hkv, D, _stream(src_cache)))


def paged_attn_decode_append(out, query, k_cache, v_cache, key, value, positions, block_tables, seq_lens, sm_scale,
                             slot_mapping=None, partition_size=0, sink_tokens=0, window_tokens=0, workspace=None,
                             stream_kv=False):
    """Decode with the step's slot write fused in (``pkv_paged_attn_decode_append``):
    key/value [S, Hkv, D] of each sequence's new token go to position
    positions[s] (= seq_lens[s] - 1, or < 0 for none), then attention over
    seq_lens tokens; the slots go to ``slot_mapping`` when given."""
    _contig(out, query, k_cache, v_cache, key, value, positions, block_tables, seq_lens, slot_mapping, workspace)
    S, Hq, D = query.shape
    NB, BS, Hkv = k_cache.shape[:3]
    if k_cache.shape[3] != D or tuple(v_cache.shape) != tuple(k_cache.shape) or tuple(out.shape) != tuple(query.shape):
        raise ValueError("shape mismatch between query, caches and out")
    if tuple(key.shape) != (S, Hkv, D) or value.shape != key.shape or key.dtype != k_cache.dtype:
        raise ValueError("key/value must be [S, Hkv, D] of the cache's dtype")
    _check_tables(block_tables, seq_lens, S)
    workspace = _workspace_for(query, k_cache, block_tables, partition_size, workspace, None)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.pkv_paged_attn_decode_append(
        _ptr(out), _ptr(query), _dtype(query), _ptr(k_cache), _ptr(v_cache), _dtype(k_cache), _ptr(key), _ptr(value),
        _ptr(positions), _ptr(slot_mapping), _ptr(block_tables), block_tables.shape[1], _ptr(seq_lens), S, Hq, Hkv, D,
        BS, NB, float(sm_scale), int(partition_size), int(sink_tokens), int(window_tokens),
        DECODE_STREAM_KV if stream_kv else 0, _ptr(workspace), ws_bytes, _stream(query)))
    return out


def paged_attn_shared_prefix_workspace_bytes(kv_dtype, num_seqs, num_q_heads, num_kv_heads, head_dim, max_seq_len,
                                            prefix_blocks, partition_size=0):
    return lib.pkv_paged_attn_shared_prefix_workspace_bytes(_dtype_code(kv_dtype), num_seqs, num_q_heads,
                                                            num_kv_heads, head_dim, max_seq_len, prefix_blocks,
                                                            partition_size)


def paged_attn_decode_shared_prefix(out, query, k_cache, v_cache, block_tables, seq_lens, sm_scale, prefix_blocks,
                                    key=None, value=None, positions=None, slot_mapping=None, partition_size=0,
                                    workspace=None, stream_kv=False):
    """Decode over a batch whose sequences all start with the same
    ``prefix_blocks`` physical blocks (``pkv_paged_attn_decode_shared_prefix``):
    the result of ``paged_attn_decode``, with the shared blocks read once per
    32 query rows.  key/value/positions/slot_mapping: the optional fused slot
    write of ``paged_attn_decode_append`` (the new token lies past the prefix)."""
    _contig(out, query, k_cache, v_cache, key, value, positions, block_tables, seq_lens, slot_mapping, workspace)
    S, Hq, D = query.shape
    NB, BS, Hkv = k_cache.shape[:3]
    if k_cache.shape[3] != D or tuple(v_cache.shape) != tuple(k_cache.shape) or tuple(out.shape) != tuple(query.shape):
        raise ValueError("shape mismatch between query, caches and out")
    _check_tables(block_tables, seq_lens, S)
    if key is not None and (tuple(key.shape) != (S, Hkv, D) or value is None or value.shape != key.shape
                            or key.dtype != k_cache.dtype or positions is None):
        raise ValueError("key/value must be [S, Hkv, D] of the cache's dtype, with positions")
    mbs = block_tables.shape[1]
    if workspace is None:
        nbytes = paged_attn_shared_prefix_workspace_bytes(_dtype(k_cache), S, Hq, Hkv, D, mbs * BS,
                                                          int(prefix_blocks), partition_size)
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=query.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib.pkv_paged_attn_decode_shared_prefix(
        _ptr(out), _ptr(query), _dtype(query), _ptr(k_cache), _ptr(v_cache), _dtype(k_cache), _ptr(key),
        _ptr(value), _ptr(positions), _ptr(slot_mapping), _ptr(block_tables), mbs, _ptr(seq_lens), S, Hq, Hkv, D,
        BS, NB, float(sm_scale), int(prefix_blocks), int(partition_size), DECODE_STREAM_KV if stream_kv else 0,
        _ptr(workspace), ws_bytes, _stream(query)))
    return out


def validate_shared_prefix(block_tables, seq_lens, prefix_blocks, block_size=16):
    """Host check of the shared-prefix preconditions (``pkv_validate_shared_prefix``)."""
    bt = block_tables.detach().cpu().contiguous().to(torch.int32)
    sl = seq_lens.detach().cpu().contiguous().to(torch.int32)
    _check(lib.pkv_validate_shared_prefix(_ptr(bt), bt.shape[1], _ptr(sl), sl.shape[0], block_size,
                                          int(prefix_blocks)))


def paged_attn_decode_grouped(out, query, k_cache, v_cache, block_tables, seq_lens, sm_scale, k_tile_scales,
                              k_channel_scales, v_token_scales, partition_size=0, workspace=None, kv_dtype=None,
                              stream_kv=False):
    """Decode over a cache quantised with grouped scales
    (``pkv_paged_attn_decode_grouped``): keys per channel, values per token."""
    _contig(out, query, k_cache, v_cache, block_tables, seq_lens, k_tile_scales, k_channel_scales,
            v_token_scales, workspace)
    S, Hq, D = query.shape
    NB, BS, Hkv = k_cache.shape[:3]
    kvdt = _dtype(k_cache, kv_dtype)
    if _head_dim(k_cache, kvdt) != D or tuple(v_cache.shape) != tuple(k_cache.shape) \
            or tuple(out.shape) != tuple(query.shape):
        raise ValueError("shape mismatch between query, caches and out")
    if tuple(k_channel_scales.shape) != (NB, Hkv, D) or tuple(v_token_scales.shape) != (NB, Hkv, BS) \
            or tuple(k_tile_scales.shape) != (NB, Hkv):
        raise ValueError("scales must be [NB, Hkv] (tile), [NB, Hkv, D] (channel) and [NB, Hkv, 16] (token)")
    _check_tables(block_tables, seq_lens, S)
    workspace = _workspace_for(query, k_cache, block_tables, partition_size, workspace, kvdt)
    mbs = block_tables.shape[1]
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.pkv_paged_attn_decode_grouped(
        _ptr(out), _ptr(query), _dtype(query), _ptr(k_cache), _ptr(v_cache), kvdt, _ptr(k_tile_scales),
        _ptr(k_channel_scales), _ptr(v_token_scales), _ptr(block_tables), mbs, _ptr(seq_lens), S, Hq, Hkv, D, BS, NB,
        float(sm_scale), int(partition_size), DECODE_STREAM_KV if stream_kv else 0, _ptr(workspace), ws_bytes,
        _stream(query)))
    return out


def stream_read(src, sink=None):
    """Streaming-read probe (``pkv_stream_read``): reads all of ``src`` (a
    device tensor, size a multiple of 16 bytes) once; returns the sink."""
    _contig(src)
    if sink is None:
        sink = torch.empty(lib.pkv_stream_read_sink_words(), dtype=torch.int32, device=src.device)
    _check(lib.pkv_stream_read(_ptr(src), src.numel() * src.element_size(), _ptr(sink), _stream(src)))
    return sink


def validate_tables(block_tables, seq_lens, num_blocks, slot_mapping=None, block_size=16):
    """Host-side precondition check (``pkv_validate_tables``) on CPU int32 tensors."""
    bt = block_tables.cpu().contiguous()
    sl = seq_lens.cpu().contiguous()
    sm = slot_mapping.cpu().contiguous() if slot_mapping is not None else None
    _check(lib.pkv_validate_tables(_ptr(bt), bt.shape[1], _ptr(sl), sl.numel(), block_size, num_blocks,
                                   _ptr(sm), 0 if sm is None else sm.numel()))


# ---------------------------------------------------------------------------
# host block pool
# ---------------------------------------------------------------------------

class BlockPool:
    """The library's host block pool (FIFO free list + reference counts)."""

    def __init__(self, num_blocks, initial_order=None):
        self._keep = None
        order = None
        if initial_order is not None:
            self._keep = (ctypes.c_int32 * num_blocks)(*[int(b) for b in initial_order])
            order = ctypes.cast(self._keep, ctypes.c_void_p)
        self._h = lib.pkv_pool_create(num_blocks, order)
        if not self._h:
            raise PkvError(1, last_error())
        self.num_blocks = num_blocks

    def __del__(self, _destroy=lib.pkv_pool_destroy):
        h = getattr(self, "_h", None)
        if h:
            _destroy(h)
            self._h = None

    def alloc(self):
        b = ctypes.c_int32()
        _check(lib.pkv_pool_alloc(self._h, ctypes.byref(b)))
        return b.value

    def incref(self, block):
        _check(lib.pkv_pool_incref(self._h, int(block)))

    def decref(self, block):
        _check(lib.pkv_pool_decref(self._h, int(block)))

    def refcount(self, block):
        return lib.pkv_pool_refcount(self._h, int(block))

    def append(self, table, seq_len, block_size=16, capacity=None):
        """Reserve the slot of token ``seq_len`` of a sequence whose table is
        the python list ``table`` (updated in place).  Returns (slot, cow)
        with cow None or (src, dst)."""
        cap = capacity if capacity is not None else len(table) + 1
        arr = (ctypes.c_int32 * max(cap, 1))(*table)
        n = ctypes.c_int32(len(table))
        slot, src, dst = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        _check(lib.pkv_pool_append(self._h, ctypes.cast(arr, ctypes.c_void_p), cap, ctypes.byref(n), seq_len,
                                   block_size, ctypes.byref(slot), ctypes.byref(src), ctypes.byref(dst)))
        table[:] = list(arr[: n.value])
        return slot.value, (None if src.value < 0 else (src.value, dst.value))

    def stats(self):
        f, u, s = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        _check(lib.pkv_pool_stats(self._h, ctypes.byref(f), ctypes.byref(u), ctypes.byref(s)))
        return {"free": f.value, "used": u.value, "shared": s.value}

    def free_list(self):
        n = ctypes.c_int32()
        _check(lib.pkv_pool_free_list(self._h, None, 0, ctypes.byref(n)))
        arr = (ctypes.c_int32 * max(n.value, 1))()
        _check(lib.pkv_pool_free_list(self._h, ctypes.cast(arr, ctypes.c_void_p), n.value, ctypes.byref(n)))
        return list(arr[: n.value])

    # sequence-level operations (pkv_pool_allocate_sequence / _fork / _release)
    def allocate_sequence(self, length, block_size=16):
        cap = self.num_blocks
        arr = (ctypes.c_int32 * max(cap, 1))()
        n = ctypes.c_int32()
        _check(lib.pkv_pool_allocate_sequence(self._h, int(length), int(block_size),
                                              ctypes.cast(arr, ctypes.c_void_p), cap, ctypes.byref(n)))
        return list(arr[: n.value])

    @staticmethod
    def _array(table):
        return (ctypes.c_int32 * max(len(table), 1))(*[int(b) for b in table])

    def fork(self, table):
        arr = self._array(table)
        _check(lib.pkv_pool_fork(self._h, ctypes.cast(arr, ctypes.c_void_p), len(table)))
        return list(table)

    def release(self, table):
        arr = self._array(table)
        _check(lib.pkv_pool_release(self._h, ctypes.cast(arr, ctypes.c_void_p), len(table)))


class PrefixCache:
    """The library's prefix cache over a ``BlockPool`` (``pkv_prefix_cache_*``):
    full blocks stored under their whole token prefix."""

    def __init__(self, pool, block_size=16):
        self.pool = pool            # kept alive: the cache holds references into it
        self.block_size = block_size
        self._h = lib.pkv_prefix_cache_create(pool._h, block_size)
        if not self._h:
            raise PkvError(1, last_error())

    def __del__(self, _destroy=lib.pkv_prefix_cache_destroy):
        h = getattr(self, "_h", None)
        if h:
            _destroy(h)
            self._h = None

    @staticmethod
    def _tokens(tokens):
        t = [int(x) for x in tokens]
        return (ctypes.c_int32 * max(1, len(t)))(*t), len(t)

    def match(self, tokens):
        """Physical blocks of the cached leading full blocks of ``tokens``;
        the caller receives one pool reference per block."""
        buf, n = self._tokens(tokens)
        cap = n // self.block_size
        out = (ctypes.c_int32 * max(1, cap))()
        got = ctypes.c_int()
        _check(lib.pkv_prefix_cache_match(self._h, buf, n, out, cap, ctypes.byref(got)))
        return list(out[: got.value])

    def insert(self, tokens, blocks):
        """Stores the full blocks of ``tokens`` held in ``blocks``; returns the
        number of entries added."""
        buf, n = self._tokens(tokens)
        b = [int(x) for x in blocks]
        bb = (ctypes.c_int32 * max(1, len(b)))(*b)
        added = ctypes.c_int()
        _check(lib.pkv_prefix_cache_insert(self._h, buf, n, bb, len(b), ctypes.byref(added)))
        return added.value

    def evict(self, n):
        got = ctypes.c_int()
        _check(lib.pkv_prefix_cache_evict(self._h, int(n), ctypes.byref(got)))
        return got.value

    def __len__(self):
        return lib.pkv_prefix_cache_size(self._h)


def h2o_retain(scores, budget, recent_count):
    """Positions kept by the H2O rule (``pkv_h2o_retain``), in increasing order."""
    s = [float(x) for x in scores]
    buf = (ctypes.c_float * max(1, len(s)))(*s)
    out = (ctypes.c_int32 * max(1, len(s)))()
    n = ctypes.c_int()
    _check(lib.pkv_h2o_retain(buf, len(s), int(budget), int(recent_count), out, ctypes.byref(n)))
    return list(out[: n.value])
