"""ctypes binding of libpa.so: torch tensors -> device pointers + the current
HIP stream.  Argument marshalling only; every step of the computation runs in
the library's kernels.  There is no CPU path: if libpa.so is missing, or a
tensor is not on the GPU, the call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpa.so")

PA_F32, PA_BF16, PA_FP8_E4M3 = 0, 1, 2
PA_PARTITION_BALANCED = -1   # partition_size selecting the balanced split-KV mode
PA_STAGE_ATTENTION, PA_STAGE_MERGE, PA_STAGE_ALL = 1, 2, 3
STATUS_NAMES = {0: "PA_OK", 1: "PA_ERR_NULL", 2: "PA_ERR_SHAPE", 3: "PA_ERR_DTYPE",
                4: "PA_ERR_ALIGN", 5: "PA_ERR_UNSUPPORTED", 6: "PA_ERR_WORKSPACE", 7: "PA_ERR_HIP"}

_vp, _i, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t

# argument lists of the exported functions, in include/pa.h order
SIGNATURES = {
    "pa_status_string": (ctypes.c_char_p, [_i]),
    "pa_version": (_i, []),
    "pa_decode_workspace_size": (_sz, [_i, _i, _i, _i, _i]),
    "pa_decode": (_i, [_vp, _vp, _i, _vp, _vp, _i, _vp, _i, _vp, _i, _i, _i, _i, _i, _i, _f,
                       _vp, _vp, _i, _i, _vp, _sz, _vp]),
    "pa_decode_noalloc": (_i, [_vp, _vp, _i, _vp, _vp, _i, _vp, _i, _vp, _i, _i, _i, _i, _i, _i,
                               _f, _vp, _vp, _i, _i, _vp]),
    "pa_decode_multi_query": (_i, [_vp, _vp, _i, _i, _vp, _vp, _i, _vp, _i, _vp, _i, _i, _i, _i,
                                   _i, _i, _f, _vp, _vp, _i, _i, _vp, _sz, _vp]),
    "pa_decode_stages": (_i, [_vp, _vp, _i, _i, _vp, _vp, _i, _vp, _i, _vp, _i, _i, _i, _i,
                              _i, _i, _f, _vp, _vp, _i, _i, _vp, _sz, _i, _vp]),
    "pa_decode_shared_prefix_workspace_size": (_sz, [_i, _i, _i, _i, _i, _i, _i, _i]),
    "pa_decode_shared_prefix": (_i, [_vp, _vp, _i, _i, _vp, _vp, _i, _vp, _i, _vp, _i, _vp, _i, _i,
                                     _i, _i, _i, _i, _f, _vp, _vp, _i, _i, _vp, _sz, _vp]),
    "pa_decode_partitions": (_i, [_vp, _vp, _i, _vp, _i, _vp, _vp, _i, _vp, _i, _vp, _i, _i, _i,
                                  _i, _i, _i, _f, _vp, _vp, _i, _i, _vp]),
    "pa_merge_partitions": (_i, [_vp, _i, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _vp]),
    "pa_prefill_chunk": (_i, [_vp, _vp, _vp, _i, _vp, _i, _i, _vp, _vp, _i, _vp, _i, _vp, _i,
                              _i, _i, _i, _i, _i, _f, _vp, _vp, _vp]),
    "pa_write_kv": (_i, [_vp, _vp, _i, _vp, _vp, _i, _i, _i, _vp, _i, _i, _i, _i, _i, _vp, _vp,
                         _vp]),
    "pa_mixed_step": (_i, [_vp, _vp, _vp, _i, _vp, _i, _i, _i, _vp, _sz,
                           _vp, _vp, _vp, _vp, _i, _i, _vp, _i, _vp, _i,
                           _i, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _vp, _vp, _vp]),
    "pa_stream_read": (_i, [_vp, _sz, _i, _vp, _vp]),
}


class PAError(RuntimeError):
    """A libpa call returned a non-zero status."""

    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {status_string(status)}")


def _load(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python paged_kv_cache_22_amd/build.py`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


def status_string(status: int) -> str:
    return lib.pa_status_string(int(status)).decode()


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise PAError(fn, status)


# ---------------------------------------------------------------------------
# tensor marshalling
# ---------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _dtype_code(t, kv: bool) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return PA_F32
    if t.dtype == torch.bfloat16:
        return PA_BF16
    if kv and t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return PA_FP8_E4M3
    raise TypeError(f"unsupported dtype {t.dtype}")


def _dev(t, name: str):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (libpa has no CPU path)")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream(t) -> int:
    torch = _torch()
    return torch.cuda.current_stream(t.device).cuda_stream


def decode_workspace_size(num_seqs: int, num_q_heads: int, head_dim: int, max_seq_len: int,
                          partition_size: int) -> int:
    return int(lib.pa_decode_workspace_size(num_seqs, num_q_heads, head_dim, max_seq_len,
                                            partition_size))


def _cache_dims(k_cache, v_cache, d):
    """(NB, Hkv, block size) of a paged cache: a block of bs tokens is
    n = bs / 16 sub-blocks, k_cache [NB, n, Hkv, d/X, 16, X] (X = dims per
    16 bytes) and v_cache [NB, n, Hkv, d, 16]; 16-token blocks may leave the
    n axis out."""
    if k_cache.dim() == 5:
        NB, Hkv, nchunk, t, x = k_cache.shape
        n = 1
        vshape = (NB, Hkv, d, 16)
    elif k_cache.dim() == 6:
        NB, n, Hkv, nchunk, t, x = k_cache.shape
        vshape = (NB, n, Hkv, d, 16)
    else:
        raise ValueError("k_cache must be [NB, n, Hkv, d/X, 16, X] (or [NB, Hkv, d/X, 16, X])")
    if t != 16 or n not in (1, 2, 4):
        raise ValueError("the cache holds 16-token sub-blocks, 1, 2 or 4 per block")
    if x * k_cache.element_size() != 16 or nchunk * x != d:
        raise ValueError(f"k_cache chunks must hold 16 bytes ({16 // k_cache.element_size()} "
                         f"dims) and cover head_dim {d}")
    if tuple(v_cache.shape) != vshape:
        raise ValueError(f"v_cache must be {list(vshape)}")
    return NB, Hkv, 16 * n


def _kv_dims(q, k_cache, v_cache):
    """Shapes of q [B, Hq, d] and the paged cache."""
    B, Hq, d = q.shape
    NB, Hkv, bs = _cache_dims(k_cache, v_cache, d)
    return B, Hq, d, NB, Hkv, bs


def decode(q, k_cache, v_cache, block_table, seq_lens, *, max_seq_len: int,
           scale: Optional[float] = None, partition_size: int = 0, k_scale=None, v_scale=None,
           out=None, workspace=None):
    """Decode attention (pa_decode).  Returns ``out`` [B, Hq, d] in q's dtype.
    ``workspace`` (uint8, at least decode_workspace_size bytes) is allocated
    here when None."""
    torch = _torch()
    B, Hq, d, NB, Hkv, bs = _kv_dims(q, k_cache, v_cache)
    if out is None:
        out = torch.empty_like(q)
    if scale is None:
        scale = d ** -0.5
    ws_need = decode_workspace_size(B, Hq, d, max_seq_len, partition_size)
    if workspace is None and ws_need:
        workspace = torch.empty(ws_need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.pa_decode(_dev(out, "out"), _dev(q, "q"), _dtype_code(q, False),
                       _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _dtype_code(k_cache, True),
                       _dev(block_table, "block_table"), block_table.shape[1],
                       _dev(seq_lens, "seq_lens"), B, Hq, Hkv, d, bs, NB, float(scale),
                       _dev(k_scale, "k_scale"), _dev(v_scale, "v_scale"),
                       int(partition_size), int(max_seq_len),
                       _dev(workspace, "workspace"), ws_bytes, _stream(q))
    _check("pa_decode", st)
    return out


STATIC_WORKSPACE_BYTES = 64 << 20   # PA_STATIC_WORKSPACE_BYTES
STREAM_READ_SINK_WORDS = 2048       # PA_STREAM_READ_SINK_WORDS


def decode_noalloc(q, k_cache, v_cache, block_table, seq_lens, *, max_seq_len: int, out,
                   scale: Optional[float] = None, partition_size: int = 0, k_scale=None,
                   v_scale=None):
    """pa_decode_noalloc: pa_decode with the library's fixed device workspace;
    ``out`` (caller-owned, [B, Hq, d] in q's dtype) is written, nothing is
    allocated."""
    B, Hq, d, NB, Hkv, bs = _kv_dims(q, k_cache, v_cache)
    if scale is None:
        scale = d ** -0.5
    st = lib.pa_decode_noalloc(_dev(out, "out"), _dev(q, "q"), _dtype_code(q, False),
                               _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
                               _dtype_code(k_cache, True), _dev(block_table, "block_table"),
                               block_table.shape[1], _dev(seq_lens, "seq_lens"), B, Hq, Hkv, d,
                               bs, NB, float(scale), _dev(k_scale, "k_scale"),
                               _dev(v_scale, "v_scale"), int(partition_size), int(max_seq_len),
                               _stream(q))
    _check("pa_decode_noalloc", st)
    return out


def decode_multi_query(q, k_cache, v_cache, block_table, seq_lens, *, max_seq_len: int,
                       scale: Optional[float] = None, partition_size: int = 0, k_scale=None,
                       v_scale=None, out=None, workspace=None):
    """Multi-query decode (pa_decode_multi_query): q [B, q_len, Hq, d], the
    newest q_len cached tokens of each sequence, causal among themselves.
    Returns out with q's shape and dtype."""
    torch = _torch()
    if q.dim() != 4:
        raise ValueError("q must be [B, q_len, Hq, d]")
    B, qn, Hq, d = q.shape
    _, _, _, NB, Hkv, bs = _kv_dims(q.reshape(B, qn * Hq, d), k_cache, v_cache)
    if out is None:
        out = torch.empty_like(q)
    if scale is None:
        scale = d ** -0.5
    ws_need = decode_workspace_size(B, qn * Hq, d, max_seq_len, partition_size)
    if workspace is None and ws_need:
        workspace = torch.empty(ws_need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.pa_decode_multi_query(_dev(out, "out"), _dev(q, "q"), _dtype_code(q, False), qn,
                                   _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
                                   _dtype_code(k_cache, True), _dev(block_table, "block_table"),
                                   block_table.shape[1], _dev(seq_lens, "seq_lens"), B, Hq, Hkv, d,
                                   bs, NB, float(scale), _dev(k_scale, "k_scale"),
                                   _dev(v_scale, "v_scale"), int(partition_size), int(max_seq_len),
                                   _dev(workspace, "workspace"), ws_bytes, _stream(q))
    _check("pa_decode_multi_query", st)
    return out


def decode_stages(q, k_cache, v_cache, block_table, seq_lens, *, max_seq_len: int, stages: int,
                  out, workspace, scale: Optional[float] = None, partition_size: int = 0,
                  k_scale=None, v_scale=None):
    """pa_decode_stages: run the attention and/or merge stage of a decode
    (q [B, Hq, d] or [B, q_len, Hq, d]) on caller-owned out and workspace."""
    qn = q.shape[1] if q.dim() == 4 else 1
    B, Hq, d = q.shape[0], q.shape[-2], q.shape[-1]
    _, _, _, NB, Hkv, bs = _kv_dims(q.reshape(B, qn * Hq, d), k_cache, v_cache)
    if scale is None:
        scale = d ** -0.5
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.pa_decode_stages(_dev(out, "out"), _dev(q, "q"), _dtype_code(q, False), qn,
                              _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
                              _dtype_code(k_cache, True), _dev(block_table, "block_table"),
                              block_table.shape[1], _dev(seq_lens, "seq_lens"), B, Hq, Hkv, d, bs,
                              NB, float(scale), _dev(k_scale, "k_scale"), _dev(v_scale, "v_scale"),
                              int(partition_size), int(max_seq_len), _dev(workspace, "workspace"),
                              ws_bytes, int(stages), _stream(q))
    _check("pa_decode_stages", st)
    return out


def decode_shared_prefix(q, k_cache, v_cache, prefix_block_table, prefix_len: int, block_table,
                         seq_lens, *, max_seq_len: int, partition_size: int = 1024,
                         scale: Optional[float] = None, k_scale=None, v_scale=None, out=None,
                         workspace=None):
    """Cascade decode over a shared prefix (pa_decode_shared_prefix).  q is
    [B, Hq, d] or [B, q_len, Hq, d]; block_table / seq_lens cover each
    sequence's tokens after the prefix."""
    torch = _torch()
    qn = q.shape[1] if q.dim() == 4 else 1
    B, Hq, d = q.shape[0], q.shape[-2], q.shape[-1]
    _, _, _, NB, Hkv, bs = _kv_dims(q.reshape(B, qn * Hq, d), k_cache, v_cache)
    if out is None:
        out = torch.empty_like(q)
    if scale is None:
        scale = d ** -0.5
    need = int(lib.pa_decode_shared_prefix_workspace_size(B, qn, Hq, Hkv, d, int(prefix_len),
                                                          int(max_seq_len), int(partition_size)))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    st = lib.pa_decode_shared_prefix(_dev(out, "out"), _dev(q, "q"), _dtype_code(q, False), qn,
                                     _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
                                     _dtype_code(k_cache, True),
                                     _dev(prefix_block_table, "prefix_block_table"), int(prefix_len),
                                     _dev(block_table, "block_table"), block_table.shape[1],
                                     _dev(seq_lens, "seq_lens"), B, Hq, Hkv, d, bs, NB, float(scale),
                                     _dev(k_scale, "k_scale"), _dev(v_scale, "v_scale"),
                                     int(partition_size), int(max_seq_len),
                                     _dev(workspace, "workspace"), ws_bytes, _stream(q))
    _check("pa_decode_shared_prefix", st)
    return out


def decode_partitions(q, k_cache, v_cache, block_table, seq_lens, *, max_seq_len: int,
                      partition_size: int, scale: Optional[float] = None, k_scale=None,
                      v_scale=None, partial_out=None, partial_lse=None):
    """Split-KV partition kernel only (pa_decode_partitions).  Returns
    (partial_out [B, Hq, Pmax, d] fp32, partial_lse [B, Hq, Pmax] fp32)."""
    torch = _torch()
    B, Hq, d, NB, Hkv, bs = _kv_dims(q, k_cache, v_cache)
    pmax = max(1, -(-int(max_seq_len) // int(partition_size)))
    if partial_out is None:
        partial_out = torch.empty((B, Hq, pmax, d), dtype=torch.float32, device=q.device)
    if partial_lse is None:
        partial_lse = torch.empty((B, Hq, pmax), dtype=torch.float32, device=q.device)
    if scale is None:
        scale = d ** -0.5
    st = lib.pa_decode_partitions(_dev(partial_out, "partial_out"), _dev(partial_lse, "partial_lse"),
                                  partial_out.shape[2], _dev(q, "q"), _dtype_code(q, False),
                                  _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
                                  _dtype_code(k_cache, True), _dev(block_table, "block_table"),
                                  block_table.shape[1], _dev(seq_lens, "seq_lens"), B, Hq, Hkv, d,
                                  bs, NB, float(scale), _dev(k_scale, "k_scale"),
                                  _dev(v_scale, "v_scale"), int(partition_size), int(max_seq_len),
                                  _stream(q))
    _check("pa_decode_partitions", st)
    return partial_out, partial_lse


def merge_partitions(partial_out, partial_lse, seq_lens, *, partition_size: int,
                     out_dtype=None, out=None, out_lse=None, want_lse: bool = False):
    """Log-sum-exp merge (pa_merge_partitions).  Returns out, or (out, lse)."""
    torch = _torch()
    B, Hq, pmax, d = partial_out.shape
    if out is None:
        out = torch.empty((B, Hq, d), dtype=out_dtype or torch.float32, device=partial_out.device)
    if want_lse and out_lse is None:
        out_lse = torch.empty((B, Hq), dtype=torch.float32, device=partial_out.device)
    st = lib.pa_merge_partitions(_dev(out, "out"), _dtype_code(out, False), _dev(out_lse, "out_lse"),
                                 _dev(partial_out, "partial_out"), _dev(partial_lse, "partial_lse"),
                                 _dev(seq_lens, "seq_lens"), int(partition_size), pmax, B, Hq, d,
                                 _stream(partial_out))
    _check("pa_merge_partitions", st)
    return (out, out_lse) if want_lse else out


def prefill_chunk(q, cu_q_lens, k_cache, v_cache, block_table, seq_lens, *, max_q_len: int,
                  scale: Optional[float] = None, k_scale=None, v_scale=None, out=None,
                  out_lse=None, want_lse: bool = False):
    """Causal chunked prefill (pa_prefill_chunk).  Returns out [total_q, Hq, d]
    (and lse [total_q, Hq] when want_lse)."""
    torch = _torch()
    total_q, Hq, d, NB, Hkv, bs = _kv_dims(q, k_cache, v_cache)
    if out is None:
        out = torch.empty_like(q)
    if want_lse and out_lse is None:
        out_lse = torch.empty((total_q, Hq), dtype=torch.float32, device=q.device)
    if scale is None:
        scale = d ** -0.5
    st = lib.pa_prefill_chunk(_dev(out, "out"), _dev(out_lse, "out_lse"), _dev(q, "q"),
                              _dtype_code(q, False), _dev(cu_q_lens, "cu_q_lens"), total_q,
                              int(max_q_len), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
                              _dtype_code(k_cache, True), _dev(block_table, "block_table"),
                              block_table.shape[1], _dev(seq_lens, "seq_lens"), seq_lens.shape[0],
                              Hq, Hkv, d, bs, NB, float(scale), _dev(k_scale, "k_scale"),
                              _dev(v_scale, "v_scale"), _stream(q))
    _check("pa_prefill_chunk", st)
    return (out, out_lse) if want_lse else out


def mixed_step(dec_q, dec_block_table, dec_seq_lens, pre_q, cu_q_lens, pre_block_table,
               pre_seq_lens, k_cache, v_cache, *, max_seq_len: int, max_q_len: int,
               partition_size: int = PA_PARTITION_BALANCED, scale: Optional[float] = None,
               k_scale=None, v_scale=None, dec_out=None, pre_out=None, pre_out_lse=None,
               want_lse: bool = False, workspace=None):
    """One mixed step (pa_mixed_step): decode rows dec_q [B, Hq, d] and
    prefill chunks pre_q [total_q, Hq, d] over one cache, with the decode
    rows' merge inside the chunks' launch.  Returns (dec_out, pre_out), plus
    the chunks' lse when want_lse."""
    torch = _torch()
    B, Hq, d, NB, Hkv, bs = _kv_dims(dec_q, k_cache, v_cache)
    total_q, Hq_p, d_p = pre_q.shape
    if (Hq_p, d_p) != (Hq, d):
        raise ValueError("pre_q must have dec_q's heads and head_dim")
    if pre_q.dtype != dec_q.dtype:
        raise ValueError("pre_q and dec_q must have one dtype")
    if dec_out is None:
        dec_out = torch.empty_like(dec_q)
    if pre_out is None:
        pre_out = torch.empty_like(pre_q)
    if want_lse and pre_out_lse is None:
        pre_out_lse = torch.empty((total_q, Hq), dtype=torch.float32, device=pre_q.device)
    if scale is None:
        scale = d ** -0.5
    ws_need = decode_workspace_size(B, Hq, d, max_seq_len, partition_size)
    if workspace is None and ws_need:
        workspace = torch.empty(ws_need, dtype=torch.uint8, device=dec_q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.pa_mixed_step(_dev(dec_out, "dec_out"), _dev(dec_q, "dec_q"),
                           _dev(dec_block_table, "dec_block_table"), dec_block_table.shape[1],
                           _dev(dec_seq_lens, "dec_seq_lens"), B, int(max_seq_len),
                           int(partition_size), _dev(workspace, "workspace"), ws_bytes,
                           _dev(pre_out, "pre_out"), _dev(pre_out_lse, "pre_out_lse"),
                           _dev(pre_q, "pre_q"), _dev(cu_q_lens, "cu_q_lens"), total_q,
                           int(max_q_len), _dev(pre_block_table, "pre_block_table"),
                           pre_block_table.shape[1], _dev(pre_seq_lens, "pre_seq_lens"),
                           pre_seq_lens.shape[0], _dtype_code(dec_q, False),
                           _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
                           _dtype_code(k_cache, True), Hq, Hkv, d, bs, NB, float(scale),
                           _dev(k_scale, "k_scale"), _dev(v_scale, "v_scale"), _stream(dec_q))
    _check("pa_mixed_step", st)
    return (dec_out, pre_out, pre_out_lse) if want_lse else (dec_out, pre_out)


def _rows(t, name: str):
    """Pointer and token stride (elements) of a [T, Hkv, d] tensor whose last
    two dims are contiguous (a view into a wider projection output is fine)."""
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (libpa has no CPU path)")
    if t.dim() != 3:
        raise ValueError(f"{name} must be [T, Hkv, d]")
    T, H, D = t.shape
    row = H * D
    if t.numel() == 0:
        return t.data_ptr(), row
    # strides of size-1 dims carry no meaning
    if (D > 1 and t.stride(2) != 1) or (H > 1 and t.stride(1) != D):
        raise ValueError(f"{name} must be [T, Hkv, d] with contiguous (Hkv, d) rows")
    return t.data_ptr(), t.stride(0) if T > 1 else row


def write_kv(key, value, k_cache, v_cache, slot_mapping, *, k_scale=None, v_scale=None):
    """Store new tokens' K/V rows into their cache slots (pa_write_kv), in place.
    key/value [T, Hkv, d] (f32 or bf16); fp8 caches quantise with the per-kv-head
    scales."""
    T, Hkv, d = key.shape
    if tuple(value.shape) != (T, Hkv, d):
        raise ValueError("value must have key's shape")
    NB, Hkv_c, bs = _cache_dims(k_cache, v_cache, d)
    if Hkv_c != Hkv:
        raise ValueError("the cache's kv-heads must match key's")
    if slot_mapping.dim() != 1 or slot_mapping.shape[0] != T:
        raise ValueError("slot_mapping must be [T]")
    kp, ks_ = _rows(key, "key")
    vp, vs_ = _rows(value, "value")
    st = lib.pa_write_kv(_dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
                         _dtype_code(k_cache, True), kp, vp, _dtype_code(key, False),
                         int(ks_), int(vs_), _dev(slot_mapping, "slot_mapping"), T, Hkv, d, bs,
                         NB, _dev(k_scale, "k_scale"), _dev(v_scale, "v_scale"), _stream(key))
    _check("pa_write_kv", st)
    return k_cache, v_cache


def stream_read(buf, *, nontemporal: bool = True, sink=None):
    """Read a device buffer once (pa_stream_read): the measured HBM read rate
    beside which the attention kernels' rates are reported.  Returns the sink,
    STREAM_READ_SINK_WORDS int32 words whose XOR changes by the XOR of the
    buffer's 32-bit words (a new zeroed sink when none is given)."""
    torch = _torch()
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous GPU tensor (libpa has no CPU path)")
    if sink is None:
        sink = torch.zeros(STREAM_READ_SINK_WORDS, dtype=torch.int32, device=buf.device)
    elif sink.numel() * sink.element_size() < 4 * STREAM_READ_SINK_WORDS:
        raise ValueError(f"sink must hold {STREAM_READ_SINK_WORDS} 32-bit words")
    st = lib.pa_stream_read(buf.data_ptr() if buf.numel() else None,
                            buf.numel() * buf.element_size(), int(bool(nontemporal)),
                            _dev(sink, "sink"), _stream(buf))
    _check("pa_stream_read", st)
    return sink
