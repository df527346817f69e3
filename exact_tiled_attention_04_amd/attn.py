"""Thin ctypes binding over libeta_attn.so (see include/attn.h).

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, their device pointers and torch's current HIP stream are passed
to the C ABI, and a non-OK status raises.  Every step of the computation runs
in the library's HIP kernels.  There is no fallback: if the library has not
been built (``python -m exact_tiled_attention_04_amd.build``) the first call
raises.

Names follow the C ABI: ``attn_fwd``, ``attn_fwd_local``, ``attn_fwd_splitkv``,
``attn_fwd_splitkv_workspace_size``, ``attn_fwd_varlen``, ``attn_prefill_paged``,
``attn_fwd_block_sparse``, ``attn_decode_paged``, ``attn_bwd``, ``attn_bwd_local``,
``attn_decode_paged_workspace_size``, ``attn_bwd_workspace_size``,
``attn_plan_describe``, ``attn_status_string``.
"""

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libeta_attn.so")

ATTN_OK = 0
ATTN_ERR_INVALID_ARG = 1
ATTN_ERR_UNSUPPORTED = 2
ATTN_ERR_WORKSPACE = 3
ATTN_ERR_HIP = 4

ATTN_DTYPE_F32 = 0
ATTN_DTYPE_BF16 = 1

ATTN_PHASE_FWD = 0
ATTN_PHASE_DECODE = 1
ATTN_PHASE_BWD = 2

EXPORTED = (
    "attn_fwd",
    "attn_fwd_local",
    "attn_fwd_splitkv_workspace_size",
    "attn_fwd_splitkv",
    "attn_fwd_varlen",
    "attn_prefill_paged",
    "attn_fwd_block_sparse",
    "attn_bwd_local",
    "attn_decode_paged_workspace_size",
    "attn_decode_paged",
    "attn_decode_paged_noalloc_max_bytes",
    "attn_decode_paged_noalloc",
    "attn_bwd_workspace_size",
    "attn_bwd",
    "attn_plan_describe",
    "attn_status_string",
    "attn_last_error",
)

_lib = None


class AttnError(RuntimeError):
    """A non-OK status from the library."""

    def __init__(self, status, detail):
        self.status = status
        super().__init__(f"{_status_name(status)}: {detail}")


def load_library(path=LIB_PATH):
    """Load (once) and return the ctypes handle, with prototypes set."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m exact_tiled_attention_04_amd.build` "
            "(there is no non-HIP fallback)")
    lib = ctypes.CDLL(path)
    vp, i32, i64, f32, sz = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float,
                             ctypes.c_size_t)
    lib.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, i32, i32, vp]
    lib.attn_fwd.restype = i32
    lib.attn_fwd_local.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, i32, i32,
                                   i32, vp]
    lib.attn_fwd_local.restype = i32
    lib.attn_fwd_splitkv_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32]
    lib.attn_fwd_splitkv_workspace_size.restype = sz
    lib.attn_fwd_splitkv.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, i32,
                                     i32, i32, i32, vp, sz, vp]
    lib.attn_fwd_splitkv.restype = i32
    lib.attn_fwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                    f32, i32, i32, i32, vp]
    lib.attn_fwd_varlen.restype = i32
    lib.attn_prefill_paged.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                       i32, i32, i32, i64, i64, i64, f32, i32, i32, i32, vp]
    lib.attn_prefill_paged.restype = i32
    lib.attn_fwd_block_sparse.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32,
                                          i32, vp, vp, i32, i32, i32, vp]
    lib.attn_fwd_block_sparse.restype = i32
    lib.attn_decode_paged_workspace_size.argtypes = [i32, i32, i32, i32, i32]
    lib.attn_decode_paged_workspace_size.restype = sz
    lib.attn_decode_paged.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                      i32, i32, i64, i64, i64, f32, i32, i32, vp, sz, vp]
    lib.attn_decode_paged.restype = i32
    lib.attn_decode_paged_noalloc_max_bytes.argtypes = []
    lib.attn_decode_paged_noalloc_max_bytes.restype = sz
    lib.attn_decode_paged_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                              i32, i32, i32, i64, i64, i64, f32, i32, i32, vp]
    lib.attn_decode_paged_noalloc.restype = i32
    lib.attn_bwd_workspace_size.argtypes = [i32, i32, i32, i32]
    lib.attn_bwd_workspace_size.restype = sz
    lib.attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                             f32, i32, i32, vp, sz, vp]
    lib.attn_bwd.restype = i32
    lib.attn_bwd_local.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                   i32, f32, i32, i32, i32, vp, sz, vp]
    lib.attn_bwd_local.restype = i32
    lib.attn_plan_describe.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32, i32,
                                       ctypes.c_char_p, sz]
    lib.attn_plan_describe.restype = i32
    lib.attn_status_string.argtypes = [i32]
    lib.attn_status_string.restype = ctypes.c_char_p
    lib.attn_last_error.argtypes = []
    lib.attn_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _status_name(status):
    try:
        return load_library().attn_status_string(status).decode()
    except Exception:  # pragma: no cover - only when the library is absent
        return f"status {status}"


def _check(status):
    if status != ATTN_OK:
        raise AttnError(status, load_library().attn_last_error().decode())


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return ATTN_DTYPE_BF16
    if t.dtype == torch.float32:
        return ATTN_DTYPE_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need_device(*ts):
    for t in ts:
        if not t.is_cuda:
            raise ValueError("tensors must live on the GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


# The C ABI sees only pointers, so every extent the kernels rely on is
# checked here, before any launch: a mis-shaped tensor would otherwise be
# read or written past its end.

def _need_shape(t, shape, name):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _need_dtype(t, dtype, name):
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def _need_dims(t, n, name):
    if t.dim() != n:
        raise ValueError(f"{name} must have {n} dimensions, got {t.dim()}")


def _out_lse(out, lse, o_shape, lse_shape, dtype, device):
    """Caller-supplied outputs are checked against the result's extents;
    missing ones are allocated."""
    if out is None:
        out = torch.empty(o_shape, dtype=dtype, device=device)
    _need_shape(out, o_shape, "out")
    _need_dtype(out, dtype, "out")
    if lse is None:
        lse = torch.empty(lse_shape, dtype=torch.float32, device=device)
    _need_shape(lse, lse_shape, "lse")
    _need_dtype(lse, torch.float32, "lse")
    return out, lse


def _fwd_args(q, k, v, out, lse):
    _need_dims(q, 4, "q")
    _need_dims(k, 4, "k")
    B, H, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if k.shape != (B, Hkv, Nk, d) or v.shape != k.shape:
        raise ValueError("k and v must be [B, Hkv, Nk, d]")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share a dtype")
    out, lse = _out_lse(out, lse, (B, H, Nq, d), (B, H, Nq), q.dtype, q.device)
    _need_device(q, k, v, out, lse)
    return (B, H, Hkv, Nq, Nk, d), out, lse


def attn_fwd(q, k, v, scale, causal, out=None, lse=None, stream=None, workspace=None):
    """O, LSE = attention(q, k, v).  q [B,H,Nq,d]; k, v [B,Hkv,Nk,d].

    bf16 grids too small to fill the GPU ("Modern attention kernels", "Work
    partitioning in FlashAttention-2") go through the key-split entry point
    attn_fwd_splitkv, with a workspace of the size the library asks for
    (``workspace`` if given, else allocated here); other calls go to the C
    ABI's attn_fwd, which needs no workspace."""
    lib = load_library()
    dims, out, lse = _fwd_args(q, k, v, out, lse)
    if q.dtype == torch.bfloat16:
        B, H, _, Nq, Nk, d = dims
        right = 0 if causal else -1
        if attn_fwd_splitkv_workspace_size(B, H, Nq, Nk, d, -1, right, 0) > 0:
            return attn_fwd_splitkv(q, k, v, scale, -1, right, 0, out=out, lse=lse,
                                    workspace=workspace, stream=stream)
    _check(lib.attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), *dims, float(scale),
                        int(bool(causal)), _dtype_code(q), _stream(stream)))
    return out, lse


def attn_fwd_local(q, k, v, scale, window_left, window_right, out=None, lse=None, stream=None):
    """attn_fwd with the band p - window_left <= j <= p + window_right (-1: no
    limit on that side); (W - 1, 0) is a sliding window of W keys."""
    lib = load_library()
    dims, out, lse = _fwd_args(q, k, v, out, lse)
    _check(lib.attn_fwd_local(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), *dims,
                              float(scale), int(window_left), int(window_right), _dtype_code(q),
                              _stream(stream)))
    return out, lse


def attn_fwd_splitkv_workspace_size(B, H, Nq, Nk, d, window_left=-1, window_right=-1,
                                    chunk_keys=0):
    return int(load_library().attn_fwd_splitkv_workspace_size(B, H, Nq, Nk, d, window_left,
                                                              window_right, chunk_keys))


def attn_fwd_splitkv(q, k, v, scale, window_left=-1, window_right=-1, chunk_keys=0, out=None,
                     lse=None, workspace=None, stream=None):
    """attn_fwd_local whose query tiles may split their key range over several
    workgroups (chunk_keys = 0: the library decides; the split needs the
    workspace of attn_fwd_splitkv_workspace_size, which is 0 when it does not
    split)."""
    lib = load_library()
    dims, out, lse = _fwd_args(q, k, v, out, lse)
    B, H, _, Nq, Nk, d = dims
    need = attn_fwd_splitkv_workspace_size(B, H, Nq, Nk, d, window_left, window_right,
                                           chunk_keys)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if workspace is not None:
        _need_workspace(workspace, need)
    _check(lib.attn_fwd_splitkv(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), *dims,
                                float(scale), int(window_left), int(window_right),
                                _dtype_code(q), int(chunk_keys), _ptr(workspace),
                                0 if workspace is None else workspace.numel(), _stream(stream)))
    return out, lse


def _need_int32(*ts):
    for t in ts:
        if t.dtype != torch.int32:
            raise TypeError("offset, length and index tensors must be int32")


def _need_workspace(ws, need):
    if ws.dtype != torch.uint8 or ws.dim() != 1:
        raise TypeError("workspace must be a 1-D uint8 tensor")
    if ws.numel() < need:
        raise ValueError(f"workspace holds {ws.numel()} bytes, {need} needed")
    _need_device(ws)


def _need_cache(k_cache, v_cache, dims, strides, d, name="cache"):
    """K and V caches of the same shape and dtype whose (block, token, head)
    strides keep every element of `dims` = (num_blocks, block_size, Hkv)
    heads of d values inside the tensor."""
    if tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("k_cache and v_cache must have the same shape")
    if k_cache.dtype != v_cache.dtype:
        raise TypeError("k_cache and v_cache must share a dtype")
    nb, bs, hkv = dims
    if min(nb, bs, hkv) < 1:
        raise ValueError(f"{name} dimensions must be positive, got {dims}")
    if min(int(x) for x in strides) < 0:
        raise ValueError("cache strides must be non-negative")
    last = (nb - 1) * int(strides[0]) + (bs - 1) * int(strides[1]) + (hkv - 1) * int(strides[2]) + d
    if last > k_cache.numel():
        raise ValueError(f"{name} strides {tuple(strides)} reach element {last}, "
                         f"past the {k_cache.numel()} elements of the cache")


def attn_fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, scale, window_left=-1,
                    window_right=-1, out=None, lse=None, stream=None):
    """Ragged batch in packed layout: q [total_q, H, d]; k, v [total_k, Hkv, d];
    cu_seqlens_q/k int32 [num_seqs + 1] on the device.  Returns O [total_q, H, d]
    and LSE [H, total_q].  (-1, 0) windows give the causal mask."""
    lib = load_library()
    _need_int32(cu_seqlens_q, cu_seqlens_k)
    _need_dims(q, 3, "q")
    _need_dims(k, 3, "k")
    total_q, H, d = q.shape
    total_k, Hkv = k.shape[0], k.shape[1]
    if k.shape != (total_k, Hkv, d) or v.shape != k.shape:
        raise ValueError("k and v must be [total_k, Hkv, d]")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share a dtype")
    num_seqs = cu_seqlens_q.numel() - 1
    if cu_seqlens_k.numel() != num_seqs + 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must have num_seqs + 1 entries")
    out, lse = _out_lse(out, lse, (total_q, H, d), (H, total_q), q.dtype, q.device)
    _need_device(q, k, v, cu_seqlens_q, cu_seqlens_k, out, lse)
    _check(lib.attn_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                               _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), num_seqs, total_q, total_k,
                               int(max_seqlen_q), H, Hkv, d, float(scale), int(window_left),
                               int(window_right), _dtype_code(q), _stream(stream)))
    return out, lse


def attn_prefill_paged(q, k_cache, v_cache, block_table, cu_seqlens_q, seqlens_k, max_seqlen_q,
                       scale, window_left=-1, window_right=-1, num_blocks=None, strides=None,
                       out=None, lse=None, stream=None, cache_dims=None):
    """Ragged queries q [total_q, Hq, d] against a paged cache
    [num_blocks, block_size, Hkv, d] (or ``strides`` = (block, token, head) in
    elements, with ``cache_dims`` = (num_blocks, block_size, Hkv) for other
    shapes); block_table int32 [num_seqs, max_blocks]; cu_seqlens_q int32
    [num_seqs + 1]; seqlens_k int32 [num_seqs].  Each sequence's queries are
    the last positions of its cached context.  Returns O and LSE [Hq, total_q]."""
    lib = load_library()
    _need_int32(block_table, cu_seqlens_q, seqlens_k)
    _need_dims(q, 3, "q")
    _need_dims(block_table, 2, "block_table")
    total_q, Hq, d = q.shape
    nb, block_size, Hkv = _cache_dims(k_cache, cache_dims, d, strides is not None)
    num_blocks = nb if num_blocks is None else num_blocks
    if num_blocks > nb:
        raise ValueError(f"num_blocks {num_blocks} exceeds the cache's {nb} blocks")
    num_seqs = cu_seqlens_q.numel() - 1
    if seqlens_k.numel() != num_seqs or block_table.shape[0] != num_seqs:
        raise ValueError("seqlens_k and block_table must have num_seqs rows")
    if strides is None:
        strides = (block_size * Hkv * d, Hkv * d, d)
    _need_cache(k_cache, v_cache, (nb, block_size, Hkv), strides, d)
    if k_cache.dtype != q.dtype:
        raise TypeError("q and the caches must share a dtype")
    out, lse = _out_lse(out, lse, (total_q, Hq, d), (Hq, total_q), q.dtype, q.device)
    _need_device(q, k_cache, v_cache, block_table, cu_seqlens_q, seqlens_k, out, lse)
    _check(lib.attn_prefill_paged(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(cu_seqlens_q),
        _ptr(seqlens_k), _ptr(out), _ptr(lse), num_seqs, total_q, int(max_seqlen_q), Hq, Hkv, d,
        block_size, int(num_blocks), block_table.shape[1], int(strides[0]), int(strides[1]),
        int(strides[2]), float(scale), int(window_left), int(window_right), _dtype_code(q),
        _stream(stream)))
    return out, lse


def attn_fwd_block_sparse(q, k, v, scale, causal, row_ptr, col_idx, out=None, lse=None,
                          stream=None):
    """attn_fwd restricted to the listed 128x128 score blocks: row_ptr int32
    [num_layouts, ceil(Nq/128) + 1], col_idx int32 [nnz] (device); (b, h) uses
    layout (b*H + h) % num_layouts."""
    lib = load_library()
    dims, out, lse = _fwd_args(q, k, v, out, lse)
    _need_device(row_ptr, col_idx)
    _need_int32(row_ptr, col_idx)
    B, H, _, Nq, _, _ = dims
    if row_ptr.dim() != 2 or row_ptr.shape[1] != (Nq + 127) // 128 + 1:
        raise ValueError("row_ptr must be [num_layouts, ceil(Nq/128) + 1]")
    _check(lib.attn_fwd_block_sparse(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), *dims,
                                     float(scale), int(bool(causal)), _ptr(row_ptr),
                                     _ptr(col_idx), row_ptr.shape[0], col_idx.numel(),
                                     _dtype_code(q), _stream(stream)))
    return out, lse


def attn_decode_paged_workspace_size(num_seqs, Hq, d, max_context, chunk_tokens=0):
    return int(load_library().attn_decode_paged_workspace_size(num_seqs, Hq, d, max_context,
                                                               chunk_tokens))


def _cache_dims(k_cache, cache_dims, d, strided):
    """(num_blocks, block_size, Hkv): from a [blocks, slots, heads, d] shape
    (rows of more than d values only with explicit strides), or given
    explicitly for other layouts (e.g. head-major pages via strides)."""
    if cache_dims is not None:
        if len(cache_dims) != 3:
            raise ValueError("cache_dims must be (num_blocks, block_size, Hkv)")
        return tuple(int(x) for x in cache_dims)
    _need_dims(k_cache, 4, "k_cache")
    if k_cache.shape[3] < d or (not strided and k_cache.shape[3] != d):
        raise ValueError(f"k_cache rows hold {k_cache.shape[3]} values, q has d = {d}")
    return k_cache.shape[0], k_cache.shape[1], k_cache.shape[2]


def attn_decode_paged(q, k_cache, v_cache, block_table, context_lens, scale, max_context,
                      chunk_tokens=0, strides=None, out=None, lse=None, workspace=None,
                      stream=None, cache_dims=None):
    """Paged GQA decode.

    q [num_seqs, Hq, d]; k_cache, v_cache [num_blocks, block_size, Hkv, d]
    (or any layout described by ``strides`` = (block, token, head) in
    elements, with ``cache_dims`` = (num_blocks, block_size, Hkv) when the
    tensor's shape is not [blocks, slots, heads, d]); block_table int32
    [num_seqs, max_blocks]; context_lens int32 [num_seqs] on the device.
    ``chunk_tokens`` > 0 fixes the tokens per split work item (a multiple of
    32 up to 4064); 0 lets the device cut the contexts of all (sequence, KV
    head) pairs, laid end to end, into equal ranges.
    """
    lib = load_library()
    _need_int32(block_table, context_lens)
    _need_dims(q, 3, "q")
    _need_dims(block_table, 2, "block_table")
    num_seqs, Hq, d = q.shape
    num_blocks, block_size, Hkv = _cache_dims(k_cache, cache_dims, d, strides is not None)
    if block_table.shape[0] != num_seqs:
        raise ValueError(f"block_table has {block_table.shape[0]} rows for {num_seqs} sequences")
    if context_lens.numel() != num_seqs:
        raise ValueError(f"context_lens has {context_lens.numel()} entries for {num_seqs} sequences")
    max_blocks = block_table.shape[1]
    if strides is None:
        strides = (block_size * Hkv * d, Hkv * d, d)
    _need_cache(k_cache, v_cache, (num_blocks, block_size, Hkv), strides, d)
    if k_cache.dtype != q.dtype:
        raise TypeError("q and the caches must share a dtype")
    out, lse = _out_lse(out, lse, (num_seqs, Hq, d), (num_seqs, Hq), q.dtype, q.device)
    need = attn_decode_paged_workspace_size(num_seqs, Hq, d, max_context, chunk_tokens)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _need_workspace(workspace, need)
    _need_device(q, k_cache, v_cache, block_table, context_lens, out, lse)
    _check(lib.attn_decode_paged(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(context_lens),
        _ptr(out), _ptr(lse), num_seqs, Hq, Hkv, d, block_size, num_blocks, max_blocks,
        int(max_context), int(strides[0]), int(strides[1]), int(strides[2]), float(scale),
        _dtype_code(q), int(chunk_tokens), _ptr(workspace), workspace.numel(), _stream(stream)))
    return out, lse


def attn_decode_paged_noalloc_max_bytes():
    return int(load_library().attn_decode_paged_noalloc_max_bytes())


def attn_decode_paged_noalloc(q, k_cache, v_cache, block_table, context_lens, scale, max_context,
                              out, lse, chunk_tokens=0, strides=None, stream=None,
                              cache_dims=None):
    """attn_decode_paged without a workspace: the library's static scratch
    holds the partials, so the call allocates nothing (``out`` [num_seqs, Hq,
    d] and ``lse`` [num_seqs, Hq] float32 are the caller's).  Calls that
    overlap on one GPU share that scratch and race."""
    lib = load_library()
    _need_int32(block_table, context_lens)
    _need_dims(q, 3, "q")
    _need_dims(block_table, 2, "block_table")
    num_seqs, Hq, d = q.shape
    num_blocks, block_size, Hkv = _cache_dims(k_cache, cache_dims, d, strides is not None)
    if block_table.shape[0] != num_seqs:
        raise ValueError(f"block_table has {block_table.shape[0]} rows for {num_seqs} sequences")
    if context_lens.numel() != num_seqs:
        raise ValueError(f"context_lens has {context_lens.numel()} entries for {num_seqs} sequences")
    if strides is None:
        strides = (block_size * Hkv * d, Hkv * d, d)
    _need_cache(k_cache, v_cache, (num_blocks, block_size, Hkv), strides, d)
    if k_cache.dtype != q.dtype:
        raise TypeError("q and the caches must share a dtype")
    if out is None or lse is None:
        raise ValueError("out and lse must be given (this entry point allocates nothing)")
    _need_shape(out, (num_seqs, Hq, d), "out")
    _need_dtype(out, q.dtype, "out")
    _need_shape(lse, (num_seqs, Hq), "lse")
    _need_dtype(lse, torch.float32, "lse")
    _need_device(q, k_cache, v_cache, block_table, context_lens, out, lse)
    _check(lib.attn_decode_paged_noalloc(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(context_lens),
        _ptr(out), _ptr(lse), num_seqs, Hq, Hkv, d, block_size, num_blocks,
        block_table.shape[1], int(max_context), int(strides[0]), int(strides[1]),
        int(strides[2]), float(scale), _dtype_code(q), int(chunk_tokens), _stream(stream)))
    return out, lse


def attn_bwd_workspace_size(B, H, Nq, d):
    return int(load_library().attn_bwd_workspace_size(B, H, Nq, d))


def _bwd_args(q, k, v, o, do, lse, dq, dk, dv, workspace):
    _need_dims(q, 4, "q")
    _need_dims(k, 4, "k")
    B, H, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if k.shape != (B, Hkv, Nk, d) or v.shape != k.shape:
        raise ValueError("k and v must be [B, Hkv, Nk, d]")
    for t, name in ((k, "k"), (v, "v"), (o, "o"), (do, "do")):
        _need_dtype(t, q.dtype, name)
    _need_shape(o, q.shape, "o")
    _need_shape(do, q.shape, "do")
    _need_shape(lse, (B, H, Nq), "lse")
    _need_dtype(lse, torch.float32, "lse")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for t, ref, name in ((dq, q, "dq"), (dk, k, "dk"), (dv, v, "dv")):
        _need_shape(t, ref.shape, name)
        _need_dtype(t, q.dtype, name)
    need = attn_bwd_workspace_size(B, H, Nq, d)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _need_workspace(workspace, need)
    _need_device(q, k, v, o, do, lse, dq, dk, dv)
    return (B, H, Hkv, Nq, Nk, d), dq, dk, dv, workspace


def attn_bwd(q, k, v, o, do, lse, scale, causal, dq=None, dk=None, dv=None, workspace=None,
             stream=None):
    """dQ, dK, dV of attention given the forward's O and LSE."""
    lib = load_library()
    dims, dq, dk, dv, workspace = _bwd_args(q, k, v, o, do, lse, dq, dk, dv, workspace)
    _check(lib.attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq),
                        _ptr(dk), _ptr(dv), *dims, float(scale), int(bool(causal)),
                        _dtype_code(q), _ptr(workspace), workspace.numel(), _stream(stream)))
    return dq, dk, dv


def attn_bwd_local(q, k, v, o, do, lse, scale, window_left, window_right, dq=None, dk=None,
                   dv=None, workspace=None, stream=None):
    """attn_bwd for the band of attn_fwd_local."""
    lib = load_library()
    dims, dq, dk, dv, workspace = _bwd_args(q, k, v, o, do, lse, dq, dk, dv, workspace)
    _check(lib.attn_bwd_local(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse),
                              _ptr(dq), _ptr(dk), _ptr(dv), *dims, float(scale),
                              int(window_left), int(window_right), _dtype_code(q),
                              _ptr(workspace), workspace.numel(), _stream(stream)))
    return dq, dk, dv


def attn_plan_describe(phase, B, H, Hkv, Nq, Nk, d, causal, dtype=ATTN_DTYPE_BF16):
    lib = load_library()
    buf = ctypes.create_string_buffer(512)
    n = lib.attn_plan_describe(phase, B, H, Hkv, Nq, Nk, d, int(bool(causal)), dtype, buf, 512)
    if n < 0:
        raise ValueError("invalid arguments for attn_plan_describe")
    return buf.value.decode()


def attn_status_string(status):
    return load_library().attn_status_string(status).decode()
