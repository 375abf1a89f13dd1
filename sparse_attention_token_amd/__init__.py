"""Python binding of libdsi.so, the gfx950 DeepSeek Sparse Attention lightning-indexer library.

Argument marshalling only: every step runs in the library's HIP kernels, on the
caller's current torch stream.  PyTorch supplies device memory and streams.
There is no fallback: if the library is missing or a call is rejected, an
exception is raised.

Names mirror the C ABI in include/dsi.h (without the ``dsi_`` prefix).  bf16
arrays may be torch.bfloat16 or their 16-bit patterns (int16/uint16); FP8
codes are uint8.  Outputs can be passed with ``out=`` (no allocation on the
hot path) or are allocated here when omitted.
"""
import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdsi.so")

HEADS, HEAD_DIM, ROW_BYTES, MAX_TOPK = 64, 128, 132, 2048
ROW_BYTES_MXFP4 = 68
F32, BF16 = 0, 1


class DsiError(RuntimeError):
    """A dsi_* call returned a negative status."""


_lib = None
_p, _i32, _i64, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t

_SIGNATURES = {
    "dsi_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "dsi_abi_version": (ctypes.c_int, []),
    "dsi_k_quant_and_cache": (ctypes.c_int, [_p, _i64, _i64, _p, _p, _i64, _i32, _i64, _p]),
    "dsi_mqa_logits_prefill": (ctypes.c_int, [_p, _p, _i32, _p, _i32, _p, _p, _p, _i64, _p]),
    "dsi_paged_mqa_logits_decode": (ctypes.c_int, [_p, _p, _i32, _i32, _p, _p, _i64, _i32, _i64, _p, _i64, _i32,
                                                   _i32, _p, _i64, _p]),
    "dsi_paged_mqa_logits_decode_mxfp4": (ctypes.c_int, [_p, _p, _i32, _i32, _p, _p, _i64, _i32, _i64, _p, _i64,
                                                         _i32, _i32, _p, _i64, _p]),
    "dsi_topk_workspace_bytes": (_sz, [_i32, _i32, _i32]),
    "dsi_paged_mqa_topk_decode_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32]),
    "dsi_paged_mqa_topk_decode": (ctypes.c_int, [_p, _p, _i32, _i32, _p, _p, _i64, _i32, _i64, _p, _i64, _i32, _i32,
                                                 _p, _i64, _i32, _p, _i64, _p, _sz, _p]),
    "dsi_paged_mqa_topk_decode_mxfp4": (ctypes.c_int, [_p, _p, _i32, _i32, _p, _p, _i64, _i32, _i64, _p, _i64, _i32,
                                                       _i32, _p, _i64, _i32, _p, _i64, _p, _sz, _p]),
    "dsi_topk_select": (ctypes.c_int, [_p, _i32, _i64, _i32, _p, _p, _i32, _i32, _p, _i64, _p, _sz, _p]),
    "dsi_topk_select_noalloc": (ctypes.c_int, [_p, _i32, _i64, _i32, _p, _p, _i32, _i32, _p, _i64, _p]),
    "dsi_expand_candidates": (ctypes.c_int, [_p, _i64, _i32, _i32, _p, _i64, _p, _i64, _i32, _i32, _p, _i64, _p,
                                             _i64, _p]),
    "dsi_sparse_mqa_logits": (ctypes.c_int, [_p, _p, _i32, _p, _p, _p, _i64, _i32, _p, _i32, _p, _i64, _p, _i64,
                                             _i32, _i32, _p, _i32, _i64, _p, _i64, _p]),
    "dsi_topk_remap": (ctypes.c_int, [_p, _i64, _i32, _i32, _p, _i64, _i32, _p, _i32, _p, _i64, _p]),
    "dsi_sparse_schedule_bytes": (_sz, [_i32, _i32]),
    "dsi_sparse_schedule": (ctypes.c_int, [_i32, _p, _p, _p, _i64, _i32, _p, _i32, _i32, _i64, _p, _i64, _i32, _i32,
                                           _p, _i32, _i64, _p, _p]),
    "dsi_sparse_mqa_logits_scheduled": (ctypes.c_int, [_p, _p, _i32, _p, _i32, _i32, _p, _i64, _p, _i64, _p]),
    "dsi_sparse_mqa_logits_scheduled_mxfp4": (ctypes.c_int, [_p, _p, _i32, _p, _i32, _i32, _p, _i64, _p, _i64, _p]),
    "dsi_req_index_to_global_slot": (ctypes.c_int, [_p, _i64, _i32, _i32, _p, _p, _i64, _i32, _i32, _i32, _i32, _p,
                                                    _i64, _p]),
    "dsi_gather_prefill_k": (ctypes.c_int, [_p, _i64, _i32, _i64, _p, _i64, _i32, _p, _i32, _p, _i32, _p]),
    "dsi_topk_values": (ctypes.c_int, [_p, _i64, _i32, _p, _i32, _p, _i64, _i32, _i32, _i32, _p, _i64, _p, _i64, _p]),
    "dsi_topk_merge_workspace_bytes": (_sz, [_i32, _i32, _i32]),
    "dsi_topk_merge": (ctypes.c_int, [_p, _p, _i64, _i64, _i32, _i32, _i32, _i32, _p, _i64, _p, _sz, _p]),
    "dsi_k_quant_and_cache_mxfp4": (ctypes.c_int, [_p, _i64, _i64, _p, _p, _i64, _i32, _i64, _p]),
    "dsi_sparse_mqa_logits_mxfp4": (ctypes.c_int, [_p, _p, _i32, _p, _p, _p, _i64, _i32, _p, _i32, _p, _i64, _p,
                                                   _i64, _i32, _i32, _p, _i32, _i64, _p, _i64, _p]),
    "dsi_q_rope_quant": (ctypes.c_int, [_p, _i64, _i32, _p, _p, _i64, _i32, _p, _i64, ctypes.c_float,
                                        ctypes.c_float, _p, _p, _p]),
}

ENTRY_POINTS = tuple(_SIGNATURES)


def lib():
    """The loaded library (ctypes.CDLL); raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() or "
                              "python sparse_attention_token_amd/build.py")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def status_string(code: int) -> str:
    return lib().dsi_status_string(code).decode()


def _check(code: int, name: str):
    if code != 0:
        raise DsiError(f"dsi_{name}: {status_string(code)} (status {code})")


def _stream(t: torch.Tensor):
    return torch.cuda.current_stream(t.device).cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def _dev(*ts):
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("all tensors must be on the GPU")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("all tensors must be on the same GPU")
    return dev


def _need(t, dtypes, name, ndim=None):
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name}: expected {ndim} dims, got {tuple(t.shape)}")


def _rows(t, name):
    """Leading dimension of a 2-D tensor whose rows are contiguous."""
    if t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1):
        raise ValueError(f"{name}: need a 2-D tensor with contiguous rows")
    return t.stride(0)


def _contig(t, name):
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


_BF16 = (torch.bfloat16, torch.int16, torch.uint16)
_I32 = (torch.int32,)


def k_quant_and_cache(k, slot_mapping, pool, block_size, block_stride_bytes=None, num_blocks=None):
    """Quantize bf16 k [n, >=128] into the 132-byte rows of `pool` at `slot_mapping` (int64)."""
    dev = _dev(k, slot_mapping, pool)
    _need(k, _BF16, "k")
    _need(slot_mapping, (torch.int64,), "slot_mapping")
    _need(pool, (torch.uint8,), "pool")
    _contig(pool, "pool")
    k_ld = _rows(k, "k")
    if block_stride_bytes is None:
        block_stride_bytes = pool.stride(0) if pool.dim() > 1 else block_size * ROW_BYTES
    if num_blocks is None:
        num_blocks = pool.numel() // block_stride_bytes
    n = k.shape[0]
    with torch.cuda.device(dev):
        _check(lib().dsi_k_quant_and_cache(_ptr(k), n, k_ld, _ptr(slot_mapping), _ptr(pool), num_blocks,
                                           block_size, block_stride_bytes, _stream(k)), "k_quant_and_cache")
    return pool


def mqa_logits_prefill(q, w, k_rows, row_ks, row_ke, out=None):
    """Dense logits over gathered K rows [S,132]; fp32 out [T, >=S] (entries outside [ks,ke) untouched)."""
    dev = _dev(q, w, k_rows, row_ks, row_ke, out)
    _need(q, (torch.uint8,), "q", 3)
    _need(w, _BF16, "w", 2)
    _need(k_rows, (torch.uint8,), "k_rows")
    for t, nm in ((q, "q"), (w, "w"), (k_rows, "k_rows"), (row_ks, "row_ks"), (row_ke, "row_ke")):
        _contig(t, nm)
    T, S = q.shape[0], k_rows.numel() // ROW_BYTES
    if out is None:
        out = torch.empty((T, S), dtype=torch.float32, device=dev)
    _need(out, (torch.float32,), "out")
    ld = _rows(out, "out")
    with torch.cuda.device(dev):
        _check(lib().dsi_mqa_logits_prefill(_ptr(q), _ptr(w), T, _ptr(k_rows), S, _ptr(row_ks), _ptr(row_ke),
                                            _ptr(out), ld, _stream(q)), "mqa_logits_prefill")
    return out


def paged_mqa_logits_decode(q, w, context_lens, pool, block_size, block_table, max_context_len, next_n=1,
                            out=None, block_stride_bytes=None, num_blocks=None, bt_width=None, mxfp4=False):
    """Decode logits straight from the paged pool; fp32 out [B*next_n, >=max_context_len].
    mxfp4=True reads 68-byte MXFP4 rows (dsi_paged_mqa_logits_decode_mxfp4) instead of 132-byte FP8 rows."""
    dev = _dev(q, w, context_lens, pool, block_table, out)
    _need(q, (torch.uint8,), "q", 3)
    _need(w, _BF16, "w", 2)
    _need(context_lens, _I32, "context_lens")
    _need(block_table, _I32, "block_table")
    for t, nm in ((q, "q"), (w, "w"), (context_lens, "context_lens"), (pool, "pool")):
        _contig(t, nm)
    B = context_lens.shape[0]
    if block_stride_bytes is None:
        block_stride_bytes = pool.stride(0) if pool.dim() > 1 else block_size * (ROW_BYTES_MXFP4 if mxfp4 else ROW_BYTES)
    if num_blocks is None:
        num_blocks = pool.numel() // block_stride_bytes
    bt_ld = _rows(block_table, "block_table")
    if bt_width is None:
        bt_width = block_table.shape[1]
    if out is None:
        out = torch.empty((B * next_n, max_context_len), dtype=torch.float32, device=dev)
    _need(out, (torch.float32,), "out")
    ld = _rows(out, "out")
    fn = lib().dsi_paged_mqa_logits_decode_mxfp4 if mxfp4 else lib().dsi_paged_mqa_logits_decode
    with torch.cuda.device(dev):
        _check(fn(_ptr(q), _ptr(w), B, next_n, _ptr(context_lens), _ptr(pool), num_blocks, block_size,
                  block_stride_bytes, _ptr(block_table), bt_ld, bt_width, max_context_len, _ptr(out), ld, _stream(q)),
               "paged_mqa_logits_decode_mxfp4" if mxfp4 else "paged_mqa_logits_decode")
    return out


def paged_mqa_topk_decode_workspace_bytes(B, next_n, max_context_len, k=MAX_TOPK):
    return lib().dsi_paged_mqa_topk_decode_workspace_bytes(B, next_n, max_context_len, k)


def paged_mqa_topk_decode(q, w, context_lens, pool, block_size, block_table, max_context_len, next_n=1, k=MAX_TOPK,
                          logits=None, out=None, workspace=None, block_stride_bytes=None, num_blocks=None,
                          bt_width=None, mxfp4=False):
    """The decode step in one call: logits straight from the paged pool (fp32 [B*next_n, >=max_context_len]) and
    their top-k (int32 [B*next_n, k], request-local positions, -1 padded).  Returns (logits, out)."""
    dev = _dev(q, w, context_lens, pool, block_table, logits, out, workspace)
    _need(q, (torch.uint8,), "q", 3)
    _need(w, _BF16, "w", 2)
    _need(context_lens, _I32, "context_lens")
    _need(block_table, _I32, "block_table")
    for t, nm in ((q, "q"), (w, "w"), (context_lens, "context_lens"), (pool, "pool")):
        _contig(t, nm)
    B = context_lens.shape[0]
    if block_stride_bytes is None:
        block_stride_bytes = pool.stride(0) if pool.dim() > 1 else block_size * (ROW_BYTES_MXFP4 if mxfp4 else ROW_BYTES)
    if num_blocks is None:
        num_blocks = pool.numel() // block_stride_bytes
    bt_ld = _rows(block_table, "block_table")
    if bt_width is None:
        bt_width = block_table.shape[1]
    if logits is None:
        logits = torch.empty((B * next_n, max_context_len), dtype=torch.float32, device=dev)
    if out is None:
        out = torch.empty((B * next_n, k), dtype=torch.int32, device=dev)
    _need(logits, (torch.float32,), "logits")
    _need(out, _I32, "out")
    need = paged_mqa_topk_decode_workspace_bytes(B, next_n, max_context_len, k)
    ws_ptr, ws_bytes = None, 0
    if need:
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    fn = lib().dsi_paged_mqa_topk_decode_mxfp4 if mxfp4 else lib().dsi_paged_mqa_topk_decode
    with torch.cuda.device(dev):
        _check(fn(_ptr(q), _ptr(w), B, next_n, _ptr(context_lens), _ptr(pool), num_blocks, block_size,
                  block_stride_bytes, _ptr(block_table), bt_ld, bt_width, max_context_len, _ptr(logits),
                  _rows(logits, "logits"), k, _ptr(out), _rows(out, "out"), ws_ptr, ws_bytes, _stream(q)),
               "paged_mqa_topk_decode_mxfp4" if mxfp4 else "paged_mqa_topk_decode")
    return logits, out


def topk_workspace_bytes(rows, max_width, k):
    return lib().dsi_topk_workspace_bytes(rows, max_width, k)


def topk_select(logits, row_ends, k=MAX_TOPK, row_starts=None, max_width=None, out=None, workspace=None):
    """Top-k per row of fp32 or bf16 logits -> int32 [rows, k], request-relative, -1 padded."""
    dev = _dev(logits, row_ends, row_starts, out, workspace)
    if logits.dtype == torch.float32:
        dtype = F32
    elif logits.dtype in _BF16:
        dtype = BF16
    else:
        raise TypeError(f"logits: unsupported dtype {logits.dtype}")
    ld = _rows(logits, "logits")
    rows = logits.shape[0]
    if max_width is None:
        max_width = logits.shape[1]
    if out is None:
        out = torch.empty((rows, k), dtype=torch.int32, device=dev)
    _need(out, _I32, "out")
    out_ld = _rows(out, "out")
    need = topk_workspace_bytes(rows, max_width, k)
    ws_ptr, ws_bytes = None, 0
    if need:
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    with torch.cuda.device(dev):
        _check(lib().dsi_topk_select(_ptr(logits), dtype, ld, rows, _ptr(row_starts), _ptr(row_ends), max_width, k,
                                     _ptr(out), out_ld, ws_ptr, ws_bytes, _stream(logits)), "topk_select")
    return out


def topk_select_noalloc(logits, row_ends, out, k=MAX_TOPK, row_starts=None, max_width=None):
    """topk_select with no workspace argument and no allocation: the library's per-GPU scratch array is used
    (calls that overlap on one GPU race).  `out` int32 [rows, >=k] is required."""
    dev = _dev(logits, row_ends, row_starts, out)
    if logits.dtype == torch.float32:
        dtype = F32
    elif logits.dtype in _BF16:
        dtype = BF16
    else:
        raise TypeError(f"logits: unsupported dtype {logits.dtype}")
    _need(out, _I32, "out")
    if max_width is None:
        max_width = logits.shape[1]
    with torch.cuda.device(dev):
        _check(lib().dsi_topk_select_noalloc(_ptr(logits), dtype, _rows(logits, "logits"), logits.shape[0],
                                             _ptr(row_starts), _ptr(row_ends), max_width, k, _ptr(out),
                                             _rows(out, "out"), _stream(logits)), "topk_select_noalloc")
    return out


def _vec_stride(t, name):
    if t.dim() != 1:
        raise ValueError(f"{name}: need a 1-D tensor")
    return t.stride(0)


def expand_candidates(cand, row_ks, row_ke, candidate_block_size, sparse_block_kv, out=None):
    """-> (sparse_indices int32 [rows, K*ratio], end int32 [rows]); strided inputs allowed."""
    dev = _dev(cand, row_ks, row_ke)
    _need(cand, _I32, "cand", 2)
    cand_ld = _rows(cand, "cand")
    rows, K = cand.shape
    ratio = candidate_block_size // sparse_block_kv if sparse_block_kv else 0
    if out is None:
        out = (torch.empty((rows, K * max(ratio, 1)), dtype=torch.int32, device=dev),
               torch.empty((rows,), dtype=torch.int32, device=dev))
    si, end = out
    with torch.cuda.device(dev):
        _check(lib().dsi_expand_candidates(_ptr(cand), cand_ld, rows, K, _ptr(row_ks), _vec_stride(row_ks, "row_ks"),
                                           _ptr(row_ke), _vec_stride(row_ke, "row_ke"), candidate_block_size,
                                           sparse_block_kv, _ptr(si), _rows(si, "sparse_indices"), _ptr(end),
                                           _vec_stride(end, "end"), _stream(cand)), "expand_candidates")
    return si, end


def sparse_mqa_logits(q, w, row_ks, row_ke, sparse_indices, end, sparse_block_kv, k_src, block_table=None,
                      row_to_req=None, block_size=0, block_stride_bytes=None, num_k=None, bt_width=None,
                      num_sparse_blocks=None, out=None):
    """bf16 logits on the candidate columns: [rows, num_sparse_blocks*sbk] (as int16 bit patterns)."""
    dev = _dev(q, w, row_ks, row_ke, sparse_indices, end, k_src, block_table, row_to_req, out)
    _need(q, (torch.uint8,), "q", 3)
    _need(w, _BF16, "w", 2)
    for t, nm in ((q, "q"), (w, "w"), (row_ks, "row_ks"), (row_ke, "row_ke"), (end, "end"), (k_src, "k_src")):
        _contig(t, nm)
    rows = q.shape[0]
    si_ld = _rows(sparse_indices, "sparse_indices")
    if num_sparse_blocks is None:
        num_sparse_blocks = sparse_indices.shape[1]
    width = num_sparse_blocks * sparse_block_kv
    bt_ld, num_reqs = 0, 0
    if block_table is not None:
        bt_ld = _rows(block_table, "block_table")
        num_reqs = block_table.shape[0]
        if bt_width is None:
            bt_width = block_table.shape[1]
        if block_stride_bytes is None:
            block_stride_bytes = k_src.stride(0) if k_src.dim() > 1 else block_size * ROW_BYTES
        if num_k is None:
            num_k = k_src.numel() // block_stride_bytes
    else:
        bt_width, block_stride_bytes = 0, 0
        if num_k is None:
            num_k = k_src.numel() // ROW_BYTES
    if out is None:
        out = torch.empty((rows, width), dtype=torch.int16, device=dev)
    _need(out, _BF16, "out")
    ld = _rows(out, "out")
    with torch.cuda.device(dev):
        _check(lib().dsi_sparse_mqa_logits(_ptr(q), _ptr(w), rows, _ptr(row_ks), _ptr(row_ke), _ptr(sparse_indices),
                                           si_ld, num_sparse_blocks, _ptr(end), sparse_block_kv, _ptr(k_src), num_k,
                                           _ptr(block_table), bt_ld, bt_width, num_reqs, _ptr(row_to_req), block_size,
                                           block_stride_bytes, _ptr(out), ld, _stream(q)), "sparse_mqa_logits")
    return out


def sparse_schedule(row_ks, row_ke, sparse_indices, end, sparse_block_kv, k_src, block_table=None, row_to_req=None,
                    block_size=0, block_stride_bytes=None, num_k=None, bt_width=None, num_sparse_blocks=None,
                    mxfp4=False, out=None):
    """The per-step schedule of the sparse columns (one uint64 per row and sparse block, as int64 here): built once
    per step, then passed to sparse_mqa_logits_scheduled for every layer."""
    dev = _dev(row_ks, row_ke, sparse_indices, end, k_src, block_table, row_to_req, out)
    row_bytes = ROW_BYTES_MXFP4 if mxfp4 else ROW_BYTES
    rows = row_ks.shape[0]
    si_ld = _rows(sparse_indices, "sparse_indices")
    if num_sparse_blocks is None:
        num_sparse_blocks = sparse_indices.shape[1]
    bt_ld, num_reqs = 0, 0
    if block_table is not None:
        bt_ld = _rows(block_table, "block_table")
        num_reqs = block_table.shape[0]
        if bt_width is None:
            bt_width = block_table.shape[1]
        if block_stride_bytes is None:
            block_stride_bytes = k_src.stride(0) if k_src.dim() > 1 else block_size * row_bytes
        if num_k is None:
            num_k = k_src.numel() // block_stride_bytes
    else:
        bt_width, block_stride_bytes = 0, 0
        if num_k is None:
            num_k = k_src.numel() // row_bytes
    if out is None:
        out = torch.empty((rows, num_sparse_blocks), dtype=torch.int64, device=dev)
    _need(out, (torch.int64,), "schedule")
    _contig(out, "schedule")
    for t, nm in ((row_ks, "row_ks"), (row_ke, "row_ke"), (end, "end")):
        _contig(t, nm)
    with torch.cuda.device(dev):
        _check(lib().dsi_sparse_schedule(rows, _ptr(row_ks), _ptr(row_ke), _ptr(sparse_indices), si_ld,
                                         num_sparse_blocks, _ptr(end), sparse_block_kv, row_bytes, num_k,
                                         _ptr(block_table), bt_ld, bt_width, num_reqs, _ptr(row_to_req), block_size,
                                         block_stride_bytes, _ptr(out), _stream(row_ks)), "sparse_schedule")
    return out


def sparse_mqa_logits_scheduled(q, w, schedule, sparse_block_kv, k_src, out=None, mxfp4=False):
    """bf16 logits on the candidate columns with the columns' sources from a schedule (sparse_schedule); k_src is any
    K source of the layout the schedule was built for."""
    dev = _dev(q, w, schedule, k_src, out)
    _need(q, (torch.uint8,), "q", 3)
    _need(w, _BF16, "w", 2)
    _need(schedule, (torch.int64,), "schedule", 2)
    for t, nm in ((q, "q"), (w, "w"), (schedule, "schedule"), (k_src, "k_src")):
        _contig(t, nm)
    rows, nsb = schedule.shape
    width = nsb * sparse_block_kv
    if out is None:
        out = torch.empty((rows, width), dtype=torch.int16, device=dev)
    _need(out, _BF16, "out")
    fn = lib().dsi_sparse_mqa_logits_scheduled_mxfp4 if mxfp4 else lib().dsi_sparse_mqa_logits_scheduled
    with torch.cuda.device(dev):
        _check(fn(_ptr(q), _ptr(w), rows, _ptr(schedule), nsb, sparse_block_kv, _ptr(k_src),
                  k_src.numel() * k_src.element_size(), _ptr(out), _rows(out, "out"), _stream(q)),
               "sparse_mqa_logits_scheduled_mxfp4" if mxfp4 else "sparse_mqa_logits_scheduled")
    return out


def topk_remap(col, sparse_indices, row_ks, sparse_block_kv, out=None, num_sparse_blocks=None):
    """Sparse columns -> request-local positions (out may be `col` itself)."""
    dev = _dev(col, sparse_indices, row_ks, out)
    _need(col, _I32, "col", 2)
    rows, k = col.shape
    if out is None:
        out = torch.empty_like(col)
    if num_sparse_blocks is None:
        num_sparse_blocks = sparse_indices.shape[1]
    _contig(row_ks, "row_ks")
    with torch.cuda.device(dev):
        _check(lib().dsi_topk_remap(_ptr(col), _rows(col, "col"), rows, k, _ptr(sparse_indices),
                                    _rows(sparse_indices, "sparse_indices"), num_sparse_blocks, _ptr(row_ks),
                                    sparse_block_kv, _ptr(out), _rows(out, "out"), _stream(col)), "topk_remap")
    return out


def req_index_to_global_slot(idx, block_table, block_size, block_span, row_to_req=None, out=None, bt_width=None):
    """Request-local positions -> physical slots block*block_span + offset (out may be `idx`)."""
    dev = _dev(idx, block_table, row_to_req, out)
    _need(idx, _I32, "idx", 2)
    rows, k = idx.shape
    if out is None:
        out = torch.empty_like(idx)
    if bt_width is None:
        bt_width = block_table.shape[1]
    with torch.cuda.device(dev):
        _check(lib().dsi_req_index_to_global_slot(_ptr(idx), _rows(idx, "idx"), rows, k, _ptr(row_to_req),
                                                  _ptr(block_table), _rows(block_table, "block_table"), bt_width,
                                                  block_table.shape[0], block_size, block_span, _ptr(out), _rows(out, "out"),
                                                  _stream(idx)), "req_index_to_global_slot")
    return out


def gather_prefill_k(pool, block_size, block_table, cu_seq_lens, S=None, out=None, block_stride_bytes=None,
                     num_blocks=None, bt_width=None):
    """Paged cache -> contiguous K rows uint8 [S,132] of the chunk's requests laid end to end
    (cu_seq_lens int32 [num_reqs+1]; S defaults to the row count of `out`)."""
    dev = _dev(pool, block_table, cu_seq_lens, out)
    _need(pool, (torch.uint8,), "pool")
    _need(block_table, _I32, "block_table", 2)
    _need(cu_seq_lens, _I32, "cu_seq_lens", 1)
    _contig(pool, "pool")
    _contig(cu_seq_lens, "cu_seq_lens")
    if block_stride_bytes is None:
        block_stride_bytes = pool.stride(0) if pool.dim() > 1 else block_size * ROW_BYTES
    if num_blocks is None:
        num_blocks = pool.numel() // block_stride_bytes
    if bt_width is None:
        bt_width = block_table.shape[1]
    num_reqs = cu_seq_lens.shape[0] - 1
    if num_reqs > block_table.shape[0]:
        raise ValueError("block_table: fewer rows than requests")
    if out is None:
        if S is None:
            raise ValueError("give S (rows to write) or out")
        out = torch.empty((S, ROW_BYTES), dtype=torch.uint8, device=dev)
    _need(out, (torch.uint8,), "out")
    _contig(out, "out")
    if S is None:
        S = out.numel() // ROW_BYTES
    if out.numel() < S * ROW_BYTES:
        raise ValueError("out: fewer than S rows")
    with torch.cuda.device(dev):
        _check(lib().dsi_gather_prefill_k(_ptr(pool), num_blocks, block_size, block_stride_bytes, _ptr(block_table),
                                          _rows(block_table, "block_table"), bt_width, _ptr(cu_seq_lens), num_reqs,
                                          _ptr(out), S, _stream(pool)), "gather_prefill_k")
    return out


def q_rope_quant(q, positions, cos_sin, w, softmax_scale, head_scale, interleave=False, out=None):
    """bf16 q [T,64,128] (or [T, q_ld] rows), int64 positions [T], fp32 cos_sin [max_pos,64], bf16 w [T, >=64]
    -> (e4m3 q8 uint8 [T,64,128], bf16 weights [T,64] as int16 bit patterns)."""
    dev = _dev(q, positions, cos_sin, w)
    _need(q, _BF16, "q")
    _need(positions, (torch.int64,), "positions", 1)
    _need(cos_sin, (torch.float32,), "cos_sin", 2)
    _need(w, _BF16, "w", 2)
    _contig(positions, "positions")
    _contig(cos_sin, "cos_sin")
    T = q.shape[0]
    q2 = q.reshape(T, -1) if q.dim() == 3 and q.is_contiguous() else q
    q_ld = _rows(q2, "q")
    if cos_sin.shape[1] != 64:
        raise ValueError("cos_sin: need [max_pos, 64]")
    if out is None:
        out = (torch.empty((T, HEADS, HEAD_DIM), dtype=torch.uint8, device=dev),
               torch.empty((T, HEADS), dtype=torch.int16, device=dev))
    q8, w_out = out
    _need(q8, (torch.uint8,), "q8")
    _need(w_out, _BF16, "w_out")
    _contig(q8, "q8")
    _contig(w_out, "w_out")
    with torch.cuda.device(dev):
        _check(lib().dsi_q_rope_quant(_ptr(q2), q_ld, T, _ptr(positions), _ptr(cos_sin), cos_sin.shape[0],
                                      int(bool(interleave)), _ptr(w), _rows(w, "w"), float(softmax_scale),
                                      float(head_scale), _ptr(q8), _ptr(w_out), _stream(q)), "q_rope_quant")
    return q8, w_out


def topk_values(logits, idx, row_starts=None, index_scale=1, index_offset=0, max_width=None, out=None):
    """One rank's local top-k selection -> (fp32 values, int32 global indices) [rows, k]."""
    dev = _dev(logits, idx, row_starts)
    _need(logits, (torch.float32,), "logits", 2)
    _need(idx, _I32, "idx", 2)
    rows, k = idx.shape
    if max_width is None:
        max_width = logits.shape[1]
    if out is None:
        out = (torch.empty((rows, k), dtype=torch.float32, device=dev),
               torch.empty((rows, k), dtype=torch.int32, device=dev))
    vals, gidx = out
    with torch.cuda.device(dev):
        _check(lib().dsi_topk_values(_ptr(logits), _rows(logits, "logits"), rows, _ptr(row_starts), max_width,
                                     _ptr(idx), _rows(idx, "idx"), k, index_scale, index_offset, _ptr(vals),
                                     _rows(vals, "vals"), _ptr(gidx), _rows(gidx, "gidx"), _stream(idx)),
               "topk_values")
    return vals, gidx


def topk_merge_workspace_bytes(rows, num_lists, k_in):
    return lib().dsi_topk_merge_workspace_bytes(rows, num_lists, k_in)


def topk_merge(vals, gidx, k=MAX_TOPK, out=None, workspace=None):
    """Exchanged candidate lists [num_lists, rows, k_in] (fp32 values, int32 global indices) -> int32 [rows, k]
    global top-k indices, -1 padded."""
    dev = _dev(vals, gidx, out, workspace)
    _need(vals, (torch.float32,), "vals", 3)
    _need(gidx, _I32, "gidx", 3)
    if vals.shape != gidx.shape or vals.stride() != gidx.stride():
        raise ValueError("vals and gidx must have the same shape and layout")
    L, rows, k_in = vals.shape
    if vals.stride(2) != 1:
        raise ValueError("vals: candidate entries must be contiguous")
    if out is None:
        out = torch.empty((rows, k), dtype=torch.int32, device=dev)
    need = topk_merge_workspace_bytes(rows, L, k_in)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    with torch.cuda.device(dev):
        _check(lib().dsi_topk_merge(_ptr(vals), _ptr(gidx), vals.stride(0), vals.stride(1), L, rows, k_in, k,
                                    _ptr(out), _rows(out, "out"), workspace.data_ptr(),
                                    workspace.numel() * workspace.element_size(), _stream(vals)), "topk_merge")
    return out


def k_quant_and_cache_mxfp4(k, slot_mapping, pool, block_size, block_stride_bytes=None, num_blocks=None):
    """MXFP4-quantize bf16 k [n, >=128] into the 68-byte rows of `pool` at `slot_mapping` (int64)."""
    dev = _dev(k, slot_mapping, pool)
    _need(k, _BF16, "k")
    _need(slot_mapping, (torch.int64,), "slot_mapping")
    _need(pool, (torch.uint8,), "pool")
    _contig(pool, "pool")
    k_ld = _rows(k, "k")
    if block_stride_bytes is None:
        block_stride_bytes = pool.stride(0) if pool.dim() > 1 else block_size * ROW_BYTES_MXFP4
    if num_blocks is None:
        num_blocks = pool.numel() // block_stride_bytes
    with torch.cuda.device(dev):
        _check(lib().dsi_k_quant_and_cache_mxfp4(_ptr(k), k.shape[0], k_ld, _ptr(slot_mapping), _ptr(pool),
                                                 num_blocks, block_size, block_stride_bytes, _stream(k)),
               "k_quant_and_cache_mxfp4")
    return pool


def sparse_mqa_logits_mxfp4(q, w, row_ks, row_ke, sparse_indices, end, sparse_block_kv, k_src, block_table=None,
                            row_to_req=None, block_size=0, block_stride_bytes=None, num_k=None, bt_width=None,
                            num_sparse_blocks=None, out=None):
    """sparse_mqa_logits on 68-byte MXFP4 key rows (gathered [S,68] or a paged pool)."""
    dev = _dev(q, w, row_ks, row_ke, sparse_indices, end, k_src, block_table, row_to_req, out)
    _need(q, (torch.uint8,), "q", 3)
    _need(w, _BF16, "w", 2)
    for t, nm in ((q, "q"), (w, "w"), (row_ks, "row_ks"), (row_ke, "row_ke"), (end, "end"), (k_src, "k_src")):
        _contig(t, nm)
    rows = q.shape[0]
    si_ld = _rows(sparse_indices, "sparse_indices")
    if num_sparse_blocks is None:
        num_sparse_blocks = sparse_indices.shape[1]
    width = num_sparse_blocks * sparse_block_kv
    bt_ld, num_reqs = 0, 0
    if block_table is not None:
        bt_ld = _rows(block_table, "block_table")
        num_reqs = block_table.shape[0]
        if bt_width is None:
            bt_width = block_table.shape[1]
        if block_stride_bytes is None:
            block_stride_bytes = k_src.stride(0) if k_src.dim() > 1 else block_size * ROW_BYTES_MXFP4
        if num_k is None:
            num_k = k_src.numel() // block_stride_bytes
    else:
        bt_width, block_stride_bytes = 0, 0
        if num_k is None:
            num_k = k_src.numel() // ROW_BYTES_MXFP4
    if out is None:
        out = torch.empty((rows, width), dtype=torch.int16, device=dev)
    _need(out, _BF16, "out")
    ld = _rows(out, "out")
    with torch.cuda.device(dev):
        _check(lib().dsi_sparse_mqa_logits_mxfp4(_ptr(q), _ptr(w), rows, _ptr(row_ks), _ptr(row_ke),
                                                 _ptr(sparse_indices), si_ld, num_sparse_blocks, _ptr(end),
                                                 sparse_block_kv, _ptr(k_src), num_k, _ptr(block_table), bt_ld,
                                                 bt_width, num_reqs, _ptr(row_to_req), block_size, block_stride_bytes,
                                                 _ptr(out), ld, _stream(q)), "sparse_mqa_logits_mxfp4")
    return out
