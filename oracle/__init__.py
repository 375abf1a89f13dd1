"""CPU oracle for the DSA lightning-indexer hot path.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` may import this package; the product path
(``sparse_attention_token_amd``) never does, and this package never imports
the product path.  The arithmetic lives in ``dsi_oracle.c`` (plain
single-threaded C, fp32 on dequantized FP8); this module only marshals numpy
arrays.  bf16 values travel as ``uint16`` bit patterns, FP8 as ``uint8`` codes.

Functions follow the three pages the indexer is described on; each C function
cites its passage (P1: vLLM PR 56254 summary, "V4.1 indexer uses sparse MQA
logits"; P2: vLLM PR 47493 summary, packed-KV sparse-MLA address fix; P3:
"DeepSeek V3.2 sparse attention DSA inference flow").
"""
import ctypes
import os

import numpy as np

from .build import LIB, build

H, D, ROW = 64, 128, 132

_lib = None

_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB):
        build()
    lib = ctypes.CDLL(LIB)
    sig = {
        "orc_e4m3_decode": (ctypes.c_float, [ctypes.c_uint8]),
        "orc_e4m3_encode": (ctypes.c_uint8, [ctypes.c_float]),
        "orc_bf16_rne": (ctypes.c_uint16, [ctypes.c_float]),
        "orc_bf16_to_f32": (ctypes.c_float, [ctypes.c_uint16]),
        "orc_k_quant_and_cache": (None, [_p, _i64, _i64, _p, _p, _i32, _i64]),
        "orc_mqa_logits_gathered": (None, [_p, _p, _i32, _p, _i32, _p, _p, _p, _i64]),
        "orc_mqa_logits_paged": (None, [_p, _p, _i32, _i32, _p, _p, _i32, _i64, _p, _i64, _i32, _p, _i64]),
        "orc_topk_select_f32": (ctypes.c_int, [_p, _i64, _i32, _p, _p, _i32, _i32, _p, _i64]),
        "orc_topk_select_bf16": (ctypes.c_int, [_p, _i64, _i32, _p, _p, _i32, _i32, _p, _i64]),
        "orc_req_index_to_global_slot": (None, [_p, _i64, _i32, _i32, _p, _p, _i64, _i32, _i32, _p, _i64]),
        "orc_expand_candidates": (ctypes.c_int, [_p, _i64, _i32, _i32, _p, _i64, _p, _i64, _i32, _i32, _p, _i64,
                                                 _p, _i64]),
        "orc_sparse_mqa_logits": (None, [_p, _p, _i32, _p, _p, _p, _i64, _i32, _p, _i32, _p, _p, _i64, _p, _i32,
                                         _i64, _i32, _p, _i64]),
        "orc_topk_remap": (None, [_p, _i64, _i32, _i32, _p, _i64, _p, _i32, _p, _i64]),
        "orc_gather_prefill_k": (None, [_p, _i64, _i32, _i64, _p, _i64, _i32, _p, _i32, _p, _i32]),
        "orc_topk_values": (None, [_p, _i64, _i32, _p, _i32, _p, _i64, _i32, _i32, _i32, _p, _i64, _p, _i64]),
        "orc_topk_merge": (ctypes.c_int, [_p, _p, _i64, _i64, _i32, _i32, _i32, _i32, _p, _i64]),
        "orc_fp4_decode": (ctypes.c_float, [ctypes.c_uint8]),
        "orc_fp4_encode": (ctypes.c_uint8, [ctypes.c_float]),
        "orc_k_quant_and_cache_mxfp4": (None, [_p, _i64, _i64, _p, _p, _i32, _i64]),
        "orc_sparse_mqa_logits_mxfp4": (None, [_p, _p, _i32, _p, _p, _p, _i64, _i32, _p, _i32, _p, _p, _i64, _p,
                                               _i32, _i64, _i32, _p, _i64]),
        "orc_q_rope_quant": (None, [_p, _p, _i32, _p, _i64, _i32, _p, ctypes.c_float, ctypes.c_float, _p, _p]),
        "orc_mqa_logits_paged_mxfp4": (None, [_p, _p, _i32, _i32, _p, _p, _i32, _i64, _p, _i64, _i32, _p, _i64]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _rows(a, dtype):
    """2-D array with unit inner stride; returns (array, leading dim in elements)."""
    a = np.asarray(a)
    assert a.dtype == dtype, (a.dtype, dtype)
    assert a.ndim == 2
    if a.strides[1] != a.itemsize or a.strides[0] % a.itemsize:
        a = np.ascontiguousarray(a)
    return a, a.strides[0] // a.itemsize


# ---------------------------------------------------------------- O0 codecs
def e4m3_decode(codes):
    lib = _load()
    c = np.asarray(codes, dtype=np.uint8)
    return np.array([lib.orc_e4m3_decode(int(b)) for b in c.ravel()], dtype=np.float32).reshape(c.shape)


def e4m3_encode(x):
    lib = _load()
    x = np.asarray(x, dtype=np.float32)
    return np.array([lib.orc_e4m3_encode(float(v)) for v in x.ravel()], dtype=np.uint8).reshape(x.shape)


def bf16_rne(x):
    lib = _load()
    x = np.asarray(x, dtype=np.float32)
    return np.array([lib.orc_bf16_rne(float(v)) for v in x.ravel()], dtype=np.uint16).reshape(x.shape)


def bf16_to_f32(h):
    lib = _load()
    h = np.asarray(h, dtype=np.uint16)
    return np.array([lib.orc_bf16_to_f32(int(v)) for v in h.ravel()], dtype=np.float32).reshape(h.shape)


# ---------------------------------------------------------------- O1
def k_quant_and_cache(k_bf16, slot_mapping, pool, block_size, block_stride):
    """Quantize bf16 k rows [n,128] (uint16 bits) into the uint8 pool in place."""
    lib = _load()
    k, k_ld = _rows(k_bf16, np.uint16)
    assert k.shape[1] == D
    slots = _c(slot_mapping, np.int64)
    assert pool.dtype == np.uint8 and pool.flags["C_CONTIGUOUS"]
    lib.orc_k_quant_and_cache(_ptr(k), k.shape[0], k_ld, _ptr(slots), _ptr(pool), block_size, block_stride)
    return pool


# ---------------------------------------------------------------- O2
def mqa_logits_gathered(q, w, k_rows, ks, ke, S=None):
    """q uint8 [T,64,128], w uint16 [T,64], k_rows uint8 [S,132] -> fp32 [T,S] (-inf outside [ks,ke))."""
    lib = _load()
    q = _c(q, np.uint8)
    w = _c(w, np.uint16)
    k_rows = _c(k_rows, np.uint8)
    T = q.shape[0]
    if S is None:
        S = k_rows.shape[0]
    assert q.shape == (T, H, D) and w.shape == (T, H) and k_rows.shape[1] == ROW and k_rows.shape[0] >= S
    ks = _c(ks, np.int32)
    ke = _c(ke, np.int32)
    out = np.empty((T, S), dtype=np.float32)
    lib.orc_mqa_logits_gathered(_ptr(q), _ptr(w), T, _ptr(k_rows), S, _ptr(ks), _ptr(ke), _ptr(out), S)
    return out


def mqa_logits_paged(q, w, next_n, context_lens, pool, block_size, block_stride, block_table, width):
    """Decode rows straight from the paged pool -> fp32 [B*next_n, width]."""
    lib = _load()
    q = _c(q, np.uint8)
    w = _c(w, np.uint16)
    cl = _c(context_lens, np.int32)
    B = cl.shape[0]
    assert q.shape == (B * next_n, H, D) and w.shape == (B * next_n, H)
    bt, bt_ld = _rows(block_table, np.int32)
    assert pool.dtype == np.uint8 and pool.flags["C_CONTIGUOUS"]
    out = np.empty((B * next_n, width), dtype=np.float32)
    lib.orc_mqa_logits_paged(_ptr(q), _ptr(w), B, next_n, _ptr(cl), _ptr(pool), block_size, block_stride, _ptr(bt),
                             bt_ld, width, _ptr(out), width)
    return out


# ---------------------------------------------------------------- O3
def topk_select(x, ends, k, starts=None, bf16=False, max_width=None):
    """Top-k per row of finite values in [start, end): int32 [rows, k], col - start, -1 padded."""
    lib = _load()
    x, ld = _rows(x, np.uint16 if bf16 else np.float32)
    rows = x.shape[0]
    if max_width is None:
        max_width = x.shape[1]
    ends = _c(ends, np.int32)
    st = None if starts is None else _c(starts, np.int32)
    out = np.empty((rows, k), dtype=np.int32)
    fn = lib.orc_topk_select_bf16 if bf16 else lib.orc_topk_select_f32
    rc = fn(_ptr(x), ld, rows, _ptr(st), _ptr(ends), max_width, k, _ptr(out), k)
    assert rc == 0
    return out


# ---------------------------------------------------------------- O4
def req_index_to_global_slot(idx, block_table, block_size, block_span, row_to_req=None):
    lib = _load()
    idx, ld = _rows(idx, np.int32)
    bt, bt_ld = _rows(block_table, np.int32)
    r2r = None if row_to_req is None else _c(row_to_req, np.int32)
    out = np.empty(idx.shape, dtype=np.int32)
    lib.orc_req_index_to_global_slot(_ptr(idx), ld, idx.shape[0], idx.shape[1], _ptr(r2r), _ptr(bt), bt_ld,
                                     block_size, block_span, _ptr(out), idx.shape[1])
    return out


# ---------------------------------------------------------------- O6
def expand_candidates(cand, ks, ke, candidate_block_size, sparse_block_kv):
    """-> (sparse_indices int32 [rows, K*ratio], end int32 [rows])."""
    lib = _load()
    cand, ld = _rows(cand, np.int32)
    rows, K = cand.shape
    ratio = candidate_block_size // sparse_block_kv
    ks = _c(ks, np.int32)
    ke = _c(ke, np.int32)
    si = np.empty((rows, K * ratio), dtype=np.int32)
    end = np.empty((rows,), dtype=np.int32)
    rc = lib.orc_expand_candidates(_ptr(cand), ld, rows, K, _ptr(ks), 1, _ptr(ke), 1, candidate_block_size,
                                   sparse_block_kv, _ptr(si), K * ratio, _ptr(end), 1)
    if rc != 0:
        raise ValueError("bad candidate/sparse block sizes")
    return si, end


# ---------------------------------------------------------------- O7
def sparse_mqa_logits(q, w, ks, ke, sparse_indices, end, sparse_block_kv, k_src, block_table=None, row_to_req=None,
                      block_size=0, block_stride=0, out_f32=False):
    """-> bf16 bits uint16 [rows, nsb*sbk] (or fp32 with out_f32)."""
    lib = _load()
    q = _c(q, np.uint8)
    w = _c(w, np.uint16)
    rows = q.shape[0]
    ks = _c(ks, np.int32)
    ke = _c(ke, np.int32)
    si, si_ld = _rows(sparse_indices, np.int32)
    nsb = si.shape[1]
    end = _c(end, np.int32)
    k_src = np.ascontiguousarray(k_src, dtype=np.uint8)
    bt, bt_ld = (None, 0) if block_table is None else _rows(block_table, np.int32)
    r2r = None if row_to_req is None else _c(row_to_req, np.int32)
    width = nsb * sparse_block_kv
    out = np.empty((rows, width), dtype=np.float32 if out_f32 else np.uint16)
    lib.orc_sparse_mqa_logits(_ptr(q), _ptr(w), rows, _ptr(ks), _ptr(ke), _ptr(si), si_ld, nsb, _ptr(end),
                              sparse_block_kv, _ptr(k_src), _ptr(bt), bt_ld, _ptr(r2r), block_size, block_stride,
                              1 if out_f32 else 0, _ptr(out), width)
    return out


# ---------------------------------------------------------------- O8
def topk_remap(col, sparse_indices, ks, sparse_block_kv):
    lib = _load()
    col, ld = _rows(col, np.int32)
    si, si_ld = _rows(sparse_indices, np.int32)
    ks = _c(ks, np.int32)
    out = np.empty(col.shape, dtype=np.int32)
    lib.orc_topk_remap(_ptr(col), ld, col.shape[0], col.shape[1], _ptr(si), si_ld, _ptr(ks), sparse_block_kv,
                       _ptr(out), col.shape[1])
    return out


# ---------------------------------------------------------------- O5 (oracle-only reference)
def candidate_token_mask(cand, ks, ke, candidate_block_size, S):
    """Token s (gathered index) is a candidate token of row r when it lies in [ks, ke) and its block
    (s - ks) // candidate_block_size is one of the row's candidate ids (P1 motivation: the old consumer
    path scores the whole context and masks everything outside the candidate blocks)."""
    cand = np.asarray(cand)
    rows = cand.shape[0]
    m = np.zeros((rows, S), dtype=bool)
    for r in range(rows):
        lo, hi = int(ks[r]), int(ke[r])
        for s in range(max(lo, 0), min(hi, S)):
            if ((s - lo) // candidate_block_size) in set(int(c) for c in cand[r]):
                m[r, s] = True
    return m


def dense_masked_topk(q, w, k_rows, ks, ke, cand, candidate_block_size, k):
    """Dense logits over [ks, ke), non-candidate tokens set to -inf, then top-k (positions relative to ks)."""
    S = k_rows.shape[0]
    logits = mqa_logits_gathered(q, w, k_rows, ks, ke, S)
    mask = candidate_token_mask(cand, ks, ke, candidate_block_size, S)
    logits = np.where(mask, logits, np.float32(-np.inf)).astype(np.float32)
    idx = topk_select(logits, ke, k, starts=ks)
    return idx, logits


# ---------------------------------------------------------------- O9
def gather_prefill_k(pool, num_blocks, block_size, block_stride, block_table, cu_seq_lens, S, bt_width=None):
    """Paged pool (uint8) -> contiguous cache rows uint8 [S,132] of the requests laid end to end (cu_seq_lens
    int32 [num_reqs+1]); rows no request owns and tokens without a valid page are zero."""
    lib = _load()
    pool = _c(pool, np.uint8)
    assert pool.size >= num_blocks * block_stride
    bt, bt_ld = _rows(np.asarray(block_table, dtype=np.int32), np.int32)
    cu = _c(cu_seq_lens, np.int32)
    num_reqs = cu.size - 1
    assert num_reqs <= bt.shape[0]
    if bt_width is None:
        bt_width = bt.shape[1]
    out = np.empty((S, ROW), dtype=np.uint8)
    lib.orc_gather_prefill_k(_ptr(pool), num_blocks, block_size, block_stride, _ptr(bt), bt_ld, bt_width, _ptr(cu),
                             num_reqs, _ptr(out), S)
    return out


# ---------------------------------------------------------------- O10
def q_rope_quant(q_bf16, positions, cos_sin, w_bf16, softmax_scale, head_scale, interleave=False):
    """q bf16 [T,64,128] (uint16), positions int64 [T], cos_sin fp32 [max_pos,64] (32 cosines then 32 sines),
    w bf16 [T,64] -> (FP8 codes uint8 [T,64,128], bf16 weights uint16 [T,64])."""
    lib = _load()
    q = _c(q_bf16, np.uint16)
    T = q.shape[0]
    assert q.shape == (T, H, D)
    pos = _c(positions, np.int64)
    cs = _c(cos_sin, np.float32)
    assert cs.ndim == 2 and cs.shape[1] == 64
    w = _c(w_bf16, np.uint16)
    assert w.shape == (T, H)
    q8 = np.empty((T, H, D), dtype=np.uint8)
    w_out = np.empty((T, H), dtype=np.uint16)
    lib.orc_q_rope_quant(_ptr(q), _ptr(pos), T, _ptr(cs), cs.shape[0], int(bool(interleave)), _ptr(w),
                         float(softmax_scale), float(head_scale), _ptr(q8), _ptr(w_out))
    return q8, w_out


# ---------------------------------------------------------------- O11, O12
def topk_values(logits, idx, starts=None, index_scale=1, index_offset=0, max_width=None):
    """(values fp32, global indices int32) [rows, k] of one rank's local top-k selection `idx` (relative to
    the row starts) over its fp32 logits [rows, >=max_width]."""
    lib = _load()
    x, ld = _rows(np.asarray(logits, dtype=np.float32), np.float32)
    ix, ild = _rows(np.asarray(idx, dtype=np.int32), np.int32)
    rows, k = ix.shape
    st = None if starts is None else _c(starts, np.int32)
    if max_width is None:
        max_width = x.shape[1]
    vals = np.empty((rows, k), dtype=np.float32)
    g = np.empty((rows, k), dtype=np.int32)
    lib.orc_topk_values(_ptr(x), ld, rows, _ptr(st), max_width, _ptr(ix), ild, k, index_scale, index_offset,
                        _ptr(vals), k, _ptr(g), k)
    return vals, g


def topk_merge(vals, gidx, k):
    """Candidate lists [num_lists, rows, k_in] (fp32 values, int32 global indices) -> int32 [rows, k]: the
    indices of the k largest finite values with index >= 0, (value desc, index asc), then -1."""
    lib = _load()
    v = _c(vals, np.float32)
    g = _c(gidx, np.int32)
    assert v.shape == g.shape and v.ndim == 3
    L, rows, k_in = v.shape
    out = np.empty((rows, k), dtype=np.int32)
    assert lib.orc_topk_merge(_ptr(v), _ptr(g), rows * k_in, k_in, L, rows, k_in, k, _ptr(out), k) == 0
    return out


# ---------------------------------------------------------------- O13, O14 (MXFP4 cache)
ROW4 = 68


def fp4_decode(codes):
    lib = _load()
    c = np.asarray(codes, dtype=np.uint8)
    return np.array([lib.orc_fp4_decode(int(b)) for b in c.ravel()], dtype=np.float32).reshape(c.shape)


def fp4_encode(x):
    lib = _load()
    x = np.asarray(x, dtype=np.float32)
    return np.array([lib.orc_fp4_encode(float(v)) for v in x.ravel()], dtype=np.uint8).reshape(x.shape)


def k_quant_and_cache_mxfp4(k_bf16, slot_mapping, pool, block_size, block_stride):
    """MXFP4-quantize bf16 k rows [n,128] (uint16 bits) into 68-byte rows of the uint8 pool in place."""
    lib = _load()
    k, k_ld = _rows(k_bf16, np.uint16)
    assert k.shape[1] == D
    slots = _c(slot_mapping, np.int64)
    assert pool.dtype == np.uint8 and pool.flags["C_CONTIGUOUS"]
    lib.orc_k_quant_and_cache_mxfp4(_ptr(k), k.shape[0], k_ld, _ptr(slots), _ptr(pool), block_size, block_stride)
    return pool


def sparse_mqa_logits_mxfp4(q, w, ks, ke, sparse_indices, end, sbk, k_src, block_table=None, row_to_req=None,
                            block_size=0, block_stride=0, out_f32=False):
    """As sparse_mqa_logits, on 68-byte MXFP4 key rows."""
    lib = _load()
    q = _c(q, np.uint8)
    w = _c(w, np.uint16)
    rows = q.shape[0]
    si, si_ld = _rows(np.asarray(sparse_indices, dtype=np.int32), np.int32)
    nsb = si.shape[1]
    width = nsb * sbk
    ks, ke, end = _c(ks, np.int32), _c(ke, np.int32), _c(end, np.int32)
    k_src = _c(k_src, np.uint8)
    bt, bt_ld = (None, 0) if block_table is None else _rows(np.asarray(block_table, dtype=np.int32), np.int32)
    r2r = None if row_to_req is None else _c(row_to_req, np.int32)
    out = np.empty((rows, width), dtype=np.float32 if out_f32 else np.uint16)
    lib.orc_sparse_mqa_logits_mxfp4(_ptr(q), _ptr(w), rows, _ptr(ks), _ptr(ke), _ptr(si), si_ld, nsb, _ptr(end),
                                    sbk, _ptr(k_src), _ptr(bt), bt_ld, _ptr(r2r), block_size, block_stride,
                                    int(out_f32), _ptr(out), width)
    return out

# ---------------------------------------------------------------- O15
def mqa_logits_paged_mxfp4(q, w, next_n, context_lens, pool, block_size, block_stride, block_table, width):
    """Decode rows straight from a paged pool of 68-byte MXFP4 rows -> fp32 [B*next_n, width]."""
    lib = _load()
    q = _c(q, np.uint8)
    w = _c(w, np.uint16)
    cl = _c(context_lens, np.int32)
    B = cl.shape[0]
    assert q.shape == (B * next_n, H, D) and w.shape == (B * next_n, H)
    bt, bt_ld = _rows(block_table, np.int32)
    assert pool.dtype == np.uint8 and pool.flags["C_CONTIGUOUS"]
    out = np.empty((B * next_n, width), dtype=np.float32)
    lib.orc_mqa_logits_paged_mxfp4(_ptr(q), _ptr(w), B, next_n, _ptr(cl), _ptr(pool), block_size, block_stride,
                                   _ptr(bt), bt_ld, width, _ptr(out), width)
    return out
