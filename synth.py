"""Seeded synthetic inputs for the indexer hot path (shared by tests and bench).

This module draws random inputs and lays them out; it holds none of the
arithmetic under test.  The one preparation step it performs, the per-128
FP8 quantization of q with its scale folded into the bf16 head weights, is
the pages' indexer step ④ ("DeepSeek V3.2 sparse attention DSA inference
flow", indexer internals ④), which happens before the hot path; it is done
here with torch's own float8/bfloat16 casts (library rounding), so neither
the oracle nor the HIP library implements it.  k is produced as bf16 and is
quantized by each side itself (the k_quant_and_cache step).

Draw order per case (fixed): lengths, q, k, weight factors u, block-table
permutation, candidates.  numpy.random.default_rng(seed).

All arrays are numpy: bf16 as uint16 bit patterns, FP8 as uint8 codes.
"""
import math

import numpy as np
import torch

H, D, ROW = 64, 128, 132


def _bf16_bits(x_f32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x_f32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _bf16_value(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def draw_q(rng, rows):
    """q ~ N(0,1) rounded to bf16, FP8 codes with one scale per (row, head) of 128 values, and the
    scale folded into bf16 weights w = u * q_scale with u ~ U(0.5, 1.5), rounded once."""
    qf = _bf16_value(_bf16_bits(rng.standard_normal((rows, H, D), dtype=np.float32)))
    return qf


def finish_q(rng, qf):
    rows = qf.shape[0]
    t = torch.from_numpy(qf)
    amax = t.abs().amax(dim=-1, keepdim=True)
    scale = torch.clamp(amax, min=1e-4) / 448.0
    codes = torch.clamp(t / scale, -448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    u = rng.uniform(0.5, 1.5, size=(rows, H)).astype(np.float32)
    w = _bf16_bits(u * scale[..., 0].numpy())
    return np.ascontiguousarray(codes), np.ascontiguousarray(w)


def draw_k(rng, n):
    return _bf16_bits(rng.standard_normal((n, D), dtype=np.float32))


# --------------------------------------------------------------------------- prefill (dense)
def prefill_case(seed, T, S, first_pos):
    """One request: T query tokens at positions first_pos..first_pos+T-1 over S history tokens
    gathered contiguously; causal rows ks = 0, ke = pos + 1."""
    rng = np.random.default_rng(seed)
    qf = draw_q(rng, T)
    k = draw_k(rng, S)
    q, w = finish_q(rng, qf)
    pos = np.arange(first_pos, first_pos + T, dtype=np.int32)
    ks = np.zeros(T, dtype=np.int32)
    ke = (pos + 1).astype(np.int32)
    return dict(q=q, w=w, k=k, ks=ks, ke=ke, S=S, T=T,
                slot_mapping=np.arange(S, dtype=np.int64))


# --------------------------------------------------------------------------- paged decode
def paged_layout(rng, lens, block_size, extra_blocks=0):
    """Random permutation of the pool's blocks into per-request block tables."""
    nblk = [int(math.ceil(int(L) / block_size)) for L in lens]
    total = sum(nblk) + extra_blocks
    perm = rng.permutation(total).astype(np.int32)
    width = max(nblk) if nblk else 1
    bt = np.zeros((len(lens), max(width, 1)), dtype=np.int32)
    off = 0
    for b, n in enumerate(nblk):
        bt[b, :n] = perm[off:off + n]
        off += n
    return bt, total


def slots_for(lens, bt, block_size):
    """slot of token s of request b = bt[b][s // bs] * bs + s % bs, requests concatenated."""
    out = []
    for b, L in enumerate(lens):
        s = np.arange(int(L), dtype=np.int64)
        out.append(bt[b, s // block_size].astype(np.int64) * block_size + s % block_size)
    return np.concatenate(out) if out else np.zeros(0, dtype=np.int64)


def decode_case(seed, B, next_n, lmin, lmax, block_size=64, lens=None):
    """B requests x next_n query rows; lengths ~ U{lmin..lmax}; pool of block_size-token blocks
    (132 B per token, unpacked: block stride = block_size * 132) under a random block permutation."""
    rng = np.random.default_rng(seed)
    if lens is None:
        lens = rng.integers(lmin, lmax + 1, size=B).astype(np.int32)
    else:
        lens = np.asarray(lens, dtype=np.int32)
    qf = draw_q(rng, B * next_n)
    k = draw_k(rng, int(lens.sum()))
    q, w = finish_q(rng, qf)
    bt, nblocks = paged_layout(rng, lens, block_size)
    return dict(q=q, w=w, k=k, context_lens=lens, block_table=bt, num_blocks=nblocks, block_size=block_size,
                block_stride=block_size * ROW, next_n=next_n, B=B,
                slot_mapping=slots_for(lens, bt, block_size))


def gather_case(seed, lens, block_size, span=None, extra_blocks=3):
    """Prefill requests laid end to end (cu_seq_lens) over a paged pool whose blocks are a random permutation;
    span = tokens per block stride (>= block_size: a packed pool leaves span - block_size unused rows)."""
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens, dtype=np.int32)
    k = draw_k(rng, int(lens.sum()))
    bt, nblocks = paged_layout(rng, lens, block_size, extra_blocks)
    span = block_size if span is None else span
    cu = np.zeros(len(lens) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lens)
    return dict(k=k, lens=lens, cu=cu, block_table=bt, num_blocks=nblocks, block_size=block_size,
                block_stride=span * ROW, slot_mapping=slots_for(lens, bt, block_size), S=int(cu[-1]))


def rope_cache(max_pos, base=10000.0):
    """Rotary table [max_pos, 64] fp32: cos of the 32 frequencies base^(-2i/64) times the position, then their
    sines (computed in fp64, rounded once)."""
    inv = base ** (-np.arange(32, dtype=np.float64) * 2.0 / 64.0)
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * inv[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)


def q_prep_case(seed, T, max_pos=65536):
    """Unrotated bf16 q [T,64,128] ~ N(0,1), positions ~ U{0..max_pos-1}, raw bf16 head weights ~ N(0,1)."""
    rng = np.random.default_rng(seed)
    pos = rng.integers(0, max_pos, size=T).astype(np.int64)
    q = _bf16_bits(rng.standard_normal((T, H, D), dtype=np.float32))
    w = _bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
    return dict(q=q, positions=pos, w=w, cos_sin=rope_cache(max_pos), T=T,
                softmax_scale=float(D) ** -0.5, head_scale=float(H) ** -0.5)


# --------------------------------------------------------------------------- hierarchical sparse
def draw_candidates(rng, maxb, num=64, distinct=60, dup=2):
    """Per row: `distinct` different ids from [0, maxb), `dup` repeats of those, one -1 and one id >= maxb,
    shuffled."""
    rows = len(maxb)
    out = np.empty((rows, num), dtype=np.int32)
    for r in range(rows):
        m = int(maxb[r])
        d = min(distinct, m)
        ids = rng.choice(m, size=d, replace=False).astype(np.int32)
        dups = rng.choice(ids, size=dup).astype(np.int32)
        oob = np.array([-1, m + int(rng.integers(0, 64))], dtype=np.int32)
        row = np.concatenate([ids, dups, oob])
        if row.size < num:  # short contexts: fill with more out-of-range ids
            row = np.concatenate([row, np.full(num - row.size, -1, dtype=np.int32)])
        rng.shuffle(row)
        out[r] = row[:num]
    return out


def sparse_case(seed, n_decode, chunk, lmin, lmax, sbk=128, cbs=128, num_cand=64, decode_block_size=128,
                lens=None):
    """Hierarchical (candidate-block) indexer step: n_decode decode requests (one row each, paged cache of
    decode_block_size-token pages) plus one prefill request whose last `chunk` tokens are the query rows
    (gathered K).  Rows: decode rows first, then the prefill chunk.  All lengths ~ U{lmin..lmax}."""
    rng = np.random.default_rng(seed)
    if lens is None:
        lens = rng.integers(lmin, lmax + 1, size=n_decode + 1).astype(np.int32)
    else:
        lens = np.asarray(lens, dtype=np.int32)
    dec_lens, Lp = lens[:n_decode], int(lens[n_decode])
    rows = n_decode + chunk
    qf = draw_q(rng, rows)
    k_dec = draw_k(rng, int(dec_lens.sum()))
    k_pre = draw_k(rng, Lp)
    q, w = finish_q(rng, qf)
    bt, nblocks = paged_layout(rng, dec_lens, decode_block_size)
    pos = np.arange(Lp - chunk, Lp, dtype=np.int32)
    ks = np.zeros(rows, dtype=np.int32)
    ke = np.concatenate([dec_lens, pos + 1]).astype(np.int32)
    maxb = (np.maximum(ke - ks, 0) + cbs - 1) // cbs
    cand = draw_candidates(rng, maxb, num=num_cand)
    return dict(q=q, w=w, k_dec=k_dec, k_pre=k_pre, dec_lens=dec_lens, Lp=Lp, block_table=bt, num_blocks=nblocks,
                block_size=decode_block_size, block_stride=decode_block_size * ROW, ks=ks, ke=ke, cand=cand,
                sbk=sbk, cbs=cbs, n_decode=n_decode, chunk=chunk, rows=rows,
                row_to_req=np.arange(n_decode, dtype=np.int32),
                dec_slot_mapping=slots_for(dec_lens, bt, decode_block_size))


# --------------------------------------------------------------------------- the five workloads
# 1: tiny dense indexer; 2: prefill chunk; 3: paged decode; 4: long-context decode (next-n 2);
# 5: hierarchical sparse.  Seeds are the workload numbers.
def workload(n):
    if n == 1:
        return prefill_case(1, T=8, S=3072, first_pos=3064)
    if n == 2:
        return prefill_case(2, T=2048, S=8192, first_pos=6144)
    if n == 3:
        return decode_case(3, B=64, next_n=1, lmin=4096, lmax=65536, block_size=64)
    if n == 4:
        return decode_case(4, B=16, next_n=2, lmin=98304, lmax=131072, block_size=64)
    if n == 5:
        return sparse_case(5, n_decode=32, chunk=1024, lmin=32768, lmax=131072)
    raise ValueError(n)
