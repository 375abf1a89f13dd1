"""Benchmark of the DSA lightning-indexer hot path on one MI355X.

Headline line (stdout, one JSON object): the prefill-chunk workload — one request, T=2048 query tokens at
positions 6144..8191 over S=8192 history tokens, 64 heads x 128 dims, FP8 q/k.  One step = quantize and
insert the chunk's 2048 new k rows, dense indexer logits over the gathered K (causal), top-2048 per row.
`value` = scored query-key pairs per second (masked pairs not counted).  Inputs are resident in HBM before
the timed region; every step launches the same three kernels on the current stream.

Also reported (same JSON line): the roofline of the dominant kernel (prefill logits: FP8 codes decoded
exactly to f16 and contracted on the f16 matrix cores, so its peak is the dense f16 MFMA peak), ceilings
measured on this device (register-only MFMA loops, a 4 GiB streaming read), the oracle's single-thread CPU
rate on a bounded row sample, and the decode and hierarchical workloads (paged decode 64 x U{4096..65536};
long-context decode 16 x 2 rows x U{98304..131072}; hierarchical sparse 32 decode rows + 1024 prefill rows)
with their HBM roofline fractions, the prefill K gather out of the paged cache (8192 and 131072 tokens) and the q
preparation (RoPE, FP8 quantization, weight fold) of the 2048-token chunk, the context-parallel merge of 8 ranks'
top-2048 lists for 64 decode rows, and the hierarchical workload again on the MXFP4 K cache.
Diagnostics go to stderr.

`roofline.traffic` (HBM bytes per launch of the prefill logits kernel) comes from the committed counter
summary in profiles/ (FETCH_SIZE and WRITE_SIZE, each scaled by what the same counter reads for a plain copy
of known size); it is null when the kernel's sources no longer hash to the ones the counters were taken on.
"""
import argparse
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import sparse_attention_token_amd as dsi  # noqa: E402
from sparse_attention_token_amd import ceiling  # noqa: E402
import synth  # noqa: E402

ROW, K = 132, 2048
ROW_MXFP4 = 68  # MXFP4 cache row: 64 bytes of FP4 codes + 4 E8M0 block scales
F16_PEAK_TFLOPS = 2500.0  # MI355X dense f16 MFMA (published)
FP8_PEAK_TFLOPS = 5000.0  # MI355X dense FP8 MFMA (published)
HBM_PEAK_GBS = 8000.0     # MI355X HBM3E (published)
PAGED_CEILING = None      # the measured ceilings, once taken (the paged-read rates are read by the decode lines)
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "prefill_logits_T2048_S8192_traffic.md")
PREFILL_SOURCES = [os.path.join(ROOT, "sparse_attention_token_amd", "csrc", f) for f in ("prefill.hip", "common.h")]
FLOP_PER_PAIR = 2 * 64 * 128
ALL_WORKLOADS = ["decode_w3", "decode_w4", "decode_w3_mxfp4", "decode_w4_mxfp4", "sparse_w5", "sparse_w5_mxfp4",
                 "prefill_gather", "q_prep", "cp_merge"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def dev(a):
    a = np.ascontiguousarray(a)
    return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).cuda()


class EventTimer:
    """Pairs of HIP events on the current stream around one kernel; averaged after a sync."""

    def __init__(self):
        self.pairs = []

    def start(self):
        e = torch.cuda.Event(enable_timing=True)
        e.record()
        return e

    def stop(self, s):
        e = torch.cuda.Event(enable_timing=True)
        e.record()
        self.pairs.append((s, e))

    def mean_ms(self):
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in self.pairs])) if self.pairs else float("nan")


def queue_ahead(steps, us_per_step=250):
    """Occupy the GPU with a spin kernel (about us_per_step per step to come) so that the host enqueues the
    timed launches while it runs: the events then bracket device time, not the binding's Python overhead."""
    torch.cuda._sleep(int(steps * us_per_step * 2200))


# --------------------------------------------------------------------------- measured ceilings
def timed_ms(fn, reps=5):
    best = float("inf")
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        torch.cuda.synchronize()
        best = min(best, a.elapsed_time(b))
    return best


def measure_ceilings():
    """Register-only MFMA loops (f16 16x16x32 and 32x32x16, FP8 16x16x128; the f16 ones also on random FP8 codes, which
    run at the power limit), a streaming read of 4 GiB (16x the 256 MB
    Infinity Cache) and a 1 GiB copy.  The copy is also the calibration dispatch of the byte counters.  The reads are
    taken with the default cache policy and with the non-temporal load hint (`_nt` keys)."""
    out = {}
    wg = 256 * 8
    sink = torch.empty(wg * ceiling.THREADS, dtype=torch.float32, device="cuda")
    for kind, name, iters in ((0, "mfma_f16_tflops", 1000), (2, "mfma_f16_32x32x16_tflops", 1000),
                              (1, "mfma_fp8_tflops", 500)):
        best = 0.0
        for g in (wg, wg // 4):  # 8 or 2 wavefronts per SIMD
            flop = [0]

            def run():
                flop[0] = ceiling.mfma_loop(kind, g, iters * wg // g, sink)
            run()
            best = max(best, flop[0] / (timed_ms(run) * 1e-3) / 1e12)
        out[name] = round(best, 1)
    # The f16 loops on random FP8 codes, sustained (three back-to-back launches of ~9 ms after one more): the chip
    # settles at its power limit within milliseconds, and short bursts run above it.
    for kind, name in ((3, "mfma_f16_random_sustained_tflops"), (4, "mfma_f16_32x32x16_random_sustained_tflops")):
        best = 0.0
        for g in (wg, wg // 4):
            flop = [0]

            def run():
                flop[0] = sum(ceiling.mfma_loop(kind, g, 8000 * wg // g, sink) for _ in range(3))
            ceiling.mfma_loop(kind, g, 8000 * wg // g, sink)  # one launch first, to reach the settled clock
            ms = timed_ms(run, reps=1)
            best = max(best, flop[0] / (ms * 1e-3) / 1e12)
        out[name] = round(best, 1)
    big = torch.empty(4 << 30, dtype=torch.uint8, device="cuda")
    isink = torch.empty(4096 * ceiling.THREADS, dtype=torch.int32, device="cuda")
    nb = [0]
    for nt, key in ((False, "hbm_read_gbs"), (True, "hbm_read_nt_gbs")):
        best = 0.0
        for wg in (1024, 2048, 4096):
            def run():
                nb[0] = ceiling.stream_read(big, wg, isink, nontemporal=nt)
            run()
            best = max(best, nb[0] / (timed_ms(run) * 1e-3) / 1e9)
        out[key] = round(best, 1)
    src, dst = big[: 1 << 30], big[2 << 30: 3 << 30]

    def run():
        nb[0] = ceiling.copy(src, dst, 4096)
    out["copy_gbs"] = round(2 * (1 << 30) / (timed_ms(run) * 1e-3) / 1e9, 1)
    out["copy_bytes"] = 1 << 30
    # The paged cache's read pattern alone: 64-token pages (132- or 68-byte rows) in a random order over 1 GiB.
    pool = big[: 1 << 30]
    rng = np.random.default_rng(11)
    for name, page in (("fp8_pages", 64 * ROW), ("mxfp4_pages", 64 * ROW_MXFP4)):
        n = (1 << 30) // page
        pages = torch.from_numpy(rng.permutation(n).astype(np.int32)).cuda()
        for nt, key in ((False, "paged_read_gbs_"), (True, "paged_read_nt_gbs_")):
            best = 0.0
            for wg in (1024, 2048, 4096):
                for ppr in (4, 8):
                    def run():  # three reads per timing, so that one launch's dispatch weighs less
                        nb[0] = sum(ceiling.paged_read(pool, page, pages, page, wg, isink, ppr, nontemporal=nt)
                                    for _ in range(3))
                    run()
                    best = max(best, nb[0] / (timed_ms(run) * 1e-3) / 1e9)
            out[key + name] = round(best, 1)
    del big, pool
    torch.cuda.empty_cache()
    return out


def sources_digest(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def committed_traffic():
    """HBM bytes per prefill-logits launch from the committed counter summary, or None when it is missing or
    was taken on other kernel sources.  The summary holds `key: value` lines."""
    if not os.path.exists(TRAFFIC_SUMMARY):
        return None
    kv = {}
    for line in open(TRAFFIC_SUMMARY):
        if ":" in line and line.startswith("- `"):
            k, v = line[3:].split("`", 1)
            kv[k] = v.split(":", 1)[1].strip().strip("`")
    if kv.get("kernel_sources_sha256") != sources_digest(PREFILL_SOURCES):
        return None
    try:
        return int(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# --------------------------------------------------------------------------- prefill chunk (headline)
def bench_prefill(steps, warmup):
    c = synth.workload(2)
    T, S = c["T"], c["S"]
    first = S - T
    pairs = int((c["ke"] - c["ks"]).sum())
    q, w, ks, ke = dev(c["q"]), dev(c["w"]), dev(c["ks"]), dev(c["ke"])
    k_all = dev(c["k"])
    rows = torch.zeros((S, ROW), dtype=torch.uint8, device="cuda")
    slots = torch.arange(S, dtype=torch.int64, device="cuda")
    # history already in the cache; each step inserts the chunk's own k rows
    dsi.k_quant_and_cache(k_all[:first], slots[:first], rows.view(-1), S, S * ROW, 1)
    k_chunk, s_chunk = k_all[first:], slots[first:]
    logits = torch.empty((T, S), dtype=torch.float32, device="cuda")
    idx = torch.empty((T, K), dtype=torch.int32, device="cuda")
    timer = EventTimer()

    def step(timed):
        dsi.k_quant_and_cache(k_chunk, s_chunk, rows.view(-1), S, S * ROW, 1)
        s = timer.start() if timed else None
        dsi.mqa_logits_prefill(q, w, rows, ks, ke, out=logits)
        if timed:
            timer.stop(s)
        dsi.topk_select(logits, ke, k=K, row_starts=ks, out=idx)

    for _ in range(warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    queue_ahead(steps)
    t0.record()
    for _ in range(steps):
        step(True)
    t1.record()
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / steps
    ms_logits = timer.mean_ms()
    # top-k alone, for the report
    tk = EventTimer()
    queue_ahead(steps)
    for _ in range(steps):
        s = tk.start()
        dsi.topk_select(logits, ke, k=K, row_starts=ks, out=idx)
        tk.stop(s)
    ms_topk = tk.mean_ms()
    return dict(c=c, pairs=pairs, ms_step=ms_step, ms_logits=ms_logits, ms_topk=ms_topk, T=T, S=S)


def host_cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def _decode_bytes(L, nn, bs):
    """Algorithmic bytes of one request's decode logits + top-k (the GPU figure's formula): its K once, its block
    table, q and weights per row, the logits written and read back, the index rows written."""
    V = sum(L - nn + i + 1 for i in range(nn))
    return ROW * L + 4 * ((L + bs - 1) // bs) + nn * (64 * 128 + 64 * 2) + 8 * V + nn * K * 4


def cpu_baselines(c2, budget_s):
    """The oracle as it is (single thread, never tuned) on a bounded sample of each workload, the whole chain
    the GPU runs: k quantization, logits, top-k and slot conversion (or expansion, sparse logits, top-k, remap
    and slots).  Rows or requests are taken in a seeded random order until each workload's share of the time
    budget is spent.  Returns the headline object (workload 2) with every workload under `per_config`."""
    import oracle
    per = {}
    share = budget_s / 5.0

    # workloads 1 and 2: quantize the whole history, then logits + top-2048 per query row
    def dense(c, seconds):
        T, S = c["T"], c["S"]
        t0 = time.perf_counter()
        rows = np.zeros((S, ROW), np.uint8)
        oracle.k_quant_and_cache(c["k"], np.arange(S), rows.reshape(-1), S, S * ROW)
        done, pairs = 0, 0
        for t in np.random.default_rng(0).permutation(T):
            sl = slice(int(t), int(t) + 1)
            lg = oracle.mqa_logits_gathered(c["q"][sl], c["w"][sl], rows, c["ks"][sl], c["ke"][sl])
            oracle.topk_select(lg, c["ke"][sl], K, starts=c["ks"][sl])
            pairs += int(c["ke"][t] - c["ks"][t])
            done += 1
            if time.perf_counter() - t0 > seconds:
                break
        dt = time.perf_counter() - t0
        return dict(value=pairs / dt, unit="pairs/s", seconds=round(dt, 2),
                    sample=f"{done} of {T} query rows (all {S} k rows quantized first)")

    per["1_tiny_dense"] = dense(synth.workload(1), share)
    per["2_prefill_chunk"] = dense(c2, 2 * share)

    # workloads 3 and 4: per request, its k rows quantized into a pool of its own pages, paged logits for its
    # next-n rows, top-2048 and slot conversion
    for n, name in ((3, "3_paged_decode"), (4, "4_long_context_decode")):
        c = synth.workload(n)
        nn, bs = c["next_n"], c["block_size"]
        lens = c["context_lens"]
        starts = np.concatenate([[0], np.cumsum(lens)])
        t0 = time.perf_counter()
        done, pairs, nbytes = 0, 0, 0
        for b in np.random.default_rng(n).permutation(c["B"]):
            L = int(lens[b])
            nblk = (L + bs - 1) // bs
            pool = np.zeros(nblk * bs * ROW, np.uint8)
            bt = np.arange(nblk, dtype=np.int32)[None, :]
            oracle.k_quant_and_cache(c["k"][starts[b]:starts[b + 1]], np.arange(L), pool, bs, bs * ROW)
            rr = slice(b * nn, (b + 1) * nn)
            lg = oracle.mqa_logits_paged(c["q"][rr], c["w"][rr], nn, lens[b:b + 1], pool, bs, bs * ROW, bt, L)
            ends = np.array([L - nn + i + 1 for i in range(nn)], np.int32)
            idx = oracle.topk_select(lg, ends, K)
            oracle.req_index_to_global_slot(idx, bt, bs, bs, row_to_req=np.zeros(nn, np.int32))
            pairs += int(ends.sum())
            nbytes += _decode_bytes(L, nn, bs)
            done += 1
            if time.perf_counter() - t0 > share:
                break
        dt = time.perf_counter() - t0
        per[name] = dict(value=pairs / dt, unit="pairs/s", gbs_equivalent=round(nbytes / dt / 1e9, 4),
                         rows_per_s=round(done * nn / dt, 2), seconds=round(dt, 2),
                         sample=f"{done} of {c['B']} requests ({done * nn} rows), each quantized, scored, selected "
                                f"and converted to slots")

    # workload 5: expansion of every row, then per sampled row sparse logits (bf16), top-2048, remap (+ slots)
    c = synth.workload(5)
    sbk, cbs, nd, nrows = c["sbk"], c["cbs"], c["n_decode"], c["rows"]
    bs = c["block_size"]
    t0 = time.perf_counter()
    si, end = oracle.expand_candidates(c["cand"], c["ks"], c["ke"], cbs, sbk)
    pre = np.zeros((c["Lp"], ROW), np.uint8)
    oracle.k_quant_and_cache(c["k_pre"], np.arange(c["Lp"]), pre.reshape(-1), c["Lp"], c["Lp"] * ROW)
    dstarts = np.concatenate([[0], np.cumsum(c["dec_lens"])])
    done, scored = 0, 0
    for r in np.random.default_rng(5).permutation(nrows):
        sl = slice(int(r), int(r) + 1)
        if r < nd:
            L = int(c["dec_lens"][r])
            nblk = (L + bs - 1) // bs
            pool = np.zeros(nblk * bs * ROW, np.uint8)
            oracle.k_quant_and_cache(c["k_dec"][dstarts[r]:dstarts[r + 1]], np.arange(L), pool, bs, bs * ROW)
            bt = np.arange(nblk, dtype=np.int32)[None, :]
            kw = dict(k_src=pool, block_table=bt, row_to_req=np.zeros(1, np.int32), block_size=bs,
                      block_stride=bs * ROW)
        else:
            kw = dict(k_src=pre)
        lg = oracle.sparse_mqa_logits(c["q"][sl], c["w"][sl], c["ks"][sl], c["ke"][sl], si[sl], end[sl], sbk, **kw)
        col = oracle.topk_select(lg, end[sl], K, bf16=True)
        pos = oracle.topk_remap(col, si[sl], c["ks"][sl], sbk)
        if r < nd:
            oracle.req_index_to_global_slot(pos, kw["block_table"], bs, bs, row_to_req=np.zeros(1, np.int32))
        scored += int(end[r])
        done += 1
        if time.perf_counter() - t0 > share:
            break
    dt = time.perf_counter() - t0
    per["5_hierarchical_sparse"] = dict(value=scored / dt, unit="scored pairs/s", seconds=round(dt, 2),
                                        sample=f"expansion of all {nrows} rows, the 131K-token prefill history "
                                               f"quantized, then {done} rows scored, selected and remapped")
    head = per["2_prefill_chunk"]
    return dict(value=head["value"], unit="pairs/s", cores=1, kind="oracle",
                sample=f"prefill chunk: {head['sample']}, {head['seconds']} s; one thread on a host "
                       f"{host_cpu_model()} with {os.cpu_count()} logical CPUs",
                per_config=per)


# --------------------------------------------------------------------------- paged decode
def bench_decode(n, steps, warmup, copies=4, mxfp4=False):
    """Decode workload n: logits straight from the paged cache (132-byte FP8 rows, or 68-byte MXFP4 rows),
    top-2048, slot conversion."""
    c = synth.workload(n)
    bs, nb, nn, B = c["block_size"], c["num_blocks"], c["next_n"], c["B"]
    row = ROW_MXFP4 if mxfp4 else ROW
    stride = bs * row if mxfp4 else c["block_stride"]
    quant = dsi.k_quant_and_cache_mxfp4 if mxfp4 else dsi.k_quant_and_cache
    lens = c["context_lens"]
    maxc = int(lens.max())
    sumL = int(lens.sum())
    q, w, cl = dev(c["q"]), dev(c["w"]), dev(lens)
    ends_np = (np.repeat(lens, nn) - nn + np.tile(np.arange(nn), B) + 1).astype(np.int32)
    ends = dev(ends_np)
    r2r = dev(np.repeat(np.arange(B, dtype=np.int32), nn))
    k_t, slot_t = dev(c["k"]), dev(c["slot_mapping"])
    # independent pool copies, each with its own block permutation, so the 256 MB MALL cannot hold K
    pools, tables = [], []
    rng = np.random.default_rng(100 + n)
    for i in range(copies):
        perm = rng.permutation(nb).astype(np.int32)
        bt = perm[c["block_table"]]
        sl = (bt[np.repeat(np.arange(B), lens), np.concatenate([np.arange(L) for L in lens]) // bs].astype(np.int64)
              * bs + np.concatenate([np.arange(L) for L in lens]) % bs)
        pool = torch.zeros(nb * stride, dtype=torch.uint8, device="cuda")
        quant(k_t, dev(sl), pool, bs, stride, nb)
        pools.append(pool)
        tables.append(dev(bt))
    del k_t, slot_t
    rows = B * nn
    logits = torch.empty((rows, maxc), dtype=torch.float32, device="cuda")
    idx = torch.empty((rows, K), dtype=torch.int32, device="cuda")
    slots = torch.empty((rows, K), dtype=torch.int32, device="cuda")
    ws = torch.empty(max(dsi.paged_mqa_topk_decode_workspace_bytes(B, nn, maxc, K), 16), dtype=torch.uint8,
                     device="cuda")
    ws_sep = torch.empty(max(dsi.topk_workspace_bytes(rows, maxc, K), 16), dtype=torch.uint8, device="cuda")
    tlt, ts = EventTimer(), EventTimer()

    def decode_topk(i):
        dsi.paged_mqa_topk_decode(q, w, cl, pools[i % copies], bs, tables[i % copies], maxc, next_n=nn, k=K,
                                  logits=logits, out=idx, workspace=ws, block_stride_bytes=stride, num_blocks=nb,
                                  mxfp4=mxfp4)

    def logits_only(i):
        dsi.paged_mqa_logits_decode(q, w, cl, pools[i % copies], bs, tables[i % copies], maxc, next_n=nn,
                                    out=logits, block_stride_bytes=stride, num_blocks=nb, mxfp4=mxfp4)

    def step(i, timed):
        s = tlt.start() if timed else None
        decode_topk(i)
        if timed:
            tlt.stop(s)
            s = ts.start()
        dsi.req_index_to_global_slot(idx, tables[i % copies], bs, bs, row_to_req=r2r, out=slots)
        if timed:
            ts.stop(s)

    for i in range(warmup):
        step(i, False)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    queue_ahead(steps)
    a.record()
    for i in range(steps):
        step(i, True)
    b.record()
    torch.cuda.synchronize()
    ms_step = a.elapsed_time(b) / steps
    ms_lt, ms_s = tlt.mean_ms(), ts.mean_ms()
    # breakdown: the logits kernel alone, and the two separate calls (logits, then dsi_topk_select)
    tl, tsep = EventTimer(), EventTimer()
    queue_ahead(steps)
    for i in range(steps):
        s = tl.start()
        logits_only(i)
        tl.stop(s)
    ms_l = tl.mean_ms()
    queue_ahead(steps)
    for i in range(steps):
        s = tsep.start()
        logits_only(i)
        dsi.topk_select(logits, ends, k=K, out=idx, workspace=ws_sep)
        tsep.stop(s)
    ms_sep = tsep.mean_ms()
    V = int(ends_np.sum())
    nblk = int(sum((int(L) + bs - 1) // bs for L in lens))
    bytes_logits = row * sumL + 4 * nblk + rows * (64 * 128 + 64 * 2) + 4 * V
    bytes_topk = 4 * V + rows * K * 4
    gbs = (bytes_logits + bytes_topk) / (ms_lt * 1e-3) / 1e9
    cache = ", MXFP4 cache (68 B per token)" if mxfp4 else ""
    # the logits kernel against the measured rate of reading the same kind of pages with no scoring (the better of
    # the default cache policy and the non-temporal hint)
    kind = "mxfp4_pages" if mxfp4 else "fp8_pages"
    rates = [(PAGED_CEILING or {}).get(k + kind) for k in ("paged_read_gbs_", "paged_read_nt_gbs_")]
    ceil_gbs = max((r for r in rates if r), default=None)
    vs_paged = (round(bytes_logits / (ms_l * 1e-3) / 1e9 / ceil_gbs, 4) if ceil_gbs else None)
    return dict(workload=f"paged decode {B} x next_n {nn}, lengths U{{{int(lens.min())}..{int(lens.max())}}}{cache}",
                rows=rows, sum_tokens=sumL, ms_step=round(ms_step, 4), ms_logits_topk=round(ms_lt, 4),
                ms_logits=round(ms_l, 4), ms_topk=round(ms_lt - ms_l, 4), ms_slot=round(ms_s, 4),
                ms_separate_calls=round(ms_sep, 4),
                logits_gbs=round(bytes_logits / (ms_l * 1e-3) / 1e9, 1),
                logits_topk_gbs=round(gbs, 1), hbm_frac=round(gbs / HBM_PEAK_GBS, 4),
                logits_vs_paged_read_ceiling=vs_paged,
                rows_per_s=round(rows / (ms_lt * 1e-3), 1),
                algorithmic_bytes=bytes_logits + bytes_topk,
                timing="ms_logits_topk: dsi_paged_mqa_topk_decode (one call); ms_logits: the logits call alone; "
                       "ms_topk: their difference; ms_separate_calls: the logits call then dsi_topk_select")


# --------------------------------------------------------------------------- prefill K gather
def bench_gather(steps, warmup, pool_bytes=512 << 20):
    """Prefill K gather out of a paged pool: the prefill chunk's 8192-token history (64-token pages) and the
    longest hierarchical prefill request (131072 tokens, 128-token pages).  The pool holds 512 MB of random
    cache rows; each timed call reads a different, disjoint random set of its blocks, so K comes from HBM."""
    res = {}
    for name, L, bs in (("prefill_chunk_history", 8192, 64), ("longest_prefill_request", 131072, 128)):
        stride = bs * ROW
        nblk = (L + bs - 1) // bs
        nb = pool_bytes // stride
        copies = nb // nblk
        pool = torch.randint(0, 256, (nb * stride,), dtype=torch.uint8, device="cuda")
        perm = np.random.default_rng(L).permutation(nb)[:copies * nblk].astype(np.int32).reshape(copies, 1, nblk)
        tables = [dev(perm[i]) for i in range(copies)]
        cu = dev(np.array([0, L], dtype=np.int32))
        out = torch.empty((L, ROW), dtype=torch.uint8, device="cuda")
        tg = EventTimer()
        for i in range(warmup):
            dsi.gather_prefill_k(pool, bs, tables[i % copies], cu, out=out, block_stride_bytes=stride,
                                 num_blocks=nb)
        torch.cuda.synchronize()
        queue_ahead(steps, 50)
        for i in range(warmup, warmup + steps):
            s = tg.start() if i >= warmup else None
            dsi.gather_prefill_k(pool, bs, tables[i % copies], cu, out=out, block_stride_bytes=stride,
                                 num_blocks=nb)
            if i >= warmup:
                tg.stop(s)
        ms = tg.mean_ms()
        nbytes = 2 * ROW * L + 4 * nblk + 8
        gbs = nbytes / (ms * 1e-3) / 1e9
        res[name] = dict(tokens=L, block_size=bs, us=round(ms * 1e3, 2), algorithmic_bytes=nbytes,
                         gbs=round(gbs, 1), hbm_frac=round(gbs / HBM_PEAK_GBS, 4))
        del pool, tables, out
    return res


# --------------------------------------------------------------------------- q preparation
def bench_qprep(steps, warmup, T=2048, copies=16):
    """q RoPE + FP8 quantization + weight fold for the prefill chunk's 2048 tokens.  16 copies of the bf16 q
    (537 MB) rotate so that each call reads q from HBM."""
    c = synth.q_prep_case(2, T, max_pos=8192)
    qs = [dev(c["q"]) for _ in range(copies)]
    pos, cs, w = dev(c["positions"]), dev(c["cos_sin"]), dev(c["w"])
    q8 = torch.empty((T, 64, 128), dtype=torch.uint8, device="cuda")
    wo = torch.empty((T, 64), dtype=torch.int16, device="cuda")
    for i in range(warmup):
        dsi.q_rope_quant(qs[i % copies], pos, cs, w, c["softmax_scale"], c["head_scale"], out=(q8, wo))
    torch.cuda.synchronize()
    tq = EventTimer()
    queue_ahead(steps, 50)
    for i in range(steps):
        s = tq.start()
        dsi.q_rope_quant(qs[i % copies], pos, cs, w, c["softmax_scale"], c["head_scale"], out=(q8, wo))
        tq.stop(s)
    ms = tq.mean_ms()
    nbytes = T * (64 * (256 + 128 + 2 + 2) + 256 + 8)
    gbs = nbytes / (ms * 1e-3) / 1e9
    return dict(tokens=T, us=round(ms * 1e3, 2), algorithmic_bytes=nbytes, gbs=round(gbs, 1),
                hbm_frac=round(gbs / HBM_PEAK_GBS, 4))


# --------------------------------------------------------------------------- context-parallel merge
def bench_merge(steps, warmup, rows=64, ranks=8):
    """Merge of 8 ranks' local top-2048 candidate lists for the 64 rows of a decode step (what each rank
    receives from the all-gather): global top-2048 per row."""
    g = torch.Generator(device="cuda").manual_seed(7)
    vals = torch.randn((ranks, rows, K), generator=g, device="cuda", dtype=torch.float32)
    gidx = torch.arange(ranks * rows * K, dtype=torch.int32, device="cuda").view(ranks, rows, K)
    out = torch.empty((rows, K), dtype=torch.int32, device="cuda")
    ws = torch.empty(dsi.topk_merge_workspace_bytes(rows, ranks, K), dtype=torch.uint8, device="cuda")
    for _ in range(warmup):
        dsi.topk_merge(vals, gidx, k=K, out=out, workspace=ws)
    torch.cuda.synchronize()
    tm = EventTimer()
    queue_ahead(steps, 100)
    for _ in range(steps):
        s = tm.start()
        dsi.topk_merge(vals, gidx, k=K, out=out, workspace=ws)
        tm.stop(s)
    ms = tm.mean_ms()
    return dict(rows=rows, ranks=ranks, candidates_per_row=ranks * K, us=round(ms * 1e3, 2),
                exchanged_bytes_per_rank=rows * K * 8)


# --------------------------------------------------------------------------- hierarchical sparse
def bench_sparse(steps, warmup, c, mxfp4=False):
    """Workload 5, one step: expansion and the columns' schedule (both once per step, shared by every layer), sparse
    logits from the schedule (decode rows from the paged pool, prefill rows from the gathered chunk), bf16 top-k,
    remap and slot conversion.  mxfp4: the K cache in 68-byte MXFP4 rows.  The one-shot logits call (no schedule)
    is timed beside it."""
    sbk, cbs, nd, rows = c["sbk"], c["cbs"], c["n_decode"], c["rows"]
    bs, nb = c["block_size"], c["num_blocks"]
    row = ROW_MXFP4 if mxfp4 else ROW
    stride = bs * row
    quant = dsi.k_quant_and_cache_mxfp4 if mxfp4 else dsi.k_quant_and_cache
    logits_fn = dsi.sparse_mqa_logits_mxfp4 if mxfp4 else dsi.sparse_mqa_logits
    q, w, ks, ke, cand = dev(c["q"]), dev(c["w"]), dev(c["ks"]), dev(c["ke"]), dev(c["cand"])
    pool = torch.zeros(nb * stride, dtype=torch.uint8, device="cuda")
    quant(dev(c["k_dec"]), dev(c["dec_slot_mapping"]), pool, bs, stride, nb)
    Lp = c["Lp"]
    pre = torch.zeros((Lp, row), dtype=torch.uint8, device="cuda")
    quant(dev(c["k_pre"]), torch.arange(Lp, dtype=torch.int64, device="cuda"), pre.view(-1), Lp, Lp * row, 1)
    bt, r2r = dev(c["block_table"]), dev(c["row_to_req"])
    nsb = cand.shape[1] * (cbs // sbk)
    width = nsb * sbk
    si = torch.empty((rows, nsb), dtype=torch.int32, device="cuda")
    end = torch.empty((rows,), dtype=torch.int32, device="cuda")
    sched = torch.empty((rows, nsb), dtype=torch.int64, device="cuda")
    out = torch.empty((rows, width), dtype=torch.int16, device="cuda")
    col = torch.empty((rows, K), dtype=torch.int32, device="cuda")
    slots = torch.empty((nd, K), dtype=torch.int32, device="cuda")
    te, tl, tt, tr = EventTimer(), EventTimer(), EventTimer(), EventTimer()

    def step(timed):
        s = te.start() if timed else None
        dsi.expand_candidates(cand, ks, ke, cbs, sbk, out=(si, end))
        dsi.sparse_schedule(ks[:nd], ke[:nd], si[:nd], end[:nd], sbk, pool, block_table=bt, row_to_req=r2r,
                            block_size=bs, block_stride_bytes=stride, num_k=nb, mxfp4=mxfp4, out=sched[:nd])
        dsi.sparse_schedule(ks[nd:], ke[nd:], si[nd:], end[nd:], sbk, pre.view(-1), num_k=Lp, mxfp4=mxfp4,
                            out=sched[nd:])
        if timed:
            te.stop(s)
            s = tl.start()
        dsi.sparse_mqa_logits_scheduled(q[:nd], w[:nd], sched[:nd], sbk, pool, out=out[:nd], mxfp4=mxfp4)
        dsi.sparse_mqa_logits_scheduled(q[nd:], w[nd:], sched[nd:], sbk, pre.view(-1), out=out[nd:], mxfp4=mxfp4)
        if timed:
            tl.stop(s)
            s = tt.start()
        dsi.topk_select(out, end, k=K, out=col)
        if timed:
            tt.stop(s)
            s = tr.start()
        dsi.topk_remap(col, si, ks, sbk, out=col)
        dsi.req_index_to_global_slot(col[:nd], bt, bs, bs, row_to_req=r2r, out=slots)
        if timed:
            tr.stop(s)

    for _ in range(warmup):
        step(False)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    queue_ahead(steps)
    a.record()
    for _ in range(steps):
        step(True)
    b.record()
    torch.cuda.synchronize()
    ms_step = a.elapsed_time(b) / steps
    scored = int(host_end(end).sum())
    ms_l = tl.mean_ms()
    # the one-shot logits calls (columns' sources worked out inside the kernel), for comparison
    t1 = EventTimer()
    queue_ahead(steps)
    for _ in range(steps):
        s = t1.start()
        logits_fn(q[:nd], w[:nd], ks[:nd], ke[:nd], si[:nd], end[:nd], sbk, pool, block_table=bt, row_to_req=r2r,
                  block_size=bs, block_stride_bytes=stride, num_k=nb, out=out[:nd])
        logits_fn(q[nd:], w[nd:], ks[nd:], ke[nd:], si[nd:], end[nd:], sbk, pre.view(-1), num_k=Lp, out=out[nd:])
        t1.stop(s)
    ms_once = t1.mean_ms()
    return dict(workload=f"hierarchical sparse: {nd} decode rows + {rows - nd} prefill rows, {nsb} sparse blocks "
                         f"of {sbk}, {'MXFP4' if mxfp4 else 'FP8'} K cache ({row} B per token)", rows=rows,
                ms_step=round(ms_step, 4), ms_expand_schedule=round(te.mean_ms(), 4), ms_logits=round(ms_l, 4),
                ms_logits_one_shot=round(ms_once, 4), ms_topk=round(tt.mean_ms(), 4),
                ms_remap_slot=round(tr.mean_ms(), 4), scored_pairs=scored,
                pairs_per_s=round(scored / (ms_step * 1e-3), 1),
                logits_tflops=round(scored * FLOP_PER_PAIR / (ms_l * 1e-3) / 1e12, 1),
                effective_gathered_gbs=round(scored * row / (ms_l * 1e-3) / 1e9, 1),
                timing="expansion and schedule once per step (shared by every layer); ms_logits: the scheduled "
                       "logits calls of one layer; ms_logits_one_shot: the calls without a schedule")


def host_end(t):
    return t.cpu().numpy().astype(np.int64)


def bars(achieved_tflops, extra):
    """The stated targets and where this run stands against each (met or not, said plainly)."""
    fp8 = achieved_tflops / FP8_PEAK_TFLOPS
    out = {"prefill_logits_vs_fp8_peak": {
        "target": 0.5, "achieved": round(fp8, 4), "met": fp8 >= 0.5,
        "note": "the FP8 x FP8 contraction runs on the f16 matrix cores (codes decoded exactly to f16): gfx950's "
                "FP8-operand MFMAs truncate inside one instruction by more than the 1e-3 (1 + |ref|) logit "
                "tolerance; the f16 peak is half the FP8 peak, so 0.5 of FP8 is 1.0 of f16, unreachable on this "
                "path"}}
    rates = [(PAGED_CEILING or {}).get(k) for k in ("paged_read_gbs_fp8_pages", "paged_read_nt_gbs_fp8_pages")]
    ceil = max((r for r in rates if r), default=None)
    for n in (3, 4):
        w = extra.get(f"decode_w{n}")
        if w:
            bar = {"target": 0.6, "achieved": w["hbm_frac"], "met": w["hbm_frac"] >= 0.6}
            if ceil:
                bar["note"] = (f"reading the cache's 8448-byte pages alone, in a random order and with no scoring, "
                               f"measured {ceil:.0f} GB/s here ({ceil / HBM_PEAK_GBS:.3f} of the HBM peak); the "
                               f"logits kernel reaches {w['logits_vs_paged_read_ceiling']} of that rate, and the "
                               f"selection adds its own time after it")
            out[f"decode_w{n}_logits_topk_vs_hbm"] = bar
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-seconds", type=float, default=25.0)
    ap.add_argument("--only-headline", action="store_true")
    ap.add_argument("--no-ceilings", action="store_true")
    ap.add_argument("--workloads", default=None,
                    help="comma-separated subset of the reported workloads (default: all): " + ",".join(ALL_WORKLOADS))
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the indexer path runs on one GPU and has no multi-GPU mode "
              f"(--gpus {args.gpus} requested).", file=sys.stderr)
        sys.exit(2)
    chosen = ALL_WORKLOADS if args.workloads is None else [w for w in args.workloads.split(",") if w]
    unknown = [w for w in chosen if w not in ALL_WORKLOADS]
    if unknown:
        raise SystemExit(f"unknown workloads {unknown}; choose from {ALL_WORKLOADS}")
    if args.only_headline:
        chosen = []
    torch.cuda.set_device(0)
    dsi.lib()

    ceil = None
    if not args.no_ceilings:
        log("measured ceilings ...")
        ceil = measure_ceilings()
        log(ceil)
    global PAGED_CEILING
    PAGED_CEILING = ceil
    log("prefill chunk ...")
    pf = bench_prefill(args.steps, args.warmup)
    value = pf["pairs"] / (pf["ms_step"] * 1e-3)
    flops = pf["pairs"] * FLOP_PER_PAIR
    achieved = flops / (pf["ms_logits"] * 1e-3) / 1e12
    extra = {}
    for n in (3, 4):
        if f"decode_w{n}" in chosen:
            log(f"decode workload {n} ...")
            extra[f"decode_w{n}"] = bench_decode(n, args.steps, args.warmup)
    for n in (3, 4):
        if f"decode_w{n}_mxfp4" in chosen:
            log(f"decode workload {n}, MXFP4 cache ...")
            extra[f"decode_w{n}_mxfp4"] = bench_decode(n, args.steps, args.warmup, mxfp4=True)
    if "sparse_w5" in chosen or "sparse_w5_mxfp4" in chosen:
        c5 = synth.workload(5)
        if "sparse_w5" in chosen:
            log("hierarchical sparse ...")
            extra["sparse_w5"] = bench_sparse(args.steps, args.warmup, c5)
        if "sparse_w5_mxfp4" in chosen:
            log("hierarchical sparse, MXFP4 cache ...")
            extra["sparse_w5_mxfp4"] = bench_sparse(args.steps, args.warmup, c5, mxfp4=True)
        del c5
    if "prefill_gather" in chosen:
        log("prefill K gather ...")
        extra["prefill_gather"] = bench_gather(args.steps, args.warmup)
    if "q_prep" in chosen:
        log("q preparation ...")
        extra["q_prep"] = bench_qprep(args.steps, args.warmup)
    if "cp_merge" in chosen:
        log("context-parallel merge ...")
        extra["cp_merge"] = bench_merge(args.steps, args.warmup)
    log("cpu baseline ...")
    cpu = cpu_baselines(pf["c"], args.cpu_seconds)
    line = {
        "metric": "indexer q.k pairs/s (prefill chunk: k insert + dense FP8 logits + top-2048)",
        "value": round(value, 1),
        "unit": "pairs/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(pf["ms_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3 (decoded exactly to f16 for the f16 MFMA) -> f32 accumulate",
        "data": "synthetic (seeded numpy: q,k ~ N(0,1) to bf16, FP8 e4m3 with per-128 scales)",
        "config": {"workload": "prefill chunk: 1 request, T=2048 query tokens at positions 6144..8191, S=8192, "
                               "H=64, D=128, causal, top-2048", "T": pf["T"], "S": pf["S"], "pairs": pf["pairs"],
                   "ms_logits": round(pf["ms_logits"], 4), "ms_topk": round(pf["ms_topk"], 4)},
        "roofline": {"bound": "mfma", "kernel": "prefill_logits_kernel", "achieved": round(achieved, 1),
                     "peak": F16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / F16_PEAK_TFLOPS, 4),
                     "traffic": committed_traffic(), "algorithmic_flops_per_launch": flops,
                     "mfma_dtype": "f16 (v_mfma_f32_16x16x32_f16)",
                     "frac_of_fp8_peak": round(achieved / FP8_PEAK_TFLOPS, 4),
                     # the same instruction in a register-only loop on random FP8 codes (the chip's power limit)
                     "frac_of_random_operand_loop": (round(achieved / ceil["mfma_f16_random_sustained_tflops"], 4)
                                                     if ceil and ceil.get("mfma_f16_random_sustained_tflops")
                                                     else None),
                     "measured_ceiling": ceil},
        "cpu_baseline": cpu,
        "bars": bars(achieved, extra),
        "pages_cost_context": {
            "indexer": "64 heads x 128 dims, FP8 q and k", "main_mla": "128 heads x 576 dims, bf16",
            "indexer_cache_bytes_per_token": 132, "main_mla_cache_bytes_per_token": 1152,
            "source": "DeepSeek V3.2 DSA inference flow page, the scorer cost table"},
        "workloads": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
