"""Every call only enqueues work and never synchronises or allocates, so a whole indexer step can be captured
into a HIP graph once and replayed (page "V4.1 indexer uses sparse MQA logits": the path is exercised under
CUDA-graph capture, with the expansion and schedule reused by later layers).

The decode step (k insert, paged logits, split top-k with its workspace, slot conversion; on the FP8 and on the
MXFP4 cache) and the hierarchical
step (expansion, sparse logits, bf16 top-k, remap) are captured, then replayed several times with eager work and
synchronisation between the replays; every replay must reproduce the eager outputs (selections compared by their value multisets, since the order of the output and
the choice among tied values are free).
"""
import numpy as np
import pytest
import torch

import sparse_attention_token_amd as dsi
import synth
from parity_util import ROW, dev, host

pytestmark = pytest.mark.gpu
K = 2048


@pytest.mark.parametrize("mxfp4", [False, True])
def test_decode_step_graph_replays(mxfp4):
    c = synth.decode_case(90, B=8, next_n=1, lmin=3000, lmax=40000, block_size=64)
    bs, nb = c["block_size"], c["num_blocks"]
    stride = bs * 68 if mxfp4 else c["block_stride"]
    quant = dsi.k_quant_and_cache_mxfp4 if mxfp4 else dsi.k_quant_and_cache
    lens = c["context_lens"]
    maxc = int(lens.max())
    pool = torch.zeros(nb * stride, dtype=torch.uint8, device="cuda")
    k_t, slots_t = dev(c["k"]), dev(c["slot_mapping"])
    q, w, cl, bt = dev(c["q"]), dev(c["w"]), dev(lens), dev(c["block_table"])
    ends = dev(lens.astype(np.int32))
    logits = torch.empty((8, maxc), dtype=torch.float32, device="cuda")
    idx = torch.empty((8, K), dtype=torch.int32, device="cuda")
    slots = torch.empty((8, K), dtype=torch.int32, device="cuda")
    ws = torch.empty(max(dsi.topk_workspace_bytes(8, maxc, K), 16), dtype=torch.uint8, device="cuda")
    assert dsi.topk_workspace_bytes(8, maxc, K) > 0  # the split path with its workspace is in the graph

    def step():
        quant(k_t, slots_t, pool, bs, stride, nb)
        dsi.paged_mqa_logits_decode(q, w, cl, pool, bs, bt, maxc, out=logits, block_stride_bytes=stride,
                                    num_blocks=nb, mxfp4=mxfp4)
        dsi.topk_select(logits, ends, k=K, out=idx, workspace=ws)
        dsi.req_index_to_global_slot(idx, bt, bs, bs, out=slots)

    step()
    torch.cuda.synchronize()
    ref_logits, ref_idx = host(logits).copy(), host(idx).copy()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm-up on the capture stream
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        logits.fill_(0.0)
        idx.fill_(-7)
        slots.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = host(logits)
        for r in range(8):
            L = int(lens[r])
            assert np.array_equal(got[r, :L], ref_logits[r, :L]), (rep, r)
        ix, sl = host(idx), host(slots)
        for r in range(8):  # the selection by its value multiset (unique even under ties)
            assert np.array_equal(np.sort(got[r][ix[r][ix[r] >= 0]]), np.sort(ref_logits[r][ref_idx[r][ref_idx[r] >= 0]]))
        p = np.maximum(ix, 0)
        want = np.where(ix >= 0, np.take_along_axis(c["block_table"], p // bs, axis=1) * bs + p % bs, -1)
        assert np.array_equal(sl, want), rep


@pytest.mark.parametrize("mxfp4,next_n", [(False, 1), (True, 1), (False, 2)])
def test_fused_decode_call_graph_replays(mxfp4, next_n):
    """The decode step through dsi_paged_mqa_topk_decode (logits with the top-k's histograms counted in the decode
    kernel when there is one row per request, the split top-k, slot conversion) captured once and replayed; the
    workspace is overwritten with other bytes before every replay, since the call keeps no state in it."""
    c = synth.decode_case(93, B=12, next_n=next_n, lmin=1000, lmax=50000, block_size=64)
    bs, nb = c["block_size"], c["num_blocks"]
    stride = bs * 68 if mxfp4 else c["block_stride"]
    quant = dsi.k_quant_and_cache_mxfp4 if mxfp4 else dsi.k_quant_and_cache
    lens = c["context_lens"]
    maxc = int(lens.max())
    B, rows = 12, 12 * next_n
    pool = torch.zeros(nb * stride, dtype=torch.uint8, device="cuda")
    quant(dev(c["k"]), dev(c["slot_mapping"]), pool, bs, stride, nb)
    q, w, cl, bt = dev(c["q"]), dev(c["w"]), dev(lens), dev(c["block_table"])
    logits = torch.empty((rows, maxc), dtype=torch.float32, device="cuda")
    idx = torch.empty((rows, K), dtype=torch.int32, device="cuda")
    slots = torch.empty((rows, K), dtype=torch.int32, device="cuda")
    r2r = dev(np.repeat(np.arange(B, dtype=np.int32), next_n))
    need = dsi.paged_mqa_topk_decode_workspace_bytes(B, next_n, maxc)
    # one row per request: the fused path (slots per workgroup and request); two: the top-k's own split path
    plain = dsi.topk_workspace_bytes(rows, maxc, K)
    assert plain > 0 and (need > plain if next_n == 1 else need == plain)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")

    def step():
        dsi.paged_mqa_topk_decode(q, w, cl, pool, bs, bt, maxc, next_n=next_n, logits=logits, out=idx, workspace=ws,
                                  block_stride_bytes=stride, num_blocks=nb, mxfp4=mxfp4)
        dsi.req_index_to_global_slot(idx, bt, bs, bs, row_to_req=r2r, out=slots)

    step()
    torch.cuda.synchronize()
    ref_logits, ref_idx = host(logits).copy(), host(idx).copy()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        logits.fill_(0.0)
        idx.fill_(-7)
        slots.fill_(-7)
        ws.fill_(0x5A + rep)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got, ix, sl = host(logits), host(idx), host(slots)
        for r in range(rows):
            L = int(lens[r // next_n]) - next_n + r % next_n + 1  # the row's visible tokens
            assert np.array_equal(got[r, :L], ref_logits[r, :L]), (rep, r)
            assert np.array_equal(np.sort(got[r][ix[r][ix[r] >= 0]]),
                                  np.sort(ref_logits[r][ref_idx[r][ref_idx[r] >= 0]])), (rep, r)
            assert np.all(ix[r][min(K, L):] == -1)
        p = np.maximum(ix, 0)
        bt_rows = np.repeat(c["block_table"], next_n, axis=0)
        want = np.where(ix >= 0, np.take_along_axis(bt_rows, p // bs, axis=1) * bs + p % bs, -1)
        assert np.array_equal(sl, want), rep


@pytest.mark.parametrize("scheduled", [False, True])
def test_hierarchical_step_graph_replays(scheduled):
    rng = np.random.default_rng(91)
    T, S, sbk = 64, 6000, 64
    c = synth.prefill_case(92, T=T, S=S, first_pos=S - T)
    rows = torch.zeros((S, ROW), dtype=torch.uint8, device="cuda")
    dsi.k_quant_and_cache(dev(c["k"]), dev(np.arange(S, dtype=np.int64)), rows.view(-1), S, S * ROW, 1)
    ks, ke = np.zeros(T, np.int32), c["ke"]
    maxb = (ke + sbk - 1) // sbk
    cand = synth.draw_candidates(rng, maxb, num=48, distinct=40, dup=4)
    q, w, ks_t, ke_t, cand_t = dev(c["q"]), dev(c["w"]), dev(ks), dev(ke), dev(cand)
    si = torch.empty((T, 48), dtype=torch.int32, device="cuda")
    end = torch.empty((T,), dtype=torch.int32, device="cuda")
    out = torch.empty((T, 48 * sbk), dtype=torch.int16, device="cuda")
    col = torch.empty((T, K), dtype=torch.int32, device="cuda")
    pos = torch.empty((T, K), dtype=torch.int32, device="cuda")

    sched = torch.empty((T, 48), dtype=torch.int64, device="cuda")

    def step():
        dsi.expand_candidates(cand_t, ks_t, ke_t, sbk, sbk, out=(si, end))
        if scheduled:  # the per-step schedule, then the logits from it
            dsi.sparse_schedule(ks_t, ke_t, si, end, sbk, rows, out=sched)
            dsi.sparse_mqa_logits_scheduled(q, w, sched, sbk, rows, out=out)
        else:
            dsi.sparse_mqa_logits(q, w, ks_t, ke_t, si, end, sbk, rows, out=out)
        dsi.topk_select(out, end, k=K, out=col)
        dsi.topk_remap(col, si, ks_t, sbk, out=pos)

    def selected_values(o, cl):
        # bf16 logits tie often (and duplicated candidate blocks repeat tokens), so the selection is compared
        # by its value multiset, which is unique
        vals = o.view(np.uint16).astype(np.uint32) << 16
        return [np.sort(vals.view(np.float32)[r][cl[r][cl[r] >= 0]]) for r in range(T)]

    step()
    torch.cuda.synchronize()
    ref = [host(t).copy() for t in (si, end, out)]
    ref_sel = selected_values(ref[2], host(col))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        for t in (si, end, out, col, pos, sched):
            t.fill_(-3)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip((si, end, out), ref):
            assert np.array_equal(host(a), b), rep
        cl, ps, sih = host(col), host(pos), host(si)
        for r, (a, b) in enumerate(zip(selected_values(ref[2], cl), ref_sel)):
            assert np.array_equal(a, b), (rep, r)
        cc = np.maximum(cl, 0)
        want = np.where(cl >= 0, (np.take_along_axis(sih, cc // sbk, axis=1) - (ks[:, None] // sbk)) * sbk + cc % sbk,
                        -1)
        assert np.array_equal(ps, want), rep
