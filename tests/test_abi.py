"""The C-ABI library loads without a GPU, exports every entry point include/dsi.h declares, and rejects
bad host-known arguments before any HIP call (fail closed, never a slower fallback: vLLM PR 56254 summary,
review highlights)."""
import ctypes
import os
import re
import subprocess

import pytest

import sparse_attention_token_amd as dsi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EINVAL, EUNSUP, EALIGN, EWS = -1, -2, -3, -5
A16 = 0x10000  # a fake, 16-byte aligned non-null "device" pointer.  Every call below is either invalid
# (rejected on the host) or empty (returns before any launch), so no kernel ever sees this pointer.


def declared():
    src = open(os.path.join(ROOT, "include", "dsi.h")).read()
    return sorted(set(re.findall(r"DSI_API\s+[\w\s\*]*?\b(dsi_\w+)\s*\(", src)))


def test_header_declares_the_eight_steps():
    names = declared()
    for step in ["k_quant_and_cache", "mqa_logits_prefill", "paged_mqa_logits_decode", "topk_select",
                 "expand_candidates", "sparse_mqa_logits", "topk_remap", "req_index_to_global_slot"]:
        assert "dsi_" + step in names


def test_library_exports_every_declared_symbol():
    lib = dsi.lib()
    for name in declared():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", dsi.LIB_PATH], capture_output=True, text=True).stdout
    exported = sorted(set(re.findall(r" T (dsi_\w+)", out)))
    assert exported == declared()
    assert sorted(dsi.ENTRY_POINTS) == declared()


def test_status_strings():
    for code in (0, -1, -2, -3, -4, -5):
        assert dsi.status_string(code)
    assert dsi.status_string(-99) == "unknown status"
    assert dsi.lib().dsi_abi_version() >= 1


def test_k_quant_validation():
    L = dsi.lib()
    assert L.dsi_k_quant_and_cache(None, -1, 128, None, None, 1, 64, 64 * 132, None) == EINVAL
    assert L.dsi_k_quant_and_cache(None, 4, 127, None, None, 1, 64, 64 * 132, None) == EINVAL
    assert L.dsi_k_quant_and_cache(None, 4, 128, None, None, 1, 64, 64 * 132, None) == EINVAL  # nulls
    assert L.dsi_k_quant_and_cache(A16, 4, 128, A16, A16, 1, 64, 64 * 132 - 4, None) == EINVAL  # stride < row
    assert L.dsi_k_quant_and_cache(A16, 4, 128, A16, A16, 1, 0, 0, None) == EINVAL
    assert L.dsi_k_quant_and_cache(A16 + 2, 4, 128, A16, A16, 1, 64, 64 * 132, None) == EALIGN
    assert L.dsi_k_quant_and_cache(A16, 4, 129, A16, A16, 1, 64, 64 * 132, None) == EALIGN
    assert L.dsi_k_quant_and_cache(A16, 4, 128, A16, A16, 1, 64, 64 * 132 + 2, None) == EALIGN
    assert L.dsi_k_quant_and_cache(None, 0, 128, None, None, 0, 64, 64 * 132, None) == 0  # empty: no-op


def test_prefill_validation():
    L = dsi.lib()
    f = L.dsi_mqa_logits_prefill
    assert f(None, None, -1, None, 10, None, None, None, 10, None) == EINVAL
    assert f(A16, A16, 4, A16, 10, A16, A16, A16, 9, None) == EINVAL  # ld < S
    assert f(A16, A16, 4, None, 10, A16, A16, A16, 10, None) == EINVAL
    assert f(A16 + 8, A16, 4, A16, 10, A16, A16, A16, 10, None) == EALIGN
    assert f(A16, A16, 4, A16 + 4, 10, A16, A16, A16, 10, None) == EALIGN
    assert f(A16, A16 + 4, 4, A16, 10, A16, A16, A16, 10, None) == EALIGN
    assert f(None, None, 0, None, 10, None, None, None, 10, None) == 0


def test_decode_validation():
    L = dsi.lib()

    def call(**kw):
        a = dict(q=A16, w=A16, B=2, next_n=1, cl=A16, pool=A16, nb=10, bs=64, stride=64 * 132, bt=A16, bt_ld=4,
                 bt_w=4, maxc=256, out=A16, ld=256)
        a.update(kw)
        return L.dsi_paged_mqa_logits_decode(a["q"], a["w"], a["B"], a["next_n"], a["cl"], a["pool"], a["nb"],
                                             a["bs"], a["stride"], a["bt"], a["bt_ld"], a["bt_w"], a["maxc"],
                                             a["out"], a["ld"], None)
    assert call(next_n=0) == EUNSUP and call(next_n=5) == EUNSUP
    assert call(bs=8) == EUNSUP and call(bs=24) == EUNSUP
    assert call(ld=255) == EINVAL and call(B=-1) == EINVAL and call(bt_ld=3) == EINVAL
    assert call(stride=64 * 132 - 16) == EINVAL
    assert call(pool=None) == EINVAL and call(bt=None) == EINVAL
    assert call(stride=64 * 132 + 4) == EALIGN and call(q=A16 + 4) == EALIGN and call(pool=A16 + 8) == EALIGN
    assert call(B=0) == 0


def test_topk_validation():
    L = dsi.lib()
    f = L.dsi_topk_select
    assert f(A16, 0, 10, 2, None, A16, 10, 0, A16, 10, None, 0, None) == EUNSUP  # k = 0
    assert f(A16, 0, 10, 2, None, A16, 10, 2049, A16, 2049, None, 0, None) == EUNSUP
    assert f(A16, 7, 10, 2, None, A16, 10, 4, A16, 4, None, 0, None) == EUNSUP  # dtype
    assert f(A16, 0, 9, 2, None, A16, 10, 4, A16, 4, None, 0, None) == EINVAL  # ld < width
    assert f(A16, 0, 10, 2, None, A16, 10, 4, A16, 3, None, 0, None) == EINVAL  # out_ld < k
    assert f(None, 0, 10, 2, None, A16, 10, 4, A16, 4, None, 0, None) == EINVAL
    assert f(A16 + 2, 0, 10, 2, None, A16, 10, 4, A16, 4, None, 0, None) == EALIGN
    assert f(A16 + 1, 1, 10, 2, None, A16, 10, 4, A16, 4, None, 0, None) == EALIGN
    assert f(None, 0, 10, 0, None, None, 10, 4, None, 4, None, 0, None) == 0
    assert L.dsi_topk_workspace_bytes(64, 131072, 2048) > 0  # few long rows are split: workspace needed
    assert L.dsi_topk_workspace_bytes(2048, 8192, 2048) == 0  # one workgroup per row
    assert f(A16, 0, 40000, 4, None, A16, 40000, 2048, A16, 2048, None, 0, None) == EWS
    need = L.dsi_topk_workspace_bytes(4, 40000, 2048)
    assert f(A16, 0, 40000, 4, None, A16, 40000, 2048, A16, 2048, A16, need - 1, None) == EWS
    assert f(A16, 0, 40000, 4, None, A16, 40000, 2048, A16, 2048, A16 + 4, need, None) == EALIGN


def test_expand_validation():
    L = dsi.lib()

    def call(cbs=16, sbk=16, K=4, cand_ld=4, si_ld=4, rows=2, cand=A16):
        return L.dsi_expand_candidates(cand, cand_ld, rows, K, A16, 1, A16, 1, cbs, sbk, A16, si_ld, A16, 1, None)
    assert call(cbs=48, sbk=16) == EUNSUP  # ratio 3
    assert call(cbs=24, sbk=16) == EUNSUP  # not exact
    assert call(sbk=12, cbs=12) == EUNSUP and call(sbk=256, cbs=256) == EUNSUP and call(sbk=4, cbs=4) == EUNSUP
    assert call(cbs=32, sbk=16, si_ld=7) == EINVAL  # si_ld < K*ratio
    assert call(cand_ld=3) == EINVAL and call(K=0) == EINVAL and call(cand=None) == EINVAL
    assert call(K=1025, cand_ld=1025, si_ld=1025) == EUNSUP
    assert call(rows=0) == 0


def test_sparse_validation():
    L = dsi.lib()

    def call(sbk=16, nsb=4, si_ld=4, ld=64, bt=None, bs=0, stride=0, k_src=A16, q=A16):
        return L.dsi_sparse_mqa_logits(q, A16, 2, A16, A16, A16, si_ld, nsb, A16, sbk, k_src, 100, bt, 4, 4, 2,
                                       None, bs, stride, A16, ld, None)
    assert call(sbk=12) == EUNSUP and call(sbk=4) == EUNSUP
    assert call(si_ld=3) == EINVAL and call(ld=63) == EINVAL and call(nsb=0) == EINVAL
    assert call(bt=A16, bs=24, stride=24 * 132) == EUNSUP  # block_size not a multiple of sbk
    assert call(bt=A16, bs=64, stride=64 * 132 - 16) == EINVAL
    assert call(bt=A16, bs=64, stride=64 * 132 + 4) == EALIGN
    assert call(k_src=None) == EINVAL
    assert call(q=A16 + 4) == EALIGN


def test_remap_and_slot_validation():
    L = dsi.lib()
    assert L.dsi_topk_remap(A16, 4, 2, 4, A16, 4, 4, A16, 0, A16, 4, None) == EUNSUP
    assert L.dsi_topk_remap(A16, 3, 2, 4, A16, 4, 4, A16, 16, A16, 4, None) == EINVAL
    assert L.dsi_topk_remap(None, 4, 2, 4, A16, 4, 4, A16, 16, A16, 4, None) == EINVAL
    assert L.dsi_topk_remap(A16, 4, 0, 4, A16, 4, 4, A16, 16, A16, 4, None) == 0
    f = L.dsi_req_index_to_global_slot
    assert f(A16, 4, 2, 4, None, A16, 8, 8, 2, 0, 64, A16, 4, None) == EUNSUP
    assert f(A16, 4, 2, 4, None, A16, 8, 8, 2, 64, 63, A16, 4, None) == EUNSUP  # span < block_size
    assert f(A16, 4, 2, 4, None, A16, 7, 8, 2, 64, 64, A16, 4, None) == EINVAL  # bt_ld < bt_width
    assert f(A16, 4, 2, 4, None, None, 8, 8, 2, 64, 64, A16, 4, None) == EINVAL
    assert f(A16, 4, 2, 0, None, A16, 8, 8, 2, 64, 64, A16, 4, None) == 0


def test_gather_validation():
    f = dsi.lib().dsi_gather_prefill_k

    def call(pool=A16, nb=4, bs=64, stride=64 * 132, bt=A16, bt_ld=8, bt_width=8, cu=A16, nreq=2, out=A16, S=10):
        return f(pool, nb, bs, stride, bt, bt_ld, bt_width, cu, nreq, out, S, None)

    assert call(S=-1) == EINVAL and call(nreq=-1) == EINVAL and call(bs=0) == EINVAL and call(nb=-1) == EINVAL
    assert call(bt_ld=7) == EINVAL and call(stride=64 * 132 - 4) == EINVAL and call(bt_width=-1) == EINVAL
    assert call(pool=None) == EINVAL and call(bt=None) == EINVAL and call(cu=None) == EINVAL
    assert call(out=None) == EINVAL
    assert call(out=A16 + 4) == EALIGN and call(pool=A16 + 2) == EALIGN and call(stride=64 * 132 + 2) == EALIGN
    assert call(S=0x7FFFFFFF) == EUNSUP
    assert call(S=0, pool=None, out=None) == 0


def test_q_rope_quant_validation():
    f = dsi.lib().dsi_q_rope_quant

    def call(q=A16, q_ld=8192, T=4, pos=A16, cs=A16, max_pos=16, w=A16, w_ld=64, q8=A16, wo=A16):
        return f(q, q_ld, T, pos, cs, max_pos, 0, w, w_ld, 1.0, 1.0, q8, wo, None)

    assert call(T=-1) == EINVAL and call(q_ld=8191) == EINVAL and call(w_ld=63) == EINVAL
    assert call(max_pos=0) == EINVAL
    for k in ("q", "pos", "cs", "w", "q8", "wo"):
        assert call(**{k: None}) == EINVAL, k
    assert call(q=A16 + 8) == EALIGN and call(q_ld=8196) == EALIGN and call(cs=A16 + 4) == EALIGN
    assert call(pos=A16 + 4) == EALIGN and call(q8=A16 + 4) == EALIGN and call(wo=A16 + 1) == EALIGN
    assert call(T=0, q=None) == 0


def test_cp_merge_validation():
    L = dsi.lib()
    f = L.dsi_topk_values
    assert f(A16, 8, 2, None, 9, A16, 4, 4, 1, 0, A16, 4, A16, 4, None) == EINVAL  # ld < max_width
    assert f(A16, 8, 2, None, 8, A16, 3, 4, 1, 0, A16, 4, A16, 4, None) == EINVAL  # idx_ld < k
    assert f(None, 8, 2, None, 8, A16, 4, 4, 1, 0, A16, 4, A16, 4, None) == EINVAL
    assert f(A16 + 2, 8, 2, None, 8, A16, 4, 4, 1, 0, A16, 4, A16, 4, None) == EALIGN
    assert f(None, 8, 0, None, 8, None, 4, 4, 1, 0, None, 4, None, 4, None) == 0
    need = L.dsi_topk_merge_workspace_bytes(4, 2, 64)
    assert need >= 4 * 2 * 64 * 4 and L.dsi_topk_merge_workspace_bytes(0, 2, 64) == 0
    m = L.dsi_topk_merge
    assert m(A16, A16, 256, 64, 2, 4, 64, 0, A16, 64, A16, need, None) == EUNSUP      # k = 0
    assert m(A16, A16, 256, 64, 2, 4, 64, 2049, A16, 4096, A16, need, None) == EUNSUP
    assert m(A16, A16, 256, 63, 2, 4, 64, 16, A16, 64, A16, need, None) == EINVAL     # row_ld < k_in
    assert m(A16, A16, 256, 64, 0, 4, 64, 16, A16, 64, A16, need, None) == EINVAL     # no lists
    assert m(A16, A16, 256, 64, 2, 4, 64, 16, A16, 15, A16, need, None) == EINVAL     # out_ld < k
    assert m(A16, A16, 256, 64, 2, 4, 64, 16, A16, 64, A16, need - 1, None) == EWS
    assert m(A16, A16, 256, 64, 2, 4, 64, 16, A16, 64, A16 + 4, need, None) == EALIGN
    assert m(None, A16, 256, 64, 2, 4, 64, 16, A16, 64, A16, need, None) == EINVAL
    assert m(None, None, 256, 64, 2, 0, 64, 16, None, 64, None, 0, None) == 0


def test_mxfp4_validation():
    L = dsi.lib()
    f = L.dsi_k_quant_and_cache_mxfp4
    assert f(A16, 4, 128, A16, A16, 1, 64, 64 * 68 - 4, None) == EINVAL  # stride < 64 rows of 68
    assert f(A16, 4, 127, A16, A16, 1, 64, 64 * 68, None) == EINVAL
    assert f(A16 + 2, 4, 128, A16, A16, 1, 64, 64 * 68, None) == EALIGN
    assert f(None, 0, 128, None, None, 1, 64, 64 * 68, None) == 0
    g = L.dsi_sparse_mqa_logits_mxfp4

    def call(sbk=16, nsb=4, si_ld=4, ld=64, bt=None, bs=0, stride=0, k_src=A16, q=A16):
        return g(q, A16, 2, A16, A16, A16, si_ld, nsb, A16, sbk, k_src, 10, bt, 8, 8, 2, None, bs, stride, A16, ld,
                 None)

    assert call(sbk=12) == EUNSUP and call(si_ld=3) == EINVAL and call(ld=63) == EINVAL
    assert call(bt=A16, bs=64, stride=64 * 68 - 16) == EINVAL
    assert call(bt=A16, bs=64, stride=64 * 68 + 8) == EALIGN
    assert call(bt=A16, bs=24) == EUNSUP and call(k_src=None) == EINVAL and call(q=A16 + 8) == EALIGN


def test_decode_mxfp4_validation():
    """The MXFP4 paged decode takes the FP8 decode's checks, with 68-byte rows in the page stride."""
    L = dsi.lib()

    def call(**kw):
        a = dict(q=A16, w=A16, B=2, next_n=1, cl=A16, pool=A16, nb=10, bs=64, stride=64 * 68, bt=A16, bt_ld=4,
                 bt_w=4, maxc=256, out=A16, ld=256)
        a.update(kw)
        return L.dsi_paged_mqa_logits_decode_mxfp4(a["q"], a["w"], a["B"], a["next_n"], a["cl"], a["pool"], a["nb"],
                                                   a["bs"], a["stride"], a["bt"], a["bt_ld"], a["bt_w"], a["maxc"],
                                                   a["out"], a["ld"], None)
    assert call(next_n=0) == EUNSUP and call(next_n=5) == EUNSUP and call(bs=24) == EUNSUP
    assert call(ld=255) == EINVAL and call(B=-1) == EINVAL and call(bt_ld=3) == EINVAL
    assert call(stride=64 * 68 - 16) == EINVAL  # a page must hold block_size rows of 68 bytes
    assert call(pool=None) == EINVAL and call(out=None) == EINVAL
    assert call(stride=64 * 68 + 4) == EALIGN and call(q=A16 + 4) == EALIGN and call(w=A16 + 2) == EALIGN
    assert call(B=0) == 0


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(dsi, "_lib", None)
    monkeypatch.setattr(dsi, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        dsi.lib()


def test_ceiling_library_exports_and_validation():
    from sparse_attention_token_amd import ceiling
    src = open(os.path.join(ROOT, "include", "dsi_ceiling.h")).read()
    names = sorted(set(re.findall(r"DSIC_API\s+[\w\s\*]*?\b(dsic_\w+)\s*\(", src)))
    assert names == sorted(ceiling.ENTRY_POINTS)
    out = subprocess.run(["nm", "-D", "--defined-only", ceiling.LIB_PATH], capture_output=True, text=True).stdout
    assert sorted(set(re.findall(r" T (dsic_\w+)", out))) == names
    L = ceiling.lib()
    assert L.dsic_mfma_loop(5, 1, 1, A16, None) == EINVAL
    assert L.dsic_mfma_loop(-1, 1, 1, A16, None) == EINVAL
    assert L.dsic_mfma_loop(0, 0, 1, A16, None) == EINVAL
    assert L.dsic_mfma_loop(0, 1, 1, None, None) == EINVAL
    assert L.dsic_stream_read(A16, 24, 1, 0, A16, None) == EINVAL
    assert L.dsic_stream_read(A16, 32, 1, 2, A16, None) == EINVAL                     # nontemporal 0 or 1
    assert L.dsic_stream_read(A16 + 4, 32, 1, 0, A16, None) == EALIGN
    assert L.dsic_copy(A16, A16 + 8, 32, 1, None) == EALIGN
    assert L.dsic_copy(None, A16, 32, 1, None) == EINVAL
    P = 1 << 20
    assert L.dsic_paged_read(A16, P, 8448, A16, 1, 8448 + 8, 4, 0, 1, A16, None) == EINVAL   # page not whole 16 B
    assert L.dsic_paged_read(A16, P, 8448, A16, 1, 12304, 4, 0, 1, A16, None) == EINVAL      # page over 12 KB
    assert L.dsic_paged_read(A16, P, 4096, A16, 1, 8448, 4, 0, 1, A16, None) == EINVAL       # stride below a page
    assert L.dsic_paged_read(A16, P, 8448, A16, 0, 8448, 4, 0, 1, A16, None) == EINVAL       # no pages
    assert L.dsic_paged_read(A16, P, 8448, A16, 1, 8448, 6, 0, 1, A16, None) == EINVAL       # 4 or 8 per round
    assert L.dsic_paged_read(A16, P, 8448, A16, 1, 8448, 4, 3, 1, A16, None) == EINVAL       # nontemporal 0 or 1
    assert L.dsic_paged_read(A16, 4096, 8448, A16, 1, 8448, 4, 0, 1, A16, None) == EINVAL    # pool below a page
    assert L.dsic_paged_read(A16 + 4, P, 8448, A16, 1, 8448, 4, 0, 1, A16, None) == EALIGN


def test_probe_library_exports_and_validation():
    from sparse_attention_token_amd import probe
    src = open(os.path.join(ROOT, "include", "dsi_probe.h")).read()
    names = sorted(set(re.findall(r"DSI_PROBE_API\s+[\w\s\*]*?\b(dsip_\w+)\s*\(", src)))
    assert names == sorted(probe.ENTRY_POINTS)
    out = subprocess.run(["nm", "-D", "--defined-only", probe.LIB_PATH], capture_output=True, text=True).stdout
    assert sorted(set(re.findall(r" T (dsip_\w+)", out))) == names
    L = probe.lib()
    assert L.dsip_e4m3_encode_changes(0, 0, A16, 4, A16, A16, None) == EINVAL  # n < 1
    assert L.dsip_e4m3_encode_changes(0xFFFFFFF0, 32, A16, 4, A16, A16, None) == EINVAL  # past 2^32
    assert L.dsip_e4m3_encode_changes(0, 16, None, 4, A16, A16, None) == EINVAL
    assert L.dsip_e4m3_decode_all(None, A16, None) == EINVAL
    assert L.dsip_fp4_decode_all(None, None) == EINVAL


def test_decode_topk_call_validation():
    L = dsi.lib()

    def call(**kw):
        a = dict(q=A16, w=A16, B=2, next_n=1, cl=A16, pool=A16, nb=10, bs=64, stride=64 * 132, bt=A16, bt_ld=4,
                 bt_w=4, maxc=256, logits=A16, ld=256, k=2048, out=A16, out_ld=2048, ws=A16, ws_bytes=1 << 30)
        a.update(kw)
        return L.dsi_paged_mqa_topk_decode(a["q"], a["w"], a["B"], a["next_n"], a["cl"], a["pool"], a["nb"], a["bs"],
                                           a["stride"], a["bt"], a["bt_ld"], a["bt_w"], a["maxc"], a["logits"],
                                           a["ld"], a["k"], a["out"], a["out_ld"], a["ws"], a["ws_bytes"], None)
    assert call(k=0) == EUNSUP and call(k=2049) == EUNSUP
    assert call(out_ld=100, k=128) == EINVAL
    assert call(ld=255) == EINVAL
    assert call(next_n=5) == EUNSUP
    assert call(out=None) == EINVAL
    assert call(out=A16 + 2) == EALIGN
    assert call(B=8, maxc=40000, ld=40000, ws_bytes=16) == EWS  # the split path needs a workspace
    assert call(B=0) == 0
    assert L.dsi_paged_mqa_topk_decode_workspace_bytes(8, 1, 40000, 2048) > L.dsi_topk_workspace_bytes(8, 40000, 2048)
    # two or more rows per request: the two steps as they are
    assert L.dsi_paged_mqa_topk_decode_workspace_bytes(8, 2, 40000, 2048) == L.dsi_topk_workspace_bytes(16, 40000, 2048)
    assert L.dsi_paged_mqa_topk_decode_workspace_bytes(8, 3, 40000, 2048) == L.dsi_topk_workspace_bytes(24, 40000, 2048)
    assert L.dsi_paged_mqa_topk_decode_workspace_bytes(8, 1, 4000, 2048) == 0
