"""dsi_topk_select_noalloc, the top-k for callers that cannot allocate: through the C ABI its output equals
dsi_topk_select's (with a caller workspace) on the same logits, on two calls in a row whose second is
smaller (the scratch array keeps the first call's contents), and sizes beyond its array are refused on the
host before any HIP call."""
import ctypes

import numpy as np
import pytest
import torch

import sparse_attention_token_amd as dsi

K = 2048
EWORKSPACE = -5


def test_too_large_is_refused_on_the_host():
    lib = dsi.lib()
    rows, width = 511, 20000  # split path: its workspace exceeds the array
    assert dsi.topk_workspace_bytes(rows, width, K) > (16 << 20)
    fake = ctypes.c_void_p(0x10000)  # never dereferenced: the call returns before any HIP call
    assert lib.dsi_topk_select_noalloc(fake, 0, width, rows, None, fake, width, K, fake, K, None) == EWORKSPACE


def _distinct_logits(rng, rows, width):
    # distinct values per row (a permutation of a fixed grid), so the top-k set is unique
    base = np.linspace(-50.0, 50.0, width, dtype=np.float32)
    return np.stack([base[rng.permutation(width)] for _ in range(rows)])


@pytest.mark.gpu
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_noalloc_matches_workspace_call_twice(dtype):
    rng = np.random.default_rng(11)
    shapes = [(64, 65536), (24, 30000)]  # both on the split path (few long rows); the second call is smaller
    for rows, width in shapes:
        x = _distinct_logits(rng, rows, width)
        ends = rng.integers(1, width + 1, size=rows).astype(np.int32)
        ends[:4] = [width, 1, K - 1, K]  # full row, one column, fewer than k, exactly k
        if dtype == "bf16":
            bits = (torch.from_numpy(x).to(torch.bfloat16).view(torch.int16)).cuda()
            logits = bits
        else:
            logits = torch.from_numpy(x).cuda()
        assert dsi.topk_workspace_bytes(rows, width, K) > 0, "expected the split path"
        ends_t = torch.from_numpy(ends).cuda()
        ref = dsi.topk_select(logits, ends_t, k=K)
        out = torch.full((rows, K), -7, dtype=torch.int32, device="cuda")
        dsi.topk_select_noalloc(logits, ends_t, out, k=K)
        got, exp = out.cpu().numpy(), ref.cpu().numpy()
        for r in range(rows):
            n = min(K, int(ends[r]))
            if dtype == "bf16":  # equal bf16 values may tie at the boundary: compare the selected values
                v = logits[r].cpu().view(torch.bfloat16).float().numpy()
                assert np.array_equal(np.sort(v[got[r][:n]]), np.sort(v[exp[r][:n]])), (rows, r)
            else:
                assert np.array_equal(np.sort(got[r][:n]), np.sort(exp[r][:n])), (rows, r)
            assert np.all(got[r][n:] == -1) and np.all(got[r][:n] >= 0)
