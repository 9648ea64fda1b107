"""w4a16_gemm_noalloc (split partials in the library's fixed device array, no workspace) against
w4a16_gemm (caller workspace), through the C ABI.  The two entry points run the same kernels with
the same plan, so their outputs must be identical bit for bit; the array keeps the previous call's
contents, so two calls in a row are checked, the second on a smaller problem, and one call that
needs no split.  Sizes whose workspace exceeds the array are rejected before anything is enqueued."""
import numpy as np
import pytest
import torch

import exact_tiled_attention_15_amd as eta
from exact_tiled_attention_15_amd import inputs
from tests.gpu_util import say

pytestmark = pytest.mark.gpu

G = eta.W4A16_GROUP


def _upload(d):
    x = torch.from_numpy(d["x"].view(np.int16)).view(torch.float16).cuda()
    packed = torch.from_numpy(d["packed"].view(np.int32)).cuda()
    scales = torch.from_numpy(d["scales"].view(np.int16)).view(torch.float16).cuda()
    zeros = torch.from_numpy(d["zeros"]).cuda()
    return x, packed, scales, zeros


def _both(M, N, K, seed):
    d = inputs.make_w4a16_inputs(M, N, K, G, seed)
    x, packed, scales, zeros = _upload(d)
    nw = eta.w4a16_work_floats(M, N, K)
    work = torch.full((nw,), float("nan"), device="cuda") if nw else None
    y_ref = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")
    y_na = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")
    eta.w4a16_gemm(x, packed, scales, zeros, y_ref, work)
    eta.w4a16_gemm_noalloc(x, packed, scales, zeros, y_na)
    torch.cuda.synchronize()
    return nw, y_ref, y_na


def test_noalloc_matches_workspace_entry_point_two_calls():
    for (M, N, K) in [(16, 8192, 28672), (5, 3000, 16384)]:  # the second call is smaller
        say(f"w4a16_gemm_noalloc M={M} N={N} K={K}")
        nw, y_ref, y_na = _both(M, N, K, 31 + M)
        say(f"  split workspace {nw} floats (array holds {eta.W4A16_NOALLOC_MAX_WORK_FLOATS})")
        assert 0 < nw <= eta.W4A16_NOALLOC_MAX_WORK_FLOATS
        assert not torch.isnan(y_na.float()).any()
        assert torch.equal(y_na.view(torch.int16), y_ref.view(torch.int16))


def test_noalloc_without_split():
    say("w4a16_gemm_noalloc M=16 N=28672 K=8192 (no split)")
    nw, y_ref, y_na = _both(16, 28672, 8192, 77)
    assert nw == 0
    assert torch.equal(y_na.view(torch.int16), y_ref.view(torch.int16))


def test_noalloc_rejects_workspace_beyond_the_array():
    """Checked on the host before any launch: small real buffers stand in for the operands, which
    the call must not touch."""
    M, N, K = 16, 65536, 32768
    nw = eta.w4a16_work_floats(M, N, K)
    say(f"w4a16_gemm_noalloc M={M} N={N} K={K}: workspace {nw} floats > {eta.W4A16_NOALLOC_MAX_WORK_FLOATS}")
    assert nw > eta.W4A16_NOALLOC_MAX_WORK_FLOATS
    buf = torch.full((4096,), float("nan"), dtype=torch.float16, device="cuda")
    p = buf.data_ptr()
    st = eta.lib().w4a16_gemm_noalloc(p, p, p, p, p, M, N, K, G, None)
    assert st == eta.ATTN_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert torch.isnan(buf.float()).all()  # nothing was enqueued
