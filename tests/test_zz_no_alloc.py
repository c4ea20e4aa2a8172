"""GPU test of sage_attn_fwd_noalloc (the entry point that allocates nothing and keeps
its workspace in the library's device array), through the C ABI: its output must be
bit-identical to sage_attn_fwd's on the same inputs, on two calls in a row of which the
second is smaller, so the second runs on what the first left in the array."""
import pytest
import torch

import quantized_attention_diffusion_amd as sage
from gpu_helpers import require_gpu, random_qkv

pytestmark = pytest.mark.gpu


def setup_module(module):
    require_gpu()


def _same(a, b):
    return torch.equal(a.contiguous().view(torch.int16), b.contiguous().view(torch.int16))


def test_noalloc_matches_sage_attn_fwd_on_two_calls():
    # first the Flux-like shape (43 MiB of workspace), then a smaller, ragged one
    for (B, N, H, d, seed) in [(1, 4608, 24, 128, 51), (2, 1000, 3, 64, 52)]:
        print(f"[noalloc] B={B} N={N} H={H} d={d}", flush=True)
        q, k, v = (t.cuda() for t in random_qkv(B, N, H, d, seed))
        want = sage.sage_attn_fwd(q, k, v)
        out = torch.empty_like(q)
        got = sage.sage_attn_fwd_noalloc(q, k, v, out)
        torch.cuda.synchronize()
        assert got.data_ptr() == out.data_ptr()
        assert _same(got, want), f"noalloc output differs for B={B} N={N} H={H} d={d}"
        assert torch.isfinite(got.float()).all()


def test_noalloc_strided_views_and_sm_scale():
    # fused-qkv slices and an explicit sm_scale, against the workspace entry point
    q, k, v = random_qkv(1, 300, 3, 128, 53)
    qkv = torch.stack([q, k, v], dim=2).cuda()
    want = sage.sage_attn_fwd(qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2], sm_scale=0.07)
    out = torch.empty(1, 300, 3, 128, dtype=torch.bfloat16, device="cuda")
    got = sage.sage_attn_fwd_noalloc(qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2], out, sm_scale=0.07)
    torch.cuda.synchronize()
    assert _same(got, want)


def test_noalloc_step_captured_in_a_graph():
    # the callers this entry point is for capture it in a HIP graph: replays, with eager
    # calls and synchronisations between them, give the eager output bit for bit
    q, k, v = (t.cuda() for t in random_qkv(1, 1000, 2, 128, 54, 2))
    out = torch.empty_like(q)
    sage.sage_attn_fwd_noalloc(q, k, v, out)
    torch.cuda.synchronize()
    eager = out.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        sage.sage_attn_fwd_noalloc(q, k, v, out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sage.sage_attn_fwd_noalloc(q, k, v, out)
    for i in range(3):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert _same(out, eager), f"replay {i}"
        sage.sage_attn_fwd_noalloc(q, k, v, out)
        torch.cuda.synchronize()
        assert _same(out, eager), f"eager after replay {i}"


def test_noalloc_rejects_a_shape_beyond_its_array():
    q, k, v = (torch.zeros(1, 8192, 24, 128, dtype=torch.bfloat16, device="cuda") for _ in range(3))
    with pytest.raises(sage.SageError, match="no-allocation"):
        sage.sage_attn_fwd_noalloc(q, k, v, torch.empty_like(q))
