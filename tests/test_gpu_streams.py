"""Calls on separate streams with separate workspaces share nothing: two streams that
run steps concurrently (different shapes, modes and inputs) reproduce the outputs of
the same calls run one after the other, bit for bit."""
import pytest
import torch

import quantized_attention_diffusion_amd as sage
from gpu_helpers import require_gpu, random_qkv

pytestmark = pytest.mark.gpu


def setup_module(module):
    require_gpu()


def test_concurrent_streams_match_sequential_calls():
    jobs = [  # (B, N, H, d, seed, options)
        (1, 4608, 6, 128, 61, dict()),
        (1, 2000, 4, 64, 62, dict(pv="bf16", per_token=True)),
        (2, 1500, 3, 128, 63, dict(k_block_mean=True)),
    ]
    inputs, wss, want = [], [], []
    for B, N, H, d, seed, opts in jobs:
        q, k, v = (t.cuda() for t in random_qkv(B, N, H, d, seed))
        mode = sage.mode_bits(opts.get("pv", "fp8"), opts.get("per_token", False), opts.get("k_block_mean", False))
        ws = torch.empty(sage.sage_workspace_bytes_ex(B, H, N, d, mode), dtype=torch.uint8, device="cuda")
        inputs.append((q, k, v, opts))
        wss.append(ws)
        want.append(sage.sage_attn_fwd_ex(q, k, v, workspace=ws, **opts))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in jobs]
    outs = [torch.empty_like(x[0]) for x in inputs]
    for rep in range(4):
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        for _ in range(3):                  # several steps per stream, all in flight together
            for s, (q, k, v, opts), ws, o in zip(streams, inputs, wss, outs):
                with torch.cuda.stream(s):
                    sage.sage_attn_fwd_ex(q, k, v, out=o, workspace=ws, **opts)
        torch.cuda.synchronize()
        for j, (o, w) in enumerate(zip(outs, want)):
            assert torch.equal(o.view(torch.int16), w.view(torch.int16)), f"job {j}, repetition {rep}"
