"""The entry points allocate and synchronise nothing, so a HIP graph can capture them:
a captured dense step, a captured quality-mode step (bf16 P.V, per-token scales) and a
captured block-sparse step, replayed several times with eager work and
synchronisations in between, reproduce the eager outputs bit for bit."""
import pytest
import torch

import quantized_attention_diffusion_amd as sage
from gpu_helpers import require_gpu, random_qkv

pytestmark = pytest.mark.gpu


def setup_module(module):
    require_gpu()


@pytest.mark.parametrize("kind", ["dense", "quality", "sparse"])
def test_captured_step_replays_match_eager(kind):
    B, N, H, d = 1, 1000, 2, 128
    q, k, v = (t.cuda() for t in random_qkv(B, N, H, d, 31, 2))
    if kind == "sparse":
        nbytes = sage.sage_workspace_bytes_sparse(B, H, N, d)
    elif kind == "quality":
        nbytes = sage.sage_workspace_bytes_ex(B, H, N, d, sage.mode_bits("bf16", per_token=True))
    else:
        nbytes = sage.sage_workspace_bytes(B, H, N, d)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)

    def step():
        if kind == "sparse":
            sage.sage_attn_fwd_sparse(q, k, v, 0.5, out=out, workspace=ws)
        elif kind == "quality":
            sage.sage_attn_fwd_ex(q, k, v, out=out, workspace=ws, pv="bf16", per_token=True)
        else:
            sage.sage_attn_fwd(q, k, v, out=out, workspace=ws)

    step()
    torch.cuda.synchronize()
    eager = out.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # warm-up on the capture stream, as torch advises
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for i in range(3):
        out.zero_()
        ws.fill_(0x5a)                      # the captured step must not depend on old workspace contents
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {i}"
        step()                              # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"eager after replay {i}"
