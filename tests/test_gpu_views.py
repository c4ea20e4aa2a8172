"""Strided views through the C ABI: q, k, v and out as views into larger buffers with
padded head, token and channel strides, in both layouts and every mode.  The output
must equal the output on contiguous tensors bit for bit, and nothing outside the out
view may be written."""
import numpy as np
import pytest
import torch

import quantized_attention_diffusion_amd as sage
from gpu_helpers import require_gpu, random_qkv

pytestmark = pytest.mark.gpu

MODES = [dict(), dict(pv="bf16"), dict(per_token=True), dict(k_block_mean=True),
         dict(pv="bf16", per_token=True), "sparse"]
CASES = [  # (B, H, N, d, mode index, layout, paddings (token, head, channel) in elements)
    (1, 3, 200, 128, 0, "bnhd", (8, 0, 16)),
    (2, 2, 777, 64, 1, "bhnd", (16, 8, 8)),
    (1, 1, 1, 128, 2, "bnhd", (8, 8, 8)),
    (2, 3, 1300, 128, 3, "bhnd", (0, 8, 0)),
    (1, 2, 513, 64, 4, "bnhd", (24, 16, 0)),
    (2, 2, 900, 128, 5, "bhnd", (8, 0, 24)),
]


def setup_module(module):
    require_gpu()


def _padded(x, layout, pads, fill=7.0):
    """A view of a larger buffer holding x ([B, N, H, d]); returns (buffer, view in the
    library's layout, the view's region of the buffer as a boolean mask)."""
    B, N, H, d = x.shape
    pn, ph, pd = pads
    if layout == "bnhd":
        buf = torch.full((B, N + pn, H + ph, d + pd), fill, dtype=x.dtype, device=x.device)
        view = buf[:, :N, :H, :d]
        view.copy_(x)
    else:
        buf = torch.full((B, H + ph, N + pn, d + pd), fill, dtype=x.dtype, device=x.device)
        view = buf[:, :H, :N, :d]
        view.copy_(x.transpose(1, 2))
    mask = torch.zeros(buf.shape, dtype=torch.bool, device=x.device)
    mask[:, :view.shape[1], :view.shape[2], :d] = True
    return buf, view, mask


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c[0]}_H{c[1]}_N{c[2]}_d{c[3]}_m{c[4]}_{c[5]}")
def test_padded_views_match_contiguous_and_write_only_the_view(case):
    B, H, N, d, mi, layout, pads = case
    mode = MODES[mi]
    print(f"[views] B={B} H={H} N={N} d={d} mode={mode} {layout} pads={pads}", flush=True)
    q, k, v = (t.cuda() for t in random_qkv(B, N, H, d, seed=900 + mi))

    def run(qa, ka, va, out=None, layout="bnhd"):
        if mode == "sparse":
            return sage.sage_attn_fwd_sparse(qa, ka, va, 0.4, out=out, layout=layout)
        return sage.sage_attn_fwd_ex(qa, ka, va, out=out, layout=layout, **mode)

    want = run(q, k, v)
    views = [_padded(t, layout, pads)[1] for t in (q, k, v)]
    obuf, oview, omask = _padded(torch.zeros_like(q), layout, pads)
    before = obuf.clone()
    run(*views, out=oview, layout=layout)
    torch.cuda.synchronize()
    got = oview if layout == "bnhd" else oview.transpose(1, 2)
    assert torch.equal(got.contiguous().view(torch.int16), want.view(torch.int16))
    assert torch.equal(obuf[~omask], before[~omask]), "bytes outside the out view were written"
    assert np.isfinite(got.float().cpu().numpy()).all()
