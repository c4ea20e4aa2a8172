"""Ragged last key tiles against the CPU oracle, for every attention body: tail lengths
on each side of every boundary of the lane layouts (16-key register runs, the 32-key
halves a lane pair splits, the 64-key scale blocks), dense and block-sparse."""
import numpy as np
import pytest
import torch

import oracle
import quantized_attention_diffusion_amd as sage
from gpu_helpers import require_gpu, to_np, random_qkv, check_oracle

pytestmark = pytest.mark.gpu

KV_TILE = 128
TAILS = [2, 15, 16, 17, 31, 32, 33, 47, 48, 63, 64, 95, 96, 97, 111, 112, 113, 126, 127]

# (d, pv, per_token, k_block_mean): the 32x32 body (d = 128, mode 0) and the 16x16 ones
BODIES = {
    "d128_fp8": (128, "fp8", False, False),
    "d128_fp8_tok": (128, "fp8", True, False),
    "d128_fp8_kbm": (128, "fp8", False, True),
    "d128_bf16": (128, "bf16", False, False),
    "d64_fp8": (64, "fp8", False, False),
}


def _np(t):
    return t.float().numpy()


def setup_module(module):
    require_gpu()
    assert sage.sage_kernel_info()["kv_tile"] == KV_TILE


@pytest.mark.parametrize("tail", TAILS)
@pytest.mark.parametrize("body", list(BODIES))
def test_ragged_last_tile(body, tail):
    d, pv, tok, kbm = BODIES[body]
    N = 2 * KV_TILE + tail                       # two full tiles, then the ragged one
    print(f"[tail] {body} N={N}", flush=True)
    q, k, v = random_qkv(1, N, 2, d, seed=1000 + tail, outliers=1)
    out = sage.sage_attn_fwd_ex(q.cuda(), k.cuda(), v.cuda(), pv=pv, per_token=tok, k_block_mean=kbm)
    o = to_np(out)
    assert np.isfinite(o).all()
    ref = oracle.quantize(_np(q), _np(k), _np(v), block=1 if tok else 64, k_block_mean=kbm)
    kw = dict(kv_tile=KV_TILE, quant=ref)
    if pv == "bf16":
        kw.update(fp8_p=False, bf16_p=True, fp8_v=False)
    check_oracle(o, f"{body} N={N}", _np(q), _np(k), _np(v), **kw)


@pytest.mark.parametrize("tail", [2, 31, 32, 33, 63, 64, 95, 96, 127])
@pytest.mark.parametrize("d", [64, 128])
def test_ragged_last_tile_sparse(d, tail):
    """Block-sparse steps over 5 key tiles whose last is ragged, at a density that keeps
    3 of them: the masked tile is visited when it is kept and skipped otherwise."""
    N = 4 * KV_TILE + tail
    print(f"[tail sparse] d={d} N={N}", flush=True)
    q, k, v = random_qkv(1, N, 2, d, seed=2000 + tail, outliers=0)
    qc, kc, vc = q.cuda(), k.cuda(), v.cuda()
    density = 0.5
    out = sage.sage_attn_fwd_sparse(qc, kc, vc, density)
    o = to_np(out)
    ref = oracle.quantize(_np(q), _np(k), _np(v))
    gq = sage.sage_quant_qk(qc, kc, vc)
    cnt, lst = sage.sage_block_select(gq, density)
    torch.cuda.synchronize()
    cnt, lst = cnt.cpu().numpy(), lst.cpu().numpy()
    # the kept-tile lists are the oracle's (the decisions are exact), and the output is
    # the oracle pipeline restricted to them
    counts, tiles = oracle.select_tiles(ref, density)
    last_kept = 0
    for h in range(2):
        for I, want in enumerate(tiles[0][h]):
            n = int(cnt[0, h, I])
            assert n == counts[0, h, I] == len(want) == 3
            assert lst[0, h, I, :n].tolist() == want, (h, I)
            last_kept += int(4 in want)
    print(f"    query blocks keeping the ragged tile: {last_kept} of {2 * len(tiles[0][0])}", flush=True)
    check_oracle(o, f"sparse d={d} N={N}", _np(q), _np(k), _np(v), kv_tile=KV_TILE, quant=ref, tiles=tiles)
