"""Randomised GPU parity sweep against the CPU oracle: a fixed, seeded list of shapes
(batch, heads, ragged lengths), head sizes, layouts (including fused-qkv slices),
softmax scales, modes and block-sparse densities, each checked against both oracle
readings, so that combinations no hand-written case names still meet the bound."""
import numpy as np
import pytest
import torch

import oracle
import quantized_attention_diffusion_amd as sage
from gpu_helpers import require_gpu, to_np, random_qkv, check_oracle

pytestmark = pytest.mark.gpu

KV_TILE = 128
MODES = [  # (pv, per_token, k_block_mean); "sparse": the block-sparse step
    ("fp8", False, False), ("fp8", True, False), ("fp8", False, True), ("fp8", True, True),
    ("bf16", False, False), ("bf16", True, False), ("sparse", False, False),
]


def _cases(n=48, seed=20261203):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        B = int(rng.integers(1, 3))
        H = int(rng.integers(1, 4))
        N = int(rng.integers(1, 1700))
        d = int(rng.choice([64, 128]))
        mode = MODES[int(rng.integers(len(MODES)))]
        layout = str(rng.choice(["bnhd", "bhnd", "fused"]))
        outl = int(rng.choice([0, 0, 2, 4]))
        sm = float(rng.choice([0.0, 0.05, 0.2, 0.3]))   # 0: the default 1/sqrt(d)
        dens = float(rng.choice([0.1, 0.3, 0.6]))       # block-sparse steps only
        out.append((i, B, H, N, d, mode, layout, outl, sm, dens))
    return out


CASES = _cases()


def _np(t):
    return t.float().numpy()


def setup_module(module):
    require_gpu()
    assert sage.sage_kernel_info()["kv_tile"] == KV_TILE


@pytest.mark.parametrize("case", CASES, ids=lambda c: "r{}_B{}_H{}_N{}_d{}_{}{}{}_{}".format(
    c[0], c[1], c[2], c[3], c[4], c[5][0], "_tok" if c[5][1] else "", "_kbm" if c[5][2] else "", c[6]))
def test_random_case_matches_oracle(case):
    i, B, H, N, d, (pv, tok, kbm), layout, outl, sm, dens = case
    print(f"[random] case {i}: B={B} H={H} N={N} d={d} pv={pv} tok={tok} kbm={kbm} {layout} "
          f"outliers={outl} sm={sm}" + (f" density={dens}" if pv == "sparse" else ""), flush=True)
    q, k, v = random_qkv(B, N, H, d, seed=5000 + i, outliers=outl)
    sm_scale = sm if sm > 0 else None
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    call_layout = layout
    if layout == "bhnd":
        qd, kd, vd = (t.transpose(1, 2).contiguous() for t in (qd, kd, vd))
    elif layout == "fused":                     # strided slices of one [B, N, 3, H, d] tensor
        qkv = torch.stack([qd, kd, vd], dim=2)
        qd, kd, vd = qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2]
        call_layout = "bnhd"
    if pv == "sparse":
        out = sage.sage_attn_fwd_sparse(qd, kd, vd, dens, sm_scale=sm_scale, layout=call_layout)
    else:
        out = sage.sage_attn_fwd_ex(qd, kd, vd, sm_scale=sm_scale, layout=call_layout, pv=pv, per_token=tok,
                                    k_block_mean=kbm)
    if layout == "bhnd":
        out = out.transpose(1, 2)
    o = to_np(out)
    assert np.isfinite(o).all()
    ref = oracle.quantize(_np(q), _np(k), _np(v), block=1 if tok else 64, k_block_mean=kbm)
    kw = dict(kv_tile=KV_TILE, quant=ref, sm_scale=sm_scale)
    if pv == "bf16":
        kw.update(fp8_p=False, bf16_p=True, fp8_v=False)
    if pv == "sparse":
        kw["tiles"] = oracle.select_tiles(ref, dens)[1]
    err, err32, _ = check_oracle(o, f"random case {i}", _np(q), _np(k), _np(v), **kw)
    print(f"    max|gpu-pipe| = {err:.2e} (fp32 reading {err32:.2e})", flush=True)
