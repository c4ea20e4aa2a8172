"""GPU parity of the block-sparse path (kept key tiles per query block) against the
oracle, through the C ABI: the fp64 tile importances and the kept-tile lists
bit-exact, the attention over the kept tiles within the max-abs bound of the oracle's
pipeline restricted to the same tiles, density 1 identical to the dense kernel, and
the full-size workloads on sampled heads and rows."""
import numpy as np
import pytest
import torch

import oracle
import workloads
import quantized_attention_diffusion_amd as sage
from gpu_helpers import require_gpu, to_np, random_qkv, check_oracle

pytestmark = pytest.mark.gpu

CASES = [  # (B, N, H, d, seed, outliers)
    (1, 1, 1, 128, 1, 0),       # one tile of one key
    (1, 129, 2, 64, 6, 0),      # last tile of one key
    (1, 256, 2, 64, 0, 0),      # the 'tiny' workload shape: 2 tiles
    (1, 1000, 2, 128, 8, 4),    # ragged last tile of 104 keys, outlier channels
    (2, 700, 3, 64, 3, 0),      # last tile of 60 keys; its second scale block lies past N
    (1, 1100, 2, 64, 9, 0),
    (1, 2048, 1, 128, 11, 0),   # 16 tiles
]
DENSITIES = [0.05, 0.3, 0.5, 1.0]


def _case_id(c):
    return "B{}_N{}_H{}_d{}".format(*c[:4])


def _np(t):
    return t.float().numpy()


def setup_module(module):
    require_gpu()
    info = sage.sage_kernel_info()
    assert info["kv_tile"] == oracle.SPARSE_TILE and info["block_m"] == oracle.SPARSE_TILE


def _check_selection(cnt, lst, imp, ref, density, heads=None, label=""):
    """GPU tile_count/tile_list/importance of (all or some) heads against the oracle."""
    B, H = cnt.shape[:2]
    heads = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    cnt, lst, imp = cnt.cpu().numpy(), lst.cpu().numpy(), imp.cpu().numpy()
    for (b, h) in heads:
        sub = {key: (val[b:b + 1, h:h + 1] if isinstance(val, np.ndarray) and val.ndim >= 2 else val)
               for key, val in ref.items()}
        want_imp = oracle.tile_importance(sub)[0, 0]
        got_imp = imp[b, h]
        assert np.array_equal(got_imp.view(np.int64), want_imp.view(np.int64)), \
            f"{label} head {(b, h)}: importance differs at {np.argwhere(got_imp != want_imp)[:4].tolist()}"
        counts, tiles = oracle.select_tiles(sub, density)
        for I, want in enumerate(tiles[0][0]):
            k = int(cnt[b, h, I])
            assert k == counts[0, 0, I] == len(want), f"{label} head {(b, h)} block {I}: count {k}"
            assert lst[b, h, I, :k].tolist() == want, f"{label} head {(b, h)} block {I}: tiles differ"


@pytest.mark.parametrize("density", DENSITIES)
@pytest.mark.parametrize("case", CASES, ids=_case_id)
def test_tile_selection_bit_exact(case, density):
    B, N, H, d, seed, outl = case
    print(f"[select] {_case_id(case)} density={density}", flush=True)
    q, k, v = random_qkv(B, N, H, d, seed, outl)
    gq = sage.sage_quant_qk(q.cuda(), k.cuda(), v.cuda())
    cnt, lst, imp = sage.sage_block_select(gq, density, return_importance=True)
    torch.cuda.synchronize()
    ref = oracle.quantize(_np(q), _np(k), _np(v))
    _check_selection(cnt, lst, imp, ref, density, label=_case_id(case))


@pytest.mark.parametrize("density", DENSITIES[:3])
@pytest.mark.parametrize("case", CASES, ids=_case_id)
def test_sparse_attention_matches_oracle_pipeline(case, density):
    B, N, H, d, seed, outl = case
    print(f"[sparse attn] {_case_id(case)} density={density}", flush=True)
    q, k, v = random_qkv(B, N, H, d, seed, outl)
    out = sage.sage_attn_fwd_sparse(q.cuda(), k.cuda(), v.cuda(), density)
    o = to_np(out)
    ref = oracle.quantize(_np(q), _np(k), _np(v))
    _, tiles = oracle.select_tiles(ref, density)
    err, _, _ = check_oracle(o, f"{_case_id(case)} density {density}", _np(q), _np(k), _np(v),
                             quant=ref, tiles=tiles)
    print(f"    max|gpu-pipe| = {err:.2e}", flush=True)


@pytest.mark.parametrize("case", CASES, ids=_case_id)
def test_full_density_is_the_dense_kernel(case):
    B, N, H, d, seed, outl = case
    q, k, v = (t.cuda() for t in random_qkv(B, N, H, d, seed, outl))
    dense = sage.sage_attn_fwd(q, k, v)
    for density in (1.0, 4.0):
        sparse = sage.sage_attn_fwd_sparse(q, k, v, density)
        assert torch.equal(sparse.view(torch.int16), dense.view(torch.int16)), density


def test_sparse_layouts_and_workspace_reuse():
    q, k, v = random_qkv(1, 1000, 2, 128, 21, 0)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    ref = sage.sage_attn_fwd_sparse(qd, kd, vd, 0.4)
    # [B, H, N, d] views of the same data, and one workspace used twice
    qh, kh, vh = (t.transpose(1, 2) for t in (qd, kd, vd))
    ws = torch.empty(sage.sage_workspace_bytes_sparse(1, 2, 1000, 128), dtype=torch.uint8, device="cuda")
    for _ in range(2):
        o = sage.sage_attn_fwd_sparse(qh, kh, vh, 0.4, layout="bhnd", workspace=ws)
        assert torch.equal(o.transpose(1, 2).contiguous().view(torch.int16), ref.view(torch.int16))
    # strided q/k/v slices of one fused [B, N, 3, H, d] projection output
    qkv = torch.stack([qd, kd, vd], dim=2).contiguous()
    o = sage.sage_attn_fwd_sparse(qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2], 0.4)
    assert torch.equal(o.view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("kind", ["random", "equal_tiles", "zero_q"])
@pytest.mark.parametrize("N,d,density", [(129 * 128, 64, 0.3), (200 * 128 - 77, 128, 0.05)],
                         ids=["nt129", "nt200"])
def test_selection_above_the_rank_limit(N, d, density, kind):
    # more than 128 key tiles per head: the radix selection.  equal_tiles: every key
    # tile holds the same keys, so each query block's importances tie and the lowest
    # tiles must be kept; zero_q: all importances are signed zeros, equal in fp64.
    print(f"[select radix] N={N} d={d} density={density} {kind}", flush=True)
    q, k, v = random_qkv(1, N, 2, d, seed=31, outliers=0)
    if kind == "equal_tiles":
        reps = -(-N // 128)
        k = k[:, :128].repeat(1, reps, 1, 1)[:, :N].contiguous()
    elif kind == "zero_q":
        q = torch.zeros_like(q)
    gq = sage.sage_quant_qk(q.cuda(), k.cuda(), v.cuda())
    cnt, lst, imp = sage.sage_block_select(gq, density, return_importance=True)
    torch.cuda.synchronize()
    ref = oracle.quantize(_np(q), _np(k), _np(v))
    _check_selection(cnt, lst, imp, ref, density, label=f"radix {kind}")
    if kind == "zero_q" or (kind == "equal_tiles" and N % 128 == 0):   # a ragged last tile differs
        keep = oracle.keep_count(density, -(-N // 128))
        assert (lst[..., :keep].cpu() == torch.arange(keep, dtype=torch.int32)).all()


@pytest.mark.parametrize("name,density,n_heads", [("flux_like", 0.3, 24), ("stress", 0.25, 2)])
def test_full_size_sparse(name, density, n_heads):
    w = workloads.get(name)
    print(f"[sparse full] {name} B={w.B} H={w.H} N={w.N} d={w.d} density={density}", flush=True)
    q, k, v = workloads.make_qkv(w)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    out = sage.sage_attn_fwd_sparse(qd, kd, vd, density)
    gq = sage.sage_quant_qk(qd, kd, vd)
    cnt, lst, imp = sage.sage_block_select(gq, density, return_importance=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(99)
    heads = list(range(w.H)) if n_heads >= w.H else sorted({0, w.H - 1, *rng.choice(w.H, n_heads, replace=False).tolist()})[:n_heads]
    N = w.N
    for h in heads:
        qh, kh, vh = (t[:, :, h:h + 1, :].float().numpy() for t in (q, k, v))
        ref = oracle.quantize(qh, kh, vh)
        one = (cnt[:, h:h + 1], lst[:, h:h + 1], imp[:, h:h + 1])
        _check_selection(*one, ref, density, label=f"{name} head {h}")
        if h in heads[:2]:
            _, tiles = oracle.select_tiles(ref, density)
            rows = np.unique(np.concatenate([[0, N - 1], rng.choice(N, size=24, replace=False)]))
            err, _, _ = check_oracle(to_np(out[:, rows, h:h + 1, :]), f"{name} head {h}", qh, kh, vh,
                                     quant=ref, rows=rows, tiles=tiles)
            print(f"    head {h}: max|gpu-pipe| = {err:.2e}", flush=True)


def test_sparse_with_a_given_sm_scale():
    q, k, v = random_qkv(1, 700, 2, 64, 41, 0)
    sm = 0.05
    out = sage.sage_attn_fwd_sparse(q.cuda(), k.cuda(), v.cuda(), 0.5, sm_scale=sm)
    ref = oracle.quantize(_np(q), _np(k), _np(v))
    _, tiles = oracle.select_tiles(ref, 0.5)      # the selection does not depend on sm_scale
    check_oracle(to_np(out), "sparse sm_scale 0.05", _np(q), _np(k), _np(v), sm_scale=sm, quant=ref,
                 tiles=tiles)
