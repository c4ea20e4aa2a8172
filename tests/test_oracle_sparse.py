"""Pins of the oracle's block-sparse tile selection and of the pipeline restricted to
the kept tiles: the importance against the brute-force mean of the dequantised logit
block, the keep count's closed form, the selection's order and tie rule, a planted
structure that the selection must find, and the reduction of the sparse pipeline to the
dense one (all tiles kept; kept tiles gathered into a shorter key sequence)."""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import attention_exact, attention_pipeline, rel_l2, select_tiles, tile_importance

F32 = np.float32


def _qkv(B, N, H, d, seed, kbias=0.0):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, N, H, d, generator=g).to(torch.bfloat16).float().numpy()
    k = (torch.randn(B, N, H, d, generator=g) + kbias).to(torch.bfloat16).float().numpy()
    v = torch.randn(B, N, H, d, generator=g).to(torch.bfloat16).float().numpy()
    return q, k, v


def test_importance_is_mean_dequantised_logit():
    # ragged: N = 300 gives tiles of 128, 128, 44 keys and a half-empty last scale block
    q, k, v = _qkv(1, 300, 2, 64, seed=11, kbias=1.5)
    quant = oracle.quantize(q, k, v)
    imp = tile_importance(quant)
    N, T = 300, 128
    nt = -(-N // T)
    assert imp.shape == (1, 2, nt, nt)
    for h in range(2):
        S = oracle.qk_int32(quant["q_i8"][0, h], quant["k_i8"][0, h]).astype(np.float64)
        qs = quant["q_scale"][0, h][np.arange(N) // 64].astype(np.float64)
        ks = quant["k_scale"][0, h][np.arange(N) // 64].astype(np.float64)
        deq = qs[:, None] * ks[None, :] * S
        for I in range(nt):
            for J in range(nt):
                want = deq[I * T:(I + 1) * T, J * T:(J + 1) * T].mean()
                assert abs(imp[0, h, I, J] - want) <= 1e-12 * max(1.0, abs(want)), (h, I, J)


def test_keep_count_closed_form():
    assert oracle.keep_count(1.0, 36) == 36
    assert oracle.keep_count(4.0, 36) == 36
    assert oracle.keep_count(0.5, 36) == 18
    assert oracle.keep_count(0.01, 36) == 1
    assert oracle.keep_count(0.25, 512) == 128
    # tau is an fp32 value: fp32(0.3) * 10 = 3.0000001..., so 4 of 10 tiles are kept
    assert oracle.keep_count(0.3, 10) == 4
    for bad in (0.0, -0.5, float("nan")):
        with pytest.raises(ValueError):
            oracle.keep_count(bad, 10)


@pytest.mark.parametrize("density", [0.05, 0.4, 0.75])
def test_selection_keeps_the_most_important_tiles(density):
    q, k, v = _qkv(1, 1000, 1, 128, seed=3, kbias=3.0)
    quant = oracle.quantize(q, k, v)
    imp = tile_importance(quant)
    counts, tiles = select_tiles(quant, density)
    nt = imp.shape[-1]
    k_keep = max(1, min(nt, math.ceil(float(F32(density)) * nt)))
    for I in range(nt):
        sel = tiles[0][0][I]
        assert counts[0, 0, I] == k_keep == len(sel)
        assert sel == sorted(sel) and len(set(sel)) == len(sel)
        rest = [J for J in range(nt) if J not in sel]
        if rest:
            assert min(imp[0, 0, I, sel]) >= max(imp[0, 0, I, rest])


def test_selection_ties_prefer_lower_tiles():
    # every key tile holds the same 128 keys: all importances of a query block are equal
    q, k, v = _qkv(1, 512, 1, 64, seed=5)
    k = np.tile(k[:, :128], (1, 4, 1, 1))
    quant = oracle.quantize(q, k, v)
    imp = tile_importance(quant)
    assert np.all(imp == imp[..., :1])
    _, tiles = select_tiles(quant, 0.5)
    assert all(tiles[0][0][I] == [0, 1] for I in range(4))


def test_selection_finds_a_planted_tile():
    # query block I is aligned with the direction of key tile perm[I] only
    rng = np.random.default_rng(7)
    N, d, T = 1024, 64, 128
    nt = N // T
    dirs = np.linalg.qr(rng.standard_normal((d, d)))[0][:nt] * 4.0
    perm = rng.permutation(nt)
    q = np.zeros((1, N, 1, d), dtype=F32)
    k = np.zeros((1, N, 1, d), dtype=F32)
    for I in range(nt):
        q[0, I * T:(I + 1) * T, 0] = dirs[I] + 0.3 * rng.standard_normal((T, d))
        k[0, perm[I] * T:(perm[I] + 1) * T, 0] = dirs[I] + 0.3 * rng.standard_normal((T, d))
    q = oracle.bf16_round(q)
    k = oracle.bf16_round(k)
    v = oracle.bf16_round(rng.standard_normal((1, N, 1, d)).astype(F32))
    _, tiles = select_tiles(oracle.quantize(q, k, v), 1.0 / nt)
    assert [tiles[0][0][I] for I in range(nt)] == [[int(perm[I])] for I in range(nt)]


def test_sparse_pipeline_with_every_tile_is_dense():
    q, k, v = _qkv(1, 700, 2, 64, seed=9, kbias=2.0)
    quant = oracle.quantize(q, k, v)
    nt = -(-700 // 128)
    every = [[list(range(nt)) for _ in range(nt)] for _ in range(2)]
    a = attention_pipeline(q, k, v, quant=quant)
    b = attention_pipeline(q, k, v, quant=quant, tiles=[every])
    assert np.array_equal(a, b)


@pytest.mark.parametrize("density", [0.3, 0.6])
def test_sparse_pipeline_is_dense_on_the_gathered_keys(density):
    N, H, d, T = 700, 2, 64, 128
    q, k, v = _qkv(1, N, H, d, seed=21, kbias=2.0)
    quant = oracle.quantize(q, k, v)
    _, tiles = select_tiles(quant, density)
    nt = -(-N // T)
    for h in range(H):
        for I in range(nt):
            sel = tiles[0][h][I]
            rows_k = np.concatenate([np.arange(J * T, min(N, (J + 1) * T)) for J in sel])
            blocks = np.concatenate([np.arange(2 * J, min(-(-N // 64), 2 * J + 2)) for J in sel])
            g = dict(quant)
            g["k_i8"] = quant["k_i8"][:, :, rows_k]
            g["v_f8"] = quant["v_f8"][:, :, rows_k]
            g["k_scale"] = quant["k_scale"][:, :, blocks]
            rows = np.arange(I * T, min(N, (I + 1) * T))
            sparse = attention_pipeline(q, k, v, quant=quant, rows=rows, tiles=tiles)[:, :, h]
            dense = attention_pipeline(q, k, v, quant=g, rows=rows)[:, :, h]
            assert np.array_equal(sparse, dense), (h, I, sel)


def test_sparse_error_falls_as_density_rises():
    q, k, v = _qkv(1, 1024, 1, 64, seed=13, kbias=2.0)
    quant = oracle.quantize(q, k, v)
    exact = attention_exact(q, k, v)
    errs = []
    for density in (0.25, 0.5, 0.75, 1.0):
        _, tiles = select_tiles(quant, density)
        errs.append(rel_l2(attention_pipeline(q, k, v, quant=quant, tiles=tiles), exact))
    assert errs == sorted(errs, reverse=True)
    assert errs[-1] == rel_l2(attention_pipeline(q, k, v, quant=quant), exact)
