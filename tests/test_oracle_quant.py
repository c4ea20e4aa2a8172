"""Pins of the oracle's quantisation steps: bf16 rounding, the K token mean, the INT8
block codes and the FP8 V codes."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle import (QUANT_BLOCK, bf16_round, k_token_mean, quantize_int8_blocks,
                    quantize_v_fp8, e4m3_decode, e4m3_table)

F32 = np.float32


def _bf16_values(shape, seed, scale=1.0, shift=0.0):
    g = torch.Generator().manual_seed(seed)
    t = (torch.randn(shape, generator=g) * scale + shift).to(torch.bfloat16)
    return t.float().numpy()


# ---------------------------------------------------------------- bf16 rounding
def test_bf16_round_matches_torch_cast():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(100000) * 10.0 ** rng.integers(-6, 6, 100000),
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8),
                                  65504.0, 1e-38, 0.0, -0.0])]).astype(F32)
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    got = bf16_round(x)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


# ---------------------------------------------------------------- K token mean
def _f32_rne_of_fraction(fr: Fraction) -> np.float32:
    """Correctly rounded fp32 of an exact rational (ties to even)."""
    approx = np.float32(float(fr))
    cands = [np.nextafter(approx, F32(-np.inf)), approx, np.nextafter(approx, F32(np.inf))]
    dists = [abs(Fraction(float(c)) - fr) for c in cands]
    best = min(dists)
    winners = [c for c, dd in zip(cands, dists) if dd == best]
    if len(winners) == 1:
        return winners[0]
    return [c for c in winners if np.array([c], F32).view(np.uint32)[0] % 2 == 0][0]


def test_k_mean_equals_exact_rational_mean_rounded():
    k = _bf16_values((2, 37, 3, 8), seed=2, scale=1.0, shift=2.5)
    mu = k_token_mean(k)
    for b in range(2):
        for h in range(3):
            for c in range(8):
                exact = sum(Fraction(float(x)) for x in k[b, :, h, c]) / 37
                want = bf16_round(np.array([_f32_rne_of_fraction(exact)], F32))[0]
                assert mu[b, h, c] == want


def test_k_block_means_equal_exact_rational_means_rounded():
    from oracle.quant import k_block_means
    k = _bf16_values((1, 150, 2, 4), seed=12, scale=1.0, shift=1.5)
    mu = k_block_means(k)
    assert mu.shape == (1, 2, 3, 4)
    for h in range(2):
        for j, (r0, r1) in enumerate([(0, 64), (64, 128), (128, 150)]):
            for c in range(4):
                exact = sum(Fraction(float(x)) for x in k[0, r0:r1, h, c]) / (r1 - r0)
                want = bf16_round(np.array([_f32_rne_of_fraction(exact)], F32))[0]
                assert mu[0, h, j, c] == want


def test_k_mean_is_bitwise_permutation_invariant():
    k = _bf16_values((1, 301, 2, 16), seed=3, scale=1.0, shift=-4.0)
    perm = np.random.default_rng(0).permutation(301)
    assert np.array_equal(k_token_mean(k), k_token_mean(k[:, perm]))


# ---------------------------------------------------------------- INT8 blocks
def _rne(y: float) -> int:
    f = int(np.floor(y))
    r = y - f
    if r > 0.5 or (r == 0.5 and f % 2 == 1):
        return f + 1
    return f


def _int8_bruteforce(x, block=QUANT_BLOCK):
    """Scalar loops over blocks and elements (x: [N, d] float32 of one head)."""
    N, d = x.shape
    codes = np.zeros((N, d), np.int8)
    scales = []
    for b0 in range(0, N, block):
        rows = range(b0, min(N, b0 + block))
        amax = F32(0)
        for i in rows:
            for c in range(d):
                amax = max(amax, abs(x[i, c]))
        if amax == 0:
            scales.append(F32(0))
            continue
        scales.append(F32(amax) / F32(127))
        inv = F32(127) / F32(amax)
        for i in rows:
            for c in range(d):
                codes[i, c] = max(-127, min(127, _rne(float(F32(x[i, c]) * inv))))
    return codes, np.array(scales, F32)


@pytest.mark.parametrize("n", [1, 63, 64, 65, 130])
def test_int8_blocks_equal_scalar_loops(n):
    x = _bf16_values((1, 2, n, 8), seed=n, scale=2.0)
    codes, scales = quantize_int8_blocks(x)
    for h in range(2):
        bc, bs = _int8_bruteforce(x[0, h])
        assert np.array_equal(codes[0, h], bc)
        assert np.array_equal(scales[0, h].view(np.uint32), bs.view(np.uint32))


@pytest.mark.parametrize("n", [1, 5, 70])
def test_int8_per_token_equals_scalar_loops(n):
    # block = 1: every token row has its own scale
    x = _bf16_values((1, 2, n, 16), seed=40 + n, scale=2.0)
    codes, scales = quantize_int8_blocks(x, block=1)
    assert scales.shape == (1, 2, n)
    for h in range(2):
        bc, bs = _int8_bruteforce(x[0, h], block=1)
        assert np.array_equal(codes[0, h], bc)
        assert np.array_equal(scales[0, h].view(np.uint32), bs.view(np.uint32))
        rowmax = np.abs(x[0, h]) == np.abs(x[0, h]).max(axis=1, keepdims=True)
        nz = np.abs(x[0, h]).max(axis=1) > 0
        assert np.all(np.abs(codes[0, h][rowmax & nz[:, None]]) == 127)


def test_int8_amax_element_maps_to_127_and_error_is_half_step():
    x = _bf16_values((2, 3, 200, 64), seed=7, scale=3.0)
    codes, scales = quantize_int8_blocks(x)
    for b0 in range(0, 200, QUANT_BLOCK):
        blk = x[:, :, b0:b0 + QUANT_BLOCK]
        cb = codes[:, :, b0:b0 + QUANT_BLOCK].astype(np.float64)
        s = scales[:, :, b0 // QUANT_BLOCK].astype(np.float64)[:, :, None, None]
        amax_pos = np.abs(blk) == np.abs(blk).max(axis=(2, 3), keepdims=True)
        assert np.all(np.abs(cb[amax_pos]) == 127)
        # half a step, plus the fp32 rounding of inv and scale (< 1e-4 step at |code| <= 127)
        assert np.all(np.abs(cb * s - blk) <= (0.5 + 1e-4) * s)
    assert codes.min() >= -127


def test_int8_ties_round_half_to_even_and_zero_block():
    # amax = 127 gives inv = 1 exactly, so codes are rint of the values themselves
    vals = np.array([0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 126.5, 127.0], F32)
    x = np.zeros((1, 1, 128, 8), F32)
    x[0, 0, 0, :] = vals
    codes, scales = quantize_int8_blocks(x)
    assert list(codes[0, 0, 0]) == [0, 2, 2, 0, -2, -2, 126, 127]
    assert scales[0, 0, 0] == F32(1.0)
    assert scales[0, 0, 1] == 0 and not codes[0, 0, 64:].any()   # all-zero block


def test_int8_tail_block_uses_valid_rows_only():
    x = _bf16_values((1, 1, 70, 4), seed=9)
    codes, scales = quantize_int8_blocks(x)
    assert scales.shape == (1, 1, 2)
    assert scales[0, 0, 1] == F32(np.abs(x[0, 0, 64:]).max()) / F32(127)


# ---------------------------------------------------------------- FP8 V
def test_v_fp8_channel_max_maps_to_448_and_error_bound():
    v = _bf16_values((1, 150, 2, 16), seed=11, scale=1.5)
    codes, scales = quantize_v_fp8(v)
    table = e4m3_table()
    for h in range(2):
        vh = v[0, :, h, :]
        deq = e4m3_decode(codes[0, h]) * scales[0, h][None, :].astype(np.float64)
        for c in range(16):
            j = np.argmax(np.abs(vh[:, c]))
            assert abs(e4m3_decode(codes[0, h, j, c])) == 448.0
        # e4m3 relative spacing is at most 2^-3 (normal range), subnormal step 2^-9
        step = np.maximum(np.abs(deq) * 2.0 ** -3, 2.0 ** -9 * scales[0, h][None, :])
        assert np.all(np.abs(deq - vh) <= 0.5 * step * (1 + 1e-6) + 1e-12)


def test_v_fp8_zero_channel():
    v = _bf16_values((1, 10, 1, 4), seed=12)
    v[:, :, :, 2] = 0
    codes, scales = quantize_v_fp8(v)
    assert scales[0, 0, 2] == 0 and not codes[0, 0, :, 2].any()


def test_quantize_smoothing_removes_channel_bias():
    w = workloads.get("tiny")
    q, k, v = (t.float().numpy() for t in workloads.make_qkv(w))
    qs = oracle.quantize(q, k, v)
    raw = oracle.quantize(q, k, v, smooth_k=False)
    # the bias N(0, 9) dominates K's range; removing it shrinks the K scales
    assert qs["k_scale"].mean() < 0.6 * raw["k_scale"].mean()
    kr = k.transpose(0, 2, 1, 3) - qs["k_mean"][:, :, None, :]
    # what is left of the channel mean is the bf16 rounding of the mean (half an ulp)
    left = np.abs(kr.astype(np.float64).mean(axis=2))
    assert np.all(left <= np.abs(qs["k_mean"]) * 2.0 ** -8 + 1e-6)
