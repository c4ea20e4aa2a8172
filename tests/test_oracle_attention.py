"""Pins of the oracle's attention: exact attention by brute force and invariants, the
quantised pipeline against the exact definition with quantisation switched off, closed
forms, and sanity bounds on the quantisation error."""
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle import attention_exact, attention_pipeline, qk_int32, rel_l2

F32 = np.float32


def _qkv(B, N, H, d, seed, kbias=0.0):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, N, H, d, generator=g).to(torch.bfloat16).float().numpy()
    k = (torch.randn(B, N, H, d, generator=g) + kbias).to(torch.bfloat16).float().numpy()
    v = torch.randn(B, N, H, d, generator=g).to(torch.bfloat16).float().numpy()
    return q, k, v


def _exact_loops(q, k, v, sm):
    """Literal scalar definition with math.fsum, one (b, h) at a time."""
    B, N, H, d = q.shape
    out = np.zeros((B, N, H, d))
    for b in range(B):
        for h in range(H):
            for i in range(N):
                s = [sm * math.fsum(float(q[b, i, h, c]) * float(k[b, j, h, c]) for c in range(d))
                     for j in range(N)]
                mx = max(s)
                e = [math.exp(x - mx) for x in s]
                z = math.fsum(e)
                for c in range(d):
                    out[b, i, h, c] = math.fsum(e[j] * float(v[b, j, h, c]) for j in range(N)) / z
    return out


@pytest.mark.parametrize("N,d", [(1, 4), (2, 4), (3, 4), (63, 4), (64, 4), (65, 4), (130, 4), (3, 64), (65, 64)])
def test_exact_equals_scalar_definition(N, d):
    q, k, v = _qkv(1, N, 2 if N < 100 else 1, d, seed=N * 10 + d)
    sm = oracle.default_sm_scale(d)
    assert np.abs(attention_exact(q, k, v) - _exact_loops(q, k, v, sm)).max() < 1e-13


def test_exact_single_token_returns_v():
    q, k, v = _qkv(2, 1, 3, 16, seed=5)
    assert np.array_equal(attention_exact(q, k, v), v.astype(np.float64))


def test_exact_rows_are_convex_weights():
    # V = identity: the output rows are the softmax rows themselves
    N = 32
    q, k, _ = _qkv(1, N, 1, N, seed=6)
    v = np.eye(N, dtype=F32)[None, :, None, :]
    p = attention_exact(q, k, v)[0, :, 0, :]
    assert np.all(p > 0)
    assert np.abs(p.sum(axis=1) - 1).max() < N * 2.0 ** -52 * 4


@pytest.mark.parametrize("shift", ["mean", "random"])
def test_exact_invariant_to_key_shift(shift):
    q, k, v = _qkv(1, 100, 2, 32, seed=7, kbias=3.0)
    # shifts with few significant bits, so that K - c is exact in fp32
    if shift == "mean":
        c = oracle.k_token_mean(k)[:, None]                      # the smoothing mean, bf16
    else:
        c = np.round(np.random.default_rng(0).standard_normal((1, 1, 2, 32)) * 20) / 4
    kc = k.astype(np.float64) - c
    assert np.array_equal(kc.astype(F32).astype(np.float64), kc)
    a = attention_exact(q, k, v)
    b = attention_exact(q, kc, v)
    assert rel_l2(b, a) < 1e-12


def test_qk_int32_fp64_product_is_exact():
    rng = np.random.default_rng(3)
    a = rng.integers(-127, 128, (40, 128)).astype(np.int8)
    b = rng.integers(-127, 128, (50, 128)).astype(np.int8)
    a[0] = 127
    b[0] = 127
    b[1] = -127
    ref = a.astype(np.int64) @ b.astype(np.int64).T
    got = qk_int32(a, b)
    assert np.array_equal(got, ref)
    assert got[0, 0] == 128 * 127 * 127


@pytest.mark.parametrize("T", [16, 64, 128, 1000])
def test_pipeline_without_quantisation_is_exact_softmax(T):
    q, k, v = _qkv(1, 300, 2, 64, seed=8, kbias=2.0)
    ex = attention_exact(q, k, v)
    pp = attention_pipeline(q, k, v, kv_tile=T, int8_qk=False, fp8_p=False, fp8_v=False)
    # the only rounding left is the fp32 base-2 logit and exp2
    assert np.abs(pp - ex).max() < 2e-6


def test_pipeline_normalisation_with_constant_v():
    # V = 1 everywhere: with unrounded P the output is sum(p) / l = 1 exactly
    q, k, v = _qkv(1, 200, 2, 16, seed=9, kbias=3.0)
    ones = np.ones_like(v)
    o = attention_pipeline(q, k, ones, kv_tile=64, fp8_p=False, fp8_v=False)
    assert np.abs(o - 1).max() < 1e-12
    # with P in e4m3 the output is sum(p8)/sum(p): within the e4m3 relative step
    o8 = attention_pipeline(q, k, ones, kv_tile=64)
    assert np.abs(o8 - 1).max() < 2.0 ** -4


def test_pipeline_uniform_case_closed_form():
    # identical key rows: K' = 0, S = 0, every p equals 448 (up to exp2 rounding),
    # and the output is the token mean of the dequantised V
    q, k, v = _qkv(1, 150, 2, 32, seed=10)
    k[:] = k[:, :1]
    quant = oracle.quantize(q, k, v)
    assert not quant["k_i8"].any()
    o = attention_pipeline(q, k, v, kv_tile=64, quant=quant)
    vd = oracle.e4m3_decode(quant["v_f8"]) * quant["v_scale"][:, :, None, :]
    want = vd.mean(axis=2)                                   # [B, H, d]
    assert np.abs(o - want[:, None]).max() < 1e-6 * np.abs(want).max()
    # Q = 0 gives the same uniform weights
    _, k_rand, _ = _qkv(1, 150, 2, 32, seed=13, kbias=2.0)
    o0 = attention_pipeline(np.zeros_like(q), k_rand, v, kv_tile=64)
    assert np.abs(o0 - want[:, None]).max() < 1e-6 * np.abs(want).max()


def test_pipeline_rows_subset_is_bitwise_consistent():
    q, k, v = _qkv(1, 333, 2, 64, seed=11, kbias=3.0)
    full = attention_pipeline(q, k, v)
    rows = [0, 5, 64, 200, 332]
    sub = attention_pipeline(q, k, v, rows=rows)
    assert np.array_equal(sub, full[:, rows])


def _golden(name):
    path = os.path.join(os.path.dirname(__file__), "golden", "pages_accuracy.txt")
    for line in open(path):
        if line.strip() and not line.startswith("#"):
            key, val = line.split()
            if key == name:
                return float(val)
    raise KeyError(name)


def test_error_budget_sanity_on_tiny_workload():
    w = workloads.get("tiny")
    q, k, v = (t.float().numpy() for t in workloads.make_qkv(w))
    ex = attention_exact(q, k, v)
    full = rel_l2(attention_pipeline(q, k, v), ex)
    int8_only = rel_l2(attention_pipeline(q, k, v, fp8_p=False, fp8_v=False), ex)
    int8_raw = rel_l2(attention_pipeline(q, k, v, fp8_p=False, fp8_v=False, smooth_k=False), ex)
    # full-key INT8 without smoothing: the page's ratio implies about 0.008 * 3.7
    implied = _golden("block_residual_k_rel_l2") * _golden("full_key_int8_closeness_ratio")
    assert implied / 2 < int8_raw < implied * 2
    assert int8_only < int8_raw                      # smoothing helps
    # FP8 rounding of P and V (relative step 2^-3) dominates the full pipeline
    assert 0.02 < full < 0.06


# ---- quality mode: INT8 Q.K^T, P rounded to bf16, V unquantised ----

def _quality(q, k, v, **kw):
    return attention_pipeline(q, k, v, fp8_p=False, bf16_p=True, fp8_v=False, **kw)


def test_quality_uniform_case_is_exact_token_mean():
    # identical key rows: every p is 448, which bf16 holds exactly, so the output is
    # the fp64 token mean of the bf16 V values
    q, k, v = _qkv(1, 150, 2, 32, seed=21)
    k[:] = k[:, :1]
    o = _quality(q, k, v, kv_tile=64)
    want = v.astype(np.float64).mean(axis=1)                   # [B, H, d]
    assert np.abs(o - want[:, None]).max() < 1e-12 * max(1.0, np.abs(want).max())


def test_quality_p_rounding_is_bf16_and_bounded():
    # against the same pipeline with unrounded p: the only difference is the bf16
    # rounding of p (relative step 2^-8, error at most 2^-9 of each p), so each output
    # moves by at most 2^-9 * max|v| of its head, and it does move
    q, k, v = _qkv(1, 257, 2, 64, seed=22, kbias=2.0)
    oq = _quality(q, k, v, kv_tile=128)
    oe = attention_pipeline(q, k, v, kv_tile=128, fp8_p=False, fp8_v=False)
    vmax = np.abs(v.astype(np.float64)).max(axis=(1, 3))        # [B, H]
    diff = np.abs(oq - oe)
    assert (diff <= 2.0 ** -9 * vmax[:, None, :, None] * (1 + 1e-9)).all()
    assert diff.max() > 0
    # e4m3 rounding of p instead would exceed that bound somewhere
    o8 = attention_pipeline(q, k, v, kv_tile=128, fp8_v=False)
    assert (np.abs(o8 - oe) > 2.0 ** -9 * vmax[:, None, :, None]).any()


def test_quality_mode_error_budget():
    # with P.V in 16 bits the error left is the INT8 Q.K^T quantisation: well below the
    # speed mode's and within 0.02 of exact attention on the tiny workload
    w = workloads.get("tiny")
    q, k, v = (t.float().numpy() for t in workloads.make_qkv(w))
    ex = attention_exact(q, k, v)
    rq = oracle.rel_l2(_quality(q, k, v, kv_tile=128), ex)
    rs = oracle.rel_l2(attention_pipeline(q, k, v, kv_tile=128), ex)
    assert rq < 0.02 and rq < 0.6 * rs


# ---- the fused multiply-add of the decision arithmetic ----

def test_fma_is_single_rounding_against_exact_rationals():
    from fractions import Fraction
    from oracle.attention import _fma_f32

    def rne_f32(fr):
        # nearest fp32 to the exact rational, ties to the even pattern
        c = np.float32(float(fr))
        cands = [c, np.nextafter(c, np.float32(np.inf)), np.nextafter(c, np.float32(-np.inf))]
        return min(cands, key=lambda z: (abs(Fraction(float(z)) - fr),
                                         int(np.array(z, np.float32).view(np.uint32)) & 1))

    rng = np.random.default_rng(5)
    x = rng.integers(-2 ** 23, 2 ** 23, 400).astype(np.float64)
    c = (rng.standard_normal(400) * 1e-3).astype(np.float32)
    b = (rng.standard_normal(400) * 10).astype(np.float32)
    got = _fma_f32(x, c, b)
    for i in range(400):
        want = rne_f32(Fraction(float(x[i])) * Fraction(float(c[i])) + Fraction(float(b[i])))
        assert got[i] == want
    # sums that land exactly halfway between two fp32 values after fp64 rounding: the
    # exact value decides (above, below, exact tie -> even)
    xs = np.array([2.0 ** 6 + 2.0 ** -30, 2.0 ** 6 - 2.0 ** -30, 2.0 ** 6, -(2.0 ** 6 + 2.0 ** -30)])
    bs = np.array([2.0 ** 30, 2.0 ** 30, 2.0 ** 30, -(2.0 ** 30)], np.float32)
    got = _fma_f32(xs, np.ones(4, np.float32), bs).astype(np.float64)
    assert list(got - np.array([2.0 ** 30, 2.0 ** 30, 2.0 ** 30, -(2.0 ** 30)])) == [128.0, 0.0, 0.0, -128.0]


# ---- per-token INT8 scales ----

def test_per_token_quality_mode_meets_the_rel_l2_gate():
    # one INT8 scale per token for Q and K, with bf16 P.V: the configuration whose
    # error stays under 0.01 of exact attention on the tiny workload
    w = workloads.get("tiny")
    q, k, v = (t.float().numpy() for t in workloads.make_qkv(w))
    ex = attention_exact(q, k, v)
    r_tok = oracle.rel_l2(_quality(q, k, v, kv_tile=128, block=1), ex)
    r_blk = oracle.rel_l2(_quality(q, k, v, kv_tile=128), ex)
    assert r_tok <= 0.01 < r_blk


def test_per_token_uniform_case_and_scales():
    q, k, v = _qkv(1, 150, 2, 32, seed=23)
    k[:] = k[:, :1]
    quant = oracle.quantize(q, k, v, block=1)
    assert quant["q_scale"].shape == (1, 2, 150) and quant["block"] == 1
    o = _quality(q, k, v, kv_tile=64, quant=quant)
    want = v.astype(np.float64).mean(axis=1)
    assert np.abs(o - want[:, None]).max() < 1e-12 * max(1.0, np.abs(want).max())
    # without fp8/bf16 rounding of P and V the per-token pipeline is the exact softmax
    # of the dequantised operands
    q2, k2, v2 = _qkv(1, 90, 1, 16, seed=24, kbias=2.0)
    qt = oracle.quantize(q2, k2, v2, block=1)
    got = attention_pipeline(q2, k2, v2, kv_tile=32, quant=qt, fp8_p=False, fp8_v=False)
    qd = qt["q_i8"][0, 0].astype(np.float64) * qt["q_scale"][0, 0][:, None]
    kd = qt["k_i8"][0, 0].astype(np.float64) * qt["k_scale"][0, 0][:, None]
    s = qd @ kd.T / np.sqrt(16)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    want = (p / p.sum(axis=1, keepdims=True)) @ v2[0, :, 0, :].astype(np.float64)
    assert np.abs(got[0, :, 0, :] - want).max() < 2e-5


# ---- block-residual K ----

def test_block_mean_closed_form_block_constant_keys():
    # K constant inside every 64-token block (different across blocks): the block
    # means reproduce K exactly, the residual codes are 0, and with unrounded P and V
    # the pipeline is the exact softmax of (dequantised Q) . K^T
    q, k, v = _qkv(1, 150, 2, 32, seed=31, kbias=2.0)
    for j in range(0, 150, 64):
        k[:, j:j + 64] = k[:, j:j + 1]
    quant = oracle.quantize(q, k, v, k_block_mean=True)
    assert not quant["k_i8"].any()
    got = attention_pipeline(q, k, v, kv_tile=64, quant=quant, fp8_p=False, fp8_v=False)
    for h in range(2):
        qd = quant["q_i8"][0, h].astype(np.float64) * np.repeat(quant["q_scale"][0, h], 64)[:150, None]
        s = qd @ k[0, :, h, :].astype(np.float64).T / np.sqrt(32)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        want = (p / p.sum(axis=1, keepdims=True)) @ v[0, :, h, :].astype(np.float64)
        assert np.abs(got[0, :, h, :] - want).max() < 1e-5


def test_block_mean_error_budget_matches_token_mean_on_synthetic_keys():
    # the synthetic keys have no token-local structure, so block means neither help
    # nor hurt noticeably
    w = workloads.get("tiny")
    q, k, v = (t.float().numpy() for t in workloads.make_qkv(w))
    ex = attention_exact(q, k, v)
    r_tok = oracle.rel_l2(attention_pipeline(q, k, v, kv_tile=128), ex)
    r_blk = oracle.rel_l2(attention_pipeline(q, k, v, kv_tile=128, k_block_mean=True), ex)
    assert abs(r_blk - r_tok) < 0.003


# ---- the plain (fp64) pipeline against definitions it must reduce to ----

def _dequant_softmax(quant, v, b, h, sm):
    """Textbook fp64 attention of the dequantised INT8 operands (natural exp, no base-2
    logits, no tiles): q_deq = q_scale * q8, k_deq = k_scale * k8 (+ the block mean)."""
    qb = quant["block"]
    q8 = quant["q_i8"][b, h].astype(np.float64)
    k8 = quant["k_i8"][b, h].astype(np.float64)
    n = k8.shape[0]
    qd = q8 * quant["q_scale"][b, h][np.arange(q8.shape[0]) // qb][:, None]
    kd = k8 * quant["k_scale"][b, h][np.arange(n) // qb][:, None]
    if "k_bmean" in quant:
        kd = kd + quant["k_bmean"][b, h][np.arange(n) // 64].astype(np.float64)
    s = (qd @ kd.T) * sm
    e = np.exp(s - s.max(axis=1, keepdims=True))
    return (e / e.sum(axis=1, keepdims=True)) @ v[b, :, h, :].astype(np.float64)


@pytest.mark.parametrize("mode", ["block64", "per_token", "block_mean"])
def test_int8_pipeline_is_softmax_of_dequantised_operands(mode):
    # FP8 rounding of P and V off: what is left is exact softmax of the dequantised
    # Q and K, for any key tile.  A wrong scale index, a missing scale or a dropped
    # block-mean term changes the logits and fails this.
    q, k, v = _qkv(2, 300, 2, 64, seed=41, kbias=3.0)
    k[:, :, :, 7] *= 20                                       # an outlier channel
    quant = oracle.quantize(q, k, v, block=1 if mode == "per_token" else 64,
                            k_block_mean=mode == "block_mean")
    sm = oracle.default_sm_scale(64)
    for T in (64, 128):
        got64 = attention_pipeline(q, k, v, kv_tile=T, quant=quant, fp8_p=False, fp8_v=False)
        got32 = attention_pipeline(q, k, v, kv_tile=T, quant=quant, fp8_p=False, fp8_v=False, arith="fp32")
        for b in range(2):
            for h in range(2):
                want = _dequant_softmax(quant, v, b, h, sm)
                assert np.abs(got64[b, :, h] - want).max() < 1e-12
                assert np.abs(got32[b, :, h] - want).max() < 2e-5


def test_online_single_tile_equals_two_pass_bitwise():
    # T >= N: one tile, so the running maximum is the row maximum and the online
    # recurrence must reduce to the two-pass form bit for bit, FP8 P and V included
    q, k, v = _qkv(1, 200, 2, 64, seed=42, kbias=2.0)
    quant = oracle.quantize(q, k, v)
    sm = oracle.default_sm_scale(64)
    got = attention_pipeline(q, k, v, kv_tile=256, quant=quant)
    rows = np.arange(200)
    for h in range(2):
        s = oracle.pipeline_logits(q, k, quant, 0, h, rows, sm)
        m = s.max(axis=1)
        p = np.exp2(s - m[:, None])
        l = p.sum(axis=1)
        p8 = oracle.e4m3_decode(oracle.e4m3_encode(448.0 * p))
        vv = oracle.e4m3_decode(quant["v_f8"][0, h])
        two_pass = (p8 @ vv) / (448.0 * l[:, None]) * quant["v_scale"][0, h].astype(np.float64)[None, :]
        assert np.array_equal(got[0, :, h], two_pass)


@pytest.mark.parametrize("T", [32, 64, 128])
def test_online_recurrence_equals_closed_form_over_tile_maxima(T):
    # With FP8 P each code is rounded against the running maximum m_t after tile t.
    # Unrolled, the recurrence is O = sum_t 2^(m_t - m_last) sum_{j in t}
    # e4m3(448 * 2^(s_j - m_t)) v_j / (448 sum_j 2^(s_j - m_last)).
    q, k, v = _qkv(1, 333, 2, 64, seed=43, kbias=2.0)
    quant = oracle.quantize(q, k, v)
    sm = oracle.default_sm_scale(64)
    got = attention_pipeline(q, k, v, kv_tile=T, quant=quant)
    rows = np.arange(333)
    for h in range(2):
        s = oracle.pipeline_logits(q, k, quant, 0, h, rows, sm)
        vv = oracle.e4m3_decode(quant["v_f8"][0, h])
        starts = list(range(0, 333, T))
        mt = np.maximum.accumulate(np.stack([s[:, t0:t0 + T].max(axis=1) for t0 in starts]), axis=0)
        m_last = mt[-1]
        num = np.zeros((333, 64))
        for t, t0 in enumerate(starts):
            p8 = oracle.e4m3_decode(oracle.e4m3_encode(448.0 * np.exp2(s[:, t0:t0 + T] - mt[t][:, None])))
            num += np.exp2(mt[t] - m_last)[:, None] * (p8 @ vv[t0:t0 + T])
        den = 448.0 * np.exp2(s - m_last[:, None]).sum(axis=1)
        want = num / den[:, None] * quant["v_scale"][0, h].astype(np.float64)[None, :]
        assert np.abs(got[0, :, h] - want).max() < 1e-13


def _two_key_case(delta_codes):
    """One query, two keys whose base-2 logits differ by L * delta_codes (L = sm_scale *
    log2 e with sm_scale 0.1), and one-hot V rows of 448 (v_scale 1/448), built
    directly as quantised operands."""
    d = 2
    z = np.zeros((1, 2, 1, d), dtype=F32)
    quant = dict(q_i8=np.array([[[[1, 0], [0, 0]]]], np.int8),
                 q_scale=np.array([[[1.0]]], F32),
                 k_i8=np.array([[[[0, 0], [-delta_codes, 0]]]], np.int8),
                 k_scale=np.array([[[1.0]]], F32),
                 k_mean=np.zeros((1, 1, d), F32),
                 v_f8=np.array([[[[0x7E, 0], [0, 0x7E]]]], np.uint8),
                 v_scale=np.full((1, 1, d), 1 / 448, F32), block=64)
    return z, quant


def test_p_codes_carry_the_static_scale_448():
    # p0 = 1 and p1 = 2^(-0.1 * log2(e) * 3) = 0.7408: 448 * p1 = 331.9 rounds to the
    # e4m3 value 320, while e4m3(p1) alone would be 0.75.  O = (p8 * v8 * v_scale) /
    # (448 * l) with l = 1 + p1.
    z, quant = _two_key_case(3)
    p1 = 2.0 ** (-0.1 * oracle.LOG2E * 3)
    assert oracle.e4m3_decode(oracle.e4m3_encode(448 * p1)) == 320.0
    want = np.array([448.0, 320.0]) / (448.0 * (1 + p1))
    for arith in ("fp64", "fp32"):
        got = attention_pipeline(z, z, z, sm_scale=0.1, quant=quant, rows=[0], arith=arith)[0, 0, 0]
        assert np.abs(got - want).max() < 1e-6, arith
    # the same logits without the 448 would give 0.75 / (1 + p1) in channel 1
    assert abs(0.75 / (1 + p1) - want[1]) > 0.02


def test_fp32_reading_saturates_p_codes_at_huge_logits():
    # With |logits| near 2^21 the fp32 roundings of the running maximum and of
    # log2(448) - m leave up to ~1/4 in the exponent either way, so the row maximum's
    # p lies anywhere in about [377, 608]; above 464 an unsaturated e4m3 conversion
    # gives NaN.  The reading saturates the code at 448 while l keeps the unrounded p,
    # so every output row is a finite positive multiple of one dequantised V row, and
    # the rows whose p passed 464 have a factor below 448/464.
    q, k, v = _qkv(1, 256, 1, 128, seed=44)
    q, k = q * 1000, k * 1000
    quant = oracle.quantize(q, k, v)
    o = attention_pipeline(q, k, v, quant=quant, arith="fp32")[0, :, 0]
    assert np.isfinite(o).all()
    vd = oracle.e4m3_decode(quant["v_f8"][0, 0]) * quant["v_scale"][0, 0].astype(np.float64)[None, :]
    s = oracle.pipeline_logits(q, k, quant, 0, 0, np.arange(256), oracle.default_sm_scale(128))
    jmax = s.argmax(axis=1)
    ratio = (o * vd[jmax]).sum(axis=1) / (vd[jmax] ** 2).sum(axis=1)
    assert np.abs(o - ratio[:, None] * vd[jmax]).max() < 1e-9
    assert (ratio > 448 / 620).all() and (ratio < 1.1).all() and (ratio < 448 / 464).sum() >= 10
    # the plain reading keeps p = 1 at the maximum: exactly the V row
    o64 = attention_pipeline(q, k, v, quant=quant)[0, :, 0]
    assert np.abs(o64 - vd[jmax]).max() < 1e-12


def test_fp32_and_fp64_readings_agree_on_the_workloads():
    # the two readings differ only where an fp32 rounding moves a P code across an
    # e4m3 rounding boundary: within 1e-4 on the tiny workload and on sampled rows of
    # one head of the Flux-like and stress shapes
    cases = [(workloads.get("tiny"), None),
             (workloads.Workload("flux_head", B=1, H=1, N=4608, d=128), 48),
             (workloads.Workload("stress_head", B=1, H=1, N=65536, d=128, outliers=4), 12)]
    for w, nrows in cases:
        q, k, v = (t.float().numpy() for t in workloads.make_qkv(w))
        quant = oracle.quantize(q, k, v)
        rows = None if nrows is None else np.random.default_rng(0).choice(w.N, nrows, replace=False)
        a = attention_pipeline(q, k, v, quant=quant, rows=rows)
        b = attention_pipeline(q, k, v, quant=quant, rows=rows, arith="fp32")
        assert np.abs(a - b).max() < 1e-4, w.name


def test_code_margin_covers_the_fp32_reading():
    # the two readings differ only through P codes that an fp32 evaluation may round the
    # other way; the plain reading's margin bounds that: |fp64 - fp32| <= margin + 1e-5
    # everywhere, in every mode, on inputs whose outlier channels and block means give
    # logits of several hundred (where codes do flip)
    w = workloads.Workload("case", B=2, H=3, N=200, d=128, outliers=2, seed=7)
    q, k, v = (t.float().numpy() for t in workloads.make_qkv(w))
    flipped = False
    for kw in [dict(block=64), dict(block=1), dict(block=64, k_block_mean=True),
               dict(block=1, k_block_mean=True)]:
        quant = oracle.quantize(q, k, v, **kw)
        for pk in [dict(), dict(fp8_p=False, bf16_p=True, fp8_v=False)]:
            if "k_block_mean" in kw and pk:
                continue
            a, mg = attention_pipeline(q, k, v, quant=quant, code_margin=True, **pk)
            b = attention_pipeline(q, k, v, quant=quant, arith="fp32", **pk)
            assert (np.abs(a - b) <= mg + 1e-5).all(), (kw, pk)
            flipped |= bool((np.abs(a - b) > 1e-4).any())
    assert flipped                       # the case does exercise code flips
    # with P unrounded no code can flip: the margin is zero
    quant = oracle.quantize(q, k, v)
    _, mg = attention_pipeline(q, k, v, quant=quant, code_margin=True, fp8_p=False, fp8_v=False)
    assert not mg.any()
