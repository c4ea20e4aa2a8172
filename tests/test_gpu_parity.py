"""GPU parity of the HIP path against the CPU oracle, through the C ABI: quantised
operands bit-exact, int32 Q.K^T tiles bit-exact, attention output within the
max-abs bound of the oracle's quantised pipeline, on small and ragged shapes."""
import numpy as np
import pytest
import torch

import oracle
import workloads
import quantized_attention_diffusion_amd as sage
from gpu_helpers import (require_gpu, to_np, random_qkv, compare_quant, check_oracle)

pytestmark = pytest.mark.gpu

KV_TILE = 128          # must equal sage_kernel_info()["kv_tile"] (checked below)

CASES = [  # (B, N, H, d, seed, outliers)
    (1, 256, 2, 64, 0, 0),      # the 'tiny' workload shape
    (1, 1, 1, 128, 1, 0),
    (1, 63, 3, 64, 2, 0),
    (2, 64, 2, 128, 3, 0),
    (1, 65, 2, 128, 4, 0),
    (1, 127, 1, 64, 5, 0),
    (1, 129, 2, 128, 6, 0),
    (2, 200, 3, 128, 7, 2),
    (1, 1000, 2, 128, 8, 4),
    (1, 1100, 2, 64, 9, 0),     # tail of 76 keys: the last 64-key scale block is all padding
]


def _case_id(c):
    return "B{}_N{}_H{}_d{}".format(*c[:4])


def _np(t):
    return t.float().numpy()


def setup_module(module):
    require_gpu()
    info = sage.sage_kernel_info()
    assert info["kv_tile"] == KV_TILE and info["arch"] == "gfx950"


@pytest.mark.parametrize("case", CASES, ids=_case_id)
def test_quant_bit_exact(case):
    B, N, H, d, seed, outl = case
    print(f"[quant] {_case_id(case)}", flush=True)
    q, k, v = random_qkv(B, N, H, d, seed, outl)
    gq = sage.sage_quant_qk(q.cuda(), k.cuda(), v.cuda())
    torch.cuda.synchronize()
    ref = oracle.quantize(_np(q), _np(k), _np(v))
    compare_quant(gq, ref, N)


@pytest.mark.parametrize("case", CASES, ids=_case_id)
def test_qk_int32_tiles_bit_exact(case):
    B, N, H, d, seed, outl = case
    print(f"[qk_i32] {_case_id(case)}", flush=True)
    q, k, v = random_qkv(B, N, H, d, seed, outl)
    gq = sage.sage_quant_qk(q.cuda(), k.cuda(), v.cuda())
    ref = oracle.quantize(_np(q), _np(k), _np(v))
    npad = gq["q_i8"].shape[2]
    info = sage.sage_kernel_info()
    nqb, nkt = npad // info["block_m"], npad // info["kv_tile"]
    # at d = 128 mode 0 runs the 32x32 body and the other modes the 16x16 one; the
    # debug entry point takes the same staging and products as the body of its mode
    modes = (0, sage.SAGE_QK_PER_TOKEN) if d == 128 else (0,)
    for mode in modes:
        for b in range(B):
            for h in range(H):
                s = sage.sage_debug_qk_i32_ex(gq["q_i8"], gq["k_i8"], N, b, h, 0, 0, nqb, nkt,
                                              mode=mode).cpu().numpy()
                want = oracle.qk_int32(ref["q_i8"][b, h], ref["k_i8"][b, h])        # [N, N]
                assert np.array_equal(s[:N, :N], want), f"S differs at head ({b}, {h}), mode {mode}"
                assert not s[N:, :].any() and not s[:, N:].any()                    # zero padding


@pytest.mark.parametrize("case", CASES, ids=_case_id)
def test_attention_matches_oracle_pipeline(case):
    B, N, H, d, seed, outl = case
    print(f"[attn] {_case_id(case)}", flush=True)
    q, k, v = random_qkv(B, N, H, d, seed, outl)
    out = sage.sage_attn_fwd(q.cuda(), k.cuda(), v.cuda())
    o = to_np(out)
    err, err32, pipe = check_oracle(o, _case_id(case), _np(q), _np(k), _np(v), kv_tile=KV_TILE)
    exact = oracle.attention_exact(_np(q), _np(k), _np(v))
    # the GPU adds no error beyond the specified quantisation
    assert oracle.rel_l2(o, exact) <= oracle.rel_l2(pipe, exact) + 0.002
    print(f"    max|gpu-pipe| = {err:.2e} (fp32 reading {err32:.2e})  relL2(gpu, exact) = "
          f"{oracle.rel_l2(o, exact):.4f}  relL2(pipe, exact) = {oracle.rel_l2(pipe, exact):.4f}", flush=True)


def test_tiny_workload_end_to_end():
    w = workloads.get("tiny")
    q, k, v = workloads.make_qkv(w)
    out = sage.sage_attn_fwd(q.cuda(), k.cuda(), v.cuda())
    check_oracle(to_np(out), "tiny", _np(q), _np(k), _np(v), kv_tile=KV_TILE)


def test_layouts_and_fused_qkv_views():
    B, N, H, d = 1, 300, 3, 128
    q, k, v = random_qkv(B, N, H, d, seed=21)
    ref = to_np(sage.sage_attn_fwd(q.cuda(), k.cuda(), v.cuda()))
    # [B, H, N, d] tensors
    qh, kh, vh = (t.transpose(1, 2).contiguous().cuda() for t in (q, k, v))
    oh = sage.sage_attn_fwd(qh, kh, vh, layout="bhnd")
    assert np.array_equal(to_np(oh).transpose(0, 2, 1, 3), ref)
    # strided slices of a fused qkv projection [B, N, 3, H, d] (no copies)
    qkv = torch.stack([q, k, v], dim=2).cuda()
    of = sage.sage_attn_fwd(qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2])
    assert np.array_equal(to_np(of), ref)
    # output written through a strided view (every other head of a wider tensor)
    wide = torch.zeros(B, N, 2 * H, d, dtype=torch.bfloat16, device="cuda")
    sage.sage_attn_fwd(q.cuda(), k.cuda(), v.cuda(), out=wide[:, :, ::2])
    assert np.array_equal(to_np(wide[:, :, ::2]), ref)
    assert not wide[:, :, 1::2].any()


def test_prequant_path_equals_fused_entry_point():
    q, k, v = random_qkv(2, 333, 2, 128, seed=22)
    qc, kc, vc = q.cuda(), k.cuda(), v.cuda()
    gq = sage.sage_quant_qk(qc, kc, vc)
    a = sage.sage_attn_fwd_prequant(gq)
    b = sage.sage_attn_fwd(qc, kc, vc)
    assert torch.equal(a, b)


def test_deterministic_runs():
    q, k, v = random_qkv(1, 777, 4, 128, seed=23)
    qc, kc, vc = q.cuda(), k.cuda(), v.cuda()
    outs = [sage.sage_attn_fwd(qc, kc, vc) for _ in range(3)]
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[1], outs[2])


GRID_MODES = [  # (pv, per_token, k_block_mean): every dense instance family
    ("fp8", False, False), ("fp8", True, False), ("fp8", False, True), ("fp8", True, True),
    ("bf16", False, False), ("bf16", True, False)]


@pytest.mark.parametrize("d", [64, 128])
def test_short_and_long_grids_agree(d):
    # Grids of at most 4 x (compute units) workgroups launch the instance with
    # workgroup-pair issue priorities, longer grids the plain one; the priorities only
    # reorder instruction issue, so a head's output bits must not depend on the grid,
    # in every mode.
    cus = torch.cuda.get_device_properties(torch.cuda.current_device()).multi_processor_count
    N = 1000                                           # 8 query blocks per head
    H = 4 * cus // 8 + 2
    print(f"[grids] d={d} H={H} N={N}: {8 * H} workgroups against {8 * 2} for two heads", flush=True)
    q, k, v = (t.cuda() for t in random_qkv(1, N, H, d, seed=25))
    heads = slice(H - 2, H)
    for pv, tok, kbm in GRID_MODES:
        long_dense = sage.sage_attn_fwd_ex(q, k, v, pv=pv, per_token=tok, k_block_mean=kbm)
        short_dense = sage.sage_attn_fwd_ex(q[:, :, heads], k[:, :, heads], v[:, :, heads], pv=pv,
                                            per_token=tok, k_block_mean=kbm)
        assert torch.equal(long_dense[:, :, heads].contiguous().view(torch.int16),
                           short_dense.view(torch.int16)), (pv, tok, kbm)
    long_sparse = sage.sage_attn_fwd_sparse(q, k, v, 0.5)
    short_sparse = sage.sage_attn_fwd_sparse(q[:, :, heads], k[:, :, heads], v[:, :, heads], 0.5)
    assert torch.equal(long_sparse[:, :, heads].contiguous().view(torch.int16), short_sparse.view(torch.int16))


def test_sm_scale_argument():
    q, k, v = random_qkv(1, 200, 2, 64, seed=24)
    out = sage.sage_attn_fwd(q.cuda(), k.cuda(), v.cuda(), sm_scale=0.05)
    check_oracle(to_np(out), "sm_scale=0.05", _np(q), _np(k), _np(v), sm_scale=0.05, kv_tile=KV_TILE)


def test_degenerate_inputs():
    B, N, H, d = 1, 150, 2, 64
    q, k, v = random_qkv(B, N, H, d, seed=25)
    k[:] = k[:, :1]                      # identical keys: K' = 0, all k scales 0
    q[:, 64:128] = 0                     # an all-zero Q block: q scale 0
    v[:, :, :, 5] = 0                    # a zero V channel: v scale 0
    gq = sage.sage_quant_qk(q.cuda(), k.cuda(), v.cuda())
    ref = oracle.quantize(_np(q), _np(k), _np(v))
    compare_quant(gq, ref, N)
    out = sage.sage_attn_fwd(q.cuda(), k.cuda(), v.cuda())
    check_oracle(to_np(out), "degenerate", _np(q), _np(k), _np(v), kv_tile=KV_TILE)
    assert torch.isfinite(out.float()).all()


@pytest.mark.parametrize("kind", ["peaked", "huge_logits", "huge_v", "tiny_qk", "outlier_key"])
@pytest.mark.parametrize("pv", ["fp8", "bf16"])
def test_extreme_magnitudes(kind, pv):
    # peaked: Q and K times 300, base-2 logits of order 3e5: every p but the row
    # maximum's underflows to 0;
    # huge_logits: Q and K times 1000, logits near 2^21: the fp32 roundings of the
    # running maximum and of log2(448) - m leave up to 1/4 in the exponent, so the row
    # maximum's p passes 464 in many rows and its e4m3 conversion must saturate at 448;
    # huge_v: V times 2^13, which scales the V codes' scales and every later product by
    # exactly 2^13, so the output must be 2^13 times the unscaled one, bit for bit (the
    # absolute 2e-3 term of the bound is for V of order 1); tiny_qk: scales of order
    # 1e-22 and logits that vanish against the exp2 offset (uniform attention);
    # outlier_key: one key 1000x larger.
    # In the first two the logits pass 2^16, where an fp32 logit carries an absolute
    # error of 2^-8 or more: the method's fp32 softmax cannot follow fp64 logits there,
    # so these compare with the reading that decides P in fp32 only.
    B, N, H, d = 1, 700, 2, 128
    q, k, v = random_qkv(B, N, H, d, seed=26)
    readings = ("fp64", "fp32")
    if kind in ("peaked", "huge_logits"):
        f = 300 if kind == "peaked" else 1000
        q, k = (q.float() * f).to(torch.bfloat16), (k.float() * f).to(torch.bfloat16)
        readings = ("fp32",)
    elif kind == "huge_v":
        base = sage.sage_attn_fwd_ex(q.cuda(), k.cuda(), v.cuda(), pv=pv)
        big = sage.sage_attn_fwd_ex(q.cuda(), k.cuda(), (v.float() * 8192).to(torch.bfloat16).cuda(), pv=pv)
        assert torch.equal(big.float(), base.float() * 8192)
        assert torch.isfinite(big.float()).all()
    elif kind == "tiny_qk":
        q, k = (q.float() * 1e-20).to(torch.bfloat16), (k.float() * 1e-20).to(torch.bfloat16)
    else:
        k[:, 333] = (k[:, 333].float() * 1000).to(torch.bfloat16)
    print(f"[extreme] {kind} pv={pv}", flush=True)
    out = sage.sage_attn_fwd_ex(q.cuda(), k.cuda(), v.cuda(), pv=pv)
    assert torch.isfinite(out.float()).all()
    check_oracle(to_np(out), f"extreme {kind} {pv}", _np(q), _np(k), _np(v), kv_tile=KV_TILE,
                 fp8_p=pv == "fp8", fp8_v=pv == "fp8", bf16_p=pv == "bf16", readings=readings)


def test_e4m3_conversion_matches_oracle_encoder():
    t = oracle.e4m3_table()[:0x7F]
    mids = (t[:-1] + t[1:]) / 2
    base = np.concatenate([t, mids]).astype(np.float32)
    u = base.view(np.uint32).astype(np.int64)
    near = np.concatenate([u + dlt for dlt in range(-3, 4)])
    near = np.clip(near, 0, None).astype(np.uint32).view(np.float32)
    top = np.array([480.0], np.float32).view(np.uint32)[0]
    sweep = np.arange(0, int(top) + 1, 997, dtype=np.uint32).view(np.float32)
    x = np.concatenate([near, sweep, np.array([464.0, 470.0, 1e6, 1e-30], np.float32)])
    x = np.concatenate([x, -x]).astype(np.float32)
    got = sage.sage_debug_e4m3(torch.from_numpy(x).cuda()).cpu().numpy()
    assert np.array_equal(got, oracle.e4m3_encode(x))


# ---- quality mode: INT8 Q.K^T, bf16 P.V ----

def _quality_check(o, label, q, k, v, **kw):
    return check_oracle(o, label, _np(q), _np(k), _np(v), kv_tile=KV_TILE, fp8_p=False,
                        bf16_p=True, fp8_v=False, **kw)


@pytest.mark.parametrize("case", CASES, ids=_case_id)
def test_quality_mode_matches_oracle_pipeline(case):
    B, N, H, d, seed, outl = case
    print(f"[quality] {_case_id(case)}", flush=True)
    q, k, v = random_qkv(B, N, H, d, seed, outl)
    out = sage.sage_attn_fwd_ex(q.cuda(), k.cuda(), v.cuda(), pv="bf16")
    o = to_np(out)
    err, _, pipe = _quality_check(o, "quality " + _case_id(case), q, k, v)
    exact = oracle.attention_exact(_np(q), _np(k), _np(v))
    assert oracle.rel_l2(o, exact) <= oracle.rel_l2(pipe, exact) + 0.002
    print(f"    max|gpu-pipe| = {err:.2e}  relL2(gpu, exact) = {oracle.rel_l2(o, exact):.4f}", flush=True)


def test_quality_mode_layouts_degenerate_and_fp8_entry():
    B, N, H, d = 1, 300, 3, 128
    q, k, v = random_qkv(B, N, H, d, seed=31)
    ref = to_np(sage.sage_attn_fwd_ex(q.cuda(), k.cuda(), v.cuda(), pv="bf16"))
    qkv = torch.stack([q, k, v], dim=2).cuda()
    of = sage.sage_attn_fwd_ex(qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2], pv="bf16")
    assert np.array_equal(to_np(of), ref)
    qh, kh, vh = (t.transpose(1, 2).contiguous().cuda() for t in (q, k, v))
    oh = sage.sage_attn_fwd_ex(qh, kh, vh, layout="bhnd", pv="bf16")
    assert np.array_equal(to_np(oh).transpose(0, 2, 1, 3), ref)
    # the fp8 mode of the extended entry point is sage_attn_fwd
    a = sage.sage_attn_fwd_ex(q.cuda(), k.cuda(), v.cuda(), pv="fp8")
    b = sage.sage_attn_fwd(q.cuda(), k.cuda(), v.cuda())
    assert torch.equal(a, b)
    # identical keys: every p = 448 (exact in bf16), the output is the token mean of V
    k2 = k.clone()
    k2[:] = k2[:, :1]
    o2 = sage.sage_attn_fwd_ex(q.cuda(), k2.cuda(), v.cuda(), pv="bf16")
    _quality_check(to_np(o2), "quality uniform", q, k2, v)



# ---- per-token Q/K scales (with FP8 or bf16 P.V) ----

def _head_slice(d, b, h):
    return {k: (v[b:b + 1, h:h + 1] if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


@pytest.mark.parametrize("pv", ["fp8", "bf16"])
@pytest.mark.parametrize("case", CASES[:6] + CASES[7:9], ids=_case_id)
def test_per_token_mode_matches_oracle(case, pv):
    B, N, H, d, seed, outl = case
    print(f"[per-token {pv}] {_case_id(case)}", flush=True)
    q, k, v = random_qkv(B, N, H, d, seed, outl)
    qc, kc, vc = q.cuda(), k.cuda(), v.cuda()
    mode = sage.mode_bits(pv, per_token=True)
    ref = oracle.quantize(_np(q), _np(k), _np(v), block=1)
    # per-token codes and scales bit-exact
    gq = sage.sage_quant_qk_ex(qc, kc, vc, mode)
    torch.cuda.synchronize()
    for name in ("q", "k"):
        codes = gq[f"{name}_i8"].cpu().numpy()
        assert np.array_equal(codes[:, :, :N], ref[f"{name}_i8"]), f"{name}_i8 differs"
        assert not codes[:, :, N:].any()
        sc = gq[f"{name}_scale"].cpu().numpy()
        assert np.array_equal(sc[:, :, :N].view(np.uint32), ref[f"{name}_scale"].view(np.uint32)), f"{name}_scale differs"
        assert not sc[:, :, N:].any()
    if pv == "bf16":
        # V is transposed, not quantised
        v16 = gq["v_f8"].float().cpu().numpy().transpose(0, 1, 3, 2)
        assert np.array_equal(v16[:, :, :N], _np(v).transpose(0, 2, 1, 3)) and not v16[:, :, N:].any()
    out = sage.sage_attn_fwd_ex(qc, kc, vc, pv=pv, per_token=True)
    o = to_np(out)
    err, _, pipe = check_oracle(o, f"per-token {pv} " + _case_id(case), _np(q), _np(k), _np(v),
                                kv_tile=KV_TILE, quant=ref, fp8_p=(pv == "fp8"), bf16_p=(pv == "bf16"),
                                fp8_v=(pv == "fp8"))
    exact = oracle.attention_exact(_np(q), _np(k), _np(v))
    assert oracle.rel_l2(o, exact) <= oracle.rel_l2(pipe, exact) + 0.002
    print(f"    max|gpu-pipe| = {err:.2e}  relL2(gpu, exact) = {oracle.rel_l2(o, exact):.4f}", flush=True)


def test_per_token_quality_mode_meets_rel_l2_gate_on_tiny():
    w = workloads.get("tiny")
    q, k, v = workloads.make_qkv(w)
    out = sage.sage_attn_fwd_ex(q.cuda(), k.cuda(), v.cuda(), pv="bf16", per_token=True)
    exact = oracle.attention_exact(_np(q), _np(k), _np(v))
    assert oracle.rel_l2(to_np(out), exact) <= 0.01



# ---- block-residual K (FP8 P.V) ----

@pytest.mark.parametrize("per_token", [False, True], ids=["block64", "per_token"])
@pytest.mark.parametrize("case", CASES[:6] + CASES[7:9], ids=_case_id)
def test_block_mean_mode_matches_oracle(case, per_token):
    B, N, H, d, seed, outl = case
    print(f"[block-mean per_token={per_token}] {_case_id(case)}", flush=True)
    q, k, v = random_qkv(B, N, H, d, seed, outl)
    qc, kc, vc = q.cuda(), k.cuda(), v.cuda()
    mode = sage.mode_bits("fp8", per_token=per_token, k_block_mean=True)
    ref = oracle.quantize(_np(q), _np(k), _np(v), block=1 if per_token else 64, k_block_mean=True)
    gq = sage.sage_quant_qk_ex(qc, kc, vc, mode)
    torch.cuda.synchronize()
    nb = -(-N // 64)
    km = gq["k_mean"].float().cpu().numpy()                   # [B, H, Npad/64, d]
    assert np.array_equal(km[:, :, :nb].view(np.uint32), ref["k_bmean"].view(np.uint32)), "block means differ"
    assert not km[:, :, nb:].any()
    for name in ("q", "k"):
        codes = gq[f"{name}_i8"].cpu().numpy()
        assert np.array_equal(codes[:, :, :N], ref[f"{name}_i8"]), f"{name}_i8 differs"
        sc = gq[f"{name}_scale"].cpu().numpy()
        nsc = N if per_token else nb
        assert np.array_equal(sc[:, :, :nsc].view(np.uint32), ref[f"{name}_scale"].view(np.uint32)), f"{name}_scale differs"
    out = sage.sage_attn_fwd_ex(qc, kc, vc, per_token=per_token, k_block_mean=True)
    o = to_np(out)
    err, _, pipe = check_oracle(o, f"block-mean {_case_id(case)}", _np(q), _np(k), _np(v),
                                kv_tile=KV_TILE, quant=ref)
    exact = oracle.attention_exact(_np(q), _np(k), _np(v))
    assert oracle.rel_l2(o, exact) <= oracle.rel_l2(pipe, exact) + 0.002
    print(f"    max|gpu-pipe| = {err:.2e}  relL2(gpu, exact) = {oracle.rel_l2(o, exact):.4f}", flush=True)


def test_block_mean_mode_block_constant_keys():
    # keys constant inside each 64-token block: K' = 0, the logits come only from the
    # block-mean products
    B, N, H, d = 1, 300, 2, 128
    q, k, v = random_qkv(B, N, H, d, seed=41)
    for j in range(0, N, 64):
        k[:, j:j + 64] = k[:, j:j + 1]
    out = sage.sage_attn_fwd_ex(q.cuda(), k.cuda(), v.cuda(), k_block_mean=True)
    ref = oracle.quantize(_np(q), _np(k), _np(v), k_block_mean=True)
    assert not ref["k_i8"].any()
    check_oracle(to_np(out), "block-constant keys", _np(q), _np(k), _np(v), kv_tile=KV_TILE, quant=ref)
