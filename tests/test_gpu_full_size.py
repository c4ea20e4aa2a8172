"""GPU parity at the benchmark's full sizes, through the C ABI, in the launch
configuration the bench times (one sage_attn_fwd over the whole workload).

The oracle cannot evaluate every output at these sizes, so each test checks samples it
can compute one by one:

- quantised operands of three heads, bit-exact: every scale, the K mean, all V codes,
  and sampled 64-token blocks of Q and K codes;
- int32 S tiles at sampled (query block, key tile) positions, including the last,
  ragged key tile;
- the attention output of sampled query rows of those heads against the oracle's
  quantised pipeline (rows are independent given the quantised K and V), plus
  rel-L2 against fp64 exact attention on the same rows.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
import quantized_attention_diffusion_amd as sage
from gpu_helpers import require_gpu, to_np, compare_quant, check_oracle

pytestmark = pytest.mark.gpu

FULL = ["flux_like", "sweep8k", "sweep16k", "video", "stress"]
N_ROWS = 40          # sampled query rows per head
N_BLOCKS = 12        # sampled 64-token Q/K code blocks per head
N_TILES = 3          # sampled S tiles per head


def setup_module(module):
    require_gpu()


def _head(t, h):
    """[B, N, H, d] bf16 CPU tensor -> float32 numpy [B, N, 1, d] of head h."""
    return t[:, :, h:h + 1, :].float().numpy()


def _head_quant(gq, h):
    return {key: (val[:, h:h + 1] if isinstance(val, torch.Tensor) else val) for key, val in gq.items()}


@pytest.mark.parametrize("name", FULL)
def test_full_size_parity(name):
    _full_size_parity(workloads.get(name))


def test_large_d64_two_batches_ragged():
    # d = 64, B = 2 and a ragged last tile at a 16K-class length (the named workloads are
    # all d = 128, B = 1)
    _full_size_parity(workloads.Workload("d64_b2", B=2, H=8, N=16384 - 37, d=64, seed=5))


def test_offsets_beyond_int32():
    # B*H*Npad*d = 3*100*65536*128 > 2^31 elements per tensor: heads past element 2^31 of
    # every operand, the dense and the block-sparse step, checked on sampled rows of the
    # first head and of the last heads
    B, H, N, d = 3, 100, 65536, 128
    assert B * H * N * d > 2 ** 31
    print(f"[int64] B={B} H={H} N={N} d={d}", flush=True)
    g = torch.Generator(device="cuda").manual_seed(77)
    q = torch.randn((B, N, H, d), generator=g, device="cuda").to(torch.bfloat16)
    k = (torch.randn((B, N, H, d), generator=g, device="cuda")
         + 3.0 * torch.randn((H, d), generator=g, device="cuda")).to(torch.bfloat16)
    v = torch.randn((B, N, H, d), generator=g, device="cuda").to(torch.bfloat16)
    out = sage.sage_attn_fwd(q, k, v)
    sparse = sage.sage_attn_fwd_sparse(q, k, v, 0.25)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    for b, h in [(0, 0), (B - 1, H - 1), (B - 1, H - 45)]:
        print(f"    (b, h) = {(b, h)}: element offset {((b * H + h) * N * d) / 2 ** 31:.2f} x 2^31", flush=True)
        qh, kh, vh = (t[b:b + 1, :, h:h + 1].float().cpu().numpy() for t in (q, k, v))
        ref = oracle.quantize(qh, kh, vh)
        rows = np.unique(np.concatenate([[0, N - 1], rng.choice(N, size=12, replace=False)]))
        check_oracle(to_np(out[b:b + 1, rows, h:h + 1, :]), f"int64 dense {(b, h)}", qh, kh, vh,
                     rows=rows, quant=ref)
        _, tiles = oracle.select_tiles(ref, 0.25)
        check_oracle(to_np(sparse[b:b + 1, rows, h:h + 1, :]), f"int64 sparse {(b, h)}", qh, kh, vh,
                     rows=rows, quant=ref, tiles=tiles)
    del q, k, v, out, sparse
    torch.cuda.empty_cache()


def test_maximum_sequence_length():
    # N = 2^22, the longest sequence the library accepts (one token more is refused):
    # the quantised operands bit-exact (every scale, the K mean, all V codes, sampled Q
    # and K code blocks), and sampled rows (the first, the last and two between) against
    # the oracle's plain reading
    B, H, N, d = 1, 1, 1 << 22, 64
    with pytest.raises(sage.SageError):
        sage.sage_workspace_bytes(B, H, N + 1, d)
    print(f"[max N] B={B} H={H} N={N} d={d}", flush=True)
    g = torch.Generator(device="cuda").manual_seed(78)
    q = torch.randn((B, N, H, d), generator=g, device="cuda").to(torch.bfloat16)
    k = (torch.randn((B, N, H, d), generator=g, device="cuda")
         + 3.0 * torch.randn((H, d), generator=g, device="cuda")).to(torch.bfloat16)
    v = torch.randn((B, N, H, d), generator=g, device="cuda").to(torch.bfloat16)
    out = sage.sage_attn_fwd(q, k, v)
    gq = sage.sage_quant_qk(q, k, v)
    torch.cuda.synchronize()
    qh, kh, vh = (t.float().cpu().numpy() for t in (q, k, v))
    ref = oracle.quantize(qh, kh, vh)
    compare_quant(gq, ref, N, blocks=[0, 1, N // 128, N // 64 - 1])
    rows = np.array([0, 1, N // 2 + 5, N - 1])
    err, _, _ = check_oracle(to_np(out[:, rows]), "max N", qh, kh, vh, rows=rows, quant=ref, readings=("fp64",))
    print(f"    max|gpu-pipe| = {err:.2e}", flush=True)
    del q, k, v, out, gq
    torch.cuda.empty_cache()


def test_maximum_head_count():
    # B = 1 with H = 65535 heads (the largest grid dimension the quantisation kernels
    # launch; H = 65536 is refused), a ragged N: the dense and the block-sparse step on
    # sampled heads, including the last
    B, H, N, d = 1, 65535, 200, 64
    with pytest.raises(sage.SageError):
        sage.sage_workspace_bytes(B, H + 1, N, d)
    print(f"[max H] B={B} H={H} N={N} d={d}", flush=True)
    g = torch.Generator(device="cuda").manual_seed(79)
    q = torch.randn((B, N, H, d), generator=g, device="cuda").to(torch.bfloat16)
    k = (torch.randn((B, N, H, d), generator=g, device="cuda")
         + 3.0 * torch.randn((H, d), generator=g, device="cuda")).to(torch.bfloat16)
    v = torch.randn((B, N, H, d), generator=g, device="cuda").to(torch.bfloat16)
    out = sage.sage_attn_fwd(q, k, v)
    sparse = sage.sage_attn_fwd_sparse(q, k, v, 0.5)
    torch.cuda.synchronize()
    for h in (0, 12345, H - 1):
        qh, kh, vh = (t[:, :, h:h + 1].float().cpu().numpy() for t in (q, k, v))
        ref = oracle.quantize(qh, kh, vh)
        check_oracle(to_np(out[:, :, h:h + 1]), f"max H dense head {h}", qh, kh, vh, quant=ref)
        _, tiles = oracle.select_tiles(ref, 0.5)
        check_oracle(to_np(sparse[:, :, h:h + 1]), f"max H sparse head {h}", qh, kh, vh, quant=ref, tiles=tiles)
    del q, k, v, out, sparse
    torch.cuda.empty_cache()


def _full_size_parity(w):
    name = w.name
    print(f"[full] {name} B={w.B} H={w.H} N={w.N} d={w.d}", flush=True)
    q, k, v = workloads.make_qkv(w)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    out = sage.sage_attn_fwd(qd, kd, vd)
    gq = sage.sage_quant_qk(qd, kd, vd)
    torch.cuda.synchronize()
    info = sage.sage_kernel_info()
    N, T, bm = w.N, info["kv_tile"], info["block_m"]
    npad = sage.sage_padded_tokens(N)
    rng = np.random.default_rng(1234)
    heads = sorted({0, w.H - 1, int(rng.integers(1, w.H - 1))})
    nb = -(-N // 64)
    for h in heads:
        qh, kh, vh = _head(q, h), _head(k, h), _head(v, h)
        ref = oracle.quantize(qh, kh, vh)
        # quantised operands
        blocks = sorted({0, nb - 1, *rng.choice(nb, size=N_BLOCKS - 2, replace=False).tolist()})
        compare_quant(_head_quant(gq, h), ref, N, blocks=blocks)
        # int32 S tiles (query block, key tile), the last key tile always included
        nqb, nkt = npad // bm, npad // T
        tiles = [(int(rng.integers(nqb)), nkt - 1)] + \
                [(int(rng.integers(nqb)), int(rng.integers(nkt))) for _ in range(N_TILES - 1)]
        for qb, kt in tiles:
            s = sage.sage_debug_qk_i32(gq["q_i8"], gq["k_i8"], N, 0, h, qb, kt).cpu().numpy()
            r0, c0 = qb * bm, kt * T
            r1, c1 = min(N, r0 + bm), min(N, c0 + T)
            want = oracle.qk_int32(ref["q_i8"][0, 0, r0:r1], ref["k_i8"][0, 0, c0:c1])
            assert np.array_equal(s[:r1 - r0, :c1 - c0], want), f"{name} head {h}: S tile {(qb, kt)} differs"
            assert not s[r1 - r0:, :].any() and not s[:, c1 - c0:].any()
        # attention output of sampled rows
        rows = np.unique(np.concatenate([[0, N - 1], np.arange(max(0, N - 5), N),
                                         rng.choice(N, size=N_ROWS, replace=False)]))
        o = to_np(out[:, rows, h:h + 1, :])
        err, err32, pipe = check_oracle(o, f"{name} head {h}", qh, kh, vh, kv_tile=T, rows=rows, quant=ref)
        exact = oracle.attention_exact(qh, kh, vh, rows=rows)
        r_gpu, r_pipe = oracle.rel_l2(o, exact), oracle.rel_l2(pipe, exact)
        print(f"    head {h}: max|gpu-pipe| = {err:.2e} (fp32 reading {err32:.2e})  relL2 gpu {r_gpu:.4f}  "
              f"pipe {r_pipe:.4f}", flush=True)
        assert r_gpu <= r_pipe + 0.002


@pytest.mark.parametrize("per_token", [False, True], ids=["block64", "per_token"])
@pytest.mark.parametrize("name", ["flux_like", "video"])
def test_full_size_quality_mode(name, per_token):
    w = workloads.get(name)
    print(f"[full quality] {name} B={w.B} H={w.H} N={w.N} d={w.d} per_token={per_token}", flush=True)
    q, k, v = workloads.make_qkv(w)
    out = sage.sage_attn_fwd_ex(q.cuda(), k.cuda(), v.cuda(), pv="bf16", per_token=per_token)
    torch.cuda.synchronize()
    rng = np.random.default_rng(4321)
    N = w.N
    for h in sorted({0, int(rng.integers(1, w.H))}):
        qh, kh, vh = _head(q, h), _head(k, h), _head(v, h)
        rows = np.unique(np.concatenate([[0, N - 1], rng.choice(N, size=N_ROWS, replace=False)]))
        o = to_np(out[:, rows, h:h + 1, :])
        err, _, pipe = check_oracle(o, f"{name} quality head {h}", qh, kh, vh, kv_tile=128, rows=rows,
                                    fp8_p=False, bf16_p=True, fp8_v=False, block=1 if per_token else 64)
        exact = oracle.attention_exact(qh, kh, vh, rows=rows)
        r_gpu, r_pipe = oracle.rel_l2(o, exact), oracle.rel_l2(pipe, exact)
        print(f"    head {h}: max|gpu-pipe| = {err:.2e}  relL2 gpu {r_gpu:.4f}  pipe {r_pipe:.4f}", flush=True)
        assert r_gpu <= r_pipe + 0.002


# The quality options at full size and on long grids.  Grids of more than 4 x (compute
# units) workgroups launch the plain instances of the attention kernel (the shorter
# ones the workgroup-pair instances), so these sizes run the instances the bench times.
MODES = {  # name: (per_token, k_block_mean)
    "fp8_per_token": (True, False),
    "block_mean_block64": (False, True),
    "block_mean_per_token": (True, True),
}


@pytest.mark.parametrize("mode", list(MODES))
@pytest.mark.parametrize("name", ["sweep16k", "stress", "d64_long"])
def test_full_size_fp8_modes(name, mode):
    per_token, kbm = MODES[mode]
    w = (workloads.Workload("d64_long", B=2, H=8, N=16384 - 37, d=64, seed=6) if name == "d64_long"
         else workloads.get(name))
    cus = torch.cuda.get_device_properties(torch.cuda.current_device()).multi_processor_count
    grid = w.B * w.H * (sage.sage_padded_tokens(w.N) // sage.sage_kernel_info()["block_m"])
    assert grid > 4 * cus, "the case must launch the plain (long-grid) instance"
    print(f"[full {mode}] {name} B={w.B} H={w.H} N={w.N} d={w.d} grid={grid}", flush=True)
    q, k, v = workloads.make_qkv(w)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    out = sage.sage_attn_fwd_ex(qd, kd, vd, per_token=per_token, k_block_mean=kbm)
    gq = sage.sage_quant_qk_ex(qd, kd, vd, sage.mode_bits("fp8", per_token=per_token, k_block_mean=kbm))
    torch.cuda.synchronize()
    rng = np.random.default_rng(2024)
    N = w.N
    nb = -(-N // 64)
    for b, h in sorted({(0, 0), (w.B - 1, w.H - 1), (int(rng.integers(w.B)), int(rng.integers(1, w.H - 1)))}):
        qh, kh, vh = (t[b:b + 1, :, h:h + 1, :].float().numpy() for t in (q, k, v))
        ref = oracle.quantize(qh, kh, vh, block=1 if per_token else 64, k_block_mean=kbm)
        # scales (and block means) bit-exact for the whole head, codes on sampled rows
        nsc = N if per_token else nb
        for nm in ("q", "k"):
            sc = gq[f"{nm}_scale"][b, h].cpu().numpy()
            assert np.array_equal(sc[:nsc].view(np.uint32), ref[f"{nm}_scale"][0, 0].view(np.uint32)), nm
        if kbm:
            km = gq["k_mean"][b, h].float().cpu().numpy()
            assert np.array_equal(km[:nb].view(np.uint32), ref["k_bmean"][0, 0].view(np.uint32))
        rows = np.unique(np.concatenate([[0, N - 1], np.arange(max(0, N - 5), N),
                                         rng.choice(N, size=N_ROWS, replace=False)]))
        for nm in ("q", "k"):
            codes = gq[f"{nm}_i8"][b, h].cpu().numpy()
            assert np.array_equal(codes[rows], ref[f"{nm}_i8"][0, 0][rows]), f"{nm}_i8 rows differ"
        o = to_np(out[b:b + 1, rows, h:h + 1, :])
        err, err32, pipe = check_oracle(o, f"{name} {mode} ({b}, {h})", qh, kh, vh, rows=rows, quant=ref)
        exact = oracle.attention_exact(qh, kh, vh, rows=rows)
        r_gpu, r_pipe = oracle.rel_l2(o, exact), oracle.rel_l2(pipe, exact)
        print(f"    ({b}, {h}): max|gpu-pipe| = {err:.2e} (fp32 reading {err32:.2e})  relL2 gpu {r_gpu:.4f}  "
              f"pipe {r_pipe:.4f}", flush=True)
        assert r_gpu <= r_pipe + 0.002
