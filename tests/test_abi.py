"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every
entry point the header declares, and rejects bad arguments with the documented status
before making any HIP call (fake device addresses are safe here for that reason)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sage_attn.h")


@pytest.fixture(scope="module")
def lib():
    from quantized_attention_diffusion_amd import _capi
    if not os.path.exists(_capi.lib_path):
        from quantized_attention_diffusion_amd import build
        build.build()
    return _capi.load()


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sage_\w+)\s*\(", text)))


def test_exports_every_declared_function(lib):
    from quantized_attention_diffusion_amd import _capi
    declared = _declared()
    assert declared == sorted(_capi.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


def _st(b, h, n):
    from quantized_attention_diffusion_amd._capi import sage_strides
    return sage_strides(b, h, n)


A = 1 << 32           # fake, 256-byte aligned device addresses: never dereferenced
B_ = 2 << 32
C = 3 << 32
O = 4 << 32
W = 5 << 32


def _fwd(lib, q=A, k=B_, v=C, o=O, B=1, H=2, N=100, d=128, sm=0.088, strides=None, ws=W, wsb=None):
    from quantized_attention_diffusion_amd._capi import sage_strides
    st = strides or [_st(N * H * d, d, H * d)] * 4
    arr = (sage_strides * 4)(*st)
    if wsb is None:
        n = ctypes.c_size_t()
        wsb = n.value if lib.sage_workspace_bytes(B, H, N, d, ctypes.byref(n)) == 0 else 1 << 40
    return lib.sage_attn_fwd(q, k, v, o, B, H, N, d, ctypes.c_float(sm), arr, None, ws, wsb)


def _err(lib):
    return lib.sage_last_error().decode()


def test_kernel_info_and_sizes(lib):
    from quantized_attention_diffusion_amd import _capi
    info = _capi.sage_kernel_info()
    assert info["arch"] == "gfx950" and info["quant_block"] == 64 and info["p_scale"] == 448.0
    assert info["d_supported"] == [64, 128]
    assert _capi.sage_padded_tokens(1) == 128 and _capi.sage_padded_tokens(4608) == 4608
    assert _capi.sage_padded_tokens(32760) == 32768 and _capi.sage_padded_tokens(0) == 0
    # the workspace holds 3 padded byte tensors plus scales and scratch
    ws = _capi.sage_workspace_bytes(1, 24, 4608, 128)
    assert ws >= 3 * 24 * 4608 * 128
    assert _capi.sage_quant_scratch_bytes(1, 24, 4608, 128) < ws


@pytest.mark.parametrize("kw,status,msg", [
    (dict(q=0), -1, "q is NULL"),
    (dict(o=0), -1, "out is NULL"),
    (dict(d=96), -2, "head dim"),
    (dict(N=0), -1, "must be >= 1"),
    (dict(N=(1 << 22) + 1), -2, "SAGE_MAX_TOKENS"),
    (dict(sm=float("nan")), -1, "sm_scale"),
    (dict(sm=-1.0), -1, "sm_scale"),
    (dict(sm=0.0, ws=0), -4, "workspace is NULL"),    # 0 selects 1/sqrt(d): accepted
    (dict(q=A + 8), -3, "16-byte aligned"),
    (dict(ws=0), -4, "workspace is NULL"),
    (dict(ws=W + 64), -4, "256-byte aligned"),
    (dict(wsb=1024), -4, "needed"),
    (dict(o=A), -1, "overlaps"),
])
def test_fwd_rejects_bad_arguments_before_any_hip_call(lib, kw, status, msg):
    assert _fwd(lib, **kw) == status
    assert msg in _err(lib)


def test_error_text_is_per_thread(lib):
    """sage_last_error is thread-local: threads that fail different checks at the same
    time each read back their own message."""
    import threading
    cases = [(dict(N=0), "must be >= 1"), (dict(sm=-1.0), "sm_scale"), (dict(q=A + 8), "16-byte aligned"),
             (dict(ws=0), "workspace is NULL")]
    bad = []
    barrier = threading.Barrier(len(cases))

    def worker(kw, msg):
        barrier.wait()
        for _ in range(200):
            _fwd(lib, **kw)
            if msg not in _err(lib):
                bad.append((msg, _err(lib)))
                return

    threads = [threading.Thread(target=worker, args=c) for c in cases]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not bad, bad


def test_fwd_rejects_misaligned_and_overlapping_strides(lib):
    N, H, d = 100, 2, 128
    bad = [_st(N * H * d, d, H * d + 4)] * 4
    assert _fwd(lib, strides=bad) == -3 and "multiples of 8" in _err(lib)
    same_row = [_st(N * H * d, d, H * d)] * 3 + [_st(N * H * d, d, 0)]    # out rows collide
    assert _fwd(lib, strides=same_row) == -1 and "overlap" in _err(lib)


def test_quant_and_debug_entry_points_validate(lib):
    from quantized_attention_diffusion_amd._capi import sage_strides
    st = _st(100 * 2 * 64, 64, 2 * 64)
    rc = lib.sage_quant_qk(A, B_, C, ctypes.byref(st), ctypes.byref(st), ctypes.byref(st),
                           1, 2, 100, 64, O, O + (1 << 20), O + (2 << 20), O + (3 << 20),
                           O + (4 << 20), O + (5 << 20), O + (6 << 20), 0, 0, None)
    assert rc == -4 and "scratch" in _err(lib)
    rc = lib.sage_quant_qk(A, B_, C, ctypes.byref(st), ctypes.byref(st), ctypes.byref(st),
                           1, 2, 100, 64, O, O, O + (2 << 20), O + (3 << 20),
                           O + (4 << 20), O + (5 << 20), O + (6 << 20), W, 1 << 20, None)
    assert rc == -1 and "overlaps" in _err(lib)
    rc = lib.sage_debug_qk_i32(A, B_, 1, 2, 100, 64, 0, 0, 0, 1, 2, 1, O, None)
    assert rc == -1 and "tile range" in _err(lib)
    rc = lib.sage_debug_qk_i32(A, B_, 1, 2, 100, 64, 0, 5, 0, 0, 1, 1, O, None)
    assert rc == -1 and "out of range" in _err(lib)
    rc = lib.sage_debug_qk_i32_ex(A, B_, 1, 2, 100, 128, 0, 0, 0, 0, 1, 1, 0x100, O, None)
    assert rc == -1 and "mode" in _err(lib)
    rc = lib.sage_debug_qk_i32_ex(A, B_, 1, 2, 100, 128, 0, 0, 0, 0, 1, 1, 5, O, None)
    assert rc == -2 and "SAGE_K_BLOCK_MEAN" in _err(lib)        # bf16 P.V with block-residual K
    rc = lib.sage_debug_qk_i32_ex(A, B_, 1, 2, 100, 128, 0, 0, 0, 1, 2, 1, 2, O, None)
    assert rc == -1 and "tile range" in _err(lib)
    assert lib.sage_debug_e4m3(A, O, -1, None) == -1
    assert lib.sage_debug_e4m3(0, 0, 0, None) == 0          # nothing to do, no launch
    rc = lib.sage_attn_fwd_prequant(A, A + 4096, B_, B_ + 4096, C, C + 4096, O,
                                    ctypes.byref(st), 1, 2, 100, 64, ctypes.c_float(float("inf")), None)
    assert rc == -1 and "sm_scale" in _err(lib)


def test_mode_entry_points_validate(lib):
    from quantized_attention_diffusion_amd import _capi
    from quantized_attention_diffusion_amd._capi import sage_strides
    B, H, N, d = 1, 24, 4608, 128
    base = _capi.sage_workspace_bytes_ex(B, H, N, d, 0)
    bf16 = _capi.sage_workspace_bytes_ex(B, H, N, d, _capi.mode_bits("bf16"))
    tok = _capi.sage_workspace_bytes_ex(B, H, N, d, _capi.mode_bits("fp8", per_token=True))
    assert base == _capi.sage_workspace_bytes(B, H, N, d)
    assert bf16 - base == B * H * N * d                  # the V region holds 2-byte values
    assert tok - base == 2 * 4 * B * H * (N - N // 64)   # two scale arrays grow to one per token
    n = ctypes.c_size_t()
    assert lib.sage_workspace_bytes_ex(B, H, N, d, 8, ctypes.byref(n)) == -1 and "mode" in _err(lib)
    # block-residual K: the k_mean region holds one mean per 64-token block
    kbm = _capi.sage_workspace_bytes_ex(B, H, N, d, _capi.mode_bits(k_block_mean=True))
    assert kbm - base == 2 * B * H * d * (N // 64 - 1)  # both sizes are multiples of 256 here
    assert lib.sage_workspace_bytes_ex(B, H, N, d, 5, ctypes.byref(n)) == -2 and "FP8" in _err(lib)
    st = (sage_strides * 4)(*([_st(100 * 2 * 128, 128, 2 * 128)] * 4))
    # unknown mode bits are rejected before anything else
    rc = lib.sage_attn_fwd_ex(A, B_, C, O, 1, 2, 100, 128, ctypes.c_float(0.088), st, 16, None, W, 1 << 40)
    assert rc == -1 and "mode" in _err(lib)
    # the quality mode needs its larger workspace
    lib.sage_workspace_bytes_ex(1, 2, 100, 128, 0, ctypes.byref(n))
    rc = lib.sage_attn_fwd_ex(A, B_, C, O, 1, 2, 100, 128, ctypes.c_float(0.088), st, 1, None, W, n.value)
    assert rc == -4 and "needed" in _err(lib)
    rc = lib.sage_attn_fwd_ex(0, B_, C, O, 1, 2, 100, 128, ctypes.c_float(0.088), st, 3, None, W, 1 << 40)
    assert rc == -1 and "q is NULL" in _err(lib)
    s1 = _st(100 * 2 * 64, 64, 2 * 64)
    rc = lib.sage_quant_qk_ex(A, B_, C, ctypes.byref(s1), ctypes.byref(s1), ctypes.byref(s1),
                              1, 2, 100, 64, 16, O, O + (1 << 20), O + (2 << 20), O + (3 << 20),
                              O + (4 << 20), O + (5 << 20), O + (6 << 20), W, 1 << 20, None)
    assert rc == -1 and "mode" in _err(lib)


def test_sparse_entry_points_validate(lib):
    from quantized_attention_diffusion_amd import _capi
    from quantized_attention_diffusion_amd._capi import sage_strides
    B, H, N, d = 1, 24, 4608, 128
    nt = N // 128
    n = ctypes.c_size_t()
    # scratch: Q and K code sums per 64-token block (two int8 digits per channel) + the
    # fp64 importance matrix
    assert lib.sage_select_scratch_bytes(B, H, N, d, ctypes.byref(n)) == 0
    assert n.value == 2 * B * H * (N // 64) * 2 * d + B * H * nt * nt * 8
    # the sparse workspace appends the scratch, tile_count and tile_list to the mode-0 one
    extra = _capi.sage_workspace_bytes_sparse(B, H, N, d) - _capi.sage_workspace_bytes(B, H, N, d)
    r256 = lambda x: -(-x // 256) * 256
    assert extra == n.value + r256(B * H * nt * 4) + r256(B * H * nt * nt * 4)
    # limits: key tiles per head, B*H
    assert lib.sage_select_scratch_bytes(1, 1, 4096 * 128 + 1, 64, ctypes.byref(n)) == -2
    assert "key tiles" in _err(lib)
    assert lib.sage_workspace_bytes_sparse(300, 300, 1024, 64, ctypes.byref(n)) == -2
    st = (sage_strides * 4)(*([_st(100 * 2 * 128, 128, 2 * 128)] * 4))
    for bad in (0.0, -1.0, float("nan")):
        rc = lib.sage_attn_fwd_sparse(A, B_, C, O, 1, 2, 100, 128, ctypes.c_float(0.088), st,
                                      ctypes.c_float(bad), None, W, 1 << 40)
        assert rc == -1 and "density" in _err(lib)
        rc = lib.sage_block_select(A, A + (1 << 20), B_, B_ + (1 << 20), 1, 2, 100, 128, ctypes.c_float(bad),
                                   C, C + (1 << 20), W, 1 << 30, None)
        assert rc == -1 and "density" in _err(lib)
    # the dense workspace is too small for the sparse call
    rc = lib.sage_attn_fwd_sparse(A, B_, C, O, 1, 2, 100, 128, ctypes.c_float(0.088), st,
                                  ctypes.c_float(0.5), None, W, _capi.sage_workspace_bytes(1, 2, 100, 128))
    assert rc == -4 and "needed" in _err(lib)
    rc = lib.sage_block_select(A, A + (1 << 20), B_, B_ + (1 << 20), 1, 2, 100, 128, ctypes.c_float(0.5),
                               0, C, W, 1 << 30, None)
    assert rc == -1 and "tile_count" in _err(lib)
    rc = lib.sage_block_select(A, A + (1 << 20), B_, B_ + (1 << 20), 1, 2, 100, 128, ctypes.c_float(0.5),
                               C, C + 4096, W, 16, None)
    assert rc == -4 and "needed" in _err(lib)
    rc = lib.sage_block_select(A, A + (1 << 20), B_, B_ + (1 << 20), 1, 2, 100, 128, ctypes.c_float(0.5),
                               A + 64, C, W, 1 << 30, None)
    assert rc == -1 and "overlap" in _err(lib)


def test_density_schedule_moves_from_sparse_to_dense(lib):
    """The host-only schedule helper: linear in the step index from tau_start (first
    step) to tau_end (last step), fp64 arithmetic rounded once to fp32."""
    import numpy as np
    import quantized_attention_diffusion_amd as sage
    n, t0, t1 = 30, 0.25, 1.0
    taus = [sage.sage_density_schedule(i, n, t0, t1) for i in range(n)]
    assert taus[0] == np.float32(t0) and taus[-1] == np.float32(t1)
    assert all(a < b for a, b in zip(taus, taus[1:]))                       # sparse early, dense late
    want = [float(np.float32(t0 + (t1 - t0) * i / (n - 1))) for i in range(n)]
    assert taus == want
    assert sage.sage_density_schedule(0, 1, 0.3, 0.9) == np.float32(0.9)    # one step: the last
    assert sage.sage_density_schedule(2, 5, 0.5, 0.5) == np.float32(0.5)    # constant
    assert sage.sage_density_schedule(4, 5, 1.0, 0.2) == np.float32(0.2)    # any direction
    tau = ctypes.c_float(-7.0)
    for args in ((5, 5, 0.5, 1.0), (-1, 5, 0.5, 1.0), (0, 0, 0.5, 1.0), (0, 5, 0.0, 1.0),
                 (0, 5, 0.5, float("inf")), (0, 5, float("nan"), 1.0)):
        rc = lib.sage_density_schedule(args[0], args[1], ctypes.c_float(args[2]), ctypes.c_float(args[3]),
                                       ctypes.byref(tau))
        assert rc == -1 and tau.value == -7.0
    assert lib.sage_density_schedule(0, 5, ctypes.c_float(0.5), ctypes.c_float(1.0), None) == -1


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    from quantized_attention_diffusion_amd import _capi
    monkeypatch.setattr(_capi, "_lib", None)
    monkeypatch.setattr(_capi, "lib_path", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        _capi.load()


def test_binding_rejects_operands_of_another_mode():
    # the prequant entry point takes mode-0 operands only, and a caller's operand dict
    # must match the layout the library writes for the requested mode
    import torch
    from quantized_attention_diffusion_amd import _capi
    with pytest.raises(ValueError, match="mode-0"):
        _capi.sage_attn_fwd_prequant({"mode": _capi.SAGE_QK_PER_TOKEN})
    B, H, N, d = 1, 2, 300, 64
    cpu = torch.device("cpu")
    good = _capi._alloc_quant(B, H, N, d, cpu, 0)
    _capi._check_quant_out(good, B, H, N, d, cpu, 0)
    with pytest.raises(ValueError, match="q_scale"):        # per-token scales need Npad entries
        _capi._check_quant_out(good, B, H, N, d, cpu, _capi.SAGE_QK_PER_TOKEN)
    with pytest.raises(ValueError, match="v_f8"):           # bf16 V needs 2 bytes per element
        _capi._check_quant_out(dict(good, q_scale=_capi._alloc_quant(B, H, N, d, cpu, 2)["q_scale"],
                                    k_scale=_capi._alloc_quant(B, H, N, d, cpu, 2)["k_scale"]),
                               B, H, N, d, cpu, _capi.SAGE_QK_PER_TOKEN | _capi.SAGE_PV_BF16)
    bad = dict(good)
    del bad["k_mean"]
    with pytest.raises(ValueError, match="k_mean"):
        _capi._check_quant_out(bad, B, H, N, d, cpu, 0)


def test_noalloc_entry_point_rejects_shapes_beyond_its_scratch(lib):
    # host-side size check before any HIP call: 8K tokens x 24 heads need 76.6 MiB of
    # workspace, more than the 64 MiB device array
    from quantized_attention_diffusion_amd import _capi
    from quantized_attention_diffusion_amd._capi import sage_strides
    B, H, N, d = 1, 24, 8192, 128
    assert _capi.sage_workspace_bytes(B, H, N, d) > _capi.NOALLOC_SCRATCH_BYTES
    st = (sage_strides * 4)(*[_st(N * H * d, d, H * d)] * 4)
    rc = lib.sage_attn_fwd_noalloc(A, B_, C, O, B, H, N, d, ctypes.c_float(0.0), st, None)
    assert rc == -4 and "no-allocation" in _err(lib)
    # argument errors come first, as for sage_attn_fwd
    rc = lib.sage_attn_fwd_noalloc(0, B_, C, O, 1, 2, 100, 128, ctypes.c_float(0.0),
                                   (sage_strides * 4)(*[_st(100 * 2 * 128, 128, 2 * 128)] * 4), None)
    assert rc == -1 and "q is NULL" in _err(lib)
