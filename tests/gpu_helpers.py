"""Shared helpers of the GPU parity tests: device inputs, oracle references,
comparisons.  Expected values come only from the oracle package."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import workloads

F32 = np.float32


def require_gpu():
    import pytest
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy() if t.dtype == torch.bfloat16 else t.detach().cpu().numpy()


def random_qkv(B, N, H, d, seed, outliers=0):
    w = workloads.Workload("case", B=B, H=H, N=N, d=d, outliers=outliers, seed=seed)
    return workloads.make_qkv(w)


def bf16_half_ulp(x: np.ndarray) -> np.ndarray:
    """Half a bf16 unit in the last place at |x| (bf16 keeps 8 significant bits)."""
    a = np.maximum(np.abs(x), 2.0 ** -126)
    e = np.floor(np.log2(a))
    return 0.5 * 2.0 ** (e - 7)


def compare_quant(gq: dict, ref: dict, N: int, blocks=None, v_rows=None):
    """Bit-exact comparison of the library's quantised operands with the oracle's.
    ``blocks``: 64-token blocks to compare (default all); ``v_rows``: V tokens."""
    B, H, npad, d = gq["q_i8"].shape
    nb = -(-N // 64)
    blocks = range(nb) if blocks is None else blocks
    q_i8, k_i8 = gq["q_i8"].cpu().numpy(), gq["k_i8"].cpu().numpy()
    for name, codes in (("q", q_i8), ("k", k_i8)):
        for j in blocks:
            r0, r1 = 64 * j, min(N, 64 * j + 64)
            got = codes[:, :, r0:r1]
            want = ref[f"{name}_i8"][:, :, r0:r1]
            assert np.array_equal(got, want), f"{name}_i8 block {j} differs ({np.count_nonzero(got != want)} codes)"
        assert not codes[:, :, N:].any(), f"{name}_i8 padding rows are not zero"
        sc = gq[f"{name}_scale"].cpu().numpy()
        assert np.array_equal(sc[:, :, :nb].view(np.uint32), ref[f"{name}_scale"].view(np.uint32)), f"{name}_scale differs"
        assert not sc[:, :, nb:].any(), f"{name}_scale padding blocks are not zero"
    km = gq["k_mean"].float().cpu().numpy()
    assert np.array_equal(km.view(np.uint32), ref["k_mean"].astype(F32).view(np.uint32)), "k_mean differs"
    vs = gq["v_scale"].cpu().numpy()
    assert np.array_equal(vs.view(np.uint32), ref["v_scale"].view(np.uint32)), "v_scale differs"
    v8 = gq["v_f8"].cpu().numpy().transpose(0, 1, 3, 2)        # -> [B, H, Npad, d]
    rows = np.arange(N) if v_rows is None else np.asarray(v_rows)
    vref = ref["v_f8"] if v_rows is None else ref["v_f8_rows"]
    assert np.array_equal(v8[:, :, rows], vref), f"v_f8 differs ({np.count_nonzero(v8[:, :, rows] != vref)} codes)"
    assert not v8[:, :, N:].any(), "v_f8 padding rows are not zero"


def attn_tolerance(o_pipe: np.ndarray) -> np.ndarray:
    """Bound on |GPU bf16 output - oracle fp64 output|: 2e-3 (the method's max-abs
    parity bound) plus the final bf16 rounding of the GPU output."""
    return 2e-3 + bf16_half_ulp(o_pipe)


def check_attention(o_gpu: np.ndarray, o_pipe: np.ndarray, label="", margin=None):
    """max |o_gpu - o_pipe| after checking it against attn_tolerance (plus ``margin``,
    the oracle's allowance for P codes that an fp32 evaluation may round either way)."""
    err = np.abs(o_gpu.astype(np.float64) - o_pipe)
    tol = attn_tolerance(o_pipe) + (0.0 if margin is None else margin)
    bad = err > tol
    assert not bad.any(), (f"{label}: {bad.sum()} outputs exceed the bound; max err "
                           f"{err.max():.3e}, worst excess {(err - tol).max():.3e}")
    return float(err.max())


def check_oracle(o_gpu: np.ndarray, label: str, *args, readings=("fp64", "fp32"), **kw):
    """Compare the GPU output with the oracle's quantised pipeline under both of its
    readings: the one whose P codes are decided in fp32, the softmax precision of the
    method, to the bound of ``check_attention``; and the plain one (fp64 logits and
    softmax) to that bound plus the oracle's margin for the P codes whose fp64 value
    lies within the fp32 evaluation error of an e4m3 (bf16) rounding boundary, which an
    fp32 softmax may round to the neighbouring code.  With block-residual K the fp32
    reading takes the block-mean products D exactly and rounds them once, while the
    kernel sums them on the matrix cores in their own order; that order is not modelled,
    so there the fp32 comparison allows the same margin.  ``args``/``kw`` go to
    ``oracle.attention_pipeline``.  Returns (max error against the first reading, max
    error against the second or None, the first reading's output)."""
    quant = kw.get("quant")
    kbm = bool(kw.get("k_block_mean")) or (quant is not None and quant.get("k_bmean") is not None)
    plain = None
    if "fp64" in readings or kbm:
        plain = oracle.attention_pipeline(*args, arith="fp64", code_margin=True, **kw)
    errs, first = [], None
    for r in readings:
        if r == "fp64":
            pipe, margin = plain
        else:
            pipe, margin = oracle.attention_pipeline(*args, arith=r, **kw), (plain[1] if kbm else None)
        errs.append(check_attention(o_gpu, pipe, f"{label} [{r}]", margin))
        first = pipe if first is None else first
    return errs[0], (errs[1] if len(errs) > 1 else None), first
